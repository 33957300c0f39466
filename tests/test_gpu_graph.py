"""HIP graphs over the C ABI.  The entry points enqueue kernels only (no allocation, no
memset, no host synchronisation), so a serving loop can capture a call in a graph once and
replay it.  Each test captures one call with every buffer passed in, replays it several
times with new inputs copied into the captured buffers (with unrelated eager work and a
synchronisation between replays), and compares every replay bit for bit with the same call
run eagerly on the same inputs; the first replay's inputs also go through the fp64 oracle.
"""
import numpy as np
import pytest

import kda_workloads as W
from kda_testlib import err, oracle_prefill, say, to_dev, to_np

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4   # the recurrent (decode) kernel
BF16_TOL = 1e-2   # the chunked kernels on bf16 inputs
REPLAYS = 3


def _other_work():
    """Eager work of the program between replays (a reduction over many blocks)."""
    import torch
    x = torch.arange(1 << 20, device="cuda", dtype=torch.float32)
    return float(x.sum().item())


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_step_graph_replays():
    """One decode step of 16 requests x 4 heads on a 24-row state pool (slot indices),
    captured once and replayed for three consecutive tokens: each replay advances the pool
    rows in place exactly as the eager steps do."""
    import torch
    import gated_delta_rule_kda_amd as kda
    B, H, rows = 16, 4, 24
    bf, f32 = torch.bfloat16, torch.float32
    steps = [W.gen_decode(W.DecodeSpec(batch=B, heads=H, seed=70 + i)) for i in range(REPLAYS)]
    x0 = steps[0]
    rng = np.random.default_rng(77)
    slots = rng.permutation(rows)[:B].astype(np.int32)
    pool = (rng.standard_normal((rows, H, W.D, W.D)) * 0.02).astype(np.float32)
    pool[slots] = x0["state"]
    cpool = W.bf16_round(rng.standard_normal((rows, 3, 3, H * W.D)).astype(np.float32))
    cpool[slots] = x0["conv_state"]
    cw = to_dev(x0["conv_w"], f32)
    sl = to_dev(slots, torch.int32)
    names = {"q": bf, "k": bf, "v": bf, "g": bf, "log_alpha": f32, "beta": f32}
    cfg = kda.config(H, io_dtype="bf16", out_dtype="f32", prologue=True, epilogue=True)

    def step(buf, st, cs, o):
        kda.decode_step(buf["q"], buf["k"], buf["v"], buf["log_alpha"], buf["beta"], st,
                        g=buf["g"], conv_w=cw, conv_state=cs, slots=sl, o=o, cfg=cfg)

    # eager steps
    st_e, cs_e = to_dev(pool, f32), to_dev(cpool, bf)
    o_e = torch.empty((B, H, W.D), dtype=f32, device="cuda")
    ref = []
    for x in steps:
        step({n: to_dev(x[n], t) for n, t in names.items()}, st_e, cs_e, o_e)
        torch.cuda.synchronize()
        ref.append((o_e.clone(), st_e.clone(), cs_e.clone()))
    # the first step against the oracle
    import oracle
    ro, rs, rc = oracle.decode_step(x0["q"], x0["k"], x0["v"], x0["log_alpha"], x0["beta"], x0["state"],
                                    g=x0["g"], conv_w=x0["conv_w"], conv_state=x0["conv_state"])
    assert err(to_np(ref[0][0]), ro) <= FP32_TOL
    assert err(to_np(ref[0][1])[slots], rs) <= FP32_TOL
    assert np.array_equal(to_np(ref[0][2])[slots], rc)

    # captured step on static buffers
    st_g, cs_g = to_dev(pool, f32), to_dev(cpool, bf)
    o_g = torch.zeros((B, H, W.D), dtype=f32, device="cuda")
    buf = {n: torch.zeros(x0[n].shape, dtype=t, device="cuda") for n, t in names.items()}
    graph = _capture(lambda: step(buf, st_g, cs_g, o_g))
    # capturing ran nothing
    assert torch.equal(st_g, to_dev(pool, f32)) and int(torch.count_nonzero(o_g)) == 0
    for i, x in enumerate(steps):
        for n, t in names.items():
            buf[n].copy_(to_dev(x[n], t))
        graph.replay()
        _other_work()
        torch.cuda.synchronize()
        say(f"decode graph replay {i}")
        assert torch.equal(o_g, ref[i][0]), f"replay {i}: output"
        assert torch.equal(st_g, ref[i][1]), f"replay {i}: state pool"
        assert torch.equal(cs_g, ref[i][2]), f"replay {i}: conv pool"


def _prefill_case(algo, lens, heads, seeds, no_alloc=False):
    """Eager prefill and a captured one on the same inputs, replayed once per seed."""
    import torch
    import gated_delta_rule_kda_amd as kda
    bf, f32 = torch.bfloat16, torch.float32
    specs = [W.PrefillSpec(lens=lens, heads=heads, state_std=0.02, conv_in=True, seed=s) for s in seeds]
    inps = [W.gen_prefill(s) for s in specs]
    x0 = inps[0]
    T, N = int(np.sum(lens)), len(lens)
    names = {"q": bf, "k": bf, "v": bf, "g": bf, "log_alpha": f32, "beta": f32,
             "state_in": f32, "conv_in": bf}
    cu = to_dev(x0["cu_seqlens"].astype(np.int32), torch.int32)
    cw = to_dev(x0["conv_w"], f32)
    cfg = kda.config(heads, io_dtype="bf16", out_dtype="f32", prologue=True, epilogue=True, algo=algo)
    ws_bytes = 0 if no_alloc else kda.workspace_size(cfg, N, T)
    say(f"graph prefill {algo}: lens {lens} x {heads} heads, workspace {ws_bytes} B, no_alloc={no_alloc}")

    def outputs():
        return (torch.zeros((T, heads, W.D), dtype=f32, device="cuda"),
                torch.zeros((N, heads, W.D, W.D), dtype=f32, device="cuda"),
                torch.zeros((N, 3, 3, heads * W.D), dtype=bf, device="cuda"),
                torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda"))

    def run(buf, out):
        o, so, co, ws = out
        kda.prefill(buf["q"], buf["k"], buf["v"], buf["log_alpha"], buf["beta"], cu, g=buf["g"],
                    conv_w=cw, conv_in=buf["conv_in"], state_in=buf["state_in"], o=o, state_out=so,
                    conv_out=co, workspace=None if no_alloc else ws, cfg=cfg, no_alloc=no_alloc)

    ref = []
    out_e = outputs()
    for x in inps:
        run({n: to_dev(x[n], t) for n, t in names.items()}, out_e)
        torch.cuda.synchronize()
        ref.append(tuple(t.clone() for t in out_e[:3]))
    r = oracle_prefill(x0)
    assert err(to_np(ref[0][0]), r["o"]) <= BF16_TOL
    assert err(to_np(ref[0][1]), r["state"]) <= BF16_TOL
    assert np.array_equal(to_np(ref[0][2]), r["conv"])

    buf = {n: torch.zeros(x0[n].shape, dtype=t, device="cuda") for n, t in names.items()}
    out_g = outputs()
    graph = _capture(lambda: run(buf, out_g))
    for i, x in enumerate(inps):
        for n, t in names.items():
            buf[n].copy_(to_dev(x[n], t))
        graph.replay()
        _other_work()
        torch.cuda.synchronize()
        say(f"graph prefill {algo} replay {i}")
        for what, a, b in zip(("output", "final state", "conv cache"), out_g[:3], ref[i]):
            assert torch.equal(a, b), f"replay {i}: {what}"


def test_chunked_prefill_graph_replays():
    """The chunked prefill (order kernel + chunk kernel) on three ragged sequences."""
    _prefill_case("chunked_throughput", [300, 77, 16], 4, [81, 82, 83])


def test_segmented_prefill_graph_replays():
    """The segmented prefill: segment table, first pass, scan and rerun launches, all in
    one graph, on one 2048-token sequence of 2 heads."""
    _prefill_case("chunked_scan", [2048], 2, [84, 85, 86])


def test_no_alloc_prefill_graph_replays():
    """The entry point for callers that cannot allocate, captured: its static scratch is
    resolved on the eager calls before the capture."""
    _prefill_case("chunked_throughput", [130, 9], 2, [87, 88, 89], no_alloc=True)
