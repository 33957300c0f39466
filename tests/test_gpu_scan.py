"""GPU parity of the segmented prefill (KDA_ALGO_CHUNKED_SCAN) against the fp64 oracle.

Each sequence is cut into segments run in parallel; the middle segments' transitions
S -> M S + B are composed by a scan, and the segments rerun from the states it gives.
With the algorithm named, segments are 64 tokens, so the small cases below have up to
16 segments per sequence, a one-token last segment and sequences that fit one segment.
The slow decay keeps tens of tokens of memory, so the state and the conv history do
cross segment boundaries; the oracle runs every sequence token by token.
"""
import numpy as np
import pytest

import kda_workloads as W
import oracle
from kda_testlib import err, gpu_prefill, oracle_prefill, say, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = 1e-2
LENS = [300, 64, 1000, 0, 17, 129]


@pytest.mark.parametrize("decay", ["slow", "fast", "none"])
def test_scan_ragged(decay):
    """Ragged lengths (16, 5, 3 and 1 segments, an empty sequence), random S0 and conv
    history; outputs, final states and conv caches against the oracle, and against the
    sequential throughput pass."""
    import gated_delta_rule_kda_amd as kda
    inp = W.gen_prefill(W.PrefillSpec(lens=LENS, heads=3, state_std=0.05, conv_in=True, decay=decay, seed=111))
    say(f"scan ragged, decay {decay}")
    assert kda.resolved_algo(kda.config(3, algo="chunked_scan"), len(LENS), sum(LENS)) == "chunked_scan"
    g = gpu_prefill(inp, algo="chunked_scan")
    r = oracle_prefill(inp)
    eo, es = err(g["o"], r["o"]), err(g["state"], r["state"])
    say(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL and es <= TOL
    assert np.array_equal(g["conv"], r["conv"])
    t = gpu_prefill(inp, algo="chunked_throughput")
    assert err(g["o"], t["o"]) <= 2e-3 and err(g["state"], t["state"]) <= 2e-3


def test_scan_slow_decay_long():
    """One 3000-token sequence with memory of tens of tokens (47 segments): the composed
    transitions carry S0 and every segment's contribution to the end."""
    inp = W.gen_prefill(W.PrefillSpec(lens=[3000], heads=2, state_std=0.05, conv_in=True, decay="slow", seed=113))
    g = gpu_prefill(inp, algo="chunked_scan")
    r = oracle_prefill(inp)
    assert err(g["o"], r["o"]) <= TOL and err(g["state"], r["state"]) <= TOL
    assert np.array_equal(g["conv"], r["conv"])


def test_scan_no_decay_keeps_s0():
    """No decay and beta = 0: every transition is the identity and every offset zero, so
    the final state is S0 through 16 segments, and each output reads S0."""
    inp = W.gen_prefill(W.PrefillSpec(lens=[1000], heads=2, state_std=0.05, decay="none", seed=115))
    inp["beta"] = np.zeros_like(inp["beta"])
    g = gpu_prefill(inp, algo="chunked_scan", out="f32")
    r = oracle_prefill(inp)
    assert err(g["state"], inp["state_in"].astype(np.float64)) <= 1e-4
    assert err(g["o"], r["o"]) <= TOL


@pytest.mark.parametrize("gate", ["lowrank", "head"])
def test_scan_gates(gate):
    """The in-kernel low-rank gate and the per-head gate through the segmented prefill."""
    import torch
    import gated_delta_rule_kda_amd as kda
    inp = W.gen_prefill(W.PrefillSpec(lens=[700, 33, 250], heads=2, state_std=0.05, conv_in=True, decay="slow",
                                      seed=117))
    bf = torch.bfloat16
    cu = to_dev(inp["cu_seqlens"].astype(np.int32), torch.int32)
    common = dict(g=to_dev(inp["g"], bf), conv_w=to_dev(inp["conv_w"], torch.float32),
                  conv_in=to_dev(inp["conv_in"], bf), state_in=to_dev(inp["state_in"], torch.float32))
    if gate == "lowrank":
        gf = W.gen_gate(inp["cu_seqlens"], 2, 64, seed=118)
        gf["gate_bias"] = (gf["gate_bias"] - 5.0).astype(np.float32)  # long memory
        la = oracle.lowrank_log_alpha(gf["gate_z"], gf["gate_w"], gf["gate_bias"], gf["gate_a"])
        cfg = kda.config(2, out_dtype="f32", algo="chunked_scan", gate="lowrank", gate_rank=64)
        o, s, c = kda.prefill(to_dev(inp["q"], bf), to_dev(inp["k"], bf), to_dev(inp["v"], bf), None,
                              to_dev(inp["beta"], torch.float32), cu, gate_z=to_dev(gf["gate_z"], bf),
                              gate_w=to_dev(gf["gate_w"], bf), gate_bias=to_dev(gf["gate_bias"], torch.float32),
                              gate_a=to_dev(gf["gate_a"], torch.float32), cfg=cfg, **common)
        ref = dict(inp, log_alpha=la)
    else:
        lah = np.ascontiguousarray(inp["log_alpha"][..., 0])
        cfg = kda.config(2, out_dtype="f32", algo="chunked_scan", gate="head")
        o, s, c = kda.prefill(to_dev(inp["q"], bf), to_dev(inp["k"], bf), to_dev(inp["v"], bf),
                              to_dev(lah, torch.float32), to_dev(inp["beta"], torch.float32), cu, cfg=cfg, **common)
        ref = dict(inp, log_alpha=np.repeat(lah[..., None], W.D, axis=-1))
    torch.cuda.synchronize()
    r = oracle_prefill(ref)
    assert err(to_np(o), r["o"]) <= TOL and err(to_np(s), r["state"]) <= TOL
    assert np.array_equal(to_np(c), r["conv"])


def test_scan_pools_and_in_place():
    """Slot-indexed pools (read rows 4, 1, 0; write rows 2, 5, 1) and, second, the state and
    conv cache updated in place."""
    import torch
    import gated_delta_rule_kda_amd as kda
    H = 2
    inp = W.gen_prefill(W.PrefillSpec(lens=[260, 0, 500], heads=H, decay="slow", seed=119))
    rng = np.random.default_rng(120)
    rows, ins, outs = 6, [4, 1, 0], [2, 5, 1]
    st = (rng.standard_normal((rows, H, W.D, W.D)) * 0.05).astype(np.float32)
    cv = W.bf16_round(rng.standard_normal((rows, 3, 3, H * W.D)).astype(np.float32))
    r = oracle_prefill(dict(inp, state_in=st[ins], conv_in=cv[ins]))
    bf = torch.bfloat16
    st_d, cv_d = to_dev(st, torch.float32), to_dev(cv, bf)
    cfg = kda.config(H, out_dtype="f32", algo="chunked_scan")
    o, _, _ = kda.prefill(to_dev(inp["q"], bf), to_dev(inp["k"], bf), to_dev(inp["v"], bf),
                          to_dev(inp["log_alpha"], torch.float32), to_dev(inp["beta"], torch.float32),
                          to_dev(inp["cu_seqlens"].astype(np.int32), torch.int32), g=to_dev(inp["g"], bf),
                          conv_w=to_dev(inp["conv_w"], torch.float32), conv_in=cv_d, conv_out=cv_d,
                          state_in=st_d, state_out=st_d,
                          state_in_slots=to_dev(np.asarray(ins, np.int32), torch.int32),
                          state_out_slots=to_dev(np.asarray(outs, np.int32), torch.int32),
                          cfg=cfg, return_state=False, return_conv=False)
    torch.cuda.synchronize()
    st_n, cv_n = to_np(st_d), to_np(cv_d)
    assert err(to_np(o), r["o"]) <= TOL
    assert err(st_n[outs], r["state"]) <= TOL
    assert np.array_equal(cv_n[outs], r["conv"])
    keep = [i for i in range(rows) if i not in outs]
    assert np.array_equal(st_n[keep], st[keep].astype(np.float64))
    # in place, no pools
    inp2 = W.gen_prefill(W.PrefillSpec(lens=[400, 90], heads=H, state_std=0.05, conv_in=True, decay="slow",
                                       seed=121))
    r2 = oracle_prefill(inp2)
    g2 = gpu_prefill(inp2, algo="chunked_scan", in_place=True)
    assert err(g2["o"], r2["o"]) <= TOL and err(g2["state"], r2["state"]) <= TOL
    assert np.array_equal(g2["conv"], r2["conv"])


def test_scan_tp8_shape_sampled():
    """The per-GPU share of one 131072-token sequence at 12 heads (the head count of one
    GPU when 96 heads are split eight ways), AUTO algorithm: sampled heads."""
    import gated_delta_rule_kda_amd as kda
    spec = W.PrefillSpec(lens=[131072], heads=12, state_std=0.02, seed=123)
    assert kda.resolved_algo(kda.config(12), 1, 131072) == "chunked_scan"
    say("131072 x 12: generating inputs")
    inp = W.gen_prefill(spec)
    say("131072 x 12: gpu")
    from kda_testlib import gpu_rows, subset
    g = gpu_prefill(inp, io="bf16", out="bf16", algo="auto")
    heads = [0, 11]
    r = oracle_prefill(subset(inp, [0], heads))
    gs = gpu_rows(g, inp, [0], heads)
    from kda_testlib import err_bf16
    eo, es = err_bf16(gs["o"], r["o"]), err(gs["state"], r["state"])
    say(f"  heads {heads}: o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL and es <= TOL
    assert np.isfinite(g["o"]).all()


def test_auto_splits_few_items():
    """Few (sequence, head) items over moderate lengths (2 sequences of 1536 and 1200
    tokens x 4 heads, 8 items): AUTO takes the segmented prefill, which meets the oracle;
    the no-allocation entry point, whose scratch cannot hold the segment matrices, runs the
    throughput kernel instead, bit for bit as kda_prefill does when that kernel is named."""
    import torch
    import gated_delta_rule_kda_amd as kda
    H, lens = 4, [1536, 1200]
    inp = W.gen_prefill(W.PrefillSpec(lens=lens, heads=H, state_std=0.05, conv_in=True, decay="slow", seed=125))
    assert kda.resolved_algo(kda.config(H), len(lens), sum(lens)) == "chunked_scan"
    say("auto on 8 items: scan")
    g = gpu_prefill(inp, algo="auto")
    r = oracle_prefill(inp)
    assert err(g["o"], r["o"]) <= TOL and err(g["state"], r["state"]) <= TOL
    assert np.array_equal(g["conv"], r["conv"])
    bf, f32 = torch.bfloat16, torch.float32
    args = (to_dev(inp["q"], bf), to_dev(inp["k"], bf), to_dev(inp["v"], bf), to_dev(inp["log_alpha"], f32),
            to_dev(inp["beta"], f32), to_dev(inp["cu_seqlens"].astype(np.int32), torch.int32))
    kw = dict(g=to_dev(inp["g"], bf), conv_w=to_dev(inp["conv_w"], f32), conv_in=to_dev(inp["conv_in"], bf),
              state_in=to_dev(inp["state_in"], f32))
    say("auto on 8 items: no-alloc entry point")
    na = kda.prefill(*args, **kw, cfg=kda.config(H, out_dtype="f32"), no_alloc=True)
    tp = kda.prefill(*args, **kw, cfg=kda.config(H, out_dtype="f32", algo="chunked_throughput"))
    torch.cuda.synchronize()
    for a, b in zip(na, tp):
        assert torch.equal(a, b)
    assert err(to_np(na[0]), r["o"]) <= TOL


def test_tp_share_auto_deterministic():
    """The 4 x 4096 prefill at 12 heads (its share of one GPU under 8-way tensor
    parallelism), AUTO algorithm (the segmented prefill): two launches bitwise equal (no
    atomics, fixed orders), and heads 0 and 11 of sequences 0 and 3 against the oracle."""
    import torch
    import gated_delta_rule_kda_amd as kda
    from kda_testlib import err_bf16, gpu_rows, subset
    spec = W.PrefillSpec(lens=[4096] * 4, heads=12, seed=127)
    assert kda.resolved_algo(kda.config(12), 4, 4 * 4096) == "chunked_scan"
    inp = W.gen_prefill(spec)
    say("4 x 4096 x 12: gpu (twice)")
    o1, s1, c1 = gpu_prefill(inp, io="bf16", out="bf16", algo="auto", keep_device=True)
    o2, s2, c2 = gpu_prefill(inp, io="bf16", out="bf16", algo="auto", keep_device=True)
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(c1, c2), "not deterministic"
    g = dict(o=to_np(o1), state=to_np(s1), conv=to_np(c1))
    for seqs, heads in (([0], [0, 11]), ([3], [0, 11])):
        r = oracle_prefill(subset(inp, seqs, heads))
        gs = gpu_rows(g, inp, seqs, heads)
        eo, es = err_bf16(gs["o"], r["o"]), err(gs["state"], r["state"])
        say(f"  seqs {seqs} heads {heads}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= TOL and es <= TOL
        assert np.array_equal(gs["conv"], r["conv"])
