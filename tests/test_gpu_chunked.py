"""GPU parity of the chunked MFMA prefill against the fp64 oracle, through the C ABI.

Tolerances (max|x - ref| / RMS(ref), per tensor):
  * bf16-input full-layer path: 1e-2 (the bar stated for this path).
  * The chunked kernel's own arithmetic: every contraction uses bf16 hi/lo
    operand splits (three MFMAs, ~2^-16 relative error per product) with
    fp32 accumulation.  Its raw read (no epilogue) stays within 2e-3 of the
    oracle.  The chunked algorithms take bf16 io only; the fp32-io
    reference-precision path is the recurrent kernel (test_gpu_recurrent.py).
"""
import numpy as np
import pytest

import kda_workloads as W
from kda_testlib import err, err_bf16, gpu_prefill, gpu_rows, oracle_prefill, say, subset, to_np

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2
CHUNKED_RAW_TOL = 2e-3

# the chunked kernel: two 8-wave workgroups per CU
VARIANTS = ["chunked_throughput"]
variants = pytest.mark.parametrize("algo", VARIANTS)


def _check(g, r, out, tol=BF16_TOL, conv=True):
    eo = err(g["o"], r["o"]) if out == "f32" else err_bf16(g["o"], r["o"])
    es = err(g["state"], r["state"])
    say(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= tol, eo
    assert es <= tol, es
    if conv and r.get("conv") is not None:
        assert np.array_equal(g["conv"], r["conv"]), "conv cache must be a bitwise shift of the inputs"
    return eo, es


@variants
def test_core_recurrence_unit_keys(algo):
    """B=1, H=2, T=256 core recurrence (no prologue/epilogue) on the chunked path, with the
    core workload's inputs rounded to bf16 (the chunked kernel's io type)."""
    spec = W.workload("core_fp32")
    spec.io = "bf16"
    inp = W.gen_prefill(spec)
    say("chunked core (bf16 io)")
    g = gpu_prefill(inp, io="bf16", out="f32", algo=algo)
    r = oracle_prefill(inp)
    _check(g, r, "f32", tol=CHUNKED_RAW_TOL)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@variants
def test_full_layer_ragged(out, algo):
    """Several chunks with ragged tails, random S0 and conv history, bf16 io."""
    spec = W.PrefillSpec(lens=[5, 64, 130, 1, 33, 0, 97], heads=4, state_std=0.02, conv_in=True, seed=41)
    inp = W.gen_prefill(spec)
    say(f"chunked full layer ragged out={out}")
    g = gpu_prefill(inp, io="bf16", out=out, algo=algo)
    r = oracle_prefill(inp)
    _check(g, r, out)


@variants
def test_full_layer_slow_decay(algo):
    """Slow decay (memory ~50 tokens) carries S0 and the inter-chunk state far."""
    spec = W.PrefillSpec(lens=[300, 77], heads=3, state_std=0.02, conv_in=True, decay="slow", seed=42)
    inp = W.gen_prefill(spec)
    say("chunked slow decay")
    g = gpu_prefill(inp, io="bf16", out="f32", algo=algo)
    r = oracle_prefill(inp)
    _check(g, r, "f32")


@variants
def test_raw_read_precision_slow_decay(algo):
    """No epilogue: the raw read o~ and S from the chunked kernel's split-bf16 arithmetic."""
    spec = W.PrefillSpec(lens=[200, 45], heads=2, state_std=0.02, conv_in=True, decay="slow",
                         epilogue=False, seed=43)
    inp = W.gen_prefill(spec)
    g = gpu_prefill(inp, io="bf16", out="f32", algo=algo)
    r = oracle_prefill(inp)
    _check(g, r, "f32", tol=CHUNKED_RAW_TOL)


@variants
def test_edge_lengths(algo):
    lens = [0, 1, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 0]
    inp = W.gen_prefill(W.PrefillSpec(lens=lens, heads=2, state_std=0.05, conv_in=True, seed=44))
    say("chunked edge lengths")
    g = gpu_prefill(inp, io="bf16", out="f32", algo=algo)
    r = oracle_prefill(inp)
    _check(g, r, "f32")
    # zero-length sequences pass state and conv history through unchanged
    assert np.array_equal(g["state"][0], inp["state_in"][0].astype(np.float64))
    assert np.array_equal(g["state"][-1], inp["state_in"][-1].astype(np.float64))


@variants
def test_in_place_state_and_conv(algo):
    inp = W.gen_prefill(W.PrefillSpec(lens=[70, 9, 2], heads=2, state_std=0.05, conv_in=True, seed=45))
    r = oracle_prefill(inp)
    g = gpu_prefill(inp, io="bf16", out="f32", algo=algo, in_place=True)
    _check(g, r, "f32")


@variants
def test_random_rms_gain(algo):
    """A random RMSNorm gain vector (shared by the heads) on the full layer."""
    spec = W.PrefillSpec(lens=[45, 7], heads=3, state_std=0.05, conv_in=True, seed=46)
    inp = W.gen_prefill(spec)
    rw = np.random.default_rng(5).uniform(0.5, 1.5, 128).astype(np.float32)
    g = gpu_prefill(inp, io="bf16", out="f32", algo=algo, rms_w=rw)
    r = oracle_prefill(inp, rms_w=rw)
    _check(g, r, "f32")


@pytest.mark.parametrize("algo", ["chunked_throughput", "chunked_scan"])
def test_beta_from_logit(algo):
    """beta passed as its pre-activation w ("Kimi K3 - KDA layer" step list: beta =
    sigmoid(w)), formed in the kernel; the oracle takes sigmoid(w) from its own fp64 step."""
    import oracle
    spec = W.PrefillSpec(lens=[5, 64, 130, 0, 33, 97], heads=3, state_std=0.02, conv_in=True, seed=50)
    inp = W.gen_prefill(spec)
    w = (np.random.default_rng(51).standard_normal(inp["beta"].shape) * 2.0).astype(np.float32)
    say(f"beta from logit ({algo})")
    g = gpu_prefill(dict(inp, beta=w), io="bf16", out="f32", algo=algo, beta_mode="logit")
    r = oracle_prefill(dict(inp, beta=oracle.beta_from_logit(w)))
    _check(g, r, "f32")


@variants
def test_orthonormal_keys_store_all(algo):
    """alpha = 1, beta = 1, S0 = 0 and 128 orthonormal keys: S = K^T V exactly,
    and every key reads back its own value (crosstalk-free delta writes)."""
    import torch
    import gated_delta_rule_kda_amd as kda
    from kda_testlib import to_dev
    rng = np.random.default_rng(47)
    # orthonormal keys that bf16 holds exactly: 32 diagonal blocks of the 4 x 4 Hadamard
    # matrix / 2 (entries +-1/2), then a random signed permutation of the channels and of
    # the key order
    H4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], np.float64) / 2.0
    B = np.kron(np.eye(32), H4)
    B = B[:, rng.permutation(128)] * rng.choice([-1.0, 1.0], 128)[None, :]
    K = B[rng.permutation(128)].astype(np.float32)
    assert np.allclose(K @ K.T, np.eye(128), atol=0)
    V = W.bf16_round(rng.standard_normal((128, 128)).astype(np.float32))
    T = 128
    inp = {"cu_seqlens": np.array([0, T], np.int32), "q": K[:, None, :], "k": K[:, None, :],
           "v": V[:, None, :], "log_alpha": np.zeros((T, 1, 128), np.float32),
           "beta": np.ones((T, 1), np.float32)}
    g = gpu_prefill(inp, io="bf16", out="f32", algo=algo, prologue=False, epilogue=False)
    S = g["state"][0, 0]
    ref = K.astype(np.float64).T @ V.astype(np.float64)
    e = err(S, ref)
    say(f"  orthonormal S err {e:.2e}")
    assert e <= CHUNKED_RAW_TOL
    # the read of k_t right after its write returns v_t (scale 1/sqrt(128))
    assert err(g["o"][:, 0] * np.sqrt(128.0), V) <= CHUNKED_RAW_TOL


@variants
def test_chaining_matches_one_call(algo):
    """prefill(a) then prefill(b) from the returned state and conv cache equals prefill(a|b)."""
    import torch
    spec = W.PrefillSpec(lens=[150], heads=2, state_std=0.02, conv_in=True, seed=48)
    full = W.gen_prefill(spec)
    cut = 77
    a = {k: (v[:cut] if k in ("q", "k", "v", "g", "log_alpha", "beta") else v) for k, v in full.items()}
    a["cu_seqlens"] = np.array([0, cut], np.int32)
    ga = gpu_prefill(a, io="bf16", out="f32", algo=algo)
    b = {k: (v[cut:] if k in ("q", "k", "v", "g", "log_alpha", "beta") else v) for k, v in full.items()}
    b["cu_seqlens"] = np.array([0, 150 - cut], np.int32)
    b["state_in"] = ga["state"].astype(np.float32)
    b["conv_in"] = ga["conv"].astype(np.float32)
    gb = gpu_prefill(b, io="bf16", out="f32", algo=algo)
    r = oracle_prefill(full)
    o = np.concatenate([ga["o"], gb["o"]])
    assert err(o, r["o"]) <= BF16_TOL
    assert err(gb["state"], r["state"]) <= BF16_TOL
    assert np.array_equal(gb["conv"], r["conv"])


@variants
def test_varlen_subset(algo):
    """Eight sequences drawn from the packed variable-length workload's length
    distribution (lognormal, mean 8192, clipped to [16, 65536]), 2 heads."""
    lens = W.varlen_lengths(n_seqs=8, seed=49)
    lens = [min(l, 6000) for l in lens]
    inp = W.gen_prefill(W.PrefillSpec(lens=lens, heads=2, state_std=0.02, seed=49))
    say(f"chunked varlen subset lens={lens}")
    g = gpu_prefill(inp, io="bf16", out="bf16", algo=algo)
    r = oracle_prefill(inp)
    _check(g, r, "bf16")


def test_side_stream_owns_its_allocations():
    """prefill on a side stream with no workspace or outputs passed: the binding allocates
    them for that stream (the longest-first order table and, for the segmented prefill, its
    M / B matrices), so allocations queued on the current stream right after cannot take
    that memory while the kernels still run.  The results equal the same calls on the
    current stream bit for bit, and the oracle."""
    import torch
    inp = W.gen_prefill(W.PrefillSpec(lens=[300, 17, 129, 64], heads=3, state_std=0.02, conv_in=True, seed=71))
    r = oracle_prefill(inp)
    side = torch.cuda.Stream()
    for algo in ("chunked_throughput", "chunked_scan"):
        say(f"side stream: {algo}")
        ref = gpu_prefill(inp, io="bf16", out="f32", algo=algo)
        g = gpu_prefill(inp, io="bf16", out="f32", algo=algo, stream=side, churn=True)
        for n in ("o", "state", "conv"):
            assert np.array_equal(g[n], ref[n]), (algo, n)
        _check(g, r, "f32")


def test_full_size_prefill_sampled():
    """The benchmark's launch (4 x 4096 tokens, 96 heads, bf16 io and output, AUTO
    algorithm): all 96 heads of sequence 0 and one head of each other sequence against the
    oracle, and a second launch bitwise equal to the first (no atomics, fixed orders)."""
    import torch
    import gated_delta_rule_kda_amd as kda
    spec = W.workload("prefill_4x4096")
    say("prefill_4x4096: generating inputs")
    inp = W.gen_prefill(spec)
    say("prefill_4x4096: gpu (twice)")
    o1, s1, c1 = gpu_prefill(inp, io="bf16", out="bf16", algo="auto", keep_device=True)
    o2, s2, c2 = gpu_prefill(inp, io="bf16", out="bf16", algo="auto", keep_device=True)
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(c1, c2), "prefill is not deterministic"
    g = dict(o=to_np(o1), state=to_np(s1), conv=to_np(c1))
    del o1, s1, c1, o2, s2, c2
    assert kda.resolved_algo(kda.config(96), 4, 16384) == "chunked_throughput"
    for seqs, heads in (([0], list(range(96))), ([1], [17]), ([2], [58]), ([3], [95])):
        sub = subset(inp, seqs, heads)
        r = oracle_prefill(sub)
        gs = gpu_rows(g, inp, seqs, heads)
        say(f"  seqs {seqs} heads {heads if len(heads) < 4 else 'all 96'}")
        _check(gs, r, "bf16")
    # every output is finite
    assert np.isfinite(g["o"]).all() and np.isfinite(g["state"]).all()


def test_long_context_sampled():
    """One 131072-token sequence, 96 heads, random fp32 S0 (the long-context launch):
    sampled heads against the oracle, for the AUTO choice (the segmented prefill) and the
    chunked kernel in one sequential pass."""
    import gated_delta_rule_kda_amd as kda
    spec = W.workload("prefill_131072")
    say("prefill_131072: generating inputs")
    inp = W.gen_prefill(spec)
    say("prefill_131072: gpu")
    assert kda.resolved_algo(kda.config(96), 1, 131072) == "chunked_scan"
    heads = [0, 3, 21, 40, 59, 77, 88, 95]
    r = oracle_prefill(subset(inp, [0], heads))
    for algo in ("auto", "chunked_throughput"):
        g = gpu_prefill(inp, io="bf16", out="bf16", algo=algo)
        gs = gpu_rows(g, inp, [0], heads)
        say(f"  {algo}: heads {heads}")
        _check(gs, r, "bf16")
        assert np.isfinite(g["o"]).all() and np.isfinite(g["state"]).all()


def test_varlen_full_size_sampled():
    """The packed variable-length launch as the benchmark times it: 64 sequences of
    lognormal lengths (578k tokens), 96 heads, per-sequence S0, bf16 io and output, AUTO
    algorithm.  Inputs are generated one sequence at a time straight into device buffers;
    ten sequences, from the longest to the shortest, are regenerated on the host and
    checked on one head each against the oracle."""
    import torch
    import gated_delta_rule_kda_amd as kda
    spec = W.workload("varlen_64")
    lens = [int(x) for x in spec.lens]
    N, H, T = len(lens), spec.heads, int(sum(lens))
    dev, bf = torch.device("cuda:0"), torch.bfloat16
    say(f"varlen_64: generating {T} tokens")
    bufs = {k: torch.empty((T, H, W.D), dtype=bf, device=dev) for k in ("q", "k", "v", "g")}
    la = torch.empty((T, H, W.D), dtype=torch.float32, device=dev)
    beta = torch.empty((T, H), dtype=torch.float32, device=dev)
    s0 = torch.empty((N, H, W.D, W.D), dtype=torch.float32, device=dev)
    off, cw = 0, None

    def seq(n):
        return W.gen_prefill(W.PrefillSpec(lens=[lens[n]], heads=H, state_std=spec.state_std, seed=spec.seed,
                                           first_seq=n))

    for n, L in enumerate(lens):
        x = seq(n)
        for k in bufs:
            bufs[k][off:off + L].copy_(torch.from_numpy(x[k]).to(bf))
        la[off:off + L].copy_(torch.from_numpy(x["log_alpha"]))
        beta[off:off + L].copy_(torch.from_numpy(x["beta"]))
        s0[n].copy_(torch.from_numpy(x["state_in"][0]))
        cw = x["conv_w"]
        off += L
        del x
    cu_np = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(cu_np).to(dev)
    say("varlen_64: gpu")
    cfg = kda.config(H, io_dtype="bf16", out_dtype="bf16")
    o, s, _ = kda.prefill(bufs["q"], bufs["k"], bufs["v"], la, beta, cu, g=bufs["g"],
                          conv_w=torch.from_numpy(cw).to(dev), state_in=s0, cfg=cfg, return_conv=False)
    torch.cuda.synchronize()
    del bufs, la, beta
    order = np.argsort(lens)
    picks = [int(order[i]) for i in np.linspace(N - 1, 0, 10).round().astype(int)]
    for n, h in zip(picks, (7, 45, 90, 3, 66, 12, 31, 80, 54, 95)):
        x = seq(n)
        sub = subset(x, [0], [h])
        r = oracle_prefill(sub)
        g_o = o[int(cu_np[n]):int(cu_np[n + 1]), h].float().cpu().numpy().astype(np.float64)
        g_s = s[n, h].cpu().numpy().astype(np.float64)
        eo, es = err_bf16(g_o, r["o"][:, 0]), err(g_s, r["state"][0, 0])
        say(f"  sequence {n} ({lens[n]} tokens) head {h}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= BF16_TOL and es <= BF16_TOL
    assert torch.isfinite(o).all()


def test_many_sequences_natural_order():
    """More sequences (8200, of 0 to 40 tokens) than the longest-first order table holds:
    the kernels take the sequences in their natural order, with no workspace."""
    import gated_delta_rule_kda_amd as kda
    lens = [int(x) for x in np.random.default_rng(131).integers(0, 41, 8200)]
    assert kda.workspace_size(kda.config(1), len(lens), sum(lens)) == 0
    inp = W.gen_prefill(W.PrefillSpec(lens=lens, heads=1, state_std=0.05, conv_in=True, seed=132))
    say(f"8200 sequences, {sum(lens)} tokens")
    g = gpu_prefill(inp, io="bf16", out="f32", algo="auto")
    r = oracle_prefill(inp)
    _check(g, r, "f32")
