"""GPU parity of the token-sequential fp32 kernel (fp32 prefill path and the
decode step) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import kda_workloads as W
from kda_testlib import err, err_bf16, gpu_prefill, gpu_rows, oracle_prefill, say, subset, to_dev, to_np

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4   # fp32 path
BF16_TOL = 1e-2   # bf16-input path


def test_core_fp32_workload():
    """B=1, H=2, T=256 fp32 core recurrence (no prologue / epilogue)."""
    inp = W.gen_prefill(W.workload("core_fp32"))
    say("core_fp32: gpu")
    g = gpu_prefill(inp, io="f32", out="f32")
    r = oracle_prefill(inp)
    assert err(g["o"], r["o"]) <= FP32_TOL
    assert err(g["state"], r["state"]) <= FP32_TOL


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_full_layer_recurrent_bf16_inputs(out):
    spec = W.PrefillSpec(lens=[5, 64, 130, 1], heads=4, state_std=0.02, conv_in=True, seed=21)
    inp = W.gen_prefill(spec)
    say(f"full layer recurrent out={out}")
    g = gpu_prefill(inp, io="bf16", out=out, algo="recurrent")
    r = oracle_prefill(inp)
    e = err(g["o"], r["o"]) if out == "f32" else err_bf16(g["o"], r["o"])
    assert e <= FP32_TOL, e  # fp32 arithmetic: well inside the bf16-input bar
    assert err(g["state"], r["state"]) <= FP32_TOL
    assert np.array_equal(g["conv"], r["conv"]), "conv cache must be a bitwise shift of the inputs"


def test_full_layer_recurrent_fp32_io_with_gain():
    spec = W.PrefillSpec(lens=[33, 7], heads=3, io="f32", state_std=0.05, conv_in=True, seed=22)
    inp = W.gen_prefill(spec)
    rw = np.random.default_rng(5).uniform(0.5, 1.5, 128).astype(np.float32)
    g = gpu_prefill(inp, io="f32", out="f32", rms_w=rw)
    r = oracle_prefill(inp, rms_w=rw)
    assert err(g["o"], r["o"]) <= FP32_TOL
    assert err(g["state"], r["state"]) <= FP32_TOL
    assert np.array_equal(g["conv"], r["conv"])


def test_beta_from_logit_recurrent_and_decode():
    """beta given as its pre-activation (sigmoid formed in the kernel), fp32 io, at the fp32
    bar; then one decode step the same way."""
    import torch
    import gated_delta_rule_kda_amd as kda
    import oracle
    spec = W.PrefillSpec(lens=[33, 7, 1], heads=3, io="f32", state_std=0.05, conv_in=True, seed=25)
    inp = W.gen_prefill(spec)
    w = np.random.default_rng(26).standard_normal(inp["beta"].shape).astype(np.float32) * 3.0
    g = gpu_prefill(dict(inp, beta=w), io="f32", out="f32", algo="recurrent", beta_mode="logit")
    r = oracle_prefill(dict(inp, beta=oracle.beta_from_logit(w)))
    assert err(g["o"], r["o"]) <= FP32_TOL
    assert err(g["state"], r["state"]) <= FP32_TOL
    x = _decode_inputs(5, 3, 27)
    wd = np.random.default_rng(28).standard_normal(x["beta"].shape).astype(np.float32) * 3.0
    ro, rs, _ = oracle.decode_step(x["q"], x["k"], x["v"], x["log_alpha"], oracle.beta_from_logit(wd),
                                   x["state"], g=x["g"], conv_w=x["conv_w"], conv_state=x["conv_state"])
    bf = torch.bfloat16
    st, cs = to_dev(x["state"], torch.float32), to_dev(x["conv_state"], bf)
    o = kda.decode_step(to_dev(x["q"], bf), to_dev(x["k"], bf), to_dev(x["v"], bf),
                        to_dev(x["log_alpha"], torch.float32), to_dev(wd, torch.float32), st,
                        g=to_dev(x["g"], bf), conv_w=to_dev(x["conv_w"], torch.float32), conv_state=cs,
                        out_dtype="f32", beta_mode="logit")
    torch.cuda.synchronize()
    assert err(to_np(o), ro) <= FP32_TOL and err(to_np(st), rs) <= FP32_TOL


def test_edge_lengths_recurrent():
    lens = [0, 1, 3, 15, 16, 17, 63, 64, 65, 0]
    inp = W.gen_prefill(W.PrefillSpec(lens=lens, heads=2, state_std=0.05, conv_in=True, seed=23))
    g = gpu_prefill(inp, io="bf16", out="f32", algo="recurrent")
    r = oracle_prefill(inp)
    assert err(g["o"], r["o"]) <= FP32_TOL
    assert err(g["state"], r["state"]) <= FP32_TOL
    assert np.array_equal(g["conv"], r["conv"])
    assert np.array_equal(g["state"][0], inp["state_in"][0].astype(np.float64))


def test_in_place_state_and_conv():
    inp = W.gen_prefill(W.PrefillSpec(lens=[40, 9], heads=2, state_std=0.05, conv_in=True, seed=24))
    r = oracle_prefill(inp)
    g = gpu_prefill(inp, io="bf16", out="f32", algo="recurrent", in_place=True)
    assert err(g["state"], r["state"]) <= FP32_TOL
    assert np.array_equal(g["conv"], r["conv"])


def _decode_inputs(B, H, seed):
    return W.gen_decode(W.DecodeSpec(batch=B, heads=H, seed=seed))


def _oracle_decode(x, sel=None):
    import oracle
    if sel is None:
        sel = slice(None)
    return oracle.decode_step(x["q"][sel], x["k"][sel], x["v"][sel], x["log_alpha"][sel],
                              x["beta"][sel], x["state"][sel], g=x["g"][sel], conv_w=x["conv_w"],
                              conv_state=x["conv_state"][sel])


def _gpu_decode(x, out="bf16", slots=None, state=None, conv=None):
    import torch
    import gated_delta_rule_kda_amd as kda
    bf = torch.bfloat16
    st = to_dev(x["state"], torch.float32) if state is None else state
    cs = to_dev(x["conv_state"], bf) if conv is None else conv
    o = kda.decode_step(to_dev(x["q"], bf), to_dev(x["k"], bf), to_dev(x["v"], bf),
                        to_dev(x["log_alpha"], torch.float32), to_dev(x["beta"], torch.float32), st,
                        g=to_dev(x["g"], bf), conv_w=to_dev(x["conv_w"], torch.float32),
                        conv_state=cs, slots=slots, out_dtype=out)
    torch.cuda.synchronize()
    return o, st, cs


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_decode_small(out):
    x = _decode_inputs(8, 4, 31)
    o, st, cs = _gpu_decode(x, out=out)
    ro, rs, rc = _oracle_decode(x)
    e = err(to_np(o), ro) if out == "f32" else err_bf16(to_np(o), ro)
    assert e <= FP32_TOL
    assert err(to_np(st), rs) <= FP32_TOL
    assert np.array_equal(to_np(cs), rc)


def test_decode_slots():
    """Requests address a larger state pool through slot indices."""
    import torch
    x = _decode_inputs(6, 3, 32)
    pool = 10
    perm = np.array([7, 2, 9, 0, 4, 5], np.int32)
    big = np.random.default_rng(1).standard_normal((pool, 3, 128, 128)).astype(np.float32) * 0.02
    big[perm] = x["state"]
    bigc = np.random.default_rng(2).standard_normal((pool, 3, 3, 3 * 128)).astype(np.float32)
    bigc = W.bf16_round(bigc)
    bigc[perm] = x["conv_state"]
    st = to_dev(big, torch.float32)
    cs = to_dev(bigc, torch.bfloat16)
    o, st, cs = _gpu_decode(x, out="f32", slots=to_dev(perm, torch.int32), state=st, conv=cs)
    ro, rs, rc = _oracle_decode(x)
    assert err(to_np(o), ro) <= FP32_TOL
    stn, csn = to_np(st), to_np(cs)
    assert err(stn[perm], rs) <= FP32_TOL
    assert np.array_equal(csn[perm], rc)
    untouched = np.setdiff1d(np.arange(pool), perm)
    assert np.array_equal(stn[untouched], big[untouched].astype(np.float64))


def test_prefill_then_decode_chain():
    """prefill(T) then three decode steps equals prefill(T + 3)."""
    import torch
    spec = W.PrefillSpec(lens=[21], heads=2, state_std=0.02, conv_in=True, seed=33)
    full = W.gen_prefill(spec)
    head = {k: (v[:18] if k not in ("cu_seqlens", "conv_w", "conv_in", "state_in") else v)
            for k, v in full.items()}
    head["cu_seqlens"] = np.array([0, 18], np.int32)
    o, s, c = gpu_prefill(head, io="bf16", out="f32", algo="recurrent", keep_device=True)
    outs = [to_np(o)]
    for t in range(18, 21):
        x = {k: full[k][t:t + 1] for k in ("q", "k", "v", "g", "log_alpha", "beta")}
        x["conv_w"] = full["conv_w"]
        oo, s, c = _gpu_decode(x, out="f32", state=s, conv=c)
        outs.append(to_np(oo))
    r = oracle_prefill(full)
    assert err(np.concatenate(outs), r["o"]) <= FP32_TOL
    assert err(to_np(s), r["state"]) <= FP32_TOL
    assert np.array_equal(to_np(c), r["conv"])


def test_decode_full_size_all_pairs():
    """B=256 requests x 96 heads, the launch the benchmark times: every (request, head)
    pair's output and new state against the oracle's fp64 step, the conv shift checked
    everywhere, and a second launch from the same inputs bitwise equal to the first."""
    import torch
    import oracle
    say("decode_256: generating inputs")
    x = W.gen_decode(W.workload("decode_256"))
    say("decode_256: gpu step (twice)")
    o, st, cs = _gpu_decode(x, out="bf16")
    o2, st2, cs2 = _gpu_decode(x, out="bf16")
    assert torch.equal(o, o2) and torch.equal(st, st2) and torch.equal(cs, cs2), "decode is not deterministic"
    del o2, st2, cs2
    on, stn, csn = to_np(o), to_np(st), to_np(cs)
    del st
    say("decode_256: oracle on all 24576 (request, head) pairs")
    ro, rs, rc = _oracle_decode(x)
    eo, es = err_bf16(on, ro), err(stn, rs)
    say(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= BF16_TOL / 100
    assert es <= FP32_TOL
    # per (request, head) as well: no pair hides behind the global RMS
    d = np.abs(stn - rs).reshape(256 * 96, -1).max(axis=1)
    rms = np.sqrt((rs.reshape(256 * 96, -1) ** 2).mean(axis=1))
    assert (d <= FP32_TOL * np.maximum(rms, 1e-30) * 20).all()
    assert np.array_equal(csn, rc)
    cin = x["conv_state"].reshape(256, 3, 3, 96 * 128)
    assert np.array_equal(csn[:, :, :2], cin[:, :, 1:])
    newest = np.stack([x["q"], x["k"], x["v"]], axis=1).reshape(256, 3, 96 * 128)
    assert np.array_equal(csn[:, :, 2], newest)
