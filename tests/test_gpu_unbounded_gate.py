"""GPU parity of decays without a floor against the fp64 oracle, through the C ABI.

Kimi Linear's log-decay -e^A softplus(z) takes any value below 0 ("Kimi K3's
Architecture: ...", section "Channel-wise decay, and the floor K3 puts under it"), so a
channel can decay past e^-80 within one 16-token chunk, where the chunked kernel's
factorised decay would leave the fp32 range.  The chunked kernel finds such chunks and
runs them token by token; these tests mix such chunks with ordinary ones (per head, and
at chosen positions inside chunks) and compare both kernels with the oracle:
gate "lowrank_softplus" forms the gate in the kernels from its low-rank factors (the
oracle forms it with oracle.softplus_log_alpha, pinned on the CPU), and gate
"log_alpha_unbounded" reads log alpha given without a floor.
"""
import numpy as np
import pytest

import kda_workloads as W
import oracle
from kda_testlib import err, err_bf16, gpu_prefill, gpu_rows, oracle_prefill, say, subset, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = {"recurrent": 1e-4, "chunked_throughput": 1e-2, "auto": 1e-2}


def _gpu_softplus(inp, gate, algo, out="f32"):
    import torch
    import gated_delta_rule_kda_amd as kda
    bf = torch.bfloat16
    H = inp["q"].shape[1]
    cfg = kda.config(H, io_dtype="bf16", out_dtype=out, prologue=True, epilogue=True, algo=algo,
                     gate="lowrank_softplus", gate_rank=gate["gate_z"].shape[1])
    o, s, c = kda.prefill(
        to_dev(inp["q"], bf), to_dev(inp["k"], bf), to_dev(inp["v"], bf), None,
        to_dev(inp["beta"], torch.float32), to_dev(inp["cu_seqlens"].astype(np.int32), torch.int32),
        g=to_dev(inp["g"], bf), conv_w=to_dev(inp["conv_w"], torch.float32),
        conv_in=to_dev(inp.get("conv_in"), bf), state_in=to_dev(inp.get("state_in"), torch.float32),
        gate_z=to_dev(gate["gate_z"], bf), gate_w=to_dev(gate["gate_w"], bf),
        gate_bias=to_dev(gate["gate_bias"], torch.float32), gate_a=to_dev(gate["gate_a"], torch.float32),
        cfg=cfg)
    torch.cuda.synchronize()
    return dict(o=to_np(o), state=to_np(s), conv=to_np(c))


@pytest.mark.parametrize("algo", ["chunked_throughput", "recurrent"])
def test_softplus_gate_prefill_ragged(algo):
    """Heads 1 and 3 decay past the factorised range in most chunks, heads 0 and 2 stay
    inside it; ragged lengths with partial chunks and an empty sequence, random S0 and
    conv history."""
    inp = W.gen_prefill(W.PrefillSpec(lens=[5, 64, 130, 0, 33, 97], heads=4, state_std=0.02,
                                      conv_in=True, seed=91))
    gate = W.gen_softplus_gate(inp["cu_seqlens"], 4, 128, seed=92, wild_heads=(1, 3))
    la = oracle.softplus_log_alpha(gate["gate_z"], gate["gate_w"], gate["gate_bias"], gate["gate_a"])
    say(f"softplus gate prefill {algo}: log alpha min {la.min():.1f}")
    g = _gpu_softplus(inp, gate, algo)
    r = oracle_prefill(dict(inp, log_alpha=la))
    for h in range(4):
        eo, es = err(g["o"][:, h], r["o"][:, h]), err(g["state"][:, h], r["state"][:, h])
        say(f"  head {h}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= TOL[algo] and es <= TOL[algo], h
    assert np.array_equal(g["conv"], r["conv"])


def _spiky_log_alpha(inp, seed, depth=-300.0):
    """The slow-decay workload's log alpha with deep one-token decays planted in head 1:
    at chunk positions 0, 7 and 15 of channel 3, in the last (partial) chunk of a
    sequence, and at 1% of random (token, channel) places; head 0 keeps the slow decay,
    so its chunks stay on the matrix cores."""
    la = inp["log_alpha"].copy()
    cu = inp["cu_seqlens"].astype(np.int64)
    rng = np.random.default_rng(seed)
    T = la.shape[0]
    for n in range(len(cu) - 1):
        for pos in (0, 7, 15, 16 * ((cu[n + 1] - cu[n] - 1) // 16) + 1):
            if cu[n] + pos < cu[n + 1]:
                la[cu[n] + pos, 1, 3] = depth
    m = rng.random((T, W.D)) < 0.01
    la[:, 1][m] = depth
    return la


@pytest.mark.parametrize("io", ["bf16"])
def test_unbounded_log_alpha_spikes(io):
    """log alpha given without a floor: a slow decay (memory of tens of tokens, so S0 and
    the carried state matter) with one-token decays of e^-300 planted in one head."""
    inp = W.gen_prefill(W.PrefillSpec(lens=[200, 37, 16, 1], heads=2, io=io, state_std=0.05, conv_in=True,
                                      decay="slow", seed=93))
    inp["log_alpha"] = _spiky_log_alpha(inp, 94)
    say(f"unbounded log alpha ({io}): min {inp['log_alpha'].min():.0f}")
    g = gpu_prefill(inp, io=io, algo="chunked_throughput", gate="log_alpha_unbounded")
    r = oracle_prefill(inp)
    tol = 1e-2 if io == "bf16" else 2e-3
    for h in range(2):
        eo, es = err(g["o"][:, h], r["o"][:, h]), err(g["state"][:, h], r["state"][:, h])
        say(f"  head {h}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= tol and es <= tol, h
    assert np.array_equal(g["conv"], r["conv"])


def test_unbounded_log_alpha_recurrent_and_decode():
    """The recurrent kernel takes any log alpha as it is; then one decode step with a
    decay of e^-1000 in some channels."""
    import torch
    import gated_delta_rule_kda_amd as kda
    inp = W.gen_prefill(W.PrefillSpec(lens=[40, 9], heads=2, state_std=0.05, conv_in=True, decay="slow", seed=95))
    inp["log_alpha"] = _spiky_log_alpha(inp, 96)
    g = gpu_prefill(inp, algo="recurrent", gate="log_alpha_unbounded")
    r = oracle_prefill(inp)
    assert err(g["o"], r["o"]) <= TOL["recurrent"] and err(g["state"], r["state"]) <= TOL["recurrent"]
    B, H = 4, 2
    x = W.gen_decode(W.DecodeSpec(batch=B, heads=H, seed=97))
    x["log_alpha"][:, 1, ::5] = -1000.0
    ro, rs, rc = oracle.decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state"], g=x["g"],
                                    conv_w=x["conv_w"], conv_state=x["conv_state"])
    bf = torch.bfloat16
    st, cs = to_dev(x["state"], torch.float32), to_dev(x["conv_state"], bf)
    o = kda.decode_step(to_dev(x["q"], bf), to_dev(x["k"], bf), to_dev(x["v"], bf),
                        to_dev(x["log_alpha"], torch.float32), to_dev(x["beta"], torch.float32), st,
                        g=to_dev(x["g"], bf), conv_w=to_dev(x["conv_w"], torch.float32), conv_state=cs,
                        gate="log_alpha_unbounded", out_dtype="f32")
    torch.cuda.synchronize()
    assert err(to_np(o), ro) <= TOL["recurrent"] and err(to_np(st), rs) <= TOL["recurrent"]


def test_softplus_gate_decode():
    """One decode step with Kimi Linear's gate formed in the kernel."""
    import torch
    import gated_delta_rule_kda_amd as kda
    B, H = 6, 3
    x = W.gen_decode(W.DecodeSpec(batch=B, heads=H, seed=98))
    gate = W.gen_softplus_gate(np.arange(B + 1), H, 64, seed=99, wild_heads=(2,))
    la = oracle.softplus_log_alpha(gate["gate_z"], gate["gate_w"], gate["gate_bias"], gate["gate_a"])
    ro, rs, rc = oracle.decode_step(x["q"], x["k"], x["v"], la, x["beta"], x["state"], g=x["g"],
                                    conv_w=x["conv_w"], conv_state=x["conv_state"])
    bf = torch.bfloat16
    st, cs = to_dev(x["state"], torch.float32), to_dev(x["conv_state"], bf)
    o = kda.decode_step(to_dev(x["q"], bf), to_dev(x["k"], bf), to_dev(x["v"], bf), None,
                        to_dev(x["beta"], torch.float32), st, g=to_dev(x["g"], bf),
                        conv_w=to_dev(x["conv_w"], torch.float32), conv_state=cs,
                        gate_z=to_dev(gate["gate_z"], bf), gate_w=to_dev(gate["gate_w"], bf),
                        gate_bias=to_dev(gate["gate_bias"], torch.float32),
                        gate_a=to_dev(gate["gate_a"], torch.float32), gate="lowrank_softplus", out_dtype="f32")
    torch.cuda.synchronize()
    assert err(to_np(o), ro) <= TOL["recurrent"]
    assert err(to_np(st), rs) <= TOL["recurrent"]
    assert np.array_equal(to_np(cs), rc)


def test_softplus_gate_full_size_sampled():
    """The 4 x 4096 x 96 launch with Kimi Linear's gate, every eighth head decaying past
    the factorised range (bf16 output), checked on sampled (sequence, head) pairs, one of
    each kind."""
    spec = W.workload("prefill_4x4096")
    say("prefill_4x4096 softplus gate: generating inputs")
    inp = W.gen_prefill(spec)
    wild = tuple(range(0, spec.heads, 8))
    gate = W.gen_softplus_gate(inp["cu_seqlens"], spec.heads, 128, seed=100, wild_heads=wild)
    say("prefill_4x4096 softplus gate: gpu")
    g = _gpu_softplus(inp, gate, "auto", out="bf16")
    for seqs, heads in (([2], [8]), ([1], [13])):
        sub = subset(inp, seqs, heads)
        ch = np.concatenate([np.arange(h * W.D, (h + 1) * W.D) for h in heads])
        cu = inp["cu_seqlens"].astype(np.int64)
        tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs])
        sub["log_alpha"] = oracle.softplus_log_alpha(gate["gate_z"][tok], gate["gate_w"][ch],
                                                     gate["gate_bias"][ch], gate["gate_a"][heads])
        r = oracle_prefill(sub)
        gs = gpu_rows(g, inp, seqs, heads)
        eo, es = err_bf16(gs["o"], r["o"]), err(gs["state"], r["state"])
        say(f"  seqs {seqs} heads {heads}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= TOL["auto"] and es <= TOL["auto"]
