"""GPU parity of the scalar per-head gate against the fp64 oracle, through the C ABI.

With cfg.gate == "head" every key channel of a head shares one decay per token, the
Mamba-2 / Gated DeltaNet gate that KDA refines to one decay per channel ("Kimi K3's
Architecture: ...", section "Channel-wise decay").  The kernels read log alpha [T, H]; the
oracle runs the channel-wise recurrence on that value repeated over the 128 channels, which
is the same recurrence.  The per-head values are channel 0 of the channel-wise workloads'
log alpha, so they follow the same distributions (fast, slow and no decay).
"""
import numpy as np
import pytest

import kda_workloads as W
from kda_testlib import err, err_bf16, gpu_prefill, gpu_rows, oracle_prefill, say, subset, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = {"recurrent": 1e-4, "chunked_throughput": 1e-2, "auto": 1e-2}


def _head(inp):
    """(GPU inputs with log alpha [T, H], oracle inputs with it repeated over channels)."""
    la = np.ascontiguousarray(inp["log_alpha"][..., 0])
    return dict(inp, log_alpha=la), dict(inp, log_alpha=np.repeat(la[..., None], W.D, axis=-1))


@pytest.mark.parametrize("decay", ["fast", "slow", "none"])
@pytest.mark.parametrize("algo", ["chunked_throughput", "recurrent"])
def test_head_gate_prefill_ragged(algo, decay):
    """Ragged lengths (partial chunks, an empty sequence), random S0 and conv history."""
    inp = W.gen_prefill(W.PrefillSpec(lens=[5, 64, 130, 0, 33, 97], heads=3, state_std=0.02,
                                      conv_in=True, decay=decay, seed=81))
    gin, rin = _head(inp)
    say(f"head gate prefill {algo} decay={decay}")
    g = gpu_prefill(gin, algo=algo, gate="head")
    r = oracle_prefill(rin)
    eo, es = err(g["o"], r["o"]), err(g["state"], r["state"])
    say(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL[algo] and es <= TOL[algo]
    assert np.array_equal(g["conv"], r["conv"])


def test_head_gate_core():
    """Without the prologue and epilogue, on the chunked kernel: the recurrence core alone,
    over a long sequence with a slow decay that carries S across chunks."""
    inp = W.gen_prefill(W.PrefillSpec(lens=[400, 17], heads=2, prologue=False, epilogue=False,
                                      unit_qk=True, state_std=0.05, decay="slow", seed=83))
    gin, rin = _head(inp)
    g = gpu_prefill(gin, io="bf16", algo="chunked_throughput", gate="head")
    r = oracle_prefill(rin)
    assert err(g["o"], r["o"]) <= 1e-2 and err(g["state"], r["state"]) <= 1e-2


def test_head_gate_strong_decay_underflow():
    """Per-token log alpha of -40: a chunk's cumulative decay underflows fp32, so the
    state is forgotten within a chunk; the result must stay finite and equal the oracle's."""
    inp = W.gen_prefill(W.PrefillSpec(lens=[50, 16], heads=2, state_std=0.05, conv_in=True, seed=85))
    gin, rin = _head(inp)
    gin["log_alpha"] = np.full_like(gin["log_alpha"], -40.0)
    rin["log_alpha"] = np.full_like(rin["log_alpha"], -40.0)
    g = gpu_prefill(gin, algo="chunked_throughput", gate="head")
    r = oracle_prefill(rin)
    assert np.isfinite(g["o"]).all() and np.isfinite(g["state"]).all()
    assert err(g["o"], r["o"]) <= 1e-2 and err(g["state"], r["state"]) <= 1e-2


def test_head_gate_decode():
    """One decode step with per-head log alpha [B, H]."""
    import torch
    import gated_delta_rule_kda_amd as kda
    import oracle
    B, H = 6, 3
    x = W.gen_decode(W.DecodeSpec(batch=B, heads=H, seed=87))
    la = np.ascontiguousarray(x["log_alpha"][..., 0])
    ro, rs, rc = oracle.decode_step(x["q"], x["k"], x["v"], np.repeat(la[..., None], W.D, axis=-1),
                                    x["beta"], x["state"], g=x["g"], conv_w=x["conv_w"],
                                    conv_state=x["conv_state"])
    bf = torch.bfloat16
    st, cs = to_dev(x["state"], torch.float32), to_dev(x["conv_state"], bf)
    o = kda.decode_step(to_dev(x["q"], bf), to_dev(x["k"], bf), to_dev(x["v"], bf),
                        to_dev(la, torch.float32), to_dev(x["beta"], torch.float32), st,
                        g=to_dev(x["g"], bf), conv_w=to_dev(x["conv_w"], torch.float32), conv_state=cs,
                        gate="head", out_dtype="f32")
    torch.cuda.synchronize()
    assert err(to_np(o), ro) <= TOL["recurrent"]
    assert err(to_np(st), rs) <= TOL["recurrent"]
    assert np.array_equal(to_np(cs), rc)


def test_head_gate_full_size_sampled():
    """The 4 x 4096 x 96 launch with the per-head gate (bf16 output), checked on sampled
    (sequence, head) pairs against the oracle."""
    spec = W.workload("prefill_4x4096")
    say("prefill_4x4096 head gate: generating inputs")
    inp = W.gen_prefill(spec)
    gin, _ = _head(inp)
    say("prefill_4x4096 head gate: gpu")
    g = gpu_prefill(gin, out="bf16", gate="head")
    for seqs, heads in (([0], [3]), ([3], [95])):
        _, rin = _head(subset(inp, seqs, heads))
        r = oracle_prefill(rin)
        gs = gpu_rows(g, inp, seqs, heads)
        eo, es = err_bf16(gs["o"], r["o"]), err(gs["state"], r["state"])
        say(f"  seqs {seqs} heads {heads}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= TOL["auto"] and es <= TOL["auto"]
