"""GPU parity of the in-kernel low-rank gate against the fp64 oracle, through the C ABI.

With cfg.gate == "lowrank" the kernels form log alpha = -5 sigmoid(e^{A_h} (z_down W_up^T
+ b)) themselves ("Kimi K3 - KDA layer" step list) instead of reading it.  The oracle
forms the same log alpha in fp64 (oracle.lowrank_log_alpha, pinned on the CPU) and runs
the recurrence on it; the GPU results are compared with that, at the tolerance of each
path (1e-2 for the bf16 chunked path, 1e-4 for the fp32 recurrent kernel).
"""
import numpy as np
import pytest

import kda_workloads as W
import oracle
from kda_testlib import err, err_bf16, gpu_rows, oracle_prefill, say, subset, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = {"recurrent": 1e-4, "chunked_throughput": 1e-2, "auto": 1e-2}


def _with_gate(inp, rank, seed):
    g = W.gen_gate(inp["cu_seqlens"], inp["q"].shape[1], rank=rank, seed=seed)
    la = oracle.lowrank_log_alpha(g["gate_z"], g["gate_w"], g["gate_bias"], g["gate_a"])
    return g, dict(inp, log_alpha=la)


def _gpu_lowrank(inp, gate, algo, out="f32"):
    import torch
    import gated_delta_rule_kda_amd as kda
    bf = torch.bfloat16
    H = inp["q"].shape[1]
    cfg = kda.config(H, io_dtype="bf16", out_dtype=out, prologue=True, epilogue=True, algo=algo,
                     gate="lowrank", gate_rank=gate["gate_z"].shape[1])
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


@pytest.mark.parametrize("rank", [128, 64])
@pytest.mark.parametrize("algo", ["chunked_throughput", "recurrent"])
def test_lowrank_gate_prefill_ragged(algo, rank):
    """Ragged lengths (partial chunks, an empty sequence), random S0 and conv history."""
    inp = W.gen_prefill(W.PrefillSpec(lens=[5, 64, 130, 0, 33, 97], heads=3, state_std=0.02,
                                      conv_in=True, seed=71))
    gate, ref_in = _with_gate(inp, rank, 72)
    say(f"lowrank gate prefill {algo} r={rank}")
    g = _gpu_lowrank(inp, gate, algo)
    r = oracle_prefill(ref_in)
    eo, es = err(g["o"], r["o"]), err(g["state"], r["state"])
    say(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL[algo] and es <= TOL[algo]
    assert np.array_equal(g["conv"], r["conv"])


def test_lowrank_gate_slow_decay_carries_state():
    """A negative bias moves the gate towards alpha = 1 (memory of tens of tokens), so the
    state and S0 are carried across many chunks; also checks that padding rows of the
    last chunk do not decay the final state."""
    inp = W.gen_prefill(W.PrefillSpec(lens=[300, 77], heads=2, state_std=0.05, conv_in=True, seed=73))
    gate = W.gen_gate(inp["cu_seqlens"], 2, 128, seed=74)
    gate["gate_bias"] = (gate["gate_bias"] - 6.0).astype(np.float32)
    la = oracle.lowrank_log_alpha(gate["gate_z"], gate["gate_w"], gate["gate_bias"], gate["gate_a"])
    assert la.mean() > -0.1
    g = _gpu_lowrank(inp, gate, "auto")
    r = oracle_prefill(dict(inp, log_alpha=la))
    assert err(g["o"], r["o"]) <= TOL["auto"]
    assert err(g["state"], r["state"]) <= TOL["auto"]


def test_lowrank_gate_decode():
    """One decode step with the gate formed in the kernel, from the given state pool."""
    import torch
    import gated_delta_rule_kda_amd as kda
    B, H = 6, 3
    x = W.gen_decode(W.DecodeSpec(batch=B, heads=H, seed=75))
    gate = W.gen_gate(np.arange(B + 1), H, 96, seed=76)
    la = oracle.lowrank_log_alpha(gate["gate_z"], gate["gate_w"], gate["gate_bias"], gate["gate_a"])
    ro, rs, rc = oracle.decode_step(x["q"], x["k"], x["v"], la, x["beta"], x["state"], g=x["g"],
                                    conv_w=x["conv_w"], conv_state=x["conv_state"])
    bf = torch.bfloat16
    st, cs = to_dev(x["state"], torch.float32), to_dev(x["conv_state"], bf)
    o = kda.decode_step(to_dev(x["q"], bf), to_dev(x["k"], bf), to_dev(x["v"], bf), None,
                        to_dev(x["beta"], torch.float32), st, g=to_dev(x["g"], bf),
                        conv_w=to_dev(x["conv_w"], torch.float32), conv_state=cs,
                        gate_z=to_dev(gate["gate_z"], bf), gate_w=to_dev(gate["gate_w"], bf),
                        gate_bias=to_dev(gate["gate_bias"], torch.float32),
                        gate_a=to_dev(gate["gate_a"], torch.float32), out_dtype="f32")
    torch.cuda.synchronize()
    assert err(to_np(o), ro) <= TOL["recurrent"]
    assert err(to_np(st), rs) <= TOL["recurrent"]
    assert np.array_equal(to_np(cs), rc)


def test_lowrank_gate_full_size_sampled():
    """The 4 x 4096 x 96 launch with the gate formed in the kernel (bf16 output), checked
    on sampled (sequence, head) pairs against the oracle."""
    spec = W.workload("prefill_4x4096")
    say("prefill_4x4096 lowrank: generating inputs")
    inp = W.gen_prefill(spec)
    gate = W.gen_gate(inp["cu_seqlens"], spec.heads, 128, seed=77)
    say("prefill_4x4096 lowrank: gpu")
    g = _gpu_lowrank(inp, gate, "auto", out="bf16")
    for seqs, heads in (([1], [5]), ([2], [90])):
        sub = subset(inp, seqs, heads)
        ch = np.concatenate([np.arange(h * W.D, (h + 1) * W.D) for h in heads])
        cu = inp["cu_seqlens"].astype(np.int64)
        tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs])
        sub["log_alpha"] = oracle.lowrank_log_alpha(gate["gate_z"][tok], gate["gate_w"][ch],
                                                    gate["gate_bias"][ch], gate["gate_a"][heads])
        r = oracle_prefill(sub)
        gs = gpu_rows(g, inp, seqs, heads)
        eo, es = err_bf16(gs["o"], r["o"]), err(gs["state"], r["state"])
        say(f"  seqs {seqs} heads {heads}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= TOL["auto"] and es <= TOL["auto"]
