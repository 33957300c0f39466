"""kda_prefill_no_alloc (the static-scratch entry point for callers that cannot allocate)
against kda_prefill with a caller workspace, through the C ABI: the same kernels, so the
results must be bitwise equal; two calls in a row, the second on a smaller input, so that
the scratch left by the first call cannot leak into the second."""
import numpy as np
import pytest
import torch

import kda_workloads as W
from kda_testlib import err, oracle_prefill, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _run(inp, algo, no_alloc):
    import gated_delta_rule_kda_amd as kda
    bf = torch.bfloat16
    H = inp["q"].shape[1]
    cfg = kda.config(H, io_dtype="bf16", out_dtype="f32", algo=algo)
    T = inp["q"].shape[0]
    N = len(inp["cu_seqlens"]) - 1
    o = torch.empty((T, H, 128), dtype=torch.float32, device="cuda")
    st = torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")
    cv = torch.empty((N, 3, 3, H * 128), dtype=bf, device="cuda")
    kda.prefill(to_dev(inp["q"], bf), to_dev(inp["k"], bf), to_dev(inp["v"], bf),
                to_dev(inp["log_alpha"], torch.float32), to_dev(inp["beta"], torch.float32),
                to_dev(inp["cu_seqlens"].astype(np.int32), torch.int32), g=to_dev(inp["g"], bf),
                conv_w=to_dev(inp["conv_w"], torch.float32), conv_in=to_dev(inp["conv_in"], bf),
                state_in=to_dev(inp["state_in"], torch.float32), o=o, state_out=st, conv_out=cv,
                cfg=cfg, no_alloc=no_alloc)
    torch.cuda.synchronize()
    return o, st, cv


@pytest.mark.parametrize("algo", ["chunked_throughput", "recurrent"])
def test_no_alloc_matches_workspace_entry_point(algo):
    big = W.gen_prefill(W.PrefillSpec(lens=[70, 0, 33, 150, 5, 17, 64], heads=3, state_std=0.03,
                                      conv_in=True, seed=301))
    small = W.gen_prefill(W.PrefillSpec(lens=[9, 40, 2], heads=3, state_std=0.03, conv_in=True, seed=302))
    for name, inp in (("big", big), ("small", small)):
        say(f"no-alloc {algo} {name}")
        ref = _run(inp, algo, no_alloc=False)
        got = _run(inp, algo, no_alloc=True)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"{algo} {name}: no-alloc result differs from kda_prefill"
        r = oracle_prefill(inp)
        tol = 1e-4 if algo == "recurrent" else 1e-2
        assert err(to_np(got[0]), r["o"]) <= tol and err(to_np(got[1]), r["state"]) <= tol
        assert np.array_equal(to_np(got[2]), r["conv"])
