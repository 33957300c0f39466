"""The seeded input generators: ranges the pages fix, bf16 exactness, slice
regeneration.  CPU only."""
import numpy as np

import kda_workloads as W


def test_gate_ranges_follow_the_floor():
    # log alpha = -5 sigmoid(x) lies in (-5, 0), so alpha in (e^-5, 1) ("The lower bound
    # on decay is a hardware decision": g_min = -5, exp(-5) ~ 6.7e-3); beta = sigmoid in (0, 1)
    x = W.gen_prefill(W.PrefillSpec(lens=[300, 17], heads=3, seed=7))
    la, b = x["log_alpha"], x["beta"]
    assert la.min() > -5.0 and la.max() < 0.0
    assert b.min() > 0.0 and b.max() < 1.0
    assert abs(np.exp(-5.0) - 6.7e-3) < 1e-4


def test_bf16_rounding_is_exact_and_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3, 0.0], np.float32)
    r = W.bf16_round(vals)
    # ties to even: 1 + 2^-8 -> 1.0 ; 1 + 3*2^-8 -> 1 + 2^-6
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0 + 2 ** -6)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    x = W.gen_prefill(W.PrefillSpec(lens=[33], heads=2, seed=3))
    for key in ("q", "k", "v", "g"):
        assert np.all((x[key].view(np.uint32) & 0xFFFF) == 0)


def test_slices_regenerate_independently():
    a = W.gen_prefill(W.PrefillSpec(lens=[40, 25], heads=4, state_std=0.02, seed=9))
    b = W.gen_prefill(W.PrefillSpec(lens=[40, 25, 10], heads=4, state_std=0.02, seed=9))
    for key in ("q", "k", "v", "g", "log_alpha", "beta"):
        assert np.array_equal(a[key], b[key][:65]), key
    assert np.array_equal(a["state_in"], b["state_in"][:2])


def test_core_workload_unit_keys():
    x = W.gen_prefill(W.workload("core_fp32"))
    n = np.linalg.norm(x["q"].astype(np.float64), axis=-1)
    assert np.allclose(n, 1.0, atol=1e-6)
    assert x["q"].shape == (256, 2, 128) and "g" not in x and "conv_w" not in x


def test_varlen_lengths():
    lens = W.varlen_lengths()
    assert len(lens) == 64 and min(lens) >= 16 and max(lens) <= 65536
    # distribution mean 8192 for sigma = 1 (checked on many draws, not the 64 used)
    many = W.varlen_lengths(n_seqs=200000, lo=0, hi=10 ** 9, seed=11)
    assert abs(np.mean(many) / 8192.0 - 1.0) < 0.03


def test_sequence_slices_of_a_larger_workload():
    # a workload can be generated one sequence at a time (first_seq), matching the whole
    a = W.gen_prefill(W.PrefillSpec(lens=[40, 25, 10], heads=3, state_std=0.02, seed=9))
    b = W.gen_prefill(W.PrefillSpec(lens=[25], heads=3, state_std=0.02, seed=9, first_seq=1))
    for key in ("q", "k", "v", "g", "log_alpha", "beta"):
        assert np.array_equal(a[key][40:65], b[key]), key
    assert np.array_equal(a["state_in"][1], b["state_in"][0])
