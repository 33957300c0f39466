"""Seeded synthetic inputs for the KDA layer core.

This module only draws random numbers with the shapes and distributions of
the workloads below; it holds none of the layer's arithmetic and is the one
piece shared by the GPU path's tests/benchmark and the CPU oracle.

Every tensor is drawn block by block from numpy's PCG64, seeded with
SeedSequence([workload_seed, tensor_id, seq, head]), so any (sequence, head)
slice can be regenerated on its own.  Values are drawn in float32 (float64
for the gates, then rounded to float32); tensors stored as bf16 are rounded
to nearest-even bf16 here and returned as float32 arrays holding exactly
bf16-representable values, so both sides see identical inputs.

Workloads (H heads of width d = 128):
  core_fp32   B=1, H=2, T=256; fp32; q, k ~ N(0,1) then unit-normalised per
              (token, head); v ~ N(0,1); log alpha = -5*sigmoid(x), x ~ N(0,1);
              beta = sigmoid(y), y ~ N(0,1); S0 = 0; no prologue/epilogue.
  prefill_4x4096   B=4, H=96, T=4096; bf16 q, k, v, g ~ N(0,1); conv weights
              ~ N(0, 0.5^2) fp32; gates as above; S0 = 0; prologue + epilogue.
  prefill_131072   one sequence of T=131072, as above, S0 ~ N(0, 0.02^2).
  decode_256  B=256 requests, one token each; state ~ N(0, 0.02^2) fp32;
              bf16 q, k, v, g ~ N(0,1); conv caches ~ N(0,1) bf16.
  varlen_64   64 sequences, lengths lognormal with mean 8192 and sigma 1
              (mu = ln 8192 - 1/2), rounded and clipped to [16, 65536];
              per-sequence S0 ~ N(0, 0.02^2).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

D = 128

# tensor ids inside one workload's seed space
T_Q, T_K, T_V, T_G, T_ALPHA, T_BETA, T_CONVW, T_CONVIN, T_STATE, T_LENS = range(10)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bf16 (ties to even); returns a new
    float32 array.  (Finite inputs only: u + 0x8000 cannot wrap below the NaN range.)"""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _workers() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def _rng(seed: int, tensor: int, n: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, n, h])))


@dataclass
class PrefillSpec:
    lens: Sequence[int]
    heads: int = 96
    io: str = "bf16"               # "bf16" or "f32"
    prologue: bool = True
    epilogue: bool = True
    state_std: Optional[float] = None   # None -> S0 = 0 (no state given)
    conv_in: bool = False          # draw a conv history per sequence
    decay: str = "fast"            # "fast": -5*sigmoid(x); "slow": -5*sigmoid(x-6); "none": 0
    unit_qk: bool = False          # normalise q, k per (token, head) (prologue off)
    seed: int = 1
    name: str = "custom"
    first_seq: int = 0             # index of the first sequence in the seed space (slices of a larger workload)

    @property
    def total(self) -> int:
        return int(np.sum(self.lens))


def _fill_blocks(out: np.ndarray, seed: int, tensor: int, cu: np.ndarray, draw,
                 bf16: bool = False, per_head: bool = True, n0: int = 0) -> None:
    """out[cu[n]:cu[n+1], h] for every (sequence n, head h) from its own generator
    (or out[cu[n]:cu[n+1]] for every sequence n from one generator when
    per_head is False), rounded to bf16 values when asked.  Workers write
    their rows directly."""
    N = len(cu) - 1
    H = out.shape[1]
    heads = range(H) if per_head else [None]
    jobs = [(n, h) for n in range(N) for h in heads if cu[n + 1] > cu[n]]

    def one(job):
        n, h = job
        s, e = int(cu[n]), int(cu[n + 1])
        if h is None:
            blk = draw(_rng(seed, tensor, n0 + n, H), (e - s,) + out.shape[1:])
            out[s:e] = _bf16_inplace(blk) if bf16 else blk
            return
        blk = draw(_rng(seed, tensor, n0 + n, h), (e - s,) + out.shape[2:])
        if bf16:
            blk = _bf16_inplace(blk)
        out[s:e, h] = blk

    if out.size >= 1 << 16:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)


def _bf16_inplace(a: np.ndarray) -> np.ndarray:
    u = a.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return a


def _normal32(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _log_alpha(mode: str):
    def draw(rng, shape):
        x = rng.standard_normal(shape)
        if mode == "fast":
            return (-5.0 / (1.0 + np.exp(-x))).astype(np.float32)
        if mode == "slow":
            return (-5.0 / (1.0 + np.exp(-(x - 6.0)))).astype(np.float32)
        if mode == "none":
            return np.zeros(shape, np.float32)
        raise ValueError(mode)
    return draw


def _beta(rng, shape):
    y = rng.standard_normal(shape)
    return (1.0 / (1.0 + np.exp(-y))).astype(np.float32)


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


def gen_prefill(spec: PrefillSpec) -> Dict[str, np.ndarray]:
    """Draw every input of one prefill call as host float32 arrays.

    Keys: cu_seqlens (int32 [N+1]), q, k, v, g ([T,H,128]), log_alpha ([T,H,128]),
    beta ([T,H]), conv_w ([3,H*128,4]), conv_in ([N,3,3,H*128]) and state_in
    ([N,H,128,128]) -- the last four only when the spec asks for them.
    """
    lens = np.asarray(spec.lens, dtype=np.int64)
    cu = np.zeros(len(lens) + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    T, H, N = int(cu[-1]), spec.heads, len(lens)
    sd = spec.seed
    n0 = spec.first_seq
    out: Dict[str, np.ndarray] = {"cu_seqlens": cu.astype(np.int32)}
    for name, tid in (("q", T_Q), ("k", T_K), ("v", T_V)):
        a = np.empty((T, H, D), np.float32)
        draw = _unit if (spec.unit_qk and name != "v") else _normal32
        _fill_blocks(a, sd, tid, cu, draw, bf16=spec.io == "bf16", n0=n0)
        out[name] = a
    if spec.epilogue:
        a = np.empty((T, H, D), np.float32)
        _fill_blocks(a, sd, T_G, cu, _normal32, bf16=spec.io == "bf16", n0=n0)
        out["g"] = a
    a = np.empty((T, H, D), np.float32)
    _fill_blocks(a, sd, T_ALPHA, cu, _log_alpha(spec.decay), n0=n0)
    out["log_alpha"] = a
    b = np.empty((T, H), np.float32)
    _fill_blocks(b, sd, T_BETA, cu, _beta, n0=n0)
    out["beta"] = b
    if spec.prologue:
        out["conv_w"] = (_rng(sd, T_CONVW).standard_normal((3, H * D, 4)) * 0.5).astype(np.float32)
        if spec.conv_in:
            ci = np.empty((N, 3, 3, H * D), np.float32)
            for n in range(N):
                ci[n] = _rng(sd, T_CONVIN, n0 + n).standard_normal((3, 3, H * D), dtype=np.float32)
            out["conv_in"] = ci
    if spec.state_std is not None:
        st = np.empty((N, H, D, D), np.float32)

        def one(nh):
            n, h = nh
            st[n, h] = _rng(sd, T_STATE, n0 + n, h).standard_normal((D, D)) * spec.state_std

        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, [(n, h) for n in range(N) for h in range(H)]))
        out["state_in"] = st
    if spec.io == "bf16" and "conv_in" in out:
        out["conv_in"] = bf16_round(out["conv_in"])
    return out


@dataclass
class DecodeSpec:
    batch: int = 256
    heads: int = 96
    io: str = "bf16"
    state_std: float = 0.02
    decay: str = "fast"
    seed: int = 3
    name: str = "decode_256"


def gen_decode(spec: DecodeSpec) -> Dict[str, np.ndarray]:
    """Inputs of one decode step: q, k, v, g, log_alpha [B,H,128]; beta [B,H];
    state [B,H,128,128]; conv_state [B,3,3,H*128]; conv_w [3,H*128,4]."""
    B, H, sd = spec.batch, spec.heads, spec.seed
    cu = np.arange(B + 1, dtype=np.int64)
    out: Dict[str, np.ndarray] = {}
    # one generator per request (all heads at once)
    for name, tid in (("q", T_Q), ("k", T_K), ("v", T_V), ("g", T_G)):
        a = np.empty((B, H, D), np.float32)
        _fill_blocks(a, sd, tid, cu, _normal32, bf16=spec.io == "bf16", per_head=False)
        out[name] = a
    a = np.empty((B, H, D), np.float32)
    _fill_blocks(a, sd, T_ALPHA, cu, _log_alpha(spec.decay), per_head=False)
    out["log_alpha"] = a
    b = np.empty((B, H), np.float32)
    _fill_blocks(b, sd, T_BETA, cu, _beta, per_head=False)
    out["beta"] = b
    out["conv_w"] = (_rng(sd, T_CONVW).standard_normal((3, H * D, 4)) * 0.5).astype(np.float32)
    cs = np.empty((B, 3, 3, H * D), np.float32)
    st = np.empty((B, H, D, D), np.float32)

    def one(n):
        cs[n] = _rng(sd, T_CONVIN, n).standard_normal((3, 3, H * D), dtype=np.float32)
        _rng(sd, T_STATE, n).standard_normal((H, D, D), dtype=np.float32, out=st[n])
        st[n] *= np.float32(spec.state_std)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(B)))
    out["state"] = st
    out["conv_state"] = bf16_round(cs) if spec.io == "bf16" else cs
    return out


def gen_gate(cu_seqlens, heads: int, rank: int = 128, seed: int = 1, io: str = "bf16",
             first_seq: int = 0) -> Dict[str, np.ndarray]:
    """Low-rank gate factors of the "Kimi K3 - KDA layer" step list for packed sequences:
    z_down [T, r] per token (one generator per sequence, so slices of a workload match),
    W_up stored output-major [H*128, r] with N(0, 1/r) entries (z_down W_up ~ N(0, 1)),
    b_alpha [H*128] ~ N(0, 1) and A [H] ~ N(0.5, 0.2), so that e^A (z + b) spreads
    log alpha over (-5, 0) around -2.5 like the log-alpha workloads.  bf16-rounded for
    bf16 io (z_down, W_up); b_alpha and A are fp32."""
    cu = np.asarray(cu_seqlens, np.int64)
    T = int(cu[-1])
    z = np.zeros((T, 1, rank), np.float32)
    _fill_blocks(z, seed, 20, cu, lambda rng, shape: _normal32(rng, shape), bf16=(io == "bf16"),
                 per_head=False, n0=first_seq)
    rng = _rng(seed, 21)
    w = (rng.standard_normal((heads * D, rank)) / np.sqrt(rank)).astype(np.float32)
    if io == "bf16":
        w = _bf16_inplace(w)
    b = rng.standard_normal(heads * D).astype(np.float32)
    a = (0.5 + 0.2 * rng.standard_normal(heads)).astype(np.float32)
    return {"gate_z": z[:, 0], "gate_w": w, "gate_bias": b, "gate_a": a}


def gen_softplus_gate(cu_seqlens, heads: int, rank: int = 128, seed: int = 1, wild_heads=(),
                      first_seq: int = 0) -> Dict[str, np.ndarray]:
    """Factors of Kimi Linear's gate (log alpha = -e^A softplus(z_down W_up + b)), laid
    out as gen_gate's.  z_down ~ N(0, 1) and W_up ~ N(0, 1/r) (bf16-rounded); A [H] is
    the log of U(1, 16), one rate per head.  b_alpha: U(-7, -2.3) per channel, so that the
    per-token decay is mostly small (softplus(b) ~ e^b in (1e-3, 0.1)); the heads listed in
    wild_heads draw b ~ N(1, 1) instead, per-token log-decays of order -e^A (up to about
    -30), which takes most of their 16-token chunks past e^-80 in some channel."""
    cu = np.asarray(cu_seqlens, np.int64)
    T = int(cu[-1])
    z = np.zeros((T, 1, rank), np.float32)
    _fill_blocks(z, seed, 22, cu, lambda rng, shape: _normal32(rng, shape), bf16=True,
                 per_head=False, n0=first_seq)
    rng = _rng(seed, 23)
    w = _bf16_inplace((rng.standard_normal((heads * D, rank)) / np.sqrt(rank)).astype(np.float32))
    a = np.log(rng.uniform(1.0, 16.0, heads)).astype(np.float32)
    b = rng.uniform(-7.0, -2.3, heads * D)
    wild = rng.normal(1.0, 1.0, heads * D)
    for h in wild_heads:
        b[h * D:(h + 1) * D] = wild[h * D:(h + 1) * D]
    return {"gate_z": z[:, 0], "gate_w": w, "gate_bias": b.astype(np.float32), "gate_a": a}


def varlen_lengths(n_seqs: int = 64, mean: float = 8192.0, sigma: float = 1.0,
                   lo: int = 16, hi: int = 65536, seed: int = 4) -> List[int]:
    """Lognormal lengths whose distribution mean is `mean` (mu = ln mean - sigma^2/2)."""
    z = _rng(seed, T_LENS).standard_normal(n_seqs)
    mu = np.log(mean) - 0.5 * sigma * sigma
    return [int(x) for x in np.clip(np.rint(np.exp(mu + sigma * z)), lo, hi)]


def workload(name: str) -> object:
    """The named workloads; see the module docstring."""
    if name == "core_fp32":
        return PrefillSpec(lens=[256], heads=2, io="f32", prologue=False, epilogue=False,
                           unit_qk=True, seed=0, name=name)
    if name == "prefill_4x4096":
        return PrefillSpec(lens=[4096] * 4, heads=96, seed=1, name=name)
    if name == "prefill_131072":
        return PrefillSpec(lens=[131072], heads=96, state_std=0.02, seed=2, name=name)
    if name == "decode_256":
        return DecodeSpec(batch=256, heads=96, seed=3, name=name)
    if name == "varlen_64":
        return PrefillSpec(lens=varlen_lengths(), heads=96, state_std=0.02, seed=4, name=name)
    raise KeyError(name)
