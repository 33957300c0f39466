"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
C-ABI library, run the oracle on the same inputs (optionally on a subset of
sequences and heads, which are independent), and measure errors.

Error metric (per tensor): max|x - ref| / RMS(ref).  For bf16 outputs the
output rounding itself is allowed for: rounding to nearest bf16 moves a value
by at most 2^-8 of its magnitude, so |x - ref| <= 2^-8 |ref| + (1 + 2^-8) e,
where e is the error before rounding; the bf16 metric subtracts 2^-8 |ref|
elementwise before taking the max.
"""
from __future__ import annotations

import sys
from typing import Dict, Optional, Sequence

import numpy as np

import kda_workloads as W
import oracle

BF16_HALF_ULP = 2.0 ** -8


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def err(x, ref) -> float:
    x = np.asarray(x, np.float64); ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(x - ref)) / rms) if rms > 0 else float(np.max(np.abs(x - ref)))


def err_bf16(x, ref) -> float:
    x = np.asarray(x, np.float64); ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref * ref))
    d = np.maximum(np.abs(x - ref) - BF16_HALF_ULP * np.abs(ref), 0.0)
    return float(np.max(d) / rms)


def to_dev(a: Optional[np.ndarray], dtype):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda").to(dtype)


def to_np(t) -> Optional[np.ndarray]:
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_prefill(inp: Dict[str, np.ndarray], io: str = "bf16", out: str = "f32", algo: str = "auto",
                prologue: Optional[bool] = None, epilogue: Optional[bool] = None,
                rms_w: Optional[np.ndarray] = None, in_place: bool = False,
                keep_device: bool = False, gate: str = "log_alpha", beta_mode: str = "value",
                stream=None, churn: bool = False):
    import torch
    import gated_delta_rule_kda_amd as kda
    io_t = torch.bfloat16 if io == "bf16" else torch.float32
    prologue = ("conv_w" in inp) if prologue is None else prologue
    epilogue = ("g" in inp) if epilogue is None else epilogue
    d = {n: to_dev(inp.get(n), io_t) for n in ("q", "k", "v", "g", "conv_in")}
    la = to_dev(inp["log_alpha"], torch.float32)
    b = to_dev(inp["beta"], torch.float32)
    cu = to_dev(inp["cu_seqlens"].astype(np.int32), torch.int32)
    cw = to_dev(inp.get("conv_w"), torch.float32) if prologue else None
    s0 = to_dev(inp.get("state_in"), torch.float32)
    rw = to_dev(rms_w, torch.float32)
    cfg = kda.config(inp["q"].shape[1], io_dtype=io, out_dtype=out, prologue=prologue,
                     epilogue=epilogue, algo=algo, gate=gate, beta_mode=beta_mode)
    kw = {}
    if in_place and s0 is not None:
        kw["state_out"] = s0
    if in_place and d["conv_in"] is not None:
        kw["conv_out"] = d["conv_in"]
    if stream is not None:
        kw["stream"] = stream
    o, s, c = kda.prefill(d["q"], d["k"], d["v"], la, b, cu, g=d["g"] if epilogue else None,
                          conv_w=cw, conv_in=d["conv_in"] if prologue else None, rms_w=rw,
                          state_in=s0, cfg=cfg, **kw)
    if churn:
        # allocations and writes on the current stream while the call may still run on
        # `stream`: memory the call freed early would be handed out and overwritten here
        for _ in range(8):
            torch.full((1 << 20,), -7.0, device=o.device).add_(1.0)
    torch.cuda.synchronize()
    if keep_device:
        return o, s, c
    return dict(o=to_np(o), state=to_np(s), conv=to_np(c))


def subset(inp: Dict[str, np.ndarray], seqs: Sequence[int], heads: Sequence[int]) -> Dict[str, np.ndarray]:
    """The inputs of a subset of sequences and heads (they do not interact)."""
    cu = inp["cu_seqlens"].astype(np.int64)
    seqs = list(seqs); heads = list(heads)
    tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs]) if seqs else np.zeros(0, np.int64)
    lens = [int(cu[n + 1] - cu[n]) for n in seqs]
    out = {"cu_seqlens": np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)}
    for n in ("q", "k", "v", "g", "log_alpha"):
        if n in inp:
            out[n] = inp[n][tok][:, heads]
    out["beta"] = inp["beta"][tok][:, heads]
    ch = np.concatenate([np.arange(h * W.D, (h + 1) * W.D) for h in heads])
    if "conv_w" in inp:
        out["conv_w"] = inp["conv_w"][:, ch]
    if "conv_in" in inp:
        out["conv_in"] = inp["conv_in"][seqs][:, :, :, ch]
    if "state_in" in inp:
        out["state_in"] = inp["state_in"][seqs][:, heads]
    return out


def oracle_prefill(inp: Dict[str, np.ndarray], prologue: Optional[bool] = None,
                   epilogue: Optional[bool] = None, rms_w=None, threads=None):
    prologue = ("conv_w" in inp) if prologue is None else prologue
    epilogue = ("g" in inp) if epilogue is None else epilogue
    o, s, c = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                             inp["cu_seqlens"], g=inp.get("g") if epilogue else None,
                             conv_w=inp.get("conv_w") if prologue else None,
                             conv_in=inp.get("conv_in") if prologue else None, rms_w=rms_w,
                             state_in=inp.get("state_in"), prologue=prologue, epilogue=epilogue,
                             threads=threads)
    return dict(o=o, state=s, conv=c)


def gpu_rows(res: Dict[str, np.ndarray], inp: Dict[str, np.ndarray], seqs, heads):
    """Restrict full GPU results to the subset used by `subset`."""
    cu = inp["cu_seqlens"].astype(np.int64)
    tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs])
    ch = np.concatenate([np.arange(h * W.D, (h + 1) * W.D) for h in heads])
    out = {"o": res["o"][tok][:, list(heads)]}
    if res.get("state") is not None:
        out["state"] = res["state"][list(seqs)][:, list(heads)]
    if res.get("conv") is not None:
        out["conv"] = res["conv"][list(seqs)][:, :, :, ch]
    return out
