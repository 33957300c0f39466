"""Benchmark of the KDA layer core on one MI355X.

One step is one pass of the whole hot path: a full-layer prefill (conv4 +
SiLU + L2 prologue, chunked recurrence, sigma(g) * RMSNorm epilogue) over
4 sequences x 4096 tokens x 96 heads (bf16 q, k, v, g; fp32 gates; S0 = 0),
followed by one decode step for 256 requests x 96 heads that updates a
[256, 96, 128, 128] fp32 state in place.

Printed (one JSON line): prefill tokens/s as `value`, decode state GB/s
(2 * B * H * 128^2 * 4 bytes per step / step time) beside it, a roofline
entry for each kernel (algorithmic bytes per launch / mean launch time, from
HIP events on the launch stream), and the fp64 CPU oracle timed on one
sequence of the same workload on the host's cores.  Also in the line: first,
the measured ceilings of this GPU (a streaming HBM copy, an HBM read stream
and a loop of bf16 matrix-core instructions), against which every fraction
is also given beside the vendor's spec peaks; then, before the step loop,
the long-context prefill (1 x 131072 tokens x 96 heads, random S0) and the
packed variable-length prefill (64 lognormal lengths, 578k tokens,
per-sequence S0), each with its roofline fractions.

    python bench.py [--steps K] [--warmup W] [--algo auto|chunked|recurrent] [--no-long]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA
D = 128


def prefill_algorithmic_bytes(T: int, H: int, N: int, gate_rank: int = 0, head_gate: bool = False) -> int:
    """Bytes the prefill must move: per token-head q, k, v, g (bf16, 4 x 256 B),
    log alpha (fp32, 512 B), beta (4 B) and o (bf16, 256 B) = 1796 B; per
    (sequence, head) the 64 KiB fp32 final state; the fp32 conv weights
    (3 x H*128 x 4) and the bf16 conv cache out (N x 3 x 3 x H*128).  With the
    in-kernel low-rank gate of rank r (gate_rank > 0) log alpha is replaced by
    z_down (bf16, T x r), W_up (bf16, H*128 x r), b_alpha and A.  With the scalar per-head
    gate (head_gate) log alpha is one fp32 value per token-head (4 B)."""
    la = 0 if gate_rank else (4 if head_gate else 4 * D)
    per_token_head = 4 * 2 * D + la + 4 + 2 * D
    gate = T * gate_rank * 2 + H * D * gate_rank * 2 + H * D * 4 + H * 4 if gate_rank else 0
    return (T * H * per_token_head + N * H * D * D * 4 + 3 * H * D * 4 * 4 +
            N * 9 * H * D * 2 + gate)


def decode_algorithmic_bytes(B: int, H: int) -> int:
    """Bytes one decode step must move: the fp32 state read and written
    (2 x 64 KiB per (request, head)), q, k, v, g in and o out (bf16), log alpha
    (fp32) and beta, the conv cache read and written (bf16, 3 x 3 x H*128 per
    request) and the conv weights."""
    state = 2 * B * H * D * D * 4
    act = B * H * (5 * D * 2 + D * 4 + 4)
    conv = 2 * B * 9 * H * D * 2 + 3 * H * D * 4 * 4
    return state + act + conv


def prefill_mfma_flops(T: int, H: int, C: int = 16) -> int:
    """Matrix-core flops of the chunked algorithm at the kernel's chunk of C = 16 tokens,
    per token-head (each contraction counted once, not the three bf16 products that
    split operands take): X = V - Kbar S, Qbar S and the state update, 3 x 2 d^2; the
    Gram blocks A and P, 2 x 2 C d; U = T X and P U, 2 x 2 C d.  = 114,688 at C = 16."""
    return T * H * (6 * D * D + 8 * C * D)


def prefill_mfma_flops_ref(T: int, H: int, C: int = 64) -> int:
    """The reference matrix-core count of the chunked form at 64-token chunks with 16-token
    triangles, 6 d^2 + 5 (C + 16) d = 149,504 per token-head: the figure the work was
    scoped with, reported beside the kernel's own count for comparison."""
    return T * H * (6 * D * D + 5 * (C + 16) * D)


def measure_peaks(dev, stream, log, gib: int = 2) -> dict:
    """This GPU's measured ceilings (libkda_peaks.so): a streaming copy of `gib` GiB (bytes
    read + written / time), a read stream of the same size, and a loop of independent
    v_mfma_f32_16x16x32_bf16 chains on every SIMD (dense bf16 flops / time).  Each is the
    best of 5 timed launches after 2 warm-up launches."""
    import ctypes
    import torch
    from gated_delta_rule_kda_amd import _build
    L = ctypes.CDLL(_build.PEAKS_LIB)
    for f in (L.kda_peak_copy, L.kda_peak_read, L.kda_peak_mfma):
        f.restype = ctypes.c_int
    L.kda_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    L.kda_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.kda_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    nbytes = gib << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    blocks = 256 * 32  # 8192 groups: the fastest copy of a sweep from 1024 to 32768
    red = torch.empty(blocks, dtype=torch.int32, device=dev)
    mblocks, iters = 256 * 8, 4096
    mout = torch.empty(mblocks * 4, dtype=torch.float32, device=dev)
    sp = stream.cuda_stream

    def best(fn):
        for _ in range(2):
            assert fn() == 0
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            assert fn() == 0
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return min(ts)

    t_copy = best(lambda: L.kda_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks, sp))
    t_read = best(lambda: L.kda_peak_read(src.data_ptr(), nbytes, red.data_ptr(), blocks, sp))
    t_mfma = best(lambda: L.kda_peak_mfma(mout.data_ptr(), mblocks, iters, sp))
    flops = mblocks * 4 * iters * 8 * 16 * 16 * 32 * 2
    copy_gbps, read_gbps = 2 * nbytes / (t_copy * 1e-3) / 1e9, nbytes / (t_read * 1e-3) / 1e9
    out = {"hbm_GBps": max(copy_gbps, read_gbps), "hbm_copy_GBps": copy_gbps, "hbm_read_GBps": read_gbps,
           "mfma_bf16_TFLOPs": flops / (t_mfma * 1e-3) / 1e12,
           "how": f"best of 5: {gib} GiB nontemporal 16-byte copy (bytes read + written) and read streams "
                  f"over {blocks} 256-thread groups, hbm_GBps the faster; {mblocks * 4} waves x {iters} x 8 "
                  f"independent 16x16x32 bf16 MFMAs"}
    log(f"measured ceilings: copy {copy_gbps:.0f} GB/s, read {read_gbps:.0f} GB/s, "
        f"bf16 MFMA {out['mfma_bf16_TFLOPs']:.0f} TFLOP/s")
    del src, dst, red, mout
    torch.cuda.empty_cache()
    return out


def cpu_info() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


KERNEL_SOURCES = {
    "prefill": ["gated_delta_rule_kda_amd/csrc/kda_chunked.hip", "gated_delta_rule_kda_amd/csrc/kda_chunk_common.h",
                "gated_delta_rule_kda_amd/csrc/kda_internal.h"],
    "decode": ["gated_delta_rule_kda_amd/csrc/kda_recurrent.hip", "gated_delta_rule_kda_amd/csrc/kda_internal.h"],
}


def source_digest(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(path: str) -> dict:
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE passes
    (scaled by the same counters on a copy of known size), per kernel, kept only
    while the kernel's sources hash to what they were when the counters were taken."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    out = {}
    for kind, entry in rec.get("kernels", {}).items():
        if kind in KERNEL_SOURCES and entry.get("source_sha256") == source_digest(KERNEL_SOURCES[kind]):
            out[kind] = entry.get("hbm_bytes_per_launch")
    return out


def oracle_single_thread(W, oracle, decode_sample: int = 16) -> dict:
    """The oracle on one thread: the whole 256-token x 2-head core case (fp32 io, no
    projections around the recurrence), and the first `decode_sample` requests of the
    256-request decode step (all 96 heads, full layer), scaled to requests per second."""
    out = {}
    spec = W.workload("core_fp32")
    x = W.gen_prefill(spec)
    t0 = time.perf_counter()
    oracle.prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"],
                   prologue=False, epilogue=False, threads=1)
    ct = time.perf_counter() - t0
    T = int(x["cu_seqlens"][-1])
    out["core_fp32"] = {"value": T / ct, "unit": "tokens/s", "ms": ct * 1e3, "cores": 1,
                        "sample": f"whole workload: {T} tokens x {spec.heads} heads"}
    dspec = W.workload("decode_256")
    y = W.gen_decode(dspec)
    b = min(decode_sample, dspec.batch)
    t0 = time.perf_counter()
    oracle.decode_step(y["q"][:b], y["k"][:b], y["v"][:b], y["log_alpha"][:b], y["beta"][:b],
                       y["state"][:b], g=y["g"][:b], conv_w=y["conv_w"],
                       conv_state=y["conv_state"][:b], threads=1)
    ct = time.perf_counter() - t0
    out["decode_256"] = {"value": b / ct, "unit": "requests/s", "ms_per_step": dspec.batch / b * ct * 1e3,
                         "cores": 1, "sample": f"{b} of {dspec.batch} requests x {dspec.heads} heads, "
                                               f"scaled to the whole step"}
    return out


def time_long_workload(kda, W, dev, stream, log, name, spec, algos, reps=3, warmup=1, hold=None) -> dict:
    """Time one long prefill workload (all sequences start from a random S0): inputs are
    generated one sequence at a time (the seeded generator the parity tests use) straight
    into device buffers; each algorithm in `algos` is run `warmup` times, then timed over
    `reps` launches with HIP events.  With a list `hold`, the device buffers are appended
    to it rather than freed."""
    import torch
    out = {}
    lens = [int(x) for x in spec.lens]
    N, H, T = len(lens), spec.heads, int(sum(lens))
    bf = torch.bfloat16
    bufs = {k: torch.empty((T, H, D), dtype=bf, device=dev) for k in ("q", "k", "v", "g")}
    la = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    beta = torch.empty((T, H), dtype=torch.float32, device=dev)
    s0 = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    t0 = time.perf_counter()
    off = 0
    cw = None
    for n, L in enumerate(lens):
        x = W.gen_prefill(W.PrefillSpec(lens=[L], heads=H, state_std=spec.state_std, seed=spec.seed,
                                        first_seq=n))
        for k in bufs:
            bufs[k][off:off + L].copy_(torch.from_numpy(x[k]).to(bf))
        la[off:off + L].copy_(torch.from_numpy(x["log_alpha"]))
        beta[off:off + L].copy_(torch.from_numpy(x["beta"]))
        s0[n].copy_(torch.from_numpy(x["state_in"][0]))
        cw = x["conv_w"]
        off += L
    log(f"{name}: generated {T} tokens in {time.perf_counter() - t0:.1f}s")
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=dev)
    cwd = torch.from_numpy(cw).to(dev)
    o = torch.empty((T, H, D), dtype=bf, device=dev)
    s_out = torch.empty_like(s0)
    for a in algos:
        cfg = kda.config(H, io_dtype="bf16", out_dtype="bf16", prologue=True, epilogue=True, algo=a)
        ws_n = kda.workspace_size(cfg, N, T)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

        def run():
            kda.prefill(bufs["q"], bufs["k"], bufs["v"], la, beta, cu, g=bufs["g"], conv_w=cwd,
                        state_in=s0, o=o, state_out=s_out, workspace=ws if ws_n else None, cfg=cfg,
                        stream=stream, return_conv=False)

        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        ms, med = time_events(run, reps, stream)
        nb = prefill_algorithmic_bytes(T, H, N) + N * H * D * D * 4  # + the initial states read
        key = name if a == algos[0] else f"{name}_{a}"
        ran = kda.resolved_algo(cfg, N, T)
        out[key] = {"workload": f"{N} x {lens[0] if len(set(lens)) == 1 else 'lognormal'} tokens, H={H}, d=128, full layer, "
                                f"bf16 io, random fp32 S0", "tokens": T, "sequences": N, "heads": H,
                    "max_len": max(lens), "algo": ran, "ms": ms, "ms_median": med, "reps": reps,
                    "tokens_per_s": T / (ms * 1e-3), "algorithmic_bytes": nb,
                    "GBps": nb / (ms * 1e-3) / 1e9,
                    "frac_of_hbm_roofline": nb / (ms * 1e-3) / (HBM_PEAK_GBPS * 1e9)}
        log(f"{key} ({ran}): {ms:.2f} ms, {T / (ms * 1e-3) / 1e6:.2f} M tokens/s")
        del ws
    if hold is not None:
        hold.append((bufs, la, beta, s0, o, s_out))
    del bufs, la, beta, s0, o, s_out
    if hold is None:
        torch.cuda.empty_cache()
    return out


def run_extra_workloads(kda, W, dev, stream, log, algo="auto") -> dict:
    """The long context in one sequential pass (the chunked kernel, next to AUTO's
    segmented prefill in the main line) and at 12 heads (one GPU's share of 96 heads split
    eight ways), by AUTO and in one pass; and the 4 x 4096 prefill at 12 heads, by AUTO
    (the segmented prefill) and in one pass."""
    import dataclasses
    out = {}
    long12 = dataclasses.replace(W.workload("prefill_131072"), heads=12, name="prefill_131072_h12")
    out.update(time_long_workload(kda, W, dev, stream, log, "prefill_131072_one_pass", W.workload("prefill_131072"),
                                  ["chunked_throughput"]))
    out.update(time_long_workload(kda, W, dev, stream, log, "prefill_131072_h12", long12,
                                  [algo, "chunked_throughput"]))
    share12 = dataclasses.replace(W.workload("prefill_4x4096"), heads=12, state_std=0.02, name="prefill_4x4096_h12")
    out.update(time_long_workload(kda, W, dev, stream, log, "prefill_4x4096_h12", share12,
                                  [algo, "chunked_throughput"], reps=20, warmup=20))
    return out


def run_lowrank_gate_workload(kda, W, dev, stream, log, rank=128, softplus=False, wild_every=0) -> dict:
    """The 4 x 4096 x 96 prefill with log alpha formed in the kernel from rank-`rank`
    gate factors (the fp32 log alpha stream is not read): K3's floored gate, or Kimi
    Linear's unbounded softplus gate (softplus), with every `wild_every`-th head decaying
    fast enough to take its chunks off the matrix cores."""
    import torch
    spec = W.workload("prefill_4x4096")
    x = W.gen_prefill(spec)
    if softplus:
        wild = tuple(range(0, spec.heads, wild_every)) if wild_every else ()
        gate = W.gen_softplus_gate(x["cu_seqlens"], spec.heads, rank, seed=spec.seed, wild_heads=wild)
    else:
        gate = W.gen_gate(x["cu_seqlens"], spec.heads, rank, seed=spec.seed)
    bf = torch.bfloat16
    T, H, N = x["q"].shape[0], spec.heads, len(spec.lens)
    t = {n: torch.from_numpy(x[n]).to(dev).to(bf) for n in ("q", "k", "v", "g")}
    del x["log_alpha"]
    beta = torch.from_numpy(x["beta"]).to(dev)
    cu = torch.from_numpy(x["cu_seqlens"].astype(np.int32)).to(dev)
    cw = torch.from_numpy(x["conv_w"]).to(dev)
    gz, gw = (torch.from_numpy(gate[n]).to(dev).to(bf) for n in ("gate_z", "gate_w"))
    gb, ga = (torch.from_numpy(gate[n]).to(dev) for n in ("gate_bias", "gate_a"))
    cfg = kda.config(H, io_dtype="bf16", out_dtype="bf16", gate="lowrank_softplus" if softplus else "lowrank",
                     gate_rank=rank)
    o = torch.empty((T, H, D), dtype=bf, device=dev)
    s_out = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    c_out = torch.empty((N, 3, 3, H * D), dtype=bf, device=dev)
    ws = torch.empty(max(kda.workspace_size(cfg, N, T), 1), dtype=torch.uint8, device=dev)

    def run():
        kda.prefill(t["q"], t["k"], t["v"], None, beta, cu, g=t["g"], conv_w=cw, o=o, state_out=s_out,
                    conv_out=c_out, gate_z=gz, gate_w=gw, gate_bias=gb, gate_a=ga, workspace=ws, cfg=cfg,
                    stream=stream)

    warm_up(run)
    ms, _ = time_events(run, 20, stream)
    nb = prefill_algorithmic_bytes(T, H, N, gate_rank=rank)
    name = "prefill_4x4096_" + (f"softplus_gate_wild{wild_every}" if softplus else "lowrank_gate")
    log(f"{name} (r={rank}): {ms:.3f} ms, {T / (ms * 1e-3) / 1e6:.2f} M tokens/s")
    return {name: {"tokens": T, "rank": rank, "ms": ms, "tokens_per_s": T / (ms * 1e-3),
                   "algorithmic_bytes": nb, "frac_of_hbm_roofline": nb / (ms * 1e-3) / (HBM_PEAK_GBPS * 1e9)}}


def run_head_gate_workload(kda, W, dev, stream, log) -> dict:
    """The 4 x 4096 x 96 prefill with one decay per (token, head) instead of one per key
    channel (log alpha [T, H]: channel 0 of the channel-wise workload's values)."""
    import torch
    spec = W.workload("prefill_4x4096")
    x = W.gen_prefill(spec)
    bf = torch.bfloat16
    T, H, N = x["q"].shape[0], spec.heads, len(spec.lens)
    t = {n: torch.from_numpy(x[n]).to(dev).to(bf) for n in ("q", "k", "v", "g")}
    la = torch.from_numpy(np.ascontiguousarray(x["log_alpha"][..., 0])).to(dev)
    del x["log_alpha"]
    beta = torch.from_numpy(x["beta"]).to(dev)
    cu = torch.from_numpy(x["cu_seqlens"].astype(np.int32)).to(dev)
    cw = torch.from_numpy(x["conv_w"]).to(dev)
    cfg = kda.config(H, io_dtype="bf16", out_dtype="bf16", gate="head")
    o = torch.empty((T, H, D), dtype=bf, device=dev)
    s_out = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    c_out = torch.empty((N, 3, 3, H * D), dtype=bf, device=dev)
    ws = torch.empty(max(kda.workspace_size(cfg, N, T), 1), dtype=torch.uint8, device=dev)

    def run():
        kda.prefill(t["q"], t["k"], t["v"], la, beta, cu, g=t["g"], conv_w=cw, o=o, state_out=s_out,
                    conv_out=c_out, workspace=ws, cfg=cfg, stream=stream)

    warm_up(run)
    ms, _ = time_events(run, 20, stream)
    nb = prefill_algorithmic_bytes(T, H, N, head_gate=True)
    log(f"prefill_4x4096 per-head gate: {ms:.3f} ms, {T / (ms * 1e-3) / 1e6:.2f} M tokens/s")
    return {"prefill_4x4096_head_gate": {"tokens": T, "ms": ms, "tokens_per_s": T / (ms * 1e-3),
                                         "algorithmic_bytes": nb,
                                         "frac_of_hbm_roofline": nb / (ms * 1e-3) / (HBM_PEAK_GBPS * 1e9)}}


def run_serving_workloads(kda, dev, stream, log, H=96, B=256, drafts=4) -> dict:
    """Serving-state calls on synthetic device inputs (seeded torch draws with the
    workloads' value ranges): a copy-on-write decode step (B requests read checkpoint rows
    of a state pool and write other rows), and one speculative round: verification of
    `drafts` tokens per request from the committed rows (nothing written), then an
    in-place replay of accepted prefixes of random length 0 .. drafts."""
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    bf = torch.bfloat16

    def normal(*shape, std=1.0, dtype=bf):
        return (torch.randn(*shape, generator=gen, device=dev) * std).to(dtype)

    def gates(*shape):
        la = -5.0 * torch.sigmoid(torch.randn(*shape, D, generator=gen, device=dev))
        beta = torch.sigmoid(torch.randn(*shape, generator=gen, device=dev))
        return la.contiguous(), beta.contiguous()

    out = {}
    rows = 2 * B
    pool = normal(rows, H, D, D, std=0.02, dtype=torch.float32)
    conv = normal(rows, 3, 3, H * D)
    cw = normal(3, H * D, 4, std=0.5, dtype=torch.float32)
    perm = torch.randperm(rows, generator=gen, device=dev).to(torch.int32)
    s_in, s_out = perm[:B].contiguous(), perm[B:].contiguous()
    q, k, v, g = (normal(B, H, D) for _ in range(4))
    la, beta = gates(B, H)
    o = torch.empty((B, H, D), dtype=bf, device=dev)
    cfg = kda.config(H, io_dtype="bf16", out_dtype="bf16", prologue=True, epilogue=True)

    def cow():
        kda.decode_step(q, k, v, la, beta, pool, g=g, conv_w=cw, conv_state=conv, slots=s_in,
                        slots_out=s_out, o=o, cfg=cfg, stream=stream)

    warm_up(cow)
    ms, _ = time_events(cow, 20, stream)
    out["decode_copy_on_write"] = {"requests": B, "heads": H, "ms": ms,
                                   "state_GBps": 2 * B * H * D * D * 4 / (ms * 1e-3) / 1e9}
    log(f"decode copy-on-write: {ms:.4f} ms, {out['decode_copy_on_write']['state_GBps']:.0f} GB/s of state")

    T = B * drafts
    dq, dk, dv, dg = (normal(T, H, D) for _ in range(4))
    dla, dbeta = gates(T, H)
    cu = torch.arange(0, T + 1, drafts, dtype=torch.int32, device=dev)
    acc = torch.randint(0, drafts + 1, (B,), generator=gen, device=dev)
    cu_acc = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    cu_acc[1:] = torch.cumsum(acc, 0).to(torch.int32)
    Ta = int(cu_acc[-1].item())
    idx = torch.cat([torch.arange(i * drafts, i * drafts + int(a), device=dev) for i, a in enumerate(acc.tolist())])
    aq, ak, av, ag = (t[idx].contiguous() for t in (dq, dk, dv, dg))
    ala, abeta = dla[idx].contiguous(), dbeta[idx].contiguous()
    o_ver = torch.empty((T, H, D), dtype=bf, device=dev)
    o_acc = torch.empty((max(Ta, 1), H, D), dtype=bf, device=dev)[:Ta]
    ws = torch.empty(max(kda.workspace_size(cfg, B, T), 1), dtype=torch.uint8, device=dev)
    slots = s_in

    def verify():
        kda.prefill(dq, dk, dv, dla, dbeta, cu, g=dg, conv_w=cw, conv_in=conv, state_in=pool, o=o_ver,
                    state_in_slots=slots, workspace=ws, cfg=cfg, return_state=False, return_conv=False,
                    stream=stream)

    def replay():
        kda.prefill(aq, ak, av, ala, abeta, cu_acc, g=ag, conv_w=cw, conv_in=conv, conv_out=conv,
                    state_in=pool, state_out=pool, o=o_acc, state_in_slots=slots, state_out_slots=slots,
                    workspace=ws, cfg=cfg, stream=stream)

    warm_up(verify)
    vms, _ = time_events(verify, 20, stream)
    warm_up(replay, 5)
    rms_, _ = time_events(replay, 20, stream)
    out["speculative_round"] = {"requests": B, "heads": H, "draft_tokens": drafts, "accepted_tokens": Ta,
                                "verify_ms": vms, "replay_ms": rms_,
                                "verified_tokens_per_s": T / (vms * 1e-3)}
    log(f"speculative round: verify {T} tokens {vms:.3f} ms, replay {Ta} tokens {rms_:.3f} ms")
    del pool, conv

    # Small batches, where a step's launch costs as much as its state traffic: `steps`
    # decode steps launched one by one, against the same steps captured once in a HIP graph.
    steps = 32
    for Bs in (1, 8):
        pool_s = normal(Bs, H, D, D, std=0.02, dtype=torch.float32)
        conv_s = normal(Bs, 3, 3, H * D)
        sq, sk, sv, sg = (normal(Bs, H, D) for _ in range(4))
        sla, sbeta = gates(Bs, H)
        so = torch.empty((Bs, H, D), dtype=bf, device=dev)

        def small_step(s):
            kda.decode_step(sq, sk, sv, sla, sbeta, pool_s, g=sg, conv_w=cw, conv_state=conv_s, o=so,
                            cfg=cfg, stream=s)

        def eager_loop():
            for _ in range(steps):
                small_step(stream)

        warm_up(eager_loop, 3)
        ems, _ = time_events(eager_loop, 10, stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):  # the binding launches on the capturing stream
            for _ in range(steps):
                small_step(None)

        def graph_loop():
            with torch.cuda.stream(stream):
                graph.replay()

        warm_up(graph_loop, 3)
        gms, _ = time_events(graph_loop, 10, stream)
        state_bytes = 2 * Bs * H * D * D * 4
        out[f"decode_{Bs}x{H}_graph"] = {
            "requests": Bs, "heads": H, "steps": steps,
            "eager_us_per_step": ems * 1e3 / steps, "graph_us_per_step": gms * 1e3 / steps,
            "graph_state_GBps": state_bytes * steps / (gms * 1e-3) / 1e9}
        log(f"decode {Bs} x {H}: {ems * 1e3 / steps:.1f} us per step launched one by one, "
            f"{gms * 1e3 / steps:.1f} us in a HIP graph of {steps} steps")
        del graph, pool_s, conv_s
    torch.cuda.empty_cache()
    return out


def warm_up(fn, n: int = 20):
    """n untimed calls, then a device synchronisation: the clocks of a fresh box settle over
    the first launches (up to 20% slower than later ones)."""
    import torch
    for _ in range(n):
        fn()
    torch.cuda.synchronize()


def time_events(fn, steps: int, stream):
    """Mean ms of fn() over `steps` calls, from HIP events recorded on `stream`."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return float(np.mean(ts)), float(np.median(ts))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--algo", default="auto",
                    choices=["auto", "recurrent", "chunked", "chunked_throughput"])
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context and variable-length prefills and the measured ceilings "
                         "(profiling runs of the main step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run one fp32 device copy of this many MiB after the timed region "
                         "(the known-size reference for HBM byte counters)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="counter-derived HBM bytes per launch, used while the kernel sources "
                         "they were measured on are unchanged")
    ap.add_argument("--extra-workloads", action="store_true",
                    help="also time the long context in one pass and at 12 heads, the gate variants "
                         "and the serving cases")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the KDA core shards by head and by request with no "
              f"collective inside it, and this build runs on a single MI355X; --gpus {args.gpus} "
              f"is not supported.", file=sys.stderr)
        return 2

    import torch
    import gated_delta_rule_kda_amd as kda
    import kda_workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    bf = torch.bfloat16

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- prefill inputs
    spec = W.workload("prefill_4x4096")
    t0 = time.perf_counter()
    x = W.gen_prefill(spec)
    log(f"generated prefill inputs in {time.perf_counter() - t0:.1f}s")
    T, H, N = spec.total, spec.heads, len(spec.lens)

    def dev_t(a, dt):
        return torch.from_numpy(a).to(dev).to(dt)

    q, k, v, g = (dev_t(x[n], bf) for n in ("q", "k", "v", "g"))
    la = dev_t(x["log_alpha"], torch.float32)
    beta = dev_t(x["beta"], torch.float32)
    cw = dev_t(x["conv_w"], torch.float32)
    cu = dev_t(x["cu_seqlens"], torch.int32)
    cfg = kda.config(H, io_dtype="bf16", out_dtype="bf16", prologue=True, epilogue=True,
                     algo=args.algo)
    o = torch.empty((T, H, D), dtype=bf, device=dev)
    s_out = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    c_out = torch.empty((N, 3, 3, H * D), dtype=bf, device=dev)
    ws_n = kda.workspace_size(cfg, N, T)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def run_prefill():
        kda.prefill(q, k, v, la, beta, cu, g=g, conv_w=cw, o=o, state_out=s_out, conv_out=c_out,
                    workspace=ws if ws_n else None, cfg=cfg, stream=stream)

    # ---------------------------------------------------------------- decode inputs
    dspec = W.workload("decode_256")
    t0 = time.perf_counter()
    y = W.gen_decode(dspec)
    log(f"generated decode inputs in {time.perf_counter() - t0:.1f}s")
    B = dspec.batch
    dq, dk_, dv_, dg = (dev_t(y[n], bf) for n in ("q", "k", "v", "g"))
    dla = dev_t(y["log_alpha"], torch.float32)
    dbeta = dev_t(y["beta"], torch.float32)
    dcw = dev_t(y["conv_w"], torch.float32)
    dstate = dev_t(y["state"], torch.float32)
    dconv = dev_t(y["conv_state"], bf)
    del y
    dcfg = kda.config(H, io_dtype="bf16", out_dtype="bf16", prologue=True, epilogue=True)
    do = torch.empty((B, H, D), dtype=bf, device=dev)

    def run_decode():
        kda.decode_step(dq, dk_, dv_, dla, dbeta, dstate, g=dg, conv_w=dcw, conv_state=dconv,
                        o=do, cfg=dcfg, stream=stream)

    # ---------------------------------------------------------------- this GPU's ceilings
    # (first: they characterise the machine the rest runs on)
    peaks = None if args.no_long else measure_peaks(dev, stream, log)

    # ---------------------------------------------------------------- long launches
    # The long-context and packed variable-length prefills, before the step loop, which
    # then follows them without a pause: the GPU lowers its clock within a fraction of a
    # second of idling and raises it again over tens of milliseconds of this kernel (right
    # after a 0.3 s pause the 4 x 4096 prefill measured 1.8 ms on its second launch, 1.45 ms
    # by its tenth and 1.29 ms from about its thirtieth).  Their buffers (about 100 GB) are
    # therefore freed after the step loop: the frees take long enough to idle the GPU.
    long_runs = None
    held = []
    if not args.no_long:
        long_runs = {}
        long_runs.update(time_long_workload(kda, W, dev, stream, log, "prefill_131072", W.workload("prefill_131072"),
                                            [args.algo], reps=5, warmup=2))
        long_runs.update(time_long_workload(kda, W, dev, stream, log, "varlen_64", W.workload("varlen_64"),
                                            [args.algo], reps=5, warmup=2, hold=held))
        for e in long_runs.values():
            e["frac_of_measured_hbm"] = e["GBps"] / peaks["hbm_GBps"]

    # ---------------------------------------------------------------- timing
    for _ in range(args.warmup):
        run_prefill()
        run_decode()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    t_wall0 = time.perf_counter()
    pre_mean, pre_med = time_events(run_prefill, args.steps, stream)
    dec_mean, dec_med = time_events(run_decode, args.steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    log(f"prefill {pre_mean:.3f} ms (median {pre_med:.3f}); decode {dec_mean:.4f} ms "
        f"(median {dec_med:.4f}); wall {wall:.2f}s")
    held.clear()
    torch.cuda.empty_cache()

    copy_cal = None
    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        xs = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        ys = torch.empty_like(xs)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        ys.copy_(xs)
        ev1.record(stream)
        torch.cuda.synchronize()
        copy_cal = {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ev0.elapsed_time(ev1)}
        del xs, ys

    tok_s = T / (pre_mean * 1e-3)
    pb = prefill_algorithmic_bytes(T, H, N)
    pf = prefill_mfma_flops(T, H)
    pre_gbps = pb / (pre_mean * 1e-3) / 1e9
    db = decode_algorithmic_bytes(B, H)
    state_bytes = 2 * B * H * D * D * 4
    dec_state_gbps = state_bytes / (dec_mean * 1e-3) / 1e9
    dec_gbps = db / (dec_mean * 1e-3) / 1e9
    algo_name = kda.resolved_algo(cfg, N)

    # ---------------------------------------------------------------- CPU oracle
    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        L0 = int(spec.lens[0])
        sub = {n: x[n][:L0] for n in ("q", "k", "v", "g", "log_alpha", "beta")}
        t0 = time.perf_counter()
        oracle.prefill(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"], [0, L0],
                       g=sub["g"], conv_w=x["conv_w"], threads=threads)
        ct = time.perf_counter() - t0
        cpu = {"value": L0 / ct, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"sequence 0 of the prefill workload: {L0} tokens x {H} heads, full layer, "
                         f"fp64, {ct:.1f}s wall on {threads} threads ({cpu_info()})"}
        log(f"oracle: {L0} tokens x {H} heads in {ct:.1f}s on {threads} threads")
        cpu1 = oracle_single_thread(W, oracle)
        log(f"oracle, one thread: {json.dumps(cpu1)}")

    traffic = load_traffic(args.traffic)
    extra = None
    if args.extra_workloads:
        extra = run_extra_workloads(kda, W, dev, stream, log, args.algo)
        extra.update(run_lowrank_gate_workload(kda, W, dev, stream, log))
        extra.update(run_head_gate_workload(kda, W, dev, stream, log))
        extra.update(run_lowrank_gate_workload(kda, W, dev, stream, log, softplus=True))
        extra.update(run_lowrank_gate_workload(kda, W, dev, stream, log, softplus=True, wild_every=8))
        extra.update(run_serving_workloads(kda, dev, stream, log))

    res = {
        "metric": "KDA prefill tokens/sec (H=96,d=128) + decode state GB/s at B=256",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre_mean + dec_mean,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill B=4 x T=4096, H=96, d=128, full layer (conv4+SiLU+L2, "
                               "sigma(g)*RMSNorm), bf16 io, fp32 gates and state; decode B=256, H=96",
                   "prefill_algo": algo_name, "global_batch": N, "seq_len": spec.lens[0],
                   "heads": H, "head_dim": D, "decode_batch": B},
        "prefill": {"ms": pre_mean, "ms_median": pre_med, "tokens_per_s": tok_s,
                    "algorithmic_bytes": pb, "mfma_flops_c16": pf,
                    "mfma_tflops": pf / (pre_mean * 1e-3) / 1e12,
                    "mfma_frac_of_peak": pf / (pre_mean * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                    "mfma_flops_ref_c64": prefill_mfma_flops_ref(T, H),
                    "mfma_frac_of_peak_ref_c64": prefill_mfma_flops_ref(T, H) / (pre_mean * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                    "hbm_roofline_tokens_per_s": T / (pb / (HBM_PEAK_GBPS * 1e9))},
        "decode": {"ms": dec_mean, "ms_median": dec_med, "state_GBps": dec_state_gbps,
                   "algorithmic_bytes": db, "GBps": dec_gbps,
                   "frac_of_hbm_peak": dec_gbps / HBM_PEAK_GBPS},
        "roofline": {"kernel": f"prefill ({algo_name})", "bound": "hbm", "achieved": pre_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": pre_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic.get("prefill")},
        "roofline_decode": {"kernel": "decode step", "bound": "hbm", "achieved": dec_gbps,
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dec_gbps / HBM_PEAK_GBPS,
                            "traffic": traffic.get("decode")},
        "cpu_baseline": cpu,
    }
    if peaks:
        res["measured_ceilings"] = peaks
        res["roofline"]["frac_of_measured"] = pre_gbps / peaks["hbm_GBps"]
        res["roofline_decode"]["frac_of_measured"] = dec_gbps / peaks["hbm_GBps"]
        res["prefill"]["mfma_frac_of_measured"] = pf / (pre_mean * 1e-3) / 1e12 / peaks["mfma_bf16_TFLOPs"]
    if long_runs:
        res["long_context"] = long_runs.get("prefill_131072")
        res["varlen"] = long_runs.get("varlen_64")
    if cpu1:
        res["cpu_baseline_1thread"] = cpu1
    if copy_cal:
        res["copy_calibration"] = copy_cal
    if extra:
        res["extra_workloads"] = extra
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
