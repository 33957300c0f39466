// kda_internal.h -- declarations shared by the host dispatcher and the
// kernels of libkda.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

constexpr int D = KDA_HEAD_DIM;  // d_k = d_v = 128
constexpr int CONV_HIST = 3;     // kernel size 4 minus the current token

// One segment of a sequence in the segmented prefill (KDA_ALGO_CHUNKED_SCAN).
struct SegDesc {
    int32_t n;      // sequence, or -1 for an unused slot
    int32_t ts;     // first token of the segment, counted from the start of the sequence
    int32_t len;    // tokens in the segment
    int32_t p;      // index of the segment within its sequence
    int32_t np;     // segments of the sequence
    int32_t first;  // slot of the sequence's segment 0
    int32_t pad0, pad1;
};

// Everything a kernel needs to know about one call.  Pointers are device
// pointers; activations are token-major [tokens][H][128].
struct LayerParams {
    int32_t H;
    int32_t num_items;           // work items = sequences (or requests) x heads
    const int32_t *cu_seqlens;   // prefill: [N+1]; decode: NULL (one token per request)
    const int32_t *slots_in;     // row of state_in / conv_in of each sequence or request (NULL = identity)
    const int32_t *slots_out;    // row of state_out / conv_out of each sequence or request (NULL = identity)
    const int32_t *order;        // prefill: longest-first sequence order (NULL = identity)
    const void *q, *k, *v, *g;
    const float *log_alpha, *beta;
    const float *conv_w, *rms_w;
    const void *conv_in;
    void *conv_out;
    const float *state_in;
    float *state_out;
    void *o;
    float scale, l2_eps, rms_eps;
    int32_t prologue, epilogue;
    int32_t beta_logit;          // beta holds the pre-activation w: the kernels form sigmoid(w)
    // KDA_GATE_LOWRANK: log alpha = -5 sigmoid(e^{A_h} (z W^T + b)) formed in the kernel;
    // KDA_GATE_LOWRANK_SOFTPLUS: log alpha = -e^{A_h} softplus(z W^T + b)
    int32_t gate, gate_rank;
    const void *gate_z;          // [tokens][r] io dtype
    const void *gate_w;          // [H*128][r] io dtype
    const float *gate_bias;      // [H*128]
    const float *gate_a;         // [H]
    // segmented prefill: the segment table, the pass (1: first segments, M and B of the
    // middle ones; 3: the rerun of segments 1 ..), slots in the table, and the per (slot,
    // head) fp32 [128][128] matrices M and B (B later holds the state entering slot + 1)
    const SegDesc *seg;
    int32_t seg_pass, seg_slots;
    float *seg_m, *seg_b;
};

// ---------------------------------------------------------------- launchers
hipError_t launch_recurrent(const LayerParams &p, int io_dtype, int out_dtype, hipStream_t s);
// bf16 io only (checked by the caller)
hipError_t launch_chunked_throughput(const LayerParams &p, int out_dtype, hipStream_t s);
hipError_t launch_order(const int32_t *cu_seqlens, int32_t n, int32_t *order, hipStream_t s);
// one pass of the segmented prefill over grid workgroups (bf16 io)
hipError_t launch_chunked_segments(const LayerParams &p, int out_dtype, int grid, hipStream_t s);
// the segmented prefill: table, first pass, scan of the segment transitions, rerun
hipError_t launch_chunked_scan(LayerParams p, int out_dtype, int32_t num_seqs, int32_t seg_tokens,
                               int32_t seg_slots, void *workspace, hipStream_t s);
size_t scan_workspace_bytes(int32_t num_heads, int32_t num_seqs, int32_t seg_slots);
size_t order_workspace_bytes(int32_t n);

// ------------------------------------------------------------ device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct IoTraits;
template <> struct IoTraits<float> {
    static __device__ __forceinline__ float load(const void *p, size_t i) {
        return static_cast<const float *>(p)[i];
    }
    static __device__ __forceinline__ void store(void *p, size_t i, float x) {
        static_cast<float *>(p)[i] = x;
    }
};
template <> struct IoTraits<uint16_t> {  // bf16 stored as raw bits
    static __device__ __forceinline__ float load(const void *p, size_t i) {
        return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
    }
    static __device__ __forceinline__ void store(void *p, size_t i, float x) {
        static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
    }
};

// sigma(x) and x * sigma(x) with the hardware reciprocal (about 1 ulp) in place of
// an IEEE division; exp(-x) overflowing to inf gives the correct limit 0.
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

}  // namespace kda
