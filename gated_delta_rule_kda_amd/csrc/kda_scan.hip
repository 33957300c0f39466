// kda_scan.hip -- the segmented prefill (KDA_ALGO_CHUNKED_SCAN): each long sequence is
// cut into segments that run on different compute units.
//
// One chunk of the recurrence maps its entering state affinely,
//   S -> (Diag(Gamma_C) - Khat^T T Kbar) S + Khat^T T V,
// (the per-token update of "Inside Kimi K3 ...", "KDA writes corrections into a recurrent
// matrix", regrouped over the chunk), so a segment of chunks maps S -> M S + B with
// M the product of its chunks' matrices and B its result from S = 0.  M is the
// segment's final state when it starts from S = I with v = 0, and B its final state
// from S = 0; both come out of the chunked kernel unchanged.  The passes:
//   1. segment 0 of each sequence runs from the given state (outputs included) and
//      leaves the state entering segment 1; every middle segment runs twice, for its
//      M and its B (all in one launch);
//   2. the scan below: S_{p+1} = M_p S_p + B_p for p = 1 .. P-2, in fp32, one
//      workgroup per (sequence, head), written over B_p;
//   3. segments 1 .. P-1 run again from their entering states, with outputs; the last
//      one writes the final state and conv cache.
// The same composition is what a split of one sequence over GPUs would exchange.
#include <stdio.h>
#include <stdlib.h>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int SCAN_THREADS = 512;

// Segment table: sequence n has max(1, ceil(L_n / seg)) segments in consecutive slots
// starting at firsts[n]; slots past the last segment get n = -1.
__global__ __launch_bounds__(256) void seg_table_kernel(const int32_t *cu, int32_t num_seqs, int32_t seg,
                                                        int32_t slots, int32_t *firsts, SegDesc *desc) {
    __shared__ int32_t total;
    if (threadIdx.x == 0) {
        int32_t f = 0;
        for (int32_t n = 0; n < num_seqs; ++n) {
            firsts[n] = f;
            const int32_t L = cu[n + 1] - cu[n];
            f += L > seg ? (L + seg - 1) / seg : 1;
        }
        firsts[num_seqs] = f;
        total = f;
    }
    __syncthreads();
    const int32_t used = min(total, slots);
    for (int32_t s = threadIdx.x; s < slots; s += blockDim.x) {
        SegDesc d{-1, 0, 0, 0, 0, 0, 0, 0};
        if (s < used) {
            int32_t lo = 0, hi = num_seqs - 1;  // the last n with firsts[n] <= s
            while (lo < hi) {
                const int32_t mid = (lo + hi + 1) / 2;
                if (firsts[mid] <= s) lo = mid; else hi = mid - 1;
            }
            const int32_t L = cu[lo + 1] - cu[lo];
            d.n = lo;
            d.first = firsts[lo];
            d.p = s - d.first;
            d.np = firsts[lo + 1] - d.first;
            d.ts = d.p * seg;
            d.len = min(seg, L - d.ts);
        }
        desc[s] = d;
    }
}

// S_{p+1} = M_p S_p + B_p over the middle segments of one (sequence, head).  S_p is
// staged in LDS (fp32, 64 KiB); M_p is read from memory (it stays in the caches: each
// element is read by the 16 threads of a row group).  Thread x computes rows
// 4(x/16) .. +3 and columns 8(x%16) .. +7 of the product in fp32.  B_p is overwritten in
// place with S_{p+1}, which the rerun of segment p+1 reads.
__global__ __launch_bounds__(SCAN_THREADS) void seg_combine_kernel(const int32_t *firsts, int32_t H,
                                                                   const float *mm, float *bb) {
    __shared__ __attribute__((aligned(16))) float SS[D * D];  // the current entering state
    const int n = blockIdx.x / H, h = blockIdx.x % H;
    const int32_t first = firsts[n], np = firsts[n + 1] - firsts[n];
    if (np < 3) return;  // nothing between the first and the last segment
    const int tid = threadIdx.x;
    const int i0 = 4 * (tid >> 4), j0 = 8 * (tid & 15);
    const size_t mat = static_cast<size_t>(D) * D;
    // S_1, left by segment 0's run in its B slot
    const float *src = bb + (static_cast<size_t>(first) * H + h) * mat;
    for (int e = tid; e < D * D / 4; e += SCAN_THREADS)
        reinterpret_cast<float4 *>(SS)[e] = reinterpret_cast<const float4 *>(src)[e];
    __syncthreads();
    for (int32_t q = 1; q + 1 < np; ++q) {
        const size_t off = (static_cast<size_t>(first + q) * H + h) * mat;
        const float *m = mm + off + static_cast<size_t>(i0) * D;
        float *b = bb + off;
        float acc[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[r][c] = 0.0f;
        for (int k0 = 0; k0 < D; k0 += 4) {
            float4 mr[4];  // M[i0 + r][k0 .. k0 + 3]
#pragma unroll
            for (int r = 0; r < 4; ++r) mr[r] = *reinterpret_cast<const float4 *>(m + r * D + k0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float4 s0 = *reinterpret_cast<const float4 *>(SS + (k0 + kk) * D + j0);
                const float4 s1 = *reinterpret_cast<const float4 *>(SS + (k0 + kk) * D + j0 + 4);
                const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float mv = kk == 0 ? mr[r].x : kk == 1 ? mr[r].y : kk == 2 ? mr[r].z : mr[r].w;
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(mv, sv[c], acc[r][c]);
                }
            }
        }
        __syncthreads();  // every thread is done with SS
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float4 *const bo = reinterpret_cast<float4 *>(b + static_cast<size_t>(i0 + r) * D + j0);
            float4 *const so = reinterpret_cast<float4 *>(SS + (i0 + r) * D + j0);
            const float4 b0 = bo[0], b1 = bo[1];
            const float4 n0 = make_float4(acc[r][0] + b0.x, acc[r][1] + b0.y, acc[r][2] + b0.z, acc[r][3] + b0.w);
            const float4 n1 = make_float4(acc[r][4] + b1.x, acc[r][5] + b1.y, acc[r][6] + b1.z, acc[r][7] + b1.w);
            bo[0] = n0;
            bo[1] = n1;
            so[0] = n0;
            so[1] = n1;
        }
        __syncthreads();  // SS holds S_{q+1} before the next product reads it
    }
}

constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// With KDA_TRACE set, a failed launch names its stage.
hipError_t stage(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        const char *t = getenv("KDA_TRACE");
        if (t && t[0] && t[0] != '0') fprintf(stderr, "[kda] scan %s: %s\n", what, hipGetErrorString(e));
    }
    return e;
}

}  // namespace

size_t scan_workspace_bytes(int32_t num_heads, int32_t num_seqs, int32_t seg_slots) {
    const size_t mat = static_cast<size_t>(D) * D * sizeof(float);
    return align256(static_cast<size_t>(seg_slots) * sizeof(SegDesc)) +
           align256(static_cast<size_t>(num_seqs + 1) * sizeof(int32_t)) +
           2 * static_cast<size_t>(seg_slots) * num_heads * mat;
}

hipError_t launch_chunked_scan(LayerParams p, int out_dtype, int32_t num_seqs, int32_t seg_tokens,
                               int32_t seg_slots, void *workspace, hipStream_t s) {
    char *w = static_cast<char *>(workspace);
    SegDesc *desc = reinterpret_cast<SegDesc *>(w);
    w += align256(static_cast<size_t>(seg_slots) * sizeof(SegDesc));
    int32_t *firsts = reinterpret_cast<int32_t *>(w);
    w += align256(static_cast<size_t>(num_seqs + 1) * sizeof(int32_t));
    const size_t mats = static_cast<size_t>(seg_slots) * p.H * D * D;
    p.seg = desc;
    p.seg_slots = seg_slots;
    p.seg_m = reinterpret_cast<float *>(w);
    p.seg_b = p.seg_m + mats;
    p.order = nullptr;
    hipLaunchKernelGGL(seg_table_kernel, dim3(1), dim3(256), 0, s, p.cu_seqlens, num_seqs, seg_tokens, seg_slots,
                       firsts, desc);
    hipError_t e = stage(hipGetLastError(), "segment table");
    if (e != hipSuccess) return e;
    p.seg_pass = 1;
    e = stage(launch_chunked_segments(p, out_dtype, 2 * seg_slots * p.H, s), "first pass");
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(seg_combine_kernel, dim3(num_seqs * p.H), dim3(SCAN_THREADS), 0, s, firsts, p.H, p.seg_m,
                       p.seg_b);
    e = stage(hipGetLastError(), "combine");
    if (e != hipSuccess) return e;
    p.seg_pass = 3;
    return stage(launch_chunked_segments(p, out_dtype, seg_slots * p.H, s), "rerun");
}

}  // namespace kda
