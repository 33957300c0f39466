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
//   2. the scan below: S_{p+1} = M_p S_p + B_p for p = 1 .. P-2, in fp32, eight
//      workgroups per (sequence, head) over its value columns, written over B_p;
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

// S_{p+1} = M_p S_p + B_p over the middle segments of one (sequence, head), for 16 of
// its 128 value columns (the columns evolve independently: M acts on the key side), so
// that eight workgroups share each (sequence, head).  The 128 x 16 slice of S_p is staged
// in LDS; thread x computes row x / 4, columns 4 (x % 4) .. +3 of the slice in fp32, with
// M_p's row read from memory four elements at a time (it stays in the caches).  B_p is
// overwritten in place with S_{p+1}, which the rerun of segment p+1 reads.
constexpr int COMBINE_COLS = 16;
constexpr int COMBINE_GROUPS = D / COMBINE_COLS;
__global__ __launch_bounds__(SCAN_THREADS) void seg_combine_kernel(const int32_t *firsts, int32_t H,
                                                                   const float *mm, float *bb) {
    __shared__ __attribute__((aligned(16))) float SS[D * COMBINE_COLS];  // S_p[:, cols]
    const int cg = blockIdx.x % COMBINE_GROUPS;
    const int nh = blockIdx.x / COMBINE_GROUPS;
    const int n = nh / H, h = nh % H;
    const int32_t first = firsts[n], np = firsts[n + 1] - firsts[n];
    if (np < 3) return;  // nothing between the first and the last segment
    const int tid = threadIdx.x;
    const int r = tid >> 2, c0 = 4 * (tid & 3);   // output row, first of 4 columns of the slice
    const int col = cg * COMBINE_COLS;
    const size_t mat = static_cast<size_t>(D) * D;
    // S_1, left by segment 0's run in its B slot
    {
        const float *src = bb + (static_cast<size_t>(first) * H + h) * mat;
        *reinterpret_cast<float4 *>(SS + r * COMBINE_COLS + c0) =
            *reinterpret_cast<const float4 *>(src + static_cast<size_t>(r) * D + col + c0);
    }
    __syncthreads();
    for (int32_t q = 1; q + 1 < np; ++q) {
        const size_t off = (static_cast<size_t>(first + q) * H + h) * mat;
        const float *m = mm + off + static_cast<size_t>(r) * D;
        float *const b = bb + off + static_cast<size_t>(r) * D + col + c0;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k0 = 0; k0 < D; k0 += 4) {
            const float4 m4 = *reinterpret_cast<const float4 *>(m + k0);
            const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float4 s4 = *reinterpret_cast<const float4 *>(SS + (k0 + kk) * COMBINE_COLS + c0);
                acc[0] = fmaf(mv[kk], s4.x, acc[0]);
                acc[1] = fmaf(mv[kk], s4.y, acc[1]);
                acc[2] = fmaf(mv[kk], s4.z, acc[2]);
                acc[3] = fmaf(mv[kk], s4.w, acc[3]);
            }
        }
        const float4 b4 = *reinterpret_cast<const float4 *>(b);
        const float4 nx = make_float4(acc[0] + b4.x, acc[1] + b4.y, acc[2] + b4.z, acc[3] + b4.w);
        *reinterpret_cast<float4 *>(b) = nx;
        __syncthreads();  // every thread is done with SS
        *reinterpret_cast<float4 *>(SS + r * COMBINE_COLS + c0) = nx;
        __syncthreads();  // SS holds the slice of S_{q+1}
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
    hipLaunchKernelGGL(seg_combine_kernel, dim3(num_seqs * p.H * COMBINE_GROUPS), dim3(SCAN_THREADS), 0, s, firsts,
                       p.H, p.seg_m, p.seg_b);
    e = stage(hipGetLastError(), "combine");
    if (e != hipSuccess) return e;
    p.seg_pass = 3;
    return stage(launch_chunked_segments(p, out_dtype, seg_slots * p.H, s), "rerun");
}

}  // namespace kda
