// kda_chunked.hip -- chunked KDA prefill on the gfx950 matrix cores.
//
// The per-token recurrence of the "Kimi K3 - KDA layer" step list
// (S <- Diag(alpha) S;  S <- S + beta k (v - S^T k)^T;  o~ = S^T q / sqrt(128))
// is regrouped over chunks of C = 32 tokens.  For one chunk entering with
// state S0, with G the running sum of log alpha from the chunk start
// (per key channel) and Gamma = e^G:
//
//   A[s][j] = beta_s sum_c k_s[c] k_j[c] e^{G_s[c] - G_j[c]}      (j < s)
//   P[r][j] =        sum_c q_r[c] k_j[c] e^{G_r[c] - G_j[c]}      (j <= r)
//   T       = (I + A)^{-1} Diag(beta)
//   U       = T (V - Kbar S0),            Kbar = Gamma (.) K
//   O       = scale (Qbar S0 + P U),      Qbar = Gamma (.) Q
//   S1      = Diag(Gamma_C) S0 + Khat^T U, Khat = e^{G_C - G} (.) K
//
// which is the recurrence unrolled over the chunk (u_r = beta_r (v_r -
// (Diag(alpha_r) S_{r-1})^T k_r) is the per-token correction; stacking the
// u_r gives the unit-lower triangular system (I + A) U = Diag(beta)(V -
// Kbar S0)).  The decay factors are kept finite by the 16-token sub-tile
// references of "Kimi K3's Architecture ..." (section "Channel-wise decay,
// and the floor K3 puts under it"): within a sub-tile the factors are taken
// relative to the sub-tile start, so no factor exceeds e^{5*16} = e^80.
//
// Layout of the work: one workgroup of 8 waves per (sequence, head), looping
// over the sequence's chunks.  Wave w owns value columns 16w .. 16w+15 of S
// and keeps that 128x16 fp32 slice in registers, in the accumulator layout
// of v_mfma_f32_16x16x32_bf16 (lane l holds rows 16t + 4(l/16) + i, column
// l%16).  The contractions that touch S, U or X take that layout directly
// as their B operand: the 32 K-slots of one MFMA read rows pi(8h+i) =
// 16(i/4) + 4h + (i%4) of two stacked accumulator tiles, so the A operands
// (staged in LDS) store their K index in the same permuted order.
//
// Precision: every contraction splits both operands into bf16 hi + lo parts
// and sums hi*hi + hi*lo + lo*hi in fp32 (three MFMAs), which keeps each
// product to ~2^-16 relative error; S itself stays fp32 throughout.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int C = 32;          // tokens per chunk
constexpr int SUBT = 16;       // decay sub-tile
constexpr int NW = 8;          // waves per workgroup
constexpr int THREADS = NW * 64;
constexpr int OPK = D + 8;     // padded row (bf16 elements) of [*][128] operand planes
constexpr int OPT = C + 8;     // padded row of [*][32] operand planes
constexpr int FPK = D + 4;     // padded row (floats) of [32][128] fp32 buffers

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ LDS map
// Byte offsets inside one dynamic-size-free static buffer.  The "gram"
// region holds the Gram-matrix operands until the Gram products are done,
// then the fp32 V tile (at +0) and the fp32 output staging tile (at +QL).
constexpr int PL_C_D = C * OPK;          // bf16 elements of one [32][128] plane
constexpr int PL_S_D = SUBT * OPK;       // one [16][128] plane
constexpr int PL_D_C = D * OPT;          // one [128][32] plane
constexpr int PL_C_C = C * OPT;          // one [32][32] plane

constexpr int OFF_KL = 0;                                  // kl = k^ e^{G-R}        hi,lo [32][136]
constexpr int OFF_QL = OFF_KL + 2 * PL_C_D * 2;            // ql = q^ e^{G-R}        hi,lo
constexpr int OFF_KRD = OFF_QL + 2 * PL_C_D * 2;           // krd = k^ e^{R-G}       hi,lo
constexpr int OFF_KR10 = OFF_KRD + 2 * PL_C_D * 2;         // k^ e^{R1-G}, sub-tile 0 hi,lo [16][136]
constexpr int OFF_GRAM_END = OFF_KR10 + 2 * PL_S_D * 2;
constexpr int OFF_V = OFF_KL;                              // fp32 [32][132] (after the Gram products)
constexpr int OFF_O = OFF_QL;                              // fp32 [32][132] (output staging)
constexpr int OFF_KBN = OFF_GRAM_END;                      // -Kbar, K-permuted       hi,lo [32][136]
constexpr int OFF_QB = OFF_KBN + 2 * PL_C_D * 2;           // Qbar, K-permuted        hi,lo [32][136]
constexpr int OFF_KHT = OFF_QB + 2 * PL_C_D * 2;           // Khat^T, K-permuted      hi,lo [128][40]
constexpr int OFF_LA = OFF_KHT + 2 * PL_D_C * 2;           // log alpha -> local cumsum fp32 [32][128]
constexpr int OFF_AF = OFF_LA + C * D * 4;                 // A (beta-scaled) fp32 [32][33]
constexpr int OFF_TS = OFF_AF + C * 33 * 4;                // D0^-1, D1^-1, Z fp32 [3][16][17]
constexpr int OFF_PM = OFF_TS + 3 * 16 * 17 * 4;           // P, K-permuted           hi,lo [32][40]
constexpr int OFF_TM = OFF_PM + 2 * PL_C_C * 2;            // T, K-permuted           hi,lo [32][40]
constexpr int OFF_BETA = OFF_TM + 2 * PL_C_C * 2;          // fp32 [32]
constexpr int OFF_ER1 = OFF_BETA + C * 4;                  // e^{R1}  = e^{G at token 15}     [128]
constexpr int OFF_ET1 = OFF_ER1 + D * 4;                   // e^{G_C - R1}                    [128]
constexpr int OFF_EGC = OFF_ET1 + D * 4;                   // e^{G_C}                          [128]
constexpr int OFF_CW = OFF_EGC + D * 4;                    // conv weights fp32 [3][128][4]
constexpr int OFF_RW = OFF_CW + 3 * D * 4 * 4;             // rms gain fp32 [128]
constexpr int LDS_BYTES = OFF_RW + D * 4;

static_assert(C * FPK * 4 <= 2 * PL_C_D * 2, "V / O staging must fit in one operand slot");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 workgroup");

// Position of K index j (0..31) inside a 32-wide K block of an A operand
// whose B operand comes from two stacked accumulator tiles: B slot 8h + i
// holds row 16(i/4) + 4h + (i%4), so true index j goes to slot
// ((j>>2)&3)*8 + ((j>>4)&1)*4 + (j&3).
__device__ __forceinline__ int kperm(int j) {
    return ((j & 12) << 1) | ((j & 16) >> 2) | (j & 3);
}

// Round-to-nearest-even bf16 split of two floats: x = hi + lo + O(2^-18 |x|).
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    f32x2_t x = {a, b};
    uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
    f32x2_t r = {a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u)};
    hi = h;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
}

__device__ __forceinline__ void split8(const float *x, uint4 &hi, uint4 &lo) {
    split2(x[0], x[1], hi.x, lo.x);
    split2(x[2], x[3], hi.y, lo.y);
    split2(x[4], x[5], hi.z, lo.z);
    split2(x[6], x[7], hi.w, lo.w);
}

__device__ __forceinline__ void split1(float a, uint16_t &hi, uint16_t &lo) {
    uint32_t h, l;
    split2(a, 0.0f, h, l);
    hi = static_cast<uint16_t>(h);
    lo = static_cast<uint16_t>(l);
}

__device__ __forceinline__ f32x4_t mma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// (a_hi + a_lo)(b_hi + b_lo) without the lo*lo term.
__device__ __forceinline__ f32x4_t mma3(uint4 ahi, uint4 alo, uint4 bhi, uint4 blo, f32x4_t c) {
    c = mma(alo, bhi, c);
    c = mma(ahi, blo, c);
    return mma(ahi, bhi, c);
}

template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Eight consecutive io values starting at element i (i a multiple of 8).
template <typename IO> struct Vec8;
template <> struct Vec8<uint16_t> {
    static __device__ __forceinline__ void load(const void *p, size_t i, float *x) {
        uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + i);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(void *p, size_t i, const float *x) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = static_cast<uint32_t>(f32_to_bf16(x[2 * e])) |
                   (static_cast<uint32_t>(f32_to_bf16(x[2 * e + 1])) << 16);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p) + i) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    static __device__ __forceinline__ void copy(const void *src, size_t i, void *dst, size_t j) {
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(dst) + j) =
            *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + i);
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const void *p, size_t i, float *x) {
        const float4 *q = reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
        float4 a = q[0], b = q[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    static __device__ __forceinline__ void store(void *p, size_t i, const float *x) {
        float4 *q = reinterpret_cast<float4 *>(static_cast<float *>(p) + i);
        q[0] = make_float4(x[0], x[1], x[2], x[3]);
        q[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    static __device__ __forceinline__ void copy(const void *src, size_t i, void *dst, size_t j) {
        const float4 *s = reinterpret_cast<const float4 *>(static_cast<const float *>(src) + i);
        float4 *d = reinterpret_cast<float4 *>(static_cast<float *>(dst) + j);
        float4 a = s[0], b = s[1];
        d[0] = a;
        d[1] = b;
    }
};

template <typename IO, typename OUT>
__global__ __launch_bounds__(THREADS) void chunked_kernel(LayerParams p) {
    using IV = Vec8<IO>;
    using OV = Vec8<OUT>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
    uint16_t *const KLh = reinterpret_cast<uint16_t *>(smem + OFF_KL);
    uint16_t *const QLh = reinterpret_cast<uint16_t *>(smem + OFF_QL);
    uint16_t *const KRDh = reinterpret_cast<uint16_t *>(smem + OFF_KRD);
    uint16_t *const KR10h = reinterpret_cast<uint16_t *>(smem + OFF_KR10);
    uint16_t *const KBNh = reinterpret_cast<uint16_t *>(smem + OFF_KBN);
    uint16_t *const QBh = reinterpret_cast<uint16_t *>(smem + OFF_QB);
    uint16_t *const KHTh = reinterpret_cast<uint16_t *>(smem + OFF_KHT);
    uint16_t *const PMh = reinterpret_cast<uint16_t *>(smem + OFF_PM);
    uint16_t *const TMh = reinterpret_cast<uint16_t *>(smem + OFF_TM);
    float *const VB = reinterpret_cast<float *>(smem + OFF_V);
    float *const OB = reinterpret_cast<float *>(smem + OFF_O);
    float *const LA = reinterpret_cast<float *>(smem + OFF_LA);
    float *const AF = reinterpret_cast<float *>(smem + OFF_AF);
    float *const TS = reinterpret_cast<float *>(smem + OFF_TS);
    float *const BETA = reinterpret_cast<float *>(smem + OFF_BETA);
    float *const ER1 = reinterpret_cast<float *>(smem + OFF_ER1);
    float *const ET1 = reinterpret_cast<float *>(smem + OFF_ET1);
    float *const EGC = reinterpret_cast<float *>(smem + OFF_EGC);
    float *const CW = reinterpret_cast<float *>(smem + OFF_CW);
    float *const RW = reinterpret_cast<float *>(smem + OFF_RW);

    const int H = p.H;
    const int item = blockIdx.x;
    const int h = item % H;
    const int idx = item / H;
    const int n = p.order ? p.order[idx] : idx;
    const int64_t t0 = p.cu_seqlens[n];
    const int L = static_cast<int>(p.cu_seqlens[n + 1] - t0);
    const size_t HD = static_cast<size_t>(H) * D;
    const size_t hD = static_cast<size_t>(h) * D;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 15;   // MFMA row / column index
    const int lh = lane >> 4;   // MFMA K group
    const int et = tid >> 4;    // element-wise token (0..31)
    const int ec0 = (tid & 15) * 8;  // element-wise first channel
    const int col = wave * 16 + ln;  // this lane's value column of S

    // ---- per-head constants -------------------------------------------------------
    if (p.prologue) {
        for (int i = tid; i < 3 * D; i += THREADS) {
            const int s = i / D, c = i % D;
            const float4 w = *reinterpret_cast<const float4 *>(p.conv_w + ((s * HD) + hD + c) * 4);
            *reinterpret_cast<float4 *>(CW + i * 4) = w;
        }
    }
    if (tid < D) RW[tid] = p.rms_w ? p.rms_w[tid] : 1.0f;

    // ---- state slice in accumulator layout ------------------------------------------
    const size_t sbase = (static_cast<size_t>(n) * H + h) * D * D;
    f32x4_t S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[t][i] = p.state_in ? p.state_in[sbase + static_cast<size_t>(16 * t + 4 * lh + i) * D + col] : 0.0f;

    const int nchunks = (L + C - 1) / C;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int pos = ch * C + et;          // position of this thread's token in the sequence
        const bool valid = pos < L;
        const size_t grow = static_cast<size_t>(t0 + pos);

        // ---- 1. prologue: conv4 + SiLU (+ L2 for q, k), gates ---------------------------
        float xq[8], xk[8], xv[8];
        {
            float *outs[3] = {xq, xk, xv};
            const void *srcs[3] = {p.q, p.k, p.v};
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                float *a = outs[s];
                float x0[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x0[e] = 0.0f;
                if (valid) IV::load(srcs[s], grow * HD + hD + ec0, x0);
                if (p.prologue) {
                    float acc[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = CW[(s * D + ec0 + e) * 4] * x0[e];
#pragma unroll
                    for (int j = 1; j <= 3; ++j) {
                        float xj[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) xj[e] = 0.0f;
                        const int pj = pos - j;
                        if (valid) {
                            if (pj >= 0)
                                IV::load(srcs[s], (grow - j) * HD + hD + ec0, xj);
                            else if (p.conv_in)
                                IV::load(p.conv_in, ((static_cast<size_t>(n) * 3 + s) * CONV_HIST + (CONV_HIST + pj)) * HD + hD + ec0, xj);
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[e] = fmaf(CW[(s * D + ec0 + e) * 4 + j], xj[e], acc[e]);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = siluf_(acc[e]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = x0[e];
                }
            }
            if (p.prologue) {
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sq = fmaf(xq[e], xq[e], sq);
                    sk = fmaf(xk[e], xk[e], sk);
                }
                sq = group_sum<16>(sq);
                sk = group_sum<16>(sk);
                const float iq = rsqrtf(sq + p.l2_eps), ik = rsqrtf(sk + p.l2_eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xq[e] *= iq;
                    xk[e] *= ik;
                }
            }
            if (!valid) {
#pragma unroll
                for (int e = 0; e < 8; ++e) xq[e] = xk[e] = xv[e] = 0.0f;
            }
            float la[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) la[e] = 0.0f;
            if (valid) Vec8<float>::load(p.log_alpha, grow * HD + hD + ec0, la);
            Vec8<float>::store(LA, et * D + ec0, la);
            if ((tid & 15) == 0) BETA[et] = valid ? p.beta[grow * H + h] : 0.0f;
        }
        __syncthreads();

        // ---- 2. local cumulative log-decay inside each 16-token sub-tile --------------------
        if (tid < D) {
            const int c = tid;
            float g[C];
#pragma unroll
            for (int r = 0; r < C; ++r) g[r] = LA[r * D + c];
#pragma unroll
            for (int r = 1; r < SUBT; ++r) {
                g[r] += g[r - 1];
                g[SUBT + r] += g[SUBT + r - 1];
            }
#pragma unroll
            for (int r = 0; r < C; ++r) LA[r * D + c] = g[r];
            const float tot0 = g[SUBT - 1], tot1 = g[C - 1];
            ER1[c] = __expf(tot0);
            ET1[c] = __expf(tot1);
            EGC[c] = __expf(tot0 + tot1);
        }
        __syncthreads();

        // ---- 3. staged operands (hi/lo bf16) ------------------------------------------
        {
            const int sig = et >> 4;  // sub-tile of this token
            float gl[8], er[8], egcr[8];
            Vec8<float>::load(LA, et * D + ec0, gl);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                er[e] = sig ? ER1[ec0 + e] : 1.0f;
                egcr[e] = sig ? ET1[ec0 + e] : EGC[ec0 + e];
            }
            float kl[8], ql[8], krd[8], tmp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float E = __expf(gl[e]);
                const float rE = __expf(-gl[e]);
                kl[e] = xk[e] * E;
                ql[e] = xq[e] * E;
                krd[e] = xk[e] * rE;
            }
            uint4 hi, lo;
            const int ro = et * OPK + ec0;
            split8(kl, hi, lo);
            *reinterpret_cast<uint4 *>(KLh + ro) = hi;
            *reinterpret_cast<uint4 *>(KLh + PL_C_D + ro) = lo;
            split8(ql, hi, lo);
            *reinterpret_cast<uint4 *>(QLh + ro) = hi;
            *reinterpret_cast<uint4 *>(QLh + PL_C_D + ro) = lo;
            split8(krd, hi, lo);
            *reinterpret_cast<uint4 *>(KRDh + ro) = hi;
            *reinterpret_cast<uint4 *>(KRDh + PL_C_D + ro) = lo;
            if (sig == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) tmp[e] = krd[e] * ER1[ec0 + e];
                split8(tmp, hi, lo);
                *reinterpret_cast<uint4 *>(KR10h + ro) = hi;
                *reinterpret_cast<uint4 *>(KR10h + PL_S_D + ro) = lo;
            }
            // K-permuted channel position of channels ec0..ec0+3 and ec0+4..ec0+7
            const int cb = ec0 & ~31, a4 = (ec0 >> 3) & 3;
            const int pc0 = cb + 16 * (a4 & 1) + 4 * (a4 >> 1);
            const int pc1 = pc0 + 8;
            const int rp = et * OPK;
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = -kl[e] * er[e];
            split8(tmp, hi, lo);
            *reinterpret_cast<uint2 *>(KBNh + rp + pc0) = make_uint2(hi.x, hi.y);
            *reinterpret_cast<uint2 *>(KBNh + rp + pc1) = make_uint2(hi.z, hi.w);
            *reinterpret_cast<uint2 *>(KBNh + PL_C_D + rp + pc0) = make_uint2(lo.x, lo.y);
            *reinterpret_cast<uint2 *>(KBNh + PL_C_D + rp + pc1) = make_uint2(lo.z, lo.w);
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = ql[e] * er[e];
            split8(tmp, hi, lo);
            *reinterpret_cast<uint2 *>(QBh + rp + pc0) = make_uint2(hi.x, hi.y);
            *reinterpret_cast<uint2 *>(QBh + rp + pc1) = make_uint2(hi.z, hi.w);
            *reinterpret_cast<uint2 *>(QBh + PL_C_D + rp + pc0) = make_uint2(lo.x, lo.y);
            *reinterpret_cast<uint2 *>(QBh + PL_C_D + rp + pc1) = make_uint2(lo.z, lo.w);
            // Khat^T: row = channel, column = K-permuted token
            const int pt = kperm(et);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint16_t sh, sl;
                split1(krd[e] * egcr[e], sh, sl);
                KHTh[(ec0 + e) * OPT + pt] = sh;
                KHTh[PL_D_C + (ec0 + e) * OPT + pt] = sl;
            }
        }
        __syncthreads();

        // ---- 4. intra-chunk Gram blocks on MFMA ----------------------------------------
        // waves 0-2: A blocks (0,0), (1,0), (1,1); waves 3-5: P blocks; wave 6 clears P's
        // upper-right block.
        if (wave < 6) {
            const bool isP = wave >= 3;
            const int pr = wave % 3;
            const int sg = pr == 0 ? 0 : 1;          // row sub-tile
            const int tg = pr == 2 ? 1 : 0;          // column sub-tile
            const uint16_t *Lh = isP ? QLh : KLh;
            const uint16_t *Rh = pr == 1 ? KR10h : KRDh;
            const int rplane = pr == 1 ? PL_S_D : PL_C_D;
            const int rrow = pr == 1 ? 0 : 16 * tg;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                const int ka = (16 * sg + ln) * OPK + 32 * s + 8 * lh;
                const int kb = (rrow + ln) * OPK + 32 * s + 8 * lh;
                const uint4 ah = *reinterpret_cast<const uint4 *>(Lh + ka);
                const uint4 al = *reinterpret_cast<const uint4 *>(Lh + PL_C_D + ka);
                const uint4 bh = *reinterpret_cast<const uint4 *>(Rh + kb);
                const uint4 bl = *reinterpret_cast<const uint4 *>(Rh + rplane + kb);
                acc = mma3(ah, al, bh, bl, acc);
            }
            const bool diag = sg == tg;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * sg + 4 * lh + i;  // output token (row)
                const int j = 16 * tg + ln;          // input token (column)
                if (!isP) {
                    AF[r * 33 + j] = (diag && j >= r) ? 0.0f : acc[i] * BETA[r];
                } else {
                    uint16_t sh, sl;
                    split1((diag && j > r) ? 0.0f : acc[i], sh, sl);
                    PMh[r * OPT + kperm(j)] = sh;
                    PMh[PL_C_C + r * OPT + kperm(j)] = sl;
                }
            }
        } else if (wave == 6) {
            // P[r][j] = 0 for r < 16 <= j
            for (int e = lane; e < 16 * 16; e += 64) {
                const int r = e >> 4, j = 16 + (e & 15);
                PMh[r * OPT + kperm(j)] = 0;
                PMh[PL_C_C + r * OPT + kperm(j)] = 0;
            }
        }
        __syncthreads();

        // ---- 5. V tile (fp32) and T = (I + A)^{-1} Diag(beta) -----------------------------
        Vec8<float>::store(VB, et * FPK + ec0, xv);
        if (tid < 32) {
            // column c of the inverse of the unit-lower 16x16 block I + A_bb
            const int b = tid >> 4, c = tid & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == c) ? 1.0f : 0.0f;
#pragma unroll
                for (int j = 0; j < r; ++j) acc = fmaf(-AF[(16 * b + r) * 33 + 16 * b + j], x[j], acc);
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) TS[(b * 16 + r) * 17 + c] = x[r];
        }
        __syncthreads();
        if (tid < 256) {
            // Z = A_10 D0^{-1}
            const int r = tid >> 4, c = tid & 15;
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) acc = fmaf(AF[(16 + r) * 33 + j], TS[j * 17 + c], acc);
            TS[(32 + r) * 17 + c] = acc;
        }
        __syncthreads();
        if (tid < 256) {
            // T_10 = -D1^{-1} Z Diag(beta_0..15)
            const int r = tid >> 4, c = tid & 15;
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) acc = fmaf(TS[(16 + r) * 17 + j], TS[(32 + j) * 17 + c], acc);
            uint16_t sh, sl;
            split1(-acc * BETA[c], sh, sl);
            TMh[(16 + r) * OPT + kperm(c)] = sh;
            TMh[PL_C_C + (16 + r) * OPT + kperm(c)] = sl;
        } else {
            for (int e = tid - 256; e < 3 * 256; e += 256) {
                const int blk = e >> 8, r = (e >> 4) & 15, c = e & 15;
                float v;
                int rr, cc;
                if (blk == 0) { v = TS[r * 17 + c] * BETA[c]; rr = r; cc = c; }
                else if (blk == 1) { v = TS[(16 + r) * 17 + c] * BETA[16 + c]; rr = 16 + r; cc = 16 + c; }
                else { v = 0.0f; rr = r; cc = 16 + c; }
                uint16_t sh, sl;
                split1(v, sh, sl);
                TMh[rr * OPT + kperm(cc)] = sh;
                TMh[PL_C_C + rr * OPT + kperm(cc)] = sl;
            }
        }
        __syncthreads();

        // ---- 6. state contractions (this wave's 16 value columns) -------------------------
        {
            // S as B operand: K step s holds rows 32s + pi(slot)
            uint4 Sh[4], Sl[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float v8[8] = {S[2 * s][0], S[2 * s][1], S[2 * s][2], S[2 * s][3],
                                     S[2 * s + 1][0], S[2 * s + 1][1], S[2 * s + 1][2], S[2 * s + 1][3]};
                split8(v8, Sh[s], Sl[s]);
            }
            // X = V - Kbar S
            f32x4_t X[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) X[mt][i] = VB[(16 * mt + 4 * lh + i) * FPK + col];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int ka = (16 * mt + ln) * OPK + 32 * s + 8 * lh;
                    const uint4 ah = *reinterpret_cast<const uint4 *>(KBNh + ka);
                    const uint4 al = *reinterpret_cast<const uint4 *>(KBNh + PL_C_D + ka);
                    X[mt] = mma3(ah, al, Sh[s], Sl[s], X[mt]);
                }
            }
            // U = T X
            uint4 Xh, Xl;
            {
                const float v8[8] = {X[0][0], X[0][1], X[0][2], X[0][3], X[1][0], X[1][1], X[1][2], X[1][3]};
                split8(v8, Xh, Xl);
            }
            f32x4_t U[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int ka = (16 * mt + ln) * OPT + 8 * lh;
                const uint4 ah = *reinterpret_cast<const uint4 *>(TMh + ka);
                const uint4 al = *reinterpret_cast<const uint4 *>(TMh + PL_C_C + ka);
                U[mt] = mma3(ah, al, Xh, Xl, f32x4_t{0.f, 0.f, 0.f, 0.f});
            }
            uint4 Uh, Ul;
            {
                const float v8[8] = {U[0][0], U[0][1], U[0][2], U[0][3], U[1][0], U[1][1], U[1][2], U[1][3]};
                split8(v8, Uh, Ul);
            }
            // O = scale (Qbar S + P U)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                f32x4_t O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int ka = (16 * mt + ln) * OPK + 32 * s + 8 * lh;
                    const uint4 ah = *reinterpret_cast<const uint4 *>(QBh + ka);
                    const uint4 al = *reinterpret_cast<const uint4 *>(QBh + PL_C_D + ka);
                    O = mma3(ah, al, Sh[s], Sl[s], O);
                }
                {
                    const int ka = (16 * mt + ln) * OPT + 8 * lh;
                    const uint4 ah = *reinterpret_cast<const uint4 *>(PMh + ka);
                    const uint4 al = *reinterpret_cast<const uint4 *>(PMh + PL_C_C + ka);
                    O = mma3(ah, al, Uh, Ul, O);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) OB[(16 * mt + 4 * lh + i) * FPK + col] = O[i] * p.scale;
            }
            // S <- Diag(Gamma_C) S + Khat^T U
#pragma unroll
            for (int t = 0; t < 8; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) S[t][i] *= EGC[16 * t + 4 * lh + i];
                const int ka = (16 * t + ln) * OPT + 8 * lh;
                const uint4 ah = *reinterpret_cast<const uint4 *>(KHTh + ka);
                const uint4 al = *reinterpret_cast<const uint4 *>(KHTh + PL_D_C + ka);
                S[t] = mma3(ah, al, Uh, Ul, S[t]);
            }
        }
        __syncthreads();

        // ---- 7. epilogue: sigma(g) * RMSNorm(o~) * w -------------------------------------
        {
            float o[8];
            Vec8<float>::load(OB, et * FPK + ec0, o);
            if (p.epilogue) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(o[e], o[e], ss);
                ss = group_sum<16>(ss);
                const float inv = rsqrtf(ss * (1.0f / D) + p.rms_eps);
                if (valid) {
                    float g[8];
                    IV::load(p.g, grow * HD + hD + ec0, g);
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = sigmoidf_(g[e]) * (o[e] * inv) * RW[ec0 + e];
                }
            }
            if (valid) OV::store(p.o, grow * HD + hD + ec0, o);
        }
        // the next chunk's first barrier orders these LDS reads before any rewrite
    }

    // ---- final state and conv cache -----------------------------------------------------
    if (p.state_out) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p.state_out[sbase + static_cast<size_t>(16 * t + 4 * lh + i) * D + col] = S[t][i];
    }
    if (p.prologue && p.conv_out) {
        // the last three pre-conv inputs of each stream, oldest first; rows before the
        // sequence start come from conv_in (which conv_out may alias: read all, then write)
        const int task = tid;  // (stream, slot, channel group) = 3 * 3 * 16 = 144 tasks
        const bool active = task < 3 * CONV_HIST * 16;
        const int s = task / (CONV_HIST * 16), j = (task / 16) % CONV_HIST, cg = task & 15;
        const int pj = L - CONV_HIST + j;  // source position
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        const void *srcs[3] = {p.q, p.k, p.v};
        if (active) {
            if (pj >= 0)
                IV::load(srcs[s], static_cast<size_t>(t0 + pj) * HD + hD + cg * 8, x);
            else if (p.conv_in)
                IV::load(p.conv_in, ((static_cast<size_t>(n) * 3 + s) * CONV_HIST + (CONV_HIST + pj)) * HD + hD + cg * 8, x);
        }
        __syncthreads();
        if (active)
            IV::store(p.conv_out, ((static_cast<size_t>(n) * 3 + s) * CONV_HIST + j) * HD + hD + cg * 8, x);
    }
}

template <typename IO, typename OUT>
hipError_t launch(const LayerParams &p, hipStream_t s) {
    if (p.num_items == 0) return hipSuccess;
    hipLaunchKernelGGL((chunked_kernel<IO, OUT>), dim3(p.num_items), dim3(THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunked(const LayerParams &p, int io_dtype, int out_dtype, hipStream_t s) {
    if (io_dtype == KDA_DTYPE_BF16)
        return out_dtype == KDA_DTYPE_BF16 ? launch<uint16_t, uint16_t>(p, s)
                                           : launch<uint16_t, float>(p, s);
    return out_dtype == KDA_DTYPE_BF16 ? launch<float, uint16_t>(p, s) : launch<float, float>(p, s);
}

}  // namespace kda
