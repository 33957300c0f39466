// kda_chunked_pipe.hip -- chunked KDA prefill on the gfx950 matrix cores, latency
// variant: one 8-wave workgroup per CU runs a producer/consumer pipeline over the
// chunks (for launches with at most one (sequence, head) item per CU, where
// each item's chain of chunks is the critical path).
//
// The per-token recurrence of the "Kimi K3 - KDA layer" step list
// (S <- Diag(alpha) S;  S <- S + beta k (v - S^T k)^T;  o~ = S^T q / sqrt(128))
// is regrouped over chunks of C = 16 tokens.  For one chunk entering with
// state S0, with G the running sum of log alpha from the chunk start (per
// key channel), Gamma = e^G and G_C its value at the last token:
//
//   A[s][j] = beta_s sum_c k_s[c] k_j[c] e^{G_s[c] - G_j[c]}      (j < s)
//   P[r][j] =        sum_c q_r[c] k_j[c] e^{G_r[c] - G_j[c]}      (j <= r)
//   T       = (I + A)^{-1} Diag(beta)
//   U       = T (V - Kbar S0),            Kbar = Gamma (.) K
//   O       = scale (Qbar S0 + P U),      Qbar = Gamma (.) Q
//   S1      = Diag(Gamma_C) S0 + Khat^T U, Khat = e^{G_C - G} (.) K
//
// which is the recurrence unrolled over the chunk: u_r = beta_r (v_r -
// (Diag(alpha_r) S_{r-1})^T k_r) is the per-token correction, and stacking
// the u_r gives the unit-lower triangular system (I + A) U = Diag(beta)(V -
// Kbar S0).  The Gram blocks use the factorisation e^{G_s - G_j} =
// e^{G_s} e^{-G_j} within the chunk; at the log-decay floor of -5 per token
// ("Kimi K3's Architecture ...", section "Channel-wise decay, and the floor
// K3 puts under it") a 16-token chunk keeps e^{-G} <= e^80, inside the fp32 /
// bf16 exponent range.
//
// Work layout: one workgroup of 8 waves per (sequence, head).  Only S carries
// a dependence from one chunk to the next, so the workgroup is a two-stage
// pipeline:
//   * waves 0-3 (consumers) own S -- wave w keeps value columns 32w .. 32w+31
//     as a 128 x 32 fp32 slice in registers, in the accumulator layout of the
//     16x16 MFMAs -- and run the state products and the epilogue of chunk c;
//   * waves 4-7 (producers) stage, convolve and normalise chunk c+1, build its
//     operands in the other half of a double-buffered LDS area, and compute
//     the Gram blocks and T of chunk c just before the consumers need them.
// Three workgroup barriers per chunk separate the stages.
//
// Contractions over the 16 tokens of a chunk (v_mfma_f32_16x16x16_bf16) take
// accumulator tiles directly as their B operand.  Contractions over the 128
// key channels (v_mfma_f32_16x16x32_bf16) read S from the same registers: K
// slot 8h + i of a 32-channel step holds channel 16(i/4) + 4h + (i%4), so the
// channel-indexed operands in LDS store their channels in that permuted order
// (the Gram products contract two such operands, which the permutation leaves
// unchanged).
//
// Precision: every contraction splits both operands into bf16 hi + lo parts
// and sums hi*hi + hi*lo + lo*hi in fp32 (three MFMAs), which keeps each
// product to ~2^-16 relative error; S itself stays fp32 throughout.
#include "kda_chunk_common.h"

namespace kda {
namespace {

using namespace chunk;

constexpr int THREADS = 512;   // 4 consumer + 4 producer waves
constexpr int GROUP = 256;     // threads per role


// ------------------------------------------------------------------ LDS map (bytes)

// double-buffered operands of one chunk (buffer b at +b * BUF)
constexpr int B_KL = 0;                            // k^ Gamma (= Kbar), channel-permuted      hi,lo
constexpr int B_QL = B_KL + 2 * PL_CD * 2;         // q^ Gamma (= Qbar), channel-permuted      hi,lo
constexpr int B_KHT = B_QL + 2 * PL_CD * 2;        // Khat^T [channel][token], swizzled        hi,lo
constexpr int B_V = B_KHT + 2 * PL_DC * 2;         // V fp32 [16][132]
constexpr int B_EGC = B_V + C * FPK * 4;           // e^{G_C} fp32 [128]
constexpr int B_BETA = B_EGC + D * 4;              // beta fp32 [16]
constexpr int BUF = B_BETA + C * 4;
// single-buffered
constexpr int OFF_KRD = 2 * BUF;                   // k^ / Gamma, channel-permuted             hi,lo
constexpr int OFF_TM = OFF_KRD + 2 * PL_CD * 2;    // T                                        hi,lo [16][20]
constexpr int OFF_PM = OFF_TM + 2 * PL_CC * 2;     // P                                        hi,lo [16][20]
constexpr int OFF_AF = OFF_PM + 2 * PL_CC * 2;     // -A (beta-scaled) fp32 [16][17]
constexpr int OFF_O = OFF_AF + C * 17 * 4;         // output staging fp32 [16][132]
constexpr int OFF_LA = OFF_O + C * FPK * 4;        // log alpha -> cumulative, fp32 [16][128]
constexpr int OFF_CW = OFF_LA + C * D * 4;         // conv weights fp32 [3 streams][4 taps][128]
constexpr int OFF_RW = OFF_CW + 3 * 4 * D * 4;     // rms gain fp32 [128]
constexpr int OFF_RAW = OFF_RW + D * 4;            // raw q, k, v rows of a chunk [3][16][128] io
// ... then the last three raw rows of the previous chunks, double-buffered [2][3][3][128] io
template <typename IO> struct RawLds {
    static constexpr int CUR = OFF_RAW;
    static constexpr int HIST = CUR + 3 * C * D * static_cast<int>(sizeof(IO));
    static constexpr int BYTES = HIST + 2 * 3 * CONV_HIST * D * static_cast<int>(sizeof(IO));
};
static_assert(RawLds<float>::BYTES <= 160 * 1024, "LDS budget of one gfx950 workgroup");
static_assert(BUF % 16 == 0 && OFF_RAW % 16 == 0, "16-byte aligned LDS regions");

template <typename IO, typename OUT>
__global__ __launch_bounds__(THREADS, 1) void chunked_pipe_kernel(LayerParams p) {
    using IV = Vec8<IO>;
    using IB = BufLoad8<IO>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[RawLds<IO>::BYTES];
    IO *const RAWC = reinterpret_cast<IO *>(smem + RawLds<IO>::CUR);
    IO *const RAWH = reinterpret_cast<IO *>(smem + RawLds<IO>::HIST);
    uint16_t *const KRDh = reinterpret_cast<uint16_t *>(smem + OFF_KRD);
    uint16_t *const TMh = reinterpret_cast<uint16_t *>(smem + OFF_TM);
    uint16_t *const PMh = reinterpret_cast<uint16_t *>(smem + OFF_PM);
    float *const AF = reinterpret_cast<float *>(smem + OFF_AF);
    float *const OB = reinterpret_cast<float *>(smem + OFF_O);
    float *const LA = reinterpret_cast<float *>(smem + OFF_LA);
    float *const CW = reinterpret_cast<float *>(smem + OFF_CW);
    float *const RW = reinterpret_cast<float *>(smem + OFF_RW);
    auto KLh = [&](int b) { return reinterpret_cast<uint16_t *>(smem + b * BUF + B_KL); };
    auto QLh = [&](int b) { return reinterpret_cast<uint16_t *>(smem + b * BUF + B_QL); };
    auto KHTh = [&](int b) { return reinterpret_cast<uint16_t *>(smem + b * BUF + B_KHT); };
    auto VB = [&](int b) { return reinterpret_cast<float *>(smem + b * BUF + B_V); };
    auto EGC = [&](int b) { return reinterpret_cast<float *>(smem + b * BUF + B_EGC); };
    auto BETA = [&](int b) { return reinterpret_cast<float *>(smem + b * BUF + B_BETA); };

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
    const bool prod = tid >= GROUP;  // producer waves 4-7
    const int gt = tid & (GROUP - 1);
    const int gw = gt >> 6;          // wave within the role group
    const int lane = tid & 63;
    const int ln = lane & 15;        // MFMA row / column index
    const int lh = lane >> 4;        // MFMA K group
    const int et = gt >> 4;          // element-wise token (0..15)
    const int ec0 = (gt & 15) * 8;   // element-wise first channel
    const int col0 = gw * 32 + ln;   // consumer: value column of N-tile 0 (tile 1: +16)

    // ---- per-head constants -------------------------------------------------------------
    if (p.prologue) {
        for (int i = tid; i < 3 * D; i += THREADS) {
            const int s = i / D, c = i % D;
            const float4 w = *reinterpret_cast<const float4 *>(p.conv_w + ((s * HD) + hD + c) * 4);
            CW[(s * 4 + 0) * D + c] = w.x;
            CW[(s * 4 + 1) * D + c] = w.y;
            CW[(s * 4 + 2) * D + c] = w.z;
            CW[(s * 4 + 3) * D + c] = w.w;
        }
    }
    if (tid < D) RW[tid] = p.rms_w ? p.rms_w[tid] : 1.0f;

    const int nchunks = (L + C - 1) / C;
    const uint32_t rowb_io = static_cast<uint32_t>(HD * sizeof(IO));
    const uint32_t rowb_f = static_cast<uint32_t>(HD * 4);
    const size_t first = static_cast<size_t>(t0) * HD + hD;
    const uint32_t off_io = static_cast<uint32_t>(et) * rowb_io + ec0 * sizeof(IO);
    const uint32_t off_f = static_cast<uint32_t>(et) * rowb_f + ec0 * 4u;
    const int row_in = p.slots_in ? p.slots_in[n] : n;     // state_in / conv_in row
    const int row_out = p.slots_out ? p.slots_out[n] : n;  // state_out / conv_out row
    const size_t sbase = (static_cast<size_t>(row_in) * H + h) * D * D;
    const size_t sbase_out = (static_cast<size_t>(row_out) * H + h) * D * D;

    // ---- role state ----------------------------------------------------------------------
    // consumer: the state slice S[t][nt][i] = S(16t + 4lh + i, col0 + 16nt), and the gate
    // rows of the chunk it finishes next; producer: the raw rows of the chunk it stages next
    f32x4_t S[8][2];
    typename IV::Raw graw{};
    typename IV::Raw cur[3];
    typename Vec8<float>::Raw lar{};
    float bet = 0.0f;
    float xq[8], xk[8], xv[8];

    const char *qkv_base[3] = {static_cast<const char *>(p.q) + first * sizeof(IO),
                               static_cast<const char *>(p.k) + first * sizeof(IO),
                               static_cast<const char *>(p.v) + first * sizeof(IO)};
    auto load_current = [&](int c) {  // producer: q, k, v, log alpha, beta rows of chunk c
        const int r0 = c * C, nrow = min(L, r0 + C) - r0;
        const size_t cio = static_cast<size_t>(r0) * rowb_io;
#pragma unroll
        for (int s = 0; s < 3; ++s)
            cur[s] = IB::load(rows_view(qkv_base[s] + cio, nrow, rowb_io, D * sizeof(IO)), off_io);
        lar = BufLoad8<float>::load(
            rows_view(reinterpret_cast<const char *>(p.log_alpha + first) + static_cast<size_t>(r0) * rowb_f, nrow,
                      rowb_f, D * 4),
            off_f);
        bet = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rows_view(reinterpret_cast<const char *>(p.beta + static_cast<size_t>(t0) * H + h) +
                          static_cast<size_t>(r0) * H * 4,
                      nrow, H * 4, 4),
            static_cast<uint32_t>(et * H) * 4u, 0, 0));
    };
    auto load_gate = [&](int c) {  // consumer: g rows of chunk c
        const int r0 = c * C, nrow = min(L, r0 + C) - r0;
        if (p.epilogue)
            graw = IB::load(rows_view(static_cast<const char *>(p.g) + first * sizeof(IO) + static_cast<size_t>(r0) * rowb_io,
                                      nrow, rowb_io, D * sizeof(IO)),
                            off_io);
    };

    if (!prod) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[t][nt][i] = p.state_in ? p.state_in[sbase + static_cast<size_t>(16 * t + 4 * lh + i) * D + col0 + 16 * nt] : 0.0f;
        if (nchunks > 0) load_gate(0);
    } else {
        if (nchunks > 0) load_current(0);
        if (p.prologue && gt < 3 * CONV_HIST * 16) {
            // history of the first chunk: the given conv cache (oldest first) or zeros
            const int s = gt / (CONV_HIST * 16), j = (gt / 16) % CONV_HIST, c0 = (gt & 15) * 8;
            typename IV::Raw r{};
            if (p.conv_in) r = IV::raw(p.conv_in, ((static_cast<size_t>(row_in) * 3 + s) * CONV_HIST + j) * HD + hD + c0);
            *reinterpret_cast<typename IV::Raw *>(RAWH + ((1 * 3 + s) * CONV_HIST + j) * D + c0) = r;
        }
    }
    __syncthreads();

    // Iteration c: consumers finish chunk c (c >= 0); producers compute the Gram blocks and T
    // of chunk c and prepare chunk c + 1.
    for (int c = -1; c < nchunks; ++c) {
        const int cn = c + 1;
        const bool has_c = c >= 0, has_n = cn < nchunks;
        const int bc = c & 1, bn = cn & 1;  // operand buffers of chunks c and c + 1

        // ================================ segment 1 ================================
        if (prod) {
            if (has_c && gw < 2) {
                // Gram blocks of chunk c: wave 4 -> A and then T, wave 5 -> P
                const uint16_t *Lh = gw == 0 ? KLh(bc) : QLh(bc);
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < D / 32; ++s) {
                    const int ka = ln * OPK + 32 * s + 8 * lh;
                    const uint4 ah = *reinterpret_cast<const uint4 *>(Lh + ka);
                    const uint4 al = *reinterpret_cast<const uint4 *>(Lh + PL_CD + ka);
                    const uint4 bh = *reinterpret_cast<const uint4 *>(KRDh + ka);
                    const uint4 bl = *reinterpret_cast<const uint4 *>(KRDh + PL_CD + ka);
                    acc = mma3(ah, al, bh, bl, acc);
                }
                const int j = ln;
                if (gw == 0) {
                    // T = (I + A)^{-1} Diag(beta).  With B = -A (strictly lower, so B^16 = 0),
                    // (I + A)^{-1} = sum_{k<16} B^k = (I + B)(I + B^2)(I + B^4)(I + B^8): four
                    // levels of 16x16 products.  A matrix M is held in two register forms:
                    // "b" = B-operand / accumulator layout (lane (n, g) holds M[4g+i][n]) and
                    // "a" = A-operand layout (lane (m, g) holds M[m][4g+i]); the product XY
                    // takes (a of X, b of Y) and gives b of XY, while (b of Y, a of X) gives
                    // b of (XY)^T = a of XY.
                    const float *beta = BETA(bc);
                    float bb[4], ba[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 4 * lh + i;
                        bb[i] = j < r ? -acc[i] * beta[r] : 0.0f;
                        AF[r * 17 + j] = bb[i];
                    }
                    // one transpose through LDS for the a form of B (lanes of this wave only)
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
                    for (int i = 0; i < 4; ++i) ba[i] = AF[ln * 17 + 4 * lh + i];
                    // only the a form of the sum is needed (T is an A operand); each operand
                    // is split into bf16 hi/lo once and reused by the products that read it
                    float sa[4];  // a form of S1 = I + B
#pragma unroll
                    for (int i = 0; i < 4; ++i) sa[i] = ba[i] + ((4 * lh + i) == ln ? 1.0f : 0.0f);
                    Split4 Ba(ba), Bb(bb);
                    Split4 B2b(mm16s(Ba, Bb)), B2a(mm16s(Bb, Ba));  // B^2
                    float t[4];
                    mm16s(B2b, Split4(sa), t);                        // S2 = S1 + S1 B^2
#pragma unroll
                    for (int i = 0; i < 4; ++i) sa[i] += t[i];
                    Split4 B4b(mm16s(B2a, B2b)), B4a(mm16s(B2b, B2a));  // B^4
                    mm16s(B4b, Split4(sa), t);                        // S4 = S2 + S2 B^4
#pragma unroll
                    for (int i = 0; i < 4; ++i) sa[i] += t[i];
                    Split4 B8b(mm16s(B4a, B4b));                      // B^8
                    mm16s(B8b, Split4(sa), t);                        // S8 = S4 + S4 B^8
                    // T[m][k] = S8[m][k] beta_k: lane (m, g) stores row m, columns 4g .. 4g+3
                    float tv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) tv[i] = (sa[i] + t[i]) * beta[4 * lh + i];
                    uint2 th, tl;
                    split4(tv, th, tl);
                    *reinterpret_cast<uint2 *>(TMh + ln * OPT + 4 * lh) = th;
                    *reinterpret_cast<uint2 *>(TMh + PL_CC + ln * OPT + 4 * lh) = tl;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 4 * lh + i;
                        uint16_t sh, sl;
                        split1(j <= r ? acc[i] : 0.0f, sh, sl);
                        PMh[r * OPT + j] = sh;
                        PMh[PL_CC + r * OPT + j] = sl;
                    }
                }
            }
            if (has_n) {
                // stage chunk c + 1 (rows prefetched one chunk ahead), then prefetch chunk c + 2
#pragma unroll
                for (int s = 0; s < 3; ++s) {
                    *reinterpret_cast<typename IV::Raw *>(RAWC + (s * C + et) * D + ec0) = cur[s];
                    if (et >= C - CONV_HIST)
                        *reinterpret_cast<typename IV::Raw *>(RAWH + ((bn * 3 + s) * CONV_HIST + et - (C - CONV_HIST)) * D + ec0) = cur[s];
                }
                float la[8];
                Vec8<float>::unpack(lar, la);
                Vec8<float>::store(LA, et * D + ec0, la);
                if ((gt & 15) == 0) BETA(bn)[et] = bet;
                if (cn + 1 < nchunks) load_current(cn + 1);
            }
        } else if (has_c) {
            // X = V - Kbar S0 and O1 = Qbar S0; S0 is the B operand, K step s holding rows
            // 32s + pi(slot), split into bf16 hi/lo right before use
            const uint16_t *kl = KLh(bc);
            const uint16_t *ql = QLh(bc);
            f32x4_t X[2], O1[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                X[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                O1[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ka = ln * OPK + 32 * s + 8 * lh;
                const uint4 kh = *reinterpret_cast<const uint4 *>(kl + ka);
                const uint4 kl_ = *reinterpret_cast<const uint4 *>(kl + PL_CD + ka);
                const uint4 qh = *reinterpret_cast<const uint4 *>(ql + ka);
                const uint4 ql_ = *reinterpret_cast<const uint4 *>(ql + PL_CD + ka);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const float v8[8] = {S[2 * s][nt][0], S[2 * s][nt][1], S[2 * s][nt][2], S[2 * s][nt][3],
                                         S[2 * s + 1][nt][0], S[2 * s + 1][nt][1], S[2 * s + 1][nt][2], S[2 * s + 1][nt][3]};
                    uint4 sh, sl;
                    split8(v8, sh, sl);
                    X[nt] = mma3(kh, kl_, sh, sl, X[nt]);
                    O1[nt] = mma3(qh, ql_, sh, sl, O1[nt]);
                }
            }
            const float *vb = VB(bc);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) X[nt][i] = vb[(4 * lh + i) * FPK + col0 + 16 * nt] - X[nt][i];
            // keep X and O1 for segment 2 in the accumulators of this wave
            xq[0] = X[0][0]; xq[1] = X[0][1]; xq[2] = X[0][2]; xq[3] = X[0][3];
            xq[4] = X[1][0]; xq[5] = X[1][1]; xq[6] = X[1][2]; xq[7] = X[1][3];
            xk[0] = O1[0][0]; xk[1] = O1[0][1]; xk[2] = O1[0][2]; xk[3] = O1[0][3];
            xk[4] = O1[1][0]; xk[5] = O1[1][1]; xk[6] = O1[1][2]; xk[7] = O1[1][3];
        }
        __syncthreads();

        // ================================ segment 2 ================================
        if (prod) {
            if (has_n) {
                // conv4 + SiLU (+ L2 for q, k) of chunk c + 1 from the staged rows
                const int pos = cn * C + et;
                float *outs[3] = {xq, xk, xv};
#pragma unroll
                for (int s = 0; s < 3; ++s) {
                    float *a = outs[s];
                    IV::unpack(*reinterpret_cast<const typename IV::Raw *>(RAWC + (s * C + et) * D + ec0), a);
                    if (p.prologue) {
                        float acc[8], w[8];
                        Vec8<float>::load(CW, (s * 4) * D + ec0, w);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[e] = w[e] * a[e];
#pragma unroll
                        for (int j = 1; j <= 3; ++j) {
                            const int r = et - j;  // row in this chunk, or (r + 3) in the history
                            const IO *src = r >= 0 ? RAWC + (s * C + r) * D
                                                   : RAWH + (((bn ^ 1) * 3 + s) * CONV_HIST + r + CONV_HIST) * D;
                            float xj[8];
                            IV::unpack(*reinterpret_cast<const typename IV::Raw *>(src + ec0), xj);
                            Vec8<float>::load(CW, (s * 4 + j) * D + ec0, w);
#pragma unroll
                            for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[e], xj[e], acc[e]);
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) a[e] = siluf_(acc[e]);
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
                    if (pos >= L) {  // padding tokens past the end see real history rows: clear them
#pragma unroll
                        for (int e = 0; e < 8; ++e) xq[e] = xk[e] = xv[e] = 0.0f;
                    }
                }
                // cumulative log-decay over the chunk (threads 0-127 of the group), e^{G_C}
                if (gt < D) {
                    float g = 0.0f;
#pragma unroll
                    for (int r = 0; r < C; ++r) {
                        g += LA[r * D + gt];
                        LA[r * D + gt] = g;
                    }
                    EGC(bn)[gt] = __expf(g);
                }
            }
        } else if (has_c) {
            // U = T X, O = scale (O1 + P U) -> staging, S <- Diag(Gamma_C) S + Khat^T U
            const uint2 Th = *reinterpret_cast<const uint2 *>(TMh + ln * OPT + 4 * lh);
            const uint2 Tl = *reinterpret_cast<const uint2 *>(TMh + PL_CC + ln * OPT + 4 * lh);
            const uint2 Ph = *reinterpret_cast<const uint2 *>(PMh + ln * OPT + 4 * lh);
            const uint2 Pl = *reinterpret_cast<const uint2 *>(PMh + PL_CC + ln * OPT + 4 * lh);
            uint2 Uh[2], Ul[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                uint2 xh, xl;
                split4(xq + 4 * nt, xh, xl);
                const f32x4_t U = mma16_3(Th, Tl, xh, xl, f32x4_t{0.f, 0.f, 0.f, 0.f});
                const float u4[4] = {U[0], U[1], U[2], U[3]};
                split4(u4, Uh[nt], Ul[nt]);
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                // P U goes to its own accumulator: a K = 16 MFMA accumulating onto the result of
                // a K = 32 MFMA read stale accumulator rows on gfx950 (observed, not documented),
                // so the two chains never share an accumulator and are summed on the VALU.
                const f32x4_t O2 = mma16_3(Ph, Pl, Uh[nt], Ul[nt], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int i = 0; i < 4; ++i) OB[(4 * lh + i) * FPK + col0 + 16 * nt] = (xk[4 * nt + i] + O2[i]) * p.scale;
            }
            const uint16_t *kht = KHTh(bc);
            const float *egc = EGC(bc);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int ch = 16 * t + ln;
                const int ka = ch * OPT + kht_col(ch, 4 * lh);
                const uint2 ah = *reinterpret_cast<const uint2 *>(kht + ka);
                const uint2 al = *reinterpret_cast<const uint2 *>(kht + PL_DC + ka);
                float g4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) g4[i] = egc[16 * t + 4 * lh + i];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[t][nt][i] *= g4[i];
                    S[t][nt] = mma16_3(ah, al, Uh[nt], Ul[nt], S[t][nt]);
                }
            }
        }
        __syncthreads();

        // ================================ segment 3 ================================
        if (prod) {
            if (has_n) {
                // operands of chunk c + 1 (bf16 hi/lo) into buffer bn
                float gl[8];
                Vec8<float>::load(LA, et * D + ec0, gl);
                float kl[8], ql[8], krd[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float E = __expf(gl[e]);
                    const float rE = __expf(-gl[e]);
                    kl[e] = xk[e] * E;
                    ql[e] = xq[e] * E;
                    krd[e] = xk[e] * rE;
                }
                const int pc0 = cperm(ec0), pc1 = cperm(ec0 + 4);
                const int rp = et * OPK;
                uint4 hi, lo;
                uint16_t *klb = KLh(bn), *qlb = QLh(bn), *khtb = KHTh(bn);
                split8(kl, hi, lo);
                *reinterpret_cast<uint2 *>(klb + rp + pc0) = make_uint2(hi.x, hi.y);
                *reinterpret_cast<uint2 *>(klb + rp + pc1) = make_uint2(hi.z, hi.w);
                *reinterpret_cast<uint2 *>(klb + PL_CD + rp + pc0) = make_uint2(lo.x, lo.y);
                *reinterpret_cast<uint2 *>(klb + PL_CD + rp + pc1) = make_uint2(lo.z, lo.w);
                split8(ql, hi, lo);
                *reinterpret_cast<uint2 *>(qlb + rp + pc0) = make_uint2(hi.x, hi.y);
                *reinterpret_cast<uint2 *>(qlb + rp + pc1) = make_uint2(hi.z, hi.w);
                *reinterpret_cast<uint2 *>(qlb + PL_CD + rp + pc0) = make_uint2(lo.x, lo.y);
                *reinterpret_cast<uint2 *>(qlb + PL_CD + rp + pc1) = make_uint2(lo.z, lo.w);
                split8(krd, hi, lo);
                *reinterpret_cast<uint2 *>(KRDh + rp + pc0) = make_uint2(hi.x, hi.y);
                *reinterpret_cast<uint2 *>(KRDh + rp + pc1) = make_uint2(hi.z, hi.w);
                *reinterpret_cast<uint2 *>(KRDh + PL_CD + rp + pc0) = make_uint2(lo.x, lo.y);
                *reinterpret_cast<uint2 *>(KRDh + PL_CD + rp + pc1) = make_uint2(lo.z, lo.w);
                // Khat^T[c][t] = k^_t[c] e^{G_C[c] - G_t[c]}
                const float *egc = EGC(bn);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ch = ec0 + e;
                    uint16_t sh, sl;
                    split1(krd[e] * egc[ch], sh, sl);
                    khtb[ch * OPT + kht_col(ch, et)] = sh;
                    khtb[PL_DC + ch * OPT + kht_col(ch, et)] = sl;
                }
                Vec8<float>::store(VB(bn), et * FPK + ec0, xv);
            }
        } else if (has_c) {
            // epilogue of chunk c: sigma(g) * RMSNorm(o~) * w, then prefetch the next gate rows
            const int r0 = c * C, rend = min(L, r0 + C);
            float o[8];
            Vec8<float>::load(OB, et * FPK + ec0, o);
            if (p.epilogue) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(o[e], o[e], ss);
                ss = group_sum<16>(ss);
                const float inv = rsqrtf(ss * (1.0f / D) + p.rms_eps);
                float g[8];
                IV::unpack(graw, g);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = sigmoidf_(g[e]) * (o[e] * inv) * RW[ec0 + e];
            }
            OutStore<OUT>::store(rows_view(static_cast<char *>(p.o) + (first + static_cast<size_t>(r0) * HD) * sizeof(OUT),
                                           rend - r0, static_cast<uint32_t>(HD * sizeof(OUT)), D * sizeof(OUT)),
                                 static_cast<uint32_t>(et) * static_cast<uint32_t>(HD * sizeof(OUT)) + ec0 * sizeof(OUT), o);
            if (c + 1 < nchunks) load_gate(c + 1);
        }
        __syncthreads();
    }

    // ---- final state and conv cache -----------------------------------------------------------
    if (!prod && p.state_out) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.state_out[sbase_out + static_cast<size_t>(16 * t + 4 * lh + i) * D + col0 + 16 * nt] = S[t][nt][i];
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
                IV::load(p.conv_in, ((static_cast<size_t>(row_in) * 3 + s) * CONV_HIST + (CONV_HIST + pj)) * HD + hD + cg * 8, x);
        }
        __syncthreads();
        if (active)
            IV::store(p.conv_out, ((static_cast<size_t>(row_out) * 3 + s) * CONV_HIST + j) * HD + hD + cg * 8, x);
    }
}

template <typename IO, typename OUT>
hipError_t launch(const LayerParams &p, hipStream_t s) {
    if (p.num_items == 0) return hipSuccess;
    hipLaunchKernelGGL((chunked_pipe_kernel<IO, OUT>), dim3(p.num_items), dim3(THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunked_latency(const LayerParams &p, int io_dtype, int out_dtype, hipStream_t s) {
    if (io_dtype == KDA_DTYPE_BF16)
        return out_dtype == KDA_DTYPE_BF16 ? launch<uint16_t, uint16_t>(p, s)
                                           : launch<uint16_t, float>(p, s);
    return out_dtype == KDA_DTYPE_BF16 ? launch<float, uint16_t>(p, s) : launch<float, float>(p, s);
}

}  // namespace kda
