// kda_chunked.hip -- chunked KDA prefill on the gfx950 matrix cores: two 8-wave
// workgroups share a CU, one per (sequence, head), or per segment of a sequence in
// the segmented prefill.  bf16 io.
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
//   S1      = Diag(Gamma_C) (S0 + Kdiv^T U),  Kdiv = e^{-G} (.) K
//           ( = Diag(Gamma_C) S0 + Khat^T U with Khat = e^{G_C - G} (.) K )
//
// which is the recurrence unrolled over the chunk: u_r = beta_r (v_r -
// (Diag(alpha_r) S_{r-1})^T k_r) is the per-token correction, and stacking
// the u_r gives the unit-lower triangular system (I + A) U = Diag(beta)(V -
// Kbar S0).  The Gram blocks use the factorisation e^{G_s - G_j} =
// e^{G_s} e^{-G_j} within the chunk; at the log-decay floor of -5 per token
// ("Kimi K3's Architecture ...", section "Channel-wise decay, and the floor
// K3 puts under it") a 16-token chunk keeps e^{-G} <= e^80, inside the fp32 /
// bf16 exponent range.  Without the floor (Kimi Linear's unbounded gate, same
// section) a channel can decay further within one chunk; such a chunk is found
// by a vote over the channels' chunk totals and takes the per-token recurrence
// instead, in fp32 on the vector units, with the state in the same registers
// (the position-pair fallback of that section, taken only where it is needed).
//
// Work layout: one workgroup of 8 waves per (sequence, head), walking the
// sequence's chunks; about 69 KB of LDS and at most 128 VGPRs, so two
// workgroups share a CU (four waves per SIMD) and hide each other's
// latencies.  Wave w owns value columns 16w .. 16w+15 of S and keeps that
// 128 x 16 fp32 slice in registers, in the accumulator layout of the 16x16
// MFMAs (lane l holds rows 16t + 4(l/16) + i, column l%16).  Element-wise
// work maps thread x to token x/32 and four adjacent channels 4(x%32) ..
// 4(x%32)+3.  Every contraction runs on v_mfma_f32_16x16x32_bf16.  Those over
// the 16 tokens of a chunk take accumulator tiles directly as their B operand,
// with a lane's 8 K slots carrying the hi and then the lo parts of its 4 tokens.
// Those over the 128 key channels read S from the same registers: K slot 8h + i of a 32-channel step holds
// channel 16(i/4) + 4h + (i%4), so the channel-indexed operands in LDS store
// their channels in that permuted order (the Gram products contract two such
// operands, which the permutation leaves unchanged).
//
// Precision: every contraction splits both operands into bf16 hi + lo parts
// and sums hi*hi + hi*lo + lo*hi in fp32 (three MFMAs), which keeps each
// product to ~2^-16 relative error; S itself stays fp32 throughout.
#include "kda_chunk_common.h"

namespace kda {
namespace {

using namespace chunk;

constexpr int NW = 8;          // waves per workgroup
constexpr int THREADS = NW * 64;


// ------------------------------------------------------------------ LDS map (bytes)

// Kdiv^T plane (the head gate's K^T): row c holds the 16 hi parts of the chunk's tokens,
// then the 16 lo parts, then 4 padding elements (KHTR = 36 bf16), so one 16-byte pair of reads fetches both
// parts of a 4-token group.  Token t sits at t XOR 2 ((c / 16) % 8) inside each part:
// every aligned group of four tokens stays contiguous (the MFMA operand reads; odd
// c / 16 swaps the group's two halves), and both the transposing 16-bit stores (32
// lanes: 32 channels 4 apart, one token) and the operand reads (16 lanes: 16
// consecutive channels) hit 32 distinct banks.
constexpr int KHTR = 2 * C + 4;
__device__ __forceinline__ int kht_pos(int c, int t) { return c * KHTR + (t ^ (2 * ((c >> 4) & 7))); }

// Pre-conv q, k, v rows staged as fp32, row-major [token][stream][128] for token
// positions -3 .. 15 of the chunk: the three history rows come first, so the four
// taps of a token are four fixed offsets from one address.  The history rows persist
// from chunk to chunk; the chunk's own rows are dead once the convolution has read
// them, and share their bytes with the K / Q / Kdiv operand planes written after it.
constexpr int RAW_ROW = 3 * D * 4;                   // one token position, three streams
constexpr int OFF_HIST = 0;                          // positions -3 .. -1
constexpr int OFF_CUR = OFF_HIST + CONV_HIST * RAW_ROW;  // positions 0 .. 15
constexpr int OFF_KL = OFF_CUR;                      // k^ Gamma (= Kbar), channel-permuted      hi,lo
constexpr int OFF_QL = OFF_KL + 2 * PL_CD * 2;       // q^ Gamma (= Qbar), channel-permuted      hi,lo
constexpr int OFF_KRD = OFF_QL + 2 * PL_CD * 2;      // k^ / Gamma (= Kdiv), channel-permuted    hi,lo
constexpr int OFF_KHT = OFF_KRD + 2 * PL_CD * 2;     // Kdiv^T [channel][hi 16 | lo 16 | pad]   swizzled
constexpr int OFF_V = OFF_KHT + D * KHTR * 2;        // fp32 [16][132]
constexpr int OFF_LA = OFF_V + C * FPK * 4;          // log2(alpha) -> cumulative, fp32 [16][128]
// fp32 [16][132] output rows of a chunk: written at its state update, read by its epilogue
// during the next chunk's Gram / T phase
constexpr int OFF_O = OFF_LA + C * D * 4;
constexpr int OFF_PM = OFF_O + C * FPK * 4;          // P                                        hi,lo [16][20]
constexpr int OFF_TM = OFF_PM + 2 * PL_CC * 2;       // T                                        hi,lo [16][20]
constexpr int OFF_BETA = OFF_TM + 2 * PL_CC * 2;     // fp32 [16]
constexpr int OFF_EGC = OFF_BETA + C * 4;            // e^{G_C} fp32 [128]
constexpr int OFF_CW = OFF_EGC + D * 4;              // conv weights fp32 [3 streams][4 taps][128]
constexpr int OFF_RW = OFF_CW + 3 * 4 * D * 4;       // rms gain fp32 [128]
constexpr int OFF_GH = OFF_RW + D * 4;               // head gate: cumulative log2-decay [16], e^{G_C}
constexpr int LDS_BYTES = OFF_GH + 32 * 4;
// In-kernel low-rank gate: the chunk's z_down rows, bf16 [16][r + 8] (r <= 128)
constexpr int ZPK = 128 + 8;
constexpr int OFF_ZL = LDS_BYTES;
constexpr int LDS_BYTES_LOWRANK = OFF_ZL + C * ZPK * 2;

// Per-token path of a chunk whose decay leaves the factorised range: fp32 k^ and q^ rows
// [16][FPK] in the K / Q planes; alpha [16][128] in the Kdiv^T plane, written with the
// running sums (that plane is free from the first barrier of a chunk until the operands
// are built, and a chunk on this path builds no Kdiv^T; the planes before it hold the
// staged rows that the convolution is still reading then); the V rows; outputs go to the
// output rows as on the matrix-core path.  The vote flag shares the head-gate slot.
constexpr int OFF_KF = OFF_KL;
constexpr int OFF_QF = OFF_KF + C * FPK * 4;
constexpr int OFF_AL = OFF_KHT;
constexpr int OFF_FLAG = OFF_GH;
// a chunk keeps the factorised path while every channel's decay over it stays above
// 2^-WIDE_LOG2: e^{-G} <= 2^116 then, and the lo parts of e^{G} k^ stay normal in bf16
constexpr float WIDE_LOG2 = 116.0f;
static_assert(OFF_QF + C * FPK * 4 <= OFF_KRD, "fp32 k^ and q^ rows must fit in the K / Q planes");
static_assert(C * D * 4 <= D * KHTR * 2, "alpha must fit in the Kdiv^T plane");
static_assert(OFF_AL >= OFF_CUR + C * RAW_ROW, "alpha, written during the convolution, must not overlap the staged rows");
static_assert(C * RAW_ROW <= OFF_KHT - OFF_CUR, "staged rows must fit under the K / Q / Kdiv planes");
static_assert(2 * LDS_BYTES_LOWRANK <= 160 * 1024, "two workgroups per gfx950 CU");

constexpr float LOG2E = 1.4426950408889634f;


// What a workgroup runs.  WHOLE: a whole sequence from its given state.  In the segmented
// prefill, the first pass runs FIRST (segment 0, from the given state, entering state of
// segment 1 out), M (a middle segment from S = I with v = 0: its transition matrix) and
// B (the same segment from S = 0: its offset), and the second pass RERUNs segments 1 ..
// from the state the scan gave them; only the last segment writes the final state and
// conv cache.
enum Role { WHOLE, FIRST, SEG_M, SEG_B, RERUN, SKIP };

struct Place {
    int n, h, len, role, slot;
    int32_t ts;   // first token of the segment within the sequence
    bool last;    // the sequence ends with this segment
};

__device__ __forceinline__ Place place_whole(const LayerParams &p, int item) {
    Place w;
    w.h = item % p.H;
    const int idx = item / p.H;
    w.n = p.order ? p.order[idx] : idx;
    w.ts = 0;
    w.len = p.cu_seqlens[w.n + 1] - p.cu_seqlens[w.n];
    w.role = WHOLE;
    w.slot = 0;
    w.last = true;
    return w;
}

// pass 1 items: [2][slots][H] (the second half runs B); pass 3 items: [slots][H]
__device__ __forceinline__ Place place_segment(const LayerParams &p, int item) {
    Place w;
    const int per = p.seg_slots * p.H;
    const int which = item / per;
    const int rem = item - which * per;
    w.slot = rem / p.H;
    w.h = rem - w.slot * p.H;
    const SegDesc d = p.seg[w.slot];
    w.n = d.n;
    w.ts = d.ts;
    w.len = d.len;
    w.last = d.p == d.np - 1;
    if (d.n < 0)
        w.role = SKIP;
    else if (p.seg_pass == 1)
        w.role = d.p == 0 ? (which ? SKIP : (w.last ? WHOLE : FIRST)) : (w.last ? SKIP : (which ? SEG_B : SEG_M));
    else
        w.role = d.p == 0 ? SKIP : RERUN;
    return w;
}

// The second bound is waves per SIMD: two workgroups of 8 waves per CU need four
// (at most 128 VGPRs).
// GATE (KDA_GATE_*): log alpha read per channel, formed in the kernel from the low-rank
// gate factors (bf16 io; K3's floored sigmoid or Kimi Linear's softplus), or read as one
// value per (token, head).  WIDE: chunks whose decay leaves the factorised range take the
// per-token path (decays without a floor).  SEG: a workgroup runs one segment of a
// sequence in a pass of the segmented prefill (Role).
template <typename IO, typename OUT, int GATE, bool WIDE, bool SEG>
__global__ __launch_bounds__(THREADS, 4) void chunked_tp_kernel(LayerParams p) {
    constexpr bool SOFTPLUS = GATE == KDA_GATE_LOWRANK_SOFTPLUS;
    constexpr bool LOWRANK = GATE == KDA_GATE_LOWRANK || SOFTPLUS;
    // One decay per (token, head): Gamma is a row scale of the chunk's tokens, so it leaves
    // the channel contractions.  The operand planes hold k^ and q^ unscaled (the k^ plane
    // also serves as the Gram's B operand and, transposed, as Khat^T), and the factors are
    // applied to the 16 x 16 Gram tiles and to the rows of the products: X = V - Diag(Gamma)
    // (K^ S), O1 = Diag(Gamma) (Q^ S), S <- Gamma_C S + K^T (Diag(e^{G_C - G}) U).
    constexpr bool HEADG = GATE == KDA_GATE_HEAD;
    static_assert(!(HEADG && WIDE), "the head gate's factors never exceed 1");
    using IV = Vec8<IO>;   // eight-wide rows of the conv cache
    using I4 = Vec4<IO>;
    using IB = BufLoad4<IO>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LOWRANK ? LDS_BYTES_LOWRANK : LDS_BYTES];
    float *const RAW = reinterpret_cast<float *>(smem + OFF_HIST);  // [3 + 16][3][128]
    uint16_t *const KLh = reinterpret_cast<uint16_t *>(smem + OFF_KL);
    uint16_t *const QLh = reinterpret_cast<uint16_t *>(smem + OFF_QL);
    uint16_t *const KRDh = reinterpret_cast<uint16_t *>(smem + OFF_KRD);
    uint16_t *const KHTh = reinterpret_cast<uint16_t *>(smem + OFF_KHT);
    uint16_t *const PMh = reinterpret_cast<uint16_t *>(smem + OFF_PM);
    uint16_t *const TMh = reinterpret_cast<uint16_t *>(smem + OFF_TM);
    float *const OB = reinterpret_cast<float *>(smem + OFF_O);
    float *const VB = reinterpret_cast<float *>(smem + OFF_V);
    float *const LA = reinterpret_cast<float *>(smem + OFF_LA);
    float *const BETA = reinterpret_cast<float *>(smem + OFF_BETA);
    float *const EGC = reinterpret_cast<float *>(smem + OFF_EGC);
    float *const CW = reinterpret_cast<float *>(smem + OFF_CW);
    float *const RW = reinterpret_cast<float *>(smem + OFF_RW);
    float *const GH = reinterpret_cast<float *>(smem + OFF_GH);  // head gate only
    uint16_t *const ZL = reinterpret_cast<uint16_t *>(smem + OFF_ZL);  // LOWRANK only
    float *const KF = reinterpret_cast<float *>(smem + OFF_KF);          // per-token path only
    float *const QF = reinterpret_cast<float *>(smem + OFF_QF);
    float *const AL = reinterpret_cast<float *>(smem + OFF_AL);
    int *const FLAG = reinterpret_cast<int *>(smem + OFF_FLAG);

    const int H = p.H;
    const Place pl = SEG ? place_segment(p, blockIdx.x) : place_whole(p, blockIdx.x);
    if (pl.role == SKIP) return;  // the whole workgroup, before any barrier
    const int h = pl.h;
    const int n = pl.n;
    const int64_t t0 = static_cast<int64_t>(p.cu_seqlens[n]) + pl.ts;  // first token of the run
    const int L = pl.len;
    const int role = pl.role;
    const bool has_out = role == WHOLE || role == FIRST || role == RERUN;  // writes o
    // q enters only the outputs: the M and B runs of the segmented prefill skip its
    // convolution, operands and products, and the M run (v = 0) the convolution of v
    const bool qside = !SEG || has_out;
    const size_t HD = static_cast<size_t>(H) * D;
    const size_t hD = static_cast<size_t>(h) * D;

    const int tid = threadIdx.x;
    // the wave index is the same in every lane of a wave: read it into a scalar, so that the
    // per-wave roles below branch on scalars and their buffer views need no lane reads
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int ln = lane & 15;        // MFMA row / column index
    const int lh = lane >> 4;        // MFMA K group
    const int et = tid >> 5;         // element-wise token (0..15)
    const int ec0 = (tid & 31) * 4;  // element-wise first channel
    const int col = wave * 16 + ln;  // value column of this lane's accumulator tiles

    // ---- per-head constants -----------------------------------------------------------
    // The q and k weights are stored times log2(e): the convolution then yields
    // z = log2(e) x, so that sigma(x) = 1 / (1 + 2^-z) needs no further scaling, and
    // SiLU(x) log2(e) = z sigma(x), a constant factor that the L2 normalisation removes
    // (its epsilon is scaled by log2(e)^2 to match).
    if (p.prologue) {
        for (int i = tid; i < 3 * D; i += THREADS) {
            const int s = i / D, c = i % D;
            const float4 w = *reinterpret_cast<const float4 *>(p.conv_w + ((s * HD) + hD + c) * 4);
            const float f = s < 2 ? LOG2E : 1.0f;
            CW[(s * 4 + 0) * D + c] = w.x * f;
            CW[(s * 4 + 1) * D + c] = w.y * f;
            CW[(s * 4 + 2) * D + c] = w.z * f;
            CW[(s * 4 + 3) * D + c] = w.w * f;
        }
    }
    if (tid < D) RW[tid] = p.rms_w ? p.rms_w[tid] : 1.0f;
    const float l2_eps = p.l2_eps * (LOG2E * LOG2E);
    // low-rank gate: this lane's channel bias and e^{A_h} log2(e) (inside the sigmoid), or
    // e^{A_h} (outside the softplus, which works in log2 units)
    const float gscale = LOWRANK ? __expf(p.gate_a[h]) * (SOFTPLUS ? 1.0f : LOG2E) : 0.0f;
    // the bias times the factor that multiplies z + b (so that one fma forms it)
    const float gbias = LOWRANK ? p.gate_bias[hD + col] * (SOFTPLUS ? LOG2E : gscale) : 0.0f;

    // ---- state slice in accumulator layout: S[t][i] = S(16t + 4lh + i, col) ----------------
    const int row_in = p.slots_in ? p.slots_in[n] : n;     // state_in / conv_in row
    const int row_out = p.slots_out ? p.slots_out[n] : n;  // state_out / conv_out row
    // entering state: the given one, the one the scan left in the previous slot's B, or
    // (M) the identity, or (B) zero
    const float *s_src = nullptr;
    if ((role == WHOLE || role == FIRST) && p.state_in)
        s_src = p.state_in + (static_cast<size_t>(row_in) * H + h) * D * D;
    else if (SEG && role == RERUN)
        s_src = p.seg_b + (static_cast<size_t>(pl.slot - 1) * H + h) * D * D;
    f32x4_t S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * t + 4 * lh + i;
            S[t][i] = s_src ? s_src[static_cast<size_t>(r) * D + col] : (SEG && role == SEG_M && r == col ? 1.0f : 0.0f);
        }
    // Settle the state loads here, once: the state's first readers in the loop are written
    // out as assembly, and without this the compiler waits for every outstanding memory
    // operation before them in each chunk (the next chunk's rows included).
#pragma unroll
    for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(S[t]));

    const int nchunks = (L + C - 1) / C;

    // Current-row loads of a chunk (q, k, v, log alpha, beta): issued one chunk ahead,
    // right after the previous chunk's staging, so that a whole chunk of work hides them.
    typename I4::Raw cur[3];
    typename Vec4<float>::Raw lar;
    float lah = 0.0f;  // head gate: this token's log alpha
    float bet = 0.0f;
    // byte addresses of this (sequence, head)'s first row in each token-major tensor; a
    // chunk's rows start C rows further per chunk, and offsets inside a chunk fit 32 bits
    const uint32_t rowb_io = static_cast<uint32_t>(HD * sizeof(IO));
    const uint32_t rowb_f = static_cast<uint32_t>(HD * 4);
    const size_t first = static_cast<size_t>(t0) * HD + hD;
    const char *qkv_base[3] = {static_cast<const char *>(p.q) + first * sizeof(IO),
                               static_cast<const char *>(p.k) + first * sizeof(IO),
                               static_cast<const char *>(p.v) + first * sizeof(IO)};
    const char *la_base = LOWRANK ? nullptr
                          : HEADG ? reinterpret_cast<const char *>(p.log_alpha + static_cast<size_t>(t0) * H + h)
                                  : reinterpret_cast<const char *>(p.log_alpha + first);
    const char *beta_base = reinterpret_cast<const char *>(p.beta + static_cast<size_t>(t0) * H + h);
    // (without an epilogue the g views hold no rows and read nothing: any base will do)
    const char *g_base = static_cast<const char *>(p.epilogue ? p.g : p.q) + first * sizeof(IO);
    char *o_base = static_cast<char *>(p.o) + first * sizeof(OUT);

    // Low-rank gate: z_down rows of a chunk (fetched with the chunk's q, k, v rows a whole
    // chunk ahead, parked in ZL when the chunk starts) and this lane's W_up operand (the B
    // operand of z_down W_up^T for the channels 16 wave .. 16 wave + 15, fetched at the end
    // of the previous chunk's state update, so that the staging phase covers its latency).
    const int rank = p.gate_rank;
    const int zsteps = rank / 32;
    uint2 zr = make_uint2(0u, 0u);
    uint4 wb[4];
    const char *z_base = LOWRANK ? static_cast<const char *>(p.gate_z) + static_cast<size_t>(t0) * rank * 2 : nullptr;
    auto load_z = [&](int c) {
        const int x = opaque(tid), xt = x >> 5, xc = (x & 31) * 4;
        const int r0 = c * C, nrow = min(L, r0 + C) - r0;
        const __amdgpu_buffer_rsrc_t v = rows_view(z_base + static_cast<size_t>(r0) * rank * 2, nrow, rank * 2, rank * 2);
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t z = __builtin_amdgcn_raw_buffer_load_b64(v, static_cast<uint32_t>(xt * rank + xc) * 2u, 0, 0);
        zr = make_uint2(z[0], z[1]);  // (lanes past the rank are not parked)
    };
    // Per-thread offsets of the prefetches are rebuilt from an opaque copy of the thread
    // index at each use rather than kept live across the loop: a spilled offset would
    // be reloaded with a wait that also drains the prefetches in flight.
    auto load_current = [&](int c) {
        const int x = opaque(tid), xt = x >> 5, xc = (x & 31) * 4;
        const int r0 = c * C, nrow = min(L, r0 + C) - r0;
        const size_t cio = static_cast<size_t>(r0) * rowb_io;
        const uint32_t off_io = static_cast<uint32_t>(xt) * rowb_io + xc * sizeof(IO);
#pragma unroll
        for (int s = 0; s < 3; ++s)
            cur[s] = IB::load(rows_view(qkv_base[s] + cio, nrow, rowb_io, D * sizeof(IO)), off_io);
        if (HEADG)
            lah = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rows_view(la_base + static_cast<size_t>(r0) * H * 4, nrow, H * 4, 4), static_cast<uint32_t>(xt * H) * 4u, 0, 0));
        else if (!LOWRANK)
            lar = BufLoad4<float>::load(rows_view(la_base + static_cast<size_t>(r0) * rowb_f, nrow, rowb_f, D * 4),
                                        static_cast<uint32_t>(xt) * rowb_f + xc * 4u);
        bet = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rows_view(beta_base + static_cast<size_t>(r0) * H * 4, nrow, H * 4, 4), static_cast<uint32_t>(xt * H) * 4u, 0, 0));
        if (LOWRANK) load_z(c);
    };
    auto park_z = [&]() {
        const int x = opaque(tid), xt = x >> 5, xc = (x & 31) * 4;
        if (xc < rank) *reinterpret_cast<uint2 *>(ZL + xt * ZPK + xc) = zr;
    };
    auto load_w = [&]() {
        const int x = opaque(tid), xl = x & 63;
        const __amdgpu_buffer_rsrc_t wv =
            rows_view(static_cast<const char *>(p.gate_w) + hD * rank * 2, D, rank * 2, rank * 2);
        const uint32_t off = (static_cast<uint32_t>((x >> 6) * 16 + (xl & 15)) * rank + 8 * (xl >> 4)) * 2u;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            // a step past the rank reads past this lane's row: zeros
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wv, st < zsteps ? off + 64u * st : 0x80000000u, 0, 0);
            wb[st] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    // The epilogue of a chunk runs on waves 2, 3, 6 and 7 during the next chunk's Gram / T
    // phase, where they would otherwise wait for the triangular solve of wave 0.  Wave w shares
    // its SIMD with wave w + 4, so these four waves sit on the two SIMDs that do not host the
    // Gram / T waves 0 and 1 (on waves 4-7 instead, the epilogue took issue slots from them and
    // the launch ran 2.5% longer).  Epilogue thread x (0 .. 255, waves 2, 3, 6, 7 in order)
    // takes token x / 16 and channels 8 (x % 16) .. + 7, so a token's 128 channels form one
    // 16-lane row and its RMS sum takes four DPP steps.  Every wave issues the same memory
    // operations in the same order whether or not it has outputs (views without bytes are
    // dropped without a memory access), so that the wait for a chunk's rows always counts the
    // same younger operations and never has to wait for an output store as well.
    const bool epi_wave = (wave & 2) != 0;
    auto epi_thread = [&]() {
        const int t = opaque(tid), w = t >> 6;
        return ((((w >> 1) & 2) | (w & 1)) << 6) | (t & 63);
    };
    const bool do_epi = !SEG || has_out;
    typename Vec8<IO>::Raw graw;
    // g rows of chunk c for the epilogue threads (use = false: an empty load in their place)
    auto load_gate = [&](int c, bool use) {
        const int x = epi_thread();
        use = use && p.epilogue && do_epi && epi_wave;
        const int r0 = c * C;
        const int nrow = use ? min(L, r0 + C) - r0 : 0;
        const char *const gb = g_base + static_cast<size_t>(r0) * rowb_io;  // no rows when unused
        graw = BufLoad8<IO>::load(rows_view(gb, nrow, rowb_io, D * sizeof(IO)),
                                  use ? static_cast<uint32_t>(x >> 4) * rowb_io + (x & 15) * 8 * sizeof(IO) : 0u);
    };
    // the memory operations of an epilogue's output store, dropped
    auto store_dummy = [&]() {
        const __amdgpu_buffer_rsrc_t none = rows_view(o_base, 0, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(0u, none, 0u, 0, 0);
        if (sizeof(OUT) == 4) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 0u, 0, 0);
    };
    // sigma(g) * RMSNorm(o~) * w of chunk c from its output rows (epilogue waves only)
    auto epilogue = [&](int c) {
        const int x = epi_thread(), xt = x >> 4, xc = (x & 15) * 8;
        const int r0 = c * C, nrow = min(L, r0 + C) - r0;
        float o[8];
        load4f(OB + xt * FPK + xc, o);
        load4f(OB + xt * FPK + xc + 4, o + 4);
        if (p.epilogue) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(o[e], o[e], ss);
            ss += dpp<0xB1>(ss);   // quad_perm [1, 0, 3, 2]
            ss += dpp<0x4E>(ss);   // quad_perm [2, 3, 0, 1]
            ss += dpp<0x141>(ss);  // row_half_mirror
            ss += dpp<0x140>(ss);  // row_mirror: the sum over the 16-lane row
            const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.rms_eps);
            float g[8], rw[8];
            Vec8<IO>::unpack(graw, g);
            load4f(RW + xc, rw);
            load4f(RW + xc + 4, rw + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = sigmoidf_(g[e]) * (o[e] * inv) * rw[e];
        }
        OutStore<OUT>::store(rows_view(o_base + static_cast<size_t>(r0) * HD * sizeof(OUT), nrow,
                                       static_cast<uint32_t>(HD * sizeof(OUT)), D * sizeof(OUT)),
                             static_cast<uint32_t>(xt) * static_cast<uint32_t>(HD * sizeof(OUT)) + xc * sizeof(OUT), o);
    };
    // At the start of chunk ch's Gram / T phase: the outputs of chunk ch - 1 (or the same
    // memory operations, dropped).  At the end of its state update: the g rows of chunk ch
    // and the low-rank gate's W_up operand for chunk ch + 1, so that neither is held in
    // registers through the triangular solve and the state products.
    auto epilogue_stage = [&](int ch) {
        if (epi_wave && do_epi && ch > 0)
            epilogue(ch - 1);
        else
            store_dummy();
    };
    auto next_loads = [&](int ch) {
        load_gate(ch, true);
        if (LOWRANK) load_w();  // this lane's W_up operand, for the next chunk's gate
    };
    if (p.prologue && tid < 3 * CONV_HIST * 16) {
        // history of the first chunk: the given conv cache (oldest first) or zeros
        const int s = tid / (CONV_HIST * 16), j = (tid / 16) % CONV_HIST, c0 = (tid & 15) * 8;
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (SEG && pl.ts > 0) {  // a later segment: the sequence's own preceding inputs
            const void *srcs[3] = {p.q, p.k, p.v};
            IV::load(srcs[s], static_cast<size_t>(t0 - CONV_HIST + j) * HD + hD + c0, x);
        } else if (p.conv_in) {
            IV::load(p.conv_in, ((static_cast<size_t>(row_in) * 3 + s) * CONV_HIST + j) * HD + hD + c0, x);
        }
        store4f(RAW + (j * 3 + s) * D + c0, x);
        store4f(RAW + (j * 3 + s) * D + c0 + 4, x + 4);
    }

    if (nchunks > 0) {
        load_current(0);
        // the memory operations of an epilogue stage (an empty store and an empty g load):
        // the same operations then follow a chunk's rows on both ways into the loop, and the
        // wait for the rows at the top of the loop need not cover the output store
        store_dummy();
        load_gate(0, false);
        if (LOWRANK) load_w();
    }
    // this thread's staged row (position et) and the same row three positions earlier
    float *const raw_t = RAW + ((CONV_HIST + et) * 3) * D + ec0;

    for (int ch = 0; ch < nchunks; ++ch) {
        const int r0 = ch * C;                 // first position of the chunk
        const int rend = min(L, r0 + C);       // end of the chunk's valid rows
        const int pos = r0 + et;               // this thread's token position
        const bool valid = pos < L;

        // ---- 1. stage this chunk's rows (fetched during the previous chunk) as fp32 -----------
        float xr[3][4];  // this thread's pre-conv values: tap 0 of its convolution
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            I4::unpack(cur[s], xr[s]);
            store4f(raw_t + s * D, xr[s]);
        }
        if (LOWRANK) {
            park_z();  // ZL was last read before the previous chunk's second barrier
        } else if (HEADG) {
            if ((tid & 31) == 0) GH[opaque(tid) >> 5] = lah * LOG2E;
        } else {
            float la[4];
            Vec4<float>::unpack(lar, la);
#pragma unroll
            for (int e = 0; e < 4; ++e) la[e] *= LOG2E;
            store4f(LA + et * D + ec0, la);
        }
        // (the address from an opaque thread index: a spilled address costs a reload that waits
        // for every memory operation in flight)
        if ((tid & 31) == 0) BETA[opaque(tid) >> 5] = p.beta_logit ? sigmoidf_(bet) : bet;
        if (WIDE && tid == 0) *FLAG = 0;
        // the next chunk's rows: a whole chunk of work hides their latency (past the last
        // chunk the views are empty: zeros, no memory access, and the same count of memory
        // operations on every path, so that later waits stay exact)
        load_current(ch + 1);
        __syncthreads();

        // ---- 2. conv4 + SiLU (+ L2 for q, k) from the staged rows; cumulative log-decay -------
        // Wave priorities rise through the chunk: staging and the epilogue 0, the convolution 1,
        // the operands and the products 2, the Gram blocks and T 3, the state update 3.  When
        // two workgroups share a CU, the one further into its chunk (its matrix-core chains,
        // short on instructions but long in latency) then issues ahead of the other's
        // vector-heavy phases, which fill the gaps; with the arbiter's default (older waves
        // first) one workgroup of the pair ran far behind the other.
        __builtin_amdgcn_s_setprio(1);
        f32x4_t zacc = {0.f, 0.f, 0.f, 0.f};
        if (LOWRANK) {
            // log2(alpha) = -5 log2(e) sigmoid(e^{A_h} (z_down W_up^T + b)) for the chunk's
            // tokens (rows) and this wave's 16 channels (columns), on the matrix cores (the
            // bf16 factors multiply exactly and accumulate in fp32), then its running sum
            // over the tokens: within the lane's 4 rows, then across the 4 row groups with
            // two lane permutes.  Rows past the end of the sequence get log alpha = 0, so
            // that they do not decay the carried state.
            // (LDS addresses from an opaque lane index, as elsewhere: a spilled address costs a
            // reload that waits for every memory operation in flight)
            const int y = opaque(lane);
            const uint16_t *const zrow = ZL + (y & 15) * ZPK + 8 * (y >> 4);
#pragma unroll
            for (int st = 0; st < 4; ++st)
                if (st < zsteps) zacc = mma(*reinterpret_cast<const uint4 *>(zrow + 32 * st), wb[st], zacc);
        }
        float xq[4], xk[4], xv[4];
        {
            float *outs[3] = {xq, xk, xv};
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                float *a = outs[s];
                if (SEG && ((s == 0 && !qside) || (s == 2 && role == SEG_M))) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[e] = 0.0f;
                    continue;
                }
                if (p.prologue) {
                    float acc[4], w[4];
                    load4f(CW + (s * 4) * D + ec0, w);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = w[e] * xr[s][e];
#pragma unroll
                    for (int j = 1; j <= 3; ++j) {
                        float xj[4];
                        load4f(raw_t + (s - 3 * j) * D, xj);
                        load4f(CW + (s * 4 + j) * D + ec0, w);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[e] = fmaf(w[e], xj[e], acc[e]);
                    }
                    if (s < 2) {  // acc = log2(e) x:  z sigma(x) = z / (1 + 2^-z)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            a[e] = acc[e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-acc[e]));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[e] = siluf_(acc[e]);
                    }
                } else {
                    const float f = s == 0 ? p.scale : 1.0f;  // q carries the read scale
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[e] = xr[s][e] * f;
                }
            }
            if (p.prologue) {
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sq = fmaf(xq[e], xq[e], sq);
                    sk = fmaf(xk[e], xk[e], sk);
                }
                sq = half_wave_sum(sq);
                sk = half_wave_sum(sk);
                // q also carries the read scale (O = scale (Qbar S + P U) is linear in q)
                const float iq = __builtin_amdgcn_rsqf(sq + l2_eps) * p.scale, ik = __builtin_amdgcn_rsqf(sk + l2_eps);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xq[e] *= iq;
                    xk[e] *= ik;
                }
                // padding tokens past the end of a partial chunk see real history rows: clear
                // them (a branch on the chunk, the same in every thread, skips this for full ones)
                if (rend - r0 < C && !valid) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) xq[e] = xk[e] = xv[e] = 0.0f;
                }
            }
        }
        if (LOWRANK) {
            // the rest of the gate, after the convolution, which hides the latency of the
            // z_down W_up^T products
            const int y = opaque(lane), yl = y & 15, yh = y >> 4, ycol = wave * 16 + yl;
            float run[4];
            float acc_sum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float la2;
                if (SOFTPLUS) {
                    // -e^{A_h} softplus(u) log2(e) = -e^{A_h} log2(1 + 2^t), t = u log2(e),
                    // as max(t, 0) + log2(1 + 2^-|t|) so that 2^t never overflows
                    const float t = fmaf(zacc[i], LOG2E, gbias);
                    la2 = -gscale * (fmaxf(t, 0.0f) + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-fabsf(t))));
                } else {
                    const float t = fmaf(zacc[i], gscale, gbias);  // e^{A_h} (z + b) log2(e)
                    la2 = (-5.0f * LOG2E) * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t));
                }
                la2 = r0 + 4 * yh + i < L ? la2 : 0.0f;
                if (WIDE) AL[(4 * yh + i) * D + ycol] = __builtin_amdgcn_exp2f(la2);
                acc_sum += la2;
                run[i] = acc_sum;
            }
            float x1 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((y - 16) * 4, __builtin_bit_cast(int, acc_sum)));
            x1 = acc_sum + (yh >= 1 ? x1 : 0.0f);
            float x2 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((y - 32) * 4, __builtin_bit_cast(int, x1)));
            x2 = x1 + (yh >= 2 ? x2 : 0.0f);
            const float before = x2 - acc_sum;  // sum over the rows of the earlier row groups
            float *const larow = LA + 4 * yh * D + ycol;
#pragma unroll
            for (int i = 0; i < 4; ++i) larow[i * D] = run[i] + before;
            if (yh == 3) {
                EGC[ycol] = __builtin_amdgcn_exp2f(run[3] + before);
                if (WIDE && run[3] + before < -WIDE_LOG2) *FLAG = 1;
            }
        }
        if (SEG && role == SEG_M) {  // the transition matrix: the recurrence with v = 0
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[e] = 0.0f;
        }
        if (HEADG) {
            if (tid == 0) {
                float g = 0.0f;
#pragma unroll
                for (int r = 0; r < C; ++r) {
                    g += GH[r];
                    GH[r] = g;
                }
                GH[C] = __builtin_amdgcn_exp2f(g);
            }
        } else if (!LOWRANK && tid < D) {
            const int c = tid;
            float g = 0.0f;
#pragma unroll
            for (int r = 0; r < C; ++r) {
                const float x = LA[r * D + c];
                if (WIDE) AL[r * D + c] = __builtin_amdgcn_exp2f(x);  // for the per-token path
                g += x;
                LA[r * D + c] = g;
            }
            EGC[c] = __builtin_amdgcn_exp2f(g);
            if (WIDE && g < -WIDE_LOG2) *FLAG = 1;
        }
        __syncthreads();
        // one channel decays past the factorised range within this chunk: the chunk takes
        // the per-token path (the same value in every thread)
        const bool wide = WIDE && *FLAG != 0;

        // ---- 3. staged operands (bf16 hi/lo); the next chunk's conv history ------------------
        __builtin_amdgcn_s_setprio(2);  // (the order of the phases' priorities: see the convolution)
        if (et >= C - CONV_HIST) {
            // the last three positions become positions -3 .. -1 of the next chunk (the
            // convolution has read the old ones: the barrier above orders it)
#pragma unroll
            for (int s = 0; s < 3; ++s) store4f(raw_t + (s - 3 * C) * D, xr[s]);
        }
        if (wide) {
            // fp32 k^, q^ and v (the per-token alpha is in place since the gate stage)
            store4f(KF + et * FPK + ec0, xk);
            store4f(QF + et * FPK + ec0, xq);
            store4f(VB + et * FPK + ec0, xv);
        } else if (HEADG) {
            // k^ and q^ unscaled; the k^ split also fills the transposed K^T plane
            const int at = et * OPK + cperm(ec0);
            uint2 qhi, qlo, hi, lo;
            split4x2_dot(xq, xk, qhi, qlo, hi, lo);
            *reinterpret_cast<uint2 *>(QLh + at) = qhi;
            *reinterpret_cast<uint2 *>(QLh + PL_CD + at) = qlo;
            *reinterpret_cast<uint2 *>(KLh + at) = hi;
            *reinterpret_cast<uint2 *>(KLh + PL_CD + at) = lo;
            const uint32_t hw[4] = {hi.x, hi.x >> 16, hi.y, hi.y >> 16};
            const uint32_t lw[4] = {lo.x, lo.x >> 16, lo.y, lo.y >> 16};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = ec0 + e;
                KHTh[kht_pos(c, et)] = static_cast<uint16_t>(hw[e]);
                KHTh[C + kht_pos(c, et)] = static_cast<uint16_t>(lw[e]);
            }
            store4f(VB + et * FPK + ec0, xv);
        } else {
            float gl[4];
            load4f(LA + et * D + ec0, gl);
            float kl[4], ql[4], krd[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float E = __builtin_amdgcn_exp2f(gl[e]);
                const float rE = __builtin_amdgcn_exp2f(-gl[e]);
                kl[e] = xk[e] * E;
                ql[e] = xq[e] * E;
                krd[e] = xk[e] * rE;
            }
            // channels ec0 .. ec0+3 keep their order at channel-permuted position cperm(ec0)
            const int at = et * OPK + cperm(ec0);
            uint2 hi, lo, h2, l2;
            split4x2_dot(kl, krd, hi, lo, h2, l2);
            *reinterpret_cast<uint2 *>(KLh + at) = hi;
            *reinterpret_cast<uint2 *>(KLh + PL_CD + at) = lo;
            *reinterpret_cast<uint2 *>(KRDh + at) = h2;
            *reinterpret_cast<uint2 *>(KRDh + PL_CD + at) = l2;
            if (qside) {  // q^ Gamma (stored when q is used)
                split4_dot(ql, hi, lo);
                *reinterpret_cast<uint2 *>(QLh + at) = hi;
                *reinterpret_cast<uint2 *>(QLh + PL_CD + at) = lo;
            }
            // the state update takes k^ / Gamma transposed: Kdiv^T[c][t] = k^_t[c] e^{-G_t[c]}
            const uint32_t hw[4] = {h2.x, h2.x >> 16, h2.y, h2.y >> 16};
            const uint32_t lw[4] = {l2.x, l2.x >> 16, l2.y, l2.y >> 16};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = ec0 + e;
                KHTh[kht_pos(c, et)] = static_cast<uint16_t>(hw[e]);
                KHTh[C + kht_pos(c, et)] = static_cast<uint16_t>(lw[e]);
            }
            store4f(VB + et * FPK + ec0, xv);
        }
        __syncthreads();
        if (wide) {
            // ---- 4-5, per-token path: for each token u of the chunk in order,
            //   S <- Diag(alpha_u) S;  r = S^T k_u;  du = beta_u (v_u - r);
            //   S <- S + k_u du^T;     o~_u = S^T q_u   (q carries the read scale)
            // in two passes over the lane's rows, each ending in one column sum over the four
            // row groups.  Lane (lh, ln) of wave w holds rows 16t + 4lh + i of column
            // 16w + ln; each row step waits for its own two operand loads (with more of them
            // in flight the loop needs registers that the matrix-core path then spills).
            // The lane offsets are rebuilt from an opaque thread index rather than kept live.
            // First the previous chunk's epilogue, which reads the output rows this path rewrites.
            epilogue_stage(ch);
            __syncthreads();
            const int x = opaque(tid);
            const int lrow = 4 * ((x & 63) >> 4), lcol = ((x >> 6) << 4) + (x & 15);
            for (int u = 0; u < rend - r0; ++u) {
                const float *const al = AL + u * D + lrow;
                const float *const kf = KF + u * FPK + lrow;
                const float *const qf = QF + u * FPK + lrow;
                float r4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float4 a4 = *reinterpret_cast<const float4 *>(al + 16 * t);
                    const float4 k4 = *reinterpret_cast<const float4 *>(kf + 16 * t);
                    S[t][0] *= a4.x;
                    S[t][1] *= a4.y;
                    S[t][2] *= a4.z;
                    S[t][3] *= a4.w;
                    r4[0] = fmaf(S[t][0], k4.x, r4[0]);
                    r4[1] = fmaf(S[t][1], k4.y, r4[1]);
                    r4[2] = fmaf(S[t][2], k4.z, r4[2]);
                    r4[3] = fmaf(S[t][3], k4.w, r4[3]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const float r = row_group_sum((r4[0] + r4[1]) + (r4[2] + r4[3]));
                const float du = BETA[u] * (VB[u * FPK + lcol] - r);
                float o4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float4 k4 = *reinterpret_cast<const float4 *>(kf + 16 * t);
                    const float4 q4 = *reinterpret_cast<const float4 *>(qf + 16 * t);
                    S[t][0] = fmaf(k4.x, du, S[t][0]);
                    S[t][1] = fmaf(k4.y, du, S[t][1]);
                    S[t][2] = fmaf(k4.z, du, S[t][2]);
                    S[t][3] = fmaf(k4.w, du, S[t][3]);
                    o4[0] = fmaf(S[t][0], q4.x, o4[0]);
                    o4[1] = fmaf(S[t][1], q4.y, o4[1]);
                    o4[2] = fmaf(S[t][2], q4.z, o4[2]);
                    o4[3] = fmaf(S[t][3], q4.w, o4[3]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const float o = row_group_sum((o4[0] + o4[1]) + (o4[2] + o4[3]));
                if (lrow == 0) OB[u * FPK + lcol] = o;
            }
            next_loads(ch);
            __syncthreads();
        } else {
            __builtin_amdgcn_s_setprio(2);
            // the previous chunk's epilogue, on waves 2, 3, 6, 7, which would otherwise wait in this
            // phase for the triangular solve of wave 0
            epilogue_stage(ch);
            // ---- 4. Gram blocks and T (waves 0, 1); X = V - Kbar S (all waves) -------------------
            // X = V - Kbar S0 and O1 = Qbar S0, one K step of 32 channels at a time.  S0 is the B
            // operand: K step s holds rows 32s + pi(slot), split into bf16 hi/lo right before use.
            f32x4_t X = {0.f, 0.f, 0.f, 0.f}, O1 = {0.f, 0.f, 0.f, 0.f};
            auto xo1_step = [&](int s) {
                const int ka = ln * OPK + 32 * s + 8 * lh;
                const uint4 kh = *reinterpret_cast<const uint4 *>(KLh + ka);
                const uint4 kl_ = *reinterpret_cast<const uint4 *>(KLh + PL_CD + ka);
                const float v8[8] = {S[2 * s][0], S[2 * s][1], S[2 * s][2], S[2 * s][3],
                                     S[2 * s + 1][0], S[2 * s + 1][1], S[2 * s + 1][2], S[2 * s + 1][3]};
                uint4 sh, sl;
                split8_dot(v8, sh, sl);
                X = mma3(kh, kl_, sh, sl, X);
                if (qside) {
                    const uint4 qh = *reinterpret_cast<const uint4 *>(QLh + ka);
                    const uint4 ql_ = *reinterpret_cast<const uint4 *>(QLh + PL_CD + ka);
                    O1 = mma3(qh, ql_, sh, sl, O1);
                }
            };
            // The Gram tile of wave 0 (A, transposed: Kdiv Kbar^T, so that lane (lh, ln) holds
            // row ln of A, columns 4lh .. 4lh+3) or wave 1 (P = Qbar Kdiv^T as it stands), with
            // two independent accumulation chains (channels 0-63 and 64-127) that halve the
            // dependent-MFMA latency on this critical path.
            auto gram = [&](bool tw) {
                const uint16_t *const Ap = tw ? (HEADG ? KLh : KRDh) : QLh;
                const uint16_t *const Bp = tw ? KLh : (HEADG ? KLh : KRDh);  // k^ / Gamma, or k^ for the head gate
                f32x4_t acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int s = 0; s < D / 32; ++s) {
                    const int ka = ln * OPK + 32 * s + 8 * lh;
                    const uint4 ah = *reinterpret_cast<const uint4 *>(Ap + ka);
                    const uint4 al = *reinterpret_cast<const uint4 *>(Ap + PL_CD + ka);
                    const uint4 bh = *reinterpret_cast<const uint4 *>(Bp + ka);
                    const uint4 bl = *reinterpret_cast<const uint4 *>(Bp + PL_CD + ka);
                    acc2[s >> 1] = mma3(ah, al, bh, bl, acc2[s >> 1]);
                }
                f32x4_t acc = acc2[0] + acc2[1];
                if (HEADG) {  // entry (s, j) of the Gram tile times e^{G_s - G_j} (<= 1 for j <= s)
                    const float4 g4 = *reinterpret_cast<const float4 *>(GH + 4 * lh);
                    const float g1 = GH[ln];
                    const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)  // wave 0's tile is transposed: s = ln, j = 4lh + i
                        acc[i] *= __builtin_amdgcn_exp2f(fminf(tw ? g1 - gv[i] : gv[i] - g1, 0.0f));
                }
                return acc;
            };
            if (wave == 0) {
                // the Gram block and T gate the next barrier for the whole workgroup: this wave
                // takes issue priority over the other wave of its SIMD meanwhile
                __builtin_amdgcn_s_setprio(3);
                // beta, read before the products, off the solve's chain
                const int xb = opaque(lane);
                const float bs = BETA[xb & 15];
                const float4 bc = *reinterpret_cast<const float4 *>(BETA + 4 * (xb >> 4));
                const f32x4_t acc = gram(true);
                // T = (I + A)^{-1} Diag(beta) by forward substitution in fp32.  Lane (c, r) =
                // 16c + r carries row r of X = (I + A)^{-1}, columns 4c .. 4c+3, and the whole
                // of row r of -A in registers: the lane's own four entries, A[r][4lh + i] =
                // beta_r Gram[r][4lh + i] for 4lh + i < r, gathered from the four 16-lane rows
                // of the wave with the gfx950 row swaps.  Step k then adds -A[r][k] X[k][j],
                // X[k][j] broadcast from lane k of the lane's own 16-lane row (DPP
                // row_newbcast), as one multiply-add per column: no LDS on the chain, and
                // each step depends on the previous one through one instruction.  This wave's
                // own X / O1 products, independent of the solve, sit between its quarters and
                // fill the gaps of its dependent chain.
                const int x = opaque(lane), r = x & 15, c = x >> 4;
                float na[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) na[i] = 4 * c + i < r ? -(acc[i] * bs) : 0.0f;
                float nA[C];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // permlane16_swap: rows 0, 1 get row 0 (first result) and row 1 (second),
                    // rows 2, 3 get rows 2 and 3; permlane32_swap then spreads each to all rows
                    const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(na[i]), __float_as_uint(na[i]), false, false);
                    const auto q = __builtin_amdgcn_permlane32_swap(pr[0], pr[0], false, false);
                    const auto w = __builtin_amdgcn_permlane32_swap(pr[1], pr[1], false, false);
                    nA[i] = __uint_as_float(q[0]);       // row group 0: columns 0 .. 3
                    nA[4 + i] = __uint_as_float(w[0]);   // row group 1
                    nA[8 + i] = __uint_as_float(q[1]);   // row group 2
                    nA[12 + i] = __uint_as_float(w[1]);  // row group 3
                }
                float xv[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) xv[m] = r == 4 * c + m ? 1.0f : 0.0f;
                xo1_step(0);
                forward_substitute4<0>(xv, nA);
                xo1_step(1);
                forward_substitute4<4>(xv, nA);
                xo1_step(2);
                forward_substitute4<8>(xv, nA);
                xo1_step(3);
                forward_substitute4<12>(xv, nA);
                const float tv[4] = {xv[0] * bc.x, xv[1] * bc.y, xv[2] * bc.z, xv[3] * bc.w};
                uint2 th, tl;
                split4_dot(tv, th, tl);
                // row r, columns 4c .. 4c+3: the A operand the state update reads in this lane
                *reinterpret_cast<uint2 *>(TMh + r * OPT + 4 * c) = th;
                *reinterpret_cast<uint2 *>(TMh + PL_CC + r * OPT + 4 * c) = tl;
                __builtin_amdgcn_s_setprio(2);
            } else {
                if (wave == 1 && qside) {
                    __builtin_amdgcn_s_setprio(3);
                    const f32x4_t acc = gram(false);
                    const int y = opaque(lane), j = y & 15, lg = y >> 4;
                    const int r = 4 * lg;
                    const float pv[4] = {j <= r ? acc[0] : 0.0f, j <= r + 1 ? acc[1] : 0.0f,
                                         j <= r + 2 ? acc[2] : 0.0f, j <= r + 3 ? acc[3] : 0.0f};
                    uint2 ph, pl;
                    split4_dot(pv, ph, pl);
                    store_halves(PMh + r * OPT + j, OPT, ph);
                    store_halves(PMh + PL_CC + r * OPT + j, OPT, pl);
                    __builtin_amdgcn_s_setprio(2);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) xo1_step(s);
            }
            if (HEADG) {  // the row scales Gamma of Kbar = Diag(Gamma) K^ and Qbar = Diag(Gamma) Q^
                const float4 gr = *reinterpret_cast<const float4 *>(GH + 4 * lh);
                const float e4[4] = {__builtin_amdgcn_exp2f(gr.x), __builtin_amdgcn_exp2f(gr.y),
                                     __builtin_amdgcn_exp2f(gr.z), __builtin_amdgcn_exp2f(gr.w)};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    X[i] *= e4[i];
                    O1[i] *= e4[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) X[i] = VB[(4 * lh + i) * FPK + col] - X[i];
            Split4 Xs;
            {
                const float x4[4] = {X[0], X[1], X[2], X[3]};
                split4_dot(x4, Xs.h, Xs.l);
            }
            // Head gate: S has been read, so decay it now, S <- e^{G_C} S, in the time the Gram /
            // T waves need before the barrier (they decay theirs after it).  Channel gates:
            // the state update adds Kdiv^T U first and decays after it (phase 5).
            const bool late_decay = wave == 0;
            // The next chunk's staging rewrites GH while slower waves may still be in the state
            // update below (there is no barrier between them): the head gate takes the values it
            // needs there now.
            float4 gh_r = make_float4(0.f, 0.f, 0.f, 0.f);
            float gh_last = 0.f, gh_exp = 0.f;
            if (HEADG) {
                gh_r = *reinterpret_cast<const float4 *>(GH + 4 * lh);
                gh_last = GH[C - 1];
                gh_exp = GH[C];
            }
            auto decay = [&]() {
                if (HEADG) {
                    const float g = gh_exp;  // e^{G_C}, one factor for the whole state
#pragma unroll
                    for (int t = 0; t < 8; ++t) S[t] *= g;
                    return;
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float4 g4 = *reinterpret_cast<const float4 *>(EGC + 16 * t + 4 * lh);
                    S[t][0] *= g4.x;
                    S[t][1] *= g4.y;
                    S[t][2] *= g4.z;
                    S[t][3] *= g4.w;
                }
            };
            if (HEADG && !late_decay) decay();
            __syncthreads();

            // ---- 5. U = T X, O = scale (Qbar S + P U), S <- Diag(Gamma_C) (S + Kdiv^T U) ----------
            // (Khat = e^{G_C - G} (.) K = Diag(Gamma_C) Kdiv: the exit state Diag(Gamma_C) S +
            // Khat^T U needs no plane of its own; Kdiv <= e^80 at the log-decay floor, and the
            // vote bounds it by 2^116 without a floor, so the sum stays inside fp32)
            __builtin_amdgcn_s_setprio(3);  // the chunk's last dependent chain
            {
                const int y = opaque(lane), tp = (y & 15) * OPT + 4 * (y >> 4);
                const uint2 Th = *reinterpret_cast<const uint2 *>(TMh + tp);
                const uint2 Tl = *reinterpret_cast<const uint2 *>(TMh + PL_CC + tp);
                const uint2 Ph = *reinterpret_cast<const uint2 *>(PMh + tp);
                const uint2 Pl = *reinterpret_cast<const uint2 *>(PMh + PL_CC + tp);
                const f32x4_t Uf = mma16x2(Th, Tl, Xs.h, Xs.l, f32x4_t{0.f, 0.f, 0.f, 0.f});
                const Split4 Us(Uf);
                if (qside) {
                    const f32x4_t O = mma16x2(Ph, Pl, Us.h, Us.l, O1);  // Qbar S + P U
#pragma unroll
                    for (int i = 0; i < 4; ++i) OB[(4 * lh + i) * FPK + col] = O[i];
                }
                if (HEADG && late_decay) decay();
                // Kdiv^T U (head gate: K^T (Diag(e^{G_C - G}) U)) with the products split as in
                // mma16x2.  Rows of odd tiles hold their two token pairs swapped (the plane's bank
                // swizzle), so those tiles take the U operand with its pairs swapped to match.
                Split4 Uk = Us;
                if (HEADG) {  // Khat^T U = K^T (Diag(e^{G_C - G}) U): scale the rows of U
                    const float4 gr = gh_r;
                    const float gc = gh_last;
                    const float u4[4] = {Uf[0] * __builtin_amdgcn_exp2f(gc - gr.x), Uf[1] * __builtin_amdgcn_exp2f(gc - gr.y),
                                         Uf[2] * __builtin_amdgcn_exp2f(gc - gr.z), Uf[3] * __builtin_amdgcn_exp2f(gc - gr.w)};
                    Uk = Split4(u4);
                }
                const uint4 ub_e = make_uint4(Uk.h.x, Uk.h.y, Uk.h.x, Uk.h.y), ul_e = make_uint4(Uk.l.x, Uk.l.y, 0u, 0u);
                const uint4 ub_o = make_uint4(Uk.h.y, Uk.h.x, Uk.h.y, Uk.h.x), ul_o = make_uint4(Uk.l.y, Uk.l.x, 0u, 0u);
                // (an opaque lane index for the gates whose register pressure otherwise spills
                // these addresses; the compiler keeps them in registers for the others)
                const int yk = (LOWRANK || WIDE) ? opaque(lane) : lane, ykl = yk & 15, ykh = yk >> 4;
                const uint16_t *const krow = KHTh + ykl * KHTR;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    // tokens 4lh .. 4lh+3 of row c = 16 t + ln sit at group lh ^ (t / 2)
                    const int ka = 16 * t * KHTR + 4 * (ykh ^ (t >> 1));
                    const uint2 ah = *reinterpret_cast<const uint2 *>(krow + ka);
                    const uint2 al = *reinterpret_cast<const uint2 *>(krow + C + ka);
                    const uint4 a = make_uint4(ah.x, ah.y, al.x, al.y);
                    S[t] = mma(a, (t & 1) ? ub_o : ub_e, S[t]);
                    S[t] = mma(a, (t & 1) ? ul_o : ul_e, S[t]);
                }
                if (!HEADG) decay();
            }
            __builtin_amdgcn_s_setprio(0);  // the next staging
            next_loads(ch);
        }
        // No barrier between this chunk's state update and the next chunk's staging: the
        // staging writes the K / Q / Kdiv planes (last read before the previous barrier), log
        // alpha (read when the operands were built), beta (read by the triangular solve) and,
        // for the head gate, GH (read into registers above); the state update reads T, P and
        // Kdiv^T and writes the output rows, which nothing in the staging touches.
    }
    // the last chunk's epilogue, once its output rows are written
    if (nchunks > 0) {
        __syncthreads();
        if (epi_wave && do_epi) epilogue(nchunks - 1);
    }

    // ---- final state and conv cache ------------------------------------------------------
    // a sequence's last run writes them; the segment passes leave M, or B / the state
    // entering the next segment, in the workspace
    const bool final_out = role == WHOLE || (SEG && role == RERUN && pl.last);
    float *s_dst = nullptr;
    if (final_out)
        s_dst = p.state_out ? p.state_out + (static_cast<size_t>(row_out) * H + h) * D * D : nullptr;
    else if (SEG && (role == FIRST || role == SEG_B))
        s_dst = p.seg_b + (static_cast<size_t>(pl.slot) * H + h) * D * D;
    else if (SEG && role == SEG_M)
        s_dst = p.seg_m + (static_cast<size_t>(pl.slot) * H + h) * D * D;
    if (s_dst) {
        const int x = opaque(tid);  // addresses built here, not kept live through the loop
        float *const so = s_dst + static_cast<size_t>(4 * ((x & 63) >> 4)) * D + (x >> 6) * 16 + (x & 15);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) so[(16 * t + i) * D] = S[t][i];
    }
    if (p.prologue && p.conv_out && final_out) {
        // the last three pre-conv inputs of each stream, oldest first; rows before the
        // sequence start come from conv_in (which conv_out may alias: read all, then write)
        const int task = tid;  // (stream, slot, channel group) = 3 * 3 * 16 = 144 tasks
        const bool active = task < 3 * CONV_HIST * 16;
        const int s = task / (CONV_HIST * 16), j = (task / 16) % CONV_HIST, cg = task & 15;
        const int pj = L - CONV_HIST + j;  // source position, from the start of this run
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        const void *srcs[3] = {p.q, p.k, p.v};
        if (active) {
            if (pl.ts + pj >= 0)
                IV::load(srcs[s], static_cast<size_t>(t0 + pj) * HD + hD + cg * 8, x);
            else if (p.conv_in)
                IV::load(p.conv_in, ((static_cast<size_t>(row_in) * 3 + s) * CONV_HIST + (CONV_HIST + pl.ts + pj)) * HD + hD + cg * 8, x);
        }
        __syncthreads();
        if (active)
            IV::store(p.conv_out, ((static_cast<size_t>(row_out) * 3 + s) * CONV_HIST + j) * HD + hD + cg * 8, x);
    }
}

template <typename OUT>
hipError_t launch(const LayerParams &p, hipStream_t s) {
    if (p.num_items == 0) return hipSuccess;
    // log alpha with the floor of -5 never leaves the factorised range; without a floor the
    // chunks past it are found by the vote and take the per-token path
    if (p.gate == KDA_GATE_HEAD)
        hipLaunchKernelGGL((chunked_tp_kernel<uint16_t, OUT, KDA_GATE_HEAD, false, false>), dim3(p.num_items), dim3(THREADS), 0, s, p);
    else if (p.gate == KDA_GATE_LOG_ALPHA_UNBOUNDED)
        hipLaunchKernelGGL((chunked_tp_kernel<uint16_t, OUT, KDA_GATE_LOG_ALPHA, true, false>), dim3(p.num_items), dim3(THREADS), 0, s, p);
    else
        hipLaunchKernelGGL((chunked_tp_kernel<uint16_t, OUT, KDA_GATE_LOG_ALPHA, false, false>), dim3(p.num_items), dim3(THREADS), 0, s, p);
    return hipGetLastError();
}

template <typename OUT>
hipError_t launch_lowrank(const LayerParams &p, hipStream_t s) {
    if (p.num_items == 0) return hipSuccess;
    // K3's gate stays above its floor of -5 per token, so its chunks never leave the
    // factorised range; Kimi Linear's softplus gate has no floor
    if (p.gate == KDA_GATE_LOWRANK_SOFTPLUS)
        hipLaunchKernelGGL((chunked_tp_kernel<uint16_t, OUT, KDA_GATE_LOWRANK_SOFTPLUS, true, false>), dim3(p.num_items),
                           dim3(THREADS), 0, s, p);
    else
        hipLaunchKernelGGL((chunked_tp_kernel<uint16_t, OUT, KDA_GATE_LOWRANK, false, false>), dim3(p.num_items), dim3(THREADS),
                           0, s, p);
    return hipGetLastError();
}

template <typename OUT>
hipError_t launch_segments(const LayerParams &p, int grid, hipStream_t s) {
    if (p.gate == KDA_GATE_HEAD)
        hipLaunchKernelGGL((chunked_tp_kernel<uint16_t, OUT, KDA_GATE_HEAD, false, true>), dim3(grid), dim3(THREADS), 0, s, p);
    else if (p.gate == KDA_GATE_LOWRANK)
        hipLaunchKernelGGL((chunked_tp_kernel<uint16_t, OUT, KDA_GATE_LOWRANK, false, true>), dim3(grid), dim3(THREADS), 0, s, p);
    else
        hipLaunchKernelGGL((chunked_tp_kernel<uint16_t, OUT, KDA_GATE_LOG_ALPHA, false, true>), dim3(grid), dim3(THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace

// bf16 io and the floored gates only (checked by the caller)
hipError_t launch_chunked_segments(const LayerParams &p, int out_dtype, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    return out_dtype == KDA_DTYPE_BF16 ? launch_segments<uint16_t>(p, grid, s) : launch_segments<float>(p, grid, s);
}

// bf16 io only (checked by the caller)
hipError_t launch_chunked_throughput(const LayerParams &p, int out_dtype, hipStream_t s) {
    if (p.gate == KDA_GATE_LOWRANK || p.gate == KDA_GATE_LOWRANK_SOFTPLUS)
        return out_dtype == KDA_DTYPE_BF16 ? launch_lowrank<uint16_t>(p, s) : launch_lowrank<float>(p, s);
    return out_dtype == KDA_DTYPE_BF16 ? launch<uint16_t>(p, s) : launch<float>(p, s);
}

}  // namespace kda
