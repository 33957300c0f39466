// kda_chunk_common.h -- operand helpers of the chunked prefill kernel
// (kda_chunked.hip): chunk geometry, bf16 hi/lo
// operand splits, the gfx950 MFMA wrappers, the K-slot permutation that lets
// accumulator tiles serve as B operands, and range-checked buffer views.
#pragma once

#include "kda_internal.h"

namespace kda {
namespace chunk {

constexpr int C = 16;          // tokens per chunk
// Padded row (bf16 elements) of the [16][128] operand planes: 288 bytes.  The MFMA
// operand reads (lane: row l % 16, 16 bytes at column 8 (l / 16) of a 32-column step)
// measured free of LDS bank conflicts with this stride on gfx950 and with no other
// stride tried (272, 304 and 320 bytes, or XOR swizzles of the 16-byte groups); 272
// bytes (the 16-byte minimum padding) cost a stall on most of these reads.
constexpr int OPK = D + 16;
constexpr int OPT = C + 4;     // padded row of [*][16] operand planes
constexpr int FPK = D + 4;     // padded row (floats) of [16][128] fp32 tiles

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int PL_CD = C * OPK;           // bf16 elements of one [16][128] plane
constexpr int PL_DC = D * OPT;           // one [128][16] plane
constexpr int PL_CC = C * OPT;           // one [16][16] plane

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

// The same splits with the residuals x - hi taken from the bf16 dot product
// x + (hi_a, hi_b) . (-1, 0) (and (0, -1)), which is exact (x - hi has at most 16
// significant bits) and one instruction per element instead of three.  The compiler emits
// only the accumulator-tied form of that instruction, so the dot products alone are written
// out, in groups of four pairs; the conversions before and after them stay the compiler's,
// which therefore keeps the waits it owes the producers of x (a matrix-core result, say) and
// the consumers of the hi and lo parts.  The one wait it cannot see, a dot product's result
// read by another vector instruction, is the trailing s_nop: three wait states after the
// last dot product, and more after the earlier ones.
__device__ __forceinline__ void dot_residuals4(const uint32_t *h, const float *x, float *r) {
    const uint32_t na = 0x0000bf80u, nb = 0xbf800000u;  // bf16 pairs (-1, 0) and (0, -1)
    asm volatile(
        "v_dot2_f32_bf16 %0, %8, %12, %14\n\t"
        "v_dot2_f32_bf16 %1, %8, %13, %15\n\t"
        "v_dot2_f32_bf16 %2, %9, %12, %16\n\t"
        "v_dot2_f32_bf16 %3, %9, %13, %17\n\t"
        "v_dot2_f32_bf16 %4, %10, %12, %18\n\t"
        "v_dot2_f32_bf16 %5, %10, %13, %19\n\t"
        "v_dot2_f32_bf16 %6, %11, %12, %20\n\t"
        "v_dot2_f32_bf16 %7, %11, %13, %21\n\t"
        "s_nop 2"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "s"(na), "s"(nb),
          "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ void split8_dot(const float *x, uint4 &hi, uint4 &lo) {
    const uint32_t h[4] = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
    float r[8];
    dot_residuals4(h, x, r);
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3]), pack_bf16(r[4], r[5]), pack_bf16(r[6], r[7]));
}

__device__ __forceinline__ void split4_dot(const float *x, uint2 &hi, uint2 &lo) {
    const uint32_t na = 0x0000bf80u, nb = 0xbf800000u;
    const uint32_t h0 = pack_bf16(x[0], x[1]), h1 = pack_bf16(x[2], x[3]);
    float r0, r1, r2, r3;
    asm volatile(
        "v_dot2_f32_bf16 %0, %4, %6, %8\n\t"
        "v_dot2_f32_bf16 %1, %4, %7, %9\n\t"
        "v_dot2_f32_bf16 %2, %5, %6, %10\n\t"
        "v_dot2_f32_bf16 %3, %5, %7, %11\n\t"
        "s_nop 2"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(h0), "v"(h1), "s"(na), "s"(nb), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
    hi = make_uint2(h0, h1);
    lo = make_uint2(pack_bf16(r0, r1), pack_bf16(r2, r3));
}

// The four bf16 values of a pair of packed words written to p[0], p[stride], p[2 stride]
// and p[3 stride] (a column or row of a 16-bit plane).
__device__ __forceinline__ void store_halves(uint16_t *p, int stride, uint2 w) {
    p[0] = static_cast<uint16_t>(w.x);
    p[stride] = static_cast<uint16_t>(w.x >> 16);
    p[2 * stride] = static_cast<uint16_t>(w.y);
    p[3 * stride] = static_cast<uint16_t>(w.y >> 16);
}

// Two groups of four floats split with one block of dot products.
__device__ __forceinline__ void split4x2_dot(const float *x, const float *y, uint2 &xh, uint2 &xl, uint2 &yh, uint2 &yl) {
    const float v[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    uint4 h, l;
    split8_dot(v, h, l);
    xh = make_uint2(h.x, h.y);
    yh = make_uint2(h.z, h.w);
    xl = make_uint2(l.x, l.y);
    yl = make_uint2(l.z, l.w);
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

__device__ __forceinline__ void split4(const float *x, uint2 &hi, uint2 &lo) {
    split2(x[0], x[1], hi.x, lo.x);
    split2(x[2], x[3], hi.y, lo.y);
}

__device__ __forceinline__ f32x4_t mma16(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                     __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}

// (a_hi + a_lo)(b_hi + b_lo) without the lo*lo term, K = 16.
__device__ __forceinline__ f32x4_t mma16_3(uint2 ahi, uint2 alo, uint2 bhi, uint2 blo, f32x4_t c) {
    c = mma16(alo, bhi, c);
    c = mma16(ahi, blo, c);
    return mma16(ahi, bhi, c);
}

// A 16x16 fp32 matrix fragment (4 values per lane) split into bf16 hi/lo.
struct Split4 {
    uint2 h, l;
    Split4() = default;
    __device__ __forceinline__ explicit Split4(const float *x) { split4_dot(x, h, l); }
    __device__ __forceinline__ explicit Split4(const f32x4_t &x) {
        const float v[4] = {x[0], x[1], x[2], x[3]};
        split4_dot(v, h, l);
    }
};

// x y for 16x16 matrices held as (a form of x, b form of y), on a fresh accumulator.
__device__ __forceinline__ f32x4_t mm16s(const Split4 &xa, const Split4 &yb) {
    return mma16_3(xa.h, xa.l, yb.h, yb.l, f32x4_t{0.f, 0.f, 0.f, 0.f});
}
__device__ __forceinline__ void mm16s(const Split4 &xa, const Split4 &yb, float *d) {
    const f32x4_t r = mm16s(xa, yb);
    d[0] = r[0]; d[1] = r[1]; d[2] = r[2]; d[3] = r[3];
}

__device__ __forceinline__ f32x4_t mma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// (a_hi + a_lo)(b_hi + b_lo) without the lo*lo term for a K = 16 contraction held in
// K = 16 operand layouts (lane group g: K indices 4g .. 4g+3), as two K = 32 MFMAs (the
// same issue cost as one K = 16 MFMA on gfx950).  Slots 0-3 of a lane carry the hi parts
// of its four K indices and slots 4-7 the lo parts: (a_hi, a_lo) against (b_hi, b_hi),
// then against (b_lo, 0).  Accumulating a K = 16 MFMA onto a K = 32 result read stale
// accumulator rows on gfx950 (observed, not documented), so the kernels never mix the
// two shapes on one accumulator.
__device__ __forceinline__ f32x4_t mma16x2(uint2 ahi, uint2 alo, uint2 bhi, uint2 blo, f32x4_t c) {
    const uint4 a = make_uint4(ahi.x, ahi.y, alo.x, alo.y);
    c = mma(a, make_uint4(bhi.x, bhi.y, bhi.x, bhi.y), c);
    return mma(a, make_uint4(blo.x, blo.y, 0u, 0u), c);
}

// (a_hi + a_lo)(b_hi + b_lo) without the lo*lo term.
__device__ __forceinline__ f32x4_t mma3(uint4 ahi, uint4 alo, uint4 bhi, uint4 blo, f32x4_t c) {
    c = mma(alo, bhi, c);
    c = mma(ahi, blo, c);
    return mma(ahi, bhi, c);
}

// Forward substitution for one 16 x 16 unit lower-triangular system, four columns per lane:
// lane (c, r) = 16c + r holds x[m] = X[r][4c + m] and nA[k] = -A[r][k] (zero for k >= r);
// step k adds nA[k] X[k][4c + m], X[k][.] broadcast from lane k of the lane's 16-lane row
// (DPP row_newbcast, gfx90a and later) inside the multiply-add itself.  Written out because
// the compiler does not fold the broadcast into the accumulating multiply-add.  A DPP read of
// a register written by a vector instruction needs two wait states: the leading s_nop covers
// the inputs, and inside the block each column's register is written three instructions
// before the next step reads it.  The products and sums are the fused ones of fmaf.
__device__ __forceinline__ void forward_substitute16(float *x, const float *nA) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])
        : "v"(nA[0]), "v"(nA[1]), "v"(nA[2]), "v"(nA[3]), "v"(nA[4]), "v"(nA[5]), "v"(nA[6]), "v"(nA[7]),
          "v"(nA[8]), "v"(nA[9]), "v"(nA[10]), "v"(nA[11]), "v"(nA[12]), "v"(nA[13]), "v"(nA[14]), "v"(nA[15]));
}

// Steps k0 .. k0+3 of the same substitution (four calls, k0 = 0, 4, 8, 12, make the whole), so
// that independent work can be placed between them; each part starts with the two wait
// states its first DPP read needs after whatever vector instruction wrote x last.
#define KDA_FS4_BODY(K0, K1, K2, K3)                                                          \
    asm volatile(                                                                             \
        "s_nop 1\n\t"                                                                         \
        "v_fmac_f32_dpp %0, %0, %4 row_newbcast:" #K0 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %1, %1, %4 row_newbcast:" #K0 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %2, %2, %4 row_newbcast:" #K0 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %3, %3, %4 row_newbcast:" #K0 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %0, %0, %5 row_newbcast:" #K1 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %1, %1, %5 row_newbcast:" #K1 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %2, %2, %5 row_newbcast:" #K1 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %3, %3, %5 row_newbcast:" #K1 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %0, %0, %6 row_newbcast:" #K2 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %1, %1, %6 row_newbcast:" #K2 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %2, %2, %6 row_newbcast:" #K2 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %3, %3, %6 row_newbcast:" #K2 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %0, %0, %7 row_newbcast:" #K3 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %1, %1, %7 row_newbcast:" #K3 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %2, %2, %7 row_newbcast:" #K3 " row_mask:0xf bank_mask:0xf\n\t"       \
        "v_fmac_f32_dpp %3, %3, %7 row_newbcast:" #K3 " row_mask:0xf bank_mask:0xf\n\t"       \
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])                                      \
        : "v"(nA[K0]), "v"(nA[K1]), "v"(nA[K2]), "v"(nA[K3]))
template <int K0>
__device__ __forceinline__ void forward_substitute4(float *x, const float *nA);
template <>
__device__ __forceinline__ void forward_substitute4<0>(float *x, const float *nA) { KDA_FS4_BODY(0, 1, 2, 3); }
template <>
__device__ __forceinline__ void forward_substitute4<4>(float *x, const float *nA) { KDA_FS4_BODY(4, 5, 6, 7); }
template <>
__device__ __forceinline__ void forward_substitute4<8>(float *x, const float *nA) { KDA_FS4_BODY(8, 9, 10, 11); }
template <>
__device__ __forceinline__ void forward_substitute4<12>(float *x, const float *nA) { KDA_FS4_BODY(12, 13, 14, 15); }
#undef KDA_FS4_BODY

// A copy of x that the compiler cannot see through: values derived from it are
// recomputed where they are used instead of being hoisted out of a loop and kept
// live (or spilled) across it.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Sum over each half wave (lanes 0-31 and 32-63 separately), returned to every lane of
// the half: two quad permutes, the half-row and row mirrors (DPP operands of the adds)
// and one ds_swizzle that exchanges the two 16-lane rows of the half.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float half_wave_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]: lane ^ 1
    x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]: lane ^ 2
    x += dpp<0x141>(x);  // row_half_mirror: quad sums of the two halves of each 8 lanes
    x += dpp<0x140>(x);  // row_mirror: the two 8-lane halves of each 16-lane row
    // bit-mask swizzle inside 32 lanes: and 0x1f, or 0, xor 0x10
    x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
    return x;
}

// Sum over the four 16-lane rows of the wave (lanes l, l ^ 16, l ^ 32, l ^ 48), with the
// gfx950 row swaps: permlane16_swap exchanges rows 1 <-> 0 and 3 <-> 2 between its two
// operands, permlane32_swap the upper half of one with the lower half of the other, so
// that the two results of each add up to the xor-16 and then the xor-32 butterfly.
__device__ __forceinline__ float row_group_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Eight consecutive io values starting at element i (i a multiple of 8): a raw
// 16- or 32-byte load, and its conversion to fp32, kept apart so that a batch
// of loads can be issued before any of them is consumed.
template <typename IO> struct Vec8;
template <> struct Vec8<uint16_t> {
    struct Raw { uint4 u; };
    static __device__ __forceinline__ Raw raw(const void *p, size_t i) {
        return Raw{*reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + i)};
    }
    static __device__ __forceinline__ void unpack(const Raw &r, float *x) {
        const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void load(const void *p, size_t i, float *x) { unpack(raw(p, i), x); }
    static __device__ __forceinline__ uint4 pack(const float *x) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x[2 * e], x[2 * e + 1]}, bf16x2_t));
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
    static __device__ __forceinline__ void store(void *p, size_t i, const float *x) {
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p) + i) = pack(x);
    }
};
template <> struct Vec8<float> {
    struct Raw { float4 a, b; };
    static __device__ __forceinline__ Raw raw(const void *p, size_t i) {
        const float4 *q = reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
        return Raw{q[0], q[1]};
    }
    static __device__ __forceinline__ void unpack(const Raw &r, float *x) {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
        x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
    }
    static __device__ __forceinline__ void load(const void *p, size_t i, float *x) { unpack(raw(p, i), x); }
    static __device__ __forceinline__ void store(void *p, size_t i, const float *x) {
        float4 *q = reinterpret_cast<float4 *>(static_cast<float *>(p) + i);
        q[0] = make_float4(x[0], x[1], x[2], x[3]);
        q[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
};

// Storage column of key channel c in a channel-permuted [*][128] plane.
__device__ __forceinline__ int cperm(int c) { return (c & ~31) | kperm(c & 31); }

// Column swizzle of the Khat^T planes: row c keeps its 4-token groups
// contiguous (8-byte MFMA operand reads) but XORs the group index with
// (c / 8) % 4, spreading the transposed stores of 16 lanes (rows 8 apart)
// over four bank groups.
__device__ __forceinline__ int kht_col(int c, int j) { return j ^ (((c >> 3) & 3) << 2); }

// Range-checked buffer view of n_rows rows of one head, starting at byte address
// `base`, rows `row_bytes` apart, each `len_bytes` long: loads past the view (or
// before it, through a negative offset that wraps) return zeros and stores past
// it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_view(const char *base, int n_rows, uint32_t row_bytes,
                                                             uint32_t len_bytes) {
    const int bytes = n_rows > 0 ? static_cast<int>((n_rows - 1) * row_bytes + len_bytes) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), static_cast<short>(0), bytes, 0x00020000);
}

template <typename IO> struct BufLoad8;
template <> struct BufLoad8<uint16_t> {
    using Raw = typename Vec8<uint16_t>::Raw;
    static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
        u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
        return Raw{make_uint4(v[0], v[1], v[2], v[3])};
    }
};
template <> struct BufLoad8<float> {
    using Raw = typename Vec8<float>::Raw;
    static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
        u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
        u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off + 16, 0, 0);
        return Raw{make_float4(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3])),
                   make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3]))};
    }
};

template <typename OUT> struct OutStore;
template <> struct OutStore<uint16_t> {
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float *x) {
        const uint4 w = Vec8<uint16_t>::pack(x);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{w.x, w.y, w.z, w.w}, r, off, 0, 0);
    }
};
template <> struct OutStore<float> {
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float *x) {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])}, r, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])}, r, off + 16, 0, 0);
    }
};


// Four consecutive io values starting at element i (i a multiple of 4), raw and
// converted; the 4-wide counterparts of Vec8 / BufLoad8 / OutStore.
template <typename IO> struct Vec4;
template <> struct Vec4<uint16_t> {
    struct Raw { uint2 u; };
    static __device__ __forceinline__ Raw raw(const void *p, size_t i) {
        return Raw{*reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i)};
    }
    static __device__ __forceinline__ void unpack(const Raw &r, float *x) {
        x[0] = __uint_as_float(r.u.x << 16);
        x[1] = __uint_as_float(r.u.x & 0xffff0000u);
        x[2] = __uint_as_float(r.u.y << 16);
        x[3] = __uint_as_float(r.u.y & 0xffff0000u);
    }
    static __device__ __forceinline__ uint2 pack(const float *x) {
        return make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x[0], x[1]}, bf16x2_t)),
                          __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x[2], x[3]}, bf16x2_t)));
    }
};
template <> struct Vec4<float> {
    struct Raw { float4 a; };
    static __device__ __forceinline__ Raw raw(const void *p, size_t i) {
        return Raw{*reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i)};
    }
    static __device__ __forceinline__ void unpack(const Raw &r, float *x) {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    }
};
__device__ __forceinline__ void load4f(const float *p, float *x) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void store4f(float *p, const float *x) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

template <typename IO> struct BufLoad4;
template <> struct BufLoad4<uint16_t> {
    using Raw = typename Vec4<uint16_t>::Raw;
    static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
        return Raw{make_uint2(v[0], v[1])};
    }
};
template <> struct BufLoad4<float> {
    using Raw = typename Vec4<float>::Raw;
    static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
        return Raw{make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]))};
    }
};

template <typename OUT> struct OutStore4;
template <> struct OutStore4<uint16_t> {
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float *x) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const uint2 w = Vec4<uint16_t>::pack(x);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{w.x, w.y}, r, off, 0, 0);
    }
};
template <> struct OutStore4<float> {
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float *x) {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])}, r, off, 0, 0);
    }
};

}  // namespace chunk
}  // namespace kda
