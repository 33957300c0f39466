// kda_recurrent.hip -- token-sequential KDA recurrence in fp32 (gfx950).
//
// One workgroup of 256 lanes owns one (sequence, head) pair and walks its
// tokens in order, holding the 128x128 fp32 state in registers: lane t keeps
// rows 16*(t/32) .. +15 and columns 4*(t%32) .. +3 (64 floats).  Per token:
//
//   prologue  conv4 + SiLU on q, k, v (lanes 0-127: q and k of channel t;
//             lanes 128-255: v of channel t-128), L2 norms of q and k by wave
//             reductions ("Kimi K3 - KDA layer" (OpenModelAtlas), conv/SiLU/L2
//             steps; "Inside Kimi K3", short-convolution section)
//   decay     S <- Diag(alpha) S, alpha per row = key channel; alpha is given as
//             log alpha (per channel, or one value per head), or formed from the
//             low-rank gate factors, alpha = exp(-5 sigmoid(e^{A_h} (z_down W_up^T
//             + b))) ("Kimi K3 - KDA layer")
//   predict   r = S^T k^  and  p = S^T q^ on the decayed state, in one pass
//   write     S <- S + beta k^ (v - r)^T
//   read      o~ = scale * S_new^T q^ = scale * (p + (q^.k^) beta (v - r))
//   epilogue  sigmoid(g) * o~ / sqrt(mean o~^2 + eps) * w  over 128 channels
//
// The read uses the identity S_new^T q = (Diag(alpha)S)^T q + (q.k) beta (v-r),
// which is exactly the post-write read of the step list ("Kimi K3 - KDA
// layer": S <- Diag(alpha)S; S <- S + beta k(v - S^T k)^T; o~ = S^T q/sqrt(128))
// with both column reductions taken in one pass over S.
//
// This kernel is the fp32 prefill path (the reference-precision path for fp32
// inputs) and, at one token per request, the decode step: S is streamed from
// HBM once, updated, and written back once, which is what bounds decode.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int THREADS = 256;
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int W>
__device__ __forceinline__ float group_sum(float x) {
    // butterfly over aligned groups of W lanes (W divides 64)
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// log alpha of key channel c of head h at token t from the low-rank gate factors: an
// fp32 dot product over the rank, then -5 sigmoid(e^{A_h} (z + b)), or for Kimi Linear's
// gate -e^{A_h} softplus(z + b) = -e^{A_h} (max(u, 0) + log(1 + e^{-|u|})).
template <typename IO>
__device__ __forceinline__ float lowrank_log_alpha(const LayerParams &p, int64_t t, int h, int c, float e_a) {
    using IOT = IoTraits<IO>;
    const int r = p.gate_rank;
    const size_t zrow = static_cast<size_t>(t) * r;
    const size_t wrow = (static_cast<size_t>(h) * D + c) * r;
    float acc0 = 0.f, acc1 = 0.f;
    for (int j = 0; j < r; j += 2) {
        acc0 = fmaf(IOT::load(p.gate_z, zrow + j), IOT::load(p.gate_w, wrow + j), acc0);
        acc1 = fmaf(IOT::load(p.gate_z, zrow + j + 1), IOT::load(p.gate_w, wrow + j + 1), acc1);
    }
    const float u = (acc0 + acc1) + p.gate_bias[static_cast<size_t>(h) * D + c];
    if (p.gate == KDA_GATE_LOWRANK_SOFTPLUS) return -e_a * (fmaxf(u, 0.0f) + log1pf(__expf(-fabsf(u))));
    return -5.0f * sigmoidf_(e_a * u);
}

template <typename IO, typename OUT>
__global__ __launch_bounds__(THREADS) void recurrent_kernel(LayerParams p) {
    using IOT = IoTraits<IO>;
    using OT = IoTraits<OUT>;
    const int H = p.H;
    const int item = blockIdx.x;
    const int h = item % H;
    const int idx = item / H;

    int64_t t0, t1;
    int n;  // sequence (prefill) or request (decode)
    if (p.cu_seqlens) {
        n = p.order ? p.order[idx] : idx;
        t0 = p.cu_seqlens[n];
        t1 = p.cu_seqlens[n + 1];
    } else {
        n = idx;
        t0 = idx;
        t1 = idx + 1;
    }
    const int row_in = p.slots_in ? p.slots_in[n] : n;     // state_in / conv_in row
    const int row_out = p.slots_out ? p.slots_out[n] : n;  // state_out / conv_out row

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = tid & 31;    // column group: columns j0 .. j0+3
    const int rg = tid >> 5;    // row group: rows i0 .. i0+15
    const int j0 = cg * 4;
    const int i0 = rg * 16;
    const int c = tid & 127;    // prologue channel
    const bool qk_lane = tid < 128;

    __shared__ float sh_q[2][D], sh_k[2][D], sh_v[2][D], sh_g[2][D], sh_a[2][D];
    __shared__ float sh_red[2][4][2][D];
    __shared__ float sh_norm[2][2][3];
    __shared__ float sh_beta[2];

    // ---- state in registers -------------------------------------------------
    const size_t sbase = (static_cast<size_t>(row_in) * H + h) * D * D;
    float S[16][4];
    if (p.state_in) {
        const float4 *src = reinterpret_cast<const float4 *>(p.state_in + sbase);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // the state is streamed: read once, written once, no reuse through the caches
            const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(&src[((i0 + r) * D + j0) / 4]));
            S[r][0] = x[0]; S[r][1] = x[1]; S[r][2] = x[2]; S[r][3] = x[3];
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[r][jj] = 0.0f;
    }

    // ---- conv weights and history for this lane's channel ---------------------
    const size_t HD = static_cast<size_t>(H) * D;
    const int sA = qk_lane ? 0 : 2;  // stream of the first value this lane convolves
    float wA[4] = {1.f, 0.f, 0.f, 0.f}, wB[4] = {1.f, 0.f, 0.f, 0.f};
    float hA[CONV_HIST] = {0.f, 0.f, 0.f}, hB[CONV_HIST] = {0.f, 0.f, 0.f};
    if (p.prologue) {
        const float *wa = p.conv_w + (sA * HD + static_cast<size_t>(h) * D + c) * 4;
        const float *wb = p.conv_w + (1 * HD + static_cast<size_t>(h) * D + c) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wA[j] = wa[j];
            wB[j] = qk_lane ? wb[j] : 0.f;
        }
        if (p.conv_in) {
            const size_t base = static_cast<size_t>(row_in) * 3 * CONV_HIST * HD + h * D + c;
#pragma unroll
            for (int j = 0; j < CONV_HIST; ++j) {
                hA[j] = IOT::load(p.conv_in, base + (sA * CONV_HIST + j) * HD);
                hB[j] = qk_lane ? IOT::load(p.conv_in, base + (1 * CONV_HIST + j) * HD) : 0.f;
            }
        }
    }
    float wr[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wr[jj] = p.rms_w ? p.rms_w[j0 + jj] : 1.0f;

    const float e_a = p.gate_z ? __expf(p.gate_a[h]) : 0.0f;
    for (int64_t t = t0; t < t1; ++t) {
        const int buf = static_cast<int>((t - t0) & 1);
        const size_t row = (static_cast<size_t>(t) * H + h) * D;

        // ---- stage A: prologue ----------------------------------------------
        float xa = 0.f, xb = 0.f;
        if (qk_lane) {
            float rq = IOT::load(p.q, row + c);
            float rk = IOT::load(p.k, row + c);
            if (p.prologue) {
                float yq = wA[0] * rq + wA[1] * hA[2] + wA[2] * hA[1] + wA[3] * hA[0];
                float yk = wB[0] * rk + wB[1] * hB[2] + wB[2] * hB[1] + wB[3] * hB[0];
                hA[0] = hA[1]; hA[1] = hA[2]; hA[2] = rq;
                hB[0] = hB[1]; hB[1] = hB[2]; hB[2] = rk;
                xa = siluf_(yq);
                xb = siluf_(yk);
            } else {
                xa = rq;
                xb = rk;
            }
            float ssq = group_sum<64>(xa * xa);
            float ssk = group_sum<64>(xb * xb);
            float sqk = group_sum<64>(xa * xb);
            if (lane == 0) {
                sh_norm[buf][wave][0] = ssq;
                sh_norm[buf][wave][1] = ssk;
                sh_norm[buf][wave][2] = sqk;
            }
        } else {
            float rv = IOT::load(p.v, row + c);
            float xv = rv;
            if (p.prologue) {
                float yv = wA[0] * rv + wA[1] * hA[2] + wA[2] * hA[1] + wA[3] * hA[0];
                hA[0] = hA[1]; hA[1] = hA[2]; hA[2] = rv;
                xv = siluf_(yv);
            }
            sh_v[buf][c] = xv;
            if (p.epilogue) sh_g[buf][c] = sigmoidf_(IOT::load(p.g, row + c));
            const float la = p.gate_z ? lowrank_log_alpha<IO>(p, t, h, c, e_a)
                             : p.gate == KDA_GATE_HEAD ? p.log_alpha[static_cast<size_t>(t) * H + h]
                                                       : p.log_alpha[row + c];
            sh_a[buf][c] = __expf(la);
            if (c == 0) {
                const float b = p.beta[static_cast<size_t>(t) * H + h];
                sh_beta[buf] = p.beta_logit ? sigmoidf_(b) : b;  // beta = sigmoid(w) from its pre-activation
            }
        }
        __syncthreads();
        const float tq = sh_norm[buf][0][0] + sh_norm[buf][1][0];
        const float tk = sh_norm[buf][0][1] + sh_norm[buf][1][1];
        const float tqk = sh_norm[buf][0][2] + sh_norm[buf][1][2];
        const float invq = p.prologue ? rsqrtf(tq + p.l2_eps) : 1.0f;
        const float invk = p.prologue ? rsqrtf(tk + p.l2_eps) : 1.0f;
        if (qk_lane) {
            sh_q[buf][c] = xa * invq;
            sh_k[buf][c] = xb * invk;
        }
        const float qkdot = tqk * invq * invk;
        __syncthreads();

        // ---- stage B: decay, predict and partial read ----------------------------
        float r[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float a = sh_a[buf][i0 + rr];
            const float kk = sh_k[buf][i0 + rr];
            const float qq = sh_q[buf][i0 + rr];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float s = S[rr][jj] * a;
                S[rr][jj] = s;
                r[jj] = fmaf(kk, s, r[jj]);
                pq[jj] = fmaf(qq, s, pq[jj]);
            }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            r[jj] += __shfl_xor(r[jj], 32, 64);
            pq[jj] += __shfl_xor(pq[jj], 32, 64);
        }
        if ((tid & 32) == 0) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                sh_red[buf][wave][0][j0 + jj] = r[jj];
                sh_red[buf][wave][1][j0 + jj] = pq[jj];
            }
        }
        __syncthreads();

        // ---- write and read ---------------------------------------------------
        const float beta = sh_beta[buf];
        float e[4], ot[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = j0 + jj;
            const float rs = (sh_red[buf][0][0][j] + sh_red[buf][1][0][j]) +
                             (sh_red[buf][2][0][j] + sh_red[buf][3][0][j]);
            const float ps = (sh_red[buf][0][1][j] + sh_red[buf][1][1][j]) +
                             (sh_red[buf][2][1][j] + sh_red[buf][3][1][j]);
            e[jj] = beta * (sh_v[buf][j] - rs);
            ot[jj] = p.scale * fmaf(qkdot, e[jj], ps);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float kk = sh_k[buf][i0 + rr];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[rr][jj] = fmaf(kk, e[jj], S[rr][jj]);
        }

        // ---- epilogue (row group 0 stores) -----------------------------------------
        if (rg == 0) {
            float outv[4];
            if (p.epilogue) {
                float ss = ot[0] * ot[0] + ot[1] * ot[1] + ot[2] * ot[2] + ot[3] * ot[3];
                ss = group_sum<32>(ss);
                const float inv = rsqrtf(ss * (1.0f / D) + p.rms_eps);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    outv[jj] = sh_g[buf][j0 + jj] * (ot[jj] * inv) * wr[jj];
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) outv[jj] = ot[jj];
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) OT::store(p.o, row + j0 + jj, outv[jj]);
        }
    }

    // ---- final state and conv cache ----------------------------------------------
    if (p.state_out) {
        float4 *dst = reinterpret_cast<float4 *>(p.state_out + (static_cast<size_t>(row_out) * H + h) * D * D);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const f32x4v y = {S[r][0], S[r][1], S[r][2], S[r][3]};
            __builtin_nontemporal_store(y, reinterpret_cast<f32x4v *>(&dst[((i0 + r) * D + j0) / 4]));
        }
    }
    if (p.prologue && p.conv_out) {
        const size_t base = static_cast<size_t>(row_out) * 3 * CONV_HIST * HD + h * D + c;
#pragma unroll
        for (int j = 0; j < CONV_HIST; ++j) {
            IOT::store(p.conv_out, base + (sA * CONV_HIST + j) * HD, hA[j]);
            if (qk_lane) IOT::store(p.conv_out, base + (1 * CONV_HIST + j) * HD, hB[j]);
        }
    }
}

template <typename IO, typename OUT>
hipError_t launch(const LayerParams &p, hipStream_t s) {
    if (p.num_items == 0) return hipSuccess;
    hipLaunchKernelGGL((recurrent_kernel<IO, OUT>), dim3(p.num_items), dim3(THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_recurrent(const LayerParams &p, int io_dtype, int out_dtype, hipStream_t s) {
    if (io_dtype == KDA_DTYPE_BF16)
        return out_dtype == KDA_DTYPE_BF16 ? launch<uint16_t, uint16_t>(p, s)
                                           : launch<uint16_t, float>(p, s);
    return out_dtype == KDA_DTYPE_BF16 ? launch<float, uint16_t>(p, s) : launch<float, float>(p, s);
}

}  // namespace kda
