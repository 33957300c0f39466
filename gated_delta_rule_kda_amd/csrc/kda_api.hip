// kda_api.hip -- the C ABI of libkda.so: host-side validation, workspace
// sizing and dispatch to the gfx950 kernels.  Nothing here synchronises with
// the device; a call only enqueues work on the caller's stream.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

// Sequences are ranked longest first so that, in a packed batch of very
// different lengths, the workgroups with the longest sequential scans start
// first.  The rank of sequence i is the number of sequences that are longer,
// or equally long with a smaller index; order[rank] = i.  One launch of
// ceil(N/256) workgroups, each staging all N lengths in LDS.
constexpr int ORDER_MAX_SEQS = 8192;  // beyond this the natural order is used

__global__ __launch_bounds__(256) void order_kernel(const int32_t *cu, int32_t n, int32_t *order) {
    __shared__ int32_t len[ORDER_MAX_SEQS];
    for (int i = threadIdx.x; i < n; i += blockDim.x) len[i] = cu[i + 1] - cu[i];
    __syncthreads();
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int32_t li = len[i];
    int32_t rank = 0;
    for (int j = 0; j < n; ++j) {
        const int32_t lj = len[j];
        rank += (lj > li) || (lj == li && j < i);
    }
    order[rank] = i;
}

bool valid_algo(int32_t a) { return a >= KDA_ALGO_AUTO && a <= KDA_ALGO_CHUNKED_SCAN; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool trace_enabled() {
    static const bool on = [] {
        const char *e = getenv("KDA_TRACE");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

// the gates formed in the kernels from z_down, W_up, b and A
bool lowrank_gate(const kda_config *cfg) {
    return cfg->gate == KDA_GATE_LOWRANK || cfg->gate == KDA_GATE_LOWRANK_SOFTPLUS;
}

kda_status check_config(const kda_config *cfg) {
    if (!cfg) return KDA_ERR_INVALID_ARGUMENT;
    if (cfg->head_dim != D) return KDA_ERR_UNSUPPORTED;
    if (cfg->num_heads <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (cfg->io_dtype != KDA_DTYPE_F32 && cfg->io_dtype != KDA_DTYPE_BF16) return KDA_ERR_INVALID_ARGUMENT;
    if (cfg->out_dtype != KDA_DTYPE_F32 && cfg->out_dtype != KDA_DTYPE_BF16) return KDA_ERR_INVALID_ARGUMENT;
    if ((cfg->prologue != 0 && cfg->prologue != 1) || (cfg->epilogue != 0 && cfg->epilogue != 1))
        return KDA_ERR_INVALID_ARGUMENT;
    if (!valid_algo(cfg->algo)) return KDA_ERR_INVALID_ARGUMENT;
    if (cfg->gate < KDA_GATE_LOG_ALPHA || cfg->gate > KDA_GATE_LOG_ALPHA_UNBOUNDED) return KDA_ERR_INVALID_ARGUMENT;
    if (lowrank_gate(cfg) && (cfg->gate_rank < 32 || cfg->gate_rank > 128 || cfg->gate_rank % 32 != 0))
        return KDA_ERR_UNSUPPORTED;
    if (cfg->beta_mode != KDA_BETA_VALUE && cfg->beta_mode != KDA_BETA_LOGIT) return KDA_ERR_INVALID_ARGUMENT;
    if (!isfinite(cfg->scale) || !(cfg->l2_eps >= 0.f) || !(cfg->rms_eps >= 0.f) ||
        !isfinite(cfg->l2_eps) || !isfinite(cfg->rms_eps))
        return KDA_ERR_INVALID_ARGUMENT;
    return KDA_OK;
}

// A required pointer must be non-null; every given pointer must be 16-byte aligned.
bool ok_ptr(const void *p, bool required) {
    if (!p) return !required;
    return aligned16(p);
}

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Gate inputs: log alpha for KDA_GATE_LOG_ALPHA and KDA_GATE_HEAD, the low-rank factors
// for the two LOWRANK gates.
bool ok_gate(const kda_config *cfg, const float *log_alpha, const void *z, const void *w, const float *bias,
             const float *a, bool needed) {
    const bool low = lowrank_gate(cfg);
    return ok_ptr(log_alpha, needed && !low) && ok_ptr(z, needed && low) && ok_ptr(w, needed && low) &&
           ok_ptr(bias, needed && low) && ok_ptr(a, needed && low);
}

void set_gate(LayerParams &p, const kda_config *cfg, const float *log_alpha, const void *z, const void *w,
              const float *bias, const float *a) {
    p.gate = cfg->gate;
    p.gate_rank = cfg->gate_rank;
    const bool low = lowrank_gate(cfg);
    p.log_alpha = low ? nullptr : log_alpha;
    p.gate_z = low ? z : nullptr;
    p.gate_w = low ? w : nullptr;
    p.gate_bias = low ? bias : nullptr;
    p.gate_a = low ? a : nullptr;
}

// Compute units the segment plan assumes: a whole MI355X (gfx950) has 256.  The plan is
// made without a HIP call, so that the host-only sizing and resolution functions never
// initialise the runtime (and give the same answer on a host without a GPU); with fewer
// compute units (a partitioned GPU) it is still correct, only split more finely.
constexpr int PLAN_CUS = 256;
int device_cu_count() { return PLAN_CUS; }

// The segmented prefill takes bf16 io and the gates whose chunks never leave the
// factorised range (the per-token path is not built into its kernel).
bool scan_supported(const kda_config *cfg) {
    return cfg->io_dtype == KDA_DTYPE_BF16 &&
           (cfg->gate == KDA_GATE_LOG_ALPHA || cfg->gate == KDA_GATE_LOWRANK || cfg->gate == KDA_GATE_HEAD);
}

// Segment length (tokens, a multiple of the 16-token chunk, at least 64) and table slots
// of the segmented prefill.  P segments per sequence rerun P - 1 of them in the last pass;
// P - 1 = floor(2 CUs / items) fills the two workgroup slots of every CU once there, and
// one more segment would need a second round (131072 tokens: 96 heads, P = 6 took 23.9 ms,
// P = 5 25.6 and P = 7 29.9; 12 heads, P = 43 took 3.45 ms and P = 42 3.8).
struct ScanPlan {
    int32_t seg_tokens, slots;
};
ScanPlan scan_plan(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    const int64_t items = static_cast<int64_t>(num_seqs) * cfg->num_heads;
    const int64_t per_seq = std::max<int64_t>(2, 1 + 2 * device_cu_count() / std::max<int64_t>(items, 1));
    const int64_t avg = (total_tokens + num_seqs - 1) / num_seqs;
    int64_t seg = ((avg + per_seq - 1) / per_seq + 15) / 16 * 16;
    seg = std::max<int64_t>(seg, 64);
    seg = std::min<int64_t>(seg, 1LL << 30);
    const int64_t slots = num_seqs + (total_tokens + seg - 1) / seg;
    return {static_cast<int32_t>(seg), static_cast<int32_t>(std::min<int64_t>(slots, 0x7fffffffLL))};
}

// AUTO and CHUNKED: the throughput kernel, or the segmented prefill when one sequential
// pass would leave most CUs idle (scan_ok false: never, for the no-allocation entry point,
// whose scratch cannot hold the segment matrices).  Measured with the full layer on bf16
// inputs: at most 3/8 as many (sequence, head) items as CUs, over sequences averaging 1024
// tokens or more, gain 1.1x (96 items of 4096 tokens: 0.92 -> 0.83 ms) to 4.5x (12 items
// of 8192: 1.79 -> 0.40 ms); at half as many items as CUs only long sequences gain (128
// items of 32768 tokens: 7.08 -> 6.68 ms; of 4096: 0.93 -> 0.97 ms, a loss); with more
// items the split loses at every length measured (160 items of 65536 tokens: 14.1 -> 16.2
// ms; 192 of 32768: 7.1 -> 10.5 ms), since those items already occupy most CUs.
int32_t resolve_algo(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens, bool scan_ok = true) {
    int algo = cfg->algo;
    if (algo == KDA_ALGO_AUTO) algo = cfg->io_dtype == KDA_DTYPE_BF16 ? KDA_ALGO_CHUNKED : KDA_ALGO_RECURRENT;
    if (algo == KDA_ALGO_CHUNKED) {
        const int64_t items = static_cast<int64_t>(num_seqs) * cfg->num_heads;
        const bool few = items <= 3 * device_cu_count() / 8 && total_tokens >= 1024LL * num_seqs;
        const bool long_seqs = items <= device_cu_count() / 2 && total_tokens >= 16384LL * num_seqs;
        algo = scan_ok && scan_supported(cfg) && (few || long_seqs) ? KDA_ALGO_CHUNKED_SCAN
                                                                    : KDA_ALGO_CHUNKED_THROUGHPUT;
    }
    return algo;
}

// Whether the resolved algorithm runs this configuration.  The chunked kernels take bf16
// io only (their split-bf16 products meet the bf16-input bar, not the fp32 one); the
// pipelined latency variant is retired; the segmented prefill lacks the per-token path of
// the gates without a floor; the low-rank gates need bf16 factors on the matrix cores.
bool supported(const kda_config *cfg, int32_t algo) {
    if (algo == KDA_ALGO_CHUNKED_LATENCY) return false;
    if (algo == KDA_ALGO_RECURRENT) return true;
    if (cfg->io_dtype != KDA_DTYPE_BF16) return false;
    return algo != KDA_ALGO_CHUNKED_SCAN || scan_supported(cfg);
}

size_t workspace_bytes(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens, int32_t algo) {
    if (algo != KDA_ALGO_CHUNKED_SCAN) return order_workspace_bytes(num_seqs);
    const ScanPlan sp = scan_plan(cfg, num_seqs, total_tokens);
    return scan_workspace_bytes(cfg->num_heads, num_seqs, sp.slots);
}

}  // namespace


size_t order_workspace_bytes(int32_t n) {
    if (n <= 1 || n > ORDER_MAX_SEQS) return 0;
    return (static_cast<size_t>(n) * sizeof(int32_t) + 255u) & ~static_cast<size_t>(255u);
}

hipError_t launch_order(const int32_t *cu_seqlens, int32_t n, int32_t *order, hipStream_t s) {
    hipLaunchKernelGGL(order_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cu_seqlens, n, order);
    return hipGetLastError();
}

}  // namespace kda

using namespace kda;

extern "C" {

void kda_config_init(kda_config *cfg, int32_t num_heads) {
    if (!cfg) return;
    cfg->num_heads = num_heads;
    cfg->head_dim = D;
    cfg->io_dtype = KDA_DTYPE_BF16;
    cfg->out_dtype = KDA_DTYPE_BF16;
    cfg->prologue = 1;
    cfg->epilogue = 1;
    cfg->algo = KDA_ALGO_AUTO;
    cfg->scale = 1.0f / sqrtf(static_cast<float>(D));
    cfg->l2_eps = 1e-6f;
    cfg->rms_eps = 1e-6f;
    cfg->gate = KDA_GATE_LOG_ALPHA;
    cfg->gate_rank = 128;
    cfg->beta_mode = KDA_BETA_VALUE;
}

int32_t kda_prefill_resolved_algo(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens) {
    if (check_config(cfg) != KDA_OK || num_seqs <= 0 || total_tokens < 0) return -1;
    const int32_t algo = resolve_algo(cfg, num_seqs, total_tokens);
    return supported(cfg, algo) ? algo : -1;
}

kda_status kda_prefill_workspace_size(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens,
                                      size_t *bytes) {
    kda_status st = check_config(cfg);
    if (st != KDA_OK) return st;
    if (!bytes || num_seqs <= 0 || total_tokens < 0) return KDA_ERR_INVALID_ARGUMENT;
    *bytes = workspace_bytes(cfg, num_seqs, total_tokens, resolve_algo(cfg, num_seqs, total_tokens));
    return KDA_OK;
}

}  // extern "C"

namespace {

// Host validation shared by both prefill entry points: everything but the workspace.
// On success *algo is the algorithm that will run (AUTO resolved as resolve_algo does with
// scan_ok) and *need the workspace bytes it uses.
kda_status check_prefill(const kda_config *cfg, const kda_prefill_args *a, const void *workspace, int32_t *algo,
                         size_t *need, bool scan_ok) {
    kda_status st = check_config(cfg);
    if (st != KDA_OK) return st;
    if (!a || a->num_seqs <= 0 || a->total_tokens < 0) return KDA_ERR_INVALID_ARGUMENT;
    const int64_t H = cfg->num_heads;
    if (static_cast<int64_t>(a->num_seqs) * H > 0x7fffffffLL) return KDA_ERR_UNSUPPORTED;
    const bool tok = a->total_tokens > 0;
    if (!ok_ptr(a->cu_seqlens, true) || !ok_ptr(a->q, tok) || !ok_ptr(a->k, tok) ||
        !ok_ptr(a->v, tok) || !ok_gate(cfg, a->log_alpha, a->gate_z, a->gate_w, a->gate_bias, a->gate_a, tok) ||
        !ok_ptr(a->beta, tok) ||
        !ok_ptr(a->o, tok) || !ok_ptr(a->g, tok && cfg->epilogue) ||
        !ok_ptr(a->conv_w, cfg->prologue != 0) || !ok_ptr(a->conv_in, false) ||
        !ok_ptr(a->conv_out, false) || !ok_ptr(a->rms_w, false) || !ok_ptr(a->state_in, false) ||
        !ok_ptr(a->state_out, false) || !ok_ptr(workspace, false) ||
        !ok_ptr(a->state_in_slots, false) || !ok_ptr(a->state_out_slots, false))
        return KDA_ERR_INVALID_ARGUMENT;
    *algo = resolve_algo(cfg, a->num_seqs, a->total_tokens, scan_ok);
    *need = workspace_bytes(cfg, a->num_seqs, a->total_tokens, *algo);
    return KDA_OK;
}

// A validated prefill call and its launches, with the workspace given apart from the
// arguments (the caller's, or the library's static scratch): a workspace smaller than the
// resolved algorithm needs (or NULL where one is needed) is refused, then a configuration
// the algorithm does not run, and only then is anything enqueued.
kda_status prefill_with(const kda_config *cfg, const kda_prefill_args *a, void *hip_stream, void *workspace,
                        size_t ws_bytes, bool scan_ok) {
    int32_t algo = 0;
    size_t need = 0;
    kda_status st = check_prefill(cfg, a, workspace, &algo, &need, scan_ok);
    if (st != KDA_OK) return st;
    if (need > 0 && (!workspace || ws_bytes < need)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (!supported(cfg, algo)) return KDA_ERR_UNSUPPORTED;
    if (algo == KDA_ALGO_CHUNKED_SCAN) {
        // the segmented prefill's grids, 2 x slots x H workgroups for the first pass and
        // 8 x N x H for the scan, must fit one 32-bit grid dimension
        const ScanPlan sp = scan_plan(cfg, a->num_seqs, a->total_tokens);
        if (2LL * sp.slots * cfg->num_heads > 0x7fffffffLL || 8LL * a->num_seqs * cfg->num_heads > 0x7fffffffLL)
            return KDA_ERR_UNSUPPORTED;
    }

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    // the launches below are checked with hipGetLastError: drop an error another call of
    // this thread left recorded in the (process-wide) runtime
    (void)hipGetLastError();
    int32_t *order = need > 0 && algo != KDA_ALGO_CHUNKED_SCAN ? static_cast<int32_t *>(workspace) : nullptr;
    if (order) {
        st = from_hip(launch_order(a->cu_seqlens, a->num_seqs, order, s));
        if (st != KDA_OK) return st;
    }
    LayerParams p{};
    p.H = cfg->num_heads;
    p.num_items = a->num_seqs * cfg->num_heads;
    p.cu_seqlens = a->cu_seqlens;
    p.order = order;
    p.q = a->q; p.k = a->k; p.v = a->v; p.g = cfg->epilogue ? a->g : nullptr;
    p.beta = a->beta;
    set_gate(p, cfg, a->log_alpha, a->gate_z, a->gate_w, a->gate_bias, a->gate_a);
    p.conv_w = cfg->prologue ? a->conv_w : nullptr;
    p.rms_w = a->rms_w;
    p.conv_in = cfg->prologue ? a->conv_in : nullptr;
    p.conv_out = cfg->prologue ? a->conv_out : nullptr;
    p.state_in = a->state_in; p.state_out = a->state_out; p.o = a->o;
    p.slots_in = a->state_in_slots; p.slots_out = a->state_out_slots;
    p.scale = cfg->scale; p.l2_eps = cfg->l2_eps; p.rms_eps = cfg->rms_eps;
    p.prologue = cfg->prologue; p.epilogue = cfg->epilogue;
    p.beta_logit = cfg->beta_mode == KDA_BETA_LOGIT;
    if (trace_enabled())
        fprintf(stderr, "[kda] prefill N=%d H=%d T=%lld io=%d out=%d algo=%d prologue=%d epilogue=%d\n",
                a->num_seqs, cfg->num_heads, static_cast<long long>(a->total_tokens), cfg->io_dtype,
                cfg->out_dtype, algo, cfg->prologue, cfg->epilogue);
    hipError_t e;
    if (algo == KDA_ALGO_CHUNKED_SCAN) {
        const ScanPlan sp = scan_plan(cfg, a->num_seqs, a->total_tokens);
        if (trace_enabled()) fprintf(stderr, "[kda] scan: %d-token segments, %d slots\n", sp.seg_tokens, sp.slots);
        e = launch_chunked_scan(p, cfg->out_dtype, a->num_seqs, sp.seg_tokens, sp.slots, workspace, s);
    } else if (algo == KDA_ALGO_CHUNKED_THROUGHPUT)
        e = launch_chunked_throughput(p, cfg->out_dtype, s);
    else
        e = launch_recurrent(p, cfg->io_dtype, cfg->out_dtype, s);
    return from_hip(e);
}

// Scratch of kda_prefill_no_alloc: one static array per GPU, held for the life of the
// process.  In host code `scratch` names a host-side stand-in, not the device array, so
// host code uses only the per-device address looked up below.
__device__ __align__(256) unsigned char scratch[KDA_NO_ALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 256;
std::mutex scratch_mu;
void *scratch_ptr[SCRATCH_MAX_DEVICES];

// Device address of `scratch` on the device of `s` (the current device for the null
// stream), looked up once per device with that device current.
kda_status device_scratch(hipStream_t s, void **out) {
    int cur = -1, dev = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KDA_ERR_HIP;
    dev = cur;
    if (s && hipStreamGetDevice(s, &dev) != hipSuccess) return KDA_ERR_HIP;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return KDA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return KDA_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return KDA_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill(const kda_config *cfg, const kda_prefill_args *a, void *hip_stream) {
    return prefill_with(cfg, a, hip_stream, a ? a->workspace : nullptr, a ? a->workspace_bytes : 0, true);
}

kda_status kda_prefill_no_alloc(const kda_config *cfg, const kda_prefill_args *a, void *hip_stream) {
    int32_t algo = 0;
    size_t need = 0;
    kda_status st = check_prefill(cfg, a, nullptr, &algo, &need, false);
    if (st != KDA_OK) return st;
    if (need > KDA_NO_ALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (!supported(cfg, algo)) return KDA_ERR_UNSUPPORTED;
    void *ws = nullptr;
    st = device_scratch(static_cast<hipStream_t>(hip_stream), &ws);
    if (st != KDA_OK) return st;
    return prefill_with(cfg, a, hip_stream, ws, KDA_NO_ALLOC_SCRATCH_BYTES, false);
}

kda_status kda_decode_step(const kda_config *cfg, const kda_decode_args *a, void *hip_stream) {
    kda_status st = check_config(cfg);
    if (st != KDA_OK) return st;
    if (!a || a->batch <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (static_cast<int64_t>(a->batch) * cfg->num_heads > 0x7fffffffLL) return KDA_ERR_UNSUPPORTED;
    if (!ok_ptr(a->q, true) || !ok_ptr(a->k, true) || !ok_ptr(a->v, true) ||
        !ok_gate(cfg, a->log_alpha, a->gate_z, a->gate_w, a->gate_bias, a->gate_a, true) ||
        !ok_ptr(a->beta, true) || !ok_ptr(a->o, true) ||
        !ok_ptr(a->state, true) || !ok_ptr(a->g, cfg->epilogue != 0) ||
        !ok_ptr(a->conv_w, cfg->prologue != 0) || !ok_ptr(a->conv_state, cfg->prologue != 0) ||
        !ok_ptr(a->rms_w, false) || !ok_ptr(a->slots, false) || !ok_ptr(a->slots_out, false))
        return KDA_ERR_INVALID_ARGUMENT;
    LayerParams p{};
    p.H = cfg->num_heads;
    p.num_items = a->batch * cfg->num_heads;
    p.cu_seqlens = nullptr;
    p.slots_in = a->slots;
    p.slots_out = a->slots_out ? a->slots_out : a->slots;
    p.q = a->q; p.k = a->k; p.v = a->v; p.g = cfg->epilogue ? a->g : nullptr;
    p.beta = a->beta;
    set_gate(p, cfg, a->log_alpha, a->gate_z, a->gate_w, a->gate_bias, a->gate_a);
    p.conv_w = cfg->prologue ? a->conv_w : nullptr;
    p.rms_w = a->rms_w;
    p.conv_in = cfg->prologue ? a->conv_state : nullptr;
    p.conv_out = cfg->prologue ? a->conv_state : nullptr;
    p.state_in = a->state; p.state_out = a->state; p.o = a->o;
    p.scale = cfg->scale; p.l2_eps = cfg->l2_eps; p.rms_eps = cfg->rms_eps;
    p.prologue = cfg->prologue; p.epilogue = cfg->epilogue;
    p.beta_logit = cfg->beta_mode == KDA_BETA_LOGIT;
    if (trace_enabled())
        fprintf(stderr, "[kda] decode B=%d H=%d io=%d out=%d\n", a->batch, cfg->num_heads,
                cfg->io_dtype, cfg->out_dtype);
    (void)hipGetLastError();  // as in kda_prefill
    return from_hip(launch_recurrent(p, cfg->io_dtype, cfg->out_dtype, static_cast<hipStream_t>(hip_stream)));
}

const char *kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case KDA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

uint32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

size_t kda_state_bytes(int32_t num_heads) {
    return num_heads > 0 ? static_cast<size_t>(num_heads) * D * D * sizeof(float) : 0;
}

}  // extern "C"
