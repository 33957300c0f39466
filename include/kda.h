/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) core.
 *
 * What is computed (per head h, per token t of each packed sequence), as the
 * KDA step list of the OpenModelAtlas page "Kimi K3 - KDA layer" states it:
 *
 *   prologue  x^c_t = SiLU(sum_{j=0..3} w_x[j] * x^p_{t-j})  for x in {q, k, v}
 *             q^ = q^c / ||q^c||,  k^ = k^c / ||k^c||  (per head, 128 channels;
 *             v gets no normalisation -- "Inside Kimi K3: How KDA, AttnRes,
 *             and 896 Experts Work", section "Short convolutions give KDA
 *             local order before recurrence")
 *   decay     S <- Diag(alpha_t) S,  alpha_t = exp(log_alpha_t) per key channel
 *   delta     S <- S + beta_t k^ (v - S^T k^)^T
 *   read      o~ = S^T q^ * scale   (scale = 1/sqrt(128))
 *   epilogue  o = sigmoid(g) * RMSNorm(o~)  (per head over the 128 value
 *             channels, gain w_rms shared by all heads, no bias)
 *
 * The order decay -> predict -> error -> write -> read is the one given in
 * section "KDA writes corrections into a recurrent matrix" of the same
 * "Inside Kimi K3" page; alpha scales row i of S (the key channel) as in
 * "Kimi K3: Architecture and SGLang Day-0 Support", "Math details: how KDA
 * gates and rewrites the same S".
 *
 * Conventions shared by every entry point:
 *  - d_k = d_v = 128 (KDA_HEAD_DIM); H = num_heads heads; all activations are
 *    token-major [tokens][H][128] (the projection output [tokens][H*128]).
 *  - The recurrent state is fp32 [.., H, 128, 128], S[i][j], i = key channel
 *    (row), j = value channel, row-major.
 *  - Conv caches are [N][3 streams q,k,v][3 taps, oldest first][H*128] in
 *    io_dtype: the last three pre-conv inputs of each stream.  Conv weights
 *    are fp32 [3 streams][H*128][4]; tap j multiplies x_{t-j}; no bias.
 *  - log_alpha is fp32 and must lie in [-5, 0] (the log-decay floor of "The
 *    lower bound on decay is a hardware decision", "Inside Kimi K3") unless the
 *    gate is KDA_GATE_LOG_ALPHA_UNBOUNDED (any value <= 0); beta is fp32 in
 *    [0, 1].  These are documented preconditions, not checked on the device:
 *    values outside them may produce inf/NaN in the chunked kernels.
 *  - Pointers are device pointers unless marked "host".  Every device pointer
 *    must be 16-byte aligned.  The caller owns every buffer; the library
 *    allocates no device memory in these calls and keeps no pointer after it
 *    returns.
 *  - Calls are asynchronous on the given HIP stream (0 = the null stream),
 *    reentrant and thread-safe; results are valid once the stream reaches
 *    the call.  Host-side validation failures return an error status and
 *    enqueue nothing.  No call aborts or throws.
 *  - The calls enqueue kernel launches only (no memset, copy, allocation or
 *    host synchronisation), so a call can be captured in a HIP graph and the
 *    graph replayed; the buffers it names are then fixed.  kda_prefill_no_alloc
 *    resolves its per-GPU scratch on its first call on a GPU: make that first
 *    call outside a capture.
 *  - Initialisation order: the library shares the process's HIP runtime and
 *    registers its kernels when it is loaded.  Initialise the runtime first
 *    (any HIP call that touches the device, e.g. hipSetDevice or hipFree(0),
 *    from the thread that will load the library), then load the library, then
 *    start other threads that call it.  Loaded into a runtime that was not yet
 *    initialised while other threads were already running, every later launch
 *    of the library has been seen to fail with hipErrorNoDevice (KDA_ERR_HIP);
 *    the cause inside the runtime is not known.  The Python binding follows
 *    this order (it initialises torch's device before loading the library).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128
#define KDA_ABI_VERSION 5u

/* Status codes. */
typedef int32_t kda_status;
#define KDA_OK 0
#define KDA_ERR_INVALID_ARGUMENT 1   /* null / misaligned pointer, bad size or enum */
#define KDA_ERR_UNSUPPORTED 2        /* head_dim != 128 or an unsupported combination */
#define KDA_ERR_WORKSPACE_TOO_SMALL 3
#define KDA_ERR_HIP 4                /* a HIP runtime call or launch failed */

/* Element types of activations. */
#define KDA_DTYPE_F32 0
#define KDA_DTYPE_BF16 1

/* Prefill algorithm.  AUTO picks CHUNKED for bf16 inputs and RECURRENT for fp32.
 * CHUNKED resolves to THROUGHPUT, or to CHUNKED_SCAN for a few long sequences (below).
 * The chunked algorithms take bf16 io only (fp32 io returns KDA_ERR_UNSUPPORTED): they
 * compute in 16-token chunks on the matrix cores with bf16 hi/lo operand splits and
 * fp32 accumulation, which keeps the raw read o~ and the state within about 6e-4 of an
 * fp64 evaluation (max |err| / RMS), inside the 1e-2 bar of the bf16-input path but
 * not the 1e-4 bar of the fp32 path.  RECURRENT is the fp32 reference-precision path
 * (within 1e-4), and takes either io type. */
#define KDA_ALGO_AUTO 0
#define KDA_ALGO_RECURRENT 1            /* token-sequential fp32 recurrence */
#define KDA_ALGO_CHUNKED 2              /* chunked, the variant the library prefers */
#define KDA_ALGO_CHUNKED_THROUGHPUT 3   /* 8-wave workgroups, two per compute unit */
#define KDA_ALGO_CHUNKED_LATENCY 4      /* retired (it was slower at every shape measured):
                                           returns KDA_ERR_UNSUPPORTED */
/* CHUNKED_SCAN: the THROUGHPUT kernel over segments of each sequence, run in parallel.
 * A chunk's effect on the state is affine, S -> M S + B (the composition that
 * "Inside Kimi K3 ...", "KDA writes corrections into a recurrent matrix", unrolls
 * token by token), so each segment but the first and last is run from S = I with
 * v = 0 (its M) and from S = 0 (its B); the first segment runs from the given
 * state.  A scan S_{p+1} = M_p S_p + B_p over the segments then gives every
 * segment's entering state, and segments 1 .. P-1 run again from it to produce
 * their outputs.  About 2.6x the arithmetic of one pass, for up to P-fold
 * parallelism, with P segments per sequence (at least 64 tokens each) such that the
 * rerun of P - 1 of them fills two workgroup slots on each compute unit.  AUTO and
 * CHUNKED take it for bf16 inputs when one pass would leave most compute units idle:
 * at most 3/8 as many (sequence, head) items as compute units over sequences averaging
 * 1024 tokens or more (12 items of 8192 tokens: 4.5x faster; 96 items of 4096: 1.1x),
 * or at most half as many items as compute units over sequences averaging 16384 tokens
 * or more (with more items the split measured slower at every length).
 * bf16 io and the LOG_ALPHA, LOWRANK and HEAD gates only; its M and B matrices live in
 * the workspace. */
#define KDA_ALGO_CHUNKED_SCAN 5

/* Where the decay comes from ("Kimi K3 - KDA layer" step list: z_down = x W_down,
 * z = z_down W_up, alpha = exp(-5 sigmoid(e^A (z + b_alpha)))).  LOG_ALPHA: the
 * caller passes log alpha per (token, head, key channel).  LOWRANK: the caller
 * passes the rank-r projection z_down and the up-projection, bias and per-head A,
 * and the kernels form log alpha = -5 sigmoid(e^{A_h} (z_down W_up^T + b)) on the
 * fly, which removes the fp32 log alpha stream (512 B per token-head). */
#define KDA_GATE_LOG_ALPHA 0
#define KDA_GATE_LOWRANK 1
/* HEAD: one decay per (token, head) shared by the 128 key channels, the scalar gate
 * of Mamba-2 / Gated DeltaNet that KDA generalises ("Kimi K3's Architecture ...",
 * section "Channel-wise decay, and the floor K3 puts under it"): log_alpha is
 * [T][H].  The decay factors leave the channel contractions, so the kernel forms
 * fewer operand planes and exponentials and spends part of the saving on the row
 * scales of the products: at 4 x 4096 tokens x 96 heads it measured 5% faster than the
 * channel gate (1.24 against 1.30 ms). */
#define KDA_GATE_HEAD 2
/* LOWRANK_SOFTPLUS: Kimi Linear's gate, formed in the kernels from the same factors as
 * LOWRANK: log alpha = -e^{A_h} softplus(z_down W_up^T + b), which has no floor
 * ("Kimi K3's Architecture ...", section "Channel-wise decay, and the floor K3 puts
 * under it").  Chunks in which some channel decays by more than 2^-116 take an exact
 * per-token path in the chunked kernel; the others keep the matrix-core path. */
#define KDA_GATE_LOWRANK_SOFTPLUS 3
/* LOG_ALPHA_UNBOUNDED: log alpha passed as for LOG_ALPHA but with any value <= 0 (no
 * floor, e.g. a Kimi Linear gate formed outside the library), handled as described for
 * LOWRANK_SOFTPLUS.  On the per-token path each token's decay alpha = exp(log alpha)
 * is formed from its own log alpha, not from differences of running sums, so a very
 * deep decay loses no precision. */
#define KDA_GATE_LOG_ALPHA_UNBOUNDED 4

/* What the beta array holds.  VALUE: beta itself, in [0, 1].  LOGIT: the pre-activation
 * w = x W_beta of the "Kimi K3 - KDA layer" step list, any finite value; the kernels
 * form beta = sigmoid(w) themselves. */
#define KDA_BETA_VALUE 0
#define KDA_BETA_LOGIT 1

typedef struct {
    int32_t num_heads;   /* H > 0 */
    int32_t head_dim;    /* must be 128 */
    int32_t io_dtype;    /* KDA_DTYPE_*: q, k, v, g and the conv caches */
    int32_t out_dtype;   /* KDA_DTYPE_*: o */
    int32_t prologue;    /* 1: conv4 + SiLU + L2 on q, k (SiLU only on v); 0: q, k, v used as given */
    int32_t epilogue;    /* 1: o = sigmoid(g) * RMSNorm(o~) * w_rms; 0: o = o~ */
    int32_t algo;        /* KDA_ALGO_* (prefill only) */
    float scale;         /* read scale; 1/sqrt(128) in the layer */
    float l2_eps;        /* x / sqrt(sum x^2 + l2_eps) */
    float rms_eps;       /* x / sqrt(mean x^2 + rms_eps) */
    int32_t gate;        /* KDA_GATE_* */
    int32_t gate_rank;   /* r of the LOWRANK gates: a multiple of 32 in [32, 128] */
    int32_t beta_mode;   /* KDA_BETA_*: what the beta array holds */
} kda_config;

/* Fills *cfg with the layer's defaults for H heads: bf16 io and output,
 * prologue and epilogue on, AUTO algorithm, scale 1/sqrt(128), eps 1e-6,
 * log alpha given (gate_rank 128 for when LOWRANK is chosen), beta given as a value. */
void kda_config_init(kda_config *cfg, int32_t num_heads);

/* ------------------------------------------------------------------ prefill
 * Runs the whole layer core over N packed variable-length sequences.
 * Sequence n covers tokens [cu_seqlens[n], cu_seqlens[n+1]); it starts from
 * state_in[r_in] (zeros when NULL) and conv_in[r_in] (zeros when NULL) and
 * leaves its final state in state_out[r_out] and its last three pre-conv
 * inputs in conv_out[r_out].  The rows are r_in = state_in_slots[n] and
 * r_out = state_out_slots[n], or n where a slot array is NULL, so the state
 * and conv arrays can be pools of per-request rows.  Reading a read-only prefix
 * checkpoint row and writing the request's own row is the copy-on-write fork of
 * "Kimi K3: Architecture and SGLang Day-0 Support", section "RadixAttention:
 * prefix caching for KDA state".  A row written by one sequence must not be
 * read or written by another sequence of the same call.  A zero-length
 * sequence copies state and cache from its in row to its out row.
 * Speculative verification runs draft tokens from the committed rows with
 * state_out and conv_out NULL, then replays the accepted tokens in place (the
 * replay of accepted inputs in "Inside Kimi K3: How KDA, AttnRes, and 896
 * Experts Work", section "What could go wrong").
 */
typedef struct {
    int32_t num_seqs;             /* N > 0 */
    const int32_t *cu_seqlens;    /* device [N+1]: cu[0] = 0, non-decreasing, cu[N] = total_tokens */
    int64_t total_tokens;         /* T >= 0 */
    const void *q, *k, *v;        /* [T][H][128] io_dtype */
    const float *log_alpha;       /* [T][H][128] fp32 in [-5, 0] (gate LOG_ALPHA) or <= 0 (LOG_ALPHA_UNBOUNDED),
                                     or [T][H] (gate HEAD); else unused */
    const float *beta;            /* [T][H] fp32: beta in [0, 1], or its pre-activation (beta_mode LOGIT) */
    const void *g;                /* [T][H][128] io_dtype; required iff epilogue */
    const float *conv_w;          /* [3][H*128][4] fp32; required iff prologue */
    const void *conv_in;          /* [rows][3][3][H*128] io_dtype or NULL (zero history) */
    void *conv_out;               /* same layout or NULL (not written); may alias conv_in */
    const float *rms_w;           /* [128] fp32 or NULL (ones) */
    const float *state_in;        /* [rows][H][128][128] fp32 or NULL (zeros) */
    float *state_out;             /* same layout or NULL (not written); may alias state_in */
    void *o;                      /* [T][H][128] out_dtype; must not alias any input */
    void *workspace;              /* device scratch of at least kda_prefill_workspace_size bytes */
    size_t workspace_bytes;
    const int32_t *state_in_slots;   /* device [N] rows of state_in / conv_in, or NULL (row n) */
    const int32_t *state_out_slots;  /* device [N] rows of state_out / conv_out, or NULL (row n) */
    /* gate == LOWRANK only (required then, ignored otherwise): */
    const void *gate_z;           /* [T][r] io_dtype: z_down of each token (shared by the heads) */
    const void *gate_w;           /* [H*128][r] io_dtype: W_up stored output-major (row c = channel c) */
    const float *gate_bias;       /* [H*128] fp32: b_alpha */
    const float *gate_a;          /* [H] fp32: A_h (the multiplier is e^{A_h}) */
} kda_prefill_args;

/* Bytes of device workspace kda_prefill needs for N sequences of total_tokens
 * tokens: the longest-first order of the sequences, or, when the algorithm resolves
 * to CHUNKED_SCAN, the segment table and two fp32 128 x 128 matrices per (segment,
 * head) (about 128 KiB x H x (N + total_tokens / segment length)).  Writes the
 * size to *bytes. */
kda_status kda_prefill_workspace_size(const kda_config *cfg, int32_t num_seqs,
                                      int64_t total_tokens, size_t *bytes);

kda_status kda_prefill(const kda_config *cfg, const kda_prefill_args *args, void *hip_stream);

/* kda_prefill for callers that cannot allocate device memory: code being captured into a
 * HIP graph, tight serving loops, and harnesses that forbid allocation.  The arguments are
 * those of kda_prefill except that args->workspace and args->workspace_bytes are ignored:
 * the library's own static scratch of KDA_NO_ALLOC_SCRATCH_BYTES per GPU takes their
 * place.  That array is a file-scope device array, one per GPU the library runs on, held
 * until the process ends; no call here allocates or frees memory.  Limit: configurations
 * whose workspace (kda_prefill_workspace_size) exceeds KDA_NO_ALLOC_SCRATCH_BYTES return
 * KDA_ERR_WORKSPACE_TOO_SMALL and enqueue nothing: the segmented prefill
 * (KDA_ALGO_CHUNKED_SCAN) never fits, so here AUTO and CHUNKED never select it (they
 * run the throughput kernel where kda_prefill would split the sequences), and naming
 * it is refused; the other algorithms need at most 32 KiB (the longest-first order of
 * up to 8192 sequences).  Every call on one
 * GPU shares that GPU's array, and the kernels overwrite all of it that they read, so no
 * state carries from one call to the next; calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race on the array and
 * must not be made.  The first call on a GPU looks up the array's device address
 * (hipGetSymbolAddress, with that GPU made current for the lookup); a failure there
 * returns KDA_ERR_HIP. */
#define KDA_NO_ALLOC_SCRATCH_BYTES 65536u
kda_status kda_prefill_no_alloc(const kda_config *cfg, const kda_prefill_args *args, void *hip_stream);

/* The KDA_ALGO_* that kda_prefill runs for this configuration, num_seqs sequences
 * and total_tokens tokens on the current device (AUTO and CHUNKED resolved; the
 * no-allocation entry point runs CHUNKED_THROUGHPUT where this says CHUNKED_SCAN), or -1
 * when the configuration is invalid, num_seqs <= 0 or total_tokens < 0.  Host only;
 * enqueues nothing. */
int32_t kda_prefill_resolved_algo(const kda_config *cfg, int32_t num_seqs, int64_t total_tokens);

/* -------------------------------------------------------------- decode step
 * One token per request, the same layer core as prefill at T = 1 per
 * sequence: the conv caches are shifted and the state is updated in place.
 * A decode step touches only the fixed-size state, no history, and replaces
 * it where it lies ("Kimi K3: Architecture and SGLang Day-0 Support", the
 * linear-attention section and "SGLang's day-0 adaptations").  Request b reads pool row
 * slots[b] and writes pool row slots_out[b] (the same row when slots_out is
 * NULL); a distinct out row forks the request from a read-only checkpoint
 * (copy on write).  A row written by one request must not be read or written
 * by another request of the same call.
 */
typedef struct {
    int32_t batch;                /* B > 0 requests */
    const void *q, *k, *v;        /* [B][H][128] io_dtype */
    const float *log_alpha;       /* [B][H][128] fp32 (gate LOG_ALPHA) or [B][H] (gate HEAD); else unused */
    const float *beta;            /* [B][H] fp32: beta, or its pre-activation (beta_mode LOGIT) */
    const void *g;                /* [B][H][128] io_dtype; required iff epilogue */
    const float *conv_w;          /* [3][H*128][4] fp32; required iff prologue */
    void *conv_state;             /* [slots][3][3][H*128] io_dtype, updated in place; required iff prologue */
    const float *rms_w;           /* [128] fp32 or NULL (ones) */
    float *state;                 /* [slots][H][128][128] fp32, updated in place */
    const int32_t *slots;         /* device [B] pool row each request reads, or NULL (row b) */
    void *o;                      /* [B][H][128] out_dtype */
    const int32_t *slots_out;     /* device [B] pool row each request writes, or NULL (its slots row) */
    const void *gate_z;           /* gate == LOWRANK: [B][r] io_dtype (as in kda_prefill_args) */
    const void *gate_w;           /* [H*128][r] io_dtype */
    const float *gate_bias;       /* [H*128] fp32 */
    const float *gate_a;          /* [H] fp32 */
} kda_decode_args;

kda_status kda_decode_step(const kda_config *cfg, const kda_decode_args *args, void *hip_stream);

/* ------------------------------------------------------------------- misc */
const char *kda_status_string(kda_status status); /* static string, never NULL */
uint32_t kda_abi_version(void);                    /* KDA_ABI_VERSION */
size_t kda_state_bytes(int32_t num_heads);          /* bytes of one sequence's state: H*128*128*4 */

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
