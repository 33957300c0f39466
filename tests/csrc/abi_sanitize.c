/*
 * abi_sanitize.c -- the library's host-side argument checks under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Built (by tests/test_sanitizers.py) from the library's
 * sources compiled for the host only, so no call here can reach a GPU: every call below
 * is refused by the checks that run before the first HIP call, and the program verifies
 * each refusal's status.  The pointers are fake, aligned and never dereferenced.
 * Exit status 0 when every check holds; a sanitizer report aborts with a nonzero status.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int failures = 0;

#define EXPECT(call, want)                                                                \
    do {                                                                                  \
        const int got_ = (int)(call);                                                     \
        if (got_ != (int)(want)) {                                                        \
            fprintf(stderr, "line %d: %s = %d, want %d\n", __LINE__, #call, got_, (int)(want)); \
            ++failures;                                                                   \
        }                                                                                 \
    } while (0)

#define FAKE ((void *)(uintptr_t)0x10000)

static kda_prefill_args prefill_args(void) {
    kda_prefill_args a;
    memset(&a, 0, sizeof a);
    a.num_seqs = 2;
    a.cu_seqlens = (const int32_t *)FAKE;
    a.total_tokens = 10;
    a.q = a.k = a.v = FAKE;
    a.log_alpha = (const float *)FAKE;
    a.beta = (const float *)FAKE;
    a.g = FAKE;
    a.conv_w = (const float *)FAKE;
    a.o = FAKE;
    a.state_out = (float *)FAKE;
    a.workspace = FAKE;
    a.workspace_bytes = 256;
    return a;
}

static kda_decode_args decode_args(void) {
    kda_decode_args a;
    memset(&a, 0, sizeof a);
    a.batch = 4;
    a.q = a.k = a.v = FAKE;
    a.log_alpha = (const float *)FAKE;
    a.beta = (const float *)FAKE;
    a.g = FAKE;
    a.conv_w = (const float *)FAKE;
    a.conv_state = FAKE;
    a.state = (float *)FAKE;
    a.o = FAKE;
    return a;
}

int main(void) {
    kda_config c;
    kda_prefill_args a;
    size_t bytes = 0;

    EXPECT(kda_abi_version(), KDA_ABI_VERSION);
    EXPECT(kda_state_bytes(96) == (size_t)96 * 128 * 128 * 4, 1);
    EXPECT(kda_state_bytes(0), 0);
    for (int s = -3; s < 12; ++s) EXPECT(kda_status_string((kda_status)s) != NULL, 1);

    kda_config_init(&c, 96);
    EXPECT(c.num_heads, 96);
    EXPECT(kda_prefill_workspace_size(&c, 1, 100, &bytes), KDA_OK);
    EXPECT(bytes, 0);
    EXPECT(kda_prefill_workspace_size(&c, 0, 10, &bytes), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_prefill_workspace_size(&c, 1, 131072, &bytes), KDA_OK);
    EXPECT(bytes > 0, 1);
    EXPECT(kda_prefill_workspace_size(NULL, 1, 10, &bytes), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_prefill_resolved_algo(&c, 1, 131072), KDA_ALGO_CHUNKED_SCAN);
    EXPECT(kda_prefill_resolved_algo(&c, 4, 16384), KDA_ALGO_CHUNKED_THROUGHPUT);
    EXPECT(kda_prefill_resolved_algo(&c, 0, 0), -1);
    EXPECT(kda_prefill_resolved_algo(&c, 1, -1), -1);
    EXPECT(kda_prefill_resolved_algo(NULL, 1, 1), -1);

    /* prefill: each required pointer missing, misaligned pointers, bad sizes and configs */
    kda_config_init(&c, 4);
    a = prefill_args();
    EXPECT(kda_prefill(NULL, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_prefill(&c, NULL, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.cu_seqlens = NULL; EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.q = NULL;          EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.k = NULL;          EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.v = NULL;          EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.log_alpha = NULL;  EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.beta = NULL;       EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.g = NULL;          EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.conv_w = NULL;     EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.o = NULL;          EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.q = (const char *)FAKE + 2;  EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.state_in = (const float *)((const char *)FAKE + 8);
    EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.state_in_slots = (const int32_t *)((const char *)FAKE + 4);
    EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.num_seqs = 0;      EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.total_tokens = -1; EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a = prefill_args(); a.workspace = NULL;  EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_WORKSPACE_TOO_SMALL);
    a = prefill_args(); a.workspace_bytes = 8; EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_WORKSPACE_TOO_SMALL);
    a = prefill_args();
    c.head_dim = 64; EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_UNSUPPORTED);
    kda_config_init(&c, 4); c.num_heads = 0; EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    kda_config_init(&c, 4); c.io_dtype = 7;  EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    kda_config_init(&c, 4); c.algo = 9;      EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    kda_config_init(&c, 4); c.gate = 5;      EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    kda_config_init(&c, 4); c.beta_mode = 2; EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    kda_config_init(&c, 4); c.rms_eps = -1.0f; EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    /* the chunked kernels refuse fp32 io; the retired latency variant refuses everything */
    kda_config_init(&c, 4); c.io_dtype = KDA_DTYPE_F32; c.algo = KDA_ALGO_CHUNKED_THROUGHPUT;
    a = prefill_args(); a.num_seqs = 1; a.workspace_bytes = (size_t)1 << 40;
    EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_UNSUPPORTED);
    kda_config_init(&c, 4); c.algo = KDA_ALGO_CHUNKED_LATENCY;
    EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_UNSUPPORTED);
    /* low-rank gate: its four factors are required, the rank is checked */
    kda_config_init(&c, 4); c.gate = KDA_GATE_LOWRANK;
    a = prefill_args(); a.log_alpha = NULL;
    EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);
    a.gate_z = a.gate_w = FAKE; a.gate_bias = a.gate_a = (const float *)FAKE; a.workspace = NULL;
    EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_WORKSPACE_TOO_SMALL);
    c.gate_rank = 48; EXPECT(kda_prefill(&c, &a, NULL), KDA_ERR_UNSUPPORTED);

    /* the no-allocation entry point validates the same way, before any HIP call (the
       segmented prefill, named, needs more than its scratch; AUTO never selects it there) */
    kda_config_init(&c, 96); c.algo = KDA_ALGO_CHUNKED_SCAN;
    a = prefill_args(); a.num_seqs = 1; a.total_tokens = 131072; a.workspace = NULL; a.workspace_bytes = 0;
    EXPECT(kda_prefill_no_alloc(&c, &a, NULL), KDA_ERR_WORKSPACE_TOO_SMALL);
    kda_config_init(&c, 4);
    a = prefill_args(); a.q = NULL; EXPECT(kda_prefill_no_alloc(&c, &a, NULL), KDA_ERR_INVALID_ARGUMENT);

    /* decode */
    kda_decode_args d;
    kda_config_init(&c, 4);
    d = decode_args(); d.q = NULL;          EXPECT(kda_decode_step(&c, &d, NULL), KDA_ERR_INVALID_ARGUMENT);
    d = decode_args(); d.state = NULL;      EXPECT(kda_decode_step(&c, &d, NULL), KDA_ERR_INVALID_ARGUMENT);
    d = decode_args(); d.conv_state = NULL; EXPECT(kda_decode_step(&c, &d, NULL), KDA_ERR_INVALID_ARGUMENT);
    d = decode_args(); d.batch = 0;         EXPECT(kda_decode_step(&c, &d, NULL), KDA_ERR_INVALID_ARGUMENT);
    d = decode_args(); d.slots = (const int32_t *)((const char *)FAKE + 4);
    EXPECT(kda_decode_step(&c, &d, NULL), KDA_ERR_INVALID_ARGUMENT);
    c.head_dim = 256; d = decode_args();    EXPECT(kda_decode_step(&c, &d, NULL), KDA_ERR_UNSUPPORTED);
    EXPECT(kda_decode_step(NULL, &d, NULL), KDA_ERR_INVALID_ARGUMENT);

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi checks passed\n");
    return 0;
}
