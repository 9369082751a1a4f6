/* Host driver for a build of libkda whose host code carries AddressSanitizer
 * and UndefinedBehaviorSanitizer.  It drives every entry point of include/kda.h
 * through its host-side checks only: size queries at extreme sizes, and calls
 * whose arguments are rejected (NULL, unknown dtype, unsupported sizes,
 * misalignment, overlaps, short workspaces), so no call reaches the device.
 * The pointers are addresses inside a host buffer that is never dereferenced.
 * Refuses to run (exit 77) where a GPU is visible.  Exit status 0 on success. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <unistd.h>

#include "kda.h"

static int failures = 0;
#define TRUE_OR_FAIL(c)                                                  \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "line %d: %s does not hold\n", __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)
#define EXPECT(call, want)                                                                    \
    do {                                                                                      \
        const int st_ = (call);                                                               \
        if (st_ != (want)) {                                                                  \
            fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, st_, \
                    (int)(want), kda_last_error());                                           \
            ++failures;                                                                       \
        } else if (st_ != KDA_OK && kda_last_error()[0] == '\0') {                            \
            fprintf(stderr, "line %d: %s gave no message\n", __LINE__, #call);                \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

static _Alignas(64) unsigned char arena[1 << 16];

int main(void) {
    if (access("/dev/kfd", F_OK) == 0) {
        puts("a GPU is visible: this driver only runs host-side checks on a machine without one");
        return 77;
    }
    void* A = arena;              /* aligned, distinct addresses inside the arena */
    void* Bp = arena + 4096;
    void* C = arena + 8192;
    void* D = arena + 12288;
    void* E = arena + 16384;
    void* F = arena + 20480;
    void* G = arena + 24576;
    void* Hp = arena + 28672;
    void* mis = arena + 4;        /* not 16-byte aligned */
    size_t bytes = 0;

    TRUE_OR_FAIL(kda_abi_version() == KDA_ABI_VERSION);
    for (int s = -3; s < 12; ++s) TRUE_OR_FAIL(kda_status_string(s) && kda_status_string(s)[0]);

    /* size queries */
    EXPECT(kda_chunk_fwd_workspace_size(1, 65536, 16, 128, 128, 0, &bytes), KDA_OK);
    EXPECT(kda_chunk_fwd_workspace_size(1, 65536, 16, 128, 128, 1, &bytes), KDA_OK);
    TRUE_OR_FAIL(bytes == 0);   /* one segment needs no workspace */
    EXPECT(kda_chunk_fwd_workspace_size(1, 65536, 16, 128, 128, 4096, &bytes), KDA_OK);
    EXPECT(kda_chunk_fwd_workspace_size(1, 65536, 16, 128, 128, INT_MAX, &bytes), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd_workspace_size(1, INT_MAX, 1, 16, 16, 0, &bytes), KDA_OK);
    EXPECT(kda_chunk_fwd_workspace_size(1, INT_MAX, 1, 16, 16, 1 << 20, &bytes), KDA_OK);
    EXPECT(kda_chunk_fwd_workspace_size(INT_MAX, INT_MAX, INT_MAX, 128, 128, 0, &bytes), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd_workspace_size(1, 16, 1 << 20, 128, 128, 0, &bytes), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd_workspace_size(1, 0, 16, 128, 128, 0, &bytes), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd_workspace_size(1, 16, 16, 48, 48, 0, &bytes), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd_workspace_size(1, 16, 16, 64, 64, -1, &bytes), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd_workspace_size(1, 16, 16, 64, 64, 0, NULL), KDA_ERR_NULL);
    EXPECT(kda_chunk_bwd_workspace_size(32, 4096, 16, 128, 128, &bytes), KDA_OK);
    TRUE_OR_FAIL(bytes > 0);
    EXPECT(kda_chunk_bwd_workspace_size(INT_MAX, INT_MAX, 2, 128, 128, &bytes), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_bwd_workspace_size(1, INT_MAX, 1, 16, 16, &bytes), KDA_OK);
    EXPECT(kda_chunk_bwd_workspace_size(1, 16, 1 << 20, 128, 128, &bytes), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_bwd_workspace_size(1, -5, 2, 128, 128, &bytes), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_bwd_workspace_size(1, 5, 2, 128, 128, NULL), KDA_ERR_NULL);
    TRUE_OR_FAIL(kda_chunk_fwd_auto_segments(1, 65536, 16, 128, 128) >= 1);
    TRUE_OR_FAIL(kda_chunk_fwd_auto_segments(1, INT_MAX, 1, 16, 16) >= 1);
    TRUE_OR_FAIL(kda_chunk_fwd_auto_segments(INT_MAX, INT_MAX, INT_MAX, 128, 128) <= 0);
    TRUE_OR_FAIL(kda_chunk_fwd_auto_segments(1, 0, 1, 16, 16) <= 0);

    /* kda_chunk_fwd */
    EXPECT(kda_chunk_fwd(7, 1, 64, 1, 16, 16, 1, A, Bp, C, D, E, NULL, F, NULL, NULL, 0, NULL), KDA_ERR_DTYPE);
    EXPECT(kda_chunk_fwd(KDA_BF16, 0, 64, 1, 16, 16, 1, A, Bp, C, D, E, NULL, F, NULL, NULL, 0, NULL), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd(KDA_BF16, 1, 64, 1, 16, 32, 1, A, Bp, C, D, E, NULL, F, NULL, NULL, 0, NULL), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd(KDA_BF16, 1, 0, 1, 16, 16, 1, A, Bp, C, D, E, NULL, F, NULL, NULL, 0, NULL), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd(KDA_BF16, 1, 64, 1, 16, 16, 1, NULL, Bp, C, D, E, NULL, F, NULL, NULL, 0, NULL), KDA_ERR_NULL);
    EXPECT(kda_chunk_fwd(KDA_BF16, 1, 64, 1, 16, 16, 1, A, Bp, C, D, E, NULL, NULL, NULL, NULL, 0, NULL), KDA_ERR_NULL);
    EXPECT(kda_chunk_fwd(KDA_BF16, 1, 64, 1, 16, 16, 1, mis, Bp, C, D, E, NULL, F, NULL, NULL, 0, NULL), KDA_ERR_ALIGN);
    EXPECT(kda_chunk_fwd(KDA_BF16, 1, 64, 1, 16, 16, 1, A, Bp, C, D, E, NULL, A, NULL, NULL, 0, NULL), KDA_ERR_ALIAS);
    EXPECT(kda_chunk_fwd(KDA_F32, 1, 640, 1, 16, 16, 4, A, Bp, C, D, E, NULL, F, NULL, NULL, 0, NULL), KDA_ERR_WORKSPACE);
    EXPECT(kda_chunk_fwd(KDA_F32, 1, 640, 1, 16, 16, 4, A, Bp, C, D, E, NULL, F, NULL, G, 16, NULL), KDA_ERR_WORKSPACE);

    /* kda_chunk_fwd_noalloc: the scratch limit is checked before any device call */
    EXPECT(kda_chunk_fwd_noalloc(KDA_BF16, 64, 1 << 20, 16, 128, 128, 4096, A, Bp, C, D, E, NULL, F, NULL, NULL),
           KDA_ERR_WORKSPACE);
    EXPECT(kda_chunk_fwd_noalloc(KDA_BF16, 1, 64, 1, 16, 16, 1, NULL, Bp, C, D, E, NULL, F, NULL, NULL), KDA_ERR_NULL);

    /* kda_chunk_fwd_gated */
    EXPECT(kda_chunk_fwd_gated(KDA_BF16, 1, 64, 1, 16, 16, 1, A, Bp, C, D, E, NULL, NULL, F, NULL, NULL, 0, NULL),
           KDA_ERR_NULL);
    EXPECT(kda_chunk_fwd_gated(KDA_BF16, 1, 64, 1, 16, 16, 1, A, Bp, C, D, E, NULL, mis, F, NULL, NULL, 0, NULL),
           KDA_ERR_ALIGN);

    /* kda_chunk_fwd_unbounded */
    EXPECT(kda_chunk_fwd_unbounded(KDA_BF16, 1, 64, 1, 24, 24, A, Bp, C, D, E, NULL, F, NULL, NULL), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd_unbounded(KDA_BF16, 1, 64, 1, 16, 16, A, Bp, C, NULL, E, NULL, F, NULL, NULL), KDA_ERR_NULL);

    /* kda_chunk_bwd */
    EXPECT(kda_chunk_bwd(KDA_BF16, 1, 64, 1, 16, 16, A, Bp, C, D, E, NULL, F, NULL, NULL, G, Hp, A, Bp, NULL,
                         NULL, 0, NULL), KDA_ERR_NULL);
    EXPECT(kda_chunk_bwd(9, 1, 64, 1, 16, 16, A, Bp, C, D, E, NULL, F, NULL, G, Hp, G, Hp, G, NULL, NULL, 0, NULL),
           KDA_ERR_DTYPE);
    EXPECT(kda_chunk_bwd(KDA_BF16, 1, 64, 1, 16, 16, A, Bp, C, D, E, NULL, F, NULL, mis, G, Hp, A, Bp, NULL,
                         NULL, 0, NULL), KDA_ERR_ALIGN);

    /* decode */
    EXPECT(kda_decode_step(KDA_BF16, 0, 1, 16, 16, A, Bp, C, D, E, F, G, NULL), KDA_ERR_SHAPE);
    EXPECT(kda_decode_step(KDA_BF16, 1, 1, 16, 16, A, Bp, C, D, E, NULL, G, NULL), KDA_ERR_NULL);
    EXPECT(kda_decode_step(KDA_BF16, 1, 1, 16, 16, A, Bp, C, D, E, F, mis, NULL), KDA_ERR_ALIGN);
    EXPECT(kda_decode_step_gated(KDA_BF16, 1, 1, 16, 16, A, Bp, C, D, E, F, NULL, G, NULL), KDA_ERR_NULL);

    /* gate */
    EXPECT(kda_gate(1, 64, 1, 16, NULL, (float*)A, NULL, NULL), KDA_ERR_NULL);
    EXPECT(kda_gate(1, 64, 1, 16, (const float*)mis, (float*)A, NULL, NULL), KDA_ERR_ALIGN);
    EXPECT(kda_gate(1, -1, 1, 16, (const float*)Bp, (float*)A, NULL, NULL), KDA_ERR_SHAPE);
    EXPECT(kda_gate(1, INT_MAX, 1 << 20, 128, (const float*)Bp, (float*)A, NULL, NULL), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd(KDA_BF16, 1, INT_MAX, 1, 16, 16, INT_MAX, A, Bp, C, D, E, NULL, F, NULL, NULL, 0, NULL),
           KDA_ERR_SHAPE);

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    puts("abi driver: ok");
    return 0;
}
