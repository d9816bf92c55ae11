/*
 * Host-only driver for the sanitizer build of libmoe's C ABI (AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code): every argument check of every entry point, each of
 * which must return its error status before any HIP call.  No GPU is touched.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/moe.h"

static int failures = 0;
#define EXPECT(cond)                                                      \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static moe_shape shape(int T, int H, int N, int K, int Ks, int I, int gating, int act, int dtype) {
    moe_shape s;
    memset(&s, 0, sizeof(s));
    s.T = T; s.H = H; s.N_r = N; s.K_r = K; s.Ks = Ks; s.I = I;
    s.gating = gating; s.act = act; s.dtype = dtype;
    return s;
}

int main(void) {
    /* fake, never dereferenced addresses (16-byte aligned, and one misaligned) */
    char* const p = (char*)(uintptr_t)0x100000;
    char* const mis = p + 2;
    size_t bytes = 0;

    const moe_shape v3 = shape(16384, 7168, 256, 8, 1, 2048, MOE_GATE_SIGMOID_BIAS_NORM, MOE_ACT_SWIGLU, MOE_BF16);
    EXPECT(moe_workspace_size(&v3, &bytes) == MOE_OK && bytes > (size_t)16384 * 8 * (7168 + 2048) * 2);
    EXPECT(moe_workspace_size(&v3, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_workspace_size(NULL, &bytes) == MOE_ERR_INVALID_ARG);

    /* invalid shapes, one field at a time */
    moe_shape b;
    b = v3; b.T = -1;           EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.H = 100;          EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.I = 65;           EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.K_r = 257;        EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.gating = 7;       EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.act = -1;         EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.dtype = 5;        EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.n_group = 3; b.topk_group = 1;              EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.n_group = 8; b.topk_group = 9;              EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.mask_top_r = 250;                           EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_INVALID_ARG);
    b = v3; b.N_r = 2048;                                 EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_UNSUPPORTED);
    b = v3; b.T = 0x7FFFFFFF;                             EXPECT(moe_workspace_size(&b, &bytes) == MOE_ERR_UNSUPPORTED);

    /* entry points: missing or misaligned pointers, workspace too small, contract violations */
    EXPECT(moe_route(&v3, NULL, p, NULL, (int32_t*)p, (float*)p, p, bytes, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_route(&v3, mis, p, NULL, (int32_t*)p, (float*)p, p, bytes, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_route(&v3, p, p, NULL, (int32_t*)p, (float*)p, p, 16, NULL) == MOE_ERR_WORKSPACE);
    EXPECT(moe_route(&v3, p, p, NULL, (int32_t*)p, (float*)p, NULL, bytes, NULL) == MOE_ERR_WORKSPACE);
    const moe_shape sm = shape(64, 128, 16, 4, 1, 64, MOE_GATE_SOFTMAX, MOE_ACT_RELU_BIAS, MOE_F32);
    EXPECT(moe_route(&sm, p, p, (const float*)p, (int32_t*)p, (float*)p, p, bytes, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_dispatch(&v3, (int32_t*)p, NULL, (int32_t*)p, (int32_t*)p, NULL, NULL, p, bytes, NULL) ==
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_dispatch(&v3, (int32_t*)p, (int32_t*)p, (int32_t*)p, (int32_t*)p, p, NULL, p, bytes, NULL) ==
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_dispatch(&v3, (int32_t*)p, (int32_t*)p, (int32_t*)p, (int32_t*)p, p, mis, p, bytes, NULL) ==
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_expert_ffn(&v3, p, NULL, (int32_t*)p, p, (const float*)p, p, p, p, bytes, NULL) ==
           MOE_ERR_INVALID_ARG);   /* b1 with SwiGLU */
    EXPECT(moe_expert_ffn(&v3, NULL, NULL, (int32_t*)p, p, NULL, p, p, p, bytes, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_expert_ffn_packed(&sm, p, NULL, (int32_t*)p, p, NULL, p, p, p, bytes, NULL) ==
           MOE_ERR_INVALID_ARG);   /* packed banks are bf16 only */
    EXPECT(moe_shared_ffn(&v3, p, NULL, NULL, p, p, p, bytes, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_combine(&v3, p, p, p, (int32_t*)p, (float*)p, mis, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_combine(&v3, p, p, NULL, (int32_t*)p, (float*)p, p, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_layer_forward(&v3, p, p, NULL, p, NULL, p, p, NULL, p, 64, p, NULL, NULL, p, bytes, NULL) ==
           MOE_ERR_INVALID_ARG);   /* unknown flag */
    EXPECT(moe_layer_forward(&sm, p, p, NULL, p, NULL, p, p, NULL, p, MOE_FLAG_PACKED_WEIGHTS, p, NULL, NULL, p,
                             bytes, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_layer_forward(&v3, p, p, NULL, p, NULL, p, NULL, NULL, NULL, 0, p, NULL, NULL, p, bytes, NULL) ==
           MOE_ERR_INVALID_ARG);   /* shared banks missing */
    EXPECT(moe_layer_forward(&v3, p, p, NULL, p, NULL, p, p, NULL, p, 0, p, NULL, NULL, p, 1024, NULL) ==
           MOE_ERR_WORKSPACE);
    moe_shape empty = v3;
    empty.T = 0;               /* no tokens: nothing to do, nothing touched */
    EXPECT(moe_layer_forward(&empty, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL,
                             NULL, 0, NULL) == MOE_OK);
    EXPECT(moe_layer_forward_noalloc(&v3, p, p, NULL, p, NULL, p, p, NULL, p, 0, p, NULL, NULL, NULL) ==
           MOE_ERR_SCRATCH);
    EXPECT(moe_noalloc_scratch_bytes() >= ((size_t)16 << 20));
    EXPECT(moe_bias_update(&v3, NULL, 0.01f, (float*)p, NULL, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_pack_weights(p, p, 4, 96, 100, NULL) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_pack_weights(p, p + 64, 4, 64, 128, NULL) == MOE_ERR_INVALID_ARG);   /* overlapping */
    EXPECT(moe_pack_weights(p, p, 1, 32768, 65536, NULL) == MOE_ERR_UNSUPPORTED);
    int64_t n = 0;
    double ms = 0.0;
    EXPECT(moe_profile_query(99, &n, &ms) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_profile_query(0, NULL, &ms) == MOE_ERR_INVALID_ARG);
    for (int st = -6; st <= 1; ++st) EXPECT(moe_status_string(st) != NULL && moe_status_string(st)[0] != 0);
    EXPECT(moe_last_hip_error() == 0);

    if (failures) {
        fprintf(stderr, "%d failed\n", failures);
        return 1;
    }
    printf("abi checks ok\n");
    return 0;
}
