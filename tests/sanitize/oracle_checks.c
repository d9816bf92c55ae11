/*
 * Driver for the sanitizer build of the fp64 oracle (AddressSanitizer and UndefinedBehaviorSanitizer):
 * routing, expert FFNs, whole layers (own and forced selection, with and without the residual, ReLU
 * and SwiGLU, fp32 and bf16, group-limited routing, the masking probe) and the balance controller on
 * small seeded inputs, plus the argument checks.  Memory errors and undefined behaviour abort the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t T, H, N_r, K_r, Ks, I, gating, act, dtype, n_group, topk_group, mask_top_r;
} orc_shape;

int orc_route(const orc_shape* s, const void* u, const void* e, const float* bias, const int64_t* tok,
              int64_t ntok, int32_t* sel, double* g, double* gap, double* logits_out, double* scores_out);
int orc_expert_ffn(int32_t H, int32_t I, int32_t act, int32_t dtype, const void* w1, const float* b1,
                   const void* w2, const double* x, double* y);
int orc_layer(const orc_shape* s, const void* u, const void* e, const float* bias, const void* w1,
              const float* b1, const void* w2, const void* w1_sh, const float* b1_sh, const void* w2_sh,
              const int64_t* tok, int64_t ntok, const int32_t* forced_sel, int32_t residual, double* out,
              int32_t* sel, double* g, double* gap);
int orc_bias_update(int32_t N_r, int64_t T, int32_t K_r, const int32_t* counts, float gamma, const float* b_in,
                    float* b_out);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uni(void) {   /* xorshift64*, uniform in [-1, 1) */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

static void* fill(size_t n, int dtype, double scale) {
    if (dtype == 0) {
        float* a = (float*)malloc(n * sizeof(float));
        for (size_t i = 0; i < n; ++i) a[i] = (float)(scale * uni());
        return a;
    }
    uint16_t* a = (uint16_t*)malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        const float f = (float)(scale * uni());
        uint32_t bits;
        memcpy(&bits, &f, 4);
        a[i] = (uint16_t)(bits >> 16);
    }
    return a;
}

static int run(orc_shape s) {
    const size_t n1 = (size_t)(s.act == 1 ? 2 * s.I : s.I);
    void* u = fill((size_t)s.T * s.H, s.dtype, 1.0);
    void* e = fill((size_t)s.N_r * s.H, s.dtype, 0.2);
    void* w1 = fill((size_t)s.N_r * n1 * s.H, s.dtype, 0.1);
    void* w2 = fill((size_t)s.N_r * s.H * s.I, s.dtype, 0.1);
    void* w1s = s.Ks ? fill((size_t)s.Ks * n1 * s.H, s.dtype, 0.1) : NULL;
    void* w2s = s.Ks ? fill((size_t)s.Ks * s.H * s.I, s.dtype, 0.1) : NULL;
    float* b1 = s.act == 0 ? (float*)fill((size_t)s.N_r * s.I, 0, 0.1) : NULL;
    float* bias = s.gating == 1 ? (float*)fill((size_t)s.N_r, 0, 0.1) : NULL;
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)s.T);
    for (int t = 0; t < s.T; ++t) tok[t] = s.T - 1 - t;
    const size_t K = (size_t)(s.K_r > 0 ? s.K_r : 1);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * K * s.T);
    int32_t* sel2 = (int32_t*)malloc(sizeof(int32_t) * K * s.T);
    double* g = (double*)malloc(sizeof(double) * K * s.T);
    double* gap = (double*)malloc(sizeof(double) * s.T);
    double* lo = (double*)malloc(sizeof(double) * (size_t)s.N_r * s.T);
    double* sc = (double*)malloc(sizeof(double) * (size_t)s.N_r * s.T);
    double* out = (double*)malloc(sizeof(double) * (size_t)s.H * s.T);
    double* out2 = (double*)malloc(sizeof(double) * (size_t)s.H * s.T);
    int bad = 0;
    if (s.K_r > 0 && orc_route(&s, u, e, bias, tok, s.T, sel, g, gap, lo, sc) != 0) bad = 1;
    if (orc_layer(&s, u, e, bias, w1, b1, w2, w1s, b1 ? b1 : NULL, w2s, tok, s.T, NULL, 1, out, sel2, g, gap) != 0)
        bad = 1;
    if (s.K_r > 0 && memcmp(sel, sel2, sizeof(int32_t) * K * s.T) != 0) bad = 1;   /* same selection */
    if (orc_layer(&s, u, e, bias, w1, b1, w2, w1s, b1 ? b1 : NULL, w2s, tok, s.T, s.K_r ? sel : NULL, 0, out2, sel2,
                  g, gap) != 0)
        bad = 1;
    for (size_t i = 0; i < (size_t)s.H * s.T; ++i)
        if (!isfinite(out[i]) || !isfinite(out2[i])) bad = 1;
    if (bad) fprintf(stderr, "layer T=%d N=%d K=%d gating=%d act=%d dtype=%d failed\n", s.T, s.N_r, s.K_r,
                     s.gating, s.act, s.dtype);
    free(u); free(e); free(w1); free(w2); free(w1s); free(w2s); free(b1); free(bias); free(tok);
    free(sel); free(sel2); free(g); free(gap); free(lo); free(sc); free(out); free(out2);
    return bad;
}

int main(void) {
    int bad = 0;
    orc_shape s;
    memset(&s, 0, sizeof(s));
    s = (orc_shape){17, 64, 8, 2, 1, 64, 0, 0, 0, 0, 0, 0}; bad |= run(s);     /* ReLU, softmax, fp32 */
    s = (orc_shape){13, 128, 16, 4, 2, 64, 1, 1, 1, 0, 0, 0}; bad |= run(s);   /* SwiGLU, sigmoid+bias, bf16 */
    s = (orc_shape){9, 64, 12, 3, 0, 128, 2, 1, 1, 0, 0, 0}; bad |= run(s);    /* masked softmax, no shared */
    s = (orc_shape){11, 64, 16, 4, 1, 64, 1, 1, 1, 4, 2, 0}; bad |= run(s);    /* group-limited */
    s = (orc_shape){7, 64, 16, 3, 1, 64, 0, 1, 1, 0, 0, 2}; bad |= run(s);     /* masking probe */
    s = (orc_shape){5, 64, 8, 8, 1, 64, 0, 0, 0, 0, 0, 0}; bad |= run(s);      /* K_r = N_r */
    s = (orc_shape){6, 64, 8, 0, 1, 64, 0, 1, 1, 0, 0, 0}; bad |= run(s);      /* K_r = 0 */
    /* argument checks */
    orc_shape x = (orc_shape){4, 64, 8, 9, 1, 64, 0, 1, 1, 0, 0, 0};
    int32_t sel[64];
    double g[64], gap[8], out[512];
    int64_t tok[4] = {0, 1, 2, 5};
    uint16_t buf[8192] = {0};
    if (orc_route(&x, buf, buf, NULL, tok, 1, sel, g, gap, NULL, NULL) == 0) bad = 1;   /* K_r > N_r */
    x.K_r = 2;
    if (orc_route(&x, buf, buf, NULL, tok, 4, sel, g, gap, NULL, NULL) == 0) bad = 1;   /* token 5 >= T */
    if (orc_layer(&x, buf, buf, NULL, buf, NULL, buf, NULL, NULL, NULL, tok, 1, NULL, 1, out, sel, g, gap) == 0)
        bad = 1;   /* shared banks missing */
    if (orc_expert_ffn(0, 64, 1, 1, buf, NULL, buf, out, out) == 0) bad = 1;
    int32_t counts[3] = {5, 1, 0};
    float b_in[3] = {0.f, 0.f, 0.f}, b_out[3];
    if (orc_bias_update(3, 2, 3, counts, 0.5f, b_in, b_out) != 0 || b_out[0] != -0.5f || b_out[1] != 0.5f ||
        b_out[2] != 0.5f)
        bad = 1;
    if (bad) {
        fprintf(stderr, "oracle checks failed\n");
        return 1;
    }
    printf("oracle checks ok\n");
    return 0;
}
