/*
 * fp64 CPU oracle for the DeepSeekMoE layer forward pass.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
 * baseline call this code.  It shares nothing with the HIP library: no header,
 * no kernel, no helper, no table.  It is deliberately plain and slow: every
 * sum is a left-to-right fp64 loop, selection is a full sort, and no step is
 * blocked, fused or reordered.
 *
 * What it computes, per token t (pages cited by title and equation):
 *
 *   llm-infra-atlas "02 Fine-grained MoE", section 2.1, DeepSeekMoE Eq. 6-8:
 *     l_i = u_t . e_i,   s_i = softmax_i(l),   g_i = s_i if s_i is among the
 *     top-K_r scores, else 0 (no renormalisation).
 *   Same page, section 3.1, DeepSeek-V3 Eq. 12-15:
 *     s_i = sigmoid(u_t . e_i), g'_i = s_i on the top-K set, g = g' / sum g'.
 *   ibossgateway "MoE watershed", section 7.4 (aux-loss-free balancing):
 *     the top-k ranks s_i + b_i; the output weights use the raw s_i.
 *   tomabc "DeepSeekMoE" explainer, fine-grained section: the masked gate
 *     (non-top scores set to -inf before the softmax), i.e. the softmax taken
 *     over the selected logits only.  Gating mode 2 here.
 *   llm-infra-atlas section 4: node/group-limited routing, scores summed per
 *     group, groups chosen first, experts then chosen inside them.
 *   llm-infra-atlas section 1: the masking probe (drop each token's
 *     highest-ranked routed experts, re-select top-k from the rest).
 *   tomabc explainer: expert FFN a = ReLU(x W_i + b_i), output a V_i.
 *   ibossgateway section 7.6 names "SwiGLU": FFN(x) = W2 (SiLU(Wg x) * (Wu x)),
 *     SiLU(z) = z / (1 + e^-z), no biases (plain reading; the pages give no
 *     formula).
 *   llm-infra-atlas section 3.1, DeepSeekMoE Eq. 9-11:
 *     h_t = sum_{j<Ks} FFN^shared_j(u_t) + sum_i g_i FFN_i(u_t) + u_t.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): ties in a ranking go to the lower index; the softmax runs over
 * the routed experts only; the bias is added to the post-sigmoid score; if the
 * selected sigmoid scores sum to zero each weight is 1/K_r; no routed scaling
 * factor; group scores are the sum of the selection keys in the group.
 *
 * Storage: weights are [out, in] row-major (nn.Linear layout).  For SwiGLU the
 * first-layer rows [0, I) are the gate and rows [I, 2I) the up projection.
 * dtype 0 = fp32, dtype 1 = bf16 (uint16 bits); both are widened to fp64
 * exactly.  The ReLU bias b1 is always fp32; the selection bias is fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t T, H, N_r, K_r, Ks, I;
    int32_t gating;     /* 0 softmax, 1 sigmoid + selection bias + normalise, 2 softmax over the selected */
    int32_t act;        /* 0 ReLU(xW+b)V, 1 SwiGLU */
    int32_t dtype;      /* 0 fp32, 1 bf16 */
    int32_t n_group;    /* group-limited routing: number of contiguous groups, 0 = off */
    int32_t topk_group; /* groups kept per token */
    int32_t mask_top_r; /* masking probe: drop the r highest-key experts, 0 = off */
} orc_shape;

enum { ORC_OK = 0, ORC_BAD = -1 };

static double ld(const void* p, int dtype, size_t i) {
    if (dtype == 0) return (double)((const float*)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* sum_h w[off + h] * x[h], left to right. */
static double dot(const void* w, int dtype, size_t off, const double* x, int n) {
    double acc = 0.0;
    if (dtype == 0) {
        const float* p = (const float*)w + off;
        for (int h = 0; h < n; ++h) acc += (double)p[h] * x[h];
    } else {
        const uint16_t* p = (const uint16_t*)w + off;
        for (int h = 0; h < n; ++h) {
            uint32_t bits = (uint32_t)p[h] << 16;
            float f;
            memcpy(&f, &bits, 4);
            acc += (double)f * x[h];
        }
    }
    return acc;
}

static int check_shape(const orc_shape* s) {
    if (!s || s->T < 0 || s->H <= 0 || s->N_r < 0 || s->K_r < 0 || s->Ks < 0 || s->I <= 0) return ORC_BAD;
    if (s->K_r > s->N_r) return ORC_BAD;
    if (s->gating < 0 || s->gating > 2 || s->act < 0 || s->act > 1 || s->dtype < 0 || s->dtype > 1) return ORC_BAD;
    if (s->n_group) {
        if (s->n_group < 0 || s->N_r % s->n_group || s->topk_group <= 0 || s->topk_group > s->n_group) return ORC_BAD;
        if (s->topk_group * (s->N_r / s->n_group) < s->K_r) return ORC_BAD;
        if (s->mask_top_r) return ORC_BAD;
    }
    if (s->mask_top_r < 0 || s->mask_top_r + s->K_r > s->N_r) return ORC_BAD;
    return ORC_OK;
}

/* ---- ranking: (key descending, index ascending) ---------------------------------------- */

typedef struct { double key; int32_t idx; } orc_item;

static int by_key_desc_idx_asc(const void* a, const void* b) {
    const orc_item* x = (const orc_item*)a;
    const orc_item* y = (const orc_item*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/* Scores s_i and selection keys kappa_i of one token from its logits. */
static void scores_and_keys(const orc_shape* s, const double* l, const float* bias, double* sc, double* key) {
    const int N = s->N_r;
    if (s->gating == 1) {
        for (int i = 0; i < N; ++i) {
            sc[i] = 1.0 / (1.0 + exp(-l[i]));
            key[i] = sc[i] + (bias ? (double)bias[i] : 0.0);
        }
    } else {
        double m = -INFINITY;
        for (int i = 0; i < N; ++i) m = l[i] > m ? l[i] : m;
        double z = 0.0;
        for (int i = 0; i < N; ++i) z += exp(l[i] - m);
        for (int i = 0; i < N; ++i) {
            sc[i] = exp(l[i] - m) / z;
            key[i] = sc[i];
        }
    }
}

/*
 * Selection of one token.  Writes sel[K_r] in (key desc, index asc) order and
 * the smallest key margin at any decision boundary the selection crossed
 * (+inf when no other choice was possible).
 */
static void select_token(const orc_shape* s, const double* key, int32_t* sel, double* gap_out) {
    const int N = s->N_r, K = s->K_r;
    double gap = INFINITY;
    orc_item* it = (orc_item*)malloc(sizeof(orc_item) * (size_t)(N > 0 ? N : 1));
    int ncand = 0;
    if (s->n_group) {
        const int G = s->n_group, per = N / G;
        orc_item* gi = (orc_item*)malloc(sizeof(orc_item) * (size_t)G);
        for (int g = 0; g < G; ++g) {
            double sum = 0.0;
            for (int j = 0; j < per; ++j) sum += key[g * per + j];
            gi[g].key = sum;
            gi[g].idx = g;
        }
        qsort(gi, (size_t)G, sizeof(orc_item), by_key_desc_idx_asc);
        if (s->topk_group < G) gap = gi[s->topk_group - 1].key - gi[s->topk_group].key;
        /* candidates: experts of the chosen groups */
        char* chosen = (char*)calloc((size_t)G, 1);
        for (int r = 0; r < s->topk_group; ++r) chosen[gi[r].idx] = 1;
        for (int i = 0; i < N; ++i)
            if (chosen[i / per]) { it[ncand].key = key[i]; it[ncand].idx = i; ++ncand; }
        free(chosen);
        free(gi);
        qsort(it, (size_t)ncand, sizeof(orc_item), by_key_desc_idx_asc);
        for (int k = 0; k < K; ++k) sel[k] = it[k].idx;
        if (K > 0 && K < ncand) {
            double g2 = it[K - 1].key - it[K].key;
            gap = g2 < gap ? g2 : gap;
        }
    } else {
        for (int i = 0; i < N; ++i) { it[i].key = key[i]; it[i].idx = i; }
        ncand = N;
        qsort(it, (size_t)N, sizeof(orc_item), by_key_desc_idx_asc);
        const int r = s->mask_top_r;
        for (int k = 0; k < K; ++k) sel[k] = it[r + k].idx;
        if (r > 0 && r < N) gap = it[r - 1].key - it[r].key;
        if (K > 0 && r + K < N) {
            double g2 = it[r + K - 1].key - it[r + K].key;
            gap = g2 < gap ? g2 : gap;
        }
    }
    free(it);
    *gap_out = gap;
}

/* Gate weights of the selected experts. */
static void weights(const orc_shape* s, const double* l, const double* sc, const int32_t* sel, double* g) {
    const int K = s->K_r;
    if (s->gating == 0) {
        for (int k = 0; k < K; ++k) g[k] = sc[sel[k]];
    } else if (s->gating == 1) {
        double z = 0.0;
        for (int k = 0; k < K; ++k) z += sc[sel[k]];
        for (int k = 0; k < K; ++k) g[k] = z > 0.0 ? sc[sel[k]] / z : 1.0 / K;
    } else {
        double m = -INFINITY;
        for (int k = 0; k < K; ++k) m = l[sel[k]] > m ? l[sel[k]] : m;
        double z = 0.0;
        for (int k = 0; k < K; ++k) z += exp(l[sel[k]] - m);
        for (int k = 0; k < K; ++k) g[k] = exp(l[sel[k]] - m) / z;
    }
}

static void logits_of(const orc_shape* s, const void* e, const double* x, double* l) {
    for (int i = 0; i < s->N_r; ++i) l[i] = dot(e, s->dtype, (size_t)i * s->H, x, s->H);
}

static void widen_row(const void* u, int dtype, size_t row, int H, double* x) {
    for (int h = 0; h < H; ++h) x[h] = ld(u, dtype, row * (size_t)H + h);
}

/*
 * Routing only, for the tokens listed in tok[0..ntok).  Outputs per listed
 * token: sel[K_r] (key desc, index asc), g[K_r], gap, and optionally the
 * logits and scores [N_r].
 */
int orc_route(const orc_shape* s, const void* u, const void* e, const float* bias,
              const int64_t* tok, int64_t ntok,
              int32_t* sel, double* g, double* gap, double* logits_out, double* scores_out) {
    if (check_shape(s) != ORC_OK) return ORC_BAD;
    if (bias && s->gating != 1) return ORC_BAD;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t j = 0; j < ntok; ++j) {
        if (tok[j] < 0 || tok[j] >= s->T) { bad |= 1; continue; }
        double* x = (double*)malloc(sizeof(double) * (size_t)s->H);
        double* l = (double*)malloc(sizeof(double) * (size_t)(s->N_r + 1));
        double* sc = (double*)malloc(sizeof(double) * (size_t)(s->N_r + 1));
        double* key = (double*)malloc(sizeof(double) * (size_t)(s->N_r + 1));
        widen_row(u, s->dtype, (size_t)tok[j], s->H, x);
        logits_of(s, e, x, l);
        scores_and_keys(s, l, bias, sc, key);
        select_token(s, key, sel + j * s->K_r, gap + j);
        weights(s, l, sc, sel + j * s->K_r, g + j * s->K_r);
        if (logits_out) memcpy(logits_out + j * s->N_r, l, sizeof(double) * (size_t)s->N_r);
        if (scores_out) memcpy(scores_out + j * s->N_r, sc, sizeof(double) * (size_t)s->N_r);
        free(x); free(l); free(sc); free(key);
    }
    return bad ? ORC_BAD : ORC_OK;
}

/*
 * One expert FFN on one fp64 vector x[H] -> y[H].
 * act 0: y = V ReLU(W x + b), W = w1 [I, H], b = b1 [I] (fp32, NULL = 0), V = w2 [H, I].
 * act 1: y = W2 (SiLU(Wg x) * (Wu x)), w1 = [Wg; Wu] [2I, H], w2 = W2 [H, I].
 */
int orc_expert_ffn(int32_t H, int32_t I, int32_t act, int32_t dtype,
                   const void* w1, const float* b1, const void* w2, const double* x, double* y) {
    if (H <= 0 || I <= 0 || (act != 0 && act != 1) || (dtype != 0 && dtype != 1)) return ORC_BAD;
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    for (int i = 0; i < I; ++i) {
        if (act == 0) {
            double z = dot(w1, dtype, (size_t)i * H, x, H) + (b1 ? (double)b1[i] : 0.0);
            a[i] = z > 0.0 ? z : 0.0;
        } else {
            double zg = dot(w1, dtype, (size_t)i * H, x, H);
            double zu = dot(w1, dtype, (size_t)(I + i) * H, x, H);
            a[i] = zg / (1.0 + exp(-zg)) * zu;
        }
    }
    for (int h = 0; h < H; ++h) y[h] = dot(w2, dtype, (size_t)h * I, a, I);
    free(a);
    return ORC_OK;
}

/*
 * Full layer for the listed tokens.
 *   out[j, :] = (residual ? u_t : 0) + sum_{j<Ks} FFN^sh_j(u_t) + sum_k g_k FFN_{sel_k}(u_t)
 * forced_sel [ntok, K_r] (optional) replaces the oracle's own selection; the
 * weights are then those the gating formula gives for the forced set.
 * Expert weight banks: w1 [N_r, n1, H], b1 [N_r, I] fp32 | NULL, w2 [N_r, H, I];
 * shared banks w1_sh [Ks, n1, H], b1_sh [Ks, I] | NULL, w2_sh [Ks, H, I].
 */
int orc_layer(const orc_shape* s, const void* u, const void* e, const float* bias,
              const void* w1, const float* b1, const void* w2,
              const void* w1_sh, const float* b1_sh, const void* w2_sh,
              const int64_t* tok, int64_t ntok, const int32_t* forced_sel, int32_t residual,
              double* out, int32_t* sel, double* g, double* gap) {
    if (check_shape(s) != ORC_OK) return ORC_BAD;
    if (bias && s->gating != 1) return ORC_BAD;
    if (s->Ks > 0 && (!w1_sh || !w2_sh)) return ORC_BAD;
    if (s->K_r > 0 && (!w1 || !w2 || !e)) return ORC_BAD;
    const int H = s->H, I = s->I, K = s->K_r;
    const size_t n1 = (size_t)(s->act == 1 ? 2 * I : I);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t j = 0; j < ntok; ++j) {
        if (tok[j] < 0 || tok[j] >= s->T) { bad |= 1; continue; }
        double* x = (double*)malloc(sizeof(double) * (size_t)H);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        double* acc = out + j * H;
        double* l = (double*)malloc(sizeof(double) * (size_t)(s->N_r + 1));
        double* sc = (double*)malloc(sizeof(double) * (size_t)(s->N_r + 1));
        double* key = (double*)malloc(sizeof(double) * (size_t)(s->N_r + 1));
        int32_t* sj = sel + j * K;
        double* gj = g + j * K;
        widen_row(u, s->dtype, (size_t)tok[j], H, x);
        if (K > 0) {
            logits_of(s, e, x, l);
            scores_and_keys(s, l, bias, sc, key);
            if (forced_sel) {
                memcpy(sj, forced_sel + j * K, sizeof(int32_t) * (size_t)K);
                gap[j] = NAN;
                for (int k = 0; k < K; ++k)
                    if (sj[k] < 0 || sj[k] >= s->N_r) bad |= 1;
            } else {
                select_token(s, key, sj, gap + j);
            }
            weights(s, l, sc, sj, gj);
        } else {
            gap[j] = INFINITY;
        }
        for (int h = 0; h < H; ++h) acc[h] = residual ? x[h] : 0.0;
        for (int js = 0; js < s->Ks; ++js) {
            const float* bb = b1_sh ? b1_sh + (size_t)js * I : NULL;
            if (s->dtype == 0) {
                orc_expert_ffn(H, I, s->act, 0, (const float*)w1_sh + (size_t)js * n1 * H, bb,
                               (const float*)w2_sh + (size_t)js * H * I, x, y);
            } else {
                orc_expert_ffn(H, I, s->act, 1, (const uint16_t*)w1_sh + (size_t)js * n1 * H, bb,
                               (const uint16_t*)w2_sh + (size_t)js * H * I, x, y);
            }
            for (int h = 0; h < H; ++h) acc[h] += y[h];
        }
        for (int k = 0; k < K && !bad; ++k) {
            const int ex = sj[k];
            const float* bb = b1 ? b1 + (size_t)ex * I : NULL;
            if (s->dtype == 0) {
                orc_expert_ffn(H, I, s->act, 0, (const float*)w1 + (size_t)ex * n1 * H, bb,
                               (const float*)w2 + (size_t)ex * H * I, x, y);
            } else {
                orc_expert_ffn(H, I, s->act, 1, (const uint16_t*)w1 + (size_t)ex * n1 * H, bb,
                               (const uint16_t*)w2 + (size_t)ex * H * I, x, y);
            }
            for (int h = 0; h < H; ++h) acc[h] += gj[k] * y[h];
        }
        free(x); free(y); free(l); free(sc); free(key);
    }
    return bad ? ORC_BAD : ORC_OK;
}

/*
 * Aux-loss-free balance controller (ibossgateway section 7.4): after a step,
 * an overloaded expert (load above the mean T*K_r/N_r) has b_i lowered by
 * gamma, an underloaded one raised by gamma, one exactly at the mean is kept.
 * The update is taken in fp64 and stored as fp32.
 */
int orc_bias_update(int32_t N_r, int64_t T, int32_t K_r, const int32_t* counts, float gamma,
                    const float* b_in, float* b_out) {
    if (N_r <= 0 || T < 0 || K_r < 0) return ORC_BAD;
    const int64_t total = T * (int64_t)K_r;
    for (int i = 0; i < N_r; ++i) {
        const int64_t lhs = (int64_t)counts[i] * N_r; /* load_i > total / N_r  <=>  load_i * N_r > total */
        double b = (double)b_in[i];
        if (lhs > total) b -= (double)gamma;
        else if (lhs < total) b += (double)gamma;
        b_out[i] = (float)b;
    }
    return ORC_OK;
}
