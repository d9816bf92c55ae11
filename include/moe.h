/*
 * moe.h - C ABI of libmoe, the MI355X (gfx950) DeepSeekMoE layer forward pass.
 *
 * The layer (llm-infra-atlas "02 Fine-grained MoE", section 3.1, DeepSeekMoE
 * Eq. 9-11):
 *
 *   h_t = sum_{j<Ks} FFN^shared_j(u_t) + sum_{i in TopK} g_{i,t} FFN_i(u_t) + u_t
 *
 * with fine-grained routed experts (same page, section 2.1: mN experts of
 * intermediate width M/m, top-mK; the API takes the routed count N_r and
 * routed top-k K_r directly) and Ks always-active shared experts.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are device memory owned by the caller, row-major, contiguous.
 *   The library never allocates or frees device memory: scratch space comes
 *   from the caller's workspace `ws` of `ws_bytes` bytes (see
 *   moe_workspace_size), or, for moe_layer_forward_noalloc, from a static
 *   device array the library holds.  Host pointers: only `shape` (and the
 *   out-params of moe_workspace_size / moe_profile_query).
 * - Process-wide state: the profiling counters of moe_profile_* (every other
 *   call only reads whether profiling is on), the last HIP error (per thread)
 *   and the static scratch of moe_layer_forward_noalloc.  None of it changes
 *   a result.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on that stream and returns; nothing is read back to the host
 *   and the host never waits.
 * - Errors: argument checks run on the host before any launch and return a
 *   negative moe_status with nothing enqueued.  A failed launch returns
 *   MOE_ERR_HIP (moe_last_hip_error() gives the hipError_t).  No exception
 *   crosses this interface.
 * - dtype (MOE_F32 or MOE_BF16) applies to u, centroids, expert weights,
 *   intermediate rows and out.  Gate weights, the selection bias and the ReLU
 *   bias b1 are always fp32; indices and offsets are int32.
 * - Expert weights are stored [out, in] (nn.Linear layout):
 *     SwiGLU: w1 [G, 2I, H] with the gate rows [0, I) before the up rows
 *             [I, 2I); w2 [G, H, I].  FFN(x) = w2 (SiLU(w1_gate x) * (w1_up x)).
 *     ReLU:   w1 [G, I, H], b1 [G, I] fp32, w2 [G, H, I].
 *             FFN(x) = w2 ReLU(w1 x + b1)  (tomabc DeepSeekMoE explainer:
 *             a = ReLU(x W_i + b_i), output a V_i).
 * - Preconditions: T >= 0, 0 <= K_r <= N_r <= 1024, Ks >= 0, H % 64 == 0,
 *   I % 64 == 0, H >= 64, I >= 64.  Inputs must be finite.
 *   Calls on one stream are ordered; calls that share a workspace must not
 *   overlap in time on different streams.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* a pointer, size or enum is out of contract */
    MOE_ERR_UNSUPPORTED = -2, /* a valid shape this build does not cover (e.g. N_r > 1024) */
    MOE_ERR_WORKSPACE = -3,   /* ws is NULL or smaller than moe_workspace_size() */
    MOE_ERR_HIP = -4,         /* a HIP launch or event call failed */
    MOE_ERR_SCRATCH = -5      /* moe_layer_forward_noalloc: the shape needs more scratch than the
                                 library's static buffer (moe_noalloc_scratch_bytes()) holds */
} moe_status;

/* Gating (scores and gate weights of the routed experts). */
enum {
    /* llm-infra-atlas 02, section 2.1, DeepSeekMoE Eq. 7-8:
       s = softmax over the N_r routed logits; g = s on the top-K_r, no renormalisation. */
    MOE_GATE_SOFTMAX = 0,
    /* llm-infra-atlas 02, section 3.1, DeepSeek-V3 Eq. 12-15, with the selection-only bias of
       ibossgateway chapter 7, section 7.4: s = sigmoid(l); rank s + b; g = s / sum of selected s. */
    MOE_GATE_SIGMOID_BIAS_NORM = 1,
    /* tomabc DeepSeekMoE explainer, fine-grained section: non-top scores set to -inf before the
       softmax, i.e. g = softmax over the selected logits (sums to 1). */
    MOE_GATE_SOFTMAX_RENORM = 2
};

enum { MOE_ACT_RELU_BIAS = 0, MOE_ACT_SWIGLU = 1 };
enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* moe_layer_forward flags */
enum {
    MOE_FLAG_NO_RESIDUAL = 1,      /* drop the + u_t term: returns the MoE part only */
    MOE_FLAG_PACKED_WEIGHTS = 2,   /* routed banks w1, w2 are in fragment order (moe_pack_weights) */
    MOE_FLAG_PACKED_SHARED_UP = 4  /* the shared up bank w1_sh is in fragment order (moe_pack_weights) */
};

typedef struct moe_shape {
    int32_t T;          /* tokens */
    int32_t H;          /* hidden size */
    int32_t N_r;        /* routed experts (mN, or mN - Ks in Eq. 9-11) */
    int32_t K_r;        /* routed experts per token (mK, or mK - Ks) */
    int32_t Ks;         /* shared experts, always active with weight 1 */
    int32_t I;          /* intermediate width of every expert (M/m) */
    int32_t gating;     /* MOE_GATE_* */
    int32_t act;        /* MOE_ACT_* */
    int32_t dtype;      /* MOE_F32 | MOE_BF16 */
    /* Group-limited routing (llm-infra-atlas 02, section 4, node-limited routing): experts are
       split into n_group contiguous groups of N_r / n_group; each group's score is the sum of
       its experts' selection keys; the topk_group best groups are kept and the top-K_r experts
       are chosen inside them.  n_group = 0 turns it off. */
    int32_t n_group;
    int32_t topk_group;
    /* Masking probe (llm-infra-atlas 02, section 1, Fig. 4): drop each token's mask_top_r
       highest-ranked routed experts, then select the top-K_r of the rest.  0 = off. */
    int32_t mask_top_r;
} moe_shape;

/* Bytes of device workspace every entry point below needs for `shape` (the maximum over
   them).  Returns MOE_OK and writes *bytes, or a negative status for an invalid shape. */
int moe_workspace_size(const moe_shape* shape, size_t* bytes);

/*
 * Router: logits l[t,i] = u_t . e_i (llm-infra-atlas 02, Eq. 8), scores, top-K_r selection
 * and gate weights per the gating mode (see MOE_GATE_*).  Ties in the ranking go to the lower
 * expert index; in softmax modes the ranking uses the logits (softmax is monotone).
 *   u          [T, H]      dtype
 *   centroids  [N_r, H]    dtype
 *   bias       [N_r] fp32  selection bias, MOE_GATE_SIGMOID_BIAS_NORM only (NULL = 0);
 *                          non-NULL in any other mode -> MOE_ERR_INVALID_ARG
 *   topk_idx   [T, K_r] int32 out: selected experts, descending key
 *   topk_w     [T, K_r] fp32  out: their gate weights
 */
int moe_route(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
              int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream);

/*
 * Dispatch (llm-infra-atlas 02, section 4: no token dropping, so every selected pair is kept):
 * a histogram of topk_idx, its exclusive prefix sum and a stable scatter into contiguous
 * per-expert segments, ordered by (token, slot) inside each segment.
 *   topk_idx   [T, K_r]  int32 in: entries in [0, N_r), distinct per token (entries outside
 *                        the range are skipped; results are then undefined but no access
 *                        leaves the buffers)
 *   offsets    [N_r + 1] int32 out: segment e is rows [offsets[e], offsets[e+1])
 *   row_token  [T*K_r]   int32 out: token of each permuted row
 *   pair_row   [T*K_r]   int32 out: permuted row of pair (t, k), index t*K_r + k
 *   u, x_perm  optional (both or neither): x_perm [T*K_r, H] dtype receives u[row_token[r]]
 */
int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, int32_t* offsets, int32_t* row_token,
                 int32_t* pair_row, const void* u, void* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * Routed expert FFNs as one grouped GEMM pair over the N_r segments of the permuted rows.
 * Row r (0 <= r < T*K_r) of segment e computes y[r] = FFN_e(x[row_token[r]]) when row_token is
 * not NULL (fused gather from u), else y[r] = FFN_e(x[r]) (x = x_perm).
 *   x          [T, H] (with row_token) or [T*K_r, H]   dtype
 *   offsets    [N_r + 1] int32 (device; as moe_dispatch writes it, offsets[N_r] == T*K_r)
 *   w1, b1, w2 routed banks with G = N_r (b1 only for ReLU, NULL = 0)
 *   y          [T*K_r, H] dtype out
 */
int moe_expert_ffn(const moe_shape* shape, const void* x, const int32_t* row_token, const int32_t* offsets,
                   const void* w1, const float* b1, const void* w2, void* y, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * Weight repacking for the routed experts (a storage layout of the same FFN weights; the result of
 * every FFN is bit-identical to the one computed from the [out, in] banks).  Expert weights are
 * static, so they can be stored once in the order in which the matrix cores read them: G bf16
 * matrices [N, K] (row-major) become, per matrix, (N / 32) * (K / 16) blocks of 1 KB; block
 * nb * (K / 16) + kc holds rows 32 nb .. 32 nb + 31 and columns 16 kc .. 16 kc + 15, and its
 * 16-byte piece l (0 <= l < 64) holds row 32 nb + l % 32, columns 16 kc + 8 (l / 32) .. + 7.
 * `packed` has the size of `w` (G*N*K*2 bytes) and must not overlap it; both 16-byte aligned.
 * N % 32 == 0 and K % 64 == 0 (else MOE_ERR_INVALID_ARG); N*K*2 < 2^31 (else MOE_ERR_UNSUPPORTED).
 * Routed banks: w1 with (G, N, K) = (N_r, 2I, H) (SwiGLU) or (N_r, I, H) (ReLU), w2 with (N_r, H, I).
 * Enqueued on `stream` like every call; pack once when the weights are loaded.
 */
int moe_pack_weights(const void* w, void* packed, int32_t G, int32_t N, int32_t K, void* stream);

/*
 * moe_expert_ffn with w1 and w2 in the packed order of moe_pack_weights (bf16 only; fp32 ->
 * MOE_ERR_INVALID_ARG).  Same arguments, same results bit for bit.
 */
int moe_expert_ffn_packed(const moe_shape* shape, const void* x, const int32_t* row_token,
                          const int32_t* offsets, const void* w1, const float* b1, const void* w2, void* y,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Shared experts (DeepSeekMoE Eq. 9, first term): y[t] = sum_{j<Ks} FFN^shared_j(x[t]) for all
 * T tokens, computed as one FFN of width Ks*I (the Ks experts' intermediate rows side by side).
 *   x [T, H]; w1_sh, b1_sh, w2_sh banks with G = Ks; y [T, H] dtype out.  Ks == 0 -> MOE_OK, no work.
 */
int moe_shared_ffn(const moe_shape* shape, const void* x, const void* w1_sh, const float* b1_sh,
                   const void* w2_sh, void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Combine (DeepSeekMoE Eq. 9): out[t] = residual[t] + y_shared[t] + sum_k topk_w[t,k] *
 * y_perm[pair_row[t*K_r+k]], accumulated in fp32 in that order (k ascending), then stored.
 *   residual, y_shared [T, H] or NULL (term omitted); y_perm [T*K_r, H]; out [T, H] dtype.
 */
int moe_combine(const moe_shape* shape, const void* residual, const void* y_shared, const void* y_perm,
                const int32_t* pair_row, const float* topk_w, void* out, void* stream);

/*
 * The whole layer: route -> dispatch -> routed FFNs + shared FFNs -> combine + residual.
 *   u [T, H]; centroids [N_r, H]; bias [N_r] | NULL; routed banks (G = N_r); shared banks
 *   (G = Ks, NULL when Ks == 0); flags: MOE_FLAG_*; out [T, H] dtype.
 *   MOE_FLAG_PACKED_WEIGHTS: w1 and w2 (routed) are packed by moe_pack_weights (bf16 only).
 *   MOE_FLAG_PACKED_SHARED_UP: w1_sh (the shared experts' gate/up bank, [Ks, n1, H]) is packed by
 *   moe_pack_weights (bf16 only); w2_sh stays [out, in] (its GEMM also performs the combine).
 *   Either way the output is bit-identical to the unpacked call.
 *   topk_idx_out [T, K_r], topk_w_out [T, K_r]: optional copies of the routing (NULL = none).
 */
int moe_layer_forward(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                      const void* w1, const float* b1, const void* w2,
                      const void* w1_sh, const float* b1_sh, const void* w2_sh,
                      int32_t flags, void* out, int32_t* topk_idx_out, float* topk_w_out,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward for callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same arguments and results
 * as moe_layer_forward (bit for bit) without ws / ws_bytes: the scratch is a static device array of
 * moe_noalloc_scratch_bytes() = 64 MiB that the library holds on each GPU it runs on until the process
 * ends (the V3-style decode step, T = 128, needs about 21 MB).  The array of the current device is used
 * (make the stream's device current, as for any HIP call).  Calls no allocating routine.
 *   - A shape whose moe_workspace_size exceeds that size -> MOE_ERR_SCRATCH, nothing enqueued.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents; every
 *     kernel writes the scratch it later reads, so nothing needs clearing.  Calls that overlap in time
 *     on one GPU (different streams, or threads without ordering) race on it: serialise them.
 */
int moe_layer_forward_noalloc(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                              const void* w1, const float* b1, const void* w2,
                              const void* w1_sh, const float* b1_sh, const void* w2_sh,
                              int32_t flags, void* out, int32_t* topk_idx_out, float* topk_w_out, void* stream);

/* Bytes of the static scratch array of moe_layer_forward_noalloc. */
size_t moe_noalloc_scratch_bytes(void);

/*
 * Aux-loss-free balance controller (ibossgateway chapter 7, section 7.4; llm-infra-atlas 02,
 * section 5): from the dispatch offsets, counts[e] = load of expert e, and
 * bias[e] -= gamma if load > T*K_r/N_r, += gamma if below, unchanged at the mean (fp32, in place).
 *   offsets [N_r + 1] int32; bias [N_r] fp32 in/out; counts [N_r] int32 out (NULL = not stored).
 */
int moe_bias_update(const moe_shape* shape, const int32_t* offsets, float gamma, float* bias,
                    int32_t* counts, void* stream);

/* Text for a moe_status value. */
const char* moe_status_string(int status);

/* The hipError_t of the last failed HIP call in this thread (0 = none). */
int moe_last_hip_error(void);

/*
 * Per-kernel timing with HIP events recorded on the launch stream around every kernel the
 * library launches (for measurement; adds a little launch overhead).  moe_profile_enable(1)
 * clears the counters and starts recording, (0) stops.  moe_profile_query waits for the
 * recorded events and returns the launch count and summed duration of kernel class `kernel`
 * (MOE_PROF_*).  Not thread-safe; one recording at a time per process.
 */
enum {
    MOE_PROF_ROUTER = 0, MOE_PROF_DISPATCH = 1, MOE_PROF_FFN_UP = 2, MOE_PROF_FFN_DOWN = 3,
    MOE_PROF_SHARED_UP = 4, MOE_PROF_SHARED_DOWN = 5, MOE_PROF_COMBINE = 6, MOE_PROF_OTHER = 7,
    MOE_PROF_COUNT = 8
};
int moe_profile_enable(int32_t on);
int moe_profile_query(int32_t kernel, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
