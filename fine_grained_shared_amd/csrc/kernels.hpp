// Host-side launchers of the libmoe kernels (internal; the public ABI is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- router
// logits = u [T, H] . centroids [N, H]^T in fp32: [T, N] (fp32), or for bf16 the logits_groups(H)
// partial sums of the fixed summation order side by side, [T, G N]; the selection adds them
hipError_t launch_logits(int dtype, const void* u, const void* e, float* logits, int T, int H, int N,
                         hipStream_t s);
int logits_groups(int H);
// per-token scores, selection and gate weights from the logits
struct SelectArgs {
    const float* logits;      // [T, groups N]
    int groups;               // 1, 2 or 4 partial sums per logit, added in group order
    const float* bias;
    int T, N, K;
    int gating;
    int n_group, topk_group, mask_r;
    int32_t* topk_idx;
    float* topk_w;
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

// ---------------------------------------------------------------- dispatch
constexpr int kChunk = 256;  // tokens per dispatch workgroup
hipError_t launch_count(const int32_t* idx, int T, int K, int N, int32_t* chunk_counts, hipStream_t s);
// counts [nchunk, N] -> bases [nchunk, N] (absolute start of chunk c's rows of expert e) and offsets [N + 1]
hipError_t launch_scan(const int32_t* chunk_counts, int32_t* chunk_base, int nchunk, int N, int32_t* offsets,
                       hipStream_t s);
hipError_t launch_scatter(const int32_t* idx, int T, int K, int N, const int32_t* chunk_base,
                          int32_t* row_token, int32_t* pair_row, hipStream_t s);
// all of the above for one chunk (1 <= T <= kChunk, K >= 1) in one launch
hipError_t launch_dispatch1(const int32_t* idx, int T, int K, int N, int32_t* offsets, int32_t* row_token,
                            int32_t* pair_row, hipStream_t s);
// x_perm [R, H] = u [T, H] rows row_token[r], each index clamped into [0, T)
hipError_t launch_gather(int dtype, const void* u, const int32_t* row_token, int T, int R, int H, void* x_perm,
                         hipStream_t s);

// ---------------------------------------------------------------- expert FFN (grouped GEMM)
// GM_DOWN_COMBINE: the shared experts' down GEMM whose epilogue also adds the residual and the
// gate-weighted routed rows (Eq. 9) and writes the layer output.
// GM_F32OUT: plain product stored in fp32 (router logits).
enum { GM_UP_SWIGLU = 0, GM_UP_RELU = 1, GM_DOWN = 2, GM_DOWN_COMBINE = 3, GM_F32OUT = 4 };

struct GemmParams {
    const void* A;            // activation rows
    long long lda;            // elements per A row
    const int32_t* a_rows;    // row-space row -> A row (NULL: identity)
    long long sA_group;       // dense mode: group g reads A + g * sA_group (split reduction; else 0)
    long long a_nrows;        // rows of A (gathered indices are clamped into range)
    const void* B;            // weight bank base
    long long sB_group;       // elements between groups in the bank
    long long ldb;            // elements per weight row
    int K;                    // reduction length
    int Kseg;                 // reduction segment length; segment q reads B + q * sB_seg
    long long sB_seg;
    int N;                    // output columns
    int up_off;               // SwiGLU: first up row inside a group's w1 (= I)
    const int32_t* offsets;   // grouped mode: [G+1] row-space segments (NULL: dense mode)
    const int32_t* tiles;     // grouped mode: [G+1] prefix of m-tiles per group
    const int32_t* tiles32;   // grouped mode: [G+1] prefix of 32-row m-tiles per group (decode kernel)
    int M_dense;              // dense mode: every group covers rows [0, M_dense)
    int G;
    int max_rows;             // upper bound of the row space (grid sizing)
    void* C;                  // output
    long long ldc;
    long long sC_group;       // dense mode: column offset of group g in C is g * sC_group
    const float* bias;        // ReLU bias [G, N] (NULL = 0)
    long long sbias_group;
    // GM_DOWN_COMBINE only: out[t] = resid[t] + C_acc[t] + sum_k topk_w[t,k] * y_perm[pair_row[t,k]]
    const void* resid;        // [M_dense, N] or NULL
    const void* y_perm;       // [R, N]
    const int32_t* pair_row;  // [M_dense, K_r]
    const float* topk_w;      // [M_dense, K_r]
    int K_r;
    long long R;
    // set by launch_gemm: byte spans of A and of one group's weights when both are below 2^31
    // (kernels addressing them with 32-bit buffer offsets are chosen only then), else 0
    int a_bytes;
    int b_bytes;
    // weights in MFMA fragment order (launch_pack_b); grouped bf16 up/down GEMMs with one K segment only
    int packed;
};
// m-tile prefixes of the groups defined by offsets (grouped mode): tiles[0..G] for tiles of bm rows,
// tiles[G+1 .. 2G+1] for tiles of 32 rows.
constexpr int kTilePlans = 2;
hipError_t launch_tile_plan(const int32_t* offsets, int G, int bm, int32_t* tiles, hipStream_t s);
int gemm_bm(int dtype);
hipError_t launch_gemm(int dtype, int mode, const GemmParams& p, hipStream_t s);
// G bf16 matrices [N, K] -> fragment order: 1 KB block nb * (K / 16) + kc holds rows 32 nb .. + 31,
// columns 16 kc .. + 15, 16-byte piece l = row 32 nb + l % 32, columns 16 kc + 8 (l / 32) .. + 7
hipError_t launch_pack_b(const void* w, void* out, int G, int N, int K, hipStream_t s);

// ---------------------------------------------------------------- combine, controller
hipError_t launch_combine(int dtype, const void* residual, const void* y_shared, const void* y_perm,
                          const int32_t* pair_row, const float* topk_w, void* out, int T, int H, int K,
                          hipStream_t s);
hipError_t launch_bias_update(const int32_t* offsets, int N, long long T, int K, float gamma, float* bias,
                              int32_t* counts, hipStream_t s);

}  // namespace moe
