// C ABI of libmoe (declared in include/moe.h): argument checks, workspace carving, launches.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

// ---------------------------------------------------------------- kernel timing
struct Prof {
    bool on = false;
    std::vector<hipEvent_t> ev;  // pairs
    std::vector<int> cls;
    size_t used = 0;
};
Prof g_prof;
constexpr size_t kProfPairs = 8192;

struct ProfScope {
    bool rec = false;
    hipEvent_t b = nullptr;
    hipStream_t s;
    ProfScope(int c, hipStream_t st) : s(st) {
        if (!g_prof.on || g_prof.used >= kProfPairs) return;
        const size_t i = g_prof.used++;
        g_prof.cls[i] = c;
        rec = hipEventRecord(g_prof.ev[2 * i], s) == hipSuccess;
        b = g_prof.ev[2 * i + 1];
    }
    ~ProfScope() {
        if (rec) (void)hipEventRecord(b, s);
    }
};

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return MOE_ERR_HIP;
}
#define MOE_TRY(cls, stream, expr)                     \
    do {                                               \
        hipError_t e_;                                 \
        {                                              \
            ProfScope ps_(cls, stream);                \
            e_ = (expr);                               \
        }                                              \
        if (e_ != hipSuccess) return hip_fail(e_);     \
    } while (0)

// ---------------------------------------------------------------- validation
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const moe_shape* s) {
    if (!s) return MOE_ERR_INVALID_ARG;
    if (s->T < 0 || s->H <= 0 || s->N_r < 0 || s->K_r < 0 || s->Ks < 0 || s->I <= 0) return MOE_ERR_INVALID_ARG;
    if (s->K_r > s->N_r) return MOE_ERR_INVALID_ARG;
    if (s->gating < 0 || s->gating > 2 || s->act < 0 || s->act > 1 || s->dtype < 0 || s->dtype > 1)
        return MOE_ERR_INVALID_ARG;
    if (s->H % 64 || s->I % 64) return MOE_ERR_INVALID_ARG;
    if (s->n_group < 0 || s->mask_top_r < 0 || s->mask_top_r + s->K_r > s->N_r) return MOE_ERR_INVALID_ARG;
    if (s->n_group > 0) {
        if (s->N_r % s->n_group || s->topk_group <= 0 || s->topk_group > s->n_group) return MOE_ERR_INVALID_ARG;
        if ((long long)s->topk_group * (s->N_r / s->n_group) < s->K_r) return MOE_ERR_INVALID_ARG;
        if (s->mask_top_r) return MOE_ERR_INVALID_ARG;
    }
    if (s->N_r > 1024 || s->K_r > 64 || s->n_group > 64) return MOE_ERR_UNSUPPORTED;
    if ((long long)s->T * (s->K_r > 0 ? s->K_r : 1) > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

size_t esz(const moe_shape* s) { return s->dtype == MOE_F32 ? 4 : 2; }

// Routed banks in fragment order: bf16 only, and each expert's matrix addressed with 32-bit offsets.
constexpr long long kPackedMatrixMaxBytes = 0x7FFFFFF0LL;
int check_packed(const moe_shape* s) {
    if (s->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    const long long n1 = s->act == MOE_ACT_SWIGLU ? 2LL * s->I : (long long)s->I;
    if (n1 * s->H * 2 > kPackedMatrixMaxBytes) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Workspace regions (byte offsets, each 256-byte aligned).
struct Layout {
    size_t logits, topk_idx, topk_w, offsets, row_token, pair_row, chunks, tiles, act, y_perm, act_sh, y_sh, total;
};

Layout layout_of(const moe_shape* s) {
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += (bytes + 255) / 256 * 256;
        return at;
    };
    const size_t T = (size_t)s->T, R = (size_t)s->T * s->K_r, E = esz(s);
    const size_t nchunk = (T + moe::kChunk - 1) / moe::kChunk;
    L.logits = take(T * s->N_r * 4 * (s->dtype == MOE_BF16 ? moe::logits_groups(s->H) : 1));
    L.topk_idx = take(R * 4);
    L.topk_w = take(R * 4);
    L.offsets = take(((size_t)s->N_r + 1) * 4);
    L.row_token = take(R * 4);
    L.pair_row = take(R * 4);
    L.chunks = take(2 * nchunk * s->N_r * 4);   // per-chunk counts, then the segment bases
    L.tiles = take(moe::kTilePlans * ((size_t)s->N_r + 1) * 4);
    L.act = take(R * s->I * E);
    L.y_perm = take(R * s->H * E);
    L.act_sh = take(T * s->Ks * s->I * E);
    L.y_sh = take(T * s->H * E);
    L.total = o;
    return L;
}

template <typename P>
P* at(void* ws, size_t off) {
    return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int check_ws(const moe_shape* s, void* ws, size_t ws_bytes) {
    const Layout L = layout_of(s);
    if (L.total > 0 && (!ws || ws_bytes < L.total || !aligned16(ws))) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// ---------------------------------------------------------------- steps
int do_route(const moe_shape* s, const void* u, const void* e, const float* bias, int32_t* idx, float* w,
             float* logits, hipStream_t st) {
    if (s->T == 0 || s->K_r == 0) return MOE_OK;
    const int groups = s->dtype == MOE_BF16 ? moe::logits_groups(s->H) : 1;
    moe::SelectArgs a{logits, groups, bias, s->T, s->N_r, s->K_r, s->gating, s->n_group, s->topk_group,
                      s->mask_top_r, idx, w};
    MOE_TRY(MOE_PROF_ROUTER, st, moe::launch_logits(s->dtype, u, e, logits, s->T, s->H, s->N_r, st));
    MOE_TRY(MOE_PROF_ROUTER, st, moe::launch_select(a, st));
    return MOE_OK;
}

int do_dispatch(const moe_shape* s, const int32_t* idx, int32_t* offsets, int32_t* row_token, int32_t* pair_row,
                int32_t* chunks, hipStream_t st) {
    const int nchunk = (s->T + moe::kChunk - 1) / moe::kChunk;
    if (nchunk == 1 && s->K_r > 0) {   // a decode step: one launch
        MOE_TRY(MOE_PROF_DISPATCH, st,
                moe::launch_dispatch1(idx, s->T, s->K_r, s->N_r, offsets, row_token, pair_row, st));
        return MOE_OK;
    }
    MOE_TRY(MOE_PROF_DISPATCH, st, moe::launch_count(idx, s->T, s->K_r, s->N_r, chunks, st));
    int32_t* bases = chunks + (size_t)nchunk * s->N_r;
    MOE_TRY(MOE_PROF_DISPATCH, st,
            moe::launch_scan(chunks, bases, s->K_r > 0 ? nchunk : 0, s->N_r, offsets, st));
    MOE_TRY(MOE_PROF_DISPATCH, st, moe::launch_scatter(idx, s->T, s->K_r, s->N_r, bases, row_token, pair_row, st));
    return MOE_OK;
}

int do_expert_ffn(const moe_shape* s, const void* x, const int32_t* row_token, const int32_t* offsets,
                  const void* w1, const float* b1, const void* w2, void* y, int32_t* tiles, void* act,
                  hipStream_t st, bool packed) {
    const long long R = (long long)s->T * s->K_r;
    if (R == 0 || s->N_r == 0) return MOE_OK;
    const int n1 = s->act == MOE_ACT_SWIGLU ? 2 * s->I : s->I;
    if (s->dtype == MOE_BF16)
        MOE_TRY(MOE_PROF_OTHER, st, moe::launch_tile_plan(offsets, s->N_r, moe::gemm_bm(s->dtype), tiles, st));
    moe::GemmParams up{};
    up.A = x;
    up.lda = s->H;
    up.a_rows = row_token;
    up.a_nrows = row_token ? s->T : R;
    up.B = w1;
    up.sB_group = (long long)n1 * s->H;
    up.ldb = s->H;
    up.K = s->H;
    up.Kseg = s->H;
    up.sB_seg = 0;
    up.N = s->I;
    up.up_off = s->I;
    up.offsets = offsets;
    up.tiles = tiles;
    up.tiles32 = tiles + (s->N_r + 1);
    up.G = s->N_r;
    up.max_rows = (int)R;
    up.C = act;
    up.ldc = s->I;
    up.bias = b1;
    up.sbias_group = s->I;
    up.packed = packed;
    const int up_mode = s->act == MOE_ACT_SWIGLU ? moe::GM_UP_SWIGLU : moe::GM_UP_RELU;
    MOE_TRY(MOE_PROF_FFN_UP, st, moe::launch_gemm(s->dtype, up_mode, up, st));
    moe::GemmParams dn{};
    dn.A = act;
    dn.lda = s->I;
    dn.a_rows = nullptr;
    dn.a_nrows = R;
    dn.B = w2;
    dn.sB_group = (long long)s->H * s->I;
    dn.ldb = s->I;
    dn.K = s->I;
    dn.Kseg = s->I;
    dn.N = s->H;
    dn.offsets = offsets;
    dn.tiles = tiles;
    dn.tiles32 = tiles + (s->N_r + 1);
    dn.G = s->N_r;
    dn.max_rows = (int)R;
    dn.C = y;
    dn.ldc = s->H;
    dn.packed = packed;
    MOE_TRY(MOE_PROF_FFN_DOWN, st, moe::launch_gemm(s->dtype, moe::GM_DOWN, dn, st));
    return MOE_OK;
}

// Shared experts.  With `comb` (bf16 only) the down GEMM's epilogue also adds the residual and the
// gate-weighted routed rows and writes the layer output to y.
struct Combine {
    const void* resid;
    const void* y_perm;
    const int32_t* pair_row;
    const float* topk_w;
};

int do_shared_ffn(const moe_shape* s, const void* x, const void* w1, const float* b1, const void* w2, void* y,
                  void* act, hipStream_t st, const Combine* comb = nullptr, bool packed_up = false) {
    if (s->T == 0 || s->Ks == 0) return MOE_OK;
    const int n1 = s->act == MOE_ACT_SWIGLU ? 2 * s->I : s->I;
    moe::GemmParams up{};
    up.A = x;
    up.lda = s->H;
    up.a_nrows = s->T;
    up.B = w1;
    up.sB_group = (long long)n1 * s->H;
    up.ldb = s->H;
    up.K = s->H;
    up.Kseg = s->H;
    up.N = s->I;
    up.up_off = s->I;
    up.M_dense = s->T;
    up.G = s->Ks;
    up.max_rows = s->T;
    up.C = act;
    up.ldc = (long long)s->Ks * s->I;
    up.sC_group = s->I;
    up.bias = b1;
    up.sbias_group = s->I;
    up.packed = packed_up;
    const int up_mode = s->act == MOE_ACT_SWIGLU ? moe::GM_UP_SWIGLU : moe::GM_UP_RELU;
    MOE_TRY(MOE_PROF_SHARED_UP, st, moe::launch_gemm(s->dtype, up_mode, up, st));
    // down: one GEMM whose reduction runs over the Ks intermediates side by side
    moe::GemmParams dn{};
    dn.A = act;
    dn.lda = (long long)s->Ks * s->I;
    dn.a_nrows = s->T;
    dn.B = w2;
    dn.sB_group = 0;
    dn.ldb = s->I;
    dn.K = s->Ks * s->I;
    dn.Kseg = s->I;
    dn.sB_seg = (long long)s->H * s->I;
    dn.N = s->H;
    dn.M_dense = s->T;
    dn.G = 1;
    dn.max_rows = s->T;
    dn.C = y;
    dn.ldc = s->H;
    if (comb) {
        dn.resid = comb->resid;
        dn.y_perm = comb->y_perm;
        dn.pair_row = comb->pair_row;
        dn.topk_w = comb->topk_w;
        dn.K_r = s->K_r;
        dn.R = (long long)s->T * s->K_r;
    }
    MOE_TRY(MOE_PROF_SHARED_DOWN, st,
            moe::launch_gemm(s->dtype, comb ? moe::GM_DOWN_COMBINE : moe::GM_DOWN, dn, st));
    return MOE_OK;
}

int layer_forward(const moe_shape* s, const void* u, const void* centroids, const float* bias, const void* w1,
                  const float* b1, const void* w2, const void* w1_sh, const float* b1_sh, const void* w2_sh,
                  int32_t flags, void* out, int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                  void* stream);

// ---------------------------------------------------------------- library-held scratch
// moe_layer_forward_noalloc takes its workspace from this array instead of a caller's buffer.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code never uses the array's name
// as an address (on the host it is a stand-in, not device memory): the device address is looked up once
// per device with hipGetSymbolAddress, with that device current, and kept in g_scratch.  Every kernel
// writes the workspace regions it later reads (nothing has to start at zero), so the array is never
// cleared; calls that overlap in time on one GPU share it and race.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(void** ptr) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (r != hipSuccess) return hip_fail(r);
            if (!p || ((uintptr_t)p & 255u)) return MOE_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_workspace_size(const moe_shape* shape, size_t* bytes) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = layout_of(shape).total;
    return MOE_OK;
}

int moe_route(const moe_shape* s, const void* u, const void* centroids, const float* bias, int32_t* topk_idx,
              float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (bias && s->gating != MOE_GATE_SIGMOID_BIAS_NORM) return MOE_ERR_INVALID_ARG;
    if (s->T == 0 || s->K_r == 0) return MOE_OK;
    if (!u || !centroids || !topk_idx || !topk_w || !aligned16(u) || !aligned16(centroids))
        return MOE_ERR_INVALID_ARG;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout_of(s);
    return do_route(s, u, centroids, bias, topk_idx, topk_w, at<float>(ws, L.logits), (hipStream_t)stream);
}

int moe_dispatch(const moe_shape* s, const int32_t* topk_idx, int32_t* offsets, int32_t* row_token,
                 int32_t* pair_row, const void* u, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (!offsets) return MOE_ERR_INVALID_ARG;
    const long long R = (long long)s->T * s->K_r;
    if (R > 0 && (!topk_idx || !row_token || !pair_row)) return MOE_ERR_INVALID_ARG;
    if ((u == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARG;
    if (x_perm && (!aligned16(u) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout_of(s);
    hipStream_t st = (hipStream_t)stream;
    rc = do_dispatch(s, topk_idx, offsets, row_token, pair_row, at<int32_t>(ws, L.chunks), st);
    if (rc != MOE_OK) return rc;
    if (x_perm) MOE_TRY(MOE_PROF_DISPATCH, st, moe::launch_gather(s->dtype, u, row_token, s->T, (int)R, s->H, x_perm, st));
    return MOE_OK;
}

static int expert_ffn(const moe_shape* s, const void* x, const int32_t* row_token, const int32_t* offsets,
                      const void* w1, const float* b1, const void* w2, void* y, void* ws, size_t ws_bytes,
                      void* stream, bool packed) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    const long long R = (long long)s->T * s->K_r;
    if (R == 0) return MOE_OK;
    if (!x || !offsets || !w1 || !w2 || !y) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
    if (b1 && s->act != MOE_ACT_RELU_BIAS) return MOE_ERR_INVALID_ARG;
    if (packed && (rc = check_packed(s)) != MOE_OK) return rc;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout_of(s);
    return do_expert_ffn(s, x, row_token, offsets, w1, b1, w2, y, at<int32_t>(ws, L.tiles), at<void>(ws, L.act),
                         (hipStream_t)stream, packed);
}

int moe_expert_ffn(const moe_shape* s, const void* x, const int32_t* row_token, const int32_t* offsets,
                   const void* w1, const float* b1, const void* w2, void* y, void* ws, size_t ws_bytes,
                   void* stream) {
    return expert_ffn(s, x, row_token, offsets, w1, b1, w2, y, ws, ws_bytes, stream, false);
}

int moe_expert_ffn_packed(const moe_shape* s, const void* x, const int32_t* row_token, const int32_t* offsets,
                          const void* w1, const float* b1, const void* w2, void* y, void* ws, size_t ws_bytes,
                          void* stream) {
    return expert_ffn(s, x, row_token, offsets, w1, b1, w2, y, ws, ws_bytes, stream, true);
}

int moe_pack_weights(const void* w, void* packed, int32_t G, int32_t N, int32_t K, void* stream) {
    if (G < 0 || N <= 0 || K <= 0 || N % 32 || K % 64) return MOE_ERR_INVALID_ARG;
    if ((long long)N * K * 2 > kPackedMatrixMaxBytes) return MOE_ERR_UNSUPPORTED;
    if (G == 0) return MOE_OK;
    if (!w || !packed || !aligned16(w) || !aligned16(packed)) return MOE_ERR_INVALID_ARG;
    const uintptr_t bytes = (uintptr_t)G * (uintptr_t)N * (uintptr_t)K * 2u;
    const uintptr_t a = (uintptr_t)w, b = (uintptr_t)packed;
    if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;   // overlapping buffers
    hipStream_t st = (hipStream_t)stream;
    MOE_TRY(MOE_PROF_OTHER, st, moe::launch_pack_b(w, packed, G, N, K, st));
    return MOE_OK;
}

int moe_shared_ffn(const moe_shape* s, const void* x, const void* w1_sh, const float* b1_sh, const void* w2_sh,
                   void* y, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (s->T == 0 || s->Ks == 0) return MOE_OK;
    if (!x || !w1_sh || !w2_sh || !y) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w1_sh) || !aligned16(w2_sh) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
    if (b1_sh && s->act != MOE_ACT_RELU_BIAS) return MOE_ERR_INVALID_ARG;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout_of(s);
    return do_shared_ffn(s, x, w1_sh, b1_sh, w2_sh, y, at<void>(ws, L.act_sh), (hipStream_t)stream);
}

int moe_combine(const moe_shape* s, const void* residual, const void* y_shared, const void* y_perm,
                const int32_t* pair_row, const float* topk_w, void* out, void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (s->T == 0) return MOE_OK;
    if (!out || !aligned16(out)) return MOE_ERR_INVALID_ARG;
    if (s->K_r > 0 && (!y_perm || !pair_row || !topk_w || !aligned16(y_perm))) return MOE_ERR_INVALID_ARG;
    if ((residual && !aligned16(residual)) || (y_shared && !aligned16(y_shared))) return MOE_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    MOE_TRY(MOE_PROF_COMBINE, st, moe::launch_combine(s->dtype, residual, y_shared, y_perm, pair_row, topk_w, out,
                                                      s->T, s->H, s->K_r, st));
    return MOE_OK;
}

int moe_layer_forward(const moe_shape* s, const void* u, const void* centroids, const float* bias, const void* w1,
                      const float* b1, const void* w2, const void* w1_sh, const float* b1_sh, const void* w2_sh,
                      int32_t flags, void* out, int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      void* stream) {
    return layer_forward(s, u, centroids, bias, w1, b1, w2, w1_sh, b1_sh, w2_sh, flags, out, topk_idx_out, topk_w_out,
                         ws, ws_bytes, stream);
}

int moe_layer_forward_noalloc(const moe_shape* s, const void* u, const void* centroids, const float* bias,
                              const void* w1, const float* b1, const void* w2, const void* w1_sh, const float* b1_sh,
                              const void* w2_sh, int32_t flags, void* out, int32_t* topk_idx_out, float* topk_w_out,
                              void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (layout_of(s).total > kScratchBytes) return MOE_ERR_SCRATCH;
    void* ws = nullptr;
    if ((rc = scratch_of_current_device(&ws)) != MOE_OK) return rc;
    return layer_forward(s, u, centroids, bias, w1, b1, w2, w1_sh, b1_sh, w2_sh, flags, out, topk_idx_out, topk_w_out,
                         ws, kScratchBytes, stream);
}

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"

namespace {

int layer_forward(const moe_shape* s, const void* u, const void* centroids, const float* bias, const void* w1,
                  const float* b1, const void* w2, const void* w1_sh, const float* b1_sh, const void* w2_sh,
                  int32_t flags, void* out, int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                  void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (flags & ~(MOE_FLAG_NO_RESIDUAL | MOE_FLAG_PACKED_WEIGHTS | MOE_FLAG_PACKED_SHARED_UP))
        return MOE_ERR_INVALID_ARG;
    const bool packed = (flags & MOE_FLAG_PACKED_WEIGHTS) != 0;
    const bool packed_sh = (flags & MOE_FLAG_PACKED_SHARED_UP) != 0;
    if ((packed || packed_sh) && (rc = check_packed(s)) != MOE_OK) return rc;
    if (bias && s->gating != MOE_GATE_SIGMOID_BIAS_NORM) return MOE_ERR_INVALID_ARG;
    if ((b1 || b1_sh) && s->act != MOE_ACT_RELU_BIAS) return MOE_ERR_INVALID_ARG;
    if (s->T == 0) return MOE_OK;
    if (!u || !out || !aligned16(u) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
    if (s->K_r > 0 && (!centroids || !w1 || !w2 || !aligned16(centroids) || !aligned16(w1) || !aligned16(w2)))
        return MOE_ERR_INVALID_ARG;
    if (s->Ks > 0 && (!w1_sh || !w2_sh || !aligned16(w1_sh) || !aligned16(w2_sh))) return MOE_ERR_INVALID_ARG;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout_of(s);
    hipStream_t st = (hipStream_t)stream;
    int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.topk_idx);
    float* wts = topk_w_out ? topk_w_out : at<float>(ws, L.topk_w);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* pair_row = at<int32_t>(ws, L.pair_row);
    void* y_perm = at<void>(ws, L.y_perm);
    void* y_sh = at<void>(ws, L.y_sh);
    if (s->K_r > 0) {
        if ((rc = do_route(s, u, centroids, bias, idx, wts, at<float>(ws, L.logits), st)) != MOE_OK) return rc;
        if ((rc = do_dispatch(s, idx, offsets, at<int32_t>(ws, L.row_token), pair_row, at<int32_t>(ws, L.chunks),
                              st)) != MOE_OK)
            return rc;
        if ((rc = do_expert_ffn(s, u, at<int32_t>(ws, L.row_token), offsets, w1, b1, w2, y_perm,
                                at<int32_t>(ws, L.tiles), at<void>(ws, L.act), st, packed)) != MOE_OK)
            return rc;
    }
    const void* resid = (flags & MOE_FLAG_NO_RESIDUAL) ? nullptr : u;
    if (s->Ks > 0 && s->dtype == MOE_BF16) {
        // combine fused into the shared experts' down GEMM: the shared output never leaves the
        // fp32 accumulators, and the layer output is written once
        const Combine comb{resid, y_perm, pair_row, wts};
        return do_shared_ffn(s, u, w1_sh, b1_sh, w2_sh, out, at<void>(ws, L.act_sh), st, &comb, packed_sh);
    }
    if (s->Ks > 0) {
        if ((rc = do_shared_ffn(s, u, w1_sh, b1_sh, w2_sh, y_sh, at<void>(ws, L.act_sh), st, nullptr, packed_sh)) !=
            MOE_OK)
            return rc;
    }
    MOE_TRY(MOE_PROF_COMBINE, st,
            moe::launch_combine(s->dtype, resid, s->Ks > 0 ? y_sh : nullptr, y_perm, pair_row, wts, out, s->T, s->H,
                                s->K_r, st));
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_bias_update(const moe_shape* s, const int32_t* offsets, float gamma, float* bias, int32_t* counts,
                    void* stream) {
    int rc = check_shape(s);
    if (rc != MOE_OK) return rc;
    if (s->N_r == 0) return MOE_OK;
    if (!offsets || !bias) return MOE_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    MOE_TRY(MOE_PROF_OTHER, st, moe::launch_bias_update(offsets, s->N_r, s->T, s->K_r, gamma, bias, counts, st));
    return MOE_OK;
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP error";
        case MOE_ERR_SCRATCH: return "shape needs more scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int moe_profile_enable(int32_t on) {
    if (on) {
        if (g_prof.ev.empty()) {
            g_prof.ev.resize(2 * kProfPairs);
            g_prof.cls.resize(kProfPairs);
            for (size_t i = 0; i < g_prof.ev.size(); ++i) {
                const hipError_t r = hipEventCreate(&g_prof.ev[i]);
                if (r != hipSuccess) {
                    for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(g_prof.ev[j]);
                    g_prof.ev.clear();
                    g_prof.cls.clear();
                    return hip_fail(r);
                }
            }
        }
        g_prof.used = 0;
        g_prof.on = true;
    } else {
        g_prof.on = false;
    }
    return MOE_OK;
}

int moe_profile_query(int32_t kernel, int64_t* launches, double* total_ms) {
    if (kernel < 0 || kernel >= MOE_PROF_COUNT || !launches || !total_ms) return MOE_ERR_INVALID_ARG;
    int64_t n = 0;
    double ms = 0.0;
    for (size_t i = 0; i < g_prof.used; ++i) {
        if (g_prof.cls[i] != kernel) continue;
        const hipError_t r = hipEventSynchronize(g_prof.ev[2 * i + 1]);
        if (r != hipSuccess) return hip_fail(r);
        float t = 0.f;
        const hipError_t r2 = hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (r2 != hipSuccess) return hip_fail(r2);
        ++n;
        ms += t;
    }
    *launches = n;
    *total_ms = ms;
    return MOE_OK;
}

}  // extern "C"
