// Expert FFNs as grouped GEMMs.
//
// Routed experts (llm-infra-atlas "02 Fine-grained MoE", section 2.1: mN experts of width
// M/m) are groups of consecutive rows of the permuted pair list; the shared experts
// (section 3.1, Eq. 9) are dense groups over all tokens.  Each expert is
//   SwiGLU: y = W2 (SiLU(Wg x) * (Wu x))      ReLU: y = V ReLU(W x + b)   (tomabc explainer)
// computed as an "up" GEMM with the activation fused into its epilogue, then a "down" GEMM.
//
// bf16 path, all on v_mfma_f32_32x32x16_bf16 with persistent XCD-aware grids:
//  - k_gemm_bf16_w4p: routed weights in MFMA fragment order (launch_pack_b); 128 x 512 x 64 tiles,
//    four waves of 128 x 128, each wave loading its weight fragments straight into registers and
//    the activation tile going through a ring of direct-to-LDS loads (the prefill default); a
//    128 x 256 instantiation at two workgroups per CU serves reductions of at most 512;
//  - k_gemm_bf16_w4: the same 128 x 512 tile on [out, in] weights, both operands register-staged
//    with buffer loads into double-buffered LDS (also the dense shared up projection);
//  - k_gemm_bf16_wide8: 128 x 512 tiles, eight waves of 128 x 64, direct-to-LDS loads (operands
//    spanning 2 GiB or more);
//  - k_gemm_bf16: 128 x 128 x 64 tiles, four waves of 64 x 64, two workgroups per CU (the fused
//    shared-down + combine, the prefill router logits, small problems);
//  - k_gemm_bf16_dec: 32-row tiles with a deep direct-to-LDS load ring for decode-sized groups
//    (four waves of 64 weight rows) and a one-wave variant for the few dense rows of a decode step.
// Every kernel accumulates an output in one fp32 chain over ascending 16-deep k-chunks, so the
// choice of kernel does not change a result bit.  For SwiGLU the weight rows of a tile are gate
// rows and the matching up rows, so the epilogue has both halves of every output element in the
// same lane.  fp32 path: plain VALU kernels (the tiny fp32 layer only).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int BM = 128, BN = 128, BK = 64;

int gemm_bm(int dtype) { return dtype == 0 ? 1 : BM; }

// Compute units of the current device (cached per device id).
static int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// ---------------------------------------------------------------- tile plan
// Exclusive prefix over g < G of v (one value per thread of the single 1024-thread workgroup);
// out[G] = total.
__device__ __forceinline__ void block_prefix(int v, int G, int32_t* __restrict__ out, int32_t* wsum) {
    const int g = threadIdx.x, lane = g & 63, w = g >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(incl, o);
        if (lane >= o) incl += x;
    }
    __syncthreads();   // wsum may still be read by a previous call
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (g == 0) {
        int acc = 0;
        for (int q = 0; q < 16; ++q) {
            const int x = wsum[q];
            wsum[q] = acc;
            acc += x;
        }
        out[G] = acc;
    }
    __syncthreads();
    if (g < G) out[g] = wsum[w] + incl - v;
}

// tiles[g] = sum_{g' < g} ceil(rows(g') / bm), tiles[G] = total; then the same prefix for 32-row
// tiles at tiles + G + 1.  One workgroup, G <= 1024.
__global__ __launch_bounds__(1024) void k_tile_plan(const int32_t* __restrict__ offsets, int G, int bm,
                                                    int32_t* __restrict__ tiles) {
    __shared__ int32_t wsum[16];
    const int g = threadIdx.x;
    const int rows = g < G ? offsets[g + 1] - offsets[g] : 0;
    block_prefix(rows > 0 ? (rows + bm - 1) / bm : 0, G, tiles, wsum);
    block_prefix(rows > 0 ? (rows + 31) / 32 : 0, G, tiles + G + 1, wsum);
}

hipError_t launch_tile_plan(const int32_t* offsets, int G, int bm, int32_t* tiles, hipStream_t s) {
    hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(1024), 0, s, offsets, G, bm, tiles);
    return hipGetLastError();
}

// ---------------------------------------------------------------- tile decode
struct TileInfo {
    int g, row0, rows, nt;
};

// Inside a group of nm m-tiles x NT n-tiles the tiles are visited in blocks of kGroupM m-tiles
// (m fastest, then n), so that a window of concurrently running tiles covers a few m-tiles
// times a few n-tiles and reuses both operands from L2 instead of streaming one of them.
constexpr int kGroupM = 8;

__device__ __forceinline__ void blocked_mn(int Lg, int nm, int NT, int& ml, int& nt) {
    const int blk = Lg / (kGroupM * NT);
    const int m0 = blk * kGroupM;
    const int bm = min(kGroupM, nm - m0);
    const int r = Lg - blk * kGroupM * NT;
    nt = r / bm;
    ml = m0 + (r - nt * bm);
}

__device__ __forceinline__ bool decode_tile(const GemmParams& p, int NT, int bm, int L, TileInfo& ti) {
    if (p.offsets) {
        const int total = p.tiles[p.G];
        if (L >= total * NT) return false;
        const int mt = L / NT;  // tiles[g] * NT <= L  <=>  tiles[g] <= L / NT
        int lo = 0, hi = p.G;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.tiles[mid] <= mt) lo = mid;
            else hi = mid;
        }
        const int g = lo;
        const int t0 = p.tiles[g], nm = p.tiles[g + 1] - t0;
        int ml;
        blocked_mn(L - t0 * NT, nm, NT, ml, ti.nt);
        ti.g = g;
        ti.row0 = p.offsets[g] + ml * bm;
        ti.rows = min(bm, p.offsets[g + 1] - ti.row0);
    } else {
        const int nm = (p.M_dense + bm - 1) / bm;
        const int per = nm * NT;
        if (L >= p.G * per) return false;
        ti.g = L / per;
        int ml;
        blocked_mn(L - ti.g * per, nm, NT, ml, ti.nt);
        ti.row0 = ml * bm;
        ti.rows = min(bm, p.M_dense - ti.row0);
    }
    return true;
}

// Grouped GEMMs keep the group table (an m-tile prefix and the row offsets, G + 1 entries each, G <=
// 1024) in LDS: finding a tile's group is then a binary search over LDS instead of a chain of
// dependent global loads at the start of every tile.
constexpr int kGroupTabBytes = 2 * 1025 * 4;
__device__ __forceinline__ void load_group_tab(const int32_t* tiles, const int32_t* offsets, int G, int32_t* gt) {
    for (int i = threadIdx.x; i <= G; i += blockDim.x) {
        gt[i] = tiles[i];
        gt[G + 1 + i] = offsets[i];
    }
    __syncthreads();
}
// The tile L of the list whose m-tile prefix (tiles, of bm-row tiles) and offsets are in gt.
__device__ __forceinline__ void decode_tile_tab(const int32_t* gt, int G, int NT, int bm, int L, TileInfo& ti) {
    const int32_t* tiles = gt;
    const int32_t* offs = gt + G + 1;
    const int mt = L / NT;
    int lo = 0, hi = G;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tiles[mid] <= mt) lo = mid;
        else hi = mid;
    }
    const int t0 = tiles[lo], nm = tiles[lo + 1] - t0;
    int ml;
    blocked_mn(L - t0 * NT, nm, NT, ml, ti.nt);
    ti.g = lo;
    ti.row0 = offs[lo] + ml * bm;
    ti.rows = min(bm, offs[lo + 1] - ti.row0);
}

// ---------------------------------------------------------------- bf16 MFMA grouped GEMM
// Persistent: the grid holds two workgroups per CU; the workgroups of one XCD walk a
// contiguous range of the tile list (so concurrently running tiles of an XCD share weight
// and activation tiles in its L2), strided by the number of workgroups on that XCD.
//
// Operand tiles (128 rows x 64 k, bf16) move global -> LDS with global_load_lds_dwordx4: one
// instruction moves 64 lanes x 16 bytes into 1 KB of LDS (lane i -> bytes [16 i, 16 i + 16)),
// so there is no register staging.  LDS rows are 128 bytes, unpadded; the 16-byte chunk c of
// row r is stored in slot c ^ ((r >> 1) & 7).  Two rows share one 256-byte window of the 64
// banks, so this spreads the fragment reads of 16 consecutive rows at one k offset over all
// 64 banks.  The compiler does not track these LDS writes, so every hand-off
// is an explicit vmcnt(0) wait plus a workgroup barrier.  Epilogues stage the fp32 tile
// through LDS and store 16-byte vectors.
constexpr int EPW = BN + 4;                               // fp32 staging row (floats)
constexpr int kTileBytes = BM * BK * 2;                   // one operand tile (16 KB)
constexpr int kStageBytes = 2 * kTileBytes;               // A + B
constexpr int kSmemBytes = BM * EPW * 4 > 2 * kStageBytes ? BM * EPW * 4 : 2 * kStageBytes;
// Fused combine: the routed-row indices and gate weights of a tile's rows, read into LDS behind the
// staging area when the tile starts (up to kCombKmax per row; two workgroups still fit a CU).
constexpr int kCombKmax = 12;
constexpr int kCombBytes = BM * kCombKmax * 8;
static_assert(2 * (kSmemBytes + kCombBytes) <= 160 * 1024, "two workgroups per CU");
static_assert(BM == BN && BM == 128 && BK == 64, "tile layout assumes 128 x 128 x 64");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dma16(const void* g, unsigned char* lds_chunk) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_chunk, 16, 0, 0);
}
// the same with the non-temporal cache policy (cache-policy operand 2: nt), for bytes read once
__device__ __forceinline__ void dma16_nt(const void* g, unsigned char* lds_chunk) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_chunk, 16, 0, 2);
}

__device__ __forceinline__ void mma_tile(f32x16& c00, f32x16& c01, f32x16& c10, f32x16& c11,
                                         const unsigned char* sa, const unsigned char* sb, int arow, int br0,
                                         int br1, int lane) {
    const int rA0 = arow + (lane & 31), rA1 = rA0 + 32;
    const int rB0 = br0 + (lane & 31), rB1 = br1 + (lane & 31);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
        const int kc = 2 * s + (lane >> 5);   // logical 16-byte chunk of the 64-wide k-tile
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(sa + rA0 * 128 + ((kc ^ ((rA0 >> 1) & 7)) << 4));
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(sa + rA1 * 128 + ((kc ^ ((rA1 >> 1) & 7)) << 4));
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(sb + rB0 * 128 + ((kc ^ ((rB0 >> 1) & 7)) << 4));
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(sb + rB1 * 128 + ((kc ^ ((rB1 >> 1) & 7)) << 4));
        c00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c00, 0, 0, 0);
        c01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c01, 0, 0, 0);
        c10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c10, 0, 0, 0);
        c11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c11, 0, 0, 0);
    }
}

__device__ __forceinline__ uint4 pack8_bf16(const float (&v)[8]) {
    uint4 o;
    o.x = pack2_bf16(v[0], v[1]);
    o.y = pack2_bf16(v[2], v[3]);
    o.z = pack2_bf16(v[4], v[5]);
    o.w = pack2_bf16(v[6], v[7]);
    return o;
}

__device__ __forceinline__ void add8_bf16(float (&v)[8], uint4 q) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] += __uint_as_float(w[e] << 16);
        v[2 * e + 1] += __uint_as_float(w[e] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ void fma8_bf16(float (&v)[8], float g, uint4 q) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = fmaf(g, __uint_as_float(w[e] << 16), v[2 * e]);
        v[2 * e + 1] = fmaf(g, __uint_as_float(w[e] & 0xFFFF0000u), v[2 * e + 1]);
    }
}

// Epilogue of one 8-column piece of output row rl (tile-local) starting at column col0:
// bias + ReLU (ReLU up), residual + gate-weighted routed rows (shared down + combine),
// then one bf16 rounding and a 16-byte store.
template <int MODE>
__device__ __forceinline__ void epilogue_row(const GemmParams& p, const TileInfo& ti, float (&v)[8], int rl,
                                             int col0) {
    const long long row = ti.row0 + rl;
    if (MODE == GM_UP_RELU) {
        if (p.bias) {
            const float* bb = p.bias + (long long)ti.g * p.sbias_group + col0;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += bb[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaxf(v[e], 0.0f);
    }
    if (MODE == GM_DOWN_COMBINE) {
        // fixed order: residual + shared experts, then the routed rows k = 0 .. K_r-1
        if (p.resid) {
            const uint4 q = ld_once16((const uint16_t*)p.resid + row * p.N + col0);
            float u8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            add8_bf16(u8, q);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = u8[e] + v[e];
        }
        const int32_t* prr = p.pair_row + row * p.K_r;
        const float* gr = p.topk_w + row * p.K_r;
        int k = 0;
        for (; k + 4 <= p.K_r; k += 4) {
            long long r4[4];
            float g4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const long long x = (long long)(uint32_t)prr[k + e];
                r4[e] = x < p.R ? x : p.R - 1;
                g4[e] = gr[k + e];
            }
            uint4 y4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                y4[e] = ld_once16((const uint16_t*)p.y_perm + r4[e] * p.N + col0);
#pragma unroll
            for (int e = 0; e < 4; ++e) fma8_bf16(v, g4[e], y4[e]);
        }
        for (; k < p.K_r; ++k) {
            long long x = (long long)(uint32_t)prr[k];
            x = x < p.R ? x : p.R - 1;
            fma8_bf16(v, gr[k], ld_once16((const uint16_t*)p.y_perm + x * p.N + col0));
        }
    }
    const long long coff = p.offsets ? 0 : (long long)ti.g * p.sC_group;
    if (MODE == GM_F32OUT) {
        float* C = (float*)p.C + row * p.ldc + coff + col0;
        reinterpret_cast<float4*>(C)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(C)[1] = make_float4(v[4], v[5], v[6], v[7]);
        return;
    }
    uint16_t* C = (uint16_t*)p.C;
    *reinterpret_cast<uint4*>(C + row * p.ldc + coff + col0) = pack8_bf16(v);
}

// Fused combine of two output rows a, b (tile-local ra, rb) on the 8 columns from col0, with the pair
// rows and gates of the tile's rows in LDS (si, sg: K_r per row): the same fixed fp32 order as
// epilogue_row (residual + shared experts, then the routed rows k = 0 .. K_r-1), one bf16 rounding.
__device__ __forceinline__ void combine_rows(const GemmParams& p, const TileInfo& ti, float (&va)[8], float (&vb)[8],
                                             int ra, int rb, int col0, const int32_t* si, const float* sg) {
    const long long rowa = ti.row0 + ra, rowb = ti.row0 + rb;
    const uint16_t* Y = (const uint16_t*)p.y_perm;
    if (p.resid) {
        const uint4 qa = ld_once16((const uint16_t*)p.resid + rowa * p.N + col0);
        const uint4 qb = ld_once16((const uint16_t*)p.resid + rowb * p.N + col0);
        float ua[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, ub[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        add8_bf16(ua, qa);
        add8_bf16(ub, qb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            va[e] = ua[e] + va[e];
            vb[e] = ub[e] + vb[e];
        }
    }
    const int K = p.K_r;
    for (int k = 0; k < K; k += 4) {
        uint4 ya[4], yb[4];
        float ga[4], gb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int kk = k + e < K ? k + e : K - 1;
            long long xa = (long long)(uint32_t)si[ra * K + kk], xb = (long long)(uint32_t)si[rb * K + kk];
            xa = xa < p.R ? xa : p.R - 1;
            xb = xb < p.R ? xb : p.R - 1;
            ga[e] = sg[ra * K + kk];
            gb[e] = sg[rb * K + kk];
            ya[e] = ld_once16(Y + xa * p.N + col0);
            yb[e] = ld_once16(Y + xb * p.N + col0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (k + e < K) {
                fma8_bf16(va, ga[e], ya[e]);
                fma8_bf16(vb, gb[e], yb[e]);
            }
        }
    }
    uint16_t* C = (uint16_t*)p.C;
    *reinterpret_cast<uint4*>(C + rowa * p.ldc + col0) = pack8_bf16(va);
    if (rb != ra) *reinterpret_cast<uint4*>(C + rowb * p.ldc + col0) = pack8_bf16(vb);
}

template <int MODE>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const TileInfo& ti, unsigned char* smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;

    // DMA assignment: wave w moves 1 KB chunks c = 4 w + i (i < 4) of each operand tile; chunk c
    // is rows 8c .. 8c+7; lane l of it is row 8c + l/8, LDS slot l%8, global chunk (l%8) ^ ((row>>1)&7).
    const uint16_t* A = (const uint16_t*)p.A + (p.offsets ? 0 : (size_t)ti.g * p.sA_group);
    const uint16_t* Bg = (const uint16_t*)p.B + (size_t)ti.g * p.sB_group;
    const uint16_t* ag[4];
    const uint16_t* bg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 8 * (4 * w + i) + (lane >> 3);
        const int kcg = ((lane & 7) ^ ((row >> 1) & 7)) * 8;   // element offset of the global chunk
        const int r = min(row, ti.rows - 1);
        long long src = ti.row0 + r;
        if (p.a_rows) src = min(max((long long)p.a_rows[src], 0LL), p.a_nrows - 1);
        ag[i] = A + src * p.lda + kcg;
        int wr;
        if (MODE == GM_UP_SWIGLU) {
            const int n0 = ti.nt * 64;
            wr = row < 64 ? n0 + row : p.up_off + n0 + (row - 64);
        } else {
            wr = min(ti.nt * BN + row, p.N - 1);
        }
        bg[i] = Bg + (size_t)wr * p.ldb + kcg;
    }
    auto issue = [&](int kt, int buf) {
        const int k = kt * BK;
        const int seg = k / p.Kseg;
        const long long bo = (long long)seg * p.sB_seg + (k - seg * p.Kseg);
        unsigned char* sa = smem + buf * kStageBytes;
        unsigned char* sb = sa + kTileBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(ag[i] + k, sa + (4 * w + i) * 1024);
            dma16(bg[i] + bo, sb + (4 * w + i) * 1024);
        }
    };

    f32x16 c00, c01, c10, c11;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        c00[q] = 0.f;
        c01[q] = 0.f;
        c10[q] = 0.f;
        c11[q] = 0.f;
    }
    const int br0 = MODE == GM_UP_SWIGLU ? wn * 32 : wn * 64;
    const int br1 = MODE == GM_UP_SWIGLU ? 64 + wn * 32 : wn * 64 + 32;
    const int arow = wm * 64;
    const int nk = p.K / BK;

    __syncthreads();  // the previous tile's epilogue may still read the LDS staging area
    issue(0, 0);
    const bool comb_lds = MODE == GM_DOWN_COMBINE && p.K_r <= kCombKmax;
    if (comb_lds) {
        // this tile's pair rows and gates (rows * K_r contiguous values each), behind k-tile 0's loads
        int32_t* si = reinterpret_cast<int32_t*>(smem + kSmemBytes);
        float* sg = reinterpret_cast<float*>(smem + kSmemBytes + BM * kCombKmax * 4);
        const int n = ti.rows * p.K_r;
        const int32_t* pr = p.pair_row + (long long)ti.row0 * p.K_r;
        const float* gw = p.topk_w + (long long)ti.row0 * p.K_r;
        int32_t xi[kCombKmax * BM / 256];
        float xg[kCombKmax * BM / 256];
#pragma unroll
        for (int j = 0; j < kCombKmax * BM / 256; ++j) {
            const int o = tid + 256 * j;
            if (o < n) {
                xi[j] = pr[o];
                xg[j] = gw[o];
            }
        }
#pragma unroll
        for (int j = 0; j < kCombKmax * BM / 256; ++j) {
            const int o = tid + 256 * j;
            if (o < n) {
                si[o] = xi[j];
                sg[o] = xg[j];
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) issue(kt + 1, buf ^ 1);   // that buffer was last read before the previous barrier
        mma_tile(c00, c01, c10, c11, smem + buf * kStageBytes, smem + buf * kStageBytes + kTileBytes, arow, br0,
                 br1, lane);
        __builtin_amdgcn_s_waitcnt(0);               // the next tile has landed in LDS
        __syncthreads();
    }

    // ---- epilogue: stage through LDS, then each row is covered by 16-byte vectors.
    // D[i][j] of a 32x32 block: column j = lane % 32, row i = 8 (q / 4) + 4 (lane / 32) + (q % 4).
    constexpr int OUTW = MODE == GM_UP_SWIGLU ? 64 : BN;  // output columns of the tile
    float* st = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int rl = wm * 64 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (MODE == GM_UP_SWIGLU) {
            st[rl * EPW + wn * 32 + (lane & 31)] = silu(c00[q]) * c01[q];
            st[(rl + 32) * EPW + wn * 32 + (lane & 31)] = silu(c10[q]) * c11[q];
        } else {
            st[rl * EPW + wn * 64 + (lane & 31)] = c00[q];
            st[rl * EPW + wn * 64 + 32 + (lane & 31)] = c01[q];
            st[(rl + 32) * EPW + wn * 64 + (lane & 31)] = c10[q];
            st[(rl + 32) * EPW + wn * 64 + 32 + (lane & 31)] = c11[q];
        }
    }
    __syncthreads();
    constexpr int TPR = OUTW / 8;    // threads per row
    constexpr int RPP = 256 / TPR;   // rows per pass
    const int cq = (tid % TPR) * 8;
    const int col0 = ti.nt * OUTW + cq;
    if (col0 >= p.N) return;
    if (MODE == GM_DOWN_COMBINE && comb_lds) {
        // two rows per pass: their residual and routed-row loads are all in flight together
        const int32_t* si = reinterpret_cast<const int32_t*>(smem + kSmemBytes);
        const float* sg = reinterpret_cast<const float*>(smem + kSmemBytes + BM * kCombKmax * 4);
        for (int rl = tid / TPR; rl < ti.rows; rl += 2 * RPP) {
            const int rb = rl + RPP < ti.rows ? rl + RPP : rl;   // a lone last row is done twice (same values)
            float va[8], vb[8];
            {
                const float4 a0 = *reinterpret_cast<const float4*>(&st[rl * EPW + cq]);
                const float4 a1 = *reinterpret_cast<const float4*>(&st[rl * EPW + cq + 4]);
                const float4 b0 = *reinterpret_cast<const float4*>(&st[rb * EPW + cq]);
                const float4 b1 = *reinterpret_cast<const float4*>(&st[rb * EPW + cq + 4]);
                va[0] = a0.x; va[1] = a0.y; va[2] = a0.z; va[3] = a0.w;
                va[4] = a1.x; va[5] = a1.y; va[6] = a1.z; va[7] = a1.w;
                vb[0] = b0.x; vb[1] = b0.y; vb[2] = b0.z; vb[3] = b0.w;
                vb[4] = b1.x; vb[5] = b1.y; vb[6] = b1.z; vb[7] = b1.w;
            }
            combine_rows(p, ti, va, vb, rl, rb, col0, si, sg);
        }
        return;
    }
    for (int rl = tid / TPR; rl < ti.rows; rl += RPP) {
        const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * EPW + cq]);
        const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * EPW + cq + 4]);
        float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        epilogue_row<MODE>(p, ti, v, rl, col0);
    }
}

__device__ __forceinline__ int total_tiles(const GemmParams& p, int NT) {
    if (p.offsets) return p.tiles[p.G] * NT;
    return p.G * ((p.M_dense + BM - 1) / BM) * NT;
}

template <int MODE, bool GROUPED>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(GemmParams p, int NT) {
    if (GROUPED != (p.offsets != nullptr)) return;  // launched with the matching instantiation only
    __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes + (MODE == GM_DOWN_COMBINE ? kCombBytes : 0)];
    const int total = total_tiles(p, NT);
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
    const int beg = (int)((long long)total * xcd / 8);
    const int end = (int)((long long)total * (xcd + 1) / 8);
    for (int L = beg + loc; L < end; L += per_xcd) {
        TileInfo ti;
        decode_tile(p, NT, BM, L, ti);
        gemm_tile<MODE>(p, ti, smem);
    }
}

// ---------------------------------------------------------------- bf16 MFMA grouped GEMM, wide tile
// 128 rows x 512 output columns per workgroup (twice the arithmetic per byte moved of the
// 128 x 128 tile).  Two 80 KB operand stages fill the LDS; one workgroup per CU.  Same
// swizzled DMA staging and explicit hand-offs as the 128 x 128 kernel.
constexpr int WBN = 512;
constexpr int kWTileA = BM * BK * 2;          // 16 KB
constexpr int kWTileB = WBN * BK * 2;         // 64 KB
constexpr int kWStage = kWTileA + kWTileB;    // 80 KB
constexpr int kWSmem = 2 * kWStage;           // 160 KB
constexpr int WEPW_SW = 256 + 4;              // SwiGLU staging row: 256 outputs
constexpr int WEPW = WBN + 4;                 // other modes: 512 outputs, staged 64 rows at a time
static_assert(BM * WEPW_SW * 4 <= kWSmem && 64 * WEPW * 4 <= kWSmem, "wide epilogue staging must fit");

__device__ __forceinline__ const bf16x8& frag(const unsigned char* base, int row, int kc) {
    return *reinterpret_cast<const bf16x8*>(base + row * 128 + ((kc ^ ((row >> 1) & 7)) << 4));
}

// Epilogue of a 128 x 512 tile held as acc[i][j] (rows 32 i.., columns of wave w: SwiGLU gate / up
// blocks 32 w and 256 + 32 w, otherwise 64 w + 32 j): stage through LDS, 16-byte stores.
template <int MODE>
__device__ __forceinline__ void wide_epilogue(const GemmParams& p, const TileInfo& ti, f32x16 (&acc)[4][2],
                                              unsigned char* smem) {
    // recomputed here from an opaque copy of the thread index: the epilogue's lane-dependent
    // addresses are then not kept live (or spilled) across the k-loop and the tile loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = tid >> 6;
    float* st = reinterpret_cast<float*>(smem);
    if (MODE == GM_UP_SWIGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int rl = 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                st[rl * WEPW_SW + 32 * w + (lane & 31)] = silu(acc[i][0][q]) * acc[i][1][q];
            }
        __syncthreads();
        const int cq = (tid & 31) * 8;
        const int col0 = ti.nt * 256 + cq;
        if (col0 < p.N) {
            for (int rl = tid >> 5; rl < ti.rows; rl += 16) {
                const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * WEPW_SW + cq]);
                const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * WEPW_SW + cq + 4]);
                float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                epilogue_row<MODE>(p, ti, v, rl, col0);
            }
        }
        return;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // rows [64 h, 64 h + 64)
        if (h) __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int rl = 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    st[rl * WEPW + 64 * w + 32 * j + (lane & 31)] = acc[2 * h + i][j][q];
                }
        __syncthreads();
        const int cq = lane * 8;
        const int col0 = ti.nt * WBN + cq;
        if (col0 < p.N) {
            for (int rl = w; rl < 64 && 64 * h + rl < ti.rows; rl += 8) {
                const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * WEPW + cq]);
                const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * WEPW + cq + 4]);
                float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                epilogue_row<MODE>(p, ti, v, 64 * h + rl, col0);
            }
        }
    }
}

// Eight waves (two per SIMD), each owning a 128 x 64 block (4 x 2 accumulators).  Issue is in
// order, and a DMA issue stalls its wave for tens of cycles while the CU's address unit is busy;
// the other wave of the SIMD keeps the matrix pipe fed meanwhile.
template <int MODE>
__device__ __forceinline__ void gemm_tile_wide8(const GemmParams& p, const TileInfo& ti, unsigned char* smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;   // w < 8

    const uint16_t* A = (const uint16_t*)p.A + (p.offsets ? 0 : (size_t)ti.g * p.sA_group);
    const uint16_t* Bg = (const uint16_t*)p.B + (size_t)ti.g * p.sB_group;
    // A: 16 chunks, wave w moves chunks 2w, 2w+1 (rows 16 w + 8 i + lane/8)
    const uint16_t* ag[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 8 * (2 * w + i) + (lane >> 3);
        const int kcg = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
        const int r = min(row, ti.rows - 1);
        long long src = ti.row0 + r;
        if (p.a_rows) src = min(max((long long)p.a_rows[src], 0LL), p.a_nrows - 1);
        ag[i] = A + src * p.lda + kcg;
    }
    // B: 64 chunks, wave w moves chunks 8w .. 8w+7 (rows 64 w + 8 i + lane/8)
    int wrow0, wrow_max;
    if (MODE == GM_UP_SWIGLU) {
        const int n0 = ti.nt * 256;
        const int r0 = 64 * w + (lane >> 3);
        wrow0 = r0 < 256 ? n0 + r0 : p.up_off + n0 + (r0 - 256);
        wrow_max = r0 < 256 ? p.N - 1 : p.up_off + p.N - 1;
    } else {
        wrow0 = ti.nt * WBN + 64 * w + (lane >> 3);
        wrow_max = p.N - 1;
    }
    // the two swizzle variants of this lane's B chunks (row 64 w + 8 i + lane/8: i even / odd)
    const int kcgB0 = ((lane & 7) ^ ((lane >> 4) & 7)) * 8;
    const int kcgB1 = ((lane & 7) ^ ((4 + (lane >> 4)) & 7)) * 8;
    const unsigned ldb = (unsigned)p.ldb;
    // DMA chunk c (< 10) of a k-tile whose A column offset is kA and B offset bo, into stage
    // dst: c < 2 -> A chunk 2w + c, else B chunk 8w + (c - 2).  Per-k-step offsets are computed
    // once by the caller; a chunk costs a clamp, one multiply-add and the M0 write.
    auto dma_chunk = [&](int kA, long long bo, unsigned char* dst, int c) {
        if (c < 2) {
            dma16(ag[c] + kA, dst + (2 * w + c) * 1024);
        } else {
            const int i = c - 2;
            const int wr = min(wrow0 + 8 * i, wrow_max);
            dma16(Bg + ((size_t)(unsigned)wr * ldb + (unsigned)((i & 1) ? kcgB1 : kcgB0)) + bo,
                  dst + kWTileA + (8 * w + i) * 1024);
        }
    };
    auto koffs = [&](int kt, int& kA, long long& bo) {
        kA = kt * BK;
        const int seg = kA / p.Kseg;
        bo = (long long)seg * p.sB_seg + (kA - seg * p.Kseg);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    int brow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) brow[j] = MODE == GM_UP_SWIGLU ? 256 * j + 32 * w : 64 * w + 32 * j;
    const int nk = p.K / BK;

    // k-step schedule as in the four-wave kernel: sub-steps 0-1 carry the DMA issues, the
    // wait + barrier sits before sub-step 3, which prefetches the next tile's fragments.
    bf16x8 af[2][4], bfr[2][2];
    __syncthreads();
    {
        int kA;
        long long bo;
        koffs(0, kA, bo);
#pragma unroll
        for (int c = 0; c < 10; ++c) dma_chunk(kA, bo, smem, c);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = frag(smem, 32 * i + (lane & 31), lane >> 5);
#pragma unroll
    for (int j = 0; j < 2; ++j) bfr[0][j] = frag(smem + kWTileA, brow[j] + (lane & 31), lane >> 5);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const int kn = kt + 1 < nk ? kt + 1 : kt;
        const unsigned char* sa = smem + buf * kWStage;
        unsigned char* na = smem + (buf ^ 1) * kWStage;
        int kA;
        long long bo;
        koffs(kn, kA, bo);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int cur = s & 1;
            if (s == 3) {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            const unsigned char* fa = s < 3 ? sa : na;
            const int kc = 2 * ((s + 1) & 3) + (lane >> 5);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                __builtin_amdgcn_sched_barrier(0);
                acc[g][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][g], bfr[cur][0], acc[g][0], 0, 0, 0);
                acc[g][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][g], bfr[cur][1], acc[g][1], 0, 0, 0);
                af[cur ^ 1][g] = frag(fa, 32 * g + (lane & 31), kc);
                if (g < 2) bfr[cur ^ 1][g] = frag(fa + kWTileA, brow[g] + (lane & 31), kc);
                if (s < 2) {
                    const int c = 5 * s + g;
                    dma_chunk(kA, bo, na, c);
                    if (g == 3) dma_chunk(kA, bo, na, c + 1);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    wide_epilogue<MODE>(p, ti, acc, smem);
}

template <int MODE, bool GROUPED>
__global__ __launch_bounds__(512, 1) void k_gemm_bf16_wide8(GemmParams p, int NT) {
    if (GROUPED != (p.offsets != nullptr)) return;  // launched with the matching instantiation only
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWSmem];
    const int total = total_tiles(p, NT);
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
    const int beg = (int)((long long)total * xcd / 8);
    const int end = (int)((long long)total * (xcd + 1) / 8);
    for (int L = beg + loc; L < end; L += per_xcd) {
        TileInfo ti;
        decode_tile(p, NT, BM, L, ti);
        gemm_tile_wide8<MODE>(p, ti, smem);
    }
}

// s_waitcnt immediate (gfx9 layout): vmcnt in bits 3:0 and 15:14, expcnt 6:4 (not waited for here),
// lgkmcnt 11:8.
constexpr unsigned waitcnt_imm(int vm, int lgkm) {
    return (unsigned)(vm & 15) | ((unsigned)((vm >> 4) & 3) << 14) | (7u << 4) | ((unsigned)(lgkm & 15) << 8);
}
static_assert(waitcnt_imm(63, 0) == 0xC07F, "vmcnt field layout");

// LDS hand-off without waiting for outstanding global loads: LDS-op wait plus workgroup barrier.
// The empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));   // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Tile order of the one-workgroup-per-CU GEMMs: all workgroups walk one window of gridDim.x
// consecutive tiles of the list at a time, and in it XCD x takes the x-th run of per_xcd consecutive
// tiles.  Inside an XCD the concurrently running tiles share operands through its L2 (blocked m/n
// order); across XCDs the window covers the same few experts at the same time, so what one XCD reads
// from HBM the others find in the shared last-level (infinity) cache, instead of eight XCDs streaming
// eight different experts' weights (more than that cache holds) and re-reading them from HBM.
__device__ __forceinline__ int window_tile(int xcd, int loc, int per_xcd) { return per_xcd * xcd + loc; }

// ---------------------------------------------------------------- 4-wave 128 x 512 tile
// Four waves (one per SIMD), each owning a 128 x 128 block of the 128 x 512 tile (4 x 4
// accumulators of 32 x 32 in the accumulator registers).  Per k-step each wave reads all 128 A
// rows and its own 128 B rows from LDS: 128 KB of fragment reads per workgroup, against 192 KB
// for eight waves of 128 x 64.  Operands are staged through registers: per k-step a wave loads
// 20 chunks of 1 KB (A chunks 4w .. 4w+3, B chunks 16w .. 16w+15) with 16-byte buffer loads for
// k-tile kt+2 while k-step kt computes, and stores them to the free LDS stage during k-step
// kt+1, so a load has a whole k-step to land and the only hand-off per k-step is an LDS-store
// wait plus barrier.
// SwiGLU: B rows [128 w, 128 w + 64) of the tile are gate rows n0 + 64 w + t and rows
// [128 w + 64, 128 w + 128) the matching up rows, so wave w produces output columns
// n0 + 64 w .. n0 + 64 w + 63 from accumulator pairs (j, j + 2).
constexpr int W4EPW = WBN + 4;   // non-SwiGLU staging row (512 outputs, 64 rows per pass)

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Buffer offset of a padding row: past every buffer these kernels address (spans stay below 2^31), so
// the load returns zeros.
constexpr unsigned kZeroRow = 0x80000000u;

// Buffer resource over [ptr, ptr + bytes) for 16-byte loads with a per-lane 32-bit byte offset and a
// wave-uniform scalar byte offset.  The base is made wave-uniform explicitly.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* ptr, int bytes) {
    const unsigned long long a = (unsigned long long)ptr;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((unsigned long long)hi << 32) | lo), (short)0, bytes,
                                             0x00020000);
}

// Epilogue of the four-wave 128 x 512 tile held as acc[i][j] (rows 32 i .., wave w's columns:
// SwiGLU gate blocks j = 0, 1 and the matching up blocks j = 2, 3 of outputs 64 w .., otherwise
// 128 w + 32 j): stage the fp32 values through LDS, then 16-byte stores of 8-column row pieces.
template <int MODE>
__device__ __forceinline__ void w4_epilogue(const GemmParams& p, const TileInfo& ti, f32x16 (&acc)[4][4],
                                            unsigned char* smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    float* st = reinterpret_cast<float*>(smem);
    if (MODE == GM_UP_SWIGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int rl = 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    st[rl * WEPW_SW + 64 * w + 32 * jj + (lane & 31)] = silu(acc[i][jj][q]) * acc[i][jj + 2][q];
                }
        __syncthreads();
        const int cq = (tid & 31) * 8;
        const int col0 = ti.nt * 256 + cq;
        if (col0 < p.N) {
            for (int rl = tid >> 5; rl < ti.rows; rl += 8) {
                const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * WEPW_SW + cq]);
                const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * WEPW_SW + cq + 4]);
                float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                epilogue_row<MODE>(p, ti, v, rl, col0);
            }
        }
        return;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // rows [64 h, 64 h + 64)
        if (h) __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int rl = 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    st[rl * W4EPW + 128 * w + 32 * j + (lane & 31)] = acc[2 * h + i][j][q];
                }
        __syncthreads();
        const int cq = lane * 8;
        const int col0 = ti.nt * WBN + cq;
        if (col0 < p.N) {
            for (int rl = w; rl < 64 && 64 * h + rl < ti.rows; rl += 4) {
                const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * W4EPW + cq]);
                const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * W4EPW + cq + 4]);
                float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                epilogue_row<MODE>(p, ti, v, 64 * h + rl, col0);
            }
        }
    }
}

template <int MODE>
__device__ __forceinline__ void gemm_tile_w4(const GemmParams& p, const TileInfo& ti, unsigned char* smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;   // w < 4

    // Operands are read with buffer loads: a constant per-lane byte offset per chunk and a scalar
    // k-step offset, so a k-step needs no vector address arithmetic.  A spans p.a_bytes and one
    // group's weights p.b_bytes (both below 2^31).
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.A, p.a_bytes);
    const __amdgpu_buffer_rsrc_t rsB =
        make_rsrc((const uint16_t*)p.B + (size_t)ti.g * p.sB_group, p.b_bytes);
    // 16-byte chunk permutation of a lane for chunk parity 0 / 1 (rows 8 i + lane / 8 of an
    // 8-row chunk whose first row is a multiple of 16 for even i)
    const int kcg0 = ((lane & 7) ^ ((lane >> 4) & 7)) * 8;
    const int kcg1 = ((lane & 7) ^ ((4 + (lane >> 4)) & 7)) * 8;
    unsigned voA[4];    // byte offset of A chunk 4w + i of this lane (k-tile 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * w + 8 * i + (lane >> 3);
        const int r = min(row, ti.rows - 1);
        long long src = ti.row0 + r;
        if (p.a_rows) src = min(max((long long)p.a_rows[src], 0LL), p.a_nrows - 1);
        const long long ga = p.offsets ? 0 : (long long)ti.g * p.sA_group;   // dense group's A offset
        voA[i] = row < ti.rows ? (unsigned)(src * p.lda + ga + ((i & 1) ? kcg1 : kcg0)) * 2u : kZeroRow;   // padding: zeros
    }
    unsigned voB[16];   // byte offset of B chunk 16w + i of this lane within the group's weights
    {
        const unsigned ldb = (unsigned)p.ldb;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            int wr;
            if (MODE == GM_UP_SWIGLU) {
                const int t = 64 * w + 8 * (i & 7) + (lane >> 3);
                wr = i < 8 ? min(ti.nt * 256 + t, p.N - 1) : p.up_off + min(ti.nt * 256 + t, p.N - 1);
            } else {
                wr = min(ti.nt * WBN + 128 * w + 8 * i + (lane >> 3), p.N - 1);
            }
            voB[i] = ((unsigned)wr * ldb + (unsigned)((i & 1) ? kcg1 : kcg0)) * 2u;
        }
    }
    const int la = (4 * w) * 1024 + lane * 16;              // A chunk 4w of this lane in a stage
    const int lb = kWTileA + (16 * w) * 1024 + lane * 16;   // B chunk 16w
    const int nk = p.K / BK;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    const int brow0 = 128 * w + (lane & 31);

    // staging registers: one named variable per chunk (an array of them is not kept in registers)
    v4u r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11, r12, r13, r14, r15, r16, r17, r18, r19;
#define MOE_W4_LD(C, RV)                                                             \
    RV = (C) < 4 ? __builtin_amdgcn_raw_buffer_load_b128(rsA, voA[(C) & 3], soA, 0) \
                 : __builtin_amdgcn_raw_buffer_load_b128(rsB, voB[((C) - 4) & 15], soB, 0)
#define MOE_W4_ST(D, C, RV) \
    *reinterpret_cast<v4u*>((D) + ((C) < 4 ? la + (C) * 1024 : lb + ((C) - 4) * 1024)) = RV
#define MOE_W4_ALL(OP)                                                                          \
    OP(0, r0); OP(1, r1); OP(2, r2); OP(3, r3); OP(4, r4); OP(5, r5); OP(6, r6); OP(7, r7);     \
    OP(8, r8); OP(9, r9); OP(10, r10); OP(11, r11); OP(12, r12); OP(13, r13); OP(14, r14);      \
    OP(15, r15); OP(16, r16); OP(17, r17); OP(18, r18); OP(19, r19)
#define MOE_W4_ST0(C, RV) MOE_W4_ST(smem, C, RV)
#define MOE_W4_SL(C, RV)     \
    case C:                  \
        MOE_W4_ST(na, C, RV); \
        MOE_W4_LD(C, RV);     \
        break
    // scalar byte offsets of the k-tile loaded next: A column kA, B offset (segment base + rem)
    int soA = 0, soB = 0, rem = 0, segb = 0;
    const int kseg2 = 2 * p.Kseg, sseg2 = (int)(2 * p.sB_seg);
    auto advance = [&]() {   // to the next k-tile
        soA += 2 * BK;
        rem += 2 * BK;
        if (rem == kseg2) {
            rem = 0;
            segb += sseg2;
        }
        soB = segb + rem;
    };

    __syncthreads();   // the previous tile's epilogue may still read the LDS staging area
    MOE_W4_ALL(MOE_W4_LD);
    MOE_W4_ALL(MOE_W4_ST0);
    if (nk > 1) advance();
    MOE_W4_ALL(MOE_W4_LD);
    lds_barrier();
    bf16x8 af[2][4], bfr[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = frag(smem, 32 * i + (lane & 31), lane >> 5);
#pragma unroll
    for (int j = 0; j < 4; ++j) bfr[0][j] = frag(smem + kWTileA, brow0 + 32 * j, lane >> 5);

    // k-step kt (stage b = kt & 1), four sub-steps of 16 MFMAs in 8 fenced groups of two; groups
    // 0-3 also issue two fragment reads for the next sub-step and, in sub-steps 0-2, groups 0-6
    // the LDS store of one chunk of k-tile kt+1 (registers -> stage b^1) followed by the global
    // load of the same chunk of k-tile kt+2.  LDS-store wait + barrier before sub-step 3, whose
    // fragment reads come from stage b^1.
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const unsigned char* sa = smem + buf * kWStage;
        unsigned char* na = smem + (buf ^ 1) * kWStage;
        if (kt + 2 < nk) advance();   // this k-step loads k-tile min(kt + 2, nk - 1)
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int cur = s & 1;
            if (s == 3) {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier();
            }
            const unsigned char* fa = s < 3 ? sa : na;
            const int kc = 2 * ((s + 1) & 3) + (lane >> 5);
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                // one wave per SIMD issues in order, and an MFMA waits for the matrix pipe: each
                // MFMA of the pair is followed by its own fenced window of other work (the chunk
                // staging after the first, the fragment read after the second), which issues while
                // that MFMA executes
                const int i = g >> 1, j0 = 2 * (g & 1);
                __builtin_amdgcn_sched_barrier(0);
                acc[i][j0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j0], acc[i][j0], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                const int c = 7 * s + g;   // chunk staged by this group
                if (s < 3 && g < 7 && c < 20) {
                    switch (c) { MOE_W4_ALL(MOE_W4_SL); }
                }
                __builtin_amdgcn_sched_barrier(0);
                acc[i][j0 + 1] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j0 + 1], acc[i][j0 + 1], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                // fragment reads for the next sub-step, all in the first four groups (their
                // registers were last read by the previous sub-step), so they have landed long
                // before the next sub-step's first MFMA
                if (g < 4) {
                    bfr[cur ^ 1][g] = frag(fa + kWTileA, brow0 + 32 * g, kc);
                    af[cur ^ 1][g] = frag(fa, 32 * g + (lane & 31), kc);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#undef MOE_W4_LD
#undef MOE_W4_ST
#undef MOE_W4_ALL
#undef MOE_W4_ST0
#undef MOE_W4_SL
    __syncthreads();

    // ---- epilogue: stage through LDS, 16-byte stores
    float* st = reinterpret_cast<float*>(smem);
    if (MODE == GM_UP_SWIGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int rl = 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    st[rl * WEPW_SW + 64 * w + 32 * jj + (lane & 31)] = silu(acc[i][jj][q]) * acc[i][jj + 2][q];
                }
        __syncthreads();
        const int cq = (tid & 31) * 8;
        const int col0 = ti.nt * 256 + cq;
        if (col0 < p.N) {
            for (int rl = tid >> 5; rl < ti.rows; rl += 8) {
                const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * WEPW_SW + cq]);
                const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * WEPW_SW + cq + 4]);
                float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                epilogue_row<MODE>(p, ti, v, rl, col0);
            }
        }
        return;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // rows [64 h, 64 h + 64)
        if (h) __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int rl = 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    st[rl * W4EPW + 128 * w + 32 * j + (lane & 31)] = acc[2 * h + i][j][q];
                }
        __syncthreads();
        const int cq = lane * 8;
        const int col0 = ti.nt * WBN + cq;
        if (col0 < p.N) {
            for (int rl = w; rl < 64 && 64 * h + rl < ti.rows; rl += 4) {
                const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * W4EPW + cq]);
                const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * W4EPW + cq + 4]);
                float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                epilogue_row<MODE>(p, ti, v, 64 * h + rl, col0);
            }
        }
    }
}

template <int MODE, bool GROUPED>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16_w4(GemmParams p, int NT) {
    if (GROUPED != (p.offsets != nullptr)) return;  // launched with the matching instantiation only
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWSmem];
    const int total = total_tiles(p, NT);
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
    for (int L = window_tile(xcd, loc, per_xcd); L < total; L += (int)gridDim.x) {
        TileInfo ti;
        decode_tile(p, NT, BM, L, ti);
        gemm_tile_w4<MODE>(p, ti, smem);
    }
}

// ---------------------------------------------------------------- packed weights
// The weights are static, so they can be stored once in the order the MFMA reads its B operand:
// for every 32-row block nb and 16-wide k-chunk kc of a group's [rows, K] matrix, one contiguous
// 1 KB fragment at block index nb * (K / 16) + kc, whose 16-byte piece l (l < 64) holds row
// 32 nb + l % 32, columns 16 kc + 8 (l / 32) .. + 7: exactly the eight bf16 lane l of a wave
// feeds to v_mfma_f32_32x32x16_bf16.  One 16-byte load per lane then fetches a whole fragment as
// 1 KB of consecutive bytes, straight into the registers the MFMA reads.
__global__ __launch_bounds__(256) void k_pack_b(const uint16_t* __restrict__ w, uint16_t* __restrict__ out,
                                                long long pieces, int N, int K) {
    const long long per = (long long)N * K / 8;   // 16-byte pieces per matrix
    const int kcn = K / 16;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < pieces; i += (long long)gridDim.x * 256) {
        const long long g = i / per;
        const long long r = i - g * per;
        const int l = (int)(r & 63);
        const long long blk = r >> 6;
        const long long nb = blk / kcn;
        const int kc = (int)(blk - nb * kcn);
        const long long n = nb * 32 + (l & 31);
        const int k = kc * 16 + (l >> 5) * 8;
        reinterpret_cast<uint4*>(out)[i] = *reinterpret_cast<const uint4*>(w + g * N * (long long)K + n * K + k);
    }
}

hipError_t launch_pack_b(const void* w, void* out, int G, int N, int K, hipStream_t s) {
    const long long pieces = (long long)G * N * K / 8;
    if (pieces == 0) return hipSuccess;
    long long nb = (pieces + 255) / 256;
    nb = nb < 8192 ? nb : 8192;
    hipLaunchKernelGGL(k_pack_b, dim3((unsigned)nb), dim3(256), 0, s, (const uint16_t*)w, (uint16_t*)out, pieces, N,
                       K);
    return hipGetLastError();
}

// ---------------------------------------------------------------- 4-wave 128 x 512 tile, packed weights
// Same tile and wave split as k_gemm_bf16_w4, but the weight operand is in fragment order: each wave
// loads its own 16 fragments per k-step (4 row blocks x 4 k-chunks, 16 KB) straight into registers,
// two k-steps ahead (two register sets), and never touches LDS for them.  Only the A tile, which all
// four waves read, goes through LDS: direct-to-LDS loads into a ring of four 16 KB stages, filled
// four k-steps ahead.  Per k-step a workgroup writes 16 KB and reads 64 KB of LDS (the register-staged
// kernel: 80 KB and 128 KB), and one barrier hands the ring over.
//
// Per k-step and wave, in issue order: B loads of k-step kt+2 for chunks 0, 1, 2 (four each, after
// the last MFMA reading that register), then in chunk 3: vmcnt wait + barrier, the B load of block 0,
// the four A loads of k-tile kt+4 into the stage k-step kt just finished reading, the B loads of
// blocks 1-3.  That is 20 vector-memory operations per k-step.
constexpr int kPStage = BM * BK * 2;   // 16 KB A stage
constexpr int kPStages = 4;
// NJ = 32-column weight blocks per wave: 4 (128 x 512 tile, one workgroup per CU) or 2 (128 x 256
// tile, two workgroups per CU, so that one's prologue and epilogue overlap the other's MFMAs).  A
// k-step issues 4 A loads and 4 NJ B loads.
// The A loads of k-tile kt+1 (issued in k-step kt-3, or in the prologue) must have landed when k-step
// kt starts reading them (chunk 3).  At that point at most this many vector-memory operations were
// issued after them: 11 NJ + 8 in k-step 0 (prologue order: A0..A3, B0, B1, then three chunks of
// B loads), 12 NJ + 7 in the steady state (NJ = 4: 52 and 55).
__host__ __device__ constexpr int p_wait_a(int nj) { return 11 * nj + 8; }
// prologue: A(0) has A1..A3 (12) and B0, B1 (8 NJ) issued after it
__host__ __device__ constexpr int p_wait_a0(int nj) { return 8 * nj + 12; }
// LDS of a packed-kernel workgroup: the A ring, reused for the bf16 staging of the output tile
__host__ __device__ constexpr int p_out_cols(int mode, int nj) { return mode == GM_UP_SWIGLU ? 64 * nj : 128 * nj; }
__host__ __device__ constexpr int p_smem(int mode, int nj) {
    return kPStages * kPStage > BM / 2 * (p_out_cols(mode, nj) + 16) * 4 ? kPStages * kPStage
                                                                          : BM / 2 * (p_out_cols(mode, nj) + 16) * 4;
}
static_assert(p_smem(GM_DOWN, 4) + kGroupTabBytes <= kWSmem && 2 * (p_smem(GM_DOWN, 2) + kGroupTabBytes) <= kWSmem,
              "A ring, staging and group table must fit");

// Epilogue of the packed kernel (grouped bf16 modes: SwiGLU, ReLU, down).  Each lane holds, for every
// 32 x 32 accumulator block, rows 8 (q / 4) + 4 (lane / 32) + q % 4 of column lane % 32; the values are
// finished in registers (SwiGLU, bias + ReLU) and rounded to bf16 two rows at a time (rows r and r+1 of
// one column in one 32-bit word), so the whole tile is staged in one pass at half the bytes of fp32:
// word [row pair][column].  Threads then read the words of 8 columns of a row pair, separate the two
// rows with byte permutes and store 16 bytes per row.  Row pairs are padded by 16 words, so the two
// half-waves of a staging write fall in disjoint LDS banks.
template <int MODE, int NJ>
__device__ __forceinline__ void w4p_epilogue(const GemmParams& p, const TileInfo& ti, f32x16 (&acc)[4][NJ],
                                             unsigned char* smem) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // lane values recomputed here, not kept live across the k-loop
    const int lane = tid & 63, w = tid >> 6;
    constexpr int OUTW = p_out_cols(MODE, NJ);                // output columns of the tile
    constexpr int SW = OUTW + 16;                            // staged words per row pair
    constexpr int NJO = MODE == GM_UP_SWIGLU ? NJ / 2 : NJ;   // output column blocks per wave
    static_assert(BM / 2 * SW * 4 <= p_smem(MODE, NJ), "bf16 staging must fit");
    uint32_t* st = reinterpret_cast<uint32_t*>(smem);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jb = 0; jb < NJO; ++jb) {
            const int cl = 32 * NJO * w + 32 * jb + (lane & 31);   // tile column
            float bias = 0.f;
            if (MODE == GM_UP_RELU && p.bias) {
                const int col = min(ti.nt * OUTW + cl, p.N - 1);
                bias = p.bias[(long long)ti.g * p.sbias_group + col];
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; b += 2) {
                    const int q = 4 * a + b;
                    float x0, x1;
                    if (MODE == GM_UP_SWIGLU) {
                        x0 = silu(acc[i][jb][q]) * acc[i][jb + NJO][q];
                        x1 = silu(acc[i][jb][q + 1]) * acc[i][jb + NJO][q + 1];
                    } else if (MODE == GM_UP_RELU) {
                        x0 = fmaxf(acc[i][jb][q] + bias, 0.0f);
                        x1 = fmaxf(acc[i][jb][q + 1] + bias, 0.0f);
                    } else {
                        x0 = acc[i][jb][q];
                        x1 = acc[i][jb][q + 1];
                    }
                    const int rp = 16 * i + 4 * a + 2 * (lane >> 5) + (b >> 1);   // (32 i + r) / 2
                    st[rp * SW + cl] = pack2_bf16(x0, x1);
                }
        }
    __syncthreads();
    constexpr int G = OUTW / 8;   // 8-column groups per row pair
    uint16_t* C = (uint16_t*)p.C;
    const long long coff = p.offsets ? 0 : (long long)ti.g * p.sC_group;   // dense groups side by side
    for (int it = tid; it < BM / 2 * G; it += 256) {
        const int rp = it / G, cg = it - rp * G;
        const int r0 = 2 * rp;
        const int col0 = ti.nt * OUTW + 8 * cg;
        if (r0 >= ti.rows || col0 >= p.N) continue;
        const uint4 x = *reinterpret_cast<const uint4*>(&st[rp * SW + 8 * cg]);
        const uint4 y = *reinterpret_cast<const uint4*>(&st[rp * SW + 8 * cg + 4]);
        uint4 lo, hi;   // row r0: low halves of the words, row r0 + 1: high halves
        lo.x = __builtin_amdgcn_perm(x.y, x.x, 0x05040100u);
        lo.y = __builtin_amdgcn_perm(x.w, x.z, 0x05040100u);
        lo.z = __builtin_amdgcn_perm(y.y, y.x, 0x05040100u);
        lo.w = __builtin_amdgcn_perm(y.w, y.z, 0x05040100u);
        hi.x = __builtin_amdgcn_perm(x.y, x.x, 0x07060302u);
        hi.y = __builtin_amdgcn_perm(x.w, x.z, 0x07060302u);
        hi.z = __builtin_amdgcn_perm(y.y, y.x, 0x07060302u);
        hi.w = __builtin_amdgcn_perm(y.w, y.z, 0x07060302u);
        const long long row = ti.row0 + r0;
        uint16_t* c = C + row * p.ldc + coff + col0;
        *reinterpret_cast<uint4*>(c) = lo;
        if (r0 + 1 < ti.rows) *reinterpret_cast<uint4*>(c + p.ldc) = hi;
    }
}

// A_FLAT: A spans 2 GiB or more, so its loads take 64-bit addresses (global_load_lds).  The compiler
// counts such a load as a possible LDS access as well, and then waits for every outstanding load
// (vmcnt(0)) before the next use of a loaded register: correct, but the B prefetch no longer
// overlaps.  Otherwise A uses buffer loads into LDS with 32-bit offsets, which keep the counts exact.
template <int MODE, bool A_FLAT, int NJ>
__device__ __forceinline__ void gemm_tile_w4p(const GemmParams& p, const TileInfo& ti, unsigned char* smem) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // per-tile lane values: not hoisted out of the tile loop
    const int lane = tid & 63, w = tid >> 6;   // w < 4
    const int nk = p.K / BK;
    const unsigned kcn = (unsigned)(p.K / 16);

    // B: the group's packed matrix; fragment (nb, kc) of this lane at (nb * kcn + kc) * 1024 + 16 lane
    const __amdgpu_buffer_rsrc_t rsB = make_rsrc((const uint16_t*)p.B + (size_t)ti.g * p.sB_group, p.b_bytes);
    unsigned voB[NJ];
    {
        const int nbl = p.N / 32 - 1;   // last row block of the output columns
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            int nb;
            if (MODE == GM_UP_SWIGLU) {   // gate blocks j < NJ / 2, the matching up blocks after them
                const int t = min(ti.nt * 2 * NJ + NJ / 2 * w + j % (NJ / 2), nbl);
                nb = j < NJ / 2 ? t : p.up_off / 32 + t;
            } else {
                nb = min(ti.nt * 4 * NJ + NJ * w + j, nbl);
            }
            voB[j] = (unsigned)nb * kcn * 1024u + (unsigned)lane * 16u;
        }
    }
    // A: wave w moves 1 KB chunks 4w + i (rows 32 w + 8 i .. + 7) of each k-tile; lane l of a chunk is
    // row 8c + l / 8, LDS slot l % 8, global chunk (l % 8) ^ ((row >> 1) & 7)
    const uint16_t* A = (const uint16_t*)p.A;
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.A, A_FLAT ? 0 : p.a_bytes);
    const uint16_t* ag[4];
    unsigned voA[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * w + 8 * i + (lane >> 3);
        const int kcg = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
        const int r = min(row, ti.rows - 1);
        long long src = ti.row0 + r;
        if (p.a_rows) src = min(max((long long)p.a_rows[src], 0LL), p.a_nrows - 1);
        ag[i] = A + src * p.lda + kcg;
        // padding rows of a group's last m-tile load zeros (an offset past the buffer reads 0): their
        // products are never stored, and zero operands cost the matrix cores less power
        voA[i] = A_FLAT ? 0u : (row < ti.rows ? (unsigned)(src * p.lda + kcg) * 2u : kZeroRow);
    }
    // A chunk i of k-tile column k (elements) into LDS chunk base dst
    // zero: OR-ed into the offset (kZeroRow or 0) of the k-tiles past the end that keep the issue
    // pattern uniform: they read zeros instead of fetching a k-tile again
    auto load_a = [&](int i, int k, unsigned char* dst, unsigned zero) {
        if (A_FLAT) dma16(ag[i] + k, dst);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_ptr_t)dst, 16, voA[i] | zero, 2 * k, 0, 0);
    };

    f32x16 acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    bf16x8 af[2][4];
    v4u bq[2][4][NJ];   // [k-step parity][chunk][row block]

    __syncthreads();   // the previous tile's epilogue may still read the LDS staging area
#pragma unroll
    for (int st = 0; st < kPStages; ++st) {
        const int k = min(st, nk - 1) * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) load_a(i, k, smem + st * kPStage + (4 * w + i) * 1024, st < nk ? 0u : kZeroRow);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                bq[t][s][j] = __builtin_amdgcn_raw_buffer_load_b128(rsB, voB[j] | (t < nk ? 0u : kZeroRow),
                                                                    min(t, nk - 1) * 4096 + s * 1024, 0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(p_wait_a0(NJ), 0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = frag(smem, 32 * i + (lane & 31), lane >> 5);

    auto kstep = [&](const int kt, auto setc) {
        constexpr int SET = decltype(setc)::value;
        unsigned char* sa = smem + (kt & 3) * kPStage;               // k-tile kt; refilled with kt+4
        const unsigned char* sn = smem + ((kt + 1) & 3) * kPStage;   // k-tile kt+1
        const int kb = min(kt + 2, nk - 1) * 4096;                   // B byte offset of k-tile kt+2
        const int ka = min(kt + 4, nk - 1) * BK;                     // A column of k-tile kt+4
        const unsigned zb = kt + 2 < nk ? 0u : kZeroRow, za = kt + 4 < nk ? 0u : kZeroRow;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s == 3) {
                // A(kt+1) landed for this wave, then for all (barrier); every wave is done reading
                // stage kt, which the A loads below refill
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(p_wait_a(NJ), 0));
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    __builtin_amdgcn_sched_barrier(0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        af[s & 1][i], __builtin_bit_cast(bf16x8, bq[SET][s][j]), acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (j == 0) {   // A fragments of the next chunk
                        if (s < 3) af[(s + 1) & 1][i] = frag(sa, 32 * i + (lane & 31), 2 * (s + 1) + (lane >> 5));
                        else af[0][i] = frag(sn, 32 * i + (lane & 31), lane >> 5);
                    }
                    if (s == 3 && j == 1) load_a(i, ka, sa + (4 * w + i) * 1024, za);
                    if (i == 3)
                        bq[SET][s][j] = __builtin_amdgcn_raw_buffer_load_b128(rsB, voB[j] | zb, kb + s * 1024, 0);
                }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        kstep(kt, std::integral_constant<int, 0>());
        kstep(kt + 1, std::integral_constant<int, 1>());
    }
    if (kt < nk) kstep(kt, std::integral_constant<int, 0>());
    // drain the trailing (clamped) loads before the LDS is reused for staging
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    w4p_epilogue<MODE, NJ>(p, ti, acc, smem);
}

// GROUPED: routed segments (group table in LDS); otherwise dense groups, every group over the rows
// [0, M_dense) (the shared experts).  Separate instantiations, so a profile tells them apart.
template <int MODE, bool A_FLAT, int NJ = 4, bool GROUPED = true>
__global__ __launch_bounds__(256, 4 / NJ) void k_gemm_bf16_w4p(GemmParams p, int NT) {
    if (GROUPED != (p.offsets != nullptr)) return;  // launched with the matching instantiation only
    __shared__ __attribute__((aligned(16))) unsigned char smem[p_smem(MODE, NJ) + kGroupTabBytes];
    int32_t* gt = reinterpret_cast<int32_t*>(smem + p_smem(MODE, NJ));
    if (GROUPED) load_group_tab(p.tiles, p.offsets, p.G, gt);
    const int total = GROUPED ? gt[p.G] * NT : total_tiles(p, NT);
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
    for (int L = window_tile(xcd, loc, per_xcd); L < total; L += (int)gridDim.x) {
        TileInfo ti;
        if (GROUPED) decode_tile_tab(gt, p.G, NT, BM, L, ti);
        else decode_tile(p, NT, BM, L, ti);
        gemm_tile_w4p<MODE, A_FLAT, NJ>(p, ti, smem);
    }
}

// ---------------------------------------------------------------- decode-shaped grouped GEMM
// Few rows per group (decode: a handful of tokens per expert) make the expert GEMMs a stream of
// weight bytes.  Tiles of 32 rows x 256 weight rows x 64 k; four waves, each 32 rows x 64 weight
// rows (two 32 x 32 blocks; SwiGLU: 32 gate rows and the 32 matching up rows).  Operands go
// straight to LDS (global_load_lds_dwordx4) through a ring of four 36 KB stages with three k-tiles
// in flight, one workgroup per CU: about 108 KB of loads in flight per CU, which is what keeps
// HBM busy here.  Each k-step: wait for this wave's loads of the k-tile (vmcnt), barrier, issue the
// loads of k-tile kt+3 into the stage k-step kt-1 used, then 8 MFMAs per wave.
constexpr int DBM = 32, DBN = 256, DSTAGES = 4;
constexpr int kDTileA = DBM * BK * 2;            // 4 KB
constexpr int kDStage = kDTileA + DBN * BK * 2;  // 36 KB
constexpr int kDSmem = DSTAGES * kDStage;        // 144 KB
constexpr int DEPW = DBN + 4;                    // fp32 staging row of the epilogue
static_assert(DBM * DEPW * 4 <= kDSmem, "decode epilogue staging must fit");

// PK: the weights are in fragment order (k_pack_b); wave w's eight B chunks are then the fragments of
// its two 32-row blocks j for the four k-chunks s (chunk 4 j + s), and LDS holds them in that order.
// W: waves per workgroup; the tile is 32 rows x 64 W weight rows, each wave owning 64 weight rows.
// W = 1 serves dense GEMMs of a few rows (the shared experts of a decode step), whose few 256-wide
// tiles would leave most CUs idle.
// NTB: weights are streamed with non-temporal loads.  Routed experts of a decode step are read by one
// m-tile each (rarely two, and those run side by side); streaming them past the caches reads HBM
// faster (V3 decode routed up GEMM 1.30 -> 1.23 ms).  Dense tiles re-read their weights once per
// m-tile, so they keep the default policy.
template <int MODE, bool PK, int W = 4, bool NTB = false>
__device__ __forceinline__ void gemm_tile_dec(const GemmParams& p, const TileInfo& ti, unsigned char* smem) {
    constexpr int TN = 64 * W;                         // weight rows of the tile
    constexpr int NA = 4 / W;                          // activation chunks (8 rows each) per wave
    constexpr int STAGE = kDTileA + TN * BK * 2;
    constexpr int STG = DSTAGES;                       // ring stages; STG - 1 k-tiles in flight
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;   // w < W
    const uint16_t* A = (const uint16_t*)p.A;
    const uint16_t* Bg = (const uint16_t*)p.B + (size_t)ti.g * p.sB_group;
    // chunk permutation of a lane (chunk c of LDS row r holds global chunk c ^ ((r >> 1) & 7))
    const int kcg0 = ((lane & 7) ^ ((lane >> 4) & 7)) * 8;
    const int kcg1 = ((lane & 7) ^ ((4 + (lane >> 4)) & 7)) * 8;
    // A chunks NA w + a: tile rows 8 (NA w + a) .. + 7
    const uint16_t* ag[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        const int c = NA * w + a;
        const int r = min(8 * c + (lane >> 3), ti.rows - 1);
        long long src = ti.row0 + r;
        if (p.a_rows) src = min(max((long long)p.a_rows[src], 0LL), p.a_nrows - 1);
        ag[a] = A + src * p.lda + ((c & 1) ? kcg1 : kcg0);
    }
    // B chunks 8 w + i: tile rows 64 w + 8 i .. + 7
    const uint16_t* bg[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (PK) {
            const int nbl = p.N / 32 - 1, j = i >> 2;
            int nb;
            if (MODE == GM_UP_SWIGLU) {
                const int t = min(ti.nt * (TN / 64) + w, nbl);
                nb = j ? p.up_off / 32 + t : t;
            } else {
                nb = min(ti.nt * (TN / 32) + 2 * w + j, nbl);
            }
            bg[i] = Bg + (((size_t)nb * (p.K / 16) + (i & 3)) * 64 + lane) * 8;
            continue;
        }
        int wr;
        if (MODE == GM_UP_SWIGLU) {
            const int t = 32 * w + 8 * (i & 3) + (lane >> 3);
            const int n = min(ti.nt * (TN / 2) + t, p.N - 1);
            wr = i < 4 ? n : p.up_off + n;
        } else {
            wr = min(ti.nt * TN + 64 * w + 8 * i + (lane >> 3), p.N - 1);
        }
        bg[i] = Bg + (size_t)wr * p.ldb + ((i & 1) ? kcg1 : kcg0);
    }
    const int nk = p.K / BK;
    auto issue = [&](int kt) {   // k-tile kt (< nk) into its stage
        const int k = kt * BK;
        const int seg = k / p.Kseg;
        // packed: a 64-wide k-tile is four consecutive 1 KB fragments (2048 elements) per row block
        const long long bo = PK ? (long long)k * 32 : (long long)seg * p.sB_seg + (k - seg * p.Kseg);
        unsigned char* st = smem + (kt % STG) * STAGE;
#pragma unroll
        for (int a = 0; a < NA; ++a) dma16(ag[a] + k, st + (NA * w + a) * 1024);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (NTB) dma16_nt(bg[i] + bo, st + kDTileA + (8 * w + i) * 1024);
            else dma16(bg[i] + bo, st + kDTileA + (8 * w + i) * 1024);
        }
    };

    f32x16 acc0, acc1;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        acc0[q] = 0.f;
        acc1[q] = 0.f;
    }
    __syncthreads();   // the previous tile's epilogue may still read the LDS staging area
#pragma unroll
    for (int u = 0; u < STG - 1; ++u)
        if (u < nk) issue(u);
    for (int kt = 0; kt < nk; ++kt) {
        // this wave's loads of k-tile kt have landed once at most the STG - 2 newer k-tiles (NA + 8
        // loads each) are outstanding; the barrier then covers every wave's loads and every wave's
        // reads of the stage k-step kt-1 used, which the next issue overwrites
        asm volatile("" ::: "memory");
        // k-tiles past the end are not issued, so near the end fewer newer loads can be outstanding
        static_assert(STG == 4, "the wait counts assume four stages");
        if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * (NA + 8), 0));
        else if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_imm(NA + 8, 0));
        else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + STG - 1 < nk) issue(kt + STG - 1);
        const unsigned char* sa = smem + (kt % STG) * STAGE;
        const unsigned char* sb = sa + kDTileA;
        // all twelve fragment reads of the k-step first, then the eight MFMAs: interleaved, each MFMA
        // pair waited for its own reads (one LDS round trip each), which a wave alone on its SIMD (the
        // one-wave tiles) cannot hide
        bf16x8 fa[BK / 16], fb0[BK / 16], fb1[BK / 16];
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int kc = 2 * s + (lane >> 5);
            fa[s] = frag(sa, lane & 31, kc);
            fb0[s] = PK ? *reinterpret_cast<const bf16x8*>(sb + (8 * w + s) * 1024 + lane * 16)
                        : frag(sb, 64 * w + (lane & 31), kc);
            fb1[s] = PK ? *reinterpret_cast<const bf16x8*>(sb + (8 * w + 4 + s) * 1024 + lane * 16)
                        : frag(sb, 64 * w + 32 + (lane & 31), kc);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s], fb0[s], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s], fb1[s], acc1, 0, 0, 0);
        }
    }
    // drain the trailing (clamped) loads before the LDS is reused for staging
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- epilogue: stage the 32 x 256 (SwiGLU: 32 x 128) fp32 tile, then 8-column row pieces
    float* st = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int rl = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (MODE == GM_UP_SWIGLU) {
            st[rl * DEPW + 32 * w + (lane & 31)] = silu(acc0[q]) * acc1[q];
        } else {
            st[rl * DEPW + 64 * w + (lane & 31)] = acc0[q];
            st[rl * DEPW + 64 * w + 32 + (lane & 31)] = acc1[q];
        }
    }
    __syncthreads();
    constexpr int OUTW = MODE == GM_UP_SWIGLU ? TN / 2 : TN;
    constexpr int TPR = OUTW / 8;       // threads per row
    constexpr int RPP = 64 * W / TPR;   // rows per pass
    const int cq = (tid % TPR) * 8;
    const int col0 = ti.nt * OUTW + cq;
    if (col0 >= p.N) return;
    for (int rl = tid / TPR; rl < ti.rows; rl += RPP) {
        const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * DEPW + cq]);
        const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * DEPW + cq + 4]);
        float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        epilogue_row<MODE>(p, ti, v, rl, col0);
    }
}

// Grouped: tiles over the 32-row tile prefix; dense (a few tokens through the shared experts): every
// group covers rows [0, M_dense) in 32-row tiles.
template <int MODE, bool GROUPED, bool PK = false, int W = 4>
__global__ __launch_bounds__(64 * W) void k_gemm_bf16_dec(GemmParams p, int NT) {
    if (GROUPED != (p.offsets != nullptr)) return;  // launched with the matching instantiation only
    constexpr int SMEM = DSTAGES * (kDTileA + 64 * W * BK * 2);
    static_assert(DBM * DEPW * 4 <= SMEM, "decode epilogue staging must fit");
    static_assert(SMEM + kGroupTabBytes <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM + (GROUPED ? kGroupTabBytes : 0)];
    int32_t* gt = reinterpret_cast<int32_t*>(smem + SMEM);
    if (GROUPED) load_group_tab(p.tiles32, p.offsets, p.G, gt);
    const int nmd = (p.M_dense + DBM - 1) / DBM;     // dense: m-tiles per group
    const int total = GROUPED ? gt[p.G] * NT : p.G * nmd * NT;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
    const int beg = (int)((long long)total * xcd / 8);
    const int end = (int)((long long)total * (xcd + 1) / 8);
    for (int L = beg + loc; L < end; L += per_xcd) {
        TileInfo ti;
        int ml;
        if (GROUPED) {
            decode_tile_tab(gt, p.G, NT, DBM, L, ti);
        } else {
            const int per = nmd * NT;
            ti.g = L / per;
            blocked_mn(L - ti.g * per, nmd, NT, ml, ti.nt);
            ti.row0 = ml * DBM;
            ti.rows = min(DBM, p.M_dense - ti.row0);
        }
        gemm_tile_dec<MODE, PK, W, GROUPED>(p, ti, smem);
    }
}

__device__ __forceinline__ int wide_nt(const GemmParams& p, int mode) {
    return mode == GM_UP_SWIGLU ? (p.N + 255) / 256 : (p.N + WBN - 1) / WBN;
}

// ---------------------------------------------------------------- fp32 VALU path
// One thread per (row, output column).  Row r of the row space belongs to the group found by
// binary search in offsets (grouped) or to blockIdx.z (dense).
__device__ __forceinline__ int group_of_row(const int32_t* offsets, int G, int r) {
    int lo = 0, hi = G;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= r) lo = mid;
        else hi = mid;
    }
    return lo;
}

template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmParams p) {
    const int col = blockIdx.x * 64 + (threadIdx.x & 63);
    const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (col >= p.N) return;
    int g;
    long long rowC;
    if (p.offsets) {
        if (r >= p.offsets[p.G]) return;
        g = group_of_row(p.offsets, p.G, r);
        rowC = r;
    } else {
        if (r >= p.M_dense) return;
        g = blockIdx.z;
        rowC = r;
    }
    long long src = r;
    if (p.a_rows) src = min(max((long long)p.a_rows[r], 0LL), p.a_nrows - 1);
    const float* a = (const float*)p.A + src * p.lda;
    const float* Bg = (const float*)p.B + (size_t)g * p.sB_group;
    float* C = (float*)p.C + rowC * p.ldc + (p.offsets ? 0 : (long long)g * p.sC_group);
    if (MODE == GM_UP_SWIGLU) {
        const float* wg = Bg + (size_t)col * p.ldb;
        const float* wu = Bg + (size_t)(p.up_off + col) * p.ldb;
        float zg = 0.f, zu = 0.f;
        for (int k = 0; k < p.K; ++k) {
            zg = fmaf(a[k], wg[k], zg);
            zu = fmaf(a[k], wu[k], zu);
        }
        C[col] = zg / (1.0f + expf(-zg)) * zu;
    } else {
        float z = 0.f;
        for (int k = 0; k < p.K; ++k) {
            const int seg = k / p.Kseg;
            z = fmaf(a[k], Bg[(long long)seg * p.sB_seg + (size_t)col * p.ldb + (k - seg * p.Kseg)], z);
        }
        if (MODE == GM_UP_RELU) {
            if (p.bias) z += p.bias[(long long)g * p.sbias_group + col];
            z = fmaxf(z, 0.0f);
        }
        C[col] = z;
    }
}

hipError_t launch_gemm(int dtype, int mode, const GemmParams& p_in, hipStream_t s) {
    GemmParams p = p_in;
    if (p.G == 0 || p.max_rows == 0 || p.N == 0) return hipSuccess;
    {
        // byte spans for 32-bit buffer offsets: A rows reachable by the row space, one group's weights
        const long long a_rows_n = p.a_rows ? p.a_nrows : (p.offsets ? (long long)p.max_rows : (long long)p.M_dense);
        const long long a_span = a_rows_n * p.lda * 2;
        const long long b_rows = mode == GM_UP_SWIGLU ? (long long)p.up_off + p.N : (long long)p.N;
        const long long b_span = ((long long)(p.K / (p.Kseg > 0 ? p.Kseg : 1)) - 1) * p.sB_seg * 2 + b_rows * p.ldb * 2;
        const long long lim = 0x7FFFFFF0LL;
        p.a_bytes = a_span > 0 && a_span < lim ? (int)a_span : 0;
        p.b_bytes = b_span > 0 && b_span < lim ? (int)b_span : 0;
    }
    if (dtype == 0) {
        if (mode == GM_DOWN_COMBINE || mode == GM_F32OUT || p.packed) return hipErrorInvalidValue;  // bf16 only
        dim3 grid((p.N + 63) / 64, (p.max_rows + 3) / 4, p.offsets ? 1 : p.G);
        if (mode == GM_UP_SWIGLU) hipLaunchKernelGGL(k_gemm_f32<GM_UP_SWIGLU>, grid, dim3(256), 0, s, p);
        else if (mode == GM_UP_RELU) hipLaunchKernelGGL(k_gemm_f32<GM_UP_RELU>, grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL(k_gemm_f32<GM_DOWN>, grid, dim3(256), 0, s, p);
        return hipGetLastError();
    }
    if (mode == GM_DOWN_COMBINE && p.offsets) return hipErrorInvalidValue;  // dense (shared) groups only
    const long long cus = device_cus();
    if (p.packed) {
        // fragment-order weights: grouped (routed) or dense (shared, all groups on the same rows) up/down
        // GEMMs, one K segment, 32-bit offsets
        if ((p.offsets && !p.tiles32) || (!p.offsets && p.sA_group != 0) || p.Kseg != p.K || p.b_bytes == 0 ||
            p.N % 32 || !(mode == GM_UP_SWIGLU || mode == GM_UP_RELU || mode == GM_DOWN))
            return hipErrorInvalidValue;
        if (!p.offsets && p.M_dense < 512) {
            // a few dense rows (the shared experts of a decode step): 32-row tiles
            const int NTd = mode == GM_UP_SWIGLU ? (p.N + DBN / 2 - 1) / (DBN / 2) : (p.N + DBN - 1) / DBN;
            const long long mtd = (long long)p.G * ((p.M_dense + DBM - 1) / DBM);
            if (mtd * NTd < cus) {   // one-wave workgroups of 64 weight rows, three per CU
                const int NT1 = mode == GM_UP_SWIGLU ? (p.N + 31) / 32 : (p.N + 63) / 64;
                long long nb1 = mtd * NT1;
                nb1 = nb1 < 3 * cus ? nb1 : 3 * cus;
                const dim3 grid1((unsigned)((nb1 + 7) / 8 * 8));
                if (mode == GM_UP_SWIGLU) hipLaunchKernelGGL((k_gemm_bf16_dec<GM_UP_SWIGLU, false, true, 1>), grid1, dim3(64), 0, s, p, NT1);
                else if (mode == GM_UP_RELU) hipLaunchKernelGGL((k_gemm_bf16_dec<GM_UP_RELU, false, true, 1>), grid1, dim3(64), 0, s, p, NT1);
                else hipLaunchKernelGGL((k_gemm_bf16_dec<GM_DOWN, false, true, 1>), grid1, dim3(64), 0, s, p, NT1);
                return hipGetLastError();
            }
            long long nb = (mtd * NTd + 7) / 8 * 8;
            nb = nb < cus ? nb : cus;
            const dim3 grid((unsigned)((nb + 7) / 8 * 8));
            if (mode == GM_UP_SWIGLU) hipLaunchKernelGGL((k_gemm_bf16_dec<GM_UP_SWIGLU, false, true>), grid, dim3(256), 0, s, p, NTd);
            else if (mode == GM_UP_RELU) hipLaunchKernelGGL((k_gemm_bf16_dec<GM_UP_RELU, false, true>), grid, dim3(256), 0, s, p, NTd);
            else hipLaunchKernelGGL((k_gemm_bf16_dec<GM_DOWN, false, true>), grid, dim3(256), 0, s, p, NTd);
            return hipGetLastError();
        }
        const long long rpg = p.offsets ? p.max_rows / p.G : p.M_dense;
        if (rpg < 64) {   // decode-sized groups: 32-row tiles, deep direct-to-LDS pipeline
            const int NTd = mode == GM_UP_SWIGLU ? (p.N + DBN / 2 - 1) / (DBN / 2) : (p.N + DBN - 1) / DBN;
            const long long mtd = (p.max_rows + DBM - 1) / DBM + p.G;
            long long nb = (mtd * NTd + 7) / 8 * 8;
            nb = nb < cus ? nb : cus;
            const dim3 grid((unsigned)((nb + 7) / 8 * 8));
            if (mode == GM_UP_SWIGLU) hipLaunchKernelGGL((k_gemm_bf16_dec<GM_UP_SWIGLU, true, true>), grid, dim3(256), 0, s, p, NTd);
            else if (mode == GM_UP_RELU) hipLaunchKernelGGL((k_gemm_bf16_dec<GM_UP_RELU, true, true>), grid, dim3(256), 0, s, p, NTd);
            else hipLaunchKernelGGL((k_gemm_bf16_dec<GM_DOWN, true, true>), grid, dim3(256), 0, s, p, NTd);
            return hipGetLastError();
        }
        // reductions of at most 8 k-steps: 128 x 256 tiles, two workgroups per CU, so that one's prologue
        // and epilogue (as long as its k-loop here) overlap the other's MFMAs; longer ones lose more to the
        // doubled activation traffic than they gain
        const int nj = p.K <= 512 ? 2 : 4;
        const int NTp = (p.N + p_out_cols(mode, nj) - 1) / p_out_cols(mode, nj);
        const long long mtp = p.offsets ? (p.max_rows + BM - 1) / BM + p.G
                                        : (long long)p.G * ((p.M_dense + BM - 1) / BM);
        long long nb = (mtp * NTp + 7) / 8 * 8;
        const long long slots = nj == 2 ? 2 * cus : cus;
        nb = nb < slots ? nb : slots;
        const dim3 grid((unsigned)((nb + 7) / 8 * 8));
#define MOE_LAUNCH_P4(M, NJ, GR)                                                                                   \
    do {                                                                                                           \
        if (p.a_bytes > 0) hipLaunchKernelGGL((k_gemm_bf16_w4p<M, false, NJ, GR>), grid, dim3(256), 0, s, p, NTp); \
        else hipLaunchKernelGGL((k_gemm_bf16_w4p<M, true, NJ, GR>), grid, dim3(256), 0, s, p, NTp);                \
    } while (0)
#define MOE_LAUNCH_P(M)                                         \
    do {                                                        \
        if (p.offsets) {                                        \
            if (nj == 2) MOE_LAUNCH_P4(M, 2, true);             \
            else MOE_LAUNCH_P4(M, 4, true);                     \
        } else {                                                \
            if (nj == 2) MOE_LAUNCH_P4(M, 2, false);            \
            else MOE_LAUNCH_P4(M, 4, false);                    \
        }                                                       \
    } while (0)
        if (mode == GM_UP_SWIGLU) MOE_LAUNCH_P(GM_UP_SWIGLU);
        else if (mode == GM_UP_RELU) MOE_LAUNCH_P(GM_UP_RELU);
        else MOE_LAUNCH_P(GM_DOWN);
#undef MOE_LAUNCH_P
#undef MOE_LAUNCH_P4
        return hipGetLastError();
    }
    long long mt;  // upper bound of the m-tile count (grouped: sum of ceil(rows_g / BM) <= R / BM + G)
    if (p.offsets) mt = (p.max_rows + BM - 1) / BM + p.G;
    else mt = (long long)p.G * ((p.M_dense + BM - 1) / BM);
    const int NTw = mode == GM_UP_SWIGLU ? (p.N + 255) / 256 : (p.N + WBN - 1) / WBN;
    // the 128 x 512 tile pays off only with many rows per group (prefill); decode-sized groups
    // (a few rows per expert) stream their weights better through the 128 x 128 tile
    const long long rows_per_group = p.offsets ? p.max_rows / (p.G > 0 ? p.G : 1) : p.M_dense;
    // buffer-load kernel: the plain modes and fp32 output (its epilogue is the shared per-row one);
    // direct-to-LDS kernel: the plain modes, for operands too large for 32-bit buffer offsets.
    // The fused combine stays on the 128 x 128 tiles: its epilogue gathers K_r routed rows per
    // output row, and two workgroups per CU overlap that gather with the other's MFMAs.
    const bool w4 = p.a_bytes > 0 && p.b_bytes > 0;
    // fp32 output (router logits) with whole 512-wide column tiles takes it from one tile per CU on: the
    // 128 x 128 kernel's single-stage k-loop is slower than the wide tile's at any count
    const bool wide = mode != GM_DOWN_COMBINE && (w4 || mode != GM_F32OUT) &&
                      (mt * NTw >= 2 * cus || (mode == GM_F32OUT && p.N % WBN == 0 && mt * NTw >= cus)) &&
                      rows_per_group >= 64;
    if (wide) {
        // persistent grid: one workgroup per CU (the two operand stages fill the LDS)
        long long nb = (mt * NTw + 7) / 8 * 8;
        nb = nb < cus ? nb : cus;
        nb = (nb + 7) / 8 * 8;
        const dim3 grid((unsigned)nb);
        if (w4) {
#define MOE_LAUNCH_W4(M)                                                                        \
    do {                                                                                        \
        if (p.offsets) hipLaunchKernelGGL((k_gemm_bf16_w4<M, true>), grid, dim3(256), 0, s, p, NTw); \
        else hipLaunchKernelGGL((k_gemm_bf16_w4<M, false>), grid, dim3(256), 0, s, p, NTw);    \
    } while (0)
            if (mode == GM_UP_SWIGLU) MOE_LAUNCH_W4(GM_UP_SWIGLU);
            else if (mode == GM_UP_RELU) MOE_LAUNCH_W4(GM_UP_RELU);
            else if (mode == GM_DOWN) MOE_LAUNCH_W4(GM_DOWN);
            else hipLaunchKernelGGL((k_gemm_bf16_w4<GM_F32OUT, false>), grid, dim3(256), 0, s, p, NTw);
#undef MOE_LAUNCH_W4
            return hipGetLastError();
        }
#define MOE_LAUNCH_W(M)                                                                                  \
    do {                                                                                                 \
        if (p.offsets) hipLaunchKernelGGL((k_gemm_bf16_wide8<M, true>), grid, dim3(512), 0, s, p, NTw); \
        else hipLaunchKernelGGL((k_gemm_bf16_wide8<M, false>), grid, dim3(512), 0, s, p, NTw);    \
    } while (0)
        if (mode == GM_UP_SWIGLU) MOE_LAUNCH_W(GM_UP_SWIGLU);
        else if (mode == GM_UP_RELU) MOE_LAUNCH_W(GM_UP_RELU);
        else MOE_LAUNCH_W(GM_DOWN);
#undef MOE_LAUNCH_W
        return hipGetLastError();
    }
    // decode-shaped: 32-row tiles, deep load pipeline, one workgroup per CU.  Grouped problems with few
    // rows per group, and dense ones with few rows (the shared experts of a decode step, including the
    // fused combine).  Every GEMM kernel here accumulates an output in the same order (one fp32 MFMA
    // chain over ascending 16-deep k-chunks), so the choice does not change any result bit.
    const bool dec_grouped = p.offsets && p.tiles32 && rows_per_group < 64 &&
                             (mode == GM_UP_SWIGLU || mode == GM_UP_RELU || mode == GM_DOWN);
    const bool dec_dense = !p.offsets && p.M_dense < 512 && mode != GM_F32OUT;
    if (dec_grouped || dec_dense) {
        const int NTd = mode == GM_UP_SWIGLU ? (p.N + DBN / 2 - 1) / (DBN / 2) : (p.N + DBN - 1) / DBN;
        const long long mtd = p.offsets ? (p.max_rows + DBM - 1) / DBM + p.G   // upper bound of the m-tiles
                                        : (long long)p.G * ((p.M_dense + DBM - 1) / DBM);
        long long nb = (mtd * NTd + 7) / 8 * 8;
        nb = nb < cus ? nb : cus;
        const dim3 grid((unsigned)((nb + 7) / 8 * 8));
#define MOE_LAUNCH_D(M)                                                                          \
    do {                                                                                         \
        if (p.offsets) hipLaunchKernelGGL((k_gemm_bf16_dec<M, true>), grid, dim3(256), 0, s, p, NTd); \
        else hipLaunchKernelGGL((k_gemm_bf16_dec<M, false>), grid, dim3(256), 0, s, p, NTd);    \
    } while (0)
        if (dec_dense && mtd * NTd < cus) {
            // few rows and few 256-wide tiles: one-wave workgroups of 64 weight rows, several per CU
            const int NT1 = mode == GM_UP_SWIGLU ? (p.N + 31) / 32 : (p.N + 63) / 64;
            long long nb1 = mtd * NT1;
            nb1 = nb1 < 3 * cus ? nb1 : 3 * cus;   // three 48 KB workgroups per CU
            const dim3 grid1((unsigned)((nb1 + 7) / 8 * 8));
            if (mode == GM_UP_SWIGLU) hipLaunchKernelGGL((k_gemm_bf16_dec<GM_UP_SWIGLU, false, false, 1>), grid1, dim3(64), 0, s, p, NT1);
            else if (mode == GM_UP_RELU) hipLaunchKernelGGL((k_gemm_bf16_dec<GM_UP_RELU, false, false, 1>), grid1, dim3(64), 0, s, p, NT1);
            else if (mode == GM_DOWN) hipLaunchKernelGGL((k_gemm_bf16_dec<GM_DOWN, false, false, 1>), grid1, dim3(64), 0, s, p, NT1);
            else hipLaunchKernelGGL((k_gemm_bf16_dec<GM_DOWN_COMBINE, false, false, 1>), grid1, dim3(64), 0, s, p, NT1);
            return hipGetLastError();
        }
        if (mode == GM_UP_SWIGLU) MOE_LAUNCH_D(GM_UP_SWIGLU);
        else if (mode == GM_UP_RELU) MOE_LAUNCH_D(GM_UP_RELU);
        else if (mode == GM_DOWN) MOE_LAUNCH_D(GM_DOWN);
        else hipLaunchKernelGGL((k_gemm_bf16_dec<GM_DOWN_COMBINE, false>), grid, dim3(256), 0, s, p, NTd);
#undef MOE_LAUNCH_D
        return hipGetLastError();
    }
    const int NT = mode == GM_UP_SWIGLU ? (p.N + 63) / 64 : (p.N + BN - 1) / BN;
    // persistent grid: two workgroups per CU (LDS and registers allow two), a multiple of 8
    long long nb = 2LL * cus;
    const long long need = (mt * NT + 7) / 8 * 8;
    nb = nb < need ? nb : need;
    nb = (nb + 7) / 8 * 8;
#define MOE_LAUNCH_N(M)                                                                                  \
    do {                                                                                                 \
        if (p.offsets) hipLaunchKernelGGL((k_gemm_bf16<M, true>), dim3((unsigned)nb), dim3(256), 0, s, p, NT); \
        else hipLaunchKernelGGL((k_gemm_bf16<M, false>), dim3((unsigned)nb), dim3(256), 0, s, p, NT);    \
    } while (0)
    if (mode == GM_UP_SWIGLU) MOE_LAUNCH_N(GM_UP_SWIGLU);
    else if (mode == GM_UP_RELU) MOE_LAUNCH_N(GM_UP_RELU);
    else if (mode == GM_DOWN) MOE_LAUNCH_N(GM_DOWN);
    else if (mode == GM_F32OUT) hipLaunchKernelGGL((k_gemm_bf16<GM_F32OUT, false>), dim3((unsigned)nb), dim3(256), 0, s, p, NT);
    else hipLaunchKernelGGL((k_gemm_bf16<GM_DOWN_COMBINE, false>), dim3((unsigned)nb), dim3(256), 0, s, p, NT);
#undef MOE_LAUNCH_N
    return hipGetLastError();
}

}  // namespace moe
