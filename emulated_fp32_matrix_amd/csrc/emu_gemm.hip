// GEMM kernels for gfx950: the emulated-FP32 GEMM on bf16 MFMA (nine, six or
// three products) and the native FP32-MFMA GEMM it is compared with.
//
// Method: "Unlocking Tensor Core Performance for Machine Learning Interatomic
// Potentials", section "How Tensor Core FP32 bridges the hardware gap",
// Figure 1 (three scaled BF16 pieces per operand, nine pairwise products
// accumulated in FP32 along five anti-diagonal bands, recombined with their
// scales) and Figure 2 (a reduced variant keeps only the largest products).
//
// Design (MI355X-first):
//   * Persistent launch: one 256-thread workgroup per CU walks a static list
//     of 128x128 output tiles; the k-loop of consecutive tiles forms one
//     software pipeline, so the next tile's first loads overlap the current
//     tile's last MFMAs and its epilogue.
//   * Tile order is XCD-aware: workgroup b runs on XCD b % 8, and the
//     workgroups of one XCD take consecutive tiles (n fastest), so the rows of
//     A that a group of tiles shares stay in that XCD's L2.
//   * The split is fused into the global->LDS staging: each thread loads 16
//     FP32 values with coalesced loads, splits them in registers and writes
//     the BF16 planes (hi, mid', lo') to LDS, k-contiguous, rows padded to 80
//     bytes so the 16-byte MFMA-operand reads are bank-conflict free.
//   * Each wave owns a 64x64 block of C as 2x2 tiles of v_mfma_f32_32x32x16_bf16
//     and keeps one FP32 accumulator per band per tile (5 x 4 x 16 registers
//     in the nine-product mode).  Products are issued smallest band first.
//   * Epilogue: bands are recombined smallest first (t = S_{n-1},
//     t = S_j + 2^-8 t) and C = alpha t + beta C is stored; C is not read when
//     beta == 0.
#include "emu_device.h"
#include "emu_launch.h"

namespace emu {
namespace {

constexpr int BK = 32;
constexpr int LDS_ROW = BK + 8;    // bf16 elements per LDS row (80 bytes)
constexpr int LDSF_ROW = BK + 4;   // fp32 elements per LDS row (144 bytes)

struct Params {
    const float* A;
    const float* B;
    float* C;
    int64_t lda, ldb, ldc;
    int64_t M, N, K;
    float alpha, beta;
    int tiles_n;
    int ntiles;
    int nk;
    int vec_a, vec_b;  // 16-byte loads allowed on this operand
};

// Bijection on [0, G): hardware workgroup id -> position in the tile list,
// such that the workgroups resident on one XCD (id % 8 equal) take a
// contiguous range of positions.
__device__ __forceinline__ int xcd_position(int b, int G)
{
    const int q = G >> 3, r = G & 7;
    const int x = b & 7, s = b >> 3;
    return x * q + (x < r ? x : r) + s;
}

// Tile geometry: WM x WN waves, each owning TM x TN tiles of 32x32.
template <int WM_, int WN_, int TM_, int TN_>
struct Geo {
    static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
    static constexpr int NT = 64 * WM * WN;      // threads
    static constexpr int BM = WM * TM * 32;
    static constexpr int BN = WN * TN * 32;
    static constexpr int RPP = NT / 8;           // tile rows covered per load pass
};

// A thread's share of one BK-wide tile of an operand viewed as [rows][k]:
// ROWS/RPP rows, four consecutive k each.
//   k-contiguous storage (KC): rows t/8 + RPP*q, k offset (t%8)*4 -- eight
//     lanes read one 128-byte row segment with 16-byte loads;
//   row-contiguous storage: rows t%RPP + RPP*q, k offset (t/RPP)*4 -- a
//     wave reads 64 consecutive floats of one k row per load.
template <int ROWS, int RPP>
struct RegTile {
    static constexpr int P = ROWS / RPP;
    float v[P][4];
};

template <bool KC, int RPP>
__device__ __forceinline__ int tile_row(int t, int q)
{
    return KC ? ((t >> 3) + RPP * q) : ((t % RPP) + RPP * q);
}

template <bool KC, int RPP>
__device__ __forceinline__ int tile_k(int t)
{
    return KC ? ((t & 7) * 4) : ((t / RPP) * 4);
}

template <bool KC, int ROWS, int RPP>
__device__ __forceinline__ void load_tile(RegTile<ROWS, RPP>& rt, const float* __restrict__ X,
                                          int64_t ld, int64_t rows, int64_t K, int64_t row0,
                                          int64_t k0, bool vec)
{
    const int t = threadIdx.x;
    const int kk = tile_k<KC, RPP>(t);
    const int64_t gk = k0 + kk;
    // Uniform tile base plus a 32-bit per-lane offset.
    const float* base = KC ? X + row0 * ld + k0 : X + k0 * ld + row0;
    const bool interior = row0 + ROWS <= rows && k0 + BK <= K;
#pragma unroll
    for (int q = 0; q < RegTile<ROWS, RPP>::P; ++q) {
        const int r = tile_row<KC, RPP>(t, q);
        const int64_t gr = row0 + r;
        if (KC) {
            const uint32_t off = (uint32_t)(r * ld + kk);
            if (vec && (interior || (gr < rows && gk + 3 < K))) {
                const f32x4_t v = *reinterpret_cast<const f32x4_t*>(base + off);
                rt.v[q][0] = v[0];
                rt.v[q][1] = v[1];
                rt.v[q][2] = v[2];
                rt.v[q][3] = v[3];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rt.v[q][e] = (gr < rows && gk + e < K) ? base[off + e] : 0.0f;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t off = (uint32_t)((kk + e) * ld + r);
                rt.v[q][e] = (interior || (gr < rows && gk + e < K)) ? base[off] : 0.0f;
            }
        }
    }
}

// Split a register tile and write its NP BF16 planes (plane stride PS
// elements) to LDS.
template <bool KC, int NP, int PS, int ROWS, int RPP>
__device__ __forceinline__ void store_tile_bf16(uint16_t* __restrict__ lds,
                                                const RegTile<ROWS, RPP>& rt)
{
    const int t = threadIdx.x;
    const int kk = tile_k<KC, RPP>(t);
#pragma unroll
    for (int q = 0; q < RegTile<ROWS, RPP>::P; ++q) {
        const int off = tile_row<KC, RPP>(t, q) * LDS_ROW + kk;
        uint32_t h0, m0, l0, h1, m1, l1;
        if (NP == 3) {
            split_pair<true>(rt.v[q][0], rt.v[q][1], h0, m0, l0);
            split_pair<true>(rt.v[q][2], rt.v[q][3], h1, m1, l1);
        } else {
            split_pair_hm(rt.v[q][0], rt.v[q][1], h0, m0);
            split_pair_hm(rt.v[q][2], rt.v[q][3], h1, m1);
        }
        *reinterpret_cast<u32x2_t*>(lds + off) = u32x2_t{h0, h1};
        *reinterpret_cast<u32x2_t*>(lds + PS + off) = u32x2_t{m0, m1};
        if (NP == 3) *reinterpret_cast<u32x2_t*>(lds + 2 * PS + off) = u32x2_t{l0, l1};
    }
}

template <bool KC, int ROWS, int RPP>
__device__ __forceinline__ void store_tile_f32(float* __restrict__ lds, const RegTile<ROWS, RPP>& rt)
{
    const int t = threadIdx.x;
    const int kk = tile_k<KC, RPP>(t);
#pragma unroll
    for (int q = 0; q < RegTile<ROWS, RPP>::P; ++q) {
        const int off = tile_row<KC, RPP>(t, q) * LDSF_ROW + kk;
        *reinterpret_cast<f32x4_t*>(lds + off) =
            f32x4_t{rt.v[q][0], rt.v[q][1], rt.v[q][2], rt.v[q][3]};
    }
}

// Origin of the tile at position `pos` of the tile list.
__device__ __forceinline__ void tile_coords(const Params& p, int pos, int bm, int bn, int64_t& m0,
                                            int64_t& n0)
{
    const int tm = pos / p.tiles_n;
    m0 = (int64_t)tm * bm;
    n0 = (int64_t)(pos - tm * p.tiles_n) * bn;
}

// Store one 32x32 MFMA tile of results: lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the tile.
__device__ __forceinline__ void store_c_tile(const Params& p, const float (&t)[16], int64_t row0,
                                             int64_t col0)
{
    const int lane = threadIdx.x & 63;
    const int64_t col = col0 + (lane & 31);
    if (col >= p.N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < p.M) {
            float* c = p.C + row * p.ldc + col;
            float out = p.alpha * t[r];
            if (p.beta != 0.0f) out = __builtin_fmaf(p.beta, *c, out);
            *c = out;
        }
    }
}

// The emulated GEMM.  NB = bands kept: 5 (nine products), 3 (six), 2 (three).
// Loop structure: for each tile of this workgroup, for each BK step of K:
// MFMAs on the current LDS planes, then split the prefetched registers into
// the other LDS buffer and prefetch the step after next (which may belong to
// the next tile), one barrier per step; the epilogue follows a tile's last
// step while the next tile's loads are in flight.
template <class GEO, int NB, bool TA, bool TB>
__global__ __launch_bounds__(GEO::NT, 1) void gemm_bf16_kernel(Params p)
{
    constexpr int BM = GEO::BM, BN = GEO::BN, TM = GEO::TM, TN = GEO::TN, RPP = GEO::RPP;
    constexpr int NP = NB >= 3 ? 3 : 2;  // planes used: hi, mid' (, lo')
    constexpr int PSA = BM * LDS_ROW, PSB = BN * LDS_ROW;
    __shared__ __attribute__((aligned(16))) uint16_t smA[2][NP * PSA];
    __shared__ __attribute__((aligned(16))) uint16_t smB[2][NP * PSB];

    const int G = gridDim.x;
    const int slot = xcd_position(blockIdx.x, G);
    const int my_tiles = (p.ntiles - slot + G - 1) / G;
    const int total = my_tiles * p.nk;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / GEO::WN, wn = wave % GEO::WN;
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;

    f32x16_t acc[TM][TN][NB];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[i][j][b] = f32x16_t{};

    RegTile<BM, RPP> ra;
    RegTile<BN, RPP> rb;
    // op(A) as [m][k]: k-contiguous unless A is transposed.
    // op(B) as [n][k]: k-contiguous when B is transposed.
    auto prefetch = [&](int it2) {
        const int tl = it2 / p.nk;
        const int kt = it2 - tl * p.nk;
        int64_t m0, n0;
        tile_coords(p, slot + tl * G, BM, BN, m0, n0);
        const int64_t k0 = (int64_t)kt * BK;
        load_tile<!TA>(ra, p.A, p.lda, p.M, p.K, m0, k0, p.vec_a);
        load_tile<TB>(rb, p.B, p.ldb, p.N, p.K, n0, k0, p.vec_b);
    };

    prefetch(0);
    store_tile_bf16<!TA, NP, PSA>(smA[0], ra);
    store_tile_bf16<TB, NP, PSB>(smB[0], rb);
    if (total > 1) prefetch(1);
    __syncthreads();

    int it = 0;
    for (int tl = 0; tl < my_tiles; ++tl) {
        for (int kt = 0; kt < p.nk; ++kt, ++it) {
            const int cur = it & 1;
            const uint16_t* As = smA[cur];
            const uint16_t* Bs = smB[cur];
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                bf16x8_t bfr[NP][TN];
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int col = (wn * TN + j) * 32 + frag_row;
                        bfr[pl][j] = *reinterpret_cast<const bf16x8_t*>(
                            Bs + pl * PSB + col * LDS_ROW + ks * 16 + frag_k);
                    }
                // A planes from the smallest piece up; for each, every B piece.
#pragma unroll
                for (int u = NP - 1; u >= 0; --u) {
                    bf16x8_t af[TM];
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const int row = (wm * TM + i) * 32 + frag_row;
                        af[i] = *reinterpret_cast<const bf16x8_t*>(
                            As + u * PSA + row * LDS_ROW + ks * 16 + frag_k);
                    }
#pragma unroll
                    for (int v = NP - 1; v >= 0; --v) {
                        if (u + v < NB) {
#pragma unroll
                            for (int i = 0; i < TM; ++i)
#pragma unroll
                                for (int j = 0; j < TN; ++j)
                                    acc[i][j][u + v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                        af[i], bfr[v][j], acc[i][j][u + v], 0, 0, 0);
                        }
                    }
                }
            }
            if (it + 1 < total) {
                store_tile_bf16<!TA, NP, PSA>(smA[cur ^ 1], ra);
                store_tile_bf16<TB, NP, PSB>(smB[cur ^ 1], rb);
                if (it + 2 < total) prefetch(it + 2);
            }
            __syncthreads();
        }

        // Epilogue: recombine the bands smallest first and store C.
        int64_t cm0, cn0;
        tile_coords(p, slot + tl * G, BM, BN, cm0, cn0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                float t[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s = acc[i][j][NB - 1][r];
#pragma unroll
                    for (int b = NB - 2; b >= 0; --b)
                        s = __builtin_fmaf(s, 0.00390625f, acc[i][j][b][r]);
                    t[r] = s;
                }
                store_c_tile(p, t, cm0 + (wm * TM + i) * 32, cn0 + (wn * TN + j) * 32);
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[i][j][b] = f32x16_t{};
            }
    }
}

// Native FP32 MFMA GEMM with the same tiling and pipeline.  Each lane half h
// (lane / 32) feeds the k values h*16 .. h*16+15 of a BK step to successive
// v_mfma_f32_32x32x2_f32 instructions (A and B use the same k order, so every
// product a(i,k) b(k,j) is formed exactly once).
template <class GEO, bool TA, bool TB>
__global__ __launch_bounds__(GEO::NT, 2) void gemm_f32_kernel(Params p)
{
    constexpr int BM = GEO::BM, BN = GEO::BN, TM = GEO::TM, TN = GEO::TN, RPP = GEO::RPP;
    __shared__ __attribute__((aligned(16))) float smA[2][BM * LDSF_ROW];
    __shared__ __attribute__((aligned(16))) float smB[2][BN * LDSF_ROW];

    const int G = gridDim.x;
    const int slot = xcd_position(blockIdx.x, G);
    const int my_tiles = (p.ntiles - slot + G - 1) / G;
    const int total = my_tiles * p.nk;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / GEO::WN, wn = wave % GEO::WN;
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * (BK / 2);

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

    RegTile<BM, RPP> ra;
    RegTile<BN, RPP> rb;
    auto prefetch = [&](int it2) {
        const int tl = it2 / p.nk;
        const int kt = it2 - tl * p.nk;
        int64_t m0, n0;
        tile_coords(p, slot + tl * G, BM, BN, m0, n0);
        const int64_t k0 = (int64_t)kt * BK;
        load_tile<!TA>(ra, p.A, p.lda, p.M, p.K, m0, k0, p.vec_a);
        load_tile<TB>(rb, p.B, p.ldb, p.N, p.K, n0, k0, p.vec_b);
    };

    prefetch(0);
    store_tile_f32<!TA>(smA[0], ra);
    store_tile_f32<TB>(smB[0], rb);
    if (total > 1) prefetch(1);
    __syncthreads();

    int it = 0;
    for (int tl = 0; tl < my_tiles; ++tl) {
        for (int kt = 0; kt < p.nk; ++kt, ++it) {
            const int cur = it & 1;
            const float* As = smA[cur];
            const float* Bs = smB[cur];
#pragma unroll
            for (int kq = 0; kq < BK / 2; kq += 4) {
                f32x4_t af[TM], bfr[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = *reinterpret_cast<const f32x4_t*>(
                        As + ((wm * TM + i) * 32 + frag_row) * LDSF_ROW + frag_k + kq);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bfr[j] = *reinterpret_cast<const f32x4_t*>(
                        Bs + ((wn * TN + j) * 32 + frag_row) * LDSF_ROW + frag_k + kq);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][s], bfr[j][s],
                                                                             acc[i][j], 0, 0, 0);
            }
            if (it + 1 < total) {
                store_tile_f32<!TA>(smA[cur ^ 1], ra);
                store_tile_f32<TB>(smB[cur ^ 1], rb);
                if (it + 2 < total) prefetch(it + 2);
            }
            __syncthreads();
        }

        int64_t cm0, cn0;
        tile_coords(p, slot + tl * G, BM, BN, cm0, cn0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                float t[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) t[r] = acc[i][j][r];
                store_c_tile(p, t, cm0 + (wm * TM + i) * 32, cn0 + (wn * TN + j) * 32);
                acc[i][j] = f32x16_t{};
            }
    }
}

__global__ void scale_c_kernel(int64_t M, int64_t N, float beta, float* __restrict__ C,
                               int64_t ldc)
{
    const int64_t total = M * N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e / N, j = e - i * N;
        float* c = C + i * ldc + j;
        *c = (beta == 0.0f) ? 0.0f : beta * *c;
    }
}

Params make_params(const GemmArgs& g, int bm, int bn)
{
    Params p;
    p.A = g.A;
    p.B = g.B;
    p.C = g.C;
    p.lda = g.lda;
    p.ldb = g.ldb;
    p.ldc = g.ldc;
    p.M = g.M;
    p.N = g.N;
    p.K = g.K;
    p.alpha = g.alpha;
    p.beta = g.beta;
    const int64_t tiles_m = (g.M + bm - 1) / bm;
    const int64_t tiles_n = (g.N + bn - 1) / bn;
    p.tiles_n = (int)tiles_n;
    p.ntiles = (int)(tiles_m * tiles_n);
    p.nk = (int)((g.K + BK - 1) / BK);
    auto aligned16 = [](const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; };
    p.vec_a = (!g.trans_a && aligned16(g.A) && (g.lda & 3) == 0) ? 1 : 0;
    p.vec_b = (g.trans_b && aligned16(g.B) && (g.ldb & 3) == 0) ? 1 : 0;
    return p;
}

// Tile counts and per-tile offsets must fit the kernels' 32-bit arithmetic:
// tiles x k-steps < 2^31, and a tile's rows (or k rows) span < 2^31 elements.
bool fits_32bit(const GemmArgs& g, int bm, int bn)
{
    const int64_t tiles = ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn);
    const int64_t nk = (g.K + BK - 1) / BK;
    const int64_t lim = (int64_t)1 << 31;
    const int64_t span_a = (g.trans_a ? (int64_t)BK : (int64_t)bm) * g.lda;
    const int64_t span_b = (g.trans_b ? (int64_t)bn : (int64_t)BK) * g.ldb;
    return tiles * nk < lim && span_a < lim && span_b < lim;
}

using GeoEmu = Geo<2, 4, 2, 1>;     // 8 waves, each 64x32: 128x128 per workgroup
using GeoF32 = Geo<2, 2, 2, 2>;     // 4 waves, each 64x64: 128x128 per workgroup

template <int NB>
hipError_t launch_bands(const Params& p, bool ta, bool tb, int grid, hipStream_t s)
{
    constexpr int NT = GeoEmu::NT;
    if (!ta && !tb)
        hipLaunchKernelGGL((gemm_bf16_kernel<GeoEmu, NB, false, false>), dim3(grid), dim3(NT), 0, s, p);
    else if (!ta && tb)
        hipLaunchKernelGGL((gemm_bf16_kernel<GeoEmu, NB, false, true>), dim3(grid), dim3(NT), 0, s, p);
    else if (ta && !tb)
        hipLaunchKernelGGL((gemm_bf16_kernel<GeoEmu, NB, true, false>), dim3(grid), dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<GeoEmu, NB, true, true>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, int nbands, const DeviceInfo& dev,
                            hipStream_t stream)
{
    if (!fits_32bit(g, GeoEmu::BM, GeoEmu::BN)) return hipErrorInvalidValue;
    const Params p = make_params(g, GeoEmu::BM, GeoEmu::BN);
    const int grid = p.ntiles < dev.num_cu ? p.ntiles : dev.num_cu;
    switch (nbands) {
    case 5: return launch_bands<5>(p, g.trans_a, g.trans_b, grid, stream);
    case 3: return launch_bands<3>(p, g.trans_a, g.trans_b, grid, stream);
    case 2: return launch_bands<2>(p, g.trans_a, g.trans_b, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_native_f32(const GemmArgs& g, const DeviceInfo& dev, hipStream_t stream)
{
    if (!fits_32bit(g, GeoF32::BM, GeoF32::BN)) return hipErrorInvalidValue;
    const Params p = make_params(g, GeoF32::BM, GeoF32::BN);
    const int cap = 2 * dev.num_cu;
    const int grid = p.ntiles < cap ? p.ntiles : cap;
    constexpr int NT = GeoF32::NT;
    if (!g.trans_a && !g.trans_b)
        hipLaunchKernelGGL((gemm_f32_kernel<GeoF32, false, false>), dim3(grid), dim3(NT), 0, stream, p);
    else if (!g.trans_a && g.trans_b)
        hipLaunchKernelGGL((gemm_f32_kernel<GeoF32, false, true>), dim3(grid), dim3(NT), 0, stream, p);
    else if (g.trans_a && !g.trans_b)
        hipLaunchKernelGGL((gemm_f32_kernel<GeoF32, true, false>), dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<GeoF32, true, true>), dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_scale_c(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                          hipStream_t stream)
{
    const int64_t total = M * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(scale_c_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, M, N, beta, C,
                       ldc);
    return hipGetLastError();
}

}  // namespace emu
