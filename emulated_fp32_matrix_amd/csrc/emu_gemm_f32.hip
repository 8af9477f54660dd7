// Native FP32 GEMM on gfx950 FP32 MFMA (v_mfma_f32_32x32x2_f32): the
// baseline that the emulated modes are measured against ("Unlocking Tensor
// Core Performance for Machine Learning Interatomic Potentials", sections
// "BF16x9 on NVIDIA Blackwell GPUs" and "Limitations and decision criteria":
// speed and accuracy are both quoted relative to native FP32), plus the
// C = beta*C kernel used for K == 0 or alpha == 0.
//
// Same persistent, XCD-aware 128x128 tiling as the emulated kernel; operand
// tiles are staged through registers into padded FP32 LDS rows.
#include "emu_tile.h"

namespace emu {
namespace {

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
                               int64_t ldc, const float* __restrict__ bias)
{
    const int64_t total = M * N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e / N, j = e - i * N;
        float* c = C + i * ldc + j;
        float out = (beta == 0.0f) ? 0.0f : beta * *c;
        if (bias != nullptr) out = out + bias[j];
        *c = out;
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
    p.bias = g.bias;
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

using GeoF32 = Geo<2, 2, 2, 2>;     // 4 waves, each 64x64: 128x128 per workgroup

}  // namespace

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
                          const float* bias, hipStream_t stream)
{
    const int64_t total = M * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(scale_c_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, M, N, beta, C,
                       ldc, bias);
    return hipGetLastError();
}

}  // namespace emu
