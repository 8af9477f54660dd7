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

// ---------------------------------------------------------------------------
// Emulated GEMM, B operand pre-split.
//
// op(B) is split once per call by presplit_b_kernel into a workspace laid out
// exactly as the kernel's LDS tiles: for every (n-tile, k-step) a chunk of NP
// planes x 128 rows (n) x LDS_ROW bf16 (k, padded), rows past N and k past K
// zero.  The GEMM kernel then copies each chunk to LDS with direct
// global->LDS loads (no registers, no VALU, no bounds checks) and splits only
// op(A), whose elements it loads, splits in registers and writes to LDS.
// ---------------------------------------------------------------------------

constexpr int WS_ROWS = 128;                         // n rows per B chunk (= BN)

__host__ __device__ constexpr int64_t bchunk_elems(int np) { return (int64_t)np * WS_ROWS * LDS_ROW; }

// One thread per (n, 8-wide k group) of the padded B extent.
template <int NP>
__global__ void presplit_b_kernel(const float* __restrict__ B, int64_t ldb, int trans_b, int64_t N,
                                  int64_t K, int tiles_n, int nk, uint16_t* __restrict__ W)
{
    const int64_t npad = (int64_t)tiles_n * WS_ROWS;
    const int64_t kgroups = (int64_t)nk * (BK / 8);
    const int64_t total = npad * kgroups;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        int64_t n, kg;
        if (trans_b) {  // B stored N x K: consecutive threads walk k
            n = idx / kgroups;
            kg = idx - n * kgroups;
        } else {        // B stored K x N: consecutive threads walk n
            kg = idx / npad;
            n = idx - kg * npad;
        }
        const int64_t k0 = kg * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t k = k0 + e;
            v[e] = (n < N && k < K) ? (trans_b ? B[n * ldb + k] : B[k * ldb + n]) : 0.0f;
        }
        uint32_t h[4], m[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (NP == 3)
                split_pair<true>(v[2 * e], v[2 * e + 1], h[e], m[e], l[e]);
            else
                split_pair_hm(v[2 * e], v[2 * e + 1], h[e], m[e]);
        }
        const int64_t tn = n / WS_ROWS, nn = n - tn * WS_ROWS;
        const int64_t kt = k0 / BK, kk = k0 - kt * BK;
        uint16_t* chunk = W + (tn * nk + kt) * bchunk_elems(NP);
        const int64_t off = nn * LDS_ROW + kk;
        *reinterpret_cast<u32x4_t*>(chunk + off) = u32x4_t{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<u32x4_t*>(chunk + WS_ROWS * LDS_ROW + off) = u32x4_t{m[0], m[1], m[2], m[3]};
        if (NP == 3)
            *reinterpret_cast<u32x4_t*>(chunk + 2 * WS_ROWS * LDS_ROW + off) =
                u32x4_t{l[0], l[1], l[2], l[3]};
    }
}

// Position in the static tile list plus k-step, advanced once per k-step.
// next() saturates at the workgroup's last (tile, k-step), so prefetches past
// the end re-read valid data instead of running off the operands.
struct Cursor {
    int tile, kt, tn;
    int64_t m0;
    __device__ __forceinline__ void set(const Params& p, int t, int bm)
    {
        tile = t;
        kt = 0;
        const int tm = t / p.tiles_n;
        tn = t - tm * p.tiles_n;
        m0 = (int64_t)tm * bm;
    }
    __device__ __forceinline__ void next(const Params& p, int G, int bm)
    {
        if (kt + 1 < p.nk) {
            ++kt;
        } else if (tile + G < p.ntiles) {
            set(p, tile + G, bm);
        }
    }
};

// Per-thread element offsets of an op(A) tile (constant over the launch).
template <bool KC, int ROWS, int RPP>
struct APlan {
    static constexpr int P = ROWS / RPP;
    uint32_t off[P];   // offset of the thread's first element of row q
    int row[P];        // row of the tile
    int kk;            // first k of the thread's four
    __device__ __forceinline__ void init(int64_t ld)
    {
        const int t = threadIdx.x;
        kk = tile_k<KC, RPP>(t);
#pragma unroll
        for (int q = 0; q < P; ++q) {
            row[q] = tile_row<KC, RPP>(t, q);
            off[q] = KC ? (uint32_t)(row[q] * ld + kk) : (uint32_t)(kk * ld + row[q]);
        }
    }
};

// Loads of a full tile (all rows < M, k0 + BK <= K): no checks.
template <bool KC, int ROWS, int RPP>
__device__ __forceinline__ void load_a_fast(RegTile<ROWS, RPP>& rt, const APlan<KC, ROWS, RPP>& pl,
                                            const float* __restrict__ base, uint32_t ld, bool vec)
{
#pragma unroll
    for (int q = 0; q < APlan<KC, ROWS, RPP>::P; ++q) {
        if (KC && vec) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(base + pl.off[q]);
            rt.v[q][0] = v[0];
            rt.v[q][1] = v[1];
            rt.v[q][2] = v[2];
            rt.v[q][3] = v[3];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rt.v[q][e] = base[pl.off[q] + (KC ? (uint32_t)e : (uint32_t)e * ld)];
        }
    }
}

// Loads of an edge tile: elements outside op(A) read as zero.
template <bool KC, int ROWS, int RPP>
__device__ __forceinline__ void load_a_edge(RegTile<ROWS, RPP>& rt, const APlan<KC, ROWS, RPP>& pl,
                                            const float* __restrict__ base, uint32_t ld,
                                            int64_t rows_left, int64_t k_left)
{
#pragma unroll
    for (int q = 0; q < APlan<KC, ROWS, RPP>::P; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = pl.row[q] < rows_left && pl.kk + e < k_left;
            rt.v[q][e] = ok ? base[pl.off[q] + (KC ? (uint32_t)e : (uint32_t)e * ld)] : 0.0f;
        }
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt
    // (11:8) left at their maxima, i.e. not waited on.
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint32_t lds_offset(const void* p)
{
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// Direct global->LDS copy of 16 bytes per lane: lane l's bytes land at LDS
// offset `lds_base + 16 l` (lds_base wave-uniform).  Written as inline
// assembly so that the compiler does not guard every later LDS read with a
// wait for this load; the caller waits (wait_vmcnt) before the barrier that
// publishes the data.
__device__ __forceinline__ const void* uniform_ptr(const void* p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void copy16_to_lds(uint32_t lds_base, const void* gbase, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(uniform_ptr(gbase))
                 : "memory");
}

// The emulated GEMM.  NB = bands kept: 5 (nine products), 3 (six), 2 (three).
// Per k-step, in order: direct loads of the next B chunk into the other LDS
// buffer; MFMAs on the current buffers interleaved with the split of the
// prefetched A registers into the other buffer; loads of the A tile two steps
// ahead; wait for the B chunk; one barrier.  The epilogue follows a tile's
// last k-step while the next tile's loads are in flight.
template <class GEO, int NB, bool TA>
__global__ __launch_bounds__(GEO::NT, 1) void gemm_bf16_kernel(Params p, const uint16_t* __restrict__ W)
{
    constexpr int BM = GEO::BM, BN = GEO::BN, TM = GEO::TM, TN = GEO::TN, RPP = GEO::RPP;
    constexpr int NP = NB >= 3 ? 3 : 2;  // planes used: hi, mid' (, lo')
    constexpr int PSA = BM * LDS_ROW, PSB = BN * LDS_ROW;
    constexpr bool KC = !TA;             // op(A) k-contiguous in memory
    static_assert(BN == WS_ROWS, "B chunk rows");
    constexpr int CHUNK_BYTES = (int)(bchunk_elems(NP) * 2);
    constexpr int COPY_ROUNDS = (CHUNK_BYTES + GEO::NT * 16 - 1) / (GEO::NT * 16);
    constexpr int A_LOADS = KC ? RegTile<BM, RPP>::P : 4 * RegTile<BM, RPP>::P;
    __shared__ __attribute__((aligned(16))) uint16_t smA[2][NP * PSA];
    __shared__ __attribute__((aligned(16))) uint16_t smB[2][NP * PSB];

    const int G = gridDim.x;
    const int slot = xcd_position(blockIdx.x, G);
    const int my_tiles = (p.ntiles - slot + G - 1) / G;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / GEO::WN, wn = wave % GEO::WN;
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    const uint32_t lda = (uint32_t)p.lda;

    APlan<KC, BM, RPP> plan;
    plan.init(p.lda);

    // Issue the direct loads of B chunk (tn, kt) into LDS buffer `buf`.
    auto load_b = [&](const Cursor& c, int buf) {
        const char* src = reinterpret_cast<const char*>(W + ((int64_t)c.tn * p.nk + c.kt) * bchunk_elems(NP));
        const uint32_t dst = lds_offset(smB[buf]);
#pragma unroll
        for (int r = 0; r < COPY_ROUNDS; ++r) {
            const int byte0 = (r * GEO::NT + wave * 64) * 16;  // this wave's 1 KB piece
            if (byte0 < CHUNK_BYTES)
                copy16_to_lds(dst + byte0, src + byte0, (uint32_t)lane * 16);
        }
    };
    auto load_a = [&](RegTile<BM, RPP>& rt, const Cursor& c) {
        const int64_t k0 = (int64_t)c.kt * BK;
        const float* base = KC ? p.A + c.m0 * p.lda + k0 : p.A + k0 * p.lda + c.m0;
        if (c.m0 + BM <= p.M && k0 + BK <= p.K)
            load_a_fast<KC>(rt, plan, base, lda, p.vec_a != 0);
        else
            load_a_edge<KC>(rt, plan, base, lda, p.M - c.m0, p.K - k0);
    };

    f32x16_t acc[TM][TN][NB];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[i][j][b] = f32x16_t{};

    RegTile<BM, RPP> ra;
    Cursor cc, cb, ca;   // compute step it, B load step it+1, A load step it+2
    cc.set(p, slot, BM);
    cb = cc;
    ca = cc;
    load_b(cb, 0);
    load_a(ra, ca);
    store_tile_bf16<KC, NP, PSA>(smA[0], ra);
    cb.next(p, G, BM);
    ca.next(p, G, BM);
    load_a(ra, ca);
    ca.next(p, G, BM);
    wait_vmcnt<A_LOADS>();
    __syncthreads();

    int cur = 0;
    for (int tl = 0; tl < my_tiles; ++tl) {
        for (int kt = 0; kt < p.nk; ++kt) {
            load_b(cb, cur ^ 1);
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
            // split of the prefetched A tile (step it+1) into the other buffer
            store_tile_bf16<KC, NP, PSA>(smA[cur ^ 1], ra);
            // Interleave the split's VALU work with the MFMAs of this step.
            constexpr int N_MFMA = (BK / 16) * TM * TN * (NB == 5 ? 9 : NB == 3 ? 6 : 3);
#pragma unroll
            for (int g = 0; g < N_MFMA; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // then up to 3 VALU
            }
            load_a(ra, ca);
            cb.next(p, G, BM);
            ca.next(p, G, BM);
            wait_vmcnt<A_LOADS>();
            __syncthreads();
            cur ^= 1;
        }

        // Epilogue: recombine the bands smallest first and store C.
        const int64_t cm0 = cc.m0;
        const int64_t cn0 = (int64_t)cc.tn * BN;
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
        if (cc.tile + G < p.ntiles) cc.set(p, cc.tile + G, BM);
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
hipError_t launch_bands(const Params& p, bool ta, int grid, const uint16_t* W, hipStream_t s)
{
    constexpr int NT = GeoEmu::NT;
    if (!ta)
        hipLaunchKernelGGL((gemm_bf16_kernel<GeoEmu, NB, false>), dim3(grid), dim3(NT), 0, s, p, W);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<GeoEmu, NB, true>), dim3(grid), dim3(NT), 0, s, p, W);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, int nbands, const DeviceInfo& dev,
                            hipStream_t stream)
{
    if (nbands != 5 && nbands != 3 && nbands != 2) return hipErrorInvalidValue;
    if (!fits_32bit(g, GeoEmu::BM, GeoEmu::BN)) return hipErrorInvalidValue;
    const Params p = make_params(g, GeoEmu::BM, GeoEmu::BN);
    const int np = nbands >= 3 ? 3 : 2;
    const size_t ws_bytes = (size_t)p.tiles_n * p.nk * bchunk_elems(np) * sizeof(uint16_t);
    uint16_t* W = nullptr;
    hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&W), ws_bytes, stream);
    if (e != hipSuccess) return hipErrorOutOfMemory;

    const int64_t work = (int64_t)p.tiles_n * WS_ROWS * p.nk * (BK / 8);
    int64_t blocks = (work + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    const int tb = g.trans_b ? 1 : 0;
    if (np == 3)
        hipLaunchKernelGGL(presplit_b_kernel<3>, dim3((unsigned)blocks), dim3(256), 0, stream, g.B,
                           g.ldb, tb, g.N, g.K, p.tiles_n, p.nk, W);
    else
        hipLaunchKernelGGL(presplit_b_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, g.B,
                           g.ldb, tb, g.N, g.K, p.tiles_n, p.nk, W);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const int grid = p.ntiles < dev.num_cu ? p.ntiles : dev.num_cu;
        switch (nbands) {
        case 5: e = launch_bands<5>(p, g.trans_a, grid, W, stream); break;
        case 3: e = launch_bands<3>(p, g.trans_a, grid, W, stream); break;
        default: e = launch_bands<2>(p, g.trans_a, grid, W, stream); break;
        }
    }
    const hipError_t ef = hipFreeAsync(W, stream);
    return e != hipSuccess ? e : ef;
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
