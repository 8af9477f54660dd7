// Native FP32 GEMM on gfx950 FP32 MFMA (v_mfma_f32_32x32x2_f32): the
// baseline that the emulated modes are measured against ("Unlocking Tensor
// Core Performance for Machine Learning Interatomic Potentials", sections
// "BF16x9 on NVIDIA Blackwell GPUs" and "Limitations and decision criteria":
// speed and accuracy are both quoted relative to native FP32), plus the
// C = beta*C kernel used for K == 0 or alpha == 0.
//
// Two kernels, both persistent over XCD-aware lists of 128x128 tiles:
//   * gemm_f32_pp_kernel (k-contiguous, 16-byte addressable A: the forward
//     and input-gradient GEMMs): the two-group, turn-taking structure of the
//     emulated kernel, with A copied straight to LDS by direct loads and
//     op(B) packed once per call (pack_b_f32_kernel) into the chunk layout
//     the kernel copies from;
//   * gemm_f32_kernel (any other A): operand tiles staged through registers
//     into padded FP32 LDS rows, one barrier per k-step.
#include "emu_tile.h"
#include "emu_walk.h"

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

// WIDE: 64-bit per-lane offsets, for a tile whose rows (or k rows) span
// 2^31 elements or more.
template <bool KC, bool WIDE, int ROWS, int RPP>
__device__ __forceinline__ void load_tile(RegTile<ROWS, RPP>& rt, const float* __restrict__ X,
                                          int64_t ld, int64_t rows, int64_t K, int64_t row0,
                                          int64_t k0, bool vec)
{
    typedef typename std::conditional<WIDE, int64_t, uint32_t>::type off_t;
    const int t = threadIdx.x;
    const int kk = tile_k<KC, RPP>(t);
    const int64_t gk = k0 + kk;
    // Uniform tile base plus a per-lane offset (32-bit unless WIDE).
    const float* base = KC ? X + row0 * ld + k0 : X + k0 * ld + row0;
    const bool interior = row0 + ROWS <= rows && k0 + BK <= K;
#pragma unroll
    for (int q = 0; q < RegTile<ROWS, RPP>::P; ++q) {
        const int r = tile_row<KC, RPP>(t, q);
        const int64_t gr = row0 + r;
        if (KC) {
            const off_t off = (off_t)(r * ld + kk);
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
                const off_t off = (off_t)((kk + e) * ld + r);
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
template <class GEO, bool TA, bool TB, bool WIDE>
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
        load_tile<!TA, WIDE>(ra, p.A, p.lda, p.M, p.K, m0, k0, p.vec_a);
        load_tile<TB, WIDE>(rb, p.B, p.ldb, p.N, p.K, n0, k0, p.vec_b);
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

// ---------------------------------------------------------------------------
// FP32 chunk layout of the turn-taking kernel, in LDS and (for op(B)) in the
// packed workspace: per (tile, k-step) 128 rows of 32 floats (128 bytes, no
// padding); the eight 16-byte groups of row r (k = 4c .. 4c+3 in group c)
// are stored in the order c ^ f32_swz(r).  A fragment read (ds_read_b128,
// lane l: row l % 32, one group) is served 16 lanes at a time from 64 banks
// of 4 bytes; rows r and r+1 sit in different halves of the banks, and
// f32_swz gives each pair of rows among 16 a different group position, so
// the 16 lanes hit 16 disjoint 16-byte bank groups.
// ---------------------------------------------------------------------------
constexpr int F32_CHUNK = TILE * BK;   // floats per chunk: 16 KB

__host__ __device__ constexpr int f32_swz(int r) { return (r >> 1) & 7; }
__host__ __device__ constexpr int f32_elem(int r, int k)
{
    return r * BK + ((((k >> 2) ^ f32_swz(r)) << 2) | (k & 3));
}

// op(B) (element (k, n) = B[n*ld + k] when kc, else B[k*ld + n]) into chunks
// [n-tile][k-step][128 n][32 k] of the layout above, zero outside op(B).
// One thread per (n, 4-wide k group) of the padded extent; consecutive
// threads walk the contiguous index of B.
__global__ void pack_b_f32_kernel(const float* __restrict__ B, int64_t ld, int kc, int64_t N, int64_t K,
                                  int tiles_n, int nk, float* __restrict__ W)
{
    const int64_t npad = (int64_t)tiles_n * TILE;
    const int64_t kgroups = (int64_t)nk * (BK / 4);
    const int64_t total = npad * kgroups;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        int64_t n, kg;
        if (kc) {
            n = idx / kgroups;
            kg = idx - n * kgroups;
        } else {
            kg = idx / npad;
            n = idx - kg * npad;
        }
        const int64_t k0 = kg * 4;
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t k = k0 + e;
            v[e] = (n < N && k < K) ? (kc ? B[n * ld + k] : B[k * ld + n]) : 0.0f;
        }
        const int64_t tn = n / TILE, rr = n - tn * TILE;
        const int64_t kt = k0 / BK, kk = k0 - kt * BK;
        *reinterpret_cast<f32x4_t*>(W + (tn * nk + kt) * F32_CHUNK + f32_elem((int)rr, (int)kk)) = v;
    }
}

// ---------------------------------------------------------------------------
// Native FP32 GEMM in the turn-taking form.  The 8 waves form two groups of
// four, one wave of each per SIMD; group g owns rows 64g..64g+63 of the
// 128x128 tile, each of its waves a 64x32 block (two 32x32 MFMA tiles of
// v_mfma_f32_32x32x2_f32).  Each group alternates two phases, each closed by
// a workgroup barrier, and group 1 runs one phase behind group 0, so that on
// every SIMD one wave issues MFMAs while the other loads and stores:
//   U(s): the epilogue of the tile that ended at step s-1; direct loads of
//         the group's half of a B chunk (group 0: step s+1, group 1: step
//         s+2) and of its own A rows of step s+2; the first operand
//         fragments of M(s);
//   M(s): 32 MFMAs on the step-s A rows (LDS stage s % 3) and B chunk
//         (buffer s % 3), the cursor advances, then the wait for the loads
//         of U(s-1) (A rows of step s+1) and U(s) (B half), and on a step
//         whose k runs past K the zeroing of the A groups past K.
// A's k-groups past K were loaded from column 0 of the row (a valid
// address) and are zeroed in LDS by the thread that loaded them, after its
// own wait, so the products past K are exactly zero (B is zero there too).
// Rows past M re-read the last row and only feed outputs that are not
// stored.  LDS: three A stages and three B chunk buffers, 96 KB.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512, 1) void gemm_f32_pp_kernel(Params p, const float* __restrict__ Wb)
{
    constexpr int GT = 256;                                // threads per group
    constexpr int GROWS = TILE / 2;                        // A rows per group
    constexpr int CHUNK_BYTES = F32_CHUNK * 4;
    constexpr int B_ROUNDS = CHUNK_BYTES / (GT * 16);      // 4 KB rounds per B chunk
    constexpr int B_HALF = B_ROUNDS / 2;                   // rounds each group copies
    constexpr int A_ROUNDS = GROWS * BK * 4 / (GT * 16);   // 16-byte loads per thread
    constexpr int TM = 2;
    static_assert(A_ROUNDS == 2 && GROWS == 2 * 32, "thread t loads rows t/8 and t/8 + 32 of its group");
    static_assert(B_ROUNDS * GT * 16 == CHUNK_BYTES && B_HALF * 2 == B_ROUNDS, "B chunk in whole half rounds");
    __shared__ __attribute__((aligned(16))) float stage[3][F32_CHUNK];
    __shared__ __attribute__((aligned(16))) float smB[3][F32_CHUNK];

    const int G = gridDim.x;
    const int slot = xcd_position(blockIdx.x, G);
    const int my_items = (p.ntiles - slot + G - 1) / G;
    const int total = my_items * p.nk;

    WalkConst wc;
    const int gtile = G % p.ntiles;
    wc.nk = p.nk;
    wc.nk_item = p.nk;
    wc.th = TILE;
    wc.tiles_n = p.tiles_n;
    wc.gtn = gtile % p.tiles_n;
    wc.gm = (int64_t)(gtile / p.tiles_n) * TILE;
    wc.G = G;
    wc.split_from = p.ntiles;
    wc.nsplit = 1;
    wc.tail_k = (int)(p.K - (int64_t)(p.nk - 1) * BK);
    wc.M = p.M;
    wc.lda = p.lda;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int grp = wave >> 2;
    const int gw = wave & 3;          // wave within the group = its 32-column block
    const int gt = t & (GT - 1);
    const int frag_row = lane & 31;
    const int frag_h = lane >> 5;     // lane half: k = 16 h .. 16 h + 15 of a step

    // Thread gt of group g loads rows 64g + gt/8 + 32r (r = 0, 1) of each A
    // step.  Its direct load lands at group position gt % 8 of the row, so
    // it reads the k-group stored there: (gt % 8) ^ f32_swz(row), the same
    // for both rows.
    const int srow0 = GROWS * grp + (gt >> 3);
    const int spos = gt & 7;
    const int skc = 4 * (spos ^ f32_swz(srow0));
    uint32_t a_off[A_ROUNDS];
#pragma unroll
    for (int r = 0; r < A_ROUNDS; ++r)
        a_off[r] = (uint32_t)(((int64_t)(srow0 + 32 * r) * p.lda + skc) * 4);

    // Round r of the group's A rows of step w into stage sb: this wave's 64
    // lanes fill the 1 KB at row 64g + 8 gw + 32 r.
    auto copy_a = [&](const Walk& w, int sb) __attribute__((always_inline)) {
        const float* base = p.A + w.arow + (int64_t)w.kt * BK;
        const uint32_t dst = lds_offset(stage[sb]) + 8192 * grp + 1024 * gw;
#pragma unroll
        for (int r = 0; r < A_ROUNDS; ++r) {
            uint32_t off = a_off[r];
            if (w.rows != TILE || w.kvalid != BK) {
                const int row = srow0 + 32 * r;
                const int64_t rr = row < w.rows ? row : w.rows - 1;
                const int kk = skc < w.kvalid ? skc : 0;
                off = (uint32_t)((rr * p.lda + kk) * 4);
            }
            copy16_to_lds(dst + 4096 * r, base, off);
        }
    };
    // After this thread's load of step w into stage sb has landed: its
    // k-groups past K become zero.
    auto zero_tail = [&](const Walk& w, int sb) __attribute__((always_inline)) {
        if (skc >= w.kvalid) {
#pragma unroll
            for (int r = 0; r < A_ROUNDS; ++r)
                *reinterpret_cast<f32x4_t*>(&stage[sb][(srow0 + 32 * r) * BK + 4 * spos]) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    // This group's half of the B chunk of step w into buffer bb: rounds
    // B_HALF g .. B_HALF g + B_HALF - 1, round r the 4 KB at 4096 r, this
    // wave's 1 KB piece of it at 4096 r + 1024 gw.
    auto copy_b_half = [&](const Walk& w, int bb) __attribute__((always_inline)) {
        const char* src = reinterpret_cast<const char*>(Wb + ((int64_t)w.tn * p.nk + w.kt) * F32_CHUNK);
        const uint32_t dst = lds_offset(smB[bb]);
#pragma unroll
        for (int j = 0; j < B_HALF; ++j) {
            const int byte0 = ((grp * B_HALF + j) * GT + gw * 64) * 16;
            copy16_to_lds(dst + byte0, src + byte0, (uint32_t)lane * 16);
        }
    };

    f32x16_t acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i] = zero_acc();

    // Fragments of k-group 4h + q (q = 0..3) of this lane's row l % 32 of a
    // 32-row block: the block's rows start at multiples of 32, where f32_swz
    // repeats, so the offset within the block is the same for every block.
    const int fsw = f32_swz(frag_row);
    auto foff = [&](int q) __attribute__((always_inline)) { return frag_row * BK + (((4 * frag_h + q) ^ fsw) << 2); };
    auto load_frags = [&](int bb, int q, f32x4_t& bf, f32x4_t (&af)[TM]) __attribute__((always_inline)) {
        bf = *reinterpret_cast<const f32x4_t*>(&smB[bb][gw * 32 * BK + foff(q)]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            af[i] = *reinterpret_cast<const f32x4_t*>(&stage[bb][(grp * GROWS + i * 32) * BK + foff(q)]);
    };

    // Epilogue of this wave's 64x32 block of the tile at w: C = alpha t +
    // beta C + bias.  Lane l holds, per 32x32 block and register group q,
    // row l%32 and columns 8q + 4(l/32) .. +3 (B is the MFMAs' first
    // operand): one 16-byte buffer store each, rows outside C given an
    // out-of-range offset.  Tiles that cross column N, or a C without
    // 16-byte rows, store element by element.
    auto epilogue = [&]<bool SCALE>(const TilePos& w) __attribute__((always_inline)) {
        const int64_t n0 = (int64_t)w.tn * TILE;
        float* const dst = p.C + w.m0 * p.ldc + n0;
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, 0x7FFFFFFF, 0x00020000);
        const int64_t cl = p.N - n0;
        const int cols_left = cl < TILE ? (int)cl : TILE;
        const bool vec_c = p.vec_b != 0 && cols_left == TILE;
        const int ldc4 = (int)p.ldc * 4;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = grp * GROWS + i * 32 + (lane & 31);
            const bool row_ok = row < w.rows;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = gw * 32 + 8 * q + 4 * (lane >> 5);
                f32x4_t out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = SCALE ? p.alpha * acc[i][4 * q + e] : acc[i][4 * q + e];
                if (vec_c) {
                    const int off = row_ok ? row * ldc4 + col * 4 : (int)0x80000000;
                    if (p.beta != 0.0f) {
                        const f32x4_t old = __builtin_bit_cast(
                            f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
#pragma unroll
                        for (int e = 0; e < 4; ++e) out[e] = __builtin_fmaf(p.beta, old[e], out[e]);
                    }
                    if (p.bias != nullptr) {
                        // the wave's 8 bias values of group q, one scalar load
                        const i32x8_t bv = scalar_load8(p.bias + n0 + gw * 32 + 8 * q);
                        const bool upper = (lane >> 5) != 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            int lo = bv[e], hi = bv[4 + e];
                            asm("" : "+s"(lo));
                            asm("" : "+s"(hi));
                            out[e] = out[e] + __int_as_float(upper ? hi : lo);
                        }
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, out), rsrc, off, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (row_ok && col + e < cols_left) {
                            float* cp = dst + row * p.ldc + col + e;
                            float o = out[e];
                            if (p.beta != 0.0f) o = __builtin_fmaf(p.beta, *cp, o);
                            if (p.bias != nullptr) o = o + p.bias[n0 + col + e];
                            *cp = o;
                        }
                    }
                }
            }
        }
    };
    const bool unit_alpha = p.alpha == 1.0f;
    auto epilogue_any = [&](const TilePos& w) __attribute__((always_inline)) {
        if (unit_alpha)
            epilogue.template operator()<false>(w);
        else
            epilogue.template operator()<true>(w);
    };

    // Cursors: wm = step of the next M phase, we = the step before it, ws =
    // the step after it, wa = two steps after it (its A rows loaded in the
    // next U phase).
    Walk wm;
    wm.seg = 0;
    wm.tn = slot % p.tiles_n;
    wm.m0 = (int64_t)(slot / p.tiles_n) * TILE;
    wm.left = my_items - 1;
    wm.kt = 0;
    wm.kt_end = p.nk;
    wm.item = slot;
    wm.part = 0;
    wm.widx = 0;
    walk_set_tile(wm, wc);
    wm.kvalid = wm.kt + 1 < p.nk ? BK : wc.tail_k;
    Walk ws = wm, wa = wm;
    TilePos we{wm.m0, wm.tn, wm.rows, wm.seg, 0, 0};
    // Prologue: B chunk of step 0 (each group its half) and group 1's half
    // of chunk 1; A rows of steps 0 and 1 (stages 0 and 1).
    copy_b_half(ws, 0);
    copy_a(wa, 0);
    walk_next<false>(wa, wc);
    copy_a(wa, 1);
    walk_next<false>(wa, wc);
    walk_next<false>(ws, wc);
    if (grp == 1) copy_b_half(ws, 1);
    wait_vmcnt<0>();
    if (wm.kvalid != BK) zero_tail(wm, 0);   // (step 1's tail is zeroed at the end of M(0))
    __syncthreads();
    if (grp == 1) __builtin_amdgcn_s_barrier();   // group 1 runs one phase behind group 0

    bool epi = false;       // U(s) runs the epilogue of step s-1's tile
    int bm = 0;             // A stage and B buffer of step s: s % 3
    for (int s = 0; s < total; ++s) {
        const int bn = bm == 2 ? 0 : bm + 1;    // step s+1
        const int bn2 = bn == 2 ? 0 : bn + 1;   // step s+2
        // ---- U(s).  The epilogue comes first, so its stores issue ahead of
        // this phase's direct loads instead of queueing behind them (2-3 %
        // faster than the other order), and the compiler's waits for its C
        // loads (beta != 0) cover at most the A rows loaded in U(s-1).
        if (epi) {
            epilogue_any(we);
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[i] = zero_acc();
        }
        // Group 0 loads its half of B chunk s+1 into the buffer of step
        // s-2, group 1 its half of chunk s+2 into that of step s-1; the A
        // rows of step s+2 go to the group's rows of stage s-1.  The last
        // readers of each (M(s-2) of both groups, M(s-1) of both groups,
        // M(s-1) of this group) ended before this phase.
        if (grp == 0)
            copy_b_half(ws, bn);
        else
            copy_b_half(wa, bn2);
        copy_a(wa, bn2);
        // First fragments of M(s): A rows of step s (landed and zeroed past K
        // before the barrier that ended M(s-1)) and B chunk s (both halves
        // landed before the barrier that ended the phase before U0(s)).
        f32x4_t bq[2], aq[2][TM];
        load_frags(bm, 0, bq[0], aq[0]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // ---- M(s): k-groups q = 0..3 of each lane half, the fragments of
        // group q+1 read while group q issues.  MFMA 4q + e sums the k pair
        // (4q + e, 16 + 4q + e).
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q + 1 < 4) load_frags(bm, q + 1, bq[(q + 1) & 1], aq[(q + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    // B operand first: lane l then holds row l%32 of the
                    // block and four consecutive columns per register group
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(bq[q & 1][e], aq[q & 1][i][e], acc[i], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        epi = wm.kt == p.nk - 1;
        we = TilePos{wm.m0, wm.tn, wm.rows, wm.seg, wm.part, wm.widx};
        wm = ws;
        ws = wa;
        walk_next<false>(wa, wc);
        bm = bn;
        // Before the next barrier: this group's half of B loaded in U(s) and
        // its A rows of step s+1 (loaded in U(s-1)) have landed, while its A
        // load of U(s), issued after them, may still be in flight; then the
        // A groups of step s+1 past K are zeroed.
        wait_vmcnt<A_ROUNDS>();
        if (wm.kvalid != BK) zero_tail(wm, bm);
        wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }
    epilogue_any(we);
    wait_vmcnt<0>();   // no direct load may still be writing LDS when the workgroup ends
    if (grp == 0) __builtin_amdgcn_s_barrier();   // matches group 1's extra barrier
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

using GeoF32Staged = Geo<2, 2, 2, 2>;   // 4 waves, each 64x64: 128x128 per workgroup

// Tile counts must fit the kernel's 32-bit arithmetic (tiles x k-steps <
// 2^31); per-tile offsets need the WIDE kernel when a tile's rows (or k
// rows) span 2^31 elements or more.
bool tiles_fit_32bit(const GemmArgs& g, int bm, int bn)
{
    const int64_t tiles = ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn);
    const int64_t nk = (g.K + BK - 1) / BK;
    return tiles * nk < ((int64_t)1 << 31);
}

bool needs_wide_offsets(const GemmArgs& g, int bm, int bn)
{
    const int64_t lim = (int64_t)1 << 31;
    const int64_t span_a = (g.trans_a ? (int64_t)BK : (int64_t)bm) * g.lda;
    const int64_t span_b = (g.trans_b ? (int64_t)bn : (int64_t)BK) * g.ldb;
    return span_a >= lim || span_b >= lim;
}

template <bool WIDE>
void launch_f32_staged(const Params& p, bool ta, bool tb, int grid, hipStream_t stream)
{
    constexpr int NT = GeoF32Staged::NT;
    if (!ta && !tb)
        hipLaunchKernelGGL((gemm_f32_kernel<GeoF32Staged, false, false, WIDE>), dim3(grid), dim3(NT), 0, stream, p);
    else if (!ta && tb)
        hipLaunchKernelGGL((gemm_f32_kernel<GeoF32Staged, false, true, WIDE>), dim3(grid), dim3(NT), 0, stream, p);
    else if (ta && !tb)
        hipLaunchKernelGGL((gemm_f32_kernel<GeoF32Staged, true, false, WIDE>), dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<GeoF32Staged, true, true, WIDE>), dim3(grid), dim3(NT), 0, stream, p);
}


}  // namespace

// The turn-taking kernel applies to a k-contiguous, 16-byte addressable A
// (as the emulated kernel's fused path) whose tile and chunk counts fit its
// 32-bit arithmetic.
bool native_pp_path(const GemmArgs& g)
{
    const int64_t tiles_m = (g.M + TILE - 1) / TILE;
    const int64_t tiles_n = (g.N + TILE - 1) / TILE;
    const int64_t nk = (g.K + BK - 1) / BK;
    const int64_t lim = (int64_t)1 << 31;
    return fused_a_path(g) && tiles_m * tiles_n < lim && tiles_m * tiles_n * nk < lim && tiles_n * nk < lim;
}

size_t gemm_native_f32_workspace_bytes(const GemmArgs& g)
{
    if (!native_pp_path(g)) return 0;
    const int64_t tiles_n = (g.N + TILE - 1) / TILE;
    const int64_t nk = (g.K + BK - 1) / BK;
    return ((size_t)(tiles_n * nk * F32_CHUNK) * sizeof(float) + 255) & ~(size_t)255;
}

hipError_t launch_gemm_native_f32(const GemmArgs& g, const DeviceInfo& dev, void* workspace,
                                  hipStream_t stream)
{
    if (native_pp_path(g)) {
        if (workspace == nullptr || ((uintptr_t)workspace & 15u) != 0) return hipErrorInvalidValue;
        Params p = make_params(g, TILE, TILE);
        p.ksplit = 1;
        p.nk_item = p.nk;
        // (turn-taking kernel) C rows allow 16-byte stores at 16-byte aligned
        // columns, and the bias (if any) 16-byte loads there
        p.vec_b = (((uintptr_t)g.C & 15u) == 0 && (g.ldc & 3) == 0 &&
                   (g.bias == nullptr || ((uintptr_t)g.bias & 15u) == 0) &&
                   (int64_t)TILE * g.ldc * 4 < ((int64_t)1 << 31)) ? 1 : 0;
        float* W = static_cast<float*>(workspace);
        const int64_t work = (int64_t)p.tiles_n * TILE * p.nk * (BK / 4);
        int64_t blocks = (work + 255) / 256;
        if (blocks > 16384) blocks = 16384;
        hipLaunchKernelGGL(pack_b_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g.B, g.ldb,
                           g.trans_b ? 1 : 0, g.N, g.K, p.tiles_n, p.nk, W);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int grid = p.ntiles < dev.num_cu ? p.ntiles : dev.num_cu;
        hipLaunchKernelGGL(gemm_f32_pp_kernel, dim3(grid), dim3(512), 0, stream, p, W);
        return hipGetLastError();
    }
    if (!tiles_fit_32bit(g, GeoF32Staged::BM, GeoF32Staged::BN)) return hipErrorInvalidValue;
    const Params p = make_params(g, GeoF32Staged::BM, GeoF32Staged::BN);
    const int cap = 2 * dev.num_cu;
    const int grid = p.ntiles < cap ? p.ntiles : cap;
    if (needs_wide_offsets(g, GeoF32Staged::BM, GeoF32Staged::BN))
        launch_f32_staged<true>(p, g.trans_a, g.trans_b, grid, stream);
    else
        launch_f32_staged<false>(p, g.trans_a, g.trans_b, grid, stream);
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
