// The emulated-FP32 GEMM on gfx950 bf16 MFMA: nine, six or three products of
// the three-piece split, accumulated in FP32 per anti-diagonal band.
//
// Method: "Unlocking Tensor Core Performance for Machine Learning Interatomic
// Potentials", section "How Tensor Core FP32 bridges the hardware gap",
// Figure 1 (three scaled BF16 pieces per operand, nine pairwise products
// accumulated in FP32 along five anti-diagonal bands, recombined with their
// scales) and Figure 2 (a reduced variant keeps only the largest products).
//
// Design (MI355X-first):
//   * op(B) (the weights: small, reused by every output tile) is split once
//     per call by presplit_kernel into a workspace laid out exactly like the
//     kernel's LDS tiles: per (n-tile, k-step) one chunk of NP planes x 128
//     rows x 32 bf16 (16-byte groups permuted per row), zero outside op(B).
//     The GEMM kernel copies chunks to LDS with direct global->LDS loads:
//     no registers, no VALU, no bounds checks.
//   * op(A) (the activations: large, streamed once per n-tile) is split in
//     the kernel: its FP32 tile is copied to an LDS staging buffer with the
//     same direct loads, then each thread reads its 2 rows x 4 k, splits them
//     in registers and writes the BF16 planes.  When A is transposed or not
//     16-byte addressable, it is pre-split like B instead.
//   * Persistent launch: one 512-thread workgroup per CU walks a static,
//     XCD-aware list of 128x128 output tiles; the k-steps of consecutive
//     tiles form one software pipeline.
//   * 8 waves (two per SIMD) each own a 64x32 block of C as two
//     v_mfma_f32_32x32x16_bf16 tiles with one FP32 accumulator per band
//     (5 x 2 x 16 = 160 registers in the nine-product mode).
//   * k-contiguous A (the forward and input-gradient GEMMs): the waves form
//     two groups that take turns (gemm_bf16_pp_kernel): while one group's
//     waves issue MFMAs, the other group's waves, one per SIMD beside them,
//     load, split and store.  Otherwise (A transposed or not 16-byte
//     addressable) A is pre-split like B and gemm_bf16_kernel runs, one
//     barrier per step, the split work interleaved with the MFMAs.
//   * Epilogue: bands are recombined smallest first (t = S_{n-1},
//     t = S_j + 2^-8 t), then C = alpha t + beta C.
#include "emu_tile.h"
#include "emu_walk.h"

namespace emu {
namespace {

constexpr int PS = TILE * LDS_ROW; // elements per plane of an LDS tile

// Plane rows carry no padding.  Instead the four 16-byte chunks of row r
// (k = 8c .. 8c+7 in chunk c) are stored in the order c ^ plane_swz(r), which
// depends on r % 16 only.  The permutation was chosen by timing the two LDS
// patterns of the kernel on gfx950 with candidate permutations: the MFMA
// fragment reads (lane l: row l % 32, chunk 2 ks + l / 32, 16 bytes) run at
// 464 B/ns per CU with this one, against 433 with rows padded to 80 bytes
// and 303 with ((r >> 1) ^ (r >> 3)) & 3; the split's 8-byte writes run at
// 182 against 153 padded.  It also saves a fifth of every plane's LDS space
// and of the B chunks' load volume.
__host__ __device__ constexpr int plane_swz(int r) { return (r >> 2) & 3; }
// Element offset of (row r, k) within one plane.
__host__ __device__ constexpr int plane_elem(int r, int k)
{
    return r * LDS_ROW + ((((k >> 3) ^ plane_swz(r)) << 3) | (k & 7));
}

// Workgroup shape: NT threads; waves arranged (NT/64/WN) x WN, each owning
// TM x TN MFMA tiles of 32x32.
template <int NT_, int WN_, int TM_, int TN_>
struct Shape {
    static constexpr int NT = NT_, WN = WN_, TM = TM_, TN = TN_;
    static constexpr int WM = NT / 64 / WN;
    static_assert(WM * TM * 32 == TILE && WN * TN * 32 == TILE, "waves must cover the tile");
};
using Shape8 = Shape<512, 4, 2, 1>;   // 8 waves (2 per SIMD), 64x32 each
using Shape4 = Shape<256, 2, 2, 2>;   // 4 waves (1 per SIMD), 64x64 each

__host__ __device__ constexpr int64_t chunk_elems(int np) { return (int64_t)np * PS; }

// ---------------------------------------------------------------------------
// Pre-split of an operand viewed as [rows][k] into the chunk layout
// [tile row][k-step][plane][128][LDS_ROW] (chunks of a row permuted as
// plane_elem places them).  Element (r, k) is X[r*ld + k] when kc (k
// contiguous) and X[k*ld + r] otherwise.  One thread per (row, 8-wide k
// group) of the padded extent; rows past `rows` and k past K are zero.
// ---------------------------------------------------------------------------
template <int NP>
__global__ void presplit_kernel(const float* __restrict__ X, int64_t ld, int kc, int64_t rows,
                                int64_t K, int tiles_r, int nk, uint16_t* __restrict__ W)
{
    const int64_t rpad = (int64_t)tiles_r * TILE;
    const int64_t kgroups = (int64_t)nk * (BK / 8);
    const int64_t total = rpad * kgroups;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        int64_t r, kg;
        if (kc) {  // consecutive threads walk k
            r = idx / kgroups;
            kg = idx - r * kgroups;
        } else {   // consecutive threads walk rows
            kg = idx / rpad;
            r = idx - kg * rpad;
        }
        const int64_t k0 = kg * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t k = k0 + e;
            v[e] = (r < rows && k < K) ? (kc ? X[r * ld + k] : X[k * ld + r]) : 0.0f;
        }
        uint32_t w[4][NP];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_pieces<NP>(v[2 * e], v[2 * e + 1], w[e]);
        const int64_t tr = r / TILE, rr = r - tr * TILE;
        const int64_t kt = k0 / BK, kk = k0 - kt * BK;
        uint16_t* chunk = W + (tr * nk + kt) * chunk_elems(NP);
        const int64_t off = plane_elem((int)rr, (int)kk);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
            *reinterpret_cast<u32x4_t*>(chunk + pl * PS + off) = u32x4_t{w[0][pl], w[1][pl], w[2][pl], w[3][pl]};
    }
}

// ---------------------------------------------------------------------------
// The GEMM kernel.  NB = bands kept: 5 (nine products), 3 (six), 2 (three).
// FUSED_A: op(A) is k-contiguous FP32 split in the kernel; otherwise Wa
// holds its pre-split chunks.
//
// Step s of the workgroup's (tile, k-step) sequence, LDS buffers s%2 holding
// the planes of step s:
//   1. direct loads of the chunks of step s+1 (B; A when pre-split) into
//      the other plane buffers, and (FUSED_A) of the FP32 A tile of step s+2
//      into staging buffer s%2;
//   2. MFMAs on the current planes, interleaved (FUSED_A) with the split of
//      the FP32 A tile of step s+1 (staging buffer (s+1)%2) into the other
//      plane buffer;
//   3. wait for this step's direct loads; barrier.
// The epilogue follows the tile's last step and clears the accumulators.
// ---------------------------------------------------------------------------
template <class SH, int NB, bool FUSED_A>
__global__ __launch_bounds__(SH::NT, 1) void gemm_bf16_kernel(Params p, const uint16_t* __restrict__ Wb,
                                                              const uint16_t* __restrict__ Wa)
{
    constexpr int NT = SH::NT, WAVES_N = SH::WN, TM = SH::TM, TN = SH::TN;
    constexpr int SROWS = TILE * 8 / NT;   // A rows split per thread (NT/8 rows apart)
    constexpr int NP = NB >= 3 ? 3 : NB;  // planes used: hi (, mid' (, lo'))
    constexpr int CHUNK_BYTES = (int)chunk_elems(NP) * 2;
    constexpr int COPY_ROUNDS = (CHUNK_BYTES + NT * 16 - 1) / (NT * 16);
    constexpr int STAGE_FLOATS = TILE * BK;
    constexpr int STAGE_ROUNDS = STAGE_FLOATS * 4 / (NT * 16);
    constexpr int MFMA_PER_KS = TM * TN * (NB == 5 ? 9 : NB == 3 ? 6 : NB == 2 ? 3 : 1);
    static_assert(STAGE_ROUNDS * NT * 16 == STAGE_FLOATS * 4 && STAGE_ROUNDS == SROWS,
                  "each thread splits the rows it copied");
    __shared__ __attribute__((aligned(16))) uint16_t smA[2][chunk_elems(NP)];
    __shared__ __attribute__((aligned(16))) uint16_t smB[2][chunk_elems(NP)];
    __shared__ __attribute__((aligned(16))) float stage[FUSED_A ? 2 : 1][FUSED_A ? STAGE_FLOATS : 4];

    const int G = gridDim.x;
    const int slot = xcd_position(blockIdx.x, G);
    const int my_tiles = (p.ntiles - slot + G - 1) / G;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;

    // Split/staging geometry: thread t owns rows t/8 + (NT/8) q, k t%8*4.
    const int srow = t >> 3;
    const int skc = (t & 7) * 4;
    // Direct-load byte offsets of the FP32 A tile (interior tiles).
    uint32_t a_off[STAGE_ROUNDS];
#pragma unroll
    for (int r = 0; r < STAGE_ROUNDS; ++r)
        a_off[r] = (uint32_t)(((int64_t)(srow + (NT / 8) * r) * p.lda + skc) * 4);

    auto copy_chunk = [&](const uint16_t* W, int64_t chunk, uint16_t* dst_tile) __attribute__((always_inline)) {
        const char* src = reinterpret_cast<const char*>(W + chunk * chunk_elems(NP));
        const uint32_t dst = lds_offset(dst_tile);
#pragma unroll
        for (int r = 0; r < COPY_ROUNDS; ++r) {
            const int byte0 = (r * NT + wave * 64) * 16;  // this wave's 1 KB piece
            if (byte0 < CHUNK_BYTES) copy16_to_lds(dst + byte0, src + byte0, (uint32_t)lane * 16);
        }
    };
    // FP32 A tile of cursor c into staging buffer sb; rows past M and k past
    // K are redirected to valid addresses (their values are masked later).
    auto copy_a32 = [&](const Cursor& c, int sb) __attribute__((always_inline)) {
        const float* base = p.A + c.m0 * p.lda + c.k0();
        const uint32_t dst = lds_offset(stage[sb]);
        const bool interior = c.m0 + TILE <= p.M && c.k0() + BK <= p.K;
#pragma unroll
        for (int r = 0; r < STAGE_ROUNDS; ++r) {
            uint32_t off = a_off[r];
            if (!interior) {
                const int64_t row = srow + (NT / 8) * r;
                const int64_t rr = (c.m0 + row < p.M) ? row : (p.M - 1 - c.m0);
                const int64_t kk = (c.k0() + skc < p.K) ? skc : 0;
                off = (uint32_t)((rr * p.lda + kk) * 4);
            }
            copy16_to_lds(dst + (r * NT + wave * 64) * 16, base, off);
        }
    };
    // Step s (plane buffers pb = s%2): chunks of step s+1 into buffers pb^1,
    // FP32 A of step s+2 into staging buffer pb (its previous contents, step
    // s's A, were split during step s-1).
    auto issue_loads = [&](const Cursor& cb, const Cursor& ca, int pb) __attribute__((always_inline)) {
        copy_chunk(Wb, (int64_t)cb.tn * p.nk + cb.kt, smB[pb ^ 1]);
        if (FUSED_A)
            copy_a32(ca, pb);
        else
            copy_chunk(Wa, (cb.m0 / TILE) * p.nk + cb.kt, smA[pb ^ 1]);
    };

    // Split the FP32 tile in staging buffer sb (step described by c) into the
    // planes of plane buffer pb.
    auto split_stage = [&](const Cursor& c, int sb, int pb) __attribute__((always_inline)) {
        const bool interior = c.m0 + TILE <= p.M && c.k0() + BK <= p.K;
#pragma unroll
        for (int q = 0; q < SROWS; ++q) {
            const int row = srow + (NT / 8) * q;
            f32x4_t v = *reinterpret_cast<const f32x4_t*>(&stage[sb][row * BK + skc]);
            if (!interior) {
                const bool rok = c.m0 + row < p.M;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!(rok && c.k0() + skc + e < p.K)) v[e] = 0.0f;
            }
            uint32_t w0[NP], w1[NP];
            split_pieces<NP>(v[0], v[1], w0);
            split_pieces<NP>(v[2], v[3], w1);
            uint16_t* dst = smA[pb] + plane_elem(row, skc);
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) *reinterpret_cast<u32x2_t*>(dst + pl * PS) = u32x2_t{w0[pl], w1[pl]};
        }
    };

    f32x16_t acc[TM][TN][NB];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[i][j][b] = f32x16_t{};

    // MFMAs of k-half ks on plane buffer pb.
    auto mfma_half = [&](int pb, int ks) __attribute__((always_inline)) {
        const uint16_t* As = smA[pb];
        const uint16_t* Bs = smB[pb];
        bf16x8_t bfr[NP][TN];
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = (wn * TN + j) * 32 + frag_row;
                bfr[pl][j] = *reinterpret_cast<const bf16x8_t*>(Bs + pl * PS + plane_elem(col, ks * 16 + frag_k));
            }
#pragma unroll
        for (int u = NP - 1; u >= 0; --u) {
            bf16x8_t af[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = (wm * TM + i) * 32 + frag_row;
                af[i] = *reinterpret_cast<const bf16x8_t*>(As + u * PS + plane_elem(row, ks * 16 + frag_k));
            }
#pragma unroll
            for (int v = NP - 1; v >= 0; --v) {
                if (u + v < NB) {
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            // B operand first: lane l then holds row m = l%32 of
                            // its 32x32 block of C and four consecutive columns
                            // per register group, for 16-byte stores.
                            acc[i][j][u + v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                bfr[v][j], af[i], acc[i][j][u + v], 0, 0, 0);
                }
            }
        }
    };

    // One step's compute: the MFMAs of both k-halves, with (FUSED_A) the
    // split of the next step's A tile spread evenly between them.
    auto compute = [&](int pb, const Cursor& cnext) __attribute__((always_inline)) {
        mfma_half(pb, 0);
        mfma_half(pb, 1);
        if (FUSED_A) {
            split_stage(cnext, pb ^ 1, pb ^ 1);
#pragma unroll
            for (int g = 0; g < 2 * MFMA_PER_KS; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // then up to 3 VALU
            }
        }
    };

    // Epilogue of the tile at cursor c: recombine the bands smallest first,
    // C = alpha t + beta C, clear the accumulators.  Lane l holds, for each
    // 32x32 block and register group g, row l%32 and columns 8g + 4(l/32)
    // .. +3: one 16-byte buffer store per group, rows outside C given an
    // out-of-range offset, so exactly EPI_STORES stores are issued whatever
    // the tile's position (the step's vmcnt wait counts on it).  Tiles that
    // cross column N, or C without 16-byte rows, store element by element.
    constexpr int EPI_STORES = TM * TN * 4;
    auto epilogue = [&](const Cursor& c) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(p.C + c.m0 * p.ldc + c.n0()), (short)0, 0x7FFFFFFF, 0x00020000);
        const int64_t rows_left = p.M - c.m0, cols_left = p.N - c.n0();
        const bool vec_c = p.vec_b != 0 && cols_left >= TILE;   // vec_b carries C's alignment
        const int ldc4 = (int)p.ldc * 4;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = (wm * TM + i) * 32 + (lane & 31);
                const bool row_ok = row < rows_left;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = (wn * TN + j) * 32 + 8 * g + 4 * (lane >> 5);
                    f32x4_t out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g + e;
                        float s = acc[i][j][NB - 1][r];
#pragma unroll
                        for (int b = NB - 2; b >= 0; --b) s = __builtin_fmaf(s, 0.00390625f, acc[i][j][b][r]);
                        out[e] = p.alpha * s;
                    }
                    if (vec_c) {
                        const int off = row_ok ? row * ldc4 + col * 4 : (int)0x80000000;
                        if (p.beta != 0.0f) {
                            const f32x4_t old = __builtin_bit_cast(
                                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
#pragma unroll
                            for (int e = 0; e < 4; ++e) out[e] = __builtin_fmaf(p.beta, old[e], out[e]);
                        }
                        if (p.bias != nullptr) {
                            const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(p.bias + c.n0() + col);
#pragma unroll
                            for (int e = 0; e < 4; ++e) out[e] = out[e] + bv[e];
                        }
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, out), rsrc,
                                                               off, 0, 0);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (row_ok && col + e < cols_left) {
                                float* cp = p.C + (c.m0 + row) * p.ldc + c.n0() + col + e;
                                float o = out[e];
                                if (p.beta != 0.0f) o = __builtin_fmaf(p.beta, *cp, o);
                                if (p.bias != nullptr) o = o + p.bias[c.n0() + col + e];
                                *cp = o;
                            }
                        }
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[i][j][b] = f32x16_t{};
            }
        return vec_c;
    };

    Cursor cc, cb, ca;   // tile being computed, plane loads step s+1, FP32 A step s+2
    cc.set(p, slot);
    cb = cc;
    ca = cc;
    // Prologue: planes of step 0 into buffers 0; FP32 A of step 1 in staging 1.
    copy_chunk(Wb, (int64_t)cb.tn * p.nk + cb.kt, smB[0]);
    if (FUSED_A) {
        copy_a32(ca, 0);
        ca.next(p, G);
        copy_a32(ca, 1);
        wait_vmcnt<0>();
        __syncthreads();
        split_stage(cc, 0, 0);
    } else {
        copy_chunk(Wa, (cb.m0 / TILE) * p.nk + cb.kt, smA[0]);
        wait_vmcnt<0>();
    }
    cb.next(p, G);
    ca.next(p, G);
    __syncthreads();

    // One pipeline step.  EPI: the tile finished by the previous step gets its
    // epilogue here, after this step's direct loads are issued, so the
    // step's wait (vmcnt(EPI_STORES)) covers the loads and leaves the stores
    // draining behind the next MFMAs.
    int pb = 0;
    auto step = [&]<bool EPI>(const Cursor& ce) __attribute__((always_inline)) {
        issue_loads(cb, ca, pb);
        bool vec_stores = false;
        if (EPI) {
            vec_stores = epilogue(ce);
            __builtin_amdgcn_sched_barrier(0);  // keep the next MFMAs' operand loads out of it
        }
        compute(pb, cb);
        if (vec_stores)
            wait_vmcnt<EPI_STORES>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        cb.next(p, G);
        ca.next(p, G);
        pb ^= 1;
    };

    for (int kt = 0; kt < p.nk; ++kt) step.template operator()<false>(cc);
    for (int tl = 1; tl < my_tiles; ++tl) {
        const Cursor ce = cc;
        cc.set(p, cc.tile + G);
        step.template operator()<true>(ce);
        for (int kt = 1; kt < p.nk; ++kt) step.template operator()<false>(cc);
    }
    epilogue(cc);
}

// ---------------------------------------------------------------------------
// Ping-pong form of the GEMM kernel for a k-contiguous FP32 op(A) (split in
// the kernel).  The 8 waves form two groups of four, one wave of each group
// per SIMD; group g owns rows 64g..64g+63 of the 128x128 tile, each of its
// waves a 64x32 block (two 32x32 MFMA tiles).  Each group alternates two
// kinds of phase, each closed by a workgroup barrier:
//   U(s): reads the group's FP32 A rows of step s+1 from staging, then
//         (while those reads are in flight) runs the epilogue of the tile
//         that ended at step s-1 and issues the direct loads of its half of
//         a B chunk (group 0: step s+1, group 1: step s+2) and of its A rows
//         of step s+2, then splits the step s+1 rows into the other plane
//         buffer;
//   M(s): the MFMAs of step s, then the scalar bookkeeping (advancing the
//         step cursors, precomputing addresses) for the next U phase, and
//         the wait for the group's half of B loaded in U(s).
// Group 1 starts one phase late, so U of one group runs beside M of the
// other: on every SIMD one wave keeps the matrix unit busy while the other
// does the vector, LDS and memory work.  Since a wave issues one instruction
// at a time, scalar work costs issue slots in a U phase but fills idle ones
// between the MFMAs of an M phase, which is where it is placed.  An M
// phase's fragment reads run one group of MFMAs ahead of their use, the
// first group's (A and B) before the barrier.  The split's LDS writes are only waited
// for at the end of the next M phase, and each thread splits exactly the A
// elements it loaded itself, so its own load-counter wait publishes them to
// itself.
// LDS: two plane buffers for A (each group touches only its own rows),
// three B chunk buffers (chunks s-1 .. s+1 while group 0 loads its half of
// s+1, s .. s+2 while group 1 loads its half of s+2), two FP32
// staging buffers (step s+2 overwrites step s, split in U(s-1)): 152 KB
// with three planes.
// ---------------------------------------------------------------------------

// GENERAL: the epilogue reads C (beta != 0) or adds a bias; the plain
// instantiation (C = alpha t) carries neither path, which saves it SGPR
// spills and registers in the loop (1.6 % on the 552,960-row stack).
// TH: rows of an output tile, 128 or 64 (the 64-row tiles give shapes with
// few tiles more of them; each group then owns 32 rows).
template <int NB, bool SPLIT, bool GENERAL, int TH>
__global__ __launch_bounds__(512, 1) void gemm_bf16_pp_kernel(Params p, const uint16_t* __restrict__ Wb)
{
    static_assert(!(SPLIT && GENERAL), "a split launch reads beta and the bias at run time");
    static_assert(TH == 128 || TH == 64, "output tiles of 128 or 64 rows");
    constexpr int NP = NB >= 3 ? 3 : NB;
    constexpr int CHUNK_BYTES = (int)chunk_elems(NP) * 2;
    constexpr int GT = 256;                                // threads per group
    constexpr int GROWS = TH / 2;                          // A rows per group
    constexpr int PSA = TH * LDS_ROW;                      // elements per A plane
    constexpr int B_ROUNDS = CHUNK_BYTES / (GT * 16);      // 4 KB rounds per B chunk
    constexpr int B_HALF = B_ROUNDS / 2;                   // rounds each group copies
    constexpr int A_ROUNDS = GROWS * BK * 4 / (GT * 16);   // 16-byte loads per thread
    constexpr int TM = GROWS / 32;                         // 32x32 MFMA blocks per wave
    static_assert(A_ROUNDS == TM && GROWS == TM * 32, "thread t splits rows t/8 + 32r of its group");
    static_assert(B_ROUNDS * GT * 16 == CHUNK_BYTES && B_HALF * 2 == B_ROUNDS, "B chunk in whole half rounds");
    __shared__ __attribute__((aligned(16))) uint16_t smA[2][NP * PSA];
    __shared__ __attribute__((aligned(16))) uint16_t smB[3][chunk_elems(NP)];
    __shared__ __attribute__((aligned(16))) float stage[2][TH * BK];

    const int G = gridDim.x;
    const int slot = xcd_position(blockIdx.x, G);
    // Items: tiles 0 .. split_from-1 whole, then (SPLIT) the ksplit K
    // segments of each of the other tiles; this workgroup's are slot, slot +
    // G, ...  (split_from is 0, every tile split, or a multiple of G: whole
    // rounds of whole tiles, then the last round's tiles split.)
    const int nsplit = SPLIT ? p.ntiles - p.split_from : 0;
    const int nitems = SPLIT ? p.split_from + nsplit * p.ksplit : p.ntiles;
    const int my_items = (nitems - slot + G - 1) / G;
    const int my_whole = SPLIT ? (slot < p.split_from ? (p.split_from - slot + G - 1) / G : 0) : my_items;
    const int total = my_whole * p.nk + (my_items - my_whole) * p.nk_item;

    WalkConst wc;
    const int gtile = G % p.ntiles;   // tiles added per advance
    wc.nk = p.nk;
    wc.nk_item = p.nk_item;
    wc.th = TH;
    wc.G = G;
    wc.split_from = SPLIT ? p.split_from : p.ntiles;
    wc.nsplit = nsplit > 0 ? nsplit : 1;
    wc.tiles_n = p.tiles_n;
    wc.gtn = gtile % p.tiles_n;
    wc.gm = (int64_t)(gtile / p.tiles_n) * TH;
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
    const int frag_k = (lane >> 5) * 8;

    // Thread gt of group g loads and splits rows GROWS g + gt/8 + 32r (r <
    // A_ROUNDS), k = 4(gt%8) .. +3 of each step's FP32 A tile.
    const int srow0 = GROWS * grp + (gt >> 3);
    const int skc = (gt & 7) * 4;
    uint32_t a_off[A_ROUNDS];
#pragma unroll
    for (int r = 0; r < A_ROUNDS; ++r)
        a_off[r] = (uint32_t)(((int64_t)(srow0 + 32 * r) * p.lda + skc) * 4);

    // Round r (of A_ROUNDS) of the group's FP32 A rows of step w into
    // staging buffer sb: staging is [TH][32] floats, this wave's 64 lanes
    // fill 1 KB at row GROWS g + 8 gw + 32 r.
    auto copy_a32_round = [&](const Walk& w, int sb, int r) __attribute__((always_inline)) {
        const float* base = p.A + w.arow + (int64_t)w.kt * BK;
        const uint32_t dst = lds_offset(stage[sb]) + GROWS * BK * 4 * grp + 1024 * gw;
        uint32_t off = a_off[r];
        if (w.rows != TH || w.kvalid != BK) {
            // rows past M re-read the tile's last row, k past K column 0
            // (both masked when split)
            const int row = srow0 + 32 * r;
            const int64_t rr = row < w.rows ? row : w.rows - 1;
            const int kk = skc < w.kvalid ? skc : 0;
            off = (uint32_t)((rr * p.lda + kk) * 4);
        }
        copy16_to_lds(dst + 4096 * r, base, off);
    };
    auto copy_a32 = [&](const Walk& w, int sb) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < A_ROUNDS; ++r) copy_a32_round(w, sb, r);
    };
    // This group's half of the B chunk of step w into buffer bb: rounds
    // B_HALF g .. B_HALF g + B_HALF - 1, round r the 4 KB at 4096 r, this
    // wave's 1 KB piece of it at 4096 r + 1024 gw.
    auto copy_b_half = [&](const Walk& w, int bb) __attribute__((always_inline)) {
        const char* src = reinterpret_cast<const char*>(Wb + ((int64_t)w.tn * p.nk + w.kt) * chunk_elems(NP));
        const uint32_t dst = lds_offset(smB[bb]);
#pragma unroll
        for (int j = 0; j < B_HALF; ++j) {
            const int byte0 = ((grp * B_HALF + j) * GT + gw * 64) * 16;
            copy16_to_lds(dst + byte0, src + byte0, (uint32_t)lane * 16);
        }
    };
    // The split of the group's rows of one step, in two parts: load_rows
    // reads the thread's FP32 values from staging buffer sb (on edge tiles,
    // elements outside op(A) selected to zero); split_rows splits them into
    // plane buffer ab.
    auto load_rows = [&](const Walk& w, int sb, f32x4_t (&v)[A_ROUNDS]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < A_ROUNDS; ++q)
            v[q] = *reinterpret_cast<const f32x4_t*>(&stage[sb][(srow0 + 32 * q) * BK + skc]);
        if (w.rows != TH || w.kvalid != BK) {
#pragma unroll
            for (int q = 0; q < A_ROUNDS; ++q) {
                const bool rok = srow0 + 32 * q < w.rows;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[q][e] = (rok && skc + e < w.kvalid) ? v[q][e] : 0.0f;
            }
        }
    };
    const int split_off = plane_elem(srow0, skc);   // rows 32 apart share the chunk order
    auto split_rows = [&](const f32x4_t (&v)[A_ROUNDS], int ab) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < A_ROUNDS; ++q) {
            uint32_t w0[NP], w1[NP];
            split_pieces<NP>(v[q][0], v[q][1], w0);
            split_pieces<NP>(v[q][2], v[q][3], w1);
            uint16_t* dst = smA[ab] + split_off + 32 * q * LDS_ROW;
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) *reinterpret_cast<u32x2_t*>(dst + pl * PSA) = u32x2_t{w0[pl], w1[pl]};
        }
    };

    // Accumulators: cleared here and after each tile's epilogue.
    f32x16_t acc[TM][NB];
    auto clear_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[i][b] = zero_acc();
    };
    clear_acc();

    // Operand fragments of k-half ks: this wave's B columns (all planes) in
    // B buffer bb and its A rows of plane u in plane buffer ab.  Fragment
    // rows start at multiples of 32, so the lane's offset within a plane is
    // frag_off0 (ks = 0) or frag_off1 (ks = 1) past the first row's.
    const int frag_off0 = plane_elem(frag_row, frag_k), frag_off1 = plane_elem(frag_row, 16 + frag_k);
    auto load_bfr = [&](int bb, int ks, bf16x8_t (&bfr)[NP]) __attribute__((always_inline)) {
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
            bfr[pl] = *reinterpret_cast<const bf16x8_t*>(smB[bb] + pl * PS + gw * 32 * LDS_ROW +
                                                         (ks ? frag_off1 : frag_off0));
    };
    auto load_afr = [&](int ab, int ks, int u, bf16x8_t (&af)[TM]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            af[i] = *reinterpret_cast<const bf16x8_t*>(smA[ab] + u * PSA + (grp * GROWS + i * 32) * LDS_ROW +
                                                       (ks ? frag_off1 : frag_off0));
    };
    // The MFMAs of one plane u of A against all planes of B (fragments
    // already in registers), smallest band first.
    auto mfma_u = [&](int u, const bf16x8_t (&bfr)[NP], const bf16x8_t (&af)[TM]) __attribute__((always_inline)) {
#pragma unroll
        for (int v = NP - 1; v >= 0; --v) {
            if (u + v < NB) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    // B operand first: lane l then holds row l%32 of the
                    // 32x32 block and four consecutive columns per register
                    // group, for 16-byte stores.
                    acc[i][u + v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[v], af[i], acc[i][u + v], 0, 0, 0);
            }
        }
    };

    // Epilogue of this wave's block of the item at w: bands recombined
    // smallest first into t, then C = alpha t + beta C + bias, or for a K
    // segment of a split tile (part) t itself into the segment's slot of the
    // workspace (TH x 128 floats, rows of 128).  Lane l holds, per 32x32
    // block and register group q, row l%32 and columns 8q + 4(l/32) .. +3:
    // one 16-byte buffer store each, rows outside C given an out-of-range
    // offset.  Tiles that cross column N, or a destination without 16-byte
    // rows, store element by element.  SCALE: alpha != 1.
    // In a split launch one copy serves both kinds of item, its destination
    // and scalars chosen at run time (a part: alpha 1, which is exact, no
    // beta, no bias; a whole tile takes them here, a split one in the
    // reduction).
    auto epilogue = [&]<bool SCALE>(const TilePos& w) __attribute__((always_inline)) {
        const int64_t n0 = (int64_t)w.tn * TILE;
        int64_t ldd = p.ldc;
        float* dst = p.C + w.m0 * p.ldc + n0;
        float alpha = p.alpha;
        float beta = GENERAL || SPLIT ? p.beta : 0.0f;
        const float* bias = GENERAL || SPLIT ? p.bias : nullptr;
        bool part = false;
        if constexpr (SPLIT) {
            part = w.part != 0;
            if (part) {
                ldd = TILE;
                dst = p.wsC + (int64_t)w.widx * (TH * TILE);
                alpha = 1.0f;
                beta = 0.0f;
                bias = nullptr;
            }
        }
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, 0x7FFFFFFF, 0x00020000);
        const int64_t cl = p.N - n0;
        const int cols_left = cl < TILE ? (int)cl : TILE;
        // vec_b / vec_ws carry the destination's (and the bias') alignment
        const bool vec_c = (part ? p.vec_ws : p.vec_b) != 0 && cols_left == TILE;
        const int ldd4 = (int)ldd * 4;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = grp * GROWS + i * 32 + (lane & 31);
            const bool row_ok = row < w.rows;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = gw * 32 + 8 * q + 4 * (lane >> 5);
                f32x4_t out;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * q + e;
                    float sum = acc[i][NB - 1][r];
#pragma unroll
                    for (int b = NB - 2; b >= 0; --b) sum = __builtin_fmaf(sum, 0.00390625f, acc[i][b][r]);
                    out[e] = SCALE ? alpha * sum : sum;
                }
                if (vec_c) {
                    const int off = row_ok ? row * ldd4 + col * 4 : (int)0x80000000;
                    if (beta != 0.0f) {
                        const f32x4_t old = __builtin_bit_cast(
                            f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
#pragma unroll
                        for (int e = 0; e < 4; ++e) out[e] = __builtin_fmaf(beta, old[e], out[e]);
                    }
                    if (bias != nullptr) {
                        // The wave's 8 bias values of register group q sit at a
                        // wave-uniform address: read them with one scalar load
                        // (counted by lgkmcnt, so waiting for it never waits for
                        // the direct loads in flight) and pick this lane's four.
                        const i32x8_t bv = scalar_load8(bias + n0 + gw * 32 + 8 * q);
                        const bool upper = (lane >> 5) != 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            // (opaque copies: otherwise the two selects fold into an
                            // index into bv and a chain of compares)
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
                            float* cp = dst + row * ldd + col + e;
                            float o = out[e];
                            if (beta != 0.0f) o = __builtin_fmaf(beta, *cp, o);
                            if (bias != nullptr) o = o + bias[n0 + col + e];
                            *cp = o;
                        }
                    }
                }
            }
        }
    };
    const bool unit_alpha = p.alpha == 1.0f;
    auto epilogue_any = [&](const TilePos& w) __attribute__((always_inline)) {
        if constexpr (SPLIT)
            epilogue.template operator()<true>(w);
        else if (unit_alpha)
            epilogue.template operator()<false>(w);
        else
            epilogue.template operator()<true>(w);
    };

    // Cursors: wm = step of the next M phase, we = the step before it (its
    // tile gets the epilogue when that step was the tile's last), ws = the
    // step after it (split, and its B chunk loaded, in the next U phase),
    // wa = the step of the next A load.
    Walk wm;
    if constexpr (SPLIT) {
        walk_set_item(wm, wc, slot);
    } else {
        wm.seg = 0;
        wm.tn = slot % p.tiles_n;
        wm.m0 = (int64_t)(slot / p.tiles_n) * TH;
        wm.kt = 0;
        wm.kt_end = p.nk;
        wm.item = slot;
        wm.part = 0;
        wm.widx = 0;
        walk_set_tile(wm, wc);
    }
    wm.left = my_items - 1;
    wm.kvalid = wm.kt + 1 < p.nk ? BK : wc.tail_k;
    Walk ws = wm, wa = wm;
    TilePos we{wm.m0, wm.tn, wm.rows, wm.seg, wm.part, wm.widx};
    // Prologue: B chunk of step 0 (each group its half) and group 1's half
    // of B chunk 1, then the FP32 A rows of steps 0 and 1, all issued before
    // one wait that leaves only the step-1 rows in flight (U(0) waits for
    // them); then the split of step 0 into plane buffer 0.  One memory
    // latency before the first MFMA instead of two for group 1: a few us on
    // a GEMM of a few tiles per CU.
    copy_b_half(ws, 0);
    if (grp == 1) {
        Walk w1 = ws;
        walk_next<SPLIT>(w1, wc);
        copy_b_half(w1, 1);
    }
    copy_a32(wa, 0);
    walk_next<SPLIT>(wa, wc);
    copy_a32(wa, 1);
    walk_next<SPLIT>(wa, wc);
    wait_vmcnt<A_ROUNDS>();
    {
        f32x4_t v0[A_ROUNDS];
        load_rows(ws, 0, v0);
        split_rows(v0, 0);
    }
    walk_next<SPLIT>(ws, wc);
    wait_lgkmcnt0();   // the split's LDS writes, published by the barrier
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 1) __builtin_amdgcn_s_barrier();   // group 1 runs one phase behind group 0

    // The epilogue runs before the U phase's direct loads: its stores then
    // issue ahead of those loads instead of queueing behind them (2-3 %
    // faster than the other order, results identical), and the compiler's
    // waits for its C loads (beta != 0) find no direct load of this phase
    // in flight.  Vector memory operations complete in issue order, so the
    // waits below also cover the stores.
    bool epi = false;       // U(s) runs the epilogue of step s-1's tile
    int bm = 0;             // B buffer of step s: s % 3
    for (int s = 0; s < total; ++s) {
        const int b = s & 1;
        const int bn = bm == 2 ? 0 : bm + 1;   // B buffer of step s+1
        // ---- U(s).  The A rows of step s+1 were loaded in U(s-1) (or the
        // prologue) into staging b^1, after that phase's epilogue stores and
        // half of B chunk s.
        wait_vmcnt<0>();
        f32x4_t sv[A_ROUNDS];
        load_rows(ws, b ^ 1, sv);
        if (epi) {
            epilogue_any(we);
            clear_acc();   // here, not in each epilogue variant: one copy of the clears
        }
        // Group 0 loads its half of B chunk s+1 (ws) into the buffer of step
        // s-2, group 1 its half of chunk s+2 (wa) into that of step s-1;
        // the last readers of each, M(s-2) and M(s-1) of both groups, ended
        // before this phase.  Each group waits for its half at the end of
        // its next M phase, so chunk s+1 is whole before U0(s+1) and both
        // groups read their first B fragments before the U->M barrier.
        if (grp == 0)
            copy_b_half(ws, bn);
        else
            copy_b_half(wa, bn == 2 ? 0 : bn + 1);
        copy_a32(wa, b);   // staging b held step s, split in U(s-1)
        // The first fragments of M(s) are read before the barrier where they
        // are already published: this group's A planes (split in U(s-1),
        // published by the barrier that ended M(s-1)) and B chunk s (both
        // halves landed before the barrier that ended the phase before
        // U0(s)).  They are issued before the split, which gives the
        // staging reads of load_rows longer to land.
        bf16x8_t bfr0[NP], atop0[TM];
        load_afr(b, 0, NP - 1, atop0);
        load_bfr(bm, 0, bfr0);
        split_rows(sv, b ^ 1);   // plane buffer b^1 was last read by M(s-1)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();   // the split's writes drain during M(s)
        __builtin_amdgcn_sched_barrier(0);
        // ---- M(s) on plane buffer b (split in U(s-1)) and B buffer bm, and
        // the cursor advances for U(s+1).  The MFMAs run in 2 NP groups,
        // (k-half, A plane u) = (0, NP-1) .. (0, 0), (1, NP-1) .. (1, 0); the
        // fragments of each group are read while the group before it issues
        // (the first group's before the barrier above).
        {
            bf16x8_t bq[2][NP], aq[2][TM];
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) bq[0][pl] = bfr0[pl];
#pragma unroll
            for (int i = 0; i < TM; ++i) aq[0][i] = atop0[i];
#pragma unroll
            for (int g = 0; g < 2 * NP; ++g) {
                const int half = g / NP, u = NP - 1 - g % NP;
                if (g + 1 < 2 * NP) {
                    const int nhalf = (g + 1) / NP, nu = NP - 1 - (g + 1) % NP;
                    if (nu == NP - 1) load_bfr(bm, nhalf, bq[nhalf]);
                    load_afr(b, nhalf, nu, aq[(g + 1) & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                mfma_u(u, bq[half], aq[g & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        epi = wm.kt == (SPLIT ? wm.kt_end : p.nk) - 1;
        we = TilePos{wm.m0, wm.tn, wm.rows, wm.seg, wm.part, wm.widx};
        // wm, ws, wa are the same sequence one and two steps apart (past the
        // end all stay on the last step): one advance, two copies
        wm = ws;
        ws = wa;
        walk_next<SPLIT>(wa, wc);
        bm = bn;
        // Before the next barrier: this thread's split writes of U(s) are
        // complete (the group reads them in M(s+1)); this group's half of B
        // loaded in U(s) (and the epilogue's stores before it) has landed,
        // while its A load of U(s), issued after it, may still be in flight.
        wait_lgkmcnt0();
        wait_vmcnt<A_ROUNDS>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }
    epilogue_any(we);
    wait_vmcnt<0>();   // no direct load may still be writing LDS when the workgroup ends
    if (grp == 0) __builtin_amdgcn_s_barrier();   // matches group 1's extra barrier
}

// ---------------------------------------------------------------------------
// Reduction of the split tiles: for split tile i (tile split_from + i),
// C = alpha (t_0 + t_1 + ... + t_{S-1}) + beta C + bias over the tile's rows
// and columns inside C, the segments' results added in segment order, each
// step one FP32 operation (C not read when beta == 0).  ws holds S x nsplit
// slots of th x 128 floats (rows of 128), slot seg * nsplit + i.  Workgroup
// (i, y) takes rows 8y .. 8y+7 of split tile i, one 4-column group per
// thread, so every load of the S segments is in flight at once (VEC:
// 16-byte accesses to C and the bias; N % 4 == 0, C rows and bias 16-byte
// aligned).
// ---------------------------------------------------------------------------
constexpr int RED_ROWS = 8;   // tile rows per reduction workgroup (256 threads)
static_assert(RED_ROWS * (TILE / 4) == 256, "one 4-column group per thread");

template <bool VEC>
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(
    const float* __restrict__ ws, int S, int nsplit, int split_from, int tiles_n, int th, int64_t M,
    int64_t N, float alpha, float beta, float* C, int64_t ldc, const float* __restrict__ bias)
{
    const int i = blockIdx.x;
    const int tile = split_from + i;
    const int tm = tile / tiles_n;
    const int tn = tile - tm * tiles_n;
    const int64_t m0 = (int64_t)tm * th, n0 = (int64_t)tn * TILE;
    const int r = blockIdx.y * RED_ROWS + (int)(threadIdx.x / (TILE / 4));
    const int cg = (int)(threadIdx.x % (TILE / 4)) * 4;
    if (m0 + r >= M || n0 + cg >= N) return;
    const int cols = N - n0 < TILE ? (int)(N - n0) : TILE;
    const int64_t slot = (int64_t)th * TILE;
    const int64_t seg_stride = (int64_t)nsplit * slot;
    const float* w = ws + (int64_t)i * slot + (int64_t)r * TILE + cg;
    float* c = C + (m0 + r) * ldc + n0 + cg;
    if (VEC) {
        f32x4_t t = *reinterpret_cast<const f32x4_t*>(w);
        for (int sg = 1; sg < S; ++sg) {
            const f32x4_t u = *reinterpret_cast<const f32x4_t*>(w + sg * seg_stride);
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = t[e] + u[e];
        }
        f32x4_t out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = alpha * t[e];
        if (beta != 0.0f) {
            const f32x4_t old = *reinterpret_cast<const f32x4_t*>(c);
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = __builtin_fmaf(beta, old[e], out[e]);
        }
        if (bias != nullptr) {
            const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(bias + n0 + cg);
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = out[e] + bv[e];
        }
        *reinterpret_cast<f32x4_t*>(c) = out;
    } else {
        for (int e = 0; e < 4 && cg + e < cols; ++e) {
            float t = w[e];
            for (int sg = 1; sg < S; ++sg) t = t + w[sg * seg_stride + e];
            float o = alpha * t;
            if (beta != 0.0f) o = __builtin_fmaf(beta, c[e], o);
            if (bias != nullptr) o = o + bias[n0 + cg + e];
            c[e] = o;
        }
    }
}

int grid_for(int64_t work)
{
    int64_t blocks = (work + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

using ShapeMain = Shape8;

template <int NB, int TH>
void launch_pp(const Params& p, int grid, const uint16_t* Wb, hipStream_t s)
{
    if (p.ksplit > 1)
        hipLaunchKernelGGL((gemm_bf16_pp_kernel<NB, true, false, TH>), dim3(grid), dim3(512), 0, s, p, Wb);
    else if (p.beta != 0.0f || p.bias != nullptr)
        hipLaunchKernelGGL((gemm_bf16_pp_kernel<NB, false, true, TH>), dim3(grid), dim3(512), 0, s, p, Wb);
    else
        hipLaunchKernelGGL((gemm_bf16_pp_kernel<NB, false, false, TH>), dim3(grid), dim3(512), 0, s, p, Wb);
}

// fused: the two-group kernel with tiles of tile_m (128 or 64) rows; else
// the one-barrier kernel on pre-split A (128-row tiles).
template <int NB>
hipError_t launch_main(const Params& p, bool fused, int tile_m, int grid, const uint16_t* Wb,
                       const uint16_t* Wa, hipStream_t s)
{
    constexpr int NT = ShapeMain::NT;
    if (fused && tile_m == 64)
        launch_pp<NB, 64>(p, grid, Wb, s);
    else if (fused)
        launch_pp<NB, 128>(p, grid, Wb, s);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<ShapeMain, NB, false>), dim3(grid), dim3(NT), 0, s, p, Wb, Wa);
    return hipGetLastError();
}

hipError_t launch_presplit(int np, const float* X, int64_t ld, bool kc, int64_t rows, int64_t K,
                           int tiles_r, int nk, uint16_t* W, hipStream_t s)
{
    const int grid = grid_for((int64_t)tiles_r * TILE * nk * (BK / 8));
    if (np == 3)
        hipLaunchKernelGGL(presplit_kernel<3>, dim3(grid), dim3(256), 0, s, X, ld, kc ? 1 : 0, rows,
                           K, tiles_r, nk, W);
    else if (np == 2)
        hipLaunchKernelGGL(presplit_kernel<2>, dim3(grid), dim3(256), 0, s, X, ld, kc ? 1 : 0, rows,
                           K, tiles_r, nk, W);
    else
        hipLaunchKernelGGL(presplit_kernel<1>, dim3(grid), dim3(256), 0, s, X, ld, kc ? 1 : 0, rows,
                           K, tiles_r, nk, W);
    return hipGetLastError();
}

}  // namespace

bool fused_a_path(const GemmArgs& g)
{
    // k-contiguous, 16-byte aligned rows whose every 16-byte group lies
    // inside the row, and 32-bit direct-load offsets
    return !g.trans_a && ((uintptr_t)g.A & 15u) == 0 && (g.lda & 3) == 0 && (g.K & 3) == 0 &&
           (int64_t)TILE * g.lda * 4 < ((int64_t)1 << 32);
}

namespace {

// The workspace's parts: pre-split B (and A when not fused), then the split
// tiles' partial results (ksplit slots of tile_m x 128 floats per split
// tile), each starting at a multiple of 256 bytes.
struct WsLayout {
    size_t b, a, c;   // offsets
    size_t total;
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

int effective_tile_m(const GemmArgs& g, int tile_m) { return fused_a_path(g) ? tile_m : TILE; }

WsLayout ws_layout(const GemmArgs& g, int nbands, int ksplit, int tile_m, int64_t split_from)
{
    tile_m = effective_tile_m(g, tile_m);
    const int64_t tiles_n = (g.N + TILE - 1) / TILE;
    const int64_t ntiles = (g.M + tile_m - 1) / tile_m * tiles_n;
    const int64_t nk = (g.K + BK - 1) / BK;
    const int np = nbands >= 3 ? 3 : nbands;
    const bool fused = fused_a_path(g);
    WsLayout w;
    w.b = 0;
    w.a = g.Bplanes != nullptr ? 0 : round256((size_t)(tiles_n * nk * chunk_elems(np)) * sizeof(uint16_t));
    w.c = w.a + (fused ? 0 : round256((size_t)((g.M + TILE - 1) / TILE * nk * chunk_elems(np)) * sizeof(uint16_t)));
    const int64_t nsplit = ntiles - (split_from > 0 && split_from < ntiles ? split_from : 0);
    w.total = w.c + (ksplit > 1 ? round256((size_t)ksplit * (size_t)nsplit * (size_t)tile_m * TILE * sizeof(float)) : 0);
    return w;
}

}  // namespace

size_t gemm_bf16_workspace_bytes(const GemmArgs& g, int nbands, int ksplit, int tile_m, int64_t split_from)
{
    return ws_layout(g, nbands, ksplit, tile_m, split_from).total;
}

size_t gemm_bf16_planes_bytes(int64_t N, int64_t K, int nbands)
{
    const int np = nbands >= 3 ? 3 : nbands;
    const int64_t tiles_n = (N + TILE - 1) / TILE;
    const int64_t nk = (K + BK - 1) / BK;
    return (size_t)(tiles_n * nk * chunk_elems(np)) * sizeof(uint16_t);
}

hipError_t launch_presplit_b(const float* B, int64_t ldb, bool trans_b, int64_t N, int64_t K,
                             int nbands, uint16_t* planes, hipStream_t stream)
{
    if (nbands != 5 && nbands != 3 && nbands != 2 && nbands != 1) return hipErrorInvalidValue;
    const int64_t tiles_n = (N + TILE - 1) / TILE;
    const int64_t nk = (K + BK - 1) / BK;
    const int64_t lim = (int64_t)1 << 31;
    if (tiles_n * nk >= lim || ((uintptr_t)planes & 15u) != 0) return hipErrorInvalidValue;
    return launch_presplit(nbands >= 3 ? 3 : nbands, B, ldb, trans_b, N, K, (int)tiles_n, (int)nk,
                           planes, stream);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, int nbands, int ksplit, int64_t split_from, int tile_m,
                            const DeviceInfo& dev, void* workspace, hipStream_t stream)
{
    if (nbands != 5 && nbands != 3 && nbands != 2 && nbands != 1) return hipErrorInvalidValue;
    if (tile_m != 128 && tile_m != 64) return hipErrorInvalidValue;
    const bool fused = fused_a_path(g);
    if (!fused) tile_m = TILE;   // the pre-split kernel has 128-row tiles only
    const int64_t tiles_m = (g.M + tile_m - 1) / tile_m;
    const int64_t tiles_n = (g.N + TILE - 1) / TILE;
    const int64_t ntiles = tiles_m * tiles_n;
    const int64_t nk = (g.K + BK - 1) / BK;
    const int64_t lim = (int64_t)1 << 31;
    if (ntiles >= lim || ntiles * nk >= lim || tiles_n * nk >= lim || tiles_m * nk >= lim)
        return hipErrorInvalidValue;
    const int64_t grid_all = ntiles < dev.num_cu ? ntiles : dev.num_cu;
    // a split of only the last round: whole rounds of whole tiles first, so
    // split_from must be a positive multiple of the grid below ntiles (0:
    // every tile split)
    if (ksplit > 1 && split_from != 0 &&
        (split_from < 0 || split_from >= ntiles || split_from % grid_all != 0))
        return hipErrorInvalidValue;
    if (ksplit <= 1) split_from = 0;
    const WsLayout lay = ws_layout(g, nbands, ksplit, tile_m, split_from);
    if (ksplit < 1 || nk % ksplit != 0 || (ksplit > 1 && !fused) ||
        split_from + (ntiles - split_from) * ksplit >= lim || (workspace == nullptr && lay.total > 0) ||
        ((uintptr_t)g.Bplanes & 15u) != 0)
        return hipErrorInvalidValue;

    Params p{};
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
    p.tiles_n = (int)tiles_n;
    p.ntiles = (int)ntiles;
    p.nk = (int)nk;
    p.ksplit = ksplit;
    p.nk_item = (int)(nk / ksplit);
    p.split_from = (int)split_from;
    p.vec_a = fused ? 1 : 0;
    // (emulated kernels) C rows allow 16-byte stores at 16-byte aligned
    // columns, and the bias (if any) 16-byte loads there
    p.vec_b = (((uintptr_t)g.C & 15u) == 0 && (g.ldc & 3) == 0 &&
               (g.bias == nullptr || ((uintptr_t)g.bias & 15u) == 0) &&
               (int64_t)TILE * g.ldc * 4 < ((int64_t)1 << 31)) ? 1 : 0;
    p.vec_ws = 1;   // slots of tile_m x 128 floats at 256-byte multiples: 16-byte rows

    const int np = nbands >= 3 ? 3 : nbands;
    char* ws = static_cast<char*>(workspace);
    // (the kernels only read the B planes)
    uint16_t* Wb = g.Bplanes != nullptr ? const_cast<uint16_t*>(g.Bplanes)
                                        : reinterpret_cast<uint16_t*>(ws + lay.b);
    uint16_t* Wa = fused ? nullptr : reinterpret_cast<uint16_t*>(ws + lay.a);
    p.wsC = ksplit > 1 ? reinterpret_cast<float*>(ws + lay.c) : nullptr;

    hipError_t e = hipSuccess;
    if (g.Bplanes == nullptr)
        e = launch_presplit(np, g.B, g.ldb, g.trans_b, g.N, g.K, (int)tiles_n, (int)nk, Wb, stream);
    if (e == hipSuccess && !fused)
        e = launch_presplit(np, g.A, g.lda, !g.trans_a, g.M, g.K, (int)tiles_m, (int)nk, Wa, stream);
    if (e == hipSuccess) {
        const int64_t items = split_from + (ntiles - split_from) * ksplit;
        const int grid = items < dev.num_cu ? (int)items : dev.num_cu;
        switch (nbands) {
        case 5: e = launch_main<5>(p, fused, tile_m, grid, Wb, Wa, stream); break;
        case 3: e = launch_main<3>(p, fused, tile_m, grid, Wb, Wa, stream); break;
        case 2: e = launch_main<2>(p, fused, tile_m, grid, Wb, Wa, stream); break;
        default: e = launch_main<1>(p, fused, tile_m, grid, Wb, Wa, stream); break;
        }
    }
    if (e == hipSuccess && ksplit > 1) {
        const int nsplit = (int)(ntiles - split_from);
        const bool vec = (g.N & 3) == 0 && ((uintptr_t)g.C & 15u) == 0 && (g.ldc & 3) == 0 &&
                         (g.bias == nullptr || ((uintptr_t)g.bias & 15u) == 0);
        const dim3 rgrid(nsplit, tile_m / RED_ROWS);
        if (vec)
            hipLaunchKernelGGL(ksplit_reduce_kernel<true>, rgrid, dim3(256), 0, stream, p.wsC, ksplit,
                               nsplit, (int)split_from, (int)tiles_n, tile_m, g.M, g.N, g.alpha, g.beta,
                               g.C, g.ldc, g.bias);
        else
            hipLaunchKernelGGL(ksplit_reduce_kernel<false>, rgrid, dim3(256), 0, stream, p.wsC, ksplit,
                               nsplit, (int)split_from, (int)tiles_n, tile_m, g.M, g.N, g.alpha, g.beta,
                               g.C, g.ldc, g.bias);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace emu
