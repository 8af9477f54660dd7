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
//     rows x 40 bf16 (32 k + 8 pad), zero outside op(B).  The GEMM kernel
//     copies chunks to LDS with direct global->LDS loads: no registers, no
//     VALU, no bounds checks.
//   * op(A) (the activations: large, streamed once per n-tile) is split in
//     the kernel: its FP32 tile is copied to an LDS staging buffer with the
//     same direct loads, then each thread reads its 2 rows x 4 k, splits them
//     in registers and writes the BF16 planes.  When A is transposed or not
//     16-byte addressable, it is pre-split like B instead.
//   * Persistent launch: one 512-thread workgroup per CU walks a static,
//     XCD-aware list of 128x128 output tiles; the k-steps of consecutive
//     tiles form one software pipeline with one barrier per step.
//   * 8 waves (two per SIMD) each own a 64x32 block of C as two
//     v_mfma_f32_32x32x16_bf16 tiles with one FP32 accumulator per band
//     (5 x 2 x 16 = 160 registers in the nine-product mode).  The split work
//     of a step is interleaved with the step's MFMAs, so that the matrix
//     unit keeps running while the vector ALU splits.
//   * Epilogue: bands are recombined smallest first (t = S_{n-1},
//     t = S_j + 2^-8 t), then C = alpha t + beta C.
#include "emu_tile.h"

namespace emu {
namespace {

constexpr int PS = TILE * LDS_ROW; // elements per plane of an LDS tile

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
// [tile row][k-step][plane][128][LDS_ROW].  Element (r, k) is X[r*ld + k]
// when kc (k contiguous) and X[k*ld + r] otherwise.  One thread per (row,
// 8-wide k group) of the padded extent; rows past `rows` and k past K are
// zero.  The 8 padding columns of each row are not written (never read).
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
        uint32_t h[4], m[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (NP == 3)
                split_pair<true>(v[2 * e], v[2 * e + 1], h[e], m[e], l[e]);
            else
                split_pair_hm(v[2 * e], v[2 * e + 1], h[e], m[e]);
        }
        const int64_t tr = r / TILE, rr = r - tr * TILE;
        const int64_t kt = k0 / BK, kk = k0 - kt * BK;
        uint16_t* chunk = W + (tr * nk + kt) * chunk_elems(NP);
        const int64_t off = rr * LDS_ROW + kk;
        *reinterpret_cast<u32x4_t*>(chunk + off) = u32x4_t{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<u32x4_t*>(chunk + PS + off) = u32x4_t{m[0], m[1], m[2], m[3]};
        if (NP == 3)
            *reinterpret_cast<u32x4_t*>(chunk + 2 * PS + off) = u32x4_t{l[0], l[1], l[2], l[3]};
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
    constexpr int NP = NB >= 3 ? 3 : 2;  // planes used: hi, mid' (, lo')
    constexpr int CHUNK_BYTES = (int)chunk_elems(NP) * 2;
    constexpr int COPY_ROUNDS = (CHUNK_BYTES + NT * 16 - 1) / (NT * 16);
    constexpr int STAGE_FLOATS = TILE * BK;
    constexpr int STAGE_ROUNDS = STAGE_FLOATS * 4 / (NT * 16);
    constexpr int MFMA_PER_KS = TM * TN * (NB == 5 ? 9 : NB == 3 ? 6 : 3);
    static_assert(STAGE_ROUNDS * NT * 16 == STAGE_FLOATS * 4 && STAGE_ROUNDS == SROWS,
                  "each thread splits the rows it copied");
    __shared__ __attribute__((aligned(16))) uint16_t smA[2][chunk_elems(NP)];
    __shared__ __attribute__((aligned(16))) uint16_t smB[2][chunk_elems(NP)];
    __shared__ __attribute__((aligned(16))) float stage[FUSED_A ? 2 : 1][FUSED_A ? STAGE_FLOATS : 4];

    const int G = gridDim.x;
    const int slot = xcd_position(blockIdx.x, G);
    const int my_tiles = (p.ntiles - slot + G - 1) / G;
    const int total = my_tiles * p.nk;

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
            uint32_t h0, m0, l0, h1, m1, l1;
            if (NP == 3) {
                split_pair<true>(v[0], v[1], h0, m0, l0);
                split_pair<true>(v[2], v[3], h1, m1, l1);
            } else {
                split_pair_hm(v[0], v[1], h0, m0);
                split_pair_hm(v[2], v[3], h1, m1);
            }
            uint16_t* dst = smA[pb] + row * LDS_ROW + skc;
            *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{h0, h1};
            *reinterpret_cast<u32x2_t*>(dst + PS) = u32x2_t{m0, m1};
            if (NP == 3) *reinterpret_cast<u32x2_t*>(dst + 2 * PS) = u32x2_t{l0, l1};
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
                bfr[pl][j] = *reinterpret_cast<const bf16x8_t*>(Bs + pl * PS + col * LDS_ROW +
                                                                ks * 16 + frag_k);
            }
#pragma unroll
        for (int u = NP - 1; u >= 0; --u) {
            bf16x8_t af[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = (wm * TM + i) * 32 + frag_row;
                af[i] = *reinterpret_cast<const bf16x8_t*>(As + u * PS + row * LDS_ROW + ks * 16 +
                                                           frag_k);
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
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, out), rsrc,
                                                               off, 0, 0);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (row_ok && col + e < cols_left) {
                                float* cp = p.C + (c.m0 + row) * p.ldc + c.n0() + col + e;
                                float o = out[e];
                                if (p.beta != 0.0f) o = __builtin_fmaf(p.beta, *cp, o);
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

int grid_for(int64_t work)
{
    int64_t blocks = (work + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

using ShapeMain = Shape8;

template <int NB>
hipError_t launch_main(const Params& p, bool fused, int grid, const uint16_t* Wb,
                       const uint16_t* Wa, hipStream_t s)
{
    constexpr int NT = ShapeMain::NT;
    if (fused)
        hipLaunchKernelGGL((gemm_bf16_kernel<ShapeMain, NB, true>), dim3(grid), dim3(NT), 0, s, p, Wb, Wa);
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
    else
        hipLaunchKernelGGL(presplit_kernel<2>, dim3(grid), dim3(256), 0, s, X, ld, kc ? 1 : 0, rows,
                           K, tiles_r, nk, W);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, int nbands, const DeviceInfo& dev,
                            hipStream_t stream)
{
    if (nbands != 5 && nbands != 3 && nbands != 2) return hipErrorInvalidValue;
    const int64_t tiles_m = (g.M + TILE - 1) / TILE;
    const int64_t tiles_n = (g.N + TILE - 1) / TILE;
    const int64_t nk = (g.K + BK - 1) / BK;
    const int64_t lim = (int64_t)1 << 31;
    if (tiles_m * tiles_n >= lim || tiles_m * tiles_n * nk >= lim || tiles_n * nk >= lim ||
        tiles_m * nk >= lim)
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
    p.tiles_n = (int)tiles_n;
    p.ntiles = (int)(tiles_m * tiles_n);
    p.nk = (int)nk;
    // Fused split of A: k-contiguous, 16-byte aligned rows whose every
    // 16-byte group lies inside the row, and 32-bit direct-load offsets.
    const bool fused = !g.trans_a && ((uintptr_t)g.A & 15u) == 0 && (g.lda & 3) == 0 &&
                       (g.K & 3) == 0 && (int64_t)TILE * g.lda * 4 < ((int64_t)1 << 32);
    p.vec_a = fused ? 1 : 0;
    // (emulated kernel) C rows allow 16-byte stores at 16-byte aligned columns
    p.vec_b = (((uintptr_t)g.C & 15u) == 0 && (g.ldc & 3) == 0 &&
               (int64_t)TILE * g.ldc * 4 < ((int64_t)1 << 31)) ? 1 : 0;

    const int np = nbands >= 3 ? 3 : 2;
    const size_t bytes_b = (size_t)(tiles_n * nk * chunk_elems(np)) * sizeof(uint16_t);
    const size_t bytes_a = fused ? 0 : (size_t)(tiles_m * nk * chunk_elems(np)) * sizeof(uint16_t);
    uint16_t* ws = nullptr;
    hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&ws), bytes_b + bytes_a, stream);
    if (e != hipSuccess) return hipErrorOutOfMemory;
    uint16_t* Wb = ws;
    uint16_t* Wa = fused ? nullptr : ws + bytes_b / sizeof(uint16_t);

    e = launch_presplit(np, g.B, g.ldb, g.trans_b, g.N, g.K, (int)tiles_n, (int)nk, Wb, stream);
    if (e == hipSuccess && !fused)
        e = launch_presplit(np, g.A, g.lda, !g.trans_a, g.M, g.K, (int)tiles_m, (int)nk, Wa, stream);
    if (e == hipSuccess) {
        const int grid = p.ntiles < dev.num_cu ? p.ntiles : dev.num_cu;
        switch (nbands) {
        case 5: e = launch_main<5>(p, fused, grid, Wb, Wa, stream); break;
        case 3: e = launch_main<3>(p, fused, grid, Wb, Wa, stream); break;
        default: e = launch_main<2>(p, fused, grid, Wb, Wa, stream); break;
        }
    }
    const hipError_t ef = hipFreeAsync(ws, stream);
    return e != hipSuccess ? e : ef;
}

}  // namespace emu
