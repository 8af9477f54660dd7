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

constexpr int NT = 512;            // threads per workgroup
constexpr int WAVES_N = 4;         // waves along n (2 along m)
constexpr int TM = 2;              // 32x32 tiles per wave along m
constexpr int TN = 1;              // along n
constexpr int PS = TILE * LDS_ROW; // elements per plane of an LDS tile

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
template <int NB, bool FUSED_A>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(Params p, const uint16_t* __restrict__ Wb,
                                                          const uint16_t* __restrict__ Wa)
{
    constexpr int NP = NB >= 3 ? 3 : 2;  // planes used: hi, mid' (, lo')
    constexpr int CHUNK_BYTES = (int)chunk_elems(NP) * 2;
    constexpr int COPY_ROUNDS = (CHUNK_BYTES + NT * 16 - 1) / (NT * 16);
    constexpr int STAGE_FLOATS = TILE * BK;
    constexpr int STAGE_ROUNDS = STAGE_FLOATS * 4 / (NT * 16);   // 2
    constexpr int MFMA_PER_KS = TM * TN * (NB == 5 ? 9 : NB == 3 ? 6 : 3);
    static_assert(STAGE_ROUNDS * NT * 16 == STAGE_FLOATS * 4, "staging copy rounds");
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

    // Split/staging geometry: thread t owns rows t/8 and t/8 + 64, k t%8*4.
    const int srow = t >> 3;
    const int skc = (t & 7) * 4;
    // Direct-load byte offsets of the FP32 A tile (interior tiles).
    uint32_t a_off[STAGE_ROUNDS];
#pragma unroll
    for (int r = 0; r < STAGE_ROUNDS; ++r)
        a_off[r] = (uint32_t)(((int64_t)(srow + 64 * r) * p.lda + skc) * 4);

    auto copy_chunk = [&](const uint16_t* W, int64_t chunk, uint16_t* dst_tile) {
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
    auto copy_a32 = [&](const Cursor& c, int sb) {
        const float* base = p.A + c.m0 * p.lda + c.k0();
        const uint32_t dst = lds_offset(stage[sb]);
        const bool interior = c.m0 + TILE <= p.M && c.k0() + BK <= p.K;
#pragma unroll
        for (int r = 0; r < STAGE_ROUNDS; ++r) {
            uint32_t off = a_off[r];
            if (!interior) {
                const int64_t row = srow + 64 * r;
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
    auto issue_loads = [&](const Cursor& cb, const Cursor& ca, int pb) {
        copy_chunk(Wb, (int64_t)cb.tn * p.nk + cb.kt, smB[pb ^ 1]);
        if (FUSED_A)
            copy_a32(ca, pb);
        else
            copy_chunk(Wa, (cb.m0 / TILE) * p.nk + cb.kt, smA[pb ^ 1]);
    };

    // Split the FP32 tile in staging buffer sb (step described by c) into the
    // planes of plane buffer pb.
    auto split_stage = [&](const Cursor& c, int sb, int pb) {
        const bool interior = c.m0 + TILE <= p.M && c.k0() + BK <= p.K;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int row = srow + 64 * q;
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
    auto mfma_half = [&](int pb, int ks) {
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
                            acc[i][j][u + v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                af[i], bfr[v][j], acc[i][j][u + v], 0, 0, 0);
                }
            }
        }
    };

    // One step's compute: the MFMAs of both k-halves, with (FUSED_A) the
    // split of the next step's A tile spread evenly between them.
    auto compute = [&](int pb, const Cursor& cnext) {
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

    auto epilogue = [&](const Cursor& c) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                float tt[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s = acc[i][j][NB - 1][r];
#pragma unroll
                    for (int b = NB - 2; b >= 0; --b) s = __builtin_fmaf(s, 0.00390625f, acc[i][j][b][r]);
                    tt[r] = s;
                }
                store_c_tile(p, tt, c.m0 + (wm * TM + i) * 32, c.n0() + (wn * TN + j) * 32);
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[i][j][b] = f32x16_t{};
            }
    };

    Cursor cc, cb, ca;   // compute step s, plane loads step s+1, FP32 A step s+2
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

    int kt = 0, pb = 0;
    for (int s = 0; s < total; ++s) {
        issue_loads(cb, ca, pb);
        compute(pb, cb);
        wait_vmcnt<0>();
        __syncthreads();
        if (kt == p.nk - 1) {
            epilogue(cc);
            if (cc.tile + G < p.ntiles) cc.set(p, cc.tile + G);
        }
        cb.next(p, G);
        ca.next(p, G);
        kt = (kt + 1 == p.nk) ? 0 : kt + 1;
        pb ^= 1;
    }
}

int grid_for(int64_t work)
{
    int64_t blocks = (work + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

template <int NB>
hipError_t launch_main(const Params& p, bool fused, int grid, const uint16_t* Wb,
                       const uint16_t* Wa, hipStream_t s)
{
    if (fused)
        hipLaunchKernelGGL((gemm_bf16_kernel<NB, true>), dim3(grid), dim3(NT), 0, s, p, Wb, Wa);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<NB, false>), dim3(grid), dim3(NT), 0, s, p, Wb, Wa);
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
    p.vec_b = 0;

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
