// Tiling, scheduling and data-movement helpers shared by the GEMM kernels
// (gfx950 only).
#pragma once

#include "emu_device.h"
#include "emu_launch.h"

namespace emu {

constexpr int BK = 32;             // k extent of one pipeline step
constexpr int TILE = 128;          // output tile is TILE x TILE
constexpr int LDS_ROW = BK;        // bf16 elements per row of an LDS plane: 64 bytes, no padding
constexpr int LDSF_ROW = BK + 4;   // fp32 elements per LDS row (native kernel): 144 bytes

// One GEMM call as the kernels see it (row-major; op(A) M x K, op(B) K x N).
struct Params {
    const float* A;
    const float* B;
    float* C;
    int64_t lda, ldb, ldc;
    int64_t M, N, K;
    float alpha, beta;
    const float* bias;   // length N, added to every row of C after alpha/beta; null: none
    int tiles_n;   // output tiles along N
    int ntiles;    // output tiles in total
    int nk;        // k-steps per tile
    int vec_a;     // op(A) rows may be read with 16-byte loads
    // gemm_f32_kernel: op(B) columns may be read with 16-byte loads; kernels
    // with the 16-byte epilogue: C rows (and the bias) allow 16-byte access
    int vec_b;
    // Split of K into ksplit equal segments of nk_item k-steps (fused-A
    // kernel only; 1: none), for the tiles from split_from on (0: every
    // tile; otherwise a multiple of the grid: whole rounds of whole tiles
    // first).  With ksplit > 1 the kernel writes each (segment, split tile)
    // result t, unscaled, to its slot of wsC (tile_m x 128 floats, slot
    // seg * (ntiles - split_from) + tile - split_from; vec_ws: 16-byte stores
    // allowed there) and a reduction kernel forms C on those tiles.
    int ksplit, nk_item, split_from;
    float* wsC;
    int vec_ws;
};

// Bijection on [0, G): hardware workgroup id -> position in the tile list.
// Workgroup b runs on XCD b % 8; the workgroups of one XCD take a contiguous
// range of positions, so tiles that share rows of A run on the same XCD and
// share its L2.
__device__ __forceinline__ int xcd_position(int b, int G)
{
    const int q = G >> 3, r = G & 7;
    const int x = b & 7, s = b >> 3;
    return x * q + (x < r ? x : r) + s;
}

// Position in the workgroup's static tile list plus k-step.  next()
// saturates at the last (tile, k-step), so prefetches past the end re-read
// valid data instead of running off the operands.  Tiles are ordered with n
// fastest.
struct Cursor {
    int tile, kt, tn;
    int64_t m0;
    __device__ __forceinline__ void set(const Params& p, int t)
    {
        tile = t;
        kt = 0;
        const int tm = t / p.tiles_n;
        tn = t - tm * p.tiles_n;
        m0 = (int64_t)tm * TILE;
    }
    __device__ __forceinline__ void next(const Params& p, int G)
    {
        if (kt + 1 < p.nk)
            ++kt;
        else if (tile + G < p.ntiles)
            set(p, tile + G);
    }
    __device__ __forceinline__ int64_t n0() const { return (int64_t)tn * TILE; }
    __device__ __forceinline__ int64_t k0() const { return (int64_t)kt * BK; }
};

// Store one 32x32 MFMA result tile: lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32.  C = alpha t + beta C + bias,
// C not read when beta == 0.
__device__ __forceinline__ void store_c_tile(const Params& p, const float (&t)[16], int64_t row0,
                                             int64_t col0)
{
    const int lane = threadIdx.x & 63;
    const int64_t col = col0 + (lane & 31);
    if (col >= p.N) return;
    const float bias = p.bias != nullptr ? p.bias[col] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < p.M) {
            float* c = p.C + row * p.ldc + col;
            float out = p.alpha * t[r];
            if (p.beta != 0.0f) out = __builtin_fmaf(p.beta, *c, out);
            if (p.bias != nullptr) out = out + bias;
            *c = out;
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

// Wait until all of this wave's LDS operations have completed (vmcnt and
// expcnt left at their maxima).
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);
}

__device__ __forceinline__ uint32_t lds_offset(const void* p)
{
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

__device__ __forceinline__ const void* uniform_ptr(const void* p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Eight consecutive 32-bit words at a wave-uniform address, read through the
// scalar data cache into SGPRs (s_load_dwordx8), for read-only data such as
// a bias.  The wait is lgkmcnt(0): it never waits for vector memory
// operations.  Inline assembly, because the compiler may turn uniform loads
// whose values are then chosen per lane into one vector load per lane.
__device__ __forceinline__ i32x8_t scalar_load8(const void* p)
{
    i32x8_t v;
    asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
    return v;
}

// Direct global->LDS copy of 16 bytes per lane: lane l reads gbase + voff
// and its bytes land at LDS offset lds_base + 16 l (gbase and lds_base
// wave-uniform).  Inline assembly keeps the compiler from guarding later LDS
// reads with waits for this load: the caller waits (wait_vmcnt) before the
// barrier that publishes the data.
__device__ __forceinline__ void copy16_to_lds(uint32_t lds_base, const void* gbase, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(uniform_ptr(gbase))
                 : "memory");
}

}  // namespace emu
