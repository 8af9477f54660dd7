// The exact three-piece split as a stand-alone kernel ("Unlocking Tensor Core
// Performance for Machine Learning Interatomic Potentials", section "How
// Tensor Core FP32 bridges the hardware gap", Figure 1): FP32[n] -> BF16
// planes hi, mid', lo'.  It runs the same split_pair() as the GEMM staging,
// plus the non-finite convention (hi = +-inf or quiet NaN, mid' = lo' = +0).
//
// HBM-bound (4 bytes read, 6 written per element): each thread handles 8
// consecutive elements per step with two 16-byte loads and three 16-byte
// stores; a grid-stride loop covers n, unaligned heads and tails go scalar.
#include "emu_device.h"
#include "emu_launch.h"

namespace emu {
namespace {

// Non-finite fix-up of one packed pair: x0 in the low half, x1 in the high.
__device__ __forceinline__ void fix_nonfinite(float x0, float x1, uint32_t& hi, uint32_t& mid,
                                              uint32_t& lo)
{
    const uint32_t b[2] = {__float_as_uint(x0), __float_as_uint(x1)};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        if ((b[e] & 0x7F800000u) == 0x7F800000u) {
            const uint32_t sign = (b[e] >> 16) & 0x8000u;
            const uint32_t h = sign | ((b[e] & 0x007FFFFFu) ? 0x7FC0u : 0x7F80u);
            const uint32_t mask = e ? 0xFFFF0000u : 0x0000FFFFu;
            const uint32_t sh = e ? 16 : 0;
            hi = (hi & ~mask) | (h << sh);
            mid &= ~mask;
            lo &= ~mask;
        }
    }
}

__device__ __forceinline__ void split_fixed(float x0, float x1, uint32_t& hi, uint32_t& mid,
                                            uint32_t& lo)
{
    split_pair<true>(x0, x1, hi, mid, lo);
    fix_nonfinite(x0, x1, hi, mid, lo);
}

__global__ void split_vec_kernel(const float* __restrict__ x, int64_t n8, uint16_t* __restrict__ hi,
                                 uint16_t* __restrict__ mid, uint16_t* __restrict__ lo)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
         i += (int64_t)gridDim.x * blockDim.x) {
        const f32x4_t v0 = reinterpret_cast<const f32x4_t*>(x)[2 * i];
        const f32x4_t v1 = reinterpret_cast<const f32x4_t*>(x)[2 * i + 1];
        uint32_t h[4], m[4], l[4];
        split_fixed(v0[0], v0[1], h[0], m[0], l[0]);
        split_fixed(v0[2], v0[3], h[1], m[1], l[1]);
        split_fixed(v1[0], v1[1], h[2], m[2], l[2]);
        split_fixed(v1[2], v1[3], h[3], m[3], l[3]);
        reinterpret_cast<u32x4_t*>(hi)[i] = u32x4_t{h[0], h[1], h[2], h[3]};
        reinterpret_cast<u32x4_t*>(mid)[i] = u32x4_t{m[0], m[1], m[2], m[3]};
        reinterpret_cast<u32x4_t*>(lo)[i] = u32x4_t{l[0], l[1], l[2], l[3]};
    }
}

__global__ void split_scalar_kernel(const float* __restrict__ x, int64_t n,
                                    uint16_t* __restrict__ hi, uint16_t* __restrict__ mid,
                                    uint16_t* __restrict__ lo)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        uint32_t h, m, l;
        split_fixed(x[i], 0.0f, h, m, l);
        hi[i] = (uint16_t)h;
        mid[i] = (uint16_t)m;
        lo[i] = (uint16_t)l;
    }
}

int grid_for(int64_t work, int threads)
{
    int64_t blocks = (work + threads - 1) / threads;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

}  // namespace

hipError_t launch_split(const float* x, int64_t n, uint16_t* hi, uint16_t* mid, uint16_t* lo,
                        hipStream_t stream)
{
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
    int64_t head = 0;
    if (a16(x) && a16(hi) && a16(mid) && a16(lo)) {
        const int64_t n8 = n / 8;
        if (n8 > 0) {
            hipLaunchKernelGGL(split_vec_kernel, dim3(grid_for(n8, 256)), dim3(256), 0, stream, x,
                               n8, hi, mid, lo);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        head = n8 * 8;
    }
    const int64_t rest = n - head;
    if (rest > 0) {
        hipLaunchKernelGGL(split_scalar_kernel, dim3(grid_for(rest, 256)), dim3(256), 0, stream,
                           x + head, rest, hi + head, mid + head, lo + head);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace emu
