// The matrix units' sustained rate on this part: every SIMD issues matrix
// instructions back to back, on register operands, with nothing else to do
// (no memory traffic beyond one store per thread at the end).  It bounds
// what any GEMM can reach here, the emulated one included: under a dense
// stream of bf16 matrix instructions the chip runs into its power limit and
// lowers the clock, so the sustained rate sits below the spec peak (which
// assumes the 2.4 GHz clock).  The same for the FP32 matrix instruction,
// the native path's roof.  gfx950 only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;   // independent accumulators per wave: issue never waits on a result

// A value in [-2, 2) from an integer hash of (thread, index).
__device__ __forceinline__ float operand(int gid, int k)
{
    uint32_t h = (uint32_t)gid * 0x9E3779B1u ^ (uint32_t)k * 0x85EBCA77u;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    return (float)(h >> 8) * (4.0f / 16777216.0f) - 2.0f;
}

// One 32x32x16 bf16 (BF16 = true) or 32x32x2 FP32 matrix instruction per
// chain per iteration.  Each wave records its shader-clock cycles
// (s_memtime) and real time (s_memrealtime, 100 MHz) over the loop.
template <bool BF16>
__global__ __launch_bounds__(256) void mfma_stream_kernel(float* __restrict__ out, int iters,
                                                          unsigned long long* __restrict__ clk)
{
    const int t = threadIdx.x;
    const int gid = blockIdx.x * blockDim.x + t;
    f32x16_t acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = f32x16_t{};
    // Pseudo-random operands, different per lane and per chain, so that
    // consecutive instructions switch the multipliers as real data does (a
    // repeated operand would draw less power and flatter the rate).
    bf16x8_t a[kChains], b[kChains];
    float fa[kChains], fb[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[j][e] = (__bf16)operand(gid, 16 * j + e);
            b[j][e] = (__bf16)operand(gid, 16 * j + 8 + e);
        }
        fa[j] = operand(gid, 100 + j);
        fb[j] = operand(gid, 200 + j);
    }
    const unsigned long long t0 = wall_clock64();
    const unsigned long long c0 = clock64();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) {
            if constexpr (BF16)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j], 0, 0, 0);
            else
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[j], fb[j], acc[j], 0, 0, 0);
        }
    }
    const unsigned long long c1 = clock64();
    const unsigned long long t1 = wall_clock64();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[gid] = s;
    if ((t & 63) == 0) {
        const int w = gid >> 6;
        clk[2 * w] = c1 - c0;
        clk[2 * w + 1] = t1 - t0;
    }
}

}  // namespace

// Runs the stream on every compute unit of the current device (two
// workgroups of 256 threads per CU: two waves per SIMD), one untimed launch
// of about 0.3 s, then one timed launch of about `seconds`.  which: 0 = bf16
// (v_mfma_f32_32x32x16_bf16), 1 = FP32 (v_mfma_f32_32x32x2_f32).  Outputs:
// the sustained rate in TFLOP/s (HIP events around the timed launch), the
// mean shader clock in GHz over the waves (their s_memtime cycles over
// their s_memrealtime time), and the launch's duration in seconds.
// Returns 0, or the HIP error code of the first call that failed (nothing
// is left allocated).
extern "C" int emu_ceiling_run(int which, double seconds, double* tflops, double* ghz, double* dur_s)
{
    if ((which != 0 && which != 1) || !(seconds > 0.0) || seconds > 30.0 || tflops == nullptr ||
        ghz == nullptr || dur_s == nullptr)
        return (int)hipErrorInvalidValue;
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    const int blocks = 2 * ncu, threads = 256;
    const int waves = blocks * threads / 64;
    float* out = nullptr;
    unsigned long long* clk = nullptr;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    // FLOP per instruction per wave, and the rate a first guess assumes
    // (per SIMD at 2 GHz), to size the loop
    const double flop_inst = which == 0 ? 32.0 * 32 * 16 * 2 : 32.0 * 32 * 2 * 2;
    const double simd_rate = (which == 0 ? 1024.0 : 64.0) * 2.0e9;   // FLOP/s per SIMD
    auto iters_for = [&](double s) {
        const double per_iter = kChains * flop_inst * 2 / simd_rate;   // two waves share a SIMD
        double it = s / per_iter;
        if (it < 1000.0) it = 1000.0;
        if (it > 2.0e9) it = 2.0e9;
        return (int)it;
    };
    auto launch = [&](int iters) {
        if (which == 0)
            hipLaunchKernelGGL(mfma_stream_kernel<true>, dim3(blocks), dim3(threads), 0, 0, out, iters, clk);
        else
            hipLaunchKernelGGL(mfma_stream_kernel<false>, dim3(blocks), dim3(threads), 0, 0, out, iters, clk);
        return hipGetLastError();
    };
    std::vector<unsigned long long> host((size_t)waves * 2);
    e = hipMalloc(&out, (size_t)blocks * threads * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&clk, (size_t)waves * 2 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipEventCreate(&ev0);
    if (e == hipSuccess) e = hipEventCreate(&ev1);
    const int iters = iters_for(seconds);
    if (e == hipSuccess) e = launch(iters_for(0.3));
    if (e == hipSuccess) e = hipEventRecord(ev0, 0);
    if (e == hipSuccess) e = launch(iters);
    if (e == hipSuccess) e = hipEventRecord(ev1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(ev1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev0, ev1);
    if (e == hipSuccess)
        e = hipMemcpy(host.data(), clk, host.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    if (e == hipSuccess) {
        double cyc = 0.0, rt = 0.0;
        for (int w = 0; w < waves; ++w) {
            cyc += (double)host[2 * w];
            rt += (double)host[2 * w + 1];
        }
        *tflops = (double)waves * iters * kChains * flop_inst / (ms * 1e-3) / 1e12;
        *ghz = rt > 0.0 ? cyc / rt * 0.1 : 0.0;   // s_memrealtime ticks at 100 MHz
        *dur_s = ms * 1e-3;
    }
    if (ev0) (void)hipEventDestroy(ev0);
    if (ev1) (void)hipEventDestroy(ev1);
    if (out) (void)hipFree(out);
    if (clk) (void)hipFree(clk);
    return (int)e;
}
