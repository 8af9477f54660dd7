// Internal interface between the C-ABI layer (emu_api.hip) and the kernel
// translation units.  Not installed; callers use include/emu_sgemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace emu {

// One GEMM call after validation: row-major, op(A) M x K, op(B) K x N.
struct GemmArgs {
    bool trans_a, trans_b;
    int64_t M, N, K;
    float alpha, beta;
    const float* A;
    int64_t lda;
    const float* B;
    int64_t ldb;
    float* C;
    int64_t ldc;
    const float* bias;   // length N or null
    // op(B) already split by launch_presplit_b (same N, K and plane count),
    // or null: the call splits op(B) into its workspace
    const uint16_t* Bplanes = nullptr;
};

struct DeviceInfo {
    int device;          // HIP device index
    int num_cu;          // compute units of the current device
    hipMemPool_t pool;   // library-owned pool for the workspaces (null: the device's default pool)
};

// Bytes of freed workspace the library's pool keeps mapped for reuse; larger
// workspaces go back to the device at the stream's next synchronisation.
constexpr uint64_t kPoolKeepBytes = 256ull << 20;

// Whether the emulated path splits op(A) in its main kernel (k-contiguous,
// aligned A); otherwise A is pre-split and K cannot be split.
bool fused_a_path(const GemmArgs& g);
// Device workspace the emulated path needs (bytes, a multiple of 256), and
// the launch with it: nbands 5 (BF16X9), 3 (BF16X6), 2 (BF16X3) or 1
// (BF16X1); ksplit K segments, a divisor of ceil(K / 32), 1 unless
// fused_a_path(g), for the output tiles from split_from on (0: all; else a
// positive multiple of min(tiles, CUs) below the tile count: whole rounds
// of whole tiles, then the last round's tiles split); tile_m the rows of an output tile, 128 or 64 (64 only on the fused
// path, otherwise 128 is used; the result does not depend on it; the tiles
// split_from counts are of that height); `workspace` 256-byte aligned,
// used in stream order only.
size_t gemm_bf16_workspace_bytes(const GemmArgs& g, int nbands, int ksplit, int tile_m,
                                 int64_t split_from);
hipError_t launch_gemm_bf16(const GemmArgs& g, int nbands, int ksplit, int64_t split_from, int tile_m,
                            const DeviceInfo& dev, void* workspace, hipStream_t stream);
// The native FP32 GEMM: its device workspace (bytes, a multiple of 256; 0
// when the call takes the kernel that needs none) and the launch with it
// (`workspace` 16-byte aligned, used in stream order only).
size_t gemm_native_f32_workspace_bytes(const GemmArgs& g);
hipError_t launch_gemm_native_f32(const GemmArgs& g, const DeviceInfo& dev, void* workspace,
                                  hipStream_t stream);
// The BF16 planes of op(B) (K x N; element (k, n) is B[n*ldb + k] when
// trans_b, else B[k*ldb + n]) in the layout the emulated kernels read:
// their size in bytes, and the split into `planes` (16-byte aligned) for
// nbands 5, 3, 2 or 1.
size_t gemm_bf16_planes_bytes(int64_t N, int64_t K, int nbands);
hipError_t launch_presplit_b(const float* B, int64_t ldb, bool trans_b, int64_t N, int64_t K,
                             int nbands, uint16_t* planes, hipStream_t stream);
// C = beta * C + bias over M x N (C not read when beta == 0; bias may be null).
hipError_t launch_scale_c(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                          const float* bias, hipStream_t stream);
hipError_t launch_split(const float* x, int64_t n, uint16_t* hi, uint16_t* mid, uint16_t* lo,
                        hipStream_t stream);

}  // namespace emu
