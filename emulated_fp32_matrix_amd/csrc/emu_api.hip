// C ABI of the emulated-FP32 GEMM library (declarations and full contract in
// include/emu_sgemm.h): argument validation, the per-shape dispatcher and the
// launches on the caller's stream.
//
// The dispatcher implements the "performant" policy of "Unlocking Tensor Core
// Performance for Machine Learning Interatomic Potentials", section "BF16x9 on
// NVIDIA Blackwell GPUs": use the nine-product emulation only where it is
// predicted to be faster than native FP32, from a cost model of this
// library's own kernels on MI355X.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string.h>

#include "emu_launch.h"
#include "emu_sgemm.h"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceSlot {
    bool ready = false;
    bool supported = false;
    emu::DeviceInfo info{};
};

std::mutex g_dev_mutex;
DeviceSlot g_dev[kMaxDevices];

// Returns true and fills `info` when the current device is a gfx950.
bool current_device(emu::DeviceInfo& info)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    DeviceSlot& s = g_dev[dev];
    if (!s.ready) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        s.supported = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        s.info.num_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
        s.ready = true;
    }
    info = s.info;
    return s.supported;
}

bool valid_op(int op) { return op == EMU_OP_N || op == EMU_OP_T; }

int64_t max1(int64_t v) { return v > 1 ? v : 1; }

// Cost model of one call on MI355X (256 CUs at up to 2.4 GHz): the kernels
// process 128x128 output tiles, one workgroup per CU, so the time is the
// number of tile rounds times the time of one tile.  Rates are fractions of
// the dense MFMA peaks (bf16 2516.6 TFLOP/s, fp32 157.3 TFLOP/s); fixed
// costs cover launch, pipeline fill and the epilogue.
constexpr double kNumCU = 256.0;
constexpr double kBf16PerCU = 2516.6e12 / kNumCU;  // flop/s per CU
constexpr double kF32PerCU = 157.3e12 / kNumCU;
constexpr double kEffX9 = 0.60;                    // sustained fraction, nine-product kernel
constexpr double kEffF32 = 0.75;                   // sustained fraction, native kernel
constexpr double kTileFixedX9 = 1.5e-6;            // s per tile: fill + five-band epilogue
constexpr double kTileFixedF32 = 1.0e-6;
constexpr double kLaunch = 4.0e-6;

double predict_seconds(int64_t M, int64_t N, int64_t K, bool x9)
{
    const double tiles = (double)((M + 127) / 128) * (double)((N + 127) / 128);
    const double rounds = tiles <= kNumCU ? 1.0 : (double)((int64_t)(tiles + kNumCU - 1) / (int64_t)kNumCU);
    const double kpad = (double)((K + 31) / 32 * 32);
    const double tile_flops = 2.0 * 128.0 * 128.0 * kpad;
    const double per_tile = x9 ? kTileFixedX9 + 9.0 * tile_flops / (kBf16PerCU * kEffX9)
                               : kTileFixedF32 + tile_flops / (kF32PerCU * kEffF32);
    return kLaunch + rounds * per_tile;
}

emu_mode_t select_mode(int64_t M, int64_t N, int64_t K)
{
    if (M == 0 || N == 0 || K == 0) return EMU_MODE_NATIVE_F32;
    return predict_seconds(M, N, K, true) < predict_seconds(M, N, K, false) ? EMU_MODE_BF16X9
                                                                             : EMU_MODE_NATIVE_F32;
}

emu_status_t from_hip(hipError_t e)
{
    if (e == hipSuccess) return EMU_STATUS_SUCCESS;
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return EMU_STATUS_ALLOC_FAILED;
    return EMU_STATUS_LAUNCH_FAILED;
}

}  // namespace

extern "C" {

const char* emu_status_string(emu_status_t status)
{
    switch (status) {
    case EMU_STATUS_SUCCESS: return "EMU_STATUS_SUCCESS";
    case EMU_STATUS_INVALID_VALUE: return "EMU_STATUS_INVALID_VALUE";
    case EMU_STATUS_NOT_SUPPORTED: return "EMU_STATUS_NOT_SUPPORTED";
    case EMU_STATUS_LAUNCH_FAILED: return "EMU_STATUS_LAUNCH_FAILED";
    case EMU_STATUS_ALLOC_FAILED: return "EMU_STATUS_ALLOC_FAILED";
    case EMU_STATUS_INTERNAL: return "EMU_STATUS_INTERNAL";
    default: return "EMU_STATUS_UNKNOWN";
    }
}

int emu_abi_version(void) { return 100; }

emu_status_t emu_sgemm_select(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                              emu_mode_t* chosen)
{
    if (!valid_op(transA) || !valid_op(transB) || M < 0 || N < 0 || K < 0 || chosen == nullptr)
        return EMU_STATUS_INVALID_VALUE;
    *chosen = select_mode(M, N, K);
    return EMU_STATUS_SUCCESS;
}

emu_status_t emu_sgemm(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                       float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                       float beta, float* C, int64_t ldc, emu_mode_t mode, void* stream)
{
    // ---- validation: no HIP call before this block has passed ----
    if (!valid_op(transA) || !valid_op(transB)) return EMU_STATUS_INVALID_VALUE;
    if ((int)mode < (int)EMU_MODE_NATIVE_F32 || (int)mode > (int)EMU_MODE_AUTO)
        return EMU_STATUS_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0) return EMU_STATUS_INVALID_VALUE;
    if (lda < (transA == EMU_OP_N ? max1(K) : max1(M))) return EMU_STATUS_INVALID_VALUE;
    if (ldb < (transB == EMU_OP_N ? max1(N) : max1(K))) return EMU_STATUS_INVALID_VALUE;
    if (ldc < max1(N)) return EMU_STATUS_INVALID_VALUE;
    const bool has_c = M > 0 && N > 0;
    if (has_c && C == nullptr) return EMU_STATUS_INVALID_VALUE;
    if (has_c && K > 0 && (A == nullptr || B == nullptr)) return EMU_STATUS_INVALID_VALUE;
    if (!has_c) return EMU_STATUS_SUCCESS;

    emu::DeviceInfo dev;
    if (!current_device(dev)) return EMU_STATUS_NOT_SUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (K == 0 || alpha == 0.0f) return from_hip(emu::launch_scale_c(M, N, beta, C, ldc, s));

    if (mode == EMU_MODE_AUTO) mode = select_mode(M, N, K);
    emu::GemmArgs g;
    g.trans_a = transA == EMU_OP_T;
    g.trans_b = transB == EMU_OP_T;
    g.M = M;
    g.N = N;
    g.K = K;
    g.alpha = alpha;
    g.beta = beta;
    g.A = A;
    g.lda = lda;
    g.B = B;
    g.ldb = ldb;
    g.C = C;
    g.ldc = ldc;
    switch (mode) {
    case EMU_MODE_NATIVE_F32: return from_hip(emu::launch_gemm_native_f32(g, dev, s));
    case EMU_MODE_BF16X9: return from_hip(emu::launch_gemm_bf16(g, 5, dev, s));
    case EMU_MODE_BF16X6: return from_hip(emu::launch_gemm_bf16(g, 3, dev, s));
    case EMU_MODE_BF16X3: return from_hip(emu::launch_gemm_bf16(g, 2, dev, s));
    default: return EMU_STATUS_INTERNAL;
    }
}

emu_status_t emu_split_bf16x3(const float* x, int64_t n, uint16_t* hi, uint16_t* mid,
                              uint16_t* lo, void* stream)
{
    if (n < 0) return EMU_STATUS_INVALID_VALUE;
    if (n > 0 && (x == nullptr || hi == nullptr || mid == nullptr || lo == nullptr))
        return EMU_STATUS_INVALID_VALUE;
    if (n == 0) return EMU_STATUS_SUCCESS;
    emu::DeviceInfo dev;
    if (!current_device(dev)) return EMU_STATUS_NOT_SUPPORTED;
    return from_hip(emu::launch_split(x, n, hi, mid, lo, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
