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

#include <cmath>
#include <mutex>
#include <string.h>

#include "emu_launch.h"
#include "emu_sgemm.h"

namespace {

constexpr int kMaxDevices = 64;

// One stream's workspace on a device (see stream_workspace).
struct WsEntry {
    bool used = false;
    hipStream_t stream = nullptr;
    void* ptr = nullptr;
    size_t size = 0;
    uint64_t last = 0;
};
constexpr int kWsEntries = 16;

struct DeviceSlot {
    bool ready = false;
    bool supported = false;
    emu::DeviceInfo info{};
    WsEntry ws[kWsEntries];
    uint64_t tick = 0;
    bool pool_tried = false;       // the workspace pool is made on first use
    void* scratch = nullptr;       // this device's copy of `scratch` (null: unresolved)
};

std::mutex g_dev_mutex;
DeviceSlot g_dev[kMaxDevices];

// The workspace of emu_sgemm_noalloc: device memory that is part of the
// library's code object, so a call never allocates.  Each device holds its
// own copy, from the library's first use on that device until the process
// ends.  In host code `scratch` is only a stand-in for the symbol: its
// device address, per device, comes from hipGetSymbolAddress when the
// device is first used (current_device) and is what the kernels receive.
// Calls on one device share the copy, so emu_sgemm_noalloc calls that
// overlap on a device race; no kernel needs it zeroed (every byte a kernel
// reads, it or an earlier kernel of the same call wrote).
constexpr size_t kScratchBytes = (size_t)EMU_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// A memory pool on device `dev` that keeps up to kPoolKeepBytes of freed
// memory mapped; null (and no error left behind) if one cannot be made.
hipMemPool_t make_pool(int dev)
{
    hipMemPoolProps pp;
    memset(&pp, 0, sizeof(pp));
    pp.allocType = hipMemAllocationTypePinned;
    pp.handleTypes = hipMemHandleTypeNone;
    pp.location.type = hipMemLocationTypeDevice;
    pp.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &pp) != hipSuccess) {
        (void)hipGetLastError();   // our failure must not surface in a later launch check
        return nullptr;
    }
    uint64_t keep = emu::kPoolKeepBytes;
    if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) {
        (void)hipMemPoolDestroy(pool);
        (void)hipGetLastError();
        return nullptr;
    }
    return pool;
}

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
        s.info.device = dev;
        s.info.pool = nullptr;
        if (s.supported) {
            // this device's copy of the no-allocation scratch (the device is current)
            void* ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr != nullptr) {
                s.scratch = ptr;
            } else {
                s.scratch = nullptr;
                (void)hipGetLastError();   // reported by emu_sgemm_noalloc, not by a later launch
            }
        }
        s.ready = true;
    }
    info = s.info;
    return s.supported;
}

// A device workspace of at least `bytes` for a call on stream `st`.  Each
// stream keeps one grow-only buffer, used only by calls on that stream and
// so only in its order: calls on different streams never share one, and a
// stream's buffer is reused call after call without allocating (a
// stream-ordered allocation and free costs every call several microseconds
// of device time, and more when the sizes vary).  Growing frees the old
// buffer in the stream's order.  With kWsEntries streams in use, the least
// recently used one's buffer is released with hipFree, which waits for the
// device.  The buffers live until the process ends.
hipError_t stream_workspace(const emu::DeviceInfo& info, hipStream_t st, size_t bytes, void** out)
{
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    DeviceSlot& d = g_dev[info.device];
    if (!d.pool_tried) {
        // A pool of our own for the stream workspaces (keeping freed memory
        // mapped up to kPoolKeepBytes); without it the device's default pool
        // is used.
        d.info.pool = make_pool(info.device);
        d.pool_tried = true;
    }
    const hipMemPool_t pool = d.info.pool;
    ++d.tick;
    WsEntry* e = nullptr;
    for (WsEntry& w : d.ws)
        if (w.used && w.stream == st) e = &w;
    if (e == nullptr) {
        for (WsEntry& w : d.ws)
            if (!w.used && e == nullptr) e = &w;
        if (e == nullptr) {
            e = &d.ws[0];
            for (WsEntry& w : d.ws)
                if (w.last < e->last) e = &w;
            if (e->ptr != nullptr && hipFree(e->ptr) != hipSuccess) return hipErrorUnknown;
            *e = WsEntry{};
        }
        e->used = true;
        e->stream = st;
    }
    e->last = d.tick;
    if (e->size < bytes) {
        size_t want = e->size + e->size / 2;
        if (want < bytes) want = bytes;
        want = (want + ((size_t)1 << 20) - 1) & ~(((size_t)1 << 20) - 1);   // whole MiB
        if (e->ptr != nullptr) {
            if (hipFreeAsync(e->ptr, st) != hipSuccess) return hipErrorUnknown;
            e->ptr = nullptr;
            e->size = 0;
        }
        void* p = nullptr;
        const hipError_t r = pool != nullptr ? hipMallocFromPoolAsync(&p, want, pool, st)
                                             : hipMallocAsync(&p, want, st);
        if (r != hipSuccess) {
            (void)hipGetLastError();   // reported as EMU_STATUS_ALLOC_FAILED, not by a later launch
            return hipErrorOutOfMemory;
        }
        e->ptr = p;
        e->size = want;
    }
    *out = e->ptr;
    return hipSuccess;
}

// The device address of `scratch` on device `dev`, resolved by
// current_device() (null if that failed).
void* device_scratch(int dev)
{
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    return g_dev[dev].scratch;
}

bool valid_op(int op) { return op == EMU_OP_N || op == EMU_OP_T; }

int64_t max1(int64_t v) { return v > 1 ? v : 1; }

// Cost model of one call on MI355X: predicted device time in microseconds,
// including the B pre-split (emulated) or pack (native) of each path (their
// workspace comes from the per-stream cache).  Its form follows the kernels:
// 128x128 output tiles, K in steps of 32; both kernels keep one (tile or
// K-segment) item per CU (256 at a time), and a k-step costs more once every
// CU is busy.  The constants are a least-squares fit (log error) to device
// times measured with emulated_fp32_matrix_amd/calibrate.py over 67 shapes:
// the MLIP layer stacks, squares 128..8192, skinny shapes and a K sweep.  On
// those shapes the choice is the faster mode in 65 of 67 cases and within
// 1 % of it in the other two.
constexpr double kX9Fixed = 11.519;      // us: pre-split launch, pipeline fill
constexpr double kX9StepPart = 1.4118;   // us per k-step per round while some CUs are idle
constexpr double kX9StepFull = 1.9740;   // us per k-step per round with every CU busy
constexpr double kF32Fixed = 10.986;     // us: B pack launch, pipeline fill
constexpr double kF32StepPart = 2.0028;
constexpr double kF32StepFull = 2.4815;
constexpr double kCUs = 256.0;
// A split K (S segments of ceil(K/32)/S k-steps each) runs S times as many
// (segment, tile) items with 1/S of the k-steps each, then a reduction
// kernel that reads the S partial results and writes C.  With these two
// constants the split chosen below is the fastest measured one on all 16
// GEMMs of the two 6,144-row stacks.
constexpr double kRedFixed = 4.0;        // us: reduction launch and tail
constexpr double kRedBytesPerUs = 4.0e6; // bytes per us moved by the reduction
constexpr int kMaxSplit = 8;
// The emulated kernel's output tiles have 128 or 64 rows (fused-A path).  A
// k-step of a 64-row tile does half the MFMAs and splits half the A rows of
// a 128-row one but copies the same B chunk: it costs this fraction of it.
constexpr double kX9Step64 = 0.59;

double ceil_div(double a, double b) { return std::ceil(a / b); }

// A launch of the emulated kernel: K segments, rows of an output tile, and
// the first tile whose K is split (0: all of them, when split > 1).  With
// split_from > 0 the tiles before it (whole rounds of 256) run unsplit and
// only the last, partly filled round's tiles are split: the items of that
// round then fill the CUs.
struct Plan {
    int split = 1;
    int tile_m = 128;
    int64_t split_from = 0;
};

double predict_plan_us(int64_t M, int64_t N, int64_t K, const Plan& pl)
{
    const double tiles = ceil_div((double)M, (double)pl.tile_m) * ceil_div((double)N, 128.0);
    const double nk = ceil_div((double)K, 32.0);
    const double f64 = pl.tile_m == 64 ? kX9Step64 : 1.0;
    if (pl.split == 1) {
        const double step = (tiles >= kCUs ? kX9StepFull : kX9StepPart) * f64;
        return kX9Fixed + ceil_div(tiles, kCUs) * nk * step;
    }
    const double whole = (double)pl.split_from;   // tiles of the unsplit rounds
    const double items = (tiles - whole) * pl.split;
    double t = kX9Fixed + whole / kCUs * nk * kX9StepFull * f64;
    t += ceil_div(items, kCUs) * (nk / pl.split) * (items + whole >= kCUs ? kX9StepFull : kX9StepPart) * f64;
    const double elems = pl.split_from == 0 ? (double)M * (double)N : (tiles - whole) * pl.tile_m * 128.0;
    return t + kRedFixed + (double)(pl.split + 1) * elems * 4.0 / kRedBytesPerUs;
}

double predict_x9_us(int64_t M, int64_t N, int64_t K, int split, int tile_m)
{
    Plan pl;
    pl.split = split;
    pl.tile_m = tile_m;
    return predict_plan_us(M, N, K, pl);
}

// The rows of the emulated kernel's output tiles for a call with `split` K
// segments over every tile (fused-A path; the result does not depend on
// it): 64 where the cost model predicts them at least 3 % faster than
// 128-row tiles (too few 128-row tiles to fill the CUs, or a last round of
// tiles mostly idle).
int choose_tile_m(int64_t M, int64_t N, int64_t K, int split)
{
    if (M == 0 || N == 0 || K == 0) return 128;
    return predict_x9_us(M, N, K, split, 64) < 0.97 * predict_x9_us(M, N, K, split, 128) ? 64 : 128;
}

// The plan the emulated path uses by itself (fused-A path), from the cost
// model: for each divisor S <= kMaxSplit of ceil(K/32), every tile split
// (its tile height by the 3 % rule above) and, where the tiles leave a last
// round partly filled, only that round split (for each tile height); the
// fastest of these, and no split (tile height by the same rule) unless that
// saves at least 5 %.
Plan choose_plan(int64_t M, int64_t N, int64_t K)
{
    Plan base;
    if (M == 0 || N == 0 || K == 0) return base;
    base.tile_m = choose_tile_m(M, N, K, 1);
    const double t1 = predict_plan_us(M, N, K, base);
    const int64_t nk = (K + 31) / 32;
    const int64_t tiles_n = (N + 127) / 128;
    Plan best = base;
    double tbest = t1;
    auto consider = [&](const Plan& pl) {
        const double t = predict_plan_us(M, N, K, pl);
        if (t < tbest) {
            tbest = t;
            best = pl;
        }
    };
    for (int sp = 2; sp <= kMaxSplit && sp <= nk; ++sp) {
        if (nk % sp != 0) continue;
        Plan all;
        all.split = sp;
        all.tile_m = choose_tile_m(M, N, K, sp);
        consider(all);
        for (int th : {128, 64}) {
            const int64_t tiles = (M + th - 1) / th * tiles_n;
            const int64_t full = tiles / (int64_t)kCUs * (int64_t)kCUs;
            if (full == 0 || full == tiles) continue;
            Plan tail;
            tail.split = sp;
            tail.tile_m = th;
            tail.split_from = full;
            consider(tail);
        }
    }
    return tbest < 0.95 * t1 ? best : base;
}

void predict_us(int64_t M, int64_t N, int64_t K, double& f32, double& x9)
{
    const double tiles = ceil_div((double)M, 128.0) * ceil_div((double)N, 128.0);
    const double nk = ceil_div((double)K, 32.0);
    x9 = predict_plan_us(M, N, K, choose_plan(M, N, K));
    f32 = kF32Fixed + ceil_div(tiles, kCUs) * nk * (tiles >= kCUs ? kF32StepFull : kF32StepPart);
}

emu_mode_t select_mode(int64_t M, int64_t N, int64_t K)
{
    if (M == 0 || N == 0 || K == 0) return EMU_MODE_NATIVE_F32;
    double f32, x9;
    predict_us(M, N, K, f32, x9);
    return x9 < f32 ? EMU_MODE_BF16X9 : EMU_MODE_NATIVE_F32;
}

bool emulated(emu_mode_t m)
{
    return m == EMU_MODE_BF16X9 || m == EMU_MODE_BF16X6 || m == EMU_MODE_BF16X3 || m == EMU_MODE_BF16X1;
}

emu_status_t from_hip(hipError_t e)
{
    if (e == hipSuccess) return EMU_STATUS_SUCCESS;
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return EMU_STATUS_ALLOC_FAILED;
    return EMU_STATUS_LAUNCH_FAILED;
}

}  // namespace

namespace {

// planes: op(B) pre-split by emu_presplit_b (then B, ldb and transB are not
// used and mode must be an emulated one), or null.
// noalloc: the workspace is this device's scratch (EMU_STATUS_SCRATCH_TOO_SMALL
// when the call needs more), never the stream's allocated buffer.
emu_status_t sgemm_impl(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                        float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                        float beta, float* C, int64_t ldc, const float* bias, emu_mode_t mode,
                        int ksplit, void* stream, const void* planes = nullptr, bool noalloc = false)
{
    // ---- validation: no HIP call before this block has passed ----
    if (!valid_op(transA) || !valid_op(transB)) return EMU_STATUS_INVALID_VALUE;
    if ((int)mode < (int)EMU_MODE_NATIVE_F32 || (int)mode > (int)EMU_MODE_BF16X1)
        return EMU_STATUS_INVALID_VALUE;
    if (ksplit < EMU_KSPLIT_AUTO || (ksplit != 0 && !emulated(mode))) return EMU_STATUS_INVALID_VALUE;
    if (ksplit > 1 && (K == 0 || ((K + 31) / 32) % ksplit != 0)) return EMU_STATUS_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0) return EMU_STATUS_INVALID_VALUE;
    if (lda < (transA == EMU_OP_N ? max1(K) : max1(M))) return EMU_STATUS_INVALID_VALUE;
    if (planes == nullptr && ldb < (transB == EMU_OP_N ? max1(N) : max1(K))) return EMU_STATUS_INVALID_VALUE;
    if (ldc < max1(N)) return EMU_STATUS_INVALID_VALUE;
    const bool has_c = M > 0 && N > 0;
    if (has_c && C == nullptr) return EMU_STATUS_INVALID_VALUE;
    if (has_c && K > 0 && (A == nullptr || (B == nullptr && planes == nullptr)))
        return EMU_STATUS_INVALID_VALUE;
    if (planes != nullptr && ((uintptr_t)planes & 15u) != 0) return EMU_STATUS_INVALID_VALUE;
    if (!has_c) return EMU_STATUS_SUCCESS;

    emu::DeviceInfo dev;
    if (!current_device(dev)) return EMU_STATUS_NOT_SUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* const scratch_ptr = noalloc ? device_scratch(dev.device) : nullptr;
    if (noalloc && scratch_ptr == nullptr) return EMU_STATUS_INTERNAL;
    // the call's workspace: the stream's buffer, or the scratch
    auto workspace = [&](size_t bytes, void** ws) -> emu_status_t {
        if (noalloc) {
            if (bytes > kScratchBytes) return EMU_STATUS_SCRATCH_TOO_SMALL;
            *ws = scratch_ptr;
            return EMU_STATUS_SUCCESS;
        }
        return stream_workspace(dev, s, bytes, ws) == hipSuccess ? EMU_STATUS_SUCCESS
                                                                 : EMU_STATUS_ALLOC_FAILED;
    };

    if (K == 0 || alpha == 0.0f) return from_hip(emu::launch_scale_c(M, N, beta, C, ldc, bias, s));

    const bool auto_mode = mode == EMU_MODE_AUTO;
    if (auto_mode) mode = select_mode(M, N, K);
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
    g.bias = bias;
    g.Bplanes = static_cast<const uint16_t*>(planes);
    if (mode == EMU_MODE_NATIVE_F32) {
        void* ws = nullptr;
        const size_t ws_bytes = emu::gemm_native_f32_workspace_bytes(g);
        if (ws_bytes > 0) {
            const emu_status_t st = workspace(ws_bytes, &ws);
            if (st != EMU_STATUS_SUCCESS) return st;
        }
        return from_hip(emu::launch_gemm_native_f32(g, dev, ws, s));
    }
    const bool fused = emu::fused_a_path(g);
    if (ksplit > 1 && !fused) return EMU_STATUS_NOT_SUPPORTED;
    // ksplit 0: the performant policy (AUTO) may split where its cost model
    // predicts a gain; an explicit mode computes without a split, so a row
    // of C never depends on the other rows.  EMU_KSPLIT_AUTO: the policy's
    // plan in an explicit mode.  S > 1: every tile split.
    Plan plan;
    if (ksplit == EMU_KSPLIT_AUTO || (ksplit == 0 && auto_mode)) {
        if (fused) {
            plan = choose_plan(M, N, K);
            // a split of the last round only needs whole rounds of this
            // device's compute units before it
            const int64_t tiles = (M + plan.tile_m - 1) / plan.tile_m * ((N + 127) / 128);
            const int64_t round = tiles < dev.num_cu ? tiles : dev.num_cu;
            if (plan.split_from % round != 0) plan.split_from = 0;
        } else {
            plan.tile_m = choose_tile_m(M, N, K, 1);
        }
    } else if (ksplit > 1) {
        plan.split = ksplit;
        plan.tile_m = choose_tile_m(M, N, K, ksplit);
    } else {
        plan.tile_m = choose_tile_m(M, N, K, 1);
    }
    int nbands;
    switch (mode) {
    case EMU_MODE_BF16X9: nbands = 5; break;
    case EMU_MODE_BF16X6: nbands = 3; break;
    case EMU_MODE_BF16X3: nbands = 2; break;
    case EMU_MODE_BF16X1: nbands = 1; break;
    default: return EMU_STATUS_INTERNAL;
    }
    void* ws = nullptr;
    const size_t ws_bytes = emu::gemm_bf16_workspace_bytes(g, nbands, plan.split, plan.tile_m, plan.split_from);
    if (ws_bytes > 0) {
        const emu_status_t st = workspace(ws_bytes, &ws);
        if (st != EMU_STATUS_SUCCESS) return st;
    }
    return from_hip(emu::launch_gemm_bf16(g, nbands, plan.split, plan.split_from, plan.tile_m, dev, ws, s));
}

// Bands of an emulated mode (0 for NATIVE_F32 and AUTO).
int mode_bands(emu_mode_t mode)
{
    switch (mode) {
    case EMU_MODE_BF16X9: return 5;
    case EMU_MODE_BF16X6: return 3;
    case EMU_MODE_BF16X3: return 2;
    case EMU_MODE_BF16X1: return 1;
    default: return 0;
    }
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
    case EMU_STATUS_SCRATCH_TOO_SMALL: return "EMU_STATUS_SCRATCH_TOO_SMALL";
    default: return "EMU_STATUS_UNKNOWN";
    }
}

int emu_abi_version(void) { return 107; }

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
    return sgemm_impl(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, nullptr, mode, 0,
                      stream);
}

emu_status_t emu_sgemm_bias(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                            float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                            float beta, float* C, int64_t ldc, const float* bias, emu_mode_t mode,
                            void* stream)
{
    return sgemm_impl(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, mode, 0,
                      stream);
}

emu_status_t emu_sgemm_ex(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                          float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                          float beta, float* C, int64_t ldc, const float* bias, emu_mode_t mode,
                          int ksplit, void* stream)
{
    return sgemm_impl(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, mode,
                      ksplit, stream);
}

emu_status_t emu_presplit_b_bytes(int64_t N, int64_t K, emu_mode_t mode, size_t* bytes)
{
    if (N < 0 || K < 0 || bytes == nullptr || mode_bands(mode) == 0) return EMU_STATUS_INVALID_VALUE;
    *bytes = N == 0 || K == 0 ? 0 : emu::gemm_bf16_planes_bytes(N, K, mode_bands(mode));
    return EMU_STATUS_SUCCESS;
}

emu_status_t emu_presplit_b(emu_op_t transB, int64_t N, int64_t K, const float* B, int64_t ldb,
                            emu_mode_t mode, void* planes, void* stream)
{
    if (!valid_op(transB) || N < 0 || K < 0 || mode_bands(mode) == 0) return EMU_STATUS_INVALID_VALUE;
    if (ldb < (transB == EMU_OP_N ? max1(N) : max1(K))) return EMU_STATUS_INVALID_VALUE;
    if (N == 0 || K == 0) return EMU_STATUS_SUCCESS;
    if (B == nullptr || planes == nullptr || ((uintptr_t)planes & 15u) != 0) return EMU_STATUS_INVALID_VALUE;
    emu::DeviceInfo dev;
    if (!current_device(dev)) return EMU_STATUS_NOT_SUPPORTED;
    return from_hip(emu::launch_presplit_b(B, ldb, transB == EMU_OP_T, N, K, mode_bands(mode),
                                           static_cast<uint16_t*>(planes), static_cast<hipStream_t>(stream)));
}

emu_status_t emu_sgemm_presplit(emu_op_t transA, int64_t M, int64_t N, int64_t K, float alpha,
                                const float* A, int64_t lda, const void* planes, float beta, float* C,
                                int64_t ldc, const float* bias, emu_mode_t mode, int ksplit, void* stream)
{
    if (mode_bands(mode) == 0) return EMU_STATUS_INVALID_VALUE;
    if (M > 0 && N > 0 && K > 0 && planes == nullptr) return EMU_STATUS_INVALID_VALUE;
    // (B and ldb are not read; ldb = max(1, N) passes the op(B) check)
    return sgemm_impl(transA, EMU_OP_N, M, N, K, alpha, A, lda, nullptr, max1(N), beta, C, ldc, bias,
                      mode, ksplit, stream, planes);
}

emu_status_t emu_sgemm_noalloc(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                               float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                               float beta, float* C, int64_t ldc, const float* bias, emu_mode_t mode,
                               int ksplit, void* stream)
{
    return sgemm_impl(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, mode,
                      ksplit, stream, nullptr, true);
}

emu_status_t emu_sgemm_ksplit(int64_t M, int64_t N, int64_t K, int* ksplit)
{
    if (M < 0 || N < 0 || K < 0 || ksplit == nullptr) return EMU_STATUS_INVALID_VALUE;
    *ksplit = choose_plan(M, N, K).split;
    return EMU_STATUS_SUCCESS;
}

emu_status_t emu_sgemm_plan(int64_t M, int64_t N, int64_t K, int* ksplit, int* tile_rows,
                            int64_t* split_from)
{
    if (M < 0 || N < 0 || K < 0 || ksplit == nullptr || tile_rows == nullptr || split_from == nullptr)
        return EMU_STATUS_INVALID_VALUE;
    const Plan pl = choose_plan(M, N, K);
    *ksplit = pl.split;
    *tile_rows = pl.tile_m;
    *split_from = pl.split == 1 ? ((M + pl.tile_m - 1) / pl.tile_m) * ((N + 127) / 128) : pl.split_from;
    return EMU_STATUS_SUCCESS;
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
