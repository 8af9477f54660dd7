/*
 * emu_sgemm -- FP32 GEMM emulated on bf16 MFMA matrix cores (AMD MI355X, gfx950).
 *
 * Method: "Unlocking Tensor Core Performance for Machine Learning Interatomic
 * Potentials" (NVIDIA technical blog), section "How Tensor Core FP32 bridges
 * the hardware gap":
 *   - Figure 1: each FP32 operand is split into three scaled BF16 pieces; the
 *     nine pairwise products run on the matrix unit and are accumulated in
 *     FP32 along five anti-diagonal bands, then recombined with their scales.
 *   - Figure 2 and its equation a*b ~ a_hi*b_hi + a_hi*b_lo + a_lo*b_hi: a
 *     reduced variant keeps only the largest products.
 * Section "BF16x9 on NVIDIA Blackwell GPUs" describes the SGEMM entry point
 * (no model change) and the "performant" / "eager" policies; section "TF32x3
 * on Ampere GPUs" describes the float-in / float-out linear layer whose
 * forward GEMM and input-gradient GEMM dX = dY.W^T both use the emulation.
 *
 * Conventions (all entry points)
 *   - Row-major storage.  op(A) is M x K, op(B) is K x N, C is M x N.
 *       transA == EMU_OP_N: A stored M x K, lda >= max(1, K)
 *       transA == EMU_OP_T: A stored K x M, lda >= max(1, M)
 *       transB == EMU_OP_N: B stored K x N, ldb >= max(1, N)
 *       transB == EMU_OP_T: B stored N x K, ldb >= max(1, K)
 *       C stored M x N, ldc >= max(1, N)
 *     A column-major caller computes C^T = B^T A^T by swapping operands.
 *   - Every array pointer is device memory owned by the caller.  The library
 *     keeps no reference to it after the call returns.
 *   - Memory: the BF16X* modes need a device workspace for the BF16 planes
 *     of op(B), pre-split once per call (plus those of op(A) when A cannot
 *     be split inside the GEMM: transA == T, A not 16-byte aligned, or lda
 *     or K not a multiple of 4, and the partial results of a split K).  Size
 *     for B: planes * 2 bytes * ceil(N/128)*128 * ceil(K/32)*32 (3 planes,
 *     2 in BF16X3, 1 in BF16X1),
 *     likewise with M for A; S * T * R * 128 * 4 bytes for a split into S
 *     segments of T output tiles of R rows (every tile: T * R * 128 is
 *     about M * N; emu_sgemm_plan gives T and R of the automatic plan).  NATIVE_F32 needs one for op(B) packed as FP32, 4 bytes *
 *     ceil(N/128)*128 * ceil(K/32)*32, when A is k-contiguous and 16-byte
 *     addressable (transA == N, A 16-byte aligned, lda and K multiples of
 *     4), and none otherwise.  The library keeps one workspace per (device, stream): a
 *     buffer that grows to the largest size a call on that stream has needed
 *     and is used only by calls on that stream, so in its order.  It is
 *     allocated on the stream from a memory pool the library creates once
 *     per device (hipMallocFromPoolAsync; the device's default pool if
 *     creating one fails); growing frees the old buffer with hipFreeAsync on
 *     the stream.  Up to 16 streams per device keep a buffer; beyond that the
 *     least recently used one is released with hipFree, which waits for the
 *     device.  The buffers live until the process ends.  A call whose stream
 *     already holds a buffer as large as the call needs allocates nothing
 *     and issues only kernel launches, so it can be captured in a HIP graph
 *     on that stream: run the same calls on the stream once before the
 *     capture (emu_sgemm_noalloc needs no such run).  emu_split_bf16x3
 *     allocates nothing, and emu_sgemm_noalloc works in a fixed scratch
 *     instead of a stream's buffer.  The cache knows streams only by their handle:
 *     synchronise a stream that ran library calls before destroying it, so
 *     that a new stream that receives the same handle cannot overlap its
 *     work with the old stream's in the shared buffer.
 *   - stream is a hipStream_t (NULL = the null stream).  Work is enqueued on
 *     it asynchronously; errors during execution surface at the caller's
 *     next synchronisation of that stream.
 *   - Argument validation is synchronous and happens before any HIP call, so
 *     an EMU_STATUS_INVALID_VALUE return has touched neither device nor stream.
 *   - Re-entrant and thread-safe; calls on different streams may overlap.
 */
#ifndef EMU_SGEMM_H
#define EMU_SGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { EMU_OP_N = 0, EMU_OP_T = 1 } emu_op_t;

typedef enum {
    /* FP32 MFMA (v_mfma_f32_32x32x2_f32): the native baseline. */
    EMU_MODE_NATIVE_F32 = 0,
    /* Nine products, five FP32 band accumulators (Figure 1). */
    EMU_MODE_BF16X9 = 1,
    /* Six products: bands 0..2 (piece-index sum u + v <= 2). */
    EMU_MODE_BF16X6 = 2,
    /* Three products hi*hi, hi*mid, mid*hi: bands 0..1 (Figure 2's rule). */
    EMU_MODE_BF16X3 = 3,
    /* Per-shape choice between NATIVE_F32 and BF16X9, the "performant"
     * policy of section "BF16x9 on NVIDIA Blackwell GPUs". */
    EMU_MODE_AUTO = 4,
    /* One product hi*hi: band 0 only, operands rounded once to BF16, the
     * analog of the single-pass TF32 mode that section "TF32x3 on Ampere
     * GPUs" compares TF32x3 against.  Not FP32-accurate (about 2^-8
     * relative per product); never chosen by AUTO.  (ABI 1.2) */
    EMU_MODE_BF16X1 = 5
} emu_mode_t;

typedef enum {
    EMU_STATUS_SUCCESS = 0,
    EMU_STATUS_INVALID_VALUE = 1,  /* bad dimension, leading dimension, pointer or enum */
    EMU_STATUS_NOT_SUPPORTED = 2,  /* no gfx950 device current, or device query failed */
    EMU_STATUS_LAUNCH_FAILED = 3,  /* the kernel launch itself reported an error */
    EMU_STATUS_ALLOC_FAILED = 4,   /* the stream's workspace could not be allocated or grown */
    EMU_STATUS_INTERNAL = 5,
    /* emu_sgemm_noalloc: the call needs more workspace than the library's
     * fixed scratch holds (EMU_NOALLOC_SCRATCH_BYTES); nothing was launched.
     * (ABI 1.6) */
    EMU_STATUS_SCRATCH_TOO_SMALL = 6
} emu_status_t;

/* Bytes of the fixed per-device scratch emu_sgemm_noalloc works in. */
#define EMU_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* ksplit of emu_sgemm_ex, emu_sgemm_noalloc and emu_sgemm_presplit: the
 * plan EMU_MODE_AUTO uses for the shape (emu_sgemm_plan), in the explicit
 * emulated mode given.  (ABI 1.7) */
#define EMU_KSPLIT_AUTO (-1)

/*
 * C = alpha * op(A) . op(B) + beta * C in FP32, computed in `mode`.
 *
 * BF16X9/X6/X3 (and BF16X1): each element of op(A) and op(B) is split exactly into
 * (hi, mid', lo') with hi = R(a), mid' = R(2^8 (a - hi)), lo' = 2^8 (2^8 (a -
 * hi) - mid'), R = round to nearest even, saturating at the largest finite
 * BF16 (Figure 1's "three scaled BF16 components").  Products with piece
 * indices u + v = j are accumulated in FP32 band j; the bands kept (5, 3, 2
 * or 1) are recombined smallest first, t = S_{n-1}, t = S_j + 2^-8 t, and then
 * C = alpha * t + beta * C.  In EMU_MODE_AUTO the library chooses, per shape,
 * the mode (emu_sgemm_select) and, for an emulated mode, possibly a split of
 * K into segments on some or all output tiles (emu_sgemm_plan, emu_sgemm_ex):
 * there t is the sum, in segment order, of the segments' t.  So in AUTO a row of C may differ in its
 * last bits between shapes; in an explicit mode it never depends on the
 * other rows.  Every result is deterministic for a given shape.
 *
 * Semantics follow BLAS SGEMM:
 *   - M == 0 or N == 0: nothing is done.
 *   - K == 0 or alpha == 0: C = beta * C (C is zeroed, not read, if beta == 0).
 *   - beta == 0: C is written without being read (NaNs in C do not propagate).
 * A or B overlapping C is undefined behaviour (not checked).  Any alignment
 * and any leading dimension meeting the bounds above is accepted; 16-byte
 * aligned pointers with leading dimensions that are multiples of 4 take the
 * vectorised load path.  Non-finite inputs give non-finite outputs in every
 * mode (a NaN may appear where IEEE gives +-inf).  Finite inputs up to
 * FLT_MAX split into finite pieces in every mode (R saturates).
 *
 * Errors: EMU_STATUS_INVALID_VALUE for M, N or K < 0, a leading dimension
 * below its bound, a NULL A or B with M*N*K > 0, a NULL C with M*N > 0, or a
 * transA/transB/mode outside its enum.  EMU_STATUS_NOT_SUPPORTED if the
 * current device is not gfx950.  EMU_STATUS_ALLOC_FAILED if the stream's
 * workspace cannot be allocated or grown (nothing was launched).
 * EMU_STATUS_LAUNCH_FAILED
 * if a launch reports an error.
 */
emu_status_t emu_sgemm(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                       float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                       float beta, float* C, int64_t ldc, emu_mode_t mode, void* stream);

/*
 * emu_sgemm with a bias fused into the epilogue, for the linear layer of
 * "Unlocking Tensor Core Performance for Machine Learning Interatomic
 * Potentials", section "TF32x3 on Ampere GPUs" (a float-in / float-out
 * layer that behaves like a standard linear layer, y = x W^T + b):
 *
 *   C[i][j] = alpha * (op(A) . op(B))[i][j] + beta * C[i][j] + bias[j]
 *
 * in FP32, the bias added last, after alpha and beta.  bias: N floats of
 * device memory, any alignment (16-byte aligned takes the vectorised path),
 * owned by the caller; NULL means no bias (then identical to emu_sgemm).  With
 * K == 0 or alpha == 0: C = beta * C + bias.  Everything else (modes,
 * layout, workspace, errors, asynchrony) is as for emu_sgemm.
 */
emu_status_t emu_sgemm_bias(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                            float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                            float beta, float* C, int64_t ldc, const float* bias, emu_mode_t mode,
                            void* stream);

/*
 * emu_sgemm_bias with an explicit split of K for the emulated modes.
 *
 * Small GEMMs, like those of the 192-atom system of "Unlocking Tensor Core
 * Performance for Machine Learning Interatomic Potentials", section "BF16x9
 * on NVIDIA Blackwell GPUs" (Figures 3 and 4: the smallest GEMM and MD-step
 * speedups), have fewer 128 x 128 output tiles than the device has compute
 * units, and others leave the last round of tiles over the compute units
 * partly filled.  Splitting K runs several K segments of a tile at once.
 * The split is this library's, not the pages'.
 *
 *   ksplit = 0:  as emu_sgemm_bias: with EMU_MODE_AUTO the performant policy
 *                splits where its cost model predicts a gain (the plan
 *                emu_sgemm_plan reports); an explicit mode does not split;
 *   ksplit = EMU_KSPLIT_AUTO (-1): that policy's plan in an explicit
 *                emulated mode (no split where A does not allow one, see
 *                below): the result equals EMU_MODE_AUTO's bit for bit when
 *                AUTO runs that mode;
 *   ksplit >= 1: exactly that many segments on every output tile; it must
 *                divide n = ceil(K / 32) and needs an explicit emulated mode
 *                (BF16X9, X6, X3, X1).
 *
 * With S segments, segment s covers the k-steps [s n / S, (s + 1) n / S) of
 * 32 k each.  On a split tile each segment's product t_s is formed as
 * without a split (band accumulation, recombination), and then
 *     C = alpha (t_0 + t_1 + ... + t_{S-1}) + beta C + bias,
 * summed in segment order, every operation one FP32 rounding; elements of a
 * tile that is not split are those of the call without a split.  The result
 * is a deterministic function of (inputs, ksplit) (and, for the automatic
 * plan, the shape): it does not depend on timing.  The split adds S floats
 * per element of the split tiles to the workspace.
 *
 * Errors: as emu_sgemm_bias; EMU_STATUS_INVALID_VALUE for ksplit < -1, for
 * ksplit != 0 with EMU_MODE_NATIVE_F32 or EMU_MODE_AUTO, or for ksplit > 1
 * that does not divide ceil(K / 32) (or K = 0); EMU_STATUS_NOT_SUPPORTED for
 * ksplit > 1 when op(A) is transposed or A is not 16-byte addressable (A
 * 16-byte aligned, lda and K multiples of 4): that path splits A into BF16
 * pieces ahead of the GEMM and does not split K.
 */
emu_status_t emu_sgemm_ex(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                          float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                          float beta, float* C, int64_t ldc, const float* bias, emu_mode_t mode,
                          int ksplit, void* stream);

/*
 * emu_sgemm_ex that never allocates, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Arguments, modes, results (bit for bit), asynchrony
 * and errors are those of emu_sgemm_ex.  The only difference is the
 * workspace (the BF16 planes of op(B), of op(A) when A is not split inside
 * the GEMM, the partial results of a split K, or NATIVE_F32's packed
 * op(B); sizes in the Memory paragraph at the top of this file): instead of
 * the stream's allocated buffer, the call uses a scratch of
 * EMU_NOALLOC_SCRATCH_BYTES (64 MiB) that is part of the library's device
 * code object.  Each device holds its own copy from the library's first use
 * on that device (its address is resolved then, once per device) until the
 * process ends.  A call allocates nothing: no hipMalloc, no hipFree, no
 * memory pool, no library routine that allocates.
 *
 * Every call on a device shares that device's scratch, and the scratch
 * keeps the last call's contents (no call needs it cleared).  Calls that
 * overlap on one device race: issue them on one stream, or order them.
 * A graph that captures calls on several streams must order those calls.
 *
 * Errors: as emu_sgemm_ex; also EMU_STATUS_SCRATCH_TOO_SMALL, before any
 * launch, when the call needs more than EMU_NOALLOC_SCRATCH_BYTES (for
 * example a split K of about S * M * N * 4 bytes beyond it), and
 * EMU_STATUS_INTERNAL if the scratch's address could not be resolved.
 * (ABI 1.6)
 */
emu_status_t emu_sgemm_noalloc(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N, int64_t K,
                               float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                               float beta, float* C, int64_t ldc, const float* bias, emu_mode_t mode,
                               int ksplit, void* stream);

/*
 * The plan of the emulated kernel EMU_MODE_AUTO uses for this shape when it
 * runs the emulation and A allows a split (see emu_sgemm_ex); a caller of
 * an explicit emulated mode gets it with ksplit = EMU_KSPLIT_AUTO.  Output
 * tiles are tile_rows x 128 (tile_rows 128 or 64), numbered row by row,
 * columns fastest: tile i covers rows (i / ceil(N/128)) * tile_rows and
 * columns (i % ceil(N/128)) * 128 onwards.  The tiles from split_from on
 * have their K split into ksplit segments (emu_sgemm_ex); ksplit == 1 (no
 * split) reports split_from = the tile count, and split_from == 0 means
 * every tile.  A split of only some tiles takes whole rounds of 256 tiles
 * (one per compute unit) unsplit and splits the last, partly filled round.
 * The plan is the fastest under the library's cost model of: no split; for
 * each divisor S <= 8 of ceil(K / 32), every tile split; and the last round
 * split; and no split unless a split saves at least 5 %.  On a device
 * with another number of compute units than 256, a plan that splits the
 * last round only runs as a split of every tile (the same S).  A pure host
 * function of (M, N, K): deterministic, no device access.  (ABI 1.7)
 * Errors: EMU_STATUS_INVALID_VALUE for negative dimensions or a NULL pointer.
 */
emu_status_t emu_sgemm_plan(int64_t M, int64_t N, int64_t K, int* ksplit, int* tile_rows,
                            int64_t* split_from);

/*
 * The ksplit of emu_sgemm_plan alone.
 * Errors: EMU_STATUS_INVALID_VALUE for negative dimensions or a NULL ksplit.
 */
emu_status_t emu_sgemm_ksplit(int64_t M, int64_t N, int64_t K, int* ksplit);

/*
 * Weights split once, used by many GEMMs.  Every emulated call splits op(B)
 * into BF16 planes before its GEMM (the split of "Unlocking Tensor Core
 * Performance for Machine Learning Interatomic Potentials", section "How
 * Tensor Core FP32 bridges the hardware gap", Figure 1).  When op(B) is a
 * layer's weight matrix that does not change between calls, as in inference
 * or molecular dynamics with a fixed model, the caller can split it once
 * with emu_presplit_b and pass the planes to emu_sgemm_presplit, which then
 * skips that step (a separate launch: a sizeable part of a small GEMM's
 * time).  The result equals emu_sgemm_ex's with the same op(B), mode and
 * ksplit, bit for bit.
 *
 * emu_presplit_b_bytes: device bytes the planes of a K x N op(B) take in
 * `mode` (EMU_MODE_BF16X9, X6, X3 or X1; the planes depend on the mode: 3
 * planes for X9 and X6, 2 for X3, 1 for X1); 0 when N or K is 0.
 * Errors: EMU_STATUS_INVALID_VALUE for negative dimensions, a NULL `bytes`
 * or a mode other than those four.
 */
emu_status_t emu_presplit_b_bytes(int64_t N, int64_t K, emu_mode_t mode, size_t* bytes);

/*
 * emu_presplit_b: write the planes of op(B) (K x N; B stored as for
 * emu_sgemm with transB and ldb) to `planes`: caller-owned device memory of
 * at least emu_presplit_b_bytes(N, K, mode) bytes, 16-byte aligned.  The
 * layout is the library's own (opaque; it may change with the ABI version).
 * Asynchronous on `stream`; `planes` is ready for calls ordered after it.
 * Errors: EMU_STATUS_INVALID_VALUE for a bad enum, a mode other than the
 * four emulated ones, negative dimensions, ldb too small, or (N, K > 0) a
 * NULL B or planes or planes not 16-byte aligned; NOT_SUPPORTED /
 * LAUNCH_FAILED as for emu_sgemm.
 */
emu_status_t emu_presplit_b(emu_op_t transB, int64_t N, int64_t K, const float* B, int64_t ldb,
                            emu_mode_t mode, void* planes, void* stream);

/*
 * emu_sgemm_presplit: as emu_sgemm_ex, with op(B) given by planes that
 * emu_presplit_b wrote for the same N, K and mode (a mismatch is not
 * detected: the caller keeps them together).  `mode` must be one of the
 * four emulated modes; ksplit 0 or 1 is no split, S > 1 and
 * EMU_KSPLIT_AUTO (the plan EMU_MODE_AUTO would use) as in emu_sgemm_ex.
 * Errors: as emu_sgemm_ex (without the op(B) checks); also
 * EMU_STATUS_INVALID_VALUE for NATIVE_F32 or AUTO, or (M, N, K > 0) NULL or
 * non-16-byte-aligned planes.
 */
emu_status_t emu_sgemm_presplit(emu_op_t transA, int64_t M, int64_t N, int64_t K, float alpha,
                                const float* A, int64_t lda, const void* planes, float beta, float* C,
                                int64_t ldc, const float* bias, emu_mode_t mode, int ksplit,
                                void* stream);

/*
 * The exact three-piece split on its own (Figure 1): for i < n,
 *   hi[i], mid[i], lo[i] = BF16 bit patterns of hi, mid', lo' of x[i]
 * with x[i] == hi + 2^-8 mid' + 2^-16 lo' exactly for every finite x[i].
 * Non-finite x[i]: hi = +-inf (0x7F80 | sign) or the quiet NaN
 * 0x7FC0 | sign, and mid' = lo' = +0.
 * x: n floats; hi, mid, lo: n uint16 each; all device memory, any alignment.
 * Errors: EMU_STATUS_INVALID_VALUE if n < 0 or a pointer is NULL with n > 0;
 * EMU_STATUS_NOT_SUPPORTED / EMU_STATUS_LAUNCH_FAILED as for emu_sgemm.
 */
emu_status_t emu_split_bf16x3(const float* x, int64_t n, uint16_t* hi, uint16_t* mid,
                              uint16_t* lo, void* stream);

/*
 * The mode EMU_MODE_AUTO runs for this shape: EMU_MODE_BF16X9 where the
 * library's cost model predicts it faster than EMU_MODE_NATIVE_F32, else
 * EMU_MODE_NATIVE_F32 (the "performant" policy; a caller who wants the
 * "eager" policy passes EMU_MODE_BF16X9 directly).  A pure host function of
 * (transA, transB, M, N, K): deterministic, no device access.
 * Errors: EMU_STATUS_INVALID_VALUE for negative dimensions, a bad enum or a
 * NULL `chosen`.
 */
emu_status_t emu_sgemm_select(emu_op_t transA, emu_op_t transB, int64_t M, int64_t N,
                              int64_t K, emu_mode_t* chosen);

/* Static, NUL-terminated name of a status code ("EMU_STATUS_..."); unknown
 * codes give "EMU_STATUS_UNKNOWN".  Never NULL. */
const char* emu_status_string(emu_status_t status);

/* ABI version of this header (major * 100 + minor): 107 (1.1 added
 * emu_sgemm_bias, 1.2 EMU_MODE_BF16X1, 1.3 emu_sgemm_ex and
 * emu_sgemm_ksplit, 1.4 emu_presplit_b_bytes, emu_presplit_b and
 * emu_sgemm_presplit, 1.5 a stream workspace for NATIVE_F32, which may
 * therefore return EMU_STATUS_ALLOC_FAILED, 1.6 emu_sgemm_noalloc and
 * EMU_STATUS_SCRATCH_TOO_SMALL, 1.7 emu_sgemm_plan, EMU_KSPLIT_AUTO and
 * AUTO plans that split the K of the last round of tiles only). */
int emu_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EMU_SGEMM_H */
