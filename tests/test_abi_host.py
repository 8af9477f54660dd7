"""Host-side checks of the C-ABI library (no GPU needed, no compute calls).

The shared library must load, export every function declared in
include/emu_sgemm.h, and reject invalid arguments with
EMU_STATUS_INVALID_VALUE before making any HIP call.
"""
import os
import re
import subprocess

import pytest

import emulated_fp32_matrix_amd as emu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "emu_sgemm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(emu_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert _declared_functions() == sorted(emu.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", emu.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (emu_[a-z0-9_]+)$", out, flags=re.M))
    missing = set(_declared_functions()) - exported
    assert not missing, missing


def test_header_compiles_as_c():
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                   check=True)


def test_status_strings_and_version():
    assert emu.emu_status_string(0) == "EMU_STATUS_SUCCESS"
    assert emu.emu_status_string(1) == "EMU_STATUS_INVALID_VALUE"
    assert emu.emu_status_string(2) == "EMU_STATUS_NOT_SUPPORTED"
    assert emu.emu_status_string(3) == "EMU_STATUS_LAUNCH_FAILED"
    assert emu.emu_status_string(4) == "EMU_STATUS_ALLOC_FAILED"
    assert emu.emu_status_string(5) == "EMU_STATUS_INTERNAL"
    assert emu.emu_status_string(6) == "EMU_STATUS_SCRATCH_TOO_SMALL"
    assert emu.emu_status_string(99) == "EMU_STATUS_UNKNOWN"
    assert emu.emu_abi_version() == 107


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define EMU_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == emu.NOALLOC_SCRATCH_BYTES


FAKE = 0x1000  # never dereferenced: validation fails (or returns) before any HIP call


@pytest.mark.parametrize("args", [
    dict(transA=2),
    dict(transB=-1),
    dict(mode=6),
    dict(mode=-1),
    dict(M=-1),
    dict(N=-3),
    dict(K=-1),
    dict(lda=7),            # NN: lda >= K = 8
    dict(transA=1, lda=9),  # TN: lda >= M = 10
    dict(ldb=5),            # NN: ldb >= N = 6
    dict(transB=1, ldb=7),  # NT: ldb >= K = 8
    dict(ldc=5),            # ldc >= N = 6
    dict(A=0),
    dict(B=0),
    dict(C=0),
    dict(M=0, ldc=0),       # ld bounds hold for empty shapes too (ldc >= 1)
])
def test_invalid_arguments_rejected(args):
    call = dict(transA=0, transB=0, M=10, N=6, K=8, alpha=1.0, A=FAKE, lda=8, B=FAKE, ldb=6,
                beta=0.0, C=FAKE, ldc=6, mode=1, stream=0)
    if args.get("transA") == 1 and "lda" not in args:
        call["lda"] = 10
    if args.get("transB") == 1 and "ldb" not in args:
        call["ldb"] = 8
    call.update(args)
    assert emu.emu_sgemm(**call) == emu.STATUS_INVALID_VALUE


@pytest.mark.parametrize("args", [
    dict(transA=2), dict(mode=7), dict(M=-1), dict(K=-1), dict(lda=7), dict(ldb=5), dict(ldc=5),
    dict(A=0), dict(B=0), dict(C=0),
])
def test_bias_entry_point_invalid_arguments_rejected(args):
    call = dict(transA=0, transB=0, M=10, N=6, K=8, alpha=1.0, A=FAKE, lda=8, B=FAKE, ldb=6,
                beta=0.0, C=FAKE, ldc=6, bias=FAKE, mode=1, stream=0)
    call.update(args)
    assert emu.emu_sgemm_bias(**call) == emu.STATUS_INVALID_VALUE


@pytest.mark.parametrize("args", [
    dict(ksplit=-2),
    dict(ksplit=2, mode=0),     # a split needs an emulated mode: not NATIVE_F32
    dict(ksplit=2, mode=4),     # nor AUTO
    dict(ksplit=-1, mode=0),    # EMU_KSPLIT_AUTO too
    dict(ksplit=-1, mode=4),
    dict(ksplit=1, mode=0),
    dict(ksplit=3),             # K = 64: 2 k-steps, 3 does not divide them
    dict(ksplit=4),
    dict(ksplit=2, K=0, lda=1, ldb=6),   # nothing to split
    dict(transA=2), dict(mode=6), dict(M=-1), dict(lda=7), dict(C=0),
])
@pytest.mark.parametrize("fn", ["emu_sgemm_ex", "emu_sgemm_noalloc"])
def test_split_entry_point_invalid_arguments_rejected(args, fn):
    call = dict(transA=0, transB=0, M=10, N=6, K=64, alpha=1.0, A=FAKE, lda=64, B=FAKE, ldb=6,
                beta=0.0, C=FAKE, ldc=6, bias=0, mode=1, ksplit=2, stream=0)
    call.update(args)
    assert getattr(emu, fn)(**call) == emu.STATUS_INVALID_VALUE


def test_presplit_sizes():
    """Planes of a K x N op(B): ceil(N/128) tiles x ceil(K/32) k-steps x
    planes x 128 x 32 BF16 values; 0 when N or K is 0."""
    for mode, planes in (("BF16X9", 3), ("BF16X6", 3), ("BF16X3", 2), ("BF16X1", 1)):
        st, n = emu.emu_presplit_b_bytes(256, 256, mode)
        assert st == emu.STATUS_SUCCESS and n == 2 * 8 * planes * 128 * 32 * 2, (mode, n)
        st, n = emu.emu_presplit_b_bytes(129, 33, mode)   # ragged: 2 tiles, 2 k-steps
        assert st == emu.STATUS_SUCCESS and n == 2 * 2 * planes * 128 * 32 * 2, (mode, n)
        assert emu.emu_presplit_b_bytes(0, 64, mode) == (emu.STATUS_SUCCESS, 0)
        assert emu.emu_presplit_b_bytes(64, 0, mode) == (emu.STATUS_SUCCESS, 0)


@pytest.mark.parametrize("N,K,mode", [(-1, 4, "BF16X9"), (4, -1, "BF16X9"), (4, 4, "NATIVE_F32"),
                                      (4, 4, "AUTO")])
def test_presplit_bytes_invalid(N, K, mode):
    assert emu.emu_presplit_b_bytes(N, K, mode)[0] == emu.STATUS_INVALID_VALUE


def test_presplit_bytes_null_output():
    assert emu._lib.emu_presplit_b_bytes(4, 4, 1, None) == emu.STATUS_INVALID_VALUE


@pytest.mark.parametrize("args", [
    dict(transB=2), dict(mode="NATIVE_F32"), dict(mode="AUTO"), dict(N=-1), dict(K=-2),
    dict(ldb=5),                    # NN: ldb >= N = 6
    dict(transB=1, ldb=63),         # NT: ldb >= K = 64
    dict(B=0), dict(planes=0), dict(planes=FAKE + 4),   # planes must be 16-byte aligned
])
def test_presplit_invalid_arguments_rejected(args):
    call = dict(transB=0, N=6, K=64, B=FAKE, ldb=6, mode="BF16X9", planes=FAKE, stream=0)
    call.update(args)
    assert emu.emu_presplit_b(**call) == emu.STATUS_INVALID_VALUE


@pytest.mark.parametrize("args", [
    dict(mode="NATIVE_F32"), dict(mode="AUTO"), dict(planes=0), dict(planes=FAKE + 8),
    dict(transA=2), dict(M=-1), dict(lda=63), dict(C=0), dict(A=0), dict(ldc=5),
    dict(ksplit=-2), dict(ksplit=3),   # K = 64: 2 k-steps, 3 does not divide them
])
def test_sgemm_presplit_invalid_arguments_rejected(args):
    call = dict(transA=0, M=10, N=6, K=64, alpha=1.0, A=FAKE, lda=64, planes=FAKE, beta=0.0, C=FAKE,
                ldc=6, bias=0, mode="BF16X9", ksplit=0, stream=0)
    call.update(args)
    assert emu.emu_sgemm_presplit(**call) == emu.STATUS_INVALID_VALUE


def test_presplit_empty_shapes_return_before_touching_the_device():
    assert emu.emu_presplit_b(0, 0, 64, 0, 1, "BF16X9", 0, 0) == emu.STATUS_SUCCESS
    assert emu.emu_presplit_b(0, 6, 0, 0, 6, "BF16X9", 0, 0) == emu.STATUS_SUCCESS
    assert emu.emu_sgemm_presplit(0, 0, 6, 64, 1.0, 0, 64, 0, 0.0, 0, 6, 0, "BF16X9", 0, 0) == \
        emu.STATUS_SUCCESS


def test_ksplit_choice_is_pure_and_follows_the_cost_model():
    """emu_sgemm_ksplit: no device access; 1 for outputs with many tiles;
    a divisor of the k-steps, at most 8, for few tiles and a long K."""
    assert emu.emu_sgemm_ksplit(-1, 4, 4)[0] == emu.STATUS_INVALID_VALUE
    for M, N, K in [(552960, 768, 256), (552960, 256, 768), (4096, 4096, 4096), (0, 5, 5),
                    (5, 5, 0)]:
        assert emu.select_ksplit(M, N, K) == 1, (M, N, K)
    for M, N, K in [(512, 256, 4096), (2048, 256, 4096), (1024, 512, 8192)]:
        S = emu.select_ksplit(M, N, K)
        nk = -(-K // 32)
        assert 1 < S <= 8 and nk % S == 0, (M, N, K, S)
        assert all(emu.select_ksplit(M, N, K) == S for _ in range(3))


def _plan_ok(M, N, K, plan):
    S, th, sf = plan
    tiles = -(-M // th) * -(-N // 128)
    nk = -(-K // 32)
    assert th in (64, 128) and 1 <= S <= 8, plan
    if S == 1:
        assert sf == tiles, plan
    else:
        assert nk % S == 0, plan
        assert sf == 0 or (0 < sf < tiles and sf % 256 == 0), plan


def test_plan_is_pure_and_consistent():
    """emu_sgemm_plan: no device access, deterministic, its ksplit that of
    emu_sgemm_ksplit; split_from is the tile count without a split, else 0
    or whole rounds of 256 tiles below the tile count."""
    assert emu.emu_sgemm_plan(-1, 4, 4)[0] == emu.STATUS_INVALID_VALUE
    assert emu._lib.emu_sgemm_plan(4, 4, 4, None, None, None) == emu.STATUS_INVALID_VALUE
    assert emu.select_plan(0, 5, 5)[0] == 1
    shapes = [(552960, 768, 256), (552960, 256, 768), (6144, 768, 256), (6144, 256, 768),
              (6144, 3072, 1024), (6144, 1024, 1024), (6144, 1024, 4096), (6144, 4096, 1024),
              (2048, 2048, 2048), (256, 256, 256), (512, 256, 4096), (333, 777, 1000),
              (4096, 4096, 4096), (1, 1, 1)]
    for M, N, K in shapes:
        plan = emu.select_plan(M, N, K)
        _plan_ok(M, N, K, plan)
        assert plan[0] == emu.select_ksplit(M, N, K)
        assert all(emu.select_plan(M, N, K) == plan for _ in range(3))


def test_plan_splits_the_last_round_of_tiles():
    """At 6,144 rows and d = 1024 the 128 x 128 tiles fill whole rounds of
    256 and leave part of one: the plan splits that round only."""
    for M, N, K in [(6144, 1024, 1024), (6144, 3072, 1024), (6144, 1024, 3072)]:
        S, th, sf = emu.select_plan(M, N, K)
        tiles = -(-M // th) * -(-N // 128)
        assert S > 1 and 0 < sf < tiles and sf % 256 == 0, (M, N, K, S, th, sf)


def test_empty_shapes_return_before_touching_the_device():
    base = dict(transA=0, transB=0, alpha=1.0, A=0, B=0, beta=0.0, C=0, mode=1, stream=0)
    assert emu.emu_sgemm(M=0, N=5, K=4, lda=4, ldb=5, ldc=5, **base) == emu.STATUS_SUCCESS
    assert emu.emu_sgemm(M=5, N=0, K=4, lda=4, ldb=1, ldc=1, **base) == emu.STATUS_SUCCESS
    assert emu.emu_sgemm_bias(M=0, N=5, K=4, lda=4, ldb=5, ldc=5, bias=0, **base) == \
        emu.STATUS_SUCCESS
    assert emu.emu_sgemm_noalloc(M=0, N=5, K=4, lda=4, ldb=5, ldc=5, bias=0, ksplit=0, **base) == \
        emu.STATUS_SUCCESS
    assert emu.emu_split_bf16x3(0, 0, 0, 0, 0, 0) == emu.STATUS_SUCCESS


def test_split_invalid_arguments():
    assert emu.emu_split_bf16x3(FAKE, -1, FAKE, FAKE, FAKE, 0) == emu.STATUS_INVALID_VALUE
    for k in range(4):
        ptrs = [FAKE] * 4
        ptrs[k] = 0
        assert emu.emu_split_bf16x3(ptrs[0], 16, ptrs[1], ptrs[2], ptrs[3], 0) == \
            emu.STATUS_INVALID_VALUE


def test_select_is_pure_and_deterministic():
    st, _ = emu.emu_sgemm_select(0, 0, -1, 4, 4)
    assert st == emu.STATUS_INVALID_VALUE
    st, _ = emu.emu_sgemm_select(3, 0, 4, 4, 4)
    assert st == emu.STATUS_INVALID_VALUE
    shapes = [(552960, 768, 256), (6144, 256, 256), (64, 64, 8), (6144, 4096, 1024), (1, 1, 1),
              (0, 5, 5)]
    for M, N, K in shapes:
        for ta in (0, 1):
            for tb in (0, 1):
                st, first = emu.emu_sgemm_select(ta, tb, M, N, K)
                assert st == emu.STATUS_SUCCESS and first in ("BF16X9", "NATIVE_F32")
                assert all(emu.emu_sgemm_select(ta, tb, M, N, K)[1] == first for _ in range(3))
    # large MLIP shapes go to the emulation
    assert emu.select_mode(552960, 768, 256) == "BF16X9"


def test_select_mode_follows_measured_winners():
    """The dispatcher's choices on shapes whose winner was clear (by more than
    25 %) in device times measured on MI355X (the calibration table kept with
    the profiles).  Every such winner is the emulation: MLIP layers at 6,144
    and 552,960 rows, squares, skinny shapes and long K; native FP32 wins
    only near-ties (at most 6 %: 2048 x 2048 x 32 and skinny shapes with
    K = 64)."""
    import emulated_fp32_matrix_amd as emu

    for M, N, K in [(552960, 256, 256), (6144, 256, 768), (6144, 256, 512), (6144, 3072, 1024),
                    (6144, 1024, 4096), (512, 512, 512), (1024, 1024, 1024), (3072, 3072, 3072),
                    (1024, 64, 256), (4096, 256, 2048), (65536, 256, 2048), (65536, 2048, 256),
                    (2048, 2048, 4096)]:
        assert emu.select_mode(M, N, K) == "BF16X9", (M, N, K)