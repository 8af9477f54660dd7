"""The emulated modes' per-stream workspace (include/emu_sgemm.h, "Memory"):
a stream's buffer grows to the largest call, calls on different streams never
share one, and more than 16 streams per device evict the least recently used
buffer.  Every result is compared bit for bit with the oracle's model of the
same evaluation (oracle.emu_gemm_mfma) or with the same call on one stream.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def _case(seed, M, N, K):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, K)).astype(np.float32),
            rng.standard_normal((K, N)).astype(np.float32))


def test_growth_on_one_stream():
    """small -> large (pre-split B grows) -> split K (partials) -> small again."""
    import torch

    import emulated_fp32_matrix_amd as emu

    for i, (M, N, K, S) in enumerate([(64, 64, 32, None), (300, 1024, 1024, None),
                                      (640, 256, 768, 3), (33, 17, 40, None), (256, 256, 256, 2)]):
        a, b = _case(i, M, N, K)
        out = emu.sgemm(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), mode="BF16X9",
                        ksplit=S)
        torch.cuda.synchronize()
        want = oracle.emu_gemm_mfma(a, b, "BF16X9", ksplit=S or 1)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32)), (M, N, K, S)


def test_concurrent_streams_do_not_share_a_workspace():
    """Four streams with different shapes (and workspace sizes) issued
    back to back, several rounds: each result equals the same call alone."""
    import torch

    import emulated_fp32_matrix_amd as emu

    shapes = [(512, 768, 256, None), (384, 256, 768, 2), (700, 512, 512, None), (256, 128, 1024, 4)]
    cases = [_case(10 + i, *s[:3]) for i, s in enumerate(shapes)]
    dev = [(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()) for a, b in cases]
    alone = []
    for (da, db), s in zip(dev, shapes):
        alone.append(emu.sgemm(da, db, mode="BF16X9", ksplit=s[3]).cpu().numpy())
    streams = [torch.cuda.Stream() for _ in shapes]
    torch.cuda.synchronize()
    for _ in range(4):
        outs = []
        for (da, db), s, st in zip(dev, shapes, streams):
            with torch.cuda.stream(st):
                outs.append(emu.sgemm(da, db, mode="BF16X9", ksplit=s[3]))
        torch.cuda.synchronize()
        for o, want in zip(outs, alone):
            assert np.array_equal(o.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_more_streams_than_kept_buffers():
    """20 streams round-robin (16 keep a buffer): evicted buffers are released
    and replaced without disturbing the results."""
    import torch

    import emulated_fp32_matrix_amd as emu

    a, b = _case(3, 200, 300, 96)
    da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    want = oracle.emu_gemm_mfma(a, b, "BF16X9")
    streams = [torch.cuda.Stream() for _ in range(20)]
    for _ in range(2):
        outs = []
        for st in streams:
            with torch.cuda.stream(st):
                outs.append(emu.sgemm(da, db, mode="BF16X9"))
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(o.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_host_threads_each_on_its_own_stream():
    """Four host threads, each on a stream of its own, issue 12 calls each at
    the same time (the binding releases the GIL in the library call): mixed
    modes and shapes whose workspaces grow call after call, K splits,
    NATIVE_F32's packed B.  Every result equals the same call made alone
    from one thread."""
    import threading

    import torch

    import emulated_fp32_matrix_amd as emu

    plans = []
    for t in range(4):
        rng = np.random.default_rng(100 + t)
        calls = []
        for i in range(12):
            M, N = int(rng.integers(64, 1500)), int(rng.integers(32, 1200))
            K = int(rng.integers(8, 300)) * 4
            mode = ["BF16X9", "BF16X6", "AUTO", "NATIVE_F32", "BF16X3"][(t + i) % 5]
            nk = -(-K // 32)
            ksplit = 2 if mode in ("BF16X9", "BF16X6") and nk % 2 == 0 and i % 3 == 0 else None
            a = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).cuda()
            b = torch.from_numpy(rng.standard_normal((K, N)).astype(np.float32)).cuda()
            calls.append((a, b, mode, ksplit))
        plans.append(calls)
    alone = [[emu.sgemm(a, b, mode=m, ksplit=s).cpu() for a, b, m, s in calls] for calls in plans]
    torch.cuda.synchronize()

    results = [None] * 4
    errors = []

    def worker(t):
        try:
            st = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(st):
                for a, b, m, s in plans[t]:
                    outs.append(emu.sgemm(a, b, mode=m, ksplit=s))
            st.synchronize()
            results[t] = [o.cpu() for o in outs]
        except Exception as e:   # reported by the main thread
            errors.append((t, repr(e)))

    for _ in range(2):
        threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
        for th in threads:
            th.start()
        for th in threads:
            th.join(timeout=120)
        assert not any(th.is_alive() for th in threads), "a thread did not finish"
        assert not errors, errors
        for t in range(4):
            for i, (o, want) in enumerate(zip(results[t], alone[t])):
                assert torch.equal(o.view(torch.int32), want.view(torch.int32)), (t, i, plans[t][i][2])
