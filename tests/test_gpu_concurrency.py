"""Reentrancy on an MI355X: four host threads, each with its own HIP stream
(default priority) and its own buffers, call the library at the same time
(quantize with in-kernel K, with prebuilt K, fused AdaLN quantize, GEMM, and
kq_tune, whose process-wide table is shared); every result must equal the one
the same call gives alone.  ctypes releases the GIL during foreign calls, so
the library's host code runs concurrently."""
import threading

import numpy as np
import pytest
import torch

import synth

kq = pytest.importorskip("w4a4_diffusion_transformer_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kq.lib()
    kq.kq_tune_reset()
    yield
    kq.kq_tune_reset()


def dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def make_job(i):
    T, d = 512 + 96 * i, 1152 * (1 + i % 3)
    X = dev(synth.random_matrix(T, d, seed=90 + i, n_outliers=d // 100, mult=60.0))
    P = dev(synth.random_params(d // 32, seed=95 + i))
    Kbf = torch.empty((d // 32, 3, 32, 32), dtype=torch.int16, device="cuda:0")
    kq.kq_build_blocks(P, d // 32, None, Kbf, 3)
    stats = torch.empty((T, 2), dtype=torch.float32, device="cuda:0")
    rng = np.random.default_rng(99 + i)
    msc = torch.from_numpy(rng.normal(0, 0.5, (1, d)).astype(np.float32)).to("cuda:0")
    msh = torch.from_numpy(rng.normal(0, 0.1, (1, d)).astype(np.float32)).to("cuda:0")
    outs = [kq.alloc_outputs(X) for _ in range(4)]
    y = torch.empty((T, 256), dtype=torch.bfloat16, device="cuda:0")
    W = dev(synth.random_matrix(256, d, seed=80 + i, n_outliers=0, mult=1.0))
    cw, sw = kq.alloc_outputs(W)

    def run(stream, tune):
        with torch.cuda.stream(stream):
            kq.kq_quantize(X, P, *outs[0])
            kq.kq_quantize_ex(X, None, 15, Kbf, kq.KQ_MFMA_DENSE, *outs[1])
            kq.kq_row_stats(X, 1e-6, stats)
            kq.kq_quantize_adaln(X, stats, msc, msh, T, P, *outs[2])
            kq.kq_quantize_ex(W, P, 15, None, kq.KQ_MFMA_OTF, cw, sw)
            kq.kq_gemm_mx(outs[0][0], outs[0][1], cw, sw, y_bf16=y)
            if tune:
                kq.kq_tune(X, P, Kbf, *outs[3], reps=2)

    def result():
        return [t.clone() for pair in outs[:3] for t in pair] + [stats.clone(), cw.clone(), sw.clone(), y.clone()]

    def clear():
        for pair in outs:
            for t in pair:
                t.zero_()
        for t in (stats, cw, sw, y):
            t.zero_()

    return run, result, clear


def test_threads_on_own_streams_match_single_calls():
    jobs = [make_job(i) for i in range(4)]
    streams = [torch.cuda.Stream() for _ in jobs]
    ref = []
    for (run, result, clear), s in zip(jobs, streams):
        run(s, tune=False)
        torch.cuda.synchronize()
        ref.append(result())
    for rep in range(3):
        for _, _, clear in jobs:
            clear()
        torch.cuda.synchronize()
        errors = []

        def worker(k):
            try:
                for _ in range(5):
                    jobs[k][0](streams[k], tune=(k == rep))
            except Exception as e:  # reported below, in the main thread
                errors.append(e)

        threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(jobs))]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        assert not errors, errors
        for k, (_, result, _) in enumerate(jobs):
            got = result()
            for a, b in zip(got, ref[k]):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"job {k}, round {rep}"
