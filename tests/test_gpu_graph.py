"""The library under HIP graph capture on an MI355X: a DiT linear layer's
quantized path (row statistics, fused AdaLN quantize, plain quantize of a
second activation, weight-side quantize, W4A4 GEMM) captured once into a HIP
graph (torch.cuda.graph, whose capture stream the binding passes to every
call) and replayed several times, with eager work and synchronisations of the
program's own between replays; every replay must reproduce the eager results
bit for bit.  The library allocates nothing, never synchronizes and sets no
memory with memset, so capture needs nothing from it."""
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


def dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def test_graph_replays_match_eager():
    T, d, N = 640, 3072, 1152
    X = dev(synth.random_matrix(T, d, seed=71, n_outliers=15, mult=100.0))
    X2 = dev(synth.random_matrix(T, d, seed=72, n_outliers=15, mult=100.0))
    W = dev(synth.random_matrix(N, d, seed=73, n_outliers=0, mult=1.0))
    P = dev(synth.random_params(d // 32, seed=74))
    rng = np.random.default_rng(75)
    mscale = torch.from_numpy(rng.normal(0, 0.5, (2, d)).astype(np.float32)).to("cuda:0")
    mshift = torch.from_numpy(rng.normal(0, 0.1, (2, d)).astype(np.float32)).to("cuda:0")
    Kinv = torch.empty((d // 32, 3, 32, 32), dtype=torch.int16, device="cuda:0")
    kq.kq_build_blocks_inverse_t(P, d // 32, None, Kinv, 3)
    torch.cuda.synchronize()

    stats = torch.empty((T, 2), dtype=torch.float32, device="cuda:0")
    ca, sa = kq.alloc_outputs(X)
    c2, s2 = kq.alloc_outputs(X2)
    cw, sw = kq.alloc_outputs(W)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda:0")

    def layer():
        kq.kq_row_stats(X, 1e-6, stats)
        kq.kq_quantize_adaln(X, stats, mscale, mshift, 320, P, ca, sa)
        kq.kq_quantize(X2, P, c2, s2)
        kq.kq_quantize_ex(W, None, 15, Kinv, kq.KQ_MFMA_DENSE, cw, sw)
        kq.kq_gemm_mx(ca, sa, cw, sw, y_bf16=y)

    outs = (stats, ca, sa, c2, s2, cw, sw, y)
    layer()
    pc, ps = kq.alloc_outputs(X)
    kq.kq_quantize(X, P, pc, ps)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()  # warm-up on the side stream, as torch's capture recipe asks
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    torch.cuda.synchronize()

    other_c, other_s = kq.alloc_outputs(X2)
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}"
        # eager work of the program's own between replays
        other_c.zero_()
        kq.kq_quantize(X, P, other_c, other_s)
        torch.cuda.synchronize()
        assert torch.equal(other_c, pc) and torch.equal(other_s, ps)
