"""The per-shape tuner on an MI355X: kq_tune times the variants the inputs
allow, records the fastest for KQ_AUTO at that shape, leaves that variant's
result in the outputs, and kq_tune_reset forgets it."""
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


@pytest.mark.parametrize("T,d", [(4608, 3072), (8192, 1152)])
def test_tune_records_and_reproduces(T, d):
    X = synth.random_matrix(T, d, seed=T + d, n_outliers=d // 100, mult=50.0)
    P = synth.random_params(d // 32, seed=d)
    Xd, Pd = dev(X), dev(P)
    Kbf = torch.empty((d // 32, 3, 32, 32), dtype=torch.int16, device="cuda:0")
    kq.kq_build_blocks(Pd, d // 32, None, Kbf, 3)
    codes, scales = kq.alloc_outputs(Xd)
    v = kq.kq_tune(Xd, Pd, Kbf, codes, scales, reps=5)
    torch.cuda.synchronize()
    assert v in (kq.KQ_MFMA_OTF, kq.KQ_MFMA_DENSE, kq.KQ_BUTTERFLY)
    assert kq.kq_auto_variant(T, d, True, True) == v
    # the outputs are that variant's result, and KQ_AUTO now runs it
    c2, s2 = kq.alloc_outputs(Xd)
    kq.kq_quantize_ex(Xd, None if v == kq.KQ_MFMA_DENSE else Pd, 15, Kbf if v == kq.KQ_MFMA_DENSE else None, v, c2, s2)
    c3, s3 = kq.alloc_outputs(Xd)
    kq.kq_quantize_ex(Xd, Pd, 15, Kbf, kq.KQ_AUTO, c3, s3)
    torch.cuda.synchronize()
    assert torch.equal(codes, c2) and torch.equal(scales, s2)
    assert torch.equal(codes, c3) and torch.equal(scales, s3)
    # other keys keep the default rule
    assert kq.kq_auto_variant(T, d, True, False) == kq.KQ_BUTTERFLY
    kq.kq_tune_reset()
    assert kq.kq_auto_variant(T, d, True, True) == kq.KQ_BUTTERFLY


@pytest.mark.parametrize("T,d", [(4096, 2240), (8192, 1152), (300, 3072)])
def test_tuned_grid_split_leaves_results_unchanged(T, d):
    """kq_tune also picks the size of the MFMA kernel's second grid part; the
    outputs after tuning are bit-identical to the untuned ones (the split only
    decides which workgroup computes a tile)."""
    kq.kq_tune_reset()
    X = synth.random_matrix(T, d, seed=3 * T + d, n_outliers=d // 50, mult=80.0)
    P = synth.random_params(d // 32, seed=d + 7)
    Xd, Pd = dev(X), dev(P)
    Kbf = torch.empty((d // 32, 3, 32, 32), dtype=torch.int16, device="cuda:0")
    kq.kq_build_blocks(Pd, d // 32, None, Kbf, 3)
    ref = {}
    for v in (kq.KQ_MFMA_OTF, kq.KQ_MFMA_DENSE):
        c, s = kq.alloc_outputs(Xd)
        kq.kq_quantize_ex(Xd, Pd if v == kq.KQ_MFMA_OTF else None, 15, Kbf if v == kq.KQ_MFMA_DENSE else None, v, c, s)
        ref[v] = (c, s)
    codes, scales = kq.alloc_outputs(Xd)
    v = kq.kq_tune(Xd, Pd, Kbf, codes, scales, reps=3)
    c2, s2 = kq.alloc_outputs(Xd)
    kq.kq_quantize_ex(Xd, Pd, 15, Kbf, kq.KQ_AUTO, c2, s2)
    torch.cuda.synchronize()
    if v in ref:
        assert torch.equal(codes, ref[v][0]) and torch.equal(scales, ref[v][1])
        assert torch.equal(c2, ref[v][0]) and torch.equal(s2, ref[v][1])
    kq.kq_tune_reset()
