"""A transform learned by the offline calibration, run through the library's W4A4 kernels on an MI355X and
compared element by element with the oracle's pipeline (Pith review, "What carries the argument": learned
per-block scalars feed the online quantizer; "What would settle it"; circularity check, Eq. (1): the folded
weight W K^-T and the product of the two quantized operands).

  * kq_quantize(X, theta) against oracle.quantize_rows(KRON): scales exact, codes exact except classified
    rounding ties;
  * the weight fold, kq_build_blocks_inverse_t + dense kq_quantize_ex, against
    oracle.build_blocks_inverse_t + oracle.quantize_rows_blocks: the same rule;
  * kq_gemm_mx on the GPU's codes against oracle.gemm_mx on the same codes: per element within
    1e-5 of sum_k |a_k b_k|; and against oracle.gemm_mx on the oracle's codes, per element, wherever
    neither operand row holds a tie code.

The relative output error against the calibration's own fp32 fake-quantized model (within 2%) stays as a
secondary check.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.compare import compare
from w4a4_diffusion_transformer_amd import calibrate as cal

kq = pytest.importorskip("w4a4_diffusion_transformer_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kq.lib()
    yield


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


@pytest.fixture(scope="module", params=[(5, 20), (5, 70)], ids=["outliers_same_block", "outliers_far_apart"])
def learned(request):
    X, W = cal.synthetic_layer(256, 256, 192, request.param, 50.0, seed=3)
    theta, _ = cal.calibrate(X, W, steps=20)
    P = np.ascontiguousarray(theta.detach().cpu().numpy(), dtype=np.float32)
    Xb = synth.f32_to_bf16(X.cpu().numpy().astype(np.float32))
    Wb = synth.f32_to_bf16(W.cpu().numpy().astype(np.float32))
    # the layer is bf16 already: the bits are its exact values
    assert np.array_equal(synth.bf16_to_f32(Xb), X.cpu().numpy())
    return request.param, X, W, theta, P, Xb, Wb


def yh_of(ref):
    return lambda rows: (ref["yhat"][rows], ref["y32"][rows])


def test_learned_theta_on_the_kernels_matches_the_oracle(learned):
    outliers, X, W, theta, P, Xb, Wb = learned
    nb = P.shape[0]
    # learned, not the initialization: the factors moved away from the Hadamard-like start
    assert np.abs(P - cal.hadamard_init(nb).numpy()).max() > 1e-3

    # ---- GPU: quantize X T, fold and quantize W, multiply
    Xd, Pd, Wd = dev(Xb), dev(P), dev(Wb)
    xc, xs = kq.alloc_outputs(Xd)
    kq.kq_quantize(Xd, Pd, xc, xs)
    Kit = torch.empty((nb, 3, 32, 32), dtype=torch.int16, device="cuda:0")
    kq.kq_build_blocks_inverse_t(Pd, nb, None, Kit, 3)
    wc, ws = kq.alloc_outputs(Wd)
    kq.kq_quantize_ex(Wd, None, 15, Kit, kq.KQ_MFMA_DENSE, wc, ws)
    Y = torch.empty((Xb.shape[0], Wb.shape[0]), dtype=torch.float32, device="cuda:0")
    kq.kq_gemm_mx(xc, xs, wc, ws, Y)
    torch.cuda.synchronize()
    gxc, gxs, gwc, gws, gy = host(xc), host(xs), host(wc), host(ws), host(Y).astype(np.float64)

    # ---- oracle pipeline
    ox = oracle.quantize_rows(oracle.KRON, Xb, P, want_y=True)
    K32it, _ = oracle.build_blocks_inverse_t(P, nb)
    ow = oracle.quantize_rows_blocks(Wb, K32it, want_y=True)

    rx = compare(gxc, gxs, ox["codes"], ox["scales"], yh_of(ox))
    rw = compare(gwc, gws, ow["codes"], ow["scales"], yh_of(ow))
    print(f"outliers {outliers}: activation {rx}; folded weight {rw}", flush=True)
    for r, n in ((rx, gxc.size * 2), (rw, gwc.size * 2)):
        assert r.scale_mismatch == 0 and r.code_unexplained == 0, str(r)
        # ties are rare: at most 1e-4 of the codes (a handful at these sizes)
        assert r.code_mismatch <= max(4, 1e-4 * n), str(r)

    # the GEMM on the GPU's own codes: per element within its accumulation bound
    bound = np.abs(oracle.dequant_rows(gxc, gxs)) @ np.abs(oracle.dequant_rows(gwc, gws)).T
    y_same = oracle.gemm_mx(gxc, gxs, gwc, gws)
    assert np.all(np.abs(gy - y_same) <= 1e-5 * bound + 1e-30), float((np.abs(gy - y_same) / np.maximum(bound, 1e-300)).max())

    # against the oracle's whole pipeline wherever neither operand row holds a tie code
    y_ref = oracle.gemm_mx(ox["codes"], ox["scales"], ow["codes"], ow["scales"])
    rows_x = np.flatnonzero(np.any(gxc != ox["codes"], axis=1))
    rows_w = np.flatnonzero(np.any(gwc != ow["codes"], axis=1))
    keep = np.ones(gy.shape, dtype=bool)
    keep[rows_x, :] = False
    keep[:, rows_w] = False
    assert keep.mean() > 0.9
    err = np.abs(gy - y_ref)[keep]
    assert np.all(err <= 1e-5 * bound[keep] + 1e-30), float((err / np.maximum(bound[keep], 1e-300)).max())

    # secondary: the output error agrees with the calibration's fp32 fake-quantized model
    e_model = cal.error_kroquant(theta, X, W)
    e_gpu = cal.error_on_gpu_path(theta, X, W)
    print(f"outliers {outliers}: tie rows X {len(rows_x)}, W {len(rows_w)}; fp32 model {e_model:.6f}, "
          f"GPU kernels {e_gpu:.6f}", flush=True)
    assert abs(e_gpu - e_model) <= 0.02 * e_model
    assert e_gpu < cal.error_plain(X, W)
