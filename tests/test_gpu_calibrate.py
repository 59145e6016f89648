"""The calibrated transform evaluated on the library's W4A4 kernels (kq_quantize of X T, the weight fold
through kq_build_blocks_inverse_t + kq_quantize_ex, kq_gemm_mx) gives the same output error as the
calibration's own fp32 fake-quantized model of that path (Pith review, Eqs. (1), (2), (9))."""
import pytest
import torch

from w4a4_diffusion_transformer_amd import calibrate as cal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("outliers", [(5, 20), (5, 70)])
def test_gpu_path_matches_fake_quant_model(outliers):
    X, W = cal.synthetic_layer(256, 256, 192, outliers, 50.0, seed=3)
    theta, _ = cal.calibrate(X, W, steps=20)
    e_model = cal.error_kroquant(theta, X, W)
    e_gpu = cal.error_on_gpu_path(theta, X, W)
    print(f"outliers {outliers}: fp32 model {e_model:.6f}, GPU kernels {e_gpu:.6f}", flush=True)
    # the model rounds X T and W T^-T in fp32, the kernels from exactly rounded sums: codes differ only where
    # a value sits within fp32 rounding of a decision threshold, a few per million
    assert abs(e_gpu - e_model) <= 0.02 * e_model
    e_plain = cal.error_plain(X, W)
    assert e_gpu < e_plain
