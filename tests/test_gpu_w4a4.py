"""Parity of the W4A4 consumer side on an MI355X (through the C ABI): the
weight-fold blocks K^-T, the folded weight's MXFP4 codes, and the scaled-FP4
GEMM, against the CPU oracle.

  * kq_build_blocks_inverse_t: bit-exact fp32 blocks and bf16 split;
  * folded weight (kq_quantize_ex with the K^-T split): scales bit-exact,
    codes exact except classified ties, as for the activation quantizer;
  * kq_gemm_mx: per element |Y_gpu - Y_exact| <= 1e-5 * sum_k |a_k b_k| (fp32
    sums of exact products), the bf16 output the nearest-even rounding of the
    fp32 one, rows/columns/K tails included;
  * the whole W4A4 pipeline (quantize X T, fold and quantize W, GEMM) against
    the oracle's pipeline, and its output error against X W^T below plain
    MXFP4's on activations with outlier channels.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.compare import compare

kq = pytest.importorskip("w4a4_diffusion_transformer_amd")

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))
REPORT = os.environ.get("KQ_PARITY_REPORT")


def record(name: str, msg) -> None:
    print(f"{name}: {msg}", flush=True)
    if REPORT:
        with open(REPORT, "a") as f:
            f.write(f"{name}: {msg}\n")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kq.lib()
    yield


def dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    return t.cpu().numpy()


def test_inverse_t_blocks_bit_exact():
    P = synth.random_params(24, seed=51, sigma_lb=0.3, sigma_a=0.3)
    K32 = torch.empty((24, 32, 32), dtype=torch.float32, device="cuda:0")
    Kbf = torch.empty((24, 3, 32, 32), dtype=torch.int16, device="cuda:0")
    kq.kq_build_blocks_inverse_t(dev(P), 24, K32, Kbf, 3)
    torch.cuda.synchronize()
    r32, rbf = oracle.build_blocks_inverse_t(P, 24)
    np.testing.assert_array_equal(host(K32), r32)
    np.testing.assert_array_equal(host(Kbf).view(np.uint16), rbf)


def fold_gpu(W: np.ndarray, P: np.ndarray):
    nb = P.shape[0]
    Kbf = torch.empty((nb, 3, 32, 32), dtype=torch.int16, device="cuda:0")
    kq.kq_build_blocks_inverse_t(dev(P), nb, None, Kbf, 3)
    Wd = dev(W)
    codes, scales = kq.alloc_outputs(Wd)
    kq.kq_quantize_ex(Wd, None, 15, Kbf, kq.KQ_MFMA_DENSE, codes, scales)
    torch.cuda.synchronize()
    return host(codes), host(scales)


@pytest.mark.parametrize("N,K", [(64, 1152), (257, 3072), (96, 12288)])
def test_folded_weight_codes(N, K):
    rng = np.random.default_rng(N + K)
    W = synth.f32_to_bf16((rng.normal(size=(N, K)) * 0.05).astype(np.float32))
    P = synth.random_params(K // 32, seed=52)
    codes, scales = fold_gpu(W, P)
    K32it, _ = oracle.build_blocks_inverse_t(P, K // 32)
    ref = oracle.quantize_rows_blocks(W, K32it, threads=THREADS)

    def yh(rows):
        o = oracle.quantize_rows_blocks(W[rows], K32it, want_y=True)
        return o["yhat"], o["y32"]

    rep = compare(codes, scales, ref["codes"], ref["scales"], yh)
    record(f"fold {N}x{K}", rep)
    assert rep.ok(), rep


def random_mx(rows: int, K: int, seed: int):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(118, 136, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales


def gemm_bound(a_codes, a_scales, b_codes, b_scales):
    A = np.abs(oracle.dequant_rows(a_codes, a_scales))
    B = np.abs(oracle.dequant_rows(b_codes, b_scales))
    return A @ B.T


def run_gemm(a_codes, a_scales, b_codes, b_scales):
    M, N = a_codes.shape[0], b_codes.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    yb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    kq.kq_gemm_mx(dev(a_codes), dev(a_scales), dev(b_codes), dev(b_scales), y, yb)
    torch.cuda.synchronize()
    return y, yb


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (128, 128, 128), (77, 200, 160), (300, 257, 2240), (512, 384, 1152),
                                   (16, 640, 5600), (256, 130, 12288), (33, 45, 96), (260, 300, 1504)])
def test_gemm_parity(M, N, K):
    ac, as_ = random_mx(M, K, seed=M * 3 + K)
    bc, bs = random_mx(N, K, seed=N * 5 + K + 1)
    y, yb = run_gemm(ac, as_, bc, bs)
    ref = oracle.gemm_mx(ac, as_, bc, bs)
    bound = gemm_bound(ac, as_, bc, bs)
    err = np.abs(host(y).astype(np.float64) - ref)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    record(f"gemm {M}x{N}x{K}", f"max error {worst:.3g} of sum|ab|")
    assert np.all(err <= 1e-5 * bound + 1e-30), worst
    # bf16 output: the nearest-even rounding of the same fp32 sums
    np.testing.assert_array_equal(host(yb.view(torch.int16)), host(y.to(torch.bfloat16).view(torch.int16)))


def test_gemm_zero_codes_give_zero():
    ac = np.zeros((64, 64), np.uint8)
    as_ = np.full((64, 4), 127, np.uint8)
    bc, bs = random_mx(32, 128, seed=3)
    y, _ = run_gemm(ac, as_, bc, bs)
    assert not np.any(host(y))


def test_gemm_full_size_sampled_rows():
    """FLUX.1-schnell MLP fc1 shape (4608 tokens x 3072 -> 12288): every column of 64 sampled rows."""
    M, N, K = 4608, 12288, 3072
    ac, as_ = random_mx(M, K, seed=61)
    bc, bs = random_mx(N, K, seed=62)
    y, _ = run_gemm(ac, as_, bc, bs)
    rows = np.random.default_rng(63).choice(M, size=64, replace=False)
    ref = oracle.gemm_mx(ac[rows], as_[rows], bc, bs)
    bound = gemm_bound(ac[rows], as_[rows], bc, bs)
    err = np.abs(host(y)[rows].astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * bound + 1e-30), float((err / bound).max())


def test_gemm_whole_and_half_tiles():
    """4352 x 4096 output: 272 tiles of 256 x 256 on 256 compute units, so the
    first 256 run whole and the 16 of the last, partial round (the band of
    rows 4096 .. 4351) run as two 128-row halves each; rows of both kinds
    checked against the oracle, every column."""
    M, N, K = 4352, 4096, 256
    ac, as_ = random_mx(M, K, seed=81)
    bc, bs = random_mx(N, K, seed=82)
    y, yb = run_gemm(ac, as_, bc, bs)
    rng = np.random.default_rng(83)
    rows = np.concatenate([rng.choice(4096, size=48, replace=False), np.arange(4096, M, 5), [M - 1]])
    ref = oracle.gemm_mx(ac[rows], as_[rows], bc, bs)
    bound = gemm_bound(ac[rows], as_[rows], bc, bs)
    err = np.abs(host(y)[rows].astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * bound + 1e-30), float((err / np.maximum(bound, 1e-300)).max())
    np.testing.assert_array_equal(host(yb.view(torch.int16)), host(y.to(torch.bfloat16).view(torch.int16)))


def test_gemm_errors():
    ac, as_ = random_mx(8, 64, seed=1)
    with pytest.raises(ValueError):
        kq.kq_gemm_mx(dev(ac), dev(as_), dev(ac[:, :16]), dev(as_[:, :1]), torch.empty((8, 8), device="cuda:0"))
    with pytest.raises(kq.KQError) as e:
        kq.kq_gemm_mx(dev(ac), dev(as_), dev(ac), dev(as_))
    assert e.value.status == 1


def test_w4a4_pipeline_against_oracle_and_plain_mx():
    """Quantize X T on the GPU, fold and quantize W, multiply; compare with the oracle's pipeline and
    check that the Hadamard-like transform lowers the output error against X W^T compared to plain MXFP4."""
    T, d, n_out = 1024, 3072, 1536
    X = synth.random_matrix(T, d, seed=71, n_outliers=15, mult=100.0, token_sigma=1.0)
    rng = np.random.default_rng(72)
    W = synth.f32_to_bf16((rng.normal(size=(n_out, d)) * 0.05).astype(np.float32))
    nb = d // 32
    sq = float(np.float32(1 / np.sqrt(2)))
    P = np.zeros((nb, 5, 3), dtype=np.float32)
    P[:, :, 0], P[:, :, 1], P[:, :, 2] = 1.0, sq, -sq
    Xd, Pd = dev(X), dev(P)
    xc, xs = kq.alloc_outputs(Xd)
    kq.kq_quantize(Xd, Pd, xc, xs)
    wc, ws = fold_gpu(W, P)
    y, _ = run_gemm(host(xc), host(xs), wc, ws)
    y = host(y).astype(np.float64)
    # the oracle's pipeline
    oxq = oracle.quantize_rows(oracle.KRON, X, P, threads=THREADS)
    K32it, _ = oracle.build_blocks_inverse_t(P, nb)
    owq = oracle.quantize_rows_blocks(W, K32it, threads=THREADS)
    y_ref = oracle.gemm_mx(oxq["codes"], oxq["scales"], owq["codes"], owq["scales"])
    bound = gemm_bound(oxq["codes"], oxq["scales"], owq["codes"], owq["scales"])
    # codes may differ from the oracle's at rounding ties (one grid step each), so the bound is loose
    rel_pipe = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
    assert rel_pipe < 1e-4, rel_pipe
    exact = synth.bf16_to_f32(X).astype(np.float64) @ synth.bf16_to_f32(W).astype(np.float64).T
    pc, ps = kq.alloc_outputs(Xd)
    kq.kq_mx_quantize(Xd, pc, ps)
    Wd = dev(W)
    wpc, wps = kq.alloc_outputs(Wd)
    kq.kq_mx_quantize(Wd, wpc, wps)
    yp, _ = run_gemm(host(pc), host(ps), host(wpc), host(wps))
    err = lambda a: np.linalg.norm(a - exact) / np.linalg.norm(exact)
    e_kq, e_plain = err(y), err(host(yp).astype(np.float64))
    record("w4a4 pipeline flux-width 1024x3072 -> 1536", f"rel. error KroQuant(Hadamard-like) {e_kq:.4f}, plain MXFP4 "
                                                          f"{e_plain:.4f}; GPU vs oracle pipeline {rel_pipe:.2e}")
    assert e_kq < 0.95 * e_plain
    assert np.all(np.abs(y - y_ref) <= 1e-5 * bound + 1e-3 * np.abs(bound).max())
