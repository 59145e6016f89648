"""Matrices past 4 GiB, on an MI355X (through the C ABI).

X [140001 x 16384] bf16 is 4.59 GB, so rows from 131072 on start beyond byte
2^32 and rows from 65536 on beyond byte 2^31: every byte offset the kernels
form must be 64-bit there.  The matrix is drawn on the GPU by torch's seeded
normal generator (with outlier channels and zero blocks added), and sampled
rows (both sides of both boundaries, the ragged last tile, random rows) are
copied to the host and checked against the oracle run on those rows alone:
rows are independent in every entry point here.
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

T, D = 140001, 16384
NB = D // 32
TPS = 4096  # tokens per sample of the AdaLN case
EPS = float(np.float32(1e-6))
THREADS = max(1, min(16, os.cpu_count() or 1))
ROWS = sorted(
    {0, 1, 31, 32, 65535, 65536, 65537, 131071, 131072, 131073, 131103, 139999, 140000}
    | {int(r) for r in np.random.default_rng(5).choice(T, 16, replace=False)})


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kq.lib()
    g = torch.Generator(device="cuda:0")
    g.manual_seed(2024)
    X = torch.randn((T, D), generator=g, device="cuda:0", dtype=torch.bfloat16)
    cols = torch.from_numpy(np.random.default_rng(6).choice(D, D // 100, replace=False)).to("cuda:0")
    X[:, cols] *= 50.0
    X[3, 64:96] = 0          # all-zero blocks (scale byte 0) near both boundaries
    X[131072, 32:64] = 0
    X[140000, :32] = 0
    Xi = X.view(torch.int16)
    Xrows = Xi[ROWS].cpu().numpy().view(np.uint16)
    codes = torch.empty((T, D // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((T, NB), dtype=torch.uint8, device="cuda:0")
    yield Xi, Xrows, codes, scales
    del X, Xi, codes, scales
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sampled(codes, scales):
    torch.cuda.synchronize()
    return codes[ROWS].cpu().numpy(), scales[ROWS].cpu().numpy()


def check(name, front, Xrows, codes, scales, P=None, m=None, exact=False):
    c, s = sampled(codes, scales)
    ref = oracle.quantize_rows(front, Xrows, P, 15, m, threads=THREADS)

    def yh(rows):
        o = oracle.quantize_rows(front, Xrows[rows], P, 15, m, want_y=True)
        return o["yhat"], o["y32"]

    rep = compare(c, s, ref["codes"], ref["scales"], yh)
    print(f"{name} past 4 GiB: {rep}", flush=True)
    assert rep.ok(exact=exact), f"{name}: {rep}"


@pytest.mark.parametrize("variant", ["mfma_otf", "mfma_dense", "butterfly"])
def test_kron_past_4gib(big, variant):
    Xi, Xrows, codes, scales = big
    P = synth.random_params(NB, seed=61)
    Pd = torch.from_numpy(P).to("cuda:0")
    codes.fill_(0xEE)
    scales.fill_(0xEE)
    if variant == "mfma_dense":
        Kbf = torch.empty((NB, 3, 32, 32), dtype=torch.int16, device="cuda:0")
        kq.kq_build_blocks(Pd, NB, None, Kbf, 3)
        kq.kq_quantize_ex(Xi, None, 15, Kbf, kq.KQ_MFMA_DENSE, codes, scales)
    else:
        v = kq.KQ_MFMA_OTF if variant == "mfma_otf" else kq.KQ_BUTTERFLY
        kq.kq_quantize_ex(Xi, Pd, 15, None, v, codes, scales)
    check(variant, oracle.KRON, Xrows, codes, scales, P=P)


@pytest.mark.parametrize("front", ["plain", "smooth", "hadamard"])
def test_comparison_front_ends_past_4gib(big, front):
    Xi, Xrows, codes, scales = big
    codes.fill_(0xEE)
    scales.fill_(0xEE)
    m = None
    if front == "plain":
        kq.kq_mx_quantize(Xi, codes, scales)
        of = oracle.PLAIN
    elif front == "smooth":
        m = synth.smooth_mult(Xrows)
        kq.kq_smooth_quantize(Xi, torch.from_numpy(m).to("cuda:0"), codes, scales)
        of = oracle.SMOOTH
    else:
        kq.kq_hadamard_quantize(Xi, codes, scales)
        of = oracle.HADAMARD
    check(front, of, Xrows, codes, scales, m=m, exact=front != "hadamard")


def test_row_stats_and_adaln_past_4gib(big):
    Xi, Xrows, codes, scales = big
    st = torch.empty((T, 2), dtype=torch.float32, device="cuda:0")
    kq.kq_row_stats(Xi, EPS, st)
    torch.cuda.synchronize()
    ref_st = oracle.row_stats(Xrows, eps=EPS)
    got = st[ROWS].cpu().numpy()
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref_st.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, f"row stats: max {ulps.max()} ulp"

    # The fused kernel reads only its own row's statistics: the sampled rows
    # get the oracle's, every other row (mean 0, rstd 1).
    st_in = torch.zeros((T, 2), dtype=torch.float32, device="cuda:0")
    st_in[:, 1] = 1.0
    st_in[ROWS] = torch.from_numpy(ref_st).to("cuda:0")
    ns = (T + TPS - 1) // TPS
    sc, sh = synth.adaln_vectors(ns, D, seed=62)
    P = synth.random_params(NB, seed=63)
    codes.fill_(0xEE)
    scales.fill_(0xEE)
    kq.kq_quantize_adaln(Xi, st_in, torch.from_numpy(sc).to("cuda:0"), torch.from_numpy(sh).to("cuda:0"), TPS,
                         torch.from_numpy(P).to("cuda:0"), codes, scales)
    # each sampled row modulated with its own sample's vectors
    Xmod = np.concatenate([
        oracle.adaln_rows(Xrows[i:i + 1], ref_st[i:i + 1], sc[r // TPS:r // TPS + 1], sh[r // TPS:r // TPS + 1],
                          tokens_per_sample=1) for i, r in enumerate(ROWS)])
    check("adaln", oracle.KRON, Xmod, codes, scales, P=P)


def test_gemm_past_4gib():
    """Y [66000 x 32768]: the fp32 output passes byte 2^32 at row 32768, the
    bf16 one at row 65536; the last tile row is partial (66000 = 257 x 256 + 208).
    Random MXFP4 operands (K = 64), sampled rows, every column, against the
    oracle: |Y - exact| <= 1e-5 sum|a b|, bf16 = nearest-even rounding of the fp32."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M, N, K = 66000, 32768, 64
    rng = np.random.default_rng(71)
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    as_ = rng.integers(118, 136, size=(M, K // 32), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    bs = rng.integers(118, 136, size=(N, K // 32), dtype=np.uint8)
    t = lambda a: torch.from_numpy(a).to("cuda:0")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    yb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    kq.kq_gemm_mx(t(ac), t(as_), t(bc), t(bs), y, yb)
    torch.cuda.synchronize()
    rows = sorted({0, 32767, 32768, 32769, 65535, 65536, 65537, 65791, 65792, 65999}
                  | {int(r) for r in rng.choice(M, 12, replace=False)})
    got = y[rows].cpu().numpy().astype(np.float64)
    gotb = yb[rows].view(torch.int16).cpu().numpy()
    del y, yb
    torch.cuda.empty_cache()
    ref = oracle.gemm_mx(ac[rows], as_[rows], bc, bs)
    A = np.abs(oracle.dequant_rows(ac[rows], as_[rows]))
    B = np.abs(oracle.dequant_rows(bc, bs))
    bound = A @ B.T
    err = np.abs(got - ref)
    assert np.all(err <= 1e-5 * bound + 1e-30), float((err / np.maximum(bound, 1e-300)).max())
    np.testing.assert_array_equal(gotb, torch.from_numpy(got.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy())
