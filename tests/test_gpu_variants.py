"""Parity of the variant kernels with the CPU oracle on an MI355X (through the C ABI):
block-Hadamard front-ends of size 32..512 and 16-wide, 4-factor KroQuant
blocks (built on the GPU, applied by the dense MFMA quantizer).  Scales
bit-exact, codes exact except classified ties (>= 99.99% exact)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.compare import compare

kq = pytest.importorskip("w4a4_diffusion_transformer_amd")

pytestmark = pytest.mark.gpu

REPORT = os.environ.get("KQ_PARITY_REPORT")


def record(name: str, rep) -> None:
    print(f"{name}: {rep}", flush=True)
    if REPORT:
        with open(REPORT, "a") as f:
            f.write(f"{name}: {rep}\n")


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


def run_hadamard(X, B):
    Xd = dev(X)
    codes, scales = kq.alloc_outputs(Xd)
    kq.kq_hadamard_quantize_ex(Xd, B, codes, scales)
    torch.cuda.synchronize()
    return host(codes), host(scales)


def check_hadamard(name, X, B, rows=None):
    codes, scales = run_hadamard(X, B)
    Xs = X if rows is None else X[rows]
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    ref = oracle.quantize_rows_hadamard(Xs, B)

    def yh(r):
        o = oracle.quantize_rows_hadamard(Xs[r], B, want_y=True)
        return o["yhat"], o["y32"]

    rep = compare(codes, scales, ref["codes"], ref["scales"], yh)
    record(name, rep)
    assert rep.ok(), rep


@pytest.mark.parametrize("B", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("T,d", [(64, 1024), (37, 3072), (9, 12288)])
def test_hadamard_block_sizes(T, d, B):
    X = synth.random_matrix(T, d, seed=T + B, n_outliers=max(1, d // 100), mult=50.0)
    check_hadamard(f"hadamard{B} {T}x{d}", X, B)


def test_hadamard_ragged_and_partial_group():
    # d = 1152: the last 512-channel column group holds 4 blocks; B = 128 divides d
    X = synth.random_matrix(257, 1152, seed=5, n_outliers=12, mult=50.0)
    check_hadamard("hadamard128 257x1152", X, 128)


def test_hadamard_32_is_the_existing_kernel():
    X = synth.random_matrix(100, 2240, seed=6, n_outliers=20, mult=50.0)
    a = run_hadamard(X, 32)
    Xd = dev(X)
    c, s = kq.alloc_outputs(Xd)
    kq.kq_hadamard_quantize(Xd, c, s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a[0], host(c))
    np.testing.assert_array_equal(a[1], host(s))


@pytest.mark.parametrize("B", [128, 512])
def test_hadamard_full_flux_x2_sampled_rows(B):
    spec = synth.CONFIGS[3][1]
    X = synth.matrix(spec)
    rows = np.sort(np.random.default_rng(B).choice(spec.T, size=48, replace=False))
    check_hadamard(f"hadamard{B} flux_x2 (48 sampled rows)", X, B, rows=rows)


def params16(nb16, seed, sigma=0.1):
    rng = np.random.default_rng(seed)
    P = np.empty((nb16, 4, 3), dtype=np.float32)
    P[:, :, 0] = rng.normal(0, sigma, (nb16, 4))
    P[:, :, 1] = np.exp(rng.normal(0, sigma, (nb16, 4)))
    P[:, :, 2] = rng.normal(0, sigma, (nb16, 4))
    return P


def test_blocks16_bit_exact():
    P = params16(40, seed=1, sigma=0.3)
    K32 = torch.empty((20, 32, 32), dtype=torch.float32, device="cuda:0")
    Kbf = torch.empty((20, 3, 32, 32), dtype=torch.int16, device="cuda:0")
    kq.kq_build_blocks16(dev(P), 40, K32, Kbf, 3)
    torch.cuda.synchronize()
    ref = oracle.build_blocks16(P)
    np.testing.assert_array_equal(host(K32), ref)
    # the split reconstructs the blocks exactly
    parts = host(Kbf).view(np.uint16)
    recon = synth.bf16_to_f32(parts).astype(np.float64).sum(axis=1).transpose(0, 2, 1).astype(np.float32)
    np.testing.assert_array_equal(recon, ref)


@pytest.mark.parametrize("T,d", [(64, 1152), (300, 3072), (33, 12288), (4608, 3072)])
def test_blocks16_quantize(T, d):
    X = synth.random_matrix(T, d, seed=T * 3 + d, n_outliers=max(1, d // 100), mult=50.0)
    P = params16(d // 16, seed=d)
    nb = d // 32
    Kbf = torch.empty((nb, 3, 32, 32), dtype=torch.int16, device="cuda:0")
    kq.kq_build_blocks16(dev(P), d // 16, None, Kbf, 3)
    Xd = dev(X)
    codes, scales = kq.alloc_outputs(Xd)
    kq.kq_quantize_ex(Xd, None, 15, Kbf, kq.KQ_MFMA_DENSE, codes, scales)
    torch.cuda.synchronize()
    K32 = oracle.build_blocks16(P)
    ref = oracle.quantize_rows_blocks(X, K32, threads=8)

    def yh(r):
        o = oracle.quantize_rows_blocks(X[r], K32, want_y=True)
        return o["yhat"], o["y32"]

    rep = compare(host(codes), host(scales), ref["codes"], ref["scales"], yh)
    record(f"kroquant16 {T}x{d}", rep)
    assert rep.ok(), rep
