"""Parity of the fused AdaLN producer step + quantizer, and of the LayerNorm
row statistics, with the CPU oracle, on an MI355X (through the C ABI).

The fused entry point must produce exactly what the quantizer produces on the
bf16 matrix the oracle's producer step writes: scales bit-exact, codes exact
except at rounding ties inside the transform's error bound, and bit-identical
to kq_quantize_ex on the oracle's modulated matrix (the GPU rounds to the same
bf16 values and then runs the same transform).  Row statistics within one fp32
ulp of the oracle's sequential fp64 evaluation.
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
EPS = float(np.float32(1e-6))


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
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    return t.cpu().numpy()


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def inputs(T, d, tps, seed, kind=synth.BASE_NORMAL):
    X = synth.random_matrix(T, d, seed, kind=kind, n_outliers=max(1, d // 100), mult=50.0, token_sigma=0.5)
    P = synth.random_params(d // 32, seed=seed + 100)
    ns = (T + tps - 1) // tps
    sc, sh = synth.adaln_vectors(ns, d, seed=seed + 200)
    st = oracle.row_stats(X, eps=EPS)
    return X, P, st, sc, sh


def run_fused(X, P, st, sc, sh, tps, variant):
    Xd = dev(X)
    codes, scales = kq.alloc_outputs(Xd)
    Pd = dev(P)
    Kbf = None
    if variant == kq.KQ_MFMA_DENSE:
        Kbf = torch.empty((P.shape[0], 3, 32, 32), dtype=torch.int16, device="cuda:0")
        kq.kq_build_blocks(Pd, P.shape[0], None, Kbf, 3)
        Pd = None
    kq.kq_quantize_adaln(Xd, dev(st), dev(sc), dev(sh), tps, Pd, codes, scales, 15, Kbf, variant)
    torch.cuda.synchronize()
    return host(codes), host(scales)


def run_plain_kron(Xmod, P, variant=kq.KQ_MFMA_OTF):
    Xd = dev(Xmod)
    codes, scales = kq.alloc_outputs(Xd)
    Pd, Kbf = dev(P), None
    if variant == kq.KQ_MFMA_DENSE:
        Kbf = torch.empty((P.shape[0], 3, 32, 32), dtype=torch.int16, device="cuda:0")
        kq.kq_build_blocks(Pd, P.shape[0], None, Kbf, 3)
        Pd = None
    kq.kq_quantize_ex(Xd, Pd, 15, Kbf, variant, codes, scales)
    torch.cuda.synchronize()
    return host(codes), host(scales)


def check(name, X, P, st, sc, sh, tps, variant, against_unfused=True):
    codes, scales = run_fused(X, P, st, sc, sh, tps, variant)
    Xmod = oracle.adaln_rows(X, st, sc, sh, tokens_per_sample=tps)
    ref = oracle.quantize_rows(oracle.KRON, Xmod, P, threads=THREADS)

    def yh(rows):
        o = oracle.quantize_rows(oracle.KRON, Xmod[rows], P, want_y=True)
        return o["yhat"], o["y32"]

    rep = compare(codes, scales, ref["codes"], ref["scales"], yh)
    record(name, rep)
    assert rep.ok(), f"{name}: {rep}"
    if against_unfused:
        # the same variant on the oracle's modulated matrix: bit for bit
        c2, s2 = run_plain_kron(Xmod, P, variant)
        np.testing.assert_array_equal(scales, s2)
        np.testing.assert_array_equal(codes, c2)


# ---------------------------------------------------------------- row statistics


@pytest.mark.parametrize("T,d", [(1, 32), (7, 64), (33, 1152), (300, 3072), (64, 12288), (1000, 160), (5, 16416),
                                 (37, 4608), (19, 8224)])
def test_row_stats(T, d):
    X = synth.random_matrix(T, d, seed=T + d, n_outliers=max(1, d // 64), mult=80.0)
    st = torch.empty((T, 2), dtype=torch.float32, device="cuda:0")
    kq.kq_row_stats(dev(X), EPS, st)
    torch.cuda.synchronize()
    ref = oracle.row_stats(X, eps=EPS)
    got = host(st)
    u = ulp_diff(got, ref)
    assert u.max() <= 1, f"max ulp {u.max()}"
    assert (u == 0).mean() >= 0.99


@pytest.mark.parametrize("d", [1152, 3072, 12288])
def test_row_stats_offset_rows(d):
    """Rows whose mean is large against their spread: the kernel takes
    sum (x - mean)^2 as sum x^2 - mean sum x only while that stays accurate,
    and these rows (mean^2 / var from about 1 to about 10^5) land on both
    sides of that test, next to plain rows, in one launch."""
    rng = np.random.default_rng(d)
    T = 64
    base = [(0.0, 1.0), (30.0, 1.0), (1000.0, 8.0), (-200.0, 0.5), (5.0, 0.05), (64.0, 2.0), (2.0, 1.0), (-1.0, 0.02)]
    rows = [rng.normal(base[i % len(base)][0], base[i % len(base)][1], d).astype(np.float32) for i in range(T)]
    X = synth.f32_to_bf16(np.stack(rows))
    st = torch.empty((T, 2), dtype=torch.float32, device="cuda:0")
    kq.kq_row_stats(dev(X), EPS, st)
    torch.cuda.synchronize()
    ref = oracle.row_stats(X, eps=EPS)
    got = host(st)
    u = ulp_diff(got, ref)
    assert u.max() <= 1, f"max ulp {u.max()}"
    assert (u == 0).mean() >= 0.99


def test_row_stats_constant_and_zero_rows():
    X = np.zeros((4, 64), dtype=np.uint16)
    X[1] = synth.f32_to_bf16(np.full(64, 3.0, np.float32))
    st = torch.empty((4, 2), dtype=torch.float32, device="cuda:0")
    kq.kq_row_stats(dev(X), EPS, st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(st), oracle.row_stats(X, eps=EPS))


# ---------------------------------------------------------------- fused producer step


MODES = {
    "all": (True, True, True),
    "stats_only": (True, False, False),
    "modulation_only": (False, True, True),
    "scale_only": (False, True, False),
}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("T,d,tps", [(64, 1152, 32), (300, 3072, 300), (257, 2240, 128), (96, 5600, 64)])
@pytest.mark.parametrize("variant", [3, 2, 1])
def test_fused_small(T, d, tps, mode, variant):
    X, P, st, sc, sh = inputs(T, d, tps, seed=T * 7 + d)
    us, usc, ush = MODES[mode]
    check(f"adaln {T}x{d} tps{tps} {mode} v{variant}", X, P, st if us else None, sc if usc else None,
          sh if ush else None, tps, variant)


@pytest.mark.parametrize("variant", [3, 2])
def test_fused_without_producer_inputs_equals_quantizer(variant):
    X, P, _, _, _ = inputs(200, 1152, 200, seed=5)
    codes, scales = run_fused(X, P, None, None, None, 200, variant)
    c2, s2 = run_plain_kron(X, P, variant)
    np.testing.assert_array_equal(codes, c2)
    np.testing.assert_array_equal(scales, s2)


@pytest.mark.parametrize("name,T,d,tps,kind", [
    ("flux_x1", 4608, 3072, 4608, synth.BASE_NORMAL),        # FLUX.1-schnell width, one sample of 4096 + 512 tokens
    ("pixart_x1", 8192, 1152, 4096, synth.BASE_NORMAL),      # PixArt-Sigma width, batch 2 x 4096 tokens
    ("sana_x1", 4096, 2240, 1024, synth.BASE_NORMAL),        # SANA width, batch 4 x 1024 tokens
])
@pytest.mark.parametrize("variant", [0, 2], ids=["auto", "mfma_otf"])
def test_fused_full_workloads(name, T, d, tps, kind, variant):
    X, P, st, sc, sh = inputs(T, d, tps, seed={"flux_x1": 31, "pixart_x1": 32, "sana_x1": 33}[name], kind=kind)
    check(f"adaln {name} v{variant}", X, P, st, sc, sh, tps, variant)


@pytest.mark.parametrize("T,d,tps", [
    (4096, 2240, 32),    # 128 samples: every wave's run of units crosses many sample boundaries
    (2048, 3072, 96),    # 22 samples of 96 rows, the last one short
    (1536, 1152, 1504),  # two samples, the boundary inside a unit (36 blocks per row)
    (1000, 160, 64),     # 5 blocks per row (phases of 5 units; units span 12.8 rows)
])
def test_fused_sample_boundaries(T, d, tps):
    """Batches of several samples: the default kernel gives each wave a
    contiguous band of rows and loads the vectors of the band's first sample
    for the whole workgroup; lanes whose rows lie in a later sample load
    their own.  Every case against the oracle's producer step + quantizer."""
    X, P, st, sc, sh = inputs(T, d, tps, seed=T + d + tps)
    check(f"adaln {T}x{d} tps{tps} boundaries", X, P, st, sc, sh, tps, 3)


def test_modulation_vectors_at_an_offset():
    """Modulation vectors passed as views 16 bytes into larger buffers (the
    alignment the entry point requires) give the same bytes as contiguous ones;
    a view 4 bytes in is refused (KQ_ERR_ALIGN)."""
    T, d, tps = 128, 1152, 64
    X, P, st, sc, sh = inputs(T, d, tps, seed=77)
    codes, scales = run_fused(X, P, st, sc, sh, tps, kq.KQ_MFMA_OTF)
    big_sc = torch.zeros(sc.size + 4, dtype=torch.float32, device="cuda:0")
    big_sh = torch.zeros(sh.size + 4, dtype=torch.float32, device="cuda:0")
    big_sc[4:] = dev(sc).reshape(-1)
    big_sh[4:] = dev(sh).reshape(-1)
    Xd, std, Pd = dev(X), dev(st), dev(P)  # held for the duration of the calls
    c2, s2 = kq.alloc_outputs(Xd)
    L = kq.lib()
    stream = torch.cuda.current_stream().cuda_stream
    args = lambda off_sc, off_sh: (Xd.data_ptr(), T, d, std.data_ptr(), big_sc.data_ptr() + off_sc,
                                   big_sh.data_ptr() + off_sh, tps, Pd.data_ptr(), 15, None, kq.KQ_MFMA_OTF,
                                   c2.data_ptr(), s2.data_ptr(), stream)
    assert L.kq_quantize_adaln(*args(16, 16)) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(c2), codes)
    np.testing.assert_array_equal(host(s2), scales)
    assert L.kq_quantize_adaln(*args(12, 16)) == 3
    assert L.kq_quantize_adaln(*args(16, 4)) == 3


def test_fused_error_codes():
    X, P, st, sc, sh = inputs(100, 64, 64, seed=9)
    Xd = dev(X)
    codes, scales = kq.alloc_outputs(Xd)
    with pytest.raises(kq.KQError) as e:
        kq.kq_quantize_adaln(Xd, dev(st), dev(sc), dev(sh), 40, dev(P), codes, scales)
    assert e.value.status == 2
    with pytest.raises(kq.KQError) as e:  # the prebuilt-split variant without a split
        kq.kq_quantize_adaln(Xd, dev(st), dev(sc), dev(sh), 64, dev(P), codes, scales, 15, None, kq.KQ_MFMA_DENSE)
    assert e.value.status == 4


_CHILD = r"""
import sys
import numpy as np, torch
sys.path.insert(0, sys.argv[1])
import synth
import w4a4_diffusion_transformer_amd as kq
T, d = 96, 1152
X = torch.from_numpy(synth.random_matrix(T, d, seed=3, n_outliers=12, mult=50.0, token_sigma=0.5).view(np.int16)).cuda()
P = torch.from_numpy(synth.random_params(d // 32, seed=4)).cuda()
sc, sh = (torch.from_numpy(a).cuda() for a in synth.adaln_vectors(1, d, seed=5))
st = torch.empty((T, 2), dtype=torch.float32, device="cuda")
kq.kq_row_stats(X, 1e-6, st)
assert kq.kq_auto_variant(T, d, True, False) == kq.KQ_MFMA_OTF, "override not in effect"
auto = kq.kq_quantize_adaln(X, st, sc, sh, T, P, *kq.alloc_outputs(X))
otf = kq.kq_quantize_adaln(X, st, sc, sh, T, P, *kq.alloc_outputs(X), variant=kq.KQ_MFMA_OTF)
plain = kq.kq_quantize_ex(X, P, 15, None, kq.KQ_AUTO, *kq.alloc_outputs(X))
torch.cuda.synchronize()
assert all(torch.equal(a, b) for a, b in zip(auto, otf)), "AUTO under the mfma_otf override differs from mfma_otf"
assert not torch.equal(auto[0], plain[0]), "modulation not applied"
print("ok")
"""


def test_auto_follows_the_variant_override():
    """With KQ_VARIANT=mfma_otf (read once per process, hence a child
    process), KQ_AUTO resolves to mfma_otf for the fused AdaLN entry point as
    for the plain quantizer: the same bytes as an explicit mfma_otf call, and
    not the unmodulated quantization."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, KQ_VARIANT="mfma_otf")
    r = subprocess.run([sys.executable, "-c", _CHILD, root], env=env, capture_output=True, text=True, timeout=180)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]
