"""Offline calibration of KroQuant's transform on a synthetic linear layer, and the falsifier.

The method's offline half (Pith review, "What carries the argument" and the
ledger: the 15 scalars per 32-channel block are learned per layer by
minimising the quantized output error with auxiliary per-operand terms,
starting from the Hadamard transform, with Adam and a straight-through
estimator through the quantizer, 100 steps at learning rate 1e-2).  Readings
of what the pages leave open:

  * output term (Eqs. (2), (7), (9)): ||Q(X T) Q(W T^-T)^T - X W^T||^2 over
    ||X W^T||^2, with Q the MXFP4 quantize-dequantize along the channel axis;
  * auxiliary terms (Eq. (10)): lambda_A ||Q(X T) - X T||^2 / ||X||^2 and
    lambda_W ||Q(W T^-T) - W T^-T||^2 / ||W||^2, the lambdas set so that each
    auxiliary term equals the output term at the initialization;
  * straight-through estimator: Q's Jacobian taken as the identity;
  * initialization: the determinant-+1 Hadamard-like factors l = 1,
    a = 1/sqrt(2), b = -1/sqrt(2) (every block's transform is then a signed,
    orthonormal 32-point Hadamard matrix).

Training runs on PyTorch autograd in fp32 (this is not the online path);
evaluation of a parameter set on the real W4A4 path uses the library's
kernels (kq_quantize, the weight fold, kq_gemm_mx) when a GPU is present.

The falsifier (Pith review, "What would settle it"): activations with two
large outlier channels more than 32 indices apart, so that no 32 x 32 block
can mix them, and a random channel permutation of a learned transform.
"""
from __future__ import annotations

import json
import math

import torch

E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
SQ = 1.0 / math.sqrt(2.0)


# ---------------------------------------------------------------- transform

def factors(theta: torch.Tensor) -> torch.Tensor:
    """(l, a, b) [nb, 5, 3] -> G [nb, 5, 2, 2] = [[a, b], [l a, l b + 1/a]]."""
    l, a, b = theta[..., 0], theta[..., 1], theta[..., 2]
    top = torch.stack([a, b], dim=-1)
    bottom = torch.stack([l * a, l * b + 1.0 / a], dim=-1)
    return torch.stack([top, bottom], dim=-2)


def inverse_transpose(G: torch.Tensor) -> torch.Tensor:
    """G^-T of unit-determinant 2x2 factors: [[g11, -g10], [-g01, g00]]."""
    g00, g01, g10, g11 = G[..., 0, 0], G[..., 0, 1], G[..., 1, 0], G[..., 1, 1]
    return torch.stack([torch.stack([g11, -g10], -1), torch.stack([-g01, g00], -1)], -2)


def kron_blocks(G: torch.Tensor) -> torch.Tensor:
    """[nb, 5, 2, 2] -> [nb, 32, 32]: G1 (x) G2 (x) ... (x) G5, G1 on the most significant index bit."""
    K = G[:, 0]
    for k in range(1, G.shape[1]):
        n = K.shape[-1]
        K = torch.einsum("nab,ncd->nacbd", K, G[:, k]).reshape(G.shape[0], 2 * n, 2 * n)
    return K


def apply_blocks(X: torch.Tensor, K: torch.Tensor) -> torch.Tensor:
    """Row vectors times the block-diagonal matrix: X [T, d] -> X blockdiag(K) (row-vector convention of Eq. (1))."""
    T, d = X.shape
    nb = K.shape[0]
    return torch.einsum("tnr,nrc->tnc", X.reshape(T, nb, 32), K).reshape(T, d)


def hadamard_init(nb: int, device=None) -> torch.Tensor:
    theta = torch.empty((nb, 5, 3), dtype=torch.float32, device=device)
    theta[..., 0], theta[..., 1], theta[..., 2] = 1.0, SQ, -SQ
    return theta


def identity_params(nb: int, device=None) -> torch.Tensor:
    theta = torch.zeros((nb, 5, 3), dtype=torch.float32, device=device)
    theta[..., 1] = 1.0
    return theta


# ---------------------------------------------------------------- MXFP4 fake quantization

def mx_fake_quant(Y: torch.Tensor) -> torch.Tensor:
    """MXFP4 quantize-dequantize along the last axis in blocks of 32 (OCP MX v1.0 rules as the library
    applies them: scale 2^(floor(log2 amax) - 2) with the exponent field clamped at 0, E2M1 round to
    nearest with ties to the even code, saturation at 6, amax 0 -> zeros)."""
    shape = Y.shape
    Yb = Y.reshape(-1, 32)
    amax = Yb.abs().amax(dim=1, keepdim=True)
    exp_field = torch.where(amax > 0, torch.frexp(amax.float()).exponent - 1 + 127, torch.zeros_like(amax, dtype=torch.int32))
    byte = torch.clamp(exp_field - 2, min=0)
    scale = torch.ldexp(torch.ones_like(amax), (byte - 127).to(torch.int32))
    m = (Yb / scale).abs()
    idx = ((m > 0.25).int() + (m >= 0.75).int() + (m > 1.25).int() + (m >= 1.75).int() + (m > 2.5).int()
           + (m >= 3.5).int() + (m > 5.0).int())
    grid = torch.tensor(E2M1, dtype=Yb.dtype, device=Yb.device)
    q = grid[idx] * torch.sign(Yb) * scale
    q = torch.where(amax > 0, q, torch.zeros_like(q))
    return q.reshape(shape)


def ste(Y: torch.Tensor) -> torch.Tensor:
    """Straight-through estimator: forward Q(Y), backward identity."""
    return Y + (mx_fake_quant(Y) - Y).detach()


# ---------------------------------------------------------------- objective and training

def losses(theta: torch.Tensor, X: torch.Tensor, W: torch.Tensor, quantize: bool = True):
    """(output term, activation term, weight term) of the objective for parameters theta."""
    G = factors(theta)
    K = kron_blocks(G)
    Kit = kron_blocks(inverse_transpose(G))
    Xt = apply_blocks(X, K)
    Wt = apply_blocks(W, Kit)
    Xq = ste(Xt) if quantize else Xt
    Wq = ste(Wt) if quantize else Wt
    ref = X @ W.T
    out = ((Xq @ Wq.T - ref) ** 2).sum() / (ref ** 2).sum()
    la = ((Xq - Xt) ** 2).sum() / (X ** 2).sum()
    lw = ((Wq - Wt) ** 2).sum() / (W ** 2).sum()
    return out, la, lw


def calibrate(X: torch.Tensor, W: torch.Tensor, theta0: torch.Tensor | None = None, steps: int = 100,
              lr: float = 1e-2, regularize: bool = True):
    """Adam on the objective from theta0 (Hadamard-like by default); returns (theta, history of output terms)."""
    nb = X.shape[1] // 32
    theta = (hadamard_init(nb, X.device) if theta0 is None else theta0.clone()).requires_grad_(True)
    with torch.no_grad():
        o0, a0, w0 = losses(theta, X, W)
        lam_a = float(o0 / a0) if a0 > 0 else 0.0
        lam_w = float(o0 / w0) if w0 > 0 else 0.0
    if not regularize:
        lam_a = lam_w = 0.0
    opt = torch.optim.Adam([theta], lr=lr)
    hist = []
    for _ in range(steps):
        opt.zero_grad(set_to_none=True)
        out, la, lw = losses(theta, X, W)
        loss = out + lam_a * la + lam_w * lw
        loss.backward()
        opt.step()
        hist.append(float(out.detach()))
    with torch.no_grad():
        hist.append(float(losses(theta, X, W)[0]))
    return theta.detach(), hist


# ---------------------------------------------------------------- baselines and evaluation

def output_error(Xq: torch.Tensor, Wq: torch.Tensor, X: torch.Tensor, W: torch.Tensor) -> float:
    ref = X @ W.T
    return float(((Xq @ Wq.T - ref) ** 2).sum() / (ref ** 2).sum())


def error_plain(X, W) -> float:
    return output_error(mx_fake_quant(X), mx_fake_quant(W), X, W)


def error_smooth(X, W, alpha: float = 0.5) -> float:
    """Per-channel scaling (SmoothQuant, s_c = max|X_c|^alpha / max|W_c|^(1-alpha)) then MXFP4."""
    s = X.abs().amax(0).clamp_min(1e-8) ** alpha / W.abs().amax(0).clamp_min(1e-8) ** (1 - alpha)
    return output_error(mx_fake_quant(X / s), mx_fake_quant(W * s), X, W)


def error_kroquant(theta, X, W) -> float:
    with torch.no_grad():
        return float(losses(theta, X, W)[0])


def error_kroquant_permuted(theta, X, W, seed: int = 0) -> float:
    """The learned block transform applied to a random channel permutation of the layer: the transform
    no longer meets the channels (and outliers) it was learned on."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(X.shape[1], generator=g).to(X.device)
    return error_kroquant(theta, X[:, perm], W[:, perm])


def error_on_gpu_path(theta: torch.Tensor, X: torch.Tensor, W: torch.Tensor) -> float:
    """The same output error through the library's W4A4 kernels: kq_quantize(X, theta), the folded weight
    (kq_build_blocks_inverse_t + dense kq_quantize_ex) and kq_gemm_mx.  X, W are rounded to bf16 first."""
    import w4a4_diffusion_transformer_amd as kq

    dev = torch.device("cuda:0")
    Xb = X.to(dev, torch.bfloat16).contiguous()
    Wb = W.to(dev, torch.bfloat16).contiguous()
    P = theta.to(dev, torch.float32).contiguous()
    nb = P.shape[0]
    xc, xs = kq.alloc_outputs(Xb)
    kq.kq_quantize(Xb.view(torch.int16), P, xc, xs)
    Kit = torch.empty((nb, 3, 32, 32), dtype=torch.int16, device=dev)
    kq.kq_build_blocks_inverse_t(P, nb, None, Kit, 3)
    wc, ws = kq.alloc_outputs(Wb)
    kq.kq_quantize_ex(Wb.view(torch.int16), None, 15, Kit, kq.KQ_MFMA_DENSE, wc, ws)
    Y = torch.empty((X.shape[0], W.shape[0]), dtype=torch.float32, device=dev)
    kq.kq_gemm_mx(xc, xs, wc, ws, Y)
    torch.cuda.synchronize()
    ref = Xb.double() @ Wb.double().T
    return float(((Y.double() - ref) ** 2).sum() / (ref ** 2).sum())


# ---------------------------------------------------------------- synthetic layers

def synthetic_layer(T: int, d: int, n_out: int, outliers, mult: float, seed: int, device=None):
    """X [T, d]: N(0,1) with the given outlier channels multiplied by `mult` and a per-token scale
    (1 + N(0, 0.5)); W [n_out, d]: N(0, 1/d).  Both rounded to bf16 values (the layer's precision)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    X = torch.randn((T, d), generator=g)
    X[:, list(outliers)] *= mult
    X *= (1.0 + 0.5 * torch.randn((T, 1), generator=g))
    W = torch.randn((n_out, d), generator=g) / math.sqrt(d)
    X = X.to(torch.bfloat16).float()
    W = W.to(torch.bfloat16).float()
    return X.to(device), W.to(device)


def experiment(T: int = 1024, d: int = 1152, n_out: int = 1152, steps: int = 100, device=None, use_gpu_path=None):
    """Calibration on two synthetic layers and the falsifier; returns a dict of relative output errors
    ||Y_q - X W^T||^2 / ||X W^T||^2, measured on tokens held out from calibration."""
    res = {}
    cases = {
        # outliers inside one 32-channel block (channels 5 and 20): a block transform can mix them
        "outliers_same_block": (5, 20),
        # outliers more than 32 channels apart (5 and 70, blocks 0 and 2): no block can mix them
        "outliers_far_apart": (5, 70),
    }
    seeds = {"outliers_same_block": 11, "outliers_far_apart": 12}
    for name, outl in cases.items():
        # 2T tokens of one layer: the first T calibrate, the other T are held out for every error below
        X2, W = synthetic_layer(2 * T, d, n_out, outl, 50.0, seed=seeds[name], device=device)
        Xc, X = X2[:T].contiguous(), X2[T:].contiguous()
        nb = d // 32
        theta, hist = calibrate(Xc, W, steps=steps)
        r = {
            "plain_mx": error_plain(X, W),
            "smoothquant_mx": error_smooth(X, W),
            "hadamard_init": error_kroquant(hadamard_init(nb, X.device), X, W),
            "kroquant_learned": error_kroquant(theta, X, W),
            "kroquant_learned_channel_permuted": error_kroquant_permuted(theta, X, W),
            "objective_first_last_calibration_tokens": [hist[0], hist[-1]],
        }
        if use_gpu_path:
            r["kroquant_learned_on_gpu_kernels"] = error_on_gpu_path(theta, X, W)
        res[name] = r
    return res


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser(description="KroQuant calibration on synthetic layers and the falsifier")
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--tokens", type=int, default=1024)
    ap.add_argument("--d", type=int, default=1152)
    args = ap.parse_args()
    gpu = torch.cuda.is_available()
    out = experiment(args.tokens, args.d, args.d, args.steps, device="cuda:0" if gpu else "cpu", use_gpu_path=gpu)
    print(json.dumps(out, indent=1))
