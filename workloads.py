"""Seeded synthetic inputs for the HiF4 hot path (shared by tests and bench).

This module draws random numbers and nothing else: it holds none of the
method's arithmetic. Both the HIP path and the oracle read the SAME bf16 bytes
that these functions return (generate once, copy), so no cross-device RNG
agreement is needed. Values are drawn in float32 and rounded to bf16 (RNE).

Shapes follow the Wan2.2 setting of the Tail-Aware HiFloat4 report
(agents-report.net, section "實驗設計與結果摘要": 720x1280, 61 frames ->
57,600 latent tokens; hidden 5120, FFN 13824). The pages' own data (video
activations, calibration prompts) is not available; these draws stand in.

Workloads (seed = workload index unless given):
  tiny      X 64x256 ~N(0,1), 1% of entries x30; W 128x256 ~0.02 N(0,1);
            percentile q=0.99 over 64 rows, 13 protected channels.
  attn      X 8192x5120 = Student-t(3) * c[ch], c ~ LogNormal(0,1), 0.1% of
            channels (5) x50; W 5120x5120 ~0.02 N(0,1).
  ffn_up    as attn with M=57600, N=13824, K=5120.
  ffn_down  X 57600x13824 = GELU_erf(1.5 N(0,1)); W 5120x13824 ~0.015 N(0,1).
  calib     16 batches of 57600x5120: Student-t(2.5) * c[ch] * d_b[ch],
            c ~ LogNormal(0,1), d_b ~ LogNormal(0,0.5); q=0.999, 52 protected;
            W 13824x5120 ~0.02 N(0,1) quantized with that mask.
  higptq    W 13824x5120 ~0.02 N(0,1) and the upper factor U of an inverse
            Hessian (H^-1 = U^T U): for the tests, U drawn directly
            (higptq_factor: any upper-triangular U with a positive diagonal is
            one); for the bench, GPTQ's H = 2 X^T X / rows (+1% dampening) of
            the FFN-up X (higptq_factor_from_x), and of that X mixed across
            channels by I + 0.8 A / sqrt(k), A ~ N(0,1) (the FFN-up recipe's
            channels are independent, its H nearly diagonal).
"""
import math

import torch

WORKLOADS = {
    "tiny": dict(index=0, M=64, N=128, K=256, q=0.99, n_protect=13),
    "attn": dict(index=1, M=8192, N=5120, K=5120),
    "ffn_up": dict(index=2, M=57600, N=13824, K=5120, q=0.999, n_protect=52),
    "ffn_down": dict(index=3, M=57600, N=5120, K=13824),
    "calib": dict(index=4, rows_per_batch=57600, batches=16, C=5120, N=13824,
                  q=0.999, n_protect=52),
    "higptq": dict(index=5, N=13824, K=5120),
}


def n_protect_for(fraction: float, channels: int) -> int:
    """Protected-channel count for a top-`fraction` mask: ceil(p * C)."""
    return int(math.ceil(fraction * channels - 1e-9))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _student_t(shape, nu, g, device):
    # t = Z / sqrt(V / nu), V ~ chi2(nu) = 2 Gamma(nu / 2)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    alpha = torch.full(shape, nu / 2.0, device=device, dtype=torch.float32)
    v = 2.0 * torch._standard_gamma(alpha, generator=g)
    del alpha
    return z / torch.sqrt(v / nu)


def _lognormal(shape, sigma, g, device):
    return torch.exp(sigma * torch.randn(shape, generator=g, device=device, dtype=torch.float32))


def normal_bf16(rows, cols, std, device="cpu", seed=0):
    """std * N(0,1) [rows][cols] as bf16."""
    g = _gen(device, seed)
    return (std * torch.randn((rows, cols), generator=g, device=device)).to(torch.bfloat16)


def tiny_x(rows=64, cols=256, device="cpu", seed=0, outlier_p=0.01, outlier_scale=30.0):
    """N(0,1) with a fraction of entries multiplied by outlier_scale."""
    g = _gen(device, seed)
    x = torch.randn((rows, cols), generator=g, device=device)
    o = torch.rand((rows, cols), generator=g, device=device) < outlier_p
    x[o] *= outlier_scale
    return x.to(torch.bfloat16)


def heavy_tailed_x(rows, cols, device="cpu", seed=1, nu=3.0, outlier_channels=None,
                   outlier_scale=50.0, chunk_rows=8192):
    """Student-t(nu) values times a LogNormal(0,1) per-channel scale; a set of
    channels (default round(0.001 * cols)) carries an extra outlier factor."""
    g = _gen(device, seed)
    c = _lognormal((cols,), 1.0, g, device)
    n_out = round(0.001 * cols) if outlier_channels is None else outlier_channels
    if n_out > 0:
        out = torch.randperm(cols, generator=g, device=device)[:n_out]
        c[out] *= outlier_scale
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x[r0:r1] = (_student_t((r1 - r0, cols), nu, g, device) * c).to(torch.bfloat16)
    return x


def gelu_x(rows, cols, device="cpu", seed=3, std=1.5, chunk_rows=4096):
    """GELU (exact erf form) of std * N(0,1): non-negative-skewed, long right tail."""
    g = _gen(device, seed)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        z = std * torch.randn((r1 - r0, cols), generator=g, device=device)
        x[r0:r1] = torch.nn.functional.gelu(z, approximate="none").to(torch.bfloat16)
    return x


def calib_x(batches, rows_per_batch, cols, device="cpu", seed=4, nu=2.5, chunk_rows=8192,
            out=None):
    """Stacked calibration activations [batches * rows_per_batch][cols]:
    Student-t(nu) * c[ch] * d_b[ch] with c ~ LogNormal(0,1) shared and a
    per-batch drift d_b ~ LogNormal(0,0.5)."""
    g = _gen(device, seed)
    c = _lognormal((cols,), 1.0, g, device)
    x = out if out is not None else torch.empty((batches * rows_per_batch, cols),
                                                dtype=torch.bfloat16, device=device)
    for b in range(batches):
        d = _lognormal((cols,), 0.5, g, device)
        scale = c * d
        base = b * rows_per_batch
        for r0 in range(0, rows_per_batch, chunk_rows):
            r1 = min(rows_per_batch, r0 + chunk_rows)
            x[base + r0:base + r1] = (_student_t((r1 - r0, cols), nu, g, device)
                                      * scale).to(torch.bfloat16)
    return x


def workload(name, device="cpu", seed=None):
    """Inputs of a named workload as a dict of bf16 tensors (+ scalars)."""
    w = WORKLOADS[name]
    s = w["index"] if seed is None else seed
    if name == "tiny":
        return dict(x=tiny_x(w["M"], w["K"], device, s),
                    w=normal_bf16(w["N"], w["K"], 0.02, device, s + 1000),
                    q=w["q"], n_protect=w["n_protect"])
    if name in ("attn", "ffn_up"):
        d = dict(x=heavy_tailed_x(w["M"], w["K"], device, s),
                 w=normal_bf16(w["N"], w["K"], 0.02, device, s + 1000))
        if "q" in w:
            d.update(q=w["q"], n_protect=w["n_protect"])
        return d
    if name == "ffn_down":
        return dict(x=gelu_x(w["M"], w["K"], device, s),
                    w=normal_bf16(w["N"], w["K"], 0.015, device, s + 1000))
    if name == "calib":
        return dict(x=calib_x(w["batches"], w["rows_per_batch"], w["C"], device, s),
                    w=normal_bf16(w["N"], w["C"], 0.02, device, s + 1000),
                    q=w["q"], n_protect=w["n_protect"])
    raise KeyError(name)


def bits(t: torch.Tensor):
    """uint16 numpy view of a bf16 tensor's bit patterns (host copy)."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def higptq_factor_from_x(x, damp=0.01):
    """Upper factor U (fp32 [k][k]) of H^-1 = U^T U for the Hessian GPTQ takes
    from calibration activations x [rows][k] (the layer's inputs): H =
    2 x^T x / rows, with damp * mean(diag H) added to the diagonal (GPTQ's
    dampening), on x's device; the inverse and factors in fp64."""
    xf = x.float()
    h = (xf.T @ xf).double() * (2.0 / x.shape[0])
    h.diagonal().add_(damp * h.diagonal().mean())
    hinv = torch.cholesky_inverse(torch.linalg.cholesky(h))
    return torch.linalg.cholesky(hinv, upper=True).float().contiguous(), h.float()


def higptq_factor(k, device="cpu", seed=5, spread=0.5, coupling=1.0):
    """Random upper-triangular U [k][k] (fp32) with a positive diagonal: the
    factor of a synthetic inverse Hessian H^-1 = U^T U. Row i is scaled by
    d_i ~ LogNormal(0, spread) (channel scales); the entries above the diagonal
    are d_i * coupling * N(0,1) / sqrt(k) (channel correlations)."""
    g = _gen(device, seed)
    d = _lognormal((k, 1), spread, g, device)
    z = torch.randn((k, k), generator=g, device=device, dtype=torch.float32) * (coupling / math.sqrt(k))
    u = torch.triu(z, diagonal=1) + torch.eye(k, device=device, dtype=torch.float32)
    return (u * d).contiguous()
