"""Shared helpers for the parity tests: conversions, the GEMM tolerance and
sampled references.

GEMM tolerance (per element): |gpu - ref| <= 1e-2 * rms(ref) + ulp_bf16(|ref|),
with ulp_bf16(y) = 2^(floor(log2 y) - 7) for y >= 2^-126 and 2^-133 below;
the oracle reference accumulates exact dequantised fp8 products in fp64.
"""
import numpy as np
import torch

import oracle


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (any device)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().float().numpy().astype(np.float64)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def f32_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


def np_f32_bits(x) -> np.uint32:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def bf16_ulp(y: np.ndarray) -> np.ndarray:
    a = np.abs(y)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def gemm_check(got: np.ndarray, ref: np.ndarray, rms: float = None, what: str = ""):
    """Asserts the GEMM tolerance; rms defaults to the rms of `ref`."""
    if rms is None:
        rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    tol = 1e-2 * rms + bf16_ulp(ref)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; first {idx.tolist()} "
                             f"got {got[tuple(idx[0])]} ref {ref[tuple(idx[0])]} rms {rms}")
    return float(err.max() / max(rms, 1e-300)) if err.size else 0.0


def sample_rows(n: int, k: int, seed: int) -> np.ndarray:
    """k distinct row indices in [0, n) that always include the first and the
    last 16 (the edge tiles) plus a seeded random spread."""
    if n <= k:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    edge = np.concatenate([np.arange(min(16, n)), np.arange(max(0, n - 16), n)])
    rest = rng.choice(n, size=k, replace=False)
    return np.unique(np.concatenate([edge, rest]))


def forward_rows(x8, w8, sx, sw, rows):
    """Rows `rows` of the oracle's Y (same definition, on a row subset)."""
    return oracle.forward_ref(x8[rows], w8, sx, sw)


def dgrad_rows(dy8, w8, sdy, sw, rows):
    return oracle.dgrad_ref(dy8[rows], w8, sdy, sw)


def wgrad_rows(dy8, x8, sdy, sx, rows):
    """Rows `rows` of the oracle's dW = dY8^T X8 (rows index N)."""
    return oracle.wgrad_ref(np.ascontiguousarray(dy8[:, rows]), x8, sdy, sx)
