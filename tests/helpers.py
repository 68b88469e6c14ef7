"""Shared helpers for the parity tests: conversions and the GEMM tolerance,
checked on whole outputs.

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
    """2^(floor(log2 |y|) - 7) for |y| >= 2^-126, else 2^-133.  frexp gives
    |y| = m 2^e with m in [0.5, 1), so floor(log2 |y|) = e - 1 exactly."""
    a = np.abs(y)
    _, e = np.frexp(np.maximum(a, 2.0 ** -126))
    return np.where(a >= 2.0 ** -126, np.ldexp(1.0, e - 8), 2.0 ** -133)


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


def rms_of(ref: np.ndarray) -> float:
    """Root mean square of a whole fp64 array (one BLAS dot, no temporary)."""
    flat = ref.reshape(-1)
    return float(np.sqrt(np.dot(flat, flat) / flat.size)) if flat.size else 0.0


def gemm_check_dev(got_dev: torch.Tensor, ref: np.ndarray, what: str = "", chunk_rows: int = 4096) -> float:
    """gemm_check of a whole device output against the whole fp64 reference,
    copied to the host and compared in blocks of rows (every element is
    checked; rms is taken over the whole reference)."""
    assert tuple(got_dev.shape) == ref.shape, (what, tuple(got_dev.shape), ref.shape)
    rms = rms_of(ref)
    worst = 0.0
    for r0 in range(0, ref.shape[0], chunk_rows):
        r1 = min(ref.shape[0], r0 + chunk_rows)
        worst = max(worst, gemm_check(bf16_to_f64(got_dev[r0:r1]), ref[r0:r1], rms=rms, what=f"{what} rows {r0}:{r1}"))
    return worst
