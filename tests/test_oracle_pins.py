"""Pins the CPU oracle to things other than itself.

Each test checks one oracle function against what the format definitions and
mathematics fix: closed-form values of the OCP 8-bit formats (golden table),
brute-force nearest-value search over the decoded grid, exact rational
arithmetic, torch's own float8 conversions (a library implementation), and
invariants (half-ulp error, monotonicity, sign symmetry, transposition).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2, FMAX

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMT_NAMES = {"e4m3": E4M3, "e5m2": E5M2}
TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
MBITS = {E4M3: 3, E5M2: 2}
EMIN = {E4M3: -6, E5M2: -14}


def _f32_from_bits(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def _torch_encode(v32: np.ndarray, fmt: int) -> np.ndarray:
    """torch's fp32 -> float8 conversion (round-to-nearest-even, not
    saturating) after clamping to +-fmax, as uint8 codes."""
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    t = torch.clamp(t, -FMAX[fmt], FMAX[fmt])
    return t.to(TORCH_DT[fmt]).view(torch.uint8).numpy()


def _finite_positive_codes(fmt):
    return [c for c in range(0x80) if math.isfinite(oracle.fp8_decode_scalar(c, fmt))]


# ------------------------------------------------------------------ decode

def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "ofp8_format_table.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            fmt, code, val = line.split()
            rows.append((FMT_NAMES[fmt], int(code, 16), val))
    return rows


@pytest.mark.parametrize("fmt,code,val", _golden_rows())
def test_decode_matches_ofp8_table(fmt, code, val):
    got = oracle.fp8_decode_scalar(code, fmt)
    if val == "nan":
        assert math.isnan(got)
    elif val in ("inf", "-inf"):
        assert got == float(val)
    else:
        want = float.fromhex(val)
        assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_matches_torch_float8(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()
    got = oracle.decode_table(fmt)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_grid_structure(fmt):
    pos = _finite_positive_codes(fmt)
    vals = [oracle.fp8_decode_scalar(c, fmt) for c in pos]
    # positive codes enumerate the grid in increasing order, with no gaps
    assert pos == list(range(len(pos)))
    assert all(b > a for a, b in zip(vals, vals[1:]))
    # 254 finite e4m3 values (2 NaN codes); 248 finite e5m2 values (2 Inf + 6 NaN)
    assert 2 * len(pos) == (254 if fmt == E4M3 else 248)
    for c in pos:  # sign-magnitude
        assert oracle.fp8_decode_scalar(c | 0x80, fmt) == -oracle.fp8_decode_scalar(c, fmt)
    # subnormal spacing is uniform and equals the min-normal binade's spacing
    q = 2.0 ** (EMIN[fmt] - MBITS[fmt])
    for c in range(1 << MBITS[fmt]):
        assert oracle.fp8_decode_scalar(c, fmt) == c * q


# ------------------------------------------------------------------ encode

def _brute_encode(v: float, fmt: int) -> int:
    """Nearest code by linear scan of the decoded positive grid, exact
    (rational) distances, ties to the code with an even mantissa LSB,
    after saturating |v| to fmax; the sign bit is copied from v."""
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    if math.isnan(v):
        return sign | 0x7F
    a = Fraction(min(abs(v), FMAX[fmt])) if math.isfinite(v) else Fraction(FMAX[fmt])
    best = None
    for c in _finite_positive_codes(fmt):
        d = abs(Fraction(oracle.fp8_decode_scalar(c, fmt)) - a)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return sign | best[1]


def _probe_values(fmt):
    """Every grid point, every midpoint between neighbours, the fp32 values
    one ulp either side of each, and values beyond the largest finite value."""
    pos = _finite_positive_codes(fmt)
    grid = [np.float32(oracle.fp8_decode_scalar(c, fmt)) for c in pos]
    vals = set()
    for g in grid:
        vals.add(float(g))
    for a, b in zip(grid, grid[1:]):
        mid = np.float32((np.float64(a) + np.float64(b)) / 2)  # exact: <= 5 significant bits
        vals.update([float(mid), float(np.nextafter(mid, np.float32(0))), float(np.nextafter(mid, np.float32(1e9)))])
    top = np.float32(FMAX[fmt])
    step = float(top) - float(grid[-2])
    vals.update([float(top) + step / 2, float(top) + step / 2 - 1.0, float(top) + step, float(top) * 4, 1e30,
                 float("inf"), 2.0 ** (EMIN[fmt] - MBITS[fmt] - 1), 2.0 ** (EMIN[fmt] - MBITS[fmt] - 2), 1e-40,
                 float(np.nextafter(np.float32(2.0 ** (EMIN[fmt] - MBITS[fmt] - 1)), np.float32(1)))])
    out = sorted(vals)
    return out + [-v for v in out]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_matches_brute_force_scan(fmt):
    for v in _probe_values(fmt):
        assert oracle.fp8_encode_scalar(v, fmt) == _brute_encode(v, fmt), (fmt, v)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_known_roundings(fmt):
    # ties to even inside a binade, at the subnormal/zero boundary and at the top
    if fmt == E4M3:
        cases = [(1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01), (248.0, 0x78),
                 (464.0, 0x7E), (470.0, 0x7E), (1e9, 0x7E), (float("inf"), 0x7E), (-float("inf"), 0xFE),
                 (0.0, 0x00), (-0.0, 0x80), (-1e-40, 0x80), (7.5 * 2.0 ** -9, 0x08)]
    else:
        cases = [(1.125, 0x3C), (1.375, 0x3E), (2.0 ** -17, 0x00), (1.5 * 2.0 ** -17, 0x01), (61440.0, 0x7B),
                 (1e9, 0x7B), (float("inf"), 0x7B), (-float("inf"), 0xFB), (0.0, 0x00), (-0.0, 0x80)]
    for v, code in cases:
        assert oracle.fp8_encode_scalar(v, fmt) == code, (fmt, v)
    assert oracle.decode_table(fmt)[oracle.fp8_encode_scalar(float("nan"), fmt)] != \
        oracle.decode_table(fmt)[oracle.fp8_encode_scalar(float("nan"), fmt)]  # a NaN code


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_matches_torch_on_random_bit_patterns(fmt):
    rng = np.random.default_rng(1234 + fmt)
    bits = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    v = _f32_from_bits(bits)
    v = v[~np.isnan(v)]
    assert np.array_equal(oracle.encode_f32(v, fmt), _torch_encode(v, fmt))


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_exhaustive_nonnegative_binary32(fmt):
    """Every non-negative binary32 bit pattern up to twice the format's max
    (all larger finite values and +Inf saturate, checked on samples above)
    against torch's conversion after the clamp."""
    hi = int(np.float32(2 * FMAX[fmt]).view(np.uint32))
    chunk = 1 << 25
    for lo in range(0, hi, chunk):
        n = min(chunk, hi - lo)
        got = oracle.encode_bits_range(lo, n, fmt)
        v = _f32_from_bits(np.arange(lo, lo + n, dtype=np.uint32))
        ref = _torch_encode(v, fmt)
        if not np.array_equal(got, ref):
            bad = np.nonzero(got != ref)[0][:5]
            raise AssertionError(f"fmt {fmt}: mismatch at bit patterns {[hex(lo + int(b)) for b in bad]}")


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_sign_symmetry_and_monotonic(fmt):
    rng = np.random.default_rng(7)
    v = np.sort(rng.uniform(-2 * FMAX[fmt], 2 * FMAX[fmt], 200000).astype(np.float32))
    v = np.concatenate([v, np.float32(2.0) ** rng.uniform(-30, 8, 200000).astype(np.float32)])
    v = np.sort(v)
    q = oracle.encode_f32(v, fmt)
    qn = oracle.encode_f32(-v, fmt)
    assert np.array_equal(qn, q ^ 0x80)
    d = oracle.decode(q, fmt)
    assert np.all(np.diff(d) >= 0)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_half_ulp_bound(fmt):
    """For |v| <= fmax: |decode(encode(v)) - v| <= half the grid spacing at v's binade."""
    rng = np.random.default_rng(11)
    v = (np.float32(2.0) ** rng.uniform(-20, math.log2(FMAX[fmt]), 500000)).astype(np.float32)
    v = v[v <= FMAX[fmt]]
    q = oracle.encode_f32(v, fmt)
    err = np.abs(oracle.decode(q, fmt) - v.astype(np.float64))
    e = np.maximum(np.floor(np.log2(v.astype(np.float64))), EMIN[fmt])
    half_ulp = 2.0 ** (e - MBITS[fmt] - 1)
    assert np.all(err <= half_ulp)


# -------------------------------------------------------------------- amax

def test_amax_every_single_bf16_value():
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = _bf16_to_f32(bits)
    one = np.zeros(1, dtype=np.uint16)
    for b in range(1 << 16):
        one[0] = b
        got = oracle.amax(one)
        want = abs(vals[b])
        if np.isnan(want):
            assert np.isnan(got)
        else:
            assert got == want and not np.signbit(got), hex(b)


def test_amax_invariants():
    rng = np.random.default_rng(3)
    x = rng.integers(0, 1 << 16, size=1_000_003, dtype=np.uint32).astype(np.uint16)
    finite = x[~np.isnan(_bf16_to_f32(x))]
    want = np.max(np.abs(_bf16_to_f32(finite).astype(np.float64)))
    assert float(oracle.amax(finite)) == want
    assert np.isnan(oracle.amax(x))  # the random draw holds NaN patterns
    assert oracle.amax(np.zeros(0, dtype=np.uint16)) == 0.0
    # the maximum at the first and at the last position, negative values only
    y = np.full(4097, 0xBF80, dtype=np.uint16)  # -1.0
    y[-1] = 0xC040  # -3.0
    assert oracle.amax(y) == 3.0
    y[-1] = 0xBF80
    y[0] = 0xC000  # -2.0
    assert oracle.amax(y) == 2.0
    # bf16 subnormals are kept
    assert oracle.amax(np.array([0x0001, 0x8003], dtype=np.uint16)) == _bf16_to_f32([0x0003])[0]


# ------------------------------------------------------------------- scale

@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_scale_exhaustive_over_bf16_magnitudes(fmt):
    """s = fl32(fmax / max(a, eps)): a quotient of two binary32 values
    rounded once from fp64 (53 >= 2*24 + 2 bits) is the correctly rounded
    binary32 quotient, so fp64-then-round is an independent reference."""
    bits = np.arange(0, 0x7F81, dtype=np.uint32)  # +0 .. +Inf
    mags = _bf16_to_f32(bits)
    eps = np.float64(np.float32(1e-12))
    for a in mags.tolist() + [1e-30, float(np.float32(1e-12))]:
        s, inv = oracle.scale(a, fmt)
        d = max(np.float64(a), eps)
        assert s == np.float32(np.float64(FMAX[fmt]) / d), a
        if s != 0.0:
            assert inv == np.float32(1.0 / np.float64(s)), a
    s, _ = oracle.scale(0.0, fmt)
    assert s == np.float32(FMAX[fmt] / np.float64(np.float32(1e-12)))
    s, _ = oracle.scale(FMAX[fmt], fmt)
    assert s == 1.0
    s, inv = oracle.scale(float("nan"), fmt)
    assert np.isnan(s) and np.isnan(inv)


# -------------------------------------------------------------------- cast

def test_cast_transposed_copy_and_torch_cross_check():
    rng = np.random.default_rng(5)
    for fmt, (rows, cols) in [(E4M3, (48, 80)), (E5M2, (80, 48)), (E4M3, (1, 16)), (E5M2, (16, 1))]:
        x = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32) * 3).to(torch.bfloat16)
        xb = x.view(torch.int16).numpy().view(np.uint16)
        a = oracle.amax(xb)
        s, _ = oracle.scale(a, fmt)
        q, qt, nsat = oracle.cast(xb, fmt, s)
        assert np.array_equal(qt, q.T)
        # an independent cast: torch fp32 multiply, clamp, torch float8 conversion
        v = (x.float() * torch.tensor(float(s), dtype=torch.float32)).numpy()
        assert np.array_equal(q, _torch_encode(v, fmt))
        # only elements of magnitude amax can land above fmax (by at most one
        # binary32 rounding of the scale and one of the product)
        n_at_amax = int(np.sum(np.abs(x.float().numpy()) == float(a)))
        assert nsat <= n_at_amax


def test_cast_two_step_rounding_reading():
    """The product is rounded to binary32 first, then to fp8.  With amax
    0.1259765625 and x = bf16 0x3601 (about 1.92e-6) the two-step result is
    code 0x04 although the exact product would round to 0x03."""
    s, _ = oracle.scale(0.1259765625, E4M3)
    x = np.array([[0x3601]], dtype=np.uint16)
    q, _, _ = oracle.cast(x, E4M3, s)
    assert q[0, 0] == 0x04
    exact = Fraction(float(_bf16_to_f32([0x3601])[0])) * Fraction(float(s))
    assert _brute_encode_exact(exact, E4M3) == 0x03


def _brute_encode_exact(a: Fraction, fmt: int) -> int:
    best = None
    for c in _finite_positive_codes(fmt):
        key = (abs(Fraction(oracle.fp8_decode_scalar(c, fmt)) - a), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_cast_special_tensors(fmt):
    # a constant tensor maps to the largest code everywhere (sign kept)
    c = np.full((16, 32), 0x3FC0, dtype=np.uint16)  # 1.5
    c[3, 5] = 0xBFC0  # -1.5
    s, _ = oracle.scale(oracle.amax(c), fmt)
    q, _, nsat = oracle.cast(c, fmt, s)
    maxc = 0x7E if fmt == E4M3 else 0x7B
    assert np.all(q[c == 0x3FC0] == maxc) and q[3, 5] == (maxc | 0x80)
    # a tensor holding +-fmax (exact in bf16) gets scale 1: the cast is the
    # identity on values already on the fp8 grid
    codes = np.array(_finite_positive_codes(fmt), dtype=np.uint8)
    codes = np.concatenate([codes, codes | 0x80])
    vals = oracle.decode(codes, fmt).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(_bf16_to_f32(bits), vals)  # every fp8 value is a bf16 value
    s, _ = oracle.scale(oracle.amax(bits), fmt)
    assert s == 1.0
    q, _, _ = oracle.cast(bits.reshape(1, -1), fmt, s)
    assert np.array_equal(q.reshape(-1), codes)
    # a power-of-two scale makes every product exact: single rounding
    x = np.array([[0x4060, 0x3F81, 0x3A83, 0xB6F1] * 4], dtype=np.uint16)  # amax 3.5
    s, _ = oracle.scale(oracle.amax(x), E4M3)
    assert s == 128.0
    q, _, _ = oracle.cast(x, E4M3, s)
    for j in range(x.shape[1]):
        exact = Fraction(float(_bf16_to_f32([x[0, j]])[0])) * 128
        want = _brute_encode_exact(abs(exact), E4M3) | (0x80 if exact < 0 else 0)
        assert q[0, j] == want


def test_cast_saturation_count_is_brute_count():
    rng = np.random.default_rng(9)
    x = torch.from_numpy(rng.standard_normal((64, 64)).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    s, _ = oracle.scale(0.5, E4M3)  # a stale (too small) amax: many products saturate
    _, _, nsat = oracle.cast(xb, E4M3, s)
    v = x.float().numpy() * np.float32(s)
    assert nsat == int(np.sum(np.abs(v) > 448.0)) and nsat > 0


# ------------------------------------------------------------------- GEMMs

def _exact_matmul(a_vals, b_vals, transpose_b):
    """Triple loop over Fractions, written from the index definition."""
    m = len(a_vals)
    kk = len(a_vals[0])
    n = len(b_vals) if transpose_b else len(b_vals[0])
    out = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for k in range(kk):
                bv = b_vals[j][k] if transpose_b else b_vals[k][j]
                acc += a_vals[i][k] * bv
            out[i][j] = acc
    return out


def _codes(rng, shape, fmt):
    pos = _finite_positive_codes(fmt)
    c = rng.choice(pos, size=shape).astype(np.uint8)
    return c | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)


def _frac(codes, fmt):
    return [[Fraction(oracle.fp8_decode_scalar(int(c), fmt)) for c in row] for row in codes]


def test_gemm_refs_against_exact_rational_arithmetic():
    rng = np.random.default_rng(21)
    M, N, K = 5, 7, 9  # distinct, not multiples of 16: a swapped operand cannot fit
    x8 = _codes(rng, (M, K), E4M3)
    w8 = _codes(rng, (N, K), E4M3)
    dy8 = _codes(rng, (M, N), E5M2)
    sx, sw, sdy = np.float32(3.25), np.float32(0.375), np.float32(1536.0)
    X, W, DY = _frac(x8, E4M3), _frac(w8, E4M3), _frac(dy8, E5M2)
    Wt = [list(r) for r in zip(*W)]
    DYt = [list(r) for r in zip(*DY)]
    y = _exact_matmul(X, W, transpose_b=True)
    dx = _exact_matmul(DY, W, transpose_b=False)
    dw = _exact_matmul(DYt, X, transpose_b=False)
    assert len(Wt) == K
    cases = [(oracle.forward_ref(x8, w8, sx, sw), y, Fraction(float(sx)) * Fraction(float(sw))),
             (oracle.dgrad_ref(dy8, w8, sdy, sw), dx, Fraction(float(sdy)) * Fraction(float(sw))),
             (oracle.wgrad_ref(dy8, x8, sdy, sx), dw, Fraction(float(sdy)) * Fraction(float(sx)))]
    for got, exact, den in cases:
        assert got.shape == (len(exact), len(exact[0]))
        for i in range(got.shape[0]):
            for j in range(got.shape[1]):
                want = exact[i][j] / den
                assert abs(Fraction(float(got[i, j])) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)])
def test_gemm_ref_any_formats_against_exact_rational_arithmetic(fa, fb):
    """The format-generic reference C = A8 B8^T / (s_a s_b): every operand
    code over its whole finite range (both signs), each format decoded as
    its own, against the Fraction triple loop; distinct M, N, K so that a
    transposed or swapped operand cannot fit."""
    rng = np.random.default_rng(31 + 2 * fa + fb)
    M, N, K = 4, 6, 11
    a8 = _codes(rng, (M, K), fa)
    b8 = _codes(rng, (N, K), fb)
    sa, sb = np.float32(0.1875), np.float32(640.0)
    exact = _exact_matmul(_frac(a8, fa), _frac(b8, fb), transpose_b=True)
    den = Fraction(float(sa)) * Fraction(float(sb))
    got = oracle.gemm_ref(a8, fa, b8, fb, sa, sb)
    assert got.shape == (M, N)
    for i in range(M):
        for j in range(N):
            want = exact[i][j] / den
            assert abs(Fraction(float(got[i, j])) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)
    # decoding with the other format changes the result: the formats are not mixed up
    if fa != fb:
        assert not np.array_equal(got, oracle.gemm_ref(a8, fb, b8, fa, sa, sb))


def test_bias_refs_against_exact_rational_arithmetic():
    """Y = X8 W8^T / (s_x s_w) + b and db = column sums of dY, against
    Fractions written from the definitions."""
    rng = np.random.default_rng(23)
    M, N, K = 6, 5, 7
    x8 = _codes(rng, (M, K), E4M3)
    w8 = _codes(rng, (N, K), E4M3)
    sx, sw = np.float32(2.5), np.float32(0.75)
    bias = rng.integers(0, 0x10000, N).astype(np.uint16)
    bias[(bias & 0x7F80) == 0x7F80] = 0x3F80  # finite biases only
    dy = rng.integers(0, 0x10000, (M, N)).astype(np.uint16)
    dy[(dy & 0x7F80) == 0x7F80] = 0xBF00
    bvals = [Fraction(float(v)) for v in _bf16_to_f32(bias)]
    y = _exact_matmul(_frac(x8, E4M3), _frac(w8, E4M3), transpose_b=True)
    den = Fraction(float(sx)) * Fraction(float(sw))
    got = oracle.forward_ref(x8, w8, sx, sw, bias)
    for i in range(M):
        for j in range(N):
            want = y[i][j] / den + bvals[j]
            assert abs(Fraction(float(got[i, j])) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)
    dvals = [[Fraction(float(v)) for v in _bf16_to_f32(row)] for row in dy]
    db = oracle.dbias_ref(dy)
    for j in range(N):
        want = sum((dvals[i][j] for i in range(M)), Fraction(0))
        assert abs(Fraction(float(db[j])) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_dbias_ref_invariants():
    # ones -> the row count; row order does not matter; a transposed input
    # would give the row sums instead (a distinct shape catches the swap)
    M, N = 37, 11
    ones = np.full((M, N), 0x3F80, dtype=np.uint16)
    assert np.array_equal(oracle.dbias_ref(ones), np.full(N, float(M)))
    rng = np.random.default_rng(5)
    dy = (rng.standard_normal((M, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    perm = rng.permutation(M)
    assert np.allclose(oracle.dbias_ref(dy), oracle.dbias_ref(dy[perm]), rtol=0, atol=1e-12)
    assert oracle.dbias_ref(dy).shape == (N,)
    ref_sum = _bf16_to_f32(dy.reshape(-1)).reshape(M, N).astype(np.float64).sum(axis=0)
    assert np.allclose(oracle.dbias_ref(dy), ref_sum, rtol=1e-15, atol=1e-12)


def test_gemm_sampled_entries_equal_full_refs():
    rng = np.random.default_rng(22)
    M, N, K = 33, 47, 65
    x8 = _codes(rng, (M, K), E4M3)
    w8 = _codes(rng, (N, K), E4M3)
    dy8 = _codes(rng, (M, N), E5M2)
    sx, sw, sdy = np.float32(2.0), np.float32(0.5), np.float32(4096.0)
    y = oracle.forward_ref(x8, w8, sx, sw)
    dx = oracle.dgrad_ref(dy8, w8, sdy, sw)
    dw = oracle.wgrad_ref(dy8, x8, sdy, sx)
    r = rng.integers(0, M, 50)
    c = rng.integers(0, N, 50)
    assert np.allclose(oracle.forward_ref_at(x8, w8, sx, sw, r, c), y[r, c], rtol=1e-14, atol=0)
    c2 = rng.integers(0, K, 50)
    assert np.allclose(oracle.dgrad_ref_at(dy8, w8, sdy, sw, r, c2), dx[r, c2], rtol=1e-14, atol=0)
    r3 = rng.integers(0, N, 50)
    assert np.allclose(oracle.wgrad_ref_at(dy8, x8, sdy, sx, r3, c2), dw[r3, c2], rtol=1e-14, atol=0)


def test_gemm_integer_exact_case():
    """Small-integer fp8 values with scale 1: every partial sum is an integer
    far below 2^24, so the reference is exact and equals integer matmul."""
    rng = np.random.default_rng(23)
    ints = {1: 0x38, 2: 0x40, 3: 0x44, -1: 0xB8, -2: 0xC0, 0: 0x00}
    keys = np.array(list(ints))
    M, N, K = 16, 48, 1600
    xa = rng.choice(keys, (M, K))
    wa = rng.choice(keys, (N, K))
    x8 = np.vectorize(ints.get)(xa).astype(np.uint8)
    w8 = np.vectorize(ints.get)(wa).astype(np.uint8)
    y = oracle.forward_ref(x8, w8, 1.0, 1.0)
    assert np.array_equal(y, (xa.astype(np.int64) @ wa.T.astype(np.int64)).astype(np.float64))


# ------------------------------------------------------------ delayed scaling

def test_history_ring_and_window():
    h = oracle.DelayedHistory()
    amaxes = [float(i + 1) for i in range(20)]
    for a in amaxes:
        h.push(a)
    assert h.count == 16 and h.pos == 20 % 16
    assert sorted(h.hist.tolist()) == amaxes[-16:]
    x = np.array([0x3F80], dtype=np.uint16)
    assert h.amax_for_scale(x) == 20.0  # history max, not the current tensor
    fresh = oracle.DelayedHistory()
    assert fresh.amax_for_scale(np.array([0x4040], dtype=np.uint16)) == 3.0  # first step: current amax
    part = oracle.DelayedHistory()
    for a in [5.0, 2.0, 7.0]:
        part.push(a)
    assert part.count == 3 and part.pos == 3 and part.amax_for_scale(x) == 7.0


def test_delayed_same_tensor_equals_dynamic_after_first_step():
    x = torch.randn(32, 48, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    h = oracle.DelayedHistory()
    s_dyn, _ = oracle.scale(oracle.amax(xb), E4M3)
    q_dyn, _, _ = oracle.cast(xb, E4M3, s_dyn)
    for _ in range(3):
        s, _ = oracle.scale(h.amax_for_scale(xb), E4M3)
        q, _, _ = oracle.cast(xb, E4M3, s)
        assert np.array_equal(q, q_dyn)
        h.push(oracle.amax(xb))


def test_delayed_spike_only_affects_later_steps():
    gen = torch.Generator().manual_seed(6)
    xs = [torch.randn(16, 32, generator=gen).to(torch.bfloat16) for _ in range(4)]
    xs[2] = xs[2] * 50  # a spike at step 2
    h = oracle.DelayedHistory()
    sats = []
    scales = []
    for x in xs:
        xb = x.view(torch.int16).numpy().view(np.uint16)
        s, _ = oracle.scale(h.amax_for_scale(xb), E4M3)
        _, _, nsat = oracle.cast(xb, E4M3, s)
        sats.append(nsat)
        scales.append(s)
        h.push(oracle.amax(xb))
    assert sats[2] > 0  # the spike saturates against the stale history
    assert scales[3] < scales[2] / 10  # and only the next step sees it


def test_delayed_checkpoint_restore_is_exact():
    gen = torch.Generator().manual_seed(8)
    xs = [(torch.randn(8, 16, generator=gen) * (1 + i)).to(torch.bfloat16) for i in range(20)]

    def run(h, seq):
        out = []
        for x in seq:
            xb = x.view(torch.int16).numpy().view(np.uint16)
            s, _ = oracle.scale(h.amax_for_scale(xb), E4M3)
            out.append(oracle.cast(xb, E4M3, s)[0])
            h.push(oracle.amax(xb))
        return out

    full = run(oracle.DelayedHistory(), xs)
    h = oracle.DelayedHistory()
    first = run(h, xs[:10])
    saved = h.copy()
    second = run(saved, xs[10:])
    for a, b in zip(full, first + second):
        assert np.array_equal(a, b)


def test_linear_step_shapes_and_scales():
    gen = torch.Generator().manual_seed(0)
    x = torch.randn(32, 48, generator=gen).to(torch.bfloat16)
    w = (torch.randn(64, 48, generator=gen) / 48 ** 0.5).to(torch.bfloat16)
    dy = (torch.randn(32, 64, generator=gen) * 1e-3 ** 0.5).to(torch.bfloat16)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    r = oracle.linear_step(bits(x), bits(w), bits(dy))
    assert r["y"].shape == (32, 64) and r["dx"].shape == (32, 48) and r["dw"].shape == (64, 48)
    assert r["x"]["q"].shape == (32, 48) and r["x"]["qt"].shape == (48, 32)
    # the dequantised GEMMs approximate the bf16 products to fp8 accuracy
    yf = x.double() @ w.double().T
    assert np.abs(r["y"] - yf.numpy()).max() < 0.1 * np.abs(yf.numpy()).max()
    dxf = dy.double() @ w.double()
    assert np.abs(r["dx"] - dxf.numpy()).max() < 0.2 * np.abs(dxf.numpy()).max()
    dwf = dy.double().T @ x.double()
    assert np.abs(r["dw"] - dwf.numpy()).max() < 0.2 * np.abs(dwf.numpy()).max()
