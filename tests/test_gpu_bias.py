"""Bias (the linear layers of pytorch/ao issue #1297's GPT repro keep
nn.Linear's default bias): Y = X8 W8^T / (s_x s_w) + b from the forward's
epilogue, and the bias gradient db = column sums of dY from the backward's
cast pass, against the oracle.

Tolerances.  Y: the GEMM tolerance.  db: the kernels sum the bf16 dY values
in fp32 along a fixed tree whose depth is at most 17 + ceil(M / 1024)
additions (4 rows per thread, 3 shuffle levels, 3 wave adds, ceil(M / 128) / 8
tiles per group, 7 group adds), so |db - ref| <= depth * 2^-24 * sum_m |dY|
before the final rounding to bf16 adds half an ulp; the test allows
1e-5 * sum_m |dY| + ulp_bf16(|ref|), which covers every M used here."""
import numpy as np
import pytest
import torch

import oracle
from float8linear_tensorwise_amax_amd import inputs
from helpers import bf16_to_f64, bf16_ulp, bits, gemm_check, gemm_check_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def f8():
    from float8linear_tensorwise_amax_amd import f8lin
    return f8lin


def _dbias_check(got, dy_bits):
    ref = oracle.dbias_ref(dy_bits)
    absum = np.abs(oracle.bf16_to_f64(dy_bits)).sum(axis=0)
    tol = 1e-5 * absum + bf16_ulp(ref)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    assert not bad.any(), f"dbias: {int(bad.sum())} of {bad.size} out of tolerance, first {np.argwhere(bad)[:3].ravel()}"


def _run(f8, M, N, K, seed, algo="twopass", dy_std=1e-3 ** 0.5):
    gen = torch.Generator().manual_seed(seed)
    x = (torch.randn((M, K), generator=gen)).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=gen) * K ** -0.5).to(torch.bfloat16)
    dy = (torch.randn((M, N), generator=gen) * dy_std).to(torch.bfloat16)
    b = (torch.randn((N,), generator=gen) * 0.1).to(torch.bfloat16)
    buf = f8.LinearBuffers(M, N, K, DEV, with_bias=True)
    buf.forward(x.to(DEV), w.to(DEV), "dynamic", algo, bias=b.to(DEV))
    buf.backward(dy.to(DEV), "dynamic", algo)
    torch.cuda.synchronize()
    return buf, x, w, dy, b


@pytest.mark.parametrize("algo", ["atomic", "twopass"])
@pytest.mark.parametrize("mnk", [(144, 160, 96), (16, 4096, 4096), (300 // 16 * 16, 272, 400), (1024, 1024, 256)])
def test_bias_forward_and_gradient(f8, mnk, algo):
    M, N, K = mnk
    print(f"bias M={M} N={N} K={K} {algo}", flush=True)
    buf, x, w, dy, b = _run(f8, M, N, K, seed=M + N + K)
    ref = oracle.linear_step(bits(x), bits(w), bits(dy), bias_bits=bits(b))
    gemm_check(bf16_to_f64(buf.y), ref["y"], what=f"Y + b {mnk}")
    gemm_check(bf16_to_f64(buf.dx), ref["dx"], what=f"dX {mnk}")
    gemm_check(bf16_to_f64(buf.dw), ref["dw"], what=f"dW {mnk}")
    _dbias_check(bf16_to_f64(buf.dbias), bits(dy))


def test_bias_gpt_qkv_full_size(f8):
    """The repro's attention projection (12288 tokens, 1600 -> 4800) with its
    bias: Y and db in full."""
    M, N, K = 12288, 4800, 1600
    buf, x, w, dy, b = _run(f8, M, N, K, seed=11)
    qx = oracle.cast(bits(x), oracle.E4M3, oracle.scale(oracle.amax(bits(x)), oracle.E4M3)[0])[0]
    qw = oracle.cast(bits(w), oracle.E4M3, oracle.scale(oracle.amax(bits(w)), oracle.E4M3)[0])[0]
    sx = oracle.scale(oracle.amax(bits(x)), oracle.E4M3)[0]
    sw = oracle.scale(oracle.amax(bits(w)), oracle.E4M3)[0]
    gemm_check_dev(buf.y, oracle.forward_ref(qx, qw, sx, sw, bits(b)), what="gpt qkv Y + b")
    _dbias_check(bf16_to_f64(buf.dbias), bits(dy))


def test_bias_with_the_row_split(f8):
    """9424 x 1600 outputs are 259 tiles of 256 x 256, a second round of
    three: Y and dX each run as two launches (36 tile rows on 256 x 256
    tiles, 208 rows on 64 x 128 tiles), both adding the bias to Y."""
    M, N, K = 9424, 1600, 1600
    buf, x, w, dy, b = _run(f8, M, N, K, seed=13)
    ref = oracle.linear_step(bits(x), bits(w), bits(dy), bias_bits=bits(b))
    gemm_check(bf16_to_f64(buf.y), ref["y"], what="Y + b, row split")
    gemm_check(bf16_to_f64(buf.dx), ref["dx"], what="dX, row split")
    gemm_check(bf16_to_f64(buf.dw), ref["dw"], what="dW")
    _dbias_check(bf16_to_f64(buf.dbias), bits(dy))


def test_bias_gradient_is_run_to_run_identical_and_empty_m(f8):
    buf, x, w, dy, b = _run(f8, 4096, 1024, 256, seed=5)
    first = buf.dbias.clone()
    buf.backward(dy.to(DEV), "dynamic", "twopass")
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), buf.dbias.view(torch.int16))
    # no tokens: the bias gradient is zero, Y is empty
    buf0 = f8.LinearBuffers(0, 48, 32, DEV, with_bias=True)
    buf0.dbias.fill_(7.0)
    bias = torch.ones(48, dtype=torch.bfloat16, device=DEV)
    buf0.forward(torch.empty((0, 32), dtype=torch.bfloat16, device=DEV), w[:48, :32].contiguous().to(DEV),
                 bias=bias)
    buf0.backward(torch.empty((0, 48), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert torch.count_nonzero(buf0.dbias).item() == 0


def test_bias_does_not_change_the_rest(f8):
    """With a zero bias, Y, dX, dW and every fp8 byte equal the bias-free run
    bit for bit."""
    M, N, K = 256, 512, 384
    gen = torch.Generator().manual_seed(9)
    x = torch.randn((M, K), generator=gen).to(torch.bfloat16).to(DEV)
    w = (torch.randn((N, K), generator=gen) * K ** -0.5).to(torch.bfloat16).to(DEV)
    dy = (torch.randn((M, N), generator=gen) * 0.03).to(torch.bfloat16).to(DEV)
    a = f8.LinearBuffers(M, N, K, DEV)
    bb = f8.LinearBuffers(M, N, K, DEV, with_bias=True)
    a.forward(x, w)
    a.backward(dy)
    bb.forward(x, w, bias=torch.zeros(N, dtype=torch.bfloat16, device=DEV))
    bb.backward(dy)
    torch.cuda.synchronize()
    for name in ("y", "dx", "dw", "x8", "x8t", "w8", "w8t", "dy8", "dy8t"):
        assert torch.equal(getattr(a, name).view(torch.uint8), getattr(bb, name).view(torch.uint8)), name
