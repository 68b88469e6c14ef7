"""The amax of a GEMM's own bf16 output, taken in its epilogue, handed to the
next layer so that its dynamic-scaling cast skips the amax pass (the float8
ops fused with the op that produces their input: pytorch/ao issue #1199, the
reply on the ops not being fused with surrounding ops).

A chain of two linears, X1 -> lin1 -> Y1 = X2 -> lin2 -> Y2, and back:
  * y_amax of lin1's forward is max |Y1| bit for bit (the oracle's amax of
    the Y1 bytes the same call wrote: a property of the output, at any size),
    and dx_amax of lin2's backward is max |dX2|;
  * lin2's forward with that amax handed in (x_amax_given) gives the same
    bits, in every output and state, as lin2's ordinary forward with its own
    amax pass; lin1's backward with dY1 = dX2's amax handed in likewise;
  * the amax word is cleared by the call itself (it held garbage before).
Shapes take every GEMM variant that can write an amax: 256 x 256 tiles,
128 x 128 tiles with ragged edges and a bias (whose padding rows are not
stored and must not count), 64 x 128 tiles, the skinny kernel (M <= 64), a
K-split dX whose amax comes from the reduce kernel, the work-queue backward,
a lone problem split by rows into two launches that fold into one amax word,
and a shared-X forward with an amax per output."""
import numpy as np
import pytest
import torch

import oracle
from float8linear_tensorwise_amax_amd import inputs
from helpers import bits, f32_bits, gemm_check_dev, np_f32_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def f8():
    from float8linear_tensorwise_amax_amd import f8lin
    return f8lin


def _garbage_word():
    return torch.full((1,), 3.0e38, dtype=torch.float32, device=DEV)


def _same(a, b, what):
    a = a.view(torch.uint8) if a.dtype != torch.uint8 else a
    b = b.view(torch.uint8) if b.dtype != torch.uint8 else b
    assert torch.equal(a, b), what


@pytest.mark.parametrize("M,K1,N1,N2,bias,split", [
    (48, 160, 272, 96, True, True),         # small tiles, ragged, bias
    (16, 4096, 4096, 1024, False, True),    # skinny GEMMs
    (256, 1024, 4096, 4096, False, True),   # 64x128 tiles; dX of lin2 split along K (reduce kernel)
    (4096, 4096, 4096, 1024, True, True),   # big tiles with a bias; lin2's dW split, dX alone
    (4096, 4096, 4096, 1024, False, False),  # no split scratch: lin2's dX and dW through the work queue
    (9424, 1600, 1600, 1600, True, True)])   # lin1's Y and lin2's dX in two launches each (row split)
def test_chain_amax_from_epilogue(f8, M, K1, N1, N2, bias, split):
    print(f"chain M={M} K1={K1} N1={N1} N2={N2} bias={bias} split={split}", flush=True)
    x1 = inputs.random_bf16((M, K1), seed=1).to(DEV)
    w1 = inputs.random_bf16((N1, K1), seed=2, std=K1 ** -0.5).to(DEV)
    w2 = inputs.random_bf16((N2, N1), seed=3, std=N1 ** -0.5).to(DEV)
    dy2 = inputs.random_bf16((M, N2), seed=4, std=1e-3 ** 0.5).to(DEV)
    b1 = inputs.random_bf16((N1,), seed=5, std=0.5).to(DEV) if bias else None
    l1 = f8.LinearBuffers(M, N1, K1, DEV)
    l2 = f8.LinearBuffers(M, N2, N1, DEV)
    ref2 = f8.LinearBuffers(M, N2, N1, DEV)
    ref1 = f8.LinearBuffers(M, N1, K1, DEV)
    if not split:
        for b in (l1, l2, ref1, ref2):
            b.gemm_ws = None
    y_amax, dx_amax = _garbage_word(), _garbage_word()

    # forward: lin1 takes the amax of its output Y1 in the epilogue
    f8.forward(x1, w1, l1.y, l1.x8, l1.x8t, l1.w8, l1.w8t, l1.sx, l1.sw, l1.ws, algo="twopass", bias=b1,
               y_amax=y_amax)
    torch.cuda.synchronize()
    y1 = l1.y
    assert f32_bits(y_amax)[0] == np_f32_bits(oracle.amax(bits(y1))), "amax(Y1)"
    # lin2 with amax(X2) handed in == lin2 with its own amax pass
    l2.sx.amax.copy_(y_amax)
    f8.forward(y1, w2, l2.y, l2.x8, l2.x8t, l2.w8, l2.w8t, l2.sx, l2.sw, l2.ws, algo="twopass", x_amax_given=True)
    ref2.forward(y1, w2, "dynamic", "twopass")
    torch.cuda.synchronize()
    for nm in ("y", "x8", "x8t", "w8", "w8t"):
        _same(getattr(l2, nm), getattr(ref2, nm), f"lin2 {nm}")
    _same(l2.sx.scale, ref2.sx.scale, "lin2 X scale")
    _same(l2.sx.amax, ref2.sx.amax, "lin2 X amax")

    # backward: lin2 takes amax(dX2) in the dgrad epilogue; dX2 is lin1's dY
    f8.backward(dy2, l2.x8t, l2.w8t, l2.dx, l2.dw, l2.dy8, l2.dy8t, l2.sx, l2.sw, l2.sdy, l2.ws, algo="atomic",
                gemm_ws=l2.gemm_ws, dx_amax=dx_amax)
    ref2.backward(dy2, "dynamic", "atomic")
    torch.cuda.synchronize()
    _same(l2.dx, ref2.dx, "lin2 dX")
    _same(l2.dw, ref2.dw, "lin2 dW")
    dx2 = l2.dx
    assert f32_bits(dx_amax)[0] == np_f32_bits(oracle.amax(bits(dx2))), "amax(dX2)"
    l1.sdy.amax.copy_(dx_amax)
    f8.backward(dx2, l1.x8t, l1.w8t, l1.dx, l1.dw, l1.dy8, l1.dy8t, l1.sx, l1.sw, l1.sdy, l1.ws, algo="atomic",
                gemm_ws=l1.gemm_ws, dy_amax_given=True)
    ref1.forward(x1, w1, "dynamic", "twopass", bias=b1)
    ref1.backward(dx2, "dynamic", "atomic")
    torch.cuda.synchronize()
    for nm in ("dx", "dw", "dy8", "dy8t"):
        _same(getattr(l1, nm), getattr(ref1, nm), f"lin1 {nm}")
    _same(l1.sdy.scale, ref1.sdy.scale, "lin1 dY scale")
    # and the chain's first output against the oracle (the bias included)
    q = oracle.linear_step(bits(x1), bits(w1), bits(dx2), gemms=False)
    gemm_check_dev(y1, oracle.forward_ref(q["x"]["q"], q["w"]["q"], q["x"]["scale"], q["w"]["scale"],
                                          None if b1 is None else bits(b1)), what="Y1")


def test_shared_x_forward_amax_per_output(f8):
    """q, k, v from one X (one launch of three GEMMs): each output's amax word
    gets that output's amax, and a call without amax words gives the same
    outputs."""
    M, K = 1024, 512
    Ns = (512, 128, 128)
    x = inputs.random_bf16((M, K), seed=11).to(DEV)
    ws = [inputs.random_bf16((n, K), seed=12 + i, std=K ** -0.5).to(DEV) for i, n in enumerate(Ns)]
    bufs = [f8.LinearBuffers(M, n, K, DEV) for n in Ns]
    refs = [torch.empty_like(b.y) for b in bufs]
    words = [_garbage_word() for _ in Ns]
    lead = bufs[0]
    for with_amax, outs in ((True, [b.y for b in bufs]), (False, refs)):
        lin = [{"w": w, "y": y, "w8": b.w8, "w8t": b.w8t, "sw": b.sw} for w, y, b in zip(ws, outs, bufs)]
        if with_amax:
            for d, wd in zip(lin, words):
                d["y_amax"] = wd
        f8.forward_shared_x(x, lead.x8, lead.x8t, lead.sx, lead.ws, lin, algo="atomic")
    torch.cuda.synchronize()
    for b, r, wd in zip(bufs, refs, words):
        _same(b.y, r, "shared-X output")
        assert f32_bits(wd)[0] == np_f32_bits(oracle.amax(bits(b.y)))
    # an empty output (M = 0) leaves its amax at zero
    e = f8.LinearBuffers(0, 32, 64, DEV)
    wd = _garbage_word()
    f8.forward(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), inputs.random_bf16((32, 64), seed=20).to(DEV),
               e.y, e.x8, e.x8t, e.w8, e.w8t, e.sx, e.sw, e.ws, y_amax=wd)
    torch.cuda.synchronize()
    assert float(wd.item()) == 0.0
