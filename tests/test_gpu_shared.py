"""Cast reuse: linears that read the same input cast it once
(f8lin_forward_shared_x: the q, k, v projections of an attention block, the
two input projections of a gated MLP -- pytorch/torchtitan PR #778's Llama3
8B training table), and a weight whose cast is still valid is not cast again
(w_cast_valid: micro-batches of one optimizer step).  Both must give, bit for
bit, what separate f8lin_forward calls give; those are checked against the
oracle elsewhere, and here once more for the shared X."""
import numpy as np
import pytest
import torch

import oracle
from float8linear_tensorwise_amax_amd import inputs
from helpers import bf16_to_f64, bits, f32_bits, gemm_check, np_f32_bits, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def f8():
    from float8linear_tensorwise_amax_amd import f8lin
    return f8lin


def _lin(f8, M, N, K, seed, bias=False):
    w = inputs.random_bf16((N, K), seed=seed, std=K ** -0.5).to(DEV)
    d = {"w": w, "y": torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
         "w8": torch.empty((N, K), dtype=torch.uint8, device=DEV),
         "w8t": f8.new_transposed(K, N, DEV), "sw": f8.ScalingState(DEV)}
    if bias:
        d["bias"] = inputs.random_bf16((N,), seed=seed + 1, std=0.1).to(DEV)
    return d


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("algo", ["atomic", "twopass"])
@pytest.mark.parametrize("shape", [(512, 256, (256, 64, 64)), (8192, 4096, (4096, 1024, 1024)), (8192, 4096, (14336, 14336)),
                                   (16, 4096, (4096, 4096)), (300 // 16 * 16, 160, (96, 48, 32, 16))])
def test_shared_x_equals_separate_forwards(f8, shape, algo):
    M, K, Ns = shape
    print(f"shared-x M={M} K={K} Ns={Ns} {algo}", flush=True)
    x = inputs.random_bf16((M, K), seed=M + K).to(DEV)
    lins = [_lin(f8, M, N, K, seed=10 + i, bias=(i == 1)) for i, N in enumerate(Ns)]
    x8 = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    x8t = f8.new_transposed(K, M, DEV)
    sx = f8.ScalingState(DEV)
    ws = f8.new_workspace(DEV)
    f8.forward_shared_x(x, x8, x8t, sx, ws, lins, "dynamic", algo)
    torch.cuda.synchronize()
    for i, l in enumerate(lins):
        ref = _lin(f8, M, l["w"].shape[0], K, seed=10 + i, bias=(i == 1))
        rx8, rx8t, rsx, rws = torch.empty_like(x8), f8.new_transposed(K, M, DEV), f8.ScalingState(DEV), f8.new_workspace(DEV)
        f8.forward(x, ref["w"], ref["y"], rx8, rx8t, ref["w8"], ref["w8t"], rsx, ref["sw"], rws, "dynamic", "dynamic",
                   algo, bias=ref.get("bias"))
        torch.cuda.synchronize()
        assert _same(l["y"], ref["y"]) and _same(l["w8"], ref["w8"]) and _same(l["w8t"], ref["w8t"]), i
        assert _same(l["sw"].scale, ref["sw"].scale) and _same(l["sw"].amax, ref["sw"].amax), i
        assert _same(x8, rx8) and _same(x8t, rx8t) and _same(sx.scale, rsx.scale), i
    # and the shared X cast itself against the oracle
    qx = oracle.linear_step(bits(x), bits(lins[0]["w"]), np.zeros((M, Ns[0]), np.uint16), gemms=False)["x"]
    assert np.array_equal(u8(x8), qx["q"]) and np.array_equal(u8(x8t), qx["qt"])
    assert f32_bits(sx.scale)[0] == np_f32_bits(qx["scale"])


@pytest.mark.parametrize("algo", ["atomic", "twopass"])
def test_weight_cast_reuse_across_micro_batches(f8, algo):
    """Two micro-batches with one weight: the second forward reuses W8, W8^T
    and W's scale (w not even passed) and gives the same bits as a full
    forward of that micro-batch."""
    M, N, K = 1024, 768, 512
    w = inputs.random_bf16((N, K), seed=3, std=K ** -0.5).to(DEV)
    xs = [inputs.random_bf16((M, K), seed=20 + i).to(DEV) for i in range(2)]
    buf = f8.LinearBuffers(M, N, K, DEV)
    buf.forward(xs[0], w, "dynamic", algo)
    f8.forward(xs[1], None, buf.y, buf.x8, buf.x8t, buf.w8, buf.w8t, buf.sx, buf.sw, buf.ws, algo=algo,
               w_cast_valid=True)
    ref = f8.LinearBuffers(M, N, K, DEV)
    ref.forward(xs[1], w, "dynamic", algo)
    torch.cuda.synchronize()
    for name in ("y", "x8", "x8t", "w8", "w8t"):
        assert _same(getattr(buf, name), getattr(ref, name)), name
    r = oracle.linear_step(bits(xs[1]), bits(w), np.zeros((M, N), np.uint16), gemms=True)
    gemm_check(bf16_to_f64(buf.y), r["y"], what="reused-weight Y")


def test_shared_x_mixed_modes_and_reuse(f8):
    """Entries may mix a delayed-scaling weight, a dynamic one and a reused
    cast; each output still equals its separate forward."""
    M, K = 256, 384
    x = inputs.random_bf16((M, K), seed=41).to(DEV)
    a = _lin(f8, M, 128, K, seed=42)
    b = _lin(f8, M, 64, K, seed=43)
    c = _lin(f8, M, 96, K, seed=44)
    b["sw"].history.fill_(0.25)  # delayed: a history max of 0.25
    b["mode_w"] = "delayed"
    # c's cast comes from an earlier forward of the same weight
    x8 = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    x8t = f8.new_transposed(K, M, DEV)
    sx, ws = f8.ScalingState(DEV), f8.new_workspace(DEV)
    f8.forward(x, c["w"], c["y"], x8, x8t, c["w8"], c["w8t"], sx, c["sw"], ws)
    c["w_cast_valid"] = True
    f8.forward_shared_x(x, x8, x8t, sx, ws, [a, b, c])
    torch.cuda.synchronize()
    for l in (a, b, c):
        N = l["w"].shape[0]
        ref = _lin(f8, M, N, K, seed=0)
        ref["w"] = l["w"]
        if l.get("mode_w") == "delayed":
            ref["sw"].history.fill_(0.25)
        rx8, rx8t = torch.empty_like(x8), f8.new_transposed(K, M, DEV)
        f8.forward(x, l["w"], ref["y"], rx8, rx8t, ref["w8"], ref["w8t"], f8.ScalingState(DEV), ref["sw"],
                   f8.new_workspace(DEV), "dynamic", l.get("mode_w", "dynamic"))
        torch.cuda.synchronize()
        assert _same(l["y"], ref["y"]) and _same(l["w8"], ref["w8"]), N
