"""The GroupedLinear wrapper (autograd over the C ABI) on the GPU, for the
a4w4, a8w4 and blockwise recipes: forward, input gradient and the weight
gradient accumulated into fp32 main_grad match the fp64 oracle on the oracle's
quantized operands (tolerance 2^-7 |ref| + 1e-3 rms(ref)); two microbatches
accumulate; the weight quantization is reused until the weight changes; a
delayed weight gradient equals the immediate one bit for bit."""
import numpy as np
import pytest

from oracle import blockwise as ob
from oracle import grouped as og
from oracle import mx as omx
from synth import bf16_normal

from .gpu_util import assert_gemm_close, dev_bf16, have_gpu, host, host_bf16_f64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import torch  # noqa: E402

from moe_grouped_block_mx_amd.grouped_linear import RECIPES, GroupedLinear  # noqa: E402

SPLITS = [96, 0, 160, 33]          # ragged, an empty expert
G, K, N = 4, 256, 384


def _bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle(recipe, x_bits, w_bits, dy_bits, splits):
    """fp64 forward output, input gradient and weight gradient on the
    oracle's quantized operands of the recipe."""
    r = RECIPES[recipe]
    if recipe == "blockwise":
        X = ob.dequantize_1x128(*ob.quantize_1x128(x_bits))
        W = ob.dequantize_128x128(*ob.quantize_128x128(w_bits)).reshape(G, N, K)
        DY = ob.dequantize_1x128(*ob.quantize_1x128(dy_bits))
        y = og.grouped_fwd(X, W, splits)
        dx = og.grouped_fwd(DY, np.ascontiguousarray(W.transpose(0, 2, 1)), splits)
        dyc = ob.dequantize_1x128(*ob.quantize_colwise_segpad_128(dy_bits, splits))
        xc = ob.dequantize_1x128(*ob.quantize_colwise_segpad_128(x_bits, splits))
        dw = og.grouped_wgrad(dyc, xc, splits, pad=128)
        return y, dx, dw
    a, wf, gf = r["act"], r["wgt"], r["grad"]
    X = omx.dequantize_rowwise(*omx.quantize_rowwise(x_bits, a), a)
    W = omx.dequantize_rowwise(*omx.quantize_rowwise(w_bits, wf), wf).reshape(G, N, K)
    y = og.grouped_fwd(X, W, splits)
    DY = omx.dequantize_rowwise(*omx.quantize_rowwise(dy_bits, gf), gf)
    WC = omx.dequantize_rowwise(*omx.quantize_colwise_segpad(w_bits, [N] * G, wf), wf)
    dx = og.grouped_dgrad(DY, WC, splits)
    dyc = omx.dequantize_rowwise(*omx.quantize_colwise_segpad(dy_bits, splits, gf), gf)
    xc = omx.dequantize_rowwise(*omx.quantize_colwise_segpad(x_bits, splits, a), a)
    dw = og.grouped_wgrad(dyc, xc, splits)
    return y, dx, dw


def _layer(recipe, delay=False):
    gen = torch.Generator(device="cuda").manual_seed(5)
    return GroupedLinear(G, K, N, recipe=recipe, delay_wgrad=delay, weight_std=0.05, generator=gen)


@pytest.mark.parametrize("recipe", ["a4w4", "a8w4", "blockwise"])
def test_forward_backward_match_oracle(recipe):
    layer = _layer(recipe)
    M = sum(SPLITS)
    x_bits = bf16_normal((M, K), 1.0, seed=1)
    dy_bits = bf16_normal((M, N), 1.0, seed=3)
    x = dev_bf16(x_bits).requires_grad_(True)
    y = layer(x, SPLITS)
    y.backward(dev_bf16(dy_bits))
    torch.cuda.synchronize()
    assert layer.weight.grad is None       # accumulated into main_grad instead
    ry, rdx, rdw = _oracle(recipe, x_bits, _bits(layer.weight), dy_bits, SPLITS)
    assert_gemm_close(host_bf16_f64(y), ry, what=f"{recipe} forward")
    assert_gemm_close(host_bf16_f64(x.grad), rdx, what=f"{recipe} input gradient")
    assert_gemm_close(host(layer.weight.main_grad).astype(np.float64), rdw, what=f"{recipe} weight gradient")


def test_microbatches_accumulate_and_weight_cache():
    layer = _layer("a4w4")
    M = sum(SPLITS)
    xs = [bf16_normal((M, K), 1.0, seed=10 + i) for i in range(2)]
    dys = [bf16_normal((M, N), 1.0, seed=20 + i) for i in range(2)]
    layer(dev_bf16(xs[0]), SPLITS).backward(dev_bf16(dys[0]))
    q0 = layer._cache.fwd[0]
    layer(dev_bf16(xs[1]), SPLITS).backward(dev_bf16(dys[1]))
    torch.cuda.synchronize()
    assert layer._cache.fwd[0] is q0           # same weight version: quantized once
    w_bits = _bits(layer.weight)
    rdw = sum(_oracle("a4w4", xs[i], w_bits, dys[i], SPLITS)[2] for i in range(2))
    assert_gemm_close(host(layer.weight.main_grad).astype(np.float64), rdw, what="two microbatches")
    # an optimizer-style in-place update bumps the version: requantized
    with torch.no_grad():
        layer.weight.mul_(0.5)
    y = layer(dev_bf16(xs[0]), SPLITS)
    torch.cuda.synchronize()
    assert layer._cache.fwd[0] is not q0
    ry = _oracle("a4w4", xs[0], _bits(layer.weight), dys[0], SPLITS)[0]
    assert_gemm_close(host_bf16_f64(y), ry, what="forward after the update")


@pytest.mark.parametrize("recipe", ["a4w4", "a8w4"])
def test_delayed_wgrad_equals_immediate(recipe):
    M = sum(SPLITS)
    x_bits, dy_bits = bf16_normal((M, K), 1.0, seed=7), bf16_normal((M, N), 1.0, seed=8)
    outs = []
    for delay in (False, True):
        layer = _layer(recipe, delay=delay)
        layer(dev_bf16(x_bits), SPLITS).backward(dev_bf16(dy_bits))
        torch.cuda.synchronize()
        if delay:
            assert not layer.weight.main_grad.any()   # nothing launched yet
            layer.backward_dw()
            torch.cuda.synchronize()
        outs.append(host(layer.weight.main_grad))
    assert np.array_equal(outs[0], outs[1])


def test_frozen_input_and_empty_batch():
    layer = _layer("a4w4")
    x = dev_bf16(bf16_normal((sum(SPLITS), K), 1.0, seed=2))     # no grad wanted for x
    y = layer(x, SPLITS)
    y.sum().backward()
    torch.cuda.synchronize()
    assert layer.weight.main_grad.abs().sum() > 0
    e = layer(torch.empty((0, K), dtype=torch.bfloat16, device="cuda", requires_grad=True), [0] * G)
    e.sum().backward()
    torch.cuda.synchronize()
    assert e.shape == (0, N)
