"""The GroupedLinear wrapper (autograd over the C ABI) on the GPU, for the
a4w4, a8w4 and blockwise recipes: forward, input gradient and the weight
gradient accumulated into fp32 main_grad match the fp64 oracle on the oracle's
quantized operands (tolerance 2^-7 |ref| + 1e-3 rms(ref)); two microbatches
accumulate; the weight quantization is reused until the weight changes and
follows is_first_microbatch; overwrite_main_grad makes the first microbatch
overwrite main_grad (immediate and delayed); preallocated out / dgrad_out are
written and returned; a delayed weight gradient equals the immediate one bit
for bit."""
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


def _oracle(recipe, x_bits, w_bits, dy_bits, splits, gnk=(G, N, K)):
    """fp64 forward output, input gradient and weight gradient on the
    oracle's quantized operands of the recipe."""
    G, N, K = gnk
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
    assert layer._cache.fwd[0].dim() == 3  # K-blocked codes (K and N are multiples of 128)
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


def test_overwrite_main_grad_on_the_first_microbatch():
    # overwrite_main_grad set for the first microbatch: its weight gradient
    # replaces whatever main_grad held (experts with no tokens become zero);
    # cleared afterwards: later microbatches add ("Add ROCm Triton blockwise
    # FP8 grouped GEMM", first-microbatch accumulation logic)
    M = sum(SPLITS)
    xs = [bf16_normal((M, K), 1.0, seed=40 + i) for i in range(2)]
    dys = [bf16_normal((M, N), 1.0, seed=50 + i) for i in range(2)]
    for delay in (False, True):
        layer = _layer("a4w4", delay=delay)
        layer.weight.main_grad.fill_(7.0)                       # stale contents
        layer.weight.overwrite_main_grad = True
        layer(dev_bf16(xs[0]), SPLITS).backward(dev_bf16(dys[0]))
        layer.weight.overwrite_main_grad = False                 # the mode of each backward is kept
        layer(dev_bf16(xs[1]), SPLITS).backward(dev_bf16(dys[1]))
        if delay:
            layer.backward_dw()
        torch.cuda.synchronize()
        w_bits = _bits(layer.weight)
        rdw = [_oracle("a4w4", xs[i], w_bits, dys[i], SPLITS)[2] for i in range(2)]
        got = host(layer.weight.main_grad).astype(np.float64)
        assert not got[1].any(), "the empty expert was not zero-filled"
        assert_gemm_close(got, rdw[0] + rdw[1], what=f"overwrite then accumulate (delay={delay})")


def test_preallocated_out_and_dgrad_out_are_written_and_returned():
    layer = _layer("a4w4")
    M = sum(SPLITS)
    x_bits, dy_bits = bf16_normal((M, K), 1.0, seed=60), bf16_normal((M, N), 1.0, seed=61)
    x = dev_bf16(x_bits).requires_grad_(True)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dgrad_out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    y = layer(x, SPLITS, out=out, dgrad_out=dgrad_out)
    (gx,) = torch.autograd.grad(y, x, dev_bf16(dy_bits))
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr() and gx.data_ptr() == dgrad_out.data_ptr()
    ry, rdx, _ = _oracle("a4w4", x_bits, _bits(layer.weight), dy_bits, SPLITS)
    assert_gemm_close(host_bf16_f64(out), ry, what="forward into out")
    assert_gemm_close(host_bf16_f64(dgrad_out), rdx, what="input gradient into dgrad_out")
    with pytest.raises(ValueError, match="dgrad_out"):
        layer(x, SPLITS, dgrad_out=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("recipe", ["a4w4", "a8w4"])
def test_mx_layer_with_features_off_128_keeps_plain_codes(recipe):
    # K-blocked MX codes need K and N to be multiples of 128; other layers
    # run on plain rows
    g, k, n, splits = 3, 160, 96, [40, 0, 57]
    gen = torch.Generator(device="cuda").manual_seed(6)
    layer = GroupedLinear(g, k, n, recipe=recipe, weight_std=0.05, generator=gen)
    m = sum(splits)
    x_bits = bf16_normal((m, k), 1.0, seed=11)
    dy_bits = bf16_normal((m, n), 1.0, seed=13)
    x = dev_bf16(x_bits).requires_grad_(True)
    y = layer(x, splits)
    y.backward(dev_bf16(dy_bits))
    torch.cuda.synchronize()
    assert layer._cache.fwd[0].dim() == 2
    ry, rdx, rdw = _oracle(recipe, x_bits, _bits(layer.weight), dy_bits, splits, gnk=(g, n, k))
    assert_gemm_close(host_bf16_f64(y), ry, what=f"{recipe} forward, K={k} N={n}")
    assert_gemm_close(host_bf16_f64(x.grad), rdx, what=f"{recipe} input gradient, K={k} N={n}")
    assert_gemm_close(host(layer.weight.main_grad).astype(np.float64), rdw, what=f"{recipe} weight gradient")


@pytest.mark.parametrize("recipe", ["a4w4", "a8w4", "blockwise"])
def test_is_first_microbatch_controls_weight_quantization(recipe):
    layer = _layer(recipe)
    M = sum(SPLITS)
    x = dev_bf16(bf16_normal((M, K), 1.0, seed=70))
    with pytest.raises(RuntimeError, match="is_first_microbatch=False"):
        layer(x, SPLITS, is_first_microbatch=False)           # nothing cached yet
    y0 = layer(x, SPLITS, is_first_microbatch=True)
    q0 = layer._cache.fwd[0]
    with torch.no_grad():
        layer.weight.data.mul_(0.5)                            # not seen by the version counter
    y1 = layer(x, SPLITS, is_first_microbatch=False)          # cached quantization reused
    assert layer._cache.fwd[0] is q0 and torch.equal(y0, y1)
    y2 = layer(x, SPLITS, is_first_microbatch=True)           # quantized again
    torch.cuda.synchronize()
    assert layer._cache.fwd[0] is not q0
    ry = _oracle(recipe, _bits(x), _bits(layer.weight), bf16_normal((M, N), 1.0, seed=1), SPLITS)[0]
    assert_gemm_close(host_bf16_f64(y2), ry, what="forward after is_first_microbatch=True")
