"""The MFMA scale layout (MXGG_LAYOUT_MFMA) through the C ABI: pre-arranged
UE8M0 scales in units of 32 rows x 4 blocks, lane-ordered for the scaled
32x32x64 MFMA ("Integrate MXFP4 hipblaslt GEMM support": plain against
pre-swizzled scale layouts).

The expected layout is written here from its definition in include/mxgg.h
(byte (g, u, L, j) = scale of row 32u + L%32, block 4g + 2j + L/32) as a numpy
reshape of row-major scales, and checked against: the relayout in every
direction; the quantizers (row-wise, column-wise, dual), whose codes must
equal the block-major ones and whose scales must equal the oracle's; the
forward and input gradient fed MFMA-layout weight scales, which must equal the
block-major results bit for bit (the same arithmetic), including the full fc1
shapes, and the oracle within the GEMM tolerance."""
import numpy as np
import pytest

from oracle import grouped as og
from oracle import mx as omx
from synth import bf16_normal

from .gpu_util import assert_gemm_close, dev_bf16, have_gpu, host, host_bf16_f64, mx_scales_rowmajor

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import moe_grouped_block_mx_amd as mxg  # noqa: E402
import torch  # noqa: E402

MFMA = mxg.LAYOUT_MFMA


def mfma_layout(rm: np.ndarray) -> np.ndarray:
    """Row-major u8 [rows, blocks] -> the MFMA layout u8 [blocks/4, R32*4]."""
    rows, blocks = rm.shape
    assert blocks % 4 == 0
    r32 = (rows + 31) // 32 * 32
    pad = np.zeros((r32, blocks), dtype=np.uint8)
    pad[:rows] = rm
    # row r = 32u + l, block b = 4g + 2j + h  ->  [g, u, h, l, j], lane L = 32h + l
    t = pad.reshape(r32 // 32, 32, blocks // 4, 2, 2).transpose(2, 0, 4, 1, 3)
    return np.ascontiguousarray(t).reshape(blocks // 4, r32 * 4)


def test_layout_reference_matches_its_definition():
    # the reshape above against the header's per-byte statement, element by element
    rows, blocks = 45, 8
    rm = np.arange(rows * blocks, dtype=np.int64).reshape(rows, blocks) % 251 + 1
    ref = mfma_layout(rm.astype(np.uint8)).reshape(blocks // 4, 2, 64, 2)
    for r in range(64):
        for b in range(blocks):
            L = r % 32 + 32 * (b % 2)
            want = rm[r, b] if r < rows else 0
            assert ref[b // 4, r // 32, L, (b % 4) // 2] == want


@pytest.mark.parametrize("rows,blocks", [(1, 4), (31, 8), (33, 4), (150, 72), (301, 128), (4097, 4)])
def test_relayout_to_and_from_mfma(rows, blocks):
    rng = np.random.default_rng(rows * 1000 + blocks)
    rm = rng.integers(1, 256, size=(rows, blocks), dtype=np.uint8)
    R, B = mxg.LAYOUT_ROW_MAJOR, mxg.LAYOUT_BLOCK_MAJOR
    src = torch.from_numpy(rm).cuda()
    want = mfma_layout(rm)
    dst = torch.full(want.shape, 0xAB, dtype=torch.uint8, device="cuda")   # padding must be rewritten
    mf = mxg.mx_scales_relayout(src, rows, blocks, R, MFMA, dst=dst)
    bm = mxg.mx_scales_relayout(src, rows, blocks, R, B)
    mf2 = mxg.mx_scales_relayout(bm, rows, blocks, B, MFMA)
    back_r = mxg.mx_scales_relayout(mf, rows, blocks, MFMA, R)
    back_b = mxg.mx_scales_relayout(mf, rows, blocks, MFMA, B)
    torch.cuda.synchronize()
    assert np.array_equal(host(mf), want)
    assert np.array_equal(host(mf2), want)
    assert np.array_equal(host(back_r), rm)
    assert np.array_equal(host(back_b), host(bm))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("rows", [1, 45, 200, 1031])
def test_rowwise_quantizer_writes_the_mfma_layout(fmt, rows):
    K = 384
    x = bf16_normal((rows, K), 1.0, seed=rows + 7)
    f = mxg.FORMATS[fmt]
    q_b, s_b = mxg.quantize_rowwise(dev_bf16(x), f)
    # garbage in the scale padding must be overwritten
    s_m = torch.full((K // 128, (rows + 31) // 32 * 128), 0xCD, dtype=torch.uint8, device="cuda")
    q_m, _ = mxg.quantize_rowwise(dev_bf16(x), f | MFMA, scales=s_m)
    torch.cuda.synchronize()
    assert torch.equal(q_b, q_m)
    _, s_ref = omx.quantize_rowwise(x, fmt)                          # oracle, row-major [rows, K/32]
    assert np.array_equal(host(s_m), mfma_layout(np.asarray(s_ref, dtype=np.uint8)))
    assert np.array_equal(mx_scales_rowmajor(s_b, rows), s_ref)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_colwise_and_dual_quantizers_write_the_mfma_layout(fmt):
    sp = [256, 0, 128, 384]                      # multiples of 128, one empty expert
    rows, cols = sum(sp), 160
    x = bf16_normal((rows, cols), 1.0, seed=21)
    f = mxg.FORMATS[fmt]
    qc_b, sc_b, mpad = mxg.quantize_colwise_segpad(dev_bf16(x), sp, f)
    qc_m, sc_m, mpad_m = mxg.quantize_colwise_segpad(dev_bf16(x), sp, f | MFMA)
    xd = bf16_normal((rows, 256), 1.0, seed=22)
    qr_s, sr_s = mxg.quantize_rowwise(dev_bf16(xd), f | MFMA)
    qcs, scs, _ = mxg.quantize_colwise_segpad(dev_bf16(xd), sp, f | MFMA)
    qr_d, sr_d, qc_d, sc_d, _ = mxg.quantize_dual(dev_bf16(xd), sp, f | MFMA)
    torch.cuda.synchronize()
    assert mpad == mpad_m == rows
    assert torch.equal(qc_b, qc_m)
    # block-major column scales [mpad/32, cols] are the row-major [cols, mpad/32] transposed
    _, s_ref = omx.quantize_colwise_segpad(x, sp, fmt)
    assert np.array_equal(host(sc_b).T, s_ref)
    assert np.array_equal(host(sc_m), mfma_layout(np.ascontiguousarray(s_ref)))
    # dual == the two single-output quantizers, in the MFMA layout too
    assert torch.equal(qr_d, qr_s) and torch.equal(sr_d, sr_s)
    assert torch.equal(qc_d, qcs) and torch.equal(sc_d, scs)


def _quant_w(w_bits, G, N, fmt_bits):
    """W [G*N, K]: the forward's row-wise and the input gradient's column-wise
    operands, scales in the layout fmt_bits says."""
    qr, sr, qc, sc, _ = mxg.quantize_dual(dev_bf16(w_bits), [N] * G, mxg.MXFP4 | fmt_bits)
    return qr, sr, qc, sc


@pytest.mark.parametrize("a_fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("K", [256, 640])
def test_forward_and_input_gradient_with_mfma_weight_scales(a_fmt, K):
    sp = [100, 0, 300, 37]
    G, N, M = 4, 384, sum(sp)
    af = mxg.FORMATS[a_fmt]
    x = bf16_normal((M, K), 1.0, seed=31)
    w = bf16_normal((G * N, K), 0.05, seed=32)
    dy = bf16_normal((M, N), 1.0, seed=33)
    aq, as_ = mxg.quantize_rowwise(dev_bf16(x), af)
    dq, ds = mxg.quantize_rowwise(dev_bf16(dy), af)
    wq_b, ws_b, wc_b, wcs_b = _quant_w(w, G, N, 0)
    wq_m, ws_m, wc_m, wcs_m = _quant_w(w, G, N, MFMA)
    y_b = mxg.grouped_fwd(aq, as_, wq_b, ws_b, sp, N, K, a_fmt=af)
    y_m = mxg.grouped_fwd(aq, as_, wq_m, ws_m, sp, N, K, a_fmt=af, w_fmt=mxg.MXFP4 | MFMA)
    dx_b = mxg.grouped_dgrad(dq, ds, wc_b, wcs_b, sp, N, K, fmt=af)
    dx_m = mxg.grouped_dgrad(dq, ds, wc_m, wcs_m, sp, N, K, fmt=af | MFMA)
    torch.cuda.synchronize()
    assert torch.equal(wq_b, wq_m) and torch.equal(wc_b, wc_m)
    assert torch.equal(y_b, y_m), "forward: MFMA-layout weight scales change the result"
    assert torch.equal(dx_b, dx_m), "input gradient: MFMA-layout weight scales change the result"
    # and against the oracle on its own quantized operands
    X = omx.dequantize_rowwise(*omx.quantize_rowwise(x, a_fmt), a_fmt)
    W = omx.dequantize_rowwise(*omx.quantize_rowwise(w, "mxfp4"), "mxfp4").reshape(G, N, K)
    assert_gemm_close(host_bf16_f64(y_m), og.grouped_fwd(X, W, sp), what="forward, MFMA weight scales")
    DY = omx.dequantize_rowwise(*omx.quantize_rowwise(dy, a_fmt), a_fmt)
    WC = omx.dequantize_rowwise(*omx.quantize_colwise_segpad(w, [N] * G, "mxfp4"), "mxfp4")
    assert_gemm_close(host_bf16_f64(dx_m), og.grouped_dgrad(DY, WC, sp), what="input gradient, MFMA weight scales")


def test_full_size_fc1_forward_and_input_gradient_are_bit_identical():
    # MoE FC1 shapes: 32 experts, 32768 routed rows, K = 4096, N = 3072
    from synth import splits_for
    G, M, K, N = 32, 32768, 4096, 3072
    sp = [int(v) for v in splits_for("fc1")]
    gen = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
    w = (torch.randn((G * N, K), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    dy = torch.randn((M, N), device="cuda", generator=gen).to(torch.bfloat16)
    aq, as_ = mxg.quantize_rowwise(x, mxg.MXFP4)
    dq, ds = mxg.quantize_rowwise(dy, mxg.MXFP4)
    out = {}
    for lay in (0, MFMA):
        wq, ws, wc, wcs, _ = mxg.quantize_dual(w, [N] * G, mxg.MXFP4 | lay)
        out[lay] = (mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, w_fmt=mxg.MXFP4 | lay),
                    mxg.grouped_dgrad(dq, ds, wc, wcs, sp, N, K, fmt=mxg.MXFP4 | lay))
        del wq, ws, wc, wcs
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[MFMA][0])
    assert torch.equal(out[0][1], out[MFMA][1])


def test_mfma_layout_refused_for_activation_and_weight_gradient_scales():
    sp = [128, 128]
    M, N, K = 256, 128, 128
    x = dev_bf16(bf16_normal((M, K), 1.0, seed=41))
    aq, as_m = mxg.quantize_rowwise(x, mxg.MXFP4 | MFMA)
    wq, ws = mxg.quantize_rowwise(dev_bf16(bf16_normal((2 * N, K), 0.05, seed=42)), mxg.MXFP4)
    with pytest.raises(mxg.MxggError, match="MXGG_ERR_FORMAT"):
        mxg.grouped_fwd(aq, as_m, wq, ws, sp, N, K, a_fmt=mxg.MXFP4 | MFMA)
    qc, sc, mpad = mxg.quantize_colwise_segpad(x, sp, mxg.MXFP4 | MFMA)
    mg = torch.zeros((2, K, K), dtype=torch.float32, device="cuda")
    with pytest.raises(mxg.MxggError, match="MXGG_ERR_FORMAT"):
        mxg.grouped_wgrad(qc, sc, qc, sc, sp, K, K, mpad, mg, fmt=mxg.MXFP4 | MFMA)
    torch.cuda.synchronize()
    assert not mg.any()
