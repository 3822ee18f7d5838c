"""The K-blocked MX code layouts (MXGG_KBLOCK_ROWS, MXGG_KBLOCK_COLS) through
the C ABI: codes in 64-byte blocks along the row, u8 [bytes per row / 64, rows,
64] (byte j of row r at ((j/64)*rows + r)*64 + j%64, the header's definition).

Checked against: the definition, element by element, on a small case; the
quantizers (row-wise, column-wise, dual in every combination of the two bits,
with block-major and MFMA scales), whose codes, read back through the
definition, must equal the plain-layout codes, and whose scales must be the
plain-layout scales; the forward and input gradient (a4w4 and a8w4, block-major
and MFMA weight scales) on K-blocked operands, which must equal the plain-layout
results bit for bit (the same arithmetic), including the full fc1 shapes, and
the oracle within the GEMM tolerance; and the refusals the header lists."""
import numpy as np
import pytest

from oracle import grouped as og
from oracle import mx as omx
from synth import bf16_normal

from .gpu_util import assert_gemm_close, dev_bf16, have_gpu, host, host_bf16_f64, kblocked_rows

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import moe_grouped_block_mx_amd as mxg  # noqa: E402
import torch  # noqa: E402

KR, KC, MFMA = mxg.KBLOCK_ROWS, mxg.KBLOCK_COLS, mxg.LAYOUT_MFMA


def test_kblocked_rows_helper_matches_the_definition():
    rows, nbytes = 37, 192
    q = np.arange(rows * nbytes, dtype=np.int64).reshape(rows, nbytes) % 251
    blocked = np.zeros((nbytes // 64, rows, 64), dtype=np.int64)
    for r in range(rows):
        for j in range(nbytes):
            blocked.reshape(-1)[((j // 64) * rows + r) * 64 + j % 64] = q[r, j]
    assert np.array_equal(kblocked_rows(torch.from_numpy(blocked)), q)


@pytest.mark.parametrize("lay", [0, MFMA], ids=["block-major", "mfma"])
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("rows", [1, 37, 300])
def test_rowwise_quantizer_writes_k_blocks(fmt, rows, lay):
    f = mxg.FORMATS[fmt] | lay
    x = dev_bf16(bf16_normal((rows, 384), 1.0, seed=rows))
    q0, s0 = mxg.quantize_rowwise(x, f)
    q1, s1 = mxg.quantize_rowwise(x, f | KR)
    torch.cuda.synchronize()
    assert q1.shape == (q0.shape[1] // 64, rows, 64)
    assert np.array_equal(kblocked_rows(q1), host(q0))
    assert torch.equal(s0, s1)


@pytest.mark.parametrize("lay", [0, MFMA], ids=["block-major", "mfma"])
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_rowwise_k_blocks_past_the_grid_row_limit(fmt, lay):
    # more than 65535 groups of 16 rows: workgroups loop over row groups, so
    # the LDS staging of the K blocks runs several times per workgroup
    rows, cols = 65535 * 16 + 1003, 256
    f = mxg.FORMATS[fmt] | lay
    gen = torch.Generator(device="cuda").manual_seed(17)
    x = torch.randn((rows, cols), device="cuda", generator=gen).to(torch.bfloat16)
    q0, s0 = mxg.quantize_rowwise(x, f)
    q1, s1 = mxg.quantize_rowwise(x, f | KR)
    torch.cuda.synchronize()
    nb = q0.shape[1] // 64
    assert q1.shape == (nb, rows, 64)
    assert torch.equal(q1, q0.reshape(rows, nb, 64).permute(1, 0, 2))
    assert torch.equal(s0, s1)


@pytest.mark.parametrize("lay", [0, MFMA], ids=["block-major", "mfma"])
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("bits", [KC, KR, KR | KC], ids=["cols", "rows", "both"])
def test_colwise_and_dual_quantizers_write_k_blocks(fmt, bits, lay):
    sp = [128, 0, 256, 384]  # column blocks (and MFMA column scales) need splits % 128
    f = mxg.FORMATS[fmt] | lay
    x = dev_bf16(bf16_normal((sum(sp), 256), 1.0, seed=7))  # row blocks need cols % 128
    qr0, sr0, qc0, sc0, mpad = mxg.quantize_dual(x, sp, f)
    qr1, sr1, qc1, sc1, mpad1 = mxg.quantize_dual(x, sp, f | bits)
    torch.cuda.synchronize()
    assert mpad1 == mpad
    assert torch.equal(sr0, sr1) and torch.equal(sc0, sc1)
    assert np.array_equal(kblocked_rows(qr1) if bits & KR else host(qr1), host(qr0))
    assert np.array_equal(kblocked_rows(qc1) if bits & KC else host(qc1), host(qc0))
    if bits == KC:  # the column-wise quantizer alone writes the same
        qc2, sc2, _ = mxg.quantize_colwise_segpad(x, sp, f | KC)
        torch.cuda.synchronize()
        assert torch.equal(qc2, qc1) and torch.equal(sc2, sc1)


def _weights(w, G, N, f):
    wq, ws, wc, wcs, _ = mxg.quantize_dual(dev_bf16(w), [N] * G, f)
    return wq, ws, wc, wcs


@pytest.mark.parametrize("lay", [0, MFMA], ids=["block-major", "mfma"])
@pytest.mark.parametrize("a_fmt", ["mxfp4", "mxfp8"])
def test_forward_and_input_gradient_on_k_blocks(a_fmt, lay):
    sp = [300, 0, 5, 129]
    G, N, K, M = 4, 256, 384, sum(sp)
    af = mxg.FORMATS[a_fmt]
    x = bf16_normal((M, K), 1.0, seed=31)
    w = bf16_normal((G * N, K), 0.05, seed=32)
    dy = bf16_normal((M, N), 1.0, seed=33)
    wf = mxg.MXFP4 | lay
    res = {}
    for kb in (0, KR | KC):
        aq, as_ = mxg.quantize_rowwise(dev_bf16(x), af | (kb & KR))
        dq, ds = mxg.quantize_rowwise(dev_bf16(dy), af | (kb & KR))
        wq, ws, wc, wcs = _weights(w, G, N, wf | kb)
        res[kb] = (mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt=af | (kb & KR), w_fmt=wf | (kb & KR)),
                   mxg.grouped_dgrad(dq, ds, wc, wcs, sp, N, K, fmt=af | lay | kb))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[KR | KC][0]), "forward: K-blocked codes change the result"
    assert torch.equal(res[0][1], res[KR | KC][1]), "input gradient: K-blocked codes change the result"
    X = omx.dequantize_rowwise(*omx.quantize_rowwise(x, a_fmt), a_fmt)
    W = omx.dequantize_rowwise(*omx.quantize_rowwise(w, "mxfp4"), "mxfp4").reshape(G, N, K)
    assert_gemm_close(host_bf16_f64(res[KR | KC][0]), og.grouped_fwd(X, W, sp), what="forward, K blocks")
    DY = omx.dequantize_rowwise(*omx.quantize_rowwise(dy, a_fmt), a_fmt)
    WC = omx.dequantize_rowwise(*omx.quantize_colwise_segpad(w, [N] * G, "mxfp4"), "mxfp4")
    assert_gemm_close(host_bf16_f64(res[KR | KC][1]), og.grouped_dgrad(DY, WC, sp), what="input gradient, K blocks")


def test_full_size_fc1_forward_and_input_gradient_are_bit_identical():
    # MoE FC1 shapes: 32 experts, 32768 routed rows, K = 4096, N = 3072
    from synth import splits_for
    G, M, K, N = 32, 32768, 4096, 3072
    sp = [int(v) for v in splits_for("fc1")]
    gen = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
    w = (torch.randn((G * N, K), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    dy = torch.randn((M, N), device="cuda", generator=gen).to(torch.bfloat16)
    out = {}
    for kb in (0, KR | KC):
        f = mxg.MXFP4 | kb
        aq, as_, _, _, _ = mxg.quantize_dual(x, sp, mxg.MXFP4 | (kb & KR))
        dq, ds, _, _, _ = mxg.quantize_dual(dy, sp, mxg.MXFP4 | (kb & KR))
        wq, ws, wc, wcs, _ = mxg.quantize_dual(w, [N] * G, f)
        out[kb] = (mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt=mxg.MXFP4 | (kb & KR),
                                   w_fmt=mxg.MXFP4 | (kb & KR)),
                   mxg.grouped_dgrad(dq, ds, wc, wcs, sp, N, K, fmt=f))
        del aq, as_, dq, ds, wq, ws, wc, wcs
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[KR | KC][0])
    assert torch.equal(out[0][1], out[KR | KC][1])


def test_full_size_a8w4_forward_and_input_gradient_are_bit_identical():
    # a8w4 shapes: 128 experts, 65536 routed rows, K = 7168, N = 2048; MXFP8
    # activations and output gradients, MXFP4 weights
    from synth import splits_for
    G, M, K, N = 128, 65536, 7168, 2048
    sp = [int(v) for v in splits_for("a8w4")]
    gen = torch.Generator(device="cuda").manual_seed(9)
    x = torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
    w = (torch.randn((G * N, K), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    dy = torch.randn((M, N), device="cuda", generator=gen).to(torch.bfloat16)
    out = {}
    for kb in (0, KR | KC):
        aq, as_ = mxg.quantize_rowwise(x, mxg.MXFP8 | (kb & KR))
        dq, ds = mxg.quantize_rowwise(dy, mxg.MXFP8 | (kb & KR))
        wq, ws, wc, wcs, _ = mxg.quantize_dual(w, [N] * G, mxg.MXFP4 | kb)
        out[kb] = (mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt=mxg.MXFP8 | (kb & KR),
                                   w_fmt=mxg.MXFP4 | (kb & KR)),
                   mxg.grouped_dgrad(dq, ds, wc, wcs, sp, N, K, fmt=mxg.MXFP8 | kb))
        del aq, as_, dq, ds, wq, ws, wc, wcs
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[KR | KC][0])
    assert torch.equal(out[0][1], out[KR | KC][1])


def test_k_blocks_with_512_experts_most_empty_and_an_empty_batch():
    # the largest expert count, 30 % of the experts empty and ragged tiny
    # segments: forward and input gradient on K-blocked codes equal the plain
    # layout bit for bit; then an empty batch, which launches nothing
    rng = np.random.default_rng(21)
    G, N, K = 512, 128, 256
    sp = rng.integers(0, 9, size=G)
    sp[rng.random(G) < 0.3] = 0
    sp = [int(v) for v in sp]
    M = sum(sp)
    x = dev_bf16(bf16_normal((M, K), 1.0, seed=22))
    w = dev_bf16(bf16_normal((G * N, K), 0.05, seed=23))
    dy = dev_bf16(bf16_normal((M, N), 1.0, seed=24))
    out = {}
    for kb in (0, KR | KC):
        aq, as_ = mxg.quantize_rowwise(x, mxg.MXFP4 | (kb & KR))
        dq, ds = mxg.quantize_rowwise(dy, mxg.MXFP4 | (kb & KR))
        wq, ws, wc, wcs, _ = mxg.quantize_dual(w, [N] * G, mxg.MXFP4 | kb)
        out[kb] = (mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt=mxg.MXFP4 | (kb & KR),
                                   w_fmt=mxg.MXFP4 | (kb & KR)),
                   mxg.grouped_dgrad(dq, ds, wc, wcs, sp, N, K, fmt=mxg.MXFP4 | kb))
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[KR | KC][0]) and torch.equal(out[0][1], out[KR | KC][1])
    e = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    eq, es = mxg.quantize_rowwise(e, mxg.MXFP4 | KR)
    y = mxg.grouped_fwd(eq, es, wq, ws, [0] * G, N, K, a_fmt=mxg.MXFP4 | KR, w_fmt=mxg.MXFP4 | KR)
    torch.cuda.synchronize()
    assert eq.shape == (K // 128, 0, 64) and y.shape == (0, N)


def test_k_block_bits_refused_where_the_header_says():
    sp = [128, 128]
    M, N, K = 256, 128, 128
    x = dev_bf16(bf16_normal((M, K), 1.0, seed=41))
    aq, as_ = mxg.quantize_rowwise(x, mxg.MXFP4 | KR)
    wq, ws = mxg.quantize_rowwise(dev_bf16(bf16_normal((2 * N, K), 0.05, seed=42)), mxg.MXFP4)
    with pytest.raises(mxg.MxggError, match="MXGG_ERR_FORMAT"):  # A blocked, W plain
        mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt=mxg.MXFP4 | KR, w_fmt=mxg.MXFP4)
    qc, sc, mpad = mxg.quantize_colwise_segpad(x, sp, mxg.MXFP4)
    qb = qc.reshape(mpad // 128, K, 64)  # a buffer of the blocked shape
    mg = torch.zeros((2, K, K), dtype=torch.float32, device="cuda")
    with pytest.raises(mxg.MxggError, match="MXGG_ERR_FORMAT"):  # the weight gradient takes no K blocks
        mxg.grouped_wgrad(qb, sc, qb, sc, sp, K, K, mpad, mg, fmt=mxg.MXFP4 | KC)
    with pytest.raises(mxg.MxggError, match="MXGG_ERR_SPLITS"):  # column blocks need splits % 128
        mxg.quantize_colwise_segpad(x, [100, 156], mxg.MXFP4 | KC)
    torch.cuda.synchronize()
    assert not mg.any()
