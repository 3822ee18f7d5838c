"""GPU parity of the blockwise FP8 path (1x128 activations, 128x128 weights,
1x128 column-wise segment-padded wgrad operands) through the C ABI against the
oracle: quantized codes and fp32 scales bit-exact, in power-of-two and fp32
scale modes, on ragged shapes and special blocks; grouped forward and weight
gradient within 2^-7 |ref| + 1e-3 rms(ref) of the fp64 contraction of the
oracle's dequantized operands; and a sampled check at the full blockwise FP8
MoE shapes (64 experts, 32768 rows, K=7168, N=4096)."""
import numpy as np
import pytest

from oracle import blockwise as ob
from oracle import grouped as og
from synth import bf16_normal, f32_normal, fp32_to_bf16_bits, splits_for

from .gpu_util import assert_gemm_close, dev_bf16, dev_f32, have_gpu, host, host_bf16_f64, kblocked_rows

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import moe_grouped_block_mx_amd as mxg  # noqa: E402
import torch  # noqa: E402

POW2 = mxg.POW2_SCALES


def _special_rows(cols, seed):
    """bf16 rows that exercise the scale rule: an all-zero block, a block below
    the 1e-4 amax floor, bf16 subnormals, the largest bf16 magnitudes, exact
    powers of two and signed zeros."""
    rng = np.random.default_rng(seed)
    rows = []
    z = np.zeros(cols, dtype=np.float32)
    rows.append(z)
    rows.append(np.where(rng.random(cols) < 0.5, -0.0, 0.0).astype(np.float32))
    rows.append((rng.standard_normal(cols) * 1e-6).astype(np.float32))
    rows.append((rng.standard_normal(cols) * 1e-39).astype(np.float32))  # bf16 subnormals
    rows.append((rng.standard_normal(cols) * 1e37).astype(np.float32))
    rows.append(np.ldexp(1.0, rng.integers(-20, 20, size=cols)).astype(np.float32) * np.sign(rng.standard_normal(cols)))
    bits = fp32_to_bf16_bits(np.stack(rows))
    bits[-1, :3] = [0x7F7F, 0xFF7F, 0x0001]  # max finite, -max finite, smallest subnormal
    return bits


@pytest.mark.parametrize("pow2", [True, False])
@pytest.mark.parametrize("shape", [(1, 128), (37, 384), (300, 1024)])
def test_quantize_1x128_rowwise(pow2, shape):
    x = bf16_normal(shape, 1.0, seed=11)
    if shape[0] >= 6:
        x[:6] = _special_rows(shape[1], 5)
    q, s = mxg.quantize_rowwise(dev_bf16(x), "fp8_1x128", flags=POW2 if pow2 else 0)
    torch.cuda.synchronize()
    rq, rs = ob.quantize_1x128(x, pow2=pow2)
    assert s.shape == (shape[1] // 128, shape[0])  # block-major
    assert np.array_equal(kblocked_rows(q), rq.astype(np.uint8))
    assert np.array_equal(host(s).T.copy().view(np.uint32), rs.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("pow2", [True, False])
def test_quantize_1x128_rowwise_past_the_grid_row_limit(pow2):
    # more than 65535 groups of 16 rows: workgroups loop over row groups (the
    # LDS staging of the K-blocked codes runs several times per workgroup);
    # rows from the first and the last groups against the oracle
    rows, cols = 65535 * 16 + 1003, 256
    gen = torch.Generator(device="cuda").manual_seed(19)
    x = torch.randn((rows, cols), device="cuda", generator=gen).to(torch.bfloat16)
    q, s = mxg.quantize_rowwise(x, "fp8_1x128", flags=POW2 if pow2 else 0)
    torch.cuda.synchronize()
    assert q.shape == (cols // 64, rows, 64) and s.shape == (cols // 128, rows)
    for sl in (slice(0, 40), slice(65535 * 16 - 8, 65535 * 16 + 40), slice(rows - 40, rows)):
        xb = host(x[sl].contiguous().view(torch.int16)).view(np.uint16)
        rq, rs = ob.quantize_1x128(xb, pow2=pow2)
        assert np.array_equal(kblocked_rows(q[:, sl, :].contiguous()), rq.astype(np.uint8)), sl
        assert np.array_equal(host(s[:, sl]).T.copy().view(np.uint32), rs.astype(np.float32).view(np.uint32)), sl


def test_quantize_1x128_strided_input():
    full = bf16_normal((50, 512), 1.0, seed=12)
    xt = dev_bf16(full)[:, 128:384]
    q, s = mxg.quantize_rowwise(xt, "fp8_1x128")
    torch.cuda.synchronize()
    rq, rs = ob.quantize_1x128(np.ascontiguousarray(full[:, 128:384]))
    assert np.array_equal(kblocked_rows(q), rq.astype(np.uint8))
    assert np.array_equal(host(s).T, rs.astype(np.float32))


@pytest.mark.parametrize("pow2", [True, False])
@pytest.mark.parametrize("shape", [(128, 128), (384, 256), (256, 640), (256, 512), (384, 1536)])
def test_quantize_128x128(pow2, shape):
    w = bf16_normal(shape, 0.02, seed=13)
    w[128:134] = _special_rows(shape[1], 6) if shape[0] > 128 else w[128:134]
    q, s = mxg.quantize_rowwise(dev_bf16(w), "fp8_128x128", flags=POW2 if pow2 else 0)
    torch.cuda.synchronize()
    rq, rs = ob.quantize_128x128(w, pow2=pow2)
    assert np.array_equal(kblocked_rows(q), rq.astype(np.uint8))
    assert np.array_equal(host(s).view(np.uint32), rs.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("cols", [256, 512])
def test_quantize_128x128_all_zero_block(cols):
    w = np.zeros((256, cols), dtype=np.uint16)
    w[128:, 128:256] = bf16_normal((128, 128), 1.0, seed=3)
    q, s = mxg.quantize_rowwise(dev_bf16(w), "fp8_128x128")
    torch.cuda.synchronize()
    rq, rs = ob.quantize_128x128(w)
    assert np.array_equal(kblocked_rows(q), rq.astype(np.uint8))
    assert np.array_equal(host(s), rs.astype(np.float32))


COL_CASES = [
    ([5, 0, 300], 64),
    ([128], 96),
    ([0, 0, 7], 160),
    ([129, 1, 255, 0, 40], 32),
    ([129, 1, 255, 0, 40], 256),         # cols % 128 == 0: 128 columns per workgroup
]


@pytest.mark.parametrize("pow2", [True, False])
@pytest.mark.parametrize("case", COL_CASES, ids=[f"{len(c[0])}x{c[1]}" for c in COL_CASES])
def test_quantize_colwise_1x128(pow2, case):
    splits, cols = case
    rows = int(np.sum(splits))
    x = bf16_normal((rows, cols), 1.0, seed=14)
    if rows >= 6:
        x[:6] = _special_rows(cols, 7)
    q, s, mpad = mxg.quantize_colwise_segpad(dev_bf16(x), splits, "fp8_1x128", flags=POW2 if pow2 else 0)
    torch.cuda.synchronize()
    rq, rs = ob.quantize_colwise_segpad_128(x, splits, pow2=pow2)
    assert mpad == rq.shape[1]
    assert s.shape == (mpad // 128, cols)  # block-major
    assert q.shape == (mpad // 64, cols, 64)  # 64-byte K blocks
    assert np.array_equal(kblocked_rows(q), rq.astype(np.uint8))
    assert np.array_equal(host(s).T.copy().view(np.uint32), rs.astype(np.float32).view(np.uint32))


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------
def _fwd_case(splits, N, K, pow2, seed=0, p2=(False, False)):
    """p2: (A, W) given as the power-of-two formats (quantized through them
    too); both set selects the GEMM path that applies the scales in the MFMA."""
    splits = np.asarray(splits, dtype=np.int64)
    G, M = len(splits), int(splits.sum())
    a = bf16_normal((M, K), 1.0, seed=seed + 1)
    w = bf16_normal((G * N, K), 0.02, seed=seed + 2)
    fl = POW2 if pow2 else 0
    af = "fp8_1x128_p2" if p2[0] else "fp8_1x128"
    wf = "fp8_128x128_p2" if p2[1] else "fp8_128x128"
    aq, as_ = mxg.quantize_rowwise(dev_bf16(a), af, flags=fl)
    wq, ws = mxg.quantize_rowwise(dev_bf16(w), wf, flags=fl)
    out = mxg.grouped_fwd(aq, as_, wq, ws, splits, N, K, a_fmt=af, w_fmt=wf)
    torch.cuda.synchronize()
    ra, ras = ob.quantize_1x128(a, pow2=pow2)
    rw, rws = ob.quantize_128x128(w, pow2=pow2)
    ref = og.grouped_fwd(ob.dequantize_1x128(ra, ras), ob.dequantize_128x128(rw, rws).reshape(G, N, K), splits)
    return host_bf16_f64(out), ref


FWD_CASES = [
    ([64, 0, 96, 96], 256, 256),
    ([1], 128, 128),
    ([300, 0, 5], 384, 640),
    ([513, 255, 1, 0, 40], 256, 1024),
]


@pytest.mark.parametrize("pow2", [True, False])
@pytest.mark.parametrize("case", FWD_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in FWD_CASES])
def test_blockwise_fwd(pow2, case):
    gpu, ref = _fwd_case(*case, pow2=pow2)
    assert_gemm_close(gpu, ref, what=f"blockwise fwd {case} pow2={pow2}")


@pytest.mark.parametrize("case", FWD_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in FWD_CASES])
def test_blockwise_fwd_pow2_formats(case):
    """Power-of-two formats on both sides: the scales are applied by the MFMA."""
    gpu, ref = _fwd_case(*case, pow2=True, p2=(True, True))
    assert_gemm_close(gpu, ref, what=f"blockwise fwd P2 {case}")


def test_blockwise_fwd_mixed_pow2_flags_take_the_general_path():
    gpu, ref = _fwd_case([300, 0, 5], 384, 640, pow2=True, p2=(True, False))
    assert_gemm_close(gpu, ref, what="blockwise fwd P2 x general")


def _wgrad_case(splits, N, K, pow2, out_bf16, accumulate, seed=0, p2=False):
    splits = np.asarray(splits, dtype=np.int64)
    G, M = len(splits), int(splits.sum())
    dy = bf16_normal((M, N), 1.0, seed=seed + 3)
    x = bf16_normal((M, K), 1.0, seed=seed + 1)
    fl = POW2 if pow2 else 0
    fmt = "fp8_1x128_p2" if p2 else "fp8_1x128"
    dq, ds, mpad = mxg.quantize_colwise_segpad(dev_bf16(dy), splits, fmt, flags=fl)
    xq, xs, _ = mxg.quantize_colwise_segpad(dev_bf16(x), splits, fmt, flags=fl)
    if out_bf16:
        mg0 = bf16_normal((G, N, K), 1.0, seed=seed + 4)
        mg = dev_bf16(mg0).reshape(G, N, K)
        mg0_f = host_bf16_f64(mg)
    else:
        mg0_f = f32_normal((G, N, K), seed=seed + 4).astype(np.float64)
        mg = dev_f32(mg0_f)
    mxg.grouped_wgrad(dq, ds, xq, xs, splits, N, K, mpad, mg, accumulate=accumulate, fmt=fmt)
    torch.cuda.synchronize()
    rd, rds = ob.quantize_colwise_segpad_128(dy, splits, pow2=pow2)
    rx, rxs = ob.quantize_colwise_segpad_128(x, splits, pow2=pow2)
    dw = og.grouped_wgrad(ob.dequantize_1x128(rd, rds), ob.dequantize_1x128(rx, rxs), splits, pad=128)
    if accumulate:
        ref = mg0_f + dw
    else:
        ref = dw
    gpu = host_bf16_f64(mg) if out_bf16 else host(mg).astype(np.float64)
    return gpu, ref


WG_CASES = [
    ([64, 0, 96, 96], 256, 256),
    ([300, 0, 5], 128, 384),
    ([129, 1, 255, 0, 40], 384, 128),
]


@pytest.mark.parametrize("mode", ["bf16_overwrite", "fp32_accumulate", "fp32_overwrite"])
@pytest.mark.parametrize("pow2", [True, False])
@pytest.mark.parametrize("case", WG_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in WG_CASES])
def test_blockwise_wgrad(mode, pow2, case):
    out_bf16 = mode.startswith("bf16")
    acc = mode.endswith("accumulate")
    gpu, ref = _wgrad_case(*case, pow2=pow2, out_bf16=out_bf16, accumulate=acc)
    splits = np.asarray(case[0])
    if acc:
        # untouched experts keep main_grad exactly
        for g in np.nonzero(splits == 0)[0]:
            assert np.array_equal(gpu[g], ref[g])
    assert_gemm_close(gpu, ref, what=f"blockwise wgrad {case} {mode} pow2={pow2}")


# The _P2 formats take the power-of-two kernel (the MFMA applies the scales).
# Its 4x256x256 overwrite case gives one workgroup a single empty-contraction
# tile, the case that once read an uninitialised DMA plan.
@pytest.mark.parametrize("mode", ["bf16_overwrite", "fp32_accumulate", "fp32_overwrite"])
@pytest.mark.parametrize("case", WG_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in WG_CASES])
def test_blockwise_wgrad_pow2_format(mode, case):
    out_bf16 = mode.startswith("bf16")
    acc = mode.endswith("accumulate")
    gpu, ref = _wgrad_case(*case, pow2=True, out_bf16=out_bf16, accumulate=acc, p2=True)
    splits = np.asarray(case[0])
    if acc:
        for g in np.nonzero(splits == 0)[0]:
            assert np.array_equal(gpu[g], ref[g])
    assert_gemm_close(gpu, ref, what=f"blockwise wgrad P2 {case} {mode}")


def test_blockwise_rejects_mixed_pairs():
    a = dev_bf16(bf16_normal((128, 256), 1.0, seed=1))
    aq, as_ = mxg.quantize_rowwise(a, "fp8_1x128")
    wq, ws = mxg.quantize_rowwise(dev_bf16(bf16_normal((128, 256), 0.02, seed=2)), "mxfp4")
    with pytest.raises(mxg.MxggError):
        mxg.grouped_fwd(aq, as_, wq, ws, [128], 128, 256, a_fmt="fp8_1x128", w_fmt="mxfp4")


# ---------------------------------------------------------------------------
# full blockwise FP8 MoE shapes, sampled
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def c5():
    from synth import WORKLOADS
    wl = WORKLOADS["blockwise"]
    G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
    sp = splits_for("blockwise")
    gen = torch.Generator(device="cuda").manual_seed(77)
    a = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((G * N, K), generator=gen, device="cuda") * wl["w_std"]).to(torch.bfloat16)
    return dict(G=G, M=M, K=K, N=N, sp=sp, a=a, w=w)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("p2", [False, True], ids=["general", "pow2"])
def test_c5_full_size_fwd_sampled(c5, p2):
    G, M, K, N, sp, a, w = (c5[k] for k in ("G", "M", "K", "N", "sp", "a", "w"))
    af, wf = ("fp8_1x128_p2", "fp8_128x128_p2") if p2 else ("fp8_1x128", "fp8_128x128")
    aq, as_ = mxg.quantize_rowwise(a, af)
    wq, ws = mxg.quantize_rowwise(w, wf)
    out = mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt=af, w_fmt=wf)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    offs = np.concatenate([[0], np.cumsum(sp)])
    nz = np.nonzero(sp)[0]
    for g in rng.choice(nz, size=6, replace=False):
        rows = offs[g] + rng.choice(sp[g], size=min(4, sp[g]), replace=False)
        blk = int(rng.integers(0, N // 128))
        cols = blk * 128 + rng.choice(128, size=16, replace=False)
        # the sampled activation rows and the sampled weight 128-row block,
        # quantized by the oracle, must equal the library's bytes
        ra, ras = ob.quantize_1x128(_bits(a[torch.as_tensor(rows, device="cuda")]))
        assert np.array_equal(kblocked_rows(aq[:, torch.as_tensor(rows, device="cuda")]), ra.astype(np.uint8))
        assert np.array_equal(host(as_[:, torch.as_tensor(rows, device="cuda")]).T, ras.astype(np.float32))
        r0 = g * N + blk * 128
        rw, rws = ob.quantize_128x128(_bits(w[r0:r0 + 128]))
        assert np.array_equal(kblocked_rows(wq[:, r0:r0 + 128]), rw.astype(np.uint8))
        assert np.array_equal(host(ws[r0 // 128:r0 // 128 + 1]), rws.astype(np.float32))
        wdeq = ob.dequantize_128x128(rw, rws)[cols - blk * 128]
        ref = ob.dequantize_1x128(ra, ras) @ wdeq.T
        gpu = host_bf16_f64(out[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")])
        # rms over the sampled block stands in for the whole output's rms
        assert_gemm_close(gpu, ref, what=f"c5 fwd expert {g}")


@pytest.mark.parametrize("mode", ["bf16-overwrite", "fp32-accumulate"])
@pytest.mark.parametrize("p2", [False, True], ids=["general", "pow2"])
def test_c5_full_size_wgrad_sampled(c5, p2, mode):
    G, M, K, N, sp, a = (c5[k] for k in ("G", "M", "K", "N", "sp", "a"))
    fmt = "fp8_1x128_p2" if p2 else "fp8_1x128"
    gen = torch.Generator(device="cuda").manual_seed(78)
    dy = torch.randn((M, N), generator=gen, device="cuda").to(torch.bfloat16)
    dq, ds, mpad = mxg.quantize_colwise_segpad(dy, sp, fmt)
    xq, xs, _ = mxg.quantize_colwise_segpad(a, sp, fmt)
    acc = mode == "fp32-accumulate"
    if acc:  # main_grad [G, N, K] fp32 (7.5 GB) accumulated in place
        out = torch.randn((G, N, K), generator=gen, device="cuda", dtype=torch.float32)
    else:
        out = torch.empty((G, N, K), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(6)
    picks = [(int(g), rng.choice(N, size=8, replace=False), rng.choice(K, size=8, replace=False))
             for g in rng.choice(np.nonzero(sp)[0], size=4, replace=False)]
    before = {g: host(out[g][torch.as_tensor(ns, device="cuda")][:, torch.as_tensor(ks, device="cuda")])
              for g, ns, ks in picks} if acc else {}
    mxg.grouped_wgrad(dq, ds, xq, xs, sp, N, K, mpad, out, accumulate=acc, fmt=fmt)
    torch.cuda.synchronize()
    row_offs, pad_offs = np.concatenate([[0], np.cumsum(sp)]), np.concatenate([[0], np.cumsum((sp + 127) // 128 * 128)])
    for g, ns, ks in picks:
        p0, p1 = int(pad_offs[g]), int(pad_offs[g + 1])
        r0, r1 = int(row_offs[g]), int(row_offs[g + 1])
        # oracle quantization of the expert's columns, compared with the library's
        rd, rds = ob.quantize_colwise_segpad_128(_bits(dy[r0:r1][:, torch.as_tensor(ns, device="cuda")]), [r1 - r0])
        rx, rxs = ob.quantize_colwise_segpad_128(_bits(a[r0:r1][:, torch.as_tensor(ks, device="cuda")]), [r1 - r0])
        assert np.array_equal(kblocked_rows(dq[p0 // 64:p1 // 64][:, torch.as_tensor(ns, device="cuda")]),
                              rd.astype(np.uint8))
        assert np.array_equal(host(xs[p0 // 128:p1 // 128][:, torch.as_tensor(ks, device="cuda")]).T,
                              rxs.astype(np.float32))
        ref = ob.dequantize_1x128(rd, rds) @ ob.dequantize_1x128(rx, rxs).T
        sample = out[g][torch.as_tensor(ns, device="cuda")][:, torch.as_tensor(ks, device="cuda")]
        if acc:
            ref = ref + before[g].astype(np.float64)
            gpu = host(sample).astype(np.float64)
        else:
            gpu = host_bf16_f64(sample)
        assert_gemm_close(gpu, ref, what=f"c5 wgrad {mode} expert {g}")
