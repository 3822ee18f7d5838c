"""GPU parity of the backward variants beyond a4w4 through the C ABI, against
the fp64 oracle on the oracle's own quantized operands (tolerance
2^-7 |ref| + 1e-3 rms(ref)):

- a8w4 input gradient: dY in MXFP8 (E4M3, UE8M0 per 32) x W column-wise MXFP4;
- MXFP8 weight gradient: both column-wise segment-padded operands in MXFP8;
- blockwise FP8 input gradient: dY 1x128 x the transposed 128x128 weight
  blocks (same codes, same scales), general and power-of-two (_P2) scales;
- the 128x128 block transpose itself, bit-exact;
- sampled full-size checks at the a8w4 shapes (128 experts, 65536 rows,
  K=7168, N=2048; forward and input gradient) and the blockwise shapes (64
  experts, 32768 rows, K=7168, N=4096).
"""
import numpy as np
import pytest

from oracle import blockwise as ob
from oracle import grouped as og
from oracle import mx as omx
from synth import bf16_normal, f32_normal, splits_for

from .gpu_util import assert_gemm_close, dev_bf16, dev_f32, have_gpu, host, host_bf16_f64, kblocked_rows

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import moe_grouped_block_mx_amd as mxg  # noqa: E402
import torch  # noqa: E402


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# a8w4 input gradient
# ---------------------------------------------------------------------------
DGRAD_CASES = [
    ([64, 0, 96, 96], 256, 256),
    ([300, 0, 5], 96, 192),           # contraction over N = 96: a tail inside a stage
    ([513, 1, 0, 40], 384, 320),      # several M tiles, K tail
    ([1], 32, 32),
]


@pytest.mark.parametrize("case", DGRAD_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in DGRAD_CASES])
def test_dgrad_a8w4(case):
    splits, N, K = case
    splits = np.asarray(splits, dtype=np.int64)
    G, M = len(splits), int(splits.sum())
    dy = bf16_normal((M, N), 1.0, seed=13)
    w = bf16_normal((G * N, K), 0.05, seed=12)
    dq, ds = mxg.quantize_rowwise(dev_bf16(dy), "mxfp8")
    wq, ws, _ = mxg.quantize_colwise_segpad(dev_bf16(w), [N] * G, "mxfp4")
    dx = mxg.grouped_dgrad(dq, ds, wq, ws, splits, N, K, fmt="mxfp8")
    torch.cuda.synchronize()
    rd, rds = omx.quantize_rowwise(dy, "mxfp8")
    rw, rws = omx.quantize_colwise_segpad(w, [N] * G, "mxfp4")
    ref = og.grouped_dgrad(omx.dequantize_rowwise(rd, rds, "mxfp8"), omx.dequantize_rowwise(rw, rws, "mxfp4"),
                           splits)
    assert_gemm_close(host_bf16_f64(dx), ref, what=f"a8w4 dgrad {case}")


# ---------------------------------------------------------------------------
# MXFP8 weight gradient
# ---------------------------------------------------------------------------
WGRAD_CASES = [
    ([64, 0, 96, 96], 256, 256),      # an empty expert; with overwrite, a workgroup of empty tiles only
    ([33, 0, 1, 300], 96, 192),       # variable K incl. 32 and 320 (not a multiple of 64)
    ([0, 0, 0], 64, 64),              # all experts empty
    ([640, 40], 320, 288),            # N and K tails
]


@pytest.mark.parametrize("accumulate", [True, False])
@pytest.mark.parametrize("case", WGRAD_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in WGRAD_CASES])
def test_wgrad_mxfp8(case, accumulate):
    splits, N, K = case
    splits = np.asarray(splits, dtype=np.int64)
    G, M = len(splits), int(splits.sum())
    dy = bf16_normal((M, N), 1.0, seed=23)
    x = bf16_normal((M, K), 1.0, seed=21)
    dq, ds, mpad = mxg.quantize_colwise_segpad(dev_bf16(dy), splits, "mxfp8")
    xq, xs, _ = mxg.quantize_colwise_segpad(dev_bf16(x), splits, "mxfp8")
    main0 = f32_normal((G, N, K), seed=24)
    mg = dev_f32(main0)
    mxg.grouped_wgrad(dq, ds, xq, xs, splits, N, K, mpad, mg, accumulate=accumulate, fmt="mxfp8")
    torch.cuda.synchronize()
    gpu = host(mg).astype(np.float64)
    rd, rds = omx.quantize_colwise_segpad(dy, splits, "mxfp8")
    rx, rxs = omx.quantize_colwise_segpad(x, splits, "mxfp8")
    ref = og.grouped_wgrad(omx.dequantize_rowwise(rd, rds, "mxfp8"), omx.dequantize_rowwise(rx, rxs, "mxfp8"),
                           splits, main_grad0=main0.astype(np.float64), accumulate=accumulate)
    for g, m in enumerate(splits):
        if m == 0:
            if accumulate:
                assert np.array_equal(gpu[g], main0[g].astype(np.float64)), f"expert {g} modified"
            else:
                assert np.all(gpu[g] == 0), f"expert {g} not zeroed"
    if splits.sum():
        assert_gemm_close(gpu, ref, what=f"mxfp8 wgrad acc={accumulate} {case}")


# ---------------------------------------------------------------------------
# 128x128 block transpose and the blockwise input gradient
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("G,N,K", [(1, 128, 128), (3, 256, 384), (2, 640, 128)])
def test_transpose_128x128_bit_exact(G, N, K):
    w = bf16_normal((G * N, K), 0.05, seed=31)
    wq, ws = mxg.quantize_rowwise(dev_bf16(w), "fp8_128x128")
    tq, ts = mxg.transpose_128x128(wq, ws, G, N, K)
    torch.cuda.synchronize()
    # codes in 64-byte K blocks on both sides: compared as rows
    q, s = kblocked_rows(wq).reshape(G, N, K), host(ws).reshape(G, N // 128, K // 128)
    assert np.array_equal(kblocked_rows(tq), q.transpose(0, 2, 1).reshape(G * K, N))
    assert np.array_equal(host(ts), s.transpose(0, 2, 1).reshape(G * K // 128, N // 128))
    # and the transposed blocks are the oracle's 128x128 quantization of W^T
    wt = np.ascontiguousarray(w.reshape(G, N, K).transpose(0, 2, 1).reshape(G * K, N))
    rq, rs = ob.quantize_128x128(wt)
    assert np.array_equal(kblocked_rows(tq), rq.astype(np.uint8))
    assert np.array_equal(host(ts), rs.astype(np.float32))


BLK_DGRAD_CASES = [
    ([64, 0, 96, 96], 256, 256),
    ([300, 0, 5], 128, 384),          # one N block, K tail of a 256-wide tile
    ([129, 1, 255, 0, 40], 384, 128),
]


@pytest.mark.parametrize("fmt", ["fp8_1x128", "fp8_1x128_p2"])
@pytest.mark.parametrize("case", BLK_DGRAD_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in BLK_DGRAD_CASES])
def test_dgrad_blockwise(case, fmt):
    splits, N, K = case
    splits = np.asarray(splits, dtype=np.int64)
    G, M = len(splits), int(splits.sum())
    dy = bf16_normal((M, N), 1.0, seed=43)
    w = bf16_normal((G * N, K), 0.05, seed=42)
    # the general format with general fp32 scales (the per-128 partial
    # path); the _P2 formats with power-of-two scales (applied by the MFMA)
    p2 = fmt.endswith("_p2")
    wfmt = "fp8_128x128_p2" if p2 else "fp8_128x128"
    flags = None if p2 else 0
    dq, ds = mxg.quantize_rowwise(dev_bf16(dy), fmt, flags=flags)
    wq, ws = mxg.quantize_rowwise(dev_bf16(w), wfmt, flags=flags)
    tq, ts = mxg.transpose_128x128(wq, ws, G, N, K)
    dx = mxg.grouped_dgrad(dq, ds, tq, ts, splits, N, K, fmt=fmt)
    torch.cuda.synchronize()
    rd, rds = ob.quantize_1x128(dy, pow2=p2)
    rw, rws = ob.quantize_128x128(w, pow2=p2)
    assert np.array_equal(kblocked_rows(dq), rd.astype(np.uint8)) and np.array_equal(host(ds).T, rds.astype(np.float32))
    W = ob.dequantize_128x128(rw, rws).reshape(G, N, K)
    # dx = dY_g . W_g: the forward's contraction with W_g^T as the weight
    ref = og.grouped_fwd(ob.dequantize_1x128(rd, rds), np.ascontiguousarray(W.transpose(0, 2, 1)), splits)
    assert_gemm_close(host_bf16_f64(dx), ref, what=f"blockwise dgrad {fmt} {case}")


# ---------------------------------------------------------------------------
# full size, sampled
# ---------------------------------------------------------------------------
def test_a8w4_full_size_fwd_sampled():
    """a8w4 forward at its workload's shapes and launch (128 experts, 65536
    rows, Zipf splits with empty experts, K=7168, N=2048; activations MXFP8,
    weights MXFP4): sampled rows of five random experts and the largest one,
    16 sampled output columns each, against the oracle's quantize-dequantize
    and fp64 contraction."""
    from synth import WORKLOADS
    wl = WORKLOADS["a8w4"]
    G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
    sp = splits_for("a8w4")
    gen = torch.Generator(device="cuda").manual_seed(93)
    a = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((G * N, K), generator=gen, device="cuda") * wl["w_std"]).to(torch.bfloat16)
    aq, as_ = mxg.quantize_rowwise(a, "mxfp8")
    wq, ws = mxg.quantize_rowwise(w, "mxfp4")
    out = mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt="mxfp8", w_fmt="mxfp4")
    torch.cuda.synchronize()
    rng = np.random.default_rng(94)
    offs = np.concatenate([[0], np.cumsum(sp)])
    nz = np.nonzero(sp)[0]
    for g in list(rng.choice(nz, size=5, replace=False)) + [int(np.argmax(sp))]:
        rows = offs[g] + np.sort(rng.choice(sp[g], size=min(8, sp[g]), replace=False))
        cols = np.sort(rng.choice(N, size=16, replace=False))
        ra, ras = omx.quantize_rowwise(_bits(a[torch.as_tensor(rows, device="cuda")]), "mxfp8")
        rw, rws = omx.quantize_rowwise(_bits(w[torch.as_tensor(g * N + cols, device="cuda")]), "mxfp4")
        ref = omx.dequantize_rowwise(ra, ras, "mxfp8") @ omx.dequantize_rowwise(rw, rws, "mxfp4").T
        gpu = host_bf16_f64(out[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")])
        assert_gemm_close(gpu, ref, what=f"a8w4 fwd expert {g}")


def test_a8w4_full_size_dgrad_sampled():
    """a8w4 input gradient at the a8w4 shapes (128 experts, 65536 rows, Zipf
    splits with empty experts; N=2048 contracted, K=7168 out)."""
    from synth import WORKLOADS
    wl = WORKLOADS["a8w4"]
    G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
    sp = splits_for("a8w4")
    gen = torch.Generator(device="cuda").manual_seed(91)
    dy = torch.randn((M, N), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((G * N, K), generator=gen, device="cuda") * wl["w_std"]).to(torch.bfloat16)
    dq, ds = mxg.quantize_rowwise(dy, "mxfp8")
    wq, ws, _ = mxg.quantize_colwise_segpad(w, [N] * G, "mxfp4")
    dx = mxg.grouped_dgrad(dq, ds, wq, ws, sp, N, K, fmt="mxfp8")
    torch.cuda.synchronize()
    rng = np.random.default_rng(92)
    offs = np.concatenate([[0], np.cumsum(sp)])
    nz = np.nonzero(sp)[0]
    for g in list(rng.choice(nz, size=5, replace=False)) + [int(np.argmax(sp))]:
        rows = offs[g] + np.sort(rng.choice(sp[g], size=min(8, sp[g]), replace=False))
        kcols = np.sort(rng.choice(K, size=16, replace=False))
        rt = torch.as_tensor(rows, device="cuda")
        rd, rds = omx.quantize_rowwise(_bits(dy[rt]), "mxfp8")
        # W_g along N for the sampled output columns: rows of W_g^T
        wt = _bits(w[g * N:(g + 1) * N][:, torch.as_tensor(kcols, device="cuda")].t().contiguous())
        rw, rws = omx.quantize_rowwise(wt, "mxfp4")
        ref = omx.dequantize_rowwise(rd, rds, "mxfp8") @ omx.dequantize_rowwise(rw, rws, "mxfp4").T
        gpu = host_bf16_f64(dx[rt][:, torch.as_tensor(kcols, device="cuda")])
        assert_gemm_close(gpu, ref, what=f"a8w4 dgrad expert {g}")


def test_a8w4_full_size_mxfp8_wgrad_sampled():
    """MXFP8 weight gradient at the a8w4 shapes (128 experts, 65536 rows, Zipf
    splits with empty experts; [128, 2048, 7168] fp32 main_grad accumulated in
    place): 16 x 16 sampled entries of every eighth nonempty expert and the
    largest, against the oracle's column-wise segment-padded quantization of
    the expert's rows and an fp64 contraction plus the old values."""
    from synth import WORKLOADS
    wl = WORKLOADS["a8w4"]
    G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
    sp = splits_for("a8w4")
    gen = torch.Generator(device="cuda").manual_seed(95)
    x = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    dy = torch.randn((M, N), generator=gen, device="cuda").to(torch.bfloat16)
    dq, ds, mpad = mxg.quantize_colwise_segpad(dy, sp, "mxfp8")
    xq, xs, _ = mxg.quantize_colwise_segpad(x, sp, "mxfp8")
    main0 = torch.randn((G, N, K), generator=gen, device="cuda", dtype=torch.float32)
    rng = np.random.default_rng(96)
    nz = [g for g in range(G) if sp[g] > 0]
    picks = {g: (np.sort(rng.choice(N, 16, replace=False)), np.sort(rng.choice(K, 16, replace=False)))
             for g in nz[::8] + [int(np.argmax(sp))]}
    m0 = {g: host(main0[g][np.ix_(ns, ks)]).astype(np.float64) for g, (ns, ks) in picks.items()}
    mxg.grouped_wgrad(dq, ds, xq, xs, sp, N, K, mpad, main0, fmt="mxfp8", accumulate=True)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(sp)])
    gpu_all, ref_all = [], []
    for g, (ns, ks) in picks.items():
        seg = torch.arange(int(offs[g]), int(offs[g + 1]), device="cuda")
        dyg = _bits(dy[seg][:, torch.as_tensor(ns, device="cuda")].contiguous())
        xg = _bits(x[seg][:, torch.as_tensor(ks, device="cuda")].contiguous())
        rd, rds = omx.quantize_colwise_segpad(dyg, [sp[g]], "mxfp8")
        rx, rxs = omx.quantize_colwise_segpad(xg, [sp[g]], "mxfp8")
        ref = og.grouped_wgrad(omx.dequantize_rowwise(rd, rds, "mxfp8"), omx.dequantize_rowwise(rx, rxs, "mxfp8"),
                               [sp[g]], main_grad0=m0[g][None], accumulate=True)[0]
        gpu_all.append(host(main0[g][np.ix_(ns, ks)]).astype(np.float64))
        ref_all.append(ref)
    assert_gemm_close(np.stack(gpu_all), np.stack(ref_all), what="a8w4 MXFP8 wgrad accumulate")


@pytest.mark.parametrize("p2", [False, True], ids=["general", "pow2"])
def test_blockwise_full_size_dgrad_sampled(p2):
    """Blockwise input gradient at the blockwise shapes (64 experts, 32768
    rows; N=4096 contracted, K=7168 out) through the weight transpose."""
    from synth import WORKLOADS
    wl = WORKLOADS["blockwise"]
    G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
    sp = splits_for("blockwise")
    gen = torch.Generator(device="cuda").manual_seed(93)
    dy = torch.randn((M, N), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((G * N, K), generator=gen, device="cuda") * wl["w_std"]).to(torch.bfloat16)
    af, wf = ("fp8_1x128_p2", "fp8_128x128_p2") if p2 else ("fp8_1x128", "fp8_128x128")
    dq, ds = mxg.quantize_rowwise(dy, af)
    wq, ws = mxg.quantize_rowwise(w, wf)
    del w
    tq, ts = mxg.transpose_128x128(wq, ws, G, N, K)
    dx = mxg.grouped_dgrad(dq, ds, tq, ts, sp, N, K, fmt=af)
    torch.cuda.synchronize()
    rng = np.random.default_rng(94)
    offs = np.concatenate([[0], np.cumsum(sp)])
    nz = np.nonzero(sp)[0]
    for g in rng.choice(nz, size=5, replace=False):
        rows = offs[g] + np.sort(rng.choice(sp[g], size=min(8, sp[g]), replace=False))
        kb = int(rng.integers(0, K // 128))
        kcols = kb * 128 + np.sort(rng.choice(128, size=16, replace=False))
        rt = torch.as_tensor(rows, device="cuda")
        rd, rds = ob.quantize_1x128(_bits(dy[rt]))
        assert np.array_equal(kblocked_rows(dq[:, rt]), rd.astype(np.uint8))
        # the library's transposed codes and scales of the sampled columns,
        # dequantized by the oracle's rule: W^T[k, n] = code * scale[k/128, n/128]
        ct = kblocked_rows(tq[:, g * K + torch.as_tensor(kcols, device="cuda")])
        st = host(ts[g * K // 128 + kb])
        assert np.array_equal(ct, kblocked_rows(wq[:, g * N:(g + 1) * N])[:, kcols].T)
        assert np.array_equal(st, host(ws[g * N // 128:(g + 1) * N // 128, kb]))
        Wt = ob.dequantize_1x128(ct, np.broadcast_to(st, (len(kcols), N // 128)))
        ref = ob.dequantize_1x128(rd, rds) @ Wt.T
        gpu = host_bf16_f64(dx[rt][:, torch.as_tensor(kcols, device="cuda")])
        assert_gemm_close(gpu, ref, what=f"blockwise dgrad expert {g}")
