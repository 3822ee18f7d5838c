"""GPU parity of the grouped GEMMs through the C ABI against the fp64 oracle on
the oracle's own quantized operands (tolerance 2^-7 |ref| + 1e-3 rms(ref)):
tiny and ragged shapes that span several tiles and partial tiles, empty
experts, short contractions, accumulate / overwrite, and a full-size sampled
check of each pass at the fc1 shapes."""
import numpy as np
import pytest

from oracle import grouped as og
from oracle import mx as omx
from synth import bf16_normal, f32_normal, splits_for

from .gpu_util import assert_gemm_close, dev_bf16, dev_f32, have_gpu, host, host_bf16_f64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import moe_grouped_block_mx_amd as mxg  # noqa: E402
import torch  # noqa: E402


def _fwd_case(splits, N, K, a_fmt, seed=0, w_std=0.05):
    splits = np.asarray(splits, dtype=np.int64)
    G, M = len(splits), int(splits.sum())
    a = bf16_normal((M, K), 1.0, seed=seed + 1)
    w = bf16_normal((G * N, K), w_std, seed=seed + 2)
    aq, as_ = mxg.quantize_rowwise(dev_bf16(a), a_fmt)
    wq, ws = mxg.quantize_rowwise(dev_bf16(w), "mxfp4")
    out = mxg.grouped_fwd(aq, as_, wq, ws, splits, N, K, a_fmt=a_fmt)
    torch.cuda.synchronize()
    ra, ras = omx.quantize_rowwise(a, a_fmt)
    rw, rws = omx.quantize_rowwise(w, "mxfp4")
    ref = og.grouped_fwd(omx.dequantize_rowwise(ra, ras, a_fmt),
                         omx.dequantize_rowwise(rw, rws, "mxfp4").reshape(G, N, K), splits)
    return host_bf16_f64(out), ref


FWD_CASES = [
    ([64, 0, 96, 96], 256, 256),        # the tiny config: an empty expert, partial tiles
    ([1], 32, 32),                       # one row, one block
    ([300, 0, 5], 192, 96),              # partial N tile, K tail inside a stage
    ([256], 128, 128),                   # single full M tile, one stage
    ([0, 0, 7], 64, 1024),               # leading empty experts
    ([513, 255, 1, 0, 40], 320, 352),    # several M tiles, N tail, K tail
    ([700, 333], 512, 4096),             # long contraction
    # every stage full (K % 128 == 0: the scalar-base DMA issue)
    ([513, 255, 1, 0, 40], 320, 384),    # several M tiles, N tail
    ([300, 0, 5], 192, 128),             # one stage, partial N tile
]


@pytest.mark.parametrize("a_fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("case", FWD_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in FWD_CASES])
def test_fwd(a_fmt, case):
    gpu, ref = _fwd_case(*case, a_fmt=a_fmt)
    assert_gemm_close(gpu, ref, what=f"fwd {a_fmt} {case}")


def test_fwd_many_experts_max_G():
    rng = np.random.default_rng(9)
    sp = rng.integers(0, 6, size=512)
    sp[rng.random(512) < 0.3] = 0
    gpu, ref = _fwd_case(sp, 64, 64, "mxfp4", seed=3)
    assert_gemm_close(gpu, ref, what="G=512")
    gpu, ref = _fwd_case(sp, 64, 128, "mxfp4", seed=4)     # every stage full
    assert_gemm_close(gpu, ref, what="G=512, K=128")


def test_fwd_empty_batch_writes_nothing():
    out = torch.full((0, 64), 1.0, dtype=torch.bfloat16, device="cuda")
    # block-major MX scales: [K/32 blocks, rows rounded up to a multiple of 4]
    aq = torch.empty((0, 32), dtype=torch.uint8, device="cuda")
    as_ = torch.empty((2, 0), dtype=torch.uint8, device="cuda")
    wq = torch.empty((128, 32), dtype=torch.uint8, device="cuda")
    ws = torch.empty((2, 128), dtype=torch.uint8, device="cuda")
    mxg.grouped_fwd(aq, as_, wq, ws, [0, 0], 64, 64, out=out)
    torch.cuda.synchronize()


def test_fwd_preallocated_output_and_determinism():
    sp = [100, 28]
    a = dev_bf16(bf16_normal((128, 256), 1.0, seed=1))
    w = dev_bf16(bf16_normal((2 * 64, 256), 0.05, seed=2))
    aq, as_ = mxg.quantize_rowwise(a)
    wq, ws = mxg.quantize_rowwise(w)
    out = torch.zeros((128, 64), dtype=torch.bfloat16, device="cuda")
    r = mxg.grouped_fwd(aq, as_, wq, ws, sp, 64, 256, out=out)
    assert r.data_ptr() == out.data_ptr()
    r2 = mxg.grouped_fwd(aq, as_, wq, ws, sp, 64, 256)
    torch.cuda.synchronize()
    assert torch.equal(out, r2)


def _dgrad_case(splits, N, K, seed=0):
    splits = np.asarray(splits, dtype=np.int64)
    G, M = len(splits), int(splits.sum())
    dy = bf16_normal((M, N), 1.0, seed=seed + 3)
    w = bf16_normal((G * N, K), 0.05, seed=seed + 2)
    dq, ds = mxg.quantize_rowwise(dev_bf16(dy), "mxfp4")
    wq, ws, _ = mxg.quantize_colwise_segpad(dev_bf16(w), [N] * G, "mxfp4")
    dx = mxg.grouped_dgrad(dq, ds, wq, ws, splits, N, K)
    torch.cuda.synchronize()
    rd, rds = omx.quantize_rowwise(dy, "mxfp4")
    rw, rws = omx.quantize_colwise_segpad(w, [N] * G, "mxfp4")
    ref = og.grouped_dgrad(omx.dequantize_rowwise(rd, rds, "mxfp4"), omx.dequantize_rowwise(rw, rws, "mxfp4"),
                           splits)
    return host_bf16_f64(dx), ref


DGRAD_CASES = [
    ([64, 0, 96, 96], 256, 256),
    ([300, 0, 5], 96, 192),           # contraction over N = 96: tail inside a stage
    ([513, 1, 0, 40], 384, 320),
    ([1], 32, 32),
]


@pytest.mark.parametrize("case", DGRAD_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in DGRAD_CASES])
def test_dgrad(case):
    gpu, ref = _dgrad_case(*case)
    assert_gemm_close(gpu, ref, what=f"dgrad {case}")


def _wgrad_case(splits, N, K, accumulate, seed=0):
    splits = np.asarray(splits, dtype=np.int64)
    G, M = len(splits), int(splits.sum())
    dy = bf16_normal((M, N), 1.0, seed=seed + 3)
    x = bf16_normal((M, K), 1.0, seed=seed + 1)
    dq, ds, mpad = mxg.quantize_colwise_segpad(dev_bf16(dy), splits, "mxfp4")
    xq, xs, _ = mxg.quantize_colwise_segpad(dev_bf16(x), splits, "mxfp4")
    main0 = f32_normal((G, N, K), seed=seed + 4)
    mg = dev_f32(main0)
    mxg.grouped_wgrad(dq, ds, xq, xs, splits, N, K, mpad, mg, accumulate=accumulate)
    torch.cuda.synchronize()
    rd, rds = omx.quantize_colwise_segpad(dy, splits, "mxfp4")
    rx, rxs = omx.quantize_colwise_segpad(x, splits, "mxfp4")
    ref = og.grouped_wgrad(omx.dequantize_rowwise(rd, rds, "mxfp4"), omx.dequantize_rowwise(rx, rxs, "mxfp4"),
                           splits, main_grad0=main0.astype(np.float64), accumulate=accumulate)
    return host(mg).astype(np.float64), ref, main0


WGRAD_CASES = [
    ([64, 0, 96, 96], 256, 256),
    ([33, 0, 1, 300], 96, 192),        # variable K incl. 32 and 320 (not a multiple of 128)
    ([0, 0, 0], 64, 64),               # all experts empty
    ([640, 40], 320, 288),             # N and K tails
    # 384 tiles: a quarter of the workgroups take two, those of odd XCDs in
    # reverse when accumulating (their segment cursor moves back)
    ([37, 250, 0, 128, 5, 299, 64, 1, 190, 33, 0, 256, 77, 140, 12, 288, 96, 0, 45, 210, 160, 3, 31, 129],
     1024, 1024),
]


@pytest.mark.parametrize("accumulate", [True, False])
@pytest.mark.parametrize("case", WGRAD_CASES, ids=[f"{len(c[0])}x{c[1]}x{c[2]}" for c in WGRAD_CASES])
def test_wgrad(case, accumulate):
    gpu, ref, main0 = _wgrad_case(*case, accumulate=accumulate)
    for g, m in enumerate(case[0]):
        if m == 0:
            if accumulate:   # untouched, bit for bit
                assert np.array_equal(gpu[g], main0[g].astype(np.float64)), f"expert {g} modified"
            else:            # zero-filled
                assert np.all(gpu[g] == 0), f"expert {g} not zeroed"
    if np.asarray(case[0]).sum():
        assert_gemm_close(gpu, ref, what=f"wgrad acc={accumulate} {case}")


def _max_g_splits(seed):
    """512 experts (the ABI's maximum), about 30 % of them empty, the others
    0..5 rows: every expert table in LDS is full and most tiles are partial."""
    rng = np.random.default_rng(seed)
    sp = rng.integers(0, 6, size=512)
    sp[rng.random(512) < 0.3] = 0
    return sp


def test_dgrad_many_experts_max_G():
    gpu, ref = _dgrad_case(_max_g_splits(10), 64, 96)
    assert_gemm_close(gpu, ref, what="dgrad G=512")


@pytest.mark.parametrize("accumulate", [True, False])
def test_wgrad_many_experts_max_G(accumulate):
    sp = _max_g_splits(11)
    gpu, ref, main0 = _wgrad_case(sp, 64, 96, accumulate=accumulate)
    empty = np.nonzero(sp == 0)[0]
    if accumulate:
        assert np.array_equal(gpu[empty], main0[empty].astype(np.float64)), "an empty expert was modified"
    else:
        assert np.all(gpu[empty] == 0), "an empty expert was not zero-filled"
    assert_gemm_close(gpu, ref, what=f"wgrad G=512 acc={accumulate}")


def test_error_paths_on_gpu():
    x = bf16_normal((32, 64), 1.0, seed=0)
    xd = dev_bf16(x)
    q = torch.empty((32, 32), dtype=torch.uint8)          # host memory: must be refused
    s = torch.empty((32, 2), dtype=torch.uint8, device="cuda")
    import ctypes
    st = mxg.lib.mxgg_quantize_rowwise(ctypes.c_void_p(xd.data_ptr()), 32, 64, 64, 0, 0,
                                       ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(s.data_ptr()), None)
    assert st == 7, mxg.lib.mxgg_last_error()
    # well-formed buffers (block-major scales), splits summing to 3 of 4 rows:
    # the library's own split check refuses the call
    with pytest.raises(mxg.MxggError, match="MXGG_ERR_SPLITS"):
        mxg.grouped_fwd(torch.empty((4, 32), dtype=torch.uint8, device="cuda"),
                        torch.empty((2, 4), dtype=torch.uint8, device="cuda"),
                        torch.empty((64, 32), dtype=torch.uint8, device="cuda"),
                        torch.empty((2, 64), dtype=torch.uint8, device="cuda"), [2, 1], 32, 64)


# ---------------------------------------------------------------------------
# full size, fc1 shapes (32 experts, 32768 rows, K=4096, N=3072), sampled
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def fc1():
    sp = splits_for("fc1")
    M, K, N, G = 32768, 4096, 3072, 32
    a = bf16_normal((M, K), 1.0, seed=1)
    w = bf16_normal((G * N, K), 0.02, seed=2)
    dy = bf16_normal((M, N), 1.0, seed=3)
    return dict(sp=sp, M=M, K=K, N=N, G=G, a=a, w=w, dy=dy,
                offs=np.concatenate([[0], np.cumsum(sp)]))


def _sample_rows_cols(fc1, nrow, ncol, seed):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(fc1["M"], size=nrow, replace=False))
    return rows, rng


def test_fc1_fwd_full_size_sampled(fc1):
    K, N, G = fc1["K"], fc1["N"], fc1["G"]
    aq, as_ = mxg.quantize_rowwise(dev_bf16(fc1["a"]))
    wq, ws = mxg.quantize_rowwise(dev_bf16(fc1["w"]))
    out = mxg.grouped_fwd(aq, as_, wq, ws, fc1["sp"], N, K)
    torch.cuda.synchronize()
    gout = host_bf16_f64(out)
    rows, rng = _sample_rows_cols(fc1, 256, 0, 10)
    cols = np.sort(rng.choice(N, size=64, replace=False))
    ra, ras = omx.quantize_rowwise(fc1["a"][rows], "mxfp4")
    A = omx.dequantize_rowwise(ra, ras, "mxfp4")
    experts = np.searchsorted(fc1["offs"], rows, side="right") - 1
    ref = np.empty((len(rows), len(cols)))
    for g in np.unique(experts):
        wr = fc1["w"][g * N + cols]
        rw, rws = omx.quantize_rowwise(wr, "mxfp4")
        Wg = omx.dequantize_rowwise(rw, rws, "mxfp4")
        sel = experts == g
        ref[sel] = A[sel] @ Wg.T
    assert_gemm_close(gout[np.ix_(rows, cols)], ref, what="fc1 fwd")


def test_fc1_dgrad_full_size_sampled(fc1):
    K, N, G = fc1["K"], fc1["N"], fc1["G"]
    dq, ds = mxg.quantize_rowwise(dev_bf16(fc1["dy"]))
    wq, ws, _ = mxg.quantize_colwise_segpad(dev_bf16(fc1["w"]), [N] * G, "mxfp4")
    dx = mxg.grouped_dgrad(dq, ds, wq, ws, fc1["sp"], N, K)
    torch.cuda.synchronize()
    gdx = host_bf16_f64(dx)
    rows, rng = _sample_rows_cols(fc1, 256, 0, 11)
    kcols = np.sort(rng.choice(K, size=64, replace=False))
    rd, rds = omx.quantize_rowwise(fc1["dy"][rows], "mxfp4")
    DY = omx.dequantize_rowwise(rd, rds, "mxfp4")
    experts = np.searchsorted(fc1["offs"], rows, side="right") - 1
    ref = np.empty((len(rows), len(kcols)))
    for g in np.unique(experts):
        # W_g quantized along N for the sampled K columns: rows of W^T
        wt = np.ascontiguousarray(fc1["w"][g * N:(g + 1) * N][:, kcols].T)
        rw, rws = omx.quantize_rowwise(wt, "mxfp4")
        WC = omx.dequantize_rowwise(rw, rws, "mxfp4")      # [len(kcols), N]
        sel = experts == g
        ref[sel] = DY[sel] @ WC.T
    assert_gemm_close(gdx[np.ix_(rows, kcols)], ref, what="fc1 dgrad")


@pytest.mark.parametrize("accumulate", [True, False], ids=["accumulate", "overwrite"])
def test_fc1_wgrad_full_size_sampled(fc1, accumulate):
    K, N, G, sp = fc1["K"], fc1["N"], fc1["G"], fc1["sp"]
    dq, ds, mpad = mxg.quantize_colwise_segpad(dev_bf16(fc1["dy"]), sp, "mxfp4")
    xq, xs, _ = mxg.quantize_colwise_segpad(dev_bf16(fc1["a"]), sp, "mxfp4")
    main0 = torch.randn((G, N, K), generator=torch.Generator(device="cuda").manual_seed(4),
                        device="cuda", dtype=torch.float32)
    m0 = {}
    rng = np.random.default_rng(12)
    experts = [g for g in range(G) if sp[g] > 0][::5] + [int(np.argmax(sp))]
    empty = [g for g in range(G) if sp[g] == 0]
    picks = {g: (np.sort(rng.choice(N, 16, replace=False)), np.sort(rng.choice(K, 16, replace=False)))
             for g in experts}
    for g, (ns, ks) in picks.items():
        m0[g] = host(main0[g][np.ix_(ns, ks)]).astype(np.float64)
    e0 = {g: host(main0[g][:8, :8]) for g in empty}
    mxg.grouped_wgrad(dq, ds, xq, xs, sp, N, K, mpad, main0, accumulate=accumulate)
    torch.cuda.synchronize()
    for g in empty:  # experts without tokens: untouched when accumulating, zero-filled when overwriting
        assert np.array_equal(host(main0[g][:8, :8]), e0[g] if accumulate else np.zeros((8, 8), np.float32)), g
    offs = fc1["offs"]
    gpu_all, ref_all = [], []
    for g, (ns, ks) in picks.items():
        seg = slice(offs[g], offs[g + 1])
        rd, rds = omx.quantize_colwise_segpad(np.ascontiguousarray(fc1["dy"][seg][:, ns]), [sp[g]], "mxfp4")
        rx, rxs = omx.quantize_colwise_segpad(np.ascontiguousarray(fc1["a"][seg][:, ks]), [sp[g]], "mxfp4")
        ref = og.grouped_wgrad(omx.dequantize_rowwise(rd, rds, "mxfp4"), omx.dequantize_rowwise(rx, rxs, "mxfp4"),
                               [sp[g]], main_grad0=m0[g][None], accumulate=accumulate)[0]
        gpu_all.append(host(main0[g][np.ix_(ns, ks)]).astype(np.float64))
        ref_all.append(ref)
    assert_gemm_close(np.stack(gpu_all), np.stack(ref_all), what=f"fc1 wgrad accumulate={accumulate}")
