"""GPU parity of the dual-output quantizers (row-wise and column-wise
segment-padded outputs from one read) through the C ABI, MX and blockwise
1x128: bit-exact against the oracle's two quantizations and against the
library's separate row-wise and column-wise kernels, on ragged and unaligned
expert segments, column tails, strided inputs, empty experts, the largest
expert count, special blocks, and the full-size fc1 and blockwise-workload
activations and fc1 weights (equality with the separate kernels everywhere,
the oracle on sampled rows and columns)."""
import numpy as np
import pytest

from oracle import mx as omx
from synth import bf16_normal, splits_for

from .gpu_util import dev_bf16, have_gpu, host, kblocked_rows, mx_scales_rowmajor

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import moe_grouped_block_mx_amd as mxg  # noqa: E402
import torch  # noqa: E402


def _separate(x, splits, fmt):
    q, s = mxg.quantize_rowwise(x, fmt)
    qc, sc, mpad = mxg.quantize_colwise_segpad(x, splits, fmt)
    return q, s, qc, sc, mpad


def _check(bits, splits, fmt, what, x=None):
    x = dev_bf16(bits) if x is None else x
    qr, sr, qc, sc, mpad = mxg.quantize_dual(x, splits, fmt)
    q2, s2, qc2, sc2, mpad2 = _separate(x, splits, fmt)
    torch.cuda.synchronize()
    assert mpad == mpad2
    for name, a, b in (("q_row", qr, q2), ("s_row", sr, s2), ("q_col", qc, qc2), ("s_col", sc, sc2)):
        assert torch.equal(a, b), f"{what}: {name} differs from the separate kernel"
    rq, rs = omx.quantize_rowwise(bits, fmt)
    assert np.array_equal(host(qr), rq), f"{what}: row-wise data vs oracle"
    assert np.array_equal(mx_scales_rowmajor(sr, bits.shape[0]), rs), f"{what}: row-wise scales vs oracle"
    cq, cs = omx.quantize_colwise_segpad(bits, splits, fmt)
    assert np.array_equal(host(qc), cq), f"{what}: column-wise data vs oracle"
    assert np.array_equal(mx_scales_rowmajor(sc, bits.shape[1]), cs), f"{what}: column-wise scales vs oracle"


CASES = [
    ([64, 0, 96, 96], 256),            # the tiny config
    ([1], 32),                          # one row, one block
    ([300, 0, 5], 96),                  # rows % 4 != 0 (scale padding), one partial column tile
    ([513, 255, 1, 0, 40], 352),        # unaligned segment starts, column tail of 96
    ([0, 0, 7], 544),                   # leading empty experts, three column tiles
    ([33, 31, 32, 95], 288),            # segments straddling 128-row tiles
]


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("case", CASES, ids=[f"{len(c[0])}x{c[1]}" for c in CASES])
def test_dual_matches_oracle_and_separate_kernels(fmt, case):
    splits, cols = case
    rows = int(np.sum(splits))
    bits = bf16_normal((rows, cols), 1.0, seed=7)
    _check(bits, splits, fmt, f"{fmt} {case}")


def test_dual_strided_input():
    wide = bf16_normal((200, 400), 1.0, seed=3)
    x = dev_bf16(wide)[:, 16:336]                     # ldx = 400, cols = 320
    _check(np.ascontiguousarray(wide[:, 16:336]), [70, 0, 130], "mxfp4", "strided", x=x)


def test_dual_many_experts_max_G():
    rng = np.random.default_rng(11)
    sp = rng.integers(0, 9, size=512)
    sp[rng.random(512) < 0.3] = 0
    bits = bf16_normal((int(sp.sum()), 64), 1.0, seed=5)
    _check(bits, sp, "mxfp4", "G=512")


def test_dual_special_blocks():
    # outliers, all-zero blocks and tiny values inside both block directions
    bits = bf16_normal((96, 128), 1.0, seed=2)
    bits[5, :] = 0
    bits[:, 40:72] = 0
    bits[17, 3] = 0x7F00        # a large outlier (bf16 ~1.7e38)
    bits[60:92, 100] = 0x0080   # smallest normal bf16
    _check(bits, [40, 56], "mxfp4", "special")
    _check(bits, [40, 56], "mxfp8", "special fp8")


def test_dual_empty_batch():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    qr, sr, qc, sc, mpad = mxg.quantize_dual(x, [0, 0], "mxfp4")
    torch.cuda.synchronize()
    assert mpad == 0 and qr.numel() == 0 and qc.numel() == 0


def test_dual_full_size_fc1_activations_sampled():
    """X at the fc1 size (32768 x 4096, fc1 routing): equal to the separate
    kernels everywhere; the oracle on 512 sampled rows and 32 sampled columns."""
    sp = splits_for("fc1")
    bits = bf16_normal((32768, 4096), 1.0, seed=1)
    x = dev_bf16(bits)
    qr, sr, qc, sc, mpad = mxg.quantize_dual(x, sp, "mxfp4")
    q2, s2, qc2, sc2, _ = _separate(x, sp, "mxfp4")
    torch.cuda.synchronize()
    assert torch.equal(qr, q2) and torch.equal(sr, s2) and torch.equal(qc, qc2) and torch.equal(sc, sc2)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(32768, size=512, replace=False))
    rq, rs = omx.quantize_rowwise(bits[rows], "mxfp4")
    assert np.array_equal(host(qr)[rows], rq) and np.array_equal(mx_scales_rowmajor(sr, 32768)[rows], rs)
    cols = np.sort(rng.choice(4096, size=32, replace=False))
    cq, cs = omx.quantize_colwise_segpad(np.ascontiguousarray(bits[:, cols]), sp, "mxfp4")
    assert np.array_equal(host(qc)[cols], cq) and np.array_equal(mx_scales_rowmajor(sc, 4096)[cols], cs)


def test_dual_full_size_fc1_weights_equal_separate():
    """W as [32*3072, 4096] with splits [3072]*32: the forward's row-wise W and
    dgrad's W along N in one pass, equal to the separate kernels."""
    G, N, K = 32, 3072, 4096
    x = dev_bf16(bf16_normal((G * N, K), 0.02, seed=2))
    sp = [N] * G
    got = mxg.quantize_dual(x, sp, "mxfp4")
    ref = _separate(x, sp, "mxfp4")
    torch.cuda.synchronize()
    assert got[4] == ref[4] == G * N
    for a, b in zip(got[:4], ref[:4]):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# blockwise FP8 dual (1x128 row-wise + 1x128 column-wise segment-padded to 128)
# ---------------------------------------------------------------------------
from oracle import blockwise as ob  # noqa: E402

BLK_CASES = [
    ([64, 0, 96, 96], 256),             # segments shorter than a 128-row block
    ([300, 0, 5], 128),                 # one column tile; a block straddled by nothing
    ([513, 255, 1, 0, 40], 384),        # unaligned segment starts, three column tiles
    ([0, 0, 7], 128),                   # leading empty experts
    ([129, 127, 128], 256),             # a segment one row past / one short of a block
]


def _check_blk(bits, splits, fmt, what, x=None):
    x = dev_bf16(bits) if x is None else x
    pow2 = fmt.endswith("_p2")
    qr, sr, qc, sc, mpad = mxg.quantize_dual(x, splits, fmt, flags=1 if pow2 else 0)
    q2, s2 = mxg.quantize_rowwise(x, fmt, flags=1 if pow2 else 0)
    qc2, sc2, mpad2 = mxg.quantize_colwise_segpad(x, splits, fmt, flags=1 if pow2 else 0)
    torch.cuda.synchronize()
    assert mpad == mpad2
    for name, a, b in (("q_row", qr, q2), ("s_row", sr, s2), ("q_col", qc, qc2), ("s_col", sc, sc2)):
        assert torch.equal(a, b), f"{what}: {name} differs from the separate kernel"
    rq, rs = ob.quantize_1x128(bits, pow2=pow2)
    # 1x128 scales are block-major: the oracle's [rows, blocks] transposed
    assert np.array_equal(kblocked_rows(qr), rq) and np.array_equal(host(sr).T, rs), f"{what}: row-wise vs oracle"
    cq, cs = ob.quantize_colwise_segpad_128(bits, splits, pow2=pow2)
    assert np.array_equal(kblocked_rows(qc), cq) and np.array_equal(host(sc).T, cs), f"{what}: column-wise vs oracle"


@pytest.mark.parametrize("fmt", ["fp8_1x128_p2", "fp8_1x128"])
@pytest.mark.parametrize("case", BLK_CASES, ids=[f"{len(c[0])}x{c[1]}" for c in BLK_CASES])
def test_blockwise_dual_matches_oracle_and_separate_kernels(fmt, case):
    splits, cols = case
    bits = bf16_normal((int(np.sum(splits)), cols), 1.0, seed=13)
    _check_blk(bits, splits, fmt, f"{fmt} {case}")


def test_blockwise_dual_special_and_strided():
    bits = bf16_normal((200, 256), 1.0, seed=4)
    bits[7, :] = 0                       # an all-zero row block: the amax floor
    bits[:, 130:140] = 0x0080            # tiny values
    bits[150, 3] = 0x7F00                # a huge outlier
    _check_blk(bits, [90, 0, 110], "fp8_1x128_p2", "special")
    _check_blk(bits, [90, 0, 110], "fp8_1x128", "special fp32 scales")
    wide = bf16_normal((160, 512), 1.0, seed=6)
    x = dev_bf16(wide)[:, 128:384]
    _check_blk(np.ascontiguousarray(wide[:, 128:384]), [100, 60], "fp8_1x128_p2", "strided", x=x)


def test_blockwise_dual_full_size_sampled():
    """X at the blockwise workload's size (32768 x 7168, uniform-random
    routing over 64 experts): equal to the separate kernels everywhere; the
    oracle on 256 sampled rows and 16 sampled columns."""
    sp = splits_for("blockwise")
    bits = bf16_normal((32768, 7168), 1.0, seed=1)
    x = dev_bf16(bits)
    qr, sr, qc, sc, mpad = mxg.quantize_dual(x, sp, "fp8_1x128_p2")
    q2, s2 = mxg.quantize_rowwise(x, "fp8_1x128_p2")
    qc2, sc2, _ = mxg.quantize_colwise_segpad(x, sp, "fp8_1x128_p2")
    torch.cuda.synchronize()
    assert torch.equal(qr, q2) and torch.equal(sr, s2) and torch.equal(qc, qc2) and torch.equal(sc, sc2)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(32768, size=256, replace=False))
    rq, rs = ob.quantize_1x128(bits[rows])
    assert np.array_equal(kblocked_rows(qr[:, torch.as_tensor(rows, device="cuda")]), rq)
    assert np.array_equal(host(sr)[:, rows].T, rs)
    cols = np.sort(rng.choice(7168, size=16, replace=False))
    cq, cs = ob.quantize_colwise_segpad_128(np.ascontiguousarray(bits[:, cols]), sp)
    assert np.array_equal(kblocked_rows(qc[:, torch.as_tensor(cols, device="cuda")]), cq)
    assert np.array_equal(host(sc)[:, cols].T, cs)
