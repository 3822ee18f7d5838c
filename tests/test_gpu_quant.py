"""GPU parity of the MX quantizers through the C ABI: bit-exact against the
oracle on every finite bf16 pattern, special blocks, ragged shapes, strided
inputs, segment-padded layouts and a full-size sampled check. The library's MX
scales are block-major ([blocks, rows rounded up to a multiple of 4], padding
rows zero); they are compared with the oracle's row-major scales after a
transpose."""
import numpy as np
import pytest

from oracle import mx as omx
from synth import bf16_normal, fp32_to_bf16_bits, splits_for

from .gpu_util import dev_bf16, have_gpu, host, mx_scales_rowmajor

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import moe_grouped_block_mx_amd as mxg  # noqa: E402


def _check_rowwise(bits, fmt, what):
    x = dev_bf16(bits)
    q, s = mxg.quantize_rowwise(x, fmt)
    rq, rs = omx.quantize_rowwise(bits, fmt)
    gq, gs = host(q), mx_scales_rowmajor(s, bits.shape[0])
    bad_s = np.argwhere(gs != rs)
    assert bad_s.size == 0, f"{what}: scale mismatch at {bad_s[:4].tolist()}"
    bad_q = np.argwhere(gq != rq)
    assert bad_q.size == 0, f"{what}: data mismatch at {bad_q[:4].tolist()}"


def _finite_patterns():
    p = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return p[((p >> 7) & 0xFF) != 0xFF]


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_rowwise_every_bf16_pattern(fmt):
    p = _finite_patterns()
    rng = np.random.default_rng(0)
    n = -(-p.size // 256) * 256
    a = np.zeros(n, dtype=np.uint16)
    a[:p.size] = rng.permutation(p)                       # mixed magnitudes per block
    _check_rowwise(a.reshape(-1, 256), fmt, "permuted")
    b = np.zeros(n, dtype=np.uint16)
    b[:p.size] = p[np.argsort(p & 0x7FFF, kind="stable")]  # similar magnitudes per block
    _check_rowwise(b.reshape(-1, 256), fmt, "sorted")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_rowwise_special_blocks(fmt):
    blocks = []
    z = np.zeros(32, np.uint16)
    blocks.append(z)                                          # all +0
    blocks.append(np.full(32, 0x8000, np.uint16))             # all -0
    t = z.copy(); t[0] = 0x0080; blocks.append(t)              # amax 2^-126 (worked example)
    t = z.copy(); t[5] = 0x0001; t[6] = 0x8001; blocks.append(t)  # smallest subnormals
    t = np.full(32, 0x7F7F, np.uint16); t[1::2] = 0xFF7F; blocks.append(t)  # +-bf16 max
    ties = np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4, np.float32)
    blocks.append(fp32_to_bf16_bits(ties))                    # E2M1 midpoints at scale 2^0
    t8 = np.array([256.0, 1 + 1 / 16, 1 + 3 / 16, 2 ** -10, 3 * 2 ** -10, 7.5, 9.0, 17.0] * 4, np.float32)
    blocks.append(fp32_to_bf16_bits(t8))                      # E4M3 midpoints
    one = z.copy(); one[31] = 0x3F80; blocks.append(one)       # single element
    _check_rowwise(np.stack(blocks).reshape(-1, 64), fmt, "special")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("shape", [(256, 256), (333, 96), (1, 32), (7, 4096)])
def test_rowwise_random(fmt, shape):
    bits = bf16_normal(shape, 1.0, seed=sum(shape))
    _check_rowwise(bits, fmt, f"{shape}")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_rowwise_strided_input(fmt):
    wide = bf16_normal((100, 200), 1.0, seed=3)
    x = dev_bf16(wide)[:, 8:168]                               # ldx = 200, cols = 160
    q, s = mxg.quantize_rowwise(x, fmt)
    rq, rs = omx.quantize_rowwise(np.ascontiguousarray(wide[:, 8:168]), fmt)
    assert np.array_equal(host(q), rq) and np.array_equal(mx_scales_rowmajor(s, 100), rs)


def _check_colwise(bits, splits, fmt, what):
    x = dev_bf16(bits)
    q, s, mpad = mxg.quantize_colwise_segpad(x, splits, fmt)
    rq, rs = omx.quantize_colwise_segpad(bits, splits, fmt)
    assert mpad == rq.shape[1] * (2 if fmt == "mxfp4" else 1)
    gq, gs = host(q), mx_scales_rowmajor(s, bits.shape[1])
    assert np.array_equal(gs, rs), f"{what}: scales differ at {np.argwhere(gs != rs)[:4].tolist()}"
    assert np.array_equal(gq, rq), f"{what}: data differ at {np.argwhere(gq != rq)[:4].tolist()}"


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_colwise_tiny_config(fmt):
    sp = splits_for("tiny")
    _check_colwise(bf16_normal((256, 256), 1.0, seed=1), sp, fmt, "tiny")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_colwise_ragged_splits(fmt):
    rng = np.random.default_rng(4)
    sp = rng.integers(0, 90, size=13)
    sp[[0, 5, 12]] = 0
    sp[3] = 1
    rows = int(sp.sum())
    bits = bf16_normal((rows, 96), 1.0, seed=5)
    bits[::7, ::3] = 0x8000                                    # sprinkle -0
    _check_colwise(bits, sp, fmt, "ragged")


def test_colwise_more_than_512_columns():
    sp = [33, 0, 64, 2]
    _check_colwise(bf16_normal((99, 1056), 1.0, seed=6), sp, "mxfp4", "1056 cols")


def test_colwise_dgrad_weight_layout():
    G, N, K = 3, 64, 96
    w = bf16_normal((G * N, K), 0.02, seed=7)
    _check_colwise(w, [N] * G, "mxfp4", "W along N")


def test_rowwise_full_size_fc1_sampled():
    """Activation quantization at the fc1 size (32768 x 4096), the launch the
    bench times; 2048 sampled rows compared bit-exactly."""
    bits = bf16_normal((32768, 4096), 1.0, seed=1)
    x = dev_bf16(bits)
    q, s = mxg.quantize_rowwise(x, "mxfp4")
    rows = np.sort(np.random.default_rng(0).choice(32768, size=2048, replace=False))
    rq, rs = omx.quantize_rowwise(bits[rows], "mxfp4")
    assert np.array_equal(host(q)[rows], rq) and np.array_equal(mx_scales_rowmajor(s, 32768)[rows], rs)


def test_colwise_full_size_fc1_sampled_columns():
    """dY column-wise quantization at the fc1 backward size (32768 x 3072,
    splits from the fc1 routing); 64 sampled columns compared bit-exactly."""
    sp = splits_for("fc1")
    bits = bf16_normal((32768, 3072), 1.0, seed=3)
    x = dev_bf16(bits)
    q, s, mpad = mxg.quantize_colwise_segpad(x, sp, "mxfp4")
    cols = np.sort(np.random.default_rng(1).choice(3072, size=64, replace=False))
    rq, rs = omx.quantize_colwise_segpad(np.ascontiguousarray(bits[:, cols]), sp, "mxfp4")
    assert np.array_equal(host(q)[cols], rq) and np.array_equal(mx_scales_rowmajor(s, 3072)[cols], rs)
