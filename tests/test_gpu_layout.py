"""MX scale layouts through the C ABI: the relayout between plain row-major
scales (u8 [rows, blocks]) and the library's block-major layout, checked
against a numpy transpose and against the oracle's own row-major scales; a
forward fed relayouted oracle scales equals the one fed the library
quantizer's; row-major scales handed to a GEMM are refused, never misread
("Integrate MXFP4 hipblaslt GEMM support": plain and pre-arranged scale
layouts)."""
import numpy as np
import pytest

from oracle import mx as omx
from synth import bf16_normal

from .gpu_util import dev_bf16, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

import moe_grouped_block_mx_amd as mxg  # noqa: E402
import torch  # noqa: E402


def _block_major(rm: np.ndarray) -> np.ndarray:
    rows, blocks = rm.shape
    out = np.zeros((blocks, (rows + 3) // 4 * 4), dtype=np.uint8)
    out[:, :rows] = rm.T
    return out


@pytest.mark.parametrize("rows,blocks", [(1, 1), (3, 2), (64, 64), (150, 70), (301, 129), (4097, 3)])
def test_relayout_round_trip(rows, blocks):
    rng = np.random.default_rng(rows * 1000 + blocks)
    rm = rng.integers(0, 256, size=(rows, blocks), dtype=np.uint8)
    src = torch.from_numpy(rm).cuda()
    bm = mxg.mx_scales_relayout(src, rows, blocks, mxg.LAYOUT_ROW_MAJOR, mxg.LAYOUT_BLOCK_MAJOR)
    # garbage in the destination's padding must be overwritten with zeros
    dst = torch.full((blocks, mxg.mx_scale_stride(rows)), 0xAB, dtype=torch.uint8, device="cuda")
    mxg.mx_scales_relayout(src, rows, blocks, mxg.LAYOUT_ROW_MAJOR, mxg.LAYOUT_BLOCK_MAJOR, dst=dst)
    back = mxg.mx_scales_relayout(bm, rows, blocks, mxg.LAYOUT_BLOCK_MAJOR, mxg.LAYOUT_ROW_MAJOR)
    torch.cuda.synchronize()
    assert np.array_equal(host(bm), _block_major(rm))
    assert np.array_equal(host(dst), _block_major(rm))
    assert np.array_equal(host(back), rm)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_oracle_row_major_scales_relayout_to_the_quantizer_layout(fmt):
    x = bf16_normal((203, 256), 1.0, seed=5)
    _, s_lib = mxg.quantize_rowwise(dev_bf16(x), fmt)
    _, s_ref = omx.quantize_rowwise(x, fmt)                       # row-major [rows, K/32]
    s_bm = mxg.mx_scales_relayout(torch.from_numpy(np.ascontiguousarray(s_ref)).cuda(), 203, 8,
                                  mxg.LAYOUT_ROW_MAJOR, mxg.LAYOUT_BLOCK_MAJOR)
    torch.cuda.synchronize()
    assert np.array_equal(host(s_bm), host(s_lib))


def test_forward_on_relayouted_oracle_operands_matches_and_row_major_is_refused():
    sp = [100, 0, 37]
    G, N, K, M = 3, 64, 256, 137
    a = bf16_normal((M, K), 1.0, seed=11)
    w = bf16_normal((G * N, K), 0.05, seed=12)
    aq, as_ = mxg.quantize_rowwise(dev_bf16(a), "mxfp4")
    wq, ws = mxg.quantize_rowwise(dev_bf16(w), "mxfp4")
    y = mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K)
    ra, ras = omx.quantize_rowwise(a, "mxfp4")
    rw, rws = omx.quantize_rowwise(w, "mxfp4")
    cu = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()  # noqa: E731
    as2 = mxg.mx_scales_relayout(cu(ras), M, K // 32, mxg.LAYOUT_ROW_MAJOR, mxg.LAYOUT_BLOCK_MAJOR)
    ws2 = mxg.mx_scales_relayout(cu(rws), G * N, K // 32, mxg.LAYOUT_ROW_MAJOR, mxg.LAYOUT_BLOCK_MAJOR)
    y2 = mxg.grouped_fwd(cu(ra), as2, cu(rw), ws2, sp, N, K)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    with pytest.raises(mxg.MxggError, match="MXGG_ERR_FORMAT"):
        mxg.grouped_fwd(cu(ra), cu(ras), cu(rw), ws2, sp, N, K, a_fmt=mxg.MXFP4 | mxg.LAYOUT_ROW_MAJOR)
