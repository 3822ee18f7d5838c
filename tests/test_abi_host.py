"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments before any HIP call (so these run
on a machine with no GPU). Pointers here are fake, aligned device addresses
that validation never dereferences."""
import ctypes

import numpy as np
import pytest

import moe_grouped_block_mx_amd as mx
from oracle.mx import segpad_offsets

L = mx.lib
P = ctypes.c_void_p(0x100000)     # a fake 16-byte aligned device address
BAD = ctypes.c_void_p(0x100008)   # misaligned
NULL = None


def splits(*v):
    return (ctypes.c_int64 * len(v))(*v)


def last():
    return L.mxgg_last_error().decode()


def test_exports_every_declared_function():
    names = mx.header_functions()
    assert {"mxgg_quantize_rowwise", "mxgg_quantize_colwise_segpad", "mxgg_grouped_fwd",
            "mxgg_grouped_dgrad", "mxgg_grouped_wgrad", "mxgg_workspace_size",
            "mxgg_segpad_rows", "mxgg_mx_scale_stride", "mxgg_quantize_dual", "mxgg_transpose_128x128",
            "mxgg_status_string", "mxgg_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_mx_scale_stride():
    # block stride of block-major MX scales: rows rounded up to a multiple of 4
    for rows, want in ((0, 0), (-3, 0), (1, 4), (3, 4), (4, 4), (5, 8), (32768, 32768), (32769, 32772)):
        assert L.mxgg_mx_scale_stride(rows) == want, rows
    assert mx.mx_scale_stride(7) == 8


def test_dual_quantizer_validation():
    m = splits(40, 0, 24)
    mpad = 96                                               # 64 + 0 + 32

    def dual(fmt=0, mp=mpad, rows=64, cols=64, ldx=64, qr=P, qc=P, G=3):
        return L.mxgg_quantize_dual(P, rows, cols, ldx, m, G, fmt, 0, qr, P, qc, P, mp, NULL)
    assert dual(fmt=3) == 4 and "MX formats" in last()      # 128x128 blocks: no column-wise form
    assert dual(fmt=5) == 4                                  # ... nor with power-of-two scales
    assert dual(fmt=2) == 2 and "128" in last()              # 1x128: cols must be a multiple of 128
    assert dual(fmt=2, cols=128, ldx=128) == 2 and "mpad" in last()   # 1x128 pads segments to 128
    assert L.mxgg_quantize_dual(P, 64, 128, 128, m, 3, 4, 0, P, P, P, P, 256, NULL) != 4   # _P2 accepted
    assert dual(fmt=9) == 4
    assert dual(mp=64) == 2 and "mpad" in last()            # wrong padded row count
    assert dual(rows=63) == 3                               # splits do not sum to rows
    assert dual(cols=48) == 2                               # cols % 32
    assert dual(ldx=60) == 2                                # ldx < cols
    assert dual(qr=NULL) == 1 and dual(qc=NULL) == 1        # NULL outputs
    assert dual(qc=BAD) == 5                                # misaligned
    assert dual(G=0) == 2
    # an empty tensor is validated, then OK with no device work
    assert L.mxgg_quantize_dual(NULL, 0, 64, 64, splits(0, 0), 2, 0, 0, NULL, NULL, NULL, NULL, 0, NULL) == 0


def test_wgrad_mx_bf16_output_rejected():
    m = splits(32, 0)
    st = L.mxgg_grouped_wgrad(P, P, P, P, 0, m, 2, 64, 64, 32, P, 1, 0, NULL, 0, NULL)
    assert st == 4 and "fp32" in last()


def test_status_strings():
    for s in range(10):
        assert L.mxgg_status_string(s).decode().startswith(mx._lib.STATUS[s])


def fwd(m, G, M, N=64, K=64, a_fmt=0, w_fmt=0, a=P, out=P):
    return L.mxgg_grouped_fwd(a, P, a_fmt, P, P, w_fmt, m, G, M, N, K, out, NULL, 0, NULL)


def test_fwd_split_rules():
    assert fwd(splits(3, -1), 2, 2) == 3 and "negative" in last()          # negative
    assert fwd(splits(3, 4), 2, 8) == 3 and "sum" in last()                # sum != rows
    assert fwd(splits(3, 4), 2, 6) == 3                                     # sum != rows
    assert fwd(splits(3), 0, 3) == 2                                        # G = 0
    big = (ctypes.c_int64 * 513)(*([0] * 513))
    assert fwd(big, 513, 0) == 2                                            # G > 512
    assert fwd(None, 2, 0) == 1                                             # NULL splits


def test_fwd_shapes_formats_pointers():
    m = splits(2, 0, 6)
    assert fwd(m, 3, 8, K=48) == 2            # K % 32
    assert fwd(m, 3, 8, N=40) == 2            # N % 32
    assert fwd(m, 3, 8, a_fmt=1, w_fmt=1) == 4   # MXFP8 weights: not a supported pair
    assert fwd(m, 3, 8, a_fmt=0, w_fmt=3) == 4
    assert fwd(m, 3, 8, a_fmt=7) == 4
    assert fwd(m, 3, 8, a=NULL) == 1
    assert fwd(m, 3, 8, a=BAD) == 5
    assert fwd(m, 3, 8, out=NULL) == 1
    # blockwise pair needs multiples of 128
    assert fwd(m, 3, 8, N=64, K=128, a_fmt=2, w_fmt=3) == 2
    # row strides of the tiles stay below 2^23 bytes
    assert fwd(m, 3, 8, K=1 << 23) == 2 and "2^23" in last()
    assert L.mxgg_grouped_dgrad(P, P, P, P, 0, splits(2, 2, 2, 2), 4, 8, 1 << 22, 64, P, NULL, 0, NULL) == 2


def test_empty_batch_validated_then_ok_without_gpu():
    # M == 0 with valid arguments returns OK before any device work
    assert fwd(splits(0, 0), 2, 0, a=NULL, out=NULL) == 0
    # ...but the splits are still validated first
    assert fwd(splits(1, -1), 2, 0, a=NULL, out=NULL) == 3
    assert L.mxgg_quantize_rowwise(NULL, 0, 64, 64, 0, 0, NULL, NULL, NULL) == 0
    assert L.mxgg_grouped_dgrad(NULL, NULL, NULL, NULL, 0, splits(0, 0), 2, 0, 64, 64, NULL, NULL, 0, NULL) == 0


def test_dgrad_rules():
    m = splits(4, 4)
    # a8w4 (dY MXFP8) and blockwise (dY FP8_1x128) pass validation; without a
    # GPU the stream's device query is what fails (HIP)
    assert L.mxgg_grouped_dgrad(P, P, P, P, 1, m, 2, 8, 64, 64, P, NULL, 0, NULL) == 9
    assert L.mxgg_grouped_dgrad(P, P, P, P, 2, m, 2, 8, 128, 128, P, NULL, 0, NULL) == 9
    assert L.mxgg_grouped_dgrad(P, P, P, P, 4, m, 2, 8, 128, 128, P, NULL, 0, NULL) == 9   # _P2
    assert L.mxgg_grouped_dgrad(P, P, P, P, 2, m, 2, 8, 64, 128, P, NULL, 0, NULL) == 2    # blockwise N % 128
    assert L.mxgg_grouped_dgrad(P, P, P, P, 3, m, 2, 8, 128, 128, P, NULL, 0, NULL) == 4   # 128x128 is W's
    assert L.mxgg_grouped_dgrad(P, P, P, P, 0, m, 2, 9, 64, 64, P, NULL, 0, NULL) == 3
    assert L.mxgg_grouped_dgrad(P, P, P, P, 0, m, 2, 8, 64, 33, P, NULL, 0, NULL) == 2
    assert L.mxgg_grouped_dgrad(P, P, NULL, P, 0, m, 2, 8, 64, 64, P, NULL, 0, NULL) == 1


def test_transpose_128x128_rules():
    t = lambda G=2, N=128, K=256, w=P, ws=P, o=P, os=P: L.mxgg_transpose_128x128(w, ws, G, N, K, o, os, NULL)
    assert t(N=64) == 2 and "128" in last()
    assert t(K=200) == 2
    assert t(G=0) == 2 and t(G=513) == 2
    assert t(w=NULL) == 1 and t(os=NULL) == 1
    assert t(o=BAD) == 5
    assert t() == 9                          # valid; no GPU to run it on


def test_quantizer_rules():
    assert L.mxgg_quantize_rowwise(P, 4, 48, 48, 0, 0, P, P, NULL) == 2       # cols % 32
    assert L.mxgg_quantize_rowwise(P, 4, 64, 32, 0, 0, P, P, NULL) == 2       # ldx < cols
    assert L.mxgg_quantize_rowwise(P, 4, 64, 68, 0, 0, P, P, NULL) == 5       # ldx % 8
    assert L.mxgg_quantize_rowwise(P, 4, 64, 64, 9, 0, P, P, NULL) == 4       # format
    assert L.mxgg_quantize_rowwise(P, 4, 64, 64, 0, 0, BAD, P, NULL) == 5
    assert L.mxgg_quantize_rowwise(P, 100, 128, 128, 3, 0, P, P, NULL) == 2   # 128x128 rows % 128
    m = splits(5, 0, 40)
    good = 32 + 64
    assert L.mxgg_quantize_colwise_segpad(P, 45, 64, 64, m, 3, 0, 0, P, P, good + 32, NULL) == 2  # mpad
    assert L.mxgg_quantize_colwise_segpad(P, 44, 64, 64, m, 3, 0, 0, P, P, good, NULL) == 3      # sum
    assert L.mxgg_quantize_colwise_segpad(P, 45, 64, 64, m, 3, 3, 0, P, P, good, NULL) == 4      # 128x128
    assert L.mxgg_quantize_colwise_segpad(P, 45, 64, 64, splits(5, -1, 41), 3, 0, 0, P, P, good, NULL) == 3


def test_wgrad_rules():
    m = splits(5, 0, 40)
    mp = 96
    w = lambda **k: L.mxgg_grouped_wgrad(k.get("dy", P), P, P, P, k.get("fmt", 0), k.get("m", m), 3, 64, 64,
                                          k.get("mp", mp), k.get("out", P), k.get("bf16", 0), k.get("acc", 1),
                                          NULL, 0, NULL)
    assert w(mp=128) == 2
    assert w(fmt=3) == 4                     # 128x128 is a weight format
    assert w(fmt=1, bf16=1) == 4             # MXFP8: fp32 main_grad only
    assert w(fmt=1) == 9                     # MXFP8 x MXFP8 passes validation (no GPU here)
    assert w(out=NULL) == 1
    assert w(acc=2) == 2
    assert w(m=splits(5, -3, 40)) == 3
    assert w(dy=BAD) == 5
    # all experts empty with accumulate: nothing to do, OK without a GPU
    assert L.mxgg_grouped_wgrad(NULL, NULL, NULL, NULL, 0, splits(0, 0, 0), 3, 64, 64, 0, P, 0, 1,
                                NULL, 0, NULL) == 0


@pytest.mark.parametrize("fmt,pad", [(0, 32), (1, 32), (2, 128)])
def test_segpad_rows_matches_oracle(fmt, pad):
    rng = np.random.default_rng(0)
    for _ in range(20):
        G = int(rng.integers(1, 40))
        v = rng.integers(0, 300, size=G)
        v[rng.random(G) < 0.2] = 0
        _, po = segpad_offsets(v, pad)
        assert L.mxgg_segpad_rows(splits(*[int(x) for x in v]), G, fmt) == po[-1]
    assert L.mxgg_segpad_rows(splits(1, -1), 2, 0) == -1
    assert L.mxgg_segpad_rows(splits(1), 1, 3) == -1
    assert L.mxgg_workspace_size(32) == 0


def test_grouped_linear_fails_loudly_off_gpu():
    # the wrapper has no CPU path: CPU tensors are refused, never computed
    import torch
    from moe_grouped_block_mx_amd.grouped_linear import GroupedLinear
    with pytest.raises(ValueError):
        GroupedLinear(2, 64, 64, recipe="nope", device="cpu")
    layer = GroupedLinear(2, 64, 64, device="cpu")
    x = torch.zeros((8, 64), dtype=torch.bfloat16)
    with pytest.raises(Exception):
        layer(x, [4, 4])
    with pytest.raises(ValueError):
        layer(torch.zeros((8, 32), dtype=torch.bfloat16), [4, 4])


I64_MAX = 2 ** 63 - 1


def test_huge_splits_cannot_wrap_to_the_row_count():
    # 1 + 2*(2^63-1) + 3 wraps to 2 modulo 2^64: must be rejected, not passed on
    assert fwd(splits(1, I64_MAX, I64_MAX, 3), 4, 2) == 3 and "exceeds" in last()
    assert L.mxgg_grouped_dgrad(P, P, P, P, 0, splits(1, I64_MAX, I64_MAX, 3), 4, 2, 64, 64, P, NULL, 0,
                                NULL) == 3
    assert L.mxgg_quantize_colwise_segpad(P, 2, 64, 64, splits(1, I64_MAX, I64_MAX, 3), 4, 0, 0, P, P, 64,
                                          NULL) == 3
    assert L.mxgg_quantize_dual(P, 2, 64, 64, splits(1, I64_MAX, I64_MAX, 3), 4, 0, 0, P, P, P, P, 64,
                                NULL) == 3
    # a split above the row count is rejected even when the others are 0
    assert fwd(splits(0, 5), 2, 4) == 3 and "exceeds" in last()


def test_wgrad_rejects_splits_at_or_above_2_31():
    # wgrad takes no row count: each split is bounded below 2^31 before the sum
    st = L.mxgg_grouped_wgrad(P, P, P, P, 0, splits(I64_MAX, I64_MAX, 2), 3, 64, 64, 96, P, 0, 1, NULL, 0, NULL)
    assert st == 3 and "2^31" in last()
    st = L.mxgg_grouped_wgrad(P, P, P, P, 0, splits(2 ** 31, 0), 2, 64, 64, 2 ** 31, P, 0, 1, NULL, 0, NULL)
    assert st == 3
    assert L.mxgg_segpad_rows(splits(I64_MAX, 1), 2, 0) == -1
    assert L.mxgg_segpad_rows(splits(2 ** 31, 1), 2, 0) == -1
    assert L.mxgg_segpad_rows(splits(2 ** 31 - 1, 1), 2, 0) == 2 ** 31 + 32


ROW_MAJOR = 0x100
MFMA = 0x200


def _header_enum(name):
    import re
    txt = open(mx._lib.HEADER).read()
    body = re.search(r"typedef enum " + name + r" \{(.*?)\}", txt, re.S).group(1)
    return {k: int(v, 0) for k, v in re.findall(r"(MXGG_\w+)\s*=\s*(0x[0-9a-fA-F]+|\d+)", body)}


def test_scale_layout_enum_declared():
    assert _header_enum("mxgg_scale_layout") == {"MXGG_LAYOUT_BLOCK_MAJOR": 0, "MXGG_LAYOUT_ROW_MAJOR": ROW_MAJOR,
                                                 "MXGG_LAYOUT_MFMA": MFMA}
    assert mx.LAYOUT_ROW_MAJOR == ROW_MAJOR and mx.LAYOUT_BLOCK_MAJOR == 0 and mx.LAYOUT_MFMA == MFMA
    # layout bits sit above every format value
    assert max(_header_enum("mxgg_format").values()) < 0x100


def test_row_major_scales_refused_by_every_entry_point():
    m = splits(32, 0)
    f = 0 | ROW_MAJOR
    calls = {
        "rowwise": lambda: L.mxgg_quantize_rowwise(P, 32, 64, 64, f, 0, P, P, NULL),
        "colwise": lambda: L.mxgg_quantize_colwise_segpad(P, 32, 64, 64, m, 2, f, 0, P, P, 32, NULL),
        "dual": lambda: L.mxgg_quantize_dual(P, 32, 64, 64, m, 2, f, 0, P, P, P, P, 32, NULL),
        "fwd A": lambda: fwd(m, 2, 32, a_fmt=f),
        "fwd W": lambda: fwd(m, 2, 32, w_fmt=f),
        "dgrad": lambda: L.mxgg_grouped_dgrad(P, P, P, P, f, m, 2, 32, 64, 64, P, NULL, 0, NULL),
        "wgrad": lambda: L.mxgg_grouped_wgrad(P, P, P, P, f, m, 2, 64, 64, 32, P, 0, 1, NULL, 0, NULL),
    }
    for name, call in calls.items():
        assert call() == 4, name
        assert "relayout" in last(), (name, last())
    # MXFP8 with row-major scales too; unknown layout bits; a layout on a blockwise format
    assert fwd(m, 2, 32, a_fmt=1 | ROW_MAJOR) == 4
    assert fwd(m, 2, 32, a_fmt=0x300) == 4
    assert L.mxgg_quantize_rowwise(P, 128, 128, 128, 2 | ROW_MAJOR, 0, P, P, NULL) == 4
    # an empty batch is still refused: validation runs before the early return
    assert fwd(splits(0, 0), 2, 0, a_fmt=f, a=NULL, out=NULL) == 4


def test_mfma_layout_accepted_only_for_weight_scales():
    # the MFMA layout is read for the weights' scales (forward w_s, input
    # gradient wcol_s) and written by the MX quantizers; activation and
    # gradient scales and both weight-gradient operands refuse it
    m = splits(32, 0)
    refused = {
        "fwd A": lambda: fwd(m, 2, 32, K=128, a_fmt=MFMA),
        "fwd A a8w4": lambda: fwd(m, 2, 32, K=128, a_fmt=1 | MFMA),
        "wgrad": lambda: L.mxgg_grouped_wgrad(P, P, P, P, MFMA, m, 2, 64, 64, 32, P, 0, 1, NULL, 0, NULL),
        "wgrad fp8": lambda: L.mxgg_grouped_wgrad(P, P, P, P, 1 | MFMA, m, 2, 64, 64, 32, P, 0, 1, NULL, 0, NULL),
    }
    for name, call in refused.items():
        assert call() == 4, name
        assert "block-major" in last(), (name, last())
    # a layout on a blockwise format stays unknown
    assert fwd(m, 2, 32, K=128, N=128, a_fmt=2, w_fmt=3 | MFMA) == 4
    assert L.mxgg_quantize_rowwise(P, 128, 128, 128, 2 | MFMA, 0, P, P, NULL) == 4
    # accepted: validation passes (no GPU here, so the device check fails)
    assert fwd(m, 2, 32, K=128, w_fmt=MFMA) == 9
    assert fwd(m, 2, 32, K=128, a_fmt=1, w_fmt=MFMA) == 9                  # a8w4
    assert L.mxgg_grouped_dgrad(P, P, P, P, MFMA, m, 2, 32, 128, 64, P, NULL, 0, NULL) == 9
    assert L.mxgg_quantize_rowwise(P, 32, 128, 128, MFMA, 0, P, P, NULL) == 9
    assert L.mxgg_quantize_colwise_segpad(P, 256, 64, 64, splits(128, 0, 128), 3, 1 | MFMA, 0, P, P, 256,
                                          NULL) == 9
    assert L.mxgg_quantize_dual(P, 256, 128, 128, splits(128, 128), 2, MFMA, 0, P, P, P, P, 256, NULL) == 9
    # the shapes it needs: K % 128 (forward), N % 128 (input gradient), cols
    # % 128 (row-wise), every split a multiple of 128 (column-wise)
    assert fwd(m, 2, 32, K=96, w_fmt=MFMA) == 2 and "128" in last()
    assert L.mxgg_grouped_dgrad(P, P, P, P, MFMA, m, 2, 32, 96, 64, P, NULL, 0, NULL) == 2
    assert L.mxgg_quantize_rowwise(P, 32, 96, 96, MFMA, 0, P, P, NULL) == 2
    assert L.mxgg_quantize_colwise_segpad(P, 160, 64, 64, splits(128, 32), 2, MFMA, 0, P, P, 160, NULL) == 3
    assert "multiple of 128" in last()
    assert L.mxgg_quantize_dual(P, 160, 128, 128, splits(32, 128), 2, MFMA, 0, P, P, P, P, 160, NULL) == 3


def test_relayout_validation():
    R, B = 0x100, 0x000
    assert L.mxgg_mx_scales_relayout(P, R, 10, 4, P, R, NULL) == 4          # same layout
    assert L.mxgg_mx_scales_relayout(P, MFMA, 10, 4, P, MFMA, NULL) == 4
    assert L.mxgg_mx_scales_relayout(P, 0x300, 10, 4, P, B, NULL) == 4     # unknown layout
    assert L.mxgg_mx_scales_relayout(P, MFMA, 10, 6, P, B, NULL) == 2      # MFMA: blocks % 4
    assert L.mxgg_mx_scales_relayout(P, R, 10, 6, P, MFMA, NULL) == 2
    for src, dst in ((R, MFMA), (MFMA, R), (B, MFMA), (MFMA, B)):
        assert L.mxgg_mx_scales_relayout(P, src, 10, 8, P, dst, NULL) == 9  # valid; no GPU here
    assert L.mxgg_mx_scales_relayout(P, R, -1, 4, P, B, NULL) == 2
    assert L.mxgg_mx_scales_relayout(P, R, 10, 0, P, B, NULL) == 2
    assert L.mxgg_mx_scales_relayout(P, R, 10, 65535 * 64 + 1, P, B, NULL) == 2
    assert L.mxgg_mx_scales_relayout(NULL, R, 10, 4, P, B, NULL) == 1
    assert L.mxgg_mx_scales_relayout(NULL, R, 0, 4, NULL, B, NULL) == 0     # nothing to do


KR, KC = 0x1000, 0x2000           # MXGG_KBLOCK_ROWS, MXGG_KBLOCK_COLS
VALIDATION = (1, 2, 3, 4, 5, 6)   # NULL, SHAPE, SPLITS, FORMAT, ALIGN, WORKSPACE


def test_k_block_bits_validation():
    # the header's rules for the 64-byte K-block code layouts, checked before
    # any device call (a call that passes them fails later here: no GPU)
    def rowwise(fmt, cols=128):
        return L.mxgg_quantize_rowwise(P, 64, cols, cols, fmt, 0, P, P, NULL)
    assert rowwise(KR, cols=96) == 2 and "K-blocked" in last()     # cols % 128
    assert rowwise(KC) == 4 and "K-block" in last()                 # row-wise codes take the rows bit only
    assert rowwise(2 | KR) == 4                                     # blockwise codes: always K-blocked, no bits
    assert rowwise(KR) not in VALIDATION and rowwise(1 | KR | 0x200) not in VALIDATION

    def colwise(fmt, m, mpad):
        return L.mxgg_quantize_colwise_segpad(P, sum(m), 64, 64, splits(*m), len(m), fmt, 0, P, P, mpad, NULL)
    assert colwise(KC, [100, 156], 288) == 3                        # column blocks need splits % 128
    assert colwise(KR, [128, 128], 256) == 4                        # column-wise codes take the cols bit only
    assert colwise(KC, [128, 0, 256], 384) not in VALIDATION

    def dual(fmt, m=(128, 128), mpad=256, cols=128):
        return L.mxgg_quantize_dual(P, sum(m), cols, cols, splits(*m), len(m), fmt, 0, P, P, P, P, mpad, NULL)
    assert dual(KR | KC) not in VALIDATION and dual(KR, m=(100, 156), mpad=288) not in VALIDATION
    assert dual(KC, m=(100, 156), mpad=288) == 3                    # only the column output needs splits % 128
    assert dual(KR, cols=96) == 2                                   # only the row output needs cols % 128

    m = splits(64, 0, 64)
    assert fwd(m, 3, 128, K=128, a_fmt=KR, w_fmt=0) == 4 and "together" in last()
    assert fwd(m, 3, 128, K=96, a_fmt=KR, w_fmt=KR) == 2 and "K-blocked" in last()
    assert fwd(m, 3, 128, K=128, a_fmt=KC, w_fmt=KC) == 4
    assert fwd(m, 3, 128, K=128, a_fmt=KR, w_fmt=KR) not in VALIDATION
    assert fwd(m, 3, 128, K=128, a_fmt=1 | KR, w_fmt=0x200 | KR) not in VALIDATION   # a8w4, MFMA weight scales
    big = 1 << 25                                                   # a lane's 32-bit DMA offset: rows < 2^25
    assert fwd(splits(big), 1, big, K=128, a_fmt=KR, w_fmt=KR) == 2 and "2^25" in last()
    assert fwd(splits(big - 4), 1, big - 4, K=128, a_fmt=KR, w_fmt=KR) not in VALIDATION

    def dgrad(fmt, M=128, N=128, K=64, m=m, G=3):
        return L.mxgg_grouped_dgrad(P, P, P, P, fmt, m, G, M, N, K, P, NULL, 0, NULL)
    assert dgrad(KR) == 4 and dgrad(KC) == 4                        # both bits or neither
    assert dgrad(KR | KC, N=96) == 2                                # N % 128
    assert dgrad(KR | KC) not in VALIDATION and dgrad(1 | KR | KC | 0x200) not in VALIDATION
    assert dgrad(KR | KC, M=big, m=splits(big), G=1) == 2 and "2^25" in last()
    assert dgrad(KR | KC, K=big, M=128, N=128) == 2

    ms = splits(32, 0)
    assert L.mxgg_grouped_wgrad(P, P, P, P, KR, ms, 2, 64, 64, 32, P, 0, 1, NULL, 0, NULL) == 4
    assert L.mxgg_grouped_wgrad(P, P, P, P, KC, ms, 2, 64, 64, 32, P, 0, 1, NULL, 0, NULL) == 4
