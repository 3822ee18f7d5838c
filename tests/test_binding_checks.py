"""The Python binding's buffer checks, without a GPU: the C ABI receives only
pointers, so the binding compares every buffer's shape, dtype and layout with
what the call will read or write and raises before anything reaches the
library. CPU tensors suffice here because the checks run first."""
import pytest
import torch

import moe_grouped_block_mx_amd as mxg

u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16
G, N, K, M = 2, 64, 128, 40
SPLITS = [24, 16]
MPAD = 64                      # 32 + 32


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def fwd_args(**over):
    a = dict(a_q=z((M, K // 2), u8), a_s=z((K // 32, mxg.mx_scale_stride(M)), u8),
             w_q=z((G * N, K // 2), u8), w_s=z((K // 32, G * N), u8))
    a.update(over)
    return a


@pytest.mark.parametrize("bad", [
    dict(a_q=z((M, K), u8)),                                  # E4M3-sized data for an MXFP4 call
    dict(a_s=z((K // 32, M), u8)),                            # scales without the 4-row padding (40 is a
                                                              # multiple of 4: use a row count that is not)
    dict(w_q=z((G * N, K // 2), torch.int8)),                 # wrong dtype
    dict(w_s=z((G * N, K // 32), u8)),                        # row-major scales: refused, never misread
])
def test_fwd_operands(bad):
    if "a_s" in bad:                                          # 41 rows pad to 44
        args = fwd_args(a_q=z((41, K // 2), u8), **bad)
        with pytest.raises(ValueError, match="a_s"):
            mxg.grouped_fwd(args["a_q"], args["a_s"], args["w_q"], args["w_s"], [25, 16], N, K)
        return
    args = fwd_args(**bad)
    with pytest.raises(ValueError):
        mxg.grouped_fwd(args["a_q"], args["a_s"], args["w_q"], args["w_s"], SPLITS, N, K)


def test_fwd_out_buffer():
    a = fwd_args()
    for out in (z((M, N + 32), bf16), z((M, N), torch.float16), z((N, M), bf16).t()):
        with pytest.raises(ValueError, match="out"):
            mxg.grouped_fwd(a["a_q"], a["a_s"], a["w_q"], a["w_s"], SPLITS, N, K, out=out)


def test_dgrad_buffers():
    dq, ds = z((M, N // 2), u8), z((N // 32, mxg.mx_scale_stride(M)), u8)
    wq, ws = z((K, G * N // 2), u8), z((G * N // 32, K), u8)
    with pytest.raises(ValueError, match="dx"):
        mxg.grouped_dgrad(dq, ds, wq, ws, SPLITS, N, K, dx=z((M, N), bf16))
    with pytest.raises(ValueError, match="wcol_q"):
        mxg.grouped_dgrad(dq, ds, z((G * N // 2, K), u8), ws, SPLITS, N, K)
    with pytest.raises(ValueError, match="wcol_s"):
        mxg.grouped_dgrad(dq, ds, wq, z((K, G * N // 32), u8), SPLITS, N, K)


def test_wgrad_main_grad():
    dq, ds = z((N, MPAD // 2), u8), z((MPAD // 32, N), u8)
    xq, xs = z((K, MPAD // 2), u8), z((MPAD // 32, K), u8)
    for mg in (z((G, N, K), torch.float16),                  # fp16 would get fp32 writes twice its size
               z((G, K, N), f32),                            # transposed shape
               z((G, N, 2 * K), f32)[:, :, :K],              # strided view
               z((G * N, K), f32)):                          # flattened
        with pytest.raises(ValueError, match="main_grad"):
            mxg.grouped_wgrad(dq, ds, xq, xs, SPLITS, N, K, MPAD, mg)
    with pytest.raises(ValueError, match="xcol_s"):
        mxg.grouped_wgrad(dq, ds, xq, z((MPAD // 32, N), u8), SPLITS, N, K, MPAD, z((G, N, K), f32))


def test_quantizer_outputs():
    x = z((M, K), bf16)
    with pytest.raises(ValueError, match="scales"):
        mxg.quantize_rowwise(x, "mxfp4", q=z((M, K // 2), u8), scales=z((M, K // 32), u8))
    with pytest.raises(ValueError, match="q"):
        mxg.quantize_rowwise(x, "mxfp8", q=z((M, K // 2), u8))
    with pytest.raises(ValueError, match="scales"):
        mxg.quantize_rowwise(x, "fp8_1x128", scales=z((K // 128, M), u8))   # fp32 scales expected
    with pytest.raises(ValueError, match="scales"):
        mxg.quantize_rowwise(x, "fp8_1x128", scales=z((M, K // 128), f32))  # 1x128 scales are block-major
    with pytest.raises(ValueError, match="q_col"):
        mxg.quantize_dual(x, SPLITS, "mxfp4", q_col=z((K, MPAD), u8))
    with pytest.raises(ValueError, match="q"):
        mxg.quantize_colwise_segpad(x, SPLITS, "mxfp4", q=z((MPAD // 2, K), u8))
    with pytest.raises(ValueError, match="wt_s"):   # blockwise codes in 64-byte K blocks: [K/64, G*N, 64]
        mxg.transpose_128x128(z((256 // 64, G * 128, 64), u8), z((G, 2), f32), G, 128, 256, wt_s=z((G, 2), f32))
    with pytest.raises(ValueError, match="w_q"):    # rows of codes are refused
        mxg.transpose_128x128(z((G * 128, 256), u8), z((G, 2), f32), G, 128, 256)


def test_k_blocked_mx_code_shapes():
    # MXGG_KBLOCK_ROWS / _COLS: codes u8 [bytes per row / 64, rows, 64]; a buffer
    # of the other layout's shape is refused, never read as this one
    KR, KC = mxg.KBLOCK_ROWS, mxg.KBLOCK_COLS
    a = fwd_args()
    blocked_a, blocked_w = z((K // 128, M, 64), u8), z((K // 128, G * N, 64), u8)
    with pytest.raises(ValueError, match="a_q"):        # rows of codes under the K-block bit
        mxg.grouped_fwd(a["a_q"], a["a_s"], blocked_w, a["w_s"], SPLITS, N, K, a_fmt=mxg.MXFP4 | KR,
                        w_fmt=mxg.MXFP4 | KR)
    with pytest.raises(ValueError, match="w_q"):        # K blocks without the bit
        mxg.grouped_fwd(a["a_q"], a["a_s"], blocked_w, a["w_s"], SPLITS, N, K)
    x = z((M, K), bf16)
    with pytest.raises(ValueError, match="q"):
        mxg.quantize_rowwise(x, mxg.MXFP4 | KR, q=z((M, K // 2), u8))
    with pytest.raises(ValueError, match="q"):
        mxg.quantize_rowwise(x, mxg.MXFP8 | KR, q=z((K // 128, M, 64), u8))   # E4M3: K/64 blocks
    n2 = 128                                           # the input gradient's K blocks need N % 128
    dq, ds = z((n2 // 128, M, 64), u8), z((n2 // 32, mxg.mx_scale_stride(M)), u8)
    wq, ws = z((K, G * n2 // 2), u8), z((G * n2 // 32, K), u8)
    with pytest.raises(ValueError, match="wcol_q"):    # W along N in rows under MXGG_KBLOCK_COLS
        mxg.grouped_dgrad(dq, ds, wq, ws, SPLITS, n2, K, fmt=mxg.MXFP4 | KR | KC)
    with pytest.raises(ValueError, match="dy_q"):      # dY in K blocks without the bits
        mxg.grouped_dgrad(dq, ds, wq, ws, SPLITS, n2, K)
    with pytest.raises(ValueError, match="a_q"):       # the right size in the wrong layout
        mxg.grouped_fwd(blocked_a.reshape(M, K // 2), a["a_s"], blocked_w, a["w_s"], SPLITS, N, K,
                        a_fmt=mxg.MXFP4 | KR, w_fmt=mxg.MXFP4 | KR)
