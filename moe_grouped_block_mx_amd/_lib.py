"""ctypes binding of libmxgg.so (include/mxgg.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. torch supplies device memory and the current stream; output tensors
are allocated here when the caller passes none. Importing this module fails
loudly when the built library is missing -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libmxgg.so")
HEADER = os.path.join(ROOT, "include", "mxgg.h")

# mxgg_format
MXFP4, MXFP8, FP8_1x128, FP8_128x128, FP8_1x128_P2, FP8_128x128_P2 = 0, 1, 2, 3, 4, 5
FORMATS = {"mxfp4": MXFP4, "mxfp8": MXFP8, "fp8_1x128": FP8_1x128, "fp8_128x128": FP8_128x128,
           "fp8_1x128_p2": FP8_1x128_P2, "fp8_128x128_p2": FP8_128x128_P2}
POW2_SCALES = 1
MAX_EXPERTS = 512
# mxgg_scale_layout: OR-ed into an MX format to state the layout of its scales
LAYOUT_BLOCK_MAJOR, LAYOUT_ROW_MAJOR, LAYOUT_MFMA, LAYOUT_MASK = 0x000, 0x100, 0x200, 0xF00
# MX code layouts: row-wise / column-wise codes in 64-byte K blocks
KBLOCK_ROWS, KBLOCK_COLS, KBLOCK_MASK = 0x1000, 0x2000, 0x3000

STATUS = {
    0: "MXGG_OK", 1: "MXGG_ERR_NULL", 2: "MXGG_ERR_SHAPE", 3: "MXGG_ERR_SPLITS",
    4: "MXGG_ERR_FORMAT", 5: "MXGG_ERR_ALIGN", 6: "MXGG_ERR_WORKSPACE",
    7: "MXGG_ERR_DEVICE", 8: "MXGG_ERR_ARCH", 9: "MXGG_ERR_HIP",
}


class MxggError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


_vp, _i64, _i32, _u32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
_i64p = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "mxgg_quantize_rowwise": [_vp, _i64, _i64, _i64, _i32, _u32, _vp, _vp, _vp],
    "mxgg_quantize_colwise_segpad": [_vp, _i64, _i64, _i64, _i64p, _i32, _i32, _u32, _vp, _vp, _i64, _vp],
    "mxgg_quantize_dual": [_vp, _i64, _i64, _i64, _i64p, _i32, _i32, _u32, _vp, _vp, _vp, _vp, _i64, _vp],
    "mxgg_grouped_fwd": [_vp, _vp, _i32, _vp, _vp, _i32, _i64p, _i32, _i64, _i64, _i64, _vp, _vp, _sz, _vp],
    "mxgg_grouped_dgrad": [_vp, _vp, _vp, _vp, _i32, _i64p, _i32, _i64, _i64, _i64, _vp, _vp, _sz, _vp],
    "mxgg_transpose_128x128": [_vp, _vp, _i32, _i64, _i64, _vp, _vp, _vp],
    "mxgg_grouped_wgrad": [_vp, _vp, _vp, _vp, _i32, _i64p, _i32, _i64, _i64, _i64, _vp, _i32, _i32, _vp, _sz,
                           _vp],
    "mxgg_mx_scales_relayout": [_vp, _i32, _i64, _i64, _vp, _i32, _vp],
}


def _load():
    # torch's HIP runtime must be the one in the process before the library
    # binds to libamdhip64.so (it links that same runtime)
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python moe_grouped_block_mx_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.mxgg_workspace_size.argtypes = [_i32]
    lib.mxgg_workspace_size.restype = _sz
    lib.mxgg_segpad_rows.argtypes = [_i64p, _i32, _i32]
    lib.mxgg_segpad_rows.restype = _i64
    lib.mxgg_mx_scale_stride.argtypes = [_i64]
    lib.mxgg_mx_scale_stride.restype = _i64
    lib.mxgg_status_string.argtypes = [_i32]
    lib.mxgg_status_string.restype = ctypes.c_char_p
    lib.mxgg_last_error.argtypes = []
    lib.mxgg_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def header_functions() -> list[str]:
    """Names of the functions include/mxgg.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mxgg_[a-z_0-9]+)\s*\(", txt)))


def _check(status: int):
    if status != 0:
        raise MxggError(status, lib.mxgg_last_error().decode())


def _splits(m_splits):
    vals = [int(v) for v in m_splits]
    arr = (ctypes.c_int64 * max(1, len(vals)))(*vals)
    return arr, len(vals)


def _fmt(f) -> int:
    return FORMATS[f] if isinstance(f, str) else int(f)


def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_bf16_2d(x):
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bf16 tensor")
    if x.numel() and x.stride(1) != 1:
        raise ValueError("x must have unit inner stride")


def _ld(x):
    """Leading dimension in elements (the column count for an empty tensor)."""
    return x.stride(0) if x.numel() else x.shape[1]


def _expect(t, name, shape, dtypes):
    """The C ABI sees only pointers, so this is the one place where a buffer
    of the wrong shape, dtype or layout is caught before the GPU reads or
    writes past its end."""
    torch = _torch()
    shape = tuple(int(v) for v in shape)
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != shape or t.dtype not in dtypes or not t.is_contiguous():
        want = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        got = f"{str(t.dtype).replace('torch.', '')} {tuple(t.shape)}" + ("" if t.is_contiguous() else " non-contiguous")
        raise ValueError(f"{name} must be a contiguous {want} tensor of shape {shape}, got {got}")
    return t


def _is_mx(f):
    return (f & 0xFF) in (MXFP4, MXFP8)


def _row_major(f):
    return (f & LAYOUT_MASK) == LAYOUT_ROW_MAJOR


def _mfma(f):
    return (f & LAYOUT_MASK) == LAYOUT_MFMA


def _rows32(rows):
    return (rows + 31) // 32 * 32 if rows > 0 else 0


def _layout_shape(layout, rows, blocks):
    """u8 scales of an operand with `rows` rows and `blocks` blocks of 32 along
    its contraction, in one of the three MX scale layouts."""
    if layout == LAYOUT_ROW_MAJOR:
        return (rows, blocks)
    if layout == LAYOUT_MFMA:                                     # [blocks/4, R32/32, 64, 2]
        return (blocks // 4, _rows32(rows) * 4)
    return (blocks, mxgg_mx_scale_stride(rows))                   # block-major


def _code_bytes(f, n):
    """Code bytes of n elements (E2M1 packs two per byte)."""
    return n // 2 if (f & 0xFF) == MXFP4 else n


def _q_shape(f, rows, cols):
    """Codes of a [rows, cols] operand quantized along cols: rows of codes,
    or 64-byte blocks along cols, u8 [bytes per row / 64, rows, 64]
    (blockwise formats always, MX with KBLOCK_ROWS)."""
    if not _is_mx(f) or (f & KBLOCK_ROWS):
        return (_code_bytes(f, cols) // 64, rows, 64)
    return (rows, _code_bytes(f, cols))


def _q_rows(q, f):
    """Row count of a code tensor laid out as _q_shape gives it (a tensor of
    another rank then fails the shape check that follows)."""
    if _is_mx(f) and not (f & KBLOCK_ROWS):
        return q.shape[0] if q.dim() >= 1 else 0
    return q.shape[1] if q.dim() >= 2 else 0


def _col_q_shape(f, cols, mpad):
    """Codes of the column-wise segment-padded [cols, mpad] operand: rows, or
    64-byte blocks along the padded length (blockwise, MX with KBLOCK_COLS)."""
    if not _is_mx(f) or (f & KBLOCK_COLS):
        return (_code_bytes(f, mpad) // 64, cols, 64)
    return (cols, _code_bytes(f, mpad))


def _row_scale_shape(f, rows, cols):
    """Scales of a [rows, cols] operand quantized along cols (row-major scales
    when the format says so: the library refuses them, never misreads them).
    1x128 fp32 scales are block-major [cols/128, rows]."""
    if _is_mx(f):
        return _layout_shape(f & LAYOUT_MASK, rows, cols // 32)
    if (f & 0xFF) in (FP8_1x128, FP8_1x128_P2):
        return (cols // 128, rows)
    return (rows // 128, cols // 128)


def _col_scale_shape(f, cols, mpad):
    """Scales of the column-wise segment-padded [cols, mpad] operand (1x128:
    block-major f32 [mpad/128, cols])."""
    if _is_mx(f):
        return _layout_shape(f & LAYOUT_MASK, cols, mpad // 32)
    return (mpad // 128, cols)


def _sdtype(f):
    torch = _torch()
    return torch.uint8 if _is_mx(f) else torch.float32


def mxgg_workspace_size(G: int) -> int:
    return int(lib.mxgg_workspace_size(G))


def mxgg_segpad_rows(m_splits, fmt) -> int:
    arr, G = _splits(m_splits)
    r = int(lib.mxgg_segpad_rows(arr, G, _fmt(fmt) & 0xFF))
    if r < 0:
        raise MxggError(2, "invalid splits or format for mxgg_segpad_rows")
    return r


def _flags(flags, f):
    """Power-of-two scales are the blockwise default; MX formats take no flags."""
    if flags is None:
        return POW2_SCALES if (f & 0xFF) in (FP8_1x128, FP8_128x128, FP8_1x128_P2, FP8_128x128_P2) else 0
    return int(flags)


def mxgg_mx_scales_relayout(src, rows, blocks, src_layout, dst_layout, dst=None):
    """MX scales from one layout into another: row-major u8 [rows, blocks],
    block-major u8 [blocks, mx_scale_stride(rows)], MFMA u8 [blocks/4,
    R32*4] (R32 = rows rounded up to 32; padding rows 0). Returns dst."""
    torch = _torch()
    src_shape = _layout_shape(src_layout, rows, blocks)
    dst_shape = _layout_shape(dst_layout, rows, blocks)
    _expect(src, "src", src_shape, torch.uint8)
    if dst is None:
        dst = torch.empty(dst_shape, dtype=torch.uint8, device=src.device)
    _expect(dst, "dst", dst_shape, torch.uint8)
    _check(lib.mxgg_mx_scales_relayout(_ptr(src), int(src_layout), int(rows), int(blocks), _ptr(dst),
                                       int(dst_layout), _stream(src)))
    return dst


def mxgg_mx_scale_stride(rows):
    """Block stride (bytes) of block-major MX scales of an operand with `rows` rows."""
    return int(lib.mxgg_mx_scale_stride(int(rows)))


def mxgg_quantize_rowwise(x, fmt="mxfp4", flags=None, q=None, scales=None):
    """x: bf16 [rows, cols] (row stride may exceed cols). Returns (q, scales).
    flags: None = default (MXGG_POW2_SCALES for the blockwise formats)."""
    torch = _torch()
    f = _fmt(fmt)
    flags = _flags(flags, f)
    rows, cols = x.shape
    _check_bf16_2d(x)
    if q is None:
        q = torch.empty(_q_shape(f, rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        # MX: block-major, block stride = rows rounded up to a multiple of 4
        scales = torch.empty(_row_scale_shape(f, rows, cols), dtype=_sdtype(f), device=x.device)
    _expect(q, "q", _q_shape(f, rows, cols), torch.uint8)
    _expect(scales, "scales", _row_scale_shape(f, rows, cols), _sdtype(f))
    _check(lib.mxgg_quantize_rowwise(_ptr(x), rows, cols, _ld(x), f, flags, _ptr(q), _ptr(scales),
                                     _stream(x)))
    return q, scales


def mxgg_quantize_colwise_segpad(x, m_splits, fmt="mxfp4", flags=None, q=None, scales=None):
    """x: bf16 [rows, cols]. Returns (q, scales, mpad): q [cols, mpad(/2)],
    or for the 1x128 formats u8 [mpad/64, cols, 64] (64-byte K blocks)."""
    torch = _torch()
    f = _fmt(fmt)
    flags = _flags(flags, f)
    rows, cols = x.shape
    _check_bf16_2d(x)
    arr, G = _splits(m_splits)
    mpad = int(lib.mxgg_segpad_rows(arr, G, f & 0xFF))
    if mpad < 0:
        mpad = 0
    if q is None:
        q = torch.empty(_col_q_shape(f, cols, mpad), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(_col_scale_shape(f, cols, mpad), dtype=_sdtype(f), device=x.device)
    _expect(q, "q", _col_q_shape(f, cols, mpad), torch.uint8)
    _expect(scales, "scales", _col_scale_shape(f, cols, mpad), _sdtype(f))
    _check(lib.mxgg_quantize_colwise_segpad(_ptr(x), rows, cols, _ld(x), arr, G, f, flags, _ptr(q),
                                            _ptr(scales), mpad, _stream(x)))
    return q, scales, mpad


def mxgg_quantize_dual(x, m_splits, fmt="mxfp4", flags=None, q_row=None, s_row=None, q_col=None, s_col=None):
    """x: bf16 [rows, cols]. Row-wise and column-wise segment-padded
    quantization (MX, or blockwise 1x128) from one read.
    Returns (q_row, s_row, q_col, s_col, mpad)."""
    torch = _torch()
    f = _fmt(fmt)
    flags = _flags(flags, f)
    rows, cols = x.shape
    _check_bf16_2d(x)
    arr, G = _splits(m_splits)
    mpad = int(lib.mxgg_segpad_rows(arr, G, f & 0xFF))
    if mpad < 0:
        mpad = 0
    u8 = dict(dtype=torch.uint8, device=x.device)
    if q_row is None:
        q_row = torch.empty(_q_shape(f, rows, cols), **u8)
    if s_row is None:
        s_row = torch.empty(_row_scale_shape(f, rows, cols), dtype=_sdtype(f), device=x.device)
    if q_col is None:
        q_col = torch.empty(_col_q_shape(f, cols, mpad), **u8)
    if s_col is None:
        s_col = torch.empty(_col_scale_shape(f, cols, mpad), dtype=_sdtype(f), device=x.device)
    _expect(q_row, "q_row", _q_shape(f, rows, cols), torch.uint8)
    _expect(s_row, "s_row", _row_scale_shape(f, rows, cols), _sdtype(f))
    _expect(q_col, "q_col", _col_q_shape(f, cols, mpad), torch.uint8)
    _expect(s_col, "s_col", _col_scale_shape(f, cols, mpad), _sdtype(f))
    _check(lib.mxgg_quantize_dual(_ptr(x), rows, cols, _ld(x), arr, G, f, flags, _ptr(q_row), _ptr(s_row),
                                  _ptr(q_col), _ptr(s_col), mpad, _stream(x)))
    return q_row, s_row, q_col, s_col, mpad


def mxgg_grouped_fwd(a_q, a_s, w_q, w_s, m_splits, N, K, a_fmt="mxfp4", w_fmt="mxfp4", out=None, ws=None):
    """out[M, N] (bf16) = per-expert A . W_g^T; W packed [G*N, ...]."""
    torch = _torch()
    arr, G = _splits(m_splits)
    af, wf = _fmt(a_fmt), _fmt(w_fmt)
    M = _q_rows(a_q, af)
    _expect(a_q, "a_q", _q_shape(af, M, K), torch.uint8)
    _expect(a_s, "a_s", _row_scale_shape(af, M, K), _sdtype(af))
    _expect(w_q, "w_q", _q_shape(wf, G * N, K), torch.uint8)
    _expect(w_s, "w_s", _row_scale_shape(wf, G * N, K), _sdtype(wf))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    _expect(out, "out", (M, N), torch.bfloat16)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.mxgg_grouped_fwd(_ptr(a_q), _ptr(a_s), _fmt(a_fmt), _ptr(w_q), _ptr(w_s), _fmt(w_fmt), arr, G, M, N,
                                K, _ptr(out), _ptr(ws), ws_bytes, _stream(a_q)))
    return out


def mxgg_transpose_128x128(w_q, w_s, G, N, K, wt_q=None, wt_s=None):
    """128x128-block FP8 weights [G*N, K] (+ f32 [G*N/128, K/128]) transposed
    to [G*K, N] (+ f32 [G*K/128, N/128]): the input gradient's weights (codes
    in 64-byte K blocks on both sides)."""
    torch = _torch()
    if wt_q is None:
        wt_q = torch.empty(_q_shape(FP8_128x128, G * K, N), dtype=torch.uint8, device=w_q.device)
    if wt_s is None:
        wt_s = torch.empty((G * K // 128, N // 128), dtype=torch.float32, device=w_q.device)
    _expect(w_q, "w_q", _q_shape(FP8_128x128, G * N, K), torch.uint8)
    _expect(w_s, "w_s", (G * N // 128, K // 128), torch.float32)
    _expect(wt_q, "wt_q", _q_shape(FP8_128x128, G * K, N), torch.uint8)
    _expect(wt_s, "wt_s", (G * K // 128, N // 128), torch.float32)
    _check(lib.mxgg_transpose_128x128(_ptr(w_q), _ptr(w_s), G, N, K, _ptr(wt_q), _ptr(wt_s), _stream(w_q)))
    return wt_q, wt_s


def mxgg_grouped_dgrad(dy_q, dy_s, wcol_q, wcol_s, m_splits, N, K, fmt="mxfp4", dx=None, ws=None):
    """dx[M, K] (bf16) = per-expert dY . W_g. fmt is dY's format: "mxfp4" /
    "mxfp8" with W quantized along N in MXFP4, or "fp8_1x128" / "fp8_1x128_p2"
    with W^T from mxgg_transpose_128x128."""
    torch = _torch()
    arr, G = _splits(m_splits)
    f = _fmt(fmt)
    M = _q_rows(dy_q, f)
    # layout bits of fmt describe wcol_s; dY's scales are block-major
    _expect(dy_q, "dy_q", _q_shape(f, M, N), torch.uint8)
    _expect(dy_s, "dy_s", _row_scale_shape(f & 0xFF, M, N), _sdtype(f))
    if _is_mx(f):                       # W along N, MXFP4: [K, G*N/2] + [G*N/32, K]
        _expect(wcol_q, "wcol_q", _col_q_shape(MXFP4 | (f & KBLOCK_COLS), K, G * N), torch.uint8)
        _expect(wcol_s, "wcol_s", _col_scale_shape(MXFP4 | (f & LAYOUT_MASK), K, G * N), torch.uint8)
    else:                               # transposed 128x128 blocks
        _expect(wcol_q, "wcol_q", _q_shape(FP8_128x128, G * K, N), torch.uint8)
        _expect(wcol_s, "wcol_s", (G * K // 128, N // 128), torch.float32)
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dy_q.device)
    _expect(dx, "dx", (M, K), torch.bfloat16)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.mxgg_grouped_dgrad(_ptr(dy_q), _ptr(dy_s), _ptr(wcol_q), _ptr(wcol_s), _fmt(fmt), arr, G, M, N, K,
                                  _ptr(dx), _ptr(ws), ws_bytes, _stream(dy_q)))
    return dx


def mxgg_grouped_wgrad(dycol_q, dycol_s, xcol_q, xcol_s, m_splits, N, K, mpad, main_grad, accumulate=True,
                       fmt="mxfp4", ws=None):
    """main_grad [G, N, K] (fp32 or bf16) += / = per-expert dY_g^T . X_g."""
    torch = _torch()
    arr, G = _splits(m_splits)
    f = _fmt(fmt)
    _expect(dycol_q, "dycol_q", _col_q_shape(f, N, mpad), torch.uint8)
    _expect(dycol_s, "dycol_s", _col_scale_shape(f, N, mpad), _sdtype(f))
    _expect(xcol_q, "xcol_q", _col_q_shape(f, K, mpad), torch.uint8)
    _expect(xcol_s, "xcol_s", _col_scale_shape(f, K, mpad), _sdtype(f))
    _expect(main_grad, "main_grad", (G, N, K), (torch.float32, torch.bfloat16))
    out_bf16 = 1 if main_grad.dtype == torch.bfloat16 else 0
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.mxgg_grouped_wgrad(_ptr(dycol_q), _ptr(dycol_s), _ptr(xcol_q), _ptr(xcol_s), _fmt(fmt), arr, G, N, K,
                                  mpad, _ptr(main_grad), out_bf16, 1 if accumulate else 0, _ptr(ws), ws_bytes,
                                  _stream(main_grad)))
    return main_grad


# short names
quantize_rowwise = mxgg_quantize_rowwise
quantize_colwise_segpad = mxgg_quantize_colwise_segpad
quantize_dual = mxgg_quantize_dual
grouped_fwd = mxgg_grouped_fwd
grouped_dgrad = mxgg_grouped_dgrad
transpose_128x128 = mxgg_transpose_128x128
grouped_wgrad = mxgg_grouped_wgrad
workspace_size = mxgg_workspace_size
segpad_rows = mxgg_segpad_rows
mx_scale_stride = mxgg_mx_scale_stride
mx_scales_relayout = mxgg_mx_scales_relayout
