"""Helpers shared by the GPU tests: host <-> device copies and the GEMM
tolerance. No arithmetic of the method lives here."""
import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None

from oracle.formats import bf16_bits_to_f64


def have_gpu() -> bool:
    return torch is not None and torch.cuda.is_available()


def dev_bf16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def dev_f32(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def mx_scales_rowmajor(t, rows: int) -> np.ndarray:
    """The library stores MX scales block-major, u8 [blocks, R4] with R4 = rows
    rounded up to a multiple of 4 (padding rows hold 0); the oracle row-major,
    [rows, blocks]. Checks the padding, then permutes the layout."""
    a = host(t)
    r4 = (rows + 3) // 4 * 4
    assert a.shape[1] == r4, f"scale block stride {a.shape[1]} != {r4}"
    assert not a[:, rows:].any(), "MX scale padding rows are not zero"
    return np.ascontiguousarray(a[:, :rows].T)


def kblocked_rows(t) -> np.ndarray:
    """1x128 column-wise codes are stored in 64-byte blocks along the padded
    length, u8 [mpad/64, cols, 64]; the oracle keeps rows, [cols, mpad]."""
    a = host(t)
    nb, cols, w = a.shape
    assert w == 64, a.shape
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(cols, nb * 64))


def host_bf16_f64(t) -> np.ndarray:
    return bf16_bits_to_f64(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))


def gemm_bound(ref: np.ndarray, rms=None) -> np.ndarray:
    """|gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref): fp32 accumulation in any
    order plus the bf16 rounding of the output stay well inside it, while a
    wrong scale, a dropped block or a transposed operand do not."""
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return 2.0 ** -7 * np.abs(ref) + 1e-3 * rms


def assert_gemm_close(gpu: np.ndarray, ref: np.ndarray, rms=None, what=""):
    b = gemm_bound(ref, rms)
    err = np.abs(gpu - ref)
    ratio = np.where(b > 0, err / np.where(b > 0, b, 1), np.where(err > 0, np.inf, 0))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, f"{what}: max |gpu-ref|/bound = {worst:.3g} at {np.unravel_index(np.argmax(ratio), ratio.shape)}"
    return worst
