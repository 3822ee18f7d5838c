"""Grouped GEMM on dequantized operands, contracted in fp64.

Test infrastructure only (see the package docstring).

For expert g with rows R_g = [row_offs[g], row_offs[g+1]) (row_offs is the
prefix sum of m_splits, "Triton mxfp4 (and a8w4) grouped GEMM kernel", the
group offsets built from the splits):

* forward (TN):   Y[R_g]  = A[R_g] . W_g^T         A [M, K], W_g [N, K]
* dgrad (NN):     dX[R_g] = dY[R_g] . Wc_g^T       dY [M, N], Wc_g [K, N] is
  W_g quantized along N (so the contraction runs over N)
* wgrad (NT):     dW_g = dYc_g . Xc_g^T over the expert's padded token segment
  (dYc [N, Mpad], Xc [K, Mpad], pad columns are zero), either added in place to
  main_grad[g] ("accumulate") or written over it; with accumulate an empty
  expert leaves main_grad[g] unchanged, with overwrite it becomes zero (the
  fused main_grad accumulation of "Add ROCm Triton blockwise FP8 grouped
  GEMM").

Each contraction is one library matrix product per expert, in fp64.
"""
from __future__ import annotations

import numpy as np

from .mx import segpad_offsets

__all__ = ["row_offsets", "grouped_fwd", "grouped_dgrad", "grouped_wgrad"]


def row_offsets(m_splits) -> np.ndarray:
    m = np.asarray(m_splits, dtype=np.int64)
    if np.any(m < 0):
        raise ValueError("negative split")
    return np.concatenate([[0], np.cumsum(m)])


def grouped_fwd(a: np.ndarray, w: np.ndarray, m_splits) -> np.ndarray:
    """a: fp64 [M, K]; w: fp64 [G, N, K]; returns fp64 [M, N]."""
    offs = row_offsets(m_splits)
    G, N, K = w.shape
    if len(offs) - 1 != G or offs[-1] != a.shape[0] or a.shape[1] != K:
        raise ValueError("shape mismatch")
    out = np.zeros((a.shape[0], N), dtype=np.float64)
    for g in range(G):
        r0, r1 = offs[g], offs[g + 1]
        if r1 > r0:
            out[r0:r1] = a[r0:r1] @ w[g].T
    return out


def grouped_dgrad(dy: np.ndarray, wcol: np.ndarray, m_splits) -> np.ndarray:
    """dy: fp64 [M, N]; wcol: fp64 [K, G*N] (W quantized along N, expert g in
    columns [g*N, (g+1)*N)); returns fp64 [M, K]."""
    offs = row_offsets(m_splits)
    G = len(offs) - 1
    M, N = dy.shape
    K = wcol.shape[0]
    if wcol.shape[1] != G * N or offs[-1] != M:
        raise ValueError("shape mismatch")
    out = np.zeros((M, K), dtype=np.float64)
    for g in range(G):
        r0, r1 = offs[g], offs[g + 1]
        if r1 > r0:
            out[r0:r1] = dy[r0:r1] @ wcol[:, g * N:(g + 1) * N].T
    return out


def grouped_wgrad(dycol: np.ndarray, xcol: np.ndarray, m_splits,
                  main_grad0: np.ndarray | None = None,
                  accumulate: bool = False, pad: int = 32) -> np.ndarray:
    """dycol: fp64 [N, Mpad]; xcol: fp64 [K, Mpad]; returns fp64 [G, N, K].

    accumulate=True: main_grad0[g] + dW_g (empty experts keep main_grad0[g]);
    accumulate=False: dW_g (empty experts are zero).
    """
    _, pad_offs = segpad_offsets(m_splits, pad)
    G = len(pad_offs) - 1
    N, mpad = dycol.shape
    K = xcol.shape[0]
    if xcol.shape[1] != mpad or pad_offs[-1] != mpad:
        raise ValueError("shape mismatch")
    if accumulate:
        if main_grad0 is None or main_grad0.shape != (G, N, K):
            raise ValueError("accumulate needs main_grad0 [G, N, K]")
        out = np.array(main_grad0, dtype=np.float64, copy=True)
    else:
        out = np.zeros((G, N, K), dtype=np.float64)
    for g in range(G):
        p0, p1 = pad_offs[g], pad_offs[g + 1]
        if p1 > p0:
            out[g] += dycol[:, p0:p1] @ xcol[:, p0:p1].T
    return out
