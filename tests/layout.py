"""The inference layout of bf16 weights, restated in numpy for the tests.

While the LoRA adapters are folded in, the library keeps every bf16 projection
W[N][K] (and the tied embedding) in an MFMA-friendly order: W is cut into blocks of
16 rows x BW columns (BW the largest power of two <= 512 dividing K); each block
stays where it is, but its 16-byte units (8 consecutive k of one row) are
reordered so that the 16 x 32 operand of one MFMA k-step is 1 KB of consecutive
bytes, lane l holding row l % 16 and k 8 (l // 16) .. + 8.  Unit (row j, unit
column u) of a block moves to position p = (u // 4) * 64 + (u % 4) * 16 + j.
"""
import numpy as np


def block_width(K):
    bw = 512
    while bw > 32 and K % bw:
        bw //= 2
    return bw


def _positions(upr):
    j = np.arange(16)[:, None]
    u = np.arange(upr)[None, :]
    return (u // 4) * 64 + (u % 4) * 16 + j          # [16, upr]


def to_inference(W):
    """Row-major [N, K] -> the stored inference layout (same shape, same dtype)."""
    W = np.asarray(W)
    N, K = W.shape
    bw = block_width(K)
    upr = bw // 8
    rm = W.reshape(N // 16, 16, K // bw, upr, 8).transpose(0, 2, 1, 3, 4)    # [rb, c, j, u, 8]
    lin = np.empty((N // 16, K // bw, 16 * upr, 8), dtype=W.dtype)
    lin[:, :, _positions(upr), :] = rm
    return lin.reshape(N // 16, K // bw, 16, upr, 8).transpose(0, 2, 1, 3, 4).reshape(N, K)


def from_inference(S):
    """The stored inference layout [N, K] -> row-major."""
    S = np.asarray(S)
    N, K = S.shape
    bw = block_width(K)
    upr = bw // 8
    lin = S.reshape(N // 16, 16, K // bw, upr, 8).transpose(0, 2, 1, 3, 4).reshape(N // 16, K // bw, 16 * upr, 8)
    rm = lin[:, :, _positions(upr), :]                                       # [rb, c, j, u, 8]
    return rm.transpose(0, 2, 1, 3, 4).reshape(N, K)
