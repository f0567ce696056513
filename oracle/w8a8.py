"""Per-block W8A8 INT8 linear layer, written out plainly (test infrastructure
only; the HIP library never imports this).

The Vidu S1 blog (section "Infra") says per-tensor and per-channel
quantization of linear layers let outliers widen the quantization range and
lose precision, so a per-block W8A8 quantized GEMM was used instead; the
TurboDiffusion digests add that weights and activations are quantized to 8
bits block-wise and multiplied on the INT8 matrix units.  Block shapes and
the scale rule are not on the pages; the library's reading:

  Y[m, n] = bias[n] + sum_kb  dx[m, kb] * dw[n // 128, kb] * S_kb[m, n]
  S_kb[m, n] = sum over k in block kb (128 channels) of xq[m, k] * wq[n, k]

* X [M, K] (activations): one scale per (row, 128-channel group) -- a
  channel outlier only widens its own group of its own token;
* W [N, K] (weights): one scale per 128 x 128 tile;
* each block: delta = fp32(amax / 127), code = clamp(rint(fp32(x *
  fp32(127 / amax))), -127, 127), ties to even; an all-zero block has delta 0
  and codes 0 -- the same rule as the attention's Q and K blocks.

S_kb is an exact integer; ``gemm_exact`` evaluates Y in float64 (exact up to
the final sum's rounding), the value the GPU's float32 arithmetic
approximates.
"""

import numpy as np

from .constants import QMAX

GROUP = 128   # K channels per block (activations and weights); N rows per weight block


def quant_tiles(X, rows, cols):
    """Symmetric INT8 quantization of float32 X [R, C] in tiles of rows x cols
    (R and C multiples of the tile).  Returns codes int8 [R, C] and delta
    float32 [R // rows, C // cols]."""
    X = np.asarray(X, dtype=np.float32)
    R, C = X.shape
    assert R % rows == 0 and C % cols == 0
    t = X.reshape(R // rows, rows, C // cols, cols)
    amax = np.abs(t).max(axis=(1, 3))                                   # [R/rows, C/cols]
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1)).astype(np.float32)
    delta = np.where(nz, (safe / np.float32(QMAX)).astype(np.float32), np.float32(0)).astype(np.float32)
    inv = (np.float32(QMAX) / safe).astype(np.float32)
    y = (t * inv[:, None, :, None]).astype(np.float32)
    codes = np.where(nz[:, None, :, None], np.clip(np.rint(y), -QMAX, QMAX), 0).astype(np.int8)
    return codes.reshape(R, C), delta


def quantize_act(X):
    """X [M, K] -> codes int8 [M, K], delta float32 [M, K/128] (per row and group)."""
    return quant_tiles(X, 1, GROUP)


def quantize_weight(W):
    """W [N, K] -> codes int8 [N, K], delta float32 [N/128, K/128]."""
    return quant_tiles(W, GROUP, GROUP)


def block_products(xq, wq):
    """Exact integer S_kb [K/128, M, N] (float64 products of integers below 2^53)."""
    M, K = xq.shape
    out = np.empty((K // GROUP, M, wq.shape[0]))
    for kb in range(K // GROUP):
        s = slice(kb * GROUP, (kb + 1) * GROUP)
        out[kb] = xq[:, s].astype(np.float64) @ wq[:, s].astype(np.float64).T
    return out


def gemm_exact(xq, dx, wq, dw, bias=None):
    """Y = bias + sum_kb dx dw S_kb in float64 [M, N]; also returns
    sum_kb |dx dw S_kb| (what bounds float32 accumulation error)."""
    S = block_products(xq, wq)                                          # [KB, M, N]
    n_blk = np.arange(wq.shape[0]) // GROUP
    scale = dx.T.astype(np.float64)[:, :, None] * dw[n_blk].T.astype(np.float64)[:, None, :]  # [KB, M, N]
    terms = scale * S
    y = terms.sum(axis=0)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y, np.abs(terms).sum(axis=0)


def linear_fp64(X, W, bias=None):
    """The unquantized layer X W^T + bias in float64."""
    y = np.asarray(X, np.float64) @ np.asarray(W, np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y
