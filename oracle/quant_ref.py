"""smooth_k mean-centring and per-tile symmetric INT8 (oracle side; test infrastructure only).

"Krea 2 TileMix Attention (FP16/INT8 tiles)", section "The inputs that matter":
``smooth_k`` mean-centres K per head before quantisation; because it subtracts
the same vector from every key, each query's scores shift by one constant and
softmax is unchanged.  Section "What it actually patches": part of the score
matrix is computed in INT8.

The pages give no rounding rule, so this follows a stated reading that makes
every INT8 code reproducible bit for bit, with each operation a single
correctly rounded IEEE op:
  1. Column sums of K per (batch, KV head, channel) in fp64: tokens of each
     128-token block summed one after another in token order, then the block
     partials one after another in block order.  mean64 = sum / N (fp64),
     m32 = float32(mean64) (round to nearest even).
  2. K_s = float32(K) - m32 in float32 (smooth_k on), else float32(K).
  3. Per 128-token x head_dim tile of one (batch, head, block), over valid
     rows only: a = max |x|.  a == 0 gives all-zero codes and scale 0.
     Otherwise inv = float32(127 / a), scale = float32(a / 127),
     code = clamp(rint(float32(x * inv)), -127, 127), rint = half to even.
"""
from __future__ import annotations

import numpy as np

TILE = 128


def k_mean(k: np.ndarray) -> np.ndarray:
    """float32 [B, Hkv, d] mean of K over all N tokens, fixed-order fp64 sums.

    ``k`` holds the exact input values, [B, N, Hkv, d], any float dtype.
    """
    k = np.asarray(k, dtype=np.float64)
    b, n, h, d = k.shape
    total = np.zeros((b, h, d), dtype=np.float64)
    for start in range(0, n, TILE):
        part = np.zeros((b, h, d), dtype=np.float64)
        for t in range(start, min(n, start + TILE)):
            part = part + k[:, t]
        total = total + part
    mean64 = total / np.float64(n)
    return mean64.astype(np.float32)


def smooth(k: np.ndarray, m32: np.ndarray | None) -> np.ndarray:
    """K_s = float32(K) - m32 in float32; m32 None means smooth_k off."""
    k32 = np.asarray(k).astype(np.float32)
    if m32 is None:
        return k32
    return (k32 - m32[:, None, :, :]).astype(np.float32)


def quantize_tiles(x32: np.ndarray):
    """Per-tile symmetric INT8 of a float32 [B, N, H, d] tensor.

    Returns (codes int8 [B, H, nb, 128, d] with rows past N zero,
    scale float32 [B, H, nb], inv float32 [B, H, nb]).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    b, n, h, d = x32.shape
    nb = (n + TILE - 1) // TILE
    codes = np.zeros((b, h, nb, TILE, d), dtype=np.int8)
    scale = np.zeros((b, h, nb), dtype=np.float32)
    inv = np.zeros((b, h, nb), dtype=np.float32)
    one27 = np.float32(127.0)
    for blk in range(nb):
        rows = slice(blk * TILE, min(n, blk * TILE + TILE))
        tile = np.transpose(x32[:, rows], (0, 2, 1, 3))  # [B, H, rows, d]
        a = np.max(np.abs(tile), axis=(2, 3))  # [B, H], exact
        for bi in range(b):
            for hi in range(h):
                amax = a[bi, hi]
                if amax == 0:
                    continue
                iv = np.float32(one27 / amax)
                sc = np.float32(amax / one27)
                y = (tile[bi, hi] * iv).astype(np.float32)
                q = np.clip(np.rint(y), -127, 127).astype(np.int8)
                codes[bi, hi, blk, :q.shape[0]] = q
                scale[bi, hi, blk] = sc
                inv[bi, hi, blk] = iv
    return codes, scale, inv


def int_scores(q_codes: np.ndarray, k_codes: np.ndarray) -> np.ndarray:
    """Exact INT32 dot products of two INT8 tiles [rows, d] x [cols, d] -> [rows, cols].

    |sum| <= d * 127^2 < 2^53, so an fp64 product of the integer values is exact.
    """
    return q_codes.astype(np.float64) @ k_codes.astype(np.float64).T
