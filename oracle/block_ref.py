"""fp64 attention context of one Krea 2 DiT block (oracle side; test infrastructure only).

"LayerStream: Krea2 Chunking", "What the node does to the block": the block's attention
runs in two passes.  Pass one projects K and V for every token.  Pass two takes the query
tokens a slice at a time, projects their q and their attention gate, attends against the
full K/V, projects the gated result and adds it into the residual stream.  Rows are
independent once K and V exist, so the slicing changes no value here ("Be clear about
exactness": a single slice is exact; with several, only the rounding of the projections
moves).

    K = x W_k,  V = x W_v                          [B, N, Hkv, d]   (every token)
    Q = x W_q,  G = x W_gate                       [B, N, Hq, d]
    O = attention(Q, K, V)                         (attn_ref: dense, TileMix, scanline)
    y = y0 + (O * sigmoid(G)) W_o                  [B, N, D]

Readings (the pages give the two passes, not the block's algebra): the projections are
plain matrix products of the token rows (x [B, N, D] @ W [D, out], no bias); no
normalisation or rotation of q and k sits on this path; the gate multiplies the attention
output elementwise through a logistic sigmoid before the output projection.  Everything is
fp64 from the exact input values.
"""
from __future__ import annotations

import numpy as np

from . import attn_ref


def sigmoid(x: np.ndarray) -> np.ndarray:
    """The logistic function, evaluated so that it neither overflows nor loses the tails."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def project(x: np.ndarray, w: np.ndarray, heads: int) -> np.ndarray:
    """x [B, N, D] @ w [D, heads * d] -> [B, N, heads, d], fp64."""
    b, n, _ = x.shape
    out = np.asarray(x, np.float64) @ np.asarray(w, np.float64)
    return out.reshape(b, n, heads, -1)


class BlockOracle:
    """The block context for one set of inputs.  ``w`` carries the attention arguments
    (attributes as in synth.Workload); weights are [D, out] arrays of exact values."""

    def __init__(self, x, wq, wk, wv, wg, wo, y0, w):
        self.w = w
        self.x = np.asarray(x, np.float64)
        self.wq, self.wg, self.wo = (np.asarray(a, np.float64) for a in (wq, wg, wo))
        self.y0 = np.asarray(y0, np.float64)
        # pass one: K and V of every token
        self.k = project(self.x, wk, w.heads_kv)
        self.v = project(self.x, wv, w.heads_kv)

    def _pass_two(self, b: int, q_rows: np.ndarray, rows: np.ndarray) -> np.ndarray:
        """y[b, rows, :] given q for ``q_rows`` (a superset of ``rows``: TileMix scales Q per
        128-token tile, so the tiles holding ``rows`` must be whole)."""
        w = self.w
        xq = self.x[b:b + 1, q_rows]
        q = np.zeros((1, self.x.shape[1], w.heads_q, self.k.shape[3]))
        q[0, q_rows] = project(xq, self.wq, w.heads_q)[0]
        g = project(self.x[b:b + 1, rows], self.wg, w.heads_q)[0]   # [R, Hq, d]
        ora = attn_ref.Oracle(q, self.k[b:b + 1], self.v[b:b + 1], w.with_(batch=1))
        o = np.stack([ora.rows(0, h, rows) for h in range(w.heads_q)], axis=1)  # [R, Hq, d]
        og = (o * sigmoid(g)).reshape(len(rows), -1)
        return self.y0[b, rows] + og @ self.wo

    def rows(self, b: int, rows: np.ndarray) -> np.ndarray:
        """y[b, rows, :] for the given physical token rows."""
        rows = np.asarray(rows, dtype=np.int64)
        n = self.x.shape[1]
        blocks = np.unique(rows // attn_ref.TILE)
        q_rows = np.concatenate([np.arange(a * attn_ref.TILE, min(n, (a + 1) * attn_ref.TILE)) for a in blocks])
        return self._pass_two(b, q_rows, rows)

    def forward(self) -> np.ndarray:
        n = self.x.shape[1]
        y = np.empty(self.y0.shape)
        every = np.arange(n)
        for b in range(self.x.shape[0]):
            y[b] = self._pass_two(b, every, every)
        return y


def block_context(x, wq, wk, wv, wg, wo, y0, w) -> np.ndarray:
    """y = y0 + (attention(x W_q, x W_k, x W_v) * sigmoid(x W_gate)) W_o, fp64."""
    return BlockOracle(x, wq, wk, wv, wg, wo, y0, w).forward()
