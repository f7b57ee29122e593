"""fp64 bidirectional joint attention (oracle side; test infrastructure only).

Definition, for batch b, query head h, KV head g = h // (Hq / Hkv) and query
row i ("Krea 2 TileMix Attention (FP16/INT8 tiles)", "What it actually patches":
bidirectional softmax attention over the joint [text, image] sequence, 48 query
heads over 12 KV heads with the grouping of the stock repeat_interleave):

    O[b, i, h, :] = sum_j p_ij V[b, j, g, :],
    p_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij)   over admitted j.

Scores (sigma = the float32 softmax scale, default float32(1/sqrt(d)), widened):
  * dense, scanline, and FP16-routed tiles:  s_ij = sigma * q_i . (k_j - mu)
    with mu = the float32 smooth_k mean when smooth_k is on, else 0;
  * INT8-routed tiles (TileMix):  s_ij = sigma * sq[h, a] * sk[g, b] * (q8_i . k8_j)
    with the per-tile codes and scales of quant_ref.
Both routes enter one softmax per row -- the page's "one running softmax
state"; a running (online) softmax reaches the plain softmax exactly, so the
oracle uses the plain one.

Admitted keys: every key (dense, TileMix); the scanline mask of plan_ref
("Krea 2 Scanline Attention", "What the mask actually is").  Query slicing
("LayerStream: Krea2 Chunking", "What the node does to the block"): each slice
of q_chunk query positions attends against the full K/V; rows are independent,
so slicing leaves every output unchanged.
"""
from __future__ import annotations

import math

import numpy as np

from . import plan_ref, quant_ref

TILE = 128


def softmax_scale(head_dim: int, given: float = 0.0) -> float:
    """The float32 scale actually applied, widened to fp64."""
    s = np.float32(given) if given else np.float32(1.0 / math.sqrt(head_dim))
    return float(s)


def _softmax_pv(s: np.ndarray, adm: np.ndarray | None, vv: np.ndarray) -> np.ndarray:
    """Plain softmax over admitted keys, then P V, all fp64.  No admitted key -> 0."""
    if adm is not None:
        s = np.where(adm, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    den = np.sum(p, axis=1, keepdims=True)
    den = np.where(den > 0, den, 1.0)
    return (p / den) @ vv


class Oracle:
    """Prepared oracle for one set of inputs and one workload description.

    q: [B, N, Hq, d]; k, v: [B, N, Hkv, d]; float arrays holding the exact
    input values (bf16/fp16 widened).  ``w`` carries the mode arguments
    (attributes as in synth.Workload).
    """

    def __init__(self, q, k, v, w):
        self.q = np.asarray(q, dtype=np.float64)
        self.k = np.asarray(k, dtype=np.float64)
        self.v = np.asarray(v, dtype=np.float64)
        self.w = w
        b, n, hq, d = self.q.shape
        hkv = self.k.shape[2]
        if hq % hkv:
            raise ValueError("heads_q must be a multiple of heads_kv")
        self.n, self.hq, self.hkv, self.d = n, hq, hkv, d
        self.group = hq // hkv
        self.sigma = softmax_scale(d, getattr(w, "softmax_scale", 0.0))
        self.mode = w.mode
        self.kshift = self.k
        if self.mode == "tilemix":
            self.route = plan_ref.route_map(n, w.text_tokens, w.pattern, w.percentage,
                                            w.band_blocks, w.route_seed)
            self.m32 = quant_ref.k_mean(self.k) if w.smooth_k else None
            ks = quant_ref.smooth(self.k, self.m32)
            self.k8, self.sk, self.k_inv = quant_ref.quantize_tiles(ks)
            self.q8, self.sq, self.q_inv = quant_ref.quantize_tiles(self.q.astype(np.float32))
            if self.m32 is not None:
                self.kshift = self.k - self.m32.astype(np.float64)[:, None, :, :]
        elif self.mode == "scanline":
            plan_ref.check_window(w.window)
            self.lay = plan_ref.ScanLayout(w.text_tokens, w.img_rows, w.img_cols)
            if self.lay.text_tokens + self.lay.image_tokens != n:
                raise ValueError("text_tokens + img_rows * img_cols must equal N")
            self.bmask = plan_ref.block_mask(w.text_tokens, w.img_rows, w.img_cols,
                                             w.window, w.tile_aligned)
        elif self.mode != "dense":
            raise ValueError(f"unknown mode {self.mode!r}")

    # -- one (b, h) and a set of physical query rows ---------------------------
    def rows(self, b: int, h: int, rows: np.ndarray) -> np.ndarray:
        """fp64 outputs [len(rows), d] for physical query rows of head h, batch b."""
        rows = np.asarray(rows, dtype=np.int64)
        g = h // self.group
        qq = self.q[b, rows, h]
        if self.mode == "scanline":
            lay = self.lay
            logical = np.where(rows < lay.text_tokens, rows, rows + (lay.t_pad - lay.text_tokens))
            adm_l = plan_ref.admitted(lay, self.w.window, self.w.tile_aligned, logical, self.bmask)
            keys_l = np.arange(lay.length)
            keep = lay.valid(keys_l)
            phys = lay.physical(keys_l[keep])
            s = self.sigma * (qq @ self.k[b, phys, g].T)
            return _softmax_pv(s, adm_l[:, keep], self.v[b, phys, g])
        s = self.sigma * (qq @ self.kshift[b, :, g].T)
        if self.mode == "tilemix" and self.route.any():
            rb = rows // TILE
            cb = np.arange(self.n) // TILE
            is_i8 = self.route[rb][:, cb] == 1
            k8 = self.k8[b, g].reshape(-1, self.d)[: self.n]
            q8 = self.q8[b, h, rb, rows % TILE]
            acc = quant_ref.int_scores(q8, k8)
            s8 = (self.sigma * self.sq[b, h, rb].astype(np.float64)[:, None]
                  * self.sk[b, g, cb].astype(np.float64)[None, :] * acc)
            s = np.where(is_i8, s8, s)
        return _softmax_pv(s, None, self.v[b, :, g])

    # -- the whole call ---------------------------------------------------------
    def forward(self, row_chunk: int = 512, heads=None) -> np.ndarray:
        """fp64 O [B, N, Hq, d] (physical token order); ``heads`` limits the heads computed."""
        bsz = self.q.shape[0]
        out = np.zeros((bsz, self.n, self.hq, self.d), dtype=np.float64)
        heads = range(self.hq) if heads is None else heads
        q_chunk = getattr(self.w, "q_chunk", 0) or 0
        for s0, s1 in self.query_slices(q_chunk):
            for b in range(bsz):
                for h in heads:
                    for r0 in range(s0, s1, row_chunk):
                        rows = np.arange(r0, min(s1, r0 + row_chunk))
                        out[b, rows, h] = self.rows(b, h, rows)
        return out

    def query_slices(self, q_chunk: int):
        """Physical row ranges of each query slice of q_chunk logical positions."""
        if self.mode == "scanline":
            lay = self.lay
            length = lay.length
            bounds = []
            step = q_chunk if q_chunk > 0 else length
            for l0 in range(0, length, step):
                lpos = np.arange(l0, min(length, l0 + step))
                phys = lay.physical(lpos)
                phys = phys[phys >= 0]
                if phys.size:
                    bounds.append((int(phys[0]), int(phys[-1]) + 1))
            return bounds
        step = q_chunk if q_chunk > 0 else self.n
        return [(s, min(self.n, s + step)) for s in range(0, self.n, step)]


def attention(q, k, v, w, row_chunk: int = 512) -> np.ndarray:
    """Convenience: fp64 output of the whole call."""
    return Oracle(q, k, v, w).forward(row_chunk=row_chunk)
