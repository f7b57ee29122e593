"""Seeded synthetic inputs for the Krea 2 joint-attention workloads.

This module only draws random numbers and names the workloads; it holds none of
the attention arithmetic, so both the fp64 CPU oracle and the HIP path can take
their inputs from it without sharing any of the method.

Recipe (one generator per workload, numpy PCG64 ``default_rng(seed)``):
  1. Q  = standard_normal([B, N, Hq, d])  (float32 draw)
  2. Z  = standard_normal([B, N, Hkv, d])
  3. c  = normal(0, offset_std, [B, 1, Hkv, d])   (only when offset_std > 0)
  4. V  = standard_normal([B, N, Hkv, d])
  K = Z + c (float32), then every tensor is cast to the target dtype by
  round-to-nearest-even (torch CPU cast).  Tokens are laid out text first, then
  the image grid row by row, as in the joint [text, image] sequence that the
  Krea 2 TileMix Attention page describes ("What it actually patches").

The per-KV-head channel offset on K stands in for keys "with a shared channel
offset", the case the TileMix page's ``smooth_k`` option targets ("The inputs
that matter").  Unit-variance inputs follow the same page's accuracy regime of
"adversarial random inputs" ("What speedup to expect").
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """One attention call: shapes, input distribution and mode arguments."""

    name: str
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    text_tokens: int
    img_rows: int
    img_cols: int
    dtype: str  # "bf16" | "f16"
    seed: int
    offset_std: float = 0.0
    mode: str = "dense"  # "dense" | "tilemix" | "scanline"
    pattern: str = "zero"  # "zero" | "one" | "band"
    percentage: float = 0.5
    band_blocks: int = 2
    route_seed: int = 0
    smooth_k: bool = False
    window: int = 11
    tile_aligned: bool = True
    q_chunk: int = 0
    softmax_scale: float = 0.0  # 0 -> fp32(1/sqrt(head_dim))
    notes: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.text_tokens + self.img_rows * self.img_cols

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


_KREA_1MP = dict(batch=1, heads_q=48, heads_kv=12, head_dim=128, text_tokens=512,
                 img_rows=64, img_cols=64, dtype="bf16", seed=1001, offset_std=0.5)
_KREA_4MP = dict(batch=1, heads_q=48, heads_kv=12, head_dim=128, text_tokens=512,
                 img_rows=128, img_cols=128, dtype="bf16", seed=1005, offset_std=0.5)

WORKLOADS: Dict[str, Workload] = {
    # tiny dense case: 4 q heads over 1 KV head, 64 text + 8x8 image tokens, fp16
    "tiny": Workload(name="tiny", batch=1, heads_q=4, heads_kv=1, head_dim=128,
                     text_tokens=64, img_rows=8, img_cols=8, dtype="f16", seed=1000,
                     mode="dense"),
    # 1 MP Krea 2 shape (1024x1024 -> 64x64 token grid), dense
    "1mp_dense": Workload(name="1mp_dense", mode="dense", **_KREA_1MP),
    # 1 MP TileMix band: +-2 key blocks FP16, 50% of the rest INT8, smooth_k on
    "1mp_band": Workload(name="1mp_band", mode="tilemix", pattern="band", percentage=0.5,
                         band_blocks=2, smooth_k=True, **_KREA_1MP),
    # 1 MP scanline: window 11 (+-5 rows), tile-aligned block mask
    "1mp_scanline": Workload(name="1mp_scanline", mode="scanline", window=11,
                             tile_aligned=True, **_KREA_1MP),
    # 4 MP TileMix band, 75% INT8, queries sliced 4096 at a time against full K/V
    "4mp_band": Workload(name="4mp_band", mode="tilemix", pattern="band", percentage=0.75,
                         band_blocks=2, smooth_k=True, q_chunk=4096, **_KREA_4MP),
    # 4 MP dense on the same tensors (comparator for the band mode)
    "4mp_dense": Workload(name="4mp_dense", mode="dense", **_KREA_4MP),
    "4mp_dense_sliced": Workload(name="4mp_dense_sliced", mode="dense", q_chunk=4096, **_KREA_4MP),
    # 4 MP scanline: 128x128 grid, one 128-token tile per grid row, window 11 (+-5 tiles)
    "4mp_scanline": Workload(name="4mp_scanline", mode="scanline", window=11, tile_aligned=True, **_KREA_4MP),
    # 1 MP scanline with the exact row rule (no tile alignment): partial tiles masked per element
    "1mp_scanline_exact": Workload(name="1mp_scanline_exact", mode="scanline", window=11,
                                   tile_aligned=False, **_KREA_1MP),
}

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def make_qkv(w: Workload):
    """Draw Q, K, V for workload ``w`` as CPU tensors [B, N, H, d] in w.dtype."""
    rng = np.random.default_rng(w.seed)
    n = w.tokens
    q = rng.standard_normal((w.batch, n, w.heads_q, w.head_dim), dtype=np.float32)
    z = rng.standard_normal((w.batch, n, w.heads_kv, w.head_dim), dtype=np.float32)
    if w.offset_std > 0:
        c = rng.normal(0.0, w.offset_std, size=(w.batch, 1, w.heads_kv, w.head_dim)).astype(np.float32)
        k = z + c
    else:
        k = z
    v = rng.standard_normal((w.batch, n, w.heads_kv, w.head_dim), dtype=np.float32)
    dt = _TORCH_DTYPE[w.dtype]
    return (torch.from_numpy(q).to(dt), torch.from_numpy(k).to(dt), torch.from_numpy(v).to(dt))


def random_case(seed: int, batch: int, heads_q: int, heads_kv: int, head_dim: int,
                tokens: int, dtype: str = "bf16", offset_std: float = 0.0):
    """Generic seeded Q/K/V of arbitrary size (for small parity and edge cases)."""
    w = Workload(name="case", batch=batch, heads_q=heads_q, heads_kv=heads_kv,
                 head_dim=head_dim, text_tokens=tokens, img_rows=0, img_cols=0,
                 dtype=dtype, seed=seed, offset_std=offset_std)
    return make_qkv(w)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16/fp16 CPU tensor to a float64 numpy array."""
    return t.to(torch.float64).numpy()


def text_outlier_case(w: Workload, text_scale: float = 4.0, outlier_channel: int = 7,
                      outlier_value: float = 24.0):
    """Q, K, V of workload ``w`` with the text tokens made adversarial for per-tile INT8:
    text rows of Q and K scaled by ``text_scale`` and one K channel of every text token set
    to ``outlier_value`` (text-encoder activations run larger than image ones and carry
    outlier channels).  Returns CPU tensors in w.dtype."""
    q, k, v = make_qkv(w)
    t = w.text_tokens
    qf, kf = q.float(), k.float()
    qf[:, :t] *= text_scale
    kf[:, :t] *= text_scale
    kf[:, :t, :, outlier_channel] = outlier_value
    dt = _TORCH_DTYPE[w.dtype]
    return qf.to(dt), kf.to(dt), v


def make_gate(shape, dtype: str, seed: int, std: float = 2.0) -> torch.Tensor:
    """A seeded attention-gate tensor of the given shape (N(0, std) drawn in float32, cast by
    round-to-nearest-even), as a CPU tensor in ``dtype``."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(tuple(shape), dtype=np.float32) * np.float32(std)
    return torch.from_numpy(g).to(_TORCH_DTYPE[dtype])


def make_block_inputs(w: Workload, d_model: int, seed: int):
    """Seeded inputs of one block's attention context for workload ``w`` (heads and tokens
    from ``w``): x [B, N, D] ~ N(0, 1); W_q, W_gate [D, Hq d], W_k, W_v [D, Hkv d] and W_o
    [Hq d, D] ~ N(0, 1/D) and N(0, 1/(Hq d)) (unit-variance projections of unit-variance
    rows); y0 [B, N, D] ~ N(0, 1), the residual the context is added into.  CPU tensors in
    w.dtype, drawn in this order."""
    rng = np.random.default_rng(seed)
    n, hq, hkv, d = w.tokens, w.heads_q, w.heads_kv, w.head_dim
    dt = _TORCH_DTYPE[w.dtype]

    def draw(shape, std):
        return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).to(dt)

    x = draw((w.batch, n, d_model), 1.0)
    wq = draw((d_model, hq * d), d_model ** -0.5)
    wk = draw((d_model, hkv * d), d_model ** -0.5)
    wv = draw((d_model, hkv * d), d_model ** -0.5)
    wg = draw((d_model, hq * d), d_model ** -0.5)
    wo = draw((hq * d, d_model), (hq * d) ** -0.5)
    y0 = draw((w.batch, n, d_model), 1.0)
    return x, wq, wk, wv, wg, wo, y0
