"""Pins of the block-context oracle (oracle/block_ref.py) against things other than
itself: a pure-Python evaluation of the definition on a tiny case, the exact value of the
gate at zero, the identity projection, constant scores, and additivity in y0."""
import math

import numpy as np
import pytest

from oracle import attn_ref, block_ref
from synth import Workload


def _w(**kw):
    base = dict(name="blk", batch=1, heads_q=2, heads_kv=1, head_dim=3, text_tokens=2, img_rows=2, img_cols=2,
                dtype="bf16", seed=0, mode="dense")
    base.update(kw)
    return Workload(**base)


def _inputs(w, d_model, seed=0, scale=0.5):
    rng = np.random.default_rng(seed)
    n = w.tokens
    hd = w.head_dim
    x = rng.standard_normal((w.batch, n, d_model))
    wq = rng.standard_normal((d_model, w.heads_q * hd)) * scale
    wk = rng.standard_normal((d_model, w.heads_kv * hd)) * scale
    wv = rng.standard_normal((d_model, w.heads_kv * hd)) * scale
    wg = rng.standard_normal((d_model, w.heads_q * hd)) * scale
    wo = rng.standard_normal((w.heads_q * hd, d_model)) * scale
    y0 = rng.standard_normal((w.batch, n, d_model))
    return x, wq, wk, wv, wg, wo, y0


def _brute(x, wq, wk, wv, wg, wo, y0, w):
    """The definition, one scalar at a time."""
    b_, n, dm = x.shape
    hq, hkv, d = w.heads_q, w.heads_kv, w.head_dim
    sigma = float(np.float32(1.0 / math.sqrt(d)))
    y = [[[float(y0[b][i][c]) for c in range(dm)] for i in range(n)] for b in range(b_)]

    def proj(b, i, wm, col):
        return sum(float(x[b][i][r]) * float(wm[r][col]) for r in range(dm))

    for b in range(b_):
        for i in range(n):
            og = []
            for h in range(hq):
                g = h // (hq // hkv)
                q = [proj(b, i, wq, h * d + c) for c in range(d)]
                s = []
                for j in range(n):
                    k = [proj(b, j, wk, g * d + c) for c in range(d)]
                    s.append(sigma * sum(q[c] * k[c] for c in range(d)))
                mx = max(s)
                e = [math.exp(t - mx) for t in s]
                den = sum(e)
                for c in range(d):
                    o = sum(e[j] / den * proj(b, j, wv, g * d + c) for j in range(n))
                    gate = proj(b, i, wg, h * d + c)
                    og.append(o / (1.0 + math.exp(-gate)))
            for col in range(dm):
                y[b][i][col] += sum(og[r] * float(wo[r][col]) for r in range(hq * d))
    return np.array(y)


def test_block_matches_scalar_definition():
    w = _w(batch=2)
    args = _inputs(w, d_model=5)
    got = block_ref.block_context(*args, w)
    want = _brute(*args, w)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_sigmoid_tails_and_midpoint():
    x = np.array([-800.0, -40.0, -1.0, 0.0, 1.0, 40.0, 800.0])
    s = block_ref.sigmoid(x)
    assert s[3] == 0.5 and s[0] == 0.0 and s[-1] == 1.0
    assert np.all(np.isfinite(s)) and np.all(np.diff(s) >= 0)
    assert abs(s[2] + s[4] - 1.0) <= 1e-16
    assert abs(s[4] - 1.0 / (1.0 + math.exp(-1.0))) <= 1e-16


@pytest.mark.parametrize("w", [
    _w(heads_q=4, heads_kv=2, head_dim=8, text_tokens=40, img_rows=6, img_cols=20),
    _w(heads_q=4, heads_kv=1, head_dim=16, text_tokens=130, img_rows=12, img_cols=20, mode="tilemix",
       pattern="band", percentage=0.6, band_blocks=0, smooth_k=True),
    _w(heads_q=4, heads_kv=2, head_dim=8, text_tokens=77, img_rows=9, img_cols=30, mode="scanline", window=3,
       tile_aligned=False),
], ids=["dense", "tilemix", "scanline"])
def test_gate_at_zero_halves_the_context(w):
    """sigmoid(0) = 1/2 exactly, so with W_gate = 0 and W_o = I the context is half of the
    attention of the projections (the attention oracle is pinned on its own)."""
    dm = w.heads_q * w.head_dim
    x, wq, wk, wv, _, _, y0 = _inputs(w, d_model=dm, seed=3)
    wg = np.zeros((dm, dm))
    wo = np.eye(dm)
    got = block_ref.block_context(x, wq, wk, wv, wg, wo, y0, w)
    q = block_ref.project(x, wq, w.heads_q)
    k = block_ref.project(x, wk, w.heads_kv)
    v = block_ref.project(x, wv, w.heads_kv)
    o = attn_ref.attention(q, k, v, w)
    want = y0 + 0.5 * o.reshape(o.shape[0], o.shape[1], -1)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_constant_scores_give_the_mean_of_v():
    """W_q = 0 makes every score 0, so each row attends uniformly: the context is the mean
    of V (per KV head) gated and projected."""
    w = _w(heads_q=4, heads_kv=2, head_dim=4, text_tokens=10, img_rows=3, img_cols=7)
    dm = 12
    x, _, wk, wv, wg, wo, y0 = _inputs(w, d_model=dm, seed=5)
    wq = np.zeros((dm, w.heads_q * w.head_dim))
    got = block_ref.block_context(x, wq, wk, wv, wg, wo, y0, w)
    v = (x @ wv).reshape(1, w.tokens, w.heads_kv, w.head_dim)
    vmean = v.mean(axis=1)                                   # [1, Hkv, d]
    o = np.repeat(vmean, w.heads_q // w.heads_kv, axis=1)    # [1, Hq, d], the same for every row
    gate = block_ref.sigmoid((x @ wg).reshape(1, w.tokens, w.heads_q, w.head_dim))
    want = y0 + ((o[:, None] * gate).reshape(1, w.tokens, -1)) @ wo
    assert np.max(np.abs(got - want)) <= 1e-12


def test_y0_is_added_once():
    w = _w(heads_q=4, heads_kv=1, head_dim=4, text_tokens=8, img_rows=2, img_cols=5)
    args = list(_inputs(w, d_model=6, seed=7))
    with_y = block_ref.block_context(*args, w)
    args[-1] = np.zeros_like(args[-1])
    without = block_ref.block_context(*args, w)
    y0 = _inputs(w, d_model=6, seed=7)[-1]
    assert np.max(np.abs(with_y - without - y0)) <= 1e-12


@pytest.mark.parametrize("mode", ["dense", "tilemix", "scanline"])
def test_sampled_rows_equal_the_whole(mode):
    extra = dict(pattern="band", percentage=0.5, band_blocks=0, smooth_k=True) if mode == "tilemix" else {}
    w = _w(heads_q=4, heads_kv=1, head_dim=16, text_tokens=100, img_rows=8, img_cols=25, mode=mode, **extra)
    args = _inputs(w, d_model=64, seed=11)
    ora = block_ref.BlockOracle(*args, w)
    full = ora.forward()
    rows = np.array([0, 5, 99, 100, 129, 250, 299])
    part = ora.rows(0, rows)
    assert np.max(np.abs(part - full[0, rows])) <= 1e-12 * max(1.0, np.max(np.abs(full)))


def test_dense_block_equals_torch_composition():
    """Dense mode against the same algebra built from torch's CPU library routines in fp64:
    scaled_dot_product_attention on repeat_interleave-expanded K/V (the GQA grouping), a
    logistic gate and two matrix products -- code the oracle does not share."""
    torch = pytest.importorskip("torch")
    w = _w(heads_q=6, heads_kv=2, head_dim=8, text_tokens=9, img_rows=3, img_cols=5, batch=2)
    dm = 20
    x, wq, wk, wv, wg, wo, y0 = _inputs(w, d_model=dm, seed=13)
    got = block_ref.block_context(x, wq, wk, wv, wg, wo, y0, w)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    X = t(x)
    b, n = x.shape[0], x.shape[1]
    d, g = w.head_dim, w.heads_q // w.heads_kv
    Q = (X @ t(wq)).reshape(b, n, w.heads_q, d).transpose(1, 2)
    K = (X @ t(wk)).reshape(b, n, w.heads_kv, d).transpose(1, 2).repeat_interleave(g, dim=1)
    V = (X @ t(wv)).reshape(b, n, w.heads_kv, d).transpose(1, 2).repeat_interleave(g, dim=1)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)  # [b, Hq, n, d]
    G = torch.sigmoid((X @ t(wg)).reshape(b, n, w.heads_q, d).transpose(1, 2))
    want = t(y0) + ((O * G).transpose(1, 2).reshape(b, n, -1) @ t(wo))
    assert np.max(np.abs(got - want.numpy())) <= 1e-12 * max(1.0, float(want.abs().max()))
