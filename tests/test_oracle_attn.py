"""Pins for the oracle's fp64 attention (CPU only).

Independent anchors: pure-Python brute force on tiny inputs, torch's own
scaled_dot_product_attention in fp64 (a library special case, with K/V
expanded by repeat_interleave as the stock Krea path does), closed forms, and
the invariants the pages state (zero pattern = plain attention, smooth_k exact
for softmax, a window covering every row = dense, query slices = one pass).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attn_ref, plan_ref, quant_ref
from synth import Workload, make_qkv, to_f64


def _w(**kw):
    base = dict(name="t", batch=1, heads_q=4, heads_kv=2, head_dim=16, text_tokens=20,
                img_rows=0, img_cols=0, dtype="bf16", seed=1, mode="dense")
    base.update(kw)
    return Workload(**base)


def _inputs(w):
    q, k, v = make_qkv(w)
    return to_f64(q), to_f64(k), to_f64(v)


def test_brute_force_tiny_gqa():
    w = _w(batch=2, heads_q=4, heads_kv=2, head_dim=8, text_tokens=11, img_rows=3, img_cols=5)
    q, k, v = _inputs(w)
    out = attn_ref.attention(q, k, v, w)
    sigma = float(np.float32(1 / math.sqrt(8)))
    n = w.tokens
    for b in range(2):
        for h in range(4):
            g = h // 2
            for i in range(n):
                s = [sigma * sum(q[b, i, h, c] * k[b, j, g, c] for c in range(8)) for j in range(n)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                z = sum(e)
                for c in range(8):
                    want = sum(e[j] * v[b, j, g, c] for j in range(n)) / z
                    assert abs(out[b, i, h, c] - want) < 1e-12


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (6, 1)])
def test_dense_matches_torch_sdpa_fp64(hq, hkv):
    w = _w(heads_q=hq, heads_kv=hkv, head_dim=128, text_tokens=40, img_rows=9, img_cols=13)
    q, k, v = _inputs(w)
    out = attn_ref.attention(q, k, v, w)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    sigma = float(np.float32(1 / math.sqrt(128)))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=sigma)
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.abs(out - ref).max() < 1e-12


def test_explicit_scale_is_used():
    w = _w(head_dim=16, softmax_scale=0.3)
    q, k, v = _inputs(w)
    out = attn_ref.attention(q, k, v, w)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=float(np.float32(0.3)))
    assert np.abs(out - ref.permute(0, 2, 1, 3).numpy()).max() < 1e-12


def test_closed_forms():
    w = _w(head_dim=16, text_tokens=50)
    q, k, v = _inputs(w)
    # every V row the same vector -> output is that vector
    v_const = np.broadcast_to(v[:, :1], v.shape).copy()
    out = attn_ref.attention(q, k, v_const, w)
    assert np.abs(out - np.repeat(v_const[:, :, [0, 0, 1, 1]], 1, axis=2)).max() < 1e-12
    # Q = 0 -> uniform weights -> mean of V over all keys
    out0 = attn_ref.attention(np.zeros_like(q), k, v, w)
    mean_v = v.mean(axis=1)  # [B, Hkv, d]
    for h in range(4):
        assert np.abs(out0[:, :, h] - mean_v[:, None, h // 2]).max() < 1e-12
    # one dominant logit: key 7 aligned with every query, large -> output ~ v[7]
    k2 = k.copy()
    q2 = np.ones_like(q)
    k2[:, 7] = 40.0
    out2 = attn_ref.attention(q2, k2, v, w)
    for h in range(4):
        assert np.abs(out2[:, :, h] - v[:, 7:8, h // 2]).max() < 1e-9


def test_zero_pattern_is_plain_attention_and_smooth_k_exact():
    w = _w(heads_q=8, heads_kv=2, head_dim=128, text_tokens=100, img_rows=10, img_cols=20,
           offset_std=0.5)
    q, k, v = _inputs(w)
    dense = attn_ref.attention(q, k, v, w)
    z_off = attn_ref.attention(q, k, v, w.with_(mode="tilemix", pattern="zero", smooth_k=False))
    z_on = attn_ref.attention(q, k, v, w.with_(mode="tilemix", pattern="zero", smooth_k=True))
    assert (z_off == dense).all()
    assert np.abs(z_on - dense).max() < 1e-12


def _integer_case(offset):
    """Integer-valued Q and K tiles whose absmax is exactly 127 in every tile, and
    K = Z + offset with Z antisymmetric across the two halves (every column sums
    to zero): then the INT8 codes are the values themselves, every scale is 1,
    and smooth_k recovers Z exactly."""
    rng = np.random.default_rng(21)
    n, hq, hkv, d = 512, 4, 2, 128
    q = rng.integers(-127, 128, size=(1, n, hq, d)).astype(np.float64)
    q[0, ::128, :, 0] = 127
    zh = rng.integers(-127, 128, size=(1, n // 2, hkv, d)).astype(np.float64)
    zh[0, ::128, :, 0] = 127
    z = np.concatenate([zh, -zh], axis=1)
    k = z + offset
    v = rng.standard_normal((1, n, hkv, d))
    return q, k, v, z


def test_int8_route_is_exact_on_integer_tiles():
    # with unit scales and exact codes, the INT8 route must reproduce the dense
    # scores: any slip in scale, sigma, operand orientation or tile index fails
    q, k, v, z = _integer_case(0.0)
    for blk in range(4):
        assert np.abs(k[0, blk * 128:(blk + 1) * 128]).max(axis=(0, 2)).min() == 127
    w = Workload(name="int", batch=1, heads_q=4, heads_kv=2, head_dim=128, text_tokens=1,
                 img_rows=1, img_cols=511, dtype="f16", seed=0, mode="tilemix",
                 pattern="one", smooth_k=False, softmax_scale=0.01)
    o = attn_ref.Oracle(q, k, v, w)
    assert o.route.sum() == 9  # blocks 1..3 are image blocks
    assert (o.sq == 1).all() and (o.sk == 1).all()
    assert (o.k8[0].astype(np.float64) == np.transpose(z[0].reshape(4, 128, 2, 128), (2, 0, 1, 3))).all()
    dense = attn_ref.attention(q, k, v, w.with_(mode="dense"))
    assert np.abs(o.forward() - dense).max() < 1e-12


def test_int8_route_smooth_k_exact_on_integer_tiles():
    q, k, v, z = _integer_case(0.5)
    w = Workload(name="int", batch=1, heads_q=4, heads_kv=2, head_dim=128, text_tokens=1,
                 img_rows=1, img_cols=511, dtype="f16", seed=0, mode="tilemix",
                 pattern="one", smooth_k=True, softmax_scale=0.01)
    o = attn_ref.Oracle(q, k, v, w)
    assert (o.m32 == np.float32(0.5)).all()
    dense = attn_ref.attention(q, k, v, w.with_(mode="dense"))
    assert np.abs(o.forward() - dense).max() < 1e-12
    # without smooth_k the offset is quantised too and the result moves away
    o_off = attn_ref.Oracle(q, k, v, w.with_(smooth_k=False))
    assert np.abs(o_off.forward() - dense).max() > 1e-6


def test_int8_route_error_bound():
    # if every score moves by at most delta, each output moves by at most
    # (exp(2 delta) - 1) * max|V|; delta is bounded from the quantisation steps
    w = _w(heads_q=4, heads_kv=1, head_dim=128, text_tokens=128, img_rows=8, img_cols=48,
           mode="tilemix", pattern="one", smooth_k=True, offset_std=0.5)
    q, k, v = _inputs(w)
    o = attn_ref.Oracle(q, k, v, w)
    tm = o.forward()
    dense = attn_ref.attention(q, k, v, w.with_(mode="dense"))
    ks = quant_ref.smooth(k, o.m32).astype(np.float64)
    n, d = w.tokens, 128
    for h in range(4):
        for blk_q in range(1, n // 128):
            rows = np.arange(blk_q * 128, blk_q * 128 + 128)
            sq = float(o.sq[0, h, blk_q])
            qabs = np.abs(q[0, rows, h])  # [r, d]
            delta = 0.0
            for blk_k in range(1, n // 128):
                sk = float(o.sk[0, 0, blk_k])
                kab = np.abs(ks[0, blk_k * 128:(blk_k + 1) * 128, 0])
                # |q.k - sq q8 . sk k8| <= sum |q| sk/2 + sum |k8 sk| sq/2 + d sq sk / 4
                bound = (qabs.sum(1)[:, None] * sk / 2 + (kab.sum(1)[None, :] + d * sk / 2) * sq / 2)
                delta = max(delta, o.sigma * bound.max())
            err = np.abs(tm[0, rows, h] - dense[0, rows, h]).max()
            assert err <= (math.exp(2 * delta) - 1) * np.abs(v).max()
    assert np.abs(tm - dense).max() > 0  # the INT8 route is really taken


@pytest.mark.parametrize("aligned", [True, False])
def test_window_covering_all_rows_is_dense(aligned):
    # T=77 (text padding), 10x12 grid (tail padding); window >= 2*rows-1 admits all
    w = _w(heads_q=4, heads_kv=2, head_dim=32, text_tokens=77, img_rows=10, img_cols=12,
           mode="scanline", window=19, tile_aligned=aligned)
    q, k, v = _inputs(w)
    sc = attn_ref.attention(q, k, v, w)
    dense = attn_ref.attention(q, k, v, w.with_(mode="dense"))
    assert np.abs(sc - dense).max() < 1e-12


def test_window_one_zero_queries_closed_form():
    # Q = 0 and the exact rule: an image token averages V over text + its own grid row;
    # a text token averages V over every token
    t, rows, cols = 77, 10, 12
    w = _w(heads_q=2, heads_kv=1, head_dim=8, text_tokens=t, img_rows=rows, img_cols=cols,
           mode="scanline", window=1, tile_aligned=False)
    q, k, v = _inputs(w)
    out = attn_ref.attention(np.zeros_like(q), k, v, w)
    for i in range(w.tokens):
        if i < t:
            keys = np.arange(w.tokens)
        else:
            r = (i - t) // cols
            keys = np.concatenate([np.arange(t), t + r * cols + np.arange(cols)])
        want = v[0, keys, 0].mean(axis=0)
        assert np.abs(out[0, i, 0] - want).max() < 1e-12
        assert np.abs(out[0, i, 1] - want).max() < 1e-12


def test_tile_aligned_zero_queries_closed_form():
    # Q = 0, tile_aligned, window 1: image tile 1 holds grid rows 0..15 and image
    # tile 2 rows 16..29, so the image-image tiles (1,2) and (2,1) share no row and
    # stay inactive; each query averages V over the valid keys of its active tiles.
    t, rows, cols = 77, 30, 8
    w = _w(heads_q=2, heads_kv=1, head_dim=8, text_tokens=t, img_rows=rows, img_cols=cols,
           mode="scanline", window=1, tile_aligned=True)
    q, k, v = _inputs(w)
    out = attn_ref.attention(np.zeros_like(q), k, v, w)
    text = np.arange(t)
    img1 = t + np.arange(128)
    img2 = t + np.arange(128, 240)
    for i in range(w.tokens):
        if i < t:
            keys = np.arange(w.tokens)
        elif i < t + 128:
            keys = np.concatenate([text, img1])
        else:
            keys = np.concatenate([text, img2])
        want = v[0, keys, 0].mean(axis=0)
        assert np.abs(out[0, i, :] - want[None]).max() < 1e-12


@pytest.mark.parametrize("mode_kw", [
    dict(mode="dense"),
    dict(mode="tilemix", pattern="band", percentage=0.6, band_blocks=1, smooth_k=True),
    dict(mode="scanline", window=3, tile_aligned=True),
    dict(mode="scanline", window=3, tile_aligned=False),
])
def test_sliced_equals_unsliced(mode_kw):
    w = _w(heads_q=4, heads_kv=1, head_dim=32, text_tokens=130, img_rows=12, img_cols=40,
           offset_std=0.5, **mode_kw)
    q, k, v = _inputs(w)
    full = attn_ref.attention(q, k, v, w)
    sliced = attn_ref.attention(q, k, v, w.with_(q_chunk=128))
    sliced2 = attn_ref.attention(q, k, v, w.with_(q_chunk=256), row_chunk=100)
    # rows are independent; only BLAS blocking of the row chunks can change the
    # last fp64 bit
    assert np.abs(full - sliced).max() < 1e-14 and np.abs(full - sliced2).max() < 1e-14


def test_scanline_restricts_attention():
    # with a narrow window the output must differ from dense for image rows,
    # and text rows (global) must not
    w = _w(heads_q=2, heads_kv=1, head_dim=32, text_tokens=128, img_rows=16, img_cols=16,
           mode="scanline", window=1, tile_aligned=False)
    q, k, v = _inputs(w)
    sc = attn_ref.attention(q, k, v, w)
    dense = attn_ref.attention(q, k, v, w.with_(mode="dense"))
    assert np.abs(sc[:, :128] - dense[:, :128]).max() < 1e-12
    assert np.abs(sc[:, 128:] - dense[:, 128:]).max() > 1e-3
