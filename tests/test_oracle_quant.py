"""Pins for the oracle's smooth_k mean and per-tile INT8 (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import quant_ref


def _bf16_values(shape, seed, offset=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32) + np.float32(offset)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()


def test_k_mean_equals_exact_mean_correctly_rounded():
    # bf16 values: the fixed-order fp64 sum is exact, so the result must be the
    # exactly rounded mean; math.fsum gives the exact sum independently.
    k = _bf16_values((2, 300, 3, 16), seed=3, offset=0.7)
    m = quant_ref.k_mean(k)
    for b in range(2):
        for h in range(3):
            for c in range(16):
                exact = math.fsum(k[b, :, h, c].tolist()) / 300
                assert m[b, h, c] == np.float32(exact)


def test_k_mean_constant_and_offset():
    k = np.full((1, 257, 2, 8), 1.25)
    assert (quant_ref.k_mean(k) == np.float32(1.25)).all()
    # symmetric data around an offset c: mean is exactly c
    rng = np.random.default_rng(1)
    z = rng.integers(-50, 50, size=(1, 100, 2, 8)).astype(np.float64)
    k2 = np.concatenate([z, -z], axis=1) + 0.5
    assert (quant_ref.k_mean(k2) == np.float32(0.5)).all()


def test_k_mean_block_order_matters_reading():
    # values whose fp64 sum depends on order: the oracle follows the stated
    # order (tokens within each 128-block, then blocks), checked by hand here
    k = np.zeros((1, 256, 1, 1))
    k[0, 0, 0, 0] = 2.0 ** 60
    k[0, 1:128, 0, 0] = 1.0
    k[0, 128, 0, 0] = -(2.0 ** 60)
    k[0, 129:256, 0, 0] = 1.0
    # block 0 partial: each +1 is lost against 2^60 (its ulp is 256) -> 2^60;
    # block 1 partial likewise -> -2^60; blocks summed -> 0.  One running sum
    # over all tokens would give 127 instead (the ones after the cancel survive).
    assert quant_ref.k_mean(k)[0, 0, 0] == np.float32(0.0)


def test_quantize_properties():
    rng = np.random.default_rng(5)
    for scale in [1e-3, 1.0, 37.0, 1e3]:
        x = (rng.standard_normal((1, 300, 2, 128)) * scale).astype(np.float32)
        codes, s, inv = quant_ref.quantize_tiles(x)
        assert codes.shape == (1, 2, 3, 128, 128)
        for blk in range(3):
            n = min(300, blk * 128 + 128) - blk * 128
            for h in range(2):
                tile = x[0, blk * 128: blk * 128 + n, h]
                q = codes[0, h, blk, :n].astype(np.float64)
                a = np.abs(tile).max()
                assert s[0, h, blk] == np.float32(a / np.float32(127))
                assert np.abs(q).max() == 127
                # the absmax element maps to +-127 with its sign
                idx = np.unravel_index(np.argmax(np.abs(tile)), tile.shape)
                assert q[idx] == np.sign(tile[idx]) * 127
                err = np.abs(tile.astype(np.float64) - q * np.float64(s[0, h, blk]))
                assert err.max() <= 0.50001 * s[0, h, blk]
                assert not codes[0, h, blk, n:].any()


def test_quantize_round_half_even_and_zero_tile():
    x = np.zeros((1, 128, 2, 128), dtype=np.float32)
    x[0, 0, 0, 0] = 127.0  # absmax 127 -> inv = scale = 1 exactly
    x[0, 1, 0, :6] = [0.5, 1.5, 2.5, -0.5, -2.5, 126.5]
    codes, s, inv = quant_ref.quantize_tiles(x)
    assert s[0, 0, 0] == 1.0 and inv[0, 0, 0] == 1.0
    assert codes[0, 0, 0, 1, :6].tolist() == [0, 2, 2, 0, -2, 126]
    # head 1 is all zero: codes 0 and scale 0
    assert s[0, 1, 0] == 0 and not codes[0, 1].any()


def test_smooth_is_float32_subtract():
    k = _bf16_values((1, 10, 1, 4), seed=2, offset=3.0)
    m = quant_ref.k_mean(k)
    ks = quant_ref.smooth(k, m)
    assert ks.dtype == np.float32
    assert (ks == (k.astype(np.float32) - m[:, None])).all()
    assert (quant_ref.smooth(k, None) == k.astype(np.float32)).all()


def test_int_scores_exact_vs_int64():
    rng = np.random.default_rng(8)
    a = rng.integers(-127, 128, size=(128, 128)).astype(np.int8)
    b = rng.integers(-127, 128, size=(128, 128)).astype(np.int8)
    want = a.astype(np.int64) @ b.astype(np.int64).T
    got = quant_ref.int_scores(a, b)
    assert (got == want).all()
    # worst case magnitude stays exact
    full = np.full((1, 128), 127, np.int8)
    assert quant_ref.int_scores(full, -full)[0, 0] == -128 * 127 * 127
