"""Pins for the oracle's route map and scanline masks (CPU only).

Each check is fixed by something other than the oracle itself: published
SplitMix64 outputs, closed-form tile and pair counts derived from the grid
geometry, the pages' stated rules (text never quantised, window // 2 rows each
side), and brute-force recomputation on tiny grids.
"""
import math
import os

import numpy as np
import pytest

from oracle import plan_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=")
            out[k.strip()] = int(v)
    return out


def test_splitmix64_published_outputs():
    with open(os.path.join(GOLDEN, "splitmix64.txt")) as f:
        want = [int(l, 16) for l in f if l.strip() and not l.startswith("#")]
    state, got = 0, []
    for _ in want:
        got.append(plan_ref.splitmix64(state))
        state = (state + 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
    assert got == want


def _band_closed_form(n_image_blocks, w):
    # tiles with |a-b| <= w inside an n x n block grid
    n = n_image_blocks
    band = n * (2 * w + 1) - w * (w + 1)
    return band, n * n - band


@pytest.mark.parametrize("tokens,text,pct,w,n_img", [
    (4608, 512, 0.5, 2, 32),     # 1 MP: 512 text + 64x64 image
    (16896, 512, 0.75, 2, 128),  # 4 MP: 512 text + 128x128 image
])
def test_route_counts_closed_form(tokens, text, pct, w, n_img):
    r = plan_ref.route_map(tokens, text, "band", pct, w, seed=0)
    nb = plan_ref.n_blocks(tokens)
    assert r.shape == (nb, nb)
    band, left = _band_closed_form(n_img, w)
    assert int(r.sum()) == math.floor(pct * left)
    n_text = text // 128
    assert not r[:n_text, :].any() and not r[:, :n_text].any()
    a, b = np.nonzero(r)
    assert (np.abs(a - b) > w).all()


def test_route_counts_krea_values():
    # the same closed forms evaluated: 154 band / 870 left / 435 INT8 at 1 MP,
    # 634 / 15750 / 11812 at 4 MP
    assert _band_closed_form(32, 2) == (154, 870)
    assert _band_closed_form(128, 2) == (634, 15750)
    assert int(plan_ref.route_map(4608, 512, "band", 0.5, 2).sum()) == 435
    assert int(plan_ref.route_map(16896, 512, "band", 0.75, 2).sum()) == 11812


@pytest.mark.parametrize("seed", [0, 1, 12345, 2**63 + 7])
@pytest.mark.parametrize("pct", [0.0, 0.1, 0.5, 0.999, 1.0])
def test_route_text_never_int8(seed, pct):
    # text blocks include a partial one (T=200 -> blocks 0, 1 hold text)
    r = plan_ref.route_map(1500, 200, "band", pct, 1, seed)
    assert not r[:2].any() and not r[:, :2].any()
    r1 = plan_ref.route_map(1500, 200, "one", pct, 1, seed)
    assert not r1[:2].any() and not r1[:, :2].any()


def test_route_patterns():
    nb = plan_ref.n_blocks(1500)
    z = plan_ref.route_map(1500, 200, "zero")
    assert not z.any()
    one = plan_ref.route_map(1500, 200, "one", 0.3, 1)
    assert int(one.sum()) == (nb - 2) ** 2
    full = plan_ref.route_map(1500, 200, "band", 1.0, 1)
    band, left = _band_closed_form(nb - 2, 1)
    assert int(full.sum()) == left
    assert int(plan_ref.route_map(1500, 200, "band", 0.0, 1).sum()) == 0
    # the comparison baseline quantizes every tile, text included
    assert int(plan_ref.route_map(1500, 200, "all", 0.0, 5).sum()) == nb * nb


def test_route_pick_is_smallest_keys_brute_force():
    # tiny case: recompute the pick by scanning all tiles by hand
    tokens, text, pct, w, seed = 1100, 130, 0.4, 1, 99
    r = plan_ref.route_map(tokens, text, "band", pct, w, seed)
    nb = plan_ref.n_blocks(tokens)
    cands = []
    for a in range(nb):
        for b in range(nb):
            if a * 128 < text or b * 128 < text or abs(a - b) <= w:
                continue
            cands.append((plan_ref.splitmix64(seed ^ (a << 32 | b)), a, b))
    k = int(pct * len(cands))
    chosen = set((a, b) for _, a, b in sorted(cands)[:k])
    got = set(zip(*map(list, np.nonzero(r))))
    assert got == chosen
    # nested: a larger percentage keeps every tile a smaller one picked
    r2 = plan_ref.route_map(tokens, text, "band", 0.8, w, seed)
    assert (r2 >= r).all()


def test_scanline_window_rows_golden():
    g = _golden_kv("scanline_grid.txt")
    assert g["latent_side"] // 2 == g["grid_rows"]
    lay = plan_ref.ScanLayout(0, g["grid_rows"], g["grid_cols"])
    mid = 30 * g["grid_cols"] + 7  # interior token, row 30
    m = plan_ref.token_rule(lay, g["window"], np.array([mid]), np.arange(lay.image_tokens))[0]
    rows_seen = sorted(set((np.nonzero(m)[0] // g["grid_cols"]).tolist()))
    assert rows_seen == list(range(30 - g["rows_each_side"], 30 + g["rows_each_side"] + 1))
    assert m.sum() == (2 * g["rows_each_side"] + 1) * g["grid_cols"]


def test_scanline_counts_closed_form_1mp():
    # 512 text + 64x64 image; 128-token image block = 2 grid rows
    t, rows, cols, window = 512, 64, 64, 11
    hw = window // 2
    bm = plan_ref.block_mask(t, rows, cols, window, tile_aligned=True)
    nb = bm.shape[0]
    assert nb == 36
    n_text, n_img = 4, 32
    # image blocks a', b' hold rows {2a', 2a'+1}, {2b', 2b'+1}; nearest rows 2|a'-b'|-1 apart
    img_active = sum(1 for a in range(n_img) for b in range(n_img)
                     if max(0, 2 * abs(a - b) - 1) <= hw)
    assert img_active == 212
    assert int((bm != 0).sum()) == n_text * nb + n_img * n_text + img_active == 484
    # admitted pairs, exact rule: text rows see all; image rows see text + rows within hw
    per_row = sum(min(rows - 1, r + hw) - max(0, r - hw) + 1 for r in range(rows))
    exact_pairs = t * (t + rows * cols) + rows * cols * t + cols * cols * per_row
    assert exact_pairs == 7_217_152
    aligned_pairs = t * (t + rows * cols) + rows * cols * t + img_active * 128 * 128
    assert aligned_pairs == 7_929_856
    lay = plan_ref.ScanLayout(t, rows, cols)
    n_exact = n_aligned = 0
    for a in range(nb):
        rws = np.arange(a * 128, (a + 1) * 128)
        n_exact += int(plan_ref.admitted(lay, window, False, rws).sum())
        n_aligned += int(plan_ref.admitted(lay, window, True, rws, bm).sum())
    assert n_exact == exact_pairs and n_aligned == aligned_pairs
    # tile kinds: aligned -> no padding here, so every active tile is full;
    # exact rule -> image tiles at block distance 3 are cut inside (partial)
    assert set(np.unique(bm)) <= {0, 1}
    bm0 = plan_ref.block_mask(t, rows, cols, window, tile_aligned=False)
    assert ((bm0 != 0) == (bm != 0)).all()
    part = np.argwhere(bm0 == 2)
    assert len(part) > 0 and all(abs(a - b) == 3 for a, b in part)


def _brute_block_mask(t, rows, cols, window, aligned):
    # independent recomputation from the page's rule with explicit loops
    tp = -(-t // 128) * 128
    length = -(-(tp + rows * cols) // 128) * 128
    nb = length // 128

    def info(p):
        if p < t:
            return True, True, -1
        if tp <= p < tp + rows * cols:
            return True, False, (p - tp) // cols
        return False, False, -1

    inf = [info(p) for p in range(length)]
    out = np.zeros((nb, nb), np.uint8)
    for a in range(nb):
        for b in range(nb):
            any_m, all_adm = False, True
            for i in range(a * 128, a * 128 + 128):
                vi, ti, ri = inf[i]
                for j in range(b * 128, b * 128 + 128):
                    vj, tj, rj = inf[j]
                    m = vi and vj and (ti or tj or abs(ri - rj) <= window // 2)
                    any_m |= m
                    adm = (vi and vj) if aligned else m
                    all_adm &= adm
            if any_m:
                out[a, b] = 1 if all_adm else 2
    return out


@pytest.mark.parametrize("t,rows,cols,window,aligned", [
    (77, 10, 12, 3, True), (77, 10, 12, 3, False), (5, 7, 9, 1, False), (130, 6, 40, 5, True),
])
def test_block_mask_brute_force(t, rows, cols, window, aligned):
    got = plan_ref.block_mask(t, rows, cols, window, aligned)
    want = _brute_block_mask(t, rows, cols, window, aligned)
    assert (got == want).all()


@pytest.mark.parametrize("bad", [0, 2, 12, 256, 257, -1])
def test_window_validation(bad):
    with pytest.raises(ValueError):
        plan_ref.check_window(bad)


def test_layout_padding():
    lay = plan_ref.ScanLayout(77, 10, 12)
    assert lay.t_pad == 128 and lay.length == 256
    pos = np.arange(lay.length)
    v = lay.valid(pos)
    assert v.sum() == 77 + 120
    phys = lay.physical(pos)
    assert sorted(phys[v].tolist()) == list(range(197))
    assert (phys[~v] == -1).all()


def test_scanline_counts_closed_form_4mp():
    # 512 text + 128x128 image: each 128-token image block is exactly one grid row, so image
    # tiles (a, b) are active iff |a - b| <= window // 2; text rows and text keys are global
    t, rows, cols, window = 512, 128, 128, 11
    hw = window // 2
    bm = plan_ref.block_mask(t, rows, cols, window, tile_aligned=True)
    nb = bm.shape[0]
    assert nb == 132
    per_row = sum(min(rows - 1, r + hw) - max(0, r - hw) + 1 for r in range(rows))
    assert per_row == 1378
    assert int((bm != 0).sum()) == 4 * nb + rows * 4 + per_row == 2418
    # whole rows per tile: the exact rule and tile_aligned admit the same pairs, all tiles full
    assert set(np.unique(bm)) <= {0, 1}
    assert (plan_ref.block_mask(t, rows, cols, window, tile_aligned=False) == bm).all()


@pytest.mark.parametrize("tokens,text,pct,w,seed", [(4608, 512, 0.5, 2, 0), (1500, 200, 0.37, 1, 12345),
                                                    (1100, 130, 0.4, 1, 99)])
def test_sage_pick_same_budget_any_tile_brute_force(tokens, text, pct, w, seed):
    """The 'sage' pattern: exactly as many INT8 tiles as 'band' with the same percentage and
    band width, the k smallest (key, a, b) over every tile, text and band included."""
    band = plan_ref.route_map(tokens, text, "band", pct, w, seed)
    sage = plan_ref.route_map(tokens, text, "sage", pct, w, seed)
    assert int(sage.sum()) == int(band.sum())
    nb = plan_ref.n_blocks(tokens)
    keys = sorted((plan_ref.splitmix64(seed ^ (a << 32 | b)), a, b) for a in range(nb) for b in range(nb))
    chosen = set((a, b) for _, a, b in keys[:int(band.sum())])
    assert set(zip(*map(list, np.nonzero(sage)))) == chosen


def test_sage_pick_reaches_text_and_band_tiles():
    # at the 1 MP Krea shape (4 text blocks of 36) the same-budget pick over all tiles sends
    # text tiles and band tiles to INT8, which the band pattern never does
    sage = plan_ref.route_map(4608, 512, "sage", 0.5, 2, 0)
    text = np.zeros_like(sage, dtype=bool)
    text[:4, :] = True
    text[:, :4] = True
    a, b = np.indices(sage.shape)
    assert int(sage[text].sum()) > 0 and int(sage[np.abs(a - b) <= 2].sum()) > 0
    assert int(sage.sum()) == 435
