"""HIP path vs the fp64 CPU oracle, through the C ABI, on an MI355X.

Tolerance for outputs (unit-variance inputs): max |err| <= 2e-2 and mean |err| <= 2e-3
against the fp64 oracle, plus relative RMS <= 1e-2 as an internal gate.  Route maps,
masks, INT8 codes, scales and INT32 accumulators are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import diffusion_transformer_attention_bidirectional_amd as ka
from oracle import attn_ref, block_ref, plan_ref, quant_ref
from synth import WORKLOADS, Workload, make_gate, make_qkv, text_outlier_case, to_f64

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, REL_RMS = 2e-2, 2e-3, 1e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ka.load_library()
    return torch.device("cuda:0")


def _w(**kw):
    base = dict(name="case", batch=1, heads_q=8, heads_kv=2, head_dim=128, text_tokens=40, img_rows=10,
                img_cols=26, dtype="bf16", seed=7, offset_std=0.5, mode="dense")
    base.update(kw)
    return Workload(**base)


def _kw(w):
    return dict(text_tokens=w.text_tokens, img_rows=w.img_rows, img_cols=w.img_cols, mode=w.mode,
                pattern=w.pattern, percentage=w.percentage, band_blocks=w.band_blocks, seed=w.route_seed,
                smooth_k=w.smooth_k, window=w.window, tile_aligned=w.tile_aligned, q_chunk=w.q_chunk,
                softmax_scale=w.softmax_scale)


def _run(w, dev, q=None, k=None, v=None, **over):
    """One call on the GPU; the output starts as NaN, so a row the kernel fails to write shows."""
    if q is None:
        q, k, v = make_qkv(w)
    kw = _kw(w)
    kw.update(over)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dev)
    ka.attention(q.to(dev), k.to(dev), v.to(dev), out=out, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), (q, k, v)


def _assert_close(got, ref, what=""):
    err = np.abs(got - ref)
    rel = np.sqrt(np.mean((got - ref) ** 2) / max(np.mean(ref ** 2), 1e-30))
    assert np.isfinite(got).all(), what
    assert err.max() <= MAX_ABS, f"{what}: max abs {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean abs {err.mean():.3e}"
    assert rel <= REL_RMS, f"{what}: rel rms {rel:.3e}"
    return err.max(), err.mean(), rel


# ----------------------------------------------------------------------------- small, full oracle
SMALL = [
    ("tiny_f16", WORKLOADS["tiny"]),
    ("dense_bf16_ragged", _w()),
    ("dense_f16_ragged", _w(dtype="f16")),
    ("dense_b2_g8", _w(batch=2, heads_q=8, heads_kv=1, text_tokens=64, img_rows=9, img_cols=21)),
    ("tilemix_band", _w(mode="tilemix", pattern="band", percentage=0.6, band_blocks=1, smooth_k=True,
                        text_tokens=130, img_rows=12, img_cols=40)),
    ("tilemix_band_f16", _w(dtype="f16", mode="tilemix", pattern="band", percentage=0.5, band_blocks=0,
                            smooth_k=True, text_tokens=130, img_rows=12, img_cols=40)),
    ("tilemix_one_nosmooth", _w(mode="tilemix", pattern="one", smooth_k=False, text_tokens=100, img_rows=8,
                                img_cols=50)),
    ("tilemix_zero_smooth", _w(mode="tilemix", pattern="zero", smooth_k=True)),
    ("scan_aligned", _w(mode="scanline", window=3, tile_aligned=True, text_tokens=77)),
    ("scan_exact", _w(mode="scanline", window=3, tile_aligned=False, text_tokens=77)),
    ("scan_w1_exact", _w(mode="scanline", window=1, tile_aligned=False, text_tokens=130, img_rows=12,
                         img_cols=40)),
    ("scan_textpad_tail", _w(mode="scanline", window=5, tile_aligned=True, text_tokens=200, img_rows=7,
                             img_cols=33)),
    ("tilemix_b2_g8", _w(batch=2, heads_q=8, heads_kv=1, mode="tilemix", pattern="band", percentage=0.7,
                         band_blocks=1, smooth_k=True, text_tokens=90, img_rows=10, img_cols=38)),
    ("tilemix_band_all", _w(mode="tilemix", pattern="band", percentage=1.0, band_blocks=0, smooth_k=True,
                            text_tokens=40, img_rows=16, img_cols=32)),
    ("scan_f16_b2", _w(dtype="f16", batch=2, mode="scanline", window=5, tile_aligned=False, text_tokens=64,
                       img_rows=9, img_cols=30)),
    ("dense_scale", _w(softmax_scale=0.05, offset_std=0.0)),
    ("tilemix_all", _w(mode="tilemix", pattern="all", smooth_k=True, text_tokens=130, img_rows=12, img_cols=40)),
    ("tilemix_sage", _w(mode="tilemix", pattern="sage", percentage=0.6, band_blocks=1, smooth_k=True,
                        text_tokens=130, img_rows=16, img_cols=40)),
]


@pytest.mark.parametrize("name,w", SMALL, ids=[n for n, _ in SMALL])
def test_small_vs_oracle(dev, name, w):
    got, (q, k, v) = _run(w, dev)
    ref = attn_ref.attention(to_f64(q), to_f64(k), to_f64(v), w)
    mx, mn, rel = _assert_close(got, ref, name)
    print(f"{name}: max {mx:.2e} mean {mn:.2e} rel {rel:.2e}")


def _random_cases(count=30, seed=20261203):
    """Seeded random shapes and mode arguments: dtype, batch, GQA ratio, text length, image
    grid (ragged in both directions), mode, TileMix pattern / percentage / band / smooth_k,
    scanline window / tile alignment, q_chunk."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        hq, hkv = [(4, 1), (8, 2), (8, 1), (12, 3), (16, 2)][rng.integers(5)]
        mode = ["dense", "tilemix", "scanline"][i % 3]
        rows, cols = int(rng.integers(1, 25)), int(rng.integers(1, 65))
        kw = dict(name=f"rand{i}", batch=int(rng.integers(1, 3)), heads_q=hq, heads_kv=hkv, head_dim=128,
                  text_tokens=int(rng.integers(0, 401)), img_rows=rows, img_cols=cols,
                  dtype=["bf16", "f16"][rng.integers(2)], seed=1000 + i, offset_std=0.5, mode=mode,
                  q_chunk=[0, 128, 256][rng.integers(3)])
        if mode == "tilemix":
            kw.update(pattern=["band", "band", "one", "all", "sage", "zero"][rng.integers(6)],
                      percentage=float(rng.uniform(0, 1)), band_blocks=int(rng.integers(0, 3)),
                      smooth_k=bool(rng.integers(2)), route_seed=int(rng.integers(0, 1 << 31)))
        elif mode == "scanline":
            kw.update(window=int(2 * rng.integers(0, 8) + 1), tile_aligned=bool(rng.integers(2)))
        cases.append(Workload(**kw))
    return cases


@pytest.mark.parametrize("w", _random_cases(), ids=lambda w: w.name)
def test_random_shapes_vs_oracle(dev, w):
    """Every element of a seeded random configuration against the oracle."""
    got, (q, k, v) = _run(w, dev)
    ref = attn_ref.attention(to_f64(q), to_f64(k), to_f64(v), w)
    mx, mn, rel = _assert_close(got, ref, w.name)
    print(f"{w.name} {w.mode} {w.dtype} B={w.batch} H={w.heads_q}/{w.heads_kv} N={w.text_tokens}+{w.img_rows}x"
          f"{w.img_cols} chunk={w.q_chunk}: max {mx:.2e} mean {mn:.2e} rel {rel:.2e}", flush=True)


@pytest.mark.parametrize("w", [
    _w(),
    _w(mode="tilemix", pattern="band", percentage=0.6, band_blocks=1, smooth_k=True, text_tokens=130,
       img_rows=12, img_cols=40),
    _w(mode="scanline", window=3, tile_aligned=False, text_tokens=77),
    # 32 query tiles x 12 head groups = 384 items: on 256 CUs the last 128 (ranks 256..383,
    # a partial row of query tiles) split in two, across slice boundaries
    _w(heads_q=48, heads_kv=12, text_tokens=100, img_rows=30, img_cols=64),
    _w(heads_q=48, heads_kv=12, mode="tilemix", pattern="band", percentage=0.5, band_blocks=1, smooth_k=True,
       text_tokens=100, img_rows=30, img_cols=64),
], ids=["dense", "tilemix", "scanline", "dense_split_tail", "tilemix_split_tail"])
def test_slices_match_unsliced(dev, w):
    """Rows are independent and see the full K/V in every slice ("LayerStream: Krea2
    Chunking", "Be clear about exactness"): slicing changes no bit.  Which work items split
    their key range depends only on the item's global position, so each row is computed the
    same way in every slicing."""
    full, qkv = _run(w, dev)
    for chunk in (128, 256, 512):
        sliced, _ = _run(w, dev, *qkv, q_chunk=chunk)
        assert (sliced == full).all(), f"q_chunk {chunk}"


GATED = [
    ("dense", _w()),
    ("tilemix", _w(mode="tilemix", pattern="band", percentage=0.6, band_blocks=1, smooth_k=True, text_tokens=130,
                   img_rows=12, img_cols=40)),
    ("scanline", _w(mode="scanline", window=3, tile_aligned=False, text_tokens=77)),
    ("dense_f16_sliced", _w(dtype="f16", q_chunk=128)),
]


@pytest.mark.parametrize("name,w", GATED, ids=[n for n, _ in GATED])
def test_gated_vs_oracle(dev, name, w):
    """attn_forward_gated: attention * sigmoid(gate), the gate of the block's pass two."""
    q, k, v = make_qkv(w)
    gate = make_gate(q.shape, w.dtype, seed=99)
    got, _ = _run(w, dev, q, k, v, gate=gate.to(dev))
    ref = attn_ref.attention(to_f64(q), to_f64(k), to_f64(v), w) * block_ref.sigmoid(to_f64(gate))
    mx, mn, rel = _assert_close(got, ref, name)
    print(f"gated {name}: max {mx:.2e} mean {mn:.2e} rel {rel:.2e}")


def test_gate_zero_halves_exactly(dev):
    """sigmoid(0) is 1/2 in the kernel too, and halving commutes with the rounding."""
    w = _w()
    plain, qkv = _run(w, dev)
    gate = torch.zeros(qkv[0].shape, dtype=qkv[0].dtype)
    gated, _ = _run(w, dev, *qkv, gate=gate.to(dev))
    assert (gated == 0.5 * plain).all()


def test_zero_pattern_bit_identical_to_dense(dev):
    w = _w(offset_std=0.5)
    dense, qkv = _run(w, dev)
    for smooth in (False, True):
        z, _ = _run(w, dev, *qkv, mode="tilemix", pattern="zero", smooth_k=smooth)
        assert (z == dense).all()


def test_deterministic(dev):
    w = _w(mode="tilemix", pattern="band", percentage=0.5, band_blocks=1, smooth_k=True, text_tokens=130,
           img_rows=12, img_cols=40)
    a, qkv = _run(w, dev)
    b, _ = _run(w, dev, *qkv)
    assert (a == b).all()


@pytest.mark.parametrize("t,rows,cols", [(1, 0, 0), (5, 0, 0), (0, 1, 1), (129, 0, 0), (0, 3, 43), (7, 11, 13)])
def test_edge_sizes_dense(dev, t, rows, cols):
    w = _w(heads_q=4, heads_kv=1, text_tokens=t, img_rows=rows, img_cols=cols)
    got, (q, k, v) = _run(w, dev)
    ref = attn_ref.attention(to_f64(q), to_f64(k), to_f64(v), w)
    _assert_close(got, ref, f"N={w.tokens}")


def test_edge_scanline_pure_image_and_tiny_grid(dev):
    for w in (_w(mode="scanline", window=1, tile_aligned=False, text_tokens=0, img_rows=9, img_cols=30),
              _w(mode="scanline", window=255, tile_aligned=True, text_tokens=3, img_rows=2, img_cols=2)):
        got, (q, k, v) = _run(w, dev)
        ref = attn_ref.attention(to_f64(q), to_f64(k), to_f64(v), w)
        _assert_close(got, ref, f"scan {w.text_tokens}+{w.img_rows}x{w.img_cols}")


def test_strided_bhnd_layout(dev):
    # [B, H, N, d] storage viewed as [B, N, H, d]: strides are passed through the ABI
    w = _w(batch=2)
    q, k, v = make_qkv(w)
    qs = q.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    ks = k.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    vs = v.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    out = torch.empty(q.shape[0], q.shape[2], q.shape[1], 128, dtype=q.dtype, device=dev).permute(0, 2, 1, 3)
    ka.attention(qs, ks, vs, out=out, **_kw(w))
    torch.cuda.synchronize()
    ref = attn_ref.attention(to_f64(q), to_f64(k), to_f64(v), w)
    _assert_close(out.float().cpu().numpy().astype(np.float64), ref, "strided")


# ----------------------------------------------------------------------------- bit-exact pieces
def _quant_check(w, dev):
    q, k, v = make_qkv(w)
    args = ka.args_for(q, k, **{kk: vv for kk, vv in _kw(w).items()})
    res = ka.quantize(q.to(dev), k.to(dev), args)
    torch.cuda.synchronize()
    qf, kf = to_f64(q), to_f64(k)
    m32 = quant_ref.k_mean(kf) if w.smooth_k else np.zeros((w.batch, w.heads_kv, 128), np.float32)
    k8, sk, _ = quant_ref.quantize_tiles(quant_ref.smooth(kf, m32 if w.smooth_k else None))
    q8, sq, _ = quant_ref.quantize_tiles(qf.astype(np.float32))
    if w.smooth_k:
        assert (res["k_mean"].cpu().numpy().view(np.uint32) == m32.view(np.uint32)).all()
    assert (res["k_scale"].cpu().numpy().view(np.uint32) == sk.view(np.uint32)).all()
    assert (res["q_scale"].cpu().numpy().view(np.uint32) == sq.view(np.uint32)).all()
    assert (res["k_codes"].cpu().numpy() == k8).all()
    assert (res["q_codes"].cpu().numpy() == q8).all()
    return q, k, args, q8, k8


def test_quantiser_bit_exact_small(dev):
    _quant_check(_w(mode="tilemix", smooth_k=True, text_tokens=130, img_rows=12, img_cols=40), dev)
    _quant_check(_w(mode="tilemix", smooth_k=False, dtype="f16", text_tokens=10, img_rows=3, img_cols=50), dev)


def test_quantiser_bit_exact_long(dev):
    """More than 64 blocks per head (here 71): the smooth_k mean comes from its own kernel
    instead of the quantiser's workgroups; both must give the oracle's bits."""
    w = _w(mode="tilemix", smooth_k=True, batch=2, text_tokens=77, img_rows=90, img_cols=100)
    assert (w.tokens + 127) // 128 > 64
    _quant_check(w, dev)


def test_int8_scores_bit_exact(dev):
    w = _w(mode="tilemix", smooth_k=True, text_tokens=130, img_rows=12, img_cols=40)
    q, k, args, q8, k8 = _quant_check(w, dev)
    nb = q8.shape[2]
    tiles = [(0, h, a, b) for h in (0, 3, 7) for a in range(nb) for b in (0, nb - 1, 2)]
    got = ka.int8_scores(q.to(dev), k.to(dev), args, tiles).cpu().numpy()
    for i, (b, h, a, kb) in enumerate(tiles):
        want = quant_ref.int_scores(q8[b, h, a], k8[b, h // 4, kb])
        assert (got[i] == want).all(), (b, h, a, kb)


@pytest.mark.parametrize("t,rows,cols,window,aligned", [
    (512, 64, 64, 11, True), (512, 64, 64, 11, False), (77, 10, 26, 3, True), (77, 10, 26, 3, False),
    (0, 9, 30, 1, False), (200, 7, 33, 5, True)])
def test_mask_row_counts_bit_exact(dev, t, rows, cols, window, aligned):
    args = ka.make_args(text_tokens=t, img_rows=rows, img_cols=cols, mode="scanline", window=window,
                        tile_aligned=aligned)
    got = ka.mask_row_counts(args, device=dev).cpu().numpy()
    lay = plan_ref.ScanLayout(t, rows, cols)
    bm = plan_ref.block_mask(t, rows, cols, window, aligned)
    want = np.zeros(lay.length, np.int64)
    for a in range(lay.length // 128):
        r = np.arange(a * 128, a * 128 + 128)
        want[r] = plan_ref.admitted(lay, window, aligned, r, bm).sum(axis=1)
    assert (got == want).all()


def test_mask_row_counts_dense_and_tilemix(dev):
    for mode in ("dense", "tilemix"):
        args = ka.make_args(text_tokens=40, img_rows=10, img_cols=26, mode=mode)
        got = ka.mask_row_counts(args, device=dev).cpu().numpy()
        assert (got == 300).all()


# ----------------------------------------------------------------------------- full Krea shapes
def _sample_rows(n, t, rng, count=48):
    rows = set([0, t - 1, t, t + 1, n - 1, n // 2, 127, 128]) | set(rng.integers(0, n, count).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n))


@pytest.mark.parametrize("name,dtype", [("1mp_dense", "bf16"), ("1mp_band", "bf16"), ("1mp_scanline", "bf16"),
                                        ("1mp_scanline_exact", "bf16"), ("1mp_dense", "f16"), ("1mp_band", "f16")],
                         ids=["1mp_dense", "1mp_band", "1mp_scanline", "1mp_scanline_exact", "1mp_dense_f16",
                              "1mp_band_f16"])
def test_krea_1mp_full(dev, name, dtype):
    """The 1 MP Krea shape against the oracle on every element (all 48 heads, all 4608 rows);
    the fp16 cases run the fp16 instantiations of the kernels on the same seeded values
    rounded to fp16."""
    w = WORKLOADS[name].with_(dtype=dtype)
    got, (q, k, v) = _run(w, dev)
    print(f"{name} {dtype}: GPU done, oracle ...", flush=True)
    ref = attn_ref.Oracle(to_f64(q), to_f64(k), to_f64(v), w).forward()
    mx, mn, rel = _assert_close(got, ref, f"{name} {dtype}")
    print(f"{name} {dtype}: max {mx:.2e} mean {mn:.2e} rel {rel:.2e}", flush=True)


@pytest.mark.parametrize("name", ["4mp_dense", "4mp_band", "4mp_scanline"])
def test_krea_4mp_one_head_per_group(dev, name):
    """The 4 MP Krea shape (N = 16896; TileMix band 75 % with 4096-token query slices;
    scanline with one 128-token tile per grid row, window 11) against the oracle on every row
    of one query head of each of the 12 KV groups, so every query tile of every head group,
    the split tail's items among them, is compared element by element."""
    w = WORKLOADS[name]
    got, (q, k, v) = _run(w, dev)
    ora = attn_ref.Oracle(to_f64(q), to_f64(k), to_f64(v), w)
    assert np.isfinite(got).all()
    for g in range(12):
        h = 4 * g + g % 4
        ref = np.concatenate([ora.rows(0, h, np.arange(r0, min(w.tokens, r0 + 2048)))
                              for r0 in range(0, w.tokens, 2048)])
        mx, mn, rel = _assert_close(got[0, :, h], ref, f"{name} head {h}")
        print(f"{name} head {h}: max {mx:.2e} mean {mn:.2e} rel {rel:.2e}", flush=True)


def test_krea_4mp_scanline_sampled(dev):
    """4 MP scanline (one 128-token tile per grid row, window 11) on sampled rows of four heads."""
    w = WORKLOADS["4mp_scanline"]
    got, (q, k, v) = _run(w, dev)
    assert np.isfinite(got).all()
    ora = attn_ref.Oracle(to_f64(q), to_f64(k), to_f64(v), w)
    rows = _sample_rows(w.tokens, w.text_tokens, np.random.default_rng(3))
    for h in (0, 5, 22, 47):
        _assert_close(got[0, rows, h], ora.rows(0, h, rows), f"4mp scanline head {h}")


@pytest.mark.parametrize("dtype,mode", [("f16", "dense"), ("f16", "tilemix"), ("bf16", "dense"), ("bf16", "tilemix")])
def test_aligned_large_key_in_late_block(dev, dtype, mode):
    """A key in a later block aligned with a query at 1.5x the usual key norm: its score sits
    about 20 log2 units above the running maximum that the first blocks set, while the bound
    that lets a step skip the row maximum (scale |q| max |k|) stays within reach.  The skip
    must not admit probabilities beyond what the P operand holds (fp16: 65504); the result
    matches the oracle.  TileMix puts the keys on FP16 tiles (text rows, the band) and INT8
    tiles (percentage 1)."""
    w = _w(dtype=dtype, mode=mode, pattern="band", percentage=1.0, band_blocks=0, smooth_k=True, text_tokens=130,
           img_rows=12, img_cols=40)  # N = 610: blocks 0, 1 hold text; block 4 ragged
    q, k, v = make_qkv(w)
    qf, kf = q.float(), k.float()
    # (query, key): image rows of block 2 against keys of blocks 2 (band, FP16) and 3 (INT8),
    # text rows against keys of blocks 2 and 3 (FP16: text rows never go INT8)
    pairs = [(300, 296), (301, 401), (20, 484), (140, 261), (370, 450)]
    for g in range(w.heads_kv):
        h = 4 * g + g % 4
        for i, j in pairs:
            qi = qf[0, i, h]
            kf[0, j, g] = qi / qi.norm() * 17.0
    k = kf.to(k.dtype)
    got, _ = _run(w, dev, q, k, v)
    ref = attn_ref.attention(to_f64(q), to_f64(k), to_f64(v), w)
    mx, mn, rel = _assert_close(got, ref, f"{dtype} {mode} aligned key")
    print(f"{dtype} {mode}: max {mx:.2e} mean {mn:.2e} rel {rel:.2e}")


# ----------------------------------------------------------------------------- the device plan
PLAN_CASES = [
    ("tilemix", dict(text_tokens=512, img_rows=64, img_cols=64, pattern="band", percentage=0.5, band_blocks=2)),
    ("tilemix", dict(text_tokens=512, img_rows=128, img_cols=128, pattern="band", percentage=0.75, band_blocks=2)),
    ("tilemix", dict(text_tokens=130, img_rows=12, img_cols=40, pattern="band", percentage=0.6, band_blocks=1,
                     seed=77)),
    ("tilemix", dict(text_tokens=100, img_rows=8, img_cols=50, pattern="one")),
    ("tilemix", dict(text_tokens=130, img_rows=12, img_cols=40, pattern="all")),
    ("tilemix", dict(text_tokens=512, img_rows=64, img_cols=64, pattern="sage", percentage=0.5, band_blocks=2)),
    ("tilemix", dict(text_tokens=0, img_rows=300, img_cols=100, pattern="band", percentage=0.3, band_blocks=0,
                     seed=5)),
    ("scanline", dict(text_tokens=512, img_rows=64, img_cols=64, window=11, tile_aligned=True)),
    ("scanline", dict(text_tokens=512, img_rows=64, img_cols=64, window=11, tile_aligned=False)),
    ("scanline", dict(text_tokens=512, img_rows=128, img_cols=128, window=11, tile_aligned=True)),
    ("scanline", dict(text_tokens=77, img_rows=10, img_cols=26, window=3, tile_aligned=False)),
    ("scanline", dict(text_tokens=200, img_rows=7, img_cols=33, window=5, tile_aligned=True)),
    ("scanline", dict(text_tokens=0, img_rows=9, img_cols=30, window=1, tile_aligned=False)),
    ("scanline", dict(text_tokens=3, img_rows=40, img_cols=300, window=255, tile_aligned=False)),
]


@pytest.mark.parametrize("mode,kw", PLAN_CASES, ids=[f"{m}{i}" for i, (m, _) in enumerate(PLAN_CASES)])
def test_device_plan_matches_oracle(dev, mode, kw):
    """The plan attn_forward builds on the device, in its workspace, each call: the route map
    or block mask equals the oracle's bit for bit (and the host view's), and each query
    block's tile list is the order the kernel visits: TileMix FP16 full tiles, INT8 full tiles,
    ragged block; scanline full tiles, then partial ones."""
    args = ka.make_args(mode=mode, **kw)
    res = {k2: t.cpu().numpy() for k2, t in ka.device_plan(args, device=dev).items()}
    t, rows, cols = kw["text_tokens"], kw["img_rows"], kw["img_cols"]
    n = t + rows * cols
    if mode == "tilemix":
        want = plan_ref.route_map(n, t, kw["pattern"], kw.get("percentage", 0.5), kw.get("band_blocks", 2),
                                  kw.get("seed", 0))
        assert (ka.route_map(args) == want).all()
    else:
        want = plan_ref.block_mask(t, rows, cols, kw["window"], kw["tile_aligned"])
        assert (ka.block_mask(args) == want).all()
    assert (res["map"] == want).all()
    nb = want.shape[0]
    for a in range(nb):
        if mode == "tilemix":
            nfull = nb - 1 if n % 128 else nb
            row = [b for b in range(nfull) if want[a, b] == 0] + [b for b in range(nfull) if want[a, b] == 1]
            row += [nb - 1] if nfull < nb else []
            nf = sum(1 for b in range(nfull) if want[a, b] == 0)
        else:
            row = [b for b in range(nb) if want[a, b] == 1] + [b | (1 << 16) for b in range(nb) if want[a, b] == 2]
            nf = int((want[a] == 1).sum())
        assert res["row_count"][a] == len(row) and res["full_count"][a] == nf, a
        assert res["lists"][a, :len(row)].tolist() == row, a


def test_krea_1mp_batch2_band_full(dev):
    """Two samples at the 1 MP shape in TileMix band mode: batch strides, the per-sample
    smooth_k mean and K codes, every element of both samples against the oracle."""
    w = WORKLOADS["1mp_band"].with_(batch=2)
    got, (q, k, v) = _run(w, dev)
    print("1mp band batch 2: GPU done, oracle ...", flush=True)
    ref = attn_ref.Oracle(to_f64(q), to_f64(k), to_f64(v), w).forward()
    for b in range(2):
        mx, mn, rel = _assert_close(got[b], ref[b], f"batch 2 sample {b}")
        print(f"1mp band batch 2 sample {b}: max {mx:.2e} mean {mn:.2e} rel {rel:.2e}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_krea_1mp_quantiser_bit_exact(dev, dtype):
    _quant_check(WORKLOADS["1mp_band"].with_(dtype=dtype), dev)


def test_krea_1mp_scanline_counts(dev):
    w = WORKLOADS["1mp_scanline"]
    args = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, mode="scanline", window=11, tile_aligned=True)
    got = ka.mask_row_counts(args, device=dev).cpu().numpy()
    assert int(got.sum()) == 7_929_856
    args0 = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, mode="scanline", window=11,
                         tile_aligned=False)
    assert int(ka.mask_row_counts(args0, device=dev).cpu().numpy().sum()) == 7_217_152
    del w


def test_kernel_events_hook(dev):
    """The measurement hook brackets only the attention launches and leaves results unchanged."""
    w = _w(mode="tilemix", pattern="band", percentage=0.5, band_blocks=1, smooth_k=True, q_chunk=128)
    ref, (q, k, v) = _run(w, dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    stream = torch.cuda.current_stream(dev)
    outer = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    inner = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in inner:
        e.record(stream)
    torch.cuda.synchronize()
    try:
        ka.set_kernel_events(*inner)
        outer[0].record(stream)
        out = ka.attention(qd, kd, vd, **_kw(w))
        outer[1].record(stream)
    finally:
        ka.set_kernel_events()
    torch.cuda.synchronize()
    assert (out.float().cpu().numpy().astype(np.float64) == ref).all()
    span, whole = inner[0].elapsed_time(inner[1]), outer[0].elapsed_time(outer[1])
    assert 0.0 < span <= whole
    with pytest.raises(ka.KreaAttnError):
        ka.set_kernel_events(inner[0], None)


@pytest.mark.parametrize("mode", ["dense", "tilemix"])
def test_growing_key_norms(dev, mode):
    """Keys whose norms grow block by block (and large queries): the bound that lets a step
    skip the row max fails on later blocks, which must then rescale; results stay exact."""
    w = _w(mode=mode, pattern="band", percentage=0.5, band_blocks=1, smooth_k=True, text_tokens=64, img_rows=20,
           img_cols=32)
    q, k, v = make_qkv(w)
    n = w.tokens
    grow = torch.tensor([1.0 + 0.75 * (t // 128) for t in range(n)], dtype=torch.float32).view(1, n, 1, 1)
    k = (k.float() * grow).to(k.dtype)
    q = (q.float() * 2.0).to(q.dtype)
    got, _ = _run(w, dev, q, k, v)
    ref = attn_ref.Oracle(to_f64(q), to_f64(k), to_f64(v), w).forward()
    _assert_close(got, ref, f"growing norms {mode}")


def test_int8_baseline_on_text_outliers(dev):
    """The kernel against the oracle in the TileMix band pattern, the same-budget pick over
    all tiles ('sage') and the all-INT8 baseline, on inputs with large text tokens and an
    outlier K channel ("What speedup to expect"): each matches the oracle of its own routing,
    and quantizing text tiles costs more error against exact attention."""
    w = _w(heads_q=4, heads_kv=1, mode="tilemix", pattern="band", percentage=0.5, band_blocks=1, smooth_k=True,
           text_tokens=128, img_rows=16, img_cols=32, seed=21)
    q, k, v = text_outlier_case(w)
    qd, kd, vd = to_f64(q), to_f64(k), to_f64(v)
    exact = attn_ref.attention(qd, kd, vd, w.with_(pattern="zero", smooth_k=False))
    rel = {}
    for pattern in ("band", "sage", "all"):
        wp = w.with_(pattern=pattern)
        got, _ = _run(wp, dev, q, k, v)
        _assert_close(got, attn_ref.attention(qd, kd, vd, wp), f"{pattern} vs its oracle")
        rel[pattern] = float(np.sqrt(np.mean((got - exact) ** 2) / np.mean(exact ** 2)))
    print("rel RMS error against exact attention:", rel)
    assert rel["all"] > 10.0 * rel["band"] and rel["sage"] > rel["band"]


# ----------------------------------------------------------------------------- block context
BLOCK = [
    ("dense", _w(heads_q=8, heads_kv=2), 256),
    ("dense_sliced", _w(heads_q=8, heads_kv=2, q_chunk=128), 256),
    ("tilemix_sliced", _w(heads_q=8, heads_kv=2, mode="tilemix", pattern="band", percentage=0.6, band_blocks=0,
                          smooth_k=True, text_tokens=130, img_rows=12, img_cols=40, q_chunk=256), 512),
    ("scanline_sliced", _w(heads_q=4, heads_kv=1, mode="scanline", window=3, tile_aligned=False, text_tokens=77,
                           q_chunk=128), 128),
    ("dense_f16_b2", _w(dtype="f16", batch=2, heads_q=4, heads_kv=1, text_tokens=64, img_rows=9, img_cols=21), 192),
]


def _block_run(w, d_model, dev, y0_zero=True, seed=5):
    from synth import make_block_inputs
    x, wq, wk, wv, wg, wo, y0 = make_block_inputs(w, d_model, seed)
    if y0_zero:
        y0 = torch.zeros_like(y0)
    y = y0.clone().to(dev)
    ka.block_forward(*(t.to(dev) for t in (x, wq, wk, wv, wg, wo)), y, heads_q=w.heads_q, heads_kv=w.heads_kv,
                     **_kw(w))
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), (x, wq, wk, wv, wg, wo, y0)


@pytest.mark.parametrize("name,w,d_model", BLOCK, ids=[n for n, _, _ in BLOCK])
def test_block_vs_oracle(dev, name, w, d_model):
    """attn_block_forward (K/V for every token, then per slice q, gate, gated attention and
    the output projection added into y) against the fp64 block oracle, y0 = 0."""
    got, ins = _block_run(w, d_model, dev)
    ref = block_ref.block_context(*(to_f64(t) for t in ins), w)
    mx, mn, rel = _assert_close(got, ref, name)
    print(f"block {name}: max {mx:.2e} mean {mn:.2e} rel {rel:.2e}")


def test_block_adds_into_y(dev):
    """y is the residual: the call adds the context into it (one rounding of the sum)."""
    w = _w(heads_q=8, heads_kv=2)
    delta, _ = _block_run(w, 256, dev)
    got, ins = _block_run(w, 256, dev, y0_zero=False)
    y0 = to_f64(ins[-1])
    want = y0 + delta
    # The GPU rounds y0 + c once to bf16 (c the fp32 context); delta = bf16(c).  So
    # |got - want| <= u |y0 + c| + u |c| <= u (|y0| + 2 |c|), u = 2^-8 the bf16 unit
    # roundoff (plus the fp32 difference between the two GEMM runs).
    bound = 2.0 ** -8 * (np.abs(y0) + 2.0 * np.abs(delta)) * 1.01 + 1e-6
    ratio = np.abs(got - want) / bound
    i = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (ratio.max(), got[i], want[i], y0[i], delta[i])


def test_block_krea_1mp_full(dev):
    """The Krea 2 block at 1 MP (D = 6144, 48 / 12 heads, 4096-token query slices, the
    chunking node's default) against the oracle on every element of y."""
    w = WORKLOADS["1mp_dense"].with_(q_chunk=4096)
    got, ins = _block_run(w, 6144, dev, seed=21)
    print("block 1mp: GPU done, oracle ...", flush=True)
    ora = block_ref.BlockOracle(*(to_f64(t) for t in ins), w)
    ref = np.concatenate([ora.rows(0, np.arange(r0, min(w.tokens, r0 + 512))) for r0 in range(0, w.tokens, 512)])
    mx, mn, rel = _assert_close(got[0], ref, "block 1mp")
    print(f"block 1mp: max {mx:.2e} mean {mn:.2e} rel {rel:.2e}", flush=True)


def test_block_krea_4mp_sampled(dev):
    """The Krea 2 block at 4 MP (N = 16896, D = 6144, 4096-token query slices: four full
    slices and a 512-row one) against the oracle on the first and last row of every slice
    and 256 seeded rows."""
    w = WORKLOADS["4mp_dense"].with_(q_chunk=4096)
    got, ins = _block_run(w, 6144, dev, seed=23)
    print("block 4mp: GPU done, oracle ...", flush=True)
    ora = block_ref.BlockOracle(*(to_f64(t) for t in ins), w)
    edges = [r for s0 in range(0, w.tokens, 4096) for r in (s0, min(w.tokens, s0 + 4096) - 1)]
    rows = np.unique(np.concatenate([edges, np.random.default_rng(13).integers(0, w.tokens, 256)]))
    mx, mn, rel = _assert_close(got[0, rows], ora.rows(0, rows), "block 4mp")
    print(f"block 4mp sampled ({len(rows)} rows): max {mx:.2e} mean {mn:.2e} rel {rel:.2e}", flush=True)


@pytest.mark.parametrize("kind,per", [("bf16", 2 * 32 * 32 * 16), ("f16", 2 * 32 * 32 * 16), ("i8", 2 * 32 * 32 * 32),
                                      ("bf16_random", 2 * 32 * 32 * 16)])
def test_mfma_probe_runs_and_counts(dev, kind, per):
    """The MFMA throughput probe reports the operations of 4 * iters products per wave of 8
    waves per workgroup, and its products run: the accumulator checksum changes with iters
    and repeats exactly for the same iters."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sums = []
    for iters in (1, 2, 2):
        ops = ka.mfma_probe(kind, 4, iters, sink)
        torch.cuda.synchronize()
        assert ops == per * 4 * iters * 8 * 4
        sums.append(sink.item())
    assert sums[0] != sums[1] and sums[1] == sums[2]
