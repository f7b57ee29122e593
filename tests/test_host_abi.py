"""C-ABI library on the CPU: symbols, host planner vs oracle (bit-exact), validation.

No compute call reaches a GPU here: only host exports, and attn_forward calls that
fail validation before any device work.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import diffusion_transformer_attention_bidirectional_amd as ka
from oracle import plan_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ka.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ka.load_library()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "krea_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(ka.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header(tmp_path):
    # compile a probe against the header and compare every offset with the ctypes mirror
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "krea_attn.h"', "int main(void) {"]
    for struct, cls in (("attn_args", ka.AttnArgs), ("attn_tensor", ka.AttnTensor),
                        ("attn_plan_info", ka.AttnPlanInfo), ("attn_block_weights", ka.AttnBlockWeights)):
        lines.append(f'printf("{struct} %zu\\n", sizeof({struct}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{struct}.{f} %zu\\n", offsetof({struct}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    for struct, cls in (("attn_args", ka.AttnArgs), ("attn_tensor", ka.AttnTensor),
                        ("attn_plan_info", ka.AttnPlanInfo), ("attn_block_weights", ka.AttnBlockWeights)):
        assert int(got[struct]) == ctypes.sizeof(cls)
        for f, _ in cls._fields_:
            assert int(got[f"{struct}.{f}"]) == getattr(cls, f).offset, (struct, f)


ROUTE_CASES = [
    (4608, 512, "band", 0.5, 2, 0),
    (16896, 512, "band", 0.75, 2, 0),
    (1500, 200, "band", 0.37, 1, 12345),
    (1500, 200, "one", 0.3, 1, 7),
    (1500, 200, "zero", 0.5, 2, 0),
    (300, 0, "band", 0.9, 0, 2**63 + 5),
    (129, 1, "band", 1.0, 0, 3),
    (5000, 77, "band", 0.2, 3, 99),
    (1500, 200, "all", 0.5, 2, 0),
    (4608, 512, "all", 0.0, 0, 1),
    (4608, 512, "sage", 0.5, 2, 0),
    (16896, 512, "sage", 0.75, 2, 0),
    (1500, 200, "sage", 0.37, 1, 12345),
    (300, 0, "sage", 0.9, 0, 2**63 + 5),
]


@pytest.mark.parametrize("n,t,pattern,pct,w,seed", ROUTE_CASES)
def test_route_map_bit_exact_vs_oracle(lib, n, t, pattern, pct, w, seed):
    args = ka.make_args(text_tokens=t, img_rows=1, img_cols=n - t, mode="tilemix", pattern=pattern,
                        percentage=pct, band_blocks=w, seed=seed)
    got = ka.route_map(args)
    want = plan_ref.route_map(n, t, pattern, pct, w, seed)
    assert got.shape == want.shape and (got == want).all()
    assert ka.plan_info(args)["int8_tiles"] == int(want.sum())


MASK_CASES = [
    (512, 64, 64, 11, True), (512, 64, 64, 11, False), (77, 10, 12, 3, True), (77, 10, 12, 3, False),
    (5, 7, 9, 1, False), (130, 6, 40, 5, True), (0, 20, 20, 1, False), (300, 1, 50, 255, False),
    (64, 8, 8, 1, True), (512, 30, 17, 7, False),
]


@pytest.mark.parametrize("t,rows,cols,window,aligned", MASK_CASES)
def test_block_mask_bit_exact_vs_oracle(lib, t, rows, cols, window, aligned):
    args = ka.make_args(text_tokens=t, img_rows=rows, img_cols=cols, mode="scanline", window=window,
                        tile_aligned=aligned)
    got = ka.block_mask(args)
    want = plan_ref.block_mask(t, rows, cols, window, aligned)
    assert (got == want).all()
    info = ka.plan_info(args)
    assert info["active_tiles"] == int((want != 0).sum())
    assert info["partial_tiles"] == int((want == 2).sum())
    assert info["logical_tokens"] == plan_ref.ScanLayout(t, rows, cols).length


@pytest.mark.slow
def test_block_mask_4mp_vs_oracle(lib):
    args = ka.make_args(text_tokens=512, img_rows=128, img_cols=128, mode="scanline", window=11)
    assert (ka.block_mask(args) == plan_ref.block_mask(512, 128, 128, 11, True)).all()
    info = ka.plan_info(args)
    assert info["active_tiles"] == 2418 and info["partial_tiles"] == 0


ORDER_CASES = [
    # text, rows, cols, window, aligned, q_chunk, batch, heads_q
    (512, 64, 64, 11, 1, 0, 1, 48),     # the 1 MP Scanline call
    (512, 128, 128, 11, 1, 4096, 1, 48),  # 4 MP, five query slices
    (77, 9, 13, 3, 0, 256, 2, 8),        # ragged text, padding tiles, batch 2
    (64, 8, 8, 1, 1, 0, 1, 4),           # fewer items than XCDs * CUs
]


@pytest.mark.parametrize("t,rows,cols,window,aligned,chunk,batch,hq", ORDER_CASES)
def test_scanline_item_order(lib, t, rows, cols, window, aligned, chunk, batch, hq):
    """Each launch runs a permutation of its items; XCD x (workgroups L = x + 8 i) runs its
    contiguous range of items, the query tiles holding text queries first (they visit every
    key tile, the others only their band), each kind in item order.  The text tiles are the
    longest items: checked against the block mask."""
    args = ka.make_args(batch=batch, heads_q=hq, heads_kv=hq // 4, text_tokens=t, img_rows=rows, img_cols=cols,
                        mode="scanline", window=window, tile_aligned=aligned, q_chunk=chunk)
    mask = plan_ref.block_mask(t, rows, cols, window, bool(aligned))
    lay = plan_ref.ScanLayout(t, rows, cols)
    length = lay.length
    step = chunk if chunk > 0 else length
    for si, q0 in enumerate(range(0, length, step)):
        q1 = min(length, q0 + step)
        nq = (q1 - q0 + 63) // 64
        n = nq * (hq // 4) * batch
        order = ka.item_order(args, si)
        assert order.shape == (n,) and sorted(order.tolist()) == list(range(n))

        def is_text(item):
            return q0 + 64 * (item % nq) < t

        def cost(item):
            lo = q0 + 64 * (item % nq)
            hi = min(lo + 64, q1)
            valid = lo < min(hi, t) or max(lo, lay.t_pad) < min(hi, lay.t_pad + rows * cols)
            return int((mask[lo // 128] != 0).sum()) if valid else 0

        costs = [cost(i) for i in range(n)]
        if any(is_text(i) for i in range(n)):
            assert min(costs[i] for i in range(n) if is_text(i)) == max(costs)
        per, rem = divmod(n, 8)
        for x in range(8):
            base = x * (per + 1) if x < rem else rem * (per + 1) + (x - rem) * per
            cnt = per + 1 if x < rem else per
            got = order[x::8].tolist()
            assert len(got) == cnt and sorted(got) == list(range(base, base + cnt))
            keys = [(0 if is_text(i) else 1, i) for i in got]
            assert keys == sorted(keys)
    with pytest.raises(ka.KreaAttnError):
        ka.item_order(args, len(range(0, length, step)))
    dense = ka.make_args(text_tokens=t, img_rows=rows, img_cols=cols, mode="dense")
    assert lib.attn_item_order(ctypes.byref(dense), 0, np.zeros(8, np.int32).ctypes.data, 8) == -1


TAIL_PART_BYTES = 8 * 66 * 64 * 4  # 8 waves x (64 O values, max, sum) x 64 lanes, fp32


def _a256(x):
    return (x + 255) // 256 * 256


def test_workspace_sizes(lib):
    # every mode: V^T tiles (12 KV heads x 36 blocks x 128 x 128 bf16) and the fp32 key-norm
    # bound of each 128-key block
    vt = 12 * 36 * 128 * 128 * 2
    kn = _a256(12 * 36 * 4)
    # dense adds 256 tail counters and room for 256 partial states (864 items x 8 parts > 256)
    dense = ka.workspace_bytes(ka.make_args(text_tokens=512, img_rows=64, img_cols=64))
    assert dense == vt + kn + 256 * 4 + 256 * TAIL_PART_BYTES
    # a single 128-token block never splits: counters only
    one = ka.make_args(text_tokens=100, img_rows=0, img_cols=0, heads_q=4, heads_kv=1)
    assert ka.workspace_bytes(one) == 128 * 128 * 2 + 256 + 1024
    # 2 blocks, 4 items (4 query tiles of 64 x 1 head group): room for items x min(nb, 8) parts
    two = ka.make_args(text_tokens=200, img_rows=0, img_cols=0, heads_q=4, heads_kv=1)
    assert ka.workspace_bytes(two) == 2 * 128 * 128 * 2 + 256 + 1024 + 4 * 2 * TAIL_PART_BYTES
    # scanline: padded logical length 256 (nb = 2), never split; the per-call plan: map
    # [nb, nb] uint8, lists [nb, nb] int32, row and full counts [nb] int32
    scan = ka.make_args(text_tokens=77, img_rows=10, img_cols=12, heads_q=4, heads_kv=1, mode="scanline")
    assert ka.workspace_bytes(scan) == 2 * 128 * 128 * 2 + 256 + 4 * 256
    tm = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, mode="tilemix")
    n = ka.workspace_bytes(tm)
    # plus the plan (36 blocks) and at least the INT8 K codes: 12 KV heads x 36 blocks x 128 x 128
    plan = _a256(36 * 36) + _a256(36 * 36 * 4) + 2 * _a256(36 * 4)
    assert n >= dense + plan + 12 * 36 * 128 * 128


def test_block_workspace_and_validation(lib):
    """attn_block_workspace_bytes: K, V of every token, q / gate / output of one query slice,
    the attention workspace and 32 MiB for the GEMM library; bad model dims are refused."""
    args = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, q_chunk=1024)
    n, hq, hkv = 4608, 48 * 128, 12 * 128
    want = (_a256(n * hkv * 2) * 2 + _a256(1024 * hq * 2) * 3 + _a256(ka.workspace_bytes(args))
            + (32 << 20))
    assert ka.block_workspace_bytes(args, 6144) == want
    out = ctypes.c_size_t()
    assert lib.attn_block_workspace_bytes(ctypes.byref(args), 6150, ctypes.byref(out)) == -1
    assert lib.attn_block_workspace_bytes(ctypes.byref(args), 0, ctypes.byref(out)) == -1
    weights = ka.AttnBlockWeights(None, None, None, None, None, 6144, 0)
    assert lib.attn_block_forward(ctypes.byref(args), ctypes.byref(weights), None, None, None, 0, None) == -1


def _status(fn, *a):
    return fn(*a)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype="f32"), -2),
    (dict(head_dim=64), -3),
    (dict(heads_q=48, heads_kv=7), -3),
    (dict(heads_q=12, heads_kv=6), -3),
    (dict(batch=0), -3),
    (dict(text_tokens=0, img_rows=0, img_cols=0), -3),
    (dict(mode=7), -1),
    (dict(q_chunk=100), -1),
    (dict(q_chunk=-128), -1),
    (dict(mode="tilemix", percentage=1.5), -1),
    (dict(mode="tilemix", percentage=-0.1), -1),
    (dict(mode="tilemix", pattern=9), -1),
    (dict(mode="tilemix", band_blocks=-1), -1),
    (dict(mode="scanline", window=10), -1),
    (dict(mode="scanline", window=257), -1),
    (dict(mode="scanline", window=0), -1),
    (dict(softmax_scale=-1.0), -1),
])
def test_validation_codes(lib, kw, status):
    base = dict(text_tokens=512, img_rows=64, img_cols=64)
    base.update(kw)
    args = ka.make_args(**base)
    n = ctypes.c_size_t(0)
    assert lib.attn_workspace_bytes(ctypes.byref(args), ctypes.byref(n)) == status
    assert lib.attn_last_error()  # a message is set
    info = ka.AttnPlanInfo()
    assert lib.attn_plan_info_get(ctypes.byref(args), ctypes.byref(info)) == status


def _fake(h):
    # aligned, non-null fake device pointers: validation must fail before any use
    return ka.AttnTensor(0x100000, 4608 * h * 128, h * 128, 128)


def test_forward_validation_before_device_work(lib):
    args = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, mode="tilemix")
    q, k = _fake(48), _fake(12)
    # every mode needs a workspace
    st = lib.attn_forward(ctypes.byref(args), ctypes.byref(q), ctypes.byref(k), ctypes.byref(k),
                          ctypes.byref(q), None, 0, None)
    assert st == -4
    # misaligned and null tensors, bad strides
    bad = ka.AttnTensor(0x100004, 4608 * 48 * 128, 48 * 128, 128)
    st = lib.attn_forward(ctypes.byref(args), ctypes.byref(bad), ctypes.byref(k), ctypes.byref(k),
                          ctypes.byref(q), None, 0, None)
    assert st == -1
    null = ka.AttnTensor(0, 0, 0, 0)
    st = lib.attn_forward(ctypes.byref(args), ctypes.byref(null), ctypes.byref(k), ctypes.byref(k),
                          ctypes.byref(q), None, 0, None)
    assert st == -1
    odd = ka.AttnTensor(0x100000, 4608 * 48 * 128, 48 * 128 + 4, 128)
    st = lib.attn_forward(ctypes.byref(args), ctypes.byref(odd), ctypes.byref(k), ctypes.byref(k),
                          ctypes.byref(q), None, 0, None)
    assert st == -1
    st = lib.attn_forward(None, ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(q), None, 0, None)
    assert st == -1
    # fp32 refused before anything else
    a32 = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, dtype="f32")
    st = lib.attn_forward(ctypes.byref(a32), ctypes.byref(q), ctypes.byref(k), ctypes.byref(k),
                          ctypes.byref(q), None, 0, None)
    assert st == -2


def test_route_and_mask_reject_wrong_mode(lib):
    args = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, mode="dense")
    out = np.zeros((36, 36), np.uint8)
    assert lib.attn_route_map(ctypes.byref(args), out.ctypes.data, 36) == -1
    assert lib.attn_block_mask(ctypes.byref(args), out.ctypes.data, 36) == -1
    tm = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, mode="tilemix")
    assert lib.attn_route_map(ctypes.byref(tm), out.ctypes.data, 35) == -1


def test_mfma_probe_validation(lib):
    """The probe rejects bad arguments before any device work (no GPU needed)."""
    ops = ctypes.c_int64(-7)
    sink = ctypes.c_void_p(0x100000)
    assert lib.attn_mfma_probe(4, 1, 1, sink, ctypes.byref(ops), None) == -1
    assert lib.attn_mfma_probe(-1, 1, 1, sink, ctypes.byref(ops), None) == -1
    assert lib.attn_mfma_probe(0, 0, 1, sink, ctypes.byref(ops), None) == -1
    assert lib.attn_mfma_probe(0, 1, 0, sink, ctypes.byref(ops), None) == -1
    assert lib.attn_mfma_probe(0, 1, 1, None, ctypes.byref(ops), None) == -1
    assert lib.attn_mfma_probe(0, 1, 1, sink, None, None) == -1
    assert ops.value == -7


def test_status_strings(lib):
    for code, text in ka.STATUS.items():
        assert lib.attn_status_string(code).decode() == text


def test_python_raises_loudly_without_library(tmp_path):
    # a missing library is an error, never a silent fallback
    saved = ka._lib
    try:
        ka._lib = None
        with pytest.raises(ka.KreaAttnError):
            ka.load_library(str(tmp_path / "nope.so"))
    finally:
        ka._lib = saved


def test_caller_policy_helpers(lib):
    assert ka.should_use(4608)
    assert not ka.should_use(4608, enabled=False)
    assert not ka.should_use(1000, min_tokens=1024) and ka.should_use(1024, min_tokens=1024)
    band = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, mode="tilemix", pattern="band",
                        percentage=0.5, band_blocks=2)
    assert ka.describe(band) == ("krea_attn tilemix: 48 q / 12 kv heads, 4608 tokens, 36x36 tiles, pattern band: "
                                 "435 INT8 (33.6 %), smooth_k on")
    scan = ka.make_args(text_tokens=512, img_rows=64, img_cols=64, mode="scanline", window=11, q_chunk=1024)
    assert ka.describe(scan) == ("krea_attn scanline: 48 q / 12 kv heads, 4608 tokens, 36x36 tiles, window 11 "
                                 "tile-aligned: 484 active (37.3 %), queries in slices of 1024")
    assert ka.describe(ka.make_args(text_tokens=5)).startswith("krea_attn dense: 48 q / 12 kv heads, 5 tokens")


LAUNCH_CASES = [
    # text, rows, cols, batch, heads_q, mode, chunks
    (512, 64, 64, 1, 48, "dense", (0, 4096, 2048, 1024, 128)),    # 1 MP: 864 items, 96 in the last wave
    (512, 128, 128, 1, 48, "tilemix", (0, 4096, 2048)),           # 4 MP: 3168 items
    (77, 9, 13, 2, 8, "dense", (0, 128, 256)),                     # ragged, batch 2
    (40, 10, 26, 1, 8, "tilemix", (0, 128)),
    (512, 64, 64, 1, 48, "scanline", (0, 4096)),
]


def _launch_workgroups(args, lay_len, chunk, cus):
    step = chunk if chunk > 0 else lay_len
    jn = (args.heads_q // 4) * args.batch
    items = {}
    for si, q0 in enumerate(range(0, lay_len, step)):
        nq = (min(lay_len, q0 + step) - q0 + 63) // 64
        for qt, j, part, parts in ka.launch_items(args, si, cus).tolist():
            assert q0 // 64 <= qt < q0 // 64 + nq and 0 <= j < jn
            items.setdefault((qt, j), []).append((part, parts))
    return items


@pytest.mark.parametrize("t,rows,cols,batch,hq,mode,chunks", LAUNCH_CASES)
@pytest.mark.parametrize("cus", [256, 80, 304])
def test_split_rule_independent_of_slicing(lib, t, rows, cols, batch, hq, mode, chunks, cus):
    """Every launch runs each of its (query tile, pair) items once, whole or as parts 0..s-1,
    and which items split (and into how many parts) is the same under every query slicing:
    so each query row is computed the same way whatever q_chunk is.  In the whole call the
    split items are exactly the last wave's (G mod cus) items of highest rank."""
    base = None
    for chunk in chunks:
        args = ka.make_args(batch=batch, heads_q=hq, heads_kv=hq // 4, text_tokens=t, img_rows=rows, img_cols=cols,
                            mode=mode, q_chunk=chunk)
        length = ka.plan_info(args)["logical_tokens"]
        items = _launch_workgroups(args, length, chunk, cus)
        nq_all = (length + 63) // 64
        jn = (hq // 4) * batch
        assert sorted(items) == [(q, j) for q in range(nq_all) for j in range(jn)]
        split_of = {}
        for key, parts in items.items():
            s = parts[0][1]
            assert sorted(parts) == [(p, s) for p in range(s)], (key, parts)
            split_of[key] = s
        if base is None:
            base = split_of
            G = nq_all * jn
            rem = G % cus
            split = {k: v for k, v in split_of.items() if v > 1}
            if split:
                assert mode != "scanline"
                ranks = sorted(q * jn + j for q, j in split)
                assert ranks == list(range(G - rem, G))
        else:
            assert split_of == base, f"q_chunk {chunk} splits differently"
    if mode != "scanline" and (t, rows, cols) == (512, 64, 64) and cus == 256:
        assert max(base.values()) == 2 and sum(v > 1 for v in base.values()) == 96
