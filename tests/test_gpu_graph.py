"""HIP graph capture of the library's calls: a call captured into a graph must give the eager
result on every replay, with the program's own eager work and synchronisations between the
replays.  The attention path launches kernels only -- no allocation, memset, host copy or
synchronisation, not even on the first call of a shape: each call's pre-pass builds the tile
lists in the call's workspace and resets the split tail's counters, so replays start from
the same state, and the host plan cache holds no device memory a replay could read after an
eviction.  The block path picks its GEMM algorithms on its first call of a shape, which
waits for the stream, so it is captured after one eager call."""
import numpy as np
import pytest
import torch

import diffusion_transformer_attention_bidirectional_amd as ka
from synth import WORKLOADS, make_block_inputs, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ka.load_library()
    return torch.device("cuda:0")


def _kw(w):
    return dict(text_tokens=w.text_tokens, img_rows=w.img_rows, img_cols=w.img_cols, mode=w.mode,
                pattern=w.pattern, percentage=w.percentage, band_blocks=w.band_blocks, seed=w.route_seed,
                smooth_k=w.smooth_k, window=w.window, tile_aligned=w.tile_aligned, q_chunk=w.q_chunk)


# the 1 MP shapes: 864 work items on 256 CUs, so the split tail and its counters run
@pytest.mark.parametrize("name,chunk", [("1mp_dense", 0), ("1mp_band", 0), ("1mp_scanline", 0),
                                        ("1mp_band", 2048)], ids=["dense", "band", "scanline", "band_sliced"])
def test_attention_graph_replays_match_eager(dev, name, chunk):
    w = WORKLOADS[name].with_(q_chunk=chunk)
    q, k, v = (t.to(dev) for t in make_qkv(w))
    kw = _kw(w)
    eager = ka.attention(q, k, v, **kw)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    ws = torch.empty(max(ka.workspace_bytes(ka.args_for(q, k, **kw)), 256), dtype=torch.uint8, device=dev)
    ka.attention(q, k, v, out=out, workspace=ws, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ka.attention(q, k, v, out=out, workspace=ws, **kw)
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"{name} replay {rep}"
        # eager work on the same workspace between replays
        ka.attention(q, k, v, out=torch.empty_like(q), workspace=ws, **kw)
        torch.cuda.synchronize()


def test_block_graph_replays_match_eager(dev):
    w = WORKLOADS["1mp_dense"].with_(q_chunk=4096, heads_q=8, heads_kv=2)
    x, wq, wk, wv, wg, wo, y0 = (t.to(dev) for t in make_block_inputs(w, 1024, seed=3))
    kw = dict(text_tokens=w.text_tokens, img_rows=w.img_rows, img_cols=w.img_cols, heads_q=w.heads_q,
              heads_kv=w.heads_kv, q_chunk=w.q_chunk)
    args = ka.make_args(heads_q=w.heads_q, heads_kv=w.heads_kv, text_tokens=w.text_tokens, img_rows=w.img_rows,
                        img_cols=w.img_cols, q_chunk=w.q_chunk)
    ws = torch.empty(ka.block_workspace_bytes(args, 1024), dtype=torch.uint8, device=dev)
    y = y0.clone()
    ka.block_forward(x, wq, wk, wv, wg, wo, y, workspace=ws, **kw)  # plan, GEMM algorithms
    torch.cuda.synchronize()
    eager = y.float().cpu().numpy()
    graph = torch.cuda.CUDAGraph()
    y.copy_(y0)
    with torch.cuda.graph(graph):
        ka.block_forward(x, wq, wk, wv, wg, wo, y, workspace=ws, **kw)
    y0f = y0.float().cpu().numpy()
    for rep in range(3):
        y.copy_(y0)
        graph.replay()
        torch.cuda.synchronize()
        got = y.float().cpu().numpy()
        # the same algorithms on the same data: equal up to one bf16 rounding of the sum
        bound = 2.0 ** -8 * (np.abs(y0f) + 2.0 * np.abs(eager - y0f)) + 1e-6
        assert np.all(np.abs(got - eager) <= bound), f"block replay {rep}"
        ka.block_forward(x, wq, wk, wv, wg, wo, y.clone(), workspace=ws, **kw)
        torch.cuda.synchronize()


def _other_shapes(n):
    """n small calls of distinct shapes (each its own plan) in every mode."""
    from synth import Workload
    out = []
    for i in range(n):
        mode = ("dense", "tilemix", "scanline")[i % 3]
        extra = dict(pattern="band", percentage=0.5, band_blocks=1, smooth_k=True) if mode == "tilemix" else {}
        out.append(Workload(name=f"o{i}", batch=1, heads_q=4, heads_kv=1, head_dim=128, text_tokens=30 + 7 * i,
                            img_rows=5 + i, img_cols=17 + 2 * i, dtype="bf16", seed=300 + i, offset_std=0.5,
                            mode=mode, window=3, **extra))
    return out


@pytest.mark.parametrize("name", ["1mp_band", "1mp_scanline"])
def test_graph_captured_on_first_call_survives_plan_eviction(dev, name):
    """A shape captured into a graph on its very first call, then more than the cache's 8
    other plans built (the captured shape's plan is evicted and rebuilt) between replays:
    every replay equals the eager result."""
    w = WORKLOADS[name].with_(text_tokens=500)  # a shape no other test uses
    w = w.with_(img_rows=63, img_cols=64)
    q, k, v = (t.to(dev) for t in make_qkv(w))
    kw = _kw(w)
    ws = torch.empty(max(ka.workspace_bytes(ka.args_for(q, k, **kw)), 256), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ka.attention(q, k, v, out=out, workspace=ws, **kw)  # the shape's first call
    others = [(o, tuple(t.to(dev) for t in make_qkv(o))) for o in _other_shapes(10)]
    eager = None
    for rep in range(3):
        for o, (qo, ko, vo) in others:  # evicts the captured shape's plan
            ka.attention(qo, ko, vo, **_kw(o))
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        if eager is None:
            eager = ka.attention(q, k, v, **kw)
            torch.cuda.synchronize()
        assert torch.equal(out, eager), f"{name} replay {rep}"
