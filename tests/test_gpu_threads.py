"""The library from several host threads at once, each on its own stream (default
priority): more distinct shapes than the plan cache holds, so plans are built, shared and
evicted while other threads' kernels run.  Every result must equal the single-threaded
one bit for bit (the kernels are deterministic)."""
import threading

import pytest
import torch

import diffusion_transformer_attention_bidirectional_amd as ka
from synth import Workload, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ka.load_library()
    return torch.device("cuda:0")


def _w(i):
    mode = ("dense", "tilemix", "scanline")[i % 3]
    extra = dict(pattern="band", percentage=0.5, band_blocks=1, smooth_k=True) if mode == "tilemix" else {}
    return Workload(name=f"t{i}", batch=1, heads_q=8, heads_kv=2, head_dim=128, text_tokens=40 + 13 * i,
                    img_rows=6 + i, img_cols=20 + 3 * i, dtype="bf16", seed=100 + i, offset_std=0.5, mode=mode,
                    window=3, **extra)


def _kw(w):
    return dict(text_tokens=w.text_tokens, img_rows=w.img_rows, img_cols=w.img_cols, mode=w.mode,
                pattern=w.pattern, percentage=w.percentage, band_blocks=w.band_blocks, seed=w.route_seed,
                smooth_k=w.smooth_k, window=w.window, tile_aligned=w.tile_aligned, q_chunk=w.q_chunk)


def test_threads_share_the_plan_cache(dev):
    cases = [_w(i) for i in range(10)]  # more shapes than the 8 cached plans
    inputs = [tuple(t.to(dev) for t in make_qkv(w)) for w in cases]
    want = []
    for w, (q, k, v) in zip(cases, inputs):
        want.append(ka.attention(q, k, v, **_kw(w)))
    torch.cuda.synchronize()
    errors = []

    def worker(tid):
        try:
            stream = torch.cuda.Stream(device=dev)
            order = list(range(len(cases)))[tid::1] + list(range(len(cases)))[:tid]
            with torch.cuda.stream(stream):
                for rep in range(3):
                    for j in (order if rep % 2 == 0 else order[::-1]):
                        q, k, v = inputs[j]
                        out = ka.attention(q, k, v, **_kw(cases[j]))
                        stream.synchronize()
                        if not torch.equal(out, want[j]):
                            errors.append(f"thread {tid} case {j} rep {rep}: differs")
        except Exception as e:  # reported below, with the thread that raised it
            errors.append(f"thread {tid}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors[:5]
