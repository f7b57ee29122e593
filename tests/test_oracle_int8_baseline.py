"""TileMix routing against the all-INT8 baseline, in the oracle.

"Krea 2 TileMix Attention (FP16/INT8 tiles)", "What speedup to expect": the page compares
its error with a kernel that quantizes the text tiles too, on adversarial random inputs, and
reports a lower error for TileMix.  These tests reproduce the comparison with the oracle's
exact INT8 arithmetic (route map, smooth_k, per-tile symmetric codes) against exact fp64
attention, on inputs whose text tokens are large and carry an outlier K channel.
"""
import numpy as np
import pytest

from oracle import attn_ref
from synth import Workload, text_outlier_case, to_f64


def _w(pattern, **kw):
    base = dict(name="adv", batch=1, heads_q=4, heads_kv=1, head_dim=128, text_tokens=128, img_rows=16,
                img_cols=32, dtype="bf16", seed=21, offset_std=0.5, mode="tilemix", pattern=pattern,
                percentage=0.5, band_blocks=1, smooth_k=True)
    base.update(kw)
    return Workload(**base)


def _errors(pattern, seed=21):
    w = _w(pattern, seed=seed)
    q, k, v = text_outlier_case(w)
    qd, kd, vd = to_f64(q), to_f64(k), to_f64(v)
    exact = attn_ref.attention(qd, kd, vd, w.with_(pattern="zero", smooth_k=False))
    got = attn_ref.attention(qd, kd, vd, w)
    d = got - exact
    return float(np.sqrt(np.mean(d ** 2) / np.mean(exact ** 2))), float(np.abs(d).max())


@pytest.mark.parametrize("seed", [21, 22])
def test_tilemix_band_beats_all_int8_on_text_outliers(seed):
    rel_band, max_band = _errors("band", seed)
    rel_one, max_one = _errors("one", seed)
    rel_all, max_all = _errors("all", seed)
    print(f"seed {seed}: rel RMS band {rel_band:.3e} one {rel_one:.3e} all {rel_all:.3e}; "
          f"max abs band {max_band:.3e} one {max_one:.3e} all {max_all:.3e}")
    # text tiles kept in FP16: routing more image tiles to INT8 ('one') stays close to the
    # band pattern, quantizing the text tiles ('all') costs several times the error
    assert rel_band <= rel_one
    assert rel_all > 2.0 * rel_one
    assert max_all > 2.0 * max_one
