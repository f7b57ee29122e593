"""Benchmark: Krea 2 joint attention on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-detail] [--no-cpu]

One step = one attention call (attn_forward through the C ABI) on the 1 MP Krea 2 shape
(B=1, 48 query / 12 KV heads, head_dim 128, 512 text + 64x64 image tokens, bf16, dense),
inputs resident in HBM (every workload's inputs are drawn and moved to the GPU before any
timing).  W untimed warm-up steps, continued until at least WARMUP_MS of work has run
(the first milliseconds of work after an idle period run up to ~10 % slower, so a count
alone does not reach the steady state), then K timed steps bracketed by
torch.cuda.synchronize(); one JSON line on stdout.

value = effective TFLOP/s = 4 * Hq * N^2 * d / time per call (dense-equivalent flops).
roofline: the attention kernel's algorithmic flops per launch / its mean launch duration
(HIP events on the stream the kernel runs on), against MI355X's dense bf16 MFMA peak; also
against the rates the library's MFMA probe sustains on the same GPU (measured_mfma_peak: on
repeating operands, and for bf16 also on operands that change every product, as random data
does; toggling operand bits draw more power, so the chip holds a lower clock).
cpu_baseline: the fp64 numpy oracle on a bounded sample of the same workload (a few
query heads), timed on this host's cores, scaled to TFLOP/s.
detail: the same timing for the other Krea workloads (1 MP TileMix band, 1 MP scanline with
and without tile alignment, 4 MP TileMix band sliced, 4 MP dense unsliced and sliced, 4 MP scanline), for the
band-vs-dense and 4 MP comparisons, each after its own warm-up; an A/B of band against dense at
equal shape (1 MP, and 4 MP with the same slicing), timed in alternation; and the block's attention context
(attn_block_forward: projections, gated attention in 4096-token query slices, output
projection into the residual) at 1 MP and 4 MP with the Krea 2 width 6144.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_I8_TOPS = 5000.0       # MI355X dense int8 MFMA
HEADLINE = "1mp_dense"
DETAIL = ["1mp_band", "1mp_scanline", "1mp_scanline_exact", "4mp_dense", "4mp_dense_sliced", "4mp_band",
          "4mp_scanline"]


def algorithmic_work(w, info):
    """(bf16 flops, int8 ops, dense-equivalent flops) one call computes."""
    n, hq, d = w.tokens, w.heads_q, w.head_dim
    dense_eq = 4.0 * hq * n * n * d * w.batch
    tile = 2.0 * 128 * 128 * d  # one 128x128 tile of one GEMM, one head
    if w.mode == "dense":
        return dense_eq, 0.0, dense_eq
    if w.mode == "tilemix":
        nb = info["n_blocks"]
        i8 = info["int8_tiles"]
        bf = hq * w.batch * tile * ((nb * nb - i8) + nb * nb)
        return bf, hq * w.batch * tile * i8, dense_eq
    act = info["active_tiles"]
    return 2.0 * hq * w.batch * tile * act, 0.0, dense_eq


def workload_kwargs(w):
    return dict(text_tokens=w.text_tokens, img_rows=w.img_rows, img_cols=w.img_cols, mode=w.mode,
                pattern=w.pattern, percentage=w.percentage, band_blocks=w.band_blocks, seed=w.route_seed,
                smooth_k=w.smooth_k, window=w.window, tile_aligned=w.tile_aligned, q_chunk=w.q_chunk)


def roofline_time_s(bf, i8):
    return bf / (PEAK_BF16_TFLOPS * 1e12) + i8 / (PEAK_I8_TOPS * 1e12)


def roofline_peak_mixed(bf, i8):
    """Peak rate of a bf16 + int8 mix: total operations over the time each part needs at its
    own dense MFMA peak."""
    return (bf + i8) / roofline_time_s(bf, i8) / 1e12


WARMUP_MS = 300.0  # untimed calls per workload last at least this long, whatever --warmup says


_INPUTS = {}


def device_inputs(name, dev):
    """Q, K, V of a workload on the device, drawn once per distinct tensor set (workloads
    that share a seed and shape share the tensors); every set is drawn before any timing."""
    from synth import WORKLOADS, make_qkv

    w = WORKLOADS[name]
    key = (w.seed, w.batch, w.tokens, w.heads_q, w.heads_kv, w.dtype, w.offset_std)
    if key not in _INPUTS:
        _INPUTS[key] = tuple(t.to(dev) for t in make_qkv(w))
    return _INPUTS[key]


def warm_up(call, calls, min_ms):
    """Untimed calls: at least `calls` of them and at least `min_ms` of wall time, so the timed
    calls start on a GPU that has been busy (clocks up, caches and code resident) whatever
    it did before.  Returns (calls made, milliseconds spent)."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            call()
        n += 8
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        if n >= calls and ms >= min_ms:
            return n, ms


def time_workload(name, steps, warmup, dev):
    """ms per call (events around K back-to-back calls) and the attention launches alone
    (the library's kernel-event hook), both after the same warm-up."""
    import torch

    import diffusion_transformer_attention_bidirectional_amd as ka
    from synth import WORKLOADS

    w = WORKLOADS[name]
    q, k, v = device_inputs(name, dev)
    kw = workload_kwargs(w)
    args = ka.args_for(q, k, **kw)
    info = ka.plan_info(args)
    out = torch.empty_like(q)
    nbytes = ka.workspace_bytes(args)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        ka.attention(q, k, v, out=out, workspace=ws, **kw)

    torch.cuda.synchronize()
    t_plan = time.perf_counter()
    call()  # first call of the shape: the host plan is built
    torch.cuda.synchronize()
    t_plan = time.perf_counter() - t_plan
    warm_calls, warm_ms = warm_up(call, warmup, WARMUP_MS)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ms = ev0.elapsed_time(ev1) / steps
    kern_ms, kern_median = attention_kernel_time(call, steps)
    bf, i8, dense_eq = algorithmic_work(w, info)
    return {
        "workload": name, "ms": ms, "wall_ms": wall * 1e3, "plan_build_ms": t_plan * 1e3,
        "effective_tflops": dense_eq / (ms * 1e-3) / 1e12,
        "mfma_tflops": (bf + i8) / (ms * 1e-3) / 1e12,
        "roofline_frac": roofline_time_s(bf, i8) / (ms * 1e-3),
        "bf16_flops": bf, "int8_ops": i8, "int8_tiles": info["int8_tiles"],
        "active_tiles": info["active_tiles"], "steps": steps, "warmup_calls": warm_calls,
        "warmup_ms": warm_ms, "attention_kernel_ms": kern_ms, "attention_kernel_ms_median": kern_median,
        "prework_ms": max(0.0, ms - kern_ms),
        "kernel_roofline_frac": roofline_time_s(bf, i8) / (kern_ms * 1e-3),
    }


def same_conditions_ab(names, steps, rounds, dev):
    """Workloads timed back to back in alternation, `rounds` times each, on their shared
    inputs and after one common warm-up: the median ms per call of each, for comparisons
    (band against dense at equal shape) that no difference in warm-up or box state can
    bias."""
    import torch

    import diffusion_transformer_attention_bidirectional_amd as ka
    from synth import WORKLOADS

    calls = {}
    for name in names:
        w = WORKLOADS[name]
        q, k, v = device_inputs(name, dev)
        kw = workload_kwargs(w)
        out = torch.empty_like(q)
        ws = torch.empty(max(ka.workspace_bytes(ka.args_for(q, k, **kw)), 256), dtype=torch.uint8, device=dev)
        calls[name] = (lambda q=q, k=k, v=v, out=out, ws=ws, kw=kw: ka.attention(q, k, v, out=out, workspace=ws,
                                                                                  **kw))
    warm_up(lambda: [c() for c in calls.values()], 8, WARMUP_MS)
    stream = torch.cuda.current_stream(dev)
    times = {name: [] for name in names}
    for _ in range(rounds):
        for name in names:
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(steps):
                calls[name]()
            ev1.record(stream)
            torch.cuda.synchronize()
            times[name].append(ev0.elapsed_time(ev1) / steps)
    med = {name: sorted(t)[len(t) // 2] for name, t in times.items()}
    return {"ms_median": med, "ms_all": times, "rounds": rounds, "steps_per_round": steps}


BLOCK_DETAIL = {"1mp_block": "1mp_dense", "4mp_block": "4mp_dense"}
BLOCK_MODEL_DIM = 6144   # Krea 2 hidden width (48 heads x 128)
BLOCK_Q_CHUNK = 4096     # query tokens per pass-two slice


def block_work(w, d_model):
    """(projection flops, attention flops) of one block context call: five projections
    (q, gate for Hq heads, k, v for Hkv heads, the output projection) and the dense
    attention."""
    n, hq, hkv, d = w.tokens, w.heads_q, w.heads_kv, w.head_dim
    proj = 2.0 * w.batch * n * d_model * d * (2 * hq + 2 * hkv + hq)
    return proj, 4.0 * hq * n * n * d * w.batch


def time_block(name, steps, warmup, dev):
    """attn_block_forward at the Krea 2 width: ms per call and the rate of its GEMMs plus
    attention.  Inputs are seeded device draws with the variances of the block's synthetic
    inputs; y keeps accumulating (values do not change the work)."""
    import torch

    import diffusion_transformer_attention_bidirectional_amd as ka
    from synth import WORKLOADS

    w = WORKLOADS[BLOCK_DETAIL[name]].with_(q_chunk=BLOCK_Q_CHUNK)
    dm, hq, hkv, d = BLOCK_MODEL_DIM, w.heads_q, w.heads_kv, w.head_dim
    g = torch.Generator(device=dev)
    g.manual_seed(1234)

    def draw(shape, std):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)

    x = draw((w.batch, w.tokens, dm), 1.0)
    wq, wg = draw((dm, hq * d), dm ** -0.5), draw((dm, hq * d), dm ** -0.5)
    wk, wv = draw((dm, hkv * d), dm ** -0.5), draw((dm, hkv * d), dm ** -0.5)
    wo = draw((hq * d, dm), (hq * d) ** -0.5)
    y = torch.zeros_like(x)
    kw = {k: v for k, v in workload_kwargs(w).items() if k != "text_tokens"}
    args = ka.make_args(batch=w.batch, heads_q=hq, heads_kv=hkv, text_tokens=w.text_tokens, dtype="bf16", **kw)
    ws = torch.empty(ka.block_workspace_bytes(args, dm), dtype=torch.uint8, device=dev)

    def call():
        ka.block_forward(x, wq, wk, wv, wg, wo, y, text_tokens=w.text_tokens, heads_q=hq, heads_kv=hkv,
                         workspace=ws, **kw)

    call()  # first call of the shape: plan and GEMM algorithm choice
    warm_calls, warm_ms = warm_up(call, warmup, WARMUP_MS)
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    proj, att = block_work(w, dm)
    return {"ms": ms, "tflops": (proj + att) / (ms * 1e-3) / 1e12, "projection_flops": proj,
            "attention_flops": att, "roofline_frac": (proj + att) / (PEAK_BF16_TFLOPS * 1e12) / (ms * 1e-3),
            "model_dim": dm, "q_chunk": BLOCK_Q_CHUNK, "warmup_calls": warm_calls, "warmup_ms": warm_ms}


class _HipRuntime:
    """The HIP runtime already loaded in this process (torch's, which the library shares),
    for timing events torch cannot create."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        import os

        self.c = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)

    def event(self):
        ev = self.c.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(self.c.byref(ev), self.c.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return ev

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ev, self.c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = self.c.c_float()
        rc = self.lib.hipEventElapsedTime(self.c.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def attention_kernel_time(call, steps):
    """Mean and median duration of the attention kernel alone over `steps` calls of `call`
    (already warm): the library records a pair of HIP events on the call's stream just before
    the first and just after the last attention-kernel launch of each call (the V relayout,
    the plan build and the quantiser fall outside the span).  The events are created without
    the system-scope fence: with it, every stop event would wait for a write-back of the L2
    caches (tens of microseconds) that the back-to-back calls of the throughput loop never
    pay, and the next launch would start on cold caches."""
    import torch

    import diffusion_transformer_attention_bidirectional_amd as ka

    hip = _HipRuntime()
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    torch.cuda.synchronize()
    try:
        for a, b in evs:
            ka.set_kernel_events(a, b)
            call()
    finally:
        ka.set_kernel_events()
    torch.cuda.synchronize()
    times = sorted(hip.elapsed_ms(a, b) for a, b in evs)
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    return sum(times) / steps, times[len(times) // 2]


def mfma_peak(dev, kind, iters=20000, launches=5):
    """Sustained MFMA rate (TFLOP/s or TOPS) of the 32x32 product the attention kernel uses,
    from the library's probe (attn_mfma_probe): two 8-wave workgroups per CU, each wave
    issuing four independent accumulation chains; timed with the same fence-free events."""
    import torch

    import diffusion_transformer_attention_bidirectional_amd as ka

    wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ka.mfma_probe(kind, wgs, iters, sink)  # untimed: clocks up, code resident
    hip = _HipRuntime()
    a, b = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(a, stream)
    ops = sum(ka.mfma_probe(kind, wgs, iters, sink) for _ in range(launches))
    hip.record(b, stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(a, b)
    hip.destroy(a)
    hip.destroy(b)
    return ops / (ms * 1e-3) / 1e12


def copy_reference(dev, nbytes=1 << 30, launches=5):
    """A plain elementwise copy (torch.neg on bf16) of known size, to calibrate the HBM byte
    counters: each launch reads and writes exactly nbytes."""
    import torch

    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(launches):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return {"copy_reference": "torch.neg bf16", "bytes_read_per_launch": nbytes,
            "bytes_written_per_launch": nbytes, "launches": launches}


def kernel_source_digest():
    """Digest of the attention kernel sources' code (comments and whitespace removed, so that
    only a change that can change the compiled kernels changes it); counter figures taken
    under another digest are stale."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in ("kernels.hip", "kernels.hpp"):
        with open(os.path.join(ROOT, "diffusion_transformer_attention_bidirectional_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per attention-kernel launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy reference), or None when no summary exists
    for this workload or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                key, val = line[2:].split(": ", 1)
                fields[key.strip("`")] = val.strip().strip("`")
    if fields.get("kernel_source_digest") != kernel_source_digest():
        return None
    return int(fields["hbm_bytes_per_launch"])


def cpu_baseline(name, heads=48, min_seconds=10.0):
    """The oracle on a bounded sample: all query rows of `heads` query heads, repeated until
    at least min_seconds of CPU work (a whole 1 MP call takes a few seconds)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attn_ref
    from synth import WORKLOADS, make_qkv, to_f64

    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    ora = attn_ref.Oracle(to_f64(q), to_f64(k), to_f64(v), w)
    passes = 0
    t0 = time.perf_counter()
    while True:
        out = ora.forward(heads=range(heads))
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    assert np.isfinite(out[:, :, :heads]).all()
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    flops = 4.0 * heads * w.tokens * w.tokens * w.head_dim * passes
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{name}: fp64 numpy oracle, all {w.tokens} query rows of {heads} of {w.heads_q} "
                      f"query heads, {passes} passes ({dt:.1f} s); dense-equivalent flops / wall time",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--copy-ref", action="store_true",
                    help="only run the copy kernel that calibrates the HBM byte counters")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this attention path is built and measured on a single MI355X "
              "(its (batch, KV head) units would shard across GPUs without exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    dev = torch.device("cuda:0")
    if a.copy_ref:
        print(json.dumps(copy_reference(dev)), flush=True)
        return
    names = [a.workload] + ([] if a.no_detail else [n for n in DETAIL if n != a.workload])
    for name in names:  # every input set is on the device before any timing
        device_inputs(name, dev)
    torch.cuda.synchronize()
    head = time_workload(a.workload, a.steps, a.warmup, dev)
    kern_ms, kern_median_ms = head["attention_kernel_ms"], head["attention_kernel_ms_median"]
    print(f"# {a.workload}: {head['ms']:.4f} ms/call (attention {kern_ms:.4f}), {head['effective_tflops']:.1f} "
          f"TFLOP/s after {head['warmup_calls']} warm-up calls in {head['warmup_ms']:.0f} ms", file=sys.stderr,
          flush=True)
    achieved = (head["bf16_flops"] + head["int8_ops"]) / (kern_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if head["int8_ops"] == 0 else roofline_peak_mixed(head["bf16_flops"], head["int8_ops"])
    measured = {k: mfma_peak(dev, k) for k in ("bf16", "i8", "bf16_random")}
    print(f"# MFMA probe: bf16 {measured['bf16']:.0f} TFLOP/s ({measured['bf16_random']:.0f} on random operands), "
          f"i8 {measured['i8']:.0f} TOPS sustained", file=sys.stderr, flush=True)
    detail = {}
    if not a.no_detail:
        for name in names[1:]:
            r = time_workload(name, a.steps, a.warmup, dev)
            detail[name] = {k: r[k] for k in ("ms", "effective_tflops", "mfma_tflops", "roofline_frac", "int8_tiles",
                                              "active_tiles", "plan_build_ms", "attention_kernel_ms",
                                              "attention_kernel_ms_median", "prework_ms", "kernel_roofline_frac",
                                              "warmup_calls", "warmup_ms")}
            print(f"# {name}: {r['ms']:.4f} ms/call (attention {r['attention_kernel_ms']:.4f}), "
                  f"{r['effective_tflops']:.1f} eff TFLOP/s, roofline {r['roofline_frac']:.3f}", file=sys.stderr,
                  flush=True)
        # band against dense at equal shape, timed in alternation after one common warm-up
        for pair in (("1mp_dense", "1mp_band"), ("4mp_dense_sliced", "4mp_band")):
            ab = same_conditions_ab(pair, a.steps, 5, dev)
            ab["band_over_dense"] = ab["ms_median"][pair[1]] / ab["ms_median"][pair[0]]
            detail[f"ab_{pair[1]}_vs_{pair[0]}"] = ab
            print(f"# A/B {pair[1]} vs {pair[0]}: {ab['ms_median'][pair[1]]:.4f} / {ab['ms_median'][pair[0]]:.4f} "
                  f"ms = {ab['band_over_dense']:.3f}", file=sys.stderr, flush=True)
        for name in BLOCK_DETAIL:
            r = time_block(name, max(5, a.steps // 5), max(2, a.warmup // 10), dev)
            detail[name] = r
            print(f"# {name}: {r['ms']:.4f} ms/call, {r['tflops']:.1f} TFLOP/s (projections + attention)",
                  file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(a.workload)
        print(f"# cpu oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads", file=sys.stderr, flush=True)
    from synth import WORKLOADS
    w = WORKLOADS[a.workload]
    line = {
        "metric": "attention ms/call + effective TFLOP/s (% MFMA peak), Krea2 shape at 1MP and 4MP",
        "value": round(head["effective_tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": a.workload, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "head_dim": w.head_dim, "text_tokens": w.text_tokens, "image_grid": f"{w.img_rows}x{w.img_cols}",
                   "tokens": w.tokens, "mode": w.mode, "q_chunk": w.q_chunk},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": measured_traffic(a.workload),
                     "kernel": f"attn_fwd_kernel<bf16, {w.mode}>", "kernel_ms": round(kern_ms, 5),
                     "kernel_ms_median": round(kern_median_ms, 5),
                     # the same kernel against the rate the MFMA probe sustains on this GPU: on
                     # operands that repeat, and (bf16) on operands that change every product,
                     # which draw more power and hold a lower clock, as random data does
                     "measured_mfma_peak": {"bf16_tflops": round(measured["bf16"], 1),
                                            "bf16_random_operands_tflops": round(measured["bf16_random"], 1),
                                            "i8_tops": round(measured["i8"], 1)},
                     "frac_of_measured_peak": round(
                         (head["bf16_flops"] / measured["bf16"] + head["int8_ops"] / measured["i8"]) / 1e12
                         / (kern_ms * 1e-3), 4),
                     "frac_of_random_operand_peak": round(
                         (head["bf16_flops"] / measured["bf16_random"] + head["int8_ops"] / measured["i8"]) / 1e12
                         / (kern_ms * 1e-3), 4)},
        "plan_build_ms": round(head["plan_build_ms"], 3),
        # untimed calls before the K timed ones: at least --warmup and at least WARMUP_MS of work
        "warmup_calls_made": head["warmup_calls"],
        "warmup_ms": round(head["warmup_ms"], 1),
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
