"""MI355X (gfx950) joint [text, image] attention for Krea 2 -- Python binding.

Argument marshalling over the C ABI of ``libkrea_attn.so`` (declared in
include/krea_attn.h); every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream only.  If the
library is not built, every call raises ``KreaAttnError``: there is no other path.

Modes ("Krea 2 TileMix Attention (FP16/INT8 tiles)" and "Krea 2 Scanline Attention"):
  "dense"     bidirectional softmax attention, GQA resolved in the kernel;
  "tilemix"   static per-tile FP16/INT8 routing (patterns "zero", "one", "band"),
              smooth_k mean-centring of K, one running softmax;
  "scanline"  text global, image tokens see image rows within window // 2.
``q_chunk`` slices the queries against the full K/V ("LayerStream: Krea2 Chunking").
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KREA_ATTN_LIB selects another build of the same library (the host-sanitizer build)
LIB_PATH = os.environ.get("KREA_ATTN_LIB") or os.path.join(_HERE, "libkrea_attn.so")

ATTN_F16, ATTN_BF16, ATTN_F32 = 0, 1, 2
MODES = {"dense": 0, "tilemix": 1, "scanline": 2}
PATTERNS = {"zero": 0, "one": 1, "band": 2, "all": 3, "sage": 4}
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported dtype", -3: "unsupported shape",
          -4: "workspace too small", -5: "device error"}

EXPORTS = ("attn_workspace_bytes", "attn_forward", "attn_forward_gated", "attn_forward_noalloc", "attn_block_workspace_bytes",
           "attn_block_forward", "attn_plan_info_get", "attn_route_map",
           "attn_block_mask", "attn_item_order", "attn_quantize", "attn_int8_scores", "attn_mask_row_counts",
           "attn_device_plan", "attn_launch_items",
           "attn_mfma_probe", "attn_set_kernel_events", "attn_status_string", "attn_last_error")


class KreaAttnError(RuntimeError):
    """A status code other than ATTN_OK, or the library missing."""

    def __init__(self, msg: str, status: int | None = None):
        super().__init__(msg)
        self.status = status


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("text_tokens", ctypes.c_int32), ("img_rows", ctypes.c_int32),
        ("img_cols", ctypes.c_int32), ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("mode", ctypes.c_int32), ("pattern", ctypes.c_int32), ("percentage", ctypes.c_double),
        ("band_blocks", ctypes.c_int32), ("smooth_k", ctypes.c_int32), ("seed", ctypes.c_uint64),
        ("window", ctypes.c_int32), ("tile_aligned", ctypes.c_int32), ("q_chunk", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class AttnTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_t", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


class AttnBlockWeights(ctypes.Structure):
    """attn_block_weights: device pointers of W_q, W_k, W_v, W_gate [D, out] and W_o [Hq d, D]."""
    _fields_ = [("w_q", ctypes.c_void_p), ("w_k", ctypes.c_void_p), ("w_v", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("model_dim", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class AttnPlanInfo(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int32), ("text_blocks", ctypes.c_int32),
                ("logical_tokens", ctypes.c_int32), ("text_pad", ctypes.c_int32),
                ("int8_tiles", ctypes.c_int64), ("active_tiles", ctypes.c_int64),
                ("partial_tiles", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the C-ABI library once; raise KreaAttnError when it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise KreaAttnError(f"{path} is missing: build it with __graft_entry__.build() "
                            "or python diffusion_transformer_attention_bidirectional_amd/build.py")
    # torch first: the library then binds to the HIP runtime (and hipBLASLt) torch brought
    # in, so device pointers and streams from torch are valid in it.  Loaded before torch,
    # it would bind to the system copy, and torch would then load a second runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "attn_workspace_bytes": [P(AttnArgs), P(sz)],
        "attn_forward": [P(AttnArgs), P(AttnTensor), P(AttnTensor), P(AttnTensor), P(AttnTensor), vp, sz, vp],
        "attn_forward_gated": [P(AttnArgs), P(AttnTensor), P(AttnTensor), P(AttnTensor), P(AttnTensor),
                               P(AttnTensor), vp, sz, vp],
        "attn_forward_noalloc": [P(AttnArgs), P(AttnTensor), P(AttnTensor), P(AttnTensor), P(AttnTensor), vp],
        "attn_block_workspace_bytes": [P(AttnArgs), i32, P(sz)],
        "attn_block_forward": [P(AttnArgs), P(AttnBlockWeights), vp, vp, vp, sz, vp],
        "attn_plan_info_get": [P(AttnArgs), P(AttnPlanInfo)],
        "attn_route_map": [P(AttnArgs), vp, i32],
        "attn_block_mask": [P(AttnArgs), vp, i32],
        "attn_item_order": [P(AttnArgs), i32, vp, ctypes.c_int64],
        "attn_quantize": [P(AttnArgs), P(AttnTensor), P(AttnTensor), vp, sz, vp, vp, vp, vp, vp, vp],
        "attn_int8_scores": [P(AttnArgs), P(AttnTensor), P(AttnTensor), vp, sz, vp, i32, vp, vp],
        "attn_mask_row_counts": [P(AttnArgs), vp, sz, vp, vp],
        "attn_device_plan": [P(AttnArgs), vp, sz, vp, vp, vp, vp, vp],
        "attn_launch_items": [P(AttnArgs), i32, i32, vp, ctypes.c_int64, P(ctypes.c_int64)],
        "attn_mfma_probe": [i32, i32, i32, vp, P(ctypes.c_int64), vp],
        "attn_set_kernel_events": [vp, vp],
    }
    for name, argtypes in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int32
    lib.attn_status_string.argtypes = [ctypes.c_int32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise KreaAttnError(f"{lib.attn_status_string(status).decode()}: {lib.attn_last_error().decode()}",
                            status)


def make_args(*, batch=1, heads_q=48, heads_kv=12, head_dim=128, text_tokens=0, img_rows=0, img_cols=0,
              dtype="bf16", softmax_scale=0.0, mode="dense", pattern="band", percentage=0.5,
              band_blocks=2, smooth_k=True, seed=0, window=11, tile_aligned=True, q_chunk=0) -> AttnArgs:
    dt = {"bf16": ATTN_BF16, "f16": ATTN_F16, "f32": ATTN_F32}[dtype] if isinstance(dtype, str) else int(dtype)
    return AttnArgs(batch, heads_q, heads_kv, head_dim, text_tokens, img_rows, img_cols, dt,
                    float(softmax_scale), MODES[mode] if isinstance(mode, str) else int(mode),
                    PATTERNS[pattern] if isinstance(pattern, str) else int(pattern), float(percentage),
                    band_blocks, 1 if smooth_k else 0, seed & ((1 << 64) - 1), window,
                    1 if tile_aligned else 0, q_chunk, 0)


def _dtype_name(t) -> str:
    import torch
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float16:
        return "f16"
    if t.dtype == torch.float32:
        return "f32"
    raise KreaAttnError(f"unsupported dtype {t.dtype}")


def _tensor(t) -> AttnTensor:
    if t.dim() != 4 or t.stride(3) != 1:
        raise KreaAttnError("tensors must be [B, N, H, head_dim] with head_dim contiguous")
    return AttnTensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _stream_handle(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(args: AttnArgs) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().attn_workspace_bytes(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def args_for(q, k, *, text_tokens, img_rows=0, img_cols=0, **kw) -> AttnArgs:
    b, n, hq, d = q.shape
    hkv = k.shape[2]
    return make_args(batch=b, heads_q=hq, heads_kv=hkv, head_dim=d, text_tokens=text_tokens,
                     img_rows=img_rows, img_cols=img_cols, dtype=_dtype_name(q), **kw)


def attention(q, k, v, *, text_tokens, img_rows=0, img_cols=0, mode="dense", out=None, workspace=None,
              stream=None, gate=None, **kw):
    """O = attention(q, k, v) on the GPU.  q [B, N, Hq, 128], k/v [B, N, Hkv, 128], bf16 or fp16,
    N = text_tokens + img_rows * img_cols.  With ``gate`` (shaped like q), O * sigmoid(gate)
    (attn_forward_gated).  Extra keywords as in make_args().  Asynchronous on the current (or
    given) stream."""
    import torch
    args = args_for(q, k, text_tokens=text_tokens, img_rows=img_rows, img_cols=img_cols, mode=mode, **kw)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    nbytes = workspace_bytes(args)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wlen = workspace.numel() if workspace is not None else 0
    lib = load_library()
    tq, tk, tv, to = (ctypes.byref(_tensor(t)) for t in (q, k, v, out))
    st = _stream_handle(stream, q.device)
    if gate is None:
        _check(lib.attn_forward(ctypes.byref(args), tq, tk, tv, to, wptr, wlen, st))
    else:
        if tuple(gate.shape) != tuple(q.shape) or gate.dtype != q.dtype:
            raise KreaAttnError("gate must have q's shape and dtype")
        _check(lib.attn_forward_gated(ctypes.byref(args), tq, tk, tv, ctypes.byref(_tensor(gate)), to, wptr, wlen,
                                      st))
    return out


def attention_noalloc(q, k, v, out, *, text_tokens, img_rows=0, img_cols=0, mode="dense", stream=None, **kw):
    """attention() through attn_forward_noalloc: the library's static device scratch serves as
    the workspace, so nothing is allocated (the caller passes ``out``).  Calls that overlap
    on one GPU share that scratch and race."""
    args = args_for(q, k, text_tokens=text_tokens, img_rows=img_rows, img_cols=img_cols, mode=mode, **kw)
    lib = load_library()
    _check(lib.attn_forward_noalloc(ctypes.byref(args), *(ctypes.byref(_tensor(t)) for t in (q, k, v, out)),
                                    _stream_handle(stream, q.device)))
    return out


def block_workspace_bytes(args: AttnArgs, model_dim: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().attn_block_workspace_bytes(ctypes.byref(args), int(model_dim), ctypes.byref(n)))
    return n.value


def block_forward(x, wq, wk, wv, wg, wo, y, *, text_tokens, img_rows=0, img_cols=0, heads_q, heads_kv, mode="dense",
                  workspace=None, stream=None, **kw):
    """y += (attention(x W_q, x W_k, x W_v) * sigmoid(x W_gate)) W_o on the GPU, in the two passes of
    attn_block_forward.  x, y: [B, N, D] contiguous; W_q, W_gate [D, Hq 128], W_k, W_v [D, Hkv 128],
    W_o [Hq 128, D]; all in one dtype (bf16 or fp16) on one device.  Returns y."""
    import torch
    tensors = (x, wq, wk, wv, wg, wo, y)
    if any(not t.is_contiguous() or t.dtype != x.dtype or t.device != x.device for t in tensors):
        raise KreaAttnError("x, y and the weights must be contiguous, of one dtype and on one device")
    b, n, d_model = x.shape
    args = make_args(batch=b, heads_q=heads_q, heads_kv=heads_kv, text_tokens=text_tokens, img_rows=img_rows,
                     img_cols=img_cols, dtype=_dtype_name(x), mode=mode, **kw)
    weights = AttnBlockWeights(wq.data_ptr(), wk.data_ptr(), wv.data_ptr(), wg.data_ptr(), wo.data_ptr(),
                               int(d_model), 0)
    nbytes = block_workspace_bytes(args, d_model)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _check(load_library().attn_block_forward(ctypes.byref(args), ctypes.byref(weights), ctypes.c_void_p(x.data_ptr()),
                                             ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
                                             workspace.numel(), _stream_handle(stream, x.device)))
    return y


PROBE_KINDS = {"bf16": 0, "f16": 1, "i8": 2, "bf16_random": 3}


def mfma_probe(kind: str, workgroups: int, iters: int, sink, stream=None) -> int:
    """Enqueue one MFMA throughput probe launch (attn_mfma_probe) on the stream; returns
    the operations it performs.  sink: a device tensor of at least 4 bytes, which receives a
    checksum of the first wave's accumulators."""
    ops = ctypes.c_int64(0)
    _check(load_library().attn_mfma_probe(PROBE_KINDS[kind], int(workgroups), int(iters),
                                          ctypes.c_void_p(sink.data_ptr()), ctypes.byref(ops),
                                          _stream_handle(stream, sink.device)))
    return ops.value


def set_kernel_events(start=None, stop=None):
    """Record two events around the attention-kernel launches of every later attention()
    call on this thread; no arguments turns it off.  Each is a torch.cuda.Event that has
    been recorded once (torch creates the HIP event on its first record) or a raw hipEvent_t
    handle (int or ctypes.c_void_p), e.g. one created with hipEventDisableSystemFence."""
    if (start is None) != (stop is None):
        raise KreaAttnError("give both events or neither")

    def ptr(e):
        if e is None:
            return None
        if isinstance(e, ctypes.c_void_p):
            return e
        if isinstance(e, int):
            return ctypes.c_void_p(e)
        return ctypes.c_void_p(e.cuda_event)

    _check(load_library().attn_set_kernel_events(ptr(start), ptr(stop)))


# ---------------------------------------------------------------- host-only plan views
def plan_info(args: AttnArgs) -> dict:
    info = AttnPlanInfo()
    _check(load_library().attn_plan_info_get(ctypes.byref(args), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in AttnPlanInfo._fields_}


# ---------------------------------------------------------------- caller policy
# The node wrappers on the pages decide whether their kernel runs at all: TileMix has an
# `enabled` switch and leaves short sequences to the stock attention (`min_tokens`,
# "Krea 2 TileMix Attention (FP16/INT8 tiles)", "The inputs that matter"), and prints one
# line saying what is active.  The library itself has no fallback; these helpers give a
# caller the same policy around it.

def should_use(tokens: int, *, enabled: bool = True, min_tokens: int = 0) -> bool:
    """True when a caller following the node's policy would run this library for a joint
    sequence of `tokens` tokens (otherwise it keeps its own attention)."""
    return bool(enabled) and tokens >= max(0, int(min_tokens))


def describe(args: AttnArgs) -> str:
    """One line naming the mode and what the plan routes or skips, for a caller's log."""
    info = plan_info(args)
    nb, total = info["n_blocks"], info["n_blocks"] ** 2
    mode = {v: k for k, v in MODES.items()}.get(args.mode, str(args.mode))
    head = (f"krea_attn {mode}: {args.heads_q} q / {args.heads_kv} kv heads, "
            f"{info['logical_tokens']} tokens, {nb}x{nb} tiles")
    if args.mode == MODES["tilemix"]:
        pattern = {v: k for k, v in PATTERNS.items()}.get(args.pattern, str(args.pattern))
        line = (f"{head}, pattern {pattern}: {info['int8_tiles']} INT8 "
                f"({100.0 * info['int8_tiles'] / total:.1f} %), smooth_k {'on' if args.smooth_k else 'off'}")
    elif args.mode == MODES["scanline"]:
        line = (f"{head}, window {args.window}{' tile-aligned' if args.tile_aligned else ''}: "
                f"{info['active_tiles']} active ({100.0 * info['active_tiles'] / total:.1f} %)")
    else:
        line = head
    if args.q_chunk:
        line += f", queries in slices of {args.q_chunk}"
    return line


def route_map(args: AttnArgs) -> np.ndarray:
    nb = plan_info(args)["n_blocks"]
    out = np.zeros((nb, nb), dtype=np.uint8)
    _check(load_library().attn_route_map(ctypes.byref(args), out.ctypes.data, nb))
    return out


def block_mask(args: AttnArgs) -> np.ndarray:
    nb = plan_info(args)["n_blocks"]
    out = np.zeros((nb, nb), dtype=np.uint8)
    _check(load_library().attn_block_mask(ctypes.byref(args), out.ctypes.data, nb))
    return out


def item_order(args: AttnArgs, slice_index: int = 0) -> np.ndarray:
    """Scanline: the work item each workgroup of one query slice's launch runs."""
    info = plan_info(args)
    rows = info["logical_tokens"]
    chunk = args.q_chunk if args.q_chunk > 0 else rows
    lo = slice_index * chunk
    n = ((min(rows, lo + chunk) - lo + 63) // 64) * (args.heads_q // 4) * args.batch if lo < rows else 0
    out = np.zeros(max(n, 1), dtype=np.int32)
    _check(load_library().attn_item_order(ctypes.byref(args), int(slice_index), out.ctypes.data, int(n)))
    return out[:n]


def launch_items(args: AttnArgs, slice_index: int, cus: int) -> np.ndarray:
    """Work items of one attention launch (host only): int32 [workgroups, 4] of (global
    64-query tile, pair, key-range part, parts) per workgroup, on a device with `cus` compute
    units."""
    lib = load_library()
    n = ctypes.c_int64(0)
    _check(lib.attn_launch_items(ctypes.byref(args), int(slice_index), int(cus), None, 0, ctypes.byref(n)))
    out = np.zeros((max(n.value, 1), 4), dtype=np.int32)
    _check(lib.attn_launch_items(ctypes.byref(args), int(slice_index), int(cus), out.ctypes.data, n.value, None))
    return out[:n.value]


# ---------------------------------------------------------------- device debug views
def quantize(q, k, args: AttnArgs, stream=None) -> dict:
    """smooth_k mean, INT8 codes and scales of K and Q as the attention call computes them."""
    import torch
    dev = q.device
    nb = plan_info(args)["n_blocks"]
    b, hq, hkv = args.batch, args.heads_q, args.heads_kv
    ws = torch.empty(workspace_bytes(args), dtype=torch.uint8, device=dev)
    res = {
        "k_mean": torch.empty((b, hkv, 128), dtype=torch.float32, device=dev),
        "k_codes": torch.empty((b, hkv, nb, 128, 128), dtype=torch.int8, device=dev),
        "k_scale": torch.empty((b, hkv, nb), dtype=torch.float32, device=dev),
        "q_codes": torch.empty((b, hq, nb, 128, 128), dtype=torch.int8, device=dev),
        "q_scale": torch.empty((b, hq, nb), dtype=torch.float32, device=dev),
    }
    _check(load_library().attn_quantize(
        ctypes.byref(args), ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), ws.data_ptr(), ws.numel(),
        res["k_mean"].data_ptr(), res["k_codes"].data_ptr(), res["k_scale"].data_ptr(),
        res["q_codes"].data_ptr(), res["q_scale"].data_ptr(), _stream_handle(stream, dev)))
    return res


def int8_scores(q, k, args: AttnArgs, tiles, stream=None):
    """INT32 q8 . k8 of tiles [(b, h, query block, key block), ...] -> int32 [n, 128, 128]."""
    import torch
    dev = q.device
    t = torch.as_tensor(np.asarray(tiles, dtype=np.int32).reshape(-1, 4), device=dev).contiguous()
    out = torch.empty((t.shape[0], 128, 128), dtype=torch.int32, device=dev)
    ws = torch.empty(workspace_bytes(args), dtype=torch.uint8, device=dev)
    _check(load_library().attn_int8_scores(
        ctypes.byref(args), ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), ws.data_ptr(), ws.numel(),
        t.data_ptr(), t.shape[0], out.data_ptr(), _stream_handle(stream, dev)))
    return out


def mask_row_counts(args: AttnArgs, device="cuda", stream=None):
    """Keys admitted per logical query row, as the attention kernel's tile lists (built on the
    device) and element mask evaluate them."""
    import torch
    n = plan_info(args)["logical_tokens"]
    dev = torch.device(device)
    out = torch.empty(n, dtype=torch.int32, device=dev)
    ws = torch.empty(max(workspace_bytes(args), 256), dtype=torch.uint8, device=dev)
    _check(load_library().attn_mask_row_counts(ctypes.byref(args), ws.data_ptr(), ws.numel(), out.data_ptr(),
                                               _stream_handle(stream, dev)))
    return out


def device_plan(args: AttnArgs, device="cuda", stream=None) -> dict:
    """The per-call plan as attn_forward builds it on the device (TileMix with INT8 tiles,
    scanline): map [nb, nb] uint8, lists [nb, nb] int32, row_count and full_count [nb]."""
    import torch
    nb = plan_info(args)["n_blocks"]
    dev = torch.device(device)
    res = {"map": torch.empty((nb, nb), dtype=torch.uint8, device=dev),
           "lists": torch.empty((nb, nb), dtype=torch.int32, device=dev),
           "row_count": torch.empty(nb, dtype=torch.int32, device=dev),
           "full_count": torch.empty(nb, dtype=torch.int32, device=dev)}
    ws = torch.empty(max(workspace_bytes(args), 256), dtype=torch.uint8, device=dev)
    _check(load_library().attn_device_plan(ctypes.byref(args), ws.data_ptr(), ws.numel(), res["map"].data_ptr(),
                                           res["lists"].data_ptr(), res["row_count"].data_ptr(),
                                           res["full_count"].data_ptr(), _stream_handle(stream, dev)))
    return res
