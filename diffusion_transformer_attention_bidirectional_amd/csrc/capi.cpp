// C ABI: validation, plan cache, launch sequencing.  Declarations and the meaning of
// every argument are in include/krea_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <list>
#include <memory>
#include <mutex>
#include <string>

#include "gemm.hpp"
#include "kernels.hpp"
#include "krea_attn.h"
#include "plan.hpp"

namespace {

thread_local std::string g_err;
// Measurement events recorded around the attention-kernel launches of attn_forward.
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

attn_status fail(attn_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// A cached host plan: the layout, counts, the TileMix pick threshold and the scanline
// geometry.  It holds no device memory: every call builds its tile lists on the device, in
// its own workspace, from these scalars, so evicting a plan frees host memory only and never
// touches memory that queued work or a captured graph may read.
struct CachedPlan {
  std::string key;
  krea::Plan plan;
};

constexpr size_t kMaxPlans = 8;  // the Scanline page keeps at most eight masks cached
std::mutex g_mu;
std::list<std::shared_ptr<const CachedPlan>> g_cache;  // most recent first

attn_status get_plan(const attn_args& a, std::shared_ptr<const CachedPlan>* out) {
  const std::string key = krea::plan_key(a);
  {
    std::lock_guard<std::mutex> lock(g_mu);
    for (auto it = g_cache.begin(); it != g_cache.end(); ++it) {
      if ((*it)->key == key) {
        g_cache.splice(g_cache.begin(), g_cache, it);
        *out = g_cache.front();
        return ATTN_OK;
      }
    }
  }
  auto cp = std::make_shared<CachedPlan>();
  cp->key = key;
  cp->plan = krea::build_plan(a);
  const krea::Plan& p = cp->plan;
  if (std::getenv("KREA_ATTN_LOG")) {
    std::fprintf(stderr, "[krea_attn] plan built: mode %d, %d blocks, %lld INT8 tiles, %lld active, %lld partial\n",
                 a.mode, p.lay.nb, (long long)p.int8_tiles, (long long)p.active_tiles, (long long)p.partial_tiles);
  }
  std::lock_guard<std::mutex> lock(g_mu);
  g_cache.push_front(cp);
  while (g_cache.size() > kMaxPlans) g_cache.pop_back();
  *out = cp;
  return ATTN_OK;
}

attn_status check_args(const attn_args* a) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  std::string err;
  const attn_status s = krea::validate_args(*a, err);
  if (s != ATTN_OK) return fail(s, err);
  return ATTN_OK;
}

attn_status check_tensor(const attn_tensor* t, const char* name) {
  if (!t || !t->ptr) return fail(ATTN_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (((uintptr_t)t->ptr & 15) != 0) return fail(ATTN_ERR_INVALID_ARG, std::string(name) + " must be 16-byte aligned");
  if ((t->stride_b & 7) || (t->stride_t & 7) || (t->stride_h & 7))
    return fail(ATTN_ERR_INVALID_ARG, std::string(name) + " strides must be multiples of 8 elements");
  if (t->stride_b < 0 || t->stride_t < 0 || t->stride_h < 0)
    return fail(ATTN_ERR_INVALID_ARG, std::string(name) + " strides must be >= 0");
  return ATTN_OK;
}

krea::TensorRef ref(const attn_tensor* t) { return krea::TensorRef{t->ptr, t->stride_b, t->stride_t, t->stride_h}; }

float scale_of(const attn_args& a) {
  return a.softmax_scale > 0.0f ? a.softmax_scale : (float)(1.0 / std::sqrt((double)a.head_dim));
}

krea::AttnParams make_params(const attn_args& a, const krea::Plan& plan) {
  krea::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  const krea::Layout& l = plan.lay;
  p.batch = a.batch;
  p.heads_q = a.heads_q;
  p.heads_kv = a.heads_kv;
  p.group = a.heads_q / a.heads_kv;
  p.n = l.n;
  p.text = l.text;
  p.t_pad = l.t_pad;
  p.image = l.image;
  p.cols = l.cols;
  p.cols_magic = (uint32_t)(0xFFFFFFFFu / (uint32_t)l.cols);
  p.length = l.length;
  p.nb = l.nb;
  p.q_begin = 0;
  p.q_end = l.length;
  p.scale_log2 = (float)((double)scale_of(a) * 1.4426950408889634);
  p.half_window = a.window / 2;
  p.tile_aligned = a.tile_aligned ? 1 : 0;
  p.smooth_k = a.smooth_k ? 1 : 0;
  p.split = 1;
  return p;
}

// The device plan builder's rule and outputs, in workspace `ws` (TileMix with INT8 tiles and
// scanline; null otherwise), and the plan pointers the attention kernel reads.
bool plan_build(const attn_args& a, const krea::Plan& plan, const krea::WorkspaceLayout& w, unsigned char* ws,
                krea::PlanBuild* pb, krea::AttnParams* p) {
  const bool tilemix8 = a.mode == ATTN_TILEMIX && plan.int8_tiles > 0;
  if (!(tilemix8 || a.mode == ATTN_SCANLINE) || !w.has_plan) return false;
  std::memset(pb, 0, sizeof(*pb));
  pb->mode = a.mode;
  pb->nb = plan.lay.nb;
  pb->n = plan.lay.n;
  pb->route = plan.route_rule;
  pb->geom = plan.geom;
  pb->map = ws + w.plan_map;
  pb->lists = (int32_t*)(ws + w.plan_lists);
  pb->row_count = (int32_t*)(ws + w.plan_rows);
  pb->full_count = (int32_t*)(ws + w.plan_full);
  if (p != nullptr) {
    if (tilemix8) p->route = pb->map;
    p->cols_list = pb->lists;
    p->row_count = pb->row_count;
    p->full_count = pb->full_count;
  }
  return true;
}

krea::QuantParams make_quant(const attn_args& a, const attn_tensor* q, const attn_tensor* k, unsigned char* ws) {
  const krea::WorkspaceLayout w = krea::workspace_layout(a);
  const krea::Layout l = krea::make_layout(a);
  krea::QuantParams qp;
  std::memset(&qp, 0, sizeof(qp));
  qp.q = ref(q);
  qp.k = ref(k);
  qp.batch = a.batch;
  qp.heads_q = a.heads_q;
  qp.heads_kv = a.heads_kv;
  qp.n = l.n;
  qp.text = l.text;
  qp.nb = l.nb;
  qp.smooth_k = a.smooth_k ? 1 : 0;
  qp.bf16 = a.dtype == ATTN_BF16;
  qp.k_part = (double*)(ws + w.k_part);
  qp.k_mean = (float*)(ws + w.k_mean);
  qp.k_norm8 = (float*)(ws + w.k_norm8);
  qp.k_codes = (int8_t*)(ws + w.k_codes);
  qp.k_scale = (float*)(ws + w.k_scale);
  qp.q_inv = (float*)(ws + w.q_inv);
  qp.q_scale = (float*)(ws + w.q_scale);
  return qp;
}

// Compute units of the current device (cached per device id).
int cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

attn_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_workspace_bytes(const attn_args* args, size_t* bytes) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (!bytes) return fail(ATTN_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = krea::workspace_layout(*args).total;
  g_err.clear();
  return ATTN_OK;
}

}  // extern "C"

namespace {

// One attention call after validation and its pre-work (pre-pass with the plan build,
// quantiser), ready to launch its query slices: the block path changes q, gate and o
// between slices.
struct Prepared {
  krea::AttnParams p;
  std::shared_ptr<const CachedPlan> cp;
  krea::WorkspaceLayout w;
  krea::TailRule tail;
  attn_args a;
  int kmode = ATTN_DENSE;  // the attention kernel's mode
  hipStream_t st = nullptr;
  bool bf16 = true;
  int length = 0, chunk = 0;
  int slices() const { return (length + chunk - 1) / chunk; }
};

void set_output(krea::AttnParams& p, const attn_tensor* o, const attn_tensor* gate);

attn_status prepare(const attn_args* args, const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                    const attn_tensor* gate, const attn_tensor* o, void* workspace, size_t workspace_bytes,
                    void* stream, Prepared* out) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if ((s = check_tensor(q, "q")) || (s = check_tensor(k, "k")) || (s = check_tensor(v, "v")) ||
      (s = check_tensor(o, "o")) || (gate && (s = check_tensor(gate, "gate"))))
    return s;
  const attn_args& a = *args;
  if (k->stride_t >= (1 << 23))
    return fail(ATTN_ERR_INVALID_ARG, "k token stride must be below 2^23 elements (32-bit tile offsets)");
  const krea::WorkspaceLayout w = krea::workspace_layout(a);
  if (!workspace || workspace_bytes < w.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace smaller than attn_workspace_bytes()");
  if (workspace && ((uintptr_t)workspace & 255)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  std::shared_ptr<const CachedPlan> cp;
  if ((s = get_plan(a, &cp)) != ATTN_OK) return s;
  const krea::Plan& plan = cp->plan;
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  krea::AttnParams p = make_params(a, plan);
  p.q = ref(q);
  p.k = ref(k);
  p.v = ref(v);
  set_output(p, o, gate);
  const bool bf16 = a.dtype == ATTN_BF16;
  p.v_t = (const uint16_t*)(ws + w.v_t);
  p.k_norm = (float*)(ws + w.k_norm);
  if (a.mode != ATTN_SCANLINE) {
    p.tail_count = (int32_t*)(ws + w.tail_count);
    p.tail_state = (float*)(ws + w.tail_state);
  }
  krea::PlanBuild pb;
  const bool has_plan = plan_build(a, plan, w, ws, &pb, &p);
  if (a.mode == ATTN_TILEMIX && plan.int8_tiles > 0) {
    const krea::QuantParams qp = make_quant(a, q, k, ws);
    if ((s = hip_check(krea::launch_prepass(p, (uint16_t*)p.v_t, &qp, &pb, a.mode, bf16, st), "pre-pass launch")) !=
        ATTN_OK)
      return s;
    if ((s = hip_check(krea::launch_quant_finish(qp, st), "quantiser launch")) != ATTN_OK) return s;
    p.k_mean = qp.k_mean;
    p.k_codes = qp.k_codes;
    p.k_scale = qp.k_scale;
    p.k_norm8 = qp.k_norm8;
    p.q_inv = qp.q_inv;
    p.q_scale = qp.q_scale;
  } else {
    if ((s = hip_check(krea::launch_prepass(p, (uint16_t*)p.v_t, nullptr, has_plan ? &pb : nullptr, a.mode, bf16,
                                            st),
                       "pre-pass launch")) != ATTN_OK)
      return s;
  }
  out->p = p;
  out->cp = cp;
  out->w = w;
  out->tail = krea::tail_rule(a, plan.lay, a.mode != ATTN_SCANLINE ? cu_count() : 0, w.tail_parts);
  out->a = a;
  // TileMix with no INT8 tile is dense attention: the dense kernel runs it (pattern zero is
  // bit-identical to dense)
  out->kmode = (a.mode == ATTN_TILEMIX && plan.int8_tiles == 0) ? ATTN_DENSE : a.mode;
  out->st = st;
  out->bf16 = bf16;
  out->length = plan.lay.length;
  out->chunk = a.q_chunk > 0 ? a.q_chunk : out->length;
  return ATTN_OK;
}

void set_output(krea::AttnParams& p, const attn_tensor* o, const attn_tensor* gate) {
  p.o = o->ptr;
  p.o_sb = o->stride_b;
  p.o_st = o->stride_t;
  p.o_sh = o->stride_h;
  p.gate = gate ? gate->ptr : nullptr;
  p.g_sb = gate ? gate->stride_b : 0;
  p.g_st = gate ? gate->stride_t : 0;
  p.g_sh = gate ? gate->stride_h : 0;
}

// The work items of one slice's launch: whole items and split ones, by the call's global
// split rule, and the scanline order's text query tiles.
void set_launch(Prepared& pr, int slice) {
  krea::AttnParams& p = pr.p;
  p.q_begin = slice * pr.chunk;
  p.q_end = std::min(pr.length, p.q_begin + pr.chunk);
  const int nq = (p.q_end - p.q_begin + 63) / 64;
  const int64_t J = (int64_t)(pr.a.heads_q / 4) * pr.a.batch;
  p.lsplit = krea::launch_split(pr.tail, J, p.q_begin / 64, nq);
  p.split = p.lsplit.n_split > 0 ? pr.tail.split : 1;
  p.n_long = pr.a.mode == ATTN_SCANLINE ? krea::scan_long_tiles(pr.cp->plan.lay, p.q_begin, nq) : 0;
}

attn_status launch_slice(Prepared& pr, int slice) {
  set_launch(pr, slice);
  return hip_check(krea::launch_attention(pr.p, pr.kmode, pr.bf16, pr.st), "attention launch");
}

attn_status forward_impl(const attn_args* args, const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                         const attn_tensor* gate, const attn_tensor* o, void* workspace, size_t workspace_bytes,
                         void* stream) {
  Prepared pr;
  attn_status s = prepare(args, q, k, v, gate, o, workspace, workspace_bytes, stream, &pr);
  if (s != ATTN_OK) return s;
  if (g_ev_start && (s = hip_check(hipEventRecord(g_ev_start, pr.st), "timing event")) != ATTN_OK) return s;
  for (int slice = 0; slice < pr.slices(); ++slice)
    if ((s = launch_slice(pr, slice)) != ATTN_OK) return s;
  if (g_ev_stop && (s = hip_check(hipEventRecord(g_ev_stop, pr.st), "timing event")) != ATTN_OK) return s;
  g_err.clear();
  return ATTN_OK;
}

// Workspace of the block path (bytes from its start, 256-byte aligned regions).
struct BlockLayout {
  size_t k = 0, v = 0, q = 0, g = 0, o = 0, attn = 0, gemm = 0, total = 0;
  int64_t slice_rows = 0;  // most token rows of one query slice
};

BlockLayout block_layout(const attn_args& a) {
  const krea::Layout l = krea::make_layout(a);
  const int chunk = a.q_chunk > 0 ? a.q_chunk : l.length;
  BlockLayout b;
  b.slice_rows = std::min<int64_t>(l.n, chunk);
  const size_t kv = (size_t)a.batch * l.n * a.heads_kv * krea::kHeadDim * 2;
  const size_t qs = (size_t)a.batch * b.slice_rows * a.heads_q * krea::kHeadDim * 2;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  b.k = off;    off = up(off + kv);
  b.v = off;    off = up(off + kv);
  b.q = off;    off = up(off + qs);
  b.g = off;    off = up(off + qs);
  b.o = off;    off = up(off + qs);
  b.attn = off; off = up(off + krea::workspace_layout(a).total);
  b.gemm = off; off = up(off + krea::kGemmWorkspace);
  b.total = off;
  return b;
}

// Physical token rows [r0, r1) of the logical query positions [l0, l1): the same range
// for dense and TileMix; scanline drops the padding, and what remains is contiguous.
void physical_rows(const krea::Layout& l, int l0, int l1, int64_t* r0, int64_t* r1) {
  const int ta = std::min(l0, l.text), tb = std::min(l1, l.text);
  const int ia = std::max(l0, l.t_pad), ib = std::min(l1, l.t_pad + l.image);
  *r0 = ta < tb ? ta : (ia < ib ? l.text + (ia - l.t_pad) : 0);
  *r1 = ia < ib ? l.text + (ib - l.t_pad) : (ta < tb ? tb : 0);
}

attn_status gemm_check(bool ok, const std::string& err) {
  return ok ? ATTN_OK : fail(ATTN_ERR_DEVICE, err);
}

}  // namespace

extern "C" {

attn_status attn_forward(const attn_args* args, const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                         const attn_tensor* o, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(args, q, k, v, nullptr, o, workspace, workspace_bytes, stream);
}

attn_status attn_forward_noalloc(const attn_args* args, const attn_tensor* q, const attn_tensor* k,
                                 const attn_tensor* v, const attn_tensor* o, void* stream) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  const size_t need = krea::workspace_layout(*args).total;
  if (need > krea::kScratchBytes) {
    char msg[160];
    std::snprintf(msg, sizeof(msg), "this call needs %zu bytes of workspace; the library's static scratch holds %zu",
                  need, krea::kScratchBytes);
    return fail(ATTN_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if ((s = hip_check(krea::scratch_region(&ws), "static scratch address")) != ATTN_OK) return s;
  return forward_impl(args, q, k, v, nullptr, o, ws, krea::kScratchBytes, stream);
}

attn_status attn_block_workspace_bytes(const attn_args* args, int32_t model_dim, size_t* bytes) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (!bytes) return fail(ATTN_ERR_INVALID_ARG, "bytes is NULL");
  if (model_dim <= 0 || model_dim % 8) return fail(ATTN_ERR_INVALID_ARG, "model_dim must be a positive multiple of 8");
  *bytes = block_layout(*args).total;
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_block_forward(const attn_args* args, const attn_block_weights* wt, const void* x, void* y,
                               void* workspace, size_t workspace_bytes, void* stream) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (!wt || !wt->w_q || !wt->w_k || !wt->w_v || !wt->w_gate || !wt->w_o)
    return fail(ATTN_ERR_INVALID_ARG, "block weights missing");
  if (wt->model_dim <= 0 || wt->model_dim % 8 || wt->reserved != 0)
    return fail(ATTN_ERR_INVALID_ARG, "model_dim must be a positive multiple of 8 and reserved 0");
  const void* ptrs[] = {wt->w_q, wt->w_k, wt->w_v, wt->w_gate, wt->w_o, x, y};
  for (const void* ptr : ptrs)
    if (!ptr || ((uintptr_t)ptr & 15)) return fail(ATTN_ERR_INVALID_ARG, "x, y and weights must be 16-byte aligned");
  const attn_args& a = *args;
  const BlockLayout bl = block_layout(a);
  if (!workspace || workspace_bytes < bl.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace smaller than attn_block_workspace_bytes()");
  if ((uintptr_t)workspace & 255) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const krea::Layout lay = krea::make_layout(a);
  const bool bf16 = a.dtype == ATTN_BF16;
  const int64_t D = wt->model_dim, N = lay.n, B = a.batch;
  const int64_t hq = (int64_t)a.heads_q * krea::kHeadDim, hkv = (int64_t)a.heads_kv * krea::kHeadDim;
  unsigned char* ws = (unsigned char*)workspace;
  void* kbuf = ws + bl.k;
  void* vbuf = ws + bl.v;
  uint16_t* qbuf = (uint16_t*)(ws + bl.q);
  uint16_t* gbuf = (uint16_t*)(ws + bl.g);
  uint16_t* obuf = (uint16_t*)(ws + bl.o);
  void* gws = ws + bl.gemm;
  hipStream_t st = (hipStream_t)stream;
  std::string err;
  // pass one: K and V of every token
  if ((s = gemm_check(krea::gemm_rows(bf16, N, hkv, D, x, D, N * D, wt->w_k, kbuf, hkv, N * hkv, (int)B, false, gws,
                                      krea::kGemmWorkspace, st, &err),
                      err)) ||
      (s = gemm_check(krea::gemm_rows(bf16, N, hkv, D, x, D, N * D, wt->w_v, vbuf, hkv, N * hkv, (int)B, false, gws,
                                      krea::kGemmWorkspace, st, &err),
                      err)))
    return s;
  const attn_tensor kt{kbuf, N * hkv, hkv, krea::kHeadDim};
  const attn_tensor vt{vbuf, N * hkv, hkv, krea::kHeadDim};
  // the slice buffers hold the slice's rows only: a tensor view whose token r0 is the
  // buffer's first row (rows outside the slice are never touched)
  auto view = [&](uint16_t* buf, int64_t r0, int64_t rows) {
    return attn_tensor{buf - r0 * hq, rows * hq, hq, krea::kHeadDim};
  };
  int64_t r0 = 0, r1 = 0;
  const int chunk = a.q_chunk > 0 ? a.q_chunk : lay.length;
  physical_rows(lay, 0, std::min(lay.length, chunk), &r0, &r1);
  attn_tensor qv = view(qbuf, r0, std::max<int64_t>(r1 - r0, 1)), gv = view(gbuf, r0, std::max<int64_t>(r1 - r0, 1)),
              ov = view(obuf, r0, std::max<int64_t>(r1 - r0, 1));
  Prepared pr;
  if ((s = prepare(args, &qv, &kt, &vt, &gv, &ov, ws + bl.attn, krea::workspace_layout(a).total, stream, &pr)) !=
      ATTN_OK)
    return s;
  // pass two, one query slice at a time
  for (int slice = 0; slice < pr.slices(); ++slice) {
    const int l0 = slice * pr.chunk;
    physical_rows(lay, l0, std::min(pr.length, l0 + pr.chunk), &r0, &r1);
    const int64_t rows = r1 - r0;
    if (rows <= 0) continue;
    const uint16_t* xs = (const uint16_t*)x + r0 * D;
    if ((s = gemm_check(krea::gemm_rows(bf16, rows, hq, D, xs, D, N * D, wt->w_q, qbuf, hq, rows * hq, (int)B, false,
                                        gws, krea::kGemmWorkspace, st, &err),
                        err)) ||
        (s = gemm_check(krea::gemm_rows(bf16, rows, hq, D, xs, D, N * D, wt->w_gate, gbuf, hq, rows * hq, (int)B,
                                        false, gws, krea::kGemmWorkspace, st, &err),
                        err)))
      return s;
    qv = view(qbuf, r0, rows);
    gv = view(gbuf, r0, rows);
    ov = view(obuf, r0, rows);
    pr.p.q = ref(&qv);
    set_output(pr.p, &ov, &gv);
    if ((s = launch_slice(pr, slice)) != ATTN_OK) return s;
    // the gate slice has been read by the attention launch: when the projection's output
    // fits in it, it is where the first call of this shape times the GEMM's candidates
    void* tune = rows * D <= bl.slice_rows * hq ? (void*)gbuf : nullptr;
    if ((s = gemm_check(krea::gemm_rows(bf16, rows, D, hq, obuf, hq, rows * hq, wt->w_o, (uint16_t*)y + r0 * D, D,
                                        N * D, (int)B, true, gws, krea::kGemmWorkspace, st, &err, tune),
                        err)))
      return s;
  }
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_forward_gated(const attn_args* args, const attn_tensor* q, const attn_tensor* k,
                               const attn_tensor* v, const attn_tensor* gate, const attn_tensor* o,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!gate) return fail(ATTN_ERR_INVALID_ARG, "gate is NULL");
  return forward_impl(args, q, k, v, gate, o, workspace, workspace_bytes, stream);
}


attn_status attn_plan_info_get(const attn_args* args, attn_plan_info* out) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (!out) return fail(ATTN_ERR_INVALID_ARG, "out is NULL");
  const krea::Plan p = krea::build_plan(*args);
  out->n_blocks = p.lay.nb;
  out->text_blocks = (p.lay.text + krea::kTile - 1) / krea::kTile;
  out->logical_tokens = p.lay.length;
  out->text_pad = p.lay.t_pad;
  out->int8_tiles = p.int8_tiles;
  out->active_tiles = p.active_tiles;
  out->partial_tiles = p.partial_tiles;
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_route_map(const attn_args* args, uint8_t* out, int32_t nb) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (args->mode != ATTN_TILEMIX) return fail(ATTN_ERR_INVALID_ARG, "route map exists for ATTN_TILEMIX only");
  const krea::Layout l = krea::make_layout(*args);
  if (!out || nb != l.nb) return fail(ATTN_ERR_INVALID_ARG, "out is NULL or nb does not match the plan");
  const std::vector<uint8_t> r = krea::build_route_map(*args, l, nullptr);
  std::memcpy(out, r.data(), r.size());
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_block_mask(const attn_args* args, uint8_t* out, int32_t nb) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (args->mode != ATTN_SCANLINE) return fail(ATTN_ERR_INVALID_ARG, "block mask exists for ATTN_SCANLINE only");
  const krea::Layout l = krea::make_layout(*args);
  if (!out || nb != l.nb) return fail(ATTN_ERR_INVALID_ARG, "out is NULL or nb does not match the plan");
  const std::vector<uint8_t> m = krea::build_block_mask(*args, l);
  std::memcpy(out, m.data(), m.size());
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_item_order(const attn_args* args, int32_t slice, int32_t* out, int64_t n) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (args->mode != ATTN_SCANLINE) return fail(ATTN_ERR_INVALID_ARG, "item order exists for ATTN_SCANLINE only");
  const krea::Layout l = krea::make_layout(*args);
  const int chunk = args->q_chunk > 0 ? args->q_chunk : l.length;
  const int slices = (l.length + chunk - 1) / chunk;
  if (slice < 0 || slice >= slices) return fail(ATTN_ERR_INVALID_ARG, "slice out of range");
  const int q0 = slice * chunk, q1 = std::min(l.length, q0 + chunk);
  if (!out || n != krea::attention_items(*args, q1 - q0))
    return fail(ATTN_ERR_INVALID_ARG, "out is NULL or n is not the launch's size");
  const std::vector<int32_t> order = krea::scan_item_order(*args, l, q0, q1);
  std::memcpy(out, order.data(), order.size() * sizeof(int32_t));
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_launch_items(const attn_args* args, int32_t slice, int32_t cus, int32_t* out, int64_t n,
                              int64_t* workgroups) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (cus < 1) return fail(ATTN_ERR_INVALID_ARG, "cus must be >= 1");
  const krea::Layout l = krea::make_layout(*args);
  const int chunk = args->q_chunk > 0 ? args->q_chunk : l.length;
  const int slices = (l.length + chunk - 1) / chunk;
  if (slice < 0 || slice >= slices) return fail(ATTN_ERR_INVALID_ARG, "slice out of range");
  const int q0 = slice * chunk, q1 = std::min(l.length, q0 + chunk), nq = (q1 - q0 + 63) / 64;
  const krea::TailRule t = krea::tail_rule(*args, l, cus, krea::workspace_layout(*args).tail_parts);
  const int64_t J = (int64_t)(args->heads_q / 4) * args->batch;
  const krea::LaunchSplit ls = krea::launch_split(t, J, q0 / 64, nq);
  const int split = ls.n_split > 0 ? t.split : 1;
  const int64_t grid = ls.n_full + ls.n_split * split;
  if (workgroups) *workgroups = grid;
  if (!out) {
    g_err.clear();
    return ATTN_OK;
  }
  if (n != grid) return fail(ATTN_ERR_INVALID_ARG, "n is not the launch's workgroup count");
  const bool scan = args->mode == ATTN_SCANLINE;
  const int n_long = scan ? krea::scan_long_tiles(l, q0, nq) : 0;
  for (int64_t L = 0; L < grid; ++L) {
    const krea::LaunchItem li = krea::launch_item(scan, ls, split, n_long, L);
    out[4 * L] = (int32_t)(q0 / 64 + li.qt);
    out[4 * L + 1] = (int32_t)li.j;
    out[4 * L + 2] = li.part;
    out[4 * L + 3] = li.nparts;
  }
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_device_plan(const attn_args* args, void* workspace, size_t workspace_bytes, uint8_t* map,
                             int32_t* lists, int32_t* row_count, int32_t* full_count, void* stream) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  const krea::WorkspaceLayout w = krea::workspace_layout(*args);
  if (!workspace || workspace_bytes < w.total) return fail(ATTN_ERR_WORKSPACE, "workspace too small");
  if ((uintptr_t)workspace & 255) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  std::shared_ptr<const CachedPlan> cp;
  if ((s = get_plan(*args, &cp)) != ATTN_OK) return s;
  krea::PlanBuild pb;
  if (!plan_build(*args, cp->plan, w, (unsigned char*)workspace, &pb, nullptr))
    return fail(ATTN_ERR_INVALID_ARG, "a device plan exists for ATTN_SCANLINE and for ATTN_TILEMIX with INT8 tiles");
  hipStream_t st = (hipStream_t)stream;
  if ((s = hip_check(krea::launch_plan(pb, st), "plan launch")) != ATTN_OK) return s;
  const size_t nb = (size_t)pb.nb;
  if (map && (s = hip_check(hipMemcpyAsync(map, pb.map, nb * nb, hipMemcpyDeviceToDevice, st), "copy"))) return s;
  if (lists && (s = hip_check(hipMemcpyAsync(lists, pb.lists, nb * nb * 4, hipMemcpyDeviceToDevice, st), "copy")))
    return s;
  if (row_count &&
      (s = hip_check(hipMemcpyAsync(row_count, pb.row_count, nb * 4, hipMemcpyDeviceToDevice, st), "copy")))
    return s;
  if (full_count &&
      (s = hip_check(hipMemcpyAsync(full_count, pb.full_count, nb * 4, hipMemcpyDeviceToDevice, st), "copy")))
    return s;
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_quantize(const attn_args* args, const attn_tensor* q, const attn_tensor* k, void* workspace,
                          size_t workspace_bytes, float* k_mean, int8_t* k_codes, float* k_scale, int8_t* q_codes,
                          float* q_scale, void* stream) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (args->mode != ATTN_TILEMIX) return fail(ATTN_ERR_INVALID_ARG, "attn_quantize needs mode ATTN_TILEMIX");
  if ((s = check_tensor(q, "q")) || (s = check_tensor(k, "k"))) return s;
  const krea::WorkspaceLayout w = krea::workspace_layout(*args);
  if (!workspace || workspace_bytes < w.total) return fail(ATTN_ERR_WORKSPACE, "workspace too small");
  hipStream_t st = (hipStream_t)stream;
  const krea::QuantParams qp = make_quant(*args, q, k, (unsigned char*)workspace);
  if ((s = hip_check(krea::launch_quant(qp, st), "quantiser launch")) != ATTN_OK) return s;
  const size_t bk = (size_t)args->batch * args->heads_kv, bq = (size_t)args->batch * args->heads_q;
  const size_t nb = (size_t)qp.nb;
  if (k_mean && (s = hip_check(hipMemcpyAsync(k_mean, qp.k_mean, bk * 128 * 4, hipMemcpyDeviceToDevice, st), "copy")))
    return s;
  if (k_codes &&
      (s = hip_check(hipMemcpyAsync(k_codes, qp.k_codes, bk * nb * 128 * 128, hipMemcpyDeviceToDevice, st), "copy")))
    return s;
  if (k_scale && (s = hip_check(hipMemcpyAsync(k_scale, qp.k_scale, bk * nb * 4, hipMemcpyDeviceToDevice, st), "copy")))
    return s;
  if (q_scale && (s = hip_check(hipMemcpyAsync(q_scale, qp.q_scale, bq * nb * 4, hipMemcpyDeviceToDevice, st), "copy")))
    return s;
  if (q_codes && (s = hip_check(krea::launch_q_codes(qp, q_codes, st), "q codes launch"))) return s;
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_int8_scores(const attn_args* args, const attn_tensor* q, const attn_tensor* k, void* workspace,
                             size_t workspace_bytes, const int32_t* tiles, int32_t n_tiles, int32_t* out,
                             void* stream) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (args->mode != ATTN_TILEMIX) return fail(ATTN_ERR_INVALID_ARG, "attn_int8_scores needs mode ATTN_TILEMIX");
  if ((s = check_tensor(q, "q")) || (s = check_tensor(k, "k"))) return s;
  if (n_tiles < 0 || (n_tiles > 0 && (!tiles || !out))) return fail(ATTN_ERR_INVALID_ARG, "bad tile list");
  const krea::WorkspaceLayout w = krea::workspace_layout(*args);
  if (!workspace || workspace_bytes < w.total) return fail(ATTN_ERR_WORKSPACE, "workspace too small");
  std::shared_ptr<const CachedPlan> cp;
  if ((s = get_plan(*args, &cp)) != ATTN_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const krea::QuantParams qp = make_quant(*args, q, k, (unsigned char*)workspace);
  if ((s = hip_check(krea::launch_quant(qp, st), "quantiser launch")) != ATTN_OK) return s;
  krea::AttnParams p = make_params(*args, cp->plan);
  p.q = ref(q);
  p.k = ref(k);
  p.k_codes = qp.k_codes;
  p.q_inv = qp.q_inv;
  if ((s = hip_check(krea::launch_int8_scores(p, tiles, n_tiles, out, args->dtype == ATTN_BF16, st), "launch")))
    return s;
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_mask_row_counts(const attn_args* args, void* workspace, size_t workspace_bytes, int32_t* out,
                                 void* stream) {
  attn_status s = check_args(args);
  if (s != ATTN_OK) return s;
  if (!out) return fail(ATTN_ERR_INVALID_ARG, "out is NULL");
  const krea::WorkspaceLayout w = krea::workspace_layout(*args);
  if (!workspace || workspace_bytes < w.total) return fail(ATTN_ERR_WORKSPACE, "workspace too small");
  if ((uintptr_t)workspace & 255) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  std::shared_ptr<const CachedPlan> cp;
  if ((s = get_plan(*args, &cp)) != ATTN_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  krea::AttnParams p = make_params(*args, cp->plan);
  krea::PlanBuild pb;
  if (plan_build(*args, cp->plan, w, (unsigned char*)workspace, &pb, &p) &&
      (s = hip_check(krea::launch_plan(pb, st), "plan launch")) != ATTN_OK)
    return s;
  if ((s = hip_check(krea::launch_mask_counts(p, args->mode, out, st), "launch"))) return s;
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_mfma_probe(int32_t kind, int32_t workgroups, int32_t iters, void* sink, int64_t* ops,
                            void* stream) {
  if (kind < ATTN_PROBE_BF16 || kind > ATTN_PROBE_BF16_RANDOM) return fail(ATTN_ERR_INVALID_ARG, "unknown probe kind");
  if (workgroups < 1 || iters < 1) return fail(ATTN_ERR_INVALID_ARG, "workgroups and iters must be >= 1");
  if (sink == nullptr || ops == nullptr) return fail(ATTN_ERR_INVALID_ARG, "sink and ops must not be NULL");
  const int64_t per_mfma = kind == ATTN_PROBE_I8 ? 2LL * 32 * 32 * 32 : 2LL * 32 * 32 * 16;
  *ops = per_mfma * 4 * (int64_t)iters * 8 * (int64_t)workgroups;
  attn_status s;
  if ((s = hip_check(krea::launch_mfma_probe(kind, workgroups, iters, (float*)sink, (hipStream_t)stream), "launch")))
    return s;
  g_err.clear();
  return ATTN_OK;
}

attn_status attn_set_kernel_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(ATTN_ERR_INVALID_ARG, "give both events or neither");
  g_ev_start = (hipEvent_t)start_event;
  g_ev_stop = (hipEvent_t)stop_event;
  g_err.clear();
  return ATTN_OK;
}

const char* attn_status_string(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case ATTN_ERR_SHAPE: return "unsupported shape";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_err.c_str(); }

}  // extern "C"
