// Host planner.  Rules cited from the pages:
//   route map -- "Krea 2 TileMix Attention (FP16/INT8 tiles)", "What it actually
//     patches" (text tiles and a diagonal band stay FP16, the INT8 share counts the
//     image-image tiles left over) and "The inputs that matter" (patterns, percentage);
//   block mask -- "Krea 2 Scanline Attention", "What the mask actually is" (text global,
//     image rows within window / 2, padding to 128, 128-token block mask, tile_aligned)
//     and "The settings that matter" (window odd, at most 255).
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <tuple>

namespace krea {

static int blocks_of(int tokens) { return (tokens + kTile - 1) / kTile; }

attn_status validate_args(const attn_args& a, std::string& err) {
  if (a.dtype == ATTN_F32) {
    err = "fp32 inputs are not supported (bf16 or fp16 only)";
    return ATTN_ERR_UNSUPPORTED_DTYPE;
  }
  if (a.dtype != ATTN_BF16 && a.dtype != ATTN_F16) {
    err = "dtype must be ATTN_BF16 or ATTN_F16";
    return ATTN_ERR_INVALID_ARG;
  }
  if (a.head_dim != kHeadDim) {
    err = "head_dim must be 128";
    return ATTN_ERR_SHAPE;
  }
  if (a.batch < 1 || a.heads_q < 1 || a.heads_kv < 1) {
    err = "batch, heads_q and heads_kv must be >= 1";
    return ATTN_ERR_SHAPE;
  }
  if (a.heads_q % a.heads_kv != 0) {
    err = "heads_q must be a multiple of heads_kv";
    return ATTN_ERR_SHAPE;
  }
  if ((a.heads_q / a.heads_kv) % 4 != 0) {
    err = "heads_q / heads_kv must be a multiple of 4 (one workgroup serves 4 query heads of a KV head)";
    return ATTN_ERR_SHAPE;
  }
  if (a.text_tokens < 0 || a.img_rows < 0 || a.img_cols < 0) {
    err = "token counts must be >= 0";
    return ATTN_ERR_SHAPE;
  }
  const int64_t image = (int64_t)a.img_rows * a.img_cols;
  const int64_t n = (int64_t)a.text_tokens + image;
  if (n < 1) {
    err = "the joint sequence is empty";
    return ATTN_ERR_SHAPE;
  }
  if (n > (1 << 22)) {
    err = "at most 4194304 tokens";
    return ATTN_ERR_SHAPE;
  }
  if ((int64_t)a.batch * a.heads_q > 65535 * 4) {
    err = "batch * heads_q too large";
    return ATTN_ERR_SHAPE;
  }
  if (a.mode != ATTN_DENSE && a.mode != ATTN_TILEMIX && a.mode != ATTN_SCANLINE) {
    err = "mode must be ATTN_DENSE, ATTN_TILEMIX or ATTN_SCANLINE";
    return ATTN_ERR_INVALID_ARG;
  }
  if (!(a.softmax_scale >= 0.0f) || std::isinf(a.softmax_scale)) {
    err = "softmax_scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))";
    return ATTN_ERR_INVALID_ARG;
  }
  if (a.q_chunk < 0 || a.q_chunk % kTile != 0) {
    err = "q_chunk must be 0 or a positive multiple of 128";
    return ATTN_ERR_INVALID_ARG;
  }
  if (a.reserved != 0) {
    err = "reserved must be 0";
    return ATTN_ERR_INVALID_ARG;
  }
  if (a.mode == ATTN_TILEMIX) {
    if (a.pattern != ATTN_PAT_ZERO && a.pattern != ATTN_PAT_ONE && a.pattern != ATTN_PAT_BAND &&
        a.pattern != ATTN_PAT_ALL && a.pattern != ATTN_PAT_SAGE) {
      err = "pattern must be ATTN_PAT_ZERO, ATTN_PAT_ONE, ATTN_PAT_BAND, ATTN_PAT_ALL or ATTN_PAT_SAGE";
      return ATTN_ERR_INVALID_ARG;
    }
    if (!(a.percentage >= 0.0 && a.percentage <= 1.0)) {
      err = "percentage must be in [0, 1]";
      return ATTN_ERR_INVALID_ARG;
    }
    if (a.band_blocks < 0) {
      err = "band_blocks must be >= 0";
      return ATTN_ERR_INVALID_ARG;
    }
  }
  if (a.mode == ATTN_SCANLINE) {
    if (a.window < 1 || a.window > 255 || a.window % 2 == 0) {
      err = "window must be an odd integer in [1, 255]";
      return ATTN_ERR_INVALID_ARG;
    }
    if (a.img_rows < 1 || a.img_cols < 1) {
      err = "scanline needs an image grid (img_rows, img_cols >= 1)";
      return ATTN_ERR_SHAPE;
    }
  }
  if (a.mode != ATTN_DENSE) {
    const int64_t pad_text = (a.mode == ATTN_SCANLINE) ? ((int64_t)a.text_tokens + kTile - 1) / kTile * kTile
                                                       : a.text_tokens;
    if ((pad_text + image + kTile - 1) / kTile > kMaxPlanBlocks) {
      err = "TileMix and scanline take at most 4096 blocks of 128 tokens (524288 tokens)";
      return ATTN_ERR_SHAPE;
    }
  }
  err.clear();
  return ATTN_OK;
}

Layout make_layout(const attn_args& a) {
  Layout l;
  l.text = a.text_tokens;
  l.image = a.img_rows * a.img_cols;
  l.cols = a.img_cols > 0 ? a.img_cols : 1;
  l.n = l.text + l.image;
  if (a.mode == ATTN_SCANLINE) {
    l.t_pad = blocks_of(l.text) * kTile;
    l.length = blocks_of(l.t_pad + l.image) * kTile;
  } else {
    l.t_pad = l.text;
    l.length = l.n;
  }
  l.nb = blocks_of(l.length);
  return l;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t attention_items(const attn_args& a, int q_tokens) {
  return (int64_t)((q_tokens + 63) / 64) * (a.heads_q / 4) * a.batch;
}

int scan_long_tiles(const Layout& l, int q_begin, int nq) {
  // query tiles [q_begin + 64 i, + 64) with i < n hold a text query
  const int64_t n = ((int64_t)l.text - q_begin + 63) / 64;
  return (int)std::max<int64_t>(0, std::min<int64_t>(nq, l.text > q_begin ? n : 0));
}

std::vector<int32_t> scan_item_order(const attn_args& a, const Layout& l, int q_begin, int q_end) {
  const int nq = (q_end - q_begin + 63) / 64;
  const int64_t total = attention_items(a, q_end - q_begin);
  const int n_long = scan_long_tiles(l, q_begin, nq);
  std::vector<int32_t> order((size_t)total);
  for (int64_t L = 0; L < total; ++L) order[(size_t)L] = (int32_t)scan_item_of(total, nq, n_long, L);
  return order;
}

TailRule tail_rule(const attn_args& a, const Layout& l, int cus, int capacity) {
  // With one workgroup per compute unit, the G items of the whole call run in waves of
  // `cus`; the rem items of the last, partial wave each run as `split` workgroups over
  // consecutive key ranges.  Their rem * split parts take ceil(rem * split / cus) waves of
  // 1 / split of an item plus a fixed cost per part (pipeline fill, publishing and merging
  // the partial state: about 0.15 of a whole item as measured on the Krea shapes, where a
  // split of 2 beat 8), and the split is chosen to minimise that (ties: the smaller split).
  TailRule t;
  static const int max_split = [] {
    const char* e = std::getenv("KREA_ATTN_TAIL_SPLIT");  // cap on the split (0 or 1: off)
    return e ? std::atoi(e) : kMaxTailSplit;
  }();
  const int nb = l.nb;
  const int64_t G = attention_items(a, l.length);
  if (a.mode == ATTN_SCANLINE || cus <= 0 || capacity < 2 || nb < 2 || max_split < 2) return t;
  const int64_t rem = G % cus;
  if (rem == 0 || rem > kMaxTailItems) return t;
  int best = 1;
  double best_cost = 1.0;  // unsplit: one more wave of whole items
  constexpr double kPartCost = 0.15;
  for (int s = 2; s <= std::min({max_split, kMaxTailSplit, nb}); ++s) {
    if (rem * s > capacity) break;
    const double cost = (double)((rem * s + cus - 1) / cus) * (1.0 / s + kPartCost);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = s;
    }
  }
  if (best < 2) return t;
  t.split = best;
  t.split_from = G - rem;
  return t;
}

WorkspaceLayout workspace_layout(const attn_args& a) {
  WorkspaceLayout w;
  const Layout l = make_layout(a);
  const size_t bk = (size_t)a.batch * a.heads_kv, bq = (size_t)a.batch * a.heads_q;
  const size_t nb = (size_t)l.nb;
  size_t off = 0;
  w.v_t = off;     off = align256(off + bk * nb * (size_t)kTile * kHeadDim * 2);
  w.k_norm = off;  off = align256(off + bk * nb * sizeof(float));
  if (a.mode != ATTN_DENSE) {
    w.has_plan = true;
    w.plan_map = off;   off = align256(off + nb * nb);
    w.plan_lists = off; off = align256(off + nb * nb * sizeof(int32_t));
    w.plan_rows = off;  off = align256(off + nb * sizeof(int32_t));
    w.plan_full = off;  off = align256(off + nb * sizeof(int32_t));
  }
  if (a.mode == ATTN_SCANLINE) {
    w.total = off;
    return w;
  }
  if (l.nb >= 2) {
    const int64_t items = attention_items(a, l.length);
    w.tail_parts = (int)std::min<int64_t>(kMaxTailParts, items * std::min(l.nb, kMaxTailSplit));
  }
  w.tail_count = off; off = align256(off + kMaxTailItems * sizeof(int32_t));
  w.tail_state = off; off = align256(off + (size_t)w.tail_parts * kTailPartBytes);
  if (a.mode != ATTN_TILEMIX) {
    w.total = off;
    return w;
  }
  w.k_part = off;  off = align256(off + bk * nb * kHeadDim * sizeof(double));
  w.k_mean = off;  off = align256(off + bk * kHeadDim * sizeof(float));
  w.k_codes = off; off = align256(off + bk * nb * (size_t)kTile * kHeadDim);
  w.k_scale = off; off = align256(off + bk * nb * sizeof(float));
  w.k_norm8 = off; off = align256(off + bk * nb * sizeof(float));
  w.q_inv = off;   off = align256(off + bq * nb * sizeof(float));
  w.q_scale = off; off = align256(off + bq * nb * sizeof(float));
  w.total = off;
  return w;
}

RouteRule route_rule(const attn_args& a, const Layout& lay, int64_t* n_int8) {
  RouteRule r;
  const int nb = lay.nb;
  // a block is a text block when it holds any text token
  r.text_blocks = blocks_of(lay.text);
  r.band = a.band_blocks;
  r.seed = a.seed;
  int64_t count = 0;
  if (a.mode != ATTN_TILEMIX) {
    r.kind = kRouteNone;
  } else if (a.pattern == ATTN_PAT_ALL) {
    r.kind = kRouteAll;
    count = (int64_t)nb * nb;
  } else if (a.pattern == ATTN_PAT_ONE) {
    r.kind = kRouteImage;
    const int64_t img = std::max(0, nb - r.text_blocks);
    count = img * img;
  } else if (a.pattern == ATTN_PAT_BAND || a.pattern == ATTN_PAT_SAGE) {
    // the band candidates are the image-image tiles outside the band; the k smallest by
    // (SplitMix64 key, a, b) go INT8, k = floor(percentage * candidates).  The sage
    // pattern keeps that k and draws the k smallest from every tile instead.
    std::vector<std::tuple<uint64_t, int, int>> cand;
    for (int qa = r.text_blocks; qa < nb; ++qa)
      for (int kb = r.text_blocks; kb < nb; ++kb)
        if (std::abs(qa - kb) > a.band_blocks) cand.emplace_back(route_key(a.seed, qa, kb), qa, kb);
    const int64_t k = (int64_t)std::floor(a.percentage * (double)cand.size());
    if (a.pattern == ATTN_PAT_SAGE) {
      cand.clear();
      for (int qa = 0; qa < nb; ++qa)
        for (int kb = 0; kb < nb; ++kb) cand.emplace_back(route_key(a.seed, qa, kb), qa, kb);
    }
    if (k > 0) {
      std::nth_element(cand.begin(), cand.begin() + (k - 1), cand.end());
      r.kind = a.pattern == ATTN_PAT_SAGE ? kRoutePick : kRouteBand;
      r.thr_key = std::get<0>(cand[(size_t)(k - 1)]);
      r.thr_a = std::get<1>(cand[(size_t)(k - 1)]);
      r.thr_b = std::get<2>(cand[(size_t)(k - 1)]);
      count = k;
    } else {
      r.kind = kRouteNone;
    }
  } else {
    r.kind = kRouteNone;  // ATTN_PAT_ZERO: every tile FP16
  }
  if (count == 0) r.kind = kRouteNone;
  if (n_int8) *n_int8 = count;
  return r;
}

std::vector<uint8_t> build_route_map(const attn_args& a, const Layout& lay, int64_t* n_int8) {
  const RouteRule r = route_rule(a, lay, n_int8);
  const int nb = lay.nb;
  std::vector<uint8_t> m((size_t)nb * nb, 0);
  for (int qa = 0; qa < nb; ++qa)
    for (int kb = 0; kb < nb; ++kb) m[(size_t)qa * nb + kb] = route_is_int8(r, qa, kb) ? 1 : 0;
  return m;
}

ScanGeom scan_geom(const attn_args& a, const Layout& lay) {
  ScanGeom g;
  g.text = lay.text;
  g.t_pad = lay.t_pad;
  g.image = lay.image;
  g.cols = lay.cols;
  g.half_window = a.window / 2;
  g.tile_aligned = a.tile_aligned ? 1 : 0;
  return g;
}

std::vector<uint8_t> build_block_mask(const attn_args& a, const Layout& lay) {
  const int nb = lay.nb;
  const ScanGeom g = scan_geom(a, lay);
  std::vector<TileSpan> spans(nb);
  for (int b = 0; b < nb; ++b) spans[b] = tile_span(g, b);
  std::vector<uint8_t> m((size_t)nb * nb, 0);
  for (int qa = 0; qa < nb; ++qa)
    for (int kb = 0; kb < nb; ++kb) m[(size_t)qa * nb + kb] = (uint8_t)scan_tile_class(g, spans[qa], spans[kb]);
  return m;
}

Plan build_plan(const attn_args& a) {
  Plan p;
  p.mode = a.mode;
  p.lay = make_layout(a);
  const int nb = p.lay.nb;
  if (a.mode == ATTN_TILEMIX) {
    p.route_rule = route_rule(a, p.lay, &p.int8_tiles);
    p.active_tiles = (int64_t)nb * nb;
    p.partial_tiles = (p.lay.n % kTile) ? nb : 0;
  } else if (a.mode == ATTN_SCANLINE) {
    p.geom = scan_geom(a, p.lay);
    const std::vector<uint8_t> m = build_block_mask(a, p.lay);
    for (uint8_t v : m) {
      p.active_tiles += v != 0;
      p.partial_tiles += v == 2;
    }
  } else {
    p.active_tiles = (int64_t)nb * nb;
    p.partial_tiles = (p.lay.n % kTile) ? nb : 0;
  }
  return p;
}

std::string plan_key(const attn_args& a) {
  char buf[256];
  const bool tm = a.mode == ATTN_TILEMIX, sc = a.mode == ATTN_SCANLINE;
  std::snprintf(buf, sizeof(buf), "m%d t%d r%d c%d p%d pc%.17g w%d s%llu win%d ta%d",
                a.mode, a.text_tokens, a.img_rows, a.img_cols, tm ? a.pattern : -1,
                tm ? a.percentage : -1.0, tm ? a.band_blocks : -1,
                (unsigned long long)(tm ? a.seed : 0), sc ? a.window : -1,
                sc ? a.tile_aligned : -1);
  return std::string(buf);
}

}  // namespace krea
