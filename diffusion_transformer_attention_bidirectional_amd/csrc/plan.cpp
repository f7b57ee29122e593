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
        a.pattern != ATTN_PAT_ALL) {
      err = "pattern must be ATTN_PAT_ZERO, ATTN_PAT_ONE, ATTN_PAT_BAND or ATTN_PAT_ALL";
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

std::vector<int32_t> scan_item_order(const attn_args& a, const Plan& p, int q_begin, int q_end) {
  const Layout& l = p.lay;
  const int nq = (q_end - q_begin + 63) / 64;
  const int64_t total = attention_items(a, q_end - q_begin);
  std::vector<int32_t> cost(nq, 0);
  for (int qt = 0; qt < nq; ++qt) {
    const int lo = q_begin + 64 * qt, hi = std::min(lo + 64, q_end);
    const bool any = lo < std::min(hi, l.text) || std::max(lo, l.t_pad) < std::min(hi, l.t_pad + l.image);
    const int qa = lo / kTile;
    cost[qt] = any ? p.row_ptr[qa + 1] - p.row_ptr[qa] : 0;
  }
  std::vector<int32_t> order((size_t)total);
  const int64_t per = total / 8, rem = total % 8;
  std::vector<int32_t> range;
  for (int x = 0; x < 8; ++x) {
    const int64_t base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
    const int64_t cnt = x < rem ? per + 1 : per;
    range.resize((size_t)cnt);
    for (int64_t i = 0; i < cnt; ++i) range[(size_t)i] = (int32_t)(base + i);
    std::stable_sort(range.begin(), range.end(),
                     [&](int32_t u, int32_t v) { return cost[u % nq] > cost[v % nq]; });
    for (int64_t i = 0; i < cnt; ++i) order[(size_t)(x + 8 * i)] = range[(size_t)i];
  }
  return order;
}

WorkspaceLayout workspace_layout(const attn_args& a) {
  WorkspaceLayout w;
  const Layout l = make_layout(a);
  const size_t bk = (size_t)a.batch * a.heads_kv, bq = (size_t)a.batch * a.heads_q;
  size_t off = 0;
  w.v_t = off;     off = align256(off + bk * l.nb * (size_t)kTile * kHeadDim * 2);
  w.k_norm = off;  off = align256(off + bk * l.nb * sizeof(float));
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
  w.k_part = off;  off = align256(off + bk * l.nb * kHeadDim * sizeof(double));
  w.k_mean = off;  off = align256(off + bk * kHeadDim * sizeof(float));
  w.k_codes = off; off = align256(off + bk * l.nb * (size_t)kTile * kHeadDim);
  w.k_scale = off; off = align256(off + bk * l.nb * sizeof(float));
  w.k_norm8 = off; off = align256(off + bk * l.nb * sizeof(float));
  w.q_inv = off;   off = align256(off + bq * l.nb * sizeof(float));
  w.q_scale = off; off = align256(off + bq * l.nb * sizeof(float));
  w.total = off;
  return w;
}

uint64_t splitmix64(uint64_t x) {
  // SplitMix64 output function (Steele, Lea and Flood, OOPSLA 2014): advance the
  // state by the golden-ratio increment, then two xor-shift-multiply rounds.
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

std::vector<uint8_t> build_route_map(const attn_args& a, const Layout& lay, int64_t* n_int8) {
  const int nb = lay.nb;
  std::vector<uint8_t> r((size_t)nb * nb, 0);
  int64_t count = 0;
  // a block is a text block when it holds any text token
  const int first_image_block = blocks_of(lay.text);
  if (a.pattern == ATTN_PAT_ALL) {
    std::fill(r.begin(), r.end(), 1);
    count = (int64_t)nb * nb;
  } else if (a.pattern == ATTN_PAT_ONE) {
    for (int qa = first_image_block; qa < nb; ++qa)
      for (int kb = first_image_block; kb < nb; ++kb) { r[(size_t)qa * nb + kb] = 1; ++count; }
  } else if (a.pattern == ATTN_PAT_BAND) {
    std::vector<std::tuple<uint64_t, int, int>> cand;
    for (int qa = first_image_block; qa < nb; ++qa)
      for (int kb = first_image_block; kb < nb; ++kb)
        if (std::abs(qa - kb) > a.band_blocks)
          cand.emplace_back(splitmix64(a.seed ^ (((uint64_t)qa << 32) | (uint64_t)kb)), qa, kb);
    const int64_t k = (int64_t)std::floor(a.percentage * (double)cand.size());
    if (k > 0) {
      std::partial_sort(cand.begin(), cand.begin() + k, cand.end());
      for (int64_t i = 0; i < k; ++i) {
        r[(size_t)std::get<1>(cand[i]) * nb + std::get<2>(cand[i])] = 1;
      }
      count = k;
    }
  }
  if (n_int8) *n_int8 = count;
  return r;
}

// Per logical tile: which kinds of tokens it holds, as intervals.
struct TileSpan {
  int valid = 0;          // valid tokens in the tile
  bool has_text = false;
  bool has_pad = false;
  int row_lo = 0, row_hi = -1;  // image grid rows present (empty if row_hi < row_lo)
};

static TileSpan tile_span(const Layout& l, int blk) {
  TileSpan s;
  const int p0 = blk * kTile, p1 = p0 + kTile;  // [p0, p1)
  // text [0, T)
  const int t0 = std::max(p0, 0), t1 = std::min(p1, l.text);
  if (t1 > t0) { s.has_text = true; s.valid += t1 - t0; }
  // image [t_pad, t_pad + I)
  const int i0 = std::max(p0, l.t_pad), i1 = std::min(p1, l.t_pad + l.image);
  if (i1 > i0) {
    s.valid += i1 - i0;
    s.row_lo = (i0 - l.t_pad) / l.cols;
    s.row_hi = (i1 - 1 - l.t_pad) / l.cols;
  }
  s.has_pad = s.valid < kTile;
  return s;
}

std::vector<uint8_t> build_block_mask(const attn_args& a, const Layout& lay) {
  const int nb = lay.nb, hw = a.window / 2;
  std::vector<TileSpan> spans(nb);
  for (int b = 0; b < nb; ++b) spans[b] = tile_span(lay, b);
  std::vector<uint8_t> m((size_t)nb * nb, 0);
  for (int qa = 0; qa < nb; ++qa) {
    const TileSpan& Q = spans[qa];
    for (int kb = 0; kb < nb; ++kb) {
      const TileSpan& K = spans[kb];
      if (Q.valid == 0 || K.valid == 0) continue;
      const bool q_img = Q.row_hi >= Q.row_lo, k_img = K.row_hi >= K.row_lo;
      // active: a text query, a text key, or two image rows within hw
      bool active = Q.has_text || K.has_text;
      if (!active && q_img && k_img) {
        const int gap = std::max({0, K.row_lo - Q.row_hi, Q.row_lo - K.row_hi});
        active = gap <= hw;
      }
      if (!active) continue;
      bool full = !Q.has_pad && !K.has_pad;
      if (full && !a.tile_aligned && q_img && k_img) {
        // every image-image pair must be within hw
        const int far = std::max(K.row_hi - Q.row_lo, Q.row_hi - K.row_lo);
        full = far <= hw;
      }
      m[(size_t)qa * nb + kb] = full ? 1 : 2;
    }
  }
  return m;
}

Plan build_plan(const attn_args& a) {
  Plan p;
  p.mode = a.mode;
  p.lay = make_layout(a);
  const int nb = p.lay.nb;
  if (a.mode == ATTN_TILEMIX) {
    p.route = build_route_map(a, p.lay, &p.int8_tiles);
    p.active_tiles = (int64_t)nb * nb;
    p.partial_tiles = (p.lay.n % kTile) ? nb : 0;
    if (p.int8_tiles > 0) {
      // key order of each query block: its FP16 full tiles, its INT8 full tiles, then the
      // ragged last block whatever its route (online softmax does not depend on the
      // order; the kernel runs each kind in a loop of its own)
      const int nfull = (p.lay.n % kTile) ? nb - 1 : nb;
      p.full_count.assign(nb, 0);
      p.cols.reserve((size_t)nb * nb);
      for (int qa = 0; qa < nb; ++qa) {
        for (int pass = 0; pass < 2; ++pass)
          for (int kb = 0; kb < nfull; ++kb)
            if ((p.route[(size_t)qa * nb + kb] != 0) == (pass == 1)) {
              p.cols.push_back(kb);
              if (pass == 0) ++p.full_count[qa];
            }
        if (nfull < nb) p.cols.push_back(nb - 1);
      }
    }
  } else if (a.mode == ATTN_SCANLINE) {
    p.bmask = build_block_mask(a, p.lay);
    p.row_ptr.assign(nb + 1, 0);
    p.full_count.assign(nb, 0);
    for (int qa = 0; qa < nb; ++qa) {
      for (int pass = 0; pass < 2; ++pass) {
        for (int kb = 0; kb < nb; ++kb) {
          const uint8_t v = p.bmask[(size_t)qa * nb + kb];
          if (v != (pass == 0 ? 1 : 2)) continue;
          p.cols.push_back(kb | ((v == 2) << 16));
          ++p.active_tiles;
          if (v == 2) ++p.partial_tiles;
          else ++p.full_count[qa];
        }
      }
      p.row_ptr[qa + 1] = (int32_t)p.cols.size();
    }
    const int chunk = a.q_chunk > 0 ? a.q_chunk : p.lay.length;
    for (int q0 = 0; q0 < p.lay.length; q0 += chunk) {
      p.slice_begin.push_back((int32_t)p.item_order.size());
      const std::vector<int32_t> o = scan_item_order(a, p, q0, std::min(p.lay.length, q0 + chunk));
      p.item_order.insert(p.item_order.end(), o.begin(), o.end());
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
  if (sc)  // the scanline launch order depends on the item count of each slice
    std::snprintf(buf + std::strlen(buf), sizeof(buf) - std::strlen(buf), " b%d hq%d qc%d", a.batch, a.heads_q,
                  a.q_chunk);
  return std::string(buf);
}

}  // namespace krea
