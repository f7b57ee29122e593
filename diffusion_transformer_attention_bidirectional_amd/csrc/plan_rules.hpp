// Integer rules of the plan, shared by the host planner (plan.cpp: host views, counts,
// the TileMix pick threshold) and the device plan builder (kernels.hip: the per-call tile
// lists in the workspace), so both evaluate one definition:
//   * the TileMix route of a tile ("Krea 2 TileMix Attention (FP16/INT8 tiles)", "What it
//     actually patches": text tiles and a diagonal band stay FP16, a share of the
//     image-image tiles left over goes to INT8; "The inputs that matter": patterns);
//   * the scanline class of a tile ("Krea 2 Scanline Attention", "What the mask actually
//     is": text global, image rows within window / 2, padding to 128, block mask at 128
//     tiles, tile_aligned);
//   * the scanline launch order (text query tiles, which visit every key tile, first);
//   * the split-tail rule, a function of an item's global position only.
#pragma once

#include <cstdint>

#if defined(__HIP__)
#define KREA_HD __host__ __device__ inline
#else
#define KREA_HD inline
#endif

namespace krea {

// SplitMix64 output function (Steele, Lea and Flood, OOPSLA 2014): advance the state by the
// golden-ratio increment, then two xor-shift-multiply rounds.
KREA_HD uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Rank key of tile (a, b) in the seeded pick.
KREA_HD uint64_t route_key(uint64_t seed, int a, int b) {
  return splitmix64(seed ^ (((uint64_t)(uint32_t)a << 32) | (uint64_t)(uint32_t)b));
}

// How a TileMix call routes its tiles.  kRouteBand: the band-pattern candidates (image-image
// tiles with |a - b| > band) whose (key, a, b) is at most the threshold tuple -- the k-th
// smallest over all candidates, found once on the host -- are INT8: exactly the k smallest.
// kRoutePick: the same threshold test over every tile, text and band included (the
// comparison pattern that quantizes without regard to text, at the band's INT8 budget).
enum { kRouteNone = 0, kRouteAll = 1, kRouteImage = 2, kRouteBand = 3, kRoutePick = 4 };
struct RouteRule {
  int kind = kRouteNone;
  int band = 0;         // band half-width in blocks
  int text_blocks = 0;  // blocks holding a text token: ceil(text / 128)
  uint64_t seed = 0;
  uint64_t thr_key = 0;  // kRouteBand: the k-th smallest candidate tuple
  int thr_a = 0, thr_b = 0;
};

KREA_HD bool route_is_int8(const RouteRule& r, int a, int b) {
  if (r.kind == kRouteAll) return true;
  if (r.kind != kRoutePick) {
    if (r.kind == kRouteNone || a < r.text_blocks || b < r.text_blocks) return false;
    if (r.kind == kRouteImage) return true;
    const int d = a > b ? a - b : b - a;
    if (d <= r.band) return false;
  }
  const uint64_t key = route_key(r.seed, a, b);
  if (key != r.thr_key) return key < r.thr_key;
  return a != r.thr_a ? a < r.thr_a : b <= r.thr_b;
}

// Logical scanline layout: text [0, text), padding to t_pad, the image grid of `image`
// tokens (`cols` per row) from t_pad, tail padding to the 128-token multiple `length`.
struct ScanGeom {
  int text = 0, t_pad = 0, image = 0, cols = 1;
  int half_window = 0;
  int tile_aligned = 0;
};

// What a 128-token logical tile holds.
struct TileSpan {
  int valid = 0;  // valid (non-padding) tokens
  bool has_text = false, has_pad = false;
  int row_lo = 0, row_hi = -1;  // image grid rows present (none when row_hi < row_lo)
};

KREA_HD TileSpan tile_span(const ScanGeom& g, int blk) {
  TileSpan s;
  const int p0 = blk * 128, p1 = p0 + 128;
  const int t0 = p0 > 0 ? p0 : 0, t1 = p1 < g.text ? p1 : g.text;
  if (t1 > t0) {
    s.has_text = true;
    s.valid += t1 - t0;
  }
  const int i0 = p0 > g.t_pad ? p0 : g.t_pad;
  const int i1 = p1 < g.t_pad + g.image ? p1 : g.t_pad + g.image;
  if (i1 > i0) {
    s.valid += i1 - i0;
    s.row_lo = (i0 - g.t_pad) / g.cols;
    s.row_hi = (i1 - 1 - g.t_pad) / g.cols;
  }
  s.has_pad = s.valid < 128;
  return s;
}

// Class of tile (query block a, key block b): 0 skipped, 1 full (every pair admitted, no
// element mask), 2 partial (padding, or the exact row rule cuts through it).
KREA_HD int scan_tile_class(const ScanGeom& g, const TileSpan& Q, const TileSpan& K) {
  if (Q.valid == 0 || K.valid == 0) return 0;
  const bool q_img = Q.row_hi >= Q.row_lo, k_img = K.row_hi >= K.row_lo;
  bool active = Q.has_text || K.has_text;
  if (!active && q_img && k_img) {
    int gap = K.row_lo - Q.row_hi;
    if (Q.row_lo - K.row_hi > gap) gap = Q.row_lo - K.row_hi;
    active = gap <= g.half_window;  // gap <= 0: the row ranges overlap
  }
  if (!active) return 0;
  bool full = !Q.has_pad && !K.has_pad;
  if (full && !g.tile_aligned && q_img && k_img) {
    // without tile alignment every image-image pair must be within the window
    const int far1 = K.row_hi - Q.row_lo, far2 = Q.row_hi - K.row_lo;
    full = (far1 > far2 ? far1 : far2) <= g.half_window;
  }
  return full ? 1 : 2;
}

// The launch-shape rules below run at the start of every attention workgroup, so they use
// 32-bit unsigned arithmetic (a launch has fewer than 2^32 workgroups): 64-bit division is
// a long software sequence on the GPU.
typedef uint32_t u32;

// XCD-contiguous remap: the hardware deals workgroups to the 8 XCDs round robin
// (workgroup L to XCD L % 8); workgroup L = x + 8 i runs the i-th of XCD x's contiguous
// range of the `total` items, so neighbouring items (one KV head's) share an L2.
KREA_HD void xcd_range(u32 total, u32 x, u32* base, u32* cnt) {
  const u32 per = total >> 3, rem = total & 7u;
  *base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  *cnt = x < rem ? per + 1 : per;
}
KREA_HD u32 xcd_item(u32 total, u32 L) {
  u32 base, cnt;
  xcd_range(total, L & 7u, &base, &cnt);
  return base + (L >> 3);
}

// Scanline launch order.  Item t of a launch is query tile t % nq of head group / batch
// t / nq; tiles [0, n_long) of each group hold text queries and visit every key tile, the
// others only their band.  Within each XCD's contiguous range, the text items run first,
// then the others, each kind in item order, so that no long item starts late and leaves a
// tail.  Returns the item workgroup L runs.
KREA_HD u32 scan_item_of(u32 total, u32 nq, u32 n_long, u32 L) {
  u32 base, cnt;
  xcd_range(total, L & 7u, &base, &cnt);
  const u32 idx = L >> 3;
  const u32 n_short = nq - n_long;
  // long items among the first t: whole groups of nq, then the start of a partial group
  const u32 gb = base / nq, rb = base - gb * nq;
  const u32 f0 = gb * n_long + (rb < n_long ? rb : n_long);
  const u32 e = base + cnt, ge = e / nq, re = e - ge * nq;
  const u32 nl = ge * n_long + (re < n_long ? re : n_long) - f0;
  if (idx < nl) {
    const u32 f = f0 + idx;  // global index among long items
    const u32 g = f / n_long;
    return g * nq + (f - g * n_long);
  }
  const u32 s = (base - f0) + (idx - nl);  // global index among short items
  const u32 g = s / n_short;
  return g * nq + n_long + (s - g * n_short);
}

// Split tail.  With one attention workgroup per compute unit, the G items of a whole
// (unsliced) call run in waves of `cus`; the rem = G % cus items of the last, partial wave
// run as `split` workgroups each over consecutive key ranges, their partial softmax states
// merged in part order.  Which items split is a function of the item's global position
// alone: the rem items of highest rank, rank = query tile * J + pair, pair = head group +
// head groups * batch, J = head groups * batch.  So a query row is computed the same way
// whatever the query slicing, and sliced calls give the unsliced call's bits.
struct TailRule {
  int64_t split_from = 0;  // items of rank >= split_from split (none when split == 1)
  int split = 1;
};

// The items of one launch over query tiles [qt_lo, qt_lo + nq) of every pair: per pair j,
// tiles [0, u_j) run whole and [u_j, nq) split, u_j = uA for j < r and uB for j >= r.
struct LaunchSplit {
  u32 J = 1, nq = 0;
  u32 r = 0, uA = 0, uB = 0;
  u32 n_full = 0, n_split = 0;  // whole items, split items
};

KREA_HD int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

KREA_HD LaunchSplit launch_split(const TailRule& t, int64_t J, int64_t qt_lo, int64_t nq) {
  LaunchSplit s;
  s.J = (u32)J;
  s.nq = (u32)nq;
  if (t.split <= 1) {
    s.r = 0;
    s.uA = s.uB = (u32)nq;
  } else {
    // first split tile of pair j: ceil((split_from - j) / J) = P + (j < r), split_from = P J + r
    const int64_t P = t.split_from / J;
    s.r = (u32)(t.split_from % J);
    s.uA = (u32)clamp64(P + 1 - qt_lo, 0, nq);
    s.uB = (u32)clamp64(P - qt_lo, 0, nq);
  }
  s.n_full = s.r * s.uA + (s.J - s.r) * s.uB;
  s.n_split = s.J * s.nq - s.n_full;
  return s;
}

// The i-th whole item of a launch: (query tile within the launch, pair).
KREA_HD void whole_item(const LaunchSplit& s, u32 i, u32* qt, u32* j) {
  const u32 a = s.r * s.uA;
  if (i < a) {
    *j = i / s.uA;
    *qt = i - *j * s.uA;
  } else {
    const u32 i2 = i - a, q = i2 / s.uB;
    *j = s.r + q;
    *qt = i2 - q * s.uB;
  }
}
// The i-th split item of a launch.
KREA_HD void split_item(const LaunchSplit& s, u32 i, u32* qt, u32* j) {
  const u32 sA = s.nq - s.uA, sB = s.nq - s.uB, a = s.r * sA;
  if (i < a) {
    *j = i / sA;
    *qt = s.uA + (i - *j * sA);
  } else {
    const u32 i2 = i - a, q = i2 / sB;
    *j = s.r + q;
    *qt = s.uB + (i2 - q * sB);
  }
}

// What workgroup L of a launch runs: query tile (within the launch), pair, and key-range
// part.  Scanline launches (never split) run each XCD's text query tiles first; the others
// run their whole items in XCD-contiguous ranges, then the parts of their split items,
// also in XCD-contiguous ranges (the parts of one item, and the items of one KV head, on
// one XCD).
struct LaunchItem {
  u32 qt = 0, j = 0;
  int part = 0, nparts = 1, slot = -1;  // slot: index of the item among the split ones
};
KREA_HD LaunchItem launch_item(bool scanline, const LaunchSplit& s, int split, u32 n_long, u32 L) {
  LaunchItem w;
  if (scanline) {
    const u32 t = scan_item_of(s.J * s.nq, s.nq, n_long, L);
    w.j = t / s.nq;
    w.qt = t - w.j * s.nq;
  } else if (L < s.n_full) {
    whole_item(s, xcd_item(s.n_full, L), &w.qt, &w.j);
  } else {
    const u32 t = xcd_item(s.n_split * (u32)split, L - s.n_full);
    w.slot = (int)(t / (u32)split);
    w.part = (int)(t - (u32)w.slot * (u32)split);
    w.nparts = split;
    split_item(s, (u32)w.slot, &w.qt, &w.j);
  }
  return w;
}

}  // namespace krea
