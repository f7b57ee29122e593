// HIP kernels for gfx950 (MI355X): TileMix quantiser, fused joint attention, debug views.
//
// Fused attention ("Krea 2 TileMix Attention (FP16/INT8 tiles)", "What it actually
// patches"): bidirectional online-softmax attention; GQA is resolved in the kernel --
// one workgroup (8 waves) owns 64 query tokens of the 4 query heads that share one KV
// head, each wave 32 queries of one head, so each K/V tile is staged once in LDS and
// read by all eight.  Two waves per SIMD: one wave's softmax overlaps the other's MFMAs.
//
// Per wave, per step of 128 keys (one route / mask block; all matrix products on MFMA
// 32x32 tiles, in four sub-blocks of 32 keys):
//   S^T[key, q] = K Q^T            bf16/f16 MFMA (32x32x16), or i8 MFMA (32x32x32) on
//                                  INT8-routed tiles, int32 accumulate
//   online softmax per query       each lane owns one query column of S^T, so the row
//                                  max and sum stay in the lane (one swap with lane^32)
//   O^T[d, q] += V^T P^T           bf16/f16 MFMA; P^T is the S^T accumulator converted
//                                  in place; V^T comes from per-call V^T tiles that a
//                                  relayout pass writes to the workspace, so every LDS
//                                  fragment read is 16 bytes per lane (8-byte reads,
//                                  transposed or not, run ~3x slower per byte on gfx950)
// K and V^T tiles move HBM -> LDS by DMA (global_load_lds), double buffered.
//
// Hardware facts this file relies on (checked on gfx950):
//   * MFMA 32x32 result: lane l holds column l % 32 and, in register r, row
//     8*(r/4) + 4*(l/32) + r%4 (f32 and i32 results alike);
//   * ds_read_tr16_b64: inside each group of 16 lanes, result lane i receives element
//     i % 4 of the 8 bytes loaded by lanes i/4 + 4k of the group, k = 0..3;
//   * global_load_lds (16 B): lane L writes LDS bytes [base + 16 L, +16), and the
//     instruction counts in vmcnt only (an LDS read issued after it completes without
//     waiting for it).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "kernels.hpp"

namespace krea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kModeDense = 0, kModeTileMix = 1, kModeScan = 2;
constexpr int QT = 64;          // query tokens per workgroup (x 4 heads)
constexpr int KT = 128;         // keys per step = one 128-token route / mask block
constexpr int NWAVE = 8;        // waves per attention workgroup: 4 heads x 2 halves of 32 queries
constexpr int TILE_BYTES = KT * 256;     // one 128 x 128 bf16 tile (32 KB)
constexpr int V_OFF = TILE_BYTES;        // V tile after K in a stage
constexpr int STAGE = 2 * TILE_BYTES;    // bytes of LDS per pipeline stage (64 KB)
constexpr float TAU = 8.0f;     // rescale O only when the running max grows by > 2^8
// Start of the running max (log2 units): finite, below any real score, so a row that has
// seen no admitted key gives exp2(-inf - m) = 0 and the first real block always rescales
// (with alpha = exp2(m - mnew) = 0).
constexpr float kMinRunningMax = -1.0e30f;
// A step of full tiles skips the row max when no score in it can exceed the running max
// by more than tau_skip (log2 units): by Cauchy-Schwarz, scale * q . k <= scale |q| |k|,
// and |k| is bounded per 128-key block by the relayout pass.  Then every probability of the
// step is at most 2^tau_skip, which the P operand of the P V product must hold: bf16 has
// fp32's exponent range (2^24 is far inside it), fp16 stops at 65504 < 2^16, so fp16
// probabilities are kept at or below 2^15.
constexpr float tau_skip(bool bf16) { return bf16 ? 24.0f : 15.0f; }

// Loads of values that stay fixed for a whole launch (plan arrays, the pre-pass and
// quantiser outputs) at wave-uniform addresses, through the constant address space: they
// become scalar loads, counted apart from the vector-memory counter that tracks the K/V
// DMA, so waiting for one of them never waits for a tile in flight.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}
__device__ __forceinline__ int ld_uniform_u8(const uint8_t* p, int64_t i) {
  // bytes through the aligned dword that holds them
  const uint32_t w = ld_uniform((const uint32_t*)((uintptr_t)(p + i) & ~(uintptr_t)3), 0);
  return (int)((w >> (8 * ((uintptr_t)(p + i) & 3))) & 255);
}

// ---------------------------------------------------------------- layout helpers
template <int MODE>
__device__ __forceinline__ bool tok_valid(const AttnParams& p, int t) {
  if (MODE != kModeScan) return t < p.n;
  return t < p.text || (t >= p.t_pad && t < p.t_pad + p.image);
}
template <int MODE>
__device__ __forceinline__ int tok_phys(const AttnParams& p, int t) {
  if (MODE != kModeScan) return t;
  return t < p.text ? t : t - (p.t_pad - p.text);
}
// grid row of a logical image position: floor((t - t_pad) / cols), exact
__device__ __forceinline__ int grid_row(const AttnParams& p, int t) {
  const uint32_t n = (uint32_t)(t - p.t_pad);
  uint32_t q = __umulhi(n, p.cols_magic);
  if ((q + 1) * (uint32_t)p.cols <= n) ++q;
  return (int)q;
}

// Query-side facts a partial tile's element mask needs.
struct QInfo {
  bool valid, text;
  int row;
  int lo, hi;  // scanline image query: the image keys of rows row -+ half_window are [lo, hi)
};
template <int MODE>
__device__ __forceinline__ QInfo query_info(const AttnParams& p, int t) {
  QInfo qi;
  qi.valid = t < p.q_end && tok_valid<MODE>(p, t);
  qi.text = t < p.text;
  qi.row = (MODE == kModeScan && qi.valid && !qi.text) ? grid_row(p, t) : -1;
  const int rows = p.cols > 0 ? p.image / p.cols : 0;
  qi.lo = p.t_pad + max(0, qi.row - p.half_window) * p.cols;
  qi.hi = p.t_pad + (min(rows - 1, qi.row + p.half_window) + 1) * p.cols;
  return qi;
}
// Element mask of a partial tile: key validity, plus the scanline row rule
// ("Krea 2 Scanline Attention", "What the mask actually is").
template <int MODE>
__device__ __forceinline__ bool admit(const AttnParams& p, const QInfo& qi, int j) {
  if (!tok_valid<MODE>(p, j)) return false;
  if (MODE != kModeScan) return true;
  if (!qi.valid) return false;
  if (p.tile_aligned || qi.text || j < p.text) return true;
  // |row(j) - row| <= half_window for a valid image key j, without computing row(j)
  return j >= qi.lo && j < qi.hi;
}

// One step of 128 keys: logical start, whether it needs element masking, and its route.
struct StepInfo {
  int k0;
  bool partial, int8;
};
template <int MODE>
__device__ __forceinline__ StepInfo step_info(const AttnParams& p, int qa, int e0, int i) {
  StepInfo s;
  int kb;
  if (MODE == kModeScan) {
    const int e = ld_uniform(p.cols_list, e0 + i);
    kb = e & 0xffff;
    s.partial = (e >> 16) != 0;
  } else if (MODE == kModeTileMix && p.cols_list != nullptr) {
    kb = ld_uniform(p.cols_list, e0 + i);  // FP16 full tiles, INT8 full tiles, ragged block
  } else {
    kb = i;
  }
  s.k0 = kb * KT;
  if (MODE != kModeScan) s.partial = s.k0 + KT > p.n;
  s.int8 = (MODE == kModeTileMix) && p.route != nullptr && ld_uniform_u8(p.route, (int64_t)qa * p.nb + kb) != 0;
  return s;
}
template <int MODE>
__device__ __forceinline__ int step_count(const AttnParams& p, int qa, int* e0) {
  if (MODE == kModeScan) {
    *e0 = qa * p.nb;
    return ld_uniform(p.row_count, qa);
  }
  *e0 = (MODE == kModeTileMix && p.cols_list != nullptr) ? qa * p.nb : 0;
  return p.nb;
}

// ---------------------------------------------------------------- LDS layouts
// A 128-key tile of K or V (128 x 128 bf16, 32 KB) is stored as 4 slabs, one per group of
// 32 channels, each [128 rows][64 B] (four 16-byte chunks).  Every fragment read then has
// a lane-dependent base and compile-time offsets for the slab, the key block and the step.
//   V: no swizzle -- a transpose-read group touches 4 consecutive rows x 64 B = 256
//      contiguous bytes, all banks once.
//   K: the chunk is XORed with bits 2..3 of the row, so the 16 consecutive rows of a
//      fragment read (same logical chunk) land on 16 distinct 16-byte bank slots.
// INT8 K tile (128 x 128 B): 4 slabs, one per 32-channel k-step, each [128 rows][32 B];
// the chunk is XORed with bit 3 of the row for the same reason.
constexpr int SLAB = 128 * 64;    // bytes per bf16 slab
constexpr int SLAB8 = 128 * 32;   // bytes per INT8 slab
__device__ __forceinline__ int k_swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int k8_swz(int row) { return (row >> 3) & 1; }
// Channel chunk (8 channels) a lane holds in k-step s of the bf16 Q K^T product.  Any
// bijection works if Q and K agree; this one makes two consecutive steps cover 16
// contiguous channels per lane, so the INT8 Q codes built from them line up with the
// natural 16-byte chunks of the INT8 K rows.
__device__ __forceinline__ int qk_chunk(int s, int lh) { return 4 * (s >> 1) + 2 * lh + (s & 1); }
// Byte offset of the K fragment (key block kb of 32 rows, k-step s) for this lane.  Row
// 32 kb + lq has the swizzle of lq (32 kb is a multiple of 16), so each offset is one of
// two per-lane bases (by the parity of s) plus a compile-time constant: the fragment
// reads then use the ds_read immediate offset.
__device__ __forceinline__ int k_lane(int par, int lq, int lh) { return lq * 64 + (((2 * lh + par) ^ k_swz(lq)) << 4); }
__device__ __forceinline__ int k_frag_off(int kb, int s, int lq, int lh) {
  return k_lane(s & 1, lq, lh) + (s >> 1) * SLAB + kb * 2048;
}
// V^T tile in LDS: 4 slabs, one per 32-key sub-block, each [128 channel rows][64 B]: the
// 16-byte chunk 2 k2 + lh of a row holds the 8 keys a P^T B-operand lane holds in k-step
// k2 (keys 16 k2 + 8 (e / 4) + 4 lh + e % 4); swizzled like K (channel row 32 db + lq).
__device__ __forceinline__ int vt_frag_off(int db, int kb, int k2, int lq, int lh) {
  return lq * 64 + (((2 * k2 + lh) ^ k_swz(lq)) << 4) + kb * SLAB + db * 2048;
}
__device__ __forceinline__ int k8_frag_off(int kb, int s, int lq, int lh) {
  return lq * 32 + ((lh ^ k8_swz(lq)) << 4) + s * SLAB8 + kb * 1024;
}

__device__ __forceinline__ lds_void* as_lds(unsigned char* p) { return (lds_void*)p; }

// One DMA instruction HBM -> LDS, 16 bytes per lane to LDS bytes [base + 16 lane, +16),
// base wave-uniform.  Written as inline asm so that the compiler's wait-count model does
// not see it: the model counts an LDS DMA as an LDS event that may complete out of order,
// and while one is outstanding it can only wait for an LDS read with lgkmcnt(0), that is
// for every LDS read in flight, before the first product of each region.  The hardware
// counts the DMA in vmcnt alone.  Every reader of a staged tile runs after an explicit
// s_waitcnt 0 (vmcnt included) and the workgroup barrier.  The instruction writes no
// register, and M0 is declared clobbered.
__device__ __forceinline__ void dma16(const void* src, unsigned char* dst) {
  // the low 32 bits of a generic pointer into LDS are its LDS address
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(base)
               : "memory", "m0");
}

// HBM -> LDS for one step, by DMA; 16 bytes per lane per instruction, 1 KB per
// instruction (16 rows of one slab; 32 rows for INT8); the NW waves of the workgroup
// share the instructions.  K of a full tile is 128 consecutive tokens of the tensor, so
// its addresses are one uniform base per step plus a per-lane 32-bit offset; a partial
// tile clamps padding and out-of-range keys to row 0 (finite data; their probabilities
// are zero).  V^T tiles are contiguous 32 KB blocks of the workspace.  PARTS selects the
// K tile (or its INT8 codes) and / or the V^T tile.
constexpr int kDmaK = 1, kDmaV = 2, kDmaAll = 3;
// Tile kind of a step, when the loop knows it at compile time (TileMix runs its FP16 and
// its INT8 full tiles in loops of their own); a known kind also means a full tile.
constexpr int kStepAny = 0, kStepFp16 = 1, kStepInt8 = 2;
template <int MODE, int NW, int PARTS = kDmaAll, int KIND = kStepAny>
__device__ __forceinline__ void dma_stage(const AttnParams& p, int b, int g, const StepInfo& s,
                                          unsigned char* stage, int wave, int lane) {
  constexpr int PER = (4 * SLAB / 1024) / NW;  // 1 KB blocks per wave per tile
  const int64_t bg = (int64_t)b * p.heads_kv + g;
  const bool s_int8 = KIND == kStepInt8 || (KIND == kStepAny && s.int8);
  const bool s_full = KIND != kStepAny || !s.partial;
  if ((PARTS & 1) && !s_int8) {
    const char* kbase = (const char*)p.k.ptr + ((int64_t)b * p.k.sb + (int64_t)g * p.k.sh) * 2;
    if (s_full) {
      const char* kt = kbase + (int64_t)tok_phys<MODE>(p, s.k0) * p.k.st * 2;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int n = wave * PER + i;
        const int row = (n & 7) * 16 + (lane >> 2);
        const uint32_t off = (uint32_t)row * (uint32_t)(p.k.st * 2) + (4 * (n >> 3) + ((lane & 3) ^ k_swz(row))) * 16;
        dma16(kt + off, stage + n * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int n = wave * PER + i;
        const int row = (n & 7) * 16 + (lane >> 2);
        const int t = s.k0 + row;
        const int ph = tok_valid<MODE>(p, t) ? tok_phys<MODE>(p, t) : 0;
        dma16(kbase + ((int64_t)ph * p.k.st + (4 * (n >> 3) + ((lane & 3) ^ k_swz(row))) * 8) * 2, stage + n * 1024);
      }
    }
  }
  if (PARTS & 2) {
    const char* vt = (const char*)p.v_t + ((bg * p.nb + (s.k0 >> 7)) << 15);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int n = wave * PER + i;
      const int d = (n & 7) * 16 + (lane >> 2);
      const uint32_t off = d * 256 + (4 * (n >> 3) + ((lane & 3) ^ k_swz(d))) * 16;
      dma16(vt + off, stage + V_OFF + n * 1024);
    }
  }
  if ((PARTS & 1) && MODE == kModeTileMix && s_int8) {
    constexpr int PER8 = (4 * SLAB8 / 1024) / NW;
    const int8_t* kc = p.k_codes + (bg * p.nb + (s.k0 >> 7)) * (128 * 128);
#pragma unroll
    for (int i = 0; i < PER8; ++i) {
      const int n = wave * PER8 + i;
      const int slab = n >> 2;
      const int row = (n & 3) * 32 + (lane >> 1);
      const int pc = lane & 1;
      dma16(kc + row * 128 + (2 * slab + (pc ^ k8_swz(row))) * 16, stage + n * 1024);
    }
  }
}

// V^T fragment for 32 channels 32 db .. and the 16 keys of k-step (sub-block kb of 32
// keys, k2), read from a row-major V tile in LDS (4 slabs of [128 keys][64 B], no
// swizzle) by the relayout pass: two transpose reads of 4 keys each, matching
// the key order of the P^T B operand taken from the S^T accumulator (keys
// 32 kb + 16 k2 + 8 half + 4 (l/32) + 0..3).  Source lane s of each 16-lane group reads
// key (s / 4) of its four, channels 32 db + 16 (group & 1) + 4 (s & 3) .. + 3.
__device__ __forceinline__ uint4 v_frag(const unsigned char* vbuf, int db, int kb, int k2, int lane) {
  const int row = 32 * kb + 16 * k2 + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int pc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  unsigned char* base = (unsigned char*)vbuf + db * SLAB + row * 64 + pc * 16 + 8 * (lane & 1);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * 64));
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return make_uint4(l2.x, l2.y, h2.x, h2.y);
}

// ---------------------------------------------------------------- MFMA wrappers
template <bool BF16>
__device__ __forceinline__ f32x16 mma16(uint4 a, uint4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mma16<true>(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mma16<false>(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}
__device__ __forceinline__ i32x16 mma8(uint4 a, uint4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if (BF16) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}
template <bool BF16>
__device__ __forceinline__ float elem_to_f32(uint16_t bits) {
  if (BF16) return __uint_as_float((uint32_t)bits << 16);
  return (float)__builtin_bit_cast(_Float16, bits);
}

// Symmetric INT8 code of one value: clamp(rint(x * inv), -127, 127), the product a
// single correctly rounded fp32 multiply, rint = round half to even.
__device__ __forceinline__ int quant8(float x, float inv) {
  float y = rintf(__fmul_rn(x, inv));
  y = fminf(fmaxf(y, -127.0f), 127.0f);
  return (int)y;
}
template <bool BF16>
__device__ __forceinline__ uint32_t quant4(uint32_t lo2, uint32_t hi2, float inv) {
  const int c0 = quant8(elem_to_f32<BF16>(lo2 & 0xffff), inv);
  const int c1 = quant8(elem_to_f32<BF16>(lo2 >> 16), inv);
  const int c2 = quant8(elem_to_f32<BF16>(hi2 & 0xffff), inv);
  const int c3 = quant8(elem_to_f32<BF16>(hi2 >> 16), inv);
  return (uint32_t)(c0 & 255) | ((uint32_t)(c1 & 255) << 8) | ((uint32_t)(c2 & 255) << 16) |
         ((uint32_t)(c3 & 255) << 24);
}
// INT8 B operand of k-step s' (16 contiguous channels) from the Q fragments of
// bf16 k-steps 2s' and 2s'+1.
template <bool BF16>
__device__ __forceinline__ uint4 make_q8(const uint4& a, const uint4& b, float inv) {
  return make_uint4(quant4<BF16>(a.x, a.y, inv), quant4<BF16>(a.z, a.w, inv), quant4<BF16>(b.x, b.y, inv),
                    quant4<BF16>(b.z, b.w, inv));
}

// Q fragments of one 32-query block: lane (lq, lh) holds query t's channel chunk
// qk_chunk(s, lh) for s = 0..7 (the B operand of K Q^T).
template <int MODE>
__device__ __forceinline__ void load_q_frags(const AttnParams& p, int b, int h, int t, uint4 (&qf)[8]) {
  const int lh = (threadIdx.x & 63) >> 5;
  const bool ok = t < p.q_end && tok_valid<MODE>(p, t);
  const uint16_t* src = (const uint16_t*)p.q.ptr + (int64_t)b * p.q.sb +
                        (int64_t)tok_phys<MODE>(p, ok ? t : 0) * p.q.st + (int64_t)h * p.q.sh;
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = ok ? *(const uint4*)(src + 8 * qk_chunk(s, lh)) : make_uint4(0, 0, 0, 0);
}

// Workgroup -> work item (query tile, head group, batch) and key-range part.  The hardware
// deals workgroups to the 8 XCDs round robin; the remap gives each XCD a contiguous range
// of the whole items, so the workgroups sharing one KV head (and its K/V in that XCD's L2)
// run on the same XCD, and likewise a contiguous range of the split items' parts.  Whole
// and split items follow the call's split rule (a function of each item's global position,
// plan_rules.hpp); scanline never splits and runs each XCD's text query tiles first.
struct WorkItem {
  int qt, hg, b;
  int part, nparts, slot;  // slot: index of the item among the launch's split ones
};
template <int MODE>
__device__ __forceinline__ WorkItem work_item(const AttnParams& p, int n_hg) {
  const LaunchItem li = launch_item(MODE == kModeScan, p.lsplit, p.split, p.n_long, blockIdx.x);
  WorkItem w;
  const u32 bq = li.j / (u32)n_hg;
  w.qt = (int)li.qt;
  w.hg = (int)(li.j - bq * (u32)n_hg);
  w.b = (int)bq;
  w.part = li.part;
  w.nparts = li.nparts;
  w.slot = li.slot;
  return w;
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
// max over the 256 threads of the block (every thread gets the result)
__device__ __forceinline__ float block_max256(float x, float* red) {
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- fused attention
// Partial softmax states of split items: agent-scope (device-coherent) accesses.
__device__ __forceinline__ void tail_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float tail_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-wave state carried across steps.
struct WaveState {
  f32x16 O[4];  // O^T accumulators: 4 channel blocks of 32 x the wave's 32 queries
  float m, l;   // running max (log2 units) and this lane's half of the running sum
};

// Max of a value over the lane pair (l, l ^ 32): one VALU lane swap, no LDS round trip.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Sum of the two probabilities packed in one 32-bit word (bf16 or fp16 pair): the row sum
// uses exactly the rounded values the P V product sees.
template <bool BF16>
__device__ __forceinline__ float pair_sum(uint32_t pk, float acc) {
  if (BF16) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
  } else {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), one, acc, false);
  }
}

// INT8 scores without an int -> float conversion: the int32 accumulation starts from the
// bits of the MFMA inline constant 1 / (2 pi), 0x3E22F983, whose mantissa field
// (2292099) leaves room for every q8 . k8 (|acc| <= 128 * 127^2 < 2^21) inside one binade.
// Read as a float the result is exactly kInt8Base + acc * 2^-26, so the step's score
// scale and offset absorb the affine map (mul * 2^26, add - kInt8Base * mul * 2^26).
constexpr uint32_t kInt8BaseBits = 0x3E22F983u;
constexpr float kInt8Base = __builtin_bit_cast(float, kInt8BaseBits);
constexpr float kInt8Unit = 67108864.0f;  // 2^26

// Raw scores S^T[key, q] of one 32-key sub-block: f32 on FP16 tiles; on INT8 tiles the
// accumulator seeded as above, read as f32 (kInt8Base + acc * 2^-26).
template <bool BF16, bool INT8>
__device__ __forceinline__ f32x16 qk_scores(const unsigned char* __restrict__ buf, int kb, int lq, int lh,
                                            const uint4 (&qf)[8], const uint4 (&q8f)[4]) {
  if (INT8) {
    i32x16 Si;
#pragma unroll
    for (int r = 0; r < 16; ++r) Si[r] = (int)kInt8BaseBits;
#pragma unroll
    for (int s = 0; s < 4; ++s) Si = mma8(*(const uint4*)(buf + k8_frag_off(kb, s, lq, lh)), q8f[s], Si);
    return __builtin_bit_cast(f32x16, Si);
  }
  f32x16 S;
#pragma unroll
  for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) S = mma16<BF16>(*(const uint4*)(buf + k_frag_off(kb, s, lq, lh)), qf[s], S);
  return S;
}
template <bool BF16, int MODE>
__device__ __forceinline__ f32x16 qk_scores_any(const unsigned char* __restrict__ buf, bool int8, int kb, int lq,
                                                int lh, const uint4 (&qf)[8], const uint4 (&q8f)[4]) {
  if (MODE == kModeTileMix && int8) return qk_scores<BF16, true>(buf, kb, lq, lh, qf, q8f);
  return qk_scores<BF16, false>(buf, kb, lq, lh, qf, q8f);
}

// Where the step forms the score minus the running max: TileMix in region A, beside the P V
// products (same-box A/B: 4 MP band 0.6-1.0 % faster, 1 MP band within 0.3 %); dense and
// scanline beside the exponentials in region B (region A measured 0.7-1.0 % slower there).
template <int MODE>
constexpr bool shift_in_a() { return MODE == kModeTileMix; }

// Software pipeline over 32-key sub-blocks.  Sub-block j is handled in two scheduling
// regions, so that every stretch of vector work has independent MFMAs beside it:
//   A: O += V^T P^T of sub-block j - 1 (MFMA)   |  row max of S_j, lazy-rescale decision
//   (rare branch: O *= alpha)
//   B: S_{j+1} = K Q^T (MFMA)                   |  P_j = exp2(S_j), packing, row sums
// The DMA of the next step's tiles into the other stage is issued in region A of the
// first two sub-blocks (K or its INT8 codes, then V^T), so it neither arrives as one burst
// nor sits on the barrier.  At the last sub-block the workgroup barrier sits between A and
// B: every wave's share of the next step has landed, and every wave is done with this
// stage, which receives the step after next while the next step runs.
struct Pipe {
  uint4 P[2];      // P^T of the previous sub-block (two k-steps of 16 keys, packed)
  uint4 vf[2][4];  // V^T fragments of the previous sub-block
};

// P = exp2(S * mul + add - m) of one sub-block, packed as the P^T operand of the P V
// product, and the row sum of exactly those rounded values.  On partial tiles S is already
// masked and scaled; with SHIFTED (shift_in_a) S already holds the log2-domain score minus
// the running max.  The sum runs in two interleaved chains and is pinned to the calling
// region: left alone, the compiler sinks the sums of all four sub-blocks into one
// dependent chain at the end of the step.
template <bool BF16, bool PARTIAL, bool SHIFTED>
__device__ __forceinline__ void probabilities(f32x16& S, float mul, float add, float alpha, Pipe& pp,
                                              WaveState& ws) {
  if (SHIFTED) {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = __builtin_amdgcn_exp2f(S[r]);
  } else if (PARTIAL) {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = __builtin_amdgcn_exp2f(S[r] - ws.m);
  } else {
    const float c = add - ws.m;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = __builtin_amdgcn_exp2f(fmaf(S[r], mul, c));
  }
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int r0 = 8 * k2;
    pp.P[k2] = make_uint4(pack2<BF16>(S[r0], S[r0 + 1]), pack2<BF16>(S[r0 + 2], S[r0 + 3]),
                          pack2<BF16>(S[r0 + 4], S[r0 + 5]), pack2<BF16>(S[r0 + 6], S[r0 + 7]));
  }
  float ls = ws.l * alpha, lb = 0.f;
  ls = pair_sum<BF16>(pp.P[0].x, ls);
  lb = pair_sum<BF16>(pp.P[1].x, lb);
  ls = pair_sum<BF16>(pp.P[0].y, ls);
  lb = pair_sum<BF16>(pp.P[1].y, lb);
  ls = pair_sum<BF16>(pp.P[0].z, ls);
  lb = pair_sum<BF16>(pp.P[1].z, lb);
  ls = pair_sum<BF16>(pp.P[0].w, ls);
  lb = pair_sum<BF16>(pp.P[1].w, lb);
  ls += lb;
  asm volatile("" : "+v"(ls));
  ws.l = ls;
}

template <bool BF16, int MODE, bool PARTIAL, bool LAST, int NEXTK>
__device__ __forceinline__ void sub_block(const AttnParams& p, const unsigned char* __restrict__ buf,
                                          unsigned char* __restrict__ nbuf, int k0, bool int8, const StepInfo& nxt,
                                          bool has_next, int b, int g, int wave, int lane, int kb, float mul,
                                          float add, bool nomax, const uint4 (&qf)[8], const uint4 (&q8f)[4],
                                          const QInfo& qinfo, f32x16& S, f32x16& Sn, Pipe& pp, WaveState& ws) {
  const int lq = lane & 31, lh = lane >> 5;
  // NEXTK known: a next step exists, is a full tile, and is of that kind
  const bool hn = NEXTK != kStepAny || has_next;
  const bool nxt_int8 = NEXTK == kStepInt8 || (NEXTK == kStepAny && nxt.int8);
  // ---- region A
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int db = 0; db < 4; ++db) ws.O[db] = mma16<BF16>(pp.vf[k2][db], pp.P[k2], ws.O[db]);
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int db = 0; db < 4; ++db) pp.vf[k2][db] = *(const uint4*)(buf + V_OFF + vt_frag_off(db, kb, k2, lq, lh));
  if (kb == 0 && hn) dma_stage<MODE, NWAVE, kDmaK, NEXTK>(p, b, g, nxt, nbuf, wave, lane);
  if (kb == 1 && hn) dma_stage<MODE, NWAVE, kDmaV, NEXTK>(p, b, g, nxt, nbuf, wave, lane);
  float alpha = 1.0f;
  bool any_resc = false;
  if (PARTIAL || !nomax) {  // wave-uniform: the row max, unless the step is known to be safe without it
    float mx;
    if (PARTIAL) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = k0 + 32 * kb + 8 * (r >> 2) + 4 * lh + (r & 3);
        S[r] = admit<MODE>(p, qinfo, j) ? fmaf(S[r], mul, add) : -INFINITY;
      }
      mx = S[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
    } else {
      float raw = S[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) raw = fmaxf(raw, S[r]);
      mx = fmaf(raw, mul, add);
    }
    mx = pair_max(mx);
    const float mnew = fmaxf(ws.m, mx);
    const bool resc = mnew > ws.m + TAU;
    alpha = resc ? __builtin_amdgcn_exp2f(ws.m - mnew) : 1.0f;
    if (resc) ws.m = mnew;
    any_resc = __any(resc);
  }
  if (any_resc) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) ws.O[db][r] *= alpha;
  }
  if (shift_in_a<MODE>()) {
    // the log2-domain score minus the running max, here rather than beside the
    // exponentials in region B
    if (PARTIAL) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] -= ws.m;
    } else {
      const float c = add - ws.m;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = fmaf(S[r], mul, c);
    }
  }
  if (LAST) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  __builtin_amdgcn_sched_barrier(0);
  // region B holds the dependent Q K^T chain the next sub-block waits for: while it
  // runs, this wave wins issue arbitration against its SIMD partner
  __builtin_amdgcn_s_setprio(1);
  // ---- region B
  if (MODE == kModeScan && LAST) {
    // each side of the branch gets its own copy of the exponentials, so the product and
    // the vector work share one block the scheduler can interleave (measured: 1.5-1.8 %
    // faster on scanline, 0.8 % slower on dense, which keeps the shared tail)
    if (hn) {
      Sn = qk_scores_any<BF16, MODE>(nbuf, nxt_int8, 0, lq, lh, qf, q8f);
      probabilities<BF16, PARTIAL, shift_in_a<MODE>()>(S, mul, add, alpha, pp, ws);
    } else {
      probabilities<BF16, PARTIAL, shift_in_a<MODE>()>(S, mul, add, alpha, pp, ws);
    }
  } else {
    if (!LAST) Sn = qk_scores_any<BF16, MODE>(buf, int8, kb + 1, lq, lh, qf, q8f);
    else if (hn) Sn = qk_scores_any<BF16, MODE>(nbuf, nxt_int8, 0, lq, lh, qf, q8f);
    probabilities<BF16, PARTIAL, shift_in_a<MODE>()>(S, mul, add, alpha, pp, ws);
  }
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// One step of 128 keys (four sub-blocks) on stage `buf`, while the next step's tiles are
// loaded into `nbuf`.  On entry S0 holds the raw scores of this step's first sub-block; on
// exit it holds those of the next step's first sub-block.  The two stages are separate
// restrict-qualified pointers so the compiler knows the DMA cannot alias the reads.
template <bool BF16, int MODE, bool PARTIAL, int KIND = kStepAny, int NEXTK = kStepAny>
__device__ __forceinline__ void attn_step(const AttnParams& p, const unsigned char* __restrict__ buf,
                                          unsigned char* __restrict__ nbuf, const StepInfo& cur,
                                          const StepInfo& nxt, bool has_next, int b, int g, int wave, int lane,
                                          const uint4 (&qf)[8], const uint4 (&q8f)[4], const QInfo& qinfo,
                                          float qadd, float sq_l2, bool nomax, f32x16& S0, f32x16& S1, Pipe& pp,
                                          WaveState& ws) {
  const bool int8 = KIND == kStepInt8 || (KIND == kStepAny && MODE == kModeTileMix && cur.int8);
  // log2-domain score = S * mul + add (INT8: acc * sq_l2 * k_scale + qadd, through the seeded
  // accumulator's affine map)
  const float mul =
      int8 ? sq_l2 * ld_uniform(p.k_scale, ((int64_t)b * p.heads_kv + g) * p.nb + (cur.k0 >> 7)) * kInt8Unit
           : p.scale_log2;
  const float add = int8 ? qadd - kInt8Base * mul : 0.f;
  const int k0 = cur.k0;
  sub_block<BF16, MODE, PARTIAL, false, NEXTK>(p, buf, nbuf, k0, int8, nxt, has_next, b, g, wave, lane, 0, mul,
                                               add, nomax, qf, q8f, qinfo, S0, S1, pp, ws);
  sub_block<BF16, MODE, PARTIAL, false, NEXTK>(p, buf, nbuf, k0, int8, nxt, has_next, b, g, wave, lane, 1, mul,
                                               add, nomax, qf, q8f, qinfo, S1, S0, pp, ws);
  sub_block<BF16, MODE, PARTIAL, false, NEXTK>(p, buf, nbuf, k0, int8, nxt, has_next, b, g, wave, lane, 2, mul,
                                               add, nomax, qf, q8f, qinfo, S0, S1, pp, ws);
  sub_block<BF16, MODE, PARTIAL, true, NEXTK>(p, buf, nbuf, k0, int8, nxt, has_next, b, g, wave, lane, 3, mul,
                                              add, nomax, qf, q8f, qinfo, S1, S0, pp, ws);
}

// One full-tile step of the key loop: the max-skip test, the step, and the rotation of the
// step descriptors.  KIND: the tile kind when the loop knows it.
template <bool BF16, int MODE, int KIND, int NEXTK = kStepAny>
__device__ __forceinline__ void full_step(const AttnParams& p, int i, int s0, int s1, unsigned char* st0,
                                          unsigned char* st1, int qa, int e0, int b, int g, int wave, int lane,
                                          const uint4 (&qf)[8], const uint4 (&q8f)[4], const QInfo& qinfo, float qadd,
                                          float sq_l2, float qn, float qn8, const float* knorm, StepInfo& cur,
                                          StepInfo& nxt, f32x16& S0, f32x16& S1, Pipe& pp, WaveState& ws) {
  const bool has_next = i + 1 < s1;
  const StepInfo nxt2 = i + 2 < s1 ? step_info<MODE>(p, qa, e0, i + 2) : nxt;  // read a step ahead
  unsigned char* sa = ((i - s0) & 1) ? st1 : st0;
  unsigned char* sb = ((i - s0) & 1) ? st0 : st1;
  const bool int8 = KIND == kStepInt8 || (KIND == kStepAny && MODE == kModeTileMix && cur.int8);
  bool nomax;
  if (int8) {
    // |q8 . k8| <= |q8| |k8| (exact integers), so the score is at most this bound
    const int64_t tile = ((int64_t)b * p.heads_kv + g) * p.nb + (cur.k0 >> 7);
    nomax = __all(qn8 * ld_uniform(p.k_norm8, tile) * ld_uniform(p.k_scale, tile) + qadd <= ws.m + tau_skip(BF16));
  } else {
    nomax = __all(qn * ld_uniform(knorm, cur.k0 >> 7) <= ws.m + tau_skip(BF16));
  }
  attn_step<BF16, MODE, false, KIND, NEXTK>(p, sa, sb, cur, nxt, has_next, b, g, wave, lane, qf, q8f, qinfo, qadd,
                                            sq_l2, nomax, S0, S1, pp, ws);
  cur = nxt;
  nxt = nxt2;
}

template <bool BF16, int MODE>
__global__ void __launch_bounds__(512) attn_fwd_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const WorkItem wi = work_item<MODE>(p, p.heads_q / 4);
  const int qt = wi.qt, hg = wi.hg, b = wi.b;
  const int h = hg * 4 + (wave & 3);
  const int g = (hg * 4) / p.group;
  const int q0 = p.q_begin + qt * QT;
  const int qa = q0 >> 7;
  {
    // skip tiles holding no valid query (scanline text padding); uniform per workgroup
    const int lo = q0, hi = min(q0 + QT, p.q_end);
    const bool any = (MODE != kModeScan) ? lo < min(hi, p.n)
                                         : (lo < min(hi, p.text)) || (max(lo, p.t_pad) < min(hi, p.t_pad + p.image));
    if (!any) return;
  }
  const int tq = q0 + 32 * (wave >> 2) + lq;  // this lane's query (logical position)

  uint4 qf[8];
  load_q_frags<MODE>(p, b, h, tq, qf);
  const QInfo qinfo = query_info<MODE>(p, tq);
  // scale_log2 |q| (rounded up): this lane holds half of its query's channels
  float qn;
  {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t w[4] = {qf[s].x, qf[s].y, qf[s].z, qf[s].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = elem_to_f32<BF16>(w[e] & 0xffff), x1 = elem_to_f32<BF16>(w[e] >> 16);
        ss = fmaf(x0, x0, ss);
        ss = fmaf(x1, x1, ss);
      }
    }
    ss += __shfl_xor(ss, 32);
    qn = __builtin_sqrtf(ss) * p.scale_log2 * 1.001f;
  }

  // TileMix: INT8 codes of this query block, and the smooth_k row term.  Raw K is used on
  // FP16 tiles and mean-centred codes on INT8 tiles; adding scale * q . mean to every INT8
  // score puts both on the same per-row offset, which softmax ignores (smooth_k is exact
  // for softmax, "The inputs that matter").
  uint4 q8f[4];
  float qadd = 0.f, sq_l2 = 0.f;
  float qn8 = 0.f;  // sq_l2 |q8| (rounded up): the INT8 counterpart of qn
  if (MODE == kModeTileMix && p.route != nullptr) {
    // INT8 scale of this query tile (the 128 tokens of head h in block qa), computed here:
    // this wave's 32 queries are in registers, the 32 rows at the same place in the tile's
    // other 64-token half are read, and the head's two waves combine through LDS
    __shared__ float qabs[NWAVE];
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t w[4] = {qf[s].x, qf[s].y, qf[s].z, qf[s].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a = fmaxf(a, fabsf(elem_to_f32<BF16>(w[e] & 0xffff)));
        a = fmaxf(a, fabsf(elem_to_f32<BF16>(w[e] >> 16)));
      }
    }
    const int t_other = (q0 ^ 64) + 32 * (wave >> 2) + lq;
    if (t_other < p.n) {
      const uint16_t* src =
          (const uint16_t*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)t_other * p.q.st + (int64_t)h * p.q.sh + 64 * lh;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 x = *(const uint4*)(src + 8 * c);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a = fmaxf(a, fabsf(elem_to_f32<BF16>(w[e] & 0xffff)));
          a = fmaxf(a, fabsf(elem_to_f32<BF16>(w[e] >> 16)));
        }
      }
    }
    a = wave_max(a);
    if (lane == 0) qabs[wave] = a;
    __syncthreads();
    a = fmaxf(qabs[wave & 3], qabs[(wave & 3) + 4]);
    const float inv = a > 0.f ? __fdiv_rn(127.0f, a) : 0.f;
    sq_l2 = p.scale_log2 * (a > 0.f ? __fdiv_rn(a, 127.0f) : 0.f);
#pragma unroll
    for (int s = 0; s < 4; ++s) q8f[s] = make_q8<BF16>(qf[2 * s], qf[2 * s + 1], inv);
    int ss = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w[4] = {q8f[s].x, q8f[s].y, q8f[s].z, q8f[s].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int c = (int)(int8_t)(w[e] >> (8 * k));
          ss += c * c;
        }
    }
    ss += __shfl_xor(ss, 32);
    qn8 = __builtin_sqrtf((float)ss) * sq_l2 * 1.001f;
    if (p.smooth_k) {
      const float* mean = p.k_mean + ((int64_t)b * p.heads_kv + g) * 128;
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 x = qf[s];
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        const float* mc = mean + 8 * qk_chunk(s, lh);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t bits = (e & 1) ? (uint16_t)(w[e >> 1] >> 16) : (uint16_t)(w[e >> 1] & 0xffff);
          acc = fmaf(elem_to_f32<BF16>(bits), mc[e], acc);
        }
      }
      acc += __shfl_xor(acc, 32);
      qadd = p.scale_log2 * acc;
    }
  }

  int e0;
  const int nsteps = step_count<MODE>(p, qa, &e0);
  // key steps [s0, s1) of this part (all of them unless the item is split)
  const int s0 = (int)((int64_t)wi.part * nsteps / wi.nparts);
  const int s1 = (int)((int64_t)(wi.part + 1) * nsteps / wi.nparts);
  WaveState ws;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) ws.O[db][r] = 0.f;
  ws.m = kMinRunningMax;
  ws.l = 0.f;

  if (s1 > s0) {
    unsigned char* st0 = lds;
    unsigned char* st1 = lds + STAGE;
    StepInfo cur = step_info<MODE>(p, qa, e0, s0);
    StepInfo nxt = s0 + 1 < s1 ? step_info<MODE>(p, qa, e0, s0 + 1) : cur;
    dma_stage<MODE, NWAVE>(p, b, g, cur, st0, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    Pipe pp;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      pp.P[k2] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int db = 0; db < 4; ++db) pp.vf[k2][db] = make_uint4(0, 0, 0, 0);
    }
    f32x16 S0 = qk_scores_any<BF16, MODE>(st0, cur.int8, 0, lq, lh, qf, q8f), S1;
    // full tiles first, then the partial ones (padding, ragged tail, exact scanline
    // rule) with the element mask: two loops, so the lean one keeps its registers
    const int nfull = MODE == kModeScan ? ld_uniform(p.full_count, qa) : (p.n % KT ? nsteps - 1 : nsteps);
    const int f1 = min(s1, nfull);
    const float* knorm = p.k_norm + ((int64_t)b * p.heads_kv + g) * p.nb;
    if (MODE == kModeTileMix) {
      // FP16 full tiles first, then INT8 full tiles (all FP16 without INT8 tiles), each in a
      // loop that knows the kind, so no step of it branches on the route (measured: 1 MP
      // band -2.8 %, 4 MP band -2.9 % against one loop over the tiles in key order)
      const int nf16 = p.cols_list != nullptr ? ld_uniform(p.full_count, qa) : nfull;
      // within each run, every step but the last has a next step of the same kind
      int i = s0;
      const int e16 = min(f1, nf16);
      for (; i + 1 < e16; ++i)
        full_step<BF16, MODE, kStepFp16, kStepFp16>(p, i, s0, s1, st0, st1, qa, e0, b, g, wave, lane, qf, q8f, qinfo,
                                                    qadd, sq_l2, qn, qn8, knorm, cur, nxt, S0, S1, pp, ws);
      for (; i < e16; ++i)
        full_step<BF16, MODE, kStepFp16>(p, i, s0, s1, st0, st1, qa, e0, b, g, wave, lane, qf, q8f, qinfo, qadd, sq_l2,
                                         qn, qn8, knorm, cur, nxt, S0, S1, pp, ws);
      for (; i + 1 < f1; ++i)
        full_step<BF16, MODE, kStepInt8, kStepInt8>(p, i, s0, s1, st0, st1, qa, e0, b, g, wave, lane, qf, q8f, qinfo,
                                                    qadd, sq_l2, qn, qn8, knorm, cur, nxt, S0, S1, pp, ws);
      for (; i < f1; ++i)
        full_step<BF16, MODE, kStepInt8>(p, i, s0, s1, st0, st1, qa, e0, b, g, wave, lane, qf, q8f, qinfo, qadd, sq_l2,
                                         qn, qn8, knorm, cur, nxt, S0, S1, pp, ws);
    } else {
      for (int i = s0; i < f1; ++i)
        full_step<BF16, MODE, kStepAny>(p, i, s0, s1, st0, st1, qa, e0, b, g, wave, lane, qf, q8f, qinfo, qadd, sq_l2,
                                        qn, qn8, knorm, cur, nxt, S0, S1, pp, ws);
    }
    for (int i = max(s0, nfull); i < s1; ++i) {
      const bool has_next = i + 1 < s1;
      const StepInfo nxt2 = i + 2 < s1 ? step_info<MODE>(p, qa, e0, i + 2) : nxt;  // read a step ahead
      attn_step<BF16, MODE, true>(p, ((i - s0) & 1) ? st1 : st0, ((i - s0) & 1) ? st0 : st1, cur, nxt,
                                      has_next, b, g, wave, lane, qf, q8f, qinfo, qadd, sq_l2, false, S0, S1, pp, ws);
      cur = nxt;
      nxt = nxt2;
    }
    // the last sub-block's P V
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int db = 0; db < 4; ++db) ws.O[db] = mma16<BF16>(pp.vf[k2][db], pp.P[k2], ws.O[db]);
  }

  if (MODE != kModeScan && wi.nparts > 1) {
    // Split item: publish this part's state (O^T, running max, running sum per lane),
    // count the parts that are done, and let the last one merge every part and write O.
    // The states move through agent-scope atomic stores and loads, which write through
    // and bypass the per-XCD L2 caches, so publishing needs only the stores' completion
    // (no write-back of the L2, which costs tens of microseconds per fence).
    __shared__ int last_part;
    float* mine = p.tail_state + ((size_t)(wi.slot * wi.nparts + wi.part) * 8 + wave) * (66 * 64) + lane;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) tail_store(mine + (db * 16 + r) * 64, ws.O[db][r]);
    tail_store(mine + 64 * 64, ws.m);
    tail_store(mine + 65 * 64, ws.l);
    __builtin_amdgcn_s_waitcnt(0);  // the write-through stores have completed
    __syncthreads();
    if (tid == 0)
      last_part = __hip_atomic_fetch_add(&p.tail_count[wi.slot], 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) ==
                  wi.nparts - 1;
    __syncthreads();
    if (!last_part) return;
    // merge every part from memory in part order, so the result does not depend on
    // which part finished last
    const float* base = p.tail_state + ((size_t)(wi.slot * wi.nparts) * 8 + wave) * (66 * 64) + lane;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) ws.O[db][r] = tail_load(base + (db * 16 + r) * 64);
    ws.m = tail_load(base + 64 * 64);
    ws.l = tail_load(base + 65 * 64);
    for (int q = 1; q < wi.nparts; ++q) {
      const float* other = base + (size_t)q * 8 * (66 * 64);
      const float mo = tail_load(other + 64 * 64), lo = tail_load(other + 65 * 64);
      const float mn = fmaxf(ws.m, mo);
      const float a = __builtin_amdgcn_exp2f(ws.m - mn), c = __builtin_amdgcn_exp2f(mo - mn);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ws.O[db][r] = ws.O[db][r] * a + tail_load(other + (db * 16 + r) * 64) * c;
      ws.l = ws.l * a + lo * c;
      ws.m = mn;
    }
    if (tid == 0) p.tail_count[wi.slot] = 0;  // ready for the next launch
  }

  // ---- epilogue: O = O^T / l, rows of valid queries only (padding is never written); with
  // a gate, O * sigmoid(gate) ("LayerStream: Krea2 Chunking", "What the node does to the
  // block": the attention gate is applied before the output projection), in fp32 before
  // the one rounding to the output dtype
  const float lt = ws.l + __shfl_xor(ws.l, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qinfo.valid) {
    const int64_t tp = tok_phys<MODE>(p, tq);
    uint16_t* dst = (uint16_t*)p.o + (int64_t)b * p.o_sb + tp * p.o_st + (int64_t)h * p.o_sh;
    const uint16_t* gsrc = p.gate == nullptr ? nullptr
                                             : (const uint16_t*)p.gate + (int64_t)b * p.g_sb + tp * p.g_st +
                                                   (int64_t)h * p.g_sh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const f32x16& o = ws.O[db];
        float f[4] = {o[4 * grp] * inv, o[4 * grp + 1] * inv, o[4 * grp + 2] * inv, o[4 * grp + 3] * inv};
        if (gsrc != nullptr) {
          const uint2 gv = *(const uint2*)(gsrc + 32 * db + 8 * grp + 4 * lh);
          const uint32_t gw[2] = {gv.x, gv.y};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gx = elem_to_f32<BF16>((uint16_t)(gw[e >> 1] >> (16 * (e & 1))));
            // sigmoid(g) = 1 / (1 + 2^(-g log2 e)); 2^(+large) = inf gives 0, 2^(-large) = 0 gives 1
            f[e] *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gx * 1.4426950408889634f));
          }
        }
        const uint2 val = make_uint2(pack2<BF16>(f[0], f[1]), pack2<BF16>(f[2], f[3]));
        *(uint2*)(dst + 32 * db + 8 * grp + 4 * lh) = val;
      }
  }
}

// ---------------------------------------------------------------- device plan
// The per-call plan, built in the workspace from the call's scalars by the rules of
// plan_rules.hpp (the host planner evaluates the same ones): for query block a, the key
// blocks the attention kernel visits, in the order it visits them, at lists[a * nb ..].
//   TileMix ("Krea 2 TileMix Attention (FP16/INT8 tiles)", "What it actually patches"):
//     the route of every tile into map; the FP16 full tiles, then the INT8 full tiles, each
//     in key order, then the ragged last block; full_count[a] = the FP16 full tiles.
//   Scanline ("Krea 2 Scanline Attention", "What the mask actually is"): the class of every
//     tile (0 skip, 1 full, 2 partial) into map; the full tiles, then the partial ones
//     (entry | 1 << 16), each in key order; row_count[a] entries, full_count[a] full.

// Appends, in thread order, the values of the threads with `sel` to out[base ..] (256
// threads, all calling); returns the new end.  sh: 4 ints of LDS.
__device__ __forceinline__ int emit_ordered(bool sel, int value, int32_t* out, int base, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(sel);
  const int before = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) sh[wave] = __popcll(m);
  __syncthreads();
  int off = base;
  for (int w = 0; w < wave; ++w) off += sh[w];
  const int total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  if (sel) out[off + before] = value;
  return base + total;
}

// Row a of the plan, by one workgroup of 256 threads.
__device__ void build_plan_row(const PlanBuild& pb, int a, int* sh) {
  const int nb = pb.nb, tid = threadIdx.x;
  uint8_t* map = pb.map + (int64_t)a * nb;
  int32_t* list = pb.lists + (int64_t)a * nb;
  int end = 0, nfirst = 0;
  if (pb.mode == kModeTileMix) {
    const int nfull = (pb.n % KT) ? nb - 1 : nb;
    for (int pass = 0; pass < 2; ++pass) {
      for (int b0 = 0; b0 < nfull; b0 += 256) {
        const int b = b0 + tid;
        bool sel = false;
        if (b < nfull) {
          const bool i8 = route_is_int8(pb.route, a, b);
          if (pass == 0) map[b] = i8 ? 1 : 0;
          sel = i8 == (pass == 1);
        }
        end = emit_ordered(sel, b, list, end, sh);
      }
      if (pass == 0) nfirst = end;
    }
    if (nfull < nb && tid == 0) {
      map[nb - 1] = route_is_int8(pb.route, a, nb - 1) ? 1 : 0;
      list[end] = nb - 1;
    }
    end = nb;
  } else {
    const TileSpan qs = tile_span(pb.geom, a);
    for (int pass = 0; pass < 2; ++pass) {
      for (int b0 = 0; b0 < nb; b0 += 256) {
        const int b = b0 + tid;
        bool sel = false;
        if (b < nb) {
          const int cls = scan_tile_class(pb.geom, qs, tile_span(pb.geom, b));
          if (pass == 0) map[b] = (uint8_t)cls;
          sel = cls == pass + 1;
        }
        end = emit_ordered(sel, pass == 0 ? b : (b | (1 << 16)), list, end, sh);
      }
      if (pass == 0) nfirst = end;
    }
  }
  if (tid == 0) {
    pb.row_count[a] = end;
    pb.full_count[a] = nfirst;
  }
}

// The plan alone (debug views): one workgroup per query block.
__global__ void __launch_bounds__(256) plan_kernel(const PlanBuild pb) {
  __shared__ int sh[4];
  build_plan_row(pb, blockIdx.x, sh);
}

// ---------------------------------------------------------------- per-block pre-pass
// Everything the attention kernel needs from one 128-key block, in one pass over the
// tensors.  One workgroup of 256 threads per (key block kb, KV head g, batch b):
//   * V^T tiles [B, Hkv, nb, 128 channels, 128 keys] (when v_t is given): logical key order
//     (scanline padding is zero), keys of each 16-key group in P^T order.  The tile goes
//     through LDS row-major and comes back through transpose reads as exactly the
//     fragments the attention kernel reads;
//   * the bound on |k| over the block's keys (when p.k_norm is given);
//   * with pb (TileMix with INT8 tiles, scanline), row kb of the call's plan;
//   * QUANT, the TileMix quantiser inputs ("Krea 2 TileMix Attention (FP16/INT8 tiles)",
//     "The inputs that matter"): the fp64 column sums of K over the block's tokens, added in
//     token order (smooth_k), and with QSCALE the INT8 scale of query tile kb of every query
//     head that KV head g serves (a = max |q| over the tile, inv = fp32(127 / a),
//     scale = fp32(a / 127)); the attention kernel derives the same scales itself.
template <bool BF16, int MODE, bool QUANT, bool QSCALE>
__global__ void __launch_bounds__(256) prepass_kernel(const AttnParams p, uint16_t* v_t, const QuantParams qp,
                                                      const PlanBuild pb) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * SLAB];              // V tile, slab layout
  __shared__ __attribute__((aligned(1024))) unsigned char klds[QUANT ? KT * 256 : 16];  // K tile, row-major
  __shared__ float kmax[4];
  const int kb = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, lq = lane & 31, lh = lane >> 5, wave = tid >> 6;
  const int64_t bg = (int64_t)b * p.heads_kv + g;
  // Every load of the block goes out first, so the pass waits for memory once: thread
  // tid takes the 16-byte chunk c = id % 16 of row id / 16 of both tiles, id = tid + 256 i
  // (the 16 chunks of a row are 16 consecutive lanes of one wave).
  const bool need_k = p.k_norm != nullptr || (QUANT && qp.smooth_k);
  uint4 kx[8], vx[8];
  const uint16_t* kbase = (const uint16_t*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)g * p.k.sh;
  const uint16_t* vbase = (const uint16_t*)p.v.ptr + (int64_t)b * p.v.sb + (int64_t)g * p.v.sh;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int id = tid + 256 * i;
    const int row = id >> 4, c = id & 15;
    const int t = kb * KT + row;
    const bool valid = tok_valid<MODE>(p, t);
    const int64_t ph = valid ? tok_phys<MODE>(p, t) : 0;
    kx[i] = need_k && valid ? *(const uint4*)(kbase + ph * p.k.st + c * 8) : make_uint4(0, 0, 0, 0);
    vx[i] = v_t != nullptr && valid ? *(const uint4*)(vbase + ph * p.v.st + c * 8) : make_uint4(0, 0, 0, 0);
  }
  // the attention launches that follow start from zero tail counters
  if (p.tail_count != nullptr && kb == 0 && g == 0 && b == 0) p.tail_count[tid] = 0;  // 256 counters
  if (v_t != nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 4, c = id & 15;
      *(uint4*)(lds + (c >> 2) * SLAB + row * 64 + (c & 3) * 16) = vx[i];
    }
  }
  if (QUANT && qp.smooth_k) {
    // rows past n are zero, so they add nothing to the column sums
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = tid + 256 * i;
      *(uint4*)(klds + (id >> 4) * 256 + (id & 15) * 16) = kx[i];
    }
  }
  if (p.k_norm != nullptr) {
    // largest |k| over the block's keys, rounded up: each row's squared norm is summed over
    // its 16 lanes, then the maximum taken over rows
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w[4] = {kx[i].x, kx[i].y, kx[i].z, kx[i].w};
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = elem_to_f32<BF16>(w[e] & 0xffff), x1 = elem_to_f32<BF16>(w[e] >> 16);
        ss = fmaf(x0, x0, ss);
        ss = fmaf(x1, x1, ss);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o);
      mx = fmaxf(mx, ss);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (lane == 0) kmax[wave] = mx;
  }
  __syncthreads();
  if (p.k_norm != nullptr && tid == 0)
    p.k_norm[bg * p.nb + kb] = __builtin_sqrtf(fmaxf(fmaxf(kmax[0], kmax[1]), fmaxf(kmax[2], kmax[3]))) * 1.001f;
  if (v_t != nullptr) {
    const int db = tid >> 6;
    uint16_t* dst = v_t + ((bg * p.nb + kb) * 128 + 32 * db + lq) * 128;
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        *(uint4*)(dst + (4 * kb2 + 2 * k2 + lh) * 8) = v_frag(lds, db, kb2, k2, lane);
  }
  if (QUANT) {
    // TileMix layouts are unpadded: token t of the block is row t of the tensors, valid
    // when t < n.  smooth_k: one thread per channel adds the block's tokens in order.
    if (qp.smooth_k && tid < 128) {
      const int rows = min(KT, qp.n - kb * KT);
      double acc = 0.0;
#pragma unroll 16
      for (int r = 0; r < rows; ++r)
        acc = __dadd_rn(acc, (double)elem_to_f32<BF16>(*(const uint16_t*)(klds + r * 256 + tid * 2)));
      qp.k_part[(bg * qp.nb + kb) * 128 + tid] = acc;
    }
    // Q tile scales (the attention kernel computes its own): wave w takes the query heads
    // w, w + 4, ... of this KV head
    const int group = QSCALE ? qp.heads_q / qp.heads_kv : 0;
    for (int hh = wave; hh < group; hh += 4) {
      const int h = g * group + hh;
      const uint16_t* src = (const uint16_t*)qp.q.ptr + (int64_t)b * qp.q.sb + (int64_t)h * qp.q.sh + (lane & 15) * 8;
      float a = 0.f;
#pragma unroll 8
      for (int i = 0; i < 32; ++i) {
        const int t = kb * KT + (lane >> 4) + 4 * i;
        if (t < qp.n) {
          const uint4 x = *(const uint4*)(src + (int64_t)t * qp.q.st);
          const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a = fmaxf(a, fabsf(elem_to_f32<BF16>(w[e] & 0xffff)));
            a = fmaxf(a, fabsf(elem_to_f32<BF16>(w[e] >> 16)));
          }
        }
      }
      a = wave_max(a);
      if (lane == 0) {
        const int64_t idx = ((int64_t)b * qp.heads_q + h) * qp.nb + kb;
        qp.q_inv[idx] = a > 0.f ? __fdiv_rn(127.0f, a) : 0.f;
        qp.q_scale[idx] = a > 0.f ? __fdiv_rn(a, 127.0f) : 0.f;
      }
    }
  }
  // the plan: row kb, by the workgroups of the first KV head of the first sample
  if (pb.lists != nullptr && g == 0 && b == 0) {
    __shared__ int sh[4];
    build_plan_row(pb, kb, sh);
  }
}

// ---------------------------------------------------------------- quantiser
// TileMix INT8 stage ("Krea 2 TileMix Attention (FP16/INT8 tiles)", "The inputs that
// matter": smooth_k mean-centres K per head before quantisation).  Reproducible rule:
// fp64 column sums of K, tokens of each 128-block added in order (pre-pass) then the block
// sums in order; m = fp32(sum / N); K_s = fp32(K) - m; per 128-token x 128-channel tile over
// valid rows a = max |x|, inv = fp32(127 / a), scale = fp32(a / 127),
// code = clamp(rint(x * inv), -127, 127).

// smooth_k mean per (batch, KV head, channel) from the pre-pass's block partials: fp64 adds
// in block order, then one division by N rounded to fp32.  One thread per channel.
__device__ __forceinline__ float k_mean_of(const QuantParams& p, int64_t bg, int c) {
  if (!p.smooth_k) return 0.f;
  double tot = 0.0;
#pragma unroll 16
  for (int j = 0; j < p.nb; ++j) tot = __dadd_rn(tot, p.k_part[(bg * p.nb + j) * 128 + c]);
  return __double2float_rn(__ddiv_rn(tot, (double)p.n));
}

// The mean on its own: one workgroup per (KV head, batch), for long sequences, where the
// serial sum would hold up every quantiser workgroup.
__global__ void __launch_bounds__(128) k_mean_kernel(const QuantParams p) {
  const int64_t bg = (int64_t)blockIdx.y * p.heads_kv + blockIdx.x;
  p.k_mean[bg * 128 + threadIdx.x] = k_mean_of(p, bg, threadIdx.x);
}

// Heads of at most this many 128-token blocks have their mean summed by the quantiser
// itself (measured: a separate mean kernel costs 4-5 us of launch and latency at 36 blocks;
// at 132 blocks the sum in every quantiser workgroup costs 7 us more than that kernel).
constexpr int kFuseMeanMaxBlocks = 64;

// K codes: one workgroup per (batch, KV head, 128-token block).  FUSED_MEAN: every
// workgroup of a head sums the smooth_k mean itself (the same adds in the same order, so
// they all get the same value) while its tile's loads are in flight, and the head's first
// block stores it for the attention kernel; otherwise k_mean_kernel ran first.
template <bool BF16, bool FUSED_MEAN>
__global__ void __launch_bounds__(256) k_quant_kernel(const QuantParams p) {
  __shared__ float mean[128];
  __shared__ float red[4];
  const int blk = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t bg = (int64_t)b * p.heads_kv + g;
  const int c8 = (tid & 15) * 8;
  const uint16_t* src = (const uint16_t*)p.k.ptr + (int64_t)b * p.k.sb + (int64_t)g * p.k.sh + c8;
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = blk * 128 + (tid >> 4) + 16 * i;
    raw[i] = t < p.n ? *(const uint4*)(src + (int64_t)t * p.k.st) : make_uint4(0, 0, 0, 0);
  }
  if (tid < 128) {
    const float m32 = FUSED_MEAN ? k_mean_of(p, bg, tid) : p.k_mean[bg * 128 + tid];
    mean[tid] = m32;
    if (FUSED_MEAN && blk == 0) p.k_mean[bg * 128 + tid] = m32;
  }
  __syncthreads();
  float x[8][8];
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = blk * 128 + (tid >> 4) + 16 * i;
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t bits = (e & 1) ? (uint16_t)(w[e >> 1] >> 16) : (uint16_t)(w[e >> 1] & 0xffff);
      x[i][e] = (t < p.n) ? __fsub_rn(elem_to_f32<BF16>(bits), mean[c8 + e]) : 0.f;
      a = fmaxf(a, fabsf(x[i][e]));
    }
  }
  a = block_max256(a, red);
  const float inv = a > 0.f ? __fdiv_rn(127.0f, a) : 0.f;
  if (tid == 0) p.k_scale[bg * p.nb + blk] = a > 0.f ? __fdiv_rn(a, 127.0f) : 0.f;
  int8_t* dst = p.k_codes + ((bg * p.nb + blk) * 128) * 128 + c8;
  int nmax = 0;  // largest squared norm of a code row (the 16 lanes of a row group share a row)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (tid >> 4) + 16 * i;
    uint32_t lo = 0, hi = 0;
    int ss = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c0 = quant8(x[i][e], inv), c1 = quant8(x[i][e + 4], inv);
      ss += c0 * c0 + c1 * c1;
      lo |= (uint32_t)(c0 & 255) << (8 * e);
      hi |= (uint32_t)(c1 & 255) << (8 * e);
    }
    *(uint2*)(dst + (int64_t)row * 128) = make_uint2(lo, hi);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o);
    nmax = max(nmax, ss);
  }
  const float n2 = block_max256((float)nmax, red);  // integers below 2^21: exact in fp32
  if (tid == 0) p.k_norm8[bg * p.nb + blk] = __builtin_sqrtf(n2) * 1.001f;
}

// Q codes in natural layout [B, Hq, nb, 128, 128] with the attention kernel's quant8.
template <bool BF16>
__global__ void __launch_bounds__(256) q_codes_kernel(const QuantParams p, int8_t* out) {
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t bh = (int64_t)b * p.heads_q + h;
  const float inv = p.q_inv[bh * p.nb + blk];
  const int c8 = (tid & 15) * 8;
  const uint16_t* src = (const uint16_t*)p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh + c8;
  int8_t* dst = out + ((bh * p.nb + blk) * 128) * 128 + c8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (tid >> 4) + 16 * i, t = blk * 128 + row;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (t < p.n) raw = *(const uint4*)(src + (int64_t)t * p.q.st);
    *(uint2*)(dst + (int64_t)row * 128) =
        make_uint2(quant4<BF16>(raw.x, raw.y, inv), quant4<BF16>(raw.z, raw.w, inv));
  }
}

// ---------------------------------------------------------------- debug views
// INT32 q8 . k8 of chosen 128x128 tiles through the attention kernel's INT8 path:
// the same Q fragment load, in-register Q codes, INT8 K DMA staging and LDS layout,
// and the same seeded i8 MFMA accumulation (qk_scores), read back as integers.  One workgroup per tile; wave w owns query rows
// 32 w .. 32 w + 31 of the tile.
template <bool BF16>
__global__ void __launch_bounds__(256) int8_scores_kernel(const AttnParams p, const int32_t* tiles, int32_t* out) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[KT * 128];
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int* tl = tiles + 4 * blockIdx.x;
  const int b = tl[0], h = tl[1], qa = tl[2], kb = tl[3];
  const int g = h / p.group;
  uint4 qf[8];
  load_q_frags<kModeTileMix>(p, b, h, qa * 128 + 32 * wave + lq, qf);
  const float inv = p.q_inv[((int64_t)b * p.heads_q + h) * p.nb + qa];
  uint4 q8f[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) q8f[s] = make_q8<BF16>(qf[2 * s], qf[2 * s + 1], inv);
  StepInfo si;
  si.k0 = kb * KT;
  si.partial = false;
  si.int8 = true;
  dma_stage<kModeTileMix, 4, kDmaK>(p, b, g, si, lds, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int32_t* dst = out + (int64_t)blockIdx.x * 128 * 128;
#pragma unroll
  for (int kb2 = 0; kb2 < KT / 32; ++kb2) {
    // the attention kernel's own INT8 product, accumulator seeded with kInt8BaseBits; the
    // seed is taken off again in integer arithmetic
    const f32x16 S = qk_scores<BF16, true>(lds, kb2, lq, lh, qf, q8f);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * kb2 + 8 * (r >> 2) + 4 * lh + (r & 3);
      dst[(32 * wave + lq) * 128 + key] = (int32_t)(__float_as_uint(S[r]) - kInt8BaseBits);
    }
  }
}

// Keys admitted per logical query row, counted over the attention kernel's own step
// list and element mask.
template <int MODE>
__global__ void __launch_bounds__(256) mask_counts_kernel(const AttnParams p, int32_t* out) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= p.length) return;
  const QInfo qi = query_info<MODE>(p, t);
  int count = 0;
  if (qi.valid) {
    const int qa = t >> 7;
    int e0;
    const int n = step_count<MODE>(p, qa, &e0);
    for (int i = 0; i < n; ++i) {
      const StepInfo s = step_info<MODE>(p, qa, e0, i);
      if (!s.partial) {
        count += KT;
      } else {
        for (int j = s.k0; j < s.k0 + KT; ++j) count += admit<MODE>(p, qi, j) ? 1 : 0;
      }
    }
  }
  out[t] = count;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_quant_finish(const QuantParams& p, hipStream_t s) {
  const dim3 gk(p.nb, p.heads_kv, p.batch);
  if (p.nb <= kFuseMeanMaxBlocks) {
    if (p.bf16) hipLaunchKernelGGL((k_quant_kernel<true, true>), gk, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_quant_kernel<false, true>), gk, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(k_mean_kernel, dim3(p.heads_kv, p.batch), dim3(128), 0, s, p);
    if (p.bf16) hipLaunchKernelGGL((k_quant_kernel<true, false>), gk, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_quant_kernel<false, false>), gk, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_quant(const QuantParams& p, hipStream_t s) {
  // the pre-pass without V^T, key norms or tail counters, over the unpadded layout
  AttnParams a;
  memset(&a, 0, sizeof(a));
  a.q = p.q;
  a.k = p.k;
  a.batch = p.batch;
  a.heads_q = p.heads_q;
  a.heads_kv = p.heads_kv;
  a.group = p.heads_q / p.heads_kv;
  a.n = p.n;
  a.text = p.text;
  a.t_pad = p.text;
  a.image = p.n - p.text;
  a.cols = 1;
  a.length = p.n;
  a.nb = p.nb;
  const dim3 gk(p.nb, p.heads_kv, p.batch);
  PlanBuild none;
  memset(&none, 0, sizeof(none));
  if (p.bf16)
    hipLaunchKernelGGL((prepass_kernel<true, kModeTileMix, true, true>), gk, dim3(256), 0, s, a, nullptr, p, none);
  else
    hipLaunchKernelGGL((prepass_kernel<false, kModeTileMix, true, true>), gk, dim3(256), 0, s, a, nullptr, p, none);
  if (hipPeekAtLastError() != hipSuccess) return hipGetLastError();
  return launch_quant_finish(p, s);
}

hipError_t launch_q_codes(const QuantParams& p, int8_t* q_codes, hipStream_t s) {
  const dim3 gq(p.nb, p.heads_q, p.batch);
  if (p.bf16)
    hipLaunchKernelGGL(q_codes_kernel<true>, gq, dim3(256), 0, s, p, q_codes);
  else
    hipLaunchKernelGGL(q_codes_kernel<false>, gq, dim3(256), 0, s, p, q_codes);
  return hipGetLastError();
}

template <bool BF16, int MODE>
static void launch_attn_t(const AttnParams& p, hipStream_t s) {
  const int64_t grid = p.lsplit.n_full + p.lsplit.n_split * p.split;
  hipLaunchKernelGGL((attn_fwd_kernel<BF16, MODE>), dim3((uint32_t)grid), dim3(64 * NWAVE), 0, s, p);
}

hipError_t launch_attention(const AttnParams& p, int mode, bool bf16, hipStream_t s) {
  if (bf16) {
    if (mode == kModeDense) launch_attn_t<true, kModeDense>(p, s);
    else if (mode == kModeTileMix) launch_attn_t<true, kModeTileMix>(p, s);
    else launch_attn_t<true, kModeScan>(p, s);
  } else {
    if (mode == kModeDense) launch_attn_t<false, kModeDense>(p, s);
    else if (mode == kModeTileMix) launch_attn_t<false, kModeTileMix>(p, s);
    else launch_attn_t<false, kModeScan>(p, s);
  }
  return hipGetLastError();
}

hipError_t launch_prepass(const AttnParams& p, uint16_t* v_t, const QuantParams* qp, const PlanBuild* pb, int mode,
                          bool bf16, hipStream_t s) {
  const dim3 grid(p.nb, p.heads_kv, p.batch);
  QuantParams noq;
  memset(&noq, 0, sizeof(noq));
  PlanBuild nop;
  memset(&nop, 0, sizeof(nop));
  const PlanBuild& b = pb != nullptr ? *pb : nop;
  if (qp != nullptr) {
    if (bf16)
      hipLaunchKernelGGL((prepass_kernel<true, kModeTileMix, true, false>), grid, dim3(256), 0, s, p, v_t, *qp, b);
    else
      hipLaunchKernelGGL((prepass_kernel<false, kModeTileMix, true, false>), grid, dim3(256), 0, s, p, v_t, *qp, b);
  } else if (bf16) {
    if (mode == kModeScan)
      hipLaunchKernelGGL((prepass_kernel<true, kModeScan, false, false>), grid, dim3(256), 0, s, p, v_t, noq, b);
    else
      hipLaunchKernelGGL((prepass_kernel<true, kModeDense, false, false>), grid, dim3(256), 0, s, p, v_t, noq, b);
  } else {
    if (mode == kModeScan)
      hipLaunchKernelGGL((prepass_kernel<false, kModeScan, false, false>), grid, dim3(256), 0, s, p, v_t, noq, b);
    else
      hipLaunchKernelGGL((prepass_kernel<false, kModeDense, false, false>), grid, dim3(256), 0, s, p, v_t, noq, b);
  }
  return hipGetLastError();
}

hipError_t launch_plan(const PlanBuild& pb, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(pb.nb), dim3(256), 0, s, pb);
  return hipGetLastError();
}

// ---------------------------------------------------------------- static scratch
// The workspace of attn_forward_noalloc, for callers that cannot allocate: a file-scope
// device array that every GPU the library runs on holds until the process ends.  In host
// code its name is only a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_region(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------- MFMA throughput probe
// Measurement only: every wave runs four independent accumulation chains of the 32 x 32
// MFMA the attention kernel uses (bf16 / f16 32x32x16, i8 32x32x32), back to back, at the
// attention kernel's occupancy (8 waves per workgroup, 2 per SIMD).  The operands depend on
// the lane so nothing folds; the first thread stores a checksum of its accumulators, which
// keeps every chain live and shows that the products ran.  KIND 3 is the bf16 product on
// operands that change from one product to the next (random signs and mantissas): the
// matrix cores' power, and so the clock the chip holds, depends on how many operand bits
// toggle, and the attention kernel's operands are random data.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
// Two bf16 values of magnitude in [0.5, 2) with random sign and mantissa.
__device__ __forceinline__ uint32_t probe_pair(uint32_t h) {
  return ((h & 0x807Fu) | 0x3F00u) | ((((h >> 16) & 0x807Fu) | 0x3F80u) << 16);
}
__device__ __forceinline__ uint4 probe_frag(uint32_t seed) {
  return make_uint4(probe_pair(probe_hash(seed)), probe_pair(probe_hash(seed + 1)), probe_pair(probe_hash(seed + 2)),
                    probe_pair(probe_hash(seed + 3)));
}
__device__ __forceinline__ void probe_random_bf16(int iters, float* sink) {
  const uint32_t base = ((uint32_t)blockIdx.x * 512u + threadIdx.x) * 64u;
  uint4 A[8], B[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    A[k] = probe_frag(base + 8 * k);
    B[k] = probe_frag(base + 8 * k + 4);
  }
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
  // four products per iteration, on fragments that rotate every iteration
  int i = 0;
  for (; i + 1 < iters; i += 2) {
#pragma unroll
    for (int k = 0; k < 8; k += 4) {
      c0 = mma16<true>(A[k], B[k + 1], c0);
      c1 = mma16<true>(A[k + 1], B[k + 2], c1);
      c2 = mma16<true>(A[k + 2], B[k + 3], c2);
      c3 = mma16<true>(A[k + 3], B[k], c3);
    }
  }
  if (i < iters) {
    c0 = mma16<true>(A[0], B[1], c0);
    c1 = mma16<true>(A[1], B[2], c1);
    c2 = mma16<true>(A[2], B[3], c2);
    c3 = mma16<true>(A[3], B[0], c3);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *(uint32_t*)sink = __float_as_uint(c0[0] + c1[1] + c2[2] + c3[3]);
}

template <int KIND>
__global__ void __launch_bounds__(512) mfma_probe_kernel(int iters, float* sink) {
  if (KIND == 3) {
    probe_random_bf16(iters, sink);
    return;
  }
  const int lane = threadIdx.x & 63;
  const uint32_t w = 0x3C003C00u ^ (uint32_t)(lane * 0x00010001u);
  const uint4 a = make_uint4(w, w ^ 1u, w ^ 2u, w ^ 3u), bv = make_uint4(w ^ 4u, w ^ 5u, w ^ 6u, w ^ 7u);
  uint32_t probe;
  if (KIND == 2) {
    i32x16 c0, c1, c2, c3;
#pragma unroll
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = r;
    for (int i = 0; i < iters; ++i) {
      c0 = mma8(a, bv, c0);
      c1 = mma8(bv, a, c1);
      c2 = mma8(a, a, c2);
      c3 = mma8(bv, bv, c3);
    }
    probe = (uint32_t)(c0[0] ^ c1[1] ^ c2[2] ^ c3[3]);
  } else {
    f32x16 c0, c1, c2, c3;
#pragma unroll
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
    for (int i = 0; i < iters; ++i) {
      c0 = mma16<KIND == 0>(a, bv, c0);
      c1 = mma16<KIND == 0>(bv, a, c1);
      c2 = mma16<KIND == 0>(a, a, c2);
      c3 = mma16<KIND == 0>(bv, bv, c3);
    }
    probe = __float_as_uint(c0[0] + c1[1] + c2[2] + c3[3]);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *(uint32_t*)sink = probe;
}

hipError_t launch_mfma_probe(int kind, int workgroups, int iters, float* sink, hipStream_t s) {
  if (kind == 0) hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(workgroups), dim3(512), 0, s, iters, sink);
  else if (kind == 1) hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(workgroups), dim3(512), 0, s, iters, sink);
  else if (kind == 2) hipLaunchKernelGGL(mfma_probe_kernel<2>, dim3(workgroups), dim3(512), 0, s, iters, sink);
  else hipLaunchKernelGGL(mfma_probe_kernel<3>, dim3(workgroups), dim3(512), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_int8_scores(const AttnParams& p, const int32_t* tiles, int n_tiles, int32_t* out, bool bf16,
                              hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(int8_scores_kernel<true>, dim3(n_tiles), dim3(256), 0, s, p, tiles, out);
  else
    hipLaunchKernelGGL(int8_scores_kernel<false>, dim3(n_tiles), dim3(256), 0, s, p, tiles, out);
  return hipGetLastError();
}

hipError_t launch_mask_counts(const AttnParams& p, int mode, int32_t* out, hipStream_t s) {
  const dim3 grid((p.length + 255) / 256);
  if (mode == kModeDense) hipLaunchKernelGGL(mask_counts_kernel<kModeDense>, grid, dim3(256), 0, s, p, out);
  else if (mode == kModeTileMix) hipLaunchKernelGGL(mask_counts_kernel<kModeTileMix>, grid, dim3(256), 0, s, p, out);
  else hipLaunchKernelGGL(mask_counts_kernel<kModeScan>, grid, dim3(256), 0, s, p, out);
  return hipGetLastError();
}

}  // namespace krea
