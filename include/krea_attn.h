/*
 * krea_attn.h -- C ABI of the MI355X (gfx950) joint [text, image] attention library.
 *
 * The operation is the bidirectional softmax attention inside each single-stream
 * block of Krea 2 ("Krea 2 TileMix Attention (FP16/INT8 tiles)", section "What it
 * actually patches": attn(q, k, v) over the joint [text, image] sequence, 48 query
 * heads over 12 KV heads resolved in the kernel instead of by repeat_interleave):
 *
 *   O[b, i, h, :] = sum_j softmax_j(s_ij) V[b, j, h / (Hq/Hkv), :]
 *
 * in one of three modes:
 *   ATTN_DENSE    every key, s_ij = scale * q_i . k_j (FP16/BF16 MFMA, fp32 softmax);
 *   ATTN_TILEMIX  each 128x128 tile of the score matrix goes to an FP16 or an INT8
 *                 path by a static map (text tiles and a diagonal band stay FP16,
 *                 a percentage of the other image-image tiles go INT8, K mean-centred
 *                 by smooth_k); both paths feed one running softmax -- same page,
 *                 sections "What it actually patches" and "The inputs that matter";
 *   ATTN_SCANLINE text is global, an image token sees image tokens within
 *                 window / 2 grid rows of its own, text and image tail padded to
 *                 128-token tiles, block mask at 128 tiles ("Krea 2 Scanline
 *                 Attention", sections "What the mask actually is" and "The settings
 *                 that matter").
 * Any mode may run its queries in slices of q_chunk tokens, each slice against the
 * full K/V ("LayerStream: Krea2 Chunking", section "What the node does to the
 * block", attn_chunk_tokens); the result does not depend on the slicing.
 *
 * Conventions for every entry point:
 *   - Tensors are described by attn_tensor: a device pointer and element strides for
 *     batch, token and head; head_dim is contiguous.  q is [B, N, Hq, 128], k and v
 *     are [B, N, Hkv, 128], o is [B, N, Hq, 128], N = text_tokens + img_rows*img_cols,
 *     tokens text first then the image grid row by row.  Pointers must be 16-byte
 *     aligned and strides multiples of 8 elements.
 *   - The caller owns q, k, v, o, the workspace and the stream.  Device entry points
 *     only enqueue work on the given HIP stream (NULL = the null stream) and return
 *     without synchronising.  attn_forward, attn_forward_gated and attn_forward_noalloc
 *     allocate no device or pinned memory, copy nothing from the host and never wait for
 *     the device: they enqueue kernel launches only, so a call can be captured into a HIP
 *     graph, also its first call of a shape.
 *   - Plans: the library keeps a host-only cache of at most 8 plans ("Krea 2 Scanline
 *     Attention", "Where people get burned": masks cached by prompt length and
 *     resolution), keyed by every shape and mode argument: the logical layout, counts,
 *     the TileMix pick threshold and the scanline geometry (plain host memory).  Every
 *     call builds its tile lists on the device, into its own workspace, from those
 *     scalars; evicting a plan therefore frees host memory only, never memory that
 *     queued work or a captured graph reads.
 *   - Every argument is validated before any device work.  Errors are returned as
 *     attn_status codes, never thrown; attn_last_error() gives a message for the
 *     calling thread.  There is no fallback path: an unsupported input is an error.
 */
#ifndef KREA_ATTN_H
#define KREA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t attn_status;
enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,      /* null pointer, bad enum, bad percentage/window/q_chunk, misalignment */
  ATTN_ERR_UNSUPPORTED_DTYPE = -2, /* fp32 inputs are refused (the TileMix page lists fp32 as a reason the
                                      fused kernel does not run, "Where people get burned") */
  ATTN_ERR_SHAPE = -3,            /* head_dim != 128, Hq % Hkv, (Hq/Hkv) % 4, sizes <= 0 or too large */
  ATTN_ERR_WORKSPACE = -4,        /* workspace smaller than attn_workspace_bytes() */
  ATTN_ERR_DEVICE = -5            /* a HIP runtime call failed */
};

enum { ATTN_F16 = 0, ATTN_BF16 = 1, ATTN_F32 = 2 };
enum { ATTN_DENSE = 0, ATTN_TILEMIX = 1, ATTN_SCANLINE = 2 };
enum { ATTN_PAT_ZERO = 0, ATTN_PAT_ONE = 1, ATTN_PAT_BAND = 2, ATTN_PAT_ALL = 3, ATTN_PAT_SAGE = 4 };

typedef struct {
  void* ptr;        /* device pointer to element [0, 0, 0, 0] */
  int64_t stride_b; /* elements between batches */
  int64_t stride_t; /* elements between tokens */
  int64_t stride_h; /* elements between heads */
} attn_tensor;

typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t heads_q;      /* Hq; Hq % Hkv == 0 and (Hq / Hkv) % 4 == 0 */
  int32_t heads_kv;     /* Hkv */
  int32_t head_dim;     /* must be 128 (Krea 2: hidden 6144 / 48 heads) */
  int32_t text_tokens;  /* T >= 0, text first in the joint sequence */
  int32_t img_rows;     /* image token grid rows (scanline uses the rows) */
  int32_t img_cols;     /* image token grid columns; N = T + rows * cols >= 1 */
  int32_t dtype;        /* ATTN_BF16 or ATTN_F16 (ATTN_F32 -> ATTN_ERR_UNSUPPORTED_DTYPE) */
  float softmax_scale;  /* applied to q.k; 0 means 1/sqrt(head_dim) rounded to fp32 */
  int32_t mode;         /* ATTN_DENSE / ATTN_TILEMIX / ATTN_SCANLINE */
  /* TileMix ("Krea 2 TileMix Attention", "The inputs that matter") */
  int32_t pattern;      /* ATTN_PAT_ZERO (all FP16), ATTN_PAT_ONE (every image-image tile INT8),
                           ATTN_PAT_BAND (diagonal band FP16, percentage of the rest INT8),
                           ATTN_PAT_ALL (every tile INT8, text included: the comparison
                           baseline of "What speedup to expect", a kernel that quantizes the
                           text tiles too), ATTN_PAT_SAGE (that baseline at the band's INT8
                           budget: as many INT8 tiles as ATTN_PAT_BAND with the same
                           percentage and band_blocks, the seeded pick drawn from every tile,
                           text included) */
  double percentage;    /* in [0, 1]: share of the image-image tiles outside the band sent to INT8;
                           count = floor(percentage * candidates) */
  int32_t band_blocks;  /* band half-width w >= 0 in 128-token blocks: |a - b| <= w stays FP16 */
  int32_t smooth_k;     /* nonzero: subtract the per-(batch, KV head, channel) mean of K before INT8 */
  uint64_t seed;        /* seeded pick of INT8 tiles: smallest SplitMix64(seed ^ (a << 32 | b)) */
  /* Scanline ("Krea 2 Scanline Attention", "The settings that matter") */
  int32_t window;       /* odd, 1..255; image tokens see rows within window / 2 */
  int32_t tile_aligned; /* nonzero: admit every valid pair inside an active 128x128 tile */
  /* Query slicing ("LayerStream: Krea2 Chunking", attn_chunk_tokens) */
  int32_t q_chunk;      /* 0 = one pass; else a multiple of 128 query positions per slice */
  int32_t reserved;     /* must be 0 */
} attn_args;

typedef struct {
  int32_t n_blocks;       /* 128-token blocks per side of the (logical) score matrix */
  int32_t text_blocks;    /* blocks holding a text token */
  int32_t logical_tokens; /* N, or the padded length for scanline */
  int32_t text_pad;       /* text length after padding (scanline), else text_tokens */
  int64_t int8_tiles;     /* TileMix: tiles routed to INT8 */
  int64_t active_tiles;   /* tiles the kernel visits (nb*nb for dense/TileMix) */
  int64_t partial_tiles;  /* visited tiles that need element masking */
} attn_plan_info;

/* Bytes of device workspace attn_forward needs for these arguments.  Every mode holds a
 * relayout of V (V^T tiles of 128 keys, the size of V rounded up to whole tiles); dense and
 * TileMix add the split tail's counters and partial states; TileMix and scanline add the
 * per-call plan (5 nb^2 + 8 nb bytes: map and tile lists); TileMix adds the smooth_k
 * partial sums and mean, INT8 K codes and scales, and Q scales.  Host only. */
attn_status attn_workspace_bytes(const attn_args* args, size_t* bytes);

/* The attention call.  q, k, v are read, o is written (rows of every valid token;
 * padding never appears in o).  workspace: device memory of at least
 * attn_workspace_bytes() bytes, 256-byte aligned; its contents on entry do not matter
 * and are overwritten.  k's token stride must be below 2^23 elements.  Enqueued on
 * `stream` (a hipStream_t). */
attn_status attn_forward(const attn_args* args, const attn_tensor* q, const attn_tensor* k,
                         const attn_tensor* v, const attn_tensor* o, void* workspace,
                         size_t workspace_bytes, void* stream);

/* attn_forward for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid device allocation): the same call with no workspace
 * argument.  Its workspace is the library's static device scratch, a file-scope array of
 * 128 MiB (134217728 bytes) that each GPU the library runs on holds until the process ends;
 * that covers the 4 MP Krea shape (16896 tokens, 48 / 12 heads) in every mode.  A call
 * whose attn_workspace_bytes() exceeds it returns ATTN_ERR_WORKSPACE before any device
 * work.  Every call on one GPU shares that GPU's scratch, and each call overwrites what
 * it uses (the split tail's counters are cleared by the call's own pre-pass kernel, not
 * by a memset): calls that overlap on one GPU -- on different streams, or from different
 * threads without ordering -- race and give undefined results.  Calls in one stream are
 * ordered and safe.  No allocation, host copy or synchronisation, as attn_forward; the
 * first call on a device looks up the scratch's address there (hipGetSymbolAddress).
 * Arguments and errors otherwise as attn_forward. */
attn_status attn_forward_noalloc(const attn_args* args, const attn_tensor* q, const attn_tensor* k,
                                 const attn_tensor* v, const attn_tensor* o, void* stream);

/* The attention call with the block's attention gate applied as the output is stored
 * ("LayerStream: Krea2 Chunking", "What the node does to the block": pass two computes the
 * attention gate beside q and applies it before the output projection):
 * o = attention(q, k, v) * sigmoid(gate), elementwise, in fp32 before the one rounding to
 * the input dtype.  gate: [B, N, Hq, 128] in the input dtype, with its own element strides
 * (head_dim contiguous, 16-byte aligned), read only.  Everything else as attn_forward.
 * Errors: those of attn_forward; gate NULL or misaligned is ATTN_ERR_INVALID_ARG. */
attn_status attn_forward_gated(const attn_args* args, const attn_tensor* q, const attn_tensor* k,
                               const attn_tensor* v, const attn_tensor* gate, const attn_tensor* o,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Weights of one block's attention context, device pointers in the args dtype, each a
 * row-major [in][out] matrix applied to token rows as x W:
 * w_q and w_gate [D][Hq * 128], w_k and w_v [D][Hkv * 128], w_o [Hq * 128][D]. */
typedef struct {
  const void* w_q;
  const void* w_k;
  const void* w_v;
  const void* w_gate;
  const void* w_o;
  int32_t model_dim; /* D, a multiple of 8 */
  int32_t reserved;  /* 0 */
} attn_block_weights;

/* Bytes of device workspace attn_block_forward needs: K and V of every token, q, gate and
 * gated attention output of one query slice, attn_forward's workspace, and the GEMM
 * library's.  Host only. */
attn_status attn_block_workspace_bytes(const attn_args* args, int32_t model_dim, size_t* bytes);

/* The attention context of one block, in the two passes of "LayerStream: Krea2 Chunking"
 * ("What the node does to the block"):
 *   pass one:  K = x W_k and V = x W_v for every token;
 *   pass two:  for each slice of q_chunk query positions (all of them when q_chunk is 0):
 *              q = x W_q and g = x W_gate for the slice's tokens, o = attention of the slice
 *              against the full K/V with o * sigmoid(g) applied in the store (the kernels
 *              of attn_forward_gated), then y[slice] += o W_o.
 * x: [B, N, D] and y: [B, N, D], contiguous device arrays in the args dtype (16-byte
 * aligned); x is read, y is added into in place (the residual stream).  The projections
 * are plain GEMMs on hipBLASLt with fp32 accumulation and outputs in the args dtype.
 * Every mode of attn_forward applies.  Enqueued on `stream`; the library keeps one
 * hipBLASLt handle per device for the process' lifetime.  The first call of a shape picks
 * each GEMM's algorithm by timing hipBLASLt's candidates on the stream, so that call waits
 * for the stream (make one call before capturing the stream into a graph); later calls of
 * the shape enqueue only.  Errors: those of attn_forward;
 * weights or x or y NULL or misaligned, model_dim not a positive multiple of 8 or
 * reserved not 0 give ATTN_ERR_INVALID_ARG; a GEMM the library cannot run gives
 * ATTN_ERR_DEVICE. */
attn_status attn_block_forward(const attn_args* args, const attn_block_weights* weights, const void* x, void* y,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Host-only plan exports (no GPU needed). */
attn_status attn_plan_info_get(const attn_args* args, attn_plan_info* out);
/* TileMix route map, row-major uint8 [nb][nb] over (query block, key block): 0 FP16, 1 INT8. */
attn_status attn_route_map(const attn_args* args, uint8_t* out, int32_t nb);
/* Scanline block mask, row-major uint8 [nb][nb] over logical tiles: 0 skip, 1 full, 2 partial. */
attn_status attn_block_mask(const attn_args* args, uint8_t* out, int32_t nb);
/* Scanline launch order of query slice `slice` (slices of q_chunk logical rows, one
 * launch each): out[L] = the work item that workgroup L runs, for the n workgroups of the
 * launch (n = ceil(slice rows / 64) * heads_q / 4 * batch; item t = query tile t % nq,
 * head group (t / nq) % (heads_q / 4), batch t / (nq * heads_q / 4)).  Workgroup L goes
 * to XCD L % 8, which runs a contiguous range of items, longest first (the number of key
 * tiles the Scanline mask gives the tile's query block: "What the mask actually is").
 * Errors: not ATTN_SCANLINE, slice out of range, n not the launch's size, out NULL. */
attn_status attn_item_order(const attn_args* args, int32_t slice, int32_t* out, int64_t n);

/* Work items of one attention launch, as the kernel maps its workgroups to them, on a
 * device with `cus` compute units (host only).  slice: the query slice (as attn_item_order);
 * *workgroups (if not NULL) receives the launch's workgroup count (whole items plus the
 * parts of split items); out (NULL: only the count) int32 [n][4], for workgroup L = (global
 * 64-query tile, pair = head group + (Hq / 4) * batch, key-range part, parts of the item),
 * n the workgroup count.  Dense and TileMix split the items of the last,
 * partial wave of the whole call (Hq / 4 * batch * ceil(N / 64) items on `cus` units) into
 * key-range parts; which items split depends only on the item's global position (its query
 * tile and pair), so every query slicing computes each row the same way.  Errors: slice out
 * of range, cus < 1, out given and n not the launch's workgroup count. */
attn_status attn_launch_items(const attn_args* args, int32_t slice, int32_t cus, int32_t* out, int64_t n,
                              int64_t* workgroups);

/* Device debug exports.  They run the same device functions as attn_forward.
 *
 * attn_quantize: the smooth_k mean and per-tile INT8 stage of TileMix ("The inputs that
 * matter", smooth_k).  Writes (each output may be NULL) k_mean float [B, Hkv, 128],
 * k_codes int8 [B, Hkv, nb, 128, 128], k_scale float [B, Hkv, nb], q_codes int8
 * [B, Hq, nb, 128, 128], q_scale float [B, Hq, nb]; code rows past N are zero.  Codes are
 * written for every block that is not a text block. */
attn_status attn_quantize(const attn_args* args, const attn_tensor* q, const attn_tensor* k,
                          void* workspace, size_t workspace_bytes, float* k_mean,
                          int8_t* k_codes, float* k_scale, int8_t* q_codes, float* q_scale,
                          void* stream);

/* attn_int8_scores: INT32 accumulators q8 . k8 of chosen 128x128 tiles, through the INT8
 * MFMA path of the attention kernel.  tiles: device int32 [n_tiles][4] = (b, h, a, kb);
 * out: device int32 [n_tiles][128 query rows][128 keys].  Runs the quantiser first. */
attn_status attn_int8_scores(const attn_args* args, const attn_tensor* q, const attn_tensor* k,
                             void* workspace, size_t workspace_bytes, const int32_t* tiles,
                             int32_t n_tiles, int32_t* out, void* stream);

/* attn_mask_row_counts: number of keys each logical query row admits, evaluated by the
 * kernel's own tile lists (built on the device into `workspace`, as attn_forward builds
 * them) and element mask.  workspace: at least attn_workspace_bytes(), 256-byte aligned.
 * out: device int32 [logical_tokens]. */
attn_status attn_mask_row_counts(const attn_args* args, void* workspace, size_t workspace_bytes, int32_t* out,
                                 void* stream);

/* attn_device_plan: the per-call plan as attn_forward builds it on the device, copied out.
 * For ATTN_TILEMIX with INT8 tiles and for ATTN_SCANLINE (anything else is
 * ATTN_ERR_INVALID_ARG).  Each output is a device pointer or NULL:
 *   map        uint8 [nb][nb]: TileMix route (1 INT8), scanline class (0 skip, 1 full,
 *              2 partial) -- the same values as attn_route_map / attn_block_mask;
 *   lists      int32 [nb][nb]: row a holds the key blocks query block a visits, in order
 *              (TileMix: FP16 full tiles, INT8 full tiles, then the ragged last block, nb
 *              entries; scanline: full tiles then partial ones as block | 1 << 16);
 *   row_count  int32 [nb]: entries of each row (nb for TileMix);
 *   full_count int32 [nb]: leading full tiles of each row (TileMix: FP16 full tiles).
 * workspace: at least attn_workspace_bytes(), 256-byte aligned.  Async on stream. */
attn_status attn_device_plan(const attn_args* args, void* workspace, size_t workspace_bytes, uint8_t* map,
                             int32_t* lists, int32_t* row_count, int32_t* full_count, void* stream);

/* Measurement hook.  With two hipEvent_t handles (created by the caller, who keeps
 * ownership), every later attn_forward on the calling thread records start_event on its
 * stream just before its first attention-kernel launch and stop_event just after its last
 * one, so the span excludes the V relayout and the quantiser.  NULL, NULL turns it off;
 * one NULL and one event is ATTN_ERR_INVALID_ARG.  A failed record makes attn_forward
 * return ATTN_ERR_DEVICE.  Host only; enqueues nothing by itself. */
attn_status attn_set_kernel_events(void* start_event, void* stop_event);

/* MFMA throughput probe (measurement only; no attention work).  Enqueues one launch of
 * `workgroups` workgroups of 8 waves, the attention kernel's occupancy.  Each wave issues
 * 4 * iters independent MFMAs of `kind`:
 *   ATTN_PROBE_BF16, ATTN_PROBE_F16: 32x32x16 with fp32 accumulation;
 *   ATTN_PROBE_I8: 32x32x32 with int32 accumulation;
 *   ATTN_PROBE_BF16_RANDOM: the bf16 product on operands that change from one product to
 *   the next (random signs and mantissas, magnitudes in [0.5, 2)).  The matrix cores draw
 *   more power, and the chip holds a lower clock, when more operand bits toggle, so this
 *   is the rate to set beside a kernel whose operands are random data.
 * Timing the launch gives the rate the chip sustains for the products the attention
 * kernel is built from, to set beside the published dense peak.
 * - *ops (host pointer) receives the operations the launch performs (2 per multiply-add).
 * - sink: device memory of at least 4 bytes; receives a 32-bit checksum of the first
 *   wave's accumulators (the same for the same kind and iters).
 * workgroups >= 1 and iters >= 1; anything else is ATTN_ERR_INVALID_ARG.  Async on stream. */
enum { ATTN_PROBE_BF16 = 0, ATTN_PROBE_F16 = 1, ATTN_PROBE_I8 = 2, ATTN_PROBE_BF16_RANDOM = 3 };
attn_status attn_mfma_probe(int32_t kind, int32_t workgroups, int32_t iters, void* sink, int64_t* ops,
                            void* stream);

const char* attn_status_string(attn_status status);
/* Message for the last error on the calling thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KREA_ATTN_H */
