/*
 * hca.h - C ABI of the hybrid compressed-attention hot path (CSA + HCA) on gfx950.
 *
 * The method is DeepSeek-V4's hybrid attention as the pages describe it:
 *   - "DeepSeek Releases V4 with Million-Token Context Optimized for AI Agents"
 *     (botbeat.news), "Summary": CSA compresses KV entries 4x by softmax-gated
 *     pooling with a learned positional bias and selects entries with a lightning
 *     indexer; HCA compresses 128x and attends densely over all compressed entries.
 *   - "DeepSeek V4: How They Crushed the Million-Token Memory Problem"
 *     (sameershanbhag.com), "Two kinds of memory instead of one": every 4 / 128
 *     tokens become one KV entry; the indexer uses ReLU-scored multi-head dot
 *     products and keeps the top-k blocks; a separate sliding window keeps recent
 *     tokens uncompressed; storage is FP8 for most KV, FP4 for the indexer and BF16
 *     for the RoPE dimensions.
 *   - "DeepSeek V4 infrastructure" (volanea.com), "Compression only works if the
 *     attention path is engineered end to end": shared key-value multi-query
 *     attention, partial rotary embeddings, a sliding-window branch and an
 *     attention sink.
 *
 * Conventions for every entry point:
 *   - Plain C.  Every call takes one descriptor whose first field `struct_size`
 *     must equal sizeof(descriptor) (hca_struct_size reports it), and a stream
 *     (a hipStream_t passed as void*; NULL = the default stream).
 *   - Every buffer pointer inside a descriptor is a DEVICE pointer owned by the
 *     caller; rows are addressed with explicit pitches in BYTES.  The library
 *     allocates no device memory, frees nothing and never waits on the host.  It
 *     keeps no state between calls other than the thread-local error message and
 *     two things made on first use and held until the process ends: the second
 *     stream and events of indexer calls that run in query groups
 *     (hca_indexer_topk; one set per device and caller stream), and the static
 *     scratch array of hca_attn_decode_noalloc (one per device).
 *   - Scratch memory comes from a caller-owned workspace of at least
 *     hca_workspace_bytes() bytes, 256-byte aligned; its contents on entry do not
 *     matter (the library clears what it needs).  Calls that share one workspace
 *     must be ordered on one stream.
 *   - Return value: HCA_OK (0) or a negative HCA_E_* code.  Argument errors are
 *     detected on the host before anything is launched; HCA_E_LAUNCH reports a
 *     launch failure.  hca_last_error() describes the last failure of the
 *     calling thread.  Device-side CONTENTS (indices, positions, rows) are not
 *     validated: they must satisfy the preconditions stated below, otherwise
 *     results are undefined.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef HCA_H
#define HCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HCA_ABI_VERSION 7

/* status codes */
#define HCA_OK             0
#define HCA_E_NULL        -1   /* a required pointer is NULL */
#define HCA_E_SHAPE       -2   /* a size is out of range or inconsistent */
#define HCA_E_ALIGN       -3   /* a pointer or pitch is misaligned */
#define HCA_E_DTYPE       -4   /* unknown or disallowed element format */
#define HCA_E_UNSUPPORTED -5   /* a valid combination this build does not implement */
#define HCA_E_WORKSPACE   -6   /* workspace missing or too small */
#define HCA_E_LAUNCH      -7   /* kernel launch failed */
#define HCA_E_VERSION     -8   /* struct_size mismatch */

/* element formats */
#define HCA_F32      0   /* IEEE binary32 */
#define HCA_BF16     1   /* bfloat16, round-to-nearest-even */
#define HCA_FP8_E4M3 2   /* OCP FP8 E4M3FN (bias 7, max 448, no inf) */
#define HCA_MXFP4    3   /* OCP MXFP4: E2M1 codes, 2 per byte (element 2i in the low
                            nibble of byte i), one E8M0 scale byte per 32 elements */

/* attention modes */
#define HCA_MODE_CSA 0   /* attend to the indexer-selected entries */
#define HCA_MODE_HCA 1   /* attend to every visible entry */
/* attend to the sliding window and the sink only: the multi-token-prediction block
   ("DeepSeek V4: How They Crushed the Million-Token Memory Problem"
   (sameershanbhag.com), "Two kinds of memory instead of one": the final block is
   sliding-window only).  No compressed entry is read: cache, cache_row_start,
   page_table, idx, k, m and max_visible are ignored (may be NULL / 0). */
#define HCA_MODE_SWA 2

/* operation ids for hca_workspace_bytes / hca_struct_size */
#define HCA_OP_KV_COMPRESS  0
#define HCA_OP_INDEXER_TOPK 1
#define HCA_OP_ATTN_DECODE  2
#define HCA_OP_ATTN_PREFILL 3
#define HCA_OP_QKV_PROLOGUE 4
#define HCA_OP_OUT_PROJ     5
#define HCA_OP_DECODE_LAYER 6
#define HCA_STRUCT_KV_PLANES  100
#define HCA_STRUCT_IDX_PLANES 101

/*
 * Compressed KV cache planes, one row per compressed entry (or per window token
 * when used as raw storage).  D = D_n + D_r dims, the last D_r being the RoPE slice.
 *   fmt HCA_F32:      f32   [rows, D] float, already rotated.
 *   fmt HCA_FP8_E4M3: nope  [rows, D_n] E4M3 codes; value = code * scale[row]
 *                     rope  [rows, D_r] BF16, already rotated
 *                     scale [rows] float, a power of two (the smallest 2^e with
 *                           max|nope| <= 448 * 2^e, 1 for an all-zero entry).
 */
typedef struct hca_kv_planes {
  int32_t fmt;
  int32_t reserved;
  void*   f32;    int64_t f32_pitch;
  void*   nope;   int64_t nope_pitch;
  void*   rope;   int64_t rope_pitch;
  void*   scale;
} hca_kv_planes;

/*
 * Indexer vectors, one row of d_I elements per key (cache) or per (query, head).
 *   fmt HCA_F32:      data [rows, d_I] float
 *   fmt HCA_FP8_E4M3: data [rows, d_I] E4M3 codes, per-tensor scale 1
 *   fmt HCA_MXFP4:    data [rows, d_I/2] packed E2M1, scales [rows, d_I/32] E8M0
 *                     (indexer keys: scale rows 4-byte aligned, else HCA_E_ALIGN)
 */
typedef struct hca_idx_planes {
  int32_t fmt;
  int32_t reserved;
  void*   data;    int64_t pitch;
  void*   scales;  int64_t scale_pitch;
} hca_idx_planes;

/*
 * hca_kv_compress: softmax-gated pooling of aligned blocks of m raw tokens into
 * compressed entries ("DeepSeek Releases V4 ...", botbeat.news, "Summary").
 *
 * For block n (raw rows block_row[n] .. block_row[n]+m-1, first token at absolute
 * position block_pos[n], a multiple of m):
 *   z_i     = gate_w . x_i + gate_b[i]            (x_i: raw, un-rotated, D dims)
 *   alpha   = softmax(z) over the block's m tokens
 *   c       = sum_i alpha_i x_i,   y = sum_i alpha_i y_i   (y: raw indexer keys)
 *   entry   = [c_nope ; RoPE(block_pos[n] + m - 1) c_rope]
 * RoPE is half-split: dims (i, i + D_r/2) of the slice rotate by
 * pos * rope_base^(-2i/D_r).  Arithmetic is fp64; the entry is then encoded into
 * `out` at row out_row[n] (f32, or FP8 nope + per-entry power-of-two scale + BF16
 * rope), and y, when raw_idx is given, into `out_idx` (f32, FP8 with scale 1, or
 * MXFP4), every encoding rounding to nearest-even once from fp64 (FP8 and FP4
 * saturate).  `debug`, if not NULL, receives the pre-encoding values as f32
 * [n_blocks, D + d_I] (d_I = 0 without raw_idx).
 *
 * Limits: 1 <= m <= 256, D a multiple of 8 up to 1024, D_r even and <= D, d_I a
 * multiple of 8 up to 256 (of 32 for MXFP4).  raw/raw_idx rows are F32 or BF16
 * (raw_fmt) and 16-byte aligned, as is gate_w.
 * Preconditions on device data: every block's rows lie inside the raw buffers and
 * out_row values are distinct rows of the output planes.  Needs no workspace.
 */
typedef struct hca_kv_compress_desc {
  uint32_t struct_size;
  int32_t  m, D, D_r, d_I;
  int32_t  n_blocks;
  double   rope_base;
  int32_t  raw_fmt;
  int32_t  reserved;
  const void*    raw;      int64_t raw_pitch;
  const void*    raw_idx;  int64_t raw_idx_pitch;
  const int64_t* block_row;
  const int64_t* block_pos;
  const int64_t* out_row;
  const float*   gate_w;   /* [D] */
  const float*   gate_b;   /* [m] */
  hca_kv_planes  out;
  hca_idx_planes out_idx;  /* ignored when raw_idx is NULL */
  float*         debug;
} hca_kv_compress_desc;

/*
 * hca_indexer_topk: lightning-indexer scores and per-query top-k
 * ("DeepSeek V4: How They Crushed ...", sameershanbhag.com, "Two kinds of memory
 * instead of one").
 *
 * Query n belongs to sequence seq_id[n] and sits at absolute position q_pos[n];
 * it sees entries j < V = floor((q_pos[n] + 1) / m) of its sequence, stored at
 * key rows cache_row_start[seq] + j (or through the page table, below).  For
 * every visible j:
 *   d_h   = q[n, h] . key[j]                        (exact)
 *   I_j   = sum_h w[n, h] * max(d_h, 0)
 * Quantized operands (FP8 or MXFP4, same format for q and keys; d_I = 128,
 * H_I = 32 or 64): d_h is exact in binary32, and I_j = fl(S_0 + S_1) where S_u
 * starts at +0 and takes, for heads h = 32T + 8(i / 4) + 4u + (i % 4) in order
 * T = 0, 1, then i = 0..15, S_u = fl(w_h * max(d_h, +0) + S_u) (binary32, one
 * rounding per head: a fused multiply-add).  F32 operands: dots and the head sum in fp64,
 * sequential, un-fused (V <= 4096 per query).
 * Output: idx[n, 0..k) = the min(k, V) entries with the largest I (equal scores:
 * lower j first), in ascending j, padded with -1; `score` (optional) gets their
 * scores in the same order (f32, or f64 for F32 operands).
 * max_visible must bound V for every query.  q and keys share `fmt`; `q` has
 * Nq*H_I rows (row n*H_I + h).  w is [Nq, H_I] f32 with w >= 0.
 * Quantized keys: max_visible <= 2^23, key (and, for MXFP4, key-scale) pitches
 * below 2^24 bytes, and max_visible times each such pitch (page_rows times it,
 * with a page table) below 2^32 bytes; otherwise HCA_E_UNSUPPORTED.
 * Workspace (quantized operands): one f32 score row per query of a query group
 * (ceil(max_visible / 64) * 256 bytes each) plus the selection's lists (about
 * 75 KB per query).  A call whose whole workspace would exceed 896 MiB runs in
 * near-equal query groups (a multiple of 8 queries, at least 256) and keeps two
 * groups: group g is scored on `stream` while the selection of group g - 1 runs
 * on a second stream the library creates once per device and caller stream
 * (default priority),
 * joined back to `stream` through events before the call returns, so work queued
 * on `stream` afterwards sees every result.  The workspace stays within 896 MiB
 * whatever Nq (at least two groups of 256 queries' worth), and the results are
 * those of one group holding every query.
 */
typedef struct hca_indexer_topk_desc {
  uint32_t struct_size;
  int32_t  Nq, B, H_I, d_I, k, m;
  int32_t  reserved;
  int64_t  max_visible;
  hca_idx_planes q;
  const float*   w;
  hca_idx_planes keys;
  const int64_t* cache_row_start;   /* [B] */
  const int32_t* seq_id;            /* [Nq] */
  const int64_t* q_pos;             /* [Nq] */
  int32_t*       idx;               /* [Nq, k] */
  void*          score;             /* [Nq, k] or NULL */
  void*          workspace;
  size_t         workspace_bytes;
  /* Paged compressed cache (optional; NULL = contiguous rows from cache_row_start,
     which is then required).  "DeepSeek V4 infrastructure" (volanea.com), "Compression
     only works if the attention path is engineered end to end", asks for a cache
     format that holds up under continuous batching; the block table is this
     library's reading of it.  With a page table, entry j of sequence b lives at
     cache row page_table[b * page_table_pitch + j / page_rows] * page_rows +
     j % page_rows, and cache_row_start is not read (may be NULL).  page_rows is a
     power of two in [1, 2^24] (at least 32 for quantized indexer keys);
     page_table_pitch >= ceil(max_visible / page_rows); every page id a visible
     entry needs must name a page inside the cache (not checked: the table is
     device memory).  Bad page_rows or pitch: HCA_E_SHAPE; page_rows below the
     minimum: HCA_E_UNSUPPORTED. */
  const int32_t* page_table;
  int64_t        page_table_pitch;
  int32_t        page_rows;
  int32_t        reserved_page;
} hca_indexer_topk_desc;

/*
 * hca_attn_decode / hca_attn_prefill: shared-KV multi-query attention with one
 * softmax over compressed entries, the sliding window and a sink
 * ("DeepSeek V4 infrastructure", volanea.com, "Compression only works if the
 * attention path is engineered end to end").
 *
 * Query n (sequence b = seq_id[n], position t = q_pos[n]) attends, with every one
 * of its H heads, to the same key=value vectors:
 *   - CSA: the entries idx[n, 0..k) that are >= 0 (an ascending, -1 padded list
 *     as hca_indexer_topk writes it);  HCA: every entry j < floor((t+1)/m);
 *   - the window tokens u = max(0, t-n_win+1) .. t read from the ring `win`
 *     (row b*win_cap + u mod win_cap, un-rotated, io_fmt), RoPE-rotated at u;
 * and entry j lives at cache row cache_row_start[b] + j, or through the page
 * table (see the descriptor; an idx value outside
 * [0, floor((t+1)/m)) is skipped, never dereferenced).  The query's RoPE slice
 * is rotated at t.  With logits l_a = tau * q_hat . kappa_a and the per-head sink
 * logit sigma_h (not scaled by tau, zero value vector):
 *   M = max(sigma_h, max_a l_a)
 *   o = sum_a e^(l_a - M) kappa_a / (e^(sigma_h - M) + sum_a e^(l_a - M))
 *   lse = M + log(e^(sigma_h - M) + sum_a e^(l_a - M))        (optional output)
 * io_fmt HCA_F32 needs cache fmt HCA_F32 (fp64 arithmetic, any D <= 1024, at most
 * 4096 keys per query: k (CSA) or max_visible (HCA), plus n_win; HCA_E_UNSUPPORTED
 * beyond); io_fmt HCA_BF16 needs cache fmt HCA_FP8_E4M3, D = 512,
 * D_r = 64, H a multiple of 16 up to 64 (BF16 MFMA, fp32 softmax), with q, o, the
 * ring and the cache rows 16-byte aligned (HCA_E_ALIGN otherwise).
 * The ring must hold every window token of every query: win_cap >= n_win plus the
 * spread of the query positions of one sequence.  max_visible bounds
 * floor((t+1)/m) over all queries.  hca_attn_prefill takes the same descriptor
 * for a chunk of consecutive query positions and differs only in scheduling.
 */
typedef struct hca_attn_desc {
  uint32_t struct_size;
  int32_t  Nq, B, H, D, D_r, mode, m, k, n_win, win_cap;
  float    tau;
  int32_t  io_fmt;
  double   rope_base;
  int64_t  max_visible;
  const void*    q;                 /* [Nq, H, D] io_fmt, un-rotated */
  hca_kv_planes  cache;
  const int64_t* cache_row_start;   /* [B] */
  const int32_t* idx;               /* [Nq, k] (CSA), else NULL */
  const void*    win;    int64_t win_pitch;
  const float*   sink;              /* [H] */
  const int32_t* seq_id;            /* [Nq] */
  const int64_t* q_pos;             /* [Nq] */
  void*          o;                 /* [Nq, H, D] io_fmt */
  float*         lse;               /* [Nq, H] or NULL */
  void*          workspace;
  size_t         workspace_bytes;
  /* Paged compressed cache (optional; NULL = contiguous rows from cache_row_start,
     which is then required).  "DeepSeek V4 infrastructure" (volanea.com), "Compression
     only works if the attention path is engineered end to end", asks for a cache
     format that holds up under continuous batching; the block table is this
     library's reading of it.  With a page table, entry j of sequence b lives at
     cache row page_table[b * page_table_pitch + j / page_rows] * page_rows +
     j % page_rows, and cache_row_start is not read (may be NULL).  page_rows is a
     power of two in [1, 2^24] (at least 32 for quantized indexer keys);
     page_table_pitch >= ceil(max_visible / page_rows); every page id a visible
     entry needs must name a page inside the cache (not checked: the table is
     device memory).  Bad page_rows or pitch: HCA_E_SHAPE; page_rows below the
     minimum: HCA_E_UNSUPPORTED. */
  const int32_t* page_table;
  int64_t        page_table_pitch;
  int32_t        page_rows;
  /* Batch-invariant decode ("DeepSeek V4 infrastructure" (volanea.com), "TileLang
     and deterministic kernels are part of the product strategy": batch-invariant,
     deterministic kernels and bitwise reproducibility).  0 = the default decode plan, which cuts the chunks of all
     queries (64 set slots each: entries, then window tokens) into equal runs over
     the workgroups, so the rounding of a query's output depends on the rest of the
     batch.  split_chunks > 0 (hca_attn_decode, BF16): each query's own chunks are
     cut into runs of split_chunks chunks from its first chunk and the runs are
     merged in order, so o and lse of a query are the same bits whatever the batch
     holds and however it is ordered (for a fixed split_chunks).  A query may then
     need at most 256 runs: ceil(ceil((min(k, max_visible) or max_visible, plus
     n_win) / 64) / split_chunks) <= 256, else HCA_E_UNSUPPORTED; negative:
     HCA_E_SHAPE.  Ignored by hca_attn_prefill (one workgroup per query, never split)
     and by the F32 path (one workgroup per query and head); both are batch-invariant
     already, as is hca_indexer_topk (exact scores, canonical top-k). */
  int32_t        split_chunks;
} hca_attn_desc;

/*
 * Query and key-value normalization, and the append of new tokens to the window
 * ring.  "DeepSeek V4 infrastructure" (volanea.com), "Compression only works if the
 * attention path is engineered end to end": the attention path normalizes queries
 * and key-value vectors.  Read as root-mean-square normalization with a learned
 * per-dimension scale, over the D dims of a row:
 *   y_d = gamma_d * x_d / sqrt(sum_e(x_e^2) / D + eps)
 * evaluated in fp64 (the sum in a fixed order) and rounded once into io_fmt, so a
 * stored code differs from the exact one only for a value within about 1e-15 of a
 * rounding boundary.
 *   - q: the Nq * H head vectors of q_in (contiguous [Nq, H, D]) are written,
 *     normalized with gamma_q, to q_out (which may equal q_in);
 *   - new tokens: row i of kv_in (Nt rows, pitch kv_pitch) is normalized with
 *     gamma_kv and written to the ring `win` at row tok_seq[i] * W_cap +
 *     (tok_pos[i] mod W_cap) (pitch win_pitch): the sliding-window state that
 *     pooling and the window branch read.  A token whose tok_seq is outside [0, B)
 *     is skipped.  Two tokens of one call must not share a ring row;
 *   - optional index stream (CSA): row i of idx_in (d_I dims, io_fmt) is copied
 *     unchanged into win_idx at the same ring row (idx_in NULL = none).
 * io_fmt HCA_F32 or HCA_BF16 (all rows); D a multiple of 8 (BF16) or 4 (F32), at
 * most 4096 (BF16) / 2048 (F32); d_I likewise; rows and pitches 16-byte aligned;
 * gamma_q, gamma_kv: [D] float, 16-byte aligned; eps >= 0 and finite.  Nq = 0 or Nt = 0 skips a part.
 * The library needs no workspace for this call.
 */
typedef struct hca_qkv_prologue_desc {
  uint32_t struct_size;
  int32_t  io_fmt;
  int32_t  Nq, H, D;
  int32_t  Nt, B, W_cap, d_I;
  double   eps;
  const void*    q_in;
  void*          q_out;
  const float*   gamma_q;
  const void*    kv_in;    int64_t kv_pitch;
  const float*   gamma_kv;
  const int32_t* tok_seq;   /* [Nt] */
  const int64_t* tok_pos;   /* [Nt] */
  void*          win;      int64_t win_pitch;
  const void*    idx_in;   int64_t idx_pitch;
  void*          win_idx;  int64_t win_idx_pitch;
} hca_qkv_prologue_desc;

/*
 * Grouped output projection after attention.  "DeepSeek V4 infrastructure"
 * (volanea.com), "Compression only works if the attention path is engineered end to
 * end": CSA's attention ends in a grouped output projection.  Read as: the H heads
 * form G consecutive groups of H / G heads; group g's head outputs, concatenated in
 * head order (K_g = (H / G) * D values), are multiplied by the group's own weights,
 * and the G results are concatenated:
 *   y[n, g * d_g + c] = sum_{k < K_g} o[n, g * K_g + k] * W[g * d_g + c, k]
 * o: Nq rows of H * D BF16 (attention's o, heads in order; pitch o_pitch bytes);
 * W: G * d_g rows of K_g BF16 (output unit c of group g at row g * d_g + c; pitch
 * w_pitch); y: Nq rows of G * d_g values in out_fmt (HCA_F32 or HCA_BF16, pitch
 * y_pitch).  Products of BF16 values are exact; they are summed in binary32 in a
 * fixed order (up to 64 rows: partial sums over consecutive quarters or eighths of
 * k, added in order; more rows with d_g a multiple of 128: one sum over k in order),
 * then rounded once to out_fmt.  Needs H % G == 0, K_g a multiple of 256, d_g a
 * multiple of 32, 16-byte aligned rows (HCA_E_UNSUPPORTED / HCA_E_SHAPE /
 * HCA_E_ALIGN otherwise).  No workspace.
 */
typedef struct hca_out_proj_desc {
  uint32_t struct_size;
  int32_t  out_fmt;
  int32_t  Nq, H, D, G, d_g;
  const void* o;  int64_t o_pitch;
  const void* w;  int64_t w_pitch;
  void*       y;  int64_t y_pitch;
} hca_out_proj_desc;

/*
 * hca_decode_layer: one decode step of one layer, the three calls above in one:
 * pooling of the blocks that the step's new tokens complete (`pool`; NULL or
 * n_blocks = 0: nothing to pool), then, for a CSA layer (attn->mode ==
 * HCA_MODE_CSA), the indexer top-k (`indexer`, required there and NULL otherwise;
 * attention reads the idx it writes), then decode attention (`attn`).  The results
 * are bit for bit those of hca_kv_compress, hca_indexer_topk and hca_attn_decode
 * called in that order on `stream`.  "DeepSeek V4 infrastructure" (volanea.com),
 * "MegaMoE targets the real bottleneck in sparse models", counts the idle time
 * between kernel launches as a cost of its own: here the pooling needs no launch of
 * its own where the launch plan allows, and workgroups that do not read a new entry
 * never wait for it.
 *
 * Decode precondition: a pooled block's entry is the newest entry that the queries
 * of its sequence see (entry floor((t + 1) / m) - 1 for a query at t; in decode the
 * token at t completes that block exactly when (t + 1) mod m = 0).  Pooling any
 * other entry that a query of this call reads leaves its scores and output
 * undefined (every access stays inside the buffers: no fault, no hang).
 * Under it, a CSA step with FP8 keys in rows of a multiple of 128 bytes (pitch and
 * base), or MXFP4 keys and fewer than 256 queries, whose blocks hold at most 16 BF16
 * rows of 512 dims with an index stream, pools inside the scoring launch; a decode HCA step of at most 256 queries whose
 * blocks hold 17 to 128 such rows (no index stream), at most 64 of them, pools
 * inside the attention launch.  The pooling workgroups lead the grid, and only the
 * workgroup that reads a query's newest entry waits for them, inside the device and
 * for a bounded time.  Any other combination launches the pooling first.
 *
 * The descriptors are validated as their own calls validate them, before any
 * launch, and must agree: m of each equal to attn->m; for CSA, indexer->Nq, k and
 * idx equal to attn's.  The indexer and attention keep their own workspaces;
 * hca_workspace_bytes(HCA_OP_DECODE_LAYER, ...) gives 0.
 */
typedef struct hca_decode_layer_desc {
  uint32_t struct_size;
  int32_t  reserved;
  const hca_kv_compress_desc*  pool;      /* optional */
  const hca_indexer_topk_desc* indexer;   /* CSA only */
  const hca_attn_desc*         attn;      /* required */
} hca_decode_layer_desc;

/*
 * Timing hook for benchmarks (not part of the computation): hca_profiled runs the
 * call (op, desc) exactly as its own entry point does and records the event `begin`
 * on the stream immediately before, and `end` immediately after, that call's main
 * kernel: the scoring kernel of HCA_OP_INDEXER_TOPK (top-k selection excluded; of
 * the first query group when the call runs in several), the
 * attention kernel of HCA_OP_ATTN_DECODE / HCA_OP_ATTN_PREFILL (the combine of split
 * decode queries excluded), and of HCA_OP_DECODE_LAYER the scoring launch of a CSA
 * layer (with the pooling when it rides there) or the attention kernel of an HCA or
 * sliding-window layer.  begin and end are hipEvent_t values passed as void*
 * (either may be NULL).  Other ops: HCA_E_UNSUPPORTED.
 */
typedef struct hca_profile_events {
  uint32_t struct_size;
  int32_t  reserved;
  void*    begin;
  void*    end;
} hca_profile_events;
#define HCA_STRUCT_PROFILE_EVENTS 102

int         hca_abi_version(void);
const char* hca_last_error(void);
/* sizeof the descriptor of an HCA_OP_* id, or of an HCA_STRUCT_* plane struct; 0 if unknown */
size_t      hca_struct_size(int which);
/* workspace bytes the call described by (op, desc) needs.  For the indexer and
   attention only the shapes that decide the size are checked (the buffers may not
   exist yet); the other operations are validated like the call. */
int         hca_workspace_bytes(int op, const void* desc, size_t* bytes);
/* queries per group of the indexer call described by desc (only its shapes are
   read): desc->Nq when the call runs as one group, else the size of each group but
   the last, which holds the rest (see hca_indexer_topk_desc) */
int         hca_indexer_query_group(const hca_indexer_topk_desc* desc, int32_t* group);

int hca_kv_compress(const hca_kv_compress_desc* desc, void* stream);
int hca_indexer_topk(const hca_indexer_topk_desc* desc, void* stream);
int hca_attn_decode(const hca_attn_desc* desc, void* stream);
int hca_attn_prefill(const hca_attn_desc* desc, void* stream);
/*
 * hca_attn_decode_noalloc: hca_attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same descriptor, same kernels and the same results bit for bit;
 * desc->workspace and desc->workspace_bytes are ignored: the scratch is a static
 * device array of 40 MiB per GPU inside the library, held from the library's load
 * until the process ends (its address is looked up once per device, on the first
 * call made with that device current; the stream must belong to the current
 * device).  The call allocates and frees nothing.  A call needing more scratch than
 * that (hca_workspace_bytes reports the need) fails with HCA_E_WORKSPACE before
 * anything is launched; decode calls of up to 256 queries and 64 heads without a
 * fixed split always fit.  Every call on one GPU shares that GPU's array, and the
 * kernels need none of its previous contents: calls that overlap on one GPU (on
 * different streams, unordered) race on it and must not be issued.
 */
int hca_attn_decode_noalloc(const hca_attn_desc* desc, void* stream);
int hca_qkv_prologue(const hca_qkv_prologue_desc* desc, void* stream);
int hca_out_proj(const hca_out_proj_desc* desc, void* stream);
int hca_decode_layer(const hca_decode_layer_desc* desc, void* stream);
int hca_profiled(int op, const void* desc, const hca_profile_events* events, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HCA_H */
