// Shared-KV multi-query attention with one softmax over compressed entries, the
// sliding window of raw tokens and a per-head sink logit.
//
// "DeepSeek V4 infrastructure" (volanea.com), "Compression only works if the
// attention path is engineered end to end": compressed entries chosen by the
// indexer, shared key-value MQA, partial RoPE, a sliding-window branch and an
// attention sink.  "DeepSeek V4: How They Crushed the Million-Token Memory Problem"
// (sameershanbhag.com), "Two kinds of memory instead of one": HCA attends densely
// to all its compressed entries; both keep the recent tokens uncompressed.
//
// All query heads share every key, and a key is also its value.  For query t:
//   l_a = tau * q_hat . kappa_a,  M = max(sigma, max l),
//   o = sum e^(l_a - M) kappa_a / (e^(sigma - M) + sum e^(l_a - M)).
//
// BF16 path: one workgroup = one query x one contiguous slice of its attention set,
// one wave per 16 heads.  Keys are staged 32 at a time into LDS as BF16 rows (FP8
// codes widened with their power-of-two scale, window tokens rotated); QK^T reads
// them row-wise, P.V reads them transposed with ds_read_b64_tr_b16, so one copy of
// the tile serves both products.  Each slice leaves (max, sum, unnormalized o) and a
// combine kernel merges the slices in a fixed order with the sink.
#include <mutex>

#include "device_common.hpp"
#include "hca_internal.hpp"
#include "pool_block.hpp"
#include "../../include/hca.h"

namespace hca {

namespace {

constexpr double kLog2e = 1.4426950408889634;
constexpr double kTwoPi = 6.283185307179586;

struct SetInfo {
  int64_t V;         // visible compressed entries
  int64_t row0;      // first cache row of the sequence
  int n_ent;         // compressed entries in the attention set
  int64_t u0;        // first window position
  int n_w;           // window tokens
};

// everything but the first cache row, from the query position alone
__device__ __forceinline__ SetInfo set_info_pos(const AttnArgs& a, int64_t t) {
  SetInfo si;
  si.row0 = 0;
  int64_t V = (t + 1) / a.m;
  if (V > a.max_visible) V = a.max_visible;
  si.V = V;
  // CSA: the list is ascending and -1 padded, so its valid entries are a prefix of
  // at most min(k, V) slots; invalid slots inside it are masked when staged
  si.n_ent = (int)(a.mode == HCA_MODE_CSA ? (V < a.k ? V : a.k) : V);
  si.u0 = t - a.n_win + 1 > 0 ? t - a.n_win + 1 : 0;
  si.n_w = (int)(t - si.u0 + 1);
  if (a.n_win == 0) si.n_w = 0;
  return si;
}

__device__ __forceinline__ SetInfo set_info(const AttnArgs& a, int n) {
  SetInfo si = set_info_pos(a, a.q_pos[n]);
  // paged: rows through the table; no row map: no entry is ever read (window only)
  si.row0 = a.page_shift < 0 && a.cache_row_start ? a.cache_row_start[a.seq_id[n]] : 0;
  return si;
}

// ============================================================== f32 path (fp64)
constexpr int kF32MaxSet = 4096;

// an index list entry outside [0, V) is skipped (never dereferenced)
__device__ __forceinline__ bool key_ok(const AttnArgs& a, const SetInfo& si, int n, int p) {
  if (p >= si.n_ent || a.mode != HCA_MODE_CSA) return true;
  const int64_t j = a.idx[(int64_t)n * a.k + p];
  return j >= 0 && j < si.V;
}

__device__ double key_elem_f64(const AttnArgs& a, const SetInfo& si, int n, int p, int d,
                               const double* s_inv) {
  if (p < si.n_ent) {
    int64_t j = (a.mode == HCA_MODE_CSA) ? a.idx[(int64_t)n * a.k + p] : p;
    if (j < 0 || j >= si.V) return 0.0;
    const int64_t row = cache_row(a.page_table, a.page_pitch, a.page_shift, a.seq_id[n], si.row0, j);
    return (double)reinterpret_cast<const float*>(a.c_f32 + row * a.c_f32_pitch)[d];
  }
  const int64_t u = si.u0 + (p - si.n_ent);
  const int64_t row = (int64_t)a.seq_id[n] * a.win_cap + u % a.win_cap;
  const float* x = reinterpret_cast<const float*>(a.win + row * a.win_pitch);
  const int D_n = a.D - a.D_r, half = a.D_r / 2;
  if (d < D_n) return (double)x[d];
  const int i = (d - D_n) % half;
  double sn, cs;
  sincos((double)u * s_inv[i], &sn, &cs);
  const double x0 = x[D_n + i], x1 = x[D_n + half + i];
  return d - D_n < half ? x0 * cs - x1 * sn : x0 * sn + x1 * cs;
}

__global__ void __launch_bounds__(256) attn_f32_kernel(AttnArgs a) {
  __shared__ double s_q[1024];
  __shared__ double s_l[kF32MaxSet];
  __shared__ double s_inv[512];
  __shared__ double s_red[4];
  const int n = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const SetInfo si = set_info(a, n);
  const int64_t t = a.q_pos[n];
  const int D = a.D, D_n = a.D - a.D_r, half = a.D_r / 2;
  for (int i = tid; i < half; i += 256) s_inv[i] = pow(a.rope_base, -2.0 * i / a.D_r);
  __syncthreads();
  const float* q = reinterpret_cast<const float*>(a.q) + ((int64_t)n * a.H + h) * D;
  for (int d = tid; d < D; d += 256) {
    if (d < D_n) { s_q[d] = q[d]; continue; }
    const int i = (d - D_n) % half;
    double sn, cs;
    sincos((double)t * s_inv[i], &sn, &cs);
    const double x0 = q[D_n + i], x1 = q[D_n + half + i];
    s_q[d] = d - D_n < half ? x0 * cs - x1 * sn : x0 * sn + x1 * cs;
  }
  __syncthreads();
  const int n_set = si.n_ent + si.n_w;
  double mx = -INFINITY;
  for (int p = tid; p < n_set; p += 256) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += s_q[d] * key_elem_f64(a, si, n, p, d, s_inv);
    acc *= (double)a.tau;
    if (!key_ok(a, si, n, p)) acc = -INFINITY;
    s_l[p] = acc;
    mx = fmax(mx, acc);
  }
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  const double sig = (double)a.sink[h];
  double M = fmax(fmax(s_red[0], s_red[1]), fmax(s_red[2], s_red[3]));
  M = fmax(M, sig);
  __syncthreads();
  double sum = 0.0;
  for (int p = tid; p < n_set; p += 256) { double e = exp(s_l[p] - M); s_l[p] = e; sum += e; }
  sum = wave_sum(sum);
  if (lane == 0) s_red[wave] = sum;
  __syncthreads();
  const double den = exp(sig - M) + (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  float* o = reinterpret_cast<float*>(a.o) + ((int64_t)n * a.H + h) * D;
  for (int d = tid; d < D; d += 256) {
    double acc = 0.0;
    for (int p = 0; p < n_set; ++p) acc += s_l[p] * key_elem_f64(a, si, n, p, d, s_inv);
    o[d] = (float)(acc / den);
  }
  if (a.lse && tid == 0) a.lse[(int64_t)n * a.H + h] = (float)(M + log(den));
}

// ============================================================ BF16 MFMA path
//
// One workgroup of 8 waves walks a contiguous run of 64-key chunks.  Wave w
// owns head group hg = w % 4 (heads 16hg .. 16hg+15) and dim half dh = w / 4
// (dims 256dh .. 256dh+255): QK^T is summed over its dims and the two halves
// exchange partial logits through LDS (every logit is then S_dh0 + S_dh1, the
// same in both waves), so both hold identical probabilities and each accumulates
// P.V for its own 256 output dims.  The compressed entries of chunk c+1 are loaded
// into registers while chunk c is computed, then widened to BF16 into the LDS
// tile; window tokens (the set positions after the entries, any n_win) are staged
// directly from the ring.
//
// Decode (few queries): the chunks of all queries form one list that is cut into
// equal runs, one per workgroup, so ragged lengths balance.  A query whose chunks
// all fall in one run is finished there; otherwise each run leaves a partial
// (max, sum, unnormalized o) in the workspace and a combine kernel merges them in
// run order with the sink.  Prefill (many queries): one workgroup per query.
// Fixed split (decode with split_chunks > 0): each query's own chunk list is cut
// into runs of split_chunks chunks from its first chunk, one workgroup per run, so
// every run boundary, partial and merge depends on that query alone and its result
// is the same bits whatever else is in the batch.
constexpr int kD = 512, kDr = 64, kDn = 448;
constexpr int KC = 64;                     // keys per chunk
constexpr int kKsPitch = kD + 8;           // bf16 per LDS key row (1040 B: rows 4 banks apart)
constexpr int kPtPitch = 16 + 4;           // bf16 per LDS row of P^T (16 heads)
constexpr int kThreads = 512;              // 8 waves
constexpr int kIdxWin = 2048;              // index-list positions held in LDS
constexpr int kMaxDecodeQ = 256;           // queries of one flattened (decode) launch
constexpr int kMaxRuns = 256;              // runs one combine workgroup merges (one thread each)
#ifndef HCA_ATTN_GRID
#define HCA_ATTN_GRID 256                  // workgroups of a decode launch
#endif
static_assert(HCA_ATTN_GRID <= kMaxRuns, "a flattened query spans at most every workgroup");
#ifndef HCA_ATTN_MIN_CHUNKS
#define HCA_ATTN_MIN_CHUNKS 1              // fewest chunks per decode workgroup
#endif

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

// cos/sin of pos * inv: the angle is formed in fp64 and reduced to a fraction of a
// turn in [-1/2, 1/2] (exact enough at positions ~1e6), then evaluated by the
// hardware sine/cosine, whose argument is in turns.  inv_turn = inv / (2 pi).
__device__ __forceinline__ void rope_cs(int64_t pos, double inv_turn, float* c, float* s) {
  double turns = (double)pos * inv_turn;
  turns -= rint(turns);
  const float f = (float)turns;
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}

template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t w, float sc) {
  v2bf v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, sc, HI);
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

// 8 FP8 codes -> 8 BF16 values times the power-of-two scale (exact)
__device__ __forceinline__ u4 cvt8(u2 x, float sc) {
  return (u4){cvt2<false>(x[0], sc), cvt2<true>(x[0], sc), cvt2<false>(x[1], sc), cvt2<true>(x[1], sc)};
}

// What one query attends to, as the chunk walk needs it.
struct QInfo {
  int64_t row0;     // first cache row of the sequence
  int64_t u0;       // first window position
  int64_t t;        // query position
  int64_t V;        // visible compressed entries
  int n_ent;        // compressed entries in the set (a prefix of the index list for CSA)
  int n_set;        // n_ent + window tokens
  int b;            // sequence
  int pad;
};

// the query record without its first cache row (row0 = 0), for sequence b
__device__ __forceinline__ QInfo query_info_pos(const AttnArgs& a, int n, int b) {
  QInfo qi;
  const int64_t t = a.q_pos[n];
  const SetInfo si = set_info_pos(a, t);
  qi.row0 = 0;
  qi.u0 = si.u0;
  qi.t = t;
  qi.V = si.V;
  qi.n_ent = si.n_ent;
  qi.n_set = si.n_ent + si.n_w;
  qi.b = b;
  qi.pad = 0;
  return qi;
}

__device__ __forceinline__ QInfo query_info(const AttnArgs& a, int n) {
  QInfo qi;
  const SetInfo si = set_info(a, n);
  qi.row0 = si.row0;
  qi.u0 = si.u0;
  qi.t = a.q_pos[n];
  qi.V = si.V;
  qi.n_ent = si.n_ent;
  qi.n_set = si.n_ent + si.n_w;
  qi.b = a.seq_id[n];
  qi.pad = 0;
  return qi;
}

// Staging of one key by its 16 threads: thread q writes the 16-byte chunks
// q, q+16, q+32, q+48 of the key's BF16 row (dims 8j .. 8j+7 for chunk j), so the
// 16 lanes of each LDS write cover one contiguous 256-byte span.
// An entry's chunk j < 56 comes from FP8 bytes 8j .. 8j+7 of its nope row, chunk
// 56 + i from BF16 dims 8i .. 8i+7 of its (already rotated) RoPE slice.
enum { kInvalid = 0, kEntry = 1, kWindow = 2 };

struct EntryRegs {
  u2 f0, f1, f2;    // FP8 chunks q, q+16, q+32
  u2 f3;            // FP8 chunk 48 + (q & 7)       (used by q < 8)
  u4 r3;            // BF16 RoPE dims 8(q & 7) ..   (used by q >= 8)
  float sc;
  int kind;
};

__device__ __forceinline__ int key_kind(const QInfo& qi, int p, int jrow, bool csa) {
  if (p < qi.n_ent) {
    const int64_t j = csa ? (int64_t)jrow : (int64_t)p;
    return (j >= 0 && j < qi.V) ? kEntry : kInvalid;
  }
  return p < qi.n_set ? kWindow : kInvalid;
}

// Loads of one key's share, issued without any branch so that they stay in flight
// while the previous chunk is computed: a key that is not a valid entry reads
// entry 0 of its sequence (the caller guarantees V >= 1) and is masked by `kind`.
// Paged caches add one dependent load per key (its page id; the 16 threads of a key
// read the same one).
__device__ __forceinline__ EntryRegs entry_load(const AttnArgs& a, const QInfo& qi, int p, int jrow, int q,
                                                bool csa) {
  EntryRegs e;
  e.kind = key_kind(qi, p, jrow, csa);
  const int64_t j = e.kind == kEntry ? (csa ? (int64_t)jrow : (int64_t)p) : 0;
  const int64_t row = cache_row(a.page_table, a.page_pitch, a.page_shift, qi.b, qi.row0, j);
  const char* nope = a.c_nope + row * a.c_nope_pitch + 8 * q;
  e.f0 = *reinterpret_cast<const u2*>(nope);
  e.f1 = *reinterpret_cast<const u2*>(nope + 128);
  e.f2 = *reinterpret_cast<const u2*>(nope + 256);
  e.f3 = *reinterpret_cast<const u2*>(nope + 384 - 8 * (q & 8));
  e.r3 = *reinterpret_cast<const u4*>(a.c_rope + row * a.c_rope_pitch + 16 * (q & 7));
  e.sc = a.c_scale[row];
  return e;
}

// entry_load with device-coherent 32-bit loads, which bypass the XCD's L2: the chunk
// that holds the entry this launch has just pooled reads it this way, so a line of
// that entry cached on this XCD before the pooling wrote it (448-byte FP8 rows and
// 4-byte scales share lines with the previous entry's) can never be returned
__device__ __forceinline__ uint32_t ld_dev32(const char* p) {
  return __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<char*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ EntryRegs entry_load_dev(const AttnArgs& a, const QInfo& qi, int p, int jrow, int q,
                                                    bool csa) {
  EntryRegs e;
  e.kind = key_kind(qi, p, jrow, csa);
  const int64_t j = e.kind == kEntry ? (csa ? (int64_t)jrow : (int64_t)p) : 0;
  const int64_t row = cache_row(a.page_table, a.page_pitch, a.page_shift, qi.b, qi.row0, j);
  const char* nope = a.c_nope + row * a.c_nope_pitch + 8 * q;
  const char* f3 = nope + 384 - 8 * (q & 8);
  const char* r3 = a.c_rope + row * a.c_rope_pitch + 16 * (q & 7);
  e.f0 = (u2){ld_dev32(nope), ld_dev32(nope + 4)};
  e.f1 = (u2){ld_dev32(nope + 128), ld_dev32(nope + 132)};
  e.f2 = (u2){ld_dev32(nope + 256), ld_dev32(nope + 260)};
  e.f3 = (u2){ld_dev32(f3), ld_dev32(f3 + 4)};
  e.r3 = (u4){ld_dev32(r3), ld_dev32(r3 + 4), ld_dev32(r3 + 8), ld_dev32(r3 + 12)};
  e.sc = __uint_as_float(ld_dev32(reinterpret_cast<const char*>(a.c_scale + row)));
  return e;
}

// rotate 8 BF16 dims of a window token's RoPE slice: `own` holds pair indices
// i0 .. i0+7, `mate` the other member of each pair; first = own is the first half
__device__ __forceinline__ u4 rope8(u4 own, u4 mate, int i0, bool first, int64_t u, const double* s_inv) {
  u4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float c0, s0, c1, s1;
    rope_cs(u, s_inv[i0 + 2 * w], &c0, &s0);
    rope_cs(u, s_inv[i0 + 2 * w + 1], &c1, &s1);
    const float o0 = bf16_to_f32((uint16_t)own[w]), o1 = bf16_to_f32((uint16_t)(own[w] >> 16));
    const float m0 = bf16_to_f32((uint16_t)mate[w]), m1 = bf16_to_f32((uint16_t)(mate[w] >> 16));
    // first half: x0 c - x1 s with x0 = own; second half: x0 s + x1 c with x1 = own
    out[w] = first ? pack_bf16x2(o0 * c0 - m0 * s0, o1 * c1 - m1 * s1)
                   : pack_bf16x2(m0 * s0 + o0 * c0, m1 * s1 + o1 * c1);
  }
  return out;
}

// write one key's 4 chunks (this thread's share) into the LDS row
__device__ __forceinline__ void key_commit(const AttnArgs& a, const QInfo& qi, int p, const EntryRegs& e, int q,
                                           u4* rowp, const double* s_inv) {
  if (e.kind == kEntry) {
    rowp[q] = cvt8(e.f0, e.sc);
    rowp[q + 16] = cvt8(e.f1, e.sc);
    rowp[q + 32] = cvt8(e.f2, e.sc);
    rowp[q + 48] = q < 8 ? cvt8(e.f3, e.sc) : e.r3;
  } else if (e.kind == kWindow) {
    const int64_t u = qi.u0 + (p - qi.n_ent);
    const u4* src = reinterpret_cast<const u4*>(a.win + ((int64_t)qi.b * a.win_cap + u % a.win_cap) * a.win_pitch);
    const u4 x0 = src[q], x1 = src[q + 16], x2 = src[q + 32], x3 = src[q + 48];
    rowp[q] = x0;
    rowp[q + 16] = x1;
    rowp[q + 32] = x2;
    if (q < 8) {
      rowp[q + 48] = x3;
    } else {
      // chunk 56 + m (m < 4: first halves, pairs 8m .. 8m+7) pairs with chunk 60 + m
      const int m = q - 8;
      const bool first = m < 4;
      const u4 mate = src[first ? q + 52 : q + 44];
      rowp[q + 48] = rope8(x3, mate, 8 * (m & 3), first, u, s_inv);
    }
  } else {
    const u4 z = {0u, 0u, 0u, 0u};
    rowp[q] = z; rowp[q + 16] = z; rowp[q + 32] = z; rowp[q + 48] = z;
  }
}

struct PartialPtrs {
  int* pref;    // [Nq + 1] chunk prefix, then [Nq + 1] = chunks per workgroup
  float* m;     // [slots, H]  running max, log2 units
  float* l;     // [slots, H]
  __bf16* o;    // [slots, H, D]  o / l of the run (0 where l = 0)
};

__host__ __device__ inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Flat: equal chunk ranges over the workgroups.  Query: one workgroup per query.
// Split: one workgroup per run (batches of more than kMaxDecodeQ queries).
// SplitFlat: equal shares of whole runs over the workgroups.
enum { kLayoutFlat = 0, kLayoutQuery = 1, kLayoutSplit = 2, kLayoutSplitFlat = 3 };

// partial slots: one per (workgroup, query) of a flattened launch, one per run of
// a fixed-split launch
__host__ __device__ inline size_t partial_slots(int Nq, int split_runs) {
  return split_runs > 0 ? (size_t)Nq * split_runs : (size_t)HCA_ATTN_GRID + Nq;
}

__host__ __device__ inline PartialPtrs partial_ptrs(void* ws, int Nq, int H, int split_runs) {
  PartialPtrs p;
  char* b = static_cast<char*>(ws);
  const size_t slots = partial_slots(Nq, split_runs);
  const size_t hdr = round256((size_t)(Nq + 2) * 4);
  const size_t ml = round256(slots * H * 4);
  p.pref = reinterpret_cast<int*>(b);
  p.m = reinterpret_cast<float*>(b + hdr);
  p.l = reinterpret_cast<float*>(b + hdr + ml);
  p.o = reinterpret_cast<__bf16*>(b + hdr + 2 * ml);
  return p;
}

__device__ __forceinline__ int find_query(const int* pref, int nq, int c) {
  // the query whose chunk range [pref[n], pref[n+1]) holds chunk c
  int lo = 0, hi = nq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// POOL (decode layouts Flat and SplitFlat): the grid's first pool_wgs workgroups pool
// one block each (HCA: a block's tokens complete its sequence's newest entry) and set
// their flags to the call's epoch; the rest run the attention plan over
// gridDim.x - pool_wgs workgroups, and the one that stages the chunk holding a query's
// newest entry V - 1 waits for every flag first.  The pooling workgroups lead the
// dispatch order, so they are running whenever a workgroup waits; the wait is bounded
// all the same.
typedef PoolSmem<kThreads, 16, false> AttnPoolSmem;       // blocks of m <= 128 tokens, no index stream

template <int layout, bool POOL>
__device__ __forceinline__ void attn_mqa_body(const AttnArgs& a, const PoolArgs& pool) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[KC * kKsPitch];
  __shared__ __attribute__((aligned(16))) float4 s_sx[8][4][64];
  __shared__ __attribute__((aligned(16))) __bf16 Pt[8][KC * kPtPitch];
  __shared__ int32_t s_idx[kIdxWin];
  __shared__ QInfo s_qi[kMaxDecodeQ];
  __shared__ int s_pref[kMaxDecodeQ + 1];
  __shared__ int s_rpref[layout == kLayoutSplitFlat ? kMaxDecodeQ + 1 : 1];   // run prefix
  __shared__ int s_wsum[16];
  __shared__ double s_inv[32];
  __shared__ uint8_t s_kval[KC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int NHG = a.H / 16;
  const int hg = wave & 3, dh = wave >> 2;
  const bool active = hg < NHG;
  const bool csa = a.mode == HCA_MODE_CSA;
  constexpr bool per_query = layout == kLayoutQuery || layout == kLayoutSplit;
  constexpr bool split_flat = layout == kLayoutSplitFlat;
  constexpr bool fixed_split = layout == kLayoutSplit || layout == kLayoutSplitFlat;

  static_assert(sizeof(AttnPoolSmem) <= sizeof(Ks), "a pooling workgroup's LDS fits in the key tile");
  if constexpr (POOL) {
    if ((int)blockIdx.x < a.pool_wgs) {
      if ((int)blockIdx.x < pool.n_blocks) {
        pool_d512_block<kThreads, 16, false>(pool, blockIdx.x, *reinterpret_cast<AttnPoolSmem*>(Ks));
        flag_set(a.flags + blockIdx.x, a.epoch);   // stores written back, then the block's flag
      }
      return;                                       // uniform over the workgroup
    }
  }
  // this workgroup's place in the attention plan, and the plan's workgroup count
  const int bid = (int)blockIdx.x - (POOL ? a.pool_wgs : 0);
  const int nwg = (int)gridDim.x - (POOL ? a.pool_wgs : 0);
  // the chunk that holds a query's newest entry (HCA: set position n_ent - 1) waits
  // for the pooling, then reads its entries with device-coherent loads
  auto pool_chunk = [&](const QInfo& qs, int p) {
    return POOL && !csa && qs.n_ent > 0 && p <= qs.n_ent - 1 && qs.n_ent - 1 < p + KC;
  };
  auto pool_wait = [&]() {
    if (wave == 0) flags_wait(a.flags, a.pool_wgs, a.epoch);   // every block's flag, then acquire
    __syncthreads();
  };

  if (tid < 32) s_inv[tid] = a.inv_turn[tid];       // turns per position
  // ---- the chunk list and this workgroup's run [c0, c1)
  int nq_local, qbase, c0, c1;
  int run = 0, n_runs = 1;                          // fixed split: this run, the query's runs
  PartialPtrs pp{};
  if (per_query) {
    qbase = bid;
    if constexpr (layout == kLayoutSplit) {
      qbase = bid / a.split_runs;
      run = bid - qbase * a.split_runs;
    }
    nq_local = 1;
    if (tid == 0) {
      const QInfo qi = query_info(a, qbase);
      s_qi[0] = qi;
      s_pref[0] = 0;
      s_pref[1] = (qi.n_set + KC - 1) / KC;
    }
    __syncthreads();
    c0 = 0;
    c1 = s_pref[1];
    if constexpr (layout == kLayoutSplit) {
      n_runs = (c1 + a.split_chunks - 1) / a.split_chunks;
      c0 = run * a.split_chunks;
      c1 = min(c0 + a.split_chunks, c1);
      pp = partial_ptrs(a.workspace, a.Nq, a.H, a.split_runs);
    }
  } else {
    qbase = 0;
    nq_local = a.Nq;
    // the chunk counts need only the positions; the dependent cache-row load is
    // in flight during the scan and stored with the rest of the query record
    int cnt = 0, nr = 0;
    int64_t row0 = 0;
    if (tid < a.Nq) {
      const int b = a.seq_id[tid];
      row0 = a.page_shift < 0 && a.cache_row_start ? a.cache_row_start[b] : 0;   // paged / window only
      QInfo qi = query_info_pos(a, tid, b);
      s_qi[tid] = qi;
      cnt = (qi.n_set + KC - 1) / KC;
      if (split_flat) nr = (cnt + a.split_chunks - 1) / a.split_chunks;
    }
    int x = cnt, xr = nr;                  // inclusive scans of chunks (and runs)
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
      if constexpr (split_flat) {
        const int yr = __shfl_up(xr, o, 64);
        if (lane >= o) xr += yr;
      }
    }
    if (lane == 63) { s_wsum[wave] = x; if (split_flat) s_wsum[8 + wave] = xr; }
    __syncthreads();
    int base = 0, rbase = 0;
    for (int w = 0; w < wave; ++w) { base += s_wsum[w]; if (split_flat) rbase += s_wsum[8 + w]; }
    if (tid < a.Nq) { s_pref[tid + 1] = base + x; if (split_flat) s_rpref[tid + 1] = rbase + xr; }
    if (tid == 0) { s_pref[0] = 0; if (split_flat) s_rpref[0] = 0; }
    __syncthreads();
    const int total = s_pref[a.Nq];
    if constexpr (split_flat) {
      // whole runs [r0, r1): a run is never cut, so its partial depends on its query alone
      const int runs = s_rpref[a.Nq];
      const int per = (runs + nwg - 1) / nwg;
      const int r0 = bid * per, r1 = min(r0 + per, runs);
      c0 = c1 = 0;
      if (r0 < r1) {
        const int n0 = find_query(s_rpref, a.Nq, r0), n1 = find_query(s_rpref, a.Nq, r1 - 1);
        c0 = s_pref[n0] + (r0 - s_rpref[n0]) * a.split_chunks;
        c1 = min(s_pref[n1] + (r1 - s_rpref[n1]) * a.split_chunks, s_pref[n1 + 1]);
      }
      pp = partial_ptrs(a.workspace, a.Nq, a.H, a.split_runs);
      // a query with no run (empty set: nothing visible, no window) gets the sink
      // alone, o = 0, from workgroup 0 (no run and no combine writes it)
      if (bid == 0) {
        for (int nq = 0; nq < a.Nq; ++nq) {
          if (s_rpref[nq + 1] != s_rpref[nq]) continue;       // uniform
          __bf16* o = reinterpret_cast<__bf16*>(a.o) + (int64_t)nq * a.H * kD;
          for (int i = tid; i < a.H * kD; i += kThreads) o[i] = (__bf16)0.0f;
          if (a.lse && tid < a.H) a.lse[(int64_t)nq * a.H + tid] = a.sink[tid];
        }
      }
    } else {
      int per = (total + nwg - 1) / nwg;
      if (per < HCA_ATTN_MIN_CHUNKS) per = HCA_ATTN_MIN_CHUNKS;
      pp = partial_ptrs(a.workspace, a.Nq, a.H, 0);
      if (bid == 0) {
        for (int i = tid; i <= a.Nq; i += kThreads) pp.pref[i] = s_pref[i];
        if (tid == 0) pp.pref[a.Nq + 1] = per;
      }
      c0 = bid * per;
      c1 = min(c0 + per, total);
    }
    if (tid < a.Nq) s_qi[tid].row0 = row0;
  }
  if (c0 >= c1) {                           // fixed split: runs past the query's last
    if (per_query && run == 0 && active) {  // empty set: the sink alone, o = 0
      const int n = qbase;
      const int hrow0 = 16 * hg + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = hrow0 + i;
        __bf16* o = reinterpret_cast<__bf16*>(a.o) + ((int64_t)n * a.H + h) * kD + 256 * dh;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) o[16 * dt + r] = (__bf16)0.0f;
        if (a.lse && r == 0 && dh == 0) a.lse[(int64_t)n * a.H + h] = a.sink[h];
      }
    }
    return;                                 // uniform over the workgroup
  }

  // index-list window: positions of chunks [cw, cw + kIdxWin / KC) of this run
  auto fill_idx = [&](int cw) {
    for (int e = tid; e < kIdxWin; e += kThreads) {
      const int cc = cw + e / KC;
      int v = -1;
      if (cc < c1) {
        const int nl = per_query ? 0 : find_query(s_pref, nq_local, cc);
        const int p = (cc - s_pref[nl]) * KC + (e % KC);
        if (p < s_qi[nl].n_ent) v = a.idx[(int64_t)(qbase + nl) * a.k + p];
      }
      s_idx[e] = v;
    }
  };

  // staging: this thread's share q of keys kk0 and kk0 + 32
  const int q16 = tid & 15, kk0 = tid >> 4, kk1 = kk0 + 32;
  u4* const row0p = reinterpret_cast<u4*>(Ks + kk0 * kKsPitch);
  u4* const row1p = reinterpret_cast<u4*>(Ks + kk1 * kKsPitch);
  EntryRegs e0, e1;
  int idx_win = c0;
  int ns = per_query ? 0 : find_query(s_pref, nq_local, c0);   // query of the staged chunk
  int p_st = (c0 - s_pref[ns]) * KC;                              // its first set position
#define HCA_ISSUE()                                                                            \
  do {                                                                                         \
    const QInfo& qs_ = s_qi[ns];                                                               \
    const int ib_ = (c_st - idx_win) * KC;                                                     \
    const int j0_ = csa ? s_idx[ib_ + kk0] : 0, j1_ = csa ? s_idx[ib_ + kk1] : 0;              \
    if (p_st < qs_.n_ent && pool_chunk(qs_, p_st)) {   /* uniform: the newly pooled entry, */ \
      defer_ = true;                               /* loaded after the current chunk */        \
    } else if (p_st < qs_.n_ent) {                 /* uniform: the chunk holds entries */      \
      e0 = entry_load(a, qs_, p_st + kk0, j0_, q16, csa);                                      \
      e1 = entry_load(a, qs_, p_st + kk1, j1_, q16, csa);                                      \
    } else {                                                                                   \
      e0.kind = key_kind(qs_, p_st + kk0, j0_, csa);                                           \
      e1.kind = key_kind(qs_, p_st + kk1, j1_, csa);                                           \
    }                                                                                          \
  } while (0)
// the deferred chunk (it holds the entry this launch pools): wait for the pooling once
// the current chunk has been computed, then read its entries with coherent loads
#define HCA_DEFERRED()                                                                         \
  do {                                                                                         \
    if (defer_) {                                  /* uniform */                               \
      pool_wait();                                                                             \
      const QInfo& qs_ = s_qi[ns];                                                             \
      e0 = entry_load_dev(a, qs_, p_st + kk0, 0, q16, csa);                                    \
      e1 = entry_load_dev(a, qs_, p_st + kk1, 0, q16, csa);                                    \
      defer_ = false;                                                                          \
    }                                                                                          \
  } while (0)
#define HCA_COMMIT()                                                                           \
  do {                                                                                         \
    const QInfo& qs_ = s_qi[ns];                                                               \
    key_commit(a, qs_, p_st + kk0, e0, q16, row0p, s_inv);                                     \
    key_commit(a, qs_, p_st + kk1, e1, q16, row1p, s_inv);                                     \
    if (q16 == 0) { s_kval[kk0] = e0.kind != kInvalid; s_kval[kk1] = e1.kind != kInvalid; }    \
    __builtin_amdgcn_s_waitcnt(0x0F70);            /* vmcnt(0): no load of this chunk lingers */ \
  } while (0)

  if (csa) {
    fill_idx(c0);
  }
  __syncthreads();                                   // s_inv, s_idx, s_qi

  // ---- per-query state
  int nl = ns;
  int seg0 = c0;                                     // first chunk of the current query segment
  v8bf qa[8];
  v4f acc[16];
  float m_run[4], l_run[4];
  const float qscale = a.tau * (float)kLog2e;        // logits in log2 units
  // the query's rows are requested early (in flight with key loads) and rotated
  // and made current once they have arrived
  auto q_issue = [&](int nloc) {
    const int n = qbase + nloc;
    const int head = 16 * hg + r;
    const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) + ((int64_t)n * a.H + head) * kD + 256 * dh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qa[s] = *reinterpret_cast<const v8bf*>(qrow + 32 * s + 8 * g);
  };
  auto q_finish = [&](int nloc) {
    if (dh == 1) {
      // rotate the RoPE pairs (448 + i, 480 + i), i = 8g + e, held in k-steps 6 / 7
      const int64_t t = s_qi[nloc].t;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float c, s;
        rope_cs(t, s_inv[8 * g + e], &c, &s);
        const float x0 = (float)qa[6][e], x1 = (float)qa[7][e];
        qa[6][e] = (__bf16)(x0 * c - x1 * s);
        qa[7][e] = (__bf16)(x0 * s + x1 * c);
      }
    }
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) acc[dt] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  };
  int c_st = c0;
  bool defer_ = false;
  HCA_ISSUE();
  if (active) q_issue(nl);                           // in flight with the first chunk's keys
  HCA_DEFERRED();
  HCA_COMMIT();                                      // (waits for both)
  if (active) q_finish(nl);
  __syncthreads();                                   // first tile

  // per-lane LDS read bases: QK rows 16kt + r at dims 256dh + 8g (+32s);
  // transposed reads rows 8g + lr (+32ks, +4) at dims 256dh + lc (+16dt)
  const int lr = r >> 2, lc = 4 * (r & 3);
  const __bf16* kq_base = Ks + r * kKsPitch + 256 * dh + 8 * g;
  const __bf16* kv_base = Ks + (8 * g + lr) * kKsPitch + 256 * dh + lc;
  __bf16* const pt = Pt[wave];

  for (int c = c0; c < c1; ++c) {
    const bool more = c + 1 < c1;
    if (more) {
      c_st = c + 1;
      while (s_pref[ns + 1] <= c_st) ++ns;           // uniform
      p_st = (c_st - s_pref[ns]) * KC;
      if (csa && c_st - idx_win >= kIdxWin / KC) {   // next window of the index list
        __syncthreads();
        idx_win = c_st;
        fill_idx(idx_win);
        __syncthreads();
      }
      HCA_ISSUE();
    }
    v4f sc[4];
    if (active) {
      // ---- partial logits over this wave's 256 dims: 4 key tiles of 16
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sc[kt] = (v4f){0.f, 0.f, 0.f, 0.f};
      // the reads of k-step s+1 are in flight while k-step s multiplies
      v8bf kb0[4], kb1[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kb0[kt] = *reinterpret_cast<const v8bf*>(kq_base + 16 * kt * kKsPitch);
#pragma unroll
      for (int s = 0; s < 8; s += 2) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          kb1[kt] = *reinterpret_cast<const v8bf*>(kq_base + 16 * kt * kKsPitch + 32 * (s + 1));
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], kb0[kt], sc[kt], 0, 0, 0);
        if (s + 2 < 8) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            kb0[kt] = *reinterpret_cast<const v8bf*>(kq_base + 16 * kt * kKsPitch + 32 * (s + 2));
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s + 1], kb1[kt], sc[kt], 0, 0, 0);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s_sx[wave][kt][lane] = make_float4(sc[kt][0], sc[kt][1], sc[kt][2], sc[kt][3]);
    }
    // a segment ends with its query's chunks, or (fixed split) with its run
    const bool last_of_query = !more || s_pref[nl + 1] == c + 1 || (fixed_split && c + 1 - seg0 == a.split_chunks);
    if (more && last_of_query && active) q_issue(ns);  // the next query's rows, in flight from here
    __syncthreads();
    if (active) {
      // full logits S = S_dh0 + S_dh1 (the same sum in both waves), in log2 units;
      // lane (r, g) holds key 16kt + r of head rows 4g + i
      float x[4][4];
      bool need = false;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const float4 o4 = s_sx[wave ^ 4][kt][lane];
        const float ov[4] = {o4.x, o4.y, o4.z, o4.w};
        const bool kv = s_kval[16 * kt + r];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float S = dh == 0 ? sc[kt][i] + ov[i] : ov[i] + sc[kt][i];
          x[kt][i] = kv ? S * qscale : -INFINITY;
          need |= x[kt][i] > m_run[i] + 8.0f;
        }
      }
      // m_run is a reference maximum per head row: probabilities are
      // exp2(x - m_run) and o is rescaled only when a logit exceeds the reference
      // by more than 2^8 (wave-uniform branch); the final normalization makes the
      // choice of reference exact.
      if (__builtin_amdgcn_read_exec() & __ballot(need)) {
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float mx = fmaxf(fmaxf(x[0][i], x[1][i]), fmaxf(x[2][i], x[3][i]));
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
          const float m_new = fmaxf(m_run[i], mx);
          alpha[i] = (m_run[i] == -INFINITY) ? 0.0f : exp2f(m_run[i] - m_new);
          l_run[i] *= alpha[i];
          m_run[i] = m_new;
        }
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
          acc[dt][0] *= alpha[0]; acc[dt][1] *= alpha[1];
          acc[dt][2] *= alpha[2]; acc[dt][3] *= alpha[3];
        }
      }
      // P^T in LDS: row = key, this lane's 4 heads in one 8-byte write
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        float ev[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ev[i] = (m_run[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[kt][i] - m_run[i]);
          l_run[i] += ev[i];
        }
        *reinterpret_cast<u2*>(pt + (16 * kt + r) * kPtPitch + 4 * g) =
            (u2){pack_bf16x2(ev[0], ev[1]), pack_bf16x2(ev[2], ev[3])};
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // O += P V over 2 k-steps of 32 keys; both operands by transposed LDS reads
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const __bf16* pb = pt + (32 * ks + 8 * g + lr) * kPtPitch + lc;
        v4s p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)pb);
        v4s p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)(pb + 4 * kPtPitch));
        v8bf pa;
        __builtin_memcpy(&pa, &p0, 8);
        __builtin_memcpy(reinterpret_cast<char*>(&pa) + 8, &p1, 8);
        const __bf16* vbase = kv_base + 32 * ks * kKsPitch;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
          const __bf16* b0 = vbase + 16 * dt;
          v4s t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)b0);
          v4s t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)(b0 + 4 * kKsPitch));
          v8bf vb;
          __builtin_memcpy(&vb, &t0, 8);
          __builtin_memcpy(reinterpret_cast<char*>(&vb) + 8, &t1, 8);
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[dt], 0, 0, 0);
        }
        // P^T and the first two V^T tiles, then each product with the reads of the
        // tile two ahead in flight
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
        for (int dt = 0; dt < 14; ++dt) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      }
    }
    // ---- end of this query's chunks in the run: finish it
    if (last_of_query) {
      if (active) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float l = l_run[i];
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o, 64);
          l_run[i] = l;
        }
        const int n = qbase + nl;
        const int hrow0 = 16 * hg + 4 * g;
        bool direct;
        if constexpr (layout == kLayoutQuery) direct = true;
        else if constexpr (layout == kLayoutSplit) direct = n_runs == 1;
        else if constexpr (split_flat) direct = s_rpref[nl + 1] - s_rpref[nl] == 1;
        else direct = s_pref[nl] >= c0 && s_pref[nl + 1] <= c1;
        if (direct) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = hrow0 + i;
            const float sig = a.sink[h] * (float)kLog2e;
            const float M = fmaxf(sig, m_run[i]);
            const float sc_o = exp2f(m_run[i] - M);
            const float den = exp2f(sig - M) + l_run[i] * sc_o;
            const float f = sc_o / den;
            __bf16* o = reinterpret_cast<__bf16*>(a.o) + ((int64_t)n * a.H + h) * kD + 256 * dh;
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) o[16 * dt + r] = (__bf16)(acc[dt][i] * f);
            if (a.lse && r == 0 && dh == 0) a.lse[(int64_t)n * a.H + h] = (M + log2f(den)) / (float)kLog2e;
          }
        } else {
          size_t slot;
          if constexpr (fixed_split) slot = (size_t)n * a.split_runs + (seg0 - s_pref[nl]) / a.split_chunks;
          else slot = (size_t)bid + n;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = hrow0 + i;
            const size_t base = slot * a.H + h;
            if (r == 0 && dh == 0) { pp.m[base] = m_run[i]; pp.l[base] = l_run[i]; }
            const float f = l_run[i] > 0.0f ? 1.0f / l_run[i] : 0.0f;
            __bf16* o = pp.o + base * kD + 256 * dh;
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) o[16 * dt + r] = (__bf16)(acc[dt][i] * f);
          }
        }
      }
    }
    if (more) {
      HCA_DEFERRED();
      __syncthreads();                     // every wave is done with Ks, Pt, s_sx
      HCA_COMMIT();                        // (also waits for the next query's rows)
      if (last_of_query) {
        if constexpr (fixed_split) seg0 = c + 1;
        nl = ns;                           // the staged chunk's query is next (or its next run)
        if (active) q_finish(nl);
      }
      __syncthreads();
    }
  }
}

template <int layout>
__global__ void __launch_bounds__(kThreads) attn_mqa_kernel(AttnArgs a) {
  const PoolArgs none{};
  attn_mqa_body<layout, false>(a, none);
}

// the same attention with the step's pooling in the leading workgroups (decode)
template <int layout>
__global__ void __launch_bounds__(kThreads) attn_pool_kernel(AttnArgs a, PoolArgs p) {
  attn_mqa_body<layout, true>(a, p);
}

#undef HCA_ISSUE
#undef HCA_DEFERRED
#undef HCA_COMMIT

// merge the runs of one (query, head) in run order, with the sink: run s holds
// (m_s, l_s, o_s / l_s), so o = sum_s w_s (o_s / l_s) / (e^(sigma - M) + sum_s w_s)
// with w_s = 2^(m_s - M) l_s
// Fixed split (split_runs > 0): query n's runs are slots n * split_runs + s, s <
// its run count; the attention kernel has already finished queries with one run.
// One wave per (query, head, P-th part of the dims), four heads per workgroup: every
// wave reduces the runs' (max, sum) itself with cross-lane operations (lane t holds
// runs t, t + 64, ...; its own runs in order, then a fixed butterfly), the weights go
// through the wave's own LDS row, and lane t merges 8 / P consecutive dims of its part
// (part blockIdx.z) of every run in run order.  With very few queries (a grid under
// half the CUs, e.g. 4 queries of 64 heads merging about 63 runs each) the dims are
// split in four, so 4x the workgroups, and 2x the runs per wave, have their rows in
// flight; each element's sum is the same.
#ifndef HCA_COMBINE_SPLIT_BELOW
#define HCA_COMBINE_SPLIT_BELOW 128
#endif
constexpr int kCombineSplitBelow = HCA_COMBINE_SPLIT_BELOW;   // workgroups of the unsplit grid
template <int P>
__global__ void __launch_bounds__(256) combine_kernel(AttnArgs a) {
  static_assert(P == 1 || P == 4, "dims per lane: 8 or 2");
  constexpr int W = 4 / P;                                // 32-bit words (2 dims each) per lane and run
  constexpr int kBatch = P == 1 ? 16 : 32;                // runs whose rows are in flight together
  __shared__ float s_w[4][kMaxRuns];
  const int n = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;                    // H is a multiple of 16
  const int d0 = (kD / P) * blockIdx.z + 2 * W * lane;    // this lane's first dim
  PartialPtrs pp = partial_ptrs(a.workspace, a.Nq, a.H, a.split_runs);
  const float sig = a.sink[h] * (float)kLog2e;
  __bf16* out = reinterpret_cast<__bf16*>(a.o) + ((int64_t)n * a.H + h) * kD;
  int S;                                   // runs to merge
  size_t slot0;
  const int cnt = a.split_runs > 0 ? (query_info(a, n).n_set + KC - 1) / KC : pp.pref[n + 1] - pp.pref[n];
  if (cnt == 0) {                          // empty set (no window, nothing visible): the sink alone, o = 0
    if (a.split_runs > 0) return;          // written by the attention kernel
#pragma unroll
    for (int e = 0; e < W; ++e) reinterpret_cast<uint32_t*>(out + d0)[e] = 0u;
    if (a.lse && blockIdx.z == 0 && lane == 0) a.lse[(int64_t)n * a.H + h] = a.sink[h];
    return;
  }
  if (a.split_runs > 0) {
    S = (cnt + a.split_chunks - 1) / a.split_chunks;
    if (S <= 1) return;                    // finished by its single run
    slot0 = (size_t)n * a.split_runs * a.H + h;
  } else {
    const int cb = pp.pref[n], ce = pp.pref[n + 1], per = pp.pref[a.Nq + 1];
    const int w0 = cb / per, w1 = (ce - 1) / per;
    if (w0 == w1) return;                  // finished by its single run
    S = w1 - w0 + 1;                       // <= the number of workgroups
    slot0 = ((size_t)w0 + n) * a.H + h;
  }
  const size_t sstride = (size_t)a.H;
  float mr[kMaxRuns / 64], lr[kMaxRuns / 64];
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < kMaxRuns / 64; ++r) {
    const int sidx = lane + 64 * r;
    mr[r] = -INFINITY;
    lr[r] = 0.0f;
    if (sidx < S) { mr[r] = pp.m[slot0 + sidx * sstride]; lr[r] = pp.l[slot0 + sidx * sstride]; }
    mx = fmaxf(mx, mr[r]);
  }
  const float M = fmaxf(wave_max(mx), sig);
  float ws = 0.0f;                         // this lane's runs in order, then the butterfly
#pragma unroll
  for (int r = 0; r < kMaxRuns / 64; ++r) {
    const int sidx = lane + 64 * r;
    if (sidx < S) {
      const float w = exp2f(mr[r] - M) * lr[r];
      s_w[wave][sidx] = w;
      ws += w;
    }
  }
  const float den = exp2f(sig - M) + wave_sum(ws);
  const float inv = 1.0f / den;
  // the wave's own LDS writes above are complete before these reads (in-order LDS)
  const __bf16* po = pp.o + slot0 * kD + d0;
  const size_t ostride = sstride * kD;
  float acc[2 * W];
#pragma unroll
  for (int e = 0; e < 2 * W; ++e) acc[e] = 0.f;
  // kBatch runs' rows requested at once, then added in run order (the order, and so
  // the bits, do not depend on the batch or the split)
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    uint32_t v[kBatch][W];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(po + (size_t)(s0 + u) * ostride);
      if constexpr (W == 4) {
        const uint4 q = s0 + u < S ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
        const uint32_t* qw = &q.x;
#pragma unroll
        for (int e = 0; e < W; ++e) v[u][e] = qw[e];
      } else {
        v[u][0] = s0 + u < S ? *src : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u < S) {
        const float w = s_w[wave][s0 + u];
#pragma unroll
        for (int e = 0; e < W; ++e) {
          acc[2 * e] += bf16_to_f32((uint16_t)v[u][e]) * w;
          acc[2 * e + 1] += bf16_to_f32((uint16_t)(v[u][e] >> 16)) * w;
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < W; ++e) reinterpret_cast<uint32_t*>(out + d0)[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  if (a.lse && blockIdx.z == 0 && lane == 0) a.lse[(int64_t)n * a.H + h] = (M + log2f(den)) / (float)kLog2e;
}

void launch_combine(const AttnArgs& a, hipStream_t s) {
  const int wgs = a.Nq * (a.H / 4);
  if (wgs < kCombineSplitBelow) hipLaunchKernelGGL(combine_kernel<4>, dim3(a.Nq, a.H / 4, 4), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(combine_kernel<1>, dim3(a.Nq, a.H / 4, 1), dim3(256), 0, s, a);
}

// Decode layout: few queries spread over one flattened chunk list (chunk counts
// must stay far from int overflow); otherwise one workgroup per query.
bool decode_layout(int Nq, int prefill, int mode, int k, int n_win, int64_t max_visible) {
  const int64_t n_ent = mode == HCA_MODE_CSA ? (k < max_visible ? (int64_t)k : max_visible) : max_visible;
  const int64_t chunks = (n_ent + n_win + KC - 1) / KC;
  return !prefill && Nq <= kMaxDecodeQ && (int64_t)Nq * chunks < (1LL << 30);
}

}  // namespace

int64_t attention_max_chunks(int mode, int k, int n_win, int64_t max_visible) {
  const int64_t n_ent = mode == HCA_MODE_CSA ? (k < max_visible ? (int64_t)k : max_visible) : max_visible;
  return (n_ent + n_win + KC - 1) / KC;
}

int64_t attention_split_runs(int mode, int k, int n_win, int64_t max_visible, int split_chunks) {
  if (split_chunks <= 0) return 0;
  return (attention_max_chunks(mode, k, n_win, max_visible) + split_chunks - 1) / split_chunks;
}

int attention_max_runs() { return kMaxRuns; }

// ---------------------------------------------------------------- static scratch
// The scratch memory of the allocation-free decode entry point: one array per GPU,
// held from the library's load until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: its device address comes
// from hipGetSymbolAddress, once per device with that device current, and only that
// address is handed to kernels.
namespace {
constexpr size_t kStaticScratchBytes = (size_t)40 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

size_t attention_static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t attention_static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {
constexpr int kMaxAttnPoolBlocks = 64;     // blocks one fused attention launch pools at most
// bytes of the split partials (the prefix header, max and sum, o); the fused pooling's
// flags follow them
size_t partial_bytes(int Nq, int H, int runs) {
  const size_t slots = partial_slots(Nq, runs);
  return round256((size_t)(Nq + 2) * 4) + 2 * round256(slots * H * 4) + round256(slots * H * kD * 2);
}

// The step's pooling can ride in the attention launch: a decode plan shared over the
// workgroups (few queries), BF16 rows of 512 dims without an index stream in blocks of
// 17 to 128 tokens (the configuration the pooling kernel itself uses for them: the same
// bits), and few enough blocks that pooling and attention workgroups are resident
// together.
bool attn_pool_fusable(const AttnArgs& a, const PoolArgs& p) {
  if (a.io_f32 || a.prefill || a.mode == HCA_MODE_CSA || !a.workspace) return false;
  if (!decode_layout(a.Nq, a.prefill, a.mode, a.k, a.n_win, a.max_visible)) return false;
  return pool_fast_path(p) && p.m > 16 && p.m <= 128 && p.idx_fmt < 0 && p.n_blocks <= kMaxAttnPoolBlocks;
}
}  // namespace

size_t attention_workspace_bytes(int Nq, int H, int D, int mode, int k, int n_win,
                                 int64_t max_visible, int io_f32, int prefill, int split_chunks) {
  (void)D;
  if (io_f32 || prefill) return 0;
  const int64_t runs = attention_split_runs(mode, k, n_win, max_visible, split_chunks);
  if (runs <= 0 && !decode_layout(Nq, prefill, mode, k, n_win, max_visible)) return 0;
  return partial_bytes(Nq, H, (int)runs) + 8 * kMaxAttnPoolBlocks;   // + the fused pooling's flags
}

hipError_t launch_attention(const AttnArgs& a0, hipStream_t s, const PoolArgs* pool) {
  if (pool && pool->n_blocks == 0) pool = nullptr;
  if (pool && (a0.Nq == 0 || !attn_pool_fusable(a0, *pool))) {   // pooled by its own launch, first
    const hipError_t e = launch_pool(*pool, s);
    if (e != hipSuccess) return e;
    pool = nullptr;
  }
  if (a0.Nq == 0) return hipSuccess;
  AttnArgs a = a0;
  if (pool) {
    // the blocks' epoch flags live after the partials (no clearing: a fresh epoch per call)
    a.flags = reinterpret_cast<uint64_t*>(static_cast<char*>(a.workspace) +
                                          partial_bytes(a.Nq, a.H, a.split_runs > 0 ? a.split_runs : 0));
    a.pool_wgs = pool->n_blocks;
    a.epoch = fused_epoch();
  }
  if (a.io_f32) {
    if (a.prof_begin) (void)hipEventRecord(a.prof_begin, s);
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.Nq, a.H), dim3(256), 0, s, a);
    if (a.prof_end) (void)hipEventRecord(a.prof_end, s);
    return hipGetLastError();
  }
  if (a.split_runs > 0 && !a.prefill) {
    // few queries: whole runs shared over the workgroups; otherwise one workgroup per run
    const bool flat = decode_layout(a.Nq, a.prefill, a.mode, a.k, a.n_win, a.max_visible);
    const unsigned grid = flat ? HCA_ATTN_GRID : (unsigned)((int64_t)a.Nq * a.split_runs);
    if (a.prof_begin) (void)hipEventRecord(a.prof_begin, s);
    if (pool)          // one CU each: the pooling workgroups take the place of plan workgroups
      hipLaunchKernelGGL(attn_pool_kernel<kLayoutSplitFlat>, dim3(HCA_ATTN_GRID), dim3(kThreads), 0, s, a, *pool);
    else if (flat) hipLaunchKernelGGL(attn_mqa_kernel<kLayoutSplitFlat>, dim3(grid), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(attn_mqa_kernel<kLayoutSplit>, dim3(grid), dim3(kThreads), 0, s, a);
    if (a.prof_end) (void)hipEventRecord(a.prof_end, s);
    if (a.split_runs > 1) launch_combine(a, s);
    return hipGetLastError();
  }
  AttnArgs b = a;
  b.split_runs = 0;                        // prefill never splits a query
  const bool dec = decode_layout(b.Nq, b.prefill, b.mode, b.k, b.n_win, b.max_visible);
  if (b.prof_begin) (void)hipEventRecord(b.prof_begin, s);
  if (pool)            // one CU each: the pooling workgroups take the place of plan workgroups
    hipLaunchKernelGGL(attn_pool_kernel<kLayoutFlat>, dim3(HCA_ATTN_GRID), dim3(kThreads), 0, s, b, *pool);
  else if (dec) hipLaunchKernelGGL(attn_mqa_kernel<kLayoutFlat>, dim3(HCA_ATTN_GRID), dim3(kThreads), 0, s, b);
  else hipLaunchKernelGGL(attn_mqa_kernel<kLayoutQuery>, dim3(b.Nq), dim3(kThreads), 0, s, b);
  if (b.prof_end) (void)hipEventRecord(b.prof_end, s);
  if (dec) launch_combine(b, s);
  return hipGetLastError();
}

}  // namespace hca
