// Lightning indexer scores and per-query top-k selection.
//
// "DeepSeek V4: How They Crushed the Million-Token Memory Problem"
// (sameershanbhag.com), "Two kinds of memory instead of one": the indexer scores
// compressed entries with ReLU-scored multi-head dot products (in FP4) and keeps the
// top-k.  "DeepSeek V4 infrastructure" (volanea.com), "Compression only works if the
// attention path is engineered end to end": a sparse selector is only cheap if its
// scoring path does not eat the memory bandwidth - the key stream is read once,
// coalesced, and everything after the dot products stays in registers and LDS.
//
// Score of query n and entry j:  I = sum_h w[n,h] * max(q[n,h] . k[j], 0).
// Quantized operands: every head dot is exact in binary32.  FP8 operands are widened
// to BF16 (exact) and multiplied on BF16 MFMA, whose accumulation keeps the exact
// value of any dot whose partial sums are binary32 numbers; MXFP4 operands use the
// scaled FP4 MFMA, exact under the same condition.  (The FP8 MFMA is not used: it
// sums groups of eight products in a narrower window and can drop low-order bits.)
// The head sum follows one fixed order in binary32, each head one fused
// multiply-add (a single rounding):
//     S_u <- fl(w_h * max(d_h, +0) + S_u), from S_u = +0, over
//            h = 32T + 8(i / 4) + 4u + (i % 4) (T ascending, then i = 0..15),
//            for the two halves u = 0, 1;      I = fl(S_0 + S_1)
// which is exactly the order the 32x32 MFMA output layout produces: lane (j, u)
// holds heads 32T + 8(i / 4) + 4u + (i % 4) of entry j in register i, and one
// butterfly add combines the halves.  (32x32 products run at twice the rate of
// 16x16 ones on this hardware.)
//
// Selection: exact radix select on the orderable 32-bit key of each score, lower
// index first among equal scores, output in ascending index order.
#include <map>
#include <mutex>
#include <utility>

#include "device_common.hpp"
#include "hca_internal.hpp"
#include "../../include/hca.h"
#include "pool_block.hpp"

namespace hca {

namespace {

constexpr int kScoreThreads = 256;        // 4 waves
constexpr int kBins = 2048;               // first radix digit: key bits 31..21
constexpr int kSelectThreads = 1024;
constexpr int kSmallV = 4096;

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Device-coherent word access (relaxed, device scope): what one workgroup stores
// this way is seen by another's loads once the store has completed, with no cache
// write-back or invalidation (those make a device-scope fence cost microseconds).
__device__ __forceinline__ uint32_t ld_dev(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int64_t visible(const IndexerArgs& a, int n) {
  int64_t v = (a.q_pos[n] + 1) / a.m;
  return v < a.max_visible ? v : a.max_visible;
}

// 8 FP8 codes (little-endian in two dwords) -> 8 BF16 values (exact widening)
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  v2bf a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
  v2bf a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
  v2bf a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
  v2bf a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
  v8bf r;
  r[0] = a0[0]; r[1] = a0[1]; r[2] = a1[0]; r[3] = a1[1];
  r[4] = a2[0]; r[5] = a2[1]; r[6] = a3[0]; r[7] = a3[1];
  return r;
}

// Exclusive scan over the threads of a workgroup of NT threads (order = thread id).
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  constexpr int NWV = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < NWV ? s_wave[lane] : 0;
    uint32_t u = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      uint32_t y = __shfl_up(u, o, 64);
      if (lane >= o) u += y;
    }
    if (lane < NWV) s_wave[lane] = u - t;
    if (lane == NWV - 1) s_wave[NWV] = u;
  }
  __syncthreads();
  uint32_t res = s_wave[wave] + x - v;
  *total = s_wave[NWV];
  __syncthreads();
  return res;
}

// ----------------------------------------------------------- f32 operands (fp64)
__global__ void __launch_bounds__(256) score_f64_kernel(IndexerArgs a) {
#pragma clang fp contract(off)
  extern __shared__ float s_q[];                  // [H_I * d_I]
  const int n = blockIdx.y;
  const int64_t V = visible(a, n);
  const int HD = a.H_I * a.d_I;
  const float* qrow = reinterpret_cast<const float*>(a.q + (int64_t)n * a.H_I * a.q_pitch);
  for (int i = threadIdx.x; i < HD; i += blockDim.x) {
    int h = i / a.d_I, d = i % a.d_I;
    s_q[i] = reinterpret_cast<const float*>(a.q + ((int64_t)n * a.H_I + h) * a.q_pitch)[d];
  }
  (void)qrow;
  __syncthreads();
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= V) return;
  const int b = a.seq_id[n];
  const int64_t row = cache_row(a.page_table, a.page_pitch, a.page_shift, b,
                                a.page_shift < 0 ? a.cache_row_start[b] : 0, j);
  const float* k = reinterpret_cast<const float*>(a.keys + row * a.key_pitch);
  double acc = 0.0;
  for (int h = 0; h < a.H_I; ++h) {
    double d = 0.0;
    for (int i = 0; i < a.d_I; ++i) d = d + (double)s_q[h * a.d_I + i] * (double)k[i];
    acc = acc + (double)a.w[(int64_t)n * a.H_I + h] * (d > 0.0 ? d : 0.0);
  }
  reinterpret_cast<double*>(a.scores)[(int64_t)n * a.score_pitch + j] = acc;
}

// exact top-k for small V with 64-bit keys (rank counting), one workgroup per query
__global__ void __launch_bounds__(256) select_small_f64_kernel(IndexerArgs a) {
  __shared__ uint64_t s_key[kSmallV];
  __shared__ uint8_t s_sel[kSmallV];
  __shared__ int s_cnt[256];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int V = (int)visible(a, n);
  const int K = V < a.k ? V : a.k;
  const double* sc = reinterpret_cast<const double*>(a.scores) + (int64_t)n * a.score_pitch;
  for (int j = tid; j < V; j += 256) s_key[j] = double_key(sc[j]);
  __syncthreads();
  for (int j = tid; j < V; j += 256) {
    const uint64_t kj = s_key[j];
    int rank = 0;
    for (int i = 0; i < V; ++i) {
      uint64_t ki = s_key[i];
      rank += (ki > kj) || (ki == kj && i < j);
    }
    s_sel[j] = rank < K;
  }
  __syncthreads();
  // ascending output: contiguous chunk per thread, prefix over threads
  const int chunk = (V + 255) / 256;
  const int lo = tid * chunk, hi = min(V, lo + chunk);
  int c = 0;
  for (int j = lo; j < hi; ++j) c += s_sel[j];
  s_cnt[tid] = c;
  __syncthreads();
  int base = 0;
  for (int t = 0; t < tid; ++t) base += s_cnt[t];
  int32_t* out = a.idx + (int64_t)n * a.k;
  double* so = reinterpret_cast<double*>(a.score_out);
  for (int j = lo; j < hi; ++j)
    if (s_sel[j]) {
      out[base] = j;
      if (so) so[(int64_t)n * a.k + base] = sc[j];
      ++base;
    }
  for (int p = K + tid; p < a.k; p += 256) {
    out[p] = -1;
    if (so) so[(int64_t)n * a.k + p] = 0.0;
  }
}

// -------------------------------------------------------- quantized operands
#ifndef HCA_SCORE_TPW
#define HCA_SCORE_TPW 8                                   // FP8 keys (decode: few queries)
#endif
#ifndef HCA_SCORE_TPW4
#define HCA_SCORE_TPW4 64                                 // MXFP4 keys (prefill: many queries)
#endif
#ifndef HCA_SCORE_RING
#define HCA_SCORE_RING 2
#endif
// 32-entry tiles per wave: fewer, larger workgroups amortize the per-workgroup
// query/weight loads and histogram traffic when there are thousands of queries
// MXFP4 keys with few queries (decode: each query reads its own sequence's keys, nothing
// shared through L2) use the decode tiling of the FP8 path
#ifndef HCA_SCORE_TPW4D
#define HCA_SCORE_TPW4D 8
#endif
constexpr int kFewQ = 256;                               // fewer queries: decode tiling for MXFP4
constexpr int entries_per_wg_t(int tpw) { return 4 * 32 * tpw; }
constexpr int kRing = HCA_SCORE_RING;                    // tiles in flight per wave

typedef float v16f __attribute__((ext_vector_type(16)));

// One float per lane into a buffer of `bytes` bytes at `base`: a lane whose byte
// offset is at or past the end writes nothing (the buffer range check drops it).
// All lanes execute the store, so a score store needs no branch, and the memory
// counter waits of the key ring stay exact (a store under a branch would make
// the compiler assume the path without it and wait for one load too many).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t score_range(float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void store_ranged(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, 0);
}
constexpr uint32_t kNoStore = 0x80000000u;              // past any score row
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// Canonical head sum of one tile: this lane's 16 heads per head tile, head tiles in
// order, each head one fused multiply-add into the running sum (one rounding), then
// the two halves of the wave (lanes j and j + 32) added.
template <int FMT, int HT>
__device__ __forceinline__ float head_sum(const v16f (&acc)[2], const float (&wv)[2][16]) {
  float S = 0.0f;
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    if (T < HT) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // max(d, +0) of a finite dot; with MXFP4 keys (ALU-bound) as one integer
        // max of its bits (a negative float, -0 included, is a negative integer),
        // which needs no NaN canonicalization; both give the same bits
        const float d = acc[T][i];
        const float r = FMT == HCA_MXFP4 ? __int_as_float(max(__float_as_int(d), 0)) : (d > 0.0f ? d : 0.0f);
        S = __builtin_fmaf(wv[T][i], r, S);
      }
    }
  }
  return S + __shfl_xor(S, 32, 64);
}

// Lane (j, u) = (lane % 32, lane / 32) of a 32-entry tile.  FP8: it holds bytes
// [64u, 64u + 64) of entry j's key and, per k-step s of the BF16 32x32x16 product,
// dims 64u + 8s .. 64u + 8s + 7; the query rows use the same dims.  MXFP4: it holds
// the 32-element blocks u and 2 + u (k-steps 0 and 1 of the scaled 32x32x64
// product).  Every head dot is the exact sum over all 128 dims either way.
#ifndef HCA_SCORE_WAVES
#define HCA_SCORE_WAVES 4                                // MXFP4: waves per SIMD the registers allow
#endif
// Workgroup order.  Chunk-major (XQ = false): the chunks of one query run together,
// so concurrent workgroups stream one contiguous key range (queries of different
// sequences touch different ranges).  XCD-major (XQ = true): linear workgroup L runs
// on XCD L mod 8; XCD x takes queries x, x + 8, ... and walks the entry chunks in
// order with its queries fastest, so a chunk of a shared key cache is read from
// memory once per XCD and then served by that XCD's L2 to all of its queries.
#ifndef HCA_SCORE_XCD_MAJOR
#define HCA_SCORE_XCD_MAJOR 1
#endif
// TPW: 32-entry tiles per wave (1024 entries per workgroup at 8).  PAGED: key rows
// come through the page table, one page per 32-entry tile.
// POOL (decode, chunk-major): the grid's leading pool_rows rows pool the step's
// blocks (the block's tokens complete its sequence's newest entry) and count
// themselves; in the workgroup whose range holds a query's newest entry V - 1, the
// one wave whose tiles hold it waits for every count just before it loads that tile.
// The pooling workgroups lead the dispatch order, so they are running whenever a
// wave waits; the wait is bounded all the same.
typedef PoolSmem<kScoreThreads, 4, true> ScorePoolSmem;     // blocks of m <= 16 tokens
constexpr uint32_t kPoolSpinMax = 1u << 22;

template <int FMT, bool XQ, int HT, int TPW, bool PAGED, bool POOL>
__device__ __forceinline__ void score_quant_body(const IndexerArgs& a, const PoolArgs& pool) {
#pragma clang fp contract(off)
  // scores staged in LDS and written once per wave (whole 16-byte groups per lane)
  constexpr bool kStage = TPW <= 16 && (32 * TPW) % 256 == 0;
  constexpr int kQa = FMT == HCA_FP8_E4M3 ? 8 : 1;       // MXFP4 keeps its query operands in registers
  struct Lds {
    uint32_t hist[kBins];
    v8bf qa[2][kQa][64];                                 // FP8 path: widened query operands, per lane
    float st[kStage ? kScoreThreads / 64 : 1][kStage ? 32 * TPW : 4];
  };
  union Shared {
    Lds s;
    char pool[POOL ? sizeof(ScorePoolSmem) : 1];         // a pooling workgroup's LDS
  };
  __shared__ __attribute__((aligned(16))) Shared sh;
  uint32_t* const s_hist = sh.s.hist;
  v8bf (*const s_qa)[kQa][64] = sh.s.qa;
  float (*const s_st)[kStage ? 32 * TPW : 4] = sh.s.st;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int jl = lane & 31, u = lane >> 5;
  int n;
  int64_t chunk;
  if constexpr (POOL) {
    if ((int)blockIdx.y < a.pool_rows) {
      const int nb = (int)(blockIdx.y * gridDim.x + blockIdx.x);
      if (nb < pool.n_blocks) {
        pool_d512_block<kScoreThreads, 4, true>(pool, nb, *reinterpret_cast<ScorePoolSmem*>(sh.pool));
        // every thread's stores complete, then the XCD's cache is written back before
        // the count is raised
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        if (tid == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          atomicAdd(a.pool_done, 1u);
        }
      }
      return;                                           // uniform over the workgroup
    }
  }
  if (XQ) {
    const int64_t L = blockIdx.x, r = L >> 3;
    const int64_t nper = ((int64_t)a.Nq + 7) >> 3;
    n = (int)(8 * (r % nper) + (L & 7));
    chunk = r / nper;
    if (n >= a.Nq) return;                              // uniform over the workgroup
  } else {
    n = (int)blockIdx.y - (POOL ? a.pool_rows : 0);
    chunk = blockIdx.x;
  }
  const int64_t V = visible(a, n);
  constexpr int kTilesPerWave = TPW;
  const int64_t ebase = chunk * entries_per_wg_t(TPW);
  if (ebase >= V) return;                               // uniform over the workgroup
  const int bseq = a.seq_id[n];
  const int64_t row0 = PAGED ? 0 : a.cache_row_start[bseq];
  const int64_t wbase = ebase + wave * 32 * kTilesPerWave;

  // keys stream through a ring of kRing tiles per wave: tile t + kRing is loaded
  // as soon as tile t has been widened, so kRing - 1 tiles stay in flight while
  // one is multiplied
  uint4 kr[kRing][4];
  int ks[kRing][2];
  // Lanes past the last visible entry load the last one instead (branch-free, so
  // the load counters stay exact); a column of the product depends on its own
  // key only, and those columns are never stored.
  // Rows are addressed by 32-bit byte offsets from the sequence's first row
  // (entries < 2^23 and max_visible x pitch < 2^32, checked by the caller), so a
  // tile costs one full-rate 24-bit multiply per plane.  Paged, the offsets are
  // from the first row of the tile's page (pages hold a power of two >= 32 rows).
  const char* const kseq = a.keys + row0 * a.key_pitch;
  const uint8_t* const sseq = FMT == HCA_MXFP4 ? a.key_scales + row0 * a.key_scale_pitch : nullptr;
  const uint32_t j0 = (uint32_t)(wbase + jl), jmax = (uint32_t)(V - 1);
  const uint32_t lane_off = FMT == HCA_FP8_E4M3 ? 64u * u : 16u * u;
  // MXFP4: the entry's four E8M0 block scales are one aligned 32-bit word; shifted
  // by 8u, its bytes 0 and 2 are this lane's blocks u and 2 + u, which the scaled
  // product selects with op_sel
  // Paged: lane t < TPW loads the page id of the wave's tile t up front, in one
  // vector load, so no key load waits on a lookup of its own.  Every lane of tile t
  // reads an entry of the 32-entry tile that starts at ts: the tile's own start, or
  // the last visible entry's tile when the tile lies wholly past it.
  static_assert(TPW <= 64, "one page id per lane");
  int page_of_tile = 0;
  if constexpr (PAGED) {
    const uint32_t ts = min((uint32_t)wbase + 32u * (uint32_t)min(lane, TPW - 1), jmax & ~31u);
    page_of_tile = a.page_table[(int64_t)bseq * a.page_pitch + (ts >> a.page_shift)];
  }
  // COH: device-coherent 32-bit loads that bypass the L1 and L2 (the MXFP4 tile that
  // holds a newly pooled entry: its 64-byte rows and 4-byte scales share cache lines
  // with neighbouring rows that plain loads may have cached before the pooling wrote)
  auto ld32 = [](const void* q) {
    return __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<void*>(q)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  };
  auto load_tile = [&](int t, uint4 (&dst)[4], int (&dsc)[2], bool coh = false) {
    uint32_t j = min(j0 + 32u * (uint32_t)t, jmax);
    const char* kb = kseq;
    const uint8_t* sb = sseq;
    if constexpr (PAGED) {
      const int64_t prow = (int64_t)__builtin_amdgcn_readlane(page_of_tile, t) << a.page_shift;
      kb = a.keys + prow * a.key_pitch;
      if (FMT == HCA_MXFP4) sb = a.key_scales + prow * a.key_scale_pitch;
      j &= (1u << a.page_shift) - 1u;
    }
    const char* key = kb + (uint32_t)((uint32_t)__umul24(j, (uint32_t)a.key_pitch) + lane_off);
    if (FMT == HCA_FP8_E4M3) {
      const uint4* p = reinterpret_cast<const uint4*>(key);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = p[q];
    } else if (coh) {
      const char* sw = reinterpret_cast<const char*>(sb) + (uint32_t)__umul24(j, (uint32_t)a.key_scale_pitch);
      dst[0] = make_uint4(ld32(key), ld32(key + 4), ld32(key + 8), ld32(key + 12));
      dst[1] = make_uint4(ld32(key + 32), ld32(key + 36), ld32(key + 40), ld32(key + 44));
      dsc[0] = (int)(ld32(sw) >> (8 * u));
    } else {
      dst[0] = *reinterpret_cast<const uint4*>(key);
      dst[1] = *reinterpret_cast<const uint4*>(key + 32);
      const uint32_t w = *reinterpret_cast<const uint32_t*>(sb + (uint32_t)__umul24(j, (uint32_t)a.key_scale_pitch));
      dsc[0] = (int)(w >> (8 * u));
    }
  };
  for (int i = tid; i < kBins; i += kScoreThreads) s_hist[i] = 0;

  // Query rows and weights are all requested first (raw), then the first kRing
  // key tiles in tile order (the scheduling barriers keep that order), so that
  // waiting for the query or for tile t never waits for a later tile.
  // HT = H_I / 32 head tiles (1 or 2), a template argument so the tile loop has no branches
  uint4 qraw[2][4];
  int qs[2][2];
  float wv[2][16];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    if (T < HT) {
      const int64_t qr = (int64_t)n * a.H_I + 32 * T + jl;
      if (FMT == HCA_FP8_E4M3) {
        if (wave == 0) {                                 // widened once, into LDS, for all waves
          const uint4* p = reinterpret_cast<const uint4*>(a.q + qr * a.q_pitch + 64 * u);
#pragma unroll
          for (int q = 0; q < 4; ++q) qraw[T][q] = p[q];
        }
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          qraw[T][s2] = *reinterpret_cast<const uint4*>(a.q + qr * a.q_pitch + 32 * s2 + 16 * u);
          qs[T][s2] = a.q_scales[qr * a.q_scale_pitch + 2 * s2 + u];
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) wv[T][i] = a.w[(int64_t)n * a.H_I + 32 * T + 8 * (i >> 2) + 4 * u + (i & 3)];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // A wave wholly past V (in a query's last chunk) loads and scores nothing: its lanes
  // would all read entry V - 1 as padding.  POOL: the wave whose tiles hold the
  // query's newest entry V - 1 waits for the pooling just before it loads that tile
  // (its earlier tiles stream meanwhile), then acquires; with the idle waves skipped,
  // no other wave ever reads the new row.
  const int64_t rel = V - 1 - wbase;
  const bool idle = rel < 0;                            // uniform over the wave
  int t_wait = -1;
  if constexpr (POOL) {
    if (rel >= 0 && rel < 32 * kTilesPerWave) t_wait = (int)(rel >> 5);
  }
  // (MXFP4 rows share cache lines, so that tile is read with coherent loads)
  auto pool_wait = [&](int t) {
    if constexpr (POOL) {
      if (t == t_wait) {
        for (uint32_t it = 0; ld_dev(a.pool_done) < (uint32_t)a.pool_target && it < kPoolSpinMax; ++it)
          __builtin_amdgcn_s_sleep(2);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        return FMT == HCA_MXFP4;
      }
    }
    return false;
  };
#pragma unroll
  for (int t = 0; t < kRing; ++t) {
    if (t < kTilesPerWave && !idle) {
      const bool coh = pool_wait(t);
      load_tile(t, kr[t], ks[t], coh);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  v8i qf4[2][2];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    if (T < HT) {
      if (FMT == HCA_FP8_E4M3) {
        if (wave == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            s_qa[T][2 * q][lane] = fp8x8_to_bf16(qraw[T][q].x, qraw[T][q].y);
            s_qa[T][2 * q + 1][lane] = fp8x8_to_bf16(qraw[T][q].z, qraw[T][q].w);
          }
        }
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          qf4[T][s2] = (v8i){(int)qraw[T][s2].x, (int)qraw[T][s2].y, (int)qraw[T][s2].z, (int)qraw[T][s2].w, 0, 0, 0, 0};
      }
    }
  }
  __syncthreads();

  // MXFP4: the query's V scores, one store per tile; FP8 (staged): the whole padded
  // row (a multiple of 64 floats), so a 16-byte group is either in the row or past it
  float* const sc_row = reinterpret_cast<float*>(a.scores) + (int64_t)n * a.score_pitch;
  const __amdgpu_buffer_rsrc_t srange = score_range(sc_row, kStage ? 4u * (uint32_t)a.score_pitch : 4u * (uint32_t)V);
  if (!idle) {
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const uint32_t j = j0 + 32u * (uint32_t)t;
    const int slot = t % kRing;
    v16f acc[2];
    if (FMT == HCA_FP8_E4M3) {
      v8bf kb[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kb[2 * q] = fp8x8_to_bf16(kr[slot][q].x, kr[slot][q].y);
        kb[2 * q + 1] = fp8x8_to_bf16(kr[slot][q].z, kr[slot][q].w);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (t + kRing < kTilesPerWave) {
        (void)pool_wait(t + kRing);
        load_tile(t + kRing, kr[slot], ks[slot]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        if (T < HT) {
          v16f c = {};
#pragma unroll
          for (int s2 = 0; s2 < 8; ++s2) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s_qa[T][s2][lane], kb[s2], c, 0, 0, 0);
          acc[T] = c;
        }
      }
    } else {
      const v8i kv0 = {(int)kr[slot][0].x, (int)kr[slot][0].y, (int)kr[slot][0].z, (int)kr[slot][0].w, 0, 0, 0, 0};
      const v8i kv1 = {(int)kr[slot][1].x, (int)kr[slot][1].y, (int)kr[slot][1].z, (int)kr[slot][1].w, 0, 0, 0, 0};
      const int ksw = ks[slot][0];
      __builtin_amdgcn_sched_barrier(0);
      if (t + kRing < kTilesPerWave) {
        const bool coh = pool_wait(t + kRing);
        load_tile(t + kRing, kr[slot], ks[slot], coh);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        if (T < HT) {
          v16f c = {};
          c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf4[T][0], kv0, c, 4, 4, 0, qs[T][0], 0, ksw);
          c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf4[T][1], kv1, c, 4, 4, 0, qs[T][1], 2, ksw);
          acc[T] = c;
        }
      }
    }
    const float S = head_sum<FMT, HT>(acc, wv);
    if (kStage) {
      if (u == 0) s_st[wave][32 * t + jl] = S;
    } else {
      store_ranged(srange, u == 0 ? 4u * j : kNoStore, S);      // j >= V: past the range
    }
    if (u == 0 && j < (uint32_t)V) {
      // first digit of float_key(S): S is never -0 (each half-sum starts from +0,
      // and a rounded sum is -0 only if both addends are), so the sign flip needs no case
      const uint32_t b = __float_as_uint(S);
      atomicAdd(&s_hist[(b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u)) >> 21], 1u);
    }
  }
  }
  if (kStage && !idle) {
    // the wave's 32 x tiles scores in entry order, 16 bytes per lane; entries past V
    // land in the row's padding (never read), groups past the row are dropped
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int h = 0; h < 32 * kTilesPerWave / 256; ++h) {
      const uint32_t f = 256u * h + 4u * lane;
      const u4v v = *reinterpret_cast<const u4v*>(&s_st[wave][f]);
      __builtin_amdgcn_raw_buffer_store_b128(v, srange, (int)(4u * ((uint32_t)wbase + f)), 0, 0);
    }
  }
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)n * kBins;
  for (int i = tid; i < kBins; i += kScoreThreads) {
    uint32_t c = s_hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

template <int FMT, bool XQ, int HT, int TPW, bool PAGED>
__global__ void __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(FMT == HCA_MXFP4 ? HCA_SCORE_WAVES : 2)))
score_quant_kernel(IndexerArgs a) {
  const PoolArgs none{};
  score_quant_body<FMT, XQ, HT, TPW, PAGED, false>(a, none);
}

// the same scoring with the step's pooling in the leading grid rows (decode), at the
// scoring kernel's own occupancy (FP8: three waves per SIMD)
template <int FMT, int HT, int TPW, bool PAGED>
__global__ void __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(FMT == HCA_MXFP4 ? HCA_SCORE_WAVES : 3)))
score_pool_kernel(IndexerArgs a, PoolArgs p) {
  score_quant_body<FMT, false, HT, TPW, PAGED, true>(a, p);
}

__global__ void __launch_bounds__(256) zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

// ------------------------------------------------------------------- select
// Top-k in three parallel phases over the materialized scores.  The first radix
// digit (key bits 31..21) was histogrammed by the scoring kernel.
//   collect:   every 4096-entry chunk counts its keys above the threshold digit d1
//              and appends those in d1 (the candidates) to a per-query list;
//   threshold: one workgroup per query resolves digits 2 and 3 on the candidates,
//              giving the exact k-th key T and how many keys equal to T to keep
//              (the lowest indices), and turns per-chunk counts into output offsets;
//   emit:      every chunk writes its selected indices, ascending, at its offset.
constexpr int kChunk1 = 4096;
constexpr int kCandCap2 = 8192;
constexpr int kMaxChunks = 2048;
// Many queries (>= kDigitMinQ) and k <= kMergedMaxK: collect also keeps the keys above
// d1 (fewer than k per query) and the threshold phase writes the selection itself,
// each selected entry placed by the rank of its index, so the scores are not read a
// second time (no emit phase).
constexpr int kMergedMaxK = 2048;

struct SelectWs {
  uint32_t* d1;           // [Nq] first digit found once per query (many queries), else null
  uint32_t* cand_count;   // [Nq] (cleared with the histogram, as the next)
  uint32_t* above_count;  // [Nq]  merged selection: keys above the first digit
  uint32_t* done;         // [Nq]  fused decode select: chunks of the query collected
  uint32_t* above_key;    // [Nq, k]
  int32_t* above_idx;     // [Nq, k]
  uint32_t* cand_key;     // [Nq, kCandCap2]
  int32_t* cand_idx;      // [Nq, kCandCap2]
  uint32_t* chunk_gt;     // [Nq, nch]
  uint32_t* out_off;      // [Nq, nch]
  uint32_t* eq_before;    // [Nq, nch]
  uint32_t* state;        // [Nq, 2]: threshold key, number of equal keys kept
  int nch;
};

// The digit holding the need-th largest key of a histogram (digits ordered by key);
// *need becomes the rank still needed inside that digit.
template <int NT>
__device__ int find_digit(const uint32_t* hist, int nbins, uint32_t* need, uint32_t* s_wave,
                          int* s_found, uint32_t* s_need) {
  const int tid = threadIdx.x;
  if (tid == 0) { *s_found = 0; *s_need = 1; }
  const int per = nbins / NT;
  const int top = nbins - 1 - tid * per;
  uint32_t c = 0;
  for (int q = 0; q < per; ++q) c += hist[top - q];
  uint32_t tot;
  uint32_t above = block_exclusive_scan<NT>(c, s_wave, &tot);
  const uint32_t nd = *need;
  for (int q = 0; q < per; ++q) {
    const uint32_t h = hist[top - q];
    if (above < nd && nd <= above + h) { *s_found = top - q; *s_need = nd - above; }
    above += h;
  }
  __syncthreads();
  *need = *s_need;
  const int d = *s_found;
  __syncthreads();
  return d;
}

// 16 consecutive scores of a 4096-entry chunk per thread (4 aligned 16-byte loads;
// the score rows are padded to a multiple of 64, so no load passes the row)
constexpr int kPerThread1 = kChunk1 / 256;
__device__ __forceinline__ void load_chunk_keys(const float* sc, int64_t jt, int64_t j1, uint32_t (&key)[kPerThread1]) {
#pragma unroll
  for (int v = 0; v < kPerThread1 / 4; ++v) {
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (jt + 4 * v < j1) f = *reinterpret_cast<const float4*>(sc + jt + 4 * v);
    key[4 * v] = float_key(f.x); key[4 * v + 1] = float_key(f.y);
    key[4 * v + 2] = float_key(f.z); key[4 * v + 3] = float_key(f.w);
  }
}

// With many queries, every chunk workgroup finding the first digit again (8 KB of
// histogram and a 2048-bin scan each) costs more than one extra launch: one
// workgroup per query finds it once.
constexpr int kDigitMinQ = 256;
__global__ void __launch_bounds__(256) select_digit_kernel(IndexerArgs a, SelectWs ws) {
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_wave[256 / 64 + 1];
  __shared__ int s_found;
  __shared__ uint32_t s_need;
  const int n = blockIdx.x, tid = threadIdx.x;
  const int64_t V = visible(a, n);
  const int64_t K = V < a.k ? V : a.k;
  if (V <= K) return;                                    // uniform
  const uint32_t* gh = a.hist + (int64_t)n * kBins;
  for (int i = tid; i < kBins; i += 256) s_hist[i] = gh[i];
  __syncthreads();
  uint32_t need = (uint32_t)K;
  const uint32_t d1 = (uint32_t)find_digit<256>(s_hist, kBins, &need, s_wave, &s_found, &s_need);
  if (tid == 0) ws.d1[n] = d1;
}

template <bool PRE>                                      // PRE: the first digit was found per query
__global__ void __launch_bounds__(256) select_collect_kernel(IndexerArgs a, SelectWs ws) {
  __shared__ uint32_t s_hist[PRE ? 1 : kBins];
  __shared__ uint32_t s_ck[kChunk1];                   // candidates from the front, keys above d1 from the back
  __shared__ uint16_t s_cj[kChunk1];                   // their offsets in the chunk
  __shared__ uint32_t s_wave[256 / 64 + 1];
  __shared__ uint32_t s_n, s_base, s_na, s_abase;
  __shared__ int s_found;
  __shared__ uint32_t s_need;
  const int n = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int64_t V = visible(a, n);
  const int64_t K = V < a.k ? V : a.k;
  const int64_t j0 = (int64_t)c * kChunk1;
  if (V <= K || j0 >= V) return;
  const bool merged = ws.above_key != nullptr;          // uniform
  // the scores do not depend on the threshold digit: request them first
  const float* sc = reinterpret_cast<const float*>(a.scores) + (int64_t)n * a.score_pitch;
  const int64_t j1 = j0 + kChunk1 < V ? j0 + kChunk1 : V;
  const int64_t jt = j0 + (int64_t)kPerThread1 * tid;
  // raw score bits; the first digit is taken from them exactly as the scoring kernel
  // histogrammed it (a score is never -0), the full orderable key only for the keys
  // that are appended
  uint32_t bits[kPerThread1];
#pragma unroll
  for (int v = 0; v < kPerThread1 / 4; ++v) {
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (jt + 4 * v < j1) f = *reinterpret_cast<const float4*>(sc + jt + 4 * v);   // rows padded to 64
    bits[4 * v] = __float_as_uint(f.x); bits[4 * v + 1] = __float_as_uint(f.y);
    bits[4 * v + 2] = __float_as_uint(f.z); bits[4 * v + 3] = __float_as_uint(f.w);
  }
  const int64_t rem = j1 - jt;
  const int nv = rem <= 0 ? 0 : (rem >= kPerThread1 ? kPerThread1 : (int)rem);   // this thread's scores
  uint32_t d1;
  if constexpr (PRE) {
    d1 = ws.d1[n];
    if (tid == 0) { s_n = 0; s_na = 0; }
    __syncthreads();
  } else {
    const uint32_t* gh = a.hist + (int64_t)n * kBins;
    for (int i = tid; i < kBins; i += 256) s_hist[i] = gh[i];
    if (tid == 0) { s_n = 0; s_na = 0; }
    __syncthreads();
    uint32_t need = (uint32_t)K;
    d1 = (uint32_t)find_digit<256>(s_hist, kBins, &need, s_wave, &s_found, &s_need);
  }
  uint32_t gt = 0;
#pragma unroll
  for (int e = 0; e < kPerThread1; ++e) {
    const uint32_t b = bits[e];
    const uint32_t dg = (b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u)) >> 21;
    const bool in = e < nv;
    gt += (in && dg > d1) ? 1u : 0u;
    if (in && dg >= d1 && (dg == d1 || merged)) {      // rare: a candidate, or a key above d1
      const uint32_t p = dg == d1 ? atomicAdd(&s_n, 1u) : kChunk1 - 1 - atomicAdd(&s_na, 1u);
      s_ck[p] = float_key(__uint_as_float(b));
      s_cj[p] = (uint16_t)(jt + e - j0);
    }
  }
  uint32_t tot;
  block_exclusive_scan<256>(gt, s_wave, &tot);         // also orders the appends above
  if (tid == 0) {
    ws.chunk_gt[(int64_t)n * ws.nch + c] = tot;
    s_base = s_n ? atomicAdd(&ws.cand_count[n], s_n) : 0;
    s_abase = s_na ? atomicAdd(&ws.above_count[n], s_na) : 0;
  }
  __syncthreads();
  const uint32_t cnt = s_n, base = s_base;
  for (uint32_t i = tid; i < cnt; i += 256) {
    const uint32_t p = base + i;
    if (p < (uint32_t)kCandCap2) {
      ws.cand_key[(int64_t)n * kCandCap2 + p] = s_ck[i];
      ws.cand_idx[(int64_t)n * kCandCap2 + p] = (int32_t)(j0 + s_cj[i]);
    }
  }
  const uint32_t na = s_na, abase = s_abase;
  for (uint32_t i = tid; i < na; i += 256) {
    const uint32_t p = abase + i;                        // < k: fewer than k keys lie above d1
    if (p < (uint32_t)a.k) {
      ws.above_key[(int64_t)n * a.k + p] = s_ck[kChunk1 - 1 - i];
      ws.above_idx[(int64_t)n * a.k + p] = (int32_t)(j0 + s_cj[kChunk1 - 1 - i]);
    }
  }
}

// Writes, in index order, the keys of one stretch above T and its keys equal to T
// while fewer than take_eq equal keys precede them in the whole row (NT threads,
// kPerThread1 consecutive keys each): pos_base = entries selected before the
// stretch, eqb = keys equal to T before it.  Returns the stretch's count of keys
// above T | keys equal to T << 16.
template <int NT>
__device__ uint32_t emit_ordered(const IndexerArgs& a, int n, const uint32_t (&key)[kPerThread1], int64_t jt,
                                 int64_t j1, uint32_t T, uint32_t take_eq, uint32_t pos_base, uint32_t eqb,
                                 int64_t K, const float* sc, uint32_t* s_wave) {
  static_assert(NT * kPerThread1 < 65536, "16-bit counts per stretch");
  int32_t* out = a.idx + (int64_t)n * a.k;
  float* so = reinterpret_cast<float*>(a.score_out);
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int e = 0; e < kPerThread1; ++e) {
    if (jt + e < j1) {
      ngt += key[e] > T;
      neq += key[e] == T;
    }
  }
  uint32_t tot;
  const uint32_t pre = block_exclusive_scan<NT>(ngt | (neq << 16), s_wave, &tot);
  uint32_t gt_before = pre & 0xFFFF;
  uint32_t eq_before = eqb + (pre >> 16);
  const uint32_t eq_taken0 = eqb < take_eq ? eqb : take_eq;     // equal keys taken before the stretch
#pragma unroll
  for (int e = 0; e < kPerThread1; ++e) {
    if (jt + e < j1) {
      const bool is_gt = key[e] > T, is_eq = key[e] == T;
      if (is_gt || (is_eq && eq_before < take_eq)) {
        const uint32_t eq_sel_before = (eq_before < take_eq ? eq_before : take_eq) - eq_taken0;
        const uint32_t pos = pos_base + gt_before + eq_sel_before;
        if (pos < (uint32_t)K) {
          out[pos] = (int32_t)(jt + e);
          if (so) so[(int64_t)n * a.k + pos] = sc[jt + e];
        }
      }
      gt_before += is_gt;
      eq_before += is_eq;
    }
  }
  return tot;
}

// Position of this lane's item in a list appended to through *counter (LDS or
// global): one atomic per wave for the lanes with pred set, in lane order.  Called
// by every active lane of the wave; the result is meaningful where pred is set.
__device__ __forceinline__ uint32_t wave_append(uint32_t* counter, bool pred) {
  const uint64_t m = __ballot(pred);
  if (!m) return 0;
  const int lane = threadIdx.x & 63;
  const int leader = __builtin_ctzll(m);
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(m));
  base = __shfl(base, leader, 64);
  return base + (uint32_t)__builtin_popcountll(m & ((1ull << lane) - 1ull));
}


__device__ __forceinline__ float key_float(uint32_t k) {        // inverse of float_key (no -0 arises)
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Digits 2 and 3 of the k-th largest key T (digit 1 = d1; *need = its rank inside d1
// on entry, the number of keys equal to T to keep on return), from the candidate
// list (key_at(i), i < n1: every key whose first digit is d1) or, when the list
// overflowed (!have), from the query's scores.  *n_eq: candidates equal to T.
template <int NT, class KeyAt>
__device__ uint32_t resolve_threshold(const float* sc, int64_t V, uint32_t d1, uint32_t* need, bool have, KeyAt key_at,
                                      uint32_t n1, uint32_t* s_hist, uint32_t* s_wave, int* s_found, uint32_t* s_need,
                                      uint32_t* n_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = d1;
  for (int round = 0; round < 2; ++round) {
    const int shift = round == 0 ? 10 : 0;
    const int nbits = round == 0 ? 11 : 10;
    const int nb = 1 << nbits;
    for (int i = tid; i < kBins; i += NT) s_hist[i] = 0;
    __syncthreads();
    if (have) {
      for (uint32_t i = tid; i < n1; i += NT) {
        const uint32_t key = key_at(i);
        if ((key >> (shift + nbits)) == prefix) atomicAdd(&s_hist[(key >> shift) & (nb - 1)], 1u);
      }
    } else {
      for (int64_t j = tid; j < V; j += NT) {
        const uint32_t key = float_key(sc[j]);
        if ((key >> (shift + nbits)) == prefix) atomicAdd(&s_hist[(key >> shift) & (nb - 1)], 1u);
      }
    }
    __syncthreads();
    const int dd = find_digit<NT>(s_hist, nb, need, s_wave, s_found, s_need);
    if (round == 1) *n_eq = s_hist[dd];
    prefix = (prefix << nbits) | (uint32_t)dd;
  }
  __syncthreads();                                       // every thread has read n_eq before s_hist is reused
  return prefix;
}

// The selection of one query from its threshold T: every key above d1 (the caller
// has put the na of them in s_sk/s_sj[0, na)), the candidates above T and the
// take_eq lowest-index candidates equal to T, each written at the rank of its index
// (ascending); or, when the candidate list overflowed (!have), one ordered pass over
// the scores.
template <int NT, class KeyAt, class IdxAt>
__device__ void emit_merged(const IndexerArgs& a, const SelectWs& ws, int n, int64_t V, int64_t K, uint32_t T,
                            uint32_t take_eq, uint32_t n_eq, bool have, KeyAt key_at, IdxAt idx_at, uint32_t n1,
                            uint32_t na,
                            const float* sc, uint32_t* s_hist, uint32_t* s_sk, int32_t* s_sj, uint32_t* s_fill,
                            uint32_t* s_tk, int32_t* s_tj, uint32_t* s_wave, int* s_found, uint32_t* s_need,
                            uint32_t* s_ns) {
  const int tid = threadIdx.x;
  int32_t* const out = a.idx + (int64_t)n * a.k;
  float* const so = reinterpret_cast<float*>(a.score_out);
  if (!have) {
    uint32_t sel_before = 0, eq_seen = 0;
    constexpr int64_t kStretch = (int64_t)NT * kPerThread1;
    for (int64_t b0 = 0; b0 < V; b0 += kStretch) {
      const int64_t b1 = b0 + kStretch < V ? b0 + kStretch : V;
      const int64_t bt = b0 + (int64_t)kPerThread1 * tid;
      uint32_t kk[kPerThread1];
      load_chunk_keys(sc, bt, b1, kk);
      const uint32_t tt = emit_ordered<NT>(a, n, kk, bt, b1, T, take_eq, sel_before, eq_seen, K, sc, s_wave);
      const uint32_t gt = tt & 0xFFFF, eq = tt >> 16;
      const uint32_t took = (eq_seen + eq < take_eq ? eq_seen + eq : take_eq) - (eq_seen < take_eq ? eq_seen : take_eq);
      sel_before += gt + took;
      eq_seen += eq;
    }
    return;
  }
  // equal keys: the take_eq lowest indices, i.e. the take_eq largest of 2^30 - 1 - j
  // (three 10-bit digits)
  uint32_t inv_min = 0;
  if (take_eq < n_eq) {
    uint32_t need_i = take_eq, pre = 0;
    for (int round = 0; round < 3; ++round) {
      const int shift = 20 - 10 * round;
      for (int i = tid; i < 1024; i += NT) s_hist[i] = 0;
      __syncthreads();
      for (uint32_t i = tid; i < n1; i += NT) {
        if (key_at(i) != T) continue;
        const uint32_t inv = 0x3FFFFFFFu - (uint32_t)idx_at(i);
        if ((inv >> (shift + 10)) == pre) atomicAdd(&s_hist[(inv >> shift) & 1023], 1u);
      }
      __syncthreads();
      const int dd = find_digit<NT>(s_hist, 1024, &need_i, s_wave, s_found, s_need);
      pre = (pre << 10) | (uint32_t)dd;
    }
    inv_min = pre;
  }
  // the selected entries (exactly K; the checks below only guard the LDS bounds),
  // then each one's output position is the rank of its index
  if (tid == 0) *s_ns = na;                              // the keys above d1: s_sk/s_sj[0, na), placed by the caller
  __syncthreads();
  for (uint32_t i0 = 0; i0 < n1; i0 += NT) {
    const uint32_t i = i0 + tid;
    uint32_t k2 = 0;
    int32_t j = 0;
    bool take = false;
    if (i < n1) {
      k2 = key_at(i);
      j = idx_at(i);
      take = k2 > T || (k2 == T && 0x3FFFFFFFu - (uint32_t)j >= inv_min);
    }
    const uint32_t p = wave_append(s_ns, take);
    if (take && p < (uint32_t)kMergedMaxK) {
      s_sk[p] = k2;
      s_sj[p] = j;
    }
  }
  __syncthreads();
  const uint32_t ns = min(*s_ns, (uint32_t)kMergedMaxK);  // == K <= kMergedMaxK
  // ---- order by index: counting sort on the index's high bits (at most kBins
  // buckets), then each entry's rank among the entries of its bucket
  int shift = 0;
  while (((V - 1) >> shift) >= kBins) ++shift;
  for (int b = tid; b < kBins; b += NT) { s_hist[b] = 0; s_fill[b] = 0; }
  __syncthreads();
  for (uint32_t e = tid; e < ns; e += NT) atomicAdd(&s_hist[s_sj[e] >> shift], 1u);
  __syncthreads();
  {
    constexpr int kPerB = kBins / NT;
    uint32_t c[kPerB], sum = 0;
#pragma unroll
    for (int q = 0; q < kPerB; ++q) { c[q] = s_hist[kPerB * tid + q]; sum += c[q]; }
    uint32_t tot;
    uint32_t off = block_exclusive_scan<NT>(sum, s_wave, &tot);
#pragma unroll
    for (int q = 0; q < kPerB; ++q) { s_hist[kPerB * tid + q] = off; off += c[q]; }
  }
  __syncthreads();
  for (uint32_t e = tid; e < ns; e += NT) {
    const int32_t j = s_sj[e];
    const int b = j >> shift;
    const uint32_t p = s_hist[b] + atomicAdd(&s_fill[b], 1u);
    s_tj[p] = j;
    s_tk[p] = s_sk[e];
  }
  __syncthreads();
  for (uint32_t p = tid; p < ns; p += NT) {
    const int32_t j = s_tj[p];
    const int b = j >> shift;
    const uint32_t b0 = s_hist[b], b1 = b0 + s_fill[b];
    uint32_t r = b0;
    for (uint32_t q = b0; q < b1; ++q) r += (uint32_t)(s_tj[q] < j);
    if (r < (uint32_t)K) {
      out[r] = j;
      if (so) so[(int64_t)n * a.k + r] = key_float(s_tk[p]);
    }
  }
}

__global__ void __launch_bounds__(kSelectThreads) select_threshold_kernel(IndexerArgs a, SelectWs ws) {
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_ck[kCandCap2];
  __shared__ int32_t s_cj[kCandCap2];
  __shared__ uint32_t s_selc[kMaxChunks];
  __shared__ uint32_t s_eqc[kMaxChunks];
  __shared__ uint32_t s_wave[kSelectThreads / 64 + 1];
  __shared__ int s_found;
  __shared__ uint32_t s_need, s_ns;
  __shared__ __attribute__((aligned(16))) uint32_t s_sk[kMergedMaxK];      // merged: the selected entries
  __shared__ __attribute__((aligned(16))) int32_t s_sj[kMergedMaxK + 32];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int64_t V = visible(a, n);
  const int64_t K = V < a.k ? V : a.k;
  const bool merged = ws.above_key != nullptr;          // uniform: this kernel writes the selection
  const float* sc = reinterpret_cast<const float*>(a.scores) + (int64_t)n * a.score_pitch;
  int32_t* const out = a.idx + (int64_t)n * a.k;
  float* const so = reinterpret_cast<float*>(a.score_out);
  if (V <= K) {
    if (merged) {                                        // every visible entry, at its own position
      for (int64_t p = tid; p < a.k; p += kSelectThreads) {
        out[p] = p < V ? (int32_t)p : -1;
        if (so) so[(int64_t)n * a.k + p] = p < V ? sc[p] : 0.0f;
      }
    } else if (tid == 0) {
      ws.state[2 * n] = 0;
      ws.state[2 * n + 1] = 0xFFFFFFFFu;
    }
    return;
  }
  const int nch = (int)((V + kChunk1 - 1) / kChunk1);
  uint32_t gtc[2];                                      // chunks 2t, 2t + 1: keys above digit d1
#pragma unroll
  for (int e = 0; e < 2; ++e) gtc[e] = 2 * tid + e < nch ? ws.chunk_gt[(int64_t)n * ws.nch + 2 * tid + e] : 0;
  const uint32_t* gh = a.hist + (int64_t)n * kBins;
  for (int i = tid; i < kBins; i += kSelectThreads) s_hist[i] = gh[i];
  for (int i = tid; i < nch; i += kSelectThreads) { s_selc[i] = 0; s_eqc[i] = 0; }
  __syncthreads();
  uint32_t need = (uint32_t)K;
  const uint32_t d1 = (uint32_t)find_digit<kSelectThreads>(s_hist, kBins, &need, s_wave, &s_found, &s_need);
  const uint32_t n1 = ws.cand_count[n];
  const bool in_lds = n1 <= (uint32_t)kCandCap2;
  if (in_lds) {
    for (uint32_t i = tid; i < n1; i += kSelectThreads) {
      s_ck[i] = ws.cand_key[(int64_t)n * kCandCap2 + i];
      s_cj[i] = ws.cand_idx[(int64_t)n * kCandCap2 + i];
    }
  }
  const uint32_t na = merged ? min(ws.above_count[n], (uint32_t)a.k) : 0;
  for (uint32_t i = tid; i < na && i < (uint32_t)kMergedMaxK; i += kSelectThreads) {
    s_sk[i] = ws.above_key[(int64_t)n * a.k + i];
    s_sj[i] = ws.above_idx[(int64_t)n * a.k + i];
  }
  __syncthreads();
  uint32_t n_eq = 0;                                     // candidates equal to T (in the list)
  auto lds_key = [&](uint32_t i) { return s_ck[i]; };
  auto lds_idx = [&](uint32_t i) { return s_cj[i]; };
  const uint32_t T = resolve_threshold<kSelectThreads>(sc, V, d1, &need, in_lds, lds_key, n1, s_hist, s_wave, &s_found,
                                                       &s_need, &n_eq);
  const uint32_t take_eq = need;
  if (merged) {
    emit_merged<kSelectThreads>(a, ws, n, V, K, T, take_eq, n_eq, in_lds, lds_key, lds_idx, n1, na, sc, s_hist, s_sk, s_sj,
                                s_ck, s_ck + kBins, s_cj, s_wave, &s_found, &s_need, &s_ns);
    return;
  }
  // per-chunk counts of the candidates above T and equal to T
  if (in_lds) {
    for (uint32_t i = tid; i < n1; i += kSelectThreads) {
      const uint32_t key = s_ck[i];
      const int ch = s_cj[i] / kChunk1;
      if (key > T) atomicAdd(&s_selc[ch], 1u);
      else if (key == T) atomicAdd(&s_eqc[ch], 1u);
    }
  } else {
    for (int64_t j = tid; j < V; j += kSelectThreads) {
      const uint32_t key = float_key(sc[j]);
      if ((key >> 21) != d1) continue;
      const int ch = (int)(j / kChunk1);
      if (key > T) atomicAdd(&s_selc[ch], 1u);
      else if (key == T) atomicAdd(&s_eqc[ch], 1u);
    }
  }
  __syncthreads();
  // output offsets in chunk order: a chunk keeps its keys above digit d1, its
  // candidates above T and the equal keys that earlier chunks left to take
  // (thread t: chunks 2t, 2t + 1; two block scans)
  uint32_t eqc[2], keep[2], eqb[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) eqc[e] = 2 * tid + e < nch ? s_eqc[2 * tid + e] : 0;
  uint32_t tot;
  eqb[0] = block_exclusive_scan<kSelectThreads>(eqc[0] + eqc[1], s_wave, &tot);
  eqb[1] = eqb[0] + eqc[0];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t left = eqb[e] >= take_eq ? 0 : take_eq - eqb[e];
    keep[e] = 2 * tid + e < nch ? gtc[e] + s_selc[2 * tid + e] + (eqc[e] < left ? eqc[e] : left) : 0;
  }
  const uint32_t off0 = block_exclusive_scan<kSelectThreads>(keep[0] + keep[1], s_wave, &tot);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int ch = 2 * tid + e;
    if (ch < nch) {
      ws.out_off[(int64_t)n * ws.nch + ch] = e ? off0 + keep[0] : off0;
      ws.eq_before[(int64_t)n * ws.nch + ch] = eqb[e];
    }
  }
  if (tid == 0) {
    ws.state[2 * n] = T;
    ws.state[2 * n + 1] = take_eq;
  }
}

__global__ void __launch_bounds__(256) select_emit_kernel(IndexerArgs a, SelectWs ws) {
  __shared__ uint32_t s_wave[256 / 64 + 1];
  const int n = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int64_t V = visible(a, n);
  const int64_t K = V < a.k ? V : a.k;
  const int64_t j0 = (int64_t)c * kChunk1;
  int32_t* out = a.idx + (int64_t)n * a.k;
  float* so = reinterpret_cast<float*>(a.score_out);
  const float* sc = reinterpret_cast<const float*>(a.scores) + (int64_t)n * a.score_pitch;
  if (V <= K) {                     // every visible entry is kept, at its own position
    for (int64_t j = j0 + tid; j < V && j < j0 + kChunk1; j += 256) {
      out[j] = (int32_t)j;
      if (so) so[(int64_t)n * a.k + j] = sc[j];
    }
    if (c == 0)
      for (int64_t p = V + tid; p < a.k; p += 256) {
        out[p] = -1;
        if (so) so[(int64_t)n * a.k + p] = 0.0f;
      }
    return;
  }
  if (j0 >= V) return;
  // the scores first (independent of the threshold), then the chunk's offsets
  const int64_t j1 = j0 + kChunk1 < V ? j0 + kChunk1 : V;
  const int64_t jt = j0 + (int64_t)kPerThread1 * tid;
  uint32_t key[kPerThread1];
  load_chunk_keys(sc, jt, j1, key);
  const uint32_t T = ws.state[2 * n], take_eq = ws.state[2 * n + 1];
  const uint32_t pos_base = ws.out_off[(int64_t)n * ws.nch + c];
  const uint32_t eqb = ws.eq_before[(int64_t)n * ws.nch + c];
  emit_ordered<256>(a, n, key, jt, j1, T, take_eq, pos_base, eqb, K, sc, s_wave);
}

// Decode (fewer than kDigitMinQ queries, k <= kMergedMaxK): the whole selection in one
// launch.  The (query, 4096-entry chunk) items are spread over the workgroups; each
// finds d1 from the scoring kernel's histogram, appends its chunk's candidates (first
// digit d1) and its keys above d1 to the query's lists, then counts itself done.  The
// workgroup that completes a query's count resolves T and writes the selection.  The
// lists pass between workgroups through device-coherent stores and loads, each store
// complete before its workgroup's count is raised.  No workgroup waits for another.
constexpr int kFusedThreads = 512;
constexpr int kFusedPer = kChunk1 / kFusedThreads;     // scores per thread of a chunk
constexpr int kFusedCandLds = 4096;                      // candidates the finisher holds in LDS
#ifndef HCA_SELECT_FUSED_GRID
#define HCA_SELECT_FUSED_GRID 512
#endif
__global__ void __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(4))) select_fused_kernel(IndexerArgs a, SelectWs ws) {
  __shared__ uint32_t s_hist[kBins];
  // collect: a chunk's candidates from the front, its keys above d1 from the back;
  // finish: the query's candidates (kChunk1 <= kFusedCandLds)
  __shared__ __attribute__((aligned(16))) uint32_t s_ck[kFusedCandLds];
  __shared__ int32_t s_cj[kFusedCandLds];
  __shared__ __attribute__((aligned(16))) uint32_t s_sk[kMergedMaxK];
  __shared__ __attribute__((aligned(16))) int32_t s_sj[kMergedMaxK + 32];
  __shared__ int s_pref[kDigitMinQ + 1];
  __shared__ uint32_t s_wave[kFusedThreads / 64 + 1];
  __shared__ int s_found;
  __shared__ uint32_t s_need, s_ns, s_n, s_na, s_base, s_abase, s_last;
  static_assert(kChunk1 <= kFusedCandLds, "a chunk's appends fit the candidate arrays");
  static_assert(kFusedCandLds >= kBins + kMergedMaxK && kFusedCandLds >= kMergedMaxK, "ordering scratch fits");
  const int tid = threadIdx.x;
  // items of query t: one per chunk of its visible entries (one when it keeps them all)
  {
    int items = 0;
    if (tid < a.Nq) {
      const int64_t V = visible(a, tid);
      items = V <= (int64_t)a.k ? 1 : (int)((V + kChunk1 - 1) / kChunk1);
    }
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan<kFusedThreads>((uint32_t)items, s_wave, &tot);
    if (tid < a.Nq) s_pref[tid] = (int)pre;
    if (tid == 0) s_pref[a.Nq] = (int)tot;
    __syncthreads();
  }
  const int total = s_pref[a.Nq];
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int lo = 0, hi = a.Nq - 1;                           // the query whose items hold `item`
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int n = lo, c = item - s_pref[n];
    const int nitems = s_pref[n + 1] - s_pref[n];
    const int64_t V = visible(a, n);
    const int64_t K = V < a.k ? V : a.k;
    const float* sc = reinterpret_cast<const float*>(a.scores) + (int64_t)n * a.score_pitch;
    int32_t* const out = a.idx + (int64_t)n * a.k;
    float* const so = reinterpret_cast<float*>(a.score_out);
    if (V <= K) {                                        // every visible entry, at its own position
      for (int64_t p = tid; p < a.k; p += kFusedThreads) {
        out[p] = p < V ? (int32_t)p : -1;
        if (so) so[(int64_t)n * a.k + p] = p < V ? sc[p] : 0.0f;
      }
      continue;
    }
    // ---- collect: this chunk's scores (requested first), the first digit d1
    const int64_t j0 = (int64_t)c * kChunk1;
    const int64_t j1 = j0 + kChunk1 < V ? j0 + kChunk1 : V;
    const int64_t jt = j0 + (int64_t)kFusedPer * tid;
    uint32_t key[kFusedPer];
#pragma unroll
    for (int v = 0; v < kFusedPer / 4; ++v) {
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      if (jt + 4 * v < j1) f = *reinterpret_cast<const float4*>(sc + jt + 4 * v);   // rows padded to 64
      key[4 * v] = float_key(f.x); key[4 * v + 1] = float_key(f.y);
      key[4 * v + 2] = float_key(f.z); key[4 * v + 3] = float_key(f.w);
    }
    const uint32_t* gh = a.hist + (int64_t)n * kBins;
    for (int i = tid; i < kBins; i += kFusedThreads) s_hist[i] = gh[i];
    if (tid == 0) { s_n = 0; s_na = 0; }
    __syncthreads();
    uint32_t need = (uint32_t)K;
    const uint32_t d1 = (uint32_t)find_digit<kFusedThreads>(s_hist, kBins, &need, s_wave, &s_found, &s_need);
#pragma unroll
    for (int e = 0; e < kFusedPer; ++e) {
      const bool in = jt + e < j1;
      const uint32_t dg = key[e] >> 21;
      const bool cand = in && dg == d1, above = in && dg > d1;
      const uint32_t pc = wave_append(&s_n, cand);
      const uint32_t pa = wave_append(&s_na, above);
      if (cand || above) {
        const uint32_t p = cand ? pc : kChunk1 - 1 - pa;
        s_ck[p] = key[e];
        s_cj[p] = (int32_t)(jt + e);
      }
    }
    __syncthreads();
    if (tid == 0) {
      s_base = s_n ? atomicAdd(&ws.cand_count[n], s_n) : 0;
      s_abase = s_na ? atomicAdd(&ws.above_count[n], s_na) : 0;
    }
    __syncthreads();
    const uint32_t cnt = s_n, base = s_base, cna = s_na, abase = s_abase;
    uint32_t* const gk = ws.cand_key + (int64_t)n * kCandCap2;
    uint32_t* const gj = reinterpret_cast<uint32_t*>(ws.cand_idx + (int64_t)n * kCandCap2);
    for (uint32_t i = tid; i < cnt; i += kFusedThreads) {
      const uint32_t p = base + i;
      if (p < (uint32_t)kCandCap2) {
        st_dev(gk + p, s_ck[i]);
        st_dev(gj + p, (uint32_t)s_cj[i]);
      }
    }
    for (uint32_t i = tid; i < cna; i += kFusedThreads) {
      const uint32_t p = abase + i;                      // < k: fewer than k keys lie above d1
      if (p < (uint32_t)a.k) {
        st_dev(ws.above_key + (int64_t)n * a.k + p, s_ck[kChunk1 - 1 - i]);
        st_dev(reinterpret_cast<uint32_t*>(ws.above_idx + (int64_t)n * a.k + p), (uint32_t)s_cj[kChunk1 - 1 - i]);
      }
    }
    // ---- count this chunk done; the last of the query's chunks finishes it.  Every
    // thread's device-coherent stores have completed (the wait) before the count is
    // raised, and the finisher reads the lists with device-coherent loads.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&ws.done[n], 1u) == (uint32_t)(nitems - 1);
    __syncthreads();
    if (!s_last) continue;                               // uniform
    const uint32_t n1 = ld_dev(&ws.cand_count[n]);
    const uint32_t na = min(ld_dev(&ws.above_count[n]), (uint32_t)a.k);
    uint32_t n_eq = 0;
    {
      // the keys above d1 (at most kMergedMaxK) and, when they fit in LDS, the
      // candidates: every load requested before any is stored
      constexpr int kPerC = kFusedCandLds / kFusedThreads, kPerA = kMergedMaxK / kFusedThreads;
      const bool cand_lds = n1 <= (uint32_t)kFusedCandLds;
      uint32_t* const ak = ws.above_key + (int64_t)n * a.k;
      uint32_t* const aj = reinterpret_cast<uint32_t*>(ws.above_idx + (int64_t)n * a.k);
      uint32_t vk[kPerC], vj[kPerC], wk[kPerA], wj[kPerA];
#pragma unroll
      for (int u = 0; u < kPerC; ++u) {
        const uint32_t i = tid + (uint32_t)kFusedThreads * u;
        if (cand_lds && i < n1) { vk[u] = ld_dev(gk + i); vj[u] = ld_dev(gj + i); }
      }
#pragma unroll
      for (int u = 0; u < kPerA; ++u) {
        const uint32_t i = tid + (uint32_t)kFusedThreads * u;
        if (i < na) { wk[u] = ld_dev(ak + i); wj[u] = ld_dev(aj + i); }
      }
#pragma unroll
      for (int u = 0; u < kPerC; ++u) {
        const uint32_t i = tid + (uint32_t)kFusedThreads * u;
        if (cand_lds && i < n1) { s_ck[i] = vk[u]; s_cj[i] = (int32_t)vj[u]; }
      }
#pragma unroll
      for (int u = 0; u < kPerA; ++u) {
        const uint32_t i = tid + (uint32_t)kFusedThreads * u;
        if (i < na) { s_sk[i] = wk[u]; s_sj[i] = (int32_t)wj[u]; }
      }
    }
    if (n1 <= (uint32_t)kFusedCandLds) {
      __syncthreads();
      auto key_at = [&](uint32_t i) { return s_ck[i]; };
      auto idx_at = [&](uint32_t i) { return s_cj[i]; };
      const uint32_t T = resolve_threshold<kFusedThreads>(sc, V, d1, &need, true, key_at, n1, s_hist, s_wave, &s_found,
                                                          &s_need, &n_eq);
      emit_merged<kFusedThreads>(a, ws, n, V, K, T, need, n_eq, true, key_at, idx_at, n1, na, sc, s_hist, s_sk, s_sj,
                                 s_ck, s_ck + kBins, s_cj, s_wave, &s_found, &s_need, &s_ns);
    } else {                                             // in place (or, past kCandCap2, from the scores)
      const bool have = n1 <= (uint32_t)kCandCap2;
      auto key_at = [&](uint32_t i) { return ld_dev(gk + i); };
      auto idx_at = [&](uint32_t i) { return (int32_t)ld_dev(gj + i); };
      const uint32_t T = resolve_threshold<kFusedThreads>(sc, V, d1, &need, have, key_at, n1, s_hist, s_wave, &s_found,
                                                          &s_need, &n_eq);
      emit_merged<kFusedThreads>(a, ws, n, V, K, T, need, n_eq, have, key_at, idx_at, n1, na, sc, s_hist, s_sk, s_sj,
                                 s_ck, s_ck + kBins, s_cj, s_wave, &s_found, &s_need, &s_ns);
    }
    __syncthreads();                                     // LDS reused by the next item
  }
}

}  // namespace

namespace {
struct WsLayout {
  size_t scores, hist, cand_key, cand_idx, chunk_gt, out_off, eq_before, state, d1, above_key, above_idx, total;
  int nch;
  bool merged;
};
WsLayout ws_layout(int Nq, int64_t max_visible, int fmt, int k) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  WsLayout L{};
  const int64_t pitch = (max_visible + 63) / 64 * 64;
  L.scores = 0;
  size_t o = up((size_t)Nq * pitch * (fmt == HCA_F32 ? 8 : 4));
  L.total = o;
  if (fmt == HCA_F32) return L;
  L.nch = (int)((max_visible + kChunk1 - 1) / kChunk1);
  if (L.nch < 1) L.nch = 1;
  L.hist = o;  o = up(o + (size_t)Nq * (kBins + 3) * 4 + 4);    // histogram; candidate, above, done counts; pooling count
  L.cand_key = o; o = up(o + (size_t)Nq * kCandCap2 * 4);
  L.cand_idx = o; o = up(o + (size_t)Nq * kCandCap2 * 4);
  L.chunk_gt = o; o = up(o + (size_t)Nq * L.nch * 4);
  L.out_off = o; o = up(o + (size_t)Nq * L.nch * 4);
  L.eq_before = o; o = up(o + (size_t)Nq * L.nch * 4);
  L.state = o; o = up(o + (size_t)Nq * 2 * 4);
  L.d1 = o; o = up(o + (size_t)Nq * 4);
  L.merged = k >= 1 && k <= kMergedMaxK;
  const size_t kf = L.merged ? (size_t)k : 0;           // keys above the first digit
  L.above_key = o; o = up(o + (size_t)Nq * kf * 4);
  L.above_idx = o; o = up(o + (size_t)Nq * kf * 4);
  L.total = o;
  return L;
}
}  // namespace

// one scoring launch; the head-tile count (H_I / 32) and paging are template arguments
template <int FMT, bool XQ, int TPW>
void launch_score(const IndexerArgs& a, dim3 grid, hipStream_t s, const PoolArgs* pool = nullptr) {
  const bool h2 = a.H_I == 64;
  if constexpr (!XQ && TPW <= 16) {                    // the decode tilings pool_fusable admits
    if (pool) {                                          // grid rows [0, pool_rows) pool
      const dim3 gp(grid.x, grid.y + (unsigned)a.pool_rows);
      if (a.page_shift >= 0) {
        if (h2) hipLaunchKernelGGL((score_pool_kernel<FMT, 2, TPW, true>), gp, dim3(kScoreThreads), 0, s, a, *pool);
        else hipLaunchKernelGGL((score_pool_kernel<FMT, 1, TPW, true>), gp, dim3(kScoreThreads), 0, s, a, *pool);
      } else {
        if (h2) hipLaunchKernelGGL((score_pool_kernel<FMT, 2, TPW, false>), gp, dim3(kScoreThreads), 0, s, a, *pool);
        else hipLaunchKernelGGL((score_pool_kernel<FMT, 1, TPW, false>), gp, dim3(kScoreThreads), 0, s, a, *pool);
      }
      return;
    }
  }
  if (a.page_shift >= 0) {
    if (h2) hipLaunchKernelGGL((score_quant_kernel<FMT, XQ, 2, TPW, true>), grid, dim3(kScoreThreads), 0, s, a);
    else hipLaunchKernelGGL((score_quant_kernel<FMT, XQ, 1, TPW, true>), grid, dim3(kScoreThreads), 0, s, a);
  } else {
    if (h2) hipLaunchKernelGGL((score_quant_kernel<FMT, XQ, 2, TPW, false>), grid, dim3(kScoreThreads), 0, s, a);
    else hipLaunchKernelGGL((score_quant_kernel<FMT, XQ, 1, TPW, false>), grid, dim3(kScoreThreads), 0, s, a);
  }
}

namespace {

// The launches of one query group: the score phase (clear the counters, score) and
// the select phase, each on its own stream.
struct GroupPlan {
  IndexerArgs a;
  WsLayout L;
  SelectWs sw;
};

GroupPlan plan_group(const IndexerArgs& a0) {
  GroupPlan p;
  p.a = a0;
  IndexerArgs& a = p.a;
  p.L = ws_layout(a.Nq, a.max_visible, a.fmt, a.k);
  const WsLayout& L = p.L;
  char* wsb = static_cast<char*>(a.scores);
  a.hist = reinterpret_cast<uint32_t*>(wsb + L.hist);
  const bool many = a.Nq >= kDigitMinQ || a.many;
  SelectWs& sw = p.sw;
  sw.d1 = many ? reinterpret_cast<uint32_t*>(wsb + L.d1) : nullptr;
  sw.cand_count = a.hist + (int64_t)a.Nq * kBins;
  sw.above_count = sw.cand_count + a.Nq;
  sw.done = sw.above_count + a.Nq;
  a.pool_done = sw.done + a.Nq;                          // cleared with the histogram
  sw.above_key = L.merged ? reinterpret_cast<uint32_t*>(wsb + L.above_key) : nullptr;
  sw.above_idx = L.merged ? reinterpret_cast<int32_t*>(wsb + L.above_idx) : nullptr;
  sw.cand_key = reinterpret_cast<uint32_t*>(wsb + L.cand_key);
  sw.cand_idx = reinterpret_cast<int32_t*>(wsb + L.cand_idx);
  sw.chunk_gt = reinterpret_cast<uint32_t*>(wsb + L.chunk_gt);
  sw.out_off = reinterpret_cast<uint32_t*>(wsb + L.out_off);
  sw.eq_before = reinterpret_cast<uint32_t*>(wsb + L.eq_before);
  sw.state = reinterpret_cast<uint32_t*>(wsb + L.state);
  sw.nch = L.nch;
  return p;
}

// pool: the step's pooling, fused into this scoring launch (pool_fusable)
void launch_score_phase(const GroupPlan& p, hipStream_t s, const PoolArgs* pool = nullptr) {
  const IndexerArgs& a = p.a;
  {
    // the scoring kernel histograms the first digit and the collect phase counts
    // candidates and keys above the first digit: clear them first (they are adjacent,
    // and so is the fused pooling's count)
    const int64_t n16 = ((int64_t)a.Nq * (kBins + 3) * 4 + 4 + 15) / 16;
    const unsigned grid = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<uint4*>(a.hist), n16);
  }
  // MXFP4 with few queries takes the decode tiling (chunk-major, HCA_SCORE_TPW4D tiles)
  const bool few4 = a.fmt == HCA_MXFP4 && a.Nq < kFewQ && !p.sw.d1;
  const int tpw = a.fmt == HCA_FP8_E4M3 ? HCA_SCORE_TPW : few4 ? HCA_SCORE_TPW4D : HCA_SCORE_TPW4;
  const int64_t epw = entries_per_wg_t(tpw);
  const int64_t chunks = (a.max_visible + epw - 1) / epw;
  if (a.prof_begin) hipEventRecord(a.prof_begin, s);
  if (chunks > 0) {
    const dim3 g2((unsigned)chunks, a.Nq), gx((unsigned)(chunks * (((int64_t)a.Nq + 7) / 8 * 8)));
    constexpr int T8 = HCA_SCORE_TPW, T4 = HCA_SCORE_TPW4, T4D = HCA_SCORE_TPW4D;
    if (a.fmt == HCA_FP8_E4M3) launch_score<HCA_FP8_E4M3, false, T8>(a, g2, s, pool);
    else if (few4) launch_score<HCA_MXFP4, false, T4D>(a, g2, s, pool);
    else if (HCA_SCORE_XCD_MAJOR) launch_score<HCA_MXFP4, true, T4>(a, gx, s);
    else launch_score<HCA_MXFP4, false, T4>(a, g2, s);
  }
  if (a.prof_end) hipEventRecord(a.prof_end, s);
}

void launch_select_phase(const GroupPlan& p, hipStream_t s) {
  const IndexerArgs& a = p.a;
  const WsLayout& L = p.L;
  const SelectWs& sw = p.sw;
  dim3 cgrid((unsigned)L.nch, a.Nq);
  if (L.merged && !sw.d1) {                              // few queries: one launch
    hipLaunchKernelGGL(select_fused_kernel, dim3(HCA_SELECT_FUSED_GRID), dim3(kFusedThreads), 0, s, a, sw);
    return;
  }
  if (sw.d1) {
    hipLaunchKernelGGL(select_digit_kernel, dim3(a.Nq), dim3(256), 0, s, a, sw);
    hipLaunchKernelGGL(select_collect_kernel<true>, cgrid, dim3(256), 0, s, a, sw);
  } else {
    hipLaunchKernelGGL(select_collect_kernel<false>, cgrid, dim3(256), 0, s, a, sw);
  }
  hipLaunchKernelGGL(select_threshold_kernel, dim3(a.Nq), dim3(kSelectThreads), 0, s, a, sw);
  if (!L.merged) hipLaunchKernelGGL(select_emit_kernel, cgrid, dim3(256), 0, s, a, sw);
}

// Per (device, caller stream), created on first use and kept until the process
// ends: the stream the select phases of a grouped call run on (default priority),
// and one "scored" and one "selected" event per workspace half.  Calls on one
// caller stream are ordered, so they can share these; calls on different caller
// streams get their own, so their event records never interleave.
struct AuxStreams {
  hipStream_t st = nullptr;
  hipEvent_t scored[2] = {nullptr, nullptr}, selected[2] = {nullptr, nullptr}, start = nullptr;
};
std::mutex g_aux_mu;
std::map<std::pair<int, hipStream_t>, AuxStreams> g_aux;   // node-based: entries never move

hipError_t aux_streams(hipStream_t caller, AuxStreams** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_aux_mu);
  AuxStreams& x = g_aux[std::make_pair(dev, caller)];
  if (!x.st) {                                           // all made, or none kept
    AuxStreams y;
    e = hipStreamCreateWithFlags(&y.st, hipStreamNonBlocking);
    for (int h = 0; h < 2 && e == hipSuccess; ++h) {
      e = hipEventCreateWithFlags(&y.scored[h], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&y.selected[h], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&y.start, hipEventDisableTiming);
    if (e != hipSuccess) {
      for (hipEvent_t ev : {y.scored[0], y.scored[1], y.selected[0], y.selected[1], y.start})
        if (ev) (void)hipEventDestroy(ev);
      if (y.st) (void)hipStreamDestroy(y.st);
      return e;
    }
    x = y;
  }
  *out = &x;
  return hipSuccess;
}

}  // namespace

// Queries per launch group: the quantized path materializes one f32 score row per
// query, so a call with many queries is processed in near-equal groups (a multiple
// of 8 queries, at least kDigitMinQ).  The workspace holds two groups: group g is
// scored on the caller's stream into half g mod 2 while the select phase of group
// g - 1 runs on a second stream (scoring is bound by the vector ALU, the select by
// memory, so the two overlap); each half - score rows and selection lists - fits in
// HCA_INDEXER_WS_BUDGET / 2 bytes.  Every group takes the many-query plan: the same
// scores and the same selection as one launch over all queries.
#ifndef HCA_INDEXER_WS_BUDGET
#define HCA_INDEXER_WS_BUDGET (896ull << 20)
#endif
int indexer_group(int Nq, int64_t max_visible, int fmt, int k) {
  if (fmt == HCA_F32 || Nq <= kDigitMinQ) return Nq;
  const size_t per_q = ws_layout(kDigitMinQ, max_visible, fmt, k).total / kDigitMinQ + 1;
  const size_t budget = ws_layout(Nq, max_visible, fmt, k).total <= HCA_INDEXER_WS_BUDGET ? HCA_INDEXER_WS_BUDGET
                                                                                        : HCA_INDEXER_WS_BUDGET / 2;
  if (budget == HCA_INDEXER_WS_BUDGET) return Nq;                  // one group fits whole
  int64_t gmax = (int64_t)(budget / per_q) / 8 * 8;
  if (gmax < kDigitMinQ) gmax = kDigitMinQ;
  if (gmax >= Nq) return Nq;
  const int64_t ng = (Nq + gmax - 1) / gmax;
  const int64_t g = ((Nq + ng - 1) / ng + 7) / 8 * 8;
  return g < Nq ? (int)g : Nq;
}

size_t indexer_workspace_bytes(int Nq, int64_t max_visible, int fmt, int k) {
  const int G = indexer_group(Nq, max_visible, fmt, k);
  const size_t half = ws_layout(G, max_visible, fmt, k).total;
  return G < Nq ? 2 * half : half;
}

namespace {
// tiles per wave of the chunk-major scoring launch a decode call takes
int fused_tpw(const IndexerArgs& a) { return a.fmt == HCA_FP8_E4M3 ? HCA_SCORE_TPW : HCA_SCORE_TPW4D; }

// The step's pooling can ride in the scoring launch: one query group scored chunk-major
// (FP8, or MXFP4 with few queries), blocks of at most 16 BF16 rows of 512 dims with an
// index stream (the fast pooling path at 256 threads), and at least one key to score.
// No stale copy of a new row can be read: FP8 rows must fill whole 128-byte cache lines
// (pitch and base multiples of 128), so a new row shares no line with a row another
// wave reads, and after its wait and acquire the one wave that reads it cannot meet a
// cached copy, whatever the workgroup-to-XCD mapping; MXFP4 rows (64 bytes, 4-byte
// scales) share lines with their neighbours, so the tile holding the new row is read
// with coherent loads.
bool pool_fusable(const IndexerArgs& a, const PoolArgs& p) {
  if (a.fmt == HCA_F32 || a.max_visible <= 0) return false;
  if (indexer_group(a.Nq, a.max_visible, a.fmt, a.k) < a.Nq) return false;
  if (a.fmt == HCA_FP8_E4M3 && (a.key_pitch % 128 != 0 || reinterpret_cast<uintptr_t>(a.keys) % 128 != 0))
    return false;
  const bool many = a.Nq >= kDigitMinQ || a.many;
  if (a.fmt == HCA_MXFP4 && (a.Nq >= kFewQ || many)) return false;
  return pool_fast_path(p) && p.m <= 16 && p.idx_fmt >= 0 && p.out_idx == a.keys && p.idx_pitch == a.key_pitch;
}
}  // namespace

hipError_t launch_indexer_topk(const IndexerArgs& a0, hipStream_t s, const PoolArgs* pool) {
  if (pool && pool->n_blocks == 0) pool = nullptr;
  if (pool && (a0.Nq == 0 || !pool_fusable(a0, *pool))) {   // pooled by its own launch, first
    const hipError_t e = launch_pool(*pool, s);
    if (e != hipSuccess) return e;
    pool = nullptr;
  }
  if (a0.Nq == 0) return hipSuccess;
  if (a0.fmt == HCA_F32) {
    const int64_t chunks_f64 = (a0.max_visible + 255) / 256;
    if (a0.prof_begin) hipEventRecord(a0.prof_begin, s);
    if (a0.max_visible > 0) {
      size_t lds = (size_t)a0.H_I * a0.d_I * sizeof(float);
      hipLaunchKernelGGL(score_f64_kernel, dim3((unsigned)chunks_f64, a0.Nq), dim3(256), lds, s, a0);
    }
    if (a0.prof_end) hipEventRecord(a0.prof_end, s);
    hipLaunchKernelGGL(select_small_f64_kernel, dim3(a0.Nq), dim3(256), 0, s, a0);
    return hipGetLastError();
  }
  const int G = indexer_group(a0.Nq, a0.max_visible, a0.fmt, a0.k);
  if (G >= a0.Nq) {                                      // one group, one stream
    GroupPlan p = plan_group(a0);
    if (pool) {
      const int64_t chunks = (p.a.max_visible + entries_per_wg_t(fused_tpw(p.a)) - 1) / entries_per_wg_t(fused_tpw(p.a));
      const int64_t cx = chunks > 0 ? chunks : 1;
      p.a.pool_rows = (int)((pool->n_blocks + cx - 1) / cx);
      p.a.pool_target = pool->n_blocks;
    }
    launch_score_phase(p, s, pool);
    launch_select_phase(p, s);
    return hipGetLastError();
  }
  AuxStreams* x = nullptr;
  hipError_t e = aux_streams(s, &x);
  if (e != hipSuccess) return e;
  const size_t half = ws_layout(G, a0.max_visible, a0.fmt, a0.k).total;
  // the second stream starts after everything the caller enqueued before this call
  if ((e = hipEventRecord(x->start, s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(x->st, x->start, 0)) != hipSuccess) return e;
  int ng = 0;
  for (int g0 = 0; g0 < a0.Nq; g0 += G, ++ng) {
    const int h = ng & 1;
    IndexerArgs a = a0;
    a.Nq = a0.Nq - g0 < G ? a0.Nq - g0 : G;
    a.q = a0.q + (int64_t)g0 * a0.H_I * a0.q_pitch;
    if (a0.q_scales) a.q_scales = a0.q_scales + (int64_t)g0 * a0.H_I * a0.q_scale_pitch;
    a.w = a0.w + (int64_t)g0 * a0.H_I;
    a.seq_id = a0.seq_id + g0;
    a.q_pos = a0.q_pos + g0;
    a.idx = a0.idx + (int64_t)g0 * a0.k;
    if (a0.score_out) a.score_out = static_cast<float*>(a0.score_out) + (int64_t)g0 * a0.k;
    if (g0 > 0) a.prof_begin = a.prof_end = nullptr;     // the events bracket the first group's scoring
    a.many = 1;                                          // several groups: the many-query plan for each
    a.scores = static_cast<char*>(a0.scores) + h * half;
    const GroupPlan p = plan_group(a);
    // half h is free once the select phase of group ng - 2 is done
    if (ng >= 2 && (e = hipStreamWaitEvent(s, x->selected[h], 0)) != hipSuccess) return e;
    launch_score_phase(p, s);
    if ((e = hipEventRecord(x->scored[h], s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(x->st, x->scored[h], 0)) != hipSuccess) return e;
    launch_select_phase(p, x->st);
    if ((e = hipEventRecord(x->selected[h], x->st)) != hipSuccess) return e;
  }
  // the caller's stream continues after every group's selection
  for (int h = 0; h < 2 && h < ng; ++h)
    if ((e = hipStreamWaitEvent(s, x->selected[h], 0)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace hca
