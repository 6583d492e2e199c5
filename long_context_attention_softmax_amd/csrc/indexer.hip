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
// The head sum follows one fixed order - binary32, un-fused:
//     S_g = (((+0 + t_{h0}) + t_{h1}) + ...) over h = 16T + 4g + i (T asc, i asc)
//     I   = (S_0 + S_1) + (S_2 + S_3),      t_h = fl(w_h * max(d_h, +0))
// which is exactly the order the 16x16 MFMA output layout produces: lane (n, g)
// holds heads 16T + 4g + i of entry n, and two butterfly adds combine the groups.
//
// Selection: exact radix select on the orderable 32-bit key of each score, lower
// index first among equal scores, output in ascending index order.
#include "device_common.hpp"
#include "hca_internal.hpp"
#include "../../include/hca.h"

namespace hca {

namespace {

constexpr int kScoreThreads = 256;        // 4 waves x 64 entries
constexpr int kEntriesPerWG = 256;
constexpr int kBins = 2048;               // first radix digit: key bits 31..21
constexpr int kSelectThreads = 1024;
constexpr int kCandCap = 4096;
constexpr int kSmallV = 4096;

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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
  const float* k = reinterpret_cast<const float*>(a.keys + (a.cache_row_start[a.seq_id[n]] + j) * a.key_pitch);
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
// One workgroup scores 256 consecutive entries of one query: each wave takes 64
// entries as four 16-entry MFMA tiles; rows of the MFMA are indexer heads.
template <int FMT>
__global__ void __launch_bounds__(kScoreThreads) score_quant_kernel(IndexerArgs a) {
#pragma clang fp contract(off)
  __shared__ uint32_t s_hist[kBins];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n = blockIdx.y;
  const int64_t V = visible(a, n);
  const int64_t ebase = (int64_t)blockIdx.x * kEntriesPerWG;
  if (ebase >= V) return;                               // uniform over the workgroup
  for (int i = tid; i < kBins; i += kScoreThreads) s_hist[i] = 0;

  const int HT = a.H_I / 16;                            // head tiles (<= 4)
  const int64_t row0 = a.cache_row_start[a.seq_id[n]];
  // A operands: query head rows; lane (r, g) holds head 16T + r
  v8bf qa[4][4];
  v8i qf4[4];
  int qs[4];
  float wv[4][4];
  for (int T = 0; T < 4; ++T) {
    if (T < HT) {
      const int64_t qr = (int64_t)n * a.H_I + 16 * T + r;
      if (FMT == HCA_FP8_E4M3) {
        const uint4* p = reinterpret_cast<const uint4*>(a.q + qr * a.q_pitch + 32 * g);
        uint4 u0 = p[0], u1 = p[1];
        qa[T][0] = fp8x8_to_bf16(u0.x, u0.y);
        qa[T][1] = fp8x8_to_bf16(u0.z, u0.w);
        qa[T][2] = fp8x8_to_bf16(u1.x, u1.y);
        qa[T][3] = fp8x8_to_bf16(u1.z, u1.w);
      } else {
        const uint4 u = *reinterpret_cast<const uint4*>(a.q + qr * a.q_pitch + 16 * g);
        v8i v = {(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
        qf4[T] = v;
        qs[T] = a.q_scales[qr * a.q_scale_pitch + g];
      }
      for (int i = 0; i < 4; ++i) wv[T][i] = a.w[(int64_t)n * a.H_I + 16 * T + 4 * g + i];
    }
  }
  __syncthreads();

  for (int tile = 0; tile < 4; ++tile) {
    const int64_t j = ebase + wave * 64 + tile * 16 + r;
    const bool valid = j < V;
    v4f acc[4];
    if (FMT == HCA_FP8_E4M3) {
      uint4 u0 = {0, 0, 0, 0}, u1 = {0, 0, 0, 0};
      if (valid) {
        const uint4* p = reinterpret_cast<const uint4*>(a.keys + (row0 + j) * a.key_pitch + 32 * g);
        u0 = p[0];
        u1 = p[1];
      }
      v8bf kb[4] = {fp8x8_to_bf16(u0.x, u0.y), fp8x8_to_bf16(u0.z, u0.w),
                    fp8x8_to_bf16(u1.x, u1.y), fp8x8_to_bf16(u1.z, u1.w)};
      for (int T = 0; T < 4; ++T) {
        if (T < HT) {
          v4f c = {0.f, 0.f, 0.f, 0.f};
          for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[T][s], kb[s], c, 0, 0, 0);
          acc[T] = c;
        }
      }
    } else {
      uint4 u = {0, 0, 0, 0};
      int ks = 127;
      if (valid) {
        u = *reinterpret_cast<const uint4*>(a.keys + (row0 + j) * a.key_pitch + 16 * g);
        ks = a.key_scales[(row0 + j) * a.key_scale_pitch + g];
      }
      v8i kv = {(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
      for (int T = 0; T < 4; ++T) {
        if (T < HT) {
          v4f c = {0.f, 0.f, 0.f, 0.f};
          acc[T] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf4[T], kv, c, 4, 4, 0, qs[T], 0, ks);
        }
      }
    }
    // canonical head sum
    float S = 0.0f;
    for (int T = 0; T < 4; ++T) {
      if (T < HT) {
        for (int i = 0; i < 4; ++i) {
          float d = acc[T][i];
          float t = wv[T][i] * (d > 0.0f ? d : 0.0f);
          S = S + t;
        }
      }
    }
    S = S + __shfl_xor(S, 16, 64);
    S = S + __shfl_xor(S, 32, 64);
    if (g == 0 && valid) {
      reinterpret_cast<float*>(a.scores)[(int64_t)n * a.score_pitch + j] = S;
      atomicAdd(&s_hist[float_key(S) >> 21], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)n * kBins;
  for (int i = tid; i < kBins; i += kScoreThreads) {
    uint32_t c = s_hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

__global__ void __launch_bounds__(256) zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

// ------------------------------------------------------------------- select
// Exclusive scan over the 1024 threads of a workgroup (scan order = thread order).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
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
    uint32_t t = lane < kSelectThreads / 64 ? s_wave[lane] : 0;
    uint32_t u = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      uint32_t y = __shfl_up(u, o, 64);
      if (lane >= o) u += y;
    }
    if (lane < kSelectThreads / 64) s_wave[lane] = u - t;   // exclusive wave offsets
    if (lane == kSelectThreads / 64 - 1) s_wave[kSelectThreads / 64] = u;
  }
  __syncthreads();
  uint32_t r = s_wave[wave] + x - v;
  *total = s_wave[kSelectThreads / 64];
  __syncthreads();
  return r;
}

// Given a histogram (counts per digit, digits ordered by key), find the digit that
// holds the need-th largest key.  Returns the digit and sets *need to the rank
// still needed inside it.
__device__ int find_digit(const uint32_t* hist, int nbins, uint32_t* need, uint32_t* s_wave,
                          int* s_found, uint32_t* s_need) {
  const int tid = threadIdx.x;
  if (tid == 0) { *s_found = 0; *s_need = 1; }
  // thread t covers digits [per*t', per*t'+per) counted from the top
  const int per = nbins / kSelectThreads;           // 2 (2048 bins) or 1 (1024 bins)
  const int top = nbins - 1 - tid * per;            // highest digit of this thread
  uint32_t c = 0;
  for (int q = 0; q < per; ++q) c += hist[top - q];
  uint32_t tot;
  uint32_t above = block_exclusive_scan(c, s_wave, &tot);
  const uint32_t nd = *need;
  for (int q = 0; q < per; ++q) {
    uint32_t h = hist[top - q];
    if (above < nd && nd <= above + h) {
      *s_found = top - q;
      *s_need = nd - above;
    }
    above += h;
  }
  __syncthreads();
  *need = *s_need;
  int d = *s_found;
  __syncthreads();
  return d;
}

__global__ void __launch_bounds__(kSelectThreads) select_radix_kernel(IndexerArgs a) {
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_ck[kCandCap];
  __shared__ int32_t s_cj[kCandCap];
  __shared__ uint32_t s_wave[kSelectThreads / 64 + 1];
  __shared__ int s_found;
  __shared__ uint32_t s_need, s_ncand;
  const int tid = threadIdx.x;
  const int n = blockIdx.x;
  const int64_t V = visible(a, n);
  const uint32_t K = (uint32_t)(V < a.k ? V : a.k);
  const float* sc = reinterpret_cast<const float*>(a.scores) + (int64_t)n * a.score_pitch;
  float* so = reinterpret_cast<float*>(a.score_out);
  int32_t* out = a.idx + (int64_t)n * a.k;
  uint32_t* gh = a.hist + (int64_t)n * kBins;

  for (int i = tid; i < kBins; i += kSelectThreads) s_hist[i] = gh[i];
  __syncthreads();

  uint32_t T = 0, take_eq = 0;          // threshold key and how many keys == T to keep
  if ((int64_t)K < V) {
    uint32_t need = K;
    const int d1 = find_digit(s_hist, kBins, &need, s_wave, &s_found, &s_need);
    uint32_t prefix = (uint32_t)d1;
    const uint32_t n1 = s_hist[d1];
    const bool in_lds = n1 <= (uint32_t)kCandCap;
    if (in_lds) {
      if (tid == 0) s_ncand = 0;
      __syncthreads();
      for (int64_t j = tid; j < V; j += kSelectThreads) {
        uint32_t key = float_key(sc[j]);
        if ((key >> 21) == prefix) {
          uint32_t p = atomicAdd(&s_ncand, 1u);
          if (p < (uint32_t)kCandCap) {
            s_ck[p] = key;
            s_cj[p] = (int32_t)j;
          }
        }
      }
      __syncthreads();
    }
    // digits 2 (bits 20..10) and 3 (bits 9..0)
    for (int round = 0; round < 2; ++round) {
      const int shift = round == 0 ? 10 : 0;
      const int nbits = round == 0 ? 11 : 10;
      const int nb = 1 << nbits;
      for (int i = tid; i < kBins; i += kSelectThreads) s_hist[i] = 0;
      __syncthreads();
      if (in_lds) {
        for (uint32_t c = tid; c < n1; c += kSelectThreads) {
          uint32_t key = s_ck[c];
          if ((key >> (shift + nbits)) == prefix) atomicAdd(&s_hist[(key >> shift) & (nb - 1)], 1u);
        }
      } else {
        for (int64_t j = tid; j < V; j += kSelectThreads) {
          uint32_t key = float_key(sc[j]);
          if ((key >> (shift + nbits)) == prefix) atomicAdd(&s_hist[(key >> shift) & (nb - 1)], 1u);
        }
      }
      __syncthreads();
      const int dd = find_digit(s_hist, nb < 1024 ? 1024 : nb, &need, s_wave, &s_found, &s_need);
      prefix = (prefix << nbits) | (uint32_t)dd;
    }
    T = prefix;
    take_eq = need;
  } else {
    T = 0;              // every visible entry is kept
    take_eq = 0xFFFFFFFFu;
  }

  // ordered output pass: tiles of 4 consecutive entries per thread
  uint32_t run_gt = 0, run_eq = 0;
  for (int64_t base = 0; base < V; base += 4 * kSelectThreads) {
    const int64_t j0 = base + 4 * (int64_t)tid;
    uint32_t kk[4];
    int ngt = 0, neq = 0;
    for (int e = 0; e < 4; ++e) {
      int64_t j = j0 + e;
      kk[e] = 0;
      if (j < V) {
        kk[e] = float_key(sc[j]);
        if ((int64_t)K >= V) { ngt++; }
        else if (kk[e] > T) ngt++;
        else if (kk[e] == T) neq++;
      }
    }
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan((uint32_t)ngt | ((uint32_t)neq << 16), s_wave, &tot);
    uint32_t gt_before = run_gt + (pre & 0xFFFF);
    uint32_t eq_before = run_eq + (pre >> 16);
    for (int e = 0; e < 4; ++e) {
      int64_t j = j0 + e;
      if (j >= V) break;
      bool is_gt = ((int64_t)K >= V) || kk[e] > T;
      bool is_eq = !is_gt && kk[e] == T;
      if (is_gt || (is_eq && eq_before < take_eq)) {
        uint32_t pos = gt_before + (eq_before < take_eq ? eq_before : take_eq);
        if (pos >= K) continue;      // only reachable with inconsistent counts
        out[pos] = (int32_t)j;
        if (so) so[(int64_t)n * a.k + pos] = sc[j];
      }
      if (is_gt) gt_before++;
      if (is_eq) eq_before++;
    }
    run_gt += tot & 0xFFFF;
    run_eq += tot >> 16;
  }
  for (int p = (int)K + tid; p < a.k; p += kSelectThreads) {
    out[p] = -1;
    if (so) so[(int64_t)n * a.k + p] = 0.0f;
  }
}

}  // namespace

size_t indexer_workspace_bytes(int Nq, int64_t max_visible, int fmt) {
  const int64_t pitch = (max_visible + 63) / 64 * 64;
  size_t b = (size_t)Nq * pitch * (fmt == HCA_F32 ? 8 : 4);
  b = (b + 255) / 256 * 256;
  if (fmt != HCA_F32) b += (size_t)Nq * kBins * 4;
  return b;
}

hipError_t launch_indexer_topk(const IndexerArgs& a0, hipStream_t s) {
  IndexerArgs a = a0;
  if (a.Nq == 0) return hipSuccess;
  const int64_t chunks_f64 = (a.max_visible + 255) / 256;
  if (a.fmt == HCA_F32) {
    if (a.prof_begin) hipEventRecord(a.prof_begin, s);
    if (a.max_visible > 0) {
      size_t lds = (size_t)a.H_I * a.d_I * sizeof(float);
      hipLaunchKernelGGL(score_f64_kernel, dim3((unsigned)chunks_f64, a.Nq), dim3(256), lds, s, a);
    }
    if (a.prof_end) hipEventRecord(a.prof_end, s);
    hipLaunchKernelGGL(select_small_f64_kernel, dim3(a.Nq), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int64_t chunks = (a.max_visible + kEntriesPerWG - 1) / kEntriesPerWG;
  {
    // the first radix digit is histogrammed by the scoring kernel: clear it first
    const int64_t n16 = (int64_t)a.Nq * kBins * 4 / 16;
    const unsigned grid = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<uint4*>(a.hist), n16);
  }
  if (a.prof_begin) hipEventRecord(a.prof_begin, s);
  if (chunks > 0) {
    if (a.fmt == HCA_FP8_E4M3)
      hipLaunchKernelGGL(score_quant_kernel<HCA_FP8_E4M3>, dim3((unsigned)chunks, a.Nq), dim3(kScoreThreads), 0, s, a);
    else
      hipLaunchKernelGGL(score_quant_kernel<HCA_MXFP4>, dim3((unsigned)chunks, a.Nq), dim3(kScoreThreads), 0, s, a);
  }
  if (a.prof_end) hipEventRecord(a.prof_end, s);
  hipLaunchKernelGGL(select_radix_kernel, dim3(a.Nq), dim3(kSelectThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hca
