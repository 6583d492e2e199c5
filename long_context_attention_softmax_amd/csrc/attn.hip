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
#include "device_common.hpp"
#include "hca_internal.hpp"
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

__device__ __forceinline__ SetInfo set_info(const AttnArgs& a, int n) {
  SetInfo si;
  const int b = a.seq_id[n];
  const int64_t t = a.q_pos[n];
  si.row0 = a.cache_row_start[b];
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
    return (double)reinterpret_cast<const float*>(a.c_f32 + (si.row0 + j) * a.c_f32_pitch)[d];
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
constexpr int kD = 512, kDr = 64, kDn = 448;
constexpr int kChunk = 32;                 // keys staged per step
constexpr int kKsPitch = kD + 8;           // bf16 elements per LDS key row (pad vs bank conflicts)
constexpr int kPPitch = kChunk + 8;
constexpr int kMaxSplitKeys = 1024;        // keys of one slice (index list preloaded in LDS)
constexpr int kMaxSplits = 4096;

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

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

struct PartialPtrs {
  float* m;     // [Nq, S, H]  running max, log2 units
  float* l;     // [Nq, S, H]
  float* o;     // [Nq, S, H, D]
};

__device__ __forceinline__ PartialPtrs partial_ptrs(void* ws, int Nq, int S, int H) {
  PartialPtrs p;
  char* b = static_cast<char*>(ws);
  size_t ml = ((size_t)Nq * S * H * 4 + 255) / 256 * 256;
  p.m = reinterpret_cast<float*>(b);
  p.l = reinterpret_cast<float*>(b + ml);
  p.o = reinterpret_cast<float*>(b + 2 * ml);
  return p;
}

// Staging of set positions [p0, p0 + 32) of a query into Ks as BF16 rows.
// Task (kk, seg): key kk of the chunk, dims [64 seg, 64 seg + 64).  Every branch
// keeps its data in named registers and writes LDS itself (no aggregates that
// would be placed in scratch memory).
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t w, float sc) {
  v2bf v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, sc, HI);
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

// 16 FP8 codes -> 16 BF16 values times the power-of-two scale (exact)
__device__ __forceinline__ void cvt16(uint4 x, float sc, uint4* dst) {
  dst[0] = make_uint4(cvt2<false>(x.x, sc), cvt2<true>(x.x, sc), cvt2<false>(x.y, sc), cvt2<true>(x.y, sc));
  dst[1] = make_uint4(cvt2<false>(x.z, sc), cvt2<true>(x.z, sc), cvt2<false>(x.w, sc), cvt2<true>(x.w, sc));
}

__device__ __forceinline__ uint32_t word(const uint4& u, int i) {
  return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// rotate the 32 pairs (i, 32 + i) of a 64-element BF16 RoPE slice held as 8 uint4
// at position u; writes the rotated slice to dst[0..7]
__device__ __forceinline__ void rope64(const uint4 (&x)[8], int64_t u, const double* s_inv, uint4* dst) {
  uint32_t outw[32];
#pragma unroll
  for (int i2 = 0; i2 < 16; ++i2) {          // pairs 2*i2 and 2*i2+1 share a word
    float c0, s0, c1, s1;
    rope_cs(u, s_inv[2 * i2], &c0, &s0);
    rope_cs(u, s_inv[2 * i2 + 1], &c1, &s1);
    const uint32_t lo = word(x[i2 >> 2], i2 & 3), hi = word(x[4 + (i2 >> 2)], i2 & 3);
    const float a0 = bf16_to_f32((uint16_t)lo), a1 = bf16_to_f32((uint16_t)(lo >> 16));
    const float b0 = bf16_to_f32((uint16_t)hi), b1 = bf16_to_f32((uint16_t)(hi >> 16));
    outw[i2] = pack_bf16x2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
    outw[16 + i2] = pack_bf16x2(a0 * s0 + b0 * c0, a1 * s1 + b1 * c1);
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) dst[v] = make_uint4(outw[4 * v], outw[4 * v + 1], outw[4 * v + 2], outw[4 * v + 3]);
}

__device__ __forceinline__ void stage_task(const AttnArgs& a, const SetInfo& si, int b, int p0, int p_beg,
                                           int p_end, const int32_t* s_idx, int task, __bf16* Ks,
                                           uint8_t* kvalid, const double* s_inv) {
  const int kk = task >> 3, seg = task & 7;
  const int p = p0 + kk;
  uint4* dst = reinterpret_cast<uint4*>(Ks + kk * kKsPitch + seg * 64);
  bool ok = p < p_end;
  int64_t row = 0;
  if (ok && p < si.n_ent) {
    const int64_t j = (a.mode == HCA_MODE_CSA) ? (int64_t)s_idx[p - p_beg] : p;
    ok = j >= 0 && j < si.V;
    row = si.row0 + j;
  }
  if (seg == 0) kvalid[kk] = ok;
  if (!ok) {
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 8; ++v) dst[v] = z;
  } else if (p < si.n_ent && seg < 7) {            // entry: FP8 nope dims
    const uint4* src = reinterpret_cast<const uint4*>(a.c_nope + row * a.c_nope_pitch + seg * 64);
    const uint4 x0 = src[0], x1 = src[1], x2 = src[2], x3 = src[3];
    const float sc = a.c_scale[row];
    cvt16(x0, sc, dst + 0);
    cvt16(x1, sc, dst + 2);
    cvt16(x2, sc, dst + 4);
    cvt16(x3, sc, dst + 6);
  } else if (p < si.n_ent) {                       // entry: BF16 RoPE dims (already rotated)
    const uint4* src = reinterpret_cast<const uint4*>(a.c_rope + row * a.c_rope_pitch);
    uint4 x[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) x[v] = src[v];
#pragma unroll
    for (int v = 0; v < 8; ++v) dst[v] = x[v];
  } else {                                         // window token, raw BF16
    const int64_t u = si.u0 + (p - si.n_ent);
    const int64_t wrow = (int64_t)b * a.win_cap + u % a.win_cap;
    const uint4* src = reinterpret_cast<const uint4*>(a.win + wrow * a.win_pitch + seg * 128);
    uint4 x[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) x[v] = src[v];
    if (seg == 7) {
      rope64(x, u, s_inv, dst);
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) dst[v] = x[v];
    }
  }
}

template <int NW>   // waves per workgroup = H / 16
__global__ void __launch_bounds__(64 * NW) attn_bf16_kernel(AttnArgs a, int n_splits, int keys_per_split) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kChunk * kKsPitch];
  __shared__ __attribute__((aligned(16))) __bf16 Pb[NW][16 * kPPitch];
  __shared__ double s_inv[32];
  __shared__ uint8_t s_kval[kChunk];
  __shared__ int32_t s_idx[kMaxSplitKeys];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, n = blockIdx.y;
  const SetInfo si = set_info(a, n);
  const int n_set = si.n_ent + si.n_w;
  const int p_beg = split * keys_per_split;
  if (p_beg >= n_set) return;                        // uniform: this split is empty
  const int p_end = min(n_set, p_beg + keys_per_split);
  const int b = a.seq_id[n];
  const int64_t t = a.q_pos[n];
  if (tid < 32) s_inv[tid] = pow(a.rope_base, -2.0 * tid / kDr) / kTwoPi;   // turns per position
  if (a.mode == HCA_MODE_CSA) {
    const int p_ent_end = min(p_end, si.n_ent);
    for (int p = p_beg + tid; p < p_ent_end; p += 64 * NW) s_idx[p - p_beg] = a.idx[(int64_t)n * a.k + p];
  }
  __syncthreads();
  constexpr int TPT = (kChunk * 8) / (64 * NW);      // staging tasks per thread

  // Q operands: lane (r, g) of wave w holds head 16w + r, dims 32s + 8g .. +7
  const int head = 16 * wave + r;
  const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) + ((int64_t)n * a.H + head) * kD;
  v8bf qa[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) qa[s] = *reinterpret_cast<const v8bf*>(qrow + 32 * s + 8 * g);
  {
    // rotate the RoPE pairs (448 + i, 480 + i), i = 8g + e, held in k-steps 14 / 15
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c, s;
      rope_cs(t, s_inv[8 * g + e], &c, &s);
      const float x0 = (float)qa[14][e], x1 = (float)qa[15][e];
      qa[14][e] = (__bf16)(x0 * c - x1 * s);
      qa[15][e] = (__bf16)(x0 * s + x1 * c);
    }
  }
  const float qscale = a.tau * (float)kLog2e;        // logits in log2 units

  v4f acc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float l_run[4] = {0.f, 0.f, 0.f, 0.f};

  for (int p0 = p_beg; p0 < p_end; p0 += kChunk) {
#pragma unroll
    for (int q = 0; q < TPT; ++q) stage_task(a, si, b, p0, p_beg, p_end, s_idx, tid + q * 64 * NW, Ks, s_kval, s_inv);
    __syncthreads();
    // S = Q K^T for 32 keys: two 16-key tiles
    v4f sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      v4f c = {0.f, 0.f, 0.f, 0.f};
      const __bf16* kr = Ks + (16 * kt + r) * kKsPitch + 8 * g;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        v8bf kb = *reinterpret_cast<const v8bf*>(kr + 32 * s);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], kb, c, 0, 0, 0);
      }
      sc[kt] = c;
    }
    // online softmax for heads 4g + i (this lane's rows); key = p0 + 16kt + r.
    // m_run is a reference maximum: probabilities are exp2(x - m_run), and O is
    // rescaled only when a row's maximum exceeds its reference by more than 2^8
    // (wave-uniform branch); the final normalization makes the choice exact.
    float x0[4], x1[4], mx[4];
    bool need = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x0[i] = s_kval[r] ? sc[0][i] * qscale : -INFINITY;
      x1[i] = s_kval[16 + r] ? sc[1][i] * qscale : -INFINITY;
      float m = fmaxf(x0[i], x1[i]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      mx[i] = m;
      need |= m > m_run[i] + 8.0f;
    }
    if (__builtin_amdgcn_read_exec() & __ballot(need)) {
      float alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float m_new = fmaxf(m_run[i], mx[i]);
        alpha[i] = (m_run[i] == -INFINITY) ? 0.0f : exp2f(m_run[i] - m_new);
        l_run[i] *= alpha[i];
        m_run[i] = m_new;
      }
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        acc[dt][0] *= alpha[0]; acc[dt][1] *= alpha[1];
        acc[dt][2] *= alpha[2]; acc[dt][3] *= alpha[3];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool live = m_run[i] != -INFINITY;
      const float e0 = live ? exp2f(x0[i] - m_run[i]) : 0.0f;
      const float e1 = live ? exp2f(x1[i] - m_run[i]) : 0.0f;
      l_run[i] += e0 + e1;
      Pb[wave][(4 * g + i) * kPPitch + r] = (__bf16)e0;
      Pb[wave][(4 * g + i) * kPPitch + 16 + r] = (__bf16)e1;
    }
    // P (A operand): lane (r, g) needs P[head r][keys 8g .. 8g+7], written above by
    // other lanes of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const v8bf pa = *reinterpret_cast<const v8bf*>(&Pb[wave][r * kPPitch + 8 * g]);
    // O += P V: V^T operand via transposed LDS reads of the row-major key tile
    const int lr = r >> 2, lc = 4 * (r & 3);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const __bf16* base0 = Ks + (8 * g + lr) * kKsPitch + 16 * dt + lc;
      const __bf16* base1 = base0 + 4 * kKsPitch;
      v4s t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)base0);
      v4s t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)base1);
      v8bf vb;
      __builtin_memcpy(&vb, &t0, 8);
      __builtin_memcpy(reinterpret_cast<char*>(&vb) + 8, &t1, 8);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[dt], 0, 0, 0);
    }
    __syncthreads();
  }
  // full row sums
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float l = l_run[i];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o, 64);
    l_run[i] = l;
  }
  const int hrow0 = 16 * wave + 4 * g;             // this lane's 4 head rows
  if (n_splits == 1) {
    // finalize with the sink
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hrow0 + i;
      const float sig = a.sink[h] * (float)kLog2e;
      const float M = fmaxf(sig, m_run[i]);
      const float sc_o = exp2f(m_run[i] - M);
      const float den = exp2f(sig - M) + l_run[i] * sc_o;
      const float f = sc_o / den;
      __bf16* o = reinterpret_cast<__bf16*>(a.o) + ((int64_t)n * a.H + h) * kD;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) o[16 * dt + r] = (__bf16)(acc[dt][i] * f);
      if (a.lse && r == 0) a.lse[(int64_t)n * a.H + h] = (M + log2f(den)) / (float)kLog2e;
    }
  } else {
    PartialPtrs pp = partial_ptrs(a.workspace, a.Nq, n_splits, a.H);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hrow0 + i;
      const size_t base = ((size_t)n * n_splits + split) * a.H + h;
      if (r == 0) { pp.m[base] = m_run[i]; pp.l[base] = l_run[i]; }
      float* o = pp.o + base * kD;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) o[16 * dt + r] = acc[dt][i];
    }
  }
}

// merge the slices of one (query, head) in slice order, with the sink
__global__ void __launch_bounds__(256) combine_kernel(AttnArgs a, int n_splits, int keys_per_split) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[4];
  const int n = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const SetInfo si = set_info(a, n);
  const int n_set = si.n_ent + si.n_w;
  const int S = (n_set + keys_per_split - 1) / keys_per_split;
  PartialPtrs pp = partial_ptrs(a.workspace, a.Nq, n_splits, a.H);
  const size_t base0 = (size_t)n * n_splits * a.H + h;          // + s * H
  const float sig = a.sink[h] * (float)kLog2e;
  float mx = -INFINITY;
  for (int s = tid; s < S; s += 256) mx = fmaxf(mx, pp.m[base0 + (size_t)s * a.H]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3])), sig);
  __syncthreads();
  for (int s = tid; s < S; s += 256) s_w[s] = exp2f(pp.m[base0 + (size_t)s * a.H] - M);
  __syncthreads();
  if (wave == 0) {                     // fixed-order denominator
    float l = 0.f;
    for (int s = lane; s < S; s += 64) l += pp.l[base0 + (size_t)s * a.H] * s_w[s];
    l = wave_sum(l);
    if (lane == 0) s_red[0] = l;
  }
  __syncthreads();
  const float den = exp2f(sig - M) + s_red[0];
  const float inv = 1.0f / den;
  for (int d = tid; d < kD; d += 256) {
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) acc += pp.o[(base0 + (size_t)s * a.H) * kD + d] * s_w[s];
    reinterpret_cast<__bf16*>(a.o)[((int64_t)n * a.H + h) * kD + d] = (__bf16)(acc * inv);
  }
  if (a.lse && tid == 0) a.lse[(int64_t)n * a.H + h] = (M + log2f(den)) / (float)kLog2e;
}

void split_plan(int Nq, int mode, int k, int n_win, int64_t max_visible, int prefill,
                int* n_splits, int* kps) {
  int64_t max_set = (mode == HCA_MODE_CSA ? (int64_t)k : max_visible) + n_win;
  if (max_set < 1) max_set = 1;
  const int64_t chunks = (max_set + kChunk - 1) / kChunk;
  // aim at >= 512 workgroups, at least 4 chunks per slice
  const int64_t nq = Nq > 0 ? Nq : 1;
  int64_t want = (512 + nq - 1) / nq;
  int64_t s = want < chunks / 4 ? want : chunks / 4;
  if (prefill) s = 1;
  if (s < 1) s = 1;
  const int64_t max_chunks_per_split = kMaxSplitKeys / kChunk;   // CSA index lists live in LDS
  if (mode == HCA_MODE_CSA && (chunks + s - 1) / s > max_chunks_per_split)
    s = (chunks + max_chunks_per_split - 1) / max_chunks_per_split;
  int64_t per = (chunks + s - 1) / s;
  if ((chunks + per - 1) / per > kMaxSplits) per = (chunks + kMaxSplits - 1) / kMaxSplits;
  *kps = (int)(per * kChunk);
  *n_splits = (int)((max_set + *kps - 1) / *kps);
}

}  // namespace

size_t attention_workspace_bytes(int Nq, int H, int D, int mode, int k, int n_win,
                                 int64_t max_visible, int io_f32, int prefill) {
  if (io_f32) return 0;
  int S, kps;
  split_plan(Nq, mode, k, n_win, max_visible, prefill, &S, &kps);
  if (S == 1) return 0;
  size_t ml = ((size_t)Nq * S * H * 4 + 255) / 256 * 256;
  return 2 * ml + (size_t)Nq * S * H * D * 4;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.Nq == 0) return hipSuccess;
  if (a.io_f32) {
    if (a.prof_begin) hipEventRecord(a.prof_begin, s);
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.Nq, a.H), dim3(256), 0, s, a);
    if (a.prof_end) hipEventRecord(a.prof_end, s);
    return hipGetLastError();
  }
  int S, kps;
  split_plan(a.Nq, a.mode, a.k, a.n_win, a.max_visible, a.prefill, &S, &kps);
  const int nw = a.H / 16;
  dim3 grid(S, a.Nq);
  if (a.prof_begin) hipEventRecord(a.prof_begin, s);
  switch (nw) {
    case 1: hipLaunchKernelGGL(attn_bf16_kernel<1>, grid, dim3(64), 0, s, a, S, kps); break;
    case 2: hipLaunchKernelGGL(attn_bf16_kernel<2>, grid, dim3(128), 0, s, a, S, kps); break;
    case 3: hipLaunchKernelGGL(attn_bf16_kernel<3>, grid, dim3(192), 0, s, a, S, kps); break;
    default: hipLaunchKernelGGL(attn_bf16_kernel<4>, grid, dim3(256), 0, s, a, S, kps); break;
  }
  if (a.prof_end) hipEventRecord(a.prof_end, s);
  if (S > 1) hipLaunchKernelGGL(combine_kernel, dim3(a.Nq, a.H), dim3(256), 0, s, a, S, kps);
  return hipGetLastError();
}

}  // namespace hca
