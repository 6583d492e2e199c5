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
  if (a.mode == HCA_MODE_CSA) {
    const int32_t* ix = a.idx + (int64_t)n * a.k;
    int c = 0;
    // ascending list padded with -1: count the valid prefix by binary search on the first -1
    int lo = 0, hi = a.k;
    while (lo < hi) { int mid = (lo + hi) >> 1; if (ix[mid] >= 0) lo = mid + 1; else hi = mid; }
    c = lo;
    si.n_ent = c;
  } else {
    si.n_ent = (int)V;
  }
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

// Stage set positions [p0, p0 + 32) of query n into Ks as BF16 rows.
__device__ __forceinline__ void stage_chunk(const AttnArgs& a, const SetInfo& si, int n, int b,
                                            int p0, int p_end, __bf16* Ks, uint8_t* kvalid,
                                            const double* s_inv, int nthreads) {
  for (int task = threadIdx.x; task < kChunk * 8; task += nthreads) {
    const int kk = task >> 3, seg = task & 7;
    const int p = p0 + kk;
    uint32_t w[32];
    const int64_t j = (p < si.n_ent && a.mode == HCA_MODE_CSA) ? a.idx[(int64_t)n * a.k + p] : p;
    const bool ok = p < p_end && (p >= si.n_ent || (j >= 0 && j < si.V));
    if (seg == 0) kvalid[kk] = ok;
    if (!ok) {
#pragma unroll
      for (int i = 0; i < 32; ++i) w[i] = 0;
    } else if (p < si.n_ent) {
      const int64_t row = si.row0 + j;
      if (seg < 7) {
        const float sc = a.c_scale[row];
        const uint4* src = reinterpret_cast<const uint4*>(a.c_nope + row * a.c_nope_pitch + seg * 64);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          uint4 u = src[v];
          uint32_t x[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v2bf lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[e], sc, false);
            v2bf hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[e], sc, true);
            uint32_t ulo, uhi;
            __builtin_memcpy(&ulo, &lo, 4);
            __builtin_memcpy(&uhi, &hi, 4);
            w[v * 8 + e * 2] = ulo;
            w[v * 8 + e * 2 + 1] = uhi;
          }
        }
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(a.c_rope + row * a.c_rope_pitch);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          uint4 u = src[v];
          w[v * 4] = u.x; w[v * 4 + 1] = u.y; w[v * 4 + 2] = u.z; w[v * 4 + 3] = u.w;
        }
      }
    } else {
      const int64_t u = si.u0 + (p - si.n_ent);
      const int64_t row = (int64_t)b * a.win_cap + u % a.win_cap;
      const uint4* src = reinterpret_cast<const uint4*>(a.win + row * a.win_pitch + seg * 128);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        uint4 x = src[v];
        w[v * 4] = x.x; w[v * 4 + 1] = x.y; w[v * 4 + 2] = x.z; w[v * 4 + 3] = x.w;
      }
      if (seg == 7) {   // dims 448..511: rotate pairs (448+i, 480+i) at u
        uint32_t rw[32];
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) {        // pairs i = 2*i2, 2*i2+1 share words
          float c0, s0, c1, s1;
          rope_cs(u, s_inv[2 * i2], &c0, &s0);
          rope_cs(u, s_inv[2 * i2 + 1], &c1, &s1);
          const uint32_t lo = w[i2], hi = w[16 + i2];
          const float a0 = bf16_to_f32((uint16_t)lo), a1 = bf16_to_f32((uint16_t)(lo >> 16));
          const float b0 = bf16_to_f32((uint16_t)hi), b1 = bf16_to_f32((uint16_t)(hi >> 16));
          rw[i2] = pack_bf16x2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
          rw[16 + i2] = pack_bf16x2(a0 * s0 + b0 * c0, a1 * s1 + b1 * c1);
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) w[i] = rw[i];
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(Ks + kk * kKsPitch + seg * 64);
#pragma unroll
    for (int v = 0; v < 8; ++v) dst[v] = make_uint4(w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]);
  }
}

template <int NW>   // waves per workgroup = H / 16
__global__ void __launch_bounds__(64 * NW) attn_bf16_kernel(AttnArgs a, int n_splits, int keys_per_split) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kChunk * kKsPitch];
  __shared__ __attribute__((aligned(16))) __bf16 Pb[NW][16 * kPPitch];
  __shared__ double s_inv[32];
  __shared__ uint8_t s_kval[kChunk];
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
  __syncthreads();

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
    stage_chunk(a, si, n, b, p0, p_end, Ks, s_kval, s_inv, 64 * NW);
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
    // online softmax for heads 4g + i (this lane's rows); key = p0 + 16kt + r
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x0 = s_kval[r] ? sc[0][i] * qscale : -INFINITY;
      float x1 = s_kval[16 + r] ? sc[1][i] * qscale : -INFINITY;
      float mx = fmaxf(x0, x1);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float m_new = fmaxf(m_run[i], mx);
      const float al = (m_new == -INFINITY) ? 1.0f : exp2f(m_run[i] - m_new);
      const float e0 = (m_new == -INFINITY) ? 0.0f : exp2f(x0 - m_new);
      const float e1 = (m_new == -INFINITY) ? 0.0f : exp2f(x1 - m_new);
      l_run[i] = l_run[i] * al + (e0 + e1);
      m_run[i] = m_new;
      alpha[i] = al;
      Pb[wave][(4 * g + i) * kPPitch + r] = (__bf16)e0;
      Pb[wave][(4 * g + i) * kPPitch + 16 + r] = (__bf16)e1;
    }
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      acc[dt][0] *= alpha[0]; acc[dt][1] *= alpha[1];
      acc[dt][2] *= alpha[2]; acc[dt][3] *= alpha[3];
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
  const int n = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const SetInfo si = set_info(a, n);
  const int n_set = si.n_ent + si.n_w;
  const int S = (n_set + keys_per_split - 1) / keys_per_split;
  PartialPtrs pp = partial_ptrs(a.workspace, a.Nq, n_splits, a.H);
  const float sig = a.sink[h] * (float)kLog2e;
  float M = sig;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pp.m[((size_t)n * n_splits + s) * a.H + h]);
  float den = exp2f(sig - M);
  for (int s = 0; s < S; ++s) {
    const size_t base = ((size_t)n * n_splits + s) * a.H + h;
    den += pp.l[base] * exp2f(pp.m[base] - M);
  }
  const float inv = 1.0f / den;
  for (int d = tid; d < kD; d += 256) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const size_t base = ((size_t)n * n_splits + s) * a.H + h;
      acc += pp.o[base * kD + d] * exp2f(pp.m[base] - M);
    }
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
  int64_t per = (chunks + s - 1) / s;
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
