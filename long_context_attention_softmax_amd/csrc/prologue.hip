// Query and key-value normalization ahead of attention, fused with the append of
// each new token to the sliding-window ring ("DeepSeek V4 infrastructure"
// (volanea.com), "Compression only works if the attention path is engineered end to
// end": queries and key-value vectors are normalized on the attention path).
//
// One wave per four query head vectors, or per new token: the rows are loaded once
// into registers (16 bytes per lane per step), each row's sum of squares is formed
// in fp64 (each lane in order, then a fixed butterfly over the wave), and every
// element is scaled in fp64 and rounded once into the storage format.  A row is
// read in full before any of it is written, so q may be normalized in place.  The
// work is one pass over the rows: bound by HBM bandwidth.
#include "device_common.hpp"
#include "hca_internal.hpp"

namespace hca {
namespace {

constexpr int kWaves = 4;         // waves per workgroup
#ifndef HCA_PRO_QROWS
#define HCA_PRO_QROWS 4
#endif
constexpr int kQRows = HCA_PRO_QROWS;   // query rows per wave (their loads issued together)
constexpr int kMaxVec = 8;        // 16-byte vectors per lane: D <= 64 * 8 * (8 BF16 | 4 F32)

template <bool F32>
__device__ __forceinline__ double lane_elem(const uint4& v, int e) {
  const uint32_t w = (&v.x)[F32 ? e : e >> 1];
  if (F32) return (double)__uint_as_float(w);
  return (double)bf16_to_f32((uint16_t)(w >> (16 * (e & 1))));
}

// BF16 bits of y rounded to nearest (ties to even) in one step: y is first rounded
// to binary32 toward zero with the discarded part kept as a sticky last bit (round
// to odd), which leaves 16 bits below the BF16 mantissa, so the second rounding
// cannot differ from a direct one (Boldo and Melquiond's round-to-odd property).
__device__ __forceinline__ uint16_t bf16_rne(double y) {
  const float f = (float)y;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != y) {
    if (fabs(back) > fabs(y)) u -= 1;       // rounded away from zero: step back toward it
    u |= 1u;
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Normalizes R rows (row r: src + r * src_pitch -> dst + r * dst_pitch; rows past
// nrows are skipped): every load is issued before the first reduction.
template <bool F32, int R, int VEC>
__device__ __forceinline__ void norm_rows(const char* src, int64_t src_pitch, char* dst, int64_t dst_pitch,
                                          int nrows, const float* gamma, int D, double eps, int lane) {
  constexpr int kPer = F32 ? 4 : 8;                // elements per 16-byte vector
  const int nv = D / kPer;
  uint4 v[R][VEC];
  float4 gm[VEC][kPer / 4];                          // this lane's scales, loaded once for all rows
  double ss[R];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    const int vi = lane + 64 * i;
    if (vi < nv) {
#pragma unroll
      for (int k = 0; k < kPer / 4; ++k) gm[i][k] = reinterpret_cast<const float4*>(gamma + vi * kPer)[k];
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int vi = lane + 64 * i;
      if (r < nrows && vi < nv) v[r][i] = reinterpret_cast<const uint4*>(src + r * src_pitch)[vi];
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int vi = lane + 64 * i;
      if (r < nrows && vi < nv) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const double x = lane_elem<F32>(v[r][i], e);
          acc += x * x;
        }
      }
    }
    ss[r] = wave_sum(acc);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= nrows) break;
    const double inv = 1.0 / sqrt(ss[r] / (double)D + eps);
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int vi = lane + 64 * i;
      if (vi < nv) {
        uint4 o;
        uint32_t* ow = &o.x;
        const float* g = &gm[i][0].x;                // element e's scale: g[e]
        if (F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            ow[e] = __float_as_uint((float)(lane_elem<true>(v[r][i], e) * inv * (double)g[e]));
        } else {
          // fast path: the binary32 product x * fl32(inv * gamma) is within two binary32
          // units of the exact value, so unless its low 16 bits lie within 4 units of
          // the BF16 midpoint its nearest-even BF16 code is the exact value's; lanes
          // with such an element redo the vector in fp64
          bool slow = false;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t hw[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float sc = (float)(inv * (double)g[2 * e + h]);
              const uint32_t y = __float_as_uint((float)lane_elem<false>(v[r][i], 2 * e + h) * sc);
              slow |= (y & 0xFFFFu) - 0x7FFCu <= 8u;
              hw[h] = (y + 0x7FFFu + ((y >> 16) & 1u)) >> 16;
            }
            ow[e] = hw[0] | (hw[1] << 16);
          }
          if (slow) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint16_t lo = bf16_rne(lane_elem<false>(v[r][i], 2 * e) * inv * (double)g[2 * e]);
              const uint16_t hi = bf16_rne(lane_elem<false>(v[r][i], 2 * e + 1) * inv * (double)g[2 * e + 1]);
              ow[e] = (uint32_t)lo | ((uint32_t)hi << 16);
            }
          }
        }
        reinterpret_cast<uint4*>(dst + r * dst_pitch)[vi] = o;
      }
    }
  }
}

// waves [0, ceil(Nq*H / kQRows)) take kQRows query rows each, the next Nt waves one token each
// VEC: 16-byte vectors per lane and row (D <= 64 * VEC * elements per vector)
template <bool F32, int VEC>
__global__ void __launch_bounds__(64 * kWaves) prologue_kernel(PrologueArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nq = (int64_t)a.Nq * a.H;
  const int64_t qwaves = (nq + kQRows - 1) / kQRows;
  const int64_t rb = (int64_t)a.D * (F32 ? 4 : 2);           // bytes of a q row (contiguous)
  if (wv < qwaves) {
    const int64_t row = wv * kQRows;
    const int n = (int)(nq - row < kQRows ? nq - row : kQRows);
    norm_rows<F32, kQRows, VEC>(a.q_in + row * rb, rb, a.q_out + row * rb, rb, n, a.gamma_q, a.D, a.eps, lane);
    return;
  }
  const int64_t i = wv - qwaves;
  if (i >= a.Nt) return;
  const int b = a.tok_seq[i];
  if (b < 0 || b >= a.B) return;                             // not a sequence of the ring: skipped
  int64_t slot = a.tok_pos[i] % a.W_cap;
  if (slot < 0) slot += a.W_cap;
  const int64_t r = (int64_t)b * a.W_cap + slot;
  norm_rows<F32, 1, VEC>(a.kv_in + i * a.kv_pitch, 0, a.win + r * a.win_pitch, 0, 1, a.gamma_kv, a.D, a.eps, lane);
  if (a.idx_in) {                                            // the index stream: copied as is
    const int n16 = a.d_I * (F32 ? 4 : 2) / 16;
    const uint4* s = reinterpret_cast<const uint4*>(a.idx_in + i * a.idx_pitch);
    uint4* d = reinterpret_cast<uint4*>(a.win_idx + r * a.win_idx_pitch);
    for (int v = lane; v < n16; v += 64) d[v] = s[v];
  }
}

}  // namespace

int prologue_max_dim(int f32) { return 64 * kMaxVec * (f32 ? 4 : 8); }

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s) {
  const int64_t waves = ((int64_t)a.Nq * a.H + kQRows - 1) / kQRows + a.Nt;
  if (waves == 0) return hipSuccess;
  const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
  const int nv = a.D / (a.f32 ? 4 : 8);                      // 16-byte vectors per row
  const dim3 block(64 * kWaves);
#define HCA_PRO(F, V) hipLaunchKernelGGL((prologue_kernel<F, V>), grid, block, 0, s, a)
  if (a.f32) {
    if (nv <= 64) HCA_PRO(true, 1); else if (nv <= 128) HCA_PRO(true, 2);
    else if (nv <= 256) HCA_PRO(true, 4); else HCA_PRO(true, 8);
  } else {
    if (nv <= 64) HCA_PRO(false, 1); else if (nv <= 128) HCA_PRO(false, 2);
    else if (nv <= 256) HCA_PRO(false, 4); else HCA_PRO(false, 8);
  }
#undef HCA_PRO
  return hipGetLastError();
}

}  // namespace hca
