// Softmax-gated pooling of aligned blocks of m raw tokens into compressed entries.
//
// "DeepSeek Releases V4 with Million-Token Context Optimized for AI Agents"
// (botbeat.news), "Summary": CSA compresses KV 4x by softmax-gated pooling with a
// learned positional bias; HCA compresses 128x.  "DeepSeek V4: How They Crushed the
// Million-Token Memory Problem" (sameershanbhag.com), "Two kinds of memory instead
// of one": one entry per 4 / 128 tokens; FP8 KV, FP4 indexer, BF16 RoPE dims.
//
// One workgroup pools one block.  The gate, the softmax, the weighted sum and the
// RoPE rotation run in fp64 (this step is far below 1% of the path's bytes), so the
// single rounding into the storage format is the only rounding that matters.
#include "device_common.hpp"
#include "hca_internal.hpp"
#include "../../include/hca.h"

namespace hca {

namespace {

constexpr int kPoolThreads = 256;
constexpr int kMaxM = 256, kMaxD = 1024, kMaxDI = 256;

__device__ __forceinline__ double load_raw(const char* base, int64_t pitch, int64_t row, int d, int is_f32) {
  const char* p = base + row * pitch;
  if (is_f32) return (double)reinterpret_cast<const float*>(p)[d];
  return (double)bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[d]);
}

__global__ void __launch_bounds__(kPoolThreads) pool_kernel(PoolArgs a) {
  __shared__ double s_z[kMaxM];
  __shared__ double s_c[kMaxD];
  __shared__ double s_y[kMaxDI];
  __shared__ double s_red[kPoolThreads / 64];
  __shared__ double s_bamax[kMaxDI / 32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = blockIdx.x;
  const int64_t r0 = a.block_row[nb];
  const int64_t p_last = a.block_pos[nb] + a.m - 1;     // RoPE position of the entry
  const int64_t orow = a.out_row[nb];
  const char* raw = static_cast<const char*>(a.raw);
  const char* raw_idx = static_cast<const char*>(a.raw_idx);

  // gate logits z_i = g . x_i + b_i : one wave per token, lanes over dims
  for (int i = wave; i < a.m; i += kPoolThreads / 64) {
    double acc = 0.0;
    for (int d = lane; d < a.D; d += 64)
      acc += (double)a.gate_w[d] * load_raw(raw, a.raw_pitch, r0 + i, d, a.raw_is_f32);
    acc = wave_sum(acc);
    if (lane == 0) s_z[i] = acc + (double)a.gate_b[i];
  }
  __syncthreads();
  // softmax over the block (wave 0)
  if (wave == 0) {
    double mx = -INFINITY;
    for (int i = lane; i < a.m; i += 64) mx = fmax(mx, s_z[i]);
    mx = wave_max(mx);
    double sum = 0.0;
    for (int i = lane; i < a.m; i += 64) { double e = exp(s_z[i] - mx); s_z[i] = e; sum += e; }
    sum = wave_sum(sum);
    for (int i = lane; i < a.m; i += 64) s_z[i] = s_z[i] / sum;
  }
  __syncthreads();
  // weighted sums, sequential over the block's tokens
  for (int d = tid; d < a.D; d += kPoolThreads) {
    double c = 0.0;
    for (int i = 0; i < a.m; ++i) c += s_z[i] * load_raw(raw, a.raw_pitch, r0 + i, d, a.raw_is_f32);
    s_c[d] = c;
  }
  if (a.idx_fmt >= 0) {
    for (int d = tid; d < a.d_I; d += kPoolThreads) {
      double y = 0.0;
      for (int i = 0; i < a.m; ++i) y += s_z[i] * load_raw(raw_idx, a.raw_idx_pitch, r0 + i, d, a.raw_is_f32);
      s_y[d] = y;
    }
  }
  __syncthreads();
  // half-split RoPE of the entry's slice at the block's last position
  const int half = a.D_r / 2, D_n = a.D - a.D_r;
  for (int i = tid; i < half; i += kPoolThreads) {
    double inv = pow(a.rope_base, -2.0 * (double)i / (double)a.D_r);
    double sn, cs;
    sincos((double)p_last * inv, &sn, &cs);
    double x0 = s_c[D_n + i], x1 = s_c[D_n + half + i];
    s_c[D_n + i] = x0 * cs - x1 * sn;
    s_c[D_n + half + i] = x0 * sn + x1 * cs;
  }
  __syncthreads();

  if (a.debug) {
    const int W = a.D + (a.idx_fmt >= 0 ? a.d_I : 0);
    for (int d = tid; d < a.D; d += kPoolThreads) a.debug[(int64_t)nb * W + d] = (float)s_c[d];
    if (a.idx_fmt >= 0)
      for (int d = tid; d < a.d_I; d += kPoolThreads) a.debug[(int64_t)nb * W + a.D + d] = (float)s_y[d];
  }

  // encode the entry
  if (a.kv_fmt == HCA_F32) {
    float* o = reinterpret_cast<float*>(a.out_f32 + orow * a.out_f32_pitch);
    for (int d = tid; d < a.D; d += kPoolThreads) o[d] = (float)s_c[d];
  } else {
    double am = 0.0;
    for (int d = tid; d < D_n; d += kPoolThreads) am = fmax(am, fabs(s_c[d]));
    am = wave_max(am);
    if (lane == 0) s_red[wave] = am;
    __syncthreads();
    double amax = s_red[0];
    for (int w = 1; w < kPoolThreads / 64; ++w) amax = fmax(amax, s_red[w]);
    const int se = fp8_entry_scale_exp(amax);
    uint8_t* on = reinterpret_cast<uint8_t*>(a.out_nope + orow * a.nope_pitch);
    for (int d = tid; d < D_n; d += kPoolThreads) on[d] = encode_fp8(ldexp(s_c[d], -se));
    uint16_t* orp = reinterpret_cast<uint16_t*>(a.out_rope + orow * a.rope_pitch);
    for (int d = tid; d < a.D_r; d += kPoolThreads) orp[d] = encode_bf16(s_c[D_n + d]);
    if (tid == 0) a.out_scale[orow] = ldexpf(1.0f, se);
  }
  // encode the indexer key
  if (a.idx_fmt == HCA_F32) {
    float* o = reinterpret_cast<float*>(a.out_idx + orow * a.idx_pitch);
    for (int d = tid; d < a.d_I; d += kPoolThreads) o[d] = (float)s_y[d];
  } else if (a.idx_fmt == HCA_FP8_E4M3) {
    uint8_t* o = reinterpret_cast<uint8_t*>(a.out_idx + orow * a.idx_pitch);
    for (int d = tid; d < a.d_I; d += kPoolThreads) o[d] = encode_fp8(s_y[d]);
  } else if (a.idx_fmt == HCA_MXFP4) {
    const int nblk = a.d_I / 32;
    for (int b = tid; b < nblk; b += kPoolThreads) {
      double m = 0.0;
      for (int e = 0; e < 32; ++e) m = fmax(m, fabs(s_y[b * 32 + e]));
      s_bamax[b] = m;
    }
    __syncthreads();
    uint8_t* o = reinterpret_cast<uint8_t*>(a.out_idx + orow * a.idx_pitch);
    uint8_t* os = reinterpret_cast<uint8_t*>(a.out_idx_scales + orow * a.idx_scale_pitch);
    for (int p = tid; p < a.d_I / 2; p += kPoolThreads) {
      const int se = mx_scale_exp(s_bamax[(2 * p) / 32]);
      uint8_t lo = encode_e2m1(ldexp(s_y[2 * p], -se));
      uint8_t hi = encode_e2m1(ldexp(s_y[2 * p + 1], -se));
      o[p] = (uint8_t)(lo | (hi << 4));
    }
    for (int b = tid; b < nblk; b += kPoolThreads) os[b] = (uint8_t)(mx_scale_exp(s_bamax[b]) + 127);
  }
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  if (a.n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_kernel, dim3(a.n_blocks), dim3(kPoolThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hca
