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
#include "pool_block.hpp"

#include <atomic>
#include <chrono>
#include <random>

namespace hca {

namespace {

constexpr int kPoolThreads = 256;
constexpr int kMaxM = 256, kMaxD = 1024, kMaxDI = 256;

// Raw storage of 8 consecutive elements [8g, 8g+8) of a row: one uint4 (BF16) or
// two (f32); decoded to fp64 on use.
template <bool F32> struct Raw8 { uint4 v[F32 ? 2 : 1]; };

template <bool F32>
__device__ __forceinline__ Raw8<F32> load8(const char* base, int64_t pitch, int64_t row, int g) {
  Raw8<F32> r;
  const uint4* q = reinterpret_cast<const uint4*>(base + row * pitch) + (F32 ? 2 * g : g);
  r.v[0] = q[0];
  if (F32) r.v[F32 ? 1 : 0] = q[1];
  return r;
}

template <bool F32>
__device__ __forceinline__ double elem(const Raw8<F32>& r, int e) {
  if (F32) {
    const uint4 u = r.v[e >> 2];
    const uint32_t w = (e & 3) == 0 ? u.x : (e & 3) == 1 ? u.y : (e & 3) == 2 ? u.z : u.w;
    return (double)__uint_as_float(w);
  }
  const uint4 u = r.v[0];
  const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
  return (double)bf16_to_f32((uint16_t)(w >> (16 * (e & 1))));
}

constexpr int kTokU = 16;     // tokens of one wave in flight
constexpr int kOne = 4;       // tokens of one wave kept in registers (blocks of m <= 16)
constexpr int kPoolHostInv = (int)(sizeof(PoolArgs::rope_inv) / sizeof(double));   // RoPE frequencies from the host

// Partial weighted sums of one wave over the tokens i = wave, wave+4, ... of the block;
// lane handles 8-element groups g = lane, lane+64, ...
template <bool F32>
__device__ __forceinline__ void pool_partial(const char* base, int64_t pitch, int64_t r0, int m, int ngroups,
                                             const double* alpha, double* part, int wave, int lane) {
  for (int g = lane; g < ngroups; g += 64) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i0 = wave; i0 < m; i0 += 4 * kTokU) {
      Raw8<F32> x[kTokU];
#pragma unroll
      for (int j = 0; j < kTokU; ++j)
        if (i0 + 4 * j < m) x[j] = load8<F32>(base, pitch, r0 + i0 + 4 * j, g);
#pragma unroll
      for (int j = 0; j < kTokU; ++j)
        if (i0 + 4 * j < m) {
          const double al = alpha[i0 + 4 * j];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += al * elem<F32>(x[j], e);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[8 * g + e] = acc[e];
  }
}

template <bool F32>
__global__ void __launch_bounds__(kPoolThreads) pool_kernel(PoolArgs a) {
  __shared__ double s_z[kMaxM];
  __shared__ double s_c[kMaxD];
  __shared__ double s_y[kMaxDI];
  __shared__ double s_part[4][kMaxD];
  __shared__ double s_party[4][kMaxDI];
  __shared__ double s_red[kPoolThreads / 64];
  __shared__ double s_bamax[kMaxDI / 32];
  __shared__ double s_rc[kMaxD / 2], s_rs[kMaxD / 2];   // RoPE cos / sin at the entry's position

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = blockIdx.x;
  const int64_t r0 = a.block_row[nb];
  const int64_t p_last = a.block_pos[nb] + a.m - 1;     // RoPE position of the entry
  const int64_t orow = a.out_row[nb];
  const char* raw = static_cast<const char*>(a.raw);
  const char* raw_idx = static_cast<const char*>(a.raw_idx);
  const int ng = a.D / 8, ngi = a.d_I / 8;

  // Small BF16 blocks (m <= 4 kOne tokens, one 8-element group per lane) load each
  // token row (and index-stream row) once: the rows loaded for the gate logits stay
  // in registers for the weighted sums, which add the same terms in the same order
  // as the general path.
  const bool one_pass = !F32 && a.m <= 4 * kOne && ng <= 64 && ngi <= 64;   // uniform
  Raw8<F32> xr[kOne], yr[kOne];
  if (one_pass) {
    if (a.idx_fmt >= 0 && lane < ngi) {
#pragma unroll
      for (int j = 0; j < kOne; ++j)
        if (wave + 4 * j < a.m) yr[j] = load8<F32>(raw_idx, a.raw_idx_pitch, r0 + wave + 4 * j, lane);
    }
    if (lane < ng) {
#pragma unroll
      for (int j = 0; j < kOne; ++j)
        if (wave + 4 * j < a.m) xr[j] = load8<F32>(raw, a.raw_pitch, r0 + wave + 4 * j, lane);
    }
  }
  // gate logits z_i = g . x_i + b_i : wave w takes tokens w, w+4, ...; kTokU in flight
  for (int i0 = wave; i0 < a.m; i0 += 4 * kTokU) {
    double acc[kTokU];
#pragma unroll
    for (int j = 0; j < kTokU; ++j) acc[j] = 0.0;
    for (int g = lane; g < ng; g += 64) {
      const float4* gw4 = reinterpret_cast<const float4*>(a.gate_w) + 2 * g;
      const float4 ga = gw4[0], gb = gw4[1];
      const double gw[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
      Raw8<F32> x[kTokU];
#pragma unroll
      for (int j = 0; j < kTokU; ++j)
        if (i0 + 4 * j < a.m) x[j] = one_pass && j < kOne ? xr[j < kOne ? j : 0] : load8<F32>(raw, a.raw_pitch, r0 + i0 + 4 * j, g);
#pragma unroll
      for (int j = 0; j < kTokU; ++j)
        if (i0 + 4 * j < a.m) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j] += gw[e] * elem<F32>(x[j], e);
        }
    }
#pragma unroll
    for (int j = 0; j < kTokU; ++j) {
      if (i0 + 4 * j >= a.m) break;                      // uniform over the wave
      const double z = wave_sum(acc[j]);
      if (lane == 0) s_z[i0 + 4 * j] = z + (double)a.gate_b[i0 + 4 * j];
    }
  }
  __syncthreads();
  // softmax over the block (wave 0); meanwhile the other waves form the rotation
  // of the entry's RoPE slice (half-split pairs i, half + i) at its last position
  const int half = a.D_r / 2, D_n = a.D - a.D_r;
  if (wave == 0) {
    double mx = -INFINITY;
    for (int i = lane; i < a.m; i += 64) mx = fmax(mx, s_z[i]);
    mx = wave_max(mx);
    double sum = 0.0;
    for (int i = lane; i < a.m; i += 64) { double e = exp(s_z[i] - mx); s_z[i] = e; sum += e; }
    sum = wave_sum(sum);
    for (int i = lane; i < a.m; i += 64) s_z[i] = s_z[i] / sum;
  } else {
    for (int i = tid - 64; i < half; i += kPoolThreads - 64) {
      const double inv = half <= kPoolHostInv ? a.rope_inv[i] : pow(a.rope_base, -2.0 * (double)i / (double)a.D_r);
      double sn, cs;
      sincos((double)p_last * inv, &sn, &cs);
      s_rc[i] = cs;
      s_rs[i] = sn;
    }
  }
  __syncthreads();
  // weighted sums: per-wave partials over interleaved tokens, merged in wave order
  if (one_pass) {
    auto partial = [&](const Raw8<F32> (&r)[kOne], int ngr, double* part) {
      if (lane >= ngr) return;
      double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < kOne; ++j)
        if (wave + 4 * j < a.m) {
          const double al = s_z[wave + 4 * j];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += al * elem<F32>(r[j], e);
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) part[8 * lane + e] = acc[e];
    };
    partial(xr, ng, s_part[wave]);
    if (a.idx_fmt >= 0) partial(yr, ngi, s_party[wave]);
  } else {
    pool_partial<F32>(raw, a.raw_pitch, r0, a.m, ng, s_z, s_part[wave], wave, lane);
    if (a.idx_fmt >= 0)
      pool_partial<F32>(raw_idx, a.raw_idx_pitch, r0, a.m, ngi, s_z, s_party[wave], wave, lane);
  }
  __syncthreads();
  for (int d = tid; d < a.D; d += kPoolThreads)
    s_c[d] = ((s_part[0][d] + s_part[1][d]) + s_part[2][d]) + s_part[3][d];
  if (a.idx_fmt >= 0)
    for (int d = tid; d < a.d_I; d += kPoolThreads)
      s_y[d] = ((s_party[0][d] + s_party[1][d]) + s_party[2][d]) + s_party[3][d];
  __syncthreads();
  // half-split RoPE of the entry's slice at the block's last position
  for (int i = tid; i < half; i += kPoolThreads) {
    const double cs = s_rc[i], sn = s_rs[i];
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

// ---------------------------------------------------------------- D = 512 fast path
// one workgroup per block (the block's arithmetic is pool_d512_block)
template <int NT, int TOK, bool Y>
__global__ void __launch_bounds__(NT) pool_d512_kernel(PoolArgs a) {
  __shared__ PoolSmem<NT, TOK, Y> sm;
  pool_d512_block<NT, TOK, Y>(a, blockIdx.x, sm);
}

}  // namespace

uint64_t fused_epoch() {
  static std::atomic<uint64_t> next{[] {
    std::random_device rd;
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    return (((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ (t * 0x9E3779B97F4A7C15ull)) | 1ull;
  }()};
  return next.fetch_add(2);                            // odd values only: never 0
}

bool pool_fast_path(const PoolArgs& a) {
  return !a.raw_is_f32 && a.D == kFastD && a.D_r == kFastDr && a.m <= 128 &&
         (a.idx_fmt < 0 || (a.d_I % 8 == 0 && a.d_I <= kFastMaxDI)) &&
         (a.D_r / 2 <= (int)(sizeof(PoolArgs::rope_inv) / sizeof(double)));
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  if (a.n_blocks == 0) return hipSuccess;
  if (pool_fast_path(a)) {
    // tokens per wave x waves >= m; the index stream's registers only where it exists
    const bool y = a.idx_fmt >= 0;
    if (a.m <= 16 && y) hipLaunchKernelGGL((pool_d512_kernel<256, 4, true>), dim3(a.n_blocks), dim3(256), 0, s, a);
    else if (a.m <= 16) hipLaunchKernelGGL((pool_d512_kernel<256, 4, false>), dim3(a.n_blocks), dim3(256), 0, s, a);
    else if (y) hipLaunchKernelGGL((pool_d512_kernel<512, 16, true>), dim3(a.n_blocks), dim3(512), 0, s, a);
    // the configuration the attention launch pools with, so both give the same bits
    else hipLaunchKernelGGL((pool_d512_kernel<512, 16, false>), dim3(a.n_blocks), dim3(512), 0, s, a);
    return hipGetLastError();
  }
  if (a.raw_is_f32)
    hipLaunchKernelGGL(pool_kernel<true>, dim3(a.n_blocks), dim3(kPoolThreads), 0, s, a);
  else
    hipLaunchKernelGGL(pool_kernel<false>, dim3(a.n_blocks), dim3(kPoolThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hca
