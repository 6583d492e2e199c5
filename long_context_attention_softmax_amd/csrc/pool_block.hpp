// Softmax-gated pooling of one block of BF16 rows of 512 dims (the last 64 the RoPE
// slice), as a device function: the pooling kernel runs one block per workgroup, and
// the fused decode launches (pooling inside the scoring or the attention launch) run
// it in their leading workgroups.
//
// "DeepSeek Releases V4 with Million-Token Context Optimized for AI Agents"
// (botbeat.news), "Summary": CSA compresses KV 4x by softmax-gated pooling with a
// learned positional bias; HCA compresses 128x.
#pragma once
#include "device_common.hpp"
#include "hca_internal.hpp"
#include "../../include/hca.h"

namespace hca {

constexpr int kFastD = 512, kFastDr = 64, kFastMaxDI = 256;

// ---------------------------------------------------------------- fused launches
// A pooling workgroup of a fused attention launch signals its block with a 64-bit flag
// set to the call's epoch, a number the host draws once per call (hca::fused_epoch: a
// counter seeded at random per process), so no flag needs clearing before the launch:
// a flag left by an earlier call, or uninitialised memory, holds another value (a
// chance match is one in 2^64).
constexpr uint32_t kFlagSpinMax = 1u << 22;              // polls before a wait gives up

// every thread of the workgroup: its stores complete and written back past the XCD's
// cache, then the workgroup's flag set
__device__ __forceinline__ void flag_set(uint64_t* flag, uint64_t epoch) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// one whole wave: until flags[0 .. n) all hold epoch (bounded), then acquire
__device__ __forceinline__ void flags_wait(uint64_t* flags, int n, uint64_t epoch) {
  const int lane = threadIdx.x & 63;
  for (uint32_t it = 0; it < kFlagSpinMax; ++it) {
    bool ok = true;
    for (int i = lane; i < n; i += 64)
      ok = ok && __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
    if (__all(ok)) break;
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// LDS of one pooling workgroup of NT threads, TOK tokens per wave
template <int NT, int TOK, bool Y>
struct PoolSmem {
  double z[NT / 64 * TOK], e[NT / 64 * TOK];          // gate logits, e^(z_t - max)
  double part[NT / 64][kFastD];
  double party[Y ? NT / 64 : 1][Y ? kFastMaxDI : 1];
  double red[NT / 64];
};

// ---------------------------------------------------------------- D = 512 fast path
// BF16 raw rows of 512 dims (the last 64 the RoPE slice) and an index stream of at
// most 256 dims: one workgroup per block, NT / 64 waves.  Wave w holds tokens
// w, w + NW, ... of the block (TOK at most), lane g the 8-dim group g of each of them,
// all loaded at once and kept in registers from the gate logits to the weighted
// sums; the index stream rides on lanes g < d_I / 8.  Every wave forms the block's
// softmax itself (no barrier between the gate logits and the weighted sums), the
// per-wave partial sums meet in LDS, thread t then owns dims t + NT k; the RoPE pairs
// (448 + i, 480 + i) sit in lanes i and 32 + i of one wave, which formed their
// rotation at the block's last position while the rows were in flight.  Same fp64
// arithmetic and single rounding as the general kernel (sums in another order).

template <int NT, int TOK, bool Y>
__device__ __forceinline__ void pool_d512_block(const PoolArgs& a, int nb, PoolSmem<NT, TOK, Y>& sm) {
  constexpr int NW = NT / 64;
  constexpr int PER = kFastD / NT > 0 ? kFastD / NT : 1;          // dims per thread in the final stage
  constexpr int RW = (448 % NT) / 64;                            // the wave holding dims 448 .. 511
  constexpr int RK = 448 / NT;                                   // ... in its slot RK
  double* const s_z = sm.z;
  double* const s_e = sm.e;
  double (*const s_part)[kFastD] = sm.part;
  double (*const s_party)[Y ? kFastMaxDI : 1] = sm.party;
  double* const s_red = sm.red;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = a.m;
  const int64_t r0 = a.block_row[nb];
  const int64_t p_last = a.block_pos[nb] + m - 1;
  const int64_t orow = a.out_row[nb];
  const bool has_y = Y && a.idx_fmt >= 0;
  const int ngi = has_y ? a.d_I / 8 : 0;
  const char* raw = static_cast<const char*>(a.raw);
  const char* raw_idx = static_cast<const char*>(a.raw_idx);

  // the RoPE frequency of the rotating wave first: waiting for it then does not wait
  // for the rows requested after it
  const double rinv = wave == RW ? a.rope_inv[lane & 31] : 0.0;
  __builtin_amdgcn_sched_barrier(0);
  // every row of this wave's tokens (and index-stream rows), and the gate weights
  uint4 xr[TOK], yr[Y ? TOK : 1];
#pragma unroll
  for (int j = 0; j < TOK; ++j) {
    const int t = wave + NW * j;
    if (t < m) xr[j] = reinterpret_cast<const uint4*>(raw + (r0 + t) * a.raw_pitch)[lane];
    if (Y && t < m && lane < ngi) yr[Y ? j : 0] = reinterpret_cast<const uint4*>(raw_idx + (r0 + t) * a.raw_idx_pitch)[lane];
  }
  const float4* gw4 = reinterpret_cast<const float4*>(a.gate_w) + 2 * lane;
  const float4 ga = gw4[0], gb = gw4[1];
  // the rotation of RoPE pair lane % 32 at the entry's position, while rows load
  double rc = 1.0, rs = 0.0;
  if (wave == RW) sincos((double)p_last * rinv, &rs, &rc);

  // gate logits z_t = g . x_t + b_t
  const double gw[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
  auto el = [](const uint4& u, int e) {
    const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
    return (double)bf16_to_f32((uint16_t)(w >> (16 * (e & 1))));
  };
  double zt[TOK];
#pragma unroll
  for (int j = 0; j < TOK; ++j) {
    double acc = 0.0;
    if (wave + NW * j < m) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += gw[e] * el(xr[j], e);
    }
    zt[j] = acc;
  }
  // the TOK partial dots summed over the wave at once: a reduce-scatter over lane
  // bits 5, 4, ... (each step halves the values a lane keeps), then a butterfly over
  // the remaining bits; lane L ends with the sum of token j = L >> (6 - log2 TOK)
  constexpr int kLogT = TOK >= 16 ? 4 : TOK >= 8 ? 3 : TOK >= 4 ? 2 : TOK >= 2 ? 1 : 0;
  static_assert((1 << kLogT) == TOK, "TOK is a power of two");
#pragma unroll
  for (int st = 0; st < kLogT; ++st) {
    const int o = 32 >> st, half = TOK >> (st + 1);
    const bool upper = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const double mine = upper ? zt[i + half] : zt[i];
      const double give = upper ? zt[i] : zt[i + half];
      zt[i] = mine + __shfl_xor(give, o, 64);
    }
  }
  double zs = zt[0];
#pragma unroll
  for (int o = 32 >> kLogT; o >= 1; o >>= 1) zs += __shfl_xor(zs, o, 64);
  {
    const int t = wave + NW * (lane >> (6 - kLogT));
    if ((lane & ((64 >> kLogT) - 1)) == 0 && t < m) s_z[t] = zs + (double)a.gate_b[t];
  }
  __syncthreads();
  // softmax over the block: alpha_t = e^(z_t - max) / sum; each exponential formed
  // once (thread t), the max and the sum by every wave from LDS in one order
  double mx = -INFINITY;
  for (int i = lane; i < m; i += 64) mx = fmax(mx, s_z[i]);
  mx = wave_max(mx);
  if (tid < m) s_e[tid] = exp(s_z[tid] - mx);
  __syncthreads();
  double esum = 0.0;
  for (int i = lane; i < m; i += 64) esum += s_e[i];
  const double inv = 1.0 / wave_sum(esum);
  // weighted sums of this wave's tokens
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, accy[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < TOK; ++j) {
    const int t = wave + NW * j;
    if (t < m) {
      const double al = s_e[t] * inv;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += al * el(xr[j], e);
      if (Y && lane < ngi) {
#pragma unroll
        for (int e = 0; e < 8; ++e) accy[e] += al * el(yr[Y ? j : 0], e);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_part[wave][8 * lane + e] = acc[e];
  if (Y && lane < ngi) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_party[Y ? wave : 0][8 * lane + e] = accy[e];
  }
  __syncthreads();
  // thread t: dims t + NT k, partials added in wave order
  double c[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = tid + NT * k;
    double v = 0.0;
    if (d < kFastD) {
      v = s_part[0][d];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += s_part[w][d];
    }
    c[k] = v;
  }
  // half-split RoPE of the slice: pair (448 + i, 480 + i) = lanes (i, 32 + i) of wave RW
  if (wave == RW) {
    const double mate = __shfl_xor(c[RK], 32, 64);
    const double x0 = lane < 32 ? c[RK] : mate, x1 = lane < 32 ? mate : c[RK];
    c[RK] = lane < 32 ? x0 * rc - x1 * rs : x0 * rs + x1 * rc;
  }
  double yv = 0.0;
  const int dy = tid;
  if (Y && dy < a.d_I && has_y) {
    yv = s_party[0][dy];
#pragma unroll
    for (int w = 1; w < NW; ++w) yv += s_party[Y ? w : 0][dy];
  }
  if (a.debug) {
    const int W = kFastD + (has_y ? a.d_I : 0);
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (tid + NT * k < kFastD) a.debug[(int64_t)nb * W + tid + NT * k] = (float)c[k];
    if (has_y && dy < a.d_I) a.debug[(int64_t)nb * W + kFastD + dy] = (float)yv;
  }
  // the entry
  if (a.kv_fmt == HCA_F32) {
    float* o = reinterpret_cast<float*>(a.out_f32 + orow * a.out_f32_pitch);
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (tid + NT * k < kFastD) o[tid + NT * k] = (float)c[k];
  } else {
    double am = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (tid + NT * k < kFastD - kFastDr) am = fmax(am, fabs(c[k]));
    am = wave_max(am);
    if (lane == 0) s_red[wave] = am;
    __syncthreads();
    double amax = s_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) amax = fmax(amax, s_red[w]);
    const int se = fp8_entry_scale_exp(amax);
    uint8_t* on = reinterpret_cast<uint8_t*>(a.out_nope + orow * a.nope_pitch);
    uint16_t* orp = reinterpret_cast<uint16_t*>(a.out_rope + orow * a.rope_pitch);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = tid + NT * k;
      if (d < kFastD - kFastDr) on[d] = encode_fp8(ldexp(c[k], -se));
      else if (d < kFastD) orp[d - (kFastD - kFastDr)] = encode_bf16(c[k]);
    }
    if (tid == 0) a.out_scale[orow] = ldexpf(1.0f, se);
  }
  // the index key (thread t: dim t)
  if (a.idx_fmt == HCA_F32) {
    if (dy < a.d_I) reinterpret_cast<float*>(a.out_idx + orow * a.idx_pitch)[dy] = (float)yv;
  } else if (a.idx_fmt == HCA_FP8_E4M3) {
    if (dy < a.d_I) reinterpret_cast<uint8_t*>(a.out_idx + orow * a.idx_pitch)[dy] = encode_fp8(yv);
  } else if (a.idx_fmt == HCA_MXFP4) {
    // 32-element blocks are 32 consecutive lanes of one wave
    double bm = dy < a.d_I ? fabs(yv) : 0.0;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) bm = fmax(bm, __shfl_xor(bm, o, 64));
    const int se = mx_scale_exp(bm);
    const uint8_t code = encode_e2m1(ldexp(yv, -se));
    const uint8_t mate = (uint8_t)__shfl_xor((int)code, 1, 64);
    if (dy < a.d_I && (dy & 1) == 0)
      reinterpret_cast<uint8_t*>(a.out_idx + orow * a.idx_pitch)[dy / 2] = (uint8_t)(code | (mate << 4));
    if (dy < a.d_I && (dy & 31) == 0)
      reinterpret_cast<uint8_t*>(a.out_idx_scales + orow * a.idx_scale_pitch)[dy / 32] = (uint8_t)(se + 127);
  }
}


}  // namespace hca
