// Grouped output projection after attention ("DeepSeek V4 infrastructure"
// (volanea.com), "Compression only works if the attention path is engineered end to
// end": CSA's attention ends in a grouped output projection):
//   y[n, g, c] = sum_{k < K_g} o[n, g * K_g + k] * W[g, c, k],   K_g = (H / G) * D,
// a batch of G products of o's group slice [M, K_g] with W[g]^T [K_g, d_g].
//
// A workgroup computes one group's tile of 64 rows (two 32-row blocks; one when M
// <= 32) by 32 output units.  Its four waves split K_g in four slices; in each,
// lane (j, u) streams 64 contiguous bytes of output unit j's weights (k = kb + 32u
// .. kb + 32u + 31) and of the matching activation rows per 64-k chunk, and the
// chunk feeds four 32x32x16 BF16 MFMAs per row block (MFMA s takes the lane's
// elements 8s .. 8s + 7: the same k permutation for both operands).  Loads run
// one chunk ahead of the products.  The four partial tiles are summed through LDS
// in wave order (deterministic).  With M <= 64 every
// weight is read once per launch: bound by HBM bandwidth on W.
#include "device_common.hpp"
#include "hca_internal.hpp"

namespace hca {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int kGpWaves = 4;

__device__ __forceinline__ v8bf as_bf(const uint4& x) {
  v8bf r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

__device__ __forceinline__ uint16_t bf16_of(float f) {          // round to nearest, ties to even
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int RB, bool OUT_F32>
__global__ void __launch_bounds__(64 * kGpWaves) gproj_kernel(GprojArgs a) {
  __shared__ float s_part[kGpWaves - 1][RB][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 31, u = lane >> 5;
  const int tiles_g = a.d_g / 32;
  const int g = blockIdx.x / tiles_g, c0 = (blockIdx.x - g * tiles_g) * 32;
  const int m0 = blockIdx.y * 32 * RB;
  const int64_t kslice = a.K_g / kGpWaves;
  // this lane's weight row (output unit c0 + j) and activation rows; rows past M read
  // row 0 instead (a row of the product depends on its own activation row only, and
  // such rows are not stored)
  const char* wrow = a.w + ((int64_t)g * a.d_g + c0 + j) * a.w_pitch + (wave * kslice + 32 * u) * 2;
  const char* arow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = m0 + 32 * rb + j;
    arow[rb] = a.o + (int64_t)(r < a.M ? r : 0) * a.o_pitch + (g * a.K_g + wave * kslice + 32 * u) * 2;
  }
  v16f acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb] = (v16f){};
  const int nch = (int)(kslice / 64);
  uint4 wb[4], xb[RB][4];
  auto load = [&](int ch, uint4 (&w4)[4], uint4 (&x4)[RB][4]) {
    const uint4* wp = reinterpret_cast<const uint4*>(wrow + (int64_t)ch * 128);
#pragma unroll
    for (int q = 0; q < 4; ++q) w4[q] = wp[q];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint4* xp = reinterpret_cast<const uint4*>(arow[rb] + (int64_t)ch * 128);
#pragma unroll
      for (int q = 0; q < 4; ++q) x4[rb][q] = xp[q];
    }
  };
  load(0, wb, xb);
  for (int ch = 0; ch < nch; ++ch) {
    uint4 wn[4], xn[RB][4];
    if (ch + 1 < nch) load(ch + 1, wn, xn);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(xb[rb][s]), as_bf(wb[s]), acc[rb], 0, 0, 0);
    }
    if (ch + 1 < nch) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wb[q] = wn[q];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) xb[rb][q] = xn[rb][q];
      }
    }
  }
  // partial tiles of waves 1..3 through LDS; wave 0 sums in wave order and stores
  if (wave > 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s_part[wave - 1][rb][i][lane] = acc[rb][i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = acc[rb][i];
#pragma unroll
      for (int w = 0; w < kGpWaves - 1; ++w) v += s_part[w][rb][i][lane];
      // accumulator layout of the 32x32 product: lane (j, u), element i holds row
      // 8 (i / 4) + 4u + i % 4 of column j
      const int row = m0 + 32 * rb + 8 * (i >> 2) + 4 * u + (i & 3);
      if (row < a.M) {
        char* yp = a.y + (int64_t)row * a.y_pitch + ((int64_t)g * a.d_g + c0 + j) * (OUT_F32 ? 4 : 2);
        if (OUT_F32) *reinterpret_cast<float*>(yp) = v;
        else *reinterpret_cast<uint16_t*>(yp) = bf16_of(v);
      }
    }
  }
}

}  // namespace

int gproj_k_multiple() { return kGpWaves * 64; }

hipError_t launch_gproj(const GprojArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const bool one = a.M <= 32;
  const dim3 grid((unsigned)(a.G * (a.d_g / 32)), (unsigned)((a.M + (one ? 31 : 63)) / (one ? 32 : 64)));
  const dim3 block(64 * kGpWaves);
  if (one) {
    if (a.out_f32) hipLaunchKernelGGL((gproj_kernel<1, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gproj_kernel<1, false>), grid, block, 0, s, a);
  } else {
    if (a.out_f32) hipLaunchKernelGGL((gproj_kernel<2, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gproj_kernel<2, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hca
