// Grouped output projection after attention ("DeepSeek V4 infrastructure"
// (volanea.com), "Compression only works if the attention path is engineered end to
// end": CSA's attention ends in a grouped output projection):
//   y[n, g, c] = sum_{k < K_g} o[n, g * K_g + k] * W[g, c, k],   K_g = (H / G) * D,
// a batch of G products of o's group slice [M, K_g] with W[g]^T [K_g, d_g].
//
// Three kernels by shape.  Up to 64 rows (decode), gproj_kernel: a workgroup
// computes one group's tile of 64 rows (two 32-row blocks; one when M <= 32) by 32
// output units.  Its four waves split K_g in four slices; per 64-k
// chunk each wave loads its weight tile (32 units x 128 bytes) and activation tiles
// with coalesced 16-byte loads (eight lanes per 128-byte row), stages them in its own
// LDS region, and reads them back in the MFMA operand layout for four 32x32x16 BF16
// MFMAs per row block (MFMA s: lane (j, u) takes row j's k = 32u + 8s .. + 7 of
// both tiles).  Loads run one chunk ahead of the products.  The four partial tiles are summed through LDS
// in wave order (deterministic).  With M <= 64 every
// weight is read once per launch: bound by HBM bandwidth on W.  More rows: the
// 128 x 128 tiled kernel, or for d_g a multiple of 256 and M > 128 (prefill) the
// 256 x 256 four-wave kernel, both over all of K_g with both operand tiles staged
// in double-buffered LDS.
#include "device_common.hpp"
#include "hca_internal.hpp"

namespace hca {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int kGpWaves = 4;

// 16 bytes as a plain vector value: copies of it stay in registers (HIP's v4i is a
// struct, copied through memory when a scheduling barrier sits between its load and
// its store)
__device__ __forceinline__ v8bf as_bf(const v4i& x) { return __builtin_bit_cast(v8bf, x); }

__device__ __forceinline__ uint16_t bf16_of(float f) {          // round to nearest, ties to even
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// LDS tile rows: 64 k of BF16 (128 bytes) plus 16 bytes of padding, so the lanes of
// an MFMA operand read (32 rows, the same 16-byte column) spread over the banks
constexpr int kTileRow = 144;

// NW waves split K_g (8 with one row block, 4 with two: LDS holds both)
template <int RB, bool OUT_F32, int NW>
__global__ void __launch_bounds__(64 * NW) gproj_kernel(GprojArgs a) {
  __shared__ float s_part[NW - 1][RB][16][64];
  // per wave: the weight tile (32 units) and RB activation tiles (32 rows each) of a chunk
  __shared__ __attribute__((aligned(16))) char s_tile[NW][1 + RB][32 * kTileRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 31, u = lane >> 5;
  const int tiles_g = a.d_g / 32;
  const int g = blockIdx.x / tiles_g, c0 = (blockIdx.x - g * tiles_g) * 32;
  const int m0 = blockIdx.y * 32 * RB;
  const int64_t kslice = a.K_g / NW;
  // coalesced loads: in load q, lane l brings 16 bytes (k = 8 (l % 8) .. + 7 of the
  // chunk) of tile row 8q + l / 8; rows past M read row 0 instead (a row of the
  // product depends on its own activation row only, and such rows are not stored)
  const int lr = lane >> 3, lc = lane & 7;
  const char* const wsrc = a.w + ((int64_t)g * a.d_g + c0 + lr) * a.w_pitch + (wave * kslice + 8 * lc) * 2;
  const int64_t wstep = 8 * a.w_pitch;                       // tile row t + 8
  const char* xsrc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = m0 + 32 * rb + 8 * q + lr;
      xsrc[rb][q] = a.o + (int64_t)(r < a.M ? r : 0) * a.o_pitch + (g * a.K_g + wave * kslice + 8 * lc) * 2;
    }
  char* const tiles = s_tile[wave][0];
  const int st_off = lr * kTileRow + 16 * lc;                // this lane's staging slot (tile row lr + 8q)
  v16f acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb] = (v16f){};
  const int nch = (int)(kslice / 64);
  {                                                // chunk 0 into the tiles
    v4i w0[4], x0[RB][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w0[q] = *reinterpret_cast<const v4i*>(wsrc + q * wstep);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) x0[rb][q] = *reinterpret_cast<const v4i*>(xsrc[rb][q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<v4i*>(tiles + st_off + 8 * q * kTileRow) = w0[q];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        *reinterpret_cast<v4i*>(tiles + (1 + rb) * 32 * kTileRow + st_off + 8 * q * kTileRow) = x0[rb][q];
    }
  }
  for (int ch = 0; ch < nch; ++ch) {
    const bool more = ch + 1 < nch;                // uniform
    const int64_t nxt = (int64_t)(more ? ch + 1 : ch) * 128;
    v4i wn[4], xn[RB][4];                        // the next chunk, in flight while this one multiplies
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wn[q] = *reinterpret_cast<const v4i*>(wsrc + q * wstep + nxt);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) xn[rb][q] = *reinterpret_cast<const v4i*>(xsrc[rb][q] + nxt);
    }
    __builtin_amdgcn_sched_barrier(0);            // the loads stay ahead of the products
    // MFMA s: lane (j, u) supplies row j's k = 32u + 8s .. + 7 of both tiles
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int off = j * kTileRow + 64 * u + 16 * s;
      const v4i b = *reinterpret_cast<const v4i*>(tiles + off);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf(*reinterpret_cast<const v4i*>(tiles + (1 + rb) * 32 * kTileRow + off)), as_bf(b), acc[rb], 0, 0, 0);
    }
    // one wave's LDS operations run in order: the reads above complete before the
    // next chunk overwrites the tiles.  Stored also after the last chunk (nothing
    // reads the tiles then): a store under a condition would let the compiler sink
    // the loads above down to it
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<v4i*>(tiles + st_off + 8 * q * kTileRow) = wn[q];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        *reinterpret_cast<v4i*>(tiles + (1 + rb) * 32 * kTileRow + st_off + 8 * q * kTileRow) = xn[rb][q];
    }
  }
  // partial tiles of waves 1..3 through LDS; wave 0 sums in wave order and stores
  if (wave > 0) {   // partial tiles of the other waves
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
      for (int w = 0; w < NW - 1; ++w) v += s_part[w][rb][i][lane];
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

// Many rows (> 64): one group's 128-row x 128-unit tile per workgroup over the whole
// of K_g.  Per 64-k chunk the four waves load both operand tiles together (eight
// lanes per 128-byte row, coalesced) into a double-buffered LDS pair; wave w then
// computes rows 64 (w / 2) .. + 63 by units 64 (w % 2) .. + 63 as 2 x 2 blocks of
// 32x32x16 BF16 MFMAs, each operand fragment read once per k step and used twice.
// Each output is one wave's sum over k in order (deterministic).
constexpr int kTB = 128;          // tile rows and units

template <bool OUT_F32>
__global__ void __launch_bounds__(256) gproj_tiled_kernel(GprojArgs a) {
  __shared__ __attribute__((aligned(16))) char s_a[2][kTB * kTileRow];
  __shared__ __attribute__((aligned(16))) char s_w[2][kTB * kTileRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, u = lane >> 5;
  const int tiles_g = a.d_g / kTB;
  const int g = blockIdx.x / tiles_g, c0 = (blockIdx.x - g * tiles_g) * kTB;
  const int m0 = blockIdx.y * kTB;
  // load slot q of thread t: tile row (256 q + t) / 8, 16-byte column t % 8
  const int lr = tid >> 3, lc = tid & 7;
  const char* asrc[4];
  const char* wsrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = 32 * q + lr;
    const int r = m0 + t;
    asrc[q] = a.o + (int64_t)(r < a.M ? r : 0) * a.o_pitch + ((int64_t)g * a.K_g + 8 * lc) * 2;
    wsrc[q] = a.w + ((int64_t)g * a.d_g + c0 + t) * a.w_pitch + 8 * lc * 2;
  }
  const int st = lr * kTileRow + 16 * lc;                    // + 32 q rows
  v16f acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = (v16f){};
  const int nch = (int)(a.K_g / 64);
  {
    v4i ra[4], rw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = *reinterpret_cast<const v4i*>(asrc[q]);
      rw[q] = *reinterpret_cast<const v4i*>(wsrc[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<v4i*>(s_a[0] + st + 32 * q * kTileRow) = ra[q];
      *reinterpret_cast<v4i*>(s_w[0] + st + 32 * q * kTileRow) = rw[q];
    }
  }
  __syncthreads();
  const int ar = 64 * (wave >> 1), wr = 64 * (wave & 1);    // this wave's rows and units in the tile
  for (int ch = 0; ch < nch; ++ch) {
    const int b = ch & 1;
    const bool more = ch + 1 < nch;                          // uniform
    const int64_t nxt = (int64_t)(more ? ch + 1 : ch) * 128;
    v4i ra[4], rw[4];                                      // the next chunk, in flight
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = *reinterpret_cast<const v4i*>(asrc[q] + nxt);
      rw[q] = *reinterpret_cast<const v4i*>(wsrc[q] + nxt);
    }
    __builtin_amdgcn_sched_barrier(0);                      // the loads stay ahead of the products
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int off = j * kTileRow + 64 * u + 16 * s;
      v8bf fa[2], fw[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        fa[x] = as_bf(*reinterpret_cast<const v4i*>(s_a[b] + (ar + 32 * x) * kTileRow + off));
        fw[x] = as_bf(*reinterpret_cast<const v4i*>(s_w[b] + (wr + 32 * x) * kTileRow + off));
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[x], fw[y], acc[x][y], 0, 0, 0);
    }
    // the other buffer (no one reads it now), also after the last chunk: a store
    // under a condition would let the compiler sink the loads above down to it
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<v4i*>(s_a[b ^ 1] + st + 32 * q * kTileRow) = ra[q];
      *reinterpret_cast<v4i*>(s_w[b ^ 1] + st + 32 * q * kTileRow) = rw[q];
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + ar + 32 * x + 8 * (i >> 2) + 4 * u + (i & 3);
        if (row < a.M) {
          char* yp = a.y + (int64_t)row * a.y_pitch + ((int64_t)g * a.d_g + c0 + wr + 32 * y + j) * (OUT_F32 ? 4 : 2);
          if (OUT_F32) *reinterpret_cast<float*>(yp) = acc[x][y][i];
          else *reinterpret_cast<uint16_t*>(yp) = bf16_of(acc[x][y][i]);
        }
      }
}

// Many rows, wide groups (M > 128, d_g a multiple of 256): a 256-row x 256-unit
// tile per workgroup of four waves, one per SIMD.  Wave w computes rows
// 128 (w / 2) .. + 127 by units 128 (w % 2) .. + 127 as 4 x 4 blocks of 32x32x16
// BF16 MFMAs (256 accumulators a lane), so per k step eight operand fragments read
// from LDS feed sixteen products: half the LDS reads per product of the 128-tile
// kernel.  Same staging (double-buffered LDS, the next 64-k chunk in registers)
// and the same order over k per output.  Workgroups take tiles in an XCD-aware
// order: the dispatcher deals workgroups round-robin to the eight XCDs, so
// workgroup L takes tile (L % 8) * (n / 8) + L / 8 of a group-major, row-block,
// unit-tile order and each XCD works through one contiguous run of it (its
// workgroups share the operand rows in its own L2).
constexpr int kBT = 256;          // tile rows and units

template <bool OUT_F32>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gproj_big_kernel(GprojArgs a) {
  __shared__ __attribute__((aligned(16))) char s_a[2][kBT * kTileRow];
  __shared__ __attribute__((aligned(16))) char s_w[2][kBT * kTileRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, u = lane >> 5;
  const int tiles_g = a.d_g / kBT, mblocks = (a.M + kBT - 1) / kBT;
  const int n = (int)gridDim.x;
  int L = (int)blockIdx.x;
  if ((n & 7) == 0) L = (L & 7) * (n >> 3) + (L >> 3);
  const int g = L / (tiles_g * mblocks);
  const int rem = L - g * tiles_g * mblocks;
  const int mb = rem / tiles_g;
  const int c0 = (rem - mb * tiles_g) * kBT, m0 = mb * kBT;
  // load slot q of thread t: tile row 32 q + t / 8, 16-byte column t % 8
  const int lr = tid >> 3, lc = tid & 7;
  const char* asrc[8];
  const char* wsrc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int t = 32 * q + lr;
    const int r = m0 + t;
    asrc[q] = a.o + (int64_t)(r < a.M ? r : 0) * a.o_pitch + ((int64_t)g * a.K_g + 8 * lc) * 2;
    wsrc[q] = a.w + ((int64_t)g * a.d_g + c0 + t) * a.w_pitch + 8 * lc * 2;
  }
  const int st = lr * kTileRow + 16 * lc;                    // + 32 q rows
  v16f acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = (v16f){};
  const int nch = (int)(a.K_g / 64);
  {
    v4i ra[8], rw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ra[q] = *reinterpret_cast<const v4i*>(asrc[q]);
      rw[q] = *reinterpret_cast<const v4i*>(wsrc[q]);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      *reinterpret_cast<v4i*>(s_a[0] + st + 32 * q * kTileRow) = ra[q];
      *reinterpret_cast<v4i*>(s_w[0] + st + 32 * q * kTileRow) = rw[q];
    }
  }
  __syncthreads();
  const int ar = 128 * (wave >> 1), wr = 128 * (wave & 1);  // this wave's rows and units in the tile
  for (int ch = 0; ch < nch; ++ch) {
    const int b = ch & 1;
    const bool more = ch + 1 < nch;                          // uniform
    const int64_t nxt = (int64_t)(more ? ch + 1 : ch) * 128;
    v4i ra[8], rw[8];                                      // the next chunk, in flight
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ra[q] = *reinterpret_cast<const v4i*>(asrc[q] + nxt);
      rw[q] = *reinterpret_cast<const v4i*>(wsrc[q] + nxt);
    }
    // k steps s = 0..3, the fragments of step s + 1 read while step s multiplies
    v8bf fa[2][4], fw[2][4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      fa[0][x] = as_bf(*reinterpret_cast<const v4i*>(s_a[b] + (ar + 32 * x) * kTileRow + j * kTileRow + 64 * u));
      fw[0][x] = as_bf(*reinterpret_cast<const v4i*>(s_w[b] + (wr + 32 * x) * kTileRow + j * kTileRow + 64 * u));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
        const int off = j * kTileRow + 64 * u + 16 * (s + 1);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          fa[(s + 1) & 1][x] = as_bf(*reinterpret_cast<const v4i*>(s_a[b] + (ar + 32 * x) * kTileRow + off));
          fw[(s + 1) & 1][x] = as_bf(*reinterpret_cast<const v4i*>(s_w[b] + (wr + 32 * x) * kTileRow + off));
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][x], fw[s & 1][y], acc[x][y], 0, 0, 0);
    }
    // the other buffer (no one reads it now), also after the last chunk: a store
    // under a condition would let the compiler sink the loads above down to it
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      *reinterpret_cast<v4i*>(s_a[b ^ 1] + st + 32 * q * kTileRow) = ra[q];
      *reinterpret_cast<v4i*>(s_w[b ^ 1] + st + 32 * q * kTileRow) = rw[q];
    }
    // Issue order of the chunk (one wave per SIMD, so nothing else hides a stall):
    // the step-0 fragments; steps 0 and 1 with a fragment read of the next step
    // after each of their first eight products and one of the sixteen global loads
    // after every second product (issued all at once, they queue behind each other
    // in the memory pipeline and hold up the first products); step 2 with the
    // fragment reads of step 3; step 3 with one LDS store of the next chunk after
    // each product.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);       // 8 LDS reads
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // an MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // an LDS read
        if (i % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // a global load
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);     // an LDS store
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + ar + 32 * x + 8 * (i >> 2) + 4 * u + (i & 3);
        if (row < a.M) {
          char* yp = a.y + (int64_t)row * a.y_pitch + ((int64_t)g * a.d_g + c0 + wr + 32 * y + j) * (OUT_F32 ? 4 : 2);
          if (OUT_F32) *reinterpret_cast<float*>(yp) = acc[x][y][i];
          else *reinterpret_cast<uint16_t*>(yp) = bf16_of(acc[x][y][i]);
        }
      }
}

}  // namespace

int gproj_k_multiple() { return kGpWaves * 64; }

hipError_t launch_gproj(const GprojArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (a.M > 128 && a.d_g % kBT == 0) {                      // many rows, wide groups: 256-wide tiles
    const dim3 grid((unsigned)(a.G * (a.d_g / kBT) * ((a.M + kBT - 1) / kBT)));
    if (a.out_f32) hipLaunchKernelGGL(gproj_big_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(gproj_big_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (a.M > 64 && a.d_g % kTB == 0) {                       // many rows: shared operand tiles
    const dim3 grid((unsigned)(a.G * (a.d_g / kTB)), (unsigned)((a.M + kTB - 1) / kTB));
    if (a.out_f32) hipLaunchKernelGGL(gproj_tiled_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(gproj_tiled_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const bool one = a.M <= 32;
  const dim3 grid((unsigned)(a.G * (a.d_g / 32)), (unsigned)((a.M + (one ? 31 : 63)) / (one ? 32 : 64)));
  if (one && a.K_g % (8 * 64) == 0) {
    if (a.out_f32) hipLaunchKernelGGL((gproj_kernel<1, true, 8>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gproj_kernel<1, false, 8>), grid, dim3(512), 0, s, a);
  } else if (one) {
    if (a.out_f32) hipLaunchKernelGGL((gproj_kernel<1, true, kGpWaves>), grid, dim3(64 * kGpWaves), 0, s, a);
    else hipLaunchKernelGGL((gproj_kernel<1, false, kGpWaves>), grid, dim3(64 * kGpWaves), 0, s, a);
  } else {
    if (a.out_f32) hipLaunchKernelGGL((gproj_kernel<2, true, kGpWaves>), grid, dim3(64 * kGpWaves), 0, s, a);
    else hipLaunchKernelGGL((gproj_kernel<2, false, kGpWaves>), grid, dim3(64 * kGpWaves), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hca
