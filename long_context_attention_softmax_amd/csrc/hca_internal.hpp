// Internal launch interface between the C ABI layer (hca_abi.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hca {

struct PoolArgs {
  int m, D, D_r, d_I, n_blocks;
  double rope_base;
  int raw_is_f32;
  const void* raw; int64_t raw_pitch;
  const void* raw_idx; int64_t raw_idx_pitch;
  const int64_t* block_row; const int64_t* block_pos; const int64_t* out_row;
  const float* gate_w; const float* gate_b;
  int kv_fmt;                         // HCA_F32 | HCA_FP8_E4M3
  char* out_f32; int64_t out_f32_pitch;
  char* out_nope; int64_t nope_pitch;
  char* out_rope; int64_t rope_pitch;
  float* out_scale;
  int idx_fmt;                        // HCA_F32 | HCA_FP8_E4M3 | HCA_MXFP4 ; -1 = none
  char* out_idx; int64_t idx_pitch;
  char* out_idx_scales; int64_t idx_scale_pitch;
  float* debug;
  double rope_inv[64];                // rope_base^(-2i/D_r), i < D_r / 2, when D_r / 2 <= 64
};
hipError_t launch_pool(const PoolArgs& a, hipStream_t s);

// Cache row of entry j of sequence b: contiguous from row0, or through the page table.
__device__ __forceinline__ int64_t cache_row(const int32_t* pt, int64_t pitch, int shift, int b, int64_t row0,
                                             int64_t j) {
  if (shift < 0) return row0 + j;
  return ((int64_t)pt[(int64_t)b * pitch + (j >> shift)] << shift) + (j & ((1LL << shift) - 1));
}

struct IndexerArgs {
  int Nq, H_I, d_I, k, m, fmt;        // fmt: HCA_F32 | HCA_FP8_E4M3 | HCA_MXFP4
  int64_t max_visible, score_pitch;   // score_pitch: elements per query row of the workspace
  const char* q; int64_t q_pitch; const uint8_t* q_scales; int64_t q_scale_pitch;
  const float* w;
  const char* keys; int64_t key_pitch; const uint8_t* key_scales; int64_t key_scale_pitch;
  const int64_t* cache_row_start; const int32_t* seq_id; const int64_t* q_pos;
  int32_t* idx; void* score_out;
  void* scores;                       // workspace: f32 (quantized) or f64 (F32) [Nq, score_pitch]
  uint32_t* hist;                     // workspace: [Nq, 2048] (quantized only)
  hipEvent_t prof_begin, prof_end;    // optional, around the scoring kernel
  const int32_t* page_table; int64_t page_pitch; int page_shift;   // paged keys (page_shift >= 0)
  int many;                           // set per group of a grouped call: the many-query plan
  // fused decode pooling: grid rows y < pool_rows pool the step's blocks and count
  // themselves in *pool_done; a workgroup that reads its query's newest entry waits
  // for pool_target counts first (0: no pooling in this launch)
  int pool_rows, pool_target;
  uint32_t* pool_done;
};
// pool (optional, decode): blocks to pool before the scores are formed, in the same
// call; fused into the scoring launch where the launch plan allows, else launched first
hipError_t launch_indexer_topk(const IndexerArgs& a, hipStream_t s, const PoolArgs* pool = nullptr);
bool pool_fast_path(const PoolArgs& a);
// a fresh 64-bit epoch for one fused launch (never 0)
uint64_t fused_epoch();
size_t indexer_workspace_bytes(int Nq, int64_t max_visible, int fmt, int k);
// queries per launch group of a call with Nq queries (its workspace holds one group)
int indexer_group(int Nq, int64_t max_visible, int fmt, int k);

struct AttnArgs {
  int Nq, H, D, D_r, mode, m, k, n_win, win_cap, io_f32;
  float tau; double rope_base;
  int64_t max_visible;
  const void* q;
  int cache_fmt;
  const char* c_f32; int64_t c_f32_pitch;
  const char* c_nope; int64_t c_nope_pitch;
  const char* c_rope; int64_t c_rope_pitch;
  const float* c_scale;
  const int64_t* cache_row_start; const int32_t* idx;
  const char* win; int64_t win_pitch;
  const float* sink; const int32_t* seq_id; const int64_t* q_pos;
  void* o; float* lse;
  void* workspace;
  int prefill;
  hipEvent_t prof_begin, prof_end;    // optional, around the attention kernel
  const int32_t* page_table; int64_t page_pitch; int page_shift;   // paged entries (page_shift >= 0)
  int split_chunks, split_runs;       // decode fixed split: chunks per run, most runs of a query (0 = off)
  double inv_turn[32];                // BF16 path: rope_base^(-2i/64) / (2 pi), turns per position
  // fused decode pooling (HCA): workgroups [0, pool_wgs) pool the step's blocks, each
  // setting its flag (flags[0 .. pool_wgs)) to epoch; the one staging a query's newest
  // entry waits for all of them
  int pool_wgs;
  uint64_t* flags;
  uint64_t epoch;
};
// pool (optional, decode): blocks to pool before attention, in the same call; fused
// into the attention launch where the launch plan allows, else launched first
hipError_t launch_attention(const AttnArgs& a, hipStream_t s, const PoolArgs* pool = nullptr);
size_t attention_workspace_bytes(int Nq, int H, int D, int mode, int k, int n_win,
                                 int64_t max_visible, int io_f32, int prefill, int split_chunks);
// most runs of one query under a fixed split of split_chunks chunks (0 when split_chunks <= 0)
int64_t attention_split_runs(int mode, int k, int n_win, int64_t max_visible, int split_chunks);
int attention_max_runs();
// the allocation-free decode entry point's scratch: its size, and its device address
// on the current device (looked up once per device)
size_t attention_static_scratch_bytes();
hipError_t attention_static_scratch(void** ptr);

struct PrologueArgs {
  int Nq, H, D, Nt, W_cap, B, d_I, f32;
  double eps;
  const char* q_in; char* q_out; const float* gamma_q;      // q rows: [Nq * H, D], contiguous
  const char* kv_in; int64_t kv_pitch; const float* gamma_kv;
  const int32_t* tok_seq; const int64_t* tok_pos;
  char* win; int64_t win_pitch;                             // ring row: seq * W_cap + pos mod W_cap
  const char* idx_in; int64_t idx_pitch;                    // optional index stream (copied)
  char* win_idx; int64_t win_idx_pitch;
};
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s);
int prologue_max_dim(int f32);

struct GprojArgs {
  int M, G, d_g, out_f32;
  int64_t K_g;
  const char* o; int64_t o_pitch;     // [M] rows of G * K_g BF16
  const char* w; int64_t w_pitch;     // [G * d_g] rows of K_g BF16
  char* y; int64_t y_pitch;           // [M] rows of G * d_g (f32 or BF16)
};
hipError_t launch_gproj(const GprojArgs& a, hipStream_t s);
int gproj_k_multiple();

}  // namespace hca
