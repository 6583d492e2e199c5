// C ABI of the hybrid compressed-attention library: host-side argument checks,
// workspace sizing and kernel dispatch.  Every check runs before anything is
// launched, so argument errors never touch the device.
#include <cmath>
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string>

#include "../../include/hca.h"
#include "hca_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define REQUIRE(cond, code, ...) \
  do { if (!(cond)) return fail(code, __VA_ARGS__); } while (0)

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// The optional page table of a cache (indexer keys or attention entries).
int check_pages(const int32_t* table, int64_t pitch, int32_t rows, int64_t max_visible, const int64_t* crs,
                int min_rows) {
  if (!table) {
    REQUIRE(crs, HCA_E_NULL, "cache_row_start is required without a page table");
    return HCA_OK;
  }
  REQUIRE(rows >= 1 && rows <= (1 << 24) && (rows & (rows - 1)) == 0, HCA_E_SHAPE,
          "page_rows=%d must be a power of two in [1, 2^24]", rows);
  REQUIRE(rows >= min_rows, HCA_E_UNSUPPORTED, "page_rows=%d below %d", rows, min_rows);
  REQUIRE(pitch >= (max_visible + rows - 1) / rows, HCA_E_SHAPE,
          "page_table_pitch %lld < ceil(max_visible / page_rows)", (long long)pitch);
  REQUIRE(aligned(table, 4), HCA_E_ALIGN, "page_table misaligned");
  return HCA_OK;
}

int log2_exact(int32_t v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}


int check_kv_planes(const hca_kv_planes& p, int D, int D_r, const char* what, bool need) {
  if (p.fmt == HCA_F32) {
    if (!need) return HCA_OK;
    REQUIRE(p.f32, HCA_E_NULL, "%s.f32 is NULL", what);
    REQUIRE(p.f32_pitch >= 4LL * D, HCA_E_SHAPE, "%s.f32_pitch %lld < 4*D", what, (long long)p.f32_pitch);
    REQUIRE(aligned(p.f32, 4) && p.f32_pitch % 4 == 0, HCA_E_ALIGN, "%s.f32 not 4-byte aligned", what);
  } else if (p.fmt == HCA_FP8_E4M3) {
    if (!need) return HCA_OK;
    REQUIRE(p.nope && p.rope && p.scale, HCA_E_NULL, "%s: nope/rope/scale plane is NULL", what);
    REQUIRE(p.nope_pitch >= D - D_r, HCA_E_SHAPE, "%s.nope_pitch too small", what);
    REQUIRE(p.rope_pitch >= 2LL * D_r, HCA_E_SHAPE, "%s.rope_pitch too small", what);
    REQUIRE(aligned(p.rope, 2) && p.rope_pitch % 2 == 0 && aligned(p.scale, 4), HCA_E_ALIGN,
            "%s: rope must be 2-byte and scale 4-byte aligned", what);
  } else {
    return fail(HCA_E_DTYPE, "%s.fmt %d is not F32 or FP8_E4M3", what, p.fmt);
  }
  return HCA_OK;
}

int elem_bytes(int fmt) { return fmt == HCA_F32 ? 4 : (fmt == HCA_BF16 ? 2 : 1); }

// ------------------------------------------------------------------ kv_compress
int validate_kv_compress(const hca_kv_compress_desc* d) {
  REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
  REQUIRE(d->struct_size == sizeof(hca_kv_compress_desc), HCA_E_VERSION,
          "struct_size %u != %zu", d->struct_size, sizeof(hca_kv_compress_desc));
  REQUIRE(d->m >= 1 && d->m <= 256, HCA_E_SHAPE, "m=%d outside [1, 256]", d->m);
  REQUIRE(d->D >= 8 && d->D <= 1024 && d->D % 8 == 0, HCA_E_SHAPE, "D=%d must be a multiple of 8 in [8, 1024]", d->D);
  REQUIRE(d->D_r >= 0 && d->D_r <= d->D && d->D_r % 2 == 0, HCA_E_SHAPE, "D_r=%d must be even, <= D", d->D_r);
  REQUIRE(d->n_blocks >= 0, HCA_E_SHAPE, "n_blocks=%d < 0", d->n_blocks);
  REQUIRE(d->raw_fmt == HCA_F32 || d->raw_fmt == HCA_BF16, HCA_E_DTYPE, "raw_fmt %d not F32/BF16", d->raw_fmt);
  REQUIRE(d->rope_base > 0.0, HCA_E_SHAPE, "rope_base must be > 0");
  if (d->n_blocks == 0) return HCA_OK;
  REQUIRE(d->raw && d->block_row && d->block_pos && d->out_row && d->gate_w && d->gate_b,
          HCA_E_NULL, "raw, block_row, block_pos, out_row, gate_w and gate_b are required");
  const int eb = elem_bytes(d->raw_fmt);
  REQUIRE(d->raw_pitch >= (int64_t)eb * d->D, HCA_E_SHAPE, "raw_pitch too small");
  REQUIRE(aligned(d->raw, 16) && d->raw_pitch % 16 == 0, HCA_E_ALIGN, "raw rows must be 16-byte aligned");
  REQUIRE(aligned(d->gate_w, 16) && aligned(d->gate_b, 4) && aligned(d->block_row, 8) &&
          aligned(d->block_pos, 8) && aligned(d->out_row, 8), HCA_E_ALIGN, "gate or block arrays misaligned");
  int rc = check_kv_planes(d->out, d->D, d->D_r, "out", true);
  if (rc) return rc;
  if (d->raw_idx) {
    REQUIRE(d->d_I >= 8 && d->d_I <= 256 && d->d_I % 8 == 0, HCA_E_SHAPE, "d_I=%d must be a multiple of 8 in [8, 256]", d->d_I);
    REQUIRE(d->raw_idx_pitch >= (int64_t)eb * d->d_I, HCA_E_SHAPE, "raw_idx pitch too small");
    REQUIRE(aligned(d->raw_idx, 16) && d->raw_idx_pitch % 16 == 0, HCA_E_ALIGN, "raw_idx rows must be 16-byte aligned");
    const hca_idx_planes& o = d->out_idx;
    REQUIRE(o.data, HCA_E_NULL, "out_idx.data is NULL");
    if (o.fmt == HCA_F32) {
      REQUIRE(o.pitch >= 4LL * d->d_I && aligned(o.data, 4) && o.pitch % 4 == 0, HCA_E_SHAPE, "out_idx f32 pitch");
    } else if (o.fmt == HCA_FP8_E4M3) {
      REQUIRE(o.pitch >= d->d_I, HCA_E_SHAPE, "out_idx fp8 pitch");
    } else if (o.fmt == HCA_MXFP4) {
      REQUIRE(d->d_I % 32 == 0, HCA_E_SHAPE, "MXFP4 needs d_I %% 32 == 0");
      REQUIRE(o.scales, HCA_E_NULL, "out_idx.scales is NULL");
      REQUIRE(o.pitch >= d->d_I / 2 && o.scale_pitch >= d->d_I / 32, HCA_E_SHAPE, "out_idx mxfp4 pitch");
    } else {
      return fail(HCA_E_DTYPE, "out_idx.fmt %d unknown", o.fmt);
    }
  }
  return HCA_OK;
}

// ----------------------------------------------------------------- indexer_topk
int validate_indexer(const hca_indexer_topk_desc* d, size_t* ws) {
  REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
  REQUIRE(d->struct_size == sizeof(hca_indexer_topk_desc), HCA_E_VERSION,
          "struct_size %u != %zu", d->struct_size, sizeof(hca_indexer_topk_desc));
  REQUIRE(d->Nq >= 0 && d->B >= 1 && d->H_I >= 1 && d->d_I >= 1 && d->m >= 1, HCA_E_SHAPE,
          "Nq>=0, B>=1, H_I>=1, d_I>=1, m>=1 required");
  REQUIRE(d->k >= 1 && d->k <= (1 << 20), HCA_E_SHAPE, "k=%d outside [1, 2^20]", d->k);
  REQUIRE(d->max_visible >= 0 && d->max_visible < (1LL << 31), HCA_E_SHAPE, "max_visible out of range");
  const int fmt = d->q.fmt;
  REQUIRE(fmt == d->keys.fmt, HCA_E_DTYPE, "q.fmt %d != keys.fmt %d", fmt, d->keys.fmt);
  REQUIRE(fmt == HCA_F32 || fmt == HCA_FP8_E4M3 || fmt == HCA_MXFP4, HCA_E_DTYPE, "indexer fmt %d unknown", fmt);
  if (fmt == HCA_F32) {
    REQUIRE(d->max_visible <= 4096, HCA_E_UNSUPPORTED, "F32 indexer supports at most 4096 visible entries");
    REQUIRE((int64_t)d->H_I * d->d_I <= 16384, HCA_E_UNSUPPORTED, "F32 indexer needs H_I*d_I <= 16384");
  } else {
    REQUIRE(d->d_I == 128, HCA_E_UNSUPPORTED, "quantized indexer needs d_I = 128 (got %d)", d->d_I);
    REQUIRE(d->H_I == 32 || d->H_I == 64, HCA_E_UNSUPPORTED, "quantized indexer needs H_I in {32, 64}");
    REQUIRE(d->max_visible <= 2048LL * 4096, HCA_E_UNSUPPORTED, "quantized indexer supports at most 2^23 visible entries");
  }
  *ws = hca::indexer_workspace_bytes(d->Nq, d->max_visible, fmt, d->k);
  if (d->Nq == 0) return HCA_OK;
  REQUIRE(d->q.data && d->keys.data && d->w && d->seq_id && d->q_pos && d->idx,
          HCA_E_NULL, "q, keys, w, seq_id, q_pos and idx are required");
  int prc = check_pages(d->page_table, d->page_table_pitch, d->page_rows, d->max_visible, d->cache_row_start,
                        fmt == HCA_F32 ? 1 : 32);     // quantized scoring: a 32-entry tile within one page
  if (prc) return prc;
  const int64_t row_bytes = fmt == HCA_F32 ? 4LL * d->d_I : (fmt == HCA_FP8_E4M3 ? d->d_I : d->d_I / 2);
  REQUIRE(d->q.pitch >= row_bytes && d->keys.pitch >= row_bytes, HCA_E_SHAPE, "q/keys pitch < row bytes");
  if (fmt != HCA_F32) {
    REQUIRE(aligned(d->q.data, 16) && aligned(d->keys.data, 16) && d->q.pitch % 16 == 0 && d->keys.pitch % 16 == 0,
            HCA_E_ALIGN, "quantized q/keys need 16-byte aligned rows");
  } else {
    REQUIRE(aligned(d->q.data, 4) && aligned(d->keys.data, 4) && d->q.pitch % 4 == 0 && d->keys.pitch % 4 == 0,
            HCA_E_ALIGN, "f32 q/keys need 4-byte aligned rows");
  }
  if (fmt == HCA_MXFP4) {
    REQUIRE(d->q.scales && d->keys.scales && d->q.scale_pitch >= 4 && d->keys.scale_pitch >= 4, HCA_E_NULL,
            "MXFP4 q/keys need scale planes");
    REQUIRE(aligned(d->keys.scales, 4) && d->keys.scale_pitch % 4 == 0, HCA_E_ALIGN,
            "MXFP4 key scale rows must be 4-byte aligned");
  }
  if (fmt != HCA_F32) {   // the scoring kernel addresses key rows with 32-bit offsets from a sequence or page base
    const int64_t span = d->page_table ? (int64_t)d->page_rows : d->max_visible;
    REQUIRE(d->keys.pitch * span < (1LL << 32) && (fmt != HCA_MXFP4 || d->keys.scale_pitch * span < (1LL << 32)),
            HCA_E_UNSUPPORTED, "max_visible (page_rows with pages) x key pitch must be < 2^32 bytes");
    // ... formed by a 24-bit multiply of the row number and the pitch
    REQUIRE(d->keys.pitch < (1LL << 24) && (fmt != HCA_MXFP4 || d->keys.scale_pitch < (1LL << 24)),
            HCA_E_UNSUPPORTED, "quantized key pitches must be < 2^24 bytes");
  }
  REQUIRE(aligned(d->w, 4) && aligned(d->idx, 4) && aligned(d->cache_row_start, 8) && aligned(d->q_pos, 8) &&
          aligned(d->seq_id, 4), HCA_E_ALIGN, "w/idx/cache_row_start/q_pos/seq_id misaligned");
  REQUIRE(d->workspace && d->workspace_bytes >= *ws, HCA_E_WORKSPACE, "workspace needs %zu bytes, got %zu",
          *ws, d->workspace_bytes);
  REQUIRE(aligned(d->workspace, 256), HCA_E_ALIGN, "workspace must be 256-byte aligned");
  return HCA_OK;
}

// ---------------------------------------------------------------------- attention
int validate_attn(const hca_attn_desc* d, int prefill, size_t* ws, bool skip_workspace = false) {
  REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
  REQUIRE(d->struct_size == sizeof(hca_attn_desc), HCA_E_VERSION, "struct_size %u != %zu",
          d->struct_size, sizeof(hca_attn_desc));
  REQUIRE(d->Nq >= 0 && d->B >= 1 && d->H >= 1 && (d->m >= 1 || d->mode == HCA_MODE_SWA) && d->n_win >= 0,
          HCA_E_SHAPE, "Nq>=0, B>=1, H>=1, m>=1, n_win>=0 required");
  REQUIRE(d->mode == HCA_MODE_CSA || d->mode == HCA_MODE_HCA || d->mode == HCA_MODE_SWA, HCA_E_SHAPE,
          "mode %d unknown", d->mode);
  const bool swa = d->mode == HCA_MODE_SWA;
  REQUIRE(d->mode != HCA_MODE_CSA || (d->k >= 1 && d->k <= (1 << 20)), HCA_E_SHAPE, "CSA needs 1 <= k <= 2^20");
  REQUIRE(d->win_cap >= 1 && d->win_cap >= d->n_win, HCA_E_SHAPE, "win_cap must be >= max(1, n_win)");
  REQUIRE(swa || (d->max_visible >= 0 && d->max_visible < (1LL << 31)), HCA_E_SHAPE, "max_visible out of range");
  REQUIRE(d->D_r >= 0 && d->D_r % 2 == 0 && d->D_r <= d->D, HCA_E_SHAPE, "D_r must be even and <= D");
  REQUIRE(d->rope_base > 0.0, HCA_E_SHAPE, "rope_base must be > 0");
  // the window-only mode runs as HCA over no visible entry
  const int emode = swa ? HCA_MODE_HCA : d->mode;
  const int64_t evis = swa ? 0 : d->max_visible;
  const int ek = d->mode == HCA_MODE_CSA ? d->k : 0;
  const int64_t max_set = (emode == HCA_MODE_CSA ? (int64_t)ek : evis) + d->n_win;
  if (d->io_fmt == HCA_F32) {
    REQUIRE(swa || d->cache.fmt == HCA_F32, HCA_E_DTYPE, "io_fmt F32 needs an F32 cache");
    REQUIRE(d->D <= 1024 && d->D >= 2, HCA_E_SHAPE, "F32 attention needs 2 <= D <= 1024");
    REQUIRE(d->D_r <= 1024, HCA_E_SHAPE, "D_r too large");
    REQUIRE(max_set <= 4096, HCA_E_UNSUPPORTED, "F32 attention supports at most 4096 keys per query");
  } else if (d->io_fmt == HCA_BF16) {
    REQUIRE(swa || d->cache.fmt == HCA_FP8_E4M3, HCA_E_DTYPE, "io_fmt BF16 needs an FP8_E4M3 cache");
    REQUIRE(d->D == 512 && d->D_r == 64, HCA_E_UNSUPPORTED, "BF16 attention needs D=512, D_r=64");
    REQUIRE(d->H % 16 == 0 && d->H <= 64, HCA_E_UNSUPPORTED, "BF16 attention needs H in {16,32,48,64}");
  } else {
    return fail(HCA_E_DTYPE, "io_fmt %d is not F32 or BF16", d->io_fmt);
  }
  REQUIRE(d->split_chunks >= 0, HCA_E_SHAPE, "split_chunks=%d < 0", d->split_chunks);
  if (!prefill && d->io_fmt == HCA_BF16 && d->split_chunks > 0) {
    const int64_t runs = hca::attention_split_runs(emode, ek, d->n_win, evis, d->split_chunks);
    REQUIRE(runs <= hca::attention_max_runs(), HCA_E_UNSUPPORTED,
            "split_chunks=%d cuts a query into up to %lld runs (at most %d)", d->split_chunks, (long long)runs,
            hca::attention_max_runs());
    REQUIRE((int64_t)d->Nq * runs < (1LL << 31), HCA_E_UNSUPPORTED, "Nq x runs per query must be < 2^31");
  }
  *ws = hca::attention_workspace_bytes(d->Nq, d->H, d->D, emode, ek, d->n_win, evis,
                                       d->io_fmt == HCA_F32, prefill, d->split_chunks);
  if (d->Nq == 0) return HCA_OK;
  REQUIRE(d->q && d->o && d->win && d->sink && d->seq_id && d->q_pos, HCA_E_NULL,
          "q, o, win, sink, seq_id and q_pos are required");
  if (!swa) {
    int prc = check_pages(d->page_table, d->page_table_pitch, d->page_rows, d->max_visible, d->cache_row_start, 1);
    if (prc) return prc;
  }
  REQUIRE(d->mode != HCA_MODE_CSA || d->idx, HCA_E_NULL, "CSA needs idx");
  int rc = check_kv_planes(d->cache, d->D, d->D_r, "cache", !swa);
  if (rc && !swa) return rc;
  const int eb = elem_bytes(d->io_fmt);
  REQUIRE(d->win_pitch >= (int64_t)eb * d->D, HCA_E_SHAPE, "win_pitch too small");
  if (d->io_fmt == HCA_BF16) {
    REQUIRE(aligned(d->q, 16) && aligned(d->o, 16) && aligned(d->win, 16) && d->win_pitch % 16 == 0 &&
            (swa || (aligned(d->cache.nope, 16) && d->cache.nope_pitch % 16 == 0 && aligned(d->cache.rope, 16) &&
                     d->cache.rope_pitch % 16 == 0)), HCA_E_ALIGN, "BF16 attention needs 16-byte aligned rows");
  } else {
    REQUIRE(aligned(d->q, 4) && aligned(d->o, 4) && aligned(d->win, 4) && d->win_pitch % 4 == 0,
            HCA_E_ALIGN, "F32 attention needs 4-byte aligned rows");
  }
  REQUIRE(aligned(d->sink, 4) && aligned(d->seq_id, 4) && aligned(d->q_pos, 8) && aligned(d->cache_row_start, 8) &&
          (!d->idx || aligned(d->idx, 4)) && (!d->lse || aligned(d->lse, 4)), HCA_E_ALIGN, "index arrays misaligned");
  if (*ws && !skip_workspace) {
    REQUIRE(d->workspace && d->workspace_bytes >= *ws, HCA_E_WORKSPACE, "workspace needs %zu bytes, got %zu",
            *ws, d->workspace_bytes);
    REQUIRE(aligned(d->workspace, 256), HCA_E_ALIGN, "workspace must be 256-byte aligned");
  }
  return HCA_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(HCA_E_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return HCA_OK;
}

// --------------------------------------------------------------- output projection
int validate_out_proj(const hca_out_proj_desc* d) {
  REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
  REQUIRE(d->struct_size == sizeof(hca_out_proj_desc), HCA_E_VERSION, "struct_size %u != %zu",
          d->struct_size, sizeof(hca_out_proj_desc));
  REQUIRE(d->out_fmt == HCA_F32 || d->out_fmt == HCA_BF16, HCA_E_DTYPE, "out_fmt %d is not F32 or BF16",
          d->out_fmt);
  REQUIRE(d->Nq >= 0 && d->H >= 1 && d->D >= 1 && d->G >= 1 && d->d_g >= 1, HCA_E_SHAPE, "bad shapes");
  REQUIRE(d->H % d->G == 0, HCA_E_SHAPE, "H=%d is not a multiple of G=%d", d->H, d->G);
  const int64_t K_g = (int64_t)(d->H / d->G) * d->D;
  REQUIRE(K_g % hca::gproj_k_multiple() == 0 && K_g < (1LL << 30), HCA_E_UNSUPPORTED,
          "K_g = H/G * D = %lld must be a multiple of %d", (long long)K_g, hca::gproj_k_multiple());
  REQUIRE(d->d_g % 32 == 0 && (int64_t)d->G * (d->d_g / 32) < (1LL << 31), HCA_E_UNSUPPORTED,
          "d_g=%d must be a multiple of 32", d->d_g);
  REQUIRE(((int64_t)d->Nq + 31) / 32 < 65536, HCA_E_UNSUPPORTED, "Nq too large for one launch");
  if (d->Nq == 0) return HCA_OK;
  REQUIRE(d->o && d->w && d->y, HCA_E_NULL, "o, w and y are required");
  const int eb = d->out_fmt == HCA_F32 ? 4 : 2;
  REQUIRE(d->o_pitch >= 2LL * d->H * d->D && d->w_pitch >= 2 * K_g &&
          d->y_pitch >= (int64_t)eb * d->G * d->d_g, HCA_E_SHAPE, "o/w/y pitch shorter than a row");
  REQUIRE(aligned(d->o, 16) && aligned(d->w, 16) && aligned(d->y, eb) && d->o_pitch % 16 == 0 &&
          d->w_pitch % 16 == 0 && d->y_pitch % eb == 0, HCA_E_ALIGN, "o / w rows must be 16-byte aligned");
  return HCA_OK;
}

// ------------------------------------------------------------------- qkv prologue
int validate_prologue(const hca_qkv_prologue_desc* d) {
  REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
  REQUIRE(d->struct_size == sizeof(hca_qkv_prologue_desc), HCA_E_VERSION, "struct_size %u != %zu",
          d->struct_size, sizeof(hca_qkv_prologue_desc));
  REQUIRE(d->io_fmt == HCA_F32 || d->io_fmt == HCA_BF16, HCA_E_DTYPE, "io_fmt %d is not F32 or BF16", d->io_fmt);
  const bool f32 = d->io_fmt == HCA_F32;
  const int per = f32 ? 4 : 8, eb = f32 ? 4 : 2;
  REQUIRE(d->Nq >= 0 && d->Nt >= 0, HCA_E_SHAPE, "Nq and Nt must be >= 0");
  REQUIRE(d->D >= per && d->D % per == 0 && d->D <= hca::prologue_max_dim(f32), HCA_E_SHAPE,
          "D=%d must be a multiple of %d in [%d, %d]", d->D, per, per, hca::prologue_max_dim(f32));
  REQUIRE(d->eps >= 0.0 && std::isfinite(d->eps), HCA_E_SHAPE, "eps must be finite and >= 0");
  REQUIRE(d->Nq == 0 || (d->H >= 1 && (int64_t)d->Nq * d->H + d->Nt < (1LL << 33)), HCA_E_SHAPE,
          "H must be >= 1 (and Nq * H + Nt < 2^33)");
  if (d->Nq > 0) {
    REQUIRE(d->q_in && d->q_out && d->gamma_q, HCA_E_NULL, "q_in, q_out and gamma_q are required");
    REQUIRE(aligned(d->q_in, 16) && aligned(d->q_out, 16) && aligned(d->gamma_q, 16), HCA_E_ALIGN,
            "q rows must be 16-byte aligned");
  }
  if (d->Nt > 0) {
    REQUIRE(d->kv_in && d->gamma_kv && d->tok_seq && d->tok_pos && d->win, HCA_E_NULL,
            "kv_in, gamma_kv, tok_seq, tok_pos and win are required");
    REQUIRE(d->B >= 1 && d->W_cap >= 1, HCA_E_SHAPE, "B and W_cap must be >= 1");
    REQUIRE(d->kv_pitch >= (int64_t)eb * d->D && d->win_pitch >= (int64_t)eb * d->D, HCA_E_SHAPE,
            "kv_pitch / win_pitch < D elements");
    REQUIRE(aligned(d->kv_in, 16) && aligned(d->win, 16) && d->kv_pitch % 16 == 0 && d->win_pitch % 16 == 0 &&
            aligned(d->gamma_kv, 16) && aligned(d->tok_seq, 4) && aligned(d->tok_pos, 8), HCA_E_ALIGN,
            "token rows must be 16-byte aligned");
    if (d->idx_in) {
      REQUIRE(d->win_idx, HCA_E_NULL, "idx_in needs win_idx");
      REQUIRE(d->d_I >= per && d->d_I % per == 0 && d->d_I <= hca::prologue_max_dim(f32), HCA_E_SHAPE,
              "d_I=%d must be a multiple of %d", d->d_I, per);
      REQUIRE(d->idx_pitch >= (int64_t)eb * d->d_I && d->win_idx_pitch >= (int64_t)eb * d->d_I, HCA_E_SHAPE,
              "idx_pitch / win_idx_pitch < d_I elements");
      REQUIRE(aligned(d->idx_in, 16) && aligned(d->win_idx, 16) && d->idx_pitch % 16 == 0 &&
              d->win_idx_pitch % 16 == 0, HCA_E_ALIGN, "index-stream rows must be 16-byte aligned");
    }
  }
  return HCA_OK;
}

// validate an attention call and fill its launch arguments (a.Nq = 0: nothing to launch)
int build_attn(const hca_attn_desc* d, int prefill, const hca_profile_events* ev, hca::AttnArgs& a) {
  size_t ws = 0;
  int rc = validate_attn(d, prefill, &ws);
  if (rc) return rc;
  a = hca::AttnArgs{};
  if (d->Nq == 0) return HCA_OK;
  const bool swa = d->mode == HCA_MODE_SWA;   // runs as HCA with no visible entry: no cache read
  a.Nq = d->Nq; a.H = d->H; a.D = d->D; a.D_r = d->D_r; a.mode = swa ? HCA_MODE_HCA : d->mode;
  a.m = swa ? 1 : d->m;
  a.k = d->mode == HCA_MODE_CSA ? d->k : 0; a.n_win = d->n_win; a.win_cap = d->win_cap;
  a.io_f32 = d->io_fmt == HCA_F32; a.tau = d->tau; a.rope_base = d->rope_base;
  // RoPE frequencies of the 32 pairs in turns per position, formed once here in fp64
  for (int i = 0; i < 32; ++i) a.inv_turn[i] = std::pow(d->rope_base, -2.0 * i / 64.0) / (2.0 * M_PI);
  a.max_visible = swa ? 0 : d->max_visible; a.q = d->q; a.cache_fmt = d->cache.fmt;
  a.c_f32 = static_cast<const char*>(d->cache.f32); a.c_f32_pitch = d->cache.f32_pitch;
  a.c_nope = static_cast<const char*>(d->cache.nope); a.c_nope_pitch = d->cache.nope_pitch;
  a.c_rope = static_cast<const char*>(d->cache.rope); a.c_rope_pitch = d->cache.rope_pitch;
  a.c_scale = static_cast<const float*>(d->cache.scale);
  a.cache_row_start = swa ? nullptr : d->cache_row_start; a.idx = d->mode == HCA_MODE_CSA ? d->idx : nullptr;
  a.page_table = swa ? nullptr : d->page_table; a.page_pitch = d->page_table_pitch;
  a.page_shift = a.page_table ? log2_exact(d->page_rows) : -1;
  a.win = static_cast<const char*>(d->win); a.win_pitch = d->win_pitch;
  a.sink = d->sink; a.seq_id = d->seq_id; a.q_pos = d->q_pos; a.o = d->o; a.lse = d->lse;
  a.workspace = d->workspace; a.prefill = prefill;
  a.split_chunks = prefill || a.io_f32 ? 0 : d->split_chunks;
  a.split_runs = (int)hca::attention_split_runs(a.mode, a.k, a.n_win, a.max_visible, a.split_chunks);
  if (ev) { a.prof_begin = static_cast<hipEvent_t>(ev->begin); a.prof_end = static_cast<hipEvent_t>(ev->end); }
  return HCA_OK;
}

int attn_call(const hca_attn_desc* d, void* stream, int prefill, const hca_profile_events* ev = nullptr) {
  hca::AttnArgs a;
  const int rc = build_attn(d, prefill, ev, a);
  if (rc || a.Nq == 0) return rc;
  return launched(hca::launch_attention(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int hca_abi_version(void) { return HCA_ABI_VERSION; }

const char* hca_last_error(void) { return g_err.c_str(); }

size_t hca_struct_size(int which) {
  switch (which) {
    case HCA_OP_KV_COMPRESS: return sizeof(hca_kv_compress_desc);
    case HCA_OP_INDEXER_TOPK: return sizeof(hca_indexer_topk_desc);
    case HCA_OP_ATTN_DECODE:
    case HCA_OP_ATTN_PREFILL: return sizeof(hca_attn_desc);
    case HCA_OP_QKV_PROLOGUE: return sizeof(hca_qkv_prologue_desc);
    case HCA_OP_OUT_PROJ: return sizeof(hca_out_proj_desc);
    case HCA_OP_DECODE_LAYER: return sizeof(hca_decode_layer_desc);
    case HCA_STRUCT_KV_PLANES: return sizeof(hca_kv_planes);
    case HCA_STRUCT_IDX_PLANES: return sizeof(hca_idx_planes);
    case HCA_STRUCT_PROFILE_EVENTS: return sizeof(hca_profile_events);
    default: return 0;
  }
}

int hca_indexer_query_group(const hca_indexer_topk_desc* d, int32_t* group) {
  REQUIRE(group, HCA_E_NULL, "group is NULL");
  *group = 0;
  REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
  REQUIRE(d->struct_size == sizeof(hca_indexer_topk_desc), HCA_E_VERSION, "struct_size mismatch");
  REQUIRE(d->Nq >= 0 && d->max_visible >= 0, HCA_E_SHAPE, "Nq and max_visible must be >= 0");
  *group = hca::indexer_group(d->Nq, d->max_visible, d->q.fmt, d->k);
  return HCA_OK;
}

int hca_workspace_bytes(int op, const void* desc, size_t* bytes) {
  REQUIRE(bytes, HCA_E_NULL, "bytes is NULL");
  *bytes = 0;
  size_t ws = 0;
  int rc;
  switch (op) {
    case HCA_OP_KV_COMPRESS: rc = validate_kv_compress(static_cast<const hca_kv_compress_desc*>(desc)); break;
    case HCA_OP_INDEXER_TOPK: {
      // the size depends only on shapes: validate those, not the buffers
      const hca_indexer_topk_desc* d = static_cast<const hca_indexer_topk_desc*>(desc);
      REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
      REQUIRE(d->struct_size == sizeof(hca_indexer_topk_desc), HCA_E_VERSION, "struct_size mismatch");
      REQUIRE(d->Nq >= 0 && d->max_visible >= 0, HCA_E_SHAPE, "Nq and max_visible must be >= 0");
      ws = hca::indexer_workspace_bytes(d->Nq, d->max_visible, d->q.fmt, d->k);
      rc = HCA_OK;
      break;
    }
    case HCA_OP_ATTN_DECODE:
    case HCA_OP_ATTN_PREFILL: {
      const hca_attn_desc* d = static_cast<const hca_attn_desc*>(desc);
      REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
      REQUIRE(d->struct_size == sizeof(hca_attn_desc), HCA_E_VERSION, "struct_size mismatch");
      REQUIRE(d->Nq >= 0 && d->H >= 1 && d->D >= 1 && (d->max_visible >= 0 || d->mode == HCA_MODE_SWA),
              HCA_E_SHAPE, "bad shapes");
      const bool swa = d->mode == HCA_MODE_SWA;
      ws = hca::attention_workspace_bytes(d->Nq, d->H, d->D, swa ? HCA_MODE_HCA : d->mode,
                                          d->mode == HCA_MODE_CSA ? d->k : 0, d->n_win, swa ? 0 : d->max_visible,
                                          d->io_fmt == HCA_F32, op == HCA_OP_ATTN_PREFILL, d->split_chunks);
      rc = HCA_OK;
      break;
    }
    case HCA_OP_QKV_PROLOGUE:
      rc = validate_prologue(static_cast<const hca_qkv_prologue_desc*>(desc));
      ws = 0;
      break;
    case HCA_OP_OUT_PROJ:
      rc = validate_out_proj(static_cast<const hca_out_proj_desc*>(desc));
      ws = 0;
      break;
    case HCA_OP_DECODE_LAYER: {           // the indexer and attention keep their own workspaces
      const hca_decode_layer_desc* d = static_cast<const hca_decode_layer_desc*>(desc);
      REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
      REQUIRE(d->struct_size == sizeof(hca_decode_layer_desc), HCA_E_VERSION, "struct_size mismatch");
      rc = HCA_OK;
      ws = 0;
      break;
    }
    default: return fail(HCA_E_SHAPE, "unknown op %d", op);
  }
  if (rc) return rc;
  *bytes = ws;
  return HCA_OK;
}

namespace {
// validate a pooling call and fill its launch arguments (a.n_blocks = 0: nothing to launch)
int build_pool(const hca_kv_compress_desc* d, hca::PoolArgs& a) {
  int rc = validate_kv_compress(d);
  if (rc) return rc;
  a = hca::PoolArgs{};
  if (d->n_blocks == 0) return HCA_OK;
  a.m = d->m; a.D = d->D; a.D_r = d->D_r; a.d_I = d->raw_idx ? d->d_I : 0; a.n_blocks = d->n_blocks;
  a.rope_base = d->rope_base; a.raw_is_f32 = d->raw_fmt == HCA_F32;
  if (d->D_r / 2 <= 64)
    for (int i = 0; i < d->D_r / 2; ++i) a.rope_inv[i] = std::pow(d->rope_base, -2.0 * i / (double)d->D_r);
  a.raw = d->raw; a.raw_pitch = d->raw_pitch; a.raw_idx = d->raw_idx; a.raw_idx_pitch = d->raw_idx_pitch;
  a.block_row = d->block_row; a.block_pos = d->block_pos; a.out_row = d->out_row;
  a.gate_w = d->gate_w; a.gate_b = d->gate_b;
  a.kv_fmt = d->out.fmt;
  a.out_f32 = static_cast<char*>(d->out.f32); a.out_f32_pitch = d->out.f32_pitch;
  a.out_nope = static_cast<char*>(d->out.nope); a.nope_pitch = d->out.nope_pitch;
  a.out_rope = static_cast<char*>(d->out.rope); a.rope_pitch = d->out.rope_pitch;
  a.out_scale = static_cast<float*>(d->out.scale);
  a.idx_fmt = d->raw_idx ? d->out_idx.fmt : -1;
  a.out_idx = static_cast<char*>(d->out_idx.data); a.idx_pitch = d->out_idx.pitch;
  a.out_idx_scales = static_cast<char*>(d->out_idx.scales); a.idx_scale_pitch = d->out_idx.scale_pitch;
  a.debug = d->debug;
  return HCA_OK;
}
}  // namespace

int hca_kv_compress(const hca_kv_compress_desc* d, void* stream) {
  hca::PoolArgs a;
  const int rc = build_pool(d, a);
  if (rc || a.n_blocks == 0) return rc;
  return launched(hca::launch_pool(a, static_cast<hipStream_t>(stream)));
}

namespace {
// validate an indexer call and fill its launch arguments (a.Nq = 0: nothing to launch)
int build_indexer(const hca_indexer_topk_desc* d, const hca_profile_events* ev, hca::IndexerArgs& a) {
  size_t ws = 0;
  int rc = validate_indexer(d, &ws);
  if (rc) return rc;
  a = hca::IndexerArgs{};
  if (d->Nq == 0) return HCA_OK;
  a.Nq = d->Nq; a.H_I = d->H_I; a.d_I = d->d_I; a.k = d->k; a.m = d->m; a.fmt = d->q.fmt;
  a.max_visible = d->max_visible;
  a.score_pitch = (d->max_visible + 63) / 64 * 64;
  a.q = static_cast<const char*>(d->q.data); a.q_pitch = d->q.pitch;
  a.q_scales = static_cast<const uint8_t*>(d->q.scales); a.q_scale_pitch = d->q.scale_pitch;
  a.w = d->w;
  a.keys = static_cast<const char*>(d->keys.data); a.key_pitch = d->keys.pitch;
  a.key_scales = static_cast<const uint8_t*>(d->keys.scales); a.key_scale_pitch = d->keys.scale_pitch;
  a.cache_row_start = d->cache_row_start; a.seq_id = d->seq_id; a.q_pos = d->q_pos;
  a.page_table = d->page_table; a.page_pitch = d->page_table_pitch;
  a.page_shift = d->page_table ? log2_exact(d->page_rows) : -1;
  a.idx = d->idx; a.score_out = d->score;
  a.scores = d->workspace;             // the workspace layout is laid out by the launcher
  a.hist = nullptr;
  if (ev) { a.prof_begin = static_cast<hipEvent_t>(ev->begin); a.prof_end = static_cast<hipEvent_t>(ev->end); }
  return HCA_OK;
}

int indexer_call(const hca_indexer_topk_desc* d, void* stream, const hca_profile_events* ev) {
  hca::IndexerArgs a;
  const int rc = build_indexer(d, ev, a);
  if (rc || a.Nq == 0) return rc;
  return launched(hca::launch_indexer_topk(a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- decode layer step
int decode_layer_call(const hca_decode_layer_desc* d, void* stream, const hca_profile_events* ev) {
  REQUIRE(d, HCA_E_NULL, "descriptor is NULL");
  REQUIRE(d->struct_size == sizeof(hca_decode_layer_desc), HCA_E_VERSION,
          "struct_size %u != %zu", d->struct_size, sizeof(hca_decode_layer_desc));
  REQUIRE(d->attn, HCA_E_NULL, "attn is NULL");
  const bool csa = d->attn->mode == HCA_MODE_CSA;
  REQUIRE(csa == (d->indexer != nullptr), HCA_E_SHAPE, "indexer is required for a CSA layer and only there");
  hca::PoolArgs pa{};
  if (d->pool) {
    const int rc = build_pool(d->pool, pa);
    if (rc) return rc;
    REQUIRE(pa.n_blocks == 0 || d->pool->m == d->attn->m, HCA_E_SHAPE, "pool m %d != attn m %d",
            d->pool->m, d->attn->m);
  }
  hca::IndexerArgs ia{};
  if (csa) {
    const int rc = build_indexer(d->indexer, ev, ia);
    if (rc) return rc;
    REQUIRE(d->indexer->m == d->attn->m && d->indexer->Nq == d->attn->Nq && d->indexer->k == d->attn->k &&
            d->indexer->idx == d->attn->idx, HCA_E_SHAPE, "indexer and attn disagree on m, Nq, k or idx");
  }
  hca::AttnArgs aa;
  {
    const int rc = build_attn(d->attn, 0, csa ? nullptr : ev, aa);
    if (rc) return rc;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hca::PoolArgs* pool = pa.n_blocks > 0 ? &pa : nullptr;
  hipError_t e = hipSuccess;
  if (csa) {
    e = hca::launch_indexer_topk(ia, s, pool);           // pools inside the scoring launch where it can
    if (e == hipSuccess && aa.Nq > 0) e = hca::launch_attention(aa, s);
  } else {
    e = hca::launch_attention(aa, s, pool);              // pools inside the attention launch where it can
  }
  return launched(e);
}
}  // namespace

int hca_indexer_topk(const hca_indexer_topk_desc* d, void* stream) { return indexer_call(d, stream, nullptr); }

int hca_profiled(int op, const void* desc, const hca_profile_events* ev, void* stream) {
  REQUIRE(ev, HCA_E_NULL, "events is NULL");
  REQUIRE(ev->struct_size == sizeof(hca_profile_events), HCA_E_VERSION, "events struct_size %u != %zu",
          ev->struct_size, sizeof(hca_profile_events));
  switch (op) {
    case HCA_OP_INDEXER_TOPK: return indexer_call(static_cast<const hca_indexer_topk_desc*>(desc), stream, ev);
    case HCA_OP_ATTN_DECODE: return attn_call(static_cast<const hca_attn_desc*>(desc), stream, 0, ev);
    case HCA_OP_ATTN_PREFILL: return attn_call(static_cast<const hca_attn_desc*>(desc), stream, 1, ev);
    case HCA_OP_DECODE_LAYER: return decode_layer_call(static_cast<const hca_decode_layer_desc*>(desc), stream, ev);
    default: return fail(HCA_E_UNSUPPORTED, "op %d has no profiled form", op);
  }
}

int hca_attn_decode(const hca_attn_desc* d, void* stream) { return attn_call(d, stream, 0); }

int hca_decode_layer(const hca_decode_layer_desc* d, void* stream) { return decode_layer_call(d, stream, nullptr); }

int hca_attn_prefill(const hca_attn_desc* d, void* stream) { return attn_call(d, stream, 1); }

int hca_attn_decode_noalloc(const hca_attn_desc* d, void* stream) {
  size_t ws = 0;
  int rc = validate_attn(d, 0, &ws, true);
  if (rc) return rc;
  if (d->Nq == 0) return HCA_OK;
  const size_t cap = hca::attention_static_scratch_bytes();
  REQUIRE(ws <= cap, HCA_E_WORKSPACE,
          "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu (use hca_attn_decode "
          "with a workspace)", ws, cap);
  hca_attn_desc c = *d;
  c.workspace = nullptr;
  c.workspace_bytes = 0;
  if (ws) {
    hipError_t e = hca::attention_static_scratch(&c.workspace);
    if (e != hipSuccess) return fail(HCA_E_LAUNCH, "static scratch lookup failed: %s", hipGetErrorString(e));
    c.workspace_bytes = cap;
  }
  return attn_call(&c, stream, 0);
}

int hca_out_proj(const hca_out_proj_desc* d, void* stream) {
  int rc = validate_out_proj(d);
  if (rc) return rc;
  hca::GprojArgs a{};
  a.M = d->Nq; a.G = d->G; a.d_g = d->d_g; a.out_f32 = d->out_fmt == HCA_F32;
  a.K_g = (int64_t)(d->H / d->G) * d->D;
  a.o = static_cast<const char*>(d->o); a.o_pitch = d->o_pitch;
  a.w = static_cast<const char*>(d->w); a.w_pitch = d->w_pitch;
  a.y = static_cast<char*>(d->y); a.y_pitch = d->y_pitch;
  return launched(hca::launch_gproj(a, static_cast<hipStream_t>(stream)));
}

int hca_qkv_prologue(const hca_qkv_prologue_desc* d, void* stream) {
  int rc = validate_prologue(d);
  if (rc) return rc;
  hca::PrologueArgs a{};
  a.Nq = d->Nq; a.H = d->Nq > 0 ? d->H : 0; a.D = d->D; a.Nt = d->Nt; a.W_cap = d->W_cap; a.B = d->B;
  a.d_I = d->d_I; a.f32 = d->io_fmt == HCA_F32; a.eps = d->eps;
  a.q_in = static_cast<const char*>(d->q_in); a.q_out = static_cast<char*>(d->q_out); a.gamma_q = d->gamma_q;
  a.kv_in = static_cast<const char*>(d->kv_in); a.kv_pitch = d->kv_pitch; a.gamma_kv = d->gamma_kv;
  a.tok_seq = d->tok_seq; a.tok_pos = d->tok_pos;
  a.win = static_cast<char*>(d->win); a.win_pitch = d->win_pitch;
  a.idx_in = d->Nt > 0 ? static_cast<const char*>(d->idx_in) : nullptr; a.idx_pitch = d->idx_pitch;
  a.win_idx = static_cast<char*>(d->win_idx); a.win_idx_pitch = d->win_idx_pitch;
  return launched(hca::launch_prologue(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
