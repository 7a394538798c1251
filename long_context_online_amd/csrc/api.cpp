// Host side of the C ABI: argument validation (all before the first HIP call), threshold
// resolution, kernel selection and launch.  See include/blasst.h for the contract.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/blasst.h"
#include "common.hpp"
#include "host.hpp"

namespace blasst {
hipError_t launch_prefill_bf16(const PrefillArgs &a, int D, int BC, bool out_f32, hipStream_t st);
hipError_t launch_prefill_f32(const PrefillArgs &a, int D, hipStream_t st);
hipError_t launch_decode_gqa(const DecodeArgs &a, hipStream_t st);
hipError_t launch_decode_latent(const DecodeArgs &a, hipStream_t st);
hipError_t launch_prefill_bwd(const BwdArgs &a, hipStream_t st);
hipError_t launch_prefill_paged(const PrefillArgs &a, bool out_f32, hipStream_t st);
}  // namespace blasst

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace blasst {

blasst_status fail(blasst_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

blasst_status ok() {
  g_err[0] = '\0';
  return BLASST_OK;
}

}  // namespace blasst

namespace {

using blasst::fail;
using blasst::ok;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ln(lambda) for a fixed threshold or for a / L; returns false when the threshold is invalid.
bool resolve_threshold(const blasst_threshold &t, double L, double *ln_lam, const char **why) {
  if (t.reserved != 0) { *why = "thr.reserved must be 0"; return false; }
  if (t.mode == BLASST_THR_LAMBDA) {
    if (!(t.lambda >= 0.0 && t.lambda <= 1.0)) { *why = "lambda must lie in [0, 1]"; return false; }
    *ln_lam = t.lambda == 0.0 ? -INFINITY : std::log(t.lambda);
    return true;
  }
  if (t.mode == BLASST_THR_NONE) {
    *ln_lam = -INFINITY;
    return true;
  }
  if (t.mode == BLASST_THR_A_OVER_L) {
    if (!(t.a >= 0.0) || !std::isfinite(t.a)) { *why = "a must be finite and >= 0"; return false; }
    if (L <= 0) { *why = "L must be > 0"; return false; }
    const double lam = std::fmin(1.0, t.a / L);
    *ln_lam = lam == 0.0 ? -INFINITY : std::log(lam);
    return true;
  }
  *why = "unknown threshold mode";
  return false;
}

float thr_raw_from(double ln_lam, double scale) {
  if (std::isinf(ln_lam)) return -INFINITY;
  return static_cast<float>(ln_lam / scale);
}

}  // namespace

extern "C" {

const char *blasst_status_string(blasst_status s) {
  switch (s) {
    case BLASST_OK: return "ok";
    case BLASST_ERR_INVALID_ARG: return "invalid argument";
    case BLASST_ERR_UNSUPPORTED: return "unsupported configuration";
    case BLASST_ERR_HIP: return "HIP error";
    case BLASST_ERR_WORKSPACE: return "workspace missing or too small";
  }
  return "unknown status";
}

const char *blasst_last_error(void) { return g_err; }
int32_t blasst_version(void) { return 10000; }
size_t blasst_prefill_params_size(void) { return sizeof(blasst_prefill_params); }
size_t blasst_decode_params_size(void) { return sizeof(blasst_decode_params); }
size_t blasst_prefill_backward_params_size(void) { return sizeof(blasst_prefill_backward_params); }
size_t blasst_prefill_paged_params_size(void) { return sizeof(blasst_prefill_paged_params); }

blasst_status blasst_prefill_paged(const blasst_prefill_paged_params *p, void *stream) {
  if (!p) return fail(BLASST_ERR_INVALID_ARG, "params is NULL");
  if (p->struct_size != sizeof(blasst_prefill_paged_params))
    return fail(BLASST_ERR_INVALID_ARG, "struct_size %zu != %zu", p->struct_size, sizeof(blasst_prefill_paged_params));
  if (!p->q || !p->k_cache || !p->v_cache || !p->block_table || !p->seq_lens)
    return fail(BLASST_ERR_INVALID_ARG, "q, k_cache, v_cache, block_table and seq_lens must be non-NULL");
  if (!p->stats_only && !p->o) return fail(BLASST_ERR_INVALID_ARG, "o must be non-NULL unless stats_only");
  if (p->batch < 1 || p->seqlen_q < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim_qk < 1 ||
      p->head_dim_v < 1)
    return fail(BLASST_ERR_INVALID_ARG, "sizes must be >= 1");
  if (p->num_q_heads % p->num_kv_heads)
    return fail(BLASST_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (p->page_size < 1 || p->max_pages_per_seq < 1 || p->num_pages < 1)
    return fail(BLASST_ERR_INVALID_ARG, "page_size, max_pages_per_seq and num_pages must be >= 1");
  if (p->block_q < 1 || p->block_k < 1) return fail(BLASST_ERR_INVALID_ARG, "block sizes must be >= 1");
  if (p->num_splits < 1) return fail(BLASST_ERR_INVALID_ARG, "num_splits must be >= 1");
  if (p->in_dtype != BLASST_BF16 && p->in_dtype != BLASST_FP32) return fail(BLASST_ERR_INVALID_ARG, "bad in_dtype");
  if (p->out_dtype != BLASST_BF16 && p->out_dtype != BLASST_FP32) return fail(BLASST_ERR_INVALID_ARG, "bad out_dtype");
  if (!std::isfinite(p->softmax_scale)) return fail(BLASST_ERR_INVALID_ARG, "softmax_scale must be finite");
  for (int i = 0; i < 3; ++i)
    if (p->q_stride[i] < 0 || p->o_stride[i] < 0) return fail(BLASST_ERR_INVALID_ARG, "strides must be >= 0");
  double ln_lam;
  const char *why = "";
  if (!resolve_threshold(p->thr, 1.0, &ln_lam, &why)) return fail(BLASST_ERR_INVALID_ARG, "%s", why);
  if (p->thr.mode == BLASST_THR_NONE && (p->skip_mask || p->crit || p->stats_only))
    return fail(BLASST_ERR_INVALID_ARG, "threshold mode NONE takes no skip_mask, crit or stats_only");
  // ---- kernel coverage ----
  if (p->in_dtype != BLASST_BF16) return fail(BLASST_ERR_UNSUPPORTED, "paged prefill supports bf16 inputs");
  if (p->head_dim_qk != 128 || p->head_dim_v != 128 || p->block_q != 128 || p->block_k != 128 || p->page_size != 16)
    return fail(BLASST_ERR_UNSUPPORTED, "paged prefill supports head dim 128, 128 x 128 blocks and 16-token pages");
  const int oelem = p->out_dtype == BLASST_BF16 ? 2 : 4;
  for (int i = 0; i < 3; ++i)
    if (p->q_stride[i] % 8 || p->o_stride[i] % (16 / oelem))
      return fail(BLASST_ERR_UNSUPPORTED, "strides must be multiples of 16 bytes");
  if (!aligned16(p->q) || !aligned16(p->k_cache) || !aligned16(p->v_cache) || (p->o && !aligned16(p->o)))
    return fail(BLASST_ERR_UNSUPPORTED, "q, caches and o must be 16-byte aligned");
  // 32-bit key positions, and the pool's (page, kv head) units counted in 32 bits
  if ((double)p->max_pages_per_seq * p->page_size > 2147483647.0 ||
      (double)p->num_pages * p->num_kv_heads > 4294967295.0)
    return fail(BLASST_ERR_UNSUPPORTED, "problem too large for one launch");
  const double scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0 / std::sqrt((double)p->head_dim_qk);
  blasst::PrefillArgs a{};
  a.q = p->q; a.k = p->k_cache; a.v = p->v_cache; a.o = p->o; a.lse = p->lse;
  a.mask = p->skip_mask; a.crit = p->crit; a.counters = p->counters;
  for (int i = 0; i < 3; ++i) { a.qs[i] = p->q_stride[i]; a.os[i] = p->o_stride[i]; }
  a.B = p->batch; a.Lq = p->seqlen_q; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads;
  a.Lk = p->max_pages_per_seq * p->page_size;
  a.nqt = (p->seqlen_q + 127) / 128;
  a.nkb = (int)(((int64_t)p->max_pages_per_seq * p->page_size + 127) / 128);
  a.causal = 1; a.num_splits = p->num_splits; a.stats_only = p->stats_only ? 1 : 0;
  a.scale = (float)scale;
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  a.decide = 1;
  a.table = p->block_table; a.seq_lens = p->seq_lens; a.max_pages = p->max_pages_per_seq;
  if (p->thr.mode == BLASST_THR_A_OVER_L) {
    a.thr_mode = 1;
    a.a_thr = (float)p->thr.a;
  } else {
    a.thr_mode = 0;
    a.thr_raw = thr_raw_from(p->thr.mode == BLASST_THR_NONE || p->thr.lambda == 0.0 ? -INFINITY
                                                                                      : std::log(p->thr.lambda), scale);
  }
  if ((double)a.B * a.Hq * a.nqt > 2147483647.0 || (double)a.B * a.Hq * a.nqt * a.nkb > 2147483647.0)
    return fail(BLASST_ERR_UNSUPPORTED, "problem too large for one launch");
  hipError_t e = blasst::launch_prefill_paged(a, p->out_dtype == BLASST_FP32, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BLASST_ERR_HIP, "paged prefill launch: %s", hipGetErrorString(e));
  return ok();
}

static blasst_status validate_prefill(const blasst_prefill_params *p, bool need_ptrs) {
  if (!p) return fail(BLASST_ERR_INVALID_ARG, "params is NULL");
  if (p->struct_size != sizeof(blasst_prefill_params))
    return fail(BLASST_ERR_INVALID_ARG, "struct_size %zu != %zu", p->struct_size, sizeof(blasst_prefill_params));
  if (need_ptrs) {
    if (!p->q || !p->k || !p->v) return fail(BLASST_ERR_INVALID_ARG, "q, k and v must be non-NULL");
    if (!p->stats_only && !p->o) return fail(BLASST_ERR_INVALID_ARG, "o must be non-NULL unless stats_only");
  }
  if (p->batch < 1 || p->seqlen_q < 1 || p->seqlen_k < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 ||
      p->head_dim_qk < 1 || p->head_dim_v < 1)
    return fail(BLASST_ERR_INVALID_ARG, "sizes must be >= 1");
  if (p->num_q_heads % p->num_kv_heads)
    return fail(BLASST_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->block_q < 1 || p->block_k < 1) return fail(BLASST_ERR_INVALID_ARG, "block sizes must be >= 1");
  if (p->num_splits < 1) return fail(BLASST_ERR_INVALID_ARG, "num_splits must be >= 1");
  if (p->in_dtype != BLASST_BF16 && p->in_dtype != BLASST_FP32) return fail(BLASST_ERR_INVALID_ARG, "bad in_dtype");
  if (p->out_dtype != BLASST_BF16 && p->out_dtype != BLASST_FP32) return fail(BLASST_ERR_INVALID_ARG, "bad out_dtype");
  if (p->causal != 0 && p->causal != 1) return fail(BLASST_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(p->softmax_scale)) return fail(BLASST_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (p->v_staging != BLASST_V_KEPT && p->v_staging != BLASST_V_ALL)
    return fail(BLASST_ERR_INVALID_ARG, "v_staging must be BLASST_V_KEPT or BLASST_V_ALL");
  for (int i = 0; i < 3; ++i)
    if (p->q_stride[i] < 0 || p->k_stride[i] < 0 || p->v_stride[i] < 0 || p->o_stride[i] < 0)
      return fail(BLASST_ERR_INVALID_ARG, "strides must be >= 0");
  double ln_lam;
  const char *why = "";
  if (!resolve_threshold(p->thr, p->seqlen_k, &ln_lam, &why)) return fail(BLASST_ERR_INVALID_ARG, "%s", why);
  if (p->thr.mode == BLASST_THR_NONE && (p->skip_mask || p->crit || p->stats_only))
    return fail(BLASST_ERR_INVALID_ARG, "threshold mode NONE takes no skip_mask, crit or stats_only");

  // ---- kernel coverage ----
  const int D = p->head_dim_qk;
  if (p->head_dim_v != D) return fail(BLASST_ERR_UNSUPPORTED, "head_dim_v must equal head_dim_qk");
  if (p->block_q != p->block_k) return fail(BLASST_ERR_UNSUPPORTED, "block_q must equal block_k");
  const int elem = p->in_dtype == BLASST_BF16 ? 2 : 4;
  const int vec = 16 / elem;
  if (p->in_dtype == BLASST_BF16) {
    if (!((D == 64 || D == 128) && (p->block_k == 64 || p->block_k == 128)))
      return fail(BLASST_ERR_UNSUPPORTED, "bf16 prefill supports head dim 64/128 and blocks 64/128");
    // K and V rows are addressed with 24-bit byte offsets inside a block
    if (p->k_stride[2] >= (1 << 22) || p->v_stride[2] >= (1 << 22))
      return fail(BLASST_ERR_UNSUPPORTED, "k and v token strides must be below 2^22 elements");
    // a block is staged through one buffer resource that spans its rows back to back, so rows must
    // not overlap (a token stride of 0, an expanded tensor, would read as zeros)
    if (p->k_stride[2] < D || p->v_stride[2] < D)
      return fail(BLASST_ERR_UNSUPPORTED, "bf16 prefill needs k and v token strides >= head_dim");
  } else {
    if (!((D == 64 || D == 128) && p->block_k == 64 && p->out_dtype == BLASST_FP32))
      return fail(BLASST_ERR_UNSUPPORTED, "fp32 prefill supports head dim 64/128, blocks 64, fp32 out");
  }
  if (need_ptrs && (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || (p->o && !aligned16(p->o))))
    return fail(BLASST_ERR_UNSUPPORTED, "q, k, v and o must be 16-byte aligned");
  const int oelem = p->out_dtype == BLASST_BF16 ? 2 : 4;
  for (int i = 0; i < 3; ++i)
    if (p->q_stride[i] % vec || p->k_stride[i] % vec || p->v_stride[i] % vec || p->o_stride[i] % (16 / oelem))
      return fail(BLASST_ERR_UNSUPPORTED, "strides must be multiples of 16 bytes");
  const double nqt = ((int64_t)p->seqlen_q + p->block_q - 1) / p->block_q;
  const double nkb = ((int64_t)p->seqlen_k + p->block_k - 1) / p->block_k;
  if ((double)p->batch * p->num_q_heads * nqt > 2147483647.0 || (double)p->batch * p->num_q_heads * nqt * nkb > 2147483647.0)
    return fail(BLASST_ERR_UNSUPPORTED, "problem too large for one launch");
  return BLASST_OK;
}

size_t blasst_prefill_workspace_size(const blasst_prefill_params *p) {
  if (validate_prefill(p, false) != BLASST_OK) return 0;
  ok();
  return 0;
}

blasst_status blasst_prefill(const blasst_prefill_params *p, void *stream) {
  const blasst_status st = validate_prefill(p, true);
  if (st != BLASST_OK) return st;
  const int D = p->head_dim_qk;
  const double scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0 / std::sqrt((double)p->head_dim_qk);
  double ln_lam;
  const char *why = "";
  resolve_threshold(p->thr, p->seqlen_k, &ln_lam, &why);
  const bool no_decision = p->thr.mode == BLASST_THR_NONE;

  blasst::PrefillArgs a{};
  a.q = p->q; a.k = p->k; a.v = p->v; a.o = p->o; a.lse = p->lse;
  a.mask = p->skip_mask; a.crit = p->crit; a.counters = p->counters; a.head_counters = p->head_counters;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = p->q_stride[i]; a.ks[i] = p->k_stride[i]; a.vs[i] = p->v_stride[i]; a.os[i] = p->o_stride[i];
  }
  a.B = p->batch; a.Lq = p->seqlen_q; a.Lk = p->seqlen_k; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads;
  a.nqt = (p->seqlen_q + p->block_q - 1) / p->block_q;
  a.nkb = (p->seqlen_k + p->block_k - 1) / p->block_k;
  a.causal = p->causal; a.num_splits = p->num_splits; a.stats_only = p->stats_only ? 1 : 0;
  a.scale = (float)scale;
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  a.thr_raw = thr_raw_from(ln_lam, scale);
  a.decide = no_decision ? 0 : 1;
  a.v_all = p->v_staging == BLASST_V_ALL ? 1 : 0;

  hipError_t e;
  if (p->in_dtype == BLASST_BF16)
    e = blasst::launch_prefill_bf16(a, D, p->block_k, p->out_dtype == BLASST_FP32, (hipStream_t)stream);
  else
    e = blasst::launch_prefill_f32(a, D, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BLASST_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

static blasst_status validate_decode(const blasst_decode_params *p, bool need_ptrs, size_t *ws_bytes) {
  if (!p) return fail(BLASST_ERR_INVALID_ARG, "params is NULL");
  if (p->struct_size != sizeof(blasst_decode_params))
    return fail(BLASST_ERR_INVALID_ARG, "struct_size %zu != %zu", p->struct_size, sizeof(blasst_decode_params));
  if (p->num_q_tokens < 0) return fail(BLASST_ERR_INVALID_ARG, "num_q_tokens must be >= 0");
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim_qk < 1 || p->head_dim_v < 1)
    return fail(BLASST_ERR_INVALID_ARG, "sizes must be >= 1");
  if (p->num_q_heads % p->num_kv_heads)
    return fail(BLASST_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (p->page_size < 1 || p->max_pages_per_seq < 1 || p->num_pages < 1)
    return fail(BLASST_ERR_INVALID_ARG, "page_size, max_pages_per_seq and num_pages must be >= 1");
  if (p->block_k < 1 || p->block_k % p->page_size)
    return fail(BLASST_ERR_INVALID_ARG, "block_k must be a positive multiple of page_size");
  if (p->num_splits < 1) return fail(BLASST_ERR_INVALID_ARG, "num_splits must be >= 1");
  const int G = p->num_q_heads / p->num_kv_heads;
  const int tr = p->tile_rows == 0 ? G : p->tile_rows;
  if (tr < 1 || G % tr) return fail(BLASST_ERR_INVALID_ARG, "tile_rows must divide num_q_heads/num_kv_heads");
  if (p->in_dtype != BLASST_BF16 && p->in_dtype != BLASST_FP32) return fail(BLASST_ERR_INVALID_ARG, "bad in_dtype");
  if (p->out_dtype != BLASST_BF16 && p->out_dtype != BLASST_FP32) return fail(BLASST_ERR_INVALID_ARG, "bad out_dtype");
  if (!std::isfinite(p->softmax_scale)) return fail(BLASST_ERR_INVALID_ARG, "softmax_scale must be finite");
  double ln_lam;
  const char *why = "";
  if (!resolve_threshold(p->thr, 1.0, &ln_lam, &why)) return fail(BLASST_ERR_INVALID_ARG, "%s", why);
  if (p->thr.mode == BLASST_THR_NONE && (p->skip_mask || p->crit || p->stats_only))
    return fail(BLASST_ERR_INVALID_ARG, "threshold mode NONE takes no skip_mask, crit or stats_only");
  if (need_ptrs) {
    if (!p->q || !p->k_cache || !p->block_table || !p->seq_lens)
      return fail(BLASST_ERR_INVALID_ARG, "q, k_cache, block_table and seq_lens must be non-NULL");
    if (!p->stats_only && !p->o) return fail(BLASST_ERR_INVALID_ARG, "o must be non-NULL unless stats_only");
  }
  // ---- kernel coverage ----
  if (p->in_dtype != BLASST_BF16) return fail(BLASST_ERR_UNSUPPORTED, "decode supports bf16 inputs");
  if (p->page_size != 16 || p->block_k != 64) return fail(BLASST_ERR_UNSUPPORTED, "decode supports page 16, block 64");
  const bool latent = p->v_cache == nullptr;
  const int T = p->num_q_tokens == 0 ? 1 : p->num_q_tokens;
  if (latent) {
    if (p->num_kv_heads != 1 || p->num_q_heads != 128 || p->head_dim_qk != 576 || p->head_dim_v != 512 ||
        !((int64_t)T * tr == 128 || (int64_t)T * tr == 64))
      return fail(BLASST_ERR_UNSUPPORTED,
                  "latent decode supports 128 q heads on 1 kv head, dims 576/512, and tiles of 128 or 64 rows "
                  "(num_q_tokens * tile_rows == 128 or 64)");
  } else {
    if (p->head_dim_qk != 128 || p->head_dim_v != 128 || (int64_t)T * tr > 16)
      return fail(BLASST_ERR_UNSUPPORTED, "decode supports head dim 128 and num_q_tokens * tile_rows <= 16");
  }
  if (need_ptrs && (!aligned16(p->q) || !aligned16(p->k_cache) || (p->v_cache && !aligned16(p->v_cache)) ||
                    (p->o && !aligned16(p->o))))
    return fail(BLASST_ERR_UNSUPPORTED, "q, caches and o must be 16-byte aligned");
  // the kernels index contexts, workgroups and mask rows with 32-bit integers
  const double nkb = std::ceil((double)p->max_pages_per_seq * p->page_size / p->block_k);
  if ((double)p->max_pages_per_seq * p->page_size > 2147483647.0 ||
      (double)p->batch * T * p->num_q_heads * p->num_splits > 2147483647.0 ||
      (double)p->batch * p->num_q_heads * nkb > 2147483647.0)
    return fail(BLASST_ERR_UNSUPPORTED, "problem too large for one launch");
  const size_t parts = (size_t)p->batch * T * p->num_q_heads * p->num_splits;
  size_t bytes = 0;
  if (p->num_splits > 1) {
    const size_t o_bytes = (parts * p->head_dim_v * sizeof(float) + 255) / 256 * 256;
    bytes = o_bytes + (parts * sizeof(float) + 255) / 256 * 256;
  }
  *ws_bytes = bytes;
  return BLASST_OK;
}

static blasst_status validate_backward(const blasst_prefill_backward_params *p, bool need_ptrs, size_t *ws) {
  if (!p) return fail(BLASST_ERR_INVALID_ARG, "params is NULL");
  if (p->struct_size != sizeof(blasst_prefill_backward_params))
    return fail(BLASST_ERR_INVALID_ARG, "struct_size %zu != %zu", p->struct_size,
                sizeof(blasst_prefill_backward_params));
  if (p->batch < 1 || p->seqlen_q < 1 || p->seqlen_k < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 ||
      p->head_dim_qk < 1 || p->head_dim_v < 1)
    return fail(BLASST_ERR_INVALID_ARG, "sizes must be >= 1");
  if (p->num_q_heads % p->num_kv_heads)
    return fail(BLASST_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (p->block_q < 1 || p->block_k < 1) return fail(BLASST_ERR_INVALID_ARG, "block sizes must be >= 1");
  if (p->in_dtype != BLASST_BF16 && p->in_dtype != BLASST_FP32) return fail(BLASST_ERR_INVALID_ARG, "bad in_dtype");
  if (p->grad_dtype != BLASST_BF16 && p->grad_dtype != BLASST_FP32)
    return fail(BLASST_ERR_INVALID_ARG, "bad grad_dtype");
  if (p->o_dtype != BLASST_BF16 && p->o_dtype != BLASST_FP32) return fail(BLASST_ERR_INVALID_ARG, "bad o_dtype");
  if (p->causal != 0 && p->causal != 1) return fail(BLASST_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(p->softmax_scale)) return fail(BLASST_ERR_INVALID_ARG, "softmax_scale must be finite");
  for (int i = 0; i < 3; ++i)
    if (p->q_stride[i] < 0 || p->k_stride[i] < 0 || p->v_stride[i] < 0 || p->o_stride[i] < 0 ||
        p->dout_stride[i] < 0 || p->dq_stride[i] < 0 || p->dk_stride[i] < 0 || p->dv_stride[i] < 0)
      return fail(BLASST_ERR_INVALID_ARG, "strides must be >= 0");
  if (need_ptrs) {
    if (!p->q || !p->k || !p->v || !p->o || !p->dout || !p->lse || !p->dq || !p->dk || !p->dv)
      return fail(BLASST_ERR_INVALID_ARG, "q, k, v, o, dout, lse, dq, dk and dv must be non-NULL");
  }
  // ---- kernel coverage ----
  if (p->in_dtype != BLASST_BF16) return fail(BLASST_ERR_UNSUPPORTED, "the backward supports bf16 inputs");
  if (p->head_dim_qk != 128 || p->head_dim_v != 128 || p->block_q != 128 || p->block_k != 128)
    return fail(BLASST_ERR_UNSUPPORTED, "the backward supports head dim 128 and 128 x 128 blocks");
  for (int i = 0; i < 3; ++i)
    if (p->q_stride[i] % 8 || p->k_stride[i] % 8 || p->v_stride[i] % 8 || p->o_stride[i] % 4 ||
        p->dout_stride[i] % 8 || p->dq_stride[i] % 8 || p->dk_stride[i] % 8 || p->dv_stride[i] % 8)
      return fail(BLASST_ERR_UNSUPPORTED, "strides must be multiples of 8 elements");
  if (need_ptrs && (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->o) ||
                    !aligned16(p->dout) || !aligned16(p->dq) || !aligned16(p->dk) || !aligned16(p->dv)))
    return fail(BLASST_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  const double nqt = (p->seqlen_q + 127) / 128, nkb = (p->seqlen_k + 127) / 128;
  if ((double)p->batch * p->num_q_heads * nqt * nkb > 2147483647.0 ||
      (double)p->batch * p->num_q_heads * p->seqlen_q > 2147483647.0)
    return fail(BLASST_ERR_UNSUPPORTED, "problem too large for one launch");
  *ws = ((size_t)p->batch * p->num_q_heads * p->seqlen_q * sizeof(float) + 255) / 256 * 256;
  return BLASST_OK;
}

size_t blasst_prefill_backward_workspace_size(const blasst_prefill_backward_params *p) {
  size_t ws = 0;
  if (validate_backward(p, false, &ws) != BLASST_OK) return 0;
  ok();
  return ws;
}

blasst_status blasst_prefill_backward(const blasst_prefill_backward_params *p, void *stream) {
  size_t ws = 0;
  blasst_status st = validate_backward(p, true, &ws);
  if (st != BLASST_OK) return st;
  if (!p->workspace || p->workspace_bytes < ws)
    return fail(BLASST_ERR_WORKSPACE, "workspace of %zu bytes required", ws);
  if (reinterpret_cast<uintptr_t>(p->workspace) & 255u)
    return fail(BLASST_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const double scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0 / std::sqrt((double)p->head_dim_qk);
  blasst::BwdArgs a{};
  a.q = p->q; a.k = p->k; a.v = p->v; a.o = p->o; a.dout = p->dout; a.lse = p->lse; a.mask = p->skip_mask;
  a.dq = p->dq; a.dk = p->dk; a.dv = p->dv; a.dvec = (float *)p->workspace;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = p->q_stride[i]; a.ks[i] = p->k_stride[i]; a.vs[i] = p->v_stride[i]; a.os[i] = p->o_stride[i];
    a.dos[i] = p->dout_stride[i]; a.dqs[i] = p->dq_stride[i]; a.dks[i] = p->dk_stride[i]; a.dvs[i] = p->dv_stride[i];
  }
  a.B = p->batch; a.Lq = p->seqlen_q; a.Lk = p->seqlen_k; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads;
  a.nqt = (p->seqlen_q + 127) / 128;
  a.nkb = (p->seqlen_k + 127) / 128;
  a.causal = p->causal;
  a.out_f32 = p->grad_dtype == BLASST_FP32;
  a.o_f32 = p->o_dtype == BLASST_FP32;
  a.scale = (float)scale;
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  hipError_t e = blasst::launch_prefill_bwd(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BLASST_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return ok();
}

size_t blasst_decode_workspace_size(const blasst_decode_params *p) {
  size_t bytes = 0;
  if (validate_decode(p, false, &bytes) != BLASST_OK) return 0;
  ok();
  return bytes;
}

blasst_status blasst_decode(const blasst_decode_params *p, void *stream) {
  size_t ws = 0;
  blasst_status st = blasst::decode_validate(p, &ws);
  if (st != BLASST_OK) return st;
  if (ws > 0) {
    if (!p->workspace || p->workspace_bytes < ws)
      return fail(BLASST_ERR_WORKSPACE, "workspace of %zu bytes required", ws);
    if (reinterpret_cast<uintptr_t>(p->workspace) & 255u)
      return fail(BLASST_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  return blasst::decode_launch(p, p->workspace, (hipStream_t)stream);
}

}  // extern "C"

namespace blasst {

blasst_status decode_validate(const blasst_decode_params *p, size_t *ws_bytes) {
  const blasst_status st = validate_decode(p, true, ws_bytes);
  if (st == BLASST_OK && p->stats_only) *ws_bytes = 0;   // a stats pass writes no partials
  return st;
}

blasst_status decode_launch(const blasst_decode_params *p, void *workspace, hipStream_t stream) {
  const double scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0 / std::sqrt((double)p->head_dim_qk);
  const int G = p->num_q_heads / p->num_kv_heads;
  const int tr = p->tile_rows == 0 ? G : p->tile_rows;
  DecodeArgs a{};
  a.q = p->q; a.kc = p->k_cache; a.vc = p->v_cache; a.table = p->block_table; a.seq_lens = p->seq_lens;
  a.o = p->o; a.lse = p->lse; a.mask = p->skip_mask; a.crit = p->crit; a.counters = p->counters;
  const int T = p->num_q_tokens == 0 ? 1 : p->num_q_tokens;
  if (p->num_splits > 1 && !p->stats_only) {   // the layout decode_validate sized
    const size_t parts = (size_t)p->batch * T * p->num_q_heads * p->num_splits;
    const size_t o_bytes = (parts * p->head_dim_v * sizeof(float) + 255) / 256 * 256;
    a.ws_o = (float *)workspace;
    a.ws_lse = (float *)((char *)workspace + o_bytes);
  }
  a.B = p->batch; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.G = G; a.tile_rows = tr; a.n_rt = G / tr;
  a.T = T;
  a.page = p->page_size; a.max_pages = p->max_pages_per_seq; a.block_k = p->block_k;
  a.nkb = (int)(((int64_t)p->max_pages_per_seq * p->page_size + p->block_k - 1) / p->block_k);
  a.num_splits = p->num_splits; a.stats_only = p->stats_only ? 1 : 0; a.out_f32 = p->out_dtype == BLASST_FP32;
  a.scale = (float)scale;
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  a.decide = 1;
  if (p->thr.mode == BLASST_THR_A_OVER_L) {
    a.thr_mode = 1;
    a.a = (float)p->thr.a;
  } else {
    // a fixed lambda; NONE keeps every block (lambda = 0) and, for the GQA kernel, runs the variant
    // without any decision logic
    a.thr_mode = 0;
    a.thr_raw = thr_raw_from(p->thr.mode == BLASST_THR_NONE || p->thr.lambda == 0.0 ? -INFINITY
                                                                                    : std::log(p->thr.lambda), scale);
    if (p->thr.mode == BLASST_THR_NONE) a.decide = 0;
  }
  hipError_t e = p->v_cache ? launch_decode_gqa(a, stream) : launch_decode_latent(a, stream);
  if (e == hipErrorNotSupported) return fail(BLASST_ERR_UNSUPPORTED, "no decode kernel for this shape");
  if (e != hipSuccess) return fail(BLASST_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace blasst
