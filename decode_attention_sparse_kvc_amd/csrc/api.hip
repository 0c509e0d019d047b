// C ABI: host-side validation and dispatch.  Nothing here allocates, frees or
// synchronizes; on a validation error nothing is enqueued.

#include <limits.h>
#include <math.h>

#include "internal.h"

using namespace kvc;

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

kvc_status check_cache(const kvc_cache* c) {
  if (!c) return KVC_ERR_INVALID;
  if (c->abi_version != KVC_ABI_VERSION) return KVC_ERR_INVALID;
  if (c->format < KVC_FMT_FP16 || c->format > KVC_FMT_FP8) return KVC_ERR_UNSUPPORTED;
  if (c->head_dim != KVC_HEAD_DIM || c->group_size != KVC_GROUP) return KVC_ERR_UNSUPPORTED;
  if (c->batch < 1 || c->num_kv_heads < 1) return KVC_ERR_SHAPE;
  if (c->max_tokens < KVC_GROUP || c->max_tokens % KVC_GROUP) return KVC_ERR_SHAPE;
  if (!c->seq_lens) return KVC_ERR_INVALID;
  if (c->page_size < 0) return KVC_ERR_SHAPE;
  if (c->page_size > 0) {
    const int unit = c->format == KVC_FMT_INT1 ? KVC_GROUP : 16;
    if (c->page_size % unit || c->max_tokens % c->page_size) return KVC_ERR_SHAPE;
    if ((int64_t)c->max_pages * c->page_size < c->max_tokens) return KVC_ERR_SHAPE;
    if (!c->block_table || c->num_pages < 1) return KVC_ERR_INVALID;
    if (c->kT) return KVC_ERR_UNSUPPORTED;   // channel-major copy needs a contiguous cache
  }
  if (c->format == KVC_FMT_FP16) {
    if (!c->k16 || !c->v16) return KVC_ERR_INVALID;
  } else if (c->format == KVC_FMT_FP8) {
    if (!c->k_codes || !c->v_codes || !aligned(c->k_codes, 16) || !aligned(c->v_codes, 16))
      return KVC_ERR_INVALID;
  } else {
    if (!c->k_codes || !c->v_codes || !c->k_meta || !c->v_meta || !c->k_tail || !c->v_tail)
      return KVC_ERR_INVALID;
    if (!aligned(c->k_codes, 16) || !aligned(c->v_codes, 16) || !aligned(c->k_meta, 8) ||
        !aligned(c->v_meta, 8) || !aligned(c->k_tail, 16) || !aligned(c->v_tail, 16))
      return KVC_ERR_INVALID;
  }
  if ((c->k16 && !aligned(c->k16, 16)) || (c->v16 && !aligned(c->v16, 16)) ||
      (c->kT && !aligned(c->kT, 16)) || (c->k_absmax && !aligned(c->k_absmax, 16)))
    return KVC_ERR_INVALID;
  if ((c->k16 == nullptr) != (c->v16 == nullptr)) return KVC_ERR_INVALID;
  if (c->n_outlier < 0 || c->n_outlier > KVC_MAX_OUTLIERS) return KVC_ERR_INVALID;
  if (c->n_outlier > 0) {
    if (c->format != KVC_FMT_INT4) return KVC_ERR_UNSUPPORTED;
    if (!c->outlier_ch || !c->k_outlier || !aligned(c->outlier_ch, 16) || !aligned(c->k_outlier, 8) ||
        (c->v_outlier && !aligned(c->v_outlier, 8)))
      return KVC_ERR_INVALID;
  }
  return KVC_OK;
}

inline kvc_status hip_status(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_ERR_HIP; }

// Shared by kvc_attend_decode, kvc_accum_scores and the workspace query.
kvc_status check_attend_args(const kvc_cache* c, int32_t hq, int32_t mode, const int32_t* sel,
                             int32_t k_max, int32_t n_sink, int32_t n_window, int32_t workgroups,
                             bool sizing_only = false) {
  if (workgroups < 0 || workgroups > KVC_MAX_WORKGROUPS) return KVC_ERR_INVALID;
  if (hq < 1 || hq % c->num_kv_heads) return KVC_ERR_SHAPE;
  const int G = hq / c->num_kv_heads;
  if (G > KVC_MAX_GQA) return KVC_ERR_UNSUPPORTED;
  if (mode < KVC_ATTEND_DENSE || mode > KVC_ATTEND_BLOCKS) return KVC_ERR_INVALID;
  if (mode != KVC_ATTEND_DENSE) {
    if (k_max < 0 || n_sink < 0 || n_window < 0) return KVC_ERR_INVALID;
    // positions of the fp16-rows role; its plan (8 bytes each) is addressed with 32-bit offsets
    const int64_t nsel = mode == KVC_ATTEND_BLOCKS ? (int64_t)KVC_GROUP * k_max : k_max;
    if ((int64_t)n_sink + nsel + n_window + KVC_GROUP > ((int64_t)1 << 28)) return KVC_ERR_SHAPE;
    if (k_max > 0 && !sel && !sizing_only) return KVC_ERR_INVALID;
    if (sel && !aligned(sel, 4)) return KVC_ERR_INVALID;
  }
  if (mode == KVC_ATTEND_KEEP && (!grouped(c->format) || !c->k16)) return KVC_ERR_UNSUPPORTED;
  if (!attend_plan_ok(*c, mode, k_max, n_sink, n_window, workgroups)) return KVC_ERR_UNSUPPORTED;
  return KVC_OK;
}

// Logits row length an attend call writes (its stride must be at least this).
int64_t logits_positions(const kvc_cache* c, int32_t mode, int32_t k_max, int32_t n_sink,
                         int32_t n_window) {
  return mode == KVC_ATTEND_DROP ? (int64_t)n_sink + k_max + n_window
         : mode == KVC_ATTEND_BLOCKS ? (int64_t)n_sink + (int64_t)KVC_GROUP * k_max + n_window
                                     : (int64_t)c->max_tokens;
}

// Everything both attend entry points validate; *ws receives the workspace
// bytes the call needs.
kvc_status check_attend_call(const kvc_cache* cache, const uint16_t* q, int32_t num_q_heads,
                             float sm_scale, int32_t mode, const int32_t* sel, int32_t k_max,
                             int32_t n_sink, int32_t n_window, float* out, float* lse,
                             float* logits, int64_t logits_stride, int32_t workgroups, size_t* ws) {
  kvc_status st = check_cache(cache);
  if (st != KVC_OK) return st;
  st = check_attend_args(cache, num_q_heads, mode, sel, k_max, n_sink, n_window, workgroups);
  if (st != KVC_OK) return st;
  if (!q || !aligned(q, 16) || !out || !lse) return KVC_ERR_INVALID;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return KVC_ERR_INVALID;
  if (logits && logits_stride < logits_positions(cache, mode, k_max, n_sink, n_window))
    return KVC_ERR_SHAPE;
  *ws = attend_workspace_bytes(*cache, num_q_heads, mode, k_max, n_sink, n_window, workgroups);
  return KVC_OK;
}

}  // namespace

extern "C" {

int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

#ifndef KVC_BUILD_DIGEST
#define KVC_BUILD_DIGEST "unknown"
#endif
const char* kvc_build_digest(void) { return KVC_BUILD_DIGEST; }

const char* kvc_status_str(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID: return "invalid argument (null pointer, range or alignment)";
    case KVC_ERR_SHAPE: return "inconsistent shapes";
    case KVC_ERR_UNSUPPORTED: return "unsupported format, mode or size";
    case KVC_ERR_WORKSPACE: return "workspace missing or too small";
    case KVC_ERR_HIP: return "HIP kernel launch failed";
    case KVC_ERR_SCRATCH:
      return "the call needs more than the static scratch of kvc_attend_decode_noalloc "
             "(KVC_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

kvc_status kvc_quantize_append(const kvc_cache* cache, const uint16_t* k_new,
                               const uint16_t* v_new, const int32_t* n_new,
                               int32_t n_new_max, int32_t* overflow, hipStream_t stream) {
  kvc_status st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (n_new_max < 0 || n_new_max > cache->max_tokens) return KVC_ERR_SHAPE;
  if (n_new_max == 0) return KVC_OK;
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return KVC_ERR_INVALID;
  if (n_new && !aligned(n_new, 4)) return KVC_ERR_INVALID;
  return hip_status(launch_append(*cache, k_new, v_new, n_new, n_new_max, overflow, stream));
}

kvc_status kvc_score_topk(const kvc_cache* cache, const uint16_t* q, int32_t num_q_heads,
                          int32_t score_mode, int32_t n_crit, const float* ext,
                          int32_t n_sink, int32_t n_window, const int32_t* k_per_seq,
                          int32_t k_max, int32_t* out_idx, double* out_scores,
                          int32_t* out_channels, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  kvc_status st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads) return KVC_ERR_SHAPE;
  if (num_q_heads / cache->num_kv_heads > 16) return KVC_ERR_UNSUPPORTED;
  if (cache->max_tokens > KVC_TOPK_MAX_ITEMS) return KVC_ERR_UNSUPPORTED;
  const int32_t base_mode = score_mode & ~KVC_SCORE_BLOCKS;
  if (base_mode < KVC_SCORE_EXACT || base_mode > KVC_SCORE_EXTERNAL) return KVC_ERR_INVALID;
  if (n_sink < 0 || n_window < 0 || k_max < 0) return KVC_ERR_INVALID;
  if (!out_idx || !aligned(out_idx, 4)) return KVC_ERR_INVALID;
  if (k_per_seq && !aligned(k_per_seq, 4)) return KVC_ERR_INVALID;
  if (out_scores && !aligned(out_scores, 8)) return KVC_ERR_INVALID;
  if (base_mode == KVC_SCORE_EXTERNAL) {
    if (!ext || !aligned(ext, 4)) return KVC_ERR_INVALID;
  } else {
    if (!q || !aligned(q, 2)) return KVC_ERR_INVALID;
  }
  if (base_mode == KVC_SCORE_CRITICAL) {
    if (n_crit < 1 || n_crit > KVC_HEAD_DIM) return KVC_ERR_INVALID;
    if (!cache->k_absmax) return KVC_ERR_INVALID;
    if (out_channels && !aligned(out_channels, 4)) return KVC_ERR_INVALID;
  } else {
    out_channels = nullptr;
  }
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < topk_workspace_bytes(*cache))
    return KVC_ERR_WORKSPACE;
  if (k_max == 0) return KVC_OK;
  return hip_status(launch_score_topk(*cache, q, num_q_heads, score_mode, n_crit, ext, n_sink,
                                      n_window, k_per_seq, k_max, out_idx, out_scores,
                                      out_channels, workspace, stream));
}

kvc_status kvc_attend_decode(const kvc_cache* cache, const uint16_t* q, int32_t num_q_heads,
                             float sm_scale, int32_t mode, const int32_t* sel, int32_t k_max,
                             int32_t n_sink, int32_t n_window, float* out, float* lse,
                             float* logits, int64_t logits_stride, int32_t workgroups,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  size_t ws = 0;
  const kvc_status st = check_attend_call(cache, q, num_q_heads, sm_scale, mode, sel, k_max,
                                          n_sink, n_window, out, lse, logits, logits_stride,
                                          workgroups, &ws);
  if (st != KVC_OK) return st;
  if (!workspace || workspace_bytes < ws || !aligned(workspace, 16)) return KVC_ERR_WORKSPACE;
  return hip_status(launch_attend(*cache, q, num_q_heads, sm_scale, mode, sel, k_max, n_sink,
                                  n_window, out, lse, logits, logits_stride, workgroups, workspace,
                                  stream));
}

kvc_status kvc_attend_decode_noalloc(const kvc_cache* cache, const uint16_t* q,
                                     int32_t num_q_heads, float sm_scale, int32_t mode,
                                     const int32_t* sel, int32_t k_max, int32_t n_sink,
                                     int32_t n_window, float* out, float* lse, float* logits,
                                     int64_t logits_stride, hipStream_t stream) {
  size_t ws = 0;
  const kvc_status st = check_attend_call(cache, q, num_q_heads, sm_scale, mode, sel, k_max,
                                          n_sink, n_window, out, lse, logits, logits_stride, 0, &ws);
  if (st != KVC_OK) return st;
  // the size check comes before any HIP call: an oversized request is
  // rejected without touching the device
  if (ws > (size_t)KVC_NOALLOC_SCRATCH_BYTES) return KVC_ERR_SCRATCH;
  void* scratch = nullptr;
  if (noalloc_scratch(&scratch) != hipSuccess) return KVC_ERR_HIP;
  return hip_status(launch_attend(*cache, q, num_q_heads, sm_scale, mode, sel, k_max, n_sink,
                                  n_window, out, lse, logits, logits_stride, 0, scratch, stream));
}

kvc_status kvc_accum_scores(const kvc_cache* cache, int32_t num_q_heads, const float* logits,
                            int64_t logits_stride, const float* lse, int32_t mode,
                            const int32_t* sel, int32_t k_max, int32_t n_sink, int32_t n_window,
                            float* acc, hipStream_t stream) {
  kvc_status st = check_cache(cache);
  if (st != KVC_OK) return st;
  st = check_attend_args(cache, num_q_heads, mode, sel, k_max, n_sink, n_window, 0);
  if (st != KVC_OK && !(st == KVC_ERR_UNSUPPORTED && mode == KVC_ATTEND_KEEP)) return st;
  if (!logits || !lse || !acc || !aligned(logits, 4) || !aligned(lse, 4) || !aligned(acc, 4))
    return KVC_ERR_INVALID;
  if (logits_stride < logits_positions(cache, mode, k_max, n_sink, n_window)) return KVC_ERR_SHAPE;
  return hip_status(launch_accum(*cache, num_q_heads, logits, logits_stride, lse, mode, sel, k_max,
                                 n_sink, n_window, acc, stream));
}

kvc_status kvc_topk_mass(const kvc_cache* cache, int32_t num_q_heads, const float* logits,
                         int64_t logits_stride, const float* lse, int32_t k, float* out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  kvc_status st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads) return KVC_ERR_SHAPE;
  if (!logits || !lse || !out || !aligned(logits, 4) || !aligned(lse, 4) || !aligned(out, 4))
    return KVC_ERR_INVALID;
  if (k < 0) return KVC_ERR_INVALID;
  if (logits_stride < cache->max_tokens) return KVC_ERR_SHAPE;
  if (!workspace || !aligned(workspace, 16) ||
      workspace_bytes < topk_mass_workspace_bytes(*cache, num_q_heads))
    return KVC_ERR_WORKSPACE;
  return hip_status(launch_topk_mass(*cache, num_q_heads, logits, logits_stride, lse, k, out,
                                     workspace, stream));
}

kvc_status kvc_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                           hipStream_t stream) {
  if (!src || !sink || !aligned(src, 4096) || !aligned(sink, 4) || bytes % 4096) return KVC_ERR_INVALID;
  if (workgroups < 1 || workgroups > KVC_MAX_WORKGROUPS) return KVC_ERR_INVALID;
  if (bytes == 0) return KVC_OK;
  return hip_status(launch_stream_read(src, bytes, sink, workgroups, stream));
}

size_t kvc_workspace_bytes(int32_t op, const kvc_cache* cache, int32_t num_q_heads, int32_t mode,
                           int32_t k_max, int32_t n_sink, int32_t n_window, int32_t workgroups) {
  if (check_cache(cache) != KVC_OK) return 0;
  if (op == KVC_OP_ATTEND) {
    if (check_attend_args(cache, num_q_heads, mode, nullptr, k_max, n_sink, n_window, workgroups,
                          true) != KVC_OK)
      return 0;
    return attend_workspace_bytes(*cache, num_q_heads, mode, k_max, n_sink, n_window, workgroups);
  }
  if (op == KVC_OP_SCORE_TOPK) return topk_workspace_bytes(*cache);
  if (op == KVC_OP_TOPK_MASS) {
    if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads) return 0;
    return topk_mass_workspace_bytes(*cache, num_q_heads);
  }
  return 0;
}

}  // extern "C"
