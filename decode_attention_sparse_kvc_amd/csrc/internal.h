// Internal helpers shared by the kvc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>

#include "../../include/kvc.h"

namespace kvc {

constexpr int D = KVC_HEAD_DIM;    // channels per head
constexpr int GS = KVC_GROUP;      // quantization group (tokens for K, channels for V)
constexpr int TILE = 16;           // tokens per INT4 code tile / matrix-core tile
constexpr int UNIT_BYTES = 1024;   // bytes per INT4 tile (16 tokens) or INT1 unit (64 tokens)

// Tokens per page: the page size, or the whole capacity when contiguous.
__host__ __device__ inline int page_tokens(const kvc_cache& c) {
  return c.page_size > 0 ? c.page_size : c.max_tokens;
}

// Slot of token t of (sequence b, KV head g): (phys * Hkv + g) * P + t % P.
// Returns -1 when the block table names a page outside the pools, so callers
// skip the token instead of touching memory they do not own.
__device__ inline int64_t slot_of(const kvc_cache& c, int b, int g, int t) {
  if (c.page_size == 0) return ((int64_t)b * c.num_kv_heads + g) * (int64_t)c.max_tokens + t;
  const int P = page_tokens(c);
  const int page = t / P;
  const int off = t - page * P;
  int64_t phys = b;
  if (c.page_size > 0) {
    if (page >= c.max_pages) return -1;
    phys = c.block_table[(int64_t)b * c.max_pages + page];
    if (phys < 0 || phys >= c.num_pages) return -1;
  }
  return (phys * c.num_kv_heads + g) * (int64_t)P + off;
}

// Division by the page length without a divide instruction: for 0 <= t < 2^31
// and P >= 1, t / P == (t * M) >> (32 + l) with l = ceil(log2 P) and
// M = ceil(2^(32 + l) / P) (the rounding error of M stays below one step).
struct PageDiv {
  uint64_t M;
  int sh;   // 32 + l
  int P;
};
inline PageDiv make_page_div(const kvc_cache& c) {
  PageDiv d;
  d.P = page_tokens(c);
  int l = 0;
  while ((1ll << l) < d.P) ++l;
  d.sh = 32 + l;
  d.M = (uint64_t)((((unsigned __int128)1 << d.sh) + (unsigned)d.P - 1) / (unsigned)d.P);
  return d;
}
__device__ inline int page_of(const PageDiv& d, int t) {
  return (int)(((uint64_t)(uint32_t)t * d.M) >> d.sh);
}
// slot_of with the division replaced by a PageDiv of the same cache.
__device__ inline int64_t slot_fast(const kvc_cache& c, const PageDiv& d, int b, int g, int t) {
  if (c.page_size == 0) return ((int64_t)b * c.num_kv_heads + g) * (int64_t)c.max_tokens + t;
  const int page = page_of(d, t);
  const int off = t - page * d.P;
  if (page >= c.max_pages) return -1;
  const int64_t phys = c.block_table[(int64_t)b * c.max_pages + page];
  if (phys < 0 || phys >= c.num_pages) return -1;
  return (phys * c.num_kv_heads + g) * (int64_t)d.P + off;
}

// Bit position of nibble slot j (0..7) in an INT4 code dword.
__host__ __device__ constexpr int nib_pos(int j) { return 16 * (j & 1) + 4 * (j >> 1); }

// Bit position of code k (0..31) in an INT1 code dword.
__host__ __device__ constexpr int bit_pos(int k) {
  const int w = k >> 1, h = k & 1, v = w >> 2, p = 6 + (w & 3);
  return v == 0 ? p + 16 * h
       : v == 1 ? p + 4 + 16 * h
       : v == 2 ? p - 4 + 16 * h
       : (h ? p + 8 : (p + 24) & 31);
}

// INT1 V: code index k inside lane dword for (channel tile ct, token i of the quad).
__host__ __device__ constexpr int v1_code(int ct, int i) {
  return 2 * (4 * ((ct >> 2) * 2 + (i >> 1)) + (ct & 3)) + (i & 1);
}

// Formats stored as 64-token groups of codes with scale/zero metadata and an
// fp16 tail (INT4, INT1), as opposed to per-token rows (fp16, FP8).
__host__ __device__ constexpr bool grouped(int fmt) { return fmt == KVC_FMT_INT4 || fmt == KVC_FMT_INT1; }

// FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals,
// largest finite 448) of the two fp16 values in w (low half first), as two
// bytes in the low 16 bits: the nearest value, ties to the even code,
// saturating at +-448, sign kept.  gfx950's packed conversion rounds to
// nearest even and agrees with that on every fp16 input of magnitude below
// 464 (an in-bounds probe of all 65536 inputs against an integer encoder of
// the definition; test_codes_every_fp16_value checks the codes the append
// kernel writes for every finite input against the oracle); from 464 up it
// returns NaN instead of saturating, so inputs of magnitude >= 448 (0x5F00,
// also inf and NaN) are set to the saturated code here.
typedef short kvc_s2v __attribute__((ext_vector_type(2)));
typedef _Float16 kvc_h2v __attribute__((ext_vector_type(2)));
__device__ inline uint32_t fp8_encode2(uint32_t w) {
  const kvc_s2v r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(kvc_s2v{0, 0},
                                                             __builtin_bit_cast(kvc_h2v, w), 1.0f, false);
  uint32_t c = __builtin_bit_cast(uint32_t, r) & 0xFFFFu;
  if ((w & 0x7FFFu) >= 0x5F00u) c = (c & 0xFF00u) | ((w >> 8) & 0x80u) | 0x7Eu;
  if (((w >> 16) & 0x7FFFu) >= 0x5F00u) c = (c & 0x00FFu) | ((((w >> 24) & 0x80u) | 0x7Eu) << 8);
  return c;
}

// E4M3 code c -> fp16 bits of value / 256, exactly: sign to bit 15 and the
// exponent and mantissa fields shifted into fp16's (bias 15 = 7 + 8, and an
// E4M3 subnormal lands on the matching fp16 subnormal).
__host__ __device__ inline uint32_t fp8_h16_over256(uint32_t c) {
  return ((c & 0x80u) << 8) | ((c & 0x7Fu) << 7);
}

__device__ inline float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ inline uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// ---- launchers (host side, defined next to their kernels) ----
hipError_t launch_append(const kvc_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* n_new, int32_t n_new_max, int32_t* overflow,
                         hipStream_t s);

// workgroups: the attention launch's planned workgroup count (0 = default)
bool attend_plan_ok(const kvc_cache& c, int mode, int k_max, int n_sink, int n_window,
                    int workgroups);
size_t attend_workspace_bytes(const kvc_cache& c, int hq, int mode, int k_max, int n_sink,
                              int n_window, int workgroups);
hipError_t launch_attend(const kvc_cache& c, const uint16_t* q, int hq, float sm_scale, int mode,
                         const int32_t* sel, int k_max, int n_sink, int n_window, float* out,
                         float* lse, float* logits, int64_t logits_stride, int workgroups,
                         void* ws, hipStream_t s);

// Device address of the current device's static scratch (kvc_attend_decode_noalloc);
// looked up with hipGetSymbolAddress on the device's first call, then cached.
hipError_t noalloc_scratch(void** ptr);

size_t topk_workspace_bytes(const kvc_cache& c);
hipError_t launch_score_topk(const kvc_cache& c, const uint16_t* q, int hq, int mode, int n_crit,
                             const float* ext, int n_sink, int n_window, const int32_t* k_per_seq,
                             int k_max, int32_t* out_idx, double* out_scores,
                             int32_t* out_channels, void* ws, hipStream_t s);
hipError_t launch_accum(const kvc_cache& c, int hq, const float* logits, int64_t stride,
                        const float* lse, int mode, const int32_t* sel, int k_max, int n_sink,
                        int n_window, float* acc, hipStream_t s);

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t s);

// Top-k mass: workspace bytes and the three launches.
size_t topk_mass_workspace_bytes(const kvc_cache& c, int hq);
hipError_t launch_topk_mass(const kvc_cache& c, int hq, const float* logits, int64_t stride,
                            const float* lse, int k, float* out, void* workspace, hipStream_t s);

}  // namespace kvc
