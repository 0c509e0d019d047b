// H2O cumulative attention scores (StreamingLLM / H2O survey, section 3.2):
// after a decode step, every attended token of (sequence b, KV head g) gains
// the attention probabilities exp(logit - lse) of all query heads that read
// that KV head.  Positions follow kvc_attend_decode's logits layout, so one
// thread per position adds one token; every token appears at most once.

#include <math.h>

#include "internal.h"

namespace kvc {
namespace {

constexpr int AT = 256;

__global__ __launch_bounds__(AT) void accum_kernel(kvc_cache c, int hq, const float* __restrict__ logits,
                                                   int64_t stride, const float* __restrict__ lse,
                                                   int mode, const int32_t* __restrict__ sel, int k_max,
                                                   int n_sink, int n_window, float* __restrict__ acc) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int p = blockIdx.x * AT + threadIdx.x;
  const int G = hq / c.num_kv_heads;
  const int n = max(c.seq_lens[b], 0);
  int t;
  bool ok;
  if (mode == KVC_ATTEND_DROP || mode == KVC_ATTEND_BLOCKS) {
    const int w0 = max(n - n_window, min(n_sink, n));
    const int nsel = mode == KVC_ATTEND_BLOCKS ? GS * k_max : k_max;
    if (p < n_sink) {
      t = p;
      ok = p < n;
    } else if (p < n_sink + nsel) {
      const int32_t* s = sel + ((int64_t)b * c.num_kv_heads + g) * k_max;
      if (mode == KVC_ATTEND_BLOCKS) {   // token (p - n_sink) % 64 of kept block (p - n_sink) / 64
        const int blk = s[(p - n_sink) / GS];
        t = blk * GS + (p - n_sink) % GS;
        ok = blk >= (n_sink + GS - 1) / GS && blk < max(n - n_window, 0) / GS;
      } else {
        t = s[p - n_sink];
        ok = t >= n_sink && t < n - n_window;
      }
    } else {
      t = w0 + (p - n_sink - nsel);
      ok = p < n_sink + nsel + n_window && t < n;
    }
  } else {
    t = p;
    ok = p < n;
  }
  if (!ok) return;
  float s = 0.f;
  for (int h = 0; h < G; ++h) {
    const int64_t row = (int64_t)b * hq + g * G + h;
    s += expf(logits[row * stride + p] - lse[row]);
  }
  acc[((int64_t)b * c.num_kv_heads + g) * c.max_tokens + t] += s;
}

// Dense / keep modes (position = token): four consecutive tokens a thread,
// 16-byte loads of each head's logits and of the accumulators; the same
// per-token arithmetic in the same order as accum_kernel.
__global__ __launch_bounds__(AT) void accum4_kernel(kvc_cache c, int hq, const float* __restrict__ logits,
                                                    int64_t stride, const float* __restrict__ lse,
                                                    float* __restrict__ acc) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int p0 = 4 * (blockIdx.x * AT + threadIdx.x);
  const int G = hq / c.num_kv_heads;
  const int n = max(c.seq_lens[b], 0);
  if (p0 >= n) return;   // (p0 + 3 < max_tokens <= stride: the loads stay in the row)
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int h = 0; h < G; ++h) {
    const int64_t row = (int64_t)b * hq + g * G + h;
    const float l = lse[row];
    const float4 x = *reinterpret_cast<const float4*>(logits + row * stride + p0);
    s[0] += expf(x.x - l);
    s[1] += expf(x.y - l);
    s[2] += expf(x.z - l);
    s[3] += expf(x.w - l);
  }
  float* ap = acc + ((int64_t)b * c.num_kv_heads + g) * c.max_tokens + p0;
  if (p0 + 4 <= n) {
    float4 v = *reinterpret_cast<const float4*>(ap);
    v.x += s[0];
    v.y += s[1];
    v.z += s[2];
    v.w += s[3];
    *reinterpret_cast<float4*>(ap) = v;
  } else {
    for (int k = 0; k < n - p0; ++k) ap[k] += s[k];
  }
}

}  // namespace

hipError_t launch_accum(const kvc_cache& c, int hq, const float* logits, int64_t stride,
                        const float* lse, int mode, const int32_t* sel, int k_max, int n_sink,
                        int n_window, float* acc, hipStream_t s) {
  const int64_t np = mode == KVC_ATTEND_DROP ? (int64_t)n_sink + k_max + n_window
                    : mode == KVC_ATTEND_BLOCKS ? (int64_t)n_sink + (int64_t)GS * k_max + n_window
                                                : c.max_tokens;
  if (np <= 0) return hipSuccess;
  const bool contiguous = mode != KVC_ATTEND_DROP && mode != KVC_ATTEND_BLOCKS;
  if (contiguous && stride % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(acc) & 15) == 0) {
    const dim3 grid4((unsigned)((np / 4 + AT - 1) / AT), c.num_kv_heads, c.batch);
    accum4_kernel<<<grid4, AT, 0, s>>>(c, hq, logits, stride, lse, acc);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((np + AT - 1) / AT), c.num_kv_heads, c.batch);
  accum_kernel<<<grid, AT, 0, s>>>(c, hq, logits, stride, lse, mode, sel, k_max, n_sink, n_window, acc);
  return hipGetLastError();
}

}  // namespace kvc
