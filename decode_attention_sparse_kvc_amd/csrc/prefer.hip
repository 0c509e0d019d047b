// Top-k attention probability mass per query head (TailorKV article, section
// 2.1: the dense preference score P = n_q - sum of the top-k softmax entries
// of the last n_q query rows decides whether a layer is quantization- or
// sparsity-friendly).  One workgroup per (sequence, query head) reads the
// row's logits (positions t < n, as a dense kvc_attend_decode writes them),
// finds the k-th largest by an exact 4-pass radix select over order-
// preserving 32-bit keys with LDS histograms, then sums exp(logit - lse) over
// the keys above it plus the needed copies of the k-th itself (the sum does
// not depend on which equal entries are taken).

#include <math.h>

#include "internal.h"

namespace kvc {
namespace {

constexpr int PT = 1024;   // threads per workgroup

__device__ inline uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ inline float fkey_value(uint32_t k) {
  return __uint_as_float((k >> 31) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ __launch_bounds__(PT) void topmass_kernel(kvc_cache c, int hq, const float* __restrict__ logits,
                                                     int64_t stride, const float* __restrict__ lse,
                                                     int k, float* __restrict__ out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_krem;
  __shared__ float s_part[PT / 64];
  const int bh = blockIdx.x, b = bh / hq, tid = threadIdx.x;
  const int n = max(c.seq_lens[b], 0);
  const int kk = min(max(k, 0), n);
  const float* row = logits + (int64_t)bh * stride;
  if (kk == 0) {
    if (tid == 0) out[bh] = 0.f;
    return;
  }
  if (tid == 0) {
    s_prefix = 0u;
    s_krem = (uint32_t)kk;
  }
  for (int p = 3; p >= 0; --p) {   // byte p of the key, most significant first
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    const int hs = 8 * (p + 1);     // bits above byte p
    for (int t = tid; t < n; t += PT) {
      const uint32_t key = fkey(row[t]);
      if (hs == 32 || (key >> hs) == prefix) atomicAdd(&hist[(key >> (8 * p)) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {   // the bucket holding the krem-th largest remaining key
      uint32_t krem = s_krem, above = 0u;
      int d = 255;
      for (; d > 0; --d) {
        if (above + hist[d] >= krem) break;
        above += hist[d];
      }
      s_krem = krem - above;
      s_prefix = (prefix << 8) | (uint32_t)d;
    }
    __syncthreads();
  }
  const uint32_t T = s_prefix;   // the k-th largest key; s_krem copies of it are taken
  const float l0 = lse[bh];
  float s = 0.f;
  for (int t = tid; t < n; t += PT) {
    const float x = row[t];
    if (fkey(x) > T) s += expf(x - l0);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) s_part[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
    for (int w = 0; w < PT / 64; ++w) tot += s_part[w];
    out[bh] = tot + (float)s_krem * expf(fkey_value(T) - l0);
  }
}

}  // namespace

hipError_t launch_topk_mass(const kvc_cache& c, int hq, const float* logits, int64_t stride,
                            const float* lse, int k, float* out, hipStream_t s) {
  topmass_kernel<<<c.batch * hq, PT, 0, s>>>(c, hq, logits, stride, lse, k, out);
  return hipGetLastError();
}

}  // namespace kvc
