// Top-k attention probability mass per query head (TailorKV article, section
// 2.1: the dense preference score P = n_q - sum of the top-k softmax entries
// of the last n_q query rows decides whether a layer is quantization- or
// sparsity-friendly).  One workgroup per (sequence, query head) reads the
// row's logits (positions t < n, as a dense kvc_attend_decode writes them),
// finds the k-th largest by an exact 4-pass radix select over order-
// preserving 32-bit keys with LDS histograms, then sums exp(logit - lse) over
// the keys above it plus the needed copies of the k-th itself (the sum does
// not depend on which equal entries are taken).  The row is read twice: once
// for the top byte, once to sum the higher buckets and stage the chosen
// bucket's keys in LDS, where the three remaining passes and the final sum run
// (a bucket too large for LDS is re-read from memory instead).

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

// Bucket of the krem-th largest key among histogram hist (thread 0 only).
__device__ inline void pick_bucket(const uint32_t* hist, uint32_t& krem, uint32_t& prefix) {
  uint32_t above = 0u;
  int d = 255;
  for (; d > 0; --d) {
    if (above + hist[d] >= krem) break;
    above += hist[d];
  }
  krem -= above;
  prefix = (prefix << 8) | (uint32_t)d;
}

constexpr int CAP = 30720;   // keys of the k-th largest key's top-byte bucket staged in LDS

__global__ __launch_bounds__(PT) void topmass_kernel(kvc_cache c, int hq, const float* __restrict__ logits,
                                                     int64_t stride, const float* __restrict__ lse,
                                                     int k, float* __restrict__ out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t skeys[CAP];
  __shared__ uint32_t s_prefix, s_krem, s_cnt;
  __shared__ float s_part[PT / 64];
  const int bh = blockIdx.x, b = bh / hq, tid = threadIdx.x, lane = tid & 63;
  const int n = max(c.seq_lens[b], 0);
  const int kk = min(max(k, 0), n);
  const float* row = logits + (int64_t)bh * stride;
  if (kk == 0) {
    if (tid == 0) out[bh] = 0.f;
    return;
  }
  const float l0 = lse[bh];
  if (tid < 256) hist[tid] = 0u;
  if (tid == 0) {
    s_prefix = 0u;
    s_krem = (uint32_t)kk;
    s_cnt = 0u;
  }
  __syncthreads();
  // pass over the top byte, from the row in memory
  for (int t = tid; t < n; t += PT) atomicAdd(&hist[fkey(row[t]) >> 24], 1u);
  __syncthreads();
  if (tid == 0) pick_bucket(hist, s_krem, s_prefix);
  __syncthreads();
  // second read of the row: the mass of every key in a higher top-byte bucket,
  // and the keys of the chosen bucket staged in LDS (while they fit)
  const uint32_t d0 = s_prefix;
  float s = 0.f;
  for (int t0 = 0; t0 < n; t0 += PT) {
    const int t = t0 + tid;
    const float x = t < n ? row[t] : -INFINITY;
    const uint32_t key = fkey(x);
    const bool in = t < n && (key >> 24) == d0;
    if (t < n && (key >> 24) > d0) s += expf(x - l0);
    const uint64_t m = __ballot(in);
    uint32_t base = 0u;
    if (lane == 0 && m) base = atomicAdd(&s_cnt, (uint32_t)__popcll(m));
    base = __shfl(base, 0);
    const uint32_t idx = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    if (in && idx < (uint32_t)CAP) skeys[idx] = key;
  }
  __syncthreads();
  const uint32_t cnt = s_cnt;
  const bool staged = cnt <= (uint32_t)CAP;
  // passes over bytes 2, 1, 0 (staged keys, or the row again when they did not fit)
  for (int p = 2; p >= 0; --p) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    const int hs = 8 * (p + 1);
    if (staged) {
      for (uint32_t i = tid; i < cnt; i += PT) {
        const uint32_t key = skeys[i];
        if ((key >> hs) == prefix) atomicAdd(&hist[(key >> (8 * p)) & 255u], 1u);
      }
    } else {
      for (int t = tid; t < n; t += PT) {
        const uint32_t key = fkey(row[t]);
        if ((key >> hs) == prefix) atomicAdd(&hist[(key >> (8 * p)) & 255u], 1u);
      }
    }
    __syncthreads();
    if (tid == 0) pick_bucket(hist, s_krem, s_prefix);
    __syncthreads();
  }
  const uint32_t T = s_prefix;   // the k-th largest key; s_krem copies of it are taken
  if (staged) {   // keys above T inside the bucket (the higher buckets are in s)
    for (uint32_t i = tid; i < cnt; i += PT) {
      const uint32_t key = skeys[i];
      if (key > T) s += expf(fkey_value(key) - l0);
    }
  } else {        // every key above T
    s = 0.f;
    for (int t = tid; t < n; t += PT) {
      const float x = row[t];
      if (fkey(x) > T) s += expf(x - l0);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) s_part[tid >> 6] = s;
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
