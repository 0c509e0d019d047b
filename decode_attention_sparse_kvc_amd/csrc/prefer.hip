// Top-k attention probability mass per query head (TailorKV article, section
// 2.1: the dense preference score P = n_q - sum of the top-k softmax entries
// of the last n_q query rows decides whether a layer is quantization- or
// sparsity-friendly).  Each (sequence, query head) row of logits (positions
// t < n, as a dense kvc_attend_decode writes them) is split into S slices,
// so a layer's few rows still spread over the whole GPU:
//   1. mass_hist_kernel (slice): histogram of the top 11 bits (sign, exponent,
//      two mantissa bits) of the row's order-preserving 32-bit keys, written
//      per slice (no atomics, no clearing);
//   2. mass_pick_kernel (row): adds the row's slice histograms and finds the
//      bucket d0 holding the k-th largest key;
//   3. mass_collect_kernel (slice): reads its slice again, sums
//      exp(logit - lse) over the keys of higher buckets and copies the keys of
//      bucket d0 to its own region of the workspace;
//   4. mass_finish_kernel (row): gathers the bucket's keys (into LDS when they
//      fit, else they are re-read from the regions), runs the exact radix
//      select over the remaining 21 bits (digits of 8, 8 and 5 bits), and adds
//      the keys above the k-th, the needed copies of the k-th itself (the sum
//      does not depend on which equal entries are taken) and the slices'
//      higher-bucket sums.

#include <math.h>

#include "internal.h"

namespace kvc {
namespace {

constexpr int ST = 256;     // threads of a slice workgroup
constexpr int FT = 1024;    // threads of a finishing workgroup
constexpr int CAP = 30720;  // keys of bucket d0 staged in LDS by the finishing workgroup
constexpr int B1 = 11, NB1 = 1 << B1;   // first-level bits and buckets

__device__ inline uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ inline float fkey_value(uint32_t k) {
  return __uint_as_float((k >> 31) ? (k & 0x7FFFFFFFu) : ~k);
}

// Workspace layout for rows R = B * Hq, S slices of SL positions each:
// hist uint32 [R][S][NB1], mass float [R][S], cnt uint32 [R][S],
// info uint32 [R][4] (d0, krem of the first level), cand uint32 [R][S][SL].
struct MassLayout {
  int S, SL;
  size_t hist, mass, cnt, info, cand, total;
};

MassLayout mass_layout(const kvc_cache& c, int hq) {
  MassLayout L;
  const int R = c.batch * hq;
  int S = (512 + R - 1) / R;                        // about two slice workgroups a CU
  S = std::max(1, std::min(std::min(S, 64), c.max_tokens / 1024));
  L.S = S;
  L.SL = ((c.max_tokens + S - 1) / S + 255) / 256 * 256;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L.hist = 0;
  L.mass = al(L.hist + (size_t)R * S * NB1 * 4);
  L.cnt = al(L.mass + (size_t)R * S * 4);
  L.info = al(L.cnt + (size_t)R * S * 4);
  L.cand = al(L.info + (size_t)R * 16);
  L.total = al(L.cand + (size_t)R * S * L.SL * 4);
  return L;
}

struct MassArgs {
  kvc_cache c;
  int hq, k, S, SL;
  const float* logits;
  int64_t stride;
  const float* lse;
  float* out;
  uint32_t* hist;
  float* mass;
  uint32_t* cnt;
  uint32_t* info;
  uint32_t* cand;
};

// Row r's length n and its k_b = min(k, n).
__device__ inline void row_len(const MassArgs& a, int r, int& n, int& kk) {
  n = max(a.c.seq_lens[r / a.hq], 0);
  kk = min(max(a.k, 0), n);
}

// Bucket of the krem-th largest key given 256 bucket counts in LDS (buckets
// taken from 255 down): threads 0..255 scan, every thread must call.
// Writes s_pick[0] = the bucket, s_pick[1] = the count in higher buckets.
__device__ inline void pick_bucket(const uint32_t* hist, uint32_t krem, uint32_t* s_wt, uint32_t* s_pick) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t v = 0u;
  if (tid < 256) {
    v = hist[tid];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {   // suffix sums within the wave
      const uint32_t x = __shfl_down(v, o);
      if (lane + o < 64) v += x;
    }
    if (lane == 0) s_wt[w] = v;
  }
  __syncthreads();
  if (tid < 256) {
    uint32_t hi = 0u;
    for (int w2 = w + 1; w2 < 4; ++w2) hi += s_wt[w2];
    const uint32_t ge = v + hi, gt = ge - hist[tid];   // keys in buckets >= tid, > tid
    if (ge >= krem && gt < krem) {
      s_pick[0] = (uint32_t)tid;
      s_pick[1] = gt;
    }
  }
  __syncthreads();
}

// As pick_bucket over the NB1 first-level buckets with ST threads: thread t
// owns buckets [8t, 8t + 8).
__device__ inline void pick_bucket1(const uint32_t* hist, uint32_t krem, uint32_t* s_wt, uint32_t* s_pick) {
  constexpr int PER = NB1 / ST;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t own = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) own += hist[PER * tid + j];
  uint32_t v = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {   // suffix sums of the blocks within the wave
    const uint32_t x = __shfl_down(v, o);
    if (lane + o < 64) v += x;
  }
  if (lane == 0) s_wt[w] = v;
  __syncthreads();
  uint32_t hi = 0u;
  for (int w2 = w + 1; w2 < ST / 64; ++w2) hi += s_wt[w2];
  uint32_t gt = v + hi - own;   // keys in buckets above this thread's block
  if (gt < krem && gt + own >= krem) {
    for (int j = PER - 1; j >= 0; --j) {
      const uint32_t c = hist[PER * tid + j];
      if (gt + c >= krem) {
        s_pick[0] = (uint32_t)(PER * tid + j);
        s_pick[1] = gt;
        break;
      }
      gt += c;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(ST) void mass_hist_kernel(MassArgs a) {
  __shared__ uint32_t h[NB1];
  const int r = (int)blockIdx.x / a.S, s = (int)blockIdx.x - r * a.S, tid = threadIdx.x;
  int n, kk;
  row_len(a, r, n, kk);
  for (int j = tid; j < NB1; j += ST) h[j] = 0u;
  __syncthreads();
  if (kk > 0) {
    const float* row = a.logits + (int64_t)r * a.stride;
    const int t0 = s * a.SL, t1 = min(n, t0 + a.SL);
    // eight loads in flight a thread
    for (int t = t0 + tid; t < t1; t += 8 * ST) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = row[min(t + u * ST, t1 - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (t + u * ST < t1) atomicAdd(&h[fkey(x[u]) >> (32 - B1)], 1u);
    }
  }
  __syncthreads();
  for (int j = tid; j < NB1; j += ST) a.hist[((int64_t)r * a.S + s) * NB1 + j] = h[j];
}

// One workgroup per row: the row's histogram (sum of its slices') and the
// first-level bucket d0 of the k-th largest key, with krem = the keys of d0
// still to take.
__global__ __launch_bounds__(ST) void mass_pick_kernel(MassArgs a) {
  __shared__ uint32_t h[NB1];
  __shared__ uint32_t s_wt[ST / 64], s_pick[2];
  const int r = blockIdx.x, tid = threadIdx.x;
  int n, kk;
  row_len(a, r, n, kk);
  if (kk == 0) return;   // (uniform) the finishing kernel writes 0
  {
    constexpr int PER = NB1 / ST;
    uint32_t tot[PER] = {};
    // eight slices a trip: 8 * PER loads in flight a thread, a round trip per
    // eight slices instead of one per slice
    constexpr int SB = 8;
    int s2 = 0;
    for (; s2 + SB <= a.S; s2 += SB) {
      const uint32_t* hs = a.hist + ((int64_t)r * a.S + s2) * NB1 + tid;
      uint32_t v[SB][PER];
#pragma unroll
      for (int q = 0; q < SB; ++q)
#pragma unroll
        for (int j = 0; j < PER; ++j) v[q][j] = hs[q * NB1 + j * ST];
#pragma unroll
      for (int q = 0; q < SB; ++q)
#pragma unroll
        for (int j = 0; j < PER; ++j) tot[j] += v[q][j];
    }
    for (; s2 < a.S; ++s2) {
      const uint32_t* hs = a.hist + ((int64_t)r * a.S + s2) * NB1;
#pragma unroll
      for (int j = 0; j < PER; ++j) tot[j] += hs[tid + j * ST];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) h[tid + j * ST] = tot[j];
  }
  __syncthreads();
  pick_bucket1(h, (uint32_t)kk, s_wt, s_pick);
  if (tid == 0) {
    a.info[(int64_t)r * 4] = s_pick[0];
    a.info[(int64_t)r * 4 + 1] = (uint32_t)kk - s_pick[1];
  }
}

__global__ __launch_bounds__(ST) void mass_collect_kernel(MassArgs a) {
  __shared__ uint32_t s_cnt;
  __shared__ float s_part[ST / 64];
  const int r = (int)blockIdx.x / a.S, s = (int)blockIdx.x - r * a.S, tid = threadIdx.x, lane = tid & 63;
  int n, kk;
  row_len(a, r, n, kk);
  if (kk == 0) return;   // (uniform) the finishing kernel writes 0
  if (tid == 0) s_cnt = 0u;
  __syncthreads();
  const uint32_t d0 = a.info[(int64_t)r * 4];
  const float l0 = a.lse[r];
  const float* row = a.logits + (int64_t)r * a.stride;
  uint32_t* region = a.cand + ((int64_t)r * a.S + s) * a.SL;
  const int t0 = s * a.SL, t1 = min(n, t0 + a.SL);
  float sum = 0.f;
  for (int tb = t0 + tid; tb < t1; tb += 8 * ST) {   // eight loads in flight a thread
    float xs[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) xs[u] = row[min(tb + u * ST, t1 - 1)];
    uint32_t keys[8];
    uint64_t ms[8];
    uint32_t nin = 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = tb + u * ST;
      keys[u] = fkey(xs[u]);
      const uint32_t bk = keys[u] >> (32 - B1);
      if (t < t1 && bk > d0) sum += expf(xs[u] - l0);
      ms[u] = __ballot(t < t1 && bk == d0);
      nin += (uint32_t)__popcll(ms[u]);
    }
    if (nin) {   // (uniform) one slot range of the region per wave and step
      uint32_t base = 0u;
      if (lane == 0) base = atomicAdd(&s_cnt, nin);
      base = __shfl(base, 0);
      const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if ((ms[u] >> lane) & 1ull) region[base + (uint32_t)__popcll(ms[u] & below)] = keys[u];
        base += (uint32_t)__popcll(ms[u]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) s_part[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) {
    float tsum = 0.f;
    for (int w = 0; w < ST / 64; ++w) tsum += s_part[w];
    a.mass[(int64_t)r * a.S + s] = tsum;
    a.cnt[(int64_t)r * a.S + s] = s_cnt;
  }
}

__global__ __launch_bounds__(FT) void mass_finish_kernel(MassArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t skeys[CAP];
  __shared__ uint32_t s_off[65];
  __shared__ uint32_t s_wt[4], s_pick[2], s_prefix, s_krem;
  __shared__ float s_part[FT / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  int n, kk;
  row_len(a, r, n, kk);
  if (kk == 0) {
    if (tid == 0) a.out[r] = 0.f;
    return;
  }
  const int S = a.S;
  if (tid < 64) {   // region offsets: a scan of the S <= 64 counts in wave 0
    const uint32_t c = tid < S ? a.cnt[(int64_t)r * S + tid] : 0u;
    uint32_t v = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t x = __shfl_up(v, o);
      if (lane >= o) v += x;
    }
    if (tid < S) s_off[tid] = v - c;
    if (tid == S - 1) s_off[S] = v;     // the total
    if (tid == 0) {
      s_prefix = a.info[(int64_t)r * 4];
      s_krem = a.info[(int64_t)r * 4 + 1];
    }
  }
  __syncthreads();
  const uint32_t total = s_off[S];
  const bool staged = total <= (uint32_t)CAP;
  const uint32_t* cand = a.cand + (int64_t)r * S * a.SL;
  // key number i of the bucket, from its slice's region (s_off is ascending)
  auto region_key = [&](uint32_t i) -> uint32_t {
    int lo = 0, hi = S - 1;   // the last slice s with s_off[s] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return cand[(int64_t)lo * a.SL + (i - s_off[lo])];
  };
  // f(key) for every key of the bucket: from LDS when staged, else from the regions
  auto each_key = [&](auto&& f) {
    if (staged) {
      for (uint32_t i = tid; i < total; i += FT) f(skeys[i]);
    } else {
      for (uint32_t i = tid; i < total; i += FT) f(region_key(i));
    }
  };
  if (staged) {   // eight loads in flight a thread
    for (uint32_t i = tid; i < total; i += 8 * FT) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = region_key(min(i + u * FT, total - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i + u * FT < total) skeys[i + u * FT] = v[u];
    }
  }
  __syncthreads();
  // passes over the remaining 21 bits: digits of 8, 8 and 5 bits
  int low = 32 - B1;   // bits below the selected prefix
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    const int wd = p < 2 ? 8 : 5, sh = low - wd;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    each_key([&](uint32_t key) {
      if ((key >> low) == prefix) atomicAdd(&hist[(key >> sh) & ((1u << wd) - 1u)], 1u);
    });
    __syncthreads();
    pick_bucket(hist, s_krem, s_wt, s_pick);
    if (tid == 0) {
      s_krem -= s_pick[1];
      s_prefix = (prefix << wd) | s_pick[0];
    }
    __syncthreads();
    low = sh;
  }
  const uint32_t T = s_prefix;   // the k-th largest key; s_krem copies of it are taken
  const float l0 = a.lse[r];
  float sum = 0.f;
  each_key([&](uint32_t key) {
    if (key > T) sum += expf(fkey_value(key) - l0);
  });
  if (tid < S) sum += a.mass[(int64_t)r * S + tid];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) s_part[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
    for (int w = 0; w < FT / 64; ++w) tot += s_part[w];
    a.out[r] = tot + (float)s_krem * expf(fkey_value(T) - l0);
  }
}

}  // namespace

size_t topk_mass_workspace_bytes(const kvc_cache& c, int hq) { return mass_layout(c, hq).total; }

hipError_t launch_topk_mass(const kvc_cache& c, int hq, const float* logits, int64_t stride,
                            const float* lse, int k, float* out, void* workspace, hipStream_t st) {
  const MassLayout L = mass_layout(c, hq);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  MassArgs a;
  a.c = c;
  a.hq = hq;
  a.k = k;
  a.S = L.S;
  a.SL = L.SL;
  a.logits = logits;
  a.stride = stride;
  a.lse = lse;
  a.out = out;
  a.hist = reinterpret_cast<uint32_t*>(ws + L.hist);
  a.mass = reinterpret_cast<float*>(ws + L.mass);
  a.cnt = reinterpret_cast<uint32_t*>(ws + L.cnt);
  a.info = reinterpret_cast<uint32_t*>(ws + L.info);
  a.cand = reinterpret_cast<uint32_t*>(ws + L.cand);
  const int R = c.batch * hq;
  const dim3 grid((uint32_t)L.S * (uint32_t)R);   // workgroup r * S + s: slice s of row r
  mass_hist_kernel<<<grid, ST, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mass_pick_kernel<<<R, ST, 0, st>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  mass_collect_kernel<<<grid, ST, 0, st>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  mass_finish_kernel<<<R, FT, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvc
