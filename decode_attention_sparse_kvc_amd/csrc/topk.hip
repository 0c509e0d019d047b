// Token scoring and exact Top-K selection (TailorKV article, section 2.3:
// channel importance |q_i| * max|K_i|, approximate scores on the critical
// channels, Top-K retrieval; meeting-LLM article, section 2.2: query-aware
// scores; StreamingLLM / H2O survey, section 3: sinks, recent window and
// cumulative scores).
//
// Kernels, all on the caller's stream:
//   prep    per (sequence, KV head): critical channels (exact fp64 products,
//           rank with ties to the lower channel) and zeroed histograms.
//   score   one thread per token: the fp64 score, summed channel by channel in
//           ascending order from +0.0 (the order the interface fixes, so results
//           are reproducible bit for bit), max over the query group, turned into
//           an order-preserving 64-bit key (0 = not a candidate); histogram of
//           the key's top byte.
//   radix   passes 1..7: histogram of the next byte among keys that share the
//           bytes chosen so far (each workgroup re-derives those bytes from the
//           earlier histograms).
//   mark    bitmaps of keys above the k-th largest key T and equal to T.
//   emit    one workgroup per (sequence, KV head): the first k - #above keys
//           equal to T by index, then every selected index in ascending order.

#include <math.h>

#include "internal.h"

namespace kvc {
namespace {

constexpr int ST = 256;        // threads of the scoring / radix workgroups
constexpr int TPB = 1024;      // tokens per radix / mark workgroup
constexpr int ET = 1024;       // threads of the emit workgroup
constexpr int PASSES = 8;

struct TopkArgs {
  kvc_cache c;
  const uint16_t* q;
  int hq, G, mode, n_crit;
  const float* ext;
  int n_sink, n_window;
  const int32_t* k_per_seq;
  int k_max;
  int32_t* out_idx;
  double* out_scores;
  int32_t* out_channels;
  // workspace
  uint64_t* keys;      // [B][Hkv][max_tokens]
  uint32_t* hist;      // [B][Hkv][PASSES][256]
  uint32_t* above;     // [B][Hkv][max_tokens / 32]
  uint32_t* equal;     // [B][Hkv][max_tokens / 32]
  int32_t* channels;   // [B][Hkv][128]
};

__device__ inline uint64_t order_key(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ inline int64_t pair_index(const TopkArgs& a, int b, int g) {
  return (int64_t)b * a.c.num_kv_heads + g;
}

// Number of tokens to select and the candidate range of (sequence b).
__device__ inline void cand_range(const TopkArgs& a, int b, int& lo, int& hi, int& k) {
  const int n = max(a.c.seq_lens[b], 0);
  lo = a.n_sink;
  hi = n - a.n_window;
  const int ncand = max(0, hi - lo);
  int want = a.k_per_seq ? a.k_per_seq[b] : a.k_max;
  want = min(max(want, 0), a.k_max);
  k = min(want, ncand);
}

// ------------------------------------------------------------------ prep
__global__ __launch_bounds__(D) void prep_kernel(TopkArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  uint32_t* h = a.hist + pi * PASSES * 256;
  for (int e = c; e < PASSES * 256; e += D) h[e] = 0u;
  __shared__ double s[D];
  __shared__ int chosen[D];
  if (a.mode == KVC_SCORE_CRITICAL) {
    double qm = 0.0;
    for (int hh = 0; hh < a.G; ++hh)
      qm = fmax(qm, fabs((double)h2f(a.q[((int64_t)b * a.hq + g * a.G + hh) * D + c])));
    const double kabs = (double)a.c.k_absmax[pi * D + c];
    s[c] = __dmul_rn(qm, kabs);
    __syncthreads();
    int rank = 0;
    for (int o = 0; o < D; ++o) rank += (s[o] > s[c]) || (s[o] == s[c] && o < c);
    chosen[c] = rank < a.n_crit;
    __syncthreads();
    if (chosen[c]) {
      int pos = 0;
      for (int o = 0; o < c; ++o) pos += chosen[o];
      a.channels[pi * D + pos] = c;
      if (a.out_channels) a.out_channels[pi * a.n_crit + pos] = c;
    }
  }
}

// ------------------------------------------------------------------ score
// k value of token t, channel ch as an exact double: fp16 row, tail row, or
// code * scale + zero (fp64 multiply then add, both exact).
__device__ inline double key_value(const TopkArgs& a, int b, int g, int t, int ch, int nq,
                                   int64_t slot) {
  const kvc_cache& c = a.c;
  const int fmt = c.format;
  if (fmt == KVC_FMT_FP16) {
    if (c.kT && c.page_size == 0)
      return (double)h2f(c.kT[((int64_t)(b * c.num_kv_heads + g) * D + ch) * c.max_tokens + t]);
    return (double)h2f(c.k16[slot * D + ch]);
  }
  if (t >= nq)
    return (double)h2f(c.k_tail[(((int64_t)b * c.num_kv_heads + g) * GS + (t - nq)) * D + ch]);
  uint32_t code;
  if (fmt == KVC_FMT_INT4) {
    const int n = (int)(slot % TILE);
    const int lane = 16 * (ch / 32) + n, d = (ch % 32) / 8, j = ch % 8;
    const uint32_t u = reinterpret_cast<const uint32_t*>(c.k_codes + (slot / TILE) * UNIT_BYTES)[lane * 4 + d];
    code = (u >> nib_pos(j)) & 15u;
  } else {
    const int n = (int)(slot % GS);
    const int lane = 16 * (ch / 32) + n % 16, d = n / 16;
    const uint32_t u = reinterpret_cast<const uint32_t*>(c.k_codes + (slot / GS) * UNIT_BYTES)[lane * 4 + d];
    code = (u >> bit_pos(ch % 32)) & 1u;
  }
  const uint16_t* meta = c.k_meta +
      ((((int64_t)b * c.num_kv_heads + g) * (c.max_tokens / GS) + t / GS) * 2) * D;
  return __dadd_rn(__dmul_rn((double)code, (double)h2f(meta[ch])), (double)h2f(meta[D + ch]));
}

constexpr int GMAX = 16;       // query heads per KV head supported by scoring

__global__ __launch_bounds__(ST) void score_kernel(TopkArgs a) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int t = blockIdx.x * ST + tid;
  const int64_t pi = pair_index(a, b, g);
  __shared__ double sq[GMAX * D];   // q as fp64, [head][channel slot]
  __shared__ int sch[D];
  __shared__ uint32_t sh[256];
  const int G = a.G;
  const int nch = a.mode == KVC_SCORE_CRITICAL ? a.n_crit : (a.mode == KVC_SCORE_EXACT ? D : 0);
  for (int e = tid; e < nch; e += ST)
    sch[e] = a.mode == KVC_SCORE_CRITICAL ? a.channels[pi * D + e] : e;
  sh[tid] = 0u;
  __syncthreads();
  for (int e = tid; e < G * nch; e += ST) {
    const int hh = e / nch, k = e % nch;
    sq[hh * D + k] = (double)h2f(a.q[((int64_t)b * a.hq + g * G + hh) * D + sch[k]]);
  }
  __syncthreads();

  int lo, hi, kk;
  cand_range(a, b, lo, hi, kk);
  const int n = max(a.c.seq_lens[b], 0);
  const bool in = t < a.c.max_tokens;
  uint64_t key = 0;
  if (in && t >= lo && t < hi) {
    double r;
    if (a.mode == KVC_SCORE_EXTERNAL) {
      r = (double)a.ext[pi * a.c.max_tokens + t];
    } else {
      const int nq = a.c.format == KVC_FMT_FP16 ? n : (n & ~(GS - 1));
      const int64_t slot = slot_of(a.c, b, g, t);
      r = -INFINITY;
      if (slot >= 0) {
        // per head: +0.0, then one channel at a time in ascending order
        double acc[GMAX];
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh) acc[hh] = 0.0;
        for (int k = 0; k < nch; ++k) {
          const double kv = key_value(a, b, g, t, sch[k], nq, slot);
#pragma unroll
          for (int hh = 0; hh < GMAX; ++hh)
            if (hh < G) acc[hh] = __dadd_rn(acc[hh], __dmul_rn(sq[hh * D + k], kv));
        }
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh)
          if (hh < G) r = fmax(r, acc[hh]);
      }
    }
    r = __dadd_rn(r, 0.0);
    key = order_key(r);
    if (a.out_scores) a.out_scores[pi * a.c.max_tokens + t] = r;
  }
  if (in) a.keys[pi * a.c.max_tokens + t] = key;
  if (key) atomicAdd(&sh[key >> 56], 1u);
  __syncthreads();
  if (sh[tid]) atomicAdd(&a.hist[pi * PASSES * 256 + tid], sh[tid]);
}

// ------------------------------------------------------------------ radix passes
// From the histograms of passes [0, p): the byte chosen at each pass, the key
// prefix, and how many keys of the current bucket still have to be taken.
// Executed redundantly by every workgroup (256 threads); returns via LDS.
__device__ void derive_prefix(const uint32_t* hist, int p, int k, uint64_t* s_prefix, int* s_krem,
                              uint32_t* s_scan) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int krem = k;
  for (int pp = 0; pp < p; ++pp) {
    // suffix sums: number of keys in the bucket with byte >= d
    s_scan[tid] = hist[pp * 256 + tid];
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const uint32_t v = tid + o < 256 ? s_scan[tid + o] : 0u;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    // chosen byte d: suffix(d) >= krem > suffix(d + 1)
    const uint32_t ge = s_scan[tid];
    const uint32_t gt = tid < 255 ? s_scan[tid + 1] : 0u;
    if (ge >= (uint32_t)krem && gt < (uint32_t)krem) {
      s_prefix[0] = (prefix << 8) | (uint64_t)tid;
      s_krem[0] = krem - (int)gt;
    }
    __syncthreads();
    prefix = s_prefix[0];
    krem = s_krem[0];
    __syncthreads();
  }
  if (tid == 0) {
    s_prefix[0] = prefix;
    s_krem[0] = krem;
  }
  __syncthreads();
}

__global__ __launch_bounds__(ST) void radix_kernel(TopkArgs a, int p) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  __shared__ uint64_t s_prefix[1];
  __shared__ int s_krem[1];
  __shared__ uint32_t s_scan[256];
  __shared__ uint32_t sh[256];
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  if (k <= 0) return;
  uint32_t* hist = a.hist + pi * PASSES * 256;
  derive_prefix(hist, p, k, s_prefix, s_krem, s_scan);
  const uint64_t prefix = s_prefix[0];
  sh[tid] = 0u;
  __syncthreads();
  const int shift = 64 - 8 * p;   // bits above the current byte
  const int t0 = blockIdx.x * TPB;
  const uint64_t* keys = a.keys + pi * a.c.max_tokens;
  for (int t = t0 + tid; t < min(t0 + TPB, a.c.max_tokens); t += ST) {
    const uint64_t key = keys[t];
    if (key && (key >> shift) == prefix) atomicAdd(&sh[(key >> (shift - 8)) & 255u], 1u);
  }
  __syncthreads();
  if (sh[tid]) atomicAdd(&hist[p * 256 + tid], sh[tid]);
}

// ------------------------------------------------------------------ mark
__global__ __launch_bounds__(ST) void mark_kernel(TopkArgs a) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  __shared__ uint64_t s_prefix[1];
  __shared__ int s_krem[1];
  __shared__ uint32_t s_scan[256];
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  uint64_t T = ~0ull;     // nothing is above the all-ones key and nothing equals it
  if (k > 0) {
    derive_prefix(a.hist + pi * PASSES * 256, PASSES, k, s_prefix, s_krem, s_scan);
    T = s_prefix[0];
  }
  const int words = a.c.max_tokens / 32;
  const uint64_t* keys = a.keys + pi * a.c.max_tokens;
  const int w0 = blockIdx.x * (TPB / 32);
  for (int wd = w0 + tid; wd < min(w0 + TPB / 32, words); wd += ST) {
    uint32_t ab = 0u, eq = 0u;
    for (int i = 0; i < 32; ++i) {
      const uint64_t key = keys[wd * 32 + i];
      ab |= (uint32_t)(key != 0 && key > T && k > 0) << i;
      eq |= (uint32_t)(key != 0 && key == T && k > 0) << i;
    }
    a.above[pi * words + wd] = ab;
    a.equal[pi * words + wd] = eq;
  }
}

// ------------------------------------------------------------------ emit
__device__ inline int block_exclusive_scan(int v, int* s, int& total) {
  const int tid = threadIdx.x;
  s[tid] = v;
  __syncthreads();
  for (int o = 1; o < ET; o <<= 1) {
    const int x = tid >= o ? s[tid - o] : 0;
    __syncthreads();
    s[tid] += x;
    __syncthreads();
  }
  total = s[ET - 1];
  const int excl = s[tid] - v;
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(ET) void emit_kernel(TopkArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  __shared__ int s[ET];
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  const int words = a.c.max_tokens / 32;
  const int per = (words + ET - 1) / ET;
  const int wa = tid * per, wb = min(wa + per, words);
  const uint32_t* ab = a.above + pi * words;
  const uint32_t* eq = a.equal + pi * words;
  int32_t* out = a.out_idx + pi * a.k_max;
  // how many equal keys to take: k - #above
  int n_ab = 0, n_eq = 0;
  for (int wd = wa; wd < wb; ++wd) {
    n_ab += __popc(ab[wd]);
    n_eq += __popc(eq[wd]);
  }
  int tot_ab, tot_eq;
  block_exclusive_scan(n_ab, s, tot_ab);
  const int eq_before = block_exclusive_scan(n_eq, s, tot_eq);
  const int take_eq = max(0, k - tot_ab);
  // selected = above | (first take_eq equal bits by index)
  int n_sel = 0;
  int eq_seen = eq_before;
  for (int wd = wa; wd < wb; ++wd) {
    uint32_t e = eq[wd];
    uint32_t keep = 0u;
    while (e && eq_seen < take_eq) {
      const uint32_t bit = e & (0u - e);
      keep |= bit;
      e ^= bit;
      ++eq_seen;
    }
    n_sel += __popc(ab[wd] | keep);
  }
  int total;
  int pos = block_exclusive_scan(n_sel, s, total);
  eq_seen = eq_before;
  for (int wd = wa; wd < wb; ++wd) {
    uint32_t e = eq[wd];
    uint32_t keep = 0u;
    while (e && eq_seen < take_eq) {
      const uint32_t bit = e & (0u - e);
      keep |= bit;
      e ^= bit;
      ++eq_seen;
    }
    uint32_t m = ab[wd] | keep;
    while (m) {
      const int i = __ffs(m) - 1;
      m &= m - 1;
      if (pos < a.k_max) out[pos] = wd * 32 + i;
      ++pos;
    }
  }
  for (int e = total + tid; e < a.k_max; e += ET) out[e] = -1;
}

}  // namespace

size_t topk_workspace_bytes(const kvc_cache& c) {
  const size_t pairs = (size_t)c.batch * c.num_kv_heads;
  const size_t words = c.max_tokens / 32;
  size_t bytes = pairs * c.max_tokens * sizeof(uint64_t);
  bytes += pairs * PASSES * 256 * sizeof(uint32_t);
  bytes += 2 * pairs * words * sizeof(uint32_t);
  bytes += pairs * D * sizeof(int32_t);
  return bytes;
}

hipError_t launch_score_topk(const kvc_cache& c, const uint16_t* q, int hq, int mode, int n_crit,
                             const float* ext, int n_sink, int n_window, const int32_t* k_per_seq,
                             int k_max, int32_t* out_idx, double* out_scores,
                             int32_t* out_channels, void* ws, hipStream_t s) {
  TopkArgs a;
  a.c = c;
  a.q = q;
  a.hq = hq;
  a.G = hq / c.num_kv_heads;
  a.mode = mode;
  a.n_crit = n_crit;
  a.ext = ext;
  a.n_sink = n_sink;
  a.n_window = n_window;
  a.k_per_seq = k_per_seq;
  a.k_max = k_max;
  a.out_idx = out_idx;
  a.out_scores = out_scores;
  a.out_channels = out_channels;
  const size_t pairs = (size_t)c.batch * c.num_kv_heads;
  const size_t words = c.max_tokens / 32;
  char* p = static_cast<char*>(ws);
  a.keys = reinterpret_cast<uint64_t*>(p);
  p += pairs * c.max_tokens * sizeof(uint64_t);
  a.hist = reinterpret_cast<uint32_t*>(p);
  p += pairs * PASSES * 256 * sizeof(uint32_t);
  a.above = reinterpret_cast<uint32_t*>(p);
  p += pairs * words * sizeof(uint32_t);
  a.equal = reinterpret_cast<uint32_t*>(p);
  p += pairs * words * sizeof(uint32_t);
  a.channels = reinterpret_cast<int32_t*>(p);

  const int Hkv = c.num_kv_heads, B = c.batch;
  prep_kernel<<<dim3(Hkv, B), D, 0, s>>>(a);
  score_kernel<<<dim3((c.max_tokens + ST - 1) / ST, Hkv, B), ST, 0, s>>>(a);
  const dim3 rgrid((c.max_tokens + TPB - 1) / TPB, Hkv, B);
  for (int pass = 1; pass < PASSES; ++pass) radix_kernel<<<rgrid, ST, 0, s>>>(a, pass);
  mark_kernel<<<rgrid, ST, 0, s>>>(a);
  emit_kernel<<<dim3(Hkv, B), ET, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvc
