// Token scoring and exact Top-K selection (TailorKV article, section 2.3:
// channel importance |q_i| * max|K_i|, approximate scores on the critical
// channels, Top-K retrieval; meeting-LLM article, section 2.2: query-aware
// scores; StreamingLLM / H2O survey, section 3: sinks, recent window and
// cumulative scores).
//
// Kernels, all on the caller's stream:
//   prep     per (sequence, KV head): critical channels (exact fp64 products,
//            rank with ties to the lower channel) and a zeroed histogram.
//   score    one thread per token: the fp64 score, summed channel by channel in
//            ascending order from +0.0 (the order the interface fixes, so results
//            are reproducible bit for bit), max over the query group, turned into
//            an order-preserving 64-bit key (0 = not a candidate); histogram of
//            the keys' 12-bit coarse bins (sign, clamped exponent, 4 mantissa
//            bits: a monotone function of the key).
//   compact  (long ranges) per 4096 items: the coarse bin tb holding the k-th
//            largest key (from the histogram); a bitmap of the items in bins
//            above tb, and the items of bin tb (key, index) in index order.
//   finish   one workgroup per (sequence, KV head): exact radix select among
//            the keys of bin tb (LDS passes over 8-bit digits, from the first
//            digit where they differ), lower index first among equal keys, then
//            every selected index in ascending order.  Short ranges skip
//            compact: finish reads the keys itself.
// Block mode (meeting-LLM article, section 8.1: importance averaged over
// 64-token blocks, the top blocks kept): score writes each token's fp64 score
// and no key; block_key averages every candidate block's 64 scores into the
// block's key (item j of the pair's key row) and histograms it; the kernels
// above then select blocks instead of tokens.

#include <math.h>

#include "internal.h"

namespace kvc {
namespace {

constexpr int ST = 256;        // threads of the block-key and compaction workgroups
constexpr int SCT = 1024;      // threads (= tokens) of a scoring workgroup
constexpr int CBINS = 4096;    // coarse bins of the keys
constexpr int HREP = 2;        // copies of the coarse histogram (spread the global atomics)
constexpr int HW = CBINS * HREP;   // histogram words per (sequence, KV head)
constexpr int CT = 4096;       // items per compaction workgroup
constexpr int FT = 1024;       // threads of the finish workgroup
constexpr int CAP = 8192;      // bin-tb items the finish workgroup holds in LDS
constexpr int DIRECT_MAX = 8192;   // items up to which finish reads the keys itself (in LDS)
constexpr int MAXR = 4096;     // compaction regions finish can index (items <= MAXR * CT)
constexpr int EW = 4096;       // bitmap words per emission chunk (EW / FT words a thread)

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
  uint64_t* keys;      // [B][Hkv][max_tokens] item keys (0: not a candidate)
  uint32_t* hist;      // [B][Hkv][HREP][CBINS] coarse histogram
  uint32_t* above;     // [B][Hkv][max_tokens / 32] items in bins above the threshold bin
  uint64_t* ckey;      // [B][Hkv][nreg * CT] keys of the threshold bin, per compaction region
  int32_t* cidx;       // [B][Hkv][nreg * CT] their item indices
  int32_t* ccount;     // [B][Hkv][nreg] entries per region
  int nreg;            // compaction regions per pair (ceil(items / CT))
  int32_t* channels;   // [B][Hkv][128]
  double* qsel;        // critical mode: [B][Hkv][GMAX][128] q of the group's heads on the
                       // channel list (slot k = k-th critical channel), fp64
  bool blocks;         // rank 64-token blocks (items = block ids)
  double* tscore;      // block mode: [B][Hkv][max_tokens] token scores
};

__device__ inline uint64_t order_key(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// 12-bit coarse bin of a key: its top bit (the score's sign), its exponent
// field clamped to a window of 128 binades (2^-64 .. 2^63 in magnitude; keys
// outside it share the end bins), then the top 4 mantissa bits (0 below the
// window, 15 above it).  Non-decreasing in the key, so every key in a higher
// bin is larger than every key in a lower one.
__device__ inline uint32_t coarse_of(uint64_t key) {
  const uint32_t t = (uint32_t)(key >> 63);
  const int e = (int)((key >> 52) & 0x7FFu) - (t ? 959 : 961);
  const uint32_t m4 = (uint32_t)(key >> 48) & 15u;
  const uint32_t e7 = e < 0 ? 0u : e > 127 ? 127u : (uint32_t)e;
  const uint32_t mm = e < 0 ? 0u : e > 127 ? 15u : m4;
  return (t << 11) | (e7 << 4) | mm;
}

// Items the selection runs over per (sequence, KV head): tokens, or blocks.
__host__ __device__ inline int item_count(const kvc_cache& c, bool blocks) {
  return blocks ? c.max_tokens / GS : c.max_tokens;
}

__device__ inline int64_t pair_index(const TopkArgs& a, int b, int g) {
  return (int64_t)b * a.c.num_kv_heads + g;
}

// Number of items to select and the candidate range of (sequence b): tokens
// [n_sink, n - n_window), or in block mode the complete 64-token blocks
// wholly inside that range.
__device__ inline void cand_range(const TopkArgs& a, int b, int& lo, int& hi, int& k) {
  const int n = max(a.c.seq_lens[b], 0);
  if (a.blocks) {
    lo = (a.n_sink + GS - 1) / GS;
    hi = max(lo, max(n - a.n_window, 0) / GS);
  } else {
    lo = a.n_sink;
    hi = n - a.n_window;
  }
  const int ncand = max(0, hi - lo);
  int want = a.k_per_seq ? a.k_per_seq[b] : a.k_max;
  want = min(max(want, 0), a.k_max);
  k = min(want, ncand);
}

// ------------------------------------------------------------------ prep
constexpr int GMAX_PREP = 16;
__global__ __launch_bounds__(D) void prep_kernel(TopkArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  uint4* h = reinterpret_cast<uint4*>(a.hist + pi * HW);
  for (int e = c; e < HW / 4; e += D) h[e] = uint4{0u, 0u, 0u, 0u};
  __shared__ double s[D];
  __shared__ int chosen[D];
  if (a.mode == KVC_SCORE_CRITICAL) {
    // every load is issued before any is used: heads past the group re-read
    // head 0 (the maximum is unchanged), so no load sits behind a branch
    const float kabs_f = a.c.k_absmax[pi * D + c];
    const uint16_t* qg = a.q + ((int64_t)b * a.hq + g * a.G) * D + c;
    uint16_t qh[GMAX_PREP];
#pragma unroll
    for (int hh = 0; hh < GMAX_PREP; ++hh) qh[hh] = qg[(hh < a.G ? hh : 0) * D];
    double qm = 0.0;
#pragma unroll
    for (int hh = 0; hh < GMAX_PREP; ++hh) qm = fmax(qm, fabs((double)h2f(qh[hh])));
    const double kabs = (double)kabs_f;
    s[c] = __dmul_rn(qm, kabs);
    __syncthreads();
    // rank of channel c under (s desc, c asc); the LDS reads are independent
    const double sc = s[c];
    int rank = 0;
#pragma unroll 32
    for (int o = 0; o < D; ++o) {
      const double so = s[o];
      rank += (so > sc) || (so == sc && o < c);
    }
    // position in the ascending list: chosen channels below c (ballots of the two waves)
    const bool mine = rank < a.n_crit;
    const uint64_t bal = __ballot(mine);
    if ((c & 63) == 0) chosen[c >> 6] = __popcll(bal);
    __syncthreads();
    if (mine) {
      const int pos = __popcll(bal & ((1ull << (c & 63)) - 1ull)) + (c >= 64 ? chosen[0] : 0);
      a.channels[pi * D + pos] = c;
      if (a.out_channels) a.out_channels[pi * a.n_crit + pos] = c;
      // the scoring kernel's q operands, so it needs no gather through the list
#pragma unroll
      for (int hh = 0; hh < GMAX_PREP; ++hh)
        if (hh < a.G) a.qsel[(pi * GMAX_PREP + hh) * D + pos] = (double)h2f(qh[hh]);
    }
  }
}

// ------------------------------------------------------------------ score
constexpr int GMAX = 16;       // query heads per KV head supported by scoring
static_assert(GMAX == GMAX_PREP, "prep writes the q operands the scoring kernel reads");
constexpr int CB_CRIT = 8;     // channels whose loads are issued together (critical channels)
constexpr int CB_EXACT = 32;   // (every channel)
constexpr uint32_t OUT_TAG = 0xFFFF0000u;   // staged K metadata word of an outlier channel

// Scores of one token on the channel list: per query head, +0.0 then one
// channel at a time in ascending order.  The loads of CB channels are issued
// together, then their q values are read from LDS, then the adds run.  GT is
// the query group size when it is known at compile time (0: up to GMAX).
// ALL: the list is every channel in order (exact mode), known at compile time,
// so loads of channels that share a code word are issued once.
template <int GT, int CB, bool ALL = false, typename Load, typename Aux, typename Value>
__device__ inline double token_score(int G, int nch_, const int* sch, const double* sq, Load load,
                                     Aux aux, Value value) {
  constexpr int GN = GT > 0 ? GT : GMAX;
  const int nch = ALL ? D : nch_;
  double acc[GN];
#pragma unroll
  for (int hh = 0; hh < GN; ++hh) acc[hh] = 0.0;
  // (batches stay a loop: unrolling the 128-channel exact sum over G heads
  // leaves more live values than the registers hold)
#pragma unroll 1
  for (int k0 = 0; k0 < (ALL ? D : nch); k0 += CB) {
    int ch[CB];
    uint32_t raw[CB], mx[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) ch[u] = ALL ? k0 + u : sch[min(k0 + u, nch - 1)];
#pragma unroll
    for (int u = 0; u < CB; ++u) raw[u] = load(ch[u]);   // global loads, all in flight
#pragma unroll
    for (int u = 0; u < CB; ++u) mx[u] = aux(ch[u]);     // LDS reads, all in flight
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const bool on = k0 + u < nch;
      const double v = value(ch[u], raw[u], mx[u]);
      const int kq = min(k0 + u, nch - 1);
#pragma unroll
      for (int hh = 0; hh < GN; ++hh) {
        if (GT > 0 || hh < G) {
          const double nx = __dadd_rn(acc[hh], __dmul_rn(sq[hh * (ALL ? D : nch) + kq], v));
          acc[hh] = on ? nx : acc[hh];
        }
      }
    }
  }
  double r = acc[0];
#pragma unroll
  for (int hh = 1; hh < GN; ++hh)
    if (GT > 0 || hh < G) r = fmax(r, acc[hh]);
  return r;
}

// One thread per token: the score on the channel list (max over the query
// group), an order-preserving key, and the coarse histogram of the keys
// (counted in LDS, then one global atomic per non-empty bin of the workgroup).
// Workgroup size: 1024 tokens (one histogram flush per 1024 keys), except in
// exact mode and for query groups of 8 or more heads, whose sums need the
// registers of 256-thread groups.
template <bool EXACT, int GT>
constexpr int score_threads() { return EXACT || GT == 0 || GT >= 8 ? ST : SCT; }

template <int FMT, bool KT, int GT, bool EXACT>
__global__ __launch_bounds__((score_threads<EXACT, GT>())) void score_kernel(TopkArgs a) {
  constexpr int NT = score_threads<EXACT, GT>();
  constexpr int CB = EXACT ? CB_EXACT : CB_CRIT;
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int t = blockIdx.x * NT + tid;
  const int64_t pi = pair_index(a, b, g);
  extern __shared__ double sq[];    // q as fp64, [head][channel slot], G x nch (sized at launch)
  __shared__ int sch[D];
  __shared__ uint32_t sh[CBINS];
  __shared__ uint32_t smeta[grouped(FMT) ? (NT / GS) * D : 1];   // (scale | zero << 16) per channel
  const int G = a.G;
  const kvc_cache& c = a.c;
  const int nch = a.mode == KVC_SCORE_CRITICAL ? a.n_crit : (a.mode == KVC_SCORE_EXACT ? D : 0);
  for (int e = tid; e < nch; e += NT)
    sch[e] = a.mode == KVC_SCORE_CRITICAL ? a.channels[pi * D + e] : e;
  for (int e = tid; e < CBINS; e += NT) sh[e] = 0u;
  if (grouped(FMT) && nch > 0) {   // K metadata of the block's groups, channel pairs a thread
    const int groups = c.max_tokens / GS;
    const int gq = blockIdx.x * (NT / GS) + tid / 64, j = tid % 64;
    uint32_t s2 = 0u, z2 = 0u;
    if (gq < groups) {
      const uint32_t* km = reinterpret_cast<const uint32_t*>(c.k_meta + (pi * groups + gq) * 2 * D);
      s2 = km[j];
      z2 = km[D / 2 + j];
    }
    uint32_t m0 = (s2 & 0xFFFFu) | (z2 << 16), m1 = (s2 >> 16) | (z2 & 0xFFFF0000u);
    // outlier channels (INT4): the word names the outlier store entry instead
    // (a zero-point field of all ones is a NaN no quantized group stores)
    for (int e = 0; e < c.n_outlier; ++e) {
      const int oc = c.outlier_ch[g * KVC_MAX_OUTLIERS + e];
      if (oc == 2 * j) m0 = OUT_TAG | e;
      if (oc == 2 * j + 1) m1 = OUT_TAG | e;
    }
    smeta[(tid / 64) * D + 2 * j] = m0;
    smeta[(tid / 64) * D + 2 * j + 1] = m1;
  }
  // q on the channel list: gathered by prep (critical mode) or channel k itself
  for (int e = tid; e < G * nch; e += NT) {
    const int hh = e / nch, k = e % nch;
    sq[hh * nch + k] = a.mode == KVC_SCORE_CRITICAL
                         ? a.qsel[(pi * GMAX + hh) * D + k]
                         : (double)h2f(a.q[((int64_t)b * a.hq + g * G + hh) * D + k]);
  }
  __syncthreads();

  int lo, hi, kk;
  cand_range(a, b, lo, hi, kk);
  if (a.blocks) {   // every token of the candidate blocks
    lo *= GS;
    hi *= GS;
  }
  const int n = max(c.seq_lens[b], 0);
  const bool in = t < c.max_tokens;
  uint64_t key = 0;
  if (in && t >= lo && t < hi) {
    double r;
    if (a.mode == KVC_SCORE_EXTERNAL) {
      r = (double)a.ext[pi * c.max_tokens + t];
    } else {
      const int nq = grouped(FMT) ? (n & ~(GS - 1)) : n;
      const int64_t slot = slot_of(c, b, g, t);
      r = -INFINITY;
      if (slot >= 0) {
        const int64_t bg = (int64_t)b * c.num_kv_heads + g;
        if (FMT == KVC_FMT_FP16) {
          auto load = [&](int ch) -> uint32_t {
            if (KT) return c.kT[(bg * D + ch) * c.max_tokens + t];
            return c.k16[slot * D + ch];
          };
          auto aux = [&](int) -> uint32_t { return 0u; };
          auto value = [&](int, uint32_t raw, uint32_t) { return (double)h2f((uint16_t)raw); };
          r = token_score<GT, CB, EXACT && FMT != KVC_FMT_INT1>(G, nch, sch, sq, load, aux, value);
        } else if (FMT == KVC_FMT_FP8) {   // E4M3 row, decoded exactly
          const uint8_t* row = c.k_codes + slot * D;
          auto load = [&](int ch) -> uint32_t { return row[ch]; };
          auto aux = [&](int) -> uint32_t { return 0u; };
          auto value = [&](int, uint32_t raw, uint32_t) {
            return (double)h2f((uint16_t)fp8_h16_over256(raw)) * 256.0;
          };
          r = token_score<GT, CB, EXACT>(G, nch, sch, sq, load, aux, value);
        } else if (t >= nq) {   // fp16 tail row of a quantized cache
          const uint16_t* row = c.k_tail + (bg * GS + (t - nq)) * D;
          auto load = [&](int ch) -> uint32_t { return row[ch]; };
          auto aux = [&](int) -> uint32_t { return 0u; };
          auto value = [&](int, uint32_t raw, uint32_t) { return (double)h2f((uint16_t)raw); };
          r = token_score<GT, CB, EXACT && FMT != KVC_FMT_INT1>(G, nch, sch, sq, load, aux, value);
        } else {
          const uint32_t* meta = smeta + (tid / GS) * D;
          const int n16 = FMT == KVC_FMT_INT4 ? (int)(slot % TILE) : (int)(slot % GS) % 16;
          const uint32_t* unit = reinterpret_cast<const uint32_t*>(
              c.k_codes + (FMT == KVC_FMT_INT4 ? slot / TILE : slot / GS) * UNIT_BYTES);
          const int dsel = FMT == KVC_FMT_INT4 ? 0 : (int)(slot % GS) / 16;
          auto load = [&](int ch) -> uint32_t {
            const int lane = 16 * (ch / 32) + n16;
            return unit[lane * 4 + (FMT == KVC_FMT_INT4 ? (ch % 32) / 8 : dsel)];
          };
          auto aux = [&](int ch) -> uint32_t { return meta[ch]; };
          const bool has_out = FMT == KVC_FMT_INT4 && c.n_outlier > 0;
          auto value = [&](int ch, uint32_t raw, uint32_t m) {
            if (has_out && (m & 0xFFFF0000u) == OUT_TAG)   // fp16 outlier store entry
              return (double)h2f(c.k_outlier[slot * KVC_MAX_OUTLIERS + (m & 3u)]);
            const uint32_t code = FMT == KVC_FMT_INT4 ? (raw >> nib_pos(ch % 8)) & 15u
                                                      : (raw >> bit_pos(ch % 32)) & 1u;
            return __dadd_rn(__dmul_rn((double)code, (double)h2f((uint16_t)(m & 0xFFFFu))),
                             (double)h2f((uint16_t)(m >> 16)));
          };
          r = token_score<GT, CB, EXACT && FMT != KVC_FMT_INT1>(G, nch, sch, sq, load, aux, value);
        }
      }
    }
    r = __dadd_rn(r, 0.0);
    if (a.blocks) {
      a.tscore[pi * c.max_tokens + t] = r;
    } else {
      key = order_key(r);
      if (a.out_scores) a.out_scores[pi * c.max_tokens + t] = r;
    }
  }
  if (in) a.keys[pi * c.max_tokens + t] = key;
  if (key) atomicAdd(&sh[coarse_of(key)], 1u);
  __syncthreads();
  uint32_t* h = a.hist + pi * HW + (blockIdx.x % HREP) * CBINS;
  for (int e = tid; e < CBINS; e += NT)
    if (sh[e]) atomicAdd(&h[e], sh[e]);
}

// ------------------------------------------------------------------ block keys
// Block mode: 64 candidate blocks a workgroup.  Their 64 x 64 token scores are
// staged in LDS with coalesced loads, then thread j adds block j's scores one
// at a time in ascending token order from +0.0, divides by 64 (exact), and
// writes the block's key and its coarse histogram entry.  Items that are not
// candidates keep the zero key the score kernel wrote.
constexpr int BPW = 64;
__global__ __launch_bounds__(ST) void block_key_kernel(TopkArgs a) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  __shared__ double ss[BPW * GS];
  __shared__ uint32_t sh[CBINS];
  int lo, hi, kk;
  cand_range(a, b, lo, hi, kk);
  const int j0 = blockIdx.x * BPW;
  const double* ts = a.tscore + pi * a.c.max_tokens;
  for (int e = tid; e < CBINS; e += ST) sh[e] = 0u;
  for (int e = tid; e < BPW * GS; e += ST) {
    const int j = j0 + e / GS;
    ss[e] = j >= lo && j < hi ? ts[(int64_t)j0 * GS + e] : 0.0;
  }
  __syncthreads();
  if (tid < BPW) {
    const int j = j0 + tid;
    if (j >= lo && j < hi) {
      double sum = 0.0;
      for (int i = 0; i < GS; ++i) sum = __dadd_rn(sum, ss[tid * GS + i]);
      const double r = __dadd_rn(__ddiv_rn(sum, (double)GS), 0.0);
      const uint64_t key = order_key(r);
      a.keys[pi * a.c.max_tokens + j] = key;
      if (a.out_scores) a.out_scores[pi * a.c.max_tokens + j] = r;
      atomicAdd(&sh[coarse_of(key)], 1u);
    }
  }
  __syncthreads();
  uint32_t* h = a.hist + pi * HW + (blockIdx.x % HREP) * CBINS;
  for (int e = tid; e < CBINS; e += ST)
    if (sh[e]) atomicAdd(&h[e], sh[e]);
}

// ------------------------------------------------------------------ selection helpers
// Inclusive scan of x over the NT threads of the workgroup (wave scans, then
// the wave totals through s_wsum[NT / 64]); *total receives the sum.
template <int NT>
__device__ inline uint32_t block_scan(uint32_t x, uint32_t* s_wsum, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wsum[wv] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const uint32_t v = s_wsum[k];
    before += k < wv ? v : 0u;
    all += v;
  }
  __syncthreads();
  *total = all;
  return before + x;
}

// The coarse bin tb holding the k-th largest key of the pair (1 <= k <= keys
// counted) and n_gt, the keys in the bins above it, from the pair's histogram
// copies: thread t sums bins [CBINS - BPT (t + 1), CBINS - BPT t) (the highest
// bins first), a scan gives the keys above each thread's bins, and the thread
// whose bins the k-th key falls in walks them.  Results in s_res[0] (tb) and
// s_res[1] (n_gt).
template <int NT>
__device__ void coarse_threshold(const uint32_t* hist, int k, int* s_res, uint32_t* s_wsum) {
  constexpr int BPT = CBINS / NT;
  static_assert(BPT % 4 == 0, "bins a thread reads as 16-byte words");
  const int top = CBINS - BPT * (int)threadIdx.x;   // bins [top - BPT, top)
  uint32_t cnt[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) cnt[i] = 0u;
#pragma unroll
  for (int r = 0; r < HREP; ++r) {
#pragma unroll
    for (int v = 0; v < BPT / 4; ++v) {
      const uint4 w = *reinterpret_cast<const uint4*>(hist + r * CBINS + top - BPT + 4 * v);
      cnt[4 * v] += w.x;
      cnt[4 * v + 1] += w.y;
      cnt[4 * v + 2] += w.z;
      cnt[4 * v + 3] += w.w;
    }
  }
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) sum += cnt[i];
  if (threadIdx.x == 0) {   // (k is at most the keys counted, so some thread overwrites these)
    s_res[0] = 0;
    s_res[1] = 0;
  }
  uint32_t total;
  uint32_t run = block_scan<NT>(sum, s_wsum, &total) - sum;   // keys in the bins above
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {   // bin top - BPT + i, highest first
    if (run < (uint32_t)k && run + cnt[i] >= (uint32_t)k) {
      s_res[0] = top - BPT + i;
      s_res[1] = (int)run;
    }
    run += cnt[i];
  }
  __syncthreads();
}

// ------------------------------------------------------------------ compact
// Long candidate ranges: CT items a workgroup (ST threads, CT / ST rounds).
// Bits of the items whose coarse bin is above tb go to the `above` bitmap
// (every word of the pair is written by some workgroup); the items of bin tb
// go, in index order, to this workgroup's region of ckey / cidx, with their
// count in ccount.
__global__ __launch_bounds__(ST) void compact_kernel(TopkArgs a) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t pi = pair_index(a, b, g);
  constexpr int R = CT / ST;   // rounds
  __shared__ int s_res[2];
  __shared__ uint32_t s_wsum[ST / 64];
  __shared__ uint32_t s_cnt[R * (ST / 64)];
  __shared__ uint32_t s_off[R * (ST / 64)];
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  if (k <= 0) return;   // (finish writes the -1 padding)
  coarse_threshold<ST>(a.hist + pi * HW, k, s_res, s_wsum);
  const uint32_t tb = (uint32_t)s_res[0];
  const int N = item_count(a.c, a.blocks);
  const int nwords = (N + 31) / 32;
  const uint64_t* keys = a.keys + pi * a.c.max_tokens;
  const int base = blockIdx.x * CT;
  uint64_t kv[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = base + j * ST + tid;
    kv[j] = i < N ? keys[i] : 0ull;
  }
  uint64_t cand[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint32_t cb = coarse_of(kv[j]);
    const uint64_t ab = __ballot(kv[j] != 0 && cb > tb);
    cand[j] = __ballot(kv[j] != 0 && cb == tb);
    const int wd = (base + j * ST + wv * 64) / 32;   // the wave's first word
    uint32_t* aw = a.above + pi * (a.c.max_tokens / 32);
    if (lane == 0 && wd < nwords) aw[wd] = (uint32_t)ab;
    if (lane == 32 && wd + 1 < nwords) aw[wd + 1] = (uint32_t)(ab >> 32);
    if (lane == 0) s_cnt[j * (ST / 64) + wv] = (uint32_t)__popcll(cand[j]);
  }
  __syncthreads();
  if (tid < 64) {   // exclusive scan over the R * 4 (round, wave) counts, in index order
    uint32_t x = tid < R * (ST / 64) ? s_cnt[tid] : 0u;
    const uint32_t own = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (tid < R * (ST / 64)) s_off[tid] = x - own;
    if (tid == R * (ST / 64) - 1) a.ccount[pi * a.nreg + blockIdx.x] = (int32_t)x;
  }
  __syncthreads();
  const int64_t reg = (pi * a.nreg + blockIdx.x) * (int64_t)CT;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if ((cand[j] >> lane) & 1ull) {
      const uint32_t pos = s_off[j * (ST / 64) + wv] + (uint32_t)__popcll(cand[j] & below);
      a.ckey[reg + pos] = kv[j];
      a.cidx[reg + pos] = base + j * ST + tid;
    }
  }
}

// ------------------------------------------------------------------ finish
// One workgroup (FT threads) per (sequence, KV head).  The k best items are
// those in coarse bins above tb plus the krem = k - n_gt best of bin tb; the
// latter are found by an exact radix select among bin tb's keys (8-bit digits
// from the first bit where those keys differ, LDS histograms; once a digit's
// bucket is taken whole the rest of it is selected by prefix), lower index
// first among keys equal to the threshold.  Bin tb's items come from the
// compaction regions (into LDS, up to CAP of them) or, for short ranges or a
// bin too large for LDS, straight from the key row (staged in LDS when it has
// at most DIRECT_MAX items).  Output: the selected items in ascending order,
// then -1.
struct FinishLds {
  uint64_t key[CAP];        // bin-tb keys (region path) or the key row (direct path)
  int32_t idx[CAP];         // their items (region path)
  uint32_t bm[EW];          // bitmap chunk (region path)
  uint8_t sel[CAP];         // selected flags of bin-tb items (region path)
  int32_t roff[MAXR + 1];   // region offsets (region path)
  uint32_t bins[256];
  uint32_t wsum[FT / 64];
  uint64_t red[2 * (FT / 64)];
  int res[4];
  uint64_t pfx;
};

__device__ inline void select_digit(FinishLds& L, uint64_t prefix, int krem, uint64_t* new_prefix,
                                    int* new_krem, int* bucket) {
  // suffix sums over the 256 bins: thread d < 256 holds bin 255 - d
  const int tid = threadIdx.x;
  uint32_t x = tid < 256 ? L.bins[255 - tid] : 0u;
  if (tid == 0) {   // (krem is at most the keys counted, so some thread overwrites these)
    L.pfx = prefix << 8;
    L.res[2] = krem;
    L.res[3] = 0;
  }
  uint32_t total;
  const uint32_t incl = block_scan<FT>(x, L.wsum, &total);   // keys in bins >= 255 - tid
  if (tid < 256) {
    const uint32_t ge = incl, gt = incl - x;
    if (ge >= (uint32_t)krem && gt < (uint32_t)krem) {
      L.pfx = (prefix << 8) | (uint64_t)(255 - tid);
      L.res[2] = krem - (int)gt;
      L.res[3] = (int)x;
    }
  }
  __syncthreads();
  *new_prefix = L.pfx;
  *new_krem = L.res[2];
  *bucket = L.res[3];
  __syncthreads();
}

__global__ __launch_bounds__(FT) void finish_kernel(TopkArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t pi = pair_index(a, b, g);
  __shared__ FinishLds L;
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  int32_t* out = a.out_idx + pi * a.k_max;
  if (k <= 0) {
    for (int e = tid; e < a.k_max; e += FT) out[e] = -1;
    return;
  }
  coarse_threshold<FT>(a.hist + pi * HW, k, L.res, L.wsum);
  const uint32_t tb = (uint32_t)L.res[0];
  const int krem0 = k - L.res[1];
  const int N = item_count(a.c, a.blocks);
  const uint64_t* gkeys = a.keys + pi * a.c.max_tokens;
  const uint64_t below = (1ull << lane) - 1ull;

  // ---- where bin tb's items are
  const bool direct = N <= DIRECT_MAX;
  int C = 0;            // region path: bin-tb items in LDS
  bool regions = false;
  if (direct) {
    for (int i = tid; i < N; i += FT) L.key[i] = gkeys[i];
    __syncthreads();
  } else if (a.nreg <= MAXR) {
    uint32_t run = 0;
    for (int r0 = 0; r0 < a.nreg; r0 += FT) {
      const int r = r0 + tid;
      const uint32_t c = r < a.nreg ? (uint32_t)a.ccount[pi * a.nreg + r] : 0u;
      uint32_t tot;
      const uint32_t incl = block_scan<FT>(c, L.wsum, &tot);
      if (r < a.nreg) L.roff[r] = (int32_t)(run + incl - c);
      run += tot;
    }
    C = (int)run;
    if (tid == 0) L.roff[a.nreg] = C;
    regions = C <= CAP;
    __syncthreads();
    if (regions) {
      for (int e = tid; e < C; e += FT) {   // region of entry e: last r with roff[r] <= e
        int rl = 0, rh = a.nreg - 1;
        while (rl < rh) {
          const int m = (rl + rh + 1) >> 1;
          if (L.roff[m] <= e) rl = m; else rh = m - 1;
        }
        const int64_t src = (pi * a.nreg + rl) * (int64_t)CT + (e - L.roff[rl]);
        L.key[e] = a.ckey[src];
        L.idx[e] = a.cidx[src];
      }
      __syncthreads();
    }
  }
  // bin-tb keys, in index order: f(key, position) for each
  auto key_row = [&](int i) -> uint64_t { return direct ? L.key[i] : gkeys[i]; };
  auto for_cand = [&](auto&& f) {
    if (regions) {
      for (int e = tid; e < C; e += FT) f(L.key[e]);
    } else {
      for (int i = tid; i < N; i += FT) {
        const uint64_t key = key_row(i);
        if (key && coarse_of(key) == tb) f(key);
      }
    }
  };

  // ---- common prefix of bin tb's keys: the digits before the first
  // differing bit need no pass
  uint64_t kand = ~0ull, kor = 0ull;
  for_cand([&](uint64_t key) {
    kand &= key;
    kor |= key;
  });
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kand &= __shfl_xor(kand, o);
    kor |= __shfl_xor(kor, o);
  }
  if (lane == 0) {
    L.red[wv] = kand;
    L.red[FT / 64 + wv] = kor;
  }
  __syncthreads();
  kand = ~0ull;
  kor = 0ull;
#pragma unroll
  for (int w2 = 0; w2 < FT / 64; ++w2) {
    kand &= L.red[w2];
    kor |= L.red[FT / 64 + w2];
  }
  const uint64_t diff = kand ^ kor;   // bits where bin tb's keys differ
  const int first = diff ? __clzll(diff) / 8 : 8;   // first digit with a difference

  // ---- radix passes
  uint64_t P = first > 0 ? (kand >> (64 - 8 * first)) : 0ull;   // the chosen top 8p bits
  int krem = krem0, bits = 0;   // bits > 0: the bucket of those top bits is taken whole
  for (int p = first; p < 8; ++p) {
    if (tid < 256) L.bins[tid] = 0u;
    __syncthreads();
    const int sh = 56 - 8 * p;
    for_cand([&](uint64_t key) {
      if (p == 0 || (key >> (sh + 8)) == P) atomicAdd(&L.bins[(key >> sh) & 255u], 1u);
    });
    __syncthreads();
    int bucket;
    select_digit(L, P, krem, &P, &krem, &bucket);
    if (bucket == krem) {
      bits = 8 * (p + 1);
      break;
    }
  }
  // selected among bin tb: top `bits` bits >= P (a bucket taken whole), or,
  // after all digits, key > T = P, or key == T for the first krem by index
  const uint64_t T = P;
  auto chosen = [&](uint64_t key, bool eq_ok) {
    return bits ? (key >> (64 - bits)) >= P : (key > T || (key == T && eq_ok));
  };

  int written = 0;
  if (regions) {
    // ranks of the keys equal to T: thread t owns entries [t per, (t + 1) per)
    const int per = (C + FT - 1) / FT;
    const int e0 = min(tid * per, C), e1 = min(e0 + per, C);
    uint32_t neq = 0;
    for (int e = e0; e < e1; ++e) neq += (!bits && L.key[e] == T) ? 1u : 0u;
    uint32_t tot;
    uint32_t rank = block_scan<FT>(neq, L.wsum, &tot) - neq;
    for (int e = e0; e < e1; ++e) {
      const bool eq = !bits && L.key[e] == T;
      L.sel[e] = chosen(L.key[e], eq && rank < (uint32_t)krem) ? 1 : 0;
      rank += eq ? 1u : 0u;
    }
    __syncthreads();
    // emission: the above bitmap chunk by chunk with the chosen bin-tb items
    // OR'ed in, then each thread's EW / FT words in order
    const int nwords = (N + 31) / 32;
    const uint32_t* aw = a.above + pi * (a.c.max_tokens / 32);
    constexpr int WPT = EW / FT;
    for (int w0 = 0; w0 < nwords; w0 += EW) {
      const int nw = min(EW, nwords - w0);
      for (int x = tid; x < EW; x += FT) L.bm[x] = x < nw ? aw[w0 + x] : 0u;
      __syncthreads();
      for (int e = tid; e < C; e += FT) {
        const int it = L.idx[e];
        if (L.sel[e] && it >= 32 * w0 && it < 32 * (w0 + nw))
          atomicOr(&L.bm[(it >> 5) - w0], 1u << (it & 31));
      }
      __syncthreads();
      uint32_t wds[WPT];
      uint32_t cnt = 0;
#pragma unroll
      for (int x = 0; x < WPT; ++x) {
        wds[x] = L.bm[tid * WPT + x];
        cnt += (uint32_t)__popc(wds[x]);
      }
      uint32_t tot2;
      int pos = written + (int)(block_scan<FT>(cnt, L.wsum, &tot2) - cnt);
#pragma unroll
      for (int x = 0; x < WPT; ++x) {
        uint32_t m = wds[x];
        while (m) {
          const int j = __ffs(m) - 1;
          m &= m - 1u;
          if (pos < a.k_max) out[pos] = 32 * (w0 + tid * WPT + x) + j;
          ++pos;
        }
      }
      written += (int)tot2;
      __syncthreads();
    }
  } else {
    // emission straight from the key row, FT items a round in index order
    uint32_t eq_taken = 0;
    for (int c0 = 0; c0 < N; c0 += FT) {
      const int i = c0 + tid;
      const uint64_t key = i < N ? key_row(i) : 0ull;
      const uint32_t cb = coarse_of(key);
      const bool above = key != 0 && cb > tb;
      const bool inb = key != 0 && cb == tb;
      const bool eq = inb && !bits && key == T;
      uint32_t eq_tot;
      const uint32_t eq_incl = block_scan<FT>(eq ? 1u : 0u, L.wsum, &eq_tot);
      const bool take = above || (inb && chosen(key, eq_taken + eq_incl - 1u < (uint32_t)krem));
      uint32_t take_tot;
      const uint32_t take_incl = block_scan<FT>(take ? 1u : 0u, L.wsum, &take_tot);
      const int pos = written + (int)take_incl - 1;
      if (take && pos < a.k_max) out[pos] = i;
      written += (int)take_tot;
      eq_taken += eq_tot;
    }
  }
  for (int e = written + tid; e < a.k_max; e += FT) out[e] = -1;
}

}  // namespace

size_t topk_workspace_bytes(const kvc_cache& c) {
  const size_t pairs = (size_t)c.batch * c.num_kv_heads;
  const size_t words = c.max_tokens / 32;
  const size_t nreg = (c.max_tokens + CT - 1) / CT;   // (token items: the most regions)
  size_t bytes = 2 * pairs * c.max_tokens * sizeof(uint64_t);   // keys, block-mode token scores
  bytes += pairs * GMAX * D * sizeof(double);                    // critical-mode q operands
  bytes += pairs * HW * sizeof(uint32_t);                        // coarse histogram
  bytes += pairs * words * sizeof(uint32_t);                     // above bitmap
  bytes += pairs * nreg * CT * (sizeof(uint64_t) + sizeof(int32_t));   // bin-tb regions
  bytes += pairs * nreg * sizeof(int32_t);                       // region counts
  bytes += pairs * D * sizeof(int32_t);                          // channel lists
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
  a.blocks = (mode & KVC_SCORE_BLOCKS) != 0;
  mode &= ~KVC_SCORE_BLOCKS;
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
  const int items = item_count(c, a.blocks);
  const size_t nreg_ws = (c.max_tokens + CT - 1) / CT;
  a.nreg = (items + CT - 1) / CT;
  char* p = static_cast<char*>(ws);
  a.keys = reinterpret_cast<uint64_t*>(p);
  p += pairs * c.max_tokens * sizeof(uint64_t);
  a.tscore = reinterpret_cast<double*>(p);
  p += pairs * c.max_tokens * sizeof(double);
  a.qsel = reinterpret_cast<double*>(p);
  p += pairs * GMAX * D * sizeof(double);
  a.hist = reinterpret_cast<uint32_t*>(p);
  p += pairs * HW * sizeof(uint32_t);
  a.above = reinterpret_cast<uint32_t*>(p);
  p += pairs * words * sizeof(uint32_t);
  a.ckey = reinterpret_cast<uint64_t*>(p);
  p += pairs * nreg_ws * CT * sizeof(uint64_t);
  a.cidx = reinterpret_cast<int32_t*>(p);
  p += pairs * nreg_ws * CT * sizeof(int32_t);
  a.ccount = reinterpret_cast<int32_t*>(p);
  p += pairs * nreg_ws * sizeof(int32_t);
  a.channels = reinterpret_cast<int32_t*>(p);

  const int Hkv = c.num_kv_heads, B = c.batch;
  prep_kernel<<<dim3(Hkv, B), D, 0, s>>>(a);
  const bool exact = mode == KVC_SCORE_EXACT;
  const int snt = exact || (a.G != 1 && a.G != 2 && a.G != 4) ? ST : SCT;
  const dim3 sgrid((c.max_tokens + snt - 1) / snt, Hkv, B);
  // the scorer's q operands in LDS: G heads x the channels it sums over
  const int nch = mode == KVC_SCORE_CRITICAL ? n_crit : (exact ? D : 0);
  const size_t sq_bytes = (size_t)std::max(1, a.G * nch) * sizeof(double);
#define KVC_SCORE_E(F, KT, GG)                                                \
  do {                                                                        \
    if (exact) score_kernel<F, KT, GG, true><<<sgrid, snt, sq_bytes, s>>>(a); \
    else score_kernel<F, KT, GG, false><<<sgrid, snt, sq_bytes, s>>>(a);      \
  } while (0)
#define KVC_SCORE_G(F, KT)                                                    \
  do {                                                                        \
    switch (a.G) {                                                            \
      case 1: KVC_SCORE_E(F, KT, 1); break;                                   \
      case 2: KVC_SCORE_E(F, KT, 2); break;                                   \
      case 4: KVC_SCORE_E(F, KT, 4); break;                                   \
      case 8: KVC_SCORE_E(F, KT, 8); break;                                   \
      default: KVC_SCORE_E(F, KT, 0); break;                                  \
    }                                                                         \
  } while (0)
  if (c.format == KVC_FMT_INT4) KVC_SCORE_G(KVC_FMT_INT4, false);
  else if (c.format == KVC_FMT_INT1) KVC_SCORE_G(KVC_FMT_INT1, false);
  else if (c.kT && c.page_size == 0) KVC_SCORE_G(KVC_FMT_FP16, true);   // (FP8: kT holds decoded values)
  else if (c.format == KVC_FMT_FP8) KVC_SCORE_G(KVC_FMT_FP8, false);
  else KVC_SCORE_G(KVC_FMT_FP16, false);
#undef KVC_SCORE_G
#undef KVC_SCORE_E
  if (a.blocks)
    block_key_kernel<<<dim3((c.max_tokens / GS + BPW - 1) / BPW, Hkv, B), ST, 0, s>>>(a);
  if (items > DIRECT_MAX) compact_kernel<<<dim3(a.nreg, Hkv, B), ST, 0, s>>>(a);
  finish_kernel<<<dim3(Hkv, B), FT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvc
