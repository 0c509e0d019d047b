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
//           bytes chosen so far; each pass derives the byte of the previous
//           pass from its histogram and the stored state of the pass before.
//   mark    bitmaps of keys above the k-th largest key T and equal to T.
//   emit    one workgroup per (sequence, KV head): the first k - #above keys
//           equal to T by index, then every selected index in ascending order.
// Block mode (meeting-LLM article, section 8.1: importance averaged over
// 64-token blocks, the top blocks kept): score writes each token's fp64 score
// and no key; block_key averages every candidate block's 64 scores into the
// block's key (item j of the pair's key row) and histograms it; the passes
// above then select blocks instead of tokens.

#include <math.h>

#include "internal.h"

namespace kvc {
namespace {

constexpr int ST = 256;        // threads of the scoring / radix workgroups
constexpr int TPB = 1024;      // tokens per radix / mark workgroup
constexpr int ET = 1024;       // threads of the emit workgroup
constexpr int PASSES = 8;
constexpr int HREP = 8;        // copies of each histogram (spread the global atomics)
constexpr int HSTRIDE = PASSES * HREP * 256;   // histogram words per (sequence, KV head)

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
  uint32_t* hist;      // [B][Hkv][PASSES][HREP][256]
  uint32_t* above;     // [B][Hkv][max_tokens / 32]
  uint32_t* equal;     // [B][Hkv][max_tokens / 32]
  int32_t* channels;   // [B][Hkv][128]
  uint64_t* prefix;    // [B][Hkv][PASSES] slot s: key prefix of the s + 1 bytes chosen by pass s
  int32_t* krem;       // [B][Hkv][PASSES] slot s: keys still to take from pass s's bucket
  int32_t* done;       // [B][Hkv] 0, or 8p once pass p found its bucket taken whole
  int hist_words;      // histogram words per pair that prep clears (all passes, or pass 0 only)
  double* qsel;        // critical mode: [B][Hkv][GMAX][128] q of the group's heads on the
                       // channel list (slot k = k-th critical channel), fp64
  bool blocks;         // rank 64-token blocks (items = block ids)
  double* tscore;      // block mode: [B][Hkv][max_tokens] token scores
};

__device__ inline uint64_t order_key(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
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
  uint4* h = reinterpret_cast<uint4*>(a.hist + pi * HSTRIDE);
  for (int e = c; e < a.hist_words / 4; e += D) h[e] = uint4{0u, 0u, 0u, 0u};
  if (c == 0) a.done[pi] = 0;
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
#pragma unroll
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
// group), an order-preserving key, and the histogram of the key's top byte.
template <int FMT, bool KT, int GT, bool EXACT>
__global__ __launch_bounds__(ST) void score_kernel(TopkArgs a) {
  constexpr int CB = EXACT ? CB_EXACT : CB_CRIT;
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int t = blockIdx.x * ST + tid;
  const int64_t pi = pair_index(a, b, g);
  extern __shared__ double sq[];    // q as fp64, [head][channel slot], G x nch (sized at launch)
  __shared__ int sch[D];
  __shared__ uint32_t sh[256];
  __shared__ uint32_t smeta[grouped(FMT) ? (ST / GS) * D : 1];   // (scale | zero << 16) per channel
  const int G = a.G;
  const kvc_cache& c = a.c;
  const int nch = a.mode == KVC_SCORE_CRITICAL ? a.n_crit : (a.mode == KVC_SCORE_EXACT ? D : 0);
  for (int e = tid; e < nch; e += ST)
    sch[e] = a.mode == KVC_SCORE_CRITICAL ? a.channels[pi * D + e] : e;
  sh[tid] = 0u;
  if (grouped(FMT) && nch > 0) {   // K metadata of the block's groups, channel pairs a thread
    const int groups = c.max_tokens / GS;
    const int gq = blockIdx.x * (ST / GS) + tid / 64, j = tid % 64;
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
  for (int e = tid; e < G * nch; e += ST) {
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
  if (key) atomicAdd(&sh[key >> 56], 1u);
  __syncthreads();
  if (sh[tid]) atomicAdd(&a.hist[pi * HSTRIDE + (blockIdx.x % HREP) * 256 + tid], sh[tid]);
}

// ------------------------------------------------------------------ block keys
// Block mode: 64 candidate blocks a workgroup.  Their 64 x 64 token scores are
// staged in LDS with coalesced loads, then thread j adds block j's scores one
// at a time in ascending token order from +0.0, divides by 64 (exact), and
// writes the block's key and its pass-0 histogram entry.  Items that are not
// candidates keep the zero key the score kernel wrote.
constexpr int BPW = 64;
__global__ __launch_bounds__(ST) void block_key_kernel(TopkArgs a) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  __shared__ double ss[BPW * GS];
  __shared__ uint32_t sh[256];
  int lo, hi, kk;
  cand_range(a, b, lo, hi, kk);
  const int j0 = blockIdx.x * BPW;
  const double* ts = a.tscore + pi * a.c.max_tokens;
  sh[tid] = 0u;
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
      atomicAdd(&sh[key >> 56], 1u);
    }
  }
  __syncthreads();
  if (sh[tid]) atomicAdd(&a.hist[pi * HSTRIDE + (blockIdx.x % HREP) * 256 + tid], sh[tid]);
}

// ------------------------------------------------------------------ radix passes
// One selection step (256 threads; hist_pp holds HREP copies of the pass's
// histogram; s_krem[1] receives the chosen bucket's size): given the prefix of the bytes chosen so far
// and the number of keys still to take, pick the byte d of pass pp whose
// bucket holds the krem-th largest key (suffix count of buckets >= d reaches
// krem, of buckets > d does not).  Results through LDS.
__device__ void select_byte(const uint32_t* hist_pp, uint64_t prefix, int krem, uint64_t* s_prefix,
                            int* s_krem, uint32_t* s_scan) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // suffix sum over bins: inclusive scan of the reversed histogram (copies summed)
  uint32_t x = 0;
#pragma unroll
  for (int r = 0; r < HREP; ++r) x += hist_pp[r * 256 + 255 - tid];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_scan[256 + wv] = x;
  __syncthreads();
  for (int k = 0; k < wv; ++k) x += s_scan[256 + k];
  s_scan[255 - tid] = x;   // s_scan[d] = keys in buckets >= d
  __syncthreads();
  const uint32_t ge = s_scan[tid];
  const uint32_t gt = tid < 255 ? s_scan[tid + 1] : 0u;
  if (ge >= (uint32_t)krem && gt < (uint32_t)krem) {
    s_prefix[0] = (prefix << 8) | (uint64_t)tid;
    s_krem[0] = krem - (int)gt;
    s_krem[1] = (int)(ge - gt);   // keys in the chosen bucket
  }
  __syncthreads();
}

// State after pass p - 1 (prefix of p bytes) for (pair pi): pass 0's comes from
// k alone; later ones from the state the kernel of pass p - 1 stored in slot
// p - 2.  Each pass writes its own slot, so the workgroups of one launch that
// read the previous slot never see a value written in the same launch.
__device__ void state_after(const TopkArgs& a, int64_t pi, int p, int k, uint64_t* s_prefix,
                            int* s_krem, uint32_t* s_scan) {
  const uint32_t* hist = a.hist + pi * HSTRIDE;
  const uint64_t prefix = p == 1 ? 0ull : a.prefix[pi * PASSES + p - 2];
  const int krem = p == 1 ? k : a.krem[pi * PASSES + p - 2];
  select_byte(hist + (p - 1) * HREP * 256, prefix, krem, s_prefix, s_krem, s_scan);
}

__global__ __launch_bounds__(ST) void radix_kernel(TopkArgs a, int p) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  __shared__ uint64_t s_prefix[1];
  __shared__ int s_krem[2];
  __shared__ uint32_t s_scan[256 + 4];
  __shared__ uint32_t sh[256];
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  if (k <= 0 || a.done[pi]) return;
  // this workgroup's keys, loaded while the state is derived
  constexpr int KPT = TPB / ST;
  const int t0 = blockIdx.x * TPB;
  const uint64_t* keys = a.keys + pi * a.c.max_tokens;
  uint64_t kv[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int t = t0 + tid + i * ST;
    kv[i] = t < a.c.max_tokens ? keys[t] : 0ull;
  }
  sh[tid] = 0u;
  state_after(a, pi, p, k, s_prefix, s_krem, s_scan);
  const uint64_t prefix = s_prefix[0];
  const bool whole = s_krem[1] == s_krem[0];   // every key of the bucket is taken: done
  if (blockIdx.x == 0 && tid == 0) {   // every workgroup derived the same state
    a.prefix[pi * PASSES + p - 1] = prefix;
    a.krem[pi * PASSES + p - 1] = s_krem[0];
    if (whole) a.done[pi] = 8 * p;
  }
  if (whole) return;
  const int shift = 64 - 8 * p;   // bits above the current byte
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (kv[i] && (kv[i] >> shift) == prefix) atomicAdd(&sh[(kv[i] >> (shift - 8)) & 255u], 1u);
  __syncthreads();
  if (sh[tid]) atomicAdd(&a.hist[pi * HSTRIDE + (p * HREP + blockIdx.x % HREP) * 256 + tid], sh[tid]);
}

// ------------------------------------------------------------------ mark
// One thread per key; a wave's ballots are two 32-token words of each bitmap.
__global__ __launch_bounds__(ST) void mark_kernel(TopkArgs a) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, lane = tid & 63;
  const int64_t pi = pair_index(a, b, g);
  __shared__ uint64_t s_prefix[1];
  __shared__ int s_krem[2];
  __shared__ uint32_t s_scan[256 + 4];
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  // keys of this workgroup, loaded while the threshold is derived
  constexpr int KPT = TPB / ST;
  const uint64_t* keys = a.keys + pi * a.c.max_tokens;
  uint64_t kv[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int t = blockIdx.x * TPB + tid + i * ST;
    kv[i] = t < a.c.max_tokens ? keys[t] : 0ull;
  }
  // selected: key above the k-th largest key T, or equal to it (first ones by
  // index, in emit); when a pass found its bucket taken whole, every key whose
  // top `bits` bits reach the stored prefix
  uint64_t T = ~0ull;     // nothing is above the all-ones key and nothing equals it
  int bits = 0;
  uint64_t P = 0;
  if (k > 0) {
    bits = a.done[pi];
    if (bits) {
      P = a.prefix[pi * PASSES + bits / 8 - 1];   // the prefix of the pass that found it whole
    } else {
      state_after(a, pi, PASSES, k, s_prefix, s_krem, s_scan);
      T = s_prefix[0];
    }
  }
  const int words = a.c.max_tokens / 32;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int t = blockIdx.x * TPB + tid + i * ST;
    if (t >= a.c.max_tokens) break;   // whole waves (max_tokens and TPB are multiples of 64)
    const uint64_t key = kv[i];
    const bool ab_t = bits ? (key >> (64 - bits)) >= P : key > T;
    const uint64_t ab = __ballot(key != 0 && ab_t && k > 0);
    const uint64_t eq = __ballot(key != 0 && !bits && key == T && k > 0);
    const int wd = (t - lane) / 32;   // first of the wave's two words
    if (lane == 0) {
      a.above[pi * words + wd] = (uint32_t)ab;
      a.equal[pi * words + wd] = (uint32_t)eq;
    } else if (lane == 32) {
      a.above[pi * words + wd + 1] = (uint32_t)(ab >> 32);
      a.equal[pi * words + wd + 1] = (uint32_t)(eq >> 32);
    }
  }
}

// ------------------------------------------------------------------ emit
// Exclusive prefix sum over the ET threads (wave scans, then the wave totals).
__device__ inline int block_exclusive_scan(int v, int* s, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s[wv] = x;
  __syncthreads();
  int before = 0;
  total = 0;
  for (int k = 0; k < ET / 64; ++k) {
    const int t = s[k];
    before += k < wv ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

constexpr int EPR = 8;   // bitmap words a thread loads at once
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
  // how many equal keys to take: k - #above.  A thread's words are read
  // EPR at a time with every load issued before any is used; the first EPR
  // (all of them for caches up to 256K tokens) are read once and kept in
  // registers for the three passes below.
  typedef uint32_t Words[EPR];
  auto load_chunk = [&](int base, Words& x, Words& y) {
#pragma unroll
    for (int i = 0; i < EPR; ++i) {
      x[i] = base + i < wb ? ab[base + i] : 0u;
      y[i] = base + i < wb ? eq[base + i] : 0u;
    }
  };
  Words ab0, eq0;
  load_chunk(wa, ab0, eq0);
  auto for_chunks = [&](auto&& f) {
    for (int base = wa; base < wb; base += EPR) {
      if (base == wa) {
        f(base, ab0, eq0);
      } else {
        Words x, y;
        load_chunk(base, x, y);
        f(base, x, y);
      }
    }
  };
  int n_ab = 0, n_eq = 0;
  for_chunks([&](int, Words& abw, Words& eqw) {
#pragma unroll
    for (int i = 0; i < EPR; ++i) {
      n_ab += __popc(abw[i]);
      n_eq += __popc(eqw[i]);
    }
  });
  int tot_ab, tot_eq;
  block_exclusive_scan(n_ab, s, tot_ab);
  const int eq_before = block_exclusive_scan(n_eq, s, tot_eq);
  const int take_eq = max(0, k - tot_ab);
  // selected = above | (first take_eq equal bits by index)
  int n_sel = 0;
  int eq_seen = eq_before;
  for_chunks([&](int, Words& abw, Words& eqw) {
#pragma unroll
    for (int i = 0; i < EPR; ++i) {
      uint32_t e = eqw[i];
      uint32_t keep = 0u;
      while (e && eq_seen < take_eq) {
        const uint32_t bit = e & (0u - e);
        keep |= bit;
        e ^= bit;
        ++eq_seen;
      }
      n_sel += __popc(abw[i] | keep);
    }
  });
  int total;
  int pos = block_exclusive_scan(n_sel, s, total);
  eq_seen = eq_before;
  for_chunks([&](int base, Words& abw, Words& eqw) {
#pragma unroll
    for (int i = 0; i < EPR; ++i) {
      uint32_t e = eqw[i];
      uint32_t keep = 0u;
      while (e && eq_seen < take_eq) {
        const uint32_t bit = e & (0u - e);
        keep |= bit;
        e ^= bit;
        ++eq_seen;
      }
      uint32_t m = abw[i] | keep;
      while (m) {
        const int j = __ffs(m) - 1;
        m &= m - 1;
        if (pos < a.k_max) out[pos] = (base + i) * 32 + j;
        ++pos;
      }
    }
  });
  for (int e = total + tid; e < a.k_max; e += ET) out[e] = -1;
}

// ------------------------------------------------------------------ select (one workgroup per pair)
// After the score kernel, the remaining radix passes, the threshold and the
// ascending output of one (sequence, KV head) in one 1024-thread workgroup:
// the pass-0 histogram is summed from its copies into LDS, the candidates'
// keys are staged in LDS (re-read from L2 each pass if they do not fit), and
// each pass histograms its byte with LDS atomics.  Same passes and tie rule as
// radix / mark / emit above, without their launches; used when a pair's
// candidate range is short.
constexpr int SELT = 1024;
constexpr int SEL_LDS_KEYS = 12288;   // 96 KB of keys in LDS

// Byte of the current pass among 256 LDS bins (threads < 256 scan; every
// thread calls): the bucket holding the krem-th largest key; results through
// s_prefix / s_krem (bucket size in s_krem[1]).
__device__ void select_byte_lds(const uint32_t* bins, uint64_t prefix, int krem, uint64_t* s_prefix,
                                int* s_krem, uint32_t* s_scan) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t x = tid < 256 ? bins[255 - tid] : 0u;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (tid < 256 && lane == 63) s_scan[256 + wv] = x;
  __syncthreads();
  if (tid < 256) {
    for (int k = 0; k < wv; ++k) x += s_scan[256 + k];
    s_scan[255 - tid] = x;   // keys in buckets >= d
  }
  __syncthreads();
  if (tid < 256) {
    const uint32_t ge = s_scan[tid];
    const uint32_t gt = tid < 255 ? s_scan[tid + 1] : 0u;
    if (ge >= (uint32_t)krem && gt < (uint32_t)krem) {
      s_prefix[0] = (prefix << 8) | (uint64_t)tid;
      s_krem[0] = krem - (int)gt;
      s_krem[1] = (int)(ge - gt);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(SELT) void select_kernel(TopkArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t pi = pair_index(a, b, g);
  __shared__ uint64_t skeys[SEL_LDS_KEYS];
  __shared__ uint32_t bins[256];
  __shared__ uint32_t s_scan[256 + 4];
  __shared__ uint64_t s_prefix[1];
  __shared__ int s_krem[2];
  __shared__ int s_tot[SELT / 64];
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  int32_t* out = a.out_idx + pi * a.k_max;
  int written = 0;
  if (k > 0) {
    const uint64_t* gkeys = a.keys + pi * a.c.max_tokens;
    const int nc = hi - lo;
    const bool in_lds = nc <= SEL_LDS_KEYS;
    if (in_lds)
      for (int i = tid; i < nc; i += SELT) skeys[i] = gkeys[lo + i];
    if (tid < 256) {
      uint32_t x = 0;
      const uint32_t* h = a.hist + pi * HSTRIDE;
#pragma unroll
      for (int r = 0; r < HREP; ++r) x += h[r * 256 + tid];
      bins[tid] = x;
    }
    __syncthreads();
    auto key_at = [&](int i) -> uint64_t { return in_lds ? skeys[i] : gkeys[lo + i]; };

    // ---- passes: pick each byte; stop once a bucket is taken whole
    uint64_t prefix = 0;
    int krem = k, bits = 0;
    for (int p = 0; p < PASSES; ++p) {
      select_byte_lds(bins, prefix, krem, s_prefix, s_krem, s_scan);
      prefix = s_prefix[0];
      krem = s_krem[0];
      if (s_krem[1] == krem) {
        bits = 8 * (p + 1);
        break;
      }
      if (p == PASSES - 1) break;
      if (tid < 256) bins[tid] = 0u;
      __syncthreads();
      const int shift = 56 - 8 * p;   // bits above the next byte
      for (int i = tid; i < nc; i += SELT) {
        const uint64_t key = key_at(i);
        if (key && (key >> shift) == prefix) atomicAdd(&bins[(key >> (shift - 8)) & 255u], 1u);
      }
      __syncthreads();
    }

    // ---- selected = above the threshold, plus the first krem keys equal to it
    // by index (bits > 0: every key whose top `bits` bits reach the prefix)
    const uint64_t T = prefix;
    int eq_taken = 0;
    for (int c0 = 0; c0 < nc; c0 += SELT) {
      const int i = c0 + tid;
      const uint64_t key = i < nc ? key_at(i) : 0ull;
      const bool ab = key != 0 && (bits ? (key >> (64 - bits)) >= T : key > T);
      const bool eq = key != 0 && !bits && key == T;
      const uint64_t eb = __ballot(eq);
      if (lane == 0) s_tot[wv] = __popcll(eb);
      __syncthreads();
      int eq_before = eq_taken, eq_chunk = 0;
      for (int x = 0; x < SELT / 64; ++x) {
        const int v = s_tot[x];
        eq_before += x < wv ? v : 0;
        eq_chunk += v;
      }
      eq_before += __popcll(eb & ((1ull << lane) - 1ull));
      const bool take = ab || (eq && eq_before < krem);
      __syncthreads();
      const uint64_t tb = __ballot(take);
      if (lane == 0) s_tot[wv] = __popcll(tb);
      __syncthreads();
      int pos = written, chunk = 0;
      for (int x = 0; x < SELT / 64; ++x) {
        const int v = s_tot[x];
        pos += x < wv ? v : 0;
        chunk += v;
      }
      pos += __popcll(tb & ((1ull << lane) - 1ull));
      if (take && pos < a.k_max) out[pos] = lo + i;
      written += chunk;
      eq_taken += eq_chunk;
      __syncthreads();
    }
  }
  for (int e = written + tid; e < a.k_max; e += SELT) out[e] = -1;
}

}  // namespace

size_t topk_workspace_bytes(const kvc_cache& c) {
  const size_t pairs = (size_t)c.batch * c.num_kv_heads;
  const size_t words = c.max_tokens / 32;
  size_t bytes = 2 * pairs * c.max_tokens * sizeof(uint64_t);   // keys, block-mode token scores
  bytes += pairs * GMAX * D * sizeof(double);                    // critical-mode q operands
  bytes += pairs * HSTRIDE * sizeof(uint32_t);
  bytes += 2 * pairs * words * sizeof(uint32_t);
  bytes += pairs * D * sizeof(int32_t);
  bytes += pairs * PASSES * (sizeof(uint64_t) + sizeof(int32_t)) + pairs * sizeof(int32_t);
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
  char* p = static_cast<char*>(ws);
  a.keys = reinterpret_cast<uint64_t*>(p);
  p += pairs * c.max_tokens * sizeof(uint64_t);
  a.tscore = reinterpret_cast<double*>(p);
  p += pairs * c.max_tokens * sizeof(double);
  a.qsel = reinterpret_cast<double*>(p);
  p += pairs * GMAX * D * sizeof(double);
  a.hist = reinterpret_cast<uint32_t*>(p);
  p += pairs * HSTRIDE * sizeof(uint32_t);
  a.above = reinterpret_cast<uint32_t*>(p);
  p += pairs * words * sizeof(uint32_t);
  a.equal = reinterpret_cast<uint32_t*>(p);
  p += pairs * words * sizeof(uint32_t);
  a.channels = reinterpret_cast<int32_t*>(p);
  p += pairs * D * sizeof(int32_t);
  a.prefix = reinterpret_cast<uint64_t*>(p);
  p += pairs * PASSES * sizeof(uint64_t);
  a.krem = reinterpret_cast<int32_t*>(p);
  p += pairs * PASSES * sizeof(int32_t);
  a.done = reinterpret_cast<int32_t*>(p);

  const int Hkv = c.num_kv_heads, B = c.batch;
  // candidate ranges whose keys fit in LDS: one selection workgroup per pair
  // after scoring, instead of seven radix launches, mark and emit (measured:
  // longer ranges re-read from L2 by one workgroup lose to the radix kernels)
  const bool one_wg = (a.blocks ? c.max_tokens / GS : c.max_tokens) <= SEL_LDS_KEYS;
  a.hist_words = one_wg ? HREP * 256 : HSTRIDE;
  prep_kernel<<<dim3(Hkv, B), D, 0, s>>>(a);
  const dim3 sgrid((c.max_tokens + ST - 1) / ST, Hkv, B);
  const bool exact = mode == KVC_SCORE_EXACT;
  // the scorer's q operands in LDS: G heads x the channels it sums over
  const int nch = mode == KVC_SCORE_CRITICAL ? n_crit : (exact ? D : 0);
  const size_t sq_bytes = (size_t)std::max(1, a.G * nch) * sizeof(double);
#define KVC_SCORE_E(F, KT, GG)                                                \
  do {                                                                        \
    if (exact) score_kernel<F, KT, GG, true><<<sgrid, ST, sq_bytes, s>>>(a);  \
    else score_kernel<F, KT, GG, false><<<sgrid, ST, sq_bytes, s>>>(a);       \
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
  if (one_wg) {
    select_kernel<<<dim3(Hkv, B), SELT, 0, s>>>(a);
    return hipGetLastError();
  }
  const dim3 rgrid((c.max_tokens + TPB - 1) / TPB, Hkv, B);
  for (int pass = 1; pass < PASSES; ++pass) radix_kernel<<<rgrid, ST, 0, s>>>(a, pass);
  mark_kernel<<<rgrid, ST, 0, s>>>(a);
  emit_kernel<<<dim3(Hkv, B), ET, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvc
