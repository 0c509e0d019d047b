// Token scoring and exact Top-K selection (TailorKV article, section 2.3:
// channel importance |q_i| * max|K_i|, approximate scores on the critical
// channels, Top-K retrieval; meeting-LLM article, section 2.2: query-aware
// scores; StreamingLLM / H2O survey, section 3: sinks, recent window and
// cumulative scores).
//
// Kernels, all on the caller's stream:
//   score    the fp64 score of every candidate token, summed channel by channel
//            in ascending order from +0.0 (the order the interface fixes, so
//            results are reproducible bit for bit), max over the query group,
//            turned into an order-preserving 64-bit key (0 = not a candidate);
//            histogram of the keys' 12-bit coarse bins (sign, clamped exponent,
//            4 mantissa bits: a monotone function of the key), each workgroup's
//            stored whole in its own slot (no atomics, nothing to clear before
//            the call; the compaction sums the slots).  Critical mode
//            ranks the channels in every workgroup (importance from q and the
//            cache's per-channel maximum).  Workgroups loop over chunks of the
//            pair's tokens; external scores and channel-major fp16 keys take
//            four tokens a thread with vector loads.
//   compact  (long ranges) per 4096 items: the coarse bin tb holding the k-th
//            largest key (from the histogram); a bitmap of the items in bins
//            above tb and their count, and the items of bin tb (key, index) in
//            index order; tb and the count above it for the pair.
//   finish   (long ranges) one workgroup per 4096-item region: exact radix
//            select among the pair's bin-tb items (LDS passes over 8-bit
//            digits from the first digit where they differ), lower index first
//            among equal keys, then the region's selected indices written in
//            ascending order at the offset the earlier regions' counts give.
//            Short ranges: one workgroup per pair reads the key row itself.
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
constexpr int SCT = 1024;      // threads of a scoring workgroup (one token each a chunk)
constexpr int TPT = 4;         // tokens a thread scores a chunk (vector-load kernels)
constexpr int CUS = 256;       // compute units of an MI355X (scoring grids are sized to fill them once)
constexpr int CBINS = 4096;    // coarse bins of the keys
constexpr int SUP = CBINS / 64;    // super-bins (64 coarse bins each)
constexpr int HWS = CBINS + SUP;   // histogram words of one workgroup's slot
constexpr int NSLOT = 256;     // histogram slots (counting workgroups) per pair at most
constexpr int CT = 4096;       // items per compaction region
constexpr int RW = CT / 32;    // bitmap words per region
constexpr int FT = 1024;       // threads of the short-range finish workgroup
constexpr int DIRECT_MAX = 8192;   // items up to which one workgroup per pair selects from the key row
constexpr int FR = 256;        // threads of a region-finish workgroup
constexpr int CAP_R = 4096;    // bin-tb items a region-finish workgroup holds in LDS
constexpr int MAXR = KVC_TOPK_MAX_ITEMS / CT;   // compaction regions per pair at most
static_assert(KVC_TOPK_MAX_ITEMS % CT == 0, "whole regions");

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
  uint32_t* hist;      // [B][Hkv][nslot]: each counting workgroup's [CBINS] coarse histogram,
                       // then its [SUP] super-bin sums (written whole: nothing to clear)
  int nslot;           // counting workgroups per pair (the grid's x size)
  uint32_t* above;     // [B][Hkv][max_tokens / 32] items in bins above the threshold bin
  uint64_t* ckey;      // [B][Hkv][nreg * CT] keys of the threshold bin, per compaction region
  int32_t* cidx;       // [B][Hkv][nreg * CT] their item indices
  int32_t* ccount;     // [B][Hkv][nreg] threshold-bin entries per region
  int32_t* acount;     // [B][Hkv][nreg] items above the threshold bin per region
  int32_t* pmeta;      // [B][Hkv][2] threshold bin tb, items in the bins above it
  int nreg;            // compaction regions per pair (ceil(items / CT))
  bool blocks;         // rank 64-token blocks (items = block ids)
  bool use_hist;       // long ranges: the coarse histogram is built (short ranges select
                       // from the key row alone)
  double* tscore;      // block mode: [B][Hkv][max_tokens] token scores
};

// Workgroup barrier that orders LDS accesses only: global loads and stores
// stay in flight across it (every value these kernels pass between threads
// goes through LDS; a global value is only used by the thread that loaded it).
__device__ inline void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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


// External scores on tokens write no key row: the stages after scoring
// derive each item's key from the score itself (4 bytes read instead of 8
// written and 8 read); the same key the scorer counted.
__device__ inline bool keys_from_ext(const TopkArgs& a) {
  return a.mode == KVC_SCORE_EXTERNAL && !a.blocks;
}
__device__ inline uint64_t ext_key(float x) { return order_key(__dadd_rn((double)x, 0.0)); }

// ------------------------------------------------------------------ score
constexpr int GMAX = 16;       // query heads per KV head supported by scoring
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
  const auto add_batch = [&](int k0, const int* ch, const uint32_t* raw) {
    uint32_t mx[CB];
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
  };
  if constexpr (ALL && GT > 0 && GT <= 4) {
    // Every channel, up to 4 heads: each batch's global loads go out before
    // the previous batch's arithmetic, so the token's batches share one round
    // trip (larger groups have no registers to spare for it).
    int ch[CB];
    uint32_t raw[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) ch[u] = u;
#pragma unroll
    for (int u = 0; u < CB; ++u) raw[u] = load(ch[u]);
#pragma unroll 1
    for (int k0 = 0; k0 < D; k0 += CB) {
      int chn[CB];
      uint32_t rawn[CB] = {};
#pragma unroll
      for (int u = 0; u < CB; ++u) chn[u] = k0 + CB + u;
      if (k0 + CB < D) {
#pragma unroll
        for (int u = 0; u < CB; ++u) rawn[u] = load(chn[u]);
      }
      add_batch(k0, ch, raw);
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        ch[u] = chn[u];
        raw[u] = rawn[u];
      }
    }
  } else {
#pragma unroll 1
    for (int k0 = 0; k0 < nch; k0 += CB) {
      int ch[CB];
      uint32_t raw[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) ch[u] = ALL ? k0 + u : sch[min(k0 + u, nch - 1)];
#pragma unroll
      for (int u = 0; u < CB; ++u) raw[u] = load(ch[u]);   // global loads, all in flight
      add_batch(k0, ch, raw);
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

// Critical channels of the pair (TailorKV article, section 2.3): importance
// s_c = (max over the query group of |q_c|) * max_t |K_{t,c}| (the cache's
// running per-channel maximum), an exact fp64 product; the n_crit most
// important, ties to the lower channel, listed in ascending channel order in
// sch[0 .. n_crit) with the group's q values on them in sq[head][slot] (fp64).
// The product of an fp16 by an fp32 value has at most 35 significant bits, so
// the low 7 bits of its order-preserving key are free for the channel
// (127 - c): the keys are distinct and order (s desc, c asc) as integers.
// Each channel's rank is counted by NT / D threads over a share of the others.
// Every thread of the workgroup calls it (it synchronizes); the caller
// synchronizes before reading the lists.  GT: the group size when known at
// compile time (0: up to GMAX heads).
template <int NT, int GT>
__device__ void critical_channels(const TopkArgs& a, int b, int g, int64_t pi, int tid,
                                  uint64_t* s_key, int* s_cnt, int* s_pos, int* sch, double* sq,
                                  bool write_out) {
  constexpr int GN = GT > 0 ? GT : GMAX;
  constexpr int P = NT / D;   // threads ranking one channel
  static_assert(P >= 1 && 64 % P == 0, "a channel's rankers share a wave");
  const int G = a.G, nch = a.n_crit;
  uint16_t qh[GN];
  if (tid < D) {
    // every load is issued before any is used: heads past the group re-read
    // head 0 (the maximum is unchanged), so no load sits behind a branch
    const float kabs = a.c.k_absmax[pi * D + tid];
    const uint16_t* qg = a.q + ((int64_t)b * a.hq + g * G) * D + tid;
#pragma unroll
    for (int hh = 0; hh < GN; ++hh) qh[hh] = qg[(hh < G ? hh : 0) * D];
    double qm = 0.0;
#pragma unroll
    for (int hh = 0; hh < GN; ++hh) qm = fmax(qm, fabs((double)h2f(qh[hh])));
    const double imp = __dadd_rn(__dmul_rn(qm, (double)kabs), 0.0);   // (-0 ranks as +0)
    s_key[tid] = (order_key(imp) & ~127ull) | (uint64_t)(D - 1 - tid);
  }
  lds_sync();
  {
    const int c = tid / P, part = tid % P;
    const uint64_t kc = s_key[c];
    int rank = 0;   // channels ahead of c
#pragma unroll
    for (int i = 0; i < D / P; ++i) rank += s_key[part * (D / P) + i] > kc ? 1 : 0;
#pragma unroll
    for (int m = 1; m < P; m <<= 1) rank += __shfl_xor(rank, m);
    const bool mine = part == 0 && rank < nch;
    const uint64_t bal = __ballot(mine);
    if ((tid & 63) == 0) s_cnt[tid >> 6] = __popcll(bal);
    lds_sync();
    if (part == 0) {   // position in the ascending list: chosen channels below c
      int pos = -1;
      if (mine) {
        pos = __popcll(bal & ((1ull << (tid & 63)) - 1ull));
        for (int w = 0; w < (tid >> 6); ++w) pos += s_cnt[w];
      }
      s_pos[c] = pos;
    }
  }
  lds_sync();
  if (tid < D) {
    const int pos = s_pos[tid];
    if (pos >= 0) {
      sch[pos] = tid;
      if (write_out && a.out_channels) a.out_channels[pi * nch + pos] = tid;
#pragma unroll
      for (int hh = 0; hh < GN; ++hh)
        if (hh < G) sq[hh * nch + pos] = (double)h2f(qh[hh]);
    }
  }
}

// Stores the workgroup's LDS histogram in its slot of the pair (slot
// blockIdx.x, every bin, zeros too) with the super-bin sums after it (a
// wave's 64 consecutive bins are one super-bin, summed across the wave).
// Plain stores: no atomics, and no slot needs clearing before the call.
// In block mode only the block-key workgroups count (BK).
template <int NT, bool BK = false>
__device__ inline void flush_hist(const TopkArgs& a, int64_t pi, const uint32_t* sh, int tid) {
  static_assert(NT % 64 == 0 && CBINS % NT == 0, "whole super-bins a wave");
  if (!a.use_hist || a.blocks != BK) return;
  uint32_t* h = a.hist + (pi * a.nslot + blockIdx.x) * HWS;
  for (int e = tid; e < CBINS; e += NT) {
    const uint32_t c = sh[e];
    h[e] = c;
    uint32_t t = c;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
    if ((tid & 63) == 0) h[CBINS + (e >> 6)] = t;
  }
}

// The score of one candidate as the order-preserving key and the optional
// score outputs (block mode: the token score for block_key, no key).
__device__ inline uint64_t emit_score(const TopkArgs& a, int64_t pi, int t, double r) {
  r = __dadd_rn(r, 0.0);
  if (a.blocks) {
    a.tscore[pi * a.c.max_tokens + t] = r;
    return 0ull;
  }
  if (a.out_scores) a.out_scores[pi * a.c.max_tokens + t] = r;
  return order_key(r);
}

// Generic scorer, one token a thread per chunk of NT tokens; the workgroup's
// chunks are blockIdx.x, blockIdx.x + gridDim.x, ... of the pair.  Quantized
// caches stage the chunk's K metadata in LDS first.  Workgroup size: 1024,
// except in exact mode and for query groups of 8 or more heads, whose sums
// need the registers of 256-thread groups.
template <bool EXACT, int GT>
constexpr int score_threads() { return EXACT || GT == 0 || GT >= 8 ? ST : SCT; }

template <int FMT, bool KT, int GT, bool EXACT>
__global__ __launch_bounds__((score_threads<EXACT, GT>())) void score_kernel(TopkArgs a) {
  constexpr int NT = score_threads<EXACT, GT>();
  constexpr int CB = EXACT ? CB_EXACT : CB_CRIT;
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  extern __shared__ double sq[];    // q as fp64, [head][channel slot], G x nch (sized at launch)
  __shared__ int sch[D];
  __shared__ uint64_t s_key[D];
  __shared__ int s_cnt[NT / 64];
  __shared__ int s_pos[D];
  __shared__ uint32_t sh[CBINS];
  __shared__ uint32_t smeta[grouped(FMT) ? (NT / GS) * D : 1];   // (scale | zero << 16) per channel
  const int G = a.G;
  const kvc_cache& c = a.c;
  const int nch = a.mode == KVC_SCORE_CRITICAL ? a.n_crit : D;
  for (int e = tid; e < CBINS; e += NT) sh[e] = 0u;
  // K metadata words of a chunk's groups (quantized caches), channel pairs a
  // thread; the first chunk's go out with the setup loads, each next chunk's
  // while the current one is scored
  const int chunks = (c.max_tokens + NT - 1) / NT;
  auto meta_load = [&](int ci, uint32_t& s2, uint32_t& z2) {
    const int groups = c.max_tokens / GS;
    const int gq = ci * (NT / GS) + tid / 64, j = tid % 64;
    s2 = z2 = 0u;
    if (gq < groups) {
      const uint32_t* km = reinterpret_cast<const uint32_t*>(c.k_meta + (pi * groups + gq) * 2 * D);
      s2 = km[j];
      z2 = km[D / 2 + j];
    }
  };
  uint32_t ms2 = 0u, mz2 = 0u;
  if (grouped(FMT) && (int)blockIdx.x < chunks) meta_load(blockIdx.x, ms2, mz2);
  int lo, hi, kk;
  cand_range(a, b, lo, hi, kk);   // (its loads go out with the channel ranking's)
  if (a.blocks) {   // every token of the candidate blocks
    lo *= GS;
    hi *= GS;
  }
  const int n = max(c.seq_lens[b], 0);
  if (a.mode == KVC_SCORE_CRITICAL) {
    critical_channels<NT, GT>(a, b, g, pi, tid, s_key, s_cnt, s_pos, sch, sq, blockIdx.x == 0);
  } else {   // exact: every channel in order
    for (int e = tid; e < D; e += NT) sch[e] = e;
    for (int e = tid; e < G * D; e += NT)
      sq[e] = (double)h2f(a.q[((int64_t)b * a.hq + g * G + e / D) * D + e % D]);
  }
  lds_sync();

  for (int ci = blockIdx.x; ci < chunks; ci += gridDim.x) {
    const int t = ci * NT + tid;
    if (grouped(FMT)) {   // stage the chunk's metadata: (scale | zero << 16) per channel
      if (ci != (int)blockIdx.x) lds_sync();   // (the previous chunk's is no longer read)
      const int j = tid % 64;
      uint32_t m0 = (ms2 & 0xFFFFu) | (mz2 << 16), m1 = (ms2 >> 16) | (mz2 & 0xFFFF0000u);
      // outlier channels (INT4): the word names the outlier store entry instead
      // (a zero-point field of all ones is a NaN no quantized group stores)
      for (int e = 0; e < c.n_outlier; ++e) {
        const int oc = c.outlier_ch[g * KVC_MAX_OUTLIERS + e];
        if (oc == 2 * j) m0 = OUT_TAG | e;
        if (oc == 2 * j + 1) m1 = OUT_TAG | e;
      }
      smeta[(tid / 64) * D + 2 * j] = m0;
      smeta[(tid / 64) * D + 2 * j + 1] = m1;
      lds_sync();
      if (ci + (int)gridDim.x < chunks) meta_load(ci + gridDim.x, ms2, mz2);
    }
    const bool in = t < c.max_tokens;
    uint64_t key = 0;
    if (in && t >= lo && t < hi) {
      const int nq = grouped(FMT) ? (n & ~(GS - 1)) : n;
      const int64_t slot = slot_of(c, b, g, t);
      double r = -INFINITY;
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
      key = emit_score(a, pi, t, r);
    }
    if (key) {   // (key rows hold candidates only; block mode: none)
      __builtin_nontemporal_store(key, a.keys + pi * c.max_tokens + t);
      if (a.use_hist) atomicAdd(&sh[coarse_of(key)], 1u);
    }
  }
  lds_sync();
  flush_hist<NT>(a, pi, sh, tid);
}

// Stores a thread's TPT consecutive keys (32 bytes, aligned; nontemporal, so
// the key rows do not sit dirty in L2 when the kernel ends) and counts them.
__device__ inline void put_keys(const TopkArgs& a, int64_t pi, int t0, const uint64_t* kv, uint32_t* sh) {
  typedef __attribute__((ext_vector_type(4))) unsigned u4v;
  u4v* dst = reinterpret_cast<u4v*>(a.keys + pi * a.c.max_tokens + t0);
  __builtin_nontemporal_store(u4v{(uint32_t)kv[0], (uint32_t)(kv[0] >> 32), (uint32_t)kv[1], (uint32_t)(kv[1] >> 32)}, dst);
  __builtin_nontemporal_store(u4v{(uint32_t)kv[2], (uint32_t)(kv[2] >> 32), (uint32_t)kv[3], (uint32_t)(kv[3] >> 32)}, dst + 1);
#pragma unroll
  for (int u = 0; u < TPT; ++u)
    if (kv[u] && a.use_hist) atomicAdd(&sh[coarse_of(kv[u])], 1u);
}

// External scores (H2O cumulative scores, or any the caller gives), any
// format: four consecutive tokens a thread from one 16-byte load.
__global__ __launch_bounds__(SCT) void score_ext_kernel(TopkArgs a) {
  static_assert(TPT == 4, "one float4 a thread");
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  __shared__ uint32_t sh[CBINS];
  for (int e = tid; e < CBINS; e += SCT) sh[e] = 0u;
  int lo, hi, kk;
  cand_range(a, b, lo, hi, kk);
  if (a.blocks) {
    lo *= GS;
    hi *= GS;
  }
  lds_sync();
  const int T = a.c.max_tokens;   // a multiple of 64: a thread's tokens are all in or all out
  const float* ext = a.ext + pi * T;
  const int chunks = (T + SCT * TPT - 1) / (SCT * TPT);
  for (int ci = blockIdx.x; ci < chunks; ci += gridDim.x) {
    const int t0 = (ci * SCT + tid) * TPT;
    if (t0 >= T || t0 + TPT <= lo || t0 >= hi) continue;   // (key rows hold candidates only)
    const float4 e4 = *reinterpret_cast<const float4*>(ext + t0);
    const float ev[TPT] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
    for (int u = 0; u < TPT; ++u) {   // (no key row: later stages derive the keys from ext)
      const int t = t0 + u;
      const uint64_t key = t >= lo && t < hi ? emit_score(a, pi, t, (double)ev[u]) : 0ull;
      if (key && a.use_hist) atomicAdd(&sh[coarse_of(key)], 1u);
    }
  }
  lds_sync();
  flush_hist<SCT>(a, pi, sh, tid);
}

// Critical-channel scores from the channel-major fp16 copy of K (contiguous
// caches, query groups of up to 4 heads): four consecutive tokens a thread,
// one 8-byte load per channel.  Same sums, in the same order, as
// token_score.  Two workgroups a CU (64 registers), except for groups of 4
// heads, whose 16 fp64 sums and 8 loads in flight need more: one a CU.
template <int GT>
__global__ __launch_bounds__(SCT, GT == 4 ? 4 : 8) void score_kt_kernel(TopkArgs a) {
  static_assert(TPT == 4 && GT >= 1 && GT <= 4, "four tokens from one 8-byte load per channel");
  constexpr int CB = CB_CRIT;
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  extern __shared__ double sq[];    // [head][channel slot], GT x n_crit
  __shared__ int sch[D];
  __shared__ uint64_t s_key[D];
  __shared__ int s_cnt[SCT / 64];
  __shared__ int s_pos[D];
  __shared__ uint32_t sh[CBINS];
  for (int e = tid; e < CBINS; e += SCT) sh[e] = 0u;
  int lo, hi, kk;
  cand_range(a, b, lo, hi, kk);   // (its loads go out with the channel ranking's)
  if (a.blocks) {
    lo *= GS;
    hi *= GS;
  }
  critical_channels<SCT, GT>(a, b, g, pi, tid, s_key, s_cnt, s_pos, sch, sq, blockIdx.x == 0);
  lds_sync();
  const int T = a.c.max_tokens, nch = a.n_crit;
  const uint16_t* kt = a.c.kT + pi * D * (int64_t)T;
  const int chunks = (T + SCT * TPT - 1) / (SCT * TPT);
  for (int ci = blockIdx.x; ci < chunks; ci += gridDim.x) {
    const int t0 = (ci * SCT + tid) * TPT;
    if (t0 >= T || t0 + TPT <= lo || t0 >= hi) continue;   // (key rows hold candidates only)
    uint64_t kv[TPT] = {0ull, 0ull, 0ull, 0ull};
    {
      double acc[GT][TPT];
#pragma unroll
      for (int hh = 0; hh < GT; ++hh)
#pragma unroll
        for (int u = 0; u < TPT; ++u) acc[hh][u] = 0.0;
#pragma unroll 1
      for (int k0 = 0; k0 < nch; k0 += CB) {
        uint2 raw[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u)
          raw[u] = *reinterpret_cast<const uint2*>(kt + (int64_t)sch[min(k0 + u, nch - 1)] * T + t0);
#pragma unroll
        for (int u = 0; u < CB; ++u) {
          const bool on = k0 + u < nch;
          const int kq = min(k0 + u, nch - 1);
          const uint32_t w2[2] = {raw[u].x, raw[u].y};
#pragma unroll
          for (int v = 0; v < TPT; ++v) {
            const double x = (double)h2f((uint16_t)(w2[v / 2] >> (16 * (v % 2))));
#pragma unroll
            for (int hh = 0; hh < GT; ++hh) {
              const double nx = __dadd_rn(acc[hh][v], __dmul_rn(sq[hh * nch + kq], x));
              acc[hh][v] = on ? nx : acc[hh][v];
            }
          }
        }
      }
#pragma unroll
      for (int v = 0; v < TPT; ++v) {
        const int t = t0 + v;
        double r = acc[0][v];
#pragma unroll
        for (int hh = 1; hh < GT; ++hh) r = fmax(r, acc[hh][v]);
        kv[v] = t >= lo && t < hi ? emit_score(a, pi, t, r) : 0ull;
      }
    }
    if (!a.blocks) put_keys(a, pi, t0, kv, sh);
  }
  lds_sync();
  flush_hist<SCT>(a, pi, sh, tid);
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
  const double* ts = a.tscore + pi * a.c.max_tokens;
  for (int e = tid; e < CBINS; e += ST) sh[e] = 0u;
  const int nchunk = (a.c.max_tokens / GS + BPW - 1) / BPW;
  for (int ch = blockIdx.x; ch < nchunk; ch += gridDim.x) {   // BPW blocks a round
    const int j0 = ch * BPW;
    lds_sync();   // (the previous round's LDS reads are done)
    {   // every load is issued before the LDS stores (a load-store loop waits each time)
      constexpr int R = BPW * GS / ST;
      double v[R];
  #pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = r * ST + tid, j = j0 + e / GS;
        v[r] = ts[(int64_t)j0 * GS + (j >= lo && j < hi ? e : 0)];
      }
  #pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = r * ST + tid, j = j0 + e / GS;
        ss[e] = j >= lo && j < hi ? v[r] : 0.0;
      }
    }
    lds_sync();
    if (tid < BPW) {
      const int j = j0 + tid;
      if (j >= lo && j < hi) {
        double sum = 0.0;
        for (int i = 0; i < GS; ++i) sum = __dadd_rn(sum, ss[tid * GS + i]);
        const double r = __dadd_rn(__ddiv_rn(sum, (double)GS), 0.0);
        const uint64_t key = order_key(r);
        a.keys[pi * a.c.max_tokens + j] = key;
        if (a.out_scores) a.out_scores[pi * a.c.max_tokens + j] = r;
        if (a.use_hist) atomicAdd(&sh[coarse_of(key)], 1u);
      }
    }
  }
  lds_sync();
  flush_hist<ST, true>(a, pi, sh, tid);
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
  lds_sync();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const uint32_t v = s_wsum[k];
    before += k < wv ? v : 0u;
    all += v;
  }
  lds_sync();
  *total = all;
  return before + x;
}

// Inclusive sum of x over the lanes up to this one (one wave).
__device__ inline uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// The coarse bin tb holding the k-th largest key of the pair (1 <= k <= keys
// counted) and n_gt, the keys in the bins above it.  The NT / 64 waves sum the
// slots in shares (lane l: super-bin SUP - 1 - l, highest first; every load of
// a share in flight at once), wave 0 adds the shares and finds the super-bin
// holding the k-th key, then the same for that super-bin's 64 bins.  Results in
// s_res[0] (tb) and s_res[1] (n_gt); s_res[2..3] and s_part[NT] are scratch;
// every thread calls it.
template <int NT>
__device__ void coarse_threshold(const uint32_t* hist, int nslot, int k, int* s_res, uint32_t* s_part) {
  static_assert(SUP == 64 && NT % 64 == 0, "one super-bin a lane");
  constexpr int NWV = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t x = 0;   // super-bin SUP - 1 - lane over the wave's share of the slots
#pragma unroll 8
  for (int sl = wv; sl < nslot; sl += NWV) x += hist[sl * HWS + CBINS + (SUP - 1 - lane)];
  s_part[tid] = x;
  lds_sync();
  if (wv == 0) {
    if (lane == 0) {   // (k is at most the keys counted, so a lane overwrites these)
      s_res[0] = 0;
      s_res[1] = 0;
    }
#pragma unroll
    for (int w = 1; w < NWV; ++w) x += s_part[w * 64 + lane];
    const uint32_t incl = wave_incl_scan(x);
    const uint64_t hit = __ballot(incl - x < (uint32_t)k && incl >= (uint32_t)k);
    const int L = hit ? __ffsll((unsigned long long)hit) - 1 : SUP - 1;
    const uint32_t above = __shfl(incl - x, L);   // keys in the super-bins above S
    if (lane == 0) {
      s_res[2] = SUP - 1 - L;                     // the super-bin S
      s_res[3] = (int)above;
    }
  }
  lds_sync();
  const int S = s_res[2];
  uint32_t y = 0;   // bin 64 S + 63 - lane over the wave's share of the slots
#pragma unroll 8
  for (int sl = wv; sl < nslot; sl += NWV) y += hist[sl * HWS + S * 64 + (63 - lane)];
  s_part[tid] = y;
  lds_sync();
  if (wv == 0) {
#pragma unroll
    for (int w = 1; w < NWV; ++w) y += s_part[w * 64 + lane];
    const uint32_t incl2 = wave_incl_scan(y) + (uint32_t)s_res[3];
    if (incl2 - y < (uint32_t)k && incl2 >= (uint32_t)k) {
      s_res[0] = S * 64 + 63 - lane;
      s_res[1] = (int)(incl2 - y);
    }
  }
  lds_sync();
}

// ------------------------------------------------------------------ compact
// Long candidate ranges: CT items a workgroup (ST threads, CT / ST rounds).
// Bits of the items whose coarse bin is above tb go to the `above` bitmap
// (every word of the pair is written by some workgroup) and their number to
// acount; the items of bin tb go, in index order, to this workgroup's region
// of ckey / cidx, with their number in ccount.  The first workgroup of the
// pair also stores tb and the count of items above it.
__global__ __launch_bounds__(ST) void compact_kernel(TopkArgs a) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t pi = pair_index(a, b, g);
  constexpr int R = CT / ST;   // rounds
  __shared__ int s_res[4];
  __shared__ uint32_t s_part[ST];
  __shared__ uint32_t s_cnt[R * (ST / 64)];
  __shared__ uint32_t s_acnt[R * (ST / 64)];
  __shared__ uint32_t s_off[R * (ST / 64)];
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  if (k <= 0) return;   // (finish writes the -1 padding)
  const int N = item_count(a.c, a.blocks);
  const int nwords = (N + 31) / 32;
  const uint64_t* keys = a.keys + pi * a.c.max_tokens;
  const int base = blockIdx.x * CT;
  // the keys do not depend on the threshold: their loads go out with the
  // histogram's, so both arrive in one round trip
  // (the key row holds the candidates [lo, hi) only)
  uint64_t kv[R];
  if (keys_from_ext(a)) {
    const float* ex = a.ext + pi * a.c.max_tokens;
    float xv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) xv[j] = ex[min(max(base + j * ST + tid, lo), hi - 1)];
#pragma unroll
    for (int j = 0; j < R; ++j) kv[j] = ext_key(xv[j]);
  } else {
#pragma unroll
    for (int j = 0; j < R; ++j) kv[j] = keys[min(max(base + j * ST + tid, lo), hi - 1)];
  }
  coarse_threshold<ST>(a.hist + pi * a.nslot * HWS, a.nslot, k, s_res, s_part);
  const uint32_t tb = (uint32_t)s_res[0];
  if (blockIdx.x == 0 && tid == 0) {
    a.pmeta[2 * pi] = (int32_t)tb;
    a.pmeta[2 * pi + 1] = s_res[1];
  }
  uint64_t cand[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = base + j * ST + tid;
    const uint64_t key = i >= lo && i < hi ? kv[j] : 0ull;
    const uint32_t cb = coarse_of(key);
    const uint64_t ab = __ballot(key != 0 && cb > tb);
    cand[j] = __ballot(key != 0 && cb == tb);
    const int wd = (base + j * ST + wv * 64) / 32;   // the wave's first word
    uint32_t* aw = a.above + pi * (a.c.max_tokens / 32);
    if (lane == 0 && wd < nwords) aw[wd] = (uint32_t)ab;
    if (lane == 32 && wd + 1 < nwords) aw[wd + 1] = (uint32_t)(ab >> 32);
    if (lane == 0) {
      s_cnt[j * (ST / 64) + wv] = (uint32_t)__popcll(cand[j]);
      s_acnt[j * (ST / 64) + wv] = (uint32_t)__popcll(ab);
    }
  }
  lds_sync();
  if (tid < 64) {   // exclusive scan over the R * 4 (round, wave) counts, in index order
    uint32_t x = tid < R * (ST / 64) ? s_cnt[tid] : 0u;
    uint32_t y = tid < R * (ST / 64) ? s_acnt[tid] : 0u;
    const uint32_t own = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t xs = __shfl_up(x, o), ys = __shfl_up(y, o);
      if (lane >= o) {
        x += xs;
        y += ys;
      }
    }
    if (tid < R * (ST / 64)) s_off[tid] = x - own;
    if (tid == 63) {
      a.ccount[pi * a.nreg + blockIdx.x] = (int32_t)x;
      a.acount[pi * a.nreg + blockIdx.x] = (int32_t)y;
    }
  }
  lds_sync();
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
// Exact radix select among a set of keys (the threshold bin's): the krem
// largest, digit by digit (8 bits) from the first digit where the keys
// differ, with an LDS histogram per digit; once a digit's bucket is taken
// whole, the rest of it is selected by that prefix.  for_cand(f) calls f(key)
// for every key of the set, spread over the NT threads.
struct SelectLds {
  uint32_t bins[256];
  uint32_t wsum[FT / 64];
  uint64_t red[2 * (FT / 64)];
  uint64_t pfx;
  int res[4];   // [0], [1]: coarse_threshold's tb and count above; [2], [3]: select_digit's
};

// One digit of the selection, from the digit's histogram in L.bins: the
// bucket holding the krem-th largest key.  Wave 0 reads the 256 bins (lane l:
// bins 255 - 4l .. 252 - 4l, highest first), clears them for the next digit,
// scans the lane sums and the winning lane records the bucket; one barrier.
__device__ inline void select_digit(SelectLds& L, uint64_t prefix, int krem, uint64_t* new_prefix,
                                    int* new_krem, int* bucket) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    uint32_t x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = L.bins[255 - 4 * tid - i];
#pragma unroll
    for (int i = 0; i < 4; ++i) L.bins[255 - 4 * tid - i] = 0u;
    const uint32_t sum = x[0] + x[1] + x[2] + x[3];
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (tid >= o) incl += y;
    }
    if (tid == 0) {   // (krem is at most the keys counted, so some lane overwrites these)
      L.pfx = prefix << 8;
      L.res[2] = krem;
      L.res[3] = 0;
    }
    uint32_t run = incl - sum;   // keys in the bins above this lane's
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (run < (uint32_t)krem && run + x[i] >= (uint32_t)krem) {
        L.pfx = (prefix << 8) | (uint64_t)(255 - 4 * tid - i);
        L.res[2] = krem - (int)run;
        L.res[3] = (int)x[i];
      }
      run += x[i];
    }
  }
  lds_sync();
  *new_prefix = L.pfx;
  *new_krem = L.res[2];
  *bucket = L.res[3];
}

// Selects the krem0 largest keys of the set.  Results: bits > 0: every key
// whose top `bits` bits are >= P is selected (a bucket taken whole); bits ==
// 0: every key > P is selected, and the first krem keys equal to P (lower
// index first).
template <int NT, typename ForCand>
__device__ void exact_select(SelectLds& L, ForCand for_cand, int krem0, uint64_t& P, int& krem,
                             int& bits) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // common prefix of the keys: the digits before the first differing bit
  // need no pass
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
    L.red[NT / 64 + wv] = kor;
  }
  if (tid < 256) L.bins[tid] = 0u;   // (select_digit clears them after each digit)
  lds_sync();
  kand = ~0ull;
  kor = 0ull;
#pragma unroll
  for (int w2 = 0; w2 < NT / 64; ++w2) {
    kand &= L.red[w2];
    kor |= L.red[NT / 64 + w2];
  }
  const uint64_t diff = kand ^ kor;   // bits where the keys differ
  const int first = diff ? __clzll(diff) / 8 : 8;   // first digit with a difference
  P = first > 0 ? (kand >> (64 - 8 * first)) : 0ull;   // the chosen top 8p bits
  krem = krem0;
  bits = 0;
  for (int p = first; p < 8; ++p) {
    const int sh = 56 - 8 * p;
    const uint64_t Pp = P;
    for_cand([&](uint64_t key) {
      if (p == 0 || (key >> (sh + 8)) == Pp) atomicAdd(&L.bins[(key >> sh) & 255u], 1u);
    });
    lds_sync();
    int bucket;
    select_digit(L, P, krem, &P, &krem, &bucket);
    if (bucket == krem) {
      bits = 8 * (p + 1);
      break;
    }
  }
}

// Short ranges (at most DIRECT_MAX items, no compaction): one workgroup per
// (sequence, KV head) stages the key row in LDS, selects among the coarse bin
// tb's keys and emits straight from the row, FT items a round in index order.
struct DirectLds {
  uint64_t key[DIRECT_MAX];
  SelectLds s;
};

__global__ __launch_bounds__(FT) void finish_direct_kernel(TopkArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  __shared__ DirectLds L;
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  int32_t* out = a.out_idx + pi * a.k_max;
  if (k <= 0) {
    for (int e = tid; e < a.k_max; e += FT) out[e] = -1;
    return;
  }
  const int N = item_count(a.c, a.blocks);
  const uint64_t* gkeys = a.keys + pi * a.c.max_tokens;
  const bool fx = keys_from_ext(a);
  const float* ex = fx ? a.ext + pi * a.c.max_tokens : nullptr;
  // candidates only; every load of the row is issued before the LDS stores.
  // Each thread keeps its items (j FT + tid) in registers for the selection
  // passes; the emission reads the row back from LDS in index order.
  constexpr int R = DIRECT_MAX / FT;
  uint64_t kv[R];
  {
    if (fx) {
      float xv[R];
#pragma unroll
      for (int j = 0; j < R; ++j) xv[j] = ex[min(max(j * FT + tid, lo), hi - 1)];
#pragma unroll
      for (int j = 0; j < R; ++j) kv[j] = ext_key(xv[j]);
    } else {
#pragma unroll
      for (int j = 0; j < R; ++j) kv[j] = gkeys[min(max(j * FT + tid, lo), hi - 1)];
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int i = j * FT + tid;
      kv[j] = i >= lo && i < hi && i < N ? kv[j] : 0ull;
      if (i < N) L.key[i] = kv[j];
    }
  }
  lds_sync();
  // the selection runs over every candidate key (no histogram is built for
  // short ranges)
  const int krem0 = k;
  auto for_cand = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (kv[j]) f(kv[j]);
  };
  uint64_t P;
  int krem, bits;
  exact_select<FT>(L.s, for_cand, krem0, P, krem, bits);
  const uint64_t T = P;
  auto chosen = [&](uint64_t key, bool eq_ok) {
    return bits ? (key >> (64 - bits)) >= P : (key > T || (key == T && eq_ok));
  };
  // emission: thread t owns items [t per, (t + 1) per) of the row, so one scan
  // of the keys equal to T gives their ranks in index order and one scan of
  // the taken counts gives the output positions
  const int per = (N + FT - 1) / FT;
  const int i0 = min(tid * per, N), i1 = min(i0 + per, N);
  uint32_t neq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint64_t key = L.key[i];
    neq += key != 0 && !bits && key == T ? 1u : 0u;
  }
  uint32_t eq_tot;
  uint32_t rank = block_scan<FT>(neq, L.s.wsum, &eq_tot) - neq;
  const uint32_t rank0 = rank;
  uint32_t ntake = 0;
  for (int i = i0; i < i1; ++i) {   // (the same walk, counting what is taken)
    const uint64_t key = L.key[i];
    const bool eq = key != 0 && !bits && key == T;
    ntake += key != 0 && chosen(key, eq && rank < (uint32_t)krem) ? 1u : 0u;
    rank += eq ? 1u : 0u;
  }
  uint32_t take_tot;
  int pos = (int)(block_scan<FT>(ntake, L.s.wsum, &take_tot) - ntake);
  rank = rank0;
  for (int i = i0; i < i1; ++i) {
    const uint64_t key = L.key[i];
    const bool eq = key != 0 && !bits && key == T;
    if (key != 0 && chosen(key, eq && rank < (uint32_t)krem)) {
      if (pos < a.k_max) out[pos] = i;
      ++pos;
    }
    rank += eq ? 1u : 0u;
  }
  const int written = (int)take_tot;
  for (int e = written + tid; e < a.k_max; e += FT) out[e] = -1;
}

// Long ranges: one workgroup per (run of rpw regions, KV head, sequence).
// Every workgroup of a pair gathers the pair's threshold-bin items (the
// compaction lists, in index order; into LDS when there are at most CAP_R of
// them, else they are re-read from memory for each pass) and runs the same
// exact selection; it then counts the items selected in the regions before
// its first (above-bin counts, plus the threshold-bin items chosen there) and
// writes its regions' selected indices in ascending order from that offset.
constexpr int GB = 4;         // threshold-bin items a thread gathers a round
constexpr int RPW_MAX = 4;    // regions a finish workgroup may take
struct RegionLds {
  uint64_t key[CAP_R];
  int32_t idx[CAP_R];
  int32_t roff[MAXR + 1];   // start of each region's list in the pair's order
  uint32_t bm[RW];          // the current region's selected items
  SelectLds s;
};

__global__ __launch_bounds__(FR) void finish_region_kernel(TopkArgs a, int rpw) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pi = pair_index(a, b, g);
  __shared__ RegionLds L;
  int lo, hi, k;
  cand_range(a, b, lo, hi, k);
  int32_t* out = a.out_idx + pi * a.k_max;
  const int nreg = a.nreg;
  const int r0 = blockIdx.x * rpw, r1 = min(r0 + rpw, nreg);
  if (k <= 0) {
    if (r0 == 0)
      for (int e = tid; e < a.k_max; e += FR) out[e] = -1;
    return;
  }
  const int nwords = (item_count(a.c, a.blocks) + 31) / 32;
  // ---- loads that depend on nothing else here, issued together
  const int n_gt = a.pmeta[2 * pi + 1];
  uint32_t aw[RPW_MAX];
#pragma unroll
  for (int u = 0; u < RPW_MAX; ++u) {
    const int wd = min((r0 + u) * RW + tid, nwords - 1);
    aw[u] = a.above[pi * (a.c.max_tokens / 32) + wd];
  }
  uint32_t run = 0, abefore = 0;
  for (int q0 = 0; q0 < nreg; q0 += FR) {
    const int i = q0 + tid, ic = min(i, nreg - 1);
    const uint32_t cc = (uint32_t)a.ccount[pi * nreg + ic];
    const uint32_t ac = (uint32_t)a.acount[pi * nreg + ic];
    const uint32_t c = i < nreg ? cc : 0u;
    uint32_t tot, atot;
    const uint32_t incl = block_scan<FR>(c, L.s.wsum, &tot);
    block_scan<FR>(i < r0 ? ac : 0u, L.s.wsum, &atot);
    if (i < nreg) L.roff[i] = (int32_t)(run + incl - c);
    run += tot;
    abefore += atot;
  }
  const int C = (int)run;   // threshold-bin items of the pair (>= 1: the k-th key is one)
  if (tid == 0) L.roff[nreg] = C;
  lds_sync();
  const bool inlds = C <= CAP_R;
  if (inlds) {
    // entry e is in the last region rr with roff[rr] <= e; a round's loads are
    // all issued before its LDS stores
    for (int e0 = 0; e0 < C; e0 += FR * GB) {
      uint64_t kk[GB];
      int32_t ii[GB];
#pragma unroll
      for (int u = 0; u < GB; ++u) {
        const int e = min(e0 + u * FR + tid, C - 1);
        int rl = 0, rh = nreg - 1;
        while (rl < rh) {
          const int m = (rl + rh + 1) >> 1;
          if (L.roff[m] <= e) rl = m; else rh = m - 1;
        }
        const int64_t src = (pi * nreg + rl) * (int64_t)CT + (e - L.roff[rl]);
        kk[u] = a.ckey[src];
        ii[u] = a.cidx[src];
      }
#pragma unroll
      for (int u = 0; u < GB; ++u) {
        const int e = e0 + u * FR + tid;
        if (e < C) {
          L.key[e] = kk[u];
          L.idx[e] = ii[u];
        }
      }
    }
    lds_sync();
  }
  // threshold-bin keys of regions [q0, q1), in the pair's order
  auto for_regions = [&](int q0, int q1, auto&& f) {
    if (inlds) {
      for (int e = L.roff[q0] + tid; e < L.roff[q1]; e += FR) f(L.key[e]);
    } else {
      for (int rr = q0; rr < q1; ++rr) {
        const uint64_t* src = a.ckey + (pi * nreg + rr) * (int64_t)CT;
        const int cnt = L.roff[rr + 1] - L.roff[rr];
        for (int e = tid; e < cnt; e += FR) f(src[e]);
      }
    }
  };
  uint64_t P;
  int krem, bits;
  exact_select<FR>(L.s, [&](auto&& f) { for_regions(0, nreg, f); }, k - n_gt, P, krem, bits);
  const uint64_t T = P;
  auto chosen = [&](uint64_t key, bool eq_ok) {
    return bits ? (key >> (64 - bits)) >= P : (key > T || (key == T && eq_ok));
  };

  // ---- items selected before region r0: every above-bin item, the
  // threshold-bin keys above T (or in a bucket taken whole), and the first
  // krem keys equal to T
  uint32_t ngt = 0, neq = 0;
  for_regions(0, r0, [&](uint64_t key) {
    ngt += chosen(key, false) ? 1u : 0u;
    neq += !bits && key == T ? 1u : 0u;
  });
  uint32_t ngt_tot, neq_tot;
  block_scan<FR>(ngt, L.s.wsum, &ngt_tot);
  block_scan<FR>(neq, L.s.wsum, &neq_tot);
  int off = (int)(abefore + ngt_tot) + (bits ? 0 : min((int)neq_tot, krem));
  uint32_t eq_seen = neq_tot;   // keys equal to T in the regions before r

  for (int r = r0; r < r1; ++r) {
    // region r's bitmap: its above-bin items, then its chosen threshold-bin
    // items (thread t owns a contiguous run of the region's list, so the
    // ranks among keys equal to T follow index order)
    const int wd = r * RW + tid;
    if (tid < RW) L.bm[tid] = wd < nwords ? aw[r - r0] : 0u;
    lds_sync();
    const int o_r = L.roff[r], c_r = L.roff[r + 1] - o_r;
    const uint64_t* gk = a.ckey + (pi * nreg + r) * (int64_t)CT;
    const int32_t* gi = a.cidx + (pi * nreg + r) * (int64_t)CT;
    const int per = (c_r + FR - 1) / FR;
    const int e0 = min(tid * per, c_r), e1 = min(e0 + per, c_r);
    uint32_t m = 0;
    for (int e = e0; e < e1; ++e) m += !bits && (inlds ? L.key[o_r + e] : gk[e]) == T ? 1u : 0u;
    uint32_t mt;
    uint32_t rank = eq_seen + block_scan<FR>(m, L.s.wsum, &mt) - m;
    for (int e = e0; e < e1; ++e) {
      const uint64_t key = inlds ? L.key[o_r + e] : gk[e];
      const bool eq = !bits && key == T;
      if (chosen(key, eq && rank < (uint32_t)krem)) {
        const int it = inlds ? L.idx[o_r + e] : gi[e];
        atomicOr(&L.bm[(it >> 5) - r * RW], 1u << (it & 31));
      }
      rank += eq ? 1u : 0u;
    }
    eq_seen += mt;
    lds_sync();
    // emission in ascending order from off
    uint32_t wbits = tid < RW ? L.bm[tid] : 0u;
    const uint32_t pc = (uint32_t)__popc(wbits);
    uint32_t tot;
    int pos = off + (int)(block_scan<FR>(pc, L.s.wsum, &tot) - pc);
    while (wbits) {
      const int j = __ffs(wbits) - 1;
      wbits &= wbits - 1u;
      if (pos < a.k_max) out[pos] = 32 * (r * RW + tid) + j;
      ++pos;
    }
    off += (int)tot;
  }
  if (r0 == 0)   // the first workgroup pads
    for (int e = k + tid; e < a.k_max; e += FR) out[e] = -1;
}

}  // namespace

// Histogram slots a pair has room for: the counting grids give a pair at most
// this many workgroups (about four resident a CU over all pairs, NSLOT at most).
int topk_slots(const kvc_cache& c) {
  const int64_t pairs = (int64_t)c.batch * c.num_kv_heads;
  return (int)std::max<int64_t>(1, std::min<int64_t>(NSLOT, (4 * (int64_t)CUS + pairs - 1) / pairs));
}

size_t topk_workspace_bytes(const kvc_cache& c) {
  const size_t pairs = (size_t)c.batch * c.num_kv_heads;
  const size_t words = c.max_tokens / 32;
  const size_t nreg = (c.max_tokens + CT - 1) / CT;   // (token items: the most regions)
  size_t bytes = 2 * pairs * c.max_tokens * sizeof(uint64_t);   // keys, block-mode token scores
  bytes += pairs * topk_slots(c) * HWS * sizeof(uint32_t);       // histogram slots
  bytes += pairs * words * sizeof(uint32_t);                     // above bitmap
  bytes += pairs * nreg * CT * (sizeof(uint64_t) + sizeof(int32_t));   // threshold-bin lists
  bytes += 2 * pairs * nreg * sizeof(int32_t);                   // per-region counts
  bytes += 2 * pairs * sizeof(int32_t);                          // threshold bin, count above
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
  a.use_hist = items > DIRECT_MAX;
  char* p = static_cast<char*>(ws);
  a.keys = reinterpret_cast<uint64_t*>(p);
  p += pairs * c.max_tokens * sizeof(uint64_t);
  a.tscore = reinterpret_cast<double*>(p);
  p += pairs * c.max_tokens * sizeof(double);
  a.hist = reinterpret_cast<uint32_t*>(p);
  p += pairs * topk_slots(c) * HWS * sizeof(uint32_t);
  a.above = reinterpret_cast<uint32_t*>(p);
  p += pairs * words * sizeof(uint32_t);
  a.ckey = reinterpret_cast<uint64_t*>(p);
  p += pairs * nreg_ws * CT * sizeof(uint64_t);
  a.cidx = reinterpret_cast<int32_t*>(p);
  p += pairs * nreg_ws * CT * sizeof(int32_t);
  a.ccount = reinterpret_cast<int32_t*>(p);
  p += pairs * nreg_ws * sizeof(int32_t);
  a.acount = reinterpret_cast<int32_t*>(p);
  p += pairs * nreg_ws * sizeof(int32_t);
  a.pmeta = reinterpret_cast<int32_t*>(p);

  const int Hkv = c.num_kv_heads, B = c.batch;
  // scoring grid: as many workgroups as are resident at once (per_cu a CU,
  // from the kernel's registers and LDS), split evenly over the pairs; each
  // loops over its chunks
  // (at most topk_slots workgroups a pair: one histogram slot each)
  const int slots = topk_slots(c);
  auto score_grid = [&](int chunks, int per_cu) {
    const int64_t per_pair =
        std::max<int64_t>(1, ((int64_t)CUS * per_cu + (int64_t)pairs - 1) / (int64_t)pairs);
    const dim3 gr((unsigned)std::min<int64_t>(std::min<int64_t>(chunks, per_pair), slots), Hkv, B);
    if (!a.blocks) a.nslot = (int)gr.x;
    return gr;
  };
  const int vchunks = (c.max_tokens + SCT * TPT - 1) / (SCT * TPT);
  // the channel-major copy serves fp16 and FP8 caches (FP8: kT holds the decoded
  // values); quantized caches score their codes
  const bool kt = c.kT && c.page_size == 0 && (c.format == KVC_FMT_FP16 || c.format == KVC_FMT_FP8);
  if (mode == KVC_SCORE_EXTERNAL) {
    const dim3 grid = score_grid(vchunks, 2);   // (sets a.nslot before a is passed)
    score_ext_kernel<<<grid, SCT, 0, s>>>(a);
  } else if (mode == KVC_SCORE_CRITICAL && kt && (a.G == 1 || a.G == 2 || a.G == 4)) {
    const size_t sq_bytes = (size_t)a.G * n_crit * sizeof(double);
    const dim3 grid = score_grid(vchunks, a.G == 4 ? 1 : 2);
    if (a.G == 1) score_kt_kernel<1><<<grid, SCT, sq_bytes, s>>>(a);
    else if (a.G == 2) score_kt_kernel<2><<<grid, SCT, sq_bytes, s>>>(a);
    else score_kt_kernel<4><<<grid, SCT, sq_bytes, s>>>(a);
  } else {
    const bool exact = mode == KVC_SCORE_EXACT;
    const int snt = exact || (a.G != 1 && a.G != 2 && a.G != 4) ? ST : SCT;
    const dim3 sgrid = score_grid((c.max_tokens + snt - 1) / snt, snt == SCT ? 1 : 4);
    // the scorer's q operands in LDS: G heads x the channels it sums over
    const size_t sq_bytes = (size_t)a.G * (exact ? D : n_crit) * sizeof(double);
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
    else if (kt) KVC_SCORE_G(KVC_FMT_FP16, true);
    else if (c.format == KVC_FMT_FP8) KVC_SCORE_G(KVC_FMT_FP8, false);
    else KVC_SCORE_G(KVC_FMT_FP16, false);
#undef KVC_SCORE_G
#undef KVC_SCORE_E
  }
  if (a.blocks) {
    const int nchunk = (c.max_tokens / GS + BPW - 1) / BPW;
    const dim3 bg((unsigned)std::min(nchunk, slots), Hkv, B);
    a.nslot = (int)bg.x;
    block_key_kernel<<<bg, ST, 0, s>>>(a);
  }
  if (items > DIRECT_MAX) {
    compact_kernel<<<dim3(a.nreg, Hkv, B), ST, 0, s>>>(a);
    // finish: regions split over as many workgroups as are resident at once
    // (two a CU, by LDS), up to RPW_MAX regions each
    const int64_t per_pair = std::max<int64_t>(1, (2 * (int64_t)CUS) / (int64_t)pairs);
    const int rpw = (int)std::min<int64_t>(RPW_MAX, (a.nreg + per_pair - 1) / per_pair);
    finish_region_kernel<<<dim3((a.nreg + rpw - 1) / rpw, Hkv, B), FR, 0, s>>>(a, rpw);
  } else {
    finish_direct_kernel<<<dim3(Hkv, B), FT, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvc
