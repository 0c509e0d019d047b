// Fused dequantize -> QK^T -> softmax -> PV decode attention with GQA
// (on-device KV article, section 3.2: one fused kernel with scales and zero
// points held on chip; meeting-LLM article, section 8.1: online softmax over
// the active blocks; TailorKV article, section 2.1: softmax(QK^T / sqrt(d))).
//
// One launch covers a whole call.  Workgroup (split, KV head g, sequence b)
// takes one of two roles:
//   * quantized role (splits [0, s_q), INT4/INT1 caches): each wave walks a run
//     of complete 64-token groups straight from the code tiles;
//   * fp16-rows role (splits [s_q, s_total)): fp16 rows -- the whole cache of
//     an fp16 cache, the tail of a quantized one, the gathered tokens of the
//     drop mode, the fp16 keep set of the keep mode.
// Each workgroup writes one split partial (max, sum, unnormalized output) per
// query head; a merge kernel combines the splits with a log-sum-exp.
//
// Quantized role, per 64-token group, for query head h and channel c:
//   k~ = code * s_c + z_c  =>  q . k~ = sum_c (q_c s_c) code_c + sum_c q_c z_c.
// q'_c = q_c s_c is formed once per group as an exact fp16 pair hi + lo
// (hi = fp16(q s), lo = fma(q, s, -hi)); hi sits in matrix columns [0, G) and
// lo in columns [8, 8 + G) of the 16-wide B operand, so one 16x16x32 MFMA per
// 32 channels yields both and a row rotation adds them.  Codes enter the MFMA
// as fp16 "base + code" values built by one mask-and-or per code pair (bases
// 256/16 by nibble position for INT4, 16/8/4/2 by bit position for INT1).  Two more MFMAs per 32 channels give each tile its starting value
// sum_c q_c z_c - sum_c q'_c base_c.  For P.V the output is computed
// transposed, O^T = V^T P'^T, so a lane's accumulator column is its own query
// head; P' = p * s_v per token and V half.  sum_t p z_v is kept on the vector
// unit and sum_t P'_t base_t on the matrix cores beside the output.  When a KV
// head serves at most 4 query heads, the softmax of the four tiles of a group
// runs packed into all 64 lanes (tile j in lanes 4j..4j+3 of each row).

#include <math.h>

#include <atomic>
#include <mutex>

#include "internal.h"

namespace kvc {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Waves per workgroup.  One workgroup per CU either way; the 1-bit layer's
// per-group work is arithmetic more than bytes, so it runs two waves per SIMD
// to overlap one wave's latencies with another's work.
constexpr int waves_per_wg(int fmt) { return fmt == KVC_FMT_INT1 ? 8 : 4; }
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr int PART = 4 + D;    // floats per split partial: m (log2 units), l, pad, o[128]
constexpr int PO = 4;          // offset of o inside a partial (16-byte aligned)

struct AttendArgs {
  kvc_cache c;
  const uint16_t* q;
  int hq, G;
  float sm, sm2;              // sm_scale and sm_scale * log2(e)
  int mode;
  const int32_t* sel;
  int k_max, n_sink, n_window;
  float* logits;
  int64_t logits_stride;
  float* part;                // [B][Hq][s_total][PART]
  uint32_t* sbits;            // drop/keep: [B][Hkv][max_tokens/32] valid sel entries as bits
  int32_t* spre;              // drop/keep: [B][Hkv][max_tokens/32] sel index of the word's first token
  int2* rplan;                // drop/keep: [B][Hkv][np] fp16-rows role plan entries
  int np;                     // drop/keep: positions per (sequence, KV head) of the fp16-rows role
  int nsel;                   // positions of the selection (k_max; 64 k_max in blocks mode)
  int inline_plan;            // drop / blocks on a contiguous fp16 / FP8 cache: the rows role
                              // derives its positions from sel itself (no plan kernel)
  int32_t* glist;             // blocks mode, INT4/INT1: [B][Hkv][max_tokens/64] groups to walk
  int32_t* gcount;            // blocks mode, INT4/INT1: [B][Hkv] their number
  int32_t* kfill;             // keep mode: [B][Hkv] sel entries before the -1 padding (the
                              // fp16-rows role skips the padding's positions)
  int s_q, s_total;
  int ppw;                    // rows role: positions per wave (multiple of 16)
  int gpw;                    // quantized role: planned groups per wave
  int pairs;                  // B * Hkv
  PageDiv pd;                 // token -> page division of the cache
};

template <typename T, typename F>
__device__ inline T bc(const F& f) { return __builtin_bit_cast(T, f); }

// Buffer resource over bytes [p, p + n) (raw 32-bit buffer, gfx9 data-format
// word): a vector load through it that falls outside the range reads zero and
// never reaches memory.  Group loads use one resource per contiguous run, so
// all address arithmetic stays scalar and a lane's offset is a loop-invariant
// register.
typedef __amdgpu_buffer_rsrc_t Buf;
__device__ inline Buf make_buf(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)n, 0x00020000);
}
// Code tiles are read once per call: nontemporal loads (cache policy bit 1)
// keep them from displacing reused lines in the caches.
__device__ inline uint4 buf_load16_stream(Buf r, uint32_t off) {
  return bc<uint4>(__builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
__device__ inline uint2 buf_load8(Buf r, uint32_t off) {
  return bc<uint2>(__builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

__device__ inline float ror8(float x) {   // value of lane (l +- 8) within its row of 16
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}
// Sums / maxima over lanes l, l^16, l^32, l^48 with the gfx950 row-swap moves
// (no LDS round trip): each swap of a value with itself yields the value and
// its partner lane's value.
__device__ inline float sum_kb(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ inline float max_kb(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
// LDS accesses of one wave execute in issue order, so exchanging data through
// LDS inside a wave only needs the compiler to keep program order.
__device__ inline void wave_sync_lds() { asm volatile("" ::: "memory"); }

// exp2 on the transcendental unit (inputs here are <= 0; results below 2^-126
// flush to zero, which the softmax sums cannot see).
__device__ inline float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// A loop-invariant constant held in a VGPR, so the mask-and-or decodes below
// assemble to single three-operand VALU ops (gfx9 VOP3 takes no literals).
__device__ inline uint32_t vconst(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// INT1 dword -> word (variant v, position r): bit pair (6 + r, 22 + r) of the
// v-th shifted copy, with fp16 base 2^(4 - r) so each value is base + bit.
// mask[r] = 0x00400040 << r and base[r] = 0x4C004C00 - 0x04000400 * r in VGPRs.
__device__ inline uint32_t dec1_word(uint32_t u, int v, int r, const uint32_t* mask,
                                     const uint32_t* base) {
  const uint32_t s = v == 0 ? u : v == 1 ? (u >> 4) : v == 2 ? (u << 4) : __builtin_amdgcn_alignbit(u, u, 24);
  return (s & mask[r]) | base[r];
}

__device__ inline f4 mfma32(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ inline h8 cat(h4 a, h4 b) { return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

__device__ inline int sel_key(int e) { return e < 0 ? INT_MAX : e; }

// First index in sel[0, k) whose key is >= t (sel ascending, -1 padding last).
__device__ inline int lower_bound_sel(const int32_t* sel, int k, int t) {
  int lo = 0, hi = k;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sel_key(sel[mid]) < t) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Drop and blocks modes attend a compact set (sinks, selection, window) whose
// logits positions follow the selection; keep mode attends every token.
__device__ inline bool compact(int mode) { return mode == KVC_ATTEND_DROP || mode == KVC_ATTEND_BLOCKS; }

// Window start of the drop/keep sets.
__device__ inline int window_start(int n, int n_sink, int n_window) {
  return max(n - n_window, min(n_sink, n));
}

// ---------------------------------------------------------------- quantized role
// Raw loads of one 64-token group: code tiles, metadata words, selection bits.
// TILED: the group's four 16-token tiles are addressed one by one (pages of
// 16 or 32 tokens); otherwise the group is one contiguous run of slots.
// OUTL: INT4 with outlier channels; ko / vo hold the K / V outlier-store
// entries of token l of the group in lane l (vo zero without a V store).
template <int FMT, bool TILED, bool OUTL = false>
struct GroupData {
  uint4 k[FMT == KVC_FMT_INT4 ? 4 : 1];
  uint4 v[FMT == KVC_FMT_INT4 ? 4 : 1];
  uint2 ko, vo;
  uint2 km;
  uint2 vm[TILED ? 4 : 1];   // TILED: tile j's words in lanes 16j..16j+15, zero elsewhere
  uint2 bits;   // drop/keep: selected tokens of the group (two 32-token words)
};

// Per-wave running state of the quantized role.  m is the running maximum of
// the raw score q.k~ for the lane's head; the rest is relative to exp2(m * sm2).
struct QState {
  float m, l, sz0, sz1;
  float vo[4];      // sum_t p_t * V outlier entry e (isolated V outlier channels)
  f4 acc[8];        // O^T, channel tiles 0..7 (lane column = head)
  f4 corr0, corr1;  // sum_t P'_t * base_t per V half, replicated over rows
};

// Code decoders.  Each pair of codes becomes an fp16 pair "base + code" with
// one mask-and-or; the bases (per slot) are removed later by the matrix cores.
//  INT4 dword (nibble slot j at bit 16*(j&1) + 4*(j>>1)): slots 0,1 and 4,5
//   move to mantissa bits 2-5 (base 256), slots 2,3 and 6,7 to bits 6-9
//   (base 16), from two shifted copies of the dword.  For keys the 8 slots are
//   8 channels; for values slots 0-3 are tokens 0-3 of channel tile 2d and
//   slots 4-7 the same tokens of tile 2d + 1.
//  INT1: see dec1_word.
struct Dec {
  uint32_t mlo, mhi, blo, bhi;
  uint32_t m1[4], b1[4];
};
__device__ inline Dec make_decoder() {
  Dec d;
  d.mlo = vconst(0x003C003Cu);
  d.mhi = vconst(0x03C003C0u);
  d.blo = vconst(0x5C005C00u);   // fp16 256.0
  d.bhi = vconst(0x4C004C00u);   // fp16 16.0
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    d.m1[r] = vconst(0x00400040u << r);
    d.b1[r] = vconst(0x4C004C00u - 0x04000400u * (uint32_t)r);
  }
  return d;
}
__device__ inline uint4 dec4(uint32_t u, const Dec& dc) {
  const uint32_t a = u << 2, b = u >> 6;
  return uint4{(a & dc.mlo) | dc.blo, (a & dc.mhi) | dc.bhi, (b & dc.mlo) | dc.blo,
               (b & dc.mhi) | dc.bhi};
}
__device__ inline h8 dec4k(uint32_t u, const Dec& dc) { return bc<h8>(dec4(u, dc)); }
__device__ inline void dec4v(uint32_t u, const Dec& dc, h4& va, h4& vb) {
  const uint4 w = dec4(u, dc);
  va = bc<h4>(uint2{w.x, w.y});
  vb = bc<h4>(uint2{w.z, w.w});
}
__device__ inline uint32_t dec1w(uint32_t u, int v, int r, const Dec& dc) {
  return dec1_word(u, v, r, dc.m1, dc.b1);
}

// Read-only tables that every lane indexes alike are read through the scalar
// cache (constant address space), keeping them off the vector-memory counter
// that orders the code-tile prefetches.
template <typename T>
__device__ inline const __attribute__((address_space(4))) T* scalar_ptr(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}

// Page-table words for group gi of sequence b: the entries of the group's
// first page and the three after it, one 16-byte load through a buffer over
// the sequence's table row (a contiguous cache has none).
// The quantized role issues it a group ahead of the group's code loads, so
// the table lookup is off the loads' critical path.
__device__ inline uint4 group_table(const AttendArgs& a, Buf rtab, int gi) {
  if (a.c.page_size == 0) return uint4{0u, 0u, 0u, 0u};   // (uniform: no load at all)
  const int page0 = page_of(a.pd, gi * GS);
  return bc<uint4>(__builtin_amdgcn_raw_buffer_load_b128(rtab, (int)(4u * (uint32_t)page0), 0, 0));
}

// Slot of token t of group gi (t in the group, the same t in every lane) from
// the group's table words; -1 for a page outside the pool.
__device__ inline int64_t group_slot(const AttendArgs& a, int b, int g, int gi, int t, uint4 tw) {
  const kvc_cache& c = a.c;
  if (c.page_size == 0) return ((int64_t)b * c.num_kv_heads + g) * (int64_t)c.max_tokens + t;
  const int page = page_of(a.pd, t);
  const int e = page - page_of(a.pd, gi * GS);   // 0..3
  const uint32_t w = e == 0 ? tw.x : e == 1 ? tw.y : e == 2 ? tw.z : tw.w;
  const int phys = (int)__builtin_amdgcn_readfirstlane(w);
  const bool ok = page < c.max_pages && phys >= 0 && phys < c.num_pages;
  return ok ? ((int64_t)phys * c.num_kv_heads + g) * (int64_t)a.pd.P + (t - page * a.pd.P) : -1;
}

// Loads of group gi: a fixed set of vector loads with no branch between them,
// so the wait before a group's first use leaves the next group's loads in
// flight.  live == false (a group past the wave's last) and a page outside the
// pool give empty ranges: the loads read zero without touching memory.
template <int FMT, bool DENSE, bool TILED, bool OUTL = false>
__device__ __forceinline__ void load_group(const AttendArgs& a, int b, int g, int gi, bool live,
                                           uint4 tw, int lane, GroupData<FMT, TILED, OUTL>& d) {
  const kvc_cache& c = a.c;
  const int t0 = gi * GS;
  const uint32_t l16 = 16u * lane, l8 = 8u * lane;
  constexpr uint32_t OB = KVC_MAX_OUTLIERS * 2;   // outlier-store bytes per slot (= 8)
  if constexpr (!TILED) {   // 64 consecutive slots: one range per array
    const int64_t s0 = group_slot(a, b, g, gi, t0, tw);
    const bool ok = live && s0 >= 0;
    const int64_t sl = ok ? s0 : 0;
    const int64_t unit = FMT == KVC_FMT_INT4 ? (sl >> 4) : (sl >> 6);
    constexpr uint32_t run = FMT == KVC_FMT_INT4 ? 4 * UNIT_BYTES : UNIT_BYTES;
    const Buf rk = make_buf(c.k_codes + unit * UNIT_BYTES, ok ? run : 0u);
    const Buf rv = make_buf(c.v_codes + unit * UNIT_BYTES, ok ? run : 0u);
#pragma unroll
    for (int j = 0; j < (FMT == KVC_FMT_INT4 ? 4 : 1); ++j) {
      d.k[j] = buf_load16_stream(rk, l16 + j * UNIT_BYTES);
      d.v[j] = buf_load16_stream(rv, l16 + j * UNIT_BYTES);
    }
    d.vm[0] = buf_load8(make_buf(c.v_meta + sl * 4, ok ? GS * 8u : 0u), l8);
    if constexpr (OUTL) {
      d.ko = buf_load8(make_buf(c.k_outlier + sl * KVC_MAX_OUTLIERS, ok ? GS * OB : 0u), l8);
      const bool vok = ok && c.v_outlier;
      d.vo = buf_load8(make_buf((vok ? c.v_outlier : c.k_outlier) + sl * KVC_MAX_OUTLIERS, vok ? GS * OB : 0u), l8);
    }
  } else {                  // INT4 tiles on pages of 16 or 32 tokens
    int64_t st[4];
    bool ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      st[j] = group_slot(a, b, g, gi, t0 + TILE * j, tw);
      ok[j] = live && st[j] >= 0;
      if (!ok[j]) st[j] = 0;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d.k[j] = buf_load16_stream(make_buf(c.k_codes + (st[j] >> 4) * UNIT_BYTES, ok[j] ? UNIT_BYTES : 0u), l16);
      d.v[j] = buf_load16_stream(make_buf(c.v_codes + (st[j] >> 4) * UNIT_BYTES, ok[j] ? UNIT_BYTES : 0u), l16);
    }
    // lanes of other tiles fall outside tile j's 128-byte range (and read zero)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      d.vm[j] = buf_load8(make_buf(c.v_meta + st[j] * 4, ok[j] ? TILE * 8u : 0u), l8 - 128u * j);
    if constexpr (OUTL) {   // (as the V metadata: lanes of other tiles read zero)
      d.ko = d.vo = uint2{0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 o = buf_load8(make_buf(c.k_outlier + st[j] * KVC_MAX_OUTLIERS, ok[j] ? TILE * OB : 0u),
                                  l8 - TILE * OB * j);
        d.ko = uint2{d.ko.x | o.x, d.ko.y | o.y};
        const bool vok = ok[j] && c.v_outlier;
        const uint2 u = buf_load8(make_buf((vok ? c.v_outlier : c.k_outlier) + st[j] * KVC_MAX_OUTLIERS,
                                           vok ? TILE * OB : 0u), l8 - TILE * OB * j);
        d.vo = uint2{d.vo.x | u.x, d.vo.y | u.y};
      }
    }
  }
  const uint16_t* km = c.k_meta +
      ((((int64_t)b * c.num_kv_heads + g) * (c.max_tokens / GS) + gi) * 2) * D;
  d.km = buf_load8(make_buf(km, live ? 2 * D * 2u : 0u), l8);
  if constexpr (!DENSE) {
    const int words = c.max_tokens / 32;
    const auto* sb = scalar_ptr(a.sbits + ((int64_t)b * c.num_kv_heads + g) * words + 2 * gi);
    d.bits = uint2{sb[0], sb[1]};
  }
}

// Value from lane (l - 4k) of the same 16-lane row into lanes of bank k only.
template <int K>
__device__ inline float put_bank(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x),
                                                    0x110 + 4 * K, 0xF, 1 << K, false));
}
// Word of lane (l + 4k) of the same row (0 past the row's end).
template <int K>
__device__ inline uint32_t take_bank(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x100 + 4 * K, 0xF, 0xF, true);
}
__device__ inline float ror4(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
}

// Isolated V outlier channels: p_i times the four fp16 entries of token i of
// a lane's quad of consecutive tokens (staged in LDS, 32 bytes) into the
// running sums.
__device__ inline void vo_accum(QState& st, const float* p, const uint16_t* quad) {
  const uint4 e0 = *reinterpret_cast<const uint4*>(quad);
  const uint4 e1 = *reinterpret_cast<const uint4*>(quad + 8);
  const uint32_t w[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 e01 = bc<h2>(w[2 * i]), e23 = bc<h2>(w[2 * i + 1]);
    st.vo[0] = fmaf(p[i], (float)e01.x, st.vo[0]);
    st.vo[1] = fmaf(p[i], (float)e01.y, st.vo[1]);
    st.vo[2] = fmaf(p[i], (float)e23.x, st.vo[2]);
    st.vo[3] = fmaf(p[i], (float)e23.y, st.vo[3]);
  }
}

template <int FMT, bool DENSE, bool LOGITS, bool PACK, bool TILED, bool OUTL = false>
__device__ __forceinline__ void group_body(const AttendArgs& a, int b, int g, int gi, int lane,
                                           int w, int n, const GroupData<FMT, TILED, OUTL>& d,
                                           QState& st, const h2* qv, const h8& qo, const Dec& dc,
                                           uint16_t* sKm, uint16_t* sVm, uint16_t* sVo) {
  const int G = a.G;
  const int col = lane & 15, kb = lane >> 4, head = col & 7;
  const bool hv = head < G;
  const bool hi_lane = hv && col < 8;
  const uint32_t lo_sel = (hv && !hi_lane) ? 0xFFFFFFFFu : 0u;  // lo lanes subtract hi
  const int t0 = gi * GS;

  // ---- which tokens of this group are attended from the codes
  uint64_t att = ~0ull;
  const int w0 = window_start(n, a.n_sink, a.n_window);
  const uint64_t selm = DENSE ? 0ull : ((uint64_t)d.bits.x | ((uint64_t)d.bits.y << 32));
  if constexpr (!DENSE) {
    const int tl = t0 + lane;
    const uint64_t inset = __ballot(tl < a.n_sink || tl >= w0) | selm;
    att = a.mode != KVC_ATTEND_KEEP ? inset : ~inset;
    if (att == 0) return;
  }

  // ---- stage K scales and zeros / 2 (zeros are added back doubled, see bias) and V metadata
  {
    uint2 km = d.km;
    if (lane >= 32) {   // halves 128..255 are the zeros
      const h2 half = h2{(_Float16)0.5f, (_Float16)0.5f};
      km.x = bc<uint32_t>(bc<h2>(km.x) * half);
      km.y = bc<uint32_t>(bc<h2>(km.y) * half);
    }
    *reinterpret_cast<uint2*>(sKm + 256 * w + 4 * lane) = km;
    uint2 vm = d.vm[0];
    if constexpr (TILED) {
#pragma unroll
      for (int j = 1; j < 4; ++j) vm = uint2{vm.x | d.vm[j].x, vm.y | d.vm[j].y};
    }
    *reinterpret_cast<uint2*>(sVm + 256 * w + 4 * lane) = vm;
    if constexpr (OUTL) *reinterpret_cast<uint2*>(sVo + 256 * w + 4 * lane) = d.vo;
  }
  wave_sync_lds();

  // ---- q' = q * s as fp16 hi (columns < 8) / lo (columns >= 8); per-group bias on the MFMA:
  //      columns get sum_c (z/2) q (hi and lo alike, so they add to sum z q) minus sum_c base_c q'
  h8 qp[4];
  f4 bias = f4{0.f, 0.f, 0.f, 0.f};
  {
    const uint16_t* ks = sKm + 256 * w;
    h8 nbase;
    if constexpr (FMT == KVC_FMT_INT4) {
      const _Float16 x = (_Float16)-256.f, y = (_Float16)-16.f;
      nbase = h8{x, x, y, y, x, x, y, y};
    } else {
      nbase = h8{(_Float16)-16.f, (_Float16)-16.f, (_Float16)-8.f, (_Float16)-8.f,
                 (_Float16)-4.f, (_Float16)-4.f, (_Float16)-2.f, (_Float16)-2.f};
    }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const uint4 s4 = *reinterpret_cast<const uint4*>(ks + 32 * kb + 8 * kc);
      const uint4 z4 = *reinterpret_cast<const uint4*>(ks + D + 32 * kb + 8 * kc);
      const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
      uint32_t out[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const h2 qq = qv[4 * kc + pr];
        const h2 ss = bc<h2>(sw[pr]);
        const h2 hi = qq * ss;
        const h2 sub = bc<h2>(bc<uint32_t>(hi) & lo_sel);
        out[pr] = bc<uint32_t>(__builtin_elementwise_fma(qq, ss, -sub));
      }
      qp[kc] = bc<h8>(uint4{out[0], out[1], out[2], out[3]});
      const h8 qk = bc<h8>(uint4{bc<uint32_t>(qv[4 * kc]), bc<uint32_t>(qv[4 * kc + 1]),
                                 bc<uint32_t>(qv[4 * kc + 2]), bc<uint32_t>(qv[4 * kc + 3])});
      bias = mfma32(bc<h8>(z4), qk, bias);
      bias = mfma32(nbase, qp[kc], bias);
    }
  }

  // ---- S^T = codes x q'^T per 16-token tile; hi + lo columns added (raw units).
  // Outlier channels (scale and zero 0 in the main store) add one more product
  // per tile: A = the group's fp16 outlier entries (lane l: token l, in row
  // l % 16 at k = 8 (l / 16) + e; entries past the list masked to 0), and
  // B = q on those channels in the hi columns of the lanes whose k block is
  // the tile (qo, zero elsewhere), so tile j's rows take only tokens 16j + n.
  h8 ao = h8{};
  if constexpr (OUTL) {
    const int m = a.c.n_outlier;
    const uint32_t om0 = m >= 2 ? 0xFFFFFFFFu : (m == 1 ? 0xFFFFu : 0u);
    const uint32_t om1 = m >= 4 ? 0xFFFFFFFFu : (m == 3 ? 0xFFFFu : 0u);
    ao = bc<h8>(uint4{d.ko.x & om0, d.ko.y & om1, 0u, 0u});
  }
  float x[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f4 s = bias;
    if constexpr (OUTL) {
      const uint32_t sel = (lane >> 4) == j ? 0xFFFFFFFFu : 0u;
      const uint4 qb = bc<uint4>(qo);
      s = mfma32(ao, bc<h8>(uint4{qb.x & sel, qb.y & sel, 0u, 0u}), s);
    }
    if constexpr (FMT == KVC_FMT_INT4) {
      s = mfma32(dec4k(d.k[j].x, dc), qp[0], s);
      s = mfma32(dec4k(d.k[j].y, dc), qp[1], s);
      s = mfma32(dec4k(d.k[j].z, dc), qp[2], s);
      s = mfma32(dec4k(d.k[j].w, dc), qp[3], s);
    } else {
      const uint32_t u = j == 0 ? d.k[0].x : j == 1 ? d.k[0].y : j == 2 ? d.k[0].z : d.k[0].w;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint4 wv = uint4{dec1w(u, kc, 0, dc), dec1w(u, kc, 1, dc), dec1w(u, kc, 2, dc),
                               dec1w(u, kc, 3, dc)};
        s = mfma32(bc<h8>(wv), qp[kc], s);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) x[j][i] = s[i] + ror8(s[i]);
  }

  // ---- logits (natural units) of the attended tokens: one store per (token,
  // head); with the packed softmax they are written from the packed scores
  // below (all 64 lanes, four tokens each), otherwise here from the hi lanes
  int32_t pre0 = 0, pre1 = 0;   // sel index of the group's two 32-token words (drop mode)
  if constexpr (LOGITS) {
    if (!DENSE && compact(a.mode)) {
      const auto* sp = scalar_ptr(a.spre + ((int64_t)b * a.c.num_kv_heads + g) * (a.c.max_tokens / 32) + 2 * gi);
      pre0 = sp[0];
      pre1 = sp[1];
    }
  }
  // logit of token t0 + bit for query head hh (bit attended)
  auto put_logit = [&](int bit, int hh, float xv) {
    int pos = t0 + bit;
    if (compact(a.mode)) {
      const int t = t0 + bit;
      if (t < a.n_sink) {
        pos = t;
      } else if (t >= w0) {
        pos = a.n_sink + a.nsel + (t - w0);
      } else {
        const uint32_t word = (bit >> 5) ? d.bits.y : d.bits.x;
        const int32_t base = (bit >> 5) ? pre1 : pre0;
        pos = a.n_sink + base + __popc(word & ((1u << (t & 31)) - 1u));
      }
    }
    a.logits[((int64_t)b * a.hq + g * G + hh) * a.logits_stride + pos] = xv * a.sm;
  };
  if constexpr (LOGITS && !PACK) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bit = TILE * j + 4 * kb + i;
        const bool on = DENSE || ((att >> bit) & 1ull);
        if (hi_lane && on) put_logit(bit, head, x[j][i]);
      }
  }

  const uint16_t* vmeta = sVm + 256 * w;
  h4 B0[4], B1[4];   // P' of each tile as the B operand of P.V (lane column = head)
  float pv[PACK ? 4 : 16];   // OUTL: the probabilities, for the V outlier sums after P.V
  if constexpr (PACK) {
    // ---- pack the four tiles into all 64 lanes: lane (4j + h, kb) takes head h of tile j
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = x[0][i];
      v = put_bank<1>(v, x[1][i]);
      v = put_bank<2>(v, x[2][i]);
      v = put_bank<3>(v, x[3][i]);
      y[i] = v;
    }
    const int jj = col >> 2;
    if constexpr (LOGITS) {   // lane (4 jj + h, kb): head h's scores of tokens 16 jj + 4 kb + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bit = TILE * jj + 4 * kb + i;
        const bool on = DENSE || ((att >> bit) & 1ull);
        if ((col & 3) < G && on) put_logit(bit, col & 3, y[i]);
      }
    }
    if constexpr (!DENSE) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!((att >> (TILE * jj + 4 * kb + i)) & 1ull)) y[i] = -INFINITY;
    }
    float gmax = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
    gmax = fmaxf(gmax, ror4(gmax));
    gmax = fmaxf(gmax, ror8(gmax));
    gmax = max_kb(gmax);
    const float m_new = fmaxf(st.m, gmax);
    if (__any(m_new > st.m)) {   // rescale only when some head's maximum grows
      const float alpha = st.m == -INFINITY ? 0.f : ex2((st.m - m_new) * a.sm2);
      st.m = m_new;
      st.l *= alpha;
      st.sz0 *= alpha;
      st.sz1 *= alpha;
      st.corr0 *= alpha;
      st.corr1 *= alpha;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) st.acc[ct] *= alpha;
      if constexpr (OUTL) {
#pragma unroll
        for (int e = 0; e < 4; ++e) st.vo[e] *= alpha;
      }
    }
    const float msc = st.m == -INFINITY ? 0.f : st.m * a.sm2;
    const uint4 m01 = *reinterpret_cast<const uint4*>(vmeta + 4 * (TILE * jj + 4 * kb));
    const uint4 m23 = *reinterpret_cast<const uint4*>(vmeta + 4 * (TILE * jj + 4 * kb + 2));
    const uint32_t mwd[8] = {m01.x, m01.y, m01.z, m01.w, m23.x, m23.y, m23.z, m23.w};
    h4 A0, A1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = ex2(fmaf(y[i], a.sm2, -msc));
      st.l += p;
      const h2 s01 = bc<h2>(mwd[2 * i]);
      const h2 z01 = bc<h2>(mwd[2 * i + 1]);
      A0[i] = (_Float16)(p * (float)s01.x);
      A1[i] = (_Float16)(p * (float)s01.y);
      st.sz0 = fmaf(p, (float)z01.x, st.sz0);
      st.sz1 = fmaf(p, (float)z01.y, st.sz1);
      if constexpr (OUTL) pv[i] = p;
    }
    // ---- unpack: tile j's P' back to lanes (h, kb)
    const uint2 a0 = bc<uint2>(A0), a1 = bc<uint2>(A1);
    B0[0] = A0;
    B1[0] = A1;
    B0[1] = bc<h4>(uint2{take_bank<1>(a0.x), take_bank<1>(a0.y)});
    B1[1] = bc<h4>(uint2{take_bank<1>(a1.x), take_bank<1>(a1.y)});
    B0[2] = bc<h4>(uint2{take_bank<2>(a0.x), take_bank<2>(a0.y)});
    B1[2] = bc<h4>(uint2{take_bank<2>(a1.x), take_bank<2>(a1.y)});
    B0[3] = bc<h4>(uint2{take_bank<3>(a0.x), take_bank<3>(a0.y)});
    B1[3] = bc<h4>(uint2{take_bank<3>(a1.x), take_bank<3>(a1.y)});
  } else {
    if constexpr (!DENSE) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((att >> (TILE * j + 4 * kb + i)) & 1ull)) x[j][i] = -INFINITY;
    }
    float gmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) gmax = fmaxf(gmax, x[j][i]);
    gmax = max_kb(gmax);
    const float m_new = fmaxf(st.m, gmax);
    if (__any(m_new > st.m)) {
      const float alpha = st.m == -INFINITY ? 0.f : ex2((st.m - m_new) * a.sm2);
      st.m = m_new;
      st.l *= alpha;
      st.sz0 *= alpha;
      st.sz1 *= alpha;
      st.corr0 *= alpha;
      st.corr1 *= alpha;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) st.acc[ct] *= alpha;
      if constexpr (OUTL) {
#pragma unroll
        for (int e = 0; e < 4; ++e) st.vo[e] *= alpha;
      }
    }
    const float msc = st.m == -INFINITY ? 0.f : st.m * a.sm2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 m01 = *reinterpret_cast<const uint4*>(vmeta + 4 * (TILE * j + 4 * kb));
      const uint4 m23 = *reinterpret_cast<const uint4*>(vmeta + 4 * (TILE * j + 4 * kb + 2));
      const uint32_t mwd[8] = {m01.x, m01.y, m01.z, m01.w, m23.x, m23.y, m23.z, m23.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = ex2(fmaf(x[j][i], a.sm2, -msc));
        st.l += p;
        const h2 s01 = bc<h2>(mwd[2 * i]);
        const h2 z01 = bc<h2>(mwd[2 * i + 1]);
        B0[j][i] = (_Float16)(p * (float)s01.x);
        B1[j][i] = (_Float16)(p * (float)s01.y);
        st.sz0 = fmaf(p, (float)z01.x, st.sz0);
        st.sz1 = fmaf(p, (float)z01.y, st.sz1);
        if constexpr (OUTL) pv[(4 * j + i) % (PACK ? 4 : 16)] = p;
      }
    }
  }

  // ---- O^T += V^T P'^T, two tiles (32 tokens) per MFMA: k slots 0-3 are
  // tile 2jp's tokens of the lane's quad, k slots 4-7 tile 2jp + 1's; the bases
  // of the V codes accumulate beside it
  h8 vbase;
  if constexpr (FMT == KVC_FMT_INT4) {
    const _Float16 x1 = (_Float16)256.f, x2 = (_Float16)16.f;
    vbase = h8{x1, x1, x2, x2, x1, x1, x2, x2};
  } else {
    const _Float16 one = (_Float16)1.f;
    vbase = h8{one, one, one, one, one, one, one, one};
  }
#pragma unroll
  for (int jp = 0; jp < 2; ++jp) {
    const int j0 = 2 * jp, j1 = 2 * jp + 1;
    const h8 P0 = cat(B0[j0], B0[j1]), P1 = cat(B1[j0], B1[j1]);
    st.corr0 = mfma32(vbase, P0, st.corr0);
    st.corr1 = mfma32(vbase, P1, st.corr1);
    if constexpr (FMT == KVC_FMT_INT4) {
      const uint32_t da_[4] = {d.v[j0].x, d.v[j0].y, d.v[j0].z, d.v[j0].w};
      const uint32_t db_[4] = {d.v[j1].x, d.v[j1].y, d.v[j1].z, d.v[j1].w};
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        h4 va0, vb0, va1, vb1;
        dec4v(da_[dd], dc, va0, vb0);
        dec4v(db_[dd], dc, va1, vb1);
        st.acc[2 * dd] = mfma32(cat(va0, va1), dd < 2 ? P0 : P1, st.acc[2 * dd]);
        st.acc[2 * dd + 1] = mfma32(cat(vb0, vb1), dd < 2 ? P0 : P1, st.acc[2 * dd + 1]);
      }
    } else {
      const uint32_t u0 = jp == 0 ? d.v[0].x : d.v[0].z;
      const uint32_t u1 = jp == 0 ? d.v[0].y : d.v[0].w;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int v = 2 * (ct >> 2), r = ct & 3;
        const uint4 wv = uint4{dec1w(u0, v, r, dc), dec1w(u0, v + 1, r, dc), dec1w(u1, v, r, dc),
                               dec1w(u1, v + 1, r, dc)};
        st.acc[ct] = mfma32(bc<h8>(wv), ct < 4 ? P0 : P1, st.acc[ct]);
      }
    }
  }
  // isolated V outlier channels, while the matrix cores run the products above
  if constexpr (OUTL) {
    if constexpr (PACK) {
      vo_accum(st, pv, sVo + 256 * w + 4 * (TILE * (col >> 2) + 4 * kb));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) vo_accum(st, pv + 4 * j, sVo + 256 * w + 4 * (TILE * j + 4 * kb));
    }
  }
}

template <int FMT, bool DENSE, bool LOGITS, bool PACK, bool TILED, bool OUTL = false>
__device__ __forceinline__ void quant_role(const AttendArgs& a, int b, int g, int split, int lane, int w,
                           float* sO, float* sML, uint16_t* sKm, uint16_t* sVm, uint16_t* sVo) {
  const kvc_cache& c = a.c;
  // blocks mode walks the plan's list of groups (sink groups, kept blocks,
  // window groups); the other modes walk every complete group
  const bool listed = !DENSE && a.mode == KVC_ATTEND_BLOCKS;
  const int64_t pair = (int64_t)b * c.num_kv_heads + g;
  const int G = a.G;
  const int col = lane & 15, kb = lane >> 4, head = col & 7;
  const bool hv = head < G;
  const bool hi_lane = hv && col < 8;
  // the waves of (b, g) take groups round-robin, so at any moment they read
  // one window of adjacent groups (long runs for the DRAM pages)
  constexpr int NW = waves_per_wg(FMT);
  const int ga = split * NW + w;
  // dense: all of the pair's waves share its groups; drop / keep (ragged
  // batches): a pair uses only the waves its length needs at the planned
  // groups per wave, so short sequences free their workgroups at once.
  // Dense walks wait for the length only after issuing their first two
  // groups (ga and ga + W whatever the length; a group below the capacity
  // lies in the allocation, and one past the length is never used), so its
  // latency overlaps theirs; the length load itself goes out first, ahead of
  // the groups' bytes.
  int n = c.seq_lens[b], ngroups = 0, W = a.s_q * NW, nmine = 0;
  int vlist = 0;
  if constexpr (!DENSE) {
    n = max(n, 0);
    ngroups = listed ? *scalar_ptr(a.gcount + pair) : n >> 6;
    W = min(W, NW * ((ngroups + NW * a.gpw - 1) / (NW * a.gpw)));
    nmine = ga < ngroups && ga < W ? (ngroups - 1 - ga) / W + 1 : 0;
    if (listed) nmine = min(nmine, 64);   // (the planner keeps it there)
    // (blocks mode: the k-th entry comes from lane k of vlist, one load per
    // wave; the planner keeps nmine <= 64)
    if (listed && lane < nmine) vlist = a.glist[pair * (c.max_tokens / GS) + ga + lane * W];
  }
  // k-th group of this wave; past the last one the loads of the last repeat
  // with empty ranges (no memory traffic), so every load is unconditional and
  // the compiler's wait before a group counts exactly (a wave with no group
  // names group 0, whose selection words are in range)
  auto gid = [&](int k) {
    if (nmine <= 0) return 0;
    const int kk = min(k, nmine - 1);
    return listed ? __builtin_amdgcn_readlane(vlist, kk) : ga + kk * W;
  };
  const int cap = c.max_tokens >> 6;
  const int gi0 = DENSE ? ga : gid(0), gi1 = DENSE ? ga + W : gid(1);
  const bool live0 = DENSE ? gi0 < cap : nmine > 0, live1 = DENSE ? gi1 < cap : nmine > 1;

  // page-table words of the first groups, then q of this lane's head
  // (channels [32kb, 32kb + 32) as fp16 pairs, zero off-head), then the first
  // two groups' code loads, all before q is waited for; the table words are
  // issued first so that waiting for them leaves q in flight
  const Buf rtab = make_buf(c.block_table + (int64_t)b * c.max_pages,
                            c.page_size > 0 ? (uint32_t)c.max_pages * 4u : 0u);
  uint4 t0w = group_table(a, rtab, gi0), t1w = group_table(a, rtab, gi1);
  uint4 raw[4] = {};
  if (hv) {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.hq + g * G + head) * D + 32 * kb);
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[k] = qp[k];
  }
  // q on the outlier channels: B operand of the outlier product (the heads'
  // hi columns, entries past the list 0)
  h8 qo = h8{};
  if constexpr (OUTL) {
    if (hi_lane) {
      const uint16_t* qh = a.q + ((int64_t)b * a.hq + g * G + head) * D;
      const auto* oc = scalar_ptr(c.outlier_ch + g * KVC_MAX_OUTLIERS);
#pragma unroll
      for (int e = 0; e < KVC_MAX_OUTLIERS; ++e)
        if (e < c.n_outlier) qo[e] = bc<_Float16>(qh[min(max((int)oc[e], 0), D - 1)]);
    }
  }
  GroupData<FMT, TILED, OUTL> d0, d1;
  load_group<FMT, DENSE, TILED, OUTL>(a, b, g, gi0, live0, t0w, lane, d0);
  load_group<FMT, DENSE, TILED, OUTL>(a, b, g, gi1, live1, t1w, lane, d1);
  if constexpr (DENSE) {
    asm volatile("" : "+v"(n) :: "memory");   // the length is waited for only here
    n = max(__builtin_amdgcn_readfirstlane(n), 0);
    ngroups = n >> 6;
    nmine = ga < ngroups ? (ngroups - 1 - ga) / W + 1 : 0;
  }
  t0w = group_table(a, rtab, gid(2));
  t1w = group_table(a, rtab, gid(3));
  // q is in registers before the group loop (so no wait inside the loop, where
  // the next group's loads are in flight, is spent on it); the memory clobber
  // keeps the group loads above issued first
#pragma unroll
  for (int k = 0; k < 4; ++k)
    asm volatile("" :: "v"(raw[k].x), "v"(raw[k].y), "v"(raw[k].z), "v"(raw[k].w) : "memory");
  h2 qv[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    qv[4 * k + 0] = bc<h2>(raw[k].x);
    qv[4 * k + 1] = bc<h2>(raw[k].y);
    qv[4 * k + 2] = bc<h2>(raw[k].z);
    qv[4 * k + 3] = bc<h2>(raw[k].w);
  }

  QState st;
  st.m = -INFINITY;
  st.l = st.sz0 = st.sz1 = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) st.vo[e] = 0.f;
  st.corr0 = st.corr1 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) st.acc[ct] = f4{0.f, 0.f, 0.f, 0.f};
  const Dec dc = make_decoder();

  // two-deep software pipeline: while group k computes, group k + 1 is in
  // flight.  Pairs of groups per trip and no exit inside a trip: the loop
  // header then sees the same loads pending from both of its predecessors,
  // and its wait leaves the newer group's loads in flight.
  int k = 0;
  for (; k + 2 <= nmine; k += 2) {
    group_body<FMT, DENSE, LOGITS, PACK, TILED, OUTL>(a, b, g, gid(k), lane, w, n, d0, st, qv, qo, dc, sKm, sVm, sVo);
    load_group<FMT, DENSE, TILED, OUTL>(a, b, g, gid(k + 2), k + 2 < nmine, t0w, lane, d0);
    t0w = group_table(a, rtab, gid(k + 4));
    group_body<FMT, DENSE, LOGITS, PACK, TILED, OUTL>(a, b, g, gid(k + 1), lane, w, n, d1, st, qv, qo, dc, sKm, sVm, sVo);
    load_group<FMT, DENSE, TILED, OUTL>(a, b, g, gid(k + 3), k + 3 < nmine, t1w, lane, d1);
    t1w = group_table(a, rtab, gid(k + 5));
  }
  if (k < nmine)
    group_body<FMT, DENSE, LOGITS, PACK, TILED, OUTL>(a, b, g, gid(k), lane, w, n, d0, st, qv, qo, dc, sKm, sVm, sVo);

  // ---- finish: sums over the lanes of each head, bases and zero points
  float l = st.l, sz0 = st.sz0, sz1 = st.sz1;
  float vo[4] = {st.vo[0], st.vo[1], st.vo[2], st.vo[3]};
  if constexpr (PACK) {   // lanes h, h+4, h+8, h+12 of each row hold head h
    l += ror4(l);
    l += ror8(l);
    sz0 += ror4(sz0);
    sz0 += ror8(sz0);
    sz1 += ror4(sz1);
    sz1 += ror8(sz1);
    if constexpr (OUTL) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vo[e] += ror4(vo[e]);
        vo[e] += ror8(vo[e]);
      }
    }
  }
  l = sum_kb(l);
  sz0 = sum_kb(sz0);
  sz1 = sum_kb(sz1);
  if constexpr (OUTL) {
#pragma unroll
    for (int e = 0; e < 4; ++e) vo[e] = sum_kb(vo[e]);
  }
  if (hi_lane) {
    float* o = sO + (w * 8 + head) * D;
    const float c0 = st.corr0[0], c1 = st.corr1[0];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const float scale = FMT == KVC_FMT_INT4 ? 1.f : (float)(16 >> (ct & 3));
      const float corr = ct < 4 ? sz0 - scale * c0 : sz1 - scale * c1;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[16 * ct + 4 * kb + i] = st.acc[ct][i] + corr;
    }
    // isolated V outlier channels: their output is the fp16 store's sum (the
    // codes' value there, the group zero, is replaced; same wave, so the LDS
    // stores land in program order)
    if constexpr (OUTL) {
      if (kb == 0 && c.v_outlier) {
        const auto* oc = scalar_ptr(c.outlier_ch + g * KVC_MAX_OUTLIERS);
#pragma unroll
        for (int e = 0; e < KVC_MAX_OUTLIERS; ++e)
          if (e < c.n_outlier) o[min(max((int)oc[e], 0), D - 1)] = vo[e];
      }
    }
    if (kb == 0) {
      sML[(w * 8 + head) * 2] = st.m == -INFINITY ? -INFINITY : st.m * a.sm2;
      sML[(w * 8 + head) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------- fp16-rows role
// Row plan entry of one position of the fp16-rows role, {code, slot}:
//   code >= 0   token `code`, fp16 row `slot` of k16/v16;
//   code == -1  nothing to attend (another role owns the token, or no token);
//   code == -2  drop mode: the position holds no token (its logit is -inf);
//   code <= -3  token -3 - code, row `slot` of k_tail/v_tail.
// Slots fit in 32 bits: 2^31 fp16 rows would take 512 GB.
constexpr int ROW_SKIP = -1, ROW_NONE = -2;
__device__ inline int tail_code(int t) { return -3 - t; }
__device__ inline bool row_on(int code) { return code >= 0 || code <= -3; }

// True when token t is an entry of the ascending selection sel[0, k).
__device__ inline bool in_sel(const int32_t* sel, int k, int t) {
  const int i = lower_bound_sel(sel, k, t);
  return i < k && sel[i] == t;
}

// Plan entry of drop/keep position p of (b, g): the sinks, the selected
// tokens and the recent window (TailorKV article section 2.3, StreamingLLM /
// H2O survey section 3), then, in keep mode, the fp16 tail tokens outside the
// keep set (tail_in_sel: whether the tail token of position p is in sel).
template <bool QUANT>
__device__ inline int2 plan_entry(const AttendArgs& a, int b, int g, int n, int p, bool tail_in_sel) {
  const kvc_cache& c = a.c;
  // blocks mode on codes: the kept blocks are the quantized role's, so this
  // role's positions are the sinks and the window only (position p past the
  // sinks stands for logits position p + 64 k_max)
  if (QUANT && a.mode == KVC_ATTEND_BLOCKS && p >= a.n_sink) p += a.nsel;
  const int nq = QUANT ? (n & ~(GS - 1)) : 0;
  const int nset = a.n_sink + a.nsel + a.n_window;
  const int w0 = window_start(n, a.n_sink, a.n_window);
  const int32_t* sel = a.k_max > 0 ? a.sel + ((int64_t)b * c.num_kv_heads + g) * a.k_max : nullptr;
  const int tail_row = (b * c.num_kv_heads + g) * GS;
  if (p < nset) {
    int t;
    bool ok;
    if (p < a.n_sink) {
      t = p;
      ok = p < n;
    } else if (p < a.n_sink + a.nsel) {
      if (a.mode == KVC_ATTEND_BLOCKS) {   // token (p - n_sink) % 64 of kept block (p - n_sink) / 64
        const int blk = sel[(p - a.n_sink) / GS];
        ok = blk >= (a.n_sink + GS - 1) / GS && blk < max(n - a.n_window, 0) / GS;
        t = ok ? blk * GS + (p - a.n_sink) % GS : 0;
      } else {
        t = sel[p - a.n_sink];
        ok = t >= a.n_sink && t < n - a.n_window;
      }
    } else {
      t = w0 + (p - a.n_sink - a.nsel);
      ok = t < n;
    }
    if (!ok) return int2{compact(a.mode) ? ROW_NONE : ROW_SKIP, 0};
    if (compact(a.mode) && QUANT)   // older tokens come from the codes
      return t >= nq ? int2{tail_code(t), tail_row + (t - nq)} : int2{ROW_SKIP, 0};
    const int64_t sl = slot_fast(c, a.pd, b, g, t);
    return sl < 0 ? int2{ROW_SKIP, 0} : int2{t, (int)sl};
  }
  // keep mode: tail tokens outside the keep set
  const int t = nq + (p - nset);
  const bool ok = t < n && t >= a.n_sink && t < w0 && !tail_in_sel;
  return ok ? int2{tail_code(t), tail_row + (t - nq)} : int2{ROW_SKIP, 0};
}

// 32 E4M3 codes (two 16-byte words, channels in byte order) -> 32 fp16 values
// in four 16-byte words, two codes per conversion instruction (scale 1: every
// E4M3 value is exact in fp16).
template <bool HI>
__device__ inline uint32_t fp8_pair(uint32_t w) {
  return bc<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}
__device__ inline void fp8_row_decode(uint4 r0, uint4 r1, uint4* out) {
  const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = w[2 * i], b = w[2 * i + 1];
    out[i] = uint4{fp8_pair<false>(a), fp8_pair<true>(a), fp8_pair<false>(b), fp8_pair<true>(b)};
  }
}

// One 16-row tile in registers: lane (row, kb) holds 32 channels of its row,
// word k channels 32k + 8kb .. +7 (so each load reads 64 contiguous bytes of
// every row), of K (the matrix-core A operand of S = K q) and of V (staged
// through LDS into the transposed A operand of O^T = V^T P^T).
// (FP8 rows are half as wide: two 16-byte words of codes, channels 16kb and
// 64 + 16kb onward, which decode to words k of channels rows_ch(k, kb).)
// First channel of word k of lane group kb in the fp16-rows role (8 channels).
template <int FMT>
__device__ inline int rows_ch(int k, int kb) {
  return FMT == KVC_FMT_FP8 ? 64 * (k >> 1) + 16 * kb + 8 * (k & 1) : 32 * k + 8 * kb;
}

template <int FMT>
struct RowTile {
  uint4 k[FMT == KVC_FMT_FP8 ? 2 : 4];
  uint4 v[FMT == KVC_FMT_FP8 ? 2 : 4];
};
// Row tiles held in registers by the fp16-rows role (FP8 measured no faster
// with three or four: 72.8 / 75.3 us against 70.8 us at 128K).
constexpr int ROWS_AHEAD = 2;

// V tile staging in LDS: row t's 16-byte chunk j lives at chunk j ^ 2(t & 7)
// of the row.  Chunk pairs (2m, 2m + 1) stay adjacent, and the 32-byte block m
// of rows t and t' (t & 7 != t' & 7) lands on different banks, so a transposed
// read (one 32-byte block of each of 16 rows) runs in two conflict-free passes.
__device__ inline int vt_off(int t, int chunk) { return t * D + ((chunk ^ (2 * (t & 7))) << 3); }

// A = V^T operand of a 16x16x16 P.V product from the staged tile with one
// LDS transpose read (ds_read_b64_tr_b16).  In each 16-lane group kb, lane s
// addresses row 4kb + s/4, channels 16ct + 4(s%4) .. +3; the read hands lane
// col element col%4 of the words addressed by lanes col/4 + 4j (j = 0..3):
// channel 16ct + col of row 4kb + j, in element j.
typedef short s4v __attribute__((ext_vector_type(4)));
__device__ inline h4 vt_read_tr(const uint16_t* vt, int ct, int col, int kb) {
  const int t = 4 * kb + (col >> 2);
  const uint16_t* p = vt + vt_off(t, 2 * ct + ((col & 3) >> 1)) + 4 * (col & 1);
  const s4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4v*)(p));
  return bc<h4>(r);
}

// fp16-rows role: positions [pa, pb) of (b, g) in 16-row tiles, software
// pipelined -- the plan entries of tile i + 2 and the rows of tile i + 1 are
// in flight while tile i computes.  Plan entries come from the plan kernel
// (drop / keep) or, in dense mode, from the token index (fp16 caches read the
// page table here).  Every load is unconditional (buffer loads with empty
// ranges, or a valid row for an empty slot), so the compiler's waits count
// them exactly.
template <int FMT, bool DENSE, bool LOGITS>
__device__ __forceinline__ void rows_role(const AttendArgs& a, int b, int g, int rsplit, int lane, int w,
                                          float* sO, float* sML, int* sTok) {
  constexpr bool QUANT = grouped(FMT);
  constexpr bool FP8 = FMT == KVC_FMT_FP8;
  constexpr int NW = waves_per_wg(FMT);
  const kvc_cache& c = a.c;
  const int n = max(c.seq_lens[b], 0);
  const int nq = QUANT ? (n & ~(GS - 1)) : 0;
  const int G = a.G;
  const int col = lane & 15, kb = lane >> 4;
  const bool hv = col < G;
  // keep mode: the positions of the sel padding (ROW_SKIP entries past the
  // pair's filled entries) are left out, so a pair uses only the waves its own
  // selection needs; position p of the walk is plan position p (before the
  // padding) or p + gap (after it)
  int kf = a.k_max, gap = 0;
  if (!DENSE && a.mode == KVC_ATTEND_KEEP) {
    kf = min(max(*scalar_ptr(a.kfill + (int64_t)b * c.num_kv_heads + g), 0), a.k_max);
    gap = a.k_max - kf;
  }
  const int np = DENSE ? n - nq : a.np - gap;
  const int pa = (rsplit * NW + w) * a.ppw;
  const int pb = min(pa + a.ppw, np);
  const bool drop = compact(a.mode);
  const int ntiles = pb > pa ? (pb - pa + TILE - 1) / TILE : 0;

  float m = -INFINITY, l = 0.f;   // per head (lane column), log2 units
  f4 acc[8];                       // O^T channel tiles: lane holds channels 16ct + 4kb + i of head col
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f4{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) {
    h8 qb[4];
    {
      uint4 raw[4] = {};
      if (hv) {
        // register k holds the channels of the rows' word k (rows_ch)
        const uint16_t* qh = a.q + ((int64_t)b * a.hq + g * G + col) * D;
#pragma unroll
        for (int k = 0; k < 4; ++k) raw[k] = *reinterpret_cast<const uint4*>(qh + rows_ch<FMT>(k, kb));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) qb[k] = bc<h8>(raw[k]);
    }
    uint16_t* vt = reinterpret_cast<uint16_t*>(sO + w * 8 * D);   // 16 x 128 halves (sO is free until the end)
    int* tok0 = sTok + w * TILE * ROWS_AHEAD;   // codes of the tiles in registers
    const int row = lane & 15;
    const int Hkv = c.num_kv_heads;
    const int64_t pair = (int64_t)b * Hkv + g;

    // raw plan word(s) of this lane's row in tile i (one buffer load): the page
    // table word (dense), the sel entry (inline plan), or the plan kernel's entry
    const bool inl = !DENSE && a.inline_plan;
    const Buf rplan = DENSE ? make_buf(c.block_table + (int64_t)b * c.max_pages,
                                       (!QUANT && c.page_size > 0) ? c.max_pages * 4u : 0u)
                    : inl ? make_buf(a.sel + pair * a.k_max, (uint32_t)a.k_max * 4u)
                          : make_buf(a.rplan + pair * a.np, (uint32_t)a.np * 8u);
    const bool blocks = a.mode == KVC_ATTEND_BLOCKS;
    auto plan_load = [&](int i) -> uint2 {
      const int p = pa + TILE * i + row;
      if constexpr (DENSE) {
        const int page = (!QUANT && c.page_size > 0) ? page_of(a.pd, nq + p) : 0;
        return uint2{bc<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rplan, (int)(4u * (uint32_t)page), 0, 0)), 0u};
      } else {
        if (inl) {   // sel entry of the position (outside the sel region: past the range, reads 0)
          const int q = p - a.n_sink;
          const int si = q < 0 ? INT_MAX / 8 : (blocks ? q / GS : q);
          return uint2{bc<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rplan, (int)(4u * (uint32_t)min(si, INT_MAX / 8)), 0, 0)), 0u};
        }
        return buf_load8(rplan, 8u * (uint32_t)(p >= a.n_sink + kf ? p + gap : p));
      }
    };
    auto plan_decode = [&](uint2 raw, int i) -> int2 {
      const int p = pa + TILE * i + row;
      if (p >= pb) return int2{ROW_SKIP, 0};
      if constexpr (!DENSE) {
        if (inl) {   // as plan_entry for drop / blocks on a contiguous row store
          int t;
          bool ok;
          if (p < a.n_sink) {
            t = p;
            ok = p < n;
          } else if (p < a.n_sink + a.nsel) {
            const int e = (int)raw.x;
            if (blocks) {
              ok = e >= (a.n_sink + GS - 1) / GS && e < max(n - a.n_window, 0) / GS;
              t = ok ? e * GS + (p - a.n_sink) % GS : 0;
            } else {
              t = e;
              ok = t >= a.n_sink && t < n - a.n_window;
            }
          } else {
            t = window_start(n, a.n_sink, a.n_window) + (p - a.n_sink - a.nsel);
            ok = t < n;
          }
          return ok ? int2{t, (int)(pair * c.max_tokens + t)} : int2{ROW_NONE, 0};
        }
        return int2{(int)raw.x, (int)raw.y};
      } else {
        const int t = nq + p;
        if (QUANT) return int2{tail_code(t), (int)(pair * GS) + p};
        if (c.page_size == 0) return int2{t, (int)(pair * c.max_tokens + t)};
        const int page = page_of(a.pd, t);
        const int phys = (int)raw.x;
        if (page >= c.max_pages || phys < 0 || phys >= c.num_pages) return int2{ROW_SKIP, 0};
        return int2{t, (phys * Hkv + g) * a.pd.P + (t - page * a.pd.P)};
      }
    };
    const uint16_t* ksafe = c.k16 ? c.k16 : c.k_tail;
    const uint16_t* vsafe = c.v16 ? c.v16 : c.v_tail;
    auto load_rows = [&](int2 e, RowTile<FMT>& d, int* tok) {
      const bool on = row_on(e.x);
      if constexpr (FP8) {   // 32 codes of the row: two 16-byte loads each for K and V,
                             // a row's four lanes reading 64 contiguous bytes per load
        const int64_t off = (on ? (int64_t)e.y * D : 0) + 16 * kb;
        d.k[0] = *reinterpret_cast<const uint4*>(c.k_codes + off);
        d.k[1] = *reinterpret_cast<const uint4*>(c.k_codes + off + 64);
        d.v[0] = *reinterpret_cast<const uint4*>(c.v_codes + off);
        d.v[1] = *reinterpret_cast<const uint4*>(c.v_codes + off + 64);
      } else {
        // load k: the row's four lanes read 64 contiguous bytes (channels 32k + 8kb)
        const int64_t off = (int64_t)e.y * D + 8 * kb;
        const uint16_t* kq = on ? (e.x <= -3 ? c.k_tail : c.k16) + off : ksafe;
        const uint16_t* vq = on ? (e.x <= -3 ? c.v_tail : c.v16) + off : vsafe;
#pragma unroll
        for (int k = 0; k < 4; ++k) d.k[k] = *reinterpret_cast<const uint4*>(kq + 32 * k);
#pragma unroll
        for (int k = 0; k < 4; ++k) d.v[k] = *reinterpret_cast<const uint4*>(vq + 32 * k);
      }
      if (lane < TILE) tok[lane] = e.x;
    };
    auto compute = [&](int i, const RowTile<FMT>& d, const int* tok) {
      const int p0 = pa + TILE * i;
      wave_sync_lds();
      const int4 own = *reinterpret_cast<const int4*>(tok + 4 * kb);   // codes of this lane's S rows
      const int tk[4] = {own.x, own.y, own.z, own.w};
      const int mine = tok[row];                                      // code of the row this lane stages
      if (__ballot(row_on(mine) || (LOGITS && drop && mine == ROW_NONE)) == 0)
        return;   // a tile of empty positions (past a shorter selection)
      uint4 kr[4], vr[4];   // the tile's fp16 operands (FP8: decoded here, not at load)
      if constexpr (FP8) {
        fp8_row_decode(d.k[0], d.k[1], kr);
        fp8_row_decode(d.v[0], d.v[1], vr);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          kr[k] = d.k[k];
          vr[k] = d.v[k];
        }
      }
      // stage V (empty rows were read from a valid row; their p is 0)
#pragma unroll
      for (int k = 0; k < 4; ++k)   // vr[k]: channels rows_ch(k, kb) .. +7
        *reinterpret_cast<uint4*>(vt + vt_off(row, rows_ch<FMT>(k, kb) >> 3)) =
            row_on(mine) ? vr[k] : uint4{0u, 0u, 0u, 0u};
      f4 sc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k) sc = mfma32(bc<h8>(kr[k]), qb[k], sc);
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tv = tk[j];
        const bool on = row_on(tv);
        x[j] = on ? sc[j] * a.sm2 : -INFINITY;
        if constexpr (LOGITS) {
          if (hv && (on || (drop && tv == ROW_NONE))) {
            const int t = tv <= -3 ? -3 - tv : tv;
            const int pp = p0 + 4 * kb + j;
            const int pos = !drop ? t : (QUANT && a.mode == KVC_ATTEND_BLOCKS && pp >= a.n_sink) ? pp + a.nsel : pp;
            a.logits[((int64_t)b * a.hq + g * G + col) * a.logits_stride + pos] =
                on ? sc[j] * a.sm : -INFINITY;
          }
        }
      }
      float gmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      gmax = max_kb(gmax);
      const float m_new = fmaxf(m, gmax);
      if (__any(m_new > m)) {   // rescale only when some head's maximum grows
        const float alpha = m == -INFINITY ? 0.f : ex2(m - m_new);
        l *= alpha;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[ct] *= alpha;
        m = m_new;
      }
      const float ms = m == -INFINITY ? 0.f : m;
      h4 pt;   // P^T as the B operand: k = the lane's four rows, column = head
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pj = ex2(x[j] - ms);
        l += pj;
        pt[j] = (_Float16)pj;
      }
      wave_sync_lds();
      // O^T += V^T P^T: A = V^T (row = channel 16ct + col, k = rows 4kb..4kb+3)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16f16(vt_read_tr(vt, ct, col, kb), pt, acc[ct], 0, 0, 0);
    };

    // ROWS_AHEAD tiles in registers: while tile i computes, tiles i + 1 ..
    // i + ROWS_AHEAD - 1 are in flight; tile t lives in buffer t % ROWS_AHEAD,
    // and its plan entry is loaded ROWS_AHEAD tiles before its rows
    RowTile<FMT> d[ROWS_AHEAD];
    uint2 e[ROWS_AHEAD];
#pragma unroll
    for (int j = 0; j < ROWS_AHEAD; ++j) e[j] = plan_load(j);
#pragma unroll
    for (int j = 0; j < ROWS_AHEAD - 1; ++j) {
      load_rows(plan_decode(e[j], j), d[j], tok0 + TILE * j);
      e[j] = plan_load(j + ROWS_AHEAD);
    }
    int i = 0;
    for (; i + ROWS_AHEAD <= ntiles; i += ROWS_AHEAD) {   // whole rounds, no exit inside a trip
#pragma unroll
      for (int j = 0; j < ROWS_AHEAD; ++j) {
        const int jl = (j + ROWS_AHEAD - 1) % ROWS_AHEAD;
        load_rows(plan_decode(e[jl], i + j + ROWS_AHEAD - 1), d[jl], tok0 + TILE * jl);
        e[jl] = plan_load(i + j + 2 * ROWS_AHEAD - 1);
        compute(i + j, d[j], tok0 + TILE * j);
      }
    }
#pragma unroll
    for (int j = 0; j < ROWS_AHEAD - 1; ++j)
      if (i + j < ntiles) compute(i + j, d[j], tok0 + TILE * j);
  }

  l = sum_kb(l);
  wave_sync_lds();   // the V staging area in sO is read before the output lands there
  if (hv) {
    float* oh = sO + (w * 8 + col) * D;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) *reinterpret_cast<f4*>(oh + 16 * ct + 4 * kb) = acc[ct];
  }
  if (hv && kb == 0) {
    sML[(w * 8 + col) * 2] = m;
    sML[(w * 8 + col) * 2 + 1] = l;
  }
}

template <int FMT, bool DENSE, bool LOGITS, bool PACK, bool TILED, bool OUTL = false>
__global__ __launch_bounds__(64 * waves_per_wg(FMT), waves_per_wg(FMT) < 8 ? 8 / waves_per_wg(FMT) : 1)
void attend_kernel(AttendArgs a) {
  constexpr int NW = waves_per_wg(FMT);
  __shared__ __align__(16) float sO[NW * 8 * D];
  __shared__ float sML[NW * 8 * 2];
  __shared__ __align__(16) uint16_t sKm[NW * 256];
  __shared__ __align__(16) uint16_t sVm[NW * 256];
  __shared__ __align__(16) uint16_t sVo[OUTL ? NW * 256 : 4];   // V outlier entries per wave
  __shared__ __align__(16) int sTok[NW * TILE * ROWS_AHEAD];
  __shared__ __align__(16) float sAl[NW * 8];

  // one-dimensional grid.  Dense: pair-major, a pair's splits adjacent.
  // Drop / keep: every quantized-role workgroup (s_q per pair) before every
  // fp16-rows workgroup (s_r per pair), so the longer quantized runs of a
  // ragged batch are dispatched first.
  int id = blockIdx.x, pair, split;
  if (DENSE && a.pairs % 8 == 0) {
    // split-major: workgroup ids go round-robin over the eight XCDs, so every
    // split of a pair runs on the XCD whose L2 then holds the pair's partials
    // for the merge (whose workgroups follow the same order)
    split = id / a.pairs;
    pair = id - split * a.pairs;
  } else if (DENSE) {
    pair = id / a.s_total;
    split = id - pair * a.s_total;
  } else {
    // drop / blocks: every quantized-role workgroup before every fp16-rows one
    // (the longer quantized runs of a ragged batch start first); keep mode,
    // whose fp16 rows are a large share of the bytes: the two roles spread
    // evenly over the grid, so both run side by side from the start (ragged
    // keep batch 247 -> 229 us with eight rows workgroups a CU)
    const int64_t Q = (int64_t)a.s_q * a.pairs, T = (int64_t)a.s_total * a.pairs;
    int64_t qi, ri;
    if (a.mode == KVC_ATTEND_KEEP) {
      const int64_t qa = (int64_t)id * Q / T, qb = ((int64_t)id + 1) * Q / T;
      qi = qb > qa ? qa : -1;
      ri = id - qb;
    } else {
      qi = id < Q ? id : -1;
      ri = id - Q;
    }
    if (qi >= 0) {
      pair = (int)(qi / a.s_q);
      split = (int)(qi - (int64_t)pair * a.s_q);
    } else {
      const int s_r = a.s_total - a.s_q;
      pair = (int)(ri / s_r);
      split = a.s_q + (int)(ri - (int64_t)pair * s_r);
    }
  }
  const int b = pair / a.c.num_kv_heads, g = pair - b * a.c.num_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform per wave
  const int G = a.G;
  // (every wave of either role writes its sO / sML slots of heads < G)

  if constexpr (grouped(FMT)) {
    if (split < a.s_q)
      quant_role<FMT, DENSE, LOGITS, PACK, TILED, OUTL>(a, b, g, split, lane, w, sO, sML, sKm, sVm, sVo);
    else
      rows_role<FMT, DENSE, LOGITS>(a, b, g, split - a.s_q, lane, w, sO, sML, sTok);
  } else {
    rows_role<FMT, DENSE, LOGITS>(a, b, g, split, lane, w, sO, sML, sTok);
  }
  __syncthreads();

  // ---- combine the waves and write this split's partial per query head:
  // thread h < G finds the head's maximum and each wave's weight, then thread
  // (h, channel quad) sums the weighted outputs
  float* sWt = sAl;   // NW * 8 wave weights
  float* part = a.part + ((int64_t)b * a.hq + g * G) * a.s_total * PART + (int64_t)split * PART;
  if (tid < G) {
    float mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, sML[(ww * 8 + tid) * 2]);
    const float ms = mx == -INFINITY ? 0.f : mx;
    float l = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = sML[(ww * 8 + tid) * 2];
      const float sc = mw == -INFINITY ? 0.f : exp2f(mw - ms);
      sWt[ww * 8 + tid] = sc;
      l += sc * sML[(ww * 8 + tid) * 2 + 1];
    }
    float* ph = part + (int64_t)tid * a.s_total * PART;
    ph[0] = mx;
    ph[1] = l;
  }
  __syncthreads();
  if (tid < G * (D / 4)) {
    const int h = tid / (D / 4), cq = tid % (D / 4);
    f4 v = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < NW; ++ww)
      v += sWt[ww * 8 + h] * *reinterpret_cast<const f4*>(sO + (ww * 8 + h) * D + 4 * cq);
    *reinterpret_cast<f4*>(part + (int64_t)h * a.s_total * PART + PO + 4 * cq) = v;
  }
}

// ---------------------------------------------------------------- selection plan
// Wave-cooperative lower bounds in sel[0, k) (ascending keys, -1 padding
// last): the first index whose key is >= T0 (r0) and >= T1 (r1), in every
// lane.  Each step probes 64 evenly spaced entries at once and keeps the gap
// where the keys cross the target, so the search takes about log64(k) + 1
// round trips instead of log2(k).
__device__ inline void wave_lower_bounds(const int32_t* sel, int k, int T0, int T1, int lane,
                                         int& r0, int& r1) {
  int lo0 = 0, hi0 = k, lo1 = 0, hi1 = k;
  while (hi0 - lo0 > 64 || hi1 - lo1 > 64) {   // (uniform)
    const int s0 = (hi0 - lo0 + 63) / 64, s1 = (hi1 - lo1 + 63) / 64;
    const int i0 = lo0 + lane * s0, i1 = lo1 + lane * s1;
    const bool in0 = i0 < hi0, in1 = i1 < hi1;
    int v0 = INT_MAX, v1 = INT_MAX;
    if (in0) v0 = sel_key(sel[i0]);
    if (in1) v1 = sel_key(sel[i1]);
    // the probes below the target are a prefix (c of them): the bound lies in
    // (lo + (c - 1) s, lo + c s], or is lo when c = 0
    const int c0 = __popcll(__ballot(in0 && v0 < T0)), c1 = __popcll(__ballot(in1 && v1 < T1));
    if (hi0 - lo0 > 64) {
      const int nlo = c0 > 0 ? lo0 + (c0 - 1) * s0 + 1 : lo0;
      hi0 = min(hi0, lo0 + c0 * s0);
      lo0 = nlo;
    }
    if (hi1 - lo1 > 64) {
      const int nlo = c1 > 0 ? lo1 + (c1 - 1) * s1 + 1 : lo1;
      hi1 = min(hi1, lo1 + c1 * s1);
      lo1 = nlo;
    }
  }
  const int i0 = lo0 + lane, i1 = lo1 + lane;
  int v0 = INT_MAX, v1 = INT_MAX;
  if (i0 < hi0) v0 = sel_key(sel[i0]);
  if (i1 < hi1) v1 = sel_key(sel[i1]);
  r0 = lo0 + __popcll(__ballot(i0 < hi0 && v0 < T0));
  r1 = lo1 + __popcll(__ballot(i1 < hi1 && v1 < T1));
}

// Drop / keep modes, one thread per (32-token word, position) of (sequence,
// KV head): for quantized caches, which valid sel entries fall in the word
// (bits) and the sel index of the first entry at or after the word's first
// token (prefix); for every cache, the fp16-rows role's plan entry of the
// position.  Every word and entry is written, so no clearing is needed.
template <bool QUANT>
__global__ __launch_bounds__(256) void plan_kernel(AttendArgs a) {
  __shared__ uint32_t s_wc[4][64];   // per wave: sel entries per word
  __shared__ uint32_t s_wb[4][64];   // per wave: valid-entry bits per word
  __shared__ uint32_t s_tm[4][2];    // per wave: keep-mode tail tokens in sel (64 bits)
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int e0 = blockIdx.x * 256 + 64 * wv;   // the wave's first thread index (uniform)
  const int words = a.c.max_tokens / 32;
  const int64_t pi = (int64_t)b * a.c.num_kv_heads + g;
  const int n = max(a.c.seq_lens[b], 0);
  const int32_t* sel = a.k_max > 0 ? a.sel + pi * a.k_max : nullptr;
  const int blo = (a.n_sink + GS - 1) / GS, bhi = max(n - a.n_window, 0) / GS;   // candidate blocks
  if (QUANT && e < words && a.mode == KVC_ATTEND_BLOCKS) {
    // every token of a kept block; its logits positions start at 64 x its sel index
    const int j = e >> 1;
    const int i = lower_bound_sel(sel, a.k_max, j);
    const bool kept = i < a.k_max && sel[i] == j && j >= blo && j < bhi;
    a.sbits[pi * words + e] = kept ? ~0u : 0u;
    a.spre[pi * words + e] = GS * i + 32 * (e & 1);
  } else if (QUANT && e0 < words && a.mode != KVC_ATTEND_BLOCKS) {
    // the wave's 64 words together: the sel range [L0, L1) of their tokens,
    // then its entries binned by word in the wave's LDS (the prefix of a word
    // is L0 plus the entries of the words before it)
    int L0, L1;
    wave_lower_bounds(sel, a.k_max, 32 * e0, 32 * (e0 + 64), lane, L0, L1);
    s_wc[wv][lane] = 0u;
    s_wb[wv][lane] = 0u;
    wave_sync_lds();
    for (int i0 = L0; i0 < L1; i0 += 4 * 64) {   // (uniform) four loads in flight a lane
      int tv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + 64 * u + lane;
        tv[u] = i < L1 ? sel[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = tv[u], w = (t >> 5) - e0;
        if (i0 + 64 * u + lane < L1 && (unsigned)w < 64u) {
          atomicAdd(&s_wc[wv][w], 1u);
          if (t >= a.n_sink && t < n - a.n_window) atomicOr(&s_wb[wv][w], 1u << (t & 31));
        }
      }
    }
    wave_sync_lds();
    const uint32_t cnt = s_wc[wv][lane];
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t x = __shfl_up(incl, o);
      if (lane >= o) incl += x;
    }
    if (e < words) {
      a.sbits[pi * words + e] = s_wb[wv][lane];
      a.spre[pi * words + e] = L0 + (int)(incl - cnt);
    }
  }
  if (QUANT && a.mode == KVC_ATTEND_BLOCKS) {
    // groups the quantized role walks, ascending and disjoint: those holding
    // sink tokens, the kept blocks, those holding window tokens (complete
    // groups only; a kept block lies wholly between the sinks and the window)
    const int groups = a.c.max_tokens / GS, ng = n >> 6;
    const int ns = min((a.n_sink + GS - 1) / GS, ng);
    const int l0 = lower_bound_sel(sel, a.k_max, blo), l1 = lower_bound_sel(sel, a.k_max, max(bhi, blo));
    const int nl = l1 - l0;
    const int ws = max(window_start(n, a.n_sink, a.n_window) / GS, ns);
    const int nw = max(0, ng - ws);
    // (a selection that is not strictly ascending, which the interface rules
    // out, may list more groups or other ids: the count is capped and every
    // id clamped into the candidate range, so the walk stays in bounds)
    const int cnt = min(ns + nl + nw, groups);
    if (e < cnt)
      a.glist[pi * groups + e] = e < ns ? e
                                 : e < ns + nl ? min(max(sel[l0 + e - ns], blo), bhi - 1)
                                               : ws + (e - ns - nl);
    if (e == 0) a.gcount[pi] = cnt;
    // logits positions of sel entries that name no candidate block attend nothing
    if (a.logits) {
      const int G = a.G;
      for (int q = e; q < GS * a.k_max; q += gridDim.x * 256) {
        const int blk = sel[q / GS];
        if (blk >= blo && blk < bhi) continue;
        for (int h = 0; h < G; ++h)
          a.logits[((int64_t)b * a.hq + g * G + h) * a.logits_stride + a.n_sink + q] = -INFINITY;
      }
    }
  }
  if (a.mode == KVC_ATTEND_KEEP) {
    // the sel entries before the -1 padding: the one thread at the last filled
    // entry (or at entry 0 of an empty row) writes their number
    if (a.k_max == 0) {
      if (e == 0) a.kfill[pi] = 0;
    } else if (e < a.k_max) {
      const bool v = sel[e] >= 0, nv = e + 1 < a.k_max && sel[e + 1] >= 0;
      if (v && !nv) a.kfill[pi] = e + 1;
      else if (e == 0 && !v) a.kfill[pi] = 0;
    }
  }
  // keep mode, tail positions [nset, nset + 64): whether each tail token is in
  // sel, from the 64 entries at the lower bound of the tail's first token
  // (waves that hold such positions, uniform)
  bool tail_in = false;
  const int nset = a.n_sink + a.nsel + a.n_window;
  if (a.mode == KVC_ATTEND_KEEP && e0 < a.np && e0 + 64 > nset && e0 < nset + GS) {
    const int nq = QUANT ? (n & ~(GS - 1)) : 0;
    int lb, unused;
    wave_lower_bounds(sel, a.k_max, nq, nq, lane, lb, unused);
    if (lane < 2) s_tm[wv][lane] = 0u;
    wave_sync_lds();
    const int i = lb + lane;
    const int t = i < a.k_max ? sel[i] : -1, d = t - nq;
    if ((unsigned)d < 64u) atomicOr(&s_tm[wv][d >> 5], 1u << (d & 31));
    wave_sync_lds();
    const int dp = e - nset;   // this position's tail token is nq + dp
    if ((unsigned)dp < 64u) tail_in = (s_tm[wv][dp >> 5] >> (dp & 31)) & 1u;
  }
  if (e < a.np) a.rplan[pi * a.np + e] = plan_entry<QUANT>(a, b, g, n, e, tail_in);
}

// ---------------------------------------------------------------- split merge
// Log-sum-exp merge of the split partials (meeting-LLM article, section 8.1:
// the online-softmax rescale, applied across splits), one workgroup per
// (sequence, query head).  Thread (quad cq, replica r) folds splits r, r + 8,
// ... into a running (max, sum, o[4 cq .. 4 cq + 3]) with online rescaling,
// MB splits a round with every load of the round issued before the first is
// used; the 8 replicas are then combined through LDS.
constexpr int MT = 256;
constexpr int MR = MT / 32;   // replicas per query head
constexpr int MB = 8;         // splits a replica loads per round
__global__ __launch_bounds__(MT) void merge_kernel(const float* __restrict__ part, int s_total,
                                                   float* __restrict__ out, float* __restrict__ lse,
                                                   int pairs, int G) {
  __shared__ f4 sacc[MT];
  __shared__ float sml[2 * MT];
  // workgroup j * pairs + p merges query head j of pair p (on pair p's XCD)
  const int p = blockIdx.x % pairs, j = blockIdx.x / pairs;
  const int bh = p * G + j, tid = threadIdx.x, cq = tid & 31, r = tid >> 5;
  const float* pp = part + (int64_t)bh * s_total * PART;
  float mr = -INFINITY, lr = 0.f;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = r; s0 < s_total; s0 += MR * MB) {
    float2 ml[MB];
    f4 ov[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int64_t sp = min(s0 + i * MR, s_total - 1);
      ml[i] = *reinterpret_cast<const float2*>(pp + sp * PART);
      ov[i] = *reinterpret_cast<const f4*>(pp + sp * PART + PO + 4 * cq);
    }
    // (no early exit: a branch here lets the compiler sink each load into it,
    // one memory round trip per split; a split past the end repeats the last
    // one with weight zero instead)
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const float m = s0 + i * MR < s_total ? ml[i].x : -INFINITY, l = ml[i].y;
      const float mn = fmaxf(mr, m);
      const float sc = mr == -INFINITY ? 0.f : exp2f(mr - mn);
      const float wt = m == -INFINITY ? 0.f : exp2f(m - mn);
      acc = acc * sc + ov[i] * wt;
      lr = fmaf(lr, sc, l * wt);
      mr = mn;
    }
  }
  sacc[tid] = acc;
  sml[2 * tid] = mr;
  sml[2 * tid + 1] = lr;
  __syncthreads();
  if (r == 0) {
#pragma unroll
    for (int k = 1; k < MR; ++k) {
      const int t = tid + 32 * k;
      const float m = sml[2 * t], l = sml[2 * t + 1];
      const float mn = fmaxf(mr, m);
      const float sc = mr == -INFINITY ? 0.f : exp2f(mr - mn);
      const float wt = m == -INFINITY ? 0.f : exp2f(m - mn);
      acc = acc * sc + sacc[t] * wt;
      lr = fmaf(lr, sc, l * wt);
      mr = mn;
    }
    const f4 res = lr > 0.f ? acc / lr : f4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f4*>(out + (int64_t)bh * D + 4 * cq) = res;
    if (cq == 0) lse[bh] = lr > 0.f ? (mr + log2f(lr)) * LN2 : -INFINITY;
  }
}

constexpr int MAX_SPLITS = 2048;
// Workgroups a call is planned for by default: one four-wave workgroup per
// CU of an MI355X (measured on the 128K layers, fewer concurrent streams keep
// the DRAM pages open longer and beat two per CU).
constexpr int ATTEND_WG_DEFAULT = 256;
constexpr int LIST_MAX = 64;   // blocks mode: groups per wave (one list entry per lane)

struct Plan {
  int s_q, s_r, gpw, ppw;
};

// Positions of the fp16-rows role per (sequence, KV head) in drop / keep /
// blocks mode (blocks mode on codes: sinks and window only).
int rows_positions(int mode, int k_max, int n_sink, int n_window, bool quant) {
  const int nsel = mode != KVC_ATTEND_BLOCKS ? k_max : quant ? 0 : GS * k_max;
  return n_sink + nsel + n_window + (mode == KVC_ATTEND_KEEP ? GS : 0);
}

int walk_groups(const kvc_cache& c, int mode, int k_max, int n_sink, int n_window) {
  const int all = c.max_tokens / GS;
  if (mode != KVC_ATTEND_BLOCKS) return all;
  const int64_t w = (int64_t)k_max + (n_sink + GS - 1) / GS + (n_window + GS - 1) / GS + 1;
  return (int)std::min<int64_t>(all, w);
}

// target: workgroups the launch is planned for (see attend_target)
Plan plan_attend(const kvc_cache& c, int mode, int k_max, int n_sink, int n_window, int target) {
  Plan p{0, 0, 1, TILE};
  const int NW = waves_per_wg(c.format);
  const int pairs = c.batch * c.num_kv_heads;
  const bool quant = grouped(c.format);
  // groups the quantized role may walk per pair: every group, or in blocks
  // mode the kept blocks plus the groups holding sinks or window tokens
  const int groups = walk_groups(c, mode, k_max, n_sink, n_window);
  if (quant) {
    // dense: every pair is planned at capacity; drop / keep: four times the
    // workgroups, of which a pair uses what its length needs
    const int64_t waves = (int64_t)(mode == KVC_ATTEND_DENSE ? target : 4 * target) * NW;
    p.gpw = (int)std::max<int64_t>(1, ((int64_t)groups * pairs + waves - 1) / waves);
    // blocks mode: a wave's list entries fit in one register (<= 64 groups)
    if (mode == KVC_ATTEND_BLOCKS) p.gpw = std::min(p.gpw, LIST_MAX);
    p.s_q = (groups + NW * p.gpw - 1) / (NW * p.gpw);
  }
  int64_t np;
  if (mode == KVC_ATTEND_DENSE) np = quant ? GS : c.max_tokens;
  else np = rows_positions(mode, k_max, n_sink, n_window, quant);
  const int64_t tiles = std::max<int64_t>(1, (np + TILE - 1) / TILE);
  // a dense quantized cache leaves only its tail (< 64 tokens) to this role
  // fp16-rows workgroups per CU: one for fp16 / FP8 caches (the rows role is
  // the whole call; measured at 128K: FP8 dense 62.6 -> 59.5 us, fp16 Top-4096
  // drop 15.6 -> 13.9 us against four), four beside the quantized role of the
  // drop / blocks modes, eight in keep mode, where the keep set is about half
  // the bytes (ragged keep batch 262 us with one, 247 with four, 229 with
  // eight and the roles interleaved)
  const int rows_per_cu = quant ? (mode == KVC_ATTEND_KEEP ? 8 : 4) : 1;
  const int64_t rwaves = (quant && mode == KVC_ATTEND_DENSE) ? (int64_t)pairs * NW
                                                             : (int64_t)rows_per_cu * target * NW;
  const int64_t tpw = std::max<int64_t>(1, (tiles * pairs + rwaves - 1) / rwaves);
  p.ppw = (int)(tpw * TILE);
  p.s_r = (int)((tiles + NW * tpw - 1) / (NW * tpw));
  while (p.s_q + p.s_r > MAX_SPLITS) {   // bound the merge's work per query head
    if (p.s_q >= p.s_r && (mode != KVC_ATTEND_BLOCKS || 2 * p.gpw <= LIST_MAX)) { p.gpw *= 2; p.s_q = (groups + NW * p.gpw - 1) / (NW * p.gpw); }
    else if (p.s_r > 1) { p.ppw *= 2; p.s_r = (int)((tiles * TILE + (int64_t)NW * p.ppw - 1) / ((int64_t)NW * p.ppw)); }
    else break;   // (blocks mode on a cache too long for its list registers: rejected by the caller)
  }
  return p;
}

// Kernel instance for (format, mode, logits, packing, tile addressing, INT4
// outlier channels); fp16 caches have no quantized role, and only INT4 has
// 16-token tiles and outlier channels.
template <int F, bool DN, bool LG, bool OUTL>
void launch_tiles(dim3 grid, hipStream_t s, const AttendArgs& a, bool pk, bool tiled) {
  if (tiled) {
    if (pk) attend_kernel<F, DN, LG, true, true, OUTL><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
    else attend_kernel<F, DN, LG, false, true, OUTL><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
  } else {
    if (pk) attend_kernel<F, DN, LG, true, false, OUTL><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
    else attend_kernel<F, DN, LG, false, false, OUTL><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
  }
}
template <int F, bool DN, bool LG>
void launch_inst(dim3 grid, hipStream_t s, const AttendArgs& a, bool pk, bool tiled) {
  if constexpr (!grouped(F)) {
    attend_kernel<F, DN, LG, false, false><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
  } else if constexpr (F == KVC_FMT_INT4) {
    if (a.c.n_outlier > 0) {
      launch_tiles<F, DN, LG, true>(grid, s, a, pk, tiled);
    } else if (tiled) {
      if (pk) attend_kernel<F, DN, LG, true, true><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
      else attend_kernel<F, DN, LG, false, true><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
    } else {
      if (pk) attend_kernel<F, DN, LG, true, false><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
      else attend_kernel<F, DN, LG, false, false><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
    }
  } else {
    if (pk) attend_kernel<F, DN, LG, true, false><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
    else attend_kernel<F, DN, LG, false, false><<<grid, 64 * waves_per_wg(F), 0, s>>>(a);
  }
}
template <int F>
void launch_fmt(dim3 grid, hipStream_t s, const AttendArgs& a, bool dense, bool lg, bool pk,
                bool tiled) {
  if (dense) {
    if (lg) launch_inst<F, true, true>(grid, s, a, pk, tiled);
    else launch_inst<F, true, false>(grid, s, a, pk, tiled);
  } else {
    if (lg) launch_inst<F, false, true>(grid, s, a, pk, tiled);
    else launch_inst<F, false, false>(grid, s, a, pk, tiled);
  }
}

}  // namespace

int attend_target(int workgroups) { return workgroups > 0 ? workgroups : ATTEND_WG_DEFAULT; }

size_t attend_workspace_bytes(const kvc_cache& c, int hq, int mode, int k_max, int n_sink,
                              int n_window, int workgroups) {
  const Plan p = plan_attend(c, mode, k_max, n_sink, n_window, attend_target(workgroups));
  size_t bytes = (size_t)c.batch * hq * (p.s_q + p.s_r) * PART * sizeof(float);
  if (mode != KVC_ATTEND_DENSE && grouped(c.format))   // selection bitmap + prefix
    bytes += 2 * (size_t)c.batch * c.num_kv_heads * (c.max_tokens / 32) * sizeof(uint32_t);
  if (mode != KVC_ATTEND_DENSE)                               // fp16-rows role plan
    bytes += (size_t)c.batch * c.num_kv_heads *
             rows_positions(mode, k_max, n_sink, n_window, grouped(c.format)) * sizeof(int2);
  if (mode == KVC_ATTEND_BLOCKS && grouped(c.format))   // group list + count
    bytes += (size_t)c.batch * c.num_kv_heads * (c.max_tokens / GS + 1) * sizeof(int32_t);
  if (mode == KVC_ATTEND_KEEP)                                // filled sel entries per pair
    bytes += (size_t)c.batch * c.num_kv_heads * sizeof(int32_t);
  return bytes;
}

bool attend_plan_ok(const kvc_cache& c, int mode, int k_max, int n_sink, int n_window,
                    int workgroups) {
  const Plan p = plan_attend(c, mode, k_max, n_sink, n_window, attend_target(workgroups));
  if (p.s_q + p.s_r > MAX_SPLITS) return false;
  if (mode == KVC_ATTEND_BLOCKS && grouped(c.format))
    return (int64_t)p.s_q * waves_per_wg(c.format) * LIST_MAX >= walk_groups(c, mode, k_max, n_sink, n_window);
  return true;
}

hipError_t launch_attend(const kvc_cache& c, const uint16_t* q, int hq, float sm_scale, int mode,
                         const int32_t* sel, int k_max, int n_sink, int n_window, float* out,
                         float* lse, float* logits, int64_t logits_stride, int workgroups,
                         void* ws, hipStream_t s) {
  const Plan p = plan_attend(c, mode, k_max, n_sink, n_window, attend_target(workgroups));
  AttendArgs a;
  a.c = c;
  a.q = q;
  a.hq = hq;
  a.G = hq / c.num_kv_heads;
  a.sm = sm_scale;
  a.sm2 = sm_scale * LOG2E;
  a.mode = mode;
  a.sel = sel;
  a.k_max = k_max;
  a.n_sink = n_sink;
  a.n_window = n_window;
  a.logits = logits;
  a.logits_stride = logits_stride;
  a.part = static_cast<float*>(ws);
  a.pd = make_page_div(c);
  a.sbits = nullptr;
  a.spre = nullptr;
  a.rplan = nullptr;
  a.np = mode == KVC_ATTEND_DENSE ? 0 : rows_positions(mode, k_max, n_sink, n_window, grouped(c.format));
  a.nsel = mode == KVC_ATTEND_BLOCKS ? GS * k_max : k_max;
  a.inline_plan = !grouped(c.format) && c.page_size == 0 &&
                  (mode == KVC_ATTEND_DROP || mode == KVC_ATTEND_BLOCKS);
  a.glist = nullptr;
  a.gcount = nullptr;
  a.kfill = nullptr;
  const bool quant = grouped(c.format);
  char* wp = static_cast<char*>(ws) + (size_t)c.batch * hq * (p.s_q + p.s_r) * PART * sizeof(float);
  const size_t sel_words = (size_t)c.batch * c.num_kv_heads * (c.max_tokens / 32);
  if (mode != KVC_ATTEND_DENSE && quant) {
    a.sbits = reinterpret_cast<uint32_t*>(wp);
    a.spre = reinterpret_cast<int32_t*>(a.sbits + sel_words);
    wp += 2 * sel_words * sizeof(uint32_t);
  }
  if (mode != KVC_ATTEND_DENSE) {
    a.rplan = reinterpret_cast<int2*>(wp);
    wp += (size_t)c.batch * c.num_kv_heads * a.np * sizeof(int2);
  }
  if (mode == KVC_ATTEND_BLOCKS && quant) {
    a.glist = reinterpret_cast<int32_t*>(wp);
    a.gcount = a.glist + (size_t)c.batch * c.num_kv_heads * (c.max_tokens / GS);
  }
  if (mode == KVC_ATTEND_KEEP) a.kfill = reinterpret_cast<int32_t*>(wp);
  a.s_q = p.s_q;
  a.s_total = p.s_q + p.s_r;
  a.ppw = p.ppw;
  a.gpw = p.gpw;
  a.pairs = c.batch * c.num_kv_heads;
  const dim3 grid((unsigned)((int64_t)a.s_total * a.pairs));
  if (mode != KVC_ATTEND_DENSE && !a.inline_plan) {   // k_max == 0: all-zero bits
    const int items = std::max(quant ? c.max_tokens / 32 : 0, a.np);
    const dim3 pg((items + 255) / 256, c.num_kv_heads, c.batch);
    if (quant) plan_kernel<true><<<pg, 256, 0, s>>>(a);
    else plan_kernel<false><<<pg, 256, 0, s>>>(a);
  }
  const bool dense = mode == KVC_ATTEND_DENSE, lg = logits != nullptr;
  const bool pk = a.G <= 4;   // packed softmax (quantized role only)
  const bool tiled = c.page_size % GS != 0;   // INT4 on pages of 16 or 32 tokens
  switch (c.format) {
    case KVC_FMT_INT4: launch_fmt<KVC_FMT_INT4>(grid, s, a, dense, lg, pk, tiled); break;
    case KVC_FMT_INT1: launch_fmt<KVC_FMT_INT1>(grid, s, a, dense, lg, pk, false); break;
    case KVC_FMT_FP8: launch_fmt<KVC_FMT_FP8>(grid, s, a, dense, lg, false, false); break;
    default: launch_fmt<KVC_FMT_FP16>(grid, s, a, dense, lg, false, false); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  merge_kernel<<<c.batch * hq, MT, 0, s>>>(a.part, a.s_total, out, lse, a.pairs, a.G);
  return hipGetLastError();
}

// ---------------------------------------------------------------- static scratch
// The workspace of kvc_attend_decode_noalloc: a file-scope device array that
// every GPU the library runs on holds (its own copy, at its own address) until
// the process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
namespace {
__device__ __align__(256) uint8_t scratch[KVC_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> scratch_addr[MAX_DEVICES];
std::mutex scratch_mutex;
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mutex);
    p = scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace kvc
