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
// as fp16 "base + code" values built by one mask-and-or per code pair (base 16
// for INT4; 16/8/4/2 by bit position for INT1); the bases come back out through
// sum_c q'_c base_c.  For P.V the output is computed transposed, O^T = V^T P'^T,
// so a lane's accumulator column is its own query head and the online rescale
// needs no cross-lane traffic; P' = p * s_v per token and V half, and
// sum_t p z_v and sum_t P' base are kept beside it.

#include <math.h>

#include "internal.h"

namespace kvc {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;          // waves per workgroup
constexpr int NT = 64 * NW;
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
  int s_q, s_total;
  int gpw;                    // quantized role: 64-token groups per wave
  int ppw;                    // rows role: positions per wave (multiple of 16)
};

template <typename T, typename F>
__device__ inline T bc(const F& f) { return __builtin_bit_cast(T, f); }

__device__ inline float ror8(float x) {   // value of lane (l +- 8) within its row of 16
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}
__device__ inline float sum_kb(float x) {  // sum over lanes l, l^16, l^32, l^48
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
__device__ inline float max_kb(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
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

// INT4 dword (nibble slots j at bits 16*(j&1) + 4*(j>>1)) -> 8 fp16 values 16 + code_j.
// M = 0x03C003C0 and B = 0x4C004C00 (fp16 16.0 in both halves) come in VGPRs.
__device__ inline h8 dec4(uint32_t u, uint32_t M, uint32_t B) {
  uint4 w;
  w.x = ((u << 6) & M) | B;
  w.y = ((u << 2) & M) | B;
  w.z = ((u >> 2) & M) | B;
  w.w = ((u >> 6) & M) | B;
  return bc<h8>(w);
}

// INT1 dword -> word (variant v, position r): bit pair (6 + r, 22 + r) of the
// v-th shifted copy, with fp16 base 2^(4 - r) so each value is base + bit.
// mask[r] = 0x00400040 << r and base[r] = 0x4C004C00 - 0x04000400 * r in VGPRs.
__device__ inline uint32_t dec1_word(uint32_t u, int v, int r, const uint32_t* mask,
                                     const uint32_t* base) {
  const uint32_t s = v == 0 ? u : v == 1 ? (u >> 4) : v == 2 ? (u << 4) : __builtin_amdgcn_alignbit(u, u, 24);
  return (s & mask[r]) | base[r];
}

struct DecConst {
  uint32_t M4, B4, m1[4], b1[4];
};
__device__ inline DecConst make_dec() {
  DecConst d;
  d.M4 = vconst(0x03C003C0u);
  d.B4 = vconst(0x4C004C00u);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    d.m1[r] = vconst(0x00400040u << r);
    d.b1[r] = vconst(0x4C004C00u - 0x04000400u * (uint32_t)r);
  }
  return d;
}

__device__ inline f4 mfma32(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ inline f4 mfma16(h4 a, h4 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0); }

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

// Window start of the drop/keep sets.
__device__ inline int window_start(int n, int n_sink, int n_window) {
  return max(n - n_window, min(n_sink, n));
}

// ---------------------------------------------------------------- quantized role
// Raw loads of one 64-token group: code tiles and the two metadata words.
template <int FMT>
struct GroupData {
  uint4 k[FMT == KVC_FMT_INT4 ? 4 : 1];
  uint4 v[FMT == KVC_FMT_INT4 ? 4 : 1];
  uint2 km, vm;
};

// Per-wave running state of the quantized role.
struct QState {
  float m, l, sp0, sp1, sz0, sz1;
  f4 acc[8];
  int ptr;
};

template <int FMT>
__device__ __forceinline__ void load_group(const AttendArgs& a, int b, int g, int gi, int lane,
                                           GroupData<FMT>& d) {
  const kvc_cache& c = a.c;
  const int t0 = gi * GS;
  if constexpr (FMT == KVC_FMT_INT4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t s = slot_of(c, b, g, t0 + TILE * j);
      const int64_t off = (s < 0 ? 0 : (s / TILE)) * UNIT_BYTES + lane * 16;
      d.k[j] = *reinterpret_cast<const uint4*>(c.k_codes + off);
      d.v[j] = *reinterpret_cast<const uint4*>(c.v_codes + off);
    }
  } else {
    const int64_t s = slot_of(c, b, g, t0);
    const int64_t off = (s < 0 ? 0 : (s / GS)) * UNIT_BYTES + lane * 16;
    d.k[0] = *reinterpret_cast<const uint4*>(c.k_codes + off);
    d.v[0] = *reinterpret_cast<const uint4*>(c.v_codes + off);
  }
  const uint16_t* km = c.k_meta +
      ((((int64_t)b * c.num_kv_heads + g) * (c.max_tokens / GS) + gi) * 2) * D;
  d.km = *reinterpret_cast<const uint2*>(km + 4 * lane);
  const int64_t vs = slot_of(c, b, g, t0 + lane);
  d.vm = vs < 0 ? uint2{0u, 0u} : *reinterpret_cast<const uint2*>(c.v_meta + vs * 4);
}

template <int FMT, bool DENSE, bool LOGITS>
__device__ __forceinline__ void group_body(const AttendArgs& a, int b, int g, int gi, int lane,
                                           int w, int n, const GroupData<FMT>& d, QState& st,
                                           const h2* qv, const DecConst& dc, uint16_t* sKm,
                                           uint16_t* sVm, uint32_t* sMask, int* sPos) {
  const int G = a.G;
  const int col = lane & 15, kb = lane >> 4, head = col & 7;
  const bool hv = head < G;
  const bool hi_lane = hv && col < 8;
  const uint32_t lo_sel = (hv && !hi_lane) ? 0xFFFFFFFFu : 0u;  // lo lanes subtract hi
  const uint32_t hv_sel = hv ? 0xFFFFFFFFu : 0u;
  const int t0 = gi * GS;

  // ---- which tokens of this group are attended from the codes
  uint64_t att = ~0ull;
  if constexpr (!DENSE) {
    const int32_t* sel = a.sel ? a.sel + ((int64_t)b * a.c.num_kv_heads + g) * a.k_max : nullptr;
    const int w0 = window_start(n, a.n_sink, a.n_window);
    const int tl = t0 + lane;
    const bool in = tl < a.n_sink || tl >= w0;
    uint32_t* mw = sMask + 2 * w;
    if (lane < 2) mw[lane] = 0u;
    wave_sync_lds();
    int e = INT_MAX;
    if (sel && st.ptr + lane < a.k_max) e = sel_key(sel[st.ptr + lane]);
    const bool ing = e < t0 + GS;                 // entries before ptr are < t0
    const int cnt = __popcll(__ballot(ing));
    if (ing && e >= a.n_sink && e < n - a.n_window) {
      atomicOr(&mw[(e - t0) >> 5], 1u << ((e - t0) & 31));
      sPos[GS * w + (e - t0)] = a.n_sink + st.ptr + lane;
    }
    st.ptr += cnt;
    wave_sync_lds();
    const uint64_t selm = (uint64_t)mw[0] | ((uint64_t)mw[1] << 32);
    const uint64_t inset = __ballot(in) | selm;
    att = a.mode == KVC_ATTEND_DROP ? inset : ~inset;
    if (a.mode == KVC_ATTEND_DROP && a.logits && in)   // logits positions of sinks / window
      sPos[GS * w + lane] = tl < a.n_sink ? tl : a.n_sink + a.k_max + (tl - w0);
    wave_sync_lds();
    if (att == 0) return;
  }

  // ---- stage the group's K scales/zeros and V token metadata in LDS
  *reinterpret_cast<uint2*>(sKm + 256 * w + 4 * lane) = d.km;
  *reinterpret_cast<uint2*>(sVm + 256 * w + 4 * lane) = d.vm;
  wave_sync_lds();

  // ---- q' = q * s as fp16 hi (columns < 8) / lo (columns >= 8); bias
  h8 qp[4];
  float qz = 0.f, qb = 0.f;
  {
    const uint16_t* ks = sKm + 256 * w;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const uint4 s4 = *reinterpret_cast<const uint4*>(ks + 32 * kb + 8 * kc);
      const uint4 z4 = *reinterpret_cast<const uint4*>(ks + D + 32 * kb + 8 * kc);
      const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
      const uint32_t zw[4] = {z4.x, z4.y, z4.z, z4.w};
      uint32_t out[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const h2 qq = qv[4 * kc + pr];
        const h2 ss = bc<h2>(sw[pr]);
        const h2 hi = qq * ss;
        const h2 sub = bc<h2>(bc<uint32_t>(hi) & lo_sel);
        const h2 r = __builtin_elementwise_fma(qq, ss, -sub);
        const uint32_t rw = bc<uint32_t>(r) & hv_sel;
        out[pr] = rw;
        qz = __builtin_amdgcn_fdot2(qq, bc<h2>(zw[pr]), qz, false);
        h2 base;
        if constexpr (FMT == KVC_FMT_INT4) {
          base = h2{(_Float16)16.f, (_Float16)16.f};
        } else {
          const _Float16 bv = (_Float16)(float)(16 >> pr);   // slots 2pr, 2pr+1
          base = h2{bv, bv};
        }
        qb = __builtin_amdgcn_fdot2(bc<h2>(rw), base, qb, false);
      }
      qp[kc] = bc<h8>(uint4{out[0], out[1], out[2], out[3]});
    }
  }
  const float bias = sum_kb((hi_lane ? qz : 0.f) - qb);

  // ---- S^T = codes x q'^T per 16-token tile; hi + lo; scale to log2 units
  float x[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f4 s = f4{bias, bias, bias, bias};
    if constexpr (FMT == KVC_FMT_INT4) {
      s = mfma32(dec4(d.k[j].x, dc.M4, dc.B4), qp[0], s);
      s = mfma32(dec4(d.k[j].y, dc.M4, dc.B4), qp[1], s);
      s = mfma32(dec4(d.k[j].z, dc.M4, dc.B4), qp[2], s);
      s = mfma32(dec4(d.k[j].w, dc.M4, dc.B4), qp[3], s);
    } else {
      const uint32_t u = j == 0 ? d.k[0].x : j == 1 ? d.k[0].y : j == 2 ? d.k[0].z : d.k[0].w;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint4 wv = uint4{dec1_word(u, kc, 0, dc.m1, dc.b1), dec1_word(u, kc, 1, dc.m1, dc.b1),
                               dec1_word(u, kc, 2, dc.m1, dc.b1), dec1_word(u, kc, 3, dc.m1, dc.b1)};
        s = mfma32(bc<h8>(wv), qp[kc], s);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = s[i] + ror8(s[i]);
      const int bit = TILE * j + 4 * kb + i;
      const bool on = DENSE || ((att >> bit) & 1ull);
      x[j][i] = on ? v * a.sm2 : -INFINITY;
      if (LOGITS && hi_lane && on) {
        const int pos = a.mode == KVC_ATTEND_DROP ? sPos[GS * w + bit] : t0 + bit;
        a.logits[((int64_t)b * a.hq + g * G + head) * a.logits_stride + pos] = v * a.sm;
      }
    }
  }

  // ---- online softmax (log2 units)
  float gmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) gmax = fmaxf(gmax, x[j][i]);
  gmax = max_kb(gmax);
  const float m_new = fmaxf(st.m, gmax);
  const float ms = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = ex2(st.m - ms);
  st.m = m_new;
  st.l *= alpha;
  st.sp0 *= alpha; st.sp1 *= alpha; st.sz0 *= alpha; st.sz1 *= alpha;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) st.acc[ct] *= alpha;

  // ---- O^T += V^T P'^T per tile
  const uint16_t* vmeta = sVm + 256 * w;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = ex2(x[j][i] - ms);
      st.l += p[i];
    }
    const uint4 m01 = *reinterpret_cast<const uint4*>(vmeta + 4 * (TILE * j + 4 * kb));
    const uint4 m23 = *reinterpret_cast<const uint4*>(vmeta + 4 * (TILE * j + 4 * kb + 2));
    const uint32_t mwd[8] = {m01.x, m01.y, m01.z, m01.w, m23.x, m23.y, m23.z, m23.w};
    h4 A0, A1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const h2 s01 = bc<h2>(mwd[2 * i]);       // (s0, s1) of token i
      const h2 z01 = bc<h2>(mwd[2 * i + 1]);   // (z0, z1)
      const _Float16 P0 = (_Float16)(p[i] * (float)s01.x);
      const _Float16 P1 = (_Float16)(p[i] * (float)s01.y);
      A0[i] = P0;
      A1[i] = P1;
      st.sp0 += (float)P0;
      st.sp1 += (float)P1;
      st.sz0 = fmaf(p[i], (float)z01.x, st.sz0);
      st.sz1 = fmaf(p[i], (float)z01.y, st.sz1);
    }
    if constexpr (FMT == KVC_FMT_INT4) {
      const uint32_t dw[4] = {d.v[j].x, d.v[j].y, d.v[j].z, d.v[j].w};
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const h8 v8 = dec4(dw[dd], dc.M4, dc.B4);
        const h4 va = h4{v8[0], v8[1], v8[2], v8[3]};   // channel tile 2dd, tokens 0..3
        const h4 vb = h4{v8[4], v8[5], v8[6], v8[7]};   // channel tile 2dd + 1
        st.acc[2 * dd] = mfma16(va, dd < 2 ? A0 : A1, st.acc[2 * dd]);
        st.acc[2 * dd + 1] = mfma16(vb, dd < 2 ? A0 : A1, st.acc[2 * dd + 1]);
      }
    } else {
      const uint32_t u = j == 0 ? d.v[0].x : j == 1 ? d.v[0].y : j == 2 ? d.v[0].z : d.v[0].w;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const uint32_t w0v = dec1_word(u, 2 * (ct >> 2), ct & 3, dc.m1, dc.b1);
        const uint32_t w1v = dec1_word(u, 2 * (ct >> 2) + 1, ct & 3, dc.m1, dc.b1);
        const h4 va = bc<h4>(uint2{w0v, w1v});
        st.acc[ct] = mfma16(va, ct < 4 ? A0 : A1, st.acc[ct]);
      }
    }
  }
}

template <int FMT, bool DENSE, bool LOGITS>
__device__ void quant_role(const AttendArgs& a, int b, int g, int split, int lane, int w,
                           float* sO, float* sML, uint16_t* sKm, uint16_t* sVm,
                           uint32_t* sMask, int* sPos) {
  const kvc_cache& c = a.c;
  const int n = max(c.seq_lens[b], 0);
  const int ngroups = n >> 6;
  const int G = a.G;
  const int col = lane & 15, kb = lane >> 4, head = col & 7;
  const bool hv = head < G;
  const bool hi_lane = hv && col < 8;
  const int ga = (split * NW + w) * a.gpw;
  const int gb = min(ga + a.gpw, ngroups);

  // q of this lane's head, channels [32kb, 32kb + 32), as fp16 pairs
  h2 qv[16];
  {
    uint4 raw[4] = {};
    if (hv) {
      const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.hq + g * G + head) * D + 32 * kb);
#pragma unroll
      for (int k = 0; k < 4; ++k) raw[k] = qp[k];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qv[4 * k + 0] = bc<h2>(raw[k].x);
      qv[4 * k + 1] = bc<h2>(raw[k].y);
      qv[4 * k + 2] = bc<h2>(raw[k].z);
      qv[4 * k + 3] = bc<h2>(raw[k].w);
    }
  }

  QState st;
  st.m = -INFINITY;
  st.l = st.sp0 = st.sp1 = st.sz0 = st.sz1 = 0.f;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) st.acc[ct] = f4{0.f, 0.f, 0.f, 0.f};
  st.ptr = 0;
  if (!DENSE && a.sel && ga < gb)
    st.ptr = lower_bound_sel(a.sel + ((int64_t)b * c.num_kv_heads + g) * a.k_max, a.k_max, ga * GS);

  const DecConst dc = make_dec();

  // two-deep software pipeline: group gi + 1 is in flight while gi computes
  GroupData<FMT> da, db;
  if (ga < gb) load_group<FMT>(a, b, g, ga, lane, da);
  for (int gi = ga; gi < gb; gi += 2) {
    if (gi + 1 < gb) load_group<FMT>(a, b, g, gi + 1, lane, db);
    group_body<FMT, DENSE, LOGITS>(a, b, g, gi, lane, w, n, da, st, qv, dc, sKm, sVm, sMask, sPos);
    if (gi + 1 >= gb) break;
    if (gi + 2 < gb) load_group<FMT>(a, b, g, gi + 2, lane, da);
    group_body<FMT, DENSE, LOGITS>(a, b, g, gi + 1, lane, w, n, db, st, qv, dc, sKm, sVm, sMask, sPos);
  }

  // ---- finish: sums over the four token quads, base and zero-point corrections
  const float l = sum_kb(st.l);
  const float sp0 = sum_kb(st.sp0), sp1 = sum_kb(st.sp1);
  const float sz0 = sum_kb(st.sz0), sz1 = sum_kb(st.sz1);
  if (hi_lane) {
    float* o = sO + (w * 8 + head) * D;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const float base = FMT == KVC_FMT_INT4 ? 16.f : (float)(16 >> (ct & 3));
      const float corr = ct < 4 ? sz0 - base * sp0 : sz1 - base * sp1;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[16 * ct + 4 * kb + i] = st.acc[ct][i] + corr;
    }
    if (kb == 0) {
      sML[(w * 8 + head) * 2] = st.m;
      sML[(w * 8 + head) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------- fp16-rows role
struct RowRef {
  int t;          // token index (logits position in dense / keep mode)
  int pos;        // logits position in drop mode
  int64_t off;    // element offset of the row (k16/v16 slot * D, or tail row)
  bool tail;      // row lives in k_tail/v_tail
  bool ok;        // this role attends the position
  bool none;      // drop mode: the position attends no token at all
};

template <int FMT>
__device__ inline RowRef resolve(const AttendArgs& a, int b, int g, int n, int nq, int p) {
  const kvc_cache& c = a.c;
  RowRef r{0, p, 0, false, false, false};
  const bool quant = FMT != KVC_FMT_FP16;
  const int Hkv = c.num_kv_heads;
  if (a.mode == KVC_ATTEND_DENSE) {
    r.t = nq + p;
    r.ok = r.t < n;
    r.tail = quant;
  } else {
    const int nset = a.n_sink + a.k_max + a.n_window;
    const int w0 = window_start(n, a.n_sink, a.n_window);
    if (p < nset) {
      if (p < a.n_sink) {
        r.t = p;
        r.ok = p < n;
      } else if (p < a.n_sink + a.k_max) {
        const int e = a.sel[((int64_t)b * Hkv + g) * a.k_max + (p - a.n_sink)];
        r.t = e;
        r.ok = e >= a.n_sink && e < n - a.n_window;
      } else {
        r.t = w0 + (p - a.n_sink - a.k_max);
        r.ok = r.t < n;
      }
      r.none = !r.ok;
      if (a.mode == KVC_ATTEND_DROP && quant) {
        r.ok = r.ok && r.t >= nq;      // older tokens come from the codes
        r.tail = true;
      }
    } else {  // keep mode: tail tokens outside the keep set
      r.t = nq + (p - nset);
      r.tail = true;
      r.ok = r.t < n && r.t >= a.n_sink && r.t < w0;
      if (r.ok) {
        const int32_t* sel = a.sel + ((int64_t)b * Hkv + g) * a.k_max;
        const int i = lower_bound_sel(sel, a.k_max, r.t);
        if (i < a.k_max && sel[i] == r.t && r.t < n - a.n_window) r.ok = false;
      }
    }
  }
  if (!r.ok) return r;
  if (r.tail) {
    r.off = (((int64_t)b * Hkv + g) * GS + (r.t - nq)) * D;
  } else {
    const int64_t s = slot_of(c, b, g, r.t);
    if (s < 0) { r.ok = false; return r; }
    r.off = s * D;
  }
  return r;
}

template <int FMT>
__device__ void rows_role(const AttendArgs& a, int b, int g, int rsplit, int lane, int w,
                          float* sO, float* sML, float* sP, int* sTok, int64_t* sOff,
                          float* sAl) {
  const kvc_cache& c = a.c;
  const int n = max(c.seq_lens[b], 0);
  const int nq = FMT == KVC_FMT_FP16 ? 0 : (n & ~(GS - 1));
  const int G = a.G;
  const int col = lane & 15, kb = lane >> 4;
  const bool hv = col < G;
  int np;
  if (a.mode == KVC_ATTEND_DENSE) np = n - nq;
  else np = a.n_sink + a.k_max + a.n_window + (a.mode == KVC_ATTEND_KEEP ? GS : 0);
  const int pa = (rsplit * NW + w) * a.ppw;
  const int pb = min(pa + a.ppw, np);
  const bool drop = a.mode == KVC_ATTEND_DROP;

  h8 qb[4];
  {
    uint4 raw[4] = {};
    if (hv) {
      const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.hq + g * G + col) * D + 32 * kb);
#pragma unroll
      for (int k = 0; k < 4; ++k) raw[k] = qp[k];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) qb[k] = bc<h8>(raw[k]);
  }

  float m = -INFINITY, l = 0.f;
  float o[8][2];
#pragma unroll
  for (int h = 0; h < 8; ++h) o[h][0] = o[h][1] = 0.f;
  float* P = sP + w * 16 * 8;
  int* tok = sTok + w * 16;
  int64_t* roff = sOff + w * 16;
  float* al = sAl + w * 8;

  for (int p0 = pa; p0 < pb; p0 += TILE) {
    const int p = p0 + (lane & 15);
    RowRef r = p < pb ? resolve<FMT>(a, b, g, n, nq, p) : RowRef{0, p, 0, false, false, false};
    if (drop && r.none && a.logits && kb < G)   // lanes (row, kb) cover heads kb, kb + 4
      for (int h = kb; h < G; h += 4)
        a.logits[((int64_t)b * a.hq + g * G + h) * a.logits_stride + p] = -INFINITY;
    h8 ka[4];
    {
      uint4 raw[4] = {};
      if (r.ok) {
        const uint16_t* kbase = (r.tail ? c.k_tail : c.k16) + r.off + 32 * kb;
#pragma unroll
        for (int k = 0; k < 4; ++k) raw[k] = reinterpret_cast<const uint4*>(kbase)[k];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) ka[k] = bc<h8>(raw[k]);
    }
    if (lane < 16) {
      tok[lane] = r.ok ? (r.tail ? -2 - r.t : r.t) : -1;   // -1: none; <= -2: tail row
      roff[lane] = r.off;
    }
    f4 s = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) s = mfma32(ka[k], qb[k], s);
    wave_sync_lds();

    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tv = tok[4 * kb + i];
      const bool on = tv != -1;
      x[i] = on ? s[i] * a.sm2 : -INFINITY;
      if (a.logits && hv && on) {
        const int t = tv <= -2 ? -2 - tv : tv;
        const int pos = drop ? p0 + 4 * kb + i : t;
        a.logits[((int64_t)b * a.hq + g * G + col) * a.logits_stride + pos] = s[i] * a.sm;
      }
    }
    float gmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    gmax = max_kb(gmax);
    const float m_new = fmaxf(m, gmax);
    const float ms = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = ex2(m - ms);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pi = ex2(x[i] - ms);
      l += pi;
      if (hv) P[(4 * kb + i) * 8 + col] = pi;
    }
    if (hv && kb == 0) al[col] = alpha;
    wave_sync_lds();

    // VALU P.V: lane owns channels 2*lane, 2*lane + 1 for every head
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      if (h < G) {
        const float ah = al[h];
        o[h][0] *= ah;
        o[h][1] *= ah;
      }
    }
    for (int i = 0; i < TILE; ++i) {
      const int tv = tok[i];
      if (tv == -1) continue;
      const uint16_t* vrow = (tv <= -2 ? c.v_tail : c.v16) + roff[i];
      const h2 v = *reinterpret_cast<const h2*>(vrow + 2 * lane);
      const float v0 = (float)v.x, v1 = (float)v.y;
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        if (h < G) {
          const float ph = P[i * 8 + h];
          o[h][0] = fmaf(ph, v0, o[h][0]);
          o[h][1] = fmaf(ph, v1, o[h][1]);
        }
      }
    }
    wave_sync_lds();
  }

  l = sum_kb(l);
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h < G) {
      float* oh = sO + (w * 8 + h) * D;
      oh[2 * lane] = o[h][0];
      oh[2 * lane + 1] = o[h][1];
    }
  }
  if (hv && kb == 0) {
    sML[(w * 8 + col) * 2] = m;
    sML[(w * 8 + col) * 2 + 1] = l;
  }
}

template <int FMT, bool DENSE, bool LOGITS>
__global__ __launch_bounds__(NT, 2) void attend_kernel(AttendArgs a) {
  __shared__ float sO[NW * 8 * D];
  __shared__ float sML[NW * 8 * 2];
  __shared__ __align__(16) uint16_t sKm[NW * 256];
  __shared__ __align__(16) uint16_t sVm[NW * 256];
  __shared__ uint32_t sMask[NW * 2];
  __shared__ int sPos[NW * GS];
  __shared__ float sP[NW * 16 * 8];
  __shared__ int sTok[NW * 16];
  __shared__ int64_t sOff[NW * 16];
  __shared__ float sAl[NW * 8];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int G = a.G;
  for (int e = tid; e < NW * 8 * 2; e += NT) sML[e] = (e & 1) ? 0.f : -INFINITY;
  for (int e = tid; e < NW * 8 * D; e += NT) sO[e] = 0.f;
  __syncthreads();

  if constexpr (FMT != KVC_FMT_FP16) {
    if (split < a.s_q)
      quant_role<FMT, DENSE, LOGITS>(a, b, g, split, lane, w, sO, sML, sKm, sVm, sMask, sPos);
    else
      rows_role<FMT>(a, b, g, split - a.s_q, lane, w, sO, sML, sP, sTok, sOff, sAl);
  } else {
    rows_role<FMT>(a, b, g, split, lane, w, sO, sML, sP, sTok, sOff, sAl);
  }
  __syncthreads();

  // ---- merge the four waves and write this split's partial per query head
  for (int e = tid; e < G * (D + 2); e += NT) {
    const int h = e / (D + 2), k = e % (D + 2);
    float mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, sML[(ww * 8 + h) * 2]);
    const float ms = mx == -INFINITY ? 0.f : mx;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = sML[(ww * 8 + h) * 2];
      const float sc = mw == -INFINITY ? 0.f : exp2f(mw - ms);
      if (k == 1) v += sc * sML[(ww * 8 + h) * 2 + 1];
      else if (k >= 2) v += sc * sO[(ww * 8 + h) * D + (k - 2)];
    }
    if (k == 0) v = mx;
    float* part = a.part + (((int64_t)b * a.hq + g * G + h) * a.s_total + split) * PART;
    part[k < 2 ? k : PO + (k - 2)] = v;
  }
}

// ---------------------------------------------------------------- split merge
// One workgroup per (sequence, query head): log-sum-exp combination of the
// split partials.  Thread t adds channel quad t % 32 over splits t / 32, +8, ...
constexpr int MT = 256;
constexpr int MAX_SPLITS = 2048;

__global__ __launch_bounds__(MT) void merge_kernel(const float* __restrict__ part, int s_total,
                                                   float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float sw[MAX_SPLITS];
  __shared__ float red[MT / 64];
  __shared__ f4 racc[MT];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* pp = part + (int64_t)bh * s_total * PART;
  float mx = -INFINITY;
  for (int s = tid; s < s_total; s += MT) mx = fmaxf(mx, pp[s * PART]);
  for (int o = 32; o; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float ms = mx == -INFINITY ? 0.f : mx;
  __syncthreads();
  float L = 0.f;
  for (int s = tid; s < s_total; s += MT) {
    const float m = pp[s * PART];
    const float sc = m == -INFINITY ? 0.f : exp2f(m - ms);
    sw[s] = sc;
    L = fmaf(sc, pp[s * PART + 1], L);
  }
  for (int o = 32; o; o >>= 1) L += __shfl_xor(L, o);
  __syncthreads();
  if (lane == 0) red[wv] = L;
  __syncthreads();
  L = red[0] + red[1] + red[2] + red[3];
  const int cq = tid & 31, sl = tid >> 5;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = sl; s < s_total; s += MT / 32) {
    const f4 o = *reinterpret_cast<const f4*>(pp + s * PART + PO + 4 * cq);
    acc += sw[s] * o;
  }
  racc[tid] = acc;
  __syncthreads();
  if (tid < 32) {
    f4 t = racc[tid];
#pragma unroll
    for (int k = 1; k < MT / 32; ++k) t += racc[tid + 32 * k];
    const f4 r = L > 0.f ? t / L : f4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f4*>(out + (int64_t)bh * D + 4 * tid) = r;
    if (tid == 0) lse[bh] = L > 0.f ? (mx + log2f(L)) * LN2 : -INFINITY;
  }
}

struct Plan {
  int s_q, s_r, gpw, ppw;
};

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

Plan plan_attend(const kvc_cache& c, int mode, int k_max, int n_sink, int n_window) {
  Plan p{0, 0, 1, TILE};
  const int pairs = c.batch * c.num_kv_heads;
  const bool quant = c.format != KVC_FMT_FP16;
  // workgroups resident at once: 256 CUs x 2 four-wave workgroups (the quantized
  // role runs two waves per SIMD); one full round keeps every CU streaming
  const int target = env_int("KVC_ATTEND_TARGET_WG", 512);
  if (quant) {
    const int groups = c.max_tokens / GS;
    const int64_t waves = (int64_t)target * NW;
    p.gpw = (int)std::max<int64_t>(1, ((int64_t)groups * pairs + waves - 1) / waves);
    p.s_q = (groups + NW * p.gpw - 1) / (NW * p.gpw);
  }
  int64_t np;
  if (mode == KVC_ATTEND_DENSE) np = quant ? GS : c.max_tokens;
  else np = (int64_t)n_sink + k_max + n_window + (mode == KVC_ATTEND_KEEP ? GS : 0);
  const int64_t tiles = std::max<int64_t>(1, (np + TILE - 1) / TILE);
  const int64_t rwaves = (int64_t)(quant ? std::max(1, target / 4) : 2 * target) * NW;
  const int64_t tpw = std::max<int64_t>(1, (tiles * pairs + rwaves - 1) / rwaves);
  p.ppw = (int)(tpw * TILE);
  p.s_r = (int)((tiles + NW * tpw - 1) / (NW * tpw));
  while (p.s_q + p.s_r > MAX_SPLITS) {   // keep the merge's per-split weights in LDS
    if (p.s_q >= p.s_r) { p.gpw *= 2; p.s_q = (c.max_tokens / GS + NW * p.gpw - 1) / (NW * p.gpw); }
    else { p.ppw *= 2; p.s_r = (int)((tiles * TILE + (int64_t)NW * p.ppw - 1) / ((int64_t)NW * p.ppw)); }
  }
  return p;
}

}  // namespace

size_t attend_workspace_bytes(const kvc_cache& c, int hq, int mode, int k_max, int n_sink,
                              int n_window) {
  const Plan p = plan_attend(c, mode, k_max, n_sink, n_window);
  return (size_t)c.batch * hq * (p.s_q + p.s_r) * PART * sizeof(float);
}

hipError_t launch_attend(const kvc_cache& c, const uint16_t* q, int hq, float sm_scale, int mode,
                         const int32_t* sel, int k_max, int n_sink, int n_window, float* out,
                         float* lse, float* logits, int64_t logits_stride, void* ws,
                         hipStream_t s) {
  const Plan p = plan_attend(c, mode, k_max, n_sink, n_window);
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
  a.s_q = p.s_q;
  a.s_total = p.s_q + p.s_r;
  a.gpw = p.gpw;
  a.ppw = p.ppw;
  const dim3 grid(a.s_total, c.num_kv_heads, c.batch);
  const bool dense = mode == KVC_ATTEND_DENSE, lg = logits != nullptr;
#define KVC_LAUNCH(F, DN, LG) attend_kernel<F, DN, LG><<<grid, NT, 0, s>>>(a)
#define KVC_LAUNCH_F(F)                                   \
  do {                                                    \
    if (dense) { if (lg) KVC_LAUNCH(F, true, true); else KVC_LAUNCH(F, true, false); } \
    else { if (lg) KVC_LAUNCH(F, false, true); else KVC_LAUNCH(F, false, false); }     \
  } while (0)
  switch (c.format) {
    case KVC_FMT_INT4: KVC_LAUNCH_F(KVC_FMT_INT4); break;
    case KVC_FMT_INT1: KVC_LAUNCH_F(KVC_FMT_INT1); break;
    default: KVC_LAUNCH_F(KVC_FMT_FP16); break;
  }
#undef KVC_LAUNCH_F
#undef KVC_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  merge_kernel<<<c.batch * hq, MT, 0, s>>>(a.part, a.s_total, out, lse);
  return hipGetLastError();
}

}  // namespace kvc
