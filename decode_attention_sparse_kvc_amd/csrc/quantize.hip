// Append + quantize (TailorKV article section 2.2; on-device KV article section 3.1).
//
// One workgroup per (64-token group touched by the append, KV head, sequence).
// A complete group of new rows on a cache without fp16 copies or outlier
// channels (the bulk of a prefill) is quantized straight from the new rows,
// each wave on its own share (see quantize_group).  Any other group is staged
// in LDS (old tail rows + new rows); the workgroup writes the fp16 copies
// (k16/v16 rows, channel-major kT), folds |K| into k_absmax and, when the
// append completes the group, quantizes it:
//   K: per channel over the 64 tokens;  V: per token over each 64-channel half;
//   s = fp16((max - min) / (2^b - 1) + 0), z = fp16(min + 0),
//   code = s == 0 ? 0 : clamp(rint((x - z) / s), 0, 2^b - 1) in fp32.
// The packed code tiles follow the lane/dword layout of include/kvc.h.
// INT4 outlier channels (meeting-LLM article section 8.2) get K scale and zero
// 0 in the main store and their fp16 K values in the outlier store; with a V
// outlier store their V is left out of each token's group range (code 0) and
// stored at fp16 too.
// FP8 (E4M3) caches encode every appended row at once (no groups, no tail);
// the channel-major copy then holds the decoded values.
// A second, per-sequence kernel then rewrites the fp16 tail and seq_lens.
// A one-token append (the decode step) runs in a single launch instead: each
// workgroup takes the length with an atomic add that also counts it in bits
// 24..30 of seq_lens[b], writes its new row to the tail itself, and the last
// of the sequence's Hkv workgroups to arrive stores the new length.

#include <type_traits>

#include "internal.h"

namespace kvc {
namespace {

constexpr int NT = 256;   // threads per workgroup
static_assert(NT == GS * KVC_MAX_OUTLIERS, "one thread per (token, outlier entry) of a group");

template <int BITS>
struct GroupQuant {
  // Scale and zero for a group with fp32 extremes mn, mx (fp16 values).
  __device__ static inline void params(float mn, float mx, float& s, float& z,
                                       uint16_t& s16, uint16_t& z16) {
    constexpr float levels = float((1 << BITS) - 1);
    const float s32 = __fadd_rn(__fdiv_rn(__fsub_rn(mx, mn), levels), 0.0f);
    s16 = f2h(s32);
    // a range past the largest finite fp16 scale (1 bit, max - min > 65504)
    // stores 65504 instead of infinity
    if (s16 == 0x7C00u) s16 = 0x7BFFu;
    z16 = f2h(__fadd_rn(mn, 0.0f));
    s = h2f(s16);
    z = h2f(z16);
  }
  // code = rint(fl((x - z) / s)) clamped, from r = recip(s).  a = fl((x - z) * r)
  // lies within 2^-17.9 of fl((x - z) / s) while a < 17 (two roundings of
  // 2^-24 each on a quotient below 17, plus the quotient's own rounding), and
  // any larger a clamps to the top code either way; so rint(a) is the code
  // unless a lies within 2^-17 of a half-integer (|a - rint(a)| >= 0.5 - 2^-17),
  // where the division decides (rare: the branch is skipped by every wave
  // whose lanes all avoid it).  x >= z (z is the group's minimum; values left
  // out of the range get their code elsewhere), so a >= 0 and only the top
  // needs a clamp; s == 0 has r = 0, hence a = 0 and code 0.
  __device__ static inline float recip(float s) { return s == 0.0f ? 0.0f : __fdiv_rn(1.0f, s); }
  __device__ static inline uint32_t code(float x, float s, float z, float r) {
    constexpr float top = float((1 << BITS) - 1);
    const float d = __fsub_rn(x, z);
    const float a = __fmul_rn(d, r);
    float t = rintf(a);
    if (fabsf(__fsub_rn(a, t)) >= 0.5f - 0x1p-17f) t = rintf(__fdiv_rn(d, s));
    return (uint32_t)fminf(t, top);
  }
};

// Arrival count of the one-token path: seq_lens values stay below 2^24 there,
// and at most 127 workgroups per sequence keep the count clear of the sign bit.
constexpr int ARRIVE = 1 << 24;
constexpr int LEN_MASK = ARRIVE - 1;

// Packed-fp16 minimum / maximum of the group quantizer's extremes, written as
// the instructions: the compiler would first canonicalize both operands (two
// more instructions each time).  The inputs are fp16 K / V values; a quiet NaN
// among them is passed over as by fminf / fmaxf.
__device__ inline uint32_t pk_min(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline uint32_t pk_max(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Elementwise minimum / maximum of fp16 pairs over lanes l, l ^ 16, l ^ 32, l ^ 48
// (gfx950 row-swap moves: each swap of a value with itself yields it and the
// partner lane's value).
__device__ inline uint32_t rows_min(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = pk_min(r[0], r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return pk_min(t[0], t[1]);
}
__device__ inline uint32_t rows_max(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = pk_max(r[0], r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return pk_max(t[0], t[1]);
}
// LDS accesses of one wave execute in issue order, so values exchanged through
// LDS inside a wave only need the compiler to keep program order.
__device__ inline void wave_lds_order() { asm volatile("" ::: "memory"); }
// x | the same register of lanes l ^ 1 and l ^ 2 (DPP quad permutations).
__device__ inline uint32_t quad_or(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);   // [1, 0, 3, 2]
  x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);   // [2, 3, 0, 1]
  return x;
}

// Code of one value as a float in [0, 2^BITS - 1] from d = fl(x - z) (see
// GroupQuant::code).  The fast form rounds a = fl(d * r) and returns a - rint(a)
// in e; a caller whose wave saw |e| >= NEAR_HALF anywhere recomputes its codes
// with SLOW, which takes the division where a is that close to a half-integer.
// The fast form's rounding is written as instructions, since the compiler
// would first canonicalize the rounded value for fminf (one more instruction
// per code): 1 bit, rint with the clamp modifier, which is the code
// min(max(rint(a), 0), 1) for the a < 1.5 of an unsaturated scale, while a
// larger a (a saturated scale) lands 0.5 or more from the clamped value and
// takes the second pass; INT4, v_min_f32 with the top code.
constexpr float NEAR_HALF = 0.5f - 0x1p-17f;
// fl(h - z) for the fp16 value h in half H of the dword u and nz = -z, as
// one mixed-precision fma (h * 1 + nz, rounded once): the conversion of h
// rides in the instruction.
template <int H>
__device__ inline float sub_h(uint32_t u, float nz) {
  float d;
  if constexpr (H == 0)
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(u), "v"(nz));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(u), "v"(nz));
  return d;
}
template <int BITS, bool SLOW>
__device__ inline float qcode(float d, float s, float r, float& e) {
  constexpr float TOP = float((1 << BITS) - 1);
  const float a = __fmul_rn(d, r);
  if constexpr (SLOW) {
    float t = rintf(a);
    e = __fsub_rn(a, t);
    if (fabsf(e) >= NEAR_HALF) t = rintf(__fdiv_rn(d, s));
    return fminf(t, TOP);
  } else if constexpr (BITS == 1) {
    float t;
    asm("v_rndne_f32_e64 %0, %1 clamp" : "=v"(t) : "v"(a));
    e = __fsub_rn(a, t);
    return t;
  } else {
    const float t = rintf(a);
    e = __fsub_rn(a, t);
    float q;
    asm("v_min_f32_e32 %0, %1, %2" : "=v"(q) : "s"(TOP), "v"(t));
    return q;
  }
}
// worst of two rounding distances
__device__ inline float worst2(float w, float e0, float e1) { return fmaxf(w, fmaxf(fabsf(e0), fabsf(e1))); }

// Quantizes the complete group [g0, g0 + 64) of (sequence b, KV head g) (all
// NT threads).  Every thread first takes the values it quantizes into registers:
//   K: thread (octet o, row quad rq) = channels [8o, 8o + 8) of rows
//      [4rq, 4rq + 4), so that its codes of one row form one dword of the
//      packed tile (INT4: 8 nibbles of one token; INT1: a quarter of the 32
//      bits of one token, OR-ed over the four lanes of a quad);
//   V: thread (token nv, quarter qv) = channels [32qv, 32qv + 32) of row nv
//      (wave w: rows [16w, 16w + 16), one 16-token tile).
// The V token extremes are combined over two lanes, the K channel extremes
// over the threads of an octet.
// Staged mode (DIRECT false): the rows are in sK / sV (visible to every
// thread); octet o = tid % 16, row quad rq = tid / 16, so an octet's row quads
// span the four waves and the K extremes and parameters go through LDS with
// workgroup barriers; the rows' LDS then holds those and the one-byte V codes.
// DIRECT: row r is read from krow + r * rstride / vrow + r * rstride (a
// complete group of new rows, no outlier channels); wave w takes octets
// [4w, 4w + 4) (o = 4w + lane % 4, rq = lane / 4), so every exchange stays
// inside the wave (its own LDS area, no barrier) and the workgroup never
// synchronizes.
template <int BITS, bool DIRECT = false>
__device__ void quantize_group(const kvc_cache& c, int b, int g, int g0,
                               uint16_t (&sK)[GS][D], uint16_t (&sV)[GS][D], bool kabs,
                               const uint16_t* krow = nullptr, const uint16_t* vrow = nullptr,
                               int64_t rstride = 0) {
  using Q = GroupQuant<BITS>;
  const int tid = threadIdx.x, lane = tid & 63, Hkv = c.num_kv_heads;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_out = (BITS == 4 && !DIRECT) ? c.n_outlier : 0;
  const int G = g0 / GS;
  const int o = DIRECT ? 4 * w + (lane & 3) : (tid & 15);   // K: channel octet
  const int rq = DIRECT ? (lane >> 2) : (tid >> 4);         // K: row quad
  // Slots of the group's four 16-token tiles (a page holds whole tiles, so
  // token 16j + x has slot tslot[j] + x), from uniform tokens.  Wave w's V
  // rows (nv) and outlier rows lie in tile w.
  int64_t tslot[GS / TILE];
#pragma unroll
  for (int j = 0; j < GS / TILE; ++j) tslot[j] = slot_of(c, b, g, g0 + TILE * j);
  const int64_t wslot = w == 0 ? tslot[0] : w == 1 ? tslot[1] : w == 2 ? tslot[2] : tslot[3];

  // ---- V values into registers
  const int nv = tid >> 2, qv = tid & 3, jv = qv >> 1, c0 = 32 * qv;
  uint32_t vw[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint4 u = DIRECT ? *reinterpret_cast<const uint4*>(vrow + nv * rstride + c0 + 8 * k)
                           : *reinterpret_cast<const uint4*>(&sV[nv][c0 + 8 * k]);
    vw[4 * k] = u.x;
    vw[4 * k + 1] = u.y;
    vw[4 * k + 2] = u.z;
    vw[4 * k + 3] = u.w;
  }
  auto vval = [&](int i) { return h2f((uint16_t)(vw[i >> 1] >> (16 * (i & 1)))); };

  // ---- outlier stores: thread (token r, entry j) writes the token's fp16
  // values of outlier channel j (0 past the list)
  if (n_out > 0) {
    const int r = tid >> 2, j = tid & 3;
    const int ch = min(max(c.outlier_ch[g * KVC_MAX_OUTLIERS + j], 0), D - 1);
    if (wslot >= 0) {
      const int64_t slot = wslot + (r & (TILE - 1));
      c.k_outlier[slot * KVC_MAX_OUTLIERS + j] = j < n_out ? sK[r][ch] : (uint16_t)0;
      if (c.v_outlier) c.v_outlier[slot * KVC_MAX_OUTLIERS + j] = j < n_out ? sV[r][ch] : (uint16_t)0;
    }
  }

  // ---- V: per token over each 64-channel half (threads 2m, 2m + 1).  Isolated
  // V outlier channels (bits of vout) stay out of the range and get code 0.
  const bool viso = n_out > 0 && c.v_outlier;
  uint32_t vout = 0u;
  float vmn, vmx;
  if (viso) {
    for (int j = 0; j < n_out; ++j) {
      const int ch = c.outlier_ch[g * KVC_MAX_OUTLIERS + j] - c0;
      if (ch >= 0 && ch < 32) vout |= 1u << ch;
    }
    vmn = INFINITY;
    vmx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const bool out = (vout >> i) & 1u;
      vmn = out ? vmn : fminf(vmn, vval(i));
      vmx = out ? vmx : fmaxf(vmx, vval(i));
    }
  } else {
    uint32_t a = pk_min(vw[0], vw[1]), m = pk_max(vw[0], vw[1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) {
      a = pk_min(a, vw[i]);
      m = pk_max(m, vw[i]);
    }
    vmn = fminf(h2f((uint16_t)a), h2f((uint16_t)(a >> 16)));
    vmx = fmaxf(h2f((uint16_t)m), h2f((uint16_t)(m >> 16)));
  }
  vmn = fminf(vmn, __shfl_xor(vmn, 1));
  vmx = fmaxf(vmx, __shfl_xor(vmx, 1));
  float vs, vz;
  uint16_t vs16, vz16;
  Q::params(vmn, vmx, vs, vz, vs16, vz16);
  if ((qv & 1) == 0 && wslot >= 0) {
    const int64_t slot = wslot + (nv & (TILE - 1));
    c.v_meta[slot * 4 + jv] = vs16;
    c.v_meta[slot * 4 + 2 + jv] = vz16;
  }
  const float vr = Q::recip(vs);
  // one byte per code, channel order.  The second pass (rare, see qcode)
  // takes its parameters through an empty asm so that the compiler keeps no
  // value of the first pass alive for it.
  uint32_t vq[8];
  auto vcodes = [&](auto slow) {
    constexpr bool SLOW = decltype(slow)::value;
    float s = vs, z = vz, r = vr;
    if constexpr (SLOW) asm volatile("" : "+v"(s), "+v"(z), "+v"(r));
    float worst = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      float e0, e1;
      const float q0 = qcode<BITS, SLOW>(sub_h<0>(vw[i >> 1], -z), s, r, e0);
      const float q1 = qcode<BITS, SLOW>(sub_h<1>(vw[i >> 1], -z), s, r, e1);
      worst = worst2(worst, e0, e1);
      vq[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(q0, (uint32_t)(i & 3), (i & 3) ? vq[i >> 2] : 0u);
      vq[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(q1, (uint32_t)((i + 1) & 3), vq[i >> 2]);
    }
    return worst;
  };
  if (__builtin_amdgcn_ballot_w64(vcodes(std::false_type{}) >= NEAR_HALF) != 0)
    vcodes(std::true_type{});
  if (viso) {   // code 0 for the isolated channels: bit i of vout -> byte i of the codes
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t bits = ((((vout >> (4 * m)) & 0xFu) * 0x00204081u) & 0x01010101u);
      vq[m] &= ~((bits << 8) - bits);
    }
  }

  // ---- K values into registers; kw[k][j] = channels 8o + 2j, 8o + 2j + 1 of row 4rq + k
  uint32_t kw[4][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint4 u = DIRECT ? *reinterpret_cast<const uint4*>(krow + (4 * rq + k) * rstride + 8 * o)
                           : *reinterpret_cast<const uint4*>(&sK[4 * rq + k][8 * o]);
    kw[k][0] = u.x;
    kw[k][1] = u.y;
    kw[k][2] = u.z;
    kw[k][3] = u.w;
  }
  // ---- K extremes of the thread's 8 channels over its 4 rows, then over the
  // octet's other row quads in the wave: lanes o + 16i (staged), lanes
  // 4rq + o % 4 (DIRECT: rotations by 4 and 8 inside each 16-lane row first)
  uint32_t kmn[4], kmx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t mn = pk_min(pk_min(kw[0][j], kw[1][j]), pk_min(kw[2][j], kw[3][j]));
    uint32_t mx = pk_max(pk_max(kw[0][j], kw[1][j]), pk_max(kw[2][j], kw[3][j]));
    if constexpr (DIRECT) {
      mn = pk_min(mn, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mn, 0x124, 0xF, 0xF, false));
      mx = pk_max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x124, 0xF, 0xF, false));
      mn = pk_min(mn, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mn, 0x128, 0xF, 0xF, false));
      mx = pk_max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x128, 0xF, 0xF, false));
    }
    kmn[j] = rows_min(mn);
    kmx[j] = rows_max(mx);
  }

  // ---- K parameters, one channel per thread (staged: threads 0..127 after
  // a barrier; DIRECT: channel 32w + lane / 2 in lanes 2m, 2m + 1 of wave w),
  // from the extremes in X; they go to P
  uint8_t (&sVc)[GS][D] = *reinterpret_cast<uint8_t (*)[GS][D]>(&sV[0][0]);
  uint32_t* X;
  float* P;
  if constexpr (DIRECT) {
    X = reinterpret_cast<uint32_t*>(&sK[0][0]) + w * 32;                 // [4 octets][8]
    P = reinterpret_cast<float*>(&sK[0][0]) + (NT / 64) * 32 + w * 96;    // s[32], z[32], 1/s[32]
    if (lane < 4) {
      *reinterpret_cast<uint4*>(X + lane * 8) = uint4{kmn[0], kmn[1], kmn[2], kmn[3]};
      *reinterpret_cast<uint4*>(X + lane * 8 + 4) = uint4{kmx[0], kmx[1], kmx[2], kmx[3]};
    }
    *reinterpret_cast<uint4*>(&sVc[nv][c0]) = uint4{vq[0], vq[1], vq[2], vq[3]};
    *reinterpret_cast<uint4*>(&sVc[nv][c0 + 16]) = uint4{vq[4], vq[5], vq[6], vq[7]};
    wave_lds_order();
  } else {
    // every row value is in registers: the rows' LDS takes the K extremes
    // (per wave and octet: 4 min pairs, 4 max pairs), the K parameters and the V codes
    __syncthreads();
    X = reinterpret_cast<uint32_t*>(&sK[0][0]);                          // [4 waves][16 octets][8]
    P = reinterpret_cast<float*>(&sK[0][0]) + (NT / 64) * 16 * 8;         // s[D], z[D], 1/s[D]
    if (lane < 16) {
      *reinterpret_cast<uint4*>(X + (w * 16 + o) * 8) = uint4{kmn[0], kmn[1], kmn[2], kmn[3]};
      *reinterpret_cast<uint4*>(X + (w * 16 + o) * 8 + 4) = uint4{kmx[0], kmx[1], kmx[2], kmx[3]};
    }
    *reinterpret_cast<uint4*>(&sVc[nv][c0]) = uint4{vq[0], vq[1], vq[2], vq[3]};
    *reinterpret_cast<uint4*>(&sVc[nv][c0 + 16]) = uint4{vq[4], vq[5], vq[6], vq[7]};
    __syncthreads();
  }
  if (DIRECT || tid < D) {
    const int cl = DIRECT ? (lane >> 1) : tid;         // channel inside P
    const int ck = DIRECT ? 32 * w + cl : tid;         // channel of the head
    const int oc = cl >> 3, j = (cl & 7) >> 1, sh = 16 * (cl & 1);
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < (DIRECT ? 1 : NT / 64); ++ww) {
      mn = fminf(mn, h2f((uint16_t)(X[(ww * 16 + oc) * 8 + j] >> sh)));
      mx = fmaxf(mx, h2f((uint16_t)(X[(ww * 16 + oc) * 8 + 4 + j] >> sh)));
    }
    const bool writer = !DIRECT || (lane & 1) == 0;
    // max|K| of a group whose rows are all new: the larger magnitude of its extremes
    if (kabs && writer)
      atomicMax(reinterpret_cast<unsigned int*>(c.k_absmax) + ((int64_t)b * Hkv + g) * D + ck,
                __float_as_uint(fmaxf(fabsf(mn), fabsf(mx))));
    // outlier channels (INT4): scale and zero 0, hence codes 0; their values
    // went to the fp16 outlier store above
    for (int e = 0; e < n_out; ++e)
      if (c.outlier_ch[g * KVC_MAX_OUTLIERS + e] == ck) mn = mx = 0.0f;
    float s, z;
    uint16_t s16, z16;
    Q::params(mn, mx, s, z, s16, z16);
    if (writer) {
      uint16_t* meta = c.k_meta + ((((int64_t)b * Hkv + g) * (c.max_tokens / GS) + G) * 2) * D;
      meta[ck] = s16;
      meta[D + ck] = z16;
      const int np = DIRECT ? 32 : D;
      P[cl] = s;
      P[np + cl] = z;
      P[2 * np + cl] = Q::recip(s);
    }
  }
  if constexpr (DIRECT) wave_lds_order();
  else __syncthreads();

  // ---- K codes, one packed dword per row
  float ks[8], kz[8], kr[8];
  {
    const int np = DIRECT ? 32 : D, pc = DIRECT ? 8 * (lane & 3) : 8 * o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 s4 = *reinterpret_cast<const float4*>(P + pc + 4 * h);
      const float4 z4 = *reinterpret_cast<const float4*>(P + np + pc + 4 * h);
      const float4 r4 = *reinterpret_cast<const float4*>(P + 2 * np + pc + 4 * h);
      ks[4 * h] = s4.x; ks[4 * h + 1] = s4.y; ks[4 * h + 2] = s4.z; ks[4 * h + 3] = s4.w;
      kz[4 * h] = z4.x; kz[4 * h + 1] = z4.y; kz[4 * h + 2] = z4.z; kz[4 * h + 3] = z4.w;
      kr[4 * h] = r4.x; kr[4 * h + 1] = r4.y; kr[4 * h + 2] = r4.z; kr[4 * h + 3] = r4.w;
    }
  }
  uint32_t kd[4];
  auto kcodes = [&](auto slow) {
    constexpr bool SLOW = decltype(slow)::value;
    if constexpr (SLOW) {   // (as for V)
#pragma unroll
      for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(ks[e]), "+v"(kz[e]), "+v"(kr[e]));
    }
    float worst = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float q[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float e0, e1;
        q[2 * j] = qcode<BITS, SLOW>(sub_h<0>(kw[k][j], -kz[2 * j]), ks[2 * j], kr[2 * j], e0);
        q[2 * j + 1] = qcode<BITS, SLOW>(sub_h<1>(kw[k][j], -kz[2 * j + 1]), ks[2 * j + 1], kr[2 * j + 1], e1);
        worst = worst2(worst, e0, e1);
      }
      if constexpr (BITS == 4) {
        // channel e of the octet is nibble slot e (bit 16 (e & 1) + 4 (e >> 1)):
        // byte 0 = slots 0 | 2 << 4, byte 1 = 4 | 6 << 4, byte 2 = 1 | 3 << 4, byte 3 = 5 | 7 << 4
        uint32_t u = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[2], 16.0f, q[0]), 0u, 0u);
        u = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[6], 16.0f, q[4]), 1u, u);
        u = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[3], 16.0f, q[1]), 2u, u);
        kd[k] = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[7], 16.0f, q[5]), 3u, u);
      } else {
        // octet 0 of a 32-channel block: channel e at bit 6 + (e >> 1) + 16 (e & 1)
        // (bits 6..25, so the float sum of the set bits is exact)
        float f = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f = fmaf(q[e], float(1u << (6 + (e >> 1) + 16 * (e & 1))), f);
        kd[k] = (uint32_t)f;
      }
    }
    return worst;
  };
  if (__builtin_amdgcn_ballot_w64(kcodes(std::false_type{}) >= NEAR_HALF) != 0)
    kcodes(std::true_type{});

  if constexpr (BITS == 4) {
    // K tile of rows [16 tile, 16 tile + 16): lane 16 (c / 32) + n, dword (c % 32) / 8
    const int tq = rq >> 2;
    const int64_t slot = tq == 0 ? tslot[0] : tq == 1 ? tslot[1] : tq == 2 ? tslot[2] : tslot[3];
    if (slot >= 0) {
      uint32_t* unit = reinterpret_cast<uint32_t*>(c.k_codes + (slot / TILE) * UNIT_BYTES);
#pragma unroll
      for (int k = 0; k < 4; ++k) unit[4 * (16 * (o >> 2) + ((4 * rq + k) & 15)) + (o & 3)] = kd[k];
    }
  } else {
    // octet v = o % 4 of its 32-channel block: octet 0's bit pattern rotated
    // left by 0 / 4 / 28 / 24 bits, then OR-ed over the quad; lane v stores row 4rq + v
    const int v = o & 3;
    const uint32_t rr = v == 0 ? 0u : v == 1 ? 28u : v == 2 ? 4u : 8u;   // right rotation
#pragma unroll
    for (int k = 0; k < 4; ++k) kd[k] = quad_or(__builtin_amdgcn_alignbit(kd[k], kd[k], rr));
    const uint32_t mine = v == 0 ? kd[0] : v == 1 ? kd[1] : v == 2 ? kd[2] : kd[3];
    const int64_t slot = tslot[0];
    if (slot >= 0) {
      const int n = 4 * rq + v;
      // lane 16 (c / 32) + n % 16, dword n / 16
      reinterpret_cast<uint32_t*>(c.k_codes + (slot / GS) * UNIT_BYTES)[4 * (16 * (o >> 2) + (n & 15)) + (n >> 4)] = mine;
    }
  }

  // ---- V: pack the byte codes into the lane/dword tile layout.  Staged: thread
  // W writes dword W of every tile; DIRECT: wave w packs its own rows (tile w;
  // 1 bit: dword w of every lane), 4 dwords a lane (INT4) or 1 (1 bit).
  if constexpr (BITS == 4) {
#pragma unroll
    for (int it = 0; it < (DIRECT ? 4 : GS / TILE); ++it) {
      const int tile = DIRECT ? w : it, W = DIRECT ? lane + 64 * it : tid;
      const int64_t slot = DIRECT ? wslot : tslot[it];
      if (slot < 0) continue;
      // lane = 16*(n/4) + c%16, dword d = (c/16)/2, nibble j = 4*((c/16)%2) + n%4
      const int vl = W >> 2, d = W & 3, kb = vl >> 4, m = vl & 15;
      uint32_t u = 0;
#pragma unroll
      for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          u |= (uint32_t)sVc[TILE * tile + 4 * kb + i][16 * (2 * d + par) + m] << nib_pos(4 * par + i);
      reinterpret_cast<uint32_t*>(c.v_codes + (slot / TILE) * UNIT_BYTES)[W] = u;
    }
  } else {
    const int64_t slot = tslot[0];
    if (slot >= 0) {
      // lane = 16*((n%16)/4) + c%16, dword d = n/16, code k = v1_code(c/16, n%4)
      const int vl = DIRECT ? lane : (tid >> 2), d = DIRECT ? w : (tid & 3), kb = vl >> 4, m = vl & 15;
      uint32_t u = 0;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          u |= (uint32_t)sVc[16 * d + 4 * kb + i][16 * ct + m] << bit_pos(v1_code(ct, i));
      reinterpret_cast<uint32_t*>(c.v_codes + (slot / GS) * UNIT_BYTES)[4 * vl + d] = u;
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(NT, 5) void append_groups_kernel(
    kvc_cache c, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ n_new, int n_new_max) {
  constexpr int BITS = FMT == KVC_FMT_INT4 ? 4 : 1;
  __shared__ __align__(16) uint16_t sK[GS][D];
  __shared__ __align__(16) uint16_t sV[GS][D];

  // x = (group, KV head), the head fastest: the Hkv workgroups of one group
  // run together and read adjacent 256-byte pieces of the same new rows
  const int Hkv = c.num_kv_heads;
  const int b = blockIdx.z, gx = (int)blockIdx.x / Hkv, g = (int)blockIdx.x - gx * Hkv;
  const int tid = threadIdx.x;
  const int L = c.seq_lens[b];
  const int n = n_new ? n_new[b] : n_new_max;
  if (n <= 0 || n > n_new_max || L < 0 || L + n > c.max_tokens) return;
  const int g0 = (L / GS + gx) * GS;
  if (g0 >= L + n) return;
  const int hi = min(g0 + GS, L + n);   // tokens [g0, hi) exist after the append
  const int lo = max(g0, L);            // tokens [lo, hi) are new

  // Old rows [g0, L) are read back from the tail only when this append completes
  // the group of a quantized cache (nothing else needs them; an fp16 cache has no tail).
  const bool complete = grouped(FMT) && hi == g0 + GS;
  const int r0 = complete ? 0 : lo - g0;

  // A complete group of new rows on a cache without fp16 copies or outlier
  // channels (the bulk of a prefill) goes straight from the new rows to the
  // quantizer's registers.
  if constexpr (grouped(FMT)) {
    if (complete && lo == g0 && !c.k16 && !c.kT && (BITS == 1 || c.n_outlier == 0)) {
      const int64_t base = (((int64_t)b * n_new_max + (g0 - L)) * Hkv + g) * D;
      quantize_group<BITS, true>(c, b, g, g0, sK, sV, c.k_absmax != nullptr, k_new + base,
                                 v_new + base, (int64_t)Hkv * D);
      return;
    }
  }

  // ---- stage rows [g0 + r0, hi) in LDS: 16 threads per row, 8 halves each.
  // Every thread issues all of its (up to 4 + 4) row loads before its first
  // LDS store, with no branch between them: an element past the rows repeats
  // the last one (the same value loaded and stored to the same place again).
  constexpr int PER = GS * 16 / NT;
  const int nst = (hi - g0 - r0) * 16;
  uint4 ks[PER], vs[PER];
  int es[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = es[i] = min(tid + i * NT, nst - 1);
    const int r = r0 + (e >> 4), ch = (e & 15) * 8;
    const int t = g0 + r;
    const int64_t offT = (((int64_t)b * Hkv + g) * GS + r) * D + ch;   // old row, in the tail
    const int64_t offN = (((int64_t)b * n_new_max + max(t - L, 0)) * Hkv + g) * D + ch;
    const uint16_t* srcK = t < L ? c.k_tail + offT : k_new + offN;
    const uint16_t* srcV = t < L ? c.v_tail + offT : v_new + offN;
    ks[i] = *reinterpret_cast<const uint4*>(srcK);
    vs[i] = *reinterpret_cast<const uint4*>(srcV);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int r = r0 + (es[i] >> 4), ch = (es[i] & 15) * 8;
    *reinterpret_cast<uint4*>(&sK[r][ch]) = ks[i];
    *reinterpret_cast<uint4*>(&sV[r][ch]) = vs[i];
  }
  __syncthreads();

  // ---- fp16 row copies of the new tokens
  if (c.k16) {
    for (int e = tid; e < (hi - lo) * 16; e += NT) {
      const int r = lo - g0 + (e >> 4), ch = (e & 15) * 8;
      const int64_t slot = slot_of(c, b, g, g0 + r);
      if (slot < 0) continue;
      *reinterpret_cast<uint4*>(c.k16 + slot * D + ch) = *reinterpret_cast<const uint4*>(&sK[r][ch]);
      *reinterpret_cast<uint4*>(c.v16 + slot * D + ch) = *reinterpret_cast<const uint4*>(&sV[r][ch]);
    }
  }
  if constexpr (FMT == KVC_FMT_FP8) {   // E4M3 rows: 16 threads per row, 8 codes each
    for (int e = tid; e < (hi - lo) * 16; e += NT) {
      const int r = lo - g0 + (e >> 4), ch = (e & 15) * 8;
      const int64_t slot = slot_of(c, b, g, g0 + r);
      if (slot < 0) continue;
      const uint4 kx = *reinterpret_cast<const uint4*>(&sK[r][ch]);
      const uint4 vx = *reinterpret_cast<const uint4*>(&sV[r][ch]);
      *reinterpret_cast<uint2*>(c.k_codes + slot * D + ch) =
          uint2{fp8_encode2(kx.x) | (fp8_encode2(kx.y) << 16), fp8_encode2(kx.z) | (fp8_encode2(kx.w) << 16)};
      *reinterpret_cast<uint2*>(c.v_codes + slot * D + ch) =
          uint2{fp8_encode2(vx.x) | (fp8_encode2(vx.y) << 16), fp8_encode2(vx.z) | (fp8_encode2(vx.w) << 16)};
    }
  }
  if (c.kT) {  // channel-major: consecutive lanes write consecutive tokens of one channel
    for (int e = tid; e < (hi - lo) * D; e += NT) {
      const int ch = e / (hi - lo), r = lo - g0 + e % (hi - lo);
      uint16_t x = sK[r][ch];
      if constexpr (FMT == KVC_FMT_FP8)   // the decoded value (exact in fp16)
        x = f2h(h2f((uint16_t)fp8_h16_over256(fp8_encode2(x) & 0xFFu)) * 256.0f);
      c.kT[(((int64_t)b * Hkv + g) * D + ch) * c.max_tokens + g0 + r] = x;
    }
  }
  // (a complete group of new rows takes max|K| from its extremes instead)
  const bool abs_from_group = complete && lo == g0;
  if (c.k_absmax && tid < D && !abs_from_group) {
    float m = 0.0f;
#pragma unroll 16
    for (int r = lo - g0; r < hi - g0; ++r) m = fmaxf(m, fabsf(h2f(sK[r][tid])));
    atomicMax(reinterpret_cast<unsigned int*>(c.k_absmax) + ((int64_t)b * Hkv + g) * D + tid,
              __float_as_uint(m));
  }

  if constexpr (grouped(FMT)) {
    if (complete) quantize_group<BITS>(c, b, g, g0, sK, sV, c.k_absmax && abs_from_group);
  }
}

// One-token append (a decode step) in a single launch: one workgroup per (KV
// head g, sequence b).  Thread 0 takes the length L with an atomic add of
// ARRIVE to seq_lens[b] (bits 24..30 count the sequence's workgroups); the
// last of the Hkv to arrive stores L + 1 there, or L when n_new[b] is 0, or L
// with the overflow flag when the token does not fit (or n_new[b] > 1).  Each
// workgroup alone owns its (b, g) row of k_absmax, so max|K| is a plain
// read-compare-store.  Every other write of the
// token comes from registers: threads 0..15 hold 8 channels of the new K and V
// row each (fp16 copies, E4M3 codes, tail row), threads 0..127 one K channel
// (max|K|, channel-major copy).  Only a step that completes its group (L % 64
// == 63) stages the 63 tail rows in LDS and quantizes; the tail is then empty,
// so no workgroup writes it in that step.
template <int FMT>
__global__ __launch_bounds__(NT, 5) void append_token_kernel(
    kvc_cache c, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ n_new, int32_t* overflow) {
  constexpr int BITS = FMT == KVC_FMT_INT4 ? 4 : 1;
  __shared__ __align__(16) uint16_t sK[GS][D];
  __shared__ __align__(16) uint16_t sV[GS][D];
  __shared__ int sL;

  const int b = blockIdx.z, g = blockIdx.y, tid = threadIdx.x;
  const int Hkv = c.num_kv_heads;
  const int64_t row = ((int64_t)b * Hkv + g) * D;   // the new row in k_new / v_new
  // Every load below is independent of the length: all of them are in flight
  // together with the atomic (n_new[b] too: a sequence with nothing to append
  // still counts its workgroups and gets its length stored back unchanged).
  uint4 nk = {}, nv = {};
  uint16_t kc = 0;
  uint32_t kabs = 0u;   // max|K| so far of channel tid, as bits (this workgroup alone updates it)
  if (tid < 16) {
    nk = *reinterpret_cast<const uint4*>(k_new + row + tid * 8);
    nv = *reinterpret_cast<const uint4*>(v_new + row + tid * 8);
  }
  if (tid < D) {
    kc = k_new[row + tid];
    if (c.k_absmax) kabs = reinterpret_cast<const uint32_t*>(c.k_absmax)[row + tid];
  }
  if (tid == 0) {
    const int n = n_new ? n_new[b] : 1;
    const int old = atomicAdd(c.seq_lens + b, ARRIVE);
    const int len = old & LEN_MASK;
    const bool ok = n == 1 && len + 1 <= c.max_tokens;
    if ((old >> 24) == Hkv - 1) {   // every workgroup of sequence b holds the length now
      __hip_atomic_store(c.seq_lens + b, len + (ok ? 1 : 0), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (n > 0 && !ok && overflow) *overflow = 1;
    }
    sL = ok ? len : -1;
  }
  __syncthreads();
  const int L = sL;
  if (L < 0) return;
  const int g0 = L & ~(GS - 1), r = L - g0;
  const bool complete = grouped(FMT) && r == GS - 1;

  if (tid < 16) {
    const int ch = tid * 8;
    if (c.k16 || FMT == KVC_FMT_FP8) {
      const int64_t slot = slot_of(c, b, g, L);
      if (slot >= 0 && c.k16) {
        *reinterpret_cast<uint4*>(c.k16 + slot * D + ch) = nk;
        *reinterpret_cast<uint4*>(c.v16 + slot * D + ch) = nv;
      }
      if constexpr (FMT == KVC_FMT_FP8) {
        if (slot >= 0) {
          *reinterpret_cast<uint2*>(c.k_codes + slot * D + ch) =
              uint2{fp8_encode2(nk.x) | (fp8_encode2(nk.y) << 16), fp8_encode2(nk.z) | (fp8_encode2(nk.w) << 16)};
          *reinterpret_cast<uint2*>(c.v_codes + slot * D + ch) =
              uint2{fp8_encode2(nv.x) | (fp8_encode2(nv.y) << 16), fp8_encode2(nv.z) | (fp8_encode2(nv.w) << 16)};
        }
      }
    }
    if constexpr (grouped(FMT)) {
      if (complete) {
        *reinterpret_cast<uint4*>(&sK[r][ch]) = nk;
        *reinterpret_cast<uint4*>(&sV[r][ch]) = nv;
      } else {   // the row joins the tail
        const int64_t off = (((int64_t)b * Hkv + g) * GS + r) * D + ch;
        *reinterpret_cast<uint4*>(c.k_tail + off) = nk;
        *reinterpret_cast<uint4*>(c.v_tail + off) = nv;
      }
    }
  }
  if (tid < D) {
    if (c.kT) {
      uint16_t x = kc;
      if constexpr (FMT == KVC_FMT_FP8)   // the decoded value (exact in fp16)
        x = f2h(h2f((uint16_t)fp8_h16_over256(fp8_encode2(x) & 0xFFu)) * 256.0f);
      c.kT[(row + tid) * c.max_tokens + L] = x;
    }
    // the same order as the unsigned atomic max of the multi-token path
    const uint32_t a = __float_as_uint(fabsf(h2f(kc)));
    if (c.k_absmax && a > kabs) reinterpret_cast<uint32_t*>(c.k_absmax)[row + tid] = a;
  }

  if constexpr (grouped(FMT)) {
    if (!complete) return;
    // ---- stage the 63 old rows from the tail: 16 threads per row, 8 halves each
    for (int e = tid; e < r * 16; e += NT) {
      const int rr = e >> 4, ch = (e & 15) * 8;
      const int64_t off = (((int64_t)b * Hkv + g) * GS + rr) * D + ch;
      *reinterpret_cast<uint4*>(&sK[rr][ch]) = *reinterpret_cast<const uint4*>(c.k_tail + off);
      *reinterpret_cast<uint4*>(&sV[rr][ch]) = *reinterpret_cast<const uint4*>(c.v_tail + off);
    }
    __syncthreads();
    quantize_group<BITS>(c, b, g, g0, sK, sV, false);
  }
}

// Per sequence: move the rows of the (new) incomplete group into the tail and
// publish the new length.  Runs after append_groups_kernel on the same stream,
// so every old tail row it overwrites has already been consumed.
__global__ __launch_bounds__(NT) void append_finish_kernel(
    kvc_cache c, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ n_new, int n_new_max, int32_t* overflow) {
  const int b = blockIdx.x, tid = threadIdx.x, Hkv = c.num_kv_heads;
  const int L = c.seq_lens[b];
  const int n = n_new ? n_new[b] : n_new_max;
  if (n <= 0) return;
  if (n > n_new_max || L < 0 || L + n > c.max_tokens) {
    if (tid == 0 && overflow) *overflow = 1;
    return;
  }
  const bool quantized = grouped(c.format);
  if (quantized) {
    const int nq_old = L & ~(GS - 1), nq_new = (L + n) & ~(GS - 1);
    const int t0 = nq_new > nq_old ? nq_new : L;  // first token to place in the tail
    const int rows = L + n - t0;
    for (int e = tid; e < rows * Hkv * 16; e += NT) {
      const int ch = (e & 15) * 8, rg = e >> 4, g = rg % Hkv, r = rg / Hkv;
      const int t = t0 + r;
      const int64_t src = (((int64_t)b * n_new_max + (t - L)) * Hkv + g) * D + ch;
      const int64_t dst = (((int64_t)b * Hkv + g) * GS + (t - nq_new)) * D + ch;
      *reinterpret_cast<uint4*>(c.k_tail + dst) = *reinterpret_cast<const uint4*>(k_new + src);
      *reinterpret_cast<uint4*>(c.v_tail + dst) = *reinterpret_cast<const uint4*>(v_new + src);
    }
  }
  __syncthreads();
  if (tid == 0) c.seq_lens[b] = L + n;
}

}  // namespace

hipError_t launch_append(const kvc_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* n_new, int32_t n_new_max, int32_t* overflow,
                         hipStream_t s) {
  if (n_new_max <= 0) return hipSuccess;
  // one token: a single launch (the arrival count needs lengths below 2^24
  // and at most 127 KV heads)
  const bool one = n_new_max == 1 && c.max_tokens < ARRIVE && c.num_kv_heads <= 127;
  const dim3 grid_one(1, c.num_kv_heads, c.batch);
  const dim3 grid((uint32_t)((n_new_max + GS - 1) / GS + 1) * (uint32_t)c.num_kv_heads, 1, c.batch);
  auto run = [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    if (one)
      append_token_kernel<F><<<grid_one, NT, 0, s>>>(c, k_new, v_new, n_new, overflow);
    else
      append_groups_kernel<F><<<grid, NT, 0, s>>>(c, k_new, v_new, n_new, n_new_max);
  };
  switch (c.format) {
    case KVC_FMT_INT4: run(std::integral_constant<int, KVC_FMT_INT4>{}); break;
    case KVC_FMT_INT1: run(std::integral_constant<int, KVC_FMT_INT1>{}); break;
    case KVC_FMT_FP8: run(std::integral_constant<int, KVC_FMT_FP8>{}); break;
    default: run(std::integral_constant<int, KVC_FMT_FP16>{}); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || one) return e;
  append_finish_kernel<<<c.batch, NT, 0, s>>>(c, k_new, v_new, n_new, n_new_max, overflow);
  return hipGetLastError();
}

}  // namespace kvc
