/*
 * kvc.h -- one decode step of attention over a jointly sparsified and quantized
 * KV cache, on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operations follow the problem statement of four pages:
 *   [TKV]  TailorKV article (http://www.ijyty.com/news/1204784): 1-bit layers
 *          with K quantized per channel and V per token (section 2.2, printed
 *          quantizer), critical channels s_i = |q_i| max|K_i| and approximate
 *          scores from them, Top-K token retrieval (section 2.3), the knobs
 *          critical_channels = 8 and sparse_ratio = 0.03 (section 5.1), group
 *          sizes that are multiples of 64 (section 5.2).
 *   [MTG]  meeting-LLM KV article (https://www.ufo.work/2026/545.html):
 *          query-aware scores and Top-K (section 2.2), hot fp16 / warm
 *          quantized tiers (section 3.1), the FlashDecoding-Sparse decode step
 *          with online softmax (section 8.1).
 *   [SRV]  KV compression survey (https://bbs.huaweicloud.com/blogs/490932):
 *          16-token PagedAttention blocks and block tables (section 1),
 *          attention sinks plus a recent window (section 3.1), H2O cumulative
 *          scores (section 3.2).
 *   [DEV]  on-device KV article (https://www.ufo.work/2026/495.html): INT4 K
 *          asymmetric per channel with zero point, V in groups of 64
 *          (section 3.1); a fused dequantize -> QK^T -> softmax -> PV kernel
 *          with scales and zero points held on chip (section 3.2).
 *
 * Conventions for every entry point
 *   - All data pointers are device pointers owned by the caller.  The library
 *     allocates nothing, frees nothing and keeps no state between calls; it is
 *     reentrant.  Calls that share a workspace or outputs must not overlap.
 *   - Every call validates its arguments on the host, enqueues kernels on
 *     ``stream`` and returns without synchronizing.  On a validation error
 *     nothing is enqueued and no output is touched.  Device faults surface at
 *     the caller's next synchronization.
 *   - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *   - head_dim is 128 and the quantization group is 64; other values return
 *     KVC_ERR_UNSUPPORTED.
 *   - Code and row pointers must be 16-byte aligned, metadata pointers 8-byte
 *     aligned (KVC_ERR_INVALID otherwise).
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 4
#define KVC_HEAD_DIM 128
#define KVC_GROUP 64
#define KVC_MAX_GQA 8          /* query heads per KV head supported by attend */
#define KVC_MAX_OUTLIERS 4     /* fp16 outlier channels per KV head (INT4) */
#define KVC_MAX_WORKGROUPS 65536  /* largest workgroup count an attend call may be planned for */
#define KVC_TOPK_MAX_ITEMS (1 << 24)  /* kvc_score_topk: max_tokens at most this */
#define KVC_NOALLOC_SCRATCH_BYTES (32u << 20)  /* static scratch of kvc_attend_decode_noalloc */

typedef int32_t kvc_status;
enum {
  KVC_OK = 0,
  KVC_ERR_INVALID = 1,      /* null pointer, bad range, misalignment */
  KVC_ERR_SHAPE = 2,        /* inconsistent sizes */
  KVC_ERR_UNSUPPORTED = 3,  /* format / mode / size not built */
  KVC_ERR_WORKSPACE = 4,    /* workspace missing or too small */
  KVC_ERR_HIP = 5,          /* a kernel launch failed (hipGetLastError) */
  KVC_ERR_SCRATCH = 6       /* kvc_attend_decode_noalloc: the call needs more than the
                               static scratch (KVC_NOALLOC_SCRATCH_BYTES) */
};

enum { KVC_FMT_FP16 = 0, KVC_FMT_INT4 = 1, KVC_FMT_INT1 = 2, KVC_FMT_FP8 = 3 };
enum { KVC_SCORE_EXACT = 0, KVC_SCORE_CRITICAL = 1, KVC_SCORE_EXTERNAL = 2 };
/* OR'ed into a score mode: rank 64-token blocks instead of tokens ([MTG] 8.1) */
enum { KVC_SCORE_BLOCKS = 16 };
enum { KVC_ATTEND_DENSE = 0, KVC_ATTEND_DROP = 1, KVC_ATTEND_KEEP = 2, KVC_ATTEND_BLOCKS = 3 };
enum { KVC_OP_SCORE_TOPK = 1, KVC_OP_ATTEND = 2, KVC_OP_TOPK_MASS = 3 };

/*
 * kvc_cache -- description of one layer's KV cache (plain data, caller-owned
 * device buffers).  B sequences, Hkv KV heads, D = 128 channels.
 *
 * Token addressing.  Let P = page_size if page_size > 0, else max_tokens.
 * Token t of sequence b lives on logical page t / P at offset t % P; the
 * physical page is block_table[b * max_pages + t / P] when paged, else b.
 * Its "slot" for KV head g is  slot = (phys * Hkv + g) * P + t % P.
 * (Paging follows [SRV] section 1: logical blocks mapped to physical blocks.)
 *
 * Quantized store (format INT4 or INT1; [TKV] 2.2, [DEV] 3.1).  K is quantized
 * per channel over each complete 64-token group, V per token over each
 * 64-channel half, both asymmetric min-max with fp16 scale s and zero z:
 *     s = fp16((max - min) / (2^b - 1) + 0)   (fp32 subtract and divide; a
 *         result past the largest finite fp16 stores 65504: only a 1-bit group
 *         with max - min > 65504 reaches it)
 *     z = fp16(min + 0)
 *     code = s == 0 ? 0 : clamp(rint((x - z) / s), 0, 2^b - 1)   (fp32, half-even)
 * and dequantized as code * s + z.  A group is quantized when its 64th token
 * is appended; until then its tokens live in the fp16 tail.
 *
 *   k_codes, v_codes  Code tiles.  INT4: one 1024-byte tile per 16 slots,
 *     tile index slot / 16.  INT1: one 1024-byte unit per 64 slots, unit index
 *     slot / 64.  Within a tile/unit, byte offset 16*L + 4*d addresses dword d
 *     of "lane" L (0..63, L = 16*hi + lo); bit positions below.
 *     Nibble slot j (0..7) of an INT4 dword sits at bits 16*(j&1) + 4*(j>>1).
 *       INT4 K, token n (0..15) of the tile, channel c:
 *         L = 16*(c/32) + n, d = (c%32)/8, j = c%8.
 *       INT4 V, token n, channel c:
 *         L = 16*(n/4) + c%16, d = (c/16)/2, j = 4*((c/16)%2) + n%4.
 *     Bit positions of an INT1 dword (32 codes): code k (0..31) -> word
 *       w = k/2, half h = k%2, variant v = w/4, p = 6 + w%4; bit
 *         v=0: p + 16h      v=1: p + 4 + 16h
 *         v=2: p - 4 + 16h  v=3: h ? p + 8 : (p + 24) % 32
 *       INT1 K, token n (0..63) of the unit, channel c:
 *         L = 16*(c/32) + n%16, d = n/16, k = c%32.
 *       INT1 V, token n, channel c (ct = c/16, i = n%4):
 *         L = 16*((n%16)/4) + c%16, d = n/16,
 *         k = 2*(4*((ct/4)*2 + i/2) + ct%4) + i%2.
 *     (These orders let a shift and one mask-and-or per pair of codes produce
 *     fp16 matrix-core operands.)
 *   k_meta  fp16 [B][Hkv][max_tokens/64][2][128]: [..][0][c] scale, [..][1][c]
 *     zero of channel c for that 64-token group (per sequence, not paged).
 *   v_meta  fp16 [slot][4]: scale of channels 0-63, scale of 64-127, zero of
 *     0-63, zero of 64-127.
 *   k_tail, v_tail  fp16 [B][Hkv][64][128]: row r holds token 64*floor(n/64) + r
 *     of the incomplete group (n = seq_lens[b]).
 *
 * FP8 store (format FP8: the warm tier in E4M3, [MTG] 6.2, [SRV] 2).  Every
 * appended element is cast to E4M3 (1 sign, 4 exponent bits of bias 7, 3
 * mantissa bits, subnormals, largest finite 448): the nearest value, ties to
 * the even code, saturating at +-448, sign kept; no scale.
 *   k_codes, v_codes  uint8 [slot][128]: the codes of channel c at byte c of
 *     the slot's row.  k_meta, v_meta, k_tail, v_tail are unused (may be NULL);
 *     tokens never wait in a tail.  kT, if given, holds the decoded values.
 *   KVC_ATTEND_KEEP is not supported on FP8.
 *
 * fp16 rows (format FP16: the main store; INT4/INT1: an optional full copy of
 * every appended token, required by KVC_ATTEND_KEEP; [MTG] 3.1 hot tier,
 * [TKV] 3.1 key-token buffer):
 *   k16, v16  fp16 [slot][128].
 *   kT        optional fp16 [B][Hkv][128][max_tokens], channel-major K
 *             (page_size must be 0); lets critical-channel scoring read 8
 *             channels without touching whole rows ([TKV] 2.3).
 *   k_absmax  float32 [B][Hkv][128]: max |K| per channel over all appended
 *             tokens (fp16-exact values); zero-filled by the caller at creation.
 *   seq_lens  int32 [B]: tokens cached per sequence, each in [0, max_tokens];
 *             updated by kvc_quantize_append (while a one-token append runs,
 *             bits 24..30 count its workgroups: nothing may read seq_lens
 *             concurrently with an append).
 *
 * Outlier channels (INT4 only; [MTG] 8.2: the few channels of very large
 * magnitude are found offline by their variance and kept at full precision
 * beside the quantized main store).  With n_outlier = m in 1..4, channels
 * outlier_ch[4*g + j] (j < m; ascending, distinct, 0..127) of KV head g are
 * outlier channels; the list is device int32 [Hkv][4], 16-byte aligned (ids
 * outside 0..127 are clamped where memory is indexed: undefined results, no
 * out-of-bounds access).  When a group is quantized their K scale and zero
 * are stored as 0 (so their codes are 0) and their fp16 values go to
 *   k_outlier  fp16 [slot][4], 8-byte aligned: entry j holds channel
 *              outlier_ch[4*g + j] (entries j >= m hold 0).
 * Dequantized K is then code*s + z on the other channels and the fp16 value
 * on the outlier channels.  With v_outlier set, the same channels of V are
 * isolated too: each token's V group range (min, max) is taken over the
 * group's other channels, the outlier channels get code 0, and
 *   v_outlier  fp16 [slot][4], 8-byte aligned: entry j holds V channel
 *              outlier_ch[4*g + j] (entries j >= m hold 0),
 * which dequantized V takes on those channels; v_outlier NULL leaves V as
 * without outliers.  The channel list is the caller's (an offline analysis)
 * and must not change over the cache's life.  n_outlier = 0 ignores
 * outlier_ch, k_outlier and v_outlier.
 */
typedef struct kvc_cache {
  int32_t abi_version;     /* KVC_ABI_VERSION */
  int32_t format;          /* KVC_FMT_* */
  int32_t batch;           /* B >= 1 */
  int32_t num_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;        /* 128 */
  int32_t group_size;      /* 64 */
  int32_t page_size;       /* 0 = contiguous; else multiple of 16 (64 for INT1) */
  int32_t max_tokens;      /* per-sequence capacity, multiple of 64 (and of page_size) */
  int32_t max_pages;       /* block_table row length (paged) */
  int32_t num_pages;       /* physical pages in each pool (paged) */
  const int32_t* block_table;
  int32_t* seq_lens;
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_meta;
  uint16_t* v_meta;
  uint16_t* k_tail;
  uint16_t* v_tail;
  uint16_t* k16;
  uint16_t* v16;
  uint16_t* kT;
  float* k_absmax;
  int32_t n_outlier;         /* 0..KVC_MAX_OUTLIERS fp16 outlier channels (INT4 only) */
  const int32_t* outlier_ch; /* int32 [Hkv][4] outlier channel ids */
  uint16_t* k_outlier;       /* fp16 [slot][4] their K values */
  uint16_t* v_outlier;       /* fp16 [slot][4] their V values, or NULL (V not isolated) */
} kvc_cache;

/*
 * kvc_quantize_append -- append n_new[b] tokens to every sequence b ([TKV] 2.2,
 * [DEV] 3.1 and 3.2's online calibration from the appended values).
 *   k_new, v_new  fp16 [B][n_new_max][Hkv][128]; rows >= n_new[b] are ignored.
 *   n_new         device int32 [B], or NULL for n_new_max everywhere.
 *   overflow      device int32 or NULL: set to 1 when some sequence would
 *                 exceed max_tokens; that sequence is left unchanged.
 * Writes every 64-token group the append completes (codes, k_meta, v_meta),
 * the new tail rows, k16/v16/kT rows when those pointers are set, k_absmax,
 * and finally seq_lens[b] += n_new[b].  n_new_max == 1 (a decode step) runs
 * as one launch when max_tokens < 2^24 and num_kv_heads <= 127, else two.
 */
kvc_status kvc_quantize_append(const kvc_cache* cache, const uint16_t* k_new,
                               const uint16_t* v_new, const int32_t* n_new,
                               int32_t n_new_max, int32_t* overflow,
                               hipStream_t stream);

/*
 * kvc_score_topk -- rank tokens and select the Top-K per (sequence, KV head)
 * ([TKV] 2.3, [MTG] 2.2, [SRV] 3).
 *   q           fp16 [B][Hq][128]; query head h belongs to KV head h / (Hq/Hkv).
 *   score_mode  KVC_SCORE_EXACT: all 128 channels; KVC_SCORE_CRITICAL: the
 *               n_crit channels with largest max_h|q_{h,c}| * k_absmax[c]
 *               (ties to the lower channel); KVC_SCORE_EXTERNAL: r_t = ext[t].
 *               Exact/critical score of token t: max over the group's heads of
 *               the fp64 sum, channel by channel in ascending order from +0.0,
 *               of q_{h,c} * k~_{t,c} (k~ = fp16 row, code*s + z, or the fp16
 *               outlier-store value on an outlier channel), plus 0.0.
 *   ext         float32 [B][Hkv][max_tokens] (EXTERNAL only).
 *   candidates  tokens in [n_sink, n - n_window), n = seq_lens[b].
 *   k_per_seq   device int32 [B] or NULL (then k_max);
 *               k_b = min(max(k_per_seq[b], 0), k_max, #candidates).
 *   out_idx     int32 [B][Hkv][k_max]: the k_b best tokens under (score desc,
 *               index asc), in ascending order, then -1.
 *   out_scores  optional fp64 [B][Hkv][max_tokens]: r_t of every candidate.
 *   out_channels optional int32 [B][Hkv][n_crit]: ascending critical channels.
 *   workspace   kvc_workspace_bytes(KVC_OP_SCORE_TOPK, ...) bytes.
 * Hq/Hkv must be 1..16; n_crit 1..128.
 *
 * With KVC_SCORE_BLOCKS in score_mode (block-granular selection, [MTG] 8.1
 * and its part 2 section 1.1: importance averaged over blocks, the top blocks
 * kept for contiguous reads), the items ranked are the complete 64-token
 * blocks j lying wholly inside [n_sink, n - n_window), i.e. j in
 * [ceil(n_sink/64), floor((n - n_window)/64)); block j's score is the mean of
 * its 64 token scores r_t (their fp64 sum in ascending t from +0.0, / 64,
 * + 0.0).  k_per_seq / k_max count blocks; out_idx holds block ids (ascending,
 * -1 padded, ties to the lower block); out_scores, if given, receives the
 * block means at index j of each (sequence, KV head) row (other entries are
 * left as they were).
 */
kvc_status kvc_score_topk(const kvc_cache* cache, const uint16_t* q, int32_t num_q_heads,
                          int32_t score_mode, int32_t n_crit, const float* ext,
                          int32_t n_sink, int32_t n_window, const int32_t* k_per_seq,
                          int32_t k_max, int32_t* out_idx, double* out_scores,
                          int32_t* out_channels, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * kvc_attend_decode -- softmax(q K~^T * sm_scale) V~ for every query head over
 * its attended tokens, dequantizing inside the kernel ([DEV] 3.2, [MTG] 8.1,
 * [TKV] 2.1); query head h reads KV head h / G, G = Hq / Hkv (1..8).  On INT4
 * caches with outlier channels K~ (and V~, with a V store) take the outlier
 * stores' fp16 values on those channels ([MTG] 8.2).
 *   mode  KVC_ATTEND_DENSE: every cached token.
 *         KVC_ATTEND_DROP: sinks [0, n_sink), the valid entries of sel, and
 *           the window [max(n - n_window, n_sink), n); other tokens dropped.
 *         KVC_ATTEND_KEEP (INT4/INT1 with k16/v16): every token; those of the
 *           DROP set read from the fp16 rows, the rest from codes or tail.
 *         KVC_ATTEND_BLOCKS ([MTG] 8.1): sel holds block ids (as written by
 *           kvc_score_topk with KVC_SCORE_BLOCKS, strictly ascending among
 *           the valid ones); the sinks, all 64 tokens of every valid block,
 *           and the window.  Valid blocks are those wholly inside
 *           [n_sink, n - n_window).  INT4/INT1 read only the groups of kept
 *           blocks, sinks and window.  KVC_ERR_UNSUPPORTED when a quantized
 *           cache is too long for the per-wave block list (over 2^23 tokens).
 *   sel   int32 [B][Hkv][k_max], strictly ascending, then -1 padding
 *         (kvc_score_topk's out_idx); entries outside [n_sink, n - n_window)
 *         are ignored.  A row with a repeated or out-of-order entry gives
 *         undefined results (never an access outside the buffers).
 *   out   float32 [B][Hq][128];  lse  float32 [B][Hq] (natural log; -inf and
 *         out = 0 when nothing is attended).
 *   logits optional float32, row (b, h) at logits + (b*Hq + h)*logits_stride:
 *         DENSE/KEEP: position t = token t (t < n); DROP: position j with
 *         j < n_sink -> token j, j - n_sink < k_max -> sel entry, then window
 *         token max(n - n_window, n_sink) + (j - n_sink - k_max); BLOCKS: as
 *         DROP with 64 positions per sel entry (token 64 sel[i] + r at
 *         position n_sink + 64 i + r) and the window after n_sink + 64 k_max;
 *         positions that attend nothing hold -inf.  Values are q.k~ * sm_scale.
 *   workgroups  how many workgroups the attention launch is planned for: the
 *         context of each (sequence, KV head) is split into partials that
 *         many workgroups compute and a log-sum-exp merge combines ([MTG] 8.1
 *         online softmax).  0 = the library's default (one per compute unit
 *         of an MI355X); 1..KVC_MAX_WORKGROUPS otherwise (KVC_ERR_INVALID
 *         outside).  Results agree within rounding for every value; the same
 *         value must be passed to kvc_workspace_bytes.  Nothing else (no
 *         environment variable, no global setting) changes the plan.
 *   workspace  kvc_workspace_bytes(KVC_OP_ATTEND, ...) bytes: split partials
 *         (and, for DROP/KEEP on INT4/INT1, the selection bitmap); contents
 *         on entry are ignored.
 */
kvc_status kvc_attend_decode(const kvc_cache* cache, const uint16_t* q, int32_t num_q_heads,
                             float sm_scale, int32_t mode, const int32_t* sel, int32_t k_max,
                             int32_t n_sink, int32_t n_window, float* out, float* lse,
                             float* logits, int64_t logits_stride, int32_t workgroups,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kvc_attend_decode_noalloc -- kvc_attend_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, arguments and
 * results with workgroups = 0, but no workspace argument.  Its split partials,
 * selection bitmaps and plans live in a static device array of
 * KVC_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends (one copy per device; its address is looked up once
 * per device, on the first call with that device current).  A call that would
 * need more scratch than that returns KVC_ERR_SCRATCH before touching the
 * device.  The call allocates and frees nothing.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and give undefined results; serialize them.  The stream must
 * belong to the current device.
 */
kvc_status kvc_attend_decode_noalloc(const kvc_cache* cache, const uint16_t* q,
                                     int32_t num_q_heads, float sm_scale, int32_t mode,
                                     const int32_t* sel, int32_t k_max, int32_t n_sink,
                                     int32_t n_window, float* out, float* lse, float* logits,
                                     int64_t logits_stride, hipStream_t stream);

/*
 * kvc_accum_scores -- H2O cumulative scores ([SRV] 3.2): for every attended
 * position of a previous kvc_attend_decode with the same mode/sel/n_sink/
 * n_window, acc[b][g][t] += sum over the G query heads of KV head g of
 * exp(logit - lse).  acc is float32 [B][Hkv][max_tokens].
 */
kvc_status kvc_accum_scores(const kvc_cache* cache, int32_t num_q_heads, const float* logits,
                            int64_t logits_stride, const float* lse, int32_t mode,
                            const int32_t* sel, int32_t k_max, int32_t n_sink, int32_t n_window,
                            float* acc, hipStream_t stream);

/*
 * kvc_topk_mass -- top-k attention probability mass of each query head's row
 * ([TKV] 2.1: the dense preference score P = n_q - sum over the last n_q
 * query rows of their top-k softmax entries; a layer with P above tau = 0.2
 * is quantization-friendly, one below it sparsity-friendly).
 *   logits, lse  a dense kvc_attend_decode's outputs for one query: row
 *                (b, h) at logits + (b*Hq + h)*logits_stride, position t =
 *                token t for t < n = seq_lens[b]; logits_stride >= max_tokens.
 *   k            entries per row (k_b = min(k, n)); k >= 0.
 *   out          float32 [B][Hq]: sum over the k_b largest logits of
 *                exp(logit - lse) (fp32 sums; 0 when k_b = 0).  The value does
 *                not depend on which of several equal entries are counted.
 *   workspace    kvc_workspace_bytes(KVC_OP_TOPK_MASS, cache, num_q_heads, ...)
 *                bytes, 16-byte aligned (each row's per-slice histograms and
 *                the keys of its k-th largest key's top-byte bucket); contents
 *                on entry are ignored; KVC_ERR_WORKSPACE when missing or small.
 * Three launches: each row is split into slices spread over the GPU.
 * The caller sums 1 - out over its n_q recent queries to form P.
 */
kvc_status kvc_topk_mass(const kvc_cache* cache, int32_t num_q_heads, const float* logits,
                         int64_t logits_stride, const float* lse, int32_t k, float* out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes for op (KVC_OP_*) called with these arguments (mode, k_max,
 * n_sink, n_window and workgroups are the attend call's; they are ignored for
 * KVC_OP_SCORE_TOPK and KVC_OP_TOPK_MASS); 0 on invalid arguments.  Host only. */
size_t kvc_workspace_bytes(int32_t op, const kvc_cache* cache, int32_t num_q_heads, int32_t mode,
                           int32_t k_max, int32_t n_sink, int32_t n_window, int32_t workgroups);

/*
 * kvc_stream_read -- a measurement aid, not a step of the method: reads
 * `bytes` of device memory at src once, in 4 KB chunks spread over
 * `workgroups` 256-thread workgroups (nontemporal 16-byte loads, two chunks
 * in flight per wave), so that timing it gives the plain streaming-read rate
 * the roofline figures are set against next to the nominal HBM peak.
 *   src        device pointer, 4096-byte aligned; bytes a multiple of 4096.
 *   sink       device uint32 [4 * workgroups]; written only in the case no
 *              real data produces (it keeps the loads from being removed).
 *   workgroups 1..KVC_MAX_WORKGROUPS.
 */
kvc_status kvc_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                           hipStream_t stream);

/* Static description of a status code. */
const char* kvc_status_str(kvc_status status);

/* KVC_ABI_VERSION of the built library. */
int32_t kvc_abi_version(void);

/* Digest of the sources the library was compiled from (16 hex digits of
 * SHA-256 over the HIP sources and headers, set by the build), or "unknown"
 * when the build did not define it.  Static string; lets a loader refuse a
 * library built from other sources. */
const char* kvc_build_digest(void);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H_ */
