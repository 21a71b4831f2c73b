/*
 * kvq.h — C ABI of libkvq: pair-norm-selected mixed-precision key-cache
 * quantization, per-token value quantization and single-token decode
 * attention over the quantized cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources of the method (web pages; cited by title and section):
 *   [PN-Mix]  "PN-Mix: Pair-Norm Guided Mixed-Precision Key Cache Quantization
 *             for Efficient Long-Output LLM Inference" — abstract; podcast
 *             transcript.  Saliency of a RoPE channel pair is the product of
 *             the query pair norm and the key pair norm; the salient pairs are
 *             chosen once at prefill, reused for all of decoding, and stored
 *             at a higher precision than the remaining low-bit key channels.
 *   [PM-KVQ]  pith.science review of "PM-KVQ" — supporting_citations (KIVI):
 *             keys quantized per channel, values per token, with a window of
 *             recent tokens kept at 16 bits; key_machinery: the cache is kept
 *             at 16 bits first and shrunk later.
 *   [MixKVQ]  "MixKVQ: Query-Aware Mixed-Precision KV Cache Quantization for
 *             Long-Context Reasoning" — abstract and AI summary: per-token
 *             low-bit value quantization; channel-level mixed precision.
 *   [SemKV]   "SemKV: Semantic Mixed-Precision KV Cache Quantization ..." —
 *             abstract: an affine (scale + zero point) quantizer.
 *   [Dual-QK] "Dual-QK: Sharp Queries and Flat Keys for Prunable 2-bit KV
 *             Caches" — abstract: decode cost is dominated by key/value
 *             reads, which low-bit storage reduces.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless marked (host).  Every device
 *     pointer must be 16-byte aligned (else KVQ_EALIGN).
 *   - A call validates its arguments on the host first; a validation error
 *     returns before anything is enqueued and leaves every buffer untouched.
 *   - A call enqueues kernels on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and returns without synchronizing, except
 *     kvq_check.  No call allocates or frees memory.  A failed launch returns
 *     KVQ_EHIP.
 *   - All memory is owned by the caller.  The library keeps no state besides
 *     its loaded code objects and the static workspace of
 *     kvq_decode_attn_noalloc; calls on different caches may run concurrently.
 *   - With KVQ_LOG set in the environment (to anything but "0"), every
 *     launch prints its call, shape, split count and kept key runs on stderr
 *     (host side only).
 *   - 16-bit inputs (KVQ_FP16 or KVQ_BF16, `io_dtype`) are contiguous,
 *     row-major, last dimension = channel.  Inputs must be finite with
 *     |x| <= 32752, so that every scale below stays finite; for such inputs
 *     every intermediate of decoding stays finite too.
 *
 * Shapes: B = batch, Hq = query heads, Hkv = KV heads, G = Hq / Hkv (query
 * heads sharing one KV head; 1 <= G <= 16), D = head_dim = 128, 64 RoPE pairs.
 * Pair j owns channels j and j + 64 (rotate-half RoPE pairing).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvq_status;
enum {
  KVQ_OK = 0,
  KVQ_EINVAL = -1,    /* bad size, null pointer or inconsistent layout */
  KVQ_ENOTSUP = -2,   /* a valid but unimplemented layout option */
  KVQ_EALIGN = -3,    /* a device pointer is not 16-byte aligned */
  KVQ_ECAPACITY = -4, /* T exceeds max_tokens, or workspace too small */
  KVQ_EHIP = -5       /* the HIP runtime reported an error */
};
enum { KVQ_FP16 = 0, KVQ_BF16 = 1 };

/* Host struct, read only.  Fixes the shape and the bit allocation. */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim; /* head_dim must be 128 */
  int32_t group;       /* 32: token group of a key channel, channel group of
                          a value token */
  int32_t n_pairs_hi;  /* salient pairs, 0..8 (ranks 0 .. n_pairs_hi-1) */
  int32_t bits_hi;     /* 4 (4-bit codes) or 16 (raw 16-bit values) */
  int32_t n_pairs_lo1; /* pairs of the lowest ranks quantized at 1 bit
                          (codes 0/1 kept in their 2-bit slots of k_lo,
                          one bit each in the dense 1-bit layout: see
                          k_lo); n_pairs_hi + n_pairs_lo1 <= 64 */
  int32_t bits_lo;     /* 2: bits of every non-salient key channel */
  int32_t bits_v;      /* 2: bits of every value */
  int32_t residual;    /* R: recent tokens kept at 16 bits; multiple of 32,
                          32 <= R */
  int32_t max_tokens;  /* capacity per sequence, 1 <= max_tokens <= 2^20 */
  int32_t io_dtype;    /* KVQ_FP16 | KVQ_BF16 */
  int32_t n_vblk_hi;   /* 0..4: a group's 8 n_vblk_hi tokens of largest key
                          magnitude take bits_vhi-bit values ([SemKV]
                          abstract: two precisions chosen per token; see
                          v_hi) */
  int32_t bits_vhi;    /* 3 or 4 when n_vblk_hi > 0 (ignored otherwise) */
  int32_t prog_w8;     /* progressive precision ([PM-KVQ] review, lead and
                          key_machinery: a cache held at 16 bits first and
                          shrunk through 8, 4 and 2 bits as it ages): the
                          newest prog_w8 quantized groups of a sequence are
                          held at 8 bits, the newest prog_w4 at 4 bits or
                          more, older groups at the widths above.
                          0 <= prog_w8 <= prog_w4 <= 256; prog_w4 == 0
                          turns it off.  Requires n_pairs_lo1 == 0 and
                          n_vblk_hi == 0.  See k_pl. */
  int32_t prog_w4;
} kvq_layout;

/* Device buffers of one cache, all caller-allocated with the sizes returned
 * by kvq_cache_sizes, index order as listed there.
 *
 * Let RS = R + 32 (ring slots), NG = max(0, max_tokens - R) / 32 (capacity in
 * quantized groups).  With T tokens held, n_q(T) = 32 * floor(max(0, T-R)/32)
 * tokens are quantized (groups 0 .. n_q/32 - 1, positions [32g, 32g+32)) and
 * the n_r = T - n_q most recent tokens (R <= n_r <= R + 31 once T >= R) sit
 * in the ring at slot = position mod RS.
 *
 * Token order inside a group record ("tile order"): record index
 * e = 16*T + r (T in {0,1}, r in 0..15) holds token 8*(r/4) + 4*T + r%4.
 * Position swap pi(c) = (c & ~3) | ((c & 1) << 1) | ((c >> 1) & 1).
 * A 2-bit code at position p occupies bits [2p, 2p+2) of a little-endian
 * 32-bit word (of a 16-bit half-word for v_codes).
 *
 *  k_lo    [B][Hkv][NG][256] u32: word (w*2 + T)*16 + r holds, for the
 *          token at tile index 16T + r, channels 16w .. 16w+15 (w = 0..7),
 *          channel 16w + c at position pi(c): each 16-channel run of the
 *          group is 128 contiguous bytes.  The stored digit
 *          is the 2-bit code of a 2-bit channel, the code (0 or 1) of a
 *          1-bit channel, the low two bits of the code of a 4-bit channel,
 *          and 0 for a 16-bit channel.
 *          Dense 1-bit layout (n_pairs_hi == 0 and n_pairs_lo1 == 32, the
 *          1.5-bit point): [B][Hkv][NG][768] bytes in plane order.  Let wl
 *          list the 64 channels of the 2-bit pairs ascending and ol those of
 *          the 1-bit pairs (the 32 lowest ranks) ascending; 16-channel run
 *          2kq + u (kq = 0..3) is wl[16kq ..] for u = 0 and ol[16kq ..] for
 *          u = 1.  Bytes [0, 512): u32 words (kq*2 + T)*16 + r, for the token
 *          at tile index 16T + r, channel wl[16kq + c] at position pi(c);
 *          bytes [512, 768): u32 words kq*16 + r, for tile row r of both
 *          halves, channel ol[16kq + c] at bit 16T + 4(c&1) + ((c>>1)&1) +
 *          8((c>>2)&1) + 2(c>>3).
 *          k_meta runs follow plane order (run 2kq + u).
 *  k_hi    bits_hi == 4: [B][Hkv][NG][32] u32: word 16T + r (token at tile
 *          index 16T+r) holds the high two bits (code >> 2) of the d-th
 *          salient channel (ascending channel order, d < 2*n_pairs_hi) at
 *          position pi(d).  bits_hi == 16: [B][Hkv][NG][32][2*n_pairs_hi]
 *          16-bit raw values, tile order, salient channels ascending.
 *          Zero bytes when n_pairs_hi == 0.
 *  k_meta  [B][Hkv][NG][8][2][16] fp16: per 16-channel run w, the scales
 *          s[16w + c] (c = 0..15), then the zeros z[16w + c]; 0 for 16-bit
 *          channels.
 *  v_codes [B][Hkv][NG][256] u32: word (j*4 + kq)*16 + c holds channel
 *          32j + c in bits 0..15 and channel 32j + 16 + c in bits 16..31;
 *          token 8*kq + i of the group at position pi(i) of that half.
 *  v_meta  [B][Hkv][NG][2][4][32] fp16: scale s[j][t] then zero z[j][t] of
 *          channel group j (channels 32j .. 32j+31) of token t.
 *  ring_k  [B][Hkv][RS][128] io dtype, slot-major.
 *  ring_v  [B][Hkv][RS/32][128][32] io dtype: slot block, channel, slot%32.
 *  pairs   [B][Hkv][64] int32: pair id at each saliency rank (rank 0 first).
 *  len     [B][Hkv] int32: tokens held (T).
 *  sums    [B][Hkv][2][64] uint64: fixed-point saliency sums per pair id,
 *          [0] query side, [1] key side (see kvq_select_pairs).
 *  err     [1] int32: sticky error word, 0 = none; bit 0 = an append found
 *          the cache full; bit 1 = an append found a negative len (a cache
 *          no prefill or zero-fill initialized).
 *  k_pl    prog_w4 > 0: [B][Hkv][prog_w4 + 2 prog_w8][256] u32, the digit
 *          planes of the groups held above 2 bits.  A progressive group g
 *          of the ng = n_q(T)/32 quantized groups has age a = ng - 1 - g;
 *          while a < prog_w8 its codes have 8 bits, while a < prog_w4 4
 *          bits, then 2 (salient 4-bit channels stay at 4, 16-bit channels
 *          raw).  Every group is quantized at 8 bits (L = 255) and each
 *          shrink from 2b to b bits maps a code X to round(X / (2^b + 1))
 *          (the equivalent right shift (241 (X + 8)) >> 12 for b = 4,
 *          (13 (X + 2)) >> 6 for b = 2), keeps z and stores the step as
 *          fp16(fp32(s) * (2^b + 1)).  Digit d of a code X is (X >> 2d) & 3:
 *          k_lo holds digit 0 of every group and k_hi digit 1 of the
 *          salient channels of every group; digit 1 of a group younger than
 *          prog_w4 (every channel) is plane slot g mod prog_w4, digits 2
 *          and 3 of a group younger than prog_w8 are slots prog_w4 +
 *          2 (g mod prog_w8) and the slot after, each in the k_lo word
 *          format.  A slot's bytes belong to the youngest group that maps
 *          to it; the others are stale.  The planes are the only storage
 *          above the 2-bit records, so a cache holds (prog_w4 + 2 prog_w8)
 *          KiB of keys and as much of values beyond them per sequence and
 *          KV head, whatever its length.
 *  v_pl    prog_w4 > 0: the value digit planes, as k_pl in the v_codes word
 *          format (value codes shrink with their group the same way; v_meta
 *          holds the current steps).
 *  v_hi    n_vblk_hi > 0: [B][Hkv][NG][8 + 64 n_vblk_hi] u32.  Value
 *          precision by token ([SemKV] abstract: tokens ranked by a
 *          model-internal score get one of two adjacent precisions; the page
 *          names no indicator, so this is a reading).  A group's tokens are
 *          ranked by their key magnitude
 *            E_t = sum over the 128 channels of min(floor(4096 |k_t,c|), 2^20)
 *          (descending, ties to the lower position) and stored in that order:
 *          slot i of every key and value record of the group (the token
 *          index of the k_lo / k_hi / v_codes / v_meta formats) holds the
 *          token at position 32g + order[i]; attention does not depend on
 *          the order.  Slots 0 .. 8 n_vblk_hi - 1 quantize their values at
 *          L = 2^bits_vhi - 1 levels, the others at L = 3; v_codes always
 *          holds the low two bits of a value code.  Words 0..7 of a group
 *          record are the 32 order bytes (byte i = order[i]), and words
 *          8 + (j n_vblk_hi + kq) 16 + c hold, in the v_codes word format,
 *          the high two bits of the codes of slots 8kq .. 8kq+7
 *          (kq < n_vblk_hi) for channel group j.  Ring tokens stay in
 *          position order.  Zero bytes when n_vblk_hi == 0 (order = identity).
 */
typedef struct {
  void *k_lo, *k_hi, *k_meta, *v_codes, *v_meta, *ring_k, *ring_v;
  int32_t *pairs;
  int32_t *len;
  uint64_t *sums;
  int32_t *err;
  uint32_t *v_hi;
  uint32_t *k_pl, *v_pl;
} kvq_cache;

#define KVQ_NBUF 14

/* Bytes of each cache buffer, in kvq_cache field order (host only, no GPU).
 * Returns KVQ_EINVAL / KVQ_ENOTSUP for a layout the library rejects. */
kvq_status kvq_cache_sizes(const kvq_layout *L, size_t sizes[KVQ_NBUF] /*host*/);

/* Workspace bytes kvq_decode_attn needs for `n_splits` token splits per
 * (sequence, KV head), 1 <= n_splits <= 1024: first one 64-bit counter per
 * (sequence, KV head), each on a 256-byte line of its own (at offset 0
 * whatever the split count), then per query head and split one fp32
 * (running max, sum) record, then one fp32 [128] normalized partial output,
 * then a second copy of both record arrays (the first is stored
 * device-coherent, the second stays in the L2 of the storing XCD); each part
 * starts on a 256-byte boundary.  The caller zero-fills a workspace once
 * before its first use; every completed call leaves its counters at zero
 * again and its records right after them, so one workspace may serve calls
 * with different split counts and layouts in turn (each needing no more
 * than its size) as long as no call has more (sequence, KV head) pairs than
 * the call before it on that workspace: more pairs put counters where the
 * earlier call left records, so zero-fill again first.  One workspace
 * serves one call at a time. */
kvq_status kvq_workspace_bytes(const kvq_layout *L, int32_t n_splits,
                               size_t *bytes /*host*/);

/* Pair selection, once per sequence at prefill ([PN-Mix] abstract and
 * transcript: score = query pair norm x key pair norm; chosen once at
 * prefill).  Per (b, kv head) and pair j, with norms in fp32
 * n = sqrt(a*a + b*b) of the pair's two channel values (IEEE, correctly
 * rounded) and u(n) = floor(n * 2^24) as an unsigned 64-bit integer:
 *   sums[0][j] = sum over the G query heads of the KV head and the n_qry
 *                selection queries of u(|q^(j)|),
 *   sums[1][j] = sum over the T prefill keys of u(|k^(j)|),
 *   S_j = (double)sums[0][j] * (double)sums[1][j].
 * S_j is the product of the query-side and key-side norm sums, which ranks
 * pairs exactly like the mean of |q^(j)| |k^(j)| over all query/key
 * combinations.  pairs[] = pair ids by descending S_j, ties to the lower id.
 *   q_sel [B][Hq][n_qry][128] post-RoPE selection queries, 1 <= n_qry <= 1024
 *   k     [B][Hkv][T][128]   post-RoPE prefill keys, 1 <= T <= max_tokens
 * Writes cache->sums and cache->pairs only. */
kvq_status kvq_select_pairs(const kvq_layout *L, const void *q_sel,
                            int32_t n_qry, const void *k, int32_t T,
                            kvq_cache *cache, void *stream);

/* Alternative pair selection by a query-aware channel score ([MixKVQ]
 * abstract and AI summary: a key channel's importance joins its intrinsic
 * quantization difficulty with its relevance to the query; the page gives
 * no formula, so the score below is this library's reading).  Per (b, kv
 * head) and channel c, with fixed-point sums:
 *   A_c = sum over the G query heads and n_qry selection queries of
 *         floor(|q_c| * 2^24)                          (relevance)
 *   R_c = sum over the floor(T / 32) full 32-token groups of the prefill
 *         keys of floor(fp32(max k_c - min k_c) * 2^16) (difficulty: the
 *         range sets the quantization step)
 *   S_j = R_j A_j + R_{j+64} A_{j+64}  (IEEE double, no contraction)
 * pairs[] = pair ids by descending S_j, ties to the lower id;
 * sums[0][j] = the bits of S_j as a double, sums[1][j] = 0.  Arguments and
 * errors as for kvq_select_pairs, which it can replace before the
 * quantization calls. */
kvq_status kvq_select_pairs_qa(const kvq_layout *L, const void *q_sel,
                               int32_t n_qry, const void *k, int32_t T,
                               kvq_cache *cache, void *stream);

/* Key quantization at prefill ([PN-Mix] abstract: salient pairs at higher
 * precision; [PM-KVQ] supporting_citations: keys per channel; [SemKV]
 * abstract: affine quantizer).  Requires cache->pairs from kvq_select_pairs.
 * For each group of 32 tokens and each channel at b bits (L = 2^b - 1),
 * values x_0..x_31 widened exactly to fp32:
 *   z = fp16(min x);  s = fp16(fp32(max x - z) / L)   (IEEE fp32, RNE)
 *   s == 0: every code 0; else r = 1.0f / s and
 *   code_i = clamp(rint((x_i - z) * r), 0, L)  (fp32, ties to even)
 * Channels of the n_pairs_hi top-ranked pairs use bits_hi, those of the
 * n_pairs_lo1 lowest-ranked pairs 1 bit (L = 1), all others bits_lo.
 * Fills groups [0, n_q(T)/32), copies positions [n_q(T), T) into ring_k and
 * sets len[b][h] = T.   k: [B][Hkv][T][128], 1 <= T <= max_tokens.  With
 * n_vblk_hi > 0 it also ranks each group's tokens, stores the keys in that
 * order and writes the order to v_hi (see there). */
kvq_status kvq_quant_keys(const kvq_layout *L, const void *k, int32_t T,
                          kvq_cache *cache, void *stream);

/* Value quantization at prefill ([MixKVQ] abstract, [PM-KVQ]
 * supporting_citations: per-token values).  Same quantizer as the keys over
 * each token's channel groups [32j, 32j+32) at bits_v bits.  Fills groups
 * [0, n_q(T)/32), copies positions [n_q(T), T) into ring_v, sets len = T.
 * With n_vblk_hi > 0 it reads each group's token order from v_hi, which
 * kvq_quant_keys writes: call kvq_quant_keys for the same T first (same
 * stream, or synchronized).  Otherwise the value records are unspecified
 * (every read still stays inside the group's input rows). */
kvq_status kvq_quant_values(const kvq_layout *L, const void *v, int32_t T,
                            kvq_cache *cache, void *stream);

/* One decode-step append ([PM-KVQ] key_machinery and supporting_citations:
 * new tokens are held at 16 bits first and quantized later).  Per (b, kv
 * head): T = len; if T == max_tokens, sets err bit 0 and changes nothing.
 * Otherwise writes k_new/v_new to ring slot T mod RS, sets len = T + 1, and
 * when n_q(T+1) > n_q(T) quantizes the group of positions [n_q(T),
 * n_q(T)+32) from the ring exactly as kvq_quant_keys / kvq_quant_values
 * would, with the prefill pair ranking.  With progressive precision the new
 * group enters at the width of age 0, and the groups that this makes reach
 * age prog_w8 and age prog_w4 are shrunk in place to their new widths first
 * (codes, steps, k_hi and planes), so that the cache always equals a
 * prefill of the same tokens.
 *   k_new, v_new: [B][Hkv][128] io dtype. */
kvq_status kvq_append(const kvq_layout *L, const void *k_new,
                      const void *v_new, kvq_cache *cache, void *stream);

/* In-place precision shrink of the salient key channels ([PM-KVQ]
 * key_machinery: a cache is kept at 2b bits and later shrunk in place to b
 * bits, zero point kept, step multiplied by 2^b + 1).  For every (b, kv head)
 * and quantized group g in [g0, min(g1, n_q(T)/32)), each 4-bit salient code
 * X is moved to the 2-bit grid of step 5 s: q = round(X / 5) (computed as
 * (13 (X + 2)) >> 6), held as the 4-bit code 5 q (high and low digit both q)
 * under the unchanged scale, so it dequantizes to exactly z + 5 s q.  All
 * other channels are untouched; decoding needs no change.  This layout keeps
 * the 4-bit slots, so no bytes are freed.  A group must be shrunk at most once: the
 * caller keeps the boundary (typically the oldest groups, when memory
 * fills).  A progressive layout (prog_w4 > 0) shrinks inside kvq_append and
 * returns KVQ_ENOTSUP here.  n_pairs_hi == 0 is a no-op; bits_hi == 16 returns KVQ_ENOTSUP;
 * g0 < 0 or g1 < g0 returns KVQ_EINVAL; g1 beyond the capacity is clamped. */
kvq_status kvq_shrink(const kvq_layout *L, kvq_cache *cache, int32_t g0,
                      int32_t g1, void *stream);

/* Single-token decode attention over the quantized cache ([Dual-QK]
 * abstract and [PN-Mix] abstract: decode reads the low-bit cache).  For
 * each query head h of KV head h/G:
 *   logit_t = sm_scale * sum_c q[h][c] * k^[t][c],  o = softmax(logit) . v^
 * over all T tokens, where k^, v^ are the dequantized codes z + s*code for
 * quantized tokens and channels and the raw 16-bit values for ring tokens
 * and 16-bit channels.  The token axis is cut into n_splits ranges per
 * (b, kv head) (limits as for kvq_workspace_bytes), each reduced with an
 * online softmax; a log-sum-exp combine merges them inside the same launch.
 * Computation is fp32 with fp16 matrix operands; the result is rounded to
 * the io dtype (nearest even).  Every product of a query channel and a key
 * scale, and of a softmax weight and a value scale, enters as an exact pair
 * of fp16 values (the rounded product and its remainder), so no product is
 * rounded (barring fp16 underflow of a remainder): the roundings left are
 * the softmax weights' (to fp16; numerator and denominator take the same
 * rounded weights) and fp32 accumulation, whatever the size of the logits.
 * With progressive precision each group is dequantized at its current width
 * (digits from k_lo / v_codes, k_hi and the planes, as k_pl describes).
 * Requires T >= 1 (T = 0 writes zeros); a
 * len outside [0, max_tokens] is clamped into it (the result is then
 * unspecified, but every read stays inside the cache).
 *   q   [B][Hq][128] io dtype;  out [B][Hq][128] io dtype
 *   workspace: >= kvq_workspace_bytes(L, n_splits) bytes (else
 *   KVQ_ECAPACITY), zero-filled before its first use. */
kvq_status kvq_decode_attn(const kvq_layout *L, const void *q,
                           const kvq_cache *cache, float sm_scale,
                           int32_t n_splits, void *workspace, size_t ws_bytes,
                           void *out, void *stream);

/* Decode attention with dynamic query-channel pruning ([Dual-QK] abstract:
 * a decode query keeps its few large channels and drops the many small
 * ones, so the key cache is read only for the kept channels; the page gives
 * no rule, so this is a reading).  Per (b, kv head) the n_keep (1..8) of the
 * eight 16-channel key runs (channels 16s .. 16s+15: the contiguous runs of
 * k_lo (64 bytes per 16 tokens), k_meta and ring_k) with the largest
 *   E_s = sum over the group's query heads h and channels c of run s of
 *         min(floor(4096 |q[h][c]|), 2^20)
 * (exact in 32 bits for every 16-bit query) are kept (ties to the lower s),
 * and every logit sums q[h][c] * k^[t][c]
 * over the kept channels only, for quantized and ring tokens alike (the
 * query is zero on the pruned channels).  The pruned runs' key codes and
 * key scale/zero are not read (the group copies wait for the query and the
 * choice); n_keep = 5 drops 37.5 % of the key channels.  n_keep = 8 is
 * kvq_decode_attn; n_keep outside 1..8 returns KVQ_EINVAL.  A progressive
 * layout and the dense 1-bit layout return KVQ_ENOTSUP for n_keep < 8.  All other arguments, limits
 * and errors as for kvq_decode_attn. */
kvq_status kvq_decode_attn_pruned(const kvq_layout *L, const void *q,
                                  const kvq_cache *cache, float sm_scale,
                                  int32_t n_splits, int32_t n_keep,
                                  void *workspace, size_t ws_bytes, void *out,
                                  void *stream);

/* One decode step in one launch: kvq_append of (k_new, v_new), then
 * single-token decode attention of q over the cache including the new token
 * ([PM-KVQ] key_machinery: new tokens are held at 16 bits first and
 * quantized later; [PN-Mix] abstract: decode reads the low-bit cache).
 * Per (b, kv head), with T = len before the call:
 *  - if 0 <= T < max_tokens: the token is appended exactly as kvq_append
 *    does it (ring slot T mod RS, len = T + 1, and the group of positions
 *    [n_q(T), n_q(T) + 32) is packed when n_q(T + 1) > n_q(T)); attention
 *    runs over all T + 1 tokens, with the quantized prefix of before the
 *    append, n_q(T): a group that this call packs is attended at 16 bits in
 *    this call (it is still in the ring) and quantized from the next call on.
 *    Where no group is packed the output equals kvq_append followed by
 *    kvq_decode_attn.  With progressive precision the pack also shrinks the
 *    groups reaching ages prog_w8 and prog_w4 (as kvq_append does); this
 *    call attends them at the widths they had before it, and the shrinks
 *    run after every split of the (b, kv head) has read them.
 *  - if T == max_tokens (T < 0): sets err bit 0 (bit 1), changes nothing,
 *    and decodes over the cache as it stands.
 * Saves the append's launch.  Pruned key chunks are not offered here.
 *   k_new, v_new: [B][Hkv][128] io dtype;  q, out: as for kvq_decode_attn.
 * Other arguments, limits and errors as for kvq_decode_attn. */
kvq_status kvq_append_decode_attn(const kvq_layout *L, const void *k_new,
                                  const void *v_new, const void *q,
                                  kvq_cache *cache, float sm_scale,
                                  int32_t n_splits, void *workspace,
                                  size_t ws_bytes, void *out, void *stream);

/* kvq_decode_attn with no workspace argument and no allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * static device array of KVQ_NOALLOC_WORKSPACE_BYTES inside the library, one
 * per GPU, held until the process ends.  The first call on a GPU resolves its
 * address and enqueues one zero-fill kernel on `stream`; every completed call
 * leaves its split counters at zero again, and a call with more (sequence,
 * KV head) pairs than the one before it on that GPU first enqueues a
 * zero-fill kernel over its extra counters.  All calls on one GPU share that
 * array: calls that overlap on one GPU (different streams, or host threads
 * without ordering) race and give wrong results.  Returns KVQ_ECAPACITY when
 * kvq_workspace_bytes(L, n_splits) exceeds KVQ_NOALLOC_WORKSPACE_BYTES; all
 * other arguments, results and errors as for kvq_decode_attn.  Calls no
 * hipMalloc, hipFree or allocating library routine. */
#define KVQ_NOALLOC_WORKSPACE_BYTES (4u << 20)
kvq_status kvq_decode_attn_noalloc(const kvq_layout *L, const void *q,
                                   const kvq_cache *cache, float sm_scale,
                                   int32_t n_splits, void *out, void *stream);

/* Measurement only: the read ceiling of kvq_decode_attn.  One launch of a
 * kernel with the decode kernel's grid (n_splits workgroups per (b, kv
 * head)), workgroup-to-XCD mapping, wave work split and group copies that
 * reads every cache byte a decode step over the same cache reads, in the
 * same 16-byte-per-lane direct-to-LDS copies, and does no arithmetic on them
 * (decode cost is the read of the cache: [PN-Mix] and [Dual-QK], abstracts).
 * Its time bounds from below what any decode with these loads can reach.
 * Reads cache as kvq_decode_attn does (len, ring, every quantized group of
 * each (b, kv head)); writes nothing but, for almost no data, one word of
 * `sink` (>= 4 bytes of device memory, 16-byte aligned).  n_splits limits
 * and errors as for kvq_decode_attn; a progressive layout returns
 * KVQ_ENOTSUP. */
kvq_status kvq_read_ceiling(const kvq_layout *L, const kvq_cache *cache,
                            int32_t n_splits, void *sink, void *stream);

/* Measurement only: the issue cost of the instruction kinds the decode loop
 * is made of, on this GPU.  One launch of n_blocks workgroups of 256 threads
 * (4 waves; n_blocks = k x the compute-unit count puts k waves on every
 * SIMD), each wave running 256 iterations of one mix:
 *   kind 0: 16 v_add_u32 + 16 v_xor_b32 (integer VALU, as the code masks)
 *   kind 1: 16 v_cvt_scalef32_pk_f16_fp4 + 16 v_xor_b32 (codes to fp16)
 *   kind 2: 16 v_pk_mul_f16 (the exact q*s and p*s pairs)
 *   kind 3: 16 v_exp_f32 + 16 v_mul_f32 (softmax weights)
 *   kind 4: 4 v_mfma_f32_16x16x32_f16 on independent accumulators
 *   kind 5: kinds 4 and 0 in one loop (whether a SIMD overlaps the two)
 *   kind 6: 4 v_mfma_f32_16x16x16_f16 (half the contraction length of kind 4)
 * Every thread writes one 32-bit word of `out` (device memory of at least
 * n_blocks x 1024 bytes, 16-byte aligned); time the launch with events on
 * `stream`.  KVQ_EINVAL for a kind outside 0..6 or n_blocks < 1, KVQ_EALIGN
 * for a misaligned `out`. */
kvq_status kvq_issue_probe(int32_t kind, int32_t n_blocks, void *out, void *stream);

/* Synchronizes `stream`, then copies cache->err to *host_err (tests and
 * debugging only). */
kvq_status kvq_check(const kvq_cache *cache, int32_t *host_err /*host*/,
                     void *stream);

/* Static text for a status code. */
const char *kvq_status_str(kvq_status s);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
