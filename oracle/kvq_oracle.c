/*
 * kvq_oracle.c — CPU oracle of the quantized-KV decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or helper with the GPU library and must never be used as a fallback for it.
 *
 * Plain loops, one step at a time, in the order the method states them:
 *   - pair saliency (PN-Mix, abstract and transcript): per RoPE pair, the
 *     query pair norm times the key pair norm, aggregated over the prefill
 *     queries of the head group and the prefill keys; salient pairs chosen
 *     once at prefill;
 *   - mixed-precision keys (PN-Mix, abstract): salient pairs at a higher bit
 *     width, the rest at 2 bits, per channel over groups of 32 tokens
 *     (PM-KVQ review, supporting_citations: per-channel keys, per-token
 *     values, recent tokens at 16 bits);
 *   - affine quantizer with scale and zero point (SemKV, abstract);
 *   - per-token 2-bit values (MixKVQ, abstract);
 *   - progressive precision (PM-KVQ review, lead and key_machinery): codes
 *     held at 8 bits first and shrunk in place to 4 and 2 bits as their group
 *     ages, by the equivalent right shift (orc_prog_keys / orc_prog_values);
 *   - decode attention: the textbook softmax(scale * q.k) . v over the
 *     dequantized cache, unsplit, in fp64.
 * Floating point follows IEEE binary32 / binary64 exactly (build with
 * -ffp-contract=off, never -ffast-math).  16-bit conversions are written out
 * here from the IEEE formats.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *   saliency sums in fixed point u(n) = floor(n * 2^24) of fp32 norms;
 *   z = fp16(min), s = fp16((max - z) / L), codes rint((x - z) * (1/s));
 *   K groups = 32 tokens of one channel; V groups = 32 channels of one token;
 *   n_q(T) = 32 * floor(max(0, T - R) / 32) quantized tokens, the rest raw;
 *   the rules of orc_select_qa, orc_prune_chunks and orc_token_order, which
 *   the pages describe without a formula;
 *   the age rule of progressive precision and the fp16 step after a shrink.
 *
 * Parity unpinned: orc_select_qa, orc_prune_chunks and orc_token_order have
 * no value the pages fix.  Their tests pin each to its own stated rule
 * (float sums where they separate, invariances, planted cases), not to the
 * pages.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D 128
#define NPAIR 64
#define GS 32

/* ---------------------------------------------------------------- 16-bit */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_half_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double to_f64(uint16_t h, int bf16) {
  return bf16 ? orc_bf16_to_f64(h) : orc_half_to_f64(h);
}

/* binary32 -> binary16, round to nearest, ties to even; overflow -> inf. */
uint16_t orc_f32_to_half(float x) {
  double a = fabs((double)x);
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return sign | 0x7e00;
  if (a >= 65520.0) return sign | 0x7c00; /* rounds past the largest half */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: integer multiple of 2^-24 (rint = ties to even) */
    double m = rint(a * ldexp(1.0, 24));
    return sign | (uint16_t)m; /* m == 1024 is the smallest normal */
  }
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) -> a in [2^(e-1), 2^e) */
  int ue = e - 1; /* a in [2^ue, 2^(ue+1)) */
  double m = rint(ldexp(a, 10 - ue)); /* 11-bit significand in [1024, 2048] */
  if (m == 2048.0) {
    m = 1024.0;
    ue += 1;
  }
  return sign | (uint16_t)(((ue + 15) << 10) | ((int)m - 1024));
}

/* ---------------------------------------------------------- pair saliency */

/* Fixed-point pair norm: fp32 sqrt(a*a + b*b), scaled by 2^24, truncated. */
static uint64_t norm_fixed(double a, double b) {
  float af = (float)a, bf = (float)b;
  float s = af * af + bf * bf;
  float n = sqrtf(s);
  return (uint64_t)floor((double)n * 16777216.0);
}

/* q_sel [B][Hq][n_qry][128], k [B][Hkv][Tstride][128] (first T used).
 * sums [B][Hkv][2][64]: [0] query side, [1] key side.  pairs [B][Hkv][64]. */
int orc_select(int B, int Hq, int Hkv, int bf16, const uint16_t *q_sel,
               int n_qry, const uint16_t *k, int Tstride, int T,
               uint64_t *sums, int32_t *pairs) {
  if (Hq % Hkv) return -1;
  int G = Hq / Hkv;
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++) {
      uint64_t *qs = sums + ((size_t)(b * Hkv + kh) * 2 + 0) * NPAIR;
      uint64_t *ks = sums + ((size_t)(b * Hkv + kh) * 2 + 1) * NPAIR;
      for (int j = 0; j < NPAIR; j++) qs[j] = ks[j] = 0;
      for (int g = 0; g < G; g++) {
        int h = kh * G + g;
        for (int t = 0; t < n_qry; t++) {
          const uint16_t *row = q_sel + (((size_t)b * Hq + h) * n_qry + t) * D;
          for (int j = 0; j < NPAIR; j++)
            qs[j] += norm_fixed(to_f64(row[j], bf16), to_f64(row[j + NPAIR], bf16));
        }
      }
      for (int t = 0; t < T; t++) {
        const uint16_t *row = k + (((size_t)b * Hkv + kh) * Tstride + t) * D;
        for (int j = 0; j < NPAIR; j++)
          ks[j] += norm_fixed(to_f64(row[j], bf16), to_f64(row[j + NPAIR], bf16));
      }
      /* rank: descending score, ties to the lower pair id */
      double S[NPAIR];
      int used[NPAIR];
      for (int j = 0; j < NPAIR; j++) {
        S[j] = (double)qs[j] * (double)ks[j];
        used[j] = 0;
      }
      int32_t *pr = pairs + (size_t)(b * Hkv + kh) * NPAIR;
      for (int r = 0; r < NPAIR; r++) {
        int best = -1;
        for (int j = 0; j < NPAIR; j++)
          if (!used[j] && (best < 0 || S[j] > S[best])) best = j;
        used[best] = 1;
        pr[r] = best;
      }
    }
  return 0;
}

/* Query-aware channel score (MixKVQ, abstract and AI summary: a key
 * channel's importance joins its intrinsic quantization difficulty with its
 * relevance to the query; the page prints no formula, so this is a reading).
 * Per (b, kv head) and channel c:
 *   A_c = sum over the group's query heads and selection queries of
 *         floor(|q_c| * 2^24)                       (relevance)
 *   R_c = sum over the full 32-token groups of the T prefill keys of
 *         floor(fp32(max k_c - min k_c) * 2^16)     (difficulty: the range
 *         sets the quantization step)
 * and per pair j the score S_j = R_j A_j + R_{j+64} A_{j+64} in IEEE double
 * (products and sum each rounded once).  pairs = pair ids by descending S,
 * ties to the lower id; score_bits[j] = the bits of S_j. */
int orc_select_qa(int B, int Hq, int Hkv, int bf16, const uint16_t *q_sel,
                  int n_qry, const uint16_t *k, int T, uint64_t *score_bits,
                  int32_t *pairs) {
  if (Hq % Hkv) return -1;
  int G = Hq / Hkv, ng = T / GS;
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++) {
      uint64_t A[D], R[D];
      for (int c = 0; c < D; c++) {
        A[c] = 0;
        for (int h = kh * G; h < kh * G + G; h++)
          for (int t = 0; t < n_qry; t++) {
            double x = fabs(to_f64(q_sel[(((size_t)b * Hq + h) * n_qry + t) * D + c], bf16));
            A[c] += (uint64_t)floor(x * 16777216.0);
          }
        R[c] = 0;
        for (int g = 0; g < ng; g++) {
          float mn = INFINITY, mx = -INFINITY;
          for (int i = 0; i < GS; i++) {
            float x = (float)to_f64(k[(((size_t)b * Hkv + kh) * T + g * GS + i) * D + c], bf16);
            if (x < mn) mn = x;
            if (x > mx) mx = x;
          }
          float r = mx - mn;
          R[c] += (uint64_t)floor((double)r * 65536.0);
        }
      }
      double S[NPAIR];
      for (int j = 0; j < NPAIR; j++) {
        double p0 = (double)R[j] * (double)A[j];
        double p1 = (double)R[j + NPAIR] * (double)A[j + NPAIR];
        S[j] = p0 + p1;
        memcpy(&score_bits[((size_t)b * Hkv + kh) * NPAIR + j], &S[j], 8);
      }
      for (int j = 0; j < NPAIR; j++) {
        int rank = 0;
        for (int i = 0; i < NPAIR; i++) rank += (S[i] > S[j]) || (S[i] == S[j] && i < j);
        pairs[((size_t)b * Hkv + kh) * NPAIR + rank] = j;
      }
    }
  return 0;
}

/* Dynamic query-channel pruning at decode (Dual-QK, abstract: a decode
 * query keeps its few large channels and drops the many small ones, so the
 * key cache is read only for the kept channels; the page gives no rule, so
 * this is a reading).  The unit is the cache's 16-channel key run
 * (channels 16s .. 16s+15, s = 0..7), the smallest set of key codes that is
 * contiguous in the packed layout (64 bytes per 16 tokens), and the
 * decision is per (b, kv head), since the G query heads share one key cache:
 *   E_s = sum over the group's query heads h and channels c of run s of
 *         min(floor(4096 |q_{h,c}|), 2^20)
 * (the fixed-point magnitude also used to rank tokens; an integer sum, exact
 * for every 16-bit input).  The n_keep runs of largest E_s are kept (ties to
 * the lower s); n_keep = 5 drops 37.5 % of the channels, the step nearest
 * the page's 40 %.
 * keep[(b*Hkv + kh)*8 + s] = 1 for a kept run, else 0. */
int orc_prune_chunks(int B, int Hq, int Hkv, int bf16, const uint16_t *q, int n_keep,
                     uint8_t *keep) {
  if (Hq % Hkv || n_keep < 1 || n_keep > 8) return -1;
  int G = Hq / Hkv;
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++) {
      uint64_t E[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int h = kh * G; h < kh * G + G; h++)
        for (int c = 0; c < D; c++) {
          double u = floor(4096.0 * fabs(to_f64(q[((size_t)b * Hq + h) * D + c], bf16)));
          E[c / 16] += (uint64_t)(u < 1048576.0 ? u : 1048576.0);
        }
      for (int s = 0; s < 8; s++) {
        int rank = 0;
        for (int i = 0; i < 8; i++) rank += (E[i] > E[s]) || (E[i] == E[s] && i < s);
        keep[((size_t)b * Hkv + kh) * 8 + s] = rank < n_keep;
      }
    }
  return 0;
}

/* Bits of channel c given the rank table of its (b, kv head): the pairs of
 * the n_hi highest ranks at bits_hi, those of the n_lo1 lowest ranks at one
 * bit, all others at bits_lo (PN-Mix, abstract: more bits for the salient
 * pairs; the 1-bit share is the reading that gives a 1.5-bit average). */
int orc_channel_bits(const int32_t *pr, int n_hi, int bits_hi, int n_lo1,
                     int bits_lo, int c) {
  int j = c % NPAIR;
  for (int r = 0; r < n_hi; r++)
    if (pr[r] == j) return bits_hi;
  for (int r = NPAIR - n_lo1; r < NPAIR; r++)
    if (pr[r] == j) return 1;
  return bits_lo;
}

/* Channel c belongs to one of the n_hi top-ranked (salient) pairs. */
static int orc_is_salient(const int32_t *pr, int n_hi, int c) {
  for (int r = 0; r < n_hi; r++)
    if (pr[r] == c % NPAIR) return 1;
  return 0;
}

/* ------------------------------------------------------ precision shrink */

/* PM-KVQ review, key_machinery: the cache is kept at 2b bits first and later
 * shrunk in place to b bits, the zero point kept and the step multiplied by
 * 2^b + 1 (the b-bit grid then spans the same range as the 2b-bit one).  The
 * requantized code is the nearest b-bit level to the dequantized value,
 * round(X / (2^b + 1)); 2^b + 1 is odd, so no tie occurs.  Plain integer
 * rounding: floor((2X + d) / 2d) with d = 2^b + 1. */
int orc_shrink_code(int x, int b) {
  long long d = (1LL << b) + 1;
  return (int)((2LL * x + d) / (2 * d));
}

/* The review's integer shift form of the same map (as the review writes it):
 * ((2^2b - 2^b + 1) * (X + 2^(b-1))) >> 3b.  Kept apart from the definition
 * above so that tests can compare the two over every input. */
long long orc_ers(long long x, int b) {
  long long m = (1LL << (2 * b)) - (1LL << b) + 1;
  return (m * (x + (1LL << (b - 1)))) >> (3 * b);
}

/* Shrinks the 4-bit salient key channels of groups [g0, g1) (clamped to the
 * quantized groups [0, ng)) to the 2-bit grid with the same zero point and
 * step 5 s: the new 2-bit code is q = round(X / 5), and the channel keeps its
 * 4-bit slot and its scale s with the code 5 q, which dequantizes to exactly
 * z + (5 s) q.  Logical codes [..][NG][128][32]; s is left as it is. */
int orc_shrink_keys(int B, int Hkv, int n_hi, const int32_t *pairs, int NG, int ng,
                    int g0, int g1, uint8_t *codes, uint16_t *s) {
  (void)s;
  if (g1 > ng) g1 = ng;
  if (g0 < 0) g0 = 0;
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++) {
      const int32_t *pr = pairs + (size_t)(b * Hkv + kh) * NPAIR;
      for (int g = g0; g < g1; g++)
        for (int c = 0; c < D; c++) {
          int sal = 0;
          for (int r = 0; r < n_hi; r++) sal |= pr[r] == c % NPAIR;
          if (!sal) continue;
          size_t slot = ((size_t)(b * Hkv + kh) * NG + g) * D + c;
          for (int i = 0; i < GS; i++)
            codes[slot * GS + i] = (uint8_t)(5 * orc_shrink_code(codes[slot * GS + i], 2));
        }
    }
  return 0;
}

/* ------------------------------------------------------------- quantizer */

/* Affine min/max quantizer of one group of 32 values at L = 2^b - 1 levels.
 * x are exact widenings of 16-bit inputs.  Writes fp16 bits of s and z. */
void orc_quant_group(const float *x, int L, uint16_t *s_bits, uint16_t *z_bits,
                     uint8_t *codes) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < GS; i++) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  uint16_t zb = orc_f32_to_half(mn);
  float z = (float)orc_half_to_f64(zb);
  float diff = mx - z;
  uint16_t sb = 0;
  if (diff > 0.0f) sb = orc_f32_to_half(diff / (float)L);
  *z_bits = zb;
  *s_bits = sb;
  if (sb == 0) {
    for (int i = 0; i < GS; i++) codes[i] = 0;
    return;
  }
  float s = (float)orc_half_to_f64(sb);
  float r = 1.0f / s;
  for (int i = 0; i < GS; i++) {
    float t = (x[i] - z) * r;
    float q = rintf(t);
    if (q < 0.0f) q = 0.0f;
    if (q > (float)L) q = (float)L;
    codes[i] = (uint8_t)q;
  }
}

/* Quantized tokens for T held tokens and residual R. */
int orc_n_quant(int T, int R) {
  int over = T - R;
  return over > 0 ? (over / GS) * GS : 0;
}

/* Keys.  k [B][Hkv][Tstride][128].  Outputs (logical, for NG group slots):
 * codes [B][Hkv][NG][128][32] (channel, token), s/z [B][Hkv][NG][128] fp16
 * bits.  16-bit channels get s = z = 0 and codes 0.  Fills groups
 * [0, n_q(T)/32). */
int orc_quant_keys(int B, int Hkv, int bf16, const uint16_t *k, int Tstride,
                   int T, int R, int n_hi, int bits_hi, int n_lo1, const int32_t *pairs,
                   int NG, uint8_t *codes, uint16_t *s, uint16_t *z) {
  int ng = orc_n_quant(T, R) / GS;
  if (ng > NG) return -1;
  float x[GS];
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++) {
      const int32_t *pr = pairs + (size_t)(b * Hkv + kh) * NPAIR;
      for (int g = 0; g < ng; g++)
        for (int c = 0; c < D; c++) {
          size_t slot = ((size_t)(b * Hkv + kh) * NG + g) * D + c;
          int bits = orc_channel_bits(pr, n_hi, bits_hi, n_lo1, 2, c);
          if (bits == 16) {
            memset(codes + slot * GS, 0, GS);
            s[slot] = z[slot] = 0;
            continue;
          }
          for (int i = 0; i < GS; i++)
            x[i] = (float)to_f64(k[(((size_t)b * Hkv + kh) * Tstride + g * GS + i) * D + c], bf16);
          orc_quant_group(x, (1 << bits) - 1, s + slot, z + slot, codes + slot * GS);
        }
    }
  return 0;
}

/* Values.  v [B][Hkv][Tstride][128].  codes [B][Hkv][NG][32][128] (token,
 * channel), s/z [B][Hkv][NG][32][4] fp16 bits (token, channel group). */
/* Two value precisions by token (SemKV, abstract: tokens are ranked by a
 * model-internal score and given one of two adjacent precisions; the page
 * names no indicator and finds the indicators interchangeable above the
 * quality cliff, so this is a reading).  The indicator is the token's key
 * magnitude,
 *   E_t = sum over the 128 channels of min(floor(4096 |k_t,c|), 2^20)
 * (integer, so order-free).  Within each 32-token group the tokens are
 * stored in descending E order (ties to the lower position): order[slot] =
 * position; attention does not depend on the order.  The 8 n_vblk_hi
 * tokens in the first slots quantize their values at bits_vhi bits, the
 * others at bits_v bits.  With n_vblk_hi == 0 the order is the identity. */
int orc_token_order(int B, int Hkv, int bf16, const uint16_t *k, int Tstride, int T, int R,
                    int NG, int n_vblk_hi, uint8_t *order) {
  int ng = orc_n_quant(T, R) / GS;
  if (ng > NG) return -1;
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++)
      for (int g = 0; g < ng; g++) {
        uint8_t *ord = order + ((size_t)(b * Hkv + kh) * NG + g) * GS;
        uint64_t E[GS];
        for (int t = 0; t < GS; t++) {
          const uint16_t *row = k + (((size_t)b * Hkv + kh) * Tstride + g * GS + t) * D;
          E[t] = 0;
          for (int c = 0; c < D; c++) {
            double u = floor(4096.0 * fabs(to_f64(row[c], bf16)));
            E[t] += (uint64_t)(u < 1048576.0 ? u : 1048576.0);
          }
        }
        for (int t = 0; t < GS; t++) {
          int rank = 0;
          if (n_vblk_hi > 0)
            for (int i = 0; i < GS; i++) rank += (E[i] > E[t]) || (E[i] == E[t] && i < t);
          else
            rank = t;
          ord[rank] = (uint8_t)t;
        }
      }
  return 0;
}

int orc_quant_values(int B, int Hkv, int bf16, const uint16_t *v, int Tstride,
                     int T, int R, int bits_v, int NG, int n_vblk_hi, int bits_vhi,
                     const uint8_t *order, uint8_t *codes, uint16_t *s, uint16_t *z) {
  int ng = orc_n_quant(T, R) / GS;
  if (ng > NG || n_vblk_hi < 0 || n_vblk_hi > 4) return -1;
  float x[GS];
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++)
      for (int g = 0; g < ng; g++) {
        const uint8_t *ord = order + ((size_t)(b * Hkv + kh) * NG + g) * GS;
        for (int slot = 0; slot < GS; slot++) {
          int t = ord[slot];
          int bits = slot < 8 * n_vblk_hi ? bits_vhi : bits_v;
          size_t tok = ((size_t)(b * Hkv + kh) * NG + g) * GS + t;
          const uint16_t *row = v + (((size_t)b * Hkv + kh) * Tstride + g * GS + t) * D;
          for (int j = 0; j < D / GS; j++) {
            for (int i = 0; i < GS; i++) x[i] = (float)to_f64(row[j * GS + i], bf16);
            orc_quant_group(x, (1 << bits) - 1, s + tok * 4 + j, z + tok * 4 + j,
                            codes + tok * D + j * GS);
          }
        }
      }
  return 0;
}

/* ------------------------------------------------------------- attention */

/* Decode attention, unsplit, fp64.  q [B][Hq][128] bits; k, v raw inputs
 * [B][Hkv][Tstride][128] (used for ring tokens and 16-bit channels); the
 * logical codes / metadata from orc_quant_keys / orc_quant_values.
 * out [B][Hq][128] fp64.  Optional lse [B][Hq] (natural log of the softmax
 * denominator of the scaled logits, for split checks). */
int orc_attention(int B, int Hq, int Hkv, int bf16, const uint16_t *q,
                  const uint16_t *k, const uint16_t *v, int Tstride, int T,
                  int R, int n_hi, int bits_hi, int n_lo1, const int32_t *pairs, int NG,
                  const uint8_t *kcodes, const uint16_t *ks, const uint16_t *kz,
                  const uint8_t *vcodes, const uint16_t *vs, const uint16_t *vz,
                  double sm_scale, double *out, double *lse) {
  if (Hq % Hkv) return -1;
  int G = Hq / Hkv;
  int nq = orc_n_quant(T, R);
  double *logit = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double *kh_row = (double *)malloc(sizeof(double) * D);
  if (!logit || !kh_row) return -2;
  for (int b = 0; b < B; b++)
    for (int h = 0; h < Hq; h++) {
      int kh = h / G;
      const int32_t *pr = pairs + (size_t)(b * Hkv + kh) * NPAIR;
      double qv[D];
      for (int c = 0; c < D; c++) qv[c] = to_f64(q[((size_t)b * Hq + h) * D + c], bf16);
      /* logits */
      double m = -INFINITY;
      for (int t = 0; t < T; t++) {
        const uint16_t *raw = k + (((size_t)b * Hkv + kh) * Tstride + t) * D;
        for (int c = 0; c < D; c++) {
          int bits = orc_channel_bits(pr, n_hi, bits_hi, n_lo1, 2, c);
          if (t >= nq || bits == 16) {
            kh_row[c] = to_f64(raw[c], bf16);
          } else {
            size_t slot = ((size_t)(b * Hkv + kh) * NG + t / GS) * D + c;
            kh_row[c] = orc_half_to_f64(kz[slot]) +
                        orc_half_to_f64(ks[slot]) * (double)kcodes[slot * GS + t % GS];
          }
        }
        double acc = 0.0;
        for (int c = 0; c < D; c++) acc += qv[c] * kh_row[c];
        logit[t] = sm_scale * acc;
        if (logit[t] > m) m = logit[t];
      }
      /* softmax-weighted values */
      double l = 0.0, o[D];
      for (int c = 0; c < D; c++) o[c] = 0.0;
      for (int t = 0; t < T; t++) {
        double p = exp(logit[t] - m);
        l += p;
        const uint16_t *raw = v + (((size_t)b * Hkv + kh) * Tstride + t) * D;
        for (int c = 0; c < D; c++) {
          double vv;
          if (t >= nq) {
            vv = to_f64(raw[c], bf16);
          } else {
            size_t tok = ((size_t)(b * Hkv + kh) * NG + t / GS) * GS + t % GS;
            vv = orc_half_to_f64(vz[tok * 4 + c / GS]) +
                 orc_half_to_f64(vs[tok * 4 + c / GS]) * (double)vcodes[tok * D + c];
          }
          o[c] += p * vv;
        }
      }
      for (int c = 0; c < D; c++) out[((size_t)b * Hq + h) * D + c] = o[c] / l;
      if (lse) lse[(size_t)b * Hq + h] = m + log(l);
    }
  free(logit);
  free(kh_row);
  return 0;
}

/* ------------------------------------------------------------ byte layout */

/* Token of record index e = 16*T + r inside a group ("tile order"). */
static int tile_token(int e) {
  int T = e / 16, r = e % 16;
  return 8 * (r / 4) + 4 * T + r % 4;
}

/* Position of element c inside its 4-aligned block: bits 0 and 1 swapped. */
static int pos_swap(int c) { return (c & ~3) | ((c & 1) << 1) | ((c >> 1) & 1); }

/* The dense 1-bit layout (PN-Mix, abstract: the cache degrades gracefully
 * down to 1.5 bits; reading: with exactly half of the pairs at one bit and
 * no salient pairs, the 1-bit codes take one bit each).  Channels go in
 * "plane order": wl lists the 2-bit channels ascending, ol the 1-bit ones;
 * chunk kq (0..3) is the 2-bit run wl[16 kq ..] (u = 0) then the 1-bit run
 * ol[16 kq ..] (u = 1).  k_lo [..][NG][192] u32: words (kq*2 + T)*16 + r
 * hold the 2-bit run kq of the token at tile index 16T + r, channel
 * wl[16 kq + c] at position pos_swap(c); then (byte 512 on) u32 words
 * kq*16 + r hold the 1-bit run kq of tile row r for both tile halves,
 * channel ol[16 kq + c] at bit onebit_pos(c) + 16 T.  k_meta follows plane
 * order: run 2 kq + u. */
int orc_dense1(int n_hi, int n_lo1) { return n_hi == 0 && n_lo1 == NPAIR / 2; }

/* Bit of the code of run channel c in a 1-bit half-word, chosen so that the
 * four nibble masks (h >> i) & 0x1111 deliver the channels in order. */
static int onebit_pos(int c) {
  return 4 * (c & 1) + ((c >> 1) & 1) + 8 * ((c >> 2) & 1) + 2 * (c >> 3);
}

/* Plane lists of one (b, kv head): wl = 2-bit channels, ol = 1-bit ones,
 * each ascending (the pairs' first channels, then their second ones). */
static void orc_plane_lists(const int32_t *pr, int n_lo1, int *wl, int *ol) {
  int one[NPAIR] = {0}, nw = 0, no = 0;
  for (int r = NPAIR - n_lo1; r < NPAIR; r++) one[pr[r] & (NPAIR - 1)] = 1;
  for (int c = 0; c < D; c++) {
    if (one[c % NPAIR]) ol[no++] = c;
    else wl[nw++] = c;
  }
}

/* Packs the logical key codes of groups [0, ng) into the byte records.
 * k_lo [..][NG][256] u32 ([..][NG][192] in the dense 1-bit layout), k_hi
 * (4-bit: [..][NG][32] u32; 16-bit: [..][NG][32][2*n_hi] u16 raw), k_meta
 * [..][NG][8][2][16] u16. */
/* Key records in the group's token order: tile index e holds the token at
 * slot tile_token(e), i.e. position order[tile_token(e)]. */
int orc_pack_keys(int B, int Hkv, const uint16_t *k, int Tstride, int T, int R,
                  int n_hi, int bits_hi, int n_lo1, const int32_t *pairs, int NG,
                  const uint8_t *order, const uint8_t *codes, const uint16_t *s,
                  const uint16_t *z, uint32_t *k_lo, void *k_hi, uint16_t *k_meta) {
  int ng = orc_n_quant(T, R) / GS;
  const int dense = orc_dense1(n_hi, n_lo1);
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++) {
      const int32_t *pr = pairs + (size_t)(b * Hkv + kh) * NPAIR;
      int hil[16], nh = 0; /* salient channels, ascending */
      for (int c = 0; c < D; c++)
        if (orc_is_salient(pr, n_hi, c)) hil[nh++] = c;
      int wl[D], ol[D];
      if (dense) orc_plane_lists(pr, n_lo1, wl, ol);
      for (int g = 0; g < ng; g++) {
        size_t grp = (size_t)(b * Hkv + kh) * NG + g;
        const uint8_t *cg = codes + grp * D * GS;
        const uint8_t *ord = order + grp * GS;
        if (dense) {
          uint32_t *lo = k_lo + grp * 192;
          uint32_t *lo1 = lo + 128;
          memset(lo, 0, 192 * 4);
          for (int e = 0; e < 32; e++) {
            int t = ord[tile_token(e)], Tt = e / 16, r = e % 16;
            for (int kq = 0; kq < 4; kq++)
              for (int c = 0; c < 16; c++) {
                int w_idx = (kq * 2 + Tt) * 16 + r;
                lo[w_idx] |= (uint32_t)(cg[wl[16 * kq + c] * GS + t] & 3) << (2 * pos_swap(c));
                lo1[kq * 16 + r] |= (uint32_t)(cg[ol[16 * kq + c] * GS + t] & 1)
                                    << (onebit_pos(c) + 16 * Tt);
              }
          }
          uint16_t *meta = k_meta + grp * 256;
          for (int kq = 0; kq < 4; kq++)
            for (int c = 0; c < 16; c++) {
              meta[(2 * kq) * 32 + c] = s[grp * D + wl[16 * kq + c]];
              meta[(2 * kq) * 32 + 16 + c] = z[grp * D + wl[16 * kq + c]];
              meta[(2 * kq + 1) * 32 + c] = s[grp * D + ol[16 * kq + c]];
              meta[(2 * kq + 1) * 32 + 16 + c] = z[grp * D + ol[16 * kq + c]];
            }
          continue;
        }
        uint32_t *lo = k_lo + grp * 256;
        memset(lo, 0, 256 * 4);
        for (int e = 0; e < 32; e++) {
          int t = ord[tile_token(e)], Tt = e / 16, r = e % 16;
          for (int c = 0; c < D; c++) {
            int w = c / 16, kq = w / 2, u = w % 2;
            int bits = orc_channel_bits(pr, n_hi, bits_hi, n_lo1, 2, c);
            uint32_t digit = bits == 16 ? 0u : (uint32_t)(cg[c * GS + t] & 3);
            size_t word = ((size_t)(kq * 2 + u) * 2 + Tt) * 16 + r;
            lo[word] |= digit << (2 * pos_swap(c % 16));
          }
        }
        if (nh && bits_hi == 4) {
          uint32_t *hi = (uint32_t *)k_hi + grp * 32;
          memset(hi, 0, 32 * 4);
          for (int e = 0; e < 32; e++) {
            int t = ord[tile_token(e)];
            for (int d = 0; d < nh; d++)
              hi[e] |= (uint32_t)((cg[hil[d] * GS + t] >> 2) & 3) << (2 * pos_swap(d));
          }
        } else if (nh && bits_hi == 16) {
          uint16_t *hi = (uint16_t *)k_hi + grp * 32 * nh;
          for (int e = 0; e < 32; e++) {
            int t = ord[tile_token(e)];
            for (int d = 0; d < nh; d++)
              hi[e * nh + d] = k[(((size_t)b * Hkv + kh) * Tstride + g * GS + t) * D + hil[d]];
          }
        }
        uint16_t *meta = k_meta + grp * 256;
        for (int c = 0; c < D; c++) {
          meta[(c / 16) * 32 + c % 16] = s[grp * D + c];
          meta[(c / 16) * 32 + 16 + c % 16] = z[grp * D + c];
        }
      }
    }
  return 0;
}

/* Packs the logical value codes: v_codes [..][NG][256] u32,
 * v_meta [..][NG][2][4][32] u16. */
/* Value records in the group's token order: slot 8 kq + i of the v_codes
 * word format holds position order[8 kq + i].  v_codes holds the low two
 * bits of every value code.  With n_vblk_hi > 0, v_hi holds per group
 * 8 + 64 n_vblk_hi words: the 32 order bytes (slot -> position), then for
 * slot block kq < n_vblk_hi and channel group j the words
 * 8 + (j n_vblk_hi + kq) 16 + c, in the v_codes word format, of the codes'
 * high two bits (NULL when n_vblk_hi == 0). */
int orc_pack_values(int B, int Hkv, int T, int R, int NG, const uint8_t *codes,
                    const uint16_t *s, const uint16_t *z, int n_vblk_hi,
                    const uint8_t *order, uint32_t *v_codes, uint16_t *v_meta,
                    uint32_t *v_hi) {
  int ng = orc_n_quant(T, R) / GS;
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++)
      for (int g = 0; g < ng; g++) {
        size_t grp = (size_t)(b * Hkv + kh) * NG + g;
        const uint8_t *cg = codes + grp * GS * D; /* [token][channel] */
        const uint8_t *ord = order + grp * GS;
        uint32_t *vc = v_codes + grp * 256;
        memset(vc, 0, 256 * 4);
        for (int j = 0; j < 4; j++)
          for (int kq = 0; kq < 4; kq++)
            for (int c = 0; c < 16; c++) {
              uint32_t w = 0;
              for (int i = 0; i < 8; i++) {
                int t = ord[8 * kq + i];
                w |= (uint32_t)(cg[t * D + 32 * j + c] & 3) << (2 * pos_swap(i));
                w |= (uint32_t)(cg[t * D + 32 * j + 16 + c] & 3) << (16 + 2 * pos_swap(i));
              }
              vc[(j * 4 + kq) * 16 + c] = w;
            }
        if (n_vblk_hi > 0) {
          size_t rw = 8 + 64 * (size_t)n_vblk_hi;
          uint32_t *vh = v_hi + grp * rw;
          memset(vh, 0, rw * 4);
          memcpy(vh, ord, GS);
          for (int kq = 0; kq < n_vblk_hi; kq++)
            for (int j = 0; j < 4; j++)
              for (int c = 0; c < 16; c++) {
                uint32_t w = 0;
                for (int i = 0; i < 8; i++) {
                  int t = ord[8 * kq + i];
                  w |= (uint32_t)(cg[t * D + 32 * j + c] >> 2) << (2 * pos_swap(i));
                  w |= (uint32_t)(cg[t * D + 32 * j + 16 + c] >> 2) << (16 + 2 * pos_swap(i));
                }
                vh[8 + (j * n_vblk_hi + kq) * 16 + c] = w;
              }
        }
        uint16_t *meta = v_meta + grp * 256;
        for (int j = 0; j < 4; j++)
          for (int sl = 0; sl < GS; sl++) {
            meta[j * 32 + sl] = s[(grp * GS + ord[sl]) * 4 + j];
            meta[128 + j * 32 + sl] = z[(grp * GS + ord[sl]) * 4 + j];
          }
      }
  return 0;
}

/* ------------------------------------------------- progressive precision */

/* PM-KVQ review (lead, key_machinery, referee report summary): the cache is
 * held at 16 bits first and then at ever fewer bits as it ages, 8, 4, 2, each
 * step shrinking a 2b-bit code to b bits in place (orc_shrink_code: zero point
 * kept, step times 2^b + 1).  Readings:
 *   - a quantized group's width follows its age a = ng - 1 - g among the ng
 *     quantized groups of its (sequence, KV head): 8 bits while a < W8, 4 bits
 *     while a < W4, then the layout's final width (2 bits; salient 4-bit
 *     channels stop at 4; 16-bit channels stay raw);
 *   - every group is quantized at 8 bits first (the 16 -> 8 step is the
 *     quantizer itself, L = 255), then shrunk through the chain;
 *   - the step after a shrink is stored as fp16(s (2^b + 1)), the product
 *     exact in fp32 and rounded once to nearest even. */
int orc_prog_width(int age, int W8, int W4) { return age < W8 ? 8 : (age < W4 ? 4 : 2); }

/* One shrink of n codes sharing the scale *s, from 2b to b bits. */
static void orc_prog_step(uint8_t *codes, int n, uint16_t *s, int b) {
  for (int i = 0; i < n; i++) codes[i] = (uint8_t)orc_shrink_code(codes[i], b);
  *s = orc_f32_to_half((float)orc_half_to_f64(*s) * (float)((1 << b) + 1));
}

/* Keys of a progressive cache: as orc_quant_keys (no 1-bit pairs), but every
 * quantized channel at 8 bits first, then shrunk by the group's age. */
int orc_prog_keys(int B, int Hkv, int bf16, const uint16_t *k, int Tstride, int T, int R,
                  int n_hi, int bits_hi, const int32_t *pairs, int NG, int W8, int W4,
                  uint8_t *codes, uint16_t *s, uint16_t *z) {
  int ng = orc_n_quant(T, R) / GS;
  if (ng > NG || W8 < 0 || W4 < W8) return -1;
  float x[GS];
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++) {
      const int32_t *pr = pairs + (size_t)(b * Hkv + kh) * NPAIR;
      for (int g = 0; g < ng; g++) {
        int w = orc_prog_width(ng - 1 - g, W8, W4);
        for (int c = 0; c < D; c++) {
          size_t slot = ((size_t)(b * Hkv + kh) * NG + g) * D + c;
          int bits = orc_channel_bits(pr, n_hi, bits_hi, 0, 2, c);
          if (bits == 16) {
            memset(codes + slot * GS, 0, GS);
            s[slot] = z[slot] = 0;
            continue;
          }
          for (int i = 0; i < GS; i++)
            x[i] = (float)to_f64(k[(((size_t)b * Hkv + kh) * Tstride + g * GS + i) * D + c], bf16);
          orc_quant_group(x, 255, s + slot, z + slot, codes + slot * GS);
          if (w <= 4) orc_prog_step(codes + slot * GS, GS, s + slot, 4);
          if (w == 2 && bits == 2) orc_prog_step(codes + slot * GS, GS, s + slot, 2);
        }
      }
    }
  return 0;
}

/* Values of a progressive cache: each token's 32-channel groups at 8 bits
 * first, then shrunk by the group's age down to 2 bits. */
int orc_prog_values(int B, int Hkv, int bf16, const uint16_t *v, int Tstride, int T, int R,
                    int NG, int W8, int W4, uint8_t *codes, uint16_t *s, uint16_t *z) {
  int ng = orc_n_quant(T, R) / GS;
  if (ng > NG || W8 < 0 || W4 < W8) return -1;
  float x[GS];
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++)
      for (int g = 0; g < ng; g++) {
        int w = orc_prog_width(ng - 1 - g, W8, W4);
        for (int t = 0; t < GS; t++) {
          size_t tok = ((size_t)(b * Hkv + kh) * NG + g) * GS + t;
          const uint16_t *row = v + (((size_t)b * Hkv + kh) * Tstride + g * GS + t) * D;
          for (int j = 0; j < D / GS; j++) {
            uint8_t *cj = codes + tok * D + j * GS;
            for (int i = 0; i < GS; i++) x[i] = (float)to_f64(row[j * GS + i], bf16);
            orc_quant_group(x, 255, s + tok * 4 + j, z + tok * 4 + j, cj);
            if (w <= 4) orc_prog_step(cj, GS, s + tok * 4 + j, 4);
            if (w == 2) orc_prog_step(cj, GS, s + tok * 4 + j, 2);
          }
        }
      }
  return 0;
}

/* Digit planes of the groups held above 2 bits.  Digit d of a code X is
 * (X >> 2d) & 3; k_lo / v_codes hold digit 0 of every group.  k_pl
 * [B][Hkv][W4 + 2 W8][256] u32: digit 1 of group g (age < W4) at plane slot
 * g mod W4, digits 2 and 3 of group g (age < W8) at slots W4 + 2 (g mod W8)
 * and the one after, each in the k_lo word format; v_pl the same in the
 * v_codes word format.  Slots of no live wide group are left as they are. */
int orc_pack_planes(int B, int Hkv, int T, int R, int NG, int W8, int W4,
                    const uint8_t *kcodes, const uint8_t *vcodes, uint32_t *k_pl,
                    uint32_t *v_pl) {
  int ng = orc_n_quant(T, R) / GS;
  size_t nslot = (size_t)W4 + 2 * (size_t)W8;
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++)
      for (int g = 0; g < ng; g++) {
        int age = ng - 1 - g;
        if (age >= W4) continue;
        size_t grp = (size_t)(b * Hkv + kh) * NG + g;
        const uint8_t *kc = kcodes + grp * D * GS; /* [channel][token] */
        const uint8_t *vc = vcodes + grp * GS * D; /* [token][channel] */
        for (int d = 1; d <= (age < W8 ? 3 : 1); d++) {
          size_t ps = d == 1 ? (size_t)(g % W4) : (size_t)W4 + 2 * (size_t)(g % W8) + (d - 2);
          uint32_t *kp = k_pl + ((size_t)(b * Hkv + kh) * nslot + ps) * 256;
          uint32_t *vp = v_pl + ((size_t)(b * Hkv + kh) * nslot + ps) * 256;
          memset(kp, 0, 256 * 4);
          memset(vp, 0, 256 * 4);
          for (int e = 0; e < 32; e++) {
            int t = tile_token(e), Tt = e / 16, r = e % 16;
            for (int c = 0; c < D; c++) {
              uint32_t digit = (uint32_t)(kc[c * GS + t] >> (2 * d)) & 3u;
              kp[((size_t)(c / 16) * 2 + Tt) * 16 + r] |= digit << (2 * pos_swap(c % 16));
            }
          }
          for (int j = 0; j < 4; j++)
            for (int kq = 0; kq < 4; kq++)
              for (int c = 0; c < 16; c++) {
                uint32_t w = 0;
                for (int i = 0; i < 8; i++) {
                  int t = 8 * kq + i;
                  w |= ((uint32_t)(vc[t * D + 32 * j + c] >> (2 * d)) & 3u) << (2 * pos_swap(i));
                  w |= ((uint32_t)(vc[t * D + 32 * j + 16 + c] >> (2 * d)) & 3u)
                       << (16 + 2 * pos_swap(i));
                }
                vp[(j * 4 + kq) * 16 + c] = w;
              }
        }
      }
  return 0;
}

/* Ring contents for positions [n_q(T), T): ring_k [..][RS][128],
 * ring_v [..][RS/32][128][32]; other slots are left as they are. */
int orc_ring(int B, int Hkv, const uint16_t *k, const uint16_t *v, int Tstride,
             int T, int R, uint16_t *ring_k, uint16_t *ring_v) {
  int RS = R + GS;
  for (int b = 0; b < B; b++)
    for (int kh = 0; kh < Hkv; kh++)
      for (int p = orc_n_quant(T, R); p < T; p++) {
        int slot = p % RS;
        const size_t src = (((size_t)b * Hkv + kh) * Tstride + p) * D;
        uint16_t *rk = ring_k + ((size_t)(b * Hkv + kh) * RS + slot) * D;
        uint16_t *rv = ring_v + (size_t)(b * Hkv + kh) * RS * D;
        for (int c = 0; c < D; c++) {
          rk[c] = k[src + c];
          rv[((size_t)(slot / GS) * D + c) * GS + slot % GS] = v[src + c];
        }
      }
  return 0;
}
