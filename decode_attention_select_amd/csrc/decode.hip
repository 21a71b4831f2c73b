// decode.hip — single-token decode attention over the quantized cache.
//
// Decode cost is the read of the cache (Dual-QK, abstract: low-bit storage
// cuts key/value read volume; PN-Mix, abstract: the KV cache is a bandwidth
// bottleneck), so the kernel streams packed 2-bit codes and fp16 scale/zero
// once and dequantizes in registers.
//
// Algebra.  A key channel c of a quantized group dequantizes to
// z_c + s_c * code, so for query head h
//   q . k^_t = sum_c q_c z_c  +  sum_c (q_c s_c) code_{c,t},
// and for values (scale/zero per token t and 32-channel group j)
//   sum_t p_t v^_{t,c} = sum_t p_t z_{t,j}  +  sum_t (p_t s_{t,j}) code_{t,c}.
// Both right-hand sums are dense contractions with small integer operands,
// done on the matrix cores (v_mfma_f32_16x16x32_f16): codes become exact fp16
// integers with one scaled fp4 convert per two codes (a 2-bit code in a
// nibble is the e2m1 value code/2), the pre-scaled operands (q*s, p*s) are
// fp16, accumulation is fp32.  The z terms are one more MFMA each; an extra
// all-ones row in the value-zero MFMA yields the softmax denominator from the
// same rounded p.  Query heads of one KV head fill the 16 MFMA columns
// (G <= 16).  Ring (16-bit) tokens use the same MFMA shapes on raw values.
//
// Work split: one wave64 per (sequence, KV head, token split); each split
// runs an online softmax (base 2, scale folded into the exponent) over its
// 32-token blocks and writes (m, l, o[128]) per head; a second kernel merges
// the splits with the log-sum-exp rule.
#include "common.h"
#include "internal.h"

namespace kvq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int PART = 4 + D;  // floats per (head, split) partial: m, l, 2 pad, o[128]

__device__ inline uint32_t h2u(h2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ inline h2 u2h(uint32_t x) { return __builtin_bit_cast(h2, x); }
__device__ inline uint32_t pk_mul(uint32_t a, uint32_t b) { return h2u(u2h(a) * u2h(b)); }
// fp32 pair -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32)
__device__ inline uint32_t pk_rne(float a, float b) { return h2u(h2{(_Float16)a, (_Float16)b}); }

// Two codes of nibble pair `byte` of w (each nibble 0..3, value = code / 2 in
// e2m1) -> two exact fp16 integers.
template <int BYTE>
__device__ inline uint32_t cvt2(uint32_t w) {
  return h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, BYTE));
}

__device__ inline f4 mma_f16(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a),
                                                __builtin_bit_cast(h8, b), c, 0, 0, 0);
}
template <bool BF16>
__device__ inline f4 mma_raw(u4 a, u4 b, f4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a),
                                                   __builtin_bit_cast(b8, b), c, 0, 0, 0);
  else
    return mma_f16(a, b, c);
}

__device__ inline float wave_max_kq(float x) {  // max over lanes l, l^16, l^32, l^48
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float wave_sum_kq(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// 16-bit input pair -> fp16 pair (bf16 widened exactly, then RNE to fp16).
template <bool BF16>
__device__ inline uint32_t to_f16_pair(uint32_t w) {
  if constexpr (!BF16) return w;
  const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
  return (uint32_t)f32_to_half_bits(lo) | ((uint32_t)f32_to_half_bits(hi) << 16);
}

// Splits fp32 p into two 16-bit parts of the raw dtype with p ~= hi + lo to
// ~2^-16 relative, so that the ring's raw 16-bit values multiply p at fp32-
// like precision.
template <bool BF16>
__device__ inline void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  if constexpr (BF16) {
    const uint32_t ua = __float_as_uint(a) & 0xffff0000u, ub = __float_as_uint(b) & 0xffff0000u;
    const float ra = a - __uint_as_float(ua), rb = b - __uint_as_float(ub);
    hi = (ua >> 16) | ub;
    lo = (__float_as_uint(ra) >> 16) | (__float_as_uint(rb) & 0xffff0000u);
  } else {
    hi = pk_rne(a, b);
    const h2 h = u2h(hi);
    lo = pk_rne(a - (float)h[0], b - (float)h[1]);
  }
}

template <bool BF16, int HIMODE>
__global__ __launch_bounds__(64) void decode_split_kernel(Geo g, const uint16_t* __restrict__ q,
                                                          kvq_cache c, float scale_log2, int S,
                                                          float* __restrict__ partials) {
  const int lane = threadIdx.x, col = lane & 15, kq = lane >> 4;
  const int bh = blockIdx.x / S, s = blockIdx.x % S;
  const int b = bh / g.Hkv, kh = bh % g.Hkv;
  const bool hvalid = col < g.G;
  const int head = kh * g.G + (hvalid ? col : 0);

  const int T = c.len[bh];
  const int nq = n_quant(T, g.R), ngq = nq / GS;
  const int nrb = (T - nq + GS - 1) / GS;
  const int NB = ngq + nrb;
  const int n0 = (int)((long long)s * NB / S), n1 = (int)((long long)(s + 1) * NB / S);

  // query: lane (col, kq) holds channels 32kq .. 32kq+31 of head col
  uint32_t qraw[16], q16[16];
  {
    const u4* qp = (const u4*)(q + ((size_t)b * g.Hq + head) * D + 32 * kq);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      u4 v = hvalid ? qp[i] : u4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        qraw[4 * i + e] = v[e];
        q16[4 * i + e] = to_f16_pair<BF16>(v[e]);
      }
    }
  }

  // salient channels (ascending): pairs of rank < n_hi, then the same + 64
  __shared__ int hil[16];
  uint32_t qhi[4] = {0, 0, 0, 0};  // HIMODE 4: 4*q (fp16); HIMODE 16: raw q
  float q4f[8];                    // HIMODE 4: 4*q in fp32
  int hch[8];                      // salient channel of digit 8*(kq&1) + e
  if constexpr (HIMODE != 0) {
    __shared__ unsigned long long smask;
    if (lane == 0) smask = 0;
    if (lane < 16) hil[lane] = 0;  // stays in range even for a malformed rank table
    __syncthreads();
    if (lane < g.n_hi) atomicOr(&smask, 1ull << (c.pairs[(size_t)bh * NPAIR + lane] & 63));
    __syncthreads();
    const unsigned long long m = smask;
    if ((m >> lane) & 1) {
      const int idx = __popcll(m & ((1ull << lane) - 1));
      hil[idx] = lane;
      hil[g.n_hi + idx] = lane + NPAIR;
    }
    __syncthreads();
    const uint16_t* qrow = q + ((size_t)b * g.Hq + head) * D;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int d = 8 * (kq & 1) + e;
      // HIMODE 4: K-lanes 16..31 (kq 2, 3) repeat the digits of lanes 0..15
      // and carry the rounding residual of 4*q*s; HIMODE 16 uses lanes 0..15
      const bool ok = hvalid && d < g.nh && (HIMODE == 4 || kq < 2);
      hch[e] = ok ? (hil[d] & (D - 1)) : 0;
      float v = ok ? in_to_f32(qrow[hch[e]], BF16) : 0.0f;
      q4f[e] = 4.0f * v;
      uint32_t bits;
      if constexpr (HIMODE == 4)
        bits = f32_to_half_bits(4.0f * v);
      else
        bits = ok ? qrow[hch[e]] : 0u;
      qhi[e >> 1] |= bits << (16 * (e & 1));
    }
  }

  float m_run = -INFINITY, l_raw = 0.0f;
  f4 O[8], Cvb = {0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < 8; t++) O[t] = f4{0, 0, 0, 0};
  const uint32_t ONES = 0x3c003c00u;  // fp16 (1, 1)

  for (int n = n0; n < n1; n++) {
    f4 C[2];
    if (n < ngq) {
      // ------------------------------------------------ quantized group
      const size_t rec = (size_t)bh * g.NG + n;
      const uint32_t* kmeta = (const uint32_t*)c.k_meta + rec * (2 * D / 2);
      uint32_t qs[16];
      f4 cb = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const u4 sv = ((const u4*)(kmeta + 16 * kq))[i];
        const u4 zv = ((const u4*)(kmeta + 64 + 16 * kq))[i];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          qs[4 * i + e] = pk_mul(q16[4 * i + e], sv[e]);
        }
        cb = mma_f16(zv, u4{q16[4 * i], q16[4 * i + 1], q16[4 * i + 2], q16[4 * i + 3]}, cb);
      }
      uint32_t qshi[4];
      if constexpr (HIMODE == 4) {
        const uint16_t* ks = (const uint16_t*)c.k_meta + rec * 2 * D;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          // 4*q*s is exact in fp32 (8- or 11-bit q times 11-bit s); split it
          // into its fp16 rounding hi and the fp16 residual lo
          const uint32_t sp = (uint32_t)ks[hch[2 * e]] | ((uint32_t)ks[hch[2 * e + 1]] << 16);
          const uint32_t hi = pk_mul(qhi[e], sp);
          const h2 sh = u2h(sp), hh = u2h(hi);
          const uint32_t lo = pk_rne(fmaf(q4f[2 * e], (float)sh[0], -(float)hh[0]),
                                     fmaf(q4f[2 * e + 1], (float)sh[1], -(float)hh[1]));
          qshi[e] = kq < 2 ? hi : lo;
        }
      }
      const u2* klo = (const u2*)((const uint32_t*)c.k_lo + rec * GROUP_WORDS);
#pragma unroll
      for (int TT = 0; TT < 2; TT++) {
        const u2 w = klo[(TT * 4 + kq) * 16 + col];
        f4 acc = cb;
#pragma unroll
        for (int u = 0; u < 2; u++) {
          const uint32_t A = w[u] & 0x33333333u, Bn = (w[u] >> 2) & 0x33333333u;
          const int k0 = 8 * u;
          acc = mma_f16(u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)},
                        u4{qs[k0], qs[k0 + 1], qs[k0 + 2], qs[k0 + 3]}, acc);
          acc = mma_f16(u4{cvt2<2>(A), cvt2<2>(Bn), cvt2<3>(A), cvt2<3>(Bn)},
                        u4{qs[k0 + 4], qs[k0 + 5], qs[k0 + 6], qs[k0 + 7]}, acc);
        }
        if constexpr (HIMODE == 4) {
          const uint32_t wh = ((const uint32_t*)c.k_hi)[rec * 32 + 16 * TT + col];
          const uint32_t ws = (kq & 1) ? wh >> 16 : wh;
          const uint32_t A = ws & 0x33333333u, Bn = (ws >> 2) & 0x33333333u;
          acc = mma_f16(u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)},
                        u4{qshi[0], qshi[1], qshi[2], qshi[3]}, acc);
        }
        if constexpr (HIMODE == 16) {
          const uint16_t* raw = (const uint16_t*)c.k_hi + rec * GS * g.nh + (16 * TT + col) * g.nh;
          uint32_t a[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const int d = 8 * (kq & 1) + e;
            const uint32_t v = (kq < 2 && d < g.nh) ? raw[d] : 0u;
            a[e >> 1] |= v << (16 * (e & 1));
          }
          acc = mma_raw<BF16>(u4{a[0], a[1], a[2], a[3]}, u4{qhi[0], qhi[1], qhi[2], qhi[3]}, acc);
        }
        C[TT] = acc;
      }
      // online softmax (base 2)
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; i++) x[i] = C[i >> 2][i & 3] * scale_log2;
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; i++) mx = fmaxf(mx, x[i]);
      const float m_new = fmaxf(m_run, wave_max_kq(mx));
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 8; t++) O[t] *= alpha;
      Cvb *= alpha;
      l_raw *= alpha;
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; i++) p[i] = exp2f(x[i] - m_new);
      const uint32_t P[4] = {pk_rne(p[0], p[1]),
                             pk_rne(p[2], p[3]),
                             pk_rne(p[4], p[5]),
                             pk_rne(p[6], p[7])};
      // values
      const uint32_t* vmeta = (const uint32_t*)c.v_meta + rec * (2 * D / 2);
      u4 za;
      if (col < 4)
        za = ((const u4*)(vmeta + 64 + 16 * col))[kq];
      else if (col == 4)
        za = u4{ONES, ONES, ONES, ONES};
      else
        za = u4{0, 0, 0, 0};
      Cvb = mma_f16(za, u4{P[0], P[1], P[2], P[3]}, Cvb);
      const uint32_t* vc = (const uint32_t*)c.v_codes + rec * GROUP_WORDS;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const u4 sv = ((const u4*)(vmeta + 16 * j))[kq];
        const u4 pj = u4{pk_mul(P[0], sv[0]), pk_mul(P[1], sv[1]), pk_mul(P[2], sv[2]),
                         pk_mul(P[3], sv[3])};
        const uint32_t wv = vc[(j * 4 + kq) * 16 + col];
        const uint32_t A = wv & 0x33333333u, Bn = (wv >> 2) & 0x33333333u;
        O[2 * j] = mma_f16(u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)}, pj, O[2 * j]);
        O[2 * j + 1] =
            mma_f16(u4{cvt2<2>(A), cvt2<2>(Bn), cvt2<3>(A), cvt2<3>(Bn)}, pj, O[2 * j + 1]);
      }
    } else {
      // --------------------------------------------- ring block (16-bit)
      const int pbase = nq + GS * (n - ngq);
      const int nvalid = min(GS, T - pbase);
      const int sb = (pbase / GS) % (g.RS / GS);
      const uint16_t* rk = (const uint16_t*)c.ring_k + ((size_t)bh * g.RS + sb * GS) * D;
#pragma unroll
      for (int TT = 0; TT < 2; TT++) {
        const int t = tile_token(16 * TT + col);
        const u4* kr = (const u4*)(rk + (size_t)t * D + 32 * kq);
        f4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 4; k++)
          acc = mma_raw<BF16>(kr[k], u4{qraw[4 * k], qraw[4 * k + 1], qraw[4 * k + 2], qraw[4 * k + 3]},
                              acc);
        C[TT] = acc;
      }
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int t = 8 * kq + 4 * (i >> 2) + (i & 3);
        x[i] = t < nvalid ? C[i >> 2][i & 3] * scale_log2 : -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; i++) mx = fmaxf(mx, x[i]);
      const float m_new = fmaxf(m_run, wave_max_kq(mx));
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 8; t++) O[t] *= alpha;
      Cvb *= alpha;
      l_raw *= alpha;
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        p[i] = exp2f(x[i] - m_new);
        l_raw += p[i];
      }
      uint32_t Ph[4], Pl[4];
#pragma unroll
      for (int i = 0; i < 4; i++) split_pair<BF16>(p[2 * i], p[2 * i + 1], Ph[i], Pl[i]);
      const uint16_t* rv = (const uint16_t*)c.ring_v + (((size_t)bh * (g.RS / GS) + sb) * D) * GS;
#pragma unroll
      for (int tt = 0; tt < 8; tt++) {
        u4 a = *(const u4*)(rv + (size_t)(16 * tt + col) * GS + 8 * kq);
        // zero slots past the last token (they may hold stale data)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int t0 = 8 * kq + 2 * e;
          const uint32_t keep = (t0 < nvalid ? 0x0000ffffu : 0u) | (t0 + 1 < nvalid ? 0xffff0000u : 0u);
          a[e] &= keep;
        }
        O[tt] = mma_raw<BF16>(a, u4{Ph[0], Ph[1], Ph[2], Ph[3]}, O[tt]);
        O[tt] = mma_raw<BF16>(a, u4{Pl[0], Pl[1], Pl[2], Pl[3]}, O[tt]);
      }
    }
  }

  // softmax denominator: all-ones row (row 4 -> lane 16 + col, element 0)
  // of the value-zero MFMA, plus the ring blocks' fp32 sum
  const float l_q = __shfl(Cvb[0], 16 + col);
  const float l = l_q + wave_sum_kq(l_raw);
  float vb[4];
#pragma unroll
  for (int j = 0; j < 4; j++) vb[j] = __shfl(Cvb[j], col);  // rows 0..3 -> lane col
  if (hvalid) {
    float* out = partials + ((size_t)(b * g.Hq + head) * S + s) * PART;
    if (kq == 0) {
      out[0] = m_run;
      out[1] = l;
    }
#pragma unroll
    for (int tt = 0; tt < 8; tt++) {
      f4 v = O[tt] + vb[tt >> 1];
      *(f4*)(out + 4 + 16 * tt + 4 * kq) = v;
    }
  }
}

// Merges the splits of one (b, query head): thread c owns channel c.
template <bool BF16>
__global__ __launch_bounds__(D) void combine_kernel(int S, const float* __restrict__ partials,
                                                    uint16_t* __restrict__ out) {
  const int bhq = blockIdx.x, c = threadIdx.x;
  const float* p = partials + (size_t)bhq * S * PART;
  float M = -INFINITY;
  for (int s = 0; s < S; s++) M = fmaxf(M, p[(size_t)s * PART]);
  float L = 0.0f, acc = 0.0f;
  for (int s = 0; s < S; s++) {
    const float m = p[(size_t)s * PART];
    if (m == -INFINITY) continue;
    const float w = exp2f(m - M);
    L += w * p[(size_t)s * PART + 1];
    acc += w * p[(size_t)s * PART + 4 + c];
  }
  const float o = L > 0.0f ? acc / L : 0.0f;
  uint16_t bits;
  if constexpr (BF16) {
    const uint32_t u = __float_as_uint(o);
    bits = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  } else {
    bits = f32_to_half_bits(o);
  }
  out[(size_t)bhq * D + c] = bits;
}

template <bool BF16, int HIMODE>
static void launch_split(const Geo& g, const void* q, const kvq_cache* c, float scale_log2,
                         int S, float* partials, hipStream_t st) {
  hipLaunchKernelGGL((decode_split_kernel<BF16, HIMODE>), dim3(g.B * g.Hkv * S), dim3(64), 0, st,
                     g, (const uint16_t*)q, *c, scale_log2, S, partials);
}

hipError_t launch_decode(const Geo& g, const void* q, const kvq_cache* c, float sm_scale,
                         int S, float* partials, void* out, hipStream_t st) {
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  const int hm = g.n_hi == 0 ? 0 : g.bits_hi;
  if (g.bf16) {
    if (hm == 0) launch_split<true, 0>(g, q, c, scale_log2, S, partials, st);
    else if (hm == 4) launch_split<true, 4>(g, q, c, scale_log2, S, partials, st);
    else launch_split<true, 16>(g, q, c, scale_log2, S, partials, st);
    hipLaunchKernelGGL(combine_kernel<true>, dim3(g.B * g.Hq), dim3(D), 0, st, S,
                       (const float*)partials, (uint16_t*)out);
  } else {
    if (hm == 0) launch_split<false, 0>(g, q, c, scale_log2, S, partials, st);
    else if (hm == 4) launch_split<false, 4>(g, q, c, scale_log2, S, partials, st);
    else launch_split<false, 16>(g, q, c, scale_log2, S, partials, st);
    hipLaunchKernelGGL(combine_kernel<false>, dim3(g.B * g.Hq), dim3(D), 0, st, S,
                       (const float*)partials, (uint16_t*)out);
  }
  return hipGetLastError();
}

}  // namespace kvq
