// quant.hip — key and value quantization into the packed cache, the 16-bit
// ring of recent tokens, and the decode-step append.
//
// Keys (PN-Mix, abstract: salient RoPE pairs at a higher bit width, the other
// key channels at 2 bits; PM-KVQ review, supporting_citations: keys per
// channel) are quantized per channel over groups of 32 tokens; values
// (MixKVQ, abstract; PM-KVQ review: values per token) per token over groups of
// 32 channels.  Recent tokens stay 16-bit in a ring (PM-KVQ review,
// key_machinery and supporting_citations: 16-bit first, quantized later).
//
// One 256-thread block packs one 32-token group: 128 threads quantize (one
// key channel, or one value (token, channel group) each) into a 32x128 code
// tile in LDS, then all 256 threads assemble one 32-bit word each of the
// layout in include/kvq.h.
#include "common.h"
#include "internal.h"

namespace kvq {

constexpr int QTHREADS = 256;

struct GroupLds {
  uint8_t codes[GS][D];  // [token][channel]
  int salient[D];        // 1 if channel c belongs to a salient pair
  int hil[16];           // salient channels, ascending
};

// Source of one group's 16-bit values: src(t, c) = bits of token t (0..31 in
// the group), channel c.
struct DenseSrc {  // prefill input [..][T][128], group starting at token t0
  const uint16_t* base;
  __device__ uint16_t operator()(int t, int c) const { return base[(size_t)t * D + c]; }
};
struct RingKSrc {  // ring_k [RS][128] of one (b, kv head), group at slot s0
  const uint16_t* base;
  int s0;
  __device__ uint16_t operator()(int t, int c) const { return base[(size_t)(s0 + t) * D + c]; }
};
struct RingVSrc {  // ring_v [RS/32][128][32] of one (b, kv head), slot block sb
  const uint16_t* block;
  __device__ uint16_t operator()(int t, int c) const { return block[(size_t)c * GS + t]; }
};

template <class Src>
__device__ void quant_key_group(const Geo& g, const Src& src, const int32_t* pairs,
                                uint32_t* lo_out, void* hi_out, uint16_t* meta_out,
                                GroupLds& lds) {
  const int tid = threadIdx.x;
  if (tid < D) {
    const int c = tid, pj = c & (NPAIR - 1);
    int sal = 0, one = 0;
    for (int r = 0; r < g.n_hi; r++) sal |= pairs[r] == pj;
    for (int r = NPAIR - g.n_lo1; r < NPAIR; r++) one |= pairs[r] == pj;
    lds.salient[c] = sal;
    // salient pairs at bits_hi, the n_lo1 lowest-ranked pairs at one bit
    // (their codes 0/1 sit in the 2-bit slots of k_lo), the rest at 2 bits
    const int bits = sal ? g.bits_hi : (one ? 1 : 2);
    uint16_t s = 0, z = 0;
    uint8_t codes[GS];
    if (bits == 16) {
#pragma unroll
      for (int i = 0; i < GS; i++) codes[i] = 0;
    } else {
      float x[GS];
#pragma unroll
      for (int i = 0; i < GS; i++) x[i] = in_to_f32(src(i, c), g.bf16);
      quantize_group(x, (1 << bits) - 1, s, z, codes);
    }
#pragma unroll
    for (int i = 0; i < GS; i++) lds.codes[i][c] = codes[i];
    meta_out[c] = s;
    meta_out[D + c] = z;
  }
  __syncthreads();
  if (tid < D && lds.salient[tid]) {
    int idx = 0;
    for (int c = 0; c < tid; c++) idx += lds.salient[c];
    lds.hil[idx] = tid;
  }
  {
    // low two bits of every channel's code, token-major in tile order
    const int wi = tid, u = wi & 1, r = (wi >> 1) & 15, kq = (wi >> 5) & 3, T = wi >> 7;
    const int t = tile_token(16 * T + r), w = 2 * kq + u;
    uint32_t word = 0;
#pragma unroll
    for (int cc = 0; cc < 16; cc++)
      word |= (uint32_t)(lds.codes[t][16 * w + cc] & 3) << (2 * pos_swap(cc));
    lo_out[wi] = word;
  }
  __syncthreads();
  if (g.nh && g.bits_hi == 4 && tid < GS) {
    const int t = tile_token(tid);
    uint32_t word = 0;
    for (int d = 0; d < g.nh; d++)
      word |= (uint32_t)(lds.codes[t][lds.hil[d]] >> 2) << (2 * pos_swap(d));
    ((uint32_t*)hi_out)[tid] = word;
  } else if (g.nh && g.bits_hi == 16) {
    for (int idx = tid; idx < GS * g.nh; idx += QTHREADS) {
      const int e = idx / g.nh, d = idx % g.nh;
      ((uint16_t*)hi_out)[idx] = src(tile_token(e), lds.hil[d]);
    }
  }
  __syncthreads();
}

template <class Src>
__device__ void quant_value_group(const Geo& g, const Src& src, uint32_t* vc_out,
                                  uint16_t* meta_out, GroupLds& lds) {
  const int tid = threadIdx.x;
  if (tid < D) {
    const int t = tid >> 2, j = tid & 3;
    float x[GS];
#pragma unroll
    for (int i = 0; i < GS; i++) x[i] = in_to_f32(src(t, GS * j + i), g.bf16);
    uint16_t s, z;
    uint8_t codes[GS];
    quantize_group(x, 3, s, z, codes);
#pragma unroll
    for (int i = 0; i < GS; i++) lds.codes[t][GS * j + i] = codes[i];
    meta_out[j * GS + t] = s;
    meta_out[D + j * GS + t] = z;
  }
  __syncthreads();
  {
    const int wi = tid, c = wi & 15, kq = (wi >> 4) & 3, j = wi >> 6;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int t = 8 * kq + i, p = 2 * pos_swap(i);
      word |= (uint32_t)lds.codes[t][GS * j + c] << p;
      word |= (uint32_t)lds.codes[t][GS * j + 16 + c] << (16 + p);
    }
    vc_out[wi] = word;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ prefill

__global__ __launch_bounds__(QTHREADS) void quant_keys_kernel(Geo g, const uint16_t* __restrict__ k,
                                                              int T, kvq_cache c) {
  __shared__ GroupLds lds;
  const int bh = blockIdx.x, grp = blockIdx.y;
  const size_t rec = (size_t)bh * g.NG + grp;
  DenseSrc src{k + ((size_t)bh * T + (size_t)grp * GS) * D};
  quant_key_group(g, src, c.pairs + (size_t)bh * NPAIR, (uint32_t*)c.k_lo + rec * GROUP_WORDS,
                  (uint8_t*)c.k_hi + rec * g.khi_bytes, (uint16_t*)c.k_meta + rec * 2 * D, lds);
}

__global__ __launch_bounds__(QTHREADS) void quant_values_kernel(Geo g, const uint16_t* __restrict__ v,
                                                                int T, kvq_cache c) {
  __shared__ GroupLds lds;
  const int bh = blockIdx.x, grp = blockIdx.y;
  const size_t rec = (size_t)bh * g.NG + grp;
  DenseSrc src{v + ((size_t)bh * T + (size_t)grp * GS) * D};
  quant_value_group(g, src, (uint32_t*)c.v_codes + rec * GROUP_WORDS,
                    (uint16_t*)c.v_meta + rec * 2 * D, lds);
}

// Copies positions [n_q(T), T) of one (b, kv head) into the ring and sets
// len = T.  is_v selects the value ring's slot-block/channel/slot order.
__global__ __launch_bounds__(QTHREADS) void ring_fill_kernel(Geo g, const uint16_t* __restrict__ x,
                                                             int T, int is_v, kvq_cache c) {
  const int bh = blockIdx.x;
  const int p0 = n_quant(T, g.R);
  const int n = (T - p0) * D;
  const uint16_t* src = x + ((size_t)bh * T + p0) * D;
  uint16_t* ring = (uint16_t*)(is_v ? c.ring_v : c.ring_k) + (size_t)bh * g.RS * D;
  for (int i = threadIdx.x; i < n; i += QTHREADS) {
    const int p = p0 + i / D, ch = i % D, slot = p % g.RS;
    const size_t dst = is_v ? ((size_t)(slot / GS) * D + ch) * GS + slot % GS
                            : (size_t)slot * D + ch;
    ring[dst] = src[i];
  }
  if (threadIdx.x == 0) c.len[bh] = T;
}

// ------------------------------------------------------------------- append

__global__ __launch_bounds__(QTHREADS) void append_kernel(Geo g, const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new,
                                                          kvq_cache c) {
  __shared__ GroupLds lds;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int T = c.len[bh];
  if (T >= g.max_tokens) {
    if (tid == 0) atomicOr(c.err, 1);
    return;
  }
  uint16_t* rk = (uint16_t*)c.ring_k + (size_t)bh * g.RS * D;
  uint16_t* rv = (uint16_t*)c.ring_v + (size_t)bh * g.RS * D;
  const int slot = T % g.RS;
  if (tid < D) {
    rk[(size_t)slot * D + tid] = k_new[(size_t)bh * D + tid];
    rv[((size_t)(slot / GS) * D + tid) * GS + slot % GS] = v_new[(size_t)bh * D + tid];
  }
  const int nq0 = n_quant(T, g.R);
  if (n_quant(T + 1, g.R) > nq0) {
    // the group [nq0, nq0 + 32) ends at T + 1 - R <= T: the new token is not in it
    const int grp = nq0 / GS, s0 = nq0 % g.RS;
    const size_t rec = (size_t)bh * g.NG + grp;
    quant_key_group(g, RingKSrc{rk, s0}, c.pairs + (size_t)bh * NPAIR,
                    (uint32_t*)c.k_lo + rec * GROUP_WORDS, (uint8_t*)c.k_hi + rec * g.khi_bytes,
                    (uint16_t*)c.k_meta + rec * 2 * D, lds);
    quant_value_group(g, RingVSrc{rv + (size_t)(s0 / GS) * D * GS},
                      (uint32_t*)c.v_codes + rec * GROUP_WORDS, (uint16_t*)c.v_meta + rec * 2 * D,
                      lds);
  }
  __syncthreads();
  if (tid == 0) c.len[bh] = T + 1;
}

hipError_t launch_quant_keys(const Geo& g, const void* k, int T, kvq_cache* c, hipStream_t st) {
  const int ng = n_quant(T, g.R) / GS;
  if (ng > 0)
    hipLaunchKernelGGL(quant_keys_kernel, dim3(g.B * g.Hkv, ng), dim3(QTHREADS), 0, st, g,
                       (const uint16_t*)k, T, *c);
  hipLaunchKernelGGL(ring_fill_kernel, dim3(g.B * g.Hkv), dim3(QTHREADS), 0, st, g,
                     (const uint16_t*)k, T, 0, *c);
  return hipGetLastError();
}

hipError_t launch_quant_values(const Geo& g, const void* v, int T, kvq_cache* c, hipStream_t st) {
  const int ng = n_quant(T, g.R) / GS;
  if (ng > 0)
    hipLaunchKernelGGL(quant_values_kernel, dim3(g.B * g.Hkv, ng), dim3(QTHREADS), 0, st, g,
                       (const uint16_t*)v, T, *c);
  hipLaunchKernelGGL(ring_fill_kernel, dim3(g.B * g.Hkv), dim3(QTHREADS), 0, st, g,
                     (const uint16_t*)v, T, 1, *c);
  return hipGetLastError();
}

// In-place precision shrink of the 4-bit salient key channels (PM-KVQ
// review, key_machinery): the b-bit code of a 2b-bit code X is the review's
// shift form ((2^2b - 2^b + 1) * (X + 2^(b-1))) >> 3b, i.e. round(X / (2^b+1)),
// on the grid of step (2^b + 1) s with the zero point kept.  Here 2b = 4: the
// new value z + 5 s q is held as the 4-bit code 5 q = 4 q + q under the
// unchanged scale s, i.e. both the high and the low digit become q, so the
// step 5 s is exact and decoding keeps its precise paths.  One 64-lane
// workgroup per (b, kv head, group); lane e < 32 owns the token of tile
// index e, so its key words are written by it alone.
__device__ inline uint32_t shrink_4_to_2(uint32_t x) { return (13u * (x + 2u)) >> 6; }

__global__ __launch_bounds__(64) void shrink_kernel(Geo g, kvq_cache c, int g0, int g1) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const int ngq = n_quant(c.len[bh], g.R) / GS;
  const int grp = g0 + (int)blockIdx.y;
  if (grp >= min(g1, ngq)) return;
  const size_t rec = (size_t)bh * g.NG + grp;
  // salient channels, ascending: pairs of rank < n_hi, then the same + 64
  const int32_t* pr = c.pairs + (size_t)bh * NPAIR;
  bool sal = false;
  for (int r = 0; r < g.n_hi; r++) sal |= pr[r] == (lane & (NPAIR - 1));
  const unsigned long long m = __ballot(sal);
  __shared__ int hil[16];
  if (sal && lane < NPAIR) {
    const int idx = __popcll(m & ((1ull << lane) - 1));
    hil[idx] = lane;
    hil[g.n_hi + idx] = lane + NPAIR;
  }
  __syncthreads();
  if (lane < GS) {
    const int e = lane, T = e >> 4, r = e & 15;
    uint32_t* hi = (uint32_t*)c.k_hi + rec * 32;
    uint32_t* lo = (uint32_t*)c.k_lo + rec * GROUP_WORDS;
    uint32_t hw = hi[e];
    for (int d = 0; d < g.nh; d++) {
      const int ch = hil[d], w = ch >> 4, kq = w >> 1, u = w & 1;
      uint32_t& lw = lo[((T * 4 + kq) * 16 + r) * 2 + u];
      const int pl = 2 * pos_swap(ch & 15), ph = 2 * pos_swap(d);
      const uint32_t q = shrink_4_to_2((((hw >> ph) & 3u) << 2) | ((lw >> pl) & 3u));
      lw = (lw & ~(3u << pl)) | (q << pl);
      hw = (hw & ~(3u << ph)) | (q << ph);
    }
    hi[e] = hw;
  }
}

hipError_t launch_shrink(const Geo& g, kvq_cache* c, int g0, int g1, hipStream_t st) {
  if (g1 <= g0 || g.nh == 0 || g.NG == 0) return hipSuccess;
  hipLaunchKernelGGL(shrink_kernel, dim3(g.B * g.Hkv, g1 - g0), dim3(64), 0, st, g, *c, g0, g1);
  return hipGetLastError();
}

hipError_t launch_append(const Geo& g, const void* k_new, const void* v_new, kvq_cache* c,
                         hipStream_t st) {
  hipLaunchKernelGGL(append_kernel, dim3(g.B * g.Hkv), dim3(QTHREADS), 0, st, g,
                     (const uint16_t*)k_new, (const uint16_t*)v_new, *c);
  return hipGetLastError();
}

}  // namespace kvq
