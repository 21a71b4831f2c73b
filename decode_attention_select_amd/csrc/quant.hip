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
// One wave quantizes one 32-token group.  Each lane holds an 8 x 8 block of
// the group (8 tokens x 8 channels, two 16-byte loads' worth per token row),
// so a group is eight 16-byte loads per lane.  The min/max reductions run
// in registers and across the four lanes of a DPP quad:
//   keys:   lane = 4 * cb + tq  (channels 8cb..8cb+7, tokens 8tq..8tq+7);
//           a channel's 32 tokens lie in one quad.
//   values: lane = 16 * tq + cb; a token's 32-channel group (4 chunks of 8)
//           lies in one quad.
// Each quad lane computes the scale, zero and reciprocal of two of the
// quad's eight channels (or tokens) and hands them to the others by DPP
// broadcast, so each division runs once per quad.
#include "common.h"
#include "internal.h"
#include "quant_group.h"

namespace kvq {

constexpr int QWAVES = 4;                 // groups per prefill workgroup, one per wave
constexpr int QTHREADS = 64 * QWAVES;
constexpr int RING_ROWS = QTHREADS / 16;  // ring-fill rows per workgroup (16 B per thread)

// The device code that packs one 32-token group (one wave for its keys, one
// for its values) is in quant_group.h, shared with the decode kernel's
// append step.

// ------------------------------------------------------------------ prefill

// Positions [n_q(T), T) of one (b, kv head) into the ring, 16 rows per
// workgroup, 16 bytes per thread; the first ring workgroup sets len = T.
__device__ void ring_fill(const Geo& g, const uint16_t* __restrict__ x, int T, int ry, bool is_v,
                          kvq_cache& c) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int p = n_quant(T, g.R) + RING_ROWS * ry + (tid >> 4), ch = 8 * (tid & 15);
  if (p < T) {
    const uint4 val = *(const uint4*)(x + ((size_t)bh * T + p) * D + ch);
    const int slot = p % g.RS;
    if (!is_v) {
      *(uint4*)((uint16_t*)c.ring_k + ((size_t)bh * g.RS + slot) * D + ch) = val;
    } else {
      uint16_t* blk = (uint16_t*)c.ring_v + ((size_t)bh * g.RS + (slot / GS) * GS) * D;
#pragma unroll
      for (int k = 0; k < 8; k++) blk[(size_t)(ch + k) * GS + slot % GS] = half_of(val, k);
    }
  }
  if (ry == 0 && tid == 0) c.len[bh] = T;
}

// Layout kinds of the quantize and append kernels: each variant compiles
// only the record paths its layout can take (a path compiled in but never
// taken still costs registers, and with them occupancy).
constexpr int KIND_PLAIN = 0, KIND_DENSE1 = 1, KIND_PROG = 2;

static int layout_kind(const Geo& g) {
  return g.w4 > 0 ? KIND_PROG : (g.dense1 ? KIND_DENSE1 : KIND_PLAIN);
}

// grid (B * Hkv, qblocks + ring blocks): blocks below qblocks quantize
// QWAVES groups, one per wave; the rest fill the ring.
// VHI: each wave ranks its group's tokens, packs the keys in that order and
// writes the order to the group's v_hi header.
template <bool BF, bool VHI, int KIND>
__global__ __launch_bounds__(QTHREADS) void quant_keys_kernel(Geo g, const uint16_t* __restrict__ k,
                                                              int T, int qblocks, kvq_cache c) {
  if ((int)blockIdx.y >= qblocks) {
    ring_fill(g, k, T, blockIdx.y - qblocks, false, c);
    return;
  }
  __shared__ KeyLds lds[QWAVES];
  const int bh = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = blockIdx.y * QWAVES + wave;
  if (grp >= n_quant(T, g.R) / GS) return;
  const size_t rec = (size_t)bh * g.NG + grp;
  // progressive precision: the width of the group's age among n_q / 32
  const int width =
      KIND == KIND_PROG ? prog_width(n_quant(T, g.R) / GS - 1 - grp, g.w8, g.w4) : 0;
  key_group_wave<BF, VHI, KIND == KIND_DENSE1, KIND == KIND_PROG>(
      g, k + ((size_t)bh * T + (size_t)grp * GS) * D, pair_masks(g, c.pairs + (size_t)bh * NPAIR),
      (uint32_t*)((uint8_t*)c.k_lo + rec * g.klo_bytes), (uint8_t*)c.k_hi + rec * g.khi_bytes,
      (uint16_t*)c.k_meta + rec * 2 * D, lds[wave], width,
      width >= 4 ? plane1(g, c.k_pl, bh, grp) : nullptr,
      width == 8 ? plane23(g, c.k_pl, bh, grp) : nullptr);
  if constexpr (VHI)
    if (lane < 2) ((uint4*)(c.v_hi + rec * g.vhi_words))[lane] = ((const uint4*)lds[wave].ord)[lane];
}

// VHI: the group's token order comes from the v_hi header that the key
// kernel wrote (an earlier launch on the same stream).  Its bytes are masked
// to 0..31, so a header the key kernel never wrote cannot move a load out
// of the group.
template <bool BF, bool VHI, bool PROG>
__global__ __launch_bounds__(QTHREADS) void quant_values_kernel(Geo g, const uint16_t* __restrict__ v,
                                                                int T, int qblocks, kvq_cache c) {
  if ((int)blockIdx.y >= qblocks) {
    ring_fill(g, v, T, blockIdx.y - qblocks, true, c);
    return;
  }
  const int bh = blockIdx.x, wave = threadIdx.x >> 6, tq = (threadIdx.x & 63) >> 4;
  const int grp = blockIdx.y * QWAVES + wave;
  if (grp >= n_quant(T, g.R) / GS) return;
  const size_t rec = (size_t)bh * g.NG + grp;
  uint32_t* vhi = c.v_hi + rec * g.vhi_words;
  uint2 pos = make_uint2(0, 0);
  if constexpr (VHI) {
    pos = ((const uint2*)vhi)[tq];
    pos.x &= 0x1F1F1F1Fu;
    pos.y &= 0x1F1F1F1Fu;
  }
  const int width = PROG ? prog_width(n_quant(T, g.R) / GS - 1 - grp, g.w8, g.w4) : 0;
  value_group_wave<BF, false, VHI, PROG>(g, v + ((size_t)bh * T + (size_t)grp * GS) * D, pos,
                                   (uint32_t*)c.v_codes + rec * GROUP_WORDS,
                                   (uint16_t*)c.v_meta + rec * 2 * D, vhi, width,
                                   width >= 4 ? plane1(g, c.v_pl, bh, grp) : nullptr,
                                   width == 8 ? plane23(g, c.v_pl, bh, grp) : nullptr);
}

// ------------------------------------------------------------------- append

// One 128-thread workgroup per (b, kv head): the new token goes to ring slot
// T mod RS; when n_q grows, wave 0 packs the oldest ring group's keys and
// wave 1 its values (the new token is not in that group).  VHI: both waves
// rank the group's tokens from the ring keys (the same integer sums, so the
// same order); wave 0 also writes it to the v_hi header.
template <bool BF, bool VHI, int KIND>
__global__ __launch_bounds__(128) void append_kernel(Geo g, const uint16_t* __restrict__ k_new,
                                                     const uint16_t* __restrict__ v_new,
                                                     kvq_cache c) {
  __shared__ PackLds lds;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int T = c.len[bh];
  if (T < 0 || T >= g.max_tokens) {  // full, or a length no call of this library wrote
    if (tid == 0) atomicOr(c.err, T < 0 ? 2 : 1);
    return;
  }
  uint16_t* rk = (uint16_t*)c.ring_k + (size_t)bh * g.RS * D;
  uint16_t* rv = (uint16_t*)c.ring_v + (size_t)bh * g.RS * D;
  const int slot = T % g.RS;
  rk[(size_t)slot * D + tid] = k_new[(size_t)bh * D + tid];
  rv[((size_t)(slot / GS) * D + tid) * GS + slot % GS] = v_new[(size_t)bh * D + tid];
  const int nq0 = n_quant(T, g.R);
  if (n_quant(T + 1, g.R) > nq0) pack_ring_group<BF, VHI, KIND == KIND_PROG, KIND == KIND_DENSE1>(g, c, bh, nq0, tid, lds);
  __syncthreads();
  if (tid == 0) c.len[bh] = T + 1;
}

// Progressive precision is never combined with two value precisions (the
// host rejects that layout), so its variants exist without VHI only.
template <bool BF>
static auto keys_kernel(const Geo& g) -> decltype(&quant_keys_kernel<BF, false, KIND_PLAIN>) {
  switch (layout_kind(g)) {
    case KIND_PROG: return quant_keys_kernel<BF, false, KIND_PROG>;
    case KIND_DENSE1:
      return g.n_vhi ? quant_keys_kernel<BF, true, KIND_DENSE1>
                     : quant_keys_kernel<BF, false, KIND_DENSE1>;
    default:
      return g.n_vhi ? quant_keys_kernel<BF, true, KIND_PLAIN>
                     : quant_keys_kernel<BF, false, KIND_PLAIN>;
  }
}

template <bool BF>
static auto values_kernel(const Geo& g) -> decltype(&quant_values_kernel<BF, false, false>) {
  if (layout_kind(g) == KIND_PROG) return quant_values_kernel<BF, false, true>;
  return g.n_vhi ? quant_values_kernel<BF, true, false> : quant_values_kernel<BF, false, false>;
}

template <bool BF>
static auto append_variant(const Geo& g) -> decltype(&append_kernel<BF, false, KIND_PLAIN>) {
  switch (layout_kind(g)) {
    case KIND_PROG: return append_kernel<BF, false, KIND_PROG>;
    case KIND_DENSE1:
      return g.n_vhi ? append_kernel<BF, true, KIND_DENSE1> : append_kernel<BF, false, KIND_DENSE1>;
    default:
      return g.n_vhi ? append_kernel<BF, true, KIND_PLAIN> : append_kernel<BF, false, KIND_PLAIN>;
  }
}

static int ring_blocks(const Geo& g, int T) {
  return (T - n_quant(T, g.R) + RING_ROWS - 1) / RING_ROWS;
}

hipError_t launch_quant_keys(const Geo& g, const void* k, int T, kvq_cache* c, hipStream_t st) {
  const int qb = (n_quant(T, g.R) / GS + QWAVES - 1) / QWAVES;
  const dim3 grid(g.B * g.Hkv, qb + ring_blocks(g, T));
  const auto kern = g.bf16 ? keys_kernel<true>(g) : keys_kernel<false>(g);
  hipLaunchKernelGGL(kern, grid, dim3(QTHREADS), 0, st, g, (const uint16_t*)k, T, qb, *c);
  return hipGetLastError();
}

hipError_t launch_quant_values(const Geo& g, const void* v, int T, kvq_cache* c, hipStream_t st) {
  const int qb = (n_quant(T, g.R) / GS + QWAVES - 1) / QWAVES;
  const dim3 grid(g.B * g.Hkv, qb + ring_blocks(g, T));
  const auto kern = g.bf16 ? values_kernel<true>(g) : values_kernel<false>(g);
  hipLaunchKernelGGL(kern, grid, dim3(QTHREADS), 0, st, g, (const uint16_t*)v, T, qb, *c);
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

constexpr int SHRINK_WAVES = 4;  // groups per workgroup, one per wave

// Lane e < 32 owns the token of tile index e: its eight k_lo words (one per
// 16-channel run, kept as four (u = 0, u = 1) pairs) and its k_hi word are loaded once,
// rewritten in registers and stored once.  The salient channels are walked
// in ascending order from the salient-pair mask (uniform loop).
__global__ __launch_bounds__(64 * SHRINK_WAVES) void shrink_kernel(Geo g, kvq_cache c, int g0,
                                                                   int g1) {
  const int bh = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ngq = n_quant(c.len[bh], g.R) / GS;
  const int grp = g0 + (int)blockIdx.y * SHRINK_WAVES + wave;
  if (grp >= min(g1, ngq) || lane >= GS) return;
  const uint64_t mhi = pair_masks(g, c.pairs + (size_t)bh * NPAIR).hi;
  const size_t rec = (size_t)bh * g.NG + grp;
  const int e = lane, T = e >> 4, r = e & 15;
  uint32_t* hi = (uint32_t*)c.k_hi + rec * 32;
  uint32_t* lo = (uint32_t*)((uint8_t*)c.k_lo + rec * g.klo_bytes);
  uint2 lw[4];
#pragma unroll
  for (int kq = 0; kq < 4; kq++)
    lw[kq] = make_uint2(lo[((kq * 2) * 2 + T) * 16 + r], lo[((kq * 2 + 1) * 2 + T) * 16 + r]);
  uint32_t hw = hi[e];
  int d = 0;
  for (int side = 0; side < 2; side++) {  // channels j, then j + 64
    for (uint64_t m = mhi; m; m &= m - 1, d++) {
      const int ch = __ffsll((unsigned long long)m) - 1 + NPAIR * side, w = ch >> 4;
      const int pl = 2 * pos_swap(ch & 15), ph = 2 * pos_swap(d);
      // the word holding channel ch: static register choice under a uniform test
      uint32_t word = 0;
#pragma unroll
      for (int x = 0; x < 8; x++)
        if (w == x) word = (x & 1) ? lw[x >> 1].y : lw[x >> 1].x;
      const uint32_t q = shrink_4_to_2((((hw >> ph) & 3u) << 2) | ((word >> pl) & 3u));
      word = (word & ~(3u << pl)) | (q << pl);
      hw = (hw & ~(3u << ph)) | (q << ph);
#pragma unroll
      for (int x = 0; x < 8; x++)
        if (w == x) {
          if (x & 1)
            lw[x >> 1].y = word;
          else
            lw[x >> 1].x = word;
        }
    }
  }
#pragma unroll
  for (int kq = 0; kq < 4; kq++) {
    lo[((kq * 2) * 2 + T) * 16 + r] = lw[kq].x;
    lo[((kq * 2 + 1) * 2 + T) * 16 + r] = lw[kq].y;
  }
  hi[e] = hw;
}

hipError_t launch_shrink(const Geo& g, kvq_cache* c, int g0, int g1, hipStream_t st) {
  g1 = min(g1, g.NG);
  if (g1 <= g0 || g.nh == 0 || g.NG == 0) return hipSuccess;
  hipLaunchKernelGGL(shrink_kernel, dim3(g.B * g.Hkv, (g1 - g0 + SHRINK_WAVES - 1) / SHRINK_WAVES),
                     dim3(64 * SHRINK_WAVES), 0, st, g, *c, g0, g1);
  return hipGetLastError();
}

hipError_t launch_append(const Geo& g, const void* k_new, const void* v_new, kvq_cache* c,
                         hipStream_t st) {
  const auto kern = g.bf16 ? append_variant<true>(g) : append_variant<false>(g);
  hipLaunchKernelGGL(kern, dim3(g.B * g.Hkv), dim3(128), 0, st, g, (const uint16_t*)k_new,
                     (const uint16_t*)v_new, *c);
  return hipGetLastError();
}

}  // namespace kvq
