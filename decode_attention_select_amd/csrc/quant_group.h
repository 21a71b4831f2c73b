// quant_group.h — device code that quantizes and packs one 32-token group
// of a (sequence, KV head): its keys in one wave, its values in another.
// Shared by the prefill and append kernels (quant.hip) and by the decode
// kernel's append step (decode.hip); see quant.hip for the lane layouts.
#pragma once
#include "common.h"

namespace kvq {

// ------------------------------------------------------------ lane exchange

template <int CTRL>
__device__ inline uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>  // row_* controls (rotations within a 16-lane row)
__device__ inline uint32_t dpp_row(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
constexpr int QUAD_XOR1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int QUAD_XOR2 = 0x4E;  // quad_perm [2, 3, 0, 1]
template <int K>
struct QuadBcast {  // quad_perm [K, K, K, K]
  static constexpr int ctrl = K | (K << 2) | (K << 4) | (K << 6);
};
template <int K>
__device__ inline uint32_t quad_bcast(uint32_t x) { return dpp<QuadBcast<K>::ctrl>(x); }

// min and max over the quad (inputs are finite).  The result is the quad's
// min/max value; only the sign of a zero minimum depends on the combining
// order and on how the min instruction orders -0 and +0, and the caller
// settles that separately (sign_of_first_zero).
// One VALU instruction per step: the min/max reads the partner lane through
// its DPP source operand (written directly, since the compiler would add a
// copy and a NaN-quieting max around a separate DPP move).  s_nop 1 covers
// the wait states between a VALU write and a DPP read of the same register.
#define KVQ_QUAD_OP(name, op)                                                      \
  __device__ inline float name(float v) {                                          \
    float t, r;                                                                    \
    asm("s_nop 1\n\t" op "_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" \
        : "=&v"(t) : "v"(v));                                                      \
    asm("s_nop 1\n\t" op "_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" \
        : "=&v"(r) : "v"(t));                                                      \
    return r;                                                                      \
  }
KVQ_QUAD_OP(quad_min, "v_min_f32")
KVQ_QUAD_OP(quad_max, "v_max_f32")
#undef KVQ_QUAD_OP

// A sequential scan keeps the first of equal minima, so a minimum of zero
// carries the sign of the group's first zero element.  f = this lane's
// first zero in its eight elements (0: +0, 1: -0, 2: none), lanes of the
// quad in element order; returns the sign bit of the quad's first zero.
__device__ inline uint32_t sign_of_first_zero(uint32_t f) {
  const uint32_t f0 = quad_bcast<0>(f), f1 = quad_bcast<1>(f), f2 = quad_bcast<2>(f),
                 f3 = quad_bcast<3>(f);
  const uint32_t s = f0 != 2 ? f0 : f1 != 2 ? f1 : f2 != 2 ? f2 : f3;
  return s == 1 ? 0x80000000u : 0u;
}

// 16-bit element e (0..7) of a 16-byte row chunk, widened to fp32.
__device__ inline uint16_t half_of(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFF);
}

// Affine parameters of one group at L levels (the quantizer of common.h):
// z = fp16(min), s = fp16((max - z) / L) or 0, r = 1 / s (0 when s == 0).
struct QParam {
  uint32_t sz;  // s bits | z bits << 16
  float r;
};
__device__ inline QParam qparam(float mn, float mx, float L, bool raw) {
  if (raw) return {0u, 0.0f};
  const uint16_t zb = f32_to_half_bits(mn);
  const float diff = __fsub_rn(mx, half_bits_to_f32(zb));
  const uint16_t sb = diff > 0.0f ? f32_to_half_bits(__fdiv_rn(diff, L)) : (uint16_t)0;
  const float r = sb ? __fdiv_rn(1.0f, half_bits_to_f32(sb)) : 0.0f;
  return {(uint32_t)sb | ((uint32_t)zb << 16), r};
}

// code = clamp(rint((x - z) * r), 0, L) as an integer-valued float; 0 when
// r == 0 (s == 0).  Inputs are finite 16-bit values within the fp16 range of
// the scale and zero, so the product is never NaN.
__device__ inline float qcode(float x, float z, float r, float L) {
  const float q = rintf(__fmul_rn(__fsub_rn(x, z), r));
  return __builtin_amdgcn_fmed3f(q, 0.0f, L);
}

// Marks the loaded words as changed, so that widened copies made before are
// not kept alive in registers (widening again costs one instruction each).
__device__ inline void refresh(uint4 (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; i++)
    asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
}

// Compiler barrier for LDS traffic between lanes of one wave (the hardware
// runs a wave's LDS instructions in order).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bit j set when pair j has rank < n_hi (salient), rank >= 64 - n_lo1 (one bit).
struct PairMasks {
  uint64_t hi, one;
};
// The ranks are read in fixed-size blocks (wave-uniform scalar loads, all in
// flight together) rather than one dependent load per rank.
__device__ inline PairMasks pair_masks(const Geo& g, const int32_t* pr) {
  uint64_t hi = 0, one = 0;
  int p[8];
#pragma unroll
  for (int r = 0; r < 8; r++) p[r] = pr[r];  // n_hi <= 8
#pragma unroll
  for (int r = 0; r < 8; r++)
    if (r < g.n_hi) hi |= 1ull << (p[r] & (NPAIR - 1));
  if (g.n_lo1) {
    int t[NPAIR];
#pragma unroll
    for (int r = 0; r < NPAIR; r++) t[r] = pr[r];
#pragma unroll
    for (int r = 0; r < NPAIR; r++)
      if (r >= NPAIR - g.n_lo1) one |= 1ull << (t[r] & (NPAIR - 1));
  }
  return {hi, one};
}

// ------------------------------------------------------------- key group

struct KeyLds {  // one wave's staging of a key-group record
  union {
    struct {
      uint32_t lo[GROUP_WORDS];
      uint32_t hi[256];  // 4-bit: 32 words; raw 16-bit: 32 tokens x up to 16 halves
      uint32_t pl[3][GROUP_WORDS];  // progressive: digit planes 1..3
    };
    // two value precisions, before the record is staged: the group's 32 key
    // rows (16-byte pieces [row][cb]), then the partial scores [4][32]
    uint32_t tile[GS * 16 * 4 + 4 * GS];
  };
  uint32_t ord[8];  // two value precisions: the group's order bytes (slot -> position)
};

// Token order of one group for two value precisions by token (the SemKV
// reading documented in include/kvq.h at v_hi): token t's key magnitude
// E_t = sum over the 128 channels of min(floor(4096 |k|), 2^20) (integer, at
// most 2^27), and slot rank(t) = the number of tokens with larger E or equal
// E and lower position.  rows: token 0 of the group, row stride D.  Lanes
// 2t and 2t+1 sum the two channel halves of token t; every lane then ranks
// its token against the 32 sums read back from lanes 2a.  Writes order
// bytes (ord[rank(t)] = t) to LDS; the caller syncs before reading them.
template <bool BF>
__device__ inline uint32_t key_score(const uint4& v) {  // 8 channels of one token
  uint32_t e = 0;
#pragma unroll
  for (int k = 0; k < 8; k++)  // 4096 |x| is exact; the conversion truncates
    e += (uint32_t)fminf(4096.0f * fabsf(in_to_f32(half_of(v, k), BF)), 1048576.0f);
  return e;
}

// Writes ord[rank(t)] = t for the token whose score e lanes t < 32 hold.
__device__ inline void order_from_scores(uint32_t e, uint32_t* ord) {
  const int lane = threadIdx.x & 63;
  uint32_t rank = 0;
#pragma unroll
  for (int a = 0; a < GS; a++) {
    const uint32_t ea = __builtin_amdgcn_readlane(e, a);
    rank += (ea > e) || (ea == e && a < lane);
  }
  if (lane < GS) ((uint8_t*)ord)[rank] = (uint8_t)lane;
}

template <bool BF>
__device__ __forceinline__ void token_order_wave(const uint16_t* rows, uint32_t* ord) {
  const int lane = threadIdx.x & 63, t = lane >> 1, h = lane & 1;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = *(const uint4*)(rows + (size_t)t * D + 64 * h + 8 * i);
  uint32_t e = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) e += key_score<BF>(v[i]);
  e += dpp<QUAD_XOR1>(e);
  // token t's score to lane t
  e = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((2 * lane) & 63), (int)e);
  order_from_scores(e, ord);
}

// rows: token 0 of the group, row stride D (prefill input or ring_k slots).
// VHI: the wave first ranks the group's tokens (token_order_wave's scores,
// summed from the rows it holds), writes the order bytes to L.ord and takes
// the rows in that order through the LDS tile, so the record's token index
// is the slot (slot i = position L.ord[i]).
// width > 0 (progressive precision, not with VHI): every quantized channel
// is quantized at 8 bits, then shrunk to `width` bits (8, 4 or 2; salient
// 4-bit channels stop at 4) by the equivalent right shift, its step
// multiplied by 17, then 5, each product rounded to fp16; digit 0 goes to
// lo_out, digit 1 of salient channels to hi_out, digit 1 of every channel to
// pl1 (width >= 4) and digits 2, 3 to pl23 and pl23 + 256 (width 8).
// DENSE / PROG false compile the dense one-bit record / progressive
// precision out (width is then taken as 0), for callers whose layouts never
// take them.
template <bool BF, bool VHI, bool DENSE, bool PROG>
__device__ __forceinline__ void key_group_wave(const Geo& g, const uint16_t* rows, PairMasks pm,
                                               uint32_t* lo_out, uint8_t* hi_out,
                                               uint16_t* meta_out, KeyLds& L, int width = 0,
                                               uint32_t* pl1 = nullptr, uint32_t* pl23 = nullptr) {
  if (!PROG) width = 0;
  const int lane = threadIdx.x & 63, cb = lane >> 2, tq = lane & 3;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = *(const uint4*)(rows + (size_t)(8 * tq + i) * D + 8 * cb);
  // positions of the lane's slots 8tq .. 8tq+7, one byte each
  uint2 pos = make_uint2(0, 0);
  if constexpr (VHI) {
    uint4* tile = (uint4*)L.tile;
    uint32_t* rs = L.tile + GS * 16 * 4;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      // the lane's 8 channels, then the 4 channel blocks of its DPP row
      uint32_t e = key_score<BF>(v[i]);
      e += dpp_row<0x124>(e);  // row_ror:4 (same tq, next cb)
      e += dpp_row<0x128>(e);  // row_ror:8
      if ((cb & 3) == 0) rs[(cb >> 2) * GS + 8 * tq + i] = e;
      tile[(8 * tq + i) * 16 + cb] = v[i];
    }
    wave_lds_sync();
    const int t = lane & (GS - 1);
    order_from_scores(rs[t] + rs[GS + t] + rs[2 * GS + t] + rs[3 * GS + t], L.ord);
    wave_lds_sync();
    pos = ((const uint2*)L.ord)[tq];
  }
  auto pos_of = [&](int i) -> uint32_t {
    if constexpr (VHI) return ((i < 4 ? pos.x : pos.y) >> (8 * (i & 3))) & 0xFFu;
    return 8 * tq + i;
  };
  if constexpr (VHI) {
    const uint4* tile = (const uint4*)L.tile;
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = tile[pos_of(i) * 16 + cb];
    wave_lds_sync();  // the tile's space is reused for the record below
  }

  const bool bits4 = g.nh > 0 && g.bits_hi == 4, raw16 = g.nh > 0 && g.bits_hi == 16;
  // bit allocation of the lane's channels 8cb + k
  float lv[8];
  bool raw[8];
  int hish[8], dix[8];
  // the lane's 8 channels are the consecutive pair ids j0 .. j0+7
  const int j0 = (8 * cb) & (NPAIR - 1);
  const uint32_t hib = (uint32_t)(pm.hi >> j0) & 0xFFu, oneb = (uint32_t)(pm.one >> j0) & 0xFFu;
  const int dbase = __popcll(pm.hi & ((1ull << j0) - 1)) + (8 * cb >= NPAIR ? g.n_hi : 0);
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const bool sal = (hib >> k) & 1u, one = (oneb >> k) & 1u;
    dix[k] = dbase + __popc(hib & ((1u << k) - 1u));
    raw[k] = sal && g.bits_hi == 16;
    lv[k] = width > 0 ? 255.0f : (sal ? 15.0f : (one ? 1.0f : 3.0f));
    hish[k] = sal ? 2 * pos_swap(dix[k]) : 0;
  }
  // per-channel min / max over the 32 tokens
  float mn[8], mx[8];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    float a = in_to_f32(half_of(v[0], k), BF), b = a;
#pragma unroll
    for (int i = 1; i < 8; i += 2) {  // three-input min / max
      const float x = in_to_f32(half_of(v[i], k), BF);
      const float y = i + 1 < 8 ? in_to_f32(half_of(v[i + 1], k), BF) : x;
      a = fminf(a, fminf(x, y));
      b = fmaxf(b, fmaxf(x, y));
    }
    mn[k] = quad_min(a);
    mx[k] = quad_max(b);
  }
  bool zmin = false;
#pragma unroll
  for (int k = 0; k < 8; k++) zmin |= mn[k] == 0.0f;
  if (__any(zmin)) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      if constexpr (VHI) {
        // the first zero by position: smallest 2 * position + sign bit
        uint32_t f = 0xFFFFu;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float x = in_to_f32(half_of(v[i], k), BF);
          if (x == 0.0f) f = min(f, 2 * pos_of(i) + (__float_as_uint(x) >> 31));
        }
        f = min(f, dpp<QUAD_XOR1>(f));
        f = min(f, dpp<QUAD_XOR2>(f));
        if (mn[k] == 0.0f) mn[k] = __uint_as_float((f & 1u) << 31);
      } else {
        uint32_t f = 2;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float x = in_to_f32(half_of(v[i], k), BF);
          if (f == 2 && x == 0.0f) f = __float_as_uint(x) >> 31;
        }
        const uint32_t sgn = sign_of_first_zero(f);
        if (mn[k] == 0.0f) mn[k] = __uint_as_float(sgn);
      }
    }
  }
  // lane tq computes channels 2tq and 2tq+1 of the quad's eight
  auto pick = [&](const float (&a)[8], int o) {
    return tq == 0 ? a[o] : tq == 1 ? a[2 + o] : tq == 2 ? a[4 + o] : a[6 + o];
  };
  auto pickb = [&](const bool (&a)[8], int o) {
    return tq == 0 ? a[o] : tq == 1 ? a[2 + o] : tq == 2 ? a[4 + o] : a[6 + o];
  };
  const QParam p0 = qparam(pick(mn, 0), pick(mx, 0), pick(lv, 0), pickb(raw, 0));
  const QParam p1 = qparam(pick(mn, 1), pick(mx, 1), pick(lv, 1), pickb(raw, 1));
  uint32_t sz[8];
  float rr[8];
#define KVQ_BCAST(K)                                                              \
  sz[2 * K] = quad_bcast<K>(p0.sz);                                              \
  sz[2 * K + 1] = quad_bcast<K>(p1.sz);                                          \
  rr[2 * K] = __uint_as_float(quad_bcast<K>(__float_as_uint(p0.r)));             \
  rr[2 * K + 1] = __uint_as_float(quad_bcast<K>(__float_as_uint(p1.r)));
  KVQ_BCAST(0) KVQ_BCAST(1) KVQ_BCAST(2) KVQ_BCAST(3)
#undef KVQ_BCAST

  // codes: low digits summed into half-words as exact float integers
  // (digit * 4^position, below 2^16); the high digits of 4-bit channels as
  // integers, only for channel slots k where some lane holds a 4-bit channel
  refresh(v);
  if (DENSE && g.dense1 && width == 0) {
    // the dense 1-bit layout: channel c goes to plane run 2 kq' + u (u = 1
    // for a 1-bit pair), place cc = rank % 16, where rank counts the
    // channels of its class below it (first channels, then second ones)
    if (lane < 48) ((uint4*)L.lo)[lane] = make_uint4(0, 0, 0, 0);
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int c = 8 * cb + k, j = c & (NPAIR - 1);
      const bool one = (pm.one >> j) & 1ull;
      const uint64_t below = j ? (~0ull >> (64 - j)) : 0ull;
      const int rank = 32 * (c >> 6) + __popcll((one ? pm.one : ~pm.one) & below);
      const int kqp = rank >> 4, cc = rank & 15;
      const float z = half_bits_to_f32((uint16_t)(sz[k] >> 16));
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t code = (uint32_t)qcode(in_to_f32(half_of(v[i], k), BF), z, rr[k], lv[k]);
        const int T = i >> 2, r = 4 * tq + (i & 3);
        if (one) {  // word kq' * 16 + r, tile half T in bits 16 T ..
          if (code) atomicOr(&L.lo[128 + kqp * 16 + r], code << (onebit_pos(cc) + 16 * T));
        } else if (code) {
          atomicOr(&L.lo[(kqp * 2 + T) * 16 + r], code << (2 * pos_swap(cc)));
        }
      }
      if (tq < 2)  // run 2 kq' + u: 16 scales (tq 0), then 16 zeros (tq 1)
        meta_out[(2 * kqp + (one ? 1 : 0)) * 32 + tq * 16 + cc] =
            (uint16_t)(tq == 0 ? sz[k] & 0xFFFFu : sz[k] >> 16);
    }
    wave_lds_sync();
    if (lane < 48) ((uint4*)lo_out)[lane] = ((const uint4*)L.lo)[lane];
    return;
  }
  float hwf[8];
  uint32_t hw[8], hh[8];
  uint32_t pw[3][8];  // progressive: digits 1..3 (half-words like hw)
#pragma unroll
  for (int i = 0; i < 8; i++) {
    hwf[i] = 0.0f;
    hh[i] = 0;
    pw[0][i] = pw[1][i] = pw[2][i] = 0;
  }
  if (width > 0) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const float z = half_bits_to_f32((uint16_t)(sz[k] >> 16));
      const int sh = 2 * pos_swap(k);
      const bool salk = (hib >> k) & 1u;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        uint32_t X = (uint32_t)qcode(in_to_f32(half_of(v[i], k), BF), z, rr[k], 255.0f);
        if (width <= 4) X = ers4(X);
        if (width == 2 && !salk) X = ers2(X);
        hwf[i] += (float)((X & 3u) << sh);
        pw[0][i] |= ((X >> 2) & 3u) << sh;
        pw[1][i] |= ((X >> 4) & 3u) << sh;
        pw[2][i] |= (X >> 6) << sh;
        if (bits4 && salk) hh[i] |= ((X >> 2) & 3u) << hish[k];
      }
      // the steps of the shrinks, each rounded once to fp16
      uint32_t sb = sz[k] & 0xFFFFu;
      if (width <= 4) sb = f32_to_half_bits(half_bits_to_f32((uint16_t)sb) * 17.0f);
      if (width == 2 && !salk) sb = f32_to_half_bits(half_bits_to_f32((uint16_t)sb) * 5.0f);
      sz[k] = (sz[k] & 0xFFFF0000u) | sb;
    }
  }
#pragma unroll
  for (int k = 0; k < 8; k++) {
    if (width > 0) break;
    const float z = half_bits_to_f32((uint16_t)(sz[k] >> 16));
    const float mul = (float)(1u << (2 * pos_swap(k)));
    if (bits4 && __any(lv[k] == 15.0f)) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float q = qcode(in_to_f32(half_of(v[i], k), BF), z, rr[k], lv[k]);
        const float hd = floorf(q * 0.25f), ld = fmaf(hd, -4.0f, q);
        hwf[i] = fmaf(ld, mul, hwf[i]);
        hh[i] |= (uint32_t)hd << hish[k];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++)
        hwf[i] = fmaf(qcode(in_to_f32(half_of(v[i], k), BF), z, rr[k], lv[k]), mul, hwf[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; i++) hw[i] = (uint32_t)hwf[i];
  // stage the record in LDS: token i of this lane is tile index
  // e = 16 T + r with T = i / 4, r = 4 tq + i % 4
  if (lane < 8) ((uint4*)L.hi)[lane] = make_uint4(0, 0, 0, 0);
  wave_lds_sync();
  const int w = cb >> 1, kq = w >> 1, u = w & 1, half = cb & 1;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int T = i >> 2, r = 4 * tq + (i & 3);
    const int hx = (((kq * 2 + u) * 2 + T) * 16 + r) * 2 + half;
    ((uint16_t*)L.lo)[hx] = (uint16_t)hw[i];
    if (bits4 && hh[i]) atomicOr(&L.hi[16 * T + r], hh[i]);
    if (width >= 4) ((uint16_t*)L.pl[0])[hx] = (uint16_t)pw[0][i];
    if (width == 8) {
      ((uint16_t*)L.pl[1])[hx] = (uint16_t)pw[1][i];
      ((uint16_t*)L.pl[2])[hx] = (uint16_t)pw[2][i];
    }
  }
  if (raw16) {
#pragma unroll
    for (int k = 0; k < 8; k++)
      if (raw[k]) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const int e = 16 * (i >> 2) + 4 * tq + (i & 3);
          ((uint16_t*)L.hi)[e * g.nh + dix[k]] = half_of(v[i], k);
        }
      }
  }
  wave_lds_sync();
  ((uint4*)lo_out)[lane] = ((const uint4*)L.lo)[lane];
  if (lane < g.khi_bytes / 16) ((uint4*)hi_out)[lane] = ((const uint4*)L.hi)[lane];
  if (width >= 4) ((uint4*)pl1)[lane] = ((const uint4*)L.pl[0])[lane];
  if (width == 8) {
    ((uint4*)pl23)[lane] = ((const uint4*)L.pl[1])[lane];
    ((uint4*)pl23)[64 + lane] = ((const uint4*)L.pl[2])[lane];
  }
  if (tq < 2) {
    uint32_t m[4];
#pragma unroll
    for (int p = 0; p < 4; p++)
      m[p] = tq == 0 ? (sz[2 * p] & 0xFFFFu) | (sz[2 * p + 1] << 16)
                     : (sz[2 * p] >> 16) | (sz[2 * p + 1] & 0xFFFF0000u);
    // run cb / 2 of the record: its 16 scales, then its 16 zeros
    *(uint4*)(meta_out + (cb >> 1) * 32 + tq * 16 + 8 * (cb & 1)) =
        make_uint4(m[0], m[1], m[2], m[3]);
  }
}

// ----------------------------------------------------------- value group

// CHMAJOR false: src = token 0 of the group, row stride D (prefill input).
// CHMAJOR true:  src = a ring_v slot block [128][32] (channel, slot).
// VHI (g.n_vhi > 0: two value precisions by token, the SemKV reading
// documented in include/kvq.h at v_hi): pos holds the positions of the
// lane's slots 8tq .. 8tq+7 (one byte each, from the group's token order);
// slots below 8 n_vhi quantize at L = 2^bits_vhi - 1, and the high digits
// of their codes go to vhi_out (the group's v_hi record) after its 8-word
// order header, which the key side writes.
// width > 0 (progressive precision, not with VHI): codes at 8 bits, shrunk
// to `width` bits, digit planes 1..3 to pl1 / pl23, as for the keys (PROG
// false compiles that out and takes width as 0).
template <bool BF, bool CHMAJOR, bool VHI, bool PROG>
__device__ __forceinline__ void value_group_wave(const Geo& g, const uint16_t* src, uint2 pos,
                                                 uint32_t* vc_out, uint16_t* meta_out,
                                                 uint32_t* vhi_out, int width = 0,
                                                 uint32_t* pl1 = nullptr, uint32_t* pl23 = nullptr) {
  if (!PROG) width = 0;
  const int lane = threadIdx.x & 63, cb = lane & 15, tq = lane >> 4, m = cb & 3, j = cb >> 2;
  auto pos_of = [&](int i) -> uint32_t {
    return ((i < 4 ? pos.x : pos.y) >> (8 * (i & 3))) & 0xFFu;
  };
  // x(i, k): slot 8tq + i, channel 8cb + k
  uint4 v[8];
  if constexpr (VHI && CHMAJOR) {
    // the slot's token is scattered in the channel-major ring block: gather
    // 16-bit values, channel row n of the lane from the eight positions
#pragma unroll
    for (int n = 0; n < 8; n++) {
      const uint16_t* r = src + (size_t)(8 * cb + n) * GS;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; i++) w[i] = r[pos_of(2 * i)] | ((uint32_t)r[pos_of(2 * i + 1)] << 16);
      v[n] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
#pragma unroll
    for (int n = 0; n < 8; n++)
      v[n] = CHMAJOR ? *(const uint4*)(src + (size_t)(8 * cb + n) * GS + 8 * tq)
                     : *(const uint4*)(src + (size_t)(VHI ? pos_of(n) : 8 * tq + n) * D + 8 * cb);
  }
  auto x = [&](int i, int k) {
    return in_to_f32(CHMAJOR ? half_of(v[k], i) : half_of(v[i], k), BF);
  };
  float mn[8], mx[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float a = x(i, 0), b = a;
#pragma unroll
    for (int k = 1; k < 8; k += 2) {  // three-input min / max
      const float e = x(i, k), f = k + 1 < 8 ? x(i, k + 1) : e;
      a = fminf(a, fminf(e, f));
      b = fmaxf(b, fmaxf(e, f));
    }
    mn[i] = quad_min(a);
    mx[i] = quad_max(b);
  }
  bool zmin = false;
#pragma unroll
  for (int i = 0; i < 8; i++) zmin |= mn[i] == 0.0f;
  if (__any(zmin)) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      uint32_t f = 2;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const float e = x(i, k);
        if (f == 2 && e == 0.0f) f = __float_as_uint(e) >> 31;
      }
      const uint32_t sgn = sign_of_first_zero(f);
      if (mn[i] == 0.0f) mn[i] = __uint_as_float(sgn);
    }
  }
  const bool hiblk = VHI && tq < g.n_vhi;
  const float Lv = width > 0 ? 255.0f : (hiblk ? (float)((1 << g.bits_vhi) - 1) : 3.0f);
  auto pick = [&](const float (&a)[8], int o) {
    return m == 0 ? a[o] : m == 1 ? a[2 + o] : m == 2 ? a[4 + o] : a[6 + o];
  };
  const QParam p0 = qparam(pick(mn, 0), pick(mx, 0), Lv, false);
  const QParam p1 = qparam(pick(mn, 1), pick(mx, 1), Lv, false);
  uint32_t sz[8];
  float rr[8];
#define KVQ_BCAST(K)                                                              \
  sz[2 * K] = quad_bcast<K>(p0.sz);                                              \
  sz[2 * K + 1] = quad_bcast<K>(p1.sz);                                          \
  rr[2 * K] = __uint_as_float(quad_bcast<K>(__float_as_uint(p0.r)));             \
  rr[2 * K + 1] = __uint_as_float(quad_bcast<K>(__float_as_uint(p1.r)));
  KVQ_BCAST(0) KVQ_BCAST(1) KVQ_BCAST(2) KVQ_BCAST(3)
#undef KVQ_BCAST
  // half-word of channel k: its 8 tokens' codes at positions pi(i), summed
  // as exact float integers (digit * 4^position, below 2^16); codes above 3
  // (high-precision slots) split into a low digit here and a high digit in hh
  float hf[8], hhf[8];
  uint32_t h[8], hh[8];
  uint32_t pw[3][8];  // progressive: digits 1..3 (half-words like h)
#pragma unroll
  for (int k = 0; k < 8; k++) {
    hf[k] = hhf[k] = 0.0f;
    pw[0][k] = pw[1][k] = pw[2][k] = 0;
  }
  if (width > 0) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float z = half_bits_to_f32((uint16_t)(sz[i] >> 16));
      const int sh = 2 * pos_swap(i);
#pragma unroll
      for (int k = 0; k < 8; k++) {
        uint32_t X = (uint32_t)qcode(x(i, k), z, rr[i], 255.0f);
        if (width <= 4) X = ers4(X);
        if (width == 2) X = ers2(X);
        hf[k] += (float)((X & 3u) << sh);
        pw[0][k] |= ((X >> 2) & 3u) << sh;
        pw[1][k] |= ((X >> 4) & 3u) << sh;
        pw[2][k] |= (X >> 6) << sh;
      }
      uint32_t sb = sz[i] & 0xFFFFu;
      if (width <= 4) sb = f32_to_half_bits(half_bits_to_f32((uint16_t)sb) * 17.0f);
      if (width == 2) sb = f32_to_half_bits(half_bits_to_f32((uint16_t)sb) * 5.0f);
      sz[i] = (sz[i] & 0xFFFF0000u) | sb;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    if (width > 0) break;
    const float z = half_bits_to_f32((uint16_t)(sz[i] >> 16));
    const float mul = (float)(1u << (2 * pos_swap(i)));
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const float q = qcode(x(i, k), z, rr[i], Lv);
      if constexpr (VHI) {
        const float hd = floorf(q * 0.25f);
        hf[k] = fmaf(fmaf(hd, -4.0f, q), mul, hf[k]);
        hhf[k] = fmaf(hd, mul, hhf[k]);
      } else {
        hf[k] = fmaf(q, mul, hf[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; k++) {
    h[k] = (uint32_t)hf[k];
    hh[k] = (uint32_t)hhf[k];
  }
  // Word (j*4 + tq)*16 + c holds channel 32j + c (bits 0..15) and 32j+16+c
  // (bits 16..31).  Lane m holds channels 32j + 8m + k: m = 0, 1 are low
  // halves, m = 2, 3 the high halves of the same words (quad partner m ^ 2).
  // The low lane keeps words k = 0..3 of its eight, the high lane k = 4..7.
  const bool low = m < 2;
  auto words = [&](const uint32_t (&hv)[8], uint32_t (&wd)[4]) {
    const uint32_t s0 = low ? (hv[4] | (hv[5] << 16)) : (hv[0] | (hv[1] << 16));
    const uint32_t s1 = low ? (hv[6] | (hv[7] << 16)) : (hv[2] | (hv[3] << 16));
    const uint32_t r0 = dpp<QUAD_XOR2>(s0), r1 = dpp<QUAD_XOR2>(s1);
    const uint32_t o[4] = {r0 & 0xFFFFu, r0 >> 16, r1 & 0xFFFFu, r1 >> 16};
#pragma unroll
    for (int q = 0; q < 4; q++)
      wd[q] = low ? (hv[q] | (o[q] << 16)) : (o[q] | (hv[4 + q] << 16));
  };
  uint32_t wd[4];
  words(h, wd);
  const int c0 = 8 * (m & 1) + 4 * (m >> 1);
  *(uint4*)(vc_out + (j * 4 + tq) * 16 + c0) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  if (width >= 4) {
#pragma unroll
    for (int d = 0; d < 3; d++) {
      if (d > 0 && width < 8) break;
      uint32_t wp[4];
      words(pw[d], wp);
      uint32_t* dst = d == 0 ? pl1 : pl23 + (d - 1) * GROUP_WORDS;
      *(uint4*)(dst + (j * 4 + tq) * 16 + c0) = make_uint4(wp[0], wp[1], wp[2], wp[3]);
    }
  }
  if constexpr (VHI) {
    uint32_t wh[4];
    words(hh, wh);
    if (hiblk)
      *(uint4*)(vhi_out + 8 + (j * g.n_vhi + tq) * 16 + c0) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
  }
  if (m < 2) {
    uint32_t mm[4];
#pragma unroll
    for (int p = 0; p < 4; p++)
      mm[p] = m == 0 ? (sz[2 * p] & 0xFFFFu) | (sz[2 * p + 1] << 16)
                     : (sz[2 * p] >> 16) | (sz[2 * p + 1] & 0xFFFF0000u);
    *(uint4*)(meta_out + m * D + j * GS + 8 * tq) = make_uint4(mm[0], mm[1], mm[2], mm[3]);
  }
}

// ----------------------------------------------------------- shrink step

// Progressive precision: one shrink of a stored group, in place.  Each code
// X (digit d of a code: (X >> 2d) & 3; digit 0 in the record, digit 1 in
// plane pl1, digits 2 and 3 in pl23 and pl23 + 256 when from == 8) moves from
// `from` bits (8 or 4) to `to` bits (4 or 2) by the equivalent right shift,
// 8 -> 4 then 4 -> 2, and each step multiplies the scale by 17 or 5 (rounded
// to fp16, zero point kept).  The new digit 0 goes back to the record and,
// when to == 4, digit 1 back to pl1.  Word wi of a 256-word record covers 16
// codes at bit positions 2p; `chan(wi, p)` names the key channel of
// position p (salient channels stop at 4 bits) or -1 for values.  One wave;
// every read of a word is consumed before any write (so a later write of
// the same plane slot by the caller is ordered after the reads).
template <typename Chan>
__device__ inline void shrink_words(uint32_t* rec, uint32_t* pl1, const uint32_t* pl23, int from,
                                    int to, Chan sal_of, uint32_t (&np1)[4]) {
  const int lane = threadIdx.x & 63;
  uint32_t nlo[4];
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const int wi = lane + 64 * m;
    const uint32_t w0 = rec[wi], w1 = pl1[wi];
    const uint32_t w2 = from == 8 ? pl23[wi] : 0u, w3 = from == 8 ? pl23[GROUP_WORDS + wi] : 0u;
    uint32_t a = 0, b = 0;
#pragma unroll
    for (int p = 0; p < 16; p++) {
      uint32_t X = ((w0 >> (2 * p)) & 3u) | (((w1 >> (2 * p)) & 3u) << 2) |
                   (((w2 >> (2 * p)) & 3u) << 4) | (((w3 >> (2 * p)) & 3u) << 6);
      if (from == 8) X = ers4(X);
      if (to == 2 && !sal_of(wi, p)) X = ers2(X);
      a |= (X & 3u) << (2 * p);
      b |= ((X >> 2) & 3u) << (2 * p);
    }
    nlo[m] = a;
    np1[m] = b;
  }
#pragma unroll
  for (int m = 0; m < 4; m++) {
    rec[lane + 64 * m] = nlo[m];
    if (to == 4) pl1[lane + 64 * m] = np1[m];
  }
}

// The step of one quantizer after the shrink (fp16 bits).
__device__ inline uint16_t shrunk_step(uint16_t sb, int from, int to, bool stop4) {
  if (from == 8) sb = f32_to_half_bits(half_bits_to_f32(sb) * 17.0f);
  if (to == 2 && !stop4) sb = f32_to_half_bits(half_bits_to_f32(sb) * 5.0f);
  return sb;
}

// Key record of one group (lo, hi, meta) and its planes: channel 16 (wi / 32)
// + pi(p) sits at position p of word wi.  From 8 bits, the salient channels'
// new digit 1 is gathered into hi (word e: tile index e, the d-th salient
// channel at position pi(d)) through the LDS.
__device__ inline void shrink_key_group(const Geo& g, PairMasks pm, uint32_t* lo, uint8_t* hi,
                                        uint16_t* meta, uint32_t* pl1, const uint32_t* pl23,
                                        int from, int to, KeyLds& L) {
  const int lane = threadIdx.x & 63;
  auto sal_of = [&](int wi, int p) {
    const int c = 16 * (wi >> 5) + pos_swap(p);
    return ((pm.hi >> (c & (NPAIR - 1))) & 1ull) != 0;
  };
  uint32_t np1[4];
  shrink_words(lo, pl1, pl23, from, to, sal_of, np1);
#pragma unroll
  for (int h2 = 0; h2 < 2; h2++) {
    const int ch = 2 * lane + h2;
    uint16_t* sp = meta + (ch >> 4) * 32 + (ch & 15);
    *sp = shrunk_step(*sp, from, to, ((pm.hi >> (ch & (NPAIR - 1))) & 1ull) != 0);
  }
  if (from == 8 && g.nh > 0 && g.bits_hi == 4) {
#pragma unroll
    for (int m = 0; m < 4; m++) L.pl[0][lane + 64 * m] = np1[m];
    wave_lds_sync();
    if (lane < GS) {
      uint32_t hw = 0;
      uint64_t mk = pm.hi;
#pragma unroll
      for (int d = 0; d < 8; d++) {
        if (d >= g.n_hi) break;
        const int pc = __builtin_ctzll(mk);
        mk &= mk - 1;
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {  // channels pc (entry d) and pc + 64 (entry n_hi + d)
          const int c = pc + NPAIR * h2, dd = d + g.n_hi * h2;
          const uint32_t w = L.pl[0][(c >> 4) * 32 + lane];
          hw |= ((w >> (2 * pos_swap(c & 15))) & 3u) << (2 * pos_swap(dd));
        }
      }
      ((uint32_t*)hi)[lane] = hw;
    }
    wave_lds_sync();
  }
}

// Value record of one group: every code shrinks (one precision for all).
__device__ inline void shrink_value_group(uint32_t* vc, uint16_t* meta, uint32_t* pl1,
                                          const uint32_t* pl23, int from, int to) {
  const int lane = threadIdx.x & 63;
  uint32_t np1[4];
  shrink_words(vc, pl1, pl23, from, to, [](int, int) { return false; }, np1);
#pragma unroll
  for (int h2 = 0; h2 < 2; h2++) {  // scales s[j][t] at j * 32 + t
    uint16_t* sp = meta + 2 * lane + h2;
    *sp = shrunk_step(*sp, from, to, false);
  }
}

// Plane slots of group grp of (sequence, KV head) bh: digit 1 (slot grp mod
// w4) and digits 2, 3 (slots w4 + 2 (grp mod w8) and the next).
__device__ inline uint32_t* plane1(const Geo& g, uint32_t* base, int bh, int grp) {
  return base + ((size_t)bh * g.npl + grp % g.w4) * GROUP_WORDS;
}
__device__ inline uint32_t* plane23(const Geo& g, uint32_t* base, int bh, int grp) {
  return g.w8 > 0 ? base + ((size_t)bh * g.npl + g.w4 + 2 * (grp % g.w8)) * GROUP_WORDS : base;
}

// ------------------------------------------------------------ ring group

// LDS of the two waves that pack a group from the ring.
struct PackLds {
  KeyLds key;
  __align__(16) uint32_t vord[8];  // the value wave's copy of the token order
};

// Packs the group of positions [nq0, nq0 + 32) of (sequence, KV head) bh
// from the ring: threads 0..63 its keys, 64..127 its values (each a whole
// wave; other threads must not call).  With two value precisions both waves
// rank the group's tokens from the ring keys (the same integer sums, so the
// same order) and the key wave writes the order to the v_hi header.
// Progressive precision (g.w4 > 0): the new group enters at the width of
// age 0, and first the group that reaches age w4 shrinks from 4 to 2 bits and
// the one that reaches age w8 from 8 bits to the width of that age (in this
// order, each wave for its side: the new group's planes take the slots these
// two free).
// MAYPROG / MAYDENSE false compile progressive precision / the dense one-bit
// record out, for callers the host never launches with that layout.
template <bool BF, bool VHI, bool MAYPROG, bool MAYDENSE>
__device__ __forceinline__ void pack_ring_group(const Geo& g, kvq_cache& c, int bh, int nq0, int tid,
                                PackLds& lds) {
  const uint16_t* rk = (const uint16_t*)c.ring_k + (size_t)bh * g.RS * D;
  const uint16_t* rv = (const uint16_t*)c.ring_v + (size_t)bh * g.RS * D;
  const int grp = nq0 / GS, s0 = nq0 % g.RS;
  const size_t rec = (size_t)bh * g.NG + grp;
  uint32_t* vhi = c.v_hi + rec * g.vhi_words;
  const int width = MAYPROG && g.w4 > 0 ? prog_width(0, g.w8, g.w4) : 0;
  const int gA = grp - g.w4, gB = grp - g.w8;
  const bool shrinkA = MAYPROG && g.w4 > g.w8 && gA >= 0;
  const bool shrinkB = MAYPROG && g.w4 > 0 && g.w8 > 0 && gB >= 0;
  const int toB = shrinkB ? prog_width(g.w8, g.w8, g.w4) : 0;
  if (tid < 64) {
    const PairMasks pm = pair_masks(g, c.pairs + (size_t)bh * NPAIR);
    uint32_t* kpl = c.k_pl;
    if (shrinkA) {
      const size_t ra = (size_t)bh * g.NG + gA;
      shrink_key_group(g, pm, (uint32_t*)c.k_lo + ra * GROUP_WORDS, (uint8_t*)c.k_hi + ra * g.khi_bytes,
                       (uint16_t*)c.k_meta + ra * 2 * D, plane1(g, kpl, bh, gA),
                       plane23(g, kpl, bh, gA), 4, 2, lds.key);
    }
    if (shrinkB) {
      const size_t rb = (size_t)bh * g.NG + gB;
      shrink_key_group(g, pm, (uint32_t*)c.k_lo + rb * GROUP_WORDS, (uint8_t*)c.k_hi + rb * g.khi_bytes,
                       (uint16_t*)c.k_meta + rb * 2 * D, plane1(g, kpl, bh, gB),
                       plane23(g, kpl, bh, gB), 8, toB, lds.key);
    }
    key_group_wave<BF, VHI, MAYDENSE, MAYPROG>(g, rk + (size_t)s0 * D, pm,
                            (uint32_t*)((uint8_t*)c.k_lo + rec * g.klo_bytes),
                            (uint8_t*)c.k_hi + rec * g.khi_bytes,
                            (uint16_t*)c.k_meta + rec * 2 * D, lds.key, width,
                            width ? plane1(g, kpl, bh, grp) : nullptr,
                            width ? plane23(g, kpl, bh, grp) : nullptr);
    if constexpr (VHI)
      if (tid < 2) ((uint4*)vhi)[tid] = ((const uint4*)lds.key.ord)[tid];
  } else {
    uint2 pos = make_uint2(0, 0);
    if constexpr (VHI) {
      token_order_wave<BF>(rk + (size_t)s0 * D, lds.vord);
      wave_lds_sync();
      pos = ((const uint2*)lds.vord)[((tid & 63) >> 4)];
    }
    uint32_t* vpl = c.v_pl;
    if (shrinkA) {
      const size_t ra = (size_t)bh * g.NG + gA;
      shrink_value_group((uint32_t*)c.v_codes + ra * GROUP_WORDS, (uint16_t*)c.v_meta + ra * 2 * D,
                         plane1(g, vpl, bh, gA), plane23(g, vpl, bh, gA), 4, 2);
    }
    if (shrinkB) {
      const size_t rb = (size_t)bh * g.NG + gB;
      shrink_value_group((uint32_t*)c.v_codes + rb * GROUP_WORDS, (uint16_t*)c.v_meta + rb * 2 * D,
                         plane1(g, vpl, bh, gB), plane23(g, vpl, bh, gB), 8, toB);
    }
    value_group_wave<BF, true, VHI, MAYPROG>(g, rv + (size_t)(s0 / GS) * D * GS, pos,
                                    (uint32_t*)c.v_codes + rec * GROUP_WORDS,
                                    (uint16_t*)c.v_meta + rec * 2 * D, vhi, width,
                                    width ? plane1(g, vpl, bh, grp) : nullptr,
                                    width ? plane23(g, vpl, bh, grp) : nullptr);
  }
}

}  // namespace kvq
