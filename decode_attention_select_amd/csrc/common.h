// common.h — shared definitions of libkvq's HIP sources (gfx950 only).
//
// Byte layout of the cache (the contract with every caller) is documented in
// include/kvq.h; the helpers below compute its indices.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int D = 128;     // head dim
constexpr int NPAIR = 64;  // RoPE pairs: pair j = channels j, j + 64
constexpr int GS = 32;     // group: 32 tokens (keys) or 32 channels (values)
constexpr int GROUP_WORDS = 256;  // u32 words of k_lo / v_codes per group

// Shape and bit allocation, resolved on the host and passed by value.
struct Geo {
  int B, Hq, Hkv, G;
  int R, RS;           // residual tokens, ring slots (R + 32)
  int NG;              // quantized-group capacity per (b, kv head)
  int n_hi, bits_hi;   // salient pairs and their bits (4 or 16)
  int n_lo1;           // lowest-ranked pairs kept at 1 bit
  int nh;              // salient channels = 2 * n_hi
  int bf16;            // io dtype is bfloat16
  int max_tokens;
  int khi_bytes;       // bytes of the salient section per group
  int n_vhi, bits_vhi; // value blocks at the higher precision, their bits
  int vhi_words;       // u32 words of a group's v_hi record (0 when n_vhi == 0)
  int w8, w4;          // progressive precision: groups younger than w8 at 8 bits,
                       // younger than w4 at 4 or more (w4 == 0: off)
  int npl;             // digit-plane slots per (b, kv head): w4 + 2 w8
  int dense1;          // the dense 1-bit layout (n_hi == 0, n_lo1 == 32): k_lo in plane order
  int klo_bytes;       // bytes of a group's k_lo record: 768 dense, else 1024
};

// Bit of run channel c (0..15) in a 1-bit word of the dense layout, tile
// half 0 (half 1: + 16): the nibble masks (w >> i) & 0x11111111, i = 0..3,
// then deliver the run's channels in order through the fp4 converts.
__host__ __device__ inline int onebit_pos(int c) {
  return 4 * (c & 1) + ((c >> 1) & 1) + 8 * ((c >> 2) & 1) + 2 * (c >> 3);
}

// A uniform read of memory that nothing writes while the reading kernel
// runs (lengths, rank tables), through the constant address space, so that
// it becomes a scalar load: a vector load of it would be waited for (with a
// vmcnt count) while the kernel's direct global->LDS copies are in flight,
// and the compiler then waits for every copy.
__device__ inline int32_t load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Bits of a progressive group of age a (0 = the newest quantized group).
__host__ __device__ inline int prog_width(int a, int w8, int w4) {
  return a < w8 ? 8 : (a < w4 ? 4 : 2);
}

// The equivalent right shift: a 2b-bit code X on the b-bit grid of step
// s (2^b + 1), round(X / (2^b + 1)) = ((2^2b - 2^b + 1)(X + 2^(b-1))) >> 3b.
__host__ __device__ inline uint32_t ers4(uint32_t x) { return (241u * (x + 8u)) >> 12; }
__host__ __device__ inline uint32_t ers2(uint32_t x) { return (13u * (x + 2u)) >> 6; }

// Quantized tokens for T held tokens: 32 * floor(max(0, T - R) / 32).
__host__ __device__ inline int n_quant(int T, int R) {
  int over = T - R;
  return over > 0 ? (over / GS) * GS : 0;
}

// Record index e = 16*T + r inside a group holds token 8*(r/4) + 4*T + r%4.
__host__ __device__ inline int tile_token(int e) {
  int T = e >> 4, r = e & 15;
  return 8 * (r >> 2) + 4 * T + (r & 3);
}

// Code position of element c: bits 0 and 1 of c exchanged.  With that order
// the nibble split (w & 0x33333333, (w >> 2) & 0x33333333) of a word yields
// adjacent element pairs in each byte.
__host__ __device__ inline int pos_swap(int c) {
  return (c & ~3) | ((c & 1) << 1) | ((c >> 1) & 1);
}

// 16-bit input -> fp32 (exact for both dtypes).
__device__ inline float in_to_f32(uint16_t bits, int bf16) {
  if (bf16) return __uint_as_float((uint32_t)bits << 16);
  return (float)__builtin_bit_cast(_Float16, bits);
}

// fp32 -> fp16 bits, round to nearest even.
__device__ inline uint16_t f32_to_half_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ inline float half_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Affine min/max quantizer of one group of 32 values (exact fp32 widenings of
// 16-bit inputs) at L = 2^b - 1 levels:
//   z = fp16(min);  s = fp16((max - z) / L), 0 when max - z <= 0;
//   code = clamp(rint((x - z) * (1/s)), 0, L), all 0 when s == 0.
// Every step is one IEEE fp32 operation (correctly rounded division and
// rint, ties to even), so results are bit-identical to any IEEE
// implementation of the same steps.
__device__ inline void quantize_group(const float (&x)[GS], int L,
                                      uint16_t& s_bits, uint16_t& z_bits,
                                      uint8_t (&codes)[GS]) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < GS; i++) {
    mn = x[i] < mn ? x[i] : mn;
    mx = x[i] > mx ? x[i] : mx;
  }
  z_bits = f32_to_half_bits(mn);
  const float z = half_bits_to_f32(z_bits);
  const float diff = __fsub_rn(mx, z);
  s_bits = diff > 0.0f ? f32_to_half_bits(__fdiv_rn(diff, (float)L)) : (uint16_t)0;
  if (s_bits == 0) {
#pragma unroll
    for (int i = 0; i < GS; i++) codes[i] = 0;
    return;
  }
  const float r = __fdiv_rn(1.0f, half_bits_to_f32(s_bits));
#pragma unroll
  for (int i = 0; i < GS; i++) {
    float q = rintf(__fmul_rn(__fsub_rn(x[i], z), r));
    q = q < 0.0f ? 0.0f : q;
    q = q > (float)L ? (float)L : q;
    codes[i] = (uint8_t)q;
  }
}

}  // namespace kvq
