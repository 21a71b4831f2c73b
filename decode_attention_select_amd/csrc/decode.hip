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
// nibble is the e2m1 value code/2), accumulation is fp32.  The products q*s
// and p*s enter as an exact pair of fp16 operands, hi = fp16(x*y) and
// lo = fp16(x*y - hi) (one fused multiply-add; the residual of a product of
// two fp16 values is itself an fp16 value), each through its own MFMA into
// the same accumulator, so no product is rounded: the only roundings left
// are the fp16 softmax weights (the same rounded weights feed the numerator
// and the denominator) and fp32 accumulation.  The z terms are one more MFMA
// each (fp16 x fp16 products are exact in fp32); an extra all-ones row in the
// value-zero MFMA yields the softmax denominator from the same rounded p.
// Query heads of one KV head fill the 16 MFMA columns (G <= 16).  Ring
// (16-bit) tokens use the same MFMA shapes on raw values.  The salient keys'
// high digits weigh 4*q*s, split the same way and carried by the otherwise
// unused K-lanes 16..31 of that MFMA.
//
// Work split: an 8-wave workgroup per (sequence, KV head, token split), one
// workgroup per CU by default.  Wave w of split s owns the flat index
// f = s + S w of its (sequence, KV head); f < RS/32 also owns physical ring
// block f (32 ring slots), and the 32-token groups g = f - RS/32 + i S NW
// (i >= 0, g >= 0) are its quantized groups.  Every address a wave reads is
// fixed before the length arrives, so each wave issues all its first loads at
// entry: the query, its ring block (to registers) and its first quantized
// groups, copied straight from HBM into per-wave LDS slots by direct
// global->LDS loads (each slot one group's records; a consumed slot is
// refilled with the wave's next group).  The record in work is read from its
// slot, the 16 lanes sharing a channel slice reading the metadata as a
// broadcast.  Each wave keeps its own online softmax (base 2, scale folded
// into the exponent; the running max is raised only when a block's weights
// would exceed 2^8, or 2 in a group with very wide value scales, so most
// blocks skip the rescale and the fp16 products of weights and value scales
// stay finite).  The waves merge in LDS into one record per head (m, l, o/l,
// fp32); the last workgroups of a (sequence, KV head) to finish (atomic
// counter) merge the split records with the log-sum-exp rule, each a share of
// the heads' channels, and write the output.  The fused variant also carries
// the step's append (see FUSED at the kernel).
#include "common.h"
#include "internal.h"
#include "quant_group.h"
#include "stream.h"

#ifndef KVQ_DECODE_PART
#define KVQ_DECODE_PART 1
#endif

namespace kvq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
// 16 bytes at a 4-byte-aligned address (raw salient rows are 2*nh bytes long)
typedef uint32_t u4a __attribute__((ext_vector_type(4), aligned(4)));

constexpr int MAXG = 16;
// log2 headroom before the running max moves: the softmax weights p stay
// below 2^slack.  The value path forms p * s in fp16, so a group holding a
// value scale above 65504 / 2^8 (fp16 bits 0x5BFF) takes the slack 1 (p <= 2,
// finite for every scale up to 65504 / 3); all other groups take 8, so that
// most blocks skip the rescale.
constexpr float RESCALE_SLACK = 8.0f;
constexpr float RESCALE_SLACK_WIDE = 1.0f;
constexpr uint32_t VSCALE_WIDE = 0x5BFFu;

__device__ inline uint32_t h2u(h2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ inline h2 u2h(uint32_t x) { return __builtin_bit_cast(h2, x); }
__device__ inline uint32_t pk_mul(uint32_t a, uint32_t b) { return h2u(u2h(a) * u2h(b)); }
// fp32 pair -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32)
__device__ inline uint32_t pk_rne(float a, float b) { return h2u(h2{(_Float16)a, (_Float16)b}); }
__device__ inline float ex2(float x) { return __builtin_amdgcn_exp2f(x); }


// 16-bit input pair -> fp16 pair (bf16 widened exactly, then RNE to fp16)
template <bool BF16>
__device__ inline uint32_t to_f16_pair(uint32_t w) {
  if constexpr (!BF16) return w;
  return pk_rne(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// fp32 -> the io dtype, round to nearest even (bf16: finite values)
template <bool BF16>
__device__ inline uint16_t to_io_bits(float v) {
  if constexpr (BF16) {
    const uint32_t u = __float_as_uint(v);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  } else {
    return f32_to_half_bits(v);
  }
}

// Elementwise max of two u16 pairs.
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a),
                                                                __builtin_bit_cast(us2, b)));
}

// An io-dtype pair as two floats (exact).
template <bool BF16>
__device__ inline void io_pair_f32(uint32_t w, float& a, float& b) {
  if constexpr (BF16) {
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xffff0000u);
  } else {
    a = half_bits_to_f32((uint16_t)(w & 0xFFFF));
    b = half_bits_to_f32((uint16_t)(w >> 16));
  }
}

// An io-dtype pair times a power of two, in the io dtype (exact for bf16;
// fp16 rounds only where the product is subnormal).
template <bool BF16>
__device__ inline uint32_t scaled_io_pair(uint32_t w, float pow2) {
  float a, b;
  io_pair_f32<BF16>(w, a, b);
  a *= pow2;
  b *= pow2;
  if constexpr (BF16) return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
  return pk_rne(a, b);
}

// Two codes of nibble pair `byte` of w (each nibble 0..3, value = code / 2 in
// e2m1) -> two exact fp16 integers.
template <int BYTE>
__device__ inline uint32_t cvt2(uint32_t w) {
  return h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, BYTE));
}

// ... and with the digit times 4 (scale 8): high value digits
template <int BYTE>
__device__ inline uint32_t cvt2x4(uint32_t w) {
  return h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 8.0f, BYTE));
}

// ... and with the digit times sc / 2 (sc a power of two: digit d of a
// progressive code takes sc = 2 * 4^d)
template <int BYTE>
__device__ inline uint32_t cvt2s(uint32_t w, float sc) {
  return h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, BYTE));
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

// max over lanes l, l^16, l^32, l^48: two lane-swap VALU ops (gfx950
// v_permlane32_swap / v_permlane16_swap), no LDS round trip
__device__ inline float wave_max_kq(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(x, fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(x, fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1])));
}
__device__ inline float wave_sum_kq(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// A lane's value moved by a DPP pattern (all rows and banks enabled).
#define KVQ_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), (ctrl), 0xF, 0xF, false))
// max / sum over all 64 lanes: within each row of 16 (quad xor 1, quad xor
// 2, half-row mirror, row mirror), then across the four rows
__device__ inline float wave_max64(float x) {
  x = fmaxf(x, KVQ_DPP(x, 0xB1));
  x = fmaxf(x, KVQ_DPP(x, 0x4E));
  x = fmaxf(x, KVQ_DPP(x, 0x141));
  x = fmaxf(x, KVQ_DPP(x, 0x140));
  return wave_max_kq(x);
}
__device__ inline float wave_sum64(float x) {
  x += KVQ_DPP(x, 0xB1);
  x += KVQ_DPP(x, 0x4E);
  x += KVQ_DPP(x, 0x141);
  x += KVQ_DPP(x, 0x140);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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


// The value of lane 15 - (l % 16) of the same 16-lane row (DPP row_mirror).
__device__ inline float mirror16(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
}

// Exact residual of an fp16 pair product: fp16(a*b - hi) in one fused
// multiply-add (v_pk_fma_f16); with hi = fp16(a*b) it is the exact
// remainder, so hi + lo = a*b (barring fp16 underflow of the remainder).
__device__ inline uint32_t pk_fma_lo(uint32_t a, uint32_t b, uint32_t hi) {
  return h2u(__builtin_elementwise_fma(u2h(a), u2h(b), -u2h(hi)));
}

// Workspace of one call (zero-filled once by the caller; counters return to
// zero at the end of every call):
//   tick u32    [B*Hkv][64]          splits finished (word 0; each counter
//                                     on a 256-byte line of its own, so the
//                                     splits of different KV heads never
//                                     contend for one line).  First, so that
//                                     its place does not depend on the split
//                                     count: a workspace may serve calls with
//                                     different split counts in turn.
//   ml   float2 [B*Hkv][S][G]        per split and head: running max m (log2
//                                     units) and softmax denominator l
//   o    float  [B*Hkv][S][G][128]   per split and head: o / l
struct Ws {
  uint32_t* tick;
  float2* ml;    // device-coherent copy of the split records
  float* o;
  float2* mlL;   // the same records, stored for the L2 of the storing CU
  float* oL;
#ifdef KVQ_STAMPS
  unsigned long long* st;  // phase timestamps, STAMP_SLOTS per workgroup
#endif
};

// Phase timestamps (the KVQ_STAMPS build only; the product build compiles
// them out): s_memrealtime (a 100 MHz clock shared by the whole device) at
// fixed points of each workgroup, stored after the workspace proper.
[[maybe_unused]] constexpr int STAMP_SLOTS = 32;
// They are kept in LDS and stored once at exit, so that no store of theirs
// changes how the compiler orders the kernel's own memory accesses.
#ifdef KVQ_STAMPS
#define KVQ_STAMP(cond, slot)                                        \
  do {                                                               \
    if (cond) lds.stamp[(slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define KVQ_STAMP_FLUSH()                                                                 \
  do {                                                                                    \
    __syncthreads();                                                                      \
    if (tid < STAMP_SLOTS) ws.st[(size_t)blockIdx.x * STAMP_SLOTS + tid] = lds.stamp[tid]; \
  } while (0)
#else
#define KVQ_STAMP(cond, slot) \
  do {                        \
  } while (0)
#define KVQ_STAMP_FLUSH() \
  do {                    \
  } while (0)
#endif

constexpr int TICK_STRIDE = 64;  // u32 words between counters (256 bytes)
__host__ __device__ inline size_t ws_tick_bytes(int B, int Hkv) {
  return (size_t)B * Hkv * TICK_STRIDE * 4;
}
__host__ __device__ inline size_t ws_ml_bytes(int B, int Hq, int S) {
  return ((size_t)B * Hq * S * 8 + 255) & ~(size_t)255;
}
__host__ __device__ inline size_t ws_o_bytes(int B, int Hq, int S) {
  return (size_t)B * Hq * S * D * 4;
}

inline Ws ws_layout(void* base, int B, int Hq, int Hkv, int S) {
  Ws w;
  const size_t t = ws_tick_bytes(B, Hkv), m = ws_ml_bytes(B, Hq, S), o = ws_o_bytes(B, Hq, S);
  w.tick = (uint32_t*)base;
  w.ml = (float2*)((char*)base + t);
  w.o = (float*)((char*)base + t + m);
  w.mlL = (float2*)((char*)base + t + m + o);
  w.oL = (float*)((char*)base + t + 2 * m + o);
  return w;
}

// LDS.  Loop phase: the per-wave group slots and the query tables (every wave
// writes the same values into the tables and reads only after its own writes,
// so no workgroup barrier is needed before the stream).  Merge phase (after a
// barrier, every slot copy consumed or drained): the wave records, or the
// fused variant's packing step.
struct LdsMerge {
  float o[NW][MAXG][D + 4];  // wave results before the workgroup merge (padded rows)
  float m[NW][MAXG], l[NW][MAXG];
};
// The final merge: every split's (m, l) per head, then its weight, and per
// head 1 / L.
struct LdsFinal {
  f2 ml[1024 * MAXG];  // (m, l), then (w, l) with w = 2^(m - M) l
  float inv[MAXG];
};
template <int SLOTB, int NSLOT>
struct Lds {
  union {
    __align__(16) uint8_t slots[NW][NSLOT][SLOTB];
    LdsMerge merge;
    LdsFinal fin;
    PackLds pack;  // FUSED: the append step of the first workgroup, after its ticket
  } u;
  __align__(16) uint16_t qin[MAXG][D];       // the query as copied in (io dtype), every head
  __align__(16) uint16_t q16[MAXG][D + 8];   // query as fp16 (scaled), every head
  __align__(16) uint16_t qraw[MAXG][D + 8];  // query in the io dtype, scaled (HIMODE 16)
  int hil[16];                               // salient channels, ascending
  uint8_t plist[2][64];                      // DENSE1: the 2-bit (0) and 1-bit (1) channels, ascending
  uint8_t pone[64];                          // DENSE1: pair j is a 1-bit pair
  uint16_t sal_s[NW][16];                    // per wave: salient scales of the group in work
  int mrank;                                 // -1: not the last split; 0/1: merge (1: all splits on this XCD)
  int prog[NW];                              // per wave: quantized groups it has started
#ifdef KVQ_STAMPS
  unsigned long long stamp[STAMP_SLOTS];
#endif
  int first;                                 // FUSED: the first workgroup of its (sequence, KV head) to finish
};

// HASQ: the cache has quantized-group storage (capacity NG >= 1); without it
// no group address exists and the group stream is compiled out.
// KB > 0: query-channel pruning (Dual-QK, abstract: a decode query keeps its
// few large channels and the key cache is read only for them).  Per
// (sequence, KV head) the nkeep (1..7) 16-channel key runs of largest sum
// over the group's heads of min(floor(4096 |q_c|), 2^20) are kept (ties to
// the lower run); the query is zero on the others, whose key codes and
// scale/zero are not copied: a pruning wave issues its first copies only
// once the query has arrived and the runs are chosen.  The kept runs pair
// up into the MFMAs' 32-long contractions, KB = ceil(nkeep / 2) per tile.
// VHI: the cache has two value precisions (g.n_vhi > 0): the first n_vhi
// 8-slot blocks of each group (its tokens of largest key magnitude) add their
// high value digits (4 * digit) through more MFMAs per tile.
// FUSED: the call also appends one token per (sequence, KV head) (knew,
// vnew) and attends it (PM-KVQ, key_machinery: 16-bit first, quantized
// later).  Every wave reads the length before the append and attends the
// quantized prefix of that length plus the ring and the new token, which
// it takes from knew/vnew; a group that the append completes is attended
// from the ring at 16 bits in this call.  The first workgroup of the
// (sequence, KV head) to take its ticket writes the token to its ring slot
// and packs the completed group; the last merging workgroup, after every
// workgroup has read the length, stores the new length.  With PROG the pack
// also shrinks the groups that cross the window edges, which every split of
// this call reads: the last workgroup packs, after its merge.
// LOCOL (G <= 8): the exact pair (hi, lo) of every product q*s and p*s
// enters one MFMA, hi in column h of head h and lo in the spare column
// 15 - h; lane (col, kq) serves head col (col < G) or 15 - col (col >= 16 -
// G).  Logits and outputs add the two columns (a row_mirror DPP).  Without
// it (G > 8, every column taken) hi and lo take an MFMA each.
// PROG: progressive precision (PM-KVQ review, lead and key_machinery: codes
// held at more bits while young and shrunk as they age).  The g.w4 newest
// groups (8 or 4 bits) are "window" items: after the ring blocks, in the
// same round robin over the waves, each is copied with its digit planes
// (digit d of a code (X >> 2d) & 3; plane d enters the MFMA with the weight
// 4^d through the convert's scale) into the wave's free slots and attended
// there; the stream takes the older (2-bit) groups only.
template <bool B>
struct Wide {
  static constexpr bool value = B;
};
// DENSE1 (the dense 1-bit layout, no salient pairs): chunk kq of the keys is
// the 2-bit run of plane channels wl[16 kq ..] and the 1-bit run ol[16 kq ..]
// (k_lo words, then half-words); the query enters the group MFMAs in that
// plane order, gathered once from its LDS copy, and the 1-bit run's codes
// come from four nibble masks of its half-word.
template <bool BF16, int HIMODE, bool HASQ, int KB, bool VHI, bool FUSED, bool LOCOL,
          bool PROG = false, bool DENSE1 = false>
__global__ __launch_bounds__(WG_THREADS) void decode_kernel(Geo g, const uint16_t* __restrict__ q,
                                                            kvq_cache c, float scale_log2, int S,
                                                            Ws ws, uint16_t* __restrict__ out,
                                                            const uint16_t* __restrict__ knew,
                                                            const uint16_t* __restrict__ vnew,
                                                            int nkeep) {
  constexpr bool PRUNE = KB > 0;
  using SC = SlotCfg<HIMODE, VHI>;
  constexpr int NSLOT = SC::NSLOT, NLD = SC::NLD, SLOTB = SC::BYTES;
  static_assert(!PROG || (NSLOT >= 3 && SLOTB >= 3072 && !PRUNE && !VHI),
                "a window group takes three slots: its record and three planes per side");
  static_assert(!DENSE1 || (HIMODE == 0 && !PRUNE && !PROG), "dense 1-bit layout variants");
  __shared__ Lds<SLOTB, NSLOT> lds;
  // the wave index is wave-uniform: keeping it in a scalar register makes every
  // group address scalar (one 64-bit base per copy, no per-lane address math)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  // Workgroups are dealt to the 8 XCDs round robin (workgroup i to XCD
  // i mod 8): when the (sequence, KV head) count is a multiple of 8, the
  // splits of one (sequence, KV head) take workgroups of one residue, so
  // that they share an L2 (the final merge then reads their records there;
  // the ticket checks where every split actually ran).
  const bool xmap = (g.B * g.Hkv) % 8 == 0;
  const int bh = xmap ? (int)(blockIdx.x % 8) + 8 * (int)((blockIdx.x / 8) / S)
                      : (int)(blockIdx.x / S);
  const int s = xmap ? (int)((blockIdx.x / 8) % S) : (int)(blockIdx.x % S);
  const int b = bh / g.Hkv, kh = bh % g.Hkv;
  const int G = g.G;
  const bool hvalid = col < G;                    // lane of head col's hi column
  const bool lo_lane = LOCOL && col >= 16 - G;    // lane of head 15 - col's lo column
  const bool qvalid = hvalid || lo_lane;          // the lane carries a query
  const int hq = hvalid ? col : (lo_lane ? 15 - col : 0);
  KVQ_STAMP(tid == 0, 0);
  lds.prog[wave] = 0;

  // ---- entry.  The length and the leading ranks are scalar loads; the
  // query (every head of the group: G rows of 256 bytes) is copied straight
  // into LDS like the group records, so that no vector-register load is
  // waited for while copies are in flight (the compiler cannot count the two
  // kinds together and would wait for all of them).
  const int len = load_uniform(c.len + bh);
  int top[8];
#pragma unroll
  for (int r = 0; r < 8; r++) top[r] = load_uniform(c.pairs + (size_t)bh * NPAIR + r);
  {
    const uint8_t* qsrc = (const uint8_t*)(q + ((size_t)b * g.Hq + kh * G) * D);
    for (int i = 0; i < (G + 3) / 4; i++) {
      // 1 KB = 4 rows per copy; rows past G re-read row G - 1 (never read back)
      const int row = min(4 * i + (lane >> 4), G - 1);
      dma16(qsrc + (size_t)row * (D * 2) + (lane & 15) * 16, &lds.qin[4 * i][0]);
    }
    // DENSE1: the rank table (256 bytes, lanes past 16 repeat it) into the
    // LDS the raw-salient query would use (unused without salient pairs),
    // with the query: a load issued after the group copies would wait for them
    if constexpr (DENSE1)
      dma16((const uint8_t*)(c.pairs + (size_t)bh * NPAIR) + (lane & 15) * 16, &lds.qraw[0][0]);
  }
  const int RSB = g.RS / GS;        // physical ring blocks
  const int STR = S * NW;           // flat indices of one (sequence, KV head)
  const int f = s + S * wave;       // this wave's flat index
  const bool ring_owner = f < RSB;  // owns physical ring blocks f, f + STR, ... < RSB
  // PROG: flat items RSB .. NBLK - 1 are the window groups (age f - RSB)
  const int NBLK = RSB + (PROG ? g.w4 : 0);
  const bool blk_owner = f < NBLK;
  // quantized groups of this wave: g_i = gfirst + i STR (the first such index
  // >= 0), copied into slot i % NSLOT.  The first NSLOT copies go out at
  // once, a fixed number (past the capacity the index is clamped into it;
  // such copies are never consumed and are drained before the LDS is
  // reused).  A ring-owning wave first loads and attends its ring blocks (in
  // vector registers) and issues its copies after that.
  const size_t rec0 = (size_t)bh * g.NG;
  const int gfirst = f - NBLK + (blk_owner ? (NBLK - f + STR - 1) / STR * STR : 0);
  uint8_t* slots = &lds.u.slots[wave][0][0];
  int issued = 0;
  // kept 16-channel key runs (bit s: run s; all eight unless PRUNE) and the
  // first of them; PRUNE sets them once the query has arrived
  uint32_t kmask = 0xFFu;
  int kept0 = 0;
  auto issue_first = [&]() {
    if constexpr (HASQ) {
#pragma unroll
      for (int i = 0; i < NSLOT; i++)
        issue_group<HIMODE, VHI, PRUNE, DENSE1>(c, rec0 + (size_t)min(gfirst + i * STR, g.NG - 1),
                                        slots + i * SLOTB, lane, kmask, kept0, g.nh, g.n_vhi);
      issued = NSLOT;
    }
  };
  u4 kt[2][4], vt[8];
  u4 knk[4];
  uint16_t vnk[8];
  // ring block rb (32 slots): key rows in tile order, value columns
  auto load_ring = [&](int rb) {
    const uint16_t* rk = (const uint16_t*)c.ring_k + ((size_t)bh * g.RS + rb * GS) * D;
    const uint16_t* rv = (const uint16_t*)c.ring_v + (((size_t)bh * RSB + rb) * D) * GS;
#pragma unroll
    for (int TT = 0; TT < 2; TT++) {
      const u4* kr = (const u4*)(rk + (size_t)tile_token(16 * TT + col) * D + 32 * kq);
#pragma unroll
      for (int k = 0; k < 4; k++) kt[TT][k] = kr[k];
    }
#pragma unroll
    for (int tt = 0; tt < 8; tt++) vt[tt] = *(const u4*)(rv + (size_t)(16 * tt + col) * GS + 8 * kq);
  };
  if (ring_owner) {
    load_ring(f);
    if constexpr (FUSED) {
      const u4* kn = (const u4*)(knew + (size_t)bh * D + 32 * kq);
#pragma unroll
      for (int k = 0; k < 4; k++) knk[k] = kn[k];
#pragma unroll
      for (int tt = 0; tt < 8; tt++) vnk[tt] = vnew[(size_t)bh * D + 16 * tt + col];
    }
    wait_vmcnt<0>();
  } else if (PRUNE || blk_owner) {
    // the query; PRUNE: the group copies wait for the kept runs; a window
    // owner first takes its window groups into its slots
    wait_vmcnt<0>();
  } else {
    issue_first();
    wait_vmcnt<HASQ ? NSLOT * NLD : 0>();  // the query copies (issued before the group copies)
  }
  compiler_fence();
  // the query slice of lane (col, kq): head col, channels 32kq .. 32kq+31
  u4 qv[4];
#pragma unroll
  for (int i = 0; i < 4; i++) qv[i] = *(const u4*)&lds.qin[hq][32 * kq + 8 * i];

  // kept key runs (PRUNE), a wave-uniform mask: E_s sums min(floor(4096 |q|),
  // 2^20) over run s's 16 channels and the G heads (at most 2^28, exact in 32
  // bits); lane (col, kq) holds runs 2kq (qv[0..1]) and 2kq + 1 (qv[2..3]),
  // whose query slices are zeroed when the runs are pruned
  uint32_t cmap = 0;  // kept runs in ascending order, three bits each
  if constexpr (PRUNE) {
    // run energies E_r: lane l sums min(floor(4096 |q|), 2^20) over
    // channels 2l, 2l + 1 of every head (from the query's LDS copy; 4096 |q|
    // is exact and the conversion truncates), the 8 lanes of run l / 8 add
    // up (quad xor 1, xor 2, half-row mirror), and lane r < 8 ranks run r
    // against the eight sums (ties to the lower run)
    uint32_t e = 0;
    for (int h = 0; h < G; h++) {
      const uint32_t x = *(const uint32_t*)&lds.qin[h][2 * lane];
      e += (uint32_t)fminf(4096.0f * fabsf(in_to_f32((uint16_t)(x & 0xFFFF), BF16)), 1048576.0f);
      e += (uint32_t)fminf(4096.0f * fabsf(in_to_f32((uint16_t)(x >> 16), BF16)), 1048576.0f);
    }
    e += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0xB1, 0xF, 0xF, false);
    e += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x4E, 0xF, 0xF, false);
    e += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x141, 0xF, 0xF, false);
    const int rr = lane & 7;
    const uint32_t Er = (uint32_t)__shfl((int)e, 8 * rr);
    int rank = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t Ei = (uint32_t)__builtin_amdgcn_readlane((int)e, 8 * i);
      rank += (Ei > Er) || (Ei == Er && i < rr);
    }
    kmask = (uint32_t)(__ballot(rank < nkeep) & 0xFFull);
    kmask = __builtin_amdgcn_readfirstlane(kmask);
    kept0 = __builtin_ctz(kmask);
    int n = 0;
#pragma unroll
    for (int r = 0; r < 8; r++)
      if ((kmask >> r) & 1u) {
        cmap |= (uint32_t)r << (3 * n);
        n++;
      }
    if (!ring_owner) issue_first();  // only the kept runs' codes and scale/zero
#pragma unroll
    for (int h = 0; h < 2; h++)
      if (!((kmask >> (2 * kq + h)) & 1u)) qv[2 * h] = qv[2 * h + 1] = u4{0, 0, 0, 0};
  }
  const int kqa = kq;

  // The quantized path multiplies q by key scales in fp16 (q*s, 4*q*s), so
  // each head's query is first scaled by a power of two 2^-qe that puts its
  // largest magnitude in [1/8, 1/4): then 4 |q| s < s <= 65504 for every
  // channel.  The scaling is exact (barring fp16 subnormals); the head's
  // logits take the factor back through sc_q.  Ring tokens use the raw query.
  float qmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float a, bb;
      io_pair_f32<BF16>(qv[i][e], a, bb);
      qmax = fmaxf(qmax, fmaxf(fabsf(a), fabsf(bb)));
    }
  qmax = wave_max_kq(qmax);  // over the head's 128 channels (the 4 lanes of column col)
  KVQ_STAMP(tid == 0 && qmax >= 0.0f, 1);
  const int qbexp = (int)((__float_as_uint(qmax) >> 23) & 0xFFu);
  const int qe = qbexp ? min(max(qbexp - 124, -100), 100) : 0;  // largest |q| < 2^(qe - 2)
  const float qsc = __uint_as_float((uint32_t)(127 - qe) << 23);  // 2^-qe
  const float sc_q = scale_log2 * __uint_as_float((uint32_t)(127 + qe) << 23);
  // query as fp16 pairs, scaled (zero on lanes of no head); LOCOL: qm is the
  // same on lo lanes and zero elsewhere, so that pk_fma(q, s, -q_m s) gives
  // the rounding hi of q*s on hi lanes and its residual lo on lo lanes
  uint32_t q16[16], qm[16];
  // DENSE1: the group MFMAs take the query in plane order (k_lo layout):
  // element 8i + 2e (+1) of chunk kq is wl[16 kq + 8i + 2e (+1)] for i < 2 and
  // ol[16 kq + 8 (i - 2) + 2e (+1)] for i >= 2; the ring keeps channel order
  u4 qg[4] = {qv[0], qv[1], qv[2], qv[3]};
  if constexpr (DENSE1) {
    // the 1-bit pairs (ranks 32 .. 63): rank lane's pair gets its flag (the
    // ranks are a permutation, so every flag is written once)
    lds.pone[((const int32_t*)&lds.qraw[0][0])[lane] & (NPAIR - 1)] = lane >= NPAIR / 2;
    __builtin_amdgcn_wave_barrier();
    compiler_fence();
    const uint64_t one = __ballot(lds.pone[lane] != 0);
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const bool isone = (one >> lane) & 1ull;
    const int rk = __popcll((isone ? one : ~one) & below);
    // every wave writes the same lists and reads only after its own writes
    lds.plist[isone][rk] = (uint8_t)lane;
    lds.plist[isone][32 + rk] = (uint8_t)(lane + NPAIR);
    __builtin_amdgcn_wave_barrier();
    compiler_fence();
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const uint8_t* lst = &lds.plist[i >> 1][16 * kq + 8 * (i & 1) + 2 * e];
        qg[i][e] = (uint32_t)lds.qin[hq][lst[0]] | ((uint32_t)lds.qin[hq][lst[1]] << 16);
      }
  }
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float a, bb;
      io_pair_f32<BF16>(qg[i][e], a, bb);
      q16[4 * i + e] = qvalid ? pk_rne(a * qsc, bb * qsc) : 0u;
      qm[4 * i + e] = lo_lane ? q16[4 * i + e] : 0u;
    }
  // the query for the keys' zero-point bias: LOCOL zero on the lo lanes, so
  // that the bias lands in the hi columns only (once per call, not per group)
  uint32_t qh[16];
#pragma unroll
  for (int w = 0; w < 16; w++) qh[w] = LOCOL && lo_lane ? 0u : q16[w];

  const int T_old = min(max(len, 0), g.max_tokens);  // reads stay inside the cache
  // FUSED: whether this call appends (a full cache or a negative length is
  // reported and decoded as it stands)
  const bool app = FUSED && len >= 0 && len < g.max_tokens;
  const int T = T_old + (app ? 1 : 0);
  const int nq = n_quant(T_old, g.R), ngq = nq / GS;  // FUSED: the prefix before the append
  const int nr = T - nq;                               // raw (ring) tokens, <= RS
  // this wave's live groups: g_i < ngq
  // PROG: the stream takes groups [0, n2), the window the rest
  const int nwin = PROG ? min(g.w4, ngq) : 0, n2 = ngq - nwin;
  const int nmine = (HASQ && gfirst < n2) ? (n2 - 1 - gfirst) / STR + 1 : 0;

  uint32_t qhi[4] = {0, 0, 0, 0};  // HIMODE 4: 4*q (fp16); HIMODE 16: raw q
  uint32_t qhim[4] = {0, 0, 0, 0};  // HIMODE 4: qhi on K-lanes 16..31 (the residual lanes), else 0
  int sal_ch = 0;                  // HIMODE 4: salient channel whose scale lane%16 copies
  if constexpr (HIMODE != 0 || PRUNE) {
    // tables: every head's query rows (each wave writes the same values and
    // reads only after its own writes) and the salient channels (pairs of
    // rank < n_hi ascending, then the same + 64)
    if (hvalid) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        *(u4*)&lds.q16[col][32 * kq + 8 * i] =
            u4{q16[4 * i], q16[4 * i + 1], q16[4 * i + 2], q16[4 * i + 3]};
        if constexpr (HIMODE == 16) {  // raw salient keys meet the scaled query in its io dtype
          u4 r;
#pragma unroll
          for (int e = 0; e < 4; e++) r[e] = scaled_io_pair<BF16>(qv[i][e], qsc);
          *(u4*)&lds.qraw[col][32 * kq + 8 * i] = r;
        }
      }
    }
  }
  if constexpr (HIMODE != 0) {
    bool sal = false;
#pragma unroll
    for (int r = 0; r < 8; r++)
      sal |= r < g.n_hi && (top[r] & 63) == lane;
    const unsigned long long m = __ballot(sal);
    // the salient channel list in ascending order: entry d < n_hi is the
    // d-th set bit of m, entry n_hi + d the same + 64; entries past 2 n_hi
    // are 0 (in range even for a malformed rank table).  Lane d < 16 forms
    // entry d.
    if (lane < 16) {
      const int want = lane < g.n_hi ? lane : lane - g.n_hi;
      unsigned long long mm = m;
      int v = 0;
#pragma unroll
      for (int d = 0; d < 8; d++) {
        const int p = mm ? __builtin_ctzll(mm) : 0;
        v = d == want ? p : v;
        mm &= mm - 1;
      }
      v += lane >= g.n_hi ? NPAIR : 0;
      lds.hil[lane] = lane < 2 * g.n_hi ? v : 0;
    }
    // LDS accesses of one wave execute in order: a compiler barrier suffices
    __builtin_amdgcn_wave_barrier();
    compiler_fence();
    // (every read unconditional, in range, so that the eight go out together)
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int d = 8 * (kq & 1) + e;
      // HIMODE 4: K-lanes 16..31 (kq 2, 3) repeat the digits of lanes 0..15
      // and carry the rounding residual of 4*q*s; HIMODE 16 uses lanes 0..15.
      // Only the hi columns take the salient terms.
      const bool ok = hvalid && d < g.nh && (HIMODE == 4 || kq < 2);
      const int ch = lds.hil[d] & (D - 1);
      const uint32_t v = HIMODE == 4 ? (uint32_t)lds.q16[col][ch] : (uint32_t)lds.qraw[col][ch];
      qhi[e >> 1] |= (ok ? v : 0u) << (16 * (e & 1));
    }
    if constexpr (HIMODE == 4) {
      // 4 q (exact in fp16)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        qhi[e] = h2u(u2h(qhi[e]) * u2h(0x44004400u));
        qhim[e] = kq < 2 ? 0u : qhi[e];
      }
    }
    sal_ch = lds.hil[lane & 15] & (D - 1);
  }

  // PRUNE: the i-th MFMA contraction of a tile (i < ceil(nkeep / 2)) covers
  // the kept runs 2i (K-lanes of kq 0, 1) and 2i + 1 (kq 2, 3).  Lane (col,
  // kq) feeds the pairs 8 r + 4 (kq%2) + b, b = 0..3, of its run r (channels
  // 16 r ..): the low (kq%2 = 0) or high half of run r's k_lo word, as the
  // unpruned path takes a word's halves.  qk[i] holds head col's fp16 query
  // at those pairs; it is zero where the run is past the kept ones (odd
  // nkeep).
  const int khalf = kq & 1;
  int krun[4];
  u4 qk[4];
  if constexpr (PRUNE) {
    if constexpr (HIMODE == 0) {
      __builtin_amdgcn_wave_barrier();
      compiler_fence();
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if (i >= KB) break;
      const int n = 2 * i + (kq >> 1);
      krun[i] = (cmap >> (3 * n)) & 7u;
      const bool live = qvalid && n < nkeep;
      qk[i] = live ? *(const u4*)&lds.q16[hq][16 * krun[i] + 8 * khalf] : u4{0, 0, 0, 0};
    }
  }

  float m_run = -INFINITY, l_raw = 0.0f;
  f4 O[8], Cvb = {0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < 8; t++) O[t] = f4{0, 0, 0, 0};
  const uint32_t ONES = 0x3c003c00u;  // fp16 (1, 1)

  // online-softmax step on this block's 8 logits per lane, given unscaled as
  // c (the log2-unit logit is sc * c with sc > 0, so max c gives max x)
  // The running max moves only when some logit exceeds it by more than the
  // slack: a per-lane test and a ballot decide that; the cross-lane max is
  // taken only then.
  auto softmax_step = [&](const float (&cc)[8], float sc, float slack, float (&p)[8]) {
    const float mc = fmaxf(fmaxf(fmaxf(cc[0], cc[1]), fmaxf(cc[2], cc[3])),
                           fmaxf(fmaxf(cc[4], cc[5]), fmaxf(cc[6], cc[7])));
    if (__builtin_amdgcn_ballot_w64(mc * sc > m_run + slack)) {
      const float mx = wave_max_kq(mc) * sc;
      const bool need = mx > m_run + slack;
      const float m_new = need ? mx : m_run;
      const float alpha = ex2(m_run - m_new);
#pragma unroll
      for (int t = 0; t < 8; t++) O[t] *= alpha;
      Cvb *= alpha;
      l_raw *= alpha;
      m_run = m_new;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) p[i] = ex2(fmaf(cc[i], sc, -m_run));
  };

  // One quantized group, its records in `slot` (copies landed).  WIDE (a
  // window group of `width` 4 or 8 bits): digit planes 1.. of its keys at
  // kpl + 1024 (d - 1), of its values at vpl + 1024 (d - 1); plane 1 holds
  // the salient channels' digit 1 too, so the k_hi term is left out.
  auto process_group = [&](const uint8_t* slot, auto wide_tag, int width, const uint8_t* kpl,
                           const uint8_t* vpl) {
    constexpr bool WIDE = decltype(wide_tag)::value;
    const uint32_t* sm = (const uint32_t*)(slot + SC::META);
    // keys: q' = q * s as an exact fp16 pair (qs + qsl), bias = q . z (the
    // same for every token row); each tile's accumulator starts from the
    // bias, so no VALU adds follow
    uint32_t qs[16], qsl[16];
    f4 cb = {0, 0, 0, 0};
    if constexpr (PRUNE) {
      // contraction i's q*s pairs into qs[4i..4i+3]; pruned runs take no work
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (i >= KB) break;
        const int pb = 16 * krun[i] + 4 * khalf;  // the run's scale pairs, then its zero pairs
        const u4 spv = *(const u4*)(sm + pb), zp = *(const u4*)(sm + pb + 8);
#pragma unroll
        for (int bb = 0; bb < 4; bb++) {
          const uint32_t sp = spv[bb];
          if constexpr (LOCOL) {
            qs[4 * i + bb] = pk_fma_lo(qk[i][bb], sp, pk_mul(lo_lane ? qk[i][bb] : 0u, sp));
          } else {
            qs[4 * i + bb] = pk_mul(qk[i][bb], sp);
            qsl[4 * i + bb] = pk_fma_lo(qk[i][bb], sp, qs[4 * i + bb]);
          }
        }
        cb = mma_f16(u4{zp[0], zp[1], zp[2], zp[3]}, u4{qk[i][0], qk[i][1], qk[i][2], qk[i][3]},
                     cb);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        // chunk kq's channel pairs 4i .. 4i+3: run 2kq + i/2, its pairs 4 (i%2) ..
        const uint32_t* rm = sm + (2 * kq + (i >> 1)) * 16 + 4 * (i & 1);
        const u4 sv = *(const u4*)rm;
        const u4 zv = *(const u4*)(rm + 8);
#pragma unroll
        for (int e = 0; e < 4; e++) {
          if constexpr (LOCOL) {
            qs[4 * i + e] = pk_fma_lo(q16[4 * i + e], sv[e], pk_mul(qm[4 * i + e], sv[e]));
          } else {
            qs[4 * i + e] = pk_mul(q16[4 * i + e], sv[e]);
            qsl[4 * i + e] = pk_fma_lo(q16[4 * i + e], sv[e], qs[4 * i + e]);
          }
        }
        const u4 qb = u4{qh[4 * i], qh[4 * i + 1], qh[4 * i + 2], qh[4 * i + 3]};
        cb = mma_f16(zv, qb, cb);
      }
    }
    if constexpr (LOCOL && PRUNE) {
      // the bias enters the hi columns only (the unpruned path's qh is zero
      // on the lo lanes already)
#pragma unroll
      for (int r = 0; r < 4; r++) cb[r] = lo_lane ? 0.0f : cb[r];
    }
    uint32_t qshi[4];
    if constexpr (HIMODE == 4 && !WIDE) {
      // the salient channels' scales, gathered once into a contiguous row
      // (lane l copies digit l%16), then read 8 at a time
      uint16_t* ss = lds.sal_s[wave];
      ss[lane & 15] = ((const uint16_t*)sm)[(sal_ch >> 4) * 32 + (sal_ch & 15)];
      __builtin_amdgcn_wave_barrier();
      compiler_fence();
      const u4 spv = *(const u4*)(ss + 8 * (kq & 1));
#pragma unroll
      for (int e = 0; e < 4; e++) {
        // 4*q*s as an exact fp16 pair: K-lanes 0..15 its rounding hi,
        // K-lanes 16..31 the residual lo (qhim is zero on the former, so
        // the fma subtracts 0 there and the rounding hi elsewhere)
        qshi[e] = pk_fma_lo(qhi[e], spv[e], pk_mul(qhim[e], spv[e]));
      }
    }
    // DENSE1: the 1-bit run's word of tile row col (both halves), masked once
    uint32_t X1b[4] = {0, 0, 0, 0};
    if constexpr (DENSE1) {
      const uint32_t w1 = ((const uint32_t*)(slot + SC::KLO + 512))[kqa * 16 + col];
#pragma unroll
      for (int i = 0; i < 4; i++) X1b[i] = (w1 >> i) & 0x11111111u;
    }
    f4 C[2];
#pragma unroll
    for (int TT = 0; TT < 2; TT++) {
      f4 acc = cb;
      if constexpr (PRUNE) {
        const int sh = 16 * khalf;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if (i >= KB) break;
          // the lane's half of run krun[i]'s word: pairs 4 khalf .. +3
          const uint32_t w =
              ((const uint32_t*)(slot + SC::KLO))[(krun[i] * 2 + TT) * 16 + col] >> sh;
          const uint32_t A = w & 0x33333333u, Bn = (w >> 2) & 0x33333333u;
          const u4 cd = u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)};
          acc = mma_f16(cd, u4{qs[4 * i], qs[4 * i + 1], qs[4 * i + 2], qs[4 * i + 3]}, acc);
          if constexpr (!LOCOL)
            acc = mma_f16(cd, u4{qsl[4 * i], qsl[4 * i + 1], qsl[4 * i + 2], qsl[4 * i + 3]}, acc);
        }
      } else if constexpr (DENSE1) {
        // chunk kqa: its 2-bit run (u = 0) and its 1-bit run (u = 1; tile
        // half TT in bytes 2 TT, 2 TT + 1 of the masks shared by both halves)
        const uint32_t w2 = ((const uint32_t*)(slot + SC::KLO))[(kqa * 2 + TT) * 16 + col];
        {
          const uint32_t A = w2 & 0x33333333u, Bn = (w2 >> 2) & 0x33333333u;
          const u4 c0 = u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)};
          const u4 c1 = u4{cvt2<2>(A), cvt2<2>(Bn), cvt2<3>(A), cvt2<3>(Bn)};
          acc = mma_f16(c0, u4{qs[0], qs[1], qs[2], qs[3]}, acc);
          acc = mma_f16(c1, u4{qs[4], qs[5], qs[6], qs[7]}, acc);
          if constexpr (!LOCOL) {
            acc = mma_f16(c0, u4{qsl[0], qsl[1], qsl[2], qsl[3]}, acc);
            acc = mma_f16(c1, u4{qsl[4], qsl[5], qsl[6], qsl[7]}, acc);
          }
        }
        {
          const u4 c0 = TT == 0 ? u4{cvt2<0>(X1b[0]), cvt2<0>(X1b[1]), cvt2<1>(X1b[0]), cvt2<1>(X1b[1])}
                                : u4{cvt2<2>(X1b[0]), cvt2<2>(X1b[1]), cvt2<3>(X1b[0]), cvt2<3>(X1b[1])};
          const u4 c1 = TT == 0 ? u4{cvt2<0>(X1b[2]), cvt2<0>(X1b[3]), cvt2<1>(X1b[2]), cvt2<1>(X1b[3])}
                                : u4{cvt2<2>(X1b[2]), cvt2<2>(X1b[3]), cvt2<3>(X1b[2]), cvt2<3>(X1b[3])};
          acc = mma_f16(c0, u4{qs[8], qs[9], qs[10], qs[11]}, acc);
          acc = mma_f16(c1, u4{qs[12], qs[13], qs[14], qs[15]}, acc);
          if constexpr (!LOCOL) {
            acc = mma_f16(c0, u4{qsl[8], qsl[9], qsl[10], qsl[11]}, acc);
            acc = mma_f16(c1, u4{qsl[12], qsl[13], qsl[14], qsl[15]}, acc);
          }
        }
      } else {
        const uint32_t* kw0 = (const uint32_t*)(slot + SC::KLO) + (kqa * 4 + TT) * 16 + col;
        const u2 w = u2{kw0[0], kw0[32]};  // the two 16-channel runs of chunk kqa
#pragma unroll
        for (int u = 0; u < 2; u++) {
          const uint32_t A = w[u] & 0x33333333u, Bn = (w[u] >> 2) & 0x33333333u;
          const int k0 = 8 * u;
          const u4 c0 = u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)};
          const u4 c1 = u4{cvt2<2>(A), cvt2<2>(Bn), cvt2<3>(A), cvt2<3>(Bn)};
          acc = mma_f16(c0, u4{qs[k0], qs[k0 + 1], qs[k0 + 2], qs[k0 + 3]}, acc);
          acc = mma_f16(c1, u4{qs[k0 + 4], qs[k0 + 5], qs[k0 + 6], qs[k0 + 7]}, acc);
          if constexpr (!LOCOL) {
            acc = mma_f16(c0, u4{qsl[k0], qsl[k0 + 1], qsl[k0 + 2], qsl[k0 + 3]}, acc);
            acc = mma_f16(c1, u4{qsl[k0 + 4], qsl[k0 + 5], qsl[k0 + 6], qsl[k0 + 7]}, acc);
          }
        }
        if constexpr (WIDE) {
          // digits 1 (and 2, 3) of every channel, weighted 4^d by the convert
#pragma unroll
          for (int d = 1; d <= 3; d++) {
            if (d > 1 && width < 8) break;
            const float sc = (float)(2 << (2 * d));
            const uint32_t* pw0 = (const uint32_t*)(kpl + (d - 1) * 1024) + (kqa * 4 + TT) * 16 + col;
            const u2 wp = u2{pw0[0], pw0[32]};
#pragma unroll
            for (int u = 0; u < 2; u++) {
              const uint32_t A = wp[u] & 0x33333333u, Bn = (wp[u] >> 2) & 0x33333333u;
              const int k0 = 8 * u;
              const u4 c0 = u4{cvt2s<0>(A, sc), cvt2s<0>(Bn, sc), cvt2s<1>(A, sc), cvt2s<1>(Bn, sc)};
              const u4 c1 = u4{cvt2s<2>(A, sc), cvt2s<2>(Bn, sc), cvt2s<3>(A, sc), cvt2s<3>(Bn, sc)};
              acc = mma_f16(c0, u4{qs[k0], qs[k0 + 1], qs[k0 + 2], qs[k0 + 3]}, acc);
              acc = mma_f16(c1, u4{qs[k0 + 4], qs[k0 + 5], qs[k0 + 6], qs[k0 + 7]}, acc);
              if constexpr (!LOCOL) {
                acc = mma_f16(c0, u4{qsl[k0], qsl[k0 + 1], qsl[k0 + 2], qsl[k0 + 3]}, acc);
                acc = mma_f16(c1, u4{qsl[k0 + 4], qsl[k0 + 5], qsl[k0 + 6], qsl[k0 + 7]}, acc);
              }
            }
          }
        }
      }
      if constexpr (HIMODE == 4 && !WIDE) {
        const uint32_t kw = ((const uint32_t*)(slot + SC::KHI))[16 * TT + col];
        const uint32_t wsel = (kq & 1) ? kw >> 16 : kw;
        const uint32_t A = wsel & 0x33333333u, Bn = (wsel >> 2) & 0x33333333u;
        acc = mma_f16(u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)},
                      u4{qshi[0], qshi[1], qshi[2], qshi[3]}, acc);
      }
      if constexpr (HIMODE == 16) {
        // salient channels 8*(kq&1) .. +7 of the lane's token (entries past nh
        // are masked; the read may run past the record, inside the LDS)
        const uint16_t* kr = (const uint16_t*)(slot + SC::KHI) + (16 * TT + col) * g.nh + 8 * (kq & 1);
        const u4a v = *(const u4a*)kr;
        u4 a = u4{v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int d = 8 * (kq & 1) + 2 * e;
          const uint32_t keep = kq >= 2 ? 0u : (d < g.nh ? 0x0000ffffu : 0u) | (d + 1 < g.nh ? 0xffff0000u : 0u);
          a[e] &= keep;
        }
        acc = mma_raw<BF16>(a, u4{qhi[0], qhi[1], qhi[2], qhi[3]}, acc);
      }
      C[TT] = acc;
    }
    float cr[8], p[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
      cr[i] = LOCOL ? C[i >> 2][i & 3] + mirror16(C[i >> 2][i & 3]) : C[i >> 2][i & 3];
    // lanes 32..47 hold the group's value scales in their 16 staged bytes
    // (non-negative fp16, so their bits order as integers)
    const u4 meta = ((const u4*)sm)[lane];
    const uint32_t vs2 = pk_max_u16(pk_max_u16(meta[0], meta[1]), pk_max_u16(meta[2], meta[3]));
    const uint64_t wide =
        __builtin_amdgcn_ballot_w64(max(vs2 & 0xFFFFu, vs2 >> 16) > VSCALE_WIDE) &
        0x0000FFFF00000000ull;  // lanes 32..47
    softmax_step(cr, sc_q, wide ? RESCALE_SLACK_WIDE : RESCALE_SLACK, p);
    const u4 P = u4{pk_rne(p[0], p[1]), pk_rne(p[2], p[3]), pk_rne(p[4], p[5]), pk_rne(p[6], p[7])};
    // LOCOL: the weights on lo lanes (zero elsewhere), as qm for the query
    u4 Pm;
#pragma unroll
    for (int e = 0; e < 4; e++) Pm[e] = lo_lane ? P[e] : 0u;
    // values: p*s as an exact fp16 pair (pj + pjl) per channel group j
    const bool vkept = VHI && kq < g.n_vhi;
    const u4 za = col < 4 ? ((const u4*)(sm + 192 + 16 * col))[kq]
                          : (col == 4 ? u4{ONES, ONES, ONES, ONES} : u4{0, 0, 0, 0});
    Cvb = mma_f16(za, P, Cvb);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const u4 sv = ((const u4*)(sm + 128 + 16 * j))[kq];
      u4 pj, pjl;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        if constexpr (LOCOL) {
          pj[e] = pk_fma_lo(P[e], sv[e], pk_mul(Pm[e], sv[e]));
        } else {
          pj[e] = pk_mul(P[e], sv[e]);
          pjl[e] = pk_fma_lo(P[e], sv[e], pj[e]);
        }
      }
      const uint32_t wv = ((const uint32_t*)(slot + SC::VC))[(j * 4 + kq) * 16 + col];
      const uint32_t A = wv & 0x33333333u, Bn = (wv >> 2) & 0x33333333u;
      const u4 v0 = u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)};
      const u4 v1 = u4{cvt2<2>(A), cvt2<2>(Bn), cvt2<3>(A), cvt2<3>(Bn)};
      O[2 * j] = mma_f16(v0, pj, O[2 * j]);
      O[2 * j + 1] = mma_f16(v1, pj, O[2 * j + 1]);
      if constexpr (!LOCOL) {
        O[2 * j] = mma_f16(v0, pjl, O[2 * j]);
        O[2 * j + 1] = mma_f16(v1, pjl, O[2 * j + 1]);
      }
      if constexpr (WIDE) {
#pragma unroll
        for (int d = 1; d <= 3; d++) {
          if (d > 1 && width < 8) break;
          const float sc = (float)(2 << (2 * d));
          const uint32_t wq = ((const uint32_t*)(vpl + (d - 1) * 1024))[(j * 4 + kq) * 16 + col];
          const uint32_t Aq = wq & 0x33333333u, Bq = (wq >> 2) & 0x33333333u;
          const u4 h0 = u4{cvt2s<0>(Aq, sc), cvt2s<0>(Bq, sc), cvt2s<1>(Aq, sc), cvt2s<1>(Bq, sc)};
          const u4 h1 = u4{cvt2s<2>(Aq, sc), cvt2s<2>(Bq, sc), cvt2s<3>(Aq, sc), cvt2s<3>(Bq, sc)};
          O[2 * j] = mma_f16(h0, pj, O[2 * j]);
          O[2 * j + 1] = mma_f16(h1, pj, O[2 * j + 1]);
          if constexpr (!LOCOL) {
            O[2 * j] = mma_f16(h0, pjl, O[2 * j]);
            O[2 * j + 1] = mma_f16(h1, pjl, O[2 * j + 1]);
          }
        }
      }
      if constexpr (VHI) {
        // block kq's high digits (0 past the high-precision blocks), weighted
        // 4 by the convert
        const uint32_t wh =
            vkept ? ((const uint32_t*)(slot + SC::VH))[(j * g.n_vhi + kq) * 16 + col] : 0u;
        const uint32_t Ah = wh & 0x33333333u, Bh = (wh >> 2) & 0x33333333u;
        const u4 h0 = u4{cvt2x4<0>(Ah), cvt2x4<0>(Bh), cvt2x4<1>(Ah), cvt2x4<1>(Bh)};
        const u4 h1 = u4{cvt2x4<2>(Ah), cvt2x4<2>(Bh), cvt2x4<3>(Ah), cvt2x4<3>(Bh)};
        O[2 * j] = mma_f16(h0, pj, O[2 * j]);
        O[2 * j + 1] = mma_f16(h1, pj, O[2 * j + 1]);
        if constexpr (!LOCOL) {
          O[2 * j] = mma_f16(h0, pjl, O[2 * j]);
          O[2 * j + 1] = mma_f16(h1, pjl, O[2 * j + 1]);
        }
      }
    }
  };

  // ---- the ring blocks (16-bit keys and values) of a ring-owning wave:
  // physical slots 32 rb .. 32 rb + 31; slot sigma holds the position
  // nq + ((sigma - nq) mod RS), live when that is below T.
  for (int rb = f; ring_owner && rb < RSB; rb += STR) {
    if (rb != f) load_ring(rb);
    if (nr <= 0) continue;
    // FUSED: the appended token's index in this block (-1 if not here); its
    // key row and value column come from knew / vnew, not from the ring
    const int snew = app ? T_old % g.RS : -1;
    const int tnew = (snew >= rb * GS && snew < rb * GS + GS) ? snew - rb * GS : -1;
    auto live = [&](int t) {
      const int sigma = rb * GS + t;
      const int d = ((sigma - nq) % g.RS + g.RS) % g.RS;
      return d < nr;
    };
    // a block with no live slot adds nothing (and its logits, all -inf,
    // must not meet a running max that is still -inf)
    if (!__builtin_amdgcn_ballot_w64(lane < GS && live(lane))) continue;
    if constexpr (FUSED) {
#pragma unroll
      for (int TT = 0; TT < 2; TT++)
        if (tile_token(16 * TT + col) == tnew) {
#pragma unroll
          for (int k = 0; k < 4; k++) kt[TT][k] = knk[k];
        }
      const int dt = tnew - 8 * kq;  // the new token among this lane's 8 slots
      if (tnew >= 0 && dt >= 0 && dt < 8) {
#pragma unroll
        for (int tt = 0; tt < 8; tt++) {
          const uint32_t x = vnk[tt];
          const int e = dt >> 1, sh = 16 * (dt & 1);
          const uint32_t mk = 0xFFFFu << sh;
#pragma unroll
          for (int i = 0; i < 4; i++)
            if (i == e) vt[tt][i] = (vt[tt][i] & ~mk) | (x << sh);
        }
      }
    }
    uint32_t qraw[16];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int e = 0; e < 4; e++) qraw[4 * i + e] = hvalid ? qv[i][e] : 0u;
    f4 Cr[2];
#pragma unroll
    for (int TT = 0; TT < 2; TT++) {
      f4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 4; k++)
        acc = mma_raw<BF16>(kt[TT][k],
                            u4{qraw[4 * k], qraw[4 * k + 1], qraw[4 * k + 2], qraw[4 * k + 3]}, acc);
      Cr[TT] = acc;
    }
    float cr[8], p[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int t = 8 * kq + 4 * (i >> 2) + (i & 3);
      const float x = LOCOL ? Cr[i >> 2][i & 3] + mirror16(Cr[i >> 2][i & 3]) : Cr[i >> 2][i & 3];
      cr[i] = live(t) ? x : -INFINITY;
    }
    softmax_step(cr, scale_log2, RESCALE_SLACK, p);  // raw values: the products stay in fp32
#pragma unroll
    for (int i = 0; i < 8; i++) l_raw += p[i];
    uint32_t Ph[4], Pl[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      split_pair<BF16>(p[2 * i], p[2 * i + 1], Ph[i], Pl[i]);
      if (lo_lane) Ph[i] = Pl[i] = 0u;  // the raw values enter the hi columns only
    }
    uint32_t vkeep[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int t0 = 8 * kq + 2 * e;
      vkeep[e] = (live(t0) ? 0x0000ffffu : 0u) | (live(t0 + 1) ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int tt = 0; tt < 8; tt++) {
      u4 a = vt[tt];
      // zero dead slots (they may hold stale data)
#pragma unroll
      for (int e = 0; e < 4; e++) a[e] &= vkeep[e];
      O[tt] = mma_raw<BF16>(a, u4{Ph[0], Ph[1], Ph[2], Ph[3]}, O[tt]);
      O[tt] = mma_raw<BF16>(a, u4{Pl[0], Pl[1], Pl[2], Pl[3]}, O[tt]);
    }
  }
  // ---- PROG: the window groups of this wave (flat items RSB .. NBLK - 1,
  // age = item - RSB), each copied with its planes into the wave's slots 0
  // (record), 1 (key planes) and 2 (value planes), attended, and drained
  // before the slots take the stream's copies
  if constexpr (PROG && HASQ) {
    uint8_t* s1 = slots + SLOTB;
    uint8_t* s2 = slots + 2 * SLOTB;
    for (int it = ring_owner ? f + (RSB - f + STR - 1) / STR * STR : f; it < RSB + nwin;
         it += STR) {
      const int age = it - RSB, gw = ngq - 1 - age;
      const int width = prog_width(age, g.w8, g.w4);
      issue_group<HIMODE, VHI, false, DENSE1>(c, rec0 + gw, slots, lane, 0xFFu, 0, g.nh, g.n_vhi);
      const size_t p1 = ((size_t)bh * g.npl + gw % g.w4) * 1024 + lane * 16;
      dma16<CPOL_NT>((const uint8_t*)c.k_pl + p1, s1);
      dma16<CPOL_NT>((const uint8_t*)c.v_pl + p1, s2);
      if (width == 8) {
        const size_t p23 = ((size_t)bh * g.npl + g.w4 + 2 * (gw % g.w8)) * 1024 + lane * 16;
        dma16<CPOL_NT>((const uint8_t*)c.k_pl + p23, s1 + 1024);
        dma16<CPOL_NT>((const uint8_t*)c.k_pl + p23 + 1024, s1 + 2048);
        dma16<CPOL_NT>((const uint8_t*)c.v_pl + p23, s2 + 1024);
        dma16<CPOL_NT>((const uint8_t*)c.v_pl + p23 + 1024, s2 + 2048);
      }
      wait_vmcnt<0>();
      compiler_fence();
      process_group(slots, Wide<true>{}, width, s1, s2);
      wait_lgkmcnt0();  // every read of the slots has returned before they are refilled
      compiler_fence();
    }
  }
  if (blk_owner) issue_first();
  KVQ_STAMP(tid == 0, 2);

  // ---- the quantized groups: slot i % NSLOT holds group i; a consumed slot
  // is refilled with group i + NSLOT
  if constexpr (HASQ) {
    for (int i = 0; i < nmine; i++) {
      // wave priority: the arbiter favours the older of a SIMD's two waves
      // (waves w and w ^ 4 of the workgroup), which leaves the younger to
      // finish its last groups alone, at a lower issue rate.  A wave that has
      // started more groups than the other wave of its SIMD yields to it
      // (advisory: a stale count only delays the balance).  Eight waves on
      // four SIMDs only; other wave counts keep the arbiter's order.  The
      // counts are plain LDS words, read and written without ordering: an
      // atomic access would make the compiler wait for every copy in flight
      // (the group copies also write LDS) at each group.
      if constexpr (NW == 8) {
        const int other = __builtin_amdgcn_readfirstlane(lds.prog[wave ^ 4]);
        lds.prog[wave] = i;
        if (i > other)
          __builtin_amdgcn_s_setprio(0);
        else if (i < other)
          __builtin_amdgcn_s_setprio(2);
        else
          __builtin_amdgcn_s_setprio(1);
      }
      wait_slot<NLD, NSLOT>(issued - 1 - i);
      uint8_t* slot = slots + (i % NSLOT) * SLOTB;
      process_group(slot, Wide<false>{}, 2, nullptr, nullptr);
#ifdef KVQ_STAMPS
      if (i == 0) KVQ_STAMP(tid == 0 && O[0][0] != 12345.0f, 11);
#endif
      if (issued < nmine) {
        // every read of this slot has returned before the copy overwrites it
        wait_lgkmcnt0();
        compiler_fence();
        issue_group<HIMODE, VHI, PRUNE, DENSE1>(c, rec0 + gfirst + (size_t)issued * STR, slot, lane,
                                        kmask, kept0, g.nh, g.n_vhi);
        issued++;
      }
    }
    lds.prog[wave] = 1 << 20;  // done: the other wave of the SIMD no longer yields to it
    __builtin_amdgcn_s_setprio(0);
    // copies issued before the length was known, past the live groups: they
    // must land before the LDS is reused
    if (issued > nmine) {
      wait_vmcnt<0>();
      compiler_fence();
    }
  }

  // FUSED: the new token's key and value channel tid, for the ring write of
  // the first workgroup (loaded after the stream: only copies are in flight
  // during it)
  uint16_t knv = 0, vnv = 0;
  if constexpr (FUSED)
    if (tid < D) {
      knv = knew[(size_t)bh * D + tid];
      vnv = vnew[(size_t)bh * D + tid];
    }

  if constexpr (LOCOL) {
#pragma unroll
    for (int t = 0; t < 8; t++)
#pragma unroll
      for (int r = 0; r < 4; r++) O[t][r] += mirror16(O[t][r]);
  }

  // ---- merge the waves: per head m, l and unnormalized o
  KVQ_STAMP(lane == 0 && O[0][0] != 12345.0f, 3 + wave);
  __syncthreads();  // every wave is done with the loop-phase LDS
  KVQ_STAMP(tid == 0, 23);
  {
    const float l_q = __shfl(Cvb[0], 16 + col);  // all-ones row 4 -> lane 16 + col
    const float l = l_q + wave_sum_kq(l_raw);
    float vb[4];
#pragma unroll
    for (int j = 0; j < 4; j++) vb[j] = __shfl(Cvb[j], col);  // value-zero rows 0..3
    if (hvalid) {
      if (kq == 0) {
        lds.u.merge.m[wave][col] = m_run;
        lds.u.merge.l[wave][col] = l;
      }
#pragma unroll
      for (int tt = 0; tt < 8; tt++)
        *(f4*)&lds.u.merge.o[wave][col][16 * tt + 4 * kq] = O[tt] + vb[tt >> 1];
    }
  }
  __syncthreads();
  KVQ_STAMP(tid == 0, 24);
  // split record: (m, l) and o / l per head, fp32, one element per thread
  // (each thread forms its head's wave weights 2^(m_w - M) itself from
  // broadcast reads).  Stored twice: once device-coherent (sc1 stores, seen
  // by a merging workgroup on any XCD) and once as plain stores, which stay
  // in the L2 of this CU's XCD (read by the merging workgroup when every
  // split of the (sequence, KV head) ran on its XCD, which the ticket tells).
  const size_t rbh = (size_t)bh * S * G;  // first record of this (sequence, KV head)
  const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(
      ws.o + rbh * D, 0, (int)(S * G * D * 4), BUF_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rs_oL = __builtin_amdgcn_make_buffer_rsrc(
      ws.oL + rbh * D, 0, (int)(S * G * D * 4), BUF_RSRC_WORD3);
  for (int e = tid; e < G * D; e += WG_THREADS) {
    const int h = e / D, cc = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; w++) M = fmaxf(M, lds.u.merge.m[w][h]);
    float L = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      const float mw = lds.u.merge.m[w][h];
      const float aw = mw == -INFINITY ? 0.0f : ex2(mw - M);
      L += aw * lds.u.merge.l[w][h];
      o += aw * lds.u.merge.o[w][h][cc];
    }
    const float v = L > 0.0f ? o / L : 0.0f;
    const int ooff = ((s * G + h) * D + cc) * 4;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs_o, ooff, 0, CPOL_SC1);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs_oL, ooff, 0, 0);
    if (cc == 0) {
      const uint64_t mlv = (uint64_t)__float_as_uint(M) | ((uint64_t)__float_as_uint(L) << 32);
      __hip_atomic_store((uint64_t*)&ws.ml[rbh + (size_t)s * G + h], mlv, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      *(uint64_t*)&ws.mlL[rbh + (size_t)s * G + h] = mlv;
    }
    // one split: its record is the attention output, stored at once (no
    // split merge follows)
    if (S == 1) out[((size_t)b * g.Hq + kh * G + h) * D + cc] = to_io_bits<BF16>(v);
  }

  // ---- ticket.  Every record store has completed (s_waitcnt) before the
  // counter moves: the workgroup that takes the last ticket sees every
  // coherent record, and every plain one in its own L2 if all splits ran on
  // its XCD.  The 64-bit counter holds one byte per XCD (splits of this
  // (sequence, KV head) that ran there; S <= 255), or a plain count.
  KVQ_STAMP(tid == 0, 12);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  KVQ_STAMP(tid == 0, 13);
  uint64_t* tick = (uint64_t*)(ws.tick + (size_t)bh * TICK_STRIDE);
  if (tid == 0) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    xcc &= 7u;
    const bool bytes = S <= 255;
    const uint64_t mine = bytes ? 1ull << (8 * xcc) : 1ull;
    const uint64_t prev = __hip_atomic_fetch_add(tick, mine, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t now = prev + mine;
    // byte sums fit in a byte (S <= 255)
    const uint32_t arrived = bytes ? (uint32_t)((now * 0x0101010101010101ull) >> 56) : (uint32_t)now;
    const uint32_t before = arrived - 1;
    lds.mrank = arrived == (uint32_t)S ? (bytes && now == ((uint64_t)S << (8 * xcc)) ? 1 : 0) : -1;
    if constexpr (FUSED) lds.first = before == 0u;
#ifdef KVQ_STAMPS
    lds.stamp[14] = __builtin_amdgcn_s_memrealtime() + 0 * prev;
    lds.stamp[17] =
        (unsigned long long)bh | ((unsigned long long)s << 16) | ((unsigned long long)xcc << 32) |
        ((unsigned long long)before << 40);
#endif
  }
  __syncthreads();
  if constexpr (FUSED) {
    // the first workgroup to finish does the append's ring write and packing
    // while the others still run: nothing in this call reads the packed
    // records, the ring slot it writes is read by this call's ring block only
    // as a dead slot or replaced by knew / vnew, and the group [nq, nq + 32)
    // ends at T - R <= T_old (the new token is not in it).  The length is
    // stored by the last workgroup, after every workgroup has read it.
    if (lds.first && app) {
      const int slot = T_old % g.RS;
      if (tid < D) {
        uint16_t* rk = (uint16_t*)c.ring_k + (size_t)bh * g.RS * D;
        uint16_t* rv = (uint16_t*)c.ring_v + (size_t)bh * g.RS * D;
        rk[(size_t)slot * D + tid] = knv;
        rv[((size_t)(slot / GS) * D + tid) * GS + slot % GS] = vnv;
      }
      if (!PROG && n_quant(T, g.R) > nq && tid < 128)
        pack_ring_group<BF16, VHI, false, DENSE1>(g, c, bh, nq, tid, lds.u.pack);
    }
    __syncthreads();  // the packing's LDS is free again before the merge uses it
  }
  const int mr = lds.mrank;
  if (mr < 0) {
    KVQ_STAMP_FLUSH();
    return;
  }
  const bool local = mr == 1;  // every split ran on this XCD: read the L2 copy
  if (tid == 0) __hip_atomic_store(tick, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // with one split the workgroup merge wrote the output
  if (S > 1) {
    // The last workgroup merges all splits.  Thread (chunk q, subset r): the
    // 4 channels 4 (q % 32) .. of head q / 32, over splits r, r + NR, ...; the
    // NR threads of a chunk are adjacent lanes and add up with shuffles.  The
    // (m, l) of the first 64 splits and the records of up to 2 RB splits per
    // thread are requested at once, in that order; meanwhile each head's
    // weights w_i = 2^(m_i - M) l_i (M the largest running max) and 1 / L,
    // L = sum w_i, are formed (one wave per head, lanes over splits).
    const int NQ = G * (D / 4);
    int NR = 1;
    while (NR * 2 * NQ <= WG_THREADS) NR *= 2;
    const int qc = tid / NR, r = tid % NR;
    const bool act = qc < NQ;
    const int h = act ? qc / (D / 4) : 0, c4 = act ? 4 * (qc % (D / 4)) : 0;
    constexpr int RB = 8;
    const int nk = (S - r + NR - 1) / NR;  // this thread's splits
    const int nkmax = (S + NR - 1) / NR;   // the most any thread has
    const __amdgpu_buffer_rsrc_t rs_mlL =
        __builtin_amdgcn_make_buffer_rsrc(ws.mlL + rbh, 0, (int)(S * G * 8), BUF_RSRC_WORD3);
    auto load_ml = [&](int i, int hh) -> uint64_t {
      if (local) {
        const u2 x = __builtin_amdgcn_raw_buffer_load_b64(rs_mlL, (i * G + hh) * 8, 0, CPOL_SC0);
        return (uint64_t)x[0] | ((uint64_t)x[1] << 32);
      }
      return __hip_atomic_load((const uint64_t*)&ws.ml[rbh + (size_t)i * G + hh], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    };
    auto load_batch = [&](u4 (&ov)[RB], int k0) {
#pragma unroll
      for (int k = 0; k < RB; k++) {
        const int ooff = ((min(r + (k0 + k) * NR, S - 1) * G + h) * D + c4) * 4;  // past S: unused
        ov[k] = local ? __builtin_amdgcn_raw_buffer_load_b128(rs_oL, ooff, 0, CPOL_SC0)
                      : __builtin_amdgcn_raw_buffer_load_b128(rs_o, ooff, 0, CPOL_SC1);
      }
    };
    const uint64_t ml0 = wave < G ? load_ml(min(lane, S - 1), wave) : 0ull;
    u4 ova[RB], ovb[RB];
    load_batch(ova, 0);
    if (nkmax > RB) load_batch(ovb, RB);
    KVQ_STAMP(tid == 0, 18);
    for (int hh = wave; hh < G; hh += NW) {
      float M = -INFINITY;
      for (int i = lane; i < S; i += 64) {
        const uint64_t mv = (hh == wave && i == lane) ? ml0 : load_ml(i, hh);
        const float mi = __uint_as_float((uint32_t)mv);
        lds.u.fin.ml[i * MAXG + hh] = f2{mi, __uint_as_float((uint32_t)(mv >> 32))};
        M = fmaxf(M, mi);
      }
      M = wave_max64(M);
      float L = 0.0f;
      for (int i = lane; i < S; i += 64) {
        const f2 x = lds.u.fin.ml[i * MAXG + hh];
        const float w = x[0] == -INFINITY ? 0.0f : ex2(x[0] - M) * x[1];
        lds.u.fin.ml[i * MAXG + hh][0] = w;
        L += w;
      }
      L = wave_sum64(L);
      if (lane == 0) lds.u.fin.inv[hh] = L > 0.0f ? 1.0f / L : 0.0f;
    }
    __syncthreads();
    KVQ_STAMP(tid == 0, 19);
    f4 acc = {0, 0, 0, 0};
    auto accum = [&](const u4 (&ov)[RB], int k0) {
#pragma unroll
      for (int k = 0; k < RB; k++)
        if (k0 + k < nk)
          acc += lds.u.fin.ml[(r + (k0 + k) * NR) * MAXG + h][0] * __builtin_bit_cast(f4, ov[k]);
    };
    accum(ova, 0);
    if (nkmax > RB) accum(ovb, RB);
    for (int k0 = 2 * RB; k0 < nkmax; k0 += RB) {
      load_batch(ova, k0);
      accum(ova, k0);
    }
    for (int o = 1; o < NR; o <<= 1)
#pragma unroll
      for (int e = 0; e < 4; e++) acc[e] += __shfl_xor(acc[e], o);
    KVQ_STAMP(tid == 0, 20);
    if (act && r == 0) {
      const float inv = lds.u.fin.inv[h];
      uint16_t* op = out + ((size_t)b * g.Hq + kh * G + h) * D + c4;
      uint16_t bits[4];
#pragma unroll
      for (int e = 0; e < 4; e++) bits[e] = to_io_bits<BF16>(acc[e] * inv);
      *(u2*)op = u2{bits[0] | ((uint32_t)bits[1] << 16), bits[2] | ((uint32_t)bits[3] << 16)};
    }
  }
  KVQ_STAMP(tid == 0, 15);
#ifdef KVQ_STAMPS
  __builtin_amdgcn_s_waitcnt(0);
  KVQ_STAMP(tid == 0, 16);
#endif
  KVQ_STAMP_FLUSH();
  if constexpr (FUSED && PROG) {
    // the pack of a progressive cache: every split of this (sequence, KV
    // head) has read its window groups (its ticket followed its loads), and
    // the merge's LDS is free once every thread is past the output
    if (app && n_quant(T, g.R) > nq) {
      __syncthreads();
      if (tid < 128) pack_ring_group<BF16, VHI, true, false>(g, c, bh, nq, tid, lds.u.pack);
    }
  }
  if constexpr (FUSED) {
    // the append's length (or its error): every workgroup of this (sequence,
    // KV head) read the length before it took its ticket
    if (tid == 0) {
      if (app) c.len[bh] = T;
      else atomicOr(c.err, len < 0 ? 2 : 1);
    }
  }
}

// The launch arguments shared by every kernel variant.
struct Launch {
  const void* q;
  const kvq_cache* c;
  float scale_log2;
  int S;
  Ws ws;
  void* out;
  const void* knew;  // FUSED only
  const void* vnew;
  hipStream_t st;
};

template <bool BF16, int HIMODE, int KB, bool VHI, bool FUSED, bool LOCOL>
static void launch_cols(const Geo& g, int keep, const Launch& a) {
  const dim3 grid(g.B * g.Hkv * a.S), block(WG_THREADS);
  if constexpr (HIMODE == 0 && KB == 0) {
    if (g.NG > 0 && g.dense1) {
      hipLaunchKernelGGL((decode_kernel<BF16, 0, true, 0, VHI, FUSED, LOCOL, false, true>), grid,
                         block, 0, a.st, g, (const uint16_t*)a.q, *a.c, a.scale_log2, a.S, a.ws,
                         (uint16_t*)a.out, (const uint16_t*)a.knew, (const uint16_t*)a.vnew, keep);
      return;
    }
  }
  if constexpr (KB == 0 && !VHI) {
    if (g.NG > 0 && g.w4 > 0) {
      hipLaunchKernelGGL((decode_kernel<BF16, HIMODE, true, 0, false, FUSED, LOCOL, true>), grid,
                         block, 0, a.st, g, (const uint16_t*)a.q, *a.c, a.scale_log2, a.S, a.ws,
                         (uint16_t*)a.out, (const uint16_t*)a.knew, (const uint16_t*)a.vnew, keep);
      return;
    }
  }
  if (g.NG > 0)
    hipLaunchKernelGGL((decode_kernel<BF16, HIMODE, true, KB, VHI, FUSED, LOCOL>), grid, block,
                       0, a.st, g, (const uint16_t*)a.q, *a.c, a.scale_log2, a.S, a.ws,
                       (uint16_t*)a.out, (const uint16_t*)a.knew, (const uint16_t*)a.vnew, keep);
  else
    hipLaunchKernelGGL((decode_kernel<BF16, HIMODE, false, KB, false, FUSED, LOCOL>), grid,
                       block, 0, a.st, g, (const uint16_t*)a.q, *a.c, a.scale_log2, a.S, a.ws,
                       (uint16_t*)a.out, (const uint16_t*)a.knew, (const uint16_t*)a.vnew, keep);
}

template <bool BF16, int HIMODE, int KB, bool VHI, bool FUSED>
static void launch_one(const Geo& g, int keep, const Launch& a) {
  if (g.G <= 8) launch_cols<BF16, HIMODE, KB, VHI, FUSED, true>(g, keep, a);
  else launch_cols<BF16, HIMODE, KB, VHI, FUSED, false>(g, keep, a);
}

// keep 0: the fused append-and-decode call (every key run); 1..7: kept
// 16-channel key runs; 8: unpruned
template <bool BF16, int HIMODE, bool VHI>
static void launch_keep(const Geo& g, int keep, const Launch& a) {
  switch (keep) {
    case 0: launch_one<BF16, HIMODE, 0, VHI, true>(g, 8, a); break;
    case 1: case 2: launch_one<BF16, HIMODE, 1, VHI, false>(g, keep, a); break;
    case 3: case 4: launch_one<BF16, HIMODE, 2, VHI, false>(g, keep, a); break;
    case 5: case 6: launch_one<BF16, HIMODE, 3, VHI, false>(g, keep, a); break;
    case 7: launch_one<BF16, HIMODE, 4, VHI, false>(g, keep, a); break;
    default: launch_one<BF16, HIMODE, 0, VHI, false>(g, 8, a); break;
  }
}

// Two value precisions touch only the value side and pruning only the key
// side, so every combination has its own kernel.
template <bool BF16, int HIMODE>
static void launch_vhi(const Geo& g, int keep, const Launch& a) {
  if (g.n_vhi > 0) launch_keep<BF16, HIMODE, true>(g, keep, a);
  else launch_keep<BF16, HIMODE, false>(g, keep, a);
}

template <bool BF16>
hipError_t launch_decode_io(const Geo& g, int keep, const Launch& a) {
  const int hm = g.n_hi == 0 ? 0 : g.bits_hi;
  if (hm == 0) launch_vhi<BF16, 0>(g, keep, a);
  else if (hm == 4) launch_vhi<BF16, 4>(g, keep, a);
  else launch_vhi<BF16, 16>(g, keep, a);
  return hipGetLastError();
}

// The file is compiled twice so that the two halves of the kernel variants
// build in parallel: KVQ_DECODE_PART 0 holds the fp16 kernels, 1 the bf16
// kernels and the entry points.
#if KVQ_DECODE_PART == 0
template hipError_t launch_decode_io<false>(const Geo&, int, const Launch&);
#else
extern template hipError_t launch_decode_io<false>(const Geo&, int, const Launch&);

size_t decode_tick_bytes(int B, int Hkv) { return ws_tick_bytes(B, Hkv); }

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int S) {
  size_t n = ws_tick_bytes(B, Hkv) + 2 * (ws_ml_bytes(B, Hq, S) + ws_o_bytes(B, Hq, S));
#ifdef KVQ_STAMPS
  n += (size_t)B * Hkv * S * STAMP_SLOTS * 8;  // the timestamps of every workgroup
#endif
  return n;
}

hipError_t launch_decode(const Geo& g, const void* q, const kvq_cache* c, float sm_scale,
                         int S, int keep, void* workspace, void* out, hipStream_t st,
                         const void* k_new, const void* v_new) {
  Ws w = ws_layout(workspace, g.B, g.Hq, g.Hkv, S);
#ifdef KVQ_STAMPS
  w.st = (unsigned long long*)((char*)workspace + ws_tick_bytes(g.B, g.Hkv) +
                               2 * (ws_ml_bytes(g.B, g.Hq, S) + ws_o_bytes(g.B, g.Hq, S)));
#endif
  const Launch a{q, c, sm_scale * 1.4426950408889634f, S, w, out, k_new, v_new, st};
  return g.bf16 ? launch_decode_io<true>(g, keep, a) : launch_decode_io<false>(g, keep, a);
}
#endif

}  // namespace kvq
