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
// The salient keys' high digits weigh 4*q*s, which is split exactly into an
// fp16 value and its fp16 rounding residual carried by the otherwise unused
// K-lanes 16..31 of that MFMA.
//
// Work split: an 8-wave workgroup per (sequence, KV head, token split), one
// workgroup per CU by default.  The 32-token blocks of a (sequence, KV head)
// are dealt to its waves interleaved across splits (block b to the wave w of
// split s with s + S w = b mod S * 8), each wave with its own online softmax
// (base 2, scale folded into the exponent; the running max is raised only
// when a block's weights would exceed 2^8, or 2 in a group with very wide
// value scales, so most blocks skip the rescale and the fp16 products of
// weights and value scales stay finite).  The codes and scale/zero records of the next PF blocks are in
// flight per wave in registers; the record of the block in work is staged
// through a per-wave LDS buffer so that the 16 lanes sharing a channel slice
// read it as a broadcast.  The waves merge in LDS into one record per head
// (m, l, o/l, all fp32); the last workgroup of a (sequence, KV head) to finish
// (atomic counter) merges the split records with the log-sum-exp rule and
// writes the output.  The fused variant also carries the step's append (see
// FUSED at the kernel).
#include "common.h"
#include "internal.h"
#include "quant_group.h"

#ifndef KVQ_DECODE_PART
#define KVQ_DECODE_PART 1
#endif

namespace kvq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
// 16 bytes at a 4-byte-aligned address (raw salient rows are 2*nh bytes long)
typedef uint32_t u4a __attribute__((ext_vector_type(4), aligned(4)));

constexpr int NW = 8;                  // waves per workgroup (one workgroup per CU)
constexpr int WG_THREADS = 64 * NW;
constexpr int PF = 2;                  // quantized groups in flight per wave
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

// Buffer descriptor word 3 for raw byte-addressed buffers (gfx9 family), and
// the cache-policy bit that makes a buffer access device-coherent (sc1).
constexpr int BUF_RSRC_WORD3 = 0x00020000;
constexpr int CPOL_SC1 = 16;

// 16-bit input pair -> fp16 pair (bf16 widened exactly, then RNE to fp16)
template <bool BF16>
__device__ inline uint32_t to_f16_pair(uint32_t w) {
  if constexpr (!BF16) return w;
  return pk_rne(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
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

// Per-lane loads of one quantized group, issued one block ahead.
struct Pref {
  u2 klo[2];        // k_lo words of tile 0 and 1 (token col of the tile, channels 32kq..)
  uint32_t klc[2][4];  // pruned decode: k_lo word kq/2 of a key chunk per slot, tiles 0, 1
  uint32_t khi[2];  // k_hi word of tile 0 and 1
  u4 hraw[2];       // raw salient keys (HIMODE 16): 8 values of the lane's token, tile 0 and 1
  uint32_t vc[4];   // v_codes word of channel group j = 0..3
  u4 meta;          // 16 B of the group's k_meta (lanes 0-31) or v_meta (lanes 32-63)
  uint32_t vh[4];   // two value precisions: high-digit word of block kq, channel group j
};

// kqa: the key chunk whose low digits this lane reads (its own, kq, unless
// that chunk is pruned; then a kept chunk that other lanes read in the same
// instruction, so no extra line is fetched); mla: the same for the lane's
// 16-byte piece of the key scale/zero record.  A redirected lane's values
// only ever meet a zero query.
// CHUNKED (pruned decode): slot i (< NCH) holds, for key chunk
// (cmap >> 2i) & 3, the lane token's k_lo word kq/2 of that chunk.  Pruned
// chunks are never named in cmap, so they are never fetched.
// VHI (two value precisions by token, g.n_vhi high-precision 8-slot blocks
// per group, the group's slots in key-magnitude order): blocks kq < n have
// high-digit words; lanes of the other blocks read block n - 1's (fetched
// anyway) and drop them when the group is processed.
template <int HIMODE, bool CHUNKED, int NCH, bool VHI>
__device__ inline void load_group(const kvq_cache& c, size_t rec, int lane, int col, int kq,
                                  int kqa, int mla, uint32_t cmap, int nh, int nvhi, Pref& p) {
  if constexpr (VHI) {
    const uint32_t* vh = c.v_hi + rec * (8 + 64 * nvhi) + 8 + min(kq, nvhi - 1) * 16 + col;
#pragma unroll
    for (int j = 0; j < 4; j++) p.vh[j] = vh[j * nvhi * 16];
  }
  if constexpr (CHUNKED) {
    const uint32_t* w = (const uint32_t*)c.k_lo + rec * GROUP_WORDS;
#pragma unroll
    for (int TT = 0; TT < 2; TT++)
#pragma unroll
      for (int i = 0; i < NCH; i++) {
        const int mm = (cmap >> (2 * i)) & 3u;
        p.klc[TT][i] = w[((TT * 4 + mm) * 16 + col) * 2 + (kq >> 1)];
      }
  } else {
    const u2* klo = (const u2*)((const uint32_t*)c.k_lo + rec * GROUP_WORDS);
    p.klo[0] = klo[(0 * 4 + kqa) * 16 + col];
    p.klo[1] = klo[(1 * 4 + kqa) * 16 + col];
  }
  if constexpr (HIMODE == 4) {
    const uint32_t* kh = (const uint32_t*)c.k_hi + rec * 32;
    p.khi[0] = kh[col];
    p.khi[1] = kh[16 + col];
  }
  if constexpr (HIMODE == 16) {
    // salient channels 8*(kq&1) .. +7 of the lane's token (entries past nh
    // are masked later; the buffer carries 32 bytes of tail slack)
    const uint16_t* kh = (const uint16_t*)c.k_hi + rec * GS * nh;
#pragma unroll
    for (int TT = 0; TT < 2; TT++) {
      const u4a v = *(const u4a*)(kh + (16 * TT + col) * nh + 8 * (kq & 1));
      p.hraw[TT] = u4{v[0], v[1], v[2], v[3]};
    }
  }
  const uint32_t* vc = (const uint32_t*)c.v_codes + rec * GROUP_WORDS;
#pragma unroll
  for (int j = 0; j < 4; j++) p.vc[j] = vc[(j * 4 + kq) * 16 + col];
  const u4* meta = lane < 32 ? (const u4*)((const uint16_t*)c.k_meta + rec * 2 * D)
                             : (const u4*)((const uint16_t*)c.v_meta + rec * 2 * D);
  p.meta = meta[mla];
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
  float2* ml;
  float* o;
#ifdef KVQ_STAMPS
  unsigned long long* st;  // phase timestamps, STAMP_SLOTS per workgroup
#endif
};

// Phase timestamps (the KVQ_STAMPS build only; the product build compiles
// them out): s_memrealtime (a 100 MHz clock shared by the whole device) at
// fixed points of each workgroup, stored after the workspace proper.
constexpr int STAMP_SLOTS = 32;
#ifdef KVQ_STAMPS
#define KVQ_STAMP(cond, slot)                                                          \
  do {                                                                                 \
    if (cond)                                                                          \
      ws.st[(size_t)blockIdx.x * STAMP_SLOTS + (slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define KVQ_STAMP(cond, slot) \
  do {                        \
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
  w.tick = (uint32_t*)base;
  w.ml = (float2*)((char*)base + ws_tick_bytes(B, Hkv));
  w.o = (float*)((char*)base + ws_tick_bytes(B, Hkv) + ws_ml_bytes(B, Hq, S));
  return w;
}

// LDS, one layout per phase.  The loop phase is private to each wave (no
// workgroup barrier before the stream); a barrier separates it from the
// merge phase.
struct LdsLoop {
  uint16_t q16[NW][MAXG][D + 8];   // per wave: query as fp16 (padded rows)
  uint16_t qraw[NW][MAXG][D + 8];  // per wave: query in the io dtype (16-bit salient keys)
  uint32_t stage[NW][256];         // per wave: metadata record of the group in work
  int hil[NW][16];                 // per wave: salient channels, ascending
  uint16_t sal_s[NW][16];          // per wave: scales of the salient channels, group in work
};
struct LdsMerge {
  float o[NW][MAXG][D + 4];        // wave results before the workgroup merge (padded rows)
  float m[NW][MAXG], l[NW][MAXG];
};
struct Lds {
  union {
    LdsLoop loop;
    LdsMerge merge;
    PackLds pack;  // FUSED: the append step of the last workgroup, after the merge
  } u;
  int last;
  int first;  // FUSED: the first workgroup of its (sequence, KV head) to finish
};

// HASQ: the cache has quantized-group storage (capacity NG >= 1); without it
// no group address exists and the group stream is compiled out.
// LO1: some pairs are at 1 bit.  Their scale is the whole group range, three
// times a 2-bit channel's, so q*s is carried as an exact fp16 pair (rounded
// value + rounding residual) through a second MFMA pass over the same codes.
// KEEP < 4: query-channel pruning (Dual-QK, abstract: a decode query keeps
// its few large channels and the key cache is read only for them).  Per
// (sequence, KV head) the KEEP 32-channel key chunks of largest
// sum over the group's heads of min(floor(4096 |q_c|), 2^20) are kept (ties to the
// lower chunk); the query is zero on the others, whose key codes and
// scale/zero are not read (past the first PF prefetched groups, which are
// issued before the query arrives): their lanes load a kept chunk's words
// instead, which the same instruction fetches anyway.
// VHI: the cache has two value precisions (g.n_vhi > 0): the first n_vhi
// 8-slot blocks of each group (its tokens of largest key magnitude) add their
// high value digits (4 * digit) through one more MFMA per tile.
// FUSED: the call also appends one token per (sequence, KV head) (knew,
// vnew) and attends it (PM-KVQ, key_machinery: 16-bit first, quantized
// later).  Every wave reads the length before the append and attends the
// quantized prefix of that length plus the ring and the new token, which
// it takes from knew/vnew; a group that the append completes is attended
// from the ring at 16 bits in this call.  The last workgroup of the
// (sequence, KV head), after the merge (so after every workgroup has read
// the length and the ring), writes the token to its ring slot, packs the
// completed group and stores the new length.
template <bool BF16, int HIMODE, bool HASQ, bool LO1, int KEEP, bool VHI, bool FUSED>
__global__ __launch_bounds__(WG_THREADS) void decode_kernel(Geo g, const uint16_t* __restrict__ q,
                                                            kvq_cache c, float scale_log2, int S,
                                                            Ws ws, uint16_t* __restrict__ out,
                                                            const uint16_t* __restrict__ knew,
                                                            const uint16_t* __restrict__ vnew) {
  constexpr bool PRUNE = KEEP < 4;
  __shared__ Lds lds;
  // the wave index is wave-uniform: keeping it in a scalar register makes every
  // group address scalar (one 64-bit base per load, no per-lane address math)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int bh = blockIdx.x / S, s = blockIdx.x % S;
  const int b = bh / g.Hkv, kh = bh % g.Hkv;
  const int G = g.G;
  const bool hvalid = col < G;

  // ---- every wave starts on its own.  Its first requests are the length,
  // its query slice (head col, channels 32kq..32kq+31) and the 8 leading
  // ranks: anything requested behind the cache stream would wait for it.
  // The ranks are a buffer load, so that they stay in that order (memory
  // counters retire in order) rather than being issued where they are used.
  KVQ_STAMP(tid == 0, 0);
  int len = c.len[bh];
  u4 qv[4];
  {
    const u4* qg = (const u4*)(q + ((size_t)b * g.Hq + kh * G + min(col, G - 1)) * D + 32 * kq);
#pragma unroll
    for (int i = 0; i < 4; i++) qv[i] = qg[i];
  }
  u4 topv[2];
  if constexpr (HIMODE != 0) {
    const __amdgpu_buffer_rsrc_t rs_p = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(c.pairs + (size_t)bh * NPAIR), 0, 32, BUF_RSRC_WORD3);
    topv[0] = __builtin_amdgcn_raw_buffer_load_b128(rs_p, 0, 0, 0);
    topv[1] = __builtin_amdgcn_raw_buffer_load_b128(rs_p, 16, 0, 0);
  }
  // Quantized group g goes to wave w of split s with s + S*w = g mod S*NW,
  // so a wave's groups are first + i*STR: their addresses do not depend on
  // the length, and the first PF are requested before it arrives (clamped
  // to the capacity; loads past the wave's last group are never used).  At
  // every step the workgroups of a KV head read one contiguous band.
  const int STR = S * NW;          // group stride of one wave
  const size_t rec0 = (size_t)bh * g.NG;
  const int first = s + S * wave;  // this wave's groups: first + i*STR < ngq
  // FUSED: the new token's key and value channel tid (for the ring write of
  // the last workgroup), requested now so that the end does not wait for them
  uint16_t knv = 0, vnv = 0;
  if constexpr (FUSED)
    if (tid < D) {
      knv = knew[(size_t)bh * D + tid];
      vnv = vnew[(size_t)bh * D + tid];
    }
  Pref pf[PF];
  if constexpr (HASQ) {
#pragma unroll
    for (int k = 0; k < PF; k++)
      load_group<HIMODE, PRUNE, 4, VHI>(c, rec0 + (size_t)min(first + k * STR, g.NG - 1), lane,
                                        col, kq, kq, lane & 31, 0xE4u, g.nh, g.n_vhi, pf[k]);
  }


  // kept key chunks (all four unless PRUNE), a wave-uniform mask: E_m sums
  // min(floor(4096 |q|), 2^20) over chunk m's 32 channels and the G heads
  // (at most 2^29, exact in 32 bits); the 16 lanes of chunk kq are DPP row kq
  uint32_t kmask = 0xFu;
  if constexpr (PRUNE) {
    uint32_t e = 0;
    if (hvalid) {
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const uint32_t x = qv[i][w];  // 4096 |q| is exact; the conversion truncates
          e += (uint32_t)fminf(4096.0f * fabsf(in_to_f32((uint16_t)(x & 0xFFFF), BF16)),
                               1048576.0f);
          e += (uint32_t)fminf(4096.0f * fabsf(in_to_f32((uint16_t)(x >> 16), BF16)), 1048576.0f);
        }
    }
    e += (uint32_t)__builtin_amdgcn_update_dpp((int)e, (int)e, 0x128, 0xF, 0xF, false);  // row_ror:8
    e += (uint32_t)__builtin_amdgcn_update_dpp((int)e, (int)e, 0x124, 0xF, 0xF, false);  // row_ror:4
    e += (uint32_t)__builtin_amdgcn_update_dpp((int)e, (int)e, 0x122, 0xF, 0xF, false);  // row_ror:2
    e += (uint32_t)__builtin_amdgcn_update_dpp((int)e, (int)e, 0x121, 0xF, 0xF, false);  // row_ror:1
    uint32_t E[4];
#pragma unroll
    for (int m = 0; m < 4; m++) E[m] = (uint32_t)__builtin_amdgcn_readlane((int)e, 16 * m);
    kmask = 0;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      int rank = 0;
#pragma unroll
      for (int i = 0; i < 4; i++) rank += (E[i] > E[m]) || (E[i] == E[m] && i < m);
      if (rank < KEEP) kmask |= 1u << m;
    }
    if (!((kmask >> kq) & 1u)) {
#pragma unroll
      for (int i = 0; i < 4; i++) qv[i] = u4{0, 0, 0, 0};
    }
  }
  // lanes 0..31 read the key scales (lanes 0..15) and zeros (16..31) of
  // channels 8 (lane % 16) .. +7, i.e. of chunk (lane % 16) / 4
  const int kept0 = __builtin_ctz(kmask);
  const int kqa = ((kmask >> kq) & 1u) ? kq : kept0;
  // kept chunks in ascending order, two bits each (uniform)
  uint32_t cmap = 0;
  {
    int n = 0;
#pragma unroll
    for (int m = 0; m < 4; m++)
      if ((kmask >> m) & 1u) {
        cmap |= (uint32_t)m << (2 * n);
        n++;
      }
  }

  const int mla = (lane >= 32 || ((kmask >> ((lane & 15) >> 2)) & 1u))
                      ? (lane & 31) : ((lane & 16) | (kept0 << 2) | (lane & 3));

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
      float a, b;
      io_pair_f32<BF16>(qv[i][e], a, b);
      qmax = fmaxf(qmax, fmaxf(fabsf(a), fabsf(b)));
    }
  qmax = wave_max_kq(qmax);  // over the head's 128 channels (the 4 lanes of column col)
  KVQ_STAMP(tid == 0 && qmax >= 0.0f, 1);
  const int qbexp = (int)((__float_as_uint(qmax) >> 23) & 0xFFu);
  const int qe = qbexp ? min(max(qbexp - 124, -100), 100) : 0;  // largest |q| < 2^(qe - 2)
  const float qsc = __uint_as_float((uint32_t)(127 - qe) << 23);  // 2^-qe
  const float sc_q = scale_log2 * __uint_as_float((uint32_t)(127 + qe) << 23);
  // query as fp16 pairs, scaled (zero past the G heads)
  uint32_t q16[16];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float a, b;
      io_pair_f32<BF16>(qv[i][e], a, b);
      q16[4 * i + e] = hvalid ? pk_rne(a * qsc, b * qsc) : 0u;
    }

  const int T_old = min(max(len, 0), g.max_tokens);  // reads stay inside the cache
  // FUSED: whether this call appends (a full cache or a negative length is
  // reported and decoded as it stands)
  const bool app = FUSED && len >= 0 && len < g.max_tokens;
  const int T = T_old + (app ? 1 : 0);
  const int nq = n_quant(T_old, g.R), ngq = nq / GS;  // FUSED: the prefix before the append
  const int nrb = (T - nq + GS - 1) / GS;
  // This wave's quantized groups are first + i*STR, i < nmine.  Exactly PF
  // group loads are kept in flight (past the end the index is clamped to the
  // wave's last group, or to group 0: cache hits, never used), so the
  // compiler can count outstanding loads and never drains the prefetches.
  const int nmine = first < ngq ? (ngq - first + STR - 1) / STR : 0;
  const int nlast = nmine > 0 ? first + (nmine - 1) * STR : 0;
  auto group_at = [&](int i) { return rec0 + (size_t)min(first + i * STR, nlast); };
  // The nrb ring blocks continue the same order after the groups (block
  // ngq + r), so they fall to waves holding one group fewer than the most;
  // a ring block is worked on first, while the group stream warms up.
  const int ring0 = ((first - ngq) % STR + STR) % STR;

  uint32_t qhi[4] = {0, 0, 0, 0};  // HIMODE 4: 4*q (fp16); HIMODE 16: raw q
  float q4f[8];                    // HIMODE 4: 4*q in fp32
  int sal_ch = 0;                  // HIMODE 4: salient channel whose scale lane%16 copies
  if constexpr (HIMODE != 0) {
    // per-wave tables: this wave's query rows and the salient channels
    // (pairs of rank < n_hi ascending, then the same + 64)
    uint16_t(*wq)[D + 8] = lds.u.loop.q16[wave];
    uint16_t(*wr)[D + 8] = lds.u.loop.qraw[wave];
    int* hil = lds.u.loop.hil[wave];
    if (hvalid) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        *(u4*)&wq[col][32 * kq + 8 * i] = u4{q16[4 * i], q16[4 * i + 1], q16[4 * i + 2], q16[4 * i + 3]};
        if constexpr (HIMODE == 16) {  // raw salient keys meet the scaled query in its io dtype
          u4 r;
#pragma unroll
          for (int e = 0; e < 4; e++) r[e] = scaled_io_pair<BF16>(qv[i][e], qsc);
          *(u4*)&wr[col][32 * kq + 8 * i] = r;
        }
      }
    }
    bool sal = false;
#pragma unroll
    for (int r = 0; r < 8; r++)
      sal |= r < g.n_hi && (__builtin_amdgcn_readfirstlane((int)topv[r >> 2][r & 3]) & 63) == lane;
    const unsigned long long m = __ballot(sal);
    if (lane < 16) hil[lane] = 0;  // stays in range even for a malformed rank table
    if (sal) {
      const int idx = __popcll(m & ((1ull << lane) - 1));
      hil[idx] = lane;
      hil[g.n_hi + idx] = lane + NPAIR;
    }
    // LDS accesses of one wave execute in order: a compiler barrier suffices
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int d = 8 * (kq & 1) + e;
      // HIMODE 4: K-lanes 16..31 (kq 2, 3) repeat the digits of lanes 0..15
      // and carry the rounding residual of 4*q*s; HIMODE 16 uses lanes 0..15
      const bool ok = hvalid && d < g.nh && (HIMODE == 4 || kq < 2);
      const int ch = ok ? (hil[d] & (D - 1)) : 0;
      const float v = ok ? half_bits_to_f32(wq[col][ch]) : 0.0f;
      q4f[e] = 4.0f * v;
      const uint32_t bits = HIMODE == 4 ? (uint32_t)f32_to_half_bits(4.0f * v)
                                        : (ok ? (uint32_t)wr[col][ch] : 0u);
      qhi[e >> 1] |= bits << (16 * (e & 1));
    }
    sal_ch = hil[lane & 15] & (D - 1);
  }

  // PRUNE: each MFMA's 32-long contraction covers one key chunk m.  Lane
  // (col, kq) feeds the pairs 16m + 8(kq/2) + 2b + (kq%2), b = 0..3, of
  // chunk m: the codes of one nibble plane (kq%2) of k_lo word kq/2, in
  // byte order.  qk[i] holds head col's fp16 query at those pairs of the
  // i-th kept chunk.
  const int pb = 8 * (kq >> 1) + (kq & 1);
  uint32_t qk[4][4];
  if constexpr (PRUNE) {
    uint16_t(*wq)[D + 8] = lds.u.loop.q16[wave];
    if constexpr (HIMODE == 0) {
      if (hvalid) {
#pragma unroll
        for (int i = 0; i < 4; i++)
          *(u4*)&wq[col][32 * kq + 8 * i] =
              u4{q16[4 * i], q16[4 * i + 1], q16[4 * i + 2], q16[4 * i + 3]};
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int i = 0; i < KEEP; i++) {
      const int mm = (cmap >> (2 * i)) & 3u;
#pragma unroll
      for (int b = 0; b < 4; b++)
        qk[i][b] = hvalid ? *(const uint32_t*)&wq[col][2 * (16 * mm + pb + 2 * b)] : 0u;
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
  auto softmax_step = [&](const float (&c)[8], float sc, float slack, float (&p)[8]) {
    const float mc = fmaxf(fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3])),
                           fmaxf(fmaxf(c[4], c[5]), fmaxf(c[6], c[7])));
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
    for (int i = 0; i < 8; i++) p[i] = ex2(fmaf(c[i], sc, -m_run));
  };

  uint32_t* sm = lds.u.loop.stage[wave];
  auto process_group = [&](const Pref& cur, size_t rec) {
    // stage the metadata record: [0,64) k scale pairs, [64,128) k zero
    // pairs, [128,192) v scale pairs (j-major), [192,256) v zero pairs.
    // LDS accesses of one wave execute in order, so only the compiler must
    // not move the reads below above this write (a memory fence here would
    // also wait for the prefetches in flight).
    ((u4*)sm)[lane] = cur.meta;
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");

    // keys: q' = q * s (fp16), bias = q . z (the same for every token row);
    // each tile's accumulator starts from the bias, so no VALU adds follow
    uint32_t qs[16], qsl[16];
    f4 cb = {0, 0, 0, 0};
    if constexpr (PRUNE) {
      // kept chunk i's q*s pairs into qs[4i..4i+3]; pruned chunks take no work
#pragma unroll
      for (int i = 0; i < KEEP; i++) {
        const int mm = (cmap >> (2 * i)) & 3u;
        uint32_t zp[4];
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const uint32_t sp = sm[16 * mm + pb + 2 * b];
          zp[b] = sm[64 + 16 * mm + pb + 2 * b];
          qs[4 * i + b] = pk_mul(qk[i][b], sp);
          if constexpr (LO1) {
            const h2 a = u2h(qk[i][b]), bb = u2h(sp), h = u2h(qs[4 * i + b]);
            qsl[4 * i + b] = pk_rne(fmaf((float)a[0], (float)bb[0], -(float)h[0]),
                                    fmaf((float)a[1], (float)bb[1], -(float)h[1]));
          }
        }
        cb = mma_f16(u4{zp[0], zp[1], zp[2], zp[3]}, u4{qk[i][0], qk[i][1], qk[i][2], qk[i][3]},
                     cb);
      }
    } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const u4 sv = ((const u4*)(sm + 16 * kq))[i];
      const u4 zv = ((const u4*)(sm + 64 + 16 * kq))[i];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        qs[4 * i + e] = pk_mul(q16[4 * i + e], sv[e]);
        if constexpr (LO1) {
          // q*s is exact in fp32: its residual after the fp16 rounding
          const h2 a = u2h(q16[4 * i + e]), b = u2h(sv[e]), h = u2h(qs[4 * i + e]);
          qsl[4 * i + e] = pk_rne(fmaf((float)a[0], (float)b[0], -(float)h[0]),
                                  fmaf((float)a[1], (float)b[1], -(float)h[1]));
        }
      }
      const u4 qb = u4{q16[4 * i], q16[4 * i + 1], q16[4 * i + 2], q16[4 * i + 3]};
      cb = mma_f16(zv, qb, cb);
    }
    }
    uint32_t qshi[4];
    if constexpr (HIMODE == 4) {
      // the salient channels' scales, gathered once into a contiguous row
      // (lane l copies digit l%16), then read 8 at a time
      uint16_t* ss = lds.u.loop.sal_s[wave];
      ss[lane & 15] = ((const uint16_t*)sm)[sal_ch];
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
      const u4 spv = *(const u4*)(ss + 8 * (kq & 1));
#pragma unroll
      for (int e = 0; e < 4; e++) {
        // 4*q*s is exact in fp32; split it into its fp16 rounding hi and the
        // fp16 residual lo
        const uint32_t sp = spv[e];
        const uint32_t hi = pk_mul(qhi[e], sp);
        const h2 sh = u2h(sp), hh = u2h(hi);
        const uint32_t lo = pk_rne(fmaf(q4f[2 * e], (float)sh[0], -(float)hh[0]),
                                   fmaf(q4f[2 * e + 1], (float)sh[1], -(float)hh[1]));
        qshi[e] = kq < 2 ? hi : lo;
      }
    }
    f4 C[2];
#pragma unroll
    for (int TT = 0; TT < 2; TT++) {
      f4 acc = cb;
      if constexpr (PRUNE) {
        const int sh = 2 * (kq & 1);
#pragma unroll
        for (int i = 0; i < KEEP; i++) {
          const uint32_t x = (cur.klc[TT][i] >> sh) & 0x33333333u;
          const u4 cd = u4{cvt2<0>(x), cvt2<1>(x), cvt2<2>(x), cvt2<3>(x)};
          acc = mma_f16(cd, u4{qs[4 * i], qs[4 * i + 1], qs[4 * i + 2], qs[4 * i + 3]}, acc);
          if constexpr (LO1)
            acc = mma_f16(cd, u4{qsl[4 * i], qsl[4 * i + 1], qsl[4 * i + 2], qsl[4 * i + 3]}, acc);
        }
      } else {
      const u2 w = cur.klo[TT];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const uint32_t A = w[u] & 0x33333333u, Bn = (w[u] >> 2) & 0x33333333u;
        const int k0 = 8 * u;
        const u4 c0 = u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)};
        const u4 c1 = u4{cvt2<2>(A), cvt2<2>(Bn), cvt2<3>(A), cvt2<3>(Bn)};
        acc = mma_f16(c0, u4{qs[k0], qs[k0 + 1], qs[k0 + 2], qs[k0 + 3]}, acc);
        acc = mma_f16(c1, u4{qs[k0 + 4], qs[k0 + 5], qs[k0 + 6], qs[k0 + 7]}, acc);
        if constexpr (LO1) {
          acc = mma_f16(c0, u4{qsl[k0], qsl[k0 + 1], qsl[k0 + 2], qsl[k0 + 3]}, acc);
          acc = mma_f16(c1, u4{qsl[k0 + 4], qsl[k0 + 5], qsl[k0 + 6], qsl[k0 + 7]}, acc);
        }
      }
      }
      if constexpr (HIMODE == 4) {
        const uint32_t wsel = (kq & 1) ? cur.khi[TT] >> 16 : cur.khi[TT];
        const uint32_t A = wsel & 0x33333333u, Bn = (wsel >> 2) & 0x33333333u;
        acc = mma_f16(u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)},
                      u4{qshi[0], qshi[1], qshi[2], qshi[3]}, acc);
      }
      if constexpr (HIMODE == 16) {
        u4 a = cur.hraw[TT];
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
    for (int i = 0; i < 8; i++) cr[i] = C[i >> 2][i & 3];
    // lanes 32..47 staged the group's value scales (non-negative fp16, so
    // their bits order as integers)
    const uint32_t vs2 = pk_max_u16(pk_max_u16(cur.meta[0], cur.meta[1]),
                                    pk_max_u16(cur.meta[2], cur.meta[3]));
    const bool wide = lane >= 32 && lane < 48 && max(vs2 & 0xFFFFu, vs2 >> 16) > VSCALE_WIDE;
    softmax_step(cr, sc_q, __builtin_amdgcn_ballot_w64(wide) ? RESCALE_SLACK_WIDE : RESCALE_SLACK,
                 p);
    const u4 P = u4{pk_rne(p[0], p[1]), pk_rne(p[2], p[3]), pk_rne(p[4], p[5]), pk_rne(p[6], p[7])};
    // values
    const bool vkept = VHI && kq < g.n_vhi;
    const u4 za = col < 4 ? ((const u4*)(sm + 192 + 16 * col))[kq]
                          : (col == 4 ? u4{ONES, ONES, ONES, ONES} : u4{0, 0, 0, 0});
    Cvb = mma_f16(za, P, Cvb);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const u4 sv = ((const u4*)(sm + 128 + 16 * j))[kq];
      const u4 pj = u4{pk_mul(P[0], sv[0]), pk_mul(P[1], sv[1]), pk_mul(P[2], sv[2]),
                       pk_mul(P[3], sv[3])};
      const uint32_t wv = cur.vc[j];
      const uint32_t A = wv & 0x33333333u, Bn = (wv >> 2) & 0x33333333u;
      O[2 * j] = mma_f16(u4{cvt2<0>(A), cvt2<0>(Bn), cvt2<1>(A), cvt2<1>(Bn)}, pj, O[2 * j]);
      O[2 * j + 1] = mma_f16(u4{cvt2<2>(A), cvt2<2>(Bn), cvt2<3>(A), cvt2<3>(Bn)}, pj, O[2 * j + 1]);
      if constexpr (VHI) {
        // block kq's high digits (0 past the high-precision blocks), weighted
        // 4 by the convert
        const uint32_t wh = vkept ? cur.vh[j] : 0u;
        const uint32_t Ah = wh & 0x33333333u, Bh = (wh >> 2) & 0x33333333u;
        O[2 * j] = mma_f16(u4{cvt2x4<0>(Ah), cvt2x4<0>(Bh), cvt2x4<1>(Ah), cvt2x4<1>(Bh)}, pj,
                           O[2 * j]);
        O[2 * j + 1] = mma_f16(u4{cvt2x4<2>(Ah), cvt2x4<2>(Bh), cvt2x4<3>(Ah), cvt2x4<3>(Bh)}, pj,
                               O[2 * j + 1]);
      }
    }
  };

  // ring blocks (16-bit keys and values) of this wave: blocks n < nrb.  Key
  // and value tiles are requested together (one round trip); the query is
  // the raw one already in registers.
  for (int n = ring0; n < nrb; n += STR) {
    const int pbase = nq + GS * n;
    const int nvalid = min(GS, T - pbase);
    const int sb = (pbase / GS) % (g.RS / GS);
    const uint16_t* rk = (const uint16_t*)c.ring_k + ((size_t)bh * g.RS + sb * GS) * D;
    const uint16_t* rv = (const uint16_t*)c.ring_v + (((size_t)bh * (g.RS / GS) + sb) * D) * GS;
    // FUSED: the appended token's index in this block (-1 if not here); its
    // key row and value column come from knew / vnew, not from the ring
    const int tnew = app ? T_old - pbase : -1;
    u4 kt[2][4], vt[8];
#pragma unroll
    for (int TT = 0; TT < 2; TT++) {
      const int tok = tile_token(16 * TT + col);
      const u4* kr = (const u4*)(rk + (size_t)tok * D + 32 * kqa);
      if constexpr (FUSED)
        if (tok == tnew) kr = (const u4*)(knew + (size_t)bh * D + 32 * kqa);
#pragma unroll
      for (int k = 0; k < 4; k++) kt[TT][k] = kr[k];
    }
#pragma unroll
    for (int tt = 0; tt < 8; tt++) vt[tt] = *(const u4*)(rv + (size_t)(16 * tt + col) * GS + 8 * kq);
    if constexpr (FUSED) {
      const int dt = tnew - 8 * kq;  // the new token among this lane's 8 slots
      if (dt >= 0 && dt < 8) {
#pragma unroll
        for (int tt = 0; tt < 8; tt++) {
          const uint32_t x = vnew[(size_t)bh * D + 16 * tt + col];
          const int e = dt >> 1, sh = 16 * (dt & 1);
          const uint32_t m = 0xFFFFu << sh;
#pragma unroll
          for (int i = 0; i < 4; i++)
            if (i == e) vt[tt][i] = (vt[tt][i] & ~m) | (x << sh);
        }
      }
    }
    uint32_t qraw[16];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int e = 0; e < 4; e++) qraw[4 * i + e] = hvalid ? qv[i][e] : 0u;
    f4 C[2];
#pragma unroll
    for (int TT = 0; TT < 2; TT++) {
      f4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 4; k++)
        acc = mma_raw<BF16>(kt[TT][k],
                            u4{qraw[4 * k], qraw[4 * k + 1], qraw[4 * k + 2], qraw[4 * k + 3]}, acc);
      C[TT] = acc;
    }
    float cr[8], p[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int t = 8 * kq + 4 * (i >> 2) + (i & 3);
      cr[i] = t < nvalid ? C[i >> 2][i & 3] : -INFINITY;
    }
    softmax_step(cr, scale_log2, RESCALE_SLACK, p);  // raw values: the products stay in fp32
#pragma unroll
    for (int i = 0; i < 8; i++) l_raw += p[i];
    uint32_t Ph[4], Pl[4];
#pragma unroll
    for (int i = 0; i < 4; i++) split_pair<BF16>(p[2 * i], p[2 * i + 1], Ph[i], Pl[i]);
#pragma unroll
    for (int tt = 0; tt < 8; tt++) {
      u4 a = vt[tt];
      // zero slots past the last token (they may hold stale data)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int t0 = 8 * kq + 2 * e;
        const uint32_t keep =
            (t0 < nvalid ? 0x0000ffffu : 0u) | (t0 + 1 < nvalid ? 0xffff0000u : 0u);
        a[e] &= keep;
      }
      O[tt] = mma_raw<BF16>(a, u4{Ph[0], Ph[1], Ph[2], Ph[3]}, O[tt]);
      O[tt] = mma_raw<BF16>(a, u4{Pl[0], Pl[1], Pl[2], Pl[3]}, O[tt]);
    }
  }

  KVQ_STAMP(tid == 0, 2);
  if constexpr (HASQ) {
    if constexpr (PRUNE) {
      // the first prefetched groups hold all four chunks in chunk order:
      // move the kept ones to slots 0 .. KEEP-1 (slot i reads chunk >= i).
      // Done here, after the ring blocks, so that waiting for these loads
      // does not hold up the set-up work above.
#pragma unroll
      for (int k = 0; k < PF; k++)
#pragma unroll
        for (int TT = 0; TT < 2; TT++)
#pragma unroll
          for (int i = 0; i < KEEP; i++) {
            const uint32_t mm = (cmap >> (2 * i)) & 3u;
            const uint32_t* a = pf[k].klc[TT];
            pf[k].klc[TT][i] = mm == 0 ? a[0] : mm == 1 ? a[1] : mm == 2 ? a[2] : a[3];
          }
    }
    for (int i = 0; i < nmine; i += PF) {
#pragma unroll
      for (int k = 0; k < PF; k++) {
        if (i + k < nmine) process_group(pf[k], group_at(i + k));
#ifdef KVQ_STAMPS
        if (i + k == 0) KVQ_STAMP(tid == 0 && O[0][0] != 12345.0f, 11);
#endif
        load_group<HIMODE, PRUNE, KEEP, VHI>(c, group_at(i + k + PF), lane, col, kq, kqa, mla,
                                             cmap, g.nh, g.n_vhi, pf[k]);
      }
    }
  }

  // ---- merge the waves: per head m, l and unnormalized o
  KVQ_STAMP(lane == 0 && O[0][0] != 12345.0f, 3 + wave);
  __syncthreads();  // every wave is done with the loop-phase LDS
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
  // split record: (m, l) and o / l, fp32; thread -> (head, 8 channels).
  // Records cross workgroups (and L2 slices): every access to them is
  // device-coherent (sc1), so no cache-wide writeback or invalidate is needed.
  const size_t rbh = (size_t)bh * S * G;  // first record of this (sequence, KV head)
  const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(
      ws.o + rbh * D, 0, (int)(S * G * D * 4), BUF_RSRC_WORD3);
  for (int i = tid; i < G * (D / 8); i += WG_THREADS) {
    const int h = i / (D / 8), c8 = 8 * (i % (D / 8));
    float M = lds.u.merge.m[0][h];
#pragma unroll
    for (int w = 1; w < NW; w++) M = fmaxf(M, lds.u.merge.m[w][h]);
    f4 oa = {0, 0, 0, 0}, ob = {0, 0, 0, 0};
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      const float mw = lds.u.merge.m[w][h];
      const float a = mw == -INFINITY ? 0.0f : ex2(mw - M);
      oa += a * *(const f4*)&lds.u.merge.o[w][h][c8];
      ob += a * *(const f4*)&lds.u.merge.o[w][h][c8 + 4];
      l += a * lds.u.merge.l[w][h];
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int ooff = ((s * G + h) * D + c8) * 4;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, oa * inv), rs_o, ooff, 0, CPOL_SC1);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, ob * inv), rs_o, ooff + 16, 0,
                                           CPOL_SC1);
    if (c8 == 0)
      __hip_atomic_store((uint64_t*)&ws.ml[rbh + (size_t)s * G + h],
                         (uint64_t)__float_as_uint(M) | ((uint64_t)__float_as_uint(l) << 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- the last workgroup of this (sequence, KV head) merges all splits.
  // Every record store has completed (s_waitcnt) before the counter moves.
  KVQ_STAMP(tid == 0, 12);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  KVQ_STAMP(tid == 0, 13);
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&ws.tick[(size_t)bh * TICK_STRIDE], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    lds.last = prev == (uint32_t)(S - 1);
#ifdef KVQ_STAMPS
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    ws.st[(size_t)blockIdx.x * STAMP_SLOTS + 14] = __builtin_amdgcn_s_memrealtime() + 0 * prev;
    ws.st[(size_t)blockIdx.x * STAMP_SLOTS + 17] =
        (unsigned long long)bh | ((unsigned long long)s << 16) | ((unsigned long long)xcc << 32) |
        ((unsigned long long)prev << 40);
#endif
    if constexpr (FUSED) lds.first = prev == 0u;
  }
  __syncthreads();
  if constexpr (FUSED) {
    // the first workgroup to finish does the append's ring write and packing
    // while the others still run: nothing in this call reads the packed
    // records, and the token's ring slot held a quantized position (T_old -
    // RS < nq), which no wave reads from the ring (the new token itself
    // comes from knew / vnew).  The length is stored by the last workgroup,
    // after every workgroup has read it.
    if (lds.first && app) {
      const int slot = T_old % g.RS;
      if (tid < D) {
        uint16_t* rk = (uint16_t*)c.ring_k + (size_t)bh * g.RS * D;
        uint16_t* rv = (uint16_t*)c.ring_v + (size_t)bh * g.RS * D;
        rk[(size_t)slot * D + tid] = knv;
        rv[((size_t)(slot / GS) * D + tid) * GS + slot % GS] = vnv;
      }
      // the group [nq, nq + 32) ends at T - R <= T_old: the new token is not in it
      if (n_quant(T, g.R) > nq && tid < 128)
        pack_ring_group<BF16, VHI>(g, c, bh, nq, tid, lds.u.pack);
    }
  }
  if (!lds.last) return;
  // item = (head, 8 channels); nsub lanes (a power of two, within one wave)
  // share an item's splits, each loading up to 8 records at once, and
  // reduce with shuffles
  const int items = G * (D / 8);
  int nsub = 1;
  while (nsub < 64 && items * nsub * 2 <= WG_THREADS) nsub *= 2;
  const uint64_t* mlb = (const uint64_t*)(ws.ml + rbh);
  {
    const int t = tid;
    const int item = t / nsub, sub = t % nsub;
    const bool act = item < items;
    const int h = act ? item / (D / 8) : 0, c8 = act ? 8 * (item % (D / 8)) : 0;
    float M = -INFINITY, L = 0.0f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // a batch: KB records per lane requested at once, then merged in order
    // (each as it arrives); indices past S repeat the last record and are
    // skipped
    auto batch = [&](auto kb, int i0) {
      constexpr int KB = decltype(kb)::value;
      uint64_t mlw[KB];
      u4 ov[KB][2];
#pragma unroll
      for (int k = 0; k < KB; k++) {
        const int i = min(i0 + k * nsub, S - 1);
        mlw[k] = __hip_atomic_load(mlb + (size_t)i * G + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int ooff = ((i * G + h) * D + c8) * 4;
        ov[k][0] = __builtin_amdgcn_raw_buffer_load_b128(rs_o, ooff, 0, CPOL_SC1);
        ov[k][1] = __builtin_amdgcn_raw_buffer_load_b128(rs_o, ooff + 16, 0, CPOL_SC1);
      }
#pragma unroll
      for (int k = 0; k < KB; k++) {
        const float m = __uint_as_float((uint32_t)mlw[k]);
        const float l = __uint_as_float((uint32_t)(mlw[k] >> 32));
        if (i0 + k * nsub >= S || m == -INFINITY) continue;
        if (m > M) {
          const float a = ex2(M - m);
          L *= a;
#pragma unroll
          for (int e = 0; e < 8; e++) acc[e] *= a;
          M = m;
        }
        const float wgt = ex2(m - M) * l;
        L += wgt;
#pragma unroll
        for (int e = 0; e < 8; e++) acc[e] += wgt * __uint_as_float(ov[k][e >> 2][e & 3]);
      }
    };
    if (S <= 4 * nsub) {  // one batch of 4 covers every split
      if (act) batch(std::integral_constant<int, 4>{}, sub);
    } else {
      for (int i0 = sub; act && i0 < S; i0 += 8 * nsub) batch(std::integral_constant<int, 8>{}, i0);
    }
    for (int o = 1; o < nsub; o <<= 1) {
      const float M2 = __shfl_xor(M, o), L2 = __shfl_xor(L, o);
      const float Mn = fmaxf(M, M2);
      const float a1 = M == -INFINITY ? 0.0f : ex2(M - Mn);
      const float a2 = M2 == -INFINITY ? 0.0f : ex2(M2 - Mn);
      L = L * a1 + L2 * a2;
#pragma unroll
      for (int e = 0; e < 8; e++) acc[e] = acc[e] * a1 + __shfl_xor(acc[e], o) * a2;
      M = Mn;
    }
    if (act && sub == 0) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      uint16_t* op = out + ((size_t)b * g.Hq + kh * G + h) * D + c8;
      uint16_t bits[8];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float v = acc[e] * inv;
        if constexpr (BF16) {
          const uint32_t u = __float_as_uint(v);
          bits[e] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
        } else {
          bits[e] = f32_to_half_bits(v);
        }
      }
      *(u4*)op = u4{bits[0] | ((uint32_t)bits[1] << 16), bits[2] | ((uint32_t)bits[3] << 16),
                    bits[4] | ((uint32_t)bits[5] << 16), bits[6] | ((uint32_t)bits[7] << 16)};
    }
  }
  KVQ_STAMP(tid == 0, 15);
#ifdef KVQ_STAMPS
  __builtin_amdgcn_s_waitcnt(0);
  KVQ_STAMP(tid == 0, 16);
#endif
  if (tid == 0)  // ready for the next call
    __hip_atomic_store(&ws.tick[(size_t)bh * TICK_STRIDE], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if constexpr (FUSED) {
    // the append's length (or its error): every workgroup of this (sequence,
    // KV head) has read the length before it took its ticket
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

template <bool BF16, int HIMODE, bool LO1, int KEEP, bool VHI, bool FUSED>
static void launch_one(const Geo& g, const Launch& a) {
  const dim3 grid(g.B * g.Hkv * a.S), block(WG_THREADS);
  if (g.NG > 0)
    hipLaunchKernelGGL((decode_kernel<BF16, HIMODE, true, LO1, KEEP, VHI, FUSED>), grid, block, 0,
                       a.st, g, (const uint16_t*)a.q, *a.c, a.scale_log2, a.S, a.ws,
                       (uint16_t*)a.out, (const uint16_t*)a.knew, (const uint16_t*)a.vnew);
  else
    hipLaunchKernelGGL((decode_kernel<BF16, HIMODE, false, LO1, KEEP, false, FUSED>), grid, block,
                       0, a.st, g, (const uint16_t*)a.q, *a.c, a.scale_log2, a.S, a.ws,
                       (uint16_t*)a.out, (const uint16_t*)a.knew, (const uint16_t*)a.vnew);
}

// keep 0: the fused append-and-decode call (all four key chunks)
template <bool BF16, int HIMODE, bool LO1, bool VHI>
static void launch_keep(const Geo& g, int keep, const Launch& a) {
  switch (keep) {
    case 0: launch_one<BF16, HIMODE, LO1, 4, VHI, true>(g, a); break;
    case 1: launch_one<BF16, HIMODE, LO1, 1, VHI, false>(g, a); break;
    case 2: launch_one<BF16, HIMODE, LO1, 2, VHI, false>(g, a); break;
    case 3: launch_one<BF16, HIMODE, LO1, 3, VHI, false>(g, a); break;
    default: launch_one<BF16, HIMODE, LO1, 4, VHI, false>(g, a); break;
  }
}

// Two value precisions touch only the value side and pruning only the key
// side, so every combination has its own kernel.
template <bool BF16, int HIMODE>
static void launch_lo1(const Geo& g, int keep, const Launch& a) {
  if (g.n_lo1 > 0) {
    if (g.n_vhi > 0) launch_keep<BF16, HIMODE, true, true>(g, keep, a);
    else launch_keep<BF16, HIMODE, true, false>(g, keep, a);
  } else {
    if (g.n_vhi > 0) launch_keep<BF16, HIMODE, false, true>(g, keep, a);
    else launch_keep<BF16, HIMODE, false, false>(g, keep, a);
  }
}

template <bool BF16>
hipError_t launch_decode_io(const Geo& g, int keep, const Launch& a) {
  const int hm = g.n_hi == 0 ? 0 : g.bits_hi;
  if (hm == 0) launch_lo1<BF16, 0>(g, keep, a);
  else if (hm == 4) launch_lo1<BF16, 4>(g, keep, a);
  else launch_lo1<BF16, 16>(g, keep, a);
  return hipGetLastError();
}

// The file is compiled twice so that the two halves of the kernel variants
// build in parallel: KVQ_DECODE_PART 0 holds the fp16 kernels, 1 the bf16
// kernels and the entry points.
#if KVQ_DECODE_PART == 0
template hipError_t launch_decode_io<false>(const Geo&, int, const Launch&);
#else
extern template hipError_t launch_decode_io<false>(const Geo&, int, const Launch&);

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int S) {
  size_t n = ws_tick_bytes(B, Hkv) + ws_ml_bytes(B, Hq, S) + ws_o_bytes(B, Hq, S);
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
                               ws_ml_bytes(g.B, g.Hq, S) + ws_o_bytes(g.B, g.Hq, S));
#endif
  const Launch a{q, c, sm_scale * 1.4426950408889634f, S, w, out, k_new, v_new, st};
  return g.bf16 ? launch_decode_io<true>(g, keep, a) : launch_decode_io<false>(g, keep, a);
}
#endif

}  // namespace kvq
