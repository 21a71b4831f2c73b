// ceiling.hip — the read ceiling of decode attention.
//
// A kernel with the decode kernel's grid, workgroup-to-XCD mapping, wave
// work split and group stream (stream.h): every wave reads exactly the bytes
// its decode counterpart reads — its ring blocks into registers, its
// quantized groups by direct global->LDS copies into the same per-wave slots
// with the same waits — and does no arithmetic on them beyond one word per
// group folded into a checksum.  Decode cost is the read of the cache
// (PN-Mix and Dual-QK, abstracts), so the time of this kernel on the same
// cache is the floor a decode step can reach with these load shapes; the
// decode kernel's time above it is its arithmetic, softmax and merges.
#include "common.h"
#include "internal.h"
#include "stream.h"

namespace kvq {

typedef uint32_t cu4 __attribute__((ext_vector_type(4)));

template <int HIMODE, bool VHI, bool DENSE1>
__global__ __launch_bounds__(WG_THREADS) void ceiling_kernel(Geo g, kvq_cache c, int S,
                                                             uint32_t* sink) {
  using SC = SlotCfg<HIMODE, VHI>;
  constexpr int NSLOT = SC::NSLOT, NLD = SC::NLD, SLOTB = SC::BYTES;
  __shared__ __align__(16) uint8_t slots[NW][NSLOT][SLOTB];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // the decode kernel's mapping: with (sequence, KV head) count a multiple of
  // 8 the splits of one (sequence, KV head) share an XCD
  const bool xmap = (g.B * g.Hkv) % 8 == 0;
  const int bh = xmap ? (int)(blockIdx.x % 8) + 8 * (int)((blockIdx.x / 8) / S)
                      : (int)(blockIdx.x / S);
  const int s = xmap ? (int)((blockIdx.x / 8) % S) : (int)(blockIdx.x % S);
  const int RSB = g.RS / GS, STR = S * NW, f = s + S * wave;
  const bool ring_owner = f < RSB;
  const int gfirst = f - RSB + (ring_owner ? (RSB - f + STR - 1) / STR * STR : 0);
  const size_t rec0 = (size_t)bh * g.NG;
  uint8_t* sl = &slots[wave][0][0];
  uint32_t acc = 0;
  auto issue_first = [&]() {
    if (g.NG > 0) {
#pragma unroll
      for (int i = 0; i < NSLOT; i++)
        issue_group<HIMODE, VHI, false, DENSE1>(c, rec0 + (size_t)min(gfirst + i * STR, g.NG - 1),
                                        sl + i * SLOTB, lane, 0xFFu, 0, g.nh, g.n_vhi);
    }
  };
  if (!ring_owner) issue_first();
  const int len = load_uniform(c.len + bh);
  const int T = min(max(len, 0), g.max_tokens);
  const int ngq = n_quant(T, g.R) / GS;
  // ring blocks rb = f, f + STR, ...: 32 slots of 256-byte key rows and the
  // block's [128][32] value columns, 16 KB, read whole as the decode does
  for (int rb = f; ring_owner && rb < RSB; rb += STR) {
    const cu4* rk = (const cu4*)((const uint16_t*)c.ring_k + ((size_t)bh * g.RS + rb * GS) * D);
    const cu4* rv = (const cu4*)((const uint16_t*)c.ring_v + ((size_t)bh * RSB + rb) * D * GS);
    cu4 x[16];
#pragma unroll
    for (int k = 0; k < 8; k++) {
      x[k] = rk[lane + 64 * k];
      x[8 + k] = rv[lane + 64 * k];
    }
#pragma unroll
    for (int k = 0; k < 16; k++) acc ^= x[k][0] ^ x[k][3];
  }
  if (ring_owner) issue_first();
  const int nmine = (g.NG > 0 && gfirst < ngq) ? (ngq - 1 - gfirst) / STR + 1 : 0;
  int issued = g.NG > 0 ? NSLOT : 0;
  for (int i = 0; i < nmine; i++) {
    wait_slot<NLD, NSLOT>(issued - 1 - i);
    uint8_t* slot = sl + (i % NSLOT) * SLOTB;
    acc ^= ((const uint32_t*)slot)[lane];
    if (issued < nmine) {
      wait_lgkmcnt0();  // the slot's read is done before its refill lands
      compiler_fence();
      issue_group<HIMODE, VHI, false, DENSE1>(c, rec0 + gfirst + (size_t)issued * STR, slot, lane, 0xFFu,
                                      0, g.nh, g.n_vhi);
      issued++;
    }
  }
  wait_vmcnt<0>();  // copies past this wave's groups (clamped first copies) drained
  compiler_fence();
  // a store that almost never happens keeps every read live
  if (acc == 0x9E3779B9u) sink[0] = acc ^ (uint32_t)tid;
}

template <int HIMODE, bool DENSE1>
static void launch_ceiling_h(const Geo& g, const kvq_cache& c, int S, uint32_t* sink,
                             hipStream_t st) {
  const dim3 grid(g.B * g.Hkv * S);
  if (g.n_vhi > 0)
    hipLaunchKernelGGL((ceiling_kernel<HIMODE, true, DENSE1>), grid, dim3(WG_THREADS), 0, st, g,
                       c, S, sink);
  else
    hipLaunchKernelGGL((ceiling_kernel<HIMODE, false, DENSE1>), grid, dim3(WG_THREADS), 0, st, g,
                       c, S, sink);
}

hipError_t launch_ceiling(const Geo& g, const kvq_cache* c, int S, void* sink, hipStream_t st) {
  const int hm = g.n_hi == 0 ? 0 : g.bits_hi;
  if (hm == 0 && g.dense1) launch_ceiling_h<0, true>(g, *c, S, (uint32_t*)sink, st);
  else if (hm == 0) launch_ceiling_h<0, false>(g, *c, S, (uint32_t*)sink, st);
  else if (hm == 4) launch_ceiling_h<4, false>(g, *c, S, (uint32_t*)sink, st);
  else launch_ceiling_h<16, false>(g, *c, S, (uint32_t*)sink, st);
  return hipGetLastError();
}

// ---- issue probe.  The decode loop is made of integer VALU (code masks),
// v_cvt_scalef32_pk_f16_fp4 (codes to fp16), packed fp16 multiplies (the
// exact q*s and p*s pairs), v_exp_f32 (softmax weights) and
// v_mfma_f32_16x16x32_f16; this kernel runs each kind alone, and MFMA with
// integer VALU in one loop, so that their issue cost per SIMD and whether a
// SIMD overlaps MFMA with VALU can be read from the launch times.  Every
// thread folds its registers into one word of `out` (which keeps every
// instruction live).
typedef _Float16 ph2 __attribute__((ext_vector_type(2)));
typedef _Float16 ph4 __attribute__((ext_vector_type(4)));
typedef _Float16 ph8 __attribute__((ext_vector_type(8)));
typedef float pf4 __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(PROBE_THREADS) void issue_probe_kernel(uint32_t* out) {
  const uint32_t gid = blockIdx.x * PROBE_THREADS + threadIdx.x;
  uint32_t x[16];
  float fx[16];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    x[i] = 0x9E3779B9u * (gid + 7u * i) + i;
    fx[i] = (float)(x[i] & 255u) * 0.001f;
  }
  pf4 acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  const ph8 a = __builtin_bit_cast(ph8, cu4{x[0], x[1], x[2], x[3]});
  for (int it = 0; it < PROBE_ITERS; it++) {
    if constexpr (KIND == 4 || KIND == 5) {  // 4 MFMA, independent accumulators
#pragma unroll
      for (int i = 0; i < 4; i++) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, a, acc[i], 0, 0, 0);
    }
    if constexpr (KIND == 6) {  // 4 MFMA of half the contraction length (K = 16)
      const ph4 a4 = __builtin_shufflevector(a, a, 0, 1, 2, 3);
#pragma unroll
      for (int i = 0; i < 4; i++) acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, a4, acc[i], 0, 0, 0);
    }
    if constexpr (KIND == 0 || KIND == 5) {  // 16 v_add_u32 + 16 v_xor_b32
#pragma unroll
      for (int i = 0; i < 16; i++) x[i] = x[i] ^ (x[(i + 1) & 15] + (uint32_t)it);
    } else if constexpr (KIND == 1) {  // 16 v_cvt_scalef32_pk_f16_fp4 + 16 v_xor_b32
#define KVQ_PROBE_CVT(i, sel)                                                                \
  x[i] ^= __builtin_bit_cast(uint32_t,                                                       \
                             __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x[(i + 3) & 15], 2.0f, sel));
      KVQ_PROBE_CVT(0, 0) KVQ_PROBE_CVT(1, 1) KVQ_PROBE_CVT(2, 2) KVQ_PROBE_CVT(3, 3)
      KVQ_PROBE_CVT(4, 0) KVQ_PROBE_CVT(5, 1) KVQ_PROBE_CVT(6, 2) KVQ_PROBE_CVT(7, 3)
      KVQ_PROBE_CVT(8, 0) KVQ_PROBE_CVT(9, 1) KVQ_PROBE_CVT(10, 2) KVQ_PROBE_CVT(11, 3)
      KVQ_PROBE_CVT(12, 0) KVQ_PROBE_CVT(13, 1) KVQ_PROBE_CVT(14, 2) KVQ_PROBE_CVT(15, 3)
#undef KVQ_PROBE_CVT
    } else if constexpr (KIND == 2) {  // 16 v_pk_mul_f16
#pragma unroll
      for (int i = 0; i < 16; i++)
        x[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(ph2, x[i]) *
                                                __builtin_bit_cast(ph2, x[(i + 5) & 15]));
    } else if constexpr (KIND == 3) {  // 16 v_exp_f32 + 16 v_mul_f32
#pragma unroll
      for (int i = 0; i < 16; i++) fx[i] = __builtin_amdgcn_exp2f(fx[(i + 1) & 15]) * 0.5f;
    }
  }
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) r ^= x[i] ^ __float_as_uint(fx[i]);
#pragma unroll
  for (int i = 0; i < 4; i++) r ^= __float_as_uint(acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3]);
  out[gid] = r;
}

hipError_t launch_issue_probe(int kind, int n_blocks, void* out, hipStream_t st) {
  const dim3 grid(n_blocks), block(PROBE_THREADS);
  uint32_t* o = (uint32_t*)out;
  switch (kind) {
    case 0: hipLaunchKernelGGL(issue_probe_kernel<0>, grid, block, 0, st, o); break;
    case 1: hipLaunchKernelGGL(issue_probe_kernel<1>, grid, block, 0, st, o); break;
    case 2: hipLaunchKernelGGL(issue_probe_kernel<2>, grid, block, 0, st, o); break;
    case 3: hipLaunchKernelGGL(issue_probe_kernel<3>, grid, block, 0, st, o); break;
    case 4: hipLaunchKernelGGL(issue_probe_kernel<4>, grid, block, 0, st, o); break;
    case 5: hipLaunchKernelGGL(issue_probe_kernel<5>, grid, block, 0, st, o); break;
    default: hipLaunchKernelGGL(issue_probe_kernel<6>, grid, block, 0, st, o); break;
  }
  return hipGetLastError();
}

}  // namespace kvq
