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

}  // namespace kvq
