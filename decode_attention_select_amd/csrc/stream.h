// stream.h — the decode kernel's group stream: direct global->LDS copies of
// each quantized group's records into per-wave LDS slots, and the waits on
// them.  Shared by the decode kernel and the read-ceiling kernel, so that the
// two read the same bytes in the same shapes.
#pragma once

#include "common.h"

namespace kvq {

#ifndef KVQ_DECODE_WAVES
#define KVQ_DECODE_WAVES 8
#endif
constexpr int NW = KVQ_DECODE_WAVES;   // waves per workgroup (one workgroup per CU)
constexpr int WG_THREADS = 64 * NW;

// Buffer descriptor word 3 for raw byte-addressed buffers (gfx9 family), and
// the cache-policy bit that makes a buffer access device-coherent (sc1).
constexpr int BUF_RSRC_WORD3 = 0x00020000;
constexpr int CPOL_SC1 = 16;
constexpr int CPOL_SC0 = 1;  // bypasses the CU's L1 only: reads what the XCD's L2 holds
// non-temporal: the streamed group records go through the L2 with the
// streaming policy, so that they do not push out what is reused there (the
// kernel's code, the split records)
constexpr int CPOL_NT = 2;

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0) (LDS and scalar memory), vmcnt and expcnt left alone.
__device__ inline void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// Keeps the compiler from moving memory accesses across this point (the
// direct global->LDS copies are invisible to its LDS dependence tracking).
__device__ inline void compiler_fence() { asm volatile("" ::: "memory"); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;
// One direct global->LDS copy: every active lane moves the 16 bytes at `src`
// to LDS address `dst` + 16 * lane (dst uniform).
template <int CPOL = 0>
__device__ inline void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)dst, 16, 0, CPOL);
}

// One LDS slot holds the records of one quantized group, copied from HBM by
// direct loads (16 bytes per lane and instruction):
//   KLO  [0, 1024)     k_lo
//   META [1024, 2048)  k_meta (512) then v_meta (512): words [16w, 16w+8)
//                      the scale pairs and [16w+8, 16w+16) the zero pairs of
//                      key run w (channels 16w ..), [128,192) value scale
//                      pairs (j-major), [192,256) value zero pairs
//   VC   [2048, 3072)  v_codes
//   KHI  1024 bytes: k_hi (HIMODE 4 its 128 bytes, HIMODE 16 its 64 nh bytes)
//   VH   1024 bytes: v_hi words 8 .. 8 + 64 n_vhi (VHI only)
// Every copy is a whole-wave instruction (NLD per group), so that the
// compiler counts each one in its own waits: lanes past a short record copy
// 16 bytes of it again into the slack after it, which nothing reads.  NSLOT
// slots per wave within the LDS budget.
constexpr int SLOT_LDS_BUDGET = 147456;
template <int HIMODE, bool VHI>
struct SlotCfg {
  static constexpr int KLO = 0, META = 1024, VC = 2048, KHI = 3072;
  static constexpr int VH = KHI + (HIMODE != 0 ? 1024 : 0);
  static constexpr int BYTES = VH + (VHI ? 1024 : 0);
  static constexpr int NLD = 3 + (HIMODE != 0 ? 1 : 0) + (VHI ? 1 : 0);
  static constexpr int FIT = SLOT_LDS_BUDGET / (NW * BYTES);
  static constexpr int NSLOT = FIT < 5 ? FIT : 5;
  static_assert(NSLOT >= 2, "LDS slots");
  static_assert((NSLOT - 1) * NLD < 64, "vmcnt range");
};

// Issues the copies of quantized group `rec` into `slot`.  PRUNE (kmask bit
// s: 16-channel key run s kept): the lanes of pruned runs (their k_lo words,
// their key scale/zero) read the kept run kept0 instead, bytes the same
// instruction fetches anyway, so the pruned runs' bytes are not read; what
// those lanes write is never read.
// DENSE1: the dense 1-bit layout's 768-byte k_lo record (lanes 48..63
// re-read bytes of the record into the slack after it).
template <int HIMODE, bool VHI, bool PRUNE, bool DENSE1 = false>
__device__ inline void issue_group(const kvq_cache& c, size_t rec, uint8_t* slot, int lane,
                                   uint32_t kmask, int kept0, int nh, int nvhi) {
  using C = SlotCfg<HIMODE, VHI>;
  // k_lo: lane l holds words 4l .. 4l+3: tokens 4 (l % 4) .. +3 of tile half
  // (l / 4) % 2 of the 16-channel run l / 8 (128 bytes per run)
  int lk = lane;
  if (PRUNE && !((kmask >> (lane >> 3)) & 1u)) lk = (lane & 7) | (kept0 << 3);
  if constexpr (DENSE1)
    dma16<CPOL_NT>((const uint8_t*)c.k_lo + rec * 768 + (lane < 48 ? lane : lane - 16) * 16,
                   slot + C::KLO);
  else
    dma16<CPOL_NT>((const uint8_t*)c.k_lo + rec * 1024 + lk * 16, slot + C::KLO);
  // metadata: lanes 0..31 k_meta (64 bytes per 16-channel run: lanes 4w,
  // 4w+1 its scales, 4w+2, 4w+3 its zeros), lanes 32..63 v_meta
  {
    int lm = lane;
    if (PRUNE && lane < 32 && !((kmask >> (lane >> 2)) & 1u)) lm = (lane & 3) | (kept0 << 2);
    const uint8_t* src = lane < 32 ? (const uint8_t*)c.k_meta + rec * 512 + lm * 16
                                   : (const uint8_t*)c.v_meta + rec * 512 + (lane - 32) * 16;
    dma16<CPOL_NT>(src, slot + C::META);
  }
  dma16<CPOL_NT>((const uint8_t*)c.v_codes + rec * 1024 + lane * 16, slot + C::VC);
  if constexpr (HIMODE == 4)  // 128 bytes
    dma16<CPOL_NT>((const uint8_t*)c.k_hi + rec * 128 + (lane & 7) * 16, slot + C::KHI);
  if constexpr (HIMODE == 16)  // 32 rows of nh raw salient values: 64 nh bytes (nh >= 2)
    dma16<CPOL_NT>((const uint8_t*)c.k_hi + rec * 64 * nh + (lane < 4 * nh ? lane : lane & 3) * 16,
          slot + C::KHI);
  if constexpr (VHI)  // the high-digit words (after the 8 order words): 256 n_vhi bytes
    dma16<CPOL_NT>((const uint8_t*)(c.v_hi + rec * (8 + 64 * nvhi) + 8) +
              (lane < 16 * nvhi ? lane : lane & 15) * 16,
          slot + C::VH);
}

// Waits until the copies of the group issued `after` groups before the last
// one issued have landed (vmcnt counts this wave's vector memory operations
// in issue order; only the slot copies are outstanding in the group loop).
template <int NLD, int NSLOT>
__device__ inline void wait_slot(int after) {
  static_assert(NSLOT <= 5, "cases");
  switch (after) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<NLD>(); break;
    case 2: wait_vmcnt<2 * NLD>(); break;
    case 3: wait_vmcnt<3 * NLD < 64 ? 3 * NLD : 63>(); break;
    default: wait_vmcnt<4 * NLD < 64 ? 4 * NLD : 63>(); break;
  }
  compiler_fence();
}

}  // namespace kvq
