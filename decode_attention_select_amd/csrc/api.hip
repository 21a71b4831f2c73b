// api.hip — the C ABI of libkvq (declared in include/kvq.h): argument
// validation, buffer sizes and launch dispatch.  No call allocates or
// synchronizes (except kvq_check).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "internal.h"

using namespace kvq;

// Decode workspace of kvq_decode_attn_noalloc: one copy per GPU, held until
// the process ends.  In host code `scratch` names a host-side stand-in, never
// the device array: every host use goes through the per-device address that
// hipGetSymbolAddress returns (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
// Leading bytes of each device's scratch known to be zero once the work
// enqueued so far has run: a decode call leaves its split counters (the
// first 256 B * B * Hkv bytes) at zero and writes its split records right
// after them, so a later call with more (sequence, KV head) pairs finds
// records where its extra counters go.
size_t g_scratch_clean[MAX_DEVICES] = {};

// Zero fill of n 32-bit words (a kernel, not a memset, so that a caller's
// graph capture records a plain kernel node).
__global__ void zero_words(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The current device's scratch address, for a call whose split counters take
// the first `tick_bytes` bytes.  The first call on a device resolves it and
// enqueues one zero fill of the whole array on `st`; a later call whose
// counters reach past the bytes known to be zero first zero-fills the
// difference on `st` (the counters must start at zero).
kvq_status scratch_ptr(void** out, size_t tick_bytes, hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return KVQ_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_EHIP;
    hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, st, (uint32_t*)p,
                       (size_t)KVQ_NOALLOC_WORKSPACE_BYTES / 4);
    if (hipGetLastError() != hipSuccess) return KVQ_EHIP;
    g_scratch_ptr[dev] = p;
    g_scratch_clean[dev] = KVQ_NOALLOC_WORKSPACE_BYTES;
  }
  unsigned char* p = (unsigned char*)g_scratch_ptr[dev];
  if (tick_bytes > g_scratch_clean[dev]) {
    const size_t c = g_scratch_clean[dev];
    hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, st, (uint32_t*)(p + c),
                       (tick_bytes - c) / 4);
    if (hipGetLastError() != hipSuccess) return KVQ_EHIP;
  }
  g_scratch_clean[dev] = tick_bytes;  // records follow the counters from here on
  *out = p;
  return KVQ_OK;
}

// KVQ_LOG set (to anything but "0") in the environment: every launch prints
// its call, shape and launch geometry on stderr (host side only).
bool log_on() {
  static const bool on = [] {
    const char* e = getenv("KVQ_LOG");
    return e && *e && strcmp(e, "0") != 0;
  }();
  return on;
}

void log_launch(const char* call, const Geo& g, int T, int splits, int keep) {
  if (!log_on()) return;
  fprintf(stderr,
          "kvq: %s B=%d Hq=%d Hkv=%d G=%d T=%d R=%d groups<=%d n_hi=%d bits_hi=%d n_lo1=%d "
          "n_vhi=%d w8=%d w4=%d io=%s splits=%d keep=%d\n",
          call, g.B, g.Hq, g.Hkv, g.G, T, g.R, g.NG, g.n_hi, g.bits_hi, g.n_lo1, g.n_vhi,
          g.w8, g.w4, g.bf16 ? "bf16" : "fp16", splits, keep);
}

kvq_status check_layout(const kvq_layout* L) {
  if (!L) return KVQ_EINVAL;
  if (L->batch < 1 || L->n_q_heads < 1 || L->n_kv_heads < 1) return KVQ_EINVAL;
  if (L->n_q_heads % L->n_kv_heads) return KVQ_EINVAL;
  if (L->head_dim != D || L->group != GS) return KVQ_EINVAL;
  if (L->n_q_heads / L->n_kv_heads > 16) return KVQ_ENOTSUP;
  if (L->n_pairs_hi < 0 || L->n_pairs_hi > 8) return KVQ_EINVAL;
  if (L->bits_hi != 4 && L->bits_hi != 16) return KVQ_ENOTSUP;
  if (L->n_pairs_lo1 < 0 || L->n_pairs_hi + L->n_pairs_lo1 > NPAIR) return KVQ_EINVAL;
  if (L->bits_lo != 2 || L->bits_v != 2) return KVQ_ENOTSUP;
  if (L->residual < GS || L->residual % GS) return KVQ_EINVAL;
  if (L->max_tokens < 1 || L->max_tokens > (1 << 20)) return KVQ_EINVAL;
  if (L->io_dtype != KVQ_FP16 && L->io_dtype != KVQ_BF16) return KVQ_EINVAL;
  if (L->n_vblk_hi < 0 || L->n_vblk_hi > 4) return KVQ_EINVAL;
  if (L->n_vblk_hi > 0 && L->bits_vhi != 3 && L->bits_vhi != 4) return KVQ_ENOTSUP;
  if (L->prog_w8 < 0 || L->prog_w4 < L->prog_w8 || L->prog_w4 > 256) return KVQ_EINVAL;
  if (L->prog_w4 > 0 && (L->n_pairs_lo1 > 0 || L->n_vblk_hi > 0)) return KVQ_ENOTSUP;
  return KVQ_OK;
}

Geo make_geo(const kvq_layout* L) {
  Geo g;
  g.B = L->batch;
  g.Hq = L->n_q_heads;
  g.Hkv = L->n_kv_heads;
  g.G = g.Hq / g.Hkv;
  g.R = L->residual;
  g.RS = g.R + GS;
  g.NG = L->max_tokens > g.R ? (L->max_tokens - g.R) / GS : 0;
  g.n_hi = L->n_pairs_hi;
  g.bits_hi = L->bits_hi;
  g.n_lo1 = L->n_pairs_lo1;
  g.nh = 2 * g.n_hi;
  g.bf16 = L->io_dtype == KVQ_BF16;
  g.max_tokens = L->max_tokens;
  g.khi_bytes = g.n_hi == 0 ? 0 : (g.bits_hi == 4 ? 32 * 4 : GS * g.nh * 2);
  g.n_vhi = L->n_vblk_hi;
  g.bits_vhi = g.n_vhi ? L->bits_vhi : 2;
  g.vhi_words = g.n_vhi ? 8 + 64 * g.n_vhi : 0;
  g.w4 = L->prog_w4;
  g.w8 = g.w4 > 0 ? L->prog_w8 : 0;
  g.npl = g.w4 + 2 * g.w8;
  g.dense1 = g.n_hi == 0 && g.n_lo1 == NPAIR / 2;
  g.klo_bytes = g.dense1 ? 768 : GROUP_WORDS * 4;
  return g;
}

bool aligned(const void* p) { return ((uintptr_t)p & 15) == 0; }

kvq_status check_ptr(const void* p) {
  if (!p) return KVQ_EINVAL;
  return aligned(p) ? KVQ_OK : KVQ_EALIGN;
}

kvq_status check_cache(const Geo& g, const kvq_cache* c, bool need_groups) {
  if (!c) return KVQ_EINVAL;
  const void* ptrs[] = {c->ring_k, c->ring_v, c->pairs, c->len, c->sums, c->err};
  for (const void* p : ptrs)
    if (kvq_status s = check_ptr(p)) return s;
  if (need_groups && g.NG > 0) {
    const void* gp[] = {c->k_lo, c->k_meta, c->v_codes, c->v_meta};
    for (const void* p : gp)
      if (kvq_status s = check_ptr(p)) return s;
    if (g.khi_bytes)
      if (kvq_status s = check_ptr(c->k_hi)) return s;
    if (g.vhi_words)
      if (kvq_status s = check_ptr(c->v_hi)) return s;
    if (g.npl) {
      if (kvq_status s = check_ptr(c->k_pl)) return s;
      if (kvq_status s = check_ptr(c->v_pl)) return s;
    }
  }
  return KVQ_OK;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_EHIP; }

}  // namespace

extern "C" {

kvq_status kvq_cache_sizes(const kvq_layout* L, size_t sizes[KVQ_NBUF]) {
  if (kvq_status s = check_layout(L)) return s;
  if (!sizes) return KVQ_EINVAL;
  const Geo g = make_geo(L);
  const size_t bh = (size_t)g.B * g.Hkv, grp = bh * g.NG;
  const size_t el = 2;  // bytes of a 16-bit value
  sizes[0] = grp * g.klo_bytes;      // k_lo
  // k_hi; raw 16-bit salient rows (2*nh bytes) are read 16 bytes at a time
  // from channel 0 or 8 of a row: the last row's read ends at most 32 - 2*nh
  // bytes past the record, so 32 bytes of tail slack keep it in the buffer
  sizes[1] = grp * g.khi_bytes + (grp && g.bits_hi == 16 && g.nh ? 32 : 0);
  sizes[2] = grp * 2 * D * 2;        // k_meta
  sizes[3] = grp * GROUP_WORDS * 4;  // v_codes
  sizes[4] = grp * 2 * D * 2;        // v_meta
  sizes[5] = bh * g.RS * D * el;     // ring_k
  sizes[6] = bh * g.RS * D * el;     // ring_v
  sizes[7] = bh * NPAIR * 4;         // pairs
  sizes[8] = bh * 4;                 // len
  sizes[9] = bh * 2 * NPAIR * 8;     // sums
  sizes[10] = 4;                     // err
  sizes[11] = grp * g.vhi_words * 4; // v_hi
  sizes[12] = g.NG > 0 ? bh * g.npl * GROUP_WORDS * 4 : 0;  // k_pl
  sizes[13] = sizes[12];             // v_pl
  return KVQ_OK;
}

kvq_status kvq_workspace_bytes(const kvq_layout* L, int32_t n_splits, size_t* bytes) {
  if (kvq_status s = check_layout(L)) return s;
  if (!bytes || n_splits < 1 || n_splits > 1024) return KVQ_EINVAL;
  *bytes = decode_workspace_bytes(L->batch, L->n_q_heads, L->n_kv_heads, n_splits);
  return KVQ_OK;
}

kvq_status kvq_select_pairs(const kvq_layout* L, const void* q_sel, int32_t n_qry, const void* k,
                            int32_t T, kvq_cache* cache, void* stream) {
  if (kvq_status s = check_layout(L)) return s;
  const Geo g = make_geo(L);
  if (n_qry < 1 || n_qry > 1024 || T < 1) return KVQ_EINVAL;
  if (T > g.max_tokens) return KVQ_ECAPACITY;
  if (kvq_status s = check_ptr(q_sel)) return s;
  if (kvq_status s = check_ptr(k)) return s;
  if (kvq_status s = check_cache(g, cache, false)) return s;
  log_launch("kvq_select_pairs", g, T, 0, 0);
  return hip_status(launch_select(g, q_sel, n_qry, k, T, cache, (hipStream_t)stream));
}

kvq_status kvq_select_pairs_qa(const kvq_layout* L, const void* q_sel, int32_t n_qry,
                               const void* k, int32_t T, kvq_cache* cache, void* stream) {
  if (kvq_status s = check_layout(L)) return s;
  const Geo g = make_geo(L);
  if (n_qry < 1 || n_qry > 1024 || T < 1) return KVQ_EINVAL;
  if (T > g.max_tokens) return KVQ_ECAPACITY;
  if (kvq_status s = check_ptr(q_sel)) return s;
  if (kvq_status s = check_ptr(k)) return s;
  if (kvq_status s = check_cache(g, cache, false)) return s;
  log_launch("kvq_select_pairs_qa", g, T, 0, 0);
  return hip_status(launch_select_qa(g, q_sel, n_qry, k, T, cache, (hipStream_t)stream));
}

kvq_status kvq_quant_keys(const kvq_layout* L, const void* k, int32_t T, kvq_cache* cache,
                          void* stream) {
  if (kvq_status s = check_layout(L)) return s;
  const Geo g = make_geo(L);
  if (T < 1) return KVQ_EINVAL;
  if (T > g.max_tokens) return KVQ_ECAPACITY;
  if (kvq_status s = check_ptr(k)) return s;
  if (kvq_status s = check_cache(g, cache, true)) return s;
  log_launch("kvq_quant_keys", g, T, 0, 0);
  return hip_status(launch_quant_keys(g, k, T, cache, (hipStream_t)stream));
}

kvq_status kvq_quant_values(const kvq_layout* L, const void* v, int32_t T, kvq_cache* cache,
                            void* stream) {
  if (kvq_status s = check_layout(L)) return s;
  const Geo g = make_geo(L);
  if (T < 1) return KVQ_EINVAL;
  if (T > g.max_tokens) return KVQ_ECAPACITY;
  if (kvq_status s = check_ptr(v)) return s;
  if (kvq_status s = check_cache(g, cache, true)) return s;
  log_launch("kvq_quant_values", g, T, 0, 0);
  return hip_status(launch_quant_values(g, v, T, cache, (hipStream_t)stream));
}

kvq_status kvq_append(const kvq_layout* L, const void* k_new, const void* v_new,
                      kvq_cache* cache, void* stream) {
  if (kvq_status s = check_layout(L)) return s;
  const Geo g = make_geo(L);
  if (kvq_status s = check_ptr(k_new)) return s;
  if (kvq_status s = check_ptr(v_new)) return s;
  if (kvq_status s = check_cache(g, cache, true)) return s;
  log_launch("kvq_append", g, -1, 0, 0);
  return hip_status(launch_append(g, k_new, v_new, cache, (hipStream_t)stream));
}

kvq_status kvq_shrink(const kvq_layout* L, kvq_cache* cache, int32_t g0, int32_t g1,
                      void* stream) {
  if (kvq_status s = check_layout(L)) return s;
  const Geo g = make_geo(L);
  if (g.n_hi > 0 && g.bits_hi != 4) return KVQ_ENOTSUP;
  if (g.w4 > 0) return KVQ_ENOTSUP;
  if (g0 < 0 || g1 < g0) return KVQ_EINVAL;
  if (kvq_status s = check_cache(g, cache, true)) return s;
  if (g.NG > 0 && g1 > g.NG) g1 = g.NG;
  if (g0 > g1) g0 = g1;
  log_launch("kvq_shrink", g, -1, g1 - g0, 0);
  return hip_status(launch_shrink(g, cache, g0, g1, (hipStream_t)stream));
}

// keep 1..8: kept 16-channel key runs (8: all); 0: append k_new / v_new and
// decode in one launch
static kvq_status decode_common(const kvq_layout* L, const void* q, const kvq_cache* cache,
                                float sm_scale, int32_t n_splits, int32_t keep, void* workspace,
                                size_t ws_bytes, void* out, void* stream,
                                const void* k_new = nullptr, const void* v_new = nullptr) {
  if (kvq_status s = check_layout(L)) return s;
  const Geo g = make_geo(L);
  size_t need = 0;
  if (kvq_status s = kvq_workspace_bytes(L, n_splits, &need)) return s;
  if (ws_bytes < need) return KVQ_ECAPACITY;
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return KVQ_EINVAL;
  if (keep < 0 || keep > 8) return KVQ_EINVAL;
  if (g.w4 > 0 && keep != 8 && keep != 0) return KVQ_ENOTSUP;
  if (g.dense1 && keep >= 1 && keep < 8) return KVQ_ENOTSUP;
  if (kvq_status s = check_ptr(q)) return s;
  if (kvq_status s = check_ptr(out)) return s;
  if (kvq_status s = check_ptr(workspace)) return s;
  if (keep == 0) {
    if (kvq_status s = check_ptr(k_new)) return s;
    if (kvq_status s = check_ptr(v_new)) return s;
  }
  if (kvq_status s = check_cache(g, cache, true)) return s;
  log_launch(keep == 0 ? "kvq_append_decode_attn" : keep < 8 ? "kvq_decode_attn_pruned"
                                                             : "kvq_decode_attn",
             g, -1, n_splits, keep);
  return hip_status(launch_decode(g, q, cache, sm_scale, n_splits, keep, workspace, out,
                                  (hipStream_t)stream, k_new, v_new));
}

kvq_status kvq_decode_attn(const kvq_layout* L, const void* q, const kvq_cache* cache,
                           float sm_scale, int32_t n_splits, void* workspace, size_t ws_bytes,
                           void* out, void* stream) {
  return decode_common(L, q, cache, sm_scale, n_splits, 8, workspace, ws_bytes, out, stream);
}

kvq_status kvq_decode_attn_pruned(const kvq_layout* L, const void* q, const kvq_cache* cache,
                                  float sm_scale, int32_t n_splits, int32_t n_keep,
                                  void* workspace, size_t ws_bytes, void* out, void* stream) {
  if (n_keep < 1) return KVQ_EINVAL;
  return decode_common(L, q, cache, sm_scale, n_splits, n_keep, workspace, ws_bytes, out, stream);
}

kvq_status kvq_append_decode_attn(const kvq_layout* L, const void* k_new, const void* v_new,
                                  const void* q, kvq_cache* cache, float sm_scale,
                                  int32_t n_splits, void* workspace, size_t ws_bytes, void* out,
                                  void* stream) {
  return decode_common(L, q, cache, sm_scale, n_splits, 0, workspace, ws_bytes, out, stream,
                       k_new, v_new);
}

kvq_status kvq_decode_attn_noalloc(const kvq_layout* L, const void* q, const kvq_cache* cache,
                                   float sm_scale, int32_t n_splits, void* out, void* stream) {
  if (kvq_status s = check_layout(L)) return s;
  size_t need = 0;
  if (kvq_status s = kvq_workspace_bytes(L, n_splits, &need)) return s;
  if (need > (size_t)KVQ_NOALLOC_WORKSPACE_BYTES) return KVQ_ECAPACITY;
  void* ws = nullptr;
  if (kvq_status s = scratch_ptr(&ws, decode_tick_bytes(L->batch, L->n_kv_heads),
                                 (hipStream_t)stream))
    return s;
  return decode_common(L, q, cache, sm_scale, n_splits, 8, ws,
                       (size_t)KVQ_NOALLOC_WORKSPACE_BYTES, out, stream);
}

kvq_status kvq_read_ceiling(const kvq_layout* L, const kvq_cache* cache, int32_t n_splits,
                            void* sink, void* stream) {
  if (kvq_status s = check_layout(L)) return s;
  const Geo g = make_geo(L);
  size_t need = 0;
  if (kvq_status s = kvq_workspace_bytes(L, n_splits, &need)) return s;  // n_splits limits
  if (g.w4 > 0) return KVQ_ENOTSUP;
  if (kvq_status s = check_ptr(sink)) return s;
  if (kvq_status s = check_cache(g, cache, true)) return s;
  log_launch("kvq_read_ceiling", g, -1, n_splits, 8);
  return hip_status(launch_ceiling(g, cache, n_splits, sink, (hipStream_t)stream));
}

kvq_status kvq_issue_probe(int32_t kind, int32_t n_blocks, void* out, void* stream) {
  if (kind < 0 || kind > 6 || n_blocks < 1) return KVQ_EINVAL;
  if (kvq_status s = check_ptr(out)) return s;
  return hip_status(launch_issue_probe(kind, n_blocks, out, (hipStream_t)stream));
}

kvq_status kvq_check(const kvq_cache* cache, int32_t* host_err, void* stream) {
  if (!cache || !cache->err || !host_err) return KVQ_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return KVQ_EHIP;
  if (hipMemcpy(host_err, cache->err, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return KVQ_EHIP;
  return KVQ_OK;
}

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_ENOTSUP: return "unsupported layout option";
    case KVQ_EALIGN: return "device pointer not 16-byte aligned";
    case KVQ_ECAPACITY: return "capacity or workspace too small";
    case KVQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
