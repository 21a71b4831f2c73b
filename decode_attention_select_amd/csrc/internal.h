// internal.h — launchers shared between libkvq's translation units.
#pragma once

#include "common.h"

namespace kvq {

hipError_t launch_select(const Geo& g, const void* q_sel, int n_qry, const void* k, int T,
                         kvq_cache* c, hipStream_t st);
hipError_t launch_select_qa(const Geo& g, const void* q_sel, int n_qry, const void* k, int T,
                            kvq_cache* c, hipStream_t st);
hipError_t launch_quant_keys(const Geo& g, const void* k, int T, kvq_cache* c, hipStream_t st);
hipError_t launch_quant_values(const Geo& g, const void* v, int T, kvq_cache* c, hipStream_t st);
hipError_t launch_shrink(const Geo& g, kvq_cache* c, int g0, int g1, hipStream_t st);
hipError_t launch_append(const Geo& g, const void* k_new, const void* v_new, kvq_cache* c,
                         hipStream_t st);
// keep_runs 1..8: kept 16-channel key runs (8: unpruned); 0: the fused append and
// decode, which appends k_new / v_new (null otherwise)
hipError_t launch_decode(const Geo& g, const void* q, const kvq_cache* c, float sm_scale,
                         int n_splits, int keep_runs, void* workspace, void* out,
                         hipStream_t st, const void* k_new = nullptr,
                         const void* v_new = nullptr);
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int n_splits);
// bytes of the split counters at the start of a decode workspace
size_t decode_tick_bytes(int B, int Hkv);
// the decode kernel's grid and group stream, reading only (ceiling.hip)
hipError_t launch_ceiling(const Geo& g, const kvq_cache* c, int n_splits, void* sink,
                          hipStream_t st);
// the issue probe (ceiling.hip): workgroups of PROBE_THREADS threads, each
// wave PROBE_ITERS iterations of one instruction mix
constexpr int PROBE_THREADS = 256, PROBE_ITERS = 256;
hipError_t launch_issue_probe(int kind, int n_blocks, void* out, hipStream_t st);

}  // namespace kvq
