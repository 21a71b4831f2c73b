// select.hip — pair saliency sums and ranking (PN-Mix, abstract and podcast
// transcript: a RoPE pair's saliency is its query pair norm times its key
// pair norm; the salient pairs are chosen once, at prefill).
//
// Per (b, kv head) and pair j:
//   sums[0][j] = sum over the group's query heads and selection queries of
//                u(|q^(j)|), sums[1][j] = sum over prefill keys of u(|k^(j)|)
// with u(n) = floor(n * 2^24) of the fp32 norm n = sqrt(a*a + b*b).  Integer
// sums make the result independent of the reduction order, so any grid
// gives bit-identical ranks.  Then S_j = (double)sums[0][j] *
// (double)sums[1][j], ranked descending, ties to the lower pair id.
#include "common.h"
#include "internal.h"

namespace kvq {

constexpr int SEL_THREADS = 256;
constexpr int SEL_SLOTS = SEL_THREADS / 8;  // row slots: 8 threads (16-byte chunks) per row
constexpr int SEL_ROWS_PER_BLOCK = 8 * SEL_SLOTS;  // 8 rows per thread, all loads up front

__global__ void zero_u64_kernel(uint64_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// u(n) = floor(n * 2^24) of the fp32 norm n = RN(sqrt(RN(a*a + b*b))), as an
// integer-valued double.  a*a and b*b are exact for 16-bit inputs, so
// fma(a, a, b*b) is the rounded sum.  The square root is correctly rounded:
// the hardware estimate y (within one ulp) or a neighbour y-, y+, chosen by
// the exact signs of s - y- y and s - y y+ (fma residuals); no float s lies
// between y- y (y y+) and the squared midpoint, so these signs decide the
// rounding.  Below s = 2^-48 every candidate is under 2^-24 and u = 0, so
// subnormal estimates cannot matter.  n * 2^24 and its floor are exact in
// fp32 (a power-of-two scaling, then an fp32 floor), and so in double; a
// thread's sum of eight such terms in double stays exact for norms below
// 2^25.
template <bool BF>
__device__ inline double norm_fixed(uint16_t a_bits, uint16_t b_bits) {
  const float a = in_to_f32(a_bits, BF), b = in_to_f32(b_bits, BF);
  const float s = fmaf(a, a, __fmul_rn(b, b));
  const float y0 = __builtin_amdgcn_sqrtf(s);
  const float ym = __uint_as_float(__float_as_uint(y0) - 1u);
  const float yp = __uint_as_float(__float_as_uint(y0) + 1u);
  const float rm = fmaf(-ym, y0, s), rp = fmaf(-yp, y0, s);
  float y = rm <= 0.0f ? ym : y0;
  y = rp > 0.0f ? yp : y;
  // y * 2^24 is exact in fp32 (a power-of-two scaling), so is its floor
  return (double)floorf(y * 16777216.0f);
}

// 16-bit element e (0..7) of a 16-byte row chunk.
__device__ inline uint16_t sel_half(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFF);
}

// grid.x = B * Hkv; grid.y = key blocks + query blocks.  Thread t covers
// pairs 8 cb .. 8 cb + 7 (cb = t % 8: channels 8cb.. and 64 + 8cb.., two
// 16-byte loads per row) of rows t / 8 + 32 i, i = 0..7, of its block.
// A (b, kv head)'s selection queries are G * n_qry consecutive rows.
template <bool BF>
__global__ __launch_bounds__(SEL_THREADS) void pair_sums_kernel(
    Geo g, const uint16_t* __restrict__ q_sel, int n_qry,
    const uint16_t* __restrict__ k, int T, int key_blocks,
    uint64_t* __restrict__ sums) {
  const int bh = blockIdx.x;  // b * Hkv + kv head
  const int b = bh / g.Hkv, kh = bh % g.Hkv;
  const int cb = threadIdx.x & 7, slot = threadIdx.x >> 3;
  const bool key = (int)blockIdx.y < key_blocks;
  const uint16_t* base = key ? k + (size_t)bh * T * D
                             : q_sel + ((size_t)b * g.Hq + (size_t)kh * g.G) * n_qry * D;
  const int nrows = key ? T : g.G * n_qry;
  const int r0 = (key ? blockIdx.y : blockIdx.y - key_blocks) * SEL_ROWS_PER_BLOCK;
  uint4 va[8], vb[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int r = r0 + slot + SEL_SLOTS * i;
    va[i] = vb[i] = make_uint4(0, 0, 0, 0);  // a zero row adds u(0) = 0
    if (r < nrows) {
      const uint16_t* row = base + (size_t)r * D;
      va[i] = *(const uint4*)(row + 8 * cb);
      vb[i] = *(const uint4*)(row + NPAIR + 8 * cb);
    }
  }
  uint64_t acc[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < 8; i++) t += norm_fixed<BF>(sel_half(va[i], e), sel_half(vb[i], e));
    acc[e] = (uint64_t)t;
  }
  __shared__ uint64_t part[SEL_SLOTS][NPAIR];
#pragma unroll
  for (int e = 0; e < 8; e++) part[slot][8 * cb + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < NPAIR) {
    uint64_t s = 0;
    for (int i = 0; i < SEL_SLOTS; i++) s += part[i][threadIdx.x];
    if (s) atomicAdd((unsigned long long*)&sums[((size_t)bh * 2 + (key ? 1 : 0)) * NPAIR +
                                                threadIdx.x],
                     (unsigned long long)s);
  }
}

// One wave per (b, kv head): lane j computes its own rank.
__global__ __launch_bounds__(64) void rank_pairs_kernel(const uint64_t* __restrict__ sums,
                                                        int32_t* __restrict__ pairs) {
  const int bh = blockIdx.x, j = threadIdx.x;
  __shared__ double S[NPAIR];
  const uint64_t* qs = sums + (size_t)bh * 2 * NPAIR;
  S[j] = (double)qs[j] * (double)qs[NPAIR + j];
  __syncthreads();
  const double mine = S[j];
  int rank = 0;
  for (int i = 0; i < NPAIR; i++) rank += (S[i] > mine) || (S[i] == mine && i < j);
  pairs[(size_t)bh * NPAIR + rank] = j;
}

hipError_t launch_select(const Geo& g, const void* q_sel, int n_qry, const void* k, int T,
                         kvq_cache* c, hipStream_t st) {
  const int nsum = g.B * g.Hkv * 2 * NPAIR;
  hipLaunchKernelGGL(zero_u64_kernel, dim3((nsum + 255) / 256), dim3(256), 0, st, c->sums, nsum);
  const int key_blocks = (T + SEL_ROWS_PER_BLOCK - 1) / SEL_ROWS_PER_BLOCK;
  const int q_blocks = (g.G * n_qry + SEL_ROWS_PER_BLOCK - 1) / SEL_ROWS_PER_BLOCK;
  const dim3 grid(g.B * g.Hkv, key_blocks + q_blocks);
  if (g.bf16)
    hipLaunchKernelGGL(pair_sums_kernel<true>, grid, dim3(SEL_THREADS), 0, st, g,
                       (const uint16_t*)q_sel, n_qry, (const uint16_t*)k, T, key_blocks, c->sums);
  else
    hipLaunchKernelGGL(pair_sums_kernel<false>, grid, dim3(SEL_THREADS), 0, st, g,
                       (const uint16_t*)q_sel, n_qry, (const uint16_t*)k, T, key_blocks, c->sums);
  hipLaunchKernelGGL(rank_pairs_kernel, dim3(g.B * g.Hkv), dim3(64), 0, st,
                     (const uint64_t*)c->sums, c->pairs);
  return hipGetLastError();
}

// Query-aware channel score (MixKVQ, abstract and AI summary: a key
// channel's importance joins its intrinsic quantization difficulty with its
// relevance to the query; the page gives no formula, this is a reading).
// Per (b, kv head) and channel c:
//   A_c = sum over the group's query heads and selection queries of
//         floor(|q_c| * 2^24)
//   R_c = sum over the full 32-token groups of the prefill keys of
//         floor(fp32(max k_c - min k_c) * 2^16)
// and per pair S_j = R_j A_j + R_{j+64} A_{j+64} in IEEE double, each
// product and the sum rounded once (no contraction).  Ranked descending,
// ties to the lower pair id.  sums is scratch for R, then holds [0][j] = the
// bits of S_j and [1][j] = 0.
constexpr int QA_GROUPS_PER_WAVE = 4;
constexpr int QA_GROUPS_PER_BLOCK = 4 * QA_GROUPS_PER_WAVE;

// min / max over the four lanes of a DPP quad, one VALU instruction per
// step (the DPP source operand reads the partner lane; s_nop 1 covers the
// wait states between a VALU write and a DPP read of the same register)
#define KVQ_QA_QUAD(name, op)                                                      \
  __device__ inline float name(float v) {                                          \
    float t, r;                                                                    \
    asm("s_nop 1\n\t" op "_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" \
        : "=&v"(t) : "v"(v));                                                      \
    asm("s_nop 1\n\t" op "_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" \
        : "=&v"(r) : "v"(t));                                                      \
    return r;                                                                      \
  }
KVQ_QA_QUAD(qa_quad_min, "v_min_f32")
KVQ_QA_QUAD(qa_quad_max, "v_max_f32")
#undef KVQ_QA_QUAD

// grid (B * Hkv, ceil(groups / 16)), 4 waves of 4 groups each.  Lane
// 4 cb + tq holds channels 8cb .. 8cb+7 of tokens 8tq .. 8tq+7 of a group
// (one 16-byte load per token), so a channel's 32 tokens lie in one quad.
template <bool BF>
__global__ __launch_bounds__(256) void qa_ranges_kernel(Geo g, const uint16_t* __restrict__ k,
                                                        int T, uint64_t* __restrict__ sums) {
  const int bh = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cb = lane >> 2, tq = lane & 3;
  const int ng = T / GS;
  const uint16_t* base = k + (size_t)bh * T * D;
  uint64_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int gw = blockIdx.y * QA_GROUPS_PER_BLOCK + wave * QA_GROUPS_PER_WAVE;
  for (int h = 0; h < QA_GROUPS_PER_WAVE; h += 2) {
    uint4 v[2][8];
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int gi = min(gw + h + u, ng - 1);  // clamped: in bounds, counted below only if valid
        v[u][i] = *(const uint4*)(base + ((size_t)gi * GS + 8 * tq + i) * D + 8 * cb);
      }
#pragma unroll
    for (int u = 0; u < 2; u++) {
      if (gw + h + u >= ng) continue;  // wave-uniform
#pragma unroll
      for (int e = 0; e < 8; e++) {
        float mn = in_to_f32(sel_half(v[u][0], e), BF), mx = mn;
#pragma unroll
        for (int i = 1; i < 8; i += 2) {  // three-input min / max
          const float x = in_to_f32(sel_half(v[u][i], e), BF);
          const float y = i + 1 < 8 ? in_to_f32(sel_half(v[u][i + 1], e), BF) : x;
          mn = fminf(mn, fminf(x, y));
          mx = fmaxf(mx, fmaxf(x, y));
        }
        mn = qa_quad_min(mn);
        mx = qa_quad_max(mx);
        // range * 2^16 is exact and below 2^32 (range <= 65504): truncation = floor
        acc[e] += (uint32_t)(__fsub_rn(mx, mn) * 65536.0f);
      }
    }
  }
  __shared__ uint64_t part[4][D];
  if (tq == 0) {
#pragma unroll
    for (int e = 0; e < 8; e++) part[wave][8 * cb + e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const uint64_t s = part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] +
                       part[3][threadIdx.x];
    if (s) atomicAdd((unsigned long long*)&sums[(size_t)bh * D + threadIdx.x],
                     (unsigned long long)s);
  }
}

// One 256-thread workgroup per (b, kv head).  Thread t sums |q| of channels
// 8cb .. 8cb+7 (cb = t % 16) over rows t / 16 + 16 i of the head group's
// G * n_qry selection queries, then the pair scores and ranks follow.
__global__ __launch_bounds__(256) void qa_rank_kernel(Geo g, const uint16_t* __restrict__ q_sel,
                                                      int n_qry, uint64_t* __restrict__ sums,
                                                      int32_t* __restrict__ pairs) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int b = bh / g.Hkv, kh = bh % g.Hkv;
  const int cb = tid & 15, slot = tid >> 4;
  const uint16_t* base = q_sel + ((size_t)b * g.Hq + (size_t)kh * g.G) * n_qry * D;
  const int nrows = g.G * n_qry;
  // floor(|q| * 2^24) is an exact integer-valued double; a thread sums at most
  // 1024 rows (G * n_qry <= 16 * 1024), exact for |q| below 2^19
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r0 = 0; r0 < nrows; r0 += 256) {  // 16 rows per thread in flight
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = r0 + slot + 16 * i;
      v[i] = r < nrows ? *(const uint4*)(base + (size_t)r * D + 8 * cb) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; i++)
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float x = fabsf(in_to_f32(sel_half(v[i], e), g.bf16));
        acc[e] += (double)floorf(x * 16777216.0f);  // x * 2^24 is exact in fp32
      }
  }
  __shared__ uint64_t Ap[16][D];
  __shared__ uint64_t As[D], Rs[D];
  __shared__ double S[NPAIR];
#pragma unroll
  for (int e = 0; e < 8; e++) Ap[slot][8 * cb + e] = (uint64_t)acc[e];
  __syncthreads();
  const int c = tid;
  if (c < D) {
    uint64_t A = 0;
    for (int i = 0; i < 16; i++) A += Ap[i][c];
    As[c] = A;
    Rs[c] = sums[(size_t)bh * D + c];
  }
  __syncthreads();
  if (c < NPAIR)
    S[c] = __dadd_rn(__dmul_rn((double)Rs[c], (double)As[c]),
                     __dmul_rn((double)Rs[c + NPAIR], (double)As[c + NPAIR]));
  __syncthreads();
  if (c < NPAIR) {
    const double mine = S[c];
    int rank = 0;
    for (int i = 0; i < NPAIR; i++) rank += (S[i] > mine) || (S[i] == mine && i < c);
    pairs[(size_t)bh * NPAIR + rank] = c;
    sums[(size_t)bh * D + c] = __double_as_longlong(mine);
  } else if (c < D) {
    sums[(size_t)bh * D + c] = 0;
  }
}

hipError_t launch_select_qa(const Geo& g, const void* q_sel, int n_qry, const void* k, int T,
                            kvq_cache* c, hipStream_t st) {
  const int nsum = g.B * g.Hkv * 2 * NPAIR;
  hipLaunchKernelGGL(zero_u64_kernel, dim3((nsum + 255) / 256), dim3(256), 0, st, c->sums, nsum);
  const int ng = T / GS;
  if (ng > 0)
    hipLaunchKernelGGL(g.bf16 ? qa_ranges_kernel<true> : qa_ranges_kernel<false>,
                       dim3(g.B * g.Hkv, (ng + QA_GROUPS_PER_BLOCK - 1) / QA_GROUPS_PER_BLOCK),
                       dim3(256), 0, st, g, (const uint16_t*)k, T, c->sums);
  hipLaunchKernelGGL(qa_rank_kernel, dim3(g.B * g.Hkv), dim3(256), 0, st, g,
                     (const uint16_t*)q_sel, n_qry, c->sums, c->pairs);
  return hipGetLastError();
}

}  // namespace kvq
