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

constexpr int SEL_THREADS = 256;          // 4 rows of 64 pairs in flight
constexpr int SEL_ROWS_PER_BLOCK = 256;   // rows (tokens or queries) per block

__global__ void zero_u64_kernel(uint64_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// IEEE sqrt of a non-negative fp32, correctly rounded: the hardware estimate
// is corrected by comparing x with the exact squares (in fp64: a 25-bit
// midpoint squares exactly) of the midpoints to its neighbours.
__device__ inline float sqrt_rn(float x) {
  float y = sqrtf(x);
  if (!(x > 0.0f) || isinf(x)) return y;
  const double xd = x;
  const float up = __uint_as_float(__float_as_uint(y) + 1u);
  const double mu = 0.5 * ((double)y + (double)up);
  if (mu * mu <= xd) return up;
  const float dn = __uint_as_float(__float_as_uint(y) - 1u);
  const double md = 0.5 * ((double)y + (double)dn);
  return md * md > xd ? dn : y;
}

__device__ inline uint64_t norm_fixed(uint16_t a_bits, uint16_t b_bits, int bf16) {
  const float a = in_to_f32(a_bits, bf16), b = in_to_f32(b_bits, bf16);
  const float s = __fadd_rn(__fmul_rn(a, a), __fmul_rn(b, b));
  const float n = sqrt_rn(s);
  return (uint64_t)((double)n * 16777216.0);
}

// grid.x = B * Hkv; grid.y = key blocks + query blocks.  Thread t handles
// pair t % 64 of rows t / 64, t / 64 + 4, ... of its block's row range.
__global__ __launch_bounds__(SEL_THREADS) void pair_sums_kernel(
    Geo g, const uint16_t* __restrict__ q_sel, int n_qry,
    const uint16_t* __restrict__ k, int T, int key_blocks,
    uint64_t* __restrict__ sums) {
  const int bh = blockIdx.x;  // b * Hkv + kv head
  const int b = bh / g.Hkv, kh = bh % g.Hkv;
  const int j = threadIdx.x & 63, sub = threadIdx.x >> 6;
  uint64_t acc = 0;
  int side;
  if ((int)blockIdx.y < key_blocks) {
    side = 1;
    const int r0 = blockIdx.y * SEL_ROWS_PER_BLOCK;
    const int r1 = min(T, r0 + SEL_ROWS_PER_BLOCK);
    const uint16_t* base = k + (size_t)bh * T * D;
    for (int r = r0 + sub; r < r1; r += 4)
      acc += norm_fixed(base[(size_t)r * D + j], base[(size_t)r * D + j + NPAIR], g.bf16);
  } else {
    side = 0;
    const int nrows = g.G * n_qry;
    const int r0 = (blockIdx.y - key_blocks) * SEL_ROWS_PER_BLOCK;
    const int r1 = min(nrows, r0 + SEL_ROWS_PER_BLOCK);
    for (int r = r0 + sub; r < r1; r += 4) {
      const int h = kh * g.G + r / n_qry, t = r % n_qry;
      const uint16_t* row = q_sel + (((size_t)b * g.Hq + h) * n_qry + t) * D;
      acc += norm_fixed(row[j], row[j + NPAIR], g.bf16);
    }
  }
  __shared__ uint64_t part[SEL_THREADS];
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < 64) {
    const uint64_t s = part[j] + part[j + 64] + part[j + 128] + part[j + 192];
    if (s) atomicAdd((unsigned long long*)&sums[((size_t)bh * 2 + side) * NPAIR + j],
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
  hipLaunchKernelGGL(pair_sums_kernel, dim3(g.B * g.Hkv, key_blocks + q_blocks),
                     dim3(SEL_THREADS), 0, st, g, (const uint16_t*)q_sel, n_qry,
                     (const uint16_t*)k, T, key_blocks, c->sums);
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
constexpr int QA_GROUPS_PER_BLOCK = 16;

// grid (B * Hkv, ceil(groups / 16)); thread c sums channel c's ranges over
// the block's groups (rows of 128 channels are read coalesced)
__global__ __launch_bounds__(D) void qa_ranges_kernel(Geo g, const uint16_t* __restrict__ k,
                                                      int T, uint64_t* __restrict__ sums) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const int ng = T / GS;
  const int g0 = blockIdx.y * QA_GROUPS_PER_BLOCK, g1 = min(ng, g0 + QA_GROUPS_PER_BLOCK);
  const uint16_t* base = k + (size_t)bh * T * D;
  uint64_t acc = 0;
  for (int gi = g0; gi < g1; gi++) {
    float mn = INFINITY, mx = -INFINITY;
    for (int i = 0; i < GS; i++) {
      const float x = in_to_f32(base[(size_t)(gi * GS + i) * D + c], g.bf16);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    acc += (uint64_t)((double)__fsub_rn(mx, mn) * 65536.0);  // non-negative: truncation = floor
  }
  if (acc) atomicAdd((unsigned long long*)&sums[(size_t)bh * D + c], (unsigned long long)acc);
}

// one workgroup of 128 threads per (b, kv head)
__global__ __launch_bounds__(D) void qa_rank_kernel(Geo g, const uint16_t* __restrict__ q_sel,
                                                    int n_qry, uint64_t* __restrict__ sums,
                                                    int32_t* __restrict__ pairs) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const int b = bh / g.Hkv, kh = bh % g.Hkv;
  uint64_t A = 0;
  for (int h = kh * g.G; h < (kh + 1) * g.G; h++)
    for (int t = 0; t < n_qry; t++) {
      const float x = fabsf(in_to_f32(q_sel[(((size_t)b * g.Hq + h) * n_qry + t) * D + c], g.bf16));
      A += (uint64_t)((double)x * 16777216.0);
    }
  __shared__ uint64_t As[D], Rs[D];
  __shared__ double S[NPAIR];
  As[c] = A;
  Rs[c] = sums[(size_t)bh * D + c];
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
  } else {
    sums[(size_t)bh * D + c] = 0;
  }
}

hipError_t launch_select_qa(const Geo& g, const void* q_sel, int n_qry, const void* k, int T,
                            kvq_cache* c, hipStream_t st) {
  const int nsum = g.B * g.Hkv * 2 * NPAIR;
  hipLaunchKernelGGL(zero_u64_kernel, dim3((nsum + 255) / 256), dim3(256), 0, st, c->sums, nsum);
  const int ng = T / GS;
  if (ng > 0)
    hipLaunchKernelGGL(qa_ranges_kernel,
                       dim3(g.B * g.Hkv, (ng + QA_GROUPS_PER_BLOCK - 1) / QA_GROUPS_PER_BLOCK),
                       dim3(D), 0, st, g, (const uint16_t*)k, T, c->sums);
  hipLaunchKernelGGL(qa_rank_kernel, dim3(g.B * g.Hkv), dim3(D), 0, st, g,
                     (const uint16_t*)q_sel, n_qry, c->sums, c->pairs);
  return hipGetLastError();
}

}  // namespace kvq
