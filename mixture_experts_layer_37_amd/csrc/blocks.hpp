// Whole-workgroup steps shared by kernels of several files: each runs on one
// 256-thread workgroup with thread e standing for expert e (E <= 256), and
// every thread of the workgroup calls it.
#pragma once

#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Tile maps of the two grouped GEMMs' row tiles from each expert's kept rows
// n and first row o (threads e >= E pass n = 0).  Map layout: [E+1] first
// m-tile of every expert (exclusive scan of ceil(n / bm) over the experts),
// padded to an even count, then one int2 per m-tile:
// {first row, expert | valid rows << 16}.  tmp: 8 ints of LDS.
__device__ __forceinline__ void tile_maps_block(int e, int E, int n, int o, int bm1, int bm2,
                                                int32_t* m1, int32_t* m2, int* tmp) {
  int t1, t2;
  const int a = block_excl_scan256((n + bm1 - 1) / bm1, tmp, &t1);
  const int b = block_excl_scan256((n + bm2 - 1) / bm2, tmp + 4, &t2);
  if (e < E) {
    m1[e] = a;
    m2[e] = b;
    int2* tab1 = reinterpret_cast<int2*>(m1 + ((E + 2) & ~1));
    int2* tab2 = reinterpret_cast<int2*>(m2 + ((E + 2) & ~1));
    for (int q = 0; q * bm1 < n; ++q)
      tab1[a + q] = make_int2(o + q * bm1, e | (min(bm1, n - q * bm1) << 16));
    for (int q = 0; q * bm2 < n; ++q)
      tab2[b + q] = make_int2(o + q * bm2, e | (min(bm2, n - q * bm2) << 16));
  }
  if (e == 0) {
    m1[E] = t1;
    m2[E] = t2;
  }
}

// Load statistics (page "MoE 与专家并行", section "负载均衡辅助损失：推导与梯度":
// f_i = count_i / (T k), P_i the mean score, L_aux = E sum_i f_i P_i; MaxVio
// of section "无辅助损失的负载均衡"; the dropped assignments; the router
// z-loss from the summed LSE^2).  cnt and kp: expert e's count and kept rows
// (ignored for e >= E).  Fixed-shape tree sums: deterministic.
__device__ __forceinline__ void stats_block(const StatsParams& p, int e, int cnt_e, int kp_e) {
  __shared__ double s_fp[256];
  __shared__ int s_max[256];
  __shared__ int s_drop[256];
  double fp = 0.0;
  int cnt = INT_MIN, drop = 0;
  if (e < p.E) {
    cnt = cnt_e;
    drop = cnt_e - kp_e;
    const double ps = p.prob_total ? p.prob_total[e] : (double)p.prob_sum[e];
    const double f = p.T > 0 ? (double)cnt / ((double)p.T * p.k) : 0.0;
    const double P = p.T > 0 ? ps / p.T : 0.0;
    if (p.f) p.f[e] = (float)f;
    if (p.P) p.P[e] = (float)P;
    fp = f * P;
  }
  s_fp[e] = fp;
  s_max[e] = cnt;
  s_drop[e] = drop;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (e < w) {
      s_fp[e] += s_fp[e + w];
      s_max[e] = max(s_max[e], s_max[e + w]);
      s_drop[e] += s_drop[e + w];
    }
    __syncthreads();
  }
  if (e == 0) {
    const double mean = (double)p.T * p.k / p.E;
    if (p.aux) p.aux[0] = (float)(p.E * s_fp[0]);
    if (p.maxvio) p.maxvio[0] = p.T > 0 ? (float)((s_max[0] - mean) / mean) : 0.f;
    if (p.n_dropped) p.n_dropped[0] = s_drop[0];
    if (p.z_loss && p.prob_total)
      p.z_loss[0] = p.T > 0 ? (float)(p.prob_total[p.E] / p.T) : 0.f;
  }
}

// Router P sums: workgroup e of E + 1 reduces row e (row EP for e == E, the
// LSE^2 row) of the [EP + 1][nblk] per-block partials.  Thread j adds
// partials j, j + 256, ... in order, then a fixed-shape tree adds the 256
// sums (deterministic).  The LSE^2 sum lands in total[E] (z-loss numerator);
// out gets the E expert sums only.
__device__ __forceinline__ void prob_reduce_block(const double* part, int nblk, int EP, int E,
                                                  double* total, float* out, int e) {
  __shared__ double sh[256];
  const int col = e < E ? e : EP;
  const double* row = part + (size_t)col * nblk;
  double s = 0.0;
  for (int b0 = threadIdx.x; b0 < nblk; b0 += 8 * 256) {
    double v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = b0 + i * 256 < nblk ? row[b0 + i * 256] : 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (b0 + i * 256 < nblk) s += v[i];
  }
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (total) total[e] = sh[0];
    if (out && e < E) out[e] = (float)sh[0];
  }
}

}  // namespace moe
