// Combine with the residual, and the load-balance statistics.
//
// Method: page "MoE 与专家并行": the layer output h'_t = u_t + sum_i g_{i,t}
// FFN_i(u_t) (section "从稠密 FFN 到 MoE", eq. h'_t) with dropped assignments
// contributing nothing (section "专家容量与丢 token"); f_i, P_i and
// L_aux = E * sum f_i P_i (section "负载均衡辅助损失：推导与梯度"); MaxVio
// (section "无辅助损失的负载均衡").
//
// Combine is a weighted gather: one wave per token reads its residual row and
// its kept expert rows (16 bytes per lane per step), accumulates in float32 in
// rank order and writes the row once.  No atomics, so the result is
// deterministic and each output byte is written exactly once.
#include <limits.h>

#include <type_traits>

#include "blocks.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// KM: the most ranks a token may have (k <= KM), which sizes the loads held
// in flight
template <typename TE, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const TE* U, const TE* Y,
                                                      const int32_t* slot, const float* gate,
                                                      const TE* Ys, int ns, TE* out, int T, int h,
                                                      int k) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int sl[KM];
  float g[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) {
    sl[r] = r < k ? slot[(size_t)t * k + r] : -1;
    g[r] = r < k ? gate[(size_t)t * k + r] : 0.f;
  }
  constexpr int V = Elem<TE>::kPer16B;
  const int nvec = h / V;
  const TE* u = U + (size_t)t * h;
  TE* o = out + (size_t)t * h;
  // a dropped rank reads the token's own row (always valid) and adds nothing
  const TE* src[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) src[r] = sl[r] >= 0 ? Y + (size_t)sl[r] * h : u;
  // two 16-byte vectors per lane and pass, every row's loads issued before
  // the sums (which stay in the same order: residual, shared experts, ranks)
  for (int i0 = lane; i0 < nvec; i0 += 128) {
    const int i1 = i0 + 64;
    const bool two = i1 < nvec;
    const size_t v0 = (size_t)i0 * V, v1 = (size_t)(two ? i1 : i0) * V;
    const u32x4 a0 = ld16(u + v0), a1 = ld16(u + v1);
    u32x4 b0[KM], b1[KM];
#pragma unroll
    for (int r = 0; r < KM; ++r)
      if (r < k) {
        b0[r] = ld16(src[r] + v0);
        b1[r] = ld16(src[r] + v1);
      }
    float acc0[V], acc1[V], y[V];
    Elem<TE>::unpack(a0, acc0);
    Elem<TE>::unpack(a1, acc1);
    for (int q = 0; q < ns; ++q) {  // shared experts, weight 1, in order
      const TE* ys = Ys + ((size_t)q * T + t) * h;
      Elem<TE>::unpack(ld16(ys + v0), y);
#pragma unroll
      for (int c = 0; c < V; ++c) acc0[c] += y[c];
      Elem<TE>::unpack(ld16(ys + v1), y);
#pragma unroll
      for (int c = 0; c < V; ++c) acc1[c] += y[c];
    }
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      if (r >= k) continue;
      const bool kept = sl[r] >= 0;
      Elem<TE>::unpack(b0[r], y);
#pragma unroll
      for (int c = 0; c < V; ++c) acc0[c] = kept ? fmaf(g[r], y[c], acc0[c]) : acc0[c];
      Elem<TE>::unpack(b1[r], y);
#pragma unroll
      for (int c = 0; c < V; ++c) acc1[c] = kept ? fmaf(g[r], y[c], acc1[c]) : acc1[c];
    }
    st16(o + v0, Elem<TE>::pack(acc0));
    if (two) st16(o + v1, Elem<TE>::pack(acc1));
  }
}

__global__ __launch_bounds__(256) void stats_kernel(StatsParams p) {
  const int e = threadIdx.x;
  stats_block(p, e, e < p.E ? p.count[e] : 0, e < p.E ? p.kept[e] : 0);
}

// Loss-free balancing bias step (page "MoE 与专家并行", section
// "无辅助损失的负载均衡", equations e_i and b_i): e = mean count - count[e],
// b[e] += gamma * sign(e).  The mean is compared exactly: E * count[e]
// against the integer total.
__global__ __launch_bounds__(256) void update_bias_kernel(const int32_t* count, float* b,
                                                          float gamma, int E) {
  __shared__ long long s_tot[256];
  const int e = threadIdx.x;
  s_tot[e] = e < E ? (long long)count[e] : 0;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (e < w) s_tot[e] += s_tot[e + w];
    __syncthreads();
  }
  if (e < E) {
    const long long scaled = (long long)E * count[e];  // E * c_e vs the total
    const float step = scaled < s_tot[0] ? gamma : (scaled > s_tot[0] ? -gamma : 0.f);
    b[e] += step;
  }
}

// Router z-loss of given float32 logits [T][E] (section "各家的变体",
// subsection "Router z-loss 与数值稳定", eq. L_z): one workgroup of 16 waves,
// wave w takes tokens w, w + 16, ...; a token's E <= 256 logits are spread
// over the 64 lanes, LSE = max + log sum exp(x - max) by butterfly
// reductions; per-wave float64 sums are added in wave order.
__global__ __launch_bounds__(1024) void z_loss_kernel(const float* logits, int T, int E,
                                                      float* z_loss) {
  __shared__ double s_w[16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double acc = 0.0;
  for (int t = wave; t < T; t += 16) {
    const float* row = logits + (size_t)t * E;
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = lane + 64 * j < E ? row[lane + 64 * j] : -INFINITY;
    const float m = wave_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) z += lane + 64 * j < E ? expf(x[j] - m) : 0.f;
    const float lse = m + logf(wave_sum(z));
    acc += (double)lse * (double)lse;
  }
  if (lane == 0) s_w[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int w = 0; w < 16; ++w) s += s_w[w];
    z_loss[0] = T > 0 ? (float)(s / T) : 0.f;
  }
}

}  // namespace

hipError_t launch_z_loss(const float* logits, int T, int E, float* z_loss, hipStream_t s) {
  hipLaunchKernelGGL(z_loss_kernel, dim3(1), dim3(1024), 0, s, logits, T, E, z_loss);
  return hipGetLastError();
}

hipError_t launch_combine(const void* U, const void* Y, const int32_t* slot, const float* gate,
                          const void* Ys, int ns, void* out, int T, int h, int k, int bf16_,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!Ys) ns = 0;
  dim3 grid((T + 3) / 4);
  auto go = [&](auto km) {
    constexpr int KM = decltype(km)::value;
    if (bf16_)
      hipLaunchKernelGGL((combine_kernel<bf16, KM>), grid, dim3(256), 0, s,
                         static_cast<const bf16*>(U), static_cast<const bf16*>(Y), slot, gate,
                         static_cast<const bf16*>(Ys), ns, static_cast<bf16*>(out), T, h, k);
    else
      hipLaunchKernelGGL((combine_kernel<float, KM>), grid, dim3(256), 0, s,
                         static_cast<const float*>(U), static_cast<const float*>(Y), slot, gate,
                         static_cast<const float*>(Ys), ns, static_cast<float*>(out), T, h, k);
  };
  if (k <= 2) go(std::integral_constant<int, 2>{});
  else go(std::integral_constant<int, 8>{});
  return hipGetLastError();
}

hipError_t launch_update_bias(const int32_t* count, float* b, float gamma, int E, hipStream_t s) {
  hipLaunchKernelGGL(update_bias_kernel, dim3(1), dim3(256), 0, s, count, b, gamma, E);
  return hipGetLastError();
}

hipError_t launch_stats(const StatsParams& p, hipStream_t s) {
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
