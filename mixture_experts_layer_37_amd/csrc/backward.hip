// Backward pass of the layer: gradients of L = <dOut, out> + alpha aux +
// c_z L_z with respect to U, W_r, b_r and the experts' W_gate, W_up, W_down,
// for the routing the forward chose (top-k and the capacity cut carry no
// gradient).
//
// Method: page "MoE 与专家并行".  The gradient reaching a gate is the inner
// product of the upstream gradient with that expert's output, and it flows on
// through the score function to the logits, W_r and u_t (section
// "路由器：打分、top-k、加权求和", equation dL/dg).  The load-balance term's
// logit gradient is s_k (f_k - sum_i f_i s_i) per token (softmax scores), and
// s'_k (1 - s_k) (f_k - sum_i f_i s'_i) with s' = s / sum_j s (sigmoid), times
// E / T for aux = E sum f P (section "负载均衡辅助损失：推导与梯度").  The
// z-loss's is (2 / T) LSE softmax (section "各家的变体", "Router z-loss").  The
// expert products run backward as grouped products for the inputs and for the
// weights (section "专家计算：padding、block-sparse 与 grouped GEMM").
//
// Noisy routing adds the softplus branch of the router's noise term (router
// section, eq. G(x)); shared experts take dOut as their output gradient
// (section "细粒度专家与共享专家").
//
// This file holds the element-wise kernels, the router's backward and the
// small float32 products (dU, dW_r, the noise term); the grouped products are
// the GEMM kernels of ffn.hip.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// Combine backward, one wave per token: dY[slot] = g dOut_t for every kept
// rank, and dgate[t, r] = dOut_t . Y[slot] (0 for a dropped rank).
__global__ __launch_bounds__(256) void combine_bwd_kernel(const bf16* dOut, const bf16* Y,
                                                          const int32_t* slot, const float* gate,
                                                          bf16* dY, float* dgate, int T, int h,
                                                          int k) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int nvec = h / 8;
  const bf16* d = dOut + (size_t)t * h;
  for (int r = 0; r < k; ++r) {
    const int row = slot[(size_t)t * k + r];
    float acc = 0.f;
    if (row >= 0) {
      const float g = gate[(size_t)t * k + r];
      const bf16* y = Y + (size_t)row * h;
      bf16* dy = dY + (size_t)row * h;
      for (int i = lane; i < nvec; i += 64) {
        float a[8], b[8];
        Elem<bf16>::unpack(ld16(d + (size_t)i * 8), a);
        Elem<bf16>::unpack(ld16(y + (size_t)i * 8), b);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          acc = fmaf(a[q], b[q], acc);
          a[q] *= g;
        }
        st16(dy + (size_t)i * 8, Elem<bf16>::pack(a));
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) dgate[(size_t)t * k + r] = acc;
  }
}

// SwiGLU backward: a = SiLU(g) u gives dg = da u SiLU'(g) and du = da SiLU(g),
// with SiLU'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))).  GU and dGU hold
// [rows][2f] (g or dg in columns 0..f-1, u or du after); rows past offset[E]
// are left alone.  Eight elements per thread.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const bf16* dA, const bf16* GU,
                                                         const int32_t* offset, int E, int f,
                                                         bf16* dGU) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per = f / 8;
  const int64_t row = i / per;
  if (row >= offset[E]) return;
  const int c = (int)(i - row * per) * 8;
  float da[8], g[8], u[8], dg[8], du[8];
  Elem<bf16>::unpack(ld16(dA + row * f + c), da);
  Elem<bf16>::unpack(ld16(GU + row * 2 * f + c), g);
  Elem<bf16>::unpack(ld16(GU + row * 2 * f + f + c), u);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float sg = 1.f / (1.f + expf(-g[q]));
    du[q] = da[q] * g[q] * sg;
    dg[q] = da[q] * u[q] * sg * (1.f + g[q] * (1.f - sg));
  }
  st16(dGU + row * 2 * f + c, Elem<bf16>::pack(dg));
  st16(dGU + row * 2 * f + f + c, Elem<bf16>::pack(du));
}

// Router backward, one wave per token: scores from the float32 logits, the
// gates' gradient back to the scores (raw: ds = dg; renormalised over the
// selected set S: ds_j = (dg_j - sum_i dg_i g_i) / sum_S s), then to the
// logits (softmax: s (ds - <ds, s>); sigmoid: ds s (1 - s)), plus alpha times
// the aux-loss gradient and c_z times the z-loss gradient.  E <= 256.
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* logits, const int32_t* idx,
                                                         const float* gate, const float* dgate,
                                                         const int32_t* count, int T, int E,
                                                         int k, int score, int renorm,
                                                         float alpha, float c_z, float* dH) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  float x[4], s[4], ds[4], fr[4];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    x[j] = e < E ? logits[(size_t)t * E + e] : -INFINITY;
    fr[j] = e < E ? (float)count[e] / ((float)T * k) : 0.f;
    m = fmaxf(m, x[j]);
  }
  m = wave_max(m);
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    const float ex = e < E ? expf(x[j] - m) : 0.f;
    s[j] = ex;  // softmax numerators for now
    z += ex;
  }
  z = wave_sum(z);
  const float lse = m + logf(z);
  float sm[4];  // softmax of the logits (for the z-loss term)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sm[j] = s[j] / z;
    s[j] = score == 0 ? sm[j] : ((lane + 64 * j < E) ? 1.f / (1.f + expf(-x[j])) : 0.f);
    ds[j] = 0.f;
  }
  // gates -> scores over the selected experts
  float ssel = 0.f, dgg = 0.f;
  for (int r = 0; r < k; ++r) {
    const int e = idx[(size_t)t * k + r];
    float se = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == e) se = s[j];
    ssel += __shfl(se, e & 63, 64);
    dgg += dgate[(size_t)t * k + r] * gate[(size_t)t * k + r];
  }
  for (int r = 0; r < k; ++r) {
    const int e = idx[(size_t)t * k + r];
    const float dg = dgate[(size_t)t * k + r];
    const float v = renorm ? (dg - dgg) / ssel : dg;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == e) ds[j] += v;
  }
  float dh[4];
  if (score == 0) {
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) dot += ds[j] * s[j];
    dot = wave_sum(dot);
#pragma unroll
    for (int j = 0; j < 4; ++j) dh[j] = s[j] * (ds[j] - dot);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) dh[j] = ds[j] * s[j] * (1.f - s[j]);
  }
  if (alpha != 0.f) {
    float ssum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) ssum += s[j];
    ssum = wave_sum(ssum);
    float fw = 0.f;  // sum_i f_i s_i (softmax) or sum_i f_i s'_i (sigmoid)
#pragma unroll
    for (int j = 0; j < 4; ++j) fw += fr[j] * (score == 0 ? s[j] : s[j] / ssum);
    fw = wave_sum(fw);
    const float c = alpha * (float)E / (float)T;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dh[j] += score == 0 ? c * s[j] * (fr[j] - fw)
                          : c * (s[j] / ssum) * (1.f - s[j]) * (fr[j] - fw);
  }
  if (c_z != 0.f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dh[j] += c_z * 2.f / (float)T * lse * sm[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E) dH[(size_t)t * E + e] = dh[j];
  }
}

// dU = dOut + sum over kept ranks of dX[slot] + dH W_r^T (+ dZ W_noise^T
// for noisy routing, + the shared experts' dXs[i]).  A workgroup takes 64
// tokens x 128 columns j (a thread 4 tokens x 8 consecutive columns, so dOut,
// dX and dU move 16 bytes at a time); the products over the experts run in
// chunks of 32 with dH^T and W_r^T staged in LDS as float32.
constexpr int kGiT = 64, kGiJ = 128, kGiK = 32;

__global__ __launch_bounds__(256) void grad_input_kernel(const bf16* dOut, const bf16* dX,
                                                         const int32_t* slot, const float* dH,
                                                         const bf16* W_r, const float* dZ,
                                                         const bf16* W_n, const bf16* dXs,
                                                         int ns, bf16* dU, int T, int h, int E,
                                                         int k) {
  __shared__ __align__(16) float sh[kGiK][kGiT];  // sh[e][t] = dH[t0 + t][e0 + e]
  __shared__ __align__(16) float sw[kGiK][kGiJ];  // sw[e][j] = W_r[j0 + j][e0 + e]
  const int t0 = blockIdx.x * kGiT, j0 = blockIdx.y * kGiJ;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = 0.f;
  // the experts of (dH, W_r), then those of (dZ, W_noise), kGiK at a time
  const int chunks = (E + kGiK - 1) / kGiK;
  for (int c = 0; c < (dZ ? 2 * chunks : chunks); ++c) {
    const bool second = c >= chunks;
    const float* D = second ? dZ : dH;
    const bf16* W = second ? W_n : W_r;
    const int eb = (second ? c - chunks : c) * kGiK;
    const int kc = min(kGiK, E - eb);
    for (int i = threadIdx.x; i < kGiT * kGiK; i += 256) {
      const int tt = i / kGiK, ee = i % kGiK, t = t0 + tt, e = eb + ee;
      sh[ee][tt] = (t < T && ee < kc) ? D[(size_t)t * E + e] : 0.f;
    }
    for (int i = threadIdx.x; i < kGiJ * kGiK; i += 256) {
      const int jj = i / kGiK, ee = i % kGiK, j = j0 + jj;
      sw[ee][jj] = (j < h && ee < kc) ? bf16_to_f32(W[(size_t)j * E + eb + ee]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int ee = 0; ee < kc; ++ee) {
      const float4 a = *reinterpret_cast<const float4*>(&sh[ee][ty * 4]);
      const float4 b0 = *reinterpret_cast<const float4*>(&sw[ee][tx * 8]);
      const float4 b1 = *reinterpret_cast<const float4*>(&sw[ee][tx * 8 + 4]);
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][q] = fmaf(av[i], bv[q], acc[i][q]);
    }
    __syncthreads();
  }
  const int j = j0 + tx * 8;
  if (j >= h) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) break;
    float v[8], x[8];
    Elem<bf16>::unpack(ld16(dOut + (size_t)t * h + j), v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] += acc[i][q];
    for (int r = 0; r < k; ++r) {
      const int row = slot[(size_t)t * k + r];
      if (row < 0) continue;
      Elem<bf16>::unpack(ld16(dX + (size_t)row * h + j), x);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += x[q];
    }
    for (int i2 = 0; i2 < ns; ++i2) {
      Elem<bf16>::unpack(ld16(dXs + ((size_t)i2 * T + t) * h + j), x);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += x[q];
    }
    st16(dU + (size_t)t * h + j, Elem<bf16>::pack(v));
  }
}

// Noisy routing: the logits hold z * softplus(Z) with Z = U W_noise, so
// dZ = dH * z * sigmoid(Z) (softplus' = sigmoid; page "MoE 与专家并行",
// router section, eq. G(x)); z, the forward's standard-normal draw of the
// pair, is drawn again from its counter.  Z is recomputed in float32: a workgroup takes
// 64 tokens x 64 experts, stages 32 columns of U (transposed) and of W_noise
// at a time in LDS, and a thread accumulates 4 tokens x 4 experts.
__global__ __launch_bounds__(256) void noise_grad_kernel(const bf16* U, const bf16* W_n,
                                                         const float* dH, uint64_t seed,
                                                         uint64_t rng_offset, float* dZ, int T,
                                                         int h, int E) {
  __shared__ __align__(16) float su[32][64];  // su[j][t] = U[t0 + t][j0 + j]
  __shared__ __align__(16) float sw[32][64];  // sw[j][e] = W_noise[j0 + j][e0 + e]
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // 4 experts, 4 tokens
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.f;
  for (int j0 = 0; j0 < h; j0 += 32) {  // h is a multiple of 64
    {
      const int tt = threadIdx.x >> 2, jj = (threadIdx.x & 3) * 8, t = t0 + tt;
      float v[8];
      if (t < T) {
        Elem<bf16>::unpack(ld16(U + (size_t)t * h + j0 + jj), v);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = 0.f;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) su[jj + q][tt] = v[q];
    }
    for (int i = threadIdx.x; i < 32 * 64; i += 256) {
      const int jj = i >> 6, ee = i & 63, e = e0 + ee;
      sw[jj][ee] = e < E ? bf16_to_f32(W_n[(size_t)(j0 + jj) * E + e]) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int jj = 0; jj < 32; ++jj) {
      const float4 a = *reinterpret_cast<const float4*>(&su[jj][ty * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&sw[jj][tx * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(av[i], bv[q], acc[i][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + tx * 4 + q;
      if (e >= E) break;
      const size_t o = (size_t)t * E + e;
      const float z = (float)philox_normal(seed, (uint64_t)o + rng_offset);
      dZ[o] = dH[o] * z / (1.f + __expf(-acc[i][q]));
    }
  }
}

// dW_r[j][e] = sum_t U[t][j] dH[t][e] and db_r[e] = sum_t dH[t][e] in
// float32, computed as one product in which U has an extra column of ones
// (j = h).  Workgroup (jt, et, s) takes TJ x TE outputs over the tokens of
// split s, stages 16 tokens of U and dH at a time in LDS as float32, and a
// thread accumulates 4 x 4 outputs; the splits' partials part[s][j][e] are
// summed in split order by dwr_reduce_kernel (deterministic).
template <int TE>
__global__ __launch_bounds__(256) void dwr_part_kernel(const bf16* U, const float* dH,
                                                       float* part, int T, int h, int E,
                                                       int tchunk) {
  constexpr int NE = TE / 4, NJ = 256 / NE, TJ = 4 * NJ, KC = 16;
  __shared__ __align__(16) float su[KC][TJ];
  __shared__ __align__(16) float sd[KC][TE];
  const int j0 = blockIdx.x * TJ, e0 = blockIdx.y * TE;
  const int tb = blockIdx.z * tchunk, tend = min(T, tb + tchunk);
  const int tx = threadIdx.x % NE, ty = threadIdx.x / NE;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.f;
  const bool vec_e = (E & 3) == 0;
  for (int t0 = tb; t0 < tend; t0 += KC) {
    for (int i = threadIdx.x; i < KC * (TJ / 8); i += 256) {
      const int tt = i / (TJ / 8), jj = (i % (TJ / 8)) * 8, t = t0 + tt, j = j0 + jj;
      float v[8];
      if (t < tend && j < h) {  // h is a multiple of 8
        Elem<bf16>::unpack(ld16(U + (size_t)t * h + j), v);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = (t < tend && j + q == h) ? 1.f : 0.f;
      }
      *reinterpret_cast<float4*>(&su[tt][jj]) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(&su[tt][jj + 4]) = make_float4(v[4], v[5], v[6], v[7]);
    }
    for (int i = threadIdx.x; i < KC * NE; i += 256) {
      const int tt = i / NE, ee = (i % NE) * 4, t = t0 + tt, e = e0 + ee;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < tend) {
        const float* src = dH + (size_t)t * E + e;
        if (vec_e && e + 4 <= E) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          v.x = e < E ? src[0] : 0.f;
          v.y = e + 1 < E ? src[1] : 0.f;
          v.z = e + 2 < E ? src[2] : 0.f;
          v.w = e + 3 < E ? src[3] : 0.f;
        }
      }
      *reinterpret_cast<float4*>(&sd[tt][ee]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < KC; ++tt) {
      const float4 a = *reinterpret_cast<const float4*>(&su[tt][ty * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&sd[tt][tx * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(av[i], bv[q], acc[i][q]);
    }
    __syncthreads();
  }
  float* P = part + (size_t)blockIdx.z * (size_t)(h + 1) * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = j0 + ty * 4 + i;
    if (j > h) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + tx * 4 + q;
      if (e < E) P[(size_t)j * E + e] = acc[i][q];
    }
  }
}

__global__ __launch_bounds__(256) void dwr_reduce_kernel(const float* part, int nsplit, int h,
                                                         int E, float* dWr, float* db) {
  const size_t n = (size_t)(h + 1) * E;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float s = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) s += part[(size_t)sp * n + i];
    if (i < (size_t)h * E) dWr[i] = s;
    else if (db) db[i - (size_t)h * E] = s;
  }
}

}  // namespace

hipError_t launch_combine_bwd(const void* dOut, const void* Y, const int32_t* slot,
                              const float* gate, void* dY, float* dgate, int T, int h, int k,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_bwd_kernel, dim3((T + 3) / 4), dim3(256), 0, s,
                     static_cast<const bf16*>(dOut), static_cast<const bf16*>(Y), slot, gate,
                     static_cast<bf16*>(dY), dgate, T, h, k);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* dA, const void* GU, const int32_t* offset, int E,
                             int64_t rows_max, int f, void* dGU, hipStream_t s) {
  const int64_t n = rows_max * (f / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16*>(dA), static_cast<const bf16*>(GU), offset, E, f,
                     static_cast<bf16*>(dGU));
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* logits, const int32_t* idx, const float* gate,
                             const float* dgate, const int32_t* count, int T, int E, int k,
                             int score, int renorm, float alpha, float c_z, float* dH,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(router_bwd_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, idx, gate,
                     dgate, count, T, E, k, score, renorm, alpha, c_z, dH);
  return hipGetLastError();
}

hipError_t launch_grad_input(const void* dOut, const void* dX, const int32_t* slot,
                             const float* dH, const void* W_r, const float* dZ,
                             const void* W_noise, const void* dXs, int ns, void* dU, int T, int h,
                             int E, int k, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(grad_input_kernel, dim3((T + kGiT - 1) / kGiT, (h + kGiJ - 1) / kGiJ),
                     dim3(256), 0, s, static_cast<const bf16*>(dOut),
                     static_cast<const bf16*>(dX), slot, dH, static_cast<const bf16*>(W_r), dZ,
                     static_cast<const bf16*>(W_noise), static_cast<const bf16*>(dXs), ns,
                     static_cast<bf16*>(dU), T, h, E, k);
  return hipGetLastError();
}

hipError_t launch_noise_grad(const void* U, const void* W_noise, const float* dH,
                             uint64_t seed, uint64_t rng_offset, float* dZ, int T, int h, int E,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(noise_grad_kernel, dim3((T + 63) / 64, (E + 63) / 64), dim3(256), 0, s,
                     static_cast<const bf16*>(U), static_cast<const bf16*>(W_noise), dH, seed,
                     rng_offset, dZ, T, h, E);
  return hipGetLastError();
}

hipError_t launch_dwr(const void* U, const float* dH, float* dWr, float* db, float* part, int T,
                      int h, int E, hipStream_t s) {
  const DwrPlan p = dwr_plan(T, h, E);
  const dim3 grid(p.jt, p.et, p.nsplit);
  const bf16* u = static_cast<const bf16*>(U);
  switch (p.te) {
    case 8:
      hipLaunchKernelGGL(dwr_part_kernel<8>, grid, dim3(256), 0, s, u, dH, part, T, h, E,
                         p.tchunk);
      break;
    case 16:
      hipLaunchKernelGGL(dwr_part_kernel<16>, grid, dim3(256), 0, s, u, dH, part, T, h, E,
                         p.tchunk);
      break;
    case 32:
      hipLaunchKernelGGL(dwr_part_kernel<32>, grid, dim3(256), 0, s, u, dH, part, T, h, E,
                         p.tchunk);
      break;
    default:
      hipLaunchKernelGGL(dwr_part_kernel<64>, grid, dim3(256), 0, s, u, dH, part, T, h, E,
                         p.tchunk);
      break;
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t n = (size_t)(h + 1) * E;
  const unsigned nb = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(dwr_reduce_kernel, dim3(nb), dim3(256), 0, s, part, p.nsplit, h, E, dWr, db);
  return hipGetLastError();
}

}  // namespace moe
