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
// rank, and dgate[t, r] = dOut_t . Y[slot] (0 for a dropped rank).  A lane
// takes one 16-byte vector of the row per pass: dOut's once, and those of the
// KM rank rows (a dropped or absent rank reads dOut's row, masked to +0, and
// stores nothing).  The next pass's loads are issued before this pass's
// stores, since a load queued behind a store waits for it; each rank's dot
// product runs over the lane's vectors in row order, as before the split.
template <int KM>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const bf16* dOut, const bf16* Y,
                                                          const int32_t* slot, const float* gate,
                                                          bf16* dY, float* dgate, int T, int h,
                                                          int k) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int nvec = h / 8, iters = (nvec + 63) / 64;
  const bf16* d = dOut + (size_t)t * h;
  int sl[KM];
  float g[KM], acc[KM];
  const bf16* src[KM];
  uint32_t keep[KM];
  int sv[KM];
  float gv[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) {  // all issued at once, clamped to rank k - 1
    sv[r] = slot[(size_t)t * k + min(r, k - 1)];
    gv[r] = gate[(size_t)t * k + min(r, k - 1)];
  }
#pragma unroll
  for (int r = 0; r < KM; ++r) {
    sl[r] = r < k ? sv[r] : -1;
    g[r] = r < k ? gv[r] : 0.f;
    acc[r] = 0.f;
    src[r] = sl[r] >= 0 ? Y + (size_t)sl[r] * h : d;
    keep[r] = sl[r] >= 0 ? 0xffffffffu : 0u;
  }
  // rank r's dY row as a buffer (the wave's token, so the row is uniform)
  __amdgpu_buffer_rsrc_t rdy[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) {
    const int row = __builtin_amdgcn_readfirstlane(sl[r]);
    rdy[r] = make_rsrc(dY + (size_t)(row >= 0 ? row : 0) * h, row >= 0 ? (size_t)h * 2 : 0);
  }
  u32x4 bd[2], by[2][KM];
  // loads of pass it (lanes past the row re-read its last vector, and their
  // rank vectors are masked to +0)
  auto issue = [&](int it, u32x4& od, u32x4* oy) __attribute__((always_inline)) {
    const int i = lane + 64 * it;
    const size_t v = (size_t)min(i, nvec - 1) * 8;
    const uint32_t in = i < nvec ? 0xffffffffu : 0u;
    od = ld16(d + v);
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      const bf16* q = src[r] + v;
      asm("" : "+v"(q));  // keeps the load unconditional (see grad_input_kernel)
      const uint32_t m = keep[r] & in;
      oy[r] = *(const __attribute__((address_space(1))) u32x4*)q & u32x4{m, m, m, m};
    }
  };
  auto consume = [&](int it, const u32x4& od, const u32x4* oy) __attribute__((always_inline)) {
    const int i = lane + 64 * it;
    float a[8], y[8];
    Elem<bf16>::unpack(od, a);
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      Elem<bf16>::unpack(oy[r], y);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[r] = fmaf(a[q], y[q], acc[r]);
    }
    // buffer stores, one per rank and pass whatever the rank: a dropped
    // rank's or a lane's past the row is sent past the row's end and
    // dropped, so no branch hides from the waits how many are in flight
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      float o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = a[q] * g[r];
      __builtin_amdgcn_raw_buffer_store_b128(Elem<bf16>::pack(o), rdy[r],
                                             sl[r] >= 0 && i < nvec ? i * 16 : kPastEnd, 0, 0);
    }
  };
  issue(0, bd[0], by[0]);
  for (int it = 0; it < iters; it += 2) {
    if (it + 1 < iters) issue(it + 1, bd[1], by[1]);
    consume(it, bd[0], by[0]);
    if (it + 1 >= iters) break;
    if (it + 2 < iters) issue(it + 2, bd[0], by[0]);
    consume(it + 1, bd[1], by[1]);
  }
#pragma unroll
  for (int r = 0; r < KM; ++r) {
    if (r >= k) break;
    const float v = wave_sum(acc[r]);
    if (lane == 0) dgate[(size_t)t * k + r] = v;
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
// tokens x 128 columns j; its four waves (2 x 2) each form 32 tokens x 64
// columns of the product on 16x16x32 bf16 MFMA, with the experts as the
// contraction.  Both operands are read straight from memory, since rows of dH
// [T, E] and of W_r [h, E] already run along the experts.  dH (float32) enters
// as hi + lo, hi = bf16(dH) and lo = bf16(dH - hi); W_r is exact in bf16, so
// the two products carry dH to about 2^-17 relative, summed in float32.  The
// float32 tile then passes through LDS to a layout of 4 rows x 8 consecutive
// columns per thread, in which dOut and the dX rows (16 bytes a load) are
// added.  Row i + 1's loads are issued before row i's store, since a load
// queued behind a store waits for it.  VEC: E % 8 == 0 and 16-byte aligned
// operands; KM: the bound on k the gather is unrolled for; SH: the first
// shared expert's row joins the rows loaded ahead (ns > 0).
constexpr int kGiT = 64, kGiJ = 128;

// The operand loads read D[row][e .. e + 7] and W[row][e .. e + 7] with the
// address clamped into the row, so no lane reads out of bounds; the values
// past E are zeroed when the step is consumed (gi_mask), not at the load,
// so that waiting for them does not hold up the step before.
template <bool VEC>
__device__ __forceinline__ void gi_load_a(const float* D, size_t row, int e, int E, float* v) {
  if constexpr (VEC) {
    const float* p = D + row * E + min(e, E - 8);
    Elem<float>::unpack(ld16(p), v);
    Elem<float>::unpack(ld16(p + 4), v + 4);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = D[row * E + min(e + q, E - 1)];
  }
}

template <bool VEC>
__device__ __forceinline__ u32x4 gi_load_b(const bf16* W, size_t row, int e, int E) {
  if constexpr (VEC) {
    return ld16(W + row * E + min(e, E - 8));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = uint32_t(W[row * E + min(e + 2 * q, E - 1)]) |
             (uint32_t(W[row * E + min(e + 2 * q + 1, E - 1)]) << 16);
    return u32x4{w[0], w[1], w[2], w[3]};
  }
}

// zero the values of experts e + q >= E (q = 0 .. 7); with VEC, E % 8 == 0,
// so the eight are all in or all out
template <bool VEC>
__device__ __forceinline__ void gi_mask_a(float* v, int e, int E) {
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = (VEC ? e : e + q) < E ? v[q] : 0.f;
}

template <bool VEC>
__device__ __forceinline__ bf16x8 gi_mask_b(u32x4 w, int e, int E) {
  if constexpr (VEC) {
    if (e >= E) w = u32x4{0u, 0u, 0u, 0u};
  } else {
    uint32_t m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      m[q] = (e + 2 * q < E ? 0xffffu : 0u) | (e + 2 * q + 1 < E ? 0xffff0000u : 0u);
    w &= u32x4{m[0], m[1], m[2], m[3]};
  }
  bf16x8 r;
  __builtin_memcpy(&r, &w, 16);
  return r;
}

// x = hi + lo + O(2^-18 |x|), both halves bf16 (round to nearest even)
__device__ __forceinline__ void gi_split(const float* x, bf16x8& hi, bf16x8& lo) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hw[q] = pack_bf16x2(x[2 * q], x[2 * q + 1]);
    const float r0 = x[2 * q] - __uint_as_float(hw[q] << 16);
    const float r1 = x[2 * q + 1] - __uint_as_float(hw[q] & 0xffff0000u);
    lw[q] = pack_bf16x2(r0, r1);
  }
  __builtin_memcpy(&hi, hw, 16);
  __builtin_memcpy(&lo, lw, 16);
}

template <bool VEC, int KM, bool SH>
__global__ __launch_bounds__(256) void grad_input_kernel(const bf16* dOut, const bf16* dX,
                                                         const int32_t* slot, const float* dH,
                                                         const bf16* W_r, const float* dZ,
                                                         const bf16* W_n, const bf16* dXs,
                                                         int ns, bf16* dU, int T, int h, int E,
                                                         int k) {
  __shared__ __align__(16) float tile[kGiT][kGiJ + 4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave & 1, wn = wave >> 1, l16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * kGiT, j0 = blockIdx.y * kGiJ;
  floatx4 acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  // this lane's operand rows: tokens past T read row T - 1 and columns past
  // h row h - 1 (their results are never stored)
  size_t ar[2], br[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) ar[mb] = (size_t)min(t0 + wm * 32 + 16 * mb + l16, T - 1);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) br[nb] = (size_t)min(j0 + wn * 64 + 16 * nb + l16, h - 1);
  // the experts of (dH, W_r), then those of (dZ, W_noise), 32 per step
  const int per = (E + 31) / 32, steps = dZ ? 2 * per : per;
  float a[2][8];
  u32x4 b[4];
  int el = 0;  // this lane's first expert in the loaded step
  auto load = [&](int st) __attribute__((always_inline)) {
    const bool second = st >= per;
    const float* D = second ? dZ : dH;
    const bf16* W = second ? W_n : W_r;
    el = (second ? st - per : st) * 32 + 8 * g;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) gi_load_a<VEC>(D, ar[mb], el, E, a[mb]);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) b[nb] = gi_load_b<VEC>(W, br[nb], el, E);
  };
  // The gather: a thread's rows are ty + 16 i (rows past T read row T - 1
  // and store nothing), its columns 8 tx .. 8 tx + 7.  Its first row's loads
  // go out right after the product's first operand loads, so that their
  // latency overlaps the product.
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  // h % 64 == 0: the last tile may hold only 64 columns; the threads past
  // them read the last valid columns and store nothing
  const bool jin = j0 + tx * 8 < h;
  const size_t j = (size_t)min(j0 + tx * 8, h - 8);
  int tr[4], sl[4][KM];
#pragma unroll
  for (int i = 0; i < 4; ++i) tr[i] = min(t0 + ty + 16 * i, T - 1);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < KM; ++q) {
      const int v = slot[(size_t)tr[i] * k + min(q, k - 1)];
      sl[i][q] = q < k ? v : -1;
    }
  // per row: dOut, KM rank rows (a dropped or absent rank reads the dOut row
  // again, and its bits are masked to +0) and, with SH, the first shared
  // expert's row.  The rank rows' addresses pass through an empty asm, so
  // that the compiler sees each load as needed and keeps it ahead of the
  // store before it instead of branching around it.
  constexpr int NL = 1 + KM + (SH ? 1 : 0);
  u32x4 buf[2][NL];
  auto issue = [&](int i, u32x4* bb) __attribute__((always_inline)) {
    const bf16* orow = dOut + (size_t)tr[i] * h + j;
    bb[0] = ld16(orow);
#pragma unroll
    for (int q = 0; q < KM; ++q) {
      const bf16* src = sl[i][q] >= 0 ? dX + (size_t)sl[i][q] * h + j : orow;
      asm("" : "+v"(src));
      const uint32_t keep = sl[i][q] >= 0 ? 0xffffffffu : 0u;
      // the address space the asm hid: global memory
      const __attribute__((address_space(1))) u32x4* gp =
          (const __attribute__((address_space(1))) u32x4*)src;
      bb[1 + q] = *gp & u32x4{keep, keep, keep, keep};
    }
    if constexpr (SH) bb[1 + KM] = ld16(dXs + (size_t)tr[i] * h + j);
  };
  load(0);
  issue(0, buf[0]);
  for (int st = 0; st < steps; ++st) {
    bf16x8 hi[2], lo[2], bc[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float am[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) am[q] = a[mb][q];
      gi_mask_a<VEC>(am, el, E);
      gi_split(am, hi[mb], lo[mb]);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) bc[nb] = gi_mask_b<VEC>(b[nb], el, E);
    if (st + 1 < steps) load(st + 1);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[mb], bc[nb], acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[mb], bc[nb], acc[mb][nb], 0, 0, 0);
      }
  }
  // D layout: lane holds column l16 of rows 4 g + i
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        tile[wm * 32 + 16 * mb + 4 * g + i][wn * 64 + 16 * nb + l16] = acc[mb][nb][i];
  __syncthreads();

  if (!jin) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i + 1 < 4) issue(i + 1, buf[(i + 1) & 1]);
    const u32x4* bb = buf[i & 1];
    const int r = ty + 16 * i;
    float v[8], x[8];
    Elem<bf16>::unpack(bb[0], v);
    const float4 p0 = *reinterpret_cast<const float4*>(&tile[r][tx * 8]);
    const float4 p1 = *reinterpret_cast<const float4*>(&tile[r][tx * 8 + 4]);
    v[0] += p0.x, v[1] += p0.y, v[2] += p0.z, v[3] += p0.w;
    v[4] += p1.x, v[5] += p1.y, v[6] += p1.z, v[7] += p1.w;
#pragma unroll
    for (int q = 0; q < KM; ++q) {
      Elem<bf16>::unpack(bb[1 + q], x);
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] += x[c];
    }
    if constexpr (SH) {
      Elem<bf16>::unpack(bb[1 + KM], x);
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] += x[c];
      for (int i2 = 1; i2 < ns; ++i2) {
        Elem<bf16>::unpack(ld16(dXs + ((size_t)i2 * T + tr[i]) * h + j), x);
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] += x[c];
      }
    }
    if (t0 + r < T) st16(dU + (size_t)(t0 + r) * h + j, Elem<bf16>::pack(v));
  }
}

// Noisy routing: the logits hold z * softplus(Z) with Z = U W_noise, so
// dZ = dH * z * sigmoid(Z) (softplus' = sigmoid; page "MoE 与专家并行",
// router section, eq. G(x)); z, the forward's standard-normal draw of the
// pair, is drawn again from its counter.  Z comes from the router's logits
// GEMM run again on W_noise (bf16 MFMA, float32 sums over KS ranges of h),
// summed here in range order.
__global__ __launch_bounds__(256) void noise_grad_kernel(const float* zpart, int KS, int EP,
                                                         const float* dH, uint64_t seed,
                                                         uint64_t rng_offset, float* dZ, int T,
                                                         int E) {
  const size_t o = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= (size_t)T * E) return;
  const int t = (int)(o / E), e = (int)(o % E);
  float z = 0.f;
  for (int ks = 0; ks < KS; ++ks) z += zpart[((size_t)ks * T + t) * EP + e];
  const float n = (float)philox_normal(seed, (uint64_t)o + rng_offset);
  dZ[o] = dH[o] * n / (1.f + __expf(-z));
}

// dW_r[j][e] = sum_t U[t][j] dH[t][e] and db_r[e] = sum_t dH[t][e]: a
// product with the tokens as the contraction, in three launches.
//
// dwr_split_kernel writes dH as bf16 pairs: row t of HL holds, for each tile
// of TE experts, hi = bf16(dH) then lo = bf16(dH - hi) (experts past E zero),
// so that U, exact in bf16, times hi + lo carries dH to about 2^-17
// relative.  A thread takes 8 consecutive experts of one token.
__global__ __launch_bounds__(256) void dwr_split_kernel(const float* D, int T, int E, int TE,
                                                        int EP, bool vec, bf16* HL) {
  const int per = EP / 8;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * per) return;
  const int t = (int)(i / per), e = (int)(i % per) * 8;
  float x[8];
  const float* src = D + (size_t)t * E + e;
  if (vec && e < E) {  // E % 8 == 0, 16-byte aligned rows
    Elem<float>::unpack(ld16(src), x);
    Elem<float>::unpack(ld16(src + 4), x + 4);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = e + q < E ? src[q] : 0.f;
  }
  float hi[8], lo[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    hi[q] = bf16_to_f32(f32_to_bf16(x[q]));
    lo[q] = x[q] - hi[q];
  }
  bf16* row = HL + (size_t)t * 2 * EP + (size_t)(e / TE) * 2 * TE + e % TE;
  st16(row, Elem<bf16>::pack(hi));
  st16(row + TE, Elem<bf16>::pack(lo));
}

// dwr_mfma_kernel: workgroup (expert tile, column tile, token split) forms
// part[split][j][e] for TJ columns j x TE experts over its split's tokens on
// 16x16x32 bf16 MFMA, twice per step (hi, then lo).  Each step's 32 tokens of
// U [32][TJ] and of HL [32][hi TE | lo TE] reach LDS by direct copies (a ring
// of NS stages, 1 KB per copy, rows of the split past T read as zeros), and
// both operands come out of LDS by transposing reads, since U and HL run
// along j and e, not along the tokens.  Waves: GJ x GE, each 64 columns x WE
// experts.  With dsum, the first column tile's first waves also add up the hi
// and lo values they read, per expert, into db_r's partial (row h of part).
struct DwArgs {
  const bf16* U;
  const bf16* HL;
  float* part;  // [nsplit][h + 1][E]
  int T, h, E, EP, tchunk, jtiles, etiles, dsum;
};

template <int TJ, int TE>
struct DwCfg {
  static constexpr int GJ = TJ / 64, GE = 4 / GJ, WE = TE / GE, FE = WE / 16;
  static constexpr int UB = 32 * TJ * 2, HB = 32 * 4 * TE, SB = UB + HB;
  static constexpr int NQ = SB / 1024, NC = (NQ + 3) / 4, NS = 3;
  static_assert(GJ * GE == 4 && FE >= 1 && UB % 1024 == 0 && HB % 1024 == 0, "tile");
};

template <int TJ, int TE>
__global__ __launch_bounds__(256, 2) void dwr_mfma_kernel(DwArgs p) {
  using C = DwCfg<TJ, TE>;
  constexpr int NS = C::NS, NC = C::NC, FE = C::FE, UQ = C::UB / 1024;
  __shared__ __attribute__((aligned(16))) char lds[NS * C::SB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wj = wave % C::GJ, we = wave / C::GJ;
  const int l16 = lane & 15, g = lane >> 4, q = l16 >> 2, jl = l16 & 3;
  // workgroup -> (split, column tile, expert tile); the expert tiles of one
  // column tile, which copy the same U, are consecutive on one XCD
  const int G = gridDim.x;
  const int L = (G & 7) == 0 ? xcd_remap(blockIdx.x, G) : blockIdx.x;
  const int et = L % p.etiles, rest = L / p.etiles;
  const int jt = rest % p.jtiles, sp = rest / p.jtiles;
  const int j0 = jt * TJ, e0 = et * TE;
  const int tb = sp * p.tchunk, tn = max(0, min(p.T, tb + p.tchunk) - tb);
  const int KT = (tn + 31) / 32, h = p.h, HLP = 2 * p.EP;

  // this wave's copies: 1 KB chunks wave + 4 i of a stage (the last chunk
  // repeated where the stage has fewer), U rows then HL rows, each row's
  // 16-byte chunks placed by the wsw swizzle
  int voff[NC], dst[NC];
  bool isu[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int qq = min(wave + 4 * i, C::NQ - 1);
    const int byte = qq * 1024 + lane * 16;
    dst[i] = qq * 1024;
    isu[i] = qq < UQ;
    if (qq < UQ) {
      const int r = byte / (TJ * 2), c = ((byte % (TJ * 2)) >> 4) ^ wsw<TJ / 8>(r);
      voff[i] = r * h * 2 + j0 * 2 + c * 16;
    } else {
      const int b = byte - C::UB, r = b / (4 * TE), c = ((b % (4 * TE)) >> 4) ^ wsw<TE / 4>(r);
      voff[i] = r * HLP * 2 + c * 16;
    }
  }
  // this lane's transposing reads: k-rows 8 g + q (+ 4), columns 4 jl .. +3
  // of fragment column block col0
  int fa[4], fh[FE], fl[FE];
#pragma unroll
  for (int fj = 0; fj < 4; ++fj) {
    const int r = 8 * g + q, c = ((wj * 64 + 16 * fj) >> 3) + (jl >> 1);
    fa[fj] = r * (TJ * 2) + ((c ^ wsw<TJ / 8>(r)) << 4) + 8 * (jl & 1);
  }
#pragma unroll
  for (int fe = 0; fe < FE; ++fe) {
    const int r = 8 * g + q, col = we * C::WE + 16 * fe;
    const int ch = (col >> 3) + (jl >> 1), cl = ((col + TE) >> 3) + (jl >> 1);
    fh[fe] = C::UB + r * (4 * TE) + ((ch ^ wsw<TE / 4>(r)) << 4) + 8 * (jl & 1);
    fl[fe] = C::UB + r * (4 * TE) + ((cl ^ wsw<TE / 4>(r)) << 4) + 8 * (jl & 1);
  }

  floatx4 acc[4][FE];
#pragma unroll
  for (int fj = 0; fj < 4; ++fj)
#pragma unroll
    for (int fe = 0; fe < FE; ++fe) acc[fj][fe] = floatx4{0.f, 0.f, 0.f, 0.f};
  // db_r: this lane's 8 tokens per step of expert column l16, per fragment
  const bool dsum = p.dsum && jt == 0 && wj == 0;
  float ds[FE];
#pragma unroll
  for (int fe = 0; fe < FE; ++fe) ds[fe] = 0.f;

  const size_t ubytes = (size_t)tn * h * 2;
  const size_t hbytes = tn > 0 ? (size_t)tn * HLP * 2 - (size_t)et * TE * 4 : 0;
  // the ring's slots as restrict parameters (and the copies' sources built
  // from restrict pointers): the compiler then tells the copies into one slot
  // from the reads of another and adds no waits beyond the one per step
  auto run = [&](char* __restrict__ s0, char* __restrict__ s1, char* __restrict__ s2,
                 const char* __restrict__ gU, const char* __restrict__ gH)
                 __attribute__((always_inline)) {
    char* const S[3] = {s0, s1, s2};
    const __amdgpu_buffer_rsrc_t rU = make_rsrc(gU, ubytes);
    const __amdgpu_buffer_rsrc_t rH = make_rsrc(gH, hbytes);
    // copies of step cc into slot sl (past the range: no memory traffic, the
    // slot is never read again)
    auto issue = [&](int cc, char* sl) __attribute__((always_inline)) {
      const bool live = cc < KT;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        // the step's offset goes into the lane offset: the range check (rows
        // past the split read as zeros) covers only that one
        if (isu[i])
          dma16(rU, sl + dst[i], live ? voff[i] + cc * 64 * h : kPastEnd, 0);
        else
          dma16(rH, sl + dst[i], live ? voff[i] + cc * 64 * HLP : kPastEnd, 0);
      }
    };
    auto compute = [&](const char* sl) __attribute__((always_inline)) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s lds_v4s;
      auto tr = [&](const char* bp, int step) __attribute__((always_inline)) {
        const v4s v[2] = {__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(bp)),
                          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(bp + step))};
        bf16x8 r;
        __builtin_memcpy(&r, v, 16);
        return r;
      };
      bf16x8 a[4], bh[FE], bl[FE];
#pragma unroll
      for (int fj = 0; fj < 4; ++fj) a[fj] = tr(sl + fa[fj], 4 * TJ * 2);
#pragma unroll
      for (int fe = 0; fe < FE; ++fe) {
        bh[fe] = tr(sl + fh[fe], 4 * 4 * TE);
        bl[fe] = tr(sl + fl[fe], 4 * 4 * TE);
      }
#pragma unroll
      for (int fj = 0; fj < 4; ++fj)
#pragma unroll
        for (int fe = 0; fe < FE; ++fe) {
          acc[fj][fe] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fj], bh[fe], acc[fj][fe], 0, 0, 0);
          acc[fj][fe] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fj], bl[fe], acc[fj][fe], 0, 0, 0);
        }
      if (dsum) {
#pragma unroll
        for (int fe = 0; fe < FE; ++fe) {
          u32x4 uh, ul;
          __builtin_memcpy(&uh, &bh[fe], 16);
          __builtin_memcpy(&ul, &bl[fe], 16);
          float vh[8], vl[8];
          Elem<bf16>::unpack(uh, vh);
          Elem<bf16>::unpack(ul, vl);
#pragma unroll
          for (int k = 0; k < 8; ++k) ds[fe] += vh[k] + vl[k];
        }
      }
    };
    // step c sits in slot c % NS; it waits for its copies, then refills the
    // slot of step c - 1 (every wave is past it) with step c + NS - 1
    auto step = [&](int c, int u) __attribute__((always_inline)) {
      wait_vm_seen<(NS - 2) * NC>();
      wait_lgkm0_seen();
      barrier_only();
      issue(c + NS - 1, S[(u + NS - 1) % NS]);
      compute(S[u]);
    };
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) issue(u, S[u]);
    int c = 0;
    for (; c + NS <= KT; c += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) step(c + u, u);
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (c + u < KT) step(c + u, u);
    wait_vm_seen<0>();  // the last copies (past the range) land before the slots go away
  };
  run(lds, lds + C::SB, lds + 2 * C::SB,
      reinterpret_cast<const char*>(p.U + (size_t)tb * h),
      reinterpret_cast<const char*>(p.HL + (size_t)tb * HLP + (size_t)et * 2 * TE));

  // D layout: lane holds expert column l16 of column rows 4 g + i
  float* P = p.part + (size_t)sp * (h + 1) * p.E;
  if (dsum) {  // the four token groups g of a column, in a fixed order
#pragma unroll
    for (int fe = 0; fe < FE; ++fe) {
      float v = ds[fe];
      v += wave_partner<4>(v);
      v += wave_partner<5>(v);
      const int e = e0 + we * C::WE + 16 * fe + l16;
      if (g == 0 && e < p.E) P[(size_t)h * p.E + e] = v;
    }
  }
#pragma unroll
  for (int fe = 0; fe < FE; ++fe) {
    const int e = e0 + we * C::WE + 16 * fe + l16;
    if (e >= p.E) continue;
#pragma unroll
    for (int fj = 0; fj < 4; ++fj)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + wj * 64 + 16 * fj + 4 * g + i;
        if (j < h) P[(size_t)j * p.E + e] = acc[fj][fe][i];
      }
  }
}

// dW_r (and db_r, row h) = sum over splits of part[s], in split order:
// deterministic.  Eight partials are loaded at a time, then added in order.
__global__ __launch_bounds__(256) void dwr_reduce_kernel(const float* part, int nsplit, int h,
                                                         int E, float* dWr, float* db) {
  const size_t n = (size_t)h * E, pitch = n + E, tot = db ? pitch : n;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < tot;
       i += (size_t)gridDim.x * 256) {
    const float* src = part + i;
    float s = 0.f;
    int c = 0;
    for (; c + 8 <= nsplit; c += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(c + u) * pitch];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; c < nsplit; ++c) s += src[(size_t)c * pitch];
    if (i < n) dWr[i] = s;
    else db[i - n] = s;
  }
}

}  // namespace

hipError_t launch_combine_bwd(const void* dOut, const void* Y, const int32_t* slot,
                              const float* gate, void* dY, float* dgate, int T, int h, int k,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k < 1 || k > 8) return hipErrorInvalidValue;
  if (k <= 2)
    hipLaunchKernelGGL(combine_bwd_kernel<2>, dim3((T + 3) / 4), dim3(256), 0, s,
                       static_cast<const bf16*>(dOut), static_cast<const bf16*>(Y), slot, gate,
                       static_cast<bf16*>(dY), dgate, T, h, k);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<8>, dim3((T + 3) / 4), dim3(256), 0, s,
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
  if (h % 64 != 0 || k < 1 || k > 8) return hipErrorInvalidValue;
  const dim3 grid((T + kGiT - 1) / kGiT, (h + kGiJ - 1) / kGiJ);
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool vec = E % 8 == 0 && al16(dH) && al16(W_r) && (!dZ || (al16(dZ) && al16(W_noise)));
#define MOE_GI(V, KM, SH)                                                                     \
  hipLaunchKernelGGL((grad_input_kernel<V, KM, SH>), grid, dim3(256), 0, s,                   \
                     static_cast<const bf16*>(dOut), static_cast<const bf16*>(dX), slot, dH,  \
                     static_cast<const bf16*>(W_r), dZ, static_cast<const bf16*>(W_noise),    \
                     static_cast<const bf16*>(dXs), ns, static_cast<bf16*>(dU), T, h, E, k)
  const bool sh = ns > 0;
  if (vec) {
    if (k <= 2) {
      if (sh) MOE_GI(true, 2, true); else MOE_GI(true, 2, false);
    } else {
      if (sh) MOE_GI(true, 8, true); else MOE_GI(true, 8, false);
    }
  } else {
    if (k <= 2) {
      if (sh) MOE_GI(false, 2, true); else MOE_GI(false, 2, false);
    } else {
      if (sh) MOE_GI(false, 8, true); else MOE_GI(false, 8, false);
    }
  }
#undef MOE_GI
  return hipGetLastError();
}

hipError_t launch_noise_grad(const float* zpart, int KS, int EP, const float* dH, uint64_t seed,
                             uint64_t rng_offset, float* dZ, int T, int E, hipStream_t s) {
  const size_t n = (size_t)T * E;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(noise_grad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, zpart,
                     KS, EP, dH, seed, rng_offset, dZ, T, E);
  return hipGetLastError();
}

hipError_t launch_dwr(const void* U, const float* dH, float* dWr, float* db, void* ws, int T,
                      int h, int E, hipStream_t s) {
  const DwrPlan p = dwr_plan(T, h, E);
  char* w = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(w);
  bf16* HL = reinterpret_cast<bf16*>(w + p.hl_off);
  if (T > 0) {
    const size_t n = (size_t)T * (p.ep / 8);
    const bool vec = E % 8 == 0 && (reinterpret_cast<uintptr_t>(dH) & 15) == 0;
    hipLaunchKernelGGL(dwr_split_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dH,
                       T, E, p.te, p.ep, vec, HL);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  DwArgs a{static_cast<const bf16*>(U), HL, part, T, h, E, p.ep, p.tchunk, p.jt, p.et,
           db != nullptr};
  const dim3 grid((unsigned)(p.jt * p.et * p.nsplit));
  switch (p.te) {
    case 16: hipLaunchKernelGGL((dwr_mfma_kernel<256, 16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((dwr_mfma_kernel<256, 32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((dwr_mfma_kernel<256, 64>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((dwr_mfma_kernel<128, 128>), grid, dim3(256), 0, s, a); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t n = (size_t)h * E + (db ? E : 0);
  const unsigned nb = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(dwr_reduce_kernel, dim3(nb), dim3(256), 0, s, part, p.nsplit, h, E, dWr, db);
  return hipGetLastError();
}

}  // namespace moe
