// Router: logits H = U W_r (+ b_r) (+ z * softplus(U W_noise), z the
// counter-based standard-normal draw of each token and expert), scores,
// top-k with the (-H, expert index) key, gates, and per-workgroup sums of the
// score that enters P and of the squared log-sum-exp of the logits (the
// router z-loss, section "各家的变体", subsection "Router z-loss 与数值稳定",
// equation L_z, of the same page).
//
// Method: page "MoE 与专家并行", section "路由器：打分、top-k、加权求和"
// (eq. H = U W_r and the noisy-top-k eq. G(x)), the scoring table of section
// "softmax 门控还是 sigmoid 门控", and P_i of section "负载均衡辅助损失：推导与梯度"
// (for sigmoid scores P averages s / sum_j s).
//
// bf16 path: the logits GEMM runs on v_mfma_f32_16x16x32_bf16 with float32
// accumulation.  The four waves of a workgroup split K round-robin in 32-wide
// steps (adjacent 64-byte pieces of each U row go to different waves, so a
// row is read as one contiguous 256-byte run) and each wave keeps every
// expert column of its 16*MW tokens in registers.  The four partial sums are
// added in wave order through LDS, so the result does not depend on timing.
// The epilogue then gives each wave whole tokens: one token's E logits are
// spread over the 64 lanes, max / sum / argmax are butterfly reductions.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}

// Shared epilogue.  L (and Ln) hold the [RB][EP] float32 products of this
// workgroup's tokens.
template <int EP, int RB, bool NOISY>
__device__ void route_epilogue(const float* L, const float* Ln, double (*Ps)[EP + 1],
                               const RouteParams& p, int t0) {
  constexpr int J = (EP + 63) / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = p.E, k = p.k;
  double pacc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) pacc[j] = 0.0;
  double zacc = 0.0;  // sum over this wave's tokens of LSE(H_t)^2 (wave-uniform)

  for (int tt = wave; tt < RB; tt += 4) {
    const int t = t0 + tt;
    if (t >= p.T) break;
    float v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      float x = -INFINITY;
      if (e < E) {
        x = L[tt * EP + e];
        if (p.b_r) x += p.b_r[e];
        if (NOISY) {
          // the draw of pair (t, e): counter t * E + e + rng_offset (mod 2^64)
          const float z = (float)philox_normal(p.seed, (uint64_t)t * E + e + p.rng_offset);
          if (p.noise_out) p.noise_out[(size_t)t * E + e] = z;
          x += z * softplus_f(Ln[tt * EP + e]);
        }
        if (p.logits) p.logits[(size_t)t * E + e] = x;
      }
      v[j] = x;
    }
    // scores
    float s[J];
    float m = -INFINITY, Z = 1.f, S = 1.f;
    if (p.score == 0) {
#pragma unroll
      for (int j = 0; j < J; ++j) m = fmaxf(m, v[j]);
      m = wave_max(m);
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        s[j] = (lane + 64 * j < E) ? expf(v[j] - m) : 0.f;
        z += s[j];
      }
      Z = wave_sum(z);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        s[j] = s[j] / Z;
        pacc[j] += (double)s[j];
      }
      const float lse = m + logf(Z);
      zacc += (double)lse * (double)lse;
    } else {
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        s[j] = (lane + 64 * j < E) ? 1.f / (1.f + expf(-v[j])) : 0.f;
        z += s[j];
      }
      S = wave_sum(z);
#pragma unroll
      for (int j = 0; j < J; ++j) pacc[j] += (double)(s[j] / S);
      // z-loss of the logits: log-sum-exp with the max taken out
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < J; ++j) mx = fmaxf(mx, v[j]);
      mx = wave_max(mx);
      float ze = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) ze += (lane + 64 * j < E) ? expf(v[j] - mx) : 0.f;
      const float lse = mx + logf(wave_sum(ze));
      zacc += (double)lse * (double)lse;
    }
    // Selection keys.  Plain routing takes the top-k on the logits (the same
    // order as the scores).  With a selection bias or groups the keys are the
    // scores plus the bias (the bias decides membership only), and with
    // groups only experts of the topk_groups best groups compete, a group
    // scoring the sum of its k / topk_groups best keys.
    const bool keyed = p.b_sel != nullptr || p.n_groups > 1;
    float key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      key[j] = v[j];
      if (keyed) key[j] = e < E ? s[j] + (p.b_sel ? p.b_sel[e] : 0.f) : -INFINITY;
    }
    // arg-max over the keys of the experts with allow[j] set: larger key
    // first, lower expert index on ties (wave-uniform result)
    auto wave_argmax = [&](const bool (&allow)[J], float& bv, int& be) {
      bv = -INFINITY;
      be = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        if (allow[j] && (key[j] > bv || (key[j] == bv && e < be))) {
          bv = key[j];
          be = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oe = __shfl_xor(be, o, 64);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
    };
    if (p.n_groups > 1) {
      const int gsize = E / p.n_groups, q = k / p.topk_groups;
      float topv[8];
      int topg[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        topv[i] = -INFINITY;
        topg[i] = 0x7fffffff;
      }
      for (int g = 0; g < p.n_groups; ++g) {
        bool allow[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int e = lane + 64 * j;
          allow[j] = e >= g * gsize && e < (g + 1) * gsize;
        }
        float gs = 0.f;
        for (int r = 0; r < q; ++r) {
          float bv;
          int be;
          wave_argmax(allow, bv, be);
          gs += bv;
#pragma unroll
          for (int j = 0; j < J; ++j)
            if (lane + 64 * j == be) allow[j] = false;
        }
        // keep the topk_groups best (sum, group) pairs; an equal sum ranks
        // after the earlier (lower) group
        float cv = gs;
        int cg = g;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i < p.topk_groups && cv > topv[i]) {
            const float tv = topv[i];
            const int tg = topg[i];
            topv[i] = cv;
            topg[i] = cg;
            cv = tv;
            cg = tg;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int g = (lane + 64 * j) / gsize;
        bool in = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) in |= (i < p.topk_groups && topg[i] == g);
        if (!in) key[j] = -INFINITY;
      }
    }
    // top-k on the keys
    bool avail[J];
#pragma unroll
    for (int j = 0; j < J; ++j) avail[j] = lane + 64 * j < E && (!keyed || key[j] > -INFINITY);
    int my_idx = 0;
    float my_s = 0.f, gsum = 0.f;
    for (int r = 0; r < k; ++r) {
      float bv;
      int be;
      wave_argmax(avail, bv, be);
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (lane + 64 * j == be) avail[j] = false;
      // the gate uses the score of the chosen expert, never its key
      float mine = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (j == (be >> 6)) mine = s[j];
      const float sv = keyed ? __shfl(mine, be & 63, 64)
                             : ((p.score == 0) ? expf(bv - m) / Z : 1.f / (1.f + expf(-bv)));
      gsum += sv;
      if (lane == r) {
        my_idx = be;
        my_s = sv;
      }
    }
    if (lane < k) {
      p.topk_idx[(size_t)t * k + lane] = my_idx;
      p.topk_gate[(size_t)t * k + lane] = (p.gate == 1) ? my_s / gsum : my_s;
    }
  }
  // per-workgroup sums of the P score and (column EP) of LSE^2, waves added
  // in a fixed order
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    if (e < EP) Ps[wave][e] = pacc[j];
  }
  if (lane == 0) Ps[wave][EP] = zacc;
  __syncthreads();
  for (int e = threadIdx.x; e <= EP; e += blockDim.x)
    p.prob_part[(size_t)blockIdx.x * (EP + 1) + e] =
        ((Ps[0][e] + Ps[1][e]) + Ps[2][e]) + Ps[3][e];
}

template <int NB, int MW, bool NOISY>
__global__ __launch_bounds__(256) void route_bf16_kernel(RouteParams p) {
  constexpr int EP = 16 * NB, RB = 16 * MW;
  __shared__ float L[RB * EP];
  __shared__ float Ln[NOISY ? RB * EP : 1];
  __shared__ double Ps[4][EP + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * RB;
  const int h = p.h;

  floatx4 acc[MW][NB];
  floatx4 accn[NOISY ? MW : 1][NOISY ? NB : 1];
#pragma unroll
  for (int mb = 0; mb < MW; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (NOISY) accn[NOISY ? mb : 0][NOISY ? nb : 0] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  // A fragment: lane holds row (lane % 16), k = (lane / 16) * 8 .. +8.
  // B fragment: lane holds column (lane % 16) with the same k.
  const int lrow = lane & 15, lk = (lane >> 4) * 8;
  const bf16* U = static_cast<const bf16*>(p.U);
  const bf16* Wt = static_cast<const bf16*>(p.Wt);
  const bf16* Wnt = static_cast<const bf16*>(p.Wnt);
  const bf16* arow[MW];
#pragma unroll
  for (int mb = 0; mb < MW; ++mb) {
    const int t = min(t0 + 16 * mb + lrow, p.T - 1);
    arow[mb] = U + (size_t)t * h + lk;
  }
  const int ksteps = h / 32;

  for (int ks = wave; ks < ksteps; ks += 4) {
    const int k0 = ks * 32;
    bf16x8 a[MW], b[NB];
#pragma unroll
    for (int mb = 0; mb < MW; ++mb) a[mb] = *reinterpret_cast<const bf16x8*>(arow[mb] + k0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      b[nb] = *reinterpret_cast<const bf16x8*>(Wt + (size_t)(16 * nb + lrow) * h + lk + k0);
#pragma unroll
    for (int mb = 0; mb < MW; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
    if (NOISY) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        b[nb] = *reinterpret_cast<const bf16x8*>(Wnt + (size_t)(16 * nb + lrow) * h + lk + k0);
#pragma unroll
      for (int mb = 0; mb < MW; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          accn[NOISY ? mb : 0][NOISY ? nb : 0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a[mb], b[nb], accn[NOISY ? mb : 0][NOISY ? nb : 0], 0, 0, 0);
    }
  }
  // D layout: lane holds column (lane % 16), rows 4 * (lane / 16) + i.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mb = 0; mb < MW; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int o = (16 * mb + 4 * (lane >> 4) + i) * EP + 16 * nb + (lane & 15);
            if (w == 0) {
              L[o] = acc[mb][nb][i];
              if (NOISY) Ln[o] = accn[NOISY ? mb : 0][NOISY ? nb : 0][i];
            } else {
              L[o] += acc[mb][nb][i];
              if (NOISY) Ln[o] += accn[NOISY ? mb : 0][NOISY ? nb : 0][i];
            }
          }
    }
    __syncthreads();
  }
  route_epilogue<EP, RB, NOISY>(L, Ln, Ps, p, t0);
}

// float32 path: plain sequential dot products (small workloads only).
template <int NB, bool NOISY>
__global__ __launch_bounds__(256) void route_f32_kernel(RouteParams p) {
  constexpr int EP = 16 * NB, RB = 16;
  __shared__ float L[RB * EP];
  __shared__ float Ln[NOISY ? RB * EP : 1];
  __shared__ double Ps[4][EP + 1];
  const int t0 = blockIdx.x * RB;
  const float* U = static_cast<const float*>(p.U);
  const float* W = static_cast<const float*>(p.Wt);
  const float* Wn = static_cast<const float*>(p.Wnt);
  for (int i = threadIdx.x; i < RB * EP; i += blockDim.x) {
    const int tt = i / EP, e = i % EP, t = t0 + tt;
    float acc = 0.f, accn = 0.f;
    if (t < p.T && e < p.E) {
      const float* u = U + (size_t)t * p.h;
      for (int j = 0; j < p.h; ++j) {
        acc = fmaf(u[j], W[(size_t)j * p.E + e], acc);
        if (NOISY) accn = fmaf(u[j], Wn[(size_t)j * p.E + e], accn);
      }
    }
    L[i] = acc;
    if (NOISY) Ln[i] = accn;
  }
  __syncthreads();
  route_epilogue<EP, RB, NOISY>(L, Ln, Ps, p, t0);
}

__global__ void transpose_kernel(const bf16* W, bf16* WT, int h, int E, int EP) {
  __shared__ bf16 tile[32][33];
  const int k0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int kk = k0 + i, n = n0 + tx;
    tile[i][tx] = (kk < h && n < E) ? W[(size_t)kk * E + n] : bf16(0);
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int n = n0 + i, kk = k0 + tx;
    if (n < EP && kk < h) WT[(size_t)n * h + kk] = tile[tx][i];
  }
}

// One workgroup per column (E experts, then the LSE^2 column): thread j adds
// partials j, j + 256, ... in order, then a fixed-shape tree adds the 256
// sums (deterministic).  Column E lands in total[E] (z-loss numerator); out
// gets the E expert sums only.
__global__ __launch_bounds__(256) void prob_reduce_kernel(const double* part, int nblk, int EP,
                                                          int E, double* total, float* out) {
  __shared__ double sh[256];
  const int e = blockIdx.x;
  const int col = e < E ? e : EP;
  double s = 0.0;
  for (int b = threadIdx.x; b < nblk; b += 256) s += part[(size_t)b * (EP + 1) + col];
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

}  // namespace

RouteShape route_shape(int T, int E, int bf16, int noisy) {
  RouteShape rs;
  int NB = 1;
  while (16 * NB < E) NB *= 2;
  rs.NB = NB;
  rs.EP = 16 * NB;
  if (bf16) {
    int MW = 32 / (NB * (noisy ? 2 : 1));
    MW = MW > 4 ? 4 : (MW < 1 ? 1 : MW);
    while (MW > 1 && (T + 16 * MW - 1) / (16 * MW) < 256) MW /= 2;
    rs.MW = MW;
  } else {
    rs.MW = 1;
  }
  rs.RB = 16 * rs.MW;
  rs.nblk = (T + rs.RB - 1) / rs.RB;
  return rs;
}

hipError_t launch_transpose_router_w(const void* W, void* WT, int h, int E, int EP,
                                     hipStream_t s) {
  dim3 grid((h + 31) / 32, (EP + 31) / 32);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, static_cast<const bf16*>(W),
                     static_cast<bf16*>(WT), h, E, EP);
  return hipGetLastError();
}

#define MOE_ROUTE_BF16(NB_, MW_, NZ_)                                                     \
  if (rs.NB == NB_ && rs.MW == MW_ && (noisy != 0) == NZ_) {                              \
    hipLaunchKernelGGL((route_bf16_kernel<NB_, MW_, NZ_>), dim3(rs.nblk), dim3(256), 0, s, \
                       p);                                                                \
    return hipGetLastError();                                                             \
  }
#define MOE_ROUTE_F32(NB_, NZ_)                                                            \
  if (rs.NB == NB_ && (noisy != 0) == NZ_) {                                               \
    hipLaunchKernelGGL((route_f32_kernel<NB_, NZ_>), dim3(rs.nblk), dim3(256), 0, s, p);   \
    return hipGetLastError();                                                              \
  }

hipError_t launch_route(const RouteShape& rs, const RouteParams& p, int bf16, int noisy,
                        hipStream_t s) {
  if (rs.nblk == 0) return hipSuccess;
  if (bf16) {
    MOE_ROUTE_BF16(1, 1, false) MOE_ROUTE_BF16(1, 2, false) MOE_ROUTE_BF16(1, 4, false)
    MOE_ROUTE_BF16(2, 1, false) MOE_ROUTE_BF16(2, 2, false) MOE_ROUTE_BF16(2, 4, false)
    MOE_ROUTE_BF16(4, 1, false) MOE_ROUTE_BF16(4, 2, false) MOE_ROUTE_BF16(4, 4, false)
    MOE_ROUTE_BF16(8, 1, false) MOE_ROUTE_BF16(8, 2, false) MOE_ROUTE_BF16(8, 4, false)
    MOE_ROUTE_BF16(16, 1, false) MOE_ROUTE_BF16(16, 2, false)
    MOE_ROUTE_BF16(1, 1, true) MOE_ROUTE_BF16(1, 2, true) MOE_ROUTE_BF16(1, 4, true)
    MOE_ROUTE_BF16(2, 1, true) MOE_ROUTE_BF16(2, 2, true) MOE_ROUTE_BF16(2, 4, true)
    MOE_ROUTE_BF16(4, 1, true) MOE_ROUTE_BF16(4, 2, true) MOE_ROUTE_BF16(4, 4, true)
    MOE_ROUTE_BF16(8, 1, true) MOE_ROUTE_BF16(8, 2, true)
    MOE_ROUTE_BF16(16, 1, true)
  } else {
    MOE_ROUTE_F32(1, false) MOE_ROUTE_F32(2, false) MOE_ROUTE_F32(4, false)
    MOE_ROUTE_F32(8, false) MOE_ROUTE_F32(16, false)
    MOE_ROUTE_F32(1, true) MOE_ROUTE_F32(2, true) MOE_ROUTE_F32(4, true)
    MOE_ROUTE_F32(8, true) MOE_ROUTE_F32(16, true)
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prob_reduce(const double* part, int nblk, int EP, int E, double* total,
                              float* prob_sum, hipStream_t s) {
  // the z-loss column only when its sum has somewhere to go
  hipLaunchKernelGGL(prob_reduce_kernel, dim3(total ? E + 1 : E), dim3(256), 0, s, part, nblk,
                     EP, E, total, prob_sum);
  return hipGetLastError();
}

}  // namespace moe
