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
// bf16 path, two kernels.  route_logits_kernel computes H = U W_r (and
// U W_noise) as a tiled GEMM on v_mfma_f32_16x16x32_bf16 with float32
// accumulation: a workgroup owns 64 or 128 tokens x BN <= 128 experts (of
// both matrices when noisy) over one of KS ranges of K.  64-wide K chunks of the U rows and of
// the weight rows, read in their own [h][E] layout, are copied straight into
// a ring of LDS stages; the weight fragments come out K-contiguous through
// the transposing LDS read.  Each range's float32 products go to a
// workspace.  route_select_kernel then gives each wave whole tokens: it adds
// a token's K ranges in range order (so the result does not depend on
// timing), and the epilogue spreads its E logits over the 64 lanes, with
// max / sum / argmax as butterfly reductions (DPP and lane swaps, no LDS).
#include <math.h>

#include "blocks.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}

// Shared epilogue over the workgroup's tokens t0 .. t0 + RB - 1.  src(tt, j,
// e, hv, hn) gives token t0 + tt's float32 product with W_r column
// e = lane + 64 j (hv) and, when noisy, with W_noise column e (hn).
template <int EP, bool NOISY, class Src>
__device__ void route_epilogue(const Src& src, double (*Ps)[EP + 1], const RouteParams& p, int t0,
                               int RB) {
  constexpr int J = (EP + 63) / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = p.E, k = p.k;
  double pacc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) pacc[j] = 0.0;
  double zacc = 0.0;  // sum over this wave's tokens of LSE(H_t)^2 (wave-uniform)
  // the biases of this lane's experts, loaded once for all tokens
  float br[J], bs[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    br[j] = (p.b_r && e < E) ? p.b_r[e] : 0.f;
    bs[j] = (p.b_sel && e < E) ? p.b_sel[e] : 0.f;
  }

  for (int tt = wave; tt < RB; tt += 4) {
    const int t = t0 + tt;
    if (t >= p.T) break;
    float v[J], zn[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      float x = -INFINITY;
      zn[j] = 0.f;
      if (e < E) {
        float hv, hn = 0.f;
        src(tt, j, e, hv, hn);
        x = hv;
        if (p.b_r) x += br[j];
        if (NOISY) {
          // the draw of pair (t, e): counter t * E + e + rng_offset (mod 2^64)
          zn[j] = (float)philox_normal(p.seed, (uint64_t)t * E + e + p.rng_offset);
          x += zn[j] * softplus_f(hn);
        }
      }
      v[j] = x;
    }
    // the optional outputs are stored together, after the last read
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      if (e < E && p.logits) p.logits[(size_t)t * E + e] = v[j];
      if (NOISY && e < E && p.noise_out) p.noise_out[(size_t)t * E + e] = zn[j];
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
      if (keyed) key[j] = e < E ? s[j] + bs[j] : -INFINITY;
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
      auto take = [&](float ov, int oe) {
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      };
      take(wave_partner<0>(bv), wave_partner<0>(be));
      take(wave_partner<1>(bv), wave_partner<1>(be));
      take(wave_partner<2>(bv), wave_partner<2>(be));
      take(wave_partner<3>(bv), wave_partner<3>(be));
      take(wave_partner<4>(bv), wave_partner<4>(be));
      take(wave_partner<5>(bv), wave_partner<5>(be));
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
      // be is the same in every lane: read the chosen lane's score directly
      const int src_lane = __builtin_amdgcn_readfirstlane(be) & 63;
      const float sv = keyed ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), src_lane))
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
      // the dispatch's per-(rank, 256-token chunk) expert histogram: integer
      // sums, the same whatever order the increments land in
      if (p.hist) {
        const int nchunk = (p.T + kChunk - 1) / kChunk;
        atomicAdd(p.hist + ((size_t)lane * nchunk + t / kChunk) * E + my_idx, 1);
      }
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
    p.prob_part[(size_t)e * gridDim.x + blockIdx.x] =
        ((Ps[0][e] + Ps[1][e]) + Ps[2][e]) + Ps[3][e];
}

// ------------------------------------------------------ bf16 logits GEMM
struct LogitsArgs {
  const bf16* U;        // [T][h]
  const bf16* W0;       // W_r [h][Ew]
  const bf16* W1;       // W_noise [h][Ew] (noisy)
  float* part;          // [NSRC][KS][T][EP]
  int T, h, Ew, EP, KS, KT, nblocks;  // KT: 64-wide K chunks (h / 64)
  int32_t* zero = nullptr;  // nzero ints this launch clears (the dispatch
  int nzero = 0;            // histograms the selection kernel then fills)
};

// Stage geometry: one stage holds a 64-wide K chunk of BM U rows (128 bytes
// a row) and of BN columns of each weight matrix (64 k-rows of 2 BN bytes).
// Every wave issues the same copies per stage (a 1 KB region each), so a
// stage smaller than 4 KB is padded.
template <int BM_, int BN, int NSRC>
struct LogitsCfg {
  static constexpr int BM = BM_;
  static constexpr int ABYTES = BM * 128;
  static constexpr int BBYTES = BN * 128 >= 4096 ? BN * 128 : 4096;
  static constexpr int SBYTES = ABYTES + NSRC * BBYTES;
  static constexpr int NS = 163840 / SBYTES < 8 ? 163840 / SBYTES : 8;  // stages in the ring
  static constexpr int NAI = ABYTES / 4096, NBI = BBYTES / 4096;     // copies per wave
  static constexpr int NCOPY = NAI + NSRC * NBI;
  static_assert(NS >= 3 && (NS - 2) * NCOPY < 64, "ring");
};

template <int BM_, int BN, int NSRC, int WM>
__global__ __launch_bounds__(256) void route_logits_kernel(LogitsArgs p) {
  using C = LogitsCfg<BM_, BN, NSRC>;
  constexpr int BM = C::BM, NS = C::NS, NCH = BN / 8;
  constexpr int WN = 4 / WM, TM = BM / WM, TN = NSRC * BN / WN;
  constexpr int MB = TM / 16, NB = TN / 16;
  static_assert(TM % 16 == 0 && TN % 16 == 0 && BN % TN == 0, "wave tile");
  __shared__ __attribute__((aligned(16))) char lds[NS * C::SBYTES];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, g = lane >> 4, q = l16 >> 2, j = l16 & 3;
  // workgroup -> (token block, K range, expert block), consecutive ids on one XCD
  const int G = gridDim.x;
  const int L = (G & 7) == 0 ? xcd_remap(blockIdx.x, G) : blockIdx.x;
  const int nbk = L % p.nblocks, rest = L / p.nblocks;
  const int ks = rest % p.KS, mbk = rest / p.KS;
  const int m0 = mbk * BM, n0 = nbk * BN;
  const int kc0 = ks * p.KT / p.KS, KTl = (ks + 1) * p.KT / p.KS - kc0;
  const int rows = min(BM, p.T - m0);
  const int h = p.h, Ew = p.Ew;
  for (int i = blockIdx.x * 256 + tid; i < p.nzero; i += G * 256) p.zero[i] = 0;

  // loop-invariant parts of this lane's copy offsets
  int offA[C::NAI], offB[C::NBI];
#pragma unroll
  for (int i = 0; i < C::NAI; ++i) {
    const int byte = (wave * C::NAI + i) * 1024 + lane * 16;
    const int r = byte >> 7, c = ((byte >> 4) & 7) ^ ((r >> 1) & 7);
    offA[i] = r * h * 2 + c * 16;  // rows past `rows` fall outside the resource
  }
#pragma unroll
  for (int i = 0; i < C::NBI; ++i) {
    const int byte = (wave * C::NBI + i) * 1024 + lane * 16;
    const int r = byte / (BN * 2), c = ((byte % (BN * 2)) >> 4) ^ wsw<NCH>(r);
    offB[i] = (r < 64 && n0 + 8 * c < Ew) ? (r * Ew + 8 * c) * 2 : kPastEnd;
  }
  const size_t bbytes = ((size_t)(h - kc0 * 64) * Ew - n0) * 2;
  const size_t abytes = (size_t)rows * h * 2 - (size_t)kc0 * 128;

  // loop-invariant parts of this lane's fragment reads: U rows (16-byte
  // chunk 4 s + g of row r at chunk ^ ((r >> 1) & 7)) and transposing reads
  // of weight k-rows 32 s + 8 g + q (+ 4)
  int fa[2][MB], fb[2][NB];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wm * TM + 16 * mb + l16, c = 4 * s + g;
      fa[s][mb] = r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wn * TN + 16 * nb, src = col / BN, cs = col % BN;
      const int r = 32 * s + 8 * g + q, c = (cs >> 3) + (j >> 1);
      fb[s][nb] = C::ABYTES + src * C::BBYTES + r * (BN * 2) + ((c ^ wsw<NCH>(r)) << 4) + 8 * (j & 1);
    }
  }

  floatx4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // The ring's slots are passed as restrict parameters (and the copies'
  // sources built from restrict pointers), so the compiler can tell the
  // copies into one slot from the reads of another and adds no waits of its
  // own beyond the one at each step.
  auto run = [&](char* __restrict__ s0, char* __restrict__ s1, char* __restrict__ s2,
                 char* __restrict__ s3, char* __restrict__ s4, char* __restrict__ s5,
                 char* __restrict__ s6, char* __restrict__ s7, const char* __restrict__ gU,
                 const char* __restrict__ gW0, const char* __restrict__ gW1)
                 __attribute__((always_inline)) {
    char* const S[8] = {s0, s1, s2, s3, s4, s5, s6, s7};
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(gU, abytes);
    const __amdgpu_buffer_rsrc_t rB0 = make_rsrc(gW0, bbytes);
    const __amdgpu_buffer_rsrc_t rB1 = make_rsrc(NSRC == 2 ? gW1 : gW0, bbytes);
    // copies of local chunk cc into slot sl (past the range: no memory
    // traffic, the slot is never read again)
    auto issue = [&](int cc, char* sl) __attribute__((always_inline)) {
      const bool live = cc < KTl;
#pragma unroll
      for (int i = 0; i < C::NAI; ++i)
        dma16(rA, sl + (wave * C::NAI + i) * 1024, live ? offA[i] + cc * 128 : kPastEnd, 0);
#pragma unroll
      for (int i = 0; i < C::NBI; ++i)
        dma16(rB0, sl + C::ABYTES + (wave * C::NBI + i) * 1024,
              live ? (int)((unsigned)offB[i] + (unsigned)(cc * 128 * Ew)) : kPastEnd, 0);
      if constexpr (NSRC == 2) {
#pragma unroll
        for (int i = 0; i < C::NBI; ++i)
          dma16(rB1, sl + C::ABYTES + C::BBYTES + (wave * C::NBI + i) * 1024,
                live ? (int)((unsigned)offB[i] + (unsigned)(cc * 128 * Ew)) : kPastEnd, 0);
      }
    };
    auto compute = [&](const char* sl) __attribute__((always_inline)) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s lds_v4s;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 a[MB], b[NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) a[mb] = *reinterpret_cast<const bf16x8*>(sl + fa[s][mb]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const char* bp = sl + fb[s][nb];
          const v4s v[2] = {__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(bp)),
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(bp + 4 * BN * 2))};
          __builtin_memcpy(&b[nb], v, 16);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
      }
    };
    // chunk c sits in slot c % NS; step c waits for it, then refills the slot
    // of chunk c - 1 (every wave is past it) with chunk c + NS - 1
    auto step = [&](int c, int u) __attribute__((always_inline)) {
      wait_vm_seen<(NS - 2) * C::NCOPY>();
      wait_lgkm0_seen();
      barrier_only();
      issue(c + NS - 1, S[(u + NS - 1) % NS]);
      compute(S[u]);
    };
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) issue(u, S[u]);
    int c = 0;
    for (; c + NS <= KTl; c += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) step(c + u, u);
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (c + u < KTl) step(c + u, u);
    wait_vm_seen<0>();  // the last copies (past the range) land before the slots go away
  };
  char* const b0 = lds;
  run(b0, b0 + C::SBYTES * (1 % NS), b0 + C::SBYTES * (2 % NS), b0 + C::SBYTES * (3 % NS),
      b0 + C::SBYTES * (4 % NS), b0 + C::SBYTES * (5 % NS), b0 + C::SBYTES * (6 % NS),
      b0 + C::SBYTES * (7 % NS), reinterpret_cast<const char*>(p.U + (size_t)m0 * h + kc0 * 64),
      reinterpret_cast<const char*>(p.W0 + (size_t)kc0 * 64 * Ew + n0),
      reinterpret_cast<const char*>((NSRC == 2 ? p.W1 : p.W0) + (size_t)kc0 * 64 * Ew + n0));

  // D layout: lane holds column l16, rows 4 g + i
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = wn * TN + 16 * nb, src = col / BN;
    float* out = p.part + ((size_t)(src * p.KS + ks) * p.T) * p.EP + n0 + col % BN + l16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * TM + 16 * mb + 4 * g + i;
        if (r < rows) out[(size_t)(m0 + r) * p.EP] = acc[mb][nb][i];
      }
  }
}

// One wave per token (4 tokens a workgroup): all of the token's K-range
// products are loaded first (columns up to EP exist, so no lane branches),
// then added in range order, then the epilogue.
constexpr int kMaxKRanges = 8;
template <int NB, bool NOISY>
__global__ __launch_bounds__(256) void route_select_kernel(RouteParams p, int KS) {
  constexpr int EP = 16 * NB, J = (EP + 63) / 64, NM = NOISY ? 2 : 1;
  __shared__ double Ps[4][EP + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 4, t = t0 + wave;
  const size_t split = (size_t)p.T * EP;
  float hv[NM][J];
  if (t < p.T) {
    const float* base = p.lpart + (size_t)t * EP + lane;
    float x[NM][kMaxKRanges][J];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < kMaxKRanges; ++r)
#pragma unroll
        for (int j = 0; j < J; ++j)
          if (r < KS && lane + 64 * j < EP) x[m][r][j] = base[(m * KS + r) * split + 64 * j];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float v = lane + 64 * j < EP ? x[m][0][j] : 0.f;
#pragma unroll
        for (int r = 1; r < kMaxKRanges; ++r)
          if (r < KS && lane + 64 * j < EP) v += x[m][r][j];
        hv[m][j] = v;
      }
  }
  auto src = [&](int, int j, int, float& a, float& b) {
    a = hv[0][j];
    if (NOISY) b = hv[NM - 1][j];
  };
  route_epilogue<EP, NOISY>(src, Ps, p, t0, 4);
}

template <int NB, bool NOISY>
__global__ __launch_bounds__(256) void route_f32_kernel(RouteParams p) {
  constexpr int EP = 16 * NB, RB = 16;
  __shared__ float L[RB * EP];
  __shared__ float Ln[NOISY ? RB * EP : 1];
  __shared__ double Ps[4][EP + 1];
  const int t0 = blockIdx.x * RB;
  const float* U = static_cast<const float*>(p.U);
  const float* W = static_cast<const float*>(p.W);
  const float* Wn = static_cast<const float*>(p.Wn);
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
  auto src = [&](int tt, int, int e, float& hv, float& hn) {
    hv = L[tt * EP + e];
    if (NOISY) hn = Ln[tt * EP + e];
  };
  route_epilogue<EP, NOISY>(src, Ps, p, t0, RB);
}

__global__ void pad_rows_kernel(const bf16* W, bf16* Wp, int h, int E, int Ew) {
  const size_t n = (size_t)h * Ew;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t k = i / Ew;
    const int e = (int)(i - k * Ew);
    Wp[i] = e < E ? W[k * E + e] : bf16(0);
  }
}

__global__ __launch_bounds__(256) void prob_reduce_kernel(const double* part, int nblk, int EP,
                                                          int E, double* total, float* out) {
  prob_reduce_block(part, nblk, EP, E, total, out, blockIdx.x);
}

}  // namespace

RouteShape route_shape(int T, int E, int h, int bf16, int noisy) {
  RouteShape rs{};
  int NB = 1;
  while (16 * NB < E) NB *= 2;
  rs.NB = NB;
  rs.EP = 16 * NB;
  if (bf16) {
    rs.Ew = (E + 7) & ~7;
    rs.BN = rs.EP < 128 ? rs.EP : 128;
    rs.nblocks = rs.EP / rs.BN;
    const int KT = h / 64;
    // 128-token tiles halve the weight bytes read per U byte on wide routers
    // when they still give the chip 256 workgroups
    const int ks_max = std::min(8, std::max(1, KT / 8));
    rs.BM = (rs.BN >= 64 && (T + 127) / 128 * rs.nblocks * ks_max >= 256) ? 128 : 64;
    // waves along tokens: a wave's columns stay inside one weight matrix
    if (rs.BM == 128) rs.WM = 2;
    else rs.WM = rs.BN == 16 ? (noisy ? 2 : 4) : (rs.BN == 128 || noisy) ? 1 : 2;
    rs.mblocks = (T + rs.BM - 1) / rs.BM;
    // split K until the grid covers the chip, keeping at least 4 chunks a range
    rs.KS = 1;
    while (rs.mblocks * rs.nblocks * rs.KS < 256 && KT / (2 * rs.KS) >= 4 && rs.KS < 8) rs.KS *= 2;
    rs.RB = 4;  // one token per wave
  } else {
    rs.RB = 16;
  }
  rs.nblk = (T + rs.RB - 1) / rs.RB;
  return rs;
}

hipError_t launch_pad_router_w(const void* W, void* Wp, int h, int E, int Ew, hipStream_t s) {
  const size_t n = (size_t)h * Ew;
  const size_t nb = (n + 255) / 256;
  hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)(nb < 2048 ? nb : 2048)), dim3(256), 0, s,
                     static_cast<const bf16*>(W), static_cast<bf16*>(Wp), h, E, Ew);
  return hipGetLastError();
}

#define MOE_ROUTE_LOGITS(BM_, BN_, NS_, WM_)                                                    \
  if (rs.BM == BM_ && rs.BN == BN_ && nsrc == NS_ && rs.WM == WM_) {                              \
    hipLaunchKernelGGL((route_logits_kernel<BM_, BN_, NS_, WM_>), dim3(grid), dim3(256), 0, s, a); \
    launched = true;                                                                               \
  }
#define MOE_ROUTE_SELECT(NB_, NZ_)                                                               \
  if (rs.NB == NB_ && (noisy != 0) == NZ_) {                                                     \
    hipLaunchKernelGGL((route_select_kernel<NB_, NZ_>), dim3(rs.nblk), dim3(256), 0, s, p, rs.KS); \
    return hipGetLastError();                                                                    \
  }
#define MOE_ROUTE_F32(NB_, NZ_)                                                            \
  if (rs.NB == NB_ && (noisy != 0) == NZ_) {                                               \
    hipLaunchKernelGGL((route_f32_kernel<NB_, NZ_>), dim3(rs.nblk), dim3(256), 0, s, p);   \
    return hipGetLastError();                                                              \
  }

hipError_t launch_route(const RouteShape& rs, const RouteParams& p, int use_bf16, int noisy,
                        hipStream_t s) {
  if (rs.nblk == 0) return hipSuccess;
  if (use_bf16) {
    LogitsArgs a;
    a.U = static_cast<const bf16*>(p.U);
    a.W0 = static_cast<const bf16*>(p.W);
    a.W1 = static_cast<const bf16*>(noisy ? p.Wn : p.W);
    a.part = p.lpart;
    a.T = p.T;
    a.h = p.h;
    a.Ew = rs.Ew;
    a.EP = rs.EP;
    a.KS = rs.KS;
    a.KT = p.h / 64;
    a.nblocks = rs.nblocks;
    if (p.hist) {
      a.zero = p.hist;
      a.nzero = p.k * ((p.T + kChunk - 1) / kChunk) * p.E;
    }
    const int nsrc = noisy ? 2 : 1;
    const unsigned grid = (unsigned)(rs.mblocks * rs.nblocks * rs.KS);
    bool launched = false;
    MOE_ROUTE_LOGITS(64, 16, 1, 4) MOE_ROUTE_LOGITS(64, 16, 2, 2) MOE_ROUTE_LOGITS(64, 32, 1, 2)
    MOE_ROUTE_LOGITS(64, 32, 2, 1) MOE_ROUTE_LOGITS(64, 64, 1, 2) MOE_ROUTE_LOGITS(64, 64, 2, 1)
    MOE_ROUTE_LOGITS(64, 128, 1, 1) MOE_ROUTE_LOGITS(64, 128, 2, 1)
    MOE_ROUTE_LOGITS(128, 64, 1, 2) MOE_ROUTE_LOGITS(128, 64, 2, 2)
    MOE_ROUTE_LOGITS(128, 128, 1, 2) MOE_ROUTE_LOGITS(128, 128, 2, 2)
    if (!launched) return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    MOE_ROUTE_SELECT(1, false) MOE_ROUTE_SELECT(2, false) MOE_ROUTE_SELECT(4, false)
    MOE_ROUTE_SELECT(8, false) MOE_ROUTE_SELECT(16, false)
    MOE_ROUTE_SELECT(1, true) MOE_ROUTE_SELECT(2, true) MOE_ROUTE_SELECT(4, true)
    MOE_ROUTE_SELECT(8, true) MOE_ROUTE_SELECT(16, true)
  } else {
    MOE_ROUTE_F32(1, false) MOE_ROUTE_F32(2, false) MOE_ROUTE_F32(4, false)
    MOE_ROUTE_F32(8, false) MOE_ROUTE_F32(16, false)
    MOE_ROUTE_F32(1, true) MOE_ROUTE_F32(2, true) MOE_ROUTE_F32(4, true)
    MOE_ROUTE_F32(8, true) MOE_ROUTE_F32(16, true)
  }
  return hipErrorInvalidValue;
}

hipError_t launch_route_products(const RouteShape& rs, const void* U, const void* W, float* part,
                                 int T, int h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  LogitsArgs a;
  a.U = static_cast<const bf16*>(U);
  a.W0 = a.W1 = static_cast<const bf16*>(W);
  a.part = part;
  a.T = T;
  a.h = h;
  a.Ew = rs.Ew;
  a.EP = rs.EP;
  a.KS = rs.KS;
  a.KT = h / 64;
  a.nblocks = rs.nblocks;
  const int nsrc = 1;
  const unsigned grid = (unsigned)(rs.mblocks * rs.nblocks * rs.KS);
  bool launched = false;
  MOE_ROUTE_LOGITS(64, 16, 1, 4) MOE_ROUTE_LOGITS(64, 32, 1, 2) MOE_ROUTE_LOGITS(64, 64, 1, 2)
  MOE_ROUTE_LOGITS(64, 128, 1, 1) MOE_ROUTE_LOGITS(128, 64, 1, 2) MOE_ROUTE_LOGITS(128, 128, 1, 2)
  if (!launched) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prob_reduce(const double* part, int nblk, int EP, int E, double* total,
                              float* prob_sum, hipStream_t s) {
  // the z-loss column only when its sum has somewhere to go
  hipLaunchKernelGGL(prob_reduce_kernel, dim3(total ? E + 1 : E), dim3(256), 0, s, part, nblk,
                     EP, E, total, prob_sum);
  return hipGetLastError();
}

}  // namespace moe
