// Grouped SwiGLU experts over the ragged per-expert row blocks of the
// permuted matrix X.
//
// Method: page "MoE 与专家并行", section "从稠密 FFN 到 MoE", eq.
// FFN(u) = W_down (SiLU(W_gate u) * W_up u) with W_gate, W_up in R^{f x h} and
// W_down in R^{h x f}; section "专家计算：padding、block-sparse 与 grouped GEMM":
// one launch runs every expert's GEMM, scheduled by tiles from the per-expert
// row counts and offsets, with gate and up merged into one GEMM, the SiLU
// product in its epilogue, and a second GEMM for down.
//
// bf16 kernels (gfx950): C[M, N] = A[M, K] W[N, K]^T with both operands
// K-contiguous, v_mfma_f32_32x32x16_bf16, float32 accumulation.  A workgroup
// of 4 waves (2 x 2) owns a BM x 256 output tile; each wave a (BM/2) x 128
// block, i.e. BM/64 x 4 MFMA tiles.  K advances 64 at a time through two LDS
// buffers (global loads for step k+1 are in flight while step k is
// multiplied; one barrier per step).  LDS rows are 128 bytes; the 16-byte
// chunk index is XOR-ed with (row & 7) so the 32 rows read by one MFMA
// fragment fall on different banks.
// Gate/up tile: LDS B rows 0..127 are W_gate rows n0..n0+127 and rows
// 128..255 the W_up rows with the same indices, so each lane holds the gate
// and the up value of one output element and the epilogue writes
// a = SiLU(g) * u (rounded to bf16) directly.
// Tile order: tiles are numbered in groups of 8 n-tiles, m-tile major inside a
// group, and the numbering is spread over the XCDs in contiguous ranges, so
// workgroups running together on one XCD share A rows and B tiles in its L2.
// Ragged rows: an m-tile never crosses an expert boundary; rows past the
// expert's end read a clamped (valid) row and are not stored.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int BN = 256, BK = 64, GN = 8;

struct GemmParams {
  const bf16* A;         // [rows][K]
  const int32_t* offset; // [E+1]
  const int32_t* tmap;   // [E+1] first m-tile of each expert
  const bf16* W0;        // gate/up: W_gate [E][N][K]; down: W_down [E][N][K]
  const bf16* W1;        // gate/up: W_up
  bf16* C;               // [rows][Nout]
  int E, K, N, Nout;     // N: rows of each weight matrix (f or h)
  int ntiles, mtmax;
};

template <int BM, bool GATEUP>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmParams p) {
  constexpr int RBLK = BM / 64;      // 32-row MFMA blocks per wave
  constexpr int ACH = BM * 8 / 256;  // 16-byte A chunks per thread per K step
  constexpr int BCH = BN * 8 / 256;  // 16-byte B chunks per thread per K step
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * BK];

  // ---- which tile
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int g = L / (p.mtmax * GN);
  const int rem = L - g * p.mtmax * GN;
  const int gw = min(GN, p.ntiles - g * GN);
  if (gw <= 0) return;
  const int mt = rem / gw;
  const int nt = g * GN + rem % gw;
  if (mt >= p.mtmax || mt >= p.tmap[p.E]) return;
  int lo = 0, hi = p.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tmap[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int row0 = p.offset[e] + (mt - p.tmap[e]) * BM;
  const int rend = p.offset[e + 1];
  const int nvalid = min(BM, rend - row0);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global -> LDS addressing
  const bf16* aptr[ACH];
  int alds[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int q = tid + 256 * i, r = q >> 3, c = q & 7;
    const int gr = min(row0 + r, rend - 1);
    aptr[i] = p.A + (size_t)gr * p.K + c * 8;
    alds[i] = r * BK + ((c ^ (r & 7)) * 8);
  }
  const bf16* bptr[BCH];
  int blds[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int q = tid + 256 * i, r = q >> 3, c = q & 7;
    const bf16* W;
    int wr;
    if (GATEUP) {
      W = (r < 128) ? p.W0 : p.W1;
      wr = nt * 128 + (r & 127);
    } else {
      W = p.W0;
      wr = nt * BN + r;
    }
    wr = min(wr, p.N - 1);
    bptr[i] = W + (size_t)e * p.N * p.K + (size_t)wr * p.K + c * 8;
    blds[i] = r * BK + ((c ^ (r & 7)) * 8);
  }

  floatx16 acc[RBLK][4];
#pragma unroll
  for (int i = 0; i < RBLK; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  u32x4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[i] = ld16(aptr[i] + k0);
#pragma unroll
    for (int i = 0; i < BCH; ++i) rb[i] = ld16(bptr[i] + k0);
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) st16(&As[buf][alds[i]], ra[i]);
#pragma unroll
    for (int i = 0; i < BCH; ++i) st16(&Bs[buf][blds[i]], rb[i]);
  };

  // fragment rows in LDS: A rows of this wave, B rows of its 4 column blocks
  const int l32 = lane & 31, khalf = lane >> 5;
  int arow[RBLK], brow[4];
#pragma unroll
  for (int i = 0; i < RBLK; ++i) arow[i] = wm * (BM / 2) + i * 32 + l32;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (GATEUP)
      brow[j] = (j < 2 ? 0 : 128) + wn * 64 + (j & 1) * 32 + l32;
    else
      brow[j] = wn * 128 + j * 32 + l32;
  }

  const int KT = p.K / BK;
  gload(0);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const bf16* as = As[cur];
    const bf16* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = 2 * kk + khalf;
      bf16x8 af[RBLK], bfr[4];
#pragma unroll
      for (int i = 0; i < RBLK; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(as + arow[i] * BK + ((c ^ (arow[i] & 7)) * 8));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(bs + brow[j] * BK + ((c ^ (brow[j] & 7)) * 8));
#pragma unroll
      for (int i = 0; i < RBLK; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) swrite(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  D layout: lane holds column (lane % 32) and rows
  // 8 * (v / 4) + 4 * (lane / 32) + (v % 4), v = 0..15.
#pragma unroll
  for (int i = 0; i < RBLK; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * (BM / 2) + i * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
      if (r >= nvalid) continue;
      bf16* crow = p.C + (size_t)(row0 + r) * p.Nout;
      if (GATEUP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = nt * 128 + wn * 64 + j * 32 + l32;
          const float gv = acc[i][j][v], uv = acc[i][j + 2][v];
          const float a = gv / (1.f + __expf(-gv)) * uv;
          if (col < p.Nout) crow[col] = f32_to_bf16(a);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nt * BN + wn * 128 + j * 32 + l32;
          if (col < p.Nout) crow[col] = f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  }
}

// float32 path: one thread per output, plain dot products (small workloads).
template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* A, const int32_t* offset,
                                                       const float* W0, const float* W1,
                                                       float* C, int E, int K, int N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int rows = offset[E];
  if (i >= (int64_t)rows * N) return;
  const int row = (int)(i / N), col = (int)(i % N);
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offset[mid] <= row) lo = mid; else hi = mid;
  }
  const float* a = A + (size_t)row * K;
  const float* w0 = W0 + ((size_t)lo * N + col) * K;
  float s0 = 0.f;
  if (GATEUP) {
    const float* w1 = W1 + ((size_t)lo * N + col) * K;
    float s1 = 0.f;
    for (int j = 0; j < K; ++j) {
      s0 = fmaf(a[j], w0[j], s0);
      s1 = fmaf(a[j], w1[j], s1);
    }
    C[i] = s0 / (1.f + expf(-s0)) * s1;
  } else {
    for (int j = 0; j < K; ++j) s0 = fmaf(a[j], w0[j], s0);
    C[i] = s0;
  }
}

__global__ void tile_map_kernel(const int32_t* offset, int E, int bm1, int bm2, int32_t* m1,
                                int32_t* m2) {
  if (threadIdx.x != 0) return;
  int a = 0, b = 0;
  for (int e = 0; e < E; ++e) {
    m1[e] = a;
    m2[e] = b;
    const int n = offset[e + 1] - offset[e];
    a += (n + bm1 - 1) / bm1;
    b += (n + bm2 - 1) / bm2;
  }
  m1[E] = a;
  m2[E] = b;
}

int round8(int x) { return (x + 7) & ~7; }

}  // namespace

FfnShape ffn_shape(int64_t rows_max, int E, int h, int f, int T, int k, int bf16_) {
  FfnShape fs{};
  if (!bf16_) {
    fs.bm1 = fs.bm2 = 1;
    return fs;
  }
  // Experts with few rows (many experts, small top-k) use 128-row tiles so
  // less of each tile is padding.
  const double avg = E > 0 ? (double)T * k / E : 0.0;
  fs.bm1 = avg <= 160.0 ? 128 : 256;
  fs.bm2 = fs.bm1;
  fs.mt1 = (int)((rows_max + (int64_t)E * (fs.bm1 - 1)) / fs.bm1);
  fs.mt2 = (int)((rows_max + (int64_t)E * (fs.bm2 - 1)) / fs.bm2);
  fs.nt1 = (f + 127) / 128;
  fs.nt2 = (h + BN - 1) / BN;
  fs.grid1 = round8(fs.mt1 * fs.nt1);
  fs.grid2 = round8(fs.mt2 * fs.nt2);
  return fs;
}

hipError_t launch_tile_map(const int32_t* offset, int E, int bm1, int bm2, int32_t* map1,
                           int32_t* map2, hipStream_t s) {
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(64), 0, s, offset, E, bm1, bm2, map1, map2);
  return hipGetLastError();
}

hipError_t launch_gate_up(const FfnShape& fs, const void* X, const int32_t* offset,
                          const int32_t* map1, const void* Wg, const void* Wu, void* A, int E,
                          int h, int f, int bf16_, hipStream_t s) {
  if (!bf16_) {
    // rows are bounded by the caller's rows_max; launch for the static bound
    return hipErrorNotSupported;
  }
  if (fs.grid1 == 0) return hipSuccess;
  GemmParams p{static_cast<const bf16*>(X), offset, map1, static_cast<const bf16*>(Wg),
               static_cast<const bf16*>(Wu), static_cast<bf16*>(A), E, h, f, f,
               fs.nt1, fs.mt1};
  if (fs.bm1 == 256)
    hipLaunchKernelGGL((gemm_bf16_kernel<256, true>), dim3(fs.grid1), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<128, true>), dim3(fs.grid1), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_down(const FfnShape& fs, const void* A, const int32_t* offset,
                       const int32_t* map2, const void* Wd, void* Y, int E, int h, int f,
                       int bf16_, hipStream_t s) {
  if (!bf16_) return hipErrorNotSupported;
  if (fs.grid2 == 0) return hipSuccess;
  GemmParams p{static_cast<const bf16*>(A), offset, map2, static_cast<const bf16*>(Wd), nullptr,
               static_cast<bf16*>(Y), E, f, h, h, fs.nt2, fs.mt2};
  if (fs.bm2 == 256)
    hipLaunchKernelGGL((gemm_bf16_kernel<256, false>), dim3(fs.grid2), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<128, false>), dim3(fs.grid2), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_ffn_f32(const void* X, const int32_t* offset, const void* Wg, const void* Wu,
                          const void* Wd, void* A, void* Y, int64_t rows_max, int E, int h,
                          int f, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  const int64_t n1 = rows_max * f, n2 = rows_max * h;
  hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float*>(X), offset, static_cast<const float*>(Wg),
                     static_cast<const float*>(Wu), static_cast<float*>(A), E, h, f);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float*>(A), offset, static_cast<const float*>(Wd),
                     nullptr, static_cast<float*>(Y), E, f, h);
  return hipGetLastError();
}

}  // namespace moe
