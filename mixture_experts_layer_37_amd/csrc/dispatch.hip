// Dispatch: capacity cut, fill order and the permutation of token rows into
// per-expert contiguous blocks.
//
// Method: page "MoE 与专家并行", section "专家容量与丢 token": capacity C, slots
// filled in token order with later tokens dropped (they pass only the
// residual), and the GShard order that places every token's first choice
// before any second choice; the rows of one expert are contiguous as in the
// sort-and-group dataflow of section "路由器：打分、top-k、加权求和".
//
// The sequential definition "visit assignments in fill order, each takes the
// next free position of its expert" is computed in three data-parallel passes
// with integer arithmetic only, so positions are exact and deterministic:
//  1. per 256-token chunk and rank, a histogram of experts (LDS integer
//     counters; counts do not depend on the order of the increments);
//  2. one workgroup scans the histograms in fill order, giving each
//     (rank, chunk, expert) the number of earlier assignments to that expert,
//     plus count, kept = min(count, C) and the exclusive offsets of kept;
//  3. per chunk, each assignment adds the number of earlier assignments in its
//     own chunk (wave ballots for lanes below it, LDS counts for waves before
//     it); position < C keeps it at row offset[e] + position.
#include <mutex>

#include "blocks.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// Scratch of moe_dispatch_noalloc: the per-chunk histograms and bases of
// hist_kernel / scan_kernel, in a fixed device array instead of a caller
// workspace.  Every entry they read is written by the same call first, so
// nothing needs clearing between calls.
__device__ __align__(256) int32_t scratch[kDispatchScratchBytes / sizeof(int32_t)];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
int32_t* scratch_ptr[kMaxDevices] = {};

__device__ __forceinline__ int load_expert(const int32_t* idx, int t, int r, int T, int k, int E) {
  if (t >= T) return -1;
  const int e = idx[(size_t)t * k + r];
  return (e >= 0 && e < E) ? e : -1;  // ids outside [0, E) are ignored
}

__global__ __launch_bounds__(256) void hist_kernel(DispatchParams p) {
  __shared__ int cnt[8 * 256];
  const int nchunk = gridDim.x, c = blockIdx.x;
  for (int i = threadIdx.x; i < p.k * p.E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int t = c * kChunk + threadIdx.x;
  for (int r = 0; r < p.k; ++r) {
    const int e = load_expert(p.topk_idx, t, r, p.T, p.k, p.E);
    if (e >= 0) atomicAdd(&cnt[r * p.E + e], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < p.k * p.E; i += blockDim.x) {
    const int r = i / p.E, e = i % p.E;
    p.hist[((size_t)r * nchunk + c) * p.E + e] = cnt[i];
  }
}

__global__ __launch_bounds__(256) void scan_kernel(DispatchParams p, int nchunk) {
  if (blockIdx.x > 0) {  // the router's P sums (layer forward)
    prob_reduce_block(p.prob_part, p.prob_nblk, p.prob_EP, p.E, p.prob_total, p.prob_out,
                      blockIdx.x - 1);
    return;
  }
  __shared__ int tmp[4];
  const int e = threadIdx.x;
  int run = 0;
  if (e < p.E) {
    // Expert e's (rank, chunk) counts in fill order, 8 independent loads at a
    // time.  rank-major: (rank 0, chunk 0), (rank 0, chunk 1), ..., (rank 1,
    // chunk 0), ...; token-major: chunk by chunk, a token holding an expert at
    // most once, so the base of chunk c is the total of the chunks before it.
    const int n = p.token_major ? nchunk : p.k * nchunk;
    for (int j0 = 0; j0 < n; j0 += 8) {
      int v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q;
        v[q] = 0;
        if (j < n) {
          if (!p.token_major) {
            v[q] = p.hist[(size_t)j * p.E + e];  // j = r * nchunk + c
          } else {
            for (int r = 0; r < p.k; ++r) v[q] += p.hist[((size_t)r * nchunk + j) * p.E + e];
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q;
        if (j < n) p.base[(size_t)j * p.E + e] = run;
        run += v[q];
      }
    }
  }
  const int kp = run < p.C ? run : p.C;
  int total;
  const int off = block_excl_scan256(e < p.E ? kp : 0, tmp, &total);
  if (e < p.E) {
    p.count[e] = run;
    p.kept[e] = kp;
    p.offset[e] = off;
  }
  if (e == 0) p.offset[p.E] = total;
  // the layer forward's follow-up steps, on the values in hand
  if (p.map1) {
    __shared__ int tmp2[8];
    tile_maps_block(e, p.E, e < p.E ? kp : 0, off, p.bm1, p.bm2, p.map1, p.map2, tmp2);
  }
  if (p.stats_on && !p.prob_part) stats_block(p.stats, e, run, kp);
}

__global__ __launch_bounds__(256) void assign_kernel(DispatchParams p, int nchunk) {
  if (blockIdx.x >= nchunk) {  // the load statistics, once the scan launch's P sums are in
    const int e = threadIdx.x;
    stats_block(p.stats, e, e < p.E ? p.count[e] : 0, e < p.E ? p.kept[e] : 0);
    return;
  }
  __shared__ int wc[4][256];
  const int c = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = c * kChunk + threadIdx.x;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // k <= 8; loops over ranks are unrolled to 8 so ex[] stays in registers
  int ex[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) ex[r] = r < p.k ? load_expert(p.topk_idx, t, r, p.T, p.k, p.E) : -1;

  if (!p.token_major) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r >= p.k) break;
      for (int i = threadIdx.x; i < 4 * 256; i += blockDim.x) (&wc[0][0])[i] = 0;
      __syncthreads();
      const int e = ex[r];
      const uint64_t same = match_lanes(e, e, e >= 0);
      if (e >= 0) atomicAdd(&wc[wave][e], 1);
      __syncthreads();
      if (e >= 0) {
        int pos = p.base[((size_t)r * nchunk + c) * p.E + e] + __popcll(same & below);
        for (int w = 0; w < wave; ++w) pos += wc[w][e];
        const int row = pos < p.C ? p.offset[e] + pos : -1;
        p.slot[(size_t)t * p.k + r] = row;
        if (row >= 0) p.row_token[row] = t;
      } else if (t < p.T) {
        p.slot[(size_t)t * p.k + r] = -1;
      }
      __syncthreads();
    }
  } else {
    for (int i = threadIdx.x; i < 4 * 256; i += blockDim.x) (&wc[0][0])[i] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (ex[r] >= 0) atomicAdd(&wc[wave][ex[r]], 1);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r >= p.k) break;
      const int e = ex[r];
      // earlier assignments to expert e in this wave: every rank of the lanes
      // below that holds e, then this token's own lower ranks that hold e (a
      // caller's topk_idx may name one expert twice for a token)
      int lower = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < p.k) lower += __popcll(match_lanes(e, ex[q], ex[q] >= 0) & below);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < r && ex[q] == e) ++lower;
      if (e >= 0) {
        int pos = p.base[(size_t)c * p.E + e] + lower;
        for (int w = 0; w < wave; ++w) pos += wc[w][e];
        const int row = pos < p.C ? p.offset[e] + pos : -1;
        p.slot[(size_t)t * p.k + r] = row;
        if (row >= 0) p.row_token[row] = t;
      } else if (t < p.T) {
        p.slot[(size_t)t * p.k + r] = -1;
      }
    }
  }
}

// One wave per token: read the row once, write it to each kept slot.
template <typename TE>
__global__ __launch_bounds__(256) void permute_kernel(const TE* U, const int32_t* slot, TE* X,
                                                      int T, int h, int k) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int sl[8];
  bool any = false;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    sl[r] = r < k ? slot[(size_t)t * k + r] : -1;
    any |= sl[r] >= 0;
  }
  if (!any) return;
  constexpr int V = Elem<TE>::kPer16B;
  const int nvec = h / V;
  const TE* src = U + (size_t)t * h;
  // four vectors per lane and pass, loaded before any of their stores (a load
  // issued after stores would wait for them: memory operations retire in
  // order)
  for (int i0 = lane; i0 < nvec; i0 += 256) {
    u32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + 64 * q;
      v[q] = ld16(src + (size_t)(i < nvec ? i : i0) * V);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + 64 * q;
      if (i >= nvec) break;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (sl[r] >= 0) st16(X + (size_t)sl[r] * h + (size_t)i * V, v[q]);
    }
  }
}

// FP8 dispatch: one wave per token reads its row, takes the largest magnitude,
// and writes the row's E4M3 codes and power-of-two scale to each kept slot.
__global__ __launch_bounds__(256) void permute_fp8_kernel(const bf16* U, const int32_t* slot,
                                                          uint8_t* X8, float* xs, int T, int h,
                                                          int k) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int sl[8];
  bool any = false;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    sl[r] = r < k ? slot[(size_t)t * k + r] : -1;
    any |= sl[r] >= 0;
  }
  if (!any) return;
  const int nvec = h / 8;
  const bf16* src = U + (size_t)t * h;
  float amax = 0.f;
  for (int i = lane; i < nvec; i += 64) {
    float v[8];
    Elem<bf16>::unpack(ld16(src + (size_t)i * 8), v);
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
  }
  const int j = fp8_scale_exp(wave_max(amax));
  for (int i = lane; i < nvec; i += 64) {
    float v[8];
    Elem<bf16>::unpack(ld16(src + (size_t)i * 8), v);
    const uint2 q = to_fp8x8(v, j);
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (sl[r] >= 0) *reinterpret_cast<uint2*>(X8 + (size_t)sl[r] * h + (size_t)i * 8) = q;
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (sl[r] >= 0) xs[sl[r]] = ldexpf(1.f, j);
  }
}

// Row-wise FP8 quantisation of a bf16 matrix (weights): one wave per row.
__global__ __launch_bounds__(256) void quantize_rows_fp8_kernel(const bf16* src, int64_t rows,
                                                                int cols, uint8_t* dst,
                                                                float* scale) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;
  const bf16* row = src + (size_t)r * cols;
  const int nvec = cols / 8;
  float amax = 0.f;
  for (int i = lane; i < nvec; i += 64) {
    float v[8];
    Elem<bf16>::unpack(ld16(row + (size_t)i * 8), v);
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
  }
  const int j = fp8_scale_exp(wave_max(amax));
  for (int i = lane; i < nvec; i += 64) {
    float v[8];
    Elem<bf16>::unpack(ld16(row + (size_t)i * 8), v);
    *reinterpret_cast<uint2*>(dst + (size_t)r * cols + (size_t)i * 8) = to_fp8x8(v, j);
  }
  if (lane == 0) scale[r] = ldexpf(1.f, j);
}

// FP8 rows back to bf16: codes times the row's power-of-two scale.  Exact,
// since an E4M3 value has 4 significant bits and the scale only moves the
// exponent.  Eight elements per thread.
__global__ __launch_bounds__(256) void dequant_rows_fp8_kernel(const uint8_t* q,
                                                               const float* scale, int64_t rows,
                                                               int cols, bf16* out) {
  const int per = cols / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = i / per;
  if (r >= rows) return;
  const int c = (int)(i - r * per) * 8;
  const uint2 w = *reinterpret_cast<const uint2*>(q + (size_t)r * cols + c);
  const float sc = scale[r];
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
  const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  const f2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
  const f2 e = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  const float v[8] = {a.x * sc, a.y * sc, b.x * sc, b.y * sc, d.x * sc, d.y * sc, e.x * sc,
                      e.y * sc};
  st16(out + (size_t)r * cols + c, Elem<bf16>::pack(v));
}

}  // namespace

hipError_t launch_dequant_rows_fp8(const void* q, const float* scale, int64_t rows, int cols,
                                   void* out, hipStream_t s) {
  const int64_t n = rows * (cols / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_rows_fp8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(q), scale, rows, cols, static_cast<bf16*>(out));
  return hipGetLastError();
}

hipError_t launch_permute_fp8(const void* U, const int32_t* slot, void* X8, float* xs, int T,
                              int h, int k, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_fp8_kernel, dim3((T + 3) / 4), dim3(256), 0, s,
                     static_cast<const bf16*>(U), slot, static_cast<uint8_t*>(X8), xs, T, h, k);
  return hipGetLastError();
}

hipError_t launch_quantize_rows_fp8(const void* src, int64_t rows, int cols, void* dst,
                                    float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_fp8_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                     static_cast<const bf16*>(src), rows, cols, static_cast<uint8_t*>(dst),
                     scale);
  return hipGetLastError();
}

// The device address of this device's copy of `scratch`, looked up once per
// device (with that device current) and kept: the array's name in host code
// is not a device address.
hipError_t dispatch_scratch(int32_t** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    scratch_ptr[dev] = static_cast<int32_t*>(ptr);
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_dispatch(const DispatchParams& p, hipStream_t s) {
  const int nchunk = (p.T + kChunk - 1) / kChunk;
  if (nchunk > 0 && !p.hist_ready) {
    hipLaunchKernelGGL(hist_kernel, dim3(nchunk), dim3(256), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // with the P sums folded in, workgroups 1 .. E+1 sum them and the
  // statistics move to one more workgroup of the assignment launch
  const bool psum = p.prob_part != nullptr;
  hipLaunchKernelGGL(scan_kernel, dim3(psum ? p.E + 2 : 1), dim3(256), 0, s, p, nchunk);
  hipError_t err = hipGetLastError();
  const int ablocks = nchunk + ((psum && p.stats_on) ? 1 : 0);
  if (err != hipSuccess || ablocks == 0) return err;
  hipLaunchKernelGGL(assign_kernel, dim3(ablocks), dim3(256), 0, s, p, nchunk);
  return hipGetLastError();
}

hipError_t launch_permute(const void* U, const int32_t* slot, void* X, int T, int h, int k,
                          int bf16_, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4);
  if (bf16_)
    hipLaunchKernelGGL(permute_kernel<bf16>, grid, dim3(256), 0, s,
                       static_cast<const bf16*>(U), slot, static_cast<bf16*>(X), T, h, k);
  else
    hipLaunchKernelGGL(permute_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(U), slot, static_cast<float*>(X), T, h, k);
  return hipGetLastError();
}

}  // namespace moe
