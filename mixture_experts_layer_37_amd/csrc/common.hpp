// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16;  // storage type of bfloat16 values

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16 v) {
  return __uint_as_float(uint32_t(v) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16 f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// Element traits: how 16 bytes unpack into floats.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static void unpack(const u32x4& v, float* o) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
  __device__ static u32x4 pack(const float* o) {
    u32x4 v;
    v.x = __float_as_uint(o[0]);
    v.y = __float_as_uint(o[1]);
    v.z = __float_as_uint(o[2]);
    v.w = __float_as_uint(o[3]);
    return v;
  }
  __device__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ static void store(float* p, size_t i, float x) { p[i] = x; }
};
template <>
struct Elem<bf16> {
  static constexpr int kPer16B = 8;
  __device__ static void unpack(const u32x4& v, float* o) {
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
    o[4] = __uint_as_float(v.z << 16);
    o[5] = __uint_as_float(v.z & 0xffff0000u);
    o[6] = __uint_as_float(v.w << 16);
    o[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static u32x4 pack(const float* o) {
    u32x4 v;
    v.x = pack_bf16x2(o[0], o[1]);
    v.y = pack_bf16x2(o[2], o[3]);
    v.z = pack_bf16x2(o[4], o[5]);
    v.w = pack_bf16x2(o[6], o[7]);
    return v;
  }
  __device__ static float load(const bf16* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static void store(bf16* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// FP8 rows (page "MoE 与专家并行", section "低精度通信": activations quantised
// to FP8 with power-of-two scaling factors).  Format OCP E4M3, largest finite
// value 448 = 0.875 * 2^9.  A row with largest magnitude amax gets the scale
// 2^j with j the smallest integer such that amax / 2^j <= 448 (j = 0 for an
// all-zero row): with amax = m 2^p, 0.5 <= m < 1, that is p - 9 when
// m <= 0.875 and p - 8 otherwise.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int p;
  const float m = frexpf(amax, &p);
  return m > 0.875f ? p - 8 : p - 9;
}
// Eight values times 2^-j (exact), each rounded to the nearest E4M3 value with
// ties to even (the conversion instruction in the default rounding mode), as
// eight bytes in element order.
__device__ __forceinline__ uint2 to_fp8x8(const float* v, int j) {
  int lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -j), ldexpf(v[1], -j), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -j), ldexpf(v[3], -j), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -j), ldexpf(v[5], -j), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -j), ldexpf(v[7], -j), hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Lanes whose value `theirs` equals `mine`, among lanes with `valid` set.
// Values are in [0, 256).
// Exclusive prefix sum of v over the 256 threads of a block (blockDim.x must
// be 256; every thread calls it).  tmp: 4 ints of LDS.  *total receives the
// sum of all 256 values.
__device__ __forceinline__ int block_excl_scan256(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o, 64);
    if (lane >= o) inc += u;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < 3; ++w)
    if (w < wave) before += tmp[w];
  *total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  return before + inc - v;
}

__device__ __forceinline__ uint64_t match_lanes(int mine, int theirs, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    uint64_t bits = __ballot((theirs >> b) & 1);
    m &= ((mine >> b) & 1) ? bits : ~bits;
  }
  return m;
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup i -> XCD i % 8).
// Remap so each XCD walks one contiguous range of logical tiles: tiles that
// share operands then run together and hit the same L2.  nblk % 8 == 0.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  return (bid & 7) * (nblk >> 3) + (bid >> 3);
}

}  // namespace moe
