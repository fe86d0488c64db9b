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

// Round to nearest even (NaN stays NaN), with gfx950's v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t b = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &b, 4);
  return u;
}
__device__ __forceinline__ bf16 f32_to_bf16(float x) { return bf16(pack_bf16x2(x, 0.f)); }

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

// Standard-normal draw of the noisy router (page "MoE 与专家并行", section
// "路由器：打分、top-k、加权求和", eq. G(x): an N(0, 1) factor per token and
// expert) from a counter-based generator, so each (token, expert) pair has
// its own draw whatever the launch shape: Philox-4x64 with 10 rounds (Salmon,
// Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11), key (seed, 0) and counter (n, 0, 0, 0).  A round takes the two
// 128-bit products M0 x0 and M1 x2 and maps (x0, x1, x2, x3) to
// (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)); the key
// then grows by the two Weyl increments.  The draw is the Box-Muller
// transform of u1 = (w0 / 2^11 + 1) 2^-53 in (0, 1] and u2 = (w1 / 2^11)
// 2^-53 in [0, 1) from the block's first two words, in double precision.
__device__ __forceinline__ double philox_normal(uint64_t seed, uint64_t n) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = n, x1 = 0, x2 = 0, x3 = 0, k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
    const uint64_t hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  const double u1 = (double)((x0 >> 11) + 1) * 0x1p-53;
  const double u2 = (double)(x1 >> 11) * 0x1p-53;
  return sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
}

// Wave-wide butterflies without LDS traffic.  Step S pairs every lane with
// one lane of the other half of its group of 2^(S+1) lanes: quad
// permutations (S = 0, 1), mirrors within 8 and within 16 lanes (DPP,
// S = 2, 3), then the row swap and the half swap of gfx950 (S = 4, 5).  A
// commutative, associative combine applied after each of the six steps
// leaves the whole wave's result, bit-identical, in every lane.
template <int S>
__device__ __forceinline__ int wave_partner(int v) {
  if constexpr (S == 0) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  else if constexpr (S == 1) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  else if constexpr (S == 2) return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  else if constexpr (S == 3) return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  else if constexpr (S == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 32) ? r[0] : r[1]);
  }
}
template <int S>
__device__ __forceinline__ float wave_partner(float v) {
  return __int_as_float(wave_partner<S>(__float_as_int(v)));
}
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, wave_partner<0>(v));
  v = op(v, wave_partner<1>(v));
  v = op(v, wave_partner<2>(v));
  v = op(v, wave_partner<3>(v));
  v = op(v, wave_partner<4>(v));
  return op(v, wave_partner<5>(v));
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
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

// ------------------------------------------------ LDS-direct copies, waits
// Third dword of a raw buffer resource on gfx9-family parts (32-bit data
// format, no swizzle); loads outside num_records bytes return zero without
// touching memory.
constexpr int kBufFlags = 0x00020000;
constexpr int kPastEnd = 0x7ffffff0;  // a byte offset past every resource

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0x7fffffffull ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kBufFlags);
}

// One wave-wide 16-byte-per-lane load straight into LDS: lane i's 16 bytes
// land at lds + 16 * i.  voff: per-lane byte offset, soff: uniform byte offset.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
}

// Workgroup barrier without the release fence of __syncthreads(): that fence
// would wait for every load in flight, including the LDS copies of the next
// stages.  Callers make their own data visible first (wait_vm_seen); the
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt through the builtin rather than inline asm, so that the
// compiler's own wait insertion sees it and knows which copies have landed
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8;
// the counters not waited on are left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm_seen() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0_seen() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup i -> XCD i % 8).
// Remap so each XCD walks one contiguous range of logical tiles: tiles that
// share operands then run together and hit the same L2.  nblk % 8 == 0.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  return (bid & 7) * (nblk >> 3) + (bid >> 3);
}

// Rows of a [K][N] bf16 tile in LDS that transposing fragment reads take:
// k-row r (NCH chunks of 16 bytes) keeps logical chunk c at chunk c ^ wsw(r).
// A transposing read of one fragment touches, per half-wave, 8 k-rows (rows
// 8 g + q, g = 0/1, q = 0..3) x 2 adjacent chunks; wsw spreads those 16
// pieces over distinct 16-byte bank groups (for NCH >= 4; two-chunk rows keep
// a two-way conflict).
template <int NCH>
__device__ __forceinline__ int wsw(int r) {
  const int g1 = (r >> 3) & 1, q = r & 3;
  if constexpr (NCH >= 16) return 2 * (4 * g1 + q);
  else if constexpr (NCH == 8) return 4 * g1 + 2 * (q >> 1);
  else if constexpr (NCH == 4) return 2 * g1;
  else return 0;
}

}  // namespace moe
