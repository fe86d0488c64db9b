// Host entry points of libmoe (the C ABI declared in include/moe.h).
//
// Validation happens before any launch.  Capacity is computed as an exact
// rational ceiling (page "MoE 与专家并行", section "专家容量与丢 token", eq. C;
// top-1 form on page "Ai大模型训练教程", capacity section).  The library never
// allocates or synchronises: every intermediate lives in the caller's
// workspace, whose layout is planned here identically for size queries and
// calls.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <string.h>

#include "kernels.hpp"
#include "moe.h"

namespace moe {
hipError_t launch_ffn_f32(const void* X, const int32_t* offset, const void* Wg, const void* Wu,
                          const void* Wd, void* A, void* Y, int64_t rows_max, int E, int h,
                          int f, hipStream_t s);
}

namespace {

using namespace moe;

constexpr int64_t kMaxE = 256, kMaxK = 8;

struct Dims {
  int64_t T, h, f, E, k, C, rows_max;
  int64_t n_groups, topk_groups, ns, fs;  // group-limited selection, shared experts
  bool bf16;
};

int32_t check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->h < 1 || c->f < 1 || c->E < 1 || c->k < 1 || c->k > c->E)
    return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->score != MOE_SCORE_SOFTMAX && c->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (c->gate != MOE_GATE_RAW && c->gate != MOE_GATE_RENORM) return MOE_ERR_INVALID_ARG;
  if (c->cap_mode != MOE_CAP_ASSIGNMENTS && c->cap_mode != MOE_CAP_TOKENS)
    return MOE_ERR_INVALID_ARG;
  if (c->fill != MOE_FILL_RANK_MAJOR && c->fill != MOE_FILL_TOKEN_MAJOR)
    return MOE_ERR_INVALID_ARG;
  if (c->noisy != 0 && c->noisy != 1) return MOE_ERR_INVALID_ARG;
  if (c->min_capacity < 0) return MOE_ERR_INVALID_ARG;
  const double cf = c->capacity_factor;
  if (isnan(cf) || isinf(cf)) return MOE_ERR_INVALID_ARG;
  if (cf > 0 && (cf < 1e-6 || cf > 1e6)) return MOE_ERR_INVALID_ARG;
  if (c->E > kMaxE || c->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (c->dtype == MOE_BF16 && (c->h % 64 != 0 || c->f % 64 != 0)) return MOE_ERR_UNSUPPORTED;
  if (c->dtype == MOE_F32 && (c->h % 4 != 0 || c->f % 4 != 0)) return MOE_ERR_UNSUPPORTED;
  // group-limited selection
  if (c->n_groups < 0) return MOE_ERR_INVALID_ARG;
  if (c->n_groups > 1) {
    if (c->n_groups > 64) return MOE_ERR_UNSUPPORTED;
    if (c->E % c->n_groups != 0) return MOE_ERR_INVALID_ARG;
    if (c->topk_groups < 1 || c->topk_groups > c->n_groups || c->topk_groups > c->k)
      return MOE_ERR_INVALID_ARG;
    if (c->topk_groups > 8) return MOE_ERR_UNSUPPORTED;
    if (c->k > c->topk_groups * (c->E / c->n_groups)) return MOE_ERR_INVALID_ARG;
  }
  // shared experts
  if (c->n_shared < 0) return MOE_ERR_INVALID_ARG;
  if (c->n_shared > 0) {
    if (c->n_shared > 16) return MOE_ERR_UNSUPPORTED;
    if (c->f_shared < 1) return MOE_ERR_INVALID_ARG;
    if (c->dtype == MOE_BF16 && c->f_shared % 64 != 0) return MOE_ERR_UNSUPPORTED;
    if (c->dtype == MOE_F32 && c->f_shared % 4 != 0) return MOE_ERR_UNSUPPORTED;
  }
  // every index the kernels form stays below 2^31 elements per row block
  const int64_t lim = (int64_t)1 << 31;
  if (c->T * c->k >= lim || c->h >= lim / 8 || c->f >= lim / 8) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 0 && (c->f_shared >= lim / 8 || c->T * c->n_shared >= lim))
    return MOE_ERR_UNSUPPORTED;
  if (c->dtype == MOE_BF16) {
    // The grouped GEMMs address one expert's weight matrix (h x f elements)
    // through a buffer resource of at most 2^31 - 1 bytes and their per-lane
    // copy offsets (row < 256 of a tile, times a row of K = h or f elements)
    // as 32-bit integers.
    const int64_t fmax = std::max(c->f, c->n_shared > 0 ? c->f_shared : 0);
    if (c->h * fmax * 2 >= lim) return MOE_ERR_UNSUPPORTED;
    if (256 * std::max(c->h, fmax) * 2 >= lim) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// C = ceil(cf * n / E) with cf taken at its exact binary value: cf = m * 2^ex.
int64_t exact_capacity(const moe_config* c) {
  int64_t C;
  if (!(c->capacity_factor > 0)) {
    C = c->T;
  } else {
    const int64_t n = (c->cap_mode == MOE_CAP_ASSIGNMENTS) ? c->T * c->k : c->T;
    int ex = 0;
    const double fr = frexp(c->capacity_factor, &ex);
    uint64_t m = (uint64_t)ldexp(fr, 53);
    ex -= 53;
    while (m != 0 && (m & 1) == 0) {
      m >>= 1;
      ++ex;
    }
    __int128 num = (__int128)m * n, den = c->E;
    if (ex >= 0) num <<= ex; else den <<= -ex;
    C = (int64_t)((num + den - 1) / den);
  }
  return C > c->min_capacity ? C : c->min_capacity;
}

Dims dims_of(const moe_config* c) {
  Dims d;
  d.T = c->T;
  d.h = c->h;
  d.f = c->f;
  d.E = c->E;
  d.k = c->k;
  d.bf16 = c->dtype == MOE_BF16;
  const int64_t Cx = exact_capacity(c);
  d.C = Cx < d.T ? Cx : d.T;  // no expert can receive more than T assignments
  const int64_t a = d.T * d.k, b = d.E * d.C;
  d.rows_max = a < b ? a : b;
  d.n_groups = c->n_groups > 1 ? c->n_groups : 1;
  d.topk_groups = c->n_groups > 1 ? c->topk_groups : 1;
  d.ns = c->n_shared;
  d.fs = c->n_shared > 0 ? c->f_shared : 0;
  return d;
}

size_t elem_bytes(const Dims& d) { return d.bf16 ? 2 : 4; }

struct Plan {
  size_t bytes = 0;
  size_t add(size_t n) {
    const size_t o = bytes;
    bytes += (n + 255) & ~size_t(255);
    return o;
  }
};

struct RouteWs {
  size_t wp, wnp, lpart, part, total;
  RouteShape rs;
};
RouteWs plan_route(const Dims& d, int noisy, Plan& pl) {
  RouteWs w;
  w.rs = route_shape((int)d.T, (int)d.E, (int)d.h, d.bf16, noisy);
  // bf16: zero-padded copies of W_r and W_noise (used when E % 8 != 0 or a
  // weight is not 16-byte aligned), and the logits GEMM's float32 products
  w.wp = d.bf16 ? pl.add((size_t)w.rs.Ew * d.h * 2) : 0;
  w.wnp = (d.bf16 && noisy) ? pl.add((size_t)w.rs.Ew * d.h * 2) : 0;
  w.lpart = d.bf16 ? pl.add((size_t)(noisy ? 2 : 1) * w.rs.KS * d.T * w.rs.EP * sizeof(float)) : 0;
  // per-workgroup partials: EP score columns and one LSE^2 column
  w.part = pl.add((size_t)(w.rs.nblk > 0 ? w.rs.nblk : 1) * (w.rs.EP + 1) * sizeof(double));
  w.total = pl.add((size_t)(w.rs.EP + 1) * sizeof(double));
  return w;
}

struct DispatchWs {
  size_t hist, base;
};
DispatchWs plan_dispatch(const Dims& d, Plan& pl) {
  const int64_t nchunk = (d.T + kChunk - 1) / kChunk;
  DispatchWs w;
  const size_t n = (size_t)(nchunk > 0 ? nchunk : 1) * d.k * d.E * sizeof(int32_t);
  w.hist = pl.add(n);
  w.base = pl.add(n);
  return w;
}

struct FfnWs {
  size_t map1, map2, A, part;
  FfnShape fs;
};
// Compute units of the current device (sizes the persistent GEMM grid; a
// host query, no synchronisation).  256 on MI355X if the query fails.
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  return n;
}

FfnWs plan_ffn(const Dims& d, Plan& pl) {
  FfnWs w;
  w.fs = ffn_shape(d.rows_max, (int)d.E, (int)d.h, (int)d.f, (int)d.T, (int)d.k, d.bf16,
                   device_cus());
  w.map1 = pl.add(tile_map_bytes(d.E, w.fs.mt1));
  w.map2 = pl.add(tile_map_bytes(d.E, w.fs.mt2));
  w.A = pl.add((size_t)(d.rows_max > 0 ? d.rows_max : 1) * d.f * elem_bytes(d));
  w.part = pl.add((size_t)w.fs.part_slots * kPartSlotBytes);
  return w;
}

// Shared experts: one dense pass over all T rows per shared expert, through
// the same grouped-GEMM kernels with a single "expert" (offsets {0, T}).
struct SharedWs {
  FfnShape fs;
  size_t map1, map2, offs, part, A, Ys;
};
SharedWs plan_shared(const Dims& d, bool with_ys, Plan& pl) {
  SharedWs w{};
  if (d.ns == 0) return w;
  w.fs = ffn_shape(d.T, 1, (int)d.h, (int)d.fs, (int)d.T, 1, d.bf16, device_cus());
  w.map1 = pl.add(tile_map_bytes(1, w.fs.mt1));
  w.map2 = pl.add(tile_map_bytes(1, w.fs.mt2));
  w.offs = pl.add(2 * sizeof(int32_t));
  w.part = pl.add((size_t)w.fs.part_slots * kPartSlotBytes);
  const size_t T1 = (size_t)(d.T > 0 ? d.T : 1);
  w.A = pl.add((size_t)d.ns * T1 * d.fs * elem_bytes(d));  // one intermediate per shared expert
  w.Ys = with_ys ? pl.add((size_t)d.ns * T1 * d.h * elem_bytes(d)) : 0;
  return w;
}

struct LayerWs {
  RouteWs route;
  DispatchWs disp;
  FfnWs ffn;
  SharedWs sh;
  size_t idx, gate, slot, row_token, count, kept, offset, X, Y, xs, scal;
};
LayerWs plan_layer(const Dims& d, int noisy, Plan& pl) {
  LayerWs w;
  w.route = plan_route(d, noisy, pl);
  w.disp = plan_dispatch(d, pl);
  w.ffn = plan_ffn(d, pl);
  w.sh = plan_shared(d, true, pl);
  const size_t tk = (size_t)(d.T > 0 ? d.T : 1) * d.k;
  const size_t rows = (size_t)(d.rows_max > 0 ? d.rows_max : 1);
  w.idx = pl.add(tk * 4);
  w.gate = pl.add(tk * 4);
  w.slot = pl.add(tk * 4);
  w.row_token = pl.add(rows * 4);
  w.count = pl.add(d.E * 4);
  w.kept = pl.add(d.E * 4);
  w.offset = pl.add((d.E + 1) * 4);
  w.X = pl.add(rows * d.h * elem_bytes(d));  // also holds the FP8 rows (rows * h bytes)
  w.Y = pl.add(rows * d.h * elem_bytes(d));
  w.xs = pl.add(rows * 4);                     // FP8 row scales
  w.scal = pl.add(64);
  return w;
}

// Backward workspaces.  Every product reads its operands as stored.
// The expert products' backward: tile maps, g | u and a (when recomputed),
// dA, dG | dU and the K-split partials of the largest product (min_slots
// partial tiles at least).
struct FfnBwdWs {
  FfnWs ffn;          // tile maps and a (ffn.A); ffn.part is this part
  FfnShape fsA, fsX;  // shapes of the dA (N = f, K = h) and dX (N = h, K = 2f) products
  size_t GU, dA, dGU;
  size_t dY8, sy, dYd;  // FP8 output gradients: codes, row scales, dequantised rows
};
FfnBwdWs plan_ffn_backward(const Dims& d, Plan& pl, int min_slots = 0) {
  FfnBwdWs w;
  const int ncu = device_cus();
  w.ffn.fs = ffn_shape(d.rows_max, (int)d.E, (int)d.h, (int)d.f, (int)d.T, (int)d.k, 1, ncu);
  w.fsA = ffn_shape(d.rows_max, (int)d.E, (int)d.f, (int)d.h, (int)d.T, (int)d.k, 1, ncu);
  w.fsX = ffn_shape(d.rows_max, (int)d.E, (int)d.h, (int)(2 * d.f), (int)d.T, (int)d.k, 1, ncu);
  const size_t rows = (size_t)(d.rows_max > 0 ? d.rows_max : 1);
  w.ffn.map1 = pl.add(tile_map_bytes(d.E, w.ffn.fs.mt1));
  w.ffn.map2 = pl.add(tile_map_bytes(d.E, w.ffn.fs.mt2));
  w.ffn.A = pl.add(rows * d.f * 2);
  w.GU = pl.add(rows * 2 * d.f * 2);
  w.dA = pl.add(rows * d.f * 2);
  w.dGU = pl.add(rows * 2 * d.f * 2);
  w.dY8 = pl.add(rows * d.h);
  w.sy = pl.add(rows * 4);
  w.dYd = pl.add(rows * d.h * 2);
  const int slots = std::max(std::max(min_slots, w.ffn.fs.part_slots),
                             std::max(w.fsA.part_slots, w.fsX.part_slots));
  w.ffn.part = pl.add((size_t)slots * kPartSlotBytes);
  return w;
}

// The router's backward: dH, dZ (noisy routing), the dW_r product's space,
// and for noisy routing the products Z = U W_noise (from the logits GEMM)
// and a padded copy of W_noise when it cannot be read in place.
struct RouterBwdWs {
  size_t dH, dZ, dwr, zpart, wnp;
  RouteShape zs;
};
RouterBwdWs plan_router_backward(const Dims& d, int noisy, Plan& pl) {
  RouterBwdWs w;
  const size_t T1 = (size_t)(d.T > 0 ? d.T : 1);
  w.dH = pl.add(T1 * d.E * 4);
  w.dZ = pl.add(T1 * d.E * 4);
  w.dwr = pl.add(dwr_part_bytes(d.T, (int)d.h, (int)d.E));
  w.zs = route_shape((int)d.T, (int)d.E, (int)d.h, 1, 0);
  w.zpart = noisy ? pl.add((size_t)w.zs.KS * T1 * w.zs.EP * 4) : 0;
  w.wnp = noisy ? pl.add((size_t)w.zs.Ew * d.h * 2) : 0;
  return w;
}

// The whole layer: the two above, the recomputed X and Y, dY, dX and the
// gates' gradient, and the shared experts' dense pass (one expert of T rows:
// its maps and rows {0, T}, one expert's g | u, dA and dG | dU at a time,
// every expert's a and dX).
struct BackwardWs {
  FfnBwdWs fb;
  RouterBwdWs rb;
  size_t X, Y, dY, dX, dgate;
  SharedWs sh;
  FfnShape shA, shX;
  size_t sGU, sdA, sdGU, sdX;
};
BackwardWs plan_backward(const Dims& d, int noisy, Plan& pl) {
  BackwardWs w;
  const int ncu = device_cus();
  w.sh = plan_shared(d, false, pl);
  int sh_slots = 0;
  const size_t T1 = (size_t)(d.T > 0 ? d.T : 1);
  if (d.ns > 0) {
    w.shA = ffn_shape(d.T, 1, (int)d.fs, (int)d.h, (int)d.T, 1, 1, ncu);
    w.shX = ffn_shape(d.T, 1, (int)d.h, (int)(2 * d.fs), (int)d.T, 1, 1, ncu);
    w.sGU = pl.add(T1 * 2 * d.fs * 2);
    w.sdA = pl.add(T1 * d.fs * 2);
    w.sdGU = pl.add(T1 * 2 * d.fs * 2);
    w.sdX = pl.add((size_t)d.ns * T1 * d.h * 2);
    sh_slots = std::max(w.sh.fs.part_slots, std::max(w.shA.part_slots, w.shX.part_slots));
  }
  w.fb = plan_ffn_backward(d, pl, sh_slots);
  w.rb = plan_router_backward(d, noisy, pl);
  const size_t rows = (size_t)(d.rows_max > 0 ? d.rows_max : 1);
  w.X = pl.add(rows * d.h * 2);
  w.Y = pl.add(rows * d.h * 2);
  w.dY = pl.add(rows * d.h * 2);
  w.dX = pl.add(rows * d.h * 2);
  w.dgate = pl.add(T1 * d.k * 4);
  return w;
}

// One expert's rows (at most min(C, T), a token taking an expert once; T for
// a shared expert) are addressed with 32-bit byte offsets by the
// weight-gradient products: rows of up to 2 f or h elements, plus the ring's
// steps past the end.
bool backward_offsets_fit(const Dims& d) {
  const int64_t pitch = 2 * std::max<int64_t>(2 * d.f, std::max<int64_t>(d.h, 2 * d.fs));
  const int64_t rows = std::max<int64_t>(std::min(d.C, d.T), d.ns > 0 ? d.T : 0) + 3 * 64;
  return rows * pitch <= 0x7fffffffLL;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                        \
  do {                                       \
    const hipError_t err_ = (expr);          \
    if (err_ != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

int32_t run_route(const Dims& d, const moe_config* c, const RouteWs& w, const void* U,
                  const void* W_r, const float* b_r, const float* b_sel, const void* W_noise,
                  float* noise_out, int32_t* idx, float* gate, float* logits, void* ws,
                  hipStream_t s, int32_t* hist = nullptr) {
  RouteParams p;
  p.T = (int)d.T;
  p.h = (int)d.h;
  p.E = (int)d.E;
  p.k = (int)d.k;
  p.score = c->score;
  p.gate = c->gate;
  p.U = U;
  p.b_r = b_r;
  p.b_sel = b_sel;
  p.n_groups = (int)d.n_groups;
  p.topk_groups = (int)d.topk_groups;
  p.seed = c->seed;
  p.rng_offset = c->rng_offset;
  p.noise_out = c->noisy ? noise_out : nullptr;
  p.topk_idx = idx;
  p.topk_gate = gate;
  p.logits = logits;
  p.prob_part = at<double>(ws, w.part);
  p.W = W_r;
  p.Wn = c->noisy ? W_noise : nullptr;
  p.lpart = nullptr;
  if (d.bf16) {
    // the logits GEMM reads the weights in place in rows of a multiple of 8
    // columns at 16-byte alignment; anything else goes through a padded copy
    auto in_place = [&](const void* W) { return d.E % 8 == 0 && (uintptr_t)W % 16 == 0; };
    if (!in_place(W_r)) {
      MOE_TRY(launch_pad_router_w(W_r, at<void>(ws, w.wp), (int)d.h, (int)d.E, w.rs.Ew, s));
      p.W = at<void>(ws, w.wp);
    }
    if (c->noisy && !in_place(W_noise)) {
      MOE_TRY(launch_pad_router_w(W_noise, at<void>(ws, w.wnp), (int)d.h, (int)d.E, w.rs.Ew, s));
      p.Wn = at<void>(ws, w.wnp);
    }
    p.lpart = at<float>(ws, w.lpart);
    p.hist = hist;
  }
  MOE_TRY(launch_route(w.rs, p, d.bf16, c->noisy, s));
  return MOE_OK;
}

// xs != NULL: FP8 dispatch (X receives E4M3 codes, xs the row scales).
// fused: steps the scan workgroup also runs (the layer forward's tile maps
// and statistics), or NULL.
int32_t run_dispatch(const Dims& d, const moe_config* c, const DispatchWs& w, const void* U,
                     const int32_t* idx, void* X, int32_t* row_token, int32_t* slot,
                     int32_t* count, int32_t* kept, int32_t* offset, void* ws, hipStream_t s,
                     float* xs = nullptr, const DispatchParams* fused = nullptr) {
  DispatchParams p;
  if (fused) p = *fused;
  p.T = (int)d.T;
  p.E = (int)d.E;
  p.k = (int)d.k;
  p.C = (int)d.C;
  p.token_major = c->fill == MOE_FILL_TOKEN_MAJOR;
  p.topk_idx = idx;
  p.hist = at<int32_t>(ws, w.hist);
  p.base = at<int32_t>(ws, w.base);
  p.count = count;
  p.kept = kept;
  p.offset = offset;
  p.slot = slot;
  p.row_token = row_token;
  MOE_TRY(launch_dispatch(p, s));
  if (xs)
    MOE_TRY(launch_permute_fp8(U, slot, X, xs, (int)d.T, (int)d.h, (int)d.k, s));
  else
    MOE_TRY(launch_permute(U, slot, X, (int)d.T, (int)d.h, (int)d.k, d.bf16, s));
  return MOE_OK;
}

// The FP8 path takes bf16 inputs and K steps of 128 FP8 elements.
int32_t check_fp8(const moe_config* cfg) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16 || cfg->h % 128 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int32_t run_tile_map(const Dims& d, const FfnWs& w, const int32_t* offset, void* ws,
                     hipStream_t s) {
  if (!d.bf16) return MOE_OK;
  MOE_TRY(launch_tile_map(offset, (int)d.E, w.fs.bm1, w.fs.bm2, at<int32_t>(ws, w.map1),
                          at<int32_t>(ws, w.map2), s));
  return MOE_OK;
}

// FP8 operands of the up-projection: E4M3 weights with their row scales, and
// the scales of the dispatched rows.
struct Fp8Up {
  const void* Wg;
  const float* sg;
  const void* Wu;
  const float* su;
  const float* xs;
};

// Expects run_tile_map to have been enqueued before.  f8 != NULL: X holds
// E4M3 rows and the gate/up GEMM runs on FP8.  A: where the SwiGLU products go
// (NULL: the workspace); GU: also keep the pre-activations g, u (bf16 only).
int32_t run_gate_up(const Dims& d, const FfnWs& w, const void* X, const int32_t* offset,
                    const void* Wg, const void* Wu, const void* Wd, void* Y, void* ws,
                    hipStream_t s, const Fp8Up* f8 = nullptr, void* A = nullptr,
                    void* GU = nullptr) {
  if (!A) A = at<void>(ws, w.A);
  if (f8) {
    MOE_TRY(launch_gate_up_fp8(w.fs, X, f8->xs, offset, at<int32_t>(ws, w.map1), f8->Wg, f8->sg,
                               f8->Wu, f8->su, A, at<float>(ws, w.part), (int)d.E, (int)d.h,
                               (int)d.f, s));
    return MOE_OK;
  }
  if (!d.bf16)
    return hip_status(launch_ffn_f32(X, offset, Wg, Wu, Wd, A, Y, d.rows_max, (int)d.E,
                                     (int)d.h, (int)d.f, s));
  if (GU)
    MOE_TRY(launch_gate_up_save(w.fs, X, offset, at<int32_t>(ws, w.map1), Wg, Wu, A, GU,
                                at<float>(ws, w.part), (int)d.E, (int)d.h, (int)d.f, s));
  else
    MOE_TRY(launch_gate_up(w.fs, X, offset, at<int32_t>(ws, w.map1), Wg, Wu, A,
                           at<float>(ws, w.part), (int)d.E, (int)d.h, (int)d.f, 1, s));
  return MOE_OK;
}

int32_t run_down(const Dims& d, const FfnWs& w, const int32_t* offset, const void* Wd, void* Y,
                 void* ws, hipStream_t s, const void* A = nullptr) {
  if (!d.bf16) return MOE_OK;  // the float32 path ran both products already
  MOE_TRY(launch_down(w.fs, A ? A : at<void>(ws, w.A), offset, at<int32_t>(ws, w.map2), Wd, Y,
                      at<float>(ws, w.part), (int)d.E, (int)d.h, (int)d.f, 1, s));
  return MOE_OK;
}

const char* elem_ptr(const void* base, size_t elems, const Dims& d) {
  return static_cast<const char*>(base) + elems * elem_bytes(d);
}

// Gate/up products of every shared expert (the float32 path does the whole
// FFN here).
int32_t run_shared_gate_up(const Dims& d, const SharedWs& w, const void* U, const void* Wsg,
                           const void* Wsu, const void* Wsd, void* Ys, void* ws, hipStream_t s) {
  if (d.ns == 0 || d.T == 0) return MOE_OK;
  int32_t* offs = at<int32_t>(ws, w.offs);
  MOE_TRY(launch_dense_offsets((int)d.T, offs, s));
  const size_t fh = (size_t)d.fs * d.h, th = (size_t)d.T * d.h, tf = (size_t)d.T * d.fs;
  if (d.bf16)
    MOE_TRY(launch_tile_map(offs, 1, w.fs.bm1, w.fs.bm2, at<int32_t>(ws, w.map1),
                            at<int32_t>(ws, w.map2), s));
  for (int64_t i = 0; i < d.ns; ++i) {
    void* A = at<char>(ws, w.A) + i * tf * elem_bytes(d);
    if (d.bf16) {
      MOE_TRY(launch_gate_up(w.fs, U, offs, at<int32_t>(ws, w.map1), elem_ptr(Wsg, i * fh, d),
                             elem_ptr(Wsu, i * fh, d), A, at<float>(ws, w.part), 1, (int)d.h,
                             (int)d.fs, 1, s));
    } else {
      MOE_TRY(launch_ffn_f32(U, offs, elem_ptr(Wsg, i * fh, d), elem_ptr(Wsu, i * fh, d),
                             elem_ptr(Wsd, i * fh, d), A,
                             static_cast<char*>(Ys) + i * th * elem_bytes(d), d.T, 1, (int)d.h,
                             (int)d.fs, s));
    }
  }
  return MOE_OK;
}

int32_t run_shared_down(const Dims& d, const SharedWs& w, const void* Wsd, void* Ys, void* ws,
                        hipStream_t s) {
  if (d.ns == 0 || d.T == 0 || !d.bf16) return MOE_OK;
  const size_t fh = (size_t)d.fs * d.h, th = (size_t)d.T * d.h, tf = (size_t)d.T * d.fs;
  for (int64_t i = 0; i < d.ns; ++i)
    MOE_TRY(launch_down(w.fs, at<char>(ws, w.A) + i * tf * elem_bytes(d), at<int32_t>(ws, w.offs),
                        at<int32_t>(ws, w.map2), elem_ptr(Wsd, i * fh, d),
                        static_cast<char*>(Ys) + i * th * elem_bytes(d), at<float>(ws, w.part),
                        1, (int)d.h, (int)d.fs, 1, s));
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch failed";
    default: return "unknown moe status";
  }
}

int32_t moe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                        void* stream) {
  if (bytes % 16 != 0 || blocks <= 0 || blocks > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (bytes > 0 && (!src || !sink)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_stream_read(src, bytes, sink, blocks, static_cast<hipStream_t>(stream)));
}

int32_t moe_capacity(const moe_config* cfg, int64_t* C) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!C) return MOE_ERR_INVALID_ARG;
  *C = exact_capacity(cfg);
  return MOE_OK;
}

int32_t moe_max_rows(const moe_config* cfg, int64_t* rows_max) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!rows_max) return MOE_ERR_INVALID_ARG;
  *rows_max = dims_of(cfg).rows_max;
  return MOE_OK;
}

int32_t moe_workspace_size(const moe_config* cfg, int32_t entry, size_t* bytes) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  const Dims d = dims_of(cfg);
  Plan pl;
  switch (entry) {
    case MOE_WS_ROUTE: plan_route(d, cfg->noisy, pl); break;
    case MOE_WS_DISPATCH: plan_dispatch(d, pl); break;
    case MOE_WS_EXPERT_FFN: plan_ffn(d, pl); break;
    case MOE_WS_LAYER: plan_layer(d, cfg->noisy, pl); break;
    case MOE_WS_SHARED_FFN: plan_shared(d, false, pl); break;
    case MOE_WS_BACKWARD: plan_backward(d, cfg->noisy, pl); break;
    case MOE_WS_EXPERT_FFN_BACKWARD: plan_ffn_backward(d, pl); break;
    case MOE_WS_ROUTER_BACKWARD: plan_router_backward(d, cfg->noisy, pl); break;
    default: return MOE_ERR_INVALID_ARG;
  }
  *bytes = pl.bytes;
  return MOE_OK;
}

int32_t moe_route(const moe_config* cfg, const void* U, const void* W_r, const float* b_r,
                  const float* b_sel, const void* W_noise, float* noise_out,
                  int32_t* topk_idx, float* topk_gate, float* logits, float* prob_sum,
                  void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (d.T > 0 && (!U || !topk_idx || !topk_gate)) return MOE_ERR_INVALID_ARG;
  if (!W_r || !ws) return MOE_ERR_INVALID_ARG;
  if (cfg->noisy && !W_noise) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const RouteWs w = plan_route(d, cfg->noisy, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_route(d, cfg, w, U, W_r, b_r, b_sel, W_noise, noise_out, topk_idx, topk_gate, logits,
                 ws, s);
  if (st != MOE_OK) return st;
  if (prob_sum)
    return hip_status(launch_prob_reduce(at<double>(ws, w.part), w.rs.nblk, w.rs.EP, (int)d.E,
                                         nullptr, prob_sum, s));
  return MOE_OK;
}

int32_t moe_dispatch(const moe_config* cfg, const void* U, const int32_t* topk_idx, void* X,
                     int32_t* row_token, int32_t* slot, int32_t* count, int32_t* kept,
                     int32_t* offset, void* ws, size_t ws_bytes, void* stream) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (d.T > 0 && (!U || !topk_idx || !X || !row_token || !slot)) return MOE_ERR_INVALID_ARG;
  if (!count || !kept || !offset || !ws) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const DispatchWs w = plan_dispatch(d, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  return run_dispatch(d, cfg, w, U, topk_idx, X, row_token, slot, count, kept, offset, ws,
                      static_cast<hipStream_t>(stream));
}

int32_t moe_dispatch_noalloc(const moe_config* cfg, const void* U, const int32_t* topk_idx,
                             void* X, int32_t* row_token, int32_t* slot, int32_t* count,
                             int32_t* kept, int32_t* offset, void* stream) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (d.T > 0 && (!U || !topk_idx || !X || !row_token || !slot)) return MOE_ERR_INVALID_ARG;
  if (!count || !kept || !offset) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const DispatchWs w = plan_dispatch(d, pl);
  if (pl.bytes > kDispatchScratchBytes) return MOE_ERR_WORKSPACE;
  int32_t* scratch = nullptr;
  MOE_TRY(dispatch_scratch(&scratch));
  return run_dispatch(d, cfg, w, U, topk_idx, X, row_token, slot, count, kept, offset, scratch,
                      static_cast<hipStream_t>(stream));
}

int32_t moe_expert_ffn(const moe_config* cfg, const void* X, const int32_t* offset,
                       const void* W_gate, const void* W_up, const void* W_down, void* Y,
                       void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (!offset || !W_gate || !W_up || !W_down || !ws) return MOE_ERR_INVALID_ARG;
  if (d.rows_max > 0 && (!X || !Y)) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const FfnWs w = plan_ffn(d, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_tile_map(d, w, offset, ws, s);
  if (st != MOE_OK) return st;
  st = run_gate_up(d, w, X, offset, W_gate, W_up, W_down, Y, ws, s);
  if (st != MOE_OK) return st;
  return run_down(d, w, offset, W_down, Y, ws, s);
}

int32_t moe_shared_ffn(const moe_config* cfg, const void* U, const void* Ws_gate,
                       const void* Ws_up, const void* Ws_down, void* Y_shared, void* ws,
                       size_t ws_bytes, void* stream) {
  int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (d.ns == 0) return MOE_ERR_INVALID_ARG;
  if (!Ws_gate || !Ws_up || !Ws_down || !ws) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!U || !Y_shared || Y_shared == U)) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const SharedWs w = plan_shared(d, false, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_shared_gate_up(d, w, U, Ws_gate, Ws_up, Ws_down, Y_shared, ws, s);
  if (st != MOE_OK) return st;
  return run_shared_down(d, w, Ws_down, Y_shared, ws, s);
}

int32_t moe_combine(const moe_config* cfg, const void* U, const void* Y, const int32_t* slot,
                    const float* topk_gate, const void* Y_shared, void* out, void* stream) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (d.T > 0 && (!U || !slot || !topk_gate || !out)) return MOE_ERR_INVALID_ARG;
  if (d.rows_max > 0 && !Y) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (out == U || out == Y || (Y_shared && out == Y_shared)))
    return MOE_ERR_INVALID_ARG;
  if (Y_shared && d.ns == 0) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(U, Y, slot, topk_gate, Y_shared, (int)d.ns, out, (int)d.T,
                                   (int)d.h, (int)d.k, d.bf16,
                                   static_cast<hipStream_t>(stream)));
}

int32_t moe_update_bias(const moe_config* cfg, const int32_t* count, float* b_sel, float gamma,
                        void* stream) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!count || !b_sel || !(gamma >= 0.f) || isinf(gamma)) return MOE_ERR_INVALID_ARG;
  return hip_status(
      launch_update_bias(count, b_sel, gamma, (int)cfg->E, static_cast<hipStream_t>(stream)));
}

int32_t moe_stats(const moe_config* cfg, const int32_t* count, const int32_t* kept,
                  const float* prob_sum, float* f, float* P, float* aux_loss, float* maxvio,
                  int32_t* n_dropped, void* stream) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!count || !kept || !prob_sum) return MOE_ERR_INVALID_ARG;
  StatsParams p{(int)cfg->T, (int)cfg->E, (int)cfg->k, count, kept, nullptr,
                prob_sum, f, P, aux_loss, maxvio, n_dropped, nullptr};
  return hip_status(launch_stats(p, static_cast<hipStream_t>(stream)));
}

int32_t moe_router_z_loss(const moe_config* cfg, const float* logits, float* z_loss,
                          void* stream) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!z_loss || (cfg->T > 0 && !logits)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_z_loss(logits, (int)cfg->T, (int)cfg->E, z_loss,
                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The layer; f8 != NULL runs the FP8 dispatch and up-projection (its weights
// replace W_gate and W_up).
int32_t layer_impl(const moe_config* cfg, const void* U, const void* W_r, const float* b_r,
                   const float* b_sel, const void* W_noise, const void* W_gate,
                   const void* W_up, const void* W_down, const void* Ws_gate, const void* Ws_up, const void* Ws_down, void* out, const moe_aux_outputs* aux,
                   void* const* stage_events, void* ws, size_t ws_bytes, void* stream,
                   Fp8Up* f8) {
  int32_t st = f8 ? check_fp8(cfg) : check_config(cfg);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (d.T > 0 && (!U || !out)) return MOE_ERR_INVALID_ARG;
  if (!W_r || !W_gate || !W_up || !W_down || !ws) return MOE_ERR_INVALID_ARG;
  if (d.ns > 0 && (!Ws_gate || !Ws_up || !Ws_down)) return MOE_ERR_INVALID_ARG;
  if (cfg->noisy && !W_noise) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && out == U) return MOE_ERR_INVALID_ARG;
  if (aux && aux->GU && (!d.bf16 || f8)) return MOE_ERR_UNSUPPORTED;
  Plan pl;
  const LayerWs w = plan_layer(d, cfg->noisy, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  moe_aux_outputs o;
  memset(&o, 0, sizeof(o));
  if (aux) o = *aux;
  int32_t* idx = o.topk_idx ? o.topk_idx : at<int32_t>(ws, w.idx);
  float* gate = o.topk_gate ? o.topk_gate : at<float>(ws, w.gate);
  int32_t* slot = o.slot ? o.slot : at<int32_t>(ws, w.slot);
  int32_t* row_token = o.row_token ? o.row_token : at<int32_t>(ws, w.row_token);
  int32_t* count = o.count ? o.count : at<int32_t>(ws, w.count);
  int32_t* kept = o.kept ? o.kept : at<int32_t>(ws, w.kept);
  int32_t* offset = o.offset ? o.offset : at<int32_t>(ws, w.offset);
  // the FP8 rows stay in the workspace (aux X is typed for the input dtype)
  void* X = (o.X && !f8) ? o.X : at<void>(ws, w.X);
  void* Y = o.Y ? o.Y : at<void>(ws, w.Y);
  float* xs = f8 ? at<float>(ws, w.xs) : nullptr;
  if (f8) f8->xs = xs;
  void* Ys = d.ns == 0 ? nullptr : (o.Y_shared ? o.Y_shared : at<void>(ws, w.sh.Ys));
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    return (stage_events && stage_events[i])
               ? hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s)
               : hipSuccess;
  };

  MOE_TRY(mark(0));
  // bf16 with many experts: the selection kernel also counts the dispatch
  // histograms.  Each 256-token chunk and rank adds about 256 / E increments
  // to each counter; with few experts (E = 8: 32) those atomics queue on the
  // same addresses and cost more than the histogram launch they replace.
  const bool hist_in_select = d.bf16 && d.E >= 32;
  st = run_route(d, cfg, w.route, U, W_r, b_r, b_sel, W_noise, o.noise, idx, gate, o.logits,
                 ws, s, hist_in_select ? at<int32_t>(ws, w.disp.hist) : nullptr);
  if (st != MOE_OK) return st;
  MOE_TRY(mark(1));
  // the dispatch's scan launch also writes the GEMMs' tile maps and sums the
  // router's P partials; its assignment launch computes the load statistics
  DispatchParams fused;
  fused.hist_ready = hist_in_select;
  fused.prob_part = at<double>(ws, w.route.part);
  fused.prob_nblk = w.route.rs.nblk;
  fused.prob_EP = w.route.rs.EP;
  fused.prob_total = at<double>(ws, w.route.total);
  fused.prob_out = o.prob_sum;
  if (d.bf16) {
    fused.bm1 = w.ffn.fs.bm1;
    fused.bm2 = w.ffn.fs.bm2;
    fused.map1 = at<int32_t>(ws, w.ffn.map1);
    fused.map2 = at<int32_t>(ws, w.ffn.map2);
  }
  fused.stats_on = 1;
  fused.stats = StatsParams{(int)d.T, (int)d.E, (int)d.k, count, kept,
                            at<double>(ws, w.route.total), nullptr, o.f, o.P,
                            o.aux_loss ? o.aux_loss : at<float>(ws, w.scal),
                            o.maxvio ? o.maxvio : at<float>(ws, w.scal) + 1,
                            o.n_dropped ? o.n_dropped : at<int32_t>(ws, w.scal) + 2, o.z_loss};
  st = run_dispatch(d, cfg, w.disp, U, idx, X, row_token, slot, count, kept, offset, ws, s, xs,
                    &fused);
  if (st != MOE_OK) return st;
  MOE_TRY(mark(2));
  st = run_gate_up(d, w.ffn, X, offset, W_gate, W_up, W_down, Y, ws, s, f8, o.A, o.GU);
  if (st != MOE_OK) return st;
  st = run_shared_gate_up(d, w.sh, U, Ws_gate, Ws_up, Ws_down, Ys, ws, s);
  if (st != MOE_OK) return st;
  MOE_TRY(mark(3));
  st = run_down(d, w.ffn, offset, W_down, Y, ws, s, o.A);
  if (st != MOE_OK) return st;
  st = run_shared_down(d, w.sh, Ws_down, Ys, ws, s);
  if (st != MOE_OK) return st;
  MOE_TRY(mark(4));
  MOE_TRY(launch_combine(U, Y, slot, gate, Ys, (int)d.ns, out, (int)d.T, (int)d.h, (int)d.k,
                         d.bf16, s));
  MOE_TRY(mark(5));
  MOE_TRY(mark(6));
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_layer_forward(const moe_config* cfg, const void* U, const void* W_r,
                          const float* b_r, const float* b_sel, const void* W_noise,
                          const void* W_gate, const void* W_up,
                          const void* W_down, const void* Ws_gate, const void* Ws_up,
                          const void* Ws_down, void* out, const moe_aux_outputs* aux,
                          void* const* stage_events, void* ws, size_t ws_bytes,
                          void* stream) {
  return layer_impl(cfg, U, W_r, b_r, b_sel, W_noise, W_gate, W_up, W_down, Ws_gate,
                    Ws_up, Ws_down, out, aux, stage_events, ws, ws_bytes, stream, nullptr);
}

int32_t moe_layer_forward_fp8(const moe_config* cfg, const void* U, const void* W_r,
                              const float* b_r, const float* b_sel, const void* W_noise,
                              const void* W8_gate, const float* s_gate,
                              const void* W8_up, const float* s_up, const void* W_down,
                              const void* Ws_gate, const void* Ws_up, const void* Ws_down,
                              void* out, const moe_aux_outputs* aux, void* const* stage_events,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!s_gate || !s_up) return MOE_ERR_INVALID_ARG;
  Fp8Up f8{W8_gate, s_gate, W8_up, s_up, nullptr};
  return layer_impl(cfg, U, W_r, b_r, b_sel, W_noise, W8_gate, W8_up, W_down, Ws_gate,
                    Ws_up, Ws_down, out, aux, stage_events, ws, ws_bytes, stream, &f8);
}

}  // extern "C"

namespace {

// Steps of the backward shared by the layer call and the staged calls.

// FP8 output gradients for the dA product: the dY rows' codes and scales,
// and W_down^T's.
struct Fp8Grad {
  const void* dY8;
  const float* sy;
  const void* WdT8;
  const float* sdT;
};

// The expert products backward for dY rows (tile maps already built in
// w.ffn): dA = dY W_down[e] (on FP8 operands when f8 is set, dY then being
// the dequantised rows), SwiGLU backward from g | u, dX = [dg du]
// [W_gate[e]; W_up[e]], then the weight gradients from dY, a, dG | dU and X.
int32_t run_ffn_backward(const Dims& d, const FfnBwdWs& w, void* ws, const void* X,
                         const void* GU, const void* A, const void* dY, const int32_t* offset,
                         const void* Wg, const void* Wu, const void* Wd, void* dX, void* dWg,
                         void* dWu, void* dWd, hipStream_t s, const Fp8Grad* f8 = nullptr) {
  const int E = (int)d.E, h = (int)d.h, f = (int)d.f, ncu = device_cus();
  const int32_t* map = at<int32_t>(ws, w.ffn.map1);  // every product uses the same row tiles
  float* part = at<float>(ws, w.ffn.part);
  void* dA = at<void>(ws, w.dA);
  void* dGU = at<void>(ws, w.dGU);
  if (f8)
    MOE_TRY(launch_dgrad_fp8(w.fsA, f8->dY8, f8->sy, offset, map, f8->WdT8, f8->sdT, dA, part, E,
                             f, h, s));
  else
    MOE_TRY(launch_dgrad(w.fsA, dY, offset, map, Wd, Wd, h, dA, part, E, f, h, s));
  MOE_TRY(launch_swiglu_bwd(dA, GU, offset, E, d.rows_max, f, dGU, s));
  MOE_TRY(launch_dgrad(w.fsX, dGU, offset, map, Wg, Wu, f, dX, part, E, h, 2 * f, s));
  const int64_t rows = d.rows_max;
  MOE_TRY(launch_wgrad(dY, h, A, f, offset, dWd, E, h, f, rows, ncu, s));
  MOE_TRY(launch_wgrad(dGU, 2 * f, X, h, offset, dWg, E, f, h, rows, ncu, s));
  MOE_TRY(launch_wgrad(static_cast<const char*>(dGU) + (size_t)f * 2, 2 * f, X, h, offset, dWu,
                       E, f, h, rows, ncu, s));
  return MOE_OK;
}

// g | u and a recomputed from X (tile maps already built in w.ffn).
int32_t run_ffn_recompute(const Dims& d, const FfnBwdWs& w, void* ws, const void* X,
                          const int32_t* offset, const void* Wg, const void* Wu, void* GU,
                          void* A, hipStream_t s) {
  MOE_TRY(launch_gate_up_save(w.ffn.fs, X, offset, at<int32_t>(ws, w.ffn.map1), Wg, Wu, A, GU,
                              at<float>(ws, w.ffn.part), (int)d.E, (int)d.h, (int)d.f, s));
  return MOE_OK;
}

// The router's backward and the input gradient: dH from the gates' gradient
// and the aux and z terms (dZ for the noise term), then
// dU = dOut + sum_r dX[slot] + dH W_r^T (+ dZ W_noise^T) (+ the shared experts'
// dXs), dW_r, db_r (dW_noise).
int32_t run_router_backward(const moe_config* cfg, const Dims& d, const RouterBwdWs& w, void* ws,
                            const void* U, const void* W_r, const float* logits,
                            const int32_t* topk_idx, const float* topk_gate,
                            const int32_t* slot, const int32_t* count, const float* dgate,
                            const void* dOut, const void* dX, const void* dXs, int ns,
                            float alpha, float c_z, const moe_backward_extras* extra, void* dU,
                            float* dW_r, float* db_r, hipStream_t s) {
  const int E = (int)d.E, h = (int)d.h, T = (int)d.T, k = (int)d.k;
  float* dH = at<float>(ws, w.dH);
  MOE_TRY(launch_router_bwd(logits, topk_idx, topk_gate, dgate, count, T, E, k, cfg->score,
                            cfg->gate == MOE_GATE_RENORM, alpha, c_z, dH, s));
  float* dZ = nullptr;
  if (cfg->noisy) {
    dZ = at<float>(ws, w.dZ);
    // Z = U W_noise again, by the logits GEMM (rows of a multiple of 8
    // columns at 16-byte alignment, else from a padded copy)
    const void* Wn = extra->W_noise;
    if (E % 8 != 0 || (uintptr_t)Wn % 16 != 0) {
      MOE_TRY(launch_pad_router_w(Wn, at<void>(ws, w.wnp), h, E, w.zs.Ew, s));
      Wn = at<void>(ws, w.wnp);
    }
    float* zpart = at<float>(ws, w.zpart);
    MOE_TRY(launch_route_products(w.zs, U, Wn, zpart, T, h, s));
    MOE_TRY(launch_noise_grad(zpart, w.zs.KS, w.zs.EP, dH, cfg->seed, cfg->rng_offset, dZ, T, E,
                              s));
  }
  MOE_TRY(launch_grad_input(dOut, dX, slot, dH, W_r, dZ, cfg->noisy ? extra->W_noise : nullptr,
                            dXs, T > 0 ? ns : 0, dU, T, h, E, k, s));
  MOE_TRY(launch_dwr(U, dH, dW_r, db_r, at<float>(ws, w.dwr), T, h, E, s));
  if (cfg->noisy)
    MOE_TRY(launch_dwr(U, dZ, extra->dW_noise, nullptr, at<float>(ws, w.dwr), T, h, E, s));
  return MOE_OK;
}

int32_t check_noise_extras(const moe_config* cfg, const moe_backward_extras* extra) {
  if (cfg->noisy && (!extra || !extra->W_noise || !extra->dW_noise)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// dY rows to FP8 codes and scales, then back to bf16 in place (the values
// every other use of dY takes).
int32_t quantize_grad_rows(const Dims& d, const FfnBwdWs& w, void* ws, void* dY, hipStream_t s) {
  MOE_TRY(launch_quantize_rows_fp8(dY, d.rows_max, (int)d.h, at<void>(ws, w.dY8),
                                   at<float>(ws, w.sy), s));
  MOE_TRY(launch_dequant_rows_fp8(at<void>(ws, w.dY8), at<float>(ws, w.sy), d.rows_max,
                                  (int)d.h, dY, s));
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_combine_backward(const moe_config* cfg, const void* dOut, const void* Y,
                             const int32_t* slot, const float* topk_gate, void* dY, float* dgate,
                             void* stream) {
  const int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (cfg->T > 0 && (!dOut || !Y || !slot || !topk_gate || !dY || !dgate))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine_bwd(dOut, Y, slot, topk_gate, dY, dgate, (int)cfg->T,
                                       (int)cfg->h, (int)cfg->k,
                                       static_cast<hipStream_t>(stream)));
}

int32_t moe_expert_ffn_backward(const moe_config* cfg, const void* X, const int32_t* offset,
                                const void* W_gate, const void* W_up, const void* W_down,
                                const void* dY, const void* GU, const void* A, void* dX,
                                void* dW_gate, void* dW_up, void* dW_down, void* ws,
                                size_t ws_bytes, void* stream) {
  const int32_t st0 = check_config(cfg);
  if (st0 != MOE_OK) return st0;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const Dims d = dims_of(cfg);
  if (!offset || !W_gate || !W_up || !W_down || !dW_gate || !dW_up || !dW_down || !ws)
    return MOE_ERR_INVALID_ARG;
  if (d.rows_max > 0 && (!X || !dY || !dX)) return MOE_ERR_INVALID_ARG;
  if ((GU == nullptr) != (A == nullptr)) return MOE_ERR_INVALID_ARG;
  if (!backward_offsets_fit(d)) return MOE_ERR_UNSUPPORTED;
  Plan pl;
  const FfnBwdWs w = plan_ffn_backward(d, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t st = run_tile_map(d, w.ffn, offset, ws, s);
  if (st != MOE_OK) return st;
  if (!GU) {
    GU = at<void>(ws, w.GU);
    A = at<void>(ws, w.ffn.A);
    st = run_ffn_recompute(d, w, ws, X, offset, W_gate, W_up, const_cast<void*>(GU),
                           const_cast<void*>(A), s);
    if (st != MOE_OK) return st;
  }
  return run_ffn_backward(d, w, ws, X, GU, A, dY, offset, W_gate, W_up, W_down, dX, dW_gate,
                          dW_up, dW_down, s);
}

int32_t moe_expert_ffn_backward_fp8(const moe_config* cfg, const void* X, const int32_t* offset,
                                    const void* W_gate, const void* W_up, const void* W_downT8,
                                    const float* s_downT, const void* dY8,
                                    const float* dY_scale, const void* GU, const void* A,
                                    void* dX, void* dW_gate, void* dW_up, void* dW_down,
                                    void* ws, size_t ws_bytes, void* stream) {
  const int32_t st0 = check_fp8(cfg);
  if (st0 != MOE_OK) return st0;
  const Dims d = dims_of(cfg);
  if (!offset || !W_gate || !W_up || !W_downT8 || !s_downT || !dW_gate || !dW_up || !dW_down ||
      !ws)
    return MOE_ERR_INVALID_ARG;
  if (d.rows_max > 0 && (!X || !dY8 || !dY_scale || !dX)) return MOE_ERR_INVALID_ARG;
  if ((GU == nullptr) != (A == nullptr)) return MOE_ERR_INVALID_ARG;
  if (!backward_offsets_fit(d)) return MOE_ERR_UNSUPPORTED;
  Plan pl;
  const FfnBwdWs w = plan_ffn_backward(d, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t st = run_tile_map(d, w.ffn, offset, ws, s);
  if (st != MOE_OK) return st;
  if (!GU) {
    GU = at<void>(ws, w.GU);
    A = at<void>(ws, w.ffn.A);
    st = run_ffn_recompute(d, w, ws, X, offset, W_gate, W_up, const_cast<void*>(GU),
                           const_cast<void*>(A), s);
    if (st != MOE_OK) return st;
  }
  void* dYd = at<void>(ws, w.dYd);
  MOE_TRY(launch_dequant_rows_fp8(dY8, dY_scale, d.rows_max, (int)d.h, dYd, s));
  const Fp8Grad f8{dY8, dY_scale, W_downT8, s_downT};
  return run_ffn_backward(d, w, ws, X, GU, A, dYd, offset, W_gate, W_up, nullptr, dX, dW_gate,
                          dW_up, dW_down, s, &f8);
}

int32_t moe_router_backward(const moe_config* cfg, const void* U, const void* W_r,
                            const float* logits, const int32_t* topk_idx, const float* topk_gate,
                            const int32_t* slot, const int32_t* count, const float* dgate,
                            const void* dOut, const void* dX, float alpha, float c_z,
                            const moe_backward_extras* extra, void* dU, float* dW_r,
                            float* db_r, void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  st = check_noise_extras(cfg, extra);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (!W_r || !count || !dW_r || !ws) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!U || !logits || !topk_idx || !topk_gate || !slot || !dgate || !dOut || !dX ||
                  !dU))
    return MOE_ERR_INVALID_ARG;
  if (!isfinite(alpha) || !isfinite(c_z)) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const RouterBwdWs w = plan_router_backward(d, cfg->noisy, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  return run_router_backward(cfg, d, w, ws, U, W_r, logits, topk_idx, topk_gate, slot, count,
                             dgate, dOut, dX, nullptr, 0, alpha, c_z, extra, dU, dW_r, db_r,
                             static_cast<hipStream_t>(stream));
}

int32_t moe_layer_backward(const moe_config* cfg, const void* U, const void* W_r,
                           const void* W_gate, const void* W_up, const void* W_down,
                           const float* logits, const int32_t* topk_idx, const float* topk_gate,
                           const int32_t* slot, const int32_t* count, const int32_t* offset,
                           const void* dOut, float alpha, float c_z, void* dU, float* dW_r,
                           float* db_r, void* dW_gate, void* dW_up, void* dW_down,
                           const moe_aux_outputs* saved, const moe_backward_extras* extra,
                           void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  st = check_noise_extras(cfg, extra);
  if (st != MOE_OK) return st;
  if (cfg->n_shared > 0 &&
      (!extra || !extra->Ws_gate || !extra->Ws_up || !extra->Ws_down || !extra->dWs_gate ||
       !extra->dWs_up || !extra->dWs_down))
    return MOE_ERR_INVALID_ARG;
  const Dims d = dims_of(cfg);
  if (!W_r || !W_gate || !W_up || !W_down || !count || !offset || !dW_r || !dW_gate ||
      !dW_up || !dW_down || !ws)
    return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!U || !logits || !topk_idx || !topk_gate || !slot || !dOut || !dU))
    return MOE_ERR_INVALID_ARG;
  if (!isfinite(alpha) || !isfinite(c_z)) return MOE_ERR_INVALID_ARG;
  if (saved && (!saved->X || !saved->GU || !saved->A || !saved->Y)) return MOE_ERR_INVALID_ARG;
  const bool fp8g = extra && extra->W_downT8;
  if (fp8g) {
    if (!extra->s_downT) return MOE_ERR_INVALID_ARG;
    st = check_fp8(cfg);
    if (st != MOE_OK) return st;
  }
  if (!backward_offsets_fit(d)) return MOE_ERR_UNSUPPORTED;
  Plan pl;
  const BackwardWs w = plan_backward(d, cfg->noisy, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = (int)d.E, h = (int)d.h, f = (int)d.f, T = (int)d.T, k = (int)d.k;
  const int ncu = device_cus();
  void* X = saved ? saved->X : at<void>(ws, w.X);
  void* A = saved ? saved->A : at<void>(ws, w.fb.ffn.A);
  void* GU = saved ? saved->GU : at<void>(ws, w.fb.GU);
  void* Y = saved ? saved->Y : at<void>(ws, w.Y);
  void* dY = at<void>(ws, w.dY);
  void* dX = at<void>(ws, w.dX);
  float* dgate = at<float>(ws, w.dgate);
  float* part = at<float>(ws, w.fb.ffn.part);
  // 1. the experts' activations: kept by the forward, or recomputed (X, then
  // A = SiLU(g) u with g, u kept, then Y)
  st = run_tile_map(d, w.fb.ffn, offset, ws, s);
  if (st != MOE_OK) return st;
  if (!saved) {
    MOE_TRY(launch_permute(U, slot, X, T, h, k, 1, s));
    st = run_ffn_recompute(d, w.fb, ws, X, offset, W_gate, W_up, GU, A, s);
    if (st != MOE_OK) return st;
    MOE_TRY(launch_down(w.fb.ffn.fs, A, offset, at<int32_t>(ws, w.fb.ffn.map2), W_down, Y, part,
                        E, h, f, 1, s));
  }
  // 2. combine: dY rows and the gates' gradient
  MOE_TRY(launch_combine_bwd(dOut, Y, slot, topk_gate, dY, dgate, T, h, k, s));
  // 3. the expert products backward (FP8 output gradients: quantised rows,
  // dequantised in place for every other use)
  Fp8Grad f8{};
  if (fp8g) {
    st = quantize_grad_rows(d, w.fb, ws, dY, s);
    if (st != MOE_OK) return st;
    f8 = Fp8Grad{at<void>(ws, w.fb.dY8), at<float>(ws, w.fb.sy), extra->W_downT8,
                 extra->s_downT};
  }
  st = run_ffn_backward(d, w.fb, ws, X, GU, A, dY, offset, W_gate, W_up, W_down, dX, dW_gate,
                        dW_up, dW_down, s, fp8g ? &f8 : nullptr);
  if (st != MOE_OK) return st;
  // 4. shared experts (every token, weight 1): recomputed g | u and a, then
  // the same products with offsets {0, T}
  const int ns = (int)d.ns, fsh = (int)d.fs;
  void* sdX = ns > 0 ? at<void>(ws, w.sdX) : nullptr;
  if (ns > 0) {  // with T = 0 the weight gradients come out zero
    int32_t* offs = at<int32_t>(ws, w.sh.offs);
    const int32_t* smap = at<int32_t>(ws, w.sh.map1);  // bm1 == bm2 for one expert of T rows
    MOE_TRY(launch_dense_offsets(T, offs, s));
    MOE_TRY(launch_tile_map(offs, 1, w.sh.fs.bm1, w.sh.fs.bm2, at<int32_t>(ws, w.sh.map1),
                            at<int32_t>(ws, w.sh.map2), s));
    void* sGU = at<void>(ws, w.sGU);
    void* sdA = at<void>(ws, w.sdA);
    void* sdGU = at<void>(ws, w.sdGU);
    const size_t fh = (size_t)fsh * h, tf = (size_t)T * fsh, th = (size_t)T * h;
    for (int i = 0; i < ns; ++i) {
      const char* Wsg = static_cast<const char*>(extra->Ws_gate) + i * fh * 2;
      const char* Wsu = static_cast<const char*>(extra->Ws_up) + i * fh * 2;
      const char* Wsd = static_cast<const char*>(extra->Ws_down) + i * fh * 2;
      char* sA = at<char>(ws, w.sh.A) + i * tf * 2;
      char* dXi = static_cast<char*>(sdX) + i * th * 2;
      MOE_TRY(launch_gate_up_save(w.sh.fs, U, offs, smap, Wsg, Wsu, sA, sGU, part, 1, h, fsh,
                                  s));
      MOE_TRY(launch_dgrad(w.shA, dOut, offs, smap, Wsd, Wsd, h, sdA, part, 1, fsh, h, s));
      MOE_TRY(launch_swiglu_bwd(sdA, sGU, offs, 1, T, fsh, sdGU, s));
      MOE_TRY(launch_dgrad(w.shX, sdGU, offs, smap, Wsg, Wsu, fsh, dXi, part, 1, h, 2 * fsh, s));
      MOE_TRY(launch_wgrad(dOut, h, sA, fsh, offs, static_cast<char*>(extra->dWs_down) + i * fh * 2,
                           1, h, fsh, T, ncu, s));
      MOE_TRY(launch_wgrad(sdGU, 2 * fsh, U, h, offs,
                           static_cast<char*>(extra->dWs_gate) + i * fh * 2, 1, fsh, h, T, ncu, s));
      MOE_TRY(launch_wgrad(static_cast<char*>(sdGU) + (size_t)fsh * 2, 2 * fsh, U, h, offs,
                           static_cast<char*>(extra->dWs_up) + i * fh * 2, 1, fsh, h, T, ncu, s));
    }
  }
  // 5. router: dH (and dZ for the noise term), then dU and dW_r, db_r (dW_noise)
  return run_router_backward(cfg, d, w.rb, ws, U, W_r, logits, topk_idx, topk_gate, slot, count,
                             dgate, dOut, dX, sdX, ns, alpha, c_z, extra, dU, dW_r, db_r, s);
}

int32_t moe_quantize_rows_fp8(const void* src, int64_t rows, int64_t cols, void* dst,
                              float* scale, void* stream) {
  if (rows < 0 || cols <= 0 || cols > (int64_t)1 << 30) return MOE_ERR_INVALID_ARG;
  if (cols % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows > 0 && (!src || !dst || !scale)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_rows_fp8(src, rows, (int)cols, dst, scale,
                                             static_cast<hipStream_t>(stream)));
}

int32_t moe_dispatch_fp8(const moe_config* cfg, const void* U, const int32_t* topk_idx,
                         void* X8, float* x_scale, int32_t* row_token, int32_t* slot,
                         int32_t* count, int32_t* kept, int32_t* offset, void* ws,
                         size_t ws_bytes, void* stream) {
  const int32_t st = check_fp8(cfg);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (d.T > 0 && (!U || !topk_idx || !X8 || !x_scale || !row_token || !slot))
    return MOE_ERR_INVALID_ARG;
  if (!count || !kept || !offset || !ws) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const DispatchWs w = plan_dispatch(d, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  return run_dispatch(d, cfg, w, U, topk_idx, X8, row_token, slot, count, kept, offset, ws,
                      static_cast<hipStream_t>(stream), x_scale);
}

int32_t moe_expert_ffn_fp8(const moe_config* cfg, const void* X8, const float* x_scale,
                           const int32_t* offset, const void* W8_gate, const float* s_gate,
                           const void* W8_up, const float* s_up, const void* W_down, void* Y,
                           void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_fp8(cfg);
  if (st != MOE_OK) return st;
  const Dims d = dims_of(cfg);
  if (!offset || !W8_gate || !s_gate || !W8_up || !s_up || !W_down || !ws)
    return MOE_ERR_INVALID_ARG;
  if (d.rows_max > 0 && (!X8 || !x_scale || !Y)) return MOE_ERR_INVALID_ARG;
  Plan pl;
  const FfnWs w = plan_ffn(d, pl);
  if (ws_bytes < pl.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_tile_map(d, w, offset, ws, s);
  if (st != MOE_OK) return st;
  const Fp8Up f8{W8_gate, s_gate, W8_up, s_up, x_scale};
  st = run_gate_up(d, w, X8, offset, W8_gate, W8_up, W_down, Y, ws, s, &f8);
  if (st != MOE_OK) return st;
  return run_down(d, w, offset, W_down, Y, ws, s);
}

}  // extern "C"
