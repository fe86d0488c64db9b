// Host-side launchers of the MoE kernels (internal interface of libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

// ---------------------------------------------------------------- router
struct RouteParams {
  int T, h, E, k;
  int score;  // 0 softmax, 1 sigmoid
  int gate;   // 0 raw, 1 renorm
  const void* U;
  const float* b_r;
  const float* b_sel;    // [E] selection-only bias, or NULL
  int n_groups;          // > 1: group-limited selection over n_groups groups
  int topk_groups;       // groups a token may use
  uint64_t seed;        // noisy routing: key of the draws' generator
  uint64_t rng_offset;  // ... and the counter of token 0, expert 0
  float* noise_out;     // optional [T][E]: the standard-normal draws used
  const void* W;     // W_r [h][E]; bf16: [h][Ew] (see RouteShape), 16-byte aligned
  const void* Wn;    // same for W_noise (noisy only)
  float* lpart;      // bf16: [1 + noisy][KS][T][EP] float32 products over the K ranges
  int32_t* topk_idx;
  float* topk_gate;
  float* logits;     // optional [T][E]
  double* prob_part; // [EP + 1][nblk] per-block sums of the score entering P;
                     // row EP: sum over the block's tokens of LSE(H_t)^2
  // bf16 path, optional: the dispatch histograms [k][nchunk][E] (kChunk-token
  // chunks), cleared by the logits kernel and counted by the selection kernel
  int32_t* hist = nullptr;
};

struct RouteShape {
  int EP;    // experts padded to 16 * NB (NB a power of two)
  int NB;
  int RB;    // tokens per selection workgroup (float32: per fused workgroup)
  int nblk;  // selection (float32: fused) workgroups
  // bf16 logits GEMM: BM-token x BN-expert tiles over KS ranges of K
  int Ew;    // row pitch of the weights it reads: E rounded up to 8
  int BM, BN, WM, KS, mblocks, nblocks;
};

RouteShape route_shape(int T, int E, int h, int bf16, int noisy);
// W [h][E] -> Wp [h][Ew], zero columns E..Ew-1 (bf16; for E % 8 != 0 or a
// W that is not 16-byte aligned).
hipError_t launch_pad_router_w(const void* W, void* Wp, int h, int E, int Ew, hipStream_t s);
hipError_t launch_route(const RouteShape& rs, const RouteParams& p, int bf16, int noisy,
                        hipStream_t s);
// bf16 only: the logits GEMM alone, part[ks][t][e] = the products of U and W
// ([h][rs.Ew], 16-byte aligned) over K range ks, for rs = route_shape(T, E,
// h, 1, 0) (the backward's recomputation of the noise term's Z = U W_noise).
hipError_t launch_route_products(const RouteShape& rs, const void* U, const void* W, float* part,
                                 int T, int h, hipStream_t s);
// total[e] (double, optional; E + 1 entries, the last the sum over tokens of
// LSE(H_t)^2) and prob_sum[e] (float, optional, E entries): sums over the
// router's per-workgroup partials.
hipError_t launch_prob_reduce(const double* part, int nblk, int EP, int E, double* total,
                              float* prob_sum, hipStream_t s);

// ---------------------------------------------------------------- yardstick
// One pass of 16-byte loads over bytes (a multiple of 16) of src; sink gets one
// word per workgroup (blocks of them).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s);

// ---------------------------------------------------------------- dispatch
constexpr int kChunk = 256;  // tokens per dispatch workgroup

struct StatsParams {
  int T, E, k;
  const int32_t* count;
  const int32_t* kept;
  const double* prob_total;  // [E + 1] (layer; entry E: sum of LSE^2) or NULL
  const float* prob_sum;     // [E] (standalone) or NULL
  float* f;
  float* P;
  float* aux;
  float* maxvio;
  int32_t* n_dropped;
  float* z_loss;             // mean over tokens of LSE^2 (needs prob_total), or NULL
};
struct DispatchParams {
  int T, E, k, C;
  int token_major;
  const int32_t* topk_idx;
  int32_t* hist;   // [k][nchunk][E]
  int32_t* base;   // [k][nchunk][E]
  int32_t* count;  // [E]
  int32_t* kept;   // [E]
  int32_t* offset; // [E+1]
  int32_t* slot;   // [T][k]
  int32_t* row_token;
  // Optional steps of the scan workgroup (the layer forward): the grouped
  // GEMMs' tile maps (map1 != NULL, tiles of bm1 and bm2 rows) and the load
  // statistics (stats_on, from count, kept and stats.prob_total).
  int bm1 = 0, bm2 = 0;
  int32_t* map1 = nullptr;
  int32_t* map2 = nullptr;
  int stats_on = 0;
  StatsParams stats{};
  // The layer forward: hist already holds the histograms (counted by the
  // selection kernel), and the scan launch's workgroups 1 .. E+1 also sum the
  // router's per-block P partials [prob_EP + 1][prob_nblk] into prob_total
  // (and prob_out, the E expert sums), the statistics then running in one
  // more workgroup of the assignment launch.
  int hist_ready = 0;
  const double* prob_part = nullptr;
  int prob_nblk = 0, prob_EP = 0;
  double* prob_total = nullptr;
  float* prob_out = nullptr;
};
hipError_t launch_dispatch(const DispatchParams& p, hipStream_t s);
// Bytes of the fixed device array behind moe_dispatch_noalloc, and its
// address on the current device (looked up once per device).
constexpr size_t kDispatchScratchBytes = size_t(4) << 20;
hipError_t dispatch_scratch(int32_t** out);
// FP8 dispatch (E4M3 codes of each kept row, with its power-of-two scale);
// bf16 U, h a multiple of 8.
hipError_t launch_permute_fp8(const void* U, const int32_t* slot, void* X8, float* xs, int T,
                              int h, int k, hipStream_t s);
// Row-wise E4M3 codes and power-of-two scales of a bf16 [rows][cols] matrix
// (cols a multiple of 8).
hipError_t launch_quantize_rows_fp8(const void* src, int64_t rows, int cols, void* dst,
                                    float* scale, hipStream_t s);
hipError_t launch_permute(const void* U, const int32_t* slot, void* X, int T, int h, int k,
                          int bf16, hipStream_t s);

// ---------------------------------------------------------------- experts
struct FfnShape {
  int bm1, bm2;     // row tile of the gate/up and the down GEMMs
  int nw1, nw2;     // waves per workgroup of each GEMM
  int mt1, mt2;     // static bound on m-tiles of each GEMM
  int nt1, nt2;     // n-tiles of each GEMM
  int grid1, grid2; // persistent workgroups launched (multiple of 8)
  int rows_cap;     // rows allocated in X and in the SwiGLU intermediate
  int split_max;    // most K chunks of a tail tile
  int part_slots;   // K-split partial tiles (256 x 256 float32 each), shared by the two GEMMs
  int gn1, gn2;     // n-tiles per group of each GEMM's tile numbering
  int wstream;      // 1: experts fit one m-tile (weight-streaming copy schedule)
};
constexpr size_t kPartSlotBytes = 256 * 256 * sizeof(float);
// ncu: compute units of the device (the persistent grid size)
FfnShape ffn_shape(int64_t rows_max, int E, int h, int f, int T, int k, int bf16, int ncu);
// Bytes of one GEMM's tile map: the E+1 first m-tiles of the experts padded
// to an even count, then {first row, expert | valid rows << 16} per m-tile
// (mt: the static bound on m-tiles).
inline size_t tile_map_bytes(int64_t E, int mt) {
  return (size_t)(((E + 2) & ~int64_t(1)) + 2 * (int64_t)mt) * sizeof(int32_t);
}
hipError_t launch_tile_map(const int32_t* offset, int E, int bm1, int bm2, int32_t* map1,
                           int32_t* map2, hipStream_t s);
// offset = {0, T}: all T rows as one expert (the shared experts' dense pass)
hipError_t launch_dense_offsets(int T, int32_t* offset, hipStream_t s);
// part: room for fs.part_slots K-split partial tiles (kPartSlotBytes each);
// each GEMM is followed by the reduction of its split tail tiles
hipError_t launch_gate_up(const FfnShape& fs, const void* X, const int32_t* offset,
                          const int32_t* map1, const void* Wg, const void* Wu, void* A,
                          float* part, int E, int h, int f, int bf16, hipStream_t s);
// The gate/up GEMM with FP8 (E4M3) operands: X8 [rows][h] codes with
// x_scale [rows], Wg8 / Wu8 [E][f][h] codes with s_gate / s_up [E][f]
// (power-of-two scales); h a multiple of 128.  Writes A [rows][f] bf16.
hipError_t launch_gate_up_fp8(const FfnShape& fs, const void* X8, const float* x_scale,
                              const int32_t* offset, const int32_t* map1, const void* Wg8,
                              const float* s_gate, const void* Wu8, const float* s_up, void* A,
                              float* part, int E, int h, int f, hipStream_t s);
// Row-grouped product with the weights stored [K][N]: C[rows][N] = A[rows][K]
// B_e with B_e rows 0..K0-1 from W0 [E][K0][N] and the rest from W1
// [E][K-K0][N] (K0 and K multiples of 64); tiles and grid of fs's second
// product (bm2, nt2 = N / 256 tiles, grid2).
hipError_t launch_dgrad(const FfnShape& fs, const void* A, const int32_t* offset,
                        const int32_t* map2, const void* W0, const void* W1, int K0, void* C,
                        float* part, int E, int N, int K, hipStream_t s);
hipError_t launch_down(const FfnShape& fs, const void* A, const int32_t* offset,
                       const int32_t* map2, const void* Wd, void* Y, float* part, int E, int h,
                       int f, int bf16, hipStream_t s);

// ---------------------------------------------------------------- combine, stats
// Ys: NULL or [ns][T][h] shared-expert outputs added to the residual
hipError_t launch_combine(const void* U, const void* Y, const int32_t* slot, const float* gate,
                          const void* Ys, int ns, void* out, int T, int h, int k, int bf16,
                          hipStream_t s);
// b[e] += gamma * sign(mean count - count[e])
hipError_t launch_update_bias(const int32_t* count, float* b, float gamma, int E, hipStream_t s);

hipError_t launch_stats(const StatsParams& p, hipStream_t s);
// z_loss[0] = mean over the T tokens of LSE(logits[t, :E])^2 (E <= 256).
hipError_t launch_z_loss(const float* logits, int T, int E, float* z_loss, hipStream_t s);

// ---------------------------------------------------------------- backward
// Gate/up GEMM that also stores the pre-activations g, u into GU [rows][2f].
hipError_t launch_gate_up_save(const FfnShape& fs, const void* X, const int32_t* offset,
                               const int32_t* map1, const void* Wg, const void* Wu, void* A,
                               void* GU, float* part, int E, int h, int f, hipStream_t s);
// Weight gradients: C_e[m][n] = sum over expert e's rows r (offset[e] ..
// offset[e+1]-1) of A[r][m] B[r][n], A [rows][lda] (columns 0..M-1) and B
// [rows][ldb] (columns 0..N-1) bf16 row-major; C [E][M][N].
// FP8 rows (codes, power-of-two row scales) back to bf16, exactly; cols a
// multiple of 8.
hipError_t launch_dequant_rows_fp8(const void* q, const float* scale, int64_t rows, int cols,
                                   void* out, hipStream_t s);
// FP8 product for the experts' backward: C[rows][N] = (A8 rows x sa) (W8_e rows
// x sw)^T with A8 [rows][K] and W8 [E][N][K] codes, sw [E][N]; tiles and grid
// of fs's second product.
hipError_t launch_dgrad_fp8(const FfnShape& fs, const void* A8, const float* sa,
                            const int32_t* offset, const int32_t* map2, const void* W8,
                            const float* sw, void* C, float* part, int E, int N, int K,
                            hipStream_t s);
// rows: a bound on the experts' rows in total; with at most 512 per expert on
// average (tiles of at most 8 K steps) the tiles run as one stream of K steps
// per workgroup (gemm_wgrad_stream_kernel).
hipError_t launch_wgrad(const void* A, int lda, const void* B, int ldb, const int32_t* offset,
                        void* C, int E, int M, int N, int64_t rows, int ncu, hipStream_t s);
hipError_t launch_combine_bwd(const void* dOut, const void* Y, const int32_t* slot,
                              const float* gate, void* dY, float* dgate, int T, int h, int k,
                              hipStream_t s);
hipError_t launch_swiglu_bwd(const void* dA, const void* GU, const int32_t* offset, int E,
                             int64_t rows_max, int f, void* dGU, hipStream_t s);
hipError_t launch_router_bwd(const float* logits, const int32_t* idx, const float* gate,
                             const float* dgate, const int32_t* count, int T, int E, int k,
                             int score, int renorm, float alpha, float c_z, float* dH,
                             hipStream_t s);
// dU = dOut + sum_r dX[slot] + dH W_r^T (+ dZ W_noise^T when dZ is set)
// (+ sum over the ns shared experts of dXs[i], dXs [ns][T][h]).
hipError_t launch_grad_input(const void* dOut, const void* dX, const int32_t* slot,
                             const float* dH, const void* W_r, const float* dZ,
                             const void* W_noise, const void* dXs, int ns, void* dU, int T, int h,
                             int E, int k, hipStream_t s);
// dZ = dH * noise * sigmoid(Z), [T][E] float32, with Z the sum over the KS
// ranges of zpart [KS][T][EP] (launch_route_products with W_noise).
hipError_t launch_noise_grad(const float* zpart, int KS, int EP, const float* dH, uint64_t seed,
                             uint64_t rng_offset, float* dZ, int T, int E, hipStream_t s);
// dW_r = U^T dH on MFMA (backward.hip): column tiles of tj, expert tiles of
// te (E padded to ep = et * te), token splits of tchunk (a multiple of 32)
// whose float32 partials [nsplit][h + 1][E] (row h: db_r) are summed in
// order; dH as bf16 hi | lo rows [T][2 ep] at hl_off.
struct DwrPlan {
  int te, tj, jt, et, ep, nsplit, tchunk;
  size_t hl_off, bytes;
};
inline DwrPlan dwr_plan(int64_t T, int h, int E) {
  DwrPlan p;
  p.te = E <= 16 ? 16 : E <= 32 ? 32 : E <= 64 ? 64 : 128;
  p.tj = p.te == 128 ? 128 : 256;
  p.jt = (h + p.tj - 1) / p.tj;
  p.et = (E + p.te - 1) / p.te;
  p.ep = p.et * p.te;
  const int64_t tiles = (int64_t)p.jt * p.et;
  const int64_t want = std::max<int64_t>(1, (256 + tiles - 1) / tiles);  // about 256 workgroups
  int64_t chunk = (T + want - 1) / want;
  chunk = std::max<int64_t>(32, (chunk + 31) / 32 * 32);
  // a split's byte offsets (chunk * h * 2 for U) stay below 2^30
  chunk = std::min<int64_t>(chunk, std::max<int64_t>(32, ((int64_t(1) << 29) / h) / 32 * 32));
  p.tchunk = (int)chunk;
  p.nsplit = T > 0 ? (int)((T + chunk - 1) / chunk) : 1;
  auto al = [](size_t n) { return (n + 255) & ~size_t(255); };
  p.hl_off = al((size_t)p.nsplit * (h + 1) * E * 4);
  p.bytes = p.hl_off + al((size_t)std::max<int64_t>(T, 1) * 2 * p.ep * 2);
  return p;
}
inline size_t dwr_part_bytes(int64_t T, int h, int E) { return dwr_plan(T, h, E).bytes; }
hipError_t launch_dwr(const void* U, const float* dH, float* dWr, float* db, void* ws, int T,
                      int h, int E, hipStream_t s);

}  // namespace moe
