/*
 * moe.h - C ABI of libmoe: the forward pass of one Mixture-of-Experts layer
 * on one gfx950 GPU (MI355X).
 *
 * The layer (page "MoE 与专家并行", hs-black.github.io/posts/scaling-moe):
 *   logits  H = U W_r (+ b_r) (+ z * softplus(U W_noise), z ~ N(0,1))
 *                      section "路由器：打分、top-k、加权求和", eq. H and G(x)
 *   scores  softmax or sigmoid; top-k; gates raw or renormalised
 *                      section "softmax 门控还是 sigmoid 门控", table
 *   capacity C and token-order fill with drops
 *                      section "专家容量与丢 token", eq. C and its figure
 *   experts FFN(u) = W_down (SiLU(W_gate u) * W_up u)
 *                      section "从稠密 FFN 到 MoE", eq. FFN
 *   output  out_t = u_t + sum_r g_{t,r} FFN_{e(t,r)}(u_t) over kept (t,r)
 *                      same section, eq. h'_t
 *   stats   f_e, P_e, aux = E sum f_e P_e, MaxVio
 *                      sections "负载均衡辅助损失：推导与梯度" and
 *                      "无辅助损失的负载均衡"
 * The staged calls follow the single-GPU dataflow of the router section
 * (route, group rows by expert, grouped FFN over per-expert counts, scatter
 * back) and the grouped-GEMM option of section "专家计算：padding、
 * block-sparse 与 grouped GEMM".
 *
 * Conventions for every call:
 *  - Data pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees or synchronises; all work is enqueued on `stream` (a
 *    hipStream_t; NULL is the default stream) and the buffers must stay valid
 *    until it has run.  There is no global state: calls are re-entrant.
 *  - Arguments are validated on the host before anything is launched; on any
 *    error nothing is enqueued.  MOE_ERR_INVALID_ARG: a bad value or a NULL
 *    required pointer.  MOE_ERR_UNSUPPORTED: a valid shape this library does
 *    not handle (see moe_config).  MOE_ERR_WORKSPACE: ws_bytes smaller than
 *    moe_workspace_size().  MOE_ERR_HIP: a launch failed (hipGetLastError).
 *  - Layouts are row-major in the pages' shapes.  U, X, Y, out: [rows, h].
 *    W_r, W_noise: [h, E].  W_gate, W_up: [E, f, h].  W_down: [E, h, f].
 *    These and the expert weights have element type cfg->dtype.  b_r, noise,
 *    logits, gates, prob_sum, f, P and the scalar statistics are float32.
 *    Expert ids, slots, counts and offsets are int32.
 *  - Variable-size outputs (X, Y, row_token) are sized by the static bound
 *    moe_max_rows(), so no host synchronisation is ever needed.
 *  - Results are deterministic: no floating-point atomics decide any value.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Scoring (section "softmax 门控还是 sigmoid 门控"). */
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

/* Gates: RAW g = s (Switch, DeepSeekMoE); RENORM g = s / sum of selected s
 * (GShard top-2, DeepSeek-V3; with softmax this equals Softmax(KeepTopK)). */
typedef enum { MOE_GATE_RAW = 0, MOE_GATE_RENORM = 1 } moe_gate;

/* Fill order of capacity slots.  RANK_MAJOR: every token's first choice in
 * token order, then every second choice, ... (the GShard order in section
 * "专家容量与丢 token").  TOKEN_MAJOR: token by token, choices in rank order. */
typedef enum { MOE_FILL_RANK_MAJOR = 0, MOE_FILL_TOKEN_MAJOR = 1 } moe_fill;

/* Capacity.  ASSIGNMENTS: C = ceil(CF * T * k / E) (eq. C of section
 * "专家容量与丢 token").  TOKENS: C = ceil((T / E) * CF), the top-1 form on the
 * page "Ai大模型训练教程" (aissn.com/133.html), capacity section. */
typedef enum { MOE_CAP_ASSIGNMENTS = 0, MOE_CAP_TOKENS = 1 } moe_cap;

typedef struct {
  int64_t T;      /* tokens on this GPU, >= 0                                  */
  int64_t h;      /* hidden size                                               */
  int64_t f;      /* expert intermediate size (d_e)                            */
  int64_t E;      /* experts, 1..256                                           */
  int64_t k;      /* experts per token, 1..min(E, 8)                           */
  int32_t dtype;  /* moe_dtype.  BF16 needs h % 64 == 0 and f % 64 == 0, one
                     expert matrix below 2 GiB (h * max(f, f_shared) * 2 < 2^31)
                     and h, f, f_shared below 2^22; F32 needs h % 4 == 0 and
                     f % 4 == 0 (else UNSUPPORTED)                             */
  int32_t score;  /* moe_score                                                 */
  int32_t gate;   /* moe_gate                                                  */
  int32_t cap_mode; /* moe_cap                                                 */
  int32_t fill;   /* moe_fill                                                  */
  int32_t noisy;  /* 1: add z * softplus(U W_noise) to the logits (z below)  */
  double capacity_factor; /* > 0, finite, in [1e-6, 1e6]; <= 0 means no limit
                             (dropless: C = T)                                 */
  int64_t min_capacity;   /* C is raised to at least this (0: no floor)        */
  /* DeepSeek-V3 parts (page "MoE 与专家并行"); all zero: a plain layer.      */
  int64_t n_groups;     /* group-limited selection (section "设备受限与节点受限路由"):
                           experts form n_groups equal groups of consecutive ids
                           and a token chooses only within its topk_groups best
                           groups.  0 or 1: no limit; else 2..64 dividing E     */
  int64_t topk_groups;  /* 1..min(n_groups, 8, k); a group scores the sum of its
                           k / topk_groups best selection keys; need
                           k <= topk_groups * (E / n_groups)                    */
  int64_t n_shared;     /* shared experts taking every token with weight 1
                           (section "细粒度专家与共享专家", eq. h'_t), 0..16      */
  int64_t f_shared;     /* their intermediate size (same divisibility as f)     */
  /* Noisy routing (noisy = 1; section "路由器：打分、top-k、加权求和", eq.
   * G(x)): the standard-normal factor z[t,i] of token t and expert i is drawn
   * by the library from a counter-based generator, Philox-4x64-10 (Salmon,
   * Moraes, Dror and Shaw, SC'11) with key (seed, 0) and counter
   * (t*E + i + rng_offset mod 2^64, 0, 0, 0), mapped to N(0,1) by the
   * Box-Muller transform of the block's first two words w0, w1:
   * u1 = (w0 >> 11) * 2^-53 + 2^-53, u2 = (w1 >> 11) * 2^-53,
   * z = sqrt(-2 ln u1) cos(2 pi u2), evaluated in double precision and rounded
   * to float32.  The same (seed, rng_offset) give the same draws on every
   * call and launch shape; a caller that wants fresh noise per step advances
   * rng_offset by at least T*E.  The backward draws them again from the
   * same fields, so it must get the forward's config.                       */
  uint64_t seed;
  uint64_t rng_offset;
} moe_config;

/* Optional outputs of moe_layer_forward.  Any NULL field is kept in the
 * workspace instead (or not produced).  Shapes as in the staged calls. */
typedef struct {
  int32_t* topk_idx;   /* [T, k] expert ids, best first                       */
  float* topk_gate;    /* [T, k] gates in the same order                      */
  float* logits;       /* [T, E] the float32 logits routing used              */
  int32_t* slot;       /* [T, k] row of the permuted matrix, -1 when dropped  */
  int32_t* row_token;  /* [rows_max] token of each permuted row               */
  int32_t* count;      /* [E] assignments before the capacity cut             */
  int32_t* kept;       /* [E] min(count, C)                                   */
  int32_t* offset;     /* [E+1] exclusive scan of kept                        */
  float* prob_sum;     /* [E] sum over tokens of the score used by P          */
  float* f;            /* [E] count / (T k)                                   */
  float* P;            /* [E] prob_sum / T                                    */
  float* aux_loss;     /* [1] E * sum f P (alpha = 1)                         */
  float* maxvio;       /* [1] (max count - T k / E) / (T k / E)               */
  int32_t* n_dropped;  /* [1] sum (count - kept)                              */
  void* X;             /* [rows_max, h] permuted expert inputs                */
  void* Y;             /* [rows_max, h] expert outputs                        */
  void* Y_shared;      /* [n_shared, T, h] shared-expert outputs              */
  float* z_loss;       /* [1] router z-loss: mean over tokens of the squared
                          log-sum-exp of the logits routing used (section
                          "各家的变体", "Router z-loss 与数值稳定", eq. L_z)   */
  void* GU;            /* [rows_max, 2f] bf16 gate and up pre-activations g, u
                          (g in columns 0..f-1, u in f..2f-1); bf16 layers
                          without FP8 only (else MOE_ERR_UNSUPPORTED)          */
  void* A;             /* [rows_max, f] SwiGLU products a = SiLU(g) u         */
  float* noise;        /* [T, E] the standard-normal draws z of a noisy layer
                          (see moe_config.seed); ignored when cfg->noisy = 0 */
} moe_aux_outputs;

/* Workspace sizes per entry point. */
typedef enum {
  MOE_WS_ROUTE = 0,
  MOE_WS_DISPATCH = 1,
  MOE_WS_EXPERT_FFN = 2,
  MOE_WS_LAYER = 3,
  MOE_WS_SHARED_FFN = 4,
  MOE_WS_BACKWARD = 5,
  MOE_WS_EXPERT_FFN_BACKWARD = 6,
  MOE_WS_ROUTER_BACKWARD = 7
} moe_ws_entry;

/* Stage boundaries recorded by moe_layer_forward when stage_events != NULL:
 * events[0] before the router ... events[MOE_NUM_STAGES] after the last stage;
 * a NULL entry leaves that boundary unrecorded.  The router's P sums and the
 * load statistics are computed inside the dispatch stage, so the stats stage
 * is empty. */
enum { MOE_NUM_STAGES = 6 }; /* route, dispatch, gate_up, down, combine, stats */

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int32_t status);

/* Measurement yardstick, not part of the layer: reads `bytes` bytes (a
 * multiple of 16) of device memory at src once with 16-byte loads and writes
 * one XOR word per workgroup to sink[0 .. blocks-1] (device), so that the
 * read rate of the HBM-bound workloads can be compared with a plain read
 * stream on the same device.  Errors: MOE_ERR_INVALID_ARG for a size not a
 * multiple of 16, blocks outside 1..2^20, or NULL pointers with bytes > 0. */
int32_t moe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                        void* stream);

/* Capacity C of cfg, on the host, as an exact rational ceiling (the double
 * capacity_factor is taken at its exact binary value).  Pure; no GPU use. */
int32_t moe_capacity(const moe_config* cfg, int64_t* C);

/* Static bound on kept assignments: min(T k, E min(C, T)).  Pure. */
int32_t moe_max_rows(const moe_config* cfg, int64_t* rows_max);

/* Bytes of device workspace that entry `entry` (moe_ws_entry) needs.  Pure. */
int32_t moe_workspace_size(const moe_config* cfg, int32_t entry, size_t* bytes);

/* Router: logits, scores, top-k and gates (router section; scoring table).
 *  U [T,h], W_r [h,E]: required.  b_r [E]: optional per-expert logit bias.
 *  b_sel [E]: optional selection-only bias (section "无辅助损失的负载均衡"):
 *  the top-k is taken on s + b_sel while the gates keep using s.
 *  W_noise [h,E]: required iff cfg->noisy; the logits then get
 *  z * softplus(U W_noise) with z drawn from cfg->seed and cfg->rng_offset
 *  (see moe_config).  noise_out [T,E]: optional output of those draws.
 *  topk_idx [T,k], topk_gate [T,k]: required outputs, rank order.  Selection
 *  is by the key (-H, expert index) on the float32 logits; with b_sel or
 *  cfg->n_groups > 1 by (-(s + b_sel), expert index) on float32 scores,
 *  within the chosen groups.
 *  logits [T,E]: optional output of exactly the logits used.
 *  prob_sum [E]: optional output of sum_t s (softmax) or sum_t s/sum_j s
 *  (sigmoid), the numerator of P.
 *  ws: MOE_WS_ROUTE bytes. */
int32_t moe_route(const moe_config* cfg, const void* U, const void* W_r, const float* b_r,
                  const float* b_sel, const void* W_noise, float* noise_out,
                  int32_t* topk_idx, float* topk_gate, float* logits, float* prob_sum,
                  void* ws, size_t ws_bytes, void* stream);

/* Dispatch: capacity cut and permutation (capacity section).
 *  topk_idx [T,k] in: expert ids (values outside [0,E) are undefined input).
 *  A token may name one expert at several ranks (each is one assignment,
 *  placed in fill order like any other).
 *  count [E], kept [E], offset [E+1], slot [T,k], row_token [rows_max]: outputs
 *  (count is before the cut; offset is the exclusive scan of kept; rows of
 *  expert e are offset[e]..offset[e+1]-1 in fill order).
 *  X [rows_max, h]: output, X[row] = U[row_token[row]]; rows beyond
 *  offset[E] are left untouched.  All outputs required.  ws: MOE_WS_DISPATCH. */
int32_t moe_dispatch(const moe_config* cfg, const void* U, const int32_t* topk_idx,
                     void* X, int32_t* row_token, int32_t* slot, int32_t* count,
                     int32_t* kept, int32_t* offset, void* ws, size_t ws_bytes,
                     void* stream);

/* moe_dispatch for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same outputs, bit for bit, with the histograms and scan bases in a fixed
 * 4 MiB device array of the library (one per GPU, held until the process
 * ends) instead of a caller workspace.  It calls no allocator.  Shapes whose
 * dispatch workspace (moe_workspace_size, MOE_WS_DISPATCH) exceeds 4 MiB,
 * i.e. roughly T * k * E > 2^27, return MOE_ERR_WORKSPACE before anything
 * is launched.  Every call on one GPU uses that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race and must
 * be ordered by the caller. */
int32_t moe_dispatch_noalloc(const moe_config* cfg, const void* U, const int32_t* topk_idx,
                             void* X, int32_t* row_token, int32_t* slot, int32_t* count,
                             int32_t* kept, int32_t* offset, void* stream);

/* Grouped SwiGLU experts (FFN eq.; grouped-GEMM option of the expert-compute
 * section): for every expert e and row r in offset[e]..offset[e+1]-1,
 * Y[r] = W_down[e] (SiLU(W_gate[e] X[r]) * W_up[e] X[r]).  Accumulation is
 * float32; the SiLU product is rounded to cfg->dtype before the down
 * projection.  Rows beyond offset[E] are left untouched.  ws: MOE_WS_EXPERT_FFN. */
int32_t moe_expert_ffn(const moe_config* cfg, const void* X, const int32_t* offset,
                       const void* W_gate, const void* W_up, const void* W_down, void* Y,
                       void* ws, size_t ws_bytes, void* stream);

/* Shared experts (section "细粒度专家与共享专家", eq. h'_t): for every shared
 * expert i and token t, Y_shared[i,t] = FFN^(s)_i(U[t]) with the SwiGLU of the
 * routed experts (f_shared wide).  Ws_gate, Ws_up [n_shared, f_shared, h],
 * Ws_down [n_shared, h, f_shared], Y_shared [n_shared, T, h] out.  Needs
 * cfg->n_shared > 0.  ws: MOE_WS_SHARED_FFN bytes. */
int32_t moe_shared_ffn(const moe_config* cfg, const void* U, const void* Ws_gate,
                       const void* Ws_up, const void* Ws_down, void* Y_shared, void* ws,
                       size_t ws_bytes, void* stream);

/* Combine with residual (eq. h'_t): out[t] = U[t] + sum over shared experts i
 * of Y_shared[i,t] + sum over r with slot[t,r] >= 0, in rank order, of
 * topk_gate[t,r] * Y[slot[t,r]].  Y_shared: NULL or [cfg->n_shared, T, h].
 * Float32 accumulation in that order; out has cfg->dtype and may not alias
 * U, Y or Y_shared. */
int32_t moe_combine(const moe_config* cfg, const void* U, const void* Y, const int32_t* slot,
                    const float* topk_gate, const void* Y_shared, void* out, void* stream);

/* Loss-free balancing bias step (section "无辅助损失的负载均衡", equations e_i
 * and b_i): with c = count [E] (assignments per expert, e.g. dispatch's
 * count) and its mean, b_sel[i] += gamma * sign(mean - c[i]) in place
 * (float32).  gamma finite and >= 0. */
int32_t moe_update_bias(const moe_config* cfg, const int32_t* count, float* b_sel, float gamma,
                        void* stream);

/* Load-balance statistics from dispatch counts and the router's prob_sum
 * (aux-loss section; MaxVio of the loss-free section).  count, kept,
 * prob_sum in; f [E], P [E], aux_loss [1], maxvio [1], n_dropped [1] out
 * (each output optional).  With T = 0 every output is 0. */
int32_t moe_stats(const moe_config* cfg, const int32_t* count, const int32_t* kept,
                  const float* prob_sum, float* f, float* P, float* aux_loss, float* maxvio,
                  int32_t* n_dropped, void* stream);

/* Router z-loss L_z = (1/T) sum_t (log sum_j exp logits[t,j])^2 of given
 * float32 logits [T, E] (page "MoE 与专家并行", section "各家的变体",
 * subsection "Router z-loss 与数值稳定", eq. L_z), written to z_loss[0] (device
 * float).  The layer computes the same number from its own logits without
 * materialising them (moe_aux_outputs.z_loss); this call serves the staged
 * path.  One workgroup, a fixed summation order (deterministic).  Errors:
 * MOE_ERR_INVALID_ARG for a NULL pointer (logits may be NULL when T = 0). */
int32_t moe_router_z_loss(const moe_config* cfg, const float* logits, float* z_loss,
                          void* stream);

/* The whole layer: route, dispatch, experts (and shared experts), combine,
 * statistics.
 *  b_r, b_sel, W_noise: as in moe_route (aux->noise receives the draws).
 *  Ws_gate, Ws_up, Ws_down:
 *  shared-expert weights as in moe_shared_ffn, required iff cfg->n_shared > 0;
 *  their products run in the gate_up and down stages.
 *  out [T,h] required.  aux: optional outputs (struct pointer may be NULL).
 *  stage_events: NULL, or MOE_NUM_STAGES + 1 hipEvent_t handles (each may be
 *  NULL) recorded on `stream` at the stage boundaries (for timing).  ws: MOE_WS_LAYER bytes. */
int32_t moe_layer_forward(const moe_config* cfg, const void* U, const void* W_r,
                          const float* b_r, const float* b_sel, const void* W_noise,
                          const void* W_gate, const void* W_up,
                          const void* W_down, const void* Ws_gate, const void* Ws_up,
                          const void* Ws_down, void* out, const moe_aux_outputs* aux,
                          void* const* stage_events, void* ws, size_t ws_bytes,
                          void* stream);

/* ---------------------------------------------------------------- backward
 * The parts of the backward that only some layers have (each group NULL when
 * the layer lacks the part):
 *  noisy routing (cfg->noisy): W_noise [h,E] as given to the forward;
 *  dW_noise [h,E] float32 out.  The logits' term z * softplus(U W_noise)
 *  passes the logit gradient on through softplus' = sigmoid (page
 *  "MoE 与专家并行", router section, eq. G(x)); z is drawn again from
 *  cfg->seed and cfg->rng_offset, which must be the forward's.
 *  shared experts (cfg->n_shared > 0): Ws_gate, Ws_up [n_shared,f_shared,h],
 *  Ws_down [n_shared,h,f_shared] as given to the forward; dWs_gate, dWs_up,
 *  dWs_down of the same shapes, bf16, out.  Each takes every token with
 *  weight 1 (section "细粒度专家与共享专家", eq. h'_t), so its output gradient
 *  is dOut itself.
 *  FP8 output gradients (section "低精度通信": the activation gradients
 *  before the down-projection are quantised like the activations before the
 *  up-projection): W_downT8 [E,f,h] E4M3 codes and s_downT [E,f] power-of-two
 *  scales of W_down transposed, quantised row-wise (moe_quantize_rows_fp8 on
 *  W_down^T, a one-time step); when set, the experts' output gradients are
 *  quantised row-wise to E4M3, dA = dY W_down runs on FP8 operands, and
 *  every other use of dY takes the dequantised rows.  Needs h a multiple of
 *  128 (else MOE_ERR_UNSUPPORTED). */
typedef struct {
  const void* W_noise;
  float* dW_noise;
  const void* Ws_gate;
  const void* Ws_up;
  const void* Ws_down;
  void* dWs_gate;
  void* dWs_up;
  void* dWs_down;
  const void* W_downT8;
  const float* s_downT;
} moe_backward_extras;

/* Gradients of L = <dOut, out> + alpha * aux_loss + c_z * z_loss with respect
 * to U, W_r, b_r, W_gate, W_up and W_down (and W_noise, the shared experts'
 * weights), for the routing a moe_layer_forward call chose (page
 * "MoE 与专家并行": the gates' gradient is the inner product of the upstream
 * gradient with the expert's output and flows on through the score function,
 * section "路由器：打分、top-k、加权求和", eq. dL/dg; the load-balance term's logit
 * gradient, section "负载均衡辅助损失：推导与梯度"; the z-loss's, section
 * "各家的变体"; the experts as grouped products for inputs and weights, section
 * "专家计算：padding、block-sparse 与 grouped GEMM").  The top-k choice, the
 * capacity cut and the load fractions f carry no gradient.
 *  Inputs: U, W_r, W_gate, W_up, W_down as given to the forward; from its
 *  outputs (moe_aux_outputs) logits [T,E], topk_idx, topk_gate, slot [T,k],
 *  count [E], offset [E+1]; dOut [T,h] the upstream gradient.  alpha and c_z
 *  scale aux_loss and z_loss (finite; 0 leaves a term out).
 *  saved: NULL, and the routed experts are recomputed from U with the
 *  forward's kernels (the same values bit for bit); or the forward's aux
 *  outputs with X, GU, A and Y all set (every other field is ignored), which
 *  the backward then reads instead (MOE_ERR_INVALID_ARG if one of the four is
 *  NULL).  Shared experts are always recomputed.
 *  extra: required (with every pointer of the part) for noisy layers and
 *  layers with shared experts, else may be NULL.
 *  Outputs: dU [T,h] and dW_gate, dW_up [E,f,h], dW_down [E,h,f] in bf16;
 *  dW_r [h,E] and db_r [E] (nullable) in float32.  The logits' gradient dH
 *  is float32; its products with W_r (into dU) and with U (dW_r) run on bf16
 *  matrix cores with dH as a bf16 pair hi + lo (about 2^-17 relative), summed
 *  in float32, as do the noise term's (dZ, dW_noise).
 *  Supported: cfg->dtype == MOE_BF16 (else MOE_ERR_UNSUPPORTED); the routing
 *  may come from a selection bias or groups.  One expert's rows (at most
 *  min(C, T); T for a shared expert), plus 192, times 2 max(2 f, h, 2 f_shared)
 *  bytes must stay below 2^31 (else MOE_ERR_UNSUPPORTED).
 *  ws: MOE_WS_BACKWARD bytes. */
int32_t moe_layer_backward(const moe_config* cfg, const void* U, const void* W_r,
                           const void* W_gate, const void* W_up, const void* W_down,
                           const float* logits, const int32_t* topk_idx, const float* topk_gate,
                           const int32_t* slot, const int32_t* count, const int32_t* offset,
                           const void* dOut, float alpha, float c_z, void* dU, float* dW_r,
                           float* db_r, void* dW_gate, void* dW_up, void* dW_down,
                           const moe_aux_outputs* saved, const moe_backward_extras* extra,
                           void* ws, size_t ws_bytes, void* stream);

/* Staged backward: the three parts of moe_layer_backward as separate calls
 * (for instance with the expert rows exchanged between GPUs in between).
 * Run in this order they give exactly the layer call's results.  bf16 only
 * (else MOE_ERR_UNSUPPORTED).
 *
 * moe_combine_backward: through the weighted sum (page "MoE 与专家并行",
 * section "路由器：打分、top-k、加权求和", eq. dL/dg): dY[slot[t,r]] =
 * topk_gate[t,r] dOut_t for every kept rank (rows of dY that no token keeps
 * are left untouched) and dgate[t,r] = dOut_t . Y[slot[t,r]] (0 when
 * dropped).  dOut [T,h], Y and dY [rows_max,h] bf16; slot, topk_gate [T,k];
 * dgate [T,k] float32.  No workspace. */
int32_t moe_combine_backward(const moe_config* cfg, const void* dOut, const void* Y,
                             const int32_t* slot, const float* topk_gate, void* dY, float* dgate,
                             void* stream);

/* moe_expert_ffn_backward: the experts' grouped products backward (section
 * "专家计算：padding、block-sparse 与 grouped GEMM") for the rows X [rows_max,h]
 * of offset [E+1] and their output gradients dY [rows_max,h]: dX [rows_max,h]
 * (rows past offset[E] untouched), dW_gate, dW_up [E,f,h], dW_down [E,h,f]
 * (an expert without rows gets zeros), all bf16.  GU [rows_max,2f] and A
 * [rows_max,f]: the forward's kept g | u and a (moe_aux_outputs), or both
 * NULL to recompute them from X.  A shared expert is one expert of all T
 * rows: cfg with E = k = 1 and a capacity of T, X = U, offset {0, T},
 * dY = dOut.  Errors as moe_layer_backward.  ws: MOE_WS_EXPERT_FFN_BACKWARD. */
int32_t moe_expert_ffn_backward(const moe_config* cfg, const void* X, const int32_t* offset,
                                const void* W_gate, const void* W_up, const void* W_down,
                                const void* dY, const void* GU, const void* A, void* dX,
                                void* dW_gate, void* dW_up, void* dW_down, void* ws,
                                size_t ws_bytes, void* stream);

/* The same with the output gradients as FP8 rows (section "低精度通信"): dY8
 * [rows_max,h] E4M3 codes and dY_scale [rows_max] power-of-two row scales
 * (moe_quantize_rows_fp8 of the dY rows), W_downT8 / s_downT as in
 * moe_backward_extras.  dA = dY W_down runs on the FP8 operands; dW_down and
 * the rest use the dequantised rows.  Needs h a multiple of 128 (else
 * MOE_ERR_UNSUPPORTED).  ws: MOE_WS_EXPERT_FFN_BACKWARD. */
int32_t moe_expert_ffn_backward_fp8(const moe_config* cfg, const void* X, const int32_t* offset,
                                    const void* W_gate, const void* W_up, const void* W_downT8,
                                    const float* s_downT, const void* dY8,
                                    const float* dY_scale, const void* GU, const void* A,
                                    void* dX, void* dW_gate, void* dW_up, void* dW_down,
                                    void* ws, size_t ws_bytes, void* stream);

/* moe_router_backward: from the gates' gradient dgate [T,k] to the logits
 * (scores, renormalisation, plus alpha times the load-balance term and c_z
 * times the z-loss term, as in moe_layer_backward) and on to
 * dU = dOut + sum over kept ranks of dX[slot] + dH W_r^T, dW_r = U^T dH and
 * db_r (nullable) = column sums of dH.  dOut is the gradient that reaches u_t
 * directly (the residual; add the shared experts' input gradients to it);
 * dX [rows_max,h] the experts' input gradients.  extra: the noise part
 * (W_noise, dW_noise) for noisy layers.  ws: MOE_WS_ROUTER_BACKWARD.  The
 * products with dH run as in moe_layer_backward (bf16 hi + lo pair). */
int32_t moe_router_backward(const moe_config* cfg, const void* U, const void* W_r,
                            const float* logits, const int32_t* topk_idx, const float* topk_gate,
                            const int32_t* slot, const int32_t* count, const float* dgate,
                            const void* dOut, const void* dX, float alpha, float c_z,
                            const moe_backward_extras* extra, void* dU, float* dW_r,
                            float* db_r, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- FP8
 * FP8 dispatch and FP8 up-projection (page "MoE 与专家并行", section
 * "低精度通信": DeepSeek-V3 quantises the activations before the MoE
 * up-projection to FP8 with power-of-two scaling factors, dispatches them at
 * one byte per element, runs the up-projection in FP8 and keeps the combine
 * in BF16).  Format: OCP E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; largest finite value 448).  Row-wise scales: a row with largest
 * magnitude amax gets s = 2^j, j the smallest integer with amax / s <= 448
 * (s = 1 for an all-zero row), and its codes are x / s rounded to the nearest
 * E4M3 value, ties to even.  Only the routed experts' gate and up products
 * run on FP8; the router, the residual, W_down, the shared experts and the
 * combine keep the bf16 inputs.  Requirements of the calls below (else
 * MOE_ERR_UNSUPPORTED): cfg->dtype == MOE_BF16 and h a multiple of 128. */

/* Row-wise E4M3 codes of a bf16 matrix src [rows, cols] (device), into dst
 * [rows, cols] bytes and scale [rows] float32 (device, caller-owned), e.g.
 * the expert weights W_gate or W_up viewed as [E*f, h] (done once, outside
 * the forward).  cols a multiple of 8 (else MOE_ERR_UNSUPPORTED); NULL
 * pointers with rows > 0 or cols <= 0: MOE_ERR_INVALID_ARG. */
int32_t moe_quantize_rows_fp8(const void* src, int64_t rows, int64_t cols, void* dst,
                              float* scale, void* stream);

/* moe_dispatch with the permuted rows in FP8: X8 [rows_max, h] bytes of E4M3
 * codes and x_scale [rows_max] float32, the scale of each row's token (the
 * other outputs as in moe_dispatch).  ws: MOE_WS_DISPATCH bytes. */
int32_t moe_dispatch_fp8(const moe_config* cfg, const void* U, const int32_t* topk_idx,
                         void* X8, float* x_scale, int32_t* row_token, int32_t* slot,
                         int32_t* count, int32_t* kept, int32_t* offset, void* ws,
                         size_t ws_bytes, void* stream);

/* moe_expert_ffn with the up-projection on FP8: X8, x_scale from
 * moe_dispatch_fp8; W8_gate, W8_up [E, f, h] E4M3 codes with s_gate, s_up
 * [E, f] row scales (moe_quantize_rows_fp8 of W_gate, W_up); W_down [E, h, f]
 * bf16.  a = SiLU(g) * u with g = sum_k X8[r,k] x_scale[r] W8_gate[e,n,k]
 * s_gate[e,n] (float32 accumulation), rounded to bf16; Y as in
 * moe_expert_ffn.  ws: MOE_WS_EXPERT_FFN bytes. */
int32_t moe_expert_ffn_fp8(const moe_config* cfg, const void* X8, const float* x_scale,
                           const int32_t* offset, const void* W8_gate, const float* s_gate,
                           const void* W8_up, const float* s_up, const void* W_down, void* Y,
                           void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward with the FP8 dispatch and up-projection: W8_gate, s_gate,
 * W8_up, s_up as in moe_expert_ffn_fp8 replace W_gate and W_up; every other
 * argument as in moe_layer_forward, except that aux->X is not written (the
 * FP8 rows stay in the workspace; moe_dispatch_fp8 returns them).
 * ws: MOE_WS_LAYER bytes. */
int32_t moe_layer_forward_fp8(const moe_config* cfg, const void* U, const void* W_r,
                              const float* b_r, const float* b_sel, const void* W_noise,
                              const void* W8_gate, const float* s_gate,
                              const void* W8_up, const float* s_up, const void* W_down,
                              const void* Ws_gate, const void* Ws_up, const void* Ws_down,
                              void* out, const moe_aux_outputs* aux, void* const* stage_events,
                              void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
