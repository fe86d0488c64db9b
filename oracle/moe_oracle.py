"""Plain CPU oracle for the forward pass of one Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  This module is the independent definition that the
GPU path is checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does.
It shares no code, table or helper with the HIP library.

Everything is computed in float64 from the exact values of the inputs (bf16 or
fp32 inputs convert to float64 without rounding).  Loops are written the way the
method is stated, not the way a GPU would run it.  Library primitives used as
single steps: numpy matmul, exp/log1p, and a stable argsort.

Sources (all on the page "MoE 与专家并行", hs-black.github.io/posts/scaling-moe,
unless another page is named):
  * SwiGLU expert, section "从稠密 FFN 到 MoE", equation FFN(u).
  * Layer output with residual, same section, equation h'_t = u_t + sum g FFN.
  * Router logits H = U W_r, section "路由器：打分、top-k、加权求和".
  * Noisy top-k logits, same section, equation G(x) (Shazeer 2017); the
    standard-normal draws from Philox-4x64-10 (Salmon et al., SC'11) and the
    Box-Muller transform, one counter per (token, expert).
  * Scoring/gating variants, section "softmax 门控还是 sigmoid 门控", table.
  * Capacity C = ceil(CF * T * k / E) and token-order fill with drops,
    section "专家容量与丢 token", equation C and its figure; the GShard fill
    order (all first choices, then second choices) in the same section.
    The top-1 form ceil((T/E) * capacity_factor) is on the page
    "Ai大模型训练教程" (aissn.com/133.html), section on capacity and padding.
  * f_i, P_i and L_aux = alpha * E * sum f_i P_i, section
    "负载均衡辅助损失：推导与梯度"; for sigmoid scores P uses the scores
    normalised over all experts (same section, DeepSeek-V3 paragraph).
  * MaxVio, section "无辅助损失的负载均衡".
  * Selection-only expert bias b_i and its sign update (loss-free balancing),
    section "无辅助损失的负载均衡", equations g'_{i,t} and e_i, b_i.
  * Shared experts that every token passes through without the router,
    section "细粒度专家与共享专家", equation h'_t (DeepSeek-V3 form).
  * Group-limited (node-limited) selection, section "设备受限与节点受限路由".
  * Router z-loss L_z = (1/T) sum_t (log sum_j exp H_{t,j})^2 (ST-MoE),
    section "各家的变体", subsection "Router z-loss 与数值稳定", equation L_z.
  * Backward pass: the gradient reaching the gates is the inner product of
    the upstream gradient with the expert's output, carried on through the
    score function to the logits, W_r and u_t (section "路由器：打分、top-k、
    加权求和", equation dL/dg); the load-balance term's logit gradient
    (section "负载均衡辅助损失：推导与梯度", the equations for softmax and, with
    s' = s / sum s, for sigmoid scores); the expert products backward as
    grouped products for inputs and weights (section "专家计算：padding、
    block-sparse 与 grouped GEMM", last paragraph).
  * FP8 dispatch and FP8 up-projection with power-of-two scaling factors and
    a BF16 combine (DeepSeek-V3), section "低精度通信".  The FP8 format is OCP
    E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
    finite value 448), the one gfx950's FP8 matrix instructions read.

Readings where the pages are silent or ambiguous are listed in the design doc of the
repository; the ones that change arithmetic are restated next to the code.

Pins: every function here is pinned by tests/test_oracle_pins.py against the
pages' worked numbers, closed forms, special cases that reduce to library
routines, and brute force on tiny inputs.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

SOFTMAX = "softmax"
SIGMOID = "sigmoid"
GATE_RAW = "raw"          # g = s for the selected experts (Switch, DeepSeekMoE)
GATE_RENORM = "renorm"    # g = s / sum over selected s (GShard top-2, V3, Mixtral)
FILL_RANK_MAJOR = "rank_major"    # all first choices in token order, then all second ...
FILL_TOKEN_MAJOR = "token_major"  # token by token, each token's choices in rank order
CAP_ASSIGNMENTS = "assignments"   # C = ceil(CF * T * k / E)
CAP_TOKENS = "tokens"             # C = ceil((T / E) * CF)


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- router
def softplus(v: np.ndarray) -> np.ndarray:
    """log(1 + e^v), written in the overflow-free form log(e^0 + e^v)."""
    return np.logaddexp(0.0, v)


def router_logits(U, W_r, b_r=None, W_noise=None, noise=None) -> np.ndarray:
    """Routing logits H[t, i] for every token t and expert i.

    H = U W_r with W_r of shape [h, E] (router section, eq. H = U W_r).
    b_r, when given, is a per-expert bias added to every token's logits.
    W_noise/noise, when given, add the noisy top-k term
    noise[t, i] * softplus((U W_noise)[t, i]) (eq. G(x)); noise holds the
    standard-normal draws (philox_normals below gives the layer's).
    """
    U = f64(U)
    H = U @ f64(W_r)
    if b_r is not None:
        H = H + f64(b_r)[None, :]
    if W_noise is not None:
        if noise is None:
            raise ValueError("noisy routing needs the standard-normal draws")
        H = H + f64(noise) * softplus(U @ f64(W_noise))
    return H


# --------------------------------------------------------------------------- noise
# The noisy router's standard-normal draws (router section, eq. G(x): the
# N(0, 1) factor of each token's and expert's noise term).  The page leaves
# the generator open; here every (token t, expert i) pair has its own draw
# from a counter-based generator, so the draws do not depend on how the work
# is split.  Generator: Philox-4x64 with 10 rounds (Salmon, Moraes, Dror and
# Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), the 64-bit,
# four-word member of the Philox family, with its published multipliers and
# key increments.  Key (seed, 0); counter (t * E + i + rng_offset mod 2^64,
# 0, 0, 0).  Normal: the Box-Muller transform of two uniforms taken from the
# block's first two words, the first one in (0, 1] so its logarithm is finite.
PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)   # round multipliers
PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)   # key increments per round
PHILOX_ROUNDS = 10
_MASK64 = (1 << 64) - 1


def _mulhilo64(a: int, x: np.ndarray):
    """High and low 64-bit words of the 128-bit product a * x (x uint64 array).

    The product is formed from 32-bit halves, each partial product exact in
    uint64: a x = aH xH 2^64 + (aH xL + aL xH) 2^32 + aL xL.
    """
    m32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    aL, aH = np.uint64(a & 0xFFFFFFFF), np.uint64(a >> 32)
    xL, xH = x & m32, x >> s32
    ll, lh, hl, hh = aL * xL, aL * xH, aH * xL, aH * xH
    mid = (ll >> s32) + (lh & m32) + (hl & m32)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    lo = (mid << s32) | (ll & m32)
    return hi, lo


def philox4x64_10(counter, key):
    """Philox-4x64-10 blocks.  counter: four uint64 arrays (words 0..3, of one
    shape), key: two Python ints.  Returns the four output words.

    One round maps (x0, x1, x2, x3) under key (k0, k1) to
    (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)), where
    hi and lo are the two 64-bit halves of a 128-bit product; the key grows
    by (W0, W1) after every round.
    """
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in counter)
    k0, k1 = int(key[0]) & _MASK64, int(key[1]) & _MASK64
    for _ in range(PHILOX_ROUNDS):
        h0, l0 = _mulhilo64(PHILOX_M[0], x0)
        h1, l1 = _mulhilo64(PHILOX_M[1], x2)
        x0, x1, x2, x3 = h1 ^ x1 ^ np.uint64(k0), l1, h0 ^ x3 ^ np.uint64(k1), l0
        k0 = (k0 + PHILOX_W[0]) & _MASK64
        k1 = (k1 + PHILOX_W[1]) & _MASK64
    return x0, x1, x2, x3


def philox_normals(T: int, E: int, seed: int, rng_offset: int = 0) -> np.ndarray:
    """The standard-normal draw z[t, i] of every token t < T and expert i < E.

    Counter n = t * E + i + rng_offset (mod 2^64) in word 0, key (seed, 0).
    With w0, w1 the block's first two words: u1 = (floor(w0 / 2^11) + 1) 2^-53
    in (0, 1], u2 = floor(w1 / 2^11) 2^-53 in [0, 1), and
    z = sqrt(-2 ln u1) cos(2 pi u2) (Box-Muller).
    """
    n = (np.arange(T * E, dtype=np.uint64) + np.uint64(int(rng_offset) & _MASK64)).reshape(T, E)
    zero = np.zeros_like(n)
    w0, w1, _, _ = philox4x64_10((n, zero, zero, zero), (seed, 0))
    u1 = ((w0 >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (w1 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def scores(H, score: str) -> np.ndarray:
    """Affinities s[t, i]: softmax over the experts of each token, or sigmoid."""
    H = f64(H)
    if score == SOFTMAX:
        m = H.max(axis=1, keepdims=True)
        e = np.exp(H - m)
        return e / e.sum(axis=1, keepdims=True)
    if score == SIGMOID:
        return 1.0 / (1.0 + np.exp(-H))
    raise ValueError(score)


def select_topk(H, k: int) -> np.ndarray:
    """The k experts of each token, best first.

    Experts are ordered by the key (-H[t, i], i): larger logit first, and the
    lower expert index first among equal logits.  Softmax and sigmoid are
    strictly increasing, so this is the top-k of the scores in exact arithmetic.
    A stable argsort of -H realises exactly this key.
    """
    H = f64(H)
    order = np.argsort(-H, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def gates(s, idx, gate: str) -> np.ndarray:
    """Gate values of the selected experts, in rank order.

    RAW: g = s.  RENORM: g = s / sum of the selected s.  For softmax scores the
    renormalised gates equal a softmax over the selected logits, which is also
    Softmax(KeepTopK(H)) of the noisy router.
    """
    sel = np.take_along_axis(f64(s), np.asarray(idx), axis=1)
    if gate == GATE_RAW:
        return sel
    if gate == GATE_RENORM:
        return sel / sel.sum(axis=1, keepdims=True)
    raise ValueError(gate)


def selection_keys(s, b_sel=None) -> np.ndarray:
    """Keys that decide which experts a token takes: s[t, i] + b_i.

    Loss-free balancing adds a per-expert bias to the affinity for the top-k
    choice only; the gates keep using s (page section "无辅助损失的负载均衡").
    """
    s = f64(s)
    return s if b_sel is None else s + f64(b_sel)[None, :]


def group_limited_mask(keys, n_groups: int, topk_groups: int, per_group: int) -> np.ndarray:
    """Experts a token may choose under group-limited selection.

    The experts form n_groups equal groups of consecutive ids (the nodes of the
    node-limited routing).  A group scores the sum of its per_group highest
    keys; the topk_groups best groups are kept, the lower group first among
    equal scores; experts of the other groups are excluded (page section
    "设备受限与节点受限路由": nodes ranked by the sum of their top K_r / M
    affinities, at most M nodes per token).
    """
    keys = f64(keys)
    T, E = keys.shape
    assert E % n_groups == 0 and 1 <= topk_groups <= n_groups
    gsize = E // n_groups
    allowed = np.zeros((T, E), dtype=bool)
    for t in range(T):
        gscore = []
        for g in range(n_groups):
            members = np.sort(keys[t, g * gsize:(g + 1) * gsize])[::-1]
            gscore.append(float(members[:per_group].sum()))
        chosen = np.argsort(-np.asarray(gscore), kind="stable")[:topk_groups]
        for g in chosen:
            allowed[t, g * gsize:(g + 1) * gsize] = True
    return allowed


def select_topk_keys(keys, k: int, allowed=None) -> np.ndarray:
    """The k allowed experts with the largest keys, best first; lower index first on ties."""
    keys = f64(keys)
    if allowed is not None:
        keys = np.where(allowed, keys, -np.inf)
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def update_bias(b_sel, count, gamma: float) -> np.ndarray:
    """One step of the loss-free bias update.

    e_i = mean_j c_j - c_i and b_i <- b_i + gamma * sign(e_i): an overloaded
    expert's bias drops by gamma, an underloaded one's rises by gamma, an
    expert exactly at the mean keeps its bias (section "无辅助损失的负载均衡";
    V3 calls gamma the bias update speed).  count is the per-expert number of
    assignments of the batch.
    """
    c = f64(count)
    e = c.mean() - c
    return f64(b_sel) + gamma * np.sign(e)


# --------------------------------------------------------------------------- capacity
def capacity(T: int, E: int, k: int, capacity_factor: float,
             cap_mode: str = CAP_ASSIGNMENTS, min_capacity: int = 0) -> int:
    """Expert capacity C as an exact rational ceiling.

    ASSIGNMENTS: C = ceil(CF * T * k / E) (capacity section, eq. C).
    TOKENS:      C = ceil((T / E) * CF), the top-1 form of the training-course page.
    capacity_factor <= 0 means no capacity limit (dropless): C = T, which no
    expert can exceed because a token picks an expert at most once.
    The result is raised to min_capacity when that is larger.
    """
    if capacity_factor <= 0:
        return max(T, int(min_capacity))
    n = T * k if cap_mode == CAP_ASSIGNMENTS else T
    if cap_mode not in (CAP_ASSIGNMENTS, CAP_TOKENS):
        raise ValueError(cap_mode)
    C = math.ceil(Fraction(capacity_factor) * n / E)
    return max(C, int(min_capacity))


def fill(idx, E: int, C: int, order: str = FILL_RANK_MAJOR) -> dict:
    """Give every (token, rank) assignment its place in its expert's buffer.

    Assignments are visited one at a time in fill order; each takes the next
    free position of its expert; positions >= C are dropped (the token then
    passes only the residual for that expert).  Kept assignments of expert e
    occupy rows offset[e] .. offset[e] + kept[e] - 1 of the permuted matrix, in
    fill order.  Returns count (before the cut), kept, offset[E+1], slot[T, k]
    (row index, -1 when dropped), pos[T, k] and row_token[rows].
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    if order == FILL_RANK_MAJOR:
        visit = [(t, r) for r in range(k) for t in range(T)]
    elif order == FILL_TOKEN_MAJOR:
        visit = [(t, r) for t in range(T) for r in range(k)]
    else:
        raise ValueError(order)
    counter = [0] * E
    pos = np.full((T, k), -1, dtype=np.int64)
    for t, r in visit:
        e = int(idx[t, r])
        pos[t, r] = counter[e]
        counter[e] += 1
    count = np.array(counter, dtype=np.int64)
    kept = np.minimum(count, C)
    offset = np.zeros(E + 1, dtype=np.int64)
    offset[1:] = np.cumsum(kept)
    slot = np.full((T, k), -1, dtype=np.int64)
    row_token = np.full(int(offset[-1]), -1, dtype=np.int64)
    for t, r in visit:
        if pos[t, r] < C:
            row = int(offset[idx[t, r]] + pos[t, r])
            slot[t, r] = row
            row_token[row] = t
    return {"count": count, "kept": kept, "offset": offset, "slot": slot,
            "pos": pos, "row_token": row_token, "C": C}


# --------------------------------------------------------------------------- experts
def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v * sigmoid(v) = v / (1 + e^-v)."""
    v = f64(v)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu_expert(x, W_gate, W_up, W_down) -> np.ndarray:
    """FFN(u) = W_down (SiLU(W_gate u) * (W_up u)) for each row u of x.

    W_gate, W_up have shape [f, h] and W_down [h, f] (FFN equation), so for a
    row-major batch x [n, h] the products are x W_gate^T and a W_down^T.
    """
    x = f64(x)
    a = silu(x @ f64(W_gate).T) * (x @ f64(W_up).T)
    return a @ f64(W_down).T


# --------------------------------------------------------------------------- stats
def load_stats(s, idx, fill_result: dict, score: str) -> dict:
    """Load-balance statistics of one batch.

    count_e: assignments to expert e before the capacity cut.
    f_e = count_e / (T k): fraction of the T k assignments (sums to 1).
    P_e = mean over tokens of s_e (softmax), or of s_e / sum_j s_j (sigmoid).
    aux = E * sum_e f_e P_e (alpha = 1; a caller scales it).
    MaxVio = (max_e count_e - mean count) / mean count, mean = T k / E.
    n_dropped = sum_e (count_e - kept_e).
    """
    s = f64(s)
    T, k = np.asarray(idx).shape
    E = s.shape[1]
    count = fill_result["count"].astype(np.float64)
    f = count / (T * k)
    if score == SOFTMAX:
        st = s
    elif score == SIGMOID:
        st = s / s.sum(axis=1, keepdims=True)
    else:
        raise ValueError(score)
    prob_sum = st.sum(axis=0)
    P = prob_sum / T
    aux = E * float(np.sum(f * P))
    mean = T * k / E
    maxvio = (count.max() - mean) / mean
    n_dropped = int(np.sum(fill_result["count"] - fill_result["kept"]))
    return {"f": f, "P": P, "prob_sum": prob_sum, "aux": aux, "maxvio": float(maxvio),
            "n_dropped": n_dropped}


def router_z_loss(H) -> float:
    """Router z-loss: the mean over tokens of the squared log-sum-exp of the
    token's router logits, L_z = (1/T) sum_t (log sum_j exp H_{t,j})^2.

    H are the logits the scores are taken from (with the logit bias and the
    noise term when the router has them).  The log-sum-exp is evaluated as
    max_j H + log sum_j exp(H - max_j H), which is the same number without
    overflow.  T = 0 gives 0.
    """
    H = f64(H)
    if H.shape[0] == 0:
        return 0.0
    m = H.max(axis=1)
    lse = m + np.log(np.exp(H - m[:, None]).sum(axis=1))
    return float(np.mean(lse * lse))


# --------------------------------------------------------------------------- FP8
FP8_E4M3_MAX = 448.0


def fp8_e4m3_decode(code: int) -> float:
    """Value of an OCP E4M3 byte: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0.  Exponent field 0 holds the subnormals m/8 * 2^-6;
    the pattern S.1111.111 is NaN (the format has no infinities)."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def fp8_e4m3_round(x) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to the even mantissa, for
    |x| <= 448 (the caller scales into that range).  Between 2^p and 2^(p+1)
    the E4M3 values are spaced 2^(p-3) apart for p >= -6; below 2^-6 the
    subnormals are spaced 2^-9 apart."""
    x = f64(x)
    a = np.abs(x)
    if np.any(a > FP8_E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    _, p1 = np.frexp(np.where(a > 0, a, 1.0))       # a = m 2^p1, 0.5 <= m < 1: p = p1 - 1
    spacing = np.ldexp(1.0, np.maximum(p1 - 1, -6) - 3)
    return np.sign(x) * np.round(a / spacing) * spacing   # np.round: half to even


def fp8_row_scale(amax: float) -> float:
    """Power-of-two scaling factor of a row with largest magnitude amax: the
    smallest s = 2^j with amax / s <= 448 (1 for an all-zero row)."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    j = math.frexp(amax)[1] - 12                      # amax / 2^j >= 2048 > 448
    while amax / 2.0 ** j > FP8_E4M3_MAX:
        j += 1
    return 2.0 ** j


def quantize_rows_fp8(X):
    """Row-wise FP8 quantisation: s_r = fp8_row_scale(max_j |X[r, j]|) and
    q[r] = the E4M3 rounding of X[r] / s_r.  Returns (q, s); q * s[:, None]
    is the dequantised matrix."""
    X = f64(X)
    s = np.array([fp8_row_scale(np.abs(row).max() if row.size else 0.0) for row in X])
    q = np.stack([fp8_e4m3_round(row / sr) for row, sr in zip(X, s)]) if len(X) else X.copy()
    return q, s


def expert_outputs_fp8(Xq, xs, offset, Wq_gate, s_gate, Wq_up, s_up, W_down) -> np.ndarray:
    """Y rows with the up-projection in FP8: expert e computes
    a = SiLU((x_q s_x) (W_gate,q s_gate)^T) * ((x_q s_x) (W_up,q s_up)^T) from the
    dequantised values, then y = a W_down^T with the BF16 down weights."""
    X = f64(Xq) * f64(xs)[:, None]
    Wg = f64(Wq_gate) * f64(s_gate)[..., None]
    Wu = f64(Wq_up) * f64(s_up)[..., None]
    return expert_outputs(X, offset, Wg, Wu, W_down)


# --------------------------------------------------------------------------- backward
def dsilu(v: np.ndarray) -> np.ndarray:
    """d/dv (v sigmoid(v)) = sigmoid(v) (1 + v (1 - sigmoid(v)))."""
    sg = 1.0 / (1.0 + np.exp(-f64(v)))
    return sg * (1.0 + v * (1.0 - sg))


def aux_logit_grad(s, f, score: str) -> np.ndarray:
    """d/dH[t, k] of sum_i f_i P_i with f held constant (it has no gradient),
    times T: s_k (f_k - sum_i f_i s_i) for softmax scores, and
    s'_k (1 - s_k) (f_k - sum_i f_i s'_i) with s' = s / sum_j s for sigmoid
    scores.  The layer's aux = E sum f P and P averages over the T tokens, so
    its gradient is (E / T) times this."""
    s, f = f64(s), f64(f)
    if score == SOFTMAX:
        return s * (f[None, :] - (s * f[None, :]).sum(axis=1, keepdims=True))
    if score == SIGMOID:
        sp = s / s.sum(axis=1, keepdims=True)
        return sp * (1.0 - s) * (f[None, :] - (sp * f[None, :]).sum(axis=1, keepdims=True))
    raise ValueError(score)


def z_loss_logit_grad(H) -> np.ndarray:
    """dL_z/dH[t, k] = (2 / T) LSE(H_t) softmax(H_t)_k."""
    H = f64(H)
    T = H.shape[0]
    m = H.max(axis=1, keepdims=True)
    e = np.exp(H - m)
    lse = m[:, 0] + np.log(e.sum(axis=1))
    return 2.0 / T * lse[:, None] * e / e.sum(axis=1, keepdims=True)


def round_bf16(x) -> np.ndarray:
    """float32 values rounded to bfloat16 (8 significant bits), to nearest,
    ties to even, as float64."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def expert_backward(X, offset, W_gate, W_up, W_down, dY):
    """The experts' products backward for rows X of the experts in offset and
    their output gradients dY: a = SiLU(g) u with g = X W_gate^T, u = X W_up^T
    recomputed; dA = dY W_down, dg = dA u SiLU'(g), du = dA SiLU(g); returns
    dX = dg W_gate + du W_up and dW_gate = dg^T X, dW_up = du^T X,
    dW_down = dY^T a, expert by expert (zeros for an expert without rows)."""
    X, dY = f64(X), f64(dY)
    Wg, Wu, Wd = f64(W_gate), f64(W_up), f64(W_down)
    off = np.asarray(offset)
    dX = np.zeros(X.shape)
    dWg, dWu, dWd = np.zeros_like(Wg), np.zeros_like(Wu), np.zeros_like(Wd)
    for e in range(Wg.shape[0]):
        a, b = int(off[e]), int(off[e + 1])
        G, Up = X[a:b] @ Wg[e].T, X[a:b] @ Wu[e].T
        A = silu(G) * Up
        dA = dY[a:b] @ Wd[e]
        dWd[e] = dY[a:b].T @ A
        dG = dA * Up * dsilu(G)
        dUp = dA * silu(G)
        dWg[e] = dG.T @ X[a:b]
        dWu[e] = dUp.T @ X[a:b]
        dX[a:b] = dG @ Wg[e] + dUp @ Wu[e]
    return dX, dWg, dWu, dWd


def expert_backward_fp8(X, offset, W_gate, W_up, W_down, dYq, dY_scale):
    """expert_backward with the output gradients given as FP8 rows (codes dYq
    and power-of-two row scales, section "低精度通信": the activation
    gradients before the down-projection are quantised like the activations
    before the up-projection).  The experts use the dequantised rows
    dY = dYq * dY_scale throughout; the down-projection's input gradient
    dA = dY W_down[e] runs against W_down[e] quantised per output column (its
    transpose quantised row-wise), so each scale factors out of a dot
    product."""
    dY = f64(dYq) * f64(dY_scale)[:, None]
    Wd = f64(W_down)
    E, h, f = Wd.shape
    WdT = np.transpose(Wd, (0, 2, 1)).reshape(E * f, h)
    WdTq, sdT = quantize_rows_fp8(WdT)
    Wd_q = np.transpose((WdTq * sdT[:, None]).reshape(E, f, h), (0, 2, 1))
    # dA = dY W_down from the FP8 operands; dW_down = dY^T a does not involve
    # W_down
    return expert_backward(X, offset, W_gate, W_up, Wd_q, dY)


def layer_backward(U, W_r, W_gate, W_up, W_down, fwd: dict, dOut, *, score: str, gate: str,
                   alpha: float = 0.0, c_z: float = 0.0, W_noise=None, noise=None,
                   Ws_gate=None, Ws_up=None, Ws_down=None, fp8_down_grad: bool = False) -> dict:
    """Gradients of L = <dOut, out> + alpha * aux + c_z * L_z for the routing
    in fwd (a layer_forward result).  The top-k choice, the capacity cut and
    the load fractions f are piecewise constant and carry no gradient; a
    dropped assignment adds nothing to out, but its score still enters the
    renormalisation of the token's other gates.  Every expert product is
    recomputed from the inputs.  Returns dU, dW_r, db_r, dW_gate, dW_up,
    dW_down, and the intermediate dgate [T, k] and dH [T, E].

    Noisy routing (W_noise, noise): the logits' term noise * softplus(U W_noise)
    passes dH on through softplus' = sigmoid to W_noise and U (dW_noise).
    Shared experts (Ws_*): each adds SwiGLU(u) with weight 1 to every token,
    so its output gradient is dOut itself (dWs_gate, dWs_up, dWs_down).

    fp8_down_grad: the experts' output gradients dY, as the layer stores them
    (bf16), are quantised row-wise to FP8 before they reach the experts (as
    the activations are before the up-projection), and the experts work on
    the dequantised rows: the
    down-projection's input gradient dA = dY W_down against W_down quantised
    per output column (rows of W_down^T), and dW_down = dY^T a (see
    expert_backward_fp8).  Also returns dYq and dY_scale.
    """
    U, W_r, dOut = f64(U), f64(W_r), f64(dOut)
    Wg, Wu, Wd = f64(W_gate), f64(W_up), f64(W_down)
    T, h = U.shape
    E = W_r.shape[1]
    idx, g, slot = np.asarray(fwd["idx"]), f64(fwd["gate"]), np.asarray(fwd["slot"])
    off, row_token = np.asarray(fwd["offset"]), np.asarray(fwd["row_token"])
    k = idx.shape[1]
    rows = int(off[-1])
    # experts, recomputed
    X = U[row_token]
    Y = np.zeros((rows, h))
    dY = np.zeros((rows, h))
    dgate = np.zeros((T, k))
    G, Up = np.zeros((rows, Wg.shape[1])), np.zeros((rows, Wg.shape[1]))
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        G[a:b], Up[a:b] = X[a:b] @ Wg[e].T, X[a:b] @ Wu[e].T
        Y[a:b] = (silu(G[a:b]) * Up[a:b]) @ Wd[e].T
    # combine: out_t = u_t + sum_r g[t, r] Y[slot[t, r]]
    for t in range(T):
        for r in range(k):
            if slot[t, r] >= 0:
                dY[slot[t, r]] += g[t, r] * dOut[t]
                dgate[t, r] = dOut[t] @ Y[slot[t, r]]
    fp8 = {}
    if fp8_down_grad:
        # quantised as the layer stores dY: g dOut rounded to float32, then to
        # bf16 (the decision on each code is taken in the layer's precision)
        dYq, sy = quantize_rows_fp8(round_bf16(dY.astype(np.float32)))
        fp8 = {"dYq": dYq, "dY_scale": sy}
        dX, dWg, dWu, dWd = expert_backward_fp8(X, off, Wg, Wu, Wd, dYq, sy)
    else:
        dX, dWg, dWu, dWd = expert_backward(X, off, Wg, Wu, Wd, dY)
    dU = dOut.copy()
    for row in range(rows):
        dU[row_token[row]] += dX[row]
    # gates -> scores -> logits
    H = f64(fwd["logits"])
    s = scores(H, score)
    ds = np.zeros((T, E))
    for t in range(T):
        sel = idx[t]
        if gate == GATE_RAW:
            ds[t, sel] += dgate[t]
        elif gate == GATE_RENORM:
            S = s[t, sel].sum()
            ds[t, sel] += (dgate[t] - (dgate[t] * g[t]).sum()) / S
        else:
            raise ValueError(gate)
    if score == SOFTMAX:
        dH = s * (ds - (ds * s).sum(axis=1, keepdims=True))
    elif score == SIGMOID:
        dH = ds * s * (1.0 - s)
    else:
        raise ValueError(score)
    if alpha:
        dH += alpha * E / T * aux_logit_grad(s, fwd["f"], score)
    if c_z:
        dH += c_z * z_loss_logit_grad(H)
    dU += dH @ W_r.T
    out = {"dU": dU, "dW_r": U.T @ dH, "db_r": dH.sum(axis=0), "dW_gate": dWg, "dW_up": dWu,
           "dW_down": dWd, "dgate": dgate, "dH": dH, **fp8}
    if W_noise is not None:
        Wn = f64(W_noise)
        Z = U @ Wn
        dZ = dH * f64(noise) / (1.0 + np.exp(-Z))
        out["dW_noise"] = U.T @ dZ
        dU += dZ @ Wn.T
    if Ws_gate is not None:
        Sg, Su, Sd = f64(Ws_gate), f64(Ws_up), f64(Ws_down)
        out["dWs_gate"], out["dWs_up"] = np.zeros_like(Sg), np.zeros_like(Su)
        out["dWs_down"] = np.zeros_like(Sd)
        for i in range(Sg.shape[0]):
            G, Up = U @ Sg[i].T, U @ Su[i].T
            dA = dOut @ Sd[i]
            out["dWs_down"][i] = dOut.T @ (silu(G) * Up)
            dG = dA * Up * dsilu(G)
            dUp = dA * silu(G)
            out["dWs_gate"][i] = dG.T @ U
            out["dWs_up"][i] = dUp.T @ U
            dU += dG @ Sg[i] + dUp @ Su[i]
    return out


# --------------------------------------------------------------------------- layer
def route(H, k: int, score: str, gate: str, C: int, fill_order: str = FILL_RANK_MAJOR,
          b_sel=None, n_groups: int = 1, topk_groups: int = 1) -> dict:
    """All routing decisions from given logits: top-k, gates, fill and statistics.

    Without a selection bias and groups, the top-k is taken on the logits
    (select_topk).  With either, the choice is made on the keys s + b, among
    the experts of the chosen groups when n_groups > 1, each group scored by
    its k / topk_groups best keys; the gates still come from s.
    """
    H = f64(H)
    s = scores(H, score)
    if b_sel is None and n_groups <= 1:
        idx = select_topk(H, k)
    else:
        keys = selection_keys(s, b_sel)
        allowed = None
        if n_groups > 1:
            allowed = group_limited_mask(keys, n_groups, topk_groups, max(1, k // topk_groups))
        idx = select_topk_keys(keys, k, allowed)
    g = gates(s, idx, gate)
    fr = fill(idx, H.shape[1], C, fill_order)
    st = load_stats(s, idx, fr, score)
    st["z_loss"] = router_z_loss(H)
    out = {"logits": H, "s": s, "idx": idx, "gate": g}
    out.update(fr)
    out.update(st)
    return out


def combine(U, Y, slot, gate, Y_shared=None) -> np.ndarray:
    """out_t = u_t + sum over kept ranks r (in rank order) of g[t, r] * Y[slot[t, r]].

    Dropped assignments add nothing and the remaining gates are not rescaled;
    a token with every assignment dropped is returned as its residual u_t plus
    the shared experts' outputs Y_shared[s, t] (none when Y_shared is None).
    """
    out = f64(U).copy()
    if Y_shared is not None:
        for ys in f64(Y_shared):
            out += ys
    Y = f64(Y)
    slot = np.asarray(slot)
    g = f64(gate)
    for r in range(slot.shape[1]):
        m = slot[:, r] >= 0
        out[m] += g[m, r, None] * Y[slot[m, r]]
    return out


def expert_outputs(X, offset, W_gate, W_up, W_down) -> np.ndarray:
    """Y rows for the permuted matrix X: rows offset[e]..offset[e+1]-1 use expert e."""
    X = f64(X)
    Y = np.zeros((X.shape[0], np.asarray(W_down).shape[1]), dtype=np.float64)
    for e in range(len(offset) - 1):
        a, b = int(offset[e]), int(offset[e + 1])
        if b > a:
            Y[a:b] = swiglu_expert(X[a:b], W_gate[e], W_up[e], W_down[e])
    return Y


def shared_expert_outputs(U, Ws_gate, Ws_up, Ws_down) -> np.ndarray:
    """FFN^(s)_i(u_t) for every shared expert i and every token t: [N_s, T, h].

    Shared experts take every token with weight 1 and no router (section
    "细粒度专家与共享专家", equation h'_t).
    """
    U = f64(U)
    return np.stack([swiglu_expert(U, Ws_gate[i], Ws_up[i], Ws_down[i])
                     for i in range(np.asarray(Ws_gate).shape[0])])


def layer_forward(U, W_r, W_gate, W_up, W_down, *, k: int, score: str, gate: str,
                  capacity_factor: float, cap_mode: str = CAP_ASSIGNMENTS,
                  fill_order: str = FILL_RANK_MAJOR, min_capacity: int = 0,
                  b_r=None, W_noise=None, noise=None, logits=None, b_sel=None,
                  n_groups: int = 1, topk_groups: int = 1, Ws_gate=None, Ws_up=None,
                  Ws_down=None, fp8_up: bool = False) -> dict:
    """The whole layer for small inputs.

    logits, when given, replaces the router product (used to route from exactly
    the logits another implementation produced).  b_sel, n_groups/topk_groups
    and the shared-expert weights Ws_* add the DeepSeek-V3 parts.  fp8_up:
    the dispatched rows and the routed experts' W_gate and W_up are quantised
    row-wise to FP8 (quantize_rows_fp8) and the up-projection works on the
    dequantised values; the router, the residual, W_down, the shared experts
    and the combine keep the inputs' own values.
    """
    U = f64(U)
    T = U.shape[0]
    E = np.asarray(W_r).shape[1]
    H = router_logits(U, W_r, b_r, W_noise, noise) if logits is None else f64(logits)
    C = capacity(T, E, k, capacity_factor, cap_mode, min_capacity)
    r = route(H, k, score, gate, C, fill_order, b_sel, n_groups, topk_groups)
    X = U[r["row_token"]]
    if fp8_up:
        Xq, xs = quantize_rows_fp8(X)
        E_, f_, h_ = np.asarray(W_gate).shape
        Wgq, sg = quantize_rows_fp8(f64(W_gate).reshape(E_ * f_, h_))
        Wuq, su = quantize_rows_fp8(f64(W_up).reshape(E_ * f_, h_))
        Y = expert_outputs_fp8(Xq, xs, r["offset"], Wgq.reshape(E_, f_, h_), sg.reshape(E_, f_),
                               Wuq.reshape(E_, f_, h_), su.reshape(E_, f_), W_down)
        r["Xq"], r["x_scale"] = Xq, xs
    else:
        Y = expert_outputs(X, r["offset"], W_gate, W_up, W_down)
    r["X"] = X
    r["Y"] = Y
    r["Y_shared"] = None if Ws_gate is None else shared_expert_outputs(U, Ws_gate, Ws_up, Ws_down)
    r["out"] = combine(U, Y, r["slot"], r["gate"], r["Y_shared"])
    return r


def token_outputs(tokens, U, idx, slot, gate, expert_weights) -> np.ndarray:
    """out_t for a few tokens, one at a time.

    expert_weights(e) returns (W_gate[e], W_up[e], W_down[e]); only the experts
    the given tokens keep are requested.
    """
    U = f64(U)
    res = []
    for t in tokens:
        o = U[t].copy()
        for r in range(idx.shape[1]):
            if slot[t, r] >= 0:
                Wg, Wu, Wd = expert_weights(int(idx[t, r]))
                o += float(gate[t, r]) * swiglu_expert(U[t:t + 1], Wg, Wu, Wd)[0]
        res.append(o)
    return np.stack(res) if res else np.zeros((0, U.shape[1]))


def dense_masked_forward(U, W_gate, W_up, W_down, g_dense) -> np.ndarray:
    """The layer equation taken literally: every expert on every token.

    out_t = u_t + sum over all E experts of g_dense[t, e] * FFN_e(u_t), where
    g_dense holds the gate of a kept assignment and 0 elsewhere.  Only for tiny
    inputs; used to check the sparse path above by brute force.
    """
    U = f64(U)
    out = U.copy()
    for e in range(np.asarray(W_gate).shape[0]):
        out += f64(g_dense)[:, e:e + 1] * swiglu_expert(U, W_gate[e], W_up[e], W_down[e])
    return out
