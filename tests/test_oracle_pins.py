"""Pins of the CPU oracle to facts fixed outside it.

Each test ties one oracle function to something other than the oracle itself:
numbers printed on the pages (tests/golden, each with its citation), closed
forms, special cases that reduce to a library routine (torch in float64), or
brute force on tiny inputs.  The oracle's own formulas are never retyped here.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- printed examples
def test_renorm_figure_direct():
    g = golden("renorm_figure.json")
    s = np.array([[0.80, 0.49, 0.10, 0.05, 0.20, 0.01, 0.30, 0.02]])
    idx = O.select_topk(np.log(s), 2)
    assert idx.tolist() == [[0, 1]]
    gates = O.gates(s, idx, O.GATE_RENORM)
    np.testing.assert_allclose(np.round(gates[0], g["printed_decimals"]), g["gates"])
    assert abs(gates.sum() - 1.0) < 1e-15


def test_renorm_figure_through_sigmoid_router():
    # Logits whose sigmoid is exactly the printed scores: ln(0.8/0.2), ln(0.49/0.51).
    g = golden("renorm_figure.json")
    H = np.full((1, 8), -3.0)
    H[0, 3] = math.log(4.0)
    H[0, 6] = math.log(49.0 / 51.0)
    r = O.route(H, 2, O.SIGMOID, O.GATE_RENORM, C=1)
    assert r["idx"].tolist() == [[3, 6]]
    np.testing.assert_allclose(r["s"][0, [3, 6]], g["selected_scores"], rtol=1e-14)
    np.testing.assert_allclose(np.round(r["gate"][0], 2), g["gates"])


def test_renorm_figure_through_softmax_router():
    # softmax + renorm depends only on the gap of the two selected logits.
    g = golden("renorm_figure.json")
    a = 0.3
    H = np.array([[a - 5, a, a - 4, a - math.log(0.80 / 0.49), a - 6, a - 7, a - 3, a - 2]])
    r = O.route(H, 2, O.SOFTMAX, O.GATE_RENORM, C=1)
    assert r["idx"].tolist() == [[1, 3]]
    np.testing.assert_allclose(r["gate"][0], [0.80 / 1.29, 0.49 / 1.29], rtol=1e-14)
    np.testing.assert_allclose(np.round(r["gate"][0], 2), g["gates"])


def test_capacity_worked_numbers():
    g = golden("capacity_examples.json")
    fig, w = g["figure"], g["worked"]
    assert O.capacity(fig["T"], fig["E"], fig["k"], fig["capacity_factor"]) == fig["C"]
    C = O.capacity(w["T"], w["E"], w["k"], w["capacity_factor"])
    assert C == w["C"]
    assert w["T"] * w["k"] // w["E"] == w["balanced"]
    assert w["hot_load"] - C == w["hot_dropped"]
    assert C - w["cold_load"] == w["cold_idle"]
    # the top-1 form ceil((T/E) * CF) agrees with the assignments form at k = 1
    for T, E, cf in [(12, 4, 1.0), (8192, 128, 1.25), (1000, 7, 1.1), (5, 3, 0.3)]:
        assert O.capacity(T, E, 1, cf, O.CAP_TOKENS) == O.capacity(T, E, 1, cf)
    # and differs from it at k > 1, as the two readings predict (640 vs 80)
    assert O.capacity(4096, 64, 8, 1.25, O.CAP_TOKENS) == 80


def test_capacity_exact_ceiling_and_floor():
    # exact rational ceiling: 1.25 * 8 * 2 / 8 = 2.5 -> 3; 1.25 * 16 / 8 = 2.5 -> 3
    assert O.capacity(8, 8, 2, 1.25) == 3
    assert O.capacity(16, 8, 1, 1.25) == 3
    assert O.capacity(64, 8, 1, 1.0) == 8          # exact integer stays
    assert O.capacity(10, 3, 1, 0.1) == 1          # the double 0.1 is just above 1/10
    assert Fraction(0.1) > Fraction(1, 10)
    assert O.capacity(10, 3, 1, 0.1, min_capacity=4) == 4
    assert O.capacity(100, 4, 2, 0.0) == 100       # dropless: nothing can exceed T
    assert O.capacity(256, 8, 2, 1.25) == 80
    assert O.capacity(4096, 256, 8, 2.0) == 256
    assert O.capacity(32768, 64, 2, 1.0) == 1024


def test_capacity_figure_fill():
    # Rebuild the figure's case with loads (5, 3, 3, 1) over 12 tokens in an
    # interleaved token order; capacity 3.  The two dropped tokens must be the
    # last two that chose expert 1 (index 0 here), in token order.
    g = golden("capacity_examples.json")["figure"]
    choice = [0, 1, 0, 2, 1, 0, 3, 2, 0, 1, 2, 0]
    idx = np.array(choice)[:, None]
    C = O.capacity(g["T"], g["E"], g["k"], g["capacity_factor"])
    fr = O.fill(idx, g["E"], C)
    assert fr["count"].tolist() == [5, 3, 3, 1]
    assert fr["count"][0] == g["printed_loads"]["1"]
    assert fr["count"][3] == g["printed_loads"]["4"]
    dropped = [t for t in range(12) if fr["slot"][t, 0] < 0]
    assert dropped == [8, 11]
    assert len(dropped) == g["printed_dropped"]["1"]
    assert C - fr["kept"][3] == g["printed_padding"]["4"]
    assert fr["kept"].tolist() == [3, 3, 3, 1]
    assert fr["offset"].tolist() == [0, 3, 6, 9, 10]
    # expert 0's kept rows are tokens 0, 2, 5 in that order
    assert fr["row_token"][:3].tolist() == [0, 2, 5]


def test_zloss_bf16_example():
    g = golden("zloss_bf16_softmax.json")
    H = np.array([g["logits"]], dtype=np.float32)
    s32 = O.scores(H, O.SOFTMAX)[0, 0]
    assert round(s32, g["printed_decimals"]) == g["softmax_first_fp32_logits"]
    assert abs(s32 - 1.0 / (1.0 + 10.0 * math.exp(-0.5))) < 1e-14
    Hb = torch.tensor(g["logits"]).to(torch.bfloat16).double().numpy()[None, :]
    sb = O.scores(Hb, O.SOFTMAX)[0, 0]
    assert round(sb, g["printed_decimals"]) == g["softmax_first_bf16_logits"]
    assert abs(sb - 1.0 / 11.0) < 1e-15


def test_router_z_loss_closed_forms():
    # equal logits c over E experts: log-sum-exp = c + log E
    for E, c in ((8, 0.0), (64, -3.25), (256, 17.5)):
        H = np.full((5, E), c)
        assert abs(O.router_z_loss(H) - (c + math.log(E)) ** 2) < 1e-12 * max(1.0, (c + math.log(E)) ** 2)
    # logits (0, log 3): log-sum-exp = log 4 exactly
    H = np.array([[0.0, math.log(3.0)]])
    assert abs(O.router_z_loss(H) - math.log(4.0) ** 2) < 1e-15
    # the mean over tokens: two tokens with log-sum-exp 1 and 3 give (1 + 9) / 2
    H = np.array([[1.0 - math.log(2.0), 1.0 - math.log(2.0)], [3.0, -np.inf]])
    assert abs(O.router_z_loss(H) - 5.0) < 1e-14
    # huge logits: no overflow, the shift comes out exactly
    H = np.array([[1000.0, 1000.0, 1000.0, 1000.0]])
    assert abs(O.router_z_loss(H) - (1000.0 + math.log(4.0)) ** 2) < 1e-9
    assert O.router_z_loss(np.zeros((0, 4))) == 0.0


def test_router_z_loss_gradient_matches_page():
    # the page gives dL_z/dH_{t,k} = (2/T) LSE(H_t) softmax(H_t)_k; central
    # differences of the oracle's L_z must reproduce it
    r = rng(7)
    H = r.normal(0.0, 2.0, size=(3, 6))
    T = H.shape[0]
    lse = np.log(np.exp(H).sum(axis=1))
    sm = np.exp(H - lse[:, None])
    want = 2.0 / T * lse[:, None] * sm
    eps = 1e-6
    got = np.zeros_like(H)
    for t in range(H.shape[0]):
        for j in range(H.shape[1]):
            Hp = H.copy(); Hp[t, j] += eps
            Hm = H.copy(); Hm[t, j] -= eps
            got[t, j] = (O.router_z_loss(Hp) - O.router_z_loss(Hm)) / (2 * eps)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-9)


# ----------------------------------------------------------------- selection
def test_topk_ties_lower_index_wins():
    H = np.zeros((5, 8))
    idx = O.select_topk(H, 3)
    assert (idx == np.array([0, 1, 2])).all()
    s = O.scores(H, O.SOFTMAX)
    np.testing.assert_allclose(O.gates(s, idx, O.GATE_RENORM), 1.0 / 3, rtol=1e-15)
    np.testing.assert_allclose(O.gates(s, idx, O.GATE_RAW), 1.0 / 8, rtol=1e-15)
    # partial tie: the two equal best logits keep index order
    H = np.array([[0.5, 2.0, 1.0, 2.0]])
    assert O.select_topk(H, 3).tolist() == [[1, 3, 2]]


def test_topk_matches_python_sorted_and_torch():
    r = rng(1)
    H = np.round(r.normal(size=(50, 13)), 1)   # rounding creates many ties
    idx = O.select_topk(H, 4)
    for t in range(H.shape[0]):
        ref = sorted(range(13), key=lambda i: (-H[t, i], i))[:4]
        assert idx[t].tolist() == ref
    vals = torch.topk(torch.from_numpy(H), 4, dim=1).values.numpy()
    np.testing.assert_array_equal(np.take_along_axis(H, idx, 1), vals)


def test_renorm_identity_topk_then_softmax():
    # softmax -> renormalise over the selected == softmax of the selected logits
    r = rng(2)
    H = r.normal(size=(40, 16)) * 3
    idx = O.select_topk(H, 4)
    g = O.gates(O.scores(H, O.SOFTMAX), idx, O.GATE_RENORM)
    ref = torch.softmax(torch.from_numpy(np.take_along_axis(H, idx, 1)), dim=1).numpy()
    np.testing.assert_allclose(g, ref, rtol=1e-13)


def test_scores_vs_library():
    r = rng(3)
    H = r.normal(size=(20, 9)) * 4
    np.testing.assert_allclose(O.scores(H, O.SOFTMAX),
                               torch.softmax(torch.from_numpy(H), 1).numpy(), rtol=1e-13)
    np.testing.assert_allclose(O.scores(H, O.SIGMOID),
                               torch.sigmoid(torch.from_numpy(H)).numpy(), rtol=1e-13)
    # very large logits must not overflow (softmax is shift invariant)
    Hbig = np.array([[800.0, 799.0, -800.0], [1e3, 1e3, 1e3]])
    np.testing.assert_allclose(O.scores(Hbig, O.SOFTMAX),
                               torch.softmax(torch.from_numpy(Hbig), 1).numpy(), rtol=1e-13)


# ----------------------------------------------------------------- router
def test_router_one_hot_rows_pick_rows_of_Wr():
    r = rng(4)
    h, E = 6, 5
    W = r.normal(size=(h, E))
    U = np.eye(h)[[3, 0, 5]]
    np.testing.assert_array_equal(O.router_logits(U, W), W[[3, 0, 5]])


def test_router_vs_library_with_bias_and_noise():
    r = rng(5)
    T, h, E = 7, 11, 6
    U, W, Wn = r.normal(size=(T, h)), r.normal(size=(h, E)), r.normal(size=(h, E))
    b, z = r.normal(size=E), r.normal(size=(T, E))
    Ut, Wt, Wnt = map(torch.from_numpy, (U, W, Wn))
    ref = F.linear(Ut, Wt.T) + torch.from_numpy(b) + torch.from_numpy(z) * F.softplus(F.linear(Ut, Wnt.T))
    np.testing.assert_allclose(O.router_logits(U, W, b, Wn, z), ref.numpy(), rtol=1e-13, atol=1e-13)
    # softplus stays finite and exact-ish far out
    assert O.softplus(np.array([800.0]))[0] == 800.0
    assert O.softplus(np.array([-800.0]))[0] == 0.0


# ----------------------------------------------------------------- noise generator
def _words(n: int, count: int):
    return [np.array([(n >> (64 * j)) & ((1 << 64) - 1)], dtype=np.uint64) for j in range(count)]


@pytest.mark.parametrize("case", range(12))
def test_philox_known_answers_vs_numpy(case):
    """The integer stream against numpy's own Philox-4x64-10 (an independent
    implementation in C).  numpy's bit generator increments its 256-bit counter
    before each block, so Philox(counter=c, key=k) starts with the block of
    counter c + 1."""
    r = np.random.default_rng(100 + case)
    if case == 0:
        c, k = 0, 0
    elif case == 1:
        c, k = (1 << 64) - 2, 7          # the +1 reaches 2^64 - 1, no carry
    elif case == 2:
        c, k = (1 << 64) - 1, 12345      # the +1 carries into word 1
    else:
        c = int.from_bytes(r.bytes(32), "little") >> (case % 3)
        k = int.from_bytes(r.bytes(16), "little")
    bg = np.random.Philox(counter=c, key=k)
    want = [int(v) for v in bg.random_raw(8)]
    got = []
    for blk in (1, 2):
        n = (c + blk) % (1 << 256)
        words = O.philox4x64_10(_words(n, 4), (k & ((1 << 64) - 1), k >> 64))
        got += [int(w[0]) for w in words]
    assert got == want


def test_philox_normals_take_one_counter_per_pair():
    """z[t, i] depends only on seed and t * E + i + rng_offset, so shifting the
    offset by E moves every draw up by one token, and any single pair can be
    drawn alone."""
    T, E, seed = 9, 7, 0xDEADBEEF
    z = O.philox_normals(T, E, seed, rng_offset=5)
    z2 = O.philox_normals(T, E, seed, rng_offset=5 + E)
    np.testing.assert_array_equal(z[1:], z2[:-1])
    for t, i in [(0, 0), (3, 4), (8, 6)]:
        assert O.philox_normals(1, 1, seed, t * E + i + 5)[0, 0] == z[t, i]
    # the counter wraps modulo 2^64
    top = O.philox_normals(1, 2, seed, (1 << 64) - 1)
    assert top[0, 1] == O.philox_normals(1, 1, seed, 0)[0, 0]
    # another seed gives other draws
    assert not np.array_equal(z, O.philox_normals(T, E, seed + 1, 5))


def test_philox_normals_are_standard_normal():
    """Moments of n = 2^18 draws (mean within 4 sigma / sqrt(n), variance
    within 1%), no correlation between neighbouring counters, and a
    Kolmogorov-Smirnov test against the normal distribution."""
    from scipy import stats
    z = O.philox_normals(4096, 64, seed=0)
    n = z.size
    assert abs(z.mean()) < 4.0 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 0.01
    assert abs(stats.kurtosis(z.ravel())) < 0.05
    flat = z.ravel()
    assert abs(np.corrcoef(flat[:-1], flat[1:])[0, 1]) < 4.0 / math.sqrt(n)
    assert stats.kstest(flat, "norm").pvalue > 1e-3
    # Box-Muller bounds: |z| <= sqrt(-2 ln 2^-53)
    assert np.abs(z).max() <= math.sqrt(2.0 * 53 * math.log(2.0))


# ----------------------------------------------------------------- fill
def brute_positions(idx, order):
    """Position of each assignment = number of earlier assignments (in fill order) to its expert."""
    T, k = idx.shape
    seq = [(t, r) for r in range(k) for t in range(T)] if order == O.FILL_RANK_MAJOR \
        else [(t, r) for t in range(T) for r in range(k)]
    pos = np.zeros((T, k), dtype=np.int64)
    for n, (t, r) in enumerate(seq):
        pos[t, r] = sum(1 for (t2, r2) in seq[:n] if idx[t2, r2] == idx[t, r])
    return pos


@pytest.mark.parametrize("order", [O.FILL_RANK_MAJOR, O.FILL_TOKEN_MAJOR])
def test_fill_brute_force(order):
    r = rng(6)
    T, E, k = 23, 5, 3
    H = r.normal(size=(T, E)) + np.array([1.5, 0, 0, -1, 0.5])
    idx = O.select_topk(H, k)
    C = 4
    fr = O.fill(idx, E, C, order)
    pos = brute_positions(idx, order)
    np.testing.assert_array_equal(fr["pos"], pos)
    # slot is a bijection between kept assignments and rows, grouped by expert
    kept = pos < C
    assert fr["offset"][-1] == kept.sum()
    rows = sorted(fr["slot"][kept].tolist())
    assert rows == list(range(int(kept.sum())))
    for t in range(T):
        for j in range(k):
            s = fr["slot"][t, j]
            if kept[t, j]:
                e = idx[t, j]
                assert fr["offset"][e] <= s < fr["offset"][e + 1]
                assert fr["row_token"][s] == t
            else:
                assert s == -1


def test_fill_rank_major_keeps_first_choices():
    # token 0's second choice and token 5's first choice land on expert 2 with C = 1.
    idx = np.array([[0, 2], [1, 3], [1, 3], [3, 1], [0, 1], [2, 0]])
    rm = O.fill(idx, 4, 1, O.FILL_RANK_MAJOR)
    tm = O.fill(idx, 4, 1, O.FILL_TOKEN_MAJOR)
    assert rm["slot"][5, 0] >= 0 and rm["slot"][0, 1] == -1
    assert tm["slot"][0, 1] >= 0 and tm["slot"][5, 0] == -1


# ----------------------------------------------------------------- experts and layer
def make_layer(T, h, f, E, seed):
    r = rng(seed)
    return (r.normal(size=(T, h)), r.normal(size=(h, E)) / math.sqrt(h),
            r.normal(size=(E, f, h)) / math.sqrt(h), r.normal(size=(E, f, h)) / math.sqrt(h),
            r.normal(size=(E, h, f)) / math.sqrt(f))


def torch_swiglu(x, Wg, Wu, Wd):
    x, Wg, Wu, Wd = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (x, Wg, Wu, Wd))
    return F.linear(F.silu(F.linear(x, Wg)) * F.linear(x, Wu), Wd).numpy()


def test_swiglu_vs_library():
    U, _, Wg, Wu, Wd = make_layer(9, 12, 20, 2, 7)
    np.testing.assert_allclose(O.swiglu_expert(U, Wg[1], Wu[1], Wd[1]),
                               torch_swiglu(U, Wg[1], Wu[1], Wd[1]), rtol=1e-12, atol=1e-13)
    v = np.linspace(-50, 50, 101)
    np.testing.assert_allclose(O.silu(v), F.silu(torch.from_numpy(v)).numpy(), rtol=1e-14, atol=1e-300)


def test_single_expert_is_dense_swiglu_plus_residual():
    U, W, Wg, Wu, Wd = make_layer(17, 8, 24, 1, 8)
    r = O.layer_forward(U, W, Wg, Wu, Wd, k=1, score=O.SOFTMAX, gate=O.GATE_RENORM,
                        capacity_factor=1.0)
    assert r["n_dropped"] == 0
    np.testing.assert_allclose(r["out"], U + torch_swiglu(U, Wg[0], Wu[0], Wd[0]),
                               rtol=1e-12, atol=1e-12)


def test_k_equals_E_is_soft_mixture():
    T, h, f, E = 13, 6, 10, 4
    U, W, Wg, Wu, Wd = make_layer(T, h, f, E, 9)
    r = O.layer_forward(U, W, Wg, Wu, Wd, k=E, score=O.SOFTMAX, gate=O.GATE_RENORM,
                        capacity_factor=1.0)
    p = torch.softmax(torch.from_numpy(U @ W), dim=1).numpy()
    ref = U + sum(p[:, e:e + 1] * torch_swiglu(U, Wg[e], Wu[e], Wd[e]) for e in range(E))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("score,gate,cf,order", [
    (O.SOFTMAX, O.GATE_RENORM, 0.75, O.FILL_RANK_MAJOR),
    (O.SOFTMAX, O.GATE_RAW, 0.5, O.FILL_TOKEN_MAJOR),
    (O.SIGMOID, O.GATE_RENORM, 1.25, O.FILL_RANK_MAJOR),
])
def test_sparse_equals_dense_masked_brute_force(score, gate, cf, order):
    T, h, f, E, k = 40, 8, 12, 6, 2
    U, W, Wg, Wu, Wd = make_layer(T, h, f, E, 10)
    W[:, 0] += 0.6  # skew the load so some assignments drop
    r = O.layer_forward(U, W, Wg, Wu, Wd, k=k, score=score, gate=gate, capacity_factor=cf,
                        fill_order=order)
    if cf < 1:
        assert r["n_dropped"] > 0
    gd = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            if r["slot"][t, j] >= 0:
                gd[t, r["idx"][t, j]] = r["gate"][t, j]
    np.testing.assert_allclose(r["out"], O.dense_masked_forward(U, Wg, Wu, Wd, gd),
                               rtol=1e-12, atol=1e-12)


def test_token_outputs_match_layer():
    T, h, f, E, k = 30, 8, 12, 5, 2
    U, W, Wg, Wu, Wd = make_layer(T, h, f, E, 11)
    r = O.layer_forward(U, W, Wg, Wu, Wd, k=k, score=O.SOFTMAX, gate=O.GATE_RENORM,
                        capacity_factor=0.8)
    toks = [0, 7, 29]
    o = O.token_outputs(toks, U, r["idx"], r["slot"], r["gate"], lambda e: (Wg[e], Wu[e], Wd[e]))
    np.testing.assert_allclose(o, r["out"][toks], rtol=1e-12, atol=1e-12)


def test_fully_dropped_tokens_pass_residual():
    T, h, f, E, k = 64, 8, 12, 4, 2
    U, W, Wg, Wu, Wd = make_layer(T, h, f, E, 12)
    r = O.layer_forward(U, W, Wg, Wu, Wd, k=k, score=O.SOFTMAX, gate=O.GATE_RENORM,
                        capacity_factor=1e-3)
    assert r["C"] == 1
    assert r["kept"].tolist() == [min(1, c) for c in r["count"]]
    full_drop = (r["slot"] < 0).all(axis=1)
    assert full_drop.sum() >= T - E
    np.testing.assert_array_equal(r["out"][full_drop], U[full_drop])


# ----------------------------------------------------------------- statistics
def test_aux_balanced_is_one_and_minimum():
    g = golden("aux_balance.json")
    E, k, T = 8, 2, 64
    # every expert receives exactly T k / E assignments and P is uniform (W_r = 0)
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)])
    s = np.full((T, E), 1.0 / E)
    fr = O.fill(idx, E, T)
    st = O.load_stats(s, idx, fr, O.SOFTMAX)
    assert abs(st["aux"] - g["balanced_aux"]) < 1e-14
    assert abs(st["f"].sum() - 1) < 1e-15 and abs(st["maxvio"]) < 1e-15
    # uniform P gives 1 for any load; any load satisfies sum f^2 >= 1/E (equality iff balanced)
    r = rng(13)
    for _ in range(5):
        idx = O.select_topk(r.normal(size=(T, E)) + r.normal(size=E) * 2, k)
        fr = O.fill(idx, E, T)
        st = O.load_stats(s, idx, fr, O.SOFTMAX)
        assert abs(st["aux"] - 1.0) < 1e-13
        assert (st["f"] ** 2).sum() >= 1.0 / E - 1e-15
    # with real softmax scores, the loss equals E sum(importance * load) with
    # importance = probs.sum(0) / probs.sum() and load = one-hot counts / their sum
    H = r.normal(size=(T, E)) * 2
    s = O.scores(H, O.SOFTMAX)
    idx = O.select_topk(H, k)
    st = O.load_stats(s, idx, O.fill(idx, E, T), O.SOFTMAX)
    probs = torch.from_numpy(s)
    importance = probs.sum(0) / probs.sum()
    load = F.one_hot(torch.from_numpy(idx), E).double().sum((0, 1))
    load = load / load.sum()
    assert abs(st["aux"] - float(E * (importance * load).sum())) < 1e-13
    assert st["aux"] >= 0


def test_maxvio_and_efficiency_example():
    g = golden("aux_balance.json")
    # mean load 4 (T k / E = 16 * 2 / 8), busiest expert 6: MaxVio = 0.5
    counts = [6, 4, 4, 4, 4, 4, 3, 3]
    idx = np.array([e for e, c in enumerate(counts) for _ in range(c)]).reshape(16, 2)
    fr = O.fill(idx, 8, 100)
    st = O.load_stats(np.full((16, 8), 1 / 8), idx, fr, O.SOFTMAX)
    assert abs(st["maxvio"] - g["maxvio_example"]) < 1e-15
    assert round(1 / (1 + st["maxvio"]), 2) == g["efficiency_example"]


def test_P_sums_to_one_for_both_scores():
    r = rng(14)
    H = r.normal(size=(50, 7)) * 3
    for score in (O.SOFTMAX, O.SIGMOID):
        s = O.scores(H, score)
        idx = O.select_topk(H, 2)
        st = O.load_stats(s, idx, O.fill(idx, 7, 50), score)
        assert abs(st["P"].sum() - 1.0) < 1e-14
    # sigmoid P is the token mean of s / sum_j s (not of raw s)
    s = O.scores(H, O.SIGMOID)
    st = O.load_stats(s, idx, O.fill(idx, 7, 50), O.SIGMOID)
    ref = (torch.from_numpy(s) / torch.from_numpy(s).sum(1, keepdim=True)).mean(0).numpy()
    np.testing.assert_allclose(st["P"], ref, rtol=1e-13)


def test_gate_sums_and_dropped_count():
    r = rng(15)
    T, E, k = 200, 16, 4
    H = r.normal(size=(T, E)) + np.linspace(2, -2, E)
    for score in (O.SOFTMAX, O.SIGMOID):
        C = O.capacity(T, E, k, 1.0)
        res = O.route(H, k, score, O.GATE_RENORM, C)
        np.testing.assert_allclose(res["gate"].sum(1), 1.0, rtol=1e-14)
        assert res["n_dropped"] == int((res["slot"] < 0).sum())
        assert res["n_dropped"] > 0


# ------------------------------------------------------------- DeepSeek-V3 parts
def test_bias_update_hand_example():
    g = golden("v3_routing.json")["bias_update"]
    b = O.update_bias(g["b"], g["count"], g["gamma"])
    np.testing.assert_allclose(b, g["b_new"], rtol=0, atol=1e-15)


def test_bias_update_moves_by_fixed_step():
    rng = np.random.default_rng(7)
    b = rng.normal(0, 0.01, 16)
    count = rng.integers(0, 100, 16)
    step = O.update_bias(b, count, 0.001) - b
    assert set(np.round(np.abs(step) / 0.001).astype(int).tolist()) <= {0, 1}
    # overloaded experts (count above the mean) go down, underloaded ones up
    assert (step[count > count.mean()] < 0).all() and (step[count < count.mean()] > 0).all()


def test_bias_selects_but_does_not_weigh():
    g = golden("v3_routing.json")["bias_only_selects"]
    H = np.zeros((3, g["E"]))
    C = O.capacity(3, g["E"], g["k"], 10.0)
    r = O.route(H, g["k"], O.SIGMOID, O.GATE_RENORM, C, b_sel=g["b"])
    assert (r["idx"] == g["idx"]).all()
    np.testing.assert_allclose(r["gate"], np.tile(g["gate"], (3, 1)), rtol=0, atol=1e-15)


def test_zero_bias_and_one_group_reduce_to_plain_topk():
    rng = np.random.default_rng(8)
    H = rng.normal(size=(200, 32))
    C = O.capacity(200, 32, 4, 1.25)
    for score in (O.SOFTMAX, O.SIGMOID):
        plain = O.route(H, 4, score, O.GATE_RENORM, C)
        biased = O.route(H, 4, score, O.GATE_RENORM, C, b_sel=np.zeros(32))
        grouped = O.route(H, 4, score, O.GATE_RENORM, C, b_sel=np.zeros(32), n_groups=8,
                          topk_groups=8)
        for r in (biased, grouped):
            assert (r["idx"] == plain["idx"]).all()
            np.testing.assert_array_equal(r["gate"], plain["gate"])
            np.testing.assert_array_equal(r["slot"], plain["slot"])


def test_large_bias_forces_an_expert():
    rng = np.random.default_rng(9)
    H = rng.normal(size=(100, 16))
    b = np.zeros(16)
    b[5] = 10.0  # sigmoid scores lie in (0, 1): expert 5's key beats every other
    C = O.capacity(100, 16, 2, 10.0)
    r = O.route(H, 2, O.SIGMOID, O.GATE_RENORM, C, b_sel=b)
    assert (r["idx"][:, 0] == 5).all()
    others = np.where(np.arange(16) == 5, -np.inf, H)
    assert (r["idx"][:, 1] == np.argmax(others, axis=1)).all()
    s = 1.0 / (1.0 + np.exp(-H))
    s5, s2 = s[:, 5], s[np.arange(100), r["idx"][:, 1]]
    np.testing.assert_allclose(r["gate"][:, 0], s5 / (s5 + s2), rtol=1e-15)


def test_group_limited_hand_example():
    g = golden("v3_routing.json")["group_limited"]
    H = np.zeros((2, g["E"]))
    C = O.capacity(2, g["E"], g["k"], 10.0)
    for M, key in ((1, "idx_M1"), (2, "idx_M2")):
        r = O.route(H, g["k"], O.SIGMOID, O.GATE_RENORM, C, b_sel=g["b"],
                    n_groups=g["n_groups"], topk_groups=M)
        assert (r["idx"] == g[key]).all(), (M, r["idx"])
    r = O.route(H, g["k"], O.SIGMOID, O.GATE_RENORM, C, b_sel=g["b"])
    assert (r["idx"] == g["idx_unrestricted"]).all()


def test_group_limited_brute_force():
    # every allowed set checked against enumeration of all group subsets
    import itertools
    rng = np.random.default_rng(10)
    E, G, M, k = 12, 4, 2, 4
    keys = rng.normal(size=(50, E))
    allowed = O.group_limited_mask(keys, G, M, k // M)
    gs = E // G
    for t in range(50):
        score = [np.sort(keys[t, g * gs:(g + 1) * gs])[::-1][:k // M].sum() for g in range(G)]
        best = max(itertools.combinations(range(G), M),
                   key=lambda c: (sum(score[g] for g in c), [-g for g in c]))
        want = np.zeros(E, dtype=bool)
        for g in best:
            want[g * gs:(g + 1) * gs] = True
        assert (allowed[t] == want).all()
    idx = O.select_topk_keys(keys, k, allowed)
    assert allowed[np.arange(50)[:, None], idx].all()


def test_shared_expert_is_an_always_on_expert():
    # a shared expert is an expert every token takes with gate 1 and no capacity:
    # the sparse layer with shared experts equals the dense masked form with a
    # column of ones for each shared expert
    rng = np.random.default_rng(11)
    T, h, f, E, k, Ns = 9, 6, 5, 4, 2, 2
    U = rng.normal(size=(T, h))
    W_r = rng.normal(size=(h, E))
    Wg, Wu, Wd = rng.normal(size=(E, f, h)), rng.normal(size=(E, f, h)), rng.normal(size=(E, h, f))
    Sg, Su, Sd = rng.normal(size=(Ns, f, h)), rng.normal(size=(Ns, f, h)), rng.normal(size=(Ns, h, f))
    r = O.layer_forward(U, W_r, Wg, Wu, Wd, k=k, score=O.SIGMOID, gate=O.GATE_RENORM,
                        capacity_factor=0.6, b_sel=rng.normal(0, 0.1, E), n_groups=2,
                        topk_groups=1, Ws_gate=Sg, Ws_up=Su, Ws_down=Sd)
    g_dense = np.zeros((T, E + Ns))
    for t in range(T):
        for rr in range(k):
            if r["slot"][t, rr] >= 0:
                g_dense[t, r["idx"][t, rr]] = r["gate"][t, rr]
    g_dense[:, E:] = 1.0
    dense = O.dense_masked_forward(U, np.concatenate([Wg, Sg]), np.concatenate([Wu, Su]),
                                   np.concatenate([Wd, Sd]), g_dense)
    np.testing.assert_allclose(r["out"], dense, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------- FP8
def _torch_e4m3(x):
    """Round-trip through torch's float8_e4m3fn (round to nearest even)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).double().numpy()


def test_fp8_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([O.fp8_e4m3_decode(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert O.fp8_e4m3_decode(0x7E) == 448.0 and O.fp8_e4m3_decode(0x01) == 2.0 ** -9
    assert sum(np.isnan(got)) == 2  # S.1111.111 only


def test_fp8_rounding_matches_torch():
    r = rng(11)
    vals = [r.uniform(-448, 448, 4000), r.normal(0, 1, 4000), r.normal(0, 2 ** -7, 4000),
            np.ldexp(r.uniform(-1, 1, 2000), r.integers(-12, 9, 2000))]
    # exact midpoints between neighbouring E4M3 values (ties go to the even mantissa)
    grid = np.unique(np.abs([O.fp8_e4m3_decode(c) for c in range(0x7F)]))
    mids = (grid[1:] + grid[:-1]) / 2
    vals += [mids, -mids]
    x = np.concatenate(vals).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(O.fp8_e4m3_round(x), _torch_e4m3(x))
    with pytest.raises(ValueError):
        O.fp8_e4m3_round(np.array([449.0]))


def test_fp8_row_scale_and_quantisation():
    assert O.fp8_row_scale(448.0) == 1.0 and O.fp8_row_scale(449.0) == 2.0
    assert O.fp8_row_scale(224.0) == 0.5 and O.fp8_row_scale(0.0) == 1.0
    r = rng(12)
    for amax in np.ldexp(r.uniform(0.5, 1.0, 200), r.integers(-60, 60, 200)):
        s = O.fp8_row_scale(amax)
        assert math.frexp(s)[0] == 0.5               # a power of two
        assert 224.0 < amax / s <= 448.0              # the top binade, never past 448
    X = r.normal(0, 3, (5, 64))
    X[2] = 0.0
    q, s = O.quantize_rows_fp8(X)
    assert s[2] == 1.0 and not q[2].any()
    np.testing.assert_array_equal(q, _torch_e4m3(X / s[:, None]))
    # relative error of a normal E4M3 value is at most 2^-4
    big = np.abs(X * 1.0) >= s[:, None] * 2.0 ** -6
    assert np.all(np.abs(q * s[:, None] - X)[big] <= 2.0 ** -4 * np.abs(X)[big])
    # scaling a row by a power of two scales s and leaves the codes alone
    q2, s2 = O.quantize_rows_fp8(X * 2.0 ** 13)
    np.testing.assert_array_equal(q2, q)
    nz = np.arange(len(s)) != 2
    np.testing.assert_array_equal(s2[nz], s[nz] * 2.0 ** 13)
    assert s2[2] == 1.0  # an all-zero row keeps the scale 1


def test_fp8_layer_equals_plain_layer_on_the_grid():
    # inputs already on the E4M3 grid with every row's largest magnitude in
    # (224, 448]: quantisation is the identity and the FP8 layer is the layer
    T, h, f, E, k = 24, 16, 12, 4, 2
    r = rng(13)

    def on_grid(shape):
        a = _torch_e4m3(r.uniform(-448, 448, shape))
        a.reshape(-1, shape[-1])[:, 0] = 448.0
        return a

    U = on_grid((T, h))
    W = r.normal(0, 1 / math.sqrt(h), (h, E))
    Wg, Wu = on_grid((E, f, h)), on_grid((E, f, h))
    Wd = r.normal(0, 1e-6, (E, h, f))
    a = O.layer_forward(U, W, Wg, Wu, Wd, k=k, score=O.SOFTMAX, gate=O.GATE_RENORM,
                        capacity_factor=1.0)
    b = O.layer_forward(U, W, Wg, Wu, Wd, k=k, score=O.SOFTMAX, gate=O.GATE_RENORM,
                        capacity_factor=1.0, fp8_up=True)
    np.testing.assert_array_equal(b["idx"], a["idx"])
    np.testing.assert_array_equal(b["Xq"], a["X"])
    np.testing.assert_array_equal(b["x_scale"], 1.0)
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-13, atol=1e-13)
    # off the grid the FP8 layer differs, by about the E4M3 rounding
    U2 = U * 0.3
    c = O.layer_forward(U2, W, Wg * 0.7, Wu, Wd, k=k, score=O.SOFTMAX, gate=O.GATE_RENORM,
                        capacity_factor=1.0, fp8_up=True)
    d = O.layer_forward(U2, W, Wg * 0.7, Wu, Wd, k=k, score=O.SOFTMAX, gate=O.GATE_RENORM,
                        capacity_factor=1.0)
    rel = np.abs(c["out"] - d["out"] - (U2 - U2)).max() / np.abs(d["out"] - U2).max()
    assert 0 < rel < 0.2


# ------------------------------------------------------------------ backward
def test_aux_gradient_worked_example():
    g = golden("aux_gradient.json")
    s = np.array([g["s"]])
    H = np.log(s)  # softmax(log s) = s
    np.testing.assert_allclose(O.scores(H, O.SOFTMAX), s, rtol=1e-15)
    assert abs(float(np.dot(g["f"], g["s"])) - g["weighted_mean_load"]) < 1e-15
    np.testing.assert_allclose(O.aux_logit_grad(O.scores(H, O.SOFTMAX), g["f"], O.SOFTMAX)[0],
                               g["grad"], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("score", [O.SOFTMAX, O.SIGMOID])
def test_aux_gradient_finite_differences(score):
    # sum_i f_i P_i with f held constant, P from the oracle's own statistics
    r = rng(21)
    T, E, k = 5, 6, 2
    H = r.normal(0, 1.5, (T, E))
    f = r.dirichlet(np.ones(E))

    def fp(Hx):
        s = O.scores(Hx, score)
        idx = O.select_topk(Hx, k)
        fr = O.fill(idx, E, T * k)
        return float(np.dot(f, O.load_stats(s, idx, fr, score)["P"]))

    eps = 1e-6
    fd = np.zeros_like(H)
    for t in range(T):
        for j in range(E):
            Hp, Hm = H.copy(), H.copy()
            Hp[t, j] += eps
            Hm[t, j] -= eps
            fd[t, j] = (fp(Hp) - fp(Hm)) / (2 * eps)
    np.testing.assert_allclose(fd, O.aux_logit_grad(O.scores(H, score), f, score) / T,
                               rtol=1e-6, atol=1e-10)


@pytest.mark.parametrize("score,gate,cf", [(O.SOFTMAX, O.GATE_RENORM, 0.6),
                                           (O.SIGMOID, O.GATE_RENORM, 1.0),
                                           (O.SOFTMAX, O.GATE_RAW, 0.6)])
def test_layer_backward_finite_differences(score, gate, cf):
    # L = <dOut, out> + alpha aux + c_z L_z; routing and the capacity cut are
    # piecewise constant, so central differences of the forward oracle must
    # match every gradient of layer_backward on generic inputs
    T, h, f, E, k = 7, 4, 3, 3, 2
    r = rng(22)
    U = r.normal(0, 1, (T, h))
    W_r = r.normal(0, 0.8, (h, E))
    b_r = r.normal(0, 0.3, E)
    Wg, Wu = r.normal(0, 0.6, (E, f, h)), r.normal(0, 0.6, (E, f, h))
    Wd = r.normal(0, 0.6, (E, h, f))
    dOut = r.normal(0, 1, (T, h))
    alpha, c_z = 0.3, 0.05
    kw = dict(k=k, score=score, gate=gate, capacity_factor=cf)

    def loss(U_, W_r_, b_r_, Wg_, Wu_, Wd_):
        o = O.layer_forward(U_, W_r_, Wg_, Wu_, Wd_, b_r=b_r_, **kw)
        return float(np.sum(dOut * o["out"])) + alpha * o["aux"] + c_z * o["z_loss"]

    fwd = O.layer_forward(U, W_r, Wg, Wu, Wd, b_r=b_r, **kw)
    if cf < 1:
        assert fwd["n_dropped"] > 0
    bw = O.layer_backward(U, W_r, Wg, Wu, Wd, fwd, dOut, score=score, gate=gate, alpha=alpha,
                          c_z=c_z)
    args = [U, W_r, b_r, Wg, Wu, Wd]
    names = ["dU", "dW_r", "db_r", "dW_gate", "dW_up", "dW_down"]
    eps = 1e-6
    for i, name in enumerate(names):
        fd = np.zeros_like(args[i])
        for j in np.ndindex(args[i].shape):
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[i][j] += eps
            am[i][j] -= eps
            fd[j] = (loss(*ap) - loss(*am)) / (2 * eps)
        np.testing.assert_allclose(bw[name], fd, rtol=1e-5, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("part", ["noisy", "shared", "v3"])
def test_layer_backward_finite_differences_parts(part):
    # the noisy router's softplus branch, shared experts, and the V3 routing
    # (selection bias, groups) with a shared expert: central differences of
    # the forward oracle against layer_backward
    T, h, f, E, k = 6, 4, 3, 4, 2
    r = rng(23)
    U = r.normal(0, 1, (T, h))
    W_r = r.normal(0, 0.8, (h, E))
    Wg, Wu = r.normal(0, 0.6, (E, f, h)), r.normal(0, 0.6, (E, f, h))
    Wd = r.normal(0, 0.6, (E, h, f))
    dOut = r.normal(0, 1, (T, h))
    alpha, c_z = 0.3, 0.05
    score = O.SIGMOID if part == "v3" else O.SOFTMAX
    kw = dict(k=k, score=score, gate=O.GATE_RENORM, capacity_factor=0.8)
    extra, names = {}, ["dU", "dW_r", "dW_gate", "dW_up", "dW_down"]
    if part == "noisy":
        extra = {"W_noise": r.normal(0, 0.8, (h, E)), "noise": r.normal(0, 1, (T, E))}
        names.append("dW_noise")
    if part in ("shared", "v3"):
        extra = {"Ws_gate": r.normal(0, 0.6, (2, 2, h)), "Ws_up": r.normal(0, 0.6, (2, 2, h)),
                 "Ws_down": r.normal(0, 0.6, (2, h, 2))}
        names += ["dWs_gate", "dWs_up", "dWs_down"]
    if part == "v3":
        kw.update(b_sel=r.normal(0, 0.3, E), n_groups=2, topk_groups=1)
    keys = ["U", "W_r", "W_gate", "W_up", "W_down"] + [n for n in extra if n != "noise"]
    base = dict(U=U, W_r=W_r, W_gate=Wg, W_up=Wu, W_down=Wd, **extra)

    def loss(v):
        o = O.layer_forward(v["U"], v["W_r"], v["W_gate"], v["W_up"], v["W_down"], **kw,
                            **{n: v[n] for n in extra})
        return float(np.sum(dOut * o["out"])) + alpha * o["aux"] + c_z * o["z_loss"]

    fwd = O.layer_forward(U, W_r, Wg, Wu, Wd, **kw, **extra)
    assert fwd["n_dropped"] > 0
    bw = O.layer_backward(U, W_r, Wg, Wu, Wd, fwd, dOut, score=score, gate=O.GATE_RENORM,
                          alpha=alpha, c_z=c_z, **extra)
    eps = 1e-6
    for key, name in zip(keys, names):
        fd = np.zeros_like(base[key])
        for j in np.ndindex(base[key].shape):
            vp = {n: a.copy() for n, a in base.items()}
            vm = {n: a.copy() for n, a in base.items()}
            vp[key][j] += eps
            vm[key][j] -= eps
            fd[j] = (loss(vp) - loss(vm)) / (2 * eps)
        np.testing.assert_allclose(bw[name], fd, rtol=1e-5, atol=1e-7, err_msg=name)


def test_fp8_backward_exact_on_the_grid():
    # one expert (gate 1, so dY = dOut) with dOut and W_down on the E4M3 grid:
    # quantising them is exact, and the FP8 backward equals the plain one
    r = rng(24)
    T, h, f = 9, 16, 8
    grid = np.array([O.fp8_e4m3_decode(c) for c in range(256)])
    grid = grid[np.isfinite(grid) & (np.abs(grid) <= 8) & (np.abs(grid) >= 0.25)]
    U = r.normal(0, 1, (T, h))
    W_r = r.normal(0, 1, (h, 1))
    Wg, Wu = r.normal(0, 0.5, (1, f, h)), r.normal(0, 0.5, (1, f, h))
    Wd = r.choice(grid, (1, h, f)) / 8
    dOut = r.choice(grid, (T, h))
    kw = dict(k=1, score=O.SOFTMAX, gate=O.GATE_RENORM, capacity_factor=0.0)
    fwd = O.layer_forward(U, W_r, Wg, Wu, Wd, **kw)
    a = O.layer_backward(U, W_r, Wg, Wu, Wd, fwd, dOut, score=O.SOFTMAX, gate=O.GATE_RENORM)
    b = O.layer_backward(U, W_r, Wg, Wu, Wd, fwd, dOut, score=O.SOFTMAX, gate=O.GATE_RENORM,
                         fp8_down_grad=True)
    np.testing.assert_array_equal(b["dYq"] * b["dY_scale"][:, None], dOut)
    for n in ("dU", "dW_r", "dW_gate", "dW_up", "dW_down"):
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)


def test_fp8_backward_within_the_rounding_bound():
    # generic inputs: dY rounds to E4M3 (relative error <= 2^-4 on normals),
    # so dW_down moves by about that much and the input-side gradients by a
    # few times that; a dropped or mis-scaled term would move them by O(1)
    r = rng(25)
    T, h, f, E, k = 40, 16, 12, 4, 2
    U = r.normal(0, 1, (T, h))
    W_r = r.normal(0, 0.5, (h, E))
    Wg, Wu = r.normal(0, 0.5, (E, f, h)), r.normal(0, 0.5, (E, f, h))
    Wd = r.normal(0, 0.5, (E, h, f))
    dOut = r.normal(0, 1, (T, h))
    kw = dict(k=k, score=O.SOFTMAX, gate=O.GATE_RENORM, capacity_factor=1.0)
    fwd = O.layer_forward(U, W_r, Wg, Wu, Wd, **kw)
    a = O.layer_backward(U, W_r, Wg, Wu, Wd, fwd, dOut, score=O.SOFTMAX, gate=O.GATE_RENORM)
    b = O.layer_backward(U, W_r, Wg, Wu, Wd, fwd, dOut, score=O.SOFTMAX, gate=O.GATE_RENORM,
                         fp8_down_grad=True)
    rel = lambda n: np.linalg.norm(b[n] - a[n]) / np.linalg.norm(a[n])
    assert 0 < rel("dW_down") < 2 ** -4
    for n in ("dW_gate", "dW_up", "dU"):
        assert 0 < rel(n) < 2 ** -2, (n, rel(n))
    # the router's gradient does not see the experts' input gradients
    np.testing.assert_array_equal(a["dW_r"], b["dW_r"])


def test_round_bf16():
    # against torch's conversion, ties to even, on random values and exact
    # midpoints between neighbouring bf16 values
    import torch
    r = rng(26)
    # midpoints: a bf16 value's bits with only the half-ulp bit set below them
    hi = r.integers(0x0080, 0x7F00, 4000, dtype=np.uint32) << 16
    sign = r.integers(0, 2, 4000, dtype=np.uint32) << 31
    mid = (hi | sign | 0x8000).view(np.float32)
    x = np.concatenate([(r.normal(0, 1, 5000) * np.exp2(r.integers(-20, 20, 5000)))
                        .astype(np.float32), mid])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(O.round_bf16(x), want)


def test_fp8_gradient_codes_of_stored_rows_within_one_step():
    """layer_backward(fp8_down_grad=True) quantises dY as the layer stores it:
    the float32 products g * dOut rounded to bf16.  This is the one place the
    oracle follows a storage rounding of the layer (elsewhere it stays in
    float64), so that both sides take each E4M3 decision on the same value.
    The choice moves little: the bf16 rounding shifts a value by at most 2^-9
    of itself, far below an E4M3 step (2^-4 of it at least), so the stored
    rows' dequantised codes and the exact products' differ by at most one
    step of the coarser of the two grids, also where the rounding moves a
    row's largest magnitude across a power-of-two scale boundary."""
    r = rng(31)
    dY = r.normal(0, 1, (200, 96)) * np.exp2(r.integers(-20, 20, (200, 1)))
    # rows whose largest magnitude sits just above 448 * 2^j: the exact row
    # takes the scale 2^(j+1), the bf16 row (rounded down to 448 * 2^j) 2^j
    for i, j in enumerate(range(-6, 6)):
        dY[i] = r.uniform(-1, 1, 96) * 300.0 * 2.0 ** j
        dY[i, 5] = 448.0 * (1 + 2.0 ** -10) * 2.0 ** j
    stored = O.round_bf16(dY.astype(np.float32))
    q_x, s_x = O.quantize_rows_fp8(dY)
    q_b, s_b = O.quantize_rows_fp8(stored)
    assert (s_b[:12] * 2 == s_x[:12]).all()    # the boundary rows change scale
    a, b = q_x * s_x[:, None], q_b * s_b[:, None]

    def step(q, s):  # E4M3 spacing at |q| (scaled units), times the row scale
        _, p1 = np.frexp(np.where(q != 0, np.abs(q), 1.0))
        return np.ldexp(1.0, np.maximum(p1 - 1, -6) - 3) * s[:, None]

    assert (np.abs(a - b) <= np.maximum(step(q_x, s_x), step(q_b, s_b))).all()
    assert (a[12:] == b[12:]).mean() > 0.9    # away from the boundary most codes agree
