"""GPU parity of the layer backward (through the C ABI) against the oracle's
layer_backward, evaluated for exactly the routing the GPU forward chose."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_37_amd import binding as B
from mixture_experts_layer_37_amd import inputs as I
from oracle import moe_oracle as O

import moe_testlib as L

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-2  # bf16 activations and weight gradients, float32 accumulation
# Element and row bounds of the expert weight gradients (elements against
# |x^| + the expert's rms, rows of normal size against their norm): each is a
# sum over the expert's rows of products whose factors went through up to five
# bf16 roundings (dY, g, u, dA, dG / dU, a); the same chain evaluated on the
# CPU reaches 2-3.5% per element and 3% per row on the small shapes
# (tests/test_tolerance_derivation.py), so both bounds are 5%.  Each expert's
# whole gradient stays within TOL.
WGRAD_ELEM_TOL = 5e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


BWD = {
    "mixtral_small": L.SMALL["mixtral_small"],
    "mixtral_drops": L.SMALL["mixtral_small"].replace(name="mixtral_drops", capacity_factor=0.6),
    "switch_small": L.SMALL["switch_small"],                     # raw gates, logit bias, drops
    "deepseek_small": L.SMALL["deepseek_small"],                 # sigmoid scores, k = 8
    "v3_keyed": L.SMALL["deepseek_small"].replace(name="v3_keyed", n_groups=8, topk_groups=4,
                                                  sel_bias_var=1e-4),
    "medium": I.WORKLOADS["mixtral_bf16"].replace(name="medium", T=2048, h=1024, f=2048),
    # T not a multiple of any tile, E not a multiple of 4, drops
    "ragged": I.WORKLOADS["mixtral_bf16"].replace(name="ragged", T=1000, h=192, f=320, E=6,
                                                  capacity_factor=0.9),
    # degenerate routing: every expert selected, one expert, dropless, and
    # most assignments dropped (their scores still renormalise the kept gates)
    "k_eq_E": I.WORKLOADS["mixtral_bf16"].replace(name="k_eq_E", T=512, h=128, f=192, E=4, k=4),
    "one_expert": I.WORKLOADS["mixtral_bf16"].replace(name="one_expert", T=300, h=128, f=128,
                                                      E=1, k=1),
    "dropless": I.WORKLOADS["deepseek_v3_bf16"].replace(name="dropless", T=512, h=256, f=192,
                                                        E=32, capacity_factor=0.0),
    "heavy_drops": I.WORKLOADS["mixtral_bf16"].replace(name="heavy_drops", T=1024, h=192, f=256,
                                                       capacity_factor=0.05),
    # 6 tokens, 16 experts, k = 1: at least 10 experts get no rows, and their
    # weight gradients must be written as exact zeros
    "idle_experts": I.WORKLOADS["mixtral_bf16"].replace(name="idle_experts", T=6, h=128, f=192,
                                                        E=16, k=1),
    # 200 experts: two expert tiles of 128 in the router weight gradient, the
    # second zero-padded, and a last 32-expert step of dU's product that is
    # partly past E; k = 6 under the 8-rank gathers of dU and the combine
    # backward (two absent ranks)
    "wide_e200_k6": I.WORKLOADS["mixtral_bf16"].replace(name="wide_e200_k6", T=600, h=256,
                                                        f=128, E=200, k=6, capacity_factor=1.0),
}


def close(got, ref, name, tol=TOL):
    """Group by group and element by element (moe_testlib.check_close): dU
    and dX per token; each expert's weight gradient matrix ([E, f, h] or
    [E, h, f]) as one group, so each element is held to tol (|x^| + rms of its
    expert's gradient); dW_r and dW_noise per expert (their columns); db_r as
    one group.  A group the oracle gives as exactly zero (an expert without
    rows) must be exactly zero.

    Rows of an expert's weight gradient are held to WGRAD_ELEM_TOL, and only
    rows whose norm is at least a quarter of the expert's typical row norm: with
    g and u stored in bf16 (the forward's kept activations, or the same values
    recomputed), SiLU'(g), which crosses zero near g = -1.28, carries an
    absolute error of about 2^-9 |g| |SiLU''|, so the rows of hidden units
    whose SiLU'(g) nearly vanishes on every row of the expert (experts with
    one or two rows) are small and have a large relative error, while their
    error against the expert's scale stays near 2^-9 (the element bound
    covers them)."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    if name.startswith("dW_r") or name.startswith("dW_noise"):
        got, ref = got.T, ref.T
    wgrad = ref.ndim == 3 and name.startswith("dW")
    return L.check_close(got, ref, tol, name, group_axes=2 if wgrad else 1,
                         elem_tol=WGRAD_ELEM_TOL if wgrad else tol,
                         row_tol=WGRAD_ELEM_TOL if wgrad else tol)


def run_backward(w, x, g, dOut, alpha, c_z, saved=None):
    cfg = B.make_config(w)
    T, h, f, E = w.T, w.h, w.f, w.E
    extra = {}
    if w.noisy:
        extra = {"W_noise": x["W_noise"],
                 "dW_noise": torch.empty((h, E), dtype=torch.float32, device=DEV)}
    if w.n_shared:
        ns, fs = w.n_shared, w.f_shared
        extra.update(Ws_gate=x["Ws_gate"], Ws_up=x["Ws_up"], Ws_down=x["Ws_down"],
                     dWs_gate=torch.empty((ns, fs, h), dtype=torch.bfloat16, device=DEV),
                     dWs_up=torch.empty((ns, fs, h), dtype=torch.bfloat16, device=DEV),
                     dWs_down=torch.empty((ns, h, fs), dtype=torch.bfloat16, device=DEV))
    out = {"dU": torch.empty((T, h), dtype=torch.bfloat16, device=DEV),
           "dW_r": torch.empty((h, E), dtype=torch.float32, device=DEV),
           "db_r": torch.empty((E,), dtype=torch.float32, device=DEV),
           "dW_gate": torch.empty((E, f, h), dtype=torch.bfloat16, device=DEV),
           "dW_up": torch.empty((E, f, h), dtype=torch.bfloat16, device=DEV),
           "dW_down": torch.empty((E, h, f), dtype=torch.bfloat16, device=DEV)}
    B.moe_layer_backward(cfg, x["U"], x["W_r"], x["W_gate"], x["W_up"], x["W_down"], g["logits"],
                         g["topk_idx"], g["topk_gate"], g["slot"], g["count"], g["offset"], dOut,
                         out["dU"], out["dW_r"], out["dW_gate"], out["dW_up"], out["dW_down"],
                         db_r=out["db_r"], alpha=alpha, c_z=c_z, saved=saved, **extra)
    torch.cuda.synchronize()
    out.update({n: t for n, t in extra.items() if n.startswith("d")})
    return out


@pytest.mark.parametrize("name", list(BWD))
def test_backward(name):
    w = BWD[name]
    L.log(f"[bwd] {name} {w}")
    x = I.make_inputs(w, seed=0, device=DEV)
    cfg, g = L.run_layer(w, x)
    gen = torch.Generator(device=DEV).manual_seed(5)
    dOut = torch.randn((w.T, w.h), generator=gen, device=DEV).to(torch.bfloat16)
    alpha, c_z = 0.01, 1e-3
    got = run_backward(w, x, g, dOut, alpha, c_z)
    # the oracle on the GPU forward's own routing
    offset = L.to_np(g["offset"]).astype(np.int64)
    rows = int(offset[-1])
    fwd = {"idx": L.to_np(g["topk_idx"]).astype(np.int64), "gate": L.f64(g["topk_gate"]),
           "slot": L.to_np(g["slot"]).astype(np.int64),
           "row_token": L.to_np(g["row_token"])[:rows].astype(np.int64),
           "offset": offset, "logits": L.f64(g["logits"]),
           "f": L.to_np(g["count"]).astype(np.float64) / (w.T * w.k)}
    ref = O.layer_backward(L.f64(x["U"]), L.f64(x["W_r"]), L.f64(x["W_gate"]), L.f64(x["W_up"]),
                           L.f64(x["W_down"]), fwd, L.f64(dOut),
                           score=L.ORACLE_MODE[w.score], gate=L.ORACLE_MODE[w.gate],
                           alpha=alpha, c_z=c_z)
    # every gradient row by row; an expert without rows gets exact zeros
    kept = L.to_np(g["kept"])
    if name == "idle_experts":
        assert (kept == 0).sum() >= 10, kept
    for n in ("dW_gate", "dW_up", "dW_down"):
        assert all(not got[n][e].any() for e in range(w.E) if kept[e] == 0), n
    errs = {n: close(L.f64(got[n]), ref[n], n)
            for n in ("dU", "dW_r", "db_r", "dW_gate", "dW_up", "dW_down")}
    L.log(f"  errs {errs}")


@pytest.mark.parametrize("name", ["mixtral_drops", "switch_small", "v3_keyed"])
def test_saved_activations_equal_recompute(name):
    # the forward keeps X, g | u, a and Y; the backward reading them gives the
    # same gradients bit for bit as recomputing them, and keeping them leaves
    # the forward's own outputs unchanged
    w = BWD[name]
    x = I.make_inputs(w, seed=1, device=DEV)
    cfg, g2 = L.run_layer(w, x)
    plain = [n for n in g2 if n != "out"]
    cfg, g = L.run_layer(w, x, fields=plain + ["GU", "A"])
    rows = int(g["offset"][-1])  # row-indexed outputs are defined up to offset[E]
    for n in plain + ["out"]:
        if n in ("row_token", "X", "Y"):
            assert torch.equal(g[n][:rows], g2[n][:rows]), n
        else:
            assert torch.equal(g[n], g2[n]), n
    gen = torch.Generator(device=DEV).manual_seed(9)
    dOut = torch.randn((w.T, w.h), generator=gen, device=DEV).to(torch.bfloat16)
    ref = run_backward(w, x, g, dOut, 0.01, 1e-3)
    got = run_backward(w, x, g, dOut, 0.01, 1e-3, saved={n: g[n] for n in B.SAVED_FIELDS})
    for n in ref:
        assert torch.equal(got[n], ref[n]), n


def test_backward_alpha_and_z_terms_only():
    # dOut = 0 leaves only the aux-loss and z-loss terms: dU = dH W_r^T with
    # dH from those two gradients, and the expert gradients vanish
    w = BWD["mixtral_small"]
    x = I.make_inputs(w, seed=2, device=DEV)
    cfg, g = L.run_layer(w, x)
    dOut = torch.zeros((w.T, w.h), dtype=torch.bfloat16, device=DEV)
    got = run_backward(w, x, g, dOut, 0.5, 0.25)
    for n in ("dW_gate", "dW_up", "dW_down"):
        assert not got[n].any(), n
    H = L.f64(g["logits"])
    s = O.scores(H, O.SOFTMAX)
    f = L.to_np(g["count"]).astype(np.float64) / (w.T * w.k)
    dH = 0.5 * w.E / w.T * O.aux_logit_grad(s, f, O.SOFTMAX) + 0.25 * O.z_loss_logit_grad(H)
    close(L.f64(got["dW_r"]), L.f64(x["U"]).T @ dH, "dW_r", tol=1e-4)
    close(L.f64(got["db_r"]), dH.sum(axis=0), "db_r", tol=1e-4)
    close(L.f64(got["dU"]), dH @ L.f64(x["W_r"]).T, "dU")


def test_backward_256_experts():
    # the largest expert count: one 64-lane wave holds a token's 256 scores
    w = I.WORKLOADS["deepseek_v3_bf16"].replace(name="e256_small", T=512, h=256, f=128)
    x = I.make_inputs(w, seed=4, device=DEV)
    cfg, g = L.run_layer(w, x)
    gen = torch.Generator(device=DEV).manual_seed(6)
    dOut = torch.randn((w.T, w.h), generator=gen, device=DEV).to(torch.bfloat16)
    got = run_backward(w, x, g, dOut, 0.01, 1e-3)
    fwd = oracle_routing(w, g)
    ref = O.layer_backward(L.f64(x["U"]), L.f64(x["W_r"]), L.f64(x["W_gate"]), L.f64(x["W_up"]),
                           L.f64(x["W_down"]), fwd, L.f64(dOut), score=L.ORACLE_MODE[w.score],
                           gate=L.ORACLE_MODE[w.gate], alpha=0.01, c_z=1e-3)
    for n in ("dU", "dW_r", "db_r", "dW_gate", "dW_up", "dW_down"):
        close(L.f64(got[n]), ref[n], n)


# --------------------------------------------------------------------------- full sizes
# At the full workload sizes the float64 oracle cannot afford the whole
# backward, so the checks use sub-problems that give exactly some of the
# outputs:
#  * expert weight gradients at a sample J of the hidden index f: SwiGLU acts
#    on each hidden unit alone and dY = gate * dOut needs no expert output, so
#    the layer restricted to W_gate[:, J], W_up[:, J], W_down[:, :, J] has the
#    weight gradients dW_gate[:, J], dW_up[:, J], dW_down[:, :, J];
#  * dU at a sample S of tokens: the token's own rows and scores decide it;
#    the loss terms carry 1/T, so a sub-problem of |S| tokens scales alpha and
#    c_z by |S|/T to weigh them as in the whole layer;
#  * dW_r, db_r with dOut zero outside S: the other tokens only carry the aux
#    and z terms, a sub-problem with no expert rows at all.


def oracle_routing(w, g, tokens=None):
    """The forward's routing as the oracle's fwd dict, optionally cut down to
    the given tokens (their rows renumbered, expert by expert)."""
    offset = L.to_np(g["offset"]).astype(np.int64)
    rows = int(offset[-1])
    idx = L.to_np(g["topk_idx"]).astype(np.int64)
    slot = L.to_np(g["slot"]).astype(np.int64)
    row_token = L.to_np(g["row_token"])[:rows].astype(np.int64)
    fwd = {"idx": idx, "gate": L.f64(g["topk_gate"]), "slot": slot, "row_token": row_token,
           "offset": offset, "logits": L.f64(g["logits"]),
           "f": L.to_np(g["count"]).astype(np.float64) / (w.T * w.k)}
    if tokens is None:
        return fwd
    tokens = np.asarray(tokens)
    pos = -np.ones(w.T, dtype=np.int64)
    pos[tokens] = np.arange(len(tokens))
    old = np.flatnonzero(pos[row_token] >= 0)          # kept rows of these tokens, in order
    new_of_old = -np.ones(rows, dtype=np.int64)
    new_of_old[old] = np.arange(len(old))
    s = slot[tokens]
    s_new = np.where(s >= 0, new_of_old[np.maximum(s, 0)], -1)
    expert_of_row = np.searchsorted(offset, old, side="right") - 1
    off_new = np.zeros(w.E + 1, dtype=np.int64)
    off_new[1:] = np.cumsum(np.bincount(expert_of_row, minlength=w.E))
    return {"idx": idx[tokens], "gate": fwd["gate"][tokens], "slot": s_new,
            "row_token": pos[row_token[old]], "offset": off_new,
            "logits": fwd["logits"][tokens], "f": fwd["f"]}


FULL = ["mixtral_bf16", "deepseek_v3_bf16", "switch_bf16", "noisy_long_bf16",
        "deepseek_v3_full_bf16"]


@pytest.fixture(scope="module")
def full_cases():
    return {}


def full_case(full_cases, name):
    if name not in full_cases:
        full_cases.clear()                               # one full workload on the GPU at a time
        torch.cuda.empty_cache()
        w = I.WORKLOADS[name]
        x = I.make_inputs(w, seed=0, device=DEV)
        cfg, g = L.run_layer(w, x, fields=["logits", "topk_idx", "topk_gate", "slot",
                                           "row_token", "count", "kept", "offset"])
        full_cases[name] = (w, x, g)
    return full_cases[name]


@pytest.mark.parametrize("name,fp8", [(n, False) for n in FULL] + [("mixtral_bf16", True)])
def test_full_size_weight_gradients(full_cases, name, fp8):
    # fp8: the experts' output gradients as FP8 rows; W_down's per-column
    # scales are column-local and the dY rows do not depend on the weights,
    # so the restriction to J stays exact
    w, x, g = full_case(full_cases, name)
    L.log(f"[bwd full wgrad] {name}{' fp8 gradients' if fp8 else ''}")
    gen = torch.Generator(device=DEV).manual_seed(7)
    dOut = torch.randn((w.T, w.h), generator=gen, device=DEV).to(torch.bfloat16)
    if fp8:
        WdT8, sdT = fp8_down_weights(x)
        got = {n: torch.empty_like(x[m]) for n, m in (("dW_gate", "W_gate"), ("dW_up", "W_up"),
                                                      ("dW_down", "W_down"), ("dU", "U"))}
        got["dW_r"] = torch.empty((w.h, w.E), dtype=torch.float32, device=DEV)
        B.moe_layer_backward(B.make_config(w), x["U"], x["W_r"], x["W_gate"], x["W_up"],
                             x["W_down"], g["logits"], g["topk_idx"], g["topk_gate"], g["slot"],
                             g["count"], g["offset"], dOut, got["dU"], got["dW_r"],
                             got["dW_gate"], got["dW_up"], got["dW_down"], alpha=0.01, c_z=1e-3,
                             W_downT8=WdT8, s_downT=sdT)
        torch.cuda.synchronize()
    else:
        got = run_backward(w, x, g, dOut, 0.01, 1e-3)
    rng = np.random.default_rng(1)
    J = np.unique(np.concatenate([[0, w.f - 1], rng.choice(w.f, 14, replace=False)]))
    Jt = torch.as_tensor(J, device=DEV)
    sub = lambda t, dim: L.f64(t.index_select(dim, Jt))
    # the shared experts (output gradient dOut) restrict the same way
    shared = {}
    if w.n_shared:
        Js = torch.as_tensor(J[J < w.f_shared], device=DEV)
        ssub = lambda t, dim: L.f64(t.index_select(dim, Js))
        shared = dict(Ws_gate=ssub(x["Ws_gate"], 1), Ws_up=ssub(x["Ws_up"], 1),
                      Ws_down=ssub(x["Ws_down"], 2))
    ref = O.layer_backward(L.f64(x["U"]), L.f64(x["W_r"]), sub(x["W_gate"], 1),
                           sub(x["W_up"], 1), sub(x["W_down"], 2), oracle_routing(w, g),
                           L.f64(dOut), score=L.ORACLE_MODE[w.score],
                           gate=L.ORACLE_MODE[w.gate], fp8_down_grad=fp8, **shared)
    kept = L.to_np(g["kept"])
    for n, dim in (("dW_gate", 1), ("dW_up", 1), ("dW_down", 2)):
        G = sub(got[n], dim)
        assert all(not G[e].any() for e in range(w.E) if kept[e] == 0), n
        # each expert's sampled hidden units form one group
        err = close(G, ref[n], n)
        L.log(f"  {n} worst {err}")
    if w.n_shared:
        for n, dim in (("dWs_gate", 1), ("dWs_up", 1), ("dWs_down", 2)):
            G = L.f64(got[n].index_select(dim, Js))
            err = close(G, ref[n], n)
            L.log(f"  {n} worst {err}")


def test_full_size_input_and_router_gradients(full_cases):
    # Mixtral shape: dOut nonzero on a sample S of tokens; every dU row, dW_r
    # and db_r are then checked whole
    w, x, g = full_case(full_cases, "mixtral_bf16")
    L.log("[bwd full dU/dW_r] mixtral_bf16")
    alpha, c_z = 0.01, 1e-3
    rng = np.random.default_rng(2)
    S = np.sort(rng.choice(w.T, 24, replace=False))
    gen = torch.Generator(device=DEV).manual_seed(8)
    dOut = torch.zeros((w.T, w.h), dtype=torch.bfloat16, device=DEV)
    St = torch.as_tensor(S, device=DEV)
    dOut[St] = torch.randn((len(S), w.h), generator=gen, device=DEV).to(torch.bfloat16)
    got = run_backward(w, x, g, dOut, alpha, c_z)
    U, W_r = L.f64(x["U"]), L.f64(x["W_r"])
    mode = dict(score=L.ORACLE_MODE[w.score], gate=L.ORACLE_MODE[w.gate])
    # the sampled tokens, with the whole experts
    fS = len(S) / w.T
    refS = O.layer_backward(U[S], W_r, L.f64(x["W_gate"]), L.f64(x["W_up"]), L.f64(x["W_down"]),
                            oracle_routing(w, g, S), L.f64(dOut[St]), alpha=alpha * fS,
                            c_z=c_z * fS, **mode)
    # the other tokens: no upstream gradient, so no expert rows take part
    R = np.setdiff1d(np.arange(w.T), S)
    fwdR = oracle_routing(w, g, R)
    fwdR["slot"] = -np.ones_like(fwdR["slot"])
    fwdR["row_token"] = fwdR["row_token"][:0]
    fwdR["offset"] = np.zeros_like(fwdR["offset"])
    none = lambda t, dim: L.f64(t.narrow(dim, 0, 0))
    fR = len(R) / w.T
    refR = O.layer_backward(U[R], W_r, none(x["W_gate"], 1), none(x["W_up"], 1),
                            none(x["W_down"], 2), fwdR, np.zeros((len(R), w.h)),
                            alpha=alpha * fR, c_z=c_z * fR, **mode)
    dU = np.zeros((w.T, w.h))
    dU[S], dU[R] = refS["dU"], refR["dU"]
    errs = {"dU": close(L.f64(got["dU"]), dU, "dU"),
            "dW_r": close(L.f64(got["dW_r"]), refS["dW_r"] + refR["dW_r"], "dW_r"),
            "db_r": close(L.f64(got["db_r"]), refS["db_r"] + refR["db_r"], "db_r")}
    L.log(f"  errs {errs}")


EXTRA = {
    "noisy_small": L.SMALL["noisy_small"],
    "shared2": L.SMALL["mixtral_small"].replace(name="shared2", n_shared=2, f_shared=128,
                                                capacity_factor=0.8),
    "v3_full_small": L.SMALL["deepseek_small"].replace(name="v3_full_small", n_groups=8,
                                                       topk_groups=4, sel_bias_var=1e-4,
                                                       n_shared=1, f_shared=192),
    "ragged_noisy_shared": L.SMALL["noisy_small"].replace(name="ragged_noisy_shared", T=777,
                                                          h=192, f=192, E=6, n_shared=1,
                                                          f_shared=64),
    # E = 100 (not a multiple of 8: element-wise operand loads in dU's
    # product, a padded W_noise for the recomputed Z, one zero-padded expert
    # tile of 128 in dW_r and dW_noise) with k = 3 and a shared expert
    "noisy_e100_k3": L.SMALL["noisy_small"].replace(name="noisy_e100_k3", T=500, h=192, f=128,
                                                    E=100, k=3, n_shared=1, f_shared=64),
}


@pytest.mark.parametrize("name", list(EXTRA))
def test_backward_noisy_and_shared(name):
    w = EXTRA[name]
    L.log(f"[bwd extra] {name} {w}")
    x = I.make_inputs(w, seed=3, device=DEV)
    cfg, g = L.run_layer(w, x)
    gen = torch.Generator(device=DEV).manual_seed(10)
    dOut = torch.randn((w.T, w.h), generator=gen, device=DEV).to(torch.bfloat16)
    alpha, c_z = 0.01, 1e-3
    got = run_backward(w, x, g, dOut, alpha, c_z)
    kw = {}
    if w.noisy:
        kw.update(W_noise=L.f64(x["W_noise"]), noise=L.oracle_noise(w))
    if w.n_shared:
        kw.update(Ws_gate=L.f64(x["Ws_gate"]), Ws_up=L.f64(x["Ws_up"]),
                  Ws_down=L.f64(x["Ws_down"]))
    ref = O.layer_backward(L.f64(x["U"]), L.f64(x["W_r"]), L.f64(x["W_gate"]), L.f64(x["W_up"]),
                           L.f64(x["W_down"]), oracle_routing(w, g), L.f64(dOut),
                           score=L.ORACLE_MODE[w.score], gate=L.ORACLE_MODE[w.gate],
                           alpha=alpha, c_z=c_z, **kw)
    names = ["dU", "dW_r", "db_r", "dW_gate", "dW_up", "dW_down"]
    names += ["dW_noise"] if w.noisy else []
    names += ["dWs_gate", "dWs_up", "dWs_down"] if w.n_shared else []
    errs = {n: close(L.f64(got[n]), ref[n], n) for n in names}
    L.log(f"  errs {errs}")


def test_backward_empty_batch_with_shared_experts():
    # T = 0: every weight gradient is exactly zero
    w = EXTRA["v3_full_small"].replace(name="v3_empty", T=0)
    x = I.make_inputs(w, seed=3, device=DEV)
    cfg, g = L.run_layer(w, x)
    dOut = torch.zeros((0, w.h), dtype=torch.bfloat16, device=DEV)
    got = run_backward(w, x, g, dOut, 0.01, 1e-3)
    for n in ("dW_r", "db_r", "dW_gate", "dW_up", "dW_down", "dWs_gate", "dWs_up", "dWs_down"):
        assert not got[n].any(), n


@pytest.mark.parametrize("name,saved", [("mixtral_drops", False), ("mixtral_drops", True),
                                        ("noisy_small", False), ("v3_full_small", False)])
def test_staged_backward_equals_layer(name, saved):
    # combine backward, the experts' backward and the router backward called
    # one by one give the layer call's gradients bit for bit; only with shared
    # experts dU differs, since the caller adds their input gradients to dOut
    # in bf16 first, one more rounding (compared at the bf16 bar)
    w = {**BWD, **EXTRA}[name]
    x = I.make_inputs(w, seed=6, device=DEV)
    fields = ["logits", "topk_idx", "topk_gate", "slot", "count", "kept", "offset", "X", "Y"]
    cfg, g = L.run_layer(w, x, fields=fields + (["GU", "A"] if saved else []))
    gen = torch.Generator(device=DEV).manual_seed(12)
    dOut = torch.randn((w.T, w.h), generator=gen, device=DEV).to(torch.bfloat16)
    alpha, c_z = 0.01, 1e-3
    ref = run_backward(w, x, g, dOut, alpha, c_z)
    rows, bf = B.max_rows(cfg), torch.bfloat16
    dY = torch.empty((rows, w.h), dtype=bf, device=DEV)
    dgate = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    B.moe_combine_backward(cfg, dOut, g["Y"], g["slot"], g["topk_gate"], dY, dgate)
    dX = torch.empty((rows, w.h), dtype=bf, device=DEV)
    got = {n: torch.empty_like(ref[n]) for n in ("dU", "dW_r", "db_r", "dW_gate", "dW_up",
                                                  "dW_down")}
    B.moe_expert_ffn_backward(cfg, g["X"], g["offset"], x["W_gate"], x["W_up"], x["W_down"], dY,
                              dX, got["dW_gate"], got["dW_up"], got["dW_down"],
                              GU=g["GU"] if saved else None, A=g["A"] if saved else None)
    d_res = dOut
    if w.n_shared:
        cfg_s = B.make_config(w.replace(E=1, k=1, f=w.f_shared, n_shared=0, f_shared=0,
                                        n_groups=0, topk_groups=0, sel_bias_var=0.0,
                                        capacity_factor=0.0))
        offs = torch.tensor([0, w.T], dtype=torch.int32, device=DEV)
        acc = dOut.float()
        for n in ("dWs_gate", "dWs_up", "dWs_down"):
            got[n] = torch.empty_like(ref[n])
        for i in range(w.n_shared):
            dXs = torch.empty((w.T, w.h), dtype=bf, device=DEV)
            B.moe_expert_ffn_backward(cfg_s, x["U"], offs, x["Ws_gate"][i:i + 1],
                                      x["Ws_up"][i:i + 1], x["Ws_down"][i:i + 1], dOut, dXs,
                                      got["dWs_gate"][i:i + 1], got["dWs_up"][i:i + 1],
                                      got["dWs_down"][i:i + 1])
            acc += dXs.float()
        d_res = acc.to(bf)
    noise = {}
    if w.noisy:
        got["dW_noise"] = torch.empty_like(ref["dW_noise"])
        noise = dict(W_noise=x["W_noise"], dW_noise=got["dW_noise"])
    B.moe_router_backward(cfg, x["U"], x["W_r"], g["logits"], g["topk_idx"], g["topk_gate"],
                          g["slot"], g["count"], dgate, d_res, dX, got["dU"], got["dW_r"],
                          db_r=got["db_r"], alpha=alpha, c_z=c_z, **noise)
    torch.cuda.synchronize()
    for n in got:
        if w.n_shared and n == "dU":
            close(L.f64(got[n]), L.f64(ref[n]), n)
        else:
            assert torch.equal(got[n], ref[n]), n


def test_backward_deterministic_and_stream_ordered():
    # no atomics and fixed-order partial sums: repeated runs agree bit for bit,
    # also on other streams with their own workspaces
    w = EXTRA["v3_full_small"]
    x = I.make_inputs(w, seed=8, device=DEV)
    cfg, g = L.run_layer(w, x)
    gen = torch.Generator(device=DEV).manual_seed(13)
    dOut = torch.randn((w.T, w.h), generator=gen, device=DEV).to(torch.bfloat16)
    ref = run_backward(w, x, g, dOut, 0.01, 1e-3)
    again = run_backward(w, x, g, dOut, 0.01, 1e-3)
    for n in ref:
        assert torch.equal(ref[n], again[n]), n
    outs = []
    for _ in range(2):
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            outs.append(run_backward(w, x, g, dOut, 0.01, 1e-3))
    torch.cuda.synchronize()
    for o in outs:
        for n in ref:
            assert torch.equal(ref[n], o[n]), n


# --------------------------------------------------------------------------- FP8 gradients
FP8_DECODE = np.array([O.fp8_e4m3_decode(c) for c in range(256)])


def fp8_down_weights(x):
    """W_down^T quantised row-wise: codes [E, f, h] and scales [E, f]."""
    return B.moe_quantize_rows_fp8(x["W_down"].transpose(1, 2).contiguous())


@pytest.mark.parametrize("name", ["fp8_grad_small", "fp8_grad_v3"])
def test_fp8_output_gradients(name):
    # the experts' output gradients as FP8 rows: codes bit for bit against the
    # oracle's quantisation of the GPU's own dY rows, the staged call against
    # the oracle's expert_backward_fp8, and the layer call equal to the staged
    # path bit for bit and close to the oracle's layer_backward with FP8
    # gradients
    w = {"fp8_grad_small": L.SMALL["mixtral_small"].replace(name=name, h=256, f=384,
                                                           capacity_factor=0.8),
         "fp8_grad_v3": L.SMALL["deepseek_small"].replace(name=name, h=384, f=192)}[name]
    x = I.make_inputs(w, seed=9, device=DEV)
    fields = ["logits", "topk_idx", "topk_gate", "slot", "row_token", "count", "kept", "offset",
              "X", "Y"]
    cfg, g = L.run_layer(w, x, fields=fields)
    gen = torch.Generator(device=DEV).manual_seed(14)
    dOut = torch.randn((w.T, w.h), generator=gen, device=DEV).to(torch.bfloat16)
    WdT8, sdT = fp8_down_weights(x)
    rows_max, bf = B.max_rows(cfg), torch.bfloat16
    offset = L.to_np(g["offset"]).astype(np.int64)
    rows = int(offset[-1])
    # staged: combine backward, quantise the dY rows, the experts' FP8 backward
    dY = torch.zeros((rows_max, w.h), dtype=bf, device=DEV)
    dgate = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    B.moe_combine_backward(cfg, dOut, g["Y"], g["slot"], g["topk_gate"], dY, dgate)
    dY8, sy = B.moe_quantize_rows_fp8(dY)
    dX = torch.empty((rows_max, w.h), dtype=bf, device=DEV)
    st = {n: torch.empty_like(x[m]) for n, m in (("dW_gate", "W_gate"), ("dW_up", "W_up"),
                                                 ("dW_down", "W_down"))}
    B.moe_expert_ffn_backward_fp8(cfg, g["X"], g["offset"], x["W_gate"], x["W_up"], WdT8, sdT,
                                  dY8, sy, dX, st["dW_gate"], st["dW_up"], st["dW_down"])
    torch.cuda.synchronize()
    q_ref, s_ref = O.quantize_rows_fp8(L.f64(dY[:rows]))
    q_got = FP8_DECODE[L.to_np(dY8[:rows]).astype(np.int64)]
    np.testing.assert_array_equal(q_got, q_ref)
    np.testing.assert_array_equal(L.f64(sy[:rows]), s_ref)
    eX, eWg, eWu, eWd = O.expert_backward_fp8(L.f64(g["X"][:rows]), offset, L.f64(x["W_gate"]),
                                              L.f64(x["W_up"]), L.f64(x["W_down"]), q_ref, s_ref)
    close(L.f64(dX[:rows]), eX, "dX")
    for n, ref in (("dW_gate", eWg), ("dW_up", eWu), ("dW_down", eWd)):
        close(L.f64(st[n]), ref, n)
    # the layer call
    out = {"dU": torch.empty_like(x["U"]),
           "dW_r": torch.empty((w.h, w.E), dtype=torch.float32, device=DEV),
           "db_r": torch.empty((w.E,), dtype=torch.float32, device=DEV),
           "dW_gate": torch.empty_like(x["W_gate"]), "dW_up": torch.empty_like(x["W_up"]),
           "dW_down": torch.empty_like(x["W_down"])}
    B.moe_layer_backward(cfg, x["U"], x["W_r"], x["W_gate"], x["W_up"], x["W_down"], g["logits"],
                         g["topk_idx"], g["topk_gate"], g["slot"], g["count"], g["offset"], dOut,
                         out["dU"], out["dW_r"], out["dW_gate"], out["dW_up"], out["dW_down"],
                         db_r=out["db_r"], alpha=0.01, c_z=1e-3, W_downT8=WdT8, s_downT=sdT)
    torch.cuda.synchronize()
    for n in ("dW_gate", "dW_up", "dW_down"):
        assert torch.equal(out[n], st[n]), n
    ref = O.layer_backward(L.f64(x["U"]), L.f64(x["W_r"]), L.f64(x["W_gate"]), L.f64(x["W_up"]),
                           L.f64(x["W_down"]), oracle_routing(w, g), L.f64(dOut),
                           score=L.ORACLE_MODE[w.score], gate=L.ORACLE_MODE[w.gate],
                           alpha=0.01, c_z=1e-3, fp8_down_grad=True)
    for n in out:
        close(L.f64(out[n]), ref[n], n)
