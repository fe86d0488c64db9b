"""GPU parity of the FP8 dispatch and FP8 up-projection (through the C ABI)
against the oracle: E4M3 codes and power-of-two scales bit for bit, routing as
in the bf16 layer, outputs within the bf16 tolerance of the oracle's FP8 layer
(which works on the same quantised values in float64)."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_37_amd import binding as B
from mixture_experts_layer_37_amd import inputs as I
from oracle import moe_oracle as O

import moe_testlib as L

pytestmark = pytest.mark.gpu

DEV = "cuda"
DECODE = np.array([O.fp8_e4m3_decode(c) for c in range(256)])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def decode(codes: torch.Tensor) -> np.ndarray:
    return DECODE[codes.cpu().numpy().astype(np.int64)]


def special_rows(n, cols, gen):
    """bf16 rows covering the quantiser's cases: normal, zero, largest
    magnitude exactly 448, tiny (subnormal codes), huge, mixed signs."""
    x = torch.randn(n, cols, generator=gen)
    x[0] = 0.0
    x[1] = torch.randn(cols, generator=gen) * 1e-3
    x[1, 0] = 448.0
    x[2] = torch.randn(cols, generator=gen) * 1e-30
    x[3] = torch.randn(cols, generator=gen) * 3e30
    x[4] = torch.linspace(-7.0, 7.0, cols)
    x[5, :] = 0.0
    x[5, 3] = -1.0
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("rows,cols", [(6, 8), (37, 384), (300, 4096)])
def test_quantize_rows_fp8(rows, cols):
    gen = torch.Generator().manual_seed(rows * cols)
    x = special_rows(max(rows, 6), cols, gen)[:max(rows, 6)]
    q, s = B.moe_quantize_rows_fp8(x.to(DEV))
    torch.cuda.synchronize()
    qo, so = O.quantize_rows_fp8(x.double().numpy())
    np.testing.assert_array_equal(s.cpu().double().numpy(), so)
    np.testing.assert_array_equal(decode(q), qo)


FP8 = {
    "mixtral_fp8_small": L.SMALL["mixtral_small"].replace(name="mixtral_fp8_small", h=384,
                                                          fp8_up=True),
    "switch_fp8_small": L.SMALL["switch_small"].replace(name="switch_fp8_small", fp8_up=True),
    "deepseek_fp8_small": L.SMALL["deepseek_small"].replace(name="deepseek_fp8_small", h=512,
                                                            fp8_up=True),
    "noisy_fp8_small": L.SMALL["noisy_small"].replace(name="noisy_fp8_small", h=384,
                                                      fp8_up=True),
    "v3_fp8_small": L.SMALL["deepseek_small"].replace(name="v3_fp8_small", h=512, n_groups=8,
                                                      topk_groups=4, n_shared=1, f_shared=128,
                                                      sel_bias_var=1e-4, fp8_up=True),
    "one_k_step": L.SMALL["mixtral_small"].replace(name="one_k_step", T=300, h=128, f=192,
                                                   fp8_up=True),
    "ksplit_gate_up": L.SMALL["mixtral_small"].replace(name="ksplit_gate_up", T=2204, E=1, k=1,
                                                       h=512, f=4096, fp8_up=True),
}


def fp8_dispatch(w, cfg, x, idx):
    rows = B.max_rows(cfg)
    out = {n: torch.empty(sh, dtype=dt, device=DEV) for n, sh, dt in [
        ("X8", (rows, w.h), torch.uint8), ("x_scale", (rows,), torch.float32),
        ("row_token", (rows,), torch.int32), ("slot", (w.T, w.k), torch.int32),
        ("count", (w.E,), torch.int32), ("kept", (w.E,), torch.int32),
        ("offset", (w.E + 1,), torch.int32)]}
    B.moe_dispatch_fp8(cfg, x["U"], idx, out["X8"], out["x_scale"], out["row_token"],
                       out["slot"], out["count"], out["kept"], out["offset"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(FP8))
def test_fp8_layer_small(name):
    w = FP8[name]
    L.log(f"[fp8] {name} {w}")
    x = I.make_inputs(w, seed=0, device=DEV)
    cfg, g = L.run_layer(w, x)
    # routing and statistics: the router is the bf16 one
    r = L.check_routing_shared_logits(w, g, x.get("b_sel"))
    L.check_stats(w, g, r)
    # the dispatched FP8 rows, bit for bit against the oracle's quantisation
    d = fp8_dispatch(w, cfg, x, g["topk_idx"])
    rows = int(r["offset"][-1])
    assert torch.equal(d["slot"], g["slot"]) and torch.equal(d["offset"], g["offset"])
    U = L.f64(x["U"])
    qo, so = O.quantize_rows_fp8(U[r["row_token"]])
    np.testing.assert_array_equal(decode(d["X8"][:rows]), qo)
    np.testing.assert_array_equal(d["x_scale"][:rows].cpu().double().numpy(), so)
    # the weights' codes, then the layer against the oracle's FP8 layer routed
    # from the GPU's logits
    W8g, sg, W8u, su = L.fp8_weights(x)
    qg, sgo = O.quantize_rows_fp8(L.f64(x["W_gate"]).reshape(-1, w.h))
    np.testing.assert_array_equal(decode(W8g).reshape(-1, w.h), qg)
    np.testing.assert_array_equal(sg.cpu().double().numpy().reshape(-1), sgo)
    ref = O.layer_forward(U, L.f64(x["W_r"]), L.f64(x["W_gate"]), L.f64(x["W_up"]),
                          L.f64(x["W_down"]), k=w.k, score=L.ORACLE_MODE[w.score],
                          gate=L.ORACLE_MODE[w.gate], capacity_factor=w.capacity_factor,
                          cap_mode=L.ORACLE_MODE[w.cap_mode], fill_order=L.ORACLE_MODE[w.fill],
                          min_capacity=w.min_capacity, logits=L.f64(g["logits"]),
                          b_sel=None if x.get("b_sel") is None else L.f64(x["b_sel"]),
                          n_groups=max(1, w.n_groups), topk_groups=max(1, w.topk_groups),
                          Ws_gate=None if w.n_shared == 0 else L.f64(x["Ws_gate"]),
                          Ws_up=None if w.n_shared == 0 else L.f64(x["Ws_up"]),
                          Ws_down=None if w.n_shared == 0 else L.f64(x["Ws_down"]), fp8_up=True)
    if not L.keyed(w):  # keyed routing is checked against the GPU's own selection above
        np.testing.assert_array_equal(ref["idx"], L.to_np(g["topk_idx"]))
        L.check_close(L.to_np(g["out"]), ref["out"], L.out_tol(w), "out")
        L.check_delta(w, L.f64(g["out"]), U, ref["out"])
    ey = L.check_close(L.to_np(g["Y"][:rows]), O.expert_outputs_fp8(
        qo, so, r["offset"], qg.reshape(w.E, w.f, w.h), sgo.reshape(w.E, w.f),
        *[a.reshape(*s) for a, s in zip(O.quantize_rows_fp8(L.f64(x["W_up"]).reshape(-1, w.h)),
                                        [(w.E, w.f, w.h), (w.E, w.f)])],
        L.f64(x["W_down"])), L.out_tol(w), "Y")
    L.log(f"  drops={r['n_dropped']} Y err={ey}")


@pytest.mark.parametrize("name", ["mixtral_fp8_small", "deepseek_fp8_small"])
def test_fp8_staged_calls_match_layer(name):
    w = FP8[name]
    x = I.make_inputs(w, seed=4, device=DEV)
    cfg, g = L.run_layer(w, x)
    d = fp8_dispatch(w, cfg, x, g["topk_idx"])
    rows = B.max_rows(cfg)
    W8g, sg, W8u, su = L.fp8_weights(x)
    Y = torch.zeros((rows, w.h), dtype=torch.bfloat16, device=DEV)
    B.moe_expert_ffn_fp8(cfg, d["X8"], d["x_scale"], d["offset"], W8g, sg, W8u, su, x["W_down"], Y)
    out = torch.empty((w.T, w.h), dtype=torch.bfloat16, device=DEV)
    B.moe_combine(cfg, x["U"], Y, d["slot"], g["topk_gate"], out)
    torch.cuda.synchronize()
    n = int(d["offset"][-1])
    assert torch.equal(Y[:n], g["Y"][:n])
    assert torch.equal(out, g["out"])


def test_fp8_full_size_mixtral():
    w = I.WORKLOADS["mixtral_fp8"]
    L.log(f"[fp8 full] {w}")
    x = I.make_inputs(w, seed=0, device=DEV)
    cfg, g = L.run_layer(w, x)
    r = L.check_routing_shared_logits(w, g)
    L.check_stats(w, g, r)
    d = fp8_dispatch(w, cfg, x, g["topk_idx"])
    rows = int(r["offset"][-1])
    U = L.f64(x["U"].cpu())
    # FP8 rows of every dispatched row, then Y on sampled rows of a few experts
    qo, so = O.quantize_rows_fp8(U[r["row_token"]])
    np.testing.assert_array_equal(decode(d["X8"][:rows]), qo)
    np.testing.assert_array_equal(d["x_scale"][:rows].cpu().double().numpy(), so)
    W8g, sg, W8u, su = L.fp8_weights(x)
    Yg = L.f64(g["Y"][:rows])
    # every row of the expert with the most rows, sampled rows of others
    kept = L.to_np(g["kept"])
    e_big = int(np.argmax(kept))
    picks = [(e_big, list(range(int(r["offset"][e_big]), int(r["offset"][e_big + 1]))))]
    picks += [(e, rws) for e, rws in L.sampled_expert_rows(r, w.E) if e != e_big]
    worst = 0.0
    for e, rws in picks:
        Wg = decode(W8g[e]) * sg[e].cpu().double().numpy()[:, None]
        Wu = decode(W8u[e]) * su[e].cpu().double().numpy()[:, None]
        Wd = L.f64(x["W_down"][e])
        xr = qo[rws] * so[rws][:, None]
        ref = O.swiglu_expert(xr, Wg, Wu, Wd)
        worst = max(worst, L.check_close(Yg[rws], ref, L.out_tol(w), f"Y of expert {e}")["elem"])
    # combine on every token from the GPU's expert outputs
    out_ref = O.combine(U, Yg, r["slot"], r["gate"])
    eo = L.check_close(L.to_np(g["out"]), out_ref, L.out_tol(w), "out")
    L.check_delta(w, L.f64(g["out"]), U, out_ref)
    L.log(f"  fp8 full ok: Y(expert {e_big} whole, sampled others)={worst:.2e} out={eo}")
