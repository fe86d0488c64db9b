"""Benchmark of the MoE layer forward on one MI355X.

One step = one moe_layer_forward (router, dispatch, grouped SwiGLU experts,
combine, statistics) over one batch of seeded synthetic tokens whose inputs
are resident in HBM; with --backward, one forward followed by one
moe_layer_backward (a training step of the layer, upstream gradient seeded; the
forward keeps the expert activations for it unless --recompute).
Prints one JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--backward] [--cpu-baseline-seconds S | --no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward (bf16 workloads without FP8)")
    ap.add_argument("--fp8-grad", action="store_true",
                    help="with --backward: the experts' output gradients in FP8 (W_down^T "
                         "quantised once before the timed loop)")
    ap.add_argument("--recompute", action="store_true",
                    help="with --backward: the forward keeps no activations and the backward "
                         "recomputes them")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward captured once in a HIP graph and replayed "
                         "(reported beside the eager figures, never as the value)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes three times (for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--read-calibration", type=int, default=0, metavar="BYTES",
                    help="only time the library's read-stream kernel over BYTES bytes "
                         "(the read rate a plain stream reaches on this device) and exit")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_mixtral_bf16.txt")
GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_layer_37_amd", "csrc", "ffn.hip")


def measured_traffic(workload: str):
    """HBM bytes per launch of the gate/up GEMM from the committed counter summary.

    The summary records the sha256 of the GEMM source it was measured on; when
    the source has changed since, the figure no longer applies and None is
    returned.
    """
    import hashlib
    if workload != "mixtral_bf16" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    with open(GEMM_SOURCE, "rb") as fh:
        sha = hashlib.sha256(fh.read()).hexdigest()
    if kv.get("gemm_source_sha256") != sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stage_bandwidth(w, stage_ms, kept, e_active, eb):
    """Achieved bandwidth of each stage over the bytes it has to move at least.

    Counted per stage (bf16: eb = 2 bytes per element): the router reads U and
    W_r (and W_noise); dispatch reads U and writes the kept rows X; gate/up
    reads X and the active experts' W_gate and W_up and writes the SwiGLU rows
    A; down reads A and W_down and writes Y; combine reads U and Y and writes
    out.  Shared experts add a dense pass over all T tokens to gate/up and
    down.  Index and statistics arrays are left out (under 1% of any stage).
    """
    T, h, f, E = w.T, w.h, w.f, w.E
    ns, fs = w.n_shared, w.f_shared
    e8 = 1 if w.fp8_up else eb  # bytes of a dispatched row element and of W_gate / W_up
    b = {
        "route": eb * (T * h + h * E * (2 if w.noisy else 1)),
        "dispatch": eb * T * h + e8 * kept * h,
        "gate_up": (e8 * (kept * h + 2 * f * h * e_active) + eb * kept * f
                    + eb * ns * (T * h + 2 * fs * h + T * fs)),
        "down": eb * (kept * f + f * h * e_active + kept * h + ns * (T * fs + fs * h + T * h)),
        "combine": eb * (T * h + kept * h + T * h + ns * T * h),
    }
    out = {}
    for n, nbytes in b.items():
        t = stage_ms.get(n, 0.0)
        gbs = nbytes / (t * 1e-3) / 1e9 if t > 0 else 0.0
        out[n] = {"bytes": nbytes, "GB/s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def copy_calibration(nbytes: int):
    import torch
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    # events around each copy (no extra launches, so the counter scaling is
    # unchanged); each copy reads and writes nbytes
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for i in range(3):
        y.copy_(x)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3,
                      "ms": ms, "read_plus_write_GBps": 2 * nbytes / (min(ms) * 1e-3) / 1e9}),
          flush=True)


def read_calibration(nbytes: int):
    """The read rate of a plain stream of 16-byte loads (moe_stream_read) over
    nbytes of device memory, for several grid sizes; the best is the yardstick
    for the weight-read-bound workloads."""
    import torch

    from mixture_experts_layer_37_amd import binding as B
    nbytes -= nbytes % 16
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    x.fill_(3)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(64 * ncu, dtype=torch.int32, device="cuda")
    res = {}
    for per_cu in (2, 4, 8, 16, 32, 64):
        blocks = per_cu * ncu
        B.moe_stream_read(x, sink, blocks)  # warm-up
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record()
        for i in range(5):
            B.moe_stream_read(x, sink, blocks)
            ev[i + 1].record()
        torch.cuda.synchronize()
        ms = min(ev[i].elapsed_time(ev[i + 1]) for i in range(5))
        res[str(blocks)] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    best = max(res.values())
    print(json.dumps({"read_calibration_bytes": nbytes, "read_GBps_by_grid": res,
                      "read_GBps_best": best, "hbm_frac_of_peak": round(best / PEAK_HBM_GBS, 4)}),
          flush=True)


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), for the baseline's record."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, g, budget_s: float) -> dict:
    """The float64 oracle, as it is, on a bounded sample of the same workload.

    Routing (router product, scores, top-k, capacity fill, statistics) runs on
    all T tokens.  With the FP8 up-projection the sampled rows and the sampled
    experts' W_gate and W_up are quantised first (part of the timed work).  The expert products run on whole experts taken in order
    until the time budget is used (each expert's weights converted to float64
    plus its SwiGLU over its rows); combine runs on all tokens.  The time of the
    expert part is scaled by (all kept rows / sampled rows) plus the weight
    conversion of the experts not sampled.
    """
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O

    def f64(t):
        return t.detach().cpu().float().numpy().astype(np.float64)

    t0 = time.perf_counter()
    U = f64(x["U"])
    # the noisy router's draws from the oracle's own counter-based generator
    noise = O.philox_normals(w.T, w.E, w.rng_seed, w.rng_offset) if w.noisy else None
    H = O.router_logits(U, f64(x["W_r"]), None if x["b_r"] is None else f64(x["b_r"]),
                        None if x["W_noise"] is None else f64(x["W_noise"]), noise)
    C = O.capacity(w.T, w.E, w.k, w.capacity_factor)
    r = O.route(H, w.k, w.score, w.gate, C, w.fill,
                None if x.get("b_sel") is None else f64(x["b_sel"]), max(1, w.n_groups),
                max(1, w.topk_groups))
    t_route = time.perf_counter() - t0

    rows_total = int(r["offset"][-1])
    active = [e for e in range(w.E) if r["offset"][e + 1] > r["offset"][e]]
    t_conv, t_ffn, rows_done, experts_done = 0.0, 0.0, 0, 0
    Y = np.zeros((rows_total, w.h))
    for e in active:
        if t_conv + t_ffn > budget_s and experts_done > 0:
            break
        t1 = time.perf_counter()
        Wg, Wu, Wd = f64(x["W_gate"][e]), f64(x["W_up"][e]), f64(x["W_down"][e])
        if w.fp8_up:
            qg, sg = O.quantize_rows_fp8(Wg)
            qu, su = O.quantize_rows_fp8(Wu)
            Wg, Wu = qg * sg[:, None], qu * su[:, None]
        t2 = time.perf_counter()
        a, b = int(r["offset"][e]), int(r["offset"][e + 1])
        # cap the rows of one expert so a single expert stays inside the budget
        n = min(b - a, 1024)
        Xe = U[r["row_token"][a:a + n]]
        if w.fp8_up:
            qx, sx = O.quantize_rows_fp8(Xe)
            Xe = qx * sx[:, None]
        Y[a:a + n] = O.swiglu_expert(Xe, Wg, Wu, Wd)
        t3 = time.perf_counter()
        t_conv += t2 - t1
        t_ffn += t3 - t2
        rows_done += n
        experts_done += 1
    # shared experts: every token, timed on up to 1024 tokens and scaled
    t_sh, n_sh = 0.0, min(w.T, 1024)
    Ys = None
    if w.n_shared > 0:
        t5 = time.perf_counter()
        Ys = np.zeros((w.n_shared, w.T, w.h))
        for i in range(w.n_shared):
            Ys[i, :n_sh] = O.swiglu_expert(U[:n_sh], f64(x["Ws_gate"][i]), f64(x["Ws_up"][i]),
                                           f64(x["Ws_down"][i]))
        t_sh = (time.perf_counter() - t5) * w.T / max(n_sh, 1)
    t4 = time.perf_counter()
    O.combine(U, Y, r["slot"], r["gate"], Ys)
    t_comb = time.perf_counter() - t4
    est = (t_route + t_comb + t_sh + t_conv * len(active) / experts_done
           + t_ffn * rows_total / max(rows_done, 1))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": w.T / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"routing, statistics and combine on all {w.T} tokens; expert SwiGLU on "
                       f"{rows_done} of {rows_total} kept rows from {experts_done} of "
                       f"{len(active)} active experts (float64), scaled by rows"
                       + (f"; {w.n_shared} shared expert(s) on {n_sh} tokens, scaled to {w.T}"
                          if w.n_shared else "")
                       + f"; measured {t_route + t_comb + t_conv + t_ffn:.1f} s, estimated "
                       f"{est:.1f} s per full forward")}


def graph_replay(step, out, steps: int) -> dict:
    """The same forward captured once in a HIP graph and replayed `steps` times.

    Every kernel of the forward is enqueued on the current stream with no
    host synchronisation, memset or allocation, so it can be captured; the
    replays' output is checked bit for bit against an eager forward's first.
    """
    import torch
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out, eager))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return {"ms_per_step": e0.elapsed_time(e1) / steps, "identical_to_eager": same}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.read_calibration:
        read_calibration(args.read_calibration)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    from mixture_experts_layer_37_amd import binding as B
    from mixture_experts_layer_37_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    w = I.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"workload {w}")
    x = I.make_inputs(w, seed=args.seed, device=dev)
    cfg = B.make_config(w)
    ws = B.new_workspace(cfg, B.MOE_WS_LAYER, dev)
    fields = ["kept", "n_dropped", "aux_loss", "maxvio", "z_loss"]
    if args.backward:
        if w.dtype != "bf16" or w.fp8_up:
            print("--backward needs a bf16 workload without FP8", file=sys.stderr)
            sys.exit(2)
        fields += ["logits", "topk_idx", "topk_gate", "slot", "count", "offset"]
        if not args.recompute:  # the forward keeps X, g | u, a and Y for the backward
            fields += list(B.SAVED_FIELDS)
        bws = B.new_workspace(cfg, B.MOE_WS_BACKWARD, dev)
        gen = torch.Generator(device=dev).manual_seed(args.seed + 1)
        dOut = torch.randn((w.T, w.h), generator=gen, device=dev).to(torch.bfloat16)
        grads = {"dU": torch.empty_like(x["U"]), "dW_r": torch.empty((w.h, w.E), device=dev),
                 "db_r": torch.empty((w.E,), device=dev),
                 "dW_gate": torch.empty_like(x["W_gate"]), "dW_up": torch.empty_like(x["W_up"]),
                 "dW_down": torch.empty_like(x["W_down"])}
        extra = {}
        if w.noisy:
            extra = {"W_noise": x["W_noise"], "dW_noise": torch.empty((w.h, w.E), device=dev)}
        if args.fp8_grad:  # a one-time weight preparation, like a model load
            WdT8, sdT = B.moe_quantize_rows_fp8(x["W_down"].transpose(1, 2).contiguous())
            extra.update(W_downT8=WdT8, s_downT=sdT)
        if w.n_shared:
            extra.update(Ws_gate=x["Ws_gate"], Ws_up=x["Ws_up"], Ws_down=x["Ws_down"],
                         dWs_gate=torch.empty_like(x["Ws_gate"]),
                         dWs_up=torch.empty_like(x["Ws_up"]),
                         dWs_down=torch.empty_like(x["Ws_down"]))
    aux = B.alloc_aux(cfg, dev, fields)
    out = torch.empty((w.T, w.h), dtype=I.torch_dtype(w), device=dev)
    nst = B.MOE_NUM_STAGES

    if w.fp8_up:
        # the FP8 weights are prepared once, like a model load (not timed)
        W8g, sg = B.moe_quantize_rows_fp8(x["W_gate"])
        W8u, su = B.moe_quantize_rows_fp8(x["W_up"])

    def step(events=None):
        common = dict(aux=aux, stage_events=None if events is None else events[:nst + 1], ws=ws, b_sel=x["b_sel"],
                      Ws_gate=x["Ws_gate"], Ws_up=x["Ws_up"], Ws_down=x["Ws_down"])
        if w.fp8_up:
            B.moe_layer_forward_fp8(cfg, x["U"], x["W_r"], x["b_r"], x["W_noise"],
                                    W8g, sg, W8u, su, x["W_down"], out, **common)
        else:
            B.moe_layer_forward(cfg, x["U"], x["W_r"], x["b_r"], x["W_noise"],
                                x["W_gate"], x["W_up"], x["W_down"], out, **common)
        if args.backward:
            B.moe_layer_backward(cfg, x["U"], x["W_r"], x["W_gate"], x["W_up"], x["W_down"],
                                 aux["logits"], aux["topk_idx"], aux["topk_gate"], aux["slot"],
                                 aux["count"], aux["offset"], dOut, grads["dU"], grads["dW_r"],
                                 grads["dW_gate"], grads["dW_up"], grads["dW_down"],
                                 db_r=grads["db_r"], alpha=0.01, c_z=1e-3, ws=bws,
                                 saved=(None if args.recompute
                                        else {n: aux[n] for n in B.SAVED_FIELDS}), **extra)
            if events is not None:
                events[-1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_ev = nst + 1 + (1 if args.backward else 0)
    gu = B.STAGE_NAMES.index("gate_up")

    def make_events(every_stage: bool):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
               for _ in range(args.steps)]
        for row in evs:  # create the HIP events outside the timed region
            for e in row:
                e.record()
        if not every_stage:  # the step's ends and the gate/up stage only
            keep = {0, gu, gu + 1, nst, n_ev - 1}
            evs = [[e if j in keep else None for j, e in enumerate(row)] for row in evs]
        return evs

    events = make_events(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # every stage boundary, in a pass of its own after the timed one (the
    # markers between stages are left out of the timed steps)
    all_events = make_events(True)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(all_events[i])
    torch.cuda.synchronize()
    stage_ms = {n: 0.0 for n in B.STAGE_NAMES}
    for evs in all_events:
        for j, n in enumerate(B.STAGE_NAMES):
            stage_ms[n] += evs[j].elapsed_time(evs[j + 1]) / args.steps
    # the roofline's gate/up time comes from the timed steps themselves
    gate_up_ms = sum(evs[gu].elapsed_time(evs[gu + 1]) for evs in events) / args.steps
    ms = elapsed * 1e3 / args.steps
    # per-step times from the events around each step (the first and last
    # stage boundaries, and the backward's end with --backward)
    step_ms = sorted(evs[0].elapsed_time(evs[-1]) for evs in events)
    ms_median = (step_ms[(len(step_ms) - 1) // 2] + step_ms[len(step_ms) // 2]) / 2
    bwd_ms = (sum(evs[nst].elapsed_time(evs[nst + 1]) for evs in events) / args.steps
              if args.backward else None)
    tokens_per_s = w.T * args.steps / elapsed

    kept = int(aux["kept"].sum().item())
    n_drop = int(aux["n_dropped"].item())
    bf16 = w.dtype == "bf16"
    eb = 2 if bf16 else 4
    # algorithmic work: 6 h f FLOPs per kept (token, expert) row, plus
    # 6 h f_shared per token and shared expert; the gate/up stage does 4 h f
    # (4 h f_shared) of it
    f_sh = 6.0 * w.h * w.f_shared * w.T * w.n_shared
    f_exec = 6.0 * w.h * w.f * kept + f_sh
    f_nom = 6.0 * w.h * w.f * w.k * w.T + f_sh
    f_gate_up = 4.0 * w.h * w.f * kept + f_sh * 4.0 / 6.0
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    peak_gu = PEAK_FP8_TFLOPS if w.fp8_up else peak  # the gate/up GEMM's own dtype
    gu_ms = gate_up_ms
    achieved = f_gate_up / (gu_ms * 1e-3) / 1e12
    kept_per_e = aux["kept"].cpu().tolist()
    e_active = sum(1 for c in kept_per_e if c > 0)
    # W_gate and W_up are read as one byte per element on the FP8 path
    ew = 1 if w.fp8_up else eb
    b_alg = (ew * 2.0 * w.h * w.f * e_active + eb * w.h * w.f * e_active
             + eb * (3.0 * w.h * w.f_shared * w.n_shared + 2.0 * w.T * w.h
                     + w.h * w.E * (2 if w.noisy else 1)))

    res = {
        "metric": ("MoE layer fwd+bwd tokens/sec on 1 MI355X" if args.backward
                   else "MoE layer fwd tokens/sec on 1 MI355X"),
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_median": ms_median,
        "ms_min": step_ms[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # FP8: E4M3 operands in the gate/up GEMM, bf16 everywhere else
        "dtype": ("fp8+bf16" if w.fp8_up else "bf16") if bf16 else "f32",
        "data": "synthetic",
        "config": dict({"workload": w.name, "T": w.T, "h": w.h, "f": w.f, "E": w.E, "k": w.k,
                        "score": w.score, "gate": w.gate, "capacity_factor": w.capacity_factor,
                        "noisy": w.noisy, "seed": args.seed},
                       **({"n_groups": w.n_groups, "topk_groups": w.topk_groups}
                          if w.n_groups > 1 else {}),
                       **({"n_shared": w.n_shared, "f_shared": w.f_shared}
                          if w.n_shared else {}),
                       **({"sel_bias_std": w.sel_bias_var ** 0.5} if w.sel_bias_var else {}),
                       **({"fp8_up": True} if w.fp8_up else {})),
        "roofline": {"kernel": "grouped gate/up GEMM + SwiGLU", "bound": "mfma",
                     "achieved": achieved, "peak": peak_gu, "unit": "TFLOP/s",
                     "frac": achieved / peak_gu, "traffic": measured_traffic(w.name)},
        "layer": {"mfma_frac_nominal": f_nom / (ms * 1e-3) / 1e12 / peak,
                  "mfma_frac_exec": f_exec / (ms * 1e-3) / 1e12 / peak,
                  "hbm_frac_alg": b_alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "kept_rows": kept, "dropped": n_drop, "active_experts": e_active,
                  "aux_loss": float(aux["aux_loss"].item()),
                  "maxvio": float(aux["maxvio"].item()),
                  "z_loss": float(aux["z_loss"].item())},
        "stage_ms": stage_ms,
        "stage_gbs": stage_bandwidth(w, stage_ms, kept, e_active, eb),
    }
    if args.graph and not args.backward:
        res["graph"] = graph_replay(step, out, args.steps)
    if args.backward:
        # the backward's products: dgrad 6 h f and wgrad 6 h f per kept row and
        # per token and shared expert (useful); executed adds the recomputed
        # forward products (6 h f per kept row when recomputing, and the shared
        # experts' gate/up, 4 h f_shared per token, always)
        sh = w.h * w.f_shared * w.T * w.n_shared
        useful = 12.0 * w.h * w.f * kept + 12.0 * sh
        executed = useful + (6.0 * w.h * w.f * kept if args.recompute else 0.0) + 4.0 * sh
        res["backward"] = {"ms": bwd_ms, "forward_ms": ms - bwd_ms,
                           "activations": "recomputed" if args.recompute else "kept by the forward",
                           "output_gradients": "fp8" if args.fp8_grad else "bf16",
                           "mfma_frac_useful": useful / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                           "mfma_frac_exec": executed / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    if not args.no_cpu_baseline and not args.backward:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(w, x, aux, args.cpu_baseline_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
