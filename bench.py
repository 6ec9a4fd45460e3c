#!/usr/bin/env python3
"""Throughput of the LRMoE backward hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident in HBM:
lrm_plan_quotas -> lrm_score -> lrm_select -> lrm_compact -> lrm_grouped_dw_dx (both FC2
gradients; --separate-gemms: lrm_grouped_dw -> lrm_grouped_dx).  --overlap runs the score in its
two halves instead: lrm_score_norms on a second stream beside lrm_plan_quotas (it needs neither
the routing nor the layout), then lrm_score_combine once both are done.  The rest of the expert
backward over the same retained rows (activation, FC1 gradients, return to the tokens) is timed
after it as its own leg ("layer_backward"), outside the step.

Default workload: the GLM4.5-106B-A12B-shaped share of one GPU (128 experts, 16 local, top-8,
32768 tokens, h=4096, d_ffn=1408, bf16, retention rho = 0.5), the largest single-GPU workload.

Timing protocol: the step is captured once in a HIP graph; W warm-up replays, then K timed
replays, each bracketed by its own HIP events on the launch stream, with a 1 GiB buffer written
between replays (outside the events) so that no input is served from the 256 MB last-level cache;
the line reports the mean (value, ms_per_step) and the median / p10 / p90 of the K replays.  Stage
times come from a separate eager pass with events between the calls (same flush).  The line also
carries a plain device copy timed the same way (the bandwidth a streaming kernel reaches here),
the graphics clock sampled while the GEMMs run (MFMA fractions are given against the 2.4 GHz spec
peak and against that clock), further legs on the Qwen3-30B-A3B share and the extreme-skew sweep,
and the oracle timed on the host cores (all of them, and one).

Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config 2] [--no-cpu-baseline]
                  [--criterion lrm|grad_sq|grad_abs|random] [--quota cap|proportional|waterfill]
                  [--no-legs] [--flush-mib 1024]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "pairs/s thru LRM score+select+compact+grouped dW/dφ GEMM; % bf16 MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense matrix-core peaks, TFLOP/s
SPEC_CLOCK_MHZ = 2400.0        # the clock those peaks assume

STAGES_FUSED = ("plan", "score", "select", "compact", "gemm")
STAGES_SPLIT = ("plan", "score", "select", "compact", "dw", "dx")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--criterion", default="lrm", choices=["lrm", "grad_sq", "grad_abs", "random"],
                    help="selection score: the LRM, or one of the ablation criteria")
    ap.add_argument("--quota", default="cap", choices=["cap", "proportional", "waterfill"],
                    help="quota split of the retained total")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replays of a captured HIP graph")
    ap.add_argument("--overlap", action="store_true",
                    help="lrm_score_norms on a second stream beside lrm_plan_quotas, then "
                         "lrm_score_combine, instead of lrm_score after the plan")
    ap.add_argument("--separate-gemms", action="store_true",
                    help="lrm_grouped_dw then lrm_grouped_dx instead of lrm_grouped_dw_dx")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-experts", type=int, default=16)
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="repeat the oracle sample until at least this much CPU time has passed")
    ap.add_argument("--rho1-steps", type=int, default=None,
                    help="timed steps of the full-retention pass (default steps/2; 0 skips it)")
    ap.add_argument("--layer-steps", type=int, default=None,
                    help="timed steps of the rest of the expert backward (activation, FC1, return "
                         "to the tokens) on the retained rows (default steps/2; 0 skips it)")
    ap.add_argument("--copy-calibration-mib", type=int, default=1024,
                    help="after timing, copy a buffer of this size once (a plain copy kernel of "
                         "known traffic, to scale rocprofv3 FETCH_SIZE/WRITE_SIZE); 0 skips it")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="size of the buffer written between timed steps (0: back to back)")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the Qwen3-share leg and the extreme-skew retention sweep")
    ap.add_argument("--leg-steps", type=int, default=20,
                    help="timed steps of each extra leg")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the graphics clock while the GEMMs run")
    ap.add_argument("--cpu-one-core-seconds", type=float, default=8.0,
                    help="the oracle's one-core run: repeat its sample until this much time has "
                         "passed (0 skips it)")
    return ap.parse_args()


def algorithmic(w, oracle_like, criterion="lrm"):
    """Algorithmic bytes / flops of each stage (what the method must move or compute)."""
    sp = w.spec
    b = 2 if sp.dtype == "bf16" else 4
    L, K = oracle_like["L"], oracle_like["K"]
    k = sp.k
    loc = (w.topk_idx >= sp.e_lo) & (w.topk_idx < sp.e_lo + sp.E_loc)
    T_loc = int(np.unique(np.flatnonzero(loc) // k).size)
    T_ret = oracle_like["T_ret"]
    Ke = oracle_like["Ke"]
    h, d, E_loc = sp.h, sp.d, sp.E_loc
    score = {"lrm": T_loc * h * b + L * d * b + 12 * L,      # g rows, phi rows, alpha/map/score
             "grad_sq": T_loc * h * b + 8 * L,               # g rows, map/score
             "grad_abs": T_loc * h * b + 8 * L,
             "random": 12 * L}[criterion]                    # map, key, score
    return {
        "plan": 4 * sp.T * k + 4 * L + 16 * E_loc,
        "score": score,
        "select": 4 * L + 4 * K,
        "compact": 16 * K + T_ret * h * b + K * d * b + K * (h + d) * b,
        "dw": K * (h + d) * b + 4 * E_loc * h * d,
        "dx": K * h * b + int((Ke > 0).sum()) * h * d * b + 4 * K * d,
        "flops_dw": 2 * K * h * d,
        "flops_dx": 2 * K * h * d,
    }


def gpu_bench(w, pol_dict, steps, warmup, criterion="lrm", fused=True, graph=True, overlap=False,
              flush=None, gemm_clock=False):
    """Time the path on workload `w` under quota policy `pol_dict`.  Returns (mean ms per step,
    stage ms, info) with info holding L, K, per-expert K, per-step times and (gemm_clock) the
    graphics clock sampled while the one-launch GEMM runs."""
    if flush is None:
        flush = make_flush(0)
    import torch
    from backward_token_expert_amd import lrm, path
    from backward_token_expert_amd.path import to_device, to_host
    sp = w.spec
    L_cap = sp.T * min(sp.k, sp.E_loc)
    P = lrm.make_problem(sp.T, sp.k, sp.E, sp.e_lo, sp.E_loc, sp.h, sp.d, sp.dtype, L_cap, L_cap)
    pol = lrm.make_policy(pol_dict["full"], pol_dict["rho_num"], pol_dict["rho_den"],
                          pol_dict["cap_abs"], pol_dict.get("kind", "cap"))
    phi = w.phi
    if phi.shape[0] < L_cap:
        phi = np.concatenate([phi, np.zeros((L_cap - phi.shape[0], sp.d), phi.dtype)])
    idx, tw, g, ph, W = (to_device(a) for a in (w.topk_idx, w.topk_w, w.g, phi, w.W))
    keys = to_device(synth_keys(sp)) if criterion == "random" else None
    b = path.DeviceBuffers(P)
    stages = STAGES_FUSED if fused else STAGES_SPLIT
    split = overlap and criterion == "lrm"
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    # With stage events (ev) the two score halves run one after the other on s, so that every
    # stage has its own time; without, the norm half runs on the side stream beside the plan.
    def step(ev=None, s=None):
        s = torch.cuda.current_stream() if s is None else s
        if ev is not None:
            ev[0].record(s)
        if split and ev is None:
            fork.record(s)
            side.wait_event(fork)
            lrm.lrm_score_norms(P, g, ph, b.ws, side)
            join.record(side)
        lrm.lrm_plan_quotas(P, pol, idx, b.counts, b.fwd_off, b.row_pair, b.quota, b.cmp_off, b.ws, s)
        if ev is not None:
            ev[1].record(s)
        if split:
            if ev is None:
                s.wait_event(join)
            else:
                lrm.lrm_score_norms(P, g, ph, b.ws, s)
            lrm.lrm_score_combine(P, tw, b.row_pair, b.fwd_off, b.score, b.ws, s)
        elif criterion == "lrm":
            lrm.lrm_score(P, tw, g, ph, b.row_pair, b.fwd_off, b.score, b.ws, s)
        else:
            lrm.lrm_score_criterion(P, criterion, tw, g, ph, keys, b.row_pair, b.fwd_off, b.score,
                                    b.ws, s)
        if ev is not None:
            ev[2].record(s)
        lrm.lrm_select(P, b.score, b.fwd_off, b.quota, b.cmp_off, b.sel_row, b.ws, s)
        if ev is not None:
            ev[3].record(s)
        lrm.lrm_compact(P, b.sel_row, b.row_pair, b.cmp_off, tw, g, ph, b.Gc, b.Phic, b.sel_pair,
                        b.ws, s)
        if ev is not None:
            ev[4].record(s)
        if fused:
            lrm.lrm_grouped_dw_dx(P, b.Gc, b.Phic, W, b.cmp_off, b.dW, b.dphi, b.ws, s)
        else:
            lrm.lrm_grouped_dw(P, b.Gc, b.Phic, b.cmp_off, b.dW, b.ws, s)
            if ev is not None:
                ev[5].record(s)
            lrm.lrm_grouped_dx(P, b.Gc, W, b.cmp_off, b.dphi, b.ws, s)
        if ev is not None:
            ev[len(stages)].record(s)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    err = lrm.lrm_read_device_error(b.ws)
    if err:
        raise RuntimeError(f"device error word {err}: {lrm.deverr_names(err)}")
    s = torch.cuda.current_stream()

    # Stage times: eager steps with HIP events between the calls, on the stream the kernels are
    # launched on (the events cost nothing measurable next to the stages); the flush buffer is
    # written before each step, outside its events.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        flush(i)
        step(evs[i])
    torch.cuda.synchronize()
    stage_ms = {st: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
                for j, st in enumerate(stages)}

    # Whole-step time: the step captured once in a HIP graph and replayed (every call of the path
    # is capturable: no allocation, no host synchronisation); --eager times eager launches.
    run_step = step
    g_gemm = None
    if graph:
        g_step = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(s)
        with torch.cuda.stream(cs):
            step(None, cs)
            torch.cuda.synchronize()
            with torch.cuda.graph(g_step, stream=cs):
                step(None, cs)
        torch.cuda.synchronize()
        run_step = g_step.replay
        for _ in range(warmup):
            run_step()
    per, wall = timed_replays(run_step, steps, flush)
    # back to back (no flush), for comparison only
    per_warm, _ = timed_replays(run_step, steps, None)
    err = lrm.lrm_read_device_error(b.ws)
    if err:
        raise RuntimeError(f"device error word {err}: {lrm.deverr_names(err)}")
    fo = to_host(b.fwd_off)
    co = to_host(b.cmp_off)
    sel_pair = to_host(b.sel_pair)[:int(co[-1])]
    info = {"L": int(fo[-1]), "K": int(co[-1]), "Ke": np.diff(co),
            "T_ret": int(np.unique(sel_pair // sp.k).size),
            "step_ms": per, "warm_step_ms": per_warm, "wall_ms": wall}
    if gemm_clock and fused:
        info["clock"] = gemm_clock_sample(
            lambda st: lrm.lrm_grouped_dw_dx(P, b.Gc, b.Phic, W, b.cmp_off, b.dW, b.dphi, b.ws, st),
            stage_ms["gemm"])
    return float(np.mean(per)), stage_ms, info


def make_flush(mib):
    """A callable that writes a `mib` MiB buffer on the current stream (nothing for 0)."""
    if mib <= 0:
        return lambda i: None
    import torch
    buf = torch.empty(mib << 18, dtype=torch.float32, device="cuda")
    return lambda i: buf.fill_(float(i))


def timed_replays(run_step, steps, flush):
    """`steps` runs of `run_step`, each bracketed by its own HIP events on the current stream,
    the flush (if any) written between them outside the events.  Returns the per-step times
    (ms) and the host wall time per step (ms, flush included)."""
    import torch
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush(i)
        ev[i][0].record(s)
        run_step()
        ev[i][1].record(s)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    return [a.elapsed_time(b) for a, b in ev], wall


def step_stats(per):
    return {"mean": float(np.mean(per)), "median": float(np.median(per)),
            "p10": float(np.percentile(per, 10)), "p90": float(np.percentile(per, 90)),
            "n": len(per)}


def gemm_clock_sample(launch, ms_per_call, seconds=1.0):
    """The graphics clock and the socket power while the one-launch GEMM runs back to back for
    about `seconds`: amdsmi is polled from a second thread while the host waits for the GPU.
    Returns {"MHz_median", "socket_W_median", "power_cap_W", "samples", "source", ...} or
    {"error": ...} where amdsmi is unavailable."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        h = handles[0]
        if len(handles) > 1:                     # match the device torch uses by PCI address
            want = torch.cuda.get_device_properties(0)
            bus = getattr(want, "pci_bus_id", None)
            for x in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(x)
                if bus is not None and int(bdf.split(":")[1], 16) == bus:
                    h = x
    except Exception as e:  # noqa: BLE001
        return {"error": f"amdsmi unavailable: {type(e).__name__}: {e}"[:200]}

    cap_w = None
    try:
        c = amdsmi.amdsmi_get_power_cap_info(h)
        if isinstance(c, dict) and isinstance(c.get("power_cap"), (int, float)) and c["power_cap"] > 0:
            cap_w = float(c["power_cap"]) / 1e6          # reported in microwatts
    except Exception:  # noqa: BLE001
        pass
    power = []

    def read():
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            pw = m.get("current_socket_power")
            if isinstance(pw, (int, float)) and 0 < pw < 10000:
                power.append(float(pw))
            for key in ("current_gfxclks", "current_gfxclk", "average_gfxclk_frequency"):
                v = m.get(key)
                if isinstance(v, (list, tuple)):
                    v = [x for x in v if isinstance(x, (int, float)) and 0 < x < 10000]
                    if v:
                        return float(np.mean(v)), key
                elif isinstance(v, (int, float)) and 0 < v < 10000:
                    return float(v), key
        except Exception:  # noqa: BLE001
            pass
        try:
            c = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
            v = c.get("clk") if isinstance(c, dict) else None
            if isinstance(v, (int, float)) and 0 < v < 10000:
                return float(v), "clock_info.clk"
        except Exception:  # noqa: BLE001
            pass
        return None

    samples, src = [], set()
    stop = threading.Event()

    def poll():
        while not stop.is_set():
            r = read()
            if r is not None:
                samples.append(r[0])
                src.add(r[1])
            time.sleep(0.005)

    n = max(10, int(seconds * 1e3 / max(ms_per_call, 1e-3)))
    s = torch.cuda.current_stream()
    torch.cuda.synchronize()
    for _ in range(3):
        launch(s.cuda_stream)
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    for _ in range(n):
        launch(s.cuda_stream)
    torch.cuda.synchronize()
    stop.set()
    th.join(timeout=2.0)
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    if not samples:
        return {"error": "no clock readings"}
    # drop the first readings (the launches ramp up) and take the median
    use = samples[len(samples) // 5:] or samples
    pw = power[len(power) // 5:] or power
    return {"MHz_median": float(np.median(use)), "MHz_p10": float(np.percentile(use, 10)),
            "MHz_p90": float(np.percentile(use, 90)), "samples": len(use), "source": sorted(src),
            "calls": n, "socket_W_median": float(np.median(pw)) if pw else None,
            "power_cap_W": cap_w}


LAYER_STAGES = ("swiglu", "gather", "fc1_gemm", "scatter")


def layer_algorithmic(w, info):
    """Algorithmic bytes / flops of the rest of the expert backward over K retained rows."""
    sp = w.spec
    b = 2 if sp.dtype == "bf16" else 4
    K, T_ret, Ke = info["K"], info["T_ret"], info["Ke"]
    h, d = sp.h, sp.d
    return {
        "swiglu": 4 * K + 4 * K * d + 2 * K * d * b + 2 * K * d * b,   # sel_row, dphi, [a|c], dH
        "gather": 8 * K + T_ret * h * b + K * h * b,                    # ids, x once per token, Xc
        "fc1_dw": K * (2 * d + h) * b + 4 * sp.E_loc * 2 * d * h,
        "fc1_dx": K * 2 * d * b + int((Ke > 0).sum()) * 2 * d * h * b + 4 * K * h,
        "scatter": 8 * K + 4 * K * h + 4 * sp.T * h,                    # ids, dX rows, dx rows
        "flops_fc1": 8 * K * h * d,                                     # 2 products, 2*K*(2d)*h
    }


def layer_bench(w, pol_dict, steps, warmup, criterion="lrm"):
    """Time the rest of the expert backward after one pass of the path: lrm_swiglu_backward,
    lrm_gather_tokens, lrm_grouped_fc1_dw_dx, lrm_scatter_tokens, stage by stage."""
    import torch
    import synth
    from backward_token_expert_amd import lrm, path
    from backward_token_expert_amd.path import to_device, to_host
    sp = w.spec
    L_cap = sp.T * min(sp.k, sp.E_loc)
    P = lrm.make_problem(sp.T, sp.k, sp.E, sp.e_lo, sp.E_loc, sp.h, sp.d, sp.dtype, L_cap, L_cap)
    pol = lrm.make_policy(pol_dict["full"], pol_dict["rho_num"], pol_dict["rho_den"],
                          pol_dict["cap_abs"], pol_dict.get("kind", "cap"))
    li = synth.layer_inputs(w)
    pad = lambda a: a if a.shape[0] >= L_cap else np.concatenate(  # noqa: E731
        [a, np.zeros((L_cap - a.shape[0], a.shape[1]), a.dtype)])
    idx, tw, g, ph, W = (to_device(a) for a in (w.topk_idx, w.topk_w, w.g, pad(w.phi), w.W))
    ac, x, W1 = to_device(pad(li.ac)), to_device(li.x), to_device(li.W1)
    keys = to_device(synth_keys(sp)) if criterion == "random" else None
    b = path.DeviceBuffers(P)
    lay = path.LayerBuffers(P)
    s = torch.cuda.current_stream()
    path.run(P, pol, idx, tw, g, ph, W, b, s, criterion=criterion, keys=keys)

    def step(ev=None):
        calls = (lambda: lrm.lrm_swiglu_backward(P, b.sel_row, b.cmp_off, b.dphi, ac, lay.dH, b.ws, s),
                 lambda: lrm.lrm_gather_tokens(P, b.sel_pair, b.cmp_off, x, lay.Xc, b.ws, s),
                 lambda: lrm.lrm_grouped_fc1_dw_dx(P, lay.dH, lay.Xc, W1, b.cmp_off, lay.dW1,
                                                   lay.dX, b.ws, s),
                 lambda: lrm.lrm_scatter_tokens(P, b.sel_pair, b.cmp_off, lay.dX, lay.dx, b.ws, s))
        for j, c in enumerate(calls):
            if ev is not None:
                ev[j].record(s)
            c()
        if ev is not None:
            ev[len(calls)].record(s)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    err = lrm.lrm_read_device_error(b.ws)
    if err:
        raise RuntimeError(f"device error word {err}: {lrm.deverr_names(err)}")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(LAYER_STAGES) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    stage_ms = {st: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
                for j, st in enumerate(LAYER_STAGES)}
    co = to_host(b.cmp_off)
    sel_pair = to_host(b.sel_pair)[:int(co[-1])]
    info = {"K": int(co[-1]), "Ke": np.diff(co), "T_ret": int(np.unique(sel_pair // sp.k).size)}
    a = layer_algorithmic(w, info)
    t_mem = (stage_ms["swiglu"] + stage_ms["gather"] + stage_ms["scatter"]) * 1e-3
    by = a["swiglu"] + a["gather"] + a["scatter"]
    t_g = stage_ms["fc1_gemm"] * 1e-3
    return {"calls": ["lrm_swiglu_backward", "lrm_gather_tokens", "lrm_grouped_fc1_dw_dx",
                      "lrm_scatter_tokens"],
            "steps": steps, "ms_per_step": float(sum(stage_ms.values())),
            "K_retained": info["K"], "stages_ms": stage_ms,
            "swiglu_gather_scatter_GBps": by / t_mem / 1e9,
            "swiglu_gather_scatter_hbm_frac": by / t_mem / 1e9 / HBM_PEAK_GBS,
            "fc1_TFLOPs": a["flops_fc1"] / t_g / 1e12,
            "fc1_mfma_frac": a["flops_fc1"] / t_g / 1e12 / MFMA_PEAK_TFLOPS[sp.dtype]}


def admission_bench(w, steps):
    """Time lrm_admit_quotas: six candidates (full retention, then rho = 1, 3/4, 1/2, 1/4, 1/8 of
    the cap form) against an HBM budget sized, from the GPU's own quotas under the workload's
    policy, to admit exactly the workload's rho."""
    import torch
    from backward_token_expert_amd import lrm, path
    from backward_token_expert_amd.path import to_device, to_host
    sp = w.spec
    L_cap = sp.T * min(sp.k, sp.E_loc)
    P = lrm.make_problem(sp.T, sp.k, sp.E, sp.e_lo, sp.E_loc, sp.h, sp.d, sp.dtype, L_cap, L_cap)
    b = path.DeviceBuffers(P)
    s = torch.cuda.current_stream()
    idx = to_device(w.topk_idx)
    own = lrm.make_policy(0, sp.rho_num, sp.rho_den, sp.cap_abs)
    lrm.lrm_plan_quotas(P, own, idx, b.counts, b.fwd_off, b.row_pair, b.quota, b.cmp_off, b.ws, s)
    torch.cuda.synchronize()
    K_own = int(to_host(b.cmp_off)[-1])
    rates = [(1, 1, 1), (0, 1, 1), (0, 3, 4), (0, 1, 2), (0, 1, 4), (0, 1, 8)]
    el = 2 if sp.dtype == "bf16" else 4
    row = (sp.h + sp.d) * el + 4 * sp.d + 8          # Gc, Phic, dphi, row ids per retained row
    adm = lrm.make_admission(rates, mem_budget=(1 << 30) + K_own * row, mem_base=1 << 30,
                             mem_per_row=row, cap_abs=sp.cap_abs)
    for _ in range(3):
        lrm.lrm_admit_quotas(P, adm, b.fwd_off, b.quota, b.cmp_off, b.admitted, b.ws, s)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(steps):
        lrm.lrm_admit_quotas(P, adm, b.fwd_off, b.quota, b.cmp_off, b.admitted, b.ws, s)
    e1.record(s)
    torch.cuda.synchronize()
    return {"call": "lrm_admit_quotas", "candidates": len(rates),
            "admitted": int(to_host(b.admitted)[0]), "K_retained": int(to_host(b.cmp_off)[-1]),
            "K_budgeted": K_own, "us_per_call": e0.elapsed_time(e1) / steps * 1e3}


def synth_keys(sp):
    import synth
    return synth.pair_keys(sp)


def host_cpu():
    """Model name and the number of host cores this process may run on."""
    model = None
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count()
    return {"model": model, "cores_available": n}


def cpu_baseline(w, pol_dict, n_experts, min_seconds, criterion="lrm", threads=None):
    """The oracle, as it stands, on a bounded sample: all counting/planning plus scoring,
    selection, compaction and both GEMMs of the first `n_experts` local experts, repeated until
    `min_seconds` have passed (at least once); the rate is over all repetitions.  `threads`
    limits the BLAS thread pool (None: as configured)."""
    import contextlib
    import oracle as O
    sp = w.spec
    keys = synth_keys(sp) if criterion == "random" else None
    try:
        import threadpoolctl
        limit = (threadpoolctl.threadpool_limits(threads) if threads is not None
                 else contextlib.nullcontext())
    except Exception:  # noqa: BLE001
        threadpoolctl, limit = None, contextlib.nullcontext()

    def once():
        n = O.routed_counts(w.topk_idx, sp.E)
        row_pair, fwd_off = O.forward_layout(w.topk_idx, sp.e_lo, sp.E_loc)
        quota, cmp_off = O.plan_quotas(n[sp.e_lo:sp.e_lo + sp.E_loc], pol_dict)
        ne = min(n_experts, sp.E_loc)
        rows = slice(0, int(fwd_off[ne]))
        R = O.scores(criterion, w.topk_w, w.g, w.phi[rows], row_pair[rows], sp.k, sp.dtype, keys)
        sel = O.select_top_quota(R.astype(np.float32), fwd_off[:ne + 1], quota[:ne], row_pair)
        Gc, Phic, _ = O.compact(sel, row_pair, w.topk_w, w.g, w.phi, sp.k, sp.dtype)
        off = cmp_off[:ne + 1]
        O.grouped_dw(Gc, Phic, off, sp.dtype)
        O.grouped_dx(Gc, w.W[:ne], off, sp.dtype)
        return ne, int(fwd_off[ne]), int(off[-1])

    with limit:
        used = None
        if threadpoolctl is not None:
            info = threadpoolctl.threadpool_info()
            used = max((i.get("num_threads", 1) for i in info), default=None)
        t0 = time.perf_counter()
        reps = 0
        while True:
            ne, pairs, kept = once()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    return {"value": reps * pairs / dt, "unit": "pairs/s", "cores": used or os.cpu_count(),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle: counts/layout/quotas over all {sp.T * sp.k} pairs, "
                      f"then score/select/compact/dW/dphi for local experts 0..{ne - 1} "
                      f"({pairs} routed pairs, {kept} retained); {reps} repetition(s) in "
                      f"{dt:.1f} s"}


def recorded_counters(call, workload):
    """The committed rocprofv3 counter record (profiles/*.md, `traffic-record:` lines) of `call`'s
    kernel on `workload` -- HBM bytes per launch, the clock during the kernel, MFMA busy -- or
    None when no record matches the workload and the current sources of the kernel."""
    import glob
    from backward_token_expert_amd.rocprof_summary import source_digest
    here = os.path.dirname(os.path.abspath(__file__))
    digest = source_digest(call)
    for f in sorted(glob.glob(os.path.join(here, "profiles", "*.md"))):
        for line in open(f, encoding="utf-8"):
            if not line.startswith("traffic-record: "):
                continue
            rec = json.loads(line[len("traffic-record: "):])
            k = rec.get("kernels", {}).get(call)
            if rec.get("workload") == workload and k and k.get("source_sha256") == digest:
                return k
    return None


def recorded_traffic(call, workload):
    """HBM bytes per launch of `call`'s kernel from the committed counter record, or None."""
    k = recorded_counters(call, workload)
    return None if k is None else k["traffic_bytes"]


def fractions(st, a, dtype, clock_mhz=None):
    """HBM fraction of score+select+compact and MFMA fraction of the GEMMs from stage times."""
    t_ssc = (st["score"] + st["select"] + st["compact"]) * 1e-3
    by = a["score"] + a["select"] + a["compact"]
    t_g = (st["gemm"] if "gemm" in st else st["dw"] + st["dx"]) * 1e-3
    fl = a["flops_dw"] + a["flops_dx"]
    out = {"score_select_compact_GBps": by / t_ssc / 1e9,
           "score_select_compact_hbm_frac": by / t_ssc / 1e9 / HBM_PEAK_GBS,
           "gemms_TFLOPs": fl / t_g / 1e12,
           "gemms_mfma_frac": fl / t_g / 1e12 / MFMA_PEAK_TFLOPS[dtype],
           # the GEMMs' algorithmic bytes per second: the bound when the dW stores dominate
           "gemms_GBps": (a["dw"] + a["dx"]) / t_g / 1e9}
    if clock_mhz:
        out["gemms_mfma_frac_at_measured_clock"] = (
            fl / t_g / 1e12 / (MFMA_PEAK_TFLOPS[dtype] * clock_mhz / SPEC_CLOCK_MHZ))
    return out


def leg(w, pol, steps, warmup, crit, fused, graph, flush, label):
    """One extra timed workload / policy: value, per-step statistics, stages and fractions."""
    ms, stages, info = gpu_bench(w, pol, steps, warmup, crit, fused, graph, False, flush)
    alg = algorithmic(w, info, crit)
    return {"workload": w.spec.name, "policy": label, "value": info["L"] / (ms * 1e-3),
            "unit": "pairs/s", "ms_per_step": ms, "step_ms": step_stats(info["step_ms"]),
            "L_pairs": info["L"], "K_retained": info["K"],
            "retained_rows_per_s": info["K"] / (ms * 1e-3), "stages_ms": stages,
            "fractions": fractions(stages, alg, w.spec.dtype)}


def copy_ceiling(flush, mib=1024, reps=10):
    """A plain device-to-device copy of `mib` MiB timed like the step (events around each copy,
    the flush between copies): bytes read + written per second; and a fill of the same buffer,
    the write-only rate."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    per, _ = timed_replays(lambda: dst.copy_(src), reps, flush)
    fill, _ = timed_replays(lambda: dst.fill_(2.0), reps, flush)
    del src, dst
    med, fmed = float(np.median(per)), float(np.median(fill))
    return {"GBps": 2 * n / (med * 1e-3) / 1e9, "bytes_moved": 2 * n, "median_ms": med,
            "kernel": "torch copy_ (device to device)",
            "fill_GBps": n / (fmed * 1e-3) / 1e9, "fill_median_ms": fmed,
            "fill_kernel": "torch fill_ (writes only)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU; --gpus must be 1 (sharding across GPUs is not implemented)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import synth
    w = synth.make(args.config)
    sp = w.spec
    pol = synth.policy(sp, kind=args.quota, cap=-1 if args.quota == "proportional" else None)
    crit = args.criterion
    fused = not args.separate_gemms
    overlap = args.overlap
    graph = not args.eager
    flush = make_flush(args.flush_mib)
    ms, stages, info = gpu_bench(w, pol, args.steps, args.warmup, crit, fused, graph, overlap,
                                 flush, gemm_clock=not args.no_clock)
    alg = algorithmic(w, info, crit)
    L, K = info["L"], info["K"]
    clock = info.get("clock") or {}
    clk = clock.get("MHz_median")
    # rho = 1 (full retention) on the same input
    n1 = max(3, args.steps // 2) if args.rho1_steps is None else args.rho1_steps
    if n1 > 0:
        pol_full = synth.policy(sp, full=True)
        ms1, stages1, info1 = gpu_bench(w, pol_full, n1, 2, crit, fused, graph, overlap, flush)
        alg1 = algorithmic(w, info1, crit)

    if fused:
        dom_call = "lrm_grouped_dw_dx"
        ach = (alg["flops_dw"] + alg["flops_dx"]) / (stages["gemm"] * 1e-3) / 1e12
    else:
        dom = max(("dw", "dx"), key=lambda s: stages[s])
        dom_call = {"dw": "lrm_grouped_dw", "dx": "lrm_grouped_dx"}[dom]
        ach = alg["flops_" + dom] / (stages[dom] * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[sp.dtype]
    rec = recorded_counters(dom_call, sp.name)
    roof = {"bound": "mfma", "kernel": dom_call, "achieved": ach, "peak": peak,
            "unit": "TFLOP/s", "frac": ach / peak,
            "traffic": None if rec is None else rec["traffic_bytes"]}
    # the clock during this kernel: from its counter record (GPU cycles / duration), else the
    # clock amdsmi reported while it ran
    if rec is not None and rec.get("clock_mhz"):
        clk, clk_src = rec["clock_mhz"], "rocprofv3 GRBM_GUI_ACTIVE / duration (profiles/)"
    else:
        clk_src = "amdsmi current_gfxclks while the kernel ran" if clk else None
    if clk:
        roof["frac_at_measured_clock"] = ach / (peak * clk / SPEC_CLOCK_MHZ)
        roof["measured_clock_MHz"] = clk
        roof["clock_source"] = clk_src
    out = {
        "metric": METRIC,
        "value": L / (ms * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sp.dtype,
        "data": "synthetic",
        "config": {"workload": sp.name, "T": sp.T, "top_k": sp.k, "experts": sp.E,
                   "local_experts": sp.E_loc, "h": sp.h, "d_ffn": sp.d,
                   "rho": f"{pol['rho_num']}/{pol['rho_den']}", "quota": args.quota,
                   "criterion": crit, "L_pairs": L, "K_retained": K},
        "roofline": roof,
        "step_ms": step_stats(info["step_ms"]),
        "step_ms_back_to_back": step_stats(info["warm_step_ms"]),
        "retained_rows_per_s": K / (ms * 1e-3),
        "timing": ("eager launches" if args.eager else "replays of one captured HIP graph") +
                  (f"; {args.flush_mib} MiB written between timed steps" if args.flush_mib > 0
                   else "; back to back"),
        "overlap": ("lrm_score_norms on a second stream beside lrm_plan_quotas; stage times from "
                    "eager steps with the two halves in sequence") if overlap and crit == "lrm"
                   else None,
        "wall_ms_per_step": info["wall_ms"],
        "stages_ms": stages,
        "fractions": fractions(stages, alg, sp.dtype, clk),
        "gpu_clock": clock or None,
    }
    if n1 > 0:
        out["rho1"] = {"value": info1["L"] / (ms1 * 1e-3), "ms_per_step": ms1,
                       "step_ms": step_stats(info1["step_ms"]),
                       "K_retained": info1["K"], "stages_ms": stages1,
                       "fractions": fractions(stages1, alg1, sp.dtype, clk)}
    nl = max(3, args.steps // 2) if args.layer_steps is None else args.layer_steps
    if nl > 0:
        out["layer_backward"] = layer_bench(w, pol, nl, 2, crit)
    out["admission"] = admission_bench(w, 20)
    out["copy_ceiling"] = copy_ceiling(flush)
    if not args.no_legs:
        legs = {}
        if args.config != 1:
            w1 = synth.make(1)
            legs["qwen3_share"] = leg(w1, synth.policy(w1.spec), args.leg_steps, 3, "lrm", fused,
                                      graph, flush, "rho 1/2 (cap)")
            legs["qwen3_share_full"] = leg(w1, synth.policy(w1.spec, full=True), args.leg_steps,
                                           3, "lrm", fused, graph, flush, "full retention")
            del w1
        # every other workload at its own retention and at full retention
        for cfg, key in ((0, "fp32_small"), (4, "whole_layer"), (5, "deepseek_v2_share")):
            if cfg == args.config:
                continue
            wc = synth.make(cfg)
            pc = synth.policy(wc.spec)
            own = f"rho {pc['rho_num']}/{pc['rho_den']} (cap)"
            legs[key] = [leg(wc, pc, args.leg_steps, 3, "lrm", fused, graph, flush, own),
                         leg(wc, synth.policy(wc.spec, full=True), args.leg_steps, 3, "lrm",
                             fused, graph, flush, "full retention")]
            del wc
        w3 = synth.make(3)
        sweep = [leg(w3, synth.policy(w3.spec, full=True), args.leg_steps, 3, "lrm", fused,
                     graph, flush, "full retention")]
        for num, den in synth.RHO_SWEEP_3:
            sweep.append(leg(w3, synth.policy(w3.spec, rho=(num, den)), args.leg_steps, 3, "lrm",
                             fused, graph, flush, f"rho {num}/{den} (cap)"))
        legs["extreme_skew_sweep"] = sweep
        del w3
        out["legs"] = legs
    if args.copy_calibration_mib > 0:
        import torch
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, pol, args.cpu_sample_experts, args.cpu_min_seconds, crit)
        cb["host_cpu"] = host_cpu()
        if args.cpu_one_core_seconds > 0:
            one = cpu_baseline(w, pol, 1, args.cpu_one_core_seconds, crit, threads=1)
            cb["one_core"] = {"value": one["value"], "unit": one["unit"], "cores": one["cores"],
                              "sample": one["sample"]}
        out["cpu_baseline"] = cb
    print(json.dumps(out))


if __name__ == "__main__":
    main()
