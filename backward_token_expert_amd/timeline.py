"""Per-workgroup timeline of the one-launch GEMMs (lrm_grouped_dw_dx), from a profiling build.

  python -m backward_token_expert_amd.timeline build          # on any host (hipcc)
  python -m backward_token_expert_amd.timeline run --config 2 [--reps 3]   # on the GPU

`build` compiles the library with LRM_TIMELINE defined into _build/timeline/liblrm_timeline.so
(the default liblrm.so is not touched).  In that build each workgroup of gemm_fused records, by
one thread and from the 100 MHz clock, when it starts, when its share of the dW jobs ends, when it
claims each dphi unit and when it exits.  `run` loads that build in place of liblrm.so, runs the
path once on a workload, then times the GEMM call `--reps` times and prints a markdown summary:
kernel span, when the dW shares end (per die), idle tail, and the dphi units' durations, split
into units whose last column sub-tile is dead and the rest.  The timestamps cost one scalar
clock read and one store per event, a few per unit of 100-250 us.  The run also reports which die
and CU each workgroup ran on (the XCC_ID and HW_ID registers, read once at its start) and the
shader clock over its life (s_memtime cycles over the 100 MHz clock's elapsed time).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
OUT_DIR = os.path.join(PKG, "_build", "timeline")
LIB = os.path.join(OUT_DIR, "liblrm_timeline.so")
WGS, WORDS, UNITS = 1024, 64, 28


def build():
    from backward_token_expert_amd import build as B
    os.makedirs(OUT_DIR, exist_ok=True)
    return B.build(out=LIB, defines=("LRM_TIMELINE",), build_dir=OUT_DIR)


def run(cfg: int, reps: int, rho=None):
    if not os.path.exists(LIB):
        raise SystemExit(f"{LIB} is missing: run `python -m backward_token_expert_amd.timeline build`")
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import numpy as np
    import torch
    import synth
    from backward_token_expert_amd import lrm, path
    from backward_token_expert_amd.path import to_device, to_host
    if lrm._LIB is not None and lrm.LIB_PATH != LIB:
        raise SystemExit("the default library is already loaded in this process")
    lrm.LIB_PATH = LIB                       # the binding loads this build instead of liblrm.so
    w = synth.make(cfg)
    sp = w.spec
    L_cap = sp.T * min(sp.k, sp.E_loc)
    P = lrm.make_problem(sp.T, sp.k, sp.E, sp.e_lo, sp.E_loc, sp.h, sp.d, sp.dtype, L_cap, L_cap)
    pol = synth.policy(sp, rho=rho)
    phi = np.concatenate([w.phi, np.zeros((L_cap - w.phi.shape[0], sp.d), w.phi.dtype)])
    idx, tw, g, ph, W = (to_device(a) for a in (w.topk_idx, w.topk_w, w.g, phi, w.W))
    b = path.DeviceBuffers(P)
    for _ in range(3):
        path.run(P, lrm.make_policy(**pol), idx, tw, g, ph, W, b)
    torch.cuda.synchronize()
    lib = lrm.load_library()
    lib.lrm_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.lrm_timeline_read.restype = ctypes.c_int
    co = to_host(b.cmp_off)
    nwg = torch.cuda.get_device_properties(0).multi_processor_count
    tn = (sp.d + 383) // 384 if sp.d >= 384 else None
    rho_opt = f" --rho {pol['rho_num']}/{pol['rho_den']}" if rho is not None else ""
    print(f"# gemm_fused timeline -- {sp.name}, rho {pol['rho_num']}/{pol['rho_den']}\n")
    print(f"Command (R = repository root):\n\n```\npython -m backward_token_expert_amd.timeline build\n"
          f"python -m backward_token_expert_amd.timeline run --config {cfg} --reps {reps}{rho_opt}\n```\n")
    print(f"K = {int(co[-1])}; per-expert K = {np.diff(co).tolist()}; {nwg} workgroups "
          f"(one per CU, dies = workgroup id mod 8). Times in us from the first workgroup's start.\n")
    print("| rep | call (events) | kernel span | dW share ends: min / median / max | exits: min / "
          "median / max | idle tail | dphi units | full-width unit: median (p10-p90) | unit with dead "
          "columns: median |")
    print("|---|---|---|---|---|---|---|---|---|")
    per_die = None
    rows = int(sum((int(k) + 255) // 256 for k in np.diff(co)))

    def col_of(u):
        # the column tile of dphi unit u, as the kernel maps units (blocks of 8 row tiles, rows
        # fastest, for 4 column tiles or more; columns fastest otherwise)
        R = 8 if tn >= 4 else 1
        blk = u // (R * tn)
        within = u - blk * R * tn
        rb = np.minimum(rows - blk * R, R)
        return within // rb

    for rep in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lrm.lrm_grouped_dw_dx(P, b.Gc, b.Phic, W, b.cmp_off, b.dW, b.dphi, b.ws)
        e1.record()
        torch.cuda.synchronize()
        buf = np.zeros(WGS * WORDS, np.uint64)
        if lib.lrm_timeline_read(buf.ctypes.data, buf.size) != 0:
            raise SystemExit("lrm_timeline_read failed")
        t = buf.reshape(WGS, WORDS)[:nwg].astype(np.int64)
        t0 = t[:, 0].min()
        us = lambda x: (x - t0) / 100.0  # noqa: E731
        st, dwe, ex, nu = us(t[:, 0]), us(t[:, 1]), us(t[:, 2]), t[:, 3]
        span = ex.max()
        units = []
        for i in range(nwg):
            n = int(min(nu[i], UNITS))
            for j in range(n):
                ts = us(t[i, 4 + 2 * j])
                te = us(t[i, 4 + 2 * (j + 1)]) if j + 1 < n else ex[i]
                units.append((int(t[i, 5 + 2 * j]), te - ts))
        units = np.array(units) if units else np.zeros((0, 2))
        dead = (col_of(units[:, 0]) == tn - 1) & (sp.d % 384 != 0) if tn else np.zeros(len(units), bool)
        full = units[~dead, 1]
        part = units[dead, 1]
        fmt = lambda a, f: f"{f(a):.0f}" if len(a) else "-"  # noqa: E731
        print(f"| {rep} | {e0.elapsed_time(e1) * 1e3:.0f} | {span:.0f} | {dwe.min():.0f} / "
              f"{np.median(dwe):.0f} / {dwe.max():.0f} | {ex.min():.0f} / {np.median(ex):.0f} / "
              f"{ex.max():.0f} | {np.mean(span - ex) / span:.3f} | {len(units)} | "
              f"{fmt(full, np.median)} ({fmt(full, lambda a: np.percentile(a, 10))}-"
              f"{fmt(full, lambda a: np.percentile(a, 90))}) | {fmt(part, np.median)} |")
        x = np.arange(nwg) % 8
        per_die = [float(np.median(dwe[x == k])) for k in range(8)]
    print(f"\ndW share end per die (median over its workgroups, last rep): "
          f"{[round(v) for v in per_die]}")
    # where the workgroups ran: XCC_ID is the die; HW_ID bits 8-15 hold the CU, shader array and
    # shader engine ids
    xcc = (t[:, WORDS - 2] & 0xF).astype(int)
    cu = ((t[:, WORDS - 1] >> 8) & 0xFF).astype(int)
    same = int((xcc == np.arange(nwg) % 8).sum())
    per = [len(set(cu[xcc == k].tolist())) for k in range(8)]
    # shader clock over each workgroup's life: s_memtime cycles / 100 MHz-clock time
    cyc = (t[:, WORDS - 3] - t[:, WORDS - 4]).astype(float)
    sec = (t[:, 2] - t[:, 0]).astype(float) / 100e6
    mhz = cyc / np.maximum(sec, 1e-9) / 1e6
    print(f"\nShader clock over each workgroup's life (s_memtime cycles / elapsed time, last rep): "
          f"median {np.median(mhz):.0f} MHz, p10 {np.percentile(mhz, 10):.0f}, "
          f"p90 {np.percentile(mhz, 90):.0f}.")
    print(f"\nDies: {same} of {nwg} workgroups ran on die (workgroup id mod 8); workgroups per die "
          f"{np.bincount(xcc, minlength=8).tolist()}, distinct CUs per die {per}.")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("build")
    r = sub.add_parser("run")
    r.add_argument("--config", type=int, default=2)
    r.add_argument("--reps", type=int, default=3)
    r.add_argument("--rho", default=None, help="retention fraction num/den (default: the workload's)")
    a = ap.parse_args()
    if a.cmd == "build":
        print("built", build())
    else:
        rho = tuple(int(v) for v in a.rho.split("/")) if a.rho else None
        run(a.config, a.reps, rho)


if __name__ == "__main__":
    main()
