"""HBM throughput ceilings of the access mixes the path's memory stages use.

  python -m backward_token_expert_amd.hbm_ceiling build     # on any host (hipcc)
  python -m backward_token_expert_amd.hbm_ceiling run       # on the GPU

`build` compiles csrc/tools/hbm_ceiling.hip into _build/hbm_ceiling/libhbm_ceiling.so (liblrm.so
is not touched).  `run` times plain streaming kernels over a 1 GiB read side, well past the
256 MB last-level cache: a read-only pass and a write-only pass (non-temporal or plain stores) at three grid sizes, and a read of
each 16-byte chunk written to R = 1 (a copy), 2, 3 and 4 places.  It prints a markdown table of
bytes moved per second (reads plus writes).  These are the ceilings the score (read-only), the
compaction (about one read to three writes) and the GEMMs' stores are compared against.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
OUT_DIR = os.path.join(PKG, "_build", "hbm_ceiling")
LIB = os.path.join(OUT_DIR, "libhbm_ceiling.so")
SRC = os.path.join(PKG, "csrc", "tools", "hbm_ceiling.hip")
GIB = 1 << 30


def build() -> str:
    from backward_token_expert_amd import build as B
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = [B.HIPCC, *B.CFLAGS, "-shared", SRC, "-o", LIB]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode:
        raise SystemExit(r.stdout)
    return LIB


def run(reps: int = 5) -> None:
    if not os.path.exists(LIB):
        raise SystemExit(f"{LIB} is missing: run `python -m backward_token_expert_amd.hbm_ceiling build`")
    import torch
    lib = ctypes.CDLL(LIB)
    lib.hbm_ceiling_time.restype = ctypes.c_float
    lib.hbm_ceiling_time.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_longlong, ctypes.c_int, ctypes.c_int]
    n16 = GIB // 16
    src = torch.empty(GIB, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    dst = torch.empty(4 * GIB, dtype=torch.uint8, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 128 * 256, dtype=torch.int32, device="cuda")
    rows = []

    def t(kind, blocks):
        ms = lib.hbm_ceiling_time(kind, src.data_ptr(), dst.data_ptr(), out.data_ptr(), n16, blocks,
                                  reps)
        if ms <= 0:
            raise SystemExit(f"timing failed for kind {kind}")
        return ms

    for mult in (8, 32, 128):
        ms = t(0, cus * mult)
        rows.append((f"read, {cus * mult} workgroups", GIB, 0, ms))
    for mult in (8, 32, 128):
        rows.append((f"write (non-temporal), {cus * mult} workgroups", 0, GIB, t(1, cus * mult)))
        rows.append((f"write (plain stores), {cus * mult} workgroups", 0, GIB, t(6, cus * mult)))
    for r in (1, 2, 3, 4):
        ms = t(1 + r, cus * 32)
        rows.append((f"read 1 : write {r}, {cus * 32} workgroups", GIB, r * GIB, ms))
    torch.cuda.synchronize()
    print("# HBM ceilings (streaming kernels, 16-byte non-temporal accesses, 1 GiB read side)\n")
    print("Command (R = repository root):\n\n```\npython -m backward_token_expert_amd.hbm_ceiling build\n"
          "python -m backward_token_expert_amd.hbm_ceiling run\n```\n")
    print(f"{torch.cuda.get_device_name(0)}, {cus} CUs; mean of {reps} launches after two "
          "untimed ones.\n")
    print("| access | read GB | written GB | µs per launch | GB/s (read + written) |")
    print("|---|---|---|---|---|")
    for name, rd, wr, ms in rows:
        print(f"| {name} | {rd / 1e9:.2f} | {wr / 1e9:.2f} | {ms * 1e3:.0f} | "
              f"{(rd + wr) / (ms * 1e-3) / 1e9:.0f} |")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("build")
    r = sub.add_parser("run")
    r.add_argument("--reps", type=int, default=5)
    a = ap.parse_args()
    if a.cmd == "build":
        print("built", build())
    else:
        run(a.reps)


if __name__ == "__main__":
    main()
