"""Host-side parts of bench.py (no GPU): the one-GPU guard and the traffic record lookup."""
import json
import os
import subprocess
import sys


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120,
                       cwd=ROOT)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == 2 and "one GPU" in out["error"]


def test_committed_traffic_record_matches_the_gemm_sources():
    # profiles/ holds rocprofv3 counters of the one-launch GEMMs keyed by a digest of their
    # sources; bench.py reports the traffic only while that digest matches the tree
    sys.path.insert(0, ROOT)
    import bench
    import synth
    for cfg in (2, 1):                            # the headline workload and the Qwen3 share
        wl = synth.spec(cfg).name
        for call in ("lrm_grouped_dw_dx", "lrm_grouped_fc1_dw_dx"):
            t = bench.recorded_traffic(call, wl)
            assert t is not None and t > 1e9, (cfg, call)
    assert bench.recorded_traffic("lrm_grouped_dw_dx", "no such workload") is None


def test_step_statistics_and_host_description():
    sys.path.insert(0, ROOT)
    import bench
    st = bench.step_stats([1.0, 2.0, 3.0, 4.0, 10.0])
    assert st["mean"] == 4.0 and st["median"] == 3.0 and st["n"] == 5
    assert st["p10"] <= st["median"] <= st["p90"]
    h = bench.host_cpu()
    assert h["cores_available"] >= 1


def test_algorithmic_bytes_of_a_small_workload():
    # the per-stage byte and flop counts the fractions are formed from, on a tiny fp32 layer
    sys.path.insert(0, ROOT)
    import numpy as np
    import bench
    import synth
    w = synth.make(0, T=64)
    sp = w.spec
    L = w.phi.shape[0]
    info = {"L": L, "K": 40, "T_ret": 30, "Ke": np.array([5, 0, 7, 8, 4, 6, 5, 5])}
    a = bench.algorithmic(w, info)
    b = 4                                       # fp32
    assert a["flops_dw"] == a["flops_dx"] == 2 * 40 * sp.h * sp.d
    assert a["select"] == 4 * L + 4 * 40
    assert a["dw"] == 40 * (sp.h + sp.d) * b + 4 * sp.E_loc * sp.h * sp.d
    assert a["dx"] == 40 * sp.h * b + 7 * sp.h * sp.d * b + 4 * 40 * sp.d   # 7 experts with rows
    assert a["compact"] == 16 * 40 + 30 * sp.h * b + 40 * sp.d * b + 40 * (sp.h + sp.d) * b
