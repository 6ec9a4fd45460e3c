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
