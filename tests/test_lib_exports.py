"""The C-ABI library loads on the CPU, exports every symbol include/lrm.h declares, and rejects
invalid arguments on the host before any GPU work (no GPU needed)."""
import ctypes
import os
import re

import pytest

import backward_token_expert_amd as bte
from backward_token_expert_amd import lrm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrm.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lrm_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_six_calls():
    names = _declared()
    for f in ("lrm_plan_quotas", "lrm_score", "lrm_select", "lrm_compact", "lrm_grouped_dw",
              "lrm_grouped_dx"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = bte.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) <= set(lrm.EXPORTS)


def test_binding_types_every_argument():
    # ctypes passes an untyped Python int as a 32-bit int: every call needs its argument types so
    # that device pointers, sizes and stream handles keep their 64 bits
    lib = bte.load_library()
    for name in lrm.EXPORTS:
        assert getattr(lib, name).argtypes is not None, name


def test_workspace_bytes_and_validation_on_host():
    lib = bte.load_library()
    p = bte.make_problem(32768, 8, 128, 0, 16, 2048, 768, "bf16", 262144, 262144)
    n = bte.lrm_workspace_bytes(p)
    # per-chunk histograms + token norms + tile table, 256-byte aligned
    assert n % 256 == 0 and n >= 32768 * 8 + (262144 // 1024) * 128 * 4
    bad = [bte.make_problem(0, 8, 128, 0, 16, 2048, 768, "bf16", 1, 1),       # T = 0
           bte.make_problem(16, 9, 8, 0, 8, 64, 64, "bf16", 1, 1),            # k > E
           bte.make_problem(16, 2, 8, 4, 8, 64, 64, "bf16", 1, 1),            # e_lo + E_loc > E
           bte.make_problem(16, 2, 8, 0, 8, 60, 64, "bf16", 1, 1),            # h % 8 != 0
           bte.make_problem(16, 2, 8, 0, 8, 64, 64, 7, 1, 1)]                 # unknown dtype
    for b in bad:
        assert bte.lrm_workspace_bytes(b) == 0
    pol = bte.make_policy(0, 1, 2, -1)
    P = ctypes.byref(p)
    fake = 0x100000  # never dereferenced: each call below is rejected before any launch
    # null pointers -> INVALID_ARGUMENT (1)
    assert lib.lrm_plan_quotas(P, ctypes.byref(pol), None, fake, fake, fake, fake, fake, fake, n,
                               None) == 1
    assert lib.lrm_score(P, fake, fake, fake, fake, fake, None, fake, n, None) == 1
    # misaligned g -> UNSUPPORTED (2)
    assert lib.lrm_score(P, fake, fake + 2, fake, fake, fake, fake, fake, n, None) == 2
    # short workspace -> WORKSPACE_TOO_SMALL (3); far below any call's need, so no call can pass
    # the check and launch with these placeholder pointers
    assert lib.lrm_select(P, fake, fake, fake, fake, fake, fake, 1024, None) == 3
    # bad retention fraction
    pol0 = bte.make_policy(0, 1, 0, -1)
    assert lib.lrm_plan_quotas(P, ctypes.byref(pol0), fake, fake, fake, fake, fake, fake, fake, n,
                               None) == 1
    # quota kinds: unknown kind, or a cap with the proportional split
    for kp in (bte.make_policy(0, 1, 2, -1, kind=3), bte.make_policy(0, 1, 2, 5, kind="proportional")):
        assert lib.lrm_plan_quotas(P, ctypes.byref(kp), fake, fake, fake, fake, fake, fake, fake, n,
                                   None) == 1
    # criteria: unknown criterion; a NULL input the criterion reads; a misaligned g
    sc = lib.lrm_score_criterion
    assert sc(P, 4, fake, fake, fake, fake, fake, fake, fake, fake, n, None) == 1
    assert sc(P, 3, None, None, None, None, fake, fake, fake, fake, n, None) == 1   # no keys
    assert sc(P, 1, None, None, None, None, fake, fake, fake, fake, n, None) == 1   # no g
    assert sc(P, 2, None, fake + 2, None, None, fake, fake, fake, fake, n, None) == 2
    assert sc(P, 0, None, fake, fake, None, fake, fake, fake, fake, n, None) == 1   # LRM: no topk_w
    # the score in two halves: a NULL input, a misaligned phi, a short workspace
    assert lib.lrm_score_norms(P, None, fake, fake, n, None) == 1
    assert lib.lrm_score_norms(P, fake, fake + 8, fake, n, None) == 2
    assert lib.lrm_score_norms(P, fake, fake, fake, 1024, None) == 3
    assert lib.lrm_score_combine(P, fake, None, fake, fake, fake, n, None) == 1
    assert lib.lrm_score_combine(P, fake, fake, fake, fake, fake, 1024, None) == 3
    assert lib.lrm_status_string(3) == b"workspace too small"


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(lrm.LrmError):
        lrm.load_library(str(tmp_path / "missing.so"))


def test_layer_calls_validate_on_host():
    lib = bte.load_library()
    p = bte.make_problem(32768, 8, 128, 0, 16, 2048, 768, "bf16", 262144, 262144)
    n = bte.lrm_workspace_bytes(p)
    P = ctypes.byref(p)
    fake = 0x100000  # never dereferenced: each call below is rejected before any launch
    assert lib.lrm_swiglu_backward(P, fake, fake, fake, fake, None, fake, n, None) == 1
    assert lib.lrm_swiglu_backward(P, fake, fake, fake + 4, fake, fake, fake, n, None) == 2
    assert lib.lrm_gather_tokens(P, None, fake, fake, fake, fake, n, None) == 1
    assert lib.lrm_gather_tokens(P, fake, fake, fake + 8, fake, fake, n, None) == 2
    assert lib.lrm_scatter_tokens(P, fake, fake, fake, fake, fake, 1024, None) == 3
    assert lib.lrm_grouped_fc1_dw(P, fake, fake, fake, None, fake, n, None) == 1
    assert lib.lrm_grouped_fc1_dx(P, fake, fake, fake, fake + 4, fake, n, None) == 2
    # FC1's split-expert slots are 2d x h: the workspace is sized for them, and a workspace large
    # enough for FC2's products alone is refused by the FC1 calls
    fc2_only = n - 16 * 2048 * 768 * 4
    assert lib.lrm_grouped_fc1_dw_dx(P, fake, fake, fake, fake, fake, fake, fake, fc2_only,
                                     None) == 3
    assert lib.lrm_grouped_fc1_dw_dx(P, fake, fake, fake, None, fake, fake, fake, n, None) == 1


def test_admission_struct_and_validation_on_host():
    lib = bte.load_library()
    assert ctypes.sizeof(lrm.Admission) == 248 and lrm.Admission.mem_budget.offset == 208
    p = bte.make_problem(32768, 8, 128, 0, 16, 2048, 768, "bf16", 262144, 262144)
    n = bte.lrm_workspace_bytes(p)
    P = ctypes.byref(p)
    fake = 0x100000  # never dereferenced: each call below is rejected before any launch

    def call(a, ws_bytes=n):
        return lib.lrm_admit_quotas(P, ctypes.byref(a), fake, fake, fake, fake, fake, ws_bytes,
                                    None)
    ok = [(1, 1, 1), (0, 1, 2)]
    assert call(bte.make_admission([], 1 << 40)) == 1                                # no candidate
    many = bte.make_admission([(0, 1, 1)] * 16, 1 << 40)
    many.n_cand = 17                                                                  # too many
    assert call(many) == 1
    assert call(bte.make_admission([(0, 1, 0)], 1 << 40)) == 1                       # rho_den = 0
    assert call(bte.make_admission(ok, 1 << 40, kind="proportional", cap_abs=5)) == 1
    assert call(bte.make_admission(ok, 1 << 40, mem_per_row=-1)) == 1
    assert call(bte.make_admission(ok, 1 << 40, comm_per_row=(1 << 32) + 1)) == 1
    assert call(bte.make_admission(ok, 1 << 40), ws_bytes=1024) == 3
    assert lib.lrm_admit_quotas(P, None, fake, fake, fake, fake, fake, n, None) == 1


def test_noalloc_gemm_rejects_problems_beyond_its_scratch_on_host():
    # lrm_grouped_dw_dx_noalloc keeps its schedule in a 1 MiB static device buffer: a retained-row
    # capacity whose tile table cannot fit is refused before any launch (WORKSPACE_TOO_SMALL, 3)
    bte.load_library()
    fake = 0x100000   # never dereferenced
    P = lrm.make_problem(65536, 8, 128, 0, 16, 2048, 768, "bf16", 2 ** 25, 2 ** 26)
    with pytest.raises(lrm.LrmError, match=r"\(status 3\)"):
        lrm.lrm_grouped_dw_dx_noalloc(P, fake, fake, fake, fake, fake, fake, stream=0)
    # null pointers are refused first (INVALID_ARGUMENT, 1)
    Q = lrm.make_problem(4096, 8, 128, 0, 16, 2048, 768, "bf16", 32768, 32768)
    with pytest.raises(lrm.LrmError, match=r"\(status 1\)"):
        lrm.lrm_grouped_dw_dx_noalloc(Q, fake, None, fake, fake, fake, fake, stream=0)
