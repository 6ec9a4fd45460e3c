"""Checks of the seeded input generator (no GPU)."""
import numpy as np
import pytest

import synth


def test_counter_rng_is_layout_independent_and_standard():
    a = synth.normals(7, 3, 0, 200000)
    b = synth.normals(7, 3, 1000, 500)
    np.testing.assert_array_equal(a[1000:1500], b)          # value depends on identity only
    assert abs(a.mean()) < 0.01 and abs(a.var() - 1) < 0.01
    assert abs(((a > 1.0).mean()) - 0.15866) < 0.005         # Gaussian tail mass
    c = synth.normals(8, 3, 0, 1000)
    assert not np.array_equal(a[:1000], c)                  # seed changes values


def test_uniform_keys():
    a = synth.uniforms_f32(7, synth.S_KEYS, 0, 200000)
    b = synth.uniforms_f32(7, synth.S_KEYS, 5000, 100)
    np.testing.assert_array_equal(a[5000:5100], b)
    assert a.dtype == np.float32 and a.min() > 0.0 and a.max() <= 1.0
    assert abs(a.mean() - 0.5) < 0.005 and abs(a.var() - 1 / 12) < 0.005
    sp = synth.spec(1, T=64)
    k = synth.pair_keys(sp)
    assert k.shape == (64 * sp.k,)
    np.testing.assert_array_equal(k, synth.uniforms_f32(sp.seed, synth.S_KEYS, 0, 64 * sp.k))


def test_rows_duplicates_and_rounding():
    src = np.array([0, 1, 0, 2])
    r = synth.rows(5, synth.S_G, 4, 16, src_row=src, kind="bf16")
    assert r[0].tobytes() == r[2].tobytes() and r[0].tobytes() != r[1].tobytes()
    f = synth.rows(5, synth.S_G, 4, 16, src_row=src, kind="f32")
    # bf16 pattern is the round-to-nearest-even of the fp32 value
    u = f.view(np.uint32).astype(np.uint64)
    np.testing.assert_array_equal(r, ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16))


@pytest.mark.parametrize("cfg", [1, 5])
def test_small_workload_routing_invariants(cfg):
    w = synth.make(cfg, T=512)
    sp = w.spec
    idx = w.topk_idx.reshape(sp.T, sp.k)
    assert all(len(set(row)) == sp.k for row in idx.tolist())     # k distinct experts per token
    a = w.topk_w.reshape(sp.T, sp.k).astype(np.float64)
    np.testing.assert_allclose(a.sum(1), 1.0, atol=1e-6)        # softmax renormalised over top-k
    assert np.all(np.diff(a, axis=1) <= 0)                      # slots in descending-logit order
    loc = (w.topk_idx >= sp.e_lo) & (w.topk_idx < sp.e_lo + sp.E_loc)
    assert w.L == int(loc.sum()) == w.phi.shape[0]
    assert w.g.shape == (sp.T, sp.h) and w.W.shape == (sp.E_loc, sp.h, sp.d)
    # determinism
    w2 = synth.make(cfg, T=512)
    assert np.array_equal(w.topk_idx, w2.topk_idx) and w.phi.tobytes() == w2.phi.tobytes()


@pytest.mark.slow
def test_extreme_skew_workload_shape():
    w = synth.make(3)
    sp = w.spec
    n = np.bincount(w.topk_idx, minlength=sp.E)[sp.e_lo:sp.e_lo + sp.E_loc]
    assert 0.295 <= n[0] / n.sum() <= 0.305
    assert int((n == 0).sum()) >= 3


@pytest.mark.slow
def test_whole_layer_workload_has_duplicates_and_empty_experts():
    w = synth.make(4)
    sp = w.spec
    n = np.bincount(w.topk_idx, minlength=sp.E)
    assert int((n == 0).sum()) > 0
    dup = np.flatnonzero(w.dup_src != np.arange(sp.T))
    assert dup.size == round(0.01 * sp.T)
    t, s = dup[0], w.dup_src[dup[0]]
    assert np.array_equal(w.topk_idx.reshape(sp.T, -1)[t], w.topk_idx.reshape(sp.T, -1)[s])
    assert w.g[t].tobytes() == w.g[s].tobytes()
