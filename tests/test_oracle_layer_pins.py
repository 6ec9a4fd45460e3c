"""Pins of the oracle's rest-of-the-expert-backward functions (no GPU).

The activation backward is checked against complex-step derivatives of phi = SiLU(a) * c (exact to
float64 rounding, computed without the derivative formula), the float64 -> bfloat16 rounding
against an exact search over bf16 patterns in rational arithmetic, and the whole chain (FC2, the
activation, FC1, the return to the tokens) against torch's float64 autograd of the masked layer:
the loss sum_t <g_t, sum over retained slots of alpha * W2_e SiLU(a) * c> with [a; c] = W1_e x_t.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


# ------------------------------------------------------------------------------------------------
# float64 -> bfloat16, round to nearest even
# ------------------------------------------------------------------------------------------------

def _bf16_value(bits: int) -> Fraction:
    """Exact value of a finite non-negative bf16 pattern (bits < 0x7F80)."""
    e, m = bits >> 7, bits & 0x7F
    if e == 0:
        return Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    return (1 + Fraction(m, 1 << 7)) * (Fraction(2) ** (e - 127))


def _bf16_nearest_even(v: float) -> int:
    """The bf16 pattern nearest to v (ties to the even pattern), by bisection over the monotone
    non-negative patterns and an exact comparison of the two neighbours."""
    x = Fraction(abs(v))
    sign = 0x8000 if np.signbit(v) else 0
    lo, hi = 0, 0x7F7F                      # largest pattern with value <= x
    if x >= _bf16_value(0x7F7F):
        lo = 0x7F7F
    else:
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if _bf16_value(mid) <= x:
                lo = mid
            else:
                hi = mid
    if lo == 0x7F7F:                        # past the largest finite value: the upper neighbour
        upper = Fraction(2) ** 128          # is 2^128, which rounds to infinity
        if x == _bf16_value(0x7F7F):
            return sign | 0x7F7F
        dl, du = x - _bf16_value(0x7F7F), upper - x
        return sign | (0x7F7F if dl < du else 0x7F80)   # a tie goes to the even pattern 0x7F80
    a, b = _bf16_value(lo), _bf16_value(lo + 1)
    if x - a < b - x or (x - a == b - x and lo % 2 == 0):
        return sign | lo
    return sign | (lo + 1)


def test_f64_to_bf16_rne_exact_search():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(400) * np.exp2(rng.integers(-140, 128, 400)))
    # exact midpoints between neighbouring bf16 values (ties) and points just off them
    for bits in rng.integers(1, 0x7F7E, 300):
        mid = (_bf16_value(int(bits)) + _bf16_value(int(bits) + 1)) / 2
        m = float(mid)
        assert Fraction(m) == mid                           # representable in float64
        vals += [m, np.nextafter(m, np.inf), np.nextafter(m, -np.inf), -m]
    vals += [0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -150, 1.0, -1.0,
             float(_bf16_value(0x7F7F)), 3.3895313892515355e38, 3.40e38, -3.40e38, 1e300]
    vals = np.asarray(vals, np.float64)
    got = O.f64_to_bf16_rne(vals)
    for v, g in zip(vals, got):
        assert int(g) == _bf16_nearest_even(float(v)), (v, hex(int(g)))


def test_f64_to_bf16_agrees_with_two_step_rounding_off_ties():
    # Away from ties of the second rounding, rounding to float32 first and then to bf16 gives the
    # same pattern (torch's float32 -> bfloat16 is round to nearest even).
    import torch
    rng = np.random.default_rng(3)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))
    f = v.astype(np.float32)
    low = f.view(np.uint32) & np.uint32(0xFFFF)
    ok = low != 0x8000
    two = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16_rne(v)[ok], two[ok])


# ------------------------------------------------------------------------------------------------
# activation backward
# ------------------------------------------------------------------------------------------------

def _phi_complex(a, c):
    return a / (1.0 + np.exp(-a)) * c


def test_swiglu_backward_complex_step():
    rng = np.random.default_rng(11)
    a = np.concatenate([rng.standard_normal(500) * 3, [0.0, -1.2785, 20.0, -20.0, 40.0, -40.0]])
    c = rng.standard_normal(a.size)
    dphi = rng.standard_normal(a.size)
    eps = 1e-30
    da_ref = dphi * (_phi_complex(a + 1j * eps, c).imag / eps)
    dc_ref = dphi * (_phi_complex(a, c + 1j * eps).imag / eps)
    dA, dC = O.swiglu_backward64(dphi, a, c)
    # relative to the scale |dphi * c| where SiLU' crosses zero (a near -1.278), where 1 + a(1 - s)
    # cancels
    assert np.all(np.abs(dA - da_ref) <= 1e-13 * np.abs(da_ref) + 1e-15 * np.abs(dphi * c))
    assert np.all(np.abs(dC - dc_ref) <= 1e-13 * np.abs(dc_ref))


def test_swiglu_backward_special_points():
    dA, dC = O.swiglu_backward64(np.ones(3), np.array([0.0, 60.0, -60.0]), np.ones(3))
    assert dA[0] == 0.5 and dC[0] == 0.0          # SiLU'(0) = 1/2, SiLU(0) = 0
    assert dA[1] == 1.0 and dC[1] == 60.0         # saturates to the identity
    assert abs(dA[2]) < 1e-20 and abs(dC[2]) < 1e-20
    # SiLU' is negative below its minimum near a = -1.278 and positive above
    dA, _ = O.swiglu_backward64(np.ones(2), np.array([-2.0, -1.0]), np.ones(2))
    assert dA[0] < 0 < dA[1]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_swiglu_backward_rows_and_rounding(dtype):
    rng = np.random.default_rng(5)
    L, d, K = 30, 6, 12
    ac32 = rng.standard_normal((L, 2 * d)).astype(np.float32)
    ac = ac32 if dtype == "f32" else O.f32_to_bf16_rne(ac32)
    sel_row = np.sort(rng.choice(L, K, replace=False))
    dphi = rng.standard_normal((K, d)).astype(np.float32)
    dH = O.swiglu_backward(dphi, ac, sel_row, dtype)
    w = O.widen(ac, dtype)
    for i, r in enumerate(sel_row):
        dA, dC = O.swiglu_backward64(dphi[i].astype(np.float64), w[r, :d], w[r, d:])
        want = np.concatenate([dA, dC])
        if dtype == "f32":
            assert np.array_equal(dH[i], want.astype(np.float32))
        else:
            assert np.array_equal(dH[i], [_bf16_nearest_even(float(v)) for v in want])


# ------------------------------------------------------------------------------------------------
# return to the tokens
# ------------------------------------------------------------------------------------------------

def test_scatter_with_zeros_sums_slots_and_zero_fills():
    rng = np.random.default_rng(2)
    T, k, h = 7, 3, 5
    sel_pair = np.array([0, 4, 5, 9, 20, 2], np.int64)      # tokens 0, 1, 1, 3, 6, 0
    dXc = rng.standard_normal((sel_pair.size, h)).astype(np.float32)
    out = O.scatter_with_zeros(dXc, sel_pair, T, k)
    want = np.zeros((T, h))
    for i, p in enumerate(sel_pair):
        want[p // k] += dXc[i]
    assert np.allclose(out, want, rtol=0, atol=1e-12)
    assert not out[[2, 4, 5]].any()                          # no retained pair: exact zeros
    # the float64 sum runs in slot order: token 0 = (0 + row of slot 0) + row of slot 2
    assert np.array_equal(out[0], (0.0 + dXc[0].astype(np.float64)) + dXc[5].astype(np.float64))


# ------------------------------------------------------------------------------------------------
# the whole expert backward against autograd of the masked layer
# ------------------------------------------------------------------------------------------------

def test_layer_backward_matches_autograd_of_masked_layer():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    T, k, E, e_lo, E_loc, h, d = 24, 2, 5, 1, 3, 6, 4
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32).reshape(-1)
    alpha = rng.random(T * k).astype(np.float32)
    g = rng.standard_normal((T, h)).astype(np.float32)
    x = rng.standard_normal((T, h)).astype(np.float32)
    W1 = (rng.standard_normal((E_loc, 2 * d, h)) / np.sqrt(h)).astype(np.float32)
    W2 = (rng.standard_normal((E_loc, h, d)) / np.sqrt(d)).astype(np.float32)
    row_pair, fwd_off = O.forward_layout(idx, e_lo, E_loc)
    t_of = row_pair // k
    e_of = idx[row_pair] - e_lo
    # forward state of every local row, float64, stored as float32 like the saved context
    H1 = np.einsum("rjh,rh->rj", W1[e_of].astype(np.float64), x[t_of].astype(np.float64))
    ac = H1.astype(np.float32)
    a64, c64 = ac[:, :d].astype(np.float64), ac[:, d:].astype(np.float64)
    phi = (a64 / (1 + np.exp(-a64)) * c64).astype(np.float32)
    pol = {"full": 0, "rho_num": 1, "rho_den": 2, "cap_abs": -1, "kind": "cap"}
    o = O.run(idx, alpha, g, phi, W2, T=T, k=k, E=E, e_lo=e_lo, E_loc=E_loc, dtype="f32",
              policy=pol)
    assert 0 < o["sel_row"].size < row_pair.size            # some pairs dropped
    lay = O.run_layer(o, o["dphi"], ac, x, W1, T=T, k=k, dtype="f32")

    # autograd of the layer restricted to the retained pairs
    tW1 = torch.tensor(W1, dtype=torch.float64, requires_grad=True)
    tW2 = torch.tensor(W2, dtype=torch.float64, requires_grad=True)
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    out = torch.zeros((T, h), dtype=torch.float64)
    for r in o["sel_row"]:
        p, e, t = int(row_pair[r]), int(e_of[r]), int(t_of[r])
        hh = tW1[e] @ tx[t]
        y = tW2[e] @ (torch.nn.functional.silu(hh[:d]) * hh[d:])
        out = out.index_add(0, torch.tensor([t]), (float(alpha[p]) * y)[None])
    (out * torch.tensor(g, dtype=torch.float64)).sum().backward()

    def rel(a, b):
        return np.linalg.norm(a - b) / np.linalg.norm(b)

    assert rel(o["dW"], tW2.grad.numpy()) < 1e-6
    assert rel(lay["dW1"], tW1.grad.numpy()) < 1e-6
    assert rel(lay["dx"], tx.grad.numpy()) < 1e-6
    # experts' FC1 gradients are zero exactly where they keep no row
    for e in range(E_loc):
        if o["cmp_off"][e + 1] == o["cmp_off"][e]:
            assert not lay["dW1"][e].any()
