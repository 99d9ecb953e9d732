"""Pins for the forward-KL oracle (CPU only).

* A library routine: scipy.special.rel_entr summed over softmax rows computed
  by scipy.special.softmax (different code from the oracle's own max-shift).
* Closed forms: two-token vocabularies (Bernoulli KL), a uniform draft
  (KL = ln V - H(p)), and identical rows (KL = 0, gradient = 0).
* Invariants: Gibbs' inequality (KL >= 0), invariance under adding a constant
  to either row, gradient rows summing to zero.
* The gradient against central finite differences of the KL itself.
"""
import math

import numpy as np
import pytest
import scipy.special as sp

from oracle.kl import forward_kl, forward_kl_rows


def _rows(n, v, sigma, seed):
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, sigma, (n, v)), rng.normal(0.0, sigma, (n, v))


@pytest.mark.parametrize("v,sigma", [(7, 1.0), (1000, 3.0), (4096, 4.0)])
def test_matches_scipy_rel_entr(v, sigma):
    a, b = _rows(5, v, sigma, v)
    kl, _ = forward_kl(a, b)
    for n in range(5):
        p, q = sp.softmax(a[n]), sp.softmax(b[n])
        ref = float(np.sum(sp.rel_entr(p, q)))
        assert math.isclose(kl[n], ref, rel_tol=1e-10, abs_tol=1e-12)


@pytest.mark.parametrize("x,y", [(0.0, 0.0), (2.0, -1.0), (-3.5, 4.25), (30.0, -30.0)])
def test_two_token_bernoulli_closed_form(x, y):
    # softmax([x, 0]) = (s(x), 1 - s(x)) with s the logistic function
    p1 = 1.0 / (1.0 + math.exp(-x))
    q1 = 1.0 / (1.0 + math.exp(-y))
    want = p1 * math.log(p1 / q1) + (1 - p1) * math.log((1 - p1) / (1 - q1))
    kl, grad = forward_kl(np.array([[x, 0.0]]), np.array([[y, 0.0]]))
    assert math.isclose(kl[0], want, rel_tol=1e-9, abs_tol=1e-12)
    assert np.allclose(grad[0], [q1 - p1, (1 - q1) - (1 - p1)], atol=1e-15)


def test_uniform_draft_is_log_v_minus_entropy():
    a, _ = _rows(3, 500, 2.0, 1)
    b = np.full_like(a, 0.37)
    kl, _ = forward_kl(a, b)
    for n in range(3):
        p = sp.softmax(a[n])
        h = -float(np.sum(p * np.log(p)))
        assert math.isclose(kl[n], math.log(500) - h, rel_tol=1e-10)


def test_identical_rows_give_zero():
    a, _ = _rows(4, 300, 3.0, 2)
    kl, grad = forward_kl(a, a.copy())
    assert np.all(np.abs(kl) < 1e-13)
    assert np.all(grad == 0.0)


def test_gibbs_shift_invariance_and_gradient_sums():
    a, b = _rows(6, 257, 3.0, 3)
    kl, grad = forward_kl(a, b, grad_scale=0.25)
    assert np.all(kl >= 0.0)
    kl2, grad2 = forward_kl(a + 11.5, b - 7.25, grad_scale=0.25)
    assert np.allclose(kl, kl2, rtol=1e-11, atol=1e-13)
    assert np.allclose(grad, grad2, atol=1e-14)
    assert np.all(np.abs(grad.sum(axis=1)) < 1e-13)


def test_gradient_matches_finite_differences():
    a, b = _rows(2, 11, 1.5, 4)
    _, grad = forward_kl(a, b, grad_scale=3.0)
    h = 1e-6
    for n in range(2):
        for v in range(11):
            bp, bm = b.copy(), b.copy()
            bp[n, v] += h
            bm[n, v] -= h
            num = (forward_kl(a[n:n + 1], bp[n:n + 1])[0][0] - forward_kl(a[n:n + 1], bm[n:n + 1])[0][0]) / (2 * h)
            assert math.isclose(grad[n, v], 3.0 * num, rel_tol=1e-5, abs_tol=1e-9)


def test_selected_rows_agree():
    a, b = _rows(9, 64, 2.0, 5)
    kl, grad = forward_kl(a, b)
    kls, grads = forward_kl_rows(a, b, [7, 0, 3])
    assert np.array_equal(kls, kl[[7, 0, 3]]) and np.array_equal(grads, grad[[7, 0, 3]])
