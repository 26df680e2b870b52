"""Conjugate-gradient solve of (K + a I) A = B on the GPU (Task Map, Kernel
ridge / GP mean row) against the oracle's dense solve.

Bound used: for K positive semi-definite and a > 0 the smallest eigenvalue
of K + a I is at least a, so |A_c - A*_c| <= |r_c| / a for the true
residual r = B - (K + a I) A, which the oracle evaluates in higher
precision. The true residual itself must reach rtol up to the recurrence's
rounding drift (a few eps * |K + a I| |A|)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import bind_both, solve_report, to_dev

pytestmark = pytest.mark.gpu

def _system(seed, n, d, dtype, C, gamma=0.3):
    r = np.random.default_rng(seed)
    X = r.standard_normal((n, d)).astype(dtype)
    B = r.standard_normal((n, C)).astype(dtype)
    return X, B


def _check_solution(oe, A, B, shift, rtol, dtype, rows=None):
    ok, ratio = solve_report(oe, A, B, shift, rtol, rows)
    assert ok, ("residual / bound", ratio)


@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("C", [1, 5])
@pytest.mark.parametrize("D", [5, 16])
def test_cg_matches_dense_solve(dtype, C, D):
    n, shift = 700, 0.5
    X, B = _system(2300 + C + D, n, D, dtype, C)
    rtol = 1e-4 if dtype == np.float32 else 1e-10
    e, oe = bind_both(X, X, "rbf", 0.3 / D, [], same=True)
    A, info = e.solve(to_dev(B), shift, rtol=rtol, max_iter=500)
    assert info["converged"] and info["status"] == "converged", info
    assert 0 < info["iterations"] <= 500 and info["max_rel_residual"] <= rtol
    _check_solution(oe, A.cpu().numpy(), B, shift, rtol, dtype)


@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
def test_cg_vector_rhs_and_zero_column(dtype):
    X, B = _system(2400, 300, 8, dtype, 3)
    B[:, 1] = 0
    e, oe = bind_both(X, X, "rbf", 0.05, [], same=True)
    A, info = e.solve(to_dev(B), 2.0, rtol=1e-4)
    assert info["converged"]
    assert (A[:, 1] == 0).all()
    a1, info1 = e.solve(to_dev(B[:, 0]), 2.0, rtol=1e-4)
    assert a1.shape == (300,) and info1["converged"]
    # One column alone runs another product kernel (another summation
    # order): both solutions sit within |r| / shift of the exact one.
    _check_solution(oe, a1.cpu().numpy()[:, None], B[:, :1], 2.0, 1e-4, dtype)
    _check_solution(oe, A.cpu().numpy(), B, 2.0, 1e-4, dtype)


def test_cg_max_iter_and_determinism():
    X, B = _system(2500, 800, 16, np.float32, 2)
    e, oe = bind_both(X, X, "rbf", 0.01, [], same=True)
    A, info = e.solve(to_dev(B), 1e-3, rtol=1e-12, max_iter=3, check_every=2)
    assert not info["converged"] and info["status"] == "max_iter" and info["iterations"] == 3
    A2, info2 = e.solve(to_dev(B), 1e-3, rtol=1e-12, max_iter=3, check_every=2)
    assert torch.equal(A, A2) and info == info2


def test_cg_breakdown_on_indefinite():
    """A negative definite score (-X X^T) with a small shift is not positive
    definite: the first step's curvature is negative."""
    X, B = _system(2600, 200, 16, np.float64, 1)
    e, oe = bind_both(X, X, "linear", 1.0, [("mul", -1.0)], same=True)
    A, info = e.solve(to_dev(B), 0.1, rtol=1e-8)
    assert info["status"] == "breakdown" and not info["converged"]


@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
def test_cg_large_sampled_residual(dtype):
    """20000 points (several row blocks, column splits and reduction
    blocks): the true residual on sampled rows."""
    n = 20000
    X, B = _system(2700, n, 16, dtype, 1)
    e, oe = bind_both(X, X, "rbf", 1.0 / 32, [], same=True)
    shift = 10.0
    rtol = 1e-3 if dtype == np.float32 else 1e-8
    A, info = e.solve(to_dev(B), shift, rtol=rtol, max_iter=2000)
    assert info["converged"], info
    rows = np.unique(np.concatenate([np.arange(0, n, 97), np.arange(n - 50, n)]))
    _check_solution(oe, A.cpu().numpy(), B, shift, rtol, dtype, rows=rows)
