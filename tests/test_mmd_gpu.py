"""Squared MMD between point clouds (pw_mmd2; Task Map, MMD row) on the GPU
against the oracle's statistic from the dense oracle scores: both engines
(3 and 16+ features), both dtypes, unbiased and biased, batches with
per-element and shared clouds, ragged cloud sizes and the smallest clouds."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import to_dev
from parity import assert_values

pytestmark = pytest.mark.gpu

CASES = [(k, d, dt, u) for k in ("rbf", "linear", "cosine_distances") for d in (3, 16, 33)
         for dt in (np.float32, np.float64) for u in (True, False)]


@pytest.mark.parametrize("kernel,D,dtype,unbiased", CASES,
                         ids=["%s-D%d-%s-%s" % (k, d, np.dtype(t).name, "u" if u else "b") for k, d, t, u in CASES])
def test_mmd_batched_against_oracle(kernel, D, dtype, unbiased):
    import lazy_score_matrix_amd as pw
    r = np.random.default_rng(600 + D)
    X = r.standard_normal((2, 300, D)).astype(dtype)
    Y = (0.3 + r.standard_normal((2, 257, D))).astype(dtype)
    g = 0.5 / D
    got = pw.mmd_statistics(to_dev(X), to_dev(Y), kernel, g, unbiased).cpu().numpy()
    want, mag = oracle.mmd2(X, Y, kernel, g, unbiased)
    assert_values(got, want, mag, dtype, n_terms=300 * 257, what="mmd %s D%d" % (kernel, D))


@pytest.mark.parametrize("unbiased", (True, False))
def test_mmd_shared_cloud_and_plain_inputs(unbiased):
    """Y [1, m, D] shared by a batch of three X clouds; 2-D inputs give a
    scalar."""
    import lazy_score_matrix_amd as pw
    r = np.random.default_rng(610)
    X = r.standard_normal((3, 200, 5)).astype(np.float32)
    Y = r.standard_normal((1, 150, 5)).astype(np.float32)
    got = pw.mmd_statistics(to_dev(X), to_dev(Y), "rbf", 0.3, unbiased).cpu().numpy()
    want, mag = oracle.mmd2(X, Y, "rbf", 0.3, unbiased)
    assert_values(got, want, mag, np.float32, n_terms=200 * 150, what="shared cloud")
    one = pw.mmd_statistics(to_dev(X[1]), to_dev(Y[0]), "rbf", 0.3, unbiased)
    assert one.dim() == 0
    assert_values(one.cpu().numpy(), want[1], mag[1], np.float32, n_terms=200 * 150, what="plain inputs")


def test_mmd_smallest_clouds_and_closed_form():
    """Two points per cloud (the fewest the unbiased statistic allows), the
    two-point example of the fixture (exp(-4 gamma)/2 - 1/2), and one-point
    clouds for the biased statistic."""
    import lazy_score_matrix_amd as pw
    X = np.array([[0.0], [1.0]])
    Y = np.array([[0.0], [2.0]])
    g = pw.mmd_statistics(to_dev(X), to_dev(Y), "rbf", 0.7, True).item()
    assert abs(g - (np.exp(-2.8) / 2 - 0.5)) < 1e-14
    g = pw.mmd_statistics(to_dev(X), to_dev(Y), "rbf", 0.7, False).item()
    assert abs(g - (0.5 - np.exp(-0.7) / 2)) < 1e-14
    g = pw.mmd_statistics(to_dev(X[:1]), to_dev(Y[1:]), "rbf", 0.7, False).item()
    assert abs(g - (2 - 2 * np.exp(-2.8))) < 1e-14
    with pytest.raises(ValueError):
        pw.mmd_statistics(to_dev(X[:1]), to_dev(Y), "rbf", 0.7, True)


def test_mmd_large_clouds():
    """4000 + 3500 points, 16 features, float32: every product splits its
    columns and the upper-triangle mask spans many tiles."""
    import lazy_score_matrix_amd as pw
    r = np.random.default_rng(620)
    X = r.standard_normal((4000, 16)).astype(np.float32)
    Y = (0.1 + r.standard_normal((3500, 16))).astype(np.float32)
    got = pw.mmd_statistics(to_dev(X), to_dev(Y), "rbf", 1.0 / 32).cpu().numpy()
    want, mag = oracle.mmd2(X, Y, "rbf", 1.0 / 32)
    assert_values(got, want, mag, np.float32, n_terms=4000 * 3500, what="large mmd")


GRAD = [(k, d, dt, u) for k in ("rbf", "linear", "sqeuclidean") for d in (3, 20)
        for dt in (np.float32, np.float64) for u in (True, False)]


@pytest.mark.parametrize("kernel,D,dtype,unbiased", GRAD,
                         ids=["%s-D%d-%s-%s" % (k, d, np.dtype(t).name, "u" if u else "b") for k, d, t, u in GRAD])
def test_mmd_gradients_against_oracle(kernel, D, dtype, unbiased):
    """Autograd through mmd_statistics (pw_mmd2_backward) against the
    oracle's chain-rule gradient, per batch element and for a cloud shared
    by the batch (its gradient summed over the elements)."""
    import lazy_score_matrix_amd as pw
    from parity import grad_rule
    r = np.random.default_rng(700 + D)
    X = r.standard_normal((2, 130, D)).astype(dtype)
    Y = (0.2 + r.standard_normal((1, 110, D))).astype(dtype)
    G = np.array([0.7, -1.3])
    g = 0.5 / D
    Xt, Yt = to_dev(X).requires_grad_(True), to_dev(Y).requires_grad_(True)
    out = pw.mmd_statistics(Xt, Yt, kernel, g, unbiased)
    dX, dY = torch.autograd.grad((out * torch.as_tensor(G, dtype=out.dtype, device=out.device)).sum(), [Xt, Yt])
    (ox, oxm), (oy, oym) = oracle.mmd2_grad(X, Y, kernel, g, unbiased, G)
    for got, want, mag, what in ((dX, ox, oxm, "dX"), (dY, oy, oym, "dY")):
        ok, ratio, rel = grad_rule(got.detach().cpu().numpy(), want, mag, dtype)
        print("GRAD mmd %s D%d %s %s worst_err_over_tol=%.3g" % (kernel, D, np.dtype(dtype).name, what, ratio))
        assert ok, "%s: worst |gpu - oracle| / tol = %.3g" % (what, ratio)


def test_mmd_gradient_of_plain_inputs():
    """2-D clouds under autograd: gradients keep the inputs' shapes."""
    import lazy_score_matrix_amd as pw
    from parity import grad_rule
    r = np.random.default_rng(710)
    X, Y = r.standard_normal((90, 4)), r.standard_normal((70, 4))
    Xt, Yt = to_dev(X).requires_grad_(True), to_dev(Y).requires_grad_(True)
    out = pw.mmd_statistics(Xt, Yt, "rbf", 0.4)
    out.backward()
    (ox, oxm), (oy, oym) = oracle.mmd2_grad(X, Y, "rbf", 0.4, True, 1.0)
    assert Xt.grad.shape == Xt.shape and Yt.grad.shape == Yt.shape
    assert grad_rule(Xt.grad.cpu().numpy(), ox, oxm, np.float64)[0]
    assert grad_rule(Yt.grad.cpu().numpy(), oy, oym, np.float64)[0]
