"""Column reductions through the transposed view, means and sums, and the
cosine metric's zero-vector convention, on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import bind_both, to_dev
from parity import assert_topk, assert_values

pytestmark = pytest.mark.gpu

SWAP = {"add_rows": "add_columns", "add_columns": "add_rows", "weight_rows": "weight_columns",
        "weight_columns": "weight_rows"}


def _oracle_transposed(X, Y, metric, gamma=1.0, ops=()):
    return oracle.Expr(Y, X, metric, gamma=gamma, ops=[(SWAP.get(n, n), a) for n, a in ops])


@pytest.mark.parametrize("D", [3, 32])
@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
def test_chamfer_min_both_directions(D, dtype):
    """D.min(-1) and D.min(-2) on D = sqeuclidean(X, Y) (Task Map, Chamfer row)."""
    r = np.random.default_rng(40 + D)
    X = r.standard_normal((300, D)).astype(dtype)
    Y = r.standard_normal((411, D)).astype(dtype)
    e, oe = bind_both(X, Y, "sqeuclidean")
    for dim, ref in ((-1, oe), (-2, _oracle_transposed(X, Y, "sqeuclidean"))):
        v, i = e.min(dim)
        ov, oi, om = oracle.topk(ref, 1, extra=16)
        assert_topk(v.cpu().numpy()[:, None], i.cpu().numpy()[:, None], ov, oi, om, 1, False, dtype,
                    what="min dim=%d" % dim)


def test_transposed_view_matches_dense_tiny():
    """The transposed view's row reductions are the column reductions of the
    dense oracle scores (a pin of the view itself)."""
    r = np.random.default_rng(41)
    X = r.standard_normal((7, 4))
    Y = r.standard_normal((9, 4))
    a = r.standard_normal(7)
    b = r.standard_normal(9)
    ops = [("mul", -0.5), ("add_rows", a), ("add_columns", b)]
    e, oe = bind_both(X, Y, "sqeuclidean", ops=ops)
    dense, _ = oracle.scores(oe)
    dense = np.asarray(dense, np.float64)
    lse_cols = np.log(np.exp(dense).sum(0))
    g = e.T.logsumexp().cpu().numpy()
    assert np.allclose(g, lse_cols, rtol=1e-12, atol=1e-12)
    v, i = e.T.topk(2, largest=True)
    order = np.argsort(-dense, axis=0, kind="stable")[:2].T
    assert np.array_equal(i.cpu().numpy(), order)


@pytest.mark.parametrize("metric", ["rbf", "cosine_distances", "linear"])
@pytest.mark.parametrize("D", [3, 48])
def test_mean_and_sum(metric, D):
    """mean(-1) / sum(-1) / mean(-2) (Features page, Native Deployment:
    A.reduce("mean", -1)) against the oracle's kernel product with ones."""
    r = np.random.default_rng(50 + D)
    X = r.standard_normal((257, D)).astype(np.float32)
    Y = r.standard_normal((333, D)).astype(np.float32)
    e, oe = bind_both(X, Y, metric, gamma=0.5 / D)
    ones = np.ones((333, 1), np.float32)
    o, mag = oracle.matmul(oe, ones)
    assert_values(e.sum(-1).cpu().numpy()[:, None], o, mag, np.float32, n_terms=333, what="sum")
    assert_values(e.mean(-1).cpu().numpy()[:, None], o / 333, mag / 333, np.float32, n_terms=333, what="mean")
    ot = _oracle_transposed(X, Y, metric, gamma=0.5 / D)
    o2, mag2 = oracle.matmul(ot, np.ones((257, 1), np.float32))
    assert_values(e.mean(-2).cpu().numpy()[:, None], o2 / 257, mag2 / 257, np.float32, n_terms=257,
                  what="mean(-2)")


@pytest.mark.parametrize("D", [5, 64])
def test_cosine_zero_vectors(D):
    """A zero vector has distance 1 to everything, itself included."""
    r = np.random.default_rng(60 + D)
    X = r.standard_normal((100, D)).astype(np.float32)
    X[::7] = 0
    e, oe = bind_both(X, X, "cosine_distances", same=True)
    V = r.standard_normal((100, 16)).astype(np.float32)
    o, mag = oracle.matmul(oe, V)
    assert_values(e.matmul(to_dev(V)).cpu().numpy(), o, mag, np.float32, n_terms=100, what="cosine zeros")
    v, i = e.topk(3, largest=True)
    ov, oi, om = oracle.topk(oe, 3, largest=True, extra=16)
    assert_topk(v.cpu().numpy(), i.cpu().numpy(), ov, oi, om, 3, True, np.float32, what="cosine zeros topk")
