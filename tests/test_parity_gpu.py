"""GPU parity against the CPU oracle on seeded inputs small enough for the
oracle, spanning several row blocks and column tiles with ragged tails,
every metric, consumer, dtype and op-chain shape, and the edge cases.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_cases import bind_both, bind_case, check_consumer, to_dev

pytestmark = pytest.mark.gpu

METRICS = ("linear", "sqeuclidean", "rbf", "cosine_distances")
CONSUMERS = ("matmul", "displacement", "logsumexp", "softmax_matmul", "topk")
DTYPES = (np.float32, np.float64)


def _data(seed, n, m, d, dtype, scale=1.0):
    r = np.random.default_rng(seed)
    X = (scale * r.standard_normal((n, d))).astype(dtype)
    Y = (scale * r.standard_normal((m, d))).astype(dtype)
    return X, Y, r


def _gamma(metric, d):
    return 0.5 / d if metric == "rbf" else 1.0


def _linear_scale(metric, d):
    # keep linear scores O(1) so exp-based consumers stay in range
    return [("mul", 1.0 / np.sqrt(d))] if metric == "linear" else []


GRID = [(dt, m, c, d) for dt in DTYPES for m in METRICS for c in CONSUMERS for d in (3, 33)]


@pytest.mark.parametrize("dtype,metric,consumer,D", GRID,
                         ids=["%s-%s-%s-D%d" % (np.dtype(a).name, b, c, d) for a, b, c, d in GRID])
def test_grid_ragged(dtype, metric, consumer, D):
    """N=300 (two row blocks, ragged), M=333 (six column tiles, ragged)."""
    X, Y, r = _data(7 + D, 300, 333, D, dtype)
    V = r.standard_normal((333, 5)).astype(dtype)
    ops = _linear_scale(metric, D)
    if metric == "sqeuclidean" and consumer in ("logsumexp", "softmax_matmul"):
        ops = [("mul", -0.5)]
    e, oe = bind_both(X, Y, metric, _gamma(metric, D), ops)
    check_consumer(e, oe, consumer, V=V, k=10, exclude_self=True, what=consumer)


SPLIT_GRID = [(dt, m, c, d) for dt in DTYPES for m in METRICS for c in CONSUMERS for d in (3, 5)]


@pytest.mark.parametrize("dtype,metric,consumer,D", SPLIT_GRID,
                         ids=["%s-%s-%s-D%d" % (np.dtype(a).name, b, c, d) for a, b, c, d in SPLIT_GRID])
def test_vector_engine_column_splits(dtype, metric, consumer, D):
    """Vector-engine split partials and their merges on every consumer:
    N = 300, M = 2500 (many column splits, a ragged last tile)."""
    X, Y, r = _data(17 + D, 300, 2500, D, dtype)
    V = r.standard_normal((2500, 5)).astype(dtype)
    ops = _linear_scale(metric, D)
    if metric == "sqeuclidean" and consumer in ("logsumexp", "softmax_matmul"):
        ops = [("mul", -0.5)]
    e, oe = bind_both(X, Y, metric, _gamma(metric, D), ops)
    plan = e.plan(consumer, 5 if consumer in ("matmul", "softmax_matmul") else 0, 10 if consumer == "topk" else 0)
    assert "family=valu" in plan and "splits=1 " not in plan, plan
    check_consumer(e, oe, consumer, V=V, k=10, exclude_self=True, what=consumer)


@pytest.mark.parametrize("D", [1, 2, 4, 5, 15, 16, 17, 31, 32, 63, 64])
def test_feature_dims(D):
    X, Y, r = _data(100 + D, 70, 130, D, np.float32)
    V = r.standard_normal((130, 4)).astype(np.float32)
    e, oe = bind_both(X, Y, "rbf", 0.5 / D)
    check_consumer(e, oe, "matmul", V=V, what="matmul D=%d" % D)
    e, oe = bind_both(X, Y, "sqeuclidean")
    check_consumer(e, oe, "topk", k=8, what="topk D=%d" % D)


@pytest.mark.parametrize("C", [1, 3, 4, 5, 16, 17, 64, 65, 130])
@pytest.mark.parametrize("consumer", ["matmul", "softmax_matmul"])
def test_value_widths(C, consumer):
    X, Y, r = _data(200 + C, 90, 150, 8, np.float32)
    V = r.standard_normal((150, C)).astype(np.float32)
    e, oe = bind_both(X, Y, "linear", ops=[("mul", 0.3)])
    check_consumer(e, oe, consumer, V=V, what="%s C=%d" % (consumer, C))


def _op_chains(N, M, dtype, r):
    a = r.standard_normal(N).astype(dtype)
    b = r.standard_normal(M).astype(dtype)
    w = (0.5 + r.random(N)).astype(dtype)
    u = (0.5 + r.random(M)).astype(dtype)
    return {
        "mul": [("mul", -0.7)],
        "add": [("add", 1.5)],
        "add_rows": [("mul", 0.5), ("add_rows", a)],
        "add_columns": [("add_columns", b)],
        "weight_rows": [("weight_rows", w)],
        "weight_columns": [("weight_columns", u)],
        "offsets_both": [("mul", -0.5), ("add_rows", a), ("add_columns", b)],
        "exp_then_weights": [("mul", -0.2), ("exp", None), ("weight_rows", w), ("weight_columns", u)],
        "nonseparable_rows_then_colweight": [("add_rows", a), ("weight_columns", u)],
        "nonseparable_cols_then_rowweight": [("add_columns", b), ("weight_rows", w)],
        "scalar_moves_to_columns": [("add", 0.75), ("weight_columns", u), ("add_rows", a)],
        "two_exps": [("mul", -0.1), ("exp", None), ("mul", -1.0), ("exp", None)],
        "eight_ops": [("mul", 0.5), ("add_rows", a), ("weight_columns", u), ("add", -0.25), ("add_columns", b),
                      ("weight_rows", w), ("mul", 0.5), ("add", 0.1)],
    }


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("chain", list(_op_chains(1, 1, np.float32, np.random.default_rng(0)).keys()))
@pytest.mark.parametrize("consumer", ["matmul", "logsumexp", "softmax_matmul", "topk", "displacement"])
def test_op_chains(dtype, chain, consumer):
    X, Y, r = _data(300, 260, 200, 6, dtype, scale=0.5)
    ops = _op_chains(260, 200, dtype, r)[chain]
    V = r.standard_normal((200, 3)).astype(dtype)
    e, oe = bind_both(X, Y, "sqeuclidean", ops=ops)
    check_consumer(e, oe, consumer, V=V, k=5, largest=True, what="%s %s" % (chain, consumer))


@pytest.mark.parametrize("N,M", [(1, 1), (1, 500), (500, 1), (3, 2), (257, 65), (64, 4097)])
@pytest.mark.parametrize("consumer", CONSUMERS)
def test_small_and_ragged_sizes(N, M, consumer):
    X, Y, r = _data(N * 1000 + M, N, M, 3, np.float64)
    V = r.standard_normal((M, 2))
    e, oe = bind_both(X, Y, "rbf", 0.3)
    check_consumer(e, oe, consumer, V=V, k=min(M, 4), exclude_self=True, what="%s N=%d M=%d" % (consumer, N, M))


@pytest.mark.parametrize("N,M", [(300, 200), (200, 300), (129, 129)])
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
def test_exclude_self(N, M, dtype):
    """The pair j == i is dropped by index; rows i >= M exclude nothing."""
    X, Y, r = _data(400 + N, N, M, 4, dtype)
    for exclude in (False, True):
        e, oe = bind_both(X, Y, "linear", ops=[("mul", 2.0)])
        check_consumer(e, oe, "logsumexp", exclude_self=exclude, what="exclude=%s" % exclude)


def test_exclude_self_aliased_identical_rows():
    """X = Y with all rows equal: lse = s + log(M - 1) everywhere; one row -> -inf."""
    X = np.tile(np.array([[0.25, -0.5, 1.0]], np.float32), (1000, 1))
    e, oe = bind_both(X, X, "linear", same=True)
    check_consumer(e, oe, "logsumexp", exclude_self=True, what="identical rows")
    X1 = X[:1]
    e, oe = bind_both(X1, X1, "linear", same=True)
    out = e.logsumexp(exclude_self=True).cpu().numpy()
    assert np.isneginf(out).all()


@pytest.mark.parametrize("k", [1, 2, 5, 8, 9, 10, 16, 17, 40, 64])
@pytest.mark.parametrize("largest", [False, True])
def test_topk_exact_ties(k, largest):
    """Integer grid with duplicated reference rows: every score is exact, so
    values and indices must match the oracle bit for bit, lowest index first."""
    r = np.random.default_rng(500 + k)
    X = r.integers(-3, 4, (300, 3)).astype(np.float32)
    Y = r.integers(-3, 4, (700, 3)).astype(np.float32)
    Y[100:200] = Y[:100]
    e, oe = bind_both(X, Y, "sqeuclidean")
    check_consumer(e, oe, "topk", k=k, largest=largest, exact=True, what="exact k=%d" % k)
    e, oe = bind_both(X, Y, "linear")
    check_consumer(e, oe, "topk", k=k, largest=largest, exact=True, what="exact linear k=%d" % k)


def test_topk_full_permutation():
    """k = M returns the whole stable order."""
    r = np.random.default_rng(9)
    X = r.integers(-2, 3, (50, 2)).astype(np.float64)
    Y = r.integers(-2, 3, (64, 2)).astype(np.float64)
    e, oe = bind_both(X, Y, "sqeuclidean")
    check_consumer(e, oe, "topk", k=64, exact=True, what="k=M")


def test_matmul_exact_integers():
    """Integer inputs with the linear metric: every partial sum is exact."""
    r = np.random.default_rng(11)
    X = r.integers(-5, 6, (300, 7)).astype(np.float64)
    Y = r.integers(-5, 6, (900, 7)).astype(np.float64)
    V = r.integers(-5, 6, (900, 3)).astype(np.float64)
    e, _ = bind_both(X, Y, "linear")
    g = e.matmul(to_dev(V)).cpu().numpy()
    ref = X.astype(np.int64) @ Y.astype(np.int64).T @ V.astype(np.int64)
    assert np.array_equal(g, ref.astype(np.float64))


def test_rbf_self_pairs_are_one():
    """rbf(x, x) = 1: isolated points (100 apart) give the row mass exactly 1."""
    X = (100.0 * np.arange(600, dtype=np.float64)[:, None] * np.array([[1.0, 0.5]])).astype(np.float32)
    V = np.ones((600, 1), np.float32)
    e, _ = bind_both(X, X, "rbf", 1.0, same=True)
    g = e.matmul(to_dev(V)).cpu().numpy()
    assert np.array_equal(g, np.ones((600, 1), np.float32))


@pytest.mark.parametrize("D", (16, 32))
def test_mfma_rbf_kernel_at_most_one(D):
    """The matrix-core rbf (norm expansion, float32) clamps its exponent at
    0: every kernel value is finite and <= 1, also for points far from the
    origin where the expansion cancels; self pairs of ordinary points are
    1 within the rule's tolerance (|k - 1| <= 1e-5 (1 + gamma sum (|x| +
    |y|)^2)), and the whole kernel matrix passes the rule."""
    r = np.random.default_rng(600 + D)
    n = 300
    X = r.standard_normal((n, D)).astype(np.float32)
    X[::17] *= 3e4  # far from the origin: the expansion cancels
    eye = np.eye(n, dtype=np.float32)
    e, oe = bind_both(X, X, "rbf", 1.0 / D, same=True)
    assert e.plan("matmul", 64).startswith("family=mfma"), e.plan("matmul", 64)
    K = e.matmul(to_dev(eye)).cpu().numpy()
    assert np.all(np.isfinite(K)) and np.all(K <= 1.0) and np.all(K >= 0.0), (K.max(), K.min())
    near = np.ones(n, bool)
    near[::17] = False
    spread = 4 * np.sum(X.astype(np.float64) ** 2, axis=1)
    d = np.diag(K)[near]
    assert np.all(np.abs(d - 1.0) <= 1e-5 * (1 + spread[near] / D)), np.max(np.abs(d - 1.0))
    check_consumer(e, oe, "matmul", V=eye, what="rbf kernel matrix D%d" % D)


def test_softmax_rows_sum_to_one():
    X, Y, r = _data(12, 400, 700, 16, np.float32)
    V = np.ones((700, 1), np.float32)
    e, _ = bind_both(X, Y, "linear", ops=[("mul", 0.25)])
    g = e.softmax_matmul(to_dev(V)).cpu().numpy()
    assert np.max(np.abs(g - 1.0)) < 1e-5


@pytest.mark.parametrize("consumer", CONSUMERS)
def test_empty_columns(consumer):
    """M = 0: sums are zero, log-sum-exp is -inf; N = 0 is a no-op."""
    X = np.ones((5, 3), np.float32)
    Y = np.zeros((0, 3), np.float32)
    e, _ = bind_both(X, Y, "linear")
    V = to_dev(np.zeros((0, 2), np.float32))
    if consumer == "matmul":
        assert (e.matmul(V).cpu().numpy() == 0).all()
    elif consumer == "softmax_matmul":
        assert (e.softmax_matmul(V).cpu().numpy() == 0).all()
    elif consumer == "displacement":
        assert (e.displacement().cpu().numpy() == 0).all()
    elif consumer == "logsumexp":
        assert np.isneginf(e.logsumexp().cpu().numpy()).all()
    else:
        with pytest.raises(ValueError):
            e.topk(1)
    e0, _ = bind_both(np.zeros((0, 3), np.float32), np.ones((4, 3), np.float32), "linear")
    assert e0.matmul(to_dev(np.ones((4, 2), np.float32))).shape == (0, 2)


def test_determinism():
    """Two calls with the same plan give bitwise-identical results."""
    X, Y, r = _data(13, 2000, 3000, 32, np.float32)
    V = r.standard_normal((3000, 8)).astype(np.float32)
    e, _ = bind_both(X, Y, "rbf", 0.05)
    a = e.matmul(to_dev(V)).cpu().numpy()
    b = e.matmul(to_dev(V)).cpu().numpy()
    assert np.array_equal(a, b)
    d, _ = bind_both(X, Y, "sqeuclidean")
    va, ia = d.topk(10)
    vb, ib = d.topk(10)
    assert torch.equal(va, vb) and torch.equal(ia, ib)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS.keys()))
def test_reduced_workloads(name):
    """Every workload's distributions and op chains at a size the oracle
    finishes in seconds."""
    arrays, cases = workloads.make(name, reduced=True)
    for c in cases:
        e, oe = bind_case(arrays, c)
        V = arrays[c.v] if c.v else None
        check_consumer(e, oe, c.consumer, V=V, exclude_self=c.exclude_self, k=c.k, largest=c.largest,
                       what="%s/%s" % (name, c.name),
                       params={k: workloads.resolve(v, arrays) for k, v in c.params.items()})


# ---------------------------------------------------------------- MFMA engine
MFMA_GRID = [(dt, m, c, d, ch) for dt in DTYPES for m in METRICS for c in CONSUMERS for d in (16, 32, 64)
             for ch in ("none", "row_affine")]


def _assert_family(e, consumer, family, C=0, k=0):
    plan = e.plan(consumer, C, k)
    assert ("family=%s" % family) in plan, plan


@pytest.mark.parametrize("dtype,metric,consumer,D,chain", MFMA_GRID,
                         ids=["%s-%s-%s-D%d-%s" % (np.dtype(a).name, b, c, d, ch) for a, b, c, d, ch in MFMA_GRID])
def test_mfma_grid(dtype, metric, consumer, D, chain):
    """MFMA engine: N=300 (ragged row blocks), M=333 (ragged 64-key tiles)."""
    X, Y, r = _data(900 + D, 300, 333, D, dtype)
    V = r.standard_normal((333, 20)).astype(dtype)
    ops = _linear_scale(metric, D)
    if metric == "sqeuclidean" and consumer in ("logsumexp", "softmax_matmul"):
        ops = [("mul", -0.5 / D)]
    if chain == "row_affine":
        ops = ops + [("add_rows", r.standard_normal(300).astype(dtype)), ("weight_rows", (0.5 + r.random(300)).astype(dtype))]
    e, oe = bind_both(X, Y, metric, _gamma(metric, D), ops)
    _assert_family(e, consumer, "mfma", C=20, k=10)
    check_consumer(e, oe, consumer, V=V, k=10, exclude_self=True, what="mfma %s" % consumer)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("C", [16, 17, 32, 33, 64, 65, 130])
@pytest.mark.parametrize("consumer", ["matmul", "softmax_matmul"])
def test_mfma_value_widths(dtype, C, consumer):
    X, Y, r = _data(1000 + C, 150, 500, 32, dtype)
    V = r.standard_normal((500, C)).astype(dtype)
    e, oe = bind_both(X, Y, "linear", ops=[("mul", 0.2)])
    _assert_family(e, consumer, "mfma", C=C)
    check_consumer(e, oe, consumer, V=V, what="%s C=%d" % (consumer, C))


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("metric", METRICS)
@pytest.mark.parametrize("D", [16, 17, 64])
@pytest.mark.parametrize("chain", ["none", "row_affine"])
def test_mfma_single_column(dtype, metric, D, chain):
    """A kernel product with one value column (a weighted row sum) runs on
    the matrix-core engine with the column folded by vector FMAs; N = 300
    and M = 333 leave ragged row blocks and tiles."""
    X, Y, r = _data(1300 + D, 300, 333, D, dtype)
    w = r.standard_normal((333, 1)).astype(dtype)
    ops = _linear_scale(metric, D)
    if chain == "row_affine":
        ops = ops + [("add_rows", r.standard_normal(300).astype(dtype)), ("weight_rows", (0.5 + r.random(300)).astype(dtype))]
    e, oe = bind_both(X, Y, metric, _gamma(metric, D), ops)
    _assert_family(e, "matmul", "mfma", C=1)
    check_consumer(e, oe, "matmul", V=w, what="mfma single column %s D=%d" % (metric, D))


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("M", [1, 127, 128, 129, 5000])
def test_mfma_single_column_sizes(dtype, M):
    """Column counts around the 128-key tile and a column split."""
    X, Y, r = _data(1400 + M, 200, M, 32, dtype)
    w = r.standard_normal((M, 1)).astype(dtype)
    e, oe = bind_both(X, Y, "rbf", 1.0 / 32)
    _assert_family(e, "matmul", "mfma", C=1)
    check_consumer(e, oe, "matmul", V=w, what="mfma single column M=%d" % M)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("k", [1, 10, 16, 17, 64])
@pytest.mark.parametrize("largest", [False, True])
def test_mfma_topk(dtype, k, largest):
    X, Y, r = _data(1100 + k, 260, 1500, 32, dtype)
    e, oe = bind_both(X, Y, "sqeuclidean")
    _assert_family(e, "topk", "mfma", k=k)
    check_consumer(e, oe, "topk", k=k, largest=largest, what="mfma topk k=%d" % k)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("k", [1, 5, 16, 40])
def test_mfma_topk_exact_ties(dtype, k):
    """Integer grid in 16 dimensions with duplicated references: the norm
    expansion is exact, so indices and values must match bit for bit."""
    r = np.random.default_rng(1200 + k)
    X = r.integers(-2, 3, (200, 16)).astype(dtype)
    Y = r.integers(-2, 3, (900, 16)).astype(dtype)
    Y[300:600] = Y[:300]
    e, oe = bind_both(X, Y, "sqeuclidean")
    _assert_family(e, "topk", "mfma", k=k)
    check_consumer(e, oe, "topk", k=k, exact=True, what="mfma exact k=%d" % k)
    e, oe = bind_both(X, Y, "linear")
    check_consumer(e, oe, "topk", k=k, largest=True, exact=True, what="mfma exact linear k=%d" % k)
    # Smallest dot products: the plain search on the raw accumulator.
    check_consumer(e, oe, "topk", k=k, exact=True, what="mfma exact smallest linear k=%d" % k)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("k", [1, 10])
def test_mfma_topk_far_from_origin(dtype, k):
    """Clustered points far from the origin: |x|^2 dwarfs the distances, so
    the plain search's deferred |x_i|^2 and the clamp at 0 are exercised
    (near-equal values fall under the tolerance rule)."""
    r = np.random.default_rng(1300 + k)
    X = (50.0 + r.standard_normal((300, 32))).astype(dtype)
    Y = (50.0 + r.standard_normal((2000, 32))).astype(dtype)
    Y[1000:1100] = X[:100]  # exact copies: distance 0 for rows 0..99
    e, oe = bind_both(X, Y, "sqeuclidean")
    _assert_family(e, "topk", "mfma", k=k)
    check_consumer(e, oe, "topk", k=k, what="mfma far topk k=%d" % k)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("k", [10, 16, 40])
def test_mfma_topk_every_key_enters(dtype, D, k):
    """References on a ray with norms falling by index: every key is closer
    to every query (and has a larger dot product) than all keys before it,
    so each one enters every list and the float engine's candidate queues
    run full at every sub-block. The k last references win, in reverse
    order."""
    r = np.random.default_rng(1400 + D + k)
    X = (0.05 * r.standard_normal((300, D))).astype(dtype)
    u = r.standard_normal(D)
    u /= np.linalg.norm(u)
    M = 1700
    Y = ((1000.0 - 0.5 * np.arange(M))[:, None] * u[None, :]).astype(dtype)
    e, oe = bind_both(X, Y, "sqeuclidean")
    _assert_family(e, "topk", "mfma", k=k)
    check_consumer(e, oe, "topk", k=k, what="every key enters, sqeuclidean k=%d" % k)
    # Dot products rising with the index: queries along u, norms rising.
    Xu = (u[None, :] + 0.05 * r.standard_normal((300, D))).astype(dtype)
    Yu = ((100.0 + 0.5 * np.arange(M))[:, None] * u[None, :]).astype(dtype)
    e, oe = bind_both(Xu, Yu, "linear")
    check_consumer(e, oe, "topk", k=k, largest=True, what="every key enters, largest linear k=%d" % k)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("D", [3, 8])
@pytest.mark.parametrize("k", [2, 8, 16, 40])
def test_valu_topk_every_key_enters(dtype, D, k):
    """The vector engine under the same order: every key enters every list,
    so each thread's queue fills at every group of columns."""
    r = np.random.default_rng(1500 + D + k)
    u = r.standard_normal(D)
    u /= np.linalg.norm(u)
    M = 1700
    X = (0.05 * r.standard_normal((300, D))).astype(dtype)
    Y = ((1000.0 - 0.5 * np.arange(M))[:, None] * u[None, :]).astype(dtype)
    e, oe = bind_both(X, Y, "sqeuclidean")
    _assert_family(e, "topk", "valu", k=k)
    check_consumer(e, oe, "topk", k=k, what="vector engine, every key enters, k=%d" % k)
    Xu = (u[None, :] + 0.05 * r.standard_normal((300, D))).astype(dtype)
    Yu = ((100.0 + 0.5 * np.arange(M))[:, None] * u[None, :]).astype(dtype)
    e, oe = bind_both(Xu, Yu, "linear")
    check_consumer(e, oe, "topk", k=k, largest=True, what="vector engine, every key enters, largest k=%d" % k)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("N", [129, 300, 1000])
def test_mfma_exclude_self(dtype, N):
    X, _, r = _data(1300 + N, N, 1, 64, dtype)
    X /= np.linalg.norm(X, axis=1, keepdims=True)
    b = r.standard_normal(N).astype(dtype)
    e, oe = bind_both(X, X, "linear", ops=[("mul", 1 / 0.07), ("add_rows", b)], same=True)
    _assert_family(e, "logsumexp", "mfma")
    check_consumer(e, oe, "logsumexp", exclude_self=True, what="mfma infonce N=%d" % N)


def test_mfma_determinism():
    X, Y, r = _data(14, 3000, 5000, 64, np.float32)
    V = r.standard_normal((5000, 64)).astype(np.float32)
    e, _ = bind_both(X, Y, "linear", ops=[("mul", 0.125)])
    _assert_family(e, "softmax_matmul", "mfma", C=64)
    a = e.softmax_matmul(to_dev(V)).cpu().numpy()
    b = e.softmax_matmul(to_dev(V)).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("metric", ["linear", "sqeuclidean"])
@pytest.mark.parametrize("D", [3, 32, 64])
@pytest.mark.parametrize("chain", ["scale", "row_affine", "causal"])
@pytest.mark.parametrize("M", [333, 5000])
def test_softmax_keeps_row_logsumexp(dtype, metric, D, chain, M):
    """softmax@V with its row log-sum-exp (the statistic the backward
    replays with) equals the oracle's log-sum-exp of the same scores, on
    both engines, with and without column splits (M = 5000)."""
    import oracle
    from parity import assert_values
    X, Y, r = _data(4200 + D + M, 300, M, D, dtype)
    V = r.standard_normal((M, 12)).astype(dtype)
    ops = [("mul", (1.0 / np.sqrt(D)) if metric == "linear" else -0.5 / D)]
    if chain == "row_affine":
        ops += [("add_rows", r.standard_normal(300).astype(dtype)), ("weight_rows", (0.5 + r.random(300)).astype(dtype))]
    elif chain == "causal":
        ops += [("causal", 40)]
    e, oe = bind_both(X, Y, metric, 1.0, ops)
    lse = torch.empty(300, dtype=torch.float32 if dtype == np.float32 else torch.float64, device="cuda")
    out = e.softmax_matmul(to_dev(V), lse=lse)
    o, mag = oracle.softmax_matmul(oe, V)
    assert_values(out.cpu().numpy(), o, mag, dtype, n_terms=M, vmax=float(np.max(np.abs(V))), what="softmax")
    ol, lmag = oracle.logsumexp(oe)
    assert_values(lse.cpu().numpy(), ol, lmag, dtype, n_terms=M, what="softmax lse")
