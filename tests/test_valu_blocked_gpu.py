"""The blocked vector kernels against the oracle, each test first asserting
that the planner picked the kernel it means to cover:
  * the narrow kernel product (four rows per thread, 256-column tiles; rbf by
    the norm expansion with the row factor deferred, and its direct-form
    fallbacks for points far from the origin);
  * the row log-sum-exp (four rows per thread and 256-column tiles for dot
    products and squared distances, by the norm expansion; two rows for
    rbf) with no stage, a scalar stage (gentle and steep, positive scales
    moving the reference often), a row-vector stage, with and without the
    self pair;
  * the two-rows row minimum / maximum with exact ties (lowest index wins).
The planner takes the four-rows kernels only where their grid (1024-row
blocks times 256-column tiles) holds at least one workgroup per CU, so
their cases use 22000+ columns and compare sampled rows: every row of the
first waves, of each row-block boundary and of the ragged last block, plus
random ones. The two-rows kernels span several 512-row blocks with a ragged
last block and a ragged last column tile; small problems take the finer
kernels (the last test).
"""
import numpy as np
import pytest

from gpu_cases import bind_both, check_consumer, to_dev

pytestmark = pytest.mark.gpu


def _sample(n, seed):
    """Rows to compare: the first 70, 40 on each side of every 1024-row
    boundary, the last 60 and 60 random ones."""
    r = np.random.default_rng(seed)
    rows = set(range(min(n, 70))) | set(range(max(0, n - 60), n)) | set(r.integers(0, n, 60).tolist())
    for b in range(1024, n, 1024):
        rows |= set(range(b - 40, min(n, b + 40)))
    return np.array(sorted(rows), np.int64)


def _field(plan, key):
    for tok in plan.split():
        k, _, v = tok.partition("=")
        if k == key:
            return v
    raise AssertionError("%s not in plan %r" % (key, plan))


PROD = [(m, d, c) for m in ("linear", "sqeuclidean", "rbf") for d in (1, 2, 3, 4) for c in (1, 2, 4)]


@pytest.mark.parametrize("metric,D,C", PROD, ids=["%s-D%d-C%d" % p for p in PROD])
def test_narrow_product(metric, D, C):
    r = np.random.default_rng(100 + 10 * D + C)
    X = r.standard_normal((2100, D)).astype(np.float32)
    Y = r.standard_normal((22001, D)).astype(np.float32)
    V = r.standard_normal((22001, C)).astype(np.float32)
    e, oe = bind_both(X, Y, metric, gamma=0.5)
    plan = e.plan("matmul", C)
    assert _field(plan, "family") == "valu" and _field(plan, "rows") == "4" and _field(plan, "bn") == "256", plan
    check_consumer(e, oe, "matmul", V=V, rows=_sample(2100, D), what="narrow product %s D%d C%d" % (metric, D, C))


@pytest.mark.parametrize("D", (2, 3, 4))
def test_narrow_product_rbf_far_points(D):
    """A row far from the origin keeps its wave in the direct form (row
    factor not deferred); a far column sends its tile to the direct form
    with the factor deferred; an exact copy of a far row scores 1."""
    r = np.random.default_rng(200 + D)
    M = 22001
    X = r.standard_normal((2100, D)).astype(np.float32)
    Y = r.standard_normal((M, D)).astype(np.float32)
    X[5] *= 30.0            # wave 0 of row block 0
    X[1024 + 300] *= 30.0   # a wave of row block 1
    Y[300] *= 30.0          # column tile 1
    Y[M - 5] = X[5]         # exact copy of a far row, last (ragged) tile
    V = np.concatenate([r.standard_normal((M, 3)), np.ones((M, 1))], 1).astype(np.float32)
    e, oe = bind_both(X, Y, "rbf", gamma=0.5)
    assert _field(e.plan("matmul", 4), "rows") == "4"
    rows = np.union1d(_sample(2100, 200 + D), [5, 1324])
    check_consumer(e, oe, "matmul", V=V, rows=rows, what="rbf far points D%d" % D)
    onehot = np.zeros((M, 1), np.float32)
    onehot[M - 5] = 1.0
    g = e.matmul(to_dev(onehot)).cpu().numpy()
    assert g[5, 0] == 1.0, "an exact copy of a far point must score exactly 1 (got %r)" % g[5, 0]


LSE_CHAINS = {
    "none": lambda n, r: [],
    "mul": lambda n, r: [("mul", -0.5)],
    "steep": lambda n, r: [("mul", 6.0)],
    "rowvec": lambda n, r: [("mul", -0.5), ("add_rows", r.standard_normal(n).astype(np.float32)),
                            ("weight_rows", (0.5 + r.random(n)).astype(np.float32))],
}
LSE = [(m, d, ch, ex) for m in ("linear", "sqeuclidean", "rbf") for d in (1, 3, 4) for ch in LSE_CHAINS
       for ex in (False, True)]


@pytest.mark.parametrize("metric,D,chain,excl", LSE, ids=["%s-D%d-%s-%s" % (a, b, c, "excl" if x else "all")
                                                          for a, b, c, x in LSE])
def test_blocked_logsumexp(metric, D, chain, excl):
    r = np.random.default_rng(300 + D)
    N = 22001 if excl else 2100
    M = 22001
    X = r.standard_normal((N, D)).astype(np.float32)
    Y = X if excl else r.standard_normal((M, D)).astype(np.float32)
    ops = LSE_CHAINS[chain](N, r)
    e, oe = bind_both(X, Y, metric, gamma=0.5, ops=ops, same=excl)
    plan = e.plan("logsumexp")
    rows = "2" if metric == "rbf" else "4"
    assert _field(plan, "family") == "valu" and _field(plan, "rows") == rows, plan
    check_consumer(e, oe, "logsumexp", exclude_self=excl, rows=_sample(N, 300 + D),
                   what="blocked lse %s D%d %s" % (metric, D, chain))


MINS = [(d, lg) for d in (1, 2, 3, 4) for lg in (False, True)]


@pytest.mark.parametrize("D,largest", MINS, ids=["D%d-%s" % (d, "max" if lg else "min") for d, lg in MINS])
def test_two_rows_min_exact_ties(D, largest):
    """Integer points: every squared distance is exact and ties abound;
    the returned index must be the lowest among equal values, bit for bit,
    on rows of every row block (i and i + 256 of each 512-row block)."""
    r = np.random.default_rng(400 + D)
    X = r.integers(-3, 4, (1100, D)).astype(np.float32)
    Y = r.integers(-3, 4, (1333, D)).astype(np.float32)  # several column splits
    e, oe = bind_both(X, Y, "sqeuclidean")
    plan = e.plan("topk", 0, 1)
    assert _field(plan, "family") == "valu" and _field(plan, "rows") == "2", plan
    check_consumer(e, oe, "topk", k=1, largest=largest, exact=True, what="two-rows min D%d" % D)


@pytest.mark.parametrize("largest", (False, True), ids=("min", "max"))
def test_two_rows_min_far_points(largest):
    """Three-feature minima by the norm expansion on clustered points far
    from the origin (|x|^2 near 7500 against distances near 1), with exact
    copies among the columns (distance 0): values within the rule's
    error magnitude, indices wherever the oracle's values are separated."""
    r = np.random.default_rng(410)
    X = (50.0 + r.standard_normal((1100, 3))).astype(np.float32)
    Y = (50.0 + r.standard_normal((1333, 3))).astype(np.float32)
    Y[600:700] = X[:100]
    e, oe = bind_both(X, Y, "sqeuclidean")
    plan = e.plan("topk", 0, 1)
    assert _field(plan, "family") == "valu" and _field(plan, "rows") == "2", plan
    check_consumer(e, oe, "topk", k=1, largest=largest, what="two-rows far min")


@pytest.mark.parametrize("metric", ("linear", "sqeuclidean"))
def test_blocked_logsumexp_far_points(metric):
    """Points far from the origin: the norm expansion cancels more there,
    within the error magnitude the comparison rule allows."""
    r = np.random.default_rng(330)
    X = r.standard_normal((2100, 3)).astype(np.float32)
    Y = r.standard_normal((22001, 3)).astype(np.float32)
    X[5] *= 30.0
    Y[300] *= 30.0
    Y[21000] = X[5]
    X[1500] *= 1000.0
    Y[700] *= 1000.0
    e, oe = bind_both(X, Y, metric, ops=[("mul", -0.5)])
    assert _field(e.plan("logsumexp"), "rows") == "4"
    check_consumer(e, oe, "logsumexp", rows=np.union1d(_sample(2100, 330), [5, 1500]),
                   what="blocked lse far points %s" % metric)


SMALL = [("matmul", m) for m in ("linear", "sqeuclidean", "rbf")] + [("logsumexp", m) for m in ("linear", "sqeuclidean")]


@pytest.mark.parametrize("consumer,metric", SMALL, ids=["%s-%s" % c for c in SMALL])
def test_small_problems_take_finer_kernels(consumer, metric):
    """At 1024 x 1333 the four-rows grid would hold 4 x 6 workgroups: the
    product takes the one-row kernel and the log-sum-exp the two-rows one."""
    r = np.random.default_rng(340)
    X = r.standard_normal((1024, 3)).astype(np.float32)
    Y = r.standard_normal((1333, 3)).astype(np.float32)
    V = r.standard_normal((1333, 4)).astype(np.float32)
    ops = [("mul", -0.5)] if consumer == "logsumexp" else []
    e, oe = bind_both(X, Y, metric, gamma=0.5, ops=ops)
    plan = e.plan(consumer, 4 if consumer == "matmul" else 0)
    assert _field(plan, "rows") == ("1" if consumer == "matmul" else "2"), plan
    check_consumer(e, oe, consumer, V=V if consumer == "matmul" else None, what="small %s %s" % (consumer, metric))
