"""Masks on the GPU against the oracle: row and column masks and the pair
masks causal, band and same_group (guide, Score Expressions and Task Map,
Attention row), on both tile engines, every consumer and both dtypes.
Sizes leave ragged row blocks and key tiles; the mask shapes make tiles of
every class (skipped, checked pair by pair, kept whole)."""
import numpy as np
import pytest

from gpu_cases import bind_both, check_consumer

pytestmark = pytest.mark.gpu

CONSUMERS = ("matmul", "displacement", "logsumexp", "softmax_matmul", "topk")
DTYPES = (np.float32, np.float64)


def _data(seed, n, m, d, dtype):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, d)).astype(dtype), r.standard_normal((m, d)).astype(dtype), r


def _masks(kind, n, m, r):
    if kind == "rows":
        keep = r.random(n) < 0.7
        keep[:3] = False
        return [("mask_rows", keep)]
    if kind == "columns":
        return [("mask_columns", r.random(m) < 0.6)]
    if kind == "causal":
        return [("causal", 0)]
    if kind == "causal_shifted":
        return [("causal", -37)]
    if kind == "band":
        return [("band", (45, 70))]
    if kind == "groups_sorted":
        # Runs of varying length, as packed sequences give.
        gr = np.sort(r.integers(0, 7, n)).astype(np.int64)
        gc = np.sort(r.integers(0, 7, m)).astype(np.int64)
        return [("same_group", (gr, gc))]
    if kind == "groups_random":
        return [("same_group", (r.integers(0, 4, n).astype(np.int64), r.integers(0, 4, m).astype(np.int64)))]
    if kind == "combined":
        gr = (np.arange(n) // 97).astype(np.int64)
        gc = (np.arange(m) // 97).astype(np.int64)
        return [("causal", 3), ("mask_columns", r.random(m) < 0.8), ("same_group", (gr, gc)),
                ("mask_rows", r.random(n) < 0.9)]
    raise ValueError(kind)


KINDS = ("rows", "columns", "causal", "causal_shifted", "band", "groups_sorted", "groups_random", "combined")


def _ops(metric, D, consumer):
    if metric == "linear":
        return [("mul", 1.0 / np.sqrt(D))]
    if consumer in ("logsumexp", "softmax_matmul"):
        return [("mul", -0.5 / D)]
    return []


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("D", [3, 32, 64])
@pytest.mark.parametrize("consumer", CONSUMERS)
@pytest.mark.parametrize("kind", KINDS)
def test_masks(dtype, D, consumer, kind):
    """D = 3 runs on the vector engine, D = 32 and 64 on the matrix cores."""
    n, m = 300, 333
    metric = "sqeuclidean" if D != 32 else "linear"
    X, Y, r = _data(1500 + D, n, m, D, dtype)
    V = r.standard_normal((m, 20)).astype(dtype)
    ops = _ops(metric, D, consumer) + _masks(kind, n, m, r)
    e, oe = bind_both(X, Y, metric, 1.0, ops)
    check_consumer(e, oe, consumer, V=V, k=10, what="%s %s D=%d" % (kind, consumer, D))


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("consumer", CONSUMERS)
def test_masks_rbf_chain(dtype, consumer):
    """rbf with a row-affine chain under a band and a column mask."""
    n, m, D = 260, 410, 16
    X, Y, r = _data(1600, n, m, D, dtype)
    V = r.standard_normal((m, 17)).astype(dtype)
    ops = [("add_rows", r.standard_normal(n).astype(dtype)), ("band", (10, 120)),
           ("mask_columns", r.random(m) < 0.5)]
    e, oe = bind_both(X, Y, "rbf", 1.0 / D, ops)
    check_consumer(e, oe, consumer, V=V, k=5, what="rbf chain %s" % consumer)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("consumer", ("softmax_matmul", "logsumexp", "topk"))
def test_causal_attention_sizes(dtype, consumer):
    """Causal attention over several row blocks and column splits."""
    n = 1500
    X, Y, r = _data(1700, n, n, 64, dtype)
    V = r.standard_normal((n, 64)).astype(dtype)
    e, oe = bind_both(X, Y, "linear", 1.0, [("mul", 0.125), ("causal", 0)])
    rows = np.unique(np.concatenate([np.arange(0, n, 7), np.arange(n - 70, n)]))
    check_consumer(e, oe, consumer, V=V, k=16, rows=rows, what="causal attention %s" % consumer)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
def test_topk_fewer_kept_than_k(dtype):
    """Rows with fewer kept pairs than k pad with NaN / -1 (causal: row i
    keeps i + 1 columns)."""
    X, Y, r = _data(1800, 40, 40, 32, dtype)
    e, oe = bind_both(X, Y, "sqeuclidean", 1.0, [("causal", 0)])
    check_consumer(e, oe, "topk", k=12, what="fewer kept")
    v, i = e.topk(12)
    assert (i[0, 1:] == -1).all() and v[0, 1:].isnan().all()


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("D", [3, 32])
@pytest.mark.parametrize("consumer", CONSUMERS)
def test_band_beyond_columns(dtype, D, consumer):
    """N > M with a band below the diagonal: whole row blocks have no kept
    pair although their tile range is not empty (tiles outside the band are
    skipped, not evaluated)."""
    X, Y, r = _data(2200 + D, 300, 120, D, dtype)
    V = r.standard_normal((120, 3)).astype(dtype)
    e, oe = bind_both(X, Y, "sqeuclidean", 1.0, [("mul", -0.1), ("band", (2, 10 ** 9))])
    check_consumer(e, oe, consumer, V=V, k=4, what="band beyond columns %s D=%d" % (consumer, D))


@pytest.mark.parametrize("consumer", CONSUMERS)
def test_all_rows_masked(consumer):
    """Every row masked: the empty-row result everywhere."""
    X, Y, r = _data(1900, 70, 90, 32, np.float32)
    V = r.standard_normal((90, 4)).astype(np.float32)
    e, oe = bind_both(X, Y, "linear", 1.0, [("mask_rows", np.zeros(70, bool))])
    check_consumer(e, oe, consumer, V=V, k=3, what="all masked %s" % consumer)


def test_transposed_view_swaps_masks():
    """S.T with a causal mask keeps i - j <= 0 of the original pairs, i.e.
    the band below the diagonal of the transposed view."""
    import lazy_score_matrix_amd as pw
    from gpu_cases import to_dev
    import oracle
    X, Y, r = _data(2000, 120, 150, 32, np.float32)
    e = pw.lazy(to_dev(X), to_dev(Y), "sqeuclidean", ops=[("causal", 2)])
    v, i = e.T.topk(4)
    oe = oracle.Expr(Y, X, "sqeuclidean", ops=[("band", (2, 10 ** 9))])
    ov, oi, om = oracle.topk(oe, 4, extra=8)
    from parity import assert_topk
    assert_topk(v.cpu().numpy(), i.cpu().numpy(), ov, oi, om, 4, False, np.float32, what="transposed causal")


def test_mean_with_mask_counts_kept():
    """mean over a masked row divides by the kept count."""
    import torch
    import lazy_score_matrix_amd as pw
    from gpu_cases import to_dev
    import oracle
    X, Y, r = _data(2100, 50, 64, 8, np.float64)
    keep = r.random(64) < 0.5
    e = pw.lazy(to_dev(X), to_dev(Y), "sqeuclidean", ops=[("mask_columns", to_dev(keep))])
    got = e.mean().cpu().numpy()
    o, _ = oracle.matmul(oracle.Expr(X, Y, "sqeuclidean", ops=[("mask_columns", keep)]), np.ones((64, 1)))
    want = np.asarray(o[:, 0], np.float64) / keep.sum()
    assert np.allclose(got, want, rtol=1e-12, atol=0)
    assert torch.is_tensor(e.mean())
