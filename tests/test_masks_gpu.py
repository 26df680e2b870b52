"""Masks on the GPU against the oracle: row and column masks and the pair
masks causal, band and same_group (guide, Score Expressions and Task Map,
Attention row), on both tile engines, every consumer and both dtypes.
Sizes leave ragged row blocks and key tiles; the mask shapes make tiles of
every class (skipped, checked pair by pair, kept whole)."""
import numpy as np
import pytest

import oracle
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


def _kept(ops, n, m):
    """The kept-pair matrix of an op list, written out from the mask
    definitions (guide, Score Expressions and Task Map, Attention row)."""
    K = np.ones((n, m), bool)
    i, j = np.arange(n)[:, None], np.arange(m)[None, :]
    for name, a in ops:
        if name == "mask_rows":
            K &= np.asarray(a, bool)[:, None]
        elif name == "mask_columns":
            K &= np.asarray(a, bool)[None, :]
        elif name == "causal":
            K &= (j - i) <= a
        elif name == "band":
            K &= ((i - j) <= a[0]) & ((j - i) <= a[1])
        elif name == "same_group":
            K &= np.asarray(a[0])[:, None] == np.asarray(a[1])[None, :]
    return K


def _mean_reference(oe, ops, n, m):
    o, mag = oracle.matmul(oe, np.ones((m, 1), dtype=oe.np_dtype))
    cnt = _kept(ops, n, m).sum(1)
    with np.errstate(invalid="ignore", divide="ignore"):
        want = np.where(cnt > 0, np.asarray(o[:, 0], np.float64) / np.maximum(cnt, 1), np.nan)
    return want, np.asarray(mag[:, 0], np.float64) / np.maximum(cnt, 1), cnt


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
@pytest.mark.parametrize("kind", KINDS + ("empty_band",))
def test_mean_masked_in_library(kind, dtype):
    """pw_mean: sums over the kept pairs divided by the kept count, NaN for
    a row with none, and the inverse counts (0 for none) it reports."""
    import torch
    from parity import assert_values
    X, Y, r = _data(2200, 300, 333, 5, dtype)
    ops = [("band", (-200, 10 ** 9))] if kind == "empty_band" else _masks(kind, 300, 333, r)
    e, oe = bind_both(X, Y, "rbf", gamma=0.2, ops=ops)
    inv = torch.empty(300, dtype=e.dtype, device=e.device)
    got = e.mean(-1, inv_counts=inv).cpu().numpy().astype(np.float64)
    want, mag, cnt = _mean_reference(oe, ops, 300, 333)
    empty = cnt == 0
    if kind in ("rows", "empty_band"):
        assert empty.any()
    assert np.all(np.isnan(got[empty])), "rows with no kept pair must be NaN"
    if (~empty).any():
        assert_values(got[~empty][:, None], want[~empty][:, None], mag[~empty][:, None], dtype, n_terms=333,
                      what="mean %s" % kind)
    one = np.asarray(1, dtype)
    want_inv = np.where(cnt > 0, one / np.maximum(cnt, 1).astype(dtype), 0).astype(dtype)
    assert np.array_equal(inv.cpu().numpy(), want_inv)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f64"])
def test_mean_batched_one_call(dtype):
    """A batched handle's mean: one pw_mean call for every element, each
    against the oracle, masks shared, per-element row offsets."""
    import torch
    import lazy_score_matrix_amd as pw
    from gpu_cases import to_dev
    from parity import assert_values
    r = np.random.default_rng(2300)
    B, n, m, d = 3, 150, 170, 4
    X = r.standard_normal((B, n, d)).astype(dtype)
    Y = r.standard_normal((1, m, d)).astype(dtype)
    a = r.standard_normal((B, n)).astype(dtype)
    gr = np.sort(r.integers(0, 5, n)).astype(np.int64)
    gc = np.sort(r.integers(0, 5, m)).astype(np.int64)
    ops = [("add_rows", to_dev(a)), ("same_group", (to_dev(gr), to_dev(gc))), ("causal", 20)]
    e = pw.lazy(to_dev(X), to_dev(Y), "sqeuclidean", ops=ops)
    assert "batch=3" in e.plan("matmul", C=1)
    got = e.mean(-1).cpu().numpy().astype(np.float64)
    host_ops = [("same_group", (gr, gc)), ("causal", 20)]
    for b in range(B):
        oe = oracle.Expr(X[b], Y[0], "sqeuclidean", ops=[("add_rows", a[b])] + host_ops)
        want, mag, cnt = _mean_reference(oe, host_ops, n, m)
        empty = cnt == 0
        assert np.all(np.isnan(got[b][empty]))
        assert_values(got[b][~empty][:, None], want[~empty][:, None], mag[~empty][:, None], dtype, n_terms=m,
                      what="batched mean element %d" % b)
    assert torch.is_tensor(e.mean(-1))


def test_mean_autograd_replays_weighted_sum():
    """Gradients of sum(mean * G): the sum product's backward with G scaled
    by each row's inverse kept count (the derivative of a sum over a fixed
    kept set divided by its size)."""
    import torch
    import lazy_score_matrix_amd as pw
    from gpu_cases import grad_report, to_dev
    r = np.random.default_rng(2400)
    X = r.standard_normal((120, 6))
    Y = r.standard_normal((140, 6))
    keep = r.random(140) < 0.6
    rows = r.random(120) < 0.9
    ops = [("mask_columns", keep), ("mask_rows", rows)]
    Xt, Yt = to_dev(X).requires_grad_(True), to_dev(Y).requires_grad_(True)
    e = pw.lazy(Xt, Yt, "rbf", gamma=0.3, ops=[("mask_columns", to_dev(keep)), ("mask_rows", to_dev(rows))])
    out = e.mean(-1)
    cnt = _kept(ops, 120, 140).sum(1)
    assert np.all(np.isnan(out.detach().cpu().numpy()[cnt == 0]))
    G = torch.randn(120, dtype=torch.float64, device=out.device)
    dX, dY = torch.autograd.grad((torch.nan_to_num(out) * G).sum(), [Xt, Yt])
    Gs = np.where(cnt > 0, G.cpu().numpy() / np.maximum(cnt, 1), 0.0)
    ref = oracle.backward(oracle.Expr(X, Y, "rbf", 0.3, ops), "matmul", Gs[:, None], np.ones((140, 1)))
    for g, rv, what in ((dX, ref["dX"], "dX"), (dY, ref["dY"], "dY")):
        ok, ratio = grad_report(g, rv, np.float64, 140)
        assert ok, "%s: worst |gpu - oracle| / tol = %.3g" % (what, ratio)
