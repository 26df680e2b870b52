"""Backward by replay on the GPU against the oracle's per-pair chain rule
(itself pinned to torch autograd and finite differences): gradients of X,
Y, V and every op vector for each consumer, metric and dtype, with masks,
the excluded self pair and top-k selections; then the autograd integration.

Tolerance (gpu_cases.grad_report), the forward rule: |gpu - oracle| <=
rtol * (mag + |oracle|), rtol 1e-5 (float32) / 1e-12 (float64), mag the
oracle's first-order error magnitude of that gradient. Each check prints
its worst |gpu - oracle| / tol and the relative tolerance it needs
(`pytest -s` shows them)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import bind_both, check_backward, grad_report, to_dev

pytestmark = pytest.mark.gpu

CONSUMERS = ("matmul", "displacement", "logsumexp", "softmax_matmul", "topk")


def _compare(g, ref, dtype, terms, what):
    ok, ratio = grad_report(g, ref, dtype, terms)
    assert ok, "%s: worst |gpu - oracle| / tol = %.3g" % (what, ratio)


def _run(e, oe, consumer, dtype, r, C=7, k=4, exclude_self=False, rows=None, cols=None):
    N, M, D = oe.N, oe.M, oe.D
    V = r.standard_normal((M, C)).astype(dtype) if consumer in ("matmul", "softmax_matmul") else None
    width = {"matmul": C, "softmax_matmul": C, "displacement": D, "logsumexp": 1, "topk": k}[consumer]
    G = r.standard_normal((N, width)).astype(dtype)
    check_backward(e, oe, consumer, G, V=V, k=k, exclude_self=exclude_self, rows=rows, cols=cols,
                   what="%s" % consumer)


CHAIN = lambda r, n, m: [("mul", -0.4), ("add_rows", r.standard_normal(n)), ("weight_columns", 0.5 + r.random(m)),  # noqa: E731
                         ("add_columns", 0.3 * r.standard_normal(m)), ("weight_rows", 0.5 + r.random(n))]


@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("metric", ["linear", "sqeuclidean", "rbf", "cosine_distances"])
@pytest.mark.parametrize("consumer", CONSUMERS)
@pytest.mark.parametrize("D", [3, 20, 64])
def test_backward_grid(dtype, metric, consumer, D):
    """N = 200, M = 230: ragged tiles and column splits on both sides."""
    r = np.random.default_rng(3000 + D)
    X = r.standard_normal((200, D)).astype(dtype)
    Y = r.standard_normal((230, D)).astype(dtype)
    ops = [(n, a.astype(dtype) if isinstance(a, np.ndarray) else a) for n, a in CHAIN(r, 200, 230)]
    if metric == "linear":
        ops = [("mul", 1.0 / np.sqrt(D))] + ops
    e, oe = bind_both(X, Y, metric, 0.5 / D, ops)
    _run(e, oe, consumer, dtype, r)


@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("metric", ["linear", "sqeuclidean", "rbf", "cosine_distances"])
@pytest.mark.parametrize("consumer", ("matmul", "displacement", "logsumexp", "softmax_matmul"))
def test_backward_fast_stage(dtype, metric, consumer):
    """Ops that fold into one affine stage with row and column vectors, no
    op grads wanted: the replay-free path (s = r_i q_j f + p_i + o_j)."""
    r = np.random.default_rng(3500)
    n, m, D = 210, 190, 24
    X = r.standard_normal((n, D)).astype(dtype)
    Y = r.standard_normal((m, D)).astype(dtype)
    ops = [("mul", 0.3), ("add_rows", r.standard_normal(n).astype(dtype)),
           ("weight_columns", (0.5 + r.random(m)).astype(dtype)), ("add_columns", r.standard_normal(m).astype(dtype))]
    e, oe = bind_both(X, Y, metric, 0.5 / D, ops)
    V = r.standard_normal((m, 9)).astype(dtype) if consumer in ("matmul", "softmax_matmul") else None
    width = {"matmul": 9, "softmax_matmul": 9, "displacement": D, "logsumexp": 1}[consumer]
    G = r.standard_normal((n, width)).astype(dtype)
    check_backward(e, oe, consumer, G, V=V, want=("X", "Y", "V"), what="fast %s %s" % (metric, consumer))


@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("consumer", CONSUMERS)
def test_backward_exp_chain_and_masks(dtype, consumer):
    """An exp stage, a causal band, a column mask and groups."""
    r = np.random.default_rng(3100)
    n = 150
    X = r.standard_normal((n, 16)).astype(dtype)
    gr = (np.arange(n) // 50).astype(np.int64)
    ops = [("mul", -0.05), ("exp", None), ("weight_columns", (0.5 + r.random(n)).astype(dtype)), ("causal", 2),
           ("mask_columns", r.random(n) < 0.8), ("same_group", (gr, gr))]
    e, oe = bind_both(X, X.copy(), "sqeuclidean", 1.0, ops)
    _run(e, oe, consumer, dtype, r, k=3)


@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
def test_backward_logsumexp_exclude_self(dtype):
    r = np.random.default_rng(3200)
    X = r.standard_normal((180, 32)).astype(dtype)
    e, oe = bind_both(X, X, "linear", 1.0, [("mul", 1.0 / 0.5), ("add_rows", r.standard_normal(180).astype(dtype))],
                      same=True)
    _run(e, oe, "logsumexp", dtype, r, exclude_self=True)


@pytest.mark.parametrize("consumer", ("softmax_matmul", "logsumexp", "matmul"))
def test_backward_attention_size(consumer):
    """Attention-shaped float32, 2500 x 2500, D = C = 64, on sampled rows
    and columns (each computed over all the pairs it depends on)."""
    r = np.random.default_rng(3300)
    n = 2500
    Q = r.standard_normal((n, 64)).astype(np.float32)
    K = r.standard_normal((n, 64)).astype(np.float32)
    e, oe = bind_both(Q, K, "linear", 1.0, [("mul", 0.125)])
    rows = np.unique(np.r_[np.arange(0, n, 37), np.arange(n - 20, n)])
    _run(e, oe, consumer, np.float32, r, C=64, rows=rows, cols=rows)


@pytest.mark.parametrize("consumer", CONSUMERS)
def test_autograd_through_consumers(consumer):
    """torch.autograd.grad through a consumer equals the replayed backward
    (and the oracle): X, Y, V and a row bias require grad."""
    r = np.random.default_rng(3400)
    dtype = np.float64
    X = r.standard_normal((90, 5))
    Y = r.standard_normal((110, 5))
    V = r.standard_normal((110, 3))
    b = r.standard_normal(90)
    Xt, Yt, Vt, bt = (to_dev(a).requires_grad_(True) for a in (X, Y, V, b))
    import lazy_score_matrix_amd as pw
    e = pw.lazy(Xt, Yt, "rbf", gamma=0.3, ops=[("add_rows", bt)])
    if consumer in ("matmul", "softmax_matmul"):
        out = getattr(e, consumer)(Vt)
    elif consumer == "displacement":
        out = e.displacement()
    elif consumer == "logsumexp":
        out = e.logsumexp()
    else:
        out, idx = e.topk(4)
    G = torch.randn_like(out)
    leaves = [Xt, Yt, bt] + ([Vt] if consumer in ("matmul", "softmax_matmul") else [])
    grads = torch.autograd.grad((out * G).sum(), leaves)
    oe = oracle.Expr(X, Y, "rbf", 0.3, [("add_rows", b)])
    ref = oracle.backward(oe, consumer, G.cpu().numpy(), V if consumer in ("matmul", "softmax_matmul") else None,
                          indices=idx.cpu().numpy() if consumer == "topk" else None)
    _compare(grads[0], ref["dX"], dtype, 110, "dX")
    _compare(grads[1], ref["dY"], dtype, 90, "dY")
    _compare(grads[2], ref["ops"][0], dtype, 110, "d bias")
    if consumer in ("matmul", "softmax_matmul"):
        _compare(grads[3], ref["dV"], dtype, 90, "dV")


MFMA_BWD = [(c, D, C, chain) for c in ("softmax_matmul", "logsumexp") for D in (16, 20, 48, 64)
            for C in ((16, 33, 64) if c == "softmax_matmul" else (0,)) for chain in ("scale", "row_affine")]


@pytest.mark.parametrize("consumer,D,C,chain", MFMA_BWD, ids=["%s-D%d-C%d-%s" % t for t in MFMA_BWD])
def test_backward_matrix_cores(consumer, D, C, chain):
    """Dot-product scores with one row-only affine stage in float32: the
    matrix-core backward (no op grads asked). N = 300, M = 333: ragged row
    blocks, sub-blocks and key tiles on both sides."""
    r = np.random.default_rng(3600 + D + C)
    n, m = 300, 333
    X = r.standard_normal((n, D)).astype(np.float32)
    Y = r.standard_normal((m, D)).astype(np.float32)
    ops = [("mul", 1.0 / np.sqrt(D))]
    if chain == "row_affine":
        ops += [("add_rows", r.standard_normal(n).astype(np.float32)),
                ("weight_rows", (0.5 + r.random(n)).astype(np.float32))]
    e, oe = bind_both(X, Y, "linear", 1.0, ops)
    assert e.backward_plan(consumer, C).startswith("family=mfma_grad"), e.backward_plan(consumer, C)
    V = r.standard_normal((m, C)).astype(np.float32) if C else None
    G = r.standard_normal((n, C if C else 1)).astype(np.float32)
    check_backward(e, oe, consumer, G, V=V, want=("X", "Y", "V"), what="mfma bwd %s D=%d C=%d" % (consumer, D, C))


@pytest.mark.parametrize("n", [1, 31, 1000])
def test_backward_matrix_cores_infonce(n):
    """InfoNCE shape: X with itself, a row bias, the self pair excluded."""
    r = np.random.default_rng(3700 + n)
    z = r.standard_normal((n, 32)).astype(np.float32)
    z /= np.linalg.norm(z, axis=1, keepdims=True)
    e, oe = bind_both(z, z, "linear", 1.0, [("mul", 1 / 0.07), ("add_rows", r.standard_normal(n).astype(np.float32))],
                      same=True)
    G = r.standard_normal((n, 1)).astype(np.float32)
    check_backward(e, oe, "logsumexp", G, exclude_self=True, want=("X", "Y"), what="infonce bwd n=%d" % n)


@pytest.mark.parametrize("D", [16, 5])
def test_backward_with_saved_lse(D):
    """The backward given the forward's saved row log-sum-exp equals the one
    that recomputes it (and the oracle), on the matrix-core (D = 16) and the
    vector (D = 5) backward."""
    r = np.random.default_rng(3800 + D)
    n, m = 260, 700
    X = r.standard_normal((n, D)).astype(np.float32)
    Y = r.standard_normal((m, D)).astype(np.float32)
    V = r.standard_normal((m, 10)).astype(np.float32)
    G = r.standard_normal((n, 10)).astype(np.float32)
    e, oe = bind_both(X, Y, "linear", 1.0, [("mul", 0.25), ("add_rows", r.standard_normal(n).astype(np.float32))])
    lse = torch.empty(n, device="cuda")
    out = e.softmax_matmul(to_dev(V), lse=lse)
    got = e.backward("softmax_matmul", to_dev(G), V=to_dev(V), out=out, lse=lse, want=("X", "Y", "V"))
    ref = oracle.backward(oe, "softmax_matmul", G, V)
    for key, terms in (("X", m), ("Y", n), ("V", n)):
        ok, ratio = grad_report(got[key], ref["d" + key], np.float32, terms)
        assert ok, (key, ratio)


MASKED_BWD = [(c, D, kind) for c in ("softmax_matmul", "logsumexp") for D in (32, 64)
              for kind in ("causal", "band", "rows_cols", "causal_rows")]


@pytest.mark.parametrize("consumer,D,kind", MASKED_BWD, ids=["%s-D%d-%s" % t for t in MASKED_BWD])
def test_backward_matrix_cores_masked(consumer, D, kind):
    """The matrix-core backward under a band and row / column masks:
    skipped, whole and checked tiles on both sides (N = 400, M = 450)."""
    r = np.random.default_rng(3900 + D)
    n, m = 400, 450
    X = r.standard_normal((n, D)).astype(np.float32)
    Y = r.standard_normal((m, D)).astype(np.float32)
    ops = [("mul", 1.0 / np.sqrt(D))]
    if kind == "causal":
        ops += [("causal", 0)]
    elif kind == "band":
        ops += [("band", (70, 45))]
    elif kind == "rows_cols":
        ops += [("mask_rows", r.random(n) < 0.8), ("mask_columns", r.random(m) < 0.7)]
    else:
        ops += [("causal", -5), ("mask_rows", r.random(n) < 0.9)]
    e, oe = bind_both(X, Y, "linear", 1.0, ops)
    assert e.backward_plan(consumer, 24).startswith("family=mfma_grad")
    V = r.standard_normal((m, 24)).astype(np.float32) if consumer == "softmax_matmul" else None
    G = r.standard_normal((n, 24 if V is not None else 1)).astype(np.float32)
    check_backward(e, oe, consumer, G, V=V, want=("X", "Y", "V"), what="masked mfma bwd %s %s" % (consumer, kind))
