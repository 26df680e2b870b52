"""Leading batch dimensions: a [B, N, D] x [B, M, D] score, and a [1, N, D]
input broadcast against [B, M, D] (Task Map, MMD row; Features page, batch
broadcasting), element by element against the oracle, plus gradients
through the batch axis."""
import numpy as np
import pytest
import torch

import lazy_score_matrix_amd as pw
import oracle
from gpu_cases import check_consumer, to_dev
from parity import assert_topk, assert_values

pytestmark = pytest.mark.gpu


def _batch_of(plan):
    return int(dict(t.split("=", 1) for t in plan.split() if "=" in t)["batch"])


@pytest.mark.parametrize("bx", [1, 3])
@pytest.mark.parametrize("consumer", ["matmul", "softmax_matmul", "displacement", "logsumexp", "topk"])
def test_batched_consumers(bx, consumer):
    """One launch for the whole batch (the plan's batch field), each element
    against the oracle; X of batch one broadcasts."""
    r = np.random.default_rng(4000 + bx)
    B, N, M, D = 3, 140, 170, 20
    X = r.standard_normal((bx, N, D)).astype(np.float32)
    Y = r.standard_normal((B, M, D)).astype(np.float32)
    V = r.standard_normal((B, M, 6)).astype(np.float32)
    bias = r.standard_normal((B, N)).astype(np.float32)
    e = pw.lazy(to_dev(X), to_dev(Y), "rbf", gamma=0.05, ops=[("add_rows", to_dev(bias))])
    assert _batch_of(e.plan(consumer, 6 if consumer in ("matmul", "softmax_matmul") else 0,
                            5 if consumer == "topk" else 0)) == B
    if consumer in ("matmul", "softmax_matmul"):
        out = getattr(e, consumer)(to_dev(V))
    elif consumer == "displacement":
        out = e.displacement()
    elif consumer == "logsumexp":
        out = e.logsumexp()
    else:
        vals, idx = e.topk(5)
    for b in range(B):
        oe = oracle.Expr(X[b if bx > 1 else 0], Y[b], "rbf", 0.05, [("add_rows", bias[b])])
        if consumer == "topk":
            ov, oi, om = oracle.topk(oe, 5, extra=8)
            assert_topk(vals[b].cpu().numpy(), idx[b].cpu().numpy(), ov, oi, om, 5, False, np.float32, what="b%d" % b)
            continue
        if consumer == "matmul":
            o, mag = oracle.matmul(oe, V[b])
        elif consumer == "softmax_matmul":
            o, mag = oracle.softmax_matmul(oe, V[b])
        elif consumer == "displacement":
            o, mag = oracle.displacement(oe)
        else:
            o, mag = oracle.logsumexp(oe)
        vmax = float(np.max(np.abs(V[b]))) if consumer in ("matmul", "softmax_matmul") else 1.0
        if consumer == "displacement":
            vmax = float(max(np.max(np.abs(X)), np.max(np.abs(Y)), 1))
        assert_values(out[b].cpu().numpy(), o, mag, np.float32, n_terms=M, vmax=vmax, what="b%d" % b)


def test_batched_column_min_and_grad():
    """Chamfer in a batch: min over both dims per element, and gradients of
    a batched log-sum-exp flow back to every element's X and Y."""
    r = np.random.default_rng(4100)
    X = torch.tensor(r.standard_normal((2, 60, 3)), device="cuda", requires_grad=True)
    Y = torch.tensor(r.standard_normal((2, 80, 3)), device="cuda", requires_grad=True)
    D = pw.lazy(X, Y, "sqeuclidean")
    v1, i1 = D.min(-1)
    v2, i2 = D.min(-2)
    for b in range(2):
        S = torch.cdist(X[b].detach(), Y[b].detach()) ** 2
        assert torch.equal(i1[b], S.argmin(1)) and torch.equal(i2[b], S.argmin(0))
    lse = pw.lazy(X, Y, "sqeuclidean", ops=[("mul", -1.0)]).logsumexp()
    gX, gY = torch.autograd.grad(lse.sum(), [X, Y])
    Xd, Yd = X.detach().requires_grad_(True), Y.detach().requires_grad_(True)
    ref = torch.logsumexp(-((Xd[:, :, None, :] - Yd[:, None, :, :]) ** 2).sum(-1), -1).sum()
    rX, rY = torch.autograd.grad(ref, [Xd, Yd])
    assert torch.allclose(gX, rX, rtol=1e-9, atol=1e-10) and torch.allclose(gY, rY, rtol=1e-9, atol=1e-10)


ENGINES = [("valu", 3, np.float32), ("mfma", 32, np.float32), ("valu", 5, np.float64), ("mfma", 16, np.float64)]


@pytest.mark.parametrize("family,D,dtype", ENGINES, ids=["%s-D%d-%s" % (f, d, np.dtype(t).name) for f, d, t in ENGINES])
@pytest.mark.parametrize("consumer", ["matmul", "softmax_matmul", "displacement", "logsumexp", "topk"])
def test_many_small_batches(family, D, dtype, consumer):
    """Forty small elements in one launch on either engine, with a shared and
    a per-element op vector, a shared column mask, ragged sizes, shared Y
    for the column-norm pre-pass, and exact self exclusion per element."""
    r = np.random.default_rng(4200 + D)
    B, N, M = 40, 37, 53
    X = r.standard_normal((B, N, D)).astype(dtype)
    Y = r.standard_normal((1, M, D)).astype(dtype)
    V = r.standard_normal((B, M, 5)).astype(dtype)
    w = (0.5 + r.random((B, N))).astype(dtype)
    b = r.standard_normal(M).astype(dtype)
    keep = r.random(M) < 0.85
    # The matrix cores take a row-only stage; the vector engine any chain.
    col = [] if family == "mfma" else [("add_columns", b)]
    host_ops = [("mul", 1.0 / np.sqrt(D)), ("weight_rows", w)] + col + [("mask_columns", keep)]
    ops = [(n, to_dev(a) if isinstance(a, np.ndarray) else a) for n, a in host_ops]
    metric = "linear" if consumer in ("softmax_matmul", "logsumexp") else "sqeuclidean"
    e = pw.lazy(to_dev(X), to_dev(Y), metric, ops=ops)
    C = 5 if consumer in ("matmul", "softmax_matmul") else 0
    plan = e.plan(consumer, C, 4 if consumer == "topk" else 0)
    want = "mfma" if family == "mfma" and not (consumer in ("matmul", "softmax_matmul") and D < 32) else "valu"
    assert _batch_of(plan) == B and plan.startswith("family=" + want), plan
    if consumer == "topk":
        vals, idx = e.topk(4)
    elif consumer in ("matmul", "softmax_matmul"):
        out = getattr(e, consumer)(to_dev(V))
    elif consumer == "displacement":
        out = e.displacement()
    else:
        out = e.logsumexp()
    for bb in range(B):
        oe = oracle.Expr(X[bb], Y[0], metric, 1.0,
                         [(n, a[bb] if n == "weight_rows" else a) for n, a in host_ops])
        if consumer == "topk":
            ov, oi, om = oracle.topk(oe, 4, extra=8)
            assert_topk(vals[bb].cpu().numpy(), idx[bb].cpu().numpy(), ov, oi, om, 4, False, dtype, what="b%d" % bb)
            continue
        if consumer in ("matmul", "softmax_matmul"):
            o, mag = getattr(oracle, consumer)(oe, V[bb])
            vmax = float(np.max(np.abs(V[bb])))
        elif consumer == "displacement":
            o, mag = oracle.displacement(oe)
            vmax = float(max(np.max(np.abs(X)), np.max(np.abs(Y)), 1))
        else:
            o, mag = oracle.logsumexp(oe)
            vmax = 1.0
        assert_values(out[bb].cpu().numpy(), o, mag, dtype, n_terms=M, vmax=vmax, what="b%d" % bb)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_batched_exclude_self_per_element(dtype):
    """InfoNCE-style log-sum-exp over a batch of square elements: each
    element drops its own diagonal."""
    r = np.random.default_rng(4300)
    B, N, D = 6, 90, 24
    Z = r.standard_normal((B, N, D)).astype(dtype)
    e = pw.lazy(to_dev(Z), to_dev(Z), "linear", ops=[("mul", 0.2)])
    assert _batch_of(e.plan("logsumexp")) == B
    got = e.logsumexp(exclude_self=True).cpu().numpy()
    for bb in range(B):
        o, mag = oracle.logsumexp(oracle.Expr(Z[bb], Z[bb], "linear", 1.0, [("mul", 0.2)]), exclude_self=True)
        assert_values(got[bb], o, mag, dtype, n_terms=N, what="b%d" % bb)
