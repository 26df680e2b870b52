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


@pytest.mark.parametrize("bx", [1, 3])
@pytest.mark.parametrize("consumer", ["matmul", "softmax_matmul", "displacement", "logsumexp", "topk"])
def test_batched_consumers(bx, consumer):
    r = np.random.default_rng(4000 + bx)
    B, N, M, D = 3, 140, 170, 20
    X = r.standard_normal((bx, N, D)).astype(np.float32)
    Y = r.standard_normal((B, M, D)).astype(np.float32)
    V = r.standard_normal((B, M, 6)).astype(np.float32)
    bias = r.standard_normal((B, N)).astype(np.float32)
    e = pw.lazy(to_dev(X), to_dev(Y), "rbf", gamma=0.05, ops=[("add_rows", to_dev(bias))])
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
