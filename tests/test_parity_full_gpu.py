"""Full-size workloads on the GPU, in the launch configuration the benchmark
times, checked against the oracle on a row sample: every 61st row (or a
coarser stride for the largest sweeps) plus the first and last 256 rows, so
every tile position and both ragged ends are covered."""
import numpy as np
import pytest

import workloads
from gpu_cases import bind_both, bind_case, check_consumer

pytestmark = pytest.mark.gpu

STRIDE = {"knn": 257, "svgd": 151}


@pytest.mark.parametrize("name", list(workloads.WORKLOADS.keys()))
def test_full_size_workload(name):
    import oracle
    import os
    oracle.set_threads(len(os.sched_getaffinity(0)))
    arrays, cases = workloads.make(name)
    for c in cases:
        e, oe = bind_case(arrays, c)
        rows = workloads.sample_rows(oe.N, stride=STRIDE.get(name, 61))
        V = arrays[c.v] if c.v else None
        ratio, rel = check_consumer(e, oe, c.consumer, V=V, exclude_self=c.exclude_self, k=c.k,
                                    largest=c.largest, rows=rows, what="%s/%s" % (name, c.name),
                                    params={k: workloads.resolve(v, arrays) for k, v in c.params.items()})
        print("%s/%s: %d rows, worst err/tol %.3g, plan %s" % (name, c.name, len(rows), ratio,
                                                              e.plan(*_plan_args(c, V))))


def _plan_args(c, V):
    if c.consumer in ("mean", "cg_solve", "mmd"):
        return "matmul", 1, 0
    if c.consumer.startswith("backward_"):
        return c.consumer[len("backward_"):], V.shape[1] if V is not None else 0, c.k
    return c.consumer, V.shape[1] if V is not None else 0, c.k
