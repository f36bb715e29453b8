"""Cost profiling on the GPU: measured latencies fit a non-negative, monotone,
convex model, and that fitted model drives build_tree's adaptive budget
bit-exactly like the oracle's stop rule."""

import numpy as np
import pytest
import torch

import oracle
import tree_structured_verification_amd as tsv
from tests._helpers import DEV, assert_tree_equal, oracle_trees
from tree_structured_verification_amd.profile_cost import calibrate
from workloads import Cost

pytestmark = pytest.mark.gpu


def test_measure_fit_and_drive_the_budget():
    print("profile_cost small grid", flush=True)
    cost, (n, l, t) = calibrate(4, 8, 2, 128, c_d=1.0, n_grid=(1, 8, 32, 64),
                                l_grid=(256, 1024, 4096), reps=5, warmup=1, device=DEV)
    assert n.size == 12 and np.all(t > 0)
    coef = np.array([cost.a, cost.b, cost.c, cost.e, cost.f])
    assert np.all(coef >= 0) and cost.c_d == 1.0
    ref, _ = oracle.fit_cost(n, l, t)
    A = np.stack([np.ones_like(n), n, n * n, l * n, l], 1)
    assert abs(float(np.sum((A @ coef - t) ** 2)) - float(np.sum((A @ ref - t) ** 2))) <= \
        1e-9 * float(np.sum(t * t))
    # longer prefixes never cost less under the fit
    assert float(A[-1] @ coef) >= float(A[0] @ coef)
    rng = np.random.default_rng(2)
    lg = rng.normal(0, 3, size=(6, 10, 2000))
    marg = np.exp(lg - lg.max(-1, keepdims=True))
    marg = (marg / marg.sum(-1, keepdims=True)).astype(np.float32)
    prefix = rng.integers(256, 4096, size=6).astype(np.int32)
    fitted = Cost(a=cost.a, b=cost.b, c=cost.c, e=cost.e, c_d=cost.c_d, f=cost.f)
    m = torch.from_numpy(marg).to(DEV)
    g = tsv.build_tree_fitted(m, 16, 64, 64, cost=fitted,
                              prefix_len=torch.from_numpy(prefix).to(DEV))
    torch.cuda.synchronize()
    idx, p, trees = oracle_trees(marg, 16, 64, 64, fitted, prefix)
    assert_tree_equal(g, idx, p, trees, check_topk=False)
