"""Batch-global verification budget (test infrastructure only).

[dspark] Confidence-scheduled verification, hardware-aware prefix
scheduler: the choice of verification lengths is one global throughput
maximisation over the R active requests, Theta = tau * SPS(B), with SPS(B)
a table of engine steps per second at batch size B profiled once at start-up.
Because a request's survival probabilities a_{r,j} do not increase with j, a
global sort and greedy admission respects every request's prefix order by
itself, each admission costing one table lookup; admission stops as soon as
the throughput would fall (early stopping), which finds the global maximum
when Theta is unimodal.

Readings fixed here (applied to draft trees):
  * a_{r,j} is the prefix probability of request r's j-th node in best-first
    order (the score build_tree outputs; non-increasing in j);
  * tau = R + sum of admitted a_{r,j}: every request yields its bonus token
    plus its expected accepted nodes; B = R + number of admitted nodes: every
    request verifies its root token plus its admitted nodes;
  * global order: score descending, then request index ascending, then j
    ascending (so each request's admitted nodes are a prefix of its order);
  * admit the next candidate iff (tau + a) * SPS(B + 1) > tau * SPS(B), all in
    fp64, tau accumulated in admission order; stop at the first candidate
    that fails, or when B + 1 is past the table;
  * a request's admitted count never exceeds its available count.
"""

import numpy as np


def global_order(score, n_avail):
    """Candidates (score, r, j) in admission order."""
    cands = []
    for r, n in enumerate(n_avail):
        for j in range(int(n)):
            s = float(np.float32(score[r][j]))
            cands.append((s + 0.0, r, j))   # -0.0 == +0.0
    cands.sort(key=lambda c: (-c[0], c[1], c[2]))
    return cands


def global_budget(score, n_avail, sps):
    """Admitted node count per request (int32 [R])."""
    R = len(n_avail)
    sps = np.asarray(sps, dtype=np.float64)
    counts = np.zeros(R, dtype=np.int32)
    tau = float(R)
    B = R
    for s, r, j in global_order(score, n_avail):
        if B + 1 >= len(sps):
            break
        if not (tau + s) * float(sps[B + 1]) > tau * float(sps[B]):
            break
        tau += s
        B += 1
        counts[r] += 1
    return counts
