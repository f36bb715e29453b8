"""Round cost, throughput objective and greedy stop (test infrastructure only).

[caddtree] Methodology, item 1: a round costs C(T; l) = C_d + C_v(|T|; l),
drafting plus verification of a tree of |T| nodes at context length l, and
the builder maximises the expected number of emitted tokens 1 + Phi(T) per
unit cost.  Items 3 and 4: with a mildly convex C_v the objective is unimodal
in the node count, so nodes are added one at a time (best first) and the
builder stops as soon as the marginal gain is not positive; the budget n* is
re-chosen every round.

Readings fixed here:
  * Phi_m is the sum of the first m best-first prefix probabilities (the
    drafter's surrogate for the expected accepted length; the "1 +" is the
    target's bonus token);
  * C_v(n; l) = a + b*n + c*n^2 + e*l*n + f*l, evaluated in fp64 in exactly
    the order c_d + ((((a + b*n) + c*(n*n)) + (e*l)*n) + f*l), no fused
    multiply-add (f, the part that does not grow with n, defaults to 0);
  * Phi is accumulated in fp64 in best-first order; the gain test is
    Theta(m+1) <= Theta(m) -> stop, with Theta(m) = (1 + Phi_m) / C(m);
  * n* = 0 is legal (no tree; the round still yields the bonus token).
"""


def round_cost(n: int, prefix_len: int, cost) -> float:
    """C(n; l) in fp64, fixed evaluation order."""
    n = float(n)
    l = float(prefix_len)
    f = getattr(cost, "f", 0.0)
    return cost.c_d + ((((cost.a + cost.b * n) + cost.c * (n * n)) + (cost.e * l) * n) + f * l)


def throughput(n: int, phi: float, prefix_len: int, cost) -> float:
    """Theta(n) = (1 + Phi_n) / C(n; l)."""
    return (1.0 + phi) / round_cost(n, prefix_len, cost)


def adaptive_budget(scores, cost, prefix_len: int, n_cap: int) -> int:
    """Greedy stop over best-first scores: the first m whose successor does
    not raise the throughput, or the cap, or the end of the candidates."""
    limit = min(int(n_cap), len(scores))
    phi = 0.0
    theta = throughput(0, phi, prefix_len, cost)
    m = 0
    while m < limit:
        phi_next = phi + float(scores[m])
        theta_next = throughput(m + 1, phi_next, prefix_len, cost)
        if theta_next <= theta:
            break
        phi, theta, m = phi_next, theta_next, m + 1
    return m
