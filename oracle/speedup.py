"""O8: bookkeeping formulas for acceptance length, latency and speedup.

[SD] Module 4: under independent acceptance with rate alpha,
tau = sum_{i=0..gamma} alpha^i = (1 - alpha^(gamma+1)) / (1 - alpha), so
1 <= tau <= gamma+1.
[SSR] section 2.2 and the back-solved denominators after section 7.1:
speedup = tau / (D * t_draft / t_target + g_v), so tau / speedup is the
implied denominator.  [SSL] section 1: S(k) = (alpha k + 1) / (k c + 1) with
c = C_d / C_v, and dS/dk has the sign of alpha - c.

Pinned by the pages' own arithmetic (tests/golden/page_arithmetic.json).
"""


def tau_iid(alpha, gamma):
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def expected_accepted(alphas):
    """E[n] = sum_{m>=1} prod_{i<=m} alpha_i for position-wise acceptance rates."""
    total, run = 0.0, 1.0
    for a in alphas:
        run *= a
        total += run
    return total


def implied_denominator(tau, speedup):
    return tau / speedup


def subspec_speedup(tau, depth, t_draft, t_target, g_v):
    return tau / (depth * t_draft / t_target + g_v)


def sparsespec_speedup(alpha, k, c):
    return (alpha * k + 1.0) / (k * c + 1.0)


def sparsespec_cost_ratio(alpha, k, speedup):
    """Solve S = (alpha k + 1)/(k c + 1) for c."""
    return ((alpha * k + 1.0) / speedup - 1.0) / k


def kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_elem=2):
    return n_layers * n_kv_heads * head_dim * 2 * bytes_per_elem
