"""Error bounds of the degree-p Taylor sketch against the exact path (float64).

Derived here (the pages "Rumo a Limites Estritos para Atenção em Streaming",
"Principais Resultados", state only asymptotic space bounds):

Let s_i = <q, k_i> with |s_i| <= rho (rho = max|q| * max|k| bounds every score),
E_i = e^(s_i), T_i = T_p(s_i), delta_i = T_i - E_i.  Lagrange's remainder gives

    |delta_i| <= eps1 := rho^(p+1) / (p+1)! * e^rho                  (per term)

and since E_i >= e^(-rho):

    |Zhat - Z| / Z <= n eps1 / (n e^(-rho)) = rho^(p+1) / (p+1)! * e^(2 rho).

For the attention output, ohat - o = sum_i delta_i (v_i - o) / Zhat (expand
Ntilde/Zhat - N/Z), each coordinate of v_i - o lies within the range of that
coordinate over the v_i (o is a convex combination of them), and
Zhat >= n (e^(-rho) - eps1), so per coordinate c

    |ohat_c - o_c| <= eps1 * range_c / (e^(-rho) - eps1)   when eps1 < e^(-rho),

and no finite bound otherwise.
"""

import math

import numpy as np


def measured_radius(K, Q):
    """rho = max_i |k_i| * max_q |q| of the given (fp32 or fp64) arrays."""
    K = np.asarray(K, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    if K.shape[0] == 0 or Q.shape[0] == 0:
        return 0.0
    return float(np.linalg.norm(K, axis=1).max() * np.linalg.norm(Q, axis=1).max())


def taylor_term_bound(p, rho):
    """eps1 = rho^(p+1)/(p+1)! * e^rho >= |e^x - T_p(x)| for |x| <= rho."""
    return rho ** (p + 1) / math.factorial(p + 1) * math.exp(rho)


def kde_relative_bound(p, rho):
    """Bound on |Zhat - Z| / Z: rho^(p+1)/(p+1)! * e^(2 rho)."""
    return taylor_term_bound(p, rho) * math.exp(rho)


def attention_abs_bound(p, rho, V):
    """Per-coordinate bound on |ohat - o| (array [dv]); inf where none holds."""
    V = np.asarray(V, dtype=np.float64)
    rng = V.max(axis=0) - V.min(axis=0)
    eps1 = taylor_term_bound(p, rho)
    denom = math.exp(-rho) - eps1
    if denom <= 0:
        return np.full(V.shape[1], np.inf)
    return eps1 * rng / denom
