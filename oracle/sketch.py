"""Degree-p Taylor moment sketch of the exp kernel, float64 (test infrastructure only).

Source: "Rumo a Limites Estritos para Atenção em Streaming" (gist.science, pt),
"Metodologia", pillar "O Método Polinomial"; French page "Vers des Bornes Serrées
pour l'Attention en Flux", "Méthodologie", "La Méthode Polynomiale".  The pages
say the head of the exponential kernel is approximated by a truncated Taylor
expansion and that a sketch of the data's low-degree moments is kept.  Reading
taken (the pages give no formula):

    exp<q, k>  ~  T_p(<q, k>),   T_p(x) = sum_{j=0}^{p} x^j / j!
    <q, k>^j   =  <q^(x)j, k^(x)j>        (j-fold Kronecker powers)

so with the moments  M_j = sum_i k_i^(x)j  and  N_j = sum_i k_i^(x)j v_i^T
(j = 0..p; M_0 = n, N_0 = sum_i v_i):

    Zhat(q) = sum_j <q^(x)j, M_j> / j!
    ohat(q) = (sum_j <q^(x)j, N_j> / j!) / Zhat(q)

Two routes are given.  ``sketch_direct`` is the plain definition of the value the
method reaches: Zhat = sum_i T_p(<q, k_i>), Ntilde = sum_i T_p(<q, k_i>) v_i.
``MomentSketch`` takes the method's steps in order: build the Kronecker features
level by level, accumulate the moments chunk by chunk, merge by addition, and
answer a query from the moments with the 1/j! weights.

Feature order: level j is the row-major Kronecker power, i.e. entry
a*d + b of level j is (entry a of level j-1) * k[b]; levels are stacked j = 0..p,
so level j starts at row 1 + d + ... + d^(j-1).  D = sum_{j<=p} d^j rows in all.
"""

import math

import numpy as np


def taylor_exp(x, p):
    """T_p(x) = sum_{j=0}^{p} x^j / j!, elementwise, float64."""
    x = np.asarray(x, dtype=np.float64)
    term = np.ones_like(x)
    total = np.ones_like(x)
    for j in range(1, p + 1):
        term = term * x / j                     # x^j / j!
        total = total + term
    return total


def sketch_direct(K, V, Q, p, max_block_entries=1 << 24):
    """(ohat [m, dv], Zhat [m]) by the definition sum_i T_p(<q, k_i>) [1, v_i]."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    n, m, dv = K.shape[0], Q.shape[0], V.shape[1]
    Z = np.zeros(m)
    Nt = np.zeros((m, dv))
    bq = max(1, max_block_entries // max(n, 1))
    for q0 in range(0, m, bq):
        q1 = min(m, q0 + bq)
        w = taylor_exp(Q[q0:q1] @ K.T, p)       # T_p(<q, k_i>)
        Z[q0:q1] = w.sum(axis=1)
        Nt[q0:q1] = w @ V
    with np.errstate(invalid="ignore", divide="ignore"):
        out = Nt / Z[:, None]
    return out, Z


def feature_map(X, p):
    """Kronecker-power features of the rows of X: list of levels j = 0..p.

    Level j is an array [rows, d^j]; level 0 is all ones.  Entry a*d + b of level
    j is entry a of level j-1 times X[:, b] (row-major Kronecker order).
    """
    X = np.asarray(X, dtype=np.float64)
    rows, d = X.shape
    levels = [np.ones((rows, 1))]
    for _ in range(p):
        prev = levels[-1]
        levels.append((prev[:, :, None] * X[:, None, :]).reshape(rows, -1))
    return levels


class MomentSketch:
    """The moment sketch state and its four operations, one head, float64.

    State: M[j] (shape [d^j]) and N[j] (shape [d^j, dv]) for j = 0..p, and the
    number of keys ingested.  M[0] equals that count.
    """

    def __init__(self, d, dv, p):
        if d < 1 or dv < 1 or p < 0:
            raise ValueError("need d >= 1, dv >= 1, p >= 0")
        self.d, self.dv, self.p = d, dv, p
        self.M = [np.zeros(d ** j) for j in range(p + 1)]
        self.N = [np.zeros((d ** j, dv)) for j in range(p + 1)]
        self.count = 0

    @property
    def D(self):
        return sum(self.d ** j for j in range(self.p + 1))

    def update(self, K, V, chunk=256):
        """Ingest keys K [n, d] with values V [n, dv]: M_j += sum_i k_i^(x)j,
        N_j += sum_i k_i^(x)j v_i^T, processed ``chunk`` keys at a time."""
        K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64)
        n = K.shape[0]
        for c0 in range(0, n, chunk):
            Kc, Vc = K[c0:c0 + chunk], V[c0:c0 + chunk]
            for j, F in enumerate(feature_map(Kc, self.p)):
                self.M[j] += F.sum(axis=0)
                self.N[j] += F.T @ Vc
        self.count += n
        return self

    def merge(self, other):
        """Add another sketch of the same shape (the Merge step)."""
        if (self.d, self.dv, self.p) != (other.d, other.dv, other.p):
            raise ValueError("shape mismatch")
        for j in range(self.p + 1):
            self.M[j] += other.M[j]
            self.N[j] += other.N[j]
        self.count += other.count
        return self

    def query(self, Q):
        """(ohat [m, dv], Zhat [m]) from the moments:
        Zhat = sum_j <q^(x)j, M_j>/j!, Ntilde = sum_j <q^(x)j, N_j>/j!."""
        Q = np.asarray(Q, dtype=np.float64)
        m = Q.shape[0]
        Z = np.zeros(m)
        Nt = np.zeros((m, self.dv))
        for j, F in enumerate(feature_map(Q, self.p)):
            inv_fact = 1.0 / math.factorial(j)
            Z += (F @ self.M[j]) * inv_fact
            Nt += (F @ self.N[j]) * inv_fact
        with np.errstate(invalid="ignore", divide="ignore"):
            out = Nt / Z[:, None]
        return out, Z

    def canonical_state(self):
        """[M | N] as one array [D, 1 + dv]: levels stacked j = 0..p."""
        return np.concatenate(
            [np.concatenate([self.M[j][:, None], self.N[j]], axis=1)
             for j in range(self.p + 1)], axis=0)


def sketch_direct_centered(K, V, Q, p, c):
    """The sketch recentred at a fixed centre c, by its plain definition.

    Source: "Metodologia", pillar "Particionamento de Espaço e Recentramento"
    (French page: "Partition de l'Espace et Recentrage"): a dense cluster is
    shifted to the origin, which shrinks the radius the expansion has to cover.
    Reading taken for one fixed centre (the recursive Partition is not built):

        Zhat_c(q) = e^{<q,c>} sum_i T_p(<q, k_i - c>),
        Ntilde_c(q) = e^{<q,c>} sum_i T_p(<q, k_i - c>) v_i,   ohat = Ntilde / Zhat,

    exact in the limit p -> infinity because e^{<q,c>} e^{<q, k - c>} = e^{<q, k>}.
    The moments are those of the shifted keys k - c; the factor e^{<q,c>} cancels
    in ohat.  Returns (ohat [m, dv], Zhat [m])."""
    K = np.asarray(K, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    out, Z = sketch_direct(K - c[None, :], V, Q, p)
    return out, Z * np.exp(Q @ c)
