"""Symmetric (multiset) storage of the Taylor moments, float64 (test infrastructure only).

Source: "Rumo a Limites Estritos para Atenção em Streaming" (gist.science, pt),
"Metodologia", pillar "O Método Polinomial": the stream is summarised by its
low-degree moments; the pages leave the storage of those moments open.

The moment tensors M_j = sum_i k_i^(x)j and N_j = sum_i k_i^(x)j v_i^T are
symmetric in their j tensor indices: the entry at (a_1, ..., a_j) depends only on
the multiset {a_1, ..., a_j}.  This module keeps one entry per multiset:

    M^s_j[alpha] = sum_i k_i^alpha,   N^s_j[alpha] = sum_i k_i^alpha v_i^T,
    k^alpha = prod_l k[a_l]  for the sorted tuple alpha = (a_1 <= ... <= a_j).

A multiset alpha with multiplicities c_0 .. c_{d-1} stands for j! / alpha! index
tuples of the Kronecker power, alpha! = prod_a c_a!, so

    <q^(x)j, M_j> / j!  =  sum_alpha  q^alpha M^s_j[alpha] / alpha!

and the same for N: the query weight of a stored entry is q^alpha / alpha!.

Row order: level j holds the sorted tuples in lexicographic order (the order of
``itertools.combinations_with_replacement``), C(d + j - 1, j) rows; levels are
stacked j = 0..p, C(d + p, p) rows in all.
"""

import itertools
import math

import numpy as np


def multisets(d, j):
    """The sorted index tuples of level j, [C(d + j - 1, j), j] int array."""
    rows = list(itertools.combinations_with_replacement(range(d), j))
    return np.array(rows, dtype=np.int64).reshape(len(rows), j)


def alpha_factorial(tuples):
    """alpha! = product over distinct indices of (multiplicity)!, per row."""
    out = np.ones(tuples.shape[0])
    for r, row in enumerate(tuples):
        for _, grp in itertools.groupby(row):
            out[r] *= math.factorial(len(list(grp)))
    return out


def sym_features(X, p):
    """Monomial features X^alpha of the rows of X, list of levels j = 0..p,
    level j an array [rows, C(d + j - 1, j)] in the row order above."""
    X = np.asarray(X, dtype=np.float64)
    n, d = X.shape
    levels = []
    for j in range(p + 1):
        tup = multisets(d, j)
        if j == 0:
            levels.append(np.ones((n, 1)))
        else:
            levels.append(np.prod(X[:, tup], axis=2))
    return levels


class SymMomentSketch:
    """The moment sketch in multiset storage, one head, float64.

    State: M[j] (shape [R_j]) and N[j] (shape [R_j, dv]) for j = 0..p, R_j the
    number of multisets of size j, and the number of keys ingested (= M[0]).
    """

    def __init__(self, d, dv, p):
        if d < 1 or dv < 1 or p < 0:
            raise ValueError("need d >= 1, dv >= 1, p >= 0")
        self.d, self.dv, self.p = d, dv, p
        self.tuples = [multisets(d, j) for j in range(p + 1)]
        self.weights = [1.0 / alpha_factorial(t) for t in self.tuples]
        self.M = [np.zeros(len(t)) for t in self.tuples]
        self.N = [np.zeros((len(t), dv)) for t in self.tuples]
        self.count = 0

    @property
    def rows(self):
        return sum(len(t) for t in self.tuples)

    def update(self, K, V, chunk=256):
        """Ingest keys K [n, d] with values V [n, dv], ``chunk`` keys at a time."""
        K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64)
        n = K.shape[0]
        for c0 in range(0, n, chunk):
            Kc, Vc = K[c0:c0 + chunk], V[c0:c0 + chunk]
            for j, F in enumerate(sym_features(Kc, self.p)):
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
        """(ohat [m, dv], Zhat [m]): Zhat = sum_alpha q^alpha M^s[alpha] / alpha!,
        Ntilde likewise with N^s."""
        Q = np.asarray(Q, dtype=np.float64)
        m = Q.shape[0]
        Z = np.zeros(m)
        Nt = np.zeros((m, self.dv))
        for j, F in enumerate(sym_features(Q, self.p)):
            Fw = F * self.weights[j][None, :]
            Z += Fw @ self.M[j]
            Nt += Fw @ self.N[j]
        with np.errstate(invalid="ignore", divide="ignore"):
            out = Nt / Z[:, None]
        return out, Z

    def canonical_state(self):
        """[M^s | N^s] as one array [C(d + p, p), 1 + dv]: levels stacked j = 0..p."""
        return np.concatenate(
            [np.concatenate([self.M[j][:, None], self.N[j]], axis=1)
             for j in range(self.p + 1)], axis=0)

    def expand_full(self):
        """The same moments in the Kronecker layout [D, 1 + dv] (D = sum_j d^j,
        row-major index tuples): the entry of index tuple (a_1, ..., a_j) is the
        stored entry of its sorted tuple."""
        d, blocks = self.d, []
        for j in range(self.p + 1):
            where = {tuple(t): r for r, t in enumerate(self.tuples[j])}
            S = np.concatenate([self.M[j][:, None], self.N[j]], axis=1)
            rows = [where[tuple(sorted(idx))] for idx in itertools.product(range(d), repeat=j)]
            blocks.append(S[rows])
        return np.concatenate(blocks, axis=0)
