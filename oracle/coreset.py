"""Tail coreset of the exp kernel by discrepancy halving, kept with Merge-and-Reduce
(float64).  TEST INFRASTRUCTURE ONLY: see the package header.

What the pages say ("Rumo a Limites Estritos para Atenção em Streaming",
"Metodologia" > "1. Limites Superiores Algorítmicos"; the French page
"Vers des Bornes Serrées pour l'Attention en Flux", "Constructions de Coresets
basées sur la Discrépance"): small weighted subsets of the data (coresets) built
with discrepancy theory (they name the results of Charikar, Kapralov and
Waingarten, CKW'24, and Banaszczyk's theorem) approximate the kernel density for
every query, and serve the "tail" of the exponential kernel's expansion, while the
polynomial method's low-degree moments serve its "head"; the streaming algorithm
puts the pieces together with Merge-and-Reduce (closing paragraph of the same
section).  The pages name results, not a procedure.  The readings taken here:

* Head and tail.  e^x = T_p(x) + R_p(x), T_p the degree-p Taylor polynomial and
  R_p(x) = sum_{j > p} x^j / j! the tail.  The head sums sum_i T_p(<q,k_i>) [1, v_i]
  come from the moment sketch (exact); the tail sums sum_i R_p(<q,k_i>) [1, v_i]
  come from a weighted subset S: sum_{s in S} w_s R_p(<q,k_s>) [1, v_s].  R_p(<k,k'>)
  is a positive-definite kernel (a sum of the polynomial kernels <k,k'>^j with
  positive weights), with features phi_t(k) = (k^(x)j / sqrt(j!))_{j > p}.
* Halving (the "reduce" of Merge-and-Reduce).  The self-balancing walk of Alweiss,
  Liu and Sawhney ("Discrepancy minimization via a self-balancing walk", STOC
  2021), run on consecutive pairs as kernel thinning does (Dwivedi and Mackey,
  "Kernel Thinning", 2021): a block of 2B points is read as B pairs (x_2t,
  x_2t+1); each point has the vector u(x) = phi_t(k) (x) [1; v], so
  <u(x), u(y)> = R_p(<k_x, k_y>) (1 + <v_x, v_y>) serves the normaliser and the
  attention numerator at once.  With f_t = u(x_2t) - u(x_2t+1) and the running
  signed sum psi (psi = 0 at the start), pair t takes alpha_t = <psi, f_t>, the
  probability P_t = (1 - alpha_t / c) / 2 clamped to [0, 1], a uniform U_t, and
  eps_t = +1 when U_t < P_t, else -1; psi += eps_t f_t.  eps_t = +1 keeps x_2t+1,
  -1 keeps x_2t; the kept point's weight doubles.  Then
      sum over the 2B points of u - 2 sum over the kept points of u = psi,
  so the walk keeps the tail sums' error at <psi, phi_t(q) (x) e_c>.  Threshold
  c = c0 * max_t |f_t|^2 (the walk's unit-norm scale times c0; the published
  constant 30 log(mn/delta) serves the proof); where |alpha_t| > c the walk would
  stop in the published form, here the probability is clamped (the sign is then
  the one that shrinks psi along f_t).
* Random numbers.  U_t comes from SplitMix64 (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014) used as a
  counter-based generator: output number `counter` of the sequence started at
  state `seed` is mix(seed + (counter + 1) * 0x9E3779B97F4A7C15), and
  U = (output >> 11) * 2^-53.  The counter of pair t in the r-th reduce of a
  handle (r = 0, 1, ... in the order reduces happen), head h of H, blocks of B
  pairs, is (r * H + h) * B + t.
* Merge-and-Reduce.  Incoming points of weight 1 fill a buffer of B points; a
  full buffer becomes a block of level 0.  Two blocks of level l (the older one
  first) are merged into 2B points and halved into one block of level l + 1 (weight
  2^(l+1)), as in a binary counter.  After n points per head, level l holds a block
  exactly when bit l of floor(n / B) is set, and the buffer holds n mod B points.

Answer with the tail: Zhat = Zhat_head + tailZ, ohat = (Ntilde_head + tailN) / Zhat,
with the head from the moments and the tail from the coreset.
"""

import math

import numpy as np

from .sketch import taylor_exp

GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_M64 = (1 << 64) - 1


def splitmix64(seed, counter):
    """Output number `counter` (0-based; int or array of non-negative ints) of the
    SplitMix64 sequence whose state starts at `seed`, as numpy uint64."""
    c = np.asarray(counter, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & _M64) + (c + np.uint64(1)) * np.uint64(GOLDEN_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def uniforms(seed, serial, head, heads, B):
    """U_t in [0, 1) of the `serial`-th reduce for one head: B pairs."""
    base = (int(serial) * int(heads) + int(head)) * int(B)
    z = splitmix64(seed, np.arange(base, base + B, dtype=np.uint64))
    return (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def tail_exp(x, p):
    """R_p(x) = e^x - T_p(x) = sum_{j > p} x^j / j!, elementwise, float64.

    Two evaluations, and per element the one whose rounding is smaller: the
    series itself (terms by the ratio x / j, summed until they no longer change
    the sum; its rounding scales with its largest term) and e^x - T_p(x) (its
    rounding scales with e^x + sum_{j <= p} |x|^j / j!).  For x >= 0 the series
    has no cancellation at all."""
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    x = x.reshape(-1)
    # the series, capped at |x| <= 40 (beyond, the direct form is the accurate one)
    xs = np.clip(x, -40.0, 40.0)
    term = np.ones_like(xs)
    for j in range(1, p + 2):
        term = term * xs / j                    # x^(p+1) / (p+1)! after the loop
    acc = term.copy()
    big = np.abs(term)
    j = p + 1
    while True:
        j += 1
        term = term * xs / j
        new = acc + term
        big = np.maximum(big, np.abs(term))
        if (np.all(new == acc) and j > 2 * np.abs(xs).max()) or j > p + 400:
            break
        acc = new
    # the direct form and its magnitude
    head_mag = np.zeros_like(x)
    t = np.ones_like(x)
    for i in range(p + 1):
        if i > 0:
            t = t * np.abs(x) / i
        head_mag += t
    with np.errstate(over="ignore"):
        ex = np.exp(x)
    direct = ex - taylor_exp(x, p)
    use_series = (big <= ex + head_mag) & (np.abs(x) <= 40.0)
    return np.where(use_series, acc, direct).reshape(shape)


def tail_gram(K, V, p):
    """<u(x_i), u(x_j)> = R_p(<k_i, k_j>) (1 + <v_i, v_j>) for all point pairs."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    return tail_exp(K @ K.T, p) * (1.0 + V @ V.T)


def halve(K, V, p, c0, U):
    """One reduce: 2B points (pairs (2t, 2t+1)) -> indices of the B kept points.

    Returns a dict: kept [B] (indices into the block), eps [B] (+-1), alpha [B]
    (the walk's <psi, f_t> before each decision), prob [B], c (the threshold),
    D [B][B] (<f_t, f_s>)."""
    K = np.asarray(K, dtype=np.float64)
    n2 = K.shape[0]
    assert n2 % 2 == 0
    B = n2 // 2
    G = tail_gram(K, V, p)
    a = np.arange(0, n2, 2)
    b = a + 1
    D = G[np.ix_(a, a)] - G[np.ix_(a, b)] - G[np.ix_(b, a)] + G[np.ix_(b, b)]
    c = c0 * float(np.max(np.diag(D))) if B > 0 else 0.0
    alpha = np.zeros(B)
    run = np.zeros(B)                     # <psi, f_s> for every pair, kept current
    eps = np.zeros(B)
    prob = np.zeros(B)
    for t in range(B):
        alpha[t] = run[t]
        pt = 0.5 if c <= 0.0 else min(1.0, max(0.0, 0.5 * (1.0 - run[t] / c)))
        prob[t] = pt
        e = 1.0 if U[t] < pt else -1.0
        eps[t] = e
        run += e * D[t]                   # psi gains e f_t
    kept = np.where(eps > 0, b, a)
    return {"kept": kept, "eps": eps, "alpha": alpha, "prob": prob, "c": c, "D": D}


class MergeReduceCoreset:
    """Merge-and-Reduce coreset of one head (see the module header).

    seed, heads and head fix the uniforms: the same (seed, heads) and call
    sequence give every head of a multi-head handle its own draws."""

    def __init__(self, d, dv, p, B, c0, seed, heads=1, head=0):
        self.d, self.dv, self.p, self.B, self.c0 = d, dv, p, int(B), float(c0)
        self.seed, self.heads, self.head = int(seed), int(heads), int(head)
        self.levels = []                  # level l: None or (K [B][d], V [B][dv])
        self.fillK = np.zeros((0, d))
        self.fillV = np.zeros((0, dv))
        self.serial = 0                   # reduces done so far
        self.count = 0

    def _carry(self, K, V, l=0):
        """A block of level l enters; two blocks of one level merge and halve."""
        while True:
            while l >= len(self.levels):
                self.levels.append(None)
            if self.levels[l] is None:
                self.levels[l] = (K, V)
                return
            K0, V0 = self.levels[l]
            Km = np.concatenate([K0, K])
            Vm = np.concatenate([V0, V])
            U = uniforms(self.seed, self.serial, self.head, self.heads, self.B)
            self.serial += 1
            r = halve(Km, Vm, self.p, self.c0, U)
            K, V = Km[r["kept"]], Vm[r["kept"]]
            self.levels[l] = None
            l += 1

    def update(self, K, V):
        K = np.asarray(K, dtype=np.float64).reshape(-1, self.d)
        V = np.asarray(V, dtype=np.float64).reshape(-1, self.dv)
        self._append(K, V)
        self.count += K.shape[0]
        return self

    def merge(self, other):
        """Merge-and-Reduce across sub-streams: other's buffered points enter this
        buffer in their order (a full buffer carries in at level 0), then other's
        blocks carry in at their own levels, lowest level first.  other is
        unchanged."""
        assert (other.d, other.dv, other.p, other.B) == (self.d, self.dv, self.p, self.B)
        self._append(other.fillK, other.fillV)
        for l, blk in enumerate(other.levels):
            if blk is not None:
                self._carry(blk[0], blk[1], l)
        self.count += other.count
        return self

    def _append(self, K, V):
        i = 0
        while i < K.shape[0]:
            take = min(self.B - self.fillK.shape[0], K.shape[0] - i)
            self.fillK = np.concatenate([self.fillK, K[i:i + take]])
            self.fillV = np.concatenate([self.fillV, V[i:i + take]])
            i += take
            if self.fillK.shape[0] == self.B:
                Kb, Vb = self.fillK, self.fillV
                self.fillK = np.zeros((0, self.d))
                self.fillV = np.zeros((0, self.dv))
                self._carry(Kb, Vb)

    def points(self):
        """(K, V, w) of every point: the partial buffer (weight 1), then the blocks
        by level (weight 2^l)."""
        Ks, Vs, ws = [self.fillK], [self.fillV], [np.ones(self.fillK.shape[0])]
        for l, blk in enumerate(self.levels):
            if blk is not None:
                Ks.append(blk[0])
                Vs.append(blk[1])
                ws.append(np.full(blk[0].shape[0], float(2 ** l)))
        return np.concatenate(Ks), np.concatenate(Vs), np.concatenate(ws)

    def tail_query(self, Q):
        """(tailN [m][dv], tailZ [m]) = sum_s w_s R_p(<q, k_s>) [v_s, 1]."""
        K, V, w = self.points()
        W = tail_exp(np.asarray(Q, dtype=np.float64) @ K.T, self.p) * w[None, :]
        return W @ V, W.sum(axis=1)


def tail_direct(K, V, Q, p):
    """The exact tail sums over every key: (sum_i R_p(<q,k_i>) v_i, sum_i R_p(<q,k_i>))."""
    W = tail_exp(np.asarray(Q, np.float64) @ np.asarray(K, np.float64).T, p)
    return W @ np.asarray(V, np.float64), W.sum(axis=1)


def answer_with_tail(head_out, head_Z, tailN, tailZ):
    """Head (ohat, Zhat from the moments) plus tail sums -> (ohat, Zhat)."""
    head_out = np.asarray(head_out, np.float64)
    head_Z = np.asarray(head_Z, np.float64)
    Z = head_Z + tailZ
    return (head_out * head_Z[:, None] + tailN) / Z[:, None], Z
