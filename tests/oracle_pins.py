"""Pin checks for the float64 oracle, written against an implementation object.

Each ``pin_*`` function takes ``impl`` (anything with the attributes
``exact_attention``, ``sketch_direct``, ``MomentSketch`` and ``taylor_exp``, such as
the ``oracle`` package itself) and returns the largest error it finds against a
reference that does not come from the oracle: brute-force Kronecker powers
(``np.kron``), closed forms, identities, hand-worked examples, library routines
(``scipy.special``, ``mpmath``).  ``tests/test_oracle.py`` asserts the errors are at
rounding level; ``tests/test_oracle_mutants.py`` plants mistakes in copies of the
oracle and asserts that some pin catches each one.
"""

import json
import math
import os

import mpmath
import numpy as np
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def relmax(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300)))


def absmax(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def kron_power(x, j):
    """x^(x)j built by repeated np.kron (independent of the oracle's features)."""
    r = np.ones(1)
    for _ in range(j):
        r = np.kron(r, x)
    return r


def taylor_coeffs(p):
    """Taylor coefficients of exp at 0 from mpmath's numerical differentiation."""
    return [float(c) for c in mpmath.taylor(mpmath.exp, 0, p)]


def _small(seed, n, m, d, dv, scale=0.7):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, d)) * scale
    V = rng.standard_normal((n, dv))
    Q = rng.standard_normal((m, d)) * scale
    return K, V, Q


# P1: brute force with explicit tensor powers --------------------------------------

def pin_bruteforce(impl, d, p, n=23, m=4, dv=3, seed=1):
    K, V, Q = _small(seed + 10 * d + p, n, m, d, dv)
    coef = taylor_coeffs(p)
    Zb = np.zeros(m)
    Nb = np.zeros((m, dv))
    for qi in range(m):
        for i in range(n):
            w = sum(coef[j] * float(kron_power(Q[qi], j) @ kron_power(K[i], j))
                    for j in range(p + 1))
            Zb[qi] += w
            Nb[qi] += w * V[i]
    ob = Nb / Zb[:, None]
    od, Zd = impl.sketch_direct(K, V, Q, p)
    sk = impl.MomentSketch(d, dv, p).update(K, V, chunk=7)
    om, Zm = sk.query(Q)
    err = max(relmax(Zd, Zb), relmax(Zm, Zb), absmax(od, ob), absmax(om, ob))
    # the state itself: level j rows hold sum_i k_i^(x)j and sum_i k_i^(x)j v_i^T
    S = sk.canonical_state()
    off = 0
    for j in range(p + 1):
        Mj = sum(kron_power(K[i], j) for i in range(n))
        Nj = sum(np.outer(kron_power(K[i], j), V[i]) for i in range(n))
        err = max(err, absmax(S[off:off + d ** j, 0], Mj),
                  absmax(S[off:off + d ** j, 1:], Nj))
        off += d ** j
    if S.shape != (off, 1 + dv):
        return math.inf
    return err


# P2: moment route equals the direct route ----------------------------------------

def pin_moment_equals_direct(impl, K, V, Q, p, chunk=64):
    od, Zd = impl.sketch_direct(K, V, Q, p)
    sk = impl.MomentSketch(K.shape[1], V.shape[1], p).update(K, V, chunk=chunk)
    om, Zm = sk.query(Q)
    return max(relmax(Zm, Zd), absmax(om, od))


# P3: a stream of identical keys ---------------------------------------------------

def pin_identical_keys(impl, p, n=50, d=5, dv=3, seed=3):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal(d) * 0.4
    K = np.tile(k, (n, 1))
    V = rng.standard_normal((n, dv))
    Q = rng.standard_normal((6, d)) * 0.4
    coef = taylor_coeffs(p)
    s = Q @ k
    z_closed = n * np.array([sum(c * x ** j for j, c in enumerate(coef)) for x in s])
    vbar = V.mean(axis=0)
    od, Zd = impl.sketch_direct(K, V, Q, p)
    om, Zm = impl.MomentSketch(d, dv, p).update(K, V).query(Q)
    oe, Ze = impl.exact_attention(K, V, Q)
    ze_closed = n * np.array([math.exp(x) for x in s])
    return max(relmax(Zd, z_closed), relmax(Zm, z_closed), relmax(Ze, ze_closed),
               absmax(od, np.tile(vbar, (6, 1))), absmax(om, np.tile(vbar, (6, 1))),
               absmax(oe, np.tile(vbar, (6, 1))))


# P4: q = 0 -------------------------------------------------------------------------

def pin_zero_query(impl, p, n=40, d=4, dv=3, seed=4):
    K, V, _ = _small(seed, n, 1, d, dv)
    Q = np.zeros((2, d))
    vbar = np.tile(V.mean(axis=0), (2, 1))
    od, Zd = impl.sketch_direct(K, V, Q, p)
    om, Zm = impl.MomentSketch(d, dv, p).update(K, V).query(Q)
    oe, Ze = impl.exact_attention(K, V, Q)
    return max(relmax(Zd, [n, n]), relmax(Zm, [n, n]), relmax(Ze, [n, n]),
               absmax(od, vbar), absmax(om, vbar), absmax(oe, vbar))


# P5: p = 0 and p = 1 closed forms (linear attention) -------------------------------

def pin_low_orders(impl, n=30, d=4, dv=3, seed=5):
    K, V, Q = _small(seed, n, 5, d, dv)
    vbar = np.tile(V.mean(axis=0), (5, 1))
    err = 0.0
    od, Zd = impl.sketch_direct(K, V, Q, 0)
    om, Zm = impl.MomentSketch(d, dv, 0).update(K, V).query(Q)
    err = max(err, relmax(Zd, np.full(5, n)), relmax(Zm, np.full(5, n)),
              absmax(od, vbar), absmax(om, vbar))
    z1 = n + Q @ K.sum(axis=0)
    n1 = (1.0 + Q @ K.T) @ V
    od, Zd = impl.sketch_direct(K, V, Q, 1)
    om, Zm = impl.MomentSketch(d, dv, 1).update(K, V).query(Q)
    err = max(err, relmax(Zd, z1), relmax(Zm, z1),
              absmax(od, n1 / z1[:, None]), absmax(om, n1 / z1[:, None]))
    return err


# P6: merge is exact -----------------------------------------------------------------

def pin_merge(impl, p=3, d=3, dv=2, seed=6):
    K, V, Q = _small(seed, 90, 7, d, dv)
    a = impl.MomentSketch(d, dv, p).update(K[:40], V[:40])
    b = impl.MomentSketch(d, dv, p).update(K[40:], V[40:])
    whole = impl.MomentSketch(d, dv, p).update(K, V)
    a.merge(b)
    if a.count != whole.count or b.count != 50:
        return math.inf
    oa, Za = a.query(Q)
    ow, Zw = whole.query(Q)
    return max(absmax(a.canonical_state(), whole.canonical_state()),
               relmax(Za, Zw), absmax(oa, ow))


# P7: convergence to exp as p grows --------------------------------------------------

def pin_convergence(impl, seed=7):
    """Returns (max error at p=20 via the direct route, max error at p=8 via moments,
    number of increases of the error as p goes 0..14)."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((200, 2))
    K = g / np.linalg.norm(g, axis=1, keepdims=True)
    V = rng.uniform(-1, 1, (200, 2))
    g = rng.standard_normal((9, 2))
    Q = g / np.linalg.norm(g, axis=1, keepdims=True)
    oe, Ze = impl.exact_attention(K, V, Q)
    errs = []
    for p in range(0, 21):
        _, Zd = impl.sketch_direct(K, V, Q, p)
        errs.append(relmax(Zd, Ze))
    rises = sum(1 for a, b in zip(errs[:14], errs[1:15]) if b > a)
    _, Zm = impl.MomentSketch(2, 2, 8).update(K, V).query(Q)
    bound8 = 1.0 ** 9 / math.factorial(9) * math.exp(2.0)
    return errs[20], max(0.0, relmax(Zm, Ze) - bound8), rises


# P11: affine maps of the values -----------------------------------------------------

def pin_affine_values(impl, p=3, seed=11):
    K, V, Q = _small(seed, 60, 5, 3, 2)
    alpha, beta = -1.75, 0.625
    od, _ = impl.sketch_direct(K, V, Q, p)
    od2, _ = impl.sketch_direct(K, alpha * V + beta, Q, p)
    om, _ = impl.MomentSketch(3, 2, p).update(K, V).query(Q)
    om2, _ = impl.MomentSketch(3, 2, p).update(K, alpha * V + beta).query(Q)
    oe, _ = impl.exact_attention(K, V, Q)
    oe2, _ = impl.exact_attention(K, alpha * V + beta, Q)
    return max(absmax(od2, alpha * od + beta), absmax(om2, alpha * om + beta),
               absmax(oe2, alpha * oe + beta))


# P12: textbook softmax attention -----------------------------------------------------

def pin_textbook_attention(impl, seed=12):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((300, 6)) * 1.3
    V = rng.standard_normal((300, 4))
    Q = rng.standard_normal((11, 6)) * 1.3
    S = Q @ K.T
    o_ref = scipy.special.softmax(S, axis=1) @ V
    z_ref = np.exp(scipy.special.logsumexp(S, axis=1))
    oe, Ze = impl.exact_attention(K, V, Q, max_block_entries=900)  # several blocks
    return max(relmax(Ze, z_ref), absmax(oe, o_ref))


# P14: exact path by plain Python sums -----------------------------------------------

def pin_exact_python(impl, seed=14):
    rng = np.random.default_rng(seed)
    n, d, dv = 17, 3, 2
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, dv))
    Q = rng.standard_normal((3, d))
    Zr, Or = [], []
    for q in Q:
        e = [math.exp(math.fsum(q[a] * K[i, a] for a in range(d))) for i in range(n)]
        z = math.fsum(e)
        Zr.append(z)
        Or.append([math.fsum(e[i] * V[i, c] for i in range(n)) / z for c in range(dv)])
    oe, Ze = impl.exact_attention(K, V, Q)
    return max(relmax(Ze, Zr), absmax(oe, Or))


# hand-worked examples (tests/golden/hand_worked.json) -------------------------------

def pin_hand_worked(impl):
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        data = json.load(f)
    err = 0.0
    for ex in data["examples"]:
        K = np.array(ex["K"])
        V = np.array(ex["V"])
        Q = np.array(ex["Q"])
        p = ex["p"]
        zhat = ex["zhat"][0] / ex["zhat"][1]
        ohat = np.array([[a / b for a, b in ex["ohat"]]])
        od, Zd = impl.sketch_direct(K, V, Q, p)
        sk = impl.MomentSketch(ex["d"], ex["dv"], p).update(K, V)
        om, Zm = sk.query(Q)
        e = [math.exp(x) for x in ex["exact_exponents"]]
        z = math.fsum(e)
        o = np.array([[math.fsum(ei * V[i, c] for i, ei in enumerate(e)) / z
                       for c in range(V.shape[1])]])
        oe, Ze = impl.exact_attention(K, V, Q)
        err = max(err, relmax(Zd, [zhat]), relmax(Zm, [zhat]), absmax(od, ohat),
                  absmax(om, ohat), relmax(Ze, [z]), absmax(oe, o))
        if "canonical_state" in ex:
            err = max(err, absmax(sk.canonical_state(), np.array(ex["canonical_state"])))
    return err


# taylor_exp against the incomplete gamma identity -----------------------------------

def pin_taylor_gamma(impl):
    """For x >= 0: T_p(x) = e^x * Q(p+1, x) (regularised upper incomplete gamma);
    for x < 0 the Taylor coefficients from mpmath."""
    err = 0.0
    xs = np.linspace(0.0, 6.0, 61)
    for p in range(0, 12):
        ref = np.exp(xs) * scipy.special.gammaincc(p + 1, xs)
        err = max(err, relmax(impl.taylor_exp(xs, p), ref))
        coef = taylor_coeffs(p)
        xn = np.linspace(-3.0, -0.05, 30)
        refn = np.array([math.fsum(c * x ** j for j, c in enumerate(coef)) for x in xn])
        err = max(err, absmax(impl.taylor_exp(xn, p), refn) / max(1.0, np.abs(refn).max()))
    return err


# Multiset storage (oracle.sym) ------------------------------------------------------

def _sorted_tuples(d, j, lo=0):
    """Sorted index tuples of size j over lo..d-1 in lexicographic order, by
    recursion (independent of itertools)."""
    if j == 0:
        return [()]
    out = []
    for a in range(lo, d):
        out.extend((a,) + rest for rest in _sorted_tuples(d, j - 1, a))
    return out


def pin_sym_counts(impl, d, p):
    """S1: row counts are C(d + j - 1, j) per level and C(d + p, p) in all; the
    tuples are sorted, distinct and in lexicographic order; the multinomial
    theorem sum_alpha j!/alpha! = d^j holds for the alpha! the module computes."""
    err = 0.0
    total = 0
    for j in range(p + 1):
        t = impl.multisets(d, j)
        total += t.shape[0]
        err = max(err, abs(t.shape[0] - math.comb(d + j - 1, j)))
        ref = _sorted_tuples(d, j)
        err = max(err, 0.0 if [tuple(r) for r in t] == ref else 1.0)
        mult = math.factorial(j) / impl.alpha_factorial(t)
        err = max(err, abs(float(mult.sum()) - d ** j) / d ** j)
    err = max(err, abs(total - math.comb(d + p, p)))
    sk = impl.SymMomentSketch(d, 2, p)
    err = max(err, abs(sk.rows - math.comb(d + p, p)))
    return err


def pin_sym_bruteforce(impl, d, p, n=9, m=3, dv=2, seed=21):
    """S2: stored entries and query answers against pure-Python sums over every
    index tuple of every level (math.factorial, itertools.product)."""
    import itertools as it
    K, V, Q = _small(seed + 7 * d + p, n, m, d, dv)
    sk = impl.SymMomentSketch(d, dv, p).update(K, V, chunk=4)
    # stored entries, in the independently generated row order
    S = sk.canonical_state()
    ref_rows = []
    for j in range(p + 1):
        for alpha in _sorted_tuples(d, j):
            w = [math.prod(float(K[i][a]) for a in alpha) for i in range(n)]
            ref_rows.append([math.fsum(w)] +
                            [math.fsum(w[i] * float(V[i][c]) for i in range(n))
                             for c in range(dv)])
    ref = np.array(ref_rows)
    err = float(np.max(np.abs(S - ref) / np.maximum(np.abs(ref), 1.0)))
    # answers: sum over all index tuples, 1/j!
    Zb = np.zeros(m)
    Nb = np.zeros((m, dv))
    for qi in range(m):
        for i in range(n):
            w = 0.0
            for j in range(p + 1):
                w += math.fsum(math.prod(float(Q[qi][a]) * float(K[i][a]) for a in idx)
                               for idx in it.product(range(d), repeat=j)) / math.factorial(j)
            Zb[qi] += w
            Nb[qi] += w * V[i]
    o, Z = sk.query(Q)
    err = max(err, relmax(Z, Zb), absmax(o, Nb / Zb[:, None]))
    return err


def pin_sym_equals_direct(impl, K, V, Q, p, chunk=64):
    """S3: the multiset route answers as the plain definition sum_i T_p(<q, k_i>)."""
    d, dv = K.shape[1], V.shape[1]
    sk = impl.SymMomentSketch(d, dv, p).update(K, V, chunk=chunk)
    o, Z = sk.query(Q)
    od, Zd = impl.sketch_direct(K, V, Q, p)
    return max(relmax(Z, Zd), absmax(o, od))


def pin_sym_expand(impl, d, p, n=17, dv=3, seed=23):
    """S4: the stored entries, spread back to every index tuple, equal the
    Kronecker-layout moments built here with np.kron."""
    K, V, _ = _small(seed + d + p, n, 1, d, dv)
    sk = impl.SymMomentSketch(d, dv, p).update(K, V, chunk=5)
    full = sk.expand_full()
    blocks = []
    for j in range(p + 1):
        F = np.stack([kron_power(K[i], j) for i in range(n)])
        blocks.append(np.concatenate([F.sum(axis=0)[:, None], F.T @ V], axis=1))
    ref = np.concatenate(blocks, axis=0)
    return float(np.max(np.abs(full - ref) / np.maximum(np.abs(ref), 1.0)))


def pin_sym_merge(impl, p=3, d=3, dv=2, seed=24):
    """S5: merge(sketch(A), sketch(B)) == sketch(A u B)."""
    K, V, Q = _small(seed, 40, 5, d, dv)
    a = impl.SymMomentSketch(d, dv, p).update(K[:15], V[:15])
    b = impl.SymMomentSketch(d, dv, p).update(K[15:], V[15:])
    ab = impl.SymMomentSketch(d, dv, p).update(K, V)
    a.merge(b)
    S1, S2 = a.canonical_state(), ab.canonical_state()
    err = float(np.max(np.abs(S1 - S2) / np.maximum(np.abs(S2), 1.0)))
    return max(err, abs(a.count - ab.count))


# Recentred sketch (oracle.sketch_direct_centered) -------------------------------------

def _clustered(seed, n, m, d, dv, offset=1.2, spread=0.15):
    """Keys in a tight cluster away from the origin, queries of norm about 0.8."""
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal(d)
    mu *= offset / np.linalg.norm(mu)
    K = mu + spread * rng.standard_normal((n, d)) / np.sqrt(d)
    V = rng.standard_normal((n, dv))
    Q = rng.standard_normal((m, d))
    Q *= 0.8 / np.linalg.norm(Q, axis=1, keepdims=True)
    return K, V, Q, mu


def pin_centered_zero_centre(impl, p=3, seed=31):
    """C1: centre 0 is the plain sketch."""
    K, V, Q = _small(seed, 40, 6, 5, 3)
    o1, z1 = impl.sketch_direct_centered(K, V, Q, p, np.zeros(5))
    o2, z2 = impl.sketch_direct(K, V, Q, p)
    return max(relmax(z1, z2), absmax(o1, o2))


def pin_centered_identical_keys(impl, seed=32):
    """C2: every key equal to the centre: Zhat = n e^{<q,c>}, ohat = mean(v), for
    every p (T_p(0) = 1), against math.exp and math.fsum."""
    rng = np.random.default_rng(seed)
    c = rng.standard_normal(4)
    K = np.tile(c, (30, 1))
    V = rng.standard_normal((30, 2))
    Q = rng.standard_normal((5, 4))
    err = 0.0
    for p in (0, 1, 4):
        o, Z = impl.sketch_direct_centered(K, V, Q, p, c)
        for qi in range(5):
            zref = 30 * math.exp(math.fsum(float(Q[qi, a]) * float(c[a]) for a in range(4)))
            err = max(err, abs(Z[qi] - zref) / zref)
            vbar = [math.fsum(V[:, j]) / 30 for j in range(2)]
            err = max(err, float(np.max(np.abs(o[qi] - vbar))))
    return err


def pin_centered_kron(impl, d=3, p=3, seed=33):
    """C3: brute force with np.kron powers of k - c and math.exp(<q, c>)."""
    K, V, Q = _small(seed, 15, 3, d, 2)
    c = np.array([0.3, -0.2, 0.5][:d])
    coef = taylor_coeffs(p)
    Zb = np.zeros(3)
    Nb = np.zeros((3, 2))
    for qi in range(3):
        f = math.exp(float(Q[qi] @ c))
        for i in range(15):
            w = f * sum(coef[j] * float(kron_power(Q[qi], j) @ kron_power(K[i] - c, j))
                        for j in range(p + 1))
            Zb[qi] += w
            Nb[qi] += w * V[i]
    o, Z = impl.sketch_direct_centered(K, V, Q, p, c)
    return max(relmax(Z, Zb), absmax(o, Nb / Zb[:, None]))


def pin_centered_bound(impl, seed=34):
    """C4: on a cluster away from the origin the recentred error obeys the
    Lagrange bound with the shifted radius rho_c = max|q| max|k - c|, and falls to
    rounding as p grows; returns the largest (error / bound) and the p = 14 error."""
    K, V, Q, mu = _clustered(seed, 200, 8, 6, 3)
    o_e, Z_e = impl.exact_attention(K, V, Q)
    worst = 0.0
    for p in (1, 2, 3, 5):
        o, Z = impl.sketch_direct_centered(K, V, Q, p, mu)
        rho = float(np.max(np.linalg.norm(Q, axis=1)) * np.max(np.linalg.norm(K - mu, axis=1)))
        bound = rho ** (p + 1) / math.factorial(p + 1) * math.exp(2 * rho)
        worst = max(worst, float(np.max(np.abs(Z - Z_e) / Z_e)) / bound)
    o, Z = impl.sketch_direct_centered(K, V, Q, 14, mu)
    return worst, max(relmax(Z, Z_e), absmax(o, o_e))


def pin_centered_moments(impl, p=3, seed=35):
    """C5: the moment route on the shifted keys, answers times e^{<q,c>}, equals
    the plain definition."""
    K, V, Q, mu = _clustered(seed, 120, 5, 4, 2)
    sk = impl.MomentSketch(4, 2, p).update(K - mu, V, chunk=17)
    o, Z = sk.query(Q)
    od, Zd = impl.sketch_direct_centered(K, V, Q, p, mu)
    return max(relmax(Z * np.exp(Q @ mu), Zd), absmax(o, od))


# Bounds (oracle/bounds.py) -------------------------------------------------------------
#
# Each pin returns a violation measure: 0.0 when the bound function behaves, a
# positive number (the relative miss) otherwise.

# Closed-form value of the relative truncation bound rho^(p+1)/(p+1)! e^(2 rho) at
# rho = r^2 for the five workloads (p, r^2), evaluated by hand to five
# significant digits: e^2/24, e^2/120, 2.25^4/24 e^4.5, 0.5625^3/6 e^1.125,
# 4^7/5040 e^8.
KDE_BOUND_TABLE = [(3, 1.0, 0.30788), (4, 1.0, 0.061575), (3, 2.25, 96.127),
                   (2, 0.5625, 0.091369), (6, 4.0, 9690.5)]


def pin_bound_table(impl):
    """kde_relative_bound against the tabulated closed-form values (5 digits)."""
    worst = 0.0
    for p, rho, want in KDE_BOUND_TABLE:
        got = impl.kde_relative_bound(p, rho)
        worst = max(worst, abs(got - want) / want)
    return max(0.0, worst - 1e-4)        # five significant digits


def pin_term_bound_tight(impl):
    """taylor_term_bound is the Lagrange remainder bound: at x = +rho the true
    remainder e^x - T_p(x) = rho^(p+1)/(p+1)! e^xi with 0 < xi < rho, so
    remainder / bound lies in [e^-rho, 1].  Checked with mpmath at 50 digits."""
    worst = 0.0
    mpmath.mp.dps = 50
    for p in range(0, 7):
        for rho in (0.05, 0.3, 1.0):
            x = mpmath.mpf(rho)
            rem = mpmath.exp(x) - mpmath.fsum(x ** j / mpmath.factorial(j) for j in range(p + 1))
            ratio = float(rem) / impl.taylor_term_bound(p, rho)
            lo = math.exp(-rho)
            worst = max(worst, lo - ratio, ratio - 1.0)
    mpmath.mp.dps = 15
    return max(0.0, worst)


def pin_measured_radius(impl):
    """Hand example: the largest key norm and the largest query norm come from
    different rows (key norms 3 and 1, query norms 0.5 and 2): rho = 3 * 2 = 6.
    Also the empty stream (0) and a 3-4-5 key with a unit query (5)."""
    K = np.array([[3.0, 0.0], [0.0, 1.0]])
    Q = np.array([[0.0, 0.5], [-2.0, 0.0]])
    K2 = np.array([[3.0, 4.0]])
    Q2 = np.array([[0.0, -1.0]])
    errs = [abs(impl.measured_radius(K, Q) - 6.0) / 6.0,
            abs(impl.measured_radius(K2, Q2) - 5.0) / 5.0,
            abs(impl.measured_radius(np.zeros((0, 2)), Q) - 0.0)]
    return max(errs)


def _two_group_case(rho, a, vscale, n=1000):
    """d = 1, q = 1, p = 0: a fraction a of the keys at -rho with value +vscale,
    the rest at +rho with value -vscale.  Returns (observed |ohat - o|, V)."""
    na = int(round(a * n))
    nb = n - na
    ea, eb = math.exp(-rho), math.exp(rho)
    # exact o (softmax weights) and the p = 0 sketch's ohat (all weights 1)
    o = (na * ea * vscale - nb * eb * vscale) / (na * ea + nb * eb)
    ohat = (na * vscale - nb * vscale) / n
    V = np.array([[vscale]] * na + [[-vscale]] * nb)
    return abs(ohat - o), V


def pin_attention_bound_near_tight(impl):
    """attention_abs_bound on a near-tight d = 1, p = 0 construction: keys at
    +-rho with values at the two ends of the range (derived by hand: with rho
    small the best split gives |ohat - o| ~ rho while the bound is ~ 2 rho, so the
    observed error must sit within [0.45, 1] of the bound).  Values scaled by 10
    (the bound scales with the range).  The observed errors here are computed by
    hand from the two groups' softmax weights, not by the oracle's sketch."""
    worst = 0.0
    for rho in (1e-3, 1e-2):
        for vscale in (1.0, 10.0):
            best = 0.0
            for a in np.linspace(0.3, 0.7, 41):
                obs, V = _two_group_case(rho, a, vscale)
                bound = float(impl.attention_abs_bound(0, rho, V)[0])
                best = max(best, obs / bound)
            worst = max(worst, best - 1.0, 0.45 - best)
    return max(0.0, worst)


# Tail coreset (oracle/coreset.py) -------------------------------------------------------
#
# ``impl`` here has the attributes tail_exp, halve, uniforms, splitmix64,
# MergeReduceCoreset, tail_direct and answer_with_tail (the oracle.coreset module).

def pin_tail_exp_mpmath(impl):
    """R_p(x) against 120-digit mpmath on a grid (relative error, with an absolute
    floor of 1e-300 for R_p(0) = 0); 120 digits survive the cancellation of
    e^x - T_p(x) at x = 1e-4, p = 8 (about 42 digits)."""
    mpmath.mp.dps = 120
    worst = 0.0
    xs = np.concatenate([np.linspace(-12.0, 12.0, 97),
                         [-1e-3, 1e-4, 0.0, 15.0, -14.0, 30.0, -30.0]])
    for p in range(0, 9):
        got = impl.tail_exp(xs, p)
        for x, g in zip(xs, got):
            xm = mpmath.mpf(float(x))
            want = mpmath.exp(xm) - mpmath.fsum(xm ** j / mpmath.factorial(j)
                                                 for j in range(p + 1))
            w = float(want)
            worst = max(worst, abs(g - w) / max(abs(w), 1e-300))
    mpmath.mp.dps = 15
    return worst


def _tail_features(k, p, J):
    """phi_t(k) = (k^(x)j / sqrt(j!))_{p < j <= J}, built with np.kron."""
    return np.concatenate([kron_power(k, j) / math.sqrt(math.factorial(j))
                           for j in range(p + 1, J + 1)])


def _unit_vec(k, v, p, J):
    """u(x) = phi_t(k) (x) [1; v] as an explicit vector."""
    return np.kron(_tail_features(k, p, J), np.concatenate([[1.0], v]))


def pin_coreset_explicit_walk(impl, p=1, n=16, d=2, dv=1, seed=41, J=16):
    """The walk with explicit feature vectors (no kernel trick): alpha_t = <psi,
    f_t> and the kept points must match impl.halve; the discrepancy identity
    sum(all u) - 2 sum(kept u) = psi must hold; and the tail sums of every query
    must obey tail(all) - 2 tail(kept) = <psi, phi_t(q) (x) e>.  Keys of norm
    <= 0.6, so the explicit series cut at J = 16 is exact to ~1e-17."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, d))
    K *= 0.6 * rng.uniform(0.2, 1.0, (n, 1)) / np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((n, dv))
    U = rng.uniform(0.0, 1.0, n // 2)
    c0 = 0.7
    r = impl.halve(K, V, p, c0, U)
    u = np.array([_unit_vec(K[i], V[i], p, J) for i in range(n)])
    f = u[0::2] - u[1::2]
    c = c0 * max(float(fi @ fi) for fi in f)
    psi = np.zeros(u.shape[1])
    alpha, kept = [], []
    for t in range(n // 2):
        a = float(psi @ f[t])
        alpha.append(a)
        pt = min(1.0, max(0.0, 0.5 * (1.0 - a / c)))
        e = 1.0 if U[t] < pt else -1.0
        psi += e * f[t]
        kept.append(2 * t + 1 if e > 0 else 2 * t)
    scale = max(1.0, float(np.abs(alpha).max()))
    err = [float(np.abs(np.asarray(alpha) - r["alpha"]).max()) / scale,
           abs(c - r["c"]) / c,
           float(np.any(np.asarray(kept) != r["kept"]))]
    disc = u.sum(axis=0) - 2.0 * u[kept].sum(axis=0)
    err.append(float(np.abs(disc - psi).max()) / max(1.0, float(np.abs(psi).max())))
    # tail sums of a few queries through the kept set against <psi, phi(q) (x) e>
    Q = rng.standard_normal((4, d)) * 0.5
    n_all, z_all = impl.tail_direct(K, V, Q, p)
    n_kept, z_kept = impl.tail_direct(K[kept], V[kept], Q, p)
    for qi in range(Q.shape[0]):
        phq = _tail_features(Q[qi], p, J)
        for comp in range(1 + dv):
            e_c = np.zeros(1 + dv)
            e_c[comp] = 1.0
            lhs = (z_all[qi] - 2 * z_kept[qi]) if comp == 0 else \
                (n_all[qi, comp - 1] - 2 * n_kept[qi, comp - 1])
            rhs = float(psi @ np.kron(phq, e_c))
            err.append(abs(lhs - rhs) / max(1e-3, abs(rhs)))
    return max(err)


def pin_splitmix64_known_answers(impl):
    """The first outputs of SplitMix64 from state 0, as printed by its published
    reference implementation (Vigna's splitmix64.c, after Steele, Lea and Flood)."""
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    got = [int(x) for x in impl.splitmix64(0, np.arange(4))]
    return float(sum(g != w for g, w in zip(got, want)))


def pin_coreset_no_reduce_is_exact(impl, p=3, seed=42):
    """A block larger than the stream: no reduce happens, the coreset is the stream
    itself (weight 1), and head (plain Taylor sums) + tail = the exact answer,
    checked against scipy's softmax and logsumexp."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((300, 4)) * 0.4
    V = rng.standard_normal((300, 3))
    Q = rng.standard_normal((7, 4)) * 0.4
    cs = impl.MergeReduceCoreset(4, 3, p, 512, 1.0, 5).update(K[:100], V[:100]).update(
        K[100:], V[100:])
    tN, tZ = cs.tail_query(Q)
    S = Q @ K.T
    Th = sum(S ** j / math.factorial(j) for j in range(p + 1))
    o, Z = impl.answer_with_tail((Th @ V) / Th.sum(1)[:, None], Th.sum(1), tN, tZ)
    Zref = np.exp(scipy.special.logsumexp(S, axis=1))
    oref = scipy.special.softmax(S, axis=1) @ V
    return max(relmax(Z, Zref), absmax(o, oref))


def pin_coreset_fair_coin(impl, seed=43):
    """c0 huge: every probability is 1/2, so eps_t = +1 exactly when U_t < 1/2."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((40, 3)) * 0.5
    V = rng.standard_normal((40, 2))
    U = rng.uniform(0, 1, 20)
    r = impl.halve(K, V, 2, 1e300, U)
    want = np.where(U < 0.5, 1.0, -1.0)
    return float(np.any(r["eps"] != want))


def pin_coreset_identical_pairs(impl, seed=44):
    """Both points of every pair equal: f_t = 0, so the halved set answers every
    query exactly (twice the kept tail sums = the tail sums of all points)."""
    rng = np.random.default_rng(seed)
    K = np.repeat(rng.standard_normal((25, 3)) * 0.6, 2, axis=0)
    V = np.repeat(rng.standard_normal((25, 2)), 2, axis=0)
    Q = rng.standard_normal((5, 3)) * 0.6
    r = impl.halve(K, V, 1, 0.5, rng.uniform(0, 1, 25))
    n_all, z_all = impl.tail_direct(K, V, Q, 1)
    n_k, z_k = impl.tail_direct(K[r["kept"]], V[r["kept"]], Q, 1)
    return max(relmax(2 * z_k, z_all), absmax(2 * n_k, n_all) / np.abs(n_all).max())


def pin_coreset_levels(impl, B=16, seed=45):
    """Merge-and-Reduce as a binary counter: after n points, level l holds a block
    exactly when bit l of floor(n / B) is set, the buffer holds n mod B points, the
    weights add up to n, and every kept point is one of the input rows."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((1000, 2)) * 0.5
    V = rng.standard_normal((1000, 2))
    cs = impl.MergeReduceCoreset(2, 2, 2, B, 1.0, 9)
    bad = 0.0
    rows = {tuple(np.r_[K[i], V[i]]) for i in range(1000)}
    pos = 0
    for step in (1, 7, 16, 33, 100, 250, 593):
        cs.update(K[pos:pos + step], V[pos:pos + step])
        pos += step
        blocks = pos // B
        for l, blk in enumerate(cs.levels):
            bad += float((blk is not None) != bool((blocks >> l) & 1))
        bad += float(blocks >> len(cs.levels) != 0)
        Kp, Vp, w = cs.points()
        bad += float(Kp.shape[0] != pos % B + B * bin(blocks).count("1"))
        bad += abs(float(w.sum()) - pos)
        bad += float(sum(tuple(np.r_[Kp[i], Vp[i]]) not in rows for i in range(Kp.shape[0])))
    return bad


def pin_coreset_beats_random(impl, trials=12, B=64, seed=46):
    """The walk's halving errs less than a fair-coin halving of the same pairs:
    over random queries, the RMS error of the tail sums (2 x kept against all; the
    normaliser and the numerator) must stay below 0.7 of the fair coin's, pooled
    over the trials (measured: 0.40 and 0.56 at c0 = 0.25; a reversed drift does
    worse than the coin)."""
    rng = np.random.default_rng(seed)
    walk, coin, walkn, coinn = [], [], [], []
    for _ in range(trials):
        K = rng.standard_normal((2 * B, 4))
        K *= 1.0 / np.linalg.norm(K, axis=1, keepdims=True)
        V = rng.uniform(-1, 1, (2 * B, 2))
        Q = rng.standard_normal((32, 4))
        Q *= 1.0 / np.linalg.norm(Q, axis=1, keepdims=True)
        U = rng.uniform(0, 1, B)
        n_all, z_all = impl.tail_direct(K, V, Q, 1)
        r = impl.halve(K, V, 1, 0.25, U)
        nw, zw = impl.tail_direct(K[r["kept"]], V[r["kept"]], Q, 1)
        coin_kept = np.arange(0, 2 * B, 2) + (U < 0.5)
        nc, zc = impl.tail_direct(K[coin_kept], V[coin_kept], Q, 1)
        walk.append(2 * zw - z_all)
        coin.append(2 * zc - z_all)
        walkn.append(2 * nw - n_all)
        coinn.append(2 * nc - n_all)
    rms = lambda a: float(np.sqrt(np.mean(np.square(a))))
    ratio = max(rms(walk) / rms(coin), rms(walkn) / rms(coinn))
    return max(0.0, ratio - 0.7)


def pin_coreset_merge(impl, B=16, seed=47):
    """Merge of two sub-stream coresets.  (1) Into an empty coreset: the same
    points, no reduce.  (2) Blocks on different levels and empty buffers (3B and 4B
    points): the union, no reduce, so the tail sums add exactly.  (3) Any counts:
    the result is a binary-counter state of n1 + n2 points (level l occupied
    exactly when bit l of floor((n1 + n2) / B) is set, (n1 + n2) mod B buffered,
    weights adding up to n1 + n2)."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((600, 3)) * 0.5
    V = rng.standard_normal((600, 2))
    Q = rng.standard_normal((5, 3)) * 0.5
    mk = lambda: impl.MergeReduceCoreset(3, 2, 2, B, 0.25, 3)
    bad = 0.0
    src = mk().update(K[:100], V[:100])
    dst = mk().merge(src)
    a, b = dst.points(), src.points()
    bad += float(dst.serial != 0) + sum(float(x.shape != y.shape or np.any(x != y))
                                        for x, y in zip(a, b))
    d1 = mk().update(K[:3 * B], V[:3 * B])
    d2 = mk().update(K[3 * B:7 * B], V[3 * B:7 * B])
    n1, z1 = d1.tail_query(Q)
    n2, z2 = d2.tail_query(Q)
    serial = d1.serial
    d1.merge(d2)
    n12, z12 = d1.tail_query(Q)
    bad += float(d1.serial != serial)
    bad += relmax(z12, z1 + z2) + absmax(n12, n1 + n2)
    for c1, c2 in ((5 * B + 3, 3 * B + 7), (B - 1, B - 2), (9 * B + 11, 7 * B + 9)):
        x = mk().update(K[:c1], V[:c1])
        y = mk().update(K[c1:c1 + c2], V[c1:c1 + c2])
        x.merge(y)
        tot = c1 + c2
        blocks = tot // B
        for l, blk in enumerate(x.levels):
            bad += float((blk is not None) != bool((blocks >> l) & 1))
        Kp, _, w = x.points()
        bad += float(x.fillK.shape[0] != tot % B) + abs(float(w.sum()) - tot)
        bad += float(x.count != tot)
    return bad
