"""Plant plausible mistakes in copies of the oracle and check a pin catches each.

Every mutant is a small subclass or wrapper built here, on the CPU; the oracle
package itself is never modified.  A mutant "survives" if every pin it is run
against stays at rounding level; the test fails in that case.
"""

import math
import types

import numpy as np
import pytest

import oracle
from oracle import sketch as osk
from tests import oracle_pins as pins


def _impl(**over):
    base = dict(exact_attention=oracle.exact_attention,
                sketch_direct=oracle.sketch_direct,
                MomentSketch=oracle.MomentSketch,
                taylor_exp=oracle.taylor_exp)
    base.update(over)
    return types.SimpleNamespace(**base)


class NoFactorial(oracle.MomentSketch):
    """Drops the 1/j! weights at query time."""

    def query(self, Q):
        Q = np.asarray(Q, dtype=np.float64)
        Z = np.zeros(Q.shape[0])
        Nt = np.zeros((Q.shape[0], self.dv))
        for j, F in enumerate(osk.feature_map(Q, self.p)):
            Z += F @ self.M[j]
            Nt += F @ self.N[j]
        return Nt / Z[:, None], Z


class DroppedTopLevel(oracle.MomentSketch):
    """Forgets the degree-p level when answering."""

    def query(self, Q):
        Q = np.asarray(Q, dtype=np.float64)
        Z = np.zeros(Q.shape[0])
        Nt = np.zeros((Q.shape[0], self.dv))
        for j, F in enumerate(osk.feature_map(Q, self.p)[:-1]):
            Z += (F @ self.M[j]) / math.factorial(j)
            Nt += (F @ self.N[j]) / math.factorial(j)
        return Nt / Z[:, None], Z


class SwappedColumns(oracle.MomentSketch):
    """Stores the value moment of the first value coordinate in the M column."""

    def canonical_state(self):
        S = super().canonical_state()
        return S[:, [1, 0] + list(range(2, S.shape[1]))]


class SubtractMerge(oracle.MomentSketch):
    def merge(self, other):
        for j in range(self.p + 1):
            self.M[j] -= other.M[j]
            self.N[j] -= other.N[j]
        self.count += other.count
        return self


class LastChunkOnly(oracle.MomentSketch):
    """Overwrites instead of accumulating across chunks."""

    def update(self, K, V, chunk=256):
        K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64)
        for c0 in range(0, K.shape[0], chunk):
            for j, F in enumerate(osk.feature_map(K[c0:c0 + chunk], self.p)):
                self.M[j] = F.sum(axis=0)
                self.N[j] = F.T @ V[c0:c0 + chunk]
        self.count += K.shape[0]
        return self


def taylor_off_by_one(x, p):
    """Sums only up to degree p - 1."""
    return oracle.taylor_exp(x, max(p - 1, 0)) if p > 0 else oracle.taylor_exp(x, 0) * 0 + 1


def direct_off_by_one(K, V, Q, p, max_block_entries=1 << 24):
    return oracle.sketch_direct(K, V, Q, max(p - 1, 0) if p else 0, max_block_entries)


def direct_no_constant(K, V, Q, p, max_block_entries=1 << 24):
    """Leaves out the j = 0 term."""
    o, Z = oracle.sketch_direct(K, V, Q, p, max_block_entries)
    n = np.asarray(K).shape[0]
    Nt = o * Z[:, None] - np.asarray(V, np.float64).sum(axis=0)[None, :]
    Z = Z - n
    return Nt / Z[:, None], Z


def exact_wrong_sign(K, V, Q, max_block_entries=1 << 24):
    return oracle.exact_attention(K, V, -np.asarray(Q), max_block_entries)


def exact_transposed_values(K, V, Q, max_block_entries=1 << 24):
    """Uses the reversed key order for the values (a transposed/misindexed operand)."""
    return oracle.exact_attention(K, np.asarray(V)[::-1], Q, max_block_entries)


def exact_missing_shift(K, V, Q, max_block_entries=1 << 24):
    """Forgets to scale Z back by e^mu."""
    o, Z = oracle.exact_attention(K, V, Q, max_block_entries)
    S = np.asarray(Q, np.float64) @ np.asarray(K, np.float64).T
    return o, Z / np.exp(S.max(axis=1))


def _all_pins(impl):
    errs = [pins.pin_bruteforce(impl, 3, 3), pins.pin_bruteforce(impl, 2, 4),
            pins.pin_identical_keys(impl, 3), pins.pin_zero_query(impl, 3),
            pins.pin_low_orders(impl), pins.pin_merge(impl),
            pins.pin_affine_values(impl), pins.pin_textbook_attention(impl),
            pins.pin_exact_python(impl), pins.pin_hand_worked(impl),
            pins.pin_taylor_gamma(impl)]
    e20, excess8, rises = pins.pin_convergence(impl)
    errs += [e20 * 1e-2, excess8, float(rises)]
    return max(errs)


MUTANTS = {
    "no_factorial": _impl(MomentSketch=NoFactorial),
    "dropped_top_level": _impl(MomentSketch=DroppedTopLevel),
    "swapped_state_columns": _impl(MomentSketch=SwappedColumns),
    "subtract_merge": _impl(MomentSketch=SubtractMerge),
    "last_chunk_only": _impl(MomentSketch=LastChunkOnly),
    "taylor_off_by_one": _impl(taylor_exp=taylor_off_by_one),
    "direct_off_by_one": _impl(sketch_direct=direct_off_by_one),
    "direct_no_constant": _impl(sketch_direct=direct_no_constant),
    "exact_wrong_sign": _impl(exact_attention=exact_wrong_sign),
    "exact_transposed_values": _impl(exact_attention=exact_transposed_values),
    "exact_missing_shift": _impl(exact_attention=exact_missing_shift),
}


def test_unmutated_passes_all_pins():
    assert _all_pins(_impl()) < 1e-12


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with np.errstate(all="ignore"):
        assert _all_pins(MUTANTS[name]) > 1e-6, f"mutant {name} survived every pin"


# Multiset storage mutants ------------------------------------------------------------

from oracle import sym as osym


def _sym_impl(**over):
    base = dict(SymMomentSketch=oracle.SymMomentSketch, multisets=oracle.multisets,
                alpha_factorial=oracle.alpha_factorial, sketch_direct=oracle.sketch_direct)
    base.update(over)
    return types.SimpleNamespace(**base)


class SymJFactorial(oracle.SymMomentSketch):
    """Weights every entry of level j by 1/j! instead of 1/alpha!."""

    def __init__(self, d, dv, p):
        super().__init__(d, dv, p)
        self.weights = [np.full(len(t), 1.0 / math.factorial(j))
                        for j, t in enumerate(self.tuples)]


class SymDroppedTop(oracle.SymMomentSketch):
    """Answers without the degree-p level."""

    def query(self, Q):
        Q = np.asarray(Q, dtype=np.float64)
        Z = np.zeros(Q.shape[0])
        Nt = np.zeros((Q.shape[0], self.dv))
        for j, F in enumerate(osym.sym_features(Q, self.p)[:-1]):
            Fw = F * self.weights[j][None, :]
            Z += Fw @ self.M[j]
            Nt += Fw @ self.N[j]
        return Nt / Z[:, None], Z


class SymReversedRows(oracle.SymMomentSketch):
    """Lists each level's rows in reverse lexicographic order."""

    def canonical_state(self):
        import numpy as _np
        return _np.concatenate(
            [_np.concatenate([self.M[j][::-1, None], self.N[j][::-1]], axis=1)
             for j in range(self.p + 1)], axis=0)


def _no_replacement(d, j):
    import itertools
    rows = list(itertools.combinations(range(d), j))
    return np.array(rows, dtype=np.int64).reshape(len(rows), j)


def _alpha_fact_counts_distinct(tuples):
    """Takes alpha! as (number of distinct indices)!."""
    return np.array([float(math.factorial(len(set(r)))) for r in tuples])


class SymLastChunkOnly(oracle.SymMomentSketch):
    def update(self, K, V, chunk=256):
        K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64)
        for c0 in range(0, K.shape[0], chunk):
            for j, F in enumerate(osym.sym_features(K[c0:c0 + chunk], self.p)):
                self.M[j] = F.sum(axis=0)
                self.N[j] = F.T @ V[c0:c0 + chunk]
        self.count += K.shape[0]
        return self


def _sym_pins(impl):
    errs = [pins.pin_sym_counts(impl, 3, 4), pins.pin_sym_counts(impl, 4, 3),
            pins.pin_sym_bruteforce(impl, 3, 3), pins.pin_sym_bruteforce(impl, 2, 4),
            pins.pin_sym_expand(impl, 3, 3), pins.pin_sym_merge(impl)]
    K, V, Q = pins._small(99, 60, 6, 4, 3)
    errs.append(pins.pin_sym_equals_direct(impl, K, V, Q, 3, chunk=16))
    return max(errs)


@pytest.mark.parametrize("impl", [
    _sym_impl(SymMomentSketch=SymJFactorial),
    _sym_impl(SymMomentSketch=SymDroppedTop),
    _sym_impl(SymMomentSketch=SymReversedRows),
    _sym_impl(multisets=_no_replacement),
    _sym_impl(alpha_factorial=_alpha_fact_counts_distinct),
    _sym_impl(SymMomentSketch=SymLastChunkOnly),
], ids=["j_factorial", "dropped_top", "reversed_rows", "no_replacement",
        "alpha_fact_distinct", "last_chunk_only"])
def test_sym_mutant_caught(impl):
    with np.errstate(all="ignore"):
        try:
            err = _sym_pins(impl)
        except (AssertionError, KeyError, ValueError, IndexError):
            return
    assert not err < 1e-9, "mutant survived every multiset pin"


def test_sym_pins_pass_on_oracle():
    assert _sym_pins(_sym_impl()) < 1e-11


# Recentred sketch mutants ------------------------------------------------------------

def _centred_no_factor(K, V, Q, p, c):
    return oracle.sketch_direct(np.asarray(K) - np.asarray(c)[None, :], V, Q, p)


def _centred_plus(K, V, Q, p, c):
    o, Z = oracle.sketch_direct(np.asarray(K) + np.asarray(c)[None, :], V, Q, p)
    return o, Z * np.exp(np.asarray(Q) @ np.asarray(c))


def _centred_neg_factor(K, V, Q, p, c):
    o, Z = oracle.sketch_direct(np.asarray(K) - np.asarray(c)[None, :], V, Q, p)
    return o, Z * np.exp(-(np.asarray(Q) @ np.asarray(c)))


def _centred_pins(impl):
    ratio, err14 = pins.pin_centered_bound(impl)
    return max(pins.pin_centered_zero_centre(impl), pins.pin_centered_identical_keys(impl),
               pins.pin_centered_kron(impl), pins.pin_centered_moments(impl),
               err14, 0.0 if ratio <= 1.0 else ratio)


@pytest.mark.parametrize("fn", [_centred_no_factor, _centred_plus, _centred_neg_factor],
                         ids=["no_factor", "plus_centre", "negative_factor"])
def test_centred_mutant_caught(fn):
    impl = types.SimpleNamespace(sketch_direct_centered=fn, sketch_direct=oracle.sketch_direct,
                                 exact_attention=oracle.exact_attention,
                                 MomentSketch=oracle.MomentSketch)
    with np.errstate(all="ignore"):
        err = _centred_pins(impl)
    assert not err < 1e-9, "mutant survived every recentring pin"


def test_centred_pins_pass_on_oracle():
    impl = types.SimpleNamespace(sketch_direct_centered=oracle.sketch_direct_centered,
                                 sketch_direct=oracle.sketch_direct,
                                 exact_attention=oracle.exact_attention,
                                 MomentSketch=oracle.MomentSketch)
    assert _centred_pins(impl) < 1e-11


# Bound mutants -------------------------------------------------------------------------

from oracle import bounds as obd


def _bounds_impl(**over):
    base = dict(taylor_term_bound=obd.taylor_term_bound,
                kde_relative_bound=obd.kde_relative_bound,
                attention_abs_bound=obd.attention_abs_bound,
                measured_radius=obd.measured_radius)
    base.update(over)
    return types.SimpleNamespace(**base)


def _kde_missing_exp(p, rho):
    """Drops the e^rho that the lower bound Z >= n e^-rho brings in."""
    return obd.taylor_term_bound(p, rho)


def _attention_no_range(p, rho, V):
    """Drops the per-coordinate range of the values."""
    V = np.asarray(V, dtype=np.float64)
    eps1 = obd.taylor_term_bound(p, rho)
    denom = math.exp(-rho) - eps1
    if denom <= 0:
        return np.full(V.shape[1], np.inf)
    return np.full(V.shape[1], eps1 / denom)


def _radius_key_squared(K, Q):
    """max |k|^2 instead of max |k| * max |q|."""
    K = np.asarray(K, dtype=np.float64)
    if K.shape[0] == 0 or np.asarray(Q).shape[0] == 0:
        return 0.0
    return float(np.linalg.norm(K, axis=1).max() ** 2)


def _radius_paired_rows(K, Q):
    """max over rows i of |k_i| |q_i| (pairs rows instead of taking each maximum)."""
    K = np.asarray(K, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    if K.shape[0] == 0 or Q.shape[0] == 0:
        return 0.0
    r = min(K.shape[0], Q.shape[0])
    return float((np.linalg.norm(K[:r], axis=1) * np.linalg.norm(Q[:r], axis=1)).max())


def _term_next_factorial(p, rho):
    """(p+2)! in place of (p+1)!."""
    return rho ** (p + 1) / math.factorial(p + 2) * math.exp(rho)


def _bound_pins(impl):
    return max(pins.pin_bound_table(impl), pins.pin_term_bound_tight(impl),
               pins.pin_measured_radius(impl), pins.pin_attention_bound_near_tight(impl))


@pytest.mark.parametrize("impl", [
    _bounds_impl(kde_relative_bound=_kde_missing_exp),
    _bounds_impl(attention_abs_bound=_attention_no_range),
    _bounds_impl(measured_radius=_radius_key_squared),
    _bounds_impl(measured_radius=_radius_paired_rows),
    _bounds_impl(taylor_term_bound=_term_next_factorial),
], ids=["kde_missing_exp_rho", "attention_no_range", "radius_key_squared",
        "radius_paired_rows", "term_next_factorial"])
def test_bound_mutant_caught(impl):
    assert _bound_pins(impl) > 1e-6


def test_bound_pins_pass_on_oracle():
    assert _bound_pins(_bounds_impl()) < 1e-15


# Tail coreset mutants ------------------------------------------------------------------

from oracle import coreset as ocs


def _cs_impl(**over):
    base = dict(tail_exp=ocs.tail_exp, halve=ocs.halve, uniforms=ocs.uniforms,
                splitmix64=ocs.splitmix64, MergeReduceCoreset=ocs.MergeReduceCoreset,
                tail_direct=ocs.tail_direct, answer_with_tail=ocs.answer_with_tail)
    base.update(over)
    return types.SimpleNamespace(**base)


def _halve_variant(keep_flip=False, reverse=False, mean_c=False, no_values=False):
    def halve(K, V, p, c0, U):
        K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64)
        B = K.shape[0] // 2
        G = ocs.tail_exp(K @ K.T, p) * (1.0 if no_values else (1.0 + V @ V.T))
        a = np.arange(0, 2 * B, 2)
        b = a + 1
        D = G[np.ix_(a, a)] - G[np.ix_(a, b)] - G[np.ix_(b, a)] + G[np.ix_(b, b)]
        c = c0 * float(np.mean(np.diag(D)) if mean_c else np.max(np.diag(D)))
        run = np.zeros(B)
        alpha, eps = np.zeros(B), np.zeros(B)
        for t in range(B):
            alpha[t] = run[t]
            x = -run[t] if reverse else run[t]
            pt = min(1.0, max(0.0, 0.5 * (1.0 - x / c)))
            e = 1.0 if U[t] < pt else -1.0
            eps[t] = e
            run += e * D[t]
        kept = np.where((eps < 0) if keep_flip else (eps > 0), b, a)
        return {"kept": kept, "eps": eps, "alpha": alpha, "c": c, "D": D}
    return halve


def _tail_next_degree(x, p):
    return ocs.tail_exp(x, p + 1)


class _NoDoubling(ocs.MergeReduceCoreset):
    """Keeps weight 1 on every level."""

    def points(self):
        K, V, w = super().points()
        return K, V, np.ones_like(w)


class _MergeAtLevelZero(ocs.MergeReduceCoreset):
    """Carries every block of the other coreset in at level 0."""

    def merge(self, other):
        self._append(other.fillK, other.fillV)
        for blk in other.levels:
            if blk is not None:
                self._carry(blk[0], blk[1], 0)
        self.count += other.count
        return self


def _cs_pins(impl):
    with np.errstate(all="ignore"):
        return max(pins.pin_tail_exp_mpmath(impl),
                   pins.pin_coreset_explicit_walk(impl, p=1),
                   pins.pin_coreset_explicit_walk(impl, p=0, seed=40),
                   pins.pin_splitmix64_known_answers(impl),
                   pins.pin_coreset_no_reduce_is_exact(impl),
                   pins.pin_coreset_fair_coin(impl),
                   pins.pin_coreset_identical_pairs(impl),
                   pins.pin_coreset_levels(impl),
                   pins.pin_coreset_beats_random(impl),
                   pins.pin_coreset_merge(impl))


@pytest.mark.parametrize("impl", [
    _cs_impl(halve=_halve_variant(keep_flip=True)),
    _cs_impl(halve=_halve_variant(reverse=True)),
    _cs_impl(halve=_halve_variant(mean_c=True)),
    _cs_impl(halve=_halve_variant(no_values=True)),
    _cs_impl(tail_exp=_tail_next_degree),
    _cs_impl(MergeReduceCoreset=_NoDoubling),
    _cs_impl(MergeReduceCoreset=_MergeAtLevelZero),
], ids=["kept_flipped", "drift_reversed", "threshold_from_mean", "values_dropped",
        "tail_next_degree", "weights_not_doubled", "merge_at_level_zero"])
def test_coreset_mutant_caught(impl):
    assert _cs_pins(impl) > 1e-6


def test_coreset_pins_pass_on_oracle():
    assert _cs_pins(_cs_impl()) < 1e-10
