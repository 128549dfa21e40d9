"""Pins of the tail coreset oracle (oracle/coreset.py) against mpmath, explicit
feature vectors, a published generator's known answers, the exact answer, and the
walk's defining properties."""

import numpy as np

from oracle import coreset as ocs
from tests import oracle_pins as pins


def test_tail_exp_against_mpmath():
    assert pins.pin_tail_exp_mpmath(ocs) < 1e-12


def test_walk_against_explicit_features():
    for p in (0, 1, 2):
        assert pins.pin_coreset_explicit_walk(ocs, p=p, seed=41 + p) < 1e-10


def test_splitmix64_known_answers():
    assert pins.pin_splitmix64_known_answers(ocs) == 0.0


def test_uniforms_in_unit_interval_and_distinct_per_head():
    u0 = ocs.uniforms(7, 3, 0, 2, 1000)
    u1 = ocs.uniforms(7, 3, 1, 2, 1000)
    assert np.all((u0 >= 0) & (u0 < 1)) and abs(u0.mean() - 0.5) < 0.05
    assert not np.any(u0 == u1)


def test_no_reduce_is_exact():
    assert pins.pin_coreset_no_reduce_is_exact(ocs) < 1e-12


def test_fair_coin_limit():
    assert pins.pin_coreset_fair_coin(ocs) == 0.0


def test_identical_pairs_halve_exactly():
    assert pins.pin_coreset_identical_pairs(ocs) < 1e-14


def test_binary_counter_levels():
    assert pins.pin_coreset_levels(ocs) == 0.0


def test_walk_beats_a_fair_coin():
    assert pins.pin_coreset_beats_random(ocs) == 0.0


def test_merge_of_sub_streams():
    assert pins.pin_coreset_merge(ocs) < 1e-12
