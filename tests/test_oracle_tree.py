"""Pins for the oracle's ancestor masks and accept walk (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import pins


def test_mask_hand_examples():
    pins.check_mask_golden(oracle.build_masks)


def test_mask_closed_forms_chain_and_star():
    pins.check_mask_closed_forms(oracle.build_masks)


def test_mask_matches_transitive_closure_on_every_tree_up_to_7_nodes():
    pins.check_mask_brute_force(oracle.build_masks, max_n=7)


def test_mask_invariants_random_trees():
    rng = np.random.default_rng(11)
    for _ in range(50):
        n = int(rng.integers(1, 65))
        p = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        m, dep = oracle.build_masks(np.array([p]))
        for i in range(n):
            mi = int(m[0, i])
            assert mi & 1 and (mi >> i) & 1
            assert bin(mi).count("1") == dep[0, i] + 1
            if i:
                assert mi == int(m[0, p[i]]) | (1 << i)
            assert mi < (1 << (i + 1))          # only lower-numbered ancestors


@pytest.mark.parametrize("bad", [[0, 0], [-1, 1], [-1, 0, 2], [-1, -1], [-1, 0, 5]])
def test_mask_rejects_invalid_parents(bad):
    with pytest.raises(ValueError):
        oracle.build_masks(np.array([bad]))


def test_mask_rejects_oversize_tree():
    with pytest.raises(ValueError):
        oracle.build_masks(np.arange(-1, 64)[None])


def test_walk_hand_examples():
    pins.check_walk_golden(oracle.accept_walk)


def test_walk_brute_force_every_tree_up_to_6_nodes():
    pins.check_walk_brute_force(oracle.accept_walk, max_n=6, draws=4)


def test_walk_brute_force_7_nodes():
    pins.check_walk_brute_force(oracle.accept_walk, max_n=7, draws=1, seed=9)


def test_walk_chain_closed_forms():
    pins.check_walk_chain_closed_forms(oracle.accept_walk)


def test_walk_depth_bound_and_greedy_equivalence():
    pins.check_walk_depth_bound_and_greedy(oracle.accept_walk, oracle.build_masks)


def test_walk_rejects_out_of_range_tokens():
    with pytest.raises(ValueError):
        oracle.accept_walk(np.array([[-1, 0]]), np.array([[0, 5]]), np.array([[1, 2]]), V=5)
