"""The float64 oracle against closed forms, a library softmax, invariants,
block-size independence and central finite differences (CPU only)."""

import numpy as np
import pytest

import oracle
import workloads
from oracle import dense, tiled, tilemap
from tests import oracle_pins as P


def test_closed_forms():
    P.check_closed_forms(dense)


def test_golden_hand_derived():
    P.check_golden(dense, tiled)


def test_library_softmax():
    P.check_library_softmax(dense)


def test_invariants():
    P.check_invariants(dense)


def test_block_size_independence():
    P.check_block_independence(dense, tiled)


def test_wide_score_range():
    P.check_wide_scores(dense, tiled)


def test_dense_vjp_finite_differences():
    P.check_dense_vjp_fd(dense)


def test_tiled_reverse_finite_differences():
    P.check_tiled_reverse_fd(tiled)


def test_reverse_routes_agree():
    P.check_reverse_routes_agree(dense, tiled)


def test_gradient_identities():
    P.check_grad_identities(dense, tiled)


def test_self_attention_shared_input():
    P.check_self_attention_fd(dense)


def test_sampled_gradients():
    P.check_sampled_grads(dense)


def test_tile_map():
    P.check_tilemap(tilemap)


def test_empty_row_is_rejected():
    A = np.ones((3, 3), bool)
    A[1] = False
    with pytest.raises(ValueError):
        dense.forward(np.ones((3, 2)), np.ones((3, 2)), np.ones((3, 2)), 1.0, A)
    with pytest.raises(ValueError):
        tiled.forward(np.ones((3, 2)), np.ones((3, 2)), np.ones((3, 2)), 1.0, A, 2)
