"""The CPU oracle against its pins (see tests/oracle_pins.py for what each pins)."""
import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS, brute_force, gelu_ref, rand_layer


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(lib, pin):
    pin(lib)


def test_gelu_reference_is_tanh_form():
    # The library GELU used as the pins' reference is the tanh approximation:
    # close to the exact erf form (max gap about 5e-4 on [-6, 6]) but not equal.
    import math
    a = np.linspace(-6, 6, 2001)
    exact = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in a])
    gap = np.abs(gelu_ref(a) - exact)
    assert gap.max() < 1e-3 and gap.max() > 1e-5


def test_brute_force_rejects_inconsistent_paths():
    # The brute-force helper itself: with a single tree of depth 1 the path is
    # the sign of the root logit.
    L = rand_layer(np.random.default_rng(0), 8, 3, 1, 1, 2)
    path, _, _ = brute_force(L)
    a = L["x"] @ L["W_node"][0, 0] + L["b_node"][0, 0]
    np.testing.assert_array_equal(path[:, 0], (~(a < 0)).astype(np.int32))


def test_threads_do_not_change_results(lib):
    L = rand_layer(np.random.default_rng(11), 37, 12, 3, 4, 5)
    r1 = oracle.forward(**L, want_H=True, nthreads=1, lib=lib)
    r8 = oracle.forward(**L, want_H=True, nthreads=8, lib=lib)
    for k in ("path", "H", "y"):
        np.testing.assert_array_equal(r1[k], r8[k])


def test_bad_shape_rejected(lib):
    L = rand_layer(np.random.default_rng(0), 2, 3, 1, 1, 2)
    with pytest.raises(ValueError):
        oracle.forward(L["x"], L["W_node"], L["b_node"], L["V_node"], L["W_out"][:-1], lib=lib)


def test_bad_variant_rejected(lib):
    L = rand_layer(np.random.default_rng(0), 2, 3, 1, 1, 2)
    with pytest.raises(ValueError):
        oracle.forward(**L, variant=2, lib=lib)


def test_pruned_tree_without_alive_leaf_rejected(lib):
    L = rand_layer(np.random.default_rng(0), 3, 4, 2, 2, 3)
    alive = np.ones((2, 4), np.uint8)
    alive[1] = 0
    with pytest.raises(ValueError):
        oracle.forward(**L, leaf_alive=alive, lib=lib)
    with pytest.raises(ValueError):
        oracle.forward(**L, leaf_alive=np.ones((2, 3), np.uint8), lib=lib)
