"""The GPU parity protocol's ReLU near-kink rule, on the CPU: a mask
disagreement is accepted only where the pre-activation is within the float32
summation bound of zero, and it names the weight-gradient row it touches."""
import numpy as np
import pytest

from gpu_helpers import relu_kink_flips


def _case():
    rng = np.random.default_rng(7)
    d, F, rows = 64, 8, 5
    w1 = rng.standard_normal((2, F, d))
    x = rng.standard_normal((2 * rows, d))
    # row 3 of expert 1 and column 5: make the pre-activation exactly zero in
    # float64, then nudge it by far less than the float32 summation bound
    r, c = rows + 3, 5
    x[r, -1] = 0.0
    x[r, -1] = -(x[r] @ w1[1, c]) / w1[1, c, -1]
    z = x @ np.concatenate([w1[0], w1[1]], axis=0).T
    h = np.zeros((2 * rows, F))
    h[:rows] = np.maximum(z[:rows, :F], 0)
    h[rows:] = np.maximum(z[rows:, F:], 0)
    return x, w1, h, r, c


def test_near_kink_flip_is_accepted_and_located():
    x, w1, h_ref, r, c = _case()
    h_gpu = h_ref.copy()
    h_ref[r, c] = 1e-12   # the float64 side keeps it, the float32 side does not
    h_gpu[r, c] = 0.0
    rows = {0: (0, 5), 1: (5, 10)}
    pairs, flipped = relu_kink_flips(h_gpu, h_ref, x, w1, rows, rows, [0, 1])
    assert pairs == {(1, c)} and flipped == [r]


def test_flip_away_from_a_kink_fails():
    x, w1, h_ref, _, _ = _case()
    h_gpu = h_ref.copy()
    i, j = np.argwhere(h_ref[:5] > 0.5)[0]  # a clearly positive pre-activation
    h_gpu[i, j] = 0.0
    rows = {0: (0, 5), 1: (5, 10)}
    with pytest.raises(AssertionError, match="away from a kink"):
        relu_kink_flips(h_gpu, h_ref, x, w1, rows, rows, [0, 1])


def test_no_flip_no_pairs():
    x, w1, h_ref, _, _ = _case()
    rows = {0: (0, 5), 1: (5, 10)}
    assert relu_kink_flips(h_ref.copy(), h_ref, x, w1, rows, rows, [0, 1]) == (set(), [])
