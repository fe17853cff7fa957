"""Pins of the oracle's greedy sampling against hand-worked rows and an
independent formulation (numpy's first-maximum argmax after NaN masking)."""
import numpy as np

from oracle.sampling import greedy_token, greedy_tokens


def test_hand_worked_rows():
    nan, inf = float("nan"), float("inf")
    cases = [
        ([0.1, 0.5, 0.2], 1),
        ([3.0, 1.0, 3.0, 3.0], 0),          # ties: lowest index
        ([-1.0, -1.0], 0),
        ([nan, 2.0, nan, 2.0], 1),           # NaN never wins
        ([nan, nan, nan], 0),                # nothing valid: token 0
        ([-inf, -inf, -5.0], 2),
        ([-inf, -inf], 0),                   # -inf is a valid (lowest) value
        ([1.0, inf, inf], 1),
        ([nan, -inf], 1),
        ([-0.0, 0.0], 0),                    # -0 == +0: a tie
        ([7.5], 0),
    ]
    for row, want in cases:
        assert greedy_token(row) == want, (row, want)


def test_matches_masked_first_argmax():
    rng = np.random.default_rng(11)
    for n, v in ((5, 17), (3, 1000), (2, 4099)):
        # few distinct values, so ties are common; some NaN and infinities
        x = rng.integers(-3, 4, size=(n, v)).astype(np.float32)
        x[rng.random((n, v)) < 0.05] = np.nan
        x[rng.random((n, v)) < 0.01] = np.inf
        x[rng.random((n, v)) < 0.01] = -np.inf
        want = np.argmax(np.where(np.isnan(x), -np.inf, x), axis=1)
        got = greedy_tokens(x)
        np.testing.assert_array_equal(got, want)
        # the chosen entry is the maximum and no lower index attains it
        for r in range(n):
            valid = x[r][~np.isnan(x[r])]
            assert x[r, got[r]] == valid.max()
            assert not np.any(x[r, :got[r]] == valid.max())
