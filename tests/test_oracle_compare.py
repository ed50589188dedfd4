"""Pins of oracle.compare, the statistic behind every parity gate.

The gates are defined per output tensor (rel = max|g - o| / max|o|, the
oracle's magnitude in the denominator), per token (cosine over the feature
axis, minimum over tokens) and as a plain max-abs difference.  Every expected
value below is worked out by hand in the comment beside it, and the cases are
chosen so that the plausible mistakes fail: a cosine over the flattened
tensor instead of per token, a rel normalised by the GPU side, a max taken
over signed differences, a statistic over the wrong axis."""
import math

import numpy as np

import oracle


def test_hand_computed_values():
    # two tokens of three features
    ref = np.array([[3.0, 4.0, 0.0],
                    [0.0, 0.0, 2.0]])
    gpu = np.array([[4.0, 3.0, 0.0],
                    [0.0, 0.0, 1.5]])
    st = oracle.compare(gpu, ref)
    # |g - o| = [[1, 1, 0], [0, 0, 0.5]] -> maxabs 1
    assert st["maxabs"] == 1.0
    # max|o| = 4 -> rel = 1 / 4
    assert st["rel"] == 0.25
    # token 0: (12 + 12) / (5 * 5) = 0.96; token 1: 3 / (2 * 1.5) = 1
    assert math.isclose(st["min_cos"], 0.96, rel_tol=0, abs_tol=1e-15)
    assert st["finite"] is True


def test_cosine_is_per_token_not_flattened():
    # token 0 is orthogonal to its reference (cosine 0); token 1 dominates the
    # norm and matches, so a cosine over the flattened tensor would be
    # 10000 / sqrt(10001 * 10000) = 0.99995 and pass a 0.9999 gate
    ref = np.array([[1.0, 0.0], [0.0, 100.0]])
    gpu = np.array([[0.0, 1.0], [0.0, 100.0]])
    st = oracle.compare(gpu, ref)
    assert st["min_cos"] == 0.0
    flat = float((gpu * ref).sum() / np.sqrt((gpu * gpu).sum() * (ref * ref).sum()))
    assert flat > 0.9999  # the mistake this test exists to catch would pass


def test_rel_is_normalised_by_the_oracle():
    # max|o| = 2 and max|g| = 4: rel = 2 / 2 = 1, not 2 / 4
    ref = np.array([[1.0, 2.0]])
    gpu = np.array([[1.0, 4.0]])
    st = oracle.compare(gpu, ref)
    assert st["maxabs"] == 2.0
    assert st["rel"] == 1.0


def test_maxabs_takes_the_absolute_difference():
    # the largest difference is negative (-3); a max over signed differences
    # would report 0.5
    ref = np.array([[0.0, 3.0, 1.0]])
    gpu = np.array([[0.5, 0.0, 1.0]])
    st = oracle.compare(gpu, ref)
    assert st["maxabs"] == 3.0
    assert st["rel"] == 1.0


def test_tokens_are_the_last_axis_of_any_rank():
    # [B=2, N=2, D=2]: four tokens; only token (1, 0) is off, by a sign flip
    # of its second feature: cosine (1 - 1) / 2 = 0
    ref = np.ones((2, 2, 2))
    gpu = ref.copy()
    gpu[1, 0, 1] = -1.0
    st = oracle.compare(gpu, ref)
    assert st["min_cos"] == 0.0
    assert st["maxabs"] == 2.0


def test_cosine_runs_over_the_feature_axis():
    # rows are tokens: token 1 is [1, 1] against [0, 1], cosine 1 / sqrt(2);
    # over columns instead the minimum would be 4 / (2 sqrt(5)) = 0.894
    ref = np.array([[2.0, 0.0], [0.0, 1.0]])
    gpu = np.array([[2.0, 0.0], [1.0, 1.0]])
    st = oracle.compare(gpu, ref)
    assert math.isclose(st["min_cos"], 1.0 / math.sqrt(2.0), rel_tol=0, abs_tol=1e-15)


def test_non_finite_output_is_flagged():
    ref = np.array([[1.0, 2.0]])
    gpu = np.array([[1.0, np.nan]])
    assert oracle.compare(gpu, ref)["finite"] is False
    gpu = np.array([[np.inf, 2.0]])
    assert oracle.compare(gpu, ref)["finite"] is False


def test_identical_inputs():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((3, 5, 7))
    st = oracle.compare(ref.copy(), ref)
    assert st["maxabs"] == 0.0 and st["rel"] == 0.0
    assert abs(st["min_cos"] - 1.0) < 1e-15
