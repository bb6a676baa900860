"""Pins of the oracle's transpose (the weight preparation of the fused KV
projection, "PR #50585 完整报告", 实现拆解 item 2: the merged linear layer holds
[out, in]; the workload states the [in, out] matrix)."""
import numpy as np

import oracle


def test_matches_numpy_transpose_on_random_patterns():
    rng = np.random.default_rng(3)
    for rows, cols in ((1, 1), (3, 5), (64, 72), (130, 24)):
        a = rng.integers(0, 65536, (rows, cols)).astype(np.uint16)
        assert np.array_equal(oracle.transpose(a), a.T)


def test_strided_rows_and_involution():
    rng = np.random.default_rng(4)
    big = rng.integers(0, 65536, (40, 64)).astype(np.uint16)
    a = big[:, 8:40]                      # row stride 64, 32 columns
    t = oracle.transpose(a)
    assert t.shape == (32, 40) and np.array_equal(t, a.T)
    assert np.array_equal(oracle.transpose(t), a)


def test_closed_form_small():
    a = np.array([[1, 2, 3], [4, 5, 6]], np.uint16)
    assert oracle.transpose(a).tolist() == [[1, 4], [2, 5], [3, 6]]


def test_planted_index_swap_is_caught():
    """A transpose that confuses the two strides on a non-square matrix
    (a plausible mistake) gives a different result."""
    a = np.arange(12, dtype=np.uint16).reshape(3, 4)
    wrong = a.reshape(4, 3)               # reinterpreting instead of transposing
    assert not np.array_equal(oracle.transpose(a), wrong)
