"""The oracle's block gather / scatter (the padded per-centre block of the destination CSR and
its scatter back) against facts fixed outside it: a hand-worked example, the inverse relation,
the `order` permutation, bit patterns of special values, and the error cases."""
import numpy as np
import pytest

import workloads as W


def test_hand_example(oracle_mod):
    # centres with 2, 0 and 3 edges, cap 3, two channels
    rp = np.array([0, 2, 2, 5], np.int64)
    x = np.arange(10, dtype=np.float64).reshape(5, 2) + 1.0  # rows (1,2), (3,4), ..., (9,10)
    b = oracle_mod.block_gather(rp, x, 3)
    want = np.array([[[1, 2], [3, 4], [0, 0]],
                     [[0, 0], [0, 0], [0, 0]],
                     [[5, 6], [7, 8], [9, 10]]], dtype=np.float64)
    assert b.shape == (3, 3, 2) and np.array_equal(b, want)
    y = np.full((6, 2), -1.0)  # one row more than the CSR covers: left alone
    oracle_mod.block_scatter(rp, b * 10.0, y)
    assert np.array_equal(y[:5], x * 10.0) and np.array_equal(y[5], [-1.0, -1.0])


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_scatter_inverts_gather_and_order_relabels(oracle_mod, dtype):
    rp = W.random_rows(40, 50, 3)
    e = int(rp[-1])
    x = W.make_features(e, 24, 4, dtype)
    b = oracle_mod.block_gather(rp, x, 50)
    lens = np.diff(rp)
    for i in range(len(lens)):
        assert np.all(b[i, lens[i]:] == 0)
        assert np.array_equal(b[i, :lens[i]], x[rp[i]:rp[i + 1]])
    y = np.zeros_like(x)
    assert np.array_equal(oracle_mod.block_scatter(rp, b, y), x)
    # rows stored at perm[s] and read through order = perm give the same block
    perm = np.random.default_rng(5).permutation(e).astype(np.int32)
    x2 = np.empty_like(x)
    x2[perm] = x
    b2 = oracle_mod.block_gather(rp, x2, 50, order=perm)
    assert np.array_equal(b2, b)
    y2 = np.zeros_like(x)
    oracle_mod.block_scatter(rp, b2, y2, order=perm)
    assert np.array_equal(y2, x2)


def test_bits_are_copied_exactly(oracle_mod):
    rp = np.array([0, 4], np.int64)
    x = np.array([[np.nan, -0.0], [np.inf, -np.inf], [5e-324, -1e308], [1.0, 2.0]])
    b = oracle_mod.block_gather(rp, x, 6)
    assert np.array_equal(b[0, :4].view(np.uint64), x.view(np.uint64))
    assert np.array_equal(b[0, 4:].view(np.uint64), np.zeros((2, 2), np.uint64))


def test_errors(oracle_mod):
    x = np.zeros((5, 2))
    with pytest.raises(ValueError):
        oracle_mod.block_gather(np.array([0, 5], np.int64), x, 4)   # row longer than cap
    with pytest.raises(ValueError):
        oracle_mod.block_gather(np.array([0, 2], np.int64), x, 4,
                                order=np.array([0, 9], np.int32))  # index out of range
    with pytest.raises(ValueError):
        oracle_mod.block_gather(np.array([0, 3, 2], np.int64), x, 4)  # decreasing row_ptr
