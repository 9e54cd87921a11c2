"""Pins of the oracle's LocalAtten (one query per centre over the centre's edges).

Closed forms (one-edge rows, zero query weights), a library routine (torch's
scaled_dot_product_attention in fp64 with one query per centre), an identity with the
oracle's block self-attention (a centre whose query is one of its own edge rows gets that
edge's block-attention output), empty rows, the `order` permutation and layer composition.
"""
import numpy as np
import pytest
import torch

import workloads as W


def _normwise(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _case(n_centres, max_len, c, layers, seed, min_len=1):
    row_ptr = W.random_rows(n_centres, max_len, seed, min_len=min_len)
    e = int(row_ptr[-1])
    x = W.make_features(e, c, seed + 1)
    xc = W.make_features(n_centres, c, seed + 3)
    w = W.make_weights(layers, c, seed + 2)
    return row_ptr, xc, x, w


def test_one_edge_rows_give_value_then_output_projection(oracle_mod):
    """n_i = 1: the only weight is 1, so yc_i = (x_e Wv) Wo whatever the query."""
    row_ptr = np.arange(7, dtype=np.int64)
    x = W.make_features(6, 16, 1)
    xc = W.make_features(6, 16, 2)
    w = W.make_weights(1, 16, 3)
    yc = oracle_mod.local_atten(row_ptr, xc, x, w, heads=4)
    assert _normwise(yc, x @ w[0, 2] @ w[0, 3]) < 1e-14


def test_zero_query_weights_average_the_values(oracle_mod):
    """Wq = 0: all scores vanish, each head averages its centre's value rows."""
    row_ptr, xc, x, w = _case(15, 20, 12, 1, 11)
    w[0, 0] = 0.0
    yc = oracle_mod.local_atten(row_ptr, xc, x, w, heads=3)
    v = x @ w[0, 2]
    mean = np.stack([v[row_ptr[i]:row_ptr[i + 1]].mean(axis=0) for i in range(15)])
    assert _normwise(yc, mean @ w[0, 3]) < 1e-14


@pytest.mark.parametrize("c,heads", [(16, 4), (32, 4), (24, 3)])
def test_matches_torch_sdpa_one_query_per_centre(oracle_mod, c, heads):
    row_ptr, xc, x, w = _case(20, 30, c, 1, 21)
    yc = oracle_mod.local_atten(row_ptr, xc, x, w, heads=heads)
    d = c // heads
    t = lambda a: torch.from_numpy(a)
    q = t(xc) @ t(w[0, 0])
    k, v = t(x) @ t(w[0, 1]), t(x) @ t(w[0, 2])
    ref = np.zeros_like(xc)
    for i in range(20):
        r0, r1 = int(row_ptr[i]), int(row_ptr[i + 1])
        qi = q[i].reshape(heads, 1, d)                             # [heads][1][d]
        ki = k[r0:r1].reshape(r1 - r0, heads, d).transpose(0, 1)   # [heads][n][d]
        vi = v[r0:r1].reshape(r1 - r0, heads, d).transpose(0, 1)
        o = torch.nn.functional.scaled_dot_product_attention(qi, ki.contiguous(), vi.contiguous())
        ref[i] = (o.transpose(0, 1).reshape(c) @ t(w[0, 3])).numpy()
    assert _normwise(yc, ref) < 1e-13


def test_query_equal_to_an_own_edge_row_is_block_attention(oracle_mod):
    """With xc_i = x of the centre's first edge, LocalAtten's single query is that edge's
    query row of the block self-attention, so yc_i = y_block[first edge] (one layer)."""
    row_ptr, _, x, w = _case(30, 25, 16, 1, 31)
    xc = x[row_ptr[:-1]]
    yc = oracle_mod.local_atten(row_ptr, xc, x, w, heads=4)
    yb = oracle_mod.attn_naive(row_ptr, x, w, heads=4)
    assert _normwise(yc, yb[row_ptr[:-1]]) < 1e-13


def test_empty_rows_give_zero_and_other_rows_are_unaffected(oracle_mod):
    row_ptr, xc, x, w = _case(12, 10, 8, 1, 41)
    lens = np.diff(row_ptr)
    lens[[2, 7]] = 0
    rp2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x2 = W.make_features(int(rp2[-1]), 8, 42)
    yc = oracle_mod.local_atten(rp2, xc, x2, w, heads=2)
    assert np.all(yc[[2, 7]] == 0.0)
    keep = [i for i in range(12) if i not in (2, 7)]
    rp3 = np.concatenate([[0], np.cumsum(lens[keep])]).astype(np.int64)
    yc3 = oracle_mod.local_atten(rp3, xc[keep], x2, w, heads=2)
    assert _normwise(yc[keep], yc3) < 1e-15


def test_order_permutation_and_layer_composition(oracle_mod):
    row_ptr, xc, x, w = _case(20, 18, 12, 3, 51)
    e = x.shape[0]
    perm = np.random.default_rng(52).permutation(e).astype(np.int32)
    x2 = np.empty_like(x)
    x2[perm] = x
    y = oracle_mod.local_atten(row_ptr, xc, x, w, heads=3)
    assert _normwise(oracle_mod.local_atten(row_ptr, xc, x2, w, heads=3, order=perm), y) < 1e-14
    y1 = oracle_mod.local_atten(row_ptr, xc, x, w[:1], heads=3)
    y12 = oracle_mod.local_atten(row_ptr, y1, x, w[1:], heads=3)
    assert _normwise(y12, y) < 1e-14
