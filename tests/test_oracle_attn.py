"""Pins of the CPU oracle's block attention against facts fixed outside it.

Closed forms (one-edge rows, zero query weights, a 2-edge scalar case worked
by hand), a library routine (torch's scaled_dot_product_attention in fp64 on
the CPU, per centre), the ragged pair-axis form the pages describe (a
different summation structure, agreement to 1e-13), and structural
properties (permutation equivariance through `order`, layer composition,
per-centre closure).
"""
import math

import numpy as np
import pytest
import torch

import workloads as W


def _normwise(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _case(n_centres, max_len, c, layers, seed, min_len=0):
    row_ptr = W.random_rows(n_centres, max_len, seed, min_len=min_len)
    e = int(row_ptr[-1])
    x = W.make_features(e, c, seed + 1)
    w = W.make_weights(layers, c, seed + 2)
    return row_ptr, x, w


def test_single_edge_rows_reduce_to_value_then_output_projection(oracle_mod):
    """n_i = 1: the softmax weight is 1, so y = x Wv Wo per layer."""
    row_ptr = np.arange(6, dtype=np.int64)
    x = W.make_features(5, 12, 3)
    w = W.make_weights(3, 12, 4)
    y = oracle_mod.attn_naive(row_ptr, x, w, heads=3)
    ref = x.copy()
    for l in range(3):
        ref = ref @ w[l, 2] @ w[l, 3]
    assert _normwise(y, ref) < 1e-14


def test_zero_query_weights_give_uniform_average(oracle_mod):
    """Wq = 0: every score is 0, every weight is 1/n, so y_a = mean_b(x_b Wv) Wo for each row."""
    row_ptr, x, w = _case(7, 9, 16, 1, 10, min_len=1)
    w[0, 0] = 0.0
    y = oracle_mod.attn_naive(row_ptr, x, w, heads=4)
    for i in range(7):
        blk = x[row_ptr[i]:row_ptr[i + 1]]
        ref = (blk @ w[0, 2]).mean(axis=0) @ w[0, 3]
        assert _normwise(y[row_ptr[i]:row_ptr[i + 1]], np.broadcast_to(ref, blk.shape)) < 1e-14


def test_two_edge_scalar_case_by_hand(oracle_mod):
    """c = H = 1, x = (1, -1), wq = 1, wk = 2, wv = 3, wo = 1/2.

    Scores s_ab = q_a k_b = [[2, -2], [-2, 2]], so row 0 weights (e^2, e^-2)/(e^2 + e^-2) and
    o_0 = 3 tanh 2, o_1 = -3 tanh 2; y = o / 2.
    """
    row_ptr = np.array([0, 2], np.int64)
    x = np.array([[1.0], [-1.0]])
    w = np.array([[[[1.0]], [[2.0]], [[3.0]], [[0.5]]]])
    y = oracle_mod.attn_naive(row_ptr, x, w, heads=1)
    t = 1.5 * math.tanh(2.0)
    assert abs(y[0, 0] - t) < 1e-15 and abs(y[1, 0] + t) < 1e-15
    y2 = oracle_mod.attn_pairaxis(row_ptr, x, w, heads=1)
    assert abs(y2[0, 0] - t) < 1e-15 and abs(y2[1, 0] + t) < 1e-15


@pytest.mark.parametrize("c,heads", [(16, 4), (32, 4), (24, 3), (8, 1)])
def test_matches_torch_sdpa_per_centre(oracle_mod, c, heads):
    """Per centre, the layer is torch SDPA (scale 1/sqrt(d)) between projections."""
    row_ptr, x, w = _case(9, 20, c, 1, 20 + c, min_len=1)
    y = oracle_mod.attn_naive(row_ptr, x, w, heads=heads)
    d = c // heads
    for i in range(9):
        blk = torch.from_numpy(x[row_ptr[i]:row_ptr[i + 1]])
        n = blk.shape[0]
        Wt = torch.from_numpy(w[0])
        q, k, v = (blk @ Wt[0], blk @ Wt[1], blk @ Wt[2])
        qh = q.reshape(n, heads, d).transpose(0, 1).contiguous()
        kh = k.reshape(n, heads, d).transpose(0, 1).contiguous()
        vh = v.reshape(n, heads, d).transpose(0, 1).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh)
        ref = (o.transpose(0, 1).reshape(n, c) @ Wt[3]).numpy()
        assert _normwise(y[row_ptr[i]:row_ptr[i + 1]], ref) < 1e-13


@pytest.mark.parametrize("seed,n_centres,max_len,c,heads,layers",
                         [(1, 20, 15, 16, 4, 1), (2, 11, 33, 32, 4, 2), (3, 30, 6, 8, 2, 3),
                          (4, 5, 1, 4, 1, 1)])
def test_naive_equals_pair_axis(oracle_mod, seed, n_centres, max_len, c, heads, layers):
    row_ptr, x, w = _case(n_centres, max_len, c, layers, seed)
    y1 = oracle_mod.attn_naive(row_ptr, x, w, heads)
    y2 = oracle_mod.attn_pairaxis(row_ptr, x, w, heads)
    assert _normwise(y2, y1) < 1e-13


def test_naive_equals_pair_axis_on_diamond_64(oracle_mod):
    w_ = W.WORKLOADS[1]
    pos, box = W.workload_positions(w_)
    row_ptr, col, shift, vec = oracle_mod.nl_full(pos, box, w_.rcut, w_.sel)
    x = W.workload_features(w_, int(row_ptr[-1]))
    w = W.workload_weights(w_)
    y1 = oracle_mod.attn_naive(row_ptr, x, w, w_.heads)
    y2 = oracle_mod.attn_pairaxis(row_ptr, x, w, w_.heads)
    assert _normwise(y2, y1) < 1e-13


def test_within_row_permutation_is_equivariant(oracle_mod):
    """Reordering a centre's edges through `order` leaves each edge's output unchanged."""
    row_ptr, x, w = _case(12, 14, 16, 2, 31)
    y = oracle_mod.attn_naive(row_ptr, x, w, 4)
    rng = np.random.default_rng(5)
    order = np.arange(row_ptr[-1], dtype=np.int32)
    for i in range(12):
        seg = order[row_ptr[i]:row_ptr[i + 1]]
        order[row_ptr[i]:row_ptr[i + 1]] = rng.permutation(seg)
    y2 = oracle_mod.attn_naive(row_ptr, x, w, 4, order=order)
    assert _normwise(y2, y) < 1e-14
    y3 = oracle_mod.attn_pairaxis(row_ptr, x, w, 4, order=order)
    assert _normwise(y3, y) < 1e-13


def test_storage_permutation_through_order(oracle_mod):
    """Edges stored at permuted rows and gathered through `order` give permuted outputs."""
    row_ptr, x, w = _case(10, 12, 8, 1, 41)
    y = oracle_mod.attn_naive(row_ptr, x, w, 2)
    e = int(row_ptr[-1])
    perm = np.random.default_rng(9).permutation(e).astype(np.int32)  # slot s is stored at perm[s]
    x2 = np.empty_like(x)
    x2[perm] = x
    y2 = oracle_mod.attn_naive(row_ptr, x2, w, 2, order=perm)
    assert np.array_equal(y2[perm], y)


def test_layers_compose(oracle_mod):
    row_ptr, x, w = _case(8, 10, 12, 3, 51)
    y = oracle_mod.attn_naive(row_ptr, x, w, 3)
    step = x
    for l in range(3):
        step = oracle_mod.attn_naive(row_ptr, step, w[l:l + 1], 3)
    assert np.array_equal(step, y)


def test_centre_list_matches_layer_by_layer(oracle_mod):
    row_ptr, x, w = _case(25, 18, 16, 2, 61)
    y = oracle_mod.attn_naive(row_ptr, x, w, 4)
    centres = np.array([0, 3, 7, 24, 11])
    y2 = oracle_mod.attn_naive_centres(row_ptr, x, w, 4, centres)
    for i in centres:
        s = slice(row_ptr[i], row_ptr[i + 1])
        assert np.array_equal(y2[s], y[s])


def test_empty_rows_and_empty_input(oracle_mod):
    row_ptr = np.array([0, 0, 3, 3, 4], np.int64)
    x = W.make_features(4, 8, 1)
    w = W.make_weights(1, 8, 2)
    y = oracle_mod.attn_naive(row_ptr, x, w, 2)
    assert np.all(np.isfinite(y))
    y0 = oracle_mod.attn_naive(np.zeros(3, np.int64), np.zeros((0, 8)), w, 2)
    assert y0.shape == (0, 8)


# --- smooth attention: w_j = softmax_j * (sum_j e_j / D~), a per-segment rescale -------------

def _lse_per_segment(row_ptr, x, w, heads):
    """ln sum_j exp(s_j) per (query edge, head) of a single layer, from torch's logsumexp over
    scores formed by torch matmuls (a library routine, independent of the oracle's loops)."""
    e, c = x.shape
    d = c // heads
    xt = torch.from_numpy(x)
    q, k = xt @ torch.from_numpy(w[0, 0]), xt @ torch.from_numpy(w[0, 1])
    out = np.zeros((1, e, heads))
    for i in range(row_ptr.shape[0] - 1):
        r0, r1 = int(row_ptr[i]), int(row_ptr[i + 1])
        if r1 == r0:
            continue
        for h in range(heads):
            sl = slice(h * d, (h + 1) * d)
            s = (q[r0:r1, sl] @ k[r0:r1, sl].T) / math.sqrt(d)
            out[0, r0:r1, h] = torch.logsumexp(s, dim=1).numpy()
    return out


def test_smooth_with_dtilde_equal_to_the_segment_sum_is_vanilla(oracle_mod):
    """D~ = sum_j e_j makes the rescale 1: the smooth form reduces to plain softmax."""
    row_ptr, x, w = _case(25, 30, 16, 1, 61, min_len=1)
    ldt = _lse_per_segment(row_ptr, x, w, heads=4)
    y = oracle_mod.attn_smooth(row_ptr, x, w, 4, ldt)
    assert _normwise(y, oracle_mod.attn_naive(row_ptr, x, w, 4)) < 1e-13


def test_smooth_rescale_is_per_segment_and_exponential(oracle_mod):
    """Raising ln D~ by delta on one (query edge, head) segment scales only that segment's
    head output, by exp(-delta): with Wo = I the output columns of head h are o_h itself."""
    row_ptr, x, w = _case(12, 20, 12, 1, 62, min_len=2)
    w[0, 3] = np.eye(12)
    ldt = _lse_per_segment(row_ptr, x, w, heads=3) + 0.3
    base = oracle_mod.attn_smooth(row_ptr, x, w, 3, ldt)
    ldt2 = ldt.copy()
    edge, head, delta = 7, 1, 1.7
    ldt2[0, edge, head] += delta
    y = oracle_mod.attn_smooth(row_ptr, x, w, 3, ldt2)
    expect = base.copy()
    expect[edge, 4 * head:4 * head + 4] *= math.exp(-delta)
    assert _normwise(y, expect) < 1e-14
    # and D~ above the segment sum by e^0.3 scales the vanilla output by e^-0.3
    assert _normwise(base, math.exp(-0.3) * oracle_mod.attn_naive(row_ptr, x, w, 3)) < 1e-13


def test_smooth_single_edge_closed_form(oracle_mod):
    """n_i = 1: the one weight is e / D~ = exp(s - ln D~) with s = (x Wq).(x Wk)/sqrt(d) per
    head, so y = [exp(s_h - ln D~_h) (x Wv)_h]_h Wo."""
    x = W.make_features(4, 8, 5)
    w = W.make_weights(1, 8, 6)
    row_ptr = np.arange(5, dtype=np.int64)
    ldt = np.random.default_rng(7).normal(0.0, 1.0, (1, 4, 2))
    y = oracle_mod.attn_smooth(row_ptr, x, w, 2, ldt)
    q, k, v = x @ w[0, 0], x @ w[0, 1], x @ w[0, 2]
    o = np.zeros_like(v)
    for a in range(4):
        for h in range(2):
            sl = slice(4 * h, 4 * h + 4)
            s = float(q[a, sl] @ k[a, sl]) / 2.0
            o[a, sl] = math.exp(s - ldt[0, a, h]) * v[a, sl]
    assert _normwise(y, o @ w[0, 3]) < 1e-14


def test_smooth_layers_take_their_own_dtilde(oracle_mod):
    """Layer l reads ln D~[l]: a shift of layer 1's values leaves layer 0 alone, and with one
    layer the smooth form of a two-layer stack's first layer is the one-layer result."""
    row_ptr, x, w = _case(10, 15, 8, 2, 63, min_len=1)
    ldt = np.random.default_rng(64).normal(2.0, 0.5, (2, x.shape[0], 2))
    y2 = oracle_mod.attn_smooth(row_ptr, x, w, 2, ldt)
    y1 = oracle_mod.attn_smooth(row_ptr, x, w[:1], 2, ldt[:1])
    y12 = oracle_mod.attn_smooth(row_ptr, y1, w[1:], 2, ldt[1:])
    assert _normwise(y2, y12) < 1e-14
