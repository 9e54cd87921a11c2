"""GPU smooth attention (per-segment softmax rescale by sum_j e_j / D~) against the oracle.

Every kernel path the dispatcher can take -- the fused fp32 kernel (fp32 matrix cores, and the
f16 split-pair arithmetic asked for by NGA_F32_SPLIT16), the fused fp64 kernel, the fp64
matrix-core path and the generic path in both precisions -- against oracle.attn_smooth, normwise
(1e-12 fp64 / 2e-5 fp32), over several layers, with ln D~ drawn per layer, edge and head.
Plus: ln D~ equal to each segment's log-sum-exp reproduces the vanilla forward; the `order`
permutation keys ln D~ by edge row; factors far from one (e^-60 .. e^60, differing between the
heads of one query) keep every edge row accurate relative to its own magnitude.
"""
import math

import numpy as np
import pytest
import torch

import neighbour_graph_attention_amd as nga
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {np.float64: 1e-12, np.float32: 2e-5}


def _normwise(y, ref):
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def _run(row_ptr, x, w, heads, cap, ldt=None, order=None, ws=None, check=True, split16=False):
    ws = ws or nga.Workspace(DEV)
    y = nga.block_attn_forward(
        torch.from_numpy(row_ptr).to(DEV), torch.from_numpy(x).to(DEV),
        torch.from_numpy(w).to(DEV), heads, cap,
        order=None if order is None else torch.from_numpy(order).to(DEV), ws=ws,
        log_dtilde=None if ldt is None else torch.from_numpy(ldt).to(DEV), split16=split16)
    if check:
        nga.check_status(ws, "attention")
    return y.cpu().numpy()


def _segment_lse(row_ptr, x, w_layer, heads):
    """ln sum_j exp(s_j) per (query edge, head) of one layer with weights w_layer [4][c][c]."""
    e, c = x.shape
    d = c // heads
    xt = torch.from_numpy(x.astype(np.float64))
    q = xt @ torch.from_numpy(w_layer[0].astype(np.float64))
    k = xt @ torch.from_numpy(w_layer[1].astype(np.float64))
    out = np.zeros((e, heads))
    for i in range(row_ptr.shape[0] - 1):
        r0, r1 = int(row_ptr[i]), int(row_ptr[i + 1])
        for h in range(heads):
            sl = slice(h * d, (h + 1) * d)
            s = (q[r0:r1, sl] @ k[r0:r1, sl].T) / math.sqrt(d)
            out[r0:r1, h] = torch.logsumexp(s, dim=1).numpy()
    return out


def _log_dtilde(oracle_mod, row_ptr, x, w, heads, dtype, seed):
    """ln D~ = each segment's log-sum-exp + U(-1/2, 1/2), layer by layer along the oracle's
    smooth forward, so that every rescale lies in [e^-1/2, e^1/2]: D~ of the order of the
    segment sum, as an occupancy-corrected denominator is.  Far from it the smooth outputs
    of one layer grow or shrink without bound in the next and the comparison measures the
    conditioning of the inputs, not the kernels."""
    rng = np.random.default_rng(seed)
    layers = w.shape[0]
    cur = x.astype(np.float64)
    ldt = np.zeros((layers, x.shape[0], heads))
    for l in range(layers):
        ldt[l] = _segment_lse(row_ptr, cur, w[l], heads) + rng.uniform(-0.5, 0.5, ldt[l].shape)
        ldt[l] = ldt[l].astype(dtype)  # the values the kernel sees
        cur = oracle_mod.attn_smooth(row_ptr, cur, w[l:l + 1].astype(np.float64), heads,
                                     ldt[l:l + 1])
    return ldt.astype(dtype)


CASES = [
    # dtype, n_centres, max_len, c, heads, layers, seed, expected variant
    (np.float32, 40, 181, 64, 4, 2, 1, "fused_f32"),
    (np.float32, 40, 96, 32, 2, 3, 2, "fused_f32"),
    (np.float32, 30, 40, 16, 1, 1, 3, "fused_f32"),
    (np.float32, 40, 181, 64, 4, 2, 1, "fused_f32_split16"),
    (np.float32, 40, 96, 32, 2, 3, 2, "fused_f32_split16"),
    (np.float32, 30, 40, 16, 1, 1, 3, "fused_f32_split16"),
    (np.float64, 30, 120, 128, 4, 2, 4, "mfma_f64"),
    (np.float64, 40, 40, 32, 4, 2, 5, "fused_f64"),
    (np.float64, 30, 90, 64, 4, 2, 8, "mfma_f64"),
    (np.float64, 220, 120, 128, 4, 2, 9, "mfma_f64"),   # one work-group per centre, heads of 32
    (np.float64, 220, 100, 128, 8, 1, 10, "mfma_f64"),  # the same, heads of 16
    (np.float64, 20, 30, 20, 2, 2, 6, "generic_f64"),
    (np.float32, 20, 60, 40, 5, 2, 7, "generic_f32"),
]


@pytest.mark.parametrize("dtype,nc,maxlen,c,heads,layers,seed,variant", CASES)
def test_smooth_matches_oracle(oracle_mod, dtype, nc, maxlen, c, heads, layers, seed, variant):
    rp = W.random_rows(nc, maxlen, seed)
    lens = np.diff(rp)
    for k, v in enumerate([0, 1, maxlen, 17]):
        lens[k] = v
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    e = int(rp[-1])
    x = W.make_features(e, c, seed + 100, dtype)
    wt = W.make_weights(layers, c, seed + 200, dtype)
    ldt = _log_dtilde(oracle_mod, rp, x, wt, heads, dtype, seed + 300)
    split16 = variant.endswith("split16")
    dt = nga.NGA_F64 if dtype == np.float64 else (nga.NGA_F32_SPLIT16 if split16 else nga.NGA_F32)
    assert nga.attn_variant(dt, maxlen, c, heads) == variant
    y = _run(rp, x, wt, heads, maxlen, ldt=ldt, split16=split16)
    ref = oracle_mod.attn_smooth(rp, x.astype(np.float64), wt.astype(np.float64), heads,
                                 ldt.astype(np.float64))
    err = _normwise(y.astype(np.float64), ref)
    print(f"{variant} c={c} H={heads} L={layers}: normwise error {err:.3e}", flush=True)
    assert err < TOL[dtype]


@pytest.mark.parametrize("dtype,c,heads,cap,split16", [
    (np.float32, 64, 4, 181, False), (np.float32, 64, 4, 181, True), (np.float64, 32, 4, 60, False),
    (np.float64, 64, 4, 90, False), (np.float64, 20, 2, 40, False)])
def test_dtilde_equal_to_segment_sum_is_vanilla(dtype, c, heads, cap, split16):
    rp = W.random_rows(30, cap, 11, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, c, 12, dtype)
    wt = W.make_weights(1, c, 13, dtype)
    ldt = _segment_lse(rp, x, wt[0], heads)[None].astype(dtype)
    ys = _run(rp, x, wt, heads, cap, ldt=ldt, split16=split16)
    yv = _run(rp, x, wt, heads, cap, split16=split16)
    assert _normwise(ys.astype(np.float64), yv.astype(np.float64)) < TOL[dtype]


@pytest.mark.parametrize("dtype,c,heads,cap", [(np.float32, 64, 4, 120), (np.float64, 32, 4, 60)])
def test_smooth_order_keys_by_edge_row(oracle_mod, dtype, c, heads, cap):
    rp = W.random_rows(25, cap, 21, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, c, 22, dtype)
    wt = W.make_weights(2, c, 23, dtype)
    ldt = _log_dtilde(oracle_mod, rp, x, wt, heads, dtype, 24)  # keyed by unpermuted row
    perm = np.random.default_rng(25).permutation(e).astype(np.int32)
    x2 = np.empty_like(x)
    x2[perm] = x
    ldt2 = np.empty_like(ldt)
    ldt2[:, perm, :] = ldt  # edge row perm[s] carries slot s's ln D~
    y2 = _run(rp, x2, wt, heads, cap, ldt=ldt2, order=perm)
    ref = oracle_mod.attn_smooth(rp, x.astype(np.float64), wt.astype(np.float64), heads,
                                 ldt.astype(np.float64))
    assert _normwise(y2[perm].astype(np.float64), ref) < TOL[dtype]


def _rowwise(y, ref):
    """Largest over edge rows of max |y_r - ref_r| / max |ref_r| (rows with ref_r = 0 skipped)."""
    den = np.max(np.abs(ref), axis=1)
    num = np.max(np.abs(y - ref), axis=1)
    keep = den > 0
    return float(np.max(num[keep] / den[keep]))


@pytest.mark.parametrize("dtype,c,heads,cap,split16", [
    (np.float32, 64, 4, 120, False), (np.float32, 32, 2, 60, False), (np.float32, 64, 4, 120, True),
    (np.float32, 32, 2, 60, True), (np.float64, 32, 4, 60, False)])
def test_factors_far_from_one_match_oracle_row_by_row(oracle_mod, dtype, c, heads, cap, split16):
    """Rescale factors sum_j e_j / D~ of e^40, 1, e^-30 and e^60 on the heads of the same
    query rows, then factors spread over e^-60 .. e^60 row by row: every edge row of y must
    match the oracle to the tolerance relative to that row's own magnitude."""
    rp = W.random_rows(30, cap, 41, min_len=1)
    lens = np.diff(rp)
    lens[0] = 1
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    e = int(rp[-1])
    x = W.make_features(e, c, 42, dtype)
    wt = W.make_weights(1, c, 43, dtype)
    lse = _segment_lse(rp, x, wt[0], heads)
    per_head = np.array([-40.0, 0.0, 30.0, -60.0])[:heads]
    spread = np.random.default_rng(44).uniform(-60.0, 60.0, (e, 1))
    for shift in (per_head[None, :], spread):
        ldt = (lse + shift)[None].astype(dtype)
        y = _run(rp, x, wt, heads, cap, ldt=ldt, split16=split16)
        ref = oracle_mod.attn_smooth(rp, x.astype(np.float64), wt.astype(np.float64), heads,
                                     ldt.astype(np.float64))
        assert np.all(np.isfinite(y))
        err = _rowwise(y.astype(np.float64), ref)
        print(f"{dtype.__name__} c={c} H={heads}: row-wise error {err:.3e}", flush=True)
        assert err < TOL[dtype]
