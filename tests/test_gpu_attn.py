"""GPU block-dense attention against the oracle, normwise.

Tolerances (max |y - y_ref| / max |y_ref| over the compared rows): 1e-12 for
fp64 and 2e-5 for fp32, where the oracle runs in fp64 on the same (fp32-
rounded) inputs.  Whole outputs on the diamond workloads and on random
ragged rows (lengths across tile boundaries, empty and one-edge rows, rows
at the cap), sampled centres carried through every layer on the Fe BCC
workloads at full size, the `order` gather/scatter, run-to-run determinism,
and the device-detected error paths.
"""
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


def _run(row_ptr, x, w, heads, cap, order=None, ws=None):
    ws = ws or nga.Workspace(DEV)
    y = nga.block_attn_forward(torch.from_numpy(row_ptr).to(DEV), torch.from_numpy(x).to(DEV),
                               torch.from_numpy(w).to(DEV), heads, cap,
                               order=None if order is None else torch.from_numpy(order).to(DEV),
                               ws=ws)
    nga.check_status(ws, "attention")
    return y.cpu().numpy()


def _gpu_workload_csr(w):
    pos, box = W.workload_positions(w)
    p = torch.from_numpy(pos).to(DEV)
    nbr, nbr_shift, nnei = nga.nl_build(p, box, w.rcut, w.sel)
    csr = nga.edge_csr(nbr, nbr_shift, nnei)
    nga.check_status(csr["ws"], "csr")
    return pos, box, csr["row_ptr"].cpu().numpy(), csr["n_edges"]


@pytest.mark.parametrize("key", [1, 2, 3])
def test_diamond_workloads_whole_output(oracle_mod, key):
    w = W.WORKLOADS[key]
    pos, box, rp, e = _gpu_workload_csr(w)
    rp_ref, _, _, _ = oracle_mod.nl_full(pos, box, w.rcut, w.sel)
    assert np.array_equal(rp, rp_ref)
    x = W.workload_features(w, e)
    wt = W.workload_weights(w)
    print(f"workload {w.name} E={e} variant={nga.attn_variant(0, w.sel, w.c, w.heads)}", flush=True)
    y = _run(rp, x, wt, w.heads, w.sel)
    ref = oracle_mod.attn_naive(rp, x, wt, w.heads)
    err = _normwise(y, ref)
    print(f"normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float64]


@pytest.mark.parametrize("key", [4, 5])
def test_fe_bcc_full_size_sampled_centres(oracle_mod, key):
    w = W.WORKLOADS[key]
    pos, box, rp, e = _gpu_workload_csr(w)
    n = rp.shape[0] - 1
    x = W.workload_features(w, e)
    wt = W.workload_weights(w)
    print(f"workload {w.name} N={n} E={e} variant={nga.attn_variant(1, w.sel, w.c, w.heads)}",
          flush=True)
    y = _run(rp, x, wt, w.heads, w.sel)
    rng = np.random.default_rng(2000 + key)
    centres = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 200, replace=False)]))
    ref = oracle_mod.attn_naive_centres(rp, x.astype(np.float64), wt.astype(np.float64), w.heads,
                                        centres)
    rows = np.concatenate([np.arange(rp[i], rp[i + 1]) for i in centres])
    err = _normwise(y[rows].astype(np.float64), ref[rows])
    print(f"sampled normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float32]
    assert np.all(np.isfinite(y))


CASES = [
    # (dtype, n_centres, max_len, c, heads, layers, seed)
    (np.float64, 40, 40, 32, 4, 2, 1),
    (np.float64, 30, 120, 128, 4, 1, 2),
    (np.float64, 50, 45, 32, 4, 3, 3),
    (np.float64, 20, 33, 24, 3, 1, 4),
    (np.float64, 10, 70, 8, 1, 2, 5),
    (np.float64, 30, 128, 64, 4, 2, 11),     # head width 16, rows up to the 128 cap
    (np.float64, 20, 150, 32, 4, 1, 12),     # rows past 128: generic path
    (np.float64, 20, 30, 20, 2, 2, 13),      # head width 10: generic path
    (np.float32, 20, 60, 40, 5, 1, 14),      # 5 heads of 8: generic path
    (np.float32, 60, 181, 64, 4, 2, 6),
    (np.float32, 40, 176, 64, 4, 1, 7),
    (np.float32, 40, 96, 32, 2, 1, 8),
    (np.float32, 25, 50, 48, 3, 2, 9),
    (np.float32, 30, 20, 16, 1, 1, 10),
    (np.float32, 20, 400, 64, 4, 2, 15),     # rows past 192: generic online-softmax path
    (np.float32, 10, 512, 16, 1, 1, 16),     # rows at the 512-neighbour cap
    (np.float64, 15, 300, 32, 4, 1, 17),     # fp64 rows past 128: generic path
    (np.float64, 40, 64, 32, 4, 6, 18),      # fused fp64: rows up to its 64 cap, six layers
    (np.float64, 30, 64, 32, 2, 2, 19),      # fused fp64, heads of 16
    (np.float64, 30, 50, 16, 1, 3, 20),      # fused fp64, one head of 16
    (np.float64, 20, 64, 8, 1, 2, 21),       # fused fp64, one head of 8
    (np.float64, 20, 65, 32, 4, 2, 22),      # rows past 64: fp64 matrix-core path
    (np.float64, 25, 64, 16, 2, 2, 25),      # fused fp64, two heads of 8 (stacked Q/K tiles)
    (np.float64, 25, 48, 32, 2, 3, 26),      # fused fp64, two heads of 16, three key tiles
    (np.float64, 25, 100, 64, 2, 2, 27),     # fp64 matrix-core path, heads of 32, rows < 128
    (np.float32, 20, 192, 64, 4, 2, 23),     # fused fp32 at its 192-row cap (12 full tiles)
    (np.float32, 20, 192, 16, 1, 1, 24),     # the same with one head
]


@pytest.mark.parametrize("dtype,nc,maxlen,c,heads,layers,seed", CASES)
def test_random_ragged_rows(oracle_mod, dtype, nc, maxlen, c, heads, layers, seed):
    rp = W.random_rows(nc, maxlen, seed)
    # force the edge cases: an empty row, a one-edge row, a full-cap row, tile boundaries
    lens = np.diff(rp)
    special = [0, 1, maxlen, 15, 16, 17, 31, 32, 33, 63, 64, 65]
    for k, v in enumerate(special[: nc]):
        lens[k] = min(v, maxlen)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    e = int(rp[-1])
    x = W.make_features(e, c, seed + 100, dtype)
    wt = W.make_weights(layers, c, seed + 200, dtype)
    print(f"case dtype={dtype.__name__} c={c} H={heads} L={layers} E={e} "
          f"variant={nga.attn_variant(0 if dtype == np.float64 else 1, maxlen, c, heads)}",
          flush=True)
    y = _run(rp, x, wt, heads, maxlen)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), heads)
    assert _normwise(y.astype(np.float64), ref) < TOL[dtype]


def _per_centre_normwise(y, ref, rp):
    worst = 0.0
    for i in range(rp.shape[0] - 1):
        if rp[i + 1] > rp[i]:
            worst = max(worst, _normwise(y[rp[i]:rp[i + 1]], ref[rp[i]:rp[i + 1]]))
    return worst


def test_f32_split_rounding_ties(oracle_mod):
    """fp32 projections on f16 matrix cores take each operand as two f16 parts (hi, lo).  Both
    parts must come from one rounded fp32 value: a head-output element at an f16 rounding tie
    otherwise gets its lo part from a differently rounded copy and lands one f16 ulp off.  The
    first block is 41 seeded rows that hold such ties; the rest are 400 blocks of 30 to 48 rows,
    over a million head-output elements."""
    rp0 = W.random_rows(20, 64, 5, min_len=1)
    x0 = W.make_features(int(rp0[-1]), 64, 6, np.float32)
    wt = W.make_weights(1, 64, 7, np.float32)
    blk = np.concatenate([x0[rp0[0]:rp0[1]], x0[100:]])[:41]
    lens = np.random.default_rng(31).integers(30, 49, 400)
    rp = np.concatenate([[0, 41], 41 + np.cumsum(lens)]).astype(np.int64)
    x = np.concatenate([blk, W.make_features(int(lens.sum()), 64, 32, np.float32)])
    y = _run(rp, x, wt, 4, 64)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), 4)
    err = _per_centre_normwise(y.astype(np.float64), ref, rp)
    print(f"worst per-centre normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float32]


@pytest.mark.parametrize("heads,layers", [(4, 2), (2, 1), (1, 3)])
def test_f32_per_centre_magnitudes(oracle_mod, heads, layers):
    """Centres whose features differ in magnitude by up to 2^21 each keep fp32-class relative
    accuracy against their own scale (the f16 split is scaled per centre and layer)."""
    c = 16 * heads
    rp = W.random_rows(60, 100, 41, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, c, 42, np.float32)
    k = np.random.default_rng(43).integers(-20, 2, rp.shape[0] - 1)
    for i in range(rp.shape[0] - 1):
        x[rp[i]:rp[i + 1]] *= np.float32(2.0 ** k[i])
    wt = W.make_weights(layers, c, 44, np.float32)
    y = _run(rp, x, wt, heads, 100)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), heads)
    err = _per_centre_normwise(y.astype(np.float64), ref, rp)
    print(f"variant={nga.attn_variant(1, 100, c, heads)} worst per-centre error {err:.3e}",
          flush=True)
    assert err < TOL[np.float32]


def test_f32_weight_magnitudes(oracle_mod):
    """Weight matrices scaled far from 1 (2^-30 .. 2^30, with non-power-of-two factors) give
    the same relative accuracy; the scales are paired so that the scores keep their size."""
    rp = W.random_rows(40, 181, 51, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, 64, 52, np.float32)
    wt = W.make_weights(2, 64, 53, np.float32)
    for (l, m), s in zip([(0, 0), (0, 1), (0, 2), (0, 3), (1, 0), (1, 2), (1, 3)],
                         [2.0 ** -30 * 3, 2.0 ** 28, 2.0 ** 30, 2.0 ** -30, 0.7, 2.0 ** -12, 5.0]):
        wt[l, m] *= np.float32(s)
    y = _run(rp, x, wt, 4, 181)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), 4)
    err = _normwise(y.astype(np.float64), ref)
    print(f"normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float32]


@pytest.mark.parametrize("dtype,c,heads,cap", [(np.float64, 32, 4, 60), (np.float64, 64, 4, 100),
                                             (np.float32, 64, 4, 181)])
def test_order_gather_scatter(oracle_mod, dtype, c, heads, cap):
    rp = W.random_rows(30, cap, 77, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, c, 78, dtype)
    wt = W.make_weights(2, c, 79, dtype)
    perm = np.random.default_rng(80).permutation(e).astype(np.int32)  # slot s stored at perm[s]
    x2 = np.empty_like(x)
    x2[perm] = x
    y2 = _run(rp, x2, wt, heads, cap, order=perm)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), heads)
    assert _normwise(y2[perm].astype(np.float64), ref) < TOL[dtype]


@pytest.mark.parametrize("dtype,c,heads,cap", [(np.float64, 32, 4, 40), (np.float64, 128, 4, 110),
                                             (np.float32, 64, 4, 181)])
def test_deterministic_and_cap_independent(dtype, c, heads, cap):
    rp = W.random_rows(50, cap, 91)
    e = int(rp[-1])
    x = W.make_features(e, c, 92, dtype)
    wt = W.make_weights(1, c, 93, dtype)
    a = _run(rp, x, wt, heads, cap)
    b = _run(rp, x, wt, heads, cap)
    assert np.array_equal(a, b)
    bigger = cap + 10  # a larger cap within the same kernel variant changes nothing
    dt = 0 if dtype == np.float64 else 1
    assert nga.attn_variant(dt, bigger, c, heads) == nga.attn_variant(dt, cap, c, heads)
    c2 = _run(rp, x, wt, heads, bigger)
    assert np.array_equal(a, c2)


PATH_CASES = [  # (dtype, c, heads, kernel path)
    (np.float64, 16, 4, "generic_f64"),
    (np.float64, 16, 2, "fused_f64"),
    (np.float64, 64, 4, "mfma_f64"),
    (np.float32, 16, 1, "fused_f32_d16"),
]


def _path_check(dtype, c, heads, cap, variant):
    assert nga.attn_variant(0 if dtype == np.float64 else 1, cap, c, heads) == variant


@pytest.mark.parametrize("dtype,c,heads,variant", PATH_CASES)
def test_rows_untouched_outside_centres(dtype, c, heads, variant):
    _path_check(dtype, c, heads, 8, variant)
    rp = np.array([0, 3, 3, 7], np.int64)
    x = W.make_features(10, c, 1, dtype)
    wt = W.make_weights(1, c, 2, dtype)
    xt = torch.from_numpy(x).to(DEV)
    y = torch.full_like(xt, 7.0)
    ws = nga.Workspace(DEV)
    nga.block_attn_forward(torch.from_numpy(rp).to(DEV), xt, torch.from_numpy(wt).to(DEV), heads,
                           8, y=y, ws=ws)
    nga.check_status(ws)
    assert torch.all(y[7:] == 7.0)


@pytest.mark.parametrize("dtype,c,heads,variant", PATH_CASES)
def test_row_over_cap_is_reported(dtype, c, heads, variant):
    _path_check(dtype, c, heads, 10, variant)
    rp = np.array([0, 5, 30], np.int64)
    x = W.make_features(30, c, 1, dtype)
    wt = W.make_weights(1, c, 2, dtype)
    ws = nga.Workspace(DEV)
    nga.block_attn_forward(torch.from_numpy(rp).to(DEV), torch.from_numpy(x).to(DEV),
                           torch.from_numpy(wt).to(DEV), heads, 10, ws=ws)
    assert nga.sync_status(ws) == -4


@pytest.mark.parametrize("dtype,c,heads,variant", PATH_CASES)
def test_order_out_of_range_is_reported(dtype, c, heads, variant):
    _path_check(dtype, c, heads, 8, variant)
    rp = np.array([0, 4, 8], np.int64)
    x = W.make_features(8, c, 1, dtype)
    wt = W.make_weights(1, c, 2, dtype)
    order = torch.tensor([0, 1, 2, 3, 4, 5, 6, 99], dtype=torch.int32, device=DEV)
    ws = nga.Workspace(DEV)
    nga.block_attn_forward(torch.from_numpy(rp).to(DEV), torch.from_numpy(x).to(DEV),
                           torch.from_numpy(wt).to(DEV), heads, 8, order=order, ws=ws)
    assert nga.sync_status(ws) == -8
