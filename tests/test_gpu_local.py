"""GPU LocalAtten (one query per centre over its edges) against the oracle.

Normwise tolerances as for block attention (1e-12 fp64 / 2e-5 fp32).  All five workloads
whole (the two Fe BCC workloads at full size after a sampled pre-check), random
ragged rows across the kernel's 64-row LDS chunks (empty rows, one-edge rows, rows up to the
512-neighbour cap), several layers and head counts, `order`, and the error paths.
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


def _local(row_ptr, xc, x, w, heads, order=None, ws=None):
    ws = ws or nga.Workspace(DEV)
    t = lambda a: torch.from_numpy(a).to(DEV)
    yc = nga.local_attn_forward(t(row_ptr), t(xc), t(x), t(w), heads,
                                order=None if order is None else t(order), ws=ws)
    nga.check_status(ws, "local_attn")
    return yc.cpu().numpy()


def _gpu_csr(w):
    pos, box = W.workload_positions(w)
    nbr, nbr_shift, nnei = nga.nl_build(torch.from_numpy(pos).to(DEV), box, w.rcut, w.sel)
    csr = nga.edge_csr(nbr, nbr_shift, nnei)
    nga.check_status(csr["ws"], "csr")
    return csr["row_ptr"].cpu().numpy(), csr["n_edges"]


@pytest.mark.parametrize("key", [1, 2, 3])
def test_diamond_workloads(oracle_mod, key):
    w = W.WORKLOADS[key]
    rp, e = _gpu_csr(w)
    n = rp.shape[0] - 1
    x = W.workload_features(w, e)
    xc = W.make_features(n, w.c, 500 + key, np.float64)
    wt = W.workload_weights(w)
    y = _local(rp, xc, x, wt, w.heads)
    ref = oracle_mod.local_atten(rp, xc, x, wt, w.heads)
    err = _normwise(y, ref)
    print(f"workload {w.name} N={n} E={e}: normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float64]


@pytest.mark.parametrize("key", [4, 5])
def test_fe_bcc_full_size_whole_output(oracle_mod, key):
    """Both Fe BCC workloads at full size (one and two layers), every centre's output against
    the oracle, after a sampled pre-check on 300 centres (the oracle runs on the sub-CSR of
    those centres: a centre's output depends only on its own rows)."""
    w = W.WORKLOADS[key]
    rp, e = _gpu_csr(w)
    n = rp.shape[0] - 1
    x = W.workload_features(w, e)
    xc = W.make_features(n, w.c, 500 + key, np.float32)
    wt = W.workload_weights(w)
    y = _local(rp, xc, x, wt, w.heads)
    assert np.all(np.isfinite(y))
    centres = np.unique(np.concatenate(
        [[0, n - 1], np.random.default_rng(5000 + key).choice(n, 300, replace=False)]))
    lens = rp[centres + 1] - rp[centres]
    sub_rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    sub_x = np.concatenate([x[rp[i]:rp[i + 1]] for i in centres])
    ref_s = oracle_mod.local_atten(sub_rp, xc[centres].astype(np.float64),
                                   sub_x.astype(np.float64), wt.astype(np.float64), w.heads)
    err_s = _normwise(y[centres].astype(np.float64), ref_s)
    print(f"workload {w.name} N={n} E={e}: sampled normwise error {err_s:.3e}", flush=True)
    assert err_s < TOL[np.float32]
    ref = oracle_mod.local_atten(rp, xc.astype(np.float64), x.astype(np.float64),
                                 wt.astype(np.float64), w.heads)
    err = _normwise(y.astype(np.float64), ref)
    print(f"workload {w.name}: whole-output normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float32]


CASES = [
    # dtype, n_centres, max_len, c, heads, layers, seed
    (np.float32, 60, 181, 64, 4, 1, 1),
    (np.float32, 30, 512, 64, 4, 2, 2),      # rows up to the neighbour cap: 8 chunks
    (np.float32, 40, 100, 40, 5, 3, 3),
    (np.float32, 20, 70, 256, 16, 1, 4),     # widest rows: fewer than 64 rows per chunk
    (np.float32, 50, 20, 16, 1, 2, 5),
    (np.float64, 40, 130, 128, 4, 2, 6),     # 55 rows per chunk
    (np.float64, 30, 70, 32, 4, 6, 7),
    (np.float64, 20, 200, 20, 2, 1, 8),
    (np.float32, 30, 150, 32, 4, 2, 10),
]


@pytest.mark.parametrize("dtype,nc,maxlen,c,heads,layers,seed", CASES)
def test_random_ragged_rows(oracle_mod, dtype, nc, maxlen, c, heads, layers, seed):
    rp = W.random_rows(nc, maxlen, seed)
    lens = np.diff(rp)
    # empty, one row, the cap, and the edges of 16-row blocks and 64-row chunks
    for k, v in enumerate([0, 1, maxlen, 63, 64, 65, 128, 129, 15, 16, 17, 31, 33]):
        lens[k] = min(v, maxlen)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    e = int(rp[-1])
    x = W.make_features(e, c, seed + 100, dtype)
    xc = W.make_features(nc, c, seed + 150, dtype)
    wt = W.make_weights(layers, c, seed + 200, dtype)
    y = _local(rp, xc, x, wt, heads)
    ref = oracle_mod.local_atten(rp, xc.astype(np.float64), x.astype(np.float64),
                                 wt.astype(np.float64), heads)
    err = _normwise(y.astype(np.float64), ref)
    print(f"{dtype.__name__} c={c} H={heads} L={layers} max_len={maxlen}: {err:.3e}", flush=True)
    assert err < TOL[dtype]
    assert np.all(y[0] == 0.0)  # the empty centre


@pytest.mark.parametrize("dtype,c,heads,n", [(np.float32, 64, 4, n) for n in (13, 16, 61, 181)]
                         + [(np.float64, 32, 4, n) for n in (29, 64)] + [(np.float32, 32, 2, 47)])
def test_every_copy_of_one_centre(oracle_mod, dtype, c, heads, n):
    """2,048 copies of one centre (same rows, same centre row) in one launch: each against the
    oracle and all bit-identical, so a race or a result read too early in the streaming pass
    would show as copies that differ."""
    copies = 2048
    x1 = W.make_features(n, c, 900 + n, dtype)
    xc1 = W.make_features(1, c, 950 + n, dtype)
    wt = W.make_weights(2, c, 990 + heads, dtype)
    ref = oracle_mod.local_atten(np.array([0, n], np.int64), xc1.astype(np.float64),
                                 x1.astype(np.float64), wt.astype(np.float64), heads)
    rp = (np.arange(copies + 1) * n).astype(np.int64)
    print(f"{dtype.__name__} c={c} H={heads} n={n} copies={copies}", flush=True)
    y = _local(rp, np.tile(xc1, (copies, 1)), np.tile(x1, (copies, 1)), wt, heads)
    err = np.abs(y.astype(np.float64) - ref).max(axis=1) / np.abs(ref).max()
    assert np.all(err < TOL[dtype]), f"{int(np.sum(err >= TOL[dtype]))} copies wrong"
    assert np.array_equal(y, np.broadcast_to(y[:1], y.shape))


def _first_layer_scores(rp, xc, x, w, heads, i):
    """Scores of centre i's rows in the first layer, [rows][heads], natural units."""
    c = x.shape[1]
    d = c // heads
    q = xc[i] @ w[0, 0]
    k = x[rp[i]:rp[i + 1]] @ w[0, 1]
    return np.stack([k[:, h * d:(h + 1) * d] @ q[h * d:(h + 1) * d] for h in range(heads)],
                    axis=1) / np.sqrt(d)


@pytest.mark.parametrize("dtype,amp", [(np.float64, 8.0), (np.float32, 4.0)])
def test_large_scores_move_the_shift(oracle_mod, dtype, amp):
    """Scores far from 0: the streaming kernel's shift starts at 0 and is raised (a later
    chunk's score more than 20 natural units, 30 base-2 units, above it) or lowered (a
    centre's first chunk with every score more than that below it) in a separate step.  The
    premise that both happen is checked on the inputs."""
    c, heads = 64 if dtype == np.float32 else 32, 4
    rp = W.random_rows(40, 200, 31, min_len=1)
    lens = np.diff(rp)
    lens[:4] = [200, 130, 65, 64]
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    e = int(rp[-1])
    x = W.make_features(e, c, 32, np.float64) * amp
    xc = W.make_features(40, c, 33, np.float64) * amp
    wt = W.make_weights(1, c, 34, np.float64)
    # centre 1: every row the same vector, far along one direction: each head's scores are
    # all equal, some heads' far below 0
    v = np.random.default_rng(35).normal(size=c)
    x[rp[1]:rp[2]] = v * (60.0 / np.linalg.norm(v)) * amp
    lead = 20.0 if dtype == np.float64 else 30.0 / np.log2(np.e)
    raised = lowered = False
    for i in range(40):
        s = _first_layer_scores(rp, xc, x, wt, heads, i)
        first = s[:64]
        lowered |= bool(np.any(first.max(axis=0) < -lead))
        if s.shape[0] > 64:
            later = s[64:]
            raised |= bool(np.any(later.max(axis=0) > np.maximum(first.max(axis=0), 0.0) + lead))
    assert raised and lowered, (raised, lowered)
    y = _local(rp, xc.astype(dtype), x.astype(dtype), wt.astype(dtype), heads)
    ref = oracle_mod.local_atten(rp, xc.astype(dtype).astype(np.float64),
                                 x.astype(dtype).astype(np.float64), wt.astype(dtype).astype(np.float64),
                                 heads)
    err = _normwise(y.astype(np.float64), ref)
    print(f"{dtype.__name__} amp={amp}: {err:.3e}", flush=True)
    assert err < TOL[dtype]


@pytest.mark.parametrize("dtype,c", [(np.float64, 32), (np.float32, 64), (np.float32, 32)])
def test_order_gather(oracle_mod, dtype, c):
    rp = W.random_rows(30, 90, 77, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, c, 78, np.float64)
    xc = W.make_features(30, c, 79, np.float64)
    wt = W.make_weights(2, c, 80, np.float64)
    perm = np.random.default_rng(81).permutation(e).astype(np.int32)
    x2 = np.empty_like(x)
    x2[perm] = x
    y = _local(rp, xc.astype(dtype), x2.astype(dtype), wt.astype(dtype), 4, order=perm)
    ref = oracle_mod.local_atten(rp, xc.astype(dtype).astype(np.float64),
                                 x.astype(dtype).astype(np.float64),
                                 wt.astype(dtype).astype(np.float64), 4)
    assert _normwise(y.astype(np.float64), ref) < TOL[dtype]


@pytest.mark.parametrize("c", [16, 64])
def test_order_out_of_range_is_reported(c):
    rp = np.array([0, 4, 8], np.int64)
    x = W.make_features(8, c, 1, np.float32)
    xc = W.make_features(2, c, 2, np.float32)
    wt = W.make_weights(1, c, 3, np.float32)
    t = lambda a: torch.from_numpy(a).to(DEV)
    order = torch.tensor([0, 1, 2, 3, 4, 5, 6, 99], dtype=torch.int32, device=DEV)
    ws = nga.Workspace(DEV)
    nga.local_attn_forward(t(rp), t(xc), t(x), t(wt), 4, order=order, ws=ws)
    assert nga.sync_status(ws) == -8


@pytest.mark.parametrize("c", [16, 64])
def test_bad_row_ptr_is_reported(c):
    rp = np.array([0, 4, 20], np.int64)  # beyond the 8 edge rows
    x = W.make_features(8, c, 1, np.float32)
    xc = W.make_features(2, c, 2, np.float32)
    wt = W.make_weights(1, c, 3, np.float32)
    t = lambda a: torch.from_numpy(a).to(DEV)
    ws = nga.Workspace(DEV)
    nga.local_attn_forward(t(rp), t(xc), t(x), t(wt), 4, ws=ws)
    assert nga.sync_status(ws) == -4
