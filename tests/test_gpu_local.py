"""GPU LocalAtten (one query per centre over its edges) against the oracle.

Normwise tolerances as for block attention (1e-12 fp64 / 2e-5 fp32).  The diamond workloads
whole, the 65,536-atom Fe BCC workload at full size with 300 sampled centres (the oracle runs
on the sub-CSR of those centres: a centre's output depends only on its own rows), random
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


def test_fe_bcc_65536_sampled_centres(oracle_mod):
    w = W.WORKLOADS[4]
    rp, e = _gpu_csr(w)
    n = rp.shape[0] - 1
    x = W.workload_features(w, e)
    xc = W.make_features(n, w.c, 504, np.float32)
    wt = W.workload_weights(w)
    y = _local(rp, xc, x, wt, w.heads)
    centres = np.unique(np.concatenate(
        [[0, n - 1], np.random.default_rng(5004).choice(n, 300, replace=False)]))
    lens = rp[centres + 1] - rp[centres]
    sub_rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    sub_x = np.concatenate([x[rp[i]:rp[i + 1]] for i in centres])
    ref = oracle_mod.local_atten(sub_rp, xc[centres].astype(np.float64),
                                 sub_x.astype(np.float64), wt.astype(np.float64), w.heads)
    err = _normwise(y[centres].astype(np.float64), ref)
    print(f"workload {w.name} N={n} E={e}: sampled normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float32]
    assert np.all(np.isfinite(y))


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
]


@pytest.mark.parametrize("dtype,nc,maxlen,c,heads,layers,seed", CASES)
def test_random_ragged_rows(oracle_mod, dtype, nc, maxlen, c, heads, layers, seed):
    rp = W.random_rows(nc, maxlen, seed)
    lens = np.diff(rp)
    for k, v in enumerate([0, 1, maxlen, 63, 64, 65, 128, 129]):
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


def test_order_gather(oracle_mod):
    rp = W.random_rows(30, 90, 77, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, 32, 78, np.float64)
    xc = W.make_features(30, 32, 79, np.float64)
    wt = W.make_weights(2, 32, 80, np.float64)
    perm = np.random.default_rng(81).permutation(e).astype(np.int32)
    x2 = np.empty_like(x)
    x2[perm] = x
    y = _local(rp, xc, x2, wt, 4, order=perm)
    assert _normwise(y, oracle_mod.local_atten(rp, xc, x, wt, 4)) < TOL[np.float64]


def test_order_out_of_range_is_reported():
    rp = np.array([0, 4, 8], np.int64)
    x = W.make_features(8, 16, 1, np.float32)
    xc = W.make_features(2, 16, 2, np.float32)
    wt = W.make_weights(1, 16, 3, np.float32)
    t = lambda a: torch.from_numpy(a).to(DEV)
    order = torch.tensor([0, 1, 2, 3, 4, 5, 6, 99], dtype=torch.int32, device=DEV)
    ws = nga.Workspace(DEV)
    nga.local_attn_forward(t(rp), t(xc), t(x), t(wt), 4, order=order, ws=ws)
    assert nga.sync_status(ws) == -8


def test_bad_row_ptr_is_reported():
    rp = np.array([0, 4, 20], np.int64)  # beyond the 8 edge rows
    x = W.make_features(8, 16, 1, np.float32)
    xc = W.make_features(2, 16, 2, np.float32)
    wt = W.make_weights(1, 16, 3, np.float32)
    t = lambda a: torch.from_numpy(a).to(DEV)
    ws = nga.Workspace(DEV)
    nga.local_attn_forward(t(rp), t(xc), t(x), t(wt), 4, ws=ws)
    assert nga.sync_status(ws) == -4
