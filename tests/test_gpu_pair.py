"""GPU ragged pair-axis attention (the comparator route) against the oracle.

Same tolerances as the block-dense tests (normwise, 1e-12 fp64 / 2e-5 fp32 against the fp64
oracle).  Chunk sizes are chosen to force several chunks, including chunks that hold a
single centre.  The atomic reductions make the summation order vary from run to run, so the
checks are tolerance checks, never bitwise.
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


def _pair(row_ptr, x, w, heads, chunk, order=None):
    ws = nga.Workspace(DEV)
    y = nga.pair_attn_forward(torch.from_numpy(row_ptr).to(DEV), torch.from_numpy(x).to(DEV),
                              torch.from_numpy(w).to(DEV), heads, pair_chunk=chunk,
                              order=None if order is None else torch.from_numpy(order).to(DEV),
                              ws=ws)
    nga.check_status(ws, "pair_attn")
    return y.cpu().numpy()


def _gpu_csr(w):
    pos, box = W.workload_positions(w)
    nbr, nbr_shift, nnei = nga.nl_build(torch.from_numpy(pos).to(DEV), box, w.rcut, w.sel)
    csr = nga.edge_csr(nbr, nbr_shift, nnei)
    nga.check_status(csr["ws"], "csr")
    return csr["row_ptr"].cpu().numpy(), csr["n_edges"]


@pytest.mark.parametrize("key,chunk", [(1, 1 << 22), (2, 1 << 20), (3, 1 << 16)])
def test_diamond_workloads_whole_output(oracle_mod, key, chunk):
    w = W.WORKLOADS[key]
    rp, e = _gpu_csr(w)
    x = W.workload_features(w, e)
    wt = W.workload_weights(w)
    p = int(np.sum(np.diff(rp) ** 2))
    print(f"workload {w.name} E={e} P={p} chunks>={-(-p // chunk)}", flush=True)
    y = _pair(rp, x, wt, w.heads, chunk)
    ref = oracle_mod.attn_naive(rp, x, wt, w.heads)
    err = _normwise(y, ref)
    print(f"normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float64]


@pytest.mark.parametrize("dtype,nc,maxlen,c,heads,layers,seed", [
    (np.float64, 40, 40, 32, 4, 2, 1),
    (np.float64, 20, 70, 24, 3, 1, 2),
    (np.float32, 50, 181, 64, 4, 2, 3),
    (np.float32, 30, 33, 40, 5, 1, 4),
])
def test_random_ragged_rows(oracle_mod, dtype, nc, maxlen, c, heads, layers, seed):
    rp = W.random_rows(nc, maxlen, seed)
    lens = np.diff(rp)
    for k, v in enumerate([0, 1, maxlen, 16, 17]):
        lens[k] = v
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    e = int(rp[-1])
    x = W.make_features(e, c, seed + 100, dtype)
    wt = W.make_weights(layers, c, seed + 200, dtype)
    chunk = maxlen * maxlen  # the largest row fills a chunk on its own
    y = _pair(rp, x, wt, heads, chunk)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), heads)
    assert _normwise(y.astype(np.float64), ref) < TOL[dtype]


def test_fe_bcc_65536_against_oracle_and_block_dense(oracle_mod):
    w = W.WORKLOADS[4]
    rp, e = _gpu_csr(w)
    n = rp.shape[0] - 1
    x = W.workload_features(w, e)
    wt = W.workload_weights(w)
    p = int(np.sum(np.diff(rp) ** 2))
    print(f"workload {w.name} E={e} P={p}", flush=True)
    yp = _pair(rp, x, wt, w.heads, 1 << 26)
    ws = nga.Workspace(DEV)
    yb = nga.block_attn_forward(torch.from_numpy(rp).to(DEV), torch.from_numpy(x).to(DEV),
                                torch.from_numpy(wt).to(DEV), w.heads, w.sel, ws=ws)
    nga.check_status(ws)
    yb = yb.cpu().numpy()
    centres = np.unique(np.concatenate(
        [[0, n - 1], np.random.default_rng(4004).choice(n, 100, replace=False)]))
    ref = oracle_mod.attn_naive_centres(rp, x.astype(np.float64), wt.astype(np.float64), w.heads,
                                        centres)
    rows = np.concatenate([np.arange(rp[i], rp[i + 1]) for i in centres])
    err_p = _normwise(yp[rows].astype(np.float64), ref[rows])
    err_pb = _normwise(yp.astype(np.float64), yb.astype(np.float64))
    print(f"pair vs oracle {err_p:.3e}, pair vs block-dense (whole output) {err_pb:.3e}",
          flush=True)
    assert err_p < TOL[np.float32]
    assert err_pb < 2 * TOL[np.float32]


def test_order_gather_scatter(oracle_mod):
    rp = W.random_rows(30, 60, 77, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, 32, 78, np.float64)
    wt = W.make_weights(2, 32, 79, np.float64)
    perm = np.random.default_rng(80).permutation(e).astype(np.int32)
    x2 = np.empty_like(x)
    x2[perm] = x
    y2 = _pair(rp, x2, wt, 4, 3600, order=perm)
    ref = oracle_mod.attn_naive(rp, x, wt, 4)
    assert _normwise(y2[perm], ref) < TOL[np.float64]


def test_chunk_smaller_than_a_row_is_rejected():
    rp = np.array([0, 5, 30], np.int64)
    x = W.make_features(30, 16, 1, np.float32)
    wt = W.make_weights(1, 16, 2, np.float32)
    with pytest.raises(nga.NGAError):
        _pair(rp, x, wt, 4, 24 * 24)  # the second row has 25^2 pairs


def test_order_out_of_range_is_reported():
    rp = np.array([0, 4, 8], np.int64)
    x = W.make_features(8, 16, 1, np.float32)
    wt = W.make_weights(1, 16, 2, np.float32)
    order = torch.tensor([0, 1, 2, 3, 4, 5, 6, 99], dtype=torch.int32, device=DEV)
    ws = nga.Workspace(DEV)
    nga.pair_attn_forward(torch.from_numpy(rp).to(DEV), torch.from_numpy(x).to(DEV),
                          torch.from_numpy(wt).to(DEV), 4, order=order, pair_chunk=64, ws=ws)
    assert nga.sync_status(ws) == -8
