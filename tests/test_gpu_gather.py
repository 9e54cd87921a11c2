"""block_gather / block_scatter against the oracle: bit-exact copies.

Random ragged rows (empty rows, one-edge rows, rows at the cap) in both dtypes and at feature
widths whose rows are 16-, 8- and 4-byte multiples, with and without `order`; the padded block
of both Fe BCC workloads at full size; scatter of the gathered block restores the edge axis;
the device-detected errors.
"""
import numpy as np
import pytest
import torch

import neighbour_graph_attention_amd as nga
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("dtype,c,cap,with_order", [
    (np.float32, 64, 181, False), (np.float32, 64, 181, True), (np.float64, 32, 120, False),
    (np.float64, 32, 120, True), (np.float32, 6, 40, False), (np.float32, 3, 17, True),
    (np.float64, 5, 33, False)])
def test_random_rows_bitexact(oracle_mod, dtype, c, cap, with_order):
    rp = W.random_rows(70, cap, 11 + c)
    lens = np.diff(rp)
    for k, v in enumerate([0, 1, cap, 15, 16, 17]):
        lens[k] = v
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    e = int(rp[-1])
    x = W.make_features(e + 5, c, 12 + c, dtype)  # 5 trailing rows belong to no centre
    order = (np.random.default_rng(13).permutation(e + 5)[:e].astype(np.int32)
             if with_order else None)
    ws = nga.Workspace(DEV)
    blk = nga.block_gather(_t(rp), _t(x), cap, order=None if order is None else _t(order), ws=ws)
    nga.check_status(ws, "block_gather")
    ref = oracle_mod.block_gather(rp, x, cap, order=order)
    got = blk.cpu().numpy()
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))
    y = torch.full_like(_t(x), 3.0)
    nga.block_scatter(_t(rp), blk, y, order=None if order is None else _t(order), ws=ws)
    nga.check_status(ws, "block_scatter")
    yref = oracle_mod.block_scatter(rp, ref, np.full_like(x, 3.0), order=order)
    assert np.array_equal(y.cpu().numpy().view(np.uint8), yref.view(np.uint8))


@pytest.mark.parametrize("key", [4, 5])
def test_fe_bcc_full_size(oracle_mod, key):
    w = W.WORKLOADS[key]
    pos, box = W.workload_positions(w)
    nbr, nsh, nn = nga.nl_build(_t(pos), box, w.rcut, w.sel)
    csr = nga.edge_csr(nbr, nsh, nn)
    nga.check_status(csr["ws"], "csr")
    e = csr["n_edges"]
    rp = csr["row_ptr"].cpu().numpy()
    x = W.workload_features(w, e)
    xt = _t(x)
    print(f"workload {w.name} N={rp.shape[0] - 1} E={e} cap={w.sel}", flush=True)
    ws = nga.Workspace(DEV)
    blk = nga.block_gather(csr["row_ptr"], xt, w.sel, ws=ws)
    nga.check_status(ws, "block_gather")
    ref = oracle_mod.block_gather(rp, x, w.sel)
    assert np.array_equal(blk.cpu().numpy(), ref)
    del ref
    y = torch.empty_like(xt)
    nga.block_scatter(csr["row_ptr"], blk, y, ws=ws)
    nga.check_status(ws, "block_scatter")
    assert torch.equal(y, xt)


def test_errors_are_reported():
    x = _t(W.make_features(12, 16, 1, np.float32))
    ws = nga.Workspace(DEV)
    nga.block_gather(_t(np.array([0, 5, 12], np.int64)), x, 6, ws=ws)  # second row is 7 > 6
    assert nga.sync_status(ws) == -4
    blk = nga.block_gather(_t(np.array([0, 6, 3, 12], np.int64)), x, 16, ws=ws)  # decreasing
    assert nga.sync_status(ws) == -4
    assert torch.all(blk[1] == 0)  # the malformed centre's block is zero-filled
    order = _t(np.array([0, 1, 2, 3, 99, 5], np.int32))
    nga.block_gather(_t(np.array([0, 6], np.int64)), x, 8, order=order, ws=ws)
    assert nga.sync_status(ws) == -8
    y = torch.zeros_like(x)
    nga.block_scatter(_t(np.array([0, 6], np.int64)), torch.ones((1, 8, 16), device=DEV), y,
                      order=order, ws=ws)
    assert nga.sync_status(ws) == -8
