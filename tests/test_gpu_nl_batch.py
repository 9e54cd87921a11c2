"""Batched neighbour rows (nl_build_batch) against nl_build on each structure alone.

A mix of structures with one cutoff: diamond boxes smaller than 2 rcut (pairs through several
images), tiny random boxes, a Fe BCC lattice, an empty structure and a lone atom (its own
images only).  Every structure's rows must equal nl_build on that structure with the indices
offset by its first atom, bit for bit; the batch also runs through edge_csr as one system.
"""
import numpy as np
import pytest
import torch

import neighbour_graph_attention_amd as nga
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _structures():
    out = []
    for key in (1, 2):
        pos, box = W.workload_positions(W.WORKLOADS[key])
        out.append((pos, box))
    for k, box in enumerate([(4.0, 5.0, 6.0), (3.0, 3.0, 9.0), (7.5, 6.5, 5.5)]):
        out.append((W.random_positions(30 + 10 * k, box, 950 + k), box))
    a = 2.8665
    cells = np.array([(i, j, k) for i in range(8) for j in range(8) for k in range(8)], float)
    fe = np.concatenate([cells, cells + 0.5]) * a
    out.append((W.wrap_into_box(fe + np.random.default_rng(957).normal(0, 0.03, fe.shape),
                                (8 * a,) * 3), (8 * a,) * 3))
    out.append((np.zeros((0, 3)), (6.0, 6.0, 6.0)))
    out.append((np.array([[1.0, 1.0, 1.0]]), (3.0, 3.0, 3.0)))
    return out


@pytest.mark.parametrize("rcut,sel", [(5.0, 120), (3.2, 40)])
def test_batch_equals_per_structure(rcut, sel):
    structs = _structures()
    atom_ptr = np.concatenate([[0], np.cumsum([p.shape[0] for p, _ in structs])]).astype(np.int64)
    boxes = [b for _, b in structs]
    pos = torch.from_numpy(np.concatenate([p for p, _ in structs])).to(DEV)
    ws = nga.Workspace(DEV)
    nbr, nsh, nn = nga.nl_build_batch(pos, atom_ptr, boxes, rcut, sel, ws=ws)
    nga.check_status(ws, "nl_build_batch")
    for b, (p, box) in enumerate(structs):
        a0, a1 = int(atom_ptr[b]), int(atom_ptr[b + 1])
        if a1 == a0:
            continue
        rb, rs, rn = nga.nl_build(torch.from_numpy(p).to(DEV), box, rcut, sel)
        expect = torch.where(rb >= 0, rb + a0, rb)
        print(f"structure {b}: {a1 - a0} atoms, {int(rn.sum().item())} edges", flush=True)
        assert torch.equal(nn[a0:a1], rn)
        assert torch.equal(nbr[a0:a1], expect)
        assert torch.equal(nsh[a0:a1], rs)
    csr = nga.edge_csr(nbr, nsh, nn)
    assert csr["n_edges"] == int(nn.sum().item())


def test_batch_reports_positions_outside_their_box():
    structs = [(np.array([[1.0, 1.0, 1.0], [2.0, 2.0, 2.0]]), (3.0, 3.0, 3.0)),
               (np.array([[4.5, 1.0, 1.0]]), (4.0, 4.0, 4.0))]  # x = 4.5 >= L
    pos = torch.from_numpy(np.concatenate([p for p, _ in structs])).to(DEV)
    ws = nga.Workspace(DEV)
    nga.nl_build_batch(pos, [0, 2, 3], [b for _, b in structs], 1.5, 8, ws=ws)
    assert nga.sync_status(ws) == -2
