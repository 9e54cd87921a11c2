"""The step captured as one HIP graph (nga_step_graph_*) against the same step run eagerly.

Three replays per case, with the positions moved in place and unrelated eager work (torch ops,
an eager step) between them; every replay's neighbour rows, CSR and attention output must equal
the eager step on the same inputs bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import neighbour_graph_attention_amd as nga
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _eager(pos, box, w, x, wt):
    nbr, nbr_shift, nnei = nga.nl_build(pos, box, w.rcut, w.sel)
    csr = nga.edge_csr(nbr, nbr_shift, nnei, e_cap=pos.shape[0] * w.sel, read_n_edges=False)
    ws = nga.Workspace(DEV)
    y = nga.block_attn_forward(csr["row_ptr"], x, wt, w.heads, w.sel, ws=ws)
    nga.check_status(ws, "attention")
    nga.check_status(csr["ws"], "csr")
    return nbr, nnei, csr, y


@pytest.mark.parametrize("key", [1, 2, 4])  # 2: the merged fp64 core and projection
def test_replays_equal_eager_steps(key):
    w = W.WORKLOADS[key]
    pos_np, box = W.workload_positions(w)
    n = pos_np.shape[0]
    e_cap = n * w.sel
    dt = np.float64 if w.dtype == "f64" else np.float32
    x = torch.from_numpy(W.make_features(e_cap, w.c, 700 + key, dt)).to(DEV)
    wt = torch.from_numpy(W.workload_weights(w)).to(DEV)
    pos = torch.from_numpy(pos_np).to(DEV)
    g = nga.StepGraph(pos, box, w.rcut, w.sel, x, wt, w.heads)
    rng = np.random.default_rng(710 + key)
    for rep in range(3):
        if rep > 0:  # move the atoms in place, then unrelated eager work
            moved = W.wrap_into_box(pos_np + rng.normal(0.0, 0.02, pos_np.shape), box)
            pos.copy_(torch.from_numpy(moved))
            pos_np = moved
            _ = (x[:1000] * 2.0).sum().item()
            _eager(pos.clone(), box, w, x, wt)
        g.replay()
        g.check()
        nbr, nnei, csr, y = _eager(pos, box, w, x, wt)
        e = int(csr["row_ptr"][-1].item())
        print(f"workload {w.name} replay {rep}: E={e}", flush=True)
        assert torch.equal(g.nnei, nnei)
        assert torch.equal(g.nbr, nbr)
        assert torch.equal(g.row_ptr, csr["row_ptr"])
        assert torch.equal(g.col[:e], csr["col"][:e])
        assert torch.equal(g.shift[:e], csr["shift"][:e])
        assert torch.equal(g.y[:e], y[:e])


def test_bad_arguments_make_no_graph():
    pos = torch.zeros((8, 3), dtype=torch.float64, device=DEV)
    x = torch.zeros((8 * 4, 16), dtype=torch.float32, device=DEV)
    wt = torch.zeros((1, 4, 16, 16), dtype=torch.float32, device=DEV)
    with pytest.raises(nga.NGAError):
        nga.StepGraph(pos, (5.0, 5.0, 5.0), -1.0, 4, x, wt, 4)  # rcut <= 0
