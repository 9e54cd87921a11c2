"""Neighbour-list reuse across steps (nl_refine, nl_max_displacement) against nl_build.

Candidate rows are built once with rcut + skin; the atoms then take several steps, each within
skin / 2 of the candidate-time positions and inside the box, and every refined row set must
equal nl_build's rows at the same positions bit for bit (indices, shifts, counts).  Workloads
with several images per pair (rcut + skin beyond half the box), the Fe workloads at full size,
a tiny random box; the displacement query against numpy (plain distance: a re-wrapped atom
forces a rebuild); the stale-box guard and bad indices.
"""
import numpy as np
import pytest
import torch

import neighbour_graph_attention_amd as nga
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _steps(pos0, box, skin, seed, n_steps=3):
    """Positions within skin/2 of pos0 (each atom), inside [0, L), after each of n_steps."""
    rng = np.random.default_rng(seed)
    box = np.asarray(box)
    out = []
    for k in range(n_steps):
        d = rng.normal(0.0, 0.04 * (k + 1), pos0.shape)
        norm = np.linalg.norm(d, axis=1, keepdims=True)
        d = np.where(norm > 0.49 * skin, d * (0.49 * skin / np.maximum(norm, 1e-300)), d)
        p = pos0 + d
        inside = np.all((p >= 0.0) & (p < box), axis=1, keepdims=True)
        out.append(np.where(inside, p, pos0))
    return out


def _check_case(pos0, box, rcut, sel, skin, seed):
    cand_sel = 512
    p0 = torch.from_numpy(pos0).to(DEV)
    cn, cs, cnn = nga.nl_build(p0, box, rcut + skin, cand_sel)
    assert int(cnn.max().item()) < cand_sel  # no candidate row was cut
    for k, pk in enumerate(_steps(pos0, box, skin, seed)):
        p = torch.from_numpy(pk).to(DEV)
        dmax = float(nga.nl_max_displacement(p, p0, box).item())
        assert dmax < skin / 2
        ws = nga.Workspace(DEV)
        nbr, nsh, nn = nga.nl_refine(p, box, rcut, sel, cn, cs, cnn, box, ws=ws)
        nga.check_status(ws, "nl_refine")
        rb, rs, rn = nga.nl_build(p, box, rcut, sel)
        print(f"step {k}: max displacement {dmax:.3f}, edges {int(rn.sum().item())}", flush=True)
        assert torch.equal(nn, rn)
        assert torch.equal(nbr, rb)
        assert torch.equal(nsh, rs)


@pytest.mark.parametrize("key,skin", [(2, 1.0), (3, 1.0), (4, 1.0), (5, 1.0)])
def test_refine_equals_rebuild_on_workloads(key, skin):
    w = W.WORKLOADS[key]
    pos, box = W.workload_positions(w)
    print(f"workload {w.name} rcut {w.rcut} skin {skin}", flush=True)
    _check_case(pos, box, w.rcut, w.sel, skin, 900 + key)


def test_refine_equals_rebuild_tiny_box():
    box = (4.0, 5.0, 6.0)
    pos = W.random_positions(40, box, 901)
    _check_case(pos, box, 3.5, 200, 0.6, 902)


def test_max_displacement_is_the_plain_distance():
    """No minimum image: whole-box jumps (re-wrapped atoms) count at their full length."""
    box = np.array([9.0, 10.0, 11.0])
    rng = np.random.default_rng(903)
    a = rng.uniform(0, 1, (1000, 3)) * box
    b = a + rng.normal(0, 0.3, a.shape)
    b[::7] += box * np.array([1.0, 0.0, -1.0])
    d = b - a
    ref = float(np.max(np.sqrt((d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2])))
    got = float(nga.nl_max_displacement(torch.from_numpy(b).to(DEV),
                                        torch.from_numpy(a).to(DEV), box).item())
    assert abs(got - ref) <= 1e-12 * ref
    assert got > 14.0  # a jump of (9, 0, -11) A dominates
    # a NaN position reads as an infinite displacement, never as none
    b2 = a.copy()
    b2[5, 1] = np.nan
    got2 = float(nga.nl_max_displacement(torch.from_numpy(b2).to(DEV),
                                         torch.from_numpy(a).to(DEV), box).item())
    assert got2 == np.inf


def test_rewrapped_atom_forces_a_rebuild():
    """One atom crosses the box face by a small step and is re-wrapped into [0, L): its true
    motion is tiny, but the cached shifts no longer describe its images.  The guard must read a
    displacement of about L (so the caller rebuilds), and the rebuilt rows at the wrapped
    positions must be what nl_build gives."""
    w = W.WORKLOADS[3]
    pos0, box = W.workload_positions(w)
    L = np.asarray(box)
    skin = 1.0
    i = int(np.argmin(pos0[:, 0]))  # the atom closest to the x = 0 face
    p1 = pos0.copy()
    p1[i, 0] = pos0[i, 0] - (pos0[i, 0] + 0.05)  # moves 0.05 A past the face ...
    p1 = W.wrap_into_box(p1, box)                  # ... and is re-wrapped to x ~ L - 0.05
    assert abs(p1[i, 0] - (L[0] - 0.05)) < 1e-9
    t0, t1 = torch.from_numpy(pos0).to(DEV), torch.from_numpy(p1).to(DEV)
    dmax = float(nga.nl_max_displacement(t1, t0, box).item())
    print(f"atom {i} re-wrapped: guard reads {dmax:.3f} A", flush=True)
    assert dmax > L[0] - 1.0 and not dmax < skin / 2
    # the stale candidates would lose pairs of that atom: refine differs from a rebuild
    cn, cs, cnn = nga.nl_build(t0, box, w.rcut + skin, 512)
    ws = nga.Workspace(DEV)
    stale = nga.nl_refine(t1, box, w.rcut, w.sel, cn, cs, cnn, box, ws=ws)
    nga.check_status(ws, "nl_refine")
    rb, rs, rn = nga.nl_build(t1, box, w.rcut, w.sel)
    assert not (torch.equal(stale[0], rb) and torch.equal(stale[1], rs))


def test_stale_box_and_bad_candidates():
    box = (6.0, 6.0, 6.0)
    pos = torch.from_numpy(W.random_positions(30, box, 904)).to(DEV)
    cn, cs, cnn = nga.nl_build(pos, box, 3.0, 64)
    with pytest.raises(nga.NGAError):
        nga.nl_refine(pos, box, 2.5, 32, cn, cs, cnn, (6.0, 6.0, 6.5))  # candidates of another box
    bad = cn.clone()
    bad[3, 0] = 1000  # index beyond the atoms
    ws = nga.Workspace(DEV)
    nga.nl_refine(pos, box, 2.5, 32, bad, cs, cnn, box, ws=ws)
    assert nga.sync_status(ws) == -8
