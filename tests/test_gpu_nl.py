"""GPU neighbour rows and destination CSR against the oracle: bit-exact.

Whole-CSR comparisons on all five workloads (the three diamond workloads and
the two Fe BCC workloads at full size), ideal lattices with exact distance
ties, tiny boxes with many images, random orthorhombic boxes and hand cases,
plus the device-detected error paths.
"""
import numpy as np
import pytest
import torch

import neighbour_graph_attention_amd as nga
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _gpu_csr(pos_np, box, rcut, sel, want_vec=True):
    pos = torch.from_numpy(np.ascontiguousarray(pos_np, dtype=np.float64)).to(DEV)
    nbr, nbr_shift, nnei = nga.nl_build(pos, box, rcut, sel)
    csr = nga.edge_csr(nbr, nbr_shift, nnei, pos=pos, box=box, want_edge_vec=want_vec)
    nga.check_status(csr["ws"], "csr")
    plain = nga.edge_csr(nbr, nbr_shift, nnei)  # without edge vectors: same rows
    for k in ("row_ptr", "col", "shift", "dst"):
        assert torch.equal(plain[k], csr[k]), k
    out = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in csr.items()
           if k != "ws"}
    out["nbr"] = nbr.cpu().numpy()
    out["nbr_shift"] = nbr_shift.cpu().numpy()
    out["nnei"] = nnei.cpu().numpy()
    return out


def _assert_same_csr(g, ref):
    rp, col, shift, vec = ref
    assert np.array_equal(g["row_ptr"], rp)
    assert np.array_equal(g["col"], col)
    assert np.array_equal(g["shift"], shift)
    if g["edge_vec"] is not None:
        assert np.array_equal(g["edge_vec"], vec)  # bitwise: same fp64 formula, no contraction
    assert np.array_equal(g["nnei"], np.diff(rp))
    assert np.array_equal(g["dst"], np.repeat(np.arange(len(rp) - 1), np.diff(rp)))


@pytest.mark.parametrize("key", [1, 2, 3])
def test_diamond_workloads_bitexact(oracle_mod, key):
    w = W.WORKLOADS[key]
    pos, box = W.workload_positions(w)
    print(f"workload {w.name}", flush=True)
    g = _gpu_csr(pos, box, w.rcut, w.sel)
    _assert_same_csr(g, oracle_mod.nl_full(pos, box, w.rcut, w.sel))
    assert g["n_edges"] == pos.shape[0] * w.sel


@pytest.mark.parametrize("key", [4, 5])
def test_fe_bcc_full_size_whole_csr(oracle_mod, key):
    """Full-size Fe BCC lists: the whole CSR (row_ptr, col, shift, dst, edge_vec) bit-exact
    against the brute-force oracle, plus the relation's symmetry (rows are never cut here)."""
    w = W.WORKLOADS[key]
    pos, box = W.workload_positions(w)
    n = pos.shape[0]
    print(f"workload {w.name} N={n}", flush=True)
    g = _gpu_csr(pos, box, w.rcut, w.sel)
    ref = oracle_mod.nl_full(pos, box, w.rcut, w.sel)
    print(f"oracle E={ref[0][-1]}, GPU E={g['n_edges']}", flush=True)
    _assert_same_csr(g, ref)
    rp, col, shift = g["row_ptr"], g["col"], g["shift"]
    counts = np.diff(rp)
    assert counts.max() < w.sel and counts.min() >= 1
    # the untruncated relation is symmetric: (i, j, n) <-> (j, i, -n)
    same_row = np.repeat(np.arange(n), counts)
    code = lambda a, b, s: ((a * n + b) * 1000 + (s[:, 0] + 10) * 100 + (s[:, 1] + 10) * 10
                            + (s[:, 2] + 10))
    fwd = np.sort(code(same_row.astype(np.int64), col.astype(np.int64), shift.astype(np.int64)))
    bwd = np.sort(code(col.astype(np.int64), same_row.astype(np.int64), -shift.astype(np.int64)))
    assert np.array_equal(fwd, bwd)


@pytest.mark.parametrize("lattice,ncells,a,rcut,sel", [
    ("diamond", 3, W.DIAMOND_A, 6.0, 120),   # 24-way exact tie at the sel boundary
    ("diamond", 3, W.DIAMOND_A, 6.0, 200),   # untruncated: 158 each
    ("diamond", 2, W.DIAMOND_A, 6.0, 130),   # rcut > L/2: one cell per axis
    ("bcc", 4, W.BCC_FE_A, 8.0, 181),        # box 11.5 A: one cell per axis
    ("bcc", 8, W.BCC_FE_A, 8.0, 100),        # two cells per axis, truncated rows
    ("fcc", 3, 3.6, 5.0, 60),
])
def test_ideal_lattices_bitexact(oracle_mod, lattice, ncells, a, rcut, sel):
    pos, box = W.make_positions(lattice, ncells, a, 0.0, 0.0, seed=0)
    g = _gpu_csr(pos, box, rcut, sel)
    _assert_same_csr(g, oracle_mod.nl_full(pos, box, rcut, sel))


@pytest.mark.parametrize("n,box,rcut,sel,seed", [
    (300, (7.0, 11.0, 23.0), 3.5, 64, 1),
    (500, (12.0, 12.0, 12.0), 4.0, 20, 2),    # truncated rows
    (40, (3.0, 4.0, 5.0), 4.5, 300, 3),       # many images, reach 2 on x
    (1, (1.0, 1.0, 1.0), 2.5, 100, 4),        # one atom, 80 images, reach 3
    (2, (2.0, 9.0, 2.0), 3.0, 50, 5),
    (1000, (30.0, 30.0, 30.0), 2.0, 8, 6),    # sparse: many empty cells
    (700, (40.0, 10.0, 10.0), 2.6, 32, 7),
    (8192, (60.0, 60.0, 60.0), 3.7, 24, 8),   # one-work-group binning at its limits (4,096 cells)
    (8193, (60.0, 60.0, 60.0), 3.7, 24, 9),   # one atom past them: multi-launch binning
    (3000, (20.0, 20.0, 20.0), 5.0, 60, 10),  # ~47 atoms per cell: per-segment candidate rounds
    (1500, (20.0, 20.0, 20.0), 5.0, 60, 11),  # ~23 atoms per cell: rounds across segment ends
    # dense, five half-size cells per axis: ~1,100 candidates per centre, more than one
    # 1,024-position window of the per-centre stencil's run bitmap; ~390 neighbours, rows cut
    (2400, (11.8, 11.8, 11.8), 4.0, 300, 12),
])
def test_random_boxes_bitexact(oracle_mod, n, box, rcut, sel, seed):
    pos = W.random_positions(n, box, seed)
    g = _gpu_csr(pos, box, rcut, sel)
    _assert_same_csr(g, oracle_mod.nl_full(pos, box, rcut, sel))


def test_hand_cases(oracle_mod):
    g = _gpu_csr(np.array([[1.0, 1.0, 1.0], [8.0, 1.0, 1.0]]), (10.0, 10.0, 10.0), 4.0, 4)
    assert g["row_ptr"].tolist() == [0, 1, 2]
    assert g["col"].tolist() == [1, 0]
    assert g["shift"].tolist() == [[-1, 0, 0], [1, 0, 0]]
    assert g["edge_vec"].tolist() == [[-3.0, 0.0, 0.0], [3.0, 0.0, 0.0]]
    assert g["nbr"].tolist() == [[1, -1, -1, -1], [0, -1, -1, -1]]
    g = _gpu_csr(np.array([[1.5, 1.5, 1.5]]), (3.0, 3.0, 3.0), 3.5, 10)
    assert g["shift"].tolist() == [[-1, 0, 0], [0, -1, 0], [0, 0, -1], [0, 0, 1], [0, 1, 0],
                                   [1, 0, 0]]
    # strict cutoff: a neighbour at exactly rcut is excluded
    g = _gpu_csr(np.array([[1.0, 1.0, 1.0], [3.0, 1.0, 1.0]]), (10.0, 10.0, 10.0), 2.0, 4)
    assert g["row_ptr"].tolist() == [0, 0, 0]


def test_near_ties_within_one_distance_class(oracle_mod):
    """Neighbours whose r2 differ by far less than rc2 * 2^-23 (the resolution of the first
    sort pass) but are not equal, in the opposite order to their indices, plus six exact
    ties on the axes; sel cuts through the run.  The rows must follow the full key
    (r2, j, shift) exactly."""
    rng = np.random.default_rng(41)
    centre = np.array([5.0, 5.0, 5.0])
    k = 20
    dirs = rng.normal(size=(k, 3))
    dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
    radii = 2.0 + 1e-8 * np.arange(k, 0, -1)  # atom 1 farthest, atom k nearest
    shell = centre + dirs * radii[:, None]
    axes = centre + 2.0 * np.array([[1, 0, 0], [-1, 0, 0], [0, 1, 0], [0, -1, 0],
                                    [0, 0, 1], [0, 0, -1]], dtype=np.float64)
    pos = np.concatenate([centre[None], shell, axes])
    for sel in (10, 23, 40):
        g = _gpu_csr(pos, (10.0, 10.0, 10.0), 4.0, sel)
        _assert_same_csr(g, oracle_mod.nl_full(pos, (10.0, 10.0, 10.0), 4.0, sel))
    # the first row really is ordered by r2 among the near-tied shell atoms
    g = _gpu_csr(pos, (10.0, 10.0, 10.0), 4.0, 40)
    row0 = g["col"][g["row_ptr"][0]:g["row_ptr"][1]]
    shell_order = [j for j in row0 if 1 <= j <= k]
    assert shell_order == sorted(shell_order, reverse=True)


def test_empty_and_single_atom():
    pos = torch.zeros((0, 3), dtype=torch.float64, device=DEV)
    nbr, nbr_shift, nnei = nga.nl_build(pos, (5.0, 5.0, 5.0), 2.0, 4)
    csr = nga.edge_csr(nbr, nbr_shift, nnei)
    assert csr["n_edges"] == 0 and csr["row_ptr"].cpu().tolist() == [0]
    g = _gpu_csr(np.array([[1.0, 2.0, 3.0]]), (10.0, 10.0, 10.0), 2.0, 4)
    assert g["row_ptr"].tolist() == [0, 0] and g["nbr"].tolist() == [[-1, -1, -1, -1]]


def test_deterministic():
    w = W.WORKLOADS[3]
    pos, box = W.workload_positions(w)
    a = _gpu_csr(pos, box, w.rcut, w.sel)
    b = _gpu_csr(pos, box, w.rcut, w.sel)
    for k in ("row_ptr", "col", "shift", "edge_vec", "nbr", "nbr_shift"):
        assert np.array_equal(a[k], b[k])


def test_edge_mask_compaction_keeps_slot_order():
    """An external padded list with holes (-1) compacts in slot order (the edge mask)."""
    rng = np.random.default_rng(3)
    n, sel = 50, 37
    nbr = rng.integers(0, n, size=(n, sel)).astype(np.int32)
    nbr[rng.random((n, sel)) < 0.4] = -1
    nbr[7] = -1
    sh = rng.integers(-2, 3, size=(n, sel, 3)).astype(np.int32)
    csr = nga.edge_csr(torch.from_numpy(nbr).to(DEV), torch.from_numpy(sh).to(DEV), None)
    nga.check_status(csr["ws"], "mask csr")
    mask = nbr >= 0
    assert np.array_equal(csr["row_ptr"].cpu().numpy(), np.concatenate([[0], np.cumsum(mask.sum(1))]))
    assert np.array_equal(csr["col"].cpu().numpy(), nbr[mask])
    assert np.array_equal(csr["shift"].cpu().numpy(), sh[mask])
    assert np.array_equal(csr["dst"].cpu().numpy(), np.nonzero(mask)[0])


@pytest.mark.parametrize("n", [1, 8191, 8192, 8193, 40000, 65536, 65537, 100003])
@pytest.mark.parametrize("offset", [0, 1])
def test_row_counts_clamped_and_scanned(n, offset):
    """row_ptr is the running sum of nnei clamped to [0, sel], and each row keeps its first
    slots, at sizes on both sides of every scan tile and launch-shape boundary; offset 1
    hands nnei in at an address that is not 16-byte aligned."""
    rng = np.random.default_rng(n + offset)
    sel = 4
    nbr = rng.integers(0, n, size=(n, sel)).astype(np.int32)
    sh = rng.integers(-1, 2, size=(n, sel, 3)).astype(np.int32)
    nnei = rng.integers(-3, sel + 4, size=n + offset).astype(np.int32)
    buf = torch.from_numpy(nnei).to(DEV)
    print(f"n={n} offset={offset}", flush=True)
    csr = nga.edge_csr(torch.from_numpy(nbr).to(DEV), torch.from_numpy(sh).to(DEV), buf[offset:])
    nga.check_status(csr["ws"], "clamped csr")
    cnt = np.clip(nnei[offset:], 0, sel)
    assert np.array_equal(csr["row_ptr"].cpu().numpy(), np.concatenate([[0], np.cumsum(cnt)]))
    keep = np.arange(sel)[None, :] < cnt[:, None]
    assert np.array_equal(csr["col"].cpu().numpy(), nbr[keep])
    assert np.array_equal(csr["shift"].cpu().numpy(), sh[keep])


def test_edge_mask_compaction_long():
    """The masked path (no nnei) past the one-launch scan size."""
    rng = np.random.default_rng(11)
    n, sel = 70001, 5
    nbr = rng.integers(0, n, size=(n, sel)).astype(np.int32)
    nbr[rng.random((n, sel)) < 0.3] = -1
    sh = rng.integers(-1, 2, size=(n, sel, 3)).astype(np.int32)
    csr = nga.edge_csr(torch.from_numpy(nbr).to(DEV), torch.from_numpy(sh).to(DEV), None)
    nga.check_status(csr["ws"], "long mask csr")
    mask = nbr >= 0
    assert np.array_equal(csr["row_ptr"].cpu().numpy(), np.concatenate([[0], np.cumsum(mask.sum(1))]))
    assert np.array_equal(csr["col"].cpu().numpy(), nbr[mask])


def _expect_status(ws, code):
    assert nga.sync_status(ws) == code
    assert nga.sync_status(ws) == 0  # cleared by the read


@pytest.mark.parametrize("bad", [10.0, -1e-300, float("nan"), float("inf")])
def test_position_outside_box_is_reported(bad):
    pos = torch.tensor([[1.0, 1.0, 1.0], [2.0, bad, 3.0]], dtype=torch.float64, device=DEV)
    ws = nga.Workspace(DEV)
    nga.nl_build(pos, (10.0, 10.0, 10.0), 3.0, 4, ws=ws)
    _expect_status(ws, -2)


def test_row_capacity_is_reported():
    pos = W.random_positions(700, (3.0, 3.0, 3.0), 11) * 0.5 + 1.0  # 700 atoms inside 1.5 A
    ws = nga.Workspace(DEV)
    nga.nl_build(torch.from_numpy(pos).to(DEV), (20.0, 20.0, 20.0), 2.7, 16, ws=ws)
    _expect_status(ws, -3)


def test_edge_capacity_and_bad_index_are_reported():
    w = W.WORKLOADS[1]
    pos, box = W.workload_positions(w)
    p = torch.from_numpy(pos).to(DEV)
    nbr, nbr_shift, nnei = nga.nl_build(p, box, w.rcut, w.sel)
    with pytest.raises(nga.NGAError) as ex:
        nga.edge_csr(nbr, nbr_shift, nnei, e_cap=100)
    assert ex.value.code == -4
    nbr[3, 5] = 10 ** 6
    with pytest.raises(nga.NGAError) as ex:
        nga.edge_csr(nbr, nbr_shift, nnei)
    assert ex.value.code == -8
