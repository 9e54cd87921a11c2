"""Pins of the CPU oracle's neighbour list against facts fixed outside it.

The oracle (brute force over atoms and periodic images) defines the CSR the
GPU must reproduce bit-exactly, so it is pinned here to: a value the pages
print (the 5.14 GiB pair-axis allocation at 216 diamond atoms), the
coordination shells of ideal lattices (derived below by integer
enumeration), lattice-point counts for a one-atom box, hand cases, and
invariants (symmetry of the untruncated relation, translation, relabelling,
truncation as a prefix of the sorted row).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _shells_by_enumeration(kind, mmax):
    """Squared lengths (integer units) and multiplicities of lattice vectors."""
    out = {}
    R = int(math.isqrt(mmax)) + 2
    for v in itertools.product(range(-R, R + 1), repeat=3):
        m = v[0] ** 2 + v[1] ** 2 + v[2] ** 2
        if m == 0 or m > mmax:
            continue
        if kind == "diamond":  # units of a/4: fcc sites (even, sum = 0 mod 4) + basis (odd, sum = 3 mod 4)
            ok = (all(t % 2 == 0 for t in v) and sum(v) % 4 == 0) or (
                all(t % 2 != 0 for t in v) and sum(v) % 4 == 3)
        else:  # bcc, units of a/2: all even or all odd
            ok = all(t % 2 == 0 for t in v) or all(t % 2 != 0 for t in v)
        if ok:
            out[m] = out.get(m, 0) + 1
    return out


def test_golden_shells_match_enumeration():
    doc = json.load(open(os.path.join(GOLDEN, "lattice_shells.json")))
    for kind, mmax in (("diamond", 48), ("bcc", 32)):
        enum = _shells_by_enumeration(kind, mmax)
        gold = {m: k for m, k in doc[kind]["shells_m_count"]}
        assert enum == gold
    # textbook first shells: diamond 4 nearest, bcc 8 nearest + 6 second
    assert doc["diamond"]["shells_m_count"][0] == [3, 4]
    assert doc["bcc"]["shells_m_count"][:2] == [[3, 8], [4, 6]]


def _cumulative(kind, rcut, a):
    unit = a / 4.0 if kind == "diamond" else a / 2.0
    doc = json.load(open(os.path.join(GOLDEN, "lattice_shells.json")))
    return sum(k for m, k in doc[kind]["shells_m_count"] if math.sqrt(m) * unit < rcut)


@pytest.mark.parametrize(
    "kind,ncells,a,rcut",
    [
        ("diamond", 2, W.DIAMOND_A, 6.0),   # rcut > L/2: several images of one atom
        ("diamond", 2, W.DIAMOND_A, 4.0),
        ("diamond", 3, W.DIAMOND_A, 2.0),
        ("diamond", 3, W.DIAMOND_A, 5.5),
        ("bcc", 3, W.BCC_FE_A, 8.0),        # box 8.6 A < 2 rcut
        ("bcc", 4, W.BCC_FE_A, 3.0),
        ("bcc", 5, W.BCC_FE_A, 6.0),
    ],
)
def test_ideal_lattice_coordination(oracle_mod, kind, ncells, a, rcut):
    pos, box = W.make_positions(kind, ncells, a, 0.0, 0.0, seed=0)
    expect = _cumulative(kind, rcut, a)
    row_ptr, col, shift, vec = oracle_mod.nl_full(pos, box, rcut, sel=1000)
    counts = np.diff(row_ptr)
    assert np.all(counts == expect), (expect, np.unique(counts))


def test_pair_axis_allocation_printed_on_page(oracle_mod):
    """216 diamond atoms, rcut 6: P x 128 x 8 B must print as 5.14 GiB."""
    g = json.load(open(os.path.join(GOLDEN, "pair_axis_allocation_216_diamond.json")))
    pos, box = W.make_positions(g["lattice"], g["ncells"], g["a"], 0.0, 0.0, seed=0)
    assert pos.shape[0] == 216
    row_ptr, col, shift, vec = oracle_mod.nl_full(pos, box, g["rcut"], sel=1000)
    nnei = np.diff(row_ptr)
    P = int(np.sum(nnei.astype(np.int64) ** 2))
    gib = P * g["channels"] * g["bytes_per_value"] / 2 ** 30
    assert round(gib, g["allocation_gib_printed_digits"]) == g["allocation_gib"]
    assert abs(P / 1e6 - g["pairs_approx_millions"]) < 0.15
    assert np.all(nnei == 158)


@pytest.mark.parametrize("side,rcut", [(1.0, 2.5), (3.0, 3.5), (2.0, 4.1)])
def test_single_atom_lattice_points(oracle_mod, side, rcut):
    """One atom in a cube of side L: the neighbours are its own images n*L, 0 < |n| L < rcut."""
    pos = np.array([[0.3 * side, 0.5 * side, 0.7 * side]])
    box = (side, side, side)
    R = int(rcut / side) + 1
    expect = sum(1 for n in itertools.product(range(-R, R + 1), repeat=3)
                 if 0 < (n[0] ** 2 + n[1] ** 2 + n[2] ** 2) * side * side < rcut * rcut)
    col, shift, vec, r2, nw = oracle_mod.nl_row(pos, box, rcut, 10000, 0)
    assert nw == expect == len(col)
    assert np.all(col == 0)
    # the vectors are exactly the image translations
    assert np.array_equal(vec, shift.astype(np.float64) * side)


def test_self_image_order(oracle_mod):
    """1 atom, L = 3, rcut 3.5: six images at distance 3, ordered by shift (ties by index then n)."""
    pos = np.array([[1.5, 1.5, 1.5]])
    col, shift, vec, r2, nw = oracle_mod.nl_row(pos, (3.0, 3.0, 3.0), 3.5, 10, 0)
    assert nw == 6
    assert shift.tolist() == [[-1, 0, 0], [0, -1, 0], [0, 0, -1], [0, 0, 1], [0, 1, 0], [1, 0, 0]]
    assert np.all(r2 == 9.0)


def test_two_atom_hand_case(oracle_mod):
    """L = 10, rcut 4, atoms at x = 1 and x = 8: one neighbour each, through the x image."""
    pos = np.array([[1.0, 1.0, 1.0], [8.0, 1.0, 1.0]])
    row_ptr, col, shift, vec = oracle_mod.nl_full(pos, (10.0, 10.0, 10.0), 4.0, sel=8)
    assert row_ptr.tolist() == [0, 1, 2]
    assert col.tolist() == [1, 0]
    assert shift.tolist() == [[-1, 0, 0], [1, 0, 0]]
    assert vec.tolist() == [[-3.0, 0.0, 0.0], [3.0, 0.0, 0.0]]


def test_cutoff_is_strict(oracle_mod):
    """A neighbour at exactly rcut (exact in binary) is excluded."""
    pos = np.array([[1.0, 1.0, 1.0], [3.0, 1.0, 1.0]])
    row_ptr, col, _, _ = oracle_mod.nl_full(pos, (10.0, 10.0, 10.0), 2.0, sel=8)
    assert row_ptr.tolist() == [0, 0, 0]
    row_ptr, col, _, _ = oracle_mod.nl_full(pos, (10.0, 10.0, 10.0), 2.0000001, sel=8)
    assert row_ptr.tolist() == [0, 1, 2]


def _edges(row_ptr, col, shift):
    out = set()
    for i in range(len(row_ptr) - 1):
        for e in range(row_ptr[i], row_ptr[i + 1]):
            out.add((i, int(col[e]), tuple(int(s) for s in shift[e])))
    return out


@pytest.mark.parametrize("n,side,rcut,seed", [(24, 5.0, 6.0, 1), (60, 9.0, 3.2, 2), (7, 2.0, 3.0, 3)])
def test_untruncated_relation_is_symmetric(oracle_mod, n, side, rcut, seed):
    """(i -> j, n) within rcut iff (j -> i, -n); exact in fp64 since d(j,i,-n) = -d(i,j,n)."""
    pos = W.random_positions(n, (side, side, side), seed)
    row_ptr, col, shift, vec = oracle_mod.nl_full(pos, (side, side, side), rcut, sel=100000)
    ed = _edges(row_ptr, col, shift)
    assert len(ed) == row_ptr[-1]
    for (i, j, s) in ed:
        assert (j, i, (-s[0], -s[1], -s[2])) in ed
    # edge vectors are neighbour image minus centre
    for i in range(n):
        for e in range(row_ptr[i], row_ptr[i + 1]):
            j = col[e]
            d = (pos[j] - pos[i]) + shift[e] * side
            assert np.array_equal(d, vec[e])


@pytest.mark.parametrize("key", [1, 3])
def test_rows_sorted_and_truncation_is_prefix(oracle_mod, key):
    """Rows ascend by (r2, j, n); the sel row is the first sel entries of the full row."""
    w = W.WORKLOADS[key]
    pos, box = W.workload_positions(w)
    for i in range(0, pos.shape[0], max(1, pos.shape[0] // 17)):
        c_full, s_full, v_full, r2_full, nw = oracle_mod.nl_row(pos, box, w.rcut, 100000, i)
        assert len(c_full) == nw
        keys = [(r2_full[k], int(c_full[k]), tuple(s_full[k])) for k in range(nw)]
        assert all(keys[k] < keys[k + 1] for k in range(nw - 1))
        c, s, v, r2, _ = oracle_mod.nl_row(pos, box, w.rcut, w.sel, i)
        m = min(w.sel, nw)
        assert np.array_equal(c, c_full[:m]) and np.array_equal(s, s_full[:m])
        assert np.all(r2 < w.rcut * w.rcut)


def test_ideal_diamond_tie_break_by_index(oracle_mod):
    """sel = 120 cuts the 24-site shell at sqrt(35) a/4: the kept members are its smallest (j, n)."""
    pos, box = W.make_positions("diamond", 3, W.DIAMOND_A, 0.0, 0.0, seed=0)
    for i in (0, 5, 100, 215):
        c_full, s_full, _, r2_full, nw = oracle_mod.nl_row(pos, box, 6.0, 1000, i)
        c, s, _, r2, _ = oracle_mod.nl_row(pos, box, 6.0, 120, i)
        assert nw == 158 and len(c) == 120
        # shell radii from the golden shells: first 8 shells hold 98 sites
        assert _cumulative("diamond", 5.2, W.DIAMOND_A) == 98
        r = np.sqrt(r2_full)
        shell9 = [(int(c_full[k]), tuple(s_full[k])) for k in range(nw) if 5.2 < r[k] < 5.4]
        assert len(shell9) == 24
        kept9 = [(int(c[k]), tuple(s[k])) for k in range(98, 120)]
        # On the ideal lattice the whole 24-site shell has one fp64 r2 (exact tie), so the
        # order inside it is decided by the index alone: the kept 22 are the 22 smallest (j, n).
        assert len(set(r2_full[98:122].tolist())) == 1
        assert set(r2[98:120].tolist()) == set(r2_full[98:122].tolist())
        assert kept9 == sorted(shell9)[:22]


@pytest.mark.parametrize("key", [1, 3])
def test_capped_workloads_fill_every_row(oracle_mod, key):
    """Workloads whose within-rcut counts exceed sel give E = N * sel."""
    w = W.WORKLOADS[key]
    pos, box = W.workload_positions(w)
    row_ptr, col, shift, vec = oracle_mod.nl_full(pos, box, w.rcut, w.sel)
    assert row_ptr[-1] == pos.shape[0] * w.sel


def test_translation_invariance(oracle_mod):
    w = W.WORKLOADS[3]
    pos, box = W.workload_positions(w)
    L = np.asarray(box)
    t = np.array([3.3, -7.1, 11.9])
    raw = pos + t
    wrapped = W.wrap_into_box(raw, box)
    wrap = np.rint((raw - wrapped) / L).astype(np.int64)  # raw = wrapped + wrap * L
    for i in (0, 17, 400, 999):
        c0, s0, v0, r0, n0 = oracle_mod.nl_row(pos, box, w.rcut, w.sel, i)
        c1, s1, v1, r1, n1 = oracle_mod.nl_row(wrapped, box, w.rcut, w.sel, i)
        assert n0 == n1
        assert np.array_equal(c0, c1)
        assert np.allclose(v0, v1, atol=1e-12, rtol=0)
        # x_j + n L - x_i is unchanged: n' = n + wrap_j - wrap_i
        assert np.array_equal(s1, s0 + wrap[c0] - wrap[i])


def test_relabelling_equivariance(oracle_mod):
    w = W.WORKLOADS[1]
    pos, box = W.workload_positions(w)
    perm = np.random.default_rng(7).permutation(pos.shape[0])  # new label of atom i is perm[i]
    pos2 = np.empty_like(pos)
    pos2[perm] = pos
    rp1, c1, s1, v1 = oracle_mod.nl_full(pos, box, w.rcut, 1000)
    rp2, c2, s2, v2 = oracle_mod.nl_full(pos2, box, w.rcut, 1000)
    for i in range(pos.shape[0]):
        a = slice(rp1[i], rp1[i + 1])
        b = slice(rp2[perm[i]], rp2[perm[i] + 1])
        assert np.array_equal(perm[c1[a]], c2[b])
        assert np.array_equal(s1[a], s2[b])
        assert np.array_equal(v1[a], v2[b])


@pytest.mark.parametrize("case", ["diamond-64", "diamond-1000", "tiny-box"])
def test_nl_rows_equal_rows_of_nl_full(oracle_mod, case):
    """nl_rows over a list of centres gives, bit for bit, those centres' rows of nl_full,
    concatenated in list order (the first and last centre included, duplicates and an
    unsorted list allowed), with the row lengths as its row_ptr."""
    if case == "tiny-box":
        # 30 atoms in a box smaller than rcut on every axis: several images of every atom
        rng = np.random.default_rng(31)
        box = (2.5, 3.0, 3.5)
        pos = rng.uniform(0.0, 1.0, (30, 3)) * np.asarray(box)
        rcut, sel = 4.0, 150
    else:
        w = W.WORKLOADS[1 if case == "diamond-64" else 3]
        pos, box = W.workload_positions(w)
        rcut, sel = w.rcut, w.sel
    n = pos.shape[0]
    rp, col, shift, vec = oracle_mod.nl_full(pos, box, rcut, sel)
    rng = np.random.default_rng(32)
    centres = np.concatenate([[n - 1, 0], rng.choice(n, min(n, 25), replace=False), [0]])
    srp, scol, sshift, svec = oracle_mod.nl_rows(pos, box, rcut, sel, centres)
    assert srp.shape == (len(centres) + 1,) and srp[0] == 0
    for t, i in enumerate(centres):
        a, b = slice(srp[t], srp[t + 1]), slice(rp[i], rp[i + 1])
        assert srp[t + 1] - srp[t] == rp[i + 1] - rp[i]
        assert np.array_equal(scol[a], col[b])
        assert np.array_equal(sshift[a], shift[b])
        assert np.array_equal(svec[a], vec[b])
    assert srp[-1] == len(scol) == len(sshift) == len(svec)
    if case == "tiny-box":
        assert np.any(np.abs(shift) >= 2)  # images beyond the neighbouring cells occur
    # an empty list gives an empty CSR
    erp, ecol, eshift, evec = oracle_mod.nl_rows(pos, box, rcut, sel, np.zeros(0, np.int64))
    assert erp.tolist() == [0] and len(ecol) == len(eshift) == len(evec) == 0
