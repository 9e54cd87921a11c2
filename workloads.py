"""Seeded synthetic inputs for the neighbour-graph attention workloads.

This module only makes inputs: lattice positions with jitter and vacancies,
edge features and attention weights.  It holds none of the method's
arithmetic (no distances, no neighbour selection, no attention), so both the
CPU oracle's tests and the GPU path's tests and benchmark can draw the same
inputs from it without sharing any computation.

The five workloads follow the shapes the pages measure on:

* diamond carbon at the experimental lattice constant a = 3.567 A, the
  DPA-2 / DPA-1 graph-vs-dense runs (deepmd-kit issue "NeighborGraph
  attention is 4-9x slower than dense ...", section "Measurements"):
  64, 216 and 1000 atoms, repinit nsel 120 / rcut 6 and repformer
  nsel 40 / rcut 4, g1 = 128 channels, 4 heads, fp64;
* Fe BCC at a = 2.8665 A with sel = 181 (deepmd-kit issue "DPA4 .pt2
  LAMMPS ... 3-6x slower than Python", section "Reproduction"): 65,536 and
  101,306 lattice sites.

Recipe (for workload k = 1..5):
  1. sites = (cell + basis) * a, cells in itertools.product(range(n), repeat=3)
     order (x slowest), basis inner;
  2. rng = numpy.random.default_rng(k);
  3. with vacancies: keep sort(rng.permutation(M)[:M - floor(f * M)]);
  4. pos = sites + rng.normal(0, sigma, sites.shape); pos = mod(pos, L);
     any component that rounds to L becomes 0.0, so 0 <= pos < L;
  5. features: default_rng(100 + k).standard_normal((E, c)), cast to the
     workload dtype;
  6. weights: rw = default_rng(200 + k); per layer rw.normal(0, 1/sqrt(c),
     (4, c, c)) gives (Wq, Wk, Wv, Wo) with y = x W; cast to the workload dtype.
"""
from __future__ import annotations

import itertools
import math
from dataclasses import dataclass

import numpy as np

DIAMOND_A = 3.567
BCC_FE_A = 2.8665

# Fractional basis of the conventional cubic cells.
DIAMOND_BASIS = np.array(
    [
        (0.0, 0.0, 0.0), (0.0, 0.5, 0.5), (0.5, 0.0, 0.5), (0.5, 0.5, 0.0),
        (0.25, 0.25, 0.25), (0.25, 0.75, 0.75), (0.75, 0.25, 0.75), (0.75, 0.75, 0.25),
    ]
)
BCC_BASIS = np.array([(0.0, 0.0, 0.0), (0.5, 0.5, 0.5)])
FCC_BASIS = np.array([(0.0, 0.0, 0.0), (0.0, 0.5, 0.5), (0.5, 0.0, 0.5), (0.5, 0.5, 0.0)])

LATTICES = {"diamond": DIAMOND_BASIS, "bcc": BCC_BASIS, "fcc": FCC_BASIS}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: geometry, neighbour selection and attention shape."""

    key: int
    name: str
    lattice: str
    a: float
    ncells: int
    sigma: float
    vacancy_fraction: float
    rcut: float
    sel: int
    c: int
    heads: int
    layers: int
    dtype: str  # "f64" or "f32"

    @property
    def box(self) -> tuple[float, float, float]:
        side = self.ncells * self.a
        return (side, side, side)

    @property
    def n_sites(self) -> int:
        return len(LATTICES[self.lattice]) * self.ncells ** 3

    @property
    def n_atoms(self) -> int:
        m = self.n_sites
        return m - int(math.floor(self.vacancy_fraction * m))

    @property
    def np_dtype(self):
        return np.float64 if self.dtype == "f64" else np.float32


WORKLOADS = {
    1: Workload(1, "diamond-64", "diamond", DIAMOND_A, 2, 0.05, 0.0, 6.0, 120, 128, 4, 1, "f64"),
    2: Workload(2, "diamond-216", "diamond", DIAMOND_A, 3, 0.05, 0.0, 6.0, 120, 128, 4, 2, "f64"),
    3: Workload(3, "diamond-1000", "diamond", DIAMOND_A, 5, 0.05, 0.0, 4.0, 40, 32, 4, 6, "f64"),
    4: Workload(4, "fe-bcc-65536", "bcc", BCC_FE_A, 32, 0.03, 0.0, 8.0, 181, 64, 4, 1, "f32"),
    5: Workload(5, "fe-bcc-96241-vac5", "bcc", BCC_FE_A, 37, 0.03, 0.05, 8.0, 181, 64, 4, 2, "f32"),
}


def lattice_sites(lattice: str, ncells: int, a: float) -> np.ndarray:
    """Ideal sites of an ncells^3 supercell, cells x-slowest, basis innermost."""
    basis = LATTICES[lattice]
    cells = np.array(list(itertools.product(range(ncells), repeat=3)), dtype=np.float64)
    sites = (cells[:, None, :] + basis[None, :, :]).reshape(-1, 3) * a
    return sites


def wrap_into_box(pos: np.ndarray, box) -> np.ndarray:
    """Map positions into [0, L) per axis; a component that rounds to L becomes 0."""
    box = np.asarray(box, dtype=np.float64)
    out = np.mod(pos, box)
    out = np.where(out >= box, 0.0, out)
    return np.ascontiguousarray(out, dtype=np.float64)


def make_positions(lattice: str, ncells: int, a: float, sigma: float,
                   vacancy_fraction: float, seed: int) -> tuple[np.ndarray, tuple]:
    """Jittered lattice positions (fp64, wrapped into the cubic box) and the box."""
    sites = lattice_sites(lattice, ncells, a)
    side = ncells * a
    box = (side, side, side)
    rng = np.random.default_rng(seed)
    m = sites.shape[0]
    n_remove = int(math.floor(vacancy_fraction * m))
    if n_remove > 0:
        keep = np.sort(rng.permutation(m)[: m - n_remove])
        sites = sites[keep]
    if sigma > 0.0:
        pos = sites + rng.normal(0.0, sigma, sites.shape)
    else:
        pos = sites.copy()
    return wrap_into_box(pos, box), box


def workload_positions(w: Workload) -> tuple[np.ndarray, tuple]:
    return make_positions(w.lattice, w.ncells, w.a, w.sigma, w.vacancy_fraction, w.key)


def make_features(n_edges: int, c: int, seed: int, dtype=np.float64) -> np.ndarray:
    """Edge features ~ N(0, 1), rows in CSR edge order."""
    x = np.random.default_rng(seed).standard_normal((n_edges, c))
    return np.ascontiguousarray(x.astype(dtype))


def make_weights(layers: int, c: int, seed: int, dtype=np.float64) -> np.ndarray:
    """[layers][4][c][c] weights (Wq, Wk, Wv, Wo), entries ~ N(0, 1/c) (std 1/sqrt(c))."""
    rw = np.random.default_rng(seed)
    w = np.stack([rw.normal(0.0, 1.0 / math.sqrt(c), (4, c, c)) for _ in range(layers)])
    return np.ascontiguousarray(w.astype(dtype))


def workload_features(w: Workload, n_edges: int) -> np.ndarray:
    return make_features(n_edges, w.c, 100 + w.key, w.np_dtype)


def workload_weights(w: Workload) -> np.ndarray:
    return make_weights(w.layers, w.c, 200 + w.key, w.np_dtype)


def random_rows(n_centres: int, max_len: int, seed: int, min_len: int = 0) -> np.ndarray:
    """A random destination row_ptr (int64, [n_centres + 1]) with lengths in [min_len, max_len]."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len + 1, size=n_centres)
    row_ptr = np.zeros(n_centres + 1, dtype=np.int64)
    np.cumsum(lens, out=row_ptr[1:])
    return row_ptr


def random_positions(n_atoms: int, box, seed: int) -> np.ndarray:
    """Uniform random positions in the box (a liquid-like, non-lattice input)."""
    rng = np.random.default_rng(seed)
    pos = rng.random((n_atoms, 3)) * np.asarray(box, dtype=np.float64)
    return wrap_into_box(pos, box)
