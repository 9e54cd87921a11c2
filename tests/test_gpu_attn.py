"""GPU block-dense attention against the oracle, normwise.

Tolerances (max |y - y_ref| / max |y_ref| over the compared rows): 1e-12 for
fp64 and 2e-5 for fp32, where the oracle runs in fp64 on the same (fp32-
rounded) inputs.  Whole outputs on the diamond workloads and on random
ragged rows (lengths across tile boundaries, empty and one-edge rows, rows
at the cap), sampled centres carried through every layer on the Fe BCC
workloads at full size, the `order` gather/scatter, run-to-run determinism,
and the device-detected error paths.
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


def _run(row_ptr, x, w, heads, cap, order=None, ws=None, split16=False):
    ws = ws or nga.Workspace(DEV)
    y = nga.block_attn_forward(torch.from_numpy(row_ptr).to(DEV), torch.from_numpy(x).to(DEV),
                               torch.from_numpy(w).to(DEV), heads, cap,
                               order=None if order is None else torch.from_numpy(order).to(DEV),
                               ws=ws, split16=split16)
    nga.check_status(ws, "attention")
    return y.cpu().numpy()


def _gpu_workload_csr(w):
    pos, box = W.workload_positions(w)
    p = torch.from_numpy(pos).to(DEV)
    nbr, nbr_shift, nnei = nga.nl_build(p, box, w.rcut, w.sel)
    csr = nga.edge_csr(nbr, nbr_shift, nnei)
    nga.check_status(csr["ws"], "csr")
    return pos, box, csr["row_ptr"].cpu().numpy(), csr["n_edges"]


@pytest.mark.parametrize("key", [1, 2, 3])
def test_diamond_workloads_whole_output(oracle_mod, key):
    w = W.WORKLOADS[key]
    pos, box, rp, e = _gpu_workload_csr(w)
    rp_ref, _, _, _ = oracle_mod.nl_full(pos, box, w.rcut, w.sel)
    assert np.array_equal(rp, rp_ref)
    x = W.workload_features(w, e)
    wt = W.workload_weights(w)
    print(f"workload {w.name} E={e} variant={nga.attn_variant(0, w.sel, w.c, w.heads)}", flush=True)
    y = _run(rp, x, wt, w.heads, w.sel)
    ref = oracle_mod.attn_naive(rp, x, wt, w.heads)
    err = _normwise(y, ref)
    print(f"normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float64]


@pytest.mark.parametrize("key", [4, 5])
def test_fe_bcc_full_size_whole_output(oracle_mod, key):
    """The Fe BCC workloads at full size, every output row of every centre against the oracle
    (fp64 naive loops on the same fp32 inputs, through every layer), for the fp32 matrix-core
    kernel and for the f16 split-pair arithmetic.  A sampled comparison of 200 centres runs
    first as a quick pre-check."""
    w = W.WORKLOADS[key]
    pos, box, rp, e = _gpu_workload_csr(w)
    n = rp.shape[0] - 1
    rp_ref, _, _, _ = oracle_mod.nl_full(pos, box, w.rcut, w.sel)
    assert np.array_equal(rp, rp_ref)
    x = W.workload_features(w, e)
    wt = W.workload_weights(w)
    print(f"workload {w.name} N={n} E={e} variant={nga.attn_variant(1, w.sel, w.c, w.heads)}",
          flush=True)
    y = _run(rp, x, wt, w.heads, w.sel)
    y16 = _run(rp, x, wt, w.heads, w.sel, split16=True)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(y16))
    rng = np.random.default_rng(2000 + key)
    centres = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 200, replace=False)]))
    x64 = x.astype(np.float64)
    w64 = wt.astype(np.float64)
    ref_s = oracle_mod.attn_naive_centres(rp, x64, w64, w.heads, centres)
    rows = np.concatenate([np.arange(rp[i], rp[i + 1]) for i in centres])
    err_s = _normwise(y[rows].astype(np.float64), ref_s[rows])
    print(f"sampled normwise error {err_s:.3e}", flush=True)
    assert err_s < TOL[np.float32]
    del ref_s
    ref = oracle_mod.attn_naive(rp, x64, w64, w.heads)
    del x64
    err = _normwise(y.astype(np.float64), ref)
    err16 = _normwise(y16.astype(np.float64), ref)
    print(f"whole-output normwise error: fp32 {err:.3e}, f16 split pairs {err16:.3e}", flush=True)
    assert err < TOL[np.float32]
    assert err16 < TOL[np.float32]


CASES = [
    # (dtype, n_centres, max_len, c, heads, layers, seed)
    (np.float64, 40, 40, 32, 4, 2, 1),
    (np.float64, 30, 120, 128, 4, 1, 2),
    (np.float64, 50, 45, 32, 4, 3, 3),
    (np.float64, 20, 33, 24, 3, 1, 4),
    (np.float64, 10, 70, 8, 1, 2, 5),
    (np.float64, 30, 128, 64, 4, 2, 11),     # head width 16, rows up to the 128 cap
    (np.float64, 20, 150, 32, 4, 1, 12),     # rows past 128: generic path
    (np.float64, 20, 30, 20, 2, 2, 13),      # head width 10: generic path
    (np.float32, 20, 60, 40, 5, 1, 14),      # 5 heads of 8: generic path
    (np.float32, 60, 181, 64, 4, 2, 6),
    (np.float32, 40, 176, 64, 4, 1, 7),
    (np.float32, 40, 96, 32, 2, 1, 8),
    (np.float32, 25, 50, 48, 3, 2, 9),
    (np.float32, 30, 20, 16, 1, 1, 10),
    (np.float32, 20, 400, 64, 4, 2, 15),     # rows past 192: generic online-softmax path
    (np.float32, 10, 512, 16, 1, 1, 16),     # rows at the 512-neighbour cap
    (np.float64, 15, 300, 32, 4, 1, 17),     # fp64 rows past 128: generic path
    (np.float64, 40, 64, 32, 4, 6, 18),      # fused fp64: rows up to its 64 cap, six layers
    (np.float64, 30, 64, 32, 2, 2, 19),      # fused fp64, heads of 16
    (np.float64, 30, 50, 16, 1, 3, 20),      # fused fp64, one head of 16
    (np.float64, 20, 64, 8, 1, 2, 21),       # fused fp64, one head of 8
    (np.float64, 20, 65, 32, 4, 2, 22),      # rows past 64: fp64 matrix-core path
    (np.float64, 25, 64, 16, 2, 2, 25),      # fused fp64, two heads of 8 (stacked Q/K tiles)
    (np.float64, 25, 48, 32, 2, 3, 26),      # fused fp64, two heads of 16, three key tiles
    (np.float64, 25, 100, 64, 2, 2, 27),     # fp64 matrix-core path, heads of 32, rows < 128
    (np.float32, 20, 192, 64, 4, 2, 23),     # fused fp32 at its 192-row cap (12 full tiles)
    (np.float32, 20, 192, 16, 1, 1, 24),     # the same with one head
]


SPLIT16_CASES = [c for c in CASES if c[0] == np.float32 and c[3] == 16 * c[4] and c[4] in (1, 2, 4)
                 and c[2] <= 192]


@pytest.mark.parametrize("dtype,nc,maxlen,c,heads,layers,seed", SPLIT16_CASES)
def test_random_ragged_rows_split16(oracle_mod, dtype, nc, maxlen, c, heads, layers, seed):
    """The f16 split-pair arithmetic (NGA_F32_SPLIT16) on the fp32 cases its kernel covers."""
    assert nga.attn_variant(nga.NGA_F32_SPLIT16, maxlen, c, heads) == "fused_f32_split16"
    test_random_ragged_rows(oracle_mod, dtype, nc, maxlen, c, heads, layers, seed, split16=True)


@pytest.mark.parametrize("dtype,nc,maxlen,c,heads,layers,seed", CASES)
def test_random_ragged_rows(oracle_mod, dtype, nc, maxlen, c, heads, layers, seed, split16=False):
    rp = W.random_rows(nc, maxlen, seed)
    # force the edge cases: an empty row, a one-edge row, a full-cap row, tile boundaries
    lens = np.diff(rp)
    special = [0, 1, maxlen, 15, 16, 17, 31, 32, 33, 63, 64, 65]
    for k, v in enumerate(special[: nc]):
        lens[k] = min(v, maxlen)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    e = int(rp[-1])
    x = W.make_features(e, c, seed + 100, dtype)
    wt = W.make_weights(layers, c, seed + 200, dtype)
    dt = nga.NGA_F64 if dtype == np.float64 else (nga.NGA_F32_SPLIT16 if split16 else nga.NGA_F32)
    print(f"case dtype={dtype.__name__} c={c} H={heads} L={layers} E={e} "
          f"variant={nga.attn_variant(dt, maxlen, c, heads)}", flush=True)
    y = _run(rp, x, wt, heads, maxlen, split16=split16)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), heads)
    err = _normwise(y.astype(np.float64), ref)
    print(f"normwise error {err:.3e}", flush=True)
    assert err < TOL[dtype]


def _merged_core_wo(n_centres):
    """Whether the fp64 matrix-core path (c = 128, heads of 16 or 32) runs the core and the
    output projection as one work-group per centre: when ceil(n / CUs) rounds of that kernel
    beat n / CUs rounds of the per-head core and the row GEMM (18 ceil(r) <= 25 r)."""
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    rounds = -(-n_centres // cus)
    return 18 * rounds * cus <= 25 * n_centres


def test_f64_layer_plan_follows_its_rule():
    """The plan the library picks for c = 128 equals the rule, at every centre count up to
    three rounds of compute units, for heads of 32 and 16; heads of 8 and other widths always
    take the per-head core."""
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    for n in range(1, 3 * cus + 2):
        want = "mfma_f64.merged" if _merged_core_wo(n) else "mfma_f64.per_head"
        for heads in (4, 8):
            assert nga.attn_plan(nga.NGA_F64, n, 128, 128, heads) == want, (n, heads)
        assert nga.attn_plan(nga.NGA_F64, n, 128, 128, 16) == "mfma_f64.per_head"
        assert nga.attn_plan(nga.NGA_F64, n, 128, 64, 2) == "mfma_f64.per_head"
    assert nga.attn_plan(nga.NGA_F64, 1000, 40, 32, 4) == "fused_f64"
    assert nga.attn_plan(nga.NGA_F32, 1000, 181, 64, 4) == "fused_f32"


@pytest.mark.parametrize("side", [0, 1])
def test_f64_plans_either_side_of_the_switch(oracle_mod, side):
    """The smallest centre count that takes the merged kernel, and the one below it: both
    against the oracle, on short ragged rows."""
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    first = next(n for n in range(1, 2 * cus) if _merged_core_wo(n))
    nc = first - 1 + side
    assert nga.attn_plan(nga.NGA_F64, nc, 40, 128, 4) == (
        "mfma_f64.merged" if side else "mfma_f64.per_head")
    rp = W.random_rows(nc, 40, 60 + side, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, 128, 61 + side, np.float64)
    wt = W.make_weights(2, 128, 62 + side, np.float64)
    y = _run(rp, x, wt, 4, 40)
    ref = oracle_mod.attn_naive(rp, x, wt, 4)
    assert _normwise(y, ref) < TOL[np.float64]


@pytest.mark.parametrize("nc,maxlen,heads,layers,seed,with_order", [
    (220, 128, 4, 2, 40, False),   # heads of 32, rows up to the 128 cap, one round of CUs
    (220, 120, 8, 2, 41, False),   # heads of 16
    (600, 100, 4, 1, 42, False),   # more than one round
    (220, 128, 4, 2, 43, True),    # rows stored out of slot order (gather and scatter by order)
])
def test_f64_merged_core_and_projection(oracle_mod, nc, maxlen, heads, layers, seed, with_order):
    """fp64, c = 128, enough centres that each centre gets a work-group for all of its heads
    and the output projection.  Against the oracle, and bit for bit against the same centres
    run in launches of 20, which take the per-head core and the row GEMM: both sum every
    output element over the same channel groups in the same order."""
    c = 128
    assert nga.attn_variant(nga.NGA_F64, maxlen, c, heads) == "mfma_f64"
    assert _merged_core_wo(nc) and not _merged_core_wo(20)
    assert nga.attn_plan(nga.NGA_F64, nc, maxlen, c, heads) == "mfma_f64.merged"
    assert nga.attn_plan(nga.NGA_F64, 20, maxlen, c, heads) == "mfma_f64.per_head"
    rp = W.random_rows(nc, maxlen, seed)
    lens = np.diff(rp)
    for k, v in enumerate([0, 1, maxlen, 15, 16, 17, 31, 32, 33, 63, 64, 65, 112, 113]):
        lens[k] = min(v, maxlen)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    e = int(rp[-1])
    x = W.make_features(e, c, seed + 100, np.float64)
    wt = W.make_weights(layers, c, seed + 200, np.float64)
    if with_order:
        perm = np.random.default_rng(seed + 300).permutation(e).astype(np.int32)
        x2 = np.empty_like(x)
        x2[perm] = x
        y = _run(rp, x2, wt, heads, maxlen, order=perm)[perm]
    else:
        y = _run(rp, x, wt, heads, maxlen)
    ref = oracle_mod.attn_naive(rp, x, wt, heads)
    err = _normwise(y, ref)
    print(f"merged core and projection: {nc} centres, H={heads}, L={layers}, E={e}, "
          f"normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float64]
    y_small = np.empty_like(y)
    for i0 in range(0, nc, 20):
        i1 = min(nc, i0 + 20)
        a, b = int(rp[i0]), int(rp[i1])
        y_small[a:b] = _run(rp[i0:i1 + 1] - a, np.ascontiguousarray(x[a:b]), wt, heads, maxlen)
    assert np.array_equal(y, y_small)


def _per_centre_normwise(y, ref, rp):
    worst = 0.0
    for i in range(rp.shape[0] - 1):
        if rp[i + 1] > rp[i]:
            worst = max(worst, _normwise(y[rp[i]:rp[i + 1]], ref[rp[i]:rp[i + 1]]))
    return worst


COPY_CASES = (  # (dtype, c, heads, cap, n, split16, kernel path)
    [(np.float64, c, h, 64, n, False, "fused_f64") for c, h in [(32, 2), (16, 1), (16, 2), (32, 4)]
     for n in (29, 32, 45, 48, 61, 64)]
    + [(np.float64, 128, 4, 128, n, False, "mfma_f64") for n in (61, 120, 128)]
    + [(np.float64, 128, 8, 128, n, False, "mfma_f64") for n in (61, 128)]
    + [(np.float32, 64, 4, 192, n, False, "fused_f32") for n in (45, 48, 176, 181, 192)]
    + [(np.float32, 16, 1, 192, n, False, "fused_f32") for n in (29, 32, 189)]
    + [(np.float32, 64, 4, 192, n, True, "fused_f32_split16") for n in (48, 181)]
    + [(np.float32, 40, 5, 64, 61, False, "generic_f32")]
)


@pytest.mark.parametrize("dtype,c,heads,cap,n,split16,variant", COPY_CASES)
def test_every_copy_of_one_centre(oracle_mod, dtype, c, heads, cap, n, split16, variant):
    """Many copies of one centre in one launch, each against the oracle.  The rows end in a
    key group of four with at least one valid key, so the last P.V product of the last query
    tile contributes; a reader of a matrix-core result scheduled too early, or any other
    race, shows up as some copies differing from the rest (the fused fp64 kernel once got
    about 96% of such copies wrong on some GPUs)."""
    dt = nga.NGA_F32_SPLIT16 if split16 else (nga.NGA_F64 if dtype == np.float64 else nga.NGA_F32)
    assert nga.attn_variant(dt, cap, c, heads) == variant
    x1 = W.make_features(n, c, 700 + n + c, dtype)
    wt = W.make_weights(2, c, 800 + heads, dtype)
    ref = oracle_mod.attn_naive(np.array([0, n], np.int64), x1.astype(np.float64),
                                wt.astype(np.float64), heads)
    # fp64 at c = 128: 128 copies take the per-head core, 512 the merged core and projection
    for copies in ((128, 512) if variant == "mfma_f64" else (2048,)):
        if variant == "mfma_f64":
            assert nga.attn_plan(dt, copies, cap, c, heads) == (
                "mfma_f64.merged" if copies == 512 else "mfma_f64.per_head")
        rp = (np.arange(copies + 1) * n).astype(np.int64)
        print(f"{variant} c={c} H={heads} n={n} copies={copies}", flush=True)
        y = _run(rp, np.tile(x1, (copies, 1)), wt, heads, cap, split16=split16)
        err = (np.abs(y.reshape(copies, n, c).astype(np.float64) - ref[None]).max(axis=(1, 2))
               / np.abs(ref).max())
        bad = np.nonzero(err >= TOL[dtype])[0]
        assert len(bad) == 0, f"{len(bad)} copies wrong, worst {err.max():.3e}"
        # every copy is the same computation: the outputs agree bit for bit
        y3 = y.reshape(copies, n, c)
        assert np.array_equal(y3, np.broadcast_to(y3[:1], y3.shape))


@pytest.mark.parametrize("split16", [True, False])
def test_f32_split_rounding_ties(oracle_mod, split16):
    """fp32 projections on f16 matrix cores take each operand as two f16 parts (hi, lo).  Both
    parts must come from one rounded fp32 value: a head-output element at an f16 rounding tie
    otherwise gets its lo part from a differently rounded copy and lands one f16 ulp off.  The
    first block is 41 seeded rows that hold such ties; the rest are 400 blocks of 30 to 48 rows,
    over a million head-output elements."""
    rp0 = W.random_rows(20, 64, 5, min_len=1)
    x0 = W.make_features(int(rp0[-1]), 64, 6, np.float32)
    wt = W.make_weights(1, 64, 7, np.float32)
    blk = np.concatenate([x0[rp0[0]:rp0[1]], x0[100:]])[:41]
    lens = np.random.default_rng(31).integers(30, 49, 400)
    rp = np.concatenate([[0, 41], 41 + np.cumsum(lens)]).astype(np.int64)
    x = np.concatenate([blk, W.make_features(int(lens.sum()), 64, 32, np.float32)])
    y = _run(rp, x, wt, 4, 64, split16=split16)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), 4)
    err = _per_centre_normwise(y.astype(np.float64), ref, rp)
    print(f"worst per-centre normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float32]


@pytest.mark.parametrize("split16", [False, True])
@pytest.mark.parametrize("heads,layers", [(4, 2), (2, 1), (1, 3)])
def test_f32_per_centre_magnitudes(oracle_mod, heads, layers, split16):
    """Centres whose features differ in magnitude by up to 2^21 each keep fp32-class relative
    accuracy against their own scale (the f16 split is scaled per centre and layer)."""
    c = 16 * heads
    rp = W.random_rows(60, 100, 41, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, c, 42, np.float32)
    k = np.random.default_rng(43).integers(-20, 2, rp.shape[0] - 1)
    for i in range(rp.shape[0] - 1):
        x[rp[i]:rp[i + 1]] *= np.float32(2.0 ** k[i])
    wt = W.make_weights(layers, c, 44, np.float32)
    y = _run(rp, x, wt, heads, 100, split16=split16)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), heads)
    err = _per_centre_normwise(y.astype(np.float64), ref, rp)
    dt = nga.NGA_F32_SPLIT16 if split16 else nga.NGA_F32
    print(f"variant={nga.attn_variant(dt, 100, c, heads)} worst per-centre error {err:.3e}",
          flush=True)
    assert err < TOL[np.float32]


def _rowwise(y, ref):
    """Largest over rows of max |y_r - ref_r| / max |ref_r| (rows with ref_r = 0 skipped)."""
    den = np.max(np.abs(ref), axis=1)
    num = np.max(np.abs(y - ref), axis=1)
    keep = den > 0
    return float(np.max(num[keep] / den[keep]))


@pytest.mark.parametrize("split16", [False, True])
def test_f32_one_huge_key_per_centre(oracle_mod, split16):
    """Each centre's first edge row is 1e4 in channel 0 and every other row is 0 there, with
    identity weights: head 0's largest key norm is then some 1e4 times its scores against the
    other queries, so a softmax shifted by |q| max|k| would underflow those rows (the fp32
    kernel then recomputes them with the exact row max).  Every row must still match the
    oracle to the fp32 tolerance relative to its own magnitude."""
    rp = W.random_rows(30, 181, 61, min_len=2)
    e = int(rp[-1])
    x = W.make_features(e, 64, 62, np.float32)
    x[:, 0] = 0.0
    x[rp[:-1], 0] = 1.0e4
    wt = np.broadcast_to(np.eye(64, dtype=np.float32), (2, 4, 64, 64)).copy()
    y = _run(rp, x, wt, 4, 181, split16=split16)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), 4)
    assert np.all(np.isfinite(y))
    err = _rowwise(y.astype(np.float64), ref)
    print(f"split16={split16}: row-wise error {err:.3e}", flush=True)
    assert err < TOL[np.float32]


@pytest.mark.parametrize("split16", [False, True])
def test_f32_weight_magnitudes(oracle_mod, split16):
    """Weight matrices scaled far from 1 (2^-30 .. 2^30, with non-power-of-two factors) give
    the same relative accuracy; the scales are paired so that the scores keep their size."""
    rp = W.random_rows(40, 181, 51, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, 64, 52, np.float32)
    wt = W.make_weights(2, 64, 53, np.float32)
    for (l, m), s in zip([(0, 0), (0, 1), (0, 2), (0, 3), (1, 0), (1, 2), (1, 3)],
                         [2.0 ** -30 * 3, 2.0 ** 28, 2.0 ** 30, 2.0 ** -30, 0.7, 2.0 ** -12, 5.0]):
        wt[l, m] *= np.float32(s)
    y = _run(rp, x, wt, 4, 181, split16=split16)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), 4)
    err = _normwise(y.astype(np.float64), ref)
    print(f"normwise error {err:.3e}", flush=True)
    assert err < TOL[np.float32]


@pytest.mark.parametrize("dtype,c,heads,cap,split16", [
    (np.float64, 32, 4, 60, False), (np.float64, 64, 4, 100, False), (np.float32, 64, 4, 181, False),
    (np.float32, 64, 4, 181, True)])
def test_order_gather_scatter(oracle_mod, dtype, c, heads, cap, split16):
    rp = W.random_rows(30, cap, 77, min_len=1)
    e = int(rp[-1])
    x = W.make_features(e, c, 78, dtype)
    wt = W.make_weights(2, c, 79, dtype)
    perm = np.random.default_rng(80).permutation(e).astype(np.int32)  # slot s stored at perm[s]
    x2 = np.empty_like(x)
    x2[perm] = x
    y2 = _run(rp, x2, wt, heads, cap, order=perm, split16=split16)
    ref = oracle_mod.attn_naive(rp, x.astype(np.float64), wt.astype(np.float64), heads)
    assert _normwise(y2[perm].astype(np.float64), ref) < TOL[dtype]


@pytest.mark.parametrize("dtype,c,heads,cap,split16", [
    (np.float64, 32, 4, 40, False), (np.float64, 128, 4, 110, False), (np.float32, 64, 4, 181, False),
    (np.float32, 64, 4, 181, True)])
def test_deterministic_and_cap_independent(dtype, c, heads, cap, split16):
    rp = W.random_rows(50, cap, 91)
    e = int(rp[-1])
    x = W.make_features(e, c, 92, dtype)
    wt = W.make_weights(1, c, 93, dtype)
    a = _run(rp, x, wt, heads, cap, split16=split16)
    b = _run(rp, x, wt, heads, cap, split16=split16)
    assert np.array_equal(a, b)
    bigger = cap + 10  # a larger cap within the same kernel variant changes nothing
    dt = nga.NGA_F64 if dtype == np.float64 else (nga.NGA_F32_SPLIT16 if split16 else nga.NGA_F32)
    assert nga.attn_variant(dt, bigger, c, heads) == nga.attn_variant(dt, cap, c, heads)
    c2 = _run(rp, x, wt, heads, bigger, split16=split16)
    assert np.array_equal(a, c2)


PATH_CASES = [  # (dtype, c, heads, kernel path)
    (np.float64, 16, 4, "generic_f64"),
    (np.float64, 16, 2, "fused_f64"),
    (np.float64, 64, 4, "mfma_f64"),
    (np.float32, 16, 1, "fused_f32"),
    (np.float32, 64, 4, "fused_f32"),
    (np.float32, 16, 1, "fused_f32_split16"),
    (np.float32, 40, 5, "generic_f32"),
]


def _path_check(dtype, c, heads, cap, variant):
    split16 = variant.endswith("split16")
    dt = nga.NGA_F64 if dtype == np.float64 else (nga.NGA_F32_SPLIT16 if split16 else nga.NGA_F32)
    assert nga.attn_variant(dt, cap, c, heads) == variant
    return split16


@pytest.mark.parametrize("dtype,c,heads,variant", PATH_CASES)
def test_rows_untouched_outside_centres(dtype, c, heads, variant):
    split16 = _path_check(dtype, c, heads, 8, variant)
    rp = np.array([0, 3, 3, 7], np.int64)
    x = W.make_features(10, c, 1, dtype)
    wt = W.make_weights(1, c, 2, dtype)
    xt = torch.from_numpy(x).to(DEV)
    y = torch.full_like(xt, 7.0)
    ws = nga.Workspace(DEV)
    nga.block_attn_forward(torch.from_numpy(rp).to(DEV), xt, torch.from_numpy(wt).to(DEV), heads,
                           8, y=y, ws=ws, split16=split16)
    nga.check_status(ws)
    assert torch.all(y[7:] == 7.0)


@pytest.mark.parametrize("dtype,c,heads,variant", PATH_CASES)
def test_row_over_cap_is_reported(dtype, c, heads, variant):
    split16 = _path_check(dtype, c, heads, 10, variant)
    rp = np.array([0, 5, 30], np.int64)
    x = W.make_features(30, c, 1, dtype)
    wt = W.make_weights(1, c, 2, dtype)
    ws = nga.Workspace(DEV)
    nga.block_attn_forward(torch.from_numpy(rp).to(DEV), torch.from_numpy(x).to(DEV),
                           torch.from_numpy(wt).to(DEV), heads, 10, ws=ws, split16=split16)
    assert nga.sync_status(ws) == -4


@pytest.mark.parametrize("dtype,c,heads,variant", PATH_CASES)
def test_decreasing_row_ptr_is_reported(dtype, c, heads, variant):
    """A row_ptr whose endpoints are valid but which decreases inside: the rows it would give
    (negative length, or starting below zero) are reported as NGA_ECAP and skipped, and the
    valid rows are still computed."""
    split16 = _path_check(dtype, c, heads, 16, variant)
    x = W.make_features(12, c, 1, dtype)
    wt = W.make_weights(1, c, 2, dtype)
    for rp in (np.array([0, 6, 3, 12], np.int64),      # centre 1 has r1 < r0
               np.array([0, -4, 5, 12], np.int64)):    # centre 1 starts below zero
        ws = nga.Workspace(DEV)
        y = torch.full((12, c), 7.0, dtype=torch.float64 if dtype == np.float64 else torch.float32,
                       device=DEV)
        nga.block_attn_forward(torch.from_numpy(rp).to(DEV), torch.from_numpy(x).to(DEV),
                               torch.from_numpy(wt).to(DEV), heads, 16, y=y, ws=ws,
                               split16=split16)
        assert nga.sync_status(ws) == -4


@pytest.mark.parametrize("dtype,c,heads,variant", PATH_CASES)
def test_order_out_of_range_is_reported(dtype, c, heads, variant):
    split16 = _path_check(dtype, c, heads, 8, variant)
    rp = np.array([0, 4, 8], np.int64)
    x = W.make_features(8, c, 1, dtype)
    wt = W.make_weights(1, c, 2, dtype)
    order = torch.tensor([0, 1, 2, 3, 4, 5, 6, 99], dtype=torch.int32, device=DEV)
    ws = nga.Workspace(DEV)
    nga.block_attn_forward(torch.from_numpy(rp).to(DEV), torch.from_numpy(x).to(DEV),
                           torch.from_numpy(wt).to(DEV), heads, 8, order=order, ws=ws,
                           split16=split16)
    assert nga.sync_status(ws) == -8
