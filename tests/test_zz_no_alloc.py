"""nl_build_static, the allocation-free variant of nl_build, against nl_build itself.

Called through the C ABI (ctypes, raw device pointers, torch's current stream).  Two calls in a
row on the library's one static scratch, the second with a smaller input (the 96,241-atom
Fe BCC workload, whose cells go through the multi-launch binning, then the 1,000-atom diamond
workload, which bins in one work-group), then a third, tiny box with many images: each must
equal nl_build's rows bit for bit.  Plus the error word in the caller's status block and the
host-side size limit.
"""
import ctypes

import numpy as np
import pytest
import torch

import neighbour_graph_attention_amd as nga
from neighbour_graph_attention_amd import _lib as L
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _static_call(lib, pos, box, rcut, sel, status):
    n = pos.shape[0]
    nbr = torch.full((n, sel), -7, dtype=torch.int32, device=DEV)
    nsh = torch.full((n, sel, 3), -7, dtype=torch.int32, device=DEV)
    nn = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    b = (ctypes.c_double * 3)(*[float(v) for v in box])
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    rc = lib.nl_build_static(ctypes.c_void_p(pos.data_ptr()), n, b, float(rcut), int(sel),
                             ctypes.c_void_p(nbr.data_ptr()), ctypes.c_void_p(nsh.data_ptr()),
                             ctypes.c_void_p(nn.data_ptr()), ctypes.c_void_p(status.data_ptr()),
                             stream)
    return rc, nbr, nsh, nn


def _status_code(lib, status):
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    return lib.nga_sync_status(ctypes.c_void_p(status.data_ptr()), stream)


def test_static_equals_nl_build_on_consecutive_calls():
    lib = L.load()
    status = torch.zeros(256, dtype=torch.uint8, device=DEV)
    cases = []
    for key in (5, 3):
        w = W.WORKLOADS[key]
        pos, box = W.workload_positions(w)
        cases.append((w.name, pos, box, w.rcut, w.sel))
    box = (3.0, 4.0, 5.0)
    cases.append(("tiny-box", W.random_positions(40, box, 77), box, 4.5, 300))
    for name, pos_np, box, rcut, sel in cases:
        need = lib.nl_build_workspace_bytes(pos_np.shape[0], (ctypes.c_double * 3)(*box), rcut)
        assert 0 < need <= L.STATIC_SCRATCH_BYTES, (name, need)
        print(f"case {name}: N={pos_np.shape[0]} scratch {need} bytes", flush=True)
        pos = torch.from_numpy(pos_np).to(DEV)
        rc, nbr, nsh, nn = _static_call(lib, pos, box, rcut, sel, status)
        assert rc == L.NGA_OK, (name, rc)
        assert _status_code(lib, status) == L.NGA_OK
        rb, rs, rn = nga.nl_build(pos, box, rcut, sel)
        torch.cuda.synchronize(DEV)
        assert torch.equal(nn, rn), name
        assert torch.equal(nbr, rb), name
        assert torch.equal(nsh, rs), name


def test_static_reports_device_errors_in_the_callers_status_block():
    lib = L.load()
    status = torch.zeros(256, dtype=torch.uint8, device=DEV)
    box = (6.0, 6.0, 6.0)
    pos_np = W.random_positions(50, box, 78)
    pos_np[7, 1] = 6.5  # outside [0, L)
    rc, _, _, _ = _static_call(lib, torch.from_numpy(pos_np).to(DEV), box, 2.5, 32, status)
    assert rc == L.NGA_OK  # found on the device, reported through the status block
    assert _status_code(lib, status) == L.NGA_EBOX
    assert _status_code(lib, status) == L.NGA_OK  # read and cleared
    # the next good call on the same scratch is unaffected
    pos_np[7, 1] = 1.0
    pos = torch.from_numpy(pos_np).to(DEV)
    rc, nbr, nsh, nn = _static_call(lib, pos, box, 2.5, 32, status)
    assert rc == L.NGA_OK and _status_code(lib, status) == L.NGA_OK
    rb, rs, rn = nga.nl_build(pos, box, 2.5, 32)
    torch.cuda.synchronize(DEV)
    assert torch.equal(nbr, rb) and torch.equal(nsh, rs) and torch.equal(nn, rn)


def test_static_refuses_more_than_its_scratch():
    lib = L.load()
    box = (ctypes.c_double * 3)(400.0, 400.0, 400.0)
    n = 2_000_000
    assert lib.nl_build_workspace_bytes(n, box, 8.0) > L.STATIC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)  # never used: the size check comes first
    assert lib.nl_build_static(fake, n, box, 8.0, 181, fake, fake, fake, fake,
                               None) == L.NGA_ETOOBIG
