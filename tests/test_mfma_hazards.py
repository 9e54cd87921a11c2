"""Matrix-core result hazards in the library's device code (CPU only: hipcc -S, no GPU).

The fused fp64 attention kernel once read the last P.V product's result through a branch
that skipped a masked region, 12 wait states after the product instead of the 19 the
compiler enforces along straight code; on some GPUs every copy of a centre whose last key
group was valid came out wrong.  This test compiles every source that issues MFMAs with the
library's own flags and checks, over all branch paths, that no MFMA result is read sooner
than the compiler's own straight-line wait for that MFMA.  The synthetic listings pin the
scanner itself: it must flag exactly that shape and pass its fixed form.
"""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import hazard_scan as hs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "neighbour_graph_attention_amd", "csrc")

_SKIPPED_READER = """\
k:
\tv_mfma_f64_16x16x4_f64 v[18:25], v[16:17], v[38:39], v[18:25]
\ts_and_saveexec_b64 s[56:57], s[44:45]
\ts_cbranch_execz .LBB0_2
{masked}
.LBB0_2:
\ts_or_b64 exec, exec, s[56:57]
\tv_mul_f64 v[10:11], v[24:25], v[2:3]
\ts_endpgm
.Lfunc_end0:
"""


def test_scanner_flags_a_reader_reached_through_a_skip_branch():
    body = "\n".join(["\tv_readlane_b32 s60, v209, 47"] * 30)
    s = hs.summarise([_SKIPPED_READER.format(masked=body)])
    assert s[("v_mfma_f64_16x16x4_f64", "vector or memory")] == [33, 3]


def test_scanner_accepts_the_settled_form():
    # the product's result is multiplied before the branch, after the wait; the reader
    # behind the branch then reads the multiply's result
    text = _SKIPPED_READER.format(masked="\tv_readlane_b32 s60, v209, 47").replace(
        "\ts_and_saveexec_b64", "\ts_nop 15\n\ts_nop 1\n\tv_mul_f64 v[24:25], v[24:25], s[0:1]\n"
        "\ts_and_saveexec_b64")
    s = hs.summarise([text])
    assert s[("v_mfma_f64_16x16x4_f64", "vector or memory")] == [18, None]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc is not installed")
def test_no_mfma_result_is_read_early_through_a_branch():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "nga_build", os.path.join(ROOT, "neighbour_graph_attention_amd", "_build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    flags = [f for f in build.HIPCC_FLAGS if f != "-fPIC"]

    def issues_mfma(path):
        text = open(path).read()
        return "mfma" in text or "gemm_rows.h" in text

    sources = [s for s in build.sources() if issues_mfma(s)]
    assert any(s.endswith("block_attn_f64_fused.hip") for s in sources)
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            out = os.path.join(tmp, os.path.basename(src) + ".s")
            subprocess.run([_hipcc(), *flags, "--cuda-device-only", "-S", src, "-o", out],
                           check=True, capture_output=True)
            return open(out).read()
        with ThreadPoolExecutor(max_workers=4) as pool:
            texts = list(pool.map(compile_one, sources))
    summary = hs.summarise(texts)
    for (opc, kind), (straight, branched) in sorted(summary.items()):
        print(f"{opc:28s} {kind:17s} along the layout {straight}, through a branch {branched}")
    assert ("v_mfma_f64_16x16x4_f64", "vector or memory") in summary
    need = {}
    for (opc, kind), (straight, _) in summary.items():
        if kind == "vector or memory" and straight is not None:
            need[opc] = straight
    for (opc, kind), (straight, branched) in summary.items():
        if branched is None:
            continue
        floor = need.get(opc) if kind == "vector or memory" else straight
        if floor is not None:
            assert branched >= floor, (opc, kind, straight, branched)
