"""bench.py's roofline record carries the fields the report needs, whichever
unit bounds the kernel (host-side: the record is built from a stub timing)."""
import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_stencil_unit_by_kernel_name():
    b = _bench()
    assert b.stencil_on_matrix_cores("mta_fwd_v4 (one pass, head-split waves, fp16 matrix-core stencil)")
    assert b.stencil_on_matrix_cores("mta_fwd_v4 (four-head groups: two source-pair sweeps, head-split waves, "
                                     "fp16 matrix-core stencil)")
    assert not b.stencil_on_matrix_cores("mta_fwd_layer (fp32 VALU stencils)")
    assert not b.stencil_on_matrix_cores("mta_fwd_kernel (two passes, general)")
    assert not b.stencil_on_matrix_cores(None)


def test_roofline_record_has_traffic_and_kernel():
    src = open(os.path.join(ROOT, "bench.py")).read()
    # the roofline object gets its traffic figure and the kernel name in every branch
    assert "roof.update(traffic=traffic, kernel=kname)" in src
