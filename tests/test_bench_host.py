"""The benchmark's pricing of the path (host only): each unit's algorithmic bytes at the headline
workload (256x256 pixels, batch 2, 6 heads, B = 16, K = 8, L = 3), and every kernel a unit names
is one the library's profiler reports, so no unit silently drops out of the bench line."""
import os
import sys

from hierarchical_top_sparse_amd import _abi, profiling

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_unit_bytes_at_the_headline_workload():
    p = _abi.Problem(batch=2, heads=6, height=256, width=256, levels=3)
    units, side = bench.unit_model(p)
    T = 2 * 6 * 65536 * 64 * 2   # one bf16 token tensor
    tokens = 2 * 6 * 65536
    assert units["attn_bwd"]["bytes"] == 8 * T + 8 * tokens == 811_597_824
    assert units["attn_fwd"]["bytes"] == 4 * T + 4 * tokens == 405_798_912
    assert units["pool_select"]["bytes"] == sum(side.values()) == 360_536_064
    # per level l: the selection (n_l K int32) read, its CSC rows written, n_l + 1 offsets
    lv = [(4096, 8), (256, 8), (16, 8)]
    assert units["index_transpose"]["bytes"] == sum(12 * (2 * n * k * 4 + (n + 1) * 4)
                                                    for n, k in lv)


def test_units_name_only_profiled_kernels():
    p = _abi.Problem(batch=2, heads=6, height=256, width=256, levels=3)
    units, side = bench.unit_model(p)
    reported = {name for name, _ in profiling._KERNELS.values()} | set(
        profiling._KEY_MODES.values())
    for name, u in units.items():
        assert set(u["kernels"]) <= reported, name
    assert set(side) <= reported
    # the transposes the library launches today are priced
    assert {"csc_radix_kernel", "csc_assemble_kernel"} <= set(units["index_transpose"]["kernels"])
