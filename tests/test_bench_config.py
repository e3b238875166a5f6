"""bench.py's tables agree with the workloads and the sources (no GPU):
every configuration the default run times has a generator, and every
workload's committed counter readings are keyed to files that exist."""
import os

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ALL = set(workloads.FULL) | set(workloads.TGMM_FULL) | set(workloads.QUANT_FULL)


def test_detail_workloads_have_generators():
    names = [n for n, _, _ in bench.DETAIL_WORKLOADS]
    assert set(names) <= ALL
    # with the headline's two, every configuration is in a default run
    assert set(names) | {"moe_fwd_bf16", "moe_dlhs_bf16"} == ALL


def test_every_workload_has_its_kernel_sources():
    assert set(bench.KERNEL_SOURCES) == ALL
    for files in list(bench.KERNEL_SOURCES.values()) + [bench.KERNEL_SOURCES_COMMON]:
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "moe_grouped_matrix_amd", "csrc", f)), f


def test_memory_bound_and_evicted_sets_name_workloads():
    assert bench.MEM_BOUND <= ALL and bench.EVICT <= ALL
