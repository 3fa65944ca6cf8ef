"""The bounds-checked build (libmsda_checked.so, MSDA_CHECKED) on the GPU.

Every test of this module runs with the binding switched to the checked
library.  Parity cases from the other GPU test modules are collected here a
second time, so they run through the checked kernels and must still match
the oracle; after each of them every check counter must read zero: no
compaction write left its run or segment, no work-list, plan or pair-list
entry read lay outside its range, and no gather (forward or backward)
staged a corner row outside its sample's level and head.  A positive control plants out-of-range plan
entries (which the operator documents as skipped) and sees them counted.
"""
import numpy as np
import pytest
import torch

import scale_deformable_attention_forward_amd as msda
from gpu_util import announce, dev

from test_gpu_backward import (test_bevformer_sca_backward_atomic, test_bevformer_sca_backward_bf16_value,  # noqa: F401
                               test_bevformer_sca_backward_full, test_detr_encoder_msda_backward_full,
                               test_msda_backward_edge_cases, test_msda_backward_overlapping_levels,
                               test_sca_backward_edge_cases, test_temporal_frames_backward_full)
from test_gpu_pairs import (test_bevformer_sca_bf16_layer_in_pairs, test_operator_pairs_edge_cases,  # noqa: F401
                            test_sca_pairs_edge_cases, test_sca_pairs_stage_path_and_noalloc,
                            test_temporal_frames_in_pairs)
from test_gpu_parity import (test_bevformer_sca_full, test_detr_encoder_msda_full, test_msda_edge_cases,  # noqa: F401
                             test_msda_inconsistent_level_table_reads_zero_outside,
                             test_msda_locations_on_borders_and_far_outside, test_sca_edge_cases,
                             test_sca_stages_and_compaction_reuse, test_temporal_frames_full,
                             test_tiny_msda_bf16_value, test_tiny_msda_fp32_logits_and_probabilities)
from test_gpu_plan import test_frames_staging_paths, test_plan_from_reference_points  # noqa: F401
from test_gpu_random import test_random_sca_many_tiles_and_cameras  # noqa: F401
from test_gpu_rebatch import test_rebatch_bevformer_sca_full, test_rebatch_edge_cases  # noqa: F401

pytestmark = pytest.mark.gpu

_ZERO = {k: 0 for k in msda.CHECK_KIND_NAMES}


@pytest.fixture(scope="module", autouse=True)
def _checked_library():
    before = msda.use_library(msda.checked_library_path())
    lib = msda.load_library()
    assert lib._name == msda.checked_library_path()
    yield
    msda.use_library(None if before == msda.library_path() else before)


@pytest.fixture(autouse=True)
def _no_violations(request):
    announce(f"checked build: {request.node.nodeid}")
    msda.msda_check_counts(reset=True)
    yield
    if request.node.name.startswith("test_control_"):
        return
    got = msda.msda_check_counts(reset=True)
    assert got == _ZERO, f"bounds checks failed in {request.node.name}: {got}"


def test_control_planted_plan_entries_are_counted():
    """A plan whose order holds entries outside [0, B*Nq) and entries naming
    another batch item's queries: the operator skips (or still computes)
    them as documented, and the checked kernels count each kind of entry
    as a list-entry violation, nothing else."""
    rng = np.random.default_rng(5)
    B, Nq, nH, P = 2, 3000, 8, 4
    shapes = np.array([[40, 60], [20, 30]], dtype=np.int64)
    starts = np.array([0, 2400], dtype=np.int64)
    Nv = 3000
    L = len(shapes)
    value = dev(rng.standard_normal((B, Nv, nH, 32)).astype(np.float32))
    loc = dev(rng.uniform(-0.1, 1.1, (B, Nq, nH, L, P, 2)).astype(np.float32))
    logits = dev(rng.standard_normal((B, Nq, nH, L * P)).astype(np.float32))
    ref = dev(rng.uniform(0, 1, (B, Nq, 2)).astype(np.float32))
    sh, st = dev(shapes), dev(starts)
    plan = msda.msda_plan(ref, B, Nq, Nq * 2, 2)
    out = torch.zeros((B, Nq, nH * 32), dtype=torch.float32, device="cuda")
    msda.msda_gather(value, sh, st, loc, logits, plan, out=out)
    assert msda.msda_check_counts(reset=True) == _ZERO, "an untouched plan must pass every check"
    order = msda.plan_order(plan, B, Nq)
    order[5] = -1                  # outside [0, B*Nq): skipped
    order[17] = B * Nq + 9         # outside [0, B*Nq): skipped
    order[Nq + 3] = 11             # batch item 0's query in item 1's entries
    torch.cuda.synchronize()
    msda.msda_gather(value, sh, st, loc, logits, plan, out=out)
    got = msda.msda_check_counts(reset=True)
    assert got["list_entry"] > 0, got
    assert {k: v for k, v in got.items() if k != "list_entry"} == {k: 0 for k in _ZERO if k != "list_entry"}, got
