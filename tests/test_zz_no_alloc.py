"""sca_forward_noalloc (the SCA workspace in the library's static device
array) against sca_forward (a caller's workspace) through the C ABI, on two
calls in a row, the second smaller than the first, so that it runs on
scratch the first call left behind.  The two entry points share their
kernels: hit counts, pair lists and slots must agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")


def _outputs(w):
    B, Ncam, Nq = w["B"], w["Ncam"], w["Nq"]
    return (torch.full((B, Nq, w["nH"] * 32), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((B, Nq), -7, dtype=torch.int32, device="cuda"),
            torch.full((B * Ncam + 1,), -7, dtype=torch.int32, device="cuda"),
            torch.full((B * Ncam * Nq,), -7, dtype=torch.int32, device="cuda"))


def _inputs(w):
    return [dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "reference_points_cam", "bev_mask",
                                "sampling_offsets", "attention_logits")]


def _noalloc_through_the_c_abi(w, d, out):
    lib = msda.load_library()
    value, ss, st, rho, mask, off, lg = d
    slots, hit, offs, pq = out
    rc = lib.sca_forward_noalloc(value.data_ptr(), msda.MSDA_F32, ss.data_ptr(), st.data_ptr(), rho.data_ptr(),
                                 mask.data_ptr(), off.data_ptr(), lg.data_ptr(), w["B"], w["Ncam"], w["Nv"], w["Nq"],
                                 w["nH"], 32, w["L"], w["P"], w["D"], slots.data_ptr(), hit.data_ptr(),
                                 offs.data_ptr(), pq.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, msda.msda_last_error()


def _compare(w, what):
    announce(f"no-alloc SCA: {what}")
    d = _inputs(w)
    got = _outputs(w)
    _noalloc_through_the_c_abi(w, d, got)
    ref = _outputs(w)
    msda.sca_forward(*d, slots=ref[0], hit_count=ref[1], pair_offsets=ref[2], pair_q=ref[3])
    torch.cuda.synchronize()
    g, r = [host(t) for t in got], [host(t) for t in ref]
    n = int(r[2][-1])
    assert np.array_equal(g[1], r[1]), f"{what}: hit counts differ"
    assert np.array_equal(g[2], r[2]), f"{what}: pair offsets differ"
    assert np.array_equal(g[3][:n], r[3][:n]), f"{what}: pair lists differ"
    assert np.array_equal(g[0].view(np.uint32), r[0].view(np.uint32)), f"{what}: slots differ"
    return n


def test_noalloc_matches_sca_forward_on_two_calls_the_second_smaller():
    big = W.bevformer_sca()  # 6 cameras, 200 x 200 queries, 4 levels
    small = W.bevformer_sca(cfg=103, bev=40, shapes=((24, 40), (12, 20)))
    assert _compare(big, "BEVFormer-base SCA, 40000 queries") > 40000
    assert _compare(small, "40 x 40 queries after the full-size call") > 0


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    w = W.bevformer_sca(cfg=103, bev=40, shapes=((24, 40), (12, 20)))
    d = _inputs(w)
    slots = torch.empty((12, 40000, 256), dtype=torch.float32, device="cuda")
    lib = msda.load_library()
    value, ss, st, rho, mask, off, lg = d
    # sizes of 12 batch items of 6 cameras x 40000 queries: refused before any use of the pointers
    rc = lib.sca_forward_noalloc(value.data_ptr(), msda.MSDA_F32, ss.data_ptr(), st.data_ptr(), rho.data_ptr(),
                                 mask.data_ptr(), off.data_ptr(), lg.data_ptr(), 12, 6, w["Nv"], 40000, 8, 32,
                                 w["L"], w["P"], w["D"], slots.data_ptr(), None, None, None, None)
    assert rc == 2, "MSDA_ERR_UNSUPPORTED expected"  # MSDA_ERR_UNSUPPORTED
