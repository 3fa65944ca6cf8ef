"""Sampling locations, camera anchors and offsets far outside every map, up
to the float32 limit (finite, so inside the contract): a sample with no
corner inside its map reads nothing and adds nothing, its logit still takes
part in the head's softmax, and its location or offset gradient is zero.
The operator's and SCA's forward and backward against the oracle, which
range-checks every corner in float64 before it indexes.  Every call goes
through the C ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_fp32_close, assert_sum_close, dev, host

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")

# beyond any map, past the int32 range in pixels, and up to the float32 limit
FAR = np.array([1e5, -1e5, 2.5e9, -2.5e9, 1e30, -1e30, 3.0e38, -3.0e38], np.float32)
SHAPES = ((6, 9), (3, 4))


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _far(g, a, frac):
    """a with about `frac` of its entries replaced by values from FAR."""
    a = a.copy()
    pick = g.random(a.shape) < frac
    a[pick] = g.choice(FAR, size=int(pick.sum()))
    return a


def test_msda_far_locations():
    g = np.random.default_rng(np.random.SeedSequence([960, 1]))
    B, Nq, nH, P = 2, 70, 8, 4
    ss, starts, Nv = W.level_table(SHAPES)
    L = len(SHAPES)
    value = g.normal(size=(B, Nv, nH, 32)).astype(np.float32)
    loc = _far(g, g.uniform(-0.2, 1.2, (B, Nq, nH, L, P, 2)).astype(np.float32), 0.2)
    logits = g.normal(size=(B, Nq, nH, L * P)).astype(np.float32)
    gout = g.normal(size=(B, Nq, nH * 32)).astype(np.float32)
    args = (dev(value), dev(ss), dev(starts), dev(loc), dev(logits))
    out = host(msda.msda_forward(*args)).reshape(B * Nq, -1)
    ref_args = (value, ss, starts, loc, logits)
    assert_fp32_close(out, oracle.msda(*ref_args, weights_are_logits=True), "forward")
    gv, gl, gw = (host(t) for t in msda.msda_backward(*args, dev(gout)))
    rv, rl, rw = oracle.msda_backward(*ref_args, gout, weights_are_logits=True)
    mag = oracle.msda_backward(*ref_args, np.abs(gout), weights_are_logits=True)[0]
    assert_sum_close(gv, rv, mag, "grad value")
    assert_fp32_close(gl, rl, "grad locations")
    assert_fp32_close(gw, rw, "grad weights")
    far = ~((np.abs(loc) < 10).all(-1))
    assert (gl[far] == 0).all(), "a far sample's location gradient is zero"


def test_sca_far_anchors_and_offsets():
    g = np.random.default_rng(np.random.SeedSequence([960, 2]))
    B, Ncam, Nq, nH, P, D = 2, 3, 300, 8, 4, 2
    ss, starts, Nv = W.level_table(SHAPES)
    L = len(SHAPES)
    value = g.normal(size=(B, Ncam, Nv, nH, 32)).astype(np.float32)
    mask = (g.random((Ncam, B, Nq, D)) < 0.4).astype(np.uint8)
    rho = _far(g, g.uniform(-0.1, 1.1, (Ncam, B, Nq, D, 2)).astype(np.float32), 0.15)
    off = _far(g, g.normal(0, 2.0, (B, Nq, nH, L, P, 2)).astype(np.float32), 0.15)
    logits = g.normal(size=(B, Nq, nH, L * P)).astype(np.float32)
    gout = g.normal(size=(B, Nq, nH * 32)).astype(np.float32)
    hit = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
    offs = torch.empty(B * Ncam + 1, dtype=torch.int32, device="cuda")
    pq = torch.empty(B * Ncam * Nq, dtype=torch.int32, device="cuda")
    d = {k: dev(v) for k, v in (("value", value), ("ss", ss), ("starts", starts), ("rho", rho), ("mask", mask),
                                ("off", off), ("logits", logits), ("gout", gout))}
    slots = msda.sca_forward(d["value"], d["ss"], d["starts"], d["rho"], d["mask"], d["off"], d["logits"],
                             hit_count=hit, pair_offsets=offs, pair_q=pq)
    ref_args = (value, ss, starts, rho, mask, off, logits)
    ref = oracle.sca(*ref_args)
    assert np.array_equal(host(hit), ref["hit_count"]), "hit counts"
    assert np.array_equal(host(offs), ref["pair_offsets"]), "pair offsets"
    n = int(ref["pair_offsets"][-1])
    assert np.array_equal(host(pq)[:n], ref["pair_q"]), "pair lists"
    assert_fp32_close(host(slots).reshape(B * Nq, -1), ref["slots"], "slots")
    ws = torch.empty(msda.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device="cuda")
    msda.sca_compact(d["mask"], d["rho"], ws)
    gv, go, gl = (host(t) for t in msda.sca_backward(d["value"], d["ss"], d["starts"], d["rho"], d["off"],
                                                       d["logits"], d["gout"], ws))
    rv, ro, rl = oracle.sca_backward(*ref_args, gout)
    mag = oracle.sca_backward(*ref_args, np.abs(gout))[0]
    assert_sum_close(gv, rv, mag, "grad value")
    assert_fp32_close(go, ro, "grad offsets")
    assert_fp32_close(gl, rl, "grad logits")
