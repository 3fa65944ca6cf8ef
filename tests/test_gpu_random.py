"""Seeded random configurations against the oracle: head counts, level
tables (including 1x1 and 1xN levels), points per level, anchors, cameras,
batch sizes, query counts, value types and mask densities drawn per case,
forward and backward (both value-gradient paths), and the forward on the
value's bf16 bits in the head-pair layout, element by element.
Every call goes through the C ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_fp32_close, assert_sum_close, dev, host
from test_gpu_pairs import pairs_host

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _draw_shape(g):
    nH = int(g.choice([1, 2, 3, 4, 8, 12, 16]))
    L = int(g.integers(1, 5))
    P = int(g.integers(1, 9))
    while L * P > 64:
        P -= 1
    shapes = tuple((int(g.integers(1, 21)), int(g.integers(1, 21))) for _ in range(L))
    return nH, L, P, shapes


def _msda_case(seed):
    g = np.random.default_rng(np.random.SeedSequence([900, seed]))
    nH, L, P, shapes = _draw_shape(g)
    B, Nq = int(g.integers(1, 4)), int(g.integers(1, 150))
    ss, starts, Nv = W.level_table(shapes)
    value = g.normal(size=(B, Nv, nH, 32)).astype(np.float32)
    if g.random() < 0.3:
        value = W.bf16_bits_trunc(value)
    loc = g.uniform(-0.3, 1.3, (B, Nq, nH, L, P, 2)).astype(np.float32)
    logits = g.random() < 0.7
    weights = (g.normal(size=(B, Nq, nH, L * P)) if logits else g.uniform(0, 1, (B, Nq, nH, L * P))).astype(np.float32)
    gout = g.normal(size=(B, Nq, nH * 32)).astype(np.float32)
    return dict(value=value, ss=ss, starts=starts, loc=loc, weights=weights, logits=logits, gout=gout, nH=nH)


@pytest.mark.parametrize("seed", range(32))
def test_random_msda_forward_and_backward(seed):
    c = _msda_case(seed)
    mode = msda.MSDA_WEIGHTS_LOGITS if c["logits"] else msda.MSDA_WEIGHTS_PROB
    args = (dev(c["value"]), dev(c["ss"]), dev(c["starts"]), dev(c["loc"]), dev(c["weights"]))
    out = host(msda.msda_forward(*args, weight_mode=mode)).reshape(-1, c["nH"] * 32)
    ref = oracle.msda(c["value"], c["ss"], c["starts"], c["loc"], c["weights"], weights_are_logits=c["logits"])
    assert_fp32_close(out, ref, f"case {seed}: forward")
    # the same value's bf16 bits in the head-pair layout
    vb = c["value"] if c["value"].dtype == np.uint16 else W.bf16_bits_trunc(c["value"])
    out_p = host(msda.msda_forward(dev(pairs_host(vb)), *args[1:], weight_mode=mode)).reshape(-1, c["nH"] * 32)
    ref_p = ref if vb is c["value"] else oracle.msda(vb, c["ss"], c["starts"], c["loc"], c["weights"],
                                                      weights_are_logits=c["logits"])
    assert_fp32_close(out_p, ref_p, f"case {seed}: forward, head-pair layout")
    rv, rl, rw = oracle.msda_backward(c["value"], c["ss"], c["starts"], c["loc"], c["weights"], c["gout"],
                                      weights_are_logits=c["logits"])
    # magnitude of each value-gradient element's contributions: alpha >= 0 after a softmax, |p| otherwise
    wmag = c["weights"] if c["logits"] else np.abs(c["weights"])
    mag = oracle.msda_backward(c["value"], c["ss"], c["starts"], c["loc"], wmag, np.abs(c["gout"]),
                               weights_are_logits=c["logits"])[0]
    for atomic in (False, True):
        gv, gl, gw = (host(t) for t in msda.msda_backward(*args, dev(c["gout"]), weight_mode=mode, atomic=atomic))
        what = f"case {seed}, {'atomics' if atomic else 'gather'}"
        assert_sum_close(gv, rv, mag, what + ": grad value")
        assert_fp32_close(gl, rl, what + ": grad locations")
        assert_fp32_close(gw, rw, what + ": grad weights")


def _sca_case(seed, large=False):
    g = np.random.default_rng(np.random.SeedSequence([902 if large else 901, seed]))
    nH, L, P, shapes = _draw_shape(g)
    D = int(g.choice([d for d in (1, 2, 3, 4) if P % d == 0]))
    if large:  # many query tiles and cameras: every tile's queries start in many segments
        B, Ncam, Nq = int(g.integers(1, 4)), int(g.integers(4, 33)), int(g.integers(300, 3000))
    else:
        B, Ncam, Nq = int(g.integers(1, 4)), int(g.integers(1, 9)), int(g.integers(1, 300))
    ss, starts, Nv = W.level_table(shapes)
    value = g.normal(size=(B, Ncam, Nv, nH, 32)).astype(np.float32)
    if g.random() < 0.3:
        value = W.bf16_bits_trunc(value)
    mask = (g.random((Ncam, B, Nq, D)) < g.uniform(0.05, 0.6)).astype(np.uint8)
    rho = g.uniform(-0.2, 1.2, (Ncam, B, Nq, D, 2)).astype(np.float32)
    off = g.normal(0, g.uniform(0.5, 4.0), (B, Nq, nH, L, P, 2)).astype(np.float32)
    logits = g.normal(size=(B, Nq, nH, L * P)).astype(np.float32)
    gout = g.normal(size=(B, Nq, nH * 32)).astype(np.float32)
    return dict(value=value, ss=ss, starts=starts, mask=mask, rho=rho, off=off, logits=logits, gout=gout, B=B,
                Ncam=Ncam, Nq=Nq, nH=nH)


@pytest.mark.parametrize("seed", range(32))
def test_random_sca_forward_and_backward(seed):
    c = _sca_case(seed)
    B, Ncam, Nq, nH = c["B"], c["Ncam"], c["Nq"], c["nH"]
    hit = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
    offs = torch.empty(B * Ncam + 1, dtype=torch.int32, device="cuda")
    pq = torch.empty(B * Ncam * Nq, dtype=torch.int32, device="cuda")
    d = {k: dev(c[k]) for k in ("value", "ss", "starts", "rho", "mask", "off", "logits", "gout")}
    slots = msda.sca_forward(d["value"], d["ss"], d["starts"], d["rho"], d["mask"], d["off"], d["logits"],
                             hit_count=hit, pair_offsets=offs, pair_q=pq)
    args = (c["value"], c["ss"], c["starts"], c["rho"], c["mask"], c["off"], c["logits"])
    ref = oracle.sca(*args)
    assert np.array_equal(host(hit), ref["hit_count"]), f"case {seed}: hit counts"
    assert np.array_equal(host(offs), ref["pair_offsets"]), f"case {seed}: pair offsets"
    n = int(ref["pair_offsets"][-1])
    assert np.array_equal(host(pq)[:n], ref["pair_q"]), f"case {seed}: pair lists"
    assert_fp32_close(host(slots).reshape(B * Nq, -1), ref["slots"], f"case {seed}: slots")
    # the same value's bf16 bits in the head-pair layout
    vb = c["value"] if c["value"].dtype == np.uint16 else W.bf16_bits_trunc(c["value"])
    slots_p = msda.sca_forward(dev(pairs_host(vb)), d["ss"], d["starts"], d["rho"], d["mask"], d["off"], d["logits"])
    ref_p = ref["slots"] if vb is c["value"] else oracle.sca(vb, *args[1:])["slots"]
    assert_fp32_close(host(slots_p).reshape(B * Nq, -1), ref_p, f"case {seed}: slots, head-pair layout")

    ws = torch.empty(msda.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device="cuda")
    msda.sca_compact(d["mask"], d["rho"], ws)
    rv, ro, rl = oracle.sca_backward(*args, c["gout"])
    mag = oracle.sca_backward(*args, np.abs(c["gout"]))[0]
    for atomic, max_pairs in ((False, 0), (False, n), (True, 0)):
        gv, go, gl = (host(t) for t in msda.sca_backward(d["value"], d["ss"], d["starts"], d["rho"], d["off"],
                                                           d["logits"], d["gout"], ws, max_pairs=max_pairs,
                                                           atomic=atomic))
        what = f"case {seed}, {'atomics' if atomic else 'gather'}, max_pairs {max_pairs}"
        assert_sum_close(gv, rv, mag, what + ": grad value")
        assert_fp32_close(go, ro, what + ": grad offsets")
        assert_fp32_close(gl, rl, what + ": grad logits")


@pytest.mark.parametrize("seed", range(8))
def test_random_sca_many_tiles_and_cameras(seed):
    """Forward only, at up to 3,000 queries (a dozen query tiles) and up to
    32 cameras: the compaction's pair lists, offsets and hit counts bit for
    bit, the slots element by element."""
    c = _sca_case(seed, large=True)
    B, Ncam, Nq = c["B"], c["Ncam"], c["Nq"]
    hit = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
    offs = torch.empty(B * Ncam + 1, dtype=torch.int32, device="cuda")
    pq = torch.empty(B * Ncam * Nq, dtype=torch.int32, device="cuda")
    d = {k: dev(c[k]) for k in ("value", "ss", "starts", "rho", "mask", "off", "logits")}
    slots = msda.sca_forward(d["value"], d["ss"], d["starts"], d["rho"], d["mask"], d["off"], d["logits"],
                             hit_count=hit, pair_offsets=offs, pair_q=pq)
    ref = oracle.sca(c["value"], c["ss"], c["starts"], c["rho"], c["mask"], c["off"], c["logits"])
    assert np.array_equal(host(hit), ref["hit_count"]), f"case {seed}: hit counts"
    assert np.array_equal(host(offs), ref["pair_offsets"]), f"case {seed}: pair offsets"
    n = int(ref["pair_offsets"][-1])
    assert np.array_equal(host(pq)[:n], ref["pair_q"]), f"case {seed}: pair lists"
    assert_fp32_close(host(slots).reshape(B * Nq, -1), ref["slots"], f"case {seed}: slots")
