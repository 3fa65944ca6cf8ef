"""The largest value images the library accepts: one level of 1448 x 1448
pixels, 8 heads of 32 float32 channels, is 2,147,024,896 bytes, just under
the 2^31-byte limit per image (1449 x 1449 is rejected, see the CPU ABI
tests), so the byte offsets the kernels form inside an image come within
0.03% of it, and the second image of the batch starts past 2 GiB.  Half of
the queries sample the image's last rows and columns.  The operator's
forward and backward and the SCA forward (two cameras, each an image of that
size) against the oracle, element by element; every call goes through the C
ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_fp32_close, assert_sum_close, dev, host

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")

SIDE = 1448
NH, P = 8, 4


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def big():
    """Two images of the largest size: host copy and device copy."""
    g = np.random.default_rng(np.random.SeedSequence([950, 1]))
    ss, starts, Nv = W.level_table(((SIDE, SIDE),))
    assert Nv * NH * 32 * 4 < 1 << 31 <= (SIDE + 1) ** 2 * NH * 32 * 4
    value = g.random((2, Nv, NH, 32), dtype=np.float32)
    value -= 0.5
    d = {"value": value, "ss": ss, "starts": starts, "Nv": Nv, "value_dev": dev(value)}
    yield d
    del d["value_dev"]
    torch.cuda.empty_cache()


def _far_corner_locations(g, shape):
    """Uniform over [-0.1, 1.1]^2, and for the first half of the queries
    (axis 1) over the last rows and columns of the image and just past them."""
    loc = g.uniform(-0.1, 1.1, shape).astype(np.float32)
    half = shape[1] // 2
    loc[:, :half] = g.uniform(0.97, 1.01, (shape[0], half) + tuple(shape[2:]))
    return loc


def _touched_rows(loc, B, Nv):
    """Flat (b * Nv + pixel) indices of every in-map corner of the samples."""
    x = loc[..., 0].astype(np.float64) * SIDE - 0.5
    y = loc[..., 1].astype(np.float64) * SIDE - 0.5
    x0, y0 = np.floor(x), np.floor(y)
    b = np.broadcast_to(np.arange(B).reshape((B,) + (1,) * (x.ndim - 1)), x.shape)
    out = []
    for dx in (0, 1):
        for dy in (0, 1):
            cx, cy = x0 + dx, y0 + dy
            ok = (cx >= 0) & (cx < SIDE) & (cy >= 0) & (cy < SIDE)
            out.append(b[ok] * Nv + (cy[ok] * SIDE + cx[ok]).astype(np.int64))
    return np.unique(np.concatenate(out))


def test_msda_largest_images_forward_and_backward(big):
    B, Nq, Nv = 2, 300, big["Nv"]
    g = np.random.default_rng(np.random.SeedSequence([950, 2]))
    loc = _far_corner_locations(g, (B, Nq, NH, 1, P, 2))
    logits = g.normal(size=(B, Nq, NH, P)).astype(np.float32)
    gout = g.normal(size=(B, Nq, NH * 32)).astype(np.float32)
    args = (big["value_dev"], dev(big["ss"]), dev(big["starts"]), dev(loc), dev(logits))
    mode = msda.MSDA_WEIGHTS_LOGITS

    out = host(msda.msda_forward(*args, weight_mode=mode)).reshape(B * Nq, -1)
    ref = oracle.msda(big["value"], big["ss"], big["starts"], loc, logits, weights_are_logits=True)
    assert_fp32_close(out, ref, "forward")

    gv, gl, gw = msda.msda_backward(*args, dev(gout), weight_mode=mode)
    rv, rl, rw = oracle.msda_backward(big["value"], big["ss"], big["starts"], loc, logits, gout,
                                      weights_are_logits=True)
    assert_fp32_close(host(gl), rl, "grad locations")
    assert_fp32_close(host(gw), rw, "grad logits")
    # the value gradient: rows that a corner touches against the oracle, and
    # every other row of the 4 GiB gradient exactly zero
    rows = _touched_rows(loc, B, Nv)
    assert rows.max() >= (B - 1) * Nv + SIDE * SIDE - 2 * SIDE, "the image's last rows were sampled"
    flat = gv.view(B * Nv, NH * 32)
    nonzero = host(torch.nonzero(flat.ne(0).any(dim=1)).flatten())
    assert np.isin(nonzero, rows).all(), "value gradient outside the sampled rows"
    got = host(flat[torch.from_numpy(rows).cuda()])
    mag = oracle.msda_backward(big["value"], big["ss"], big["starts"], loc, logits, np.abs(gout),
                               weights_are_logits=True)[0]
    assert_sum_close(got, rv.reshape(B * Nv, -1)[rows], mag.reshape(B * Nv, -1)[rows], "grad value (sampled rows)")
    del gv, gl, gw, flat, rv, mag


def test_sca_largest_images_forward(big):
    """Batch 1, two cameras: the two largest images are the two cameras'."""
    B, Ncam, Nq, D = 1, 2, 400, 4
    g = np.random.default_rng(np.random.SeedSequence([950, 3]))
    value = big["value"].reshape(B, Ncam, big["Nv"], NH, 32)
    rho = _far_corner_locations(g, (Ncam, Nq, D, 2)).reshape(Ncam, B, Nq, D, 2)
    mask = (g.random((Ncam, B, Nq, D)) < 0.5).astype(np.uint8)
    off = g.normal(0, 2.0, (B, Nq, NH, 1, P, 2)).astype(np.float32)
    logits = g.normal(size=(B, Nq, NH, P)).astype(np.float32)
    hit = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
    slots = msda.sca_forward(big["value_dev"].view(B, Ncam, big["Nv"], NH, 32), dev(big["ss"]), dev(big["starts"]),
                             dev(rho), dev(mask), dev(off), dev(logits), hit_count=hit)
    ref = oracle.sca(value, big["ss"], big["starts"], rho, mask, off, logits)
    assert np.array_equal(host(hit), ref["hit_count"]), "hit counts"
    assert_fp32_close(host(slots).reshape(B * Nq, -1), ref["slots"], "slots")


@pytest.mark.parametrize("side,flat", [(1023, True), (1024, False)])
def test_frames_buffer_over_two_images(side, flat):
    """Two stacked frames of one level side x side (8 float32 heads): at 1023
    the two images, 2,143,291,392 bytes, are staged and gathered through one
    buffer of just under 2^31 bytes; at 1024 they are exactly 2^31 and go
    frame by frame.  Half of the queries sample the last rows and columns of
    both frames."""
    B, F, Nq = 1, 2, 256
    ss, starts, Nv = W.level_table(((side, side),))
    assert (F * Nv * NH * 32 * 4 < 1 << 31) == flat
    g = np.random.default_rng(np.random.SeedSequence([951, side]))
    value = g.random((B, F, Nv, NH, 32), dtype=np.float32)
    value -= 0.5
    loc = _far_corner_locations(g, (B * F, Nq, NH, 1, P, 2)).reshape(B, F, Nq, NH, 1, P, 2)
    logits = g.normal(size=(B, F, Nq, NH, P)).astype(np.float32)
    vd = dev(value)
    out = host(msda.msda_forward_frames(vd, dev(ss), dev(starts), dev(loc), dev(logits))).reshape(B * Nq, -1)
    del vd
    torch.cuda.empty_cache()
    ref = oracle.msda_frames(value, ss, starts, loc, logits, True)
    assert_fp32_close(out, ref, f"two frames of {side} x {side}")
