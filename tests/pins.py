"""Pins of the CPU oracle to facts outside itself.

Each pin checks the oracle against something the pages print, a closed form,
an invariant, or an independent library routine -- never against a retyped
copy of the oracle's own loops.  They are plain functions (raise
AssertionError on failure) so that test_oracle_pins.py runs them against the
oracle and test_oracle_mutants.py runs them against copies of the oracle with
planted mistakes, each of which must fail at least one pin.

Sources:
  [8-heads]  "BEV(三) BEVFormer：Query 参数如何与 Feature 的 8 个 Head 交互"
  [SCA-note] Tencent Cloud developer article 2321140 (Spatial Cross-Attention)
"""
import json
import os

import numpy as np

import oracle
from workloads import level_table

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol=1e-11, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert err <= tol * scale, f"{what}: max abs err {err:g}"


def _centre(i, n):
    """Normalised coordinate of the centre of cell i of n ([8-heads] 6: the
    continuous coordinate is n*s - 1/2, so cell i's centre is s = (i + 1/2)/n)."""
    return (np.asarray(i, np.float64) + 0.5) / n


# ---------------------------------------------------------------------------
# worked examples printed on the pages
# ---------------------------------------------------------------------------

def pin_worked_example_two_heads():
    """[8-heads] 15: two heads x two channels, two samples each."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_two_heads.json")))
    nH, Dh, P = 2, 2, 2
    # one 1x4 level; sample k of head h sits alone at the centre of pixel 2h+k.
    ss, starts, Nv = level_table(((1, 4),))
    g = np.random.default_rng(5)
    value = g.normal(size=(1, Nv, nH, Dh)).astype(np.float32)  # other entries are decoys
    loc = np.zeros((1, 1, nH, 1, P, 2), np.float32)
    alpha = np.zeros((1, 1, nH, P), np.float32)
    for h, head in enumerate(ex["heads"]):
        for k in range(P):
            pix = 2 * h + k
            value[0, pix, h, :] = head["samples"][k]
            loc[0, 0, h, 0, k] = (_centre(pix, 4), _centre(0, 1))
            alpha[0, 0, h, k] = head["alpha"][k]
    out = oracle.msda(value, ss, starts, loc, alpha, weights_are_logits=False)[0]
    _close(out, ex["concat"], 1e-6, "concat (probabilities)")  # alpha is float32 here
    # same weights given as logits: softmax(log alpha) = alpha
    out_l = oracle.msda(value, ss, starts, loc, np.log(alpha), weights_are_logits=True)[0]
    _close(out_l, ex["concat"], 1e-6, "concat (logits)")
    for h, head in enumerate(ex["heads"]):
        _close(out[h * Dh:(h + 1) * Dh], head["g"], 1e-6, f"g head {h}")
    # identity output projection and the residual add
    _close(np.asarray(ex["query"]) + out, ex["query_plus_output"], 1e-6, "query + output")


def pin_scalar_times_sample():
    """[8-heads] 7: a weight of 0.7 on the sample [10, 20, 30] gives [7, 14, 21]."""
    ex = json.load(open(os.path.join(GOLDEN, "scalar_times_sample.json")))
    ss, starts, Nv = level_table(((1, 1),))
    value = np.array(ex["sample"], np.float32).reshape(1, 1, 1, 3)
    loc = np.array([0.5, 0.5], np.float32).reshape(1, 1, 1, 1, 1, 2)
    w = np.array([ex["alpha"]], np.float32).reshape(1, 1, 1, 1)
    out = oracle.msda(value, ss, starts, loc, w)[0]
    _close(out, ex["weighted"], 1e-6, "alpha * f")


# ---------------------------------------------------------------------------
# softmax ([8-heads] 4.2, 4.3)
# ---------------------------------------------------------------------------

def _gather_case(seed, shapes, nH, Dh, P, Nq=7):
    """Samples placed at random pixel centres: bilinear reduces to a plain
    gather, so the expected output is a weighted sum of stored vectors.
    Power-of-two level sizes keep the centres exact in float32."""
    ss, starts, Nv = level_table(shapes)
    L = len(ss)
    g = np.random.default_rng(seed)
    value = g.normal(size=(1, Nv, nH, Dh)).astype(np.float32)
    loc = np.zeros((1, Nq, nH, L, P, 2), np.float32)
    pix = np.zeros((Nq, nH, L, P), np.int64)
    for l, (H, W) in enumerate(ss):
        xi = g.integers(0, W, size=(Nq, nH, P))
        yi = g.integers(0, H, size=(Nq, nH, P))
        loc[0, :, :, l, :, 0] = _centre(xi, W)
        loc[0, :, :, l, :, 1] = _centre(yi, H)
        pix[:, :, l, :] = starts[l] + yi * W + xi
    return value, ss, starts, loc, pix


def pin_zero_logits_give_plain_mean():
    """[8-heads] 4.3: zero logits give every one of the L*P samples weight 1/(L*P)."""
    nH, Dh, P = 3, 5, 4
    value, ss, starts, loc, pix = _gather_case(11, ((4, 8), (2, 2)), nH, Dh, P)
    Nq, L = loc.shape[1], len(ss)
    out = oracle.msda(value, ss, starts, loc, np.zeros((1, Nq, nH, L * P), np.float32), True)
    for q in range(Nq):
        for h in range(nH):
            want = value[0, pix[q, h].ravel(), h, :].astype(np.float64).mean(axis=0)
            _close(out[q, h * Dh:(h + 1) * Dh], want, 1e-12, "zero logits")


def pin_softmax_invariants():
    """[8-heads] 4.2: per-head weights are exp / sum exp, so they add up to one
    (a constant map returns the constant), a per-head shift of the logits
    changes nothing, and logits log(p) reproduce the probabilities p."""
    nH, Dh, P = 2, 3, 3
    value, ss, starts, loc, pix = _gather_case(12, ((4, 4), (2, 4)), nH, Dh, P)
    Nq, L = loc.shape[1], len(ss)
    g = np.random.default_rng(13)
    # multiples of 1/1024: adding the integer shifts below is exact in float32
    logits = (g.integers(-3000, 3000, size=(1, Nq, nH, L * P)) / 1024.0).astype(np.float32)
    base = oracle.msda(value, ss, starts, loc, logits, True)
    shift = np.float32(3.0) * np.arange(1, nH + 1, dtype=np.float32)[None, None, :, None]
    _close(oracle.msda(value, ss, starts, loc, logits + shift, True), base, 1e-12, "shift")
    p = g.random(size=(1, Nq, nH, L * P)) + 0.05
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    _close(oracle.msda(value, ss, starts, loc, np.log(p), True),
           oracle.msda(value, ss, starts, loc, p, False), 1e-6, "log p")
    const = np.broadcast_to(np.arange(1, nH * Dh + 1, dtype=np.float32).reshape(1, 1, nH, Dh),
                            value.shape).copy()
    out = oracle.msda(const, ss, starts, loc, logits, True)
    _close(out, np.broadcast_to(np.arange(1, nH * Dh + 1, dtype=np.float64), out.shape), 1e-12, "sum to 1")


# ---------------------------------------------------------------------------
# bilinear sampling ([8-heads] 6)
# ---------------------------------------------------------------------------

def pin_integer_aligned_exact_gather():
    """Samples at pixel centres return the stored vector exactly (one sample,
    one point: the weight is softmax of one logit = 1)."""
    nH, Dh = 4, 6
    value, ss, starts, loc, pix = _gather_case(21, ((4, 8), (8, 2), (1, 1)), nH, Dh, 1, Nq=9)
    Nq, L = loc.shape[1], len(ss)
    for l in range(L):
        out = oracle.msda(value, ss[l:l + 1], starts[l:l + 1], np.ascontiguousarray(loc[:, :, :, l:l + 1]),
                          np.zeros((1, Nq, nH, 1), np.float32), True)
        for q in range(Nq):
            for h in range(nH):
                _close(out[q, h * Dh:(h + 1) * Dh], value[0, pix[q, h, l, 0], h], 0.0, "gather")


def pin_constant_map_inside():
    """A constant map returns the constant wherever all four corners are
    inside the map."""
    ss, starts, Nv = level_table(((6, 9), (4, 3)))
    nH, Dh, P, Nq = 2, 4, 5, 10
    L = len(ss)
    g = np.random.default_rng(31)
    c = g.normal(size=(nH, Dh)).astype(np.float32)
    value = np.broadcast_to(c, (1, Nv, nH, Dh)).copy()
    loc = np.zeros((1, Nq, nH, L, P, 2), np.float32)
    for l, (H, W) in enumerate(ss):
        loc[..., l, :, 0] = (g.uniform(0, W - 1, (1, Nq, nH, P)) + 0.5) / W
        loc[..., l, :, 1] = (g.uniform(0, H - 1, (1, Nq, nH, P)) + 0.5) / H
    out = oracle.msda(value, ss, starts, loc, g.normal(size=(1, Nq, nH, L * P)).astype(np.float32), True)
    _close(out, np.broadcast_to(c.reshape(-1), out.shape), 1e-12, "constant map")


def pin_affine_ramp_exact():
    """Bilinear interpolation reproduces an affine function of the pixel
    coordinates exactly between pixel centres: a map V(i, j) = a*i + b*j + c
    (column i, row j) sampled at s gives a*x + b*y + c with x = W*s_x - 1/2,
    y = H*s_y - 1/2 ([8-heads] 6).  Pins the half-pixel convention, which of
    x/y pairs with W/H, and the row-major flattening.  Integer coefficients
    keep the map exact in float32."""
    shapes = ((5, 8), (7, 3))
    ss, starts, Nv = level_table(shapes)
    nH, Dh, P, Nq = 2, 3, 4, 6
    L = len(ss)
    g = np.random.default_rng(41)
    a, b, c = (g.integers(-4, 5, size=(L, nH, Dh)).astype(np.float64) for _ in range(3))
    value = np.zeros((1, Nv, nH, Dh), np.float32)
    for l, (H, W) in enumerate(ss):
        jj, ii = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")  # row j, column i
        flat = (starts[l] + jj * W + ii).ravel()
        value[0, flat] = a[l] * ii.ravel()[:, None, None] + b[l] * jj.ravel()[:, None, None] + c[l]
    loc = np.zeros((1, Nq, nH, L, P, 2), np.float32)
    for l, (H, W) in enumerate(ss):
        loc[..., l, :, 0] = (g.uniform(0, W - 1, (1, Nq, nH, P)) + 0.5) / W
        loc[..., l, :, 1] = (g.uniform(0, H - 1, (1, Nq, nH, P)) + 0.5) / H
    p = g.random((1, Nq, nH, L * P)) + 0.1
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    out = oracle.msda(value, ss, starts, loc, p, False).reshape(Nq, nH, Dh)
    want = np.zeros((Nq, nH, Dh))
    for l, (H, W) in enumerate(ss):
        x = W * loc[0, :, :, l, :, 0].astype(np.float64) - 0.5  # [Nq,nH,P]
        y = H * loc[0, :, :, l, :, 1].astype(np.float64) - 0.5
        w = p[0].reshape(Nq, nH, L, P)[:, :, l, :].astype(np.float64)
        f = a[l][None, :, None, :] * x[..., None] + b[l][None, :, None, :] * y[..., None] + c[l][None, :, None, :]
        want += np.einsum("qhp,qhpd->qhd", w, f)
    _close(out, want, 1e-11, "affine ramp")


def pin_grid_sample_special_case():
    """Library special case: for one level, head and point with weight 1,
    MSDA is torch.nn.functional.grid_sample(mode='bilinear',
    padding_mode='zeros', align_corners=False) at grid = 2*s - 1.  With
    several levels, heads and points the output is the weighted sum of such
    samples, the levels cut out of the flattened value axis by their
    (H, W) and start.  Locations cover the border and the outside."""
    import torch
    shapes = ((6, 10), (3, 5), (2, 2))
    ss, starts, Nv = level_table(shapes)
    nH, Dh, P, Nq = 3, 4, 3, 40
    L = len(ss)
    g = np.random.default_rng(51)
    value = g.normal(size=(1, Nv, nH, Dh)).astype(np.float32)
    loc = g.uniform(-0.3, 1.3, size=(1, Nq, nH, L, P, 2)).astype(np.float32)
    p = g.random((1, Nq, nH, L * P)) + 0.1
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    out = oracle.msda(value, ss, starts, loc, p, False).reshape(Nq, nH, Dh)
    want = np.zeros((Nq, nH, Dh))
    for l, (H, W) in enumerate(ss):
        lvl = value[0, starts[l]:starts[l] + H * W].reshape(H, W, nH, Dh)
        for h in range(nH):
            img = torch.from_numpy(lvl[:, :, h, :].transpose(2, 0, 1).astype(np.float64)).unsqueeze(0)
            grid = torch.from_numpy(2.0 * loc[0, :, h, l].astype(np.float64) - 1.0).unsqueeze(0)  # [1,Nq,P,2]
            smp = torch.nn.functional.grid_sample(img, grid, mode="bilinear", padding_mode="zeros",
                                                  align_corners=False)[0].numpy()  # [Dh,Nq,P]
            w = p[0, :, h, l * P:(l + 1) * P].astype(np.float64)  # [Nq,P]
            want[:, h, :] += np.einsum("qp,dqp->qd", w, smp)
    _close(out, want, 1e-10, "grid_sample")


def _tent_msda(value, ss, starts, loc, alpha):
    """Dense reformulation: bilinear weight of pixel (i, j) for a sample at
    continuous (x, y) is max(0, 1-|x-i|) * max(0, 1-|y-j|); pixels outside the
    map simply do not exist.  out[q,h] = sum over pixels of A[q,h,pix] V[pix,h]."""
    B, Nv, nH, Dh = value.shape
    _, Nq, _, L, P, _ = loc.shape
    out = np.zeros((B, Nq, nH, Dh))
    for b in range(B):
        A = np.zeros((Nq, nH, Nv))
        for l, (H, W) in enumerate(ss):
            x = W * loc[b, :, :, l, :, 0].astype(np.float64) - 0.5  # [Nq,nH,P]
            y = H * loc[b, :, :, l, :, 1].astype(np.float64) - 0.5
            ti = np.maximum(0.0, 1.0 - np.abs(x[..., None] - np.arange(W)))  # [Nq,nH,P,W]
            tj = np.maximum(0.0, 1.0 - np.abs(y[..., None] - np.arange(H)))  # [Nq,nH,P,H]
            a = alpha[b, :, :, l * P:(l + 1) * P].astype(np.float64)
            A[:, :, starts[l]:starts[l] + H * W] += np.einsum("qhp,qhpj,qhpi->qhji", a, tj, ti).reshape(Nq, nH, H * W)
        out[b] = np.einsum("qhv,vhd->qhd", A, value[b].astype(np.float64))
    return out.reshape(B * Nq, nH * Dh)


def pin_dense_reformulation():
    """Brute force on tiny inputs: the tent-function form of bilinear
    interpolation (no floor, no corner enumeration), weights as a dense
    matrix over all pixels, times the value map."""
    shapes = ((4, 7), (3, 2), (1, 3))
    ss, starts, Nv = level_table(shapes)
    B, nH, Dh, P, Nq = 2, 2, 3, 3, 6
    L = len(ss)
    g = np.random.default_rng(61)
    value = g.normal(size=(B, Nv, nH, Dh)).astype(np.float32)
    loc = g.uniform(-0.2, 1.2, size=(B, Nq, nH, L, P, 2)).astype(np.float32)
    logits = g.normal(size=(B, Nq, nH, L * P)).astype(np.float32)
    e = np.exp(logits.astype(np.float64))
    alpha = e / e.sum(-1, keepdims=True)
    _close(oracle.msda(value, ss, starts, loc, logits, True), _tent_msda(value, ss, starts, loc, alpha),
           1e-12, "dense reformulation")
    # bf16 value bits decode exactly
    bits = (value.view(np.uint32) >> 16).astype(np.uint16)
    vb = (bits.astype(np.uint32) << 16).view(np.float32)
    _close(oracle.msda(bits, ss, starts, loc, logits, True), _tent_msda(vb, ss, starts, loc, alpha),
           1e-12, "dense reformulation, bf16 value")


# ---------------------------------------------------------------------------
# frames (two stacked BEV maps)
# ---------------------------------------------------------------------------

def pin_frames_mean():
    """Frame mean: identical frames give the single-frame result; a zero frame
    halves the other frame's result; swapping frames changes nothing."""
    shapes = ((5, 5),)
    ss, starts, Nv = level_table(shapes)
    B, nH, Dh, P, Nq = 2, 2, 3, 4, 8
    g = np.random.default_rng(71)
    v1 = g.normal(size=(B, Nv, nH, Dh)).astype(np.float32)
    v2 = g.normal(size=(B, Nv, nH, Dh)).astype(np.float32)
    l1 = g.uniform(0, 1, (B, Nq, nH, 1, P, 2)).astype(np.float32)
    l2 = g.uniform(0, 1, (B, Nq, nH, 1, P, 2)).astype(np.float32)
    w1 = g.normal(size=(B, Nq, nH, P)).astype(np.float32)
    w2 = g.normal(size=(B, Nq, nH, P)).astype(np.float32)
    single = oracle.msda(v1, ss, starts, l1, w1, True)
    st = lambda a, b: np.stack([a, b], axis=1)
    _close(oracle.msda_frames(st(v1, v1), ss, starts, st(l1, l1), st(w1, w1), True), single, 1e-12, "identical")
    _close(oracle.msda_frames(st(v1, np.zeros_like(v1)), ss, starts, st(l1, l2), st(w1, w2), True),
           0.5 * single, 1e-12, "zero frame")
    _close(oracle.msda_frames(st(v1, v2), ss, starts, st(l1, l2), st(w1, w2), True),
           oracle.msda_frames(st(v2, v1), ss, starts, st(l2, l1), st(w2, w1), True), 1e-12, "swap")


# ---------------------------------------------------------------------------
# spatial cross-attention ([8-heads] 5, 10; [SCA-note])
# ---------------------------------------------------------------------------

def pin_sca_compaction_brute_force():
    """[SCA-note] rebatch and count: a camera sees a query when any anchor is
    marked; per (batch item, camera) the seen queries in ascending order;
    hit count per query.  Checked against numpy any / nonzero / sum, with
    masks that differ across the batch."""
    B, Ncam, Nq, D = 3, 4, 37, 4
    g = np.random.default_rng(81)
    mask = (g.random((Ncam, B, Nq, D)) < 0.15).astype(np.uint8)
    mask[:, 1, 5, :] = 0  # a query nobody sees
    ss, starts, Nv = level_table(((2, 2),))
    value = np.zeros((B, Ncam, Nv, 1, 1), np.float32)
    rho = np.zeros((Ncam, B, Nq, D, 2), np.float32)
    off = np.zeros((B, Nq, 1, 1, D, 2), np.float32)
    lg = np.zeros((B, Nq, 1, D), np.float32)
    r = oracle.sca(value, ss, starts, rho, mask, off, lg, want_slots=False)
    vis = mask.any(-1)
    assert np.array_equal(r["hit_count"], vis.sum(0)), "hit count"
    offs, pq, n = [0], [], 0
    for b in range(B):
        for c in range(Ncam):
            idx = np.nonzero(vis[c, b])[0]
            pq.extend(idx.tolist())
            n += len(idx)
            offs.append(n)
    assert np.array_equal(r["pair_offsets"], np.array(offs)), "pair offsets (b-major, camera-minor)"
    assert np.array_equal(r["pair_q"], np.array(pq)), "pair lists"
    assert int(r["pair_offsets"][-1]) == int(r["hit_count"].sum()), "pairs = sum of hits"


def _sca_gather_case():
    """Samples that land on known pixel centres, so the expected SCA result is
    a plain gather computed by integer arithmetic.

    Level 1 is 4x8 and level 0 is 8x16 (twice as fine).  Anchor m of
    (camera, query) sits at the centre of level-1 pixel (ax, ay), which is
    the corner point between level-0 pixels 2*ax, 2*ax+1 (and 2*ay, 2*ay+1).
    Offsets are integers (dx, dy) in level-1 cells, and (dx + 1/2, dy + 1/2)
    in level-0 cells, so point k lands on level-1 pixel (ax + dx, ay + dy) and
    on level-0 pixel (2*ax + 1 + dx, 2*ay + 1 + dy).  Power-of-two sizes keep
    every location exact in float32.  Zero logits weight all L*P points
    equally.  Queries: q0 seen by no camera, q1 by camera 1, q2 by cameras 0
    and 2, q3 by camera 2 through one marked anchor only."""
    shapes = ((8, 16), (4, 8))
    ss, starts, Nv = level_table(shapes)
    B, Ncam, Nq, D, P, nH, Dh = 1, 3, 4, 2, 4, 2, 3
    L = len(ss)
    g = np.random.default_rng(91)
    value = g.normal(size=(B, Ncam, Nv, nH, Dh)).astype(np.float32)
    mask = np.zeros((Ncam, B, Nq, D), np.uint8)
    mask[1, 0, 1] = 1
    mask[0, 0, 2] = 1
    mask[2, 0, 2] = 1
    mask[2, 0, 3, 0] = 1
    ax = g.integers(1, 7, (Ncam, B, Nq, D))
    ay = g.integers(1, 3, (Ncam, B, Nq, D))
    rho = np.stack([_centre(ax, 8), _centre(ay, 4)], axis=-1).astype(np.float32)
    dx = g.integers(-1, 2, (B, Nq, nH, L, P))
    dy = g.integers(-1, 2, (B, Nq, nH, L, P))
    half = np.array([0.5, 0.0])[None, None, None, :, None]  # level 0 carries the half cell
    off = np.stack([dx + half, dy + half], axis=-1).astype(np.float32)
    logits = np.zeros((B, Nq, nH, L * P), np.float32)
    want = np.zeros((Nq, nH, Dh))
    for q in range(Nq):
        cams = [c for c in range(Ncam) if mask[c, 0, q].any()]
        for c in cams:
            for h in range(nH):
                for l, (H, W) in enumerate(ss):
                    for k in range(P):
                        m = k % D
                        if l == 0:
                            col = 2 * ax[c, 0, q, m] + 1 + dx[0, q, h, l, k]
                            row = 2 * ay[c, 0, q, m] + 1 + dy[0, q, h, l, k]
                        else:
                            col = ax[c, 0, q, m] + dx[0, q, h, l, k]
                            row = ay[c, 0, q, m] + dy[0, q, h, l, k]
                        if 0 <= col < W and 0 <= row < H:
                            want[q, h] += value[0, c, starts[l] + row * W + col, h] / (L * P)
        if cams:
            want[q] /= len(cams)
    return value, ss, starts, rho, mask, off, logits, want.reshape(Nq, nH * Dh)


def pin_sca_exact_gather_and_camera_mean():
    """[8-heads] 5 and 10, [SCA-note]: point k of a level uses anchor k mod D
    and moves by (dx / W_l, dy / H_l); each camera that sees the query
    contributes its own result, the results are averaged over the seeing
    cameras (max(1, hits)); a query no camera sees gets zeros."""
    value, ss, starts, rho, mask, off, logits, want = _sca_gather_case()
    r = oracle.sca(value, ss, starts, rho, mask, off, logits)
    _close(r["slots"], want, 1e-12, "sca exact gather")
    assert np.all(r["slots"][0] == 0.0), "unseen query must be zero"


def pin_sca_dense_reformulation():
    """Tiny random SCA against the tent-function dense form applied per
    camera with s = rho[anchor k mod D] + (dx/W_l, dy/H_l), averaged over the
    seeing cameras; also identical cameras give the single-camera result."""
    shapes = ((5, 7), (3, 4))
    ss, starts, Nv = level_table(shapes)
    B, Ncam, Nq, D, P, nH, Dh = 2, 3, 9, 2, 4, 2, 3
    L = len(ss)
    g = np.random.default_rng(101)
    value = g.normal(size=(B, Ncam, Nv, nH, Dh)).astype(np.float32)
    mask = (g.random((Ncam, B, Nq, D)) < 0.5).astype(np.uint8)
    rho = g.uniform(-0.1, 1.1, (Ncam, B, Nq, D, 2)).astype(np.float32)
    off = g.normal(0, 1.5, (B, Nq, nH, L, P, 2)).astype(np.float32)
    logits = g.normal(size=(B, Nq, nH, L * P)).astype(np.float32)
    e = np.exp(logits.astype(np.float64))
    alpha = e / e.sum(-1, keepdims=True)
    vis = mask.any(-1)
    want = np.zeros((B, Nq, nH * Dh))
    cells = np.array([[W, H] for H, W in ss], np.float64)  # (W, H) per level
    anchor = np.arange(P) % D
    for c in range(Ncam):
        loc = rho[c][:, :, None, None, anchor, :].astype(np.float64) + off / cells[None, None, None, :, None, :]
        loc = np.broadcast_to(loc, (B, Nq, nH, L, P, 2))
        # the dense form takes float32 locations; keep them in float64 here
        res = np.zeros((B, Nq, nH, Dh))
        for b in range(B):
            A = np.zeros((Nq, nH, Nv))
            for l, (H, W) in enumerate(ss):
                x = W * loc[b, :, :, l, :, 0] - 0.5
                y = H * loc[b, :, :, l, :, 1] - 0.5
                ti = np.maximum(0.0, 1.0 - np.abs(x[..., None] - np.arange(W)))
                tj = np.maximum(0.0, 1.0 - np.abs(y[..., None] - np.arange(H)))
                a = alpha[b, :, :, l * P:(l + 1) * P]
                A[:, :, starts[l]:starts[l] + H * W] += np.einsum("qhp,qhpj,qhpi->qhji", a, tj, ti).reshape(Nq, nH, H * W)
            res[b] = np.einsum("qhv,vhd->qhd", A, value[b, c].astype(np.float64))
        want += vis[c][:, :, None] * res.reshape(B, Nq, nH * Dh)
    want /= np.maximum(1, vis.sum(0))[:, :, None]
    r = oracle.sca(value, ss, starts, rho, mask, off, logits)
    _close(r["slots"], want.reshape(B * Nq, -1), 1e-11, "sca dense")
    # identical cameras: same value and anchors in every camera
    v_same = np.broadcast_to(value[:, :1], value.shape).copy()
    rho_same = np.broadcast_to(rho[:1], rho.shape).copy()
    both = np.ones_like(mask)
    one = np.zeros_like(mask)
    one[0] = 1
    _close(oracle.sca(v_same, ss, starts, rho_same, both, off, logits)["slots"],
           oracle.sca(v_same, ss, starts, rho_same, one, off, logits)["slots"], 1e-12, "identical cameras")


def pin_sca_rebatch_equals_fused_on_exact_locations():
    """The SCA note's padded flow (oracle.sca_rebatch) against the fused
    oracle.sca: with power-of-two level sides and anchors and offsets on a
    coarse binary grid, rho + dx/W is exact in float32, so materialising the
    locations loses nothing and both forms must agree bit for bit --
    segments, padding (never added back), camera order and divide included.
    Segments of unequal length and an empty one exercise the padding."""
    shapes = ((8, 16), (4, 8))
    ss, starts, Nv = level_table(shapes)
    B, Ncam, Nq, D, P, nH, Dh = 2, 4, 11, 2, 4, 2, 3
    L = len(ss)
    g = np.random.default_rng(113)
    value = g.normal(size=(B, Ncam, Nv, nH, Dh)).astype(np.float32)
    mask = (g.random((Ncam, B, Nq, D)) < 0.4).astype(np.uint8)
    mask[2, 1] = 0  # camera 2 sees nothing of batch item 1
    rho = (g.integers(-100, 1124, (Ncam, B, Nq, D, 2)) / 1024.0).astype(np.float32)
    off = (np.round(g.normal(0, 1.5, (B, Nq, nH, L, P, 2)) * 256) / 256).astype(np.float32)
    logits = g.normal(size=(B, Nq, nH, L * P)).astype(np.float32)
    args = (value, ss, starts, rho, mask, off, logits)
    fused = oracle.sca(*args)
    pad = oracle.sca_rebatch(*args)
    lens = np.diff(pad["pair_offsets"])
    assert lens.min() == 0 and len(set(lens.tolist())) > 2, "padding is exercised"
    assert pad["max_len"] == lens.max()
    for k in ("hit_count", "pair_offsets", "pair_q"):
        assert np.array_equal(pad[k], fused[k]), k
    for bc, n in enumerate(lens):
        assert not pad["sampling_locations"][bc, n:].any() and not pad["logits"][bc, n:].any(), "padded rows"
    assert np.array_equal(pad["slots"], fused["slots"]), "padded flow differs from the fused definition"


# ---------------------------------------------------------------------------
# bf16 and the projections ([8-heads] 3 and 11)
# ---------------------------------------------------------------------------

def pin_bf16_rounding():
    """Round-to-nearest-even to bf16: fixed ties near 1, and agreement with
    torch's float32 -> bfloat16 conversion on random float32 values."""
    import torch
    cases = {1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -8: 0x3F82, 1.0 + 2 ** -8 + 2 ** -20: 0x3F81,
             -(1.0 + 2 ** -8): 0xBF80, 0.0: 0x0000, 65504.0: 0x4780, 3.0e38: 0x7F62}
    got = oracle.round_to_bf16(np.array(list(cases.keys())))
    assert [int(x) for x in got] == list(cases.values()), [hex(int(x)) for x in got]
    g = np.random.default_rng(111)
    x = (g.normal(size=4096) * np.exp(g.uniform(-30, 30, 4096))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to_bf16(x.astype(np.float64)), ref), "bf16 RNE vs torch"
    assert np.array_equal(oracle.bf16_to_float64(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()), "bf16 widening"


def pin_linear_bf16():
    """Y = X W^T + b from bf16 operands: an identity weight reproduces the
    input; the result equals a float64 matmul of the decoded operands; a
    float32 input is rounded to bf16 first (as torch's conversion does)."""
    import torch
    g = np.random.default_rng(121)
    M, N, K = 13, 6, 8
    tobf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    dec = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    X = tobf(g.normal(size=(M, K)))
    W = tobf(g.normal(size=(N, K)))
    bias = g.normal(size=N).astype(np.float32)
    _close(oracle.linear_bf16(X, W, bias), dec(X) @ dec(W).T + bias.astype(np.float64), 1e-13, "matmul")
    _close(oracle.linear_bf16_blas(X, W, bias), oracle.linear_bf16(X, W, bias), 1e-13, "blas form = loops")
    eye = tobf(np.eye(K))
    _close(oracle.linear_bf16(X, eye), dec(X), 0.0, "identity")
    Xf = g.normal(size=(M, K)).astype(np.float32)
    _close(oracle.linear_bf16(Xf, W), dec(tobf(Xf)) @ dec(W).T, 1e-13, "float32 input")


def _tobf(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _dec(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def pin_query_proj():
    """Offsets and logits from the query ([8-heads] 4.1, 4.2): the predicting
    vector is the float32 sum query + position embedding (formed here by
    torch's float32 addition), rounded to bf16; each output is a float64
    matmul of the decoded operands plus its own bias.  A sum whose exact
    value lies just above a bf16 tie but whose float32 rounding lands on the
    tie tells a float32 addition from an exact one."""
    import torch
    g = np.random.default_rng(131)
    M, K, N_off, N_att = 11, 32, 48, 16
    q = g.normal(size=(M, K)).astype(np.float32)
    e = g.normal(size=(M, K)).astype(np.float32)
    W_off, W_att = _tobf(g.normal(size=(N_off, K)) / 6), _tobf(g.normal(size=(N_att, K)) / 6)
    b_off, b_att = g.normal(size=N_off).astype(np.float32), g.normal(size=N_att).astype(np.float32)
    qt = (torch.from_numpy(q) + torch.from_numpy(e)).numpy()
    x = _dec(_tobf(qt))
    off, lg = oracle.query_proj(q, e, W_off, b_off, W_att, b_att)
    _close(off, x @ _dec(W_off).T + b_off.astype(np.float64), 1e-13, "offsets")
    _close(lg, x @ _dec(W_att).T + b_att.astype(np.float64), 1e-13, "logits")
    off0, _ = oracle.query_proj(q, None, W_off, None, W_att, None)
    _close(off0, _dec(_tobf(q)) @ _dec(W_off).T, 1e-13, "no embedding, no bias")
    # 1 + 2^-8 is a bf16 tie (rounds to 1.0); + 2^-30 is lost in float32 but
    # would lift an exact sum above the tie (to 1 + 2^-7)
    q1 = np.full((1, K), 1.0 + 2.0 ** -8, np.float32)
    e1 = np.full((1, K), 2.0 ** -30, np.float32)
    eye = _tobf(np.eye(K))
    got, _ = oracle.query_proj(q1, e1, eye, None, eye, None)
    _close(got, np.ones((1, K)), 0.0, "float32 sum rounded to bf16")


def pin_output_proj_layer_norm():
    """Output projection, residual and the layer norm ([8-heads] 11, 18.6-7):
    against torch's float64 layer_norm of residual + (decoded bf16 matmul +
    bias); a closed form (a row of +a/-a has mean 0 and variance a^2, so it
    maps to +-a/sqrt(a^2+eps) * gamma + beta); without gamma, the plain sum."""
    import torch
    g = np.random.default_rng(141)
    M, K, N = 9, 32, 24
    slots = g.normal(size=(M, K)).astype(np.float32)
    W = _tobf(g.normal(size=(N, K)) / 6)
    bias = g.normal(size=N).astype(np.float32)
    res = g.normal(size=(M, N)).astype(np.float32)
    gamma = g.uniform(0.5, 2.0, N).astype(np.float32)
    beta = g.normal(size=N).astype(np.float32)
    o = _dec(_tobf(slots)) @ _dec(W).T + bias.astype(np.float64)
    _close(oracle.output_proj(slots, W, bias), o, 1e-13, "projection")
    _close(oracle.output_proj(slots, W, bias, res), o + res, 1e-13, "residual")
    for eps in (1e-5, 0.25):
        ref = torch.nn.functional.layer_norm(torch.from_numpy(o + res), (N,), torch.from_numpy(gamma).double(),
                                             torch.from_numpy(beta).double(), eps).numpy()
        _close(oracle.output_proj(slots, W, bias, res, gamma, beta, eps), ref, 1e-12, f"layer norm eps={eps}")
    a, eps = 0.75, 0.0625
    row = np.where(np.arange(N) % 2 == 0, a, -a).astype(np.float32)[None, :]
    zeroW = np.zeros((N, K), np.uint16)
    got = oracle.output_proj(slots[:1], zeroW, None, row, np.full(N, 2.0, np.float32),
                             np.full(N, 0.5, np.float32), eps)
    _close(got, np.sign(row) * 2.0 * a / np.sqrt(a * a + eps) + 0.5, 1e-14, "alternating row")


# ---------------------------------------------------------------------------
# backward pass: derivatives of the forward definitions ([8-heads] 4.3 says
# only that offsets and weights are learned by back-propagation)
# ---------------------------------------------------------------------------

_STEP = 2.0 ** -10  # float32-exact step for locations / logits


def _interior_coord(g, n, size, lo=0.3, hi=0.7, outside=0.15):
    """Continuous coordinates on a map of `size` cells whose fractional part
    lies in [lo, hi] (so a step of at most 1/128 cell stays in the cell, where
    bilinear sampling is linear); a share of them in the cell left of the map
    (corner -1 outside) or right of it, to cover zero padding."""
    cell = g.integers(0, size, n).astype(np.float64)
    edge = g.random(n) < outside
    cell[edge] = np.where(g.random(int(edge.sum())) < 0.5, -1.0, float(size - 1))
    return cell + g.uniform(lo, hi, n)


def _bwd_msda_case(seed, B=2, Nq=4, shapes=((5, 8), (3, 4)), nH=3, Dh=4, P=3):
    ss, starts, Nv = level_table(shapes)
    L = len(ss)
    g = np.random.default_rng(seed)
    value = g.normal(size=(B, Nv, nH, Dh)).astype(np.float32)
    loc = np.zeros((B, Nq, nH, L, P, 2), np.float64)
    for l in range(L):
        H, W = ss[l]
        n = B * Nq * nH * P
        x = _interior_coord(g, n, W).reshape(B, Nq, nH, P)
        y = _interior_coord(g, n, H).reshape(B, Nq, nH, P)
        loc[:, :, :, l, :, 0] = (x + 0.5) / W
        loc[:, :, :, l, :, 1] = (y + 0.5) / H
    loc = (np.round(loc * 2.0 ** 20) / 2.0 ** 20).astype(np.float32)  # s +- step stays exact in float32
    logits = (np.round(g.normal(size=(B, Nq, nH, L * P)) * 2.0 ** 12) / 2.0 ** 12).astype(np.float32)
    probs = (np.round(g.uniform(0.0, 0.5, size=(B, Nq, nH, L * P)) * 2.0 ** 12) / 2.0 ** 12).astype(np.float32)
    grad_out = g.normal(size=(B, Nq, nH * Dh)).astype(np.float32)
    return value, ss, starts, loc, logits, probs, grad_out


def _loss(grad_out, out):
    return float(np.sum(grad_out.reshape(out.shape).astype(np.float64) * out))


def pin_msda_backward():
    """MSDA gradients against facts outside the backward code: the output is
    linear in the value and in the probabilities (adjoint identities); central
    differences of the forward oracle in every location coordinate (exact: the
    sampled function is linear inside a cell) and in every logit; the gradient
    through a softmax sums to zero over a head."""
    value, ss, starts, loc, logits, probs, gout = _bwd_msda_case(151)
    g = np.random.default_rng(152)
    for weights, are_logits in ((logits, True), (probs, False)):
        gv, gl, gw = oracle.msda_backward(value, ss, starts, loc, weights, gout, weights_are_logits=are_logits)
        fwd = lambda v=value, lc=loc, w=weights: oracle.msda(v, ss, starts, lc, w, weights_are_logits=are_logits)
        dv = g.normal(size=value.shape).astype(np.float32)
        _close(np.sum(gv * dv), _loss(gout, fwd(v=dv)), 1e-11, "value adjoint")
        if not are_logits:
            da = g.normal(size=probs.shape).astype(np.float32)
            _close(np.sum(gw * da), _loss(gout, fwd(w=da)), 1e-11, "probability adjoint")
        else:
            _close(gw.reshape(-1, gw.shape[-1]).sum(-1), np.zeros(gw.size // gw.shape[-1]), 1e-13,
                   "softmax gradient sums to zero")
        fd = np.zeros(loc.size)
        for i in range(loc.size):
            up, dn = loc.copy().reshape(-1), loc.copy().reshape(-1)
            up[i] += _STEP
            dn[i] -= _STEP
            fd[i] = (_loss(gout, fwd(lc=up.reshape(loc.shape))) -
                     _loss(gout, fwd(lc=dn.reshape(loc.shape)))) / (2 * _STEP)
        _close(gl.reshape(-1), fd, 1e-9, "location central differences")
        if are_logits:
            fd = np.zeros(weights.size)
            for i in range(weights.size):
                up, dn = weights.copy().reshape(-1), weights.copy().reshape(-1)
                up[i] += _STEP
                dn[i] -= _STEP
                fd[i] = (_loss(gout, fwd(w=up.reshape(weights.shape))) -
                         _loss(gout, fwd(w=dn.reshape(weights.shape)))) / (2 * _STEP)
            _close(gw.reshape(-1), fd, 2e-6, "logit central differences")


def pin_msda_frames_backward():
    """Gradients of the frame mean (F = 3, not a power of two) against its
    forward oracle: the value adjoint identity, and central differences of
    msda_frames in every location coordinate and every logit."""
    F = 3
    cases = [_bwd_msda_case(161 + f, B=1, Nq=3, shapes=((4, 6), (2, 3)), nH=2, Dh=4, P=2) for f in range(F)]
    value = np.stack([c[0] for c in cases], 1)  # [B, F, Nv, nH, Dh]
    ss, starts = cases[0][1], cases[0][2]
    loc = np.stack([c[3] for c in cases], 1)
    logits = np.stack([c[4] for c in cases], 1)
    gout = cases[0][6]
    gv, gl, gw = oracle.msda_frames_backward(value, ss, starts, loc, logits, gout)
    fwd = lambda v=value, lc=loc, w=logits: oracle.msda_frames(v, ss, starts, lc, w)
    dv = np.random.default_rng(162).normal(size=value.shape).astype(np.float32)
    _close(np.sum(gv * dv), _loss(gout, fwd(v=dv)), 1e-11, "frames value adjoint")
    for arr, grad, tol, what in ((loc, gl, 1e-9, "frames location central differences"),
                                 (logits, gw, 2e-6, "frames logit central differences")):
        fd = np.zeros(arr.size)
        for i in range(arr.size):
            up, dn = arr.copy().reshape(-1), arr.copy().reshape(-1)
            up[i] += _STEP
            dn[i] -= _STEP
            kw_up = {"lc": up.reshape(arr.shape)} if arr is loc else {"w": up.reshape(arr.shape)}
            kw_dn = {"lc": dn.reshape(arr.shape)} if arr is loc else {"w": dn.reshape(arr.shape)}
            fd[i] = (_loss(gout, fwd(**kw_up)) - _loss(gout, fwd(**kw_dn))) / (2 * _STEP)
        _close(grad.reshape(-1), fd, tol, what)


def _bwd_sca_case(seed, B=2, Ncam=3, Nq=6, shapes=((6, 8), (3, 4)), nH=2, Dh=4, P=4, D=2):
    ss, starts, Nv = level_table(shapes)
    L = len(ss)
    g = np.random.default_rng(seed)
    value = g.normal(size=(B, Ncam, Nv, nH, Dh)).astype(np.float32)
    mask = (g.random((Ncam, B, Nq, D)) < 0.45).astype(np.uint8)
    mask[:, 0, 0] = 0  # a query no camera sees
    mask[:, 1, 1] = 1  # a query every camera sees
    # anchors at exact multiples of 1/64 of the unit square; offsets in cells
    # so that every x = W*rho + dx - 1/2 has a fractional part in [0.3, 0.7]
    rho = (g.integers(8, 56, size=(Ncam, B, Nq, D, 2)) / 64.0).astype(np.float32)
    off = np.zeros((B, Nq, nH, L, P, 2), np.float64)
    for l in range(L):
        H, W = ss[l]
        for ax, size in ((0, W), (1, H)):
            base = rho[..., ax].astype(np.float64) * size - 0.5  # [Ncam, B, Nq, D]
            # one offset per (b, q, h, point) must suit every camera: pick the
            # fraction against camera 0's anchor and check the others below
            want = np.floor(base[0]) + g.uniform(0.3, 0.7, base[0].shape)  # [B, Nq, D]
            for k in range(P):
                off[:, :, :, l, k, ax] = (want[:, :, None, k % D] - base[0][:, :, None, k % D]
                                          + g.integers(-2, 3, (B, Nq, nH)))
    off = (np.round(off * 2.0 ** 12) / 2.0 ** 12).astype(np.float32)
    logits = (np.round(g.normal(size=(B, Nq, nH, L * P)) * 2.0 ** 12) / 2.0 ** 12).astype(np.float32)
    grad = g.normal(size=(B, Nq, nH * Dh)).astype(np.float32)
    return value, ss, starts, rho, mask, off, logits, grad


def pin_sca_backward():
    """SCA gradients: linear in the value (adjoint identity); central
    differences in every offset coordinate whose sample stays inside its cell
    for every camera (exact) and in every logit; zero for a query no camera
    sees; the gradient through each head's softmax sums to zero."""
    value, ss, starts, rho, mask, off, logits, gout = _bwd_sca_case(161)
    gv, goff, glg = oracle.sca_backward(value, ss, starts, rho, mask, off, logits, gout)
    fwd = lambda v=value, o=off, lg=logits: oracle.sca(v, ss, starts, rho, mask, o, lg)["slots"]
    dv = np.random.default_rng(162).normal(size=value.shape).astype(np.float32)
    _close(np.sum(gv * dv), _loss(gout, fwd(v=dv)), 1e-11, "value adjoint")
    assert not goff[0, 0].any() and not glg[0, 0].any(), "unseen query has a gradient"
    _close(glg.reshape(-1, glg.shape[-1]).sum(-1), np.zeros(glg.size // glg.shape[-1]), 1e-13, "softmax sums")
    step = 2.0 ** -8
    W_ = np.array([s[1] for s in ss], np.float64)
    H_ = np.array([s[0] for s in ss], np.float64)
    B, Ncam, Nv, nH, Dh = value.shape
    Nq, D = rho.shape[2], rho.shape[3]
    checked = 0
    for idx in np.ndindex(off.shape):
        b, q, h, l, k, ax = idx
        size = W_[l] if ax == 0 else H_[l]
        base = rho[:, b, q, k % D, ax].astype(np.float64) * size + off[idx] - 0.5  # x per camera
        frac = base - np.floor(base)
        if np.any((frac < 0.1) | (frac > 0.9)):
            continue  # a camera's sample sits near a cell edge: the step could cross it
        up, dn = off.copy(), off.copy()
        up[idx] += step
        dn[idx] -= step
        fd = (_loss(gout, fwd(o=up)) - _loss(gout, fwd(o=dn))) / (2 * step)
        _close(goff[idx], fd, 1e-9, f"offset central difference {idx}")
        checked += 1
    assert checked > off.size // 2, checked
    for idx in list(np.ndindex(logits.shape))[::3]:
        up, dn = logits.copy(), logits.copy()
        up[idx] += _STEP
        dn[idx] -= _STEP
        fd = (_loss(gout, fwd(lg=up)) - _loss(gout, fwd(lg=dn))) / (2 * _STEP)
        _close(glg[idx], fd, 2e-6, f"logit central difference {idx}")


ALL_PINS = [
    pin_worked_example_two_heads,
    pin_scalar_times_sample,
    pin_zero_logits_give_plain_mean,
    pin_softmax_invariants,
    pin_integer_aligned_exact_gather,
    pin_constant_map_inside,
    pin_affine_ramp_exact,
    pin_grid_sample_special_case,
    pin_dense_reformulation,
    pin_frames_mean,
    pin_sca_compaction_brute_force,
    pin_sca_exact_gather_and_camera_mean,
    pin_sca_dense_reformulation,
    pin_sca_rebatch_equals_fused_on_exact_locations,
    pin_bf16_rounding,
    pin_linear_bf16,
    pin_query_proj,
    pin_output_proj_layer_norm,
    pin_msda_backward,
    pin_msda_frames_backward,
    pin_sca_backward,
]
