"""Seeded synthetic inputs for the workloads (and smaller variants).

This module is shared by the tests, the smoke check and the benchmark.  It
draws random inputs only: it holds none of the method's arithmetic, imports
neither the oracle nor the HIP library, and both sides receive the very same
arrays.

Seeding: every tensor of a workload is drawn from its own generator
``np.random.default_rng(np.random.SeedSequence([cfg, tensor_id]))``, with
``cfg`` the workload's seed id, so a tensor does not change when another one
is added or resized.

Workloads (seed id, generator; shapes follow BEVFormer-base and a
Deformable-DETR encoder):
  1 tiny_msda           B=1, Nq=256, one 32x32 level, 8 heads x 32, P=4
  2 detr_encoder_msda   B=1, levels 100x150/50x75/25x38/13x19, Nq=Nv=19947, P=4
  3 bevformer_sca       B=1, 6 cameras, 200x200 BEV queries, levels
                        116x200/58x100/29x50/15x25, P=8, D=4 anchors, fp32 value
  4 temporal_frames     B=1, 2 stacked 200x200 BEV maps, one level, P=4 per frame
  5 bevformer_sca_bf16  the SCA layer at B=4 with bf16 projection input and weights;
    bevformer_layer_bf16 the same layer whole: offsets and logits projected
                        from the query, the output projection followed by the
                        residual and the layer norm
"""
import numpy as np

DETR_LEVELS = ((100, 150), (50, 75), (25, 38), (13, 19))
BEV_CAM_LEVELS = ((116, 200), (58, 100), (29, 50), (15, 25))

# tensor ids inside one workload's seed sequence
_T_VALUE, _T_REF, _T_OFF, _T_LOGIT, _T_MASK, _T_W_V, _T_W_O, _T_BIAS = range(8)
_T_QUERY, _T_QPOS, _T_W_OFF, _T_W_ATT, _T_NORM, _T_GRAD = range(8, 14)


def rng(cfg, tensor_id):
    return np.random.default_rng(np.random.SeedSequence([int(cfg), int(tensor_id)]))


def level_table(shapes):
    """spatial_shapes [L,2] as (H, W) rows and the start of each level in the
    flattened value axis (levels stored one after another, row-major)."""
    ss = np.asarray(shapes, np.int64).reshape(-1, 2)
    sizes = ss[:, 0] * ss[:, 1]
    starts = np.zeros(len(ss), np.int64)
    starts[1:] = np.cumsum(sizes)[:-1]
    return ss, starts, int(sizes.sum())


def bf16_bits_trunc(x):
    """Draw-time quantisation of a synthetic float32 tensor to bfloat16 bit
    patterns by keeping the upper 16 bits (round toward zero).  Only used to
    make random bf16 inputs."""
    x = np.ascontiguousarray(x, np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _normal(g, shape, scale=1.0):
    out = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def msda_workload(cfg, B, Nq, shapes, nH=8, Dh=32, P=4, value_bf16=False, ref="uniform",
                  offset_px=2.0):
    """Inputs of the MSDA operator.

    value ~ N(0,1) [B,Nv,nH,Dh]; reference point per query ~ U[0,1]^2
    (ref="uniform") or the BEV cell centre of the query (ref="grid", square
    grid of sqrt(Nq) cells); each (head, level, point) location is the
    reference point plus N(0, offset_px cells of that level) scatter;
    logits ~ N(0,1) [B,Nq,nH,L*P]; the reference points [B,Nq,2] are
    returned too.
    """
    ss, starts, Nv = level_table(shapes)
    L = len(ss)
    g = rng(cfg, _T_VALUE)
    value = _normal(g, (B, Nv, nH, Dh))
    if value_bf16:
        value = bf16_bits_trunc(value)
    r = _reference(cfg, B, Nq, ref)
    g = rng(cfg, _T_OFF)
    scatter = _normal(g, (B, Nq, nH, L, P, 2), offset_px)
    cells = np.stack([ss[:, 1], ss[:, 0]], axis=-1).astype(np.float32)  # (W, H) per level
    loc = r[:, :, None, None, None, :] + scatter / cells[None, None, None, :, None, :]
    g = rng(cfg, _T_LOGIT)
    logits = _normal(g, (B, Nq, nH, L * P))
    return {"value": value, "spatial_shapes": ss, "level_start_index": starts,
            "sampling_locations": loc.astype(np.float32), "attention_weights": logits,
            "reference_points": r.astype(np.float32),
            "B": B, "Nq": Nq, "Nv": Nv, "nH": nH, "Dh": Dh, "L": L, "P": P}


def _reference(cfg, B, Nq, kind):
    if kind == "uniform":
        return rng(cfg, _T_REF).random(size=(B, Nq, 2), dtype=np.float32)
    side = int(round(np.sqrt(Nq)))
    assert side * side == Nq, "grid reference points need a square query grid"
    i = np.arange(side, dtype=np.float64)
    cx, cy = np.meshgrid((i + 0.5) / side, (i + 0.5) / side)  # q = row*side + col
    r = np.stack([cx.ravel(), cy.ravel()], axis=-1).astype(np.float32)
    return np.broadcast_to(r, (B, Nq, 2)).copy()


def tiny_msda():
    """Tiny MSDA: B=1, 256 queries, one 32x32 level, 8x32, P=4."""
    return msda_workload(1, 1, 256, ((32, 32),), P=4)


def detr_encoder_msda():
    """Deformable-DETR encoder shapes, Nq = Nv = 19947, P=4."""
    w = msda_workload(2, 1, 19947, DETR_LEVELS, P=4)
    assert w["Nv"] == 19947
    return w


def temporal_frames(cfg=4, B=1, bev=200, F=2, nH=8, Dh=32, P=4):
    """F stacked BEV maps (one level bev x bev), BEV-centre
    reference points, per-frame offsets and logits.  Frames are an inner batch
    axis: value [B,F,Nv,nH,Dh], locations [B,F,Nq,nH,1,P,2],
    logits [B,F,Nq,nH,P]."""
    w = msda_workload(cfg, B * F, bev * bev, ((bev, bev),), nH=nH, Dh=Dh, P=P, ref="grid")
    Nq, Nv = w["Nq"], w["Nv"]
    w["value"] = w["value"].reshape(B, F, Nv, nH, Dh)
    w["sampling_locations"] = w["sampling_locations"].reshape(B, F, Nq, nH, 1, P, 2)
    w["attention_weights"] = w["attention_weights"].reshape(B, F, Nq, nH, P)
    w["B"], w["F"] = B, F
    return w


def camera_visibility(cfg, B, Ncam=6, bev=200, D=4, yaw_step_deg=60.0, half_fov_deg=35.0,
                      edge_jitter_deg=2.0, p_anchor=0.75):
    """bev_mask [Ncam,B,Nq,D] (uint8) and reference_points_cam [Ncam,B,Nq,D,2].

    Camera c looks along yaw c*yaw_step with a sector of +-half_fov; each
    sector edge is jittered by U(-j, j) degrees per (camera, batch item,
    query), so every query is seen by one or two cameras.  For a seeing
    camera, each anchor bit ~ Bernoulli(p_anchor), forced non-empty; x of the
    anchor is the query's azimuth position across the sector + N(0, 0.01);
    y = 0.5 + 0.1*(m - 1.5) + N(0, 0.02) for a marked anchor and U(1.05, 1.5)
    (below the image) for an unmarked one.  Cameras that do not see the query
    get arbitrary in-range points that are never read.
    """
    Nq = bev * bev
    g = rng(cfg, _T_MASK)
    i = np.arange(bev, dtype=np.float64)
    xs, ys = np.meshgrid(i, i)  # q = row*bev + col; x = col, y = row
    centre = (bev - 1) / 2.0
    phi = np.degrees(np.arctan2(ys - centre, xs - centre)).ravel()  # [Nq]
    mask = np.zeros((Ncam, B, Nq, D), np.uint8)
    rho = g.random(size=(Ncam, B, Nq, D, 2)).astype(np.float32)
    for b in range(B):
        for c in range(Ncam):
            d = (phi - c * yaw_step_deg + 180.0) % 360.0 - 180.0
            left = -half_fov_deg + g.uniform(-edge_jitter_deg, edge_jitter_deg, Nq)
            right = half_fov_deg + g.uniform(-edge_jitter_deg, edge_jitter_deg, Nq)
            seen = (d >= left) & (d <= right)
            bits = g.random((Nq, D)) < p_anchor
            empty = ~bits.any(axis=1)
            bits[empty, g.integers(0, D, size=int(empty.sum()))] = True
            bits &= seen[:, None]
            x = (d - left) / (right - left) + g.normal(0.0, 0.01, Nq)
            m = np.arange(D, dtype=np.float64)
            y_in = 0.5 + 0.1 * (m[None, :] - (D - 1) / 2.0) + g.normal(0.0, 0.02, (Nq, D))
            y_out = g.uniform(1.05, 1.5, (Nq, D))
            y = np.where(bits, y_in, y_out)
            sel = seen
            rho[c, b, sel, :, 0] = np.broadcast_to(x[sel, None], (int(sel.sum()), D))
            rho[c, b, sel, :, 1] = y[sel]
            mask[c, b] = bits
    return mask, rho


def bevformer_sca(cfg=3, B=1, Ncam=6, bev=200, shapes=BEV_CAM_LEVELS, nH=8, Dh=32, P=8, D=4,
                  value_bf16=False, offset_px=2.0):
    """BEVFormer-base SCA inputs (also the sampling part of the batch-4 bf16 layer).

    value ~ N(0,1) [B,Ncam,Nv,nH,Dh] (fp32, or bf16 bits by truncation);
    sampling_offsets ~ N(0, offset_px) cells [B,Nq,nH,L,P,2];
    attention_logits ~ N(0,1) [B,Nq,nH,L*P]; bev_mask and
    reference_points_cam from camera_visibility().
    """
    ss, starts, Nv = level_table(shapes)
    L = len(ss)
    Nq = bev * bev
    value = _normal(rng(cfg, _T_VALUE), (B, Ncam, Nv, nH, Dh))
    if value_bf16:
        value = bf16_bits_trunc(value)
    mask, rho = camera_visibility(cfg, B, Ncam=Ncam, bev=bev, D=D)
    offsets = _normal(rng(cfg, _T_OFF), (B, Nq, nH, L, P, 2), offset_px)
    logits = _normal(rng(cfg, _T_LOGIT), (B, Nq, nH, L * P))
    return {"value": value, "spatial_shapes": ss, "level_start_index": starts,
            "reference_points_cam": rho, "bev_mask": mask, "sampling_offsets": offsets,
            "attention_logits": logits, "B": B, "Ncam": Ncam, "Nq": Nq, "Nv": Nv, "nH": nH,
            "Dh": Dh, "L": L, "P": P, "D": D}


def projection_weights(cfg, C=256, bias=False):
    """W_v, W_o ~ N(0, 1/C) as bf16 bits [C,C]; biases zero, or N(0, 0.1)
    when bias=True (used by tests to exercise the bias term)."""
    wv = bf16_bits_trunc(_normal(rng(cfg, _T_W_V), (C, C), 1.0 / np.sqrt(C)))
    wo = bf16_bits_trunc(_normal(rng(cfg, _T_W_O), (C, C), 1.0 / np.sqrt(C)))
    if bias:
        g = rng(cfg, _T_BIAS)
        bv = _normal(g, (C,), 0.1)
        bo = _normal(g, (C,), 0.1)
    else:
        bv = np.zeros(C, np.float32)
        bo = np.zeros(C, np.float32)
    return wv, bv, wo, bo


def bevformer_sca_bf16(cfg=5, B=4, bev=200, shapes=BEV_CAM_LEVELS, bias=False, **kw):
    """Batch-4 SCA layer whose value comes from a bf16 value projection.
    Adds feat (bf16 bits [B,Ncam,Nv,256], N(0,1)), W_v/b_v/W_o/b_o; 'value' is
    left out: it is the projection's output."""
    w = bevformer_sca(cfg=cfg, B=B, bev=bev, shapes=shapes, **kw)
    B_, Ncam, Nv, nH, Dh = w["value"].shape
    del w["value"]
    C = nH * Dh
    w["feat"] = bf16_bits_trunc(_normal(rng(cfg, _T_VALUE), (B_, Ncam, Nv, C)))
    w["W_v"], w["b_v"], w["W_o"], w["b_o"] = projection_weights(cfg, C, bias=bias)
    return w


def bevformer_layer_bf16(cfg=5, B=4, bev=200, shapes=BEV_CAM_LEVELS, bias=False, offset_px=2.0, **kw):
    """The batch-4 bf16 layer widened to the whole attention layer: the sampling offsets
    and logits come from the query instead of being drawn.  Adds
    query, query_pos ~ N(0,1) float32 [B,Nq,256]; W_off bf16 [nH*L*P*2, 256]
    ~ N(0, offset_px^2 / 512) and W_att bf16 [nH*L*P, 256] ~ N(0, 1/512), so
    that with q~ = query + query_pos (variance 2) the offsets have the
    N(0, offset_px) cells and the logits the N(0, 1) of the BEVFormer-base SCA workload; biases
    zero (or N(0, 0.1) with bias=True); layer-norm gamma ~ 1 + N(0, 0.1) and
    beta ~ N(0, 0.1).  The drawn sampling_offsets / attention_logits are
    removed."""
    w = bevformer_sca_bf16(cfg=cfg, B=B, bev=bev, shapes=shapes, bias=bias, offset_px=offset_px, **kw)
    del w["sampling_offsets"], w["attention_logits"]
    B_, Nq, nH, L, P = w["B"], w["Nq"], w["nH"], w["L"], w["P"]
    C = nH * w["Dh"]
    w["query"] = _normal(rng(cfg, _T_QUERY), (B_, Nq, C))
    w["query_pos"] = _normal(rng(cfg, _T_QPOS), (B_, Nq, C))
    n_off, n_att = nH * L * P * 2, nH * L * P
    w["W_off"] = bf16_bits_trunc(_normal(rng(cfg, _T_W_OFF), (n_off, C), offset_px / np.sqrt(2.0 * C)))
    w["W_att"] = bf16_bits_trunc(_normal(rng(cfg, _T_W_ATT), (n_att, C), 1.0 / np.sqrt(2.0 * C)))
    if bias:
        g = rng(cfg, _T_BIAS + 100)
        w["b_off"], w["b_att"] = _normal(g, (n_off,), 0.1), _normal(g, (n_att,), 0.1)
    else:
        w["b_off"], w["b_att"] = np.zeros(n_off, np.float32), np.zeros(n_att, np.float32)
    g = rng(cfg, _T_NORM)
    w["gamma"] = (1.0 + _normal(g, (C,), 0.1)).astype(np.float32)
    w["beta"] = _normal(g, (C,), 0.1)
    return w


def upstream_gradient(cfg, shape):
    """d loss / d output for the backward pass: N(0, 1) float32 of `shape`,
    drawn from its own generator of workload `cfg`."""
    return _normal(rng(cfg, _T_GRAD), shape)


def sample_rows(cfg, total, n):
    """n distinct row indices in [0, total), sorted, seeded by workload."""
    n = min(n, total)
    return np.sort(rng(cfg, 99).choice(total, size=n, replace=False)).astype(np.int64)
