"""CPU oracle for multi-scale deformable attention and spatial cross-attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code with the HIP library and imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain loops, IEEE double); this module
only marshals numpy arrays into it, apart from three compositions written
out here: ``linear_bf16_blas`` (the bf16 projection with a float64 matmul as
its contraction step), ``msda_frames_backward`` (each frame's
``msda_backward``, divided by the frame count) and ``sca_rebatch`` (the SCA
note's padded flow: the compaction's segments, float32 locations, the
operator over every padded row, the scatter-add and the divide).  Every
function returns float64 arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def use_library(path):
    """Load the oracle from another build of oracle.c (the mutation tests
    compile copies with planted mistakes).  None restores the default."""
    global _lib
    _lib = None
    if path is not None:
        _load(path)


def _load(path=None):
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_msda.argtypes = [_p, _int, _p, _p, _p, _p, _int, _i64, _i64, _i64, _int, _int, _int, _int,
                                _p, _i64, _p]
    lib.oracle_msda_frames.argtypes = [_p, _int, _p, _p, _p, _p, _int, _i64, _i64, _i64, _i64, _int, _int,
                                       _int, _int, _p, _i64, _p]
    lib.oracle_sca.argtypes = [_p, _int, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int, _int,
                               _int, _int, _p, _i64, _p, _p, _p, _p]
    lib.oracle_linear_bf16.argtypes = [_p, _int, _p, _p, _i64, _i64, _i64, _p]
    lib.oracle_query_proj.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _i64, _p, _p]
    lib.oracle_output_proj.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_double, _i64, _i64, _i64, _p]
    lib.oracle_msda_backward.argtypes = [_p, _int, _p, _p, _p, _p, _int, _p, _i64, _i64, _i64, _int, _int, _int,
                                         _int, _p, _p, _p]
    lib.oracle_sca_backward.argtypes = [_p, _int, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int,
                                        _int, _int, _int, _p, _p, _p]
    lib.oracle_round_to_bf16.argtypes = [_p, _i64, _p]
    lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_double_to_bf16.restype = ctypes.c_uint16
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    for f in (lib.oracle_msda, lib.oracle_msda_frames, lib.oracle_sca, lib.oracle_linear_bf16,
              lib.oracle_query_proj, lib.oracle_output_proj, lib.oracle_msda_backward, lib.oracle_sca_backward):
        f.restype = _int
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(_p)


def _value(value):
    """float32 array, or uint16 array holding bfloat16 bit patterns."""
    if value.dtype == np.uint16:
        v, p = _c(value, np.uint16)
        return v, p, 1
    v, p = _c(value, np.float32)
    return v, p, 0


def _rows(rows, total):
    if rows is None:
        return None, None, total
    r, p = _c(rows, np.int64)
    return r, p, len(r)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: oracle rejected its arguments (code {rc})")


def msda(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
         weights_are_logits=False, rows=None):
    """MSDA operator.  value [B,Nv,nH,Dh]; locations [B,Nq,nH,L,P,2];
    weights [B,Nq,nH,L*P].  Returns [len(rows) or B*Nq, nH*Dh] float64."""
    lib = _load()
    B, Nv, nH, Dh = value.shape
    _, Nq, _, L, P, _ = sampling_locations.shape
    v, vp, vb = _value(value)
    ss, ssp = _c(spatial_shapes, np.int64)
    ls, lsp = _c(level_start_index, np.int64)
    loc, locp = _c(sampling_locations, np.float32)
    w, wp = _c(attention_weights, np.float32)
    r, rp, n = _rows(rows, B * Nq)
    out = np.zeros((n, nH * Dh), np.float64)
    rc = lib.oracle_msda(vp, vb, ssp, lsp, locp, wp, int(bool(weights_are_logits)), B, Nv, Nq, nH, Dh, L, P,
                         rp, n, out.ctypes.data_as(_p))
    _check(rc, "oracle_msda")
    del v, ss, ls, loc, w, r
    return out


def msda_frames(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
                weights_are_logits=True, rows=None):
    """Mean over F frames of per-frame MSDA.  value [B,F,Nv,nH,Dh];
    locations [B,F,Nq,nH,L,P,2]; weights [B,F,Nq,nH,L*P].  Returns
    [len(rows) or B*Nq, nH*Dh] float64."""
    lib = _load()
    B, F, Nv, nH, Dh = value.shape
    _, _, Nq, _, L, P, _ = sampling_locations.shape
    v, vp, vb = _value(value)
    ss, ssp = _c(spatial_shapes, np.int64)
    ls, lsp = _c(level_start_index, np.int64)
    loc, locp = _c(sampling_locations, np.float32)
    w, wp = _c(attention_weights, np.float32)
    r, rp, n = _rows(rows, B * Nq)
    out = np.zeros((n, nH * Dh), np.float64)
    rc = lib.oracle_msda_frames(vp, vb, ssp, lsp, locp, wp, int(bool(weights_are_logits)), B, F, Nv, Nq, nH,
                                Dh, L, P, rp, n, out.ctypes.data_as(_p))
    _check(rc, "oracle_msda_frames")
    del v, ss, ls, loc, w, r
    return out


def sca(value, spatial_shapes, level_start_index, reference_points_cam, bev_mask, sampling_offsets,
        attention_logits, rows=None, want_slots=True):
    """Spatial cross-attention.  value [B,Ncam,Nv,nH,Dh]; reference_points_cam
    [Ncam,B,Nq,D,2]; bev_mask [Ncam,B,Nq,D]; sampling_offsets [B,Nq,nH,L,P,2];
    attention_logits [B,Nq,nH,L*P].

    Returns dict with slots [n,nH*Dh] float64 (None unless want_slots),
    hit_count [B,Nq] int32, pair_offsets [B*Ncam+1] int32, pair_q [Npairs] int32.
    """
    lib = _load()
    B, Ncam, Nv, nH, Dh = value.shape
    _, _, Nq, D, _ = reference_points_cam.shape
    _, _, _, L, P, _ = sampling_offsets.shape
    v, vp, vb = _value(value)
    ss, ssp = _c(spatial_shapes, np.int64)
    ls, lsp = _c(level_start_index, np.int64)
    rpc, rpcp = _c(reference_points_cam, np.float32)
    bm, bmp = _c(bev_mask, np.uint8)
    off, offp = _c(sampling_offsets, np.float32)
    lg, lgp = _c(attention_logits, np.float32)
    r, rp, n = _rows(rows, B * Nq)
    slots = np.zeros((n, nH * Dh), np.float64) if want_slots else None
    hit = np.zeros((B, Nq), np.int32)
    offs = np.zeros(B * Ncam + 1, np.int32)
    pq = np.zeros(max(1, B * Ncam * Nq), np.int32)
    rc = lib.oracle_sca(vp, vb, ssp, lsp, rpcp, bmp, offp, lgp, B, Ncam, Nv, Nq, nH, Dh, L, P, D, rp, n,
                        slots.ctypes.data_as(_p) if want_slots else None, hit.ctypes.data_as(_p),
                        offs.ctypes.data_as(_p), pq.ctypes.data_as(_p))
    _check(rc, "oracle_sca")
    del v, ss, ls, rpc, bm, off, lg, r
    return {"slots": slots, "hit_count": hit, "pair_offsets": offs, "pair_q": pq[: int(offs[-1])].copy()}


def linear_bf16(X, W, bias=None):
    """Y = X W^T + bias in float64 from bf16 operands.  X: uint16 bf16 bits
    [M,K], or float32 [M,K] (rounded to the nearest bf16 first).  W: uint16
    [N,K].  bias: float32 [N] or None."""
    lib = _load()
    M, K = X.shape
    N = W.shape[0]
    if X.dtype == np.uint16:
        x, xp = _c(X, np.uint16)
        xf = 0
    else:
        x, xp = _c(X, np.float32)
        xf = 1
    w, wp = _c(W, np.uint16)
    if bias is not None:
        b, bp = _c(bias, np.float32)
    else:
        b, bp = None, None
    Y = np.zeros((M, N), np.float64)
    rc = lib.oracle_linear_bf16(xp, xf, wp, bp, M, N, K, Y.ctypes.data_as(_p))
    _check(rc, "oracle_linear_bf16")
    del x, w, b
    return Y


def msda_backward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights, grad_out,
                  weights_are_logits=False):
    """Gradients of msda() for d loss / d out = grad_out [B,Nq,nH*Dh].
    Returns (grad_value [B,Nv,nH,Dh], grad_locations [B,Nq,nH,L,P,2],
    grad_weights [B,Nq,nH,L*P]) float64; grad_weights is with respect to the
    weights as given (logits or probabilities)."""
    lib = _load()
    B, Nv, nH, Dh = value.shape
    _, Nq, _, L, P, _ = sampling_locations.shape
    v, vp, vb = _value(value)
    ss, ssp = _c(spatial_shapes, np.int64)
    ls, lsp = _c(level_start_index, np.int64)
    loc, locp = _c(sampling_locations, np.float32)
    w, wp = _c(attention_weights, np.float32)
    go, gop = _c(grad_out, np.float32)
    gv = np.zeros((B, Nv, nH, Dh), np.float64)
    gl = np.zeros((B, Nq, nH, L, P, 2), np.float64)
    gw = np.zeros((B, Nq, nH, L * P), np.float64)
    rc = lib.oracle_msda_backward(vp, vb, ssp, lsp, locp, wp, int(bool(weights_are_logits)), gop, B, Nv, Nq, nH, Dh,
                                  L, P, gv.ctypes.data_as(_p), gl.ctypes.data_as(_p), gw.ctypes.data_as(_p))
    _check(rc, "oracle_msda_backward")
    del v, ss, ls, loc, w, go
    return gv, gl, gw


def msda_frames_backward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights, grad_out,
                         weights_are_logits=True):
    """Gradients of msda_frames() for d loss / d out = grad_out [B,Nq,nH*Dh].
    out is the mean of the F per-frame operators, so frame f's gradients are
    msda_backward()'s of that frame for grad_out, divided by F (the division
    is done on the float64 results: exact).  Returns (grad_value
    [B,F,Nv,nH,Dh], grad_locations [B,F,Nq,nH,L,P,2], grad_weights
    [B,F,Nq,nH,L*P]) float64."""
    B, F, Nv, nH, Dh = value.shape
    _, _, Nq, _, L, P, _ = sampling_locations.shape
    gv = np.zeros((B, F, Nv, nH, Dh), np.float64)
    gl = np.zeros((B, F, Nq, nH, L, P, 2), np.float64)
    gw = np.zeros((B, F, Nq, nH, L * P), np.float64)
    for f in range(F):
        v, l, w = msda_backward(value[:, f], spatial_shapes, level_start_index, sampling_locations[:, f],
                                attention_weights[:, f], grad_out, weights_are_logits=weights_are_logits)
        gv[:, f], gl[:, f], gw[:, f] = v / F, l / F, w / F
    return gv, gl, gw


def sca_backward(value, spatial_shapes, level_start_index, reference_points_cam, bev_mask, sampling_offsets,
                 attention_logits, grad_slots):
    """Gradients of sca() for d loss / d slots = grad_slots [B,Nq,nH*Dh].
    Returns (grad_value [B,Ncam,Nv,nH,Dh], grad_offsets [B,Nq,nH,L,P,2],
    grad_logits [B,Nq,nH,L*P]) float64."""
    lib = _load()
    B, Ncam, Nv, nH, Dh = value.shape
    _, _, Nq, D, _ = reference_points_cam.shape
    _, _, _, L, P, _ = sampling_offsets.shape
    v, vp, vb = _value(value)
    ss, ssp = _c(spatial_shapes, np.int64)
    ls, lsp = _c(level_start_index, np.int64)
    rpc, rpcp = _c(reference_points_cam, np.float32)
    bm, bmp = _c(bev_mask, np.uint8)
    off, offp = _c(sampling_offsets, np.float32)
    lg, lgp = _c(attention_logits, np.float32)
    go, gop = _c(grad_slots, np.float32)
    gv = np.zeros((B, Ncam, Nv, nH, Dh), np.float64)
    goff = np.zeros((B, Nq, nH, L, P, 2), np.float64)
    glg = np.zeros((B, Nq, nH, L * P), np.float64)
    rc = lib.oracle_sca_backward(vp, vb, ssp, lsp, rpcp, bmp, offp, lgp, gop, B, Ncam, Nv, Nq, nH, Dh, L, P, D,
                                 gv.ctypes.data_as(_p), goff.ctypes.data_as(_p), glg.ctypes.data_as(_p))
    _check(rc, "oracle_sca_backward")
    del v, ss, ls, rpc, bm, off, lg, go
    return gv, goff, glg


def _opt(a, dtype):
    if a is None:
        return None, None
    return _c(a, dtype)


def query_proj(query, query_pos, W_off, b_off, W_att, b_att):
    """Sampling offsets and attention logits from the query: q~ = query +
    query_pos in float32, then W_off q~ + b_off and W_att q~ + b_att from bf16
    operands.  query, query_pos float32 [M,K] (query_pos may be None);
    W_* uint16 bf16 bits [N_*,K]; b_* float32 [N_*] or None.  Returns
    (offsets [M,N_off], logits [M,N_att]) float64."""
    lib = _load()
    M, K = query.shape
    N_off, N_att = W_off.shape[0], W_att.shape[0]
    q, qp = _c(query, np.float32)
    e, ep = _opt(query_pos, np.float32)
    wo, wop = _c(W_off, np.uint16)
    bo, bop = _opt(b_off, np.float32)
    wa, wap = _c(W_att, np.uint16)
    ba, bap = _opt(b_att, np.float32)
    off = np.zeros((M, N_off), np.float64)
    lg = np.zeros((M, N_att), np.float64)
    rc = lib.oracle_query_proj(qp, ep, M, K, wop, bop, N_off, wap, bap, N_att, off.ctypes.data_as(_p),
                               lg.ctypes.data_as(_p))
    _check(rc, "oracle_query_proj")
    del q, e, wo, bo, wa, ba
    return off, lg


def output_proj(slots, W, bias=None, residual=None, gamma=None, beta=None, eps=1e-5):
    """residual + (W bf16(slots) + bias), then the layer norm with gamma and
    beta when gamma is given.  slots float32 [M,K]; W uint16 [N,K]; bias,
    gamma, beta float32 [N] or None; residual float32 [M,N] or None.
    Returns [M,N] float64."""
    lib = _load()
    M, K = slots.shape
    N = W.shape[0]
    x, xp = _c(slots, np.float32)
    w, wp = _c(W, np.uint16)
    b, bp = _opt(bias, np.float32)
    r, rp = _opt(residual, np.float32)
    g, gp = _opt(gamma, np.float32)
    be, bep = _opt(beta, np.float32)
    Y = np.zeros((M, N), np.float64)
    rc = lib.oracle_output_proj(xp, wp, bp, rp, gp, bep, float(eps), M, N, K, Y.ctypes.data_as(_p))
    _check(rc, "oracle_output_proj")
    del x, w, b, r, g, be
    return Y


def linear_bf16_blas(X, W, bias=None):
    """Same as linear_bf16 for bf16-bit X, with the library float64 matmul as
    the contraction step (for the full-size value projection, which plain
    loops would take minutes for).  Decoding bf16 is exact, so only the
    summation order differs from the loop version."""
    assert X.dtype == np.uint16 and W.dtype == np.uint16
    dec = lambda bits: (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Y = dec(X) @ dec(W).T
    if bias is not None:
        Y += np.asarray(bias, np.float64)
    return Y


def round_to_bf16(x):
    """Nearest bf16 (ties to even) of each element, as uint16 bit patterns."""
    lib = _load()
    a, ap = _c(x, np.float64)
    out = np.zeros(a.shape, np.uint16)
    lib.oracle_round_to_bf16(ap, a.size, out.ctypes.data_as(_p))
    return out


def bf16_to_float64(bits):
    """Exact widening of bf16 bit patterns."""
    lib = _load()
    flat = np.ascontiguousarray(bits, np.uint16).ravel()
    return np.array([lib.oracle_bf16_to_double(int(b)) for b in flat], np.float64).reshape(np.shape(bits))


def sca_rebatch(value, spatial_shapes, level_start_index, reference_points_cam, bev_mask, sampling_offsets,
                attention_logits):
    """Spatial cross-attention through the padded flow of the Tencent Cloud
    SCA note (article 2321140: its rebatch code and its scatter / count /
    divide code), step by step:
      1. the compaction of sca(): per (batch item, camera), in b-major order,
         the ascending list of the queries the camera sees, and the hit counts;
      2. max_len = the longest list; every list is padded to it;
      3. rebatch: for row i of segment (b, c), query q = list[i], the sampling
         locations rho[c][b][q][p mod D] + (dx / W_l, dy / H_l) formed as the
         float32 tensor the operator takes ("BEV(三) BEVFormer：Query 参数如何与
         Feature 的 8 个 Head 交互", sections 5 and 18.4), and the query's logits;
         padded rows are zero;
      4. the operator msda() over the B*Ncam segments (value image b*Ncam + c);
      5. scatter: each camera, in ascending order, adds its segment's rows to
         the slots of its queries (padded rows are never added);
      6. count and divide: slots / max(1, hit count).
    Same arguments as sca().  Returns dict with sampling_locations
    [B*Ncam, max_len, nH, L, P, 2] float32, logits [B*Ncam, max_len, nH, L*P]
    float32, slots [B*Nq, nH*Dh] float64, max_len, and the compaction
    (hit_count, pair_offsets, pair_q)."""
    B, Ncam, Nv, nH, Dh = value.shape
    _, _, Nq, D, _ = reference_points_cam.shape
    _, _, _, L, P, _ = sampling_offsets.shape
    comp = sca(value, spatial_shapes, level_start_index, reference_points_cam, bev_mask, sampling_offsets,
               attention_logits, want_slots=False)
    offs, pq, hit = comp["pair_offsets"], comp["pair_q"], comp["hit_count"]
    max_len = int(np.diff(offs).max()) if offs.size > 1 else 0
    ss = np.asarray(spatial_shapes)
    WH = np.stack([ss[:, 1], ss[:, 0]], -1).astype(np.float32)  # (W, H) per level
    anchor = np.arange(P) % D
    loc = np.zeros((B * Ncam, max_len, nH, L, P, 2), np.float32)
    lg = np.zeros((B * Ncam, max_len, nH, L * P), np.float32)
    for b in range(B):
        for c in range(Ncam):
            bc = b * Ncam + c
            qs = pq[offs[bc]:offs[bc + 1]]
            rho = reference_points_cam[c, b][qs][:, anchor]  # [n, P, 2]
            loc[bc, :len(qs)] = rho[:, None, None] + sampling_offsets[b, qs] / WH[None, None, :, None, :]
            lg[bc, :len(qs)] = attention_logits[b, qs]
    C = nH * Dh
    slots = np.zeros((B * Nq, C), np.float64)
    if max_len > 0:
        rows = msda(value.reshape(B * Ncam, Nv, nH, Dh), spatial_shapes, level_start_index, loc, lg,
                    weights_are_logits=True).reshape(B * Ncam, max_len, C)
        for c in range(Ncam):
            for b in range(B):
                bc = b * Ncam + c
                qs = pq[offs[bc]:offs[bc + 1]]
                slots[b * Nq + qs] += rows[bc, :len(qs)]
    slots /= np.maximum(hit.reshape(-1), 1)[:, None]
    return {"sampling_locations": loc, "logits": lg, "slots": slots, "max_len": max_len, "hit_count": hit,
            "pair_offsets": offs, "pair_q": pq}
