"""libmsda.so on a machine without a GPU: the library loads, exports every
entry point include/msda.h declares, and rejects bad arguments with the
documented status before touching any device (no compute call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msda.h")

OK, INVALID, UNSUPPORTED, SHAPE, WORKSPACE, HIP = 0, 1, 2, 3, 4, 5

_p, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t

# fake, never dereferenced, suitably aligned addresses: every call below must
# fail validation before any access
A = 0x10000
B_ = 0x20000
MIS = 0x10004  # 4-byte but not 16-byte aligned


@pytest.fixture(scope="module")
def lib():
    import scale_deformable_attention_forward_amd as m
    if not os.path.exists(m.library_path()):
        from scale_deformable_attention_forward_amd import build
        build.build()
    return m.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


# the calls the boundary is planned around: the operator, the SCA workspace
# query, the SCA forward, the bf16 projection and the status names
PLANNED_BOUNDARY = ["msda_forward", "sca_plan_workspace", "sca_forward", "msda_gemm_bf16", "msda_status_string"]


def test_header_declares_the_planned_boundary_names():
    names = declared_functions()
    for n in PLANNED_BOUNDARY:
        assert n in names, n


def test_plan_workspace_equals_workspace_size(lib):
    for B, Ncam, Nq in [(1, 6, 40000), (4, 6, 40000), (2, 1, 0), (3, 32, 17)]:
        a, b = _sz(0), _sz(0)
        assert lib.sca_plan_workspace(B, Ncam, Nq, ctypes.byref(a)) == OK
        assert lib.sca_workspace_size(B, Ncam, Nq, ctypes.byref(b)) == OK
        assert a.value == b.value > 0
    assert lib.sca_plan_workspace(0, 6, 10, ctypes.byref(_sz(0))) == INVALID
    assert lib.sca_plan_workspace(1, 6, 10, None) == INVALID


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["msda_forward", "msda_forward_frames", "sca_workspace_size", "sca_forward", "msda_gemm_bf16",
              "msda_query_proj_bf16", "msda_output_proj_bf16", "sca_rebatch", "sca_scatter_mean",
              "msda_backward", "msda_backward_frames", "sca_backward", "msda_backward_workspace_size",
              "sca_backward_workspace_size",
              "msda_status_string", "msda_last_error"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in msda.h but not exported"


def test_binding_has_every_entry_point_by_name():
    """The Python binding carries the C entry points under the same names."""
    import scale_deformable_attention_forward_amd as m
    for name in declared_functions():
        assert name in m.__all__ and callable(getattr(m, name)), f"{name} missing from the binding"


def test_status_strings(lib):
    for code, name in [(OK, "MSDA_OK"), (INVALID, "MSDA_ERR_INVALID_ARG"), (UNSUPPORTED, "MSDA_ERR_UNSUPPORTED"),
                       (SHAPE, "MSDA_ERR_SHAPE"), (WORKSPACE, "MSDA_ERR_WORKSPACE"), (HIP, "MSDA_ERR_HIP")]:
        assert lib.msda_status_string(code).decode() == name
    assert lib.msda_status_string(99).decode() == "MSDA_ERR_UNKNOWN"


def _msda(lib, value=A, dtype=0, shapes=A, starts=A, loc=A, w=A, mode=1, B=1, Nv=16, Nq=4, nH=8, Dh=32, L=1,
          P=4, out=B_):
    return lib.msda_forward(value, dtype, shapes, starts, loc, w, mode, B, Nv, Nq, nH, Dh, L, P, out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(value=None), INVALID),
    (dict(out=None), INVALID),
    (dict(loc=None), INVALID),
    (dict(dtype=7), INVALID),
    (dict(mode=3), INVALID),
    (dict(B=0), INVALID),
    (dict(Nv=0), INVALID),
    (dict(nH=0), INVALID),
    (dict(Dh=16), UNSUPPORTED),
    (dict(L=5, P=13), UNSUPPORTED),
    (dict(nH=65), UNSUPPORTED),
    (dict(value=MIS), INVALID),
    (dict(loc=A + 4), INVALID),
    (dict(Nv=1 << 31), UNSUPPORTED),
    (dict(Nv=1 << 21, nH=8), UNSUPPORTED),  # 2^21 * 8 * 32 * 4 bytes = 2 GiB per image
    (dict(dtype=3), INVALID),
    (dict(dtype=2, Nv=1 << 21, nH=8), UNSUPPORTED),  # head-pair layout: 2^21 * 8 * 128 bytes = 2 GiB per image
])
def test_msda_forward_rejects(lib, kw, code):
    assert _msda(lib, **kw) == code
    assert lib.msda_last_error().decode() != ""


def test_msda_forward_empty_query_set_is_a_no_op(lib):
    assert _msda(lib, Nq=0) == OK
    # with no queries the per-query buffers may be null (torch gives null for empty tensors)
    assert _msda(lib, Nq=0, out=None, loc=None, w=None) == OK
    assert _msda(lib, Nq=4, out=None) == INVALID


def test_msda_forward_frames_rejects(lib):
    f = lib.msda_forward_frames
    assert f(A, 0, A, A, A, A, 1, 1, 0, 16, 4, 8, 32, 1, 4, B_, None) == INVALID  # F = 0
    assert f(A, 0, A, A, A, A, 1, 1, 2, 16, 4, 8, 64, 1, 4, B_, None) == UNSUPPORTED
    assert f(A, 0, A, A, A, A, 1, 1, 2, 16, 0, 8, 32, 1, 4, B_, None) == OK  # nothing to do


def test_sca_workspace_size(lib):
    n = _sz(0)
    assert lib.sca_workspace_size(1, 6, 40000, ctypes.byref(n)) == OK
    small = n.value
    assert small >= 4 * 40000 + 4 * 6 * 40000  # camera masks + pair lists at least
    assert lib.sca_workspace_size(4, 6, 40000, ctypes.byref(n)) == OK
    assert n.value > small
    assert lib.sca_workspace_size(0, 6, 10, ctypes.byref(n)) == INVALID
    assert lib.sca_workspace_size(1, 6, 10, None) == INVALID
    assert lib.sca_workspace_size(1 << 20, 32, 1 << 20, ctypes.byref(n)) == UNSUPPORTED


def _sca(lib, value=A, dtype=0, B=1, Ncam=6, Nv=16, Nq=8, nH=8, Dh=32, L=1, P=8, D=4, slots=B_, ws=A,
         ws_bytes=1 << 30, rp=A, mask=A, off=A, logits=A):
    return lib.sca_forward(value, dtype, A, A, rp, mask, off, logits, B, Ncam, Nv, Nq, nH, Dh, L, P, D, slots,
                           None, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), INVALID),
    (dict(slots=None), INVALID),
    (dict(Ncam=0), INVALID),
    (dict(D=0), INVALID),
    (dict(Ncam=33), UNSUPPORTED),
    (dict(P=6, D=4), SHAPE),
    (dict(ws=None), WORKSPACE),
    (dict(ws_bytes=16), WORKSPACE),
    (dict(ws=A + 16), WORKSPACE),
    (dict(rp=A + 4), INVALID),
    (dict(Dh=64), UNSUPPORTED),
    (dict(dtype=3), INVALID),
    (dict(dtype=2, Nv=1 << 21, nH=8), UNSUPPORTED),  # head-pair layout: 2^21 * 8 * 128 bytes = 2 GiB per image
])
def test_sca_forward_rejects(lib, kw, code):
    assert _sca(lib, **kw) == code


def test_sca_forward_empty_query_set_is_a_no_op(lib):
    assert _sca(lib, Nq=0) == OK
    assert _sca(lib, Nq=0, slots=None, rp=None, mask=None, off=None, logits=None) == OK
    assert _sca(lib, Nq=3, slots=None) == INVALID


def test_sca_stages_reject(lib):
    n = _sz(0)
    assert lib.sca_workspace_size(1, 6, 8, ctypes.byref(n)) == OK
    c = lib.sca_compact
    assert c(None, A, 1, 6, 8, 4, None, None, None, A, n.value, None) == INVALID
    assert c(A, None, 1, 6, 8, 4, None, None, None, A, n.value, None) == INVALID
    assert c(A, A + 4, 1, 6, 8, 4, None, None, None, A, n.value, None) == INVALID
    assert c(A, A, 1, 33, 8, 4, None, None, None, A, n.value, None) == UNSUPPORTED
    assert c(A, A, 1, 6, 8, 4, None, None, None, A, n.value - 1, None) == WORKSPACE
    assert c(A, A, 1, 6, 0, 4, None, None, None, A, n.value, None) == OK
    g = lib.sca_gather
    assert g(A, 0, A, A, A, A, A, 1, 6, 16, 8, 8, 32, 1, 6, 4, B_, A, n.value, None) == SHAPE
    assert g(A, 0, A, A, A, A, A, 1, 6, 16, 8, 8, 32, 1, 8, 4, B_, None, n.value, None) == WORKSPACE
    assert g(A, 0, A, A, None, A, A, 1, 6, 16, 8, 8, 32, 1, 8, 4, B_, A, n.value, None) == INVALID


@pytest.mark.parametrize("M,N,K,code", [
    (10, 256, 48, UNSUPPORTED),
    (10, 256, 512, UNSUPPORTED),
    (10, 24, 256, UNSUPPORTED),
    (-1, 256, 256, INVALID),
    (0, 256, 256, OK),
])
def test_gemm_rejects(lib, M, N, K, code):
    assert lib.msda_gemm_bf16(A, 1, A, None, B_, 1, M, N, K, None) == code


def _vp(lib, X=A, dt=1, W=A, bias=None, Y=B_, M=64, N=256, K=256, Nv=16):
    return lib.msda_value_proj_pairs_bf16(X, dt, W, bias, Y, M, N, K, Nv, None)


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), INVALID),
    (dict(W=None), INVALID),
    (dict(Y=None), INVALID),
    (dict(dt=2), INVALID),
    (dict(N=48), UNSUPPORTED),  # a multiple of 16, not of 32: heads are 32 channels
    (dict(K=48), UNSUPPORTED),
    (dict(Nv=0), INVALID),
    (dict(M=60), SHAPE),  # not a whole number of 16-row images
    (dict(M=1 << 21, Nv=1 << 21), UNSUPPORTED),  # 2^21 * 8 * 128 bytes = 2 GiB per image
    (dict(Y=MIS), INVALID),
    (dict(Y=A + 0x4000), INVALID),  # overlaps X
    (dict(M=0), OK),
])
def test_value_proj_pairs_rejects(lib, kw, code):
    assert _vp(lib, **kw) == code


def _pk(lib, v=A, p=B_, n=2, Nv=16, nH=8):
    return lib.msda_pack_pairs_bf16(v, p, n, Nv, nH, None)


@pytest.mark.parametrize("kw,code", [
    (dict(v=None), INVALID),
    (dict(p=None), INVALID),
    (dict(n=-1), INVALID),
    (dict(Nv=0), INVALID),
    (dict(nH=0), INVALID),
    (dict(nH=65), UNSUPPORTED),
    (dict(Nv=1 << 21), UNSUPPORTED),  # 2^21 * 8 * 128 bytes = 2 GiB per image
    (dict(v=MIS), INVALID),
    (dict(p=A + 0x2000), INVALID),  # overlaps value
    (dict(n=0), OK),
    (dict(n=0, v=None, p=None), OK),  # nothing to copy: empty tensors have null data
])
def test_pack_pairs_rejects(lib, kw, code):
    assert _pk(lib, **kw) == code


def test_pairs_layout_is_refused_by_the_backward_passes(lib):
    """MSDA_BF16_PAIRS is for the forward entry points: the backward ones
    refuse it before anything is read."""
    assert _mb(lib, dtype=2) == INVALID
    assert _mbf(lib, dtype=2) == INVALID


def test_gemm_rejects_null_and_dtype(lib):
    assert lib.msda_gemm_bf16(None, 1, A, None, B_, 1, 4, 256, 256, None) == INVALID
    assert lib.msda_gemm_bf16(A, 5, A, None, B_, 1, 4, 256, 256, None) == INVALID
    assert lib.msda_gemm_bf16(MIS, 1, A, None, B_, 1, 4, 256, 256, None) == INVALID


def _qp(lib, q=A, pos=None, Wo=A, bo=None, Wa=A, ba=None, off=B_, lg=B_, M=4, K=256, No=512, Na=256):
    return lib.msda_query_proj_bf16(q, pos, Wo, bo, Wa, ba, off, lg, M, K, No, Na, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID),
    (dict(Wa=None), INVALID),
    (dict(lg=None), INVALID),
    (dict(pos=MIS), INVALID),
    (dict(No=0), INVALID),
    (dict(No=48), UNSUPPORTED),   # offsets must fill whole 32-column wave slices
    (dict(Na=24), UNSUPPORTED),
    (dict(K=48), UNSUPPORTED),
    (dict(M=-2), INVALID),
    (dict(M=0), OK),
])
def test_query_proj_rejects(lib, kw, code):
    assert _qp(lib, **kw) == code


def _op(lib, X=A, dt=0, W=A, bias=None, res=None, gamma=None, beta=None, eps=1e-5, Y=B_, M=4, N=256, K=256):
    return lib.msda_output_proj_bf16(X, dt, W, bias, res, gamma, beta, ctypes.c_float(eps), Y, M, N, K, None)


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), INVALID),
    (dict(Y=None), INVALID),
    (dict(dt=4), INVALID),
    (dict(beta=A), INVALID),              # beta without gamma
    (dict(gamma=A, N=512), UNSUPPORTED),  # the norm needs one 256-column row per block
    (dict(gamma=A, eps=-1.0), INVALID),
    (dict(gamma=A, eps=float("nan")), INVALID),
    (dict(res=MIS), INVALID),
    (dict(N=24), UNSUPPORTED),
    (dict(M=0, gamma=A, beta=A, res=A), OK),
])
def test_output_proj_rejects(lib, kw, code):
    assert _op(lib, **kw) == code


def _rb(lib, po=A, pq=A, rp=A, off=A, lg=A, ss=A, B=1, Ncam=6, Nq=16, nH=8, L=4, P=8, D=4, ml=8, loc=B_, lo=B_):
    return lib.sca_rebatch(po, pq, rp, off, lg, ss, B, Ncam, Nq, nH, L, P, D, ml, loc, lo, None)


@pytest.mark.parametrize("kw,code", [
    (dict(po=None), INVALID),
    (dict(loc=None), INVALID),
    (dict(ss=None), INVALID),
    (dict(P=6), SHAPE),
    (dict(Ncam=0), INVALID),
    (dict(ml=-1), INVALID),
    (dict(Ncam=33), UNSUPPORTED),
    (dict(rp=A + 4), INVALID),
    (dict(ml=0, pq=None, rp=None, off=None, lg=None, loc=None, lo=None), OK),  # no rows: nothing to do
])
def test_rebatch_rejects(lib, kw, code):
    assert _rb(lib, **kw) == code


def _sm(lib, rows=A, po=A, pq=A, hit=A, B=1, Ncam=6, Nq=16, C=256, ml=8, slots=B_):
    return lib.sca_scatter_mean(rows, po, pq, hit, B, Ncam, Nq, C, ml, slots, None)


@pytest.mark.parametrize("kw,code", [
    (dict(slots=None), INVALID),
    (dict(hit=None), INVALID),
    (dict(rows=None), INVALID),
    (dict(C=6), UNSUPPORTED),
    (dict(C=0), INVALID),
    (dict(rows=MIS), INVALID),
    (dict(B=0, slots=None, hit=None, po=None, rows=None, pq=None), OK),
])
def test_scatter_mean_rejects(lib, kw, code):
    assert _sm(lib, **kw) == code


def _mb(lib, value=A, dtype=0, ss=A, st=A, loc=A, w=A, mode=1, go=A, B=1, Nv=16, Nq=4, nH=8, Dh=32, L=1, P=4,
        gv=B_, gl=B_, gw=B_, gws=None, gws_bytes=0):
    return lib.msda_backward(value, dtype, ss, st, loc, w, mode, go, B, Nv, Nq, nH, Dh, L, P, gv, gl, gw, gws,
                             gws_bytes, None)


def _mbf(lib, F=2, gws=None, gws_bytes=0, **kw):
    """msda_backward_frames with _mb's defaults."""
    a = dict(value=A, dtype=0, ss=A, st=A, loc=A, w=A, mode=1, go=A, B=1, Nv=16, Nq=4, nH=8, Dh=32, L=1, P=4,
             gv=B_, gl=B_, gw=B_)
    a.update(kw)
    return lib.msda_backward_frames(a["value"], a["dtype"], a["ss"], a["st"], a["loc"], a["w"], a["mode"], a["go"],
                                    a["B"], F, a["Nv"], a["Nq"], a["nH"], a["Dh"], a["L"], a["P"], a["gv"], a["gl"],
                                    a["gw"], gws, gws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(F=0), INVALID),
    (dict(B=0), INVALID),
    (dict(gv=None), INVALID),
    (dict(mode=7), INVALID),
    (dict(Dh=16), UNSUPPORTED),
    (dict(F=1 << 31), UNSUPPORTED),
])
def test_msda_backward_frames_rejects(lib, kw, code):
    assert _mbf(lib, **kw) == code


def test_msda_backward_frames_workspace_is_that_of_b_times_f_images(lib):
    rc, need = _mb_ws(lib, B=3 * 2)
    assert rc == OK
    assert _mbf(lib, F=2, B=3, gws=A, gws_bytes=need - 1) == WORKSPACE


def _mb_ws(lib, B=1, Nv=16, Nq=4, nH=8, L=1, P=4):
    n = _sz(0)
    rc = lib.msda_backward_workspace_size(B, Nv, Nq, nH, L, P, ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(gv=None), INVALID),
    (dict(go=None), INVALID),
    (dict(gl=None), INVALID),
    (dict(mode=7), INVALID),
    (dict(B=0), INVALID),
    (dict(Dh=16), UNSUPPORTED),
    (dict(gv=MIS), INVALID),
    (dict(gl=A + 4), INVALID),
    (dict(Nv=1 << 21, dtype=1), UNSUPPORTED),  # bf16 value fits, its float32 gradient image does not
])
def test_msda_backward_rejects(lib, kw, code):
    assert _mb(lib, **kw) == code


def test_backward_workspace_sizes(lib):
    """Gradient workspace sizes: about 40 bytes per record slot (each (image,
    head) rounded up to 2048 slots) plus 8 per cell key, growing with every
    size; invalid or oversized requests are refused."""
    tile = 2048 * 40  # the sort buffers of one tile of record slots
    rc, small = _mb_ws(lib)
    assert rc == OK and small >= 8 * tile  # 8 heads, 16 samples each: one tile each
    rc, same = _mb_ws(lib, Nq=500)
    assert rc == OK and same == small  # 2000 samples per head still fit one tile
    rc, more_q = _mb_ws(lib, Nq=4000)
    assert rc == OK and more_q - small >= (8 - 1) * 8 * tile  # 16000 samples per head: 8 tiles
    rc, more_v = _mb_ws(lib, Nv=1600)
    assert rc == OK and more_v - small >= (2 * 1600 - 2 * 16) * 8 * 8
    assert _mb_ws(lib, B=0)[0] == INVALID
    assert _mb_ws(lib, Nq=1 << 26)[0] == UNSUPPORTED  # 2^26 * 32 sample records
    assert _mb_ws(lib, B=1 << 14, Nq=1)[0] == UNSUPPORTED  # 2^17 (image, head) tiles of 2048 slots
    n = _sz(0)
    assert lib.msda_backward_workspace_size(1, 16, 4, 8, 1, 4, None) == INVALID
    # SCA: B=1, 6 cameras, 4096 queries, 8 heads, L*P = 4
    assert lib.sca_backward_workspace_size(1, 6, 16, 4096, 8, 1, 4, 0, ctypes.byref(n)) == OK
    every = n.value
    assert every >= (6 * 4096 * 8 * 4 // 2048 + 48) * tile
    assert lib.sca_backward_workspace_size(1, 6, 16, 4096, 8, 1, 4, 5, ctypes.byref(n)) == OK
    # 5 pairs: one tile of samples at most (tiles are allocated in eights)
    assert every - n.value >= (6 * 4096 * 8 * 4 // 2048 - 8) * tile
    assert lib.sca_backward_workspace_size(1, 33, 16, 4, 8, 1, 4, 0, ctypes.byref(n)) == UNSUPPORTED


def test_msda_backward_rejects_small_gradient_workspace(lib):
    rc, need = _mb_ws(lib)
    assert rc == OK
    assert _mb(lib, gws=A, gws_bytes=need - 1) == WORKSPACE
    assert _mb(lib, gws=A + 16, gws_bytes=need) == WORKSPACE  # not 256-byte aligned


def test_sca_backward_rejects(lib):
    n = _sz(0)
    assert lib.sca_workspace_size(1, 6, 16, ctypes.byref(n)) == OK
    b = lib.sca_backward
    args = [A, 0, A, A, A, A, A, A, 1, 6, 16, 8, 8, 32, 1, 8, 4, B_, B_, B_, A, n.value, 0, None, 0, None]
    assert b(*args[:17], None, *args[18:]) == INVALID                 # grad_value
    assert b(*args[:16], 6, *args[17:]) == SHAPE                      # P % D
    assert b(*args[:20], None, *args[21:]) == WORKSPACE               # workspace
    assert b(*args[:9], 33, *args[10:]) == UNSUPPORTED                # cameras
    assert b(*args[:7], None, *args[8:]) == INVALID                   # grad_slots
    g = _sz(0)
    assert lib.sca_backward_workspace_size(1, 6, 16, 8, 8, 1, 8, 0, ctypes.byref(g)) == OK
    assert b(*args[:23], A, g.value - 1, None) == WORKSPACE           # gradient workspace too small
    assert lib.sca_backward_workspace_size(1, 6, 16, 8, 8, 1, 8, 3, ctypes.byref(g)) == OK
    assert b(*args[:22], 3, A, g.value - 1, None) == WORKSPACE        # ... sized for max_pairs = 3



def test_binding_refuses_cpu_tensors():
    import torch
    import scale_deformable_attention_forward_amd as m
    v = torch.zeros(1, 16, 8, 32)
    with pytest.raises(ValueError):
        m.msda_forward(v, torch.zeros(1, 2, dtype=torch.int64), torch.zeros(1, dtype=torch.int64),
                       torch.zeros(1, 4, 8, 1, 4, 2), torch.zeros(1, 4, 8, 4))


def _binding_calls():
    """(call, the tensor whose size is wrong, before any '/') for the Python binding, on CPU
    tensors: the size checks come before any device use, so the calls raise
    without a GPU; with every size right they stop at the device check."""
    import torch
    import scale_deformable_attention_forward_amd as m
    i64, bf = torch.int64, torch.bfloat16
    ss, st = torch.zeros(1, 2, dtype=i64), torch.zeros(1, dtype=i64)
    v, loc, w = torch.zeros(1, 16, 8, 32), torch.zeros(1, 4, 8, 1, 4, 2), torch.zeros(1, 4, 8, 4)
    go = torch.zeros(1, 4, 256)
    sv, rho, mask = torch.zeros(1, 2, 16, 8, 32), torch.zeros(2, 1, 5, 4, 2), torch.zeros(2, 1, 5, 4, dtype=torch.uint8)
    off, lg, ws = torch.zeros(1, 5, 8, 1, 4, 2), torch.zeros(1, 5, 8, 4), torch.zeros(64, dtype=torch.uint8)
    X, Wt = torch.zeros(10, 32, dtype=bf), torch.zeros(16, 32, dtype=bf)
    return {
        None: lambda: m.msda_forward(v, ss, st, loc, w),
        "attention_weights": lambda: m.msda_forward(v, ss, st, loc, torch.zeros(1, 4, 8, 3)),
        "spatial_shapes": lambda: m.msda_forward(v, torch.zeros(2, 2, dtype=i64), st, loc, w),
        "level_start_index": lambda: m.msda_forward(v, ss, torch.zeros(2, dtype=i64), loc, w),
        "out": lambda: m.msda_forward(v, ss, st, loc, w, out=torch.zeros(1, 4, 255)),
        "grad_out": lambda: m.msda_backward(v, ss, st, loc, w, torch.zeros(1, 4, 200)),
        "grad_value": lambda: m.msda_backward(v, ss, st, loc, w, go, grad_value=torch.zeros(1, 15, 8, 32)),
        "reference_points_cam": lambda: m.sca_forward(sv, ss, st, torch.zeros(3, 1, 5, 4, 2), mask, off, lg),
        "bev_mask": lambda: m.sca_forward(sv, ss, st, rho, torch.zeros(2, 1, 5, 3, dtype=torch.uint8), off, lg),
        "sampling_offsets": lambda: m.sca_gather(sv, ss, st, rho, torch.zeros(1, 5, 8, 1, 4, 2)[:, :4], lg, ws),
        "pair_q": lambda: m.sca_compact(mask, rho, ws, pair_q=torch.zeros(9, dtype=torch.int32)),
        "grad_slots": lambda: m.sca_backward(sv, ss, st, rho, off, lg, torch.zeros(1, 5, 255), ws),
        "W": lambda: m.msda_gemm_bf16(X, torch.zeros(16, 31, dtype=bf)),
        "residual": lambda: m.msda_output_proj_bf16(X, Wt, residual=torch.zeros(10, 15)),
        "W_att": lambda: m.msda_query_proj_bf16(torch.zeros(10, 32), Wt, None, torch.zeros(8, 30, dtype=bf), None),
        "rows": lambda: m.sca_scatter_mean(torch.zeros(3, 2, 256), torch.zeros(3, dtype=torch.int32),
                                           torch.zeros(4, dtype=torch.int32), torch.zeros(2, 5, dtype=torch.int32), 5),
        # pair lists shorter than B*Ncam*Nq entries would let a kernel read past them
        "pair_q/scatter_mean": lambda: m.sca_scatter_mean(torch.zeros(2, 3, 256), torch.zeros(3, dtype=torch.int32),
                                             torch.zeros(9, dtype=torch.int32), torch.zeros(1, 5, dtype=torch.int32), 5),
        "pair_q/rebatch": lambda: m.sca_rebatch(torch.zeros(3, dtype=torch.int32), torch.zeros(9, dtype=torch.int32), rho,
                                         off, lg, ss, 2),
    }


@pytest.mark.parametrize("wrong", list(_binding_calls()), ids=lambda w: w or "all_right")
def test_binding_checks_element_counts(wrong):
    call = _binding_calls()[wrong]
    if wrong is None:
        with pytest.raises(ValueError, match="GPU device"):
            call()
    else:
        with pytest.raises(ValueError, match=f"^{wrong.split('/')[0]}: "):
            call()



def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """sca_forward_noalloc refuses, before any device call, a problem whose
    SCA workspace exceeds the static scratch array (16 MiB)."""
    need = _sz(0)
    assert lib.sca_workspace_size(12, 6, 40000, ctypes.byref(need)) == OK and need.value > 16 << 20
    args = (A, 0, A, A, A, A, A, A)
    assert lib.sca_forward_noalloc(*args, 12, 6, 16, 40000, 8, 32, 4, 8, 4, B_, None, None, None, None) == UNSUPPORTED
    assert "sca_forward_noalloc holds" in lib.msda_last_error().decode()
    assert lib.sca_forward_noalloc(*args, 0, 6, 16, 4, 8, 32, 4, 8, 4, B_, None, None, None, None) == INVALID


def test_msda_plan_rejects(lib):
    st = None
    n = _sz(0)
    assert lib.msda_plan_size(2, 1000, ctypes.byref(n)) == OK and n.value == 8192 + 2 * 16 * 1024 * 4
    assert lib.msda_plan_size(0, 10, ctypes.byref(n)) == INVALID
    assert lib.msda_plan_size(1 << 16, 1, ctypes.byref(n)) == UNSUPPORTED
    assert lib.msda_plan_size(1, 10, None) == INVALID
    assert lib.msda_plan_size(1, 20, ctypes.byref(n)) == OK
    size = n.value
    assert lib.msda_plan(None, 40, 2, 1, 20, B_, size, st) == INVALID        # null points
    assert lib.msda_plan(A, 40, 2, 1, 20, None, size, st) == WORKSPACE      # null plan
    assert lib.msda_plan(A, 40, 2, 1, 20, B_, size - 1, st) == WORKSPACE    # plan too small
    assert lib.msda_plan(A, 40, 2, 1, 20, B_ + 16, size, st) == WORKSPACE   # plan not 256-byte aligned
    assert lib.msda_plan(A, 40, 3, 1, 20, B_, size, st) == INVALID          # odd point stride
    assert lib.msda_plan(A, -2, 2, 1, 20, B_, size, st) == INVALID          # negative stride
    assert lib.msda_plan(MIS + 2, 40, 2, 1, 20, B_, size, st) == INVALID    # points not 8-byte aligned
    assert lib.msda_plan(A, 40, 2, 0, 20, B_, size, st) == INVALID          # no batch
    assert lib.msda_plan(None, 0, 2, 1, 0, B_, 1 << 20, st) == OK           # no queries: nothing to do


def test_msda_gather_rejects(lib):
    n = _sz(0)
    assert lib.msda_plan_size(1, 4, ctypes.byref(n)) == OK
    g = lambda plan=B_, size=n.value, F=2, Dh=32: lib.msda_gather(A, 0, A, A, A, A, 1, 1, F, 16, 4, 8, Dh, 1, 4,
                                                                   B_, plan, size, None)
    assert g(plan=None) == WORKSPACE                # a plan is required
    assert g(size=n.value - 4) == WORKSPACE         # a plan buffer too small
    assert g(plan=B_ + 64) == WORKSPACE             # misaligned plan
    assert g(F=0) == INVALID                        # no frames
    assert g(Dh=16) == UNSUPPORTED
    assert lib.msda_gather(A, 0, A, A, None, None, 1, 1, 2, 16, 0, 8, 32, 1, 4, None, None, 0, None) == OK  # Nq = 0


def test_check_counts_unsupported_in_the_regular_build(lib):
    """The regular library has no device-side checks: msda_check_counts
    returns MSDA_ERR_UNSUPPORTED and touches nothing (no device call)."""
    counts = (ctypes.c_ulonglong * 4)(7, 7, 7, 7)
    lib.msda_check_counts.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), _int, _int]
    assert lib.msda_check_counts(counts, 4, 0) == UNSUPPORTED
    assert list(counts) == [7, 7, 7, 7]
    assert b"libmsda_checked.so" in lib.msda_last_error()


def test_checked_build_exports_the_same_entry_points():
    """libmsda_checked.so is the same C ABI; its msda_check_counts rejects a
    short counts array before any device call."""
    import scale_deformable_attention_forward_amd as m
    path = m.checked_library_path()
    if not os.path.exists(path):
        from scale_deformable_attention_forward_amd import build
        build.build(checked=True)
    checked = ctypes.CDLL(path)
    for name in declared_functions():
        assert hasattr(checked, name), f"{name} missing from the checked build"
    checked.msda_check_counts.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), _int, _int]
    checked.msda_last_error.restype = ctypes.c_char_p
    counts = (ctypes.c_ulonglong * 4)()
    assert checked.msda_check_counts(counts, 3, 0) == INVALID
    assert checked.msda_check_counts(None, 4, 0) == INVALID
    assert b"MSDA_CHECK_KINDS" in checked.msda_last_error()
