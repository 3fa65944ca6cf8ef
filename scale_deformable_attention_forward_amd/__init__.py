"""Multi-scale deformable attention and BEVFormer spatial cross-attention,
forward and backward passes, on AMD Instinct MI355X (gfx950).

This module is the thin Python binding of libmsda.so (C ABI in
include/msda.h).  It only marshals torch tensors into pointers and sizes:
every step of the computation runs in the library's HIP kernels.  PyTorch
provides device memory and the stream: torch's current one, or the one given
as `stream=` (a torch.cuda.Stream or a raw handle), which is made current for
the call so that what the call allocates belongs to it.  If the library is
missing, importing works but every call raises: there is no fallback path.

Functions (same names as the C entry points):
  operator:     msda_forward, msda_forward_frames, msda_plan and msda_gather
                (the operator in a locality order), msda_backward,
                msda_backward_frames, msda_backward_workspace_size
  SCA:          sca_workspace_size (also as sca_plan_workspace), sca_forward,
                sca_forward_noalloc (workspace in a static device array),
                sca_compact, sca_gather, sca_backward, sca_backward_workspace_size
  padded flow:  sca_rebatch, sca_scatter_mean (and sca_forward_rebatch, which
                chains them with the compaction and msda_forward)
  projections:  msda_gemm_bf16, msda_query_proj_bf16, msda_output_proj_bf16,
                msda_value_proj_pairs_bf16 (the value projection written in the
                head-pair layout that every forward entry point also takes)
  layout:       msda_pack_pairs_bf16 (a bf16 value rewritten in that layout)
  status:       msda_status_string, msda_last_error
  checks:       msda_check_counts (the bounds-check counters of
                libmsda_checked.so; use_library(checked_library_path())
                switches the binding to that build)
"""
import ctypes
import functools
import os

import torch

__all__ = [
    "MsdaError", "MSDA_F32", "MSDA_BF16", "MSDA_BF16_PAIRS", "MSDA_WEIGHTS_PROB", "MSDA_WEIGHTS_LOGITS",
    "library_path", "load_library", "msda_forward", "msda_forward_frames", "msda_plan_size", "msda_plan",
    "msda_gather", "plan_order",
    "sca_workspace_size", "sca_plan_workspace",
    "sca_forward", "sca_forward_noalloc", "sca_compact", "sca_gather", "msda_gemm_bf16", "msda_query_proj_bf16",
    "msda_output_proj_bf16", "msda_value_proj_pairs_bf16", "msda_pack_pairs_bf16",
    "sca_rebatch", "sca_scatter_mean", "sca_forward_rebatch", "msda_backward_workspace_size",
    "sca_backward_workspace_size", "msda_backward", "msda_backward_frames", "sca_backward", "msda_status_string",
    "msda_last_error", "MSDA_CHECK_KINDS", "checked_library_path", "use_library", "msda_check_counts",
]

MSDA_F32, MSDA_BF16, MSDA_BF16_PAIRS = 0, 1, 2
MSDA_WEIGHTS_PROB, MSDA_WEIGHTS_LOGITS = 0, 1
# kinds of the checked build's bounds-check counters (msda_check_counts)
MSDA_CHECK_KINDS = 4
CHECK_KIND_NAMES = ("gather_row", "pair_write", "order_write", "list_entry")

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_p, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t


class MsdaError(RuntimeError):
    """A non-zero status from libmsda.so."""

    def __init__(self, fn, code, message):
        super().__init__(f"{fn}: {msda_status_string(code)}: {message}")
        self.code = code


def library_path():
    return os.path.join(_HERE, "libmsda.so")


def checked_library_path():
    """The in-tree build with device-side bounds checks (MSDA_CHECKED)."""
    return os.path.join(_HERE, "libmsda_checked.so")


_path = None  # set by use_library


def use_library(path=None):
    """Make every later call go through the library at `path` (None: the
    regular libmsda.so); returns the path in use before."""
    global _lib, _path
    before = _path or library_path()
    _path, _lib = path, None
    return before


def load_library():
    """Load the in-tree libmsda.so, or the library use_library() chose
    (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = _path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m scale_deformable_attention_forward_amd.build`")
    lib = ctypes.CDLL(path)
    lib.msda_forward.argtypes = [_p, _int, _p, _p, _p, _p, _int, _i64, _i64, _i64, _int, _int, _int, _int, _p, _p]
    lib.msda_forward_frames.argtypes = [_p, _int, _p, _p, _p, _p, _int, _i64, _i64, _i64, _i64, _int, _int, _int,
                                        _int, _p, _p]
    lib.msda_plan_size.argtypes = [_i64, _i64, ctypes.POINTER(_sz)]
    lib.msda_plan.argtypes = [_p, _i64, _i64, _i64, _i64, _p, _sz, _p]
    lib.msda_gather.argtypes = [_p, _int, _p, _p, _p, _p, _int, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _p, _p,
                                _sz, _p]
    lib.sca_workspace_size.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_sz)]
    lib.sca_plan_workspace.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_sz)]
    lib.sca_forward.argtypes = [_p, _int, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int, _int, _int,
                                _int, _p, _p, _p, _p, _p, _sz, _p]
    lib.sca_forward_noalloc.argtypes = [_p, _int, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int, _int,
                                        _int, _int, _p, _p, _p, _p, _p]
    lib.sca_compact.argtypes = [_p, _p, _i64, _i64, _i64, _int, _p, _p, _p, _p, _sz, _p]
    lib.sca_gather.argtypes = [_p, _int, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _int,
                               _p, _p, _sz, _p]
    lib.msda_gemm_bf16.argtypes = [_p, _int, _p, _p, _p, _int, _i64, _i64, _i64, _p]
    lib.msda_value_proj_pairs_bf16.argtypes = [_p, _int, _p, _p, _p, _i64, _i64, _i64, _i64, _p]
    lib.msda_pack_pairs_bf16.argtypes = [_p, _p, _i64, _i64, _int, _p]
    lib.msda_backward.argtypes = [_p, _int, _p, _p, _p, _p, _int, _p, _i64, _i64, _i64, _int, _int, _int, _int, _p,
                                  _p, _p, _p, _sz, _p]
    lib.msda_backward_frames.argtypes = [_p, _int, _p, _p, _p, _p, _int, _p, _i64, _i64, _i64, _i64, _int, _int, _int,
                                         _int, _p, _p, _p, _p, _sz, _p]
    lib.sca_backward.argtypes = [_p, _int, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int, _int, _int,
                                 _int, _p, _p, _p, _p, _sz, _i64, _p, _sz, _p]
    lib.msda_backward_workspace_size.argtypes = [_i64, _i64, _i64, _int, _int, _int, ctypes.POINTER(_sz)]
    lib.sca_backward_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _int, _int, _int, _i64, ctypes.POINTER(_sz)]
    lib.sca_rebatch.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _int, _int, _int, _int, _i64, _p, _p, _p]
    lib.sca_scatter_mean.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p, _p]
    lib.msda_query_proj_bf16.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p]
    lib.msda_output_proj_bf16.argtypes = [_p, _int, _p, _p, _p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i64, _p]
    for f in (lib.msda_forward, lib.msda_forward_frames, lib.msda_plan_size, lib.msda_plan, lib.msda_gather,
              lib.sca_workspace_size,
              lib.sca_plan_workspace, lib.sca_forward,
              lib.sca_forward_noalloc,
              lib.sca_compact, lib.sca_gather, lib.msda_gemm_bf16, lib.msda_value_proj_pairs_bf16,
              lib.msda_pack_pairs_bf16):
        f.restype = _int
    lib.msda_status_string.argtypes = [_int]
    lib.msda_status_string.restype = ctypes.c_char_p
    lib.msda_last_error.argtypes = []
    lib.msda_last_error.restype = ctypes.c_char_p
    lib.msda_check_counts.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), _int, _int]
    lib.msda_check_counts.restype = _int
    _lib = lib
    return lib


def msda_status_string(code):
    return load_library().msda_status_string(int(code)).decode()


def msda_last_error():
    return load_library().msda_last_error().decode()


def msda_check_counts(reset=False):
    """The bounds-check counters of libmsda_checked.so, summed over the
    library, as {kind name: count} (waits for the current device; reset
    zeroes them).  The regular library raises MsdaError
    (MSDA_ERR_UNSUPPORTED)."""
    counts = (ctypes.c_ulonglong * MSDA_CHECK_KINDS)()
    _check("msda_check_counts", load_library().msda_check_counts(counts, MSDA_CHECK_KINDS, int(bool(reset))))
    return dict(zip(CHECK_KIND_NAMES, (int(c) for c in counts)))


def _check(fn, code):
    if code != 0:
        raise MsdaError(fn, code, msda_last_error())


def _ptr(t, name, dtypes=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return t.data_ptr()


def _numel(t, name, n, at_least=False):
    """Element count of a tensor the C call reads (exactly n) or writes (at
    least n) as flat contiguous memory: a smaller one would send the kernels
    past its end."""
    if t is None:
        return
    k = t.numel()
    if k < n or (not at_least and k != n):
        raise ValueError(f"{name}: {'at least ' if at_least else ''}{n} elements expected, got {k} "
                         f"(shape {tuple(t.shape)})")


def _levels(spatial_shapes, level_start_index, L):
    _numel(spatial_shapes, "spatial_shapes", 2 * L)
    _numel(level_start_index, "level_start_index", L)


def _value_dtype(value):
    if value.dtype == torch.float32:
        return MSDA_F32
    if value.dtype == torch.bfloat16:
        return MSDA_BF16
    raise TypeError(f"value must be float32 or bfloat16, got {value.dtype}")


def _op_value(value, frames):
    """(B, F, Nv, nH, Dh, value_dtype) of the operator's value: [B,Nv,nH,Dh]
    (frames: [B,F,Nv,nH,Dh]) float32 or bfloat16, or bfloat16 in the
    head-pair layout [B,nH,Nv,2,Dh] ([B,F,nH,Nv,2,Dh]), MSDA_BF16_PAIRS."""
    plain = 5 if frames else 4
    if value.dim() == plain + 1:
        if value.dtype != torch.bfloat16 or value.shape[-2] != 2:
            raise TypeError(f"a {plain + 1}-dimensional value is the bfloat16 head-pair layout "
                            f"[B,{'F,' if frames else ''}nH,Nv,2,Dh]; got {value.dtype} {tuple(value.shape)}")
        B, F = value.shape[0], (value.shape[1] if frames else 1)
        nH, Nv, _, Dh = value.shape[-4:]
        return B, F, Nv, nH, Dh, MSDA_BF16_PAIRS
    if value.dim() != plain:
        raise ValueError(f"value: {plain} dimensions expected, got shape {tuple(value.shape)}")
    B, F = value.shape[0], (value.shape[1] if frames else 1)
    Nv, nH, Dh = value.shape[-3:]
    return B, F, Nv, nH, Dh, _value_dtype(value)


def _sca_value(value):
    """(B, Ncam, Nv, nH, Dh, value_dtype) of an SCA value: [B,Ncam,Nv,nH,Dh]
    float32 or bfloat16, or bfloat16 [B,Ncam,nH,Nv,2,Dh] in the head-pair
    layout (MSDA_BF16_PAIRS)."""
    if value.dim() == 6:
        if value.dtype != torch.bfloat16 or value.shape[4] != 2:
            raise TypeError("a 6-dimensional SCA value is the bfloat16 head-pair layout [B,Ncam,nH,Nv,2,Dh]; "
                            f"got {value.dtype} {tuple(value.shape)}")
        B, Ncam, nH, Nv, _, Dh = value.shape
        return B, Ncam, Nv, nH, Dh, MSDA_BF16_PAIRS
    B, Ncam, Nv, nH, Dh = value.shape
    return B, Ncam, Nv, nH, Dh, _value_dtype(value)


def _given_stream(fn):
    """Run fn with its `stream` argument (a torch.cuda.Stream or a raw
    hipStream_t handle) made torch's current stream for the call: the outputs
    and workspaces fn allocates then belong to that stream in torch's caching
    allocator (a workspace freed on return is not handed to other work before
    the stream's kernels are done), and a read-back through torch is ordered
    after the launches."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        if not isinstance(stream, torch.cuda.Stream):
            # handle 0 is the null stream, which is torch's default stream
            stream = torch.cuda.default_stream() if int(stream) == 0 else torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(stream):
            return fn(*args, **kw)
    return call


def _stream(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


_I64 = (torch.int64,)
_F32 = (torch.float32,)


@_given_stream
def msda_forward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
                 weight_mode=MSDA_WEIGHTS_LOGITS, out=None, stream=None):
    """value [B,Nv,nH,Dh] (float32|bfloat16, or bfloat16 [B,nH,Nv,2,Dh] in the
    head-pair layout); spatial_shapes int64 [L,2] (H,W); level_start_index
    int64 [L]; sampling_locations float32 [B,Nq,nH,L,P,2]; attention_weights
    float32 [B,Nq,nH,L*P].  Returns out float32 [B,Nq,nH*Dh]."""
    lib = load_library()
    B, _, Nv, nH, Dh, vdt = _op_value(value, False)
    _, Nq, _, L, P, _ = sampling_locations.shape
    _levels(spatial_shapes, level_start_index, L)
    _numel(sampling_locations, "sampling_locations", B * Nq * nH * L * P * 2)
    _numel(attention_weights, "attention_weights", B * Nq * nH * L * P)
    _numel(out, "out", B * Nq * nH * Dh, at_least=True)
    if out is None:
        out = torch.empty((B, Nq, nH * Dh), dtype=torch.float32, device=value.device)
    rc = lib.msda_forward(_ptr(value, "value"), vdt, _ptr(spatial_shapes, "spatial_shapes", _I64),
                          _ptr(level_start_index, "level_start_index", _I64),
                          _ptr(sampling_locations, "sampling_locations", _F32),
                          _ptr(attention_weights, "attention_weights", _F32), int(weight_mode), B, Nv, Nq, nH, Dh,
                          L, P, _ptr(out, "out", _F32), _stream(stream, value.device))
    _check("msda_forward", rc)
    return out


@_given_stream
def msda_forward_frames(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
                        weight_mode=MSDA_WEIGHTS_LOGITS, out=None, stream=None):
    """value [B,F,Nv,nH,Dh] (or bfloat16 [B,F,nH,Nv,2,Dh] in the head-pair
    layout); sampling_locations [B,F,Nq,nH,L,P,2]; attention_weights
    [B,F,Nq,nH,L*P].  Returns the frame mean, float32 [B,Nq,nH*Dh]."""
    lib = load_library()
    B, F, Nv, nH, Dh, vdt = _op_value(value, True)
    _, _, Nq, _, L, P, _ = sampling_locations.shape
    _levels(spatial_shapes, level_start_index, L)
    _numel(sampling_locations, "sampling_locations", B * F * Nq * nH * L * P * 2)
    _numel(attention_weights, "attention_weights", B * F * Nq * nH * L * P)
    _numel(out, "out", B * Nq * nH * Dh, at_least=True)
    if out is None:
        out = torch.empty((B, Nq, nH * Dh), dtype=torch.float32, device=value.device)
    rc = lib.msda_forward_frames(_ptr(value, "value"), vdt,
                                 _ptr(spatial_shapes, "spatial_shapes", _I64),
                                 _ptr(level_start_index, "level_start_index", _I64),
                                 _ptr(sampling_locations, "sampling_locations", _F32),
                                 _ptr(attention_weights, "attention_weights", _F32), int(weight_mode), B, F, Nv, Nq,
                                 nH, Dh, L, P, _ptr(out, "out", _F32), _stream(stream, value.device))
    _check("msda_forward_frames", rc)
    return out


def msda_plan_size(B, Nq):
    """Bytes of the plan buffer msda_plan fills for (B, Nq)."""
    lib = load_library()
    n = _sz(0)
    _check("msda_plan_size", lib.msda_plan_size(int(B), int(Nq), ctypes.byref(n)))
    return n.value


@_given_stream
def msda_plan(points, B, Nq, batch_stride, point_stride, plan=None, stream=None):
    """Locality plan of the operator: each batch item's queries ordered by
    the tile of the point standing for query (b, q), points[b*batch_stride +
    q*point_stride + {0,1}] (float32, strides in elements).  Returns the plan
    buffer (uint8 [msda_plan_size(B, Nq)]); its first B*Nq int32 are the
    flat query indices in visiting order (plan_order() views them)."""
    lib = load_library()
    if Nq > 0:
        _numel(points, "points", (B - 1) * batch_stride + (Nq - 1) * point_stride + 2, at_least=True)
    need = msda_plan_size(B, Nq)
    if plan is None:
        plan = torch.empty(need, dtype=torch.uint8, device=points.device)
    rc = lib.msda_plan(_ptr(points, "points", _F32), int(batch_stride), int(point_stride), int(B), int(Nq),
                       _ptr(plan, "plan"), plan.numel() * plan.element_size(), _stream(stream, points.device))
    _check("msda_plan", rc)
    return plan


def plan_order(plan, B, Nq):
    """The visiting order held by a plan buffer: int32 [B*Nq] (a view)."""
    return plan.view(torch.uint8)[:4 * B * Nq].view(torch.int32)


@_given_stream
def msda_gather(value, spatial_shapes, level_start_index, sampling_locations, attention_weights, plan,
                weight_mode=MSDA_WEIGHTS_LOGITS, out=None, stream=None):
    """msda_forward (locations [B,Nq,..]) or msda_forward_frames (locations
    [B,F,Nq,..]), with the value as they take it, visiting the queries in the
    order of the plan buffer msda_plan filled for the same B and Nq.  Same
    result, bit for bit.  Returns out float32 [B,Nq,nH*Dh]."""
    lib = load_library()
    frames = sampling_locations.dim() == 7
    B, F, Nv, nH, Dh, vdt = _op_value(value, frames)
    if frames:
        _, _, Nq, _, L, P, _ = sampling_locations.shape
    else:
        _, Nq, _, L, P, _ = sampling_locations.shape
    _levels(spatial_shapes, level_start_index, L)
    _numel(sampling_locations, "sampling_locations", B * F * Nq * nH * L * P * 2)
    _numel(attention_weights, "attention_weights", B * F * Nq * nH * L * P)
    _numel(out, "out", B * Nq * nH * Dh, at_least=True)
    if out is None:
        out = torch.empty((B, Nq, nH * Dh), dtype=torch.float32, device=value.device)
    rc = lib.msda_gather(_ptr(value, "value"), vdt, _ptr(spatial_shapes, "spatial_shapes", _I64),
                         _ptr(level_start_index, "level_start_index", _I64),
                         _ptr(sampling_locations, "sampling_locations", _F32),
                         _ptr(attention_weights, "attention_weights", _F32), int(weight_mode), B, F, Nv, Nq, nH, Dh,
                         L, P, _ptr(out, "out", _F32), _ptr(plan, "plan"), plan.numel() * plan.element_size(),
                         _stream(stream, value.device))
    _check("msda_gather", rc)
    return out


def sca_workspace_size(B, Ncam, Nq):
    lib = load_library()
    n = _sz(0)
    _check("sca_workspace_size", lib.sca_workspace_size(int(B), int(Ncam), int(Nq), ctypes.byref(n)))
    return n.value


def sca_plan_workspace(B, Ncam, Nq):
    """sca_workspace_size under the planning step's name (same result)."""
    lib = load_library()
    n = _sz(0)
    _check("sca_plan_workspace", lib.sca_plan_workspace(int(B), int(Ncam), int(Nq), ctypes.byref(n)))
    return n.value


def _sca_inputs(B, Ncam, Nq, D, nH, L, P, spatial_shapes, level_start_index, reference_points_cam, sampling_offsets,
                attention_logits):
    _levels(spatial_shapes, level_start_index, L)
    _numel(reference_points_cam, "reference_points_cam", Ncam * B * Nq * D * 2)
    _numel(sampling_offsets, "sampling_offsets", B * Nq * nH * L * P * 2)
    _numel(attention_logits, "attention_logits", B * Nq * nH * L * P)


def _sca_outputs(B, Ncam, Nq, hit_count, pair_offsets, pair_q):
    _numel(hit_count, "hit_count", B * Nq, at_least=True)
    _numel(pair_offsets, "pair_offsets", B * Ncam + 1, at_least=True)
    _numel(pair_q, "pair_q", B * Ncam * Nq, at_least=True)


@_given_stream
def sca_forward(value, spatial_shapes, level_start_index, reference_points_cam, bev_mask, sampling_offsets,
                attention_logits, slots=None, hit_count=None, pair_offsets=None, pair_q=None, workspace=None,
                stream=None):
    """value [B,Ncam,Nv,nH,Dh] float32 or bfloat16, or bfloat16 [B,Ncam,nH,Nv,2,Dh] in the
    head-pair layout (msda_pack_pairs_bf16, msda_value_proj_pairs_bf16);
    reference_points_cam float32 [Ncam,B,Nq,D,2];
    bev_mask uint8|bool [Ncam,B,Nq,D]; sampling_offsets float32
    [B,Nq,nH,L,P,2]; attention_logits float32 [B,Nq,nH,L*P].

    Returns slots float32 [B,Nq,nH*Dh].  hit_count (int32 [B,Nq]),
    pair_offsets (int32 [B*Ncam+1]) and pair_q (int32 [B*Ncam*Nq]) are
    filled when given.  workspace: uint8 tensor of >= sca_workspace_size()
    bytes, allocated here when None."""
    lib = load_library()
    B, Ncam, Nv, nH, Dh, vdt = _sca_value(value)
    _, _, Nq, D, _ = reference_points_cam.shape
    _, _, _, L, P, _ = sampling_offsets.shape
    _sca_inputs(B, Ncam, Nq, D, nH, L, P, spatial_shapes, level_start_index, reference_points_cam, sampling_offsets,
                attention_logits)
    _numel(slots, "slots", B * Nq * nH * Dh, at_least=True)
    dev = value.device
    if slots is None:
        slots = torch.empty((B, Nq, nH * Dh), dtype=torch.float32, device=dev)
    _sca_outputs(B, Ncam, Nq, hit_count, pair_offsets, pair_q)
    _numel(bev_mask, "bev_mask", Ncam * B * Nq * D)
    need = sca_workspace_size(B, Ncam, Nq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    i32 = (torch.int32,)
    rc = lib.sca_forward(_ptr(value, "value"), vdt, _ptr(spatial_shapes, "spatial_shapes", _I64),
                         _ptr(level_start_index, "level_start_index", _I64),
                         _ptr(reference_points_cam, "reference_points_cam", _F32),
                         _ptr(bev_mask, "bev_mask", (torch.uint8, torch.bool)),
                         _ptr(sampling_offsets, "sampling_offsets", _F32),
                         _ptr(attention_logits, "attention_logits", _F32), B, Ncam, Nv, Nq, nH, Dh, L, P, D,
                         _ptr(slots, "slots", _F32), _ptr(hit_count, "hit_count", i32),
                         _ptr(pair_offsets, "pair_offsets", i32), _ptr(pair_q, "pair_q", i32),
                         _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                         _stream(stream, dev))
    _check("sca_forward", rc)
    return slots


@_given_stream
def sca_forward_noalloc(value, spatial_shapes, level_start_index, reference_points_cam, bev_mask, sampling_offsets,
                        attention_logits, slots, hit_count=None, pair_offsets=None, pair_q=None, stream=None):
    """sca_forward with the SCA workspace in the library's static device
    array (16 MiB per device): neither the library nor this binding
    allocates, so slots must be given.  Calls that may overlap on one device
    race on that array; order them."""
    lib = load_library()
    B, Ncam, Nv, nH, Dh, vdt = _sca_value(value)
    _, _, Nq, D, _ = reference_points_cam.shape
    _, _, _, L, P, _ = sampling_offsets.shape
    _sca_inputs(B, Ncam, Nq, D, nH, L, P, spatial_shapes, level_start_index, reference_points_cam, sampling_offsets,
                attention_logits)
    if slots is None:
        raise ValueError("slots: sca_forward_noalloc allocates nothing; pass the output tensor")
    _numel(slots, "slots", B * Nq * nH * Dh, at_least=True)
    _sca_outputs(B, Ncam, Nq, hit_count, pair_offsets, pair_q)
    _numel(bev_mask, "bev_mask", Ncam * B * Nq * D)
    i32 = (torch.int32,)
    rc = lib.sca_forward_noalloc(_ptr(value, "value"), vdt,
                                 _ptr(spatial_shapes, "spatial_shapes", _I64),
                                 _ptr(level_start_index, "level_start_index", _I64),
                                 _ptr(reference_points_cam, "reference_points_cam", _F32),
                                 _ptr(bev_mask, "bev_mask", (torch.uint8, torch.bool)),
                                 _ptr(sampling_offsets, "sampling_offsets", _F32),
                                 _ptr(attention_logits, "attention_logits", _F32), B, Ncam, Nv, Nq, nH, Dh, L, P, D,
                                 _ptr(slots, "slots", _F32), _ptr(hit_count, "hit_count", i32),
                                 _ptr(pair_offsets, "pair_offsets", i32), _ptr(pair_q, "pair_q", i32),
                                 _stream(stream, value.device))
    _check("sca_forward_noalloc", rc)
    return slots


@_given_stream
def sca_compact(bev_mask, reference_points_cam, workspace, hit_count=None, pair_offsets=None, pair_q=None,
                stream=None):
    """Stage 1 of sca_forward: bev_mask uint8|bool [Ncam,B,Nq,D] and
    reference_points_cam float32 [Ncam,B,Nq,D,2] -> camera masks, pair lists
    and the ordered work list in `workspace` (and hit_count / pair_offsets /
    pair_q when given)."""
    lib = load_library()
    Ncam, B, Nq, D = bev_mask.shape
    _numel(reference_points_cam, "reference_points_cam", Ncam * B * Nq * D * 2)
    _sca_outputs(B, Ncam, Nq, hit_count, pair_offsets, pair_q)
    i32 = (torch.int32,)
    rc = lib.sca_compact(_ptr(bev_mask, "bev_mask", (torch.uint8, torch.bool)),
                         _ptr(reference_points_cam, "reference_points_cam", _F32), B, Ncam, Nq, D,
                         _ptr(hit_count, "hit_count", i32), _ptr(pair_offsets, "pair_offsets", i32),
                         _ptr(pair_q, "pair_q", i32), _ptr(workspace, "workspace"),
                         workspace.numel() * workspace.element_size(), _stream(stream, bev_mask.device))
    _check("sca_compact", rc)


@_given_stream
def sca_gather(value, spatial_shapes, level_start_index, reference_points_cam, sampling_offsets, attention_logits,
               workspace, slots=None, stream=None):
    """Stage 2 of sca_forward: gather, weighted sums and camera mean for the
    queries on the work list the preceding sca_compact left in `workspace`."""
    lib = load_library()
    B, Ncam, Nv, nH, Dh, vdt = _sca_value(value)
    _, _, Nq, D, _ = reference_points_cam.shape
    _, _, _, L, P, _ = sampling_offsets.shape
    _sca_inputs(B, Ncam, Nq, D, nH, L, P, spatial_shapes, level_start_index, reference_points_cam, sampling_offsets,
                attention_logits)
    _numel(slots, "slots", B * Nq * nH * Dh, at_least=True)
    dev = value.device
    if slots is None:
        slots = torch.empty((B, Nq, nH * Dh), dtype=torch.float32, device=dev)
    rc = lib.sca_gather(_ptr(value, "value"), vdt, _ptr(spatial_shapes, "spatial_shapes", _I64),
                        _ptr(level_start_index, "level_start_index", _I64),
                        _ptr(reference_points_cam, "reference_points_cam", _F32),
                        _ptr(sampling_offsets, "sampling_offsets", _F32),
                        _ptr(attention_logits, "attention_logits", _F32), B, Ncam, Nv, Nq, nH, Dh, L, P, D,
                        _ptr(slots, "slots", _F32), _ptr(workspace, "workspace"),
                        workspace.numel() * workspace.element_size(), _stream(stream, dev))
    _check("sca_gather", rc)
    return slots


@_given_stream
def msda_gemm_bf16(X, W, bias=None, y_dtype=torch.bfloat16, out=None, stream=None):
    """Y = X W^T + bias.  X [M,K] bfloat16 (or float32, rounded to bf16 as
    read); W bfloat16 [N,K]; bias float32 [N] or None.  Returns Y [M,N] of
    y_dtype (bfloat16 or float32)."""
    lib = load_library()
    M, K = X.shape
    N = W.shape[0]
    _numel(W, "W", N * K)
    _numel(bias, "bias", N)
    _numel(out, "out", M * N, at_least=True)
    if out is None:
        out = torch.empty((M, N), dtype=y_dtype, device=X.device)
    x_dt = MSDA_F32 if X.dtype == torch.float32 else MSDA_BF16
    y_dt = MSDA_F32 if out.dtype == torch.float32 else MSDA_BF16
    rc = lib.msda_gemm_bf16(_ptr(X, "X", (torch.float32, torch.bfloat16)), x_dt, _ptr(W, "W", (torch.bfloat16,)),
                            _ptr(bias, "bias", _F32), _ptr(out, "out", (torch.float32, torch.bfloat16)), y_dt,
                            M, N, K, _stream(stream, X.device))
    _check("msda_gemm_bf16", rc)
    return out


@_given_stream
def msda_value_proj_pairs_bf16(X, W, bias, Nv, out=None, stream=None):
    """The value projection X W^T + bias (X [M,K] float32 or bfloat16, W
    bfloat16 [N,K], bias float32 [N] or None) written in bfloat16 in the
    head-pair layout: returns out [M/Nv, N/32, Nv, 2, 32], the M rows being
    M/Nv value images of Nv pixels."""
    lib = load_library()
    M, K = X.shape
    N = W.shape[0]
    _numel(W, "W", N * K)
    _numel(bias, "bias", N)
    n_img = M // Nv if Nv > 0 else 0
    _numel(out, "out", n_img * (N // 32) * Nv * 64, at_least=True)
    if out is None:
        out = torch.empty((n_img, N // 32, Nv, 2, 32), dtype=torch.bfloat16, device=X.device)
    x_dt = MSDA_F32 if X.dtype == torch.float32 else MSDA_BF16
    rc = lib.msda_value_proj_pairs_bf16(_ptr(X, "X", (torch.float32, torch.bfloat16)), x_dt,
                                        _ptr(W, "W", (torch.bfloat16,)), _ptr(bias, "bias", _F32),
                                        _ptr(out, "out", (torch.bfloat16,)), M, N, K, Nv, _stream(stream, X.device))
    _check("msda_value_proj_pairs_bf16", rc)
    return out


@_given_stream
def msda_pack_pairs_bf16(value, out=None, stream=None):
    """A bfloat16 value [..., Nv, nH, 32] rewritten in the head-pair layout:
    returns out [..., nH, Nv, 2, 32] (every element keeps its bits; the
    right half of each head's last line is zero)."""
    lib = load_library()
    *lead, Nv, nH, Dh = value.shape
    if Dh != 32:
        raise ValueError(f"value: the last dimension must be 32 channels, got {Dh}")
    n_img = 1
    for d in lead:
        n_img *= d
    _numel(out, "out", n_img * nH * Nv * 64, at_least=True)
    if out is None:
        out = torch.empty((*lead, nH, Nv, 2, 32), dtype=torch.bfloat16, device=value.device)
    rc = lib.msda_pack_pairs_bf16(_ptr(value, "value", (torch.bfloat16,)), _ptr(out, "out", (torch.bfloat16,)),
                                  n_img, Nv, nH, _stream(stream, value.device))
    _check("msda_pack_pairs_bf16", rc)
    return out


@_given_stream
def msda_query_proj_bf16(query, W_off, b_off, W_att, b_att, query_pos=None, offsets=None, logits=None,
                         stream=None):
    """Sampling offsets and attention logits from the query in one launch:
    q~ = query + query_pos (float32), offsets = bf16(q~) W_off^T + b_off,
    logits = bf16(q~) W_att^T + b_att.  query, query_pos float32 [M,K];
    W_* bfloat16 [N_*,K]; b_* float32 [N_*] or None.  Returns (offsets
    [M,N_off], logits [M,N_att]) float32."""
    lib = load_library()
    M, K = query.shape
    N_off, N_att = W_off.shape[0], W_att.shape[0]
    _numel(query_pos, "query_pos", M * K)
    _numel(W_off, "W_off", N_off * K)
    _numel(W_att, "W_att", N_att * K)
    _numel(b_off, "b_off", N_off)
    _numel(b_att, "b_att", N_att)
    _numel(offsets, "offsets", M * N_off, at_least=True)
    _numel(logits, "logits", M * N_att, at_least=True)
    if offsets is None:
        offsets = torch.empty((M, N_off), dtype=torch.float32, device=query.device)
    if logits is None:
        logits = torch.empty((M, N_att), dtype=torch.float32, device=query.device)
    rc = lib.msda_query_proj_bf16(_ptr(query, "query", _F32), _ptr(query_pos, "query_pos", _F32),
                                  _ptr(W_off, "W_off", (torch.bfloat16,)), _ptr(b_off, "b_off", _F32),
                                  _ptr(W_att, "W_att", (torch.bfloat16,)), _ptr(b_att, "b_att", _F32),
                                  _ptr(offsets, "offsets", _F32), _ptr(logits, "logits", _F32), M, K, N_off, N_att,
                                  _stream(stream, query.device))
    _check("msda_query_proj_bf16", rc)
    return offsets, logits


@_given_stream
def msda_output_proj_bf16(X, W, bias=None, residual=None, gamma=None, beta=None, eps=1e-5, out=None, stream=None):
    """residual + (bf16(X) W^T + bias), then, with gamma, the layer norm of
    each row (divisor N, eps inside the square root) scaled by gamma and
    shifted by beta.  X float32 or bfloat16 [M,K]; W bfloat16 [N,K];
    residual float32 [M,N] (may be `out`); bias, gamma, beta float32 [N].
    Returns float32 [M,N]."""
    lib = load_library()
    M, K = X.shape
    N = W.shape[0]
    _numel(W, "W", N * K)
    for t, name in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        _numel(t, name, N)
    _numel(residual, "residual", M * N)
    _numel(out, "out", M * N, at_least=True)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    x_dt = MSDA_F32 if X.dtype == torch.float32 else MSDA_BF16
    rc = lib.msda_output_proj_bf16(_ptr(X, "X", (torch.float32, torch.bfloat16)), x_dt,
                                   _ptr(W, "W", (torch.bfloat16,)), _ptr(bias, "bias", _F32),
                                   _ptr(residual, "residual", _F32), _ptr(gamma, "gamma", _F32),
                                   _ptr(beta, "beta", _F32), float(eps), _ptr(out, "out", _F32), M, N, K,
                                   _stream(stream, X.device))
    _check("msda_output_proj_bf16", rc)
    return out


@_given_stream
def sca_rebatch(pair_offsets, pair_q, reference_points_cam, sampling_offsets, attention_logits, spatial_shapes,
                max_len, sampling_locations=None, logits_out=None, stream=None):
    """Padded rebatch of the pair lists (A/B baseline): sampling locations
    rho + offset / (W, H) and logits for every row of the [B*Ncam, max_len]
    segments (zeros past a segment's end).  Returns (sampling_locations
    [B*Ncam, max_len, nH, L, P, 2], logits [B*Ncam, max_len, nH, L*P])."""
    lib = load_library()
    Ncam, B, Nq, D, _ = reference_points_cam.shape
    _, _, nH, L, P, _ = sampling_offsets.shape
    _numel(spatial_shapes, "spatial_shapes", 2 * L)
    _numel(sampling_offsets, "sampling_offsets", B * Nq * nH * L * P * 2)
    _numel(attention_logits, "attention_logits", B * Nq * nH * L * P)
    _numel(pair_offsets, "pair_offsets", B * Ncam + 1)
    _numel(pair_q, "pair_q", B * Ncam * Nq, at_least=True)
    _numel(sampling_locations, "sampling_locations", B * Ncam * max_len * nH * L * P * 2, at_least=True)
    _numel(logits_out, "logits_out", B * Ncam * max_len * nH * L * P, at_least=True)
    dev = reference_points_cam.device
    if sampling_locations is None:
        sampling_locations = torch.empty((B * Ncam, max_len, nH, L, P, 2), dtype=torch.float32, device=dev)
    if logits_out is None:
        logits_out = torch.empty((B * Ncam, max_len, nH, L * P), dtype=torch.float32, device=dev)
    i32 = (torch.int32,)
    rc = lib.sca_rebatch(_ptr(pair_offsets, "pair_offsets", i32), _ptr(pair_q, "pair_q", i32),
                         _ptr(reference_points_cam, "reference_points_cam", _F32),
                         _ptr(sampling_offsets, "sampling_offsets", _F32),
                         _ptr(attention_logits, "attention_logits", _F32),
                         _ptr(spatial_shapes, "spatial_shapes", _I64), B, Ncam, Nq, nH, L, P, D, max_len,
                         _ptr(sampling_locations, "sampling_locations", _F32), _ptr(logits_out, "logits_out", _F32),
                         _stream(stream, dev))
    _check("sca_rebatch", rc)
    return sampling_locations, logits_out


@_given_stream
def sca_scatter_mean(rows, pair_offsets, pair_q, hit_count, Nq, slots=None, stream=None):
    """slots[b, q] = mean over the cameras that see q of their segment rows
    (zero where no camera does).  rows float32 [B*Ncam, max_len, C];
    hit_count int32 [B, Nq].  Returns slots float32 [B, Nq, C]."""
    lib = load_library()
    BN, max_len, C = rows.shape
    B = hit_count.shape[0]
    Ncam = BN // max(B, 1)
    if B * Ncam != BN:
        raise ValueError(f"rows: {BN} segments is not a multiple of the batch {B} of hit_count")
    _numel(hit_count, "hit_count", B * Nq)
    _numel(pair_offsets, "pair_offsets", B * Ncam + 1)
    _numel(pair_q, "pair_q", B * Ncam * Nq, at_least=True)
    _numel(slots, "slots", B * Nq * C, at_least=True)
    if slots is None:
        slots = torch.empty((B, Nq, C), dtype=torch.float32, device=rows.device)
    i32 = (torch.int32,)
    rc = lib.sca_scatter_mean(_ptr(rows, "rows", _F32), _ptr(pair_offsets, "pair_offsets", i32),
                              _ptr(pair_q, "pair_q", i32), _ptr(hit_count, "hit_count", i32), B, Ncam, Nq, C, max_len,
                              _ptr(slots, "slots", _F32), _stream(stream, rows.device))
    _check("sca_scatter_mean", rc)
    return slots


@_given_stream
def sca_forward_rebatch(value, spatial_shapes, level_start_index, reference_points_cam, bev_mask, sampling_offsets,
                        attention_logits, workspace=None, stream=None):
    """SCA through the padded rebatch flow (A/B baseline for sca_forward):
    sca_compact, the longest segment read back to the host (as the note's
    code does), sca_rebatch, msda_forward over the B*Ncam segments,
    sca_scatter_mean.  Same arguments and result as sca_forward; returns
    (slots, max_len)."""
    B, Ncam, Nv, nH, Dh = value.shape
    _, _, Nq, D, _ = reference_points_cam.shape
    dev = value.device
    if workspace is None:
        workspace = torch.empty(sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device=dev)
    hit = torch.empty((B, Nq), dtype=torch.int32, device=dev)
    offs = torch.empty(B * Ncam + 1, dtype=torch.int32, device=dev)
    pq = torch.empty(max(1, B * Ncam * Nq), dtype=torch.int32, device=dev)
    sca_compact(bev_mask, reference_points_cam, workspace, hit_count=hit, pair_offsets=offs, pair_q=pq,
                stream=stream)
    o = offs.cpu().numpy()  # the host reads the segment bounds back, as the note's code does
    max_len = int((o[1:] - o[:-1]).max()) if B * Ncam > 0 else 0
    loc, lg = sca_rebatch(offs, pq, reference_points_cam, sampling_offsets, attention_logits, spatial_shapes,
                          max_len, stream=stream)
    rows = msda_forward(value.view(B * Ncam, Nv, nH, Dh), spatial_shapes, level_start_index, loc, lg,
                        weight_mode=MSDA_WEIGHTS_LOGITS, stream=stream) if max_len > 0 else \
        torch.empty((B * Ncam, 0, nH * Dh), dtype=torch.float32, device=dev)
    slots = sca_scatter_mean(rows.view(B * Ncam, max_len, nH * Dh), offs, pq, hit, Nq, stream=stream)
    return slots, max_len


def msda_backward_workspace_size(B, Nv, Nq, nH, L, P):
    lib = load_library()
    n = _sz(0)
    _check("msda_backward_workspace_size",
           lib.msda_backward_workspace_size(int(B), int(Nv), int(Nq), int(nH), int(L), int(P), ctypes.byref(n)))
    return n.value


def sca_backward_workspace_size(B, Ncam, Nv, Nq, nH, L, P, max_pairs=0):
    lib = load_library()
    n = _sz(0)
    _check("sca_backward_workspace_size",
           lib.sca_backward_workspace_size(int(B), int(Ncam), int(Nv), int(Nq), int(nH), int(L), int(P),
                                           int(max_pairs), ctypes.byref(n)))
    return n.value


def _grad_workspace(given, nbytes, dev):
    if given is not None:
        return given
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


def _grads_of(samples, locations, weights, grad_out, n_out, grad_value, n_value, grad_locations, grad_weights,
              out_name="grad_out"):
    """Sizes of a backward call's sample inputs, upstream gradient and outputs."""
    _numel(locations, "sampling locations / offsets", 2 * samples)
    _numel(weights, "attention weights / logits", samples)
    _numel(grad_out, out_name, n_out)
    _numel(grad_value, "grad_value", n_value, at_least=True)
    _numel(grad_locations, "grad_locations / grad_offsets", 2 * samples, at_least=True)
    _numel(grad_weights, "grad_weights / grad_logits", samples, at_least=True)


@_given_stream
def msda_backward(value, spatial_shapes, level_start_index, sampling_locations, attention_weights, grad_out,
                  weight_mode=MSDA_WEIGHTS_LOGITS, grad_value=None, grad_locations=None, grad_weights=None,
                  grad_workspace=None, atomic=False, stream=None):
    """Gradients of msda_forward for grad_out = d loss / d out [B,Nq,nH*Dh].
    Returns (grad_value float32 [B,Nv,nH,Dh], grad_locations [B,Nq,nH,L,P,2],
    grad_weights [B,Nq,nH,L*P]); grad_weights is with respect to the weights
    as given (logits or probabilities, per weight_mode).  The value gradient
    is a deterministic transpose gather through a gradient workspace (made
    here unless given), or float32 atomics with atomic=True."""
    lib = load_library()
    B, Nv, nH, Dh = value.shape
    _, Nq, _, L, P, _ = sampling_locations.shape
    _levels(spatial_shapes, level_start_index, L)
    _grads_of(B * Nq * nH * L * P, sampling_locations, attention_weights, grad_out, B * Nq * nH * Dh, grad_value,
              B * Nv * nH * Dh, grad_locations, grad_weights)
    dev = value.device
    if grad_value is None:
        grad_value = torch.empty((B, Nv, nH, Dh), dtype=torch.float32, device=dev)
    if grad_locations is None:
        grad_locations = torch.empty_like(sampling_locations)
    if grad_weights is None:
        grad_weights = torch.empty_like(attention_weights)
    gws, gws_bytes = None, 0
    if not atomic:
        gws = _grad_workspace(grad_workspace, msda_backward_workspace_size(B, Nv, Nq, nH, L, P), dev)
        gws_bytes = gws.numel() * gws.element_size()
    rc = lib.msda_backward(_ptr(value, "value"), _value_dtype(value), _ptr(spatial_shapes, "spatial_shapes", _I64),
                           _ptr(level_start_index, "level_start_index", _I64),
                           _ptr(sampling_locations, "sampling_locations", _F32),
                           _ptr(attention_weights, "attention_weights", _F32), int(weight_mode),
                           _ptr(grad_out, "grad_out", _F32), B, Nv, Nq, nH, Dh, L, P,
                           _ptr(grad_value, "grad_value", _F32), _ptr(grad_locations, "grad_locations", _F32),
                           _ptr(grad_weights, "grad_weights", _F32),
                           None if gws is None else _ptr(gws, "grad_workspace"), gws_bytes, _stream(stream, dev))
    _check("msda_backward", rc)
    return grad_value, grad_locations, grad_weights


@_given_stream
def msda_backward_frames(value, spatial_shapes, level_start_index, sampling_locations, attention_weights, grad_out,
                         weight_mode=MSDA_WEIGHTS_LOGITS, grad_value=None, grad_locations=None, grad_weights=None,
                         grad_workspace=None, atomic=False, stream=None):
    """Gradients of msda_forward_frames for grad_out = d loss / d out
    [B,Nq,nH*Dh]: value [B,F,Nv,nH,Dh], locations [B,F,Nq,nH,L,P,2], weights
    [B,F,Nq,nH,L*P].  Returns (grad_value float32 [B,F,Nv,nH,Dh],
    grad_locations, grad_weights) shaped as their inputs; the value gradient
    as for msda_backward (gradient workspace of B*F images)."""
    lib = load_library()
    B, F, Nv, nH, Dh = value.shape
    _, _, Nq, _, L, P, _ = sampling_locations.shape
    _levels(spatial_shapes, level_start_index, L)
    _grads_of(B * F * Nq * nH * L * P, sampling_locations, attention_weights, grad_out, B * Nq * nH * Dh,
              grad_value, B * F * Nv * nH * Dh, grad_locations, grad_weights)
    dev = value.device
    if grad_value is None:
        grad_value = torch.empty((B, F, Nv, nH, Dh), dtype=torch.float32, device=dev)
    if grad_locations is None:
        grad_locations = torch.empty_like(sampling_locations)
    if grad_weights is None:
        grad_weights = torch.empty_like(attention_weights)
    gws, gws_bytes = None, 0
    if not atomic:
        gws = _grad_workspace(grad_workspace, msda_backward_workspace_size(B * F, Nv, Nq, nH, L, P), dev)
        gws_bytes = gws.numel() * gws.element_size()
    rc = lib.msda_backward_frames(_ptr(value, "value"), _value_dtype(value),
                                  _ptr(spatial_shapes, "spatial_shapes", _I64),
                                  _ptr(level_start_index, "level_start_index", _I64),
                                  _ptr(sampling_locations, "sampling_locations", _F32),
                                  _ptr(attention_weights, "attention_weights", _F32), int(weight_mode),
                                  _ptr(grad_out, "grad_out", _F32), B, F, Nv, Nq, nH, Dh, L, P,
                                  _ptr(grad_value, "grad_value", _F32), _ptr(grad_locations, "grad_locations", _F32),
                                  _ptr(grad_weights, "grad_weights", _F32),
                                  None if gws is None else _ptr(gws, "grad_workspace"), gws_bytes,
                                  _stream(stream, dev))
    _check("msda_backward_frames", rc)
    return grad_value, grad_locations, grad_weights


@_given_stream
def sca_backward(value, spatial_shapes, level_start_index, reference_points_cam, sampling_offsets, attention_logits,
                 grad_slots, workspace, grad_value=None, grad_offsets=None, grad_logits=None, max_pairs=0,
                 grad_workspace=None, atomic=False, stream=None):
    """Gradients of SCA for grad_slots = d loss / d slots [B,Nq,nH*Dh].  The
    workspace must hold sca_compact's result for the same mask and anchors.
    Returns (grad_value float32 [B,Ncam,Nv,nH,Dh], grad_offsets
    [B,Nq,nH,L,P,2], grad_logits [B,Nq,nH,L*P]).  The value gradient is a
    deterministic transpose gather through a gradient workspace for up to
    max_pairs camera-query pairs (0: every camera seeing every query), made
    here unless given, or float32 atomics with atomic=True."""
    lib = load_library()
    B, Ncam, Nv, nH, Dh = value.shape
    _, _, Nq, D, _ = reference_points_cam.shape
    _, _, _, L, P, _ = sampling_offsets.shape
    _sca_inputs(B, Ncam, Nq, D, nH, L, P, spatial_shapes, level_start_index, reference_points_cam, sampling_offsets,
                attention_logits)
    _grads_of(B * Nq * nH * L * P, sampling_offsets, attention_logits, grad_slots, B * Nq * nH * Dh, grad_value,
              B * Ncam * Nv * nH * Dh, grad_offsets, grad_logits, out_name="grad_slots")
    dev = value.device
    if grad_value is None:
        grad_value = torch.empty((B, Ncam, Nv, nH, Dh), dtype=torch.float32, device=dev)
    if grad_offsets is None:
        grad_offsets = torch.empty_like(sampling_offsets)
    if grad_logits is None:
        grad_logits = torch.empty_like(attention_logits)
    gws, gws_bytes = None, 0
    if not atomic:
        need = sca_backward_workspace_size(B, Ncam, Nv, Nq, nH, L, P, max_pairs)
        gws = _grad_workspace(grad_workspace, need, dev)
        gws_bytes = gws.numel() * gws.element_size()
    rc = lib.sca_backward(_ptr(value, "value"), _value_dtype(value), _ptr(spatial_shapes, "spatial_shapes", _I64),
                          _ptr(level_start_index, "level_start_index", _I64),
                          _ptr(reference_points_cam, "reference_points_cam", _F32),
                          _ptr(sampling_offsets, "sampling_offsets", _F32),
                          _ptr(attention_logits, "attention_logits", _F32), _ptr(grad_slots, "grad_slots", _F32),
                          B, Ncam, Nv, Nq, nH, Dh, L, P, D, _ptr(grad_value, "grad_value", _F32),
                          _ptr(grad_offsets, "grad_offsets", _F32), _ptr(grad_logits, "grad_logits", _F32),
                          _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                          int(max_pairs), None if gws is None else _ptr(gws, "grad_workspace"), gws_bytes,
                          _stream(stream, dev))
    _check("sca_backward", rc)
    return grad_value, grad_offsets, grad_logits
