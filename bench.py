#!/usr/bin/env python
"""Benchmark of the BEVFormer-base spatial cross-attention (SCA) forward pass
on one MI355X, through libmsda.so's C ABI.

Workload (default, "sca"): BEVFormer-base SCA, fp32 value, batch 1, 6
cameras, 200x200 BEV queries, 4 levels per camera (116x200, 58x100, 29x50,
15x25), 8 heads x 32 channels, 8 points per level over 4 pillar anchors;
seeded synthetic inputs from workloads.bevformer_sca().  One step is the
whole hot path: visibility, compaction and work ordering of the (camera,
query) pairs (sca_compact) and the fused softmax / bilinear gather /
weighted sum / camera mean (sca_gather).  Inputs are resident in HBM before
timing starts.  Other workloads: "layer_bf16" (batch 4, bf16 value
projection GEMM writing the head-pair layout -> SCA on that bf16 value ->
bf16 output projection GEMM; "layer_bf16_plain" with the row-major bf16
value layout instead), "layer_full" (the same with the sampling offsets and
logits projected from query + position embedding in one launch, and the
output projection followed by the residual and the layer norm), "sca_bf16"
(the default workload on a row-major bf16 value), "sca_rebatch"
(the default workload through the padded rebatch flow of the SCA note, an
A/B baseline: per-camera segments padded to the longest, the operator over
all of them, scatter-add and divide), "sca_train", "detr_train" and
"tsa_train" (forward and backward of the default SCA layer, of the DETR
encoder MSDA and of the two-frame mean, the value gradient by the
deterministic transpose gather; "_atomic" variants accumulate it with
float32 atomics instead; the roofline then describes the backward kernel),
"detr" (Deformable-DETR encoder MSDA: each step builds the locality plan
from the sampling locations and runs the planned gather; "detr_unplanned"
the queries in input order; "detr_encoder6" one pass of the six-layer
encoder: the plan built once from the shared reference points before the
timed steps, then six layers' planned gathers), "tsa" (two stacked BEV maps, frame mean, the
BEV-grid queries in raster order; "tsa_planned" with a plan in every step,
"tsa_gridplan" with one built from the BEV grid before the timed steps),
"sca_frame6" (one frame of the encoder: one compaction serving six SCA
layers, each with its own value maps, offsets and logits), "tiny".

Prints one JSON line.  value = bilinear samples per second (one sample = one
(camera, query, head, level, point) bilinear read of 4 corners x 32
channels) over the whole step.  The K timed steps run eagerly, one library
call per part with HIP events between the parts; a step of more than one
call then runs again as K replays of the step captured once in a HIP graph
(one launch per step; the replays, run on outputs first overwritten, must
reproduce the eager outputs bit for bit, checked after the warm-up replays
and again after the timed ones), and ms_per_step and value come from the
replays' wall-clock time
(launch.eager holds the eager figures; --eager times the eager steps only,
and the padded rebatch flow, which reads a length back to the host, always
runs eagerly).  Kernel figures come from the eager steps' HIP events,
recorded on the stream the kernels run on:
  roofline         the main kernel against the 8 TB/s HBM peak, on the bytes
                   one launch must move at least once (every value map, the
                   per-query offsets or locations and weights, anchors,
                   masks and output); traffic = the bytes it moved beyond L2
                   in the committed counter run, while its sources match;
  roofline_onchip  the corner rows inside their map that the kernel reads,
                   per second, against the same kernel's rate when every
                   one of them sits in L2 (the level sides divided by 8,
                   same samples and work order), measured in the same run:
                   the ceiling of its vector-memory path;
  effective        all 4 nominal corners x 32 channels of every sample plus
                   metadata and output, per second: most of these bytes
                   come from L1 and L2, so it is a rate, not a fraction;
breakdown = the same events around every part of the step (mean,
p10/p50/p90); cold = the same step after a 1 GiB write that evicts L2 and
the memory-side cache (the headline is warm, back to back, as a layer runs
inside a network); batch_items_per_s = batch items (scenes) per second;
cpu_baseline = the CPU oracle on the same workload (or a bounded sample of
it), on one thread and on every core this process may use.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--eager]
  python bench.py --calibrate-copy   (a plain device copy of known size, for
                                      scaling the HBM byte counters)
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_MFMA_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix, published
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
_CSRC = "scale_deformable_attention_forward_amd/csrc/"
GATHER_SOURCES = [_CSRC + f for f in ("gather.hip", "sampling.hpp", "common.hpp", "internal.hpp")]
BACKWARD_SOURCES = [_CSRC + f for f in ("backward.hip", "backward.hpp", "sampling.hpp", "common.hpp", "vgrad.hpp")]
KERNEL_SOURCES = {"sca_gather_kernel": GATHER_SOURCES, "msda_gather_kernel": GATHER_SOURCES,
                  "sca_backward_kernel": BACKWARD_SOURCES, "msda_backward_kernel": BACKWARD_SOURCES}
METRIC = "MSDA samples/sec + effective HBM GB/s, BEVFormer-base SCA layer (6 cams)"


_CODE_TOKENS = re.compile(r'''"(?:\\.|[^"\\\n])*"|'(?:\\.|[^'\\\n])*'|//[^\n]*|/\*.*?\*/|(?:[^\s"'/]|/(?![/*]))+''', re.S)


def source_digest(paths=GATHER_SOURCES):
    """Hash of the kernel sources' code: comments and layout do not count,
    so a comment edit keeps a counter run valid; any code change does not."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            toks = [t for t in _CODE_TOKENS.findall(f.read()) if not t.startswith(("//", "/*"))]
        h.update("\n".join(toks).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """Bytes per launch of the workload's main kernel moved between L2 and
    memory (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy) from the
    committed rocprofv3 counter runs, or None when there is none or the
    kernel's sources changed since it was taken.  Reads served by the
    memory-side Infinity Cache count too, so this bounds the HBM bytes from
    above."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)[workload]
    except (OSError, KeyError, ValueError):
        return None
    if c.get("source_digest") != source_digest(KERNEL_SOURCES.get(kernel, GATHER_SOURCES)):
        return None
    return c.get("hbm_bytes_per_launch")


def host_cpu():
    """The host the CPU baseline ran on: processor model and the cores this
    process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"host_cpu": model, "host_cores_available": len(os.sched_getaffinity(0))}


def calibrate_copy():
    import torch
    n = 1 << 28  # 256 Mi floats = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4}))


def _query_chunks(n, k):
    """k contiguous ranges covering range(n) (empty ones dropped)."""
    import numpy as np
    return [r for r in np.array_split(np.arange(n, dtype=np.int64), k) if len(r)]


def time_oracle(phases, n_samples, what, cores=None):
    """Times the CPU oracle over a bounded sample of a workload, given as
    phases of independent tasks (a phase may use what the one before
    wrote): first every task one after the other on one thread, then each
    phase's tasks spread over every core this process may use.  ctypes
    releases the interpreter lock while the C oracle runs, and numpy's BLAS
    is held to one thread per task, so the second figure is the same oracle
    on `cores` threads; the oracle itself is not changed for it."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    cores = cores or len(os.sched_getaffinity(0))
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for phase in phases:
            for task in phase:
                task()
        t_one = time.perf_counter() - t0
        with ThreadPoolExecutor(cores) as ex:
            t0 = time.perf_counter()
            for phase in phases:
                list(ex.map(lambda task: task(), phase))
            t_all = time.perf_counter() - t0
    tasks = sum(len(p) for p in phases)
    return {"value": n_samples / t_all, "unit": "samples/s", "cores": cores, "kind": "oracle",
            "sample": f"{what} ({n_samples} samples); {tasks} independent tasks on {cores} threads "
                      f"{t_all:.2f} s, on one thread {t_one:.2f} s",
            "seconds": t_all, "single_thread": {"value": n_samples / t_one, "cores": 1, "seconds": t_one}}


def _sca_samples(w, rows=None):
    """Bilinear samples of an SCA workload: every (camera, query) pair a
    camera sees, times heads x levels x points (restricted to flat query
    rows b*Nq + q when given).  Measurement metadata only."""
    import numpy as np
    hit = w["bev_mask"].any(-1).sum(0).reshape(-1)  # cameras seeing each (b, q)
    if rows is not None:
        hit = hit[rows]
    return int(hit.sum()) * w["nH"] * w["L"] * w["P"]


def sca_cpu_baseline(w, kind, cores=None, sampled_queries=4000):
    """The oracle on an SCA workload: the whole of it for the single-layer
    kinds; for the batch-4 layers the value projection of every row, then
    (the query projections,) SCA and the output projection of
    `sampled_queries` sampled queries."""
    import numpy as np
    import oracle
    import workloads as W
    B, Ncam, Nq, Nv, nH, L, P = w["B"], w["Ncam"], w["Nq"], w["Nv"], w["nH"], w["L"], w["P"]
    C = nH * 32
    k = 4 * (cores or len(os.sched_getaffinity(0)))
    geo = (w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"], w["bev_mask"])
    if kind not in ("layer_bf16", "layer_full"):
        value = w["value"]
        tasks = [lambda r=r: oracle.sca(value, *geo, w["sampling_offsets"], w["attention_logits"], rows=r)
                 for r in _query_chunks(B * Nq, k)]
        what = f"the whole workload: all {B * Nq} queries" + (" of the first of the six layers"
                                                              if kind == "sca_frame6" else "")
        return time_oracle([tasks], _sca_samples(w), what, cores)
    full = kind == "layer_full"
    rows = W.sample_rows(7, B * Nq, sampled_queries)
    feat = w["feat"].reshape(-1, C)
    v = np.empty((B * Ncam * Nv, C), np.uint16)

    def value_proj(r):
        v[r] = oracle.round_to_bf16(oracle.linear_bf16_blas(feat[r], w["W_v"], w["b_v"]))
    phases = [[lambda r=r: value_proj(r) for r in _query_chunks(B * Ncam * Nv, k)]]
    if full:
        q, e = w["query"].reshape(-1, C), w["query_pos"].reshape(-1, C)
        off_rows = np.zeros((B * Nq, nH * L * P * 2), np.float32)
        lg_rows = np.zeros((B * Nq, nH * L * P), np.float32)

        def query_proj(r):
            off_rows[r], lg_rows[r] = oracle.query_proj(q[r], e[r], w["W_off"], w["b_off"], w["W_att"], w["b_att"])
        phases.append([lambda r=r: query_proj(r) for r in np.array_split(rows, k) if len(r)])
        off, lg = off_rows.reshape(B, Nq, nH, L, P, 2), lg_rows.reshape(B, Nq, nH, L * P)
    else:
        off, lg = w["sampling_offsets"], w["attention_logits"]

    def sca_and_output(r):
        slots = oracle.sca(v.reshape(B, Ncam, Nv, nH, 32), *geo, off, lg, rows=r)["slots"]
        if full:
            oracle.output_proj(slots.astype(np.float32), w["W_o"], w["b_o"], q[r], w["gamma"], w["beta"])
        else:
            oracle.linear_bf16(oracle.round_to_bf16(slots), w["W_o"], w["b_o"])
    phases.append([lambda r=r: sca_and_output(r) for r in np.array_split(rows, k) if len(r)])
    what = (f"value projection of all {B * Ncam * Nv} rows, then {'query projections, ' if full else ''}SCA and "
            f"output projection of {len(rows)} sampled queries; C loops and a float64 matmul")
    return time_oracle(phases, _sca_samples(w, rows), what, cores)


def msda_cpu_baseline(w, cores=None, first_of=1):
    """The oracle's MSDA operator (or frame mean) over the whole workload (of
    its first layer when a step runs `first_of` layers)."""
    import oracle
    k = 4 * (cores or len(os.sched_getaffinity(0)))
    B, Nq, nH, L, P = w["B"], w["Nq"], w["nH"], w["L"], w["P"]
    F = w.get("F", 1)
    args = (w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"], w["attention_weights"])
    fn = oracle.msda if F == 1 else oracle.msda_frames
    tasks = [lambda r=r: fn(*args, True, rows=r) for r in _query_chunks(B * Nq, k)]
    what = f"the whole workload: all {B * Nq} queries" + (f" of the first of the {first_of} layers" if first_of > 1
                                                              else "")
    return time_oracle([tasks], B * F * Nq * nH * L * P, what, cores)


def train_cpu_baseline(w, which, grad, cores=None):
    """The oracle's forward and backward over the whole workload, split into
    query ranges, each run as a smaller problem of its own (the value
    gradient of the whole is the sum of the ranges' ones; the timing keeps
    them apart).  One range per core: each backward call fills a float64
    value gradient of the whole map."""
    import oracle
    cores = cores or len(os.sched_getaffinity(0))
    B, Nq, nH, L, P = w["B"], w["Nq"], w["nH"], w["L"], w["P"]
    ranges = [slice(int(r[0]), int(r[-1]) + 1) for r in _query_chunks(Nq, cores)]
    if which == "sca_train":
        def task(s):
            a = (w["value"], w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"][:, :, s],
                 w["bev_mask"][:, :, s], w["sampling_offsets"][:, s], w["attention_logits"][:, s])
            oracle.sca(*a)
            oracle.sca_backward(*a, grad[:, s])
        n = _sca_samples(w)
    elif which == "tsa_train":
        def task(s):
            a = (w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"][:, :, s],
                 w["attention_weights"][:, :, s])
            oracle.msda_frames(*a, True)
            oracle.msda_frames_backward(*a, grad[:, s], weights_are_logits=True)
        n = B * w["F"] * Nq * nH * L * P
    else:
        def task(s):
            a = (w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"][:, s],
                 w["attention_weights"][:, s])
            oracle.msda(*a, True)
            oracle.msda_backward(*a, grad[:, s], weights_are_logits=True)
        n = B * Nq * nH * L * P
    return time_oracle([[lambda s=s: task(s) for s in ranges]], n,
                       f"the whole workload, forward and backward, over {len(ranges)} query ranges", cores)


class Workload:
    """Inputs on the device and the step, as a list of named parts.  `main`
    names the dominant kernel's part; finish() fills in the sample count and
    the per-launch byte and flop figures after a warm-up."""

    def __init__(self, name):
        self.name = name
        self.parts = []
        self.main = None
        self.extra = {}
        self.batch = 1
        self.inbounds_corners = None  # corners inside their map, per gather launch
        self.unique_bytes = None  # bytes one launch of the main part must move at least once
        self.onchip = None  # callable: the main kernel's rate with every corner row in L2
        self.graph = True  # the step can be captured in a HIP graph (nothing read back to the host)
        self.outputs = []  # tensors a graph replay must reproduce bit for bit


def count_inbounds(shapes, x, y):
    """Corners of bilinear samples that fall inside their level's map.  x, y:
    continuous pixel coordinates (W*s_x - 1/2, H*s_y - 1/2) of shape
    [..., L, P]; shapes [L, 2] as (H, W).  Measurement metadata only."""
    import numpy as np
    H = shapes[:, 0].astype(np.float64)[:, None]
    Wd = shapes[:, 1].astype(np.float64)[:, None]
    x0, y0 = np.floor(x), np.floor(y)
    n = 0
    for dx in (0, 1):
        inx = (x0 + dx >= 0) & (x0 + dx < Wd)
        for dy in (0, 1):
            n += int(np.count_nonzero(inx & (y0 + dy >= 0) & (y0 + dy < H)))
    return n


def sca_inbounds_corners(w, shapes, offsets):
    """In-map corners of one SCA gather launch: every seen (camera, query)
    pair's samples at anchor rho[p mod D] + offset / (W_l, H_l) on the
    level table `shapes` (measurement metadata only)."""
    import numpy as np
    B, Ncam, L, P, D = w["B"], w["Ncam"], w["L"], w["P"], w["D"]
    WH = np.stack([shapes[:, 1], shapes[:, 0]], -1).astype(np.float32)  # (W, H) per level
    anchor = np.arange(P) % D
    n_in = 0
    for b in range(B):
        for c in range(Ncam):
            qs = np.nonzero(w["bev_mask"][c, b].any(-1))[0]
            rho = w["reference_points_cam"][c, b, qs][:, anchor]  # [q, P, 2]
            for l in range(L):
                loc = rho[:, None, :, :] + offsets[b, qs][:, :, l] / WH[l]  # [q, nH, P, 2]
                x = loc[..., 0].astype(np.float64) * WH[l, 0] - 0.5
                y = loc[..., 1].astype(np.float64) * WH[l, 1] - 0.5
                n_in += count_inbounds(shapes[l:l + 1], x[..., None, :], y[..., None, :])
    return n_in


CEILING_SHRINK = 8  # level sides divided by this for the on-chip ceiling


def small_levels(shapes):
    """The level table with every side divided by CEILING_SHRINK (rounded
    up): every workload's value maps then fit in one die's L2 (the SCA
    workload's six cameras: 3.2 MB in float32)."""
    import numpy as np
    ss = np.maximum(1, -(-np.asarray(shapes, np.int64) // CEILING_SHRINK))
    starts = np.concatenate([[0], np.cumsum(ss[:, 0] * ss[:, 1])[:-1]]).astype(np.int64)
    return ss.astype(np.int64), starts, int((ss[:, 0] * ss[:, 1]).sum())


def _mean_launch_ms(fn, reps=20, warm=5):
    """Mean duration of fn's launches, from HIP events recorded around each
    on torch's current stream (the stream the binding launches on)."""
    import numpy as np
    import torch
    for _ in range(warm):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))


def _ceiling(inb_bytes, ms, shapes):
    return {"GBps": inb_bytes / (ms * 1e-3) / 1e9, "kernel_ms": ms, "inbounds_bytes_per_launch": inb_bytes,
            "levels": "/".join(f"{h}x{wd}" for h, wd in shapes.tolist()),
            "how": f"the same kernel on the same samples and work order, with every level side divided by "
                   f"{CEILING_SHRINK} (offsets in cells scaled with it, so each sample keeps its normalised "
                   f"location): every value map fits in L2, so nothing waits on memory beyond it"}


def sca_onchip_ceiling(w, d, ws, offsets, bf16, pairs=False):
    """The SCA gather kernel's rate of in-map corner bytes when every corner
    row it reads sits in L2: the measured ceiling of the vector-memory path
    for this kernel and sample mix (and value layout)."""
    import numpy as np
    import torch
    import scale_deformable_attention_forward_amd as m
    ss, starts, Nv = small_levels(w["spatial_shapes"])
    scale = np.stack([ss[:, 1] / w["spatial_shapes"][:, 1], ss[:, 0] / w["spatial_shapes"][:, 0]], -1)
    off = (offsets * scale[None, None, None, :, None, :]).astype(np.float32)
    g = torch.Generator(device="cuda").manual_seed(12345)
    value = torch.randn((w["B"], w["Ncam"], Nv, w["nH"], 32), generator=g, device="cuda")
    value = value.to(torch.bfloat16) if bf16 else value
    if pairs:
        value = m.msda_pack_pairs_bf16(value)
    dss, dst, doff = _dev(ss), _dev(starts), _dev(off)
    slots = torch.empty((w["B"], w["Nq"], w["nH"] * 32), dtype=torch.float32, device="cuda")
    ms = _mean_launch_ms(lambda: m.sca_gather(value, dss, dst, d["reference_points_cam"], doff,
                                              d["attention_logits"], ws, slots=slots))
    return _ceiling(sca_inbounds_corners(w, ss, off) * 32 * (2 if bf16 else 4), ms, ss)


def msda_onchip_ceiling(w, d, F, plan=None):
    """As sca_onchip_ceiling, for the operator (or frame mean): the same
    normalised locations on the shrunken level table."""
    import numpy as np
    import torch
    import scale_deformable_attention_forward_amd as m
    ss, starts, Nv = small_levels(w["spatial_shapes"])
    B, Nq, nH = w["B"], w["Nq"], w["nH"]
    g = torch.Generator(device="cuda").manual_seed(12345)
    value = torch.randn(((B, F) if F > 1 else (B,)) + (Nv, nH, 32), generator=g, device="cuda")
    dss, dst = _dev(ss), _dev(starts)
    out = torch.empty((B, Nq, nH * 32), dtype=torch.float32, device="cuda")
    if plan is not None:  # the same work order as the measured gather
        ms = _mean_launch_ms(lambda: m.msda_gather(value, dss, dst, d["sampling_locations"], d["attention_weights"],
                                                   plan, out=out))
    else:
        fn = m.msda_forward if F == 1 else m.msda_forward_frames
        ms = _mean_launch_ms(lambda: fn(value, dss, dst, d["sampling_locations"], d["attention_weights"], out=out))
    loc = w["sampling_locations"]
    inb = count_inbounds(ss, loc[..., 0] * ss[:, 1].astype(np.float64)[:, None] - 0.5,
                         loc[..., 1] * ss[:, 0].astype(np.float64)[:, None] - 0.5)
    return _ceiling(inb * 32 * 4, ms, ss)


def _dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def sca_workload(kind):
    import torch
    import workloads as W
    import scale_deformable_attention_forward_amd as m

    full = kind == "layer_full"
    layer = kind in ("layer_bf16", "layer_full", "layer_bf16_plain")
    # the layers write the value projection in the head-pair layout, which
    # the gather reads with one line per x-adjacent corner pair ("_plain":
    # the row-major bf16 layout, as A/B)
    pairs = kind in ("layer_bf16", "layer_full")
    # one frame of the encoder: one compaction (the masks and anchors do not
    # change between layers) and the gathers of 6 layers
    layers = 6 if kind == "sca_frame6" else 1
    bf16 = kind in ("sca_bf16", "layer_bf16", "layer_full", "layer_bf16_plain")
    if full:
        w = W.bevformer_layer_bf16()
    elif layer:
        w = W.bevformer_sca_bf16()
    else:
        w = W.bevformer_sca(value_bf16=bf16)
    B, Ncam, Nq, Nv, nH, L, P, D = w["B"], w["Ncam"], w["Nq"], w["Nv"], w["nH"], w["L"], w["P"], w["D"]
    C = nH * 32
    d = {k: _dev(w[k]) for k in ("spatial_shapes", "level_start_index", "reference_points_cam", "bev_mask")}
    if full:
        for k in ("query", "query_pos", "W_off", "b_off", "W_att", "b_att", "gamma", "beta"):
            d[k] = _dev(w[k])
        d["query"], d["query_pos"] = d["query"].view(-1, C), d["query_pos"].view(-1, C)
        d["sampling_offsets"] = torch.empty((B, Nq, nH, L, P, 2), dtype=torch.float32, device="cuda")
        d["attention_logits"] = torch.empty((B, Nq, nH, L * P), dtype=torch.float32, device="cuda")
    else:
        d["sampling_offsets"] = _dev(w["sampling_offsets"])
        d["attention_logits"] = _dev(w["attention_logits"])
    if layer:
        d["feat"] = _dev(w["feat"].reshape(-1, C))
        d["W_v"], d["b_v"], d["W_o"], d["b_o"] = (_dev(w[k]) for k in ("W_v", "b_v", "W_o", "b_o"))
        d["value"] = torch.empty((B, Ncam, nH, Nv, 2, 32) if pairs else (B, Ncam, Nv, nH, 32),
                                 dtype=torch.bfloat16, device="cuda")
        d["out"] = torch.empty((B * Nq, C), dtype=torch.float32, device="cuda")
    else:
        d["value"] = _dev(w["value"])
    ws = torch.empty(m.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device="cuda")
    slots = torch.empty((B, Nq, C), dtype=torch.float32, device="cuda")
    offs = torch.empty(B * Ncam + 1, dtype=torch.int32, device="cuda")
    pq = torch.empty(B * Ncam * Nq, dtype=torch.int32, device="cuda")
    hit = torch.empty((B, Nq), dtype=torch.int32, device="cuda")

    wl = Workload(kind)
    if full:
        wl.parts.append(("query_proj", lambda: m.msda_query_proj_bf16(
            d["query"], d["W_off"], d["b_off"], d["W_att"], d["b_att"], query_pos=d["query_pos"],
            offsets=d["sampling_offsets"].view(B * Nq, -1), logits=d["attention_logits"].view(B * Nq, -1))))
    if pairs:
        wl.parts.append(("value_proj", lambda: m.msda_value_proj_pairs_bf16(d["feat"], d["W_v"], d["b_v"], Nv,
                                                                            out=d["value"].view(-1, nH, Nv, 2, 32))))
    elif layer:
        wl.parts.append(("value_proj", lambda: m.msda_gemm_bf16(d["feat"], d["W_v"], d["b_v"],
                                                                out=d["value"].view(-1, C))))
    wl.parts.append(("compact", lambda: m.sca_compact(d["bev_mask"], d["reference_points_cam"], ws, hit_count=hit,
                                                      pair_offsets=offs, pair_q=pq)))
    wl.parts.append(("gather", lambda: m.sca_gather(d["value"], d["spatial_shapes"], d["level_start_index"],
                                                    d["reference_points_cam"], d["sampling_offsets"],
                                                    d["attention_logits"], ws, slots=slots)))
    # layers 2..6 of a frame: their own value maps, offsets and logits (the
    # first layer's, shifted and scaled on the device: synthetic, like it)
    for li in range(1, layers):
        v_l = torch.roll(d["value"], shifts=997 * li, dims=2).contiguous()
        o_l = (d["sampling_offsets"] * (1.0 - 0.1 * li)).contiguous()
        g_l = torch.roll(d["attention_logits"], shifts=li, dims=-1).contiguous()
        s_l = torch.empty_like(slots)
        wl.parts.append((f"gather_{li + 1}", lambda v_l=v_l, o_l=o_l, g_l=g_l, s_l=s_l: m.sca_gather(
            v_l, d["spatial_shapes"], d["level_start_index"], d["reference_points_cam"], o_l, g_l, ws, slots=s_l)))
    if full:
        wl.parts.append(("output_proj", lambda: m.msda_output_proj_bf16(
            slots.view(-1, C), d["W_o"], d["b_o"], residual=d["query"], gamma=d["gamma"], beta=d["beta"],
            out=d["out"])))
    elif layer:
        wl.parts.append(("output_proj", lambda: m.msda_gemm_bf16(slots.view(-1, C), d["W_o"], d["b_o"],
                                                                 out=d["out"])))
    wl.main = "gather"
    wl.outputs = [slots, hit, offs] + ([d["out"]] if layer else [])

    def finish():
        import numpy as np
        n_pairs = int(offs[-1].item())
        # corners inside their map: per visible pair, from the offsets the
        # gather reads (read back after the warm-up for the whole layer)
        off_h = d["sampling_offsets"].cpu().numpy() if full else w["sampling_offsets"]
        wl.inbounds_corners = sca_inbounds_corners(w, w["spatial_shapes"], off_h)
        elem = 2 if bf16 else 4
        wl.samples = n_pairs * nH * L * P * layers
        # effective bytes of one gather launch: 4 nominal corners x 32 channels
        # per sample, the per-query offsets and logits, the anchors of each
        # pair, the camera masks and work list, and the output rows
        wl.gathered_bytes = n_pairs * nH * L * P * 4 * 32 * elem  # one launch (the first layer's)
        wl.eff_bytes = (wl.gathered_bytes + B * Nq * nH * L * P * (8 + 4) + n_pairs * D * 8 + B * Nq * (4 + 4)
                        + B * Nq * C * 4)
        # what one gather launch must move at least once: every value map,
        # the per-query offsets and logits, the seen pairs' anchors, the
        # camera masks and work list, and the output rows
        # (the head-pair layout holds every pixel twice)
        wl.unique_bytes = (B * Ncam * Nv * C * elem * (2 if pairs else 1) + B * Nq * nH * L * P * (8 + 4)
                           + n_pairs * D * 8 + B * Nq * (4 + 4) + B * Nq * C * 4)
        wl.onchip = lambda: sca_onchip_ceiling(w, d, ws, off_h, bf16, pairs)
        if layer:
            Mv, Mo = B * Ncam * Nv, B * Nq
            wl.extra["value_proj"] = {"flop": 2 * Mv * C * C,
                                      "bytes": Mv * C * 2 * (3 if pairs else 2) + C * C * 2}
            wl.extra["output_proj"] = {"flop": 2 * Mo * C * C, "bytes": Mo * C * 4 * 2 + C * C * 2}
        if full:
            Mq, Nqp = B * Nq, nH * L * P * 3
            # query and position embedding in, offsets and logits out; the
            # output side adds the residual read
            wl.extra["query_proj"] = {"flop": 2 * Mq * Nqp * C, "bytes": Mq * C * 4 * 2 + Mq * Nqp * 4 + Nqp * C * 2}
            wl.extra["output_proj"]["bytes"] += Mo * C * 4
    wl.finish = finish
    wl.batch = B
    wl.config = {"workload": "BEVFormer-base spatial cross-attention layer, 6 cameras"
                 + (", whole layer: bf16 query, value and output projections, residual and layer norm" if full
                    else ", with bf16 value and output projections" if layer
                    else "; one frame: one compaction serving 6 encoder layers, each with its own value maps, "
                         "offsets and logits" if layers > 1 else ""),
                 "batch": B, "cameras": Ncam, "bev_queries": "200x200", "levels": "116x200/58x100/29x50/15x25",
                 "heads": nH, "head_dim": 32, "points_per_level": P, "pillar_anchors": D,
                 "value_dtype": "bf16" if bf16 else "fp32", "mask": "azimuth sectors, 1-2 cameras per query"}
    if bf16:
        wl.config["value_layout"] = ("head pairs [B][Ncam][nH][Nv][2][32], written by the value projection" if pairs
                                     else "[B][Ncam][Nv][nH][32]")
    wl.dtype = "fp32 accumulate, bf16 value" if bf16 else "fp32"
    wl.kernel_key = "sca_gather_kernel_bf16" if bf16 else "sca_gather_kernel_fp32"

    wl.cpu_baseline = lambda: sca_cpu_baseline(w, "layer_full" if full else "layer_bf16" if layer else kind)
    return wl


def rebatch_workload():
    """The BEVFormer-base SCA workload through the padded rebatch flow (A/B
    baseline): compaction, the longest segment read back to the host,
    rebatch, the MSDA operator over B*Ncam padded segments, scatter-add per
    camera and divide."""
    import numpy as np
    import torch
    import workloads as W
    import scale_deformable_attention_forward_amd as m

    w = W.bevformer_sca()
    B, Ncam, Nq, Nv, nH, L, P, D = w["B"], w["Ncam"], w["Nq"], w["Nv"], w["nH"], w["L"], w["P"], w["D"]
    C = nH * 32
    d = {k: _dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "reference_points_cam", "bev_mask",
                                 "sampling_offsets", "attention_logits")}
    ws = torch.empty(m.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device="cuda")
    hit = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
    offs = torch.empty(B * Ncam + 1, dtype=torch.int32, device="cuda")
    pq = torch.empty(B * Ncam * Nq, dtype=torch.int32, device="cuda")
    S = nH * L * P
    # padded buffers sized for the largest possible segment; each step uses
    # the leading [B*Ncam, max_len] part
    loc_buf = torch.empty(B * Ncam * Nq * S * 2, dtype=torch.float32, device="cuda")
    lg_buf = torch.empty(B * Ncam * Nq * S, dtype=torch.float32, device="cuda")
    rows_buf = torch.empty(B * Ncam * Nq * C, dtype=torch.float32, device="cuda")
    slots = torch.empty((B, Nq, C), dtype=torch.float32, device="cuda")
    st = {}

    def read_max_len():
        o = offs.cpu().numpy()
        st["ml"] = int((o[1:] - o[:-1]).max())

    def views():
        ml = st["ml"]
        n = B * Ncam * ml
        return (loc_buf[:n * S * 2].view(B * Ncam, ml, nH, L, P, 2), lg_buf[:n * S].view(B * Ncam, ml, nH, L * P),
                rows_buf[:n * C].view(B * Ncam, ml, C))

    wl = Workload("sca_rebatch")
    wl.parts.append(("compact", lambda: m.sca_compact(d["bev_mask"], d["reference_points_cam"], ws, hit_count=hit,
                                                      pair_offsets=offs, pair_q=pq)))
    wl.parts.append(("max_len", read_max_len))
    wl.parts.append(("rebatch", lambda: m.sca_rebatch(offs, pq, d["reference_points_cam"], d["sampling_offsets"],
                                                      d["attention_logits"], d["spatial_shapes"], st["ml"],
                                                      *views()[:2])))
    wl.parts.append(("msda", lambda: m.msda_forward(d["value"].view(B * Ncam, Nv, nH, 32), d["spatial_shapes"],
                                                    d["level_start_index"], views()[0], views()[1],
                                                    out=views()[2])))
    wl.parts.append(("scatter_mean", lambda: m.sca_scatter_mean(views()[2], offs, pq, hit, Nq, slots=slots)))
    wl.main = "msda"
    wl.graph = False  # the segment length is read back to the host

    def finish():
        n_pairs = int(offs[-1].item())
        wl.samples = n_pairs * S
        padded = B * Ncam * st["ml"] * S
        wl.gathered_bytes = padded * 4 * 32 * 4
        wl.eff_bytes = wl.gathered_bytes + padded * 12 + B * Ncam * st["ml"] * C * 4
        wl.unique_bytes = B * Ncam * Nv * C * 4 + padded * 12 + B * Ncam * st["ml"] * C * 4
        wl.extra_info = {"max_len": st["ml"], "padded_rows": B * Ncam * st["ml"], "pairs": n_pairs,
                         "padded_samples": padded}
    wl.finish = finish
    wl.batch = B
    wl.config = {"workload": "BEVFormer-base spatial cross-attention layer, 6 cameras, padded rebatch flow "
                             "(A/B baseline for the fused path)",
                 "batch": B, "cameras": Ncam, "bev_queries": "200x200", "levels": "116x200/58x100/29x50/15x25",
                 "heads": nH, "head_dim": 32, "points_per_level": P, "pillar_anchors": D, "value_dtype": "fp32",
                 "mask": "azimuth sectors, 1-2 cameras per query"}
    wl.dtype = "fp32"
    wl.kernel_key = "msda_gather_kernel_fp32"

    wl.cpu_baseline = lambda: sca_cpu_baseline(w, "sca")
    return wl


def train_workload(which):
    """Forward and backward of one step: "sca_train" (the BEVFormer-base SCA
    workload: compaction, SCA forward, SCA backward), "detr_train" (the
    DETR-encoder workload: MSDA forward and backward) or "tsa_train" (the
    temporal workload: the frame mean's forward and backward).  The upstream gradient
    is seeded N(0, 1).  The gradient workspace is made once, for every camera
    seeing every query (no read-back of the pair count)."""
    import torch
    import workloads as W
    import scale_deformable_attention_forward_amd as m

    wl = Workload(which)
    atomic = which.endswith("_atomic")
    which = which.replace("_atomic", "")
    if which == "sca_train":
        w = W.bevformer_sca()
        B, Ncam, Nq, Nv, nH, L, P, D = w["B"], w["Ncam"], w["Nq"], w["Nv"], w["nH"], w["L"], w["P"], w["D"]
        d = {k: _dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "reference_points_cam",
                                     "bev_mask", "sampling_offsets", "attention_logits")}
        grad = W.upstream_gradient(3, (B, Nq, nH * 32))
        gout = _dev(grad)
        ws = torch.empty(m.sca_workspace_size(B, Ncam, Nq), dtype=torch.uint8, device="cuda")
        slots = torch.empty((B, Nq, nH * 32), dtype=torch.float32, device="cuda")
        offs = torch.empty(B * Ncam + 1, dtype=torch.int32, device="cuda")
        gv = torch.empty((B, Ncam, Nv, nH, 32), dtype=torch.float32, device="cuda")
        go = torch.empty_like(d["sampling_offsets"])
        gl = torch.empty_like(d["attention_logits"])
        gws = None if atomic else torch.empty(m.sca_backward_workspace_size(B, Ncam, Nv, Nq, nH, L, P),
                                              dtype=torch.uint8, device="cuda")
        args = (d["spatial_shapes"], d["level_start_index"], d["reference_points_cam"])
        wl.parts.append(("compact", lambda: m.sca_compact(d["bev_mask"], d["reference_points_cam"], ws,
                                                          pair_offsets=offs)))
        wl.parts.append(("forward", lambda: m.sca_gather(d["value"], *args, d["sampling_offsets"],
                                                         d["attention_logits"], ws, slots=slots)))
        wl.parts.append(("backward", lambda: m.sca_backward(d["value"], *args, d["sampling_offsets"],
                                                            d["attention_logits"], gout, ws, grad_value=gv,
                                                            grad_offsets=go, grad_logits=gl, grad_workspace=gws,
                                                            atomic=atomic)))
        names = "BEVFormer-base spatial cross-attention layer, 6 cameras, forward + backward"
        names += " (value gradient by float32 atomics)" if atomic else ""
        pairs = lambda: int(offs[-1].item())
        n_images = B * Ncam
        outs = [slots, gv, go, gl]
    elif which == "tsa_train":
        w = W.temporal_frames()
        B, F, Nq, Nv, nH, L, P = w["B"], w["F"], w["Nq"], w["Nv"], w["nH"], w["L"], w["P"]
        d = {k: _dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations",
                                     "attention_weights")}
        grad = W.upstream_gradient(4, (B, Nq, nH * 32))
        gout = _dev(grad)
        out = torch.empty((B, Nq, nH * 32), dtype=torch.float32, device="cuda")
        gv = torch.empty((B, F, Nv, nH, 32), dtype=torch.float32, device="cuda")
        gloc = torch.empty_like(d["sampling_locations"])
        gw = torch.empty_like(d["attention_weights"])
        gws = None if atomic else torch.empty(m.msda_backward_workspace_size(B * F, Nv, Nq, nH, L, P),
                                              dtype=torch.uint8, device="cuda")
        fargs = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"],
                 d["attention_weights"])
        wl.parts.append(("forward", lambda: m.msda_forward_frames(*fargs, out=out)))
        wl.parts.append(("backward", lambda: m.msda_backward_frames(*fargs, gout, grad_value=gv, grad_locations=gloc,
                                                                    grad_weights=gw, grad_workspace=gws,
                                                                    atomic=atomic)))
        names = ("temporal self-attention, 2 stacked 200x200 BEV maps, mean over frames, forward + backward"
                 + (" (value gradient by float32 atomics)" if atomic else ""))
        pairs = lambda: B * F * Nq
        n_images = B * F
        outs = [out, gv, gloc, gw]
    else:
        w = W.detr_encoder_msda()
        B, Nq, Nv, nH, L, P = w["B"], w["Nq"], w["Nv"], w["nH"], w["L"], w["P"]
        d = {k: _dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations",
                                     "attention_weights")}
        grad = W.upstream_gradient(2, (B, Nq, nH * 32))
        gout = _dev(grad)
        out = torch.empty((B, Nq, nH * 32), dtype=torch.float32, device="cuda")
        gv = torch.empty((B, Nv, nH, 32), dtype=torch.float32, device="cuda")
        gloc = torch.empty_like(d["sampling_locations"])
        gw = torch.empty_like(d["attention_weights"])
        gws = None if atomic else torch.empty(m.msda_backward_workspace_size(B, Nv, Nq, nH, L, P),
                                              dtype=torch.uint8, device="cuda")
        fargs = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"],
                 d["attention_weights"])
        wl.parts.append(("forward", lambda: m.msda_forward(*fargs, out=out)))
        wl.parts.append(("backward", lambda: m.msda_backward(*fargs, gout, grad_value=gv, grad_locations=gloc,
                                                             grad_weights=gw, grad_workspace=gws, atomic=atomic)))
        names = "Deformable-DETR encoder MSDA, 4 levels 100x150/50x75/25x38/13x19, Nq=Nv=19947, forward + backward"
        names += " (value gradient by float32 atomics)" if atomic else ""
        pairs = lambda: B * Nq
        n_images = B
        outs = [out, gv, gloc, gw]
    wl.main = "backward"
    # float32 atomics sum in no fixed order: only the forward output repeats bit for bit
    wl.outputs = outs[:1] if atomic else outs

    def finish():
        n = pairs()
        wl.samples = n * nH * L * P
        # backward: the corner rows read (as the forward) and, per corner, one
        # upstream-gradient row read into the value gradient (or, with atomics,
        # one value-gradient row added to), the per-query inputs and upstream
        # gradient read, the offset / location and weight gradients written,
        # and the value gradient written once (or zeroed first)
        S = wl.samples
        wl.gathered_bytes = S * 4 * 32 * 4
        rows = B * Nq * (F if which == "tsa_train" else 1)  # rows of locations / offsets and weights
        wl.eff_bytes = (2 * wl.gathered_bytes + rows * nH * L * P * (8 + 4) * 2 + B * Nq * nH * 32 * 4
                        + n_images * Nv * nH * 32 * 4)
        # the backward must read the value maps, the per-query inputs and the
        # upstream gradient once and write the three gradients once
        wl.unique_bytes = (n_images * Nv * nH * 32 * 4 * 2 + rows * nH * L * P * (8 + 4) * 2
                           + B * Nq * nH * 32 * 4)
    wl.finish = finish
    wl.batch = B
    wl.config = {"workload": names, "batch": B, "queries": Nq, "heads": nH, "head_dim": 32, "levels": L,
                 "points_per_level": P, "value_dtype": "fp32", "pass": "forward + backward",
                 "value_gradient": "float32 atomics" if atomic else "transpose gather (deterministic)"}
    if which == "tsa_train":
        wl.config["frames"] = F
    wl.dtype = "fp32"
    wl.kernel_key = ("sca_backward_kernel" if which == "sca_train" else "msda_backward_kernel") + "_fp32"

    wl.cpu_baseline = lambda: train_cpu_baseline(w, which, grad)
    return wl


def msda_workload(which):
    import numpy as np
    import torch
    import workloads as W
    import scale_deformable_attention_forward_amd as m

    # the DETR encoder's queries are placed at random: its default runs the
    # plan (inside every step); the temporal workload's BEV-grid queries
    # come in raster order and run as given (its plan: "tsa_planned" in every
    # step, "tsa_gridplan" once, from the grid cells' centres, before the
    # timed steps: the grid, and so the plan, never changes)
    # "detr_encoder6": one pass of the six-layer encoder, its plan built once
    # from the reference points (which every layer shares) before the timed
    # steps, then the six layers' planned gathers
    planned = which in ("detr", "tsa_planned", "tsa_gridplan", "detr_encoder6")
    layers = 6 if which == "detr_encoder6" else 1
    base = which.replace("_unplanned", "").replace("_planned", "").replace("_gridplan", "").replace("_encoder6", "")
    if base == "detr":
        w, F = W.detr_encoder_msda(), 1
    elif base == "tiny":
        w, F = W.tiny_msda(), 1
    else:
        w = W.temporal_frames()
        F = w["F"]
    d = {k: _dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations",
                                 "attention_weights")}
    B, Nq, nH, L, P = w["B"], w["Nq"], w["nH"], w["L"], w["P"]
    out = torch.empty((B, Nq, nH * 32), dtype=torch.float32, device="cuda")
    wl = Workload(which)
    args = (d["value"], d["spatial_shapes"], d["level_start_index"], d["sampling_locations"], d["attention_weights"])
    if planned:
        # the locality plan, from each query's first sampling location, is
        # part of every step
        row = nH * L * P * 2
        plan = torch.empty(m.msda_plan_size(B, Nq), dtype=torch.uint8, device="cuda")
        if which == "tsa_gridplan":
            side = int(round(Nq ** 0.5))
            c = (np.arange(side, dtype=np.float32) + 0.5) / side
            cx, cy = np.meshgrid(c, c)  # q = row * side + col
            cells = torch.from_numpy(np.stack([cx.ravel(), cy.ravel()], -1)).cuda().expand(B, Nq, 2).contiguous()
            m.msda_plan(cells, B, Nq, Nq * 2, 2, plan=plan)
        elif which == "detr_encoder6":
            m.msda_plan(_dev(w["reference_points"]), B, Nq, Nq * 2, 2, plan=plan)
        else:
            wl.parts.append(("plan", lambda: m.msda_plan(d["sampling_locations"], B, Nq, F * Nq * row, row,
                                                         plan=plan)))
        wl.parts.append(("gather", lambda: m.msda_gather(*args, plan, out=out)))
    else:
        fn = m.msda_forward if F == 1 else m.msda_forward_frames
        wl.parts.append(("gather", lambda: fn(*args, out=out)))
    # layers 2..6: their own value maps, locations (the same reference
    # points, the offsets scaled) and weights, derived from the first
    # layer's on the device: synthetic, like it
    ref = _dev(w["reference_points"])[:, :, None, None, None, :] if layers > 1 else None
    for li in range(1, layers):
        v_l = torch.roll(d["value"], shifts=997 * li, dims=1).contiguous()
        s_l = (ref + (d["sampling_locations"] - ref) * (1.0 - 0.1 * li)).contiguous()
        a_l = torch.roll(d["attention_weights"], shifts=li, dims=-1).contiguous()
        o_l = torch.empty_like(out)
        wl.parts.append((f"gather_{li + 1}", lambda v_l=v_l, s_l=s_l, a_l=a_l, o_l=o_l: m.msda_gather(
            v_l, d["spatial_shapes"], d["level_start_index"], s_l, a_l, plan, out=o_l)))
    wl.main = "gather"
    wl.outputs = [out]

    def finish():
        wl.samples = B * F * Nq * nH * L * P * layers
        ss = w["spatial_shapes"]
        loc = w["sampling_locations"]
        Wd = ss[:, 1].astype(np.float64)[:, None]
        H = ss[:, 0].astype(np.float64)[:, None]
        wl.inbounds_corners = count_inbounds(ss, loc[..., 0] * Wd - 0.5, loc[..., 1] * H - 0.5)
        launch = wl.samples // layers  # one gather launch (the first layer's)
        wl.gathered_bytes = launch * 4 * 32 * 4
        wl.eff_bytes = wl.gathered_bytes + launch * (8 + 4) + B * Nq * nH * 32 * 4
        wl.unique_bytes = w["value"].nbytes + launch * (8 + 4) + B * Nq * nH * 32 * 4
        if base != "tiny":  # the tiny parity workload is launch-bound: no on-chip ceiling to speak of
            wl.onchip = lambda: msda_onchip_ceiling(w, d, F, plan if planned else None)
    wl.finish = finish
    wl.batch = B
    names = {"detr": "Deformable-DETR encoder MSDA, 4 levels 100x150/50x75/25x38/13x19, Nq=Nv=19947",
             "tiny": "tiny MSDA, 256 queries, one 32x32 level",
             "tsa": "temporal self-attention, 2 stacked 200x200 BEV maps, mean over frames"}
    order = {"tsa_gridplan": ", planned gather (locality plan built once from the BEV grid, outside the step)",
             "detr_encoder6": ", one encoder pass: a locality plan built once from the reference points (outside "
                              "the step), then 6 layers' planned gathers, each with its own value map, locations "
                              "and weights"}
    wl.config = {"workload": names[base] + order.get(which, ", locality plan + planned gather" if planned
                                                     else ", queries in input order (no plan)"),
                 "batch": B, "queries": Nq, "heads": nH, "head_dim": 32,
                 "levels": L, "points_per_level": P, "frames": F, "value_dtype": "fp32"}
    wl.dtype = "fp32"
    wl.kernel_key = "msda_gather_kernel_fp32"

    wl.cpu_baseline = lambda: msda_cpu_baseline(w, first_of=layers)
    return wl


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sca",
                    choices=["sca", "layer_bf16", "layer_full", "layer_bf16_plain", "sca_bf16", "sca_rebatch",
                             "sca_train", "detr",
                             "detr_train", "sca_train_atomic", "detr_train_atomic", "tsa", "tiny", "sca_frame6",
                             "tsa_train", "tsa_train_atomic", "detr_unplanned", "tsa_planned", "tsa_gridplan",
                             "detr_encoder6"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-onchip-ceiling", action="store_true",
                    help="skip the L2-resident run of the main kernel behind roofline_onchip")
    ap.add_argument("--cold-reps", type=int, default=5,
                    help="steps timed after a 1 GiB write that evicts the caches (0: none)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the eager steps only (by default the step is also captured in a HIP graph and "
                         "the replays are timed)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy()
        return
    import scale_deformable_attention_forward_amd as m
    m.load_library()

    if args.workload in ("sca", "layer_bf16", "layer_full", "layer_bf16_plain", "sca_bf16", "sca_frame6"):
        wl = sca_workload(args.workload)
    elif args.workload == "sca_rebatch":
        wl = rebatch_workload()
    elif args.workload in ("sca_train", "detr_train", "sca_train_atomic", "detr_train_atomic", "tsa_train",
                           "tsa_train_atomic"):
        wl = train_workload(args.workload)
    else:
        wl = msda_workload(args.workload)

    for _ in range(args.warmup):
        for _, fn in wl.parts:
            fn()
    torch.cuda.synchronize()
    wl.finish()

    # events recorded on torch's current stream, which is the stream the
    # binding hands to the library, between every part of every step
    K = args.steps
    n = len(wl.parts)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record()
        for i, (_, fn) in enumerate(wl.parts):
            fn()
            ev[k][i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    import numpy as np
    per_step = {name: np.array([ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(K)])
                for i, (name, _) in enumerate(wl.parts)}
    step_ms = np.array([ev[k][0].elapsed_time(ev[k][n]) for k in range(K)])
    part_ms = {name: float(v.mean()) for name, v in per_step.items()}
    kernel_ms = part_ms[wl.main]

    def pct(v):
        return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
                "p90": float(np.percentile(v, 90))}

    # a step of several library calls captured once in a HIP graph and
    # replayed K times: one launch per step instead of one call (and its
    # host-side argument checks) per part; the replays must reproduce the
    # eager outputs bit for bit.  A one-call step gains nothing from it (the
    # temporal workload measured 0.0838 ms per replay against 0.0811 ms
    # eagerly) and runs eagerly.
    eager = {"ms_per_step": ms_per_step, "step_ms_events": pct(step_ms)}
    graph_info = None
    if wl.graph and len(wl.parts) > 1 and not args.eager:
        ref = [t.clone() for t in wl.outputs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _, fn in wl.parts:
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _, fn in wl.parts:
                fn()
        def check(when):
            for i, (a, b) in enumerate(zip(ref, wl.outputs)):
                if not torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)):
                    raise RuntimeError(f"graph replay: output {i} differs from the eager step ({when})")

        # the outputs overwritten first, so that the replays must write them
        for t in wl.outputs:
            t.fill_(float("nan") if t.is_floating_point() else -7)
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()
        check("warm-up replays")
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gev[0].record()
        for k in range(K):
            graph.replay()
            gev[k + 1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        check("timed replays")
        del graph
        ms_per_step = (t1 - t0) * 1e3 / K
        step_ms = np.array([gev[k].elapsed_time(gev[k + 1]) for k in range(K)])
        graph_info = {"replays": K, "outputs_checked": len(ref)}

    # cold: a 1 GiB write before each step evicts the inputs from L2 and
    # the memory-side cache, so the step starts from HBM
    cold = None
    if args.cold_reps > 0:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(args.cold_reps)]
        for r in range(args.cold_reps):
            scratch.fill_(float(r))
            cev[r][0].record()
            for i, (_, fn) in enumerate(wl.parts):
                fn()
                cev[r][i + 1].record()
        torch.cuda.synchronize()
        del scratch
        cold = {"reps": args.cold_reps,
                "step_ms": pct(np.array([cev[r][0].elapsed_time(cev[r][n]) for r in range(args.cold_reps)]))}
        for i, (name, _) in enumerate(wl.parts):
            cold[name + "_ms"] = pct(np.array([cev[r][i].elapsed_time(cev[r][i + 1]) for r in range(args.cold_reps)]))

    breakdown = {}
    for name, ms in part_ms.items():
        e = {"ms": ms, **pct(per_step[name])}
        if name in wl.extra:
            e["TFLOP/s"] = wl.extra[name]["flop"] / (ms * 1e-3) / 1e12
            e["GB/s"] = wl.extra[name]["bytes"] / (ms * 1e-3) / 1e9
            e["mfma_frac"] = e["TFLOP/s"] / BF16_MFMA_PEAK_TFS
            e["hbm_frac"] = e["GB/s"] / HBM_PEAK_GBS
        breakdown[name] = e
    kernel_s = kernel_ms * 1e-3
    achieved = wl.unique_bytes / kernel_s / 1e9
    line = {
        "metric": METRIC,
        "value": wl.samples / (ms_per_step * 1e-3),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded, BEVFormer-shaped; no dataset or trained weights)",
        "config": wl.config,
        # HBM roofline on the bytes the launch must move at least once
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(wl.name, wl.kernel_key.rsplit("_", 1)[0]),
                     "kernel": wl.kernel_key.rsplit("_", 1)[0], "kernel_ms": kernel_ms,
                     "bytes_per_launch": wl.unique_bytes},
        # effective bytes: all 4 nominal corners x 32 channels of every sample
        # plus metadata and output, mostly served from L1 and L2: a rate, not
        # a fraction of any memory's peak
        "effective": {"bytes_per_launch": wl.eff_bytes, "gathered_bytes_per_launch": wl.gathered_bytes,
                      "GBps": wl.eff_bytes / kernel_s / 1e9,
                      "GBps_per_step": wl.eff_bytes / (ms_per_step * 1e-3) / 1e9,
                      "times_hbm_peak": wl.eff_bytes / kernel_s / 1e9 / HBM_PEAK_GBS},
        "samples_per_step": wl.samples,
        "batch_items_per_s": wl.batch / (ms_per_step * 1e-3),
        "step_ms_events": pct(step_ms),
        # how the timed steps were launched; the breakdown and the kernel
        # figures always come from the eager steps' events
        "launch": ({"mode": "hip graph, one replay per step", **graph_info, "eager": eager} if graph_info
                   else {"mode": "eager, one library call per part"}),
        "breakdown": breakdown,
        "cold": cold,
    }
    if getattr(wl, "extra_info", None):
        line["config"].update(wl.extra_info)
    if wl.inbounds_corners is not None:
        elem = 2 if "bf16" in wl.dtype else 4
        inb = wl.inbounds_corners * 32 * elem
        line["effective"]["gathered_bytes_in_bounds_per_launch"] = inb
        if wl.onchip is not None and not args.no_onchip_ceiling:
            # the corner rows the kernel reads, against the same kernel's
            # rate when every one of them sits in L2
            c = wl.onchip()
            got = inb / kernel_s / 1e9
            line["roofline_onchip"] = {"bound": "vector memory path (L1 / texture units)", "achieved": got,
                                       "peak": c["GBps"], "unit": "GB/s", "frac": got / c["GBps"],
                                       "kernel": line["roofline"]["kernel"], "bytes_per_launch": inb,
                                       "ceiling": c}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = {**wl.cpu_baseline(), **host_cpu()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
