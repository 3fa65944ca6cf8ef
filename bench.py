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
projection GEMM -> SCA on bf16 value -> bf16 output projection GEMM),
"layer_full" (the same with the sampling offsets and logits projected from
query + position embedding in one launch, and the output projection
followed by the residual and the layer norm), "sca_bf16", "sca_rebatch"
(the default workload through the padded rebatch flow of the SCA note, an
A/B baseline: per-camera segments padded to the longest, the operator over
all of them, scatter-add and divide), "sca_train", "detr_train" and
"tsa_train" (forward and backward of the default SCA layer, of the DETR
encoder MSDA and of the two-frame mean, the value gradient by the
deterministic transpose gather; "_atomic" variants accumulate it with
float32 atomics instead; the roofline then describes the backward kernel),
"detr" (Deformable-DETR encoder MSDA), "tsa" (two stacked BEV maps, frame
mean), "sca_frame6" (one frame of the encoder: one compaction serving six
SCA layers, each with its own value maps, offsets and logits), "tiny".

Prints one JSON line.  value = bilinear samples per second (one sample = one
(camera, query, head, level, point) bilinear read of 4 corners x 32
channels) over the whole step; roofline = the gather kernel's effective
bytes (all 4 nominal corners of every sample, plus offsets, logits, anchors,
work list and output) per launch over its average launch time, measured with
HIP events recorded on the stream the kernel runs on; breakdown = the same
events around every part of the step (mean, p10/p50/p90); cold = the same
step after a 1 GiB write that evicts L2 and the memory-side cache (the
headline is warm, back to back, as a layer runs inside a network);
batch_items_per_s = batch items (scenes) per second; roofline also carries
the bytes of the corners that fall inside their map, which are the only ones
the kernel actually reads; cpu_baseline = the CPU oracle on the same
workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
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
    layer = kind in ("layer_bf16", "layer_full")
    # one frame of the encoder: one compaction (the masks and anchors do not
    # change between layers) and the gathers of 6 layers
    layers = 6 if kind == "sca_frame6" else 1
    bf16 = kind in ("sca_bf16", "layer_bf16", "layer_full")
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
        d["value"] = torch.empty((B, Ncam, Nv, nH, 32), dtype=torch.bfloat16, device="cuda")
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
    if layer:
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

    def finish():
        import numpy as np
        n_pairs = int(offs[-1].item())
        # corners inside their map: per visible pair, from the offsets the
        # gather reads (read back after the warm-up for the whole layer)
        off_h = d["sampling_offsets"].cpu().numpy() if full else w["sampling_offsets"]
        ss = w["spatial_shapes"]
        WH = np.stack([ss[:, 1], ss[:, 0]], -1).astype(np.float32)  # (W, H) per level
        anchor = np.arange(P) % D
        n_in = 0
        for b in range(B):
            for c in range(Ncam):
                qs = np.nonzero(w["bev_mask"][c, b].any(-1))[0]
                rho = w["reference_points_cam"][c, b, qs][:, anchor]  # [q, P, 2]
                for l in range(L):
                    loc = rho[:, None, :, :] + off_h[b, qs][:, :, l] / WH[l]  # [q, nH, P, 2]
                    x = loc[..., 0].astype(np.float64) * WH[l, 0] - 0.5
                    y = loc[..., 1].astype(np.float64) * WH[l, 1] - 0.5
                    n_in += count_inbounds(ss[l:l + 1], x[..., None, :], y[..., None, :])
        wl.inbounds_corners = n_in
        elem = 2 if bf16 else 4
        wl.samples = n_pairs * nH * L * P * layers
        # effective bytes of one gather launch: 4 nominal corners x 32 channels
        # per sample, the per-query offsets and logits, the anchors of each
        # pair, the camera masks and work list, and the output rows
        wl.gathered_bytes = n_pairs * nH * L * P * 4 * 32 * elem  # one launch (the first layer's)
        wl.eff_bytes = (wl.gathered_bytes + B * Nq * nH * L * P * (8 + 4) + n_pairs * D * 8 + B * Nq * (4 + 4)
                        + B * Nq * C * 4)
        if layer:
            Mv, Mo = B * Ncam * Nv, B * Nq
            wl.extra["value_proj"] = {"flop": 2 * Mv * C * C, "bytes": Mv * C * 2 * 2 + C * C * 2}
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
    wl.dtype = "fp32 accumulate, bf16 value" if bf16 else "fp32"
    wl.kernel_key = "sca_gather_kernel_bf16" if bf16 else "sca_gather_kernel_fp32"

    def cpu_baseline():
        import oracle
        if layer:
            # bounded sample: the value projection of every row (float64
            # matmul), then (query projections,) SCA and output projection of
            # 4000 sampled queries
            import numpy as np
            rows = W.sample_rows(7, B * Nq, 4000)
            t0 = time.perf_counter()
            if full:
                q, e = w["query"].reshape(-1, C), w["query_pos"].reshape(-1, C)
                o_off, o_lg = oracle.query_proj(q[rows], e[rows], w["W_off"], w["b_off"], w["W_att"], w["b_att"])
                off = np.zeros((B * Nq, o_off.shape[1]), np.float32)
                lg = np.zeros((B * Nq, o_lg.shape[1]), np.float32)
                off[rows], lg[rows] = o_off, o_lg
                off, lg = off.reshape(B, Nq, nH, L, P, 2), lg.reshape(B, Nq, nH, L * P)
            else:
                off, lg = w["sampling_offsets"], w["attention_logits"]
            v = oracle.round_to_bf16(oracle.linear_bf16_blas(w["feat"].reshape(-1, C), w["W_v"], w["b_v"]))
            r = oracle.sca(v.reshape(B, Ncam, Nv, nH, 32), w["spatial_shapes"], w["level_start_index"],
                           w["reference_points_cam"], w["bev_mask"], off, lg, rows=rows)
            if full:
                oracle.output_proj(r["slots"].astype(np.float32), w["W_o"], w["b_o"], q[rows], w["gamma"],
                                   w["beta"])
            else:
                oracle.linear_bf16(oracle.round_to_bf16(r["slots"]), w["W_o"], w["b_o"])
            t = time.perf_counter() - t0
            n = int(r["hit_count"].reshape(-1)[rows].sum()) * nH * L * P
            return {"value": n / t, "unit": "samples/s", "cores": 1, "kind": "oracle",
                    "sample": f"value projection of all rows, then {'query projections, ' if full else ''}SCA and "
                              f"output projection of 4000 sampled queries ({n} samples); C loops and a float64 "
                              f"matmul, {t:.1f} s"}
        t0 = time.perf_counter()
        oracle.sca(w["value"], w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"],
                   w["bev_mask"], w["sampling_offsets"], w["attention_logits"])
        t = time.perf_counter() - t0
        n = wl.samples // layers
        return {"value": n / t, "unit": "samples/s", "cores": 1, "kind": "oracle",
                "sample": f"the whole workload (all {B * Nq} queries, {n} samples{', the first layer' if layers > 1 else ''}), "
                          f"single-threaded C, {t:.1f} s"}
    wl.cpu_baseline = cpu_baseline
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

    def finish():
        n_pairs = int(offs[-1].item())
        wl.samples = n_pairs * S
        padded = B * Ncam * st["ml"] * S
        wl.gathered_bytes = padded * 4 * 32 * 4
        wl.eff_bytes = wl.gathered_bytes + padded * 12 + B * Ncam * st["ml"] * C * 4
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

    def cpu_baseline():
        import oracle
        t0 = time.perf_counter()
        oracle.sca(w["value"], w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"],
                   w["bev_mask"], w["sampling_offsets"], w["attention_logits"])
        t = time.perf_counter() - t0
        n = wl.samples // layers
        return {"value": n / t, "unit": "samples/s", "cores": 1, "kind": "oracle",
                "sample": f"the whole workload (all {B * Nq} queries, {n} samples{', the first layer' if layers > 1 else ''}), "
                          f"single-threaded C, {t:.1f} s"}
    wl.cpu_baseline = cpu_baseline
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
        gout = _dev(W.upstream_gradient(3, (B, Nq, nH * 32)))
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
    elif which == "tsa_train":
        w = W.temporal_frames()
        B, F, Nq, Nv, nH, L, P = w["B"], w["F"], w["Nq"], w["Nv"], w["nH"], w["L"], w["P"]
        d = {k: _dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations",
                                     "attention_weights")}
        gout = _dev(W.upstream_gradient(4, (B, Nq, nH * 32)))
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
    else:
        w = W.detr_encoder_msda()
        B, Nq, Nv, nH, L, P = w["B"], w["Nq"], w["Nv"], w["nH"], w["L"], w["P"]
        d = {k: _dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations",
                                     "attention_weights")}
        gout = _dev(W.upstream_gradient(2, (B, Nq, nH * 32)))
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
    wl.main = "backward"

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
    wl.finish = finish
    wl.batch = B
    wl.config = {"workload": names, "batch": B, "queries": Nq, "heads": nH, "head_dim": 32, "levels": L,
                 "points_per_level": P, "value_dtype": "fp32", "pass": "forward + backward",
                 "value_gradient": "float32 atomics" if atomic else "transpose gather (deterministic)"}
    if which == "tsa_train":
        wl.config["frames"] = F
    wl.dtype = "fp32"
    wl.kernel_key = ("sca_backward_kernel" if which == "sca_train" else "msda_backward_kernel") + "_fp32"

    def cpu_baseline():
        import oracle
        t0 = time.perf_counter()
        g = gout.cpu().numpy()
        if which == "sca_train":
            oracle.sca(w["value"], w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"],
                       w["bev_mask"], w["sampling_offsets"], w["attention_logits"])
            oracle.sca_backward(w["value"], w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"],
                                w["bev_mask"], w["sampling_offsets"], w["attention_logits"], g)
        elif which == "tsa_train":
            oracle.msda_frames(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"],
                               w["attention_weights"], True)
            oracle.msda_frames_backward(w["value"], w["spatial_shapes"], w["level_start_index"],
                                        w["sampling_locations"], w["attention_weights"], g, weights_are_logits=True)
        else:
            oracle.msda(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"],
                        w["attention_weights"], True)
            oracle.msda_backward(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"],
                                 w["attention_weights"], g, weights_are_logits=True)
        t = time.perf_counter() - t0
        return {"value": wl.samples / t, "unit": "samples/s", "cores": 1, "kind": "oracle",
                "sample": f"the whole workload, forward and backward ({wl.samples} samples), "
                          f"single-threaded C, {t:.1f} s"}
    wl.cpu_baseline = cpu_baseline
    return wl


def msda_workload(which):
    import numpy as np
    import torch
    import workloads as W
    import scale_deformable_attention_forward_amd as m

    if which == "detr":
        w, F = W.detr_encoder_msda(), 1
    elif which == "tiny":
        w, F = W.tiny_msda(), 1
    else:
        w = W.temporal_frames()
        F = w["F"]
    d = {k: _dev(w[k]) for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations",
                                 "attention_weights")}
    B, Nq, nH, L, P = w["B"], w["Nq"], w["nH"], w["L"], w["P"]
    out = torch.empty((B, Nq, nH * 32), dtype=torch.float32, device="cuda")
    wl = Workload(which)
    fn = m.msda_forward if F == 1 else m.msda_forward_frames
    wl.parts.append(("gather", lambda: fn(d["value"], d["spatial_shapes"], d["level_start_index"],
                                          d["sampling_locations"], d["attention_weights"], out=out)))
    wl.main = "gather"

    def finish():
        wl.samples = B * F * Nq * nH * L * P
        ss = w["spatial_shapes"]
        loc = w["sampling_locations"]
        Wd = ss[:, 1].astype(np.float64)[:, None]
        H = ss[:, 0].astype(np.float64)[:, None]
        wl.inbounds_corners = count_inbounds(ss, loc[..., 0] * Wd - 0.5, loc[..., 1] * H - 0.5)
        wl.gathered_bytes = wl.samples * 4 * 32 * 4
        wl.eff_bytes = wl.gathered_bytes + wl.samples * (8 + 4) + B * Nq * nH * 32 * 4
    wl.finish = finish
    wl.batch = B
    names = {"detr": "Deformable-DETR encoder MSDA, 4 levels 100x150/50x75/25x38/13x19, Nq=Nv=19947",
             "tiny": "tiny MSDA, 256 queries, one 32x32 level",
             "tsa": "temporal self-attention, 2 stacked 200x200 BEV maps, mean over frames"}
    wl.config = {"workload": names[which], "batch": B, "queries": Nq, "heads": nH, "head_dim": 32,
                 "levels": L, "points_per_level": P, "frames": F, "value_dtype": "fp32"}
    wl.dtype = "fp32"
    wl.kernel_key = "msda_gather_kernel_fp32"

    def cpu_baseline():
        import oracle
        t0 = time.perf_counter()
        if F == 1:
            oracle.msda(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"],
                        w["attention_weights"], True)
        else:
            oracle.msda_frames(w["value"], w["spatial_shapes"], w["level_start_index"], w["sampling_locations"],
                               w["attention_weights"], True)
        t = time.perf_counter() - t0
        return {"value": wl.samples / t, "unit": "samples/s", "cores": 1, "kind": "oracle",
                "sample": f"the whole workload ({wl.samples} samples), single-threaded C, {t:.1f} s"}
    wl.cpu_baseline = cpu_baseline
    return wl


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sca",
                    choices=["sca", "layer_bf16", "layer_full", "sca_bf16", "sca_rebatch", "sca_train", "detr",
                             "detr_train", "sca_train_atomic", "detr_train_atomic", "tsa", "tiny", "sca_frame6",
                             "tsa_train", "tsa_train_atomic"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=5,
                    help="steps timed after a 1 GiB write that evicts the caches (0: none)")
    ap.add_argument("--calibrate-copy", action="store_true")
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

    if args.workload in ("sca", "layer_bf16", "layer_full", "sca_bf16", "sca_frame6"):
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
    achieved = wl.eff_bytes / (kernel_ms * 1e-3) / 1e9
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
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(wl.name, wl.kernel_key.rsplit("_", 1)[0]),
                     "kernel": wl.kernel_key.rsplit("_", 1)[0], "kernel_ms": kernel_ms,
                     "effective_bytes_per_launch": wl.eff_bytes, "gathered_bytes_per_launch": wl.gathered_bytes},
        "effective_GBps_per_step": wl.eff_bytes / (ms_per_step * 1e-3) / 1e9,
        "samples_per_step": wl.samples,
        "batch_items_per_s": wl.batch / (ms_per_step * 1e-3),
        "step_ms_events": pct(step_ms),
        "breakdown": breakdown,
        "cold": cold,
    }
    if getattr(wl, "extra_info", None):
        line["config"].update(wl.extra_info)
    if wl.inbounds_corners is not None:
        elem = 2 if "bf16" in wl.dtype else 4
        line["roofline"]["gathered_bytes_in_bounds_per_launch"] = wl.inbounds_corners * 32 * elem
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = {**wl.cpu_baseline(), **host_cpu()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
