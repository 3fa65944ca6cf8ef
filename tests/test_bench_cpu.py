"""Host logic of bench.py (no GPU): the kernel-source digest that gates the
stored counter traffic, the traffic lookup, the in-map corner count used as
measurement metadata, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _digest_of(tmp_path, text):
    (tmp_path / "k.hip").write_text(text)
    old = bench.ROOT
    bench.ROOT = str(tmp_path)
    try:
        return bench.source_digest(["k.hip"])
    finally:
        bench.ROOT = old


def test_source_digest_ignores_comments_and_layout(tmp_path):
    base = _digest_of(tmp_path, 'int f(int a) {\n  return a + 1;  // one\n}\nconst char* s = "//x";\n')
    assert _digest_of(tmp_path, '// header\nint f(int a) { return a + 1; /* two */ }\n'
                                'const char* s = "//x";\n') == base
    # code changes, including inside a string that looks like a comment, change it
    assert _digest_of(tmp_path, 'int f(int a) {\n  return a + 2;\n}\nconst char* s = "//x";\n') != base
    assert _digest_of(tmp_path, 'int f(int a) {\n  return a + 1;\n}\nconst char* s = "//y";\n') != base
    assert _digest_of(tmp_path, 'int f(int a) {\n  return a+1;\n}\nconst char* s = "//x";\n') != base


def test_measured_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    digest = bench.source_digest(bench.GATHER_SOURCES)
    counters = {"w": {"kernel": "sca_gather_kernel", "source_digest": digest, "hbm_bytes_per_launch": 123.0},
                "stale": {"kernel": "sca_gather_kernel", "source_digest": "0" * 16, "hbm_bytes_per_launch": 5.0}}
    path = tmp_path / "counters.json"
    path.write_text(json.dumps(counters))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(path))
    assert bench.measured_traffic("w", "sca_gather_kernel") == 123.0
    assert bench.measured_traffic("stale", "sca_gather_kernel") is None
    assert bench.measured_traffic("missing", "sca_gather_kernel") is None
    # the backward kernels are gated by their own sources
    assert bench.measured_traffic("w", "sca_backward_kernel") is None


def test_count_inbounds_against_brute_force():
    g = np.random.default_rng(5)
    shapes = np.array([[3, 4], [1, 1], [2, 7]])
    x = g.uniform(-2, 8, (10, 3, 5))
    y = g.uniform(-2, 4, (10, 3, 5))
    n = 0
    for idx in np.ndindex(x.shape):
        H, Wd = shapes[idx[1]]
        x0, y0 = int(np.floor(x[idx])), int(np.floor(y[idx]))
        n += sum(0 <= x0 + dx < Wd and 0 <= y0 + dy < H for dx in (0, 1) for dy in (0, 1))
    assert bench.count_inbounds(shapes, x, y) == n


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_host_cpu_names_the_cores_it_may_use():
    h = bench.host_cpu()
    assert h["host_cores_available"] >= 1
    assert h["host_cpu"] is None or isinstance(h["host_cpu"], str)


# every workload's CPU-oracle baseline, on tiny inputs of the same recipes
# and on two threads: each must run and count the samples of what it timed
def _tiny_sca():
    import workloads as W
    return W.bevformer_sca(cfg=103, bev=24, shapes=((12, 20), (6, 10)))


def _tiny_layer(full):
    import workloads as W
    if full:
        return W.bevformer_layer_bf16(B=2, bev=12, shapes=((12, 20), (6, 10)))
    return W.bevformer_sca_bf16(B=2, bev=12, shapes=((12, 20), (6, 10)))


def _check_baseline(r, n_samples):
    assert r["kind"] == "oracle" and r["unit"] == "samples/s" and r["cores"] == 2
    assert r["value"] > 0 and r["single_thread"]["value"] > 0 and r["single_thread"]["cores"] == 1
    assert f"({n_samples} samples)" in r["sample"]


def test_sca_cpu_baselines_run_on_tiny_inputs():
    w = _tiny_sca()
    n = int(w["bev_mask"].any(-1).sum()) * w["nH"] * w["L"] * w["P"]
    for kind in ("sca", "sca_bf16", "sca_frame6"):
        _check_baseline(bench.sca_cpu_baseline(w, kind, cores=2), n)


def test_layer_cpu_baselines_run_on_tiny_inputs():
    import workloads as W
    for full in (False, True):
        w = _tiny_layer(full)
        rows = W.sample_rows(7, w["B"] * w["Nq"], 50)
        hit = w["bev_mask"].any(-1).sum(0).reshape(-1)[rows]
        r = bench.sca_cpu_baseline(w, "layer_full" if full else "layer_bf16", cores=2, sampled_queries=50)
        _check_baseline(r, int(hit.sum()) * w["nH"] * w["L"] * w["P"])


def test_msda_and_train_cpu_baselines_run_on_tiny_inputs():
    import workloads as W
    detr = W.msda_workload(2, 1, 60, ((8, 10), (4, 5)), P=4)
    tsa = W.temporal_frames(bev=8)
    _check_baseline(bench.msda_cpu_baseline(detr, cores=2), 60 * 8 * 2 * 4)
    _check_baseline(bench.msda_cpu_baseline(tsa, cores=2), 2 * 64 * 8 * 4)
    g = lambda w: W.upstream_gradient(9, (w["B"], w["Nq"], w["nH"] * 32))
    _check_baseline(bench.train_cpu_baseline(detr, "detr_train", g(detr), cores=2), 60 * 8 * 2 * 4)
    _check_baseline(bench.train_cpu_baseline(tsa, "tsa_train", g(tsa), cores=2), 2 * 64 * 8 * 4)
    sca = _tiny_sca()
    n = int(sca["bev_mask"].any(-1).sum()) * sca["nH"] * sca["L"] * sca["P"]
    _check_baseline(bench.train_cpu_baseline(sca, "sca_train", g(sca), cores=2), n)


def test_chunked_oracle_equals_the_whole():
    """The query ranges the baseline times cover the workload exactly: the
    oracle over the ranges, stacked, is the oracle over all queries."""
    import oracle
    w = _tiny_sca()
    args = (w["value"], w["spatial_shapes"], w["level_start_index"], w["reference_points_cam"], w["bev_mask"],
            w["sampling_offsets"], w["attention_logits"])
    whole = oracle.sca(*args)["slots"]
    parts = [oracle.sca(*args, rows=r)["slots"] for r in bench._query_chunks(w["B"] * w["Nq"], 7)]
    assert np.array_equal(np.concatenate(parts), whole)
