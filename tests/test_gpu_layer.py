"""The attention layer around the sampling core, against the CPU oracle:
query projections (sampling offsets and logits from query + position
embedding, one launch), the output projection with the residual and the
layer norm, and the whole layer chained on the batch-4 bf16 layer workload's shapes.  Every call
goes through the C ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_abs_close, assert_fp32_close, dev, host, oracle_by_rows

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _bf16(g, shape, scale):
    return W.bf16_bits_trunc(g.normal(size=shape).astype(np.float32) * np.float32(scale))


# ---------------------------------------------------------------------------
# query projections
# ---------------------------------------------------------------------------

def _query_proj_rows(w, q, e):
    """The oracle's offsets and logits of every row, side by side."""
    n_off = w["W_off"].shape[0]
    both = oracle_by_rows(lambda r: np.concatenate(oracle.query_proj(q[r], e[r], w["W_off"], w["b_off"], w["W_att"],
                                                                     w["b_att"]), axis=1), np.arange(q.shape[0]))
    return both[:, :n_off], both[:, n_off:]


def test_query_proj_full_size():
    """The batch-4 bf16 layer workload's query path: M = 4 x 40000 queries, K = 256, offsets 512 and
    logits 256 columns, with position embedding and biases.  Every row
    against the oracle, float32 tolerance."""
    w = W.bevformer_layer_bf16(bias=True)
    q = w["query"].reshape(-1, 256)
    e = w["query_pos"].reshape(-1, 256)
    M = q.shape[0]
    off, lg = msda.msda_query_proj_bf16(dev(q), dev(w["W_off"]), dev(w["b_off"]), dev(w["W_att"]), dev(w["b_att"]),
                                        query_pos=dev(e))
    ref_off, ref_lg = _query_proj_rows(w, q, e)
    assert_fp32_close(host(off), ref_off, f"sampling offsets, all {M} rows")
    assert_fp32_close(host(lg), ref_lg, f"attention logits, all {M} rows")


QP_EDGE = [
    # id, seed, M, K, N_off, N_att, pos, bias
    ("ragged_small_no_pos_no_bias", 1, 77, 64, 32, 16, False, False),
    ("logits_cross_a_column_block", 2, 130, 256, 96, 272, True, True),
    ("single_row", 3, 1, 32, 64, 48, True, False),
    ("tail_of_one_row", 4, 64 * 9 + 1, 128, 512, 256, True, True),
]


@pytest.mark.parametrize("case", QP_EDGE, ids=[c[0] for c in QP_EDGE])
def test_query_proj_edge_cases(case):
    _, seed, M, K, N_off, N_att, pos, bias = case
    g = np.random.default_rng(seed)
    q = g.normal(size=(M, K)).astype(np.float32)
    e = g.normal(size=(M, K)).astype(np.float32) if pos else None
    W_off, W_att = _bf16(g, (N_off, K), 0.1), _bf16(g, (N_att, K), 0.1)
    b_off = g.normal(size=N_off).astype(np.float32) if bias else None
    b_att = g.normal(size=N_att).astype(np.float32) if bias else None
    off, lg = msda.msda_query_proj_bf16(dev(q), dev(W_off), None if b_off is None else dev(b_off), dev(W_att),
                                        None if b_att is None else dev(b_att),
                                        query_pos=None if e is None else dev(e))
    ref_off, ref_lg = oracle.query_proj(q, e, W_off, b_off, W_att, b_att)
    assert_fp32_close(host(off), ref_off, "offsets")
    assert_fp32_close(host(lg), ref_lg, "logits")


# ---------------------------------------------------------------------------
# output projection, residual, layer norm
# ---------------------------------------------------------------------------

def _out_case(seed, M, N, K):
    g = np.random.default_rng(seed)
    return {"X": g.normal(size=(M, K)).astype(np.float32), "W": _bf16(g, (N, K), 1.0 / np.sqrt(K)),
            "bias": (0.1 * g.normal(size=N)).astype(np.float32), "res": g.normal(size=(M, N)).astype(np.float32),
            "gamma": (1.0 + 0.1 * g.normal(size=N)).astype(np.float32),
            "beta": (0.1 * g.normal(size=N)).astype(np.float32)}


def test_output_proj_residual_norm_full_size():
    """The batch-4 bf16 layer workload's output side: M = 160000 slots rows, K = N = 256, residual
    and layer norm; every row, float32 tolerance."""
    M = 4 * 40000
    c = _out_case(71, M, 256, 256)
    y = msda.msda_output_proj_bf16(dev(c["X"]), dev(c["W"]), dev(c["bias"]), residual=dev(c["res"]),
                                   gamma=dev(c["gamma"]), beta=dev(c["beta"]), eps=1e-5)
    ref = oracle_by_rows(lambda r: oracle.output_proj(c["X"][r], c["W"], c["bias"], c["res"][r], c["gamma"],
                                                      c["beta"], 1e-5), np.arange(M))
    assert_fp32_close(host(y), ref, f"projection + residual + norm, all {M} rows")


OP_EDGE = [
    # id, seed, M, N, K, x_bf16, residual, norm, in_place
    ("plain_ragged", 1, 77, 256, 256, False, False, False, False),
    ("residual_only_wide", 2, 200, 512, 64, False, True, False, False),
    ("residual_in_place", 3, 130, 256, 256, False, True, False, True),
    ("norm_without_residual", 4, 65, 256, 128, False, False, True, False),
    ("norm_in_place_bf16_input", 5, 129, 256, 256, True, True, True, True),
    ("norm_single_row", 6, 1, 256, 32, False, True, True, False),
]


@pytest.mark.parametrize("case", OP_EDGE, ids=[c[0] for c in OP_EDGE])
def test_output_proj_edge_cases(case):
    _, seed, M, N, K, x_bf16, residual, norm, in_place = case
    c = _out_case(seed, M, N, K)
    X = c["X"]
    if x_bf16:
        X = W.bf16_bits_trunc(X)
        x_ref = ((X.astype(np.uint32) << 16).view(np.float32))  # exact float32 value of each bf16 input
    else:
        x_ref = X
    res = dev(c["res"]) if residual else None
    out = res if in_place else None
    g, b = (dev(c["gamma"]), dev(c["beta"])) if norm else (None, None)
    y = msda.msda_output_proj_bf16(dev(X), dev(c["W"]), dev(c["bias"]), residual=res, gamma=g, beta=b, eps=1e-5,
                                   out=out)
    ref = oracle.output_proj(x_ref, c["W"], c["bias"], c["res"] if residual else None,
                             c["gamma"] if norm else None, c["beta"] if norm else None, 1e-5)
    assert_fp32_close(host(y), ref, "output projection")


def test_output_proj_norm_constant_rows():
    """Rows that are constant after the residual have zero variance: the norm
    returns beta exactly (0 * rsqrt(eps) * gamma + beta).  This needs the row
    mean to come out exact, which the kernel's power-of-two partial sums
    (pairwise across waves) give for a constant row."""
    M, N, K = 70, 256, 64
    g = np.random.default_rng(9)
    X = np.zeros((M, K), np.float32)
    Wz = np.zeros((N, K), np.uint16)
    res = np.repeat(g.normal(size=(M, 1)).astype(np.float32), N, axis=1)
    gamma = g.uniform(0.5, 2.0, N).astype(np.float32)
    beta = g.normal(size=N).astype(np.float32)
    y = msda.msda_output_proj_bf16(dev(X), dev(Wz), None, residual=dev(res), gamma=dev(gamma), beta=dev(beta))
    assert np.array_equal(host(y), np.broadcast_to(beta, (M, N)))


# ---------------------------------------------------------------------------
# the whole layer on the batch-4 bf16 layer workload's shapes
# ---------------------------------------------------------------------------

def test_whole_layer_bf16():
    """query -> offsets and logits (one launch); feat -> bf16 value; bev_mask ->
    compaction; sampling and camera mean; output projection + residual +
    layer norm.  The oracle runs its own chain (its own projections, its own
    bf16 value) on every query; 1e-2 absolute on the unit-scale result."""
    w = W.bevformer_layer_bf16(bias=True)
    B, Ncam, Nq, Nv = w["B"], w["Ncam"], w["Nq"], w["Nv"]
    C = 256
    q = w["query"].reshape(-1, C)
    e = w["query_pos"].reshape(-1, C)
    feat = w["feat"].reshape(-1, C)

    off, lg = msda.msda_query_proj_bf16(dev(q), dev(w["W_off"]), dev(w["b_off"]), dev(w["W_att"]), dev(w["b_att"]),
                                        query_pos=dev(e))
    value = msda.msda_gemm_bf16(dev(feat), dev(w["W_v"]), dev(w["b_v"]), y_dtype=torch.bfloat16)
    L, P = w["L"], w["P"]
    slots = msda.sca_forward(value.view(B, Ncam, Nv, 8, 32), dev(w["spatial_shapes"]), dev(w["level_start_index"]),
                             dev(w["reference_points_cam"]), dev(w["bev_mask"]), off.view(B, Nq, 8, L, P, 2),
                             lg.view(B, Nq, 8, L * P))
    qd = dev(q)
    out = msda.msda_output_proj_bf16(slots.view(-1, C), dev(w["W_o"]), dev(w["b_o"]), residual=qd,
                                     gamma=dev(w["gamma"]), beta=dev(w["beta"]), eps=1e-5)
    got = host(out)

    # oracle chain on every query: its own offsets and logits, its own bf16
    # value, its own slots, its own output projection + residual + norm
    ref_off, ref_lg = _query_proj_rows(w, q, e)
    ref_off = ref_off.astype(np.float32).reshape(B, Nq, 8, L, P, 2)
    ref_lg = ref_lg.astype(np.float32).reshape(B, Nq, 8, L * P)
    ref_value = oracle.round_to_bf16(oracle.linear_bf16_blas(feat, w["W_v"], w["b_v"])).reshape(B, Ncam, Nv, 8, 32)
    ref_slots = oracle_by_rows(lambda r: oracle.sca(ref_value, w["spatial_shapes"], w["level_start_index"],
                                                    w["reference_points_cam"], w["bev_mask"], ref_off, ref_lg,
                                                    rows=r)["slots"], np.arange(B * Nq))
    ref_out = oracle_by_rows(lambda r: oracle.output_proj(ref_slots[r].astype(np.float32), w["W_o"], w["b_o"], q[r],
                                                          w["gamma"], w["beta"], 1e-5), np.arange(B * Nq))
    assert_abs_close(got, ref_out, 1e-2, f"whole layer output, all {B * Nq} queries")


def test_float32_to_bf16_rounding_on_ties():
    """float32 X is rounded to bf16 on the way into the matrix cores: an
    identity W returns the rounded input (bf16 output, exact).  Ties and near
    ties around several binades must round to nearest, ties to even, as
    torch's float32 -> bfloat16 conversion does."""
    K = 64
    base = np.array([1.0, 1.5, -2.0, 3.0e-3, 7.0e5, -1.25e-20], np.float64)
    steps = np.array([0.5, 1.5, 2.5, 0.5 + 2.0 ** -10, 0.5 - 2.0 ** -10, 0.0, 1.0, 3.5])
    vals = []
    for b in base:
        ulp = 2.0 ** (np.floor(np.log2(abs(b))) - 7)  # bf16 spacing at b
        vals += [b + s * ulp * np.sign(b) for s in steps]
    X = np.resize(np.array(vals, np.float32), (8, K))
    eye = np.zeros((K, K), np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    y = msda.msda_gemm_bf16(dev(X), dev(eye), None, y_dtype=torch.bfloat16)
    ref = torch.from_numpy(X).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(host(y), ref)
