"""The library called from several host threads at once, each on its own
stream (ctypes releases the interpreter lock during the C calls, so the
library's host code runs concurrently).  Every result must equal the serial
run bit for bit, and the error text msda_last_error() returns is the calling
thread's own.  Every call goes through the C ABI (via the ctypes binding)."""
import threading

import pytest
import torch

from gpu_util import announce, dev, host
from test_gpu_streams import CASES

pytestmark = pytest.mark.gpu

msda = pytest.importorskip("scale_deformable_attention_forward_amd")

THREADS = 4
ROUNDS = 3
WIDTHS = (8, 16, 24, 40)  # head widths the library refuses, one per thread
PICKED = [c for c in CASES if c[0] in ("msda_forward", "msda_backward", "sca_forward", "sca_backward",
                                       "msda_backward_frames", "msda_output_proj_bf16")]


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _tensors(r):
    return list(r) if isinstance(r, tuple) else [r]


def _run_threads(work):
    errors = []

    def body(i):
        try:
            work(i)
        except BaseException as e:  # reported on the main thread
            errors.append((i, e))

    ts = [threading.Thread(target=body, args=(i,)) for i in range(THREADS)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ts), "a thread did not finish"
    assert not errors, errors


def test_concurrent_threads_match_the_serial_run():
    inputs = {name: {k: dev(v) for k, v in make().items()} for name, make, _ in PICKED}
    ref = {name: [host(t) for t in _tensors(call(inputs[name], None))] for name, _, call in PICKED}
    torch.cuda.synchronize()
    got = {}

    def work(i):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for r in range(ROUNDS):
                for name, _, call in PICKED:
                    out = _tensors(call(inputs[name], None))
                    s.synchronize()
                    got[(i, r, name)] = [host(t) for t in out]

    _run_threads(work)
    assert len(got) == THREADS * ROUNDS * len(PICKED)
    for (i, r, name), outs in got.items():
        for k, (a, b) in enumerate(zip(ref[name], outs)):
            assert a.tobytes() == b.tobytes(), f"thread {i}, round {r}, {name}: output {k} differs"


def test_error_text_is_per_thread():
    """Thread i makes a call the library rejects for a reason of its own (a
    head width other than 32, different in every thread, refused before any
    launch) and then a good one; the message it gets names its own width."""
    make_in = [c for c in CASES if c[0] == "msda_forward"][0][1]
    good = {k: dev(v) for k, v in make_in().items()}
    seen = {}

    def work(i):
        width = WIDTHS[i]
        bad_value = torch.zeros((1, 4, 8, width), device="cuda")
        loc = torch.zeros((1, 2, 8, 1, 4, 2), device="cuda")
        w = torch.zeros((1, 2, 8, 4), device="cuda")
        ss = torch.tensor([[2, 2]], dtype=torch.int64, device="cuda")
        st = torch.zeros(1, dtype=torch.int64, device="cuda")
        for _ in range(20):
            with pytest.raises(msda.MsdaError) as e:
                msda.msda_forward(bad_value, ss, st, loc, w)
            seen.setdefault(i, set()).add(str(e.value))
            msda.msda_forward(good["value"], good["ss"], good["starts"], good["loc"], good["logits"])

    _run_threads(work)
    for i, msgs in seen.items():
        assert len(msgs) == 1, msgs
        assert f"Dh={WIDTHS[i]}:" in next(iter(msgs)), (i, msgs)
