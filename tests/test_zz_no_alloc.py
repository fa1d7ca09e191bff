"""rq_linear_decode_noalloc (the decode linear without a workspace: its codes
and scales live in the library's own device array) through the C ABI,
against rq_linear_decode with a caller workspace: y bit for bit, on calls in
a row whose second input is smaller than the first, into guarded outputs."""

import ctypes
import sys

import numpy as np
import pytest

from rotation_w4a4_quantization_amd import datagen
from tests.guard import SENTINELS, Out, check_all

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def rq():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import rotation_w4a4_quantization_amd as rq
    rq.load_library()
    return rq


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def test_noalloc_matches_workspace_entry_point(rq):
    lib = rq.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # largest shape first (the whole scratch array), then smaller ones; m <= 4
    # takes the one-launch path, which needs no scratch
    for rep, (m, d, k, with_signs) in enumerate([(16, 8192, 3000, True), (6, 4096, 700, False),
                                                 (5, 512, 33, True), (3, 4096, 1000, True),
                                                 (16, 8192, 3000, True)]):
        rng = np.random.default_rng(1234 + rep)
        x = (rng.standard_normal((m, d)) * np.where(rng.random(d) < 0.01, 50.0, 1.0)).astype(np.float16)
        wt = (rng.standard_normal((k, d)) * 0.02).astype(np.float32)
        signs = torch.from_numpy(datagen.rademacher(rng, d)).cuda() if with_signs else None
        xd = torch.from_numpy(x).cuda()
        wc, ws, _ = rq.fold_weights(torch.from_numpy(wt).cuda(), signs)
        say(f"noalloc decode linear m={m} d={d} k={k} signs={with_signs}")
        y_ref = rq.linear_decode(xd, signs, wc, ws)
        torch.cuda.synchronize()
        yo = Out((m, k), torch.float16, SENTINELS[rep % 2])
        st = lib.rq_linear_decode_noalloc(ptr(xd), m, d, ptr(signs), ptr(wc), ptr(ws), k,
                                          ptr(yo.t), stream)
        assert st == 0, rq.status_string(st)
        check_all([yo], "noalloc y")
        assert torch.equal(yo.t.view(torch.int16), y_ref.view(torch.int16)), (m, d, k)


def test_noalloc_rejects_bad_arguments(rq):
    lib = rq.load_library()
    x = torch.zeros((17, 512), dtype=torch.float16, device="cuda")
    w = torch.zeros((8, 256), dtype=torch.uint8, device="cuda")
    s = torch.zeros((8,), dtype=torch.float16, device="cuda")
    y = torch.zeros((17, 8), dtype=torch.float16, device="cuda")
    assert lib.rq_linear_decode_noalloc(ptr(x), 17, 512, None, ptr(w), ptr(s), 8, ptr(y), None) == 2
    assert lib.rq_linear_decode_noalloc(ptr(x), 4, 16384, None, ptr(w), ptr(s), 8, ptr(y), None) == 2
    assert lib.rq_linear_decode_noalloc(None, 4, 512, None, ptr(w), ptr(s), 8, ptr(y), None) == 1
    assert lib.rq_linear_decode_noalloc(ptr(x), 0, 512, None, None, None, 8, None, None) == 0


def test_noalloc_under_graph_capture(rq):
    """The callers the entry point is for: the call captured in a HIP graph
    (it allocates nothing, so the capture holds only its kernels), replayed
    several times with eager work between the replays (including an eager
    call of the same entry point on another input, which rewrites the
    library's device array); every replay equals the eager workspace entry
    point's result bit for bit."""
    d, k = 4096, 1000
    for m in (3, 12):  # one launch; rotation into the device array, then the GEMM
        rng = np.random.default_rng(4321 + m)
        x = (rng.standard_normal((m, d)) * np.where(rng.random(d) < 0.01, 50.0, 1.0)).astype(np.float16)
        x2 = (rng.standard_normal((m, d)) * 3.0).astype(np.float16)
        wt = (rng.standard_normal((k, d)) * 0.02).astype(np.float32)
        signs = torch.from_numpy(datagen.rademacher(rng, d)).cuda()
        xd, x2d = torch.from_numpy(x).cuda(), torch.from_numpy(x2).cuda()
        wc, ws, _ = rq.fold_weights(torch.from_numpy(wt).cuda(), signs)
        y_ref = rq.linear_decode(xd, signs, wc, ws)
        y2_ref = rq.linear_decode(x2d, signs, wc, ws)
        y = torch.empty((m, k), dtype=torch.float16, device="cuda")
        y2 = torch.empty((m, k), dtype=torch.float16, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up outside the capture
            rq.linear_decode_noalloc(xd, signs, wc, ws, out=y)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        say(f"noalloc graph capture m={m}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rq.linear_decode_noalloc(xd, signs, wc, ws, out=y)
        for rep in range(4):
            y.fill_(float("nan"))  # a fill kernel, eager
            rq.linear_decode_noalloc(x2d, signs, wc, ws, out=y2)  # eager, other input
            torch.cuda.synchronize()
            assert torch.equal(y2.view(torch.int16), y2_ref.view(torch.int16)), (m, rep)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (m, rep)
        del g
        torch.cuda.synchronize()
