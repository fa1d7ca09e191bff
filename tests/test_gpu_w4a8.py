"""GPU parity of the W4A8 variant (INT8 per-token activations, INT4 weights):
rq_fwht_quant8 and rq_w4a8_gemm through the C ABI against the CPU oracle.

Rotation: bit-identical rotated rows and scales against the fp32 mirror, codes
equal up to the INT8 rounding band (tests/parity.py); GEMM: exact int32
accumulators, fp16 outputs within 1e-2.
"""

import sys

import numpy as np
import pytest

from oracle import rq_oracle as O
from rotation_w4a4_quantization_amd import datagen
from tests.guard import SENTINELS, Out, check_all
from tests.parity import check_gemm, check_rotation_result

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return None if t is None else t.cpu().numpy()


def run_fq8(rq, x, signs, debug=True, sentinel=0xFF):
    """One rq_fwht_quant8 call into guarded, sentinel-filled outputs."""
    m, n = x.shape
    specs = [((m, n), torch.int8), ((m,), torch.float16)] + ([((m, n), torch.float32)] if debug else [])
    o = [Out(sh, dt, sentinel) for sh, dt in specs]
    rq.fwht_quant8(dev(x), None if signs is None else dev(signs), debug=debug,
                   out=tuple(t.t for t in o))
    check_all(o, f"fwht_quant8 n={n}")
    return o[0].host(), o[1].host(), (o[2].host() if debug else None)


@pytest.mark.parametrize("n", [512, 1024, 2048, 4096, 8192])
def test_fwht_quant8_sizes_ragged(rq, n):
    rng = np.random.default_rng(800 + n)
    m = 37  # several 4-wave blocks plus a ragged last one
    say(f"fwht_quant8 n={n} m={m}")
    x = (rng.standard_normal((m, n)) * rng.uniform(0.1, 10, (m, 1))).astype(np.float16)
    x[0, rng.integers(n)] *= 100  # an outlier channel
    for signs in (datagen.rademacher(rng, n), None):
        c, s, r = run_fq8(rq, x, signs)
        check_rotation_result(x, signs, c, s, r, what=f"int8 n={n}", bits=8)
        for sentinel in SENTINELS:  # the launch the benchmark times, against the oracle
            c2, s2, _ = run_fq8(rq, x, signs, debug=False, sentinel=sentinel)
            check_rotation_result(x, signs, c2, s2, None, what=f"int8 n={n} timed", bits=8)
            assert np.array_equal(c, c2) and np.array_equal(s.view(np.uint16), s2.view(np.uint16))


def test_fwht_quant8_special_rows(rq):
    n = 4096
    rng = np.random.default_rng(6)
    signs = datagen.rademacher(rng, n)
    x = np.zeros((6, n), np.float16)
    x[1, 123] = 3.0                       # one-hot: every code +-127
    x[2, :3] = [6e-8, -6e-8, 0.0]         # a / 127 below half the smallest fp16 subnormal
    x[3, :4] = [4e-3, -4e-3, 1e-3, 0.0]   # fp16-subnormal scale (the clamped path)
    x[4] = rng.standard_normal(n) * 1e4   # large but finite scale
    x[5, :] = 2.0                         # constant row: all energy in element 0
    say("fwht_quant8 special rows")
    c, s, r = run_fq8(rq, x, signs)
    check_rotation_result(x, signs, c, s, r, what="int8 special rows", bits=8)
    assert not c[0].any() and s.view(np.uint16)[0] == 0
    assert set(np.abs(c[1].astype(np.int16)).tolist()) == {127}
    assert not c[2].any() and s.view(np.uint16)[2] == 0
    assert 0 < s.view(np.uint16)[3] < 0x0400
    assert np.isfinite(s.astype(np.float32)[4]) and np.abs(c[4].astype(np.int16)).max() == 127


def test_fwht_quant8_ties_round_to_even(rq):
    # x = a e_i + b e_j with a + b = 63.5, a - b = v / 2 (n = 4096, no signs):
    # x~ takes the values +-(a + b) / 64 and +-(a - b) / 64, the scale is
    # fp16(63.5 / 64 / 127) = 2^-7 exactly, and x~ / scale = +-127 or +-v
    # with no rounding anywhere (every operand is a short binary fraction).
    n, i, j = 4096, 5, 3000
    ties = {0.5: 0, 1.5: 2, 2.5: 2, 3.5: 4, 100.5: 100, 125.5: 126, 126.5: 126}
    x = np.zeros((len(ties), n), np.float16)
    for r, v in enumerate(ties):
        x[r, i], x[r, j] = 31.75 + v / 4, 31.75 - v / 4
    say("fwht_quant8 tie table")
    c, s, _ = run_fq8(rq, x, None)
    assert (s.view(np.uint16) == np.float16(2.0 ** -7).view(np.uint16)).all()
    eye = np.zeros((2, n))
    eye[0, i] = eye[1, j] = 1.0
    hi, hj = O.hadamard_transform(eye)  # rows i and j of the Sylvester matrix
    for r, (v, want) in enumerate(ties.items()):
        codes = c[r].astype(np.int16)
        # columns where the two one-hot contributions agree give +-127, the
        # others +-v rounded half to even
        big = np.abs(codes) == 127
        assert big.sum() == n // 2, (v, int(big.sum()))
        assert set(np.abs(codes[~big]).tolist()) == {want}, v
        assert np.array_equal(big, hi == hj)
        nz = codes != 0  # the +-0.5 ties round to 0
        want_sign = np.sign(x[r, i].astype(np.float64) * hi + x[r, j].astype(np.float64) * hj)
        assert np.array_equal(np.sign(codes[nz]), want_sign[nz])


# decode kernel (m <= 16, d a multiple of 256) with one and two 16-row weight
# groups per workgroup, several 2 KB chunks, and the tile kernel (m > 16 or
# d not a multiple of 256) with ragged edges; the persistent prefill kernel
# (m >= 128, k >= 224, d a multiple of 256) with full 256 x 224 tiles (the
# LDS-staged store path on the second, non-debug call), edge tiles in both
# dimensions, one tile over 64 steps of 128 codes, and the smallest shape
# (one edge tile, two steps)
GEMM8_SHAPES = [(1, 1, 64), (4, 17, 256), (16, 15, 512), (16, 12300, 512), (3, 40, 8192),
                (5, 33, 192), (17, 33, 64), (130, 129, 256), (300, 260, 1024), (129, 257, 4160),
                (512, 448, 512), (300, 456, 512), (256, 224, 8192), (128, 224, 256)]


@pytest.mark.parametrize("m,k,d", GEMM8_SHAPES)
def test_w4a8_gemm_random_codes(rq, m, k, d):
    rng = np.random.default_rng(m * 1000 + k + d + 8)
    ac = datagen.random_codes8(rng, m, d)
    wc = datagen.random_codes(rng, k, d)
    sa = datagen.random_scales(rng, m)
    sw = datagen.random_scales(rng, k)
    say(f"w4a8 gemm m={m} k={k} d={d}")
    yo, ao = Out((m, k), torch.float16), Out((m, k), torch.int32)
    rq.w4a8_gemm(dev(ac), dev(sa), dev(wc), dev(sw), debug=True, out=yo.t, acc_out=ao.t)
    check_all([yo, ao], "w4a8 debug")
    check_gemm(ac, sa, wc, sw, yo.host(), ao.host(), what=f"w4a8 {m}x{k}x{d}", a8=True)
    for sentinel in SENTINELS:  # the launch the benchmark times, against the oracle
        y2 = Out((m, k), torch.float16, sentinel)
        rq.w4a8_gemm(dev(ac), dev(sa), dev(wc), dev(sw), out=y2.t)
        check_all([y2], "w4a8 timed")
        check_gemm(ac, sa, wc, sw, y2.host(), None, what=f"w4a8 {m}x{k}x{d} timed", a8=True)
        assert np.array_equal(y2.host().view(np.uint16), yo.host().view(np.uint16))


# decode, tile and prefill kernels; d = 32768 (RQ_MAX_D) puts the MFMA sum at
# 16 * 1024 * d = 2^29
@pytest.mark.parametrize("m,k,d", [(3, 40, 16384), (64, 40, 16384), (256, 224, 16384),
                                   (3, 40, 32768), (64, 40, 32768), (256, 224, 32768)])
def test_w4a8_gemm_closed_form_extremes(rq, m, k, d):
    a = np.full((m, d), -128, np.int8)
    w = O.pack_int4(np.full((k, d), -8))
    w[1::2] = O.pack_int4(np.full((1, d), 7))
    say(f"w4a8 gemm extremes m={m} k={k} d={d}")
    y, acc = rq.w4a8_gemm(dev(a), dev(np.full(m, 2.0 ** -10, np.float16)), dev(w),
                          dev(np.full(k, 2.0 ** -10, np.float16)), debug=True)
    acc = host(acc)
    assert (acc[:, 0::2] == 1024 * d).all() and (acc[:, 1::2] == -896 * d).all()
    y = host(y).astype(np.float64)
    assert (y[:, 0::2] == 1024 * d * 2.0 ** -20).all() and (y[:, 1::2] == -896 * d * 2.0 ** -20).all()


def test_w4a8_decode_linear_end_to_end(rq):
    dec = datagen.decode_linear(0)
    s = dev(dec["signs"])
    ac, sa, xr = rq.fwht_quant8(dev(dec["x"]), s, debug=True)
    torch.cuda.synchronize()
    check_rotation_result(dec["x"], dec["signs"], host(ac), host(sa), host(xr),
                          what="w4a8 decode activations", bits=8)
    for k, wt in dec["wts"].items():
        wc, ws, _ = rq.fold_weights(dev(wt), s)
        for m in (1, 4, 16):
            say(f"w4a8 decode linear m={m} k={k}")
            y, acc = rq.w4a8_gemm(ac[:m].contiguous(), sa[:m].contiguous(), wc, ws, debug=True)
            torch.cuda.synchronize()
            check_gemm(host(ac[:m]), host(sa[:m]), host(wc), host(ws), host(y), host(acc),
                       what=f"w4a8 decode m={m} k={k}", a8=True)


# the fused W4A8 decode linear (rq_linear_decode_w4a8): every n class, one
# workgroup (k = 5), one and two 16-row weight groups per workgroup (k = 12300
# and 14336 give two), no signs, and n = 4096 with one 16-row group per
# workgroup, where 8 or 4 wavefronts rotate each token (m = 1, 2; one
# wavefront for m = 3, 4)
LD8_SHAPES = [(4, 5, 512, True), (3, 40, 8192, True), (2, 300, 1024, False),
              (1, 12300, 2048, True), (4, 14336, 4096, True), (1, 5, 4096, True),
              (2, 300, 4096, False), (3, 40, 4096, True), (4, 1000, 4096, False),
              (1, 1000, 8192, False), (2, 4096, 4096, True)]


@pytest.mark.parametrize("m,k,d,with_signs", LD8_SHAPES)
def test_linear_decode_w4a8_shapes(rq, m, k, d, with_signs):
    """y of the one-launch W4A8 linear is the two-launch path's
    (rq_fwht_quant8 then rq_w4a8_gemm) bit for bit, into guarded outputs with
    both sentinels; the two-launch pieces against the oracle: INT8 codes up to
    the rounding band, accumulators exact, y within 1e-2 of the oracle's
    epilogue on those codes."""
    rng = np.random.default_rng(m * 11 + k + d)
    x = (rng.standard_normal((m, d)) * np.where(rng.random(d) < 0.01, 50.0, 1.0)).astype(np.float16)
    wt = (rng.standard_normal((k, d)) * 0.02).astype(np.float32)
    signs = datagen.rademacher(rng, d) if with_signs else None
    sd = dev(signs) if with_signs else None
    say(f"fused w4a8 decode linear m={m} k={k} d={d} signs={with_signs}")
    wc, wsc, _ = rq.fold_weights(dev(wt), sd)
    ys = []
    for sentinel in SENTINELS:
        yo = Out((m, k), torch.float16, sentinel)
        rq.linear_decode_w4a8(dev(x), sd, wc, wsc, out=yo.t)
        check_all([yo], "fused w4a8 decode")
        ys.append(yo.host())
    assert np.array_equal(ys[0].view(np.uint16), ys[1].view(np.uint16))
    a8, sa, xr = rq.fwht_quant8(dev(x), sd, debug=True)
    y2, acc2 = rq.w4a8_gemm(a8, sa, wc, wsc, debug=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ys[0].view(np.uint16), host(y2).view(np.uint16))
    check_rotation_result(x, signs, host(a8), host(sa), host(xr), what="fused w4a8 activations",
                          bits=8)
    check_gemm(host(a8), host(sa), host(wc), host(wsc), ys[0], host(acc2),
               what=f"fused w4a8 {m}x{k}x{d}", a8=True)


@pytest.mark.parametrize("m", [1, 2, 4])
def test_linear_decode_w4a8_special_tokens(rq, m):
    """Tokens whose INT8 scale is zero or fp16-subnormal (the code clamp), a
    token of +-65504 (every code +-127 at the largest rotated value) and an
    ordinary one, at n = 4096 where several wavefronts rotate a token (m = 1,
    2) or one does (m = 4): y is the two-launch path's, bit for bit."""
    rng = np.random.default_rng(900 + m)
    d, k = 4096, 64
    signs = datagen.rademacher(rng, d)
    sd = dev(signs)
    rows = [np.zeros(d), rng.standard_normal(d) * 1e-4, 65504.0 * signs.astype(np.float64),
            rng.standard_normal(d) * np.where(rng.random(d) < 0.01, 50.0, 1.0)]
    x = np.stack(rows[1:2] if m == 1 else rows[:m]).astype(np.float16)
    wt = (rng.standard_normal((k, d)) * 0.02).astype(np.float32)
    say(f"fused w4a8 decode linear special tokens m={m}")
    wc, wsc, _ = rq.fold_weights(dev(wt), sd)
    yo = Out((m, k), torch.float16)
    rq.linear_decode_w4a8(dev(x), sd, wc, wsc, out=yo.t)
    check_all([yo], "fused w4a8 special")
    a8, sa, xr = rq.fwht_quant8(dev(x), sd, debug=True)
    y2 = rq.w4a8_gemm(a8, sa, wc, wsc)[0]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(yo.host().view(np.uint16), host(y2).view(np.uint16))
    check_rotation_result(x, signs, host(a8), host(sa), host(xr), what="w4a8 special", bits=8)
    sa = host(sa).view(np.uint16)
    if m == 1:
        assert 0 < sa[0] < 0x0400
    if m == 4:
        assert sa[0] == 0 and 0 < sa[1] < 0x0400 and sa[2] < 0x7C00


def test_linear_decode_w4a8_workload(rq):
    """The decode-linear workload (4096 -> 4096 and 4096 -> 14336, m = 1, 2,
    4): the one-launch W4A8 linear against the two-launch path, twice."""
    dec = datagen.decode_linear(0)
    s = dev(dec["signs"])
    for k, wt in dec["wts"].items():
        wc, wsc, _ = rq.fold_weights(dev(wt), s)
        for m in (1, 2, 4):
            say(f"fused w4a8 decode workload m={m} k={k}")
            x = dev(dec["x"][:m])
            for rep in range(2):
                y = rq.linear_decode_w4a8(x, s, wc, wsc)
                y_ref = rq.w4a8_linear(x, s, wc, wsc)
                torch.cuda.synchronize()
                assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (m, k, rep)


def test_w4a8_linear_beats_w4a4_error(rq):
    """INT8 activations cut the linear's error against the float product (the
    reason for the variant): on the decode workload the W4A8 output is closer
    to x W than the W4A4 output."""
    dec = datagen.decode_linear(0)
    s = dev(dec["signs"])
    k, wt = next(iter(dec["wts"].items()))
    wc, ws, _ = rq.fold_weights(dev(wt), s)
    x = dev(dec["x"])
    y8 = host(rq.w4a8_linear(x, s, wc, ws)).astype(np.float64)
    y4 = host(rq.w4a4_linear(x, s, wc, ws)).astype(np.float64)
    ref = dec["x"].astype(np.float64) @ wt.astype(np.float64).T
    e8 = np.linalg.norm(y8 - ref) / np.linalg.norm(ref)
    e4 = np.linalg.norm(y4 - ref) / np.linalg.norm(ref)
    say(f"relative error vs float linear: w4a8 {e8:.4f}, w4a4 {e4:.4f}")
    assert e8 < e4


def test_w4a8_empty(rq):
    c, s, _ = rq.fwht_quant8(torch.zeros((0, 512), dtype=torch.float16, device="cuda"))
    assert c.shape == (0, 512)
    y, _ = rq.w4a8_gemm(torch.zeros((0, 64), dtype=torch.int8, device="cuda"),
                        torch.zeros((0,), dtype=torch.float16, device="cuda"),
                        torch.zeros((5, 32), dtype=torch.uint8, device="cuda"),
                        torch.ones((5,), dtype=torch.float16, device="cuda"))
    assert y.shape == (0, 5)
    torch.cuda.synchronize()


def test_w4a8_prefill_full_size_sampled(rq):
    # the prefill configuration, launched as the benchmark does (the
    # persistent kernel with LDS-staged stores, 128-code steps): the oracle on
    # every row x sampled columns and sampled rows x every column
    w = datagen.prefill_linear(0)
    s = dev(w["signs"])
    say("w4a8 prefill: fold 28672x8192, INT8 rotation of 2048x8192")
    wc, ws, _ = rq.fold_weights(dev(w["wt"]), s)
    a8, sa, _ = rq.fwht_quant8(dev(w["x"]), s)
    say("w4a8 prefill: gemm 2048x8192 -> 28672")
    m, k = a8.shape[0], wc.shape[0]
    yo, ao = Out((m, k), torch.float16), Out((m, k), torch.int32)
    rq.w4a8_gemm(a8, sa, wc, ws, debug=True, out=yo.t, acc_out=ao.t)
    check_all([yo, ao], "w4a8 prefill debug")
    y2 = Out((m, k), torch.float16, SENTINELS[1])
    rq.w4a8_gemm(a8, sa, wc, ws, out=y2.t)  # the launch the benchmark times
    check_all([y2], "w4a8 prefill timed")
    assert torch.equal(yo.t.view(torch.int16), y2.t.view(torch.int16))
    a8, sa, wc, ws, y, acc, yt = map(host, (a8, sa, wc, ws, yo.t, ao.t, y2.t))
    del yo, ao, y2
    rng = np.random.default_rng(78)
    rows = np.sort(rng.choice(2048, 128, replace=False))
    cols = np.sort(rng.choice(28672, 256, replace=False))
    check_gemm(a8, sa, wc, ws, y, acc, what="w4a8 prefill cols", cols=cols, a8=True)
    check_gemm(a8, sa, wc, ws, y, acc, what="w4a8 prefill rows", rows=rows, a8=True)
    check_gemm(a8, sa, wc, ws, yt, None, what="w4a8 prefill timed cols", cols=cols, a8=True)
