"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases span several blocks plus a ragged tail for every supported n;
the full-size cases run the exact launch configuration bench.py times and
compare every row (or, for the largest GEMM and KV cache, seeded samples of
rows and columns that cover every tile position).

Every output is written into a guarded buffer (tests/guard.py): pre-filled
with a sentinel and surrounded by 4 KB guard bands that must be untouched
after the call.  The launch the benchmark times (no debug outputs) is run
twice, with two different sentinels, and each result is compared with the
oracle itself, so a byte it skipped or a write past an output cannot pass.
"""

import math
import sys

import numpy as np
import pytest

from oracle import rq_oracle as O
from rotation_w4a4_quantization_amd import datagen
from tests.guard import SENTINELS, Out, check_all
from tests.parity import check_codes, check_gemm, check_rotation_result

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

REPORT = []


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


def run_fq(rq, x, signs, debug=True, fold=False, sentinel=0xFF):
    """One rq_fwht_quant (or rq_fold_weights) call into guarded outputs."""
    fn = rq.fold_weights if fold else rq.fwht_quant
    m, n = x.shape
    specs = [((m, n // 2), torch.uint8), ((m,), torch.float16)]
    if debug:
        specs.append(((m, n), torch.float32))
    o = [Out(sh, dt, sentinel) for sh, dt in specs]
    fn(dev(x), None if signs is None else dev(signs), debug=debug, out=tuple(t.t for t in o))
    check_all(o, f"fwht_quant n={n}")
    return o[0].host(), o[1].host(), (o[2].host() if debug else None)


def timed_fq_matches_oracle(rq, x, signs, want_c, want_s, what, fold=False, ref=None):
    """The launch the benchmark times (no debug output), with each sentinel:
    checked against the oracle and bit-identical to the debug launch."""
    for sentinel in SENTINELS:
        c, s, _ = run_fq(rq, x, signs, debug=False, fold=fold, sentinel=sentinel)
        check_rotation_result(x, signs, c, s, None, what=f"{what} timed", ref=ref)
        assert np.array_equal(c, want_c) and np.array_equal(s.view(np.uint16), want_s.view(np.uint16))


ALL_N = [2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192]


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("n", ALL_N)
def test_fwht_quant_all_sizes_ragged(rq, n, dtype):
    rng = np.random.default_rng(n)
    rows_per_block = 64 // max(1, n // (64 if n <= 4096 else 128)) if n > 128 else 64
    m = 2 * rows_per_block + 3 if n <= 1024 else 5
    say(f"fwht_quant n={n} m={m} dtype={np.dtype(dtype).name}")
    x = (rng.standard_normal((m, n)) * rng.uniform(0.1, 10, (m, 1))).astype(dtype)
    x[0, rng.integers(n)] *= 100  # an outlier channel
    for signs in (datagen.rademacher(rng, n), None):
        c, s, r = run_fq(rq, x, signs)
        check_rotation_result(x, signs, c, s, r, what=f"n={n}", report=REPORT)
        # the debug instantiation must not change the primary outputs
        timed_fq_matches_oracle(rq, x, signs, c, s, f"n={n}")


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("m", [1, 7, 600])
def test_fwht_quant_28x512(rq, m, dtype):
    """n = 28 * 512 (H_28 (x) H_512): rotated rows bit-identical to the
    oracle's fp32 mirror, codes within the rounding band; 600 rows exceed the
    grid, so workgroups take several rows."""
    n = 14336
    rng = np.random.default_rng(m)
    say(f"fwht_quant n=28x512 m={m} dtype={np.dtype(dtype).name}")
    x = (rng.standard_normal((m, n)) * rng.uniform(0.1, 10, (m, 1))).astype(dtype)
    x[:, rng.choice(n, 14, replace=False)] *= 100  # outlier channels
    for signs in (datagen.rademacher(rng, n), None):
        c, s, r = run_fq(rq, x, signs, fold=dtype == np.float32)
        check_rotation_result(x, signs, c, s, r, what=f"n=28x512 m={m}", report=REPORT)
        timed_fq_matches_oracle(rq, x, signs, c, s, f"n=28x512 m={m}", fold=dtype == np.float32)


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("m", [1, 7, 300])
def test_fwht_quant_28x1024(rq, m, dtype):
    """n = 28 * 1024 (H_28 (x) H_1024, the 8192 -> 28672 model's down-projection
    input): rotated rows bit-identical to the oracle's fp32 mirror, codes
    within the rounding band; 300 rows exceed the grid (one workgroup per CU),
    so workgroups take several rows."""
    n = 28672
    rng = np.random.default_rng(100 + m)
    say(f"fwht_quant n=28x1024 m={m} dtype={np.dtype(dtype).name}")
    x = (rng.standard_normal((m, n)) * rng.uniform(0.1, 10, (m, 1))).astype(dtype)
    x[:, rng.choice(n, 28, replace=False)] *= 100  # outlier channels
    for signs in (datagen.rademacher(rng, n), None):
        c, s, r = run_fq(rq, x, signs, fold=dtype == np.float32)
        check_rotation_result(x, signs, c, s, r, what=f"n=28x1024 m={m}", report=REPORT)
        timed_fq_matches_oracle(rq, x, signs, c, s, f"n=28x1024 m={m}", fold=dtype == np.float32)


@pytest.mark.parametrize("n", [14336, 28672])
def test_fwht_quant_28xP_special_rows(rq, n):
    """Zero, one-hot, underflowing, overflowing and fp16-subnormal-scale rows
    (the clamp the kernel takes as a uniform branch) at n = 28 * 512 and
    28 * 1024."""
    rng = np.random.default_rng(55)
    signs = datagen.rademacher(rng, n)
    x = np.zeros((5, n), np.float32)
    x[1, 12345] = 3.0                     # one-hot: every code +-7
    x[2] = 1e-30                          # underflows the fp16 scale -> zero codes
    x[3] = rng.standard_normal(n) * 1e6   # fp16 scale overflows -> +inf, zero codes
    x[4, :4] = [4e-4, -4e-4, 1e-4, 0.0]   # fp16-subnormal scale (clamped path)
    say(f"fwht_quant n={n} special rows")
    c, s, r = run_fq(rq, x, signs)
    check_rotation_result(x, signs, c, s, r, what=f"n={n} special rows")
    q = O.unpack_int4(c)
    assert not q[0].any() and not q[2].any() and not q[3].any()
    assert set(np.abs(q[1]).tolist()) == {7}
    assert s.view(np.uint16)[3] == 0x7C00 and 0 < s.view(np.uint16)[4] < 0x0400


@pytest.mark.parametrize("m,k,d", [(4, 40, 14336), (300, 256, 14336), (4, 40, 28672),
                                   (300, 256, 28672)])
def test_linear_28x512(rq, m, k, d):
    """A W4A4 linear with d = 14336 or 28672 (the down projection widths): the
    fold and the online rotation with H_28 (x) H_512 or H_28 (x) H_1024, then
    the decode (m = 4) or the large (m = 300) GEMM, against the oracle."""
    rng = np.random.default_rng(m + k + d)
    x = (rng.standard_normal((m, d)) * np.where(rng.random(d) < 0.001, 100.0, 1.0)).astype(np.float16)
    wt = (rng.standard_normal((k, d)) * 0.02).astype(np.float32)
    signs = datagen.rademacher(rng, d)
    say(f"linear d={d} m={m} k={k}")
    s = dev(signs)
    wc, ws, wr = rq.fold_weights(dev(wt), s, debug=True)
    ac, sa, xr = rq.fwht_quant(dev(x), s, debug=True)
    y, acc = rq.w4a4_gemm(ac, sa, wc, ws, debug=True)
    torch.cuda.synchronize()
    check_rotation_result(wt, signs, host(wc), host(ws), host(wr), what=f"fold d={d}")
    check_rotation_result(x, signs, host(ac), host(sa), host(xr), what=f"activations d={d}")
    check_gemm(host(ac), host(sa), host(wc), host(ws), host(y), host(acc), what=f"gemm d={d}")


@pytest.mark.parametrize("n", [4096, 8192])
def test_fwht_quant_special_rows(rq, n):
    rng = np.random.default_rng(5)
    signs = datagen.rademacher(rng, n)
    x = np.zeros((8, n), np.float32)
    x[1, 123] = 3.0                       # one-hot: all codes +-7
    x[2] = 1e-30                          # underflows the fp16 scale -> zero codes
    x[3, :4] = [4e-4, -4e-4, 1e-4, 0.0]   # fp16-subnormal scale (clamped path)
    x[4] = rng.standard_normal(n) * 1e6   # fp16 scale overflows -> +inf, zero codes
    x[5] = -x[5 - 4]
    x[6] = rng.standard_normal(n)
    x[7, :] = 2.0                         # constant row: all energy in element 0
    say(f"fwht_quant special rows n={n}")
    c, s, r = run_fq(rq, x, signs)
    check_rotation_result(x, signs, c, s, r, what=f"special rows n={n}")
    q = O.unpack_int4(c)
    assert set(np.abs(q[1]).tolist()) == {7}
    assert not q[0].any() and not q[2].any()
    assert s.view(np.uint16)[4] == 0x7C00 and not q[4].any()
    assert s.view(np.uint16)[0] == 0 and s.view(np.uint16)[2] == 0


@pytest.mark.parametrize("n", [16, 256, 4096])
def test_fwht_quant_tie_table_through_kernel(rq, n):
    # For n = 4^j, 1/sqrt(n) is a power of two, so x = x~ H diag(s) / sqrt(n)
    # is exact in binary and the kernel's rotation returns x~ exactly.  x~ is
    # built so that x~/scale hits the half-integer ties.
    rng = np.random.default_rng(n)
    signs = datagen.rademacher(rng, n)
    vals = np.array([7.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -1.5, 6.5, -6.5, -7.0, 4.5, 0.0, 5.5, -3.5, 2.0])
    xt = np.tile(vals, n // len(vals))[None, :] * 2.0 ** -3  # scale = fp16(a/7) = 2^-3 exactly
    x = (O.hadamard_transform(xt) / math.sqrt(n)) * signs[None, :]  # inverse rotation (H symmetric)
    assert np.array_equal(O.rotate(x, signs, "f64"), xt)
    assert np.array_equal(O.rotate(x.astype(np.float32), signs, "f32").astype(np.float64), xt)
    say(f"tie table n={n}")
    c, s, r = run_fq(rq, x.astype(np.float32), signs)
    assert float(s.astype(np.float64)[0]) == 2.0 ** -3
    q = O.unpack_int4(c)[0]
    want = np.tile(np.array([7, 2, 4, -2, 0, 0, 2, -2, 6, -6, -7, 4, 0, 6, -4, 2]), n // 16)
    np.testing.assert_array_equal(q, want)


def test_empty_inputs_are_noops(rq):
    say("empty inputs")
    c, s, r = rq.fwht_quant(torch.zeros((0, 256), dtype=torch.float16, device="cuda"))
    assert c.shape == (0, 128)
    y, acc = rq.w4a4_gemm(torch.zeros((0, 32), dtype=torch.uint8, device="cuda"),
                          torch.zeros((0,), dtype=torch.float16, device="cuda"),
                          torch.zeros((5, 32), dtype=torch.uint8, device="cuda"),
                          torch.ones((5,), dtype=torch.float16, device="cuda"))
    assert y.shape == (0, 5)
    torch.cuda.synchronize()


def test_fwht_quant_full_config(rq):
    # 4096 tokens x 4096 fp16 with 0.1% outlier channels x100: the bench workload
    w = datagen.fwht_workload(0)
    say("fwht_quant 4096x4096 fp16 (bench workload)")
    ref = (O.fwht_quant(w["x"], w["signs"], "f32"), O.fwht_quant(w["x"], w["signs"], "f64"))
    c, s, r = run_fq(rq, w["x"], w["signs"])
    nb, nt = check_rotation_result(w["x"], w["signs"], c, s, r, what="4096x4096", report=REPORT,
                                   ref=ref)
    timed_fq_matches_oracle(rq, w["x"], w["signs"], c, s, "4096x4096", ref=ref)
    say(f"  in-band mismatches vs mirror: {nb}, vs fp64: {nt}")


def test_fwht_quant_full_config_deterministic(rq):
    """20 launches of the benchmark's rotation, each into freshly
    sentinel-filled guarded outputs, give bit-identical codes and scales."""
    w = datagen.fwht_workload(0)
    x, sg = dev(w["x"]), dev(w["signs"])
    m, n = w["x"].shape
    say("fwht_quant 4096x4096: 20 repeats")
    first = None
    for rep in range(20):
        o = [Out((m, n // 2), torch.uint8, SENTINELS[rep % 2]), Out((m,), torch.float16, SENTINELS[rep % 2])]
        rq.fwht_quant(x, sg, out=(o[0].t, o[1].t))
        check_all(o, f"repeat {rep}")
        if first is None:
            first = [t.t.clone() for t in o]
        else:
            assert torch.equal(o[0].t, first[0]) and torch.equal(o[1].t.view(torch.int16),
                                                                   first[1].view(torch.int16)), rep


def test_fwht_quant_prefill_activation(rq):
    w = datagen.prefill_linear(0, with_weights=False)
    say("fwht_quant 2048x8192 fp16")
    c, s, r = run_fq(rq, w["x"], w["signs"])
    check_rotation_result(w["x"], w["signs"], c, s, r, what="2048x8192", report=REPORT)


def test_fold_tiny_and_decode_weights(rq):
    cfg = datagen.tiny_linear(0)
    say("fold 512x256 fp32")
    c, s, r = run_fq(rq, cfg["wt"], cfg["signs"], fold=True)
    check_rotation_result(cfg["wt"], cfg["signs"], c, s, r, what="fold tiny", report=REPORT)
    dec = datagen.decode_linear(0)
    for k, wt in dec["wts"].items():
        say(f"fold {k}x4096 fp32")
        c, s, r = run_fq(rq, wt, dec["signs"], fold=True)
        check_rotation_result(wt, dec["signs"], c, s, r, what=f"fold {k}", report=REPORT)


# (512, 448, 512): only full 256 x 224 tiles with 16-byte output rows (the
# LDS-staged epilogue); (300, 456, 512): full and edge tiles in both dimensions;
# (16, 12300, 512): decode with two 16-row weight groups per workgroup and a
# ragged last group; (3, 40, 8192): decode over two 2 KB chunks per row;
# (256, 60000, 256), (300, 30000, 512): 256-column tiles (one round of them on
# 256 CUs against two of 224 columns), full and edge tiles, both epilogues
GEMM_SHAPES = [(1, 1, 64), (4, 17, 128), (16, 15, 192), (16, 200, 4096), (17, 33, 64),
               (130, 129, 256), (300, 260, 1024), (129, 257, 4160), (512, 448, 512),
               (300, 456, 512), (16, 12300, 512), (3, 40, 8192), (256, 60000, 256),
               (300, 30000, 512)]


@pytest.mark.parametrize("m,k,d", GEMM_SHAPES)
def test_gemm_random_codes(rq, m, k, d):
    rng = np.random.default_rng(m * 1000 + k + d)
    ac = datagen.random_codes(rng, m, d)
    wc = datagen.random_codes(rng, k, d)
    sa = datagen.random_scales(rng, m)
    sw = datagen.random_scales(rng, k)
    say(f"gemm m={m} k={k} d={d}")
    yo, ao = Out((m, k), torch.float16), Out((m, k), torch.int32)
    rq.w4a4_gemm(dev(ac), dev(sa), dev(wc), dev(sw), debug=True, out=yo.t, acc_out=ao.t)
    check_all([yo, ao], "gemm debug")
    y_ref, _ = check_gemm(ac, sa, wc, sw, yo.host(), ao.host(), what=f"gemm {m}x{k}x{d}")
    for sentinel in SENTINELS:  # the launch the benchmark times, against the oracle
        y2 = Out((m, k), torch.float16, sentinel)
        rq.w4a4_gemm(dev(ac), dev(sa), dev(wc), dev(sw), out=y2.t)
        check_all([y2], "gemm timed")
        check_gemm(ac, sa, wc, sw, y2.host(), None, what=f"gemm {m}x{k}x{d} timed")
        assert np.array_equal(y2.host().view(np.uint16), yo.host().view(np.uint16))


def epilogue_once(acc, sa, sw):
    """The epilogue the GEMM entry points document, written out on the host:
    t = fp32(fp32(acc) * sa), then t * sw rounded once to fp16 (the float64
    product of two float32 is exact, and numpy rounds float64 to float16 once).
    Also returns the twice-rounded value fp16(fp32(t * sw)) for comparison."""
    t = acc.astype(np.float32) * sa.astype(np.float32)[:, None]
    with np.errstate(over="ignore"):
        once = (t.astype(np.float64) * sw.astype(np.float64)[None, :]).astype(np.float16)
        twice = (t * sw.astype(np.float32)[None, :]).astype(np.float16)
    return once, twice


# decode (m <= 16), the tile kernel (16 < m < 128), and the persistent prefill
# kernel with full tiles only and with edge tiles; each through the debug
# launch (direct stores) and the timed launch (LDS-staged stores)
@pytest.mark.parametrize("kind,m,k,d", [("w4a4", 8, 8000, 512), ("w4a4", 64, 1000, 1024),
                                        ("w4a4", 256, 448, 512), ("w4a4", 300, 456, 512),
                                        ("asym", 256, 448, 512), ("w4a8", 256, 448, 512)])
def test_gemm_epilogue_rounds_once(rq, kind, m, k, d):
    rng = np.random.default_rng(77 + m + k + d)
    wc = datagen.random_codes(rng, k, d)
    sa = datagen.random_scales(rng, m)
    sw = datagen.random_scales(rng, k)
    say(f"gemm epilogue rounding {kind} m={m} k={k} d={d}")
    if kind == "w4a8":
        ac = datagen.random_codes8(rng, m, d)
        _, acc_ref = O.w4a8_gemm(ac, sa, wc, sw)
        run = lambda debug: rq.w4a8_gemm(dev(ac), dev(sa), dev(wc), dev(sw), debug=debug)[0]
    elif kind == "asym":
        ac = datagen.random_codes(rng, m, d)
        za = rng.integers(0, 16, m).astype(np.uint8)
        _, acc_ref = O.w4a4_gemm_asym(ac, sa, za, wc, sw)
        wsum = rq.weight_code_sums(dev(wc))
        run = lambda debug: rq.w4a4_gemm_asym(dev(ac), dev(sa), dev(za), dev(wc), dev(sw), wsum,
                                              debug=debug)[0]
    else:
        ac = datagen.random_codes(rng, m, d)
        _, acc_ref = O.w4a4_gemm(ac, sa, wc, sw)
        run = lambda debug: rq.w4a4_gemm(dev(ac), dev(sa), dev(wc), dev(sw), debug=debug)[0]
    once, twice = epilogue_once(acc_ref, sa, sw)
    assert (once.view(np.uint16) != twice.view(np.uint16)).any(), "no case where the roundings differ"
    for debug in (True, False):
        y = host(run(debug))
        bad = y.view(np.uint16) != once.view(np.uint16)
        assert not bad.any(), f"{kind} {m}x{k}x{d} debug={debug}: {int(bad.sum())} outputs differ"


# decode (m = 3), tile (m = 64) and prefill (m = 256, k = 224) kernels, at
# d = 8192 and at the largest d (RQ_MAX_D = 32768, where the W4A4 MFMA sum
# 256 * 64 * d = 2^29 is the largest the int32 path has to hold)
@pytest.mark.parametrize("m,k,d", [(3, 40, 8192), (64, 40, 8192), (3, 40, 32768), (64, 40, 32768),
                                   (256, 224, 32768)])
def test_gemm_closed_form_extremes(rq, m, k, d):
    a = O.pack_int4(np.full((m, d), -8))
    w = O.pack_int4(np.full((k, d), -8))
    w[1::2] = O.pack_int4(np.full((1, d), 7))
    say(f"gemm extremes m={m} k={k} d={d}")
    y, acc = rq.w4a4_gemm(dev(a), dev(np.ones(m, np.float16)), dev(w), dev(np.ones(k, np.float16)),
                          debug=True)
    acc = host(acc)
    assert (acc[:, 0::2] == 64 * d).all() and (acc[:, 1::2] == -56 * d).all()
    # unit scales: y = fp16(acc); 64 d >= 524288 overflows fp16 -> inf
    assert np.isinf(host(y)[:, 0]).all() and (host(y)[:, 1] < 0).all()
    # the launch the benchmark times gives the same y
    y2, _ = rq.w4a4_gemm(dev(a), dev(np.ones(m, np.float16)), dev(w), dev(np.ones(k, np.float16)))
    assert np.array_equal(host(y2).view(np.uint16), host(y).view(np.uint16))


def test_decode_linear_end_to_end(rq):
    dec = datagen.decode_linear(0)
    s = dev(dec["signs"])
    for k, wt in dec["wts"].items():
        wc, ws, _ = rq.fold_weights(dev(wt), s)
        for m in (1, 4, 16):
            say(f"decode linear m={m} k={k}")
            x = dec["x"][:m]
            ac, sa, _ = rq.fwht_quant(dev(x), s)
            y, acc = rq.w4a4_gemm(ac, sa, wc, ws, debug=True)
            torch.cuda.synchronize()
            check_gemm(host(ac), host(sa), host(wc), host(ws), host(y), host(acc),
                       what=f"decode m={m} k={k}")
        # the codes that fed the GEMM are the oracle's (up to the 1e-6 band)
        mirror_a = O.fwht_quant(dec["x"], dec["signs"], "f32")
        ac, sa, _ = rq.fwht_quant(dev(dec["x"]), s)
        check_codes(O.unpack_int4(host(ac)), mirror_a, "decode activations")


def test_linear_decode_fused_matches_two_launches(rq):
    """rq_linear_decode (one launch for m <= 4: the rotation as the GEMM's
    prologue) gives the same y as rq_fwht_quant followed by rq_w4a4_gemm, bit
    for bit, on the decode-linear workload; for m = 16 the codes and scales it
    hands over in the workspace are rq_fwht_quant's."""
    dec = datagen.decode_linear(0)
    s = dev(dec["signs"])
    ws = rq.linear_decode_workspace(16, 4096, torch.device("cuda"))
    for k, wt in dec["wts"].items():
        wc, wsc, _ = rq.fold_weights(dev(wt), s)
        for m in (1, 2, 4, 16):
            say(f"fused decode linear m={m} k={k}")
            x = dev(dec["x"][:m])
            for rep in range(2):  # the same workspace twice
                y = rq.linear_decode(x, s, wc, wsc, workspace=ws)
                torch.cuda.synchronize()
                y_ref = rq.w4a4_linear(x, s, wc, wsc)
                torch.cuda.synchronize()
                assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (m, k, rep)
        ac, sa, _ = rq.fwht_quant(dev(dec["x"]), s)
        torch.cuda.synchronize()
        assert torch.equal(ws[:16 * 2048].view(16, 2048), ac)
        assert torch.equal(ws[16 * 2048:16 * 2048 + 32].view(torch.float16), sa)


@pytest.mark.parametrize("m,k,d,with_signs", [(4, 5, 512, True), (3, 40, 8192, True),
                                              (2, 300, 1024, False), (1, 12300, 2048, True),
                                              (4, 14336, 4096, True), (16, 5, 512, True),
                                              (7, 300, 1024, False), (1, 5, 4096, True),
                                              (2, 300, 4096, False), (3, 40, 4096, True),
                                              (4, 1000, 4096, False)])
def test_linear_decode_fused_shapes(rq, m, k, d, with_signs):
    """One workgroup (k = 5), both weight-group widths (k = 12300, 14336 give
    two 16-row groups per workgroup), every n class, no signs, the two-launch
    route (m > 4), and n = 4096 with one 16-row group per workgroup, where 8
    or 4 wavefronts rotate each token (m = 1, 2; one wavefront for m = 3, 4);
    y against the oracle's pipeline and against the two-launch path."""
    rng = np.random.default_rng(m * 7 + k + d)
    x = (rng.standard_normal((m, d)) * np.where(rng.random(d) < 0.01, 50.0, 1.0)).astype(np.float16)
    wt = (rng.standard_normal((k, d)) * 0.02).astype(np.float32)
    signs = datagen.rademacher(rng, d) if with_signs else None
    sd = dev(signs) if with_signs else None
    say(f"fused decode linear m={m} k={k} d={d} signs={with_signs}")
    wc, wsc, _ = rq.fold_weights(dev(wt), sd)
    for sentinel in SENTINELS:
        yo = Out((m, k), torch.float16, sentinel)
        wso = Out((int(rq.load_library().rq_linear_decode_workspace_size(m, d)),), torch.uint8,
                  sentinel)
        rq.linear_decode(dev(x), sd, wc, wsc, workspace=wso.t, out=yo.t)
        check_all([yo, wso], "fused decode")
    y = yo.t
    y_ref = rq.w4a4_linear(dev(x), sd, wc, wsc)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    # the pieces against the oracle: codes up to the 1e-6 rounding band, the
    # GEMM of those codes exactly
    ac, sa, xr = rq.fwht_quant(dev(x), sd, debug=True)
    wr = rq.fold_weights(dev(wt), sd, debug=True)[2]
    torch.cuda.synchronize()
    check_rotation_result(x, signs, host(ac), host(sa), host(xr), what="fused decode activations")
    check_rotation_result(wt, signs, host(wc), host(wsc), host(wr), what="fused decode weights")
    y_o, _ = check_gemm(host(ac), host(sa), host(wc), host(wsc), host(y), None,
                        what="fused decode y")
    np.testing.assert_array_equal(host(y).view(np.uint16), y_o.view(np.uint16))


def test_tiny_linear_end_to_end(rq):
    cfg = datagen.tiny_linear(0)
    s = dev(cfg["signs"])
    wc, ws, _ = rq.fold_weights(dev(cfg["wt"]), s)
    ac, sa, _ = rq.fwht_quant(dev(cfg["x"]), s)
    y, acc = rq.w4a4_gemm(ac, sa, wc, ws, debug=True)
    torch.cuda.synchronize()
    say("tiny linear 8x256 -> 512")
    y_ref, _ = check_gemm(host(ac), host(sa), host(wc), host(ws), host(y), host(acc), what="tiny")
    # the whole pipeline against the oracle's own pipeline
    a_ref = O.fwht_quant(cfg["x"], cfg["signs"], "f32")
    w_ref = O.fold_weights(cfg["wt"], cfg["signs"], "f32")
    y_o, _ = O.w4a4_gemm(a_ref["codes"], a_ref["scales"], w_ref["codes"], w_ref["scales"])
    np.testing.assert_array_equal(host(y).view(np.uint16), y_o.view(np.uint16))


def test_prefill_gemm_full_size_sampled(rq):
    w = datagen.prefill_linear(0)
    s = dev(w["signs"])
    say("prefill: fold 28672x8192 fp32")
    wc, ws, _ = rq.fold_weights(dev(w["wt"]), s)
    ac, sa, _ = rq.fwht_quant(dev(w["x"]), s)
    say("prefill: gemm 2048x8192 -> 28672")
    m, k = ac.shape[0], wc.shape[0]
    yo, ao = Out((m, k), torch.float16), Out((m, k), torch.int32)
    rq.w4a4_gemm(ac, sa, wc, ws, debug=True, out=yo.t, acc_out=ao.t)
    check_all([yo, ao], "prefill debug")
    acc = ao.host()
    del ao
    ac_h, sa_h, wc_h, ws_h = map(host, (ac, sa, wc, ws))
    rng = np.random.default_rng(77)
    rows = np.sort(rng.choice(2048, 128, replace=False))
    cols = np.sort(rng.choice(28672, 256, replace=False))
    # every row x sampled columns, sampled rows x every column: every tile position
    check_gemm(ac_h, sa_h, wc_h, ws_h, yo.host(), acc, what="prefill cols", cols=cols)
    check_gemm(ac_h, sa_h, wc_h, ws_h, yo.host(), acc, what="prefill rows", rows=rows)
    # the launch the benchmark times (no int32 output), with both sentinels,
    # against the oracle on the same samples; then 20 repeats bit-identical
    first = None
    for rep in range(20):
        y2 = Out((m, k), torch.float16, SENTINELS[rep % 2])
        rq.w4a4_gemm(ac, sa, wc, ws, out=y2.t)
        check_all([y2], f"prefill timed {rep}")
        if rep < 2:
            yh = y2.host()
            check_gemm(ac_h, sa_h, wc_h, ws_h, yh, None, what="prefill timed cols", cols=cols)
            check_gemm(ac_h, sa_h, wc_h, ws_h, yh, None, what="prefill timed rows", rows=rows)
            assert torch.equal(y2.t.view(torch.int16), yo.t.view(torch.int16))
            first = y2.t.clone() if first is None else first
        else:
            assert torch.equal(y2.t.view(torch.int16), first.view(torch.int16)), rep
        del y2
    # the fold itself on sampled weight rows
    wrows = np.sort(rng.choice(28672, 512, replace=False))
    c_rows = wc_h[wrows]
    s_rows = ws_h[wrows]
    check_rotation_result(w["wt"][wrows], w["signs"], c_rows, s_rows, None, what="fold 28672 sampled")


def test_downproj_28672_full_size_sampled(rq):
    """The down projection of the prefill-shaped model as the benchmark runs
    it: 2048 tokens x 28672 fp16 (0.1% of channels x100) rotated with
    H_28 (x) H_1024, W^T 8192 x 28672 ~ N(0, 0.02^2) folded with the same
    signs, then the persistent prefill GEMM (d = 28672 -> k = 8192); the
    rotation on sampled rows, the GEMM on every row x sampled columns and
    sampled rows x every column, exact accumulators."""
    m, d, k = 2048, 28672, 8192
    rng = np.random.default_rng(7)
    x = datagen.activations(rng, m, d, datagen.outlier_channels(rng, d), 100.0)
    signs = datagen.rademacher(rng, d)
    say("down projection: fold 8192 x 28672 fp32")
    s = dev(signs)
    wt = datagen.gaussian(rng, (k, d), std=0.02)
    wc, ws, _ = rq.fold_weights(dev(wt), s)
    say("down projection: rotate 2048 x 28672, gemm 2048 x 28672 -> 8192")
    co, so = Out((m, d // 2), torch.uint8), Out((m,), torch.float16)
    rq.fwht_quant(dev(x), s, out=(co.t, so.t))
    yo, ao = Out((m, k), torch.float16), Out((m, k), torch.int32)
    rq.w4a4_gemm(co.t, so.t, wc, ws, debug=True, out=yo.t, acc_out=ao.t)
    y2 = Out((m, k), torch.float16, SENTINELS[1])
    rq.w4a4_gemm(co.t, so.t, wc, ws, out=y2.t)  # the launch the benchmark times
    check_all([co, so, yo, ao, y2], "down projection")
    assert torch.equal(yo.t.view(torch.int16), y2.t.view(torch.int16))
    ac, sa, wc_h, ws_h, y, acc = co.host(), so.host(), host(wc), host(ws), yo.host(), ao.host()
    rows = np.sort(rng.choice(m, 64, replace=False))
    cols = np.sort(rng.choice(k, 128, replace=False))
    check_rotation_result(x, signs, ac, sa, None, what="down projection rows", rows=rows)
    check_gemm(ac, sa, wc_h, ws_h, y, acc, what="down projection cols", cols=cols)
    check_gemm(ac, sa, wc_h, ws_h, y, acc, what="down projection rows", rows=rows)
    wrows = np.sort(rng.choice(k, 128, replace=False))
    check_rotation_result(wt[wrows], signs, wc_h[wrows], ws_h[wrows], None, what="fold 28672 sampled")


def test_kv_small_and_ragged(rq):
    rng = np.random.default_rng(3)
    for shape in [(1, 1, 1, 128), (2, 3, 5, 128), (1, 2, 97, 128)]:
        k = rng.standard_normal(shape).astype(np.float16)
        v = (rng.standard_normal(shape) * 5).astype(np.float16)
        for signs in (None, datagen.rademacher(rng, 128)):
            say(f"kv shape={shape} signs={signs is not None}")
            lead = shape[:-1]
            for sentinel in SENTINELS:
                o = [Out(lead + (64,), torch.uint8, sentinel), Out(lead, torch.float16, sentinel),
                     Out(lead + (64,), torch.uint8, sentinel), Out(lead, torch.float16, sentinel)]
                rq.kv_rotate_quant(dev(k), dev(v), None if signs is None else dev(signs),
                                   out=tuple(t.t for t in o))
                check_all(o, f"kv {shape}")
                kc, ks, vc, vs = (t.host() for t in o)
                for name, x, c, s in (("k", k, kc, ks), ("v", v, vc, vs)):
                    check_rotation_result(x.reshape(-1, 128), signs, c.reshape(-1, 64),
                                          s.reshape(-1), what=f"kv {name} {shape}")


def test_kv_full_cache_sampled(rq):
    kv = datagen.kv_cache(0)
    say("kv cache [32,8,4096,128] fp16")
    lead = (32, 8, 4096)
    o = [Out(lead + (64,), torch.uint8), Out(lead, torch.float16), Out(lead + (64,), torch.uint8),
         Out(lead, torch.float16)]
    rq.kv_rotate_quant(dev(kv["k"]), dev(kv["v"]), out=tuple(t.t for t in o))
    check_all(o, "kv full cache")
    kc, ks, vc, vs = (t.t for t in o)
    rows_total = 32 * 8 * 4096
    rng = np.random.default_rng(9)
    rows = np.concatenate([np.arange(128), np.sort(rng.choice(rows_total, 8192, replace=False)),
                           np.arange(rows_total - 128, rows_total)])
    for name, c, s in (("k", kc, ks), ("v", vc, vs)):
        x = kv[name].reshape(-1, 128)
        check_rotation_result(x, None, host(c).reshape(-1, 64), host(s).reshape(-1),
                              what=f"kv {name} sampled", rows=rows, report=REPORT)


@pytest.mark.parametrize("m", [1, 2, 4])
def test_linear_decode_fused_special_tokens(rq, m):
    """Tokens whose scale is zero, fp16-subnormal (the code clamp) or infinite
    (zero codes), at n = 4096 where several wavefronts rotate a token (m = 1,
    2) or one does (m = 4): y is the two-launch path's, bit for bit."""
    rng = np.random.default_rng(500 + m)
    d, k = 4096, 64
    signs = datagen.rademacher(rng, d)
    sd = dev(signs)
    # zero; fp16-subnormal values (a subnormal scale); 65504 times the signs
    # (every signed element 65504: the first rotated value is 65504 * 64, whose
    # scale overflows fp16); an ordinary token with outlier channels
    rows = [np.zeros(d), rng.standard_normal(d) * 1e-6, 65504.0 * signs.astype(np.float64),
            rng.standard_normal(d) * np.where(rng.random(d) < 0.01, 50.0, 1.0)]
    x = np.stack(rows[1:2] if m == 1 else rows[:m]).astype(np.float16)
    wt = (rng.standard_normal((k, d)) * 0.02).astype(np.float32)
    say(f"fused decode linear special tokens m={m}")
    wc, wsc, _ = rq.fold_weights(dev(wt), sd)
    y = rq.linear_decode(dev(x), sd, wc, wsc)
    torch.cuda.synchronize()
    y_ref = rq.w4a4_linear(dev(x), sd, wc, wsc)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    ac, sa, _ = rq.fwht_quant(dev(x), sd)
    torch.cuda.synchronize()
    sa = host(sa).view(np.uint16)
    if m == 4:
        assert sa[0] == 0 and 0 < sa[1] < 0x0400 and sa[2] == 0x7C00


def test_zz_report():
    for r in REPORT:
        say(str(r))
