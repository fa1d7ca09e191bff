"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test fixes the oracle against a closed form, an independent library
routine, brute force on tiny inputs, or a number the pages print.  A plausible
slip in the oracle (wrong butterfly sign or stride, signs applied after H
instead of before, a missing 1/sqrt(n), fp16 double rounding, ties rounded
away from zero, swapped nibbles, a transposed GEMM operand) fails at least one
of them.
"""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.linalg
from hypothesis import given, settings, strategies as st

from oracle import rq_oracle as O
from rotation_w4a4_quantization_amd import datagen


def sylvester_block(n):
    """+-1 Sylvester matrix from the block recursion [[H, H], [H, -H]]."""
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# ----------------------------------------------------------------- rotation

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_equals_explicit_sylvester_matmul(n):
    rng = np.random.default_rng(n)
    u = rng.standard_normal((5, n))
    h = sylvester_block(n).astype(np.float64)
    ref = u @ h.T  # row vector convention: y_j = sum_i H[j][i] u_i (H symmetric)
    got = O.hadamard_transform(u)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("n", [2, 16, 512, 2048])
def test_fwht_equals_scipy_hadamard(n):
    rng = np.random.default_rng(1000 + n)
    u = rng.standard_normal((3, n))
    ref = u @ scipy.linalg.hadamard(n).astype(np.float64)
    np.testing.assert_allclose(O.hadamard_transform(u), ref, rtol=0, atol=1e-10 * np.abs(ref).max())


@pytest.mark.parametrize("n", [2, 8, 64, 256, 1024])
def test_hadamard_rows_closed_form_and_orthogonality(n):
    # transforming the identity yields H itself; entries must be (-1)^popcount(i&j)
    h = O.hadamard_transform(np.eye(n, dtype=np.float64))
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    np.testing.assert_array_equal(h, np.where(pop % 2 == 0, 1.0, -1.0))
    hi = h.astype(np.int64)
    np.testing.assert_array_equal(hi @ hi.T, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("a,b", [(2, 8), (4, 16), (8, 32)])
def test_kronecker_structure(a, b):
    ha = scipy.linalg.hadamard(a)
    hb = scipy.linalg.hadamard(b)
    h = O.hadamard_transform(np.eye(a * b)).astype(np.int64)
    np.testing.assert_array_equal(h, np.kron(ha, hb))


@settings(max_examples=40, deadline=None)
@given(logn=st.integers(0, 11), seed=st.integers(0, 2**31 - 1))
def test_involution(logn, seed):
    n = 1 << logn
    u = np.random.default_rng(seed).standard_normal((2, n))
    back = O.hadamard_transform(O.hadamard_transform(u))
    np.testing.assert_allclose(back, n * u, rtol=0, atol=1e-9 * n * max(1.0, np.abs(u).max()))


@settings(max_examples=40, deadline=None)
@given(logn=st.integers(1, 12), seed=st.integers(0, 2**31 - 1))
def test_rotation_preserves_norm(logn, seed):
    n = 1 << logn
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((3, n)) * rng.uniform(0.1, 100)
    s = datagen.rademacher(rng, n)
    xr = O.rotate(x, s, "f64")
    np.testing.assert_allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


@pytest.mark.parametrize("n,i", [(256, 0), (256, 77), (4096, 598), (8192, 8191)])
def test_one_hot_spike_spreads_to_uniform_magnitude(n, i):
    rng = np.random.default_rng(n + i)
    s = datagen.rademacher(rng, n)
    m = 100.0
    x = np.zeros((1, n))
    x[0, i] = m
    xr = O.rotate(x, s, "f64")[0]
    j = np.arange(n)
    parity = np.array([bin(i & int(v)).count("1") % 2 for v in j])
    expected = s[i] * np.where(parity == 0, 1.0, -1.0) * m / math.sqrt(n)
    np.testing.assert_allclose(xr, expected, rtol=1e-14, atol=0)


def test_attenuation_factors_from_page(golden):
    g = golden["attenuation"]
    factors = []
    for d in g["d"]:
        x = np.zeros((1, d))
        x[0, 5] = 1.0
        xr = O.rotate(x, None, "f64")
        factors.append(1.0 / np.abs(xr).max())
    assert factors[0] == pytest.approx(g["factor_low"], rel=1e-12)  # sqrt(4096) = 64
    assert g["factor_high"] <= factors[1] < g["factor_high"] + 1  # sqrt(8192) = 90.51


def test_plain_rotation_equals_all_plus_signs():
    x = np.random.default_rng(3).standard_normal((4, 128))
    np.testing.assert_array_equal(O.rotate(x, None, "f64"), O.rotate(x, np.ones(128, np.int8), "f64"))


def test_signs_applied_before_hadamard():
    # with R = diag(s) H / sqrt(n), row e_i maps to s_i * H[i] / sqrt(n); the
    # other order (H diag(s)) would give H[i] * s instead.
    n = 16
    s = np.array([1, -1] * 8, dtype=np.int8)
    s[3] = -1
    e = np.zeros((1, n))
    e[0, 2] = 1.0
    h = sylvester_block(n).astype(np.float64)
    np.testing.assert_allclose(O.rotate(e, s, "f64")[0], s[2] * h[2] / 4.0, atol=1e-15)
    assert not np.allclose(O.rotate(e, s, "f64")[0], h[2] * s / 4.0)


def test_computational_invariance_tiny_linear():
    # (X R)(R^T W) = X W in fp64; the fold and the online rotation must use the same R.
    cfg = datagen.tiny_linear(0)
    x = cfg["x"].astype(np.float64)
    wt = cfg["wt"].astype(np.float64)
    xr = O.rotate(x, cfg["signs"], "f64")
    wr_t = O.rotate(wt, cfg["signs"], "f64")  # rows of W~^T = W^T R
    y_rot = xr @ wr_t.T
    y = x @ wt.T
    err = np.abs(y_rot - y).max() / np.abs(y).max()
    assert err < 1e-10
    # the fold entry point is that same row transform on W^T
    folded = O.fold_weights(cfg["wt"], cfg["signs"], "f64")
    np.testing.assert_array_equal(folded["x_rot"], wr_t)


@pytest.mark.parametrize("n", [2, 8, 32, 128, 512, 2048, 8192])
def test_inv_sqrt_constant_is_correctly_rounded(n):
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(n).sqrt()
    c = O._inv_sqrt_f32(n)
    below = np.nextafter(c, np.float32(0))
    above = np.nextafter(c, np.float32(1))
    err = abs(Decimal(float(c)) - exact)
    assert err <= abs(Decimal(float(below)) - exact)
    assert err <= abs(Decimal(float(above)) - exact)


def test_f32_mirror_exact_on_small_integers_and_close_otherwise():
    rng = np.random.default_rng(11)
    n = 1024  # 4^5: 1/sqrt(n) is a power of two
    x = rng.integers(-50, 50, size=(4, n)).astype(np.float32)
    s = datagen.rademacher(rng, n)
    np.testing.assert_array_equal(O.rotate(x, s, "f32").astype(np.float64), O.rotate(x, s, "f64"))
    xg = rng.standard_normal((8, 4096)).astype(np.float16)
    s = datagen.rademacher(rng, 4096)
    r32 = O.rotate(xg, s, "f32").astype(np.float64)
    r64 = O.rotate(xg, s, "f64")
    rel = np.abs(r32 - r64).max(axis=1) / np.abs(r64).max(axis=1)
    # ascending-stride fp32 butterflies: error <= log2(n) * 2^-24 * sqrt(n) * rms bound, far below 1e-5
    assert rel.max() < 1e-5


# ----------------------------------------------------------- fp16 rounding

def test_fp16_single_rounding_pins():
    cases = [
        (1 + 2**-11 + 2**-40, 1 + 2**-10),  # above the midpoint: up (a float32 detour would give 1.0)
        (1 + 2**-11, 1.0),                  # exact midpoint: tie to even
        (1 + 3 * 2**-11, 1 + 2**-9),        # exact midpoint: tie to even (up)
        (2**-25, 0.0),                      # half the smallest subnormal: tie to even zero
        (3 * 2**-25, 2**-23),               # 1.5 subnormal ulps: tie to even (2 ulps)
        (2**-25 + 2**-40, 2**-24),          # just above half an ulp
        (65519.99, 65504.0),
        (65520.0, np.inf),                  # midpoint to the next binade rounds to infinity
        (-2.5 * 2**-24, -2 * 2**-24),
    ]
    for v, want in cases:
        assert float(O.fp16_rne(v)) == want, (v, float(O.fp16_rne(v)), want)


# --------------------------------------------------------------- quantizer

def test_quantizer_round_half_even_table():
    # a = 7 -> scale = fp16(1.0) = 1, so v = x exactly
    row = np.array([7.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, 6.5, -6.5, -7.0, 0.49, -3.51])
    q, sc, v = O.quantize_rows(row[None, :])
    assert float(sc[0]) == 1.0
    np.testing.assert_array_equal(q[0], [7, 2, 4, -2, 0, 0, 2, 6, -6, -7, 0, -4])
    np.testing.assert_array_equal(v[0], row)


def test_quantizer_scale_is_single_rounded_absmax_over_7():
    # a/7 exactly on an fp16 midpoint -> tie to even
    a = 7 * (1 + 2**-11)
    q, sc, _ = O.quantize_rows(np.array([[a, -1.0, 0.0, 2.0]]))
    assert float(sc[0]) == 1.0
    assert q[0, 0] == 7  # v = 7.0034 -> 7, never 8
    q, sc, _ = O.quantize_rows(np.array([[-a * (1 + 2**-30), 1.0]]))
    assert float(sc[0]) == 1 + 2**-10
    assert q[0, 0] == -7


def test_quantizer_zero_and_underflow_rows():
    q, sc, v = O.quantize_rows(np.zeros((2, 8)))
    assert not q.any() and not sc.astype(np.float64).any()
    tiny = np.array([[0.4 * 7 * 2**-24, -0.1 * 2**-24, 0.0, 0.0]])  # a/7 < 2^-25 -> scale 0
    q, sc, v = O.quantize_rows(tiny)
    assert float(sc[0]) == 0.0 and not q.any()


def test_quantizer_clamps_when_scale_is_subnormal():
    a = 7 * 1.4 * 2**-24  # a/7 = 1.4 subnormal ulps -> scale = 2^-24, v up to 9.8
    q, sc, v = O.quantize_rows(np.array([[a, -a, a / 2, 0.0]]))
    assert float(sc[0]) == 2**-24
    np.testing.assert_array_equal(q[0], [7, -8, 5, 0])


def test_one_hot_row_codes_are_plus_minus_seven():
    n = 256
    s = datagen.rademacher(np.random.default_rng(5), n)
    x = np.zeros((1, n))
    x[0, 17] = -3.25
    r = O.fwht_quant(x, s, "f64")
    assert set(np.abs(r["q"][0]).tolist()) == {7}


def test_zero_row_codes_are_zero():
    r = O.fwht_quant(np.zeros((3, 64), np.float16), None, "f64")
    assert not r["codes"].any()
    assert not r["scales"].astype(np.float64).any()


@settings(max_examples=30, deadline=None)
@given(logn=st.integers(1, 10), seed=st.integers(0, 2**31 - 1), mag=st.floats(1e-3, 1e4))
def test_codes_within_range_and_reconstruct(logn, seed, mag):
    n = 1 << logn
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, n)) * mag
    r = O.fwht_quant(x, datagen.rademacher(rng, n), "f64")
    assert r["q"].min() >= -7 and r["q"].max() <= 7  # normal fp16 scales never reach -8
    deq = O.dequantize(r["q"], r["scales"])
    step = r["scales"].astype(np.float64)[:, None]
    assert np.all(np.abs(deq - r["x_rot"]) <= 0.5 * step * (1 + 1e-12) + 1e-300)


# ------------------------------------------------------------------ packing

def test_nibble_order_and_twos_complement():
    assert O.pack_int4(np.array([[1, -1]]))[0, 0] == 0xF1
    assert O.pack_int4(np.array([[-8, 7]]))[0, 0] == 0x78
    assert O.pack_int4(np.array([[0, -8, 5, 3]])).tolist() == [[0x80, 0x35]]
    allq = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)])
    packed = O.pack_int4(allq)
    assert sorted(packed[:, 0].tolist()) == list(range(256))
    np.testing.assert_array_equal(O.unpack_int4(packed), allq)


# --------------------------------------------------------------------- GEMM

def test_gemm_brute_force_tiny():
    rng = np.random.default_rng(21)
    m, k, d = 3, 5, 8
    ac = datagen.random_codes(rng, m, d)
    wc = datagen.random_codes(rng, k, d)
    sa = datagen.random_scales(rng, m)
    sw = datagen.random_scales(rng, k)
    y, acc = O.w4a4_gemm(ac, sa, wc, sw)

    def nib(byte, hi):
        v = (int(byte) >> (4 if hi else 0)) & 0xF
        return v - 16 if v >= 8 else v

    for i in range(m):
        for j in range(k):
            ref = 0
            for t in range(d):
                ref += nib(ac[i, t // 2], t % 2) * nib(wc[j, t // 2], t % 2)
            assert acc[i, j] == ref
            want = np.float16(float(ref) * float(sa[i]) * float(sw[j]))
            assert y[i, j] == want or (np.isnan(want) and np.isnan(y[i, j]))


def test_gemm_closed_forms():
    d = 8192
    sevens = O.pack_int4(np.full((2, d), 7))
    negs = O.pack_int4(np.full((3, d), -8))
    ones = np.ones(3, np.float16)
    _, acc = O.w4a4_gemm(sevens, ones[:2], sevens, ones[:2])
    assert (acc == 49 * d).all()
    _, acc = O.w4a4_gemm(negs, ones, negs, ones)
    assert (acc == 64 * d).all() and acc.max() == 524288
    _, acc = O.w4a4_gemm(sevens, ones[:2], negs, ones)
    assert (acc == -56 * d).all()
    # unit scales: y = fp16(acc)
    rng = np.random.default_rng(4)
    ac = datagen.random_codes(rng, 4, 64)
    wc = datagen.random_codes(rng, 6, 64)
    y, acc = O.w4a4_gemm(ac, np.ones(4, np.float16), wc, np.ones(6, np.float16))
    np.testing.assert_array_equal(y, acc.astype(np.float16))


def test_gemm_is_not_transposed():
    # rows of the output follow activation rows, columns follow weight rows
    a = O.pack_int4(np.array([[1] * 64, [2] * 64]))
    w = O.pack_int4(np.array([[1] * 64, [0] * 64, [-1] * 64]))
    _, acc = O.w4a4_gemm(a, np.ones(2, np.float16), w, np.ones(3, np.float16))
    np.testing.assert_array_equal(acc, [[64, 0, -64], [128, 0, -128]])


def test_w4a4_output_tracks_float_linear_and_rotation_helps():
    # accuracy of the method itself is not a parity target; this checks the
    # property the pages argue for: rotated W4A4 error << unrotated error
    cfg = datagen.tiny_linear(0)
    x = cfg["x"].astype(np.float64)
    wt = cfg["wt"].astype(np.float64)
    y = x @ wt.T

    def w4a4(signs_rot):
        if signs_rot is None:
            a = O.quantize_rows(x)
            w = O.quantize_rows(wt)
            ac, sa, wc, sw = O.pack_int4(a[0]), a[1], O.pack_int4(w[0]), w[1]
        else:
            a = O.fwht_quant(x, signs_rot, "f64")
            w = O.fold_weights(wt, signs_rot, "f64")
            ac, sa, wc, sw = a["codes"], a["scales"], w["codes"], w["scales"]
        yq, _ = O.w4a4_gemm(ac, sa, wc, sw)
        return np.linalg.norm(yq.astype(np.float64) - y) / np.linalg.norm(y)

    e_rot = w4a4(cfg["signs"])
    e_plain = w4a4(None)
    assert e_rot < 0.2
    assert e_rot < 0.8 * e_plain  # weight INT4 error is common to both; activation error differs


# ------------------------------------------------------- worked examples

def test_outlier_collapses_ordinary_values_into_few_bins(golden):
    g = golden["outlier_example"]
    rng = np.random.default_rng(7)
    n = 4096
    lo, hi = g["ordinary_range"]
    x = rng.uniform(lo, hi, size=(1, n))
    x[0, 7] = g["outlier_value"]
    q, _, _ = O.quantize_rows(x)
    ordinary = np.delete(q[0], 7)
    assert len(np.unique(ordinary)) <= golden["bins_for_ordinary_values"]["max_bins"]
    assert 2 ** 4 == g["int4_levels"]
    r = O.fwht_quant(x, datagen.rademacher(rng, n), "f64")
    assert len(np.unique(r["q"][0])) >= 12
    err_plain = np.linalg.norm(O.dequantize(q, O.quantize_rows(x)[1]) - x)
    err_rot = np.linalg.norm(O.dequantize(r["q"], r["scales"]) - r["x_rot"])
    assert err_rot < 0.3 * err_plain


def test_kv_memory_formula_and_saving(golden):
    # Memory = 2 * layers * heads * head_dim * seq * batch * bytes_per_element
    def kv_bytes(layers, heads, head_dim, seq, batch, bits):
        return 2 * layers * heads * head_dim * seq * batch * bits / 8

    b16 = kv_bytes(1, 8, 128, 4096, 32, 16)
    b4 = kv_bytes(1, 8, 128, 4096, 32, 4)
    assert 1 - b4 / b16 == golden["kv_memory"]["reduction_16_to_4_bit"]
    # this layout: 4-bit codes plus one fp16 scale per 128-element vector
    ours = 2 * (32 * 8 * 4096) * (128 // 2 + 2)
    assert ours == 2 * (134217728 // 2 + 2 * 32 * 8 * 4096)
    assert ours / b16 == pytest.approx(4.125 / 16)
    assert 1 - ours / b16 == pytest.approx(0.7421875)


def test_weight_bytes_quartered(golden):
    d, k = 4096, 4096
    fp16_bytes = 2 * d * k
    int4_bytes = d * k // 2
    assert int4_bytes / fp16_bytes == golden["weight_bytes"]["ratio_4_over_16"]


def test_datagen_outlier_fraction_matches_page(golden):
    g = golden["outlier_statistics"]
    for d, want in [(4096, 4), (8192, 8)]:
        ch = datagen.outlier_channels(datagen.rng_for(1, 0), d, g["channel_fraction"])
        assert len(ch) == want and len(set(ch.tolist())) == want


def test_kv_oracle_is_rowwise_fwht_quant():
    rng = np.random.default_rng(9)
    k = rng.standard_normal((2, 3, 5, 128)).astype(np.float16)
    v = rng.standard_normal((2, 3, 5, 128)).astype(np.float16)
    out = O.kv_rotate_quant(k, v)
    flat = O.fwht_quant(k.reshape(-1, 128), None, "f64")
    np.testing.assert_array_equal(out["k_codes"].reshape(-1, 64), flat["codes"])
    assert out["k_codes"].shape == (2, 3, 5, 64) and out["v_scales"].shape == (2, 3, 5)


# ---------------------------------------------------------------------------
# Non-power-of-two rotation length n = 28 * 2^k (H_28 (x) H_(n/28))

def test_paley_28_is_a_symmetric_hadamard_matrix():
    h = O.paley_hadamard_28().astype(np.int64)
    assert h.shape == (28, 28)
    assert set(np.unique(h).tolist()) == {-1, 1}
    np.testing.assert_array_equal(h @ h.T, 28 * np.eye(28, dtype=np.int64))
    np.testing.assert_array_equal(h, h.T)


def test_paley_28_conference_matrix_and_residues():
    # textbook: the quadratic residues modulo 13 are {1, 3, 4, 9, 10, 12}
    assert sorted({(a * a) % 13 for a in range(1, 13)}) == [1, 3, 4, 9, 10, 12]
    c = O._paley_conference_14()
    assert (np.diag(c) == 0).all()
    assert (c[0, 1:] == 1).all() and (c[1:, 0] == 1).all()
    # C[1 + a][1 + b] = chi(a - b), chi = +1 on the residues, -1 off them
    res = {1, 3, 4, 9, 10, 12}
    for a in range(13):
        for b in range(13):
            if a != b:
                assert c[1 + a, 1 + b] == (1 if (a - b) % 13 in res else -1)
    np.testing.assert_array_equal(c @ c.T, 13 * np.eye(14, dtype=np.int64))


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_kron28_transform_equals_dense_kronecker_product(p):
    import scipy.linalg
    rng = np.random.default_rng(p)
    x = rng.standard_normal((3, 28 * p))
    dense = np.kron(O.paley_hadamard_28().astype(np.float64), scipy.linalg.hadamard(p).astype(np.float64))
    np.testing.assert_allclose(O.kron28_transform(x, "f64"), x @ dense.T, rtol=0, atol=1e-12)
    # the structured float32 order stays within float32 rounding of the truth
    y32 = O.kron28_transform(x.astype(np.float32), "f32").astype(np.float64)
    assert np.abs(y32 - x.astype(np.float32).astype(np.float64) @ dense.T).max() <= 1e-5 * 28 * p


def test_kron28_f32_integer_inputs_are_exact():
    # small integers: every partial sum is an integer below 2^24, so the
    # structured float32 order must equal the exact product
    rng = np.random.default_rng(3)
    x = rng.integers(-50, 50, size=(4, 28 * 16))
    exact = O.kron28_transform(x.astype(np.float64), "f64")
    np.testing.assert_array_equal(O.kron28_transform(x.astype(np.float32), "f32").astype(np.float64), exact)


@pytest.mark.parametrize("n", [28, 112, 448])
def test_rotation_28_orthogonal_and_invariant(n):
    rng = np.random.default_rng(n)
    s = datagen.rademacher(rng, n)
    r = O.rotate(np.eye(n), s, "f64")          # row i of R = e_i R
    np.testing.assert_allclose(r @ r.T, np.eye(n), atol=1e-12)
    x = rng.standard_normal((5, n))
    w = rng.standard_normal((n, 7))
    xr = O.rotate(x, s, "f64")
    wt_r = O.rotate(w.T, s, "f64")             # rows of W^T R, i.e. (R^T W)^T
    np.testing.assert_allclose(xr @ wt_r.T, x @ w, rtol=0, atol=1e-10)
    np.testing.assert_allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)


@pytest.mark.parametrize("i", [0, 511, 7000, 14335])
def test_rotation_14336_one_hot_spike(i):
    n = 28 * 512
    x = np.zeros((1, n))
    x[0, i] = 3.0
    y = O.rotate(x, None, "f64")
    np.testing.assert_allclose(np.abs(y), 3.0 / np.sqrt(n), rtol=1e-14)


def test_fwht_quant_14336_codes_in_range():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 14336)).astype(np.float16)
    r = O.fwht_quant(x, datagen.rademacher(rng, 14336), "f32")
    assert r["codes"].shape == (2, 7168) and r["q"].min() >= -8 and r["q"].max() <= 7
    assert (np.abs(r["q"]).max(axis=1) == 7).all()


# ---------------------------------------------------------------------------
# W4A8 variant: INT8 per-token activations

def test_int8_quantizer_rounding_table_and_range():
    # scale = 1 exactly: max |x| = 127 -> fp16_rne(127/127) = 1
    xt = np.array([[127.0, -126.5, -125.5, 0.5, 1.5, -0.5, 2.4999, 3.5000001, -127.0]])
    q, s, v = O.quantize_rows_int8(xt)
    assert s[0] == np.float16(1.0)
    # round half to even: -126.5 -> -126, -125.5 -> -126, 0.5 -> 0, 1.5 -> 2, -0.5 -> 0
    np.testing.assert_array_equal(q[0], [127, -126, -126, 0, 2, 0, 2, 4, -127])


def test_int8_one_hot_and_zero_rows():
    n = 512
    x = np.zeros((2, n))
    x[0, 9] = 5.0
    r = O.fwht_quant8(x, None, "f64")
    # one-hot -> every rotated element is +-5/sqrt(n): all codes +-127
    assert (np.abs(r["q"][0]) == 127).all()
    assert r["scales"][1] == 0 and (r["q"][1] == 0).all()


def test_int8_scale_single_rounding_and_clamp():
    # a/127 just above an fp16 midpoint rounds up; the clamp keeps +-127 bounds
    rng = np.random.default_rng(4)
    xt = rng.standard_normal((64, 256)) * 3
    q, s, v = O.quantize_rows_int8(xt)
    a = np.abs(xt).max(axis=1)
    np.testing.assert_array_equal(s, (a / 127.0).astype(np.float16))
    assert q.min() >= -128 and q.max() <= 127
    # |x/scale| <= 127 * (1 + 2^-11) < 127.5, so -128 never appears for normal scales
    assert q.min() >= -127
    rec = q.astype(np.float64) * s.astype(np.float64)[:, None]
    assert np.all(np.abs(rec - xt) <= 0.5 * s.astype(np.float64)[:, None] + 1e-12)


def test_w4a8_gemm_brute_force_and_closed_form():
    rng = np.random.default_rng(6)
    qa = rng.integers(-128, 128, size=(3, 64)).astype(np.int8)
    qw = rng.integers(-8, 8, size=(5, 64)).astype(np.int8)
    sa = np.array([0.5, 1.0, 2.0], np.float16)
    sw = np.array([1.0, 0.25, 0.5, 1.0, 2.0], np.float16)
    y, acc = O.w4a8_gemm(qa, sa, O.pack_int4(qw), sw)
    for i in range(3):
        for j in range(5):
            want = sum(int(qa[i, t]) * int(qw[j, t]) for t in range(64))
            assert acc[i, j] == want
            assert y[i, j] == np.float16(want * float(sa[i]) * float(sw[j]))
    # extremes: -128 * -8 over d = 8192 = 8388608 (exact)
    d = 8192
    y2, acc2 = O.w4a8_gemm(np.full((1, d), -128, np.int8), np.ones(1, np.float16),
                           O.pack_int4(np.full((1, d), -8)), np.ones(1, np.float16))
    assert acc2[0, 0] == 1024 * d


def test_w4a8_tracks_float_linear_better_than_w4a4():
    rng = np.random.default_rng(12)
    d, k, m = 1024, 64, 16
    x = rng.standard_normal((m, d))
    x[:, 5] *= 100
    w = rng.standard_normal((d, k)) * 0.02
    s = datagen.rademacher(rng, d)
    ref = x @ w
    wq = O.fold_weights(w.T, s, "f64")
    a8 = O.fwht_quant8(x, s, "f64")
    a4 = O.fwht_quant(x, s, "f64")
    y8, _ = O.w4a8_gemm(a8["codes"], a8["scales"], wq["codes"], wq["scales"])
    y4, _ = O.w4a4_gemm(a4["codes"], a4["scales"], wq["codes"], wq["scales"])
    e8 = np.abs(y8.astype(np.float64) - ref).mean()
    e4 = np.abs(y4.astype(np.float64) - ref).mean()
    assert e8 < e4


# ------------------------------------------------- asymmetric INT4 (f4)
# The pages give only the step, Delta = (max - min) / (2^b - 1) ([RQ] "The
# Activation Outlier Bottleneck in Low-Bit Serving"); the zero point is the
# usual integer one, with the range widened to contain 0.

def _fp16_nearest(fr):
    """Nearest binary16 value to the rational fr >= 0 (ties to even), by
    search over neighbouring fp16 values: independent of numpy's cast."""
    from fractions import Fraction
    x = float(fr)
    cand = np.float16(x)
    best = None
    for c in {cand, np.nextafter(cand, np.float16(np.inf)), np.nextafter(cand, np.float16(0))}:
        if not np.isfinite(c):
            continue
        dist = abs(Fraction(float(c)) - fr)
        key = (dist, int(np.array(c).view(np.uint16)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _asym_brute(row):
    """Asymmetric quantiser with exact rational arithmetic (Python Fraction,
    round() on a Fraction is round-half-even)."""
    from fractions import Fraction
    xs = [Fraction(float(v)) for v in row]
    hi = max(max(xs), Fraction(0))
    lo = min(min(xs), Fraction(0))
    scale = _fp16_nearest((hi - lo) / 15)
    s = Fraction(float(scale))
    if s == 0:
        return [0] * len(xs), scale, 0
    z = min(max(round(-lo / s), 0), 15)
    q = [min(max(round(x / s) + z, 0), 15) for x in xs]
    return q, scale, z


def test_asym_worked_example():
    # [-1, 0, 2, 3]: r = 4, 4/15 -> fp16 1092 * 2^-12 = 0.2666015625;
    # z = rne(1 / 0.26660...) = rne(3.7509) = 4; 2 / Delta = 7.5018 -> 8 -> 12;
    # 3 / Delta = 11.2527 -> 11 -> 15; -1 / Delta = -3.7509 -> -4 -> 0.
    q, s, z, _, _ = O.quantize_rows_asym(np.array([[-1.0, 0.0, 2.0, 3.0]]))
    assert float(s[0]) == 1092 * 2.0 ** -12
    assert int(z[0]) == 4
    assert q[0].tolist() == [0, 4, 12, 15]


def test_asym_brute_force_rational():
    rng = np.random.default_rng(41)
    for trial in range(60):
        n = int(rng.integers(2, 40))
        row = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        if trial % 5 == 0:
            row = np.abs(row)            # one-sided rows: lo = 0, z = 0
        if trial % 7 == 0:
            row = -np.abs(row)           # hi = 0, z = 15
        q, s, z, _, _ = O.quantize_rows_asym(row.astype(np.float64)[None, :])
        qb, sb, zb = _asym_brute(row)
        assert np.float16(s[0]).view(np.uint16) == np.float16(sb).view(np.uint16), trial
        assert int(z[0]) == zb and q[0].tolist() == qb, trial


def test_asym_reduces_to_symmetric_on_a_matched_range():
    # With min = -8t and max = 7t (t a power of two) the asymmetric step is
    # 15t / 15 = t, the same as the symmetric scale 7t / 7, the zero point
    # is 8, and the codes are the symmetric codes shifted by 8.
    rng = np.random.default_rng(42)
    t = 2.0 ** -5
    x = rng.uniform(-7 * t, 7 * t, (6, 64))  # interior values within the symmetric range
    x[:, 0], x[:, 1] = -8 * t, 7 * t
    qa, sa, za, _, _ = O.quantize_rows_asym(x)
    qs, ss, _ = O.quantize_rows(np.where(x == -8 * t, -7 * t, x))  # symmetric max must be 7t
    assert (sa.astype(np.float64) == t).all() and (ss.astype(np.float64) == t).all()
    assert (za == 8).all()
    inner = np.ones_like(x, bool)
    inner[:, 0] = False
    assert np.array_equal(qa.astype(np.int16)[inner] - 8, qs.astype(np.int16)[inner])
    assert (qa[:, 0] == 0).all()


def test_asym_invariants_zero_and_constant_rows():
    x = np.zeros((4, 16))
    x[1] = 3.0
    x[2] = -3.0
    x[3, 5] = 1.0
    q, s, z, _, _ = O.quantize_rows_asym(x)
    assert float(s[0]) == 0 and z[0] == 0 and not q[0].any()
    assert z[1] == 0 and (q[1] == 15).all()
    assert z[2] == 15 and (q[2] == 0).all()
    assert z[3] == 0 and q[3, 5] == 15 and (np.delete(q[3], 5) == 0).all()
    rng = np.random.default_rng(43)
    xr = rng.standard_normal((50, 256)) * rng.uniform(0.01, 100, (50, 1))
    q, s, z, _, _ = O.quantize_rows_asym(xr)
    s64 = s.astype(np.float64)[:, None]
    deq = s64 * (q.astype(np.float64) - z.astype(np.float64)[:, None])
    assert np.all(np.abs(deq - xr) <= 0.51 * s64)
    assert np.all(q[np.arange(50), np.argmin(xr, axis=1)] == 0)
    assert q.max() <= 15


def test_asym_fwht_quant_composition_and_packing():
    rng = np.random.default_rng(44)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    signs = datagen.rademacher(rng, 256)
    r = O.fwht_quant_asym(x, signs, "f32")
    q, s, z, _, _ = O.quantize_rows_asym(O.rotate(x, signs, "f32"))
    assert np.array_equal(r["q"], q) and np.array_equal(r["zeros"], z)
    assert np.array_equal(O.unpack_uint4(r["codes"]), q)
    # packing: code 2i in the low nibble of byte i
    assert O._pack_uint4(np.array([[1, 2, 3, 15]])).tolist() == [[0x21, 0xF3]]


def test_asym_gemm_brute_force():
    rng = np.random.default_rng(45)
    m, k, d = 3, 4, 64
    qa = rng.integers(0, 16, (m, d)).astype(np.uint8)
    za = rng.integers(0, 16, m).astype(np.uint8)
    qw = rng.integers(-8, 8, (k, d))
    sa = datagen.random_scales(rng, m)
    sw = datagen.random_scales(rng, k)
    y, acc = O.w4a4_gemm_asym(O._pack_uint4(qa), sa, za, O.pack_int4(qw), sw)
    for i in range(m):
        for j in range(k):
            want = sum((int(qa[i, t]) - int(za[i])) * int(qw[j, t]) for t in range(d))
            assert acc[i, j] == want
    # the identity the GPU epilogue uses: acc = sum qa qw - za * sum qw
    assert np.array_equal(acc, qa.astype(np.int64) @ qw.T - za[:, None].astype(np.int64) * qw.sum(1)[None, :])
    # closed form: qa = 15, za = 0, qw = 7 -> 105 d
    y2, acc2 = O.w4a4_gemm_asym(O._pack_uint4(np.full((1, d), 15)), np.ones(1, np.float16),
                                np.zeros(1, np.uint8), O.pack_int4(np.full((1, d), 7)),
                                np.ones(1, np.float16))
    assert acc2[0, 0] == 105 * d and float(y2[0, 0]) == 105 * d


def test_asym_beats_symmetric_on_one_sided_rows():
    # a one-sided distribution uses all 16 asymmetric levels but only 8
    # symmetric ones, so the asymmetric error is smaller
    rng = np.random.default_rng(46)
    x = np.abs(rng.standard_normal((64, 512)))
    qa, sa, za, _, _ = O.quantize_rows_asym(x)
    qs, ss, _ = O.quantize_rows(x)
    ea = np.abs(sa.astype(np.float64)[:, None] * (qa.astype(np.float64) - za[:, None]) - x).mean()
    es = np.abs(ss.astype(np.float64)[:, None] * qs - x).mean()
    assert ea < 0.6 * es


# ---------------------------------------------- per-group weight scales (f4)

def test_groups_worked_example_and_rowwise_equivalence():
    # group 2 on [1, -2, 0.5, 0.25]: scales fp16(2/7), fp16(0.5/7)
    q, s, _ = O.quantize_groups(np.array([[1.0, -2.0, 0.5, 0.25]]), group=2)
    from fractions import Fraction
    s0, s1 = _fp16_nearest(Fraction(2, 7)), _fp16_nearest(Fraction(1, 14))
    assert s[0].tolist() == [float(s0), float(s1)]
    want = [round(Fraction(1.0) / Fraction(float(s0))), round(Fraction(-2.0) / Fraction(float(s0))),
            round(Fraction(0.5) / Fraction(float(s1))), round(Fraction(0.25) / Fraction(float(s1)))]
    assert q[0].tolist() == [max(-8, min(7, v)) for v in want]
    rng = np.random.default_rng(47)
    x = rng.standard_normal((5, 512))
    qg, sg, _ = O.quantize_groups(x, 128)
    for g in range(4):
        qr, sr, _ = O.quantize_rows(x[:, 128 * g:128 * (g + 1)])
        assert np.array_equal(qg[:, 128 * g:128 * (g + 1)], qr)
        assert np.array_equal(sg[:, g].view(np.uint16), sr.view(np.uint16))


def test_grouped_gemm_brute_force_and_per_channel_case():
    from fractions import Fraction
    rng = np.random.default_rng(48)
    m, k, d, g = 2, 3, 256, 128
    qa = rng.integers(-8, 8, (m, d))
    qw = rng.integers(-8, 8, (k, d))
    sa = datagen.random_scales(rng, m)
    sw = datagen.random_scales(rng, k * 2).reshape(k, 2)
    y, acc = O.w4a4_gemm_grouped(O.pack_int4(qa), sa, O.pack_int4(qw), sw, g)
    for i in range(m):
        for j in range(k):
            tot = Fraction(0)
            for gi in range(2):
                a = sum(int(qa[i, t]) * int(qw[j, t]) for t in range(gi * g, (gi + 1) * g))
                assert acc[i, j, gi] == a
                tot += Fraction(float(sw[j, gi])) * a
            ref = float(Fraction(float(sa[i])) * tot)
            assert abs(float(y[i, j]) - ref) <= 2.0 ** -11 * abs(ref) + 2.0 ** -24
    # equal group scales reduce to the per-channel GEMM
    sw1 = datagen.random_scales(rng, k)
    yg, _ = O.w4a4_gemm_grouped(O.pack_int4(qa), sa, O.pack_int4(qw), np.repeat(sw1[:, None], 2, 1), g)
    yc, _ = O.w4a4_gemm(O.pack_int4(qa), sa, O.pack_int4(qw), sw1)
    assert np.array_equal(yg.view(np.uint16), yc.view(np.uint16))


def test_groups_cut_weight_error_when_group_ranges_differ():
    rng = np.random.default_rng(49)
    w = rng.standard_normal((32, 1024)) * np.repeat(10.0 ** rng.uniform(-2, 0, (32, 8)), 128, axis=1)
    qg, sg, _ = O.quantize_groups(w, 128)
    qc, sc, _ = O.quantize_rows(w)
    eg = np.abs(np.repeat(sg.astype(np.float64), 128, axis=1) * qg - w).mean()
    ec = np.abs(sc.astype(np.float64)[:, None] * qc - w).mean()
    assert eg < 0.5 * ec


# ------------------------------------ attention over the 4-bit cache (f3)

def _attn_loops(q, k, v, lengths, sm):
    """Decode attention by explicit Python loops (tiny sizes)."""
    B, Hq, D = q.shape
    H, S = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = S if lengths is None else lengths[b]
        for j in range(Hq):
            h = j // (Hq // H)
            if L == 0:
                continue
            sc = [sum(q[b, j, i] * k[b, h, t, i] for i in range(D)) * sm for t in range(L)]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            tot = sum(e)
            for i in range(D):
                out[b, j, i] = sum(e[t] * v[b, h, t, i] for t in range(L)) / tot
    return out


def test_inverse_rotate_undoes_rotate():
    rng = np.random.default_rng(50)
    for n in (4, 128):
        x = rng.standard_normal((3, n))
        signs = datagen.rademacher(rng, n)
        for s in (signs, None):
            np.testing.assert_allclose(O.inverse_rotate(O.rotate(x, s, "f64"), s), x, atol=1e-13)
        # and against the explicit matrix: R = diag(s) H / sqrt(n), y R^T
        h = sylvester_block(n).astype(np.float64)
        r = np.diag(signs.astype(np.float64)) @ h / math.sqrt(n)
        y = rng.standard_normal((2, n))
        np.testing.assert_allclose(O.inverse_rotate(y, signs), y @ r.T, atol=1e-13)


def test_decode_attention_brute_force_gqa_and_lengths():
    rng = np.random.default_rng(51)
    B, H, G, S, D = 2, 2, 3, 5, 4
    q = rng.standard_normal((B, H * G, D))
    k = rng.standard_normal((B, H, S, D))
    v = rng.standard_normal((B, H, S, D))
    lengths = [3, 0]
    got = O.decode_attention(q, k, v, lengths, 0.7)
    np.testing.assert_allclose(got, _attn_loops(q, k, v, lengths, 0.7), atol=1e-13)
    np.testing.assert_allclose(O.decode_attention(q, k, v, None),
                               _attn_loops(q, k, v, None, 1 / math.sqrt(D)), atol=1e-13)
    # a single position returns its value row; a zero query averages the values
    one = O.decode_attention(q, k[:, :, :1], v[:, :, :1])
    np.testing.assert_allclose(one, np.repeat(v[:, :, 0], G, axis=1), atol=1e-14)
    avg = O.decode_attention(np.zeros_like(q), k, v)
    np.testing.assert_allclose(avg, np.repeat(v.mean(axis=2), G, axis=1), atol=1e-14)


def test_decode_attention_int4_is_exact_on_grid_representable_caches():
    # Build caches whose rotated rows lie exactly on the INT4 grid
    # (k~ = codes * scale), set K = K~ R^T; then the INT4 path (dequantise in
    # the rotated basis, rotate q, rotate the output back) must equal plain
    # attention on K, V: rotation invariance, the GQA head mapping and the
    # inverse rotation all enter.
    rng = np.random.default_rng(52)
    B, H, G, S, D = 2, 2, 2, 6, 128
    signs = datagen.rademacher(rng, D)
    caches = {}
    for name in ("k", "v"):
        qc = rng.integers(-8, 8, (B, H, S, D))
        sc = rng.uniform(0.01, 0.2, (B, H, S)).astype(np.float16)
        caches[name] = (O.pack_int4(qc), sc, O.inverse_rotate(O.dequantize(qc, sc), signs))
    q = rng.standard_normal((B, H * G, D))
    lengths = [6, 4]
    r = O.decode_attention_int4(q, caches["k"][0], caches["k"][1], caches["v"][0], caches["v"][1],
                                signs, lengths)
    ref = O.decode_attention(q, caches["k"][2], caches["v"][2], lengths)
    np.testing.assert_allclose(r["o"], ref, atol=1e-11)


def test_rotated_int4_cache_attention_beats_unrotated():
    # Outlier channels in K and V: the rotated 4-bit cache keeps attention
    # closer to full precision than a 4-bit cache of the raw rows.
    rng = np.random.default_rng(53)
    kv = datagen.kv_cache(0, batch=1, heads=2, seq=256)
    k, v = kv["k"].astype(np.float64), kv["v"].astype(np.float64)
    q = rng.standard_normal((1, 8, 128))
    ref = O.decode_attention(q, k, v)
    r = O.kv_rotate_quant(kv["k"], kv["v"], None)
    rot = O.decode_attention_int4(q, r["k_codes"], r["k_scales"], r["v_codes"], r["v_scales"], None)["o"]
    kq, ks, _ = O.quantize_rows(k)
    vq, vs, _ = O.quantize_rows(v)
    raw = O.decode_attention(q, O.dequantize(kq, ks), O.dequantize(vq, vs))
    e_rot = np.linalg.norm(rot - ref) / np.linalg.norm(ref)
    e_raw = np.linalg.norm(raw - ref) / np.linalg.norm(ref)
    assert e_rot < 0.5 * e_raw, (e_rot, e_raw)


# ---------------------------------------------------------------- F6 layout
# OCP Microscaling Formats (MX) v1.0, the FP6 E3M2 element format: exponent
# bias 3, no inf or NaN; largest normal +-28.0 (0b0_111_11), smallest normal
# +-0.25, largest subnormal +-0.1875, smallest subnormal +-0.0625.
def test_e3m2_values_match_the_format_definition():
    assert O.e3m2_value(0b011111) == 28.0 and O.e3m2_value(0b111111) == -28.0
    assert O.e3m2_value(0b000100) == 0.25
    assert O.e3m2_value(0b000011) == 0.1875
    assert O.e3m2_value(0b000001) == 0.0625
    assert O.e3m2_value(0b001100) == 1.0 and O.e3m2_value(0b101100) == -1.0
    assert O.e3m2_value(0) == 0.0
    values = sorted(O.e3m2_value(c) for c in range(64))
    assert len(set(values)) == 63  # +0 and -0 compare equal; every other value once


def test_every_int4_code_is_an_e3m2_value():
    codes = {q: O.e3m2_code(q) for q in range(-8, 9)}
    assert len(set(codes.values())) == 17
    for q, c in codes.items():
        assert O.e3m2_value(c) == q
    for q in (9, 11, 13, 15, -9):  # 2 mantissa bits: 8, 10, 12, 14 only between 8 and 16
        with pytest.raises(ValueError):
            O.e3m2_code(q)


def test_pack_f6_read_back_bit_by_bit():
    # every code read back through the layout as it is described, with Python
    # integers (not the packing's bit arrays), is the INT4 code itself
    rng = np.random.default_rng(61)
    rows, d = 5, 384
    q = rng.integers(-8, 8, (rows, d))
    out = O.pack_f6(O.pack_int4(q))
    assert out.shape == (d // 128, rows, 96) and out.dtype == np.uint8
    for r in range(rows):
        for i in range(d):
            c, b, j = i // 128, (i % 128) // 32, i % 32
            grp = out[c, r]
            tail = 64 + 16 * (b % 2) + 8 * (b // 2)
            word = int.from_bytes(bytes(grp[16 * b:16 * b + 16]) + bytes(grp[tail:tail + 8]), "little")
            assert O.e3m2_value((word >> (6 * j)) & 63) == q[r, i], (r, i)
    # the 4 heads and 4 tails tile the 96 bytes of a group exactly once
    cover = np.zeros(96, int)
    for b in range(4):
        cover[16 * b:16 * b + 16] += 1
        t = 64 + 16 * (b % 2) + 8 * (b // 2)
        cover[t:t + 8] += 1
    assert (cover == 1).all()
