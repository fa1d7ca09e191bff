"""Comparison rules between the HIP path and the CPU oracle.

Tolerances (fixed by the rotated-quantisation contract this project builds to):
  * rotated rows (fp32 debug output): bit-identical to the oracle's fp32
    mirror (same ascending butterfly order), and within 1e-5 of the row's
    max |x~| against the fp64 oracle;
  * scales: bit-identical to the mirror's (both are fp16_rne(a/7) of the same
    fp32 a, rounded once);
  * INT4 codes: the INT4 decision is compared in the kernel's precision (fp32
    rotated values, the mirror).  Codes must be equal except where the
    mirror's pre-round value x~/scale lies within 1e-6 of a half-integer; those
    differ by exactly one step and are counted.  Against the fp64 oracle, the
    remaining differences are reported and each must be explained by the
    row's measured rotation error;
  * GEMM: int32 accumulators bit-identical given identical codes; fp16 output
    within 1e-2 relative (floor 2^-14 for fp16 subnormals).
The INT8 activation variant (W4A8) is held to the same rules with its own
oracle functions (scale fp16_rne(a/127), codes in [-128, 127]), except that
the rounding band grows with the code: the kernel rounds u * fp32(c/s) (u the
unnormalised butterfly sum, c = fp32(1/sqrt(n))) where the mirror rounds
fp32(u c) / s; each side has one fp32 rounding, so the two pre-round values
differ by at most 2^-23 |v|.  For |v| <= 7.5 that is below 1e-6 (the INT4
band covers it); for |v| up to 127.5 it reaches 1.5e-5, so INT8 codes may
differ by one step where the pre-round value lies within 1e-6 + 2^-22 |v|
of a half-integer.
"""

from __future__ import annotations

import numpy as np

from oracle import rq_oracle as O

BAND = 1e-6
BAND8_REL = 2.0 ** -22
ROT_TOL = 1e-5
Y_TOL = 1e-2


def dist_to_half_integer(v: np.ndarray) -> np.ndarray:
    return np.abs(np.abs(v - np.floor(v)) - 0.5)


def check_codes(q_gpu: np.ndarray, ref: dict, what: str, band_rel: float = 0.0) -> int:
    """GPU codes against an oracle result dict; returns the in-band mismatch
    count.  The band is BAND + band_rel * |v| around each half-integer."""
    q_ref = ref["q"]
    bad = q_gpu != q_ref
    n_bad = int(bad.sum())
    if n_bad:
        v = ref["v"][bad]
        step = np.abs(q_gpu[bad].astype(np.int16) - q_ref[bad].astype(np.int16))
        near = dist_to_half_integer(v) <= BAND + band_rel * np.abs(v)
        assert np.all(step == 1), f"{what}: code differs by more than one step"
        assert np.all(near), (f"{what}: {int((~near).sum())} code mismatches outside the 1e-6 band; "
                              f"worst distance {dist_to_half_integer(v).min():.3e}")
    return n_bad


def check_rotation_result(x, signs, codes, scales, x_rot=None, what="fwht_quant",
                          rows=None, report=None, bits=4, ref=None):
    """Full check of one rq_fwht_quant / rq_fold_weights result (bits=4) or
    rq_fwht_quant8 result (bits=8, codes int8 [m, n]).

    ``rows`` optionally selects the rows (of x and of the outputs) to check.
    ``ref`` optionally passes the oracle's (fp32 mirror, fp64) results for
    the same x and signs, computed once by the caller (not with ``rows``).
    """
    quant = O.fwht_quant if bits == 4 else O.fwht_quant8
    unpack = O.unpack_int4 if bits == 4 else (lambda c: np.asarray(c).astype(np.int8))
    x = np.asarray(x)
    if rows is not None:
        x = x[rows]
        codes = codes[rows]
        scales = scales[rows]
        if x_rot is not None:
            x_rot = x_rot[rows]
    mirror = quant(x, signs, "f32") if ref is None else ref[0]
    if x_rot is not None:
        diff = x_rot.view(np.uint32) != mirror["x_rot"].view(np.uint32)
        # +0 and -0 are the same value
        diff &= ~((x_rot == 0) & (mirror["x_rot"] == 0))
        assert not diff.any(), f"{what}: rotated rows differ from the fp32 mirror in {int(diff.sum())} places"
        truth = O.rotate(x, signs, "f64")
        err = np.abs(x_rot.astype(np.float64) - truth).max(axis=-1)
        ref_max = np.abs(truth).max(axis=-1)
        assert np.all(err <= ROT_TOL * ref_max + 1e-300), f"{what}: rotation error above 1e-5 relative"
    assert np.array_equal(scales.view(np.uint16), mirror["scales"].view(np.uint16)), \
        f"{what}: scales differ from the mirror"
    q_gpu = unpack(codes)
    band_rel = 0.0 if bits == 4 else BAND8_REL
    n_band = check_codes(q_gpu, mirror, what, band_rel)
    # against the fp64 oracle: report, and require each difference to be explained
    truth = quant(x, signs, "f64") if ref is None else ref[1]
    same_scale = scales.view(np.uint16) == truth["scales"].view(np.uint16)
    d = (q_gpu != truth["q"]) & same_scale[..., None]
    n_truth = int(d.sum())
    if n_truth:
        rot_err = np.abs(mirror["x_rot"].astype(np.float64) - truth["x_rot"]).max(axis=-1, keepdims=True)
        s = truth["scales"].astype(np.float64)[..., None]
        v = truth["v"]
        allow = rot_err / s + BAND + band_rel * np.abs(v)
        assert np.all(dist_to_half_integer(v[d]) <= allow[d]), \
            f"{what}: code mismatch vs fp64 not explained by the rotation error"
    if report is not None:
        report.append({"what": what, "elements": int(q_gpu.size), "band_mismatch_vs_mirror": n_band,
                       "mismatch_vs_fp64": n_truth,
                       "scale_ulp_rows_vs_fp64": int((~same_scale).sum())})
    return n_band, n_truth


def check_gemm(a_codes, a_scales, w_codes, w_scales, y, acc=None, what="gemm",
               rows=None, cols=None, a8=False):
    """Oracle GEMM on (a subset of) the same codes; acc exact, y within 1e-2.
    a8: the activation codes are INT8 bytes (W4A8)."""
    ra = slice(None) if rows is None else rows
    cb = slice(None) if cols is None else cols
    y_ref, acc_ref = (O.w4a8_gemm if a8 else O.w4a4_gemm)(a_codes[ra], a_scales[ra], w_codes[cb], w_scales[cb])
    y_g = y[ra][:, cb]
    if acc is not None:
        acc_g = acc[ra][:, cb]
        assert np.array_equal(acc_g.astype(np.int64), acc_ref), \
            f"{what}: int32 accumulators differ in {int((acc_g != acc_ref).sum())} places"
    yr = y_ref.astype(np.float64)
    yg = y_g.astype(np.float64)
    both_inf = np.isinf(yr) & np.isinf(yg) & (np.sign(yr) == np.sign(yg))
    tol = Y_TOL * np.maximum(np.abs(yr), 2.0 ** -14)
    ok = (np.abs(yg - yr) <= tol) | both_inf
    assert ok.all(), f"{what}: {int((~ok).sum())} fp16 outputs outside 1e-2 relative"
    return y_ref, acc_ref


def check_asym_result(x, signs, codes, scales, zeros, x_rot=None, what="fwht_quant_asym",
                      report=None):
    """Full check of one rq_fwht_quant_asym result against the oracle.

    Rotated rows and scales bit-identical to the fp32 mirror (the range
    hi - lo is an fp32 difference on both sides).  The zero point and the
    codes are decisions on pre-round values that the kernel and the mirror
    compute with one fp32 rounding each (|dv| <= 2^-23 |v|): a zero point may
    differ by one only where the mirror's -lo/scale lies within
    BAND + BAND8_REL |w| of a half-integer, and a code only where x~/scale
    does; codes are compared against the mirror's level shifted by the
    kernel's own zero point.
    """
    x = np.asarray(x)
    mirror = O.fwht_quant_asym(x, signs, "f32")
    if x_rot is not None:
        diff = x_rot.view(np.uint32) != mirror["x_rot"].view(np.uint32)
        diff &= ~((x_rot == 0) & (mirror["x_rot"] == 0))
        assert not diff.any(), f"{what}: rotated rows differ from the fp32 mirror"
    assert np.array_equal(scales.view(np.uint16), mirror["scales"].view(np.uint16)), \
        f"{what}: scales differ from the mirror"
    zd = zeros.astype(np.int16) - mirror["zeros"].astype(np.int16)
    if zd.any():
        w = mirror["w"][zd != 0]
        assert np.all(np.abs(zd[zd != 0]) == 1), f"{what}: zero point off by more than one"
        assert np.all(dist_to_half_integer(w) <= BAND + BAND8_REL * np.abs(w)), \
            f"{what}: zero-point mismatch outside the rounding band"
    q_gpu = O.unpack_uint4(codes).astype(np.int16)
    v = mirror["v"]
    q_ref = np.clip(np.rint(v) + zeros.astype(np.float64)[:, None], 0, 15).astype(np.int16)
    scale_ok = (mirror["scales"].astype(np.float64) > 0) & np.isfinite(mirror["scales"].astype(np.float64))
    q_ref = np.where(scale_ok[:, None], q_ref, 0)
    bad = q_gpu != q_ref
    n_bad = int(bad.sum())
    if n_bad:
        assert np.all(np.abs(q_gpu[bad] - q_ref[bad]) == 1), f"{what}: code off by more than one"
        vb = v[bad]
        assert np.all(dist_to_half_integer(vb) <= BAND + BAND8_REL * np.abs(vb)), \
            f"{what}: {n_bad} code mismatches, some outside the rounding band"
    if report is not None:
        report.append({"what": what, "elements": int(q_gpu.size), "band_mismatch_vs_mirror": n_bad,
                       "zero_point_band_mismatch": int((zd != 0).sum())})
    return n_bad
