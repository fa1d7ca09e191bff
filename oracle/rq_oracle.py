"""Plain CPU oracle for the online rotate + INT4 + W4A4 hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
kernels, their headers or the Python binding; the two sides meet only through
seeded input arrays.

Pages cited (each function names the passage it follows):
  [QuaRot]    aicassindra.com, QuaRot explainer ("Why architecture matters
              here" / "The architecture: every piece explained" /
              "End-to-end flow").
  [RQ]        llms.blog, "Rotational Quantization: How Orthogonal Transforms
              and Hadamard Incoherence Enable Outlier-Free Low-Bit Inference".
  [SpinQuant] aicassindra.com, SpinQuant explainer (same three sections as
              [QuaRot]).

Notation (row vectors, [RQ] "The Principle of Computational Invariance"):
  X is m x d (one token per row), W is d x k, Y = X W.
  R = diag(s) . H_n / sqrt(n) with H_n the +-1 Sylvester matrix and s a
  Rademacher sign vector.  Rotated activation  X~ = X R  (each row
  x -> (x * s) H_n / sqrt(n));  folded weight  W~ = R^T W, stored as
  W~^T = W^T R, i.e. the same row transform applied to each row of W^T.

Two precisions:
  "f64"  truth mode: every floating-point step in float64.
  "f32"  mirror mode: the same steps in float32 (IEEE add/sub, no fused
         multiply-add), butterflies in ascending-stride order, and the single
         global scale applied as one multiply by fp32(1/sqrt(n)).  A GPU
         kernel that keeps this stage order can be compared bit for bit on the
         rotated activations, and its INT4 decisions are taken in the same
         (fp32) precision.

Quantizer (symmetric per row, codes in [-8, 7], nibble packed):
  a = max_j |x~_j|;  scale = fp16_rne(a / 7);  q_j = clamp(rne(x~_j / scale),
  -8, 7) with rne = round half to even; scale == 0 gives all-zero codes.
  The scale that is stored (fp16) is the one that divides, so dequantisation
  q * scale uses exactly the stored value.  Packing: byte i holds code 2i in
  its low nibble and code 2i+1 in its high nibble, two's complement.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(explicit Sylvester matrices, scipy.linalg.hadamard, closed forms, brute force
on tiny inputs, worked examples from the pages).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "hadamard_transform",
    "paley_hadamard_28",
    "kron28_transform",
    "rotate",
    "fp16_rne",
    "quantize_rows",
    "pack_int4",
    "unpack_int4",
    "fwht_quant",
    "fold_weights",
    "w4a4_gemm",
    "quantize_rows_int8",
    "fwht_quant8",
    "w4a8_gemm",
    "kv_rotate_quant",
    "dequantize",
    "quantize_rows_asym",
    "fwht_quant_asym",
    "unpack_uint4",
    "w4a4_gemm_asym",
    "quantize_groups",
    "w4a4_gemm_grouped",
    "inverse_rotate",
    "decode_attention",
    "decode_attention_int4",
]

QMIN, QMAX = -8, 7
QMIN8, QMAX8 = -128, 127
UMAX4 = 15          # asymmetric INT4: unsigned codes 0 .. 2^4 - 1
GROUP = 128         # per-group weight scales: elements per group


def _check_pow2(n: int) -> None:
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"rotation length must be a power of two, got {n}")


def _is_pow2(n: int) -> bool:
    return n >= 1 and (n & (n - 1)) == 0


def _is_28_pow2(n: int) -> bool:
    """n = 28 * 2^k (k >= 0): the non-power-of-two lengths supported."""
    return n >= 28 and n % 28 == 0 and _is_pow2(n // 28)


def _legendre(a: int, q: int) -> int:
    """Quadratic character of a modulo the odd prime q (Euler's criterion)."""
    a %= q
    if a == 0:
        return 0
    return 1 if pow(a, (q - 1) // 2, q) == 1 else -1


def paley_hadamard_28() -> np.ndarray:
    """A Hadamard matrix of order 28, by Paley's second construction.

    [RQ] "Learned Orthogonal Rotations: SpinQuant": fixed Hadamard rotations
    need power-of-two sizes or products of small Hadamard-compatible factors
    (the input of the down projection, which needs an online rotation
    ([RQ] "Weight Absorption and Online Fast Walsh-Hadamard Transforms",
    part 2), is 14336 = 28 * 512 wide in Llama-class models).  Construction
    (Paley II, q = 13, a prime with q = 1 mod 4): the Jacobsthal matrix
    Q[a][b] = chi(a - b) over GF(13), chi the quadratic character; the
    symmetric conference matrix C = [[0, 1^T], [1, Q]] of order 14 with
    C C^T = 13 I; then H = C (x) [[1, 1], [1, -1]] + I (x) [[1, -1], [-1, -1]],
    entries +-1, H H^T = 28 I, and H symmetric.  Index 2i + c of H is
    (row i of C, component c).
    """
    q = 13
    jac = np.array([[_legendre(a - b, q) for b in range(q)] for a in range(q)], dtype=np.int64)
    conf = np.zeros((q + 1, q + 1), dtype=np.int64)
    conf[0, 1:] = 1
    conf[1:, 0] = 1
    conf[1:, 1:] = jac
    h2 = np.array([[1, 1], [1, -1]], dtype=np.int64)
    j2 = np.array([[1, -1], [-1, -1]], dtype=np.int64)
    return (np.kron(conf, h2) + np.kron(np.eye(q + 1, dtype=np.int64), j2)).astype(np.int8)


def _paley_conference_14() -> np.ndarray:
    """The order-14 conference matrix C of :func:`paley_hadamard_28`."""
    h = paley_hadamard_28().astype(np.int64)
    return h[0::2, 0::2] - np.eye(14, dtype=np.int64)  # C[j][i] + delta_ij * J2[0][0]


def kron28_transform(u: np.ndarray, precision: str = "f64") -> np.ndarray:
    """Unnormalised (H_28 (x) H_P) transform along the last axis, n = 28 * P.

    Element e = P * b + p (block b of 28, position p inside the block).
    Step 1: the Sylvester FWHT of length P inside every block
    (:func:`hadamard_transform`, ascending strides).  Step 2: for every
    position, y[b'] = sum_b H_28[b'][b] t[b] (H_28 symmetric).
    "f64": step 2 is the dense 28 x 28 product in float64.
    "f32": step 2 in float32, in an order that the Paley structure
    H_28 = C (x) H_2 + I (x) J_2 gives: a_i = t[2i] + t[2i+1],
    d_i = t[2i] - t[2i+1], y[2j] = (C a)_j + d_j and y[2j+1] = (C d)_j - a_j.
    The conference matrix products use the residue structure of C: with
    S = v_1 + ... + v_13 and T_x = sum over the quadratic residues r of 13
    of v_(1 + (x - r) mod 13), row 1 + x of C has +1 exactly at those
    columns and at column 0, and -1 at the other twelve off-diagonal ones,
    so (C v)_0 = S and (C v)_(1+x) = v_0 + T_x - (S - v_(1+x) - T_x)
    = 2 T_x + ((v_0 - S) + v_(1+x)).  In float32: S accumulated left to
    right over i = 1..13, w = v_0 - S, T_x left to right over the residues
    in ascending order; then y[0] = S_a + d_0, y[1] = S_d - a_0 and, for
    j = 1 + x, y[2j] = 2 T_x(a) + (w_a + (a_j + d_j)) and
    y[2j+1] = 2 T_x(d) + (w_d + (d_j - a_j)) (2 T is exact, so each of
    these last sums rounds once).
    """
    u = np.asarray(u)
    n = u.shape[-1]
    if not _is_28_pow2(n):
        raise ValueError(f"length must be 28 * 2^k, got {n}")
    pw = n // 28
    lead = u.shape[:-1]
    dt = np.float64 if precision == "f64" else np.float32
    t = hadamard_transform(u.astype(dt).reshape(lead + (28, pw)))
    if precision == "f64":
        h = paley_hadamard_28().astype(np.float64)
        y = np.einsum("ab,...bp->...ap", h, t)
        return y.reshape(lead + (n,))
    if precision != "f32":
        raise ValueError(f"precision must be 'f64' or 'f32', got {precision!r}")
    residues = sorted({(r * r) % 13 for r in range(1, 13)})
    a = t[..., 0::2, :] + t[..., 1::2, :]   # [..., 14, P]
    d = t[..., 0::2, :] - t[..., 1::2, :]

    def conference_terms(v):
        """S, w = v_0 - S and T_x (x = 0..12) of C v, in float32."""
        s = v[..., 1, :]
        for i in range(2, 14):
            s = s + v[..., i, :]
        w = v[..., 0, :] - s
        ts = []
        for x in range(13):
            tx = v[..., 1 + (x - residues[0]) % 13, :]
            for r in residues[1:]:
                tx = tx + v[..., 1 + (x - r) % 13, :]
            ts.append(tx)
        return s, w, ts

    s_a, w_a, t_a = conference_terms(a)
    s_d, w_d, t_d = conference_terms(d)
    y = np.empty_like(t)
    y[..., 0, :] = s_a + d[..., 0, :]
    y[..., 1, :] = s_d - a[..., 0, :]
    for x in range(13):
        j = 1 + x
        y[..., 2 * j, :] = (t_a[x] + t_a[x]) + (w_a + (a[..., j, :] + d[..., j, :]))
        y[..., 2 * j + 1, :] = (t_d[x] + t_d[x]) + (w_d + (d[..., j, :] - a[..., j, :]))
    return y.reshape(lead + (n,)).astype(np.float32)


def hadamard_transform(u: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis.

    [RQ] "Weight Absorption and Online Fast Walsh-Hadamard Transforms",
    part 2 (online FWHT): the butterfly exploits the recursive Kronecker
    structure of the Sylvester matrix, costs O(n log2 n) and uses only
    additions and subtractions.  [RQ] "Incoherence Processing via Randomized
    Hadamard Transforms", recursion H_2k = [[H_k, H_k], [H_k, -H_k]] (here
    without the 1/sqrt(2) per level; the one global scale is applied by the
    caller).  Natural (Sylvester) ordering: output j = sum_i (-1)^popcount(i&j)
    u_i.  Stages run in ascending stride h = 1, 2, ..., n/2; at each stage the
    pair (a, b) at positions (i, i + h), bit h of i clear, becomes
    (a + b, a - b).  The dtype of ``u`` is kept, so float32 input is computed
    with float32 rounding after every add/sub.
    """
    out = np.array(u, copy=True)
    n = out.shape[-1]
    _check_pow2(n)
    lead = out.shape[:-1]
    h = 1
    while h < n:
        v = out.reshape(lead + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return out


def _inv_sqrt_f32(n: int) -> np.float32:
    """fp32(1/sqrt(n)): the float64 value rounded once to float32."""
    return np.float32(1.0 / np.sqrt(np.float64(n)))


def rotate(x: np.ndarray, signs: np.ndarray | None, precision: str = "f64") -> np.ndarray:
    """Row-wise randomized Hadamard rotation x -> (x * s) H_n / sqrt(n).

    [RQ] "Incoherence Processing via Randomized Hadamard Transforms": the
    randomized Hadamard transform multiplies by a Rademacher sign diagonal and
    the Sylvester matrix; the normalised matrix has entries +-1/sqrt(n).
    [RQ] "Weight Absorption and Online Fast Walsh-Hadamard Transforms": the
    butterflies use only add/sub and one global scalar multiplication at the
    end.  The sign diagonal comes first (x * s, then H), the order in which
    the rotated linear layer is specified; the fold below uses the same R.
    ``signs=None`` means s = 1 (plain H_n / sqrt(n)).  For n = 28 * 2^k the
    Hadamard factor is H_28 (x) H_(n/28) (:func:`kron28_transform`).
    """
    x = np.asarray(x)
    n = x.shape[-1]
    if not _is_28_pow2(n):
        _check_pow2(n)
    if precision == "f64":
        u = x.astype(np.float64)
        if signs is not None:
            u = u * np.asarray(signs).astype(np.float64)
        y = kron28_transform(u, "f64") if _is_28_pow2(n) else hadamard_transform(u)
        return y / np.sqrt(np.float64(n))
    if precision == "f32":
        u = x.astype(np.float32)
        if signs is not None:
            u = u * np.asarray(signs).astype(np.float32)  # exact: s = +-1
        y = kron28_transform(u, "f32") if _is_28_pow2(n) else hadamard_transform(u)
        return (y * _inv_sqrt_f32(n)).astype(np.float32)
    raise ValueError(f"precision must be 'f64' or 'f32', got {precision!r}")


def fp16_rne(v) -> np.ndarray:
    """Round float64 values to IEEE binary16, once, half to even.

    numpy's float64 -> float16 cast rounds directly from the double value
    (no detour through float32); the pins check that against hand-built
    midpoint cases, subnormals and overflow to infinity.
    """
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16)


def quantize_rows(xt: np.ndarray):
    """Symmetric per-row INT4 quantisation of rotated rows.

    [QuaRot] "End-to-end flow" (runtime: the rotated activation is quantised
    to INT4) and [RQ] "The Activation Outlier Bottleneck in Low-Bit Serving"
    (a uniform grid of 2^4 = 16 levels whose range is set by the extremes).
    Symmetric form: scale = fp16_rne(max|x~| / 7), q = clamp(rne(x~/scale),
    -8, 7); a zero scale (zero row, or a/7 below half the smallest fp16
    subnormal) gives all-zero codes.  The division runs in float64 on the
    given values, so for float32 input it is the exact quotient up to
    2^-53 relative.

    Returns (q int8 [..., n], scales float16 [...], v float64 [..., n]) where v
    is the pre-round value x~/scale (0 where the scale is 0).
    """
    xt64 = np.asarray(xt).astype(np.float64)
    a = np.max(np.abs(xt64), axis=-1)
    scales = fp16_rne(a / 7.0)
    s = scales.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s > 0, xt64 / np.where(s > 0, s, 1.0), 0.0)
    q = np.clip(np.rint(v), QMIN, QMAX).astype(np.int8)  # np.rint: half to even
    return q, scales, v


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two's-complement nibble packing: low nibble = even index."""
    q = np.asarray(q).astype(np.int16)
    if q.shape[-1] % 2:
        raise ValueError("packing needs an even number of codes per row")
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(codes: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_int4` (sign-extends each nibble)."""
    c = np.asarray(codes).astype(np.int16)
    lo = c & 0xF
    hi = (c >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---------------------------------------------------------------- F6 layout
# [RQ] "Hardware Execution and Serving Economics", part 1: the INT4 codes of a
# W4A4 layer feed a 4-bit integer matrix product.  The F6 layout carries the
# same integer codes in 6-bit OCP MX E3M2 floats, so that the product can run
# on a 6-bit matrix unit; its values, and so every product and sum, are the
# integers themselves.

def e3m2_value(code: int) -> float:
    """Value of a 6-bit E3M2 code (OCP Microscaling Formats v1.0): bit 5 is
    the sign, bits 4..2 the exponent (bias 3), bits 1..0 the mantissa; the
    exponent 0 encodes the subnormals (m / 4) * 2^(1 - 3).  No inf or NaN."""
    code = int(code)
    if not 0 <= code < 64:
        raise ValueError("E3M2 codes have 6 bits")
    sign = -1.0 if code & 0x20 else 1.0
    e, mant = (code >> 2) & 7, code & 3
    if e == 0:
        return sign * (mant / 4.0) * 2.0 ** (1 - 3)
    return sign * (1.0 + mant / 4.0) * 2.0 ** (e - 3)


def e3m2_code(q: int) -> int:
    """The E3M2 code whose value is the integer q, found by value among all 64
    codes (zero takes the positive code); raises if q is not representable."""
    hits = [c for c in range(64) if e3m2_value(c) == q and not (q == 0 and c & 0x20)]
    if len(hits) != 1:
        raise ValueError(f"{q} is not an E3M2 value")
    return hits[0]


def pack_f6(codes: np.ndarray) -> np.ndarray:
    """rq_pack_f6: packed INT4 codes [rows][d/2] -> F6 layout [d/128][rows][96].

    Block b (0..3) of the 128-code group c of a row holds the codes
    128 c + 32 b + j, j = 0..31, as one 192-bit little-endian word with the
    E3M2 code of code j in bits 6j..6j+5.  Word bytes 0..15 go to group bytes
    16b..16b+15, bytes 16..23 to group bytes 64 + 16 (b % 2) + 8 (b // 2).
    The layout is group-major: group c of row r is out[c, r]."""
    q = unpack_int4(codes).astype(np.int64)
    rows, d = q.shape
    if d % 128:
        raise ValueError("the F6 layout needs d % 128 == 0")
    lut = np.array([e3m2_code(v) for v in range(-8, 8)], dtype=np.uint64)
    e6 = lut[q + 8]                                     # [rows][d] E3M2 codes
    blocks = e6.reshape(rows, d // 32, 32)
    bits = ((blocks[..., :, None] >> np.arange(6, dtype=np.uint64)) & 1).astype(np.uint8)
    words = np.packbits(bits.reshape(rows, d // 32, 192), axis=-1, bitorder="little")  # 24 bytes
    out = np.zeros((d // 128, rows, 96), dtype=np.uint8)
    for c in range(d // 128):
        for b in range(4):
            w = words[:, 4 * c + b, :]
            out[c, :, 16 * b:16 * b + 16] = w[:, :16]
            t = 64 + 16 * (b % 2) + 8 * (b // 2)
            out[c, :, t:t + 8] = w[:, 16:]
    return out


def dequantize(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """q * scale in float64 (the value a code stands for)."""
    return np.asarray(q).astype(np.float64) * np.asarray(scales).astype(np.float64)[..., None]


def fwht_quant(x: np.ndarray, signs: np.ndarray | None, precision: str = "f64") -> dict:
    """Online rotation fused with per-token INT4 quantisation and packing.

    [QuaRot] "End-to-end flow" (runtime): an online Hadamard rotates the
    activation, which is then quantised to INT4.  [RQ] "Weight Absorption and
    Online Fast Walsh-Hadamard Transforms", part 2: the online rotation is an
    FWHT.  Returns codes uint8 [m, n/2], scales float16 [m], x_rot [m, n]
    (float64 or float32), q int8 [m, n] and v (pre-round values).
    """
    xt = rotate(x, signs, precision)
    q, scales, v = quantize_rows(xt)
    return {"codes": pack_int4(q), "scales": scales, "x_rot": xt, "q": q, "v": v}


def fold_weights(wt: np.ndarray, signs: np.ndarray | None, precision: str = "f64") -> dict:
    """Offline fold W~ = R^T W followed by per-output-channel INT4.

    [RQ] "Weight Absorption and Online Fast Walsh-Hadamard Transforms",
    part 1: an input projection's weight is pre-multiplied by R^T once,
    offline.  [QuaRot] "End-to-end flow" (offline: quantize): the folded
    weights are quantised to INT4.  [SpinQuant] "The architecture: every
    piece explained": INT4 weights with per-channel scales.

    ``wt`` is W^T stored [k][d] (output channel major).  Row j of W~^T is
    w_j R = (w_j * s) H_d / sqrt(d): exactly :func:`rotate` applied to each
    row of W^T, then :func:`quantize_rows` along d (one scale per output
    channel).
    """
    return fwht_quant(wt, signs, precision)


def _int_matmul_nt(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """Exact integer product qa @ qw.T for int4 codes (int64 result).

    Uses a float64 matrix product as the library primitive: every product
    is an integer of magnitude <= 64 and every partial sum an integer of
    magnitude <= 64 * d <= 2^20, all exactly representable in float64 (53-bit
    significand), so the result is exact whatever the summation order.
    """
    d = qa.shape[-1]
    if 64 * d >= 2 ** 53:
        raise ValueError("d too large for an exact float64 accumulation")
    acc = qa.astype(np.float64) @ qw.astype(np.float64).T
    return acc.astype(np.int64)


def w4a4_gemm(a_codes: np.ndarray, a_scales: np.ndarray, w_codes: np.ndarray,
              w_scales: np.ndarray):
    """W4A4 linear on packed codes: integer accumulation then fp16 epilogue.

    [RQ] "Hardware Execution and Serving Economics", part 1: a rotated W4A4
    layer runs as an integer GEMM.  [QuaRot] "End-to-end flow": the INT4
    rotated activation multiplies the INT4 folded weight.
    acc[m][j] = sum_i qa[m][i] * qw[j][i] (exact integers),
    y[m][j] = fp16_rne(acc * sa[m] * sw[j]) with the product in float64.
    Returns (y float16 [m, k], acc int64 [m, k]).
    """
    qa = unpack_int4(a_codes)
    qw = unpack_int4(w_codes)
    if qa.shape[-1] != qw.shape[-1]:
        raise ValueError("inner dimensions differ")
    acc = _int_matmul_nt(qa, qw)
    sa = np.asarray(a_scales).astype(np.float64)[:, None]
    sw = np.asarray(w_scales).astype(np.float64)[None, :]
    y = fp16_rne(acc.astype(np.float64) * sa * sw)
    return y, acc


def quantize_rows_int8(xt: np.ndarray):
    """Symmetric per-row INT8 quantisation of rotated rows (the W4A8 variant).

    [SpinQuant] "The architecture: every piece explained" and "End-to-end
    flow": INT4 weights with INT8 activations.  Same rule as
    :func:`quantize_rows` with 2^7 - 1 in place of 2^3 - 1:
    scale = fp16_rne(max|x~| / 127), q = clamp(rne(x~/scale), -128, 127),
    a zero scale gives zero codes.  Returns (q int8, scales float16, v).
    """
    xt64 = np.asarray(xt).astype(np.float64)
    a = np.max(np.abs(xt64), axis=-1)
    scales = fp16_rne(a / 127.0)
    s = scales.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s > 0, xt64 / np.where(s > 0, s, 1.0), 0.0)
    q = np.clip(np.rint(v), QMIN8, QMAX8).astype(np.int8)
    return q, scales, v


def fwht_quant8(x: np.ndarray, signs: np.ndarray | None, precision: str = "f64") -> dict:
    """Online rotation fused with per-token INT8 quantisation (W4A8).

    [SpinQuant] "End-to-end flow" (runtime: the rotated activation is
    quantised to INT8); the rotation is :func:`rotate`.  Returns codes int8
    [m, n] (one byte per element, two's complement), scales float16 [m],
    x_rot, q (= codes) and v.
    """
    xt = rotate(x, signs, precision)
    q, scales, v = quantize_rows_int8(xt)
    return {"codes": q.copy(), "scales": scales, "x_rot": xt, "q": q, "v": v}


def w4a8_gemm(a_codes8: np.ndarray, a_scales: np.ndarray, w_codes: np.ndarray,
              w_scales: np.ndarray):
    """W4A8 linear: INT8 activation codes times packed INT4 weight codes.

    [SpinQuant] "The architecture: every piece explained" (INT4 weights,
    INT8 activations).  acc[m][j] = sum_i qa[m][i] * qw[j][i] (exact
    integers), y = fp16_rne(acc * sa[m] * sw[j]) with the product in float64.
    Returns (y float16 [m, k], acc int64 [m, k]).
    """
    qa = np.asarray(a_codes8).astype(np.int8)
    qw = unpack_int4(w_codes)
    if qa.shape[-1] != qw.shape[-1]:
        raise ValueError("inner dimensions differ")
    d = qa.shape[-1]
    if 1024 * d >= 2 ** 53:
        raise ValueError("d too large for an exact float64 accumulation")
    acc = (qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)
    sa = np.asarray(a_scales).astype(np.float64)[:, None]
    sw = np.asarray(w_scales).astype(np.float64)[None, :]
    y = fp16_rne(acc.astype(np.float64) * sa * sw)
    return y, acc


def kv_rotate_quant(k: np.ndarray, v: np.ndarray, signs: np.ndarray | None = None,
                    precision: str = "f64") -> dict:
    """Per-head rotation and INT4 packing of the key/value cache.

    [QuaRot] "The architecture: every piece explained" (KV-cache rotation
    box) and "End-to-end flow" (the KV cache): keys and values are rotated,
    then quantised to four bits.  [RQ] "Hardware Execution and Serving
    Economics", part 2: 4-bit KV caching after rotating K and V.
    Each head_dim vector (last axis, 128 for the configured cache) is one
    row: plain H/sqrt(n) unless signs are given, then per-row INT4.
    """
    out = {}
    for name, t in (("k", k), ("v", v)):
        r = fwht_quant(np.asarray(t), signs, precision)
        out[name + "_codes"] = r["codes"]
        out[name + "_scales"] = r["scales"]
        out[name + "_q"] = r["q"]
        out[name + "_v"] = r["v"]
        out[name + "_rot"] = r["x_rot"]
    return out


# --------------------------------------------------------------- asymmetric
def quantize_rows_asym(xt: np.ndarray):
    """Asymmetric per-row INT4 quantisation (unsigned codes, integer zero point).

    [RQ] "The Activation Outlier Bottleneck in Low-Bit Serving": the step of a
    uniform b-bit grid spans the whole range, Delta = (max - min) / (2^b - 1).
    Reading of the zero point (the page gives only the step): the affine grid
    x ~ Delta * (q - z) with unsigned codes q in [0, 15] and an integer zero
    point z; the range is widened to contain 0 (lo = min(min x, 0),
    hi = max(max x, 0)) so that z = rne(-lo / Delta) lies in [0, 15] and 0 is
    exactly representable.

      r      = hi - lo, in the precision of the given values (float32 values
               give a float32 difference, as a float32 kernel computes it)
      Delta  = fp16_rne(r / 15), rounded once from the exact quotient
      z      = clamp(rne(-lo / Delta), 0, 15)
      q      = clamp(rne(x / Delta) + z, 0, 15)

    Delta == 0 (a zero row) gives z = 0 and all-zero codes; an infinite Delta
    gives z = 0 and all-zero codes.  Returns (q uint8, scales float16,
    zeros uint8, v = x / Delta float64, w = -lo / Delta float64).
    """
    xt = np.asarray(xt)
    hi = np.maximum(np.max(xt, axis=-1), 0)
    lo = np.minimum(np.min(xt, axis=-1), 0)
    r = (hi - lo).astype(np.float64)          # float32 subtraction for float32 rows
    scales = fp16_rne(r / UMAX4)
    s = scales.astype(np.float64)
    ok = (s > 0) & np.isfinite(s)
    safe = np.where(ok, s, 1.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        w = np.where(ok, -lo.astype(np.float64) / safe, 0.0)
        v = np.where(ok[..., None], xt.astype(np.float64) / safe[..., None], 0.0)
    z = np.clip(np.rint(w), 0, UMAX4)
    q = np.clip(np.rint(v) + z[..., None], 0, UMAX4)
    q = np.where(ok[..., None], q, 0)
    return q.astype(np.uint8), scales, z.astype(np.uint8), v, w


def unpack_uint4(codes: np.ndarray) -> np.ndarray:
    """Unsigned nibbles of packed codes (code 2i in the low nibble of byte i)."""
    c = np.asarray(codes).astype(np.uint8)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), np.uint8)
    out[..., 0::2] = c & 0xF
    out[..., 1::2] = c >> 4
    return out


def _pack_uint4(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q).astype(np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def fwht_quant_asym(x: np.ndarray, signs: np.ndarray | None, precision: str = "f64") -> dict:
    """Online rotation followed by asymmetric per-token INT4.

    The rotation is :func:`rotate`; the quantiser is
    :func:`quantize_rows_asym` ([RQ] "The Activation Outlier Bottleneck in
    Low-Bit Serving").  Returns codes uint8 [m, n/2] (unsigned nibbles,
    packed like the symmetric codes), scales float16 [m], zeros uint8 [m],
    x_rot, q (unsigned codes), v and w (pre-round values of the codes and of
    the zero point).
    """
    xt = rotate(x, signs, precision)
    q, scales, z, v, w = quantize_rows_asym(xt)
    return {"codes": _pack_uint4(q), "scales": scales, "zeros": z, "x_rot": xt, "q": q, "v": v,
            "w": w}


def w4a4_gemm_asym(a_codes: np.ndarray, a_scales: np.ndarray, a_zeros: np.ndarray,
                   w_codes: np.ndarray, w_scales: np.ndarray):
    """W4A4 linear with asymmetric activations and symmetric weights.

    Dequantised activation x^ = sa * (qa - za); weight w^ = sw * qw.  The
    integer accumulator is acc[m][j] = sum_i (qa[m][i] - za[m]) * qw[j][i]
    (exact), y = fp16_rne(acc * sa[m] * sw[j]) with the product in float64.
    Returns (y float16 [m, k], acc int64 [m, k]).
    """
    qa = unpack_uint4(a_codes).astype(np.int64) - np.asarray(a_zeros).astype(np.int64)[:, None]
    qw = unpack_int4(w_codes)
    if qa.shape[-1] != qw.shape[-1]:
        raise ValueError("inner dimensions differ")
    d = qa.shape[-1]
    if 128 * d >= 2 ** 53:
        raise ValueError("d too large for an exact float64 accumulation")
    acc = (qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)
    sa = np.asarray(a_scales).astype(np.float64)[:, None]
    sw = np.asarray(w_scales).astype(np.float64)[None, :]
    return fp16_rne(acc.astype(np.float64) * sa * sw), acc


# ------------------------------------------------------- per-group weights
def quantize_groups(xt: np.ndarray, group: int = GROUP):
    """Symmetric INT4 with one scale per group of `group` consecutive
    elements of each row ([SpinQuant] "End-to-end flow": INT4 weights with
    per-channel or per-group scales).

    Each group is quantised by the symmetric rule of :func:`quantize_rows`
    on its own: scale = fp16_rne(max |x~| / 7) over the group, codes
    clamp(rne(x~ / scale), -8, 7).  Returns (q int8 [..., n], scales float16
    [..., n / group], v float64 [..., n]).
    """
    xt = np.asarray(xt)
    n = xt.shape[-1]
    if n % group:
        raise ValueError("the group size must divide the row length")
    g = xt.reshape(xt.shape[:-1] + (n // group, group))
    q, scales, v = quantize_rows(g)
    return q.reshape(xt.shape), scales, v.reshape(xt.shape)


def w4a4_gemm_grouped(a_codes: np.ndarray, a_scales: np.ndarray, w_codes: np.ndarray,
                      w_group_scales: np.ndarray, group: int = GROUP):
    """W4A4 linear with per-token activation scales and per-group weight
    scales: y[m][j] = fp16_rne(sa[m] * sum_g sw[j][g] * acc[m][j][g]) with
    acc[m][j][g] = sum_{i in group g} qa[m][i] * qw[j][i] (exact integers)
    and the outer sum in float64.  Returns (y float16 [m, k], acc int64
    [m, k, d / group]).
    """
    qa = unpack_int4(a_codes)
    qw = unpack_int4(w_codes)
    m, d = qa.shape
    k = qw.shape[0]
    if qw.shape[-1] != d or d % group:
        raise ValueError("inner dimensions differ or are not a multiple of the group")
    ng = d // group
    acc = np.empty((m, k, ng), np.int64)
    for g in range(ng):
        sl = slice(g * group, (g + 1) * group)
        acc[:, :, g] = _int_matmul_nt(qa[:, sl], qw[:, sl])
    sw = np.asarray(w_group_scales).astype(np.float64).reshape(k, ng)
    sa = np.asarray(a_scales).astype(np.float64)
    y = fp16_rne(sa[:, None] * np.einsum("mkg,kg->mk", acc.astype(np.float64), sw))
    return y, acc


# ------------------------------------------- attention over the INT4 KV cache
def inverse_rotate(y: np.ndarray, signs: np.ndarray | None) -> np.ndarray:
    """y R^T for R = diag(s) H_n / sqrt(n) (float64): H is symmetric, so
    y R^T = (y H_n / sqrt(n)) * s, the transform that undoes :func:`rotate`
    ([RQ] "The Principle of Computational Invariance": R R^T = I)."""
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[-1]
    out = hadamard_transform(y) / math.sqrt(n)
    if signs is not None:
        out = out * np.asarray(signs).astype(np.float64)
    return out


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, lengths=None,
                     sm_scale: float | None = None) -> np.ndarray:
    """Single-token (decode) attention, the plain definition in float64.

    q [B, Hq, D] (the new token's queries), k, v [B, H, S, D] (the cache);
    query head j reads KV head j // (Hq / H) (grouped-query attention).  For
    batch entry b only positions < lengths[b] take part (all S when lengths
    is None); a length of 0 gives a zero output.
    o = softmax(q k^T * sm_scale) v with sm_scale = 1 / sqrt(D) by default.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, D = q.shape
    H, S = k.shape[1], k.shape[2]
    if Hq % H:
        raise ValueError("query heads must be a multiple of the KV heads")
    group = Hq // H
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = S if lengths is None else int(lengths[b])
        if L == 0:
            continue
        for j in range(Hq):
            h = j // group
            scores = k[b, h, :L] @ q[b, j] * scale
            p = np.exp(scores - scores.max())
            out[b, j] = (p / p.sum()) @ v[b, h, :L]
    return out


def decode_attention_int4(q: np.ndarray, k_codes: np.ndarray, k_scales: np.ndarray,
                          v_codes: np.ndarray, v_scales: np.ndarray, signs: np.ndarray | None,
                          lengths=None, sm_scale: float | None = None) -> dict:
    """Decode attention that reads the 4-bit rotated KV cache.

    [QuaRot] "End-to-end flow" (a later token's attention reads the
    four-bit rotated cache; rotation invariance keeps the scores) and
    [RQ] "The Principle of Computational Invariance" (q k^T = (qR)(kR)^T).
    The cache holds rotated, quantised rows (:func:`kv_rotate_quant`:
    codes [B, H, S, D/2], scales [B, H, S]); the query is rotated with the
    same R, attention runs on the dequantised cache in the rotated basis, and
    the output is rotated back: o = softmax(q~ K^_rot^T * sm_scale) V^_rot R^T.
    Returns {"o": o, "o_rot": output before the inverse rotation, "q_rot"}.
    """
    kh = dequantize(unpack_int4(k_codes), k_scales)
    vh = dequantize(unpack_int4(v_codes), v_scales)
    q_rot = rotate(np.asarray(q), signs, "f64")
    o_rot = decode_attention(q_rot, kh, vh, lengths, sm_scale)
    return {"o": inverse_rotate(o_rot, signs), "o_rot": o_rot, "q_rot": q_rot}
