"""Thin ctypes binding over librq (include/rq.h).

Argument marshalling only: shape/dtype/device checks, output allocation with
torch, then one C call that queues the HIP kernels on the current torch
stream.  Every arithmetic step runs in librq's kernels; there is no fallback.
If the library has not been built, or HIP cannot be loaded, the first call
raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

RQ_OK, RQ_ERR_NULL, RQ_ERR_SHAPE, RQ_ERR_ALIGN, RQ_ERR_DTYPE, RQ_ERR_HIP = range(6)
RQ_F16, RQ_F32 = 0, 1

EXPORTED = (
    "rq_fwht_quant",
    "rq_fold_weights",
    "rq_w4a4_gemm_workspace_size",
    "rq_w4a4_gemm",
    "rq_pack_f6",
    "rq_w4a4_gemm_f6",
    "rq_kv_rotate_quant",
    "rq_linear_decode_workspace_size",
    "rq_linear_decode",
    "rq_linear_decode_noalloc",
    "rq_linear_decode_w4a8",
    "rq_fwht_quant8",
    "rq_w4a8_gemm",
    "rq_fwht_quant_asym",
    "rq_weight_code_sums",
    "rq_w4a4_gemm_asym",
    "rq_quantize_groups",
    "rq_w4a4_gemm_grouped",
    "rq_decode_attention_workspace_size",
    "rq_decode_attention",
    "rq_status_string",
    "rq_version",
)

_lib = None


class RQError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {status_string(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librq.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"librq.so not found at {path}; build it with "
            "`python -m rotation_w4a4_quantization_amd.build`")
    lib = ctypes.CDLL(path)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.rq_fwht_quant.argtypes = [p, i32, i64, i64, p, p, p, p, p]
    lib.rq_fwht_quant.restype = i32
    lib.rq_fold_weights.argtypes = [p, i32, i64, i64, p, p, p, p, p]
    lib.rq_fold_weights.restype = i32
    lib.rq_w4a4_gemm_workspace_size.argtypes = [i64, i64, i64]
    lib.rq_w4a4_gemm_workspace_size.restype = sz
    lib.rq_w4a4_gemm.argtypes = [p, p, i64, p, p, i64, i64, p, p, p, sz, p]
    lib.rq_w4a4_gemm.restype = i32
    lib.rq_pack_f6.argtypes = [p, i64, i64, p, p]
    lib.rq_pack_f6.restype = i32
    lib.rq_w4a4_gemm_f6.argtypes = [p, p, i64, p, p, i64, i64, p, p, p]
    lib.rq_w4a4_gemm_f6.restype = i32
    lib.rq_kv_rotate_quant.argtypes = [p, p, i64, i64, p, p, p, p, p, p]
    lib.rq_kv_rotate_quant.restype = i32
    lib.rq_linear_decode_workspace_size.argtypes = [i64, i64]
    lib.rq_linear_decode_workspace_size.restype = sz
    lib.rq_linear_decode.argtypes = [p, i64, i64, p, p, p, i64, p, p, sz, p]
    lib.rq_linear_decode.restype = i32
    lib.rq_linear_decode_noalloc.argtypes = [p, i64, i64, p, p, p, i64, p, p]
    lib.rq_linear_decode_noalloc.restype = i32
    lib.rq_linear_decode_w4a8.argtypes = [p, i64, i64, p, p, p, i64, p, p]
    lib.rq_linear_decode_w4a8.restype = i32
    lib.rq_fwht_quant8.argtypes = [p, i64, i64, p, p, p, p, p]
    lib.rq_fwht_quant8.restype = i32
    lib.rq_w4a8_gemm.argtypes = [p, p, i64, p, p, i64, i64, p, p, p]
    lib.rq_w4a8_gemm.restype = i32
    lib.rq_fwht_quant_asym.argtypes = [p, i64, i64, p, p, p, p, p, p]
    lib.rq_fwht_quant_asym.restype = i32
    lib.rq_weight_code_sums.argtypes = [p, i64, i64, p, p]
    lib.rq_weight_code_sums.restype = i32
    lib.rq_w4a4_gemm_asym.argtypes = [p, p, p, i64, p, p, p, i64, i64, p, p, p]
    lib.rq_w4a4_gemm_asym.restype = i32
    lib.rq_quantize_groups.argtypes = [p, i64, i64, i64, p, p, p]
    lib.rq_quantize_groups.restype = i32
    lib.rq_w4a4_gemm_grouped.argtypes = [p, p, i64, p, p, i64, i64, p, p, p]
    lib.rq_w4a4_gemm_grouped.restype = i32
    lib.rq_decode_attention_workspace_size.argtypes = [i64, i64, i64, i64]
    lib.rq_decode_attention_workspace_size.restype = sz
    lib.rq_decode_attention.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, p,
                                        ctypes.c_float, p, p, p, sz, p]
    lib.rq_decode_attention.restype = i32
    lib.rq_status_string.argtypes = [i32]
    lib.rq_status_string.restype = ctypes.c_char_p
    lib.rq_version.argtypes = []
    lib.rq_version.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().rq_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().rq_version())


def _check(func: str, status: int) -> None:
    if status != RQ_OK:
        raise RQError(func, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_cuda(name: str, t: torch.Tensor) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _signs(signs, n, device):
    if signs is None:
        return None
    if signs.dtype != torch.int8 or signs.numel() != n:
        raise ValueError(f"signs must be int8 with {n} entries")
    _need_cuda("signs", signs)
    return signs


def _out(name: str, t, shape, dtype, device) -> torch.Tensor:
    """A caller-supplied output tensor, checked before anything is launched
    (dtype, exact shape, device, contiguity), or a new one when t is None."""
    shape = tuple(int(v) for v in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    if not t.is_cuda or t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _outs(names, shapes, dtypes, device, out):
    """Unpack an `out=` tuple (or None) into checked output tensors."""
    if out is None:
        out = (None,) * len(names)
    if not isinstance(out, (tuple, list)) or len(out) != len(names):
        raise ValueError(f"out must be a tuple ({', '.join(names)})")
    return tuple(_out(n, t, sh, dt, device) for n, t, sh, dt in zip(names, out, shapes, dtypes))


def _workspace(t, nbytes: int, device) -> torch.Tensor:
    """A caller-supplied device workspace (uint8, contiguous, at least nbytes)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    if not t.is_cuda or t.device != torch.device(device) or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if t.numel() < nbytes:
        raise ValueError(f"workspace holds {t.numel()} bytes, {nbytes} are needed")
    return t


def _rotate_quant(cfunc: str, x: torch.Tensor, signs, debug: bool, out=None):
    _need_cuda("x", x)
    if x.dtype not in (torch.float16, torch.float32):
        raise ValueError("x must be float16 or float32")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, n]")
    rows, n = x.shape
    s = _signs(signs, n, x.device)
    names = ("codes", "scales") + (("x_rot",) if debug else ())
    shapes = ((rows, n // 2), (rows,), (rows, n))
    dtypes = (torch.uint8, torch.float16, torch.float32)
    outs = _outs(names, shapes[:len(names)], dtypes[:len(names)], x.device, out)
    codes, scales = outs[0], outs[1]
    rot = outs[2] if debug else None
    dtype = RQ_F16 if x.dtype == torch.float16 else RQ_F32
    st = getattr(load_library(), cfunc)(_ptr(x), dtype, rows, n, _ptr(s), _ptr(codes),
                                        _ptr(scales), _ptr(rot), _stream())
    _check(cfunc, st)
    return codes, scales, rot


def fwht_quant(x: torch.Tensor, signs: torch.Tensor | None = None, debug: bool = False,
               out=None):
    """rq_fwht_quant: returns (codes uint8 [m, n/2], scales fp16 [m], x_rot fp32 or None).
    `out` optionally gives the output tensors (codes, scales[, x_rot])."""
    return _rotate_quant("rq_fwht_quant", x, signs, debug, out)


def fold_weights(wt: torch.Tensor, signs: torch.Tensor | None = None, debug: bool = False,
                 out=None):
    """rq_fold_weights on W^T [k][d]: returns (codes [k, d/2], scales [k], w_rot or None)."""
    return _rotate_quant("rq_fold_weights", wt, signs, debug, out)


def w4a4_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
              w_scales: torch.Tensor, debug: bool = False, out: torch.Tensor | None = None,
              acc_out: torch.Tensor | None = None):
    """rq_w4a4_gemm: returns (y fp16 [m, k], acc int32 [m, k] or None).
    `out` / `acc_out` optionally give y and (with debug) the accumulators."""
    for name, t in (("a_codes", a_codes), ("a_scales", a_scales), ("w_codes", w_codes),
                    ("w_scales", w_scales)):
        _need_cuda(name, t)
    if a_codes.dtype != torch.uint8 or w_codes.dtype != torch.uint8:
        raise ValueError("codes must be uint8")
    if a_scales.dtype != torch.float16 or w_scales.dtype != torch.float16:
        raise ValueError("scales must be float16")
    m, half_d = a_codes.shape
    k, half_d2 = w_codes.shape
    if half_d != half_d2:
        raise ValueError("activation and weight codes differ in d")
    if a_scales.numel() != m or w_scales.numel() != k:
        raise ValueError("scale counts do not match the code rows")
    d = 2 * half_d
    lib = load_library()
    ws_bytes = int(lib.rq_w4a4_gemm_workspace_size(m, k, d))
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=a_codes.device) if ws_bytes else None
    y = _out("out", out, (m, k), torch.float16, a_codes.device)
    acc = _out("acc_out", acc_out, (m, k), torch.int32, a_codes.device) if debug else None
    st = lib.rq_w4a4_gemm(_ptr(a_codes), _ptr(a_scales), m, _ptr(w_codes), _ptr(w_scales), k, d,
                          _ptr(y), _ptr(acc), _ptr(ws), ws_bytes, _stream())
    _check("rq_w4a4_gemm", st)
    return y, acc


def pack_f6(codes: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """rq_pack_f6: packed INT4 codes uint8 [rows, d/2] -> F6 layout uint8
    [d/128, rows, 96] (fp6 E3M2 containers in the 6-bit MFMA operand layout,
    group-major)."""
    _need_cuda("codes", codes)
    if codes.dtype != torch.uint8 or codes.dim() != 2:
        raise ValueError("codes must be a 2-D uint8 tensor")
    rows, half_d = codes.shape
    d = 2 * half_d
    o = _out("out", out, (d // 128, rows, 96), torch.uint8, codes.device)
    _check("rq_pack_f6", load_library().rq_pack_f6(_ptr(codes), rows, d, _ptr(o), _stream()))
    return o


def w4a4_gemm_f6(a_f6: torch.Tensor, a_scales: torch.Tensor, w_f6: torch.Tensor,
                 w_scales: torch.Tensor, debug: bool = False, out: torch.Tensor | None = None,
                 acc_out: torch.Tensor | None = None):
    """rq_w4a4_gemm_f6 on the F6 layouts [d/128, m, 96] and [d/128, k, 96]:
    returns (y fp16 [m, k], acc int32 [m, k] or None), equal to w4a4_gemm on
    the same codes."""
    for name, t in (("a_f6", a_f6), ("a_scales", a_scales), ("w_f6", w_f6),
                    ("w_scales", w_scales)):
        _need_cuda(name, t)
    if a_f6.dtype != torch.uint8 or w_f6.dtype != torch.uint8:
        raise ValueError("F6 rows must be uint8")
    if a_scales.dtype != torch.float16 or w_scales.dtype != torch.float16:
        raise ValueError("scales must be float16")
    if a_f6.dim() != 3 or w_f6.dim() != 3 or a_f6.shape[2] != 96 or w_f6.shape[2] != 96:
        raise ValueError("F6 layouts must be [d/128, rows, 96]")
    groups, m, _ = a_f6.shape
    groups2, k, _ = w_f6.shape
    if groups != groups2:
        raise ValueError("activation and weight F6 layouts differ in d")
    if a_scales.numel() != m or w_scales.numel() != k:
        raise ValueError("scale counts do not match the rows")
    d = 128 * groups
    y = _out("out", out, (m, k), torch.float16, a_f6.device)
    acc = _out("acc_out", acc_out, (m, k), torch.int32, a_f6.device) if debug else None
    st = load_library().rq_w4a4_gemm_f6(_ptr(a_f6), _ptr(a_scales), m, _ptr(w_f6),
                                        _ptr(w_scales), k, d, _ptr(y), _ptr(acc), _stream())
    _check("rq_w4a4_gemm_f6", st)
    return y, acc


def kv_rotate_quant(k: torch.Tensor, v: torch.Tensor, signs: torch.Tensor | None = None,
                    out=None):
    """rq_kv_rotate_quant on fp16 [..., 128] K and V.

    Returns (k_codes [..., 64], k_scales [...], v_codes, v_scales); `out`
    optionally gives those four tensors."""
    _need_cuda("k", k)
    _need_cuda("v", v)
    if k.dtype != torch.float16 or v.dtype != torch.float16 or k.shape != v.shape:
        raise ValueError("k and v must be float16 tensors of the same shape")
    head_dim = k.shape[-1]
    rows = k.numel() // head_dim
    s = _signs(signs, head_dim, k.device)
    lead = tuple(k.shape[:-1])
    kc, ks, vc, vs = _outs(("k_codes", "k_scales", "v_codes", "v_scales"),
                           (lead + (head_dim // 2,), lead, lead + (head_dim // 2,), lead),
                           (torch.uint8, torch.float16, torch.uint8, torch.float16), k.device, out)
    st = load_library().rq_kv_rotate_quant(_ptr(k), _ptr(v), rows, head_dim, _ptr(s), _ptr(kc),
                                           _ptr(ks), _ptr(vc), _ptr(vs), _stream())
    _check("rq_kv_rotate_quant", st)
    return kc, ks, vc, vs


def w4a4_linear(x: torch.Tensor, signs: torch.Tensor | None, w_codes: torch.Tensor,
                w_scales: torch.Tensor) -> torch.Tensor:
    """Online rotation + INT4 quantisation of x, then the W4A4 GEMM against
    weights folded with the same signs.  Two launches on the current stream."""
    codes, scales, _ = fwht_quant(x, signs)
    y, _ = w4a4_gemm(codes, scales, w_codes, w_scales)
    return y


def linear_decode_workspace(m: int, d: int, device) -> torch.Tensor:
    """A workspace for linear_decode (reusable across calls that do not
    overlap in time)."""
    nbytes = int(load_library().rq_linear_decode_workspace_size(m, d))
    return torch.empty((nbytes,), dtype=torch.uint8, device=device)


def linear_decode(x: torch.Tensor, signs: torch.Tensor | None, w_codes: torch.Tensor,
                  w_scales: torch.Tensor, workspace: torch.Tensor | None = None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """rq_linear_decode: rotation + INT4 quantisation of m <= 16 fp16 tokens
    and the decode GEMM in one call (one launch for m <= 4).  `workspace`
    comes from linear_decode_workspace (a fresh one is made when omitted)."""
    for name, t in (("x", x), ("w_codes", w_codes), ("w_scales", w_scales)):
        _need_cuda(name, t)
    if x.dtype != torch.float16 or x.dim() != 2:
        raise ValueError("x must be a float16 [m, d] tensor")
    if w_codes.dtype != torch.uint8 or w_scales.dtype != torch.float16:
        raise ValueError("weight codes must be uint8 and scales float16")
    x = x.contiguous()
    m, d = x.shape
    k, half_d = w_codes.shape
    if half_d * 2 != d or w_scales.numel() != k:
        raise ValueError("weight codes do not match x")
    s = _signs(signs, d, x.device)
    need = int(load_library().rq_linear_decode_workspace_size(m, d))
    ws = _workspace(workspace, need, x.device) if workspace is not None else \
        linear_decode_workspace(m, d, x.device)
    y = _out("out", out, (m, k), torch.float16, x.device)
    st = load_library().rq_linear_decode(_ptr(x), m, d, _ptr(s), _ptr(w_codes), _ptr(w_scales), k,
                                         _ptr(y), _ptr(ws), ws.numel(), _stream())
    _check("rq_linear_decode", st)
    return y


def linear_decode_noalloc(x: torch.Tensor, signs: torch.Tensor | None, w_codes: torch.Tensor,
                          w_scales: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """rq_linear_decode_noalloc: rq_linear_decode without a workspace (the
    library's own device array holds the codes; calls that overlap in time on
    one GPU race).  Nothing is allocated when `out` is given."""
    for name, t in (("x", x), ("w_codes", w_codes), ("w_scales", w_scales)):
        _need_cuda(name, t)
    if x.dtype != torch.float16 or x.dim() != 2:
        raise ValueError("x must be a float16 [m, d] tensor")
    if w_codes.dtype != torch.uint8 or w_scales.dtype != torch.float16:
        raise ValueError("weight codes must be uint8 and scales float16")
    m, d = x.shape
    k, half_d = w_codes.shape
    if half_d * 2 != d or w_scales.numel() != k:
        raise ValueError("weight codes do not match x")
    s = _signs(signs, d, x.device)
    y = _out("out", out, (m, k), torch.float16, x.device)
    st = load_library().rq_linear_decode_noalloc(_ptr(x), m, d, _ptr(s), _ptr(w_codes),
                                                 _ptr(w_scales), k, _ptr(y), _stream())
    _check("rq_linear_decode_noalloc", st)
    return y


def linear_decode_w4a8(x: torch.Tensor, signs: torch.Tensor | None, w_codes: torch.Tensor,
                       w_scales: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """rq_linear_decode_w4a8: rotation + per-token INT8 quantisation of m <= 4
    fp16 tokens and the W4A8 decode GEMM in one launch (y bit-identical to
    fwht_quant8 then w4a8_gemm)."""
    for name, t in (("x", x), ("w_codes", w_codes), ("w_scales", w_scales)):
        _need_cuda(name, t)
    if x.dtype != torch.float16 or x.dim() != 2:
        raise ValueError("x must be a float16 [m, d] tensor")
    if w_codes.dtype != torch.uint8 or w_scales.dtype != torch.float16:
        raise ValueError("weight codes must be uint8 and scales float16")
    m, d = x.shape
    k, half_d = w_codes.shape
    if half_d * 2 != d or w_scales.numel() != k:
        raise ValueError("weight codes do not match x")
    s = _signs(signs, d, x.device)
    y = _out("out", out, (m, k), torch.float16, x.device)
    st = load_library().rq_linear_decode_w4a8(_ptr(x), m, d, _ptr(s), _ptr(w_codes),
                                              _ptr(w_scales), k, _ptr(y), _stream())
    _check("rq_linear_decode_w4a8", st)
    return y


def fwht_quant8(x: torch.Tensor, signs: torch.Tensor | None = None, debug: bool = False,
                out=None):
    """rq_fwht_quant8 (W4A8 activations): returns (codes int8 [m, n],
    scales fp16 [m], x_rot fp32 or None)."""
    _need_cuda("x", x)
    if x.dtype != torch.float16 or x.dim() != 2:
        raise ValueError("x must be a float16 [rows, n] tensor")
    rows, n = x.shape
    s = _signs(signs, n, x.device)
    names = ("codes", "scales") + (("x_rot",) if debug else ())
    outs = _outs(names, ((rows, n), (rows,), (rows, n))[:len(names)],
                 (torch.int8, torch.float16, torch.float32)[:len(names)], x.device, out)
    codes, scales = outs[0], outs[1]
    rot = outs[2] if debug else None
    st = load_library().rq_fwht_quant8(_ptr(x), rows, n, _ptr(s), _ptr(codes), _ptr(scales),
                                       _ptr(rot), _stream())
    _check("rq_fwht_quant8", st)
    return codes, scales, rot


def w4a8_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
              w_scales: torch.Tensor, debug: bool = False, out: torch.Tensor | None = None,
              acc_out: torch.Tensor | None = None):
    """rq_w4a8_gemm: INT8 activation codes [m, d] times packed INT4 weight
    codes [k, d/2]; returns (y fp16 [m, k], acc int32 [m, k] or None)."""
    for name, t in (("a_codes", a_codes), ("a_scales", a_scales), ("w_codes", w_codes),
                    ("w_scales", w_scales)):
        _need_cuda(name, t)
    if a_codes.dtype != torch.int8 or w_codes.dtype != torch.uint8:
        raise ValueError("activation codes must be int8 and weight codes uint8")
    if a_scales.dtype != torch.float16 or w_scales.dtype != torch.float16:
        raise ValueError("scales must be float16")
    m, d = a_codes.shape
    k, half_d = w_codes.shape
    if d != 2 * half_d:
        raise ValueError("activation and weight codes differ in d")
    if a_scales.numel() != m or w_scales.numel() != k:
        raise ValueError("scale counts do not match the code rows")
    y = _out("out", out, (m, k), torch.float16, a_codes.device)
    acc = _out("acc_out", acc_out, (m, k), torch.int32, a_codes.device) if debug else None
    st = load_library().rq_w4a8_gemm(_ptr(a_codes), _ptr(a_scales), m, _ptr(w_codes),
                                     _ptr(w_scales), k, d, _ptr(y), _ptr(acc), _stream())
    _check("rq_w4a8_gemm", st)
    return y, acc


def w4a8_linear(x: torch.Tensor, signs: torch.Tensor | None, w_codes: torch.Tensor,
                w_scales: torch.Tensor) -> torch.Tensor:
    """Online rotation + INT8 quantisation of x, then the W4A8 GEMM against
    INT4 weights folded with the same signs.  Two launches."""
    codes, scales, _ = fwht_quant8(x, signs)
    y, _ = w4a8_gemm(codes, scales, w_codes, w_scales)
    return y


def fwht_quant_asym(x: torch.Tensor, signs: torch.Tensor | None = None, debug: bool = False,
                    out=None):
    """rq_fwht_quant_asym: returns (codes uint8 [m, n/2] unsigned nibbles,
    scales fp16 [m], zeros uint8 [m], x_rot fp32 or None)."""
    _need_cuda("x", x)
    if x.dtype != torch.float16 or x.dim() != 2:
        raise ValueError("x must be a float16 [rows, n] tensor")
    rows, n = x.shape
    s = _signs(signs, n, x.device)
    names = ("codes", "scales", "zeros") + (("x_rot",) if debug else ())
    outs = _outs(names, ((rows, n // 2), (rows,), (rows,), (rows, n))[:len(names)],
                 (torch.uint8, torch.float16, torch.uint8, torch.float32)[:len(names)], x.device,
                 out)
    codes, scales, zeros = outs[:3]
    rot = outs[3] if debug else None
    st = load_library().rq_fwht_quant_asym(_ptr(x), rows, n, _ptr(s), _ptr(codes), _ptr(scales),
                                           _ptr(zeros), _ptr(rot), _stream())
    _check("rq_fwht_quant_asym", st)
    return codes, scales, zeros, rot


def weight_code_sums(w_codes: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """rq_weight_code_sums: int32 [k] sums of the signed INT4 codes per row."""
    _need_cuda("w_codes", w_codes)
    if w_codes.dtype != torch.uint8 or w_codes.dim() != 2:
        raise ValueError("w_codes must be a uint8 [k, d/2] tensor")
    k, half_d = w_codes.shape
    sums = _out("out", out, (k,), torch.int32, w_codes.device)
    st = load_library().rq_weight_code_sums(_ptr(w_codes), k, 2 * half_d, _ptr(sums), _stream())
    _check("rq_weight_code_sums", st)
    return sums


def w4a4_gemm_asym(a_codes: torch.Tensor, a_scales: torch.Tensor, a_zeros: torch.Tensor,
                   w_codes: torch.Tensor, w_scales: torch.Tensor, w_sums: torch.Tensor,
                   debug: bool = False, out: torch.Tensor | None = None,
                   acc_out: torch.Tensor | None = None):
    """rq_w4a4_gemm_asym: returns (y fp16 [m, k], acc int32 [m, k] or None)."""
    for name, t in (("a_codes", a_codes), ("a_scales", a_scales), ("a_zeros", a_zeros),
                    ("w_codes", w_codes), ("w_scales", w_scales), ("w_sums", w_sums)):
        _need_cuda(name, t)
    if a_codes.dtype != torch.uint8 or w_codes.dtype != torch.uint8 or a_zeros.dtype != torch.uint8:
        raise ValueError("codes and zero points must be uint8")
    if w_sums.dtype != torch.int32:
        raise ValueError("w_sums must be int32")
    m, half_d = a_codes.shape
    k, half_d2 = w_codes.shape
    if half_d != half_d2 or a_scales.numel() != m or a_zeros.numel() != m or \
            w_scales.numel() != k or w_sums.numel() != k:
        raise ValueError("shapes do not match")
    y = _out("out", out, (m, k), torch.float16, a_codes.device)
    acc = _out("acc_out", acc_out, (m, k), torch.int32, a_codes.device) if debug else None
    st = load_library().rq_w4a4_gemm_asym(_ptr(a_codes), _ptr(a_scales), _ptr(a_zeros), m,
                                          _ptr(w_codes), _ptr(w_scales), _ptr(w_sums), k,
                                          2 * half_d, _ptr(y), _ptr(acc), _stream())
    _check("rq_w4a4_gemm_asym", st)
    return y, acc


def w4a4_linear_asym(x: torch.Tensor, signs: torch.Tensor | None, w_codes: torch.Tensor,
                     w_scales: torch.Tensor, w_sums: torch.Tensor) -> torch.Tensor:
    """Online rotation + asymmetric INT4 quantisation of x, then the GEMM."""
    codes, scales, zeros, _ = fwht_quant_asym(x, signs)
    y, _ = w4a4_gemm_asym(codes, scales, zeros, w_codes, w_scales, w_sums)
    return y


def quantize_groups(x: torch.Tensor, group: int = 128, out=None):
    """rq_quantize_groups on fp32 rows: returns (codes uint8 [rows, n/2],
    scales fp16 [rows, n / group])."""
    _need_cuda("x", x)
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be a float32 [rows, n] tensor")
    rows, n = x.shape
    codes, scales = _outs(("codes", "scales"), ((rows, n // 2), (rows, max(1, n // group))),
                          (torch.uint8, torch.float16), x.device, out)
    st = load_library().rq_quantize_groups(_ptr(x), rows, n, group, _ptr(codes), _ptr(scales),
                                           _stream())
    _check("rq_quantize_groups", st)
    return codes, scales


def fold_weights_grouped(wt: torch.Tensor, signs: torch.Tensor | None = None, group: int = 128):
    """Offline fold W~^T = W^T R (rq_fold_weights, fp32 rotated rows) followed
    by per-group INT4 (rq_quantize_groups): returns (codes [k, d/2],
    group scales [k, d / group])."""
    _, _, w_rot = fold_weights(wt, signs, debug=True)
    return quantize_groups(w_rot, group)


def w4a4_gemm_grouped(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
                      w_group_scales: torch.Tensor, out: torch.Tensor | None = None,
                      debug: bool = False, acc_out: torch.Tensor | None = None):
    """rq_w4a4_gemm_grouped (group 128): returns y fp16 [m, k], or with
    debug=True (y, acc int32 [m, k, d / 128]: every group's integer sum)."""
    for name, t in (("a_codes", a_codes), ("a_scales", a_scales), ("w_codes", w_codes),
                    ("w_group_scales", w_group_scales)):
        _need_cuda(name, t)
    if a_codes.dtype != torch.uint8 or w_codes.dtype != torch.uint8:
        raise ValueError("codes must be uint8")
    if a_scales.dtype != torch.float16 or w_group_scales.dtype != torch.float16:
        raise ValueError("scales must be float16")
    m, half_d = a_codes.shape
    k, half_d2 = w_codes.shape
    d = 2 * half_d
    if half_d != half_d2 or a_scales.numel() != m or w_group_scales.numel() != k * (d // 128):
        raise ValueError("shapes do not match")
    y = _out("out", out, (m, k), torch.float16, a_codes.device)
    acc = _out("acc_out", acc_out, (m, k, d // 128), torch.int32, a_codes.device) if debug else None
    st = load_library().rq_w4a4_gemm_grouped(_ptr(a_codes), _ptr(a_scales), m, _ptr(w_codes),
                                             _ptr(w_group_scales), k, d, _ptr(y), _ptr(acc),
                                             _stream())
    _check("rq_w4a4_gemm_grouped", st)
    return (y, acc) if debug else y


def decode_attention_workspace(batch: int, kv_heads: int, group: int, seq: int,
                               device) -> torch.Tensor:
    """A workspace for decode_attention (reusable across calls that do not
    overlap in time)."""
    nbytes = int(load_library().rq_decode_attention_workspace_size(batch, kv_heads, group, seq))
    return torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=device)


def decode_attention(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor,
                     v_codes: torch.Tensor, v_scales: torch.Tensor,
                     signs: torch.Tensor | None = None, lengths: torch.Tensor | None = None,
                     sm_scale: float | None = None, debug: bool = False,
                     workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     out_f32: torch.Tensor | None = None):
    """rq_decode_attention: q fp16 [B, H * G, 128] against the 4-bit rotated
    cache (codes [B, H, S, 64], scales [B, H, S] from kv_rotate_quant).
    Returns (out fp16 [B, H * G, 128], out fp32 or None)."""
    for name, t in (("q", q), ("k_codes", k_codes), ("k_scales", k_scales),
                    ("v_codes", v_codes), ("v_scales", v_scales)):
        _need_cuda(name, t)
    if q.dtype != torch.float16 or q.dim() != 3 or q.shape[-1] != 128:
        raise ValueError("q must be float16 [batch, query_heads, 128]")
    if k_codes.dtype != torch.uint8 or k_codes.dim() != 4 or k_codes.shape[-1] != 64:
        raise ValueError("k_codes must be uint8 [batch, kv_heads, seq, 64]")
    if v_codes.shape != k_codes.shape or k_scales.shape != k_codes.shape[:3] or \
            v_scales.shape != k_codes.shape[:3]:
        raise ValueError("cache shapes do not match")
    B, H, S, _ = k_codes.shape
    if q.shape[0] != B or q.shape[1] % H:
        raise ValueError("query heads must be a multiple of the KV heads")
    G = q.shape[1] // H
    s = _signs(signs, 128, q.device)
    if lengths is not None:
        _need_cuda("lengths", lengths)
        if lengths.dtype != torch.int32 or lengths.numel() != B:
            raise ValueError("lengths must be int32 [batch]")
    need = int(load_library().rq_decode_attention_workspace_size(B, H, G, S))
    ws = _workspace(workspace, need, q.device) if workspace is not None else \
        decode_attention_workspace(B, H, G, S, q.device)
    y = _out("out", out, tuple(q.shape), torch.float16, q.device)
    y32 = _out("out_f32", out_f32, tuple(q.shape), torch.float32, q.device) if debug else None
    scale = (1.0 / 128 ** 0.5) if sm_scale is None else float(sm_scale)
    st = load_library().rq_decode_attention(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                                            _ptr(v_scales), _ptr(lengths), B, H, G, S, 128, _ptr(s),
                                            scale, _ptr(y), _ptr(y32), _ptr(ws), ws.numel(),
                                            _stream())
    _check("rq_decode_attention", st)
    return y, y32
