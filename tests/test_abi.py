"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/*.h declares, and rejects bad arguments on the host before any HIP
call (null pointers, shapes, alignment, dtype); the binding rejects output
and workspace tensors that do not fit the call before anything runs."""

import ctypes
import os
import re

import pytest

from rotation_w4a4_quantization_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("librq.so is not built (run python -m rotation_w4a4_quantization_amd.build)")
    return binding.load_library()


def declared_functions(header="rq.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", text)))


def all_headers():
    return sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))


def test_header_declares_the_bound_entry_points():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for h in all_headers():
        for name in declared_functions(h):
            assert hasattr(lib, name), (h, name)


def test_ceiling_probe_argument_errors(lib):
    lib.rq_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.rq_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.rq_ceiling_mfma_i8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    lib.rq_ceiling_mfma_i8.restype = ctypes.c_int64
    lib.rq_ceiling_mfma_out_words.argtypes = [ctypes.c_int64]
    lib.rq_ceiling_mfma_out_words.restype = ctypes.c_size_t
    assert lib.rq_ceiling_read(None, 16, A16, None) == 1
    assert lib.rq_ceiling_read(A16, 17, A16b, None) == 3
    assert lib.rq_ceiling_read(MIS, 16, A16b, None) == 3
    assert lib.rq_ceiling_read(A16, 0, A16b, None) == 0
    assert lib.rq_ceiling_copy(A16, None, 16, None) == 1
    assert lib.rq_ceiling_copy(A16, MIS, 16, None) == 3
    lib.rq_ceiling_mfma_f6.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    lib.rq_ceiling_mfma_f6.restype = ctypes.c_int64
    assert lib.rq_ceiling_mfma_f6(None, 2, 10, None) == -1
    assert lib.rq_ceiling_mfma_f6(A16, 0, 10, None) == -2
    assert lib.rq_ceiling_mfma_f6(A16, 2, 0, None) == -2
    assert lib.rq_ceiling_mfma_i8(None, 2, 10, None) == -1
    assert lib.rq_ceiling_mfma_i8(A16, 9, 10, None) == -2
    assert lib.rq_ceiling_mfma_i8(A16, 2, 0, None) == -2
    assert lib.rq_ceiling_mfma_out_words(0) == 0
    lib.rq_ceiling_issue.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p]
    lib.rq_ceiling_issue.restype = ctypes.c_int64
    lib.rq_ceiling_issue_out_words.argtypes = [ctypes.c_int64]
    lib.rq_ceiling_issue_out_words.restype = ctypes.c_size_t
    assert lib.rq_ceiling_issue(None, 0, 2, 10, None) == -1
    assert lib.rq_ceiling_issue(A16, 5, 2, 10, None) == -2
    assert lib.rq_ceiling_issue(A16, -1, 2, 10, None) == -2
    assert lib.rq_ceiling_issue(A16, 0, 0, 10, None) == -2
    assert lib.rq_ceiling_issue(A16, 0, 2, 0, None) == -2
    assert lib.rq_ceiling_issue(A16, 0, 2, (1 << 24) + 1, None) == -2
    assert lib.rq_ceiling_issue_out_words(9) == 0


def test_version_and_status_strings(lib):
    assert binding.version() == 10000
    for st in range(6):
        assert binding.status_string(st)
    assert binding.status_string(99) == "unknown status"


A16 = ctypes.c_void_p(0x10000)   # fake 16-byte aligned addresses: never dereferenced
A16b = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)


def fq(lib, x=A16, dtype=0, m=4, n=256, signs=None, codes=A16b, scales=A16b, rot=None):
    return lib.rq_fwht_quant(x, dtype, m, n, signs, codes, scales, rot, None)


def test_fwht_quant_argument_errors(lib):
    assert fq(lib, m=0) == binding.RQ_OK  # empty: no launch, no HIP call
    assert fq(lib, m=0, x=None) == binding.RQ_OK
    assert fq(lib, x=None) == binding.RQ_ERR_NULL
    assert fq(lib, codes=None) == binding.RQ_ERR_NULL
    assert fq(lib, scales=None) == binding.RQ_ERR_NULL
    assert fq(lib, n=3) == binding.RQ_ERR_SHAPE
    assert fq(lib, n=1) == binding.RQ_ERR_SHAPE
    assert fq(lib, n=16384) == binding.RQ_ERR_SHAPE
    assert fq(lib, n=28 * 2048) == binding.RQ_ERR_SHAPE   # 28 x 2^k beyond 28 x 1024
    assert fq(lib, n=28 * 256) == binding.RQ_ERR_SHAPE
    assert fq(lib, n=28672, x=None) == binding.RQ_ERR_NULL  # 28 x 1024 is a valid length
    assert fq(lib, n=0) == binding.RQ_ERR_SHAPE
    assert fq(lib, m=-1) == binding.RQ_ERR_SHAPE
    assert fq(lib, m=1 << 31) == binding.RQ_ERR_SHAPE
    assert fq(lib, dtype=7) == binding.RQ_ERR_DTYPE
    assert fq(lib, x=MIS) == binding.RQ_ERR_ALIGN
    assert fq(lib, codes=MIS) == binding.RQ_ERR_ALIGN
    assert fq(lib, signs=MIS) == binding.RQ_ERR_ALIGN
    assert fq(lib, rot=MIS) == binding.RQ_ERR_ALIGN


def test_fold_argument_errors(lib):
    f = lib.rq_fold_weights
    assert f(A16, 1, 0, 4096, None, A16b, A16b, None, None) == binding.RQ_OK
    assert f(None, 1, 8, 4096, None, A16b, A16b, None, None) == binding.RQ_ERR_NULL
    assert f(A16, 1, 8, 4095, None, A16b, A16b, None, None) == binding.RQ_ERR_SHAPE
    assert f(A16, 2, 8, 4096, None, A16b, A16b, None, None) == binding.RQ_ERR_DTYPE


def gemm(lib, a=A16, sa=A16b, m=4, w=A16, sw=A16b, k=64, d=4096, y=A16b, acc=None):
    return lib.rq_w4a4_gemm(a, sa, m, w, sw, k, d, y, acc, None, 0, None)


def test_gemm_argument_errors(lib):
    assert lib.rq_w4a4_gemm_workspace_size(2048, 28672, 8192) == 0
    assert gemm(lib, m=0) == binding.RQ_OK
    assert gemm(lib, a=None) == binding.RQ_ERR_NULL
    assert gemm(lib, y=None) == binding.RQ_ERR_NULL
    assert gemm(lib, sw=None) == binding.RQ_ERR_NULL
    assert gemm(lib, d=96) == binding.RQ_ERR_SHAPE
    assert gemm(lib, d=32) == binding.RQ_ERR_SHAPE
    assert gemm(lib, d=32768 + 64) == binding.RQ_ERR_SHAPE  # above RQ_MAX_D
    assert gemm(lib, d=28672, a=None) == binding.RQ_ERR_NULL  # the down-projection width is valid
    assert gemm(lib, k=0) == binding.RQ_ERR_SHAPE
    assert gemm(lib, m=-3) == binding.RQ_ERR_SHAPE
    assert gemm(lib, m=128 * 65536) == binding.RQ_ERR_SHAPE
    assert gemm(lib, a=MIS) == binding.RQ_ERR_ALIGN
    assert gemm(lib, w=MIS) == binding.RQ_ERR_ALIGN


def test_kv_argument_errors(lib):
    f = lib.rq_kv_rotate_quant
    args = [A16, A16, 10, 128, None, A16b, A16b, A16b, A16b, None]
    assert f(*args[:2], 0, *args[3:]) == binding.RQ_OK
    assert f(*args[:3], 64, *args[4:]) == binding.RQ_ERR_SHAPE
    assert f(None, *args[1:]) == binding.RQ_ERR_NULL
    assert f(*args[:6], None, *args[7:]) == binding.RQ_ERR_NULL
    assert f(MIS, *args[1:]) == binding.RQ_ERR_ALIGN
    assert f(*args[:4], MIS, *args[5:]) == binding.RQ_ERR_ALIGN


def test_fwht_quant8_argument_errors(lib):
    f = lib.rq_fwht_quant8

    def call(x=A16, m=4, n=4096, signs=None, codes=A16b, scales=A16b, rot=None):
        return f(x, m, n, signs, codes, scales, rot, None)

    assert call(m=0) == binding.RQ_OK
    assert call(m=0, x=None) == binding.RQ_OK
    assert call(x=None) == binding.RQ_ERR_NULL
    assert call(codes=None) == binding.RQ_ERR_NULL
    assert call(scales=None) == binding.RQ_ERR_NULL
    assert call(n=256) == binding.RQ_ERR_SHAPE      # below the smallest length
    assert call(n=14336) == binding.RQ_ERR_SHAPE    # 28 x 512 has no INT8 kernel
    assert call(n=16384) == binding.RQ_ERR_SHAPE
    assert call(n=3000) == binding.RQ_ERR_SHAPE
    assert call(m=-1) == binding.RQ_ERR_SHAPE
    assert call(x=MIS) == binding.RQ_ERR_ALIGN
    assert call(codes=MIS) == binding.RQ_ERR_ALIGN
    assert call(signs=MIS) == binding.RQ_ERR_ALIGN
    assert call(rot=MIS) == binding.RQ_ERR_ALIGN


def test_w4a8_gemm_argument_errors(lib):
    def call(a=A16, sa=A16b, m=4, w=A16, sw=A16b, k=64, d=4096, y=A16b, acc=None):
        return lib.rq_w4a8_gemm(a, sa, m, w, sw, k, d, y, acc, None)

    assert call(m=0) == binding.RQ_OK
    assert call(a=None) == binding.RQ_ERR_NULL
    assert call(sa=None) == binding.RQ_ERR_NULL
    assert call(y=None) == binding.RQ_ERR_NULL
    assert call(d=96) == binding.RQ_ERR_SHAPE
    assert call(d=32768 + 64) == binding.RQ_ERR_SHAPE
    assert call(k=0) == binding.RQ_ERR_SHAPE
    assert call(m=-1) == binding.RQ_ERR_SHAPE
    assert call(m=128 * 65536) == binding.RQ_ERR_SHAPE
    assert call(m=2 ** 63 - 1) == binding.RQ_ERR_SHAPE  # m + 127 would overflow
    assert call(a=MIS) == binding.RQ_ERR_ALIGN
    assert call(w=MIS) == binding.RQ_ERR_ALIGN


def test_f6_argument_errors(lib):
    def gemm(a=A16, sa=A16b, m=4, w=A16, sw=A16b, k=64, d=4096, y=A16b, acc=None):
        return lib.rq_w4a4_gemm_f6(a, sa, m, w, sw, k, d, y, acc, None)

    assert gemm(m=0) == binding.RQ_OK
    assert gemm(a=None) == binding.RQ_ERR_NULL
    assert gemm(sw=None) == binding.RQ_ERR_NULL
    assert gemm(y=None) == binding.RQ_ERR_NULL
    assert gemm(d=64) == binding.RQ_ERR_SHAPE      # d % 128 != 0
    assert gemm(d=4096 + 64) == binding.RQ_ERR_SHAPE
    assert gemm(d=32768 + 128) == binding.RQ_ERR_SHAPE
    assert gemm(k=0) == binding.RQ_ERR_SHAPE
    assert gemm(m=-1) == binding.RQ_ERR_SHAPE
    assert gemm(m=2 ** 63 - 1) == binding.RQ_ERR_SHAPE
    assert gemm(a=MIS) == binding.RQ_ERR_ALIGN
    assert gemm(w=MIS) == binding.RQ_ERR_ALIGN

    def pack(c=A16, rows=4, d=4096, out=A16b):
        return lib.rq_pack_f6(c, rows, d, out, None)

    assert pack(rows=0) == binding.RQ_OK
    assert pack(c=None) == binding.RQ_ERR_NULL
    assert pack(out=None) == binding.RQ_ERR_NULL
    assert pack(d=4096 + 64) == binding.RQ_ERR_SHAPE
    assert pack(d=32768 + 128) == binding.RQ_ERR_SHAPE
    assert pack(rows=-1) == binding.RQ_ERR_SHAPE
    assert pack(rows=2 ** 31) == binding.RQ_ERR_SHAPE
    assert pack(out=MIS) == binding.RQ_ERR_ALIGN


def test_linear_decode_argument_errors(lib):
    need = lib.rq_linear_decode_workspace_size(4, 4096)
    assert need == 4 * 2048 + 64
    # shapes the call rejects have no workspace size (and no overflowing one)
    for m, d in ((17, 4096), (4, 4095), (4, 16384), (4, 2 ** 62), (-1, 4096)):
        assert lib.rq_linear_decode_workspace_size(m, d) == 0, (m, d)

    def call(x=A16, m=4, d=4096, signs=None, w=A16, sw=A16b, k=64, y=A16b, ws=A16b,
             nbytes=need):
        return lib.rq_linear_decode(x, m, d, signs, w, sw, k, y, ws, nbytes, None)

    assert call(m=0) == binding.RQ_OK
    assert call(m=17) == binding.RQ_ERR_SHAPE
    assert call(d=256) == binding.RQ_ERR_SHAPE
    assert call(d=14336) == binding.RQ_ERR_SHAPE
    assert call(k=0) == binding.RQ_ERR_SHAPE
    assert call(nbytes=need - 1) == binding.RQ_ERR_SHAPE
    assert call(x=None) == binding.RQ_ERR_NULL
    assert call(ws=None) == binding.RQ_ERR_NULL
    assert call(x=MIS) == binding.RQ_ERR_ALIGN
    assert call(ws=MIS) == binding.RQ_ERR_ALIGN


def test_linear_decode_w4a8_argument_errors(lib):
    def call(x=A16, m=4, d=4096, signs=None, w=A16, sw=A16b, k=64, y=A16b):
        return lib.rq_linear_decode_w4a8(x, m, d, signs, w, sw, k, y, None)

    assert call(m=0) == binding.RQ_OK
    assert call(m=5) == binding.RQ_ERR_SHAPE  # one launch holds at most 4 tokens
    assert call(m=-1) == binding.RQ_ERR_SHAPE
    assert call(d=256) == binding.RQ_ERR_SHAPE
    assert call(d=3072) == binding.RQ_ERR_SHAPE
    assert call(d=16384) == binding.RQ_ERR_SHAPE
    assert call(k=0) == binding.RQ_ERR_SHAPE
    assert call(x=None) == binding.RQ_ERR_NULL
    assert call(w=None) == binding.RQ_ERR_NULL
    assert call(sw=None) == binding.RQ_ERR_NULL
    assert call(y=None) == binding.RQ_ERR_NULL
    assert call(x=MIS) == binding.RQ_ERR_ALIGN
    assert call(w=MIS) == binding.RQ_ERR_ALIGN
    assert call(signs=MIS) == binding.RQ_ERR_ALIGN


def test_asym_argument_errors(lib):
    f = lib.rq_fwht_quant_asym

    def fq(x=A16, m=4, n=4096, signs=None, codes=A16b, scales=A16b, zeros=A16b, rot=None):
        return f(x, m, n, signs, codes, scales, zeros, rot, None)

    assert fq(m=0) == binding.RQ_OK
    assert fq(x=None) == binding.RQ_ERR_NULL
    assert fq(zeros=None) == binding.RQ_ERR_NULL
    assert fq(n=256) == binding.RQ_ERR_SHAPE
    assert fq(n=14336) == binding.RQ_ERR_SHAPE
    assert fq(codes=MIS) == binding.RQ_ERR_ALIGN
    s = lib.rq_weight_code_sums
    assert s(A16, 0, 4096, A16b, None) == binding.RQ_OK
    assert s(None, 4, 4096, A16b, None) == binding.RQ_ERR_NULL
    assert s(A16, 4, 4096, None, None) == binding.RQ_ERR_NULL
    assert s(A16, 4, 96, A16b, None) == binding.RQ_ERR_SHAPE
    assert s(MIS, 4, 4096, A16b, None) == binding.RQ_ERR_ALIGN
    g = lib.rq_w4a4_gemm_asym

    def gemm(a=A16, sa=A16b, za=A16b, m=4, w=A16, sw=A16b, ws=A16b, k=64, d=4096, y=A16b):
        return g(a, sa, za, m, w, sw, ws, k, d, y, None, None)

    assert gemm(m=0) == binding.RQ_OK
    assert gemm(za=None) == binding.RQ_ERR_NULL
    assert gemm(ws=None) == binding.RQ_ERR_NULL
    assert gemm(d=96) == binding.RQ_ERR_SHAPE
    assert gemm(k=0) == binding.RQ_ERR_SHAPE
    assert gemm(a=MIS) == binding.RQ_ERR_ALIGN


def test_grouped_argument_errors(lib):
    q = lib.rq_quantize_groups
    assert q(A16, 0, 4096, 128, A16b, A16b, None) == binding.RQ_OK
    assert q(None, 4, 4096, 128, A16b, A16b, None) == binding.RQ_ERR_NULL
    assert q(A16, 4, 4096, 96, A16b, A16b, None) == binding.RQ_ERR_SHAPE
    assert q(A16, 4, 4000, 128, A16b, A16b, None) == binding.RQ_ERR_SHAPE
    assert q(A16, 4, 64, 128, A16b, A16b, None) == binding.RQ_ERR_SHAPE
    assert q(MIS, 4, 4096, 128, A16b, A16b, None) == binding.RQ_ERR_ALIGN
    g = lib.rq_w4a4_gemm_grouped
    assert g(A16, A16b, 0, A16, A16b, 64, 4096, A16b, None, None) == binding.RQ_OK
    assert g(A16, A16b, 4, A16, None, 64, 4096, A16b, None, None) == binding.RQ_ERR_NULL
    assert g(A16, A16b, 4, A16, A16b, 64, 192, A16b, None, None) == binding.RQ_ERR_SHAPE
    assert g(A16, A16b, 4, A16, A16b, 0, 4096, A16b, None, None) == binding.RQ_ERR_SHAPE
    assert g(MIS, A16b, 4, A16, A16b, 64, 4096, A16b, None, None) == binding.RQ_ERR_ALIGN


def test_decode_attention_argument_errors(lib):
    need = lib.rq_decode_attention_workspace_size(2, 8, 4, 4096)
    assert need > 0 and need % 16 == 0
    for shape in ((65536, 1, 4, 4096), (4096, 4096, 4, 4096), (2 ** 62, 2 ** 62, 4, 4096),
                  (2, 8, 9, 4096), (2, 8, 4, 4095), (2, 8, 4, 2 ** 40), (0, 8, 4, 4096)):
        assert lib.rq_decode_attention_workspace_size(*shape) == 0, shape

    def call(q=A16, kc=A16, ks=A16b, vc=A16, vs=A16b, lens=None, B=2, H=8, G=4, S=4096, D=128,
             signs=None, sm=0.088, out=A16b, out32=None, ws=A16b, nbytes=need):
        return lib.rq_decode_attention(q, kc, ks, vc, vs, lens, B, H, G, S, D, signs, sm, out,
                                       out32, ws, nbytes, None)

    assert call(B=0) == binding.RQ_OK
    assert call(D=64) == binding.RQ_ERR_SHAPE
    assert call(G=9) == binding.RQ_ERR_SHAPE
    assert call(G=0) == binding.RQ_ERR_SHAPE
    assert call(S=0) == binding.RQ_ERR_SHAPE
    assert call(S=4095) == binding.RQ_ERR_SHAPE      # odd: the scales move in pairs
    assert call(ks=ctypes.c_void_p(0x20002)) == binding.RQ_ERR_ALIGN
    assert call(sm=0.0) == binding.RQ_ERR_SHAPE
    assert call(sm=float("nan")) == binding.RQ_ERR_SHAPE
    assert call(nbytes=need - 1) == binding.RQ_ERR_SHAPE
    assert call(B=65536, H=1) == binding.RQ_ERR_SHAPE
    assert call(B=2 ** 62, H=65535) == binding.RQ_ERR_SHAPE  # the product would overflow
    assert call(q=None) == binding.RQ_ERR_NULL
    assert call(ws=None) == binding.RQ_ERR_NULL
    assert call(kc=MIS) == binding.RQ_ERR_ALIGN
    assert call(q=MIS) == binding.RQ_ERR_ALIGN


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        binding.fwht_quant(torch.zeros(4, 16, dtype=torch.float16))


def test_f6_binding_rejects_bad_inputs_before_launch():
    # host tensors, wrong dtypes and F6 layouts that are not [d/128, rows, 96]
    # raise ValueError on the host, before librq is called
    import torch
    with pytest.raises(ValueError):
        binding.pack_f6(torch.zeros(4, 64, dtype=torch.uint8))
    a6 = torch.zeros(2, 4, 96, dtype=torch.uint8)
    s4 = torch.zeros(4, dtype=torch.float16)
    with pytest.raises(ValueError):
        binding.w4a4_gemm_f6(a6, s4, a6, s4)


def test_binding_rejects_unfit_outputs_before_launch():
    """Caller-supplied outputs and workspaces are checked on the host: the
    wrong dtype, shape or layout, or a host tensor, raise ValueError (an
    undersized or strided output would otherwise be written past its end)."""
    import torch
    dev = "cuda"
    ok = torch.empty((4, 8), dtype=torch.float16)
    with pytest.raises(ValueError, match="float16"):
        binding._out("out", ok.float(), (4, 8), torch.float16, dev)
    with pytest.raises(ValueError, match="shape"):
        binding._out("out", torch.empty((4, 7), dtype=torch.float16), (4, 8), torch.float16, dev)
    with pytest.raises(ValueError, match="shape"):
        binding._out("out", torch.empty((32,), dtype=torch.float16), (4, 8), torch.float16, dev)
    with pytest.raises(ValueError):
        binding._out("out", ok, (4, 8), torch.float16, dev)  # a host tensor
    with pytest.raises(ValueError, match="torch.Tensor"):
        binding._out("out", [0] * 32, (4, 8), torch.float16, dev)
    with pytest.raises(ValueError, match="tuple"):
        binding._outs(("codes", "scales"), ((4, 8), (4,)), (torch.uint8, torch.float16), dev,
                      (None,))
    with pytest.raises(ValueError, match="uint8"):
        binding._workspace(torch.empty((64,), dtype=torch.int32), 16, dev)
    with pytest.raises(ValueError):
        binding._workspace(torch.empty((64,), dtype=torch.uint8), 16, dev)  # a host tensor
