"""GPU parity of decode attention over the 4-bit rotated KV cache
(rq_decode_attention through the C ABI) against the float64 oracle.

Tolerance, from the arithmetic: the output is a convex combination of the
dequantised value rows rotated back, o_j = sum_t p_t (v^_t R^T)_j, so a
relative error eps in the weights p moves o_j by at most
eps * max_t |(v^_t R^T)_j|.  The scores carry the query split into two f16
parts (about 2^-22 relative) and fp32 sums of about 128 products, the softmax
an fp32 exp2: eps is about 1e-5; the test allows 1e-4.  fp32 rounding in the
rotated basis adds at most about 2^-20 * sqrt(128) * max |v^| after the
inverse rotation.  The fp32 output must lie within the sum of the two; the
fp16 output additionally within its rounding, 2^-11 |o|.
"""

import sys

import numpy as np
import pytest

from oracle import rq_oracle as O
from rotation_w4a4_quantization_amd import datagen
from tests.guard import SENTINELS, Out, check_all

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

REL_V = 1e-4


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


def check_attention(q, kc, ks, vc, vs, signs, lengths, out16, out32, what, sm_scale=None):
    ref = O.decode_attention_int4(q, kc, ks, vc, vs, signs, lengths, sm_scale)["o"]
    B, H = kc.shape[:2]
    G = q.shape[1] // H
    vrot = O.dequantize(O.unpack_int4(vc), vs)                            # [B, H, S, 128]
    vback = np.abs(O.inverse_rotate(vrot, signs)).max(axis=2)             # [B, H, 128]
    tol = REL_V * np.repeat(vback, G, axis=1)
    tol = tol + 2.0 ** -20 * np.sqrt(128) * np.repeat(np.abs(vrot).max(axis=(2, 3)), G, axis=1)[..., None]
    err32 = np.abs(out32.astype(np.float64) - ref)
    assert np.all(err32 <= tol), f"{what}: fp32 output off by {float((err32 / tol).max()):.2f} x tol"
    err16 = np.abs(out16.astype(np.float64) - ref)
    assert np.all(err16 <= tol + 2.0 ** -11 * np.abs(ref)), f"{what}: fp16 output outside the tolerance"
    return float((err32 / tol).max())


def random_cache(rng, B, H, S):
    kc = rng.integers(0, 256, (B, H, S, 64), dtype=np.uint8)
    vc = rng.integers(0, 256, (B, H, S, 64), dtype=np.uint8)
    ks = rng.uniform(0.01, 0.3, (B, H, S)).astype(np.float16)
    vs = rng.uniform(0.01, 0.3, (B, H, S)).astype(np.float16)
    return kc, ks, vc, vs


def run(rq, q, kc, ks, vc, vs, signs=None, lengths=None, sm_scale=None, sentinel=0xFF):
    """One rq_decode_attention call into guarded, sentinel-filled outputs and
    workspace; the fp16 output of the launch without the fp32 copy (the one
    the benchmark times) must equal the debug launch's."""
    B, H, S, _ = kc.shape
    o = [Out(q.shape, torch.float16, sentinel), Out(q.shape, torch.float32, sentinel),
         Out((max(16, int(rq.load_library().rq_decode_attention_workspace_size(
             B, H, q.shape[1] // H, S))),), torch.uint8, sentinel)]
    args = (dev(q), dev(kc), dev(ks), dev(vc), dev(vs), None if signs is None else dev(signs),
            None if lengths is None else dev(np.asarray(lengths, np.int32)))
    rq.decode_attention(*args, sm_scale=sm_scale, debug=True, workspace=o[2].t, out=o[0].t,
                        out_f32=o[1].t)
    check_all(o, "attention")
    t = Out(q.shape, torch.float16, SENTINELS[1])
    rq.decode_attention(*args, sm_scale=sm_scale, workspace=o[2].t, out=t.t)
    check_all([t], "attention timed")
    assert np.array_equal(t.host().view(np.uint16), o[0].host().view(np.uint16))
    return o[0].host(), o[1].host()


@pytest.mark.parametrize("G", [1, 3, 4, 5, 8])
def test_attention_random_cache_ragged(rq, G):
    rng = np.random.default_rng(700 + G)
    B, H, S = 2, 3, 200   # 200: a ragged last 16-position tile and split
    kc, ks, vc, vs = random_cache(rng, B, H, S)
    q = rng.standard_normal((B, H * G, 128)).astype(np.float16)
    signs = datagen.rademacher(rng, 128)
    for sg, lens in ((signs, [200, 37]), (None, None)):
        say(f"attention G={G} signs={sg is not None} lengths={lens}")
        o16, o32 = run(rq, q, kc, ks, vc, vs, sg, lens)
        r = check_attention(q, kc, ks, vc, vs, sg, lens, o16, o32, f"G={G}")
        say(f"  max err / tol = {r:.3f}")


def test_attention_lengths_edge_cases(rq):
    rng = np.random.default_rng(71)
    B, H, G, S = 4, 2, 4, 130
    kc, ks, vc, vs = random_cache(rng, B, H, S)
    q = rng.standard_normal((B, H * G, 128)).astype(np.float16)
    lens = [0, 1, 130, 1000]   # empty, a single position, full, clamped to S
    say("attention lengths 0 / 1 / S / > S")
    o16, o32 = run(rq, q, kc, ks, vc, vs, None, lens)
    assert not o32[0].any() and not o16[0].view(np.uint16).any()
    check_attention(q, kc, ks, vc, vs, None, [0, 1, 130, 130], o16, o32, "lengths")
    # one position: the output is that value row, rotated back
    v0 = O.inverse_rotate(O.dequantize(O.unpack_int4(vc[1, :, 0]), vs[1, :, 0]), None)
    np.testing.assert_allclose(o32[1].reshape(H, G, 128), np.repeat(v0[:, None], G, 1),
                               atol=1e-5 * np.abs(v0).max())


def test_attention_smallest_cache_and_sm_scale(rq):
    rng = np.random.default_rng(72)
    kc, ks, vc, vs = random_cache(rng, 3, 2, 2)   # the smallest cache (seq even)
    q = rng.standard_normal((3, 4, 128)).astype(np.float16)
    for lens in (None, [1, 2, 1]):
        o16, o32 = run(rq, q, kc, ks, vc, vs, None, lens, sm_scale=0.5)
        check_attention(q, kc, ks, vc, vs, None, lens, o16, o32, f"S=2 lengths={lens}",
                        sm_scale=0.5)
    kc, ks, vc, vs = random_cache(rng, 2, 2, 300)
    q = (rng.standard_normal((2, 8, 128)) * 4).astype(np.float16)   # peaked softmax
    o16, o32 = run(rq, q, kc, ks, vc, vs, None, None, sm_scale=0.3)
    check_attention(q, kc, ks, vc, vs, None, None, o16, o32, "sm_scale 0.3", sm_scale=0.3)


def test_attention_reads_the_cache_kv_rotate_quant_writes(rq):
    # the bench cache statistics (outlier channels x20), rotated and
    # quantised on the GPU, then attended
    kv = datagen.kv_cache(0, batch=2, heads=4, seq=512)
    rng = np.random.default_rng(73)
    signs = datagen.rademacher(rng, 128)
    kc, ks, vc, vs = rq.kv_rotate_quant(dev(kv["k"]), dev(kv["v"]), dev(signs))
    q = rng.standard_normal((2, 16, 128)).astype(np.float16)
    say("attention over rq_kv_rotate_quant's cache")
    o16, o32 = rq.decode_attention(dev(q), kc, ks, vc, vs, dev(signs), debug=True)
    torch.cuda.synchronize()
    check_attention(q, host(kc), host(ks), host(vc), host(vs), signs, None, host(o16), host(o32),
                    "kv cache")
    # and the 4-bit rotated cache keeps attention much closer to full
    # precision than a 4-bit cache of the raw rows (outlier channels)
    ref = O.decode_attention(q, kv["k"], kv["v"])
    kq, kqs, _ = O.quantize_rows(kv["k"].astype(np.float64))
    vq, vqs, _ = O.quantize_rows(kv["v"].astype(np.float64))
    raw = O.decode_attention(q, O.dequantize(kq, kqs), O.dequantize(vq, vqs))
    rel = np.linalg.norm(host(o32) - ref) / np.linalg.norm(ref)
    rel_raw = np.linalg.norm(raw - ref) / np.linalg.norm(ref)
    say(f"  relative error vs fp attention: rotated {rel:.3f}, raw 4-bit {rel_raw:.3f}")
    assert rel < 0.5 * rel_raw


def test_attention_full_cache_sampled(rq):
    # the bench configuration [32, 8, 4096, 128], 4 query heads per KV head,
    # launched exactly as bench.py does; the oracle checks three batch entries
    kv = datagen.kv_cache(0)
    kc, ks, vc, vs = rq.kv_rotate_quant(dev(kv["k"]), dev(kv["v"]))
    del kv
    rng = np.random.default_rng(74)
    q = rng.standard_normal((32, 32, 128)).astype(np.float16)
    say("attention 32 x 8 x 4096, G = 4")
    oo = [Out(q.shape, torch.float16), Out(q.shape, torch.float32)]
    rq.decode_attention(dev(q), kc, ks, vc, vs, None, debug=True, out=oo[0].t, out_f32=oo[1].t)
    check_all(oo, "attention full")
    ot = Out(q.shape, torch.float16, SENTINELS[1])
    rq.decode_attention(dev(q), kc, ks, vc, vs, None, out=ot.t)  # the launch the benchmark times
    check_all([ot], "attention full timed")
    o16, o32 = oo[0].host(), oo[1].host()
    assert np.array_equal(ot.host().view(np.uint16), o16.view(np.uint16))
    for b in (0, 17, 31):
        check_attention(q[b:b + 1], host(kc[b:b + 1]), host(ks[b:b + 1]), host(vc[b:b + 1]),
                        host(vs[b:b + 1]), None, None, o16[b:b + 1], o32[b:b + 1], f"full b={b}")


@pytest.mark.parametrize("G", [1, 4, 8])
def test_attention_one_workgroup_per_kv_head(rq, G):
    # B * H a multiple of the CU count: one 12-wavefront workgroup per KV head
    # covers the whole sequence and writes the output itself (no combine);
    # signs, and lengths 0, 1, S and ragged ones
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H = 4
    if cus % H:
        pytest.skip(f"{cus} CUs: no whole number of batch entries per round")
    B, S = cus // H, 200
    rng = np.random.default_rng(90 + G)
    kc, ks, vc, vs = random_cache(rng, B, H, S)
    q = rng.standard_normal((B, H * G, 128)).astype(np.float16)
    signs = np.where(rng.random(128) < 0.5, -1, 1).astype(np.int8)
    lens = rng.integers(2, S + 1, B)
    lens[:3] = [0, 1, S]
    say(f"attention one workgroup per KV head B={B} H={H} G={G}")
    o16, o32 = run(rq, q, kc, ks, vc, vs, signs, lens)
    check_attention(q, kc, ks, vc, vs, signs, lens, o16, o32, f"fused G={G}")
