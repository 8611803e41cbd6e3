"""Host-side checks of libhlwq (CPU only, no kernel is launched).

The library must load without a GPU, export every function include/hlwq.h
declares, carry exactly the oracle's codebook, and reject bad arguments with
the documented status codes before touching a device.
"""
import ctypes

import numpy as np
import pytest

import weight_quantization_amd as wq
from oracle import hlwq_ref as ref
from oracle import lloyd_max as lm
from oracle import tq3_ref as tq

OK, ENULL, ESHAPE, EBITS, EBLOCK, EDEV, EALIGN, ELIMIT, EOVERLAP = 0, -1, -2, -3, -4, -5, -6, -7, -8


@pytest.fixture(scope="module")
def lib():
    return wq.load_library()


def test_exports_every_declared_symbol(lib):
    names = wq.declared_functions()
    assert len(names) == 21
    raw = ctypes.CDLL(wq.binding.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), name


@pytest.mark.parametrize("bits", [5, 3])
def test_codebook_matches_oracle(bits):
    c, t = wq.hlwq_centroids(bits)
    oc, ot = lm.table(bits)
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(t.view(np.uint32), ot.view(np.uint32))


def _bucket_codes(buckets, entries, scale, bias, y):
    # u = fma(y, 2^-146, bias) lands on the denormal grid (spacing 2^-149), so
    # its bit pattern is the integer RN(8 y + bias), ties to even; 8 y + bias is
    # exact in fp64 whenever the rounding can be a tie, so np.rint reproduces it.
    assert scale == 2.0 ** -146
    y = np.asarray(y, np.float32)
    k = np.rint(8.0 * y.astype(np.float64) + bias).astype(np.int64)
    assert k.min() >= 0 and k.max() < buckets.size
    e = buckets[k].astype(np.int64)
    assert np.all(e % 8 == 0)
    thr = entries[e // 8, 0].view(np.float32)
    return entries[e // 8, 1].astype(np.int64) + (y > thr)


@pytest.mark.parametrize("kind,bits,limit", [(0, 5, 127.875), (1, 3, 127.875), (2, 3, 255.875), (3, 2, 255.875)])
def test_bucket_table_reproduces_threshold_count(kind, bits, limit):
    # The kernels find codes with two table reads and one compare; on every
    # fp32 value near a threshold or a bucket edge, and on a dense sweep of the
    # reachable range (|y| < 112 for weights, < 222 for KV vectors, even for
    # blocks whose squares underflow), that must equal the oracle's count.
    buckets, entries, scale, bias = wq.hlwq_search_table(kind)
    _, b32 = lm.table(bits)
    K = 1 << bits
    assert entries.shape == (K, 2) and np.array_equal(entries[:, 1], np.arange(K))
    assert np.array_equal(entries[:-1, 0].view(np.float32), b32) and np.isinf(entries[-1, 0].view(np.float32))
    assert buckets.size == 2 * bias and limit < bias / 8.0
    edges = (np.arange(buckets.size + 1) - bias - 0.5) / 8.0
    probes = np.concatenate([b32, edges]).astype(np.float32)
    steps = np.arange(-4096, 4097, dtype=np.int64)
    near = []
    for p in probes:
        bits_p = np.abs(p).view(np.int32).astype(np.int64) + steps
        v = bits_p[bits_p >= 0].astype(np.int32).view(np.float32)
        near.append(np.copysign(v, p) if p != 0 else np.concatenate([v, -v]))
    rng = np.random.default_rng(0)
    y = np.concatenate(near + [np.linspace(-limit, limit, 2_000_001, dtype=np.float32),
                               rng.standard_normal(200_000).astype(np.float32),
                               np.float32([0.0, -0.0, 2.0 ** -149, -2.0 ** -149])])
    y = y[np.abs(y) <= limit]
    assert np.array_equal(_bucket_codes(buckets, entries, scale, bias, y), ref.codes_from_y(y, b32))


def test_size_helpers():
    assert wq.hlwq_packed_bytes(64, 256, 128, 5) == 64 * 2 * 80
    assert wq.hlwq_packed_bytes(2816 * 128, 704, 128, 5) == 2816 * 128 * 6 * 80
    assert wq.hlwq_packed_bytes(10, 129, 128, 3) == 10 * 2 * 48
    assert wq.hlwq_norm_count(2816, 704, 128) == 2816 * 6
    assert wq.hlwq_packed_bytes(-1, 5, 128, 5) == 0
    assert wq.hlwq_norm_count(1, -5, 128) == 0
    assert wq.hlwq_packed_bytes(2 ** 62, 2 ** 40, 128, 5) == 0


def test_status_strings(lib):
    for st in (OK, ENULL, ESHAPE, EBITS, EBLOCK, EDEV, EALIGN, ELIMIT, EOVERLAP):
        assert wq.hlwq_status_string(st) != "unknown status"
    assert wq.hlwq_status_string(12345) == "unknown status"


def test_quantize_argument_errors(lib):
    q = lib.hlwq_quantize
    A = 0x100000  # an aligned, never-dereferenced address
    assert q(None, 1, 4, 128, 128, 5, A, A, None) == ENULL
    assert q(A, 1, 4, 128, 128, 5, None, A, None) == ENULL
    assert q(A, 1, 4, 128, 128, 4, A, A, None) == EBITS
    assert q(A, 1, 4, 128, 64, 5, A, A, None) == EBLOCK
    assert q(A, -1, 4, 128, 128, 5, A, A, None) == ESHAPE
    assert q(A, 1, 4, -3, 128, 5, A, A, None) == ESHAPE
    assert q(A, 2 ** 40, 2 ** 40, 128, 128, 5, A, A, None) == ESHAPE
    assert q(A, 1, 4, 128, 128, 5, A + 8, A, None) == EALIGN
    assert q(A, 1, 4, 128, 128, 5, A, A + 1, None) == EALIGN
    assert q(A + 1, 1, 4, 128, 128, 5, A, A, None) == EALIGN
    assert q(A, 1, 2 ** 31, 128 * 2, 128, 5, A, A, None) == ELIMIT
    # zero-sized work is a no-op and accepts NULL
    assert q(None, 0, 4, 128, 128, 5, None, None, None) == OK
    assert q(None, 1, 0, 128, 128, 5, None, None, None) == OK
    assert q(None, 1, 4, 0, 128, 5, None, None, None) == OK
    d = lib.hlwq_dequantize
    assert d(A, None, 1, 4, 128, 128, 5, A, None) == ENULL
    assert d(A, A, 1, 4, 128, 128, 6, A, None) == EBITS
    assert d(A, A, 1, 4, 128, 256, 5, A, None) == EBLOCK


def test_grouped_argument_errors(lib):
    A = 0x100000
    descs = (wq.MatDesc * 3)()
    descs[0] = wq.MatDesc(A, A, A, 4, 128)
    descs[1] = wq.MatDesc(A, None, A, 4, 128)
    descs[2] = wq.MatDesc(A, A, A, 4, 128)
    assert lib.hlwq_quantize_grouped(descs, 3, 5, None) == ENULL
    assert lib.hlwq_quantize_grouped(descs, -1, 5, None) == ESHAPE
    assert lib.hlwq_quantize_grouped(None, 2, 5, None) == ENULL
    assert lib.hlwq_quantize_grouped(None, 0, 5, None) == OK
    assert lib.hlwq_dequantize_grouped(descs, 3, 2, None) == EBITS
    descs[1] = wq.MatDesc(A, A, A, -4, 128)
    assert lib.hlwq_dequantize_grouped(descs, 3, 5, None) == ESHAPE
    empty = (wq.MatDesc * 2)()
    empty[0] = wq.MatDesc(None, None, None, 0, 128)
    empty[1] = wq.MatDesc(None, None, None, 7, 0)
    assert lib.hlwq_quantize_grouped(empty, 2, 3, None) == OK


def test_kv_argument_errors(lib):
    A = 0x100000
    kq, kd = lib.hlwq_kv_quantize, lib.hlwq_kv_dequantize
    assert kq(A, 1, 4, 300, 128, 3, 128, A, A, None) == EBLOCK
    assert kq(A, 1, 4, 300, 256, 5, 128, A, A, None) == EBITS
    assert kq(A, 1, 4, 300, 256, 4, 128, A, A, None) == EBITS
    assert kq(A, 1, 4, -1, 256, 3, 128, A, A, None) == ESHAPE
    assert kq(A, 1, 4, 300, 256, 3, -1, A, A, None) == ESHAPE
    assert kq(None, 1, 4, 300, 256, 3, 128, A, A, None) == ENULL
    assert kq(A, 1, 4, 300, 256, 3, 128, A + 4, A, None) == EALIGN
    assert kd(A, A, 1, 4, 300, 256, 3, 128, A + 1, None) == EALIGN
    assert kq(A + 2, 1, 4, 300, 256, 3, 128, A, A, None) == EALIGN
    assert kq(A, 1, 4, 300, 256, 3, 128, A, A + 1, None) == EALIGN
    # every token inside the residual window: nothing to do
    assert kq(None, 1, 4, 128, 256, 3, 128, None, None, None) == OK
    assert kd(None, None, 1, 4, 100, 256, 3, 128, None, None) == OK


def test_kv_append_argument_errors(lib):
    A = 0x100000
    ap = lib.hlwq_kv_append
    # new_kv, batch, heads, n_new, tokens, window, n_res, packed, norms, capacity, head_dim, bits, stream
    assert ap(A, 1, 4, 1, 500, A, 128, A, A, 400, 128, 3, None) == EBLOCK
    assert ap(A, 1, 4, 1, 500, A, 128, A, A, 400, 256, 5, None) == EBITS
    assert ap(A, 1, 4, -1, 500, A, 128, A, A, 400, 256, 3, None) == ESHAPE
    assert ap(A, 1, 4, 1, -5, A, 128, A, A, 400, 256, 3, None) == ESHAPE
    assert ap(A, 1, 4, 1, 500, A, -1, A, A, 400, 256, 3, None) == ESHAPE
    # token 372 leaves the window: capacity must reach 373
    assert ap(A, 1, 4, 1, 500, A, 128, A, A, 372, 256, 3, None) == ESHAPE
    assert ap(None, 1, 4, 1, 500, A, 128, A, A, 400, 256, 3, None) == ENULL
    assert ap(A, 1, 4, 1, 500, None, 128, A, A, 400, 256, 3, None) == ENULL
    assert ap(A, 1, 4, 1, 500, A, 128, None, A, 400, 256, 3, None) == ENULL
    assert ap(A + 8, 1, 4, 1, 500, A, 128, A, A, 400, 256, 3, None) == EALIGN
    assert ap(A, 1, 4, 1, 500, A + 8, 128, A, A, 400, 256, 3, None) == EALIGN
    assert ap(A, 1, 4, 1, 500, A, 128, A + 8, A, 400, 256, 3, None) == EALIGN
    assert ap(A, 1, 4, 1, 500, A, 128, A, A + 1, 400, 256, 2, None) == EALIGN
    # a launch of more than 2^32 - 1 work-items: one 64-lane wave per head
    # (decode path), or one wave per head for the ring of a longer append
    assert ap(A, 1, 2 ** 26, 1, 500, A, 128, A, A, 400, 256, 3, None) == ELIMIT
    assert ap(A, 1, 2 ** 26, 200, 500, A, 128, A, A, 600, 256, 3, None) == ELIMIT
    # more than 2^31 - 1 tokens of one head arriving and leaving in one call
    assert ap(A, 1, 1, 2 ** 31 + 200, 0, A, 128, A, A, 2 ** 31 + 72, 256, 3, None) == ELIMIT
    # nothing to append, or nobody to append to
    assert ap(None, 1, 4, 0, 500, None, 128, None, None, 0, 256, 3, None) == OK
    assert ap(None, 0, 4, 3, 500, None, 128, None, None, 0, 256, 3, None) == OK


def test_dequantize_int4_argument_errors(lib):
    A = 0x100000
    d4 = lib.hlwq_dequantize_int4
    # packed, norms, n_mats, out, in, block, bits, q4, scales, zeros, stream
    assert d4(A, A, 1, 4, 256, 64, 5, A, A, A, None) == EBLOCK
    assert d4(A, A, 1, 4, 256, 128, 4, A, A, A, None) == EBITS
    assert d4(A, A, 1, 4, 200, 128, 5, A, A, A, None) == ESHAPE   # not 128-aligned
    assert d4(A, A, -1, 4, 256, 128, 5, A, A, A, None) == ESHAPE
    assert d4(A, A, 1, 4, 256, 128, 5, A, A, None, None) == ENULL
    assert d4(A, A, 1, 4, 256, 128, 5, A + 8, A, A, None) == EALIGN
    assert d4(A, A, 1, 4, 256, 128, 5, A, A + 2, A, None) == EALIGN
    assert d4(A + 8, A, 1, 4, 256, 128, 5, A, A, A, None) == EALIGN
    assert d4(None, None, 1, 0, 256, 128, 5, None, None, None, None) == OK


def test_codes8_argument_errors(lib):
    A = 0x100000
    q, d = lib.hlwq_quantize_codes8, lib.hlwq_dequantize_codes8
    assert q(None, 1, 4, 128, 128, 5, A, A, None) == ENULL
    assert q(A, 1, 4, 128, 128, 4, A, A, None) == EBITS
    assert q(A, 1, 4, 128, 64, 5, A, A, None) == EBLOCK
    assert q(A, 1, 4, 128, 128, 5, A + 8, A, None) == EALIGN
    assert q(None, 0, 4, 128, 128, 5, None, None, None) == OK
    assert d(A, None, 1, 4, 128, 128, 5, A, None) == ENULL
    assert d(A, A, 1, 4, 128, 128, 6, A, None) == EBITS
    assert d(A, A, 1, -4, 128, 128, 5, A, None) == ESHAPE


def test_overlapping_buffers_are_refused(lib):
    # Every call below would write a buffer that shares bytes with another of
    # its buffers; each must be refused before anything is launched.  (Calls
    # whose buffers are disjoint would launch, so they are exercised on the
    # GPU with real tensors, not here.)
    A = 0x100000
    q, d = lib.hlwq_quantize, lib.hlwq_dequantize
    # 4 x 128 bf16 = 1024 bytes of W; 4 blocks: 320 bytes of Q5 codes, 8 of norms
    assert q(A, 1, 4, 128, 128, 5, A + 1008, A + 4096, None) == EOVERLAP   # codes over W's last 16 bytes
    assert q(A, 1, 4, 128, 128, 5, A + 4096, A + 1022, None) == EOVERLAP   # norms over W's last 2 bytes
    assert q(A + 16, 1, 4, 128, 128, 5, A, A + 4096, None) == EOVERLAP     # codes over W's first bytes
    assert q(A, 1, 4, 128, 128, 5, A + 4096, A + 4096 + 318, None) == EOVERLAP  # norms over the codes
    assert q(A, 1, 4, 128, 128, 5, A, A + 4096, None) == EOVERLAP          # in place
    assert d(A + 4096, A + 8192, 1, 4, 128, 128, 5, A + 4096 - 16, None) == EOVERLAP  # out over the codes
    assert d(A + 4096, A + 8192, 1, 4, 128, 128, 5, A + 7200, None) == EOVERLAP       # out over the norms
    assert lib.hlwq_quantize_codes8(A, 1, 4, 128, 128, 5, A + 4096, A + 4096 + 510, None) == EOVERLAP
    assert lib.hlwq_tq3_quantize(A, 1, 4, 128, 128, 42, A + 4096, A + 4096 + 188, None) == EOVERLAP
    # grouped: one matrix's output over another matrix's input
    descs = (wq.MatDesc * 2)()
    descs[0] = wq.MatDesc(A, A + 8192, A + 12288, 4, 128)
    descs[1] = wq.MatDesc(A + 16384, A + 512, A + 20480, 4, 128)
    assert lib.hlwq_quantize_grouped(descs, 2, 5, None) == EOVERLAP
    # grouped dequantize: two matrices written to overlapping outputs
    descs[1] = wq.MatDesc(A + 512, A + 24576, A + 28672, 4, 128)
    assert lib.hlwq_dequantize_grouped(descs, 2, 5, None) == EOVERLAP
    # KV [1, 4, 300, 256]: 614,400 bytes of bf16; 172 quantised tokens per head
    kq, kd = lib.hlwq_kv_quantize, lib.hlwq_kv_dequantize
    B = A + (1 << 20)
    assert kq(A, 1, 4, 300, 256, 3, 128, A + 614400 - 16, B, None) == EOVERLAP
    assert kq(A, 1, 4, 300, 256, 3, 128, B, B + 688 * 96 - 2, None) == EOVERLAP
    assert kd(B, B + (1 << 20), 1, 4, 300, 256, 3, 128, B - 614400 + 16, None) == EOVERLAP
    # append: the window over the new tokens, the codes over the norms
    ap = lib.hlwq_kv_append
    assert ap(A, 1, 4, 1, 500, A + 2048 - 16, 128, B, B + (1 << 16), 400, 256, 3, None) == EOVERLAP
    assert ap(A, 1, 4, 1, 500, A + 4096, 128, B, B + 1600 * 96 - 2, 400, 256, 3, None) == EOVERLAP
    # INT4 [4, 256]: 8 blocks; q4 512 bytes, scales 32, zeros 8
    d4 = lib.hlwq_dequantize_int4
    assert d4(A, A + 4096, 1, 4, 256, 128, 5, A + 640 - 16, A + 8192, A + 12288, None) == EOVERLAP
    assert d4(A, A + 4096, 1, 4, 256, 128, 5, A + 16384, A + 8192, A + 8192 + 28, None) == EOVERLAP


@pytest.mark.parametrize("seed", [0, 1, 42, 1234567, 2 ** 64 - 1])
def test_tq3_signs_match_oracle(seed):
    # two independent SplitMix64 implementations (C in the library, Python in
    # the oracle), both written from the generator's published definition
    d1, d2 = wq.hlwq_tq3_signs(seed)
    o1, o2 = tq.sign_vectors(seed)
    assert np.array_equal(d1, o1) and np.array_equal(d2, o2)


def test_tq3_argument_errors(lib):
    A = 0x100000
    q, d = lib.hlwq_tq3_quantize, lib.hlwq_tq3_dequantize
    assert lib.hlwq_tq3_signs(42, None) == ENULL
    assert q(None, 1, 4, 128, 128, 42, A, A, None) == ENULL
    assert q(A, 1, 4, 128, 64, 42, A, A, None) == EBLOCK
    assert q(A, 1, 4, 128, 128, 42, A + 8, A, None) == EALIGN
    assert q(A, 1, 4, 128, 128, 42, A, A + 2, None) == EALIGN  # fp32 norms: 4-byte aligned
    assert q(A, 1, -4, 128, 128, 42, A, A, None) == ESHAPE
    assert q(None, 0, 4, 128, 128, 42, None, None, None) == OK
    assert d(A, None, 1, 4, 128, 128, 42, A, None) == ENULL
    assert d(A, A + 2, 1, 4, 128, 128, 42, A, None) == EALIGN
    assert d(A, A, 1, 4, 200, 256, 42, A, None) == EBLOCK
    descs = (wq.MatDesc * 1)()
    descs[0] = wq.MatDesc(A, A, A + 2, 4, 128)
    assert lib.hlwq_tq3_quantize_grouped(descs, 1, 42, None) == EALIGN
    assert lib.hlwq_tq3_dequantize_grouped(None, 1, 42, None) == ENULL
    assert lib.hlwq_tq3_quantize_grouped(descs, -1, 42, None) == ESHAPE


def test_plain_c_client(tmp_path):
    # the header compiles as C and a C program can link and call the library
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.dirname(wq.binding.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(root, "include"),
                    os.path.join(root, "tests", "c_abi_check.c"), "-L", lib_dir, "-lhlwq",
                    "-Wl,-rpath," + lib_dir, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    # the product path has no fallback: without libhlwq.so every call raises
    monkeypatch.setattr(wq.binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        wq.binding.load_library(str(tmp_path / "libhlwq.so"))


def test_binding_rejects_host_tensors():
    # device memory only: a CPU tensor is refused before any library call
    import torch
    w = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device memory"):
        wq.hlwq_quantize(w, 5)
    with pytest.raises(ValueError, match="device memory"):
        wq.hlwq_tq3_quantize(w)
    with pytest.raises(TypeError):
        wq.hlwq_quantize(w.float(), 5)


def test_stream_probe_library_exports_and_validates():
    # libhlwq_stream (include/hlwq_stream.h) is bench.py's ceiling probe; it
    # loads without a GPU and rejects bad arguments before any HIP call
    import re
    from weight_quantization_amd import build as wqb
    text = re.sub(r"/\*.*?\*/", "", open(wqb.INCLUDE + "/hlwq_stream.h").read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(hlwq_[a-z_0-9]+)\s*\(", text)))
    assert names == ["hlwq_stream_mix"]
    s = ctypes.CDLL(wqb.STREAM_LIB)
    f = s.hlwq_stream_mix
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    buf = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation or has no work
    assert f(buf, buf, 16384, 5248, 10, 4, 1, None) == -3          # unknown variant
    assert f(buf, buf, 16384, 5248, 10, 0, 0, None) == -3          # workgroups per CU outside 1..4
    assert f(buf, buf, 16384, 5248, 10, 3, 1, None) == -2          # read unit too large for variant 3
    assert f(buf, buf, 100, 5248, 10, 0, 1, None) == -2            # not a multiple of 16
    assert f(buf, buf, 16384, 0, 10, 0, 1, None) == -2             # nothing written
    assert f(buf, buf, 16384, 65536, 10, 0, 1, None) == -2         # write unit above 32 KB
    assert f(None, buf, 16384, 5248, 10, 0, 1, None) == -1         # NULL
    assert f(ctypes.c_void_p(4100), buf, 16384, 5248, 10, 0, 1, None) == -6  # misaligned
    assert f(None, None, 16384, 5248, 0, 0, 1, None) == 0          # zero units: nothing to do
