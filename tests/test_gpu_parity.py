"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Bar: packed codes, fp16 norms and bf16 dequantised weights bit-identical to the
oracle's canonical fp32 tier on the same seeded inputs; against the fp64
definition tier, code flips only within 1e-5 of a decision boundary (fraction
< 1e-6) and dequantised weights within 1e-3 per unit of block norm.
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth
from oracle import hlwq_ref as ref
from oracle import lloyd_max as lm

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def wq():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import weight_quantization_amd as m
    m.load_library()
    return m


# The full-size tests check whole tensors against the oracle on a thread pool
# (the oracle is numpy, whose array operations release the GIL), one GPU's
# share of the host at most.
HOST_WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def host_map(fn, items):
    with ThreadPoolExecutor(HOST_WORKERS) as ex:
        return list(ex.map(fn, items))


def first_failure(results):
    """results: (key, ok...) tuples; the first one with a False, or None."""
    for r in results:
        if not all(r[1:]):
            return r
    return None


def to_dev(bits_u16: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_bits(t) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f16_bits(t) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check_matrix(wq, w_bits: np.ndarray, bits: int, label: str):
    """Quantize + dequantize one [rows, in] matrix on the GPU and compare bit for bit."""
    rows, n_in = w_bits.shape
    _say(label, "rows", rows, "in", n_in, "bits", bits)
    w = to_dev(w_bits)
    packed, norms = wq.hlwq_quantize(w, bits)
    out = wq.hlwq_dequantize(packed, norms, n_in, bits)
    torch.cuda.synchronize()
    op, on = ref.quantize_c(w_bits, bits)
    gp = packed.cpu().numpy()
    gn = f16_bits(norms)
    assert np.array_equal(gn, on.view(np.uint16)), f"{label}: fp16 norms differ"
    assert np.array_equal(gp, op), f"{label}: packed codes differ"
    od = ref.dequantize_c(op, on, n_in, bits)
    assert np.array_equal(bf16_bits(out), od), f"{label}: dequantised bf16 differs"


def test_linear_64x256_q5_matches_oracle_and_golden(wq):
    import json
    import os
    w_bits = synth.weight("linear_64x256", "W")
    check_matrix(wq, w_bits, 5, "linear_64x256")
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "linear_64x256_q5.json")))
    packed, norms = wq.hlwq_quantize(to_dev(w_bits), 5)
    assert bytes(packed.cpu().numpy().ravel()).hex() == g["packed_hex"]


@pytest.mark.parametrize("bits", [5, 3])
@pytest.mark.parametrize("n_in", [1, 7, 8, 64, 120, 127, 128, 129, 200, 256, 704, 1000])
def test_shapes_and_tails(wq, bits, n_in):
    rows = 300 if n_in <= 256 else 97
    w = synth.random_bf16((rows, n_in), seed=n_in, key=bits)
    check_matrix(wq, w, bits, f"shape-{n_in}")


@pytest.mark.parametrize("bits", [5, 3])
def test_many_tiles_with_outliers(wq, bits):
    w = synth.random_bf16((3001, 384), seed=5, outlier_frac=0.001, outlier_mult=20.0)
    check_matrix(wq, w, bits, "tiles-outliers")
    w = synth.random_bf16((257, 1536), seed=6, dist="student_t5")
    check_matrix(wq, w, bits, "tiles-t5")


def test_unaligned_rows(wq):
    # rows starting at odd element offsets take the element-wise path
    for n_in in (129, 255, 704):
        w_bits = synth.random_bf16((41, n_in), seed=n_in)
        base = torch.zeros(41 * n_in + 1, dtype=torch.bfloat16, device="cuda")
        base[1:] = to_dev(w_bits).reshape(-1)
        w = base[1:].view(41, n_in)
        assert w.data_ptr() % 16 != 0
        packed, norms = wq.hlwq_quantize(w, 5)
        outbuf = torch.zeros(41 * n_in + 1, dtype=torch.bfloat16, device="cuda")
        out = outbuf[1:].view(41, n_in)
        wq.hlwq_dequantize(packed, norms, n_in, 5, out=out)
        op, on = ref.quantize_c(w_bits, 5)
        assert np.array_equal(packed.cpu().numpy(), op)
        assert np.array_equal(f16_bits(norms), on.view(np.uint16))
        assert np.array_equal(bf16_bits(out), ref.dequantize_c(op, on, n_in, 5))
        assert bf16_bits(outbuf[:1])[0] == 0


def test_ragged_batches_touch_nothing_past_the_end(wq):
    # The last batch of a matrix is short, and rows of a tail-block matrix end
    # mid-batch: the staged loads must not pick up the bytes that follow the
    # input (NaN here), and the staged stores must not write past the outputs
    # (sentinels here), for quantize, dequantize and dequantize -> INT4.
    nan = 0x7FC0
    for rows, n_in in ((37, 256), (33, 704), (130, 1000), (5, 128)):
        nb = -(-n_in // 128)
        w_bits = synth.random_bf16((rows, n_in), seed=rows + n_in)
        base = torch.full(((rows + 9) * n_in,), float("nan"), dtype=torch.bfloat16, device="cuda")
        base[:rows * n_in] = to_dev(w_bits).reshape(-1)
        w = base[:rows * n_in].view(rows, n_in)
        pbuf = torch.full(((rows + 2) * nb * 80,), 0xA5, dtype=torch.uint8, device="cuda")
        nbuf = torch.full(((rows + 2) * nb,), -1.5, dtype=torch.float16, device="cuda")
        packed = pbuf[:rows * nb * 80].view(rows, nb, 80)
        norms = nbuf[:rows * nb].view(rows, nb)
        wq.hlwq_quantize(w, 5, packed=packed, norms=norms)
        obuf = torch.full(((rows + 3) * n_in,), -2.0, dtype=torch.bfloat16, device="cuda")
        out = obuf[:rows * n_in].view(rows, n_in)
        wq.hlwq_dequantize(packed, norms, n_in, 5, out=out)
        torch.cuda.synchronize()
        assert not np.any(bf16_bits(base[rows * n_in:]) != nan)
        op, on = ref.quantize_c(w_bits, 5)
        assert np.array_equal(packed.cpu().numpy(), op), (rows, n_in)
        assert np.array_equal(f16_bits(norms), on.view(np.uint16)), (rows, n_in)
        assert np.all(pbuf[rows * nb * 80:].cpu().numpy() == 0xA5), (rows, n_in)
        assert np.all(f16_bits(nbuf[rows * nb:]) == np.float16(-1.5).view(np.uint16)), (rows, n_in)
        assert np.array_equal(bf16_bits(out), ref.dequantize_c(op, on, n_in, 5)), (rows, n_in)
        assert np.all(bf16_bits(obuf[rows * n_in:]) == 0xC000), (rows, n_in)  # -2.0
        if n_in % 128 == 0:
            q4buf = torch.full(((rows + 2) * n_in // 2,), 0x5A, dtype=torch.uint8, device="cuda")
            q4 = q4buf[:rows * n_in // 2].view(rows, n_in // 2)
            _, sc, z = wq.hlwq_dequantize_int4(packed, norms, n_in, 5, q4=q4)
            torch.cuda.synchronize()
            eq, es, ez = ref.dequantize_to_int4_c(op, on, n_in, 5)
            assert np.array_equal(q4.cpu().numpy(), eq), (rows, n_in)
            assert np.array_equal(sc.cpu().numpy().view(np.uint32), es.view(np.uint32)), (rows, n_in)
            assert np.array_equal(z.cpu().numpy(), ez), (rows, n_in)
            assert np.all(q4buf[rows * n_in // 2:].cpu().numpy() == 0x5A), (rows, n_in)
    # KV: a token count whose last 16-token batch is short; with no window,
    # that batch's missing tokens lie past the cache, where NaN follows; the
    # outputs are followed by sentinels
    B, H, T = 1, 2, 128 + 37
    kv_bits = synth.random_bf16((B, H, T, 256), seed=11, sigma=1.0)
    kbuf = torch.full((B * H * T * 256 + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    kbuf[:B * H * T * 256] = to_dev(kv_bits).reshape(-1)
    kv = kbuf[:B * H * T * 256].view(B, H, T, 256)
    for bits, n_res in ((3, 128), (2, 0), (3, 0)):
        tq = T - n_res
        pk = torch.full(((B * H * tq + 3) * 32 * bits,), 0xA5, dtype=torch.uint8, device="cuda")
        nk = torch.full((B * H * tq + 3,), -1.5, dtype=torch.float16, device="cuda")
        p = pk[:B * H * tq * 32 * bits].view(B, H, tq, 32 * bits)
        n = nk[:B * H * tq].view(B, H, tq)
        wq.hlwq_kv_quantize(kv, n_residual=n_res, bits=bits, packed=p, norms=n)
        dbuf = torch.full((B * H * T * 256 + 4096,), -2.0, dtype=torch.bfloat16, device="cuda")
        dk = dbuf[:B * H * T * 256].view(B, H, T, 256)
        wq.hlwq_kv_dequantize(p, n, dk, n_residual=n_res, bits=bits)
        torch.cuda.synchronize()
        op, on = ref.kv_quantize_c(kv_bits, n_residual=n_res, bits=bits)
        assert np.array_equal(p.cpu().numpy(), op), (bits, n_res)
        assert np.array_equal(f16_bits(n), on.view(np.uint16)), (bits, n_res)
        assert np.all(pk[B * H * tq * 32 * bits:].cpu().numpy() == 0xA5), (bits, n_res)
        assert np.all(f16_bits(nk[B * H * tq:]) == np.float16(-1.5).view(np.uint16)), (bits, n_res)
        assert np.array_equal(bf16_bits(dk)[:, :, :tq], ref.kv_dequantize_c(op, on, bits=bits)), (bits, n_res)
        assert np.all(bf16_bits(dk)[:, :, tq:] == 0xC000), (bits, n_res)  # the window rows: -2.0, untouched
        assert np.all(bf16_bits(dbuf[B * H * T * 256:]) == 0xC000), (bits, n_res)


def _special_rows():
    f = synth.f32_to_bf16_bits
    rows = []
    z = np.zeros(256, np.float32)
    rows.append(z.copy())                                   # zero blocks
    oh = z.copy(); oh[37] = 0.03125; oh[128 + 5] = -3.0     # one-hot blocks
    rows.append(oh)
    rows.append(np.full(256, 0.015625, np.float32))         # constant
    rows.append(np.full(256, -7.5, np.float32))
    rng = np.random.default_rng(3)
    rows.append((rng.standard_normal(256) * 1e-30).astype(np.float32))   # squares underflow
    rows.append((rng.standard_normal(256) * 1e-20).astype(np.float32))
    rows.append((rng.standard_normal(256) * 2e3).astype(np.float32))     # norm near the fp16 limit
    mixed = (rng.standard_normal(256) * np.exp(rng.uniform(-40, 5, 256))).astype(np.float32)
    rows.append(mixed)
    neg0 = z.copy(); neg0[::2] = -0.0; neg0[7] = 1.0
    rows.append(neg0)
    alt = np.where(np.arange(256) % 2 == 0, 1.0, -1.0).astype(np.float32)
    rows.append(alt)
    rows.append(np.concatenate([underflow_vector(128), underflow_vector(128)[::-1]]))
    return f(np.stack(rows))


def underflow_vector(n):
    """One entry whose square rounds up to 2^-149 and n - 1 whose squares round
    to 0: the computed norm is far below the exact one, so |y| reaches about
    0.7 n, beyond sqrt(n)."""
    v = np.full(n, np.float32(255 / 256 * 2.0 ** -75))
    v[0] = np.float32(1.5 * 2.0 ** -75)
    return v


@pytest.mark.parametrize("bits", [5, 3])
def test_special_blocks(wq, bits):
    w = _special_rows()
    w[8, ::2] = 0x8000  # keep the negative zeros (rounding maps -0.0 to 0x8000 already)
    check_matrix(wq, w, bits, "special")


def test_grouped_launch_splits(wq):
    # 20 matrices of mixed shapes: two launches of up to 16 descriptors
    rng = np.random.default_rng(8)
    items, host = [], []
    for i in range(20):
        rows = int(rng.integers(1, 300))
        n_in = int(rng.choice([64, 128, 200, 512, 704]))
        wb = synth.random_bf16((rows, n_in), seed=100 + i)
        w = to_dev(wb)
        nb = -(-n_in // 128)
        p = torch.empty((rows, nb, 80), dtype=torch.uint8, device="cuda")
        n = torch.empty((rows, nb), dtype=torch.float16, device="cuda")
        items.append((w, p, n))
        host.append(wb)
    _say("grouped quantize, 20 matrices")
    wq.hlwq_quantize_grouped(items, 5)
    outs = [(torch.empty_like(w), p, n) for (w, p, n) in items]
    wq.hlwq_dequantize_grouped(outs, 5)
    torch.cuda.synchronize()
    for (w, p, n), (o, _, _), wb in zip(items, outs, host):
        op, on = ref.quantize_c(wb, 5)
        assert np.array_equal(p.cpu().numpy(), op)
        assert np.array_equal(f16_bits(n), on.view(np.uint16))
        assert np.array_equal(bf16_bits(o), ref.dequantize_c(op, on, wb.shape[1], 5))


@pytest.mark.parametrize("count", [1, 16, 17, 32, 33])
@pytest.mark.parametrize("bits", [5, 3])
def test_grouped_launch_descriptor_counts(wq, bits, count):
    # `count` non-empty matrices, with empty ones (0 rows or 0 columns, which
    # take no slot of a launch) between them: one launch holds 16, so 16 and
    # 32 fill their launches exactly and 17 and 33 leave one matrix for the
    # next.  Every matrix equal to the oracle after quantize and dequantize.
    rng = np.random.default_rng(900 + 10 * bits + count)
    items, host = [], []
    for i in range(count):
        if i % 5 == 2:  # an empty matrix before this one
            e = torch.empty((0, 256) if i % 2 else (7, 0), dtype=torch.bfloat16, device="cuda")
            ps, ns = wq.packed_shape(tuple(e.shape), bits)
            items.append((e, torch.empty(ps, dtype=torch.uint8, device="cuda"),
                          torch.empty(ns, dtype=torch.float16, device="cuda")))
            host.append(None)
        rows = int(rng.integers(1, 40))
        n_in = int(rng.choice([8, 64, 128, 200, 704]))
        wb = synth.random_bf16((rows, n_in), seed=1000 * bits + 37 * count + i)
        ps, ns = wq.packed_shape((rows, n_in), bits)
        items.append((to_dev(wb), torch.empty(ps, dtype=torch.uint8, device="cuda"),
                      torch.empty(ns, dtype=torch.float16, device="cuda")))
        host.append(wb)
    _say("grouped launch", count, "matrices, bits", bits)
    wq.hlwq_quantize_grouped(items, bits)
    outs = [(torch.empty_like(w), p, n) for (w, p, n) in items]
    wq.hlwq_dequantize_grouped(outs, bits)
    torch.cuda.synchronize()
    for (w, p, n), (o, _, _), wb in zip(items, outs, host):
        if wb is None:
            continue
        op, on = ref.quantize_c(wb, bits)
        assert np.array_equal(p.cpu().numpy(), op)
        assert np.array_equal(f16_bits(n), on.view(np.uint16))
        assert np.array_equal(bf16_bits(o), ref.dequantize_c(op, on, wb.shape[1], bits))


@pytest.mark.parametrize("bits", [5, 3])
def test_grouped_launch_mixed_paths(wq, bits):
    # one grouped launch whose matrices take every read path: whole aligned
    # blocks, aligned rows with a tail block, rows not 16-byte aligned (odd
    # column counts) and empty matrices, which the launch skips
    shapes = [(300, 512), (0, 256), (77, 37), (129, 704), (5, 0), (64, 129), (1, 1), (200, 1000)]
    items, host = [], []
    for i, (rows, n_in) in enumerate(shapes):
        wb = synth.random_bf16((rows, n_in), seed=700 + i, key=11, outlier_frac=0.01, outlier_mult=20.0)
        nb = -(-n_in // 128)
        items.append((to_dev(wb) if wb.size else torch.empty((rows, n_in), dtype=torch.bfloat16, device="cuda"),
                      torch.empty((rows, nb, 16 * bits), dtype=torch.uint8, device="cuda"),
                      torch.empty((rows, nb), dtype=torch.float16, device="cuda")))
        host.append(wb)
    _say("grouped mixed paths", bits)
    wq.hlwq_quantize_grouped(items, bits)
    outs = [(torch.empty_like(w), p, n) for (w, p, n) in items]
    wq.hlwq_dequantize_grouped(outs, bits)
    torch.cuda.synchronize()
    for (w, p, n), (o, _, _), wb in zip(items, outs, host):
        if wb.size == 0:
            continue
        op, on = ref.quantize_c(wb, bits)
        assert np.array_equal(p.cpu().numpy(), op), wb.shape
        assert np.array_equal(f16_bits(n), on.view(np.uint16)), wb.shape
        assert np.array_equal(bf16_bits(o), ref.dequantize_c(op, on, wb.shape[1], bits)), wb.shape


def test_binding_rejects_another_device(wq, monkeypatch):
    # the library launches on the current device, so tensors or a stream of
    # another device are refused before any call (one GPU here: the other
    # device is faked)
    w = to_dev(synth.random_bf16((4, 256), seed=3))
    other = w.device.index + 1

    class OtherStream:
        device_index = other
        cuda_stream = 0

    with pytest.raises(ValueError, match="stream is on"):
        wq.hlwq_quantize(w, 5, stream=OtherStream())
    monkeypatch.setattr(torch.cuda, "current_device", lambda: other)
    with pytest.raises(ValueError, match="a tensor is on"):
        wq.hlwq_quantize(w, 5, stream=OtherStream())


def test_non_default_stream_and_determinism(wq):
    wb = synth.random_bf16((512, 2048), seed=12)
    w = to_dev(wb)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        p1, n1 = wq.hlwq_quantize(w, 5)
    s.synchronize()
    p2, n2 = wq.hlwq_quantize(w, 5)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(n1, n2)
    op, on = ref.quantize_c(wb, 5)
    assert np.array_equal(p1.cpu().numpy(), op)


def _carve(buf, offset, nbytes, dtype, shape):
    """A view of nbytes of the uint8 buffer at offset, as dtype / shape."""
    offset, nbytes = int(offset), int(nbytes)
    return buf[offset:offset + nbytes].view(dtype).view(shape)


def test_buffers_back_to_back_in_one_allocation(wq):
    # Inputs and outputs that touch (each starts where the previous one ends)
    # are distinct buffers and must be accepted; so must one input shared by
    # two matrices of a grouped call.  Every result is checked bit for bit.
    rows, n_in = 64, 704  # tail blocks: 6 blocks per row, 384 blocks
    wb = synth.random_bf16((rows, n_in), seed=55, outlier_frac=0.001, outlier_mult=20.0)
    nblk = rows * 6
    sizes = [rows * n_in * 2, nblk * 80, nblk * 2, rows * n_in * 2]
    offs = np.cumsum([0] + sizes)
    buf = torch.zeros(int(offs[-1]), dtype=torch.uint8, device="cuda")
    w = _carve(buf, offs[0], sizes[0], torch.bfloat16, (rows, n_in))
    packed = _carve(buf, offs[1], sizes[1], torch.uint8, (rows, 6, 80))
    norms = _carve(buf, offs[2], sizes[2], torch.float16, (rows, 6))
    out = _carve(buf, offs[3], sizes[3], torch.bfloat16, (rows, n_in))
    w.copy_(to_dev(wb))
    wq.hlwq_quantize(w, 5, packed=packed, norms=norms)
    wq.hlwq_dequantize(packed, norms, n_in, 5, out=out)
    torch.cuda.synchronize()
    op, on = ref.quantize_c(wb, 5)
    assert np.array_equal(packed.cpu().numpy(), op) and np.array_equal(f16_bits(norms), on.view(np.uint16))
    assert np.array_equal(bf16_bits(out), ref.dequantize_c(op, on, n_in, 5))
    assert np.array_equal(bf16_bits(w), wb), "the input must stay as it was"

    # one W read by both matrices of a grouped call
    p2, n2 = torch.empty_like(packed), torch.empty_like(norms)
    p3, n3 = torch.empty_like(packed), torch.empty_like(norms)
    wq.hlwq_quantize_grouped([(w, p2, n2), (w, p3, n3)], 5)
    torch.cuda.synchronize()
    for p_, n_ in ((p2, n2), (p3, n3)):
        assert np.array_equal(p_.cpu().numpy(), op) and np.array_equal(f16_bits(n_), on.view(np.uint16))

    # KV cache, codes and norms back to back; dequantized into the cache itself
    B, H, T = 1, 3, 300
    kvb = synth.random_bf16((B, H, T, 256), seed=56, sigma=1.0)
    tq = T - 128
    ks = [B * H * T * 512, B * H * tq * 96, B * H * tq * 2]
    ko = np.cumsum([0] + ks)
    kbuf = torch.zeros(int(ko[-1]), dtype=torch.uint8, device="cuda")
    kv = _carve(kbuf, ko[0], ks[0], torch.bfloat16, (B, H, T, 256))
    kp = _carve(kbuf, ko[1], ks[1], torch.uint8, (B, H, tq, 96))
    kn = _carve(kbuf, ko[2], ks[2], torch.float16, (B, H, tq))
    kv.copy_(to_dev(kvb))
    wq.hlwq_kv_quantize(kv, n_residual=128, packed=kp, norms=kn)
    wq.hlwq_kv_dequantize(kp, kn, kv, n_residual=128)
    torch.cuda.synchronize()
    okp, okn = ref.kv_quantize_c(kvb, n_residual=128)
    assert np.array_equal(kp.cpu().numpy(), okp) and np.array_equal(f16_bits(kn), okn.view(np.uint16))
    got = bf16_bits(kv)
    assert np.array_equal(got[:, :, :tq], ref.kv_dequantize_c(okp, okn))
    assert np.array_equal(got[:, :, tq:], kvb[:, :, tq:])

    # INT4 outputs back to back after their inputs
    n4 = 512
    w4 = synth.random_bf16((rows, n4), seed=57)
    op4, on4 = ref.quantize_c(w4, 5)
    nb4 = rows * 4
    s4 = [nb4 * 80, nb4 * 2, rows * n4 // 2, nb4 * 4, nb4]
    o4 = np.cumsum([0] + s4)
    ibuf = torch.zeros(int(o4[-1]), dtype=torch.uint8, device="cuda")
    ip = _carve(ibuf, o4[0], s4[0], torch.uint8, (rows, 4, 80))
    inn = _carve(ibuf, o4[1], s4[1], torch.float16, (rows, 4))
    q4 = _carve(ibuf, o4[2], s4[2], torch.uint8, (rows, n4 // 2))
    sc = _carve(ibuf, o4[3], s4[3], torch.float32, (rows, 4))
    zp = _carve(ibuf, o4[4], s4[4], torch.uint8, (rows, 4))
    ip.copy_(torch.from_numpy(op4).cuda())
    inn.copy_(torch.from_numpy(on4.view(np.int16)).view(torch.float16).cuda())
    wq.hlwq_dequantize_int4(ip, inn, n4, 5, q4=q4, scales=sc, zeros=zp)
    torch.cuda.synchronize()
    e4, es, ez = ref.dequantize_to_int4_c(op4, on4, n4, 5)
    assert np.array_equal(q4.cpu().numpy(), e4)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), es.view(np.uint32))
    assert np.array_equal(zp.cpu().numpy(), ez)


def test_in_place_calls_are_refused(wq):
    # a call whose output overlaps another of its buffers is refused on the
    # host (status -8, nothing launched) and leaves every byte as it was
    rows, n_in = 16, 256
    wb = synth.random_bf16((rows, n_in), seed=58)
    wbytes = rows * n_in * 2
    buf = torch.zeros(wbytes + 8192, dtype=torch.uint8, device="cuda")
    w = _carve(buf, 0, wbytes, torch.bfloat16, (rows, n_in))
    w.copy_(to_dev(wb))
    good_p, good_n = wq.hlwq_quantize(w, 5)
    torch.cuda.synchronize()
    before = buf.clone()

    def refused(call):
        with pytest.raises(wq.HLWQError) as e:
            call()
        assert e.value.status == -8
        torch.cuda.synchronize()
        assert torch.equal(buf, before)

    # codes over the last KB of W; norms over W's last bytes
    refused(lambda: wq.hlwq_quantize(w, 5, packed=_carve(buf, wbytes - 1024, rows * 160, torch.uint8, (rows, 2, 80)),
                                     norms=torch.empty((rows, 2), dtype=torch.float16, device="cuda")))
    refused(lambda: wq.hlwq_quantize(w, 5, packed=torch.empty((rows, 2, 80), dtype=torch.uint8, device="cuda"),
                                     norms=_carve(buf, wbytes - 2, rows * 4, torch.float16, (rows, 2))))
    # dequantize into a region that covers its own codes
    codes = _carve(buf, wbytes, rows * 160, torch.uint8, (rows, 2, 80))
    codes.copy_(good_p)
    before = buf.clone()
    refused(lambda: wq.hlwq_dequantize(codes, good_n, n_in, 5, out=_carve(buf, 4096, wbytes, torch.bfloat16,
                                                                            (rows, n_in))))
    # a KV cache dequantized over its own codes
    kv = _carve(buf, 0, 1 * 1 * 16 * 512, torch.bfloat16, (1, 1, 16, 256))
    refused(lambda: wq.hlwq_kv_dequantize(_carve(buf, 4096, 8 * 96, torch.uint8, (1, 1, 8, 96)),
                                          torch.empty((1, 1, 8), dtype=torch.float16, device="cuda"), kv,
                                          n_residual=8))


@pytest.mark.parametrize("shape", [(1, 2, 300), (2, 3, 1000), (1, 1, 129), (1, 4, 128), (1, 1, 5)])
def test_kv_cache_small(wq, shape):
    B, H, T = shape
    kv = synth.random_bf16((B, H, T, 256), seed=T, sigma=1.0)
    _say("kv", shape)
    dev = to_dev(kv)
    packed, norms = wq.hlwq_kv_quantize(dev, n_residual=128)
    out = to_dev(np.full((B, H, T, 256), 0x3F80, np.uint16))  # 1.0 sentinel
    wq.hlwq_kv_dequantize(packed, norms, out, n_residual=128)
    torch.cuda.synchronize()
    op, on = ref.kv_quantize_c(kv, n_residual=128)
    assert np.array_equal(packed.cpu().numpy(), op)
    assert np.array_equal(f16_bits(norms), on.view(np.uint16))
    tq = max(T - 128, 0)
    got = bf16_bits(out)
    assert np.array_equal(got[:, :, :tq], ref.kv_dequantize_c(op, on))
    assert np.all(got[:, :, tq:] == 0x3F80), "residual window must stay untouched"


@pytest.mark.parametrize("nbt", [1, 2, 3, 5, 7, 64, 333])
def test_kv_batches_per_head(wq, nbt):
    # the kernels map a batch index to (head, first token) by dividing by the
    # batches per head on the scalar unit: head counts and token counts that
    # give every residue, a short last batch per head and power-of-two and
    # odd divisors
    B, H = 1, 9
    T = 128 + 16 * nbt - (3 if nbt > 1 else 0)
    kv = synth.random_bf16((B, H, T, 256), seed=1000 + nbt, sigma=1.0)
    _say("kv batches per head", nbt, T)
    dev = to_dev(kv)
    packed, norms = wq.hlwq_kv_quantize(dev, n_residual=128)
    out = to_dev(np.full((B, H, T, 256), 0x3F80, np.uint16))
    wq.hlwq_kv_dequantize(packed, norms, out, n_residual=128)
    torch.cuda.synchronize()
    op, on = ref.kv_quantize_c(kv, n_residual=128)
    assert np.array_equal(packed.cpu().numpy(), op)
    assert np.array_equal(f16_bits(norms), on.view(np.uint16))
    tq = T - 128
    got = bf16_bits(out)
    assert np.array_equal(got[:, :, :tq], ref.kv_dequantize_c(op, on))
    assert np.all(got[:, :, tq:] == 0x3F80)


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("tq", [1, 15, 16, 17, 31, 32, 33])
def test_kv_token_counts_at_batch_edges(wq, bits, tq):
    # quantised tokens per head just below, at and above multiples of the
    # 16-token batch, behind a 100-token window: last batches of 1, 15 and 16
    # tokens; 3 heads x 2 batch entries, so heads start mid-launch
    B, H, T = 2, 3, tq + 100
    kv = synth.random_bf16((B, H, T, 256), seed=4000 + 10 * tq + bits, sigma=1.0)
    _say("kv batch edges", tq, "bits", bits)
    dev = to_dev(kv)
    packed, norms = wq.hlwq_kv_quantize(dev, n_residual=100, bits=bits)
    out = to_dev(np.full((B, H, T, 256), 0x3F80, np.uint16))
    wq.hlwq_kv_dequantize(packed, norms, out, n_residual=100, bits=bits)
    torch.cuda.synchronize()
    op, on = ref.kv_quantize_c(kv, n_residual=100, bits=bits)
    assert np.array_equal(packed.cpu().numpy(), op)
    assert np.array_equal(f16_bits(norms), on.view(np.uint16))
    got = bf16_bits(out)
    assert np.array_equal(got[:, :, :tq], ref.kv_dequantize_c(op, on, bits=bits))
    assert np.all(got[:, :, tq:] == 0x3F80)


@pytest.mark.parametrize("shape", [(1, 2, 300), (2, 3, 129), (1, 1, 1000)])
def test_kv_cache_q2(wq, shape):
    B, H, T = shape
    kv = synth.random_bf16((B, H, T, 256), seed=T + 2, sigma=1.0)
    _say("kv q2", shape)
    dev = to_dev(kv)
    packed, norms = wq.hlwq_kv_quantize(dev, n_residual=128, bits=2)
    out = to_dev(np.full((B, H, T, 256), 0x3F80, np.uint16))
    wq.hlwq_kv_dequantize(packed, norms, out, n_residual=128, bits=2)
    torch.cuda.synchronize()
    op, on = ref.kv_quantize_c(kv, n_residual=128, bits=2)
    assert np.array_equal(packed.cpu().numpy(), op)
    assert np.array_equal(f16_bits(norms), on.view(np.uint16))
    tq = max(T - 128, 0)
    got = bf16_bits(out)
    assert np.array_equal(got[:, :, :tq], ref.kv_dequantize_c(op, on, bits=2))
    assert np.all(got[:, :, tq:] == 0x3F80)


def _append_case(wq, B, H, chunks, n_res, bits, seed, extra=3):
    """Stream `chunks` tokens through hlwq_kv_append and compare the cache with
    the oracle's token-by-token stream after the last call."""
    T = sum(chunks)
    kv = synth.random_bf16((B, H, T, 256), seed=seed, sigma=1.0)
    cap = max(T - n_res, 0) + extra
    packed = torch.full((B, H, cap, 32 * bits), 0xAB, dtype=torch.uint8, device="cuda")
    norms = torch.full((B, H, cap), 7.0, dtype=torch.float16, device="cuda")
    window = to_dev(np.full((B, H, n_res, 256), 0x3F80, np.uint16)) if n_res else None
    tokens, parts = 0, []
    for n in chunks:
        part = kv[:, :, tokens:tokens + n]
        parts.append(part)
        tokens = wq.hlwq_kv_append(to_dev(part), window, packed, norms, tokens, n_residual=n_res, bits=bits)
    torch.cuda.synchronize()
    op, on, ow = ref.kv_stream_c(parts, n_residual=n_res, bits=bits)
    tq = op.shape[2]
    got_p, got_n = packed.cpu().numpy(), f16_bits(norms)
    assert np.array_equal(got_p[:, :, :tq], op)
    assert np.array_equal(got_n[:, :, :tq], on.view(np.uint16))
    assert np.all(got_p[:, :, tq:] == 0xAB), "codes past the encoded tokens must stay untouched"
    assert np.all(got_n[:, :, tq:] == np.float16(7.0).view(np.uint16))
    if n_res:
        w = bf16_bits(window)
        kept = ow.shape[2]
        for i in range(kept):
            t = T - kept + i
            assert np.array_equal(w[:, :, t % n_res], ow[:, :, i]), f"ring slot of token {t}"


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("chunks,n_res", [((1,) * 150, 128), ((100, 1, 1, 60, 3, 200, 1), 128), ((300,), 128),
                                          ((5, 40, 1), 0), ((3, 1, 2, 70), 1), ((33, 64, 31, 1), 32)])
def test_kv_append_matches_token_stream(wq, bits, chunks, n_res):
    _say("kv append", bits, chunks[:8], n_res)
    _append_case(wq, 2, 3, chunks, n_res, bits, seed=len(chunks) * 10 + n_res + bits)


@pytest.mark.parametrize("case", range(12))
def test_kv_random_shapes(wq, case):
    # seeded random cache shapes, residual windows, value scales and bit
    # widths through quantize and dequantize
    rng = np.random.default_rng(3000 + case)
    B, H, T = int(rng.integers(1, 4)), int(rng.integers(1, 6)), int(rng.integers(1, 700))
    n_res = int(rng.choice([0, 1, 7, 128, 200]))
    bits = int(rng.choice([3, 2]))
    sigma = float(np.exp(rng.uniform(-12, 4)))
    kv = synth.random_bf16((B, H, T, 256), seed=4000 + case, key=9, sigma=sigma)
    _say("kv random", case, (B, H, T), "n_res", n_res, "bits", bits, f"{sigma:.3g}")
    dev = to_dev(kv)
    packed, norms = wq.hlwq_kv_quantize(dev, n_residual=n_res, bits=bits)
    out = to_dev(np.full((B, H, T, 256), 0x3F80, np.uint16))
    wq.hlwq_kv_dequantize(packed, norms, out, n_residual=n_res, bits=bits)
    torch.cuda.synchronize()
    op, on = ref.kv_quantize_c(kv, n_residual=n_res, bits=bits)
    assert np.array_equal(packed.cpu().numpy(), op)
    assert np.array_equal(f16_bits(norms), on.view(np.uint16))
    tq = max(T - n_res, 0)
    got = bf16_bits(out)
    assert np.array_equal(got[:, :, :tq], ref.kv_dequantize_c(op, on, bits=bits))
    assert np.all(got[:, :, tq:] == 0x3F80)


@pytest.mark.parametrize("case", range(6))
def test_kv_append_random_chunkings(wq, case):
    # seeded random chunkings (single tokens, decode-sized and prefill-sized
    # chunks mixed) and windows through the streaming append
    rng = np.random.default_rng(5000 + case)
    n_res = int(rng.choice([1, 5, 32, 128]))
    sizes = [1, 2, 8, 9, 16, 33, 100, 300]
    chunks = tuple(int(rng.choice(sizes)) for _ in range(int(rng.integers(2, 9))))
    bits = int(rng.choice([3, 2]))
    _say("kv append random", case, chunks, "n_res", n_res, "bits", bits)
    _append_case(wq, int(rng.integers(1, 3)), int(rng.integers(1, 4)), chunks, n_res, bits, seed=6000 + case)


def test_kv_cache_underflow_vectors(wq):
    f = synth.f32_to_bf16_bits
    kv = synth.random_bf16((1, 2, 200, 256), seed=77, sigma=1.0)
    kv[0, 0, 3] = f(underflow_vector(256))
    kv[0, 1, 71] = f(-underflow_vector(256)[::-1])
    _say("kv underflow vectors")
    dev = to_dev(kv)
    packed, norms = wq.hlwq_kv_quantize(dev, n_residual=128)
    out = torch.empty_like(dev)
    wq.hlwq_kv_dequantize(packed, norms, out, n_residual=128)
    torch.cuda.synchronize()
    op, on = ref.kv_quantize_c(kv, n_residual=128)
    assert np.array_equal(packed.cpu().numpy(), op)
    assert np.array_equal(f16_bits(norms), on.view(np.uint16))
    assert np.array_equal(bf16_bits(out)[:, :, :72], ref.kv_dequantize_c(op, on))


@pytest.mark.parametrize("bits", [5, 3])
@pytest.mark.parametrize("shape", [(1, 7, 128), (1, 100, 256), (3, 40, 1024), (1, 3001, 384)])
def test_dequantize_int4(wq, bits, shape):
    E, rows, n_in = shape
    wb = synth.random_bf16((E * rows, n_in), seed=rows + bits, dist="student_t5", sigma=0.02, outlier_frac=0.002,
                           outlier_mult=20.0)
    _say("dequantize -> int4", bits, shape)
    packed, norms = wq.hlwq_quantize(to_dev(wb).view(E, rows, n_in), bits)
    q4, scales, zeros = wq.hlwq_dequantize_int4(packed, norms, n_in, bits)
    torch.cuda.synchronize()
    op, on = ref.quantize_c(wb, bits)
    p4, s4, z4 = ref.dequantize_to_int4_c(op, on, n_in, bits)
    assert np.array_equal(q4.cpu().numpy().reshape(E * rows, -1), p4)
    assert np.array_equal(scales.cpu().numpy().reshape(E * rows, -1).view(np.uint32), s4.view(np.uint32))
    assert np.array_equal(zeros.cpu().numpy().reshape(E * rows, -1), z4)


@pytest.mark.parametrize("bits", [5, 3])
@pytest.mark.parametrize("shape", [(1, 64, 256), (1, 300, 704), (2, 33, 129), (1, 2001, 8)])
def test_codes8(wq, bits, shape):
    E, rows, n_in = shape
    wb = synth.random_bf16((E * rows, n_in), seed=rows + n_in + bits, dist="student_t5")
    _say("codes8", bits, shape)
    codes, norms = wq.hlwq_quantize_codes8(to_dev(wb).view(E, rows, n_in), bits)
    out = wq.hlwq_dequantize_codes8(codes, norms, n_in, bits)
    # only the low `bits` bits of a code byte count
    junk = codes | torch.tensor(0xE0 if bits == 5 else 0xF8, dtype=torch.uint8, device="cuda")
    out2 = wq.hlwq_dequantize_codes8(junk, norms, n_in, bits)
    torch.cuda.synchronize()
    oc, on = ref.quantize_codes8_c(wb, bits)
    assert np.array_equal(codes.cpu().numpy().reshape(oc.shape), oc)
    assert np.array_equal(f16_bits(norms).reshape(on.shape), on.view(np.uint16))
    want = ref.dequantize_codes8_c(oc, on, n_in, bits)
    assert np.array_equal(bf16_bits(out).reshape(want.shape), want)
    assert np.array_equal(bf16_bits(out2).reshape(want.shape), want)


@pytest.mark.parametrize("bits", [5, 3])
def test_dequantize_int4_grouped(wq, bits):
    # 20 matrices of mixed shapes (a few empty) in one call: split over two
    # launches of at most 16, each matrix equal to the oracle and to the
    # single-matrix entry point
    rng = np.random.default_rng(40 + bits)
    host, items = [], []
    for i in range(20):
        rows = 0 if i in (3, 11) else int(rng.integers(1, 300))
        n_in = 128 * int(rng.integers(1, 9))
        wb = synth.random_bf16((rows, n_in), seed=500 + i, outlier_frac=0.001, outlier_mult=20.0)
        nb = n_in // 128
        packed, norms = wq.hlwq_quantize(to_dev(wb), bits)
        items.append((packed, norms, torch.empty((rows, n_in // 2), dtype=torch.uint8, device="cuda"),
                      torch.empty((rows, nb), dtype=torch.float32, device="cuda"),
                      torch.empty((rows, nb), dtype=torch.uint8, device="cuda")))
        host.append(wb)
    _say("int4 grouped, 20 matrices, bits", bits)
    wq.hlwq_dequantize_int4_grouped(items, bits)
    torch.cuda.synchronize()
    for (p, n, q4, sc, z), wb in zip(items, host):
        if wb.shape[0] == 0:
            continue
        op, on = ref.quantize_c(wb, bits)
        assert np.array_equal(p.cpu().numpy(), op)
        p4, s4, z4 = ref.dequantize_to_int4_c(op, on, wb.shape[1], bits)
        assert np.array_equal(q4.cpu().numpy(), p4)
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), s4.view(np.uint32))
        assert np.array_equal(z.cpu().numpy(), z4)
        q1, s1, z1 = wq.hlwq_dequantize_int4(p, n, wb.shape[1], bits)
        torch.cuda.synchronize()
        assert torch.equal(q1, q4) and torch.equal(s1, sc) and torch.equal(z1, z)


def test_dequantize_int4_special_blocks(wq):
    w = _special_rows()
    w[8, ::2] = 0x8000
    packed, norms = wq.hlwq_quantize(to_dev(w), 5)
    q4, scales, zeros = wq.hlwq_dequantize_int4(packed, norms, 256, 5)
    torch.cuda.synchronize()
    op, on = ref.quantize_c(w, 5)
    p4, s4, z4 = ref.dequantize_to_int4_c(op, on, 256, 5)
    assert np.array_equal(q4.cpu().numpy(), p4)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s4.view(np.uint32))
    assert np.array_equal(zeros.cpu().numpy(), z4)


# --------------------------------------------------------------------------
# full-size workloads, launched as the benchmark launches them; every output
# compared with the oracle
# --------------------------------------------------------------------------

def _bank_check(wq, config, bits):
    tensors = list(synth.CONFIGS[config])
    host = {t: synth.weight(config, t) for t in tensors}
    _say(config, "generated", {t: host[t].shape for t in tensors})
    items, outs = [], []
    for t in tensors:
        w = to_dev(host[t])
        E, rows, n_in = host[t].shape
        nb = -(-n_in // 128)
        p = torch.empty((E, rows, nb, 16 * bits), dtype=torch.uint8, device="cuda")
        n = torch.empty((E, rows, nb), dtype=torch.float16, device="cuda")
        items.append((w, p, n))
    wq.hlwq_quantize_grouped(items, bits)
    for (w, p, n) in items:
        outs.append((torch.empty_like(w), p, n))
    wq.hlwq_dequantize_grouped(outs, bits)
    torch.cuda.synchronize()
    _say(config, "gpu done; checking every expert on", HOST_WORKERS, "host threads")
    for t, (w, p, n), (o, _, _) in zip(tensors, items, outs):
        gp, gn, go = p.cpu().numpy(), f16_bits(n), bf16_bits(o)
        wb_all = host[t]

        def check(e):
            op, on = ref.quantize_c(wb_all[e], bits)
            od = ref.dequantize_c(op, on, wb_all.shape[2], bits)
            return (e, np.array_equal(gp[e], op), np.array_equal(gn[e], on.view(np.uint16)),
                    np.array_equal(go[e], od))

        bad = first_failure(host_map(check, range(wb_all.shape[0])))
        assert bad is None, (config, t, "expert, codes ok, norms ok, dequant ok:", bad)
        _say(config, t, "all", wb_all.shape[0], "experts bit-exact")
    del items, outs
    torch.cuda.empty_cache()


def test_qwen36_moe_bank_full(wq):
    _bank_check(wq, "qwen36_moe_bank", 5)


def test_gemma4_moe_bank_full(wq):
    _bank_check(wq, "gemma4_moe_bank", 5)


def _row_chunks(rows, size=512):
    return [(r, min(r + size, rows)) for r in range(0, rows, size)]


@pytest.mark.parametrize("bits", [5, 3])
def test_dense_5120_full(wq, bits):
    for t in synth.CONFIGS["dense_5120"]:
        wb = synth.weight("dense_5120", t)
        _say("dense_5120", t, wb.shape, "bits", bits)
        w = to_dev(wb)
        packed, norms = wq.hlwq_quantize(w, bits)
        out = wq.hlwq_dequantize(packed, norms, wb.shape[1], bits)
        torch.cuda.synchronize()
        gp, gn, go = packed.cpu().numpy(), f16_bits(norms), bf16_bits(out)
        del w, packed, norms, out

        def check(rc):
            r0, r1 = rc
            op, on = ref.quantize_c(wb[r0:r1], bits)
            od = ref.dequantize_c(op, on, wb.shape[1], bits)
            return (rc, np.array_equal(gp[r0:r1], op), np.array_equal(gn[r0:r1], on.view(np.uint16)),
                    np.array_equal(go[r0:r1], od))

        bad = first_failure(host_map(check, _row_chunks(wb.shape[0])))
        assert bad is None, ("dense_5120", t, bits, bad)


@pytest.mark.parametrize("bits", [5, 3])
def test_dense_5120_int4_full(wq, bits):
    # the INT4 workload of the benchmark: every dense matrix, one
    # dequantize-to-INT4 launch each, every row checked
    for t in synth.CONFIGS["dense_5120"]:
        wb = synth.weight("dense_5120", t)
        _say("dense_5120 int4", t, wb.shape, "bits", bits)
        packed, norms = wq.hlwq_quantize(to_dev(wb), bits)
        q4, scales, zeros = wq.hlwq_dequantize_int4(packed, norms, wb.shape[1], bits)
        torch.cuda.synchronize()
        gp, gn = packed.cpu().numpy(), f16_bits(norms)
        g4, gs, gz = q4.cpu().numpy(), scales.cpu().numpy().view(np.uint32), zeros.cpu().numpy()
        del packed, norms, q4, scales, zeros

        def check(rc):
            r0, r1 = rc
            op, on = ref.quantize_c(wb[r0:r1], bits)
            p4, s4, z4 = ref.dequantize_to_int4_c(op, on, wb.shape[1], bits)
            return (rc, np.array_equal(gp[r0:r1], op), np.array_equal(gn[r0:r1], on.view(np.uint16)),
                    np.array_equal(g4[r0:r1], p4), np.array_equal(gs[r0:r1], s4.view(np.uint32)),
                    np.array_equal(gz[r0:r1], z4))

        bad = first_failure(host_map(check, _row_chunks(wb.shape[0])))
        assert bad is None, ("dense_5120 int4", t, bits, bad)


@pytest.mark.parametrize("bits", [3, 2])
def test_kv_h256_full(wq, bits):
    # K and V stacked as one [2, 4, 32768, 256] tensor and encoded by one
    # launch, as the benchmark does; every quantised token of every head checked
    kv = np.concatenate([synth.kv_cache("kv_h256", t) for t in ("K", "V")], axis=0)
    B, H, T, D = kv.shape
    _say("kv_h256 K+V", kv.shape, "bits", bits)
    dev = to_dev(kv)
    packed, norms = wq.hlwq_kv_quantize(dev, n_residual=128, bits=bits)
    out = torch.empty_like(dev)
    out[:, :, -128:] = dev[:, :, -128:]
    wq.hlwq_kv_dequantize(packed, norms, out, n_residual=128, bits=bits)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, -128:], dev[:, :, -128:])
    gp, gn, go = packed.cpu().numpy(), f16_bits(norms), bf16_bits(out)
    del dev, packed, norms, out
    tq = T - 128

    def check(job):
        b, h, t0, t1 = job
        codes, _, n16, _ = ref.quantize_vectors_c(ref.bf16_to_f32(kv[b, h, t0:t1]), bits)
        od = ref.f32_to_bf16_rne(ref.dequantize_vectors_c(codes, n16, bits))
        return (job, np.array_equal(gp[b, h, t0:t1], ref.pack_codes(codes, bits)),
                np.array_equal(gn[b, h, t0:t1], n16.view(np.uint16)), np.array_equal(go[b, h, t0:t1], od))

    jobs = [(b, h, t0, min(t0 + 2048, tq)) for b in range(B) for h in range(H) for t0 in range(0, tq, 2048)]
    bad = first_failure(host_map(check, jobs))
    assert bad is None, ("kv_h256", bits, bad)


@pytest.mark.parametrize("bits", [3, 2])
def test_kv_decode_full(wq, bits):
    # the benchmark's decode step: K and V caches [2, 4, 32768, 256] with a
    # 128-token window, then single-token appends; the tokens that leave the
    # window and the window itself are checked against the oracle
    kv = np.concatenate([synth.kv_cache("kv_h256", t) for t in ("K", "V")], axis=0)
    B, H, T, D = kv.shape
    steps = 3
    new = synth.random_bf16((B, H, steps, D), seed=5, sigma=1.0)
    _say("kv decode full", bits)
    dev = to_dev(kv)
    cap = T - 128 + steps
    packed = torch.empty((B, H, cap, 32 * bits), dtype=torch.uint8, device="cuda")
    norms = torch.empty((B, H, cap), dtype=torch.float16, device="cuda")
    p0, n0 = wq.hlwq_kv_quantize(dev, n_residual=128, bits=bits)
    packed[:, :, :T - 128] = p0
    norms[:, :, :T - 128] = n0
    window = torch.empty((B, H, 128, D), dtype=torch.bfloat16, device="cuda")
    for t in range(T - 128, T):
        window[:, :, t % 128] = dev[:, :, t]
    tokens = T
    for i in range(steps):
        tokens = wq.hlwq_kv_append(to_dev(new[:, :, i:i + 1]), window, packed, norms, tokens, bits=bits)
    torch.cuda.synchronize()
    left = kv[:, :, T - 128:T - 128 + steps]
    codes, _, n16, _ = ref.quantize_vectors_c(ref.bf16_to_f32(left), bits)
    assert np.array_equal(packed[:, :, T - 128:].cpu().numpy(), ref.pack_codes(codes, bits))
    assert np.array_equal(f16_bits(norms[:, :, T - 128:]), n16.view(np.uint16))
    assert np.array_equal(packed[:, :, :T - 128].cpu().numpy()[:, :, ::997], p0.cpu().numpy()[:, :, ::997])
    w = bf16_bits(window)
    for t in range(T - 128 + steps, T + steps):
        want = kv[:, :, t] if t < T else new[:, :, t - T]
        assert np.array_equal(w[:, :, t % 128], want), t


@pytest.mark.parametrize("bits", [3, 2])
def test_kv_prefill_append_full(wq, bits):
    # the whole K + V prompt [2, 4, 32768, 256] appended to an empty streaming
    # cache in one call, the tokens that leave the window in two calls split
    # mid-batch, and the static quantization of the same cache (itself checked
    # against the oracle): identical codes and norms, and the ring holds the
    # newest 128 tokens
    kv = np.concatenate([synth.kv_cache("kv_h256", t) for t in ("K", "V")], axis=0)
    B, H, T, D = kv.shape
    _say("kv prefill append", bits)
    dev = to_dev(kv)
    p0, n0 = wq.hlwq_kv_quantize(dev, n_residual=128, bits=bits)
    for split in (T, 12345):
        window = torch.zeros((B, H, 128, D), dtype=torch.bfloat16, device="cuda")
        packed = torch.zeros((B, H, T, 32 * bits), dtype=torch.uint8, device="cuda")
        norms = torch.zeros((B, H, T), dtype=torch.float16, device="cuda")
        tokens = wq.hlwq_kv_append(dev[:, :, :split].contiguous(), window, packed, norms, 0, bits=bits)
        if split < T:
            tokens = wq.hlwq_kv_append(dev[:, :, split:].contiguous(), window, packed, norms, tokens, bits=bits)
        torch.cuda.synchronize()
        assert tokens == T
        assert torch.equal(packed[:, :, :T - 128], p0) and torch.equal(norms[:, :, :T - 128], n0), split
        assert not packed[:, :, T - 128:].any() and not norms[:, :, T - 128:].any(), "rows past the encoded tokens"
        w = bf16_bits(window)
        for t in (T - 128, T - 127, T - 2, T - 1):
            assert np.array_equal(w[:, :, t % 128], kv[:, :, t]), t
    sl = kv[1:2, 3:4, 20000:20512]
    op, on = ref.kv_quantize_c(np.concatenate([sl, np.zeros((1, 1, 128, 256), np.uint16)], axis=2),
                               n_residual=128, bits=bits)
    assert np.array_equal(p0[1:2, 3:4, 20000:20512].cpu().numpy(), op)
    assert np.array_equal(f16_bits(n0[1:2, 3:4, 20000:20512]), on.view(np.uint16))


# --------------------------------------------------------------------------
# tolerances against the fp64 definition tier, over whole tensors
# --------------------------------------------------------------------------

class TierD:
    """Counts of GPU results against the fp64 definition tier, accumulated
    over chunks of blocks: code flips (and the largest distance of a flipped
    value's exact y from a decision boundary), fp16 norms that differ from
    RNE_fp16 of the exact norm, dequantised values beyond 1 bf16 ulp of the
    exact inverse, and beyond 1e-3 per unit of block norm from its bf16
    rounding."""

    def __init__(self, label, bits):
        self.label, self.bits = label, bits
        self.c32, _ = lm.table(bits)
        self.flips = self.dflips = self.values = self.distinct = 0
        self.maxdist = 0.0
        self.norm_diff = self.norms = 0
        self.ulp_bad = self.far = self.deq = 0

    def chunk(self, x, codes_g, n16_g, out_g, real=None, distinct=None):
        """One chunk: x (..., L) fp64 blocks; codes_g, n16_g, out_g (fp32 of the
        GPU's bf16 output, (..., L)); `real` masks padded entries out of the
        dequant counts; `distinct` marks rotated values that are not exact
        copies of another of the block (a block of at most 64 real values and
        zeros has y[j + 64] = y[j] exactly, in fp32 and in the definition)."""
        c32 = self.c32
        codes_d, n_d, y_d = ref.quantize_def(x, self.bits, c32)
        flips = codes_g != codes_d
        dist = ref.boundary_distance(y_d[flips], c32)
        distinct = np.ones(flips.shape, bool) if distinct is None else distinct
        m = np.ones(flips.shape, bool) if real is None else real
        dd = ref.dequantize_def(codes_g, n16_g.astype(np.float64), self.bits, c32)
        dd_bf16 = ref.bf16_to_f32(ref.f32_to_bf16_rne(dd.astype(np.float32))).astype(np.float64)
        g = out_g.astype(np.float64)
        ulp_bad = ~(np.abs(g - dd) <= 2.0 ** -8 * np.abs(dd) + 1e-7 * n_d[..., None]) & m
        far = (np.abs(g - dd_bf16) > 1e-3 * n_d[..., None]) & m
        return (int(flips.sum()), int((flips & distinct).sum()), flips.size, int(distinct.sum()),
                float(dist.max()) if dist.size else 0.0,
                int(np.sum(n16_g.view(np.uint16) != n_d.astype(np.float16).view(np.uint16))), n_d.size,
                int(ulp_bad.sum()), int(far.sum()), int(m.sum()))

    def add(self, r):
        self.flips += r[0]; self.dflips += r[1]; self.values += r[2]; self.distinct += r[3]
        self.maxdist = max(self.maxdist, r[4])
        self.norm_diff += r[5]; self.norms += r[6]
        self.ulp_bad += r[7]; self.far += r[8]; self.deq += r[9]

    def report_and_check(self):
        frac = self.dflips / self.distinct
        _say(f"definition tier {self.label}: code flips {self.flips} of {self.values}; over distinct rotated values "
             f"{self.dflips} of {self.distinct} ({frac:.2e}), max boundary distance {self.maxdist:.2e}; fp16 norms "
             f"differing from the exact norm's {self.norm_diff} of {self.norms} ({self.norm_diff / self.norms:.2e}); "
             f"dequant beyond 1e-3*n {self.far} of {self.deq} ({self.far / self.deq:.2e})")
        # Every flip is a boundary case of fp32 rounding against the exact
        # value.  The codes equal the canonical fp32 oracle's bit for bit (the
        # gate, elsewhere in this file); this fp32 operation order itself flips
        # about 1e-6 of the values against the exact definition (1.12e-6 over
        # the whole Q5 Qwen3.6-shaped gate_up bank), so the rate is reported and
        # only bounded loosely here: a wrong kernel flips values far from a
        # boundary, or orders of magnitude more of them.
        assert self.maxdist < 1e-5
        assert frac < 2e-6
        # within one bf16 ulp of the exact inverse everywhere; beyond 1e-3 per
        # unit of norm of its bf16 rounding only where fp32 rounding crossed a
        # bf16 rounding boundary
        assert self.ulp_bad == 0
        assert self.far / self.deq < 1e-5


def _bank_tier_d(wq, config, tensor, bits, label):
    wb_all = synth.weight(config, tensor)
    E, rows, n_in = wb_all.shape
    w = to_dev(wb_all)
    packed, norms = wq.hlwq_quantize(w, bits)
    out = wq.hlwq_dequantize(packed, norms, n_in, bits)
    torch.cuda.synchronize()
    gp, gn, go = packed.cpu().numpy(), f16_bits(norms).view(np.float16), bf16_bits(out)
    del w, packed, norms, out
    nb = -(-n_in // 128)
    t = TierD(label, bits)
    tail = n_in % 128

    def job(e):
        x, _ = ref.blocks_from_rows(wb_all[e])
        og = np.zeros((rows, nb * 128), np.float32)
        og[:, :n_in] = ref.bf16_to_f32(go[e])
        real = distinct = None
        if tail:
            real = np.zeros((rows, nb * 128), bool)
            real[:, :n_in] = True
            real = real.reshape(rows, nb, 128)
            if tail <= 64:
                distinct = np.ones((rows, nb, 128), bool)
                distinct[:, -1, 64:] = False
        return t.chunk(x.astype(np.float64), ref.unpack_codes(gp[e], bits), gn[e], og.reshape(rows, nb, 128),
                       real, distinct)

    for r in host_map(job, range(E)):
        t.add(r)
    t.report_and_check()


@pytest.mark.parametrize("bits", [5, 3])
def test_definition_tier_tolerances(wq, bits):
    # every block of the Qwen3.6-shaped gate_up bank (537M weights)
    _bank_tier_d(wq, "qwen36_moe_bank", "gate_up", bits, f"Q{bits} Qwen3.6 gate_up bank")


def test_definition_tier_tail_blocks(wq):
    # every block of the Gemma-4-shaped down_proj bank, in = 704: 5 whole
    # blocks and one of 64 real values + 64 zeros per row
    _bank_tier_d(wq, "gemma4_moe_bank", "down", 5, "Q5 Gemma-4 down bank (in=704, tail blocks)")


@pytest.mark.parametrize("bits", [5, 3])
def test_definition_tier_dense_student_t(wq, bits):
    # every block of the three dense hidden-5120 Linears (Student-t(5) values,
    # heavy tails: 205M weights)
    t = TierD(f"Q{bits} dense 5120 Linears (Student-t)", bits)
    for name in synth.CONFIGS["dense_5120"]:
        wb = synth.weight("dense_5120", name)
        rows, n_in = wb.shape
        w = to_dev(wb)
        packed, norms = wq.hlwq_quantize(w, bits)
        out = wq.hlwq_dequantize(packed, norms, n_in, bits)
        torch.cuda.synchronize()
        gp, gn, go = packed.cpu().numpy(), f16_bits(norms).view(np.float16), bf16_bits(out)
        del w, packed, norms, out
        nb = n_in // 128

        def job(rc):
            r0, r1 = rc
            x, _ = ref.blocks_from_rows(wb[r0:r1])
            og = ref.bf16_to_f32(go[r0:r1]).reshape(r1 - r0, nb, 128)
            return t.chunk(x.astype(np.float64), ref.unpack_codes(gp[r0:r1], bits), gn[r0:r1], og)

        for r in host_map(job, _row_chunks(rows)):
            t.add(r)
    t.report_and_check()


@pytest.mark.parametrize("bits", [3, 2])
def test_definition_tier_kv_h256(wq, bits):
    # every quantised vector of the benchmark's K and V cache (66.8M values)
    kv = np.concatenate([synth.kv_cache("kv_h256", t) for t in ("K", "V")], axis=0)
    B, H, T, D = kv.shape
    dev = to_dev(kv)
    packed, norms = wq.hlwq_kv_quantize(dev, n_residual=128, bits=bits)
    out = torch.empty_like(dev)
    wq.hlwq_kv_dequantize(packed, norms, out, n_residual=128, bits=bits)
    torch.cuda.synchronize()
    gp, gn, go = packed.cpu().numpy(), f16_bits(norms).view(np.float16), bf16_bits(out)
    del dev, packed, norms, out
    tq = T - 128
    t = TierD(f"KV H256 Q{bits}", bits)

    def job(bh):
        b, h = bh
        x = ref.bf16_to_f32(kv[b, h, :tq]).astype(np.float64)
        return t.chunk(x, ref.unpack_codes(gp[b, h], bits), gn[b, h], ref.bf16_to_f32(go[b, h, :tq]))

    for r in host_map(job, [(b, h) for b in range(B) for h in range(H)]):
        t.add(r)
    t.report_and_check()


def test_definition_tier_tq3(wq):
    # TQ3 against its fp64 definition (tq3_ref.quantize_def / dequantize_def):
    # every group of the Qwen3.6-shaped gate_up bank, seed 42
    from oracle import tq3_ref as tq
    wb_all = synth.weight("qwen36_moe_bank", "gate_up")
    E, rows, n_in = wb_all.shape
    w = to_dev(wb_all)
    packed, norms = wq.hlwq_tq3_quantize(w, 42)
    out = wq.hlwq_tq3_dequantize(packed, norms, n_in, 42)
    torch.cuda.synchronize()
    gp, gg, go = packed.cpu().numpy(), norms.cpu().numpy().astype(np.float64), bf16_bits(out)
    del w, packed, norms, out
    d1, d2 = tq.sign_vectors(42)
    c32, _ = lm.table(3)

    def job(e):
        x, _ = ref.blocks_from_rows(wb_all[e])
        codes_d, g_d, y_d, n_d = tq.quantize_def(x, d1, d2)
        codes_g = ref.unpack_codes(gp[e], 3)
        flips = codes_g != codes_d
        dist = ref.boundary_distance(y_d[flips], c32)
        # the shape-gain norm against its fp64 value on the GPU's own codes
        yhat = c32.astype(np.float64)[codes_g]
        g_own = n_d / (np.sqrt(np.sum(yhat * yhat, axis=-1)) / np.sqrt(128.0))
        rel = float(np.max(np.abs(gg[e] - g_own) / g_own))
        dd = tq.dequantize_def(codes_g, gg[e], d1, d2)
        dd_bf16 = ref.bf16_to_f32(ref.f32_to_bf16_rne(dd.astype(np.float32))).astype(np.float64)
        ghat = ref.bf16_to_f32(go[e]).astype(np.float64).reshape(x.shape)
        ulp_bad = int(np.sum(~(np.abs(ghat - dd) <= 2.0 ** -8 * np.abs(dd) + 1e-7 * n_d[..., None])))
        far = int(np.sum(np.abs(ghat - dd_bf16) > 1e-3 * n_d[..., None]))
        return int(flips.sum()), flips.size, float(dist.max()) if dist.size else 0.0, rel, ulp_bad, far

    res = host_map(job, range(E))
    flips, values = sum(r[0] for r in res), sum(r[1] for r in res)
    maxdist, rel = max(r[2] for r in res), max(r[3] for r in res)
    ulp_bad, far = sum(r[4] for r in res), sum(r[5] for r in res)
    _say(f"definition tier TQ3 (seed 42), Qwen3.6 gate_up bank: code flips {flips} of {values} "
         f"({flips / values:.2e}), max boundary distance {maxdist:.2e}; shape-gain norm max relative error "
         f"{rel:.2e}; dequant beyond 1e-3*n {far} ({far / values:.2e})")
    assert maxdist < 1e-5
    assert flips / values < 2e-6  # reported; see TierD.report_and_check
    assert rel < 1e-6
    assert ulp_bad == 0
    assert far / values < 1e-5


# --------------------------------------------------------------------------
# TQ3 ("Qwen3.6-35B-A3B-TQ3-native", section "What TQ3 actually does")
# --------------------------------------------------------------------------

def f32_bits(t) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int32).numpy().view(np.uint32)


def check_tq3(wq, w_bits: np.ndarray, seed: int, label: str, w=None, out=None):
    rows, n_in = w_bits.shape
    _say("tq3", label, "rows", rows, "in", n_in, "seed", seed)
    w = to_dev(w_bits) if w is None else w
    packed, norms = wq.hlwq_tq3_quantize(w, seed)
    out = wq.hlwq_tq3_dequantize(packed, norms, n_in, seed, out=out)
    torch.cuda.synchronize()
    from oracle import tq3_ref as tq
    op, on = tq.quantize_c(w_bits, seed)
    assert np.array_equal(f32_bits(norms), on.view(np.uint32)), f"{label}: fp32 norms differ"
    assert np.array_equal(packed.cpu().numpy(), op), f"{label}: packed codes differ"
    assert np.array_equal(bf16_bits(out), tq.dequantize_c(op, on, n_in, seed)), f"{label}: bf16 differs"
    return out


@pytest.mark.parametrize("seed", [42, 7])
@pytest.mark.parametrize("n_in", [1, 8, 127, 128, 129, 200, 704, 1000])
def test_tq3_shapes_and_tails(wq, seed, n_in):
    w = synth.random_bf16((67, n_in), seed=n_in + 1, key=5)
    check_tq3(wq, w, seed, f"tails-{n_in}")


def test_tq3_many_tiles(wq):
    w = synth.random_bf16((3001, 384), seed=15, outlier_frac=0.001, outlier_mult=20.0)
    check_tq3(wq, w, 42, "tiles-outliers")
    w = synth.random_bf16((257, 1536), seed=16, dist="student_t5")
    check_tq3(wq, w, 2 ** 64 - 1, "tiles-t5")


def test_tq3_special_blocks(wq):
    w = _special_rows()
    w[8, ::2] = 0x8000
    check_tq3(wq, w, 42, "special")


def test_tq3_unaligned_rows(wq):
    for n_in in (129, 704):
        w_bits = synth.random_bf16((41, n_in), seed=n_in, key=6)
        base = torch.zeros(41 * n_in + 1, dtype=torch.bfloat16, device="cuda")
        base[1:] = to_dev(w_bits).reshape(-1)
        outbuf = torch.zeros(41 * n_in + 1, dtype=torch.bfloat16, device="cuda")
        check_tq3(wq, w_bits, 42, f"unaligned-{n_in}", w=base[1:].view(41, n_in), out=outbuf[1:].view(41, n_in))
        assert bf16_bits(outbuf[:1])[0] == 0


def test_tq3_dequantize_arbitrary_codes(wq):
    # every code value at every position, norms over a wide range (not only
    # what the quantizer produces)
    from oracle import tq3_ref as tq
    rng = np.random.default_rng(21)
    rows, n_in = 300, 512
    packed = rng.integers(0, 256, (rows, 4, 48), dtype=np.uint8)
    norms = (np.exp(rng.uniform(-20, 20, (rows, 4))) * rng.choice([1.0, 0.0], (rows, 4), p=[0.95, 0.05]))
    norms = norms.astype(np.float32)
    _say("tq3 arbitrary codes")
    out = wq.hlwq_tq3_dequantize(torch.from_numpy(packed).cuda(), torch.from_numpy(norms).cuda(), n_in, 42)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), tq.dequantize_c(packed, norms, n_in, 42))


def test_tq3_grouped_launch(wq):
    from oracle import tq3_ref as tq
    rng = np.random.default_rng(22)
    items, host = [], []
    for i in range(18):
        rows = int(rng.integers(1, 200))
        n_in = int(rng.choice([64, 128, 200, 512, 704]))
        wb = synth.random_bf16((rows, n_in), seed=300 + i)
        nb = -(-n_in // 128)
        items.append((to_dev(wb), torch.empty((rows, nb, 48), dtype=torch.uint8, device="cuda"),
                      torch.empty((rows, nb), dtype=torch.float32, device="cuda")))
        host.append(wb)
    _say("tq3 grouped, 18 matrices")
    wq.hlwq_tq3_quantize_grouped(items, 42)
    outs = [(torch.empty_like(w), p, n) for (w, p, n) in items]
    wq.hlwq_tq3_dequantize_grouped(outs, 42)
    torch.cuda.synchronize()
    for (w, p, n), (o, _, _), wb in zip(items, outs, host):
        op, on = tq.quantize_c(wb, 42)
        assert np.array_equal(p.cpu().numpy(), op)
        assert np.array_equal(f32_bits(n), on.view(np.uint32))
        assert np.array_equal(bf16_bits(o), tq.dequantize_c(op, on, wb.shape[1], 42))


def test_tq3_qwen36_moe_bank_full(wq):
    # the page's TQ3 checkpoint is of this model: the full MoE layer in one
    # grouped launch, every expert against the oracle
    from oracle import tq3_ref as tq
    config = "qwen36_moe_bank"
    tensors = list(synth.CONFIGS[config])
    host = {t: synth.weight(config, t) for t in tensors}
    items = []
    for t in tensors:
        E, rows, n_in = host[t].shape
        nb = -(-n_in // 128)
        items.append((to_dev(host[t]), torch.empty((E, rows, nb, 48), dtype=torch.uint8, device="cuda"),
                      torch.empty((E, rows, nb), dtype=torch.float32, device="cuda")))
    _say("tq3", config, "generated")
    wq.hlwq_tq3_quantize_grouped(items, 42)
    outs = [(torch.empty_like(w), p, n) for (w, p, n) in items]
    wq.hlwq_tq3_dequantize_grouped(outs, 42)
    torch.cuda.synchronize()
    _say("tq3", config, "gpu done; checking every expert on", HOST_WORKERS, "host threads")
    for t, (w, p, n), (o, _, _) in zip(tensors, items, outs):
        gp, gn, go = p.cpu().numpy(), f32_bits(n), bf16_bits(o)
        wb_all = host[t]

        def check(e):
            op, on = tq.quantize_c(wb_all[e], 42)
            od = tq.dequantize_c(op, on, wb_all.shape[2], 42)
            return (e, np.array_equal(gp[e], op), np.array_equal(gn[e], on.view(np.uint32)),
                    np.array_equal(go[e], od))

        bad = first_failure(host_map(check, range(wb_all.shape[0])))
        assert bad is None, ("tq3", t, bad)
    del items, outs
    torch.cuda.empty_cache()


def test_kv_decode_steps_in_a_hip_graph(wq):
    # a decode loop is launch-bound, so callers capture it: 14 appends (single
    # tokens through the latency path, a 20-token chunk through the ring
    # kernels, a 200-token chunk through the KV quantize kernel as well)
    # recorded into one graph and replayed three times, each replay from the
    # same starting state (restored eagerly in between) and each checked
    # against the same appends run eagerly
    B, H, T, n_res, bits = 2, 3, 300, 128, 3
    kv = synth.random_bf16((B, H, T, 256), seed=41, sigma=1.0)
    chunks = [1] * 6 + [20] + [1] * 5 + [200, 1]
    new = synth.random_bf16((B, H, sum(chunks), 256), seed=42, sigma=1.0)
    cap = T - n_res + sum(chunks)
    packed0 = torch.full((B, H, cap, 32 * bits), 0xAB, dtype=torch.uint8, device="cuda")
    norms0 = torch.full((B, H, cap), 7.0, dtype=torch.float16, device="cuda")
    p0, n0 = wq.hlwq_kv_quantize(to_dev(kv), n_residual=n_res, bits=bits)
    packed0[:, :, :T - n_res] = p0
    norms0[:, :, :T - n_res] = n0
    window0 = torch.empty((B, H, n_res, 256), dtype=torch.bfloat16, device="cuda")
    dev = to_dev(kv)
    for t in range(T - n_res, T):
        window0[:, :, t % n_res] = dev[:, :, t]
    parts, o = [], 0
    for n in chunks:
        parts.append(to_dev(new[:, :, o:o + n]))
        o += n

    def run(window, packed, norms):
        tokens = T
        for part in parts:
            tokens = wq.hlwq_kv_append(part, window, packed, norms, tokens, n_residual=n_res, bits=bits)

    ew, ep, en = window0.clone(), packed0.clone(), norms0.clone()
    run(ew, ep, en)
    torch.cuda.synchronize()
    gw, gp, gn = window0.clone(), packed0.clone(), norms0.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(gw, gp, gn)
    for r in range(3):
        gw.copy_(window0)
        gp.copy_(packed0)
        gn.copy_(norms0)
        torch.cuda.synchronize()
        _say("kv append graph replay", r)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gp, ep) and torch.equal(gn, en) and torch.equal(gw, ew), f"replay {r}"
    # and the eager result is the oracle's
    op, on, ow = ref.kv_stream_c([kv] + [new[:, :, s:s + n] for s, n in zip(np.cumsum([0] + chunks[:-1]), chunks)],
                                 n_residual=n_res, bits=bits)
    assert np.array_equal(ep.cpu().numpy()[:, :, :op.shape[2]], op)
    assert np.array_equal(f16_bits(en)[:, :, :op.shape[2]], on.view(np.uint16))


def test_weight_kernels_in_a_hip_graph(wq):
    # grouped Q5 quantize + dequantize of two matrices (one with tail blocks)
    # and a TQ3 quantize + dequantize, captured in one HIP graph and replayed
    # three times into cleared outputs; every replay must equal the eager
    # calls, and those the oracle
    from oracle import tq3_ref as tq
    wa = synth.random_bf16((300, 1000), seed=31, key=5, outlier_frac=0.001, outlier_mult=20.0)
    wb = synth.random_bf16((257, 384), seed=32, key=5)
    ws = [to_dev(wa), to_dev(wb)]

    def buffers():  # allocated outside any capture
        qs = [wq.hlwq_quantize(w, 5) for w in ws]
        t = wq.hlwq_tq3_quantize(ws[0])
        return qs, t, [torch.empty_like(ws[0]), torch.empty_like(ws[1]), torch.empty_like(ws[0])]

    def run(qs, t, outs):
        wq.hlwq_quantize_grouped([(w, p, n) for w, (p, n) in zip(ws, qs)], 5)
        wq.hlwq_dequantize_grouped([(o, p, n) for o, (p, n) in zip(outs, qs)], 5)
        wq.hlwq_tq3_quantize(ws[0], packed=t[0], norms=t[1])
        wq.hlwq_tq3_dequantize(t[0], t[1], ws[0].shape[1], out=outs[2])

    def clear(qs, t, outs):
        for x in [v for pn in qs for v in pn] + list(t) + outs:
            x.zero_()

    eq, et, eo = buffers()
    clear(eq, et, eo)
    run(eq, et, eo)
    torch.cuda.synchronize()
    gq, gt, go = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(gq, gt, go)
    for r in range(3):
        clear(gq, gt, go)
        torch.cuda.synchronize()
        _say("weight graph replay", r)
        graph.replay()
        torch.cuda.synchronize()
        for (a, b), (c, d) in zip(gq, eq):
            assert torch.equal(a, c) and torch.equal(b, d), f"replay {r}: codes / norms"
        assert torch.equal(gt[0], et[0]) and torch.equal(gt[1], et[1]), f"replay {r}: TQ3"
        assert all(torch.equal(a, b) for a, b in zip(go, eo)), f"replay {r}: dequantized"
    for w_bits, (p, n), o in zip((wa, wb), eq, eo):
        op, on = ref.quantize_c(w_bits, 5)
        assert np.array_equal(p.cpu().numpy(), op) and np.array_equal(f16_bits(n), on.view(np.uint16))
        assert np.array_equal(bf16_bits(o), ref.dequantize_c(op, on, w_bits.shape[1], 5))
    tp, tn = tq.quantize_c(wa)
    assert np.array_equal(et[0].cpu().numpy(), tp) and np.array_equal(f32_bits(et[1]), tn.view(np.uint32))
    assert np.array_equal(bf16_bits(eo[2]), tq.dequantize_c(tp, tn, wa.shape[1]))


def test_concurrent_calls_from_threads(wq):
    # four host threads, each with its own stream and matrix, call quantize and
    # dequantize at the same time (the library keeps no per-call state; its one
    # lazily filled value, the CU count, is an atomic); all results are the
    # oracle's
    import threading
    mats = [synth.random_bf16((200 + 37 * k, 640 + 64 * k), seed=40 + k, key=5) for k in range(4)]
    devs = [to_dev(m) for m in mats]
    torch.cuda.synchronize()
    results, errors = [None] * 4, []

    def work(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    p, n = wq.hlwq_quantize(devs[k], 5)
                    o = wq.hlwq_dequantize(p, n, mats[k].shape[1], 5)
            s.synchronize()
            results[k] = (p, n, o)
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for m, (p, n, o) in zip(mats, results):
        op, on = ref.quantize_c(m, 5)
        assert np.array_equal(p.cpu().numpy(), op) and np.array_equal(f16_bits(n), on.view(np.uint16))
        assert np.array_equal(bf16_bits(o), ref.dequantize_c(op, on, m.shape[1], 5))


def test_matrix_beyond_4_gib(wq):
    # one 81920 x 32768 bf16 matrix (5.4 GB): byte offsets past 2^32 in W, the
    # codes and the output.  Rows repeat a seeded pattern of 61 rows (a prime,
    # so a row-addressing error of 2^k rows lands on a different pattern row);
    # sampled rows around the 2^32-byte boundaries and at the end are checked
    # against the oracle bit for bit
    rows, n_in, period = 81920, 32768, 61
    pattern = synth.random_bf16((period, n_in), seed=77, key=3, outlier_frac=0.001, outlier_mult=20.0)
    pat = to_dev(pattern)
    w = torch.empty((rows, n_in), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, period):
        n = min(period, rows - r0)
        w[r0:r0 + n] = pat[:n]
    _say("4 GiB+ matrix filled")
    packed, norms = wq.hlwq_quantize(w, 5)
    out = wq.hlwq_dequantize(packed, norms, n_in, 5)
    torch.cuda.synchronize()
    boundary = (1 << 31) // n_in  # first row past 2^32 bytes of W
    for r in (0, 1, boundary - 1, boundary, boundary + 1, 2 * boundary // 2 + 777, rows - 2, rows - 1):
        src = pattern[r % period][None, :]
        op, on = ref.quantize_c(src, 5)
        assert np.array_equal(packed[r].cpu().numpy(), op[0]), r
        assert np.array_equal(f16_bits(norms[r]), on[0].view(np.uint16)), r
        assert np.array_equal(bf16_bits(out[r]), ref.dequantize_c(op, on, n_in, 5)[0]), r
    del w, out, packed, norms
    torch.cuda.empty_cache()


def test_kv_cache_split_over_launches(wq):
    # 67,108,897 heads of one quantised token each (34 GB of bf16): more
    # 16-token batches than one dequantize grid of 2^24 - 1 workgroups
    # addresses, so both calls split the cache by heads over two launches.
    # Heads repeat a seeded pattern of 61 vectors (a prime); sampled heads at
    # the start, around the split and at the end are checked bit for bit.
    n_split = 4 * (0xFFFFFFFF // 256)  # batches (here heads) in the first launch
    H, period = n_split + 37, 61
    pattern = synth.random_bf16((period, 256), seed=91, sigma=1.0)
    idx = torch.arange(H, device="cuda") % period
    dev = to_dev(pattern)[idx].view(1, H, 1, 256)
    del idx
    _say("kv split", H)
    packed, norms = wq.hlwq_kv_quantize(dev, n_residual=0)
    out = torch.empty_like(dev)
    wq.hlwq_kv_dequantize(packed, norms, out, n_residual=0)
    torch.cuda.synchronize()
    heads = [0, 1, 60, 61, n_split - 2, n_split - 1, n_split, n_split + 1, H - 1]
    sl = pattern[[h % period for h in heads]].reshape(1, len(heads), 1, 256)
    op, on = ref.kv_quantize_c(sl, n_residual=0)
    hs = torch.tensor(heads, device="cuda")
    assert np.array_equal(packed[0, hs].cpu().numpy(), op[0])
    assert np.array_equal(f16_bits(norms[0, hs]), on[0].view(np.uint16))
    assert np.array_equal(bf16_bits(out[0, hs]), ref.kv_dequantize_c(op, on)[0])
    del dev, out, packed, norms
    torch.cuda.empty_cache()


@pytest.mark.parametrize("case", range(12))
def test_random_shapes(wq, case):
    # seeded random shapes and value scales, every weight entry point on the same matrix
    from oracle import tq3_ref as tq
    rng = np.random.default_rng(1000 + case)
    rows = int(rng.integers(1, 700))
    n_in = int(rng.choice([int(rng.integers(1, 1200)), 128 * int(rng.integers(1, 12))]))
    sigma = float(np.exp(rng.uniform(-12, 4)))
    dist = str(rng.choice(["normal", "student_t5"]))
    wb = synth.random_bf16((rows, n_in), seed=2000 + case, key=7, dist=dist, sigma=sigma)
    _say("random shape", case, rows, n_in, f"{sigma:.3g}", dist)
    for bits in (5, 3):
        check_matrix(wq, wb, bits, f"random-{case}-q{bits}")
        codes, norms = wq.hlwq_quantize_codes8(to_dev(wb), bits)
        torch.cuda.synchronize()
        oc, on = ref.quantize_codes8_c(wb, bits)
        assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(f16_bits(norms), on.view(np.uint16))
        if n_in % 128 == 0:  # the INT4 groups are the HLWQ blocks
            packed, n16 = wq.hlwq_quantize(to_dev(wb), bits)
            q4, scales, zeros = wq.hlwq_dequantize_int4(packed, n16, n_in, bits)
            torch.cuda.synchronize()
            op, on = ref.quantize_c(wb, bits)
            p4, s4, z4 = ref.dequantize_to_int4_c(op, on, n_in, bits)
            assert np.array_equal(q4.cpu().numpy(), p4) and np.array_equal(zeros.cpu().numpy(), z4)
            assert np.array_equal(scales.cpu().numpy().view(np.uint32), s4.view(np.uint32))
    check_tq3(wq, wb, 42 if case % 2 == 0 else int(rng.integers(0, 2 ** 63)), f"random-{case}-tq3")
