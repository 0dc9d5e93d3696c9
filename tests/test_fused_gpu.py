"""Append fused into the attend launch (kvdec_append_attend), through the C ABI.

The fused call must leave the cache and the lengths exactly as kvdec_append
does (bit for bit, NaN canaries in unused rows included) and return exactly
the output of kvdec_append followed by kvdec_attend_self at the same chunk
size (same chunks, same arithmetic, same order), which is also checked
against the f64 oracle within the usual tolerance.  Cases: linear and ring
caches, f32 and bf16, MHA, MFMA and VALU groups, one chunk and several (merge
launch), new rows landing on a chunk boundary, the first-ever row, the
device-length mode (replay mode, batches above 512: the merge launch bumps
the lengths), and kvdec_append_attend_at (explicit positions, rewinds).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from kv_cached_decode_kvdec_amd import binding as B
from kv_cached_decode_kvdec_amd import inputs as gen
from kv_cached_decode_kvdec_amd.cache import KVCache, to_device, to_host_bits

from helpers import assert_attention_close

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _pair(inp, window=0):
    """Two device caches holding the same state, plus the oracle's mirror."""
    wl = inp.wl
    Bsz = len(inp.lens)
    cap = inp.cap if window == 0 else window
    mk = lambda: KVCache(Bsz, wl.n_kv_heads, cap, wl.dtype, lens=inp.lens,
                         k=to_device(inp.k_cache), v=to_device(inp.v_cache), window=window)
    return mk(), mk()


# lengths: empty, chunk boundaries (the new row opens a chunk), ragged, long
LENS = np.array([0, 63, 64, 127, 128, 255, 1, 700, 1983], np.int32)


@pytest.mark.parametrize("dtype,Hq,Hkv", [("f32", 4, 4), ("bf16", 8, 2), ("bf16", 12, 3),
                                           ("bf16", 7, 1), ("f32", 6, 3)])
@pytest.mark.parametrize("chunk_rows", [0, 64, 256])
def test_fused_equals_append_then_attend(dtype, Hq, Hkv, chunk_rows):
    wl = gen.Workload("fused", len(LENS), Hq, Hkv, dtype, "const:1", 3, False, seed=61)
    inp = gen.make_inputs(wl, batch=len(LENS), lens=LENS, steps=3)
    _log(f"fused {dtype} {Hq}/{Hkv} chunk={chunk_rows}")
    two, one = _pair(inp)
    Kh, Vh, lens = inp.k_cache.copy(), inp.v_cache.copy(), inp.lens.copy()
    for s in range(3):
        kn, vn, q = to_device(inp.k_new[s]), to_device(inp.v_new[s]), to_device(inp.q_self[s])
        two.append(kn, vn)
        ref_dev = two.attend(q, chunk_rows=chunk_rows)
        got = one.append_attend(kn, vn, q, chunk_rows=chunk_rows)
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref_dev.cpu().numpy().tobytes(), f"step {s}"
        lens = oracle.append(Kh, Vh, inp.k_new[s], inp.v_new[s], lens)
        ref = oracle.attend(inp.q_self[s], Kh, Vh, lens)
        assert_attention_close(got.cpu().numpy(), ref, dtype, f"fused step {s}")
    assert to_host_bits(one.k).tobytes() == Kh.tobytes()
    assert to_host_bits(one.v).tobytes() == Vh.tobytes()
    assert one.lens() == lens.tolist() and one.lens_dev.cpu().tolist() == lens.tolist()


@pytest.mark.parametrize("dtype,Hq,Hkv,W", [("f32", 4, 4, 100), ("bf16", 16, 4, 96),
                                             ("bf16", 6, 2, 130)])
def test_fused_ring(dtype, Hq, Hkv, W):
    rng = np.random.default_rng(71 + W)
    Bsz, steps = 3, 150
    start = np.array([0, W - 1, W + 7], np.int32)      # empty, about to wrap, wrapped
    total = int(start.max()) + steps
    draw = lambda: rng.standard_normal((Bsz, Hkv, total, 64), dtype=np.float32)
    hist_k, hist_v = draw(), draw()
    if dtype == "bf16":
        hist_k, hist_v = gen.f32_to_bf16_bits(hist_k), gen.f32_to_bf16_bits(hist_v)
    cap_pad = gen.padded_rows(W)
    ring_k = np.zeros((Bsz, Hkv, cap_pad, 64), hist_k.dtype)
    ring_v = np.zeros_like(ring_k)
    for b in range(Bsz):
        for t in range(max(0, start[b] - W), start[b]):
            ring_k[b, :, t % W] = hist_k[b, :, t]
            ring_v[b, :, t % W] = hist_v[b, :, t]
    mk = lambda: KVCache(Bsz, Hkv, W, dtype, lens=start, k=to_device(ring_k), v=to_device(ring_v),
                         window=W)
    two, one = mk(), mk()
    lens = start.copy()
    for s in range(steps):
        kn = to_device(np.stack([hist_k[b, :, lens[b]] for b in range(Bsz)]))
        vn = to_device(np.stack([hist_v[b, :, lens[b]] for b in range(Bsz)]))
        q_h = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
        q = to_device(q_h)
        T = 64 if s % 2 else 0
        two.append(kn, vn)
        ref_dev = two.attend(q, chunk_rows=T)
        got = one.append_attend(kn, vn, q, chunk_rows=T)
        lens += 1
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref_dev.cpu().numpy().tobytes(), f"ring step {s}"
        if s % 37 == 0 or s == steps - 1:
            n = np.minimum(lens, W)
            lk = np.zeros((Bsz, Hkv, cap_pad, 64), hist_k.dtype)
            lv = np.zeros_like(lk)
            for b in range(Bsz):
                lk[b, :, :n[b]] = hist_k[b, :, lens[b] - n[b]:lens[b]]
                lv[b, :, :n[b]] = hist_v[b, :, lens[b] - n[b]:lens[b]]
            ref = oracle.attend(q_h, lk, lv, n)
            assert_attention_close(got.cpu().numpy(), ref, dtype, f"fused ring step {s}")
    assert one.lens() == lens.tolist() and one.lens_dev.cpu().tolist() == lens.tolist()
    assert to_host_bits(one.k).tobytes() == to_host_bits(two.k).tobytes()
    assert to_host_bits(one.v).tobytes() == to_host_bits(two.v).tobytes()


@pytest.mark.parametrize("name", gen.ORDER)
def test_fused_full_size_workloads(name):
    """Every self-attention workload at its real shape and automatic chunk
    size, every step, every sequence and head against the oracle, and the
    whole cache bit for bit."""
    wl = gen.WORKLOADS[name]
    _log(f"fused full {name}")
    inp = gen.make_inputs(wl)
    c = KVCache(len(inp.lens), wl.n_kv_heads, inp.cap, wl.dtype, lens=inp.lens,
                k=to_device(inp.k_cache), v=to_device(inp.v_cache))
    Kh, Vh, lens = inp.k_cache.copy(), inp.v_cache.copy(), inp.lens.copy()
    for s in range(wl.steps):
        out = c.append_attend(to_device(inp.k_new[s]), to_device(inp.v_new[s]),
                              to_device(inp.q_self[s]))
        torch.cuda.synchronize()
        lens = oracle.append(Kh, Vh, inp.k_new[s], inp.v_new[s], lens)
        ref = oracle.attend(inp.q_self[s], Kh, Vh, lens)
        assert_attention_close(out.cpu().numpy(), ref, wl.dtype, f"{name} step {s}")
    assert to_host_bits(c.k).tobytes() == Kh.tobytes()
    assert to_host_bits(c.v).tobytes() == Vh.tobytes()
    assert c.lens_dev.cpu().tolist() == lens.tolist()
    c.close()


@pytest.mark.parametrize("mode", ["large-batch", "replay"])
def test_fused_device_length_mode(mode):
    Bsz = B.KVDEC_MAX_FUSED_BATCH + 3 if mode == "large-batch" else 5
    wl = gen.Workload("fb", Bsz, 8, 2, "bf16", "uniform:0:300", 2, False, seed=67)
    inp = gen.make_inputs(wl, batch=Bsz, steps=2)
    two, one = _pair(inp)
    if mode == "replay":
        two.set_replay_mode(-1)
        one.set_replay_mode(-1)
    Kh, Vh, lens = inp.k_cache.copy(), inp.v_cache.copy(), inp.lens.copy()
    for s in range(2):
        kn, vn, q = to_device(inp.k_new[s]), to_device(inp.v_new[s]), to_device(inp.q_self[s])
        two.append(kn, vn)
        ref_dev = two.attend(q)
        got = one.append_attend(kn, vn, q)
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref_dev.cpu().numpy().tobytes()
        lens = oracle.append(Kh, Vh, inp.k_new[s], inp.v_new[s], lens)
    bs = np.arange(0, Bsz, max(1, Bsz // 16))
    ref = oracle.attend(inp.q_self[1][bs], Kh[bs], Vh[bs], lens[bs])
    assert_attention_close(got.cpu().numpy()[bs], ref, "bf16", mode)
    assert to_host_bits(one.k).tobytes() == Kh.tobytes()
    assert one.lens_dev.cpu().tolist() == lens.tolist()


def test_fused_errors_enqueue_nothing():
    c = KVCache(2, 2, 3, "f32", lens=[2, 3])
    kn = torch.zeros(2, 2, 64, device="cuda")
    q = torch.zeros(2, 4, 64, device="cuda")
    before = c.k.clone()
    with pytest.raises(B.KvdecError) as e:
        c.append_attend(kn, kn, q)                      # sequence 1 is full
    assert e.value.code == B.KVDEC_E_OVERFLOW
    c2 = KVCache(2, 2, 8, "f32", lens=[2, 3])
    with pytest.raises(B.KvdecError) as e:
        c2.append_attend(kn, kn, torch.zeros(2, 3, 64, device="cuda"))   # 3 heads over 2
    assert e.value.code == B.KVDEC_E_SHAPE
    with pytest.raises(B.KvdecError) as e:
        c2.append_attend(kn, kn, q, chunk_rows=100)
    assert e.value.code == B.KVDEC_E_INVALID
    s = KVCache(2, 2, 10, "f32", static=True, lens=[10, 10])
    with pytest.raises(B.KvdecError) as e:
        s.append_attend(kn, kn, q)
    assert e.value.code == B.KVDEC_E_STATIC
    torch.cuda.synchronize()
    assert torch.equal(c.k, before) and c.lens() == [2, 3] and c2.lens() == [2, 3]
    assert c2.lens_dev.cpu().tolist() == [2, 3] and c.lens_dev.cpu().tolist() == [2, 3]


@pytest.mark.parametrize("mode", ["one-launch", "replay", "large-batch"])
def test_append_attend_at_equals_reset_then_fused(mode):
    """kvdec_append_attend_at(lens) == kvdec_reset_lens(lens) + kvdec_append_attend, bitwise,
    including a rewind to earlier positions (their rows are overwritten)."""
    Bsz = B.KVDEC_MAX_FUSED_BATCH + 5 if mode == "large-batch" else 6
    wl = gen.Workload("at", Bsz, 8, 2, "bf16", "uniform:10:300", 3, False, seed=97)
    inp = gen.make_inputs(wl, batch=Bsz, steps=3)
    two, one = _pair(inp)
    if mode == "replay":
        two.set_replay_mode(64)
        one.set_replay_mode(64)
    rng = np.random.default_rng(98)
    Kh, Vh = inp.k_cache.copy(), inp.v_cache.copy()
    pos = inp.lens.copy()
    for s in range(3):
        if s == 2:                                   # rewind every sequence by 0..9 tokens
            pos = np.maximum(pos - rng.integers(0, 10, size=Bsz).astype(np.int32), 0)
        kn, vn, q = to_device(inp.k_new[s]), to_device(inp.v_new[s]), to_device(inp.q_self[s])
        two.reset_lens(pos)
        ref_dev = two.append_attend(kn, vn, q)
        got = one.append_attend_at(pos, kn, vn, q)
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref_dev.cpu().numpy().tobytes(), f"{mode} step {s}"
        pos = oracle.append(Kh, Vh, inp.k_new[s], inp.v_new[s], pos)
        bs = np.arange(0, Bsz, max(1, Bsz // 12))
        ref = oracle.attend(inp.q_self[s][bs], Kh[bs], Vh[bs], pos[bs])
        assert_attention_close(got.cpu().numpy()[bs], ref, "bf16", f"{mode} step {s}")
    assert one.lens() == pos.tolist() and one.lens_dev.cpu().tolist() == pos.tolist()
    assert to_host_bits(one.k).tobytes() == to_host_bits(two.k).tobytes()
    assert to_host_bits(one.v).tobytes() == to_host_bits(two.v).tobytes()


def test_append_attend_at_errors_enqueue_nothing():
    c = KVCache(2, 2, 8, "f32", lens=[3, 4])
    kn = torch.zeros(2, 2, 64, device="cuda")
    q = torch.zeros(2, 4, 64, device="cuda")
    for lens, code in (([8, 0], B.KVDEC_E_OVERFLOW), ([-1, 0], B.KVDEC_E_SHAPE),
                       ([9, 0], B.KVDEC_E_SHAPE)):
        with pytest.raises(B.KvdecError) as e:
            c.append_attend_at(lens, kn, kn, q)
        assert e.value.code == code, lens
    with pytest.raises(B.KvdecError) as e:
        c.append_attend_at([0, 0], kn, kn, torch.zeros(2, 3, 64, device="cuda"))
    assert e.value.code == B.KVDEC_E_SHAPE
    s = KVCache(2, 2, 10, "f32", static=True, lens=[10, 10])
    with pytest.raises(B.KvdecError) as e:
        s.append_attend_at([1, 1], kn, kn, q)
    assert e.value.code == B.KVDEC_E_STATIC
    torch.cuda.synchronize()
    assert c.lens() == [3, 4] and c.lens_dev.cpu().tolist() == [3, 4]
    assert torch.all(c.k == 0)
    # a ring accepts any non-negative position
    r = KVCache(2, 2, 8, "f32", lens=[0, 0], window=8)
    r.append_attend_at([100, 7], kn, kn, q)
    torch.cuda.synchronize()
    assert r.lens() == [101, 8] and r.lens_dev.cpu().tolist() == [101, 8]
