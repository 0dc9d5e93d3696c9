"""Chunk placement on the CUs (host-fused MFMA launches), through the C ABI.

A host-fused launch (kvdec_append_attend) of the MFMA kernel (bf16 K/V,
grouped query heads) whose chunks fit one residency round, with ragged
lengths and more chunks than the device has CU classes (cus / n_kv_heads),
runs its chunks on a (KV head, position) grid in an order the host picks to
balance the rows per CU, some positions empty.  The order must change
nothing: the output must equal kvdec_append + kvdec_attend_self (chunk
order, no placement) bit for bit, at the same chunk size, step after step,
the cache and lengths must equal kvdec_append's, and the output must match
the f64 oracle.  On a 256-CU MI355X every case below is placed: groups of
4 (64 and 128 classes) and 3 (32 classes), a ring whose new rows land
inside the window (the slot row read from k_new / v_new), and the paged
fused step (kvdec_paged_append_attend against kvdec_paged_append +
kvdec_paged_attend, pool bytes included).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from kv_cached_decode_kvdec_amd import inputs as gen
from kv_cached_decode_kvdec_amd.cache import KVCache, PagedKVCache, to_device, to_host_bits

from helpers import assert_attention_close

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("dtype,Hq,Hkv,B,max_len,chunk", [("bf16", 16, 4, 40, 1500, 256),
                                                          ("bf16", 8, 2, 40, 1500, 256),
                                                          ("bf16", 24, 8, 24, 400, 64)])
def test_placed_fused_equals_chunk_order(dtype, Hq, Hkv, B, max_len, chunk):
    rng = np.random.default_rng(900 + B + Hkv)
    lens = rng.integers(0, max_len, B).astype(np.int32)
    lens[:3] = [0, chunk - 1, chunk]          # empty, new row opens a chunk, ends one
    wl = gen.Workload("placed", B, Hq, Hkv, dtype, "const:1", 2, False, seed=911 + B)
    inp = gen.make_inputs(wl, batch=B, lens=lens, steps=2)
    _log(f"placed {dtype} {Hq}/{Hkv} B={B} chunk={chunk}")
    mk = lambda: KVCache(B, Hkv, inp.cap, dtype, lens=inp.lens, k=to_device(inp.k_cache),
                         v=to_device(inp.v_cache))
    two, one = mk(), mk()
    Kh, Vh, lh = inp.k_cache.copy(), inp.v_cache.copy(), inp.lens.copy()
    for s in range(2):
        kn, vn, q = to_device(inp.k_new[s]), to_device(inp.v_new[s]), to_device(inp.q_self[s])
        two.append(kn, vn)
        ref_dev = two.attend(q, chunk_rows=chunk)
        got = one.append_attend(kn, vn, q, chunk_rows=chunk)
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref_dev.cpu().numpy().tobytes(), f"step {s}"
        lh = oracle.append(Kh, Vh, inp.k_new[s], inp.v_new[s], lh)
        assert_attention_close(got.cpu().numpy(), oracle.attend(inp.q_self[s], Kh, Vh, lh), dtype,
                               f"placed step {s}")
    assert to_host_bits(one.k).tobytes() == Kh.tobytes()
    assert to_host_bits(one.v).tobytes() == Vh.tobytes()
    assert one.lens() == lh.tolist() and one.lens_dev.cpu().tolist() == lh.tolist()


def test_placed_fused_ring():
    """Rings past their window: the slot is an interior row of its chunk."""
    rng = np.random.default_rng(931)
    B, Hq, Hkv, W, chunk, steps = 40, 16, 4, 300, 64, 3
    start = rng.integers(0, 2 * W, B).astype(np.int32)
    total = int(start.max()) + steps
    hk = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv, total, 64), dtype=np.float32))
    hv = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv, total, 64), dtype=np.float32))
    cp = gen.padded_rows(W)
    rk = np.zeros((B, Hkv, cp, 64), np.uint16)
    rv = np.zeros_like(rk)
    for b in range(B):
        for t in range(max(0, start[b] - W), start[b]):
            rk[b, :, t % W], rv[b, :, t % W] = hk[b, :, t], hv[b, :, t]
    mk = lambda: KVCache(B, Hkv, W, "bf16", lens=start, k=to_device(rk), v=to_device(rv), window=W)
    two, one = mk(), mk()
    lens = start.copy()
    for s in range(steps):
        _log(f"placed ring step {s}")
        kn = to_device(np.stack([hk[b, :, lens[b]] for b in range(B)]))
        vn = to_device(np.stack([hv[b, :, lens[b]] for b in range(B)]))
        qh = rng.standard_normal((B, Hq, 64), dtype=np.float32)
        q = to_device(qh)
        two.append(kn, vn)
        ref_dev = two.attend(q, chunk_rows=chunk)
        got = one.append_attend(kn, vn, q, chunk_rows=chunk)
        lens += 1
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref_dev.cpu().numpy().tobytes(), f"ring step {s}"
        n = np.minimum(lens, W)
        lk = np.zeros((B, Hkv, cp, 64), np.uint16)
        lv = np.zeros_like(lk)
        for b in range(B):
            lk[b, :, :n[b]] = hk[b, :, lens[b] - n[b]:lens[b]]
            lv[b, :, :n[b]] = hv[b, :, lens[b] - n[b]:lens[b]]
        assert_attention_close(got.cpu().numpy(), oracle.attend(qh, lk, lv, n), "bf16",
                               f"placed ring step {s}")
    assert to_host_bits(one.k).tobytes() == to_host_bits(two.k).tobytes()
    assert to_host_bits(one.v).tobytes() == to_host_bits(two.v).tobytes()
    assert one.lens() == lens.tolist() and one.lens_dev.cpu().tolist() == lens.tolist()


@pytest.mark.parametrize("P", [16, 64])
def test_placed_paged_fused(P):
    """The paged fused step (pages of P rows, fresh pages taken by the launch)."""
    rng = np.random.default_rng(951 + P)
    B, Hq, Hkv, chunk = 40, 16, 4, 256
    lens = rng.integers(0, 1500, B).astype(np.int32)
    lens[:3] = [0, P - 1, P]                    # the new row opens a page, ends one
    wl = gen.Workload("placed-paged", B, Hq, Hkv, "bf16", "const:1", 2, False, seed=961 + P)
    inp = gen.make_inputs(wl, batch=B, lens=lens, steps=2)
    maxp = -(-inp.cap // P)
    pages = int(sum(-(-(int(n) + 2) // P) for n in lens)) + B
    _log(f"placed paged P={P}")

    def mk():
        pc = PagedKVCache(B, Hkv, P, num_pages=pages, max_pages_per_seq=maxp, dtype="bf16")
        pc.load_contiguous(to_device(inp.k_cache), to_device(inp.v_cache), lens)
        return pc

    two, one = mk(), mk()
    Kh, Vh, lh = inp.k_cache.copy(), inp.v_cache.copy(), inp.lens.copy()
    for s in range(2):
        kn, vn, q = to_device(inp.k_new[s]), to_device(inp.v_new[s]), to_device(inp.q_self[s])
        two.append(kn, vn)
        ref_dev = two.attend(q, chunk_rows=chunk)
        got = one.append_attend(kn, vn, q, chunk_rows=chunk)
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref_dev.cpu().numpy().tobytes(), f"paged step {s}"
        lh = oracle.append(Kh, Vh, inp.k_new[s], inp.v_new[s], lh)
        assert_attention_close(got.cpu().numpy(), oracle.attend(inp.q_self[s], Kh, Vh, lh), "bf16",
                               f"placed paged step {s}")
    assert one.lens() == lh.tolist() and one.table() == two.table()
    assert to_host_bits(one.k).tobytes() == to_host_bits(two.k).tobytes()
    assert to_host_bits(one.v).tobytes() == to_host_bits(two.v).tobytes()
