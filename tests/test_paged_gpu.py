"""Paged KV cache: page pool + block table + host page allocator.

Attention through the block table is compared with the oracle on each
sequence's linear history; the pool rows reached through the table must be
the appended rows bit for bit; pages are never shared, come back on
release, and an exhausted pool or a full block table changes nothing.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cached_decode_kvdec_amd import binding as B
from kv_cached_decode_kvdec_amd import inputs as gen
from kv_cached_decode_kvdec_amd.cache import PagedKVCache, to_device, to_host_bits

from helpers import assert_attention_close

pytestmark = pytest.mark.gpu


def _rows(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else gen.f32_to_bf16_bits(x)


@pytest.mark.parametrize("dtype,Hq,Hkv,P", [("f32", 8, 8, 16), ("bf16", 16, 4, 16),
                                            ("bf16", 16, 4, 64), ("f32", 6, 2, 32)])
def test_paged_parity_and_pool_contents(dtype, Hq, Hkv, P):
    rng = np.random.default_rng(5 + P + Hq)
    Bsz, steps = 4, 300
    max_pages = (steps + P - 1) // P + 1
    pc = PagedKVCache(Bsz, Hkv, P, num_pages=Bsz * max_pages, max_pages_per_seq=max_pages,
                      dtype=dtype)
    hist = [[] for _ in range(Bsz)]        # per sequence: list of (k [Hkv,64], v [Hkv,64])
    checked = 0
    for s in range(steps):
        if s == 170:                       # end sequence 2 and start it again from empty
            pc.release(2)
            hist[2] = []
        kn = _rows(rng, (Bsz, Hkv, 64), dtype)
        vn = _rows(rng, (Bsz, Hkv, 64), dtype)
        pc.append(to_device(kn), to_device(vn))
        for b in range(Bsz):
            hist[b].append((kn[b], vn[b]))
        if s % 37 == 0 or s == steps - 1 or s == 170:
            q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
            out = pc.attend(to_device(q), chunk_rows=0 if s % 2 else 64)
            torch.cuda.synchronize()
            lens = np.array([len(h) for h in hist], np.int32)
            cap = gen.padded_rows(int(lens.max()))
            K = np.zeros((Bsz, Hkv, cap, 64), kn.dtype)
            V = np.zeros_like(K)
            for b in range(Bsz):
                for r, (kr, vr) in enumerate(hist[b]):
                    K[b, :, r], V[b, :, r] = kr, vr
            ref = oracle.attend(q, K, V, lens)
            assert_attention_close(out.cpu().numpy(), ref, dtype, f"paged step {s}")
            checked += 1
    assert checked >= 9
    lens = [len(h) for h in hist]
    assert pc.lens() == lens and pc.lens_dev.cpu().tolist() == lens
    table = pc.table()
    held = [p for b in range(Bsz) for p in table[b] if p >= 0]
    assert len(held) == len(set(held)), "a page is shared between sequences"
    assert pc.free_pages() == pc.num_pages - len(held)
    assert len(held) == sum((n + P - 1) // P for n in lens)
    # the device block table agrees with the host mirror where pages are held
    tdev = pc.table_dev.cpu().numpy()
    for b in range(Bsz):
        n = (lens[b] + P - 1) // P
        assert tdev[b, :n].tolist() == table[b][:n]
    # pool rows reached through the table are the appended rows, bit for bit
    kp, vp = to_host_bits(pc.k), to_host_bits(pc.v)
    for b in range(Bsz):
        for r, (kr, vr) in enumerate(hist[b]):
            page, slot = table[b][r // P], r % P
            assert kp[:, page, slot].tobytes() == kr.tobytes()
            assert vp[:, page, slot].tobytes() == vr.tobytes()


def test_paged_allocator_limits_change_nothing():
    P = 16
    pc = PagedKVCache(2, 1, P, num_pages=3, max_pages_per_seq=2, dtype="f32")
    k = torch.ones(2, 1, 64, device="cuda")
    for _ in range(P):
        pc.append(k, k)                    # 2 pages held, 1 free
    assert pc.free_pages() == 1
    with pytest.raises(B.KvdecError) as e:
        pc.append(k, k)                    # both sequences need a page: pool exhausted
    assert e.value.code == B.KVDEC_E_OVERFLOW
    torch.cuda.synchronize()
    assert pc.lens() == [P, P] and pc.lens_dev.cpu().tolist() == [P, P]
    assert pc.free_pages() == 1 and pc.table()[1][1] == -1
    pc.release(0)
    assert pc.free_pages() == 2 and pc.lens() == [0, P]
    for _ in range(P):
        pc.append(k, k)                    # seq 0 refills one page, seq 1 takes its second
    assert pc.lens() == [P, 2 * P] and pc.free_pages() == 0
    with pytest.raises(B.KvdecError) as e:
        pc.append(k, k)                    # seq 1 is at max_pages_per_seq * P
    assert e.value.code == B.KVDEC_E_OVERFLOW
    torch.cuda.synchronize()
    assert pc.lens_dev.cpu().tolist() == [P, 2 * P]


def test_paged_reserve_truncate_roundtrip():
    rng = np.random.default_rng(77)
    Bsz, Hkv, Hq, P = 3, 4, 16, 16
    lens0 = np.array([0, 37, 300], np.int32)
    cap = 400
    K = _rows(rng, (Bsz, Hkv, gen.padded_rows(cap), 64), "bf16")
    V = _rows(rng, (Bsz, Hkv, gen.padded_rows(cap), 64), "bf16")
    pc = PagedKVCache(Bsz, Hkv, P, num_pages=60, max_pages_per_seq=(cap + P - 1) // P, dtype="bf16")
    pc.load_contiguous(to_device(K), to_device(V), lens0)
    assert pc.lens() == lens0.tolist()
    q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
    out = pc.attend(to_device(q))
    torch.cuda.synchronize()
    assert_attention_close(out.cpu().numpy(), oracle.attend(q, K, V, lens0), "bf16", "reserved")
    free0 = pc.free_pages()
    # grow by 20 tokens, then roll back to the reserved lengths
    for _ in range(20):
        kn = _rows(rng, (Bsz, Hkv, 64), "bf16")
        pc.append(to_device(kn), to_device(kn))
    assert pc.lens() == (lens0 + 20).tolist() and pc.free_pages() < free0
    pc.truncate(lens0)
    assert pc.lens() == lens0.tolist() and pc.free_pages() == free0
    out2 = pc.attend(to_device(q))
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    with pytest.raises(B.KvdecError):
        pc.reserve(1, 5)                   # not empty
    with pytest.raises(B.KvdecError):
        pc.truncate([0, 38, 300])          # cannot grow by truncation


@pytest.mark.parametrize("dtype,Hq,Hkv,P,T", [("f32", 8, 8, 16, 0), ("bf16", 16, 4, 16, 64),
                                              ("bf16", 8, 8, 64, 0), ("f32", 6, 2, 32, 128),
                                              ("bf16", 12, 3, 16, 256)])
def test_paged_fused_equals_append_then_attend(dtype, Hq, Hkv, P, T):
    """kvdec_paged_append_attend == kvdec_paged_append + kvdec_paged_attend,
    bitwise: output, pool rows, block table, lengths, free pages."""
    rng = np.random.default_rng(31 + P + Hq)
    Bsz, steps = 5, 70
    start = np.array([0, 15, 16, 47, 100], np.int32)      # empty, about to start a page, ...
    max_pages = (int(start.max()) + steps + P - 1) // P + 1
    mk = lambda: PagedKVCache(Bsz, Hkv, P, num_pages=Bsz * max_pages, max_pages_per_seq=max_pages,
                              dtype=dtype)
    two, one = mk(), mk()
    K0 = _rows(rng, (Bsz, Hkv, gen.padded_rows(int(start.max()) + 1), 64), dtype)
    V0 = _rows(rng, K0.shape, dtype)
    for c in (two, one):
        c.load_contiguous(to_device(K0), to_device(V0), start)
    hist = [[(K0[b, :, r], V0[b, :, r]) for r in range(start[b])] for b in range(Bsz)]
    for s in range(steps):
        kn = _rows(rng, (Bsz, Hkv, 64), dtype)
        vn = _rows(rng, (Bsz, Hkv, 64), dtype)
        q_h = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
        q = to_device(q_h)
        two.append(to_device(kn), to_device(vn))
        ref_dev = two.attend(q, chunk_rows=T)
        got = one.append_attend(to_device(kn), to_device(vn), q, chunk_rows=T)
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref_dev.cpu().numpy().tobytes(), f"step {s}"
        for b in range(Bsz):
            hist[b].append((kn[b], vn[b]))
        if s % 23 == 0 or s == steps - 1:
            lens = np.array([len(h) for h in hist], np.int32)
            cap = gen.padded_rows(int(lens.max()))
            K = np.zeros((Bsz, Hkv, cap, 64), kn.dtype)
            V = np.zeros_like(K)
            for b in range(Bsz):
                for r, (kr, vr) in enumerate(hist[b]):
                    K[b, :, r], V[b, :, r] = kr, vr
            assert_attention_close(got.cpu().numpy(), oracle.attend(q_h, K, V, lens), dtype,
                                   f"paged fused step {s}")
    assert one.lens() == two.lens() and one.table() == two.table()
    assert one.free_pages() == two.free_pages()
    assert one.lens_dev.cpu().tolist() == two.lens_dev.cpu().tolist()
    assert torch.equal(one.table_dev, two.table_dev)
    assert to_host_bits(one.k).tobytes() == to_host_bits(two.k).tobytes()
    assert to_host_bits(one.v).tobytes() == to_host_bits(two.v).tobytes()


def test_paged_fused_large_batch_and_errors():
    """Above KVDEC_MAX_PAGED_FUSED_BATCH the call runs the two launches (same
    results); refused calls change nothing (no page taken)."""
    rng = np.random.default_rng(41)
    Bsz, Hkv, Hq, P = B.KVDEC_MAX_PAGED_FUSED_BATCH + 3, 2, 4, 16
    mk = lambda n: PagedKVCache(Bsz, Hkv, P, num_pages=n, max_pages_per_seq=3, dtype="f32")
    two, one = mk(Bsz * 3), mk(Bsz * 3)
    for s in range(20):
        kn = to_device(_rows(rng, (Bsz, Hkv, 64), "f32"))
        vn = to_device(_rows(rng, (Bsz, Hkv, 64), "f32"))
        q = to_device(rng.standard_normal((Bsz, Hq, 64), dtype=np.float32))
        two.append(kn, vn)
        ref = two.attend(q)
        got = one.append_attend(kn, vn, q)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"large batch step {s}"
    assert one.lens() == two.lens() and one.table() == two.table()
    assert to_host_bits(one.k).tobytes() == to_host_bits(two.k).tobytes()

    small = PagedKVCache(4, Hkv, P, num_pages=4, max_pages_per_seq=2, dtype="f32")
    kn = to_device(_rows(rng, (4, Hkv, 64), "f32"))
    q = to_device(rng.standard_normal((4, Hq, 64), dtype=np.float32))
    small.append_attend(kn, kn, q)                      # every sequence takes a page: pool empty
    table, free = small.table(), small.free_pages()
    ws = small.workspace(Hq)
    with pytest.raises(B.KvdecError) as e:              # workspace one byte short
        B.kvdec_paged_append_attend(small.handle, kn.data_ptr(), kn.data_ptr(), q.data_ptr(), Hq,
                                    0.125, 0, q.data_ptr(), ws.data_ptr(), ws.numel() - 1)
    assert e.value.code == B.KVDEC_E_WORKSPACE
    torch.cuda.synchronize()
    assert small.lens() == [1] * 4 and small.lens_dev.cpu().tolist() == [1] * 4
    for _ in range(P - 1):
        small.append_attend(kn, kn, q)                  # fills the pages
    with pytest.raises(B.KvdecError) as e:
        small.append_attend(kn, kn, q)                  # next row needs a page: none free
    assert e.value.code == B.KVDEC_E_OVERFLOW
    torch.cuda.synchronize()
    assert small.lens() == [P] * 4 and small.table() == table and free == 0
    assert small.lens_dev.cpu().tolist() == [P] * 4
