"""A multi-layer decode step captured once in a HIP graph and replayed for
consecutive tokens (replay mode), checked against the oracle after every
replay, with eager library calls between replays; the step either appends
and attends in two calls or through kvdec_append_attend.  The paged form
is replayed the same way, with its pages given between replays
(kvdec_paged_prepare)."""
import gc

import numpy as np
import pytest
import torch

import oracle
from kv_cached_decode_kvdec_amd import inputs as gen
from kv_cached_decode_kvdec_amd import binding as B
from kv_cached_decode_kvdec_amd.cache import KVCache, PagedKVCache, to_device, to_host_bits

from helpers import assert_attention_close

pytestmark = pytest.mark.gpu


def _rows(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else gen.f32_to_bf16_bits(x)


def _new_graph():
    """A graph to capture into, after collecting dead Python cycles: a cycle
    left by an earlier test (an exception info holding its frame, with that
    test's graph and device tensors) must not be freed by the collector in
    the middle of a capture, where freeing device memory is not allowed."""
    gc.collect()
    torch.cuda.synchronize()
    return torch.cuda.CUDAGraph()


@pytest.mark.parametrize("rchunk", [64, 256])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype,Hq,Hkv,cross,window", [("f32", 6, 6, True, 0),
                                                        ("bf16", 16, 4, False, 0),
                                                        ("bf16", 8, 8, False, 128)])
def test_graph_replayed_multilayer_step(dtype, Hq, Hkv, cross, window, fused, rchunk):
    """rchunk 64 splits the 200-row caches over several chunks; 256 holds a
    whole linear cache in one chunk, so the replayed grid has one workgroup
    per sequence and KV head (the direct chunk lookup)."""
    rng = np.random.default_rng(7 + Hq)
    L, B, T, enc = 3, 2, 9, 300
    cap = 200 if window == 0 else window
    start = np.array([5, 150], np.int32) if window == 0 else np.array([5, 300], np.int32)
    total = int(start.max()) + T
    layers = []
    for l in range(L):
        hk = _rows(rng, (B, Hkv, total, 64), dtype)
        hv = _rows(rng, (B, Hkv, total, 64), dtype)
        cp = gen.padded_rows(cap)
        ck = np.zeros((B, Hkv, cp, 64), hk.dtype)
        cv = np.zeros_like(ck)
        for b in range(B):
            for t in range(max(0, start[b] - (window or 10**9)), start[b]):
                slot = t % window if window else t
                ck[b, :, slot] = hk[b, :, t]
                cv[b, :, slot] = hv[b, :, t]
        sc = KVCache(B, Hkv, cap, dtype, lens=start, k=to_device(ck), v=to_device(cv), window=window)
        sc.set_replay_mode(rchunk)
        lay = dict(hk=hk, hv=hv, sc=sc, kn=to_device(np.zeros((B, Hkv, 64), hk.dtype)),
                   vn=to_device(np.zeros((B, Hkv, 64), hk.dtype)),
                   q=torch.zeros(B, Hq, 64, device="cuda"), out=torch.zeros(B, Hq, 64, device="cuda"))
        sc.workspace(Hq)
        if cross:
            xk = _rows(rng, (B, enc, Hkv * 64), dtype)
            xv = _rows(rng, (B, enc, Hkv * 64), dtype)
            cc = KVCache(B, Hkv, enc, dtype, static=True, lens=[0] * B)
            cc.seed(to_device(xk), to_device(xv))
            cc.set_replay_mode(128)
            cc.workspace(Hq)
            xK = np.zeros((B, Hkv, gen.padded_rows(enc), 64), hk.dtype)
            xV = np.zeros_like(xK)
            oracle.seed(xK, xk)
            oracle.seed(xV, xv)
            lay.update(cc=cc, xK=xK, xV=xV, qc=torch.zeros(B, Hq, 64, device="cuda"),
                       cout=torch.zeros(B, Hq, 64, device="cuda"))
        layers.append(lay)
    torch.cuda.synchronize()

    g = _new_graph()
    with torch.cuda.graph(g):
        for lay in layers:
            if fused:   # replay mode: lengths read from and bumped on the device
                lay["sc"].append_attend(lay["kn"], lay["vn"], lay["q"], out=lay["out"])
            else:
                lay["sc"].append(lay["kn"], lay["vn"])
                lay["sc"].attend(lay["q"], out=lay["out"])
            if cross:
                lay["cc"].attend(lay["qc"], out=lay["cout"])

    lens = start.copy()
    for t in range(T):
        qs, qcs = [], []
        for lay in layers:                      # eager work: new token inputs
            kn = np.stack([lay["hk"][b, :, lens[b]] for b in range(B)])
            vn = np.stack([lay["hv"][b, :, lens[b]] for b in range(B)])
            lay["kn"].copy_(to_device(kn))
            lay["vn"].copy_(to_device(vn))
            q = rng.standard_normal((B, Hq, 64), dtype=np.float32)
            lay["q"].copy_(torch.from_numpy(q).cuda())
            qs.append(q)
            if cross:
                qc = rng.standard_normal((B, Hq, 64), dtype=np.float32)
                lay["qc"].copy_(torch.from_numpy(qc).cuda())
                qcs.append(qc)
        g.replay()
        torch.cuda.synchronize()
        lens = lens + 1
        for l, lay in enumerate(layers):
            n = np.minimum(lens, window) if window else lens
            cp = gen.padded_rows(cap)
            lk = np.zeros((B, Hkv, cp, 64), lay["hk"].dtype)
            lv = np.zeros_like(lk)
            for b in range(B):
                lk[b, :, :n[b]] = lay["hk"][b, :, lens[b] - n[b]:lens[b]]
                lv[b, :, :n[b]] = lay["hv"][b, :, lens[b] - n[b]:lens[b]]
            ref = oracle.attend(qs[l], lk, lv, n)
            got = lay["out"].cpu().numpy()
            assert_attention_close(got, ref, dtype, f"replay {t} layer {l} self")
            if cross:
                refc = oracle.attend(qcs[l], lay["xK"], lay["xV"], np.full(B, enc, np.int32))
                assert_attention_close(lay["cout"].cpu().numpy(), refc, dtype,
                                       f"replay {t} layer {l} cross")
            # an eager call between replays sees the same device state
            eager = lay["sc"].attend(lay["q"])
            torch.cuda.synchronize()
            assert torch.equal(eager, lay["out"])
        assert layers[0]["sc"].lens_dev.cpu().tolist() == lens.tolist()


@pytest.mark.parametrize("rchunk", [64, 192])
@pytest.mark.parametrize("dtype,Hq,Hkv", [("f32", 4, 4), ("bf16", 8, 2)])
def test_replay_fused_append_refused_at_capacity(dtype, Hq, Hkv, rchunk):
    """Replay mode cannot check capacity on the host; like kvdec_append, the
    fused call then stores nothing and keeps the length once a linear cache
    is full, and attends the full cache (with 64-row chunks and with one
    chunk per sequence)."""
    rng = np.random.default_rng(91)
    B, cap = 2, 130
    start = np.array([cap - 1, 40], np.int32)
    cp = gen.padded_rows(cap)
    K = _rows(rng, (B, Hkv, cp, 64), dtype)
    V = _rows(rng, (B, Hkv, cp, 64), dtype)
    mk = lambda: KVCache(B, Hkv, cap, dtype, lens=start, k=to_device(K), v=to_device(V))
    two, one = mk(), mk()
    for c in (two, one):
        c.set_replay_mode(rchunk)
    for s in range(3):
        kn = to_device(_rows(rng, (B, Hkv, 64), dtype))
        vn = to_device(_rows(rng, (B, Hkv, 64), dtype))
        q = torch.from_numpy(rng.standard_normal((B, Hq, 64), dtype=np.float32)).cuda()
        two.append(kn, vn)
        ref = two.attend(q)
        got = one.append_attend(kn, vn, q)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"step {s}"
    want = [cap, 43]
    assert one.lens_dev.cpu().tolist() == want and two.lens_dev.cpu().tolist() == want
    assert torch.equal(one.k, two.k) and torch.equal(one.v, two.v)


def test_leaving_replay_mode_needs_lengths_again():
    """Replays append on the device without the host mirror seeing it, so a
    dynamic cache that leaves replay mode refuses mirror-sized calls until
    its lengths are set again; a static cache keeps working."""
    from kv_cached_decode_kvdec_amd import binding as B
    rng = np.random.default_rng(93)
    Bsz, Hkv, Hq, cap = 3, 2, 4, 300
    lens = np.array([10, 0, 130], np.int32)
    cp = gen.padded_rows(cap)
    K = _rows(rng, (Bsz, Hkv, cp, 64), "f32")
    V = _rows(rng, (Bsz, Hkv, cp, 64), "f32")
    c = KVCache(Bsz, Hkv, cap, "f32", lens=lens, k=to_device(K), v=to_device(V))
    st = KVCache(Bsz, Hkv, cap, "f32", static=True, lens=lens, k=to_device(K), v=to_device(V))
    c.set_replay_mode(64)
    st.set_replay_mode(64)
    g = _new_graph()
    kn = to_device(_rows(rng, (Bsz, Hkv, 64), "f32"))
    vn = to_device(_rows(rng, (Bsz, Hkv, 64), "f32"))
    with torch.cuda.graph(g):
        c.append(kn, vn)
    for _ in range(4):                      # four appends the mirror does not see
        g.replay()
    torch.cuda.synchronize()
    c.set_replay_mode(0)
    st.set_replay_mode(0)
    q = to_device(rng.standard_normal((Bsz, Hq, 64), dtype=np.float32))
    for call in (lambda: c.attend(q), lambda: c.append(kn, vn), lambda: c.lens(),
                 lambda: c.append_attend(kn, vn, q)):
        with pytest.raises(B.KvdecError) as e:
            call()
        assert e.value.code == B.KVDEC_E_INVALID
    st.attend(q)                            # static: no appends, mirror still valid
    dev = c.lens_dev.cpu().numpy()
    assert dev.tolist() == (lens + 4).tolist()
    c.reset_lens(dev)
    out = c.attend(q)
    torch.cuda.synchronize()
    Kh, Vh = K.copy(), V.copy()
    kh, vh = kn.cpu().numpy(), vn.cpu().numpy()
    for b in range(Bsz):
        Kh[b, :, lens[b]:lens[b] + 4] = kh[b][:, None, :]
        Vh[b, :, lens[b]:lens[b] + 4] = vh[b][:, None, :]
    assert_attention_close(out.cpu().numpy(), oracle.attend(q.cpu().numpy(), Kh, Vh, dev), "f32",
                           "after reset_lens")


def _history(lay, lens, Bsz, Hkv):
    cap = gen.padded_rows(int(lens.max()))
    K = np.zeros((Bsz, Hkv, cap, 64), lay["hk"].dtype)
    V = np.zeros_like(K)
    for b in range(Bsz):
        K[b, :, :lens[b]] = lay["hk"][b, :, :lens[b]]
        V[b, :, :lens[b]] = lay["hv"][b, :, :lens[b]]
    return K, V


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype,Hq,Hkv,P,rchunk", [("f32", 4, 4, 16, 64), ("bf16", 16, 4, 16, 256),
                                                   ("bf16", 8, 2, 32, 128)])
def test_graph_replayed_paged_step(dtype, Hq, Hkv, P, rchunk, fused):
    """Two paged layers captured once and replayed for 40 tokens that cross
    page boundaries (sequences start empty, one row short of a page, and
    mid-page), pages given by kvdec_paged_prepare between replays.  After
    every replay: the oracle over each sequence's history, and an eager
    attend equal to the replayed one.  At the end: the pool rows reached
    through the block table are the appended rows bit for bit; leaving
    replay mode makes the lengths unknown until kvdec_paged_truncate, and
    the ordinary fused step then continues from them."""
    rng = np.random.default_rng(17 + Hq + P)
    L, Bsz, T = 2, 3, 40
    start = np.array([0, P - 1, 37], np.int32)
    total = int(start.max()) + T + 1
    maxp = -(-total // P)
    layers = []
    for _ in range(L):
        hk = _rows(rng, (Bsz, Hkv, gen.padded_rows(total), 64), dtype)
        hv = _rows(rng, hk.shape, dtype)
        pc = PagedKVCache(Bsz, Hkv, P, num_pages=Bsz * maxp, max_pages_per_seq=maxp, dtype=dtype)
        pc.load_contiguous(to_device(hk), to_device(hv), start)
        pc.set_replay_mode(rchunk)
        if P == 32:                                 # grids sized for the replays ahead
            pc.set_replay_horizon(T + 1)
        pc.workspace(Hq)
        layers.append(dict(hk=hk, hv=hv, pc=pc, kn=to_device(np.zeros((Bsz, Hkv, 64), hk.dtype)),
                           vn=to_device(np.zeros((Bsz, Hkv, 64), hk.dtype)),
                           q=torch.zeros(Bsz, Hq, 64, device="cuda"),
                           out=torch.zeros(Bsz, Hq, 64, device="cuda")))
    torch.cuda.synchronize()

    g = _new_graph()
    with torch.cuda.graph(g):
        for lay in layers:
            if fused:
                lay["pc"].append_attend(lay["kn"], lay["vn"], lay["q"], out=lay["out"])
            else:
                lay["pc"].append(lay["kn"], lay["vn"])
                lay["pc"].attend(lay["q"], out=lay["out"])

    lens = start.copy()
    for t in range(T):
        qs = []
        for lay in layers:
            lay["pc"].prepare(1)                    # pages for the row this replay appends
            kn = np.stack([lay["hk"][b, :, lens[b]] for b in range(Bsz)])
            vn = np.stack([lay["hv"][b, :, lens[b]] for b in range(Bsz)])
            lay["kn"].copy_(to_device(kn))
            lay["vn"].copy_(to_device(vn))
            q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
            lay["q"].copy_(torch.from_numpy(q).cuda())
            qs.append(q)
        g.replay()
        torch.cuda.synchronize()
        lens = lens + 1
        for l, lay in enumerate(layers):
            K, V = _history(lay, lens, Bsz, Hkv)
            assert_attention_close(lay["out"].cpu().numpy(), oracle.attend(qs[l], K, V, lens),
                                   dtype, f"paged replay {t} layer {l}")
            eager = lay["pc"].attend(lay["q"])
            torch.cuda.synchronize()
            assert torch.equal(eager, lay["out"])
        assert layers[0]["pc"].lens_dev.cpu().tolist() == lens.tolist()
        assert layers[0]["pc"].lens() == lens.tolist()     # the prepared rows, all appended

    for lay in layers:
        pc = lay["pc"]
        table, tdev = pc.table(), pc.table_dev.cpu().numpy()
        kp, vp = to_host_bits(pc.k), to_host_bits(pc.v)
        for b in range(Bsz):
            n = -(-int(lens[b]) // P)
            assert tdev[b, :n].tolist() == table[b][:n]
            assert (tdev[b, n:] == -1).all()
            for r in range(int(lens[b])):
                assert kp[:, table[b][r // P], r % P].tobytes() == lay["hk"][b, :, r].tobytes()
                assert vp[:, table[b][r // P], r % P].tobytes() == lay["hv"][b, :, r].tobytes()
        pc.set_replay_mode(0)
        with pytest.raises(B.KvdecError) as e:
            pc.lens()
        assert e.value.code == B.KVDEC_E_INVALID
        with pytest.raises(B.KvdecError) as e:
            pc.attend(lay["q"])
        assert e.value.code == B.KVDEC_E_INVALID
        pc.truncate(lens)
        assert pc.lens() == lens.tolist()

    # the ordinary one-launch step continues from the lengths set again
    for l, lay in enumerate(layers):
        kn = np.stack([lay["hk"][b, :, lens[b]] for b in range(Bsz)])
        vn = np.stack([lay["hv"][b, :, lens[b]] for b in range(Bsz)])
        q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
        out = lay["pc"].append_attend(to_device(kn), to_device(vn), to_device(q))
        torch.cuda.synchronize()
        K, V = _history(lay, lens + 1, Bsz, Hkv)
        assert_attention_close(out.cpu().numpy(), oracle.attend(q, K, V, lens + 1), dtype,
                               f"after replay mode, layer {l}")


def test_paged_replay_rows_without_pages_are_dropped():
    """In replay mode an append whose row has no page in the block table
    (not prepared, or a page returned to the pool) writes nothing and keeps
    that sequence's length; rows in held pages are appended.  Entering replay
    mode leaves -1 past every sequence's pages in the device table, and a
    release in replay mode clears the released pages' entries."""
    rng = np.random.default_rng(23)
    Bsz, Hkv, Hq, P = 3, 2, 4, 16
    pc = PagedKVCache(Bsz, Hkv, P, num_pages=8, max_pages_per_seq=3, dtype="f32")
    K = _rows(rng, (Bsz, Hkv, 64, 64), "f32")
    pc.load_contiguous(to_device(K), to_device(K), np.array([16, 5, 20], np.int32))
    assert pc.table_dev.cpu().numpy()[2, :2].min() >= 0
    pc.release(2)                        # its two pages return to the pool
    pc.set_replay_mode(64)
    kn = to_device(_rows(rng, (Bsz, Hkv, 64), "f32"))
    before = to_host_bits(pc.k).copy()
    pc.append(kn, kn)                    # row 16 starts a page: none; row 5: held; row 0: none
    torch.cuda.synchronize()
    assert pc.lens_dev.cpu().tolist() == [16, 6, 0]
    after = to_host_bits(pc.k)
    page1 = pc.table()[1][0]
    changed = np.argwhere((before != after).any(axis=-1))
    assert {(int(g), int(p), int(r)) for g, p, r in changed} <= {(g, page1, 5) for g in range(Hkv)}
    assert pc.table_dev.cpu().numpy()[2].tolist() == [-1, -1, -1]
    with pytest.raises(B.KvdecError) as e:
        pc.prepare(-1)
    assert e.value.code == B.KVDEC_E_INVALID
    with pytest.raises(B.KvdecError) as e:
        pc.prepare(40)                   # 16 + 40 rows > 3 pages of 16
    assert e.value.code == B.KVDEC_E_OVERFLOW
    pc.prepare(1)                        # pages for rows 16 (sequence 0) and 0 (sequence 2)
    pc.append(kn, kn)
    torch.cuda.synchronize()
    assert pc.lens_dev.cpu().tolist() == [17, 7, 1]
    pc.release(0)                        # in replay mode: its entries become -1 at once
    torch.cuda.synchronize()
    assert pc.table_dev.cpu().numpy()[0].tolist() == [-1, -1, -1]
    pc.append(kn, kn)                    # sequence 0 (row 0) has no page again
    torch.cuda.synchronize()
    assert pc.lens_dev.cpu().tolist() == [0, 8, 2]
    pc.set_replay_mode(0)
    with pytest.raises(B.KvdecError):
        pc.truncate([0, 17, 2])          # more than sequence 1's page holds
    pc.truncate([0, 8, 2])               # sequences 1 and 2 ran past their prepared lengths
    assert pc.lens() == [0, 8, 2]
    with pytest.raises(B.KvdecError):
        pc.prepare(1)                    # outside replay mode


@pytest.mark.parametrize("dtype,Hq,Hkv", [("f32", 4, 2), ("bf16", 8, 2), ("bf16", 4, 4)])
def test_paged_replay_fused_step_without_pages(dtype, Hq, Hkv):
    """The one-launch paged step in replay mode (lengths from the device, the
    new row stored in the page the table holds for it): a sequence whose new
    row has no page keeps its length and attends the rows it had; the others
    append and attend len + 1 rows.  Checked against the oracle, with the
    pool bytes of every row compared."""
    rng = np.random.default_rng(29 + Hq)
    Bsz, P = 4, 16
    lens = np.array([16, 5, 0, 70], np.int32)          # row 16 starts a page; 5 and 70 are mid-page
    K = _rows(rng, (Bsz, Hkv, 128, 64), dtype)         # 64-row chunks: sequence 3 spans two
    V = _rows(rng, (Bsz, Hkv, 128, 64), dtype)
    pc = PagedKVCache(Bsz, Hkv, P, num_pages=40, max_pages_per_seq=8, dtype=dtype)
    pc.load_contiguous(to_device(K), to_device(V), lens)
    pc.set_replay_mode(64)
    kn = _rows(rng, (Bsz, Hkv, 64), dtype)
    vn = _rows(rng, (Bsz, Hkv, 64), dtype)
    q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
    out = pc.append_attend(to_device(kn), to_device(vn), to_device(q))
    torch.cuda.synchronize()
    stored = np.array([False, True, False, True])
    new = lens + stored
    Kh, Vh = K.copy(), V.copy()
    for b in np.flatnonzero(stored):
        Kh[b, :, lens[b]], Vh[b, :, lens[b]] = kn[b], vn[b]
    assert pc.lens_dev.cpu().tolist() == new.tolist()
    assert_attention_close(out.cpu().numpy(), oracle.attend(q, Kh, Vh, new), dtype, "paged replay fused")
    table, kp, vp = pc.table(), to_host_bits(pc.k), to_host_bits(pc.v)
    for b in range(Bsz):
        for r in range(int(new[b])):
            assert kp[:, table[b][r // P], r % P].tobytes() == Kh[b, :, r].tobytes()
            assert vp[:, table[b][r // P], r % P].tobytes() == Vh[b, :, r].tobytes()
    pc.prepare(1)                                      # now every next row has a page
    q2 = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
    out2 = pc.append_attend(to_device(kn), to_device(vn), to_device(q2))
    torch.cuda.synchronize()
    for b in range(Bsz):
        Kh[b, :, new[b]], Vh[b, :, new[b]] = kn[b], vn[b]
    assert pc.lens_dev.cpu().tolist() == (new + 1).tolist()
    assert_attention_close(out2.cpu().numpy(), oracle.attend(q2, Kh, Vh, new + 1), dtype,
                           "paged replay fused, prepared")


@pytest.mark.parametrize("fused", [False, True])
def test_replay_horizon_sizes_grids_per_sequence(fused):
    """With a replay horizon the captured launches cover each sequence's rows
    at capture plus the horizon, not the capacity: replays within it match
    the oracle; the replay whose lengths outgrow the grid gives NaN rows for
    the sequence past its end (and, fused, leaves that length) and correct
    rows for the others; resetting the lengths makes the graph valid again."""
    rng = np.random.default_rng(31 + fused)
    Bsz, Hkv, Hq, cap, T, H = 3, 2, 4, 256, 64, 2
    start = np.array([62, 10, 122], np.int32)
    cp = gen.padded_rows(cap)
    hk = _rows(rng, (Bsz, Hkv, cp, 64), "f32")
    hv = _rows(rng, (Bsz, Hkv, cp, 64), "f32")
    c = KVCache(Bsz, Hkv, cap, "f32", lens=start, k=to_device(hk), v=to_device(hv))
    c.set_replay_mode(T)
    c.set_replay_horizon(H)
    c.workspace(Hq)
    kn = to_device(np.zeros((Bsz, Hkv, 64), np.float32))
    vn = to_device(np.zeros((Bsz, Hkv, 64), np.float32))
    q = torch.zeros(Bsz, Hq, 64, device="cuda")
    out = torch.zeros(Bsz, Hq, 64, device="cuda")
    torch.cuda.synchronize()
    g = _new_graph()
    with torch.cuda.graph(g):
        if fused:
            c.append_attend(kn, vn, q, out=out)
        else:
            c.append(kn, vn)
            c.attend(q, out=out)
    # rows at capture: start + 1 (the captured append advanced the mirror)
    grid = int(sum(-(-min(int(n) + 1 + H, cap) // T) for n in start))
    K, V = hk.copy(), hv.copy()
    lens = start.copy()
    for t in range(7):
        rows = np.stack([K[b, :, lens[b]] for b in range(Bsz)]), np.stack([V[b, :, lens[b]] for b in range(Bsz)])
        kn.copy_(to_device(rows[0]))
        vn.copy_(to_device(rows[1]))
        qh = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
        q.copy_(torch.from_numpy(qh).cuda())
        g.replay()
        torch.cuda.synchronize()
        n = lens + 1
        covered = np.cumsum([-(-int(x) // T) for x in n]) <= grid
        got = out.cpu().numpy()
        ref = oracle.attend(qh, K, V, n.astype(np.int32))
        for b in range(Bsz):
            if covered[b]:
                assert_attention_close(got[b:b + 1], ref[b:b + 1], "f32", f"replay {t} seq {b}")
            else:
                assert np.isnan(got[b]).all(), f"replay {t} seq {b}: outgrown grid must give NaN"
        if fused:
            lens = np.where(covered, n, lens)
        else:
            lens = n
        assert c.lens_dev.cpu().tolist() == lens.tolist()
        if t < 6:
            assert covered.all()
        else:
            assert covered.tolist() == [True, True, False]
    c.reset_lens(start)
    qh = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
    q.copy_(torch.from_numpy(qh).cuda())
    kn.copy_(to_device(np.stack([K[b, :, start[b]] for b in range(Bsz)])))
    vn.copy_(to_device(np.stack([V[b, :, start[b]] for b in range(Bsz)])))
    g.replay()
    torch.cuda.synchronize()
    assert_attention_close(out.cpu().numpy(), oracle.attend(qh, K, V, start + 1), "f32",
                           "after resetting the lengths")


@pytest.mark.parametrize("fused", [False, True])
def test_replay_horizon_one_chunk_grid_outgrown(fused):
    """A horizon grid with exactly one workgroup per sequence (rows at capture
    plus the horizon fit one chunk) while the capacity spans several chunks:
    the launch must still find each workgroup's sequence from the device
    lengths (the grid size says nothing about them).  Once sequence 0 grows
    past one chunk the grid no longer reaches sequence 2: its output rows
    are NaN and, fused, its row is not stored and its length stays; the
    other sequences stay exact, sequence 0 over its two chunks included."""
    rng = np.random.default_rng(41 + fused)
    Bsz, Hkv, Hq, cap, T, H = 3, 2, 4, 256, 64, 2
    start = np.array([60, 20, 30], np.int32)      # rows at capture: 61, 21, 31 (+2 fit 64)
    cp = gen.padded_rows(cap)
    hk = _rows(rng, (Bsz, Hkv, cp, 64), "f32")
    hv = _rows(rng, (Bsz, Hkv, cp, 64), "f32")
    c = KVCache(Bsz, Hkv, cap, "f32", lens=start, k=to_device(hk), v=to_device(hv))
    c.set_replay_mode(T)
    c.set_replay_horizon(H)
    c.workspace(Hq)
    kn = to_device(np.zeros((Bsz, Hkv, 64), np.float32))
    vn = to_device(np.zeros((Bsz, Hkv, 64), np.float32))
    q = torch.zeros(Bsz, Hq, 64, device="cuda")
    out = torch.zeros(Bsz, Hq, 64, device="cuda")
    torch.cuda.synchronize()
    g = _new_graph()
    with torch.cuda.graph(g):
        if fused:
            c.append_attend(kn, vn, q, out=out)
        else:
            c.append(kn, vn)
            c.attend(q, out=out)
    grid = Bsz                                     # one chunk per sequence at capture + H
    K, V = hk.copy(), hv.copy()
    lens = start.copy()
    cache_k = to_host_bits(c.k)
    seen_outgrown = False
    for t in range(6):
        new_k = _rows(rng, (Bsz, Hkv, 64), "f32")
        new_v = _rows(rng, (Bsz, Hkv, 64), "f32")
        kn.copy_(to_device(new_k))
        vn.copy_(to_device(new_v))
        qh = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
        q.copy_(torch.from_numpy(qh).cuda())
        g.replay()
        torch.cuda.synchronize()
        n = lens + 1
        covered = np.cumsum([-(-int(x) // T) for x in n]) <= grid
        seen_outgrown |= not covered.all()
        for b in range(Bsz):
            if covered[b] or not fused:
                K[b, :, lens[b]], V[b, :, lens[b]] = new_k[b], new_v[b]
        got = out.cpu().numpy()
        for b in range(Bsz):
            if covered[b]:
                ref = oracle.attend(qh[b:b + 1], K[b:b + 1], V[b:b + 1], n[b:b + 1].astype(np.int32))
                assert_attention_close(got[b:b + 1], ref, "f32", f"replay {t} seq {b}")
            else:
                assert np.isnan(got[b]).all(), f"replay {t} seq {b}: outgrown grid must give NaN"
        lens = np.where(covered, n, lens) if fused else n
        assert c.lens_dev.cpu().tolist() == lens.tolist(), f"replay {t}"
        if fused:
            # the sequence the grid no longer reaches got no row: its cache is as it was
            now_k = to_host_bits(c.k)
            for b in np.flatnonzero(~covered):
                assert now_k[b].tobytes() == cache_k[b].tobytes(), f"replay {t} seq {b} cache"
            cache_k = now_k
    assert seen_outgrown
