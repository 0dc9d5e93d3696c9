"""A multi-layer decode step captured once in a HIP graph and replayed for
consecutive tokens (replay mode), checked against the oracle after every
replay, with eager library calls between replays; the step either appends
and attends in two calls or through kvdec_append_attend."""
import numpy as np
import pytest
import torch

import oracle
from kv_cached_decode_kvdec_amd import inputs as gen
from kv_cached_decode_kvdec_amd.cache import KVCache, to_device

from helpers import assert_attention_close

pytestmark = pytest.mark.gpu


def _rows(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else gen.f32_to_bf16_bits(x)


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

    g = torch.cuda.CUDAGraph()
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
    g = torch.cuda.CUDAGraph()
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
