"""Edge sizes of the decode step against the f64 oracle, through the C ABI.

- one very long sequence split into more than a thousand chunks (the merge
  walks its chunk list in several 64-chunk groups and 16-chunk batches);
- a batch of 2048 short ragged sequences (the chunk lookup scans the lengths
  in 32 groups of 64; most sequences fit one chunk, some span two);
- the fused append at exactly its largest batch (512), where it still runs as
  one launch;
- group 8 over a single KV head with a ragged batch, through the fused call;
- 48 KV heads (the launch grid's second dimension) in both kernel families;
- two independent caches driven on two streams at once;
- f32 launches large enough for the 16-wave workgroups (plain, fused, paged,
  paged fused, and the device-length fused step on a replay grid sized with
  a horizon);
- ragged batches of 60,000 and 70,000 one- and two-row sequences: the grid
  of a ragged launch puts the KV heads along x and the chunks along y, up to
  y's limit of 65,535; past it the chunks go back along x.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from kv_cached_decode_kvdec_amd import binding as B
from kv_cached_decode_kvdec_amd import inputs as gen
from kv_cached_decode_kvdec_amd.cache import KVCache, PagedKVCache, to_device, to_host_bits

from helpers import assert_attention_close

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _rows(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else gen.f32_to_bf16_bits(x)


def test_one_sequence_over_a_thousand_chunks():
    rng = np.random.default_rng(81)
    L, Hkv, Hq = 100_000, 1, 8
    cap = gen.padded_rows(L)
    K = _rows(rng, (1, Hkv, cap, 64), "bf16")
    V = _rows(rng, (1, Hkv, cap, 64), "bf16")
    q = rng.standard_normal((1, Hq, 64), dtype=np.float32)
    _log(f"long sequence: {L} rows, chunk 64 -> {-(-L // 64)} chunks")
    c = KVCache(1, Hkv, L, "bf16", lens=[L], k=to_device(K), v=to_device(V))
    ref = oracle.attend(q, K, V, np.array([L], np.int32))
    for T in (64, 4096, 0):
        out = c.attend(to_device(q), chunk_rows=T)
        torch.cuda.synchronize()
        assert_attention_close(out.cpu().numpy(), ref, "bf16", f"L={L} T={T}")


def test_batch_of_2048_ragged_sequences():
    rng = np.random.default_rng(82)
    Bsz, Hkv, Hq = 2048, 2, 4
    lens = rng.integers(0, 130, size=Bsz).astype(np.int32)
    lens[::97] = 0
    cap = gen.padded_rows(int(lens.max()) + 1)
    K = _rows(rng, (Bsz, Hkv, cap, 64), "f32")
    V = _rows(rng, (Bsz, Hkv, cap, 64), "f32")
    q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
    _log(f"batch {Bsz}: lengths 0..{lens.max()}")
    c = KVCache(Bsz, Hkv, cap, "f32", lens=lens, k=to_device(K), v=to_device(V))
    ref = oracle.attend(q, K, V, lens)
    for T in (64, 128, 0):
        out = c.attend(to_device(q), chunk_rows=T)
        torch.cuda.synchronize()
        assert_attention_close(out.cpu().numpy(), ref, "f32", f"B={Bsz} T={T}")


@pytest.mark.parametrize("Bsz", [B.KVDEC_MAX_FUSED_BATCH, 1])
def test_fused_append_at_its_batch_limits(Bsz):
    rng = np.random.default_rng(83 + Bsz)
    Hkv, Hq = 1, 8                                   # group 8 on the VALU kernel
    lens = rng.integers(0, 200, size=Bsz).astype(np.int32)
    cap = gen.padded_rows(int(lens.max()) + 2)
    K = _rows(rng, (Bsz, Hkv, cap, 64), "bf16")
    V = _rows(rng, (Bsz, Hkv, cap, 64), "bf16")
    for b in range(Bsz):                             # canaries past each length
        K[b, :, lens[b]:] = 0x7FC1
        V[b, :, lens[b]:] = 0x7FC1
    _log(f"fused append at batch {Bsz}")
    c = KVCache(Bsz, Hkv, cap, "bf16", lens=lens, k=to_device(K), v=to_device(V))
    Kh, Vh, ln = K.copy(), V.copy(), lens.copy()
    for s in range(2):
        kn = _rows(rng, (Bsz, Hkv, 64), "bf16")
        vn = _rows(rng, (Bsz, Hkv, 64), "bf16")
        q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
        out = c.append_attend(to_device(kn), to_device(vn), to_device(q), chunk_rows=64 * (s + 1))
        torch.cuda.synchronize()
        ln = oracle.append(Kh, Vh, kn, vn, ln)
        ref = oracle.attend(q, Kh, Vh, ln)
        assert_attention_close(out.cpu().numpy(), ref, "bf16", f"fused B={Bsz} step {s}")
    assert to_host_bits(c.k).tobytes() == Kh.tobytes()
    assert to_host_bits(c.v).tobytes() == Vh.tobytes()
    assert c.lens() == ln.tolist() and c.lens_dev.cpu().tolist() == ln.tolist()


def test_many_kv_heads():
    """48 KV heads (grid y) with two query heads each, bf16 (MFMA) and f32 (VALU)."""
    for dtype in ("bf16", "f32"):
        rng = np.random.default_rng(84)
        Bsz, Hkv, Hq = 3, 48, 96
        lens = np.array([300, 0, 777], np.int32)
        cap = gen.padded_rows(int(lens.max()) + 1)
        K = _rows(rng, (Bsz, Hkv, cap, 64), dtype)
        V = _rows(rng, (Bsz, Hkv, cap, 64), dtype)
        q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
        _log(f"{Hkv} KV heads, {dtype}")
        c = KVCache(Bsz, Hkv, cap, dtype, lens=lens, k=to_device(K), v=to_device(V))
        ref = oracle.attend(q, K, V, lens)
        for T in (64, 0):
            out = c.attend(to_device(q), chunk_rows=T)
            torch.cuda.synchronize()
            assert_attention_close(out.cpu().numpy(), ref, dtype, f"{dtype} Hkv={Hkv} T={T}")


def test_independent_caches_on_two_streams():
    """The library keeps no state outside its handles: two caches driven on two
    streams at once (append + attend, fused and not) give the oracle's results."""
    rng = np.random.default_rng(85)
    setups = []
    for dtype, Hkv, Hq, Bsz in (("f32", 4, 8, 7), ("bf16", 2, 8, 9)):
        lens = rng.integers(50, 900, size=Bsz).astype(np.int32)
        cap = gen.padded_rows(int(lens.max()) + 4)
        K = _rows(rng, (Bsz, Hkv, cap, 64), dtype)
        V = _rows(rng, (Bsz, Hkv, cap, 64), dtype)
        setups.append(dict(dtype=dtype, Hkv=Hkv, Hq=Hq, B=Bsz, lens=lens, K=K, V=V, cap=cap))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    caches, refs, outs = [], [], []
    for st, s in zip(streams, setups):
        with torch.cuda.stream(st):
            caches.append(KVCache(s["B"], s["Hkv"], s["cap"], s["dtype"], lens=s["lens"],
                                  k=to_device(s["K"]), v=to_device(s["V"])))
    torch.cuda.synchronize()
    for step in range(3):
        inputs = []
        for s in setups:
            kn = _rows(rng, (s["B"], s["Hkv"], 64), s["dtype"])
            vn = _rows(rng, (s["B"], s["Hkv"], 64), s["dtype"])
            q = rng.standard_normal((s["B"], s["Hq"], 64), dtype=np.float32)
            inputs.append((kn, vn, q, to_device(kn), to_device(vn), to_device(q)))
        torch.cuda.synchronize()
        outs = []
        for st, c, (kn, vn, q, dkn, dvn, dq) in zip(streams, caches, inputs):
            with torch.cuda.stream(st):
                if step % 2 == 0:
                    outs.append(c.append_attend(dkn, dvn, dq, chunk_rows=64))
                else:
                    c.append(dkn, dvn)
                    outs.append(c.attend(dq, chunk_rows=128))
        torch.cuda.synchronize()
        for s, out, (kn, vn, q, *_rest) in zip(setups, outs, inputs):
            s["lens"] = oracle.append(s["K"], s["V"], kn, vn, s["lens"])
            ref = oracle.attend(q, s["K"], s["V"], s["lens"])
            assert_attention_close(out.cpu().numpy(), ref, s["dtype"], f"{s['dtype']} step {step}")
    for s, c in zip(setups, caches):
        assert to_host_bits(c.k).tobytes() == s["K"].tobytes()
        assert c.lens() == s["lens"].tolist()


@pytest.mark.parametrize("mode", ["attend", "fused", "paged", "paged_fused", "replay_fused"])
@pytest.mark.parametrize("group", [1, 2])
def test_wide_workgroups(group, mode):
    """f32 with 1 or 2 query heads per KV head and at least four residency
    rounds of 256-row chunks runs on 16-wave workgroups."""
    rng = np.random.default_rng(86 + group)
    Bsz, Hkv = 64, 8
    Hq = Hkv * group
    lens = rng.integers(1000, 1500, size=Bsz).astype(np.int32)   # >= 4 chunks each: 2048+ workgroups
    cap = gen.padded_rows(int(lens.max()) + 1)
    K = _rows(rng, (Bsz, Hkv, cap, 64), "f32")
    V = _rows(rng, (Bsz, Hkv, cap, 64), "f32")
    q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
    _log(f"wide workgroups: group {group}, {mode}")
    if mode.startswith("paged"):
        P = 32
        maxp = cap // P
        pc = PagedKVCache(Bsz, Hkv, P, num_pages=Bsz * maxp, max_pages_per_seq=maxp, dtype="f32")
        pc.load_contiguous(to_device(K), to_device(V), lens)
        if mode == "paged":
            out = pc.attend(to_device(q), chunk_rows=256)
            ref = oracle.attend(q, K, V, lens)
        else:
            kn = _rows(rng, (Bsz, Hkv, 64), "f32")
            vn = _rows(rng, (Bsz, Hkv, 64), "f32")
            out = pc.append_attend(to_device(kn), to_device(vn), to_device(q), chunk_rows=256)
            ln = oracle.append(K, V, kn, vn, lens)
            ref = oracle.attend(q, K, V, ln)
            torch.cuda.synchronize()
            table, kp = pc.table(), to_host_bits(pc.k)
            for b in range(Bsz):            # the new rows, reached through the block table
                r = int(lens[b])
                assert kp[:, table[b][r // P], r % P].tobytes() == kn[b].tobytes()
            assert pc.lens() == ln.tolist()
    elif mode == "attend":
        c = KVCache(Bsz, Hkv, cap, "f32", lens=lens, k=to_device(K), v=to_device(V))
        out = c.attend(to_device(q), chunk_rows=256)
        ref = oracle.attend(q, K, V, lens)
    else:
        c = KVCache(Bsz, Hkv, cap, "f32", lens=lens, k=to_device(K), v=to_device(V))
        kn = _rows(rng, (Bsz, Hkv, 64), "f32")
        vn = _rows(rng, (Bsz, Hkv, 64), "f32")
        if mode == "replay_fused":          # device-length fused step on a horizon-sized grid
            c.set_replay_mode(256)
            c.set_replay_horizon(1)
        out = c.append_attend(to_device(kn), to_device(vn), to_device(q), chunk_rows=256)
        ln = oracle.append(K, V, kn, vn, lens)
        ref = oracle.attend(q, K, V, ln)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu().numpy(), ref, "f32", f"wide group {group} {mode}")
    if mode in ("fused", "replay_fused"):
        assert to_host_bits(c.k).tobytes() == K.tobytes()
        assert c.lens_dev.cpu().tolist() == ln.tolist()


@pytest.mark.parametrize("dtype,Hq,Bsz", [("bf16", 2, 60_000), ("bf16", 2, 70_000),
                                         ("f32", 1, 70_000)])
def test_chunk_count_around_the_grid_y_limit(dtype, Hq, Bsz):
    rng = np.random.default_rng(85)
    Hkv = 1
    lens = rng.integers(1, 3, size=Bsz).astype(np.int32)       # ragged: 1 or 2 rows
    cap = gen.padded_rows(2)
    shape = (Bsz, Hkv, cap, 64)
    K = np.zeros(shape, np.float32 if dtype == "f32" else np.uint16)
    V = np.zeros_like(K)
    K[:, :, :2] = _rows(rng, (Bsz, Hkv, 2, 64), dtype)
    V[:, :, :2] = _rows(rng, (Bsz, Hkv, 2, 64), dtype)
    q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
    _log(f"{Bsz} ragged sequences, {dtype}, chunk 64 -> {Bsz} chunks")
    c = KVCache(Bsz, Hkv, cap, dtype, lens=lens, k=to_device(K), v=to_device(V))
    out = c.attend(to_device(q), chunk_rows=64)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu().numpy(), oracle.attend(q, K, V, lens), dtype,
                           f"{dtype} B={Bsz}")
