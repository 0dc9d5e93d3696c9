"""Sliding window that keeps an overlap (kvdec_append_slide), through the C ABI.

Against the oracle's append_slide (whisper-apr 0.3.3 decoder_generated.rs
`StreamingKVCache`): the whole cache bit for bit after every append (NaN
canaries in rows never written included), the lengths and the slid flags,
and decode attention over the kept rows within the tolerance.  Sequences
start empty, one row short of the window and full, so they slide at
different steps; f32 MHA and bf16 grouped heads (MFMA); overlaps below,
at and above half the window.  Also captured in a HIP graph in replay
mode, where the slide is decided on the device.
"""
import gc
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


def _rows(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else gen.f32_to_bf16_bits(x)


@pytest.mark.parametrize("dtype,Hq,Hkv,W,overlap", [("f32", 4, 4, 100, 30), ("bf16", 16, 4, 96, 48),
                                                     ("bf16", 8, 2, 70, 60), ("f32", 6, 3, 64, 0)])
def test_slide_matches_oracle(dtype, Hq, Hkv, W, overlap):
    rng = np.random.default_rng(300 + W + overlap)
    Bsz, steps = 3, 2 * W + 10
    print(f"slide {dtype} {Hq}/{Hkv} W={W} overlap={overlap}", file=sys.stderr, flush=True)
    cp = gen.padded_rows(W)
    K = np.full((Bsz, Hkv, cp, 64), np.nan, np.float32)
    V = np.full_like(K, np.nan)
    if dtype == "bf16":
        K, V = gen.f32_to_bf16_bits(K), gen.f32_to_bf16_bits(V)
    start = np.array([0, W - 1, W], np.int32)
    for b in range(Bsz):
        K[b, :, :start[b]] = _rows(rng, (Hkv, start[b], 64), dtype)
        V[b, :, :start[b]] = _rows(rng, (Hkv, start[b], 64), dtype)
    c = KVCache(Bsz, Hkv, W, dtype, lens=start, k=to_device(K), v=to_device(V))
    lens = start.copy()
    for s in range(steps):
        kn, vn = _rows(rng, (Bsz, Hkv, 64), dtype), _rows(rng, (Bsz, Hkv, 64), dtype)
        q = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
        slid = c.append_slide(to_device(kn), to_device(vn), overlap)
        out = c.attend(to_device(q), chunk_rows=64 if s % 2 else 0)
        torch.cuda.synchronize()
        lens, ref_slid = oracle.append_slide(K, V, kn, vn, lens, W, overlap)
        assert slid == ref_slid.tolist(), f"step {s}"
        assert c.lens() == lens.tolist() and c.lens_dev.cpu().tolist() == lens.tolist(), f"step {s}"
        assert to_host_bits(c.k).tobytes() == K.tobytes(), f"step {s}: K cache bytes"
        assert to_host_bits(c.v).tobytes() == V.tobytes(), f"step {s}: V cache bytes"
        assert_attention_close(out.cpu().numpy(), oracle.attend(q, K, V, lens), dtype, f"step {s}")


def test_slide_in_replay_mode_graph():
    """append_slide + attend captured once and replayed past two slides: the
    device decides each slide from its own lengths."""
    rng = np.random.default_rng(317)
    Bsz, Hkv, Hq, W, overlap = 2, 2, 4, 64, 20
    cp = gen.padded_rows(W)
    K = np.full((Bsz, Hkv, cp, 64), np.nan, np.float32)
    V = np.full_like(K, np.nan)
    start = np.array([60, 5], np.int32)
    for b in range(Bsz):
        K[b, :, :start[b]] = _rows(rng, (Hkv, start[b], 64), "f32")
        V[b, :, :start[b]] = _rows(rng, (Hkv, start[b], 64), "f32")
    c = KVCache(Bsz, Hkv, W, "f32", lens=start, k=to_device(K), v=to_device(V))
    c.set_replay_mode(64)
    c.workspace(Hq)
    kn = torch.zeros(Bsz, Hkv, 64, device="cuda")
    vn = torch.zeros(Bsz, Hkv, 64, device="cuda")
    q = torch.zeros(Bsz, Hq, 64, device="cuda")
    out = torch.zeros(Bsz, Hq, 64, device="cuda")
    gc.collect()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.append_slide(kn, vn, overlap)
        c.attend(q, out=out)
    lens = start.copy()
    for t in range(110):
        knh, vnh = _rows(rng, (Bsz, Hkv, 64), "f32"), _rows(rng, (Bsz, Hkv, 64), "f32")
        qh = rng.standard_normal((Bsz, Hq, 64), dtype=np.float32)
        kn.copy_(torch.from_numpy(knh).cuda())
        vn.copy_(torch.from_numpy(vnh).cuda())
        q.copy_(torch.from_numpy(qh).cuda())
        g.replay()
        torch.cuda.synchronize()
        lens, _ = oracle.append_slide(K, V, knh, vnh, lens, W, overlap)
        assert c.lens_dev.cpu().tolist() == lens.tolist(), f"replay {t}"
        assert to_host_bits(c.k).tobytes() == K.tobytes(), f"replay {t}"
        assert_attention_close(out.cpu().numpy(), oracle.attend(qh, K, V, lens), "f32", f"replay {t}")


def test_slide_refusals():
    kn = torch.zeros(2, 2, 64, device="cuda")
    ring = KVCache(2, 2, 8, "f32", lens=[3, 4], window=8)
    with pytest.raises(B.KvdecError) as e:
        ring.append_slide(kn, kn, 2)
    assert e.value.code == B.KVDEC_E_INVALID
    lin = KVCache(2, 2, 8, "f32", lens=[3, 8])
    with pytest.raises(B.KvdecError) as e:
        lin.append_slide(kn, kn, -1)
    assert e.value.code == B.KVDEC_E_INVALID
    st = KVCache(2, 2, 8, "f32", static=True, lens=[8, 8])
    with pytest.raises(B.KvdecError) as e:
        st.append_slide(kn, kn, 2)
    assert e.value.code == B.KVDEC_E_STATIC
    torch.cuda.synchronize()
    assert lin.lens() == [3, 8] and lin.lens_dev.cpu().tolist() == [3, 8]
