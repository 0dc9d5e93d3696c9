"""RoPE fused into append, against the oracle's f64 rotation.

The oracle rotates the un-rotated key and query in double at the token's
position (its length before the append), rounds to float (then to bf16 for
bf16 caches), appends and attends.  The device does the same in one launch;
both compute the rotation in double, so the stored rows agree to the last
bit except where the two sin/cos implementations straddle a rounding
boundary (at most one unit in the last place).
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cached_decode_kvdec_amd import binding as B
from kv_cached_decode_kvdec_amd import inputs as gen
from kv_cached_decode_kvdec_amd.cache import KVCache, to_device, to_host_bits

from helpers import assert_attention_close

pytestmark = pytest.mark.gpu
THETA = 1.0e6


def _round(x64, dtype):
    x32 = x64.astype(np.float32)
    return x32 if dtype == "f32" else gen.f32_to_bf16_bits(x32)


def _ulp_diff(a, b, dtype):
    if dtype == "f32":
        ia, ib = a.view(np.int32).astype(np.int64), b.view(np.int32).astype(np.int64)
    else:
        ia, ib = a.astype(np.int64), b.astype(np.int64)
    return np.abs(ia - ib)


@pytest.mark.parametrize("dtype,Hq,Hkv,window", [("f32", 16, 16, 0), ("bf16", 16, 4, 0),
                                                  ("f32", 8, 2, 0), ("bf16", 6, 6, 96)])
def test_append_rope_matches_oracle(dtype, Hq, Hkv, window):
    rng = np.random.default_rng(99 + Hq)
    Bsz, steps = 4, 5
    lens0 = np.array([0, 7, 3000, 8190], np.int32) if window == 0 else np.array([0, 5, 95, 400])
    cap = int(lens0.max()) + steps if window == 0 else window
    cp = gen.padded_rows(cap)
    Kc = np.zeros((Bsz, Hkv, cp, 64), np.float32 if dtype == "f32" else np.uint16)
    Vc = np.zeros_like(Kc)
    # prefill rows: positions 0 .. len-1, already rotated (as a prefill would leave them)
    for b in range(Bsz):
        n = int(min(lens0[b], window) if window else lens0[b])
        first = int(lens0[b]) - n
        if n:
            raw = rng.standard_normal((Hkv, n, 64))
            rot = oracle.rope(raw, np.arange(first, first + n)[None, :], THETA)
            slots = np.arange(first, first + n) % window if window else np.arange(n)
            Kc[b][:, slots] = _round(rot, dtype)
            Vc[b][:, slots] = _round(rng.standard_normal((Hkv, n, 64)), dtype)
    c = KVCache(Bsz, Hkv, cap, dtype, lens=lens0, k=to_device(Kc), v=to_device(Vc), window=window)
    lens = lens0.copy()
    worst_ulp, mismatched, total = 0, 0, 0
    for s in range(steps):
        kraw = rng.standard_normal((Bsz, Hkv, 64)).astype(np.float32)
        kin = kraw if dtype == "f32" else gen.f32_to_bf16_bits(kraw)
        vin = _round(rng.standard_normal((Bsz, Hkv, 64)), dtype)
        q = rng.standard_normal((Bsz, Hq, 64)).astype(np.float32)
        qd = to_device(q)
        q_rot = c.append_rope(to_device(kin), to_device(vin), THETA, q=qd)
        out = c.attend(q_rot)
        torch.cuda.synchronize()
        # oracle: rotate (f64) at position len, round, append, attend
        kin64 = kin.astype(np.float64) if dtype == "f32" else oracle.bf16_to_f32(kin).astype(np.float64)
        k_rot = _round(oracle.rope(kin64, lens[:, None], THETA), dtype)
        q_ref = oracle.rope(q.astype(np.float64), lens[:, None], THETA).astype(np.float32)
        for b in range(Bsz):
            slot = lens[b] % window if window else lens[b]
            Kc[b, :, slot] = k_rot[b]
            Vc[b, :, slot] = vin[b]
        lens = lens + 1
        n = np.minimum(lens, window) if window else lens
        got_q = q_rot.cpu().numpy()
        qd_ulp = _ulp_diff(got_q, q_ref, "f32")
        assert qd_ulp.max() <= 1, f"q rotation off by {qd_ulp.max()} ulp"
        got_k = to_host_bits(c.k)
        d = _ulp_diff(got_k, Kc, dtype)
        worst_ulp = max(worst_ulp, int(d.max()))
        mismatched += int(np.count_nonzero(d))
        total += d.size
        assert d.max() <= 1, f"stored key off by {d.max()} ulp"
        assert to_host_bits(c.v).tobytes() == Vc.tobytes()
        # attention on the rotated data, against the oracle's rotated cache;
        # the (linear) oracle reads rows in slot order: attention is order-free
        ref = oracle.attend(q_ref, Kc, Vc, n)
        assert_attention_close(out.cpu().numpy(), ref, dtype, f"rope step {s}")
    assert mismatched <= max(4, total // 100000), f"{mismatched} of {total} key elements differ"
    assert c.lens() == lens.tolist()


def test_append_rope_argument_errors():
    c = KVCache(1, 2, 8, "f32", lens=[0])
    k = torch.zeros(1, 2, 64, device="cuda")
    q = torch.zeros(1, 4, 64, device="cuda")
    with pytest.raises(B.KvdecError) as e:
        c.append_rope(k, k, 0.0)
    assert e.value.code == B.KVDEC_E_INVALID
    with pytest.raises(B.KvdecError) as e:
        c.append_rope(k, k, 1e4, q=torch.zeros(1, 3, 64, device="cuda"))
    assert e.value.code == B.KVDEC_E_SHAPE
    import ctypes
    with pytest.raises(B.KvdecError) as e:
        B.kvdec_append_rope(c.handle, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                            1e4, ctypes.c_void_p(q.data_ptr()), None, 4)
    assert e.value.code == B.KVDEC_E_INVALID
    assert c.lens() == [0]
    # q rotated in place (q and q_rot the same buffer) at position 0 is unchanged
    q.normal_()
    before = q.clone()
    c.append_rope(k, k, 1e4, q=q, q_rot=q)
    torch.cuda.synchronize()
    assert torch.equal(q, before) and c.lens() == [1]
