"""GPU parity of the decode step against the f64 oracle, through the C ABI.

Append must be bit-exact (whole cache bytes, NaN canaries in padding rows
included); attention must be within the row-relative tolerance of
tests/helpers.py (1e-4 for f32 K/V, 2e-2 for bf16 K/V).
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


class Run:
    """Device caches + host mirrors for one set of generated inputs."""

    def __init__(self, inp, chunk_rows=0):
        wl = inp.wl
        self.inp, self.wl, self.chunk_rows = inp, wl, chunk_rows
        Bsz = len(inp.lens)
        self.self_cache = KVCache(Bsz, wl.n_kv_heads, inp.cap, wl.dtype, lens=inp.lens,
                                  k=to_device(inp.k_cache), v=to_device(inp.v_cache))
        self.Kh, self.Vh = inp.k_cache.copy(), inp.v_cache.copy()
        self.lens = inp.lens.copy()
        self.cross = None
        if wl.cross:
            enc = inp.cross_k_tok.shape[1]
            self.cross = KVCache(Bsz, wl.n_kv_heads, enc, wl.dtype, static=True, lens=[0] * Bsz)
            self.cross.seed(to_device(inp.cross_k_tok), to_device(inp.cross_v_tok))
            cap = gen.padded_rows(enc)
            self.cKh = np.full((Bsz, wl.n_kv_heads, cap, 64), 0, inp.k_cache.dtype)
            self.cVh = np.full_like(self.cKh, 0)
            oracle.seed(self.cKh, inp.cross_k_tok)
            oracle.seed(self.cVh, inp.cross_v_tok)
            self.clens = np.full(Bsz, enc, np.int32)

    def step(self, s):
        inp = self.inp
        kn, vn = to_device(inp.k_new[s]), to_device(inp.v_new[s])
        self.self_cache.append(kn, vn)
        self.lens = oracle.append(self.Kh, self.Vh, inp.k_new[s], inp.v_new[s], self.lens)
        q = to_device(inp.q_self[s])
        out = self.self_cache.attend(q, chunk_rows=self.chunk_rows)
        cout = None
        if self.cross is not None:
            cout = self.cross.attend(to_device(inp.q_cross[s]), chunk_rows=self.chunk_rows)
        return out, cout


def _check_step(run, s, out, cout):
    """Every sequence and head of the step against the oracle."""
    inp, dt = run.inp, run.wl.dtype
    ref = oracle.attend(inp.q_self[s], run.Kh, run.Vh, run.lens)
    e1 = assert_attention_close(out.cpu().numpy(), ref, dt, f"{run.wl.name} self step {s}")
    e2 = 0.0
    if cout is not None:
        refc = oracle.attend(inp.q_cross[s], run.cKh, run.cVh, run.clens)
        e2 = assert_attention_close(cout.cpu().numpy(), refc, dt, f"{run.wl.name} cross step {s}")
    return max(e1, e2)


# --- small cases: several tiles, ragged tails, every group size -----------------

SMALL_LENS = [1, 63, 64, 65, 200, 513, 0, 1023]


@pytest.mark.parametrize("name", gen.ORDER)
@pytest.mark.parametrize("chunk_rows", [0, 64, 256])
def test_small_parity_every_workload(name, chunk_rows):
    wl = gen.WORKLOADS[name]
    lens = np.array(SMALL_LENS, np.int32)
    inp = gen.make_inputs(wl, batch=len(lens), lens=lens, steps=2, enc_len=300, seed=7)
    _log(f"small {name} chunk={chunk_rows}")
    run = Run(inp, chunk_rows)
    for s in range(2):
        out, cout = run.step(s)
        torch.cuda.synchronize()
        _check_step(run, s, out, cout)
    assert run.self_cache.lens() == run.lens.tolist()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (6, 2), (12, 4), (16, 4), (10, 2), (12, 2), (8, 1),
                                    (14, 2), (7, 7)])
def test_gqa_groups(dtype, Hq, Hkv):
    wl = gen.Workload("g", 5, Hq, Hkv, dtype, "const:1", 1, False, seed=31)
    lens = np.array([0, 1, 130, 700, 2000], np.int32)
    inp = gen.make_inputs(wl, batch=5, lens=lens, steps=1)
    _log(f"gqa {dtype} {Hq}/{Hkv}")
    run = Run(inp, 128)
    out, _ = run.step(0)
    torch.cuda.synchronize()
    _check_step(run, 0, out, None)


def test_append_bit_exact_with_canaries():
    for name in gen.ORDER:
        wl = gen.WORKLOADS[name]
        lens = np.array([0, 5, 64, 127], np.int32)
        inp = gen.make_inputs(wl, batch=4, lens=lens, steps=3, enc_len=64, seed=3)
        _log(f"append {name}")
        run = Run(inp)
        for s in range(3):
            run.self_cache.append(to_device(inp.k_new[s]), to_device(inp.v_new[s]))
            run.lens = oracle.append(run.Kh, run.Vh, inp.k_new[s], inp.v_new[s], run.lens)
        torch.cuda.synchronize()
        assert to_host_bits(run.self_cache.k).tobytes() == run.Kh.tobytes()
        assert to_host_bits(run.self_cache.v).tobytes() == run.Vh.tobytes()
        assert run.self_cache.lens_dev.cpu().numpy().tolist() == run.lens.tolist()
        assert run.self_cache.lens() == run.lens.tolist()


def test_seed_matches_head_first_permute():
    for dtype in ("f32", "bf16"):
        wl = gen.Workload("s", 3, 5, 5, dtype, "const:1", 1, True, seed=5)
        inp = gen.make_inputs(wl, batch=3, lens=np.ones(3, np.int32), steps=1, enc_len=77)
        c = KVCache(3, 5, 100, dtype, static=True, lens=[0, 0, 0])
        c.k.fill_(float("nan"))
        c.seed(to_device(inp.cross_k_tok), to_device(inp.cross_v_tok))
        torch.cuda.synchronize()
        exp = to_host_bits(torch.full_like(c.k, float("nan")))
        oracle.seed(exp, inp.cross_k_tok)
        assert to_host_bits(c.k).tobytes() == exp.tobytes()
        assert c.lens() == [77, 77, 77]
        assert c.lens_dev.cpu().tolist() == [77, 77, 77]


def test_split_count_invariance_and_batched_equals_solo():
    wl = gen.WORKLOADS["qwen2-0.5b"]
    lens = np.array([3000, 17, 640, 1], np.int32)
    inp = gen.make_inputs(wl, batch=4, lens=lens, steps=1, seed=11)
    outs = {}
    for T in (64, 128, 256, 1024, 4096):
        run = Run(inp, T)
        out, _ = run.step(0)
        torch.cuda.synchronize()
        outs[T] = out.cpu().numpy()
        _check_step(run, 0, out, None)
    for T in outs:
        assert_attention_close(outs[T], outs[4096].astype(np.float64), "f32", f"T={T} vs 4096")
    # batched == solo, bit for bit, at a fixed chunk size
    run = Run(inp, 128)
    batched = run.step(0)[0].cpu().numpy()
    for b in range(4):
        solo_inp = gen.Inputs(wl, inp.lens[b:b + 1].copy(), inp.cap, inp.k_cache[b:b + 1].copy(),
                              inp.v_cache[b:b + 1].copy(), [inp.k_new[0][b:b + 1]],
                              [inp.v_new[0][b:b + 1]], [inp.q_self[0][b:b + 1]], [])
        solo = Run(solo_inp, 128).step(0)[0].cpu().numpy()
        assert solo.tobytes() == batched[b:b + 1].tobytes(), f"sequence {b} differs solo vs batched"


def test_fail_closed_and_empty_rows():
    wl = gen.Workload("e", 3, 4, 2, "f32", "const:1", 1, False, seed=13)
    inp = gen.make_inputs(wl, batch=3, lens=np.array([0, 40, 300], np.int32), steps=1)
    inp.q_self[0][1, 0, 3] = np.nan
    inp.q_self[0][2, 3, :] = np.nan
    run = Run(inp, 64)
    out, _ = run.step(0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[1, 0] == 0.0) and np.all(got[2, 3] == 0.0)
    _check_step(run, 0, out, None)
    # a sequence that never had a row: attend without append gives zeros
    c = KVCache(2, 2, 64, "f32", lens=[0, 0])
    q = torch.randn(2, 4, 64, device="cuda")
    o = c.attend(q)
    torch.cuda.synchronize()
    assert torch.all(o == 0)


def test_single_row_returns_value_row():
    wl = gen.Workload("one", 4, 8, 8, "bf16", "const:1", 1, False, seed=17)
    inp = gen.make_inputs(wl, batch=4, lens=np.zeros(4, np.int32), steps=1)
    run = Run(inp, 0)
    out, _ = run.step(0)
    torch.cuda.synchronize()
    v = oracle.bf16_to_f32(inp.v_new[0])           # [B][H][64]
    assert np.array_equal(out.cpu().numpy(), v)


def test_errors_leave_state_unchanged():
    c = KVCache(2, 2, 3, "f32", lens=[2, 3])
    kn = torch.zeros(2, 2, 64, device="cuda")
    before = c.k.clone()
    with pytest.raises(B.KvdecError) as e:
        c.append(kn, kn)
    assert e.value.code == B.KVDEC_E_OVERFLOW
    torch.cuda.synchronize()
    assert torch.equal(c.k, before) and c.lens() == [2, 3]
    assert c.lens_dev.cpu().tolist() == [2, 3]
    q = torch.zeros(2, 3, 64, device="cuda")
    with pytest.raises(B.KvdecError) as e:
        c.attend(q)                                   # 3 heads over 2 KV heads
    assert e.value.code == B.KVDEC_E_SHAPE
    q = torch.zeros(2, 4, 64, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    import ctypes
    with pytest.raises(B.KvdecError) as e:
        B.kvdec_attend_self(c.handle, ctypes.c_void_p(q.data_ptr()), 4, 0.125, 0,
                            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), 16)
    assert e.value.code == B.KVDEC_E_WORKSPACE
    with pytest.raises(B.KvdecError) as e:
        c.attend(q, chunk_rows=100)
    assert e.value.code == B.KVDEC_E_INVALID
    with pytest.raises(B.KvdecError) as e:
        B.kvdec_attend_cross(c.handle, ctypes.c_void_p(q.data_ptr()), 4, 0.125, 0,
                             ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), 16)
    assert e.value.code == B.KVDEC_E_STATIC
    s = KVCache(2, 2, 10, "f32", static=True, lens=[10, 10])
    with pytest.raises(B.KvdecError) as e:
        s.append(kn, kn)
    assert e.value.code == B.KVDEC_E_STATIC
    # append up to exactly the capacity works; one more is rejected
    c2 = KVCache(1, 1, 2, "f32", lens=[0])
    k1 = torch.ones(1, 1, 64, device="cuda")
    c2.append(k1, k1)
    c2.append(k1, k1)
    with pytest.raises(B.KvdecError):
        c2.append(k1, k1)
    assert c2.lens() == [2]


# --- full-size workloads: every step, every sequence and head -----------------

@pytest.mark.parametrize("name", gen.ORDER)
def test_full_size_parity(name):
    wl = gen.WORKLOADS[name]
    _log(f"full {name}: generating inputs")
    inp = gen.make_inputs(wl)
    run = Run(inp)
    worst = 0.0
    for s in range(wl.steps):
        out, cout = run.step(s)
        torch.cuda.synchronize()
        worst = max(worst, _check_step(run, s, out, cout))
    # the whole cache after every append, bit for bit
    assert to_host_bits(run.self_cache.k).tobytes() == run.Kh.tobytes()
    assert to_host_bits(run.self_cache.v).tobytes() == run.Vh.tobytes()
    _log(f"full {name}: worst row-relative error {worst:.3e}")


def test_workspace_reuse_is_stable_and_shareable():
    wl = gen.WORKLOADS["gqa"]
    lens = np.array([5000, 64, 0, 1300, 129], np.int32)
    inp = gen.make_inputs(wl, batch=5, lens=lens, steps=1, seed=23)
    run = Run(inp, 64)
    out, _ = run.step(0)
    first = out.clone()
    ws = run.self_cache.workspace(wl.n_q_heads)
    for _ in range(3):
        again = run.self_cache.attend(to_device(inp.q_self[0]), chunk_rows=64)
        torch.cuda.synchronize()
        assert torch.equal(again, first)
    _check_step(run, 0, first, None)
    # the same workspace serves a different cache of a smaller size
    other = KVCache(2, wl.n_kv_heads, 700, "bf16", lens=[700, 3],
                    k=to_device(inp.k_cache[:2, :, :704]), v=to_device(inp.v_cache[:2, :, :704]))
    q2 = to_device(inp.q_self[0][:2])
    o2 = torch.empty_like(q2)
    import ctypes
    B.kvdec_attend_self(other.handle, ctypes.c_void_p(q2.data_ptr()), wl.n_q_heads, 0.125, 64,
                        ctypes.c_void_p(o2.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel())
    torch.cuda.synchronize()
    ref = oracle.attend(inp.q_self[0][:2], inp.k_cache[:2, :, :704], inp.v_cache[:2, :, :704],
                        np.array([700, 3], np.int32))
    assert_attention_close(o2.cpu().numpy(), ref, "bf16", "shared workspace")
    # garbage in the workspace does not matter: it holds nothing between calls
    ws.fill_(255)
    again = run.self_cache.attend(to_device(inp.q_self[0]), chunk_rows=64)
    torch.cuda.synchronize()
    assert torch.equal(again, first)
