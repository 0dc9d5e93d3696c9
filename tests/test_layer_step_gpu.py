"""One decoder layer's attention step in one launch (kvdec_append_attend_cross),
through the C ABI.

The call must give bitwise the outputs, cache bytes and lengths of
kvdec_append_attend on the self cache followed by kvdec_attend_cross on the
static encoder cache at the same chunk sizes, and lie within the tolerance
of the f64 oracle for every sequence and head.  Cases: the three Whisper
workload shapes at full size (every step), f32 and bf16, MHA, the MFMA and
the f32 VALU grouped-head kernels, chunk sizes that split either part
(merge launch for one part only, for both, for neither), 16-wave
workgroups in both parts, explicit chunk sizes whose parts need workgroups
of different shapes (the two-call path), replay mode (lengths read and
bumped on the device), and refused calls that enqueue nothing.
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


class Layer:
    """Two copies of one layer's self and cross caches (one for the one-launch
    call, one for the two calls) and the oracle's mirror."""

    def __init__(self, inp):
        wl = inp.wl
        Bsz = len(inp.lens)
        self.inp, self.wl = inp, wl
        mk = lambda: KVCache(Bsz, wl.n_kv_heads, inp.cap, wl.dtype, lens=inp.lens,
                             k=to_device(inp.k_cache), v=to_device(inp.v_cache))
        self.one, self.two = mk(), mk()
        enc = inp.cross_k_tok.shape[1]
        self.cross = KVCache(Bsz, wl.n_kv_heads, enc, wl.dtype, static=True, lens=[0] * Bsz)
        self.cross.seed(to_device(inp.cross_k_tok), to_device(inp.cross_v_tok))
        cap = gen.padded_rows(enc)
        self.cK = np.zeros((Bsz, wl.n_kv_heads, cap, 64), inp.k_cache.dtype)
        self.cV = np.zeros_like(self.cK)
        oracle.seed(self.cK, inp.cross_k_tok)
        oracle.seed(self.cV, inp.cross_v_tok)
        self.clens = np.full(Bsz, enc, np.int32)
        self.Kh, self.Vh, self.lens = inp.k_cache.copy(), inp.v_cache.copy(), inp.lens.copy()

    def step(self, s, cs, cx, check_oracle=True):
        inp, wl = self.inp, self.wl
        kn, vn = to_device(inp.k_new[s]), to_device(inp.v_new[s])
        qs, qx = to_device(inp.q_self[s]), to_device(inp.q_cross[s])
        got_s, got_x = self.one.append_attend_cross(self.cross, kn, vn, qs, qx, chunk_self=cs,
                                                    chunk_cross=cx)
        ref_s = self.two.append_attend(kn, vn, qs, chunk_rows=cs)
        ref_x = self.cross.attend(qx, chunk_rows=cx)
        torch.cuda.synchronize()
        assert got_s.cpu().numpy().tobytes() == ref_s.cpu().numpy().tobytes(), f"self step {s}"
        assert got_x.cpu().numpy().tobytes() == ref_x.cpu().numpy().tobytes(), f"cross step {s}"
        self.lens = oracle.append(self.Kh, self.Vh, inp.k_new[s], inp.v_new[s], self.lens)
        worst = 0.0
        if check_oracle:
            ref = oracle.attend(inp.q_self[s], self.Kh, self.Vh, self.lens)
            worst = assert_attention_close(got_s.cpu().numpy(), ref, wl.dtype, f"self step {s}")
            refx = oracle.attend(inp.q_cross[s], self.cK, self.cV, self.clens)
            worst = max(worst, assert_attention_close(got_x.cpu().numpy(), refx, wl.dtype,
                                                      f"cross step {s}"))
        return worst

    def check_state(self):
        assert to_host_bits(self.one.k).tobytes() == self.Kh.tobytes()
        assert to_host_bits(self.one.v).tobytes() == self.Vh.tobytes()
        assert self.one.lens() == self.lens.tolist()
        assert self.one.lens_dev.cpu().tolist() == self.lens.tolist()


# chunk sizes given explicitly, so that the two calls use the same ones:
# (self, cross) -- one chunk each; cross split; self split; both split; both
# at 256+ rows (16-wave workgroups for f32 MHA); shapes that differ (two calls)
CHUNKS = [(512, 2048), (512, 256), (64, 2048), (64, 128), (256, 512), (64, 256)]


@pytest.mark.parametrize("dtype,Hq,Hkv", [("f32", 8, 8), ("bf16", 8, 8), ("bf16", 16, 4),
                                           ("f32", 12, 3)])
@pytest.mark.parametrize("cs,cx", CHUNKS)
def test_layer_step_equals_the_two_calls(dtype, Hq, Hkv, cs, cx):
    wl = gen.Workload("layer", 6, Hq, Hkv, dtype, "const:1", 2, True, seed=201)
    lens = np.array([0, 63, 64, 200, 447, 300], np.int32)
    inp = gen.make_inputs(wl, batch=6, lens=lens, steps=2, enc_len=1500, seed=202)
    _log(f"layer {dtype} {Hq}/{Hkv} chunks {cs}/{cx}")
    L = Layer(inp)
    for s in range(2):
        L.step(s, cs, cx)
    L.check_state()


@pytest.mark.parametrize("name", ["whisper-tiny", "whisper-base", "whisper-large"])
def test_layer_step_full_size(name):
    """The Whisper workloads at full size with the automatic chunk sizes,
    every step: every sequence and head against the oracle, and the cache
    bytes and lengths against the oracle's appends."""
    wl = gen.WORKLOADS[name]
    inp = gen.make_inputs(wl)
    _log(f"layer full {name}")
    L = Layer(inp)
    worst = 0.0
    for s in range(wl.steps):
        kn, vn = to_device(inp.k_new[s]), to_device(inp.v_new[s])
        qs, qx = to_device(inp.q_self[s]), to_device(inp.q_cross[s])
        got_s, got_x = L.one.append_attend_cross(L.cross, kn, vn, qs, qx)
        torch.cuda.synchronize()
        L.lens = oracle.append(L.Kh, L.Vh, inp.k_new[s], inp.v_new[s], L.lens)
        ref = oracle.attend(inp.q_self[s], L.Kh, L.Vh, L.lens)
        worst = max(worst, assert_attention_close(got_s.cpu().numpy(), ref, wl.dtype,
                                                  f"{name} self step {s}"))
        refx = oracle.attend(inp.q_cross[s], L.cK, L.cV, L.clens)
        worst = max(worst, assert_attention_close(got_x.cpu().numpy(), refx, wl.dtype,
                                                  f"{name} cross step {s}"))
    L.check_state()
    _log(f"layer full {name}: worst row-relative error {worst:.3e}")


@pytest.mark.parametrize("name,cs,cx", [("whisper-base", 64, 192), ("whisper-large", 512, 2048),
                                        ("whisper-tiny", 64, 64)])
def test_layer_step_full_size_bitwise(name, cs, cx):
    """At full size, bitwise against the two calls at the chunk sizes the
    automatic choice of the one-launch call makes for these workloads on an
    MI355X (whisper-base: 64 self rows, and 192 cross rows instead of the
    cross call's own 256, which would need 16-wave workgroups;
    whisper-large: one chunk per sequence in both parts; whisper-tiny: 64
    rows in both)."""
    wl = gen.WORKLOADS[name]
    inp = gen.make_inputs(wl, steps=min(wl.steps, 4))
    _log(f"layer full bitwise {name} {cs}/{cx}")
    L = Layer(inp)
    for s in range(min(wl.steps, 4)):
        L.step(s, cs, cx, check_oracle=False)
    L.check_state()


def test_layer_step_replay_mode():
    """The self cache in replay mode: the attend launch reads the lengths from
    the device and the merge launch bumps them, for both parts in one grid."""
    wl = gen.Workload("layer-replay", 5, 6, 6, "f32", "const:1", 3, True, seed=211)
    lens = np.array([5, 70, 0, 130, 199], np.int32)
    inp = gen.make_inputs(wl, batch=5, lens=lens, steps=3, enc_len=300, seed=212)
    L = Layer(inp)
    L.one.set_replay_mode(64)
    L.two.set_replay_mode(64)
    for s in range(3):
        L.step(s, 0, 64)
    assert L.one.lens_dev.cpu().tolist() == L.lens.tolist()


def test_layer_step_errors_enqueue_nothing():
    Bsz, H = 2, 4
    self_c = KVCache(Bsz, H, 8, "f32", lens=[3, 8])            # sequence 1 is full
    cross = KVCache(Bsz, H, 16, "f32", static=True, lens=[16, 16])
    kn = torch.zeros(Bsz, H, 64, device="cuda")
    q = torch.zeros(Bsz, H, 64, device="cuda")
    with pytest.raises(B.KvdecError) as e:
        self_c.append_attend_cross(cross, kn, kn, q, q)
    assert e.value.code == B.KVDEC_E_OVERFLOW
    ok = KVCache(Bsz, H, 8, "f32", lens=[3, 4])
    with pytest.raises(B.KvdecError) as e:
        ok.append_attend_cross(ok, kn, kn, q, q)                 # cross part not static
    assert e.value.code == B.KVDEC_E_STATIC
    other = KVCache(Bsz, H, 16, "bf16", static=True, lens=[16, 16])
    with pytest.raises(B.KvdecError) as e:
        ok.append_attend_cross(other, kn, kn, q, q)              # dtype differs
    assert e.value.code == B.KVDEC_E_SHAPE
    with pytest.raises(B.KvdecError) as e:
        ok.append_attend_cross(cross, kn, kn, q, q, chunk_cross=100)
    assert e.value.code == B.KVDEC_E_INVALID
    import ctypes
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    with pytest.raises(B.KvdecError) as e:
        B.kvdec_append_attend_cross(ok.handle, cross.handle, None, p(kn), p(kn), p(q), p(q), H, 0.125,
                                    0, 0, p(out), p(out), p(small), small.numel())
    assert e.value.code == B.KVDEC_E_WORKSPACE
    # the workspace of the self cache alone is not enough for both parts
    need_self = B.kvdec_workspace_bytes(ok.handle, H)
    ws = torch.empty(need_self, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.KvdecError) as e:
        B.kvdec_append_attend_cross(ok.handle, cross.handle, None, p(kn), p(kn), p(q), p(q), H, 0.125,
                                    0, 0, p(out), p(out), p(ws), ws.numel())
    assert e.value.code == B.KVDEC_E_WORKSPACE
    torch.cuda.synchronize()
    assert self_c.lens() == [3, 8] and ok.lens() == [3, 4]
    assert ok.lens_dev.cpu().tolist() == [3, 4] and torch.all(ok.k == 0)


@pytest.mark.parametrize("mode", ["one-launch", "replay", "large-batch"])
def test_layer_step_at_positions(mode):
    """Positions given (lens): bitwise kvdec_append_attend_at followed by
    kvdec_attend_cross, a rewind included; the lengths end at positions + 1."""
    Bsz = B.KVDEC_MAX_FUSED_BATCH + 2 if mode == "large-batch" else 5
    wl = gen.Workload("layer-at", Bsz, 8, 8, "bf16", "uniform:10:300", 3, True, seed=221)
    inp = gen.make_inputs(wl, batch=Bsz, steps=3, enc_len=200, seed=222)
    L = Layer(inp)
    if mode == "replay":
        L.one.set_replay_mode(64)
        L.two.set_replay_mode(64)
    rng = np.random.default_rng(223)
    pos = inp.lens.copy()
    for s in range(3):
        if s == 2:
            pos = np.maximum(pos - rng.integers(0, 10, size=Bsz).astype(np.int32), 0)
        kn, vn = to_device(inp.k_new[s]), to_device(inp.v_new[s])
        qs, qx = to_device(inp.q_self[s]), to_device(inp.q_cross[s])
        got_s, got_x = L.one.append_attend_cross(L.cross, kn, vn, qs, qx, lens=pos)
        ref_s = L.two.append_attend_at(pos, kn, vn, qs)
        ref_x = L.cross.attend(qx)
        torch.cuda.synchronize()
        assert got_s.cpu().numpy().tobytes() == ref_s.cpu().numpy().tobytes(), f"{mode} step {s}"
        assert got_x.cpu().numpy().tobytes() == ref_x.cpu().numpy().tobytes(), f"{mode} step {s}"
        pos = oracle.append(L.Kh, L.Vh, inp.k_new[s], inp.v_new[s], pos)
        bs = np.arange(0, Bsz, max(1, Bsz // 8))
        ref = oracle.attend(inp.q_self[s][bs], L.Kh[bs], L.Vh[bs], pos[bs])
        assert_attention_close(got_s.cpu().numpy()[bs], ref, "bf16", f"{mode} step {s}")
    assert L.one.lens() == pos.tolist() and L.one.lens_dev.cpu().tolist() == pos.tolist()
    assert to_host_bits(L.one.k).tobytes() == to_host_bits(L.two.k).tobytes()
