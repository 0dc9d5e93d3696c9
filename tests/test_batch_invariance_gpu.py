"""Batched == solo, bit for bit, on every attend kernel family, through the C ABI.

For a given chunk size a sequence's output must not depend on the other
sequences of the batch: the batched decode step of franken_ocr 0.8.0
decoder_qwen2.rs must give each stream exactly its solo result.  Each case
runs a workload-shaped batch once, then every sequence alone (batch 1) at the
same chunk size, and compares the output bytes.  The batched grids are large
(several residency rounds of workgroups) and the solo grids tiny, so a kernel
choice that depended on the grid would show here.  Families: f32 VALU with 1
and 2 query heads per KV head (16-wave workgroups at chunks of 256 rows and
more), f32 VALU with 4, bf16 VALU (MHA), bf16 MFMA (grouped heads), the cross
attention over a static cache, the fused append + attend (also against the
unfused calls on the same large grid), and the paged fused step.
"""
import sys

import numpy as np
import pytest
import torch

from kv_cached_decode_kvdec_amd import inputs as gen
from kv_cached_decode_kvdec_amd.cache import KVCache, PagedKVCache, to_device, to_host_bits

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _attend(K, V, lens, q, dtype, chunk, static=False):
    Bsz, Hkv, cap = K.shape[0], K.shape[1], K.shape[2]
    c = KVCache(Bsz, Hkv, cap, dtype, static=static, lens=lens, k=to_device(K), v=to_device(V))
    out = c.attend(to_device(q), chunk_rows=chunk)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    c.close()
    return res


def _same_solo(name, K, V, lens, q, dtype, chunk, static=False):
    batched = _attend(K, V, lens, q, dtype, chunk, static)
    for b in range(len(lens)):
        solo = _attend(K[b:b + 1], V[b:b + 1], lens[b:b + 1], q[b:b + 1], dtype, chunk, static)
        assert solo.tobytes() == batched[b:b + 1].tobytes(), \
            f"{name} chunk {chunk}: sequence {b} (length {lens[b]}) differs solo vs batched"
    return batched


def _shape(name, Hq=None, Hkv=None, batch=None):
    wl = gen.WORKLOADS[name]
    return gen.Workload(name + "-bs", wl.batch if batch is None else batch,
                        wl.n_q_heads if Hq is None else Hq, wl.n_kv_heads if Hkv is None else Hkv,
                        wl.dtype, wl.lens, 1, False, seed=wl.seed + 500)


@pytest.mark.parametrize("Hq,Hkv,chunk", [(16, 16, 256), (16, 16, 512), (16, 16, 128),
                                          (16, 8, 256), (16, 4, 256)])
def test_f32_valu_batched_equals_solo(Hq, Hkv, chunk):
    """The Qwen2-0.5B shape (32 sequences, lengths U{1..4096}, f32): group 1
    and 2 run on 16-wave workgroups at 256+ row chunks, group 4 on 4-wave."""
    wl = _shape("qwen2-0.5b", Hq, Hkv)
    inp = gen.make_inputs(wl, steps=1, canary=False)
    _log(f"f32 valu {Hq}/{Hkv} chunk {chunk}: {len(inp.lens)} sequences")
    _same_solo("f32", inp.k_cache, inp.v_cache, inp.lens, inp.q_self[0], "f32", chunk)


@pytest.mark.parametrize("chunk", [512, 64])
def test_bf16_valu_batched_equals_solo(chunk):
    """The Whisper-large self-attention shape (64 sequences x 20 heads, bf16,
    449 rows): one chunk per sequence at 512 rows, eight and a merge at 64."""
    wl = _shape("whisper-large")
    inp = gen.make_inputs(wl, steps=1, canary=False, lens=np.full(64, 449, np.int32))
    _log(f"bf16 valu chunk {chunk}")
    _same_solo("bf16", inp.k_cache, inp.v_cache, inp.lens, inp.q_self[0], "bf16", chunk)


@pytest.mark.parametrize("chunk", [512, 128])
def test_mfma_gqa_batched_equals_solo(chunk):
    """The GQA shape (64 sequences, 16 q heads over 4 KV heads, bf16,
    log-uniform lengths up to 8192) on the MFMA kernel."""
    wl = _shape("gqa")
    inp = gen.make_inputs(wl, steps=1, canary=False)
    _log(f"mfma gqa chunk {chunk}")
    _same_solo("gqa", inp.k_cache, inp.v_cache, inp.lens, inp.q_self[0], "bf16", chunk)


@pytest.mark.parametrize("dtype,chunk", [("bf16", 2048), ("bf16", 256), ("f32", 256)])
def test_cross_batched_equals_solo(dtype, chunk):
    """Cross-attention over a static 1500-row cache (Whisper-large and
    Whisper-base shapes)."""
    Bsz, H = (64, 20) if dtype == "bf16" else (16, 8)
    rng = np.random.default_rng(909)
    cap = gen.padded_rows(gen.ENC_LEN)
    draw = lambda: rng.standard_normal((Bsz, H, cap, 64), dtype=np.float32)
    K, V = draw(), draw()
    if dtype == "bf16":
        K, V = gen.f32_to_bf16_bits(K), gen.f32_to_bf16_bits(V)
    q = rng.standard_normal((Bsz, H, 64), dtype=np.float32)
    lens = np.full(Bsz, gen.ENC_LEN, np.int32)
    _log(f"cross {dtype} chunk {chunk}")
    _same_solo("cross", K, V, lens, q, dtype, chunk, static=True)


@pytest.mark.parametrize("name,chunk", [("qwen2-0.5b", 256), ("gqa", 512), ("whisper-large", 512)])
def test_fused_batched_equals_solo_and_unfused(name, chunk):
    """kvdec_append_attend on the full batch == kvdec_append + kvdec_attend_self
    on the same batch == kvdec_append_attend on each sequence alone, bitwise,
    for two steps (cache bytes and lengths too)."""
    wl = gen.WORKLOADS[name]
    inp = gen.make_inputs(wl, steps=2, canary=True)
    Bsz, Hkv, cap = len(inp.lens), wl.n_kv_heads, inp.cap
    _log(f"fused {name} chunk {chunk}")
    mk = lambda sl: KVCache(len(inp.lens[sl]), Hkv, cap, wl.dtype, lens=inp.lens[sl],
                            k=to_device(inp.k_cache[sl]), v=to_device(inp.v_cache[sl]))
    fused, two = mk(slice(None)), mk(slice(None))
    outs = []
    for s in range(2):
        kn, vn, q = to_device(inp.k_new[s]), to_device(inp.v_new[s]), to_device(inp.q_self[s])
        got = fused.append_attend(kn, vn, q, chunk_rows=chunk)
        two.append(kn, vn)
        ref = two.attend(q, chunk_rows=chunk)
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref.cpu().numpy().tobytes(), f"{name} step {s}"
        outs.append(got.cpu().numpy())
    assert to_host_bits(fused.k).tobytes() == to_host_bits(two.k).tobytes()
    assert to_host_bits(fused.v).tobytes() == to_host_bits(two.v).tobytes()
    assert fused.lens_dev.cpu().tolist() == (inp.lens + 2).tolist()
    fused.close()
    two.close()
    for b in range(Bsz):
        solo = mk(slice(b, b + 1))
        for s in range(2):
            got = solo.append_attend(to_device(inp.k_new[s][b:b + 1]),
                                     to_device(inp.v_new[s][b:b + 1]),
                                     to_device(inp.q_self[s][b:b + 1]), chunk_rows=chunk)
            torch.cuda.synchronize()
            assert got.cpu().numpy().tobytes() == outs[s][b:b + 1].tobytes(), \
                f"{name}: sequence {b} step {s} differs solo vs batched"
        solo.close()


@pytest.mark.parametrize("name,chunk,P", [("qwen2-0.5b", 256, 16), ("gqa", 512, 64)])
def test_paged_fused_batched_equals_solo(name, chunk, P):
    """kvdec_paged_append_attend on the full batch against each sequence alone
    in a pool of its own, bitwise."""
    wl = gen.WORKLOADS[name]
    inp = gen.make_inputs(wl, steps=1, canary=False)
    Bsz, Hkv = len(inp.lens), wl.n_kv_heads
    maxp = -(-inp.cap // P)
    _log(f"paged fused {name} chunk {chunk} page {P}")

    def run(sl):
        lens = inp.lens[sl]
        pages = int(sum(-(-(int(n) + 1) // P) for n in lens)) + len(lens)
        pc = PagedKVCache(len(lens), Hkv, P, num_pages=pages, max_pages_per_seq=maxp,
                          dtype=wl.dtype)
        pc.load_contiguous(to_device(inp.k_cache[sl]), to_device(inp.v_cache[sl]), lens)
        out = pc.append_attend(to_device(inp.k_new[0][sl]), to_device(inp.v_new[0][sl]),
                               to_device(inp.q_self[0][sl]), chunk_rows=chunk)
        torch.cuda.synchronize()
        res = out.cpu().numpy()
        pc.close()
        return res

    batched = run(slice(None))
    for b in range(Bsz):
        solo = run(slice(b, b + 1))
        assert solo.tobytes() == batched[b:b + 1].tobytes(), \
            f"paged {name}: sequence {b} differs solo vs batched"
