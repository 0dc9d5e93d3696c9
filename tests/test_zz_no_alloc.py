"""kvdec_append_attend_noalloc (the decode step with the library's own device
scratch instead of a workspace) against kvdec_append_attend, through the C ABI.

Two calls in a row on different caches, the second smaller: a 16-sequence
f32 cache whose long sequences span several chunks (the merge reads the
partials from the scratch) in the one-launch mode, then a 3-sequence bf16
grouped-query cache in replay mode (the attend launch snapshots the lengths
into the scratch and the merge launch bumps them).  Each must give bitwise
the output, cache bytes and lengths of kvdec_append_attend with a workspace
on a twin cache, and lie within the tolerance of the f64 oracle.  A call
too large for the scratch is refused before anything is enqueued.
"""
import ctypes
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


def _noalloc(cache, kn, vn, q, chunk_rows=0):
    out = torch.empty_like(q)
    B.kvdec_append_attend_noalloc(cache.handle, ctypes.c_void_p(kn.data_ptr()),
                                  ctypes.c_void_p(vn.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                  q.shape[1], 0.125, chunk_rows, ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return out


def _twin_step(wl, lens, chunk_rows, replay, seed, steps=2):
    inp = gen.make_inputs(wl, batch=len(lens), lens=np.asarray(lens, np.int32), steps=steps,
                          seed=seed)
    mk = lambda: KVCache(len(lens), wl.n_kv_heads, inp.cap, wl.dtype, lens=inp.lens,
                         k=to_device(inp.k_cache), v=to_device(inp.v_cache))
    ref_cache, na_cache = mk(), mk()
    if replay:
        ref_cache.set_replay_mode(chunk_rows)
        na_cache.set_replay_mode(chunk_rows)
    Kh, Vh, hl = inp.k_cache.copy(), inp.v_cache.copy(), inp.lens.copy()
    for s in range(steps):
        kn, vn, q = to_device(inp.k_new[s]), to_device(inp.v_new[s]), to_device(inp.q_self[s])
        ref = ref_cache.append_attend(kn, vn, q, chunk_rows=0 if replay else chunk_rows)
        got = _noalloc(na_cache, kn, vn, q, 0 if replay else chunk_rows)
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == ref.cpu().numpy().tobytes(), f"{wl.name} step {s}"
        hl = oracle.append(Kh, Vh, inp.k_new[s], inp.v_new[s], hl)
        assert_attention_close(got.cpu().numpy(), oracle.attend(inp.q_self[s], Kh, Vh, hl),
                               wl.dtype, f"{wl.name} step {s} vs oracle")
    assert to_host_bits(na_cache.k).tobytes() == Kh.tobytes()
    assert to_host_bits(na_cache.v).tobytes() == Vh.tobytes()
    assert na_cache.lens_dev.cpu().tolist() == hl.tolist()
    if not replay:
        assert na_cache.lens() == hl.tolist()
    ref_cache.close()
    na_cache.close()


def test_noalloc_equals_workspace_call_twice_second_smaller():
    big = gen.Workload("noalloc-big", 16, 16, 16, "f32", "const:1", 2, False, seed=3)
    lens = [3000, 17, 640, 1, 0, 2047, 256, 1999, 5, 4000, 300, 64, 63, 65, 1024, 2500]
    _log("noalloc call 1: 16 f32 sequences, 256-row chunks (merge)")
    _twin_step(big, lens, 256, replay=False, seed=101)
    small = gen.Workload("noalloc-small", 3, 8, 2, "bf16", "const:1", 2, False, seed=4)
    _log("noalloc call 2: 3 bf16 GQA sequences, replay mode (device lengths)")
    _twin_step(small, [70, 0, 200], 64, replay=True, seed=102)


def test_noalloc_refuses_a_call_beyond_the_scratch():
    # 64 sequences x 64 query heads over 8 KV heads, 1000 rows at 64-row chunks:
    # 1024 chunks x 64 heads x 264 bytes > 16 MiB
    Bsz, Hkv, Hq = 64, 8, 64
    c = KVCache(Bsz, Hkv, 1100, "bf16", lens=[1000] * Bsz)
    kn = torch.zeros(Bsz, Hkv, 64, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(Bsz, Hq, 64, device="cuda")
    torch.cuda.synchronize()
    with pytest.raises(B.KvdecError) as e:
        _noalloc(c, kn, kn, q, 64)
    assert e.value.code == B.KVDEC_E_WORKSPACE
    torch.cuda.synchronize()
    assert c.lens() == [1000] * Bsz and c.lens_dev.cpu().tolist() == [1000] * Bsz
    assert torch.all(c.k == 0)
    # the same cache at 1024-row chunks needs 64 chunks x 64 heads: it runs
    out = _noalloc(c, kn, kn, q, 1024)
    torch.cuda.synchronize()
    assert c.lens() == [1001] * Bsz
    assert torch.all(out == 0)      # all-zero V rows
    c.close()
