"""The C-ABI library loads, exports every symbol include/kvdec.h declares, and
its host-side validation rejects bad arguments before touching the device
(no GPU needed: none of these calls reaches a HIP launch)."""
import ctypes
import os
import re

import pytest

from kv_cached_decode_kvdec_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "kvdec.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvdec_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"libkvdec.so does not export {n}"
    assert sorted(B.EXPORTED) == names


def test_binding_constants_match_header():
    with open(os.path.join(ROOT, "include", "kvdec.h")) as f:
        text = f.read()
    defs = dict(re.findall(r"#define\s+(KVDEC_[A-Z0-9_]+)\s+(-?\d+)", text))
    defs.update(re.findall(r"\b(KVDEC_[A-Z0-9_]+)\s*=\s*(\d+)", text))     # enumerators
    assert int(defs["KVDEC_HEAD_DIM"]) == B.HEAD_DIM
    assert int(defs["KVDEC_MIN_CHUNK"]) == B.MIN_CHUNK
    assert int(defs["KVDEC_MAX_CHUNK"]) == B.MAX_CHUNK
    assert int(defs["KVDEC_MAX_GROUP"]) == B.MAX_GROUP
    assert int(defs["KVDEC_MAX_FUSED_BATCH"]) == B.KVDEC_MAX_FUSED_BATCH
    assert int(defs["KVDEC_MAX_PAGED_FUSED_BATCH"]) == B.KVDEC_MAX_PAGED_FUSED_BATCH
    assert int(defs["KVDEC_NOALLOC_SCRATCH_BYTES"]) == B.KVDEC_NOALLOC_SCRATCH_BYTES
    for name in ("KVDEC_OK", "KVDEC_E_INVALID", "KVDEC_E_SHAPE", "KVDEC_E_OVERFLOW",
                 "KVDEC_E_STATIC", "KVDEC_E_WORKSPACE", "KVDEC_E_HIP", "KVDEC_F32", "KVDEC_BF16"):
        assert int(defs[name]) == getattr(B, name), name


def test_library_is_gfx950_native():
    # the shared object carries a gfx950 code object bundle
    with open(B.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"gfx950" in blob


def test_padded_capacity():
    assert B.kvdec_padded_capacity(0) == 0
    assert B.kvdec_padded_capacity(1) == 64
    assert B.kvdec_padded_capacity(64) == 64
    assert B.kvdec_padded_capacity(65) == 128
    assert B.kvdec_padded_capacity(449) == 512
    assert B.kvdec_padded_capacity(4097) == 4160
    assert B.kvdec_padded_capacity(8200) == 8256


def _desc(**kw):
    d = dict(batch=2, n_kv_heads=2, head_dim=64, capacity=10, dtype=0, is_static=0,
             window=0, reserved0=0, k=4096, v=8192, lens=12288)
    d.update(kw)
    return B.CacheDesc(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=32), B.KVDEC_E_SHAPE),
    (dict(head_dim=128), B.KVDEC_E_SHAPE),
    (dict(batch=0), B.KVDEC_E_INVALID),
    (dict(n_kv_heads=0), B.KVDEC_E_INVALID),
    (dict(capacity=0), B.KVDEC_E_INVALID),
    (dict(dtype=7), B.KVDEC_E_INVALID),
    (dict(is_static=2), B.KVDEC_E_INVALID),
    (dict(k=0), B.KVDEC_E_INVALID),
    (dict(v=8200), B.KVDEC_E_INVALID),       # not 16-byte aligned
    (dict(lens=0), B.KVDEC_E_INVALID),
    (dict(window=5), B.KVDEC_E_SHAPE),          # a ring's window equals its capacity
    (dict(window=10, is_static=1), B.KVDEC_E_INVALID),
    (dict(reserved0=1), B.KVDEC_E_INVALID),
])
def test_create_rejects_bad_descriptions(kw, code):
    with pytest.raises(B.KvdecError) as e:
        B.kvdec_cache_create(_desc(**kw), [0, 0])
    assert e.value.code == code
    assert B.load().kvdec_last_error().decode() != ""


@pytest.mark.parametrize("lens", [[0, 11], [-1, 0]])
def test_create_rejects_lengths_outside_capacity(lens):
    with pytest.raises(B.KvdecError) as e:
        B.kvdec_cache_create(_desc(), lens)
    assert e.value.code == B.KVDEC_E_SHAPE


def test_ring_accepts_lengths_beyond_capacity_but_not_negative():
    with pytest.raises(B.KvdecError) as e:
        B.kvdec_cache_create(_desc(window=10), [-3, 0])
    assert e.value.code == B.KVDEC_E_SHAPE
    # a length beyond the window passes validation; with no GPU the call then
    # fails at the device step (set lengths), not at the check
    try:
        B.kvdec_cache_create(_desc(window=10), [25, 3])
    except B.KvdecError as e2:
        assert e2.code == B.KVDEC_E_HIP


def test_null_handle_calls_fail_cleanly():
    lib = B.load()
    assert lib.kvdec_append(None, ctypes.c_void_p(16), ctypes.c_void_p(32), None) == B.KVDEC_E_INVALID
    assert lib.kvdec_attend_self(None, ctypes.c_void_p(16), 4, 0.125, 0, ctypes.c_void_p(32),
                                 ctypes.c_void_p(64), 1 << 20, None) == B.KVDEC_E_INVALID
    assert lib.kvdec_append_attend_noalloc(None, ctypes.c_void_p(16), ctypes.c_void_p(32),
                                           ctypes.c_void_p(48), 4, 0.125, 0, ctypes.c_void_p(64),
                                           None) == B.KVDEC_E_INVALID
    assert lib.kvdec_workspace_bytes(None, 4) == 0
    assert lib.kvdec_reset_lens(None, None, None) == B.KVDEC_E_INVALID
    lib.kvdec_cache_destroy(None)


def test_status_strings():
    lib = B.load()
    for code in range(7):
        assert lib.kvdec_status_str(code).decode()
    assert lib.kvdec_status_str(99).decode() == "unknown status"


def test_replay_mode_argument_checks():
    lib = B.load()
    assert lib.kvdec_set_replay_mode(None, 64) == B.KVDEC_E_INVALID
    assert lib.kvdec_paged_set_replay_mode(None, 64, None) == B.KVDEC_E_INVALID
    assert lib.kvdec_set_replay_horizon(None, 4) == B.KVDEC_E_INVALID
    assert lib.kvdec_paged_set_replay_horizon(None, 4) == B.KVDEC_E_INVALID
    assert lib.kvdec_paged_prepare(None, 1, None) == B.KVDEC_E_INVALID


def test_binding_signatures_match_header_arity():
    """Every ctypes signature the binding sets has as many arguments as the
    header's declaration (a missing stream or handle argument would shift
    every later argument)."""
    with open(os.path.join(ROOT, "include", "kvdec.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    lib = B.load()
    decls = re.findall(r"KVDEC_API\s+[^;]*?\b(kvdec_[a-z_]+)\s*\(([^)]*)\)\s*;", text)
    assert len(decls) == len(B.EXPORTED)
    for name, params in decls:
        params = params.strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        assert len(getattr(lib, name).argtypes) == n, name
