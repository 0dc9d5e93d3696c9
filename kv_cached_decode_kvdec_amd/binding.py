"""ctypes binding of libkvdec.so (include/kvdec.h), same names as the C ABI.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libkvdec.so.  If the library is missing, load() raises -- there
is no fallback path of any kind.  PyTorch is used for device memory and the
current HIP stream.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvdec.so")

KVDEC_OK = 0
KVDEC_E_INVALID = 1
KVDEC_E_SHAPE = 2
KVDEC_E_OVERFLOW = 3
KVDEC_E_STATIC = 4
KVDEC_E_WORKSPACE = 5
KVDEC_E_HIP = 6
KVDEC_F32 = 0
KVDEC_BF16 = 1
HEAD_DIM = 64
MIN_CHUNK = 64
MAX_CHUNK = 4096
MAX_GROUP = 8
KVDEC_MAX_FUSED_BATCH = 512
KVDEC_MAX_PAGED_FUSED_BATCH = 256
KVDEC_NOALLOC_SCRATCH_BYTES = 16777216

EXPORTED = [
    "kvdec_padded_capacity", "kvdec_cache_create", "kvdec_cache_destroy", "kvdec_reset_lens",
    "kvdec_get_lens", "kvdec_seed", "kvdec_append", "kvdec_append_rope", "kvdec_workspace_bytes",
    "kvdec_attend_self", "kvdec_attend_cross", "kvdec_append_attend", "kvdec_append_attend_at",
    "kvdec_set_replay_mode",
    "kvdec_set_replay_horizon",
    "kvdec_status_str",
    "kvdec_last_error", "kvdec_paged_create", "kvdec_paged_destroy", "kvdec_paged_append",
    "kvdec_paged_release", "kvdec_paged_reserve", "kvdec_paged_truncate",
    "kvdec_paged_get_lens", "kvdec_paged_get_table",
    "kvdec_paged_free_pages", "kvdec_paged_workspace_bytes", "kvdec_paged_attend",
    "kvdec_paged_append_attend",
    "kvdec_paged_set_replay_mode",
    "kvdec_paged_prepare",
    "kvdec_paged_set_replay_horizon",
    "kvdec_append_attend_noalloc",
    "kvdec_append_attend_cross",
    "kvdec_append_slide",
]


class KvdecError(RuntimeError):
    def __init__(self, code, where, detail):
        super().__init__(f"{where}: {detail} (status {code})")
        self.code = code


class CacheDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("is_static", ctypes.c_int32),
                ("window", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("lens", ctypes.c_void_p)]


class PagedDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("page_rows", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("lens", ctypes.c_void_p)]


_lib = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


def load():
    """Load libkvdec.so; raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import "
                          f"__graft_entry__ as g; g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "kvdec_padded_capacity": (_i32, [_i32]),
        "kvdec_cache_create": (_i32, [ctypes.POINTER(CacheDesc), _vp, _vp, ctypes.POINTER(_vp)]),
        "kvdec_cache_destroy": (None, [_vp]),
        "kvdec_reset_lens": (_i32, [_vp, _vp, _vp]),
        "kvdec_get_lens": (_i32, [_vp, _vp]),
        "kvdec_seed": (_i32, [_vp, _vp, _vp, _i32, _vp]),
        "kvdec_append": (_i32, [_vp, _vp, _vp, _vp]),
        "kvdec_append_rope": (_i32, [_vp, _vp, _vp, ctypes.c_float, _vp, _vp, _i32, _vp]),
        "kvdec_append_slide": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp]),
        "kvdec_workspace_bytes": (_sz, [_vp, _i32]),
        "kvdec_attend_self": (_i32, [_vp, _vp, _i32, ctypes.c_float, _i32, _vp, _vp, _sz, _vp]),
        "kvdec_attend_cross": (_i32, [_vp, _vp, _i32, ctypes.c_float, _i32, _vp, _vp, _sz, _vp]),
        "kvdec_set_replay_mode": (_i32, [_vp, _i32]),
        "kvdec_set_replay_horizon": (_i32, [_vp, _i32]),
        "kvdec_append_attend": (_i32, [_vp, _vp, _vp, _vp, _i32, ctypes.c_float, _i32, _vp, _vp, _sz,
                                       _vp]),
        "kvdec_append_attend_at": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, ctypes.c_float, _i32, _vp,
                                          _vp, _sz, _vp]),
        "kvdec_append_attend_noalloc": (_i32, [_vp, _vp, _vp, _vp, _i32, ctypes.c_float, _i32, _vp,
                                               _vp]),
        "kvdec_append_attend_cross": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, ctypes.c_float,
                                             _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
        "kvdec_paged_create": (_i32, [ctypes.POINTER(PagedDesc), _vp, ctypes.POINTER(_vp)]),
        "kvdec_paged_destroy": (None, [_vp]),
        "kvdec_paged_append": (_i32, [_vp, _vp, _vp, _vp]),
        "kvdec_paged_release": (_i32, [_vp, _i32, _vp]),
        "kvdec_paged_reserve": (_i32, [_vp, _i32, _i32, _vp]),
        "kvdec_paged_truncate": (_i32, [_vp, _vp, _vp]),
        "kvdec_paged_get_lens": (_i32, [_vp, _vp]),
        "kvdec_paged_get_table": (_i32, [_vp, _vp]),
        "kvdec_paged_free_pages": (_i32, [_vp]),
        "kvdec_paged_workspace_bytes": (_sz, [_vp, _i32]),
        "kvdec_paged_attend": (_i32, [_vp, _vp, _i32, ctypes.c_float, _i32, _vp, _vp, _sz, _vp]),
        "kvdec_paged_append_attend": (_i32, [_vp, _vp, _vp, _vp, _i32, ctypes.c_float, _i32, _vp,
                                             _vp, _sz, _vp]),
        "kvdec_paged_set_replay_mode": (_i32, [_vp, _i32, _vp]),
        "kvdec_paged_prepare": (_i32, [_vp, _i32, _vp]),
        "kvdec_paged_set_replay_horizon": (_i32, [_vp, _i32]),
        "kvdec_status_str": (ctypes.c_char_p, [_i32]),
        "kvdec_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(code, where):
    if code != KVDEC_OK:
        lib = load()
        raise KvdecError(code, where, lib.kvdec_last_error().decode() or
                         lib.kvdec_status_str(code).decode())


def _int_array(vals):
    arr = (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])
    return arr


# --- thin wrappers, one per C entry point --------------------------------------

def kvdec_padded_capacity(capacity):
    return load().kvdec_padded_capacity(int(capacity))


def kvdec_cache_create(desc, lens_host, stream=None):
    h = _vp()
    arr = _int_array(lens_host)
    _check(load().kvdec_cache_create(ctypes.byref(desc), arr, stream, ctypes.byref(h)),
           "kvdec_cache_create")
    return h


def kvdec_cache_destroy(handle):
    if handle:
        load().kvdec_cache_destroy(handle)


def kvdec_reset_lens(handle, lens_host, stream=None):
    _check(load().kvdec_reset_lens(handle, _int_array(lens_host), stream), "kvdec_reset_lens")


def kvdec_get_lens(handle, batch):
    arr = (ctypes.c_int32 * batch)()
    _check(load().kvdec_get_lens(handle, arr), "kvdec_get_lens")
    return list(arr)


def kvdec_seed(handle, k_tok_ptr, v_tok_ptr, rows, stream=None):
    _check(load().kvdec_seed(handle, k_tok_ptr, v_tok_ptr, int(rows), stream), "kvdec_seed")


def kvdec_append(handle, k_new_ptr, v_new_ptr, stream=None):
    _check(load().kvdec_append(handle, k_new_ptr, v_new_ptr, stream), "kvdec_append")


def kvdec_append_rope(handle, k_new_ptr, v_new_ptr, theta, q_ptr=None, q_rot_ptr=None,
                      n_q_heads=0, stream=None):
    _check(load().kvdec_append_rope(handle, k_new_ptr, v_new_ptr, float(theta), q_ptr, q_rot_ptr,
                                    int(n_q_heads), stream), "kvdec_append_rope")


def kvdec_workspace_bytes(handle, n_q_heads):
    return load().kvdec_workspace_bytes(handle, int(n_q_heads))


def kvdec_attend_self(handle, q_ptr, n_q_heads, scale, chunk_rows, out_ptr, ws_ptr, ws_bytes,
                      stream=None):
    _check(load().kvdec_attend_self(handle, q_ptr, int(n_q_heads), float(scale), int(chunk_rows),
                                    out_ptr, ws_ptr, int(ws_bytes), stream), "kvdec_attend_self")


def kvdec_attend_cross(handle, q_ptr, n_q_heads, scale, chunk_rows, out_ptr, ws_ptr, ws_bytes,
                       stream=None):
    _check(load().kvdec_attend_cross(handle, q_ptr, int(n_q_heads), float(scale), int(chunk_rows),
                                     out_ptr, ws_ptr, int(ws_bytes), stream), "kvdec_attend_cross")


def kvdec_set_replay_mode(handle, chunk_rows):
    _check(load().kvdec_set_replay_mode(handle, int(chunk_rows)), "kvdec_set_replay_mode")


def kvdec_set_replay_horizon(handle, tokens):
    _check(load().kvdec_set_replay_horizon(handle, int(tokens)), "kvdec_set_replay_horizon")


def kvdec_paged_create(desc, stream=None):
    h = _vp()
    _check(load().kvdec_paged_create(ctypes.byref(desc), stream, ctypes.byref(h)),
           "kvdec_paged_create")
    return h


def kvdec_paged_destroy(handle):
    if handle:
        load().kvdec_paged_destroy(handle)


def kvdec_paged_append(handle, k_new_ptr, v_new_ptr, stream=None):
    _check(load().kvdec_paged_append(handle, k_new_ptr, v_new_ptr, stream), "kvdec_paged_append")


def kvdec_paged_release(handle, seq, stream=None):
    _check(load().kvdec_paged_release(handle, int(seq), stream), "kvdec_paged_release")


def kvdec_paged_reserve(handle, seq, length, stream=None):
    _check(load().kvdec_paged_reserve(handle, int(seq), int(length), stream), "kvdec_paged_reserve")


def kvdec_paged_truncate(handle, lens_host, stream=None):
    _check(load().kvdec_paged_truncate(handle, _int_array(lens_host), stream), "kvdec_paged_truncate")


def kvdec_paged_get_lens(handle, batch):
    arr = (ctypes.c_int32 * batch)()
    _check(load().kvdec_paged_get_lens(handle, arr), "kvdec_paged_get_lens")
    return list(arr)


def kvdec_paged_get_table(handle, batch, max_pages):
    arr = (ctypes.c_int32 * (batch * max_pages))()
    _check(load().kvdec_paged_get_table(handle, arr), "kvdec_paged_get_table")
    return [list(arr[b * max_pages:(b + 1) * max_pages]) for b in range(batch)]


def kvdec_paged_free_pages(handle):
    return load().kvdec_paged_free_pages(handle)


def kvdec_paged_workspace_bytes(handle, n_q_heads):
    return load().kvdec_paged_workspace_bytes(handle, int(n_q_heads))


def kvdec_paged_attend(handle, q_ptr, n_q_heads, scale, chunk_rows, out_ptr, ws_ptr, ws_bytes,
                       stream=None):
    _check(load().kvdec_paged_attend(handle, q_ptr, int(n_q_heads), float(scale), int(chunk_rows),
                                     out_ptr, ws_ptr, int(ws_bytes), stream), "kvdec_paged_attend")


def kvdec_paged_append_attend(handle, k_new_ptr, v_new_ptr, q_ptr, n_q_heads, scale, chunk_rows,
                              out_ptr, ws_ptr, ws_bytes, stream=None):
    _check(load().kvdec_paged_append_attend(handle, k_new_ptr, v_new_ptr, q_ptr, int(n_q_heads),
                                            float(scale), int(chunk_rows), out_ptr, ws_ptr,
                                            int(ws_bytes), stream), "kvdec_paged_append_attend")


def kvdec_paged_set_replay_mode(handle, chunk_rows, stream=None):
    _check(load().kvdec_paged_set_replay_mode(handle, int(chunk_rows), stream),
           "kvdec_paged_set_replay_mode")


def kvdec_paged_prepare(handle, n_tokens, stream=None):
    _check(load().kvdec_paged_prepare(handle, int(n_tokens), stream), "kvdec_paged_prepare")


def kvdec_paged_set_replay_horizon(handle, tokens):
    _check(load().kvdec_paged_set_replay_horizon(handle, int(tokens)), "kvdec_paged_set_replay_horizon")


def kvdec_append_attend(handle, k_new_ptr, v_new_ptr, q_ptr, n_q_heads, scale, chunk_rows, out_ptr,
                        ws_ptr, ws_bytes, stream=None):
    _check(load().kvdec_append_attend(handle, k_new_ptr, v_new_ptr, q_ptr, int(n_q_heads),
                                      float(scale), int(chunk_rows), out_ptr, ws_ptr, int(ws_bytes),
                                      stream), "kvdec_append_attend")


def kvdec_append_attend_at(handle, lens_host, k_new_ptr, v_new_ptr, q_ptr, n_q_heads, scale,
                           chunk_rows, out_ptr, ws_ptr, ws_bytes, stream=None):
    """lens_host: a sequence of ints or a ctypes int32 array (host)."""
    if not isinstance(lens_host, ctypes.Array):
        lens_host = (ctypes.c_int32 * len(lens_host))(*[int(x) for x in lens_host])
    _check(load().kvdec_append_attend_at(handle, lens_host, k_new_ptr, v_new_ptr, q_ptr,
                                         int(n_q_heads), float(scale), int(chunk_rows), out_ptr,
                                         ws_ptr, int(ws_bytes), stream), "kvdec_append_attend_at")


def kvdec_append_attend_noalloc(handle, k_new_ptr, v_new_ptr, q_ptr, n_q_heads, scale, chunk_rows,
                                out_ptr, stream=None):
    _check(load().kvdec_append_attend_noalloc(handle, k_new_ptr, v_new_ptr, q_ptr, int(n_q_heads),
                                              float(scale), int(chunk_rows), out_ptr, stream),
           "kvdec_append_attend_noalloc")


def kvdec_append_attend_cross(self_handle, cross_handle, lens_host, k_new_ptr, v_new_ptr, q_self_ptr,
                              q_cross_ptr, n_q_heads, scale, chunk_self, chunk_cross, out_self_ptr,
                              out_cross_ptr, ws_ptr, ws_bytes, stream=None):
    """lens_host: None, a sequence of ints or a ctypes int32 array (host)."""
    if lens_host is not None and not isinstance(lens_host, ctypes.Array):
        lens_host = (ctypes.c_int32 * len(lens_host))(*[int(x) for x in lens_host])
    _check(load().kvdec_append_attend_cross(self_handle, cross_handle, lens_host, k_new_ptr, v_new_ptr,
                                            q_self_ptr, q_cross_ptr, int(n_q_heads), float(scale),
                                            int(chunk_self), int(chunk_cross), out_self_ptr,
                                            out_cross_ptr, ws_ptr, int(ws_bytes), stream),
           "kvdec_append_attend_cross")


def kvdec_append_slide(handle, k_new_ptr, v_new_ptr, overlap, batch, stream=None):
    """Returns the per-sequence slid flags (host mirror)."""
    slid = (ctypes.c_int32 * batch)()
    _check(load().kvdec_append_slide(handle, k_new_ptr, v_new_ptr, int(overlap), slid, stream),
           "kvdec_append_slide")
    return list(slid)
