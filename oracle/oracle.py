"""ctypes binding of the plain-C f64 oracle (test infrastructure only).

Arrays are numpy arrays.  bf16 tensors are carried as uint16 bit patterns.
Every entry point mirrors one function of kvdec_oracle.c; the arithmetic is
all on the C side.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

# 1/sqrt(head_dim) at head_dim 64; franken_ocr 0.8.0 decoder_qwen2.rs pins
# this as 1/8 (config tests), and every page scales scores by 1/sqrt(d_head).
SCALE_HEAD_DIM_64 = 0.125

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.kvdec_oracle_attend.argtypes = [_vp, _vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i64,
                                            _i64, _vp, ctypes.c_double, _vp]
        lib.kvdec_oracle_prefill_causal.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                    ctypes.c_double, _vp]
        lib.kvdec_oracle_append.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp]
        lib.kvdec_oracle_seed.argtypes = [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64]
        lib.kvdec_oracle_append_slide.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                                  _i64, _i64, _vp, _vp]
        lib.kvdec_oracle_rope.argtypes = [_vp, _i64, _i64, _vp, ctypes.c_double, _vp]
        for f in (lib.kvdec_oracle_attend, lib.kvdec_oracle_prefill_causal,
                  lib.kvdec_oracle_append, lib.kvdec_oracle_seed, lib.kvdec_oracle_rope,
                  lib.kvdec_oracle_append_slide):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(_vp)


def _dtype_code(a):
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"cache dtype must be float32 or uint16 (bf16 bits), got {a.dtype}")


def bf16_to_f32(bits):
    """bf16 bit patterns -> float32 (exact: the bits are the top half of a binary32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def attend(q, K, V, lens, scale=SCALE_HEAD_DIM_64):
    """Decode attention, f64.  q [B,Hq,D] f32; K,V [B,Hkv,cap,D] f32 or bf16 bits; lens [B]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    if K.dtype != V.dtype:
        raise TypeError("K and V must share a dtype")
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    B, Hq, D = q.shape
    Bk, Hkv, cap, Dk = K.shape
    if Bk != B or Dk != D or V.shape != K.shape or lens.shape != (B,):
        raise ValueError("shape mismatch")
    out = np.zeros((B, Hq, D), dtype=np.float64)
    rc = load().kvdec_oracle_attend(_ptr(q), _ptr(K), _ptr(V), _dtype_code(K), B, Hq, Hkv, D, cap,
                                    _ptr(lens), float(scale), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle attend rejected the arguments (code {rc})")
    return out


def prefill_causal(Q, K, V, scale=SCALE_HEAD_DIM_64):
    """Full-causal re-prefill with an explicit mask, f64.  Q [n,Hq,D]; K,V [n,Hkv,D]."""
    Q = np.ascontiguousarray(Q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    n, Hq, D = Q.shape
    _, Hkv, _ = K.shape
    out = np.zeros((n, Hq, D), dtype=np.float64)
    rc = load().kvdec_oracle_prefill_causal(_ptr(Q), _ptr(K), _ptr(V), n, Hq, Hkv, D,
                                            float(scale), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle prefill rejected the arguments (code {rc})")
    return out


def append(Kc, Vc, k_new, v_new, lens):
    """In-place append on numpy caches [B,Hkv,cap,D]; returns the new lens (int32)."""
    if not (Kc.flags.c_contiguous and Vc.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous")
    k_new = np.ascontiguousarray(k_new, dtype=Kc.dtype)
    v_new = np.ascontiguousarray(v_new, dtype=Kc.dtype)
    lens = np.array(lens, dtype=np.int32, copy=True)
    B, Hkv, cap, D = Kc.shape
    rc = load().kvdec_oracle_append(_ptr(Kc), _ptr(Vc), _ptr(k_new), _ptr(v_new),
                                    Kc.dtype.itemsize, B, Hkv, D, cap, _ptr(lens))
    if rc != 0:
        raise ValueError(f"oracle append rejected the arguments (code {rc})")
    return lens


def append_slide(Kc, Vc, k_new, v_new, lens, window, overlap):
    """In-place append with a sliding window keeping `overlap` rows (at most
    window // 2) on numpy caches [B,Hkv,cap,D]; returns (new lens, slid
    flags), both int32."""
    if not (Kc.flags.c_contiguous and Vc.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous")
    k_new = np.ascontiguousarray(k_new, dtype=Kc.dtype)
    v_new = np.ascontiguousarray(v_new, dtype=Kc.dtype)
    lens = np.array(lens, dtype=np.int32, copy=True)
    B, Hkv, cap, D = Kc.shape
    slid = np.zeros(B, dtype=np.int32)
    rc = load().kvdec_oracle_append_slide(_ptr(Kc), _ptr(Vc), _ptr(k_new), _ptr(v_new),
                                          Kc.dtype.itemsize, B, Hkv, D, cap, int(window),
                                          int(overlap), _ptr(lens), _ptr(slid))
    if rc != 0:
        raise ValueError(f"oracle append_slide rejected the arguments (code {rc})")
    return lens, slid


def seed(dst, src):
    """Token-major [B,rows,Hkv*D] -> head-major padded dst [B,Hkv,cap,D], in place."""
    if not dst.flags.c_contiguous:
        raise ValueError("dst must be C-contiguous")
    src = np.ascontiguousarray(src, dtype=dst.dtype)
    B, Hkv, cap, D = dst.shape
    rows = src.shape[1]
    if src.shape != (B, rows, Hkv * D):
        raise ValueError("src shape mismatch")
    rc = load().kvdec_oracle_seed(_ptr(dst), _ptr(src), dst.dtype.itemsize, B, rows, Hkv, D, cap)
    if rc != 0:
        raise ValueError(f"oracle seed rejected the arguments (code {rc})")
    return dst


def rope(x, positions, theta):
    """NEOX rotate-half RoPE in f64 on the last axis.  x [..., D]; positions
    broadcast against x.shape[:-1].  Returns float64."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    flat = np.ascontiguousarray(x.reshape(-1, D))
    pos = np.ascontiguousarray(np.broadcast_to(np.asarray(positions, dtype=np.int32),
                                               x.shape[:-1]).reshape(-1))
    out = np.empty_like(flat)
    rc = load().kvdec_oracle_rope(_ptr(flat), flat.shape[0], D, _ptr(pos), float(theta), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rope rejected the arguments (code {rc})")
    return out.reshape(x.shape)
