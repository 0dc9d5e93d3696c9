"""PyTorch-facing helpers over the C ABI: device tensors in, device tensors out.

KVCache owns torch tensors for one layer's K/V cache and lengths and a
libkvdec handle over them.  Every method only checks shapes/dtypes and
passes pointers to libkvdec.so; all work is done by its HIP kernels on the
current torch stream.
"""
import ctypes

import numpy as np
import torch

from . import binding as B

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_CODE = {"f32": B.KVDEC_F32, "bf16": B.KVDEC_BF16}


def current_stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def to_device(x, device="cuda"):
    """numpy f32 / uint16-as-bf16-bits / int32 array -> device tensor (bit-exact)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(x).to(device)


def to_host_bits(t):
    """device tensor -> numpy with the same bits (bf16 comes back as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


class KVCache:
    def __init__(self, batch, n_kv_heads, capacity, dtype="f32", static=False, lens=None,
                 device="cuda", k=None, v=None, window=0):
        self.batch, self.n_kv_heads, self.capacity = int(batch), int(n_kv_heads), int(capacity)
        self.dtype, self.static = dtype, bool(static)
        self.cap_pad = B.kvdec_padded_capacity(capacity)
        shape = (self.batch, self.n_kv_heads, self.cap_pad, B.HEAD_DIM)
        tdt = _TORCH_DTYPE[dtype]
        self.k = torch.zeros(shape, dtype=tdt, device=device) if k is None else k
        self.v = torch.zeros(shape, dtype=tdt, device=device) if v is None else v
        for t in (self.k, self.v):
            if tuple(t.shape) != shape or t.dtype != tdt or not t.is_contiguous():
                raise ValueError(f"cache tensor must be contiguous {shape} {tdt}")
        self.lens_dev = torch.zeros(self.batch, dtype=torch.int32, device=device)
        self.window = int(window)
        self.desc = B.CacheDesc(self.batch, self.n_kv_heads, B.HEAD_DIM, self.capacity,
                                _CODE[dtype], int(self.static), self.window, 0, self.k.data_ptr(),
                                self.v.data_ptr(), self.lens_dev.data_ptr())
        lens = [0] * self.batch if lens is None else [int(x) for x in lens]
        self.handle = B.kvdec_cache_create(self.desc, lens, current_stream())
        self._ws = {}

    # --- state -------------------------------------------------------------
    def lens(self):
        return B.kvdec_get_lens(self.handle, self.batch)

    def reset_lens(self, lens):
        B.kvdec_reset_lens(self.handle, [int(x) for x in lens], current_stream())

    def set_replay_mode(self, chunk_rows):
        B.kvdec_set_replay_mode(self.handle, chunk_rows)

    def set_replay_horizon(self, tokens):
        B.kvdec_set_replay_horizon(self.handle, tokens)

    def close(self):
        if getattr(self, "handle", None):
            B.kvdec_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # --- operations ---------------------------------------------------------
    def _check_rows(self, t, shape, name):
        if t.dtype != self.k.dtype or tuple(t.shape) != shape or not t.is_contiguous() \
                or t.device != self.k.device:
            raise ValueError(f"{name} must be a contiguous {shape} {self.k.dtype} tensor on "
                             f"{self.k.device}")

    def seed(self, k_tok, v_tok):
        rows = k_tok.shape[1]
        shape = (self.batch, rows, self.n_kv_heads * B.HEAD_DIM)
        self._check_rows(k_tok, shape, "k_tok")
        self._check_rows(v_tok, shape, "v_tok")
        B.kvdec_seed(self.handle, _ptr(k_tok), _ptr(v_tok), rows, current_stream())

    def append(self, k_new, v_new):
        shape = (self.batch, self.n_kv_heads, B.HEAD_DIM)
        self._check_rows(k_new, shape, "k_new")
        self._check_rows(v_new, shape, "v_new")
        B.kvdec_append(self.handle, _ptr(k_new), _ptr(v_new), current_stream())

    def append_slide(self, k_new, v_new, overlap):
        """Append; a full sequence first keeps only its last min(overlap,
        capacity // 2) rows (the streaming cache's slide).  Returns the
        per-sequence slid flags."""
        shape = (self.batch, self.n_kv_heads, B.HEAD_DIM)
        self._check_rows(k_new, shape, "k_new")
        self._check_rows(v_new, shape, "v_new")
        return B.kvdec_append_slide(self.handle, _ptr(k_new), _ptr(v_new), overlap, self.batch,
                                    current_stream())

    def append_rope(self, k_new, v_new, theta, q=None, q_rot=None):
        """Append un-rotated keys, rotating them (and q into q_rot) at each
        sequence's current position.  Returns q_rot (or None)."""
        shape = (self.batch, self.n_kv_heads, B.HEAD_DIM)
        self._check_rows(k_new, shape, "k_new")
        self._check_rows(v_new, shape, "v_new")
        qp = qr = None
        Hq = 0
        if q is not None:
            if q.dtype != torch.float32 or q.dim() != 3 or not q.is_contiguous():
                raise ValueError("q must be a contiguous float32 [batch, n_q_heads, 64] tensor")
            if q_rot is None:
                q_rot = torch.empty_like(q)
            Hq, qp, qr = q.shape[1], _ptr(q), _ptr(q_rot)
        B.kvdec_append_rope(self.handle, _ptr(k_new), _ptr(v_new), theta, qp, qr, Hq,
                            current_stream())
        return q_rot

    def workspace(self, n_q_heads):
        ws = self._ws.get(n_q_heads)
        if ws is None:
            nbytes = B.kvdec_workspace_bytes(self.handle, n_q_heads)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=self.k.device)
            self._ws[n_q_heads] = ws
        return ws

    def _q_out(self, q, out):
        """Check q ([batch, n_q_heads, 64] f32 on the cache's device) and out
        (same, allocated when None); returns out."""
        if q.dtype != torch.float32 or q.dim() != 3 or q.shape[0] != self.batch \
                or q.shape[2] != B.HEAD_DIM or not q.is_contiguous() or q.device != self.k.device:
            raise ValueError("q must be a contiguous float32 [batch, n_q_heads, 64] device tensor")
        if out is None:
            return torch.empty_like(q)
        if out.dtype != torch.float32 or out.shape != q.shape or not out.is_contiguous() \
                or out.device != q.device:
            raise ValueError("out must be a contiguous float32 tensor shaped like q")
        return out

    def append_attend(self, k_new, v_new, q, scale=0.125, chunk_rows=0, out=None):
        """Append one token and attend, as one call (one launch when possible)."""
        shape = (self.batch, self.n_kv_heads, B.HEAD_DIM)
        self._check_rows(k_new, shape, "k_new")
        self._check_rows(v_new, shape, "v_new")
        out = self._q_out(q, out)
        ws = self.workspace(q.shape[1])
        B.kvdec_append_attend(self.handle, _ptr(k_new), _ptr(v_new), _ptr(q), q.shape[1], scale,
                              chunk_rows, _ptr(out), _ptr(ws), ws.numel(), current_stream())
        return out

    def append_attend_cross(self, cross, k_new, v_new, q_self, q_cross, scale=0.125, chunk_self=0,
                            chunk_cross=0, out_self=None, out_cross=None, lens=None):
        """One decoder layer's attention step: append + self-attend on this
        cache (at positions `lens` when given) and cross-attend over the
        static cache `cross`, as one call (one attend launch).  Returns
        (out_self, out_cross)."""
        if lens is not None:
            lens = [int(x) for x in lens]
            if len(lens) != self.batch:
                raise ValueError(f"lens must hold {self.batch} positions")
        shape = (self.batch, self.n_kv_heads, B.HEAD_DIM)
        self._check_rows(k_new, shape, "k_new")
        self._check_rows(v_new, shape, "v_new")
        out_self = self._q_out(q_self, out_self)
        out_cross = cross._q_out(q_cross, out_cross)
        Hq = q_self.shape[1]
        key = ("pair", cross.cap_pad, Hq)
        ws = self._ws.get(key)
        if ws is None:
            nbytes = (B.kvdec_workspace_bytes(self.handle, Hq) +
                      B.kvdec_workspace_bytes(cross.handle, Hq))
            ws = torch.empty(nbytes, dtype=torch.uint8, device=self.k.device)
            self._ws[key] = ws
        B.kvdec_append_attend_cross(self.handle, cross.handle, lens, _ptr(k_new), _ptr(v_new), _ptr(q_self),
                                    _ptr(q_cross), Hq, scale, chunk_self, chunk_cross,
                                    _ptr(out_self), _ptr(out_cross), _ptr(ws), ws.numel(),
                                    current_stream())
        return out_self, out_cross

    def append_attend_at(self, lens, k_new, v_new, q, scale=0.125, chunk_rows=0, out=None):
        """Set the lengths to `lens` (the new token's positions), then append
        and attend, as one call."""
        shape = (self.batch, self.n_kv_heads, B.HEAD_DIM)
        self._check_rows(k_new, shape, "k_new")
        self._check_rows(v_new, shape, "v_new")
        lens = [int(x) for x in lens]
        if len(lens) != self.batch:
            raise ValueError(f"lens must hold {self.batch} positions")
        out = self._q_out(q, out)
        ws = self.workspace(q.shape[1])
        B.kvdec_append_attend_at(self.handle, lens, _ptr(k_new), _ptr(v_new), _ptr(q), q.shape[1],
                                 scale, chunk_rows, _ptr(out), _ptr(ws), ws.numel(),
                                 current_stream())
        return out

    def attend(self, q, scale=0.125, chunk_rows=0, out=None):
        Hq = q.shape[1]
        out = self._q_out(q, out)
        ws = self.workspace(Hq)
        fn = B.kvdec_attend_cross if self.static else B.kvdec_attend_self
        fn(self.handle, _ptr(q), Hq, scale, chunk_rows, _ptr(out), _ptr(ws), ws.numel(),
           current_stream())
        return out


class PagedKVCache:
    """Paged K/V pool + block table over the kvdec_paged_* entry points."""

    def __init__(self, batch, n_kv_heads, page_rows, num_pages, max_pages_per_seq, dtype="f32",
                 device="cuda"):
        self.batch, self.n_kv_heads = int(batch), int(n_kv_heads)
        self.page_rows, self.num_pages = int(page_rows), int(num_pages)
        self.max_pages = int(max_pages_per_seq)
        self.dtype = dtype
        tdt = _TORCH_DTYPE[dtype]
        shape = (self.n_kv_heads, self.num_pages, self.page_rows, B.HEAD_DIM)   # head-major pool
        self.k = torch.zeros(shape, dtype=tdt, device=device)
        self.v = torch.zeros(shape, dtype=tdt, device=device)
        self.table_dev = torch.full((self.batch, self.max_pages), -1, dtype=torch.int32,
                                    device=device)
        self.lens_dev = torch.zeros(self.batch, dtype=torch.int32, device=device)
        self.desc = B.PagedDesc(self.batch, self.n_kv_heads, B.HEAD_DIM, _CODE[dtype],
                                self.page_rows, self.num_pages, self.max_pages, 0,
                                self.k.data_ptr(), self.v.data_ptr(), self.table_dev.data_ptr(),
                                self.lens_dev.data_ptr())
        self.handle = B.kvdec_paged_create(self.desc, current_stream())
        self._ws = {}

    def lens(self):
        return B.kvdec_paged_get_lens(self.handle, self.batch)

    def table(self):
        return B.kvdec_paged_get_table(self.handle, self.batch, self.max_pages)

    def free_pages(self):
        return B.kvdec_paged_free_pages(self.handle)

    def append(self, k_new, v_new):
        shape = (self.batch, self.n_kv_heads, B.HEAD_DIM)
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            if t.dtype != self.k.dtype or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError(f"{n} must be a contiguous {shape} {self.k.dtype} tensor")
        B.kvdec_paged_append(self.handle, _ptr(k_new), _ptr(v_new), current_stream())

    def release(self, seq):
        B.kvdec_paged_release(self.handle, seq, current_stream())

    def set_replay_mode(self, chunk_rows):
        B.kvdec_paged_set_replay_mode(self.handle, chunk_rows, current_stream())

    def set_replay_horizon(self, tokens):
        B.kvdec_paged_set_replay_horizon(self.handle, tokens)

    def prepare(self, n_tokens=1):
        """Replay mode: pages for every sequence's next n_tokens rows (call
        between graph replays)."""
        B.kvdec_paged_prepare(self.handle, n_tokens, current_stream())

    def reserve(self, seq, length):
        B.kvdec_paged_reserve(self.handle, seq, length, current_stream())

    def truncate(self, lens):
        B.kvdec_paged_truncate(self.handle, [int(x) for x in lens], current_stream())

    def load_contiguous(self, k, v, lens):
        """Reserve pages for empty sequences and copy rows [0, lens[b]) of a
        contiguous [B][Hkv][cap][64] cache into them (a prefill hand-off)."""
        for b, n in enumerate(lens):
            self.reserve(b, int(n))
        table = self.table()
        P = self.page_rows
        for b, n in enumerate(lens):
            n = int(n)
            for i in range((n + P - 1) // P):
                rows = min(P, n - i * P)
                self.k[:, table[b][i], :rows] = k[b, :, i * P:i * P + rows]
                self.v[:, table[b][i], :rows] = v[b, :, i * P:i * P + rows]

    def workspace(self, n_q_heads):
        ws = self._ws.get(n_q_heads)
        if ws is None:
            ws = torch.empty(B.kvdec_paged_workspace_bytes(self.handle, n_q_heads), dtype=torch.uint8,
                             device=self.k.device)
            self._ws[n_q_heads] = ws
        return ws

    def attend(self, q, scale=0.125, chunk_rows=0, out=None):
        Hq = q.shape[1]
        out = KVCache._q_out(self, q, out)
        ws = self.workspace(Hq)
        B.kvdec_paged_attend(self.handle, _ptr(q), Hq, scale, chunk_rows, _ptr(out), _ptr(ws),
                             ws.numel(), current_stream())
        return out

    def append_attend(self, k_new, v_new, q, scale=0.125, chunk_rows=0, out=None):
        """kvdec_paged_append_attend: append the token, attend len + 1 rows."""
        shape = (self.batch, self.n_kv_heads, B.HEAD_DIM)
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            if t.dtype != self.k.dtype or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError(f"{n} must be a contiguous {shape} {self.k.dtype} tensor")
        Hq = q.shape[1]
        out = KVCache._q_out(self, q, out)
        ws = self.workspace(Hq)
        B.kvdec_paged_append_attend(self.handle, _ptr(k_new), _ptr(v_new), _ptr(q), Hq, scale,
                                    chunk_rows, _ptr(out), _ptr(ws), ws.numel(), current_stream())
        return out

    def close(self):
        if getattr(self, "handle", None):
            B.kvdec_paged_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
