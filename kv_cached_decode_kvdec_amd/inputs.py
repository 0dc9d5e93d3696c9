"""Seeded synthetic workloads for the KV-cached decode step.

This module is shared by the HIP path's tests/benchmark and by the oracle's
tests.  It only draws random numbers and lays them out; it holds none of the
decode arithmetic (no score, softmax, weighted sum or rotary embedding).

The Qwen2-shaped workload caches post-RoPE keys on the pages (franken_ocr
0.8.0 decoder_qwen2.rs, `qwen2_decode_step`: RoPE on q and k, then append).
Drawing the rotated vectors directly is the same thing in distribution: a
rotation of each dim pair (i, i+32) maps an i.i.d. normal pair to an i.i.d.
normal pair, so rotated standard-normal keys and queries are standard normal.
The RoPE arithmetic itself is exercised by the rotate-at-append entry point.

Recipe (fixed draw order, numpy PCG64, seed = 1000 + workload index):
  1. pre-append lengths per sequence;
  2. cached K, then V, at full padded capacity, head-major [B][Hkv][cap][64];
  3. per decode step: k_new, v_new [B][Hkv][64], q_self [B][Hq][64],
     and q_cross [B][H][64] where the workload has cross-attention;
  4. cross (encoder) K, then V, token-major [B][1500][H*64].
Values are standard normal drawn in float32; bf16 workloads round them to
bfloat16 with round-to-nearest-even and carry the bit patterns as uint16.
"""
from dataclasses import dataclass, field
import math

import numpy as np

HEAD_DIM = 64
ROW_ALIGN = 64          # padded capacity granule (rows per (b, kv head))
ENC_LEN = 1500          # Whisper encoder positions (30 s of audio)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    dtype: str              # "f32" or "bf16" for the K/V caches; q and out are f32
    lens: str               # length law, see draw_lens
    steps: int              # consecutive decode steps with append
    cross: bool             # cross-attention over ENC_LEN static rows
    input_scale: float = 1.0
    rope_theta: float = 0.0  # > 0: RoPE base of the model (rotate-at-append variant)
    seed: int = 0
    describe: str = field(default="", compare=False)


WORKLOADS = {
    "whisper-tiny": Workload("whisper-tiny", 1, 6, 6, "f32", "const:32", 1, True,
                             input_scale=1.0 / 8.0, seed=1001,
                             describe="B1 H6 f32, self 32 (append 1 -> attend 33) + cross 1500"),
    "whisper-base": Workload("whisper-base", 16, 8, 8, "f32", "uniform:1:448", 1, True, seed=1002,
                             describe="B16 H8 f32, self U{1..448} + cross 1500"),
    "whisper-large": Workload("whisper-large", 64, 20, 20, "bf16", "const:448", 32, True,
                              seed=1003,
                              describe="B64 H20 bf16 K/V, self 448 + 32 steps, cross 1500"),
    "qwen2-0.5b": Workload("qwen2-0.5b", 32, 16, 16, "f32", "uniform:1:4096", 1, False,
                           rope_theta=1.0e6, seed=1004,
                           describe="B32 H16 MHA f32, RoPE'd q/K, self U{1..4096}"),
    "gqa": Workload("gqa", 64, 16, 4, "bf16", "loguniform:16:8192", 8, False, seed=1005,
                    describe="B64 16 q heads / 4 KV heads bf16, log-U[16,8192], 8 steps"),
}
ORDER = ["whisper-tiny", "whisper-base", "whisper-large", "qwen2-0.5b", "gqa"]


def padded_rows(rows: int) -> int:
    return max(ROW_ALIGN, -(-rows // ROW_ALIGN) * ROW_ALIGN)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even; NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def draw_lens(rng: np.random.Generator, law: str, batch: int) -> np.ndarray:
    kind, *args = law.split(":")
    if kind == "const":
        return np.full(batch, int(args[0]), dtype=np.int32)
    if kind == "uniform":
        lo, hi = int(args[0]), int(args[1])
        return rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    if kind == "loguniform":
        lo, hi = int(args[0]), int(args[1])
        x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch))
        return np.clip(np.rint(x), lo, hi).astype(np.int32)
    raise ValueError(f"unknown length law {law!r}")


@dataclass
class Inputs:
    wl: Workload
    lens: np.ndarray          # [B] int32, pre-append lengths
    cap: int                  # padded rows per (b, kv head) of the self cache
    k_cache: np.ndarray       # [B][Hkv][cap][64] f32 or uint16 (bf16 bits)
    v_cache: np.ndarray
    k_new: list               # per step: [B][Hkv][64]
    v_new: list
    q_self: list              # per step: [B][Hq][64] f32
    q_cross: list             # per step: [B][H][64] f32 (empty without cross)
    cross_k_tok: np.ndarray = None   # [B][1500][H*64], token-major
    cross_v_tok: np.ndarray = None

    @property
    def elem(self):
        return np.float32 if self.wl.dtype == "f32" else np.uint16


def _to_cache_dtype(x, dtype):
    return x.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(x)


def make_inputs(wl: Workload, *, seed=None, batch=None, lens=None, steps=None,
                canary=True, enc_len=ENC_LEN, rows_override=None) -> Inputs:
    """Draw a workload's inputs.

    batch / lens / steps / enc_len override the workload (small parity cases);
    canary=True fills every cache row at or beyond a sequence's length with NaN
    so that any read past the valid rows poisons the result.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B = wl.batch if batch is None else batch
    S = wl.steps if steps is None else steps
    Hq, Hkv, D = wl.n_q_heads, wl.n_kv_heads, HEAD_DIM
    if lens is None:
        lens = draw_lens(rng, wl.lens, B)
    lens = np.asarray(lens, dtype=np.int32)
    assert lens.shape == (B,)
    rows = int(lens.max(initial=0)) + S if rows_override is None else rows_override
    cap = padded_rows(rows)
    sc = np.float32(wl.input_scale)

    def normal(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        return x * sc if wl.input_scale != 1.0 else x

    kc = normal((B, Hkv, cap, D))
    vc = normal((B, Hkv, cap, D))
    k_new, v_new, q_self, q_cross = [], [], [], []
    for s in range(S):
        kn = normal((B, Hkv, D))
        vn = normal((B, Hkv, D))
        qs = normal((B, Hq, D))
        if wl.cross:
            q_cross.append(normal((B, Hq, D)))
        k_new.append(_to_cache_dtype(kn, wl.dtype))
        v_new.append(_to_cache_dtype(vn, wl.dtype))
        q_self.append(qs.astype(np.float32))
    fill = np.float32(np.nan) if canary else np.float32(0.0)
    for b in range(B):
        kc[b, :, lens[b]:, :] = fill
        vc[b, :, lens[b]:, :] = fill
    inp = Inputs(wl, lens, cap, _to_cache_dtype(kc, wl.dtype), _to_cache_dtype(vc, wl.dtype),
                 k_new, v_new, q_self, q_cross)
    if wl.cross:
        inp.cross_k_tok = _to_cache_dtype(normal((B, enc_len, Hkv * D)), wl.dtype)
        inp.cross_v_tok = _to_cache_dtype(normal((B, enc_len, Hkv * D)), wl.dtype)
    return inp


def kv_bytes_per_step(wl: Workload, lens_post: np.ndarray, enc_len: int = ENC_LEN) -> int:
    """Algorithmic HBM bytes of one decode step (append + self [+ cross]).

    Each valid KV row is read once (K and V), the appended rows are read and
    written once, q is read and out written once; padding, workspace and the
    length array are implementation overhead and are not counted.
    """
    s = 4 if wl.dtype == "f32" else 2
    B, Hq, Hkv, D = len(lens_post), wl.n_q_heads, wl.n_kv_heads, HEAD_DIM
    total = int(np.sum(lens_post, dtype=np.int64)) * Hkv * D * 2 * s
    total += B * Hkv * D * 2 * s * 2          # append: read new K,V rows + write them
    total += B * Hq * D * 4 * 2               # q read + out write
    if wl.cross:
        total += B * Hkv * enc_len * D * 2 * s + B * Hq * D * 4 * 2
    return total
