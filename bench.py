"""Benchmark of the single-token KV-cached decode step on one MI355X.

One step = one decode token for every sequence of one layer: append the new
K/V row and self-attention over the cached rows and, for the Whisper-shaped
workloads, cross-attention over the 1500 static encoder rows.  Step forms
(--form):
  layer      (default) one call per step: kvdec_append_attend_cross for the
             Whisper workloads (self append + attend and cross attend in one
             attend launch), kvdec_append_attend for the others;
  two-calls  kvdec_append_attend, then kvdec_attend_cross;
  unfused    kvdec_append, kvdec_attend_self, then kvdec_attend_cross.
Workloads with several consecutive steps (Whisper-large: 32, GQA: 8) cycle
through them; the first step of each cycle runs at the workload's starting
positions (the calls' positions argument, which rewinds the lengths inside
the same launch; the unfused form rolls them back with kvdec_reset_lens, one
tiny kernel counted in the step).

Prints ONE JSON line on stdout (the headline workload, default
whisper-large: batch 64, 20 heads, bf16 K/V, self 448 -> 480 over 32 steps
plus cross-attention over 1500 rows) and a per-workload table on stderr.

Inputs are seeded synthetic tensors resident in HBM before the timed region
starts.  `value` comes from exactly K back-to-back steps bracketed by device
synchronisation, with nothing else on the stream (warm: the step's working
set may partly sit in the 256 MB Infinity Cache from the step before; the
headline moves 645 MB per step, so warm and cold agree there).  Then, per
workload:
  windows   HIP events at the boundaries of windows of back-to-back steps
            (at least 256 steps and 50 ms in all): median, p10 and p90 of
            the time per step over the windows -- one event pair per window,
            so the markers' own cost is spread over its steps;
  per-step  an event pair around each single step, warm (after a ~50 us GPU
            spin, so the host has queued the step before its first event)
            and cold (a 1 GiB buffer written before every step evicts the
            Infinity Cache): median, p10, p90 over at least 128 steps; both
            carry one marker pair per step, so they compare like with like;
  roofline  the dominant launch's algorithmic bytes over its time per launch
            from the windows (for the headline's layer form every step is
            exactly one attend launch).
"""
import argparse
import gc
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attention steps/sec + effective KV HBM GB/s (% of peak), batch 64"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
FLUSH_BYTES = 1 << 30           # written before each cold step; > 256 MB Infinity Cache
MIN_WINDOW_STEPS = 256          # windowed timing covers at least this many steps
MIN_WINDOW_MS = 50.0            # ... and at least this much GPU time
MIN_EVENT_STEPS = 128           # per-step event timing, warm and cold


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attend_bytes(wl, lens_post):
    """Algorithmic bytes of one attend over lens_post rows: each valid K and V row once, q in, out."""
    s = 4 if wl.dtype == "f32" else 2
    B = len(lens_post)
    rows = int(np.sum(lens_post, dtype=np.int64))
    return rows * wl.n_kv_heads * 64 * 2 * s + B * wl.n_q_heads * 64 * 4 * 2


def new_row_bytes(wl):
    """Bytes of the appended K and V rows of one step (one row per KV head)."""
    return wl.batch * wl.n_kv_heads * 64 * 2 * (4 if wl.dtype == "f32" else 2)


def dtype_label(wl):
    return "f32" if wl.dtype == "f32" else "bf16 K/V, f32 accumulate"


def pct(x, q):
    return round(float(np.percentile(x, q)), 3)


class Bench:
    def __init__(self, name, torch, gen, B, KVCache, to_device, form="layer"):
        wl = gen.WORKLOADS[name]
        self.wl, self.torch, self.B, self.form = wl, torch, B, form
        t0 = time.time()
        inp = gen.make_inputs(wl, canary=False)
        self.inp = inp
        nb = wl.batch
        self.lens0 = inp.lens.copy()
        self.self_cache = KVCache(nb, wl.n_kv_heads, inp.cap, wl.dtype, lens=inp.lens,
                                  k=to_device(inp.k_cache), v=to_device(inp.v_cache))
        self.kn = [to_device(x) for x in inp.k_new]
        self.vn = [to_device(x) for x in inp.v_new]
        self.q = [to_device(x) for x in inp.q_self]
        self.out = torch.empty_like(self.q[0])
        self.cross = None
        if wl.cross:
            self.cross = KVCache(nb, wl.n_kv_heads, gen.ENC_LEN, wl.dtype, static=True,
                                 lens=[0] * nb)
            self.cross.seed(to_device(inp.cross_k_tok), to_device(inp.cross_v_tok))
            self.qc = [to_device(x) for x in inp.q_cross]
            self.cout = torch.empty_like(self.qc[0])
        # free host copies of the big arrays
        inp.k_cache = inp.v_cache = inp.cross_k_tok = inp.cross_v_tok = None
        torch.cuda.synchronize()
        self.S = wl.steps
        # algorithmic bytes per step of the cycle, and of the step's dominant
        # launch (the one attend launch of a layer step; the cross launch of
        # the two-call forms of a Whisper step; the self launch otherwise)
        self.cross_bytes = attend_bytes(wl, np.full(nb, gen.ENC_LEN)) if wl.cross else 0
        self.step_bytes, self.launch_bytes = [], []
        for s in range(self.S):
            post = self.lens0 + s + 1
            self.step_bytes.append(gen.kv_bytes_per_step(wl, post))
            fused_self = attend_bytes(wl, post) + (new_row_bytes(wl) if form != "unfused" else 0)
            if wl.cross and form == "layer":
                self.launch_bytes.append(fused_self + self.cross_bytes)
            elif wl.cross:
                self.launch_bytes.append(self.cross_bytes)
            else:
                self.launch_bytes.append(fused_self)
        self._prep_raw()
        log(f"[{name}] inputs ready in {time.time() - t0:.1f}s: {wl.describe}")

    def _prep_raw(self):
        """Bind the C entry points and pointers once, so a step is 1-4 ctypes calls."""
        import ctypes
        from kv_cached_decode_kvdec_amd import binding as Bd
        lib = Bd.load()
        torch = self.torch
        self.lib = lib
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        vp = ctypes.c_void_p
        sc = self.self_cache
        self.h_self = sc.handle
        Hq = self.wl.n_q_heads
        self.ws_self = sc.workspace(Hq)
        if self.cross is not None:
            # one workspace serves the layer step (both parts) and the two calls
            self.ws_self = torch.empty(Bd.kvdec_workspace_bytes(sc.handle, Hq) +
                                       Bd.kvdec_workspace_bytes(self.cross.handle, Hq),
                                       dtype=torch.uint8, device="cuda")
        self.p_kn = [vp(t.data_ptr()) for t in self.kn]
        self.p_vn = [vp(t.data_ptr()) for t in self.vn]
        self.p_q = [vp(t.data_ptr()) for t in self.q]
        self.p_out = vp(self.out.data_ptr())
        self.p_ws = vp(self.ws_self.data_ptr())
        self.n_ws = self.ws_self.numel()
        self.lens0_c = (ctypes.c_int32 * len(self.lens0))(*self.lens0.tolist())
        if self.cross is not None:
            self.h_cross = self.cross.handle
            self.p_qc = [vp(t.data_ptr()) for t in self.qc]
            self.p_cout = vp(self.cout.data_ptr())

    def step(self, i, stream=None):
        lib, s, Hq = self.lib, i % self.S, self.wl.n_q_heads
        st = self.stream if stream is None else stream
        at = self.lens0_c if s == 0 else None     # cycle start: the starting positions
        if self.form == "layer" and self.cross is not None:
            rc = lib.kvdec_append_attend_cross(self.h_self, self.h_cross, at, self.p_kn[s],
                                               self.p_vn[s], self.p_q[s], self.p_qc[s], Hq, 0.125,
                                               0, 0, self.p_out, self.p_cout, self.p_ws, self.n_ws,
                                               st)
            assert rc == 0, lib.kvdec_last_error()
            return
        if self.form in ("layer", "two-calls"):
            if at is not None:
                rc = lib.kvdec_append_attend_at(self.h_self, at, self.p_kn[s], self.p_vn[s],
                                                self.p_q[s], Hq, 0.125, 0, self.p_out, self.p_ws,
                                                self.n_ws, st)
            else:
                rc = lib.kvdec_append_attend(self.h_self, self.p_kn[s], self.p_vn[s], self.p_q[s],
                                             Hq, 0.125, 0, self.p_out, self.p_ws, self.n_ws, st)
            assert rc == 0, lib.kvdec_last_error()
        else:
            if at is not None:
                rc = lib.kvdec_reset_lens(self.h_self, at, st)
                assert rc == 0, lib.kvdec_last_error()
            rc = lib.kvdec_append(self.h_self, self.p_kn[s], self.p_vn[s], st)
            assert rc == 0, lib.kvdec_last_error()
            rc = lib.kvdec_attend_self(self.h_self, self.p_q[s], Hq, 0.125, 0, self.p_out,
                                       self.p_ws, self.n_ws, st)
            assert rc == 0, lib.kvdec_last_error()
        if self.cross is not None:
            rc = lib.kvdec_attend_cross(self.h_cross, self.p_qc[s], Hq, 0.125, 0, self.p_cout,
                                        self.p_ws, self.n_ws, st)
            assert rc == 0, lib.kvdec_last_error()

    def _mean_bytes(self, seq, n):
        return sum(seq[i % self.S] for i in range(n)) / n

    def run(self, steps, warmup, cold=True, window_ms=MIN_WINDOW_MS):
        torch = self.torch
        Ev = lambda: torch.cuda.Event(enable_timing=True)
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        # timed region: K back-to-back steps, start index aligned to a cycle,
        # no events inside it
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        res = {"steps": steps, "ms_per_step": wall * 1e3 / steps, "steps_per_s": steps / wall,
               "bytes_per_step": self._mean_bytes(self.step_bytes, steps)}
        res["effective_gbps"] = res["bytes_per_step"] / (wall / steps) / 1e9
        res["pct_of_hbm_peak"] = 100.0 * res["effective_gbps"] / HBM_PEAK_GBPS

        # windows of W back-to-back steps (whole cycles), an event pair each
        W = self.S * max(1, math.ceil(16 / self.S))
        est_ms = max(res["ms_per_step"], 1e-4)
        n_win = max(16, math.ceil(MIN_WINDOW_STEPS / W), math.ceil(window_ms / (W * est_ms)))
        evs = [Ev() for _ in range(n_win + 1)]
        torch.cuda.synchronize()
        evs[0].record()
        for w in range(n_win):
            for i in range(W):
                self.step(i)
            evs[w + 1].record()
        torch.cuda.synchronize()
        win_us = np.array([1e3 * evs[w].elapsed_time(evs[w + 1]) / W for w in range(n_win)])
        res["window"] = {"steps_per_window": W, "windows": n_win,
                         "us_per_step_p10_p50_p90": [pct(win_us, 10), pct(win_us, 50),
                                                     pct(win_us, 90)]}
        med = float(np.median(win_us))
        res["window"]["steps_per_s_median"] = round(1e6 / med, 2)
        res["window"]["gbps_median"] = round(self._mean_bytes(self.step_bytes, W) / (med * 1e-6) / 1e9, 1)
        # dominant launch: bytes per launch over its time per launch (the
        # layer form of a Whisper step and the self-only steps are one attend
        # launch, plus a merge launch where a sequence spans several chunks)
        res["launch_bytes"] = self._mean_bytes(self.launch_bytes, W)

        # per-step event pairs: warm, then cold (flush before each).  Before
        # every warm step the GPU idles ~50 us (a spin kernel) so that the
        # host has the step's launches queued when its first event fires: the
        # pair then times the GPU, not the host's launch rate (the cold
        # steps get that from the flush).
        n_ev = self.S * max(1, math.ceil(MIN_EVENT_STEPS / self.S))
        a0, b0 = Ev(), Ev()
        a0.record()
        torch.cuda._sleep(1 << 20)
        b0.record()
        torch.cuda.synchronize()
        spin = int((1 << 20) * 50.0 / max(1e3 * a0.elapsed_time(b0), 1.0))

        def per_step(flush):
            a = [Ev() for _ in range(n_ev)]
            b = [Ev() for _ in range(n_ev)]
            torch.cuda.synchronize()
            for i in range(n_ev):
                if flush is not None:
                    flush.zero_()
                else:
                    torch.cuda._sleep(spin)
                a[i].record()
                self.step(i)
                b[i].record()
            torch.cuda.synchronize()
            return np.array([1e3 * a[i].elapsed_time(b[i]) for i in range(n_ev)])

        warm_us = per_step(None)
        res["per_step_warm_us_p10_p50_p90"] = [pct(warm_us, 10), pct(warm_us, 50), pct(warm_us, 90)]
        res["per_step_events"] = n_ev
        if cold:
            flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
            flush.zero_()
            cold_us = per_step(flush)
            del flush
            res["per_step_cold_us_p10_p50_p90"] = [pct(cold_us, 10), pct(cold_us, 50),
                                                   pct(cold_us, 90)]
            cb = self._mean_bytes(self.step_bytes, n_ev)
            res["cold_gbps_median"] = round(cb / (float(np.median(cold_us)) * 1e-6) / 1e9, 1)
            res["cold_pct_of_hbm_peak_median"] = round(100.0 * res["cold_gbps_median"] / HBM_PEAK_GBPS, 2)
        return res

    def _replay(self, on, horizon):
        for c in [self.self_cache] + ([self.cross] if self.cross is not None else []):
            c.set_replay_mode(-1 if on else 0)
            c.set_replay_horizon(horizon if on else 0)

    def run_graph(self, steps):
        """The same steps with whole workload cycles captured in one HIP graph
        (the caches in replay mode) and replayed: host launch work removed."""
        import ctypes
        torch = self.torch
        # every cycle restarts at the starting lengths, so each captured
        # launch sees the lengths it was captured at: a one-token horizon
        self._replay(True, 1)
        per_graph = self.S * max(1, -(-32 // self.S))
        gc.collect()          # no dead cycle holding device memory is freed mid-capture
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for s in range(per_graph):
                self.step(s, stream=st)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        reps = max(2, steps // per_graph)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        self._replay(False, 0)
        # leaving replay mode forgets the self cache's lengths: set them again
        self.self_cache.reset_lens(self.lens0)
        torch.cuda.synchronize()
        del g
        n = reps * per_graph
        step_bytes = reps * (per_graph // self.S) * sum(self.step_bytes)
        return {"graph_ms_per_step": wall * 1e3 / n, "graph_steps_per_s": n / wall,
                "graph_gbps": step_bytes / wall / 1e9,
                "graph_pct_of_hbm_peak": 100.0 * step_bytes / wall / 1e9 / HBM_PEAK_GBPS}

    def close(self):
        self.self_cache.close()
        if self.cross is not None:
            self.cross.close()


def run_layer_stack(name, torch, gen, B, KVCache, to_device, n_layers=4, tokens=32, reps=8):
    """A decoder of n_layers layers decoding `tokens` consecutive tokens from
    the workload's starting lengths: per token, each layer's attention step
    (kvdec_append_attend_cross for the Whisper shapes, kvdec_append_attend
    otherwise).  Timed eagerly (one call per layer and token from the host)
    and as one HIP graph holding all tokens x layers (replay mode), which is
    what removes per-launch host work.  Every layer has its own caches (the
    same seeded contents)."""
    import ctypes
    wl = gen.WORKLOADS[name]
    inp = gen.make_inputs(wl, canary=False, steps=tokens)
    nb, Hq = wl.batch, wl.n_q_heads
    lib = B.load()
    vp = ctypes.c_void_p
    layers = []
    for _ in range(n_layers):
        sc = KVCache(nb, wl.n_kv_heads, inp.cap, wl.dtype, lens=inp.lens,
                     k=to_device(inp.k_cache), v=to_device(inp.v_cache))
        cc = None
        if wl.cross:
            cc = KVCache(nb, wl.n_kv_heads, gen.ENC_LEN, wl.dtype, static=True, lens=[0] * nb)
            cc.seed(to_device(inp.cross_k_tok), to_device(inp.cross_v_tok))
        nws = B.kvdec_workspace_bytes(sc.handle, Hq) + (
            B.kvdec_workspace_bytes(cc.handle, Hq) if cc is not None else 0)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        layers.append((sc, cc, ws))
    kn = to_device(inp.k_new[0])
    vn = to_device(inp.v_new[0])
    q = to_device(inp.q_self[0])
    qc = to_device(inp.q_cross[0]) if wl.cross else None
    out = torch.empty_like(q)
    cout = torch.empty_like(q)
    lens0 = (ctypes.c_int32 * nb)(*inp.lens.tolist())
    torch.cuda.synchronize()

    def token(t, st):
        at = lens0 if t == 0 else None
        for sc, cc, ws in layers:
            if cc is not None:
                rc = lib.kvdec_append_attend_cross(sc.handle, cc.handle, at, vp(kn.data_ptr()),
                                                   vp(vn.data_ptr()), vp(q.data_ptr()),
                                                   vp(qc.data_ptr()), Hq, 0.125, 0, 0,
                                                   vp(out.data_ptr()), vp(cout.data_ptr()),
                                                   vp(ws.data_ptr()), ws.numel(), st)
            elif at is not None:
                rc = lib.kvdec_append_attend_at(sc.handle, at, vp(kn.data_ptr()), vp(vn.data_ptr()),
                                                vp(q.data_ptr()), Hq, 0.125, 0, vp(out.data_ptr()),
                                                vp(ws.data_ptr()), ws.numel(), st)
            else:
                rc = lib.kvdec_append_attend(sc.handle, vp(kn.data_ptr()), vp(vn.data_ptr()),
                                             vp(q.data_ptr()), Hq, 0.125, 0, vp(out.data_ptr()),
                                             vp(ws.data_ptr()), ws.numel(), st)
            assert rc == 0, lib.kvdec_last_error()

    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(2):
        for t in range(tokens):
            token(t, st)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        for t in range(tokens):
            token(t, st)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / (reps * tokens)
    for sc, cc, _ in layers:
        for c in (sc, cc):
            if c is not None:
                c.set_replay_mode(-1)
                c.set_replay_horizon(tokens)
    gc.collect()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gst = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for t in range(tokens):
            token(t, gst)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) * 1e6 / (reps * tokens)
    del g
    for sc, cc, _ in layers:
        sc.close()
        if cc is not None:
            cc.close()
    return {"layers": n_layers, "tokens": tokens, "eager_us_per_token": round(eager_us, 2),
            "graph_us_per_token": round(graph_us, 2),
            "graph_speedup": round(eager_us / graph_us, 3),
            "describe": f"{n_layers} layers of {wl.describe}, {tokens} consecutive tokens from the "
                        f"starting lengths, one layer-step call per layer and token"}


class VariantBench(Bench):
    """The same workload through one of the other cache forms:
      paged<P>    : paged pool with P-row pages (block table read per chunk),
                    through kvdec_paged_append_attend (the append fused into
                    the attend launch); lengths rolled back each cycle with
                    kvdec_paged_truncate;
      rope        : kvdec_append_rope (key and query rotated at the position)
                    instead of a plain append, then kvdec_attend_self;
      window<W>   : sliding-window ring of W rows (attends the last W tokens),
                    through kvdec_append_attend.
    Self-attention only (cross-attention is the same static cache as the
    plain form)."""

    def __init__(self, name, variant, torch, gen, B, KVCache, to_device):
        from kv_cached_decode_kvdec_amd.cache import PagedKVCache
        import ctypes
        wl = gen.WORKLOADS[name]
        self.wl, self.torch, self.variant = wl, torch, variant
        t0 = time.time()
        inp = gen.make_inputs(wl, canary=False)
        nb = wl.batch
        self.lens0 = inp.lens.copy()
        self.S = wl.steps
        self.cross = None
        self.kn = [to_device(x) for x in inp.k_new]
        self.vn = [to_device(x) for x in inp.v_new]
        self.q = [to_device(x) for x in inp.q_self]
        self.out = torch.empty_like(self.q[0])
        self.qrot = torch.empty_like(self.q[0])
        self.paged = None
        self.window = 0
        rows_attended = lambda post: post
        if variant.startswith("paged"):
            P = int(variant[5:])
            cap = inp.cap
            maxp = -(-cap // P)
            need = int(sum(-(-(int(l) + self.S) // P) for l in self.lens0))
            self.paged = PagedKVCache(nb, wl.n_kv_heads, P, num_pages=need + nb,
                                      max_pages_per_seq=maxp, dtype=wl.dtype)
            self.paged.load_contiguous(to_device(inp.k_cache), to_device(inp.v_cache), self.lens0)
            self.ws = self.paged._ws.setdefault(
                wl.n_q_heads, torch.empty(B.kvdec_paged_workspace_bytes(self.paged.handle,
                                                                          wl.n_q_heads),
                                          dtype=torch.uint8, device="cuda"))
        elif variant.startswith("window"):
            W = int(variant[6:])
            self.window = W
            Wp = gen.padded_rows(W)
            kc = np.zeros((nb, wl.n_kv_heads, Wp, 64), inp.k_cache.dtype)
            vc = np.zeros_like(kc)
            for b in range(nb):
                n = int(self.lens0[b])
                for t in range(max(0, n - W), n):
                    kc[b, :, t % W] = inp.k_cache[b, :, t]
                    vc[b, :, t % W] = inp.v_cache[b, :, t]
            self.self_cache = KVCache(nb, wl.n_kv_heads, W, wl.dtype, lens=self.lens0,
                                      k=to_device(kc), v=to_device(vc), window=W)
            rows_attended = lambda post: np.minimum(post, W)
        else:
            self.self_cache = KVCache(nb, wl.n_kv_heads, inp.cap, wl.dtype, lens=self.lens0,
                                      k=to_device(inp.k_cache), v=to_device(inp.v_cache))
        inp.k_cache = inp.v_cache = None
        torch.cuda.synchronize()
        self.launch_bytes, self.step_bytes = [], []
        for s in range(self.S):
            post = rows_attended(self.lens0 + s + 1)
            fused_store = new_row_bytes(wl) if variant.startswith(("window", "paged")) else 0
            self.launch_bytes.append(attend_bytes(wl, post) + fused_store)
            self.step_bytes.append(attend_bytes(wl, post) + 2 * new_row_bytes(wl))
        self.cross_bytes = 0
        lib = B.load()
        self.lib = lib
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        vp = ctypes.c_void_p
        self.p_kn = [vp(t.data_ptr()) for t in self.kn]
        self.p_vn = [vp(t.data_ptr()) for t in self.vn]
        self.p_q = [vp(t.data_ptr()) for t in self.q]
        self.p_out = vp(self.out.data_ptr())
        self.p_qrot = vp(self.qrot.data_ptr())
        self.lens0_c = (ctypes.c_int32 * len(self.lens0))(*self.lens0.tolist())
        if self.paged is None:
            self.h_self = self.self_cache.handle
            self.ws_self = self.self_cache.workspace(wl.n_q_heads)
            self.p_ws, self.n_ws = vp(self.ws_self.data_ptr()), self.ws_self.numel()
        else:
            self.p_ws, self.n_ws = vp(self.ws.data_ptr()), self.ws.numel()
        log(f"[{name}+{variant}] inputs ready in {time.time() - t0:.1f}s")

    def step(self, i, stream=None):
        lib, s, Hq = self.lib, i % self.S, self.wl.n_q_heads
        st = self.stream if stream is None else stream
        if self.paged is not None:
            h = self.paged.handle
            if s == 0:
                rc = lib.kvdec_paged_truncate(h, self.lens0_c, st)
                assert rc == 0, lib.kvdec_last_error()
            rc = lib.kvdec_paged_append_attend(h, self.p_kn[s], self.p_vn[s], self.p_q[s], Hq, 0.125,
                                               0, self.p_out, self.p_ws, self.n_ws, st)
            assert rc == 0, lib.kvdec_last_error()
            return
        if self.variant == "rope":
            if s == 0:
                rc = lib.kvdec_reset_lens(self.h_self, self.lens0_c, st)
                assert rc == 0, lib.kvdec_last_error()
            rc = lib.kvdec_append_rope(self.h_self, self.p_kn[s], self.p_vn[s],
                                       self.wl.rope_theta, self.p_q[s], self.p_qrot, Hq, st)
            assert rc == 0, lib.kvdec_last_error()
            rc = lib.kvdec_attend_self(self.h_self, self.p_qrot, Hq, 0.125, 0, self.p_out,
                                       self.p_ws, self.n_ws, st)
        elif s == 0:
            # ring (append fused into the attend launch), cycle start: the step
            # at the starting positions
            rc = lib.kvdec_append_attend_at(self.h_self, self.lens0_c, self.p_kn[s],
                                            self.p_vn[s], self.p_q[s], Hq, 0.125, 0,
                                            self.p_out, self.p_ws, self.n_ws, st)
        else:
            rc = lib.kvdec_append_attend(self.h_self, self.p_kn[s], self.p_vn[s], self.p_q[s],
                                         Hq, 0.125, 0, self.p_out, self.p_ws, self.n_ws, st)
        assert rc == 0, lib.kvdec_last_error()

    def close(self):
        if self.paged is not None:
            self.paged.close()
        else:
            self.self_cache.close()


def copy_bandwidth(torch, nbytes=2 << 30, reps=10):
    """Plain device-to-device copy (read + write), the achievable-bandwidth probe."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def read_probe(torch, nbytes=2 << 30, reps=4, blocks=8192):
    """The nontemporal 16-byte streaming read of libkvdec_probe.so over a
    buffer of known size (one launch reads it once): the calibration of
    FETCH_SIZE for the attend kernels' K/V load form."""
    import ctypes
    path = os.path.join(ROOT, "kv_cached_decode_kvdec_amd", "libkvdec_probe.so")
    lib = ctypes.CDLL(path)
    lib.kvdec_probe_stream_read.restype = ctypes.c_int
    lib.kvdec_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_void_p]
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    run = lambda: lib.kvdec_probe_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes,
                                              ctypes.c_void_p(sink.data_ptr()), blocks, st)
    assert run() == 0
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        assert run() == 0
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, sink
    return nbytes / (ms * 1e-3) / 1e9, nbytes


def cpu_baseline(name, target_s=12.0):
    """The f64 oracle, as it stands, timed on whole decode steps of the workload.

    Steps of the workload's cycle (append + self [+ cross] attention for every
    sequence) run back to back, single-threaded, until target_s has passed.
    """
    import oracle
    from kv_cached_decode_kvdec_amd import inputs as gen
    wl = gen.WORKLOADS[name]
    inp = gen.make_inputs(wl, canary=False)
    B = wl.batch
    if wl.cross:
        cK = np.zeros((B, wl.n_kv_heads, gen.padded_rows(gen.ENC_LEN), 64), inp.k_cache.dtype)
        cV = np.zeros_like(cK)
        oracle.seed(cK, inp.cross_k_tok)
        oracle.seed(cV, inp.cross_v_tok)
        clens = np.full(B, gen.ENC_LEN, np.int32)
    Kh, Vh = inp.k_cache, inp.v_cache
    lens = inp.lens.copy()
    t0 = time.perf_counter()
    steps = 0
    while True:
        s = steps % wl.steps
        if s == 0:
            lens = inp.lens.copy()
        lens = oracle.append(Kh, Vh, inp.k_new[s], inp.v_new[s], lens)
        oracle.attend(inp.q_self[s], Kh, Vh, lens)
        if wl.cross:
            oracle.attend(inp.q_cross[s], cK, cV, clens)
        steps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": steps / el, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} whole decode steps of {name} (all {B} sequences: append + self"
                      f"{' + cross' if wl.cross else ''} attention) through the f64 C oracle, "
                      f"1 thread, {el:.1f} s",
            "cpu_model": cpu, "machine": platform.machine()}


def _oracle_slice_worker(name, b0, b1, n_steps, barrier, results):
    """One worker of cpu_baseline_all_cores: the oracle on sequences [b0, b1)."""
    import oracle
    from kv_cached_decode_kvdec_amd import inputs as gen
    wl = gen.WORKLOADS[name]
    full = gen.draw_lens(np.random.default_rng(wl.seed), wl.lens, wl.batch)
    inp = gen.make_inputs(wl, batch=b1 - b0, lens=full[b0:b1], canary=False)
    nb = b1 - b0
    if wl.cross:
        cK = np.zeros((nb, wl.n_kv_heads, gen.padded_rows(gen.ENC_LEN), 64), inp.k_cache.dtype)
        cV = np.zeros_like(cK)
        oracle.seed(cK, inp.cross_k_tok)
        oracle.seed(cV, inp.cross_v_tok)
        clens = np.full(nb, gen.ENC_LEN, np.int32)
    Kh, Vh = inp.k_cache, inp.v_cache
    barrier.wait()
    t0 = time.perf_counter()
    for i in range(n_steps):
        s = i % wl.steps
        if s == 0:
            lens = inp.lens.copy()
        lens = oracle.append(Kh, Vh, inp.k_new[s], inp.v_new[s], lens)
        oracle.attend(inp.q_self[s], Kh, Vh, lens)
        if wl.cross:
            oracle.attend(inp.q_cross[s], cK, cV, clens)
    results.put(time.perf_counter() - t0)


def cpu_baseline_all_cores(name, single_rate, workers, target_s=10.0):
    """The same oracle on `workers` host cores: one process per core, each
    running whole decode steps for its share of the sequences (the oracle is
    per sequence, so the shares are independent).  Throughput = steps / the
    slowest worker's time; started together at a barrier."""
    import multiprocessing as mp
    from kv_cached_decode_kvdec_amd import inputs as gen
    wl = gen.WORKLOADS[name]
    workers = max(1, min(workers, wl.batch))
    n_steps = max(wl.steps, int(target_s * single_rate * workers * 0.8))
    bounds = np.linspace(0, wl.batch, workers + 1).astype(int)
    ctx = mp.get_context("spawn")            # fresh interpreters: no GPU state in the workers
    barrier, results = ctx.Barrier(workers), ctx.Queue()
    procs = [ctx.Process(target=_oracle_slice_worker,
                         args=(name, int(bounds[i]), int(bounds[i + 1]), n_steps, barrier, results))
             for i in range(workers)]
    for p in procs:
        p.start()
    times = []
    deadline = time.time() + 600
    while len(times) < workers:
        try:
            times.append(results.get(timeout=1.0))
        except Exception:                    # queue empty: check that no worker died
            dead = [p.exitcode for p in procs if p.exitcode not in (None, 0)]
            if dead or time.time() > deadline:
                for p in procs:
                    p.kill()
                raise RuntimeError(f"oracle worker failed (exit codes {dead}) or timed out")
    for p in procs:
        p.join()
    el = max(times)
    return {"value": n_steps / el, "unit": "steps/s", "cores": workers, "kind": "oracle",
            "sample": f"{n_steps} whole decode steps of {name}, the {wl.batch} sequences split "
                      f"over {workers} processes (one per core), f64 C oracle, {el:.1f} s"}


def measured_roofline(workload, form):
    """The committed rocprofv3 record of the workload's dominant kernel
    (profiles/roofline_<workload>.json: kernel name, its average duration
    from the kernel trace, HBM traffic per launch from FETCH_SIZE and
    WRITE_SIZE scaled by a nontemporal read of known size), or None when
    the kernel source or the step form has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"roofline_{workload}.json")
    src = os.path.join(ROOT, "kv_cached_decode_kvdec_amd", "csrc", "kvdec_kernels.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            cur = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != cur or rec.get("form") != form:
        return None
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="whisper-large")
    ap.add_argument("--per-workload", default="all",
                    help="comma list of extra workloads to report on stderr/JSON, or 'none'")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold (flushed) per-step timing")
    ap.add_argument("--window-ms", type=float, default=MIN_WINDOW_MS,
                    help="least GPU time the windowed timing covers per workload (profiled runs "
                         "use less)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="host cores for the all-cores oracle baseline (capped by the CPU count; "
                         "1 skips it)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay measurements")
    ap.add_argument("--layers", default="whisper-tiny,whisper-base",
                    help="workloads whose 4-layer decoder is timed eagerly and as one HIP graph, "
                         "or 'none'")
    ap.add_argument("--variants", default="qwen2-0.5b+paged16,gqa+paged16,qwen2-0.5b+rope,"
                                           "qwen2-0.5b+window1024",
                    help="workload+form pairs (paged<P>, rope, window<W>) to report, or 'none'")
    ap.add_argument("--form", default="layer", choices=["layer", "two-calls", "unfused"],
                    help="how a step calls the library (see the module docstring)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the plain copy kernel (for counter calibration)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only run the nontemporal 16-byte streaming read of a 2 GiB buffer "
                         "(the attend kernels' load form, for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the decode step is data-parallel over sequences "
              f"with no exchange between GPUs, and this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from kv_cached_decode_kvdec_amd import inputs as gen
    from kv_cached_decode_kvdec_amd import binding as Bd
    from kv_cached_decode_kvdec_amd.cache import KVCache, to_device
    Bd.load()    # fails loudly if libkvdec.so is missing
    torch.cuda.set_device(0)

    if args.copy_probe:
        gbps = copy_bandwidth(torch, reps=4)
        log(f"copy probe: {gbps:.0f} GB/s")
        return
    if args.read_probe:
        gbps, nbytes = read_probe(torch)
        log(f"read probe: {nbytes} bytes per launch, {gbps:.0f} GB/s")
        print(json.dumps({"read_probe_bytes_per_launch": nbytes, "read_probe_gbps": round(gbps, 1)}))
        return

    head = args.workload
    extra = [] if args.per_workload == "none" else (
        gen.ORDER if args.per_workload == "all" else args.per_workload.split(","))
    names = [head] + [n for n in extra if n != head]

    results = {}
    for name in names:
        wl = gen.WORKLOADS[name]
        bench = Bench(name, torch, gen, Bd, KVCache, to_device, form=args.form)
        if name == head:
            res = bench.run(args.steps, args.warmup, cold=not args.no_cold, window_ms=args.window_ms)
        else:
            # at least 256 steps, whatever --steps is
            K = max(args.steps, MIN_WINDOW_STEPS, wl.steps)
            res = bench.run(K, max(args.warmup, 16), cold=not args.no_cold, window_ms=args.window_ms)
        if not args.no_graph:
            res.update(bench.run_graph(max(args.steps, MIN_WINDOW_STEPS)))
        bench.close()
        del bench
        torch.cuda.empty_cache()
        results[name] = res
        w = res["window"]["us_per_step_p10_p50_p90"]
        log(f"[{name}] {res['steps_per_s']:.0f} steps/s ({res['steps']} steps), "
            f"{res['ms_per_step'] * 1e3:.1f} us/step, {res['effective_gbps']:.0f} GB/s "
            f"({res['pct_of_hbm_peak']:.1f}% of 8 TB/s); windows p10/p50/p90 {w[0]:.1f}/{w[1]:.1f}/"
            f"{w[2]:.1f} us ({res['window']['gbps_median']:.0f} GB/s median); per-step events warm "
            f"p50 {res['per_step_warm_us_p10_p50_p90'][1]:.1f} us, cold p50 "
            f"{res.get('per_step_cold_us_p10_p50_p90', [0, 0, 0])[1]:.1f} us; graph replay "
            f"{res.get('graph_ms_per_step', 0) * 1e3:.1f} us/step")

    layers = {}
    if not args.no_graph:
        for name in ([] if args.layers == "none" else args.layers.split(",")):
            layers[name] = run_layer_stack(name, torch, gen, Bd, KVCache, to_device)
            torch.cuda.empty_cache()
            r = layers[name]
            log(f"[{name} x{r['layers']} layers] eager {r['eager_us_per_token']:.1f} us/token, "
                f"one HIP graph {r['graph_us_per_token']:.1f} us/token ({r['graph_speedup']:.2f}x)")

    for spec in ([] if args.variants == "none" else args.variants.split(",")):
        name, variant = spec.split("+")
        vb = VariantBench(name, variant, torch, gen, Bd, KVCache, to_device)
        wl = gen.WORKLOADS[name]
        res = vb.run(max(args.steps, MIN_WINDOW_STEPS, wl.steps), max(args.warmup, 16), cold=False,
                     window_ms=args.window_ms)
        vb.close()
        del vb
        torch.cuda.empty_cache()
        results[spec] = res
        w = res["window"]["us_per_step_p10_p50_p90"]
        log(f"[{spec}] {res['steps_per_s']:.0f} steps/s, {res['ms_per_step'] * 1e3:.1f} us/step, "
            f"{res['effective_gbps']:.0f} GB/s ({res['pct_of_hbm_peak']:.1f}% of 8 TB/s); windows "
            f"p10/p50/p90 {w[0]:.1f}/{w[1]:.1f}/{w[2]:.1f} us")

    copy_gbps = copy_bandwidth(torch)
    log(f"plain copy kernel: {copy_gbps:.0f} GB/s (read + write)")

    h = results[head]
    wl = gen.WORKLOADS[head]
    prof = measured_roofline(head, args.form)
    launch_us = float(h["window"]["us_per_step_p10_p50_p90"][1])
    achieved = h["launch_bytes"] / (launch_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(h["steps_per_s"], 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label(wl),
        "data": "synthetic",
        "value_basis": "warm: exactly K back-to-back steps between device synchronisations; "
                       "the cold (Infinity Cache flushed) per-step figures are in "
                       "per_workload.*.per_step_cold_us_p10_p50_p90",
        "config": {"workload": head, "describe": wl.describe, "batch": wl.batch,
                   "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads, "head_dim": 64,
                   "kv_dtype": wl.dtype, "steps_per_cycle": wl.steps,
                   "cross_len": gen.ENC_LEN if wl.cross else 0, "step_form": args.form},
        "effective_kv_gbps": round(h["effective_gbps"], 1),
        "pct_of_hbm_peak": round(h["pct_of_hbm_peak"], 2),
        "graph_ms_per_step": round(h.get("graph_ms_per_step", 0.0), 5),
        "copy_kernel_gbps": round(copy_gbps, 1),
        # the step's effective rate against a plain device copy measured in the
        # same run (a copy reads and writes, so a read-mostly step can exceed it)
        "pct_of_copy_kernel": round(100.0 * h["effective_gbps"] / copy_gbps, 1) if copy_gbps > 0 else None,
        "roofline": {"bound": "hbm",
                     "kernel": prof["kernel"] if prof else "the step's attend launch",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": prof.get("traffic_bytes_per_launch") if prof else None,
                     "bytes_per_launch": int(h["launch_bytes"]),
                     "avg_launch_us": round(launch_us, 2),
                     "avg_launch_us_how": "HIP events around windows of back-to-back steps in "
                                          "bench.py (median window); one attend launch per step",
                     "profile_avg_launch_us": prof.get("avg_us") if prof else None,
                     "profile_frac": prof.get("frac") if prof else None,
                     "profile": prof.get("summary") if prof else None},
        "per_workload": {n: {k: (round(v, 4) if isinstance(v, float) else v)
                             for k, v in r.items()} for n, r in results.items()},
        "graph_layers": layers,
    }
    if not args.no_cpu_baseline:
        t0 = time.time()
        line["cpu_baseline"] = cpu_baseline(head)
        log(f"cpu baseline: {line['cpu_baseline']['value']:.3f} steps/s "
            f"({time.time() - t0:.0f}s incl. input generation)")
        if args.cpu_workers > 1:
            t0 = time.time()
            workers = min(args.cpu_workers, os.cpu_count() or 1)
            line["cpu_baseline_all_cores"] = cpu_baseline_all_cores(
                head, line["cpu_baseline"]["value"], workers)
            log(f"cpu baseline on {line['cpu_baseline_all_cores']['cores']} cores: "
                f"{line['cpu_baseline_all_cores']['value']:.2f} steps/s ({time.time() - t0:.0f}s)")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
