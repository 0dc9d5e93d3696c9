"""Benchmark of the single-token KV-cached decode step on one MI355X.

One step = one decode token for every sequence of one layer: append the new
K/V row and self-attention over the cached rows (kvdec_append_attend, one
launch; --unfused times kvdec_append then kvdec_attend_self instead) and, for
the Whisper-shaped workloads, cross-attention over the 1500 static encoder
rows (kvdec_attend_cross).  Workloads with several consecutive steps
(Whisper-large: 32, GQA: 8) cycle through them; the first step of each cycle
runs at the workload's starting positions (kvdec_append_attend_at, which
rewinds the lengths inside the same launch; --unfused rolls them back with
kvdec_reset_lens, one tiny kernel counted in the step).

Prints ONE JSON line on stdout (the headline workload, default
whisper-large: batch 64, 20 heads, bf16 K/V, self 448 -> 480 over 32 steps
plus cross-attention over 1500 rows) and a per-workload table on stderr.

Inputs are seeded synthetic tensors resident in HBM before the timed region
starts.  The timed region is K back-to-back steps bracketed by device
synchronisation, with nothing else on the stream.  A second pass over the
same K steps puts HIP events around every attend call: they give the attend
kernel's average launch duration (one kernel per attend call, plus the merge
launch when a sequence spans several chunks) and its achieved algorithmic
bandwidth; the fused call's bytes include the store of the new K/V row.
(Event markers cost the stream a few microseconds each, so the step rate is
not taken from the pass that carries them.)  "cold" figures write a 1 GiB
buffer before every step, which evicts the 256 MB Infinity Cache, and take
the step time as the difference between a pass of flush + step and a pass of
the flush alone.
"""
import argparse
import gc
import json
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attend_bytes(wl, lens_post):
    """Algorithmic bytes of one attend launch: each valid K and V row once, q in, out."""
    s = 4 if wl.dtype == "f32" else 2
    B = len(lens_post)
    rows = int(np.sum(lens_post, dtype=np.int64))
    return rows * wl.n_kv_heads * 64 * 2 * s + B * wl.n_q_heads * 64 * 4 * 2


def new_row_bytes(wl):
    """Bytes of the appended K and V rows of one step (one row per KV head)."""
    return wl.batch * wl.n_kv_heads * 64 * 2 * (4 if wl.dtype == "f32" else 2)


class Bench:
    def __init__(self, name, torch, gen, B, KVCache, to_device, fused=True):
        wl = gen.WORKLOADS[name]
        self.wl, self.torch, self.B, self.fused = wl, torch, B, fused
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
        # algorithmic bytes per step of the cycle
        self.self_bytes, self.step_bytes = [], []
        for s in range(self.S):
            post = self.lens0 + s + 1
            self.self_bytes.append(attend_bytes(wl, post) + (new_row_bytes(wl) if fused else 0))
            self.step_bytes.append(gen.kv_bytes_per_step(wl, post))
        self.cross_bytes = attend_bytes(wl, np.full(nb, gen.ENC_LEN)) if wl.cross else 0
        self._prep_raw()
        log(f"[{name}] inputs ready in {time.time() - t0:.1f}s: {wl.describe}")

    def _prep_raw(self):
        """Bind the C entry points and pointers once, so a step is 3-4 ctypes calls."""
        import ctypes
        from kv_cached_decode_kvdec_amd import binding as Bd
        lib = Bd.load()
        torch = self.torch
        self.lib = lib
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        vp = ctypes.c_void_p
        sc = self.self_cache
        self.h_self = sc.handle
        self.ws_self = sc.workspace(self.wl.n_q_heads)
        self.p_kn = [vp(t.data_ptr()) for t in self.kn]
        self.p_vn = [vp(t.data_ptr()) for t in self.vn]
        self.p_q = [vp(t.data_ptr()) for t in self.q]
        self.p_out = vp(self.out.data_ptr())
        self.p_ws = vp(self.ws_self.data_ptr())
        self.n_ws = self.ws_self.numel()
        self.lens0_c = (ctypes.c_int32 * len(self.lens0))(*self.lens0.tolist())
        if self.cross is not None:
            self.h_cross = self.cross.handle
            self.ws_cross = self.cross.workspace(self.wl.n_q_heads)
            self.p_qc = [vp(t.data_ptr()) for t in self.qc]
            self.p_cout = vp(self.cout.data_ptr())
            self.p_wsc = vp(self.ws_cross.data_ptr())
            self.n_wsc = self.ws_cross.numel()

    def step(self, i, events=None, stream=None):
        lib, s, Hq = self.lib, i % self.S, self.wl.n_q_heads
        st = self.stream if stream is None else stream
        if self.fused:
            if events is not None:
                events[0].record()
            if s == 0:      # cycle start: the step at the workload's starting positions
                rc = lib.kvdec_append_attend_at(self.h_self, self.lens0_c, self.p_kn[s],
                                                self.p_vn[s], self.p_q[s], Hq, 0.125, 0,
                                                self.p_out, self.p_ws, self.n_ws, st)
            else:
                rc = lib.kvdec_append_attend(self.h_self, self.p_kn[s], self.p_vn[s], self.p_q[s],
                                             Hq, 0.125, 0, self.p_out, self.p_ws, self.n_ws, st)
        else:
            if s == 0:
                rc = lib.kvdec_reset_lens(self.h_self, self.lens0_c, st)
                assert rc == 0, lib.kvdec_last_error()
            rc = lib.kvdec_append(self.h_self, self.p_kn[s], self.p_vn[s], st)
            assert rc == 0, lib.kvdec_last_error()
            if events is not None:
                events[0].record()
            rc = lib.kvdec_attend_self(self.h_self, self.p_q[s], Hq, 0.125, 0, self.p_out,
                                       self.p_ws, self.n_ws, st)
        assert rc == 0, lib.kvdec_last_error()
        if events is not None:
            events[1].record()
        if self.cross is not None:
            rc = lib.kvdec_attend_cross(self.h_cross, self.p_qc[s], Hq, 0.125, 0, self.p_cout,
                                        self.p_wsc, self.n_wsc, st)
            assert rc == 0, lib.kvdec_last_error()
            if events is not None:
                events[2].record()

    def run(self, steps, warmup, cold_steps=0):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        # timed region: K back-to-back steps, start index aligned to a cycle.
        # No events inside it: every event marker costs the stream a few
        # microseconds, which would be charged to the step.
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # the same K steps again, with HIP events around every attend call on
        # the stream the kernels run on: the attend kernel's launch duration
        n_ev = 3 if self.cross is not None else 2
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(steps):
            self.step(i, evs[i])
        torch.cuda.synchronize()
        wall_ev = time.perf_counter() - t1
        att_ms, att_bytes = [], []
        for i in range(steps):
            s = i % self.S
            att_ms.append(evs[i][0].elapsed_time(evs[i][1]))
            att_bytes.append(self.self_bytes[s])
            if self.cross is not None:
                att_ms.append(evs[i][1].elapsed_time(evs[i][2]))
                att_bytes.append(self.cross_bytes)
        step_bytes = sum(self.step_bytes[i % self.S] for i in range(steps))
        res = {
            "steps": steps,
            "ms_per_step": wall * 1e3 / steps,
            "steps_per_s": steps / wall,
            "ms_per_step_with_events": wall_ev * 1e3 / steps,
            "bytes_per_step": step_bytes / steps,
            "effective_gbps": step_bytes / wall / 1e9,
            "attend_launches": len(att_ms),
            "attend_avg_us": 1e3 * float(np.mean(att_ms)),
            # per call kind (with cross-attention the entries alternate self, cross)
            "self_attend_us_p10_p50_p90": [round(1e3 * float(x), 2) for x in np.percentile(
                att_ms[0::n_ev - 1], [10, 50, 90])],
            "attend_gbps": float(np.sum(att_bytes)) / (float(np.sum(att_ms)) * 1e-3) / 1e9,
            "attend_bytes_per_launch": float(np.mean(att_bytes)),
        }
        if self.cross is not None:
            res["cross_attend_us_p10_p50_p90"] = [round(1e3 * float(x), 2) for x in np.percentile(
                att_ms[1::2], [10, 50, 90])]
        res["pct_of_hbm_peak"] = 100.0 * res["effective_gbps"] / HBM_PEAK_GBPS
        res["attend_frac"] = res["attend_gbps"] / HBM_PEAK_GBPS
        if cold_steps:
            # cold: before every step, writing a 1 GiB buffer evicts the
            # 256 MB Infinity Cache.  The step time is the difference of two
            # marker-free passes, flush + step and flush alone; both passes
            # write back the same dirty lines in total, so the difference is
            # the steps' own time.
            flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
            flush.zero_()
            torch.cuda.synchronize()

            def timed(with_step):
                t = time.perf_counter()
                for i in range(cold_steps):
                    flush.zero_()
                    if with_step:
                        self.step(i)
                torch.cuda.synchronize()
                return time.perf_counter() - t

            timed(True)
            t_flush = min(timed(False), timed(False))
            t_both = min(timed(True), timed(True))
            cold_s = max(t_both - t_flush, 1e-9) / cold_steps
            cb = sum(self.step_bytes[i % self.S] for i in range(cold_steps)) / cold_steps
            res["cold_ms_per_step"] = cold_s * 1e3
            res["cold_gbps"] = cb / cold_s / 1e9
            res["cold_pct_of_hbm_peak"] = 100.0 * res["cold_gbps"] / HBM_PEAK_GBPS
            del flush
        return res

    def run_graph(self, steps):
        """The same steps with one workload cycle captured in a HIP graph (the
        caches in replay mode) and replayed: launch overhead removed."""
        import ctypes
        torch = self.torch
        caches = [self.self_cache] + ([self.cross] if self.cross is not None else [])
        for c in caches:
            c.set_replay_mode(-1)
            # every cycle restarts at the starting lengths, so each captured
            # launch sees the lengths it was captured at: a one-token horizon
            c.set_replay_horizon(1)
        # one graph holds whole cycles, at least 32 steps, so the graph launch
        # itself is amortised
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
        reps = max(1, steps // per_graph)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for c in caches:
            c.set_replay_mode(0)
            c.set_replay_horizon(0)
        n = reps * per_graph
        step_bytes = reps * (per_graph // self.S) * sum(self.step_bytes)
        return {"graph_ms_per_step": wall * 1e3 / n, "graph_steps_per_s": n / wall,
                "graph_gbps": step_bytes / wall / 1e9,
                "graph_pct_of_hbm_peak": 100.0 * step_bytes / wall / 1e9 / HBM_PEAK_GBPS}

    def close(self):
        self.self_cache.close()
        if self.cross is not None:
            self.cross.close()


def measured_traffic(workload):
    """HBM bytes per attend launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy of known size), or
    None when the kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    src = os.path.join(ROOT, "kv_cached_decode_kvdec_amd", "csrc", "kvdec_kernels.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            cur = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None, None
    if rec.get("kernel_source_sha256") != cur:
        return None, rec.get("kernel")
    return int(rec["traffic_bytes_per_launch"]), rec.get("kernel")


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
        self.self_bytes, self.step_bytes = [], []
        for s in range(self.S):
            post = rows_attended(self.lens0 + s + 1)
            fused_store = new_row_bytes(wl) if variant.startswith(("window", "paged")) else 0
            self.self_bytes.append(attend_bytes(wl, post) + fused_store)
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

    def step(self, i, events=None, stream=None):
        lib, s, Hq = self.lib, i % self.S, self.wl.n_q_heads
        st = self.stream if stream is None else stream
        if self.paged is not None:
            h = self.paged.handle
            if s == 0:
                rc = lib.kvdec_paged_truncate(h, self.lens0_c, st)
                assert rc == 0, lib.kvdec_last_error()
            if events is not None:
                events[0].record()
            rc = lib.kvdec_paged_append_attend(h, self.p_kn[s], self.p_vn[s], self.p_q[s], Hq, 0.125,
                                               0, self.p_out, self.p_ws, self.n_ws, st)
            assert rc == 0, lib.kvdec_last_error()
            if events is not None:
                events[1].record()
            return
        if s == 0 and self.variant == "rope":
            rc = lib.kvdec_reset_lens(self.h_self, self.lens0_c, st)
            assert rc == 0, lib.kvdec_last_error()
        if self.variant == "rope":
            rc = lib.kvdec_append_rope(self.h_self, self.p_kn[s], self.p_vn[s],
                                       self.wl.rope_theta, self.p_q[s], self.p_qrot, Hq, st)
            assert rc == 0, lib.kvdec_last_error()
            if events is not None:
                events[0].record()
            rc = lib.kvdec_attend_self(self.h_self, self.p_qrot, Hq, 0.125, 0, self.p_out,
                                       self.p_ws, self.n_ws, st)
        else:                 # ring: append fused into the attend launch
            if events is not None:
                events[0].record()
            if s == 0:        # cycle start at the starting positions
                rc = lib.kvdec_append_attend_at(self.h_self, self.lens0_c, self.p_kn[s],
                                                self.p_vn[s], self.p_q[s], Hq, 0.125, 0,
                                                self.p_out, self.p_ws, self.n_ws, st)
            else:
                rc = lib.kvdec_append_attend(self.h_self, self.p_kn[s], self.p_vn[s], self.p_q[s],
                                             Hq, 0.125, 0, self.p_out, self.p_ws, self.n_ws, st)
        assert rc == 0, lib.kvdec_last_error()
        if events is not None:
            events[1].record()

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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="whisper-large")
    ap.add_argument("--per-workload", default="all",
                    help="comma list of extra workloads to report on stderr/JSON, or 'none'")
    ap.add_argument("--cold-steps", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="host cores for the all-cores oracle baseline (capped by the CPU count; "
                         "1 skips it)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay measurement")
    ap.add_argument("--variants", default="qwen2-0.5b+paged16,gqa+paged16,qwen2-0.5b+rope,"
                                           "qwen2-0.5b+window1024",
                    help="workload+form pairs (paged<P>, rope, window<W>) to report, or 'none'")
    ap.add_argument("--unfused", action="store_true",
                    help="time kvdec_append + kvdec_attend_self instead of kvdec_append_attend")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the plain copy kernel (for counter calibration)")
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

    head = args.workload
    extra = [] if args.per_workload == "none" else (
        gen.ORDER if args.per_workload == "all" else args.per_workload.split(","))
    names = [head] + [n for n in extra if n != head]

    results = {}
    for name in names:
        wl = gen.WORKLOADS[name]
        bench = Bench(name, torch, gen, Bd, KVCache, to_device, fused=not args.unfused)
        K = args.steps
        if name == head:
            res = bench.run(K, args.warmup, cold_steps=args.cold_steps)
        else:
            res = bench.run(max(K // 2, wl.steps), max(args.warmup // 2, 4),
                            cold_steps=args.cold_steps)
        if not args.no_graph:
            res.update(bench.run_graph(max(K // 2, wl.steps)))
        bench.close()
        del bench
        torch.cuda.empty_cache()
        results[name] = res
        log(f"[{name}] {res['steps_per_s']:.0f} steps/s, {res['ms_per_step'] * 1e3:.1f} us/step, "
            f"{res['effective_gbps']:.0f} GB/s ({res['pct_of_hbm_peak']:.1f}% of 8 TB/s); "
            f"cold {res.get('cold_ms_per_step', 0) * 1e3:.1f} us/step "
            f"({res.get('cold_pct_of_hbm_peak', 0):.1f}%); attend kernel "
            f"{res['attend_avg_us']:.1f} us avg, {res['attend_gbps']:.0f} GB/s; graph replay "
            f"{res.get('graph_ms_per_step', 0) * 1e3:.1f} us/step "
            f"({res.get('graph_pct_of_hbm_peak', 0):.1f}%)")

    for spec in ([] if args.variants == "none" else args.variants.split(",")):
        name, variant = spec.split("+")
        vb = VariantBench(name, variant, torch, gen, Bd, KVCache, to_device)
        wl = gen.WORKLOADS[name]
        res = vb.run(max(args.steps // 2, wl.steps), max(args.warmup // 2, 4), cold_steps=0)
        vb.close()
        del vb
        torch.cuda.empty_cache()
        results[spec] = res
        log(f"[{spec}] {res['steps_per_s']:.0f} steps/s, {res['ms_per_step'] * 1e3:.1f} us/step, "
            f"{res['effective_gbps']:.0f} GB/s ({res['pct_of_hbm_peak']:.1f}% of 8 TB/s); attend "
            f"{res['attend_avg_us']:.1f} us avg, {res['attend_gbps']:.0f} GB/s")

    copy_gbps = copy_bandwidth(torch)
    log(f"plain copy kernel: {copy_gbps:.0f} GB/s (read + write)")

    h = results[head]
    wl = gen.WORKLOADS[head]
    traffic, kname = measured_traffic(head)
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
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": head, "describe": wl.describe, "batch": wl.batch,
                   "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads, "head_dim": 64,
                   "kv_dtype": wl.dtype, "steps_per_cycle": wl.steps,
                   "cross_len": gen.ENC_LEN if wl.cross else 0},
        "effective_kv_gbps": round(h["effective_gbps"], 1),
        "pct_of_hbm_peak": round(h["pct_of_hbm_peak"], 2),
        "cold_ms_per_step": round(h.get("cold_ms_per_step", 0.0), 5),
        "ms_per_step_with_events": round(h["ms_per_step_with_events"], 5),
        "graph_ms_per_step": round(h.get("graph_ms_per_step", 0.0), 5),
        "graph_steps_per_s": round(h.get("graph_steps_per_s", 0.0), 2),
        "cold_pct_of_hbm_peak": round(h.get("cold_pct_of_hbm_peak", 0.0), 2),
        "copy_kernel_gbps": round(copy_gbps, 1),
        # the step's effective rate against a plain device copy measured in the
        # same run (a copy reads and writes, so a read-mostly step can exceed it)
        "pct_of_copy_kernel": round(100.0 * h["effective_gbps"] / copy_gbps, 1) if copy_gbps > 0 else None,
        "roofline": {"bound": "hbm",
                     "kernel": kname or "attend kernel (one launch per attend call)",
                     "achieved": round(h["attend_gbps"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(h["attend_frac"], 4), "traffic": traffic,
                     "avg_launch_us": round(h["attend_avg_us"], 2),
                     "bytes_per_launch": int(h["attend_bytes_per_launch"])},
        "per_workload": {n: {k: (round(v, 4) if isinstance(v, float) else v)
                             for k, v in r.items()} for n, r in results.items()},
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
