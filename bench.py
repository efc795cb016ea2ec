#!/usr/bin/env python3
"""Throughput of the key-channel pruning hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  for every layer: think_score_select_compact (scores, kept channels and the
    thin key cache: one launch that reads K once where the cache fits the
    register files, else the score pass and the compaction)
  then for every decode step and every layer: think_decode_attn
Default workload: the 32-layer LLaMA-3-8B-like cache, 131072 tokens per
layer, 32 q / 8 kv heads, head_dim 128, window 64, keep 64 of 128 (bf16),
score+compact once then 128 decode steps.

Metric: algorithmic HBM bytes moved per second (GB/s), also as a fraction of
the 8 TB/s peak, and KV tokens per second.  Algorithmic bytes:
  score+compact, per layer : 2|K| + |K_thin| + |Q_w|   (two streaming reads of K)
  decode, per call          : |K_thin| + |V| + |q| + |out|
with |X| counted over valid tokens.  Inputs are resident in HBM before the
timed region.  The timed steps run back to back between two synchronisations
(wall clock); the per-path figures, the chunk pass's launch duration and the
graph replay come from passes after it.  Prints one JSON line.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import kvsynth  # noqa: E402

METRIC = "score+compact and pruned-K decode attn: HBM GB/s, % of peak, KV tokens/s"
PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama3-8b-128k", choices=sorted(kvsynth.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="approximate seconds of oracle work in the CPU baseline sample")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (hardware-counter scaling)")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the chunk-pass timing passes and the graph replay "
                         "(hardware-counter runs)")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="override the workload's decode steps (profiling runs only; "
                         "reported in config)")
    ap.add_argument("--also", default="mistral-7b-gqa-32k",
                    help="comma-separated workloads also measured in the same run, reported "
                         "under 'also' (empty: none)")
    ap.add_argument("--also-steps", type=int, default=200,
                    help="timed steps of each workload under --also")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the append, append+decode and prefill figures")
    ap.add_argument("--parity", action="store_true",
                    help="with --no-cpu-baseline: still check layer 0 against the oracle")
    ap.add_argument("--no-decode-shapes", action="store_true",
                    help="leave out the decode-alone figures of the general-path shapes")
    ap.add_argument("--decode-shape", action="append", default=[],
                    metavar="DTYPE,B,HQ,HKV,D,S,KEEP",
                    help="instead of the workload: time the decode alone (chunk pass + "
                         "combine) on this synthetic shape at full length, one JSON line per "
                         "shape; repeatable")
    return ap.parse_args()


def to_dev(a, torch, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


class Workload:
    """Device-resident inputs and outputs of every layer, plus pre-marshalled
    C-ABI arguments so the timed loop does no Python-side checking."""

    def __init__(self, cfg, torch, qdk, dev):
        self.cfg, self.torch, self.qdk = cfg, torch, qdk
        B, S, Hq, Hkv, D, keep = (cfg.batch, cfg.seq_capacity, cfg.n_q_heads, cfg.n_kv_heads,
                                  cfg.head_dim, cfg.keep)
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.layers = []
        t0 = time.time()
        host0 = None
        for l in range(cfg.layers):
            L = kvsynth.make_layer(cfg, l)
            if l == 0:
                host0 = L
            qd = np.stack([kvsynth.decode_q(cfg, l, s, L["channel_scale"])
                           for s in range(cfg.decode_steps)])
            ent = dict(k=to_dev(L["k_cache"], torch, dev), v=to_dev(L["v_cache"], torch, dev),
                       qo=to_dev(L["q_obs"], torch, dev), lens=to_dev(L["seq_lens"], torch, dev),
                       q=to_dev(qd, torch, dev))
            ent["scores"] = torch.empty(B, Hkv, D, dtype=torch.float32, device=dev)
            ent["idx"] = torch.empty(B, Hkv, keep, dtype=torch.int32, device=dev)
            ent["tie"] = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
            ent["thin"] = torch.empty(B, S, Hkv, keep, dtype=tdt, device=dev)
            self.layers.append(ent)
            if l == 0 or (l + 1) % 8 == 0:
                log(f"layer {l + 1}/{cfg.layers} resident ({time.time() - t0:.1f}s)")
            if l > 0:
                del L
        self.host0 = host0
        self.lens_host = host0["seq_lens"]
        # Cold protocol: a workload smaller than 1 GiB in all is replicated so
        # that successive calls rotate over copies and read from HBM rather
        # than from the 256 MB last-level cache.
        e = 2 if cfg.dtype == "bf16" else 4
        per_layer = B * S * Hkv * (2 * D + keep) * e
        self.ncopies = 1 if cfg.layers * per_layer >= (1 << 30) else -(-(1 << 30) // (cfg.layers * per_layer))
        self.sets = [self.layers]
        for _ in range(self.ncopies - 1):
            cp = []
            for ent in self.layers:
                c = {k: ent[k].clone() for k in ("k", "v", "qo", "lens", "q")}
                c["scores"] = torch.empty_like(ent["scores"])
                c["idx"] = torch.empty_like(ent["idx"])
                c["tie"] = torch.empty_like(ent["tie"])
                c["thin"] = torch.empty_like(ent["thin"])
                cp.append(c)
            self.sets.append(cp)
        if self.ncopies > 1:
            log(f"{self.ncopies} copies of the inputs rotate between calls (cold protocol)")
        self.sc_i = 0
        self.dc_i = 0
        self.out = torch.empty(B, Hq, D, dtype=tdt, device=dev)
        code = qdk.THINK_BF16 if cfg.dtype == "bf16" else qdk.THINK_F32
        self.dims = qdk.make_dims(B, Hq, Hkv, D, S, code)
        self.sel_dims = qdk.make_dims(B, Hkv, Hkv, D, 1, qdk.THINK_F32)
        self.ws_s = torch.zeros(max(qdk.think_score_compact_workspace_bytes(self.dims, keep), 16),
                                dtype=torch.uint8, device=dev)
        # 1: score, selection and compaction in one launch reading K once
        self.single_read = qdk.think_score_compact_single_read(self.dims, keep)
        self.ws_d = torch.zeros(max(qdk.think_decode_workspace_bytes(self.dims, keep), 16),
                                dtype=torch.uint8, device=dev)
        self.scale = ctypes.c_float(1.0 / np.sqrt(D))

    # ---- the path, called through the C ABI with pre-built arguments
    def score_compact(self, stream):
        from query_driven_kv_amd import _lib
        lib, P = _lib.lib, ctypes.c_void_p
        d, keep = ctypes.byref(self.dims), self.cfg.keep
        W = self.cfg.obs_window
        ws, wsn = P(self.ws_s.data_ptr()), self.ws_s.numel()
        layers = self.sets[self.sc_i % self.ncopies]
        self.sc_i += 1
        for e in layers:
            rc = lib.think_score_select_compact(
                d, P(e["k"].data_ptr()), P(e["lens"].data_ptr()), P(e["qo"].data_ptr()), W, keep,
                P(e["scores"].data_ptr()), P(e["idx"].data_ptr()), P(e["tie"].data_ptr()),
                P(e["thin"].data_ptr()), ws, wsn, stream)
            if rc:
                _lib.check("think_score_select_compact", rc)

    def prepare_decode(self):
        P = ctypes.c_void_p
        # dec_args[copy][step][layer]; successive calls take successive copies
        self.dec_args = []
        qstep = self.cfg.batch * self.cfg.n_q_heads * self.cfg.head_dim
        esz = self.out.element_size()
        for layers in self.sets:
            steps = []
            for s in range(self.cfg.decode_steps):
                row = []
                for e in layers:
                    row.append((P(e["q"].data_ptr() + s * qstep * esz), P(e["thin"].data_ptr()),
                                P(e["v"].data_ptr()), P(e["lens"].data_ptr()),
                                P(e["idx"].data_ptr())))
                steps.append(row)
            self.dec_args.append(steps)

    def decode_calls(self, steps=None):
        """The decode calls of one step, in order, rotating over the copies."""
        for s in range(self.cfg.decode_steps if steps is None else steps):
            for l in range(self.cfg.layers):
                c = self.dc_i % self.ncopies
                self.dc_i += 1
                yield self.dec_args[c][s][l]

    def decode_kernel_times(self, stream, torch, min_launches=64):
        """The chunk pass's launch duration, live, in split-phase form: one
        step's decode calls (repeated until at least `min_launches`) as chunk
        passes alone, back to back between two HIP events on the launch stream
        (mean microseconds per launch: the kernel plus the dispatch gap to the
        next); then the same calls with the merge between them and events
        around every chunk pass (10/50/90th percentiles; an event record on
        the stream adds a few microseconds to what it brackets).  Returns
        (mean, launches, percentiles)."""
        from query_driven_kv_amd import _lib
        lib, P = _lib.lib, ctypes.c_void_p
        d, keep = ctypes.byref(self.dims), self.cfg.keep
        out, ws, wsn = P(self.out.data_ptr()), P(self.ws_d.data_ptr()), self.ws_d.numel()
        per_step = self.cfg.decode_steps * self.cfg.layers
        passes = max(1, -(-min_launches // per_step))
        n = passes * per_step
        calls = [c for _ in range(passes) for c in self.decode_calls()]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for (q, thin, v, lens, idx) in calls:
            _lib.check("think_decode_attn_partial", lib.think_decode_attn_partial(
                d, q, thin, v, lens, idx, keep, self.scale, ws, wsn, stream))
        e1.record()
        torch.cuda.synchronize()
        mean_us = e0.elapsed_time(e1) * 1e3 / n
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        calls = [c for _ in range(passes) for c in self.decode_calls()]
        for k, (q, thin, v, lens, idx) in enumerate(calls):
            ev[k][0].record()
            _lib.check("think_decode_attn_partial", lib.think_decode_attn_partial(
                d, q, thin, v, lens, idx, keep, self.scale, ws, wsn, stream))
            ev[k][1].record()
            _lib.check("think_decode_attn_combine", lib.think_decode_attn_combine(
                d, lens, keep, out, ws, wsn, stream))
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
        return mean_us, n, [round(float(x), 2) for x in np.percentile(us, [10, 50, 90])]

    def path_ms(self, stream, torch, rounds):
        """Milliseconds per step of each path on its own: `rounds` steps' worth
        of score+compact calls back to back between two HIP events, then as
        many steps' decode calls (the copy rotation carries on)."""
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda.synchronize()
        e[0].record()
        for _ in range(rounds):
            self.score_compact(stream)
        e[1].record()
        for _ in range(rounds):
            self.decode(stream)
        e[2].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / rounds, e[1].elapsed_time(e[2]) / rounds

    def decode(self, stream, steps=None):
        from query_driven_kv_amd import _lib
        lib, P = _lib.lib, ctypes.c_void_p
        d, keep = ctypes.byref(self.dims), self.cfg.keep
        out, ws, wsn = P(self.out.data_ptr()), P(self.ws_d.data_ptr()), self.ws_d.numel()
        fn = lib.think_decode_attn
        for (q, thin, v, lens, idx) in self.decode_calls(steps):
            rc = fn(d, q, thin, v, lens, idx, keep, self.scale, out, ws, wsn, stream)
            if rc:
                _lib.check("think_decode_attn", rc)

    # ---- algorithmic bytes
    def bytes_model(self):
        cfg = self.cfg
        e = 2 if cfg.dtype == "bf16" else 4
        tok = int(self.lens_host.sum())
        K = tok * cfg.n_kv_heads * cfg.head_dim * e
        Kt = tok * cfg.n_kv_heads * cfg.keep * e
        Qw = cfg.batch * cfg.obs_window * cfg.n_q_heads * cfg.head_dim * e
        q = cfg.batch * cfg.n_q_heads * cfg.head_dim * e
        sc_layer = 2 * K + Kt + Qw
        dec_call = Kt + K + 2 * q          # |K_thin| + |V| + |q| + |out|  (|V| == |K|)
        return dict(tokens=tok, sc_layer=sc_layer, dec_call=dec_call,
                    sc_min_layer=K + Kt + Qw)


def append_time(cfg, torch, qdk, dev, calls=512):
    """Mean duration of one decode-time append (think_append_kv) of this
    workload's batch and head shape, over `calls` appends into fresh rows of a
    scratch cache (the bench's own caches are full and stay untouched).
    Returns (microseconds per call, bytes per call)."""
    from query_driven_kv_amd import _lib
    P = ctypes.c_void_p
    B, Hkv, D, keep = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.keep
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    S = calls + 1
    thin = torch.zeros(B, S, Hkv, keep, dtype=tdt, device=dev)
    v = torch.zeros(B, S, Hkv, D, dtype=tdt, device=dev)
    kn = torch.randn(B, Hkv, D, device=dev).to(tdt)
    vn = torch.randn(B, Hkv, D, device=dev).to(tdt)
    idx = torch.arange(keep, dtype=torch.int32, device=dev).repeat(B, Hkv, 1).contiguous()
    lens = torch.zeros(B, dtype=torch.int32, device=dev)
    dims = qdk.make_dims(B, cfg.n_q_heads, Hkv, D, S, tdt)
    sp = P(torch.cuda.current_stream().cuda_stream)
    args = (ctypes.byref(dims), P(kn.data_ptr()), P(vn.data_ptr()), P(lens.data_ptr()),
            P(idx.data_ptr()), keep, P(thin.data_ptr()), P(v.data_ptr()), sp)
    fn = _lib.lib.think_append_kv
    _lib.check("think_append_kv", fn(*args))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls - 1):
        fn(*args)
    e1.record()
    torch.cuda.synchronize()
    assert int(lens.min().item()) == calls, "append did not advance every sequence"
    e = thin.element_size()
    return e0.elapsed_time(e1) * 1e3 / (calls - 1), B * Hkv * (2 * D + keep + D) * e


def append_decode_time(wl, torch, qdk, calls=64):
    """Decode with the generated token's append, on layer 0 copied into caches
    with `calls` free rows past the workload's capacity: `calls` steps of
    think_append_kv + think_decode_attn, then the same steps again (lengths
    reset) through the fused think_append_decode_attn.  Returns microseconds
    per step for (separate, fused); both runs must leave the same caches."""
    from query_driven_kv_amd import _lib
    P = ctypes.c_void_p
    cfg, e = wl.cfg, wl.layers[0]
    B, S, Hq, Hkv, D, keep = (cfg.batch, cfg.seq_capacity, cfg.n_q_heads, cfg.n_kv_heads,
                              cfg.head_dim, cfg.keep)
    dev, tdt = e["v"].device, e["v"].dtype
    S2 = S + calls
    thin = torch.empty(B, S2, Hkv, keep, dtype=tdt, device=dev)
    v = torch.empty(B, S2, Hkv, D, dtype=tdt, device=dev)
    thin[:, :S].copy_(e["thin"])
    v[:, :S].copy_(e["v"])
    gen = torch.Generator(device="cpu").manual_seed(7)
    kn = torch.randn(calls, B, Hkv, D, generator=gen).to(tdt).to(dev)
    vn = torch.randn(calls, B, Hkv, D, generator=gen).to(tdt).to(dev)
    q = torch.randn(calls, B, Hq, D, generator=gen).to(tdt).to(dev)
    lens = e["lens"].clone()
    dims = qdk.make_dims(B, Hq, Hkv, D, S2, qdk.THINK_BF16 if cfg.dtype == "bf16" else qdk.THINK_F32)
    ws = torch.zeros(qdk.think_decode_workspace_bytes(dims, keep), dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, D, dtype=tdt, device=dev)
    sp = P(torch.cuda.current_stream().cuda_stream)
    lib, d = _lib.lib, ctypes.byref(dims)
    ptr = lambda t: P(t.data_ptr())
    rows = []
    times = []
    for fused in (False, True):
        lens.copy_(e["lens"])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(calls):
            if fused:
                _lib.check("think_append_decode_attn", lib.think_append_decode_attn(
                    d, ptr(q[i]), ptr(kn[i]), ptr(vn[i]), ptr(thin), ptr(v), ptr(lens),
                    ptr(e["idx"]), keep, wl.scale, ptr(out), ptr(ws), ws.numel(), sp))
            else:
                _lib.check("think_append_kv", lib.think_append_kv(
                    d, ptr(kn[i]), ptr(vn[i]), ptr(lens), ptr(e["idx"]), keep, ptr(thin), ptr(v),
                    sp))
                _lib.check("think_decode_attn", lib.think_decode_attn(
                    d, ptr(q[i]), ptr(thin), ptr(v), ptr(lens), ptr(e["idx"]), keep, wl.scale,
                    ptr(out), ptr(ws), ws.numel(), sp))
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / calls)
        rows.append((thin[:, S - 1:].clone(), v[:, S - 1:].clone(), lens.clone()))
    assert torch.equal(rows[0][2], e["lens"] + calls), "append did not advance every sequence"
    for a, b in zip(rows[0], rows[1]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)) if a.dtype != torch.int32 \
            else torch.equal(a, b), "fused and separate appends left different caches"
    return times[0], times[1]


def prefill_time(wl, torch, qdk, chunk=8192, reps=3):
    """Prefill-fused scoring on layer 0 of a batch-1 workload: the prompt's K/V
    rows (the resident caches serve as the rows a prefill would produce; with
    one sequence a range of cache rows is a contiguous chunk) are written
    into scratch caches chunk by chunk while their key sums are gathered, then
    the scores and selection come from the gathered sums and the key cache is
    compacted.  Returns microseconds for (the whole write, score+select from the
    sums, compaction) of one layer, each the mean of `reps` runs."""
    from query_driven_kv_amd import _lib
    P = ctypes.c_void_p
    cfg, e = wl.cfg, wl.layers[0]
    B, S, Hkv, D, keep, W = (cfg.batch, cfg.seq_capacity, cfg.n_kv_heads, cfg.head_dim, cfg.keep,
                             cfg.obs_window)
    kc, vc = torch.empty_like(e["k"]), torch.empty_like(e["v"])
    thin = torch.empty_like(e["thin"])
    idx, tie = torch.empty_like(e["idx"]), torch.empty_like(e["tie"])
    dims = wl.dims
    state = torch.zeros(qdk.think_k2_state_bytes(dims), dtype=torch.uint8, device=e["k"].device)
    sp = P(torch.cuda.current_stream().cuda_stream)
    lib = _lib.lib
    row = Hkv * D * e["k"].element_size()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    t_w, t_s, t_c = [], [], []
    for _ in range(reps + 1):
        state.zero_()
        ev[0].record()
        for t0 in range(0, S, chunk):
            n = min(chunk, S - t0)
            off = t0 * row
            _lib.check("think_prefill_write_kv", lib.think_prefill_write_kv(
                ctypes.byref(dims), P(e["k"].data_ptr() + off), P(e["v"].data_ptr() + off), t0, n,
                P(e["lens"].data_ptr()), P(kc.data_ptr()), P(vc.data_ptr()), P(state.data_ptr()),
                state.numel(), sp))
        ev[1].record()
        _lib.check("think_score_select_k2", lib.think_score_select_k2(
            ctypes.byref(dims), P(state.data_ptr()), state.numel(), P(e["qo"].data_ptr()), W, keep,
            None, P(idx.data_ptr()), P(tie.data_ptr()), sp))
        ev[2].record()
        _lib.check("think_compact_k", lib.think_compact_k(
            ctypes.byref(dims), P(kc.data_ptr()), P(e["lens"].data_ptr()), P(idx.data_ptr()), keep,
            P(thin.data_ptr()), sp))
        ev[3].record()
        torch.cuda.synchronize()
        t_w.append(ev[0].elapsed_time(ev[1]) * 1e3)
        t_s.append(ev[1].elapsed_time(ev[2]) * 1e3)
        t_c.append(ev[2].elapsed_time(ev[3]) * 1e3)
    assert torch.equal(idx, e["idx"]), "selection from the gathered sums differs from the cache path"
    return float(np.mean(t_w[1:])), float(np.mean(t_s[1:])), float(np.mean(t_c[1:]))


def probe_ceiling(torch, dev, read_bytes, write_bytes, launches=64):
    """The single-launch ceiling for a path's byte counts: back-to-back launches
    of think_probe_stream (one launch reads read_bytes and writes write_bytes
    with nothing else to do), each on a different window of a scratch buffer
    of at least 1 GiB, so that the reads come from HBM and not from the 256 MB
    last-level cache (as the workloads' own inputs rotate over copies).
    Returns microseconds per launch."""
    from query_driven_kv_amd import _lib
    P = ctypes.c_void_p
    r = (read_bytes + 255) // 256 * 256
    w = (write_bytes + 255) // 256 * 256
    nwin = min(4096, max(2, -(-(1 << 30) // max(r, 1))))
    src = torch.empty(max(r * nwin, 16), dtype=torch.uint8, device=dev)
    dst = torch.empty(max(w * nwin, 16), dtype=torch.uint8, device=dev)
    sp = P(torch.cuda.current_stream().cuda_stream)
    fn = _lib.lib.think_probe_stream
    args = [(P(src.data_ptr() + (k % nwin) * r), read_bytes, P(dst.data_ptr() + (k % nwin) * w),
             write_bytes, sp) for k in range(nwin)]
    for k in range(8):
        _lib.check("think_probe_stream", fn(*args[k % nwin]))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(launches):
        fn(*args[k % nwin])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    del src, dst
    return us


# decode-alone shapes reported in the default line: 32K tokens x 8 kv heads,
# fp32 D 128 keep 64 and bf16 D 256 keep 128 (general chunk pass), bf16 D 64
# keep 32 (matrix-core kernel, head_dim 64)
DECODE_SHAPES = ("f32,1,32,8,128,32768,64", "bf16,1,16,8,256,32768,128",
                 "bf16,1,32,8,64,32768,32")


def decode_shape_bench(spec, torch, dev, calls=200):
    """Decode alone on one synthetic shape "dtype,B,Hq,Hkv,D,S,keep" with every
    sequence at full length: mean time per think_decode_attn call (chunk pass
    + combine, back to back), the chunk pass's mean launch duration (64 chunk
    passes alone, back to back between two events), algorithmic GB/s and the
    single-launch ceiling for the call's bytes.  Inputs are N(0, 1) drawn on
    the device, in enough copies (rotated call to call) that the reads come
    from HBM."""
    from query_driven_kv_amd import _lib
    lib, P = _lib.lib, ctypes.c_void_p
    f = spec.split(",")
    dt = f[0]
    B, Hq, Hkv, D, S, keep = (int(x) for x in f[1:])
    if dt not in ("f32", "bf16"):
        raise SystemExit(f"--decode-shape: dtype must be f32 or bf16, got {dt!r}")
    tdt, code, e = (torch.float32, 0, 4) if dt == "f32" else (torch.bfloat16, 1, 2)
    per_copy = B * S * Hkv * (keep + D) * e
    ncopies = max(2, min(8, -(-(640 << 20) // per_copy)))
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260721)
    kt = [torch.randn(B, S, Hkv, keep, generator=gen, device=dev).to(tdt) for _ in range(ncopies)]
    v = [torch.randn(B, S, Hkv, D, generator=gen, device=dev).to(tdt) for _ in range(ncopies)]
    q = torch.randn(B, Hq, D, generator=gen, device=dev).to(tdt)
    idx = torch.sort(torch.rand(B * Hkv, D, generator=gen, device=dev).argsort(dim=1)[:, :keep],
                     dim=1)[0].to(torch.int32).reshape(B, Hkv, keep).contiguous()
    lens = torch.full((B,), S, dtype=torch.int32, device=dev)
    out = torch.empty(B, Hq, D, dtype=tdt, device=dev)
    dims = _lib.think_dims(B, Hq, Hkv, D, S, code)
    d = ctypes.byref(dims)
    wsn = lib.think_decode_workspace_bytes(d, keep)
    ws = torch.empty(wsn, dtype=torch.uint8, device=dev)
    sp = P(torch.cuda.current_stream().cuda_stream)
    scale = ctypes.c_float(1.0 / float(np.sqrt(D)))
    args = [(P(q.data_ptr()), P(kt[c].data_ptr()), P(v[c].data_ptr()), P(lens.data_ptr()),
             P(idx.data_ptr())) for c in range(ncopies)]

    def call(k):
        _lib.check("think_decode_attn", lib.think_decode_attn(
            d, *args[k % ncopies], keep, scale, P(out.data_ptr()), P(ws.data_ptr()), wsn, sp))

    for k in range(8):
        call(k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(calls):
        call(k)
    e1.record()
    torch.cuda.synchronize()
    us_call = e0.elapsed_time(e1) * 1e3 / calls
    nchunk = 64
    e0.record()
    for k in range(nchunk):
        _lib.check("think_decode_attn_partial", lib.think_decode_attn_partial(
            d, *args[k % ncopies], keep, scale, P(ws.data_ptr()), wsn, sp))
    e1.record()
    torch.cuda.synchronize()
    us_chunk = e0.elapsed_time(e1) * 1e3 / nchunk
    rd = B * S * Hkv * (keep + D) * e + B * Hq * D * e
    wr = B * Hq * D * e
    del kt, v
    torch.cuda.empty_cache()
    ceil_us = probe_ceiling(torch, dev, rd, wr)
    return {"decode_shape": {"dtype": dt, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                             "head_dim": D, "seq_len": S, "keep": keep},
            "us_per_call": round(us_call, 2), "chunk_pass_us": round(us_chunk, 2),
            "bytes_per_call": rd + wr, "GBps": round((rd + wr) / us_call / 1e3, 1),
            "ceiling_us": round(ceil_us, 2), "frac_of_ceiling": round(ceil_us / us_call, 3),
            "calls": calls, "input_copies": ncopies}


def decode_source_hash():
    """Hash of the chunk-pass kernel's code (its source and the shared header;
    comments and whitespace dropped), so only a change to that code retires
    the counter summary taken on it."""
    import hashlib, re
    h = hashlib.sha256()
    for f in ("decode_mfma.hip", "think_common.h"):
        with open(os.path.join(ROOT, "query_driven_kv_amd", "csrc", f)) as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per chunk-pass launch from the committed hardware-counter
    summary of this workload, if it was taken with the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_mfma_{workload}_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary for this workload"
    if rec.get("workload") != workload:
        return None, "counters taken on another workload"
    if rec.get("source_hash") != decode_source_hash():
        return None, "kernel changed since the counters were taken"
    return int(rec["hbm_bytes_per_launch"]), rec.get("command", "")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def oracle_sample(wl, budget_s, threads):
    """The oracle, untuned, at `threads` OpenMP threads on a bounded sample of
    the same workload: full score+select+compact of layer 0, then decode steps
    of layer 0 until the time budget is spent.  Same algorithmic byte
    accounting as the GPU.  Returns the figures and the oracle's outputs
    (scores, kept channels, near-tie flags, thin keys, step-0 decode rows)."""
    import oracle
    cfg, L = wl.cfg, wl.host0
    bm = wl.bytes_model()
    oracle.set_threads(threads)
    used = oracle.num_threads()
    t0 = time.perf_counter()
    s = oracle.score(L["k_cache"], L["seq_lens"], L["q_obs"])
    idx, tie = oracle.select(s, cfg.keep)
    thin = oracle.compact(L["k_cache"], L["seq_lens"], idx)
    t_sc = time.perf_counter() - t0
    scale = np.float32(1.0 / np.sqrt(cfg.head_dim))
    steps, t_dec, out0 = 0, 0.0, None
    while steps < cfg.decode_steps and (t_sc + t_dec < budget_s or steps == 0):
        q = kvsynth.decode_q(cfg, 0, steps, L["channel_scale"])
        t1 = time.perf_counter()
        o = oracle.decode(q, thin, L["v_cache"], L["seq_lens"], idx, scale)
        t_dec += time.perf_counter() - t1
        if steps == 0:
            out0 = o
        steps += 1
    total_bytes = bm["sc_layer"] + steps * bm["dec_call"]
    total_s = t_sc + t_dec
    fig = {"value": round(total_bytes / total_s / 1e9, 4), "unit": "GB/s", "cores": used,
           "seconds": round(total_s, 2),
           "sample": (f"layer 0 of {cfg.name}: score+select+compact once ({t_sc:.2f}s) and "
                      f"{steps} decode steps ({t_dec:.2f}s); fp64 C oracle, OpenMP over "
                      f"(batch, head) pairs, {used} threads"),
           "score_compact_GBps": round(bm["sc_layer"] / t_sc / 1e9, 4),
           "decode_GBps": round(steps * bm["dec_call"] / max(t_dec, 1e-9) / 1e9, 4)}
    return fig, dict(scores=s, idx=idx, tie=tie, thin=thin, out0=out0)


def cpu_baseline(wl, budget_s):
    """The oracle at all host threads (the reported figure) and at one thread,
    each on its own bounded sample; returns the record and the oracle outputs
    of the all-threads run."""
    nthreads = len(os.sched_getaffinity(0))
    fig, ref = oracle_sample(wl, budget_s, nthreads)
    one, _ = oracle_sample(wl, max(budget_s * 0.6, 1.0), 1)
    rec = {"value": fig["value"], "unit": "GB/s", "cores": fig["cores"], "kind": "oracle",
           "cpu": _cpu_model(), "sample": fig["sample"], "seconds": fig["seconds"],
           "score_compact_GBps": fig["score_compact_GBps"], "decode_GBps": fig["decode_GBps"],
           "single_thread": {k: one[k] for k in ("value", "cores", "seconds", "sample",
                                                  "score_compact_GBps", "decode_GBps")}}
    return rec, ref


def gpu_layer0(wl, torch):
    """Layer 0 of the workload through the GPU path once more (copy 0's
    inputs): scores, kept channels, near-tie flags, thin keys and the step-0
    decode rows, on the host."""
    from query_driven_kv_amd import _lib
    lib, P = _lib.lib, ctypes.c_void_p
    e = wl.layers[0]

    def to_host(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    d, keep = ctypes.byref(wl.dims), wl.cfg.keep
    sp = P(torch.cuda.current_stream().cuda_stream)
    _lib.check("think_score_select_compact", lib.think_score_select_compact(
        d, P(e["k"].data_ptr()), P(e["lens"].data_ptr()), P(e["qo"].data_ptr()),
        wl.cfg.obs_window, keep, P(e["scores"].data_ptr()), P(e["idx"].data_ptr()),
        P(e["tie"].data_ptr()), P(e["thin"].data_ptr()), P(wl.ws_s.data_ptr()), wl.ws_s.numel(),
        sp))
    st = lib.think_score_compact_status(d, wl.cfg.obs_window, keep, P(wl.ws_s.data_ptr()),
                                        wl.ws_s.numel(), sp)
    out = torch.empty_like(wl.out)
    _lib.check("think_decode_attn", lib.think_decode_attn(
        d, P(e["q"].data_ptr()), P(e["thin"].data_ptr()), P(e["v"].data_ptr()),
        P(e["lens"].data_ptr()), P(e["idx"].data_ptr()), keep, wl.scale, P(out.data_ptr()),
        P(wl.ws_d.data_ptr()), wl.ws_d.numel(), sp))
    torch.cuda.synchronize()
    return dict(scores=to_host(e["scores"]), idx=to_host(e["idx"]), tie=to_host(e["tie"]),
                thin=to_host(e["thin"]), out0=to_host(out), status=st)


def parity(wl, g, ref):
    """The GPU's layer-0 outputs against the oracle's on the same bytes: kept
    channels bit-exact outside reported near ties, thin keys bit-exact, decode
    rows within the dtype's bound, scores within 5e-6 relative."""
    cfg = wl.cfg
    lens = wl.lens_host
    rel_s = float((np.abs(g["scores"].astype(np.float64) - ref["scores"]) /
                   np.maximum(ref["scores"], 1e-30)).max())
    rows_diff = (g["idx"] != ref["idx"]).any(axis=-1)
    outside = int((rows_diff & (ref["tie"] == 0)).sum())
    thin_ref, out_ref = ref["thin"], ref["out0"]
    if rows_diff.any():
        # a near tie went the other way: the thin keys and the decode are
        # checked on the GPU's own channel choice
        import oracle
        L = wl.host0
        thin_ref = oracle.compact(L["k_cache"], lens, g["idx"])
        q = kvsynth.decode_q(cfg, 0, 0, L["channel_scale"])
        out_ref = oracle.decode(q, thin_ref, L["v_cache"], lens, g["idx"],
                                np.float32(1.0 / np.sqrt(cfg.head_dim)))
    thin_ok = all(np.array_equal(g["thin"][b, :n].view(np.uint8), thin_ref[b, :n].view(np.uint8))
                  for b, n in enumerate(lens))
    of = kvsynth.as_float(g["out0"]).astype(np.float64)
    den = np.maximum(np.abs(out_ref).max(axis=-1), 1e-300)
    row_err = float((np.abs(of - out_ref).max(axis=-1) / den).max())
    tol = 1e-5 if cfg.dtype == "f32" else 2e-2
    rec = {"workload": cfg.name, "layer": 0, "decode_step": 0,
           "scores_max_rel_err": float(f"{rel_s:.3e}"), "scores_tol": 5e-6,
           "idx_bit_exact": bool(not rows_diff.any()),
           "idx_rows_differing_outside_near_ties": outside,
           "near_ties": int(ref["tie"].sum()),
           "k_thin_bit_exact": bool(thin_ok),
           "decode_row_err": float(f"{row_err:.3e}"), "decode_tol": tol,
           "single_read_status": int(g["status"])}
    rec["pass"] = bool(rel_s <= 5e-6 and outside == 0 and thin_ok and row_err <= tol
                       and g["status"] == 0)
    return rec


def graph_step_ms(wl, torch, rounds=30):
    """The workload's step with no host launch gaps: one step per input copy
    (each advancing the copy rotation as the eager loop does) captured in one
    HIP graph, replayed `rounds` times back to back; milliseconds per step."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    sp = ctypes.c_void_p(s.cuda_stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(wl.ncopies):
                wl.score_compact(sp)
                wl.decode(sp)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (rounds * wl.ncopies)
    del g
    return ms


def measure(cfg, args, torch, qdk, dev, steps, warmup, extras):
    """Time `steps` whole steps of workload `cfg` (after `warmup`), then the
    chunk-pass launches alone; with `extras`, the append, append+decode and
    prefill figures too.  Returns (workload, record)."""
    wl = Workload(cfg, torch, qdk, dev)
    wl.prepare_decode()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    bm = wl.bytes_model()
    n_dec = cfg.decode_steps * cfg.layers

    for _ in range(max(warmup, 1 if wl.ncopies > 1 else 0)):
        for _ in range(wl.ncopies):              # every copy's thin cache is filled
            wl.score_compact(sp)
        wl.decode(sp)
    torch.cuda.synchronize()
    log(f"{cfg.name}: warmup done")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        wl.score_compact(sp)
        wl.decode(sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"{cfg.name}: timed {steps} steps: {wall:.3f}s wall")
    # each path alone, after the timed region: `steps` rounds of one path's
    # calls back to back between two events (events inside the timed loop
    # would each add a few microseconds of stream time to a small step)
    sc_ms, dec_ms = wl.path_ms(sp, torch, steps)
    log(f"{cfg.name}: per path: score+compact {sc_ms:.3f} ms, decode {dec_ms:.3f} ms per step")

    ms_per_step = wall / steps * 1e3
    # small steps: the same step replayed from a graph, without host launch gaps
    graph_ms = (graph_step_ms(wl, torch) if ms_per_step < 5.0 and not args.no_kernel_timing
                else None)
    if graph_ms is not None:
        log(f"{cfg.name}: graph-replayed step {graph_ms * 1e3:.1f} us")
    sc_moved = bm["sc_min_layer"] if wl.single_read else bm["sc_layer"]
    step_bytes = cfg.layers * sc_moved + n_dec * bm["dec_call"]
    step_bytes_eff = cfg.layers * bm["sc_layer"] + n_dec * bm["dec_call"]
    value = step_bytes / (ms_per_step / 1e3) / 1e9
    tok = bm["tokens"]
    kv_tok_s = (tok * cfg.layers * (1 + cfg.decode_steps)) / (ms_per_step / 1e3)
    sc_gbs = cfg.layers * sc_moved / (sc_ms / 1e3) / 1e9
    sc_eff = cfg.layers * bm["sc_layer"] / (sc_ms / 1e3) / 1e9
    dec_gbs = n_dec * bm["dec_call"] / (dec_ms / 1e3) / 1e9
    dec_call_us = dec_ms * 1e3 / n_dec
    near = int(sum(int(e["tie"].sum().item()) for e in wl.layers))
    # the dominant kernel's own launch duration, live, with HIP events (a
    # separate pass after the timed region, so the events do not perturb it)
    if args.no_kernel_timing:
        part_us, n_part, part_pct = float("nan"), 0, None
    else:
        part_us, n_part, part_pct = wl.decode_kernel_times(sp, torch)
        log(f"{cfg.name}: chunk-pass kernel: {part_us:.2f} us mean over {n_part} launches")
    achieved = bm["dec_call"] / (part_us * 1e-6) / 1e9 if n_part else None
    # single-launch ceilings for the same byte counts (stream-probe launches)
    e = 2 if cfg.dtype == "bf16" else 4
    K = tok * cfg.n_kv_heads * cfg.head_dim * e
    Kt = tok * cfg.n_kv_heads * cfg.keep * e
    Qw = cfg.batch * cfg.obs_window * cfg.n_q_heads * cfg.head_dim * e
    dec_ceil = probe_ceiling(torch, dev, bm["dec_call"], 0)
    sc_read = (K if wl.single_read else 2 * K) + Qw
    sc_ceil = probe_ceiling(torch, dev, sc_read, Kt)
    log(f"{cfg.name}: single-launch ceilings: decode bytes {dec_ceil:.2f} us, score+compact "
        f"bytes {sc_ceil:.2f} us")
    rec = {
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 4),
            "GBps": round(step_bytes / (graph_ms / 1e3) / 1e9, 2),
            "pct_of_peak": round(100 * step_bytes / (graph_ms / 1e3) / 1e9 / PEAK_GBS, 2),
            "GBps_effective": round(step_bytes_eff / (graph_ms / 1e3) / 1e9, 2),
            "note": "the same step's calls, one step per input copy, captured in one HIP graph "
                    "and replayed back to back (no host launch gaps); value and ms_per_step "
                    "are the eager loop's"},
        "ms_per_step": round(ms_per_step, 4),
        "GBps": round(value, 2),
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "GBps_effective": round(step_bytes_eff / (ms_per_step / 1e3) / 1e9, 2),
        "bytes_per_step": step_bytes,
        "kv_tokens_per_s": float(f"{kv_tok_s:.4g}"),
        "paths": {
            "score_compact": {"ms_per_step": round(sc_ms, 4),
                              "us_per_layer": round(sc_ms * 1e3 / cfg.layers, 2),
                              "GBps": round(sc_gbs, 1),
                              "pct_of_peak": round(100 * sc_gbs / PEAK_GBS, 2),
                              "bytes_moved_per_layer": sc_moved,
                              "GBps_effective": round(sc_eff, 1),
                              "pct_of_peak_effective": round(100 * sc_eff / PEAK_GBS, 2),
                              "two_pass_bytes_per_layer": bm["sc_layer"],
                              "kv_tokens_per_s": float(f"{tok * cfg.layers / (sc_ms / 1e3):.4g}"),
                              "path": ("single read: one launch holds K on chip"
                                       if wl.single_read else "two passes over K")},
            "decode": {"ms_per_step": round(dec_ms, 4), "GBps": round(dec_gbs, 1),
                       "pct_of_peak": round(100 * dec_gbs / PEAK_GBS, 2),
                       "us_per_call": round(dec_call_us, 2),
                       "kv_tokens_per_s": float(f"{tok * n_dec / (dec_ms / 1e3):.4g}"),
                       "bytes_per_call": bm["dec_call"]},
        },
        "roofline": {"kernel": "k_decode_mfma (think_decode_attn chunk pass)",
                     "bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
                     "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4) if achieved else None,
                     "algorithmic_bytes_per_launch": bm["dec_call"],
                     "launch_us": round(part_us, 2) if n_part else None,
                     "event_pair_launch_us_p10_p50_p90": part_pct,
                     "timing": (f"{n_part} chunk-pass launches (one step's decode calls, "
                                f"repeated to at least 64) back to back between two HIP events "
                                f"on the launch stream, after the timed steps; the percentiles "
                                f"are of the same launches timed one by one between the merges, "
                                f"an event pair around each")},
        "near_ties": near,
        "input_copies": wl.ncopies,
        "ceiling": {
            "probe": ("think_probe_stream: one launch that only reads (and writes) the path's "
                      "bytes, 2048 workgroups x 512 threads, back-to-back launches on rotating "
                      "windows so reads come from HBM"),
            "decode": {"read_bytes": bm["dec_call"], "us_per_launch": round(dec_ceil, 2),
                       "GBps": round(bm["dec_call"] / (dec_ceil * 1e-6) / 1e9, 1),
                       "call_frac_of_ceiling": round(dec_ceil / dec_call_us, 4),
                       "chunk_pass_frac_of_ceiling":
                           round(dec_ceil / part_us, 4) if n_part else None},
            "score_compact": {"read_bytes": sc_read, "write_bytes": Kt,
                              "us_per_launch": round(sc_ceil, 2),
                              "GBps": round((sc_read + Kt) / (sc_ceil * 1e-6) / 1e9, 1),
                              "frac_of_ceiling": round(sc_ceil / (sc_ms * 1e3 / cfg.layers), 4)},
        },
    }
    if extras:
        app_us, app_bytes = append_time(cfg, torch, qdk, dev)
        log(f"decode-time append: {app_us:.2f} us per call")
        sep_us, fus_us = append_decode_time(wl, torch, qdk)
        log(f"append+decode on layer 0: separate {sep_us:.2f} us, fused {fus_us:.2f} us per step")
        rec["paths"]["append"] = {"us_per_call": round(app_us, 2), "bytes_per_call": app_bytes,
                                  "note": "think_append_kv, timed apart from the step (the "
                                          "workload's caches are full)"}
        rec["paths"]["append_decode"] = {
            "separate_us_per_step": round(sep_us, 2), "fused_us_per_step": round(fus_us, 2),
            "note": "layer 0 in caches with 64 free rows: 64 steps of think_append_kv + "
                    "think_decode_attn, then of think_append_decode_attn from the same lengths"}
        pre = None
        if cfg.batch == 1:
            pw_us, ps_us, pc_us = prefill_time(wl, torch, qdk)
            e = 2 if cfg.dtype == "bf16" else 4
            K = tok * cfg.n_kv_heads * cfg.head_dim * e
            Kt = tok * cfg.n_kv_heads * cfg.keep * e
            Qw = cfg.obs_window * cfg.n_q_heads * cfg.head_dim * e
            pre = {"write_us_per_layer": round(pw_us, 1),
                   "write_GBps": round(4 * K / (pw_us * 1e-6) / 1e9, 1),
                   "score_select_from_sums_us": round(ps_us, 2),
                   "compact_us": round(pc_us, 1),
                   "prune_after_prefill_GBps": round((K + Kt + Qw) / ((ps_us + pc_us) * 1e-6) / 1e9,
                                                     1),
                   "prune_after_prefill_pct_of_peak":
                       round(100 * (K + Kt + Qw) / ((ps_us + pc_us) * 1e-6) / 1e9 / PEAK_GBS, 2),
                   "note": "layer 0: prompt written in 8192-row chunks (reads and writes K and V: "
                           "4|K| bytes) gathering the key sums; then scores+selection from the "
                           "sums and compaction, |K| + |K_thin| + |Q_w| bytes (one read of K)"}
            log(f"prefill-fused scoring: write {pw_us:.1f} us, score from sums {ps_us:.2f} us, "
                f"compact {pc_us:.1f} us per layer")
        rec["paths"]["prefill_fused_scoring"] = pre
    return wl, rec


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this path runs on a single MI355X and has no "
              f"multi-GPU mode (asked for --gpus {args.gpus}, WORLD_SIZE={world}).",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import query_driven_kv_amd as qdk

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.decode_shape:
        for spec in args.decode_shape:
            log(f"decode shape {spec}")
            print(json.dumps(decode_shape_bench(spec, torch, dev)), flush=True)
        return
    cfg = kvsynth.CONFIGS[args.workload]
    if args.decode_steps > 0:
        import dataclasses
        cfg = dataclasses.replace(cfg, decode_steps=args.decode_steps)
    log(f"workload {cfg.name}: {cfg.layers} layers, B={cfg.batch}, S={cfg.seq_capacity}, "
        f"Hq={cfg.n_q_heads}, Hkv={cfg.n_kv_heads}, D={cfg.head_dim}, keep={cfg.keep}, "
        f"{cfg.decode_steps} decode steps")
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calibrate_copy_mib} MiB done")
        del src, dst

    wl, rec = measure(cfg, args, torch, qdk, dev, args.steps, args.warmup,
                      extras=not args.no_extras)
    traffic, traffic_src = committed_traffic(cfg.name)
    rec["roofline"]["traffic"] = traffic
    rec["roofline"]["traffic_source"] = traffic_src
    result = {
        "metric": METRIC,
        "value": rec["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rec["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded log-normal channel scales, x8 outliers, rank-32 keys + noise)",
        "config": {"workload": cfg.name, "layers": cfg.layers, "batch": cfg.batch,
                   "seq_len": cfg.seq_capacity, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "obs_window": cfg.obs_window, "keep": cfg.keep,
                   "decode_steps": cfg.decode_steps,
                   "valid_tokens_per_layer": int(wl.lens_host.sum())},
        "pct_of_peak": rec["pct_of_peak"],
        "value_note": ("HBM bytes the path as run moves per step / wall time; "
                       "value_effective counts score+compact as two passes over K"),
        "value_effective": rec["GBps_effective"],
        "kv_tokens_per_s": rec["kv_tokens_per_s"],
        "paths": rec["paths"],
        "graph_replay": rec["graph_replay"],
        "roofline": rec["roofline"],
        "ceiling": rec["ceiling"],
        "near_ties": rec["near_ties"],
        "input_copies": rec["input_copies"],
    }
    g0 = gpu_layer0(wl, torch)
    ref = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, all host threads, then one thread) ...")
        result["cpu_baseline"], ref = cpu_baseline(wl, args.cpu_budget_s)
    elif args.parity:
        _, ref = oracle_sample(wl, 0.0, len(os.sched_getaffinity(0)))
    if ref is not None:
        result["parity"] = parity(wl, g0, ref)
        log(f"parity on layer 0 of {cfg.name}: {result['parity']}")
    # the other workload the throughput target names, measured in the same run
    also = [w for w in args.also.split(",") if w and w != cfg.name]
    if also:
        del wl
        torch.cuda.empty_cache()
        result["also"] = {}
        for name in also:
            c2 = kvsynth.CONFIGS[name]
            wl2, r2 = measure(c2, args, torch, qdk, dev, args.also_steps, 3, extras=False)
            r2["roofline"]["traffic"], r2["roofline"]["traffic_source"] = committed_traffic(name)
            g2 = gpu_layer0(wl2, torch)
            if not args.no_cpu_baseline or args.parity:
                _, ref2 = oracle_sample(wl2, 0.0, len(os.sched_getaffinity(0)))
                r2["parity"] = parity(wl2, g2, ref2)
                log(f"parity on layer 0 of {name}: {r2['parity']}")
            r2["config"] = {"workload": c2.name, "layers": c2.layers, "batch": c2.batch,
                            "seq_len": c2.seq_capacity, "n_q_heads": c2.n_q_heads,
                            "n_kv_heads": c2.n_kv_heads, "head_dim": c2.head_dim,
                            "obs_window": c2.obs_window, "keep": c2.keep,
                            "decode_steps": c2.decode_steps, "steps": args.also_steps}
            result["also"][name] = r2
            del wl2
            torch.cuda.empty_cache()
    # decode alone on 32K shapes that take the general chunk pass (fp32, bf16
    # head_dim 256) or the matrix-core kernel's head_dim-64 instance
    if not args.no_decode_shapes:
        if "wl" in locals():
            del wl
        torch.cuda.empty_cache()
        result["decode_shapes"] = []
        for spec in DECODE_SHAPES:
            log(f"decode shape {spec}")
            result["decode_shapes"].append(decode_shape_bench(spec, torch, dev))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
