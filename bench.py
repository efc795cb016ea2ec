#!/usr/bin/env python3
"""Throughput of the key-channel pruning hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  for every layer: think_score_select (scores + kept channels) -> think_compact_k
  then for every decode step and every layer: think_decode_attn
Default workload: the 32-layer LLaMA-3-8B-like cache, 131072 tokens per
layer, 32 q / 8 kv heads, head_dim 128, window 64, keep 64 of 128 (bf16),
score+compact once then 128 decode steps.

Metric: algorithmic HBM bytes moved per second (GB/s), also as a fraction of
the 8 TB/s peak, and KV tokens per second.  Algorithmic bytes:
  score+compact, per layer : 2|K| + |K_thin| + |Q_w|   (two streaming reads of K)
  decode, per call          : |K_thin| + |V| + |q| + |out|
with |X| counted over valid tokens.  Inputs are resident in HBM before the
timed region.  Prints one JSON line.
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
                    help="skip the per-launch event pass (hardware-counter runs)")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="override the workload's decode steps (profiling runs only; "
                         "reported in config)")
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
        """One step's decode calls (repeated until at least `min_launches`) in
        split-phase form, with HIP events on the launch stream around every
        chunk-pass launch: the chunk pass's mean launch duration in
        microseconds, the launch count and the 10/50/90th percentiles."""
        from query_driven_kv_amd import _lib
        lib, P = _lib.lib, ctypes.c_void_p
        d, keep = ctypes.byref(self.dims), self.cfg.keep
        out, ws, wsn = P(self.out.data_ptr()), P(self.ws_d.data_ptr()), self.ws_d.numel()
        per_step = self.cfg.decode_steps * self.cfg.layers
        passes = max(1, -(-min_launches // per_step))
        n = passes * per_step
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        calls = [c for _ in range(passes) for c in self.decode_calls()]
        k = 0
        for (q, thin, v, lens, idx) in calls:
            ev[k][0].record()
            _lib.check("think_decode_attn_partial", lib.think_decode_attn_partial(
                d, q, thin, v, lens, idx, keep, self.scale, ws, wsn, stream))
            ev[k][1].record()
            _lib.check("think_decode_attn_combine", lib.think_decode_attn_combine(
                d, lens, keep, out, ws, wsn, stream))
            k += 1
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
        return float(us.mean()), n, [round(float(x), 2) for x in np.percentile(us, [10, 50, 90])]

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
    summary, if it was taken on this workload with the current kernel source."""
    path = os.path.join(ROOT, "profiles", "decode_mfma_llama3-8b-128k_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary"
    if rec.get("workload") != workload:
        return None, "counters taken on another workload"
    if rec.get("source_hash") != decode_source_hash():
        return None, "kernel changed since the counters were taken"
    return int(rec["hbm_bytes_per_launch"]), rec.get("command", "")


def cpu_baseline(wl, budget_s):
    """The oracle, untuned, on a bounded sample of the same workload: full
    score+select+compact of layer 0, then decode steps of layer 0 until the
    time budget is spent.  Same algorithmic byte accounting as the GPU."""
    import oracle
    cfg, L = wl.cfg, wl.host0
    bm = wl.bytes_model()
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    s = oracle.score(L["k_cache"], L["seq_lens"], L["q_obs"])
    idx, _ = oracle.select(s, cfg.keep)
    thin = oracle.compact(L["k_cache"], L["seq_lens"], idx)
    t_sc = time.perf_counter() - t0
    scale = np.float32(1.0 / np.sqrt(cfg.head_dim))
    steps, t_dec = 0, 0.0
    while steps < cfg.decode_steps and (t_sc + t_dec < budget_s or steps == 0):
        q = kvsynth.decode_q(cfg, 0, steps, L["channel_scale"])
        t1 = time.perf_counter()
        oracle.decode(q, thin, L["v_cache"], L["seq_lens"], idx, scale)
        t_dec += time.perf_counter() - t1
        steps += 1
    total_bytes = bm["sc_layer"] + steps * bm["dec_call"]
    total_s = t_sc + t_dec
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(total_bytes / total_s / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu": model,
            "sample": (f"layer 0 of {cfg.name}: score+select+compact once ({t_sc:.2f}s) and "
                       f"{steps} decode steps ({t_dec:.2f}s); fp64 C oracle, OpenMP over "
                       f"(batch, head) pairs, {threads} threads"),
            "seconds": round(total_s, 2),
            "score_compact_GBps": round(bm["sc_layer"] / t_sc / 1e9, 4),
            "decode_GBps": round(steps * bm["dec_call"] / max(t_dec, 1e-9) / 1e9, 4)}


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
    wl = Workload(cfg, torch, qdk, dev)
    wl.prepare_decode()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    bm = wl.bytes_model()
    n_dec = cfg.decode_steps * cfg.layers

    for _ in range(max(args.warmup, 1 if wl.ncopies > 1 else 0)):
        for _ in range(wl.ncopies):              # every copy's thin cache is filled
            wl.score_compact(sp)
        wl.decode(sp)
    torch.cuda.synchronize()
    log("warmup done")

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        a, b, c = ev[k]
        a.record(stream)
        wl.score_compact(sp)
        b.record(stream)
        wl.decode(sp)
        c.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sc_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    dec_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    log(f"timed {args.steps} steps: {wall:.3f}s wall, score+compact {sc_ms:.3f} ms, "
        f"decode {dec_ms:.3f} ms per step")

    ms_per_step = wall / args.steps * 1e3
    step_bytes = cfg.layers * bm["sc_layer"] + n_dec * bm["dec_call"]
    value = step_bytes / (ms_per_step / 1e3) / 1e9
    tok = bm["tokens"]
    kv_tok_s = (tok * cfg.layers * (1 + cfg.decode_steps)) / (ms_per_step / 1e3)
    sc_gbs = cfg.layers * bm["sc_layer"] / (sc_ms / 1e3) / 1e9
    dec_gbs = n_dec * bm["dec_call"] / (dec_ms / 1e3) / 1e9
    dec_call_us = dec_ms * 1e3 / n_dec
    near = int(sum(int(e["tie"].sum().item()) for e in wl.layers))
    # the dominant kernel's own launch duration, live, with HIP events (a
    # separate pass after the timed region, so the events do not perturb it)
    if args.no_kernel_timing:
        part_us, n_part, part_pct = float("nan"), 0, None
    else:
        part_us, n_part, part_pct = wl.decode_kernel_times(sp, torch)
        log(f"chunk-pass kernel: {part_us:.2f} us mean over {n_part} launches")
    achieved = bm["dec_call"] / (part_us * 1e-6) / 1e9 if n_part else None
    app_us, app_bytes = append_time(cfg, torch, qdk, dev)
    log(f"decode-time append: {app_us:.2f} us per call")
    sep_us, fus_us = append_decode_time(wl, torch, qdk)
    log(f"append+decode on layer 0: separate {sep_us:.2f} us, fused {fus_us:.2f} us per step")
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
               "prune_after_prefill_GBps": round((K + Kt + Qw) / ((ps_us + pc_us) * 1e-6) / 1e9, 1),
               "prune_after_prefill_pct_of_peak":
                   round(100 * (K + Kt + Qw) / ((ps_us + pc_us) * 1e-6) / 1e9 / PEAK_GBS, 2),
               "note": "layer 0: prompt written in 8192-row chunks (reads and writes K and V: "
                       "4|K| bytes) gathering the key sums; then scores+selection from the sums "
                       "and compaction, |K| + |K_thin| + |Q_w| bytes (one read of K)"}
        log(f"prefill-fused scoring: write {pw_us:.1f} us, score from sums {ps_us:.2f} us, "
            f"compact {pc_us:.1f} us per layer")
    traffic, traffic_src = committed_traffic(cfg.name)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded log-normal channel scales, x8 outliers, rank-32 keys + noise)",
        "config": {"workload": cfg.name, "layers": cfg.layers, "batch": cfg.batch,
                   "seq_len": cfg.seq_capacity, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "obs_window": cfg.obs_window, "keep": cfg.keep,
                   "decode_steps": cfg.decode_steps, "valid_tokens_per_layer": tok},
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "value_note": ("bytes counted as two passes over K; the score+compact path read K once "
                       "(effective bandwidth)" if wl.single_read else
                       "algorithmic bytes of the path as run"),
        "kv_tokens_per_s": float(f"{kv_tok_s:.4g}"),
        "paths": {
            "score_compact": {"ms_per_step": round(sc_ms, 3), "GBps": round(sc_gbs, 1),
                              "pct_of_peak": round(100 * sc_gbs / PEAK_GBS, 2),
                              "kv_tokens_per_s": float(f"{tok * cfg.layers / (sc_ms / 1e3):.4g}"),
                              "bytes_per_layer": bm["sc_layer"],
                              "single_read_bytes_per_layer": bm["sc_min_layer"],
                              "path": ("single read: one launch holds K on chip"
                                       if wl.single_read else "two passes over K"),
                              "GBps_is_effective": bool(wl.single_read),
                              "GBps_moved": round(cfg.layers * (bm["sc_min_layer"] if wl.single_read
                                                                else bm["sc_layer"])
                                                  / (sc_ms / 1e3) / 1e9, 1)},
            "decode": {"ms_per_step": round(dec_ms, 3), "GBps": round(dec_gbs, 1),
                       "pct_of_peak": round(100 * dec_gbs / PEAK_GBS, 2),
                       "us_per_call": round(dec_call_us, 2),
                       "kv_tokens_per_s": float(f"{tok * n_dec / (dec_ms / 1e3):.4g}"),
                       "bytes_per_call": bm["dec_call"]},
            "prefill_fused_scoring": pre,
            "append": {"us_per_call": round(app_us, 2), "bytes_per_call": app_bytes,
                       "note": "think_append_kv, timed apart from the step (the workload's "
                               "caches are full)"},
            "append_decode": {"separate_us_per_step": round(sep_us, 2),
                              "fused_us_per_step": round(fus_us, 2),
                              "note": "layer 0 in caches with 64 free rows: 64 steps of "
                                      "think_append_kv + think_decode_attn, then of "
                                      "think_append_decode_attn from the same lengths"},
        },
        "roofline": {"kernel": "k_decode_mfma (think_decode_attn chunk pass)",
                     "bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
                     "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4) if achieved else None,
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": bm["dec_call"],
                     "launch_us": round(part_us, 2) if n_part else None,
                     "launch_us_p10_p50_p90": part_pct,
                     "timing": (f"HIP events on the launch stream around each of {n_part} "
                                f"chunk-pass launches (one step's decode calls, repeated to at "
                                f"least 64), after the timed steps"),
                     "traffic_source": traffic_src},
        "near_ties": near,
        "input_copies": wl.ncopies,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
