"""Decode-step benchmark on one MI355X.

One step = RoPE on q and the new k, the KV-cache append, split-K GQA
attention and the cross-split merge, for one layer over a batch of synthetic
sequences whose inputs are already resident in HBM: gqa_decode_step (the
split kernel rotates q and appends the new tokens itself, then the merge)
on bf16 caches with up to 16 new tokens and up to 32 query rows (new tokens
x query heads) per KV head and on INT8 caches with one new token and up to
16 query heads per KV head; rope_append_kv(_multi) + gqa_decode_attn(_multi)
otherwise or with --two-calls.  Default workload: c3, the batched variable-length Llama-3-8B-shaped
decode (B 64, H 32, G 8, D 128, bf16 KV, contexts uniform in [512, 8192]).

Timing protocol: before every timed step (and every warm-up step) a 1 GiB
scratch buffer is streamed through the caches, outside the event bracket,
so that no K/V byte is left in the 256 MB last-level cache (MALL) or the
L2s: every step reads its cache cold from HBM, as a decode step of one
layer does in a model (--flush write fills the buffer instead).
Each step is bracketed by its own pair of events; the line reports p10 /
p50 / p90 over the K steps and takes p50 as the headline.  The same
protocol, in a second pass, times the split-K kernel alone with events the
library ties to that kernel's dispatch (kvd_options; hipExtLaunchKernel
takes the kernel's own start and end times).  A third
pass times K back-to-back steps without eviction ("warm", reported apart,
never used for the roofline); --no-warm skips it (profiling runs).

Prints ONE JSON line:
  value      KV HBM GB/s of the whole step = KV bytes / p50 step time, where
             KV bytes = sum_b L_b * G * D * 2 (K and V) * 2 bytes
  roofline   the split-K attention kernel alone (with the fused step: its
             RoPE and append included): KV bytes / its p50
             duration against the 8 TB/s HBM peak; `traffic` is the HBM
             bytes per launch from the committed rocprofv3 counter summary
             of this kernel and workload (null when missing or taken from a
             different kernel source); `frac_of_read_ceiling` compares it
             with a plain cold streaming read of the same byte count (the
             read probe, same eviction and event timing)
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
             workload, in the same unit (a reported baseline only)

With --kv int8 the same workload runs on an INT8 cache (per-KV-head
scales, rope_append_kv_int8 + gqa_decode_attn_int8); KV bytes then count one
byte per element.

With --prefill T the bench times a causal prefill instead: T new tokens per
sequence (a prompt from empty when the workload's lengths equal T, e.g.
--config c5 --prefill 131072; a chunk after the cached history otherwise),
rope_append_kv_multi + gqa_prefill_attn, reported in TFLOP/s of attention
(4 * head_dim flops per query head and attended key) against the 2.5 PFLOP/s
bf16 matrix-core peak.

With --n-query T each sequence brings T new tokens (the verification pass of
speculative decoding: rope_append_kv_multi + gqa_decode_attn_multi); the KV
bytes are unchanged (the T queries of a KV head share each tile), the step
processes B * T tokens.

Usage: python bench.py [--steps K] [--warmup W] [--config c3|c4|c5|c2|c1]
                       [--kv-heads G] [--kv native|int8] [--n-query T] [--prefill T]
                       [--kernel auto|valu|mfma] [--split N]
                       [--no-cpu-baseline] [--no-warm] [--no-read-ceiling]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "kv_cache_gqa_decode_amd", "csrc")


# the sources each split-K kernel is built from (a change to any of them
# invalidates the traffic counters recorded for that kernel)
KERNEL_SOURCES = {
    "mfma": ("decode_mfma.hip", "mfma_tile.h", "kvd_internal.h", "uniform_join.h"),
    "int8": ("decode_i8.hip", "i8_codes.h", "mfma_tile.h", "kvd_internal.h", "uniform_join.h"),
    "valu": ("decode_valu.hip", "kvd_internal.h"),
    "prefill": ("prefill_mfma.hip", "mfma_tile.h", "kvd_internal.h", "uniform_join.h"),
    "prefill_i8": ("prefill_i8.hip", "i8_codes.h", "mfma_tile.h", "kvd_internal.h",
                   "uniform_join.h"),
}


def code_text(src: str) -> str:
    """C++ source without its comments and with whitespace collapsed: what
    the compiler sees, so that an edit to a comment keeps the hash."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(kernel: str = "mfma", read=None) -> str:
    """Hash of the code (comments aside) of the sources a kernel is built
    from; ``read(name)`` supplies a file's text (default: the working tree)."""
    if read is None:
        def read(name):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                return f.read()
    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES[kernel]):
        h.update(name.encode() + b"\0" + code_text(read(name)).encode())
    return h.hexdigest()[:16]


def workload_name(s) -> str:
    name = {"c1": "c1 fp32 single step B1 H8 G2 D64 L256",
            "c2": "c2 bf16 Llama-3-8B-shaped B1 H32 G8 D128 L1024",
            "c3": "c3 bf16 batched varlen B64 H32 G8 D128 L~U[512,8192]",
            "c4": f"c4 bf16 paged({s.block_size}) B32 H32 G8 D128 L~U[1024,32768] pool "
                  f"{s.num_blocks} blocks",
            "c5": f"c5 bf16 long context B1 H32 G{s.n_kv_heads} D128 L131072"}[s.name]
    if s.dtype == "i8":
        name = name.replace(" bf16 ", " INT8-KV (bf16 q, per-head scales) ", 1)
    return name


def load_traffic(key: str, src_hash: str, fused: bool):
    """HBM traffic per launch from profiles/<key>.json when it was measured
    on the current kernel sources and on the same kernel form (the split
    kernel with the RoPE and append fused, or the plain one)."""
    path = os.path.join(PROFILE_DIR, f"traffic_{key}.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != src_hash:
        return None
    if d.get("kernel_match", "").replace(" ", "").endswith(",true>") != fused:
        return None
    return d.get("hbm_bytes_per_launch")


FLUSH_BYTES = 1 << 30      # 4x the 256 MB MALL


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, np.float64), q))


def summary(xs):
    """p10 / p50 / p90 / mean of a list of milliseconds."""
    return {"p10": round(pct(xs, 10), 5), "p50": round(pct(xs, 50), 5),
            "p90": round(pct(xs, 90), 5), "mean": round(sum(xs) / len(xs), 5), "n": len(xs)}


class Flusher:
    """Evicts the K/V bytes of the previous step from the 256 MB MALL and the
    L2s before a timed step, on the current stream.

    "read" (default): streams a 1 GiB scratch buffer with plain loads (the
    read probe, default cache policy, so its lines allocate in every cache
    level), which leaves the caches full of clean, unrelated lines -- the
    state an attention call meets in a model, where the layers in between
    stream their own caches and weights.  "write": fills the 1 GiB buffer
    instead, which also evicts but leaves up to the MALL's size of dirty
    lines that the timed step then pays to write back.  "none": no eviction."""

    def __init__(self, dev, mode="read"):
        import torch
        self.mode = mode
        self.i = 0
        if mode != "none":
            self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
            self.buf.fill_(1)
            cu = torch.cuda.get_device_properties(dev).multi_processor_count
            self.nwg = 4 * cu
            self.sink = torch.empty(self.nwg, dtype=torch.int32, device=dev)

    def __call__(self):
        self.i += 1
        if self.mode == "write":
            self.buf.fill_(self.i & 0xFF)
        elif self.mode == "read":
            import kv_cache_gqa_decode_amd as kvd
            from kv_cache_gqa_decode_amd import _binding as B
            kvd.read_probe(self.buf, self.nwg, 8, B.PROBE_CHUNKED, self.sink)


def cold_times(run, n, flush):
    """Milliseconds of n calls of run(), each after a flush, each bracketed
    by its own events on the current stream (the flush outside)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in evs:
        flush()
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def cold_kernel_times(run_with_events, n, flush):
    """Milliseconds of the main kernel of n calls, each after a flush: the
    library ties the events to that kernel's dispatch (kvd_options)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:            # create the HIP events before the timed loop
        a.record()
        b.record()
    torch.cuda.synchronize()
    for a, b in evs:
        flush()
        run_with_events(a, b)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def warm_ms(run, n):
    """Mean milliseconds of n back-to-back calls (no eviction)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        run()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def read_ceiling(dev, kvd, nbytes: int, flush):
    """The practical roof for reading `nbytes` once, cold: the read probe over
    a buffer of exactly that size, after the same cache eviction as the
    timed steps, timed with events like the kernel, best median over its load
    paths (registers or HBM -> LDS copies, non-temporal) and launch shapes
    (GB/s).  At small sizes this is far below the nominal peak: the launch,
    the first requests' latency and the tail are not hidden by a long stream."""
    import torch
    from kv_cache_gqa_decode_amd import _binding as B
    nbytes = (nbytes + 1023) // 1024 * 1024
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    names = {B.PROBE_CHUNKED | B.PROBE_NONTEMPORAL: "registers, non-temporal",
             B.PROBE_CHUNKED: "registers",
             B.PROBE_LDS | B.PROBE_NONTEMPORAL: "HBM->LDS copies, non-temporal"}
    best = (0.0, None)
    for mode, name in names.items():
        for per_cu in (1, 2, 4):
            for unroll in (8, 16):
                nwg = cu * per_cu
                if mode & B.PROBE_LDS and nbytes // nwg >= (1 << 31):
                    continue
                sink = kvd.read_probe(buf, nwg, unroll, mode)
                times = cold_times(lambda: kvd.read_probe(buf, nwg, unroll, mode, sink), 9, flush)
                gbs = nbytes / (pct(times, 50) * 1e-3) / 1e9
                if gbs > best[0]:
                    best = (gbs, f"{name}, one contiguous chunk per workgroup, {per_cu} "
                                 f"workgroups/CU x 256 threads, {unroll} x 16 B in flight per lane")
    del buf
    torch.cuda.empty_cache()
    return {"gbs": round(best[0], 1), "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4),
            "shape": best[1], "bytes": nbytes,
            "protocol": "read probe over the kernel's byte count, cold, p50 of 9 event-timed launches"}


def cpu_baseline(s, p, budget_s: float):
    """Time the oracle (RoPE + append + attention, fp64, all host threads) on
    the first n sequences of the workload, n grown until ~budget_s of work."""
    import numpy as np
    import oracle
    from kv_cache_gqa_decode_amd import sizing

    threads = oracle.default_threads()
    g_all = oracle.Geometry(s.batch, s.n_heads, s.n_kv_heads, s.head_dim, s.dtype,
                            max_seq_len=s.max_seq_len, block_size=s.block_size,
                            num_blocks=s.num_blocks, max_blocks_per_seq=s.max_blocks_per_seq)

    sc = dict(k_scale=p.k_scale, v_scale=p.v_scale) if s.dtype == "i8" else {}
    T = p.n_query
    if T > 1:
        sc["n_query"] = T

    def run(n):
        idx = np.arange(n)
        kc, vc = p.k_cache, p.v_cache          # the oracle writes only the appended slots
        if s.block_size:
            g = oracle.Geometry(n, s.n_heads, s.n_kv_heads, s.head_dim, s.dtype,
                                block_size=s.block_size, num_blocks=s.num_blocks,
                                max_blocks_per_seq=s.max_blocks_per_seq)
            tab = np.ascontiguousarray(p.block_table[idx])
        else:
            g = oracle.Geometry(n, s.n_heads, s.n_kv_heads, s.head_dim, s.dtype,
                                max_seq_len=s.max_seq_len)
            kc = np.ascontiguousarray(p.k_cache[idx])
            vc = np.ascontiguousarray(p.v_cache[idx])
            tab = None
        args = [np.ascontiguousarray(a[idx]) for a in (p.q, p.k_new, p.v_new)]
        pos = np.ascontiguousarray(p.positions[idx])
        lens = np.ascontiguousarray(p.seq_lens[idx])
        t0 = time.perf_counter()
        q_rot = oracle.rope_append(g, *args, kc, vc, pos, tab, base=s.rope_base, **sc)
        oracle.decode_attn(g, q_rot, kc, vc, lens, tab, n_threads=threads, **sc)
        return time.perf_counter() - t0, lens

    del g_all
    n = 1
    dt, lens = run(n)
    while dt < budget_s / 4 and n < s.batch:
        n = min(s.batch, max(n + 1, int(n * budget_s / 2 / max(dt, 1e-3))))
        dt, lens = run(n)
    reps = [dt]
    # a workload shorter than the budget is repeated (the whole batch each
    # time) until about budget_s of work has been timed; the median is kept
    while sum(reps) < budget_s and len(reps) < 200:
        reps.append(run(n)[0])
    dt = float(sorted(reps)[len(reps) // 2])
    kvb = sizing.decode_kv_read_bytes(lens, s.n_kv_heads, s.head_dim, s.elem_bytes)
    return {"value": kvb / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {s.batch} sequences, all {s.n_heads} heads, "
                      f"{T} new token{'s' if T > 1 else ''} each, one step "
                      f"(RoPE + append + attention), median of {len(reps)} runs: {dt:.3f} s, "
                      f"{n / dt:.3g} seq-steps/s"}


def prefill_cpu_baseline(s, p, T, budget_s: float):
    """The oracle on sampled query rows of the prefill step (all host
    threads): flops of the sampled rows / time, in TFLOP/s."""
    import numpy as np
    import oracle
    g = oracle.Geometry(s.batch, s.n_heads, s.n_kv_heads, s.head_dim, s.dtype,
                        max_seq_len=s.max_seq_len, block_size=s.block_size,
                        num_blocks=s.num_blocks, max_blocks_per_seq=s.max_blocks_per_seq)
    kc, vc = p.k_cache.copy(), p.v_cache.copy()
    sc = dict(k_scale=p.k_scale, v_scale=p.v_scale) if s.dtype == "i8" else {}
    q_rot = oracle.rope_append(g, p.q, p.k_new, p.v_new, kc, vc, p.positions, p.block_table,
                               base=s.rope_base, n_query=T, **sc)
    rng = np.random.default_rng(97)
    threads = oracle.default_threads()

    def run(n):
        units = [(int(b), int(t), int(h)) for b, t, h in
                 zip(rng.integers(0, s.batch, n), rng.integers(0, T, n),
                     rng.integers(0, s.n_heads, n))]
        keys = sum(max(0, min(int(p.seq_lens[b]), int(p.seq_lens[b]) - T + 1 + t))
                   for b, t, _ in units)
        t0 = time.perf_counter()
        oracle.decode_attn_units(g, q_rot, kc, vc, p.seq_lens, units, p.block_table,
                                 n_query=T, n_threads=threads, **sc)
        return time.perf_counter() - t0, 4 * s.head_dim * keys

    n = 8
    dt, fl = run(n)
    while dt < budget_s / 4 and n < 1 << 16:
        n = max(n + 1, int(n * budget_s / 2 / max(dt, 1e-3)))
        dt, fl = run(n)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} query rows drawn uniformly over (sequence, new token, head), "
                      f"their attention over the causal bound in fp64: {dt:.3f} s"}


def run_prefill(args, s, dev):
    """Causal prefill of T new tokens per sequence: RoPE + append of the T
    tokens, then gqa_prefill_attn.  Prints one JSON line in TFLOP/s."""
    import numpy as np
    import torch
    import kv_cache_gqa_decode_amd as kvd
    from kv_cache_gqa_decode_amd import sizing
    from kv_cache_gqa_decode_amd import workloads as W
    T = args.prefill
    if s.dtype not in ("bf16", "i8"):
        print("--prefill runs on the bf16 workloads (c2..c5) or their INT8 form", file=sys.stderr)
        sys.exit(2)
    i8 = s.dtype == "i8"
    if T > s.max_seq_len:
        print(f"--prefill {T} exceeds the cache capacity {s.max_seq_len}", file=sys.stderr)
        sys.exit(2)
    t_gen = time.perf_counter()
    p = W.make_window(s, T, lengths=np.clip(W.draw_lengths(s), T, s.max_seq_len))
    print(f"# generated {s.name} prefill inputs in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    t = {k: W.as_torch(getattr(p, k), dev) for k in
         ("q", "k_new", "v_new", "k_cache", "v_cache", "positions", "seq_lens")}
    table = None if p.block_table is None else W.as_torch(p.block_table, dev)
    sc = dict(k_scale=W.as_torch(p.k_scale, dev), v_scale=W.as_torch(p.v_scale, dev)) if i8 else {}
    B, H, G, D = s.batch, s.n_heads, s.n_kv_heads, s.head_dim
    q_rot = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    out = torch.empty_like(q_rot)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    max_len = p.max_len
    base_opts = kvd.Options(dispatch_order=args.order if args.order >= 0 else None,
                            split_tokens=args.split)
    # the key-split workspace, allocated before the timed region
    ws_bytes = kvd.prefill_workspace_size(B, H, T, t["k_cache"], table, max_len, base_opts)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def step(options=None):
        kvd.rope_append_kv_multi(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                 t["positions"], table, base=s.rope_base, q_rot=q_rot, **sc)
        kvd.gqa_prefill_attn(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"], table,
                             max_seq_len=max_len, out=out, lse=lse,
                             options=options if options is not None else base_opts,
                             workspace=ws, **sc)

    flush = Flusher(dev, args.flush)
    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    steps = cold_times(step, args.steps, flush)
    t_wall = time.perf_counter() - t_wall
    kern = cold_kernel_times(lambda a, b: step(base_opts.with_events(a, b)), args.steps, flush)
    ms = pct(steps, 50)
    flops = sizing.window_attention_flops(p.seq_lens, T, H, D)
    kern_ms = pct(kern, 50)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    result = {
        "metric": "causal prefill attention TFLOP/s at 1 MI355X",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8 codes, f16 matrix cores" if i8 else "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(128) values and lengths; no datasets or weights)",
        "config": {"workload": workload_name(s) + f", prefill of {T} new tokens per sequence",
                   "batch": B, "n_heads": H, "n_kv_heads": G, "head_dim": D,
                   "new_tokens_per_seq": T, "total_context_tokens": int(p.seq_lens.sum()),
                   "attended_keys": sizing.window_key_count(p.seq_lens, T),
                   "flops_per_step": flops, "block_size": s.block_size,
                   "key_split_workspace_bytes": ws_bytes,
                   "arithmetic": ("codes converted to exact fp16 per tile, q and P rounded to "
                                  "fp16, fp32 accumulate" if i8 else
                                  "q and P rounded to bf16 on the matrix cores, fp32 accumulate"),
                   "parallelism": "single GPU"},
        "tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "timing": f"each step after a 1 GiB cache-evicting {args.flush}; ms_per_step = p50",
        "step_ms": summary(steps),
        "wall_ms_per_step": round(t_wall * 1e3 / args.steps, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(achieved / 2500.0, 4), "traffic": None,
                     "kernel": "causal prefill attention", "kernel_ms": round(kern_ms, 4),
                     "kernel_ms_pct": summary(kern), "launches_timed": len(kern),
                     "algorithmic_flops_per_launch": flops,
                     "kernel_source_hash": kernel_source_hash("prefill_i8" if i8 else "prefill")},
    }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = prefill_cpu_baseline(s, p, T, args.cpu_budget)
    print(json.dumps(result), flush=True)


def run_mixed(args, s, dev):
    """Decode step on a mixed-precision cache: the --window newest tokens of
    each sequence in bf16 rings, the older ones INT8.  KV bytes are the INT8
    history's plus the rings' (bf16) tokens attended; the kernel time spans
    both split kernels (the library ties the events to the first and the
    last)."""
    import numpy as np
    import torch
    import kv_cache_gqa_decode_amd as kvd
    from kv_cache_gqa_decode_amd import workloads as W
    Wn = int(args.window)
    t_gen = time.perf_counter()
    p = W.make_mixed(s, Wn)
    print(f"# generated {s.name} mixed inputs in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    t = {k: W.as_torch(getattr(p, k), dev) for k in
         ("q", "k_new", "v_new", "k_cache", "v_cache", "positions", "seq_lens", "k_scale",
          "v_scale", "k_recent", "v_recent")}
    table = None if p.block_table is None else W.as_torch(p.block_table, dev)
    B, H, G, D = s.batch, s.n_heads, s.n_kv_heads, s.head_dim
    max_len = p.max_len
    opts = kvd.Options(split_tokens=args.split,
                       dispatch_order=None if args.order < 0 else args.order)
    q_rot = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    out = torch.empty_like(q_rot)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws_bytes = kvd.workspace_size_mixed(B, H, t["k_cache"], Wn, table, max_len, opts)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def step(options=opts):
        kvd.rope_append_kv_mixed(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                 t["k_scale"], t["v_scale"], t["k_recent"], t["v_recent"],
                                 t["positions"], table, base=s.rope_base, q_rot=q_rot)
        kvd.gqa_decode_attn_mixed(q_rot, t["k_cache"], t["v_cache"], t["k_scale"], t["v_scale"],
                                  t["k_recent"], t["v_recent"], t["seq_lens"], table,
                                  max_seq_len=max_len, out=out, lse=lse, workspace=ws,
                                  options=options)

    flush = Flusher(dev, args.flush)
    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    steps = cold_times(step, args.steps, flush)
    kern = cold_kernel_times(lambda a, b: step(opts.with_events(a, b)), args.steps, flush)
    warm = None if args.no_warm else warm_ms(step, args.steps)
    del flush
    torch.cuda.empty_cache()
    L = p.seq_lens.astype(np.int64)
    hist = int(np.maximum(L - Wn, 0).sum())
    ring = int(np.minimum(L, Wn).sum())
    kv_bytes = 2 * G * D * (hist + 2 * ring)
    ms = pct(steps, 50)
    kern_ms = pct(kern, 50)
    achieved = kv_bytes / (kern_ms * 1e-3) / 1e9
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    ceiling = (None if args.no_read_ceiling else
               read_ceiling(dev, kvd, kv_bytes, Flusher(dev, args.flush)))
    result = {
        "metric": "decode-attention KV HBM GB/s (% of peak) and seq-steps/sec at 1 MI355X",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8+bf16",
        "data": ("synthetic (seeded INT8 codes ~ clipped N(0, 40^2) and per-head scales for the "
                 "history, seeded N(0,1)/sqrt(128) bf16 rings, seeded lengths; no datasets or "
                 "weights)"),
        "config": {"workload": workload_name(s).replace("INT8-KV", f"mixed-KV (last {Wn} bf16, "
                                                         "older INT8)", 1),
                   "batch": B, "n_heads": H, "n_kv_heads": G, "head_dim": D,
                   "window": Wn, "history_tokens": hist, "ring_tokens": ring,
                   "kv_bytes_per_step": kv_bytes, "block_size": s.block_size,
                   "max_context": max_len, "workspace_bytes": ws_bytes,
                   "parallelism": "single GPU"},
        "seq_steps_per_s": round(B / (ms * 1e-3), 1),
        "timing": (f"each step after a 1 GiB cache-evicting {args.flush}; ms_per_step and value "
                   "from the p50 of the K steps"),
        "step_ms": summary(steps),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode split-K attention, INT8 history + bf16 ring kernels",
                     "kernel_ms": round(kern_ms, 5), "kernel_ms_pct": summary(kern),
                     "launches_timed": len(kern), "algorithmic_bytes_per_launch": kv_bytes},
    }
    if ceiling is not None:
        result["roofline"]["read_ceiling_gbs"] = ceiling["gbs"]
        result["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling["gbs"], 4)
    if warm is not None:
        result["warm"] = {"ms_per_step": round(warm, 5),
                          "gbs": round(kv_bytes / (warm * 1e-3) / 1e9, 1)}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--kv-heads", type=int, default=None)
    ap.add_argument("--block-size", type=int, default=None, choices=[16, 32],
                    help="paged workload (c4) with 16- or 32-token blocks (same pool bytes)")
    ap.add_argument("--kv", default="native", choices=["native", "int8", "mixed"],
                    help="cache dtype: the workload's own (bf16 / fp32), INT8 with per-head "
                         "scales, or mixed (the --window newest tokens bf16, the rest INT8)")
    ap.add_argument("--window", type=int, default=1024,
                    help="--kv mixed: tokens per sequence kept in bf16")
    ap.add_argument("--n-query", type=int, default=1,
                    help="new tokens per sequence (T > 1: the multi-token verification step)")
    ap.add_argument("--prefill", type=int, default=0,
                    help="T > 0: time a causal prefill of T new tokens per sequence "
                         "(rope_append_kv_multi + gqa_prefill_attn; bf16 workloads) instead")
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--split", type=int, default=0)
    ap.add_argument("--tail-split", type=int, default=0,
                    help="tokens per split over the last --tail-span positions (0 = automatic)")
    ap.add_argument("--tail-span", type=int, default=-1)
    ap.add_argument("--order", type=int, default=-1,
                    help="dispatch order (-1 automatic): decode 0-4, prefill 5-7")
    ap.add_argument("--two-calls", action="store_true",
                    help="time rope_append_kv(_multi) + gqa_decode_attn(_multi) where "
                         "gqa_decode_step (the step in one launch plus the merge) would "
                         "otherwise run")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as one captured HIP graph in the timed region "
                         "(the kernel-time region stays eager)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--flush", default="read", choices=["read", "write", "none"],
                    help="how the caches are evicted before each timed step (default: a "
                         "1 GiB streaming read; 'write' fills 1 GiB, leaving dirty lines)")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm (back-to-back, no eviction) pass: every launch of "
                         "the run is then cold, as a kernel-trace profile should see them")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the cold streaming-read ceiling at the kernel's byte count (the "
                         "read probe, measured by default) that the kernel is reported against")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="only measure the cold streaming-read ceiling over 4 GiB and print it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times "
                         "(reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode step "
              "shards across GPUs by batch, heads or sequence with no change to the kernels, "
              "but this benchmark times one GPU.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_gqa_decode_amd as kvd
    from kv_cache_gqa_decode_amd import sizing
    from kv_cache_gqa_decode_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 3}))
        return
    if args.ceiling_only:
        print(json.dumps({"hbm_read_ceiling": read_ceiling(dev, kvd, 4 << 30, Flusher(dev))}))
        return
    s = W.spec(args.config, n_kv_heads=args.kv_heads, poison=False)
    if args.block_size is not None:
        if not s.block_size:
            print("--block-size applies to the paged workload (c4)", file=sys.stderr)
            sys.exit(2)
        s = W.spec(args.config, n_kv_heads=args.kv_heads, poison=False, block_size=args.block_size,
                   num_blocks=s.num_blocks * s.block_size // args.block_size,
                   max_blocks_per_seq=s.max_blocks_per_seq * s.block_size // args.block_size)
    if args.kv in ("int8", "mixed"):
        if s.dtype != "bf16":
            print(f"--kv {args.kv} applies to the bf16 workloads (c2..c5)", file=sys.stderr)
            sys.exit(2)
        s = s.replace(dtype="i8")
    if args.kv == "mixed":
        if args.prefill > 0 or args.n_query != 1 or args.graph:
            print("--kv mixed times the one-token decode step", file=sys.stderr)
            sys.exit(2)
        run_mixed(args, s, dev)
        return
    if args.prefill > 0:
        run_prefill(args, s, dev)
        return
    t_gen = time.perf_counter()
    T = args.n_query
    p = W.make_problem(s) if T == 1 else W.make_window(s, T)
    print(f"# generated {s.name} inputs in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)
    t = {k: W.as_torch(getattr(p, k), dev) for k in
         ("q", "k_new", "v_new", "k_cache", "v_cache", "positions", "seq_lens")}
    table = None if p.block_table is None else W.as_torch(p.block_table, dev)
    int8 = s.dtype == "i8"
    if int8:
        t["k_scale"] = W.as_torch(p.k_scale, dev)
        t["v_scale"] = W.as_torch(p.v_scale, dev)
    max_len = p.max_len
    opts = kvd.Options(kernel=None if args.kernel == "auto" else args.kernel,
                       split_tokens=args.split, tail_split_tokens=args.tail_split,
                       tail_span_tokens=max(args.tail_span, 0),
                       dispatch_order=None if args.order < 0 else args.order)
    if opts == kvd.Options():
        opts = None          # the automatic plan: the plain entry points
    B, H, G, D = s.batch, s.n_heads, s.n_kv_heads, s.head_dim
    lead = (B,) if T == 1 else (B, T)
    q_rot = torch.empty((*lead, H, D), dtype=torch.float32, device=dev)
    out = torch.empty((*lead, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((*lead, H), dtype=torch.float32, device=dev)
    ws_bytes = kvd.workspace_size(q_rot, t["k_cache"], table, max_len, n_query=T, options=opts)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    plan = kvd.get_plan(B, H, t["k_cache"], table, max_len, n_query=T, options=opts)
    sc = dict(k_scale=t["k_scale"], v_scale=t["v_scale"]) if int8 else {}
    # the decode step in one call where the library offers it
    fused = (not args.two_calls and args.kernel in ("auto", "mfma") and
             (T == 1 and (s.dtype == "bf16" and H // G <= 32 or s.dtype == "i8" and H // G <= 16)
              or s.dtype == "bf16" and T <= 16 and T * (H // G) <= 32))

    def step(options=opts):
        if fused:
            kvd.gqa_decode_step(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                t["positions"], table, base=s.rope_base, max_seq_len=max_len,
                                out=out, lse=lse, workspace=ws, options=options, **sc)
            return
        if T > 1:
            kvd.rope_append_kv_multi(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                     t["positions"], table, base=s.rope_base, q_rot=q_rot, **sc)
            kvd.gqa_decode_attn_multi(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"], table,
                                      max_seq_len=max_len, out=out, lse=lse, workspace=ws,
                                      options=options, **sc)
            return
        if int8:
            kvd.rope_append_kv_int8(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                    t["k_scale"], t["v_scale"], t["positions"], table,
                                    base=s.rope_base, q_rot=q_rot)
            kvd.gqa_decode_attn_int8(q_rot, t["k_cache"], t["v_cache"], t["k_scale"],
                                     t["v_scale"], t["seq_lens"], table, max_seq_len=max_len,
                                     out=out, lse=lse, workspace=ws, options=options)
            return
        kvd.rope_append_kv(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                           t["positions"], table, base=s.rope_base, q_rot=q_rot)
        kvd.gqa_decode_attn(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"], table,
                            max_seq_len=max_len, out=out, lse=lse, workspace=ws, options=options)

    flush = Flusher(dev, args.flush)
    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # the whole step (RoPE/append, work list, split kernel, merge) as one
        # graph: the kernels and their arguments are those of the eager step
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        run = graph.replay
    # pass 1: K whole steps, each after a cache-evicting write
    t_wall = time.perf_counter()
    steps = cold_times(run, args.steps, flush)
    t_wall = time.perf_counter() - t_wall
    # pass 2: the split-K kernel alone, same protocol, events the library
    # ties to its dispatch (kept out of pass 1, whose steps they would change)
    base_opts = opts if opts is not None else kvd.Options()
    kern = cold_kernel_times(lambda a, b: step(base_opts.with_events(a, b)), args.steps, flush)
    # pass 3: back-to-back steps, no eviction (reported apart)
    warm = None if args.no_warm else warm_ms(run, args.steps)
    del flush
    torch.cuda.empty_cache()
    ms_per_step = pct(steps, 50)
    kv_bytes = sizing.decode_kv_read_bytes(p.seq_lens, G, D, s.elem_bytes)
    aux = sizing.decode_aux_bytes(B, H, G, D, s.elem_bytes,
                                  int(sum(-(-int(L) // s.block_size) for L in p.seq_lens)) if table is not None else 0)
    gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    kern_ms = pct(kern, 50)
    achieved = kv_bytes / (kern_ms * 1e-3) / 1e9
    ceiling = (None if args.no_read_ceiling else
               read_ceiling(dev, kvd, kv_bytes, Flusher(dev, args.flush)))

    key = (f"{s.name}" + (f"_g{G}" if s.name == "c5" else "") + ("_i8" if int8 else "") +
           (f"_bs{s.block_size}" if s.block_size not in (0, 16) else "") +
           (f"_t{T}" if T > 1 else ""))
    src_hash = kernel_source_hash(plan["kernel"])
    traffic = load_traffic(key, src_hash, fused)
    result = {
        "metric": "decode-attention KV HBM GB/s (% of peak) and seq-steps/sec at 1 MI355X",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "i8": "i8"}[s.dtype],
        "data": ("synthetic (seeded INT8 codes ~ clipped N(0, 40^2), per-head scales, seeded "
                 "lengths; no datasets or weights)" if int8 else
                 "synthetic (seeded N(0,1)/sqrt(128) values, seeded lengths; no datasets or weights)"),
        "config": {"workload": workload_name(s), "batch": B, "n_heads": H, "n_kv_heads": G,
                   "head_dim": D, "kv_dtype": s.dtype, "accumulate": "f32" if not int8 else
                   "i32 (q K^T on int8 codes, 3 q limbs), f32 (P V in fp16 hi+lo)",
                   "block_size": s.block_size, "new_tokens_per_seq": T,
                   "total_context_tokens": int(p.seq_lens.sum()),
                   "max_context": max_len, "kv_bytes_per_step": kv_bytes,
                   "aux_bytes_per_step": aux, "split_tokens": plan["split_tokens"],
                   "n_splits": plan["n_splits"], "kernel": plan["kernel"],
                   "launch": "hip graph replay" if args.graph else "eager launches",
                   "step": ("gqa_decode_step: RoPE, append and attention in the split kernel, "
                            "then the merge" if fused else "rope_append_kv, then the attention call"
                            if T == 1 else "rope_append_kv_multi, then the attention call"),
                   "parallelism": "single GPU"},
        "seq_steps_per_s": round(B / (ms_per_step * 1e-3), 1),
        "tokens_per_s": round(B * T / (ms_per_step * 1e-3), 1),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "timing": (f"each step after a 1 GiB cache-evicting {args.flush} (MALL and L2 cold); "
                   "ms_per_step and value from the p50 of the K steps"
                   if args.flush != "none" else
                   "no eviction between steps; ms_per_step and value from the p50"),
        "step_ms": summary(steps),
        "wall_ms_per_step": round(t_wall * 1e3 / args.steps, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": ("decode split-K attention with RoPE and append fused" if fused
                                else "decode split-K attention"),
                     "kernel_ms": round(kern_ms, 5), "kernel_ms_pct": summary(kern),
                     "launches_timed": len(kern), "algorithmic_bytes_per_launch": kv_bytes,
                     "kernel_source_hash": src_hash},
    }
    if ceiling is not None:
        result["roofline"]["read_ceiling_gbs"] = ceiling["gbs"]
        result["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling["gbs"], 4)
        result["hbm_read_ceiling"] = ceiling
    if warm is not None:
        result["warm"] = {"ms_per_step": round(warm, 5),
                          "gbs": round(kv_bytes / (warm * 1e-3) / 1e9, 1),
                          "note": "back-to-back steps, no eviction; not used for the roofline"}
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(s, p, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
