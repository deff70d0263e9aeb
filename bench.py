"""Benchmark of the paged-attention hot path on one MI355X.

Headline: one engine step of the Qwen3-0.6B-shaped decode workload (batch 64, 16 q heads /
8 kv heads, head_dim 128, bf16, context U[256, 4096], block 256, 2048-block pool): store
the 64 new tokens' K/V and attend, as one paged_attn_decode_store call (split-K partials,
then the combine, which also writes the new rows into their slots). The same step as the
two separate calls (store_kvcache, then paged_attn_decode) is timed after it and reported
beside it. Consecutive steps rotate over several layer pools (each a full copy of the
2048-block K/V pool, as every layer of the engine owns its own cache), so the KV read
streams from HBM rather than from the 256 MB last-level cache.

The same JSON line also carries the prefill half of the metric (the varlen prefill, the
prefix-cached prefill and the chunked prefill workloads, in TFLOP/s against the bf16 MFMA
peak), the large decode workload (512 sequences, shared prefixes), small-batch decode steps
replayed from recorded graphs next to eager calls (one call, and a whole 28-layer step), and
the host metadata time.

``value`` is the decode step's algorithmic bytes per second (KV rows of every visible key
once per sequence and kv head, plus q, out, tables, and the store's reads and writes).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode paged-attn KV GB/s (% HBM peak); prefill attn TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


# ---------------------------------------------------------------- algorithmic work
def decode_bytes(w, unique=False):
    e = w.elem_bytes
    row = w.num_kv_heads * w.head_dim * e           # one token's K (or V) row, all kv heads
    if unique:
        prefix_used = int(w.shared_blocks.max()) if len(w.shared_blocks) else 0
        toks = int((w.seq_lens - w.shared_blocks * w.block_size).sum()) + prefix_used * w.block_size
    else:
        toks = int(w.seq_lens.sum())
    kv = 2 * toks * row
    qo = 2 * w.num_seqs * w.num_heads * w.head_dim * e
    meta = w.num_seqs * (w.max_table_len() * 4 + 4)
    return kv + qo + meta, kv


def store_bytes(w):
    n_new = int(w.q_lens.sum())
    row = w.num_kv_heads * w.head_dim * w.elem_bytes
    return 2 * 2 * n_new * row + 4 * n_new


def prefill_flops(w):
    Lq = w.q_lens.astype(np.int64)
    Lk = w.seq_lens.astype(np.int64)
    pairs = int((Lq * (Lk - Lq) + Lq * (Lq + 1) // 2).sum())
    return 4 * w.num_heads * w.head_dim * pairs, pairs


# ---------------------------------------------------------------- GPU legs
class CacheFlush:
    """A 1 GiB device buffer rewritten between timed runs (outside the timed region), so that
    every run starts with the 256 MB last-level cache and the L2s holding none of its inputs.

    read_back: also read the buffer back, so that no dirty line is left either. After the
    write alone the caches hold up to ~290 MB of the buffer's dirty lines, whose write-back
    lands inside the timed call; for an HBM-bound call that is time the call's own traffic
    does not account for (batch-512 shared-prefix decode, one process: 275.8-277.6 us after
    the write alone, 265.5-268.0 after write and read-back, 259 us with no flush). The
    compute-bound prefill calls gain nothing from it (varlen 74.0-74.6 us after the write,
    74.8-75.5 after a read alone) and lose 2-5% after the longer write-and-read flush, so the
    prefill legs keep the write alone."""

    def __init__(self, torch, nbytes=1 << 30, read_back=False):
        self.torch = torch
        self.read_back = read_back
        self.buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.empty((), dtype=torch.int64, device="cuda")
        self.val = 0

    def __call__(self):
        self.val += 1
        self.buf.fill_(self.val)
        if self.read_back:
            self.torch.sum(self.buf, dim=0, dtype=self.torch.int64, out=self.sink)


class HipTimer:
    """Timing events of the HIP runtime this process uses (the copy torch loaded, which the
    library's calls run on), created with hipEventDisableSystemFence. A default event record
    ends with a system-scope fence: an L2 write-back and invalidate between the work before
    it and the work after it, which slows what follows (the HIP header documents the flag
    for events used only to measure time). Measured on the headline loop: call 96.6 ->
    94.7 us, wall time per step 101.7 -> 98.7 us, same kernels. Results are read only after a
    device-wide synchronisation."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        self.ct = ctypes
        path = None
        try:
            with open(f"/proc/{os.getpid()}/maps") as fh:
                for line in fh:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
        except OSError:
            pass
        self.hip = ctypes.CDLL(path or "libamdhip64.so")
        P = ctypes.c_void_p
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [P, P]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        self.hip.hipEventDestroy.argtypes = [P]
        self.live = []

    def event(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        self.live.append(e)
        return e

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(e, self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b):
        f = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return f.value

    def release(self):
        for e in self.live:
            self.hip.hipEventDestroy(e)
        self.live = []


_TIMER = None


def timer():
    global _TIMER
    if _TIMER is None:
        _TIMER = HipTimer()
    return _TIMER


# Secondary workloads run their own calls for this long before timing: the part raises its
# clocks only under sustained load (varlen prefill: 94.8 us after 5 back-to-back calls, 80.3
# after 200, 78.2 after 1000, and ~94 again after half a second idle), so a few warm-up calls
# would time a part still ramping up rather than the steady state a serving loop runs in.
SECONDARY_WARMUP_S = 0.25


def _median_event_ms(torch, fn, iters, warmup, stream, flush=None, warmup_s=SECONDARY_WARMUP_S):
    """Median, p10 and p90 (ms) of `fn` bracketed by events on `stream`, each timed run
    preceded (outside the bracket) by `flush`. Before timing: `warmup` calls, then more calls
    until `warmup_s` seconds have passed."""
    for _ in range(warmup):
        fn()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < warmup_s:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    tm = timer()
    starts = [tm.event() for _ in range(iters)]
    ends = [tm.event() for _ in range(iters)]
    torch.cuda.synchronize()
    for i in range(iters):
        if flush is not None:
            flush()
        tm.record(starts[i], stream)
        fn()
        tm.record(ends[i], stream)
    torch.cuda.synchronize()
    t = np.array([tm.elapsed_ms(s, e) for s, e in zip(starts, ends)])
    tm.release()
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def bench_decode_headline(torch, args):
    from paged_kv_cache_225_amd.harness import DeviceStep
    from workloads import CONFIG_NAMES, make_config
    w = make_config(2)
    base = DeviceStep(w)
    layers = [(base.k_cache, base.v_cache)]
    for _ in range(args.layers - 1):
        layers.append((base.k_cache.clone(), base.v_cache.clone()))
    stream = torch.cuda.current_stream()
    from paged_kv_cache_225_amd import _binding as B

    # the workload's block tables do not overlap (no block is read twice in a step), so the
    # caller streams every K/V row past the caches (first streamed table column 0 for every
    # sequence)
    ksf = torch.zeros(w.num_seqs, dtype=torch.int32, device="cuda")

    def fused(i):
        kc, vc = layers[i % len(layers)]
        B.paged_attn_decode_store(base.out, base.q, base.new_k, base.new_v, base.slot_mapping,
                                  kc, vc, base.block_tables, base.context_lens, w.scale,
                                  workspace=base.workspace, kv_stream_from=ksf, stream=stream)

    def separate(i):
        kc, vc = layers[i % len(layers)]
        B.store_kvcache(base.new_k, base.new_v, kc, vc, base.slot_mapping, stream=stream)
        B.paged_attn_decode(base.out, base.q, kc, vc, base.block_tables, base.context_lens,
                            w.scale, workspace=base.workspace, kv_stream_from=ksf, stream=stream)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        # exactly K steps between two synchronisations. Calls stride, 2 stride, ... (1-based)
        # are bracketed by events on the launch stream for the per-launch time: two event
        # records between consecutive calls cost ~4 us of wall time per step (measured:
        # 97.7-98.3 vs 93.4 us per step), which bracketing every call would charge to the
        # throughput
        stride = max(1, args.steps // max(5, args.steps // 8))
        tm = timer()
        ev = [(tm.event(), tm.event()) for _ in range(args.steps // stride)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            rec = (i + 1) % stride == 0
            if rec:
                tm.record(ev[i // stride][0], stream)
            fn(i)
            if rec:
                tm.record(ev[i // stride][1], stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        call_ms = np.array([tm.elapsed_ms(a, b) for a, b in ev])
        tm.release()
        return elapsed * 1e3 / args.steps, call_ms, stride

    ms_per_step, call_ms, stride = timed(fused)
    sep_ms_per_step, sep_call_ms, _ = timed(separate)
    step_bytes_dec, kv = decode_bytes(w)
    step_bytes = step_bytes_dec + store_bytes(w)
    call_avg = float(call_ms.mean())
    achieved = step_bytes / (call_avg * 1e-3) / 1e9
    return {
        "w": w,
        "name": CONFIG_NAMES[2],
        "ms_per_step": ms_per_step,
        "value": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "tokens_per_s": w.num_seqs / (ms_per_step * 1e-3),
        "step_bytes": step_bytes,
        "kv_bytes": kv,
        "decode_call_us_avg": call_avg * 1e3,
        "decode_call_us_p10_p90": [float(np.percentile(call_ms, 10)) * 1e3,
                                   float(np.percentile(call_ms, 90)) * 1e3],
        "decode_calls_timed": f"calls {stride}, {2 * stride}, ... of the {args.steps} timed calls, {len(call_ms)} in all",
        "separate_calls": {"ms_per_step": sep_ms_per_step,
                           "value": step_bytes / (sep_ms_per_step * 1e-3) / 1e9,
                           "call_us_avg": float(sep_call_ms.mean()) * 1e3},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": decode_traffic_bytes()},
    }


def bench_prefill(torch, cfg, iters, warmup, flush=None):
    """Prefill workload `cfg` (3: varlen, 4: prefix-cached, "chunked": chunked prefill with
    unaligned resident prefixes): the step's store, then attention through the tables."""
    from paged_kv_cache_225_amd.harness import DeviceStep
    from workloads import CHUNKED_PREFILL_NAME, CONFIG_NAMES, make_chunked_prefill, make_config
    if cfg == "chunked":
        w, name = make_chunked_prefill(), CHUNKED_PREFILL_NAME
    else:
        w, name = make_config(cfg), CONFIG_NAMES[cfg]
    ds = DeviceStep(w)
    stream = torch.cuda.current_stream()
    ds.store(stream)
    med, p10, p90 = _median_event_ms(torch, lambda: ds.attend(stream), iters, warmup, stream,
                                     flush)
    st_med, _, _ = _median_event_ms(torch, lambda: ds.store(stream), iters, warmup, stream, flush)
    flops, pairs = prefill_flops(w)
    tf = flops / (med * 1e-3) / 1e12
    return {"workload": name, "attn_us_median": med * 1e3, "attn_us_p10_p90": [p10 * 1e3, p90 * 1e3],
            "flops": flops, "tflops": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
            "tokens_per_s": float(w.q_lens.sum()) / (med * 1e-3),
            "store_us_median": st_med * 1e3, "store_gbs": store_bytes(w) / (st_med * 1e-3) / 1e9}


def bench_prefill_packed(torch, iters, warmup, flush=None):
    """The varlen workload through attn_prefill_varlen: the step's own K/V rows, packed,
    no block table (the engine's path when no prefix is cached)."""
    from paged_kv_cache_225_amd import _binding as B
    from paged_kv_cache_225_amd.harness import DeviceStep
    from workloads import CONFIG_NAMES, make_config
    w = make_config(3)
    assert int(w.num_cached.sum()) == 0
    ds = DeviceStep(w)
    stream = torch.cuda.current_stream()
    mk = int(w.seq_lens.max())

    def call():
        B.attn_prefill_varlen(ds.out, ds.q, ds.new_k, ds.new_v, ds.cu_seqlens_q, ds.cu_seqlens_k,
                              ds.max_seqlen_q, mk, w.scale, stream=stream)

    med, p10, p90 = _median_event_ms(torch, call, iters, warmup, stream, flush)
    flops, _ = prefill_flops(w)
    tf = flops / (med * 1e-3) / 1e12
    return {"workload": CONFIG_NAMES[3] + "_packed_kv", "attn_us_median": med * 1e3,
            "attn_us_p10_p90": [p10 * 1e3, p90 * 1e3], "flops": flops, "tflops": tf,
            "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
            "tokens_per_s": float(w.q_lens.sum()) / (med * 1e-3)}


def _split_report(torch, ds):
    """The split-K layout the last decode call used, read back from its workspace: the call
    leaves there its share size S (keys per share) followed by the prefix sums of the context
    lengths it split. Every share covers S consecutive keys of the sequences laid end to end,
    so a sequence is cut into as many pieces as the shares its keys touch; the histogram of
    pieces per sequence is the partition count the combine merges."""
    ctx = np.asarray(ds.w.seq_lens, dtype=np.int64)
    cum = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    nb = ds.workspace.numel() // 4 * 4
    words = ds.workspace[:nb].view(torch.int32).cpu().numpy()
    n = len(cum)
    hits = np.flatnonzero(words == cum[-1])
    start = next((int(h) - n + 1 for h in hits
                  if h - n + 1 >= 1 and np.array_equal(words[h - n + 1:h + 1], cum)), None)
    if start is None:
        return None
    S = int(words[start - 1])
    first = cum[:-1] // S
    last = (cum[1:] - 1) // S
    pieces = np.where(ctx > 0, last - first + 1, 0)
    vals, counts = np.unique(pieces, return_counts=True)
    total = int(cum[-1])
    shares = -(-total // S)
    return {"share_keys": S, "shares": shares, "keys": total,
            "keys_per_share_mean": total / shares,
            "pieces_per_sequence_hist": {int(v): int(c) for v, c in zip(vals, counts)}}


def bench_large_decode(torch, iters, warmup, flush=None):
    """The 512-sequence decode workload. Half its sequences share 2-8 leading blocks (a
    common prompt prefix), which the caller knows from its block manager. The top-level
    fields time paged_attn_decode_prefix, the library's call for such a batch: each shared
    block read once for all the sequences holding it, the private rest streamed split-K.
    `plain_call` times paged_attn_decode on the same step, the shared leading blocks read
    with ordinary loads by every sharer and every other K/V row streamed."""
    from paged_kv_cache_225_amd.harness import DeviceStep
    from workloads import CONFIG_NAMES, make_config
    w = make_config(5)
    ds = DeviceStep(w, kv_stream_from="shared")
    stream = torch.cuda.current_stream()
    ds.store(stream)
    med, p10, p90 = _median_event_ms(torch, lambda: ds.attend(stream), iters, warmup, stream,
                                     flush)
    split = _split_report(torch, ds)
    uniq, kv_u = decode_bytes(w, unique=True)
    logi, kv_l = decode_bytes(w, unique=False)
    plain = {"call": "paged_attn_decode", "decode_us_median": med * 1e3,
             "decode_us_p10_p90": [p10 * 1e3, p90 * 1e3],
             "unique_gbs": uniq / (med * 1e-3) / 1e9, "logical_gbs": logi / (med * 1e-3) / 1e9,
             "frac_hbm_unique": uniq / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
             "kv_stream_from": "per sequence: its count of shared leading blocks",
             "split": split}
    ds.prefix_setup()
    pmed, pp10, pp90 = _median_event_ms(torch, lambda: ds.attend_prefix(stream), iters, warmup,
                                        stream, flush)
    return {"workload": CONFIG_NAMES[5], "call": "paged_attn_decode_prefix",
            "decode_us_median": pmed * 1e3, "decode_us_p10_p90": [pp10 * 1e3, pp90 * 1e3],
            "unique_gbs": uniq / (pmed * 1e-3) / 1e9,
            "logical_gbs": logi / (pmed * 1e-3) / 1e9,
            "frac_hbm_unique": uniq / (pmed * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tokens_per_s": w.num_seqs / (pmed * 1e-3), "shared_hist": w.meta.get("shared_hist"),
            "groups": ds.pfx["num_groups"], "largest_group": ds.pfx["max_group_size"],
            "cold_cache": None if flush is None else
            ("each timed call after a 1 GiB write and read-back (no input and no dirty line "
             "left in the caches)" if flush.read_back else
             "each timed call after a 1 GiB write (no input left in the caches)"),
            "plain_call": plain}


def bench_tiny_decode(torch, iters, warmup, flush=None):
    """The 2-sequence fp32 decode workload (contexts 300 and 700): a latency case."""
    from paged_kv_cache_225_amd.harness import DeviceStep
    from workloads import CONFIG_NAMES, make_config
    w = make_config(1)
    ds = DeviceStep(w)
    stream = torch.cuda.current_stream()
    ds.store(stream)
    med, p10, p90 = _median_event_ms(torch, lambda: ds.attend(stream), iters, warmup, stream,
                                     flush)
    _, kv = decode_bytes(w)
    return {"workload": CONFIG_NAMES[1], "decode_us_median": med * 1e3,
            "decode_us_p10_p90": [p10 * 1e3, p90 * 1e3], "kv_bytes": kv,
            "gbs": kv / (med * 1e-3) / 1e9}


def bench_graph_decode(torch, iters):
    """Decode steps of small batches replayed from the library's recorded graphs (one graph
    launch per step) next to the same call made eagerly (one library call, two kernel
    launches). Both loops issue `iters` back-to-back steps between two synchronisations;
    the rows are a seeded subset of the batch-64 workload's sequences. Before any timing
    every recorded bucket is replayed `iters` times: right after the headline loop the first
    few hundred graph launches of a process ran at ~40 us of host time each (20 us later
    on; eager calls unaffected), a transient that 10 warm-up launches did not cover."""
    from paged_kv_cache_225_amd import _binding as B
    from paged_kv_cache_225_amd.harness import DeviceStep, GraphDecodeStep
    from workloads import make_config
    w = make_config(2)
    ds = DeviceStep(w)
    gs = GraphDecodeStep(ds, 64, width=16)
    stream = torch.cuda.current_stream()
    rng = np.random.Generator(np.random.PCG64(77))
    gs.load(np.arange(64))
    for n in gs.graphs.buckets:
        for _ in range(iters):
            gs.launch(n, stream)
    torch.cuda.synchronize()
    rows = []
    for b in (1, 4, 16, 64):
        seqs = rng.choice(w.num_seqs, size=b, replace=False)
        gs.load(seqs)
        n = gs.graphs.bucket(b)

        def eager():
            B.paged_attn_decode_store(gs.out[:b], gs.q[:b], gs.key[:b], gs.value[:b],
                                      gs.slots[:b], ds.k_cache, ds.v_cache, gs.tables[:b],
                                      gs.ctx[:b], w.scale, workspace=gs.workspace, stream=stream)

        def graph():
            gs.launch(b, stream)

        res = {"batch": b, "bucket": n}
        for name, fn in (("eager", eager), ("graph", graph)):
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(iters):
                fn()
            t_host = time.perf_counter() - t0
            torch.cuda.synchronize()
            res[name + "_us_per_step"] = (time.perf_counter() - t0) / iters * 1e6
            # host time to enqueue a step (the loop's own cost, before waiting for the GPU)
            res[name + "_host_us_per_step"] = t_host / iters * 1e6
        rows.append(res)
    return {"workload": "decode steps of 1/4/16/64 sequences from the batch-64 workload "
                        "(ctx U[256,4096], 16q/8kv heads, d128, bf16)",
            "note": "wall time per step over back-to-back steps, both legs on the same "
                    "buffers; a small batch's K/V stays in the last-level cache across steps; "
                    "host_us: the enqueue loop's time per step before the final wait",
            "steps": rows}


def bench_graph_decode_layers(torch, iters, num_layers=28):
    """A whole decode step of a 28-layer model (Qwen3-0.6B's depth): one
    paged_attn_decode_store per layer, each layer its own 2048-block pool (device copies of
    the batch-64 workload's pool) and rows over the step's shared metadata. The graph leg
    replays one recorded graph per step (every layer's call); the eager leg makes the 28
    library calls from Python, as an engine without graphs does. Wall time per step over
    `iters` back-to-back steps, batches of 1, 4, 16 and 64 sequences."""
    from paged_kv_cache_225_amd import _binding as B
    from paged_kv_cache_225_amd.harness import DeviceStep, LayeredGraphDecodeStep
    from workloads import make_config
    w = make_config(2)
    ds = DeviceStep(w)
    layers = [ds] + [ds.replica() for _ in range(num_layers - 1)]
    # 28 distinct pools per step: a step's K/V (28 x ~9 MB per sequence) does not stay in the
    # last-level cache until the next step, and no block is read twice within one, so both
    # legs stream the K/V rows (kv_stream_from 0), as the headline does
    gs = LayeredGraphDecodeStep(layers, 64, width=16, kv_stream_from=0)
    stream = torch.cuda.current_stream()
    rng = np.random.Generator(np.random.PCG64(78))
    gs.load(np.arange(64))
    for n in gs.graphs.buckets:
        for _ in range(10):
            gs.launch(n, stream)
    torch.cuda.synchronize()
    rows = []
    for b in (1, 4, 16, 64):
        seqs = rng.choice(w.num_seqs, size=b, replace=False)
        gs.load(seqs)
        n = gs.graphs.bucket(b)

        def eager():
            ksf = gs.stream_from[:b]
            for l, d in enumerate(layers):
                B.paged_attn_decode_store(gs.out[l][:b], gs.q[l][:b], gs.key[l][:b],
                                          gs.value[l][:b], gs.slots[:b], d.k_cache, d.v_cache,
                                          gs.tables[:b], gs.ctx[:b], w.scale,
                                          workspace=gs.workspace, kv_stream_from=ksf,
                                          stream=stream)

        def graph():
            gs.launch(b, stream)

        res = {"batch": b, "bucket": n}
        for name, fn in (("eager", eager), ("graph", graph)):
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(iters):
                fn()
            t_host = time.perf_counter() - t0
            torch.cuda.synchronize()
            res[name + "_us_per_step"] = (time.perf_counter() - t0) / iters * 1e6
            res[name + "_host_us_per_step"] = t_host / iters * 1e6
        res["graph_speedup"] = res["eager_us_per_step"] / res["graph_us_per_step"]
        rows.append(res)
    gs.graphs.close()
    del gs, layers, ds
    torch.cuda.empty_cache()
    return {"workload": f"{num_layers}-layer decode step: per layer one paged_attn_decode_store "
                        "over its own 2048-block pool; 1/4/16/64 sequences of the batch-64 "
                        "workload (ctx U[256,4096], 16q/8kv heads, d128, bf16)",
            "note": "wall time per step over back-to-back steps; eager: 28 library calls "
                    "from Python per step; graph: one graph launch per step; both legs read "
                    "the K/V rows with non-temporal loads (kv_stream_from 0); host_us: the "
                    "enqueue loop's time per step before the final wait",
            "layers": num_layers, "steps": rows}


def bench_sampler(torch, iters):
    """Temperature sampling of one decode step's next tokens: 64 rows of Qwen3-vocabulary
    (151936) fp32 logits, the row's logits read once (HBM bytes = rows x vocab x 4)."""
    from paged_kv_cache_225_amd import _binding as B
    rows, vocab = 64, 151936
    g = torch.Generator(device="cuda").manual_seed(5)
    logits = torch.randn(rows, vocab, device="cuda", generator=g) * 3
    temps = torch.full((rows,), 0.6, device="cuda")
    tokens = torch.empty(rows, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.pkv_sample_workspace_bytes(rows, vocab), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    step = [0]

    def call():
        step[0] += 1
        B.pkv_sample(tokens, logits, temps, 1234, step[0], workspace=ws, stream=stream)

    med, p10, p90 = _median_event_ms(torch, call, iters, 5, stream)
    nbytes = rows * vocab * 4
    return {"workload": "sampler_64rows_vocab151936_f32", "us_median": med * 1e3,
            "us_p10_p90": [p10 * 1e3, p90 * 1e3], "logit_bytes": nbytes,
            "gbs": nbytes / (med * 1e-3) / 1e9, "frac_hbm": nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bound": "alu (a Philox4x64-10 block per 8 elements and two logs per element)"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_b64_hbm_traffic.json")


def decode_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in ("common.hpp", "launch.hpp", "prefix_unit.hpp", "decode.hip"):
        with open(os.path.join(ROOT, "paged_kv_cache_225_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def decode_traffic_bytes():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, or None
    when the decode kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("kernel_sources_sha256") != decode_sources_sha256():
        return None
    return d.get("traffic_bytes_per_launch")


def host_metadata_us(w, reps=20):
    from paged_kv_cache_225_amd import _binding as B
    t0 = time.perf_counter()
    for _ in range(reps):
        B.pkv_decode_metadata(w.seq_lens, w.block_tables, w.block_size)
    return (time.perf_counter() - t0) / reps * 1e6


# ---------------------------------------------------------------- CPU baseline (oracle)
def cpu_model_name():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, budget_s):
    """The oracle (numpy fp64) on the host cores this process may run on: its BLAS is given
    one thread per core of the affinity mask, and that count is reported."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from tests.oracle_pipeline import setup_pools, run_step
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        kc, vc = setup_pools(w)
        step_bytes_dec, _ = decode_bytes(w)
        step_bytes = step_bytes_dec + store_bytes(w)
        reps, t_total = 0, 0.0
        while t_total < budget_s or reps == 0:
            t0 = time.perf_counter()
            run_step(w, kc, vc)
            t_total += time.perf_counter() - t0
            reps += 1
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": step_bytes * reps / t_total / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "affinity_cores": cores, "cpu_model": cpu_model_name(),
            "sample": f"{reps} full decode step(s) of the batch-64 workload (store of 64 tokens "
                      f"+ fp64 attention over all 64 sequences), {t_total:.1f} s"}


def copy_calibration(torch, reps):
    """A plain copy of a known size: FETCH_SIZE / WRITE_SIZE per dispatch should read 1 GiB."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "reps": reps,
                      "copy_gbs": 2 * n / dt / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--layers", type=int, default=4, help="layer pools rotated over")
    ap.add_argument("--iters", type=int, default=50, help="timed runs of the secondary workloads")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--mode", choices=["bench", "copy"], default="bench",
                    help="copy: run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--no-flush", action="store_true",
                    help="secondary workloads: skip the 1 GiB cache flush between timed runs")
    ap.add_argument("--only", choices=["prefill3", "prefill4", "prefill3packed", "chunked", "large",
                                       "tiny", "graph", "graph_layers", "sampler"],
                    default=None,
                    help="run one secondary workload alone (for profiler passes)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.mode == "copy":
        copy_calibration(torch, args.steps)
        return
    if args.only is not None:
        flush = None if args.no_flush else CacheFlush(torch)
        dflush = None if args.no_flush else CacheFlush(torch, read_back=True)
        if args.only == "large":
            res = bench_large_decode(torch, args.iters, 5, dflush)
        elif args.only == "tiny":
            res = bench_tiny_decode(torch, args.iters, 5, dflush)
        elif args.only == "prefill3packed":
            res = bench_prefill_packed(torch, args.iters, 5, flush)
        elif args.only == "chunked":
            res = bench_prefill(torch, "chunked", args.iters, 5, flush)
        elif args.only == "graph":
            res = bench_graph_decode(torch, 200)
        elif args.only == "graph_layers":
            res = bench_graph_decode_layers(torch, args.iters)
        elif args.only == "sampler":
            res = bench_sampler(torch, args.iters)
        else:
            res = bench_prefill(torch, 3 if args.only == "prefill3" else 4, args.iters, 5, flush)
        print(json.dumps({"only": args.only, **res}), flush=True)
        return
    print("bench: decode headline", file=sys.stderr, flush=True)
    head = bench_decode_headline(torch, args)
    w = head.pop("w")
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["name"], "global_batch": 64, "heads_q": 16, "heads_kv": 8,
                   "head_dim": 128, "block_size": 256, "pool_blocks": 2048,
                   "context": "uniform[256,4096]", "layer_pools_rotated": args.layers,
                   "step": "paged_attn_decode_store: store of the 64 new tokens' K/V + decode attention, one call",
                   "kv_stream_from": "0 for every sequence (every K/V row non-temporal; the tables do not overlap)"},
        "roofline": head["roofline"],
        "tokens_per_s": head["tokens_per_s"],
        "decode_call_us_avg": head["decode_call_us_avg"],
        "decode_call_us_p10_p90": head["decode_call_us_p10_p90"],
        "decode_calls_timed": head["decode_calls_timed"],
        "separate_calls": head["separate_calls"],
        "step_bytes": head["step_bytes"],
        "kv_bytes": head["kv_bytes"],
        "host_metadata_us": host_metadata_us(w),
    }
    if not args.no_secondary:
        flush = None if args.no_flush else CacheFlush(torch)
        dflush = None if args.no_flush else CacheFlush(torch, read_back=True)
        line["secondary_timing"] = ("HIP events around each call on its stream; median of "
                                    f"{args.iters} runs after 5 warm-up calls and "
                                    f"{SECONDARY_WARMUP_S} s more of the workload's own calls "
                                    "(steady-state clocks); "
                                    + ("no flush" if flush is None else
                                       "a 1 GiB buffer rewritten before each timed run (the "
                                       "decode legs also read it back, leaving no dirty line)"))
        print("bench: prefill workloads", file=sys.stderr, flush=True)
        line["prefill"] = [bench_prefill(torch, 3, args.iters, 5, flush),
                           bench_prefill(torch, 4, args.iters, 5, flush),
                           bench_prefill_packed(torch, args.iters, 5, flush),
                           bench_prefill(torch, "chunked", args.iters, 5, flush)]
        print("bench: large decode workload", file=sys.stderr, flush=True)
        line["large_decode"] = bench_large_decode(torch, args.iters, 5, dflush)
        print("bench: tiny decode workload", file=sys.stderr, flush=True)
        line["tiny_decode"] = bench_tiny_decode(torch, args.iters, 5, dflush)
        print("bench: graph-replayed small-batch decode", file=sys.stderr, flush=True)
        line["graph_decode"] = bench_graph_decode(torch, 200)
        print("bench: graph-replayed 28-layer decode steps", file=sys.stderr, flush=True)
        line["graph_decode_layers"] = bench_graph_decode_layers(torch, args.iters)
        print("bench: sampler", file=sys.stderr, flush=True)
        line["sampler"] = bench_sampler(torch, args.iters)
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
