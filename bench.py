#!/usr/bin/env python3
"""Benchmark of the paged decode hot path on one MI355X.

Workload: a Llama-3-8B-shaped decode layer in bf16 -- 32 query heads on 8 KV
heads (group 4), head_dim 128, block size 16, 64 sequences with context
lengths uniform in [128, 2048], blocks scattered by a seeded permutation of a
16384-block pool (synthetic N(0,1) data).

One step = the whole hot path for one layer of one decode iteration:
  1. pa_write_kv  -- the newest token's K/V row of every sequence is written
                     through the slot mapping (position n-1);
  2. pa_decode    -- paged attention of every sequence over its n positions
                     (split over the context with the log-sum-exp merge unless
                     --partition is 0; the default -1 balances the split).
Steps rotate over --layers independent pools (distinct device memory, each
its own block permutation), as consecutive layers of a model would, so the
K/V reads come from HBM rather than from the 256 MB last-level cache.

Reported (one JSON line):
  value        KV-read GB/s of the whole step: algorithmic K/V bytes (exactly
               context_len positions x 8 heads x 128 x 2 bytes x K and V) over
               the synchronised wall time of the timed steps, enqueued back to
               back with nothing recorded between them;
  roofline     the decode kernel alone, timed with the HIP event pair its
               launch records as it begins and ends (pa_time_next_decode),
               events created for timing only (hipEventDisableSystemFence:
               recording one performs no system-scope release, the cache
               write-back a default event adds to the interval):
               algorithmic bytes per launch / MEDIAN event duration, against
               MI355X's 8 TB/s HBM peak (beside it: the mean; the same pair
               as default events, fence included; stream_bracket_mean_us,
               default events on the stream around the whole call).  `traffic` is the HBM byte
               count per launch from the committed rocprofv3 counter runs
               (profiles/decode_traffic.json: the L2-to-memory read and write
               requests counted by size), reported only while the decode
               kernel's source hash matches the one they were taken on;
               `traffic_source` names the file, the request counts and the
               copy-calibrated FETCH_SIZE/WRITE_SIZE figure beside them;
  cpu_baseline the float64 oracle (write + decode) on the same batch, on this
               host's cores (skipped with --no-cpu-baseline).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s (10^9 bytes)
METRIC = "paged decode KV-read GB/s and % of MI355X HBM peak; decode tokens/s/layer"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8, help="independent layer pools to rotate over")
    ap.add_argument("--partition", type=int, default=-1,
                    help="split-KV partition size in tokens (0 = single pass, -1 = balanced split)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=64,
                    help="sequences of the batch the oracle baseline processes")
    ap.add_argument("--partitions", default="",
                    help="with --workload other than llama3-8b: comma-separated partition sizes to time "
                         "(default: -1, 0 and the batch's own or 256)")
    ap.add_argument("--workload", default="llama3-8b",
                    choices=["llama3-8b", "mha-13b", "prefix-cow", "fp8-long", "window", "swap", "prefill",
                             "prefill-chunk"],
                    help="llama3-8b: the step above (default).  The others time pa_decode alone on the "
                         "13B-shaped fp16 batch, the prefix-sharing batch or the long-context fp8 batch "
                         "(one JSON line per partition setting)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run pa_copy_blocks over MIB MiB of blocks (counter calibration) and exit")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


DECODE_SOURCES = ("pa_decode_fast.hip", "pa_common.h", "pa_internal.h", "pa_mfma.h")


class TimingEvent:
    """A HIP event created for timing only (hipEventDisableSystemFence), in
    the HIP runtime torch has loaded.  A default event performs a
    system-scope release when it is recorded, which writes back and
    invalidates caches inside the measured interval; this one does not.
    Same surface as the torch.cuda.Event calls used here."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime already loaded (by soname)
            hip.hipGetErrorString.restype = ctypes.c_char_p
            TimingEvent._hip = hip
        h = ctypes.c_void_p()
        self._check(TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h),
                                                             ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)))
        self.cuda_event = h.value

    @staticmethod
    def _check(rc):
        if rc != 0:
            raise RuntimeError(f"HIP event call failed: {TimingEvent._hip.hipGetErrorString(rc).decode()}")

    def record(self, stream):
        import ctypes
        self._check(TimingEvent._hip.hipEventRecord(ctypes.c_void_p(self.cuda_event),
                                                    ctypes.c_void_p(stream.cuda_stream)))

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        self._check(TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                                         ctypes.c_void_p(end.cuda_event)))
        return ms.value

    def __del__(self):
        if getattr(self, "cuda_event", None) and TimingEvent._hip is not None:
            import ctypes
            TimingEvent._hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))
            self.cuda_event = None


def kernel_timed(torch, stream, steps, run, timing_only=True):
    """Durations (ms) of ``steps`` calls of ``run(i, (start, stop))``, each
    handing the event pair to the call's launch (pa_time_next_decode), so
    that the pair is recorded as its first kernel begins and its last ends."""
    if timing_only:
        pairs = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    else:
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(steps)]
    for a, b in pairs:
        a.record(stream)               # both kinds exist once recorded
        b.record(stream)
    torch.cuda.synchronize()
    for i, ev in enumerate(pairs):
        run(i, ev)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def recorded_traffic(partition):
    """HBM bytes per decode launch from the committed rocprofv3 counter runs
    (with the record they come from), or (None, None) when the decode
    kernel's source (or the partition size) differs from the one the
    counters were taken on."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "decode_traffic.json")) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for name in DECODE_SOURCES:
            with open(os.path.join(ROOT, "paged_kv_cache_91_amd", "csrc", name), "rb") as f:
                h.update(f.read())
    except (OSError, ValueError):
        return None, None
    if rec.get("kernel_source_sha256") != h.hexdigest() or rec.get("partition_size") != partition:
        return None, None
    src = {"kind": "recorded, not measured in this run", "file": "profiles/decode_traffic.json"}
    src.update({k: rec[k] for k in ("method", "read_requests_per_launch", "write_requests_per_launch",
                                    "fetch_kib_per_launch", "write_kib_per_launch", "fetch_scale",
                                    "write_scale", "calibration", "calibrated_bytes_per_launch") if k in rec})
    return rec.get("hbm_bytes_per_launch"), src


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_91_amd import pa
    from paged_kv_cache_91_amd import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.lib()

    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy, pa, torch, dev)
    if args.workload == "swap":
        return swap_workload(args, pa, torch, dev)
    if args.workload.startswith("prefill"):
        return prefill_workload(args, pa, W, torch, dev)
    if args.workload != "llama3-8b":
        return other_workload(args, pa, W, torch, dev)

    t0 = time.time()
    wl = W.config2()
    S, hkv, d, bs = wl.num_seqs, wl.num_kv_heads, wl.head_dim, wl.block_size
    new_k = W.cast_f32(W.normal_f32(2, 4, S * hkv * d), "bf16").reshape(S, hkv, d)
    new_v = W.cast_f32(W.normal_f32(2, 5, S * hkv * d), "bf16").reshape(S, hkv, d)
    log(f"[bench] workload generated in {time.time() - t0:.1f}s: S={S} kv_bytes={wl.kv_bytes()/1e6:.1f} MB")

    def bf16_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    # layer 0 from the host arrays; the others are relabelled copies made on the device
    k0, v0 = bf16_dev(wl.k_pool), bf16_dev(wl.v_pool)
    q = bf16_dev(wl.q)
    kn, vn = bf16_dev(new_k), bf16_dev(new_v)
    ctx = torch.from_numpy(wl.context_lens.astype(np.int32)).to(dev)
    pos = wl.context_lens.astype(np.int64) - 1
    layers = []
    for layer in range(args.layers):
        if layer == 0:
            perm = np.arange(wl.num_blocks)
            kp, vp = k0, v0
        else:
            perm = np.random.default_rng(1000 + layer).permutation(wl.num_blocks)
            pt = torch.from_numpy(perm).to(dev)
            kp, vp = torch.empty_like(k0), torch.empty_like(v0)
            kp[pt] = k0
            vp[pt] = v0
        tables = perm[wl.block_tables].astype(np.int32)
        slots = tables[np.arange(S), pos // bs].astype(np.int64) * bs + pos % bs
        layers.append(dict(
            k=kp, v=vp, pool=pa.make_pool(kp, vp),
            tables=torch.from_numpy(tables).to(dev), slots=torch.from_numpy(slots).to(dev)))
    maxb = wl.max_blocks_per_seq
    ws = None
    if args.partition != 0:
        ws = pa.new_workspace(S, wl.num_q_heads, hkv, d, maxb, bs, args.partition, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"[bench] {args.layers} layers resident ({2 * k0.numel() * 2 * args.layers / 2**30:.1f} GiB of pools)")

    def step(k, ev=None, kernel_ev=None):
        L = layers[k % len(layers)]
        pa.pa_write_kv(kn, vn, L["slots"], L["pool"], stream=stream)
        if ev is not None:
            ev[0].record(stream)
        if kernel_ev is not None:
            pa.pa_time_next_decode(kernel_ev[0], kernel_ev[1])
        pa.pa_decode(q, L["pool"], L["tables"], ctx, wl.scale, out=out, partition_size=args.partition,
                     workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    # at least one warmup step per rotated layer, so every pool has been
    # touched before the timed region
    warmup_run = max(args.warmup, args.layers)
    for k in range(warmup_run):
        step(k)
    torch.cuda.synchronize()
    log(f"[bench] warmup {warmup_run} steps done")

    # timed region 1 (the value): K steps as they are, nothing recorded
    # between them
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(k)
    enqueued = time.perf_counter() - t_start        # host time to issue the steps
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log(f"[bench] timed {args.steps} steps in {elapsed:.4f}s")

    # timed region 2 (the roofline): K more steps, the decode kernel recording
    # its own event pair as it begins and ends (timing-only events), then K
    # with default events for comparison.  Events cost the stream a few
    # microseconds per call, so none are recorded in region 1.
    decode_ms = kernel_timed(torch, stream, args.steps, lambda k, ev: step(k, kernel_ev=ev))
    fenced_ms = kernel_timed(torch, stream, args.steps, lambda k, ev: step(k, kernel_ev=ev), timing_only=False)
    log(f"[bench] timed 2 x {args.steps} more steps with kernel events")
    # for reference: default events on the stream around each decode call
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(k, ev=events[k])
    torch.cuda.synchronize()
    bracket_ms = [a.elapsed_time(b) for a, b in events]

    kv_bytes = wl.kv_bytes()
    ms_per_step = elapsed * 1e3 / args.steps
    value = kv_bytes * args.steps / elapsed / 1e9
    dec_mean = statistics.fmean(decode_ms)
    dec_med = statistics.median(decode_ms)
    achieved = kv_bytes / (dec_med * 1e-3) / 1e9
    traffic, traffic_src = recorded_traffic(args.partition)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_run,
        "ms_per_step": round(ms_per_step, 5),
        "host_enqueue_ms_per_step": round(enqueued * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3-8b-layer-gqa4-bf16 (Hq=32, Hkv=8, D=128, block 16, "
                        "64 seqs, ctx U[128,2048], 16384-block pool)",
            "num_seqs": S, "num_q_heads": wl.num_q_heads, "num_kv_heads": hkv, "head_dim": d,
            "block_size": bs, "pool_blocks": wl.num_blocks, "context_tokens": int(wl.context_lens.sum()),
            "partition_size": args.partition, "layers_rotated": args.layers,
            "step": "pa_write_kv (1 token/seq) + pa_decode",
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s_per_layer": round(S / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_decode (decode kernel + split-KV merge)" if args.partition else "pa_decode",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
            "timing": "HIP events recorded by the decode kernel's launch as it begins and ends, created "
                      "for timing only (hipEventDisableSystemFence); achieved uses the median",
            "achieved_at_mean": round(kv_bytes / (dec_mean * 1e-3) / 1e9, 2),
            "mean_us": round(dec_mean * 1e3, 2),
            "median_us": round(dec_med * 1e3, 2),
            "p10_us": round(sorted(decode_ms)[len(decode_ms) // 10] * 1e3, 2),
            "p90_us": round(sorted(decode_ms)[(9 * len(decode_ms)) // 10] * 1e3, 2),
            "default_events_median_us": round(statistics.median(fenced_ms) * 1e3, 2),
            "stream_bracket_mean_us": round(statistics.fmean(bracket_ms) * 1e3, 2),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, new_k, new_v, args.cpu_seqs)
    print(json.dumps(result), flush=True)


def cpu_baseline(wl, new_k, new_v, nseq, min_seconds=10.0, max_passes=50):
    """The float64 oracle on the first ``nseq`` sequences of the same batch:
    the same cache write (one token per sequence) and decode, repeated until
    about ``min_seconds`` of CPU work has been timed."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle

    cores = len(os.sched_getaffinity(0))
    idx = np.arange(min(nseq, wl.num_seqs))
    bs = wl.block_size
    pos = wl.context_lens[idx].astype(np.int64) - 1
    slots = wl.block_tables[idx, pos // bs].astype(np.int64) * bs + pos % bs
    passes, total = 0, 0.0
    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        while total < min_seconds and passes < max_passes:
            t0 = time.perf_counter()
            kp, vp = oracle.oracle_write(new_k[idx], new_v[idx], "bf16", slots, wl.k_pool, wl.v_pool,
                                         "bf16")
            oracle.oracle_decode(wl.q[idx], "bf16", kp, vp, "bf16", wl.block_tables[idx],
                                 wl.context_lens[idx], wl.scale)
            total += time.perf_counter() - t0
            passes += 1
    dt = total / passes
    kv = int(wl.context_lens[idx].astype(np.int64).sum()) * 2 * wl.num_kv_heads * wl.head_dim * 2
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(kv / dt / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} passes over {len(idx)} of {wl.num_seqs} sequences of the same batch "
                      f"(one step each: write + decode, float64 numpy), {total:.1f}s in total",
            "seconds_per_step": round(dt, 4), "host_cpus": cores, "cpu_model": cpu_model,
            "decode_tokens_per_s_per_layer": round(len(idx) / dt, 3)}


def _oracle_threads(cores):
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])


def decode_cpu_baseline(wl, window, W, min_seconds=5.0, max_passes=200, pair_budget=2_000_000):
    """The float64 oracle's decode on a bounded sample of the same batch: the
    first sequences up to about ``pair_budget`` (position, query head) pairs,
    on the pools as the GPU decode reads them (the workload's cache write for
    those sequences, or its block copies, applied first and not timed, as
    on the GPU line), repeated until about ``min_seconds`` have been timed."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    cores = len(os.sched_getaffinity(0))
    seen = [min(int(n), window) if window else int(n) for n in wl.context_lens]
    k, pairs = 0, 0
    while k < wl.num_seqs and (k == 0 or pairs + seen[k] * wl.num_q_heads <= pair_budget):
        pairs += seen[k] * wl.num_q_heads
        k += 1
    idx = np.arange(k)
    kp, vp = wl.k_pool, wl.v_pool
    with threadpool_limits(limits=cores):
        threads = _oracle_threads(cores)
        if wl.write_k is not None:
            bs = wl.block_size
            mine = np.isin(wl.slot_mapping // bs, wl.block_tables[idx].ravel())
            kp, vp = oracle.oracle_write(wl.write_k[mine], wl.write_v[mine], wl.write_src_dtype,
                                         wl.slot_mapping[mine], kp, vp, wl.kv_dtype, wl.k_scale, wl.v_scale)
        if wl.copy_pairs is not None:
            kp, vp = oracle.oracle_copy(kp, vp, wl.copy_pairs)
        passes, total = 0, 0.0
        while total < min_seconds and passes < max_passes:
            t0 = time.perf_counter()
            oracle.oracle_decode(wl.q[idx], wl.q_dtype, kp, vp, wl.kv_dtype, wl.block_tables[idx],
                                 wl.context_lens[idx], wl.scale, wl.k_scale, wl.v_scale, window=window)
            total += time.perf_counter() - t0
            passes += 1
    dt = total / passes
    kv = sum(seen[:k]) * 2 * wl.num_kv_heads * wl.head_dim * W.ELEMENT_SIZE[wl.kv_dtype]
    return {"value": round(kv / dt / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} passes of the decode of the first {k} of {wl.num_seqs} sequences "
                      f"({sum(seen[:k])} positions, float64 numpy), {total:.1f}s in total"}


def other_workload(args, pa, W, torch, dev):
    """pa_decode alone on one of the other batches, timed per call (after its
    cache write or block copies, which are not timed) by the event pair the
    launch records around its kernels, and again by events on the stream
    around the call, which also hold the launch gaps.  Their
    pools are 1-21 GB, past the 256 MB last-level cache, except the prefix
    batch's (about 40 MB of distinct blocks): its numbers are cache-warm."""
    import numpy as np
    t0 = time.time()
    window = 0
    if args.workload == "window":
        wl, window = window_batch(W), WINDOW
    else:
        wl = {"mha-13b": W.config3, "prefix-cow": W.config4, "fp8-long": W.config5}[args.workload]()
    log(f"[bench] {args.workload} generated in {time.time() - t0:.1f}s: S={wl.num_seqs} "
        f"kv_bytes={wl.kv_bytes() / 1e9:.3f} GB")
    storage = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}

    def to_dev(a, dtype):
        a = np.ascontiguousarray(a)
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # pools: only the blocks some table (or copy pair) names carry data
    tables = wl.block_tables if wl.tables_before_copy is None else wl.tables_before_copy
    kp = torch.zeros(wl.k_pool.shape, dtype=storage[wl.kv_dtype], device=dev)
    vp = torch.zeros_like(kp)
    if wl.write_k is None:
        ids = np.unique(np.concatenate([tables[s, :-(-int(n) // wl.block_size)]
                                        for s, n in enumerate(wl.context_lens)]).astype(np.int64))
        if wl.copy_pairs is not None:
            ids = np.union1d(ids, wl.copy_pairs.ravel())
        it = torch.from_numpy(ids).to(dev)
        kp[it] = to_dev(wl.k_pool[ids], wl.kv_dtype)
        vp[it] = to_dev(wl.v_pool[ids], wl.kv_dtype)
    pool = pa.make_pool(kp, vp, dtype=wl.kv_dtype, k_scale=wl.k_scale, v_scale=wl.v_scale)
    if wl.write_k is not None:
        pa.pa_write_kv(to_dev(wl.write_k, wl.write_src_dtype), to_dev(wl.write_v, wl.write_src_dtype),
                       torch.from_numpy(wl.slot_mapping.astype(np.int64)).to(dev), pool,
                       src_dtype=wl.write_src_dtype)
    tb = torch.from_numpy(np.ascontiguousarray(tables, dtype=np.int32)).to(dev)
    if wl.copy_pairs is not None:
        pa.pa_copy_blocks(pool, torch.from_numpy(wl.copy_pairs.astype(np.int64)).to(dev))
        tb = torch.from_numpy(np.ascontiguousarray(wl.block_tables, dtype=np.int32)).to(dev)
    q = to_dev(wl.q, wl.q_dtype)
    ctx = torch.from_numpy(wl.context_lens.astype(np.int32)).to(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    kv_bytes = wl.kv_bytes()
    if window:
        # bytes the windowed decode reads: min(n, window) positions per sequence
        seen = np.minimum(wl.context_lens.astype(np.int64), window)
        kv_bytes = int(seen.sum()) * 2 * wl.num_kv_heads * wl.head_dim * W.ELEMENT_SIZE[wl.kv_dtype]
    parts = [-1, 0] + ([wl.partition_size] if wl.partition_size > 0 else [256])
    if args.partitions:
        parts = [int(x) for x in args.partitions.split(",")]
    cpu = None if args.no_cpu_baseline else decode_cpu_baseline(wl, window, W)
    for part in parts:
        ws = pa.new_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                              wl.max_blocks_per_seq, wl.block_size, part, device=dev) if part else None
        def call():
            if window:
                pa.pa_decode_window(q, pool, tb, ctx, window, wl.scale, out=out, partition_size=part,
                                    workspace=ws, q_dtype=wl.q_dtype, stream=stream)
            else:
                pa.pa_decode(q, pool, tb, ctx, wl.scale, out=out, partition_size=part, workspace=ws,
                             q_dtype=wl.q_dtype, stream=stream)

        for _ in range(max(args.warmup, 3)):
            call()
        steps = max(1, min(args.steps, 50))
        # the decode kernels alone: the event pair the call's launch records
        # as its first kernel begins and its last ends (as the main bench's
        # roofline); then, for reference, events on the stream around each call
        def timed_call(i, ev):
            pa.pa_time_next_decode(ev[0], ev[1])
            call()
        us = sorted(x * 1e3 for x in kernel_timed(torch, stream, steps, timed_call))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        call_us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        med = us[len(us) // 2]
        gbs = kv_bytes / (med * 1e-6) / 1e9
        assert bool(torch.isfinite(out.float()).all()), "non-finite output"
        print(json.dumps({
            "workload": args.workload, "partition_size": part, "kv_bytes": kv_bytes, "window": window,
            "kv_dtype": wl.kv_dtype, "num_seqs": wl.num_seqs, "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads, "block_size": wl.block_size,
            "decode_us": {"median": round(med, 2), "p10": round(us[len(us) // 10], 2),
                          "p90": round(us[(9 * len(us)) // 10], 2), "calls": steps,
                          "timing": "timing-only events the launch records as its kernels begin and end"},
            "call_us": {"median": round(call_us[len(call_us) // 2], 2), "p10": round(call_us[len(call_us) // 10], 2),
                        "p90": round(call_us[(9 * len(call_us)) // 10], 2),
                        "timing": "default events on the stream around the whole call"},
            "kv_gbs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "decode_tokens_per_s_per_layer": round(wl.num_seqs / (med * 1e-6), 1),
            "cache": "warm (fits the last-level cache)" if kv_bytes < (256 << 20) else "pools exceed the last-level cache",
            "cpu_baseline": cpu,
        }), flush=True)


# sliding-window batch: the 8B layer shape with long contexts and a window
# of 4096 positions (the decode reads min(n, 4096) positions per sequence)
WINDOW = 4096


def window_batch(W):
    import numpy as np
    rng = np.random.default_rng(9)
    lens = rng.integers(4096, 16385, size=32)
    need = int(sum(-(-int(n) // 16) for n in lens))
    return W.build_decode(9, name="window-4096-bf16", q_dtype="bf16", kv_dtype="bf16", num_q_heads=32,
                          num_kv_heads=8, head_dim=128, block_size=16, num_blocks=need + 64,
                          context_lens=lens, rng=rng)


MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak


def prefill_workload(args, pa, W, torch, dev):
    """pa_prefill on the 8B layer shape (bf16, 32 q heads on 8 KV heads, head
    dim 128, block 16).  "prefill": 16 whole prompts of 2048 positions;
    "prefill-chunk": 16 chunks of 512 queries after cached prefixes uniform
    in [0, 3584].  Work = the attended (query, key) pairs x query heads x 4 x
    head_dim flops (q.K^T and P.V, 2 each), against the dense bf16 peak."""
    import numpy as np
    rng = np.random.default_rng(13)
    S = 16
    if args.workload == "prefill":
        lens = np.full(S, 2048)
        qlens = lens.copy()
    else:
        qlens = np.full(S, 512)
        lens = rng.integers(0, 3585, size=S) + qlens
    need = int(sum(-(-int(n) // 16) for n in lens))
    wl = W.build_decode(13, name=args.workload, q_dtype="bf16", kv_dtype="bf16", num_q_heads=32, num_kv_heads=8,
                        head_dim=128, block_size=16, num_blocks=need + 16, context_lens=lens, rng=rng)
    T = int(qlens.sum())
    q_host = W.cast_f32(W.normal_f32(13, 9, T * 32 * 128), "bf16").reshape(T, 32, 128)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    kp, vp, q = bf16(wl.k_pool), bf16(wl.v_pool), bf16(q_host)
    pool = pa.make_pool(kp, vp)
    tb = torch.from_numpy(wl.block_tables.astype(np.int32)).to(dev)
    ctx = torch.from_numpy(lens.astype(np.int32)).to(dev)
    qs = torch.from_numpy(np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)).to(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    pairs = sum(int(sum(range(n - L + 1, n + 1))) for n, L in zip(lens, qlens))
    flops = pairs * 32 * 4 * 128
    for _ in range(max(args.warmup, 3)):
        pa.pa_prefill(q, pool, tb, ctx, qs, wl.scale, out=out, stream=stream)
    steps = max(3, min(args.steps, 30))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        pa.pa_prefill(q, pool, tb, ctx, qs, wl.scale, out=out, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    med = us[len(us) // 2]
    tflops = flops / (med * 1e-6) / 1e12
    assert bool(torch.isfinite(out.float()).all()), "non-finite output"
    cpu = None
    if not args.no_cpu_baseline:
        # the float64 oracle on the batch's first sequence, passes until ~5 s
        import oracle
        from threadpoolctl import threadpool_limits
        cores = len(os.sched_getaffinity(0))
        L0, n0 = int(qlens[0]), int(lens[0])
        pairs0 = sum(range(n0 - L0 + 1, n0 + 1))
        passes, total = 0, 0.0
        with threadpool_limits(limits=cores):
            threads = _oracle_threads(cores)
            while total < 5.0 and passes < 20:
                t0 = time.perf_counter()
                oracle.oracle_prefill(q_host[:L0], "bf16", wl.k_pool, wl.v_pool, "bf16", wl.block_tables[:1],
                                      lens[:1], np.array([0, L0]), wl.scale)
                total += time.perf_counter() - t0
                passes += 1
        cpu = {"value": round(pairs0 * 32 * 4 * 128 / (total / passes) / 1e12, 6), "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": f"{passes} passes of the batch's first sequence ({L0} queries over {n0} positions, "
                         f"float64 numpy), {total:.1f}s in total"}
    print(json.dumps({
        "workload": args.workload, "num_seqs": S, "query_rows": T, "context_tokens": int(lens.sum()),
        "attended_pairs": pairs, "flops": flops,
        "prefill_us": {"median": round(med, 1), "p10": round(us[len(us) // 10], 1),
                       "p90": round(us[(9 * len(us)) // 10], 1), "calls": steps},
        "tflops": round(tflops, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
        "frac_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "tokens_per_s_per_layer": round(T / (med * 1e-6), 1),
        "cpu_baseline": cpu,
    }), flush=True)


def swap_workload(args, pa, torch, dev):
    """pa_swap_blocks between the GPU pool and a pinned host swap area, both
    directions, on blocks of the 8B layer shape (8 KV heads x 16 x 128, bf16:
    32 KiB each of K and V), 4096 scattered blocks (256 MiB) per call; a plain
    contiguous copy of the same bytes between device and pinned host memory
    (the DMA engines) is timed beside it as the link's practical ceiling."""
    import numpy as np
    nb_dev, nb_host, moved = 16384, 4096, 4096
    kd = torch.zeros((nb_dev, 8, 16, 128), dtype=torch.bfloat16, device=dev)
    vd = torch.zeros_like(kd)
    kh = torch.zeros((nb_host, 8, 16, 128), dtype=torch.bfloat16, pin_memory=True)
    vh = torch.zeros_like(kh).pin_memory()
    gpu, host = pa.make_pool(kd, vd), pa.make_pool(kh, vh, host=True)
    rng = np.random.default_rng(11)
    out_pairs = np.stack([rng.permutation(nb_dev)[:moved], rng.permutation(nb_host)[:moved]], 1).astype(np.int64)
    in_pairs = out_pairs[:, ::-1].copy()
    po, pi = torch.from_numpy(out_pairs).to(dev), torch.from_numpy(in_pairs).to(dev)
    block_bytes = 2 * 8 * 16 * 128 * 2
    total = moved * block_bytes
    stream = torch.cuda.current_stream()
    flat_d = torch.empty(total, dtype=torch.uint8, device=dev)
    flat_h = torch.empty(total, dtype=torch.uint8, pin_memory=True)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        return us[len(us) // 2]

    reps = max(3, min(args.steps, 20))
    res = {}
    for name, fn in (("gpu_to_host", lambda: pa.pa_swap_blocks(gpu, host, po, stream=stream)),
                     ("host_to_gpu", lambda: pa.pa_swap_blocks(host, gpu, pi, stream=stream)),
                     ("dma_copy_gpu_to_host", lambda: flat_h.copy_(flat_d, non_blocking=True)),
                     ("dma_copy_host_to_gpu", lambda: flat_d.copy_(flat_h, non_blocking=True))):
        med = timed(fn, reps)
        res[name] = {"median_us": round(med, 1), "gbs": round(total / (med * 1e-6) / 1e9, 2)}
        log(f"[bench] swap {name}: {med:.1f} us")
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's block copy between host arrays of the two pools' shapes
        # (device pool to swap area), passes until about 5 s
        import oracle
        src_k = np.zeros((nb_dev, 8, 16, 128), dtype=np.uint16)
        src_v = np.zeros_like(src_k)
        dst_k = np.zeros((nb_host, 8, 16, 128), dtype=np.uint16)
        dst_v = np.zeros_like(dst_k)
        passes, spent = 0, 0.0
        while spent < 5.0 and passes < 200:
            t0 = time.perf_counter()
            oracle.oracle_swap(src_k, src_v, dst_k, dst_v, out_pairs)
            spent += time.perf_counter() - t0
            passes += 1
        cpu = {"value": round(total / (spent / passes) / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{passes} passes of the same {moved}-block copy between host arrays (numpy), "
                         f"{spent:.1f}s in total"}
    print(json.dumps({"workload": "swap", "blocks_per_call": moved, "bytes_per_call": total,
                      "block_bytes": block_bytes, "calls": reps, "results": res, "cpu_baseline": cpu}), flush=True)


def calibrate_copy(mib, pa, torch, dev):
    """pa_copy_blocks over MIB MiB of 64 KiB blocks (K and V 32 KiB each):
    a plain copy of known size for scaling the HBM byte counters."""
    import numpy as np
    block_elems = 8 * 16 * 128
    nblocks = max(2, (mib << 20) // (block_elems * 2 * 2))
    k = torch.zeros((2 * nblocks, 8, 16, 128), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    pool = pa.make_pool(k, v)
    pairs = torch.from_numpy(np.stack([np.arange(nblocks), np.arange(nblocks, 2 * nblocks)], 1)
                             .astype(np.int64)).to(dev)
    for _ in range(3):
        pa.pa_copy_blocks(pool, pairs)
    torch.cuda.synchronize()
    moved = nblocks * block_elems * 2 * 2
    print(json.dumps({"calibration": "pa_copy_blocks", "bytes_read_per_launch": moved,
                      "bytes_written_per_launch": moved, "launches": 3}), flush=True)


if __name__ == "__main__":
    main()
