"""Benchmark one decode step of paged attention on one MI355X.

A step is the whole hot path over one seeded synthetic batch: the new
tokens' K/V are scattered into their slots and every sequence's query attends
over its paged context. On the split path (every workload without a shared
prefix) both happen in pa_decode_split_append, whose partition launch stores
each new row and attends to it, then the merge; with --unfused, or with a
shared prefix, pa_reshape_and_cache runs first as its own launch. Inputs are resident in HBM
before timing starts; the timed loop cycles through copies of the batch whose
blocks sit at different physical places, so no step re-reads the previous
step's blocks out of the 256 MB last-level cache.

Prints one JSON line. `value` is KV GB/s: the step's algorithmic bytes
(Σ context_len · 2·Hkv·D·e for K and V, plus q, the output, the block-table
entries used, the context lengths and the cache write) over the measured
step time. The line also carries the dominant launch's roofline (against the
8 TB/s peak and against a measured streaming-read ceiling), the p10/p50/p90
of single steps, the standalone scatter's time and bandwidth, and the CPU
oracle's throughput on a bounded sample of the same batch.

    python bench.py [--steps K] [--warmup W] [--workload llama13b]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 matrix-core peak of MI355X
LLC_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--path", choices=["auto", "decode", "split", "split_prefix"], default="auto")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--block-size", type=int, default=None,
                    help="re-block the workload (same tokens and cache bytes, other block size)")
    ap.add_argument("--head-dim", type=int, default=None,
                    help="the workload with another head_dim (same tokens and heads)")
    ap.add_argument("--unfused", action="store_true",
                    help="split path: run the scatter as its own launch instead of inside the "
                         "partition launch (pa_decode_split_append)")
    ap.add_argument("--out-dtype", choices=["native", "f32"], default="native")
    ap.add_argument("--rotations", type=int, default=0, help="batch copies cycled (0 = auto)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--lens", default=None,
                    help="override the context-length recipe (e.g. fixed:1094); not the headline")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="CPU time of the oracle baseline: 3 samples with every core's BLAS "
                         "threads and 3 with one thread share it (0 disables it)")
    ap.add_argument("--loops", type=int, default=5,
                    help="timed loops of K steps: the first is the headline, the median of all "
                         "is reported next to it")
    ap.add_argument("--op", choices=["decode", "copy_blocks", "swap_blocks", "prefill"],
                    default="decode",
                    help="decode: the decode step (default); copy_blocks: the copy-on-write "
                         "block copy on the workload's cache shape; swap_blocks: blocks to "
                         "pinned host memory and back; prefill: the prefill after a prefix-cache "
                         "hit (workloads prefix_prefill, prefix_prefill_gqa, prefill_tiny)")
    ap.add_argument("--prefill-entry", choices=["auto", "shared", "plain"], default="auto",
                    help="prefill: pa_prefill_shared_prefix over the cached prompt every request "
                         "shares (auto: when the workload has one) or plain pa_prefill")
    ap.add_argument("--pairs", type=int, default=1024, help="copy_blocks: block pairs per launch")
    ap.add_argument("--ceiling-gib", type=float, default=4.0,
                    help="buffer size of the streaming-read ceiling measurement (0 skips it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB 5 times (counter calibration)")
    return ap.parse_args()


def source_digest():
    """Digest of the kernel sources; stored counter readings are valid only
    for the sources they were taken on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_138_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*"))):
        if f.endswith((".hip", ".h")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(key):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE runs recorded
    in profiles/traffic.json, or None if absent or taken on other sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(mib):
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def pick_workload(args):
    """The named workload, with --lens, --block-size and --head-dim applied."""
    import dataclasses
    from paged_kv_cache_138_amd import workloads as W
    w = W.WORKLOADS[args.workload]
    if args.lens:
        w = dataclasses.replace(w, lens=args.lens, name=w.name + "+lens=" + args.lens)
    if args.block_size and args.block_size != w.block_size:
        bs, old = args.block_size, w.block_size
        tokens, per_seq = w.num_blocks * old, w.max_blocks_per_seq * old
        if tokens % bs or per_seq % bs or w.shared_prefix_tokens % bs:
            raise SystemExit("block size %d does not divide the workload's pool and tables" % bs)
        w = dataclasses.replace(w, block_size=bs, num_blocks=tokens // bs,
                                max_blocks_per_seq=per_seq // bs,
                                name=w.name + "+bs=%d" % bs)
    if args.head_dim and args.head_dim != w.head_dim:
        w = dataclasses.replace(w, head_dim=args.head_dim, name=w.name + "+d=%d" % args.head_dim)
    return w


def default_path(workload):
    # measured on MI355X: the split path (partitions of the workload's
    # partition size, then the merge) beats the single launch on every
    # workload: long sequences no longer end the launch alone; a batch whose
    # sequences share a prefix computes the prefix partitions once per 128 rows
    return "split_prefix" if workload.shared_prefix_tokens else "split"


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        return "?"


def _host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _oracle_decode_sample(batch, kc, vc, target_s):
    """Oracle decode of the batch's sequences, cycled in order, until
    target_s seconds of it have run. Returns (seconds, sequences, KV bytes)."""
    import oracle
    from paged_kv_cache_138_amd import workloads as W
    w = batch.workload
    B = len(batch.context_lens)
    bytes_per_tok = 2 * w.num_kv_heads * w.head_dim * W.element_bytes(w.dtype)
    elapsed, seqs, nbytes = 0.0, 0, 0
    while elapsed < target_s and seqs < 64 * B:
        s = seqs % B
        sl = slice(s, s + 1)
        t1 = time.perf_counter()
        oracle.decode(batch.query[sl], kc, vc, batch.block_tables[sl], batch.context_lens[sl],
                      batch.scale, w.dtype)
        elapsed += time.perf_counter() - t1
        nbytes += int(batch.context_lens[s]) * bytes_per_tok
        seqs += 1
    return elapsed, seqs, nbytes


def cpu_baseline(batch, target_s):
    """Time the fp64 CPU oracle on bounded samples of the same step: three
    samples with the BLAS threads of every core this process may run on and
    three with one thread, each about target_s / 6 seconds; the medians are
    reported (the all-cores one as `value`)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    w = batch.workload
    # the step's cache write first (not timed): the oracle attends over the
    # caches with the new rows in place
    t0 = time.perf_counter()
    kc, vc = oracle.reshape_and_cache(batch.new_key, batch.new_value, batch.key_cache,
                                      batch.value_cache, batch.slot_mapping)
    t_write = time.perf_counter() - t0
    cores = _host_cores()
    runs = {}
    for threads in (cores, 1):
        lim = threadpool_limits(limits=threads) if threadpool_limits else None
        samples = [_oracle_decode_sample(batch, kc, vc, target_s / 6.0) for _ in range(3)]
        if lim is not None:
            lim.unregister()
        gbs = sorted(nb / el / 1e9 for el, _, nb in samples)
        sps = sorted(n / el for el, n, _ in samples)
        runs[threads] = (gbs[1], sps[1], samples)
    med, med_sps, samples = runs[cores]
    one, one_sps, one_samples = runs[1]
    desc = lambda smp: ", ".join("%d seqs / %.1f s" % (n, el) for el, n, _ in smp)
    return {"value": round(med, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": "oracle decode (fp64) of the %s batch's sequences in order, all %d heads, "
                      "with the cache write done first (%.2f s, not counted); median of 3 samples "
                      "with %d BLAS threads (%s) and of 3 with 1 thread (%s)"
                      % (w.name, w.num_heads, t_write, cores, desc(samples), desc(one_samples)),
            "seq_tokens_per_s": round(med_sps, 3),
            "one_thread": {"value": round(one, 4), "unit": "GB/s", "cores": 1,
                           "seq_tokens_per_s": round(one_sps, 3)}}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.op == "copy_blocks":
        bench_copy_blocks(args)
        return
    if args.op == "swap_blocks":
        bench_swap_blocks(args)
        return
    if args.op == "prefill":
        bench_prefill(args)
        return
    import numpy as np
    import torch
    from paged_kv_cache_138_amd import lib as palib
    from paged_kv_cache_138_amd import workloads as W
    from paged_kv_cache_138_amd.pipeline import DeviceBatch, RotatedBatch

    palib.load()  # fails loudly if libpa.so is missing
    w = pick_workload(args)
    path = default_path(w) if args.path == "auto" else args.path
    t_gen = time.perf_counter()
    batch = W.make_batch(w, seed=args.seed)
    t_gen = time.perf_counter() - t_gen
    out_dtype = torch.float32 if args.out_dtype == "f32" else None
    # all GPU work runs on one dedicated stream of default priority; the
    # legacy default stream adds a few microseconds of synchronisation per step
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        base = DeviceBatch(batch, out_dtype=out_dtype, split=path.startswith("split"),
                           partition_size=args.partition_size,
                           shared_prefix=(path == "split_prefix"),
                           fused=(path == "split" and not args.unfused))
        fused = base.fused
        unique_bytes, logical_bytes = W.step_bytes(batch, None if out_dtype is None else "f32")
        write_bytes = W.cache_write_bytes(batch)
        # rotation copies: enough that the cycle's footprint is >= 8x the LLC
        kv_block = 2 * base.key_cache[0].numel() * base.key_cache.element_size()
        footprint = kv_block * len(batch.allocated_blocks)
        R = args.rotations or max(2, min(16, -(-8 * LLC_BYTES // max(footprint, 1))))
        copies = [RotatedBatch(base, seed=1000 + r) for r in range(R)]
        del base
        torch.cuda.synchronize()

        # all copies must agree bit for bit (same logical data, different placement)
        copies[0].step()
        torch.cuda.synchronize()
        ref = copies[0].out.clone()
        for c in copies[1:]:
            c.step()
        torch.cuda.synchronize()
        for c in copies[1:]:
            assert torch.equal(c.out.view(torch.int16) if c.out.dtype != torch.float32 else c.out,
                               ref.view(torch.int16) if ref.dtype != torch.float32 else ref), \
                "rotated copies disagree"
        # the streaming-read ceiling is measured right before the warm-up
        # steps: its saturating reads (about 8 ms) bring the device from the
        # idle of the host-side checks above to its working clocks, which
        # otherwise take the first 10 ms or so of steps to reach (those ran
        # 1.5-2.5% slower); the warm-up steps then find the batch copies'
        # address translations again
        ceiling = stream_ceiling(args.ceiling_gib) if args.ceiling_gib > 0 else None
        # the warm-up steps, right before the timed loops
        for k in range(args.warmup):
            copies[k % R].step()
        torch.cuda.synchronize()
        K = args.steps
        split = path.startswith("split")
        loop_ms = []
        for _ in range(max(1, args.loops)):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(K):
                copies[k % R].step()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            loop_ms.append((t1 - t0) * 1e3 / K)
        ms_per_step = loop_ms[0]  # the headline: exactly K timed steps
        # the dominant kernel alone: K back-to-back launches between two HIP events
        # on the launch stream (pa_decode, or the partition launch of the split path)
        dom = (lambda c: c.partitions()) if split else (lambda c: c.attend())
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(K):
            dom(copies[k % R])
        e1.record()
        torch.cuda.synchronize()
        attn_avg_ms = e0.elapsed_time(e1) / K
        if split:  # leave every copy's output complete
            for c in copies:
                c.merge()
            torch.cuda.synchronize()
        # the spread of single steps (each between its own events; separate
        # from the timed loop above, whose mean is the headline)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        for k in range(K):
            ev[k][0].record()
            copies[k % R].step()
            ev[k][1].record()
        torch.cuda.synchronize()
        single = sorted(a.elapsed_time(b) for a, b in ev)
        pct = lambda q: single[min(K - 1, int(round(q * (K - 1))))]
        # the scatter alone: K pa_reshape_and_cache launches recorded in a HIP
        # graph and replayed, so the host's per-call cost stays out of the
        # GPU time (each launch is a few microseconds of GPU work)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(K):
                copies[k % R].write_cache()
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        scatter_ms = e0.elapsed_time(e1) / K
        del graph
    # `value` counts the attention's algorithmic bytes (K/V rows read, q, the
    # table entries and lengths read, the output written); the step's cache
    # write of the new rows is reported on its own
    gbs = unique_bytes / (ms_per_step * 1e-3) / 1e9
    kv_bytes = W.kv_read_bytes(batch)
    attn_gbs = unique_bytes / (attn_avg_ms * 1e-3) / 1e9
    loop_sorted = sorted(loop_ms)
    median_ms = loop_sorted[len(loop_sorted) // 2]
    B = len(batch.context_lens)
    res = {
        "metric": "paged decode attn: KV GB/s (% HBM peak) + seq-tokens/s, LLaMA-13B shape",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "num_seqs": B,
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "sum_context_lens": int(batch.context_lens.sum()),
                   "path": path, "fused_append": fused,
                   "partition_size": base_partition(path, args, w),
                   "out_dtype": args.out_dtype, "rotations": R, "seed": args.seed},
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "kv_read_frac": round(kv_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "loops_ms_per_step": [round(x, 5) for x in loop_ms],
        "median_loop": {"ms_per_step": round(median_ms, 5),
                        "GB_per_s": round(unique_bytes / (median_ms * 1e-3) / 1e9, 2),
                        "hbm_peak_frac": round(unique_bytes / (median_ms * 1e-3) / 1e9
                                               / HBM_PEAK_GBS, 4)},
        "seq_tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "context_tokens_per_s": round(int(batch.context_lens.sum()) / (ms_per_step * 1e-3), 1),
        "step_bytes": {"attention_unique": unique_bytes, "attention_logical": logical_bytes,
                       "kv_read": kv_bytes, "cache_write": write_bytes},
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(traffic_key(w.name, path, fused)),
                     "kernel": "%s: %d back-to-back launches between HIP events, avg %.2f us"
                               % ("pa_decode_partitions_append" if fused else
                                  {"split": "pa_decode_partitions", "decode": "pa_decode",
                                   "split_prefix": "pa_decode_partitions_shared_prefix (prefix "
                                                   "and suffix kernels)"}[path], K,
                                  attn_avg_ms * 1e3)},
        "host_data_generation_s": round(t_gen, 2),
        "step_ms_p10_p50_p90": [round(pct(0.1), 5), round(pct(0.5), 5), round(pct(0.9), 5)],
        "reshape_and_cache": {"us_per_call": round(scatter_ms * 1e3, 2), "tokens": B,
                              "timing": "%d launches replayed from one HIP graph" % K,
                              "bytes": write_bytes,
                              "GB_per_s": round(write_bytes / (scatter_ms * 1e-3) / 1e9, 2)},
    }
    if ceiling is not None:
        res["stream_read_ceiling"] = dict(ceiling, attention_frac_of_ceiling=round(
            attn_gbs / ceiling["value"], 4))
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def traffic_key(name, path, fused):
    return "%s/%s%s" % (name, path, "+append" if fused else "")


def bench_copy_blocks(args):
    """Copy-on-write block copy on the workload's cache shape: --pairs random
    (src, dst) pairs per launch, two disjoint pair sets alternating so no
    launch finds its source blocks in the last-level cache. Bytes per launch
    = pairs x block bytes x 2 caches x (read + write)."""
    import numpy as np
    import torch
    from paged_kv_cache_138_amd import lib as palib
    from paged_kv_cache_138_amd import workloads as W
    w = pick_workload(args)
    NB, BS, Hkv, D = w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    N = min(args.pairs, NB // 4)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        kc = torch.empty((NB, BS, Hkv, D), dtype=tdt, device="cuda").normal_()
        vc = torch.empty_like(kc).normal_()
        perm = np.random.default_rng(args.seed).permutation(NB)
        # set r copies perm[2rN : 2rN + N] onto perm[2rN + N : 2(r + 1)N]
        maps = [torch.from_numpy(np.stack([perm[2 * r * N: 2 * r * N + N],
                                           perm[2 * r * N + N: 2 * (r + 1) * N]], axis=1)
                                 .astype(np.int64)).cuda() for r in range(2)]
        for m in maps:
            palib.copy_blocks(kc, vc, m)
        torch.cuda.synchronize()
        K = args.steps
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(K):
            palib.copy_blocks(kc, vc, maps[k % 2])
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
    block_bytes = BS * Hkv * D * W.element_bytes(w.dtype)
    nbytes = N * block_bytes * 2 * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"metric": "copy-on-write block copy: HBM GB/s (read + write)", "value": round(gbs, 2),
           "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": 1, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": "synthetic",
           "config": {"workload": w.name, "op": "copy_blocks", "pairs": N, "block_bytes": block_bytes},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "pa_copy_blocks: %d launches between HIP events, avg %.2f us"
                                  % (K, ms * 1e3)}}
    if args.cpu_seconds > 0:
        import oracle
        sample = max(1, min(N, 64))
        kh = np.zeros((2 * sample, BS, Hkv, D), dtype=np.uint16)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            oracle.copy_blocks(kh, kh, np.stack([np.arange(sample), sample + np.arange(sample)], 1))
            reps += 1
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(reps * sample * block_bytes * 2 * 2 / el / 1e9, 3),
                               "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": "%d runs of %d pairs (whole-cache copies included)"
                                         % (reps, sample)}
    print(json.dumps(res), flush=True)


def bench_prefill(args):
    """The prefill step after a prefix-cache hit: the new tokens' K/V stored
    by pa_reshape_and_cache, then the attention over the cached prompt
    blocks and the new tokens: pa_prefill_shared_prefix when every request's
    table starts with the same cached prompt blocks (the workload's shared
    system prompt, declared as shared_prefix_tokens), else pa_prefill. The
    attention is a matrix-core contraction: its roofline is the dense
    fp16/bf16 MFMA peak, by the exact causal flop count."""
    import numpy as np
    import torch
    from paged_kv_cache_138_amd import lib as palib
    from paged_kv_cache_138_amd import workloads as W
    from paged_kv_cache_138_amd.pipeline import DevicePrefill

    palib.load()
    name = args.workload if args.workload in W.PREFILL_WORKLOADS else "prefix_prefill"
    w = W.PREFILL_WORKLOADS[name]
    t_gen = time.perf_counter()
    batch = W.make_prefill_batch(w, seed=args.seed)
    t_gen = time.perf_counter() - t_gen
    flops = W.prefill_flops(batch)
    out_dtype = torch.float32 if args.out_dtype == "f32" else None
    unique_bytes, request_bytes = W.prefill_bytes(batch, "f32" if out_dtype is not None else None)
    shared = (args.prefill_entry == "shared" or
              (args.prefill_entry == "auto" and w.cached_tokens > 0))
    ps = w.cached_tokens if shared else None
    entry = "pa_prefill_shared_prefix" if shared else "pa_prefill"
    stream = torch.cuda.Stream()
    K = args.steps
    with torch.cuda.stream(stream):
        db = DevicePrefill(batch, out_dtype=out_dtype, shared_prefix_tokens=ps)
        for _ in range(max(args.warmup, 1)):
            db.step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # the attention launch of every step between its own pair of events
        # (on the stream it runs on), as it runs in the step: after the
        # scatter
        ea = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        eb = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        t0 = time.perf_counter()
        e0.record()
        for i in range(K):
            db.write_cache()
            ea[i].record()
            db.attend()
            eb[i].record()
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / K
        ms = e0.elapsed_time(e1) / K
        attn_ms = sum(a.elapsed_time(b) for a, b in zip(ea, eb)) / K
    tflops = flops / (ms * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    T = int(batch.query_start[-1])
    res = {
        "metric": "paged prefill attn after a prefix-cache hit: TFLOP/s (causal flops)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "op": "prefill",
                   "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "cached_tokens": w.cached_tokens,
                   "new_tokens": T, "max_query_len": batch.max_query_len,
                   "entry": entry, "shared_prefix_tokens": ps or 0,
                   "out_dtype": args.out_dtype, "seed": args.seed},
        "step_wall_ms": round(wall, 5),
        "new_tokens_per_s": round(T / (ms * 1e-3), 1),
        "attention_flops": flops,
        "attention_bytes": {"unique": unique_bytes, "per_request": request_bytes,
                            "unique_GB_per_s": round(unique_bytes / (attn_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MFMA_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic("%s/%s" % (w.name, "prefill_shared" if shared
                                                          else "prefill")),
                     "kernel": "%s: the %d timed steps' launches, each between HIP events, "
                               "avg %.2f us" % (entry, K, attn_ms * 1e3)},
        "host_data_generation_s": round(t_gen, 2),
    }
    if args.cpu_seconds > 0:
        import oracle
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(limits=1)
        except Exception:  # pragma: no cover
            limiter = None
        kc, vc = oracle.reshape_and_cache(batch.new_key, batch.new_value, batch.key_cache,
                                          batch.value_cache, batch.slot_mapping)
        qs = batch.query_start
        t0 = time.perf_counter()
        done_flops = 0
        n = 0
        while time.perf_counter() - t0 < args.cpu_seconds and n < len(batch.context_lens):
            rows = np.arange(qs[n], qs[n + 1])
            sub = W.PrefillBatch(w, batch.query[rows], None, None, batch.block_tables[n:n + 1],
                                 batch.context_lens[n:n + 1],
                                 np.array([0, len(rows)], dtype=np.int32), None, None, None,
                                 batch.scale, batch.shared_blocks)
            oracle.prefill(sub.query, kc, vc, sub.block_tables, sub.context_lens,
                           sub.query_start, batch.scale, batch.dtype)
            done_flops += W.prefill_flops(sub)
            n += 1
        el = time.perf_counter() - t0
        if limiter is not None:
            limiter.unregister()
        res["cpu_baseline"] = {"value": round(done_flops / el / 1e12, 6), "unit": "TFLOP/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "oracle.prefill (fp64, one thread) of the first %d "
                                         "requests, %.1f s" % (n, el)}
    print(json.dumps(res), flush=True)


def bench_swap_blocks(args):
    """Swap --pairs random blocks of the workload's cache shape to a pinned
    host pool (swap-out) and back (swap-in), each as one pa_swap_blocks
    launch, against the host link's measured ceiling: a DMA copy of a 1 GiB
    pinned buffer in the same direction."""
    import numpy as np
    import torch
    from paged_kv_cache_138_amd import lib as palib
    from paged_kv_cache_138_amd import workloads as W
    w = pick_workload(args)
    NB, BS, Hkv, D = w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    N = min(args.pairs, NB // 2)
    K = max(1, min(args.steps, 10))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        kc = torch.empty((NB, BS, Hkv, D), dtype=tdt, device="cuda").normal_()
        vc = torch.empty_like(kc).normal_()
        hk = torch.empty((N, BS, Hkv, D), dtype=tdt).pin_memory()
        hv = torch.empty_like(hk).pin_memory()
        perm = np.random.default_rng(args.seed).permutation(NB)
        out_map = torch.from_numpy(np.stack([perm[:N], np.arange(N)], 1).astype(np.int64)).cuda()
        in_map = torch.from_numpy(np.stack([np.arange(N), perm[N:2 * N]], 1).astype(np.int64)).cuda()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(K):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / K

        ms_out = timed(lambda: palib.swap_blocks(hk, hv, kc, vc, out_map))
        ms_in = timed(lambda: palib.swap_blocks(kc, vc, hk, hv, in_map))
        big_d = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        big_h = torch.empty(1 << 30, dtype=torch.uint8).pin_memory()
        dma_d2h = timed(lambda: big_h.copy_(big_d, non_blocking=True))
        dma_h2d = timed(lambda: big_d.copy_(big_h, non_blocking=True))
    block_bytes = BS * Hkv * D * W.element_bytes(w.dtype)
    nbytes = N * block_bytes * 2
    g = lambda b, ms: round(b / (ms * 1e-3) / 1e9, 2)
    out_gbs, in_gbs = g(nbytes, ms_out), g(nbytes, ms_in)
    ceil_out, ceil_in = g(1 << 30, dma_d2h), g(1 << 30, dma_h2d)
    res = {"metric": "swap blocks to pinned host memory and back: host-link GB/s",
           "value": round((out_gbs + in_gbs) / 2, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
           "warmup": 1, "ms_per_step": round(ms_out + ms_in, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
           "config": {"workload": w.name, "op": "swap_blocks", "pairs": N, "block_bytes": block_bytes},
           "swap_out_GB_per_s": out_gbs, "swap_in_GB_per_s": in_gbs,
           "roofline": {"bound": "host_link", "achieved": round((out_gbs + in_gbs) / 2, 2),
                        "peak": round((ceil_out + ceil_in) / 2, 2), "unit": "GB/s",
                        "frac": round((out_gbs + in_gbs) / (ceil_out + ceil_in), 4), "traffic": None,
                        "peak_is": "measured DMA copy of 1 GiB pinned <-> device (%.1f out, %.1f in GB/s)"
                                   % (ceil_out, ceil_in),
                        "kernel": "pa_swap_blocks: %d launches each way, avg %.1f / %.1f us"
                                  % (K, ms_out * 1e3, ms_in * 1e3)}}
    print(json.dumps(res), flush=True)


def stream_ceiling(gib):
    """Measured streaming-read ceiling: pa_stream_read over a buffer of `gib`
    GiB (far larger than the last-level cache), 2 warm-up and 10 timed
    launches between HIP events."""
    import torch
    from paged_kv_cache_138_amd import lib as palib
    nbytes = int(gib * (1 << 30)) // 16 * 16
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    for _ in range(2):
        palib.stream_read(buf, sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        palib.stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del buf
    return {"value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "buffer_bytes": nbytes,
            "kernel": "pa_stream_read (16-byte non-temporal loads)"}


def base_partition(path, args, w):
    if not path.startswith("split"):
        return None
    return args.partition_size or w.partition_size


if __name__ == "__main__":
    main()
