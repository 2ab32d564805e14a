"""Benchmark of the paged-attention decode step on one MI355X.

One step = the hot path over one batch of the Llama-3-8B-shape decode
workload (64 sequences, lengths uniform in [512, 4096], 32 query / 8 KV
heads, head size 128, block 16, bf16): each sequence's new token written
into its slot and the decode over every token.  By default that is one
``pa_decode_append`` call (the write happens inside the split-K decode
kernel, then the log-sum-exp reduce kernel); ``--two-calls`` times it as
``pa_cache_write`` + ``pa_decode``, whose time is reported beside it either
way.  Inputs are resident in HBM before timing starts.  Three
independent copies of the K/V pools are rotated step by step so that each
step streams its K/V from HBM rather than from the 256 MB last-level cache.

Prints ONE JSON line (rank 0):
  value       effective decode K/V read rate, GB/s (algorithmic K/V bytes of
              the step / step time; bytes = sum(seq_lens) x 4096)
  roofline    the step's decode kernel alone, timed with HIP events the
              library records around its launch: algorithmic bytes / average
              duration against the 8 TB/s HBM3E peak (and the same for the
              whole call, decode kernel + reduce kernel)
  cpu_baseline  the float64 CPU oracle on the same workload (test
              infrastructure, timed on the host cores)
  rows        event timings of the other rows of the path (long-context
              split-K, copy-on-write copy, shared prefix, fp8 decode and
              cache write, fp8 prefill chunk, the mixed step, pool blocks of
              64 and 128 tokens, chunked-prefill budget steps, the host block
              manager, swap to pinned host memory, prefix caching)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--no-rows | --rows-only GROUP] [--cpu-budget SECONDS]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode KV GB/s (% HBM peak) + tokens/s, Llama-3-8B shape bs=64, 1 GPU"
DEFAULT_WORKLOAD = "llama3_8b_decode_bf16"
N_SETS = 3


def kernel_source_digest() -> str:
    """Digest of the decode kernel sources (and the engine and worker-count
    choice in the C ABI), to tie stored counter data to code."""
    h = hashlib.sha256()
    for f in ("decode_impl.h", "decode_mfma.h", "pa_device.h", "pa_api.hip"):
        with open(os.path.join(ROOT, "paged_kv_cache_11_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes (read + written) per launch of the balanced decode kernel,
    from committed rocprofv3 counter runs, or None if they were taken on
    other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"decode_kernel_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_digest") != kernel_source_digest():
        return None
    k = d.get("kernels", {}).get("decode_balanced")
    return round(k["fetch_bytes"] + k["write_bytes"]) if k else None


def summarize_counters(fetch_csv: str, write_csv: str, workload: str, out_path: str) -> dict:
    """Turn two rocprofv3 --pmc runs of this bench (FETCH_SIZE, then
    WRITE_SIZE, both with --copy-calibration-mib) into HBM bytes per
    pa_decode call.  Each counter is scaled by the ratio of the bytes the
    calibration copy (pa_copy_blocks) really moved to what the counter read
    for it; the decode call's kernels are the balanced decode kernel and its
    reduce kernel."""
    import csv
    import statistics

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return acc

    f, w = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_name = next(k for k in f if "move_blocks_kernel" in k)
    # The calibration copy reads and writes 256 MiB (K and V halves).
    true_bytes = 256.0 * (1 << 20)
    f_scale = true_bytes / statistics.mean(f[copy_name])
    w_scale = true_bytes / statistics.mean(w[copy_name])
    parts = {}
    for tag in ("decode_balanced", "balanced_reduce"):
        kf = next(k for k in f if tag in k)
        kw = next(k for k in w if tag in k)
        parts[tag] = {"fetch_bytes": statistics.median(f[kf]) * f_scale,
                      "write_bytes": statistics.median(w[kw]) * w_scale}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in parts.values())
    d = {"workload": workload, "source_digest": kernel_source_digest(),
         "fetch_scale": f_scale, "write_scale": w_scale, "kernels": parts,
         "hbm_bytes_per_launch": round(total)}
    with open(out_path, "w") as fh:
        json.dump(d, fh, indent=1)
    return d


def cpu_baseline(b, budget_s: float = 12.0):
    """Time the float64 CPU oracle (test infrastructure) on this workload:
    build its pool with its cache write, then run its decode over the
    sequences, repeating whole passes until the time budget is spent."""
    from oracle import paged as opg
    from paged_kv_cache_11_amd import workloads as wl

    try:
        import threadpoolctl

        blas_threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()),
                           default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    kp = wl.poisoned_pool(b.num_blocks, b.num_kv_heads, b.block_size, b.head_size, b.kv_dtype)
    vp = wl.poisoned_pool(b.num_blocks, b.num_kv_heads, b.block_size, b.head_size, b.kv_dtype)
    ks = wl.storage_bits(wl.storage_tensor(b.k, b.kv_src_dtype))
    vs = wl.storage_bits(wl.storage_tensor(b.v, b.kv_src_dtype))
    opg.cache_write(kp, vp, b.kv_dtype, ks, vs, b.kv_src_dtype, b.slot_mapping, b.k_scale,
                    b.v_scale)
    q64 = wl.storage_tensor(b.q, b.q_dtype).float().numpy().astype(np.float64)
    seqs_done, tokens_read, t0, c0 = 0, 0, time.perf_counter(), time.process_time()
    while seqs_done < b.num_seqs or time.perf_counter() - t0 < budget_s:
        s = seqs_done % b.num_seqs
        opg.paged_decode(q64, kp, vp, b.block_tables, b.seq_lens, b.scale, kv_dtype=b.kv_dtype,
                         k_scale=b.k_scale, v_scale=b.v_scale, seqs=[s])
        seqs_done += 1
        tokens_read += int(b.seq_lens[s])
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    cpu = time.process_time() - c0
    return {
        "value": seqs_done / dt, "unit": "tokens/s", "cores": round(cpu / dt, 1),
        "kind": "oracle", "gbs": tokens_read * b.kv_bytes_per_token() / dt / 1e9,
        "sample": f"{seqs_done} sequence decodes of the same workload ({tokens_read} cached tokens "
                  f"read) in {dt:.1f} s; cores = process CPU time / wall time ({cpu:.1f} s / "
                  f"{dt:.1f} s), numpy BLAS pool {blas_threads} threads, host has "
                  f"{os.cpu_count()} logical cpus",
    }


def oracle_rows(budget_s: float = 2.5):
    """The oracle (test infrastructure) timed on each workload of the path,
    on a bounded sample of it (about budget_s seconds each): decode of a few
    sequences of the tiny, Llama-3-8B-shape, long-context, shared-prefix and
    fp8 70B-shape workloads, and prefill of a slice of the fp8 chunk's
    queries.  Rates are per sampled unit; cores = CPU time / wall time."""
    from oracle import paged as opg
    from paged_kv_cache_11_amd import workloads as wl

    rows = {}

    def pools(b):
        kp = wl.poisoned_pool(b.num_blocks, b.num_kv_heads, b.block_size, b.head_size, b.kv_dtype)
        vp = wl.poisoned_pool(b.num_blocks, b.num_kv_heads, b.block_size, b.head_size, b.kv_dtype)
        ks = wl.storage_bits(wl.storage_tensor(b.k, b.kv_src_dtype))
        vs = wl.storage_bits(wl.storage_tensor(b.v, b.kv_src_dtype))
        opg.cache_write(kp, vp, b.kv_dtype, ks, vs, b.kv_src_dtype, b.slot_mapping, b.k_scale,
                        b.v_scale)
        return kp, vp

    for name in ("tiny_fp32", "llama3_8b_decode_bf16", "long_context_splitk_bf16",
                 "shared_prefix_bf16", "mixed_prefill_decode_fp8"):
        b = wl.make(name)
        kp, vp = pools(b)
        q64 = wl.storage_tensor(b.q, b.q_dtype).float().numpy().astype(np.float64)
        done, toks, t0, c0 = 0, 0, time.perf_counter(), time.process_time()
        while done < b.num_seqs and (done == 0 or time.perf_counter() - t0 < budget_s):
            opg.paged_decode(q64, kp, vp, b.block_tables, b.seq_lens, b.scale,
                             kv_dtype=b.kv_dtype, k_scale=b.k_scale, v_scale=b.v_scale,
                             seqs=[done])
            toks += int(b.seq_lens[done])
            done += 1
        dt, cpu = time.perf_counter() - t0, time.process_time() - c0
        rows[name] = {"kind": "oracle", "op": "paged_decode", "sample_seqs": done,
                      "of_seqs": b.num_seqs, "s": round(dt, 3),
                      "tokens_per_s": round(done / dt, 2),
                      "gbs": round(toks * b.kv_bytes_per_token() / dt / 1e9, 4),
                      "cores": round(cpu / dt, 1)}
        if name == "mixed_prefill_decode_fp8":
            # Prefill of the first queries of the 512-query chunk.
            n = 16
            qc = wl.storage_tensor(b.chunk_q, "bf16").float().numpy().astype(np.float64)
            t0, c0 = time.perf_counter(), time.process_time()
            L = int(b.chunk_seq_lens[0])
            opg.paged_prefill(qc[:n], np.array([0, n], np.int32), kp, vp, b.chunk_block_tables,
                              np.array([L - len(qc) + n], np.int32), b.scale, kv_dtype=b.kv_dtype,
                              k_scale=b.k_scale, v_scale=b.v_scale)
            dt, cpu = time.perf_counter() - t0, time.process_time() - c0
            rows[name + "_prefill"] = {"kind": "oracle", "op": "paged_prefill",
                                       "sample_queries": n, "of_queries": len(qc),
                                       "s": round(dt, 3), "queries_per_s": round(n / dt, 2),
                                       "cores": round(cpu / dt, 1)}
    return rows

MFMA_BF16_PEAK_TFLOPS = 2500.0
# PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes, 128b/130b coding.
HOST_LINK_PEAK_GBS = 63.0


def _gpu_pools(b, dev, copies=1):
    """K/V pools filled through pa_cache_write (plus extra copies on the GPU)."""
    import torch

    from paged_kv_cache_11_amd import binding as pa
    from paged_kv_cache_11_amd import workloads as wl

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[b.kv_dtype]
    shape = (b.num_blocks, b.num_kv_heads, b.block_size, b.head_size)
    k0 = torch.zeros(shape, dtype=tdt, device=dev)
    v0 = torch.zeros(shape, dtype=tdt, device=dev)
    chunk = 1 << 16
    for a in range(0, len(b.slot_mapping), chunk):
        pa.pa_cache_write(wl.storage_tensor(b.k[a:a + chunk], b.kv_src_dtype).to(dev),
                          wl.storage_tensor(b.v[a:a + chunk], b.kv_src_dtype).to(dev), k0, v0,
                          torch.from_numpy(b.slot_mapping[a:a + chunk]).to(dev), b.k_scale,
                          b.v_scale)
    return [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]


def _time_us(fn, iters, warmup=3):
    """Average duration of fn(i) over iters calls, HIP events on the current stream."""
    import torch

    for i in range(warmup):
        fn(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(iters):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters * 1e3


def _kernel_us(fn, iters, warmup=3):
    """Mean duration of the main decode kernel of fn(i) (one decode call),
    from HIP events the library records right around that kernel
    (pa_profile_next_decode)."""
    import torch

    from paged_kv_cache_11_amd import binding as pa

    for i in range(warmup):
        fn(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for e0, e1 in evs:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    for i in range(iters):
        pa.pa_profile_next_decode(*evs[i])
        fn(i)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(c) for a, c in evs])) * 1e3


ROW_GROUPS = ("long_context", "shared_prefix", "mixed_fp8", "block_sizes", "block_manager",
              "chunked_prefill", "swap", "prefix_cache", "continuous_batching", "ceiling")


def _manager_trace(mgr, lens, samples: int, steps: int, budget_s: float = 1e9):
    """A scheduler's use of a block manager: one prompt per entry of lens,
    each forked into samples - 1 more samples (parallel sampling), then
    decode steps that append one token to every sample and read back all
    block tables.  Returns (seconds per step, steps run, copy-on-write pairs,
    logical tokens per allocated slot: below 1 is the waste of partly filled
    last blocks, above 1 the saving of shared blocks)."""
    import time as _t

    ids, next_id = [], 0
    for L in lens:
        mgr.add(next_id, int(L))
        parent = next_id
        ids.append(next_id)
        next_id += 1
        for _ in range(samples - 1):
            mgr.fork(parent, next_id)
            ids.append(next_id)
            next_id += 1
    width = int(max(lens)) // mgr.block_size + steps // mgr.block_size + 2
    pairs, done, t0 = 0, 0, _t.perf_counter()
    for _ in range(steps):
        _, p = mgr.append(ids)
        pairs += len(p)
        if hasattr(mgr, "block_tables"):
            mgr.block_tables(ids, width)
        else:  # the reference manager: padded rows built from its tables
            np.array([mgr.table(i) + [-1] * (width - len(mgr.table(i))) for i in ids], np.int32)
        done += 1
        if _t.perf_counter() - t0 > budget_s:
            break
    dt = _t.perf_counter() - t0
    used = int(sum(int(L) * samples for L in lens)) + done * len(ids)  # logical tokens
    held = (mgr.num_blocks - mgr.num_free()) * mgr.block_size
    return dt / done, done, pairs, used / held


def _prefix_cache_trace(mgr, prompts, budget_s: float = 1e9):
    """Admit the prompts through add_prompt, releasing the oldest request
    whenever 16 are live; returns (seconds per request, requests, cached
    tokens, prompt tokens, peak blocks in use)."""
    import time as _t

    cached = total = peak = 0
    t0 = _t.perf_counter()
    done = 0
    for i, p in enumerate(prompts):
        if i >= 16:
            mgr.release(i - 16)
        _, nc = mgr.add_prompt(i, p)
        cached += nc
        total += len(p)
        peak = max(peak, mgr.num_blocks - mgr.num_free())
        done += 1
        if _t.perf_counter() - t0 > budget_s:
            break
    return (_t.perf_counter() - t0) / done, done, cached, total, peak


def prefix_cache_rows(requests: int = 256):
    """Automatic prefix caching on the host: 256 requests, each a
    2000-token system prompt shared by all plus 100-400 own tokens (block
    16), 16 live at a time, admitted through the library's manager: host
    time per admitted request, the share of prompt tokens found cached
    (their K/V need no prefill), and the device blocks in use at the peak
    against the same requests without caching.  Beside it, the reference
    manager on the same requests, as its CPU baseline."""
    from oracle.block_manager import BlockManager as RefManager
    from paged_kv_cache_11_amd import binding as pa

    rng = np.random.default_rng(11)
    bs = 16
    system = rng.integers(0, 32000, 2000).astype(np.int32)
    prompts = [np.concatenate([system, rng.integers(0, 32000, int(n)).astype(np.int32)])
               for n in rng.integers(100, 401, requests)]
    nb = 16 * (2400 // bs + 2) + 2000 // bs + 64
    lib = _prefix_cache_trace(pa.BlockManager(nb, bs, prefix_caching=True), prompts)
    ref = _prefix_cache_trace(RefManager(nb, bs, prefix_caching=True), prompts, budget_s=5.0)
    private_peak = max(sum(-(-len(p) // bs) for p in prompts[i:i + 16])
                       for i in range(0, requests - 15))
    return {"prefix_cache_system_prompt_256": {
        "us_per_request": round(lib[0] * 1e6, 2), "requests": lib[1], "block_size": bs,
        "cached_token_share": round(lib[2] / lib[3], 4),
        "peak_blocks_in_use": lib[4], "peak_blocks_without_caching": private_peak,
        "cpu_baseline": {"us_per_request": round(ref[0] * 1e6, 2), "requests": ref[1],
                         "kind": "oracle", "cores": 1}}}


def block_manager_rows(steps: int = 512):
    """Host cost of the library's block manager per decode step (append one
    token to every sequence + read all block tables), through the Python
    binding, on two traces of the headline shape: 64 private sequences, and
    8 prompts x 8 samples with copy-on-write.  Beside it, the reference
    block manager (test infrastructure) on the same traces, as its CPU
    baseline."""
    from oracle.block_manager import BlockManager as RefManager
    from paged_kv_cache_11_amd import binding as pa
    from paged_kv_cache_11_amd import workloads as wl

    bs = 16
    rows = {}
    for name, lens, samples in (("private_64", wl.llama3_8b_lengths(), 1),
                                ("sampling_8x8", wl.llama3_8b_lengths(num_seqs=8), 8)):
        nb = int(sum(-(-int(L) // bs) for L in lens)) + len(lens) * samples * (steps // bs + 2)
        lib = _manager_trace(pa.BlockManager(nb, bs), lens, samples, steps)
        ref = _manager_trace(RefManager(nb, bs), lens, samples, steps, budget_s=5.0)
        rows[f"block_manager_{name}"] = {
            "us_per_step": round(lib[0] * 1e6, 2), "seqs": len(lens) * samples, "steps": lib[1],
            "block_size": bs, "cow_pairs": lib[2], "logical_tokens_per_slot": round(lib[3], 4),
            "appends_per_s": round(len(lens) * samples / lib[0], 1),
            "cpu_baseline": {"us_per_step": round(ref[0] * 1e6, 2), "steps": ref[1],
                             "kind": "oracle", "cores": 1}}
        if ref[1] == lib[1] and ref[2] != lib[2]:
            raise RuntimeError(f"{name}: the library and the reference manager disagree")
    return rows


def row_measurements(dev, iters=20, groups=ROW_GROUPS):
    """Timings of the other rows of the hot path, one workload each; groups
    picks which workloads run (all by default)."""
    import torch

    from paged_kv_cache_11_amd import binding as pa
    from paged_kv_cache_11_amd import workloads as wl

    rows = {}
    t_start = time.perf_counter()

    def done(group):
        print(f"[bench] rows {group} done at {time.perf_counter() - t_start:.1f} s", file=sys.stderr,
              flush=True)

    if "long_context" in groups:
        # Long-context split-K: 8 x 32768 tokens, 512-token partitions + LSE reduce.
        b = wl.long_context_decode()
        sets = _gpu_pools(b, dev)
        q = wl.storage_tensor(b.q, b.q_dtype).to(dev)
        out = torch.empty_like(q)
        tb, ln = torch.from_numpy(b.block_tables).to(dev), torch.from_numpy(b.seq_lens).to(dev)
        for name, ps in (("long_context_splitk_512", 512), ("long_context_balanced", -1)):
            ws = torch.empty(max(1, pa.pa_decode_workspace_size(b.num_seqs, b.num_heads, b.num_kv_heads,
                                                                b.head_size, b.max_seq_len, ps)),
                             dtype=torch.uint8, device=dev)
            us = _time_us(lambda i: pa.pa_decode(out, q, sets[0][0], sets[0][1], tb, ln, b.max_seq_len,
                                                 b.scale, partition_size=ps, workspace=ws,
                                                 flags=pa.PA_DECODE_READ_ONCE), iters)
            by = b.decode_kv_bytes()
            rows[name] = {"us": round(us, 2), "kv_bytes": by, "gbs": round(by / us / 1e3, 1),
                          "pct_hbm_peak": round(100 * by / us / 1e3 / HBM_PEAK_GBS, 2),
                          "tokens_per_s": round(b.num_seqs / us * 1e6, 1)}
        del sets
        torch.cuda.empty_cache()

    if "long_context" in groups:
        done("long_context")
    if "shared_prefix" in groups:
        # Shared prefix: 256 forks of one prefix (config 4): the literal
        # 2048-token prefix (no copy-on-write), the 2040-token variant whose
        # partly filled last prefix block every fork copies first (256
        # pairs; 127 blocks stay shared), and the 2048-token prefix in a
        # pool 4x the blocks in use (a serving pool sized to memory).  Three
        # copies of the pools are rotated so calls read HBM, not the 256 MB
        # last-level cache.  Each row times pa_decode_shared_prefix (prefix
        # once per KV head on the matrix cores + suffixes + merge) beside
        # pa_decode on the same tables with the sharing hint.
        for tag, prefix_len, pool_factor in (("c4", 2048, 1.25), ("c4_cow", 2040, 1.25),
                                             ("c4_pool4x", 2048, 4.0)):
            b = wl.shared_prefix_decode(prefix_len=prefix_len, pool_factor=pool_factor)
            sets = _gpu_pools(b, dev, copies=N_SETS)
            pairs = torch.from_numpy(b.copy_pairs).to(dev)
            blk_bytes = 2 * b.num_kv_heads * b.block_size * b.head_size * 2
            us_copy = _time_us(lambda i: pa.pa_copy_blocks(sets[i % N_SETS][0], sets[i % N_SETS][1],
                                                           pairs), iters)
            q = wl.storage_tensor(b.q, b.q_dtype).to(dev)
            out = torch.empty_like(q)
            tb, ln = torch.from_numpy(b.block_tables).to(dev), torch.from_numpy(b.seq_lens).to(dev)
            shared = (prefix_len // b.block_size) * b.block_size
            ws_sp = torch.empty(pa.pa_decode_shared_prefix_workspace_size(
                b.num_seqs, b.num_heads, b.num_kv_heads, b.head_size, shared),
                dtype=torch.uint8, device=dev)
            ws = torch.empty(pa.pa_decode_workspace_size(b.num_seqs, b.num_heads, b.num_kv_heads,
                                                         b.head_size, b.max_seq_len, -1),
                             dtype=torch.uint8, device=dev)

            def sp(i):
                kc, vc = sets[i % N_SETS]
                pa.pa_decode_shared_prefix(out, q, kc, vc, tb, ln, b.max_seq_len, shared, b.scale,
                                           workspace=ws_sp, flags=pa.PA_DECODE_READ_ONCE)

            def dec(flags):
                return lambda i: pa.pa_decode(out, q, sets[i % N_SETS][0], sets[i % N_SETS][1], tb,
                                              ln, b.max_seq_len, b.scale, partition_size=-1,
                                              workspace=ws, flags=flags)

            us_sp = _time_us(sp, iters)
            us_dec = _time_us(dec(pa.PA_DECODE_SHARED), iters)
            logical = b.decode_kv_bytes()
            unique = (int(np.unique(b.block_tables[b.block_tables >= 0]).size) * b.block_size
                      * b.kv_bytes_per_token())
            row = {"us": round(us_sp, 2), "prefix_len": prefix_len, "shared_tokens": shared,
                   "forks": b.num_seqs, "pool_blocks": b.num_blocks,
                   "unique_kv_bytes": unique, "logical_kv_bytes": logical,
                   "gbs_unique": round(unique / us_sp / 1e3, 1),
                   "pct_hbm_peak_unique": round(100 * unique / us_sp / 1e3 / HBM_PEAK_GBS, 2),
                   "effective_gbs_logical": round(logical / us_sp / 1e3, 1),
                   "tokens_per_s": round(b.num_seqs / us_sp * 1e6, 1),
                   "pa_decode_shared_hint_us": round(us_dec, 2),
                   "copy_on_write": {"pairs": len(b.copy_pairs), "us": round(us_copy, 2),
                                     "bytes_read_written": 2 * len(b.copy_pairs) * blk_bytes}}
            if tag == "c4_pool4x":
                # The hints on shared tables: none (ordinary loads), and the
                # read-once hint misapplied (evict-first loads of shared lines).
                row["pa_decode_no_hint_us"] = round(_time_us(dec(0), iters), 2)
                row["pa_decode_read_once_hint_us"] = round(
                    _time_us(dec(pa.PA_DECODE_READ_ONCE), iters), 2)
            rows[f"shared_prefix_{tag}"] = row
            del sets, ws, ws_sp
            torch.cuda.empty_cache()

    if "shared_prefix" in groups:
        done("shared_prefix")
    if "mixed_fp8" in groups:
        # Mixed fp8 step (70B shape): cache write of the step's new tokens,
        # decode of 32 sequences, prefill of a 512-query chunk.
        b = wl.mixed_fp8_step()
        sets = _gpu_pools(b, dev, copies=2)
        q = wl.storage_tensor(b.q, b.q_dtype).to(dev)
        out = torch.empty_like(q)
        tb, ln = torch.from_numpy(b.block_tables).to(dev), torch.from_numpy(b.seq_lens).to(dev)
        ws = torch.empty(pa.pa_decode_workspace_size(b.num_seqs, b.num_heads, b.num_kv_heads,
                                                     b.head_size, b.max_seq_len, -1),
                         dtype=torch.uint8, device=dev)
        ends = np.cumsum(b.seq_lens.astype(np.int64))
        dec_new = ends - 1
        chunk_idx = np.arange(int(ends[-1]) + 1536, int(ends[-1]) + 2048)
        new_idx = np.concatenate([dec_new, chunk_idx])
        k_new = wl.storage_tensor(b.k[new_idx], b.kv_src_dtype).to(dev)
        v_new = wl.storage_tensor(b.v[new_idx], b.kv_src_dtype).to(dev)
        s_new = torch.from_numpy(b.slot_mapping[new_idx]).to(dev)
        cq = wl.storage_tensor(b.chunk_q, "bf16").to(dev)
        cout = torch.empty_like(cq)
        cqs = torch.from_numpy(b.chunk_query_start).to(dev)
        ctb = torch.from_numpy(b.chunk_block_tables).to(dev)
        cln = torch.from_numpy(b.chunk_seq_lens).to(dev)
        nq = int(b.chunk_q.shape[0])

        def cw(i):
            kc, vc = sets[i % 2]
            pa.pa_cache_write(k_new, v_new, kc, vc, s_new, b.k_scale, b.v_scale)

        def dec(i):
            kc, vc = sets[i % 2]
            pa.pa_decode(out, q, kc, vc, tb, ln, b.max_seq_len, b.scale, b.k_scale, b.v_scale, -1, ws,
                         flags=pa.PA_DECODE_READ_ONCE)

        def pre(i):
            kc, vc = sets[i % 2]
            pa.pa_prefill_chunk(cout, cq, cqs, nq, kc, vc, ctb, cln, b.scale, b.k_scale, b.v_scale)

        us_cw = _time_us(cw, iters)
        n_new = len(new_idx)
        cw_bytes = n_new * b.num_kv_heads * b.head_size * (2 * 2 + 2 * 1)  # bf16 in, fp8 out, K and V
        rows["cache_write_fp8_mixed_step"] = {"us": round(us_cw, 2), "tokens": n_new,
                                              "bytes_moved": cw_bytes,
                                              "gbs": round(cw_bytes / us_cw / 1e3, 1)}
        us_dec = _time_us(dec, iters)
        kern_dec = _kernel_us(dec, iters)
        by = b.decode_kv_bytes()
        rows["decode_fp8_70b_shape"] = {"us": round(us_dec, 2), "kv_bytes": by,
                                        "gbs": round(by / us_dec / 1e3, 1),
                                        "pct_hbm_peak": round(100 * by / us_dec / 1e3 / HBM_PEAK_GBS, 2),
                                        "kernel_us": round(kern_dec, 2),
                                        "kernel_pct_hbm_peak": round(100 * by / kern_dec / 1e3 / HBM_PEAK_GBS, 2),
                                        "tokens_per_s": round(b.num_seqs / us_dec * 1e6, 1)}
        us_pre = _time_us(pre, iters)
        L, n = int(b.chunk_seq_lens[0]), nq
        pairs = sum(L - n + i + 1 for i in range(n))  # causal (query, key) pairs per head
        flops = 4.0 * b.num_heads * b.head_size * pairs
        rows["prefill_chunk_fp8_70b_shape"] = {
            "us": round(us_pre, 2), "causal_flops": flops, "tflops": round(flops / us_pre / 1e6, 1),
            "pct_mfma_bf16_peak": round(100 * flops / us_pre / 1e6 / MFMA_BF16_PEAK_TFLOPS, 2),
            "queries_per_s": round(n / us_pre * 1e6, 1)}
        us_step = _time_us(lambda i: (cw(i), dec(i), pre(i)), iters)
        # The same step with decode and prefill on two streams after the
        # cache write: whether the memory-bound and the compute-bound kernel
        # gain from running side by side.
        main = torch.cuda.current_stream()
        s_dec, s_pre = torch.cuda.Stream(), torch.cuda.Stream()

        def step_two_streams(i):
            cw(i)
            s_dec.wait_stream(main)
            s_pre.wait_stream(main)
            with torch.cuda.stream(s_dec):
                dec(i)
            with torch.cuda.stream(s_pre):
                pre(i)
            main.wait_stream(s_dec)
            main.wait_stream(s_pre)

        us_two = _time_us(step_two_streams, iters)
        rows["mixed_step_fp8"] = {"us": round(us_step, 2),
                                  "step": "cache_write(544 tokens) + decode(32 seqs) + prefill(512 queries)",
                                  "two_streams_us": round(us_two, 2)}
    if "mixed_fp8" in groups:
        done("mixed_fp8")
    if "chunked_prefill" in groups:
        # One scheduler step of varlen chunked prefill under a 512- and a
        # 2048-token budget (Llama-3-8B shape, bf16 pool): one call per step.
        for budget in (512, 2048):
            b = wl.make(f"chunked_prefill_budget{budget}_bf16")
            sets = _gpu_pools(b, dev, copies=2)
            cq = wl.storage_tensor(b.chunk_q, "bf16").to(dev)
            cout = torch.empty_like(cq)
            cqs = torch.from_numpy(b.chunk_query_start).to(dev)
            ctb = torch.from_numpy(b.chunk_block_tables).to(dev)
            cln = torch.from_numpy(b.chunk_seq_lens).to(dev)
            max_q = int(np.diff(b.chunk_query_start).max())
            us = _time_us(lambda i: pa.pa_prefill_chunk(cout, cq, cqs, max_q, sets[i % 2][0],
                                                        sets[i % 2][1], ctb, cln, b.scale), iters)
            pairs = sum(sum(first + i + 1 for i in range(n)) for _, first, n in b.chunks)
            flops = 4.0 * b.num_heads * b.head_size * pairs
            rows[f"prefill_budget{budget}_llama3_8b"] = {
                "us": round(us, 2), "chunks": [list(c) for c in b.chunks], "causal_flops": flops,
                "tflops": round(flops / us / 1e6, 1),
                "pct_mfma_bf16_peak": round(100 * flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 2),
                "tokens_per_s": round(budget / us * 1e6, 1)}
            del sets
            torch.cuda.empty_cache()
    if "chunked_prefill" in groups:
        done("chunked_prefill")
    if "swap" in groups:
        # SWAP preemption: the blocks of 8 sequences of the headline workload
        # (lengths U[512, 4096], bf16, 32 KiB per block and pool) moved to a
        # pinned host pool and back, one call each way; beside it, one DMA
        # copy of the same bytes as a single contiguous buffer (the host
        # link's practical rate), and the same blocks moved by one DMA copy
        # per block and pool.
        lens = wl.llama3_8b_lengths(num_seqs=8)
        bs, Hkv, D = 16, 8, 128
        n = int(sum(-(-int(L) // bs) for L in lens))
        nb = n + 64
        rng = np.random.default_rng(7)
        kd = torch.randn((nb, Hkv, bs, D), device=dev).to(torch.bfloat16)
        vd = torch.randn((nb, Hkv, bs, D), device=dev).to(torch.bfloat16)
        hk = torch.empty((n, Hkv, bs, D), dtype=torch.bfloat16, pin_memory=True)
        hv = torch.empty_like(hk, pin_memory=True)
        dev_ids = rng.permutation(nb)[:n]
        out_map = torch.from_numpy(np.stack([dev_ids, np.arange(n)], 1).astype(np.int64)).to(dev)
        in_map = torch.from_numpy(np.stack([np.arange(n), dev_ids], 1).astype(np.int64)).to(dev)
        moved = 2 * n * Hkv * bs * D * 2
        it = max(3, iters // 4)
        us_out = _time_us(lambda i: pa.pa_swap_blocks(kd, vd, hk, hv, out_map), it)
        us_in = _time_us(lambda i: pa.pa_swap_blocks(hk, hv, kd, vd, in_map), it)
        flat_d = torch.empty(moved, dtype=torch.uint8, device=dev)
        flat_h = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
        us_dma_out = _time_us(lambda i: flat_h.copy_(flat_d, non_blocking=True), it)
        us_dma_in = _time_us(lambda i: flat_d.copy_(flat_h, non_blocking=True), it)
        ids = dev_ids.tolist()

        def per_block(i):
            for j, d in enumerate(ids):
                hk[j].copy_(kd[d], non_blocking=True)
                hv[j].copy_(vd[d], non_blocking=True)

        us_blk = _time_us(per_block, 2, warmup=1)
        link = HOST_LINK_PEAK_GBS
        rows["swap_out_8_seqs"] = {"us": round(us_out, 1), "blocks": n, "bytes": moved,
                                   "gbs": round(moved / us_out / 1e3, 2),
                                   "pct_host_link_peak": round(100 * moved / us_out / 1e3 / link, 1)}
        rows["swap_in_8_seqs"] = {"us": round(us_in, 1), "blocks": n, "bytes": moved,
                                  "gbs": round(moved / us_in / 1e3, 2),
                                  "pct_host_link_peak": round(100 * moved / us_in / 1e3 / link, 1)}
        rows["swap_dma_reference"] = {
            "contiguous_out_gbs": round(moved / us_dma_out / 1e3, 2),
            "contiguous_in_gbs": round(moved / us_dma_in / 1e3, 2),
            "per_block_copies_out_gbs": round(moved / us_blk / 1e3, 2),
            "host_link_peak_gbs": link}
        del kd, vd, hk, hv, flat_d, flat_h
        torch.cuda.empty_cache()
    if "swap" in groups:
        done("swap")
    if "continuous_batching" in groups:
        # A continuous-batching decode step: 768 sequences of lengths
        # U[64, 1024], Llama-3-8B shape, balanced split, read-once hint,
        # three pool copies rotated.  The decode kernel is also timed alone
        # (library-recorded events around it).
        b = wl.continuous_batching_decode()
        sets = _gpu_pools(b, dev, copies=N_SETS)
        q = wl.storage_tensor(b.q, b.q_dtype).to(dev)
        out = torch.empty_like(q)
        tb, ln = torch.from_numpy(b.block_tables).to(dev), torch.from_numpy(b.seq_lens).to(dev)
        ws = torch.empty(pa.pa_decode_workspace_size(b.num_seqs, b.num_heads, b.num_kv_heads,
                                                     b.head_size, b.max_seq_len, -1),
                         dtype=torch.uint8, device=dev)

        def dec(i):
            pa.pa_decode(out, q, sets[i % N_SETS][0], sets[i % N_SETS][1], tb, ln, b.max_seq_len,
                         b.scale, partition_size=-1, workspace=ws, flags=pa.PA_DECODE_READ_ONCE)

        us = _time_us(dec, iters)
        kern = _kernel_us(dec, iters)
        by = b.decode_kv_bytes()
        rows["continuous_batching_768"] = {
            "us": round(us, 2), "kernel_us": round(kern, 2), "seqs": b.num_seqs,
            "seq_lens": f"U[{int(b.seq_lens.min())}, {int(b.seq_lens.max())}]",
            "kv_bytes": by, "gbs": round(by / us / 1e3, 1),
            "pct_hbm_peak": round(100 * by / us / 1e3 / HBM_PEAK_GBS, 2),
            "kernel_gbs": round(by / kern / 1e3, 1),
            "tokens_per_s": round(b.num_seqs / us * 1e6, 1)}
        del sets
        torch.cuda.empty_cache()
    if "continuous_batching" in groups:
        done("continuous_batching")
    if "ceiling" in groups:
        # The practical HBM ceiling of this access pattern: pa_copy_blocks
        # over 16384 scattered whole blocks of the headline pool geometry
        # (bf16, 8 KV heads, block 16: 64 KiB per block for K and V), 1 GiB
        # read and 1 GiB written per call.
        Hkv, bs, D = 8, 16, 128
        nb = 2 * 16384 + 64
        kp = torch.empty((nb, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
        vp = torch.empty_like(kp)
        perm = np.random.default_rng(9).permutation(nb)
        pairs = torch.from_numpy(np.stack([perm[:16384], perm[16384:32768]], 1)
                                 .astype(np.int64)).to(dev)
        us = _time_us(lambda i: pa.pa_copy_blocks(kp, vp, pairs), iters)
        moved = 16384 * 2 * Hkv * bs * D * 2
        rows["ceiling_copy_blocks_1gib"] = {
            "us": round(us, 2), "bytes_read": moved, "bytes_written": moved,
            "read_gbs": round(moved / us / 1e3, 1),
            "read_plus_write_gbs": round(2 * moved / us / 1e3, 1),
            "pct_hbm_peak_read_plus_write": round(100 * 2 * moved / us / 1e3 / HBM_PEAK_GBS, 2)}
        del kp, vp
        torch.cuda.empty_cache()
    if "ceiling" in groups:
        done("ceiling")
    if "block_manager" in groups:
        rows.update(block_manager_rows())
    if "block_manager" in groups:
        done("block_manager")
    if "prefix_cache" in groups:
        rows.update(prefix_cache_rows())
    if "prefix_cache" in groups:
        done("prefix_cache")
    if "block_sizes" in groups:
        # The headline decode over pool blocks of 64 and 128 tokens (same
        # lengths and values), balanced split, three pool copies rotated.
        for bs in (64, 128):
            b = wl.llama3_8b_decode(block_size=bs)
            sets = _gpu_pools(b, dev, copies=N_SETS)
            q = wl.storage_tensor(b.q, b.q_dtype).to(dev)
            out = torch.empty_like(q)
            tb, ln = torch.from_numpy(b.block_tables).to(dev), torch.from_numpy(b.seq_lens).to(dev)
            ws = torch.empty(pa.pa_decode_workspace_size(b.num_seqs, b.num_heads, b.num_kv_heads,
                                                         b.head_size, b.max_seq_len, -1),
                             dtype=torch.uint8, device=dev)
            us = _time_us(lambda i: pa.pa_decode(out, q, sets[i % N_SETS][0], sets[i % N_SETS][1],
                                                 tb, ln, b.max_seq_len, b.scale, partition_size=-1,
                                                 workspace=ws, flags=pa.PA_DECODE_READ_ONCE), iters)
            by = b.decode_kv_bytes()
            rows[f"decode_llama3_8b_bs{bs}"] = {"us": round(us, 2), "kv_bytes": by,
                                               "gbs": round(by / us / 1e3, 1),
                                               "pct_hbm_peak": round(100 * by / us / 1e3 / HBM_PEAK_GBS, 2)}
            del sets
            torch.cuda.empty_cache()
    if "block_sizes" in groups:
        done("block_sizes")
    return rows



def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="pa_decode partition_size: -1 balanced split (default), 0 none, or tokens")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--oracle-budget", type=float, default=2.0,
                    help="seconds of oracle time per workload for cpu_baseline_per_workload "
                         "(0 skips it)")
    ap.add_argument("--two-calls", action="store_true",
                    help="time the headline step as pa_cache_write + pa_decode instead of one "
                         "pa_decode_append call")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the per-row measurements of the other workloads")
    ap.add_argument("--rows-only", choices=ROW_GROUPS,
                    help="measure only this group of rows (no headline step) and print them; "
                         "for per-kernel profiling of one row")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run pa_copy_blocks over this many MiB (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/decode_kernel_<workload>_counters.json from two "
                         "rocprofv3 --pmc counter_collection.csv files and exit")
    args = ap.parse_args(argv)
    if args.summarize_counters:
        outp = os.path.join(ROOT, "profiles", f"decode_kernel_{args.workload}_counters.json")
        print(json.dumps(summarize_counters(*args.summarize_counters, args.workload, outp)))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path "
              "shards by sequence or KV head with no exchange, so it is not run on several "
              "GPUs here.", file=sys.stderr)
        return 2

    import torch

    from paged_kv_cache_11_amd import binding as pa
    from paged_kv_cache_11_amd import workloads as wl

    if args.rows_only:
        print(json.dumps({"rows": row_measurements(torch.device("cuda:0"), groups=(args.rows_only,))}),
              flush=True)
        return 0

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pa.load()
    dev = torch.device("cuda:0")
    b = wl.make(args.workload)
    print(f"[bench] workload {b.name}: {b.num_seqs} seqs, lens {int(b.seq_lens.min())}.."
          f"{int(b.seq_lens.max())}, pool {b.num_blocks} blocks, {b.kv_dtype}", file=sys.stderr,
          flush=True)

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[b.kv_dtype]
    shape = (b.num_blocks, b.num_kv_heads, b.block_size, b.head_size)
    k0 = torch.zeros(shape, dtype=tdt, device=dev)
    v0 = torch.zeros(shape, dtype=tdt, device=dev)
    chunk = 1 << 16
    for a in range(0, len(b.slot_mapping), chunk):
        pa.pa_cache_write(wl.storage_tensor(b.k[a:a + chunk], b.kv_src_dtype).to(dev),
                          wl.storage_tensor(b.v[a:a + chunk], b.kv_src_dtype).to(dev), k0, v0,
                          torch.from_numpy(b.slot_mapping[a:a + chunk]).to(dev), b.k_scale,
                          b.v_scale)
    sets = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(N_SETS - 1)]
    q = wl.storage_tensor(b.q, b.q_dtype).to(dev)
    out = torch.empty_like(q)
    tables = torch.from_numpy(b.block_tables).to(dev)
    lens = torch.from_numpy(b.seq_lens).to(dev)
    # The step's new tokens: the last token of every sequence.
    ends = np.cumsum(b.seq_lens.astype(np.int64))
    new_idx = ends - 1
    k_new = wl.storage_tensor(b.k[new_idx], b.kv_src_dtype).to(dev)
    v_new = wl.storage_tensor(b.v[new_idx], b.kv_src_dtype).to(dev)
    slots_new = torch.from_numpy(b.slot_mapping[new_idx]).to(dev)
    ps = args.partition_size
    ws_bytes = pa.pa_decode_workspace_size(b.num_seqs, b.num_heads, b.num_kv_heads, b.head_size,
                                           b.max_seq_len, ps)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # The step as two calls: the cache write of the new tokens, then the
    # decode over every token.
    def step_two_calls(i, stream=stream):
        kc, vc = sets[i % N_SETS]
        pa.pa_cache_write(k_new, v_new, kc, vc, slots_new, b.k_scale, b.v_scale, stream=stream)
        pa.pa_decode(out, q, kc, vc, tables, lens, b.max_seq_len, b.scale, b.k_scale, b.v_scale,
                     ps, ws, stream=stream, flags=pa.PA_DECODE_READ_ONCE)

    # The same step as one call: pa_decode_append writes each sequence's new
    # token into its slot inside the decode kernel (balanced split only).
    fused = ps == pa.PA_PARTITION_BALANCED and not args.two_calls

    def step_fused(i, stream=stream):
        kc, vc = sets[i % N_SETS]
        pa.pa_decode_append(out, q, k_new, v_new, kc, vc, tables, lens, b.max_seq_len, b.scale,
                            b.k_scale, b.v_scale, ws, stream=stream,
                            flags=pa.PA_DECODE_READ_ONCE)

    def time_steps(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    step = step_fused if fused else step_two_calls
    ms_per_step = time_steps(step)
    two_call_ms = time_steps(step_two_calls) if fused else ms_per_step

    kv_bytes = b.decode_kv_bytes()
    n_calls = max(args.steps, 200)

    # The step's decode call alone (decode kernel + reduce kernel; with the
    # fused step, pa_decode_append), back to back over n_calls calls, HIP
    # events on its stream around the run.
    def dec_call(i):
        if fused:
            step_fused(i)
            return
        kc, vc = sets[i % N_SETS]
        pa.pa_decode(out, q, kc, vc, tables, lens, b.max_seq_len, b.scale, b.k_scale, b.v_scale,
                     ps, ws, stream=stream, flags=pa.PA_DECODE_READ_ONCE)

    call_us = _time_us(dec_call, n_calls)

    # The dominant kernel alone: pa_profile_next_decode makes the library
    # record a pair of HIP events right around the decode kernel's launch
    # (hipExtLaunchKernelGGL, same stream), call after call.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_calls)]
    for e0, e1 in evs:  # create the events
        e0.record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    for i in range(n_calls):
        pa.pa_profile_next_decode(*evs[i])
        dec_call(i)
    torch.cuda.synchronize()
    kern_ms = np.array([a.elapsed_time(c) for a, c in evs])
    kern_us = float(kern_ms.mean()) * 1e3

    # The same step captured in HIP graphs (one per pool copy; cache write
    # + decode kernel + reduce kernel), replayed in rotation.
    graph_ms = None
    try:
        graphs = []
        gs = torch.cuda.Stream()
        for k in range(N_SETS):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                step(k, stream=torch.cuda.current_stream())
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % N_SETS].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % N_SETS].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) / args.steps * 1e3
        del graphs
    except Exception as e:  # pragma: no cover - reported, not fatal
        print(f"[bench] graph capture failed: {e}", file=sys.stderr, flush=True)

    gbs = kv_bytes / (ms_per_step / 1e3) / 1e9
    achieved = kv_bytes / (kern_us / 1e6) / 1e9
    call_gbs = kv_bytes / (call_us / 1e6) / 1e9
    print(f"[bench] step {ms_per_step * 1e3:.1f} us (graph {graph_ms * 1e3 if graph_ms else -1:.1f};"
          f" as two calls {two_call_ms * 1e3:.1f}),"
          f" decode call {call_us:.1f} us, decode kernel {kern_us:.1f} us "
          f"(p10 {np.percentile(kern_ms, 10) * 1e3:.1f}, p90 {np.percentile(kern_ms, 90) * 1e3:.1f}),"
          f" {achieved:.0f} GB/s in the kernel", file=sys.stderr, flush=True)

    calib = None
    if args.copy_calibration_mib:
        nbk = args.copy_calibration_mib * (1 << 20) // (2 * k0[0].numel() * k0.element_size())
        nbk = min(nbk, b.num_blocks // 2)
        pairs = torch.stack([torch.arange(nbk), torch.arange(nbk) + b.num_blocks // 2], 1)
        pairs = pairs.to(torch.int64).to(dev).contiguous()
        pa.pa_copy_blocks(k0, v0, pairs)
        torch.cuda.synchronize()
        calib = {"copy_bytes_read": int(2 * nbk * k0[0].numel() * k0.element_size())}

    traffic = stored_traffic(b.name)
    rows = None
    if not args.no_rows:
        del sets
        torch.cuda.empty_cache()
        rows = row_measurements(dev)
    cpu = cpu_baseline(b, args.cpu_budget)
    oracle_per_workload = oracle_rows(args.oracle_budget) if args.oracle_budget > 0 else None
    tokens_per_s = b.num_seqs / (ms_per_step / 1e3)
    res = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": b.name, "num_seqs": b.num_seqs, "num_heads": b.num_heads,
            "num_kv_heads": b.num_kv_heads, "head_size": b.head_size,
            "block_size": b.block_size, "seq_lens": f"uniform [{int(b.seq_lens.min())}, "
            f"{int(b.seq_lens.max())}] (seeded)", "sum_seq_lens": int(b.seq_lens.sum()),
            "pool_blocks": b.num_blocks, "partition_size": ps,
            "kv_bytes_per_step": kv_bytes, "input_sets_rotated": N_SETS,
            "step": ("pa_decode_append: each sequence's new token written into its slot inside "
                     "the decode kernel, then the LSE reduce (one call)") if fused else
                    "pa_cache_write(new token per sequence) + pa_decode (split-K + LSE reduce)",
        },
        "tokens_per_s": round(tokens_per_s, 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "kernel": "decode_balanced_mfma_kernel (the dominant kernel of pa_decode)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic, "avg_us": round(kern_us, 2),
            "timing": f"mean over {n_calls} launches of HIP events the library records right "
                      "around the kernel (pa_profile_next_decode, hipExtLaunchKernelGGL) on its "
                      "stream; achieved = algorithmic K/V bytes / avg_us",
            "call": {"what": ("pa_decode_append call" if fused else "pa_decode call") +
                             " = decode kernel + reduce kernel, back to back",
                     "avg_us": round(call_us, 2), "achieved": round(call_gbs, 1),
                     "frac": round(call_gbs / HBM_PEAK_GBS, 4)},
        },
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms else None,
        "two_call_ms_per_step": round(two_call_ms, 5),
        "cpu_baseline": cpu,
    }
    if oracle_per_workload:
        res["cpu_baseline_per_workload"] = oracle_per_workload
    if rows:
        res["rows"] = rows
    if calib:
        res["copy_calibration"] = calib
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
