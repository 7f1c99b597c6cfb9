#!/usr/bin/env python3
"""Benchmark of the paged decode hot path on one MI355X (gfx950).

One *step* is one decode step of a batch, as a serving loop runs it:

  a1  host block manager: reserve each sequence's slot for its new token,
      extend block tables from the free pool, emit copy-on-write pairs
      (done for every step before the timed region; its host time is
      reported separately as ``host_prep_us``)
  a2  pa_copy_blocks  (only when the step has copy-on-write pairs)
  a3  pa_write_kv     (one new token per sequence)
  a4  pa_decode       (K1, plus the partition-merge kernel K1b when
      partition_size > 0)

a3 and a4 are one call, pa_decode_write (the new tokens are stored inside
the balanced decode kernel, which reads them from the input rows), unless
``--separate-write`` asks for the two calls.

Each step appends one token per sequence, so step i attends over
``context_lens + i`` tokens; every step's metadata (slots, tables, lengths)
is uploaded to HBM before timing starts.  As in a model with several layers,
consecutive steps read different KV pools: ``--layers`` copies of the pool
are made and step i uses copy ``i % layers``, so a step never finds the
previous step's K/V in the 256 MiB Infinity Cache.  The timed region is
exactly ``--steps`` back-to-back steps between two device synchronisations.

Printed: one JSON line.  ``value`` is the achieved algorithmic HBM rate of
the whole step (K/V rows of every attended token, once per KV head, plus the
block-table entries read, plus the bytes the write / copy kernels move)
divided by the step time.  ``roofline`` is the same figure for the decode
call alone (its kernels), from HIP events recorded on the launch stream
around ``--steps`` back-to-back decode calls over the same per-step inputs.
``cold_cache`` repeats the decode after reading a 1 GiB buffer before
each call (evicts L2 and the Infinity Cache without leaving dirty lines).
``cpu_baseline`` is the fp64 CPU oracle timed on this host on a bounded
sample of the same step.

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME]
                       [--partition P] [--no-cpu-baseline] [--cold-steps N]
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) and seqs·tokens/s attended"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E peak, GB/s
FLUSH_BYTES = 1 << 30      # > 4x the 256 MiB Infinity Cache
CALIB_BYTES = 512 << 20    # plain copy of known size, read by the traffic counters

# Decode launch configuration per workload (partition_size: -1 = the balanced
# split, equal shares of all work per GPU workgroup slot).  The parity tests
# run the same configurations.
BALANCED = -1
WORKLOADS = {
    "llama3_8b_b64": (lambda: W.c2_llama8b_b64(), BALANCED),
    "long_ctx_32k": (lambda: W.c3_long_context(), BALANCED),
    "mha_b256_bs8": (lambda: W.c5_mha_sweep(block_size=8), BALANCED),
    "mha_b256_bs16": (lambda: W.c5_mha_sweep(block_size=16), BALANCED),
    "mha_b256_bs32": (lambda: W.c5_mha_sweep(block_size=32), BALANCED),
    "tiny_f32": (lambda: W.c1_tiny_f32(), BALANCED),
}
DEFAULT_WORKLOAD = "llama3_8b_b64"
# Prompt prefill (pa_write_kv of the chunk's tokens, then pa_prefill); reported
# in TFLOP/s against the dense bf16 matrix-core peak.
PREFILL_WORKLOADS = {
    "prefill_llama3_8b": lambda: W.c6_prefill_llama8b(),
    "prefill_chunked": lambda: W.c6_chunked_prefill(),
}
PREFILL_METRIC = "paged prefill attention: achieved TFLOP/s (causal QK and PV flops)"
# Swap: a quarter of the Llama-3-8B-shaped batch's sequences swapped out to a
# pinned host pool and back in (host manager decisions + pa_swap_blocks);
# GB/s over the host link in each direction.
SWAP_WORKLOADS = {"swap_llama3_8b": lambda: W.c2_llama8b_b64()}
SWAP_METRIC = "KV block swap between HBM and pinned host memory: achieved GB/s per direction"
HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, per direction
# Prefix-cached prompt admission: each step admits 64 Llama-3-8B-shaped
# requests (a cached 2048-token system prompt + private suffixes); the host
# manager finds the cached blocks, only the uncached tokens are stored and
# prefilled.  Prompt tokens admitted per second, beside the same batch
# admitted without the cache.
PREFIX_WORKLOADS = {"prefix_cached_prompts": lambda: W.c8_prefix_cached_prompts()}
PREFIX_METRIC = "prefix-cached prompt admission: prompt tokens/s (cached + computed)"
# Shared-prefix copy-on-write: 256 sequences share a 2048-token prefix; each
# of 8 steps copies 1% of the shared references, stores one token per
# sequence and decodes.  GB/s of logical bytes (every sequence's whole
# context) and of unique bytes (each distinct block's tokens once).
COW_WORKLOADS = {"shared_prefix_cow": lambda: W.c4_shared_prefix()}
COW_METRIC = "shared-prefix copy-on-write decode: logical GB/s (unique GB/s beside)"
# KV waste of a serving loop (host simulation, no kernel): 4096 requests
# through the KV slots one MI355X holds for Llama-3-8B, contiguous slabs
# against the library's paged block manager (bs 16).
WASTE_WORKLOADS = {"waste_llama3_8b_c2": lambda: W.waste_case("waste_llama3_8b_c2"),
                   "waste_llama3_8b_c5": lambda: W.waste_case("waste_llama3_8b_c5")}
WASTE_METRIC = "KV-cache waste: % of held KV slots holding no token (paged blocks; contiguous slabs beside)"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
DECODE_TIMED_CALLS = 200   # back-to-back decode calls in the roofline's event bracket (at least --steps)
DECODE_PER_CALL = 100      # decode calls timed one by one for the per-call distribution
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_{}_traffic.md")
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_354_amd", "csrc", f)
               for f in ("pa_decode.hip", "pa_decode_gqa.hip", "pa_decode_common.h")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--plan-steps", type=int, default=20,
                   help="decode workloads: distinct planned steps (lengths grow by one per step), replayed "
                        "cyclically by the warmup and the timed steps")
    p.add_argument("--warmup", type=int, default=200,
                   help="untimed steps first (200 bring the GPU to the steady state of a serving loop)")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD,
                   choices=sorted(WORKLOADS) + sorted(PREFILL_WORKLOADS) + sorted(SWAP_WORKLOADS)
                   + sorted(PREFIX_WORKLOADS) + sorted(WASTE_WORKLOADS) + sorted(COW_WORKLOADS))
    p.add_argument("--partition", type=int, default=None,
                   help="decode partition_size (default: the workload's configuration)")
    p.add_argument("--cold-steps", type=int, default=10, help="cold-cache decode calls (0: skip)")
    p.add_argument("--layers", type=int, default=4,
                   help="KV pool copies that consecutive steps rotate over (1: same pool every step)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--separate-write", action="store_true",
                   help="pa_write_kv then pa_decode (or pa_prefill) instead of one pa_decode_write "
                        "(pa_prefill_write) call")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline time budget")
    p.add_argument("--block-size", type=int, default=16,
                   help="waste workloads: tokens per KV block of the paged run (the block-size knob)")
    return p.parse_args(argv)


# --- step planning (host block manager) --------------------------------------------

class StepPlan:
    """Per-step metadata produced by the host block manager (row a1)."""

    def __init__(self, case, nsteps, pkv):
        bs = case.block_size
        b = case.num_seqs
        lens0 = case.context_lens.astype(np.int64)
        # hand blocks out in the case's shuffled order: each sequence's own
        # table first, then the rest of the pool
        used = [int(x) for s in range(b) for x in case.block_tables[s, :W.ceil_div(lens0[s], bs)]]
        rest = np.setdiff1d(np.arange(case.num_blocks), np.asarray(used, np.int64), assume_unique=False)
        order = np.concatenate([np.asarray(used, np.int32), rest.astype(np.int32)])
        need = int(sum(W.ceil_div(c + nsteps, bs) for c in lens0))
        if need > case.num_blocks:
            raise ValueError("pool too small for the planned steps")
        pool = pkv.BlockPool(case.num_blocks, bs, order)
        seqs = list(range(b))
        for s in seqs:
            pool.create(s, int(lens0[s]) - 1)
        self.max_blocks = W.ceil_div(int(lens0.max()) + nsteps, bs)
        self.slots, self.pairs, self.tables, self.lens = [], [], [], []
        t0 = time.perf_counter()
        for _ in range(nsteps):
            slots, pairs = pool.append_batch(seqs)
            tables, lens = pool.tables(seqs, self.max_blocks)
            self.slots.append(slots.copy())
            self.pairs.append(pairs.copy())
            self.tables.append(tables)
            self.lens.append(lens)
        self.host_prep_us = (time.perf_counter() - t0) / max(nsteps, 1) * 1e6
        pool.close()

    def step_bytes(self, i, case):
        """Algorithmic bytes of step i: (decode K/V + table, write, copy)."""
        lens = self.lens[i].astype(np.int64)
        elt = case.elt_bytes()
        row = case.head_dim * elt
        kv = int(lens.sum()) * case.num_kv_heads * 2 * row
        table = 4 * int(sum(W.ceil_div(c, case.block_size) for c in lens))
        ntok = int((self.slots[i] >= 0).sum())
        write = ntok * case.num_kv_heads * row * 2 * 2 + 8 * len(self.slots[i])
        block_bytes = case.num_kv_heads * case.block_size * row
        copy = len(self.pairs[i]) * block_bytes * 2 * 2
        return kv + table, write, copy


# --- traffic counters (rocprofv3 --pmc summaries) -----------------------------------

def decode_kernels(case, partition, fused=False):
    """Kernels one timed decode call launches (the library's dispatch rule);
    with the fused write, the balanced kernel stores the tokens itself and
    the other paths launch write_kv_kernel first."""
    gqa = case.dtype == W.BF16 and case.num_q_heads // case.num_kv_heads in (4, 8) and case.head_dim in (64, 128, 256)
    if gqa and partition == -1:
        return "decode_gqa_balanced+merge_balanced_kernel"
    if partition == -1:  # the vector-ALU kernel: 1024-token partitions past 1024 tokens
        partition = 1024 if case.max_context > 1024 else 0
    pre = "write_kv_kernel+" if fused else ""
    if gqa:
        return pre + "decode_gqa_kernel" + ("+merge_kernel" if partition else "")
    return pre + "decode_kernel" + ("+merge_kernel" if partition > 0 else "")


def source_digest():
    """Digest of the decode kernels' sources with comments and whitespace
    removed (the counters are tied to it: a change to the code drops them, a
    change to a comment does not)."""
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, partition):
    """HBM bytes per decode launch from the committed counter summary, if it
    was taken on the current decode source with this partition size."""
    path = TRAFFIC_FILE.format(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+).*?source_sha256_16:\s*([0-9a-f]+).*?"
                  r"partition_size:\s*(-?\d+)", text, re.S)
    if not m or m.group(2) != source_digest() or int(m.group(3)) != partition:
        return None
    return int(m.group(1))


# --- CPU baseline (oracle) -------------------------------------------------------------

def oracle_cores():
    """Cores the oracle baseline may use: this process's CPU affinity, at
    most 16 (one GPU's share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_decode_worker(job):
    """One oracle worker (a fresh process, one BLAS thread): decodes its
    sequences of the batch one after another, cycling, for ``budget``
    seconds; returns (bytes, tokens, sequence decodes, seconds)."""
    (shm_k, shm_v, pool_shape, pool_dtype, q, tables, lens, seqs, scale, dtype, budget, hkv, d, elt, bs) = job
    from multiprocessing import shared_memory

    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    mk, mv = shared_memory.SharedMemory(name=shm_k), shared_memory.SharedMemory(name=shm_v)
    try:
        k = np.ndarray(pool_shape, dtype=pool_dtype, buffer=mk.buf)
        v = np.ndarray(pool_shape, dtype=pool_dtype, buffer=mv.buf)
        done, tok, n = 0, 0, 0
        with threadpool_limits(1):
            t0 = time.perf_counter()
            while True:
                s = seqs[n % len(seqs)]
                A.decode(q[s:s + 1], k, v, tables[s:s + 1], lens[s:s + 1], scale, dtype)
                c = int(lens[s])
                done += c * hkv * 2 * d * elt + 4 * W.ceil_div(c, bs)
                tok += c
                n += 1
                if time.perf_counter() - t0 >= budget:
                    break
            dt = time.perf_counter() - t0
        del k, v
    finally:
        mk.close()
        mv.close()
    return done, tok, n, dt


def cpu_baseline(case, plan, budget_s, workers=None):
    """The fp64 oracle on the step-0 batch on this host's cores: the
    sequences are dealt round-robin to ``oracle_cores()`` worker processes
    (spawned fresh, one BLAS thread each, the pools in shared memory), each
    decoding its sequences one by one, cycling, for the time budget; the rate
    is scaled to the metric's unit.  A single worker alone is timed after
    that (a quarter of the budget) for the one-core figure."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    tables, lens = plan.tables[0], plan.lens[0]
    n_work = workers or oracle_cores()
    shms = []
    try:
        for arr in (case.k_cache, case.v_cache):
            m = shared_memory.SharedMemory(create=True, size=arr.nbytes)
            np.ndarray(arr.shape, arr.dtype, buffer=m.buf)[...] = arr
            shms.append(m)

        def jobs(n, budget):
            return [(shms[0].name, shms[1].name, case.k_cache.shape, case.k_cache.dtype, case.q, tables, lens,
                     list(range(w, case.num_seqs, n)), case.scale, case.dtype, budget, case.num_kv_heads,
                     case.head_dim, case.elt_bytes(), case.block_size) for w in range(n)]

        ctx = mp.get_context("spawn")
        t0 = time.perf_counter()
        with ctx.Pool(n_work) as pool:
            res = pool.map(_oracle_decode_worker, jobs(n_work, budget_s))
        wall = time.perf_counter() - t0
        with ctx.Pool(1) as pool:
            one = pool.map(_oracle_decode_worker, jobs(1, budget_s / 4))[0]
    finally:
        for m in shms:
            m.close()
            m.unlink()
    done = sum(r[0] for r in res)
    tok = sum(r[1] for r in res)
    n = sum(r[2] for r in res)
    dt = max(r[3] for r in res)
    return {"value": round(done / dt / 1e9, 4), "unit": "GB/s", "cores": n_work, "kind": "oracle",
            "sample": f"fp64 oracle, {n_work} worker processes x 1 BLAS thread, the {case.num_seqs} sequences "
                      f"of step 0 dealt round-robin, {n} sequence decodes ({tok} tokens x {case.num_q_heads} "
                      f"q heads) in {dt:.1f} s per worker ({wall:.1f} s with process start)",
            "tokens_per_s": round(tok / dt, 1), "seconds": round(dt, 2),
            "single_core": {"value": round(one[0] / one[3] / 1e9, 4), "unit": "GB/s",
                            "tokens_per_s": round(one[1] / one[3], 1), "seconds": round(one[3], 2),
                            "sequence_decodes": one[2]}}


def causal_flops(context_lens, cu_seqlens, num_q_heads, head_dim):
    """Algorithmic flops of one pa_prefill call: for every (query, visible
    key, query head), 2d for q.k and 2d for p.v."""
    lens = np.asarray(context_lens, dtype=np.int64)
    nq = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    pairs = 0
    for ctx, n in zip(lens, nq):
        first = ctx - n  # position of the first query
        # sum over i < n of (first + i + 1) visible keys, clipped at 0
        pos = np.arange(n, dtype=np.int64) + first + 1
        pairs += int(np.clip(pos, 0, None).sum())
    return pairs * num_q_heads * 4 * head_dim


def prefill_kernel_name(head_dim, block_size):
    """The pa_prefill kernel that serves a shape: tiles loaded straight into
    LDS for head_dim 128 at block sizes of 8 and up, staged through
    registers otherwise."""
    return "prefill_ring_kernel" if head_dim == 128 and block_size >= 8 else "prefill_kernel"


def prefill_flops(pc):
    return causal_flops(pc.case.context_lens, pc.cu_seqlens, pc.case.num_q_heads, pc.case.head_dim)


def prefill_cpu_baseline(pc, budget_s):
    """fp64 oracle rows (every head of a token) cycling over the chunk's
    tokens until the budget is spent; TFLOP/s on the same flop count."""
    from threadpoolctl import threadpool_limits
    one_core = threadpool_limits(1)  # the oracle on one BLAS thread

    from oracle import prefill as P

    c = pc.case
    grp = c.num_q_heads // c.num_kv_heads
    rows = [(s, i) for s in range(c.num_seqs) for i in range(int(pc.cu_seqlens[s + 1] - pc.cu_seqlens[s]))]
    order = np.random.default_rng(0).permutation(len(rows))
    flops, n = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        s, i = rows[order[n % len(rows)]]
        ctx = int(c.context_lens[s])
        nq = int(pc.cu_seqlens[s + 1] - pc.cu_seqlens[s])
        pos = ctx - nq + i
        for h in range(c.num_q_heads):
            P.prefill_row(pc.q[pc.cu_seqlens[s] + i, h], c.k_cache, c.v_cache, c.block_tables[s], ctx, pos, c.scale,
                          c.dtype, h // grp)
        flops += max(pos + 1, 0) * c.num_q_heads * 4 * c.head_dim
        n += 1
    dt = time.perf_counter() - t0
    threads = 1  # run under threadpool_limits(1): one core
    one_core.restore_original_limits()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle rows (all {c.num_q_heads} heads of a token), {n} tokens drawn at random "
                      f"from the chunk, {dt:.1f} s wall", "seconds": round(dt, 2)}


def prefill_main(args, torch, pkv, dev):
    """One step: the chunk's tokens stored and their queries attended, as one
    pa_prefill_write call (or pa_write_kv, then pa_prefill, with
    --separate-write)."""
    log(f"workload {args.workload}: drawing inputs")
    pc = PREFILL_WORKLOADS[args.workload]()
    c = pc.case

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    k0, v0 = dev_t(c.k_cache), dev_t(c.v_cache)
    layers = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(max(args.layers, 1) - 1)]
    q, kn, vn, slots = dev_t(pc.q), dev_t(pc.k_new), dev_t(pc.v_new), dev_t(pc.slot_mapping)
    tables, lens, cu = dev_t(c.block_tables), dev_t(c.context_lens), dev_t(pc.cu_seqlens)
    out = torch.empty_like(q)
    fused = not args.separate_write
    steps = []
    for kc, vc in layers:
        if fused:
            steps.append((pkv.prepare_prefill_write(kn, vn, slots, q, kc, vc, tables, lens, cu, pc.max_query_len,
                                                    c.max_context, c.scale, out),))
        else:
            steps.append((pkv.prepare_write_kv(kn, vn, slots, kc, vc),
                          pkv.prepare_prefill(q, kc, vc, tables, lens, cu, pc.max_query_len, c.max_context,
                                              c.scale, out)))
    torch.cuda.synchronize()
    for i in range(args.warmup):
        for call in steps[i % len(steps)]:
            call()
    torch.cuda.synchronize()
    log(f"timed {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        for call in steps[i % len(steps)]:
            call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        steps[i % len(steps)][-1]()  # the attention call (with the store when fused)
    e1.record()
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) / 1e3 / args.steps
    flops = prefill_flops(pc)
    achieved = flops / avg / 1e12
    elt = 2
    write_bytes = pc.num_tokens * c.num_kv_heads * c.head_dim * elt * 2 * 2
    result = {
        "metric": PREFILL_METRIC,
        "value": round(flops / (wall / args.steps) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled block placement)",
        "config": {"workload": args.workload, "num_seqs": c.num_seqs, "num_q_heads": c.num_q_heads,
                   "num_kv_heads": c.num_kv_heads, "head_dim": c.head_dim, "block_size": c.block_size,
                   "query_tokens": pc.num_tokens, "context_len_mean": round(float(c.context_lens.mean()), 1),
                   "context_len_max": int(c.context_lens.max()), "kv_pool_copies": len(layers),
                   "write_fused_into_prefill": fused},
        "pct_of_peak": round(100.0 * flops / (wall / args.steps) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2),
        "flops_per_step": flops,
        "write_bytes_per_step": write_bytes,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": prefill_kernel_name(c.head_dim, c.block_size), "avg_launch_us": round(avg * 1e6, 2),
                     "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        result["cpu_baseline"] = prefill_cpu_baseline(pc, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def swap_main(args, torch, pkv, dev):
    """Each step swaps every fourth sequence out (device -> pinned host) and
    back in; the host manager picks the blocks, pa_swap_blocks moves them."""
    log(f"workload {args.workload}: drawing inputs")
    c = SWAP_WORKLOADS[args.workload]()
    pool = pkv.BlockPool(c.num_blocks, c.block_size, np.random.default_rng(0).permutation(c.num_blocks))
    swap_seqs = list(range(0, c.num_seqs, 4))
    host_blocks = sum(W.ceil_div(int(c.context_lens[s]), c.block_size) for s in swap_seqs)
    pool.set_swap_space(host_blocks)
    for s in range(c.num_seqs):
        pool.create(s, int(c.context_lens[s]))

    def dev_t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    kd, vd = dev_t(c.k_cache), dev_t(c.v_cache)
    shape = (host_blocks,) + tuple(kd.shape[1:])
    kh = torch.zeros(shape, dtype=torch.bfloat16).pin_memory()
    vh = torch.zeros(shape, dtype=torch.bfloat16).pin_memory()
    block_bytes = c.num_kv_heads * c.block_size * c.head_dim * 2 * 2  # K and V

    def plan():
        """(out pairs, in pairs) of one round trip, from the manager."""
        outs = np.concatenate([pool.swap_out(s) for s in swap_seqs])
        ins = np.concatenate([pool.swap_in(s) for s in swap_seqs])
        return torch.from_numpy(outs).to(dev), torch.from_numpy(ins).to(dev)

    rounds = [plan() for _ in range(max(args.steps, args.warmup, 1))]
    n_blocks = int(rounds[0][0].shape[0])
    torch.cuda.synchronize()
    for i in range(args.warmup):
        pkv.pa_swap_blocks(kd, vd, kh, vh, rounds[i][0])
        pkv.pa_swap_blocks(kh, vh, kd, vd, rounds[i][1])
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        pkv.pa_swap_blocks(kd, vd, kh, vh, rounds[i][0])
        ev[i][1].record()
        pkv.pa_swap_blocks(kh, vh, kd, vd, rounds[i][1])
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_out = float(np.mean([a.elapsed_time(b) for a, b, _ in ev])) / 1e3
    t_in = float(np.mean([b.elapsed_time(e) for _, b, e in ev])) / 1e3
    moved = n_blocks * block_bytes
    result = {
        "metric": SWAP_METRIC,
        "value": round(2 * moved * args.steps / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V pools, shuffled block placement)",
        "config": {"workload": args.workload, "num_seqs_swapped": len(swap_seqs), "blocks_per_direction": n_blocks,
                   "bytes_per_direction": moved, "block_bytes_k_plus_v": block_bytes},
        "out_GBps": round(moved / t_out / 1e9, 2),
        "in_GBps": round(moved / t_in / 1e9, 2),
        "roofline": {"bound": "pcie", "achieved": round(moved / ((t_out + t_in) / 2) / 1e9, 2),
                     "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(moved / ((t_out + t_in) / 2) / 1e9 / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                     "kernel": "copy_blocks_kernel", "avg_launch_us": round((t_out + t_in) / 2 * 1e6, 2)},
        "cpu_baseline": None,
    }
    pool.close()
    print(json.dumps(result), flush=True)
    return 0


def prefix_cpu_baseline(plan, budget_s):
    """fp64 oracle rows (every head of a token) for suffix queries drawn at
    random, attending over the request's whole prompt (the cached path's
    work); prompt tokens/s = computed rows/s x prompt tokens per computed
    token."""
    from threadpoolctl import threadpool_limits
    one_core = threadpool_limits(1)  # the oracle on one BLAS thread

    from oracle import prefill as P

    bs, hkv, d = plan.block_size, plan.num_kv_heads, plan.head_dim
    grp = plan.num_q_heads // hkv
    cu = plan.suffix_cu
    rng = np.random.default_rng(0)
    pools = {}

    def pool_of(s):
        """Request s's whole prompt K/V laid out as a private contiguous pool."""
        if s not in pools:
            n = plan.prefix_len + int(plan.suffix_lens[s])
            nb = W.ceil_div(n, bs)
            out = []
            for pre, suf in ((plan.prefix_k, plan.suffix_k), (plan.prefix_v, plan.suffix_v)):
                rows = np.zeros((nb * bs, hkv, d), np.uint16)
                rows[:plan.prefix_len] = pre
                rows[plan.prefix_len:n] = suf[cu[s]:cu[s + 1]]
                out.append(rows.reshape(nb, bs, hkv, d).transpose(0, 2, 1, 3).copy())
            pools.clear()
            pools[s] = (out[0], out[1], np.arange(nb, dtype=np.int32), n)
        return pools[s]

    rows_done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        s = int(rng.integers(plan.num_seqs))
        kc, vc, table, n = pool_of(s)
        for i in rng.integers(0, int(plan.suffix_lens[s]), 8):
            pos = plan.prefix_len + int(i)
            for h in range(plan.num_q_heads):
                P.prefill_row(plan.suffix_q[cu[s] + i, h], kc, vc, table, n, pos, plan.scale, plan.dtype, h // grp)
            rows_done += 1
    dt = time.perf_counter() - t0
    prompt_tokens = plan.num_seqs * plan.prefix_len + int(plan.suffix_lens.sum())
    per_computed = prompt_tokens / int(plan.suffix_lens.sum())
    threads = 1  # run under threadpool_limits(1): one core
    one_core.restore_original_limits()
    return {"value": round(rows_done / dt * per_computed, 3), "unit": "prompt tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 oracle rows (all {plan.num_q_heads} heads of a token) for {rows_done} suffix queries "
                      f"drawn at random, each over its whole prompt, {dt:.1f} s wall; scaled by "
                      f"{per_computed:.2f} prompt tokens per computed token", "seconds": round(dt, 2)}


def prefix_main(args, torch, pkv, dev):
    """Admission of a batch of prompts sharing a cached system prompt.

    Host (planned before the timed region, timed on its own): the batch
    admission call (each request's cached prefix and the slots of its
    uncached tokens) and the batch tables; the batch is released after the
    step (the system
    prompt's blocks go back to the LRU list, where the next step finds
    them).  Device, per step: pa_write_kv of the uncached tokens, then
    pa_prefill of their queries over the whole prompts.  The same batch
    without the cache (every prompt stored and prefilled whole) is timed
    beside it."""
    log(f"workload {args.workload}: drawing inputs")
    plan = PREFIX_WORKLOADS[args.workload]()
    B, bs = plan.num_seqs, plan.block_size
    nsteps = args.warmup + args.steps

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    shape = (plan.num_blocks, plan.num_kv_heads, bs, plan.head_dim)
    kc, vc = torch.zeros(shape, dtype=torch.bfloat16, device=dev), torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    pool = pkv.BlockPool(plan.num_blocks, bs, plan.free_order)
    pool.enable_prefix_cache()
    # the system prompt is already cached when the measured traffic starts
    assert pool.create_cached(-1, plan.prefix_tokens) == 0
    pkv.pa_write_kv(dev_t(plan.prefix_k), dev_t(plan.prefix_v),
                    dev_t(np.asarray(pool.slots(-1, 0, plan.prefix_len), np.int64)), kc, vc)
    pool.release(-1)

    log(f"planning {nsteps} steps with the host manager")
    lens = (plan.prefix_len + plan.suffix_lens).astype(np.int32)
    mb = W.ceil_div(int(lens.max()), bs)
    host_s, plans, cached_tokens = 0.0, [], 0
    for t in range(nsteps):
        prompts = [plan.prompt(t, s) for s in range(B)]
        t0 = time.perf_counter()
        cached, slots, refused = pool.create_cached_batch(list(range(B)), prompts)
        if refused is not None:
            raise RuntimeError(f"step {t}: admission refused: {refused}")
        cached = cached.tolist()
        tables, ctx = pool.tables(list(range(B)), mb)
        for s in range(B):
            pool.release(s)
        host_s += time.perf_counter() - t0
        if any(c != plan.prefix_len for c in cached):
            raise RuntimeError(f"step {t}: expected the {plan.prefix_len}-token system prompt cached, got {cached}")
        cached_tokens += sum(cached)
        plans.append((dev_t(slots), dev_t(tables)))
    cu = dev_t(plan.suffix_cu)
    ctx_d = dev_t(lens)
    q, kn, vn = dev_t(plan.suffix_q), dev_t(plan.suffix_k), dev_t(plan.suffix_v)
    out = torch.empty_like(q)
    max_q = int(plan.suffix_lens.max())
    fused = not args.separate_write

    def store_and_attend(k, v, slots, q_, tables, cu_, max_q_, out_):
        # the step's store and attention: one pa_prefill_write call, or the two calls
        if fused:
            return (pkv.prepare_prefill_write(k, v, slots, q_, kc, vc, tables, ctx_d, cu_, max_q_, int(lens.max()),
                                              plan.scale, out_),)
        return (pkv.prepare_write_kv(k, v, slots, kc, vc),
                pkv.prepare_prefill(q_, kc, vc, tables, ctx_d, cu_, max_q_, int(lens.max()), plan.scale, out_))

    steps = [store_and_attend(kn, vn, slots, q, tables, cu, max_q, out) for slots, tables in plans]

    def timed(calls, kernel_index):
        torch.cuda.synchronize()
        for i in range(args.warmup):
            for c in calls[i % len(calls)]:
                c()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            for c in calls[(args.warmup + i) % len(calls)]:
                c()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            calls[(args.warmup + i) % len(calls)][kernel_index]()
        e1.record()
        torch.cuda.synchronize()
        return wall / args.steps, e0.elapsed_time(e1) / 1e3 / args.steps

    log(f"timed {args.steps} cached steps")
    step_s, prefill_s = timed(steps, -1)

    log("uncached comparison: every prompt stored and prefilled whole")
    pool_u = pkv.BlockPool(plan.num_blocks, bs, plan.free_order)
    for s in range(B):
        pool_u.create(s, int(lens[s]))
    tab_u, _ = pool_u.tables(list(range(B)), mb)
    slots_u = np.concatenate([np.asarray(pool_u.slots(s, 0, int(lens[s])), np.int64) for s in range(B)])
    pool_u.close()
    cu_full = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    suf_cu = plan.suffix_cu
    qp, kp, vp = dev_t(plan.prefix_q), dev_t(plan.prefix_k), dev_t(plan.prefix_v)
    qf = torch.cat([x for s in range(B) for x in (qp, q[suf_cu[s]:suf_cu[s + 1]])])
    kf = torch.cat([x for s in range(B) for x in (kp, kn[suf_cu[s]:suf_cu[s + 1]])])
    vf = torch.cat([x for s in range(B) for x in (vp, vn[suf_cu[s]:suf_cu[s + 1]])])
    out_f = torch.empty_like(qf)
    steps_u = [store_and_attend(kf, vf, dev_t(slots_u), qf, dev_t(tab_u), dev_t(cu_full), int(lens.max()), out_f)]
    step_u, prefill_u = timed(steps_u, -1)

    prompt_tokens = int(lens.sum())
    computed = int(plan.suffix_lens.sum())
    flops = causal_flops(lens, plan.suffix_cu, plan.num_q_heads, plan.head_dim)
    achieved = flops / prefill_s / 1e12
    result = {
        "metric": PREFIX_METRIC,
        "value": round(prompt_tokens / step_s, 1),
        "unit": "prompt tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/K/V, seeded token ids, shuffled block placement)",
        "config": {"workload": args.workload, "requests_per_step": B, "system_prompt_tokens": plan.prefix_len,
                   "suffix_tokens_min": int(plan.suffix_lens.min()), "suffix_tokens_max": int(plan.suffix_lens.max()),
                   "prompt_tokens_per_step": prompt_tokens, "computed_tokens_per_step": computed,
                   "num_q_heads": plan.num_q_heads, "num_kv_heads": plan.num_kv_heads,
                   "head_dim": plan.head_dim, "block_size": bs, "write_fused_into_prefill": fused},
        "cache_hit_fraction": round(cached_tokens / (nsteps * prompt_tokens), 4),
        "host_manager_us_per_request": round(host_s / (nsteps * B) * 1e6, 2),
        "uncached_tokens_per_s": round(prompt_tokens / step_u, 1),
        "uncached_ms_per_step": round(step_u * 1e3, 5),
        "speedup_vs_uncached": round(step_u / step_s, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": prefill_kernel_name(plan.head_dim, bs), "avg_launch_us": round(prefill_s * 1e6, 2),
                     "algorithmic_flops_per_launch": flops,
                     "uncached_avg_launch_us": round(prefill_u * 1e6, 2)},
        "cpu_baseline": None,
    }
    pool.close()
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        result["cpu_baseline"] = prefix_cpu_baseline(plan, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def cow_main(args, torch, pkv, dev):
    """Shared-prefix steps: copy-on-write copies, then pa_decode_write (the
    new tokens stored inside the balanced decode).  The host manager plans
    every step before the timed region; the timed region replays the planned
    steps in order (a replay copies the same blocks again and stores the same
    tokens, so the pools stay as the plan left them)."""
    log(f"workload {args.workload}: drawing inputs")
    plan = COW_WORKLOADS[args.workload]()
    bs, B, hkv, d = plan.block_size, plan.num_seqs, plan.num_kv_heads, plan.head_dim
    prefix_blocks = plan.prefix_len // bs
    block_bytes = hkv * bs * d * 2  # one pool's block, bf16

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    pool = pkv.BlockPool(plan.num_blocks, bs, plan.free_order)
    kdev = torch.zeros((plan.num_blocks, hkv, bs, d), dtype=torch.bfloat16, device=dev)
    vdev = torch.zeros_like(kdev)
    pool.create(0, plan.prefix_len)
    pkv.pa_write_kv(dev_t(plan.prefix_k.transpose(1, 0, 2)), dev_t(plan.prefix_v.transpose(1, 0, 2)),
                    dev_t(np.asarray(pool.slots(0, 0, plan.prefix_len), np.int64)), kdev, vdev)
    for s_ in range(1, B):
        pool.fork(0, s_)
    for s_ in range(B):
        n = int(plan.suffix_lens[s_])
        if n:
            sl = np.array([pool.append(s_)[0] for _ in range(n)], np.int64)
            pkv.pa_write_kv(dev_t(plan.suffix_k[s_].transpose(1, 0, 2)), dev_t(plan.suffix_v[s_].transpose(1, 0, 2)),
                            dev_t(sl), kdev, vdev)

    log(f"planning {plan.steps} steps with the host manager")
    seqs = list(range(B))
    steps, logical, unique, copies = [], [], [], []
    host_s = 0.0
    for step in range(plan.steps):
        cands = [(s_, lb) for s_ in seqs for lb, blk in enumerate(pool.table(s_)[:prefix_blocks])
                 if pool.refcount(int(blk)) > 1]
        picks = plan.pick(cands)
        t0 = time.perf_counter()  # the manager's calls only (the picks are the workload's)
        pairs = [pool.cow(s_, lb) for s_, lb in picks]
        pairs = np.array([pr for pr in pairs if pr is not None], np.int64).reshape(-1, 2)
        slots, cow = pool.append_batch(seqs)
        # copies an append asked for (none here: every tail block is private) go with the step's copies
        pairs = np.concatenate([pairs, np.asarray(cow, np.int64).reshape(-1, 2)])
        mb = max(len(pool.table(s_)) for s_ in seqs)
        tables, lens = pool.tables(seqs, mb)
        host_s += time.perf_counter() - t0
        q = plan.step_q()
        k_new, v_new = plan.step_tokens()
        # bytes: logical = every sequence's context; unique = each distinct block's used tokens once
        lens64 = lens.astype(np.int64)
        tok_bytes = hkv * 2 * d * 2
        logical.append(int(lens64.sum()) * tok_bytes + 4 * sum(W.ceil_div(int(c), bs) for c in lens64))
        used = {}
        for i, c in enumerate(lens64):
            for j in range(W.ceil_div(int(c), bs)):
                blk = int(tables[i, j])
                used[blk] = max(used.get(blk, 0), min(bs, int(c) - j * bs))
        unique.append(sum(used.values()) * tok_bytes)
        copies.append(len(pairs))
        steps.append((dev_t(pairs), dev_t(slots), dev_t(q), dev_t(k_new), dev_t(v_new), dev_t(tables), dev_t(lens),
                      int(lens.max())))
    max_ctx = max(st[-1] for st in steps)
    out = torch.empty_like(steps[0][2])
    ws_bytes = pkv.pa_decode_workspace_bytes(B, plan.num_q_heads, hkv, d, max_ctx, BALANCED)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev) if ws_bytes else None
    calls = []
    for pairs, slots, q, k_new, v_new, tables, lens, mc in steps:
        calls.append((pkv.prepare_copy_blocks(kdev, vdev, pairs),
                      pkv.prepare_decode_write(k_new, v_new, slots, q, kdev, vdev, tables, lens, mc, plan.scale, out,
                                               partition_size=BALANCED, workspace=ws)))
    nplan = len(calls)
    torch.cuda.synchronize()
    for i in range(max(args.warmup, nplan)):
        for c in calls[i % nplan]:
            c()
    torch.cuda.synchronize()
    log(f"timed {args.steps} steps (replaying the {nplan} planned steps in order)")
    t0 = time.perf_counter()
    for i in range(args.steps):
        for c in calls[i % nplan]:
            c()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        calls[i % nplan][1]()
    e1.record()
    torch.cuda.synchronize()
    dec_s = e0.elapsed_time(e1) / 1e3 / args.steps
    idx = [i % nplan for i in range(args.steps)]
    write_bytes = B * hkv * d * 2 * 2 * 2  # new K and V rows read and stored
    copy_bytes = [c * block_bytes * 2 * 2 for c in copies]  # K and V blocks read and written
    step_logical = sum(logical[i] + write_bytes + copy_bytes[i] for i in idx) / args.steps
    step_unique = sum(unique[i] + write_bytes + copy_bytes[i] for i in idx) / args.steps
    dec_logical = sum(logical[i] + write_bytes for i in idx) / args.steps
    dec_unique = sum(unique[i] + write_bytes for i in idx) / args.steps
    step_s = wall / args.steps
    result = {
        "metric": COW_METRIC, "value": round(step_logical / step_s / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": max(args.warmup, nplan),
        "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q, shuffled block placement)",
        "config": {"workload": args.workload, "num_seqs": B, "prefix_tokens": plan.prefix_len,
                   "num_q_heads": plan.num_q_heads, "num_kv_heads": hkv, "head_dim": d, "block_size": bs,
                   "planned_steps": nplan, "cow_copies_per_step": int(np.mean(copies)),
                   "pool_blocks": plan.num_blocks},
        "unique_GBps": round(step_unique / step_s / 1e9, 1),
        "logical_bytes_per_step": int(step_logical), "unique_bytes_per_step": int(step_unique),
        "host_prep_us_per_step": round(host_s / nplan * 1e6, 1),
        "roofline": {"bound": "hbm", "achieved": round(dec_unique / dec_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_unique / dec_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_gqa_balanced+merge_balanced_kernel", "avg_launch_us": round(dec_s * 1e6, 2),
                     "algorithmic_bytes_per_launch": int(dec_unique),
                     "logical_GBps": round(dec_logical / dec_s / 1e9, 1),
                     "note": "achieved counts each distinct block's used tokens once (the bytes HBM must "
                             "deliver at least); logical counts every sequence's whole context"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        from threadpoolctl import threadpool_limits
        one_core = threadpool_limits(1)  # the oracle on one BLAS thread

        from oracle import attention as A

        kh = kdev.view(torch.int16).cpu().numpy().view(np.uint16)
        vh = vdev.view(torch.int16).cpu().numpy().view(np.uint16)
        _, _, q0, _, _, t0d, l0d, _ = steps[-1]
        qh = q0.view(torch.int16).cpu().numpy().view(np.uint16)
        th, lh = t0d.cpu().numpy(), l0d.cpu().numpy()
        done, n = 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            s_ = n % B
            A.decode(qh[s_:s_ + 1], kh, vh, th[s_:s_ + 1], lh[s_:s_ + 1], plan.scale, plan.dtype)
            done += int(lh[s_]) * hkv * 2 * d * 2 + 4 * W.ceil_div(int(lh[s_]), bs)
            n += 1
        dt = time.perf_counter() - t0
        threads = 1  # run under threadpool_limits(1): one core
        one_core.restore_original_limits()
        result["cpu_baseline"] = {"value": round(done / dt / 1e9, 4), "unit": "GB/s (logical)", "cores": int(threads),
                                  "kind": "oracle",
                                  "sample": f"fp64 oracle, {n} sequence decodes of the last planned step, "
                                            f"{dt:.1f} s wall", "seconds": round(dt, 2)}
    pool.close()
    print(json.dumps(result), flush=True)
    return 0


def waste_main(args):
    """Host-only: the serving-loop simulation of both allocators, timed."""
    import paged_kv_cache_354_amd as pkv

    case = WASTE_WORKLOADS[args.workload]()
    case.block_size = args.block_size
    args_c = (case.capacity, case.block_size, case.prompt_lens, case.output_lens, case.reserve_lens)
    res, secs = {}, {}
    for mode in ("contiguous", "paged"):
        t0 = time.perf_counter()
        for _ in range(args.steps):
            res[mode] = pkv.pa_waste_simulate(mode, *args_c)
        secs[mode] = (time.perf_counter() - t0) / args.steps

    def summary(st):
        return {"waste_pct": round(100.0 * (1 - st["live_slot_steps"] / st["held_slot_steps"]), 3),
                "mean_running": round(st["running_steps"] / st["steps"], 2), "max_running": st["max_running"],
                "steps": st["steps"], "tokens_per_step": round(st["decode_tokens"] / st["steps"], 2),
                "preemptions": st["preemptions"], "frag_blocked_steps": st["frag_blocked_steps"]}

    c, pg = summary(res["contiguous"]), summary(res["paged"])
    result = {
        "metric": WASTE_METRIC, "value": pg["waste_pct"], "unit": "%",
        "n_gpus": 1, "steps": args.steps, "warmup": 0,
        "ms_per_step": round(secs["paged"] * 1e3, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "int64",
        "data": "synthetic (seeded request lengths)",
        "config": {"workload": args.workload, "requests": len(case.prompt_lens), "capacity_slots": case.capacity,
                   "block_size": case.block_size, "prompt_tokens_mean": round(float(case.prompt_lens.mean()), 1),
                   "output_tokens_mean": round(float(case.output_lens.mean()), 1),
                   "slab_slots_mean": round(float(case.reserve_lens.mean()), 1)},
        "paged": pg, "contiguous": c,
        "concurrency_gain": round(pg["mean_running"] / c["mean_running"], 3),
        "makespan_ratio_contiguous_over_paged": round(c["steps"] / pg["steps"], 3),
        "sim_seconds": {k: round(v, 4) for k, v in secs.items()},
        "roofline": None,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        one_core = threadpool_limits(1)  # the oracle on one BLAS thread

        from oracle import waste as WS

        k = 64  # about 20 s of the oracle (its manager model copies its state on every call)
        small = case.scaled(k)
        t0 = time.perf_counter()
        st = WS.simulate("paged", small.capacity, small.block_size, small.prompt_lens, small.output_lens,
                         small.reserve_lens)
        dt = time.perf_counter() - t0
        threads = 1  # run under threadpool_limits(1): one core
        one_core.restore_original_limits()
        result["cpu_baseline"] = {
            "value": round(100.0 * st.waste(), 3), "unit": "%", "cores": int(threads), "kind": "oracle",
            "sample": f"the oracle's paged run on 1/{k} of the requests and of the pool "
                      f"({len(small.prompt_lens)} requests, {small.capacity} slots), {dt:.2f} s wall",
            "seconds": round(dt, 2)}
    print(json.dumps(result), flush=True)
    return 0


# --- main ------------------------------------------------------------------------------

def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: runs on exactly one GPU (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the decode path has no multi-GPU mode", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    if args.workload in WASTE_WORKLOADS:
        return waste_main(args)

    import torch

    import paged_kv_cache_354_amd as pkv

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    pkv.load()  # raises when the HIP library is missing: there is no other path
    dev = torch.device("cuda:0")
    if args.workload in PREFILL_WORKLOADS:
        return prefill_main(args, torch, pkv, dev)
    if args.workload in SWAP_WORKLOADS:
        return swap_main(args, torch, pkv, dev)
    if args.workload in PREFIX_WORKLOADS:
        return prefix_main(args, torch, pkv, dev)
    if args.workload in COW_WORKLOADS:
        return cow_main(args, torch, pkv, dev)
    make, default_part = WORKLOADS[args.workload]
    partition = default_part if args.partition is None else args.partition

    log(f"workload {args.workload}: drawing inputs")
    case = make()
    # Warmup and timed steps replay the planned steps cyclically: a replayed
    # step stores the same tokens in the same slots and attends over the same
    # contexts, all of its work done again, so the contexts the timed steps
    # see stay within the workload's distribution (+ at most plan_steps - 1
    # tokens) however many steps are timed.
    nplan = max(1, min(args.steps, args.plan_steps))
    plan = StepPlan(case, nplan, pkv)
    log(f"planned {nplan} steps, host prep {plan.host_prep_us:.1f} us/step, pool {case.num_blocks} blocks")

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    k0, v0 = dev_t(case.k_cache), dev_t(case.v_cache)
    layers = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(max(args.layers, 1) - 1)]
    q, k_new, v_new = dev_t(case.q), dev_t(case.k_new), dev_t(case.v_new)
    slots = [dev_t(x) for x in plan.slots]
    tables = [dev_t(x) for x in plan.tables]
    lens = [dev_t(x) for x in plan.lens]
    pairs = [dev_t(x.reshape(-1, 2).astype(np.int64)) for x in plan.pairs]
    max_ctx = [int(x.max()) for x in plan.lens]
    out = torch.empty_like(q)
    ws_bytes = pkv.pa_decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                             case.head_dim, max(max_ctx), partition)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev) if ws_bytes else None

    # per step: (copy, write, decode); with the fused call the write is part
    # of the decode call
    fused = not args.separate_write
    steps = []
    for i in range(nplan):
        k_cache, v_cache = layers[i % len(layers)]
        if fused:
            write = lambda: None
            decode = pkv.prepare_decode_write(k_new, v_new, slots[i], q, k_cache, v_cache, tables[i], lens[i],
                                              max_ctx[i], case.scale, out, partition_size=partition,
                                              workspace=ws)
        else:
            write = pkv.prepare_write_kv(k_new, v_new, slots[i], k_cache, v_cache)
            decode = pkv.prepare_decode(q, k_cache, v_cache, tables[i], lens[i], max_ctx[i], case.scale, out,
                                        partition_size=partition, workspace=ws)
        steps.append((pkv.prepare_copy_blocks(k_cache, v_cache, pairs[i]), write, decode))

    # calibration copy of known size for the traffic counters (untimed)
    calib_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    del calib_src, calib_dst
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    totals = [plan.step_bytes(i % nplan, case) for i in range(max(args.steps, nplan))]
    dec_bytes = [t[0] + (t[1] if fused else 0) for t in totals]  # what one decode call moves

    # The cache-flushed, placement and read-ceiling measurements run first:
    # they are reported beside the timed steps, and they also take the GPU out
    # of its idle state before the warmup steps, as a serving loop would be.
    cold = None
    if args.cold_steps > 0:
        for i in range(10):  # untimed: out of the idle clocks before the first measured call
            steps[i % nplan][2]()
        n = args.cold_steps
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            flush_sum = flush.sum()  # reads 1 GiB: evicts L2 and the Infinity Cache (untimed)
            cev[i][0].record()
            steps[0][2]()
            cev[i][1].record()
        torch.cuda.synchronize()
        cms = [a.elapsed_time(b) for a, b in cev]
        cold = {"decode_us_median": round(float(np.median(cms)) * 1e3, 2),
                "decode_us_p10": round(float(np.percentile(cms, 10)) * 1e3, 2),
                "decode_us_p90": round(float(np.percentile(cms, 90)) * 1e3, 2),
                "decode_GBps": round(dec_bytes[0] / (float(np.median(cms)) / 1e3) / 1e9, 1),
                "frac_of_peak": round(dec_bytes[0] / (float(np.median(cms)) / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    # Indirection overhead: the same decode (step 0's inputs, no store) on the
    # shuffled pool and on a copy where every sequence's blocks sit at
    # consecutive ids (identity placement), cold cache before each call.
    indirection = None
    if args.cold_steps > 0:
        t0tab, l0 = plan.tables[0], plan.lens[0]
        nbs = [W.ceil_div(int(c), case.block_size) for c in l0]
        base = np.concatenate([[0], np.cumsum(nbs)]).astype(np.int64)
        src = torch.from_numpy(np.concatenate([t0tab[i, :nbs[i]] for i in range(case.num_seqs)]).astype(np.int64))
        src = src.to(dev)
        idk, idv = k0.index_select(0, src), v0.index_select(0, src)
        id_tab = np.full_like(t0tab, -1)
        for i in range(case.num_seqs):
            id_tab[i, :nbs[i]] = np.arange(base[i], base[i + 1])
        variants = {
            "shuffled": pkv.prepare_decode(q, k0, v0, tables[0], lens[0], max_ctx[0], case.scale, out,
                                           partition_size=partition, workspace=ws),
            "identity": pkv.prepare_decode(q, idk, idv, dev_t(id_tab), lens[0], max_ctx[0], case.scale, out,
                                           partition_size=partition, workspace=ws),
        }
        n = 2 * args.cold_steps
        cev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(n)] for name in variants}
        for i in range(n):  # the two placements alternate, so drift hits both alike
            for name, call in variants.items():
                flush_sum = flush.sum()  # untimed cache eviction, as above
                cev[name][i][0].record()
                call()
                cev[name][i][1].record()
        torch.cuda.synchronize()
        med = {name: float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3 for name, ev in cev.items()}
        indirection = {"decode_us_shuffled": round(med["shuffled"], 2), "decode_us_identity": round(med["identity"], 2),
                       "ratio_shuffled_over_identity": round(med["shuffled"] / med["identity"], 4),
                       "note": "step 0 inputs, pa_decode without the store, cold cache, median of "
                               f"{n} alternating calls each"}
        del idk, idv

    # Practical read ceiling of this device: pa_read_probe streams the 1 GiB
    # flush buffer (4x the Infinity Cache) with coalesced non-temporal loads,
    # back to back on the launch stream, timed with HIP events.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probe_s = None
    if args.cold_steps > 0:
        sink = torch.empty(pkv.PA_READ_PROBE_WORKGROUPS, dtype=torch.int32, device=dev)
        for _ in range(3):
            pkv.pa_read_probe(flush, sink)
        n = 20
        e0.record()
        for _ in range(n):
            pkv.pa_read_probe(flush, sink)
        e1.record()
        torch.cuda.synchronize()
        probe_s = e0.elapsed_time(e1) / 1e3 / n
    del flush

    log(f"warmup {args.warmup}")
    for i in range(args.warmup):
        for call in steps[i % nplan]:
            call()
    torch.cuda.synchronize()

    log(f"timed {args.steps} steps, partition_size {partition}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for call in steps[i % nplan]:
            call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Decode calls alone, back to back, over the same per-step inputs, timed
    # with HIP events on the launch stream.  One call is queued before the
    # first event, so the bracket opens on a busy queue and holds no launch
    # latency of its own; no event sits between the calls (an event between
    # launches adds its own gap on the GPU).
    n_dec = max(args.steps, DECODE_TIMED_CALLS)
    steps[nplan - 1][2]()
    e0.record()
    for i in range(n_dec):
        steps[i % nplan][2]()
    e1.record()
    torch.cuda.synchronize()
    dec_avg_s = e0.elapsed_time(e1) / 1e3 / n_dec
    # and each call on its own between two events (a distribution; each
    # bracket also holds the event's own gap, so it reads a little high)
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(DECODE_PER_CALL)]
    steps[nplan - 1][2]()
    for i in range(DECODE_PER_CALL):
        pev[i][0].record()
        steps[i % nplan][2]()
        pev[i][1].record()
    torch.cuda.synchronize()
    per_call = np.array([a.elapsed_time(b) for a, b in pev]) * 1e3  # us

    step_bytes = sum(sum(totals[i % nplan]) for i in range(args.steps))
    tokens = sum(int(plan.lens[i % nplan].astype(np.int64).sum()) for i in range(args.steps))
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / wall / 1e9
    dec_mean_bytes = float(np.mean([dec_bytes[i % nplan] for i in range(n_dec)]))
    achieved = dec_mean_bytes / dec_avg_s / 1e9
    read_ceiling = None
    if probe_s is not None:
        ceiling = FLUSH_BYTES / probe_s / 1e9
        read_ceiling = {"GBps": round(ceiling, 1), "frac_of_peak": round(ceiling / HBM_PEAK_GBS, 4),
                        "bytes": FLUSH_BYTES, "kernel": "read_probe_kernel",
                        "decode_frac_of_ceiling": round(achieved / ceiling, 4),
                        "note": "plain streaming read (pa_read_probe), mean of 20 back-to-back calls"}

    traffic = measured_traffic(args.workload, partition)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if case.dtype == W.BF16 else "f32",
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled block placement)",
        "config": {
            "workload": args.workload,
            "num_seqs": case.num_seqs, "num_q_heads": case.num_q_heads,
            "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
            "block_size": case.block_size, "pool_blocks": case.num_blocks,
            "context_len_mean": round(float(plan.lens[0].mean()), 1),
            "context_len_max": int(plan.lens[0].max()),
            "partition_size": partition, "seed": case.meta.get("seed"),
            "kv_pool_copies": len(layers), "write_fused_into_decode": fused, "planned_steps": nplan,
        },
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens / wall, 1),
        "seq_steps_per_s": round(case.num_seqs * args.steps / wall, 1),
        "step_bytes": int(step_bytes / args.steps),
        "host_prep_us": round(plan.host_prep_us, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": decode_kernels(case, partition, fused),
            "avg_launch_us": round(dec_avg_s * 1e6, 2),
            "algorithmic_bytes_per_launch": int(dec_mean_bytes),
            "timed_calls": n_dec,
        },
        "decode_per_call_us": {"median": round(float(np.median(per_call)), 2),
                               "p10": round(float(np.percentile(per_call, 10)), 2),
                               "p90": round(float(np.percentile(per_call, 90)), 2),
                               "calls": DECODE_PER_CALL,
                               "note": "each call between its own two HIP events, warm, rotating pools"},
        "cold_cache": cold,
        "indirection": indirection,
        "read_ceiling": read_ceiling,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        result["cpu_baseline"] = cpu_baseline(case, plan, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
