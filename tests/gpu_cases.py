"""Helpers shared by the GPU tests: host arrays <-> torch device tensors,
tolerance checks, and printing which case is about to run."""

import sys

import numpy as np

import workloads as W

# Tolerances of the decode output against the fp64 oracle.
F32_ABS = 1e-4            # fp32 KV, or bf16 KV with fp32 output: max |gpu - ref|
BF16_ABS, BF16_REL = 2e-2, 1e-2   # bf16 output: |gpu - ref| <= abs + rel * |ref|


def announce(*what):
    print("[gpu case]", *what, flush=True)
    sys.stdout.flush()


def to_dev(arr):
    import torch

    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(arr).cuda()


def to_host(t):
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_to_f64(t):
    from oracle.numerics import bf16_bits_to_f64
    h = to_host(t)
    return bf16_bits_to_f64(h) if h.dtype == np.uint16 else h.astype(np.float64)


class DevCase:
    """A ``workloads.DecodeCase`` uploaded to the GPU."""

    def __init__(self, case):
        self.case = case
        self.q = to_dev(case.q)
        self.k_cache = to_dev(case.k_cache)
        self.v_cache = to_dev(case.v_cache)
        self.block_tables = to_dev(case.block_tables)
        self.context_lens = to_dev(case.context_lens)
        self.k_new = to_dev(case.k_new)
        self.v_new = to_dev(case.v_new)
        self.slot_mapping = to_dev(case.slot_mapping)

    def write(self, pkv):
        pkv.pa_write_kv(self.k_new, self.v_new, self.slot_mapping, self.k_cache, self.v_cache)

    def decode(self, pkv, partition_size=0, out_dtype=None):
        c = self.case
        return pkv.pa_decode(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                             c.max_context, c.scale, partition_size=partition_size, out_dtype=out_dtype)


def oracle_after_write(case):
    """Oracle pools after the case's one-token-per-sequence write."""
    from oracle import kvcache as KV
    return KV.write_kv(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping,
                       case.block_size)


def check_decode(got, ref, bf16_out):
    """Assert the stated tolerance; returns the max abs error."""
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), "non-finite output"
    if bf16_out:
        bound = BF16_ABS + BF16_REL * np.abs(ref)
        bad = err > bound
        assert not bad.any(), f"{bad.sum()} elements outside 2e-2 + 1e-2|ref| (max err {err.max():.3g})"
    else:
        assert err.max() <= F32_ABS, f"max abs err {err.max():.3g} > {F32_ABS}"
    return float(err.max())


def small_bf16_case(seed, num_seqs=6, lo=1, hi=700, extra=(1, 15, 16, 17), **kw):
    rng = np.random.default_rng(seed)
    lens = list(rng.integers(lo, hi, size=num_seqs, endpoint=True)) + list(extra)
    return W.make_case(f"small_bf16_s{seed}", seed=seed + 1, dtype=W.BF16, context_lens=lens,
                       num_q_heads=kw.pop("num_q_heads", 32), num_kv_heads=kw.pop("num_kv_heads", 8),
                       head_dim=kw.pop("head_dim", 128), block_size=kw.pop("block_size", 16), **kw)


def oracle_decode_all(case, k_cache, v_cache, block_tables=None, context_lens=None, q=None, workers=16):
    """The fp64 oracle over every (sequence, query head) of a batch, the
    sequences split over threads (the oracle's NumPy work releases the GIL);
    each thread runs ``oracle.attention.decode`` on its own slice."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import attention as A

    q = case.q if q is None else q
    bt = case.block_tables if block_tables is None else block_tables
    cl = case.context_lens if context_lens is None else context_lens
    b = q.shape[0]
    cuts = np.linspace(0, b, min(workers, max(b, 1)) + 1).astype(int)

    def run(i):
        lo, hi = cuts[i], cuts[i + 1]
        return A.decode(q[lo:hi], k_cache, v_cache, bt[lo:hi], cl[lo:hi], case.scale, case.dtype)

    with ThreadPoolExecutor(len(cuts) - 1) as ex:
        parts = list(ex.map(run, range(len(cuts) - 1)))
    return np.concatenate(parts, axis=0) if parts else np.zeros(q.shape, np.float64)


def check_bf16_is_rounded_f32(got_bf16_dev, got_f32_dev):
    """The bf16 output is the fp32 output rounded to nearest even, element by
    element (the kernels compute in fp32 in the same order for either output
    type and round once at the store)."""
    bits = to_host(got_bf16_dev)
    f32 = to_host(got_f32_dev)
    expect = W.round_to_bf16(f32)
    bad = bits != expect
    assert not bad.any(), f"{int(bad.sum())} bf16 outputs are not the rounded fp32 outputs"
