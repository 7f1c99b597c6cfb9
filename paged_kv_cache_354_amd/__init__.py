"""Python binding of libpagedkv (PagedAttention decode hot path, MI355X).

Argument marshalling only: every step of the path runs in the HIP library
``libpagedkv.so`` built next to this file (``python -m
paged_kv_cache_354_amd.build``).  There is no fallback: if the library is
missing, every call raises.  PyTorch supplies device memory and streams.

The functions carry the C names declared in ``include/pa.h``:

* ``pa_write_kv``     -- new tokens' K/V into their slots
* ``pa_copy_blocks``  -- whole-block copies for copy-on-write
* ``pa_swap_blocks``  -- whole-block copies between a device pool and a pinned
  host swap pool
* ``pa_decode``       -- paged single-query decode attention
* ``pa_decode_write`` -- ``pa_write_kv`` then ``pa_decode`` in one call
* ``pa_decode_write_noalloc`` -- the same without a workspace, for callers
  that cannot allocate (a static scratch array in the library serves)
* ``pa_prefill``      -- causal paged attention of a chunk of new queries
* ``pa_prefill_write`` -- ``pa_write_kv`` of the chunk's keys and values, then
  ``pa_prefill``, in one call
* ``pa_decode_workspace_bytes``
* ``pa_pool_*`` / ``pa_seq_*`` -- host block manager (free pool, reference
  counts, block tables, copy-on-write decisions)

Device arguments are torch tensors on the GPU (contiguous, the documented
dtypes and shapes); they are checked here against the cache descriptor so
that no launch can address memory outside the tensors.  The stream defaults
to torch's current stream.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_ENOMEM, PA_ESTATE, PA_EHIP = range(6)
PA_F32, PA_BF16 = 0, 1
PA_PARTITION_BALANCED = -1  # pa_decode: equal shares of all work per GPU workgroup slot

_STATUS = {1: "EINVAL", 2: "EUNSUPPORTED", 3: "ENOMEM", 4: "ESTATE", 5: "EHIP"}


class PagedKVError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class PoolExhausted(PagedKVError):
    """PA_ENOMEM from the block manager: no free block, state unchanged."""


class PoolStateError(PagedKVError):
    """PA_ESTATE from the block manager."""


class PaCache(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_lib = None

_i32, _i64, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
_P32, _P64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)


class WasteStats(ctypes.Structure):
    """pa_waste_stats: integer totals of one simulated serving run."""

    _fields_ = [(n, ctypes.c_int64) for n in ("steps", "live_slot_steps", "held_slot_steps", "running_steps",
                                              "max_running", "preemptions", "frag_blocked_steps",
                                              "decode_tokens")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}

_SIGS = {
    "pa_version": (ctypes.c_char_p, []),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_write_kv": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, ctypes.POINTER(PaCache), _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, ctypes.POINTER(PaCache), _vp, _i32, _vp]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (_i32, [_vp, _i32, _i32, _vp, _vp, ctypes.POINTER(PaCache), _vp, _i32, _vp, _i32,
                         ctypes.c_float, _i32, _vp, _sz, _vp, _i32, _vp]),
    "pa_decode_write": (_i32, [_vp, _vp, _vp, _i32, _vp, _i32, _i32, _vp, _vp, ctypes.POINTER(PaCache), _vp,
                               _i32, _vp, _i32, ctypes.c_float, _i32, _vp, _sz, _vp, _i32, _vp]),
    "pa_decode_write_noalloc": (_i32, [_vp, _vp, _vp, _i32, _vp, _i32, _i32, _vp, _vp, ctypes.POINTER(PaCache),
                                       _vp, _i32, _vp, _i32, ctypes.c_float, _i32, _vp, _i32, _vp]),
    "pa_prefill": (_i32, [_vp, _i32, _i32, _vp, _i32, _i32, _vp, _vp, ctypes.POINTER(PaCache), _vp, _i32, _vp,
                          _i32, ctypes.c_float, _vp, _i32, _vp]),
    "pa_prefill_write": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _i32, _vp, _vp, ctypes.POINTER(PaCache),
                                _vp, _i32, _vp, _i32, ctypes.c_float, _vp, _i32, _vp]),
    "pa_pool_create": (_i32, [_i32, _i32, _P32, ctypes.POINTER(_vp)]),
    "pa_pool_destroy": (None, [_vp]),
    "pa_pool_num_free": (_i32, [_vp]),
    "pa_pool_refcount": (_i32, [_vp, _i32]),
    "pa_pool_free_list": (_i32, [_vp, _P32, _i32, _P32]),
    "pa_seq_create": (_i32, [_vp, _i64, _i32]),
    "pa_seq_fork": (_i32, [_vp, _i64, _i64]),
    "pa_seq_append": (_i32, [_vp, _i64, _P64, _P64]),
    "pa_seq_append_batch": (_i32, [_vp, _P64, _i32, _P64, _P64, _P32]),
    "pa_seq_cow": (_i32, [_vp, _i64, _i32, _P64]),
    "pa_seq_free": (_i32, [_vp, _i64]),
    "pa_seq_slots": (_i32, [_vp, _i64, _i32, _i32, _P64]),
    "pa_seq_table": (_i32, [_vp, _i64, _P32, _i32, _P32, _P32]),
    "pa_pool_tables": (_i32, [_vp, _P64, _i32, _P32, _i32, _P32]),
    "pa_swap_blocks": (_i32, [_vp, _vp, ctypes.POINTER(PaCache), _vp, _vp, ctypes.POINTER(PaCache), _vp, _i32,
                              _vp]),
    "pa_pool_set_swap_space": (_i32, [_vp, _i32, _P32]),
    "pa_pool_num_free_host": (_i32, [_vp]),
    "pa_pool_host_free_list": (_i32, [_vp, _P32, _i32, _P32]),
    "pa_seq_is_swapped": (_i32, [_vp, _i64]),
    "pa_seq_swap_out": (_i32, [_vp, _i64, _P64, _i32, _P32]),
    "pa_seq_swap_in": (_i32, [_vp, _i64, _P64, _i32, _P32]),
    "pa_pool_enable_prefix_cache": (_i32, [_vp]),
    "pa_pool_num_cached": (_i32, [_vp]),
    "pa_pool_is_cached": (_i32, [_vp, _i32]),
    "pa_pool_lru_list": (_i32, [_vp, _P32, _i32, _P32]),
    "pa_seq_create_cached": (_i32, [_vp, _i64, _P32, _i32, _P32]),
    "pa_seq_create_cached_batch": (_i32, [_vp, _P64, _i32, _P32, _P64, _P32, _P64, _i64, _P32, _P64]),
    "pa_waste_simulate": (_i32, [_i32, _i64, _i32, _P32, _P32, _P32, _i32, ctypes.POINTER(WasteStats)]),
    "pa_read_probe": (_i32, [_vp, _sz, _vp, _vp]),
}

EXPORTED = tuple(_SIGS)


# A host-only build of the block manager and the waste simulator (no device
# code; ``build_sanitized.py`` makes one with AddressSanitizer and
# UndefinedBehaviorSanitizer for the CPU tests).  When this variable names
# one, it is loaded instead of libpagedkv.so and only the host calls are
# bound: every device call then fails with an AttributeError.
HOST_ONLY_ENV = "PAGEDKV_HOST_ONLY_LIB"


def load():
    """Load libpagedkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        host_only = os.environ.get(HOST_ONLY_ENV)
        path = host_only or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run `python -m paged_kv_cache_354_amd.build` "
                               "(there is no non-HIP fallback)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            if host_only and not hasattr(lib, name):
                continue  # a device call: absent from the host-only build
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status, cls=PagedKVError):
    if status != PA_OK:
        msg = load().pa_last_error().decode()
        if status == PA_ENOMEM:
            raise PoolExhausted(status, msg)
        if status == PA_ESTATE:
            raise PoolStateError(status, msg)
        raise cls(status, msg)


def pa_version():
    return load().pa_version().decode()


# --- device calls ----------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported element type {t.dtype} (float32 or bfloat16)")


def _dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def cache_desc(k_cache):
    """Descriptor of a pool tensor ``[num_blocks][num_kv_heads][block_size][head_dim]``."""
    nb, hkv, bs, d = k_cache.shape
    return PaCache(nb, bs, hkv, d, _dtype_code(k_cache))


def _pools(k_cache, v_cache):
    if k_cache.dim() != 4:
        raise ValueError("pools are [num_blocks][num_kv_heads][block_size][head_dim]")
    desc = cache_desc(k_cache)
    kp = _dev(k_cache, "k_cache")
    vp = _dev(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    return desc, kp, vp


def pa_write_kv(k, v, slot_mapping, k_cache, v_cache, stream=None):
    """Store token i's K/V ``[T][Hkv][d]`` at ``slot_mapping[i]`` (int64; < 0 skips)."""
    torch = _torch()
    desc, kp, vp = _pools(k_cache, v_cache)
    t = int(slot_mapping.shape[0])
    shape = (t, desc.num_kv_heads, desc.head_dim)
    _check(load().pa_write_kv(_dev(k, "k", k_cache.dtype, shape), _dev(v, "v", k_cache.dtype, shape),
                              _dev(slot_mapping, "slot_mapping", torch.int64, (t,)), t, kp, vp,
                              ctypes.byref(desc), _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, src_dst_pairs, stream=None):
    """Copy block ``src`` to ``dst`` in both pools for each int64 (src, dst) row."""
    torch = _torch()
    desc, kp, vp = _pools(k_cache, v_cache)
    n = int(src_dst_pairs.shape[0])
    if n == 0:
        return
    _check(load().pa_copy_blocks(kp, vp, ctypes.byref(desc),
                                 _dev(src_dst_pairs, "src_dst_pairs", torch.int64, (n, 2)), n,
                                 _stream(stream)))


PA_READ_PROBE_WORKGROUPS = 8192


def pa_read_probe(buf, sink=None, stream=None):
    """Stream the contiguous device tensor ``buf`` once (a measurement helper:
    the practical read ceiling); returns the uint32 ``sink`` of
    ``PA_READ_PROBE_WORKGROUPS`` words whose XOR is the XOR of every 32-bit
    word of ``buf``."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(PA_READ_PROBE_WORKGROUPS, dtype=torch.int32, device=buf.device)
    if (not sink.is_cuda or sink.dtype not in (torch.int32, torch.uint32) or not sink.is_contiguous()
            or sink.numel() < PA_READ_PROBE_WORKGROUPS):
        raise ValueError(f"sink must be a contiguous int32 GPU tensor of >= {PA_READ_PROBE_WORKGROUPS} words")
    _check(load().pa_read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                _stream(stream)))
    return sink


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, src_dst_pairs, stream=None):
    """Copy block ``src`` of the source pools to ``dst`` of the destination
    pools for each int64 (src, dst) row; either side may be a pinned host
    tensor (``pin_memory``) or a device tensor; ``src_dst_pairs`` must be
    device-addressable (a device tensor, or pinned host memory)."""
    torch = _torch()
    sd, dd = cache_desc(src_k), cache_desc(dst_k)
    n = int(src_dst_pairs.shape[0])
    if n == 0:
        return

    def ptr(t, name, like):
        if not isinstance(t, torch.Tensor) or not (t.is_cuda or t.is_pinned()):
            raise TypeError(f"{name} must be a GPU tensor or a pinned host tensor")
        if not t.is_contiguous() or t.dtype != like.dtype or tuple(t.shape) != tuple(like.shape):
            raise ValueError(f"{name} must be contiguous, of the same dtype and shape as its pair")
        return ctypes.c_void_p(t.data_ptr())

    pairs = src_dst_pairs
    if pairs.dtype != torch.int64 or tuple(pairs.shape) != (n, 2) or not pairs.is_contiguous() or \
            not (pairs.is_cuda or pairs.is_pinned()):
        raise ValueError("src_dst_pairs must be a contiguous int64 [n][2] GPU or pinned tensor")
    _check(load().pa_swap_blocks(ptr(src_k, "src_k", src_k), ptr(src_v, "src_v", src_k), ctypes.byref(sd),
                                 ptr(dst_k, "dst_k", dst_k), ptr(dst_v, "dst_v", dst_k), ctypes.byref(dd),
                                 ctypes.c_void_p(pairs.data_ptr()), n, _stream(stream)))


def pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                              partition_size):
    return int(load().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                max_context_len, partition_size))


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                 partition_size, workspace, out, out_dtype, stream, allocate):
    """Marshalled ``pa_decode`` arguments (which follow the new-token ones in
    ``pa_decode_write``), allocating ``out`` and the workspace when
    ``allocate`` and they are not given."""
    torch = _torch()
    desc, kp, vp = _pools(k_cache, v_cache)
    b, hq, d = q.shape
    if d != desc.head_dim:
        raise ValueError("q head_dim does not match the pools")
    qp = _dev(q, "q", k_cache.dtype)
    mb = int(block_tables.shape[1]) if block_tables.dim() == 2 else -1
    tp = _dev(block_tables, "block_tables", torch.int32, (b, mb))
    lp = _dev(context_lens, "context_lens", torch.int32, (b,))
    if out_dtype is None:
        out_dtype = q.dtype if out is None else out.dtype
    if out is None:
        if not allocate:
            raise ValueError("out must be given")
        out = torch.empty((b, hq, d), dtype=out_dtype, device=q.device)
    op = _dev(out, "out", out_dtype, (b, hq, d))
    ws_need = pa_decode_workspace_bytes(b, hq, desc.num_kv_heads, d, int(max_context_len),
                                        int(partition_size))
    if partition_size and workspace is None and allocate:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=q.device)
    if workspace is not None:
        wp = _dev(workspace, "workspace")
        wbytes = workspace.numel() * workspace.element_size()
    else:
        wp, wbytes = ctypes.c_void_p(0), 0
    if wbytes < ws_need:
        raise ValueError(f"workspace of {wbytes} bytes < {ws_need} needed")
    args = (qp, b, hq, kp, vp, ctypes.byref(desc), tp, mb, lp, int(max_context_len), float(scale),
            int(partition_size), wp, wbytes, op, _dtype_code(out), _stream(stream))
    return args, out, (desc, q, k_cache, v_cache, block_tables, context_lens, workspace, out)


def _new_token_args(k, v, slot_mapping, k_cache):
    torch = _torch()
    desc = cache_desc(k_cache)
    t = int(slot_mapping.shape[0])
    shape = (t, desc.num_kv_heads, desc.head_dim)
    return (_dev(k, "k", k_cache.dtype, shape), _dev(v, "v", k_cache.dtype, shape),
            _dev(slot_mapping, "slot_mapping", torch.int64, (t,)), t)


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
              partition_size=0, workspace=None, out=None, out_dtype=None, stream=None):
    """Paged decode attention; returns ``out [B][Hq][d]``.

    ``q [B][Hq][d]`` in the cache dtype; ``block_tables int32 [B][MB]``;
    ``context_lens int32 [B]``; ``max_context_len`` a host int bounding every
    length; ``partition_size`` 0, a multiple of the block size or
    ``PA_PARTITION_BALANCED`` (the last two need a uint8 ``workspace`` of
    ``pa_decode_workspace_bytes`` bytes; one is allocated here if not given).
    """
    args, out, _ = _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                                partition_size, workspace, out, out_dtype, stream, True)
    _check(load().pa_decode(*args))
    return out


def pa_decode_write(k, v, slot_mapping, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                    scale, partition_size=0, workspace=None, out=None, out_dtype=None, stream=None):
    """``pa_write_kv(k, v, slot_mapping)`` then ``pa_decode`` as one call (one
    kernel on the balanced path when token i is sequence i's newest); the
    arguments of the two, returns ``out``."""
    args, out, _ = _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                                partition_size, workspace, out, out_dtype, stream, True)
    _check(load().pa_decode_write(*_new_token_args(k, v, slot_mapping, k_cache), *args))
    return out


# Bytes of the library's static scratch array (PA_NOALLOC_SCRATCH_BYTES).
PA_NOALLOC_SCRATCH_BYTES = 64 << 20


def pa_decode_write_noalloc(k, v, slot_mapping, q, k_cache, v_cache, block_tables, context_lens,
                            max_context_len, scale, out, partition_size=0, out_dtype=None, stream=None):
    """``pa_decode_write`` for callers that cannot allocate: no workspace (the
    library's static scratch array serves), and ``out`` must be given.
    Calls that overlap on one GPU share that scratch and must be serialised."""
    args, out, _ = _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale, 0,
                                None, out, out_dtype, stream, False)
    args = args[:11] + (int(partition_size),) + args[14:]  # no workspace, no workspace size
    _check(load().pa_decode_write_noalloc(*_new_token_args(k, v, slot_mapping, k_cache), *args))
    return out


def _prefill_args(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens, max_query_len,
                  max_context_len, scale, out, out_dtype, stream):
    torch = _torch()
    desc, kp, vp = _pools(k_cache, v_cache)
    t, hq, d = q.shape
    if d != desc.head_dim:
        raise ValueError("q head_dim does not match the pools")
    b = int(context_lens.shape[0])
    mb = int(block_tables.shape[1]) if block_tables.dim() == 2 else -1
    if out_dtype is None:
        out_dtype = q.dtype if out is None else out.dtype
    if out is None:
        out = torch.empty((t, hq, d), dtype=out_dtype, device=q.device)
    args = (_dev(q, "q", k_cache.dtype), t, hq, _dev(cu_seqlens, "cu_seqlens", torch.int32, (b + 1,)), b,
            int(max_query_len), kp, vp, ctypes.byref(desc),
            _dev(block_tables, "block_tables", torch.int32, (b, mb)), mb,
            _dev(context_lens, "context_lens", torch.int32, (b,)), int(max_context_len), float(scale),
            _dev(out, "out", out_dtype, (t, hq, d)), _dtype_code(out), _stream(stream))
    return args, out, (desc, q, k_cache, v_cache, block_tables, context_lens, cu_seqlens, out)


def pa_prefill(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens, max_query_len, max_context_len,
               scale, out=None, out_dtype=None, stream=None):
    """Causal paged attention of packed queries ``q [T][Hq][d]`` (sequence s
    owns rows ``cu_seqlens[s] .. cu_seqlens[s+1]-1``, its last positions);
    returns ``out [T][Hq][d]``."""
    args, out, _ = _prefill_args(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens, max_query_len,
                                 max_context_len, scale, out, out_dtype, stream)
    _check(load().pa_prefill(*args))
    return out


def prepare_prefill(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens, max_query_len,
                    max_context_len, scale, out, stream=None):
    """``pa_prefill`` with its arguments checked once; ``out`` must be given."""
    args, _, keep = _prefill_args(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens, max_query_len,
                                  max_context_len, scale, out, None, stream)
    fn = load().pa_prefill

    def call():
        _check(fn(*args))
    call.keep = keep
    return call


def _prefill_write_args(k, v, slot_mapping, q, k_cache, v_cache, block_tables, context_lens, cu_seqlens,
                        max_query_len, max_context_len, scale, out, out_dtype, stream):
    args, out, keep = _prefill_args(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens, max_query_len,
                                    max_context_len, scale, out, out_dtype, stream)
    nt = _new_token_args(k, v, slot_mapping, k_cache)
    if nt[3] != args[1]:
        raise ValueError("k, v and slot_mapping must have one row per query row")
    return nt[:3] + args, out, keep + (k, v, slot_mapping)


def pa_prefill_write(k, v, slot_mapping, q, k_cache, v_cache, block_tables, context_lens, cu_seqlens,
                     max_query_len, max_context_len, scale, out=None, out_dtype=None, stream=None):
    """``pa_write_kv(k, v, slot_mapping)`` then ``pa_prefill`` as one call
    (one kernel for head_dim 128 and block sizes of 8 and up): row r of
    ``k``/``v`` ``[T][Hkv][d]`` is the key and value of query row r, stored at
    ``slot_mapping[r]``; returns ``out``."""
    args, out, _ = _prefill_write_args(k, v, slot_mapping, q, k_cache, v_cache, block_tables, context_lens,
                                       cu_seqlens, max_query_len, max_context_len, scale, out, out_dtype, stream)
    _check(load().pa_prefill_write(*args))
    return out


def prepare_prefill_write(k, v, slot_mapping, q, k_cache, v_cache, block_tables, context_lens, cu_seqlens,
                          max_query_len, max_context_len, scale, out, stream=None):
    """``pa_prefill_write`` with its arguments checked once; ``out`` must be
    given."""
    args, _, keep = _prefill_write_args(k, v, slot_mapping, q, k_cache, v_cache, block_tables, context_lens,
                                        cu_seqlens, max_query_len, max_context_len, scale, out, None, stream)
    fn = load().pa_prefill_write

    def call():
        _check(fn(*args))
    call.keep = keep
    return call


# --- host block manager ------------------------------------------------------------

def _np_ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def pa_pool_create(num_blocks, block_size, free_order=None):
    handle = ctypes.c_void_p()
    order = None
    if free_order is not None:
        arr = np.ascontiguousarray(free_order, dtype=np.int32)
        if arr.shape != (num_blocks,):
            raise ValueError("free_order must have num_blocks entries")
        order = _np_ptr(arr, ctypes.c_int32)
    _check(load().pa_pool_create(num_blocks, block_size, order, ctypes.byref(handle)))
    return handle


def pa_pool_destroy(pool):
    load().pa_pool_destroy(pool)


def pa_pool_num_free(pool):
    return int(load().pa_pool_num_free(pool))


def pa_pool_refcount(pool, block):
    return int(load().pa_pool_refcount(pool, block))


def pa_pool_free_list(pool):
    n = pa_pool_num_free(pool)
    out = np.empty(max(n, 1), dtype=np.int32)
    got = ctypes.c_int32()
    _check(load().pa_pool_free_list(pool, _np_ptr(out, ctypes.c_int32), n, ctypes.byref(got)))
    return out[:got.value]


def pa_pool_set_swap_space(pool, num_host_blocks, host_free_order=None):
    order = None
    if host_free_order is not None:
        order = np.ascontiguousarray(host_free_order, dtype=np.int32)
        if order.shape != (num_host_blocks,):
            raise ValueError("host_free_order must have num_host_blocks entries")
    _check(load().pa_pool_set_swap_space(pool, num_host_blocks,
                                         _np_ptr(order, ctypes.c_int32) if order is not None else None))


def pa_pool_num_free_host(pool):
    return int(load().pa_pool_num_free_host(pool))


def pa_pool_host_free_list(pool):
    n = pa_pool_num_free_host(pool)
    out = np.empty(max(n, 1), dtype=np.int32)
    got = ctypes.c_int32()
    _check(load().pa_pool_host_free_list(pool, _np_ptr(out, ctypes.c_int32), n, ctypes.byref(got)))
    return out[:got.value]


def pa_seq_is_swapped(pool, seq):
    r = int(load().pa_seq_is_swapped(pool, seq))
    if r < 0:
        raise PoolStateError(PA_ESTATE, f"unknown sequence {seq}")
    return bool(r)


def _swap(fn, pool, seq):
    nb = ctypes.c_int32()
    lib = load()
    st = lib.pa_seq_table(pool, seq, None, 0, ctypes.byref(nb), ctypes.byref(ctypes.c_int32()))
    if st not in (PA_OK, PA_EINVAL):
        _check(st)
    pairs = np.empty((max(nb.value, 1), 2), dtype=np.int64)
    got = ctypes.c_int32()
    _check(getattr(lib, fn)(pool, seq, _np_ptr(pairs, ctypes.c_int64), nb.value, ctypes.byref(got)))
    return pairs[:got.value]


def pa_seq_swap_out(pool, seq):
    """Swap ``seq`` out; returns int64 [n][2] (device block, host block) copies to do."""
    return _swap("pa_seq_swap_out", pool, seq)


def pa_seq_swap_in(pool, seq):
    """Swap ``seq`` in; returns int64 [n][2] (host block, device block) copies to do."""
    return _swap("pa_seq_swap_in", pool, seq)


def pa_pool_enable_prefix_cache(pool):
    _check(load().pa_pool_enable_prefix_cache(pool))


def pa_pool_num_cached(pool):
    return int(load().pa_pool_num_cached(pool))


def pa_pool_is_cached(pool, block):
    r = int(load().pa_pool_is_cached(pool, block))
    if r < 0:
        raise PagedKVError(PA_EINVAL, f"block {block} outside the pool")
    return bool(r)


def pa_pool_lru_list(pool):
    n = pa_pool_num_cached(pool)
    out = np.empty(max(n, 1), dtype=np.int32)
    got = ctypes.c_int32()
    _check(load().pa_pool_lru_list(pool, _np_ptr(out, ctypes.c_int32), n, ctypes.byref(got)))
    return out[:got.value]


def pa_seq_create_cached(pool, seq, tokens):
    """Create ``seq`` from its prompt ``tokens``; returns how many leading
    tokens were found in the prefix cache."""
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    got = ctypes.c_int32()
    ptr = _np_ptr(t, ctypes.c_int32) if t.size else None
    _check(load().pa_seq_create_cached(pool, seq, ptr, int(t.size), ctypes.byref(got)))
    return got.value


PA_WASTE_CONTIGUOUS, PA_WASTE_PAGED = 0, 1


def pa_waste_simulate(mode, capacity, block_size, prompt_lens, output_lens, reserve_lens):
    """Serving loop over one pool of ``capacity`` KV slots; ``mode`` is
    "contiguous" or "paged".  Returns the totals as a dict."""
    m = {"contiguous": PA_WASTE_CONTIGUOUS, "paged": PA_WASTE_PAGED}[mode]
    arrs = [np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))
            for a in (prompt_lens, output_lens, reserve_lens)]
    n = arrs[0].size
    if any(a.size != n for a in arrs):
        raise PagedKVError(PA_EINVAL, "prompt, output and reserve lengths differ in count")
    ptrs = [_np_ptr(a, ctypes.c_int32) if n else None for a in arrs]
    st = WasteStats()
    _check(load().pa_waste_simulate(m, int(capacity), int(block_size), *ptrs, n, ctypes.byref(st)))
    return st.as_dict()


def pa_seq_create_cached_batch(pool, seqs, prompts):
    """Admit ``prompts`` (sequences of token ids) as ``seqs`` in order until
    one is refused.  Returns ``(num_cached, slots, refused)``: the cached
    token count of each admitted request (int32 [k]), the slots of their
    uncached tokens in order (int64), and None or the PoolExhausted /
    PoolStateError that refused request k."""
    seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64).reshape(-1))
    n = seqs.size
    if len(prompts) != n:
        raise PagedKVError(PA_EINVAL, "one prompt per sequence")
    lens = np.array([len(p) for p in prompts], dtype=np.int64)
    offsets = np.ascontiguousarray(np.concatenate([[0], np.cumsum(lens)]).astype(np.int64))
    tokens = np.ascontiguousarray(np.concatenate([np.asarray(p, np.int32).reshape(-1) for p in prompts])
                                  if n else np.zeros(0, np.int32))
    cached = np.zeros(max(n, 1), dtype=np.int32)
    slots = np.empty(max(int(offsets[-1]), 1), dtype=np.int64)
    na, ns = ctypes.c_int32(), ctypes.c_int64()
    st = load().pa_seq_create_cached_batch(
        pool, _np_ptr(seqs, ctypes.c_int64) if n else None, n,
        _np_ptr(tokens, ctypes.c_int32) if tokens.size else None, _np_ptr(offsets, ctypes.c_int64),
        _np_ptr(cached, ctypes.c_int32), _np_ptr(slots, ctypes.c_int64), int(offsets[-1]), ctypes.byref(na),
        ctypes.byref(ns))
    refused = None
    if st != PA_OK:
        try:
            _check(st)
        except (PoolExhausted, PoolStateError) as e:
            if st == PA_ESTATE or st == PA_ENOMEM:
                refused = e
            else:
                raise
    return cached[:na.value].copy(), slots[:ns.value].copy(), refused


def pa_seq_create(pool, seq, num_tokens):
    _check(load().pa_seq_create(pool, seq, num_tokens))


def pa_seq_fork(pool, parent, child):
    _check(load().pa_seq_fork(pool, parent, child))


def pa_seq_append(pool, seq):
    """Returns ``(slot, pair)``; ``pair`` is (src, dst) or None."""
    slot = ctypes.c_int64()
    pair = (ctypes.c_int64 * 2)()
    _check(load().pa_seq_append(pool, seq, ctypes.byref(slot), pair))
    return slot.value, (None if pair[0] < 0 else (pair[0], pair[1]))


def pa_seq_append_batch(pool, seqs):
    """Returns ``(slots int64 [n], pairs int64 [k][2])``; all or nothing."""
    s = np.ascontiguousarray(seqs, dtype=np.int64)
    n = s.shape[0]
    slots = np.empty(max(n, 1), dtype=np.int64)
    pairs = np.empty((max(n, 1), 2), dtype=np.int64)
    k = ctypes.c_int32()
    _check(load().pa_seq_append_batch(pool, _np_ptr(s, ctypes.c_int64), n,
                                      _np_ptr(slots, ctypes.c_int64), _np_ptr(pairs, ctypes.c_int64),
                                      ctypes.byref(k)))
    return slots[:n], pairs[:k.value]


def pa_seq_cow(pool, seq, logical_block):
    pair = (ctypes.c_int64 * 2)()
    _check(load().pa_seq_cow(pool, seq, logical_block, pair))
    return None if pair[0] < 0 else (pair[0], pair[1])


def pa_seq_free(pool, seq):
    _check(load().pa_seq_free(pool, seq))


def pa_seq_slots(pool, seq, start, count):
    out = np.empty(max(count, 1), dtype=np.int64)
    _check(load().pa_seq_slots(pool, seq, start, count, _np_ptr(out, ctypes.c_int64)))
    return out[:count]


def pa_seq_table(pool, seq, max_blocks=None):
    """Returns ``(row int32 [nb], length)``."""
    lib = load()
    nb, ln = ctypes.c_int32(), ctypes.c_int32()
    if max_blocks is None:
        # a zero-capacity call reports the block count (EINVAL if it is > 0)
        st = lib.pa_seq_table(pool, seq, None, 0, ctypes.byref(nb), ctypes.byref(ln))
        if st not in (PA_OK, PA_EINVAL):
            _check(st)
        max_blocks = nb.value
    row = np.empty(max(max_blocks, 1), dtype=np.int32)
    _check(lib.pa_seq_table(pool, seq, _np_ptr(row, ctypes.c_int32), max_blocks, ctypes.byref(nb),
                            ctypes.byref(ln)))
    return row[:nb.value].copy(), ln.value


def pa_pool_tables(pool, seqs, max_blocks, tables=None, context_lens=None):
    """Fill ``tables int32 [n][max_blocks]`` (-1 padded) and ``context_lens int32 [n]``."""
    s = np.ascontiguousarray(seqs, dtype=np.int64)
    n = s.shape[0]
    if tables is None:
        tables = np.empty((n, max_blocks), dtype=np.int32)
    if context_lens is None:
        context_lens = np.empty(n, dtype=np.int32)
    if tables.shape != (n, max_blocks) or tables.dtype != np.int32 or not tables.flags.c_contiguous:
        raise ValueError("tables must be C-contiguous int32 [n][max_blocks]")
    if context_lens.shape != (n,) or context_lens.dtype != np.int32:
        raise ValueError("context_lens must be int32 [n]")
    _check(load().pa_pool_tables(pool, _np_ptr(s, ctypes.c_int64), n, _np_ptr(tables, ctypes.c_int32),
                                 max_blocks, _np_ptr(context_lens, ctypes.c_int32)))
    return tables, context_lens


class BlockPool:
    """Owning wrapper of a ``pa_pool`` handle with the C calls as methods."""

    def __init__(self, num_blocks, block_size, free_order=None):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.handle = pa_pool_create(num_blocks, block_size, free_order)

    def close(self):
        if self.handle:
            pa_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def create(self, seq, n):
        pa_seq_create(self.handle, seq, n)

    def fork(self, parent, child):
        pa_seq_fork(self.handle, parent, child)

    def append(self, seq):
        return pa_seq_append(self.handle, seq)

    def append_batch(self, seqs):
        return pa_seq_append_batch(self.handle, seqs)

    def cow(self, seq, logical_block):
        return pa_seq_cow(self.handle, seq, logical_block)

    def release(self, seq):
        pa_seq_free(self.handle, seq)

    def slots(self, seq, start, count):
        return pa_seq_slots(self.handle, seq, start, count)

    def table(self, seq):
        return pa_seq_table(self.handle, seq)[0]

    def length(self, seq):
        return pa_seq_table(self.handle, seq)[1]

    def refcount(self, block):
        return pa_pool_refcount(self.handle, block)

    def num_free(self):
        return pa_pool_num_free(self.handle)

    def free_order(self):
        return pa_pool_free_list(self.handle)

    def tables(self, seqs, max_blocks, tables=None, context_lens=None):
        return pa_pool_tables(self.handle, seqs, max_blocks, tables, context_lens)

    def set_swap_space(self, num_host_blocks, host_free_order=None):
        pa_pool_set_swap_space(self.handle, num_host_blocks, host_free_order)

    def swap_out(self, seq):
        return pa_seq_swap_out(self.handle, seq)

    def swap_in(self, seq):
        return pa_seq_swap_in(self.handle, seq)

    def is_swapped(self, seq):
        return pa_seq_is_swapped(self.handle, seq)

    def num_free_host(self):
        return pa_pool_num_free_host(self.handle)

    def host_free_order(self):
        return pa_pool_host_free_list(self.handle)

    def enable_prefix_cache(self):
        pa_pool_enable_prefix_cache(self.handle)

    def create_cached(self, seq, tokens):
        return pa_seq_create_cached(self.handle, seq, tokens)

    def create_cached_batch(self, seqs, prompts):
        return pa_seq_create_cached_batch(self.handle, seqs, prompts)

    def num_cached(self):
        return pa_pool_num_cached(self.handle)

    def is_cached(self, block):
        return pa_pool_is_cached(self.handle, block)

    def lru_order(self):
        return pa_pool_lru_list(self.handle)


# --- prepared calls ----------------------------------------------------------------
#
# A decode loop issues the same calls with the same buffers every step.  These
# helpers check and marshal the arguments once and return a zero-argument
# callable that only calls the C entry point (a few microseconds of host time),
# so host overhead cannot hide the kernels' time.  The tensors must stay alive
# and keep their shapes while the callable is used.

def prepare_write_kv(k, v, slot_mapping, k_cache, v_cache, stream=None):
    torch = _torch()
    desc, kp, vp = _pools(k_cache, v_cache)
    t = int(slot_mapping.shape[0])
    shape = (t, desc.num_kv_heads, desc.head_dim)
    args = (_dev(k, "k", k_cache.dtype, shape), _dev(v, "v", k_cache.dtype, shape),
            _dev(slot_mapping, "slot_mapping", torch.int64, (t,)), t, kp, vp, ctypes.byref(desc),
            _stream(stream))
    fn = load().pa_write_kv

    def call():
        _check(fn(*args))
    call.keep = (desc, k, v, slot_mapping, k_cache, v_cache)
    return call


def prepare_copy_blocks(k_cache, v_cache, src_dst_pairs, stream=None):
    torch = _torch()
    desc, kp, vp = _pools(k_cache, v_cache)
    n = int(src_dst_pairs.shape[0])
    if n == 0:
        return lambda: None
    args = (kp, vp, ctypes.byref(desc), _dev(src_dst_pairs, "src_dst_pairs", torch.int64, (n, 2)), n,
            _stream(stream))
    fn = load().pa_copy_blocks

    def call():
        _check(fn(*args))
    call.keep = (desc, k_cache, v_cache, src_dst_pairs)
    return call


def prepare_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale, out,
                   partition_size=0, workspace=None, stream=None):
    """``pa_decode`` with its arguments checked once; ``out`` and (when
    partitioned) ``workspace`` must be given."""
    args, _, keep = _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                                 partition_size, workspace, out, None, stream, False)
    fn = load().pa_decode

    def call():
        _check(fn(*args))
    call.keep = keep
    return call


def prepare_decode_write(k, v, slot_mapping, q, k_cache, v_cache, block_tables, context_lens,
                         max_context_len, scale, out, partition_size=0, workspace=None, stream=None):
    """``pa_decode_write`` with its arguments checked once."""
    args, _, keep = _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                                 partition_size, workspace, out, None, stream, False)
    wargs = _new_token_args(k, v, slot_mapping, k_cache)
    fn = load().pa_decode_write

    def call():
        _check(fn(*wargs, *args))
    call.keep = keep + (k, v, slot_mapping)
    return call
