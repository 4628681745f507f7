"""Thin ctypes binding to ``libpa.so`` (include/pa.h).

Argument marshalling only: torch tensors supply device pointers, shapes and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if ``libpa.so`` is missing or cannot be
loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa.so")

PA_F32, PA_BF16 = 0, 1
PA_ALGO_AUTO, PA_ALGO_VECTOR, PA_ALGO_MFMA = 0, 1, 2
PA_PARTITION_AUTO, PA_PARTITION_BALANCED, PA_PARTITION_SHARED = -1, -2, -3
STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_UNSUPPORTED",
          -4: "PA_ERR_WORKSPACE", -5: "PA_ERR_LAUNCH", -6: "PA_ERR_ALGO", -7: "PA_ERR_ALIGN",
          -8: "PA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20   # PA_NOALLOC_SCRATCH_BYTES


class PAError(RuntimeError):
    def __init__(self, status: int, fn: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({status_string(status)})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_261_amd.build` (hipcc, gfx950)")
    lib = C.CDLL(LIB_PATH)
    P, I, F, SZ = C.c_void_p, C.c_int, C.c_float, C.c_size_t
    sig = {
        "pa_reshape_and_cache": (I, [P, P, P, P, P, I, I, I, I, I, I, P]),
        "pa_copy_blocks": (I, [P, P, P, I, I, I, I, I, I, P]),
        "pa_prefill": (I, [P] * 7 + [I] * 9 + [F, I, P]),
        "pa_decode_auto_partition": (I, [I, I, I, I, I, I, I]),
        "pa_decode_workspace_size": (SZ, [I, I, I, I, I, I, I, I]),
        "pa_decode": (I, [P] * 6 + [I] * 8 + [F, I, P, SZ, I, I, P]),
        "pa_decode_partitions": (I, [P] * 6 + [I] * 8 + [F, I, P, SZ, I, I, P]),
        "pa_decode_reduce": (I, [P, P, I, I, I, I, I, I, P, SZ, I, P]),
        "pa_decode_noalloc": (I, [P] * 6 + [I] * 8 + [F, I, I, I, P]),
        "pa_measure_stream_read": (I, [P, SZ, I, P, P]),
        "pa_measure_tile_read": (I, [P, P, P, I, I, P, P]),
        "pa_status_string": (C.c_char_p, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.pa_status_string(int(status)).decode()


def _check(rc: int, fn: str):
    if rc != 0:
        raise PAError(rc, fn)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"paged decode takes float32 or bfloat16 tensors, got {t.dtype}")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def pa_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, stream=None):
    """Write k/v [T, Hkv, d] into their slots of k_cache/v_cache [NB, Hkv, bs, d]."""
    t, hkv, d = k.shape
    nb, hkv2, bs, d2 = k_cache.shape
    if (hkv, d) != (hkv2, d2) or v.shape != k.shape or v_cache.shape != k_cache.shape:
        raise ValueError("k/v and cache shapes disagree")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (t,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    dt = dtype_code(k)
    if any(x.dtype != k.dtype for x in (v, k_cache, v_cache)):
        raise TypeError("k, v and both caches must share one dtype")
    _check(lib.pa_reshape_and_cache(_dev(k, "k"), _dev(v, "v"), _dev(k_cache, "k_cache"),
                                    _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping"),
                                    t, hkv, d, nb, bs, dt, _stream(k, stream)),
           "pa_reshape_and_cache")


def pa_prefill(out, q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens,
               max_context_len, max_q_len, scale, stream=None):
    """Causal prefill of a packed chunk batch q [total_q, Hq, d] over the paged
    cache (the chunk's K/V already written); out has q's shape."""
    tq, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    b = context_lens.shape[0]
    if out.shape != q.shape or d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("q/out/cache shapes disagree")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_q.shape != (b + 1,):
        raise ValueError("cu_seqlens_q must be int32 [num_seqs + 1]")
    if context_lens.dtype != torch.int32 or block_tables.dtype != torch.int32:
        raise ValueError("context_lens and block_tables must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    _check(lib.pa_prefill(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"),
                          _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
                          _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(context_lens, "context_lens"),
                          b, hq, hkv, d, nb, bs, block_tables.shape[1], int(max_context_len),
                          int(max_q_len), float(scale), dtype_code(q), _stream(q, stream)),
           "pa_prefill")


def pa_copy_blocks(k_cache, v_cache, block_pairs, stream=None):
    """Copy whole blocks src -> dst in both pools, for every row (src, dst) of
    block_pairs ([n, 2] int32, on the GPU): the device side of copy-on-write."""
    nb, hkv, bs, d = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must have the same shape and dtype")
    if block_pairs.dtype != torch.int32 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be int32 [num_pairs, 2]")
    n = block_pairs.shape[0]
    if n == 0:
        return
    _check(lib.pa_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                              _dev(block_pairs, "block_pairs"), n, nb, hkv, bs, d,
                              dtype_code(k_cache), _stream(k_cache, stream)),
           "pa_copy_blocks")


def pa_decode_auto_partition(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_context_len, dtype=PA_BF16):
    return lib.pa_decode_auto_partition(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        block_size, max_context_len, dtype)


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_context_len, partition_size=-1, dtype=PA_BF16):
    return lib.pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        block_size, max_context_len, partition_size, dtype)


def workspace_for(q, k_cache, max_context_len, partition_size=-1):
    """Allocate (with torch) the workspace pa_decode needs for these tensors."""
    b, hq, d = q.shape
    _, hkv, bs, _ = k_cache.shape
    n = pa_decode_workspace_size(b, hq, hkv, d, bs, max_context_len, partition_size,
                                 dtype_code(q))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len):
    b, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if out.shape != q.shape or d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("q/out/cache shapes disagree")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (b,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    if any(x.dtype != q.dtype for x in (out, k_cache, v_cache)):
        raise TypeError("q, out and both caches must share one dtype")
    return ([_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
             _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
             b, hq, hkv, d, nb, bs, block_tables.shape[1], int(max_context_len)])


def _ws(workspace):
    if workspace is None:
        return C.c_void_p(0), 0
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
              partition_size=-1, workspace=None, algo=PA_ALGO_AUTO, stream=None):
    """PagedAttention decode: out[b, h] = softmax(scale q k^T) v over the sequence's blocks."""
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len)
    ws, wsb = _ws(workspace)
    _check(lib.pa_decode(*args, float(scale), int(partition_size), ws, wsb, dtype_code(q),
                         int(algo), _stream(q, stream)), "pa_decode")


def pa_decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                         max_context_len, partition_size, workspace, algo=PA_ALGO_AUTO,
                         stream=None):
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len)
    ws, wsb = _ws(workspace)
    _check(lib.pa_decode_partitions(*args, float(scale), int(partition_size), ws, wsb,
                                    dtype_code(q), int(algo), _stream(q, stream)),
           "pa_decode_partitions")


def pa_decode_reduce(out, context_lens, num_kv_heads, max_context_len, partition_size, workspace,
                     stream=None):
    b, hq, d = out.shape
    ws, wsb = _ws(workspace)
    _check(lib.pa_decode_reduce(_dev(out, "out"), _dev(context_lens, "context_lens"), b, hq,
                                int(num_kv_heads), d, int(max_context_len), int(partition_size),
                                ws, wsb, dtype_code(out), _stream(out, stream)),
           "pa_decode_reduce")


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      max_context_len, partition_size=-1, algo=PA_ALGO_AUTO, stream=None):
    """pa_decode without a workspace argument: split modes use the library's
    static per-GPU scratch, so the call allocates nothing."""
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len)
    _check(lib.pa_decode_noalloc(*args, float(scale), int(partition_size), dtype_code(q),
                                 int(algo), _stream(q, stream)), "pa_decode_noalloc")


MEASURE_SINK_WORDS = 4096   # PA_MEASURE_SINK_WORDS (include/pa_measure.h)


def pa_measure_stream_read(buf, sink, nontemporal=True, stream=None):
    """Calibration only: read every byte of the device tensor `buf` once (the
    benchmark's streaming-read ceiling); sink is an int32 device tensor of
    MEASURE_SINK_WORDS words whose XOR equals the XOR of buf's 32-bit words."""
    if sink.dtype != torch.int32 or sink.numel() < MEASURE_SINK_WORDS:
        raise ValueError("sink must be an int32 tensor of MEASURE_SINK_WORDS words")
    _check(lib.pa_measure_stream_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                      1 if nontemporal else 0, _dev(sink, "sink"),
                                      _stream(buf, stream)), "pa_measure_stream_read")


def pa_measure_tile_read(k_cache, v_cache, tiles, sink, stream=None):
    """Calibration only: read the (block, KV head) tiles listed in `tiles`
    (int32, index block * num_kv_heads + head) of both caches the way the
    decode kernels read them, with no arithmetic (the paged-read ceiling)."""
    nb, hkv, bs, d = k_cache.shape
    if tiles.dtype != torch.int32 or tiles.dim() != 1:
        raise ValueError("tiles must be int32 [num_tiles]")
    if sink.dtype != torch.int32 or sink.numel() < MEASURE_SINK_WORDS:
        raise ValueError("sink must be an int32 tensor of MEASURE_SINK_WORDS words")
    _check(lib.pa_measure_tile_read(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                    _dev(tiles, "tiles"), tiles.numel(),
                                    bs * d * k_cache.element_size(), _dev(sink, "sink"),
                                    _stream(k_cache, stream)), "pa_measure_tile_read")
