"""ctypes binding to the C oracle ``liboracle.so`` (TEST INFRASTRUCTURE ONLY).

Argument marshalling only: numpy arrays in, numpy arrays out.  The arithmetic
lives in ``pao.c``; see ``pao.h`` for the pages each function follows.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1
_ERRS = {-1: "out of free blocks", -2: "unknown sequence", -3: "position outside table",
         -4: "bad argument", -5: "slot out of range or repeated", -6: "bad block id",
         -7: "invalid block-table entry"}


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: oracle status {code} ({_ERRS.get(code, '?')})")
        self.code = code


_lib = None


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build
        build.build()
    lib = C.CDLL(LIB_PATH)
    P, I, I64P, I32P = C.c_void_p, C.c_int, C.POINTER(C.c_int64), C.POINTER(C.c_int32)
    sig = {
        "pao_pool_create": (P, [I, I, P]),
        "pao_pool_destroy": (None, [P]),
        "pao_block_alloc": (I, [P]),
        "pao_block_decref": (I, [P, I]),
        "pao_block_ref": (I, [P, I]),
        "pao_seq_new": (I, [P]),
        "pao_seq_alloc_block": (I, [P, I]),
        "pao_seq_slot": (I, [P, I, I, I64P]),
        "pao_seq_fork": (I, [P, I]),
        "pao_seq_append": (I, [P, I, I64P, I32P, I32P]),
        "pao_seq_free": (I, [P, I]),
        "pao_seq_len": (I, [P, I]),
        "pao_seq_num_blocks": (I, [P, I]),
        "pao_seq_table": (I, [P, I, P, I]),
        "pao_pool_stats": (None, [P, P]),
        "pao_slot_write": (I, [P, P, P, P, P, I, I, I, I, I, I]),
        "pao_copy_block": (I, [P, P, I, I, I, I, I, I, I]),
        "pao_decode_concat_f64": (I, [P, P, P, P, P, P] + [I] * 7 + [C.c_double, I, I]),
        "pao_decode_blockwise_f64": (I, [P, P, P, P, P, P] + [I] * 7 + [C.c_double, I, I]),
        "pao_decode_partitioned_f64": (I, [P, P, P, P, P, P] + [I] * 7 + [C.c_double, I, I, I]),
        "pao_prefill_concat_f64": (I, [P] * 7 + [I] * 7 + [C.c_double, I, I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc, what):
    if rc < 0:
        raise OracleError(rc, what)
    return rc


class Pool:
    """Host block pool: LIFO free stack, reference counts, fork, copy-on-write."""

    def __init__(self, num_blocks, block_size, free_order=None):
        self.lib = load_library()
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        fo = None
        if free_order is not None:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            assert fo.shape == (num_blocks,)
        self._fo = fo
        self.h = self.lib.pao_pool_create(self.num_blocks, self.block_size, _ptr(fo))
        if not self.h:
            raise OracleError(-4, "pao_pool_create")

    def __del__(self):
        h = getattr(self, "h", None)
        if h:
            self.lib.pao_pool_destroy(h)
            self.h = None

    # pool-level
    def alloc(self):
        return _check(self.lib.pao_block_alloc(self.h), "alloc")

    def decref(self, block):
        _check(self.lib.pao_block_decref(self.h, int(block)), "decref")

    def ref(self, block):
        return _check(self.lib.pao_block_ref(self.h, int(block)), "ref")

    # sequence-level
    def seq_new(self):
        return _check(self.lib.pao_seq_new(self.h), "seq_new")

    def seq_alloc_block(self, seq):
        return _check(self.lib.pao_seq_alloc_block(self.h, int(seq)), "seq_alloc_block")

    def seq_slot(self, seq, pos):
        out = C.c_int64()
        _check(self.lib.pao_seq_slot(self.h, int(seq), int(pos), C.byref(out)), "seq_slot")
        return out.value

    def fork(self, seq):
        return _check(self.lib.pao_seq_fork(self.h, int(seq)), "fork")

    def append(self, seq):
        """Reserve the next position; returns (slot, cow_src, cow_dst)."""
        slot, src, dst = C.c_int64(), C.c_int32(), C.c_int32()
        _check(self.lib.pao_seq_append(self.h, int(seq), C.byref(slot), C.byref(src),
                                       C.byref(dst)), "append")
        return slot.value, src.value, dst.value

    def free(self, seq):
        _check(self.lib.pao_seq_free(self.h, int(seq)), "free")

    def seq_len(self, seq):
        return _check(self.lib.pao_seq_len(self.h, int(seq)), "seq_len")

    def seq_num_blocks(self, seq):
        return _check(self.lib.pao_seq_num_blocks(self.h, int(seq)), "seq_num_blocks")

    def table(self, seq, max_blocks=None):
        n = self.seq_num_blocks(seq)
        mb = n if max_blocks is None else int(max_blocks)
        row = np.empty(max(mb, 1), dtype=np.int32)
        _check(self.lib.pao_seq_table(self.h, int(seq), _ptr(row), mb), "table")
        return row[:mb]

    def stats(self):
        out = np.zeros(6, dtype=np.int64)
        self.lib.pao_pool_stats(self.h, _ptr(out))
        keys = ("n_blocks", "n_free", "n_used", "peak_used", "n_copies", "n_active")
        return dict(zip(keys, (int(x) for x in out)))


def _elem_bytes(arr):
    return arr.dtype.itemsize


def slot_write(k_cache, v_cache, k, v, slot_mapping, block_size):
    """In-place slot write into numpy pools [NB, Hkv, bs, d] (float32 or uint16 bf16 bits)."""
    lib = load_library()
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k.dtype == k_cache.dtype == v.dtype == v_cache.dtype
    nb, hkv, bs, d = k_cache.shape
    assert bs == block_size
    t = slot_mapping.shape[0]
    assert k.shape == (t, hkv, d) and v.shape == (t, hkv, d)
    _check(lib.pao_slot_write(_ptr(k_cache), _ptr(v_cache), _ptr(k), _ptr(v), _ptr(slot_mapping),
                              t, hkv, d, nb, bs, _elem_bytes(k)), "slot_write")


def copy_block(k_cache, v_cache, src, dst):
    lib = load_library()
    nb, hkv, bs, d = k_cache.shape
    _check(lib.pao_copy_block(_ptr(k_cache), _ptr(v_cache), int(src), int(dst), nb, hkv, d, bs,
                              _elem_bytes(k_cache)), "copy_block")


def _decode(fn_name, q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
            nthreads, extra=()):
    lib = load_library()
    q = np.ascontiguousarray(q)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    b, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    assert d == d2 and v_cache.shape == k_cache.shape
    assert block_tables.shape[0] == b and context_lens.shape == (b,)
    out = np.zeros((b, hq, d), dtype=np.float64)
    rc = getattr(lib, fn_name)(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_tables), _ptr(context_lens), b, hq, hkv, d, nb, bs,
                               block_tables.shape[1], float(scale), int(dtype), *extra,
                               int(nthreads))
    _check(rc, fn_name)
    return out


def prefill_concat(q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens, scale,
                   nthreads=0):
    """Causal prefill of a packed chunk batch (q [total_q, Hq, d]); float64 out."""
    lib = load_library()
    q = np.ascontiguousarray(q)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    tq, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    b = context_lens.shape[0]
    assert d == d2 and v_cache.shape == k_cache.shape
    assert block_tables.shape[0] == b and cu.shape == (b + 1,) and cu[-1] == tq
    out = np.zeros((tq, hq, d), dtype=np.float64)
    rc = lib.pao_prefill_concat_f64(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(block_tables), _ptr(cu), _ptr(context_lens), b, hq, hkv,
                                    d, nb, bs, block_tables.shape[1], float(scale),
                                    int(_dtype_code(q)), int(nthreads))
    _check(rc, "pao_prefill_concat_f64")
    return out


def _dtype_code(arr):
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {arr.dtype}")


def decode_concat(q, k_cache, v_cache, block_tables, context_lens, scale, nthreads=0):
    return _decode("pao_decode_concat_f64", q, k_cache, v_cache, block_tables, context_lens,
                   scale, _dtype_code(q), nthreads)


def decode_blockwise(q, k_cache, v_cache, block_tables, context_lens, scale, nthreads=0):
    return _decode("pao_decode_blockwise_f64", q, k_cache, v_cache, block_tables, context_lens,
                   scale, _dtype_code(q), nthreads)


def decode_partitioned(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                       nthreads=0):
    return _decode("pao_decode_partitioned_f64", q, k_cache, v_cache, block_tables, context_lens,
                   scale, _dtype_code(q), nthreads, extra=(int(partition_size),))
