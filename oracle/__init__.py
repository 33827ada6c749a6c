"""Plain CPU oracle for split-KV attention decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The GPU library never does, and this package never imports the GPU
library: the two share no code.  The arithmetic lives in ``oracle.c`` (plain C, binary64,
pthreads over output rows); this module only marshals numpy arrays into it.

Sources (cited by page title and section):

* planner -- Modular MAX API page "hip_mha_decoding_num_partitions" (regime bullets, the
  EXCEPTION paragraph, "Phase 0 sweep", "AMD reducer constraint", "Tunables");
* tile rule -- AITER issue "[Perf] pa_decode_sparse: BLOCK_K=64 is suboptimal above the CU
  count" ("Why it is not monotonic in num_queries");
* attention -- moonmath-amd README ("MLA decode" usage and constraints; gfx950 "forward_paged");
  "Numerics" fixes the target as attention over the same dequantized KV;
* merge -- base-2 log-sum-exp combination of partials (mla_splitk_reduce, mla_dcp_lse_merge_ranks);
* proportional plan -- moonmath-amd README ("VarlenPlan": a plan made on the GPU from device-side
  lengths); the length-proportional rule is a reading of that section, written here in plain
  integer Python (the one function whose arithmetic is not in ``oracle.c``).

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against page values,
closed forms, invariants and torch-CPU library routines; none is "parity unpinned" except the
planner's MHA high-occupancy branch, whose formula the page does not print (see the planner
docstring).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_dbl = ctypes.c_double
_vp = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with the host C compiler (gcc, -O2, no fast-math)."""
    src = os.path.join(_HERE, "oracle.c")
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= max(
        os.path.getmtime(src), os.path.getmtime(os.path.join(_HERE, "oracle.h"))
    ):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_e4m3_value.restype = _dbl
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint32, _int]
        lib.oracle_bf16_value.restype = _dbl
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint32]
        lib.oracle_plan_splits.restype = _i64
        lib.oracle_plan_splits.argtypes = [_i64, _i64, _i64, _i64, _int]
        lib.oracle_block_k.restype = _int
        lib.oracle_block_k.argtypes = [_i64, _i64]
        lib.oracle_plan_sparse_splits.restype = _int
        lib.oracle_plan_sparse_splits.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp]
        lib.oracle_mla_decode.restype = _int
        lib.oracle_mla_decode.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64,
                                          _vp, _vp, _vp, _dbl, _dbl, _int, _vp, _i64, _vp, _vp,
                                          _int]
        lib.oracle_mla_decode_two_caches.restype = _int
        lib.oracle_mla_decode_bf16.restype = _int
        lib.oracle_mla_decode_bf16.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64,
                                               _vp, _vp, _vp, ctypes.c_double, ctypes.c_double, _vp,
                                               _i64, _vp, _vp, _int]
        lib.oracle_mla_decode_two_caches.argtypes = [_i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                                     _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                                                     _dbl, _dbl, _vp, _i64, _vp, _vp, _int]
        lib.oracle_mla_decode_two_caches_bf16.restype = _int
        lib.oracle_mla_decode_two_caches_bf16.argtypes = lib.oracle_mla_decode_two_caches.argtypes
        lib.oracle_gqa_decode.restype = _int
        lib.oracle_gqa_decode.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64,
                                          _vp, _vp, _vp, _dbl, _vp, _i64, _vp, _vp, _int]
        lib.oracle_lse_merge.restype = _int
        lib.oracle_lse_merge.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp, _vp]
        lib.oracle_default_threads.restype = _int
        lib.oracle_default_threads.argtypes = []
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    """Contiguous numpy view of ``a`` with ``dtype`` (reinterpreting bits of equal width)."""
    a = np.asarray(a)
    if a.dtype != np.dtype(dtype):
        if a.dtype.itemsize == np.dtype(dtype).itemsize and a.dtype.kind in "iu" and np.dtype(dtype).kind in "iu":
            a = a.view(dtype)
        else:
            a = a.astype(dtype)
    return np.ascontiguousarray(a)


def e4m3_value(byte: int, fnuz: bool = False) -> float:
    return _load().oracle_e4m3_value(int(byte) & 0xFF, int(bool(fnuz)))


def e4m3_table(fnuz: bool = False) -> np.ndarray:
    """All 256 fp8 E4M3 values, decoded from the format's definition."""
    return np.array([e4m3_value(b, fnuz) for b in range(256)], dtype=np.float64)


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits) & 0xFFFF)


def plan_splits(batch_size: int, num_keys: int, heads_per_group: int, sm_count: int,
                is_mla: bool = False) -> int:
    """Planner of the "hip_mha_decoding_num_partitions" page; -1 on invalid input.

    The MHA-style high-occupancy target (work_floor) is a reading, not a printed formula:
    parity unpinned against the page for that branch (only its caps are pinned)."""
    return int(_load().oracle_plan_splits(batch_size, num_keys, heads_per_group, sm_count,
                                          int(bool(is_mla))))


def plan_sparse_splits(num_tokens: int, num_heads: int, topk: int, extra_topk: int = 0, *,
                       num_sms: int, max_splits: int = 16, head_tiles: int = 1):
    """(num_splits, chunks_per_block) of the sparse top-k planner on the FlashInfer API page
    "cake_sparse_mla_sm120_dsv4_nvfp4_plan_splits", or None where the C oracle returns -1."""
    ns = ctypes.c_int64(0)
    cpb = ctypes.c_int64(0)
    rc = _load().oracle_plan_sparse_splits(num_tokens, num_heads, topk, extra_topk, num_sms,
                                           max_splits, head_tiles, ctypes.byref(ns), ctypes.byref(cpb))
    return None if rc != 0 else (int(ns.value), int(cpb.value))


def proportional_plan(lengths, budget: int, cap: int, block_k: int):
    """Length-proportional partitions for a batch with lengths[b] keys per request.

    Under a common partition length c a request takes as many partitions of c keys as cover its
    keys, except that no request takes more than `cap`: one that would gets the fewest
    partitions of the smallest block_k multiple that covers it in cap.  c is the smallest
    multiple of block_k for which the partitions of the whole batch number at most `budget`
    (the longest request rounded up to block_k when no c does).  Returns (part_start,
    part_chunk): the exclusive prefix sum of the counts ([batch + 1]) and each request's
    partition length ([batch])."""
    lengths = [max(0, int(x)) for x in lengths]

    def split(n, c):
        k = -(-n // c)
        if k > cap:
            c = -(-(-(-n // cap)) // block_k) * block_k
            k = -(-n // c)
        return k, c

    longest_c = max(block_k, -(-max(lengths + [0]) // block_k) * block_k)
    c = block_k
    while c < longest_c and sum(split(n, c)[0] for n in lengths) > budget:
        c += block_k
    start, chunk = [0], []
    for n in lengths:
        k, cb = split(n, c)
        start.append(start[-1] + k)
        chunk.append(cb)
    return start, chunk


def block_k(ctas: int, sm_count: int) -> int:
    return int(_load().oracle_block_k(ctas, sm_count))


def default_threads() -> int:
    return int(_load().oracle_default_threads())


def _rows_arg(rows, total):
    if rows is None:
        return None, total
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, int(r.shape[0])


def mla_decode(q_lat, q_pe, pool, kv_indices, kv_indptr, seq_lens, *, B, q_len, H, d_v,
               scale, kv_scale, fnuz=False, rows=None, n_threads=0, pool2=None, kv2_indices=None,
               kv2_indptr=None):
    """fp64 unsplit attention for absorbed MLA decode.

    q_lat: uint16 bf16 bits [B*q_len, H, d_lat]; q_pe: [B*q_len, H, d_rope] or None;
    pool: uint8 fp8 bytes [N, d_lat + d_rope], or uint16 bf16 bits (the bf16-cache variant; pool2
    then holds bf16 bits too).  With pool2 (q_len 1): query b also attends the second
    cache's rows kv2_indices[kv2_indptr[b]:kv2_indptr[b+1]], in the same softmax.
    Returns (o [n_rows, d_v] float64, lse2 [n_rows])."""
    q_lat = _c(q_lat, np.uint16)
    d_lat = q_lat.shape[-1]
    if q_pe is not None:
        q_pe = _c(q_pe, np.uint16)
        d_rope = q_pe.shape[-1]
    else:
        d_rope = 0
    kv_bf16 = np.asarray(pool).dtype == np.uint16
    pool = _c(pool, np.uint16 if kv_bf16 else np.uint8)
    assert pool.shape[-1] == d_lat + d_rope, (pool.shape, d_lat, d_rope)
    kv_indices = _c(kv_indices, np.int32)
    kv_indptr = _c(kv_indptr, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    rows_a, n_rows = _rows_arg(rows, B * q_len * H)
    o = np.empty((n_rows, d_v), dtype=np.float64)
    lse2 = np.empty((n_rows,), dtype=np.float64)
    if kv_bf16 and pool2 is not None:
        assert q_len == 1 and not fnuz
        pool2 = _c(pool2, np.uint16)
        assert pool2.shape[-1] == d_lat + d_rope, (pool2.shape, d_lat, d_rope)
        kv2_indices = _c(kv2_indices, np.int32)
        kv2_indptr = _c(kv2_indptr, np.int32)
        rc = _load().oracle_mla_decode_two_caches_bf16(
            B, H, d_lat, d_rope, d_v, _ptr(q_lat), _ptr(q_pe), _ptr(pool), pool.shape[0],
            _ptr(kv_indices), _ptr(kv_indptr), _ptr(seq_lens), _ptr(pool2), pool2.shape[0],
            _ptr(kv2_indices), _ptr(kv2_indptr), float(scale), float(kv_scale), _ptr(rows_a),
            n_rows, _ptr(o), _ptr(lse2), int(n_threads))
    elif kv_bf16:
        assert not fnuz
        rc = _load().oracle_mla_decode_bf16(B, q_len, H, d_lat, d_rope, d_v, _ptr(q_lat), _ptr(q_pe),
                                            _ptr(pool), pool.shape[0], _ptr(kv_indices),
                                            _ptr(kv_indptr), _ptr(seq_lens), float(scale),
                                            float(kv_scale), _ptr(rows_a), n_rows, _ptr(o), _ptr(lse2),
                                            int(n_threads))
    elif pool2 is None:
        rc = _load().oracle_mla_decode(B, q_len, H, d_lat, d_rope, d_v, _ptr(q_lat), _ptr(q_pe),
                                       _ptr(pool), pool.shape[0], _ptr(kv_indices), _ptr(kv_indptr),
                                       _ptr(seq_lens), float(scale), float(kv_scale), int(bool(fnuz)),
                                       _ptr(rows_a), n_rows, _ptr(o), _ptr(lse2), int(n_threads))
    else:
        assert q_len == 1 and not fnuz
        pool2 = _c(pool2, np.uint8)
        assert pool2.shape[-1] == d_lat + d_rope, (pool2.shape, d_lat, d_rope)
        kv2_indices = _c(kv2_indices, np.int32)
        kv2_indptr = _c(kv2_indptr, np.int32)
        rc = _load().oracle_mla_decode_two_caches(
            B, H, d_lat, d_rope, d_v, _ptr(q_lat), _ptr(q_pe), _ptr(pool), pool.shape[0],
            _ptr(kv_indices), _ptr(kv_indptr), _ptr(seq_lens), _ptr(pool2), pool2.shape[0],
            _ptr(kv2_indices), _ptr(kv2_indptr), float(scale), float(kv_scale), _ptr(rows_a),
            n_rows, _ptr(o), _ptr(lse2), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_mla_decode rejected its arguments (rc=%d)" % rc)
    return o, lse2


def gqa_decode(q, k_cache, v_cache, kv_page_indices, kv_indptr, seq_lens, *, B, q_len, Hq, Hkv,
               scale, rows=None, n_threads=0):
    """fp64 unsplit attention for grouped-query decode over bf16 pages.

    q: uint16 [B*q_len, Hq, D]; k_cache/v_cache: uint16 [num_pages, page_size, Hkv, D]."""
    q = _c(q, np.uint16)
    k_cache = _c(k_cache, np.uint16)
    v_cache = _c(v_cache, np.uint16)
    num_pages, page_size, hkv, D = k_cache.shape
    assert hkv == Hkv and v_cache.shape == k_cache.shape and q.shape[-1] == D
    kv_page_indices = _c(kv_page_indices, np.int32)
    kv_indptr = _c(kv_indptr, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    rows_a, n_rows = _rows_arg(rows, B * q_len * Hq)
    o = np.empty((n_rows, D), dtype=np.float64)
    lse2 = np.empty((n_rows,), dtype=np.float64)
    rc = _load().oracle_gqa_decode(B, q_len, Hq, Hkv, D, page_size, _ptr(q), _ptr(k_cache),
                                   _ptr(v_cache), num_pages, _ptr(kv_page_indices),
                                   _ptr(kv_indptr), _ptr(seq_lens), float(scale), _ptr(rows_a),
                                   n_rows, _ptr(o), _ptr(lse2), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_gqa_decode rejected its arguments (rc=%d)" % rc)
    return o, lse2


def lse_merge(partial_o, partial_lse2):
    """Base-2 LSE merge.  partial_o [rows, np, dv], partial_lse2 [rows, np] -> (o, lse2)."""
    po = _c(partial_o, np.float64)
    pl = _c(partial_lse2, np.float64)
    rows, np_, dv = po.shape
    assert pl.shape == (rows, np_)
    o = np.empty((rows, dv), dtype=np.float64)
    lse2 = np.empty((rows,), dtype=np.float64)
    rc = _load().oracle_lse_merge(rows, np_, dv, _ptr(po), _ptr(pl), _ptr(o), _ptr(lse2))
    if rc != 0:
        raise ValueError("oracle_lse_merge rejected its arguments (rc=%d)" % rc)
    return o, lse2
