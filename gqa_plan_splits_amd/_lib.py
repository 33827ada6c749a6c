"""ctypes marshalling for libgqa_splits.so (argument passing only; no arithmetic here)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgqa_splits.so")

KIND_MLA_FUSED = 0
KIND_GQA_PAGED = 1
FP8_E4M3FN = 0
FP8_E4M3FNUZ = 1
KV_BF16 = 2
SCRATCH_BYTES = 64 << 20   # GQA_SCRATCH_BYTES: the device-side partials of decode_scratch

# Every function include/gqa_splits.h declares.
_SYMBOLS = ("plan_splits", "plan_sparse_splits", "plan_sparse_splits_measured", "plan_gqa_splits_measured", "plan_mla_splits_measured", "block_k_for", "device_sm_count", "decode_plan", "decode_split",
            "splitk_reduce", "splitk_reduce_f32", "merge_ranks", "decode_workspace_bytes", "decode",
            "plan_proportional_device", "decode_proportional_workspace_bytes", "decode_proportional",
            "decode_scratch", "fp8_e4m3_to_bf16", "bw_stream_read", "bw_gather_rows", "bw_gather_whole_rows",
            "status_string", "last_error_detail")


class GqaError(RuntimeError):
    def __init__(self, status: int, where: str, with_detail: bool = False):
        self.status = status
        detail = last_error_detail() if (status == -4 or with_detail) else ""
        super().__init__("%s failed: %s (status %d)%s" % (where, status_string(status), status,
                                                          (": " + detail) if detail else ""))


class DecodeProblem(ctypes.Structure):
    """Mirror of ``gqa_decode_problem`` (include/gqa_splits.h)."""
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("fp8_format", ctypes.c_int32),
        ("batch", ctypes.c_int64),
        ("q_len", ctypes.c_int64),
        ("num_heads", ctypes.c_int64),
        ("num_kv_heads", ctypes.c_int64),
        ("d_qk", ctypes.c_int64),
        ("d_rope", ctypes.c_int64),
        ("d_v", ctypes.c_int64),
        ("page_size", ctypes.c_int64),
        ("max_num_keys", ctypes.c_int64),
        ("q", ctypes.c_void_p),
        ("q_stride_tok", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("q_pe", ctypes.c_void_p),
        ("q_pe_stride_tok", ctypes.c_int64),
        ("q_pe_stride_head", ctypes.c_int64),
        ("kv", ctypes.c_void_p),
        ("kv_stride_row", ctypes.c_int64),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("kv_indices", ctypes.c_void_p),
        ("kv_indptr", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("kv_scale", ctypes.c_float),
        ("glen", ctypes.c_void_p),
        ("cp_rank", ctypes.c_int32),
        ("cp_world", ctypes.c_int32),
        ("kv2", ctypes.c_void_p),
        ("kv2_stride_row", ctypes.c_int64),
        ("kv2_indices", ctypes.c_void_p),
        ("kv2_indptr", ctypes.c_void_p),
    ]

    # tensors whose memory the struct points at (kept alive with it)
    _keep: tuple = ()

    @property
    def rows(self) -> int:
        return self.batch * self.q_len * self.num_heads


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libgqa_splits.so is not built (run `python gqa_plan_splits_amd/build.py`); "
                          "there is no fallback path")
    try:
        # load torch's HIP runtime first: the library then binds to that same runtime instance
        # (same soname), so streams and memory from torch are valid in its calls
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    pp = ctypes.POINTER(DecodeProblem)
    lib.plan_splits.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(i64)]
    lib.block_k_for.argtypes = [i64, i64]
    lib.plan_sparse_splits.argtypes = [i64, i64, i64, i64, i64, i64, i64, ctypes.POINTER(i64),
                                       ctypes.POINTER(i64)]
    lib.plan_sparse_splits_measured.argtypes = [i64, i64, i64, i64, i64, i64, i64, ctypes.POINTER(i64)]
    lib.plan_gqa_splits_measured.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64)]
    lib.plan_mla_splits_measured.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64)]
    lib.device_sm_count.argtypes = [ctypes.POINTER(i64)]
    lib.decode_plan.argtypes = [pp, i64, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(i32)]
    lib.decode_split.argtypes = [pp, i64, i32, vp, vp, vp]
    lib.splitk_reduce.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
    lib.splitk_reduce_f32.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
    lib.merge_ranks.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
    lib.decode_workspace_bytes.argtypes = [pp, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.decode.argtypes = [pp, i64, i32, vp, ctypes.c_size_t, vp, vp, vp]
    lib.plan_proportional_device.argtypes = [vp, vp, i64, i64, i64, i32, vp, vp, vp]
    lib.decode_proportional_workspace_bytes.argtypes = [pp, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.decode_proportional.argtypes = [pp, i64, i64, i32, vp, ctypes.c_size_t, vp, vp, vp]
    lib.decode_scratch.argtypes = [pp, i64, i32, vp, vp, vp]
    lib.fp8_e4m3_to_bf16.argtypes = [vp, i64, vp, vp]
    lib.bw_stream_read.argtypes = [vp, ctypes.c_size_t, i64, vp]
    lib.bw_gather_rows.argtypes = [vp, i64, vp, i64, i64, vp]
    lib.bw_gather_whole_rows.argtypes = [vp, i64, vp, i64, i64, vp]
    lib.status_string.argtypes = [i32]
    lib.status_string.restype = ctypes.c_char_p
    lib.last_error_detail.argtypes = []
    lib.last_error_detail.restype = ctypes.c_char_p
    for name in _SYMBOLS:
        if name not in ("status_string", "last_error_detail"):
            getattr(lib, name).restype = i32
    _lib = lib
    return lib


_load()


def exported_symbols():
    """Names of the C-ABI functions, resolved in the loaded library."""
    lib = _load()
    return {name: getattr(lib, name) for name in _SYMBOLS}


def status_string(status: int) -> str:
    return _load().status_string(int(status)).decode()


def last_error_detail() -> str:
    return _load().last_error_detail().decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise GqaError(rc, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# ----------------------------------------------------------------------------------------------
# planning
# ----------------------------------------------------------------------------------------------

def plan_splits(batch_size: int, num_keys: int, heads_per_group: int, sm_count: int = 0,
                is_mla: bool = False) -> int:
    out = ctypes.c_int64(0)
    _check(_load().plan_splits(batch_size, num_keys, heads_per_group, sm_count, int(bool(is_mla)),
                               ctypes.byref(out)), "plan_splits")
    return out.value


def plan_gqa_splits_measured(batch_size: int, max_num_keys: int, num_kv_heads: int,
                             sm_count: int = 0) -> int:
    out = ctypes.c_int64(0)
    _check(_load().plan_gqa_splits_measured(batch_size, max_num_keys, num_kv_heads, sm_count,
                                            ctypes.byref(out)), "plan_gqa_splits_measured")
    return out.value


def plan_mla_splits_measured(batch_size: int, max_num_keys: int, rows_per_request: int,
                             sm_count: int = 0) -> int:
    out = ctypes.c_int64(0)
    _check(_load().plan_mla_splits_measured(batch_size, max_num_keys, rows_per_request, sm_count,
                                            ctypes.byref(out)), "plan_mla_splits_measured")
    return out.value


def plan_sparse_splits(num_tokens: int, num_heads: int, topk: int, extra_topk: int = 0, *,
                       num_sms: int = 0, max_splits: int = 16, head_tiles: int = 4):
    """(num_splits, chunks_per_block) of the sparse top-k planner (chunks of 64 candidates)."""
    ns = ctypes.c_int64(0)
    cpb = ctypes.c_int64(0)
    _check(_load().plan_sparse_splits(num_tokens, num_heads, topk, extra_topk, num_sms, max_splits,
                                      head_tiles, ctypes.byref(ns), ctypes.byref(cpb)),
           "plan_sparse_splits")
    return int(ns.value), int(cpb.value)


def plan_sparse_splits_measured(num_tokens: int, num_heads: int, topk: int, extra_topk: int = 0, *,
                                sm_count: int = 0, max_splits: int = 256, rows_per_cta: int = 64) -> int:
    """Split count of the sparse planner with thresholds measured on MI355X (not the page's)."""
    out = ctypes.c_int64(0)
    _check(_load().plan_sparse_splits_measured(num_tokens, num_heads, topk, extra_topk, sm_count,
                                               max_splits, rows_per_cta, ctypes.byref(out)),
           "plan_sparse_splits_measured")
    return int(out.value)


def block_k_for(ctas: int, sm_count: int) -> int:
    rc = _load().block_k_for(ctas, sm_count)
    if rc < 0:
        raise GqaError(rc, "block_k_for")
    return rc


def device_sm_count() -> int:
    out = ctypes.c_int64(0)
    _check(_load().device_sm_count(ctypes.byref(out)), "device_sm_count")
    return out.value


def decode_plan(problem: DecodeProblem, np: int = 0, block_k: int = 0, sm_count: int = 0):
    n = ctypes.c_int64(0)
    bk = ctypes.c_int(0)
    _check(_load().decode_plan(ctypes.byref(problem), np, block_k, sm_count, ctypes.byref(n),
                               ctypes.byref(bk)), "decode_plan")
    return n.value, bk.value


# ----------------------------------------------------------------------------------------------
# problems from torch tensors
# ----------------------------------------------------------------------------------------------

def _strides(t):
    s = t.stride()
    if s[-1] != 1:
        raise ValueError("the last dimension must be contiguous")
    return s[0], s[1]


def mla_problem(q_lat, q_pe, pool, kv_indices, kv_indptr, seq_lens, *, batch, q_len, num_heads,
                max_num_keys, scale, kv_scale, d_v=None, fp8_format=None, glen=None,
                cp_rank=0, cp_world=1, pool2=None, kv2_indices=None, kv2_indptr=None) -> DecodeProblem:
    """Absorbed-MLA (or sparse top-k) problem: q_lat [B*q_len, H, d_lat], q_pe [.., H, d_rope]
    bf16 views; pool [N, d_qk] fp8 bytes (uint8 or float8), or bf16 (format KV_BF16, the default
    for a bf16 pool); int32 index tensors.  With glen
    (int32 [B] global lengths), the call is rank cp_rank of cp_world decode-context-parallel
    ranks: seq_lens and the index lists hold that rank's positions.  With pool2 (sparse rows,
    q_len 1; the pool's row stride), request b also attends the second-cache rows
    kv2_indices[kv2_indptr[b]:kv2_indptr[b+1]]; max_num_keys covers both lists."""
    p = DecodeProblem()
    p.kind = KIND_MLA_FUSED
    if fp8_format is None:
        import torch
        fp8_format = KV_BF16 if pool.dtype == torch.bfloat16 else FP8_E4M3FN
    p.fp8_format = fp8_format
    p.batch, p.q_len, p.num_heads, p.num_kv_heads = batch, q_len, num_heads, 1
    p.d_rope = q_pe.shape[-1]
    p.d_qk = q_lat.shape[-1] + p.d_rope
    p.d_v = d_v if d_v is not None else q_lat.shape[-1]
    p.page_size = 1
    p.max_num_keys = max_num_keys
    p.q = q_lat.data_ptr()
    p.q_stride_tok, p.q_stride_head = _strides(q_lat)
    p.q_pe = q_pe.data_ptr()
    p.q_pe_stride_tok, p.q_pe_stride_head = _strides(q_pe)
    p.kv = pool.data_ptr()
    p.kv_stride_row = pool.stride(0) * pool.element_size()
    p.kv_indices = kv_indices.data_ptr()
    p.kv_indptr = kv_indptr.data_ptr()
    p.seq_lens = seq_lens.data_ptr()
    p.scale = scale
    p.kv_scale = kv_scale
    if glen is not None:
        p.glen = glen.data_ptr()
        p.cp_rank, p.cp_world = cp_rank, cp_world
    if pool2 is not None:
        p.kv2 = pool2.data_ptr()
        p.kv2_stride_row = pool2.stride(0) * pool2.element_size()
        p.kv2_indices = kv2_indices.data_ptr()
        p.kv2_indptr = kv2_indptr.data_ptr()
    p._keep = (q_lat, q_pe, pool, kv_indices, kv_indptr, seq_lens, glen, pool2, kv2_indices, kv2_indptr)
    return p


def gqa_problem(q, k_cache, v_cache, kv_page_indices, kv_indptr, seq_lens, *, batch, q_len,
                max_num_keys, scale) -> DecodeProblem:
    """Paged grouped-query problem: q [B*q_len, Hq, 128] bf16; caches
    [pages, page_size, Hkv, 128] bf16 (contiguous); int32 index tensors."""
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("K/V caches must be contiguous")
    p = DecodeProblem()
    p.kind = KIND_GQA_PAGED
    p.fp8_format = FP8_E4M3FN
    p.batch, p.q_len = batch, q_len
    p.num_heads = q.shape[1]
    p.num_kv_heads = k_cache.shape[2]
    p.d_qk = p.d_v = q.shape[-1]
    p.d_rope = 0
    p.page_size = k_cache.shape[1]
    p.max_num_keys = max_num_keys
    p.q = q.data_ptr()
    p.q_stride_tok, p.q_stride_head = _strides(q)
    p.k_cache = k_cache.data_ptr()
    p.v_cache = v_cache.data_ptr()
    p.kv_indices = kv_page_indices.data_ptr()
    p.kv_indptr = kv_indptr.data_ptr()
    p.seq_lens = seq_lens.data_ptr()
    p.scale = scale
    p.kv_scale = 1.0
    p._keep = (q, k_cache, v_cache, kv_page_indices, kv_indptr, seq_lens)
    return p


# ----------------------------------------------------------------------------------------------
# split, reduce, decode
# ----------------------------------------------------------------------------------------------

def decode_split(problem: DecodeProblem, np: int, block_k: int, partial_o, partial_lse2,
                 stream=None):
    _check(_load().decode_split(ctypes.byref(problem), np, block_k, _ptr(partial_o),
                                _ptr(partial_lse2), _stream(stream)), "decode_split")


def splitk_reduce(rows: int, np: int, d_v: int, partial_o, partial_lse2, out, lse2_out=None,
                  stream=None):
    _check(_load().splitk_reduce(rows, np, d_v, _ptr(partial_o), _ptr(partial_lse2), _ptr(out),
                                 _ptr(lse2_out), _stream(stream)), "splitk_reduce")


def splitk_reduce_f32(rows: int, np: int, d_v: int, partial_o, partial_lse2, out, lse2_out=None,
                      stream=None):
    _check(_load().splitk_reduce_f32(rows, np, d_v, _ptr(partial_o), _ptr(partial_lse2), _ptr(out),
                                     _ptr(lse2_out), _stream(stream)), "splitk_reduce_f32")


def merge_ranks(world: int, rows: int, d_v: int, parts, lse2, out, lse2_out=None, stream=None):
    """Merge of decode-context-parallel rank outputs: parts [world, rows, d_v] fp32 (each rank's
    splitk_reduce_f32 output), lse2 [world, rows] fp32 -> out [rows, d_v] bf16 (+ lse2_out)."""
    _check(_load().merge_ranks(world, rows, d_v, _ptr(parts), _ptr(lse2), _ptr(out), _ptr(lse2_out),
                               _stream(stream)), "merge_ranks")


def decode_workspace_bytes(problem: DecodeProblem, np: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(_load().decode_workspace_bytes(ctypes.byref(problem), np, ctypes.byref(out)),
           "decode_workspace_bytes")
    return out.value


def decode(problem: DecodeProblem, out, lse2_out=None, *, np: int = 0, block_k: int = 0,
           workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_load().decode(ctypes.byref(problem), np, block_k, _ptr(workspace), ws_bytes, _ptr(out),
                          _ptr(lse2_out), _stream(stream)), "decode")


def decode_scratch(problem: DecodeProblem, out, lse2_out=None, *, np: int = 0, block_k: int = 0,
                   stream=None):
    rc = _load().decode_scratch(ctypes.byref(problem), np, block_k, _ptr(out), _ptr(lse2_out),
                                _stream(stream))
    if rc != 0:
        raise GqaError(rc, "decode_scratch", with_detail=True)


def bw_stream_read(src, nbytes: int, ctas: int, stream=None):
    _check(_load().bw_stream_read(_ptr(src), nbytes, ctas, _stream(stream)), "bw_stream_read")


def bw_gather_rows(pool, row_bytes: int, idx, n: int, ctas: int, stream=None):
    _check(_load().bw_gather_rows(_ptr(pool), row_bytes, _ptr(idx), n, ctas, _stream(stream)),
           "bw_gather_rows")


def bw_gather_whole_rows(pool, row_bytes: int, idx, n: int, ctas: int, stream=None):
    _check(_load().bw_gather_whole_rows(_ptr(pool), row_bytes, _ptr(idx), n, ctas, _stream(stream)),
           "bw_gather_whole_rows")


def plan_proportional_device(seq_lens, extra_indptr, batch: int, budget: int, cap: int,
                             block_k: int, part_start, part_chunk, stream=None):
    """Device-side length-proportional plan into part_start [batch + 1] and part_chunk [batch]
    (int32 device tensors)."""
    _check(_load().plan_proportional_device(_ptr(seq_lens), _ptr(extra_indptr), batch, budget, cap,
                                            block_k, _ptr(part_start), _ptr(part_chunk),
                                            _stream(stream)), "plan_proportional_device")


def decode_proportional_workspace_bytes(problem: DecodeProblem, np: int = 0, cap: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(_load().decode_proportional_workspace_bytes(ctypes.byref(problem), np, cap,
                                                       ctypes.byref(out)),
           "decode_proportional_workspace_bytes")
    return out.value


def decode_proportional(problem: DecodeProblem, out, lse2_out=None, *, np: int = 0, cap: int = 0,
                        block_k: int = 0, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_load().decode_proportional(ctypes.byref(problem), np, cap, block_k, _ptr(workspace),
                                       ws_bytes, _ptr(out), _ptr(lse2_out), _stream(stream)),
           "decode_proportional")


def fp8_e4m3_to_bf16(inp, n: int, out, stream=None):
    _check(_load().fp8_e4m3_to_bf16(_ptr(inp), n, _ptr(out), _stream(stream)), "fp8_e4m3_to_bf16")
