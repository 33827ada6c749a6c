"""Split-KV attention decode for MI355X (gfx950): Python binding of the C ABI.

Every entry point of ``include/gqa_splits.h`` has a function of the same name here; this module
only marshals arguments (device pointers, sizes, the current HIP stream) and raises
:class:`GqaError` on a non-zero status.  All arithmetic runs in the HIP kernels of
``libgqa_splits.so``; if that library has not been built, importing the binding raises.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    DecodeProblem,
    GqaError,
    KIND_GQA_PAGED,
    KIND_MLA_FUSED,
    FP8_E4M3FN,
    FP8_E4M3FNUZ,
    KV_BF16,
    block_k_for,
    bw_gather_rows,
    bw_gather_whole_rows,
    bw_stream_read,
    decode,
    decode_plan,
    decode_scratch,
    SCRATCH_BYTES,
    decode_split,
    decode_workspace_bytes,
    decode_proportional,
    decode_proportional_workspace_bytes,
    plan_proportional_device,
    device_sm_count,
    exported_symbols,
    fp8_e4m3_to_bf16,
    gqa_problem,
    last_error_detail,
    library_path,
    merge_ranks,
    mla_problem,
    plan_gqa_splits_measured,
    plan_mla_splits_measured,
    plan_sparse_splits,
    plan_sparse_splits_measured,
    plan_splits,
    splitk_reduce,
    splitk_reduce_f32,
    status_string,
)
