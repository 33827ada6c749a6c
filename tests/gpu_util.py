"""Test plumbing shared by the GPU parity tests and the smoke check: build C-ABI problems from
seeded inputs, run the HIP path, and run the oracle on the same input bytes.

Tolerances (the bar the parity tests apply to every floating-point result):
  * output: max |o_gpu - o_ref| <= 1e-2 (bf16 output), and the relative error
    max|o_gpu - o_ref| / max|o_ref| <= 1e-2 as a second, scale-free gate;
  * base-2 LSE: |lse2_gpu - lse2_ref| <= 1e-4 * max(1, |lse2_ref|);
  * rows that see no key: o == 0 exactly and lse2 == -inf on both sides.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import gqa_plan_splits_amd as g
import oracle

OUT_ATOL = 1e-2
OUT_REL = 1e-2
LSE_RTOL = 1e-4


def bits16(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def pool_np(pool):
    """A pool tensor as numpy: uint8 fp8 bytes, or uint16 bits of bf16 rows."""
    pool = pool.contiguous().cpu()
    if pool.dtype == torch.bfloat16:
        return pool.view(torch.int16).numpy().view(np.uint16)
    return pool.numpy()


def mla_problem(inp):
    return g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, inp.kv_indices, inp.kv_indptr, inp.seq_lens,
                         batch=inp.B, q_len=inp.q_len, num_heads=inp.H,
                         max_num_keys=inp.max_num_keys, scale=inp.scale, kv_scale=inp.kv_scale,
                         d_v=inp.d_v, pool2=inp.pool2, kv2_indices=inp.kv2_indices,
                         kv2_indptr=inp.kv2_indptr)


def gqa_problem(inp):
    return g.gqa_problem(inp.q, inp.k_cache, inp.v_cache, inp.kv_page_indices, inp.kv_indptr,
                         inp.seq_lens, batch=inp.B, q_len=inp.q_len, max_num_keys=inp.max_num_keys,
                         scale=inp.scale)


def run_decode(problem, d_v, np_=0, block_k=0, stream=None):
    """decode() through the C ABI; returns (out bf16 [rows, d_v], lse2 fp32 [rows]) on device."""
    dev = torch.device("cuda")
    rows = problem.rows
    out = torch.empty((rows, d_v), dtype=torch.bfloat16, device=dev)
    lse2 = torch.empty((rows,), dtype=torch.float32, device=dev)
    ws_bytes = g.decode_workspace_bytes(problem, np_)
    ws = torch.empty((max(ws_bytes, 256) // 4 + 64,), dtype=torch.float32, device=dev)
    g.decode(problem, out, lse2, np=np_, block_k=block_k, workspace=ws, stream=stream)
    return out, lse2


def oracle_mla(inp, rows=None, n_threads=0):
    """fp64 oracle over the same bytes.  With rows given, only the requests those rows belong to
    are copied to the host (their pool rows gathered in key order; storage order does not change
    attention)."""
    H, q_len = inp.H, inp.q_len
    if rows is None:
        second = {}
        if inp.pool2 is not None:
            second = dict(pool2=pool_np(inp.pool2), kv2_indices=inp.kv2_indices.cpu().numpy(),
                          kv2_indptr=inp.kv2_indptr.cpu().numpy())
        return oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), pool_np(inp.pool),
                                 inp.kv_indices.cpu().numpy(), inp.kv_indptr.cpu().numpy(),
                                 inp.seq_lens.cpu().numpy(), B=inp.B, q_len=q_len, H=H,
                                 d_v=inp.d_v, scale=inp.scale, kv_scale=inp.kv_scale,
                                 n_threads=n_threads, **second)
    assert inp.pool2 is None, "sampled rows: one cache only"
    rows = list(rows)
    reqs = sorted({r // (q_len * H) for r in rows})
    indptr = inp.kv_indptr.cpu()
    lens = inp.seq_lens.cpu()
    pools, idx, new_indptr, new_lens = [], [], [0], []
    n_pool = 0
    for b in reqs:
        a, e = int(indptr[b]), int(indptr[b]) + int(lens[b])
        sel = inp.kv_indices[a:e].long().cpu()
        ok = sel >= 0   # negative: a skipped key, kept as -1 in the new list
        pools.append(inp.pool[sel[ok].to(inp.pool.device)].cpu())
        new_idx = torch.full((e - a,), -1, dtype=torch.int32)
        new_idx[ok] = torch.arange(n_pool, n_pool + int(ok.sum()), dtype=torch.int32)
        n_pool += int(ok.sum())
        idx.append(new_idx)
        new_indptr.append(new_indptr[-1] + (e - a))
        new_lens.append(e - a)
    pool = torch.cat(pools) if pools else torch.zeros((1, inp.d_qk), dtype=inp.pool.dtype)
    if pool.shape[0] == 0:
        pool = torch.zeros((1, inp.d_qk), dtype=inp.pool.dtype)
    ql = torch.cat([inp.q_lat[b * q_len:(b + 1) * q_len].cpu() for b in reqs])
    qp = torch.cat([inp.q_pe[b * q_len:(b + 1) * q_len].cpu() for b in reqs])
    pos = {b: i for i, b in enumerate(reqs)}
    sub_rows = [pos[r // (q_len * H)] * q_len * H + r % (q_len * H) for r in rows]
    return oracle.mla_decode(bits16(ql), bits16(qp), pool_np(pool), torch.cat(idx).numpy(),
                             np.array(new_indptr, dtype=np.int32), np.array(new_lens, dtype=np.int32),
                             B=len(reqs), q_len=q_len, H=H, d_v=inp.d_v, scale=inp.scale,
                             kv_scale=inp.kv_scale, rows=sub_rows, n_threads=n_threads)


def oracle_gqa(inp, rows=None, n_threads=0):
    """fp64 oracle; with rows given, only the pages of those rows' requests are copied."""
    Hq, q_len, ps = inp.Hq, inp.q_len, inp.page_size
    if rows is None:
        return oracle.gqa_decode(bits16(inp.q), bits16(inp.k_cache), bits16(inp.v_cache),
                                 inp.kv_page_indices.cpu().numpy(), inp.kv_indptr.cpu().numpy(),
                                 inp.seq_lens.cpu().numpy(), B=inp.B, q_len=q_len, Hq=Hq,
                                 Hkv=inp.Hkv, scale=inp.scale, n_threads=n_threads)
    rows = list(rows)
    reqs = sorted({r // (q_len * Hq) for r in rows})
    indptr = inp.kv_indptr.cpu()
    lens = inp.seq_lens.cpu()
    kp, vp, pidx, new_indptr, new_lens = [], [], [], [0], []
    for b in reqs:
        a = int(indptr[b])
        npg = (int(lens[b]) + ps - 1) // ps
        sel = inp.kv_page_indices[a:a + npg].long()
        kp.append(inp.k_cache[sel].cpu())
        vp.append(inp.v_cache[sel].cpu())
        pidx.append(torch.arange(new_indptr[-1], new_indptr[-1] + npg, dtype=torch.int32))
        new_indptr.append(new_indptr[-1] + npg)
        new_lens.append(int(lens[b]))
    q = torch.cat([inp.q[b * q_len:(b + 1) * q_len].cpu() for b in reqs])
    pos = {b: i for i, b in enumerate(reqs)}
    sub_rows = [pos[r // (q_len * Hq)] * q_len * Hq + r % (q_len * Hq) for r in rows]
    return oracle.gqa_decode(bits16(q), bits16(torch.cat(kp)), bits16(torch.cat(vp)),
                             torch.cat(pidx).numpy(), np.array(new_indptr, dtype=np.int32),
                             np.array(new_lens, dtype=np.int32), B=len(reqs), q_len=q_len, Hq=Hq,
                             Hkv=inp.Hkv, scale=inp.scale, rows=sub_rows, n_threads=n_threads)


def compare(out, lse2, ref_o, ref_l, what=""):
    """Applies the tolerances above; returns (max_abs, rel, max_lse_err)."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse2.cpu().numpy().astype(np.float64)
    assert o.shape == ref_o.shape, (o.shape, ref_o.shape)
    assert np.all(np.isfinite(o)), what + ": non-finite output"
    empty = ~np.isfinite(ref_l)
    assert np.array_equal(empty, ~np.isfinite(l)), what + ": empty-row mismatch"
    assert np.all(l[empty] == -np.inf) and np.all(o[empty] == 0), what + ": empty rows"
    err = np.abs(o - ref_o)
    max_abs = float(err.max()) if err.size else 0.0
    scale = float(np.abs(ref_o).max()) if ref_o.size else 0.0
    rel = max_abs / scale if scale > 0 else max_abs
    lerr = np.abs(l[~empty] - ref_l[~empty]) / np.maximum(1.0, np.abs(ref_l[~empty]))
    max_l = float(lerr.max()) if lerr.size else 0.0
    assert max_abs <= OUT_ATOL, "%s: max|dO| %.3g > %g" % (what, max_abs, OUT_ATOL)
    assert rel <= OUT_REL, "%s: relative error %.3g > %g" % (what, rel, OUT_REL)
    assert max_l <= LSE_RTOL, "%s: lse2 error %.3g > %g" % (what, max_l, LSE_RTOL)
    return max_abs, rel, max_l


def sample_rows(B, q_len, H, n, seed):
    """n distinct rows spread over requests, draft positions and heads (always includes the
    first and the last row)."""
    total = B * q_len * H
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(total, size=min(n, total) - 2, replace=False).tolist()) | {0, total - 1}
    return sorted(pick)


def log(msg):
    print(msg, flush=True)
