"""Pins of the oracle's attention and merge against the mathematics (CPU only).

* textbook: torch CPU float64 softmax / scaled_dot_product_attention over keys decoded by
  torch's own float8 and bfloat16 conversions (library routines independent of the oracle);
* closed forms: one key, zero query, identical keys, empty windows;
* invariants: slot permutation, key order, the end-aligned draft window (moonmath-amd README,
  "MLA decode": draft position t attends KV [0, S - q_len + t]);
* merge: split + base-2 LSE merge equals the unsplit result, plus the merge's closed forms.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

LN2 = math.log(2.0)


def bits16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def u8(t):
    return t.contiguous().numpy()


def run_mla(inp, rows=None, n_threads=0):
    return oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), u8(inp.pool),
                             inp.kv_indices.numpy(), inp.kv_indptr.numpy(), inp.seq_lens.numpy(),
                             B=inp.B, q_len=inp.q_len, H=inp.H, d_v=inp.d_v, scale=inp.scale,
                             kv_scale=inp.kv_scale, rows=rows, n_threads=n_threads)


def run_gqa(inp, rows=None):
    return oracle.gqa_decode(bits16(inp.q), bits16(inp.k_cache), bits16(inp.v_cache),
                             inp.kv_page_indices.numpy(), inp.kv_indptr.numpy(),
                             inp.seq_lens.numpy(), B=inp.B, q_len=inp.q_len, Hq=inp.Hq,
                             Hkv=inp.Hkv, scale=inp.scale, rows=rows)


def torch_mla_reference(inp):
    """Textbook attention with torch CPU float64 (library decode of fp8 and bf16)."""
    q = torch.cat([inp.q_lat, inp.q_pe], dim=-1).to(torch.float64)  # [B*q_len, H, d_qk]
    pool = inp.pool.view(torch.float8_e4m3fn).to(torch.float64) * inp.kv_scale
    outs, lses = [], []
    for b in range(inp.B):
        S = int(inp.seq_lens[b])
        idx = inp.kv_indices[int(inp.kv_indptr[b]):int(inp.kv_indptr[b]) + S].long()
        K = pool[idx]                      # [S, d_qk]
        V = K[:, :inp.d_v]
        for t in range(inp.q_len):
            L = max(0, S - inp.q_len + t + 1)
            qr = q[b * inp.q_len + t]     # [H, d_qk]
            if L == 0:
                outs.append(torch.zeros(inp.H, inp.d_v, dtype=torch.float64))
                lses.append(torch.full((inp.H,), -math.inf, dtype=torch.float64))
                continue
            s = inp.scale * (qr @ K[:L].T)  # [H, L]
            outs.append(torch.softmax(s, dim=-1) @ V[:L])
            lses.append(torch.logsumexp(s, dim=-1) / LN2)
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


def small_mla(seed=11, B=3, q_len=2, H=4, lens=(5, 1, 17), d_qk=40, d_rope=8, d_v=32, pool_rows=40):
    return workloads.mla_inputs(B=B, q_len=q_len, H=H, seq_lens=list(lens), pool_rows=pool_rows,
                                d_qk=d_qk, d_rope=d_rope, d_v=d_v, seed=seed)


@pytest.mark.parametrize("shape", [
    dict(B=3, q_len=2, H=4, lens=(5, 1, 17), d_qk=40, d_rope=8, d_v=32, pool_rows=40),
    dict(B=2, q_len=1, H=16, lens=(64, 33), d_qk=576, d_rope=64, d_v=512, pool_rows=128),
    dict(B=2, q_len=4, H=3, lens=(9, 2), d_qk=576, d_rope=64, d_v=512, pool_rows=16),
    dict(B=2, q_len=1, H=5, lens=(20, 7), d_qk=512, d_rope=64, d_v=448, pool_rows=64),
])
def test_mla_matches_torch_textbook(shape):
    inp = small_mla(**shape)
    o, lse2 = run_mla(inp)
    ref_o, ref_lse = torch_mla_reference(inp)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse2))
    np.testing.assert_allclose(lse2[fin], ref_lse[fin], rtol=1e-12, atol=1e-12)
    assert np.all(lse2[~fin] == -np.inf)


def test_mla_matches_sdpa():
    inp = small_mla(seed=5, B=1, q_len=1, H=6, lens=(31,), pool_rows=31)
    o, _ = run_mla(inp)
    q = torch.cat([inp.q_lat, inp.q_pe], -1).to(torch.float64)[None]          # [1, H, 1?]
    pool = inp.pool.view(torch.float8_e4m3fn).to(torch.float64) * inp.kv_scale
    K = pool[inp.kv_indices.long()]
    qq = q.reshape(1, inp.H, 1, -1)
    kk = K[None, None].expand(1, inp.H, -1, -1)
    vv = kk[..., :inp.d_v]
    ref = F.scaled_dot_product_attention(qq, kk, vv, scale=inp.scale).reshape(inp.H, inp.d_v)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_threads_do_not_change_bits():
    inp = small_mla(seed=3)
    o1, l1 = run_mla(inp, n_threads=1)
    o4, l4 = run_mla(inp, n_threads=4)
    assert np.array_equal(o1, o4) and np.array_equal(l1, l4)


def test_row_subset_equals_full():
    inp = small_mla(seed=4)
    o, l = run_mla(inp)
    rows = [5, 0, 23, 7]
    os_, ls_ = run_mla(inp, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls_, l[rows])


def test_single_key_closed_form():
    inp = small_mla(seed=6, B=1, q_len=1, H=3, lens=(1,), pool_rows=4)
    o, l = run_mla(inp)
    k = inp.pool[int(inp.kv_indices[0])].view(torch.float8_e4m3fn).to(torch.float64) * inp.kv_scale
    q = torch.cat([inp.q_lat, inp.q_pe], -1).to(torch.float64)[0]
    s = inp.scale * (q @ k)
    for h in range(3):
        assert np.array_equal(o[h], k[:inp.d_v].numpy())          # softmax of one key is 1
        assert l[h] == pytest.approx(float(s[h]) / LN2, rel=1e-14, abs=1e-14)


def test_zero_query_closed_form():
    inp = small_mla(seed=8, B=1, q_len=1, H=2, lens=(13,), pool_rows=13)
    inp.q_lat.zero_()
    inp.q_pe.zero_()
    o, l = run_mla(inp)
    V = (inp.pool[inp.kv_indices.long()].view(torch.float8_e4m3fn).to(torch.float64)
         * inp.kv_scale)[:, :inp.d_v].numpy()
    mean = np.array([math.fsum(V[:, d]) / 13 for d in range(inp.d_v)])
    for h in range(2):
        np.testing.assert_allclose(o[h], mean, rtol=1e-14, atol=1e-15)
        assert l[h] == pytest.approx(math.log2(13), rel=1e-15)


def test_identical_keys_closed_form():
    inp = small_mla(seed=9, B=1, q_len=1, H=2, lens=(12,), pool_rows=5)
    inp.kv_indices.fill_(3)
    o, l = run_mla(inp)
    k = inp.pool[3].view(torch.float8_e4m3fn).to(torch.float64) * inp.kv_scale
    q = torch.cat([inp.q_lat, inp.q_pe], -1).to(torch.float64)[0]
    s = inp.scale * (q @ k)
    for h in range(2):
        np.testing.assert_allclose(o[h], k[:inp.d_v].numpy(), rtol=1e-14, atol=1e-15)
        assert l[h] == pytest.approx(float(s[h]) / LN2 + math.log2(12), rel=1e-14)


def test_empty_window_rows():
    # seq_len 2 with a 4-token draft window: positions 0 and 1 see no key at all
    inp = small_mla(seed=10, B=1, q_len=4, H=2, lens=(2,), pool_rows=4)
    o, l = run_mla(inp)
    o = o.reshape(4, 2, -1)
    l = l.reshape(4, 2)
    assert np.all(o[:2] == 0) and np.all(l[:2] == -np.inf)
    assert np.all(np.isfinite(l[2:]))


def test_slot_permutation_invariance():
    inp = small_mla(seed=12)
    o, l = run_mla(inp)
    g = torch.Generator().manual_seed(1)
    perm = torch.randperm(inp.pool.shape[0], generator=g)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel())
    inp.pool = inp.pool[perm].contiguous()            # row i of the new pool is old row perm[i]
    inp.kv_indices = inv[inp.kv_indices.long()].to(torch.int32)
    o2, l2 = run_mla(inp)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_key_order_invariance():
    inp = small_mla(seed=13, lens=(5, 1, 17))
    o, l = run_mla(inp)
    g = torch.Generator().manual_seed(2)
    for b in range(inp.B):
        a, e = int(inp.kv_indptr[b]), int(inp.kv_indptr[b + 1])
        seg = inp.kv_indices[a:e]
        inp.kv_indices[a:e] = seg[torch.randperm(e - a, generator=g)]
    # reordering keys changes the window's membership when q_len > 1; compare q_len-1 rows only
    o2, l2 = run_mla(inp)
    last = [r for r in range(inp.rows) if (r // inp.H) % inp.q_len == inp.q_len - 1]
    np.testing.assert_allclose(o2[last], o[last], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2[last], l[last], rtol=1e-14)


def test_draft_window_equals_shorter_decode():
    S, q_len, H = 21, 4, 3
    inp = small_mla(seed=14, B=1, q_len=q_len, H=H, lens=(S,), pool_rows=S)
    o, l = run_mla(inp)
    for t in range(q_len):
        one = small_mla(seed=14, B=1, q_len=1, H=H, lens=(S,), pool_rows=S)
        one.pool = inp.pool
        one.kv_indices = inp.kv_indices
        one.q_lat = inp.q_lat[t:t + 1].clone()
        one.q_pe = inp.q_pe[t:t + 1].clone()
        one.seq_lens = torch.tensor([S - q_len + t + 1], dtype=torch.int32)
        o1, l1 = run_mla(one)
        assert np.array_equal(o1, o[t * H:(t + 1) * H]) and np.array_equal(l1, l[t * H:(t + 1) * H])


@pytest.mark.parametrize("np_", [1, 2, 3, 7, 40])
def test_split_then_merge_equals_unsplit(np_):
    """Splitting a request's keys into contiguous partitions, attending to each, and merging the
    partial results by base-2 LSE reproduces the unsplit attention (exact in real arithmetic).
    Partitions past the end are empty and carry lse2 = -inf."""
    S, H = 37, 4
    inp = small_mla(seed=15, B=1, q_len=1, H=H, lens=(S,), pool_rows=64)
    o, l = run_mla(inp)
    chunk = -(-S // np_)
    po = np.zeros((H, np_, inp.d_v))
    pl = np.full((H, np_), -np.inf)
    for p in range(np_):
        a, e = min(S, p * chunk), min(S, (p + 1) * chunk)
        part = small_mla(seed=15, B=1, q_len=1, H=H, lens=(S,), pool_rows=64)
        part.pool, part.q_lat, part.q_pe = inp.pool, inp.q_lat, inp.q_pe
        part.kv_indices = inp.kv_indices[a:e].clone() if e > a else torch.zeros(1, dtype=torch.int32)
        part.kv_indptr = torch.tensor([0, max(e - a, 1)], dtype=torch.int32)
        part.seq_lens = torch.tensor([e - a], dtype=torch.int32)
        op, lp = run_mla(part)
        po[:, p], pl[:, p] = op, lp
    mo, ml = oracle.lse_merge(po, pl)
    np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ml, l, rtol=1e-14)


def test_merge_closed_forms():
    rng = np.random.default_rng(0)
    a = rng.normal(size=(3, 16))
    b = rng.normal(size=(3, 16))
    # two partitions of equal weight: lse2 grows by exactly 1, output is the mean
    o, l = oracle.lse_merge(np.stack([a, b], 1), np.full((3, 2), 5.25))
    np.testing.assert_allclose(o, (a + b) / 2, rtol=1e-15, atol=1e-16)
    assert np.all(l == 6.25)
    # one partition: identity
    o, l = oracle.lse_merge(a[:, None], np.array([[1.5], [-3.0], [40.0]]))
    assert np.array_equal(o, a) and np.array_equal(l, [1.5, -3.0, 40.0])
    # empty partitions carry no weight, even with garbage outputs
    po = np.stack([a, np.full_like(a, np.nan)], 1)
    o, l = oracle.lse_merge(po, np.array([[2.0, -np.inf]] * 3))
    assert np.array_equal(o, a) and np.all(l == 2.0)
    # nothing at all: zeros and -inf
    o, l = oracle.lse_merge(po, np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(l == -np.inf)
    # weights 2^lse2: lse2 = (3, 4) gives weights 1/3 and 2/3
    o, l = oracle.lse_merge(np.stack([a, b], 1), np.array([[3.0, 4.0]] * 3))
    np.testing.assert_allclose(o, a / 3 + 2 * b / 3, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l, np.log2(8.0 + 16.0), rtol=1e-15)


# --------------------------------------------------------------------------------------------
# Grouped-query decode over bf16 pages
# --------------------------------------------------------------------------------------------

def torch_gqa_reference(inp):
    q = inp.q.to(torch.float64)
    Kc = inp.k_cache.to(torch.float64)
    Vc = inp.v_cache.to(torch.float64)
    group = inp.Hq // inp.Hkv
    outs, lses = [], []
    for b in range(inp.B):
        S = int(inp.seq_lens[b])
        pages = inp.kv_page_indices[int(inp.kv_indptr[b]):int(inp.kv_indptr[b + 1])].long()
        K = Kc[pages].reshape(-1, inp.Hkv, inp.D)[:S]          # [S, Hkv, D]
        V = Vc[pages].reshape(-1, inp.Hkv, inp.D)[:S]
        K = K.repeat_interleave(group, dim=1).transpose(0, 1)    # [Hq, S, D]
        V = V.repeat_interleave(group, dim=1).transpose(0, 1)
        for t in range(inp.q_len):
            L = max(0, S - inp.q_len + t + 1)
            qr = q[b * inp.q_len + t]                             # [Hq, D]
            if L == 0:
                outs.append(torch.zeros(inp.Hq, inp.D, dtype=torch.float64))
                lses.append(torch.full((inp.Hq,), -math.inf, dtype=torch.float64))
                continue
            s = inp.scale * torch.einsum("hd,hsd->hs", qr, K[:, :L])
            outs.append(torch.einsum("hs,hsd->hd", torch.softmax(s, -1), V[:, :L]))
            lses.append(torch.logsumexp(s, -1) / LN2)
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


@pytest.mark.parametrize("shape", [
    dict(B=3, Hq=8, Hkv=2, D=16, page_size=4, lens=(9, 1, 16), num_pages=16, q_len=1),
    dict(B=2, Hq=16, Hkv=2, D=128, page_size=16, lens=(40, 17), num_pages=8, q_len=1),
    dict(B=2, Hq=4, Hkv=4, D=8, page_size=8, lens=(11, 3), num_pages=6, q_len=3),
])
def test_gqa_matches_torch_textbook(shape):
    lens = shape.pop("lens")
    inp = workloads.gqa_inputs(seq_lens=lens, seed=21, **shape)
    o, l = run_gqa(inp)
    ref_o, ref_l = torch_gqa_reference(inp)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(l))
    np.testing.assert_allclose(l[fin], ref_l[fin], rtol=1e-12)


def test_gqa_head_group_mapping():
    # query head h reads kv head h // (Hq / Hkv): zeroing one kv head's values zeroes exactly
    # that head group's outputs
    inp = workloads.gqa_inputs(B=1, Hq=8, Hkv=4, D=8, page_size=8, seq_lens=[10], num_pages=4,
                               seed=22)
    inp.v_cache[:, :, 2] = 0
    o, _ = run_gqa(inp)
    for h in range(8):
        assert np.all(o[h] == 0) == (h // 2 == 2)


def test_gqa_page_placement_invariance():
    inp = workloads.gqa_inputs(B=2, Hq=4, Hkv=2, D=8, page_size=8, seq_lens=[20, 9], num_pages=12,
                               seed=23)
    o, l = run_gqa(inp)
    g = torch.Generator().manual_seed(3)
    perm = torch.randperm(12, generator=g)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(12)
    inp.k_cache = inp.k_cache[perm].contiguous()
    inp.v_cache = inp.v_cache[perm].contiguous()
    inp.kv_page_indices = inv[inp.kv_page_indices.long()].to(torch.int32)
    o2, l2 = run_gqa(inp)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def with_skipped_keys(inp, seed, per_request):
    """The same requests with `per_request[b]` entries of -1 (skipped keys) inserted at seeded
    positions of each index list."""
    g = torch.Generator().manual_seed(seed)
    idx, indptr, lens = [], [0], []
    for b in range(inp.B):
        a, e = int(inp.kv_indptr[b]), int(inp.kv_indptr[b]) + int(inp.seq_lens[b])
        seg = list(inp.kv_indices[a:e].tolist())
        for _ in range(per_request[b]):
            seg.insert(int(torch.randint(0, len(seg) + 1, (1,), generator=g)), -1)
        idx += seg
        indptr.append(len(idx))
        lens.append(len(seg))
    return idx, indptr, lens


def test_skipped_keys_equal_their_removal():
    # skipped entries (negative slot ids; the top-k lists' has_invalid case) carry no weight:
    # every row equals the same request with those entries removed, bit for bit
    inp = small_mla(seed=41, q_len=1, lens=(5, 1, 17, 9), B=4)
    o, l = run_mla(inp)
    idx, indptr, lens = with_skipped_keys(inp, 7, [3, 2, 6, 0])
    inp.kv_indices = torch.tensor(idx, dtype=torch.int32)
    inp.kv_indptr = torch.tensor(indptr, dtype=torch.int32)
    inp.seq_lens = torch.tensor(lens, dtype=torch.int32)
    o2, l2 = run_mla(inp)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_all_skipped_request_is_empty():
    inp = small_mla(seed=42, q_len=2, lens=(5, 3, 4), B=3)
    a, e = int(inp.kv_indptr[1]), int(inp.kv_indptr[1]) + 3
    inp.kv_indices[a:e] = -1
    o, l = run_mla(inp)
    rows = [r for r in range(inp.rows) if r // (inp.q_len * inp.H) == 1]
    assert np.all(o[rows] == 0) and np.all(l[rows] == -np.inf)
    others = [r for r in range(inp.rows) if r not in rows]
    assert np.all(np.isfinite(l[others]))


def test_skipped_key_with_one_valid_key_closed_form():
    # [-1, j, -1]: the row sees one key, so o = v_j and lse2 = s_j / ln 2
    inp = small_mla(seed=43, q_len=1, lens=(3,), B=1, pool_rows=8)
    j = int(inp.kv_indices[1])
    inp.kv_indices[0] = -1
    inp.kv_indices[2] = -1
    o, l = run_mla(inp)
    pool = inp.pool.view(torch.float8_e4m3fn).to(torch.float64) * inp.kv_scale
    q = torch.cat([inp.q_lat, inp.q_pe], dim=-1).to(torch.float64)[0]   # [H, d_qk]
    s = inp.scale * (q @ pool[j])
    np.testing.assert_array_equal(o, pool[j, :inp.d_v].expand(inp.H, -1).numpy())
    np.testing.assert_allclose(l, (s / LN2).numpy(), rtol=1e-13)


def test_invalid_index_is_rejected():
    inp = small_mla(seed=30)
    inp.kv_indices[0] = inp.pool.shape[0]
    with pytest.raises(ValueError):
        run_mla(inp)


# ---- second cache (the sparse planner page's extra_topk: candidates in a second cache)

def run_mla2(inp, rows=None):
    return oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), u8(inp.pool),
                             inp.kv_indices.numpy(), inp.kv_indptr.numpy(), inp.seq_lens.numpy(),
                             B=inp.B, q_len=1, H=inp.H, d_v=inp.d_v, scale=inp.scale,
                             kv_scale=inp.kv_scale, rows=rows, pool2=u8(inp.pool2),
                             kv2_indices=inp.kv2_indices.numpy(), kv2_indptr=inp.kv2_indptr.numpy())


def two_cache_case(seed=21, d_qk=512, d_rope=64, d_v=448, lens=(9, 0, 30), extra=(5, 7, 0), skip=()):
    inp = workloads.mla_inputs(B=len(lens), q_len=1, H=3, seq_lens=list(lens), pool_rows=48,
                               d_qk=d_qk, d_rope=d_rope, d_v=d_v, seed=seed)
    return workloads.with_second_cache(inp, pool2_rows=20, extra_lens=list(extra), seed=seed + 50,
                                       skip=skip)


@pytest.mark.parametrize("shape", [dict(), dict(d_qk=576, d_rope=64, d_v=512, lens=(4, 17), extra=(12, 1))])
def test_two_caches_match_torch_textbook(shape):
    # textbook softmax attention over the main-cache keys followed by the second cache's, in
    # torch float64, against the oracle's two-cache entry
    inp = two_cache_case(**shape)
    q = torch.cat([inp.q_lat, inp.q_pe], dim=-1).to(torch.float64)
    pool = inp.pool.view(torch.float8_e4m3fn).to(torch.float64) * inp.kv_scale
    pool2 = inp.pool2.view(torch.float8_e4m3fn).to(torch.float64) * inp.kv_scale
    outs, lses = [], []
    for b in range(inp.B):
        i1 = inp.kv_indices[int(inp.kv_indptr[b]):int(inp.kv_indptr[b]) + int(inp.seq_lens[b])].long()
        i2 = inp.kv2_indices[int(inp.kv2_indptr[b]):int(inp.kv2_indptr[b + 1])].long()
        K = torch.cat([pool[i1], pool2[i2]])
        if K.shape[0] == 0:
            outs.append(torch.zeros(inp.H, inp.d_v, dtype=torch.float64))
            lses.append(torch.full((inp.H,), -math.inf, dtype=torch.float64))
            continue
        s = inp.scale * (q[b] @ K.T)
        outs.append(torch.softmax(s, dim=-1) @ K[:, :inp.d_v])
        lses.append(torch.logsumexp(s, dim=-1) / LN2)
    o, l = run_mla2(inp)
    np.testing.assert_allclose(o, torch.cat(outs).numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, torch.cat(lses).numpy(), rtol=1e-12, atol=1e-12)


def test_two_caches_equal_one_merged_pool():
    # the second cache appended to the pool, its slot ids shifted by the pool's rows and each
    # request's list extended by them, is the same attention, bit for bit
    inp = two_cache_case(lens=(9, 3, 30), extra=(5, 7, 2))
    n1 = inp.pool.shape[0]
    merged_pool = torch.cat([inp.pool, inp.pool2])
    idx, indptr, lens = [], [0], []
    for b in range(inp.B):
        a = inp.kv_indices[int(inp.kv_indptr[b]):int(inp.kv_indptr[b]) + int(inp.seq_lens[b])]
        e = inp.kv2_indices[int(inp.kv2_indptr[b]):int(inp.kv2_indptr[b + 1])] + n1
        idx.append(torch.cat([a, e]))
        lens.append(len(a) + len(e))
        indptr.append(indptr[-1] + lens[-1])
    o2, l2 = run_mla2(inp)
    o1, l1 = oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), u8(merged_pool),
                               torch.cat(idx).numpy(), np.array(indptr, np.int32),
                               np.array(lens, np.int32), B=inp.B, q_len=1, H=inp.H, d_v=inp.d_v,
                               scale=inp.scale, kv_scale=inp.kv_scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_second_cache_only_equals_single_cache_on_it():
    inp = two_cache_case(lens=(0, 0, 0), extra=(5, 7, 1))
    o2, l2 = run_mla2(inp)
    lens = (inp.kv2_indptr[1:] - inp.kv2_indptr[:-1]).numpy()
    o1, l1 = oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), u8(inp.pool2),
                               inp.kv2_indices.numpy(), inp.kv2_indptr.numpy(), lens,
                               B=inp.B, q_len=1, H=inp.H, d_v=inp.d_v, scale=inp.scale,
                               kv_scale=inp.kv_scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_skipped_second_cache_keys_equal_their_removal():
    inp = two_cache_case(lens=(9, 3, 30), extra=(5, 7, 2), skip=(1, 4, 6))
    o2, l2 = run_mla2(inp)
    keep = inp.kv2_indices >= 0
    counts = [int(keep[int(inp.kv2_indptr[b]):int(inp.kv2_indptr[b + 1])].sum()) for b in range(inp.B)]
    ptr = [0]
    for c in counts:
        ptr.append(ptr[-1] + c)
    import dataclasses
    inp_r = dataclasses.replace(inp, kv2_indices=inp.kv2_indices[keep],
                                kv2_indptr=torch.tensor(ptr, dtype=torch.int32))
    o1, l1 = run_mla2(inp_r)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_second_cache_rejections():
    inp = two_cache_case()
    bad = inp.kv2_indices.clone()
    bad[0] = 20   # the second pool has 20 rows
    with pytest.raises(ValueError):
        oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), u8(inp.pool), inp.kv_indices.numpy(),
                          inp.kv_indptr.numpy(), inp.seq_lens.numpy(), B=inp.B, q_len=1, H=inp.H,
                          d_v=inp.d_v, scale=inp.scale, kv_scale=inp.kv_scale, pool2=u8(inp.pool2),
                          kv2_indices=bad.numpy(), kv2_indptr=inp.kv2_indptr.numpy())


# --- bf16 cache: the same fused rows stored as bf16 (AITER issue "[Perf] pa_decode_sparse ...",
# closing paragraph, read as a bf16 copy of the cache dequantized by the same scale) -------------

def bf16_mla(seed=31, B=2, q_len=2, H=3, lens=(9, 4), d_qk=40, d_rope=8, d_v=32, pool_rows=24):
    return workloads.mla_inputs(B=B, q_len=q_len, H=H, seq_lens=list(lens), pool_rows=pool_rows,
                                d_qk=d_qk, d_rope=d_rope, d_v=d_v, seed=seed, kv_dtype="bf16")


def run_mla_bf16(inp, rows=None, kv_scale=None):
    return oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), bits16(inp.pool),
                             inp.kv_indices.numpy(), inp.kv_indptr.numpy(), inp.seq_lens.numpy(),
                             B=inp.B, q_len=inp.q_len, H=inp.H, d_v=inp.d_v, scale=inp.scale,
                             kv_scale=inp.kv_scale if kv_scale is None else kv_scale, rows=rows)


def torch_mla_reference_bf16(inp, kv_scale):
    """Textbook attention in torch CPU float64 over bf16 rows decoded by torch."""
    q = torch.cat([inp.q_lat, inp.q_pe], dim=-1).to(torch.float64)
    pool = inp.pool.to(torch.float64) * kv_scale
    outs, lses = [], []
    for b in range(inp.B):
        S = int(inp.seq_lens[b])
        idx = inp.kv_indices[int(inp.kv_indptr[b]):int(inp.kv_indptr[b]) + S].long()
        K = pool[idx]
        for t in range(inp.q_len):
            L = max(0, S - inp.q_len + t + 1)
            if L == 0:
                outs.append(torch.zeros(inp.H, inp.d_v, dtype=torch.float64))
                lses.append(torch.full((inp.H,), -math.inf, dtype=torch.float64))
                continue
            s = inp.scale * (q[b * inp.q_len + t] @ K[:L].T)
            outs.append(torch.softmax(s, dim=-1) @ K[:L, :inp.d_v])
            lses.append(torch.logsumexp(s, dim=-1) / LN2)
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


@pytest.mark.parametrize("shape,kv_scale", [
    (dict(), 1.0),
    (dict(), 0.375),
    (dict(B=2, q_len=1, H=16, lens=(64, 33), d_qk=576, d_rope=64, d_v=512, pool_rows=128), 1.0),
    (dict(B=3, q_len=4, H=2, lens=(9, 2, 0), d_qk=512, d_rope=64, d_v=448, pool_rows=16), 1.0),
])
def test_bf16_cache_matches_torch_textbook(shape, kv_scale):
    inp = bf16_mla(**shape)
    assert inp.pool.dtype == torch.bfloat16 and inp.kv_scale == 1.0
    o, lse2 = run_mla_bf16(inp, kv_scale=kv_scale)
    ref_o, ref_lse = torch_mla_reference_bf16(inp, kv_scale)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse2))
    np.testing.assert_allclose(lse2[fin], ref_lse[fin], rtol=1e-12, atol=1e-12)


def test_bf16_cache_holding_fp8_values_equals_fp8_cache():
    """Every e4m3 value is a bf16 value: a bf16 pool holding the fp8 pool's decoded values (times
    the scale, a power of two here) must reproduce the fp8 result bit for bit."""
    inp = small_mla(seed=12, B=2, q_len=2, H=3, lens=(11, 3), pool_rows=20)
    o8, l8 = run_mla(inp)
    vals = inp.pool.view(torch.float8_e4m3fn).to(torch.float32) * inp.kv_scale
    b16 = vals.to(torch.bfloat16)
    assert torch.equal(b16.to(torch.float32), vals)          # the conversion is exact
    o16, l16 = oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), bits16(b16),
                                 inp.kv_indices.numpy(), inp.kv_indptr.numpy(), inp.seq_lens.numpy(),
                                 B=inp.B, q_len=inp.q_len, H=inp.H, d_v=inp.d_v, scale=inp.scale,
                                 kv_scale=1.0)
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)


def test_bf16_cache_single_key_closed_form():
    inp = bf16_mla(seed=33, B=1, q_len=1, H=2, lens=(1,), pool_rows=3)
    o, l = run_mla_bf16(inp)
    k = inp.pool[int(inp.kv_indices[0])].to(torch.float64)
    s = inp.scale * (torch.cat([inp.q_lat, inp.q_pe], -1).to(torch.float64)[0] @ k)
    for h in range(2):
        assert np.array_equal(o[h], k[:inp.d_v].numpy())
        assert l[h] == pytest.approx(float(s[h]) / LN2, rel=1e-14, abs=1e-14)


def test_bf16_cache_row_stride_uses_two_bytes():
    """A wrong row stride (one byte per element) would read row k's second half as row 2k+1:
    attending only the last pool row must return that row's values."""
    inp = bf16_mla(seed=34, B=1, q_len=1, H=1, lens=(1,), pool_rows=9)
    inp.kv_indices[0] = 8
    o, _ = run_mla_bf16(inp)
    assert np.array_equal(o[0], inp.pool[8, :inp.d_v].to(torch.float64).numpy())


def test_bf16_cache_skipped_keys_equal_their_removal():
    inp = bf16_mla(seed=35, B=1, q_len=1, H=3, lens=(12,), pool_rows=12)
    o_full, l_full = run_mla_bf16(inp)
    keep = [0, 1, 2, 5, 6, 7, 8, 9, 10, 11]
    skipped = inp.kv_indices.clone()
    skipped[3], skipped[4] = -1, -1
    o_s, l_s = oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), bits16(inp.pool), skipped.numpy(),
                                 inp.kv_indptr.numpy(), inp.seq_lens.numpy(), B=1, q_len=1, H=3,
                                 d_v=inp.d_v, scale=inp.scale, kv_scale=1.0)
    sub = inp.kv_indices[keep]
    o_r, l_r = oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), bits16(inp.pool), sub.numpy(),
                                 np.array([0, len(keep)], np.int32), np.array([len(keep)], np.int32),
                                 B=1, q_len=1, H=3, d_v=inp.d_v, scale=inp.scale, kv_scale=1.0)
    np.testing.assert_allclose(o_s, o_r, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l_s, l_r, rtol=1e-13, atol=1e-13)
    assert not np.allclose(o_s, o_full)


def bf16_two_cache_case(seed=41, lens=(9, 0, 30), extra=(5, 7, 0)):
    inp = workloads.mla_inputs(B=len(lens), q_len=1, H=3, seq_lens=list(lens), pool_rows=48,
                               d_qk=512, d_rope=64, d_v=448, seed=seed, kv_dtype="bf16")
    return workloads.with_second_cache(inp, pool2_rows=20, extra_lens=list(extra), seed=seed + 50)


def run_mla2_bf16(inp):
    return oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), bits16(inp.pool),
                             inp.kv_indices.numpy(), inp.kv_indptr.numpy(), inp.seq_lens.numpy(),
                             B=inp.B, q_len=1, H=inp.H, d_v=inp.d_v, scale=inp.scale,
                             kv_scale=inp.kv_scale, pool2=bits16(inp.pool2),
                             kv2_indices=inp.kv2_indices.numpy(), kv2_indptr=inp.kv2_indptr.numpy())


def test_bf16_two_caches_match_torch_textbook():
    inp = bf16_two_cache_case()
    assert inp.pool2.dtype == torch.bfloat16
    q = torch.cat([inp.q_lat, inp.q_pe], dim=-1).to(torch.float64)
    pool, pool2 = inp.pool.to(torch.float64), inp.pool2.to(torch.float64)
    outs, lses = [], []
    for b in range(inp.B):
        i1 = inp.kv_indices[int(inp.kv_indptr[b]):int(inp.kv_indptr[b]) + int(inp.seq_lens[b])].long()
        i2 = inp.kv2_indices[int(inp.kv2_indptr[b]):int(inp.kv2_indptr[b + 1])].long()
        K = torch.cat([pool[i1], pool2[i2]])
        if K.shape[0] == 0:
            outs.append(torch.zeros(inp.H, inp.d_v, dtype=torch.float64))
            lses.append(torch.full((inp.H,), -math.inf, dtype=torch.float64))
            continue
        s = inp.scale * (q[b] @ K.T)
        outs.append(torch.softmax(s, dim=-1) @ K[:, :inp.d_v])
        lses.append(torch.logsumexp(s, dim=-1) / LN2)
    o, l = run_mla2_bf16(inp)
    np.testing.assert_allclose(o, torch.cat(outs).numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, torch.cat(lses).numpy(), rtol=1e-12, atol=1e-12)


def test_bf16_two_caches_equal_one_merged_pool():
    inp = bf16_two_cache_case(lens=(9, 3, 30), extra=(5, 7, 2))
    n1 = inp.pool.shape[0]
    merged = torch.cat([inp.pool, inp.pool2])
    idx, indptr, lens = [], [0], []
    for b in range(inp.B):
        a = inp.kv_indices[int(inp.kv_indptr[b]):int(inp.kv_indptr[b]) + int(inp.seq_lens[b])]
        e = inp.kv2_indices[int(inp.kv2_indptr[b]):int(inp.kv2_indptr[b + 1])] + n1
        idx.append(torch.cat([a, e]))
        lens.append(len(a) + len(e))
        indptr.append(indptr[-1] + lens[-1])
    o2, l2 = run_mla2_bf16(inp)
    o1, l1 = oracle.mla_decode(bits16(inp.q_lat), bits16(inp.q_pe), bits16(merged),
                               torch.cat(idx).numpy(), np.array(indptr, np.int32),
                               np.array(lens, np.int32), B=inp.B, q_len=1, H=inp.H, d_v=inp.d_v,
                               scale=inp.scale, kv_scale=inp.kv_scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
