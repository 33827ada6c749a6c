"""Seeded synthetic inputs for split-KV decode, shaped like the pages' workloads.

This module only draws random numbers and builds index lists: it holds none of the attention,
planner or merge arithmetic, so both the GPU path and the CPU oracle can be fed from it.

Shapes follow the workloads the pages describe:

* absorbed MLA decode (moonmath-amd README, "MLA decode"): bf16 ``q_lat [B*q_len, H, 512]`` and
  ``q_pe [B*q_len, H, 64]`` drawn N(0,1); one fused fp8 e4m3 row of 576 bytes per token, stored as
  N(0,1) / kv_scale with kv_scale = 1/32; page_size 1, so ``kv_indices`` is a flat slot list (a
  seeded permutation: any permutation is legal); softmax scale 576^-0.5;
* sparse top-k MLA decode (AITER issue on pa_decode_sparse, "Measurements"): 64 heads, rows of
  512 fp8 bytes (448 NoPE + 64 RoPE) in a 262144-token cache, 2048 indices per query drawn
  without replacement;
* the bf16 cache (the AITER issue's closing paragraph): the same fused rows stored as bf16 values
  N(0,1) with kv_scale 1;
* grouped-query decode over bf16 pages (moonmath-amd README, gfx950 "forward_paged"): caches
  ``[pages, 16, kv_heads, 128]``, ``kv_indptr`` counting pages per sequence and
  ``kv_page_indices`` a random placement of pages in the pool.

Seeds: workload k uses base seed 1000*k; tensor offsets +1 q_lat (or q), +2 q_pe, +3 KV,
+4 indices, +5 lengths, +6 page placement.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import torch

KV_SCALE = 1.0 / 32.0


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, seed, device, dtype=torch.float32):
    return torch.randn(shape, generator=_gen(device, seed), device=device, dtype=dtype)


def fp8_e4m3fn_bytes(x: torch.Tensor) -> torch.Tensor:
    """Encode with torch's float8_e4m3fn cast and return the raw bytes (uint8)."""
    b = x.to(torch.float8_e4m3fn).view(torch.uint8)
    nan = (b & 0x7F) == 0x7F
    if bool(nan.any()):
        raise ValueError("fp8 encode produced NaN bytes (value above the e4m3fn range)")
    return b


def _fp8_pool(rows, width, seed, device, chunk_rows=1 << 20):
    """[rows, width] fp8 bytes of N(0,1)/KV_SCALE, drawn in chunks to bound temporaries."""
    out = torch.empty((rows, width), dtype=torch.uint8, device=device)
    g = _gen(device, seed)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.randn((r1 - r0, width), generator=g, device=device, dtype=torch.float32)
        out[r0:r1] = fp8_e4m3fn_bytes(x / KV_SCALE)
    return out


def _bf16_pool(rows, width, seed, device, chunk_rows=1 << 20):
    """[rows, width] bf16 values N(0,1) (the bf16-cache variant: no quantization, kv_scale 1)."""
    out = torch.empty((rows, width), dtype=torch.bfloat16, device=device)
    g = _gen(device, seed)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0, width), generator=g, device=device, dtype=torch.float32)
    return out


@dataclasses.dataclass
class MlaInputs:
    B: int
    q_len: int
    H: int
    d_qk: int
    d_rope: int
    d_v: int
    q_lat: torch.Tensor        # bf16 [B*q_len, H, d_qk - d_rope] (may be a strided view)
    q_pe: torch.Tensor         # bf16 [B*q_len, H, d_rope] (may be a strided view)
    pool: torch.Tensor         # uint8 [N, d_qk] fp8 e4m3fn bytes, or bf16 [N, d_qk] (bf16 cache)
    kv_indices: torch.Tensor   # int32 [sum of keys]
    kv_indptr: torch.Tensor    # int32 [B+1]
    seq_lens: torch.Tensor     # int32 [B]
    max_num_keys: int
    scale: float
    kv_scale: float = KV_SCALE
    name: str = ""
    # a second cache (sparse top-k with extra candidates, q_len 1): rows of the same format;
    # request b also attends pool2 rows kv2_indices[kv2_indptr[b]:kv2_indptr[b+1]]
    pool2: Optional[torch.Tensor] = None
    kv2_indices: Optional[torch.Tensor] = None
    kv2_indptr: Optional[torch.Tensor] = None

    @property
    def rows(self) -> int:
        return self.B * self.q_len * self.H

    @property
    def kv_bf16(self) -> bool:
        return self.pool.dtype == torch.bfloat16

    @property
    def kv_bytes(self) -> int:
        """KV payload bytes one decode reads: every key of every request once (576 or 512
        elements of 1 byte, or 2 bytes for a bf16 cache)."""
        n = int(self.seq_lens.sum().item())
        if self.kv2_indices is not None:
            n += int(self.kv2_indices.numel())
        return n * self.d_qk * self.pool.element_size()


@dataclasses.dataclass
class GqaInputs:
    B: int
    q_len: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    q: torch.Tensor            # bf16 [B*q_len, Hq, D]
    k_cache: torch.Tensor      # bf16 [num_pages, page_size, Hkv, D]
    v_cache: torch.Tensor
    kv_page_indices: torch.Tensor  # int32
    kv_indptr: torch.Tensor    # int32 [B+1] (pages)
    seq_lens: torch.Tensor     # int32 [B] (tokens)
    max_num_keys: int
    scale: float
    name: str = ""

    @property
    def rows(self) -> int:
        return self.B * self.q_len * self.Hq

    @property
    def kv_bytes(self) -> int:
        """K and V bytes one decode reads: per token, per kv head, D bf16 values of each."""
        return int(self.seq_lens.sum().item()) * self.Hkv * self.D * 2 * 2


def mla_inputs(*, B: int, q_len: int, H: int, seq_lens: Sequence[int], pool_rows: Optional[int] = None,
               d_qk: int = 576, d_rope: int = 64, d_v: int = 512, seed: int = 0,
               device="cpu", shuffle: bool = True, fused_q: bool = False, name: str = "",
               kv_dtype: str = "fp8") -> MlaInputs:
    """Absorbed-MLA decode inputs; request b owns keys kv_indices[kv_indptr[b]:kv_indptr[b+1]].

    fused_q=True draws one q [B*q_len, H, d_qk] and exposes q_lat / q_pe as views of it (the
    sparse top-k workload's single 512-wide query).  kv_dtype="bf16": the pool holds bf16
    N(0,1) rows with kv_scale 1 (the bf16-cache variant)."""
    lens = [int(x) for x in seq_lens]
    assert len(lens) == B
    total = sum(lens)
    N = pool_rows if pool_rows is not None else max(total, 1)
    d_lat = d_qk - d_rope
    if fused_q:
        q = _randn((B * q_len, H, d_qk), seed + 1, device, torch.bfloat16)
        q_lat, q_pe = q[..., :d_lat], q[..., d_lat:]
    else:
        q_lat = _randn((B * q_len, H, d_lat), seed + 1, device, torch.bfloat16)
        q_pe = _randn((B * q_len, H, d_rope), seed + 2, device, torch.bfloat16)
    pool = _bf16_pool(N, d_qk, seed + 3, device) if kv_dtype == "bf16" else _fp8_pool(N, d_qk, seed + 3, device)
    if shuffle:
        if total <= N:
            idx = torch.randperm(N, generator=_gen(device, seed + 4), device=device)[:total]
        else:
            idx = torch.randint(0, N, (total,), generator=_gen(device, seed + 4), device=device)
    else:
        idx = torch.arange(total, device=device) % N
    kv_indices = idx.to(torch.int32)
    indptr = [0]
    for L in lens:
        indptr.append(indptr[-1] + L)
    kv_indptr = torch.tensor(indptr, dtype=torch.int32, device=device)
    sl = torch.tensor(lens, dtype=torch.int32, device=device)
    return MlaInputs(B=B, q_len=q_len, H=H, d_qk=d_qk, d_rope=d_rope, d_v=d_v, q_lat=q_lat,
                     q_pe=q_pe, pool=pool, kv_indices=kv_indices, kv_indptr=kv_indptr,
                     seq_lens=sl, max_num_keys=max(lens) if lens else 0,
                     scale=float(d_qk) ** -0.5, kv_scale=1.0 if kv_dtype == "bf16" else KV_SCALE,
                     name=name)


def sparse_mla_inputs(*, num_queries: int, topk: int = 2048, cache_rows: int = 262144, H: int = 64,
                      seed: int = 4000, device="cpu", name: str = "", invalid_frac: float = 0.0,
                      all_invalid: Sequence[int] = (), extra_topk: int = 0,
                      extra_rows: int = 65536, kv_dtype: str = "fp8") -> MlaInputs:
    """Sparse top-k MLA decode: each query is its own request whose keys are `topk` cache rows
    drawn without replacement; rows are 512 fp8 bytes (448 NoPE + 64 RoPE), value = NoPE part.
    invalid_frac: that fraction of the index entries (seeded positions) is -1, a skipped key;
    all_invalid: queries whose whole list is -1.  extra_topk > 0: a second cache of extra_rows
    rows of the same format, from which each query draws extra_topk more candidates.
    kv_dtype="bf16": bf16 caches of N(0,1) rows with kv_scale 1."""
    assert kv_dtype in ("fp8", "bf16")
    nq = num_queries
    q = _randn((nq, H, 512), seed + 1, device, torch.bfloat16)
    if kv_dtype == "bf16":
        pool = _bf16_pool(cache_rows, 512, seed + 3, device)
    else:
        pool = _fp8_pool(cache_rows, 512, seed + 3, device)
    g = _gen(device, seed + 4)
    rows = []
    for _ in range(nq):
        rows.append(torch.randperm(cache_rows, generator=g, device=device)[:topk])
    kv_indices = torch.cat(rows).to(torch.int32) if nq else torch.empty(0, dtype=torch.int32, device=device)
    if invalid_frac > 0 and nq:
        drop = torch.rand(kv_indices.shape, generator=_gen(device, seed + 5), device=device) < invalid_frac
        kv_indices[drop] = -1
    for qi in all_invalid:
        kv_indices[qi * topk:(qi + 1) * topk] = -1
    kv_indptr = (torch.arange(nq + 1, device=device, dtype=torch.int32) * topk)
    sl = torch.full((nq,), topk, dtype=torch.int32, device=device)
    pool2 = kv2_indices = kv2_indptr = None
    if extra_topk > 0:
        pool2 = (_bf16_pool if kv_dtype == "bf16" else _fp8_pool)(extra_rows, 512, seed + 7, device)
        g2 = _gen(device, seed + 8)
        kv2_indices = torch.cat([torch.randperm(extra_rows, generator=g2, device=device)[:extra_topk]
                                 for _ in range(nq)]).to(torch.int32)
        kv2_indptr = torch.arange(nq + 1, device=device, dtype=torch.int32) * extra_topk
    return MlaInputs(B=nq, q_len=1, H=H, d_qk=512, d_rope=64, d_v=448, q_lat=q[..., :448],
                     q_pe=q[..., 448:], pool=pool, kv_indices=kv_indices, kv_indptr=kv_indptr,
                     seq_lens=sl, max_num_keys=topk + extra_topk, scale=512.0 ** -0.5, name=name,
                     kv_scale=1.0 if kv_dtype == "bf16" else KV_SCALE,
                     pool2=pool2, kv2_indices=kv2_indices, kv2_indptr=kv2_indptr)


def with_second_cache(inp: MlaInputs, *, pool2_rows: int, extra_lens: Sequence[int], seed: int,
                      skip: Sequence[int] = ()) -> MlaInputs:
    """The same q_len-1 requests with a second cache of pool2_rows rows (the pool's format: fp8
    N(0,1)*32 bytes, or bf16 N(0,1) for a bf16 pool) from
    which request b draws extra_lens[b] candidates (with replacement allowed across requests);
    `skip` lists flat positions of the second-cache list set to -1 (skipped keys)."""
    assert inp.q_len == 1 and len(extra_lens) == inp.B
    device = inp.pool.device
    if inp.pool.dtype == torch.bfloat16:
        pool2 = _bf16_pool(pool2_rows, inp.d_qk, seed, device)
    else:
        pool2 = _fp8_pool(pool2_rows, inp.d_qk, seed, device)
    g = _gen("cpu", seed + 1)
    idx = torch.cat([torch.randperm(pool2_rows, generator=g)[:n] for n in extra_lens]).to(torch.int32)
    for k in skip:
        idx[k] = -1
    indptr = [0]
    for n in extra_lens:
        indptr.append(indptr[-1] + int(n))
    return dataclasses.replace(inp, pool2=pool2, kv2_indices=idx.to(device),
                               kv2_indptr=torch.tensor(indptr, dtype=torch.int32, device=device),
                               max_num_keys=int(inp.max_num_keys) + max(extra_lens))


def gqa_inputs(*, B: int, Hq: int, Hkv: int, D: int = 128, page_size: int = 16,
               seq_lens: Sequence[int], num_pages: int, q_len: int = 1, seed: int = 3000,
               device="cpu", name: str = "") -> GqaInputs:
    lens = [int(x) for x in seq_lens]
    assert len(lens) == B
    pages_per = [(L + page_size - 1) // page_size for L in lens]
    total_pages = sum(pages_per)
    assert total_pages <= num_pages, (total_pages, num_pages)
    q = _randn((B * q_len, Hq, D), seed + 1, device, torch.bfloat16)
    k_cache = _randn((num_pages, page_size, Hkv, D), seed + 3, device, torch.bfloat16)
    v_cache = _randn((num_pages, page_size, Hkv, D), seed + 7, device, torch.bfloat16)
    placement = torch.randperm(num_pages, generator=_gen(device, seed + 6), device=device)[:total_pages]
    indptr = [0]
    for n in pages_per:
        indptr.append(indptr[-1] + n)
    return GqaInputs(B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=D, page_size=page_size, q=q,
                     k_cache=k_cache, v_cache=v_cache,
                     kv_page_indices=placement.to(torch.int32),
                     kv_indptr=torch.tensor(indptr, dtype=torch.int32, device=device),
                     seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
                     max_num_keys=max(lens) if lens else 0, scale=float(D) ** -0.5, name=name)


def uniform_lengths(B: int, lo: int, hi: int, seed: int) -> list:
    """B lengths uniform on the integers [lo, hi] (seeded, CPU generator so the draw is the same
    on every device)."""
    g = _gen("cpu", seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=g)]


# --------------------------------------------------------------------------------------------
# The five workloads, at full size
# --------------------------------------------------------------------------------------------

def mla_tiny(device="cpu"):
    """B=1, q_len=1, H=16, 4096 shuffled keys (run with np in {1, 4, 16})."""
    return mla_inputs(B=1, q_len=1, H=16, seq_lens=[4096], pool_rows=4096, seed=0,
                      device=device, name="mla_tiny_b1_h16_s4096")


def mla_b2_s65536(device="cpu"):
    """H=64, B=2, 65536 keys each, shuffled slots in a 131072-row pool."""
    return mla_inputs(B=2, q_len=1, H=64, seq_lens=[65536] * 2, pool_rows=131072, seed=1000,
                      device=device, name="mla_h64_b2_s65536")


def mla_long(B: int, q_len: int = 1, device="cpu"):
    """H=64, B in {8, 16}, 131072 keys each; q_len=4 is the speculative-verify window."""
    return mla_inputs(B=B, q_len=q_len, H=64, seq_lens=[131072] * B, pool_rows=B * 131072,
                      seed=2000, device=device, name="mla_h64_b%d_s131072_q%d" % (B, q_len))


def mla_skewed(device="cpu"):
    """A skewed serving batch: H=64, one request of 131072 keys among 31 of 2048 (the same
    fp8 pool as the long-context workloads)."""
    lens = [131072] + [2048] * 31
    return mla_inputs(B=32, q_len=1, H=64, seq_lens=lens, pool_rows=sum(lens), seed=2100,
                      device=device, name="mla_h64_b32_skewed_1x131072_31x2048")


GQA_LEN_SEED = 3000 + 5


def gqa_paged(device="cpu"):
    """B=32, 64 query heads over 8 kv heads, D=128, page 16, lengths U[1024, 32768], pages
    placed at random in a pool of 2^21 tokens (131072 pages)."""
    lens = uniform_lengths(32, 1024, 32768, GQA_LEN_SEED)
    return gqa_inputs(B=32, Hq=64, Hkv=8, D=128, page_size=16, seq_lens=lens, num_pages=131072,
                      seed=3000, device=device, name="gqa_b32_hq64_hkv8_d128_p16")


def gqa_mqa(device="cpu"):
    """The paged GQA batch (same lengths and pool) with all 64 query heads on one kv head: the
    split CTA then carries 64 query rows."""
    lens = uniform_lengths(32, 1024, 32768, GQA_LEN_SEED)
    return gqa_inputs(B=32, Hq=64, Hkv=1, D=128, page_size=16, seq_lens=lens, num_pages=131072,
                      seed=3000, device=device, name="gqa_b32_hq64_hkv1_d128_p16")


SPARSE_QUERY_COUNTS = (24, 32, 34, 64, 128, 256)


def sparse_topk(num_queries: int, device="cpu", kv_dtype: str = "fp8"):
    tag = "" if kv_dtype == "fp8" else "_bf16"
    return sparse_mla_inputs(num_queries=num_queries, seed=4000, device=device, kv_dtype=kv_dtype,
                             name="sparse_mla_h64_topk2048_nq%d%s" % (num_queries, tag))


def mla_long_bf16(B: int, q_len: int = 1, device="cpu"):
    """The H=64 long-context workload over a bf16 cache (131072 keys per request, 1152-byte
    rows, kv_scale 1)."""
    return mla_inputs(B=B, q_len=q_len, H=64, seq_lens=[131072] * B, pool_rows=B * 131072,
                      seed=2200, device=device, kv_dtype="bf16",
                      name="mla_h64_b%d_s131072_q%d_bf16" % (B, q_len))


# --------------------------------------------------------------------------------------------
# Wide-dynamic-range variants of an MLA input (numerics stress cases).  Each returns a new
# MlaInputs with the same requests and slot lists; only values change.
# --------------------------------------------------------------------------------------------

def gqa_scaled(inp: GqaInputs, q_mul: float = 1.0, v_mul: float = 1.0) -> GqaInputs:
    """Queries and values multiplied by powers of two (exact in bf16): larger queries spread the
    scores over more octaves, larger values raise the output's magnitude."""
    return dataclasses.replace(inp, q=(inp.q.float() * q_mul).to(torch.bfloat16),
                               v_cache=(inp.v_cache.float() * v_mul).to(torch.bfloat16))


def gqa_dominant_keys(inp: GqaInputs, mul: float = 8.0, every: int = 16, seed: int = 0) -> GqaInputs:
    """K rows of one seeded token slot in every `every` slots of each page multiplied by `mul`
    (all kv heads), so that about one key per 16-token tile dominates its rows' softmax."""
    g = _gen("cpu", seed)
    k = inp.k_cache.clone()
    ps = inp.page_size
    for start in range(0, ps, every):
        width = min(every, ps - start)
        pick = start + int(torch.randint(0, width, (1,), generator=g))
        k[:, pick] = (k[:, pick].float() * mul).to(torch.bfloat16)
    return dataclasses.replace(inp, k_cache=k)


def scaled_queries(inp: MlaInputs, mul: float) -> MlaInputs:
    """q_lat and q_pe multiplied by `mul` (a power of two keeps the bf16 values exact), so that
    scores spread over many octaves within and across key tiles."""
    return dataclasses.replace(inp, q_lat=(inp.q_lat.float() * mul).to(torch.bfloat16),
                               q_pe=(inp.q_pe.float() * mul).to(torch.bfloat16))


def wide_range_queries(inp: MlaInputs, octaves: float = 20.0, mul: float = 1.0,
                       seed: int = 0) -> MlaInputs:
    """Query elements of random sign whose magnitudes are log-uniform over `octaves` binary
    octaves below `mul`: every row holds values from about 2^-octaves to 1 of its maximum."""
    dev = inp.q_lat.device
    g = _gen("cpu", seed)

    def draw(shape):
        mag = torch.exp2(-octaves * torch.rand(shape, generator=g, dtype=torch.float64))
        sgn = torch.where(torch.rand(shape, generator=g) < 0.5, -1.0, 1.0).double()
        return (sgn * mag * mul).to(torch.bfloat16).to(dev)

    return dataclasses.replace(inp, q_lat=draw(tuple(inp.q_lat.shape)),
                               q_pe=draw(tuple(inp.q_pe.shape)))


# e4m3fn codes at the edges of the format: the largest magnitudes (448, 416, 384, 352) and the
# subnormals (m * 2^-9, m = 1..7), both signs.
E4M3FN_LARGE_CODES = (0x7E, 0x7D, 0x7C, 0x7B, 0xFE, 0xFD, 0xFC, 0xFB)
E4M3FN_SUBNORMAL_CODES = tuple(range(0x01, 0x08)) + tuple(range(0x81, 0x88))


def extreme_pool(inp: MlaInputs, frac_large: float = 0.1, frac_subnormal: float = 0.1,
                 seed: int = 0) -> MlaInputs:
    """A copy of the pool in which a seeded fraction of the bytes is replaced by the largest
    e4m3fn magnitudes and another fraction by subnormal codes."""
    g = _gen("cpu", seed)
    pool = inp.pool.cpu().clone()
    r = torch.rand(pool.shape, generator=g)
    large = torch.tensor(E4M3FN_LARGE_CODES, dtype=torch.uint8)
    sub = torch.tensor(E4M3FN_SUBNORMAL_CODES, dtype=torch.uint8)
    m_large = r < frac_large
    m_sub = r >= 1.0 - frac_subnormal
    pool[m_large] = large[torch.randint(0, len(large), (int(m_large.sum()),), generator=g)]
    pool[m_sub] = sub[torch.randint(0, len(sub), (int(m_sub.sum()),), generator=g)]
    return dataclasses.replace(inp, pool=pool.to(inp.pool.device))


def extreme_bf16_pool(inp: MlaInputs, frac_large: float = 0.1, frac_small: float = 0.1,
                      seed: int = 0) -> MlaInputs:
    """A copy of a bf16 pool in which a seeded fraction of the elements is replaced by large
    magnitudes (log-uniform in [8, 16), the top of the fp8 cache's dequantized range) and another
    by tiny ones (log-uniform in [2^-24, 2^-14), fp16's subnormal range), both signs."""
    g = _gen("cpu", seed)
    pool = inp.pool.cpu().float().clone()
    r = torch.rand(pool.shape, generator=g)
    sgn = torch.where(torch.rand(pool.shape, generator=g) < 0.5, -1.0, 1.0)
    u = torch.rand(pool.shape, generator=g)
    large = sgn * torch.exp2(3.0 + u)
    small = sgn * torch.exp2(-24.0 + 10.0 * u)
    pool = torch.where(r < frac_large, large, pool)
    pool = torch.where(r >= 1.0 - frac_small, small, pool)
    return dataclasses.replace(inp, pool=pool.to(torch.bfloat16).to(inp.pool.device))


def dominant_keys(inp: MlaInputs, seed: int = 0, noise: float = 0.05, block: int = 64) -> MlaInputs:
    """Queries that share one direction u (per-head noise of relative size `noise`), and in every
    run of `block` consecutive positions of each request's slot list one key whose pool row is u
    encoded in fp8 at a seeded amplitude (row maximum 100..440 before the kv scale).  Each such
    key dominates its block for every head, and the blocks' maxima differ by many octaves."""
    dev = inp.pool.device
    g = _gen("cpu", seed)
    d_lat = inp.q_lat.shape[-1]
    d_qk = inp.pool.shape[1]
    u = torch.randn((d_qk,), generator=g, dtype=torch.float64)
    ntok, H = inp.q_lat.shape[0], inp.q_lat.shape[1]
    q = u.view(1, 1, -1) * (1.0 + noise * torch.randn((ntok, H, d_qk), generator=g, dtype=torch.float64))
    q = q.to(torch.bfloat16)
    pool = inp.pool.cpu().clone()
    idx = inp.kv_indices.cpu()
    indptr = inp.kv_indptr.cpu()
    lens = inp.seq_lens.cpu()
    unit = u / u.abs().max()
    for b in range(inp.B):
        a, n = int(indptr[b]), int(lens[b])
        for s0 in range(0, n, block):
            j = s0 + int(torch.randint(0, min(block, n - s0), (1,), generator=g))
            slot = int(idx[a + j])
            if slot < 0:
                continue
            amp = 100.0 + 340.0 * float(torch.rand((1,), generator=g))
            if pool.dtype == torch.bfloat16:   # the same stored magnitude after the kv scale
                pool[slot] = (unit * amp * KV_SCALE).to(torch.bfloat16)
            else:
                pool[slot] = fp8_e4m3fn_bytes((unit * amp).float())
    return dataclasses.replace(inp, q_lat=q[..., :d_lat].contiguous().to(dev),
                               q_pe=q[..., d_lat:].contiguous().to(dev), pool=pool.to(dev))


def sorted_slots(inp: MlaInputs, how: str) -> MlaInputs:
    """The same keys with each request's slot list reordered: "request" sorts it ascending,
    "contiguous" gives request b the pool rows kv_indptr[b] .. kv_indptr[b + 1] - 1 in order (a
    plain arange, with the pool unchanged)."""
    idx = inp.kv_indices.cpu().clone()
    indptr = inp.kv_indptr.cpu()
    if how == "contiguous":
        idx = torch.arange(idx.numel(), dtype=torch.int32) % inp.pool.shape[0]
    elif how == "request":
        for b in range(inp.B):
            a, e = int(indptr[b]), int(indptr[b + 1])
            idx[a:e] = torch.sort(idx[a:e]).values
    else:
        raise ValueError(how)
    return dataclasses.replace(inp, kv_indices=idx.to(torch.int32).to(inp.kv_indices.device))
