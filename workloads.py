"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no normalisation, lookup, attention or merge), so
both the GPU path's tests and the CPU oracle may consume what it produces.

Workload shapes follow the decode settings described by the pages (top-k
sparse MLA decode over a paged latent KV cache, DeepSeek-V3.2-like shapes):
bf16 rows of 576 values (512 latent + 64 rope), one latent KV head shared by
all query heads, page size 64, random page tables over a shared pool, top-k
2048 plus a 128-token local window and 4 sink tokens.  No trained weights or
indexer traces exist here, so values are N(0, 1) and the top-k ids are
uniform draws (or clustered runs) with the stated statistics.
"""

from dataclasses import dataclass, field
import math

import numpy as np

D_QK = 576
D_V = 512


def bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even) and return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def normal_bf16(rng, shape):
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@dataclass
class DecodeCase:
    """One batch of decode inputs (host numpy arrays, bf16 as uint16 bits)."""
    name: str
    q_bits: np.ndarray            # [T, H, 576] uint16
    topk: np.ndarray              # [T, top_k] int32, -1 padded
    req_id: np.ndarray            # [T] int32
    q_pos: np.ndarray             # [T] int32
    block_table: np.ndarray       # [R, max_blocks] int32, -1 = unmapped
    page_size: int
    window: int
    num_sinks: int
    cap: int
    kv_rows: int                  # rows in the latent KV pool
    pool_seed: int                # seed of the pool values (see pool_bits / pool_torch)
    scale: float = 1.0 / math.sqrt(D_QK)
    extra: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.q_bits.shape[0]

    @property
    def H(self):
        return self.q_bits.shape[1]

    @property
    def top_k(self):
        return self.topk.shape[1]


def pool_bits(rows, seed, chunk_rows=1 << 16):
    """Latent KV pool [rows, 576] as bf16 bits, generated on the host (numpy)."""
    out = np.empty((rows, D_QK), dtype=np.uint16)
    ss = np.random.SeedSequence(seed)
    for c, child in enumerate(ss.spawn(-(-rows // chunk_rows))):
        lo = c * chunk_rows
        hi = min(rows, lo + chunk_rows)
        out[lo:hi] = normal_bf16(np.random.default_rng(child), (hi - lo, D_QK))
    return out


def pool_torch(rows, seed, device, chunk_rows=1 << 18):
    """Latent KV pool [rows, 576] bf16 generated directly in device memory.

    Uses torch's seeded generator on the device (values N(0, 1), rounded to
    bf16 by torch's conversion).  For pools too large to build on the host.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    pool = torch.empty((rows, D_QK), dtype=torch.bfloat16, device=device)
    for lo in range(0, rows, chunk_rows):
        hi = min(rows, lo + chunk_rows)
        pool[lo:hi] = torch.randn((hi - lo, D_QK), generator=g, device=device, dtype=torch.float32)
    return pool


def _uniform_without_replacement(rng, n, k):
    return rng.choice(n, size=k, replace=False).astype(np.int32)


def tiny_case(seed=1000):
    """One request, context 256, page 64 (4 of 16 physical pages), 16 heads.

    32 dynamic ids: 28 distinct uniform draws plus 4 forced duplicates of
    members, shuffled; window 8, sinks 4.
    """
    rng = np.random.default_rng(seed)
    ctx, P, H = 256, 64, 16
    table = rng.permutation(16)[: ctx // P].astype(np.int32)[None, :]
    distinct = rng.choice(ctx, size=28, replace=False)
    dups = rng.choice(distinct, size=4, replace=False)
    topk = rng.permutation(np.concatenate([distinct, dups])).astype(np.int32)[None, :]
    q = normal_bf16(rng, (1, H, D_QK))
    return DecodeCase("tiny", q, topk, np.zeros(1, np.int32), np.full(1, ctx - 1, np.int32),
                      table, P, 8, 4, 32 + 8 + 4, 16 * P, pool_seed=seed + 1)


def deepseek_case(seed=2000, batch=32, ctx=32768, heads=128, top_k=2048, window=128,
                  sinks=4, page_size=64, pool_pages=None, variant=0):
    """Batch of decode tokens, one per request, shaped like DeepSeek-V3.2 MLA.

    Page tables are disjoint random page sets from one shared pool; the top-k
    ids are uniform without replacement over the causal range.  `variant`
    changes only the top-k draws (same pool, tables and queries), so a
    benchmark can rotate candidate sets whose union exceeds on-chip caches.
    """
    rng = np.random.default_rng(seed)
    pages_per_req = -(-ctx // page_size)
    if pool_pages is None:
        pool_pages = batch * pages_per_req
    tables = rng.permutation(pool_pages)[: batch * pages_per_req].astype(np.int32)
    tables = tables.reshape(batch, pages_per_req)
    q = normal_bf16(rng, (batch, heads, D_QK))
    rng_k = np.random.default_rng([seed, 7919, variant])
    topk = np.stack([_uniform_without_replacement(rng_k, ctx, top_k) for _ in range(batch)])
    return DecodeCase(f"deepseek_b{batch}_ctx{ctx}", q, topk, np.arange(batch, dtype=np.int32),
                      np.full(batch, ctx - 1, np.int32), tables, page_size, window, sinks,
                      top_k + window + sinks, pool_pages * page_size, pool_seed=seed + 1,
                      extra={"variant": variant})


def ragged_case(seed=2100, batch=128, n_long=8, short_ctx=96, long_ctx=32768, heads=128,
                top_k=2048, window=128, sinks=4, page_size=64, variant=0):
    """A ragged decode batch in the DeepSeek shape: most requests are short
    (context short_ctx: every position is a candidate, |S| = short_ctx), a
    few long (context long_ctx: top-k + window + sinks, |S| ~ 2180), at
    seeded positions in the batch -- the "most rows a few blocks, a few rows
    hundreds" mix of a ragged batch.  Short requests draw min(top_k, ctx)
    ids and pad with -1.  Page tables cover long_ctx for every request."""
    rng = np.random.default_rng(seed)
    pages_per_req = -(-long_ctx // page_size)
    pool_pages = batch * pages_per_req
    tables = rng.permutation(pool_pages).astype(np.int32).reshape(batch, pages_per_req)
    q = normal_bf16(rng, (batch, heads, D_QK))
    ctxs = np.full(batch, short_ctx, np.int64)
    ctxs[rng.choice(batch, size=n_long, replace=False)] = long_ctx
    rng_k = np.random.default_rng([seed, 7919, variant])
    topk = np.full((batch, top_k), -1, np.int32)
    for b in range(batch):
        k = min(top_k, int(ctxs[b]))
        topk[b, :k] = _uniform_without_replacement(rng_k, int(ctxs[b]), k)
    return DecodeCase(f"ragged_b{batch}", q, topk, np.arange(batch, dtype=np.int32),
                      (ctxs - 1).astype(np.int32), tables, page_size, window, sinks,
                      top_k + window + sinks, pool_pages * page_size, pool_seed=seed + 1,
                      extra={"contexts": ctxs, "variant": variant})


def int32_edge_case():
    """A small batch whose tables hold pages at the top of the int32 slot
    range (page size 48): page (2^31 - 1) // 48 keeps offsets 0..31 within
    int32 and loses 32..47, the page after it loses all 48."""
    c = random_small_case(19, T=6, heads=16, R=2, ctx=400, top_k=80, window=5, sinks=3,
                                    page_size=48, unmapped_frac=0.0)
    top = (2**31 - 1) // 48
    c.block_table[0, 0] = top        # slots top*48 .. top*48 + 31 fit, + 32 .. + 47 do not
    c.block_table[0, 1] = top + 1    # no slot of this page fits
    c.block_table[1, 2] = top + 5
    c.req_id[:3] = [0, 1, 0]
    c.q_pos[:3] = [350, 380, 47]
    return c


def clustered_topk(rng, ctx, top_k, run=16):
    """top_k ids as top_k/run non-overlapping runs of `run` consecutive tokens."""
    nruns = top_k // run
    while True:
        starts = np.sort(rng.integers(0, ctx - run + 1, size=nruns))
        if np.all(np.diff(starts) >= run):
            break
    ids = (starts[:, None] + np.arange(run)[None, :]).reshape(-1)
    return rng.permutation(ids).astype(np.int32)


def locality_case(seed, clustered, batch=64, ctx=131072, heads=128, top_k=2048, page_size=64):
    """Long-context sweep: top-k only (no window or sinks), scattered or clustered."""
    rng = np.random.default_rng(seed)
    pages_per_req = ctx // page_size
    pool_pages = batch * pages_per_req
    tables = rng.permutation(pool_pages).astype(np.int32).reshape(batch, pages_per_req)
    q = normal_bf16(rng, (batch, heads, D_QK))
    if clustered:
        topk = np.stack([clustered_topk(rng, ctx, top_k) for _ in range(batch)])
    else:
        topk = np.stack([_uniform_without_replacement(rng, ctx, top_k) for _ in range(batch)])
    return DecodeCase(f"locality_{'clustered' if clustered else 'scattered'}", q, topk,
                      np.arange(batch, dtype=np.int32), np.full(batch, ctx - 1, np.int32),
                      tables, page_size, 0, 0, top_k, pool_pages * page_size, pool_seed=seed + 1)


def random_small_case(seed, T=3, R=2, ctx=300, heads=8, top_k=40, window=5, sinks=2,
                      page_size=16, unmapped_frac=0.1, invalid_frac=0.1):
    """Small ragged case with unmapped pages, invalid ids, duplicates and padding."""
    rng = np.random.default_rng(seed)
    max_blocks = -(-ctx // page_size)
    pool_pages = R * max_blocks + 3
    tables = rng.permutation(pool_pages)[: R * max_blocks].astype(np.int32).reshape(R, max_blocks)
    tables[rng.random(tables.shape) < unmapped_frac] = -1
    req_id = rng.integers(0, R, size=T).astype(np.int32)
    q_pos = rng.integers(0, ctx, size=T).astype(np.int32)
    topk = rng.integers(-1, ctx + 20, size=(T, top_k)).astype(np.int32)
    dup = rng.random((T, top_k)) < 0.2
    topk[dup] = topk[:, :1].repeat(top_k, axis=1)[dup]
    topk[rng.random((T, top_k)) < invalid_frac] = -1
    q = normal_bf16(rng, (T, heads, D_QK))
    return DecodeCase(f"small_{seed}", q, topk, req_id, q_pos, tables, page_size, window, sinks,
                      top_k + window + sinks, pool_pages * page_size, pool_seed=seed + 1)


def evolve_topk(rng, prev, ctx_next, keep_frac=0.85):
    """Next step's top-k: keep floor(keep_frac*k) of the previous ids (uniform
    choice) plus fresh uniform draws without replacement from [0, ctx_next)
    outside the kept set."""
    k = len(prev)
    nkeep = int(math.floor(keep_frac * k))
    kept = rng.choice(prev, size=nkeep, replace=False)
    mask = np.ones(ctx_next, dtype=bool)
    mask[kept] = False
    pool = np.flatnonzero(mask)
    fresh = rng.choice(pool, size=k - nkeep, replace=False)
    return rng.permutation(np.concatenate([kept, fresh])).astype(np.int32)


@dataclass
class HotSteps:
    """Multi-step hot-buffer decode: per step, top-k sets for every request."""
    batch: int
    ctx0: int
    steps: int
    top_k: int
    window: int
    num_sinks: int
    page_size: int
    block_table: np.ndarray        # [batch, pages_per_req]
    topk: list                     # steps x [batch, top_k] int32
    q_bits: list                   # steps x [batch, heads, 576]
    host_rows: int
    pool_seed: int
    heads: int

    @property
    def hot_size(self):
        return 2 * self.top_k

    @property
    def region_stride(self):
        return -(-(self.hot_size + 1) // 128) * 128

    @property
    def cap(self):
        return self.top_k + self.window + self.num_sinks

    def q_pos(self, step):
        return np.full(self.batch, self.ctx0 + step - 1, dtype=np.int32)


def hot_steps_case(seed=3000, batch=64, ctx0=65536, steps=16, top_k=2048, window=128,
                   sinks=4, page_size=64, heads=128):
    """Consecutive decode steps whose top-k keeps 85% of the previous set.

    Step t decodes position ctx0 + t - 1 (context length ctx0 + t); each
    request owns a disjoint random set of pages of one shared host pool.
    """
    rng = np.random.default_rng(seed)
    ctx_max = ctx0 + steps
    pages_per_req = -(-ctx_max // page_size)
    pool_pages = batch * pages_per_req
    tables = rng.permutation(pool_pages).astype(np.int32).reshape(batch, pages_per_req)
    topk_steps, q_steps = [], []
    cur = [_uniform_without_replacement(rng, ctx0, top_k) for _ in range(batch)]
    for t in range(steps):
        if t > 0:
            cur = [evolve_topk(rng, c, ctx0 + t) for c in cur]
        topk_steps.append(np.stack(cur))
        q_steps.append(normal_bf16(rng, (batch, heads, D_QK)))
    return HotSteps(batch, ctx0, steps, top_k, window, sinks, page_size, tables, topk_steps,
                    q_steps, pool_pages * page_size, seed + 1, heads)


# ---- dense paged attention with grouped query heads -------------------------
# Token pool [slots, Hkv, 128] fp16 for K and for V, values N(0, 1); page
# size 16; each request owns a disjoint random set of pages of the pool.

D_HEAD = 128


def normal_fp16(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def dense_pool(slots, hkv, seed):
    """K and V pools [slots, hkv, 128] fp16 on the host (numpy)."""
    rng = np.random.default_rng(seed)
    return normal_fp16(rng, (slots, hkv, D_HEAD)), normal_fp16(rng, (slots, hkv, D_HEAD))


def dense_pool_torch(slots, hkv, seed, device, chunk_slots=1 << 16):
    """K and V pools generated in device memory by torch's seeded generator
    (N(0, 1) rounded to fp16 by torch's conversion)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    pools = []
    for _ in range(2):
        p = torch.empty((slots, hkv, D_HEAD), dtype=torch.float16, device=device)
        for lo in range(0, slots, chunk_slots):
            hi = min(slots, lo + chunk_slots)
            p[lo:hi] = torch.randn((hi - lo, hkv, D_HEAD), generator=g, device=device,
                                   dtype=torch.float32)
        pools.append(p)
    return pools[0], pools[1]


@dataclass
class GqaDecodeCase:
    name: str
    q: np.ndarray            # [B, Hq, 128] fp16
    block_table: np.ndarray  # [B, max_blocks] int32, -1 = unmapped
    ctx_lens: np.ndarray     # [B] int32
    page_size: int
    hkv: int
    num_slots: int
    pool_seed: int
    scale: float = 1.0 / math.sqrt(D_HEAD)


@dataclass
class ExtendCase:
    name: str
    q: np.ndarray            # [N, Hq, 128] fp16, packed by qo_indptr
    qo_indptr: np.ndarray    # [B + 1] int32
    kv_indptr: np.ndarray    # [B + 1] int32
    kv_indices: np.ndarray   # [kv_indptr[B]] int32 slot ids
    max_extend_len: int
    hkv: int
    num_slots: int
    pool_seed: int
    scale: float = 1.0 / math.sqrt(D_HEAD)


def _page_tables(rng, pages_per_req, spare=0):
    """Disjoint random page sets of one pool; ragged rows padded with -1."""
    total = int(np.sum(pages_per_req))
    perm = rng.permutation(total + spare).astype(np.int32)
    width = max(1, int(np.max(pages_per_req, initial=0)))
    tables = np.full((len(pages_per_req), width), -1, np.int32)
    off = 0
    for b, n in enumerate(pages_per_req):
        tables[b, :n] = perm[off:off + n]
        off += n
    return tables, total + spare


def gqa_decode_case(seed=5000, batch=128, ctx_lo=1024, ctx_hi=4096, hq=32, hkv=8, page_size=16):
    """Decode batch: context lengths uniform in [ctx_lo, ctx_hi], one query
    token per request, random block tables."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=batch).astype(np.int32)
    tables, pages = _page_tables(rng, -(-ctx // page_size))
    q = normal_fp16(rng, (batch, hq, D_HEAD))
    return GqaDecodeCase(f"gqa_decode_b{batch}", q, tables, ctx, page_size, hkv,
                         pages * page_size, pool_seed=seed + 1)


def extend_case(seed=5100, batch=8, prefix=4096, extend=512, hq=32, hkv=8, page_size=16):
    """Extend batch: every request has `prefix` cached tokens and `extend` new
    ones; its keys are the slots of its pages in order (prefix first)."""
    rng = np.random.default_rng(seed)
    lk = np.full(batch, prefix + extend, np.int64)
    lq = np.full(batch, extend, np.int64)
    return _extend_from_lengths(rng, f"extend_b{batch}_p{prefix}_e{extend}", lq, lk, hq, hkv,
                                page_size, seed + 1)


def _extend_from_lengths(rng, name, lq, lk, hq, hkv, page_size, pool_seed, bad_frac=0.0):
    pages_per_req = -(-np.asarray(lk) // page_size)
    tables, pages = _page_tables(rng, pages_per_req, spare=1)
    slots = []
    for b in range(len(lk)):
        t = np.arange(lk[b])
        s = (tables[b][t // page_size].astype(np.int64) * page_size + t % page_size).astype(np.int32)
        if bad_frac > 0:
            bad = rng.random(len(s)) < bad_frac
            s[bad] = rng.choice(np.asarray([-1, pages * page_size + 3, 1 << 30], np.int32),
                                size=int(bad.sum()))
        slots.append(s)
    qo = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    kv = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = normal_fp16(rng, (int(qo[-1]), hq, D_HEAD))
    kvi = np.concatenate(slots).astype(np.int32) if len(slots) else np.zeros(0, np.int32)
    return ExtendCase(name, q, qo, kv, kvi, int(np.max(lq, initial=0)), hkv, pages * page_size,
                      pool_seed)


def random_extend_case(seed, lq, lk, hq=8, hkv=2, page_size=16, bad_frac=0.05):
    """Small ragged extend batch with the given per-request query and key
    counts (Lk < Lq allowed: the first Lq - Lk queries then see nothing) and
    a fraction of bad slot ids (-1 or outside the pool)."""
    rng = np.random.default_rng(seed)
    return _extend_from_lengths(rng, f"extend_small_{seed}", np.asarray(lq, np.int64),
                                np.asarray(lk, np.int64), hq, hkv, page_size, seed + 1, bad_frac)


def random_gqa_decode_case(seed, ctx, hq=8, hkv=2, page_size=16, unmapped_frac=0.1,
                           table_slack=1):
    """Small ragged decode batch: context lengths as given, tables one block
    wider than needed (-1), a fraction of unmapped pages, and one page
    pointing outside the pool when the batch has room for it."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, np.int32)
    tables, pages = _page_tables(rng, -(-np.maximum(ctx, 0) // page_size), spare=2)
    tables = np.concatenate([tables, np.full((len(ctx), table_slack), -1, np.int32)], axis=1)
    tables[(rng.random(tables.shape) < unmapped_frac) & (tables >= 0)] = -1
    if len(ctx) > 1 and tables[1, 0] >= 0:
        tables[1, 0] = pages + 5  # a page past the pool's end
    q = normal_fp16(rng, (len(ctx), hq, D_HEAD))
    return GqaDecodeCase(f"gqa_small_{seed}", q, tables, ctx, page_size, hkv, pages * page_size,
                         pool_seed=seed + 1)


# ---- fp8_ds_mla rows ----------------------------------------------------------
# 656 bytes: 512 E4M3 codes of the latent values, 4 float32 scales (one per
# 128 values: amax / 448, the format's largest finite value), 64 bf16 RoPE
# values.  Latent and RoPE values are N(0, 1).  The rounding to E4M3 is
# torch's float8_e4m3fn conversion.

FP8_ROW_BYTES = 656


def _fp8_pack(latent, rope_bits, pow2_scales):
    """latent float32 [n, 512] (torch), rope bf16 bits [n, 64] (torch int16)
    -> [n, 656] uint8 rows (torch, same device)."""
    import torch
    n = latent.shape[0]
    g = latent.view(n, 4, 128)
    amax = g.abs().amax(dim=2).clamp_min(1e-12)
    scale = amax / 448.0
    if pow2_scales:
        scale = torch.exp2(torch.ceil(torch.log2(scale)))
    codes = (g / scale[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).view(n, 512)
    rows = torch.empty((n, FP8_ROW_BYTES), dtype=torch.uint8, device=latent.device)
    rows[:, :512] = codes
    rows[:, 512:528] = scale.to(torch.float32).contiguous().view(torch.uint8).view(n, 16)
    rows[:, 528:] = rope_bits.contiguous().view(torch.uint8).view(n, 128)
    return rows


def fp8_rows(rng, n, pow2_scales=False):
    """n fp8_ds_mla rows on the host (numpy uint8 [n, 656])."""
    import torch
    latent = torch.from_numpy(rng.standard_normal((n, 512), dtype=np.float32))
    rope = torch.from_numpy(normal_bf16(rng, (n, 64)).view(np.int16))
    return _fp8_pack(latent, rope, pow2_scales).numpy()


def fp8_pool_torch(rows, seed, device, chunk_rows=1 << 18):
    """fp8_ds_mla pool [rows, 656] uint8 generated in device memory by torch's
    seeded generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    pool = torch.empty((rows, FP8_ROW_BYTES), dtype=torch.uint8, device=device)
    for lo in range(0, rows, chunk_rows):
        hi = min(rows, lo + chunk_rows)
        latent = torch.randn((hi - lo, 512), generator=g, device=device, dtype=torch.float32)
        rope = torch.randn((hi - lo, 64), generator=g, device=device,
                           dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
        pool[lo:hi] = _fp8_pack(latent, rope, False)
    return pool
