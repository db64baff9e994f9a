"""Dense paged attention with grouped query heads (oracle, plain definition, fp64).

TEST INFRASTRUCTURE ONLY -- see the package header.

What it states ("PagedAttention 与 RadixAttention：上游机制与海光实现对照"):

  * Token pool.  Keys and values live in a pool addressed by slot id, one
    row per slot and KV head, [slots, Hkv, D] (the bshd layout of §5, item
    "layout == 1"); a paged request maps its logical token t to slot
    table[t // P] * P + t % P (§1.2, block table).
  * Grouped query heads.  Query head h reads KV head h // (Hq / Hkv)
    (§1.4 part 4).
  * Decode (§1.1).  For request b with context length n_b, every query head
    attends to tokens 0 .. n_b - 1 of its request:
        out = softmax(q K^T * scale) V,   lse = log sum_t exp(z_t).
  * Extend (§3.1-§3.3).  Request b has Lq = qo_indptr[b+1] - qo_indptr[b]
    new queries (rows qo_indptr[b] .. of the packed query tensor) and
    Lk = kv_indptr[b+1] - kv_indptr[b] keys at the slots
    kv_indices[kv_indptr[b] : kv_indptr[b+1]] (prefix first, then the new
    tokens); query i sees key j iff j <= i + (Lk - Lq), the shifted causal
    mask of §3.2.  The metadata arrays follow §3.3: qo_indptr and kv_indptr
    are exclusive prefix sums of the extend and total lengths, the prefix
    length is their difference.

Both are the dense masked softmax attention of attention.attend_dense_masked
over the gathered rows -- the definition, with a numpy matrix product per
step and no tiling.  A query row with nothing visible gives out = 0 and
lse = -inf.  Bad ids are data, as on the sparse path: a decode token whose
page is unmapped (table entry < 0, or a block past the end of the table) or
whose slot is outside the pool, and an extend key whose slot is outside the
pool, take no part.

Pins (tests/test_oracle_dense.py): the three-request ragged example of §3.3
(its printed metadata arrays, tests/golden/extend_ragged_example.txt);
pure-Python math.fsum attention over rows gathered by an independent loop on
tiny inputs, for both decode and extend; the shifted mask of §3.2 (its
printed 3 x 7 matrix, pinned with attention.shifted_causal_mask); closed
forms (identical keys give the mean of the values and lse = z + ln n; one
key gives its value row); without a prefix the extend is the causal prefill
(§3.2 reduces the mask to a lower triangle); with one query per request it
is the decode over the same slots.
"""

import numpy as np

from .attention import attend_dense_masked, shifted_causal_mask


def _f64(x):
    """fp16 (or any float) array widened exactly to float64."""
    return np.asarray(x).astype(np.float64)


def extend_metadata(extend_seq_lens, seq_lens):
    """§3.3 arrays from the per-request lengths: qo_indptr, kv_indptr (both
    [B + 1], exclusive prefix sums), extend_prefix_lens and extend_start_loc."""
    e = np.asarray(extend_seq_lens, dtype=np.int64)
    s = np.asarray(seq_lens, dtype=np.int64)
    qo = np.concatenate([[0], np.cumsum(e)])
    kv = np.concatenate([[0], np.cumsum(s)])
    return {"qo_indptr": qo, "kv_indptr": kv, "extend_prefix_lens": s - e,
            "extend_start_loc": qo[:-1]}


def decode_slots(table_row, n, page_size):
    """Slots of tokens 0 .. n - 1 of a paged request (§1.2)."""
    t = np.arange(n, dtype=np.int64)
    return np.asarray(table_row, dtype=np.int64)[t // page_size] * page_size + t % page_size


def paged_gqa_decode(q, k_pool, v_pool, block_table, ctx_lens, page_size, scale):
    """Decode: q [B, Hq, D], k_pool / v_pool [slots, Hkv, D] -> out [B, Hq, D],
    lse [B, Hq] (fp64)."""
    q = _f64(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    group = Hq // Hkv
    out = np.zeros((B, Hq, v_pool.shape[2]))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(ctx_lens[b])
        if n <= 0:
            continue  # nothing to attend to: out = 0, lse = -inf
        row = np.asarray(block_table[b], dtype=np.int64).reshape(-1)
        t = np.arange(n, dtype=np.int64)
        inside = t // page_size < len(row)  # tokens past the table: unmapped
        pages = np.where(inside, row[np.minimum(t // page_size, max(len(row) - 1, 0))]
                         if len(row) else -1, -1)
        slots = pages * page_size + t % page_size
        ok = (pages >= 0) & (slots >= 0) & (slots < k_pool.shape[0])
        slots = np.where(ok, slots, 0)
        for g in range(Hkv):
            K = _f64(k_pool[slots, g])
            V = _f64(v_pool[slots, g])
            heads = slice(g * group, (g + 1) * group)
            mask = np.broadcast_to(ok, (group, n))
            out[b, heads], lse[b, heads] = attend_dense_masked(q[b, heads], K, V, mask, scale)
    return out, lse


def extend_attention(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, scale):
    """Extend: q [N, Hq, D] packed by qo_indptr -> out [N, Hq, D], lse [N, Hq]."""
    q = _f64(q)
    N, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    group = Hq // Hkv
    out = np.zeros((N, Hq, v_pool.shape[2]))
    lse = np.full((N, Hq), -np.inf)
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        k0, k1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
        if q1 <= q0 or k1 <= k0:
            continue  # no queries, or no keys: out = 0, lse = -inf
        slots = np.asarray(kv_indices[k0:k1], dtype=np.int64)
        ok = (slots >= 0) & (slots < k_pool.shape[0])
        slots = np.where(ok, slots, 0)
        mask = shifted_causal_mask(q1 - q0, k1 - k0) & ok[None, :]
        for h in range(Hq):
            g = h // group
            out[q0:q1, h], lse[q0:q1, h] = attend_dense_masked(
                q[q0:q1, h], _f64(k_pool[slots, g]), _f64(v_pool[slots, g]), mask, scale)
    return out, lse
