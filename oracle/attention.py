"""Sparse MLA decode attention (oracle, plain definition, fp64).

TEST INFRASTRUCTURE ONLY -- see the package header.

What it states.  For one query token with candidate rows S (slot ids into
the latent KV pool, each row 576 values: 512 latent then 64 rope):

    z_t = scale * sum_{d<576} q[d] * kv[t, d]          ("5.1.1 · 从索引到 Kernel",
                                                       §3.1 eq. (4), one query row)
    m = max_t z_t,  l = sum_t exp(z_t - m)            (§3.1, the tile statistics
                                                       taken over all of S at once)
    out = sum_t exp(z_t - m) * kv[t, :512] / l,  lse = m + ln l

i.e. softmax(q K_S^T * scale) V_S, the decode attention of "PagedAttention 与
RadixAttention：上游机制与海光实现对照" §1.1 restricted to the selected rows.
Tiling, online rescaling (eq. (5)-(6)) and splits only reorder this sum, so
the oracle is the definition itself, evaluated with numpy fp64 matrix
products (a library primitive per step, no blocking or reordering).

Readings (listed in the design notes): V is the first 512 values of the same
row; an empty S gives out = 0 and lse = -inf (§3.2 allows a defined zero
output); entries outside [0, kv_rows) or at positions >= count are not part
of S; a split covers a contiguous range of ceil(n / num_splits) positions.

Pins (tests/test_oracle_attention.py): a pure-Python math.fsum triple loop on
tiny inputs, a dense masked softmax over all positions with -inf outside S
(§1.2: masking U \\ S gives back S), closed forms (one candidate -> its V row
and lse = z; q = 0 -> mean of V rows), the textbook dense decode for S = all
positions, the +ln 2 shift of a doubled key (§7.3), and the shifted causal
mask matrix printed in §3.2 of the PagedAttention page.
"""

import math

import numpy as np

D_QK = 576
D_V = 512


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rows_of(ids, count, kv_rows):
    ids = np.asarray(ids[:count], dtype=np.int64)
    return ids[(ids >= 0) & (ids < kv_rows)]


def _attend_rows(q, K, V, scale):
    """softmax(q K^T * scale) V over the given rows; q [H, d], K [n, d]."""
    H = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1])), np.full(H, -np.inf), np.full(H, -np.inf), np.zeros(H), np.zeros((H, V.shape[1]))
    z = (q @ K.T) * scale                  # [H, n]
    m = z.max(axis=1)                      # [H]
    p = np.exp(z - m[:, None])
    l = p.sum(axis=1)
    o = p @ V                              # unnormalised numerator
    return o / l[:, None], m + np.log(l), m, l, o


def attend_sparse(q_bits, kv_bits, row_ids, counts, scale, dv=D_V):
    """out [T, H, dv] and lse [T, H] (fp64) for bf16 inputs given as bits.

    kv_bits may be a 2-D array [kv_rows, 576] or a callable returning the
    fp64 rows for an index vector (used for pools too large to widen whole).
    """
    q = bf16_bits_to_f64(q_bits)
    T, H, _ = q.shape
    cap = row_ids.shape[1]
    getter, kv_rows = _kv_getter(kv_bits)
    out = np.zeros((T, H, dv))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        n = cap if counts is None else int(counts[t])
        rows = _rows_of(row_ids[t], n, kv_rows)
        K = getter(rows)
        out[t], lse[t], _, _, _ = _attend_rows(q[t], K, K[:, :dv], scale)
    return out, lse


def _kv_getter(kv_bits):
    if callable(kv_bits):
        return kv_bits, kv_bits.rows
    kv_rows = kv_bits.shape[0]
    return (lambda rows: bf16_bits_to_f64(kv_bits[rows])), kv_rows


def split_ranges(n, num_splits):
    """Contiguous position ranges [lo, hi) of ceil(n / num_splits) entries."""
    chunk = -(-n // num_splits) if n > 0 else 0
    return [(min(n, s * chunk), min(n, (s + 1) * chunk)) for s in range(num_splits)]


def attend_partial(q_bits, kv_bits, row_ids, counts, scale, num_splits, dv=D_V):
    """Per-split states (o unnormalised, m, l), the partial form of §3.2 eq. (7).

    Returns o [T, S, H, dv], m [T, S, H], l [T, S, H]; an empty split has
    o = 0, m = -inf, l = 0.
    """
    q = bf16_bits_to_f64(q_bits)
    T, H, _ = q.shape
    cap = row_ids.shape[1]
    getter, kv_rows = _kv_getter(kv_bits)
    o = np.zeros((T, num_splits, H, dv))
    m = np.full((T, num_splits, H), -np.inf)
    l = np.zeros((T, num_splits, H))
    for t in range(T):
        n = cap if counts is None else int(counts[t])
        for s, (lo, hi) in enumerate(split_ranges(n, num_splits)):
            ids = np.asarray(row_ids[t, lo:hi], dtype=np.int64)
            rows = ids[(ids >= 0) & (ids < kv_rows)]
            if len(rows) == 0:
                continue
            K = getter(rows)
            _, _, m[t, s], l[t, s], o[t, s] = _attend_rows(q[t], K, K[:, :dv], scale)
    return o, m, l


def shifted_causal_mask(Lq, Lk):
    """Visible iff j <= i + (Lk - Lq) (PagedAttention page, §3.2)."""
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    return j <= i + (Lk - Lq)


def attend_dense_masked(Q, K, V, mask, scale):
    """Dense softmax attention with a boolean visibility mask (fp64).

    Q [Lq, d], K [Lk, d], V [Lk, dv], mask [Lq, Lk] (True = visible); rows
    with nothing visible give out = 0, lse = -inf.
    """
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    z = (Q @ K.T) * scale
    z = np.where(mask, z, -np.inf)
    m = z.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.where(mask, np.exp(z - m_safe[:, None]), 0.0)
    l = p.sum(axis=1)
    out = np.where(empty[:, None], 0.0, (p @ V) / np.where(empty, 1.0, l)[:, None])
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return out, lse


def attend_fsum(q, K, V, scale):
    """Pure-Python triple loop with math.fsum, for tiny inputs only.

    q: list of H lists of d floats; K: list of n rows of d floats; V: list of
    n rows of dv floats.  Returns (out [H][dv], lse [H]).
    """
    out, lse = [], []
    for qh in q:
        z = [scale * math.fsum(a * b for a, b in zip(qh, k)) for k in K]
        if not z:
            out.append([0.0] * (len(V[0]) if V else 0))
            lse.append(-math.inf)
            continue
        m = max(z)
        p = [math.exp(x - m) for x in z]
        l = math.fsum(p)
        out.append([math.fsum(p[t] * V[t][c] for t in range(len(V))) / l for c in range(len(V[0]))])
        lse.append(m + math.log(l))
    return out, lse
