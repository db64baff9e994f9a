"""Split-KV partial-state merge (oracle, plain definition, fp64).

TEST INFRASTRUCTURE ONLY -- see the package header.

"5.1.1 · 从索引到 Kernel" §3.2 eq. (7), generalised from two splits to any
number: with m = max over splits of m_s,

    l = sum_s exp(m_s - m) * l_s,    o = sum_s exp(m_s - m) * o_s,
    out = o / l,                     lse = m + ln l,

where o_s is the split's un-normalised numerator.  A split with l_s = 0 has
no valid row and takes no part, its m_s included (§7.1, the four-split
example).  When every split is empty the output is 0 and lse = -inf.

merge_normalized restates the same merge from normalised split outputs
O_p = o_p / l_p, weighting each by l_p exp(m_p - M) / L ("PagedAttention 与
RadixAttention：上游机制与海光实现对照", §1.4 part 3, the combine derivation);
the tests check the two forms against each other.

Pins (tests/test_oracle_merge.py): the two-split hand computation of §3.2
(-> 2.0, and the naive sum of normalised outputs -> 4 must not match), the
four-split denominator of §7.1 eq. (14) (-> about 17.85), and "merging any
partition of S equals the single pass".
"""

import numpy as np


def merge(o_part, m_part, l_part):
    """o_part [..., S, H, dv], m_part / l_part [..., S, H] -> (out, lse)."""
    o_part = np.asarray(o_part, dtype=np.float64)
    m_part = np.asarray(m_part, dtype=np.float64)
    l_part = np.asarray(l_part, dtype=np.float64)
    live = l_part > 0
    m = np.where(live, m_part, -np.inf).max(axis=-2)          # [..., H]
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.where(live, np.exp(np.where(live, m_part, 0.0) - m_safe[..., None, :]), 0.0)
    l = (w * l_part).sum(axis=-2)
    o = (w[..., None] * o_part).sum(axis=-3)
    out = np.where(empty[..., None], 0.0, o / np.where(empty, 1.0, l)[..., None])
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return out, lse


def merge_normalized(O_norm, m_part, l_part):
    """Same merge from normalised split outputs O_p (the partition-combine form)."""
    O_norm = np.asarray(O_norm, dtype=np.float64)
    m_part = np.asarray(m_part, dtype=np.float64)
    l_part = np.asarray(l_part, dtype=np.float64)
    live = l_part > 0
    M = np.where(live, m_part, -np.inf).max(axis=-2)
    empty = ~np.isfinite(M)
    M_safe = np.where(empty, 0.0, M)
    lp = np.where(live, l_part * np.exp(np.where(live, m_part, 0.0) - M_safe[..., None, :]), 0.0)
    L = lp.sum(axis=-2)
    w = lp / np.where(empty, 1.0, L)[..., None, :]
    out = (w[..., None] * O_norm).sum(axis=-3)
    out = np.where(empty[..., None], 0.0, out)
    lse = np.where(empty, -np.inf, M_safe + np.log(np.where(empty, 1.0, L)))
    return out, lse
