"""Candidate-index normalisation (oracle, plain definition).

TEST INFRASTRUCTURE ONLY -- see the package header.

What it states ("5.1.1 · 从索引到 Kernel", §1.1 eq. (1), §1.2 eq. (2), §7.3
eq. (16)-(17), §7.4 eq. (19)):

  S_i = unique(D_i ∪ W_i ∪ A_i), restricted to positions the query may see
  (0 <= t <= q_pos, page mapped in the request's table), in ascending logical
  order.  Each surviving token t maps to logical block b = t // P, in-page
  offset t % P and physical slot table[r][b] * P + t % P (the slot-id
  addressing of the "HiSparse" walkthrough, section on vLLM PageAttention KV
  cache management, and of the Triton token -> global slot conversion).

Readings where the pages leave a step open (all listed in the design notes):
  * W_i = [max(0, q-w+1), q]  (the last w positions, the query's own included);
  * A_i = [0, min(a, q+1))    (the first a positions);
  * D entries < 0 are padding; entries > q, on a block outside the table or on
    an unmapped (negative) page are dropped and counted, with multiplicity;
  * a token row whose request id is outside [0, num_reqs) or whose q_pos < 0
    is a padding row: no candidates, nothing counted;
  * duplicates count once (eq. (1));
  * slot ids that do not fit in int32 are treated as unmapped.

Pins (tests/test_oracle_normalize.py): the two worked index examples of §1.2
(stored under tests/golden/), a brute-force Python-set construction on tiny
random inputs, and the invariants "duplicated D gives the same S", "S strictly
ascending", "slots injective within a request".
"""

import numpy as np

INT32_MAX = 2**31 - 1


def _valid(t, q, table_row, page_size):
    """Position t is visible to a query at q and lies on a mapped page."""
    if t < 0 or t > q:
        return False
    b = t // page_size
    if b >= len(table_row):
        return False
    page = int(table_row[b])
    if page < 0:
        return False
    if page * page_size + (t % page_size) > INT32_MAX:
        return False
    return True


def candidate_set(topk_row, q, window, num_sinks, table_row, page_size):
    """Sorted unique candidate set S and the number of dropped D entries.

    eq. (1): S = unique(D ∪ W ∪ A); the causal and page filters follow §1.1
    ("validate range, causality and batch ownership").
    """
    if q < 0:
        return [], 0
    dropped = 0
    cands = set()
    for t in topk_row:
        t = int(t)
        if t < 0:
            continue  # padding
        if _valid(t, q, table_row, page_size):
            cands.add(t)
        else:
            dropped += 1
    if window > 0:
        for t in range(max(0, q - window + 1), q + 1):
            if _valid(t, q, table_row, page_size):
                cands.add(t)
    for t in range(0, min(num_sinks, q + 1)):
        if _valid(t, q, table_row, page_size):
            cands.add(t)
    return sorted(cands), dropped


def block_view(S, table_row, page_size):
    """BSR view of one sorted candidate list (§1.2 eq. (2), §7.4 eq. (19)).

    Returns (logical blocks ascending, physical pages, in-page membership
    masks with bit t % P set for every t of S in the block).
    """
    assert page_size <= 64
    blocks, pages, masks = [], [], []
    for t in S:
        b = t // page_size
        if not blocks or blocks[-1] != b:
            blocks.append(b)
            pages.append(int(table_row[b]))
            masks.append(0)
        masks[-1] |= 1 << (t % page_size)
    return blocks, pages, masks


def normalize(topk, req_id, q_pos, window, num_sinks, block_table, page_size, cap):
    """Normalise every query token's candidates.

    topk [T, top_k] int, req_id [T], q_pos [T], block_table [R, max_blocks].
    Returns a dict of numpy arrays:
      tok [T, cap], slot [T, cap] (int32, -1 padded), count [T], dropped [T],
      blk_indptr [T+1], blk_logical [nnz], blk_page [nnz], blk_mask [nnz] (uint64).
    """
    topk = np.asarray(topk)
    T = topk.shape[0]
    R = block_table.shape[0]
    tok = np.full((T, cap), -1, dtype=np.int32)
    slot = np.full((T, cap), -1, dtype=np.int32)
    count = np.zeros(T, dtype=np.int32)
    dropped = np.zeros(T, dtype=np.int32)
    indptr = [0]
    logical, pages, masks = [], [], []
    for i in range(T):
        r = int(req_id[i])
        q = int(q_pos[i])
        if r < 0 or r >= R or q < 0:
            indptr.append(indptr[-1])
            continue
        table_row = block_table[r]
        S, nd = candidate_set(topk[i], q, window, num_sinks, table_row, page_size)
        if len(S) > cap:
            raise ValueError(f"token {i}: |S|={len(S)} exceeds cap={cap}")
        count[i] = len(S)
        dropped[i] = nd
        for j, t in enumerate(S):
            tok[i, j] = t
            slot[i, j] = int(table_row[t // page_size]) * page_size + t % page_size
        b, p, m = block_view(S, table_row, page_size)
        logical += b
        pages += p
        masks += m
        indptr.append(indptr[-1] + len(b))
    return {
        "tok": tok,
        "slot": slot,
        "count": count,
        "dropped": dropped,
        "blk_indptr": np.asarray(indptr, dtype=np.int32),
        "blk_logical": np.asarray(logical, dtype=np.int32),
        "blk_page": np.asarray(pages, dtype=np.int32),
        "blk_mask": np.asarray(masks, dtype=np.uint64),
    }
