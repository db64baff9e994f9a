"""Task tables for a ragged decode batch, and the decode run over them
(oracle; integer tables exact, attention in fp64).

TEST INFRASTRUCTURE ONLY -- see the package header.

What it states ("5.1.1 · 从索引到 Kernel"):

  * §5.1 (plan / run) and §7.4 (turning a ragged batch into a task table).
    The plan reads each row's length -- here the row's candidate count,
    clamped to [0, cap] as everywhere on this path -- and cuts the row into
    k_r = ceil(n_r / R) tasks of consecutive candidate positions, R being
    the target task size; a task is (row, start, end, split).  A
    prefix sum of the per-row task counts gives the global task ids:
    row_first[r] = sum over r' < r of ceil(n_r' / R), and the tasks of row r
    are row_first[r] .. row_first[r + 1] - 1 in split order.
  * §7.4 (stable row identity).  Tasks may run in any order; each carries
    its row, and a task's partial state goes to slot row_first[row] + split,
    read from the task itself and never from its place in the execution
    order; the split merge gathers a row's slots.  The result is the
    single-pass attention of every row (§3.2 eq. (7): merging any partition
    of S equals the single pass).

Readings: a row with n_r = 0 gets no task and its output is the empty-set
output (out = 0, lse = -inf); §7.4 fixes the number of tasks of a row
(about R candidates each, ceil(k_i / R) of them) but not where the cuts
fall: here task i of a row covers positions floor(i n / k) .. floor((i + 1)
n / k) - 1, so a row's tasks differ in size by at most one (none exceeds R,
none is empty) and no task is a short remainder that leaves the others
longer than they need to be.

Pins (tests/test_oracle_plan.py): a hand-worked table
(tests/golden/plan_example.txt); brute force over positions on random small
batches (every position of a row lies in exactly one of that row's tasks,
no task is longer than R or empty, tasks are numbered row by row in split
order, the total is sum ceil(n_r / R)); clamping of out-of-range counts;
run_tasks equal to the single-pass attention oracle, for the table as
planned and shuffled.
"""

import numpy as np

from .attention import attend_partial
from .merge import merge


def plan_tasks(counts, T, cap, rows_per_task):
    """Task table of a batch of T rows.

    counts: [T] candidate counts (None: every row has cap candidates).
    Returns (tasks [n, 4] int64 of (row, start, end, split), row_first [T + 1]).
    """
    R = int(rows_per_task)
    n_rows = []
    for r in range(T):
        n = cap if counts is None else int(counts[r])
        n_rows.append(min(max(n, 0), cap))
    per_row = [-(-n // R) for n in n_rows]           # ceil(n / R)
    row_first = np.zeros(T + 1, dtype=np.int64)
    row_first[1:] = np.cumsum(per_row)
    tasks = []
    for r, n in enumerate(n_rows):
        k = per_row[r]
        for i in range(k):
            tasks.append((r, i * n // k, (i + 1) * n // k, i))
    return np.asarray(tasks, dtype=np.int64).reshape(-1, 4), row_first


def run_tasks(q_bits, kv_bits, row_ids, tasks, row_first, scale):
    """Decode over a task table, in the table's order: each task's partial
    (o, m, l) over row_ids[row, start:end] into slot row_first[row] + split,
    then the merge of every row's slots.  Returns (out [T, H, 512], lse [T, H])."""
    T = len(row_first) - 1
    H = q_bits.shape[1]
    n_slots = int(row_first[-1])
    o = np.zeros((n_slots, H, 512))
    m = np.full((n_slots, H), -np.inf)
    l = np.zeros((n_slots, H))
    for row, start, end, split in np.asarray(tasks, dtype=np.int64):
        slot = int(row_first[row]) + int(split)
        ids = np.asarray(row_ids[row:row + 1, start:end])
        po, pm, pl = attend_partial(q_bits[row:row + 1], kv_bits, ids, None, scale, 1)
        o[slot], m[slot], l[slot] = po[0, 0], pm[0, 0], pl[0, 0]
    out = np.zeros((T, H, 512))
    lse = np.full((T, H), -np.inf)
    for r in range(T):
        a, b = int(row_first[r]), int(row_first[r + 1])
        if b > a:
            out[r], lse[r] = merge(o[a:b], m[a:b], l[a:b])
    return out, lse
