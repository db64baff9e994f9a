"""Pins for the task-table oracle (CPU only).

Fixed by the pages: the hand-worked table of tests/golden/plan_example.txt
("5.1.1 · 从索引到 Kernel" §7.4: ceil(k_i / R) tasks per row, global ids by a
prefix sum).  Fixed by brute force: every candidate position of every row
lies in exactly one task of that row, tasks are non-empty, at most R long
and numbered row by row in split order.  Fixed by the attention oracle:
running the tasks and merging each row's slots gives the single-pass
attention (§3.2 eq. (7)), whatever the order of the table (§7.4, stable row
identity).
"""

import os

import numpy as np
import pytest

import oracle
from oracle.plan import plan_tasks, run_tasks
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_example.txt")


def _golden():
    vals = {"task": []}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        key, rest = line.split(":", 1)
        nums = [int(x) for x in rest.split()]
        if key == "task":
            vals["task"].append(nums)
        else:
            vals[key] = nums
    return vals


def test_hand_worked_table():
    g = _golden()
    tasks, row_first = plan_tasks(g["counts"], len(g["counts"]), g["cap"][0],
                                  g["rows_per_task"][0])
    assert row_first.tolist() == g["row_first"]
    assert tasks.tolist() == g["task"]


@pytest.mark.parametrize("seed", range(6))
def test_positions_covered_once(seed):
    rng = np.random.default_rng(700 + seed)
    T = int(rng.integers(1, 40))
    cap = int(rng.integers(0, 300))
    R = int(rng.integers(1, 70))
    counts = rng.integers(-5, cap + 20, size=T)
    tasks, row_first = plan_tasks(counts, T, cap, R)
    n = np.clip(counts, 0, cap)
    assert len(tasks) == int(sum(-(-int(k) // R) for k in n))
    sizes = {}
    for r, a, b, _ in tasks:
        sizes.setdefault(int(r), []).append(int(b - a))
    for v in sizes.values():
        assert max(v) - min(v) <= 1  # a row's tasks differ by at most one
    assert row_first[0] == 0 and row_first[-1] == len(tasks)
    hits = [np.zeros(int(k), dtype=np.int64) for k in n]
    for i, (r, a, b, s) in enumerate(tasks):
        assert 0 < b - a <= R
        assert row_first[r] <= i < row_first[r + 1]
        assert i - row_first[r] == s  # split order inside the row
        hits[r][a:b] += 1
    for h in hits:
        assert np.all(h == 1)


def test_counts_none_means_cap():
    tasks, row_first = plan_tasks(None, 3, 20, 8)
    assert row_first.tolist() == [0, 3, 6, 9]
    assert tasks[:3].tolist() == [[0, 0, 6, 0], [0, 6, 13, 1], [0, 13, 20, 2]]


def _small_problem(seed):
    rng = np.random.default_rng(seed)
    T, H, cap, kv_rows = 5, 4, 37, 90
    q = workloads.bf16_bits(rng.standard_normal((T, H, 576)))
    kv = workloads.bf16_bits(rng.standard_normal((kv_rows, 576)))
    ids = rng.integers(-3, kv_rows + 3, size=(T, cap)).astype(np.int32)
    counts = np.array([0, 37, 12, 1, 30], dtype=np.int32)
    return q, kv, ids, counts, cap


@pytest.mark.parametrize("shuffle", [False, True])
def test_run_equals_single_pass(shuffle):
    q, kv, ids, counts, cap = _small_problem(710)
    scale = 576 ** -0.5
    tasks, row_first = plan_tasks(counts, len(counts), cap, 8)
    if shuffle:
        tasks = tasks[np.random.default_rng(711).permutation(len(tasks))]
    out, lse = run_tasks(q, kv, ids, tasks, row_first, scale)
    ref_out, ref_lse = oracle.attend_sparse(q, kv, ids, counts, scale)
    assert np.max(np.abs(out - ref_out)) < 1e-12
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - ref_lse[fin])) < 1e-12
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)  # the empty row
