"""GPU parity: plan / run of the sparse MLA decode (task tables of a capacity
tier, persistent work queue, graph capture).

The plan's task table is integer work and must equal the oracle's
(oracle.plan_tasks) exactly.  The run's output is compared with the fp64
attention oracle at the bf16 tolerance of helpers.assert_attention_close.
Reordering the run's queue entries must not change a single output bit (each
entry carries its row and the slot of its (row, split)).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_attention_close, bf16_bits_of, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu


def _stp():
    import sparse_top_paged_amd as stp
    return stp


def _plan_host(plan, T):
    n, row_first, tasks = _stp().plan_view(plan, T)
    return n, row_first.cpu().numpy(), tasks.cpu().numpy()


@pytest.mark.parametrize("T,cap,R,seed", [(1, 0, 8, 0), (7, 100, 1, 1), (33, 2180, 256, 2),
                                          (1000, 300, 64, 3), (1500, 2180, 1024, 4),
                                          (2600, 45, 7, 5)])
def test_plan_table_bit_exact(T, cap, R, seed):
    """Rows across several 1024-row chunks, counts below 0 and above cap, empty rows."""
    stp = _stp()
    rng = np.random.default_rng(900 + seed)
    counts = rng.integers(-5, cap + 30, size=T).astype(np.int32)
    counts[rng.random(T) < 0.2] = 0
    plan = stp.decode_plan(to_dev(counts), T, cap, R)
    torch.cuda.synchronize()
    n, row_first, tasks = _plan_host(plan, T)
    ref_tasks, ref_first = oracle.plan_tasks(counts, T, cap, R)
    assert n == len(ref_tasks)
    assert np.array_equal(row_first, ref_first)
    assert np.array_equal(tasks, ref_tasks)
    hdr = plan[:12].cpu().numpy()
    assert hdr[1] == T and hdr[2] == R and np.all(hdr[4:12] == 0)
    assert hdr[3] == (T * (-(-cap // R)) if cap > 0 else 0)
    # the run's queues: queue x holds the tasks of rows x, x + 8, ... in order,
    # each as (row, start, length, slot = row_first[row] + split, -1 for a
    # row's only task)
    qcount, seg = (v.cpu().numpy() for v in stp.plan_queues(plan, T))
    for x in range(8):
        one = lambda r: ref_first[r + 1] - ref_first[r] == 1  # noqa: E731
        expect = [(ref_tasks[i][0], ref_tasks[i][1], ref_tasks[i][2] - ref_tasks[i][1],
                   -1 if one(r) else ref_first[r] + ref_tasks[i][3])
                  for r in range(x, T, 8) for i in range(ref_first[r], ref_first[r + 1])]
        assert qcount[x] == len(expect)
        assert np.array_equal(seg[x, :qcount[x]].reshape(-1, 4),
                              np.asarray(expect, dtype=np.int64).reshape(-1, 4))


def test_plan_counts_none_means_cap():
    stp = _stp()
    plan = stp.decode_plan(None, 5, 70, 32, device=dev())
    torch.cuda.synchronize()
    n, row_first, tasks = _plan_host(plan, 5)
    ref_tasks, ref_first = oracle.plan_tasks(None, 5, 70, 32)
    assert np.array_equal(row_first, ref_first) and np.array_equal(tasks, ref_tasks)


def _random_problem(seed, T, H, cap, rows=700):
    rng = np.random.default_rng(seed)
    kv_bits = workloads.normal_bf16(rng, (rows, 576))
    q_bits = workloads.normal_bf16(rng, (T, H, 576))
    ids = rng.integers(-2, rows + 5, size=(T, cap)).astype(np.int32)
    counts = rng.integers(0, cap + 1, size=T).astype(np.int32)
    counts[0] = cap
    if T > 2:
        counts[2] = 0
    return q_bits, kv_bits, ids, counts


@pytest.mark.parametrize("T,H,cap,R", [(5, 16, 37, 8), (9, 128, 300, 64), (4, 80, 1030, 1024),
                                       (3, 192, 100, 1), (12, 64, 64, 32)])
def test_run_against_oracle(T, H, cap, R):
    stp = _stp()
    q_bits, kv_bits, ids, counts = _random_problem(T * 100 + H + cap, T, H, cap)
    c_dev = to_dev(counts)
    plan = stp.decode_plan(c_dev, T, cap, R)
    out, lse = stp.decode_run(bf16_dev(q_bits), bf16_dev(kv_bits), to_dev(ids), plan, R, 0.05)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, counts, 0.05)
    assert_attention_close(out, lse, o_ref, l_ref, f"run T={T} H={H} cap={cap} R={R}")
    if T > 2:
        assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))


def test_shuffled_queues_and_repeated_runs_bit_identical():
    """Any order of the queue entries (within and across the eight queues)
    gives the same bits; one plan serves many runs."""
    stp = _stp()
    T, H, cap, R = 10, 128, 500, 48
    q_bits, kv_bits, ids, counts = _random_problem(31, T, H, cap)
    q, kv, idd = bf16_dev(q_bits), bf16_dev(kv_bits), to_dev(ids)
    plan = stp.decode_plan(to_dev(counts), T, cap, R)
    out1, lse1 = stp.decode_run(q, kv, idd, plan, R, 0.05)
    out2, lse2 = stp.decode_run(q, kv, idd, plan, R, 0.05)  # queue heads were reset
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    qcount, seg = stp.plan_queues(plan, T)
    counts_q = qcount.cpu().numpy()
    where = [(x, j) for x in range(8) for j in range(int(counts_q[x]))]
    entries = torch.stack([seg[x, j].clone() for x, j in where])
    perm = np.random.default_rng(32).permutation(len(where))
    for (x, j), p in zip(where, perm):  # every entry moves, across queues too
        seg[x, j].copy_(entries[int(p)])
    out3, lse3 = stp.decode_run(q, kv, idd, plan, R, 0.05)
    torch.cuda.synchronize()
    assert torch.equal(out1, out3) and torch.equal(lse1, lse3)
    o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, counts, 0.05)
    assert_attention_close(out3, lse3, o_ref, l_ref, "shuffled table")


def test_empty_tier_and_errors():
    stp = _stp()
    T, H = 3, 16
    q = bf16_dev(workloads.normal_bf16(np.random.default_rng(1), (T, H, 576)))
    kv = bf16_dev(workloads.normal_bf16(np.random.default_rng(2), (10, 576)))
    ids = torch.full((T, 0), -1, dtype=torch.int32, device=dev())
    plan = stp.decode_plan(torch.zeros(T, dtype=torch.int32, device=dev()), T, 0, 16)
    out, lse = stp.decode_run(q, kv, ids, plan, 16, 0.05)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    with pytest.raises(RuntimeError):
        stp.decode_plan(torch.zeros(T, dtype=torch.int32, device=dev()), T, 50, 0)
    small = torch.zeros(8, dtype=torch.int32, device=dev())
    with pytest.raises(RuntimeError):
        stp.decode_plan(torch.zeros(T, dtype=torch.int32, device=dev()), T, 50, 16, plan=small)


def test_graph_capture_replays_with_new_inputs():
    """plan + run captured once; counts and candidates change in place between
    replays (with eager work and synchronisation in between); every replay
    matches the eager run on the same inputs, bit for bit."""
    stp = _stp()
    T, H, cap, R = 8, 128, 400, 64
    rng = np.random.default_rng(77)
    rows = 900
    kv = bf16_dev(workloads.normal_bf16(rng, (rows, 576)))
    q = bf16_dev(workloads.normal_bf16(rng, (T, H, 576)))
    ids = torch.zeros((T, cap), dtype=torch.int32, device=dev())
    counts = torch.zeros(T, dtype=torch.int32, device=dev())
    plan = torch.zeros(stp.decode_plan_bytes(T, cap, R) // 4, dtype=torch.int32, device=dev())
    ws = torch.zeros(stp.decode_run_workspace_bytes(T, H, cap, R), dtype=torch.uint8, device=dev())
    out = torch.zeros((T, H, 512), dtype=torch.bfloat16, device=dev())
    lse = torch.zeros((T, H), dtype=torch.float32, device=dev())

    def step():
        stp.decode_plan(counts, T, cap, R, plan=plan)
        stp.decode_run(q, kv, ids, plan, R, 0.05, workspace=ws, out=out, lse=lse)

    def fill(seed):
        r = np.random.default_rng(seed)
        ids.copy_(torch.from_numpy(r.integers(-1, rows, size=(T, cap)).astype(np.int32)))
        c = r.integers(0, cap + 1, size=T).astype(np.int32)
        c[r.integers(0, T)] = 0
        counts.copy_(torch.from_numpy(c))

    fill(0)
    step()  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k in range(1, 5):
        fill(k)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_out, got_lse = out.clone(), lse.clone()
        _ = (q.float() * 2).sum()  # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(got_out, out) and torch.equal(got_lse, lse), f"replay {k}"
        if k == 2:
            o_ref, l_ref = oracle.attend_sparse(bf16_bits_of(q), bf16_bits_of(kv),
                                                ids.cpu().numpy(), counts.cpu().numpy(), 0.05)
            assert_attention_close(got_out, got_lse, o_ref, l_ref, "graph replay")


def _sampled(case, kv, out, lse, tokens, counts, slots, where):
    for t in tokens:
        n = int(counts[t])
        rows = slots[t, :n]
        kv_rows = bf16_bits_of(kv[torch.from_numpy(rows.astype(np.int64)).to(kv.device)])
        o_ref, l_ref = oracle.attend_sparse(case.q_bits[t:t + 1], kv_rows,
                                            np.arange(n, dtype=np.int32)[None, :], None, case.scale)
        assert_attention_close(out[t:t + 1], lse[t:t + 1], o_ref, l_ref, f"{where} token {t}")


@pytest.mark.parametrize("which", ["deepseek", "ragged"])
def test_full_size_sampled(which):
    """The DeepSeek-shaped batch (32 tokens, |S| ~ 2172) and the ragged batch
    (128 tokens: 120 with |S| = 96, 8 with |S| ~ 2180), normalised on the
    device, planned with the task size the benchmark uses and run; sampled
    tokens against the oracle, and the static decode's output agrees."""
    stp = _stp()
    c = workloads.deepseek_case() if which == "deepseek" else workloads.ragged_case()
    kv = workloads.pool_torch(c.kv_rows, c.pool_seed, dev())
    norm = stp.normalize_indices(to_dev(c.topk), to_dev(c.req_id), to_dev(c.q_pos),
                                 to_dev(c.block_table), c.page_size, c.window, c.num_sinks, c.cap,
                                 block_view=False)
    T, H = c.q_bits.shape[0], c.q_bits.shape[1]
    R = stp.decode_plan_rows_per_task(T, H, c.cap) if which == "deepseek" else 256
    plan = stp.decode_plan(norm["count"], T, c.cap, R)
    out, lse = stp.decode_run(bf16_dev(c.q_bits), kv, norm["slot"], plan, R, c.scale)
    torch.cuda.synchronize()
    counts = norm["count"].cpu().numpy()
    slots = norm["slot"].cpu().numpy()
    longest = int(np.argmax(counts))
    _sampled(c, kv, out, lse, sorted({0, longest, T - 1}), counts, slots, which)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    o2, l2 = stp.sparse_mla_decode(bf16_dev(c.q_bits), kv, norm["slot"], norm["count"], c.scale)
    torch.cuda.synchronize()
    assert (out.float() - o2.float()).abs().max().item() < 2e-2
    assert (lse - l2).abs().max().item() < 1e-2
    del kv
    torch.cuda.empty_cache()


def test_smaller_batch_in_a_larger_tier():
    """A batch of 5 rows run in a tier of 8 (rows 5..7 padded with count 0):
    the real rows equal the 5-row tier's output bit for bit, the padding rows
    are out = 0, lse = -inf."""
    stp = _stp()
    T, Tt, H, cap, R = 5, 8, 64, 260, 64
    q_bits, kv_bits, ids, counts = _random_problem(51, T, H, cap)
    kv = bf16_dev(kv_bits)
    plan = stp.decode_plan(to_dev(counts), T, cap, R)
    out, lse = stp.decode_run(bf16_dev(q_bits), kv, to_dev(ids), plan, R, 0.05)
    qp = np.concatenate([q_bits, np.zeros((Tt - T, H, 576), q_bits.dtype)])
    ip = np.concatenate([ids, np.full((Tt - T, cap), -1, np.int32)])
    cp = np.concatenate([counts, np.zeros(Tt - T, np.int32)])
    plan_t = stp.decode_plan(to_dev(cp), Tt, cap, R)
    out_t, lse_t = stp.decode_run(bf16_dev(qp), kv, to_dev(ip), plan_t, R, 0.05)
    torch.cuda.synchronize()
    assert torch.equal(out_t[:T], out) and torch.equal(lse_t[:T], lse)
    assert torch.all(out_t[T:] == 0) and torch.all(torch.isneginf(lse_t[T:]))


def test_one_queue_claimed_by_every_xcd():
    """One row of 1000 one-candidate tasks: all 2000 work items sit in queue 0,
    most beyond the pre-assigned ones, so workgroups of every XCD claim them
    through the queue head; a lost item would leave its slot stale."""
    stp = _stp()
    T, H, cap, R = 1, 128, 1000, 1
    q_bits, kv_bits, ids, counts = _random_problem(61, T, H, cap, rows=1500)
    counts[:] = cap
    plan = stp.decode_plan(to_dev(counts), T, cap, R)
    ws = torch.full((stp.decode_run_workspace_bytes(T, H, cap, R),), 0x7f, dtype=torch.uint8,
                    device=dev())  # stale slots would read as large finite garbage
    out, lse = stp.decode_run(bf16_dev(q_bits), bf16_dev(kv_bits), to_dev(ids), plan, R, 0.05,
                              workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, counts, 0.05)
    assert_attention_close(out, lse, o_ref, l_ref, "single queue")
    assert torch.all(plan[4:12] == 0)  # the merge cleared the queue heads
