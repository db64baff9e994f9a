"""Decode-step benchmark of the top-k sparse MLA path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload (DeepSeek-V3.2-shaped decode, one layer): 32 requests x 1 query
token, 128 query heads, one latent KV head of bf16 rows of 576 (1152 B),
context 32768, page size 64 over a shared 1,048,576-row pool (1.2 GB, in
HBM), top-k 2048 uniform over the causal range + 128-token window + 4 sinks.

A step is one pass of the hot path over one batch: candidate normalisation
(with the block view) -> sparse MLA decode (normalised bf16 split partial
states) -> split merge, i.e. stp_normalize_indices followed by the two
launches stp_sparse_mla_decode makes, called one by one so that the decode
kernel can be timed alone.  Inputs are resident in HBM before timing starts.  Eight candidate
sets (same pool, tables and queries, different top-k draws) rotate step by
step, so a set's ~80 MB of rows is not still in the 256 MB Infinity Cache
when it comes round again.

Prints one JSON line.  `value` is query tokens per second over the timed
steps; `roofline` is the decode kernel's algorithmic bytes per launch over
its average duration, taken from a loop of its own of at least 200 launches
after the timed steps, enqueued back to back between two HIP events on the
kernel's stream;
`ceilings` times, in the same run, the decode's row gather alone
(stp_row_gather: the same rows, splits and XCD placement, no arithmetic) and
a plain device copy, the practical ceilings the decode's rate is set against;
`cpu_baseline` times the fp64 oracle on a bounded sample on the host, on all
available cores and on one.  Inside the timed steps the decode kernel is
bracketed by events on every 7th step only (reported beside the roofline
loop): an event pair costs a few microseconds of queue time, which would
otherwise be counted in every step.
"""

import argparse
import hashlib
import itertools
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROW_BYTES = 1152
METRIC = "decode query-tokens/sec and effective KV GB/s (% HBM/MFMA roofline), 1 MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
GQA_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gqa_decode_traffic.json")
FP8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fp8_decode_traffic.json")
DENSE_SRC = os.path.join(ROOT, "sparse_top_paged_amd", "csrc", "dense.hip")
COPY_CAL_BYTES = 256 << 20
DECODE_SRC = os.path.join(ROOT, "sparse_top_paged_amd", "csrc", "decode.hip")
FP8_SRC = DECODE_SRC


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sets", type=int, default=8, help="candidate sets rotated step by step")
    ap.add_argument("--splits", type=int, default=0, help="0 = library's automatic choice")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    ap.add_argument("--event-every", type=int, default=0,
                    help="bracket the decode kernel with HIP events on every n-th timed step "
                         "(coprime with --sets, so every candidate set is sampled); 0 = no "
                         "events inside the timed steps (the per-kernel split comes from a "
                         "loop of its own)")
    ap.add_argument("--roofline-launches", type=int, default=300,
                    help="event-bracketed decode launches timed for the roofline (at least 200)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=["deepseek", "hot", "locality", "gqa", "transfer",
                                           "fp8", "plan"],
                    default="deepseek",
                    help="deepseek: the headline DeepSeek-shaped step (HBM-resident pool); "
                         "hot: the HiSparse hot-buffer decode (64 requests, 16 steps, pool in "
                         "pinned host memory); locality: the long-context sweep (64 requests, "
                         "context 131072, scattered against clustered top-k, 8 splits); gqa: "
                         "dense paged decode (128 requests, 32 query / 8 KV heads) plus "
                         "prefix-extend (8 x 4096 + 512); transfer: staged bulk host<->device "
                         "transfer of cached prefix rows; fp8: the deepseek step over 656-byte "
                         "fp8_ds_mla rows; plan: the deepseek step through plan/run and HIP graphs, "
                         "plus a ragged batch; the last six are reported on their own lines")
    ap.add_argument("--locality-variant", choices=["both", "scattered", "clustered"],
                    default="both", help="locality workload: which candidate layout to run")
    ap.add_argument("--skip-auto", action="store_true",
                    help="locality workload: time only the 8-split launches (counter runs)")
    ap.add_argument("--passes", type=int, default=6, help="hot workload: timed 16-step passes")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the row-gather and device-copy ceiling measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain device copy of known size, so that rocprofv3 "
                         "counter runs can scale FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(per_launch_alg_bytes, path=TRAFFIC_FILE, src=DECODE_SRC):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    runs, valid only while the kernel source is the one they were taken on."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != source_sha(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def rows_bits(kv, rows):
    """Selected pool rows copied to the host as bf16 bit patterns."""
    import torch
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(kv.device)
    return kv[idx].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(c, rows, host_rows, budget_s):
    import oracle
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        t = done % c.T
        oracle.normalize(c.topk[t:t + 1], c.req_id[t:t + 1], c.q_pos[t:t + 1], c.window,
                         c.num_sinks, c.block_table, c.page_size, c.cap)
        n = len(rows[t])
        oracle.attend_sparse(c.q_bits[t:t + 1], host_rows[t], np.arange(n, dtype=np.int32)[None, :],
                             None, c.scale)
        done += 1
    return done, time.perf_counter() - t0


def cpu_baseline(cases, kv, budget_s):
    """Time the oracle (normalisation + fp64 attention, all 128 heads) on the
    batch's query tokens, cycling through them until the budget is spent; the
    candidate rows are copied to the host first (untimed).  Two settings: all
    the cores this process may use (BLAS at its default thread count), and one
    core (the calling thread pinned to one CPU, BLAS limited to one thread)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle

    c = cases[0]
    ref = oracle.normalize(c.topk, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                           c.page_size, c.cap)
    rows = [ref["slot"][j, :ref["count"][j]] for j in range(c.T)]
    host_rows = [rows_bits(kv, r) for r in rows]
    model = cpu_model()
    avail = sorted(os.sched_getaffinity(0))
    done, el = _oracle_rate(c, rows, host_rows, budget_s)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    one = {}
    try:
        os.sched_setaffinity(0, {avail[0]})
        with threadpool_limits(limits=1):
            d1, e1 = _oracle_rate(c, rows, host_rows, budget_s)
        one = {"value": round(d1 / e1, 2), "unit": "query-tokens/s", "cores": 1,
               "sample": f"{d1} query-token decodes in {e1:.1f} s, thread pinned to CPU {avail[0]}, "
                         f"BLAS limited to one thread"}
    finally:
        os.sched_setaffinity(0, set(avail))
    return {
        "value": round(done / el, 2),
        "unit": "query-tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} query-token decodes (the batch's {c.T} tokens cycled), each "
                  f"normalisation + fp64 attention over all {c.H} heads, {el:.1f} s on the host "
                  f"({len(avail)} CPUs available, BLAS at {threads} threads)",
        "cpu_model": model,
        "one_core": one,
    }


def copy_calibration():
    """A plain device copy of known size (256 MiB read + 256 MiB written, three
    launches), so that rocprofv3 counter runs can scale FETCH_SIZE and
    WRITE_SIZE."""
    import torch
    src = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def median_us(fn, n, sets):
    """Median duration of fn(k) over n launches (HIP events on the current stream)."""
    import torch
    for k in range(8):
        fn(k % sets)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for k in range(n):
        evs[k][0].record()
        fn(k % sets)
        evs[k][1].record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))


def throughput_us(fn, n, sets):
    """Mean time per call of fn(k) over n calls enqueued back to back between
    two HIP events (host launch cost hidden wherever the device is the slower
    side)."""
    import torch
    for k in range(8):
        fn(k % sets)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(n):
        fn(k % sets)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def graph_us(fn, reps=20, replays=20):
    """Device time of fn() for a launch too short to hide the host's launch
    cost: reps calls captured in one HIP graph, the graph replayed between
    two HIP events, divided by reps * replays."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(reps):
                fn()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * replays)


def measure_ceilings(stp, kv, norm, sets, splits, head_groups, n=200):
    """Practical ceilings measured in the same run: the decode's row gather with
    nothing else (the rows of each candidate set read once per head group, as
    the decode reads them, and read once in all), a plain device copy, a
    sequential read of the pool and a bf16 GEMM."""
    import torch

    from sparse_top_paged_amd import diag
    T = norm[0]["slot"].shape[0]
    rows = kv.view(torch.uint8).view(kv.shape[0], -1)
    kv_bytes = [int(nb["count"].sum().item()) * ROW_BYTES for nb in norm]
    mean_kv = float(np.mean(kv_bytes))
    out = {}
    for name, parts, reps in [("row_gather_decode_placement", splits, head_groups),
                              ("row_gather_each_row_once", splits * head_groups, 1)]:
        cs = torch.empty((diag.row_gather_blocks(T, parts, reps),), dtype=torch.int32,
                         device=kv.device)
        us = median_us(lambda k: diag.row_gather(rows, norm[k]["slot"], norm[k]["count"], parts,
                                                reps, checksum=cs), n, sets)
        out[name] = {"us": round(us, 3), "kv_gbs": round(mean_kv / us / 1e3, 1),
                     "parts": parts, "replicas": reps}
    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=kv.device)
    dst = torch.empty_like(src)
    us = median_us(lambda k: dst.copy_(src), 20, 1)
    out["device_copy_256MiB"] = {"us": round(us, 3), "gbs": round(2 * COPY_CAL_BYTES / us / 1e3, 1)}
    del src, dst
    # a plain sequential read of the KV pool (1.2 GB, stp_stream_read): what HBM
    # delivers to a streaming read on this device
    cs_read = torch.empty((2048,), dtype=torch.int32, device=kv.device)
    us = median_us(lambda k: diag.stream_read(kv, 2048, checksum=cs_read), 20, 1)
    nbytes = kv.numel() * kv.element_size()
    out["device_read_pool"] = {"us": round(us, 3), "gbs": round(nbytes / us / 1e3, 1),
                               "bytes": nbytes, "how": "stp_stream_read over the bf16 pool"}
    # the bf16 matrix-core ceiling: a square GEMM through torch (hipBLASLt)
    n_g = 8192
    a = torch.randn((n_g, n_g), dtype=torch.bfloat16, device=kv.device)
    b = torch.randn((n_g, n_g), dtype=torch.bfloat16, device=kv.device)
    us = median_us(lambda k: torch.matmul(a, b), 20, 1)
    out["gemm_bf16_8192"] = {"us": round(us, 3), "tflops": round(2 * n_g ** 3 / us / 1e6, 1),
                             "how": "torch.matmul, bf16, 8192^3"}
    del a, b
    return out


def bench_hot(args):
    """The HiSparse hot-buffer decode: 64 requests, context 65536 + t, 16
    steps whose top-k keeps 85% of the previous set, the whole latent pool
    (4.8 GB) in pinned host memory, a 4096-row hot region per request.  One
    step = the new KV row into its reserved hot row -> normalise -> lookup /
    LRU / swap-in from host memory -> decode over the hot cache (split path)
    -> back-up of the new rows.  Each pass starts cold (state reset), so step
    0 swaps in every candidate row; steps 1-15 are the warm steps."""
    import torch

    import sparse_top_paged_amd as stp
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = workloads.hot_steps_case()
    B, Hs, stride, P, heads = c.batch, c.hot_size, c.region_stride, c.page_size, c.heads
    pool = workloads.pool_torch(c.host_rows, c.pool_seed, dev)
    host = torch.empty((c.host_rows, ROW_BYTES), dtype=torch.uint8, pin_memory=True)
    host.copy_(pool.view(torch.uint8))
    del pool
    torch.cuda.empty_cache()
    host_ptr = stp.host_device_pointer(host)
    hot = torch.zeros((B * stride, ROW_BYTES), dtype=torch.uint8, device=dev)
    kv = hot.view(torch.bfloat16).view(-1, 576)
    dgi = torch.empty((B, Hs), dtype=torch.int32, device=dev)
    lru = torch.empty((B, Hs), dtype=torch.int16, device=dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    table, req = t(c.block_table), t(np.arange(B, dtype=np.int32))
    topk = [t(c.topk[s]) for s in range(c.steps)]
    qpos = [t(c.q_pos(s)) for s in range(c.steps)]
    newest = [t(np.asarray([c.block_table[r][c.q_pos(s)[r] // P] * P + c.q_pos(s)[r] % P
                            for r in range(B)], np.int32)) for s in range(c.steps)]
    q = [t(c.q_bits[s].view(np.int16)).view(torch.bfloat16) for s in range(c.steps)]
    rng = np.random.default_rng(7)
    new_rows = t(workloads.normal_bf16(rng, (c.steps, B, 576)).view(np.uint8)
                 .reshape(c.steps, B, ROW_BYTES))
    reserved = torch.arange(B, device=dev, dtype=torch.int64) * stride + Hs
    src32 = reserved.to(torch.int32)
    S = stp.decode_splits(B, heads, c.cap)
    ws = torch.empty((max(1, stp.decode_workspace_bytes(B, heads, c.cap)),), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, heads, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, heads), dtype=torch.float32, device=dev)
    norm = stp.normalize_indices(topk[0], req, qpos[0], table, P, c.window, c.num_sinks, c.cap,
                                 block_view=False)
    rows = torch.empty((B, c.cap), dtype=torch.int32, device=dev)
    miss = torch.empty((B, c.cap), dtype=torch.uint8, device=dev)
    stats = torch.zeros((c.steps, 2), dtype=torch.int64, device=dev)

    def run_pass(evs=None):
        stp.hot_reset(dgi, lru)
        stats.zero_()
        for s in range(c.steps):
            e = evs[s] if evs else None
            if e:
                e[0].record()
            hot.index_copy_(0, reserved, new_rows[s])
            stp.normalize_indices(topk[s], req, qpos[s], table, P, c.window, c.num_sinks, c.cap,
                                  block_view=False, out=norm)
            if e:
                e[1].record()
            stp.hot_lookup_swapin(host, hot, norm["slot"], newest[s], dgi, lru, stride,
                                  hot_rows_out=rows, miss_mask=miss, stats=stats[s],
                                  host_pool_ptr=host_ptr)
            if e:
                e[2].record()
            stp.sparse_mla_decode(q[s], kv, rows, norm["count"], 576 ** -0.5, S, workspace=ws,
                                  out=out, lse=lse)
            if e:
                e[3].record()
            stp.backup_rows(hot, host, src32, newest[s], host_pool_ptr=host_ptr)
            if e:
                e[4].record()

    # The same steps with each step's lookup / swap-in moved to a side stream,
    # chunk by chunk over the request rows: chunk k+1 swaps in while chunk k
    # decodes on the main stream (HIP events order them; the next step's first
    # swap-in follows the back-up through the step's normalisation).  A chunk's
    # decode runs with a split count that keeps its grid beside the swap-in
    # workgroups still resident.
    side = torch.cuda.Stream()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    groups = (heads + 63) // 64

    def run_pass_overlap(chunks, evs=None):
        bounds = np.linspace(0, B, chunks + 1).astype(int)
        per = int(np.max(np.diff(bounds)))
        sp = max(1, (cus - per) // (per * groups))
        sp = max(sp, stp.decode_splits(per, heads, c.cap, 1))
        stp.hot_reset(dgi, lru)
        stats.zero_()
        main = torch.cuda.current_stream()
        for s in range(c.steps):
            e = evs[s] if evs else None
            if e:
                e[0].record()
            hot.index_copy_(0, reserved, new_rows[s])
            stp.normalize_indices(topk[s], req, qpos[s], table, P, c.window, c.num_sinks, c.cap,
                                  block_view=False, out=norm)
            side.wait_event(main.record_event())
            for k in range(chunks):
                r0, r1 = int(bounds[k]), int(bounds[k + 1])
                with torch.cuda.stream(side):
                    stp.hot_lookup_swapin(host, hot[r0 * stride:r1 * stride],
                                          norm["slot"][r0:r1], newest[s][r0:r1], dgi[r0:r1],
                                          lru[r0:r1], stride, hot_rows_out=rows[r0:r1],
                                          miss_mask=miss[r0:r1], stats=stats[s],
                                          host_pool_ptr=host_ptr)
                    swapped = side.record_event()
                main.wait_event(swapped)
                kvc = hot[r0 * stride:r1 * stride].view(torch.bfloat16).view(-1, 576)
                stp.sparse_mla_decode(q[s][r0:r1], kvc, rows[r0:r1], norm["count"][r0:r1],
                                      576 ** -0.5, sp, workspace=ws_chunk, out=out[r0:r1],
                                      lse=lse[r0:r1])
            stp.backup_rows(hot, host, src32, newest[s], host_pool_ptr=host_ptr)
            if e:
                e[1].record()
        return sp

    ws_chunk = torch.empty((max(1, max(stp.decode_workspace_bytes(B // ch, heads, c.cap, sp_)
                                           for ch in (2, 4) for sp_ in range(1, 17))),),
                           dtype=torch.uint8, device=dev)

    run_pass()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    per_step = []  # (total, normalise, lookup+swap-in, decode, back-up) in us, per pass and step
    st_all = []
    for _ in range(args.passes):
        evs = [[ev() for _ in range(5)] for _ in range(c.steps)]
        run_pass(evs)
        torch.cuda.synchronize()
        per_step.append([[evs[s][0].elapsed_time(evs[s][4]) * 1e3] +
                         [evs[s][k].elapsed_time(evs[s][k + 1]) * 1e3 for k in range(4)]
                         for s in range(c.steps)])
        st_all.append(stats.cpu().numpy().copy())
    overlap = {}
    for chunks in (2, 4):
        run_pass_overlap(chunks)
        torch.cuda.synchronize()
        tot = []
        for _ in range(args.passes):
            evs = [[ev() for _ in range(2)] for _ in range(c.steps)]
            sp = run_pass_overlap(chunks, evs)
            torch.cuda.synchronize()
            tot.append([evs[s][0].elapsed_time(evs[s][1]) * 1e3 for s in range(c.steps)])
            st_ov = stats.cpu().numpy().copy()
        tot = np.asarray(tot)
        overlap[f"chunks_{chunks}"] = {
            "warm_step_us": round(float(np.median(tot[:, 1:])), 2),
            "cold_step_us": round(float(np.median(tot[:, 0])), 1),
            "decode_splits_per_chunk": int(sp),
            "same_hit_miss_counts_as_serial": bool(np.array_equal(st_ov, st_all[-1])),
        }
    a = np.asarray(per_step)         # [passes, steps, 5]
    st = np.asarray(st_all)          # [passes, steps, 2]
    warm = a[:, 1:, :].reshape(-1, 5)
    hits, misses = st[:, 1:, 0].sum(), st[:, 1:, 1].sum()
    miss_per_step = misses / (args.passes * (c.steps - 1))
    swap_us = float(np.median(warm[:, 2]))
    cold_swap_us = float(np.median(a[:, 0, 2]))
    cold_misses = float(st[:, 0, 1].mean())
    # host link ceiling in the same run: pinned host -> device copies of 64 MiB
    link = torch.empty((64 << 20,), dtype=torch.uint8, pin_memory=True)
    dst = torch.empty((64 << 20,), dtype=torch.uint8, device=dev)
    h2d_us = median_us(lambda k: dst.copy_(link, non_blocking=True), 20, 1)
    step_us = float(np.median(warm[:, 0]))
    res = {
        "metric": METRIC,
        "value": round(B / (step_us * 1e-6), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": int(args.passes * (c.steps - 1)),
        "warmup": int(c.steps + 1),
        "ms_per_step": round(step_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hisparse hot-buffer decode, one layer, warm steps", "batch": B,
                   "query_heads": heads, "context": c.ctx0, "steps_per_pass": c.steps,
                   "top_k": c.top_k, "window": c.window, "sinks": c.num_sinks,
                   "hot_rows_per_request": Hs, "host_pool_bytes": int(c.host_rows * ROW_BYTES),
                   "splits": S},
        "hot": {
            "hit_rate_warm_steps": round(float(hits / (hits + misses)), 4),
            "misses_per_warm_step": round(float(miss_per_step), 1),
            "warm_step_us": {k: round(float(np.median(warm[:, i])), 2) for i, k in
                             enumerate(["total", "normalise", "lookup_swapin", "decode_merge",
                                        "backup"])},
            "swapin_gbs_warm": round(miss_per_step * ROW_BYTES / swap_us / 1e3, 2),
            "cold_step_us": round(float(np.median(a[:, 0, 0])), 1),
            "cold_swapin_gbs": round(cold_misses * ROW_BYTES / cold_swap_us / 1e3, 2),
            "pinned_h2d_copy_gbs": round((64 << 20) / h2d_us / 1e3, 2),
            "side_stream_overlap": overlap,
            "serial_warm_step_us": round(step_us, 2),
        },
    }
    print(json.dumps(res), flush=True)


def bench_locality(args):
    """The long-context locality sweep: 64 requests at context 131072 (page
    64, a 9.66 GB pool in HBM), top-k 2048 only, either scattered uniformly or
    clustered as 128 runs of 16 consecutive positions; decode with 8 splits,
    then the merge.  Four candidate draws per layout rotate (the same tables
    and queries).  Reports per layout the normalisation, decode and merge
    times, the requested KV bytes and rate, and the page-granular efficiency
    eta_blk = k / (u P) of loading whole touched pages instead of rows
    ("5.1.1 · 从索引到 Kernel" §7.4 eq. (18))."""
    import torch

    import sparse_top_paged_amd as stp
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S = 8
    nsets = 4
    variants = ["scattered", "clustered"] if args.locality_variant == "both" else \
        [args.locality_variant]
    base = {v: workloads.locality_case(4001 if v == "scattered" else 4002, v == "clustered")
            for v in variants}
    c0 = base[variants[0]]
    kv = workloads.pool_torch(c0.kv_rows, c0.pool_seed, dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    res_v = {}
    for v in variants:
        c = base[v]
        T, H, cap, P = c.T, c.H, c.cap, c.page_size
        ctx = int(c.q_pos[0]) + 1
        draws = [c.topk]
        for d in range(1, nsets):
            rng = np.random.default_rng((4001 if v == "scattered" else 4002) * 100 + d)
            if v == "clustered":
                draws.append(np.stack([workloads.clustered_topk(rng, ctx, c.top_k)
                                       for _ in range(T)]))
            else:
                draws.append(np.stack([rng.choice(ctx, size=c.top_k, replace=False)
                                       .astype(np.int32) for _ in range(T)]))
        q = t(c.q_bits.view(np.int16)).view(torch.bfloat16)
        req, qpos, table = t(c.req_id), t(c.q_pos), t(c.block_table)
        topk = [t(d) for d in draws]
        norm = [stp.normalize_indices(tk, req, qpos, table, P, 0, 0, cap) for tk in topk]
        torch.cuda.synchronize()
        sel = np.asarray([int(n["count"].sum().item()) for n in norm], np.float64)
        blocks = np.asarray([int(n["blk_indptr"][-1].item()) for n in norm], np.float64)
        o_norm = torch.empty((T, S, H, 512), dtype=torch.bfloat16, device=dev)
        m_part = torch.empty((T, S, H), dtype=torch.float32, device=dev)
        l_part = torch.empty((T, S, H), dtype=torch.float32, device=dev)
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        n_us = median_us(lambda k: stp.normalize_indices(topk[k], req, qpos, table, P, 0, 0, cap,
                                                         out=norm[k]), 200, nsets)
        d_us = median_us(lambda k: stp.sparse_mla_decode_partial_normalized(
            q, kv, norm[k]["slot"], norm[k]["count"], c.scale, S, o_norm, m_part, l_part),
            200, nsets)
        m_us = median_us(lambda k: stp.splitkv_merge_normalized(o_norm, m_part, l_part, out, lse),
                         200, nsets)
        # the automatic split choice through the public entry point (decode + merge)
        s_auto = stp.decode_splits(T, H, cap)
        a_us = float("nan")
        if not args.skip_auto:
            ws = torch.empty((max(1, stp.decode_workspace_bytes(T, H, cap)),), dtype=torch.uint8,
                             device=dev)
            a_us = median_us(lambda k: stp.sparse_mla_decode(
                q, kv, norm[k]["slot"], norm[k]["count"], c.scale, 0, workspace=ws, out=out,
                lse=lse), 200, nsets)
        kv_bytes = float(sel.mean()) * ROW_BYTES
        alg = kv_bytes + T * H * 576 * 2 + float(sel.mean()) * 4
        part_bytes = T * S * H * (512 * 2 + 8)
        res_v[v] = {
            "normalise_us": round(n_us, 2),
            "decode_us": round(d_us, 2),
            "merge_us": round(m_us, 2),
            "selected_rows_per_token": round(float(sel.mean()) / T, 1),
            "touched_pages_per_token": round(float(blocks.mean()) / T, 1),
            "eta_blk": round(float(sel.mean() / (blocks.mean() * P)), 4),
            "requested_kv_bytes": int(kv_bytes),
            "page_granular_kv_bytes": int(blocks.mean() * P * ROW_BYTES),
            "decode_kv_gbs": round(kv_bytes / d_us / 1e3, 1),
            "decode_alg_gbs": round(alg / d_us / 1e3, 1),
            "decode_frac_of_hbm_peak": round(alg / d_us / 1e3 / HBM_PEAK_GBS, 4),
            "partial_bytes_each_way": int(part_bytes),
            "merge_gbs": round((part_bytes + T * H * (512 * 2 + 4)) / m_us / 1e3, 1),
            "auto_splits": s_auto,
            "auto_decode_and_merge_us": None if args.skip_auto else round(a_us, 2),
        }
    step_us = res_v[variants[0]]["normalise_us"] + res_v[variants[0]]["decode_us"] + \
        res_v[variants[0]]["merge_us"]
    res = {
        "metric": METRIC,
        "value": round(c0.T / (step_us * 1e-6), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": 200,
        "warmup": 8,
        "ms_per_step": round(step_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"long-context locality sweep ({variants[0]} rate as value)",
                   "batch": c0.T, "query_heads": c0.H, "context": int(c0.q_pos[0]) + 1,
                   "page_size": c0.page_size, "top_k": c0.top_k, "splits": S,
                   "candidate_sets": nsets, "kv_pool_rows": c0.kv_rows},
        "locality": res_v,
    }
    print(json.dumps(res), flush=True)


def bench_gqa(args):
    """Dense paged attention with grouped query heads: 32 query and 8 KV heads
    of dimension 128, fp16, page size 16, random block tables.  Decode: 128
    requests, contexts uniform in [1024, 4096] (1.35 GB of K and V read per
    launch, beyond the 256 MB Infinity Cache); extend: 8 requests of a 4096-token
    cached prefix + 512 new tokens under the shifted causal mask.  A step is
    one decode launch and one extend launch; each kernel is timed alone with
    HIP events (median over launches).  `value` is decode query tokens per
    second; the decode roofline is HBM bytes (K, V, queries, outputs, the
    block table) against 8 TB/s, the extend roofline fp16 MFMA flops of the
    visible (query, key) pairs against 2.5 PFLOP/s.  The ceiling times the
    plain gather of the decode's K and V rows (stp_row_gather, no
    arithmetic)."""
    import torch

    import sparse_top_paged_amd as stp
    import workloads
    from sparse_top_paged_amd import diag

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    n_launch = max(20, min(args.steps, 200))
    # decode
    c = workloads.gqa_decode_case()
    B, Hq, Hkv = c.q.shape[0], c.q.shape[1], c.hkv
    kd, vd = workloads.dense_pool_torch(c.num_slots, Hkv, c.pool_seed, dev)
    q, tab, ctx = t(c.q), t(c.block_table), t(c.ctx_lens)
    S = stp.paged_gqa_decode_splits(B, Hkv, tab.shape[1], c.page_size, args.splits)
    ws = torch.empty((max(1, stp.paged_gqa_decode_workspace_bytes(B, Hq, Hkv, tab.shape[1],
                                                                  c.page_size, S)),),
                     dtype=torch.uint8, device=dev)
    out, lse = stp.paged_gqa_decode(q, kd, vd, tab, ctx, c.page_size, c.scale, S, ws)
    d_us = median_us(lambda k: stp.paged_gqa_decode(q, kd, vd, tab, ctx, c.page_size, c.scale, S,
                                                    ws, out=out, lse=lse), n_launch, 1)
    tokens = int(c.ctx_lens.astype(np.int64).sum())
    kv_bytes = tokens * Hkv * 128 * 2 * 2
    d_alg = kv_bytes + B * Hq * 128 * 2 * 2 + B * Hq * 4 + int(np.sum(-(-c.ctx_lens // c.page_size))) * 4
    ceil_us = None
    if not args.no_ceilings:
        ids = np.full((B * Hkv, int(c.ctx_lens.max())), -1, np.int32)
        for b in range(B):
            n = int(c.ctx_lens[b])
            t_ = np.arange(n)
            sl = c.block_table[b][t_ // c.page_size].astype(np.int64) * c.page_size + t_ % c.page_size
            for g in range(Hkv):
                ids[b * Hkv + g, :n] = sl * Hkv + g
        ids_d, cnt_d = t(ids), t(np.repeat(c.ctx_lens, Hkv).astype(np.int32))
        krows, vrows = kd.view(torch.uint8).view(-1, 256), vd.view(torch.uint8).view(-1, 256)
        ceil_us = median_us(lambda k: (diag.row_gather(krows, ids_d, cnt_d, parts=2),
                                       diag.row_gather(vrows, ids_d, cnt_d, parts=2)), n_launch, 1)
        del ids_d
    traffic = load_traffic(d_alg, GQA_TRAFFIC_FILE, DENSE_SRC)
    del kd, vd
    torch.cuda.empty_cache()
    # extend
    e = workloads.extend_case()
    ke, ve = workloads.dense_pool_torch(e.num_slots, e.hkv, e.pool_seed, dev)
    qe, qo, kvp, kvi = t(e.q), t(e.qo_indptr), t(e.kv_indptr), t(e.kv_indices)
    oe, le = stp.extend_attention(qe, ke, ve, qo, kvp, kvi, e.max_extend_len, e.scale)
    e_us = median_us(lambda k: stp.extend_attention(qe, ke, ve, qo, kvp, kvi, e.max_extend_len,
                                                    e.scale, out=oe, lse=le), n_launch, 1)
    pairs = 0
    for b in range(len(e.qo_indptr) - 1):
        lq = int(e.qo_indptr[b + 1] - e.qo_indptr[b])
        lk = int(e.kv_indptr[b + 1] - e.kv_indptr[b])
        pairs += sum(max(0, min(lk, lk - lq + i + 1)) for i in range(lq))
    e_flops = pairs * e.q.shape[1] * 128 * 4
    step_us = d_us + e_us
    res = {
        "metric": METRIC,
        "value": round(B / (d_us * 1e-6), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": n_launch,
        "warmup": 8,
        "ms_per_step": round(step_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "dense paged GQA decode (value) + prefix-extend",
                   "query_heads": Hq, "kv_heads": Hkv, "head_dim": 128, "page_size": c.page_size,
                   "decode_batch": B, "decode_context": "uniform 1024..4096",
                   "decode_partitions": S, "extend_batch": len(e.qo_indptr) - 1,
                   "extend_prefix": 4096, "extend_new_tokens": 512},
        "roofline": {"bound": "hbm", "achieved": round(d_alg / d_us / 1e3, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(d_alg / d_us / 1e3 / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "paged_gqa_decode_kernel",
                     "bytes_per_launch": d_alg},
        "roofline_extend": {"bound": "mfma", "achieved": round(e_flops / e_us / 1e6, 1),
                            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(e_flops / e_us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                            "kernel": "extend_attention_kernel", "flops_per_launch": e_flops},
        "decode_us": round(d_us, 2),
        "extend_us": round(e_us, 2),
        "extend_tokens_per_s": round(int(e.qo_indptr[-1]) / (e_us * 1e-6), 1),
        "ceilings": None if ceil_us is None else {
            "kv_row_gather_us": round(ceil_us, 2),
            "kv_row_gather_gbs": round(kv_bytes / ceil_us / 1e3, 1),
            "decode_vs_gather": round(ceil_us / d_us, 4)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = gqa_cpu_baseline(c, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def bench_transfer(args):
    """Staged bulk host <-> device transfer (HiCache-style layer-wise prefix
    load): 8 layers x 16384 rows of 1152 B (bf16 MLA rows, page size 64;
    151 MB per call) between a pinned host pool of 65536 rows per layer and a
    device pool of 32768 rows per layer.  Rows are whole pages of a random
    page table, or fully scattered rows.  Reported: host-to-device and
    device-to-host GB/s for 1..16 workgroups, against hipMemcpyAsync of the
    same bytes as one contiguous copy (the copy engines; the link's
    ceiling)."""
    import torch

    import sparse_top_paged_amd as stp

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, hrows, drows, n, rb, page = 8, 65536, 32768, 16384, 1152, 64
    rng = np.random.default_rng(6000)
    host = torch.empty((L, hrows, rb), dtype=torch.uint8, pin_memory=True)
    g = torch.Generator().manual_seed(6001)
    for l in range(L):
        host[l] = torch.randint(0, 256, (hrows, rb), dtype=torch.uint8, generator=g)
    devp = torch.empty((L, drows, rb), dtype=torch.uint8, device=dev)
    hb, db = [host[l] for l in range(L)], [devp[l] for l in range(L)]
    pages = rng.permutation(hrows // page)[: n // page]
    runs = (pages[:, None] * page + np.arange(page)[None, :]).reshape(-1).astype(np.int32)
    scat = rng.choice(hrows, size=n, replace=False).astype(np.int32)
    dpos = np.arange(n, dtype=np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    runs_d, scat_d, dpos_d = t(runs), t(scat), t(dpos)
    nbytes = L * n * rb
    n_launch = 20
    res = {}
    for blocks in [1, 2, 4, 8, 16]:
        r = {}
        us = median_us(lambda k: stp.kv_transfer(hb, db, runs_d, dpos_d, num_blocks=blocks),
                       n_launch, 1)
        r["h2d_pages_gbs"] = round(nbytes / us / 1e3, 2)
        us = median_us(lambda k: stp.kv_transfer(hb, db, scat_d, dpos_d, num_blocks=blocks),
                       n_launch, 1)
        r["h2d_scattered_gbs"] = round(nbytes / us / 1e3, 2)
        us = median_us(lambda k: stp.kv_transfer(db, hb, dpos_d, runs_d, num_blocks=blocks),
                       n_launch, 1)
        r["d2h_pages_gbs"] = round(nbytes / us / 1e3, 2)
        res[str(blocks)] = r
    src_h = host.view(-1)[:nbytes]
    dst_d = devp.view(-1)[:nbytes]
    h2d_us = median_us(lambda k: dst_d.copy_(src_h, non_blocking=True), n_launch, 1)
    d2h_us = median_us(lambda k: src_h.copy_(dst_d, non_blocking=True), n_launch, 1)
    out = {
        "metric": "staged host<->device KV transfer GB/s, 1 MI355X",
        "value": res["4"]["h2d_pages_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n_launch,
        "warmup": 8,
        "ms_per_step": round(nbytes / res["4"]["h2d_pages_gbs"] / 1e6, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "layer-wise prefix load host->device, page runs, 4 workgroups "
                               "(value)", "layers": L, "rows_per_layer": n, "row_bytes": rb,
                   "page_size": page, "bytes_per_call": nbytes},
        "by_workgroups": res,
        "copy_engine": {"h2d_gbs": round(nbytes / h2d_us / 1e3, 2),
                        "d2h_gbs": round(nbytes / d2h_us / 1e3, 2)},
    }
    print(json.dumps(out), flush=True)


def bench_fp8(args):
    """The DeepSeek-shaped step over fp8_ds_mla rows: the same 32 tokens, 128
    heads, context 32768, top-k 2048 + 128 + 4, page 64, with a 1,048,576-row
    pool of 656-byte rows (688 MB) instead of 1152-byte bf16 rows (1.21 GB).
    Eight candidate sets rotate.  Timed: the normalisation (median of HIP
    event pairs), and each decode entry point with its automatic splits
    (decode + merge, calls back to back between two HIP events): fp8 rows and,
    for comparison, bf16 rows of the same shape.  KV bytes per call: selected rows x 656 (fp8) or x 1152 (bf16)."""
    import torch

    import sparse_top_paged_amd as stp
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nsets = args.sets
    cases = [workloads.deepseek_case(variant=v) for v in range(nsets)]
    c0 = cases[0]
    T, H, cap = c0.T, c0.H, c0.cap
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    q = t(c0.q_bits.view(np.int16)).view(torch.bfloat16)
    req, qpos, table = t(c0.req_id), t(c0.q_pos), t(c0.block_table)
    norm = [stp.normalize_indices(t(c.topk), req, qpos, table, c0.page_size, c0.window,
                                  c0.num_sinks, cap) for c in cases]
    torch.cuda.synchronize()
    sel = float(np.mean([int(n["count"].sum().item()) for n in norm]))
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    n_launch = max(50, min(args.steps, 400))
    kv8 = workloads.fp8_pool_torch(c0.kv_rows, c0.pool_seed, dev)
    s8 = stp.decode_fp8_splits(T, H, cap)
    ws8 = torch.empty((max(1, stp.decode_fp8_workspace_bytes(T, H, cap)),), dtype=torch.uint8,
                      device=dev)
    f_us = throughput_us(lambda k: stp.sparse_mla_decode_fp8(q, kv8, norm[k]["slot"],
                                                             norm[k]["count"], c0.scale, 0, ws8,
                                                             out, lse), n_launch, nsets)
    # the split merge of the same partial states on its own, so that the fp8
    # decode kernel's launch time is the call's time less the merge's
    n_part = T * s8 * H
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    o_norm = ws8[:n_part * 512 * 2].view(torch.bfloat16).view(T, s8, H, 512)
    m_part = ws8[a256(n_part * 1024):a256(n_part * 1024) + n_part * 4].view(torch.float32)
    l_off = a256(n_part * 1024) + a256(n_part * 4)
    l_part = ws8[l_off:l_off + n_part * 4].view(torch.float32)
    merge_us = graph_us(lambda: stp.splitkv_merge_normalized(
        o_norm, m_part.view(T, s8, H), l_part.view(T, s8, H), out, lse)) if s8 > 1 else 0.0
    dec8_us = f_us - merge_us
    del kv8
    torch.cuda.empty_cache()
    kvb = workloads.pool_torch(c0.kv_rows, c0.pool_seed, dev)
    sb = stp.decode_splits(T, H, cap)
    wsb = torch.empty((max(1, stp.decode_workspace_bytes(T, H, cap)),), dtype=torch.uint8,
                      device=dev)
    b_us = throughput_us(lambda k: stp.sparse_mla_decode(q, kvb, norm[k]["slot"],
                                                         norm[k]["count"], c0.scale, 0, wsb, out,
                                                         lse), n_launch, nsets)
    topks = [t(c.topk) for c in cases]
    n_us = median_us(lambda k: stp.normalize_indices(topks[k], req, qpos, table, c0.page_size,
                                                     c0.window, c0.num_sinks, cap, out=norm[k]),
                     n_launch, nsets)
    q_bytes = T * H * 576 * 2
    alg8 = sel * 656 + q_bytes + sel * 4
    step_us = n_us + f_us
    traffic8 = load_traffic(alg8, FP8_TRAFFIC_FILE, FP8_SRC)
    res = {
        "metric": METRIC,
        "value": round(T / (step_us * 1e-6), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": n_launch,
        "warmup": 8,
        "ms_per_step": round(step_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "deepseek-v3.2-shaped sparse MLA decode over fp8_ds_mla rows",
                   "batch": T, "query_heads": H, "context": 32768, "page_size": c0.page_size,
                   "top_k": c0.top_k, "row_bytes": 656, "kv_pool_rows": c0.kv_rows,
                   "splits": s8, "candidate_sets": nsets,
                   "mean_selected_rows_per_token": round(sel / T, 2)},
        "roofline": {"kernel": "sparse_mla_decode_kernel (fp8 rows)", "bound": "hbm",
                     "achieved": round(alg8 / dec8_us / 1e3, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(alg8 / dec8_us / 1e3 / 8000.0, 4), "traffic": traffic8,
                     "algorithmic_bytes_per_launch": int(alg8),
                     "avg_launch_us": round(dec8_us, 3),
                     "launch_time": "decode + merge call (calls back to back between two "
                                    "HIP events) less the merge's device time (20 merges in "
                                    "one HIP graph)"},
        "normalise_us": round(n_us, 2),
        "fp8_decode_and_merge_us": round(f_us, 2),
        "fp8_merge_us": round(merge_us, 2),
        "bf16_decode_and_merge_us": round(b_us, 2),
        "bf16_splits": sb,
        "kv_bytes_fp8": int(sel * 656),
        "kv_bytes_bf16": int(sel * ROW_BYTES),
        "byte_ratio": round(656 / ROW_BYTES, 4),
        "time_ratio": round(f_us / b_us, 4),
        "fp8_alg_gbs": round(alg8 / f_us / 1e3, 1),
    }
    print(json.dumps(res), flush=True)


def bench_plan(args):
    """Plan / run against the static split decode.

    DeepSeek-shaped step (32 tokens, 128 heads, |S| ~ 2172, eight candidate
    sets rotating): normalise (no block view) then either the static decode
    with automatic splits, or plan + run with the task size
    decode_plan_rows_per_task picks; eager, and the whole step replayed from
    HIP graphs (one per candidate set, each bound to its own top-k buffer).
    Ragged batch (128 tokens: 120 with |S| = 96, 8 with |S| ~ 2180, four
    candidate sets): the static decode with automatic splits against plan +
    run at several task sizes.  Mean time per call over calls enqueued back to
    back between two HIP events."""
    import torch

    import sparse_top_paged_amd as stp
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    n_launch = max(50, min(args.steps, 400))

    def setup(cases):
        c0 = cases[0]
        q = t(c0.q_bits.view(np.int16)).view(torch.bfloat16)
        req, qpos, table = t(c0.req_id), t(c0.q_pos), t(c0.block_table)
        topk = [t(c.topk) for c in cases]
        norm = [stp.normalize_indices(tk, req, qpos, table, c0.page_size, c0.window,
                                      c0.num_sinks, c0.cap, block_view=False) for tk in topk]
        return c0, q, req, qpos, table, topk, norm

    def normalise(c0, req, qpos, table, topk, norm, k):
        stp.normalize_indices(topk[k], req, qpos, table, c0.page_size, c0.window, c0.num_sinks,
                              c0.cap, block_view=False, out=norm[k])

    res_extra = {}
    # ---- DeepSeek-shaped step ----
    nsets = args.sets
    cases = [workloads.deepseek_case(variant=v) for v in range(nsets)]
    c0, q, req, qpos, table, topk, norm = setup(cases)
    T, H, cap = c0.T, c0.H, c0.cap
    kv = workloads.pool_torch(c0.kv_rows, c0.pool_seed, dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws_s = torch.empty((max(1, stp.decode_workspace_bytes(T, H, cap)),), dtype=torch.uint8,
                       device=dev)
    R = stp.decode_plan_rows_per_task(T, H, cap)
    plan = torch.empty((stp.decode_plan_bytes(T, cap, R) // 4,), dtype=torch.int32, device=dev)
    ws_r = torch.empty((max(1, stp.decode_run_workspace_bytes(T, H, cap, R)),), dtype=torch.uint8,
                       device=dev)

    def static_step(k):
        normalise(c0, req, qpos, table, topk, norm, k)
        stp.sparse_mla_decode(q, kv, norm[k]["slot"], norm[k]["count"], c0.scale, 0, ws_s, out,
                              lse)

    def plan_step(k):
        normalise(c0, req, qpos, table, topk, norm, k)
        stp.decode_plan(norm[k]["count"], T, cap, R, plan=plan)
        stp.decode_run(q, kv, norm[k]["slot"], plan, R, c0.scale, ws_r, out, lse)

    def graphs(step):
        gs = []
        s = torch.cuda.Stream()
        for k in range(nsets):
            step(k)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    step(k)
            torch.cuda.current_stream().wait_stream(s)
            gs.append(g)
        torch.cuda.synchronize()
        return gs

    static_us = throughput_us(static_step, n_launch, nsets)
    plan_us = throughput_us(plan_step, n_launch, nsets)
    g_plan = graphs(plan_step)
    graph_us = throughput_us(lambda k: g_plan[k].replay(), n_launch, nsets)
    g_static = graphs(static_step)
    static_graph_us = throughput_us(lambda k: g_static[k].replay(), n_launch, nsets)

    def run_only(k):
        stp.decode_plan(norm[k]["count"], T, cap, R, plan=plan)
        stp.decode_run(q, kv, norm[k]["slot"], plan, R, c0.scale, ws_r, out, lse)

    plan_run_us = throughput_us(run_only, n_launch, nsets)
    static_dec_us = throughput_us(lambda k: stp.sparse_mla_decode(q, kv, norm[k]["slot"],
                                                                  norm[k]["count"], c0.scale, 0,
                                                                  ws_s, out, lse),
                                  n_launch, nsets)
    del g_plan, g_static, kv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # ---- ragged batch ----
    rsets = 4
    rcases = [workloads.ragged_case(variant=v) for v in range(rsets)]
    r0, rq, rreq, rqpos, rtable, rtopk, rnorm = setup(rcases)
    for k in range(rsets):
        normalise(r0, rreq, rqpos, rtable, rtopk, rnorm, k)
    torch.cuda.synchronize()
    rT, rcap = r0.T, r0.cap
    rkv = workloads.pool_torch(r0.kv_rows, r0.pool_seed, dev)
    rout = torch.empty((rT, H, 512), dtype=torch.bfloat16, device=dev)
    rlse = torch.empty((rT, H), dtype=torch.float32, device=dev)
    rws = torch.empty((max(1, stp.decode_workspace_bytes(rT, H, rcap)),), dtype=torch.uint8,
                      device=dev)
    r_static = throughput_us(lambda k: stp.sparse_mla_decode(rq, rkv, rnorm[k]["slot"],
                                                         rnorm[k]["count"], r0.scale, 0, rws,
                                                         rout, rlse), n_launch, rsets)
    r_sel = float(np.mean([int(nb["count"].sum().item()) for nb in rnorm]))
    r_runs = {}
    for rr in (128, 256, 512, 1024):
        rplan = torch.empty((stp.decode_plan_bytes(rT, rcap, rr) // 4,), dtype=torch.int32,
                            device=dev)
        rwr = torch.empty((max(1, stp.decode_run_workspace_bytes(rT, H, rcap, rr)),),
                          dtype=torch.uint8, device=dev)

        def rstep(k, rr=rr, rplan=rplan, rwr=rwr):
            stp.decode_plan(rnorm[k]["count"], rT, rcap, rr, plan=rplan)
            stp.decode_run(rq, rkv, rnorm[k]["slot"], rplan, rr, r0.scale, rwr, rout, rlse)

        r_runs[str(rr)] = round(throughput_us(rstep, n_launch, rsets), 2)
        del rplan, rwr
    best_r = min(r_runs, key=lambda x: r_runs[x])
    res_extra.update({
        "ragged_batch": rT, "ragged_mean_selected_rows": round(r_sel / rT, 2),
        "ragged_static_decode_us": round(r_static, 2),
        "ragged_plan_run_us_by_rows_per_task": r_runs,
        "ragged_best_speedup": round(r_static / r_runs[best_r], 3),
    })
    res = {
        "metric": METRIC,
        "value": round(T / (graph_us * 1e-6), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": n_launch,
        "warmup": 8,
        "ms_per_step": round(graph_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "deepseek-v3.2-shaped step (normalise + plan + run) replayed "
                               "from HIP graphs",
                   "batch": T, "query_heads": H, "context": 32768, "page_size": c0.page_size,
                   "top_k": c0.top_k, "rows_per_task": R, "candidate_sets": nsets},
        "static_step_us": round(static_us, 2),
        "plan_step_us": round(plan_us, 2),
        "graph_step_us": round(graph_us, 2),
        "static_graph_step_us": round(static_graph_us, 2),
        "plan_and_run_us": round(plan_run_us, 2),
        "static_decode_and_merge_us": round(static_dec_us, 2),
    }
    res.update(res_extra)
    print(json.dumps(res), flush=True)


def gqa_cpu_baseline(c, budget_s):
    """The dense decode oracle on the host, one request at a time (its rows
    from the same seeded pool, regenerated on the host for the pages the
    request maps), cycling through the batch until the budget is spent."""
    from threadpoolctl import threadpool_info

    import oracle
    import workloads

    pool_k, pool_v = workloads.dense_pool(min(c.num_slots, 1 << 15), c.hkv, c.pool_seed)
    done, t0 = 0, time.perf_counter()
    B = c.q.shape[0]
    while time.perf_counter() - t0 < budget_s:
        b = done % B
        n = int(c.ctx_lens[b])
        # the request's tokens laid on consecutive slots of a host pool (the
        # arithmetic is the same for any slot mapping)
        tab = np.arange(-(-n // c.page_size), dtype=np.int32)[None, :]
        oracle.paged_gqa_decode(c.q[b:b + 1], pool_k, pool_v, tab, np.asarray([n], np.int32),
                                c.page_size, c.scale)
        done += 1
    el = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": round(done / el, 2),
        "unit": "query-tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} request decodes (the batch's {B} requests cycled, contexts "
                  f"1024..4096, all {c.q.shape[1]} heads, fp64), {el:.1f} s on the host",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the decode path "
              "has no multi-GPU mode (it would shard by request, with no exchange).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
    if args.workload == "hot":
        bench_hot(args)
        return
    if args.workload == "locality":
        bench_locality(args)
        return
    if args.workload == "gqa":
        bench_gqa(args)
        return
    if args.workload == "transfer":
        bench_transfer(args)
        return
    if args.workload == "fp8":
        bench_fp8(args)
        return
    if args.workload == "plan":
        bench_plan(args)
        return

    import torch

    import sparse_top_paged_amd as stp
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cases = [workloads.deepseek_case(variant=v) for v in range(args.sets)]
    c0 = cases[0]
    T, H, cap = c0.T, c0.H, c0.cap
    kv = workloads.pool_torch(c0.kv_rows, c0.pool_seed, dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    q = t(c0.q_bits.view(np.int16)).view(torch.bfloat16)
    req, qpos, table = t(c0.req_id), t(c0.q_pos), t(c0.block_table)
    topks = [t(c.topk) for c in cases]

    S = stp.decode_splits(T, H, cap, args.splits)
    norm = [stp.normalize_indices(tk, req, qpos, table, c0.page_size, c0.window, c0.num_sinks,
                                  cap) for tk in topks]
    # the split path of stp_normalize_and_decode, called stage by stage so
    # that its decode launch can be timed on its own: normalised bf16
    # partials, then the merge
    o_norm = torch.empty((T, S, H, 512), dtype=torch.bfloat16, device=dev)
    m_part = torch.empty((T, S, H), dtype=torch.float32, device=dev)
    l_part = torch.empty((T, S, H), dtype=torch.float32, device=dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    counts = [n["count"].cpu().numpy().astype(np.int64) for n in norm]

    # One step: the normalisation inside the decode launch (block view
    # deferred), then the merge and the block view in one launch; a single
    # pass completes the block view in a launch of its own.
    def fused(k):
        if S > 1:
            return stp.normalize_and_decode_partial_normalized(
                topks[k], req, qpos, table, c0.page_size, c0.window, c0.num_sinks, q, kv,
                c0.scale, S, o_norm, m_part, l_part, cap, norm=norm[k])
        stp.normalize_and_decode(topks[k], req, qpos, table, c0.page_size, c0.window,
                                 c0.num_sinks, q, kv, c0.scale, 1, cap, norm=norm_lists[k],
                                 out=out, lse=lse)
        return norm[k]

    norm_lists = [{key: nb[key] for key in ("tok", "slot", "count", "dropped")} for nb in norm]

    def step(i, ev=None):
        k = i % args.sets
        if ev is not None:
            ev[0].record()
        nb = fused(k)
        if ev is not None:
            ev[1].record()
        if S > 1:
            stp.splitkv_merge_with_block_view(o_norm, m_part, l_part, nb, req, qpos, table,
                                              c0.page_size, out=out, lse=lse)
        else:
            stp.block_view_fill(nb, req, qpos, table, c0.page_size)
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Event pairs cost a few microseconds of queue time each, so by default the
    # timed steps carry none (with --event-every n, every n-th step does; the
    # step time is taken over all steps either way).
    ev_every = args.event_every
    sampled = [i for i in range(args.steps) if ev_every > 0 and i % ev_every == 0]
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i, evs.get(i))
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    dec_us = np.asarray([evs[i][0].elapsed_time(evs[i][1]) for i in sampled]) * 1e3
    merge_us = np.asarray([evs[i][1].elapsed_time(evs[i][2]) for i in sampled]) * 1e3

    # The roofline's launch duration, in a loop of its own whatever --steps is:
    # args.roofline_launches decode launches (the rotated candidate sets, their
    # normalisation done beforehand) enqueued back to back between two HIP
    # events on the kernel's stream, the mean per launch; the same for the
    # merge.  A pair of events around every single launch also counts the
    # dispatch (about 2 us here); that per-launch mean is reported beside it.
    n_roof = max(200, args.roofline_launches)

    def dec_only(k):
        fused(k)

    # the decode kernel alone, over the lists the normalisation wrote (for
    # comparison with the launch that builds them itself)
    def plain_decode(k):
        nb = norm[k % args.sets]
        if S > 1:
            stp.sparse_mla_decode_partial_normalized(q, kv, nb["slot"], nb["count"], c0.scale, S,
                                                     o_norm, m_part, l_part)
        else:
            stp.sparse_mla_decode(q, kv, nb["slot"], nb["count"], c0.scale, 1, out=out, lse=lse)

    def merge_only(k):
        stp.splitkv_merge_normalized(o_norm, m_part, l_part, out, lse)

    roof_avg_us = throughput_us(dec_only, n_roof, args.sets)
    plain_avg_us = throughput_us(plain_decode, n_roof, args.sets)

    # the same step as separate launches (normalisation with its block view
    # deferred, the decode over its lists, merge with block view), timed back
    # to back like the fused one, for the comparison
    def step_fused(k):
        step(k)

    def step_separate(k):
        nb = stp.normalize_indices(topks[k], req, qpos, table, c0.page_size, c0.window,
                                   c0.num_sinks, cap, out=norm[k], defer_block_view=S > 1)
        if S > 1:
            stp.sparse_mla_decode_partial_normalized(q, kv, nb["slot"], nb["count"], c0.scale, S,
                                                     o_norm, m_part, l_part)
            stp.splitkv_merge_with_block_view(o_norm, m_part, l_part, nb, req, qpos, table,
                                              c0.page_size, out=out, lse=lse)
        else:
            stp.sparse_mla_decode(q, kv, nb["slot"], nb["count"], c0.scale, 1, out=out, lse=lse)
            stp.block_view_fill(nb, req, qpos, table, c0.page_size)

    # both step forms enqueued back to back as the timed steps are; a1 alone
    # (block view deferred) is too short to hide the host's launch cost, so
    # its launches are captured in a HIP graph (16 over the rotated sets)
    fused_step_us = throughput_us(step_fused, n_roof, args.sets)
    separate_step_us = throughput_us(step_separate, n_roof, args.sets)
    it_sets = itertools.cycle(range(args.sets))
    norm_alone_us = graph_us(
        lambda: stp.normalize_indices(topks[(k := next(it_sets))], req, qpos, table,
                                      c0.page_size, c0.window, c0.num_sinks, cap, out=norm[k],
                                      defer_block_view=True),
        reps=2 * args.sets)
    # the merge is too short for back-to-back calls to hide the host's launch
    # cost: its device time comes from merges captured in one HIP graph
    merge_avg_us = graph_us(lambda: merge_only(0)) if S > 1 else 0.0
    roof_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                 torch.cuda.Event(enable_timing=True)) for _ in range(n_roof)]
    torch.cuda.synchronize()
    for i in range(n_roof):
        step(args.warmup + args.steps + i, roof_evs[i])
    torch.cuda.synchronize()
    roof_us = np.asarray([a.elapsed_time(b) for a, b, _ in roof_evs]) * 1e3
    roof_merge_us = np.asarray([b.elapsed_time(c) for _, b, c in roof_evs]) * 1e3

    ceilings = None if args.no_ceilings else measure_ceilings(stp, kv, norm, args.sets, S,
                                                              (H + 63) // 64)

    # algorithmic bytes / flops of one decode launch (average over the rotated sets)
    q_bytes = T * H * 576 * 2
    o_bytes = T * H * (512 * 2 + 4)
    sel = np.asarray([cnt.sum() for cnt in counts], dtype=np.float64)  # sum of |S_i| per set
    roof_idx = args.warmup + args.steps + np.arange(n_roof)
    per_set_steps = np.bincount(roof_idx % args.sets, minlength=args.sets)
    mean_sel = float((sel * per_set_steps).sum() / per_set_steps.sum())
    kv_bytes = mean_sel * ROW_BYTES
    # the launch also reads each token's top-k ids and page-table row (up to
    # its position) and writes its lists (tok_out, slot_out: cap entries each)
    P = c0.page_size
    max_pos = c0.block_table.shape[1] * P - 1
    table_bytes = float(sum((min(int(qp), max_pos) // P + 1) * 4 for qp in c0.q_pos))
    norm_bytes = T * c0.top_k * 4 + table_bytes + T * cap * 8
    dec_bytes = kv_bytes + q_bytes + norm_bytes + (o_bytes if S == 1 else 0)
    plain_bytes = kv_bytes + q_bytes + mean_sel * 4 + (o_bytes if S == 1 else 0)
    flops = 2.0 * H * mean_sel * (576 + 512)
    dec_avg_s = roof_avg_us * 1e-6
    step_s = total_ms * 1e-3 / args.steps
    achieved = dec_bytes / dec_avg_s / 1e9
    traffic = load_traffic(dec_bytes)

    res = {
        "metric": METRIC,
        "value": round(T / step_s, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "deepseek-v3.2-shaped sparse MLA decode, one layer",
            "batch": T, "query_heads": H, "context": 32768, "page_size": c0.page_size,
            "top_k": c0.top_k, "window": c0.window, "sinks": c0.num_sinks, "row_bytes": ROW_BYTES,
            "kv_pool_rows": c0.kv_rows, "splits": S, "candidate_sets": args.sets,
            "mean_selected_rows_per_token": round(mean_sel / T, 2),
        },
        "roofline": {
            "kernel": "sparse_mla_decode_kernel (with normalisation)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(dec_bytes),
            "avg_launch_us": round(roof_avg_us, 3),
            "launches_timed": int(n_roof),
            "timing": "mean over a loop of its own of launches enqueued back to back between "
                      "two HIP events on the kernel's stream, after the timed steps",
            "event_pair_mean_us": round(float(roof_us.mean()), 3),
            "event_pair_median_us": round(float(np.median(roof_us)), 3),
            "bytes_counted": "KV rows + queries + top-k ids + page-table rows + the lists "
                             "written, of one launch (the split path: outputs belong to the "
                             "merge launch)" if S > 1 else
                             "KV rows + queries + top-k ids + page-table rows + the lists "
                             "written + outputs, of one launch",
            "merge_avg_us": round(merge_avg_us, 3),
            "call_frac": round((dec_bytes + (o_bytes if S > 1 else 0)) /
                               ((roof_avg_us + merge_avg_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(flops / dec_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        },
        "step_launches": "decode with the normalisation in its launch, merge with block view"
                         if S > 1 else "decode with the normalisation in its launch, block view",
        "step_back_to_back_us": {"fused": round(fused_step_us, 3),
                                 "separate_launches": round(separate_step_us, 3),
                                 "normalise_alone_graph": round(norm_alone_us, 3)},
        "effective_kv_gbps": round(kv_bytes / step_s / 1e9, 1),
        "ceilings": ceilings,
        "decode_vs_ceilings": None if ceilings is None else {
            "kv_gbs": round(kv_bytes / dec_avg_s / 1e9, 1),
            "frac_of_row_gather_decode_placement":
                round(ceilings["row_gather_decode_placement"]["us"] / (dec_avg_s * 1e6), 4),
            "frac_of_row_gather_each_row_once":
                round(ceilings["row_gather_each_row_once"]["us"] / (dec_avg_s * 1e6), 4),
        },
        "decode_kernel_alone": {
            "kernel": "sparse_mla_decode_kernel over the normalisation's lists",
            "avg_launch_us": round(plain_avg_us, 3),
            "frac": round(plain_bytes / (plain_avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "kernel_us": {
            "decode_median": round(float(np.median(roof_us)), 3),
            "decode_p95": round(float(np.percentile(roof_us, 95)), 3),
            "decode_p99": round(float(np.percentile(roof_us, 99)), 3),
            "merge_with_block_view_median" if S > 1 else "after_decode_median":
                round(float(np.median(roof_merge_us)), 3),
            "decode_in_steps_mean": round(float(dec_us.mean()), 3) if sampled else None,
            "decode_in_steps_samples": len(sampled),
        },
        "wall_s_timed": round(t_wall, 4),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cases, kv, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
