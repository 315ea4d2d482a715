"""Benchmark: one batched decode step (append_kv + paged decode attention + log-sum-exp merge) of
the B=128 ragged bf16 workload on one MI355X, through the C ABI.

Workload: 128 rows with contexts uniform in [512, 8192] (seed 2: kv_len 809..8139, sum 574 199),
32 query / 8 KV heads, head_dim 64, bf16 N(0,1) values, 16-token blocks in a shuffled pool sized
1.25x the blocks needed. One step reads 1.176 GB of K/V.

Prints one JSON line. ``value`` is K/V GB/s of whole steps (wall clock over the timed steps,
append + decode + merge, inputs resident in HBM); ``roofline`` uses HIP events recorded on the
library's stream around every decode call inside the timed region; ``cpu_baseline`` times the
fp64 oracle on the host cores over the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "paged decode-attn K/V GB/s (% HBM peak) + µs/step, B=128 ragged bf16"
METRIC_LONG = "paged decode-attn K/V GB/s (% HBM peak) + µs/step, B=4 long-context bf16"
METRIC_PADDED = ("right-padded decode-attn K/V GB/s (% HBM peak) + µs/step, B=128 ragged bf16 "
                 "(padding gaps skipped)")
# one GPU's share of a sharded step (the lengths of the whole workload, cut as the sharding cuts)
METRIC_SHARE = {
    "b128-tp2": "paged decode-attn K/V GB/s (% HBM peak), B=128 bf16, one GPU of 2 (KV heads split)",
    "b128-dp2": "paged decode-attn K/V GB/s (% HBM peak), B=128 bf16, one GPU of 2 (rows split)",
    "long-sp4": "paged decode-attn K/V GB/s (% HBM peak), B=4 long-context bf16, one GPU of 4 "
                "(each row's tokens split)",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_b128_traffic.txt")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="b128",
                   choices=["b128", "long", "mq", "mq-sparse", "b16", "mq-tokenize",
                            "b128-padded", "b128-tp2", "b128-dp2", "long-sp4"],
                   help="b128 is the reported workload; long (B=4 long-context split-K), mq "
                        "(latent cross-attention on the matrix cores; mq-sparse under the "
                        "temporal block mask), b16 (the B=16 lockstep step, paged and "
                        "right-padded), b128-padded (the B=128 step laid out right-padded) and "
                        "mq-tokenize (the fused spike tokenizer + K/V projection) measure the "
                        "other paths; b128-tp2, b128-dp2 and long-sp4 "
                        "measure one GPU's share of a sharded step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--flush-mb", type=int, default=512,
                   help="cache-flush write between the extra flushed decode timings")
    p.add_argument("--traffic-calibration", action="store_true",
                   help="finish with 5 device copies of 256 MiB (a known-size reference for "
                        "hardware byte counters)")
    return p.parse_args()


def kernel_source_hash(*names: str) -> str:
    """sha256 prefix of the named kernel sources (file names under csrc/; all sources if none):
    ties a committed counter summary to the code of the kernels it measured."""
    from paged_kv_cache_177_amd.build import sources

    h = hashlib.sha256()
    for s in sources():
        if names and os.path.basename(s) not in names:
            continue
        with open(s, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# the decode call's kernels (decode_vector_kernel, decode_persistent_kernel, lse_reduce_kernel)
DECODE_SOURCES = ("pa_decode.hip", "pa_internal.h")


def read_traffic(src_hash: str):
    """HBM bytes per decode call from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources (its 'source_hash' line matches); else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != src_hash or "hbm_bytes_per_call" not in vals:
        return None
    return float(vals["hbm_bytes_per_call"])


def blas_threads() -> int:
    import threadpoolctl

    blas = [p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
            if p.get("user_api") == "blas"]
    return int(max(blas)) if blas else 1


def cpu_baseline_mq(case, flops: float, keep=None, budget_s: float = 10.0, max_reps: int = 50):
    """The oracle on the full multi-query workload (all rows, shared latent queries); with
    ``keep``, its block-sparse form under that mask."""
    import oracle as O

    times = []
    t_start = time.perf_counter()
    while len(times) < max_reps and (time.perf_counter() - t_start) < budget_s:
        t0 = time.perf_counter()
        if keep is None:
            O.decode_paged(case.k_pool, case.v_pool, case.dtype, case.block_tables, case.kv_lens,
                           case.q, case.scale, shared_q=True)
        else:
            O.decode_paged_block_sparse(case.k_pool, case.v_pool, case.dtype, case.block_tables,
                                        case.kv_lens, case.q, case.scale, keep.astype(bool),
                                        shared_q=True)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    cores = blas_threads()
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"full {case.name} workload ({len(case.kv_lens)} rows x {case.n_q} queries) "
                       f"in fp64 numpy, median of {len(times)} run(s), {t:.2f} s each; host "
                       f"affinity {len(os.sched_getaffinity(0))} cores, BLAS threads {cores}")}


def cpu_baseline(case, budget_s: float = 10.0, max_reps: int = 50):
    """The oracle (as it stands) on the full workload's decode: gather every row through its block
    table and run two-pass fp64 attention. Repeated until ~budget_s of CPU work, median taken."""
    import oracle as O

    k2, v2, _ = O.append_kv(case.k_pool, case.v_pool, case.dtype, "paged", case.block_tables,
                            case.positions, case.dest, case.k_new, case.v_new)
    times = []
    t_start = time.perf_counter()
    while len(times) < max_reps and (time.perf_counter() - t_start) < budget_s:
        t0 = time.perf_counter()
        O.decode_paged(k2, v2, case.dtype, case.block_tables, case.kv_lens, case.q, case.scale)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    cores = blas_threads()
    return {"value": case.kv_bytes() / t / 1e9, "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"full {case.name} decode step (all {case.batch} rows, "
                       f"{case.kv_bytes() / 1e9:.3f} GB K/V) in fp64 numpy, median of "
                       f"{len(times)} run(s), {t:.2f} s each; host affinity "
                       f"{len(os.sched_getaffinity(0))} cores, BLAS threads {cores}")}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix-core peak


def main_mq(args):
    """Latent cross-attention on the matrix cores: 16 rows x 256 shared latent queries over ragged
    spike-token keys (8 heads of 32), one pa_decode_attention call per step. mq-sparse runs
    pa_decode_attention_block_sparse under the temporal-overlap block mask instead; its FLOP count
    is that of the kept (query, key) pairs."""
    import numpy as np
    import torch

    import workloads as W
    from paged_kv_cache_177_amd import binding as B
    from paged_kv_cache_177_amd.masks import temporal_block_mask
    from paged_kv_cache_177_amd.runner import MultiQueryStep

    torch.cuda.set_device(0)
    case = W.mq()
    r = MultiQueryStep(case, device="cuda:0")
    stream = torch.cuda.current_stream()
    sparse = args.workload == "mq-sparse"
    flops = 4.0 * case.n_q * float(case.kv_lens.sum()) * case.num_heads * case.head_dim
    kept_frac = 1.0
    if sparse:
        keep = temporal_block_mask(case.token_bins, case.n_q, case.n_bins, halo=1)
        # kept (query, key) pairs: per row, per query block, the valid keys of its kept blocks
        pairs = 0
        for b in range(case.batch):
            n = int(case.kv_lens[b])
            per_block = np.minimum(16, n - 16 * np.arange(keep.shape[2])).clip(0)
            for qb in range(keep.shape[1]):
                nq = min(16, case.n_q - 16 * qb)
                pairs += nq * int((keep[b, qb] * per_block).sum())
        kept_frac = pairs / (case.n_q * float(case.kv_lens.sum()))
        flops = 4.0 * pairs * case.num_heads * case.head_dim
        mask_dev = torch.from_numpy(keep).to("cuda:0")

        def call():
            B.pa_decode_attention_block_sparse(r.kv.pool, r.q, 0, case.n_q, case.num_heads,
                                               r.block_tables, r.bt_stride, r.kv_lens, r.batch,
                                               r.max_kv_len, case.scale, mask_dev, keep.shape[2],
                                               out=r.out, lse=r.lse)
    else:
        call = r.decode
    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < 1.0:
        for _ in range(10):
            call()
        done += 10
        torch.cuda.synchronize()
    # back-to-back calls between one pair of events: the average is the kernel's launch duration
    # (a call is short enough that events around each one would mostly time the host)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(args.steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    avg_ms = a.elapsed_time(b) / args.steps
    achieved = flops / (avg_ms * 1e-3) / 1e12
    out = {
        "metric": ("multi-query latent cross-attention TFLOP/s + us/call, 16 x 256 queries, bf16"
                   + (", block-sparse (temporal mask; kept pairs)" if sparse else "")),
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{case.name}: B={len(case.kv_lens)} rows x {case.n_q} shared "
                                f"latent queries, {case.num_heads} heads of {case.head_dim}, "
                                f"ragged keys {int(case.kv_lens.min())}..{int(case.kv_lens.max())} "
                                f"(sum {int(case.kv_lens.sum())}), 16-token blocks, seed "
                                f"{case.seed}"),
                   "global_batch": len(case.kv_lens), "flops_per_step": flops,
                   "step": ("one pa_decode_attention_block_sparse call" if sparse else
                            "one multi-query pa_decode_attention call"),
                   "kept_pair_fraction": round(kept_frac, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "mq_paged_mfma_kernel<32, " + ("true>" if sparse else "false>"),
                     "flops_per_launch": flops,
                     "avg_launch_us": round(avg_ms * 1e3, 2)},
        "detail": {"us_per_call": round(avg_ms * 1e3, 2),
                   "source_hash": kernel_source_hash("pa_mq.hip", "pa_internal.h")},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_mq(case, flops, keep=keep if sparse else None)
    print(json.dumps(out), flush=True)


def read_ceiling_gbs(gib: int = 2, reps: int = 10, per_cu=(1.5, 2, 3, 4, 8)):
    """The practical HBM read bandwidth on this GPU: the read probe (libpa_probe.so, a measuring
    instrument outside the attention library) streams a `gib` GiB device buffer; for each grid
    size in `per_cu` (workgroups per CU) the median of `reps` launches timed with HIP events, and
    the best of those medians is returned with its grid. (The probe's rate depends on the grid:
    on MI355X 1.5 workgroups per CU read fastest, ~7.3 TB/s.)"""
    import ctypes

    import torch

    from paged_kv_cache_177_amd.build import PROBE_LIB

    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: run the build first")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    lib.pa_probe_read.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grids = [int(cus * m) for m in per_cu]
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def launch(grid):
        rc = lib.pa_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                               ctypes.c_void_p(sink.data_ptr()), grid,
                               ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"pa_probe_read failed with HIP error {rc}")

    best = (0.0, 0)
    for grid in grids:
        for _ in range(3):
            launch(grid)
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch(grid)
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        best = max(best, (nbytes / (statistics.median(ts) * 1e-3) / 1e9, grid))
    del buf, sink
    return best


def main_tokenize(args):
    """Fused spike tokenizer + K/V projection into the paged pool: 16 rows of raw spike events
    (neuron, time bin, value), one pa_tokenize_kv call per step. The kernel's floor is HBM: every
    token writes H * dh keys and as many values (bf16) and reads its three ids; the tables and the
    two projection matrices are read once. The matrix-core FLOPs are reported beside it."""
    import numpy as np
    import torch

    import workloads as W
    from paged_kv_cache_177_amd import binding as B
    from paged_kv_cache_177_amd.runner import to_torch

    torch.cuda.set_device(0)
    c = W.mq_tokenizer()
    desc = B.make_desc("paged", "bf16", c.num_heads, c.head_dim, num_blocks=c.num_blocks)
    pool = B.alloc_pool(desc)
    pool.k.copy_(to_torch(c.k_pool, "bf16"))
    pool.v.copy_(to_torch(c.v_pool, "bf16"))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    n_emb, t_emb, v_emb = d(c.n_emb), d(c.t_emb), d(c.v_emb)
    # weights packed once into matrix-core fragment order (outside the timed calls, as a server
    # would at load time)
    w_k = B.pa_pack_projection(to_torch(c.w_k, "bf16").cuda())
    w_v = B.pa_pack_projection(to_torch(c.w_v, "bf16").cuda())
    offsets, nid, tb, vid = d(c.offsets), d(c.neuron_ids), d(c.time_bins), d(c.value_ids)
    bt = d(c.block_tables)
    me = int(c.kv_lens.max())
    E = int(c.offsets[-1])
    N = c.num_heads * c.head_dim
    Dm = c.n_emb.shape[1]
    stream = torch.cuda.current_stream()

    def call():
        B.pa_tokenize_kv(pool.pool, n_emb, t_emb, v_emb, w_k, w_v, offsets, nid, tb, vid, bt,
                         c.block_tables.shape[1], c.batch, me)

    # algorithmic bytes: K and V slots written (bf16), three int32 ids per token, the two bf16
    # weight matrices and the three fp32 tables once, the offsets and the block-table entries used
    used_blocks = int(sum((int(n) + 15) // 16 for n in c.kv_lens))
    nbytes = float(E * (2 * N * 2 + 3 * 4) + 2 * N * Dm * 2 +
                   (c.n_emb.size + c.t_emb.size + c.v_emb.size) * 4 + (c.batch + 1) * 4 +
                   used_blocks * 4)
    flops = 2.0 * E * Dm * 2 * N
    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < 1.0:
        for _ in range(10):
            call()
        done += 10
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(args.steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    avg_ms = a.elapsed_time(b) / args.steps
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    out = {
        "metric": "spike tokens tokenized and projected into the paged K/V pool per second, bf16",
        "value": round(E / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{c.name}: B={c.batch} rows of spike events "
                                f"{int(c.kv_lens.min())}..{me} (sum {E}), model dim {Dm}, "
                                f"{c.num_heads} heads of {c.head_dim}, 16-token blocks"),
                   "global_batch": c.batch, "bytes_per_step": nbytes, "flops_per_step": flops,
                   "step": "one pa_tokenize_kv call"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "tokenize_kv_kernel", "bytes_per_launch": nbytes,
                     "avg_launch_us": round(avg_ms * 1e3, 2)},
        "detail": {"us_per_call": round(avg_ms * 1e3, 2),
                   "mfma_tflops": round(flops / (avg_ms * 1e-3) / 1e12, 1),
                   "mfma_frac": round(flops / (avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                   "source_hash": kernel_source_hash("pa_tokenize.hip", "pa_internal.h")},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_tokenize(c, E)
    print(json.dumps(out), flush=True)


def cpu_baseline_tokenize(c, E: int, budget_s: float = 10.0, max_reps: int = 200):
    """The oracle's tokenize_kv on the full workload (embed, fp64 projection, pool writes)."""
    import oracle as O

    times = []
    t_start = time.perf_counter()
    while len(times) < max_reps and (time.perf_counter() - t_start) < budget_s:
        t0 = time.perf_counter()
        O.tokenize_kv(c.k_pool, c.v_pool, c.n_emb, c.t_emb, c.v_emb, c.w_k, c.w_v, c.offsets,
                      c.neuron_ids, c.time_bins, c.value_ids, c.block_tables)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    cores = blas_threads()
    return {"value": E / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"full {c.name} workload ({c.batch} rows, {E} tokens) in fp64 numpy, "
                       f"median of {len(times)} run(s), {t:.2f} s each; host affinity "
                       f"{len(os.sched_getaffinity(0))} cores, BLAS threads {cores}")}


def graph_step_timing(args, plan, timed, tokens: int = 1, one_launch: bool = True):
    """The paged B=16 step captured as a graph (per token: append + decode + merge + next positions
    in one pa_lockstep_decode_step launch, or with ``one_launch=False`` the fused call followed by
    the add-one kernel), ``tokens`` consecutive tokens per graph, replayed; and the same calls
    issued one by one (the eager counterpart of the graph). Block tables are filled for every
    position the warm-up and the timed replays reach between resets (positions are reset outside
    the timed replays). Returns ((wall, events) of the replays, (wall, events) of the eager runs),
    in microseconds per token."""
    import numpy as np
    import torch

    import workloads as W
    from paged_kv_cache_177_amd import binding as B
    from paged_kv_cache_177_amd.runner import PagedLockstepGraph, to_torch

    reset_every = max(1, 256 // tokens)      # replays between position resets
    ahead = max(args.steps, reset_every) * tokens + tokens
    n0 = plan.n_ctx0.astype(np.int32)
    extra = 16 * ((ahead + 31) // 16)
    case = W.make_paged_case("b16-graph", plan.seed, n0, plan.num_q_heads, plan.num_kv_heads,
                             plan.head_dim, plan.dtype, rope_theta=plan.rope_theta,
                             rope_max_pos=int(n0.max()) + ahead + 2,
                             num_blocks=int(((n0 + extra) // 16 + 2).sum()) + 8,
                             bt_stride=(int(n0.max()) + ahead + 16) // 16 + 1)
    # extend every row's table with free blocks for the positions ahead
    bt = case.block_tables.copy()
    used = set(int(x) for x in bt.ravel())
    free = [i for i in range(case.num_blocks) if i not in used]
    for b in range(case.batch):
        have = int((case.kv_lens[b] + 15) // 16)
        need = (int(n0[b]) + ahead + 16) // 16
        for j in range(have, need):
            bt[b, j] = free.pop()
    desc = B.make_desc("paged", case.dtype, case.num_kv_heads, case.head_dim,
                       num_blocks=case.num_blocks, rope_max_pos=case.rope_max_pos,
                       rope_theta=case.rope_theta)
    pool = B.alloc_pool(desc, device="cuda:0")
    pool.k.copy_(to_torch(case.k_pool, case.dtype))
    pool.v.copy_(to_torch(case.v_pool, case.dtype))
    start = torch.from_numpy(n0.copy()).to("cuda:0")
    g = PagedLockstepGraph(pool, torch.from_numpy(bt).to("cuda:0"), start.clone(),
                           case.num_q_heads, int(n0.max()) + ahead + 1, case.scale,
                           device="cuda:0", tokens=tokens, one_launch=one_launch)
    g.k_new.copy_(to_torch(case.k_new, case.dtype))
    g.v_new.copy_(to_torch(case.v_new, case.dtype))
    g.q_in.copy_(to_torch(case.q, case.dtype))

    def reset():
        g.set_positions(start)

    g.step()
    reset()
    torch.cuda.synchronize()
    g.capture()
    count = [0]

    def every(fn):
        def run():
            if count[0] == reset_every:
                reset()
                count[0] = 0
            fn()
            count[0] += 1
        return run

    # timed() warms up (with resets), then times args.steps replays from a fresh reset
    def timed_from_reset(fn):
        count[0] = 0
        reset()
        wall, ev = timed(fn, before_timed=lambda: (reset(), count.__setitem__(0, 0)))
        return wall / tokens, ev / tokens

    graph = timed_from_reset(every(g.replay))
    eager = timed_from_reset(every(g.step))
    return graph, eager


def append_timings(r, case, stream, calls: int = 50):
    """us per call of pa_append_kv and of pa_append_kv_qk_norm on the runner's step (same rows,
    positions, heads and inputs; the norm with unit weights and eps 1e-5)."""
    import torch

    from paged_kv_cache_177_amd import binding as B

    D = case.head_dim
    w = torch.ones(D, dtype=torch.float32, device="cuda:0")
    rope = r.kv.pool.desc.rope_max_pos > 0

    def norm_call():  # the same heads as r.append (queries only when the pool rotates them)
        B.pa_append_kv_qk_norm(r.kv.pool, r.block_tables, r.bt_stride, r.positions, r.dest,
                               r.k_new, r.v_new, r.q if rope else None,
                               r.q_rot if rope else None, case.num_q_heads if rope else 0,
                               case.batch, w if rope else None, w, 1e-5)

    out = []
    for fn in (r.append, norm_call):
        for _ in range(10):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(calls):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1e3 / calls)
    return out[0], out[1]


def b16_protocol_timing(plan, reps: int = 3):
    """The B=16 lockstep run as the plan specifies it: 32 consecutive steps over 16 ragged rows,
    two rows leaving and two sequences joining (their histories written into recycled blocks) at
    the join step, blocks allocated on demand from the shuffled pool's LIFO free list.

    Host and GPU are measured apart. The host's bookkeeping for every step (freeing and
    allocating blocks, packing the block table) runs first, timed step by step on the host clock.
    The GPU then runs the 32 steps, each one pa_append_decode_attention call on the step's own
    inputs and table (already in device memory): once with a pair of events around every step
    (median, p10, p90; each pair adds the events' own cost), and once as two back-to-back runs,
    steps before the join and steps from it, each between one pair of events, with the joiners'
    history upload between them (timed on its own). ``reps`` runs from the initial state.
    Returns a dict of microsecond figures."""
    import math

    import numpy as np
    import torch

    from paged_kv_cache_177_amd import binding as B
    from paged_kv_cache_177_amd.blocks import BlockAllocator, SequenceBlocks, block_table_array
    from paged_kv_cache_177_amd.runner import to_torch

    dev = "cuda:0"
    H_q, H, D, scale = plan.num_q_heads, plan.num_kv_heads, plan.head_dim, plan.scale
    sched = plan.schedule()
    steps, J = len(sched), plan.join_step
    stride = math.ceil(plan.rope_max_pos / 16)
    desc = B.make_desc("paged", plan.dtype, H, D, num_blocks=plan.num_blocks,
                       rope_max_pos=plan.rope_max_pos, rope_theta=plan.rope_theta)
    pool = B.alloc_pool(desc, device=dev)
    hist = {sid: tuple(to_torch(a, plan.dtype).to(dev) for a in plan.history(sid))
            for sid in range(18)}

    def stack(i):  # every step's inputs, resident before the run: [steps][16][heads][D]
        return torch.stack([torch.stack([to_torch(plan.step_inputs(sid, s)[i], plan.dtype)
                                         for _, sid, _ in rows])
                            for s, rows in enumerate(sched)]).to(dev)

    q_all, k_all, v_all = stack(0), stack(1), stack(2)
    q_rot = torch.empty((16, H_q, D), dtype=q_all.dtype, device=dev)
    out = torch.empty((16, H_q, D), dtype=torch.float32, device=dev)
    lse = torch.empty((16, H_q), dtype=torch.float32, device=dev)
    pos_np = np.array([[pos for _, _, pos in rows] for rows in sched], np.int32)
    pos_d = torch.from_numpy(pos_np).to(dev)
    len_d = pos_d + 1
    max_len = int(pos_np.max()) + 1
    stream = torch.cuda.current_stream()

    def write_history(sid, blocks):
        k, v = hist[sid]
        t = torch.arange(k.shape[0], device=dev)
        blk = torch.tensor(blocks, dtype=torch.int64, device=dev)[t // 16]
        pool.k[blk, :, t % 16, :] = k
        pool.v[blk, :, t % 16, :] = v

    def bookkeeping():
        """The host side of one run: per step, the table and the host time it took; the blocks
        of the initial and the joining sequences."""
        perm = plan.perm
        seqs, off = {}, 0
        for sid in range(16):
            n = math.ceil(plan.seq_ctx(sid) / 16)
            seqs[sid] = SequenceBlocks(perm[off:off + n])
            off += n
        alloc = BlockAllocator(perm[off:-1])
        alloc.adopt(perm[:off])
        poison = int(perm[-1])
        first = {sid: list(seqs[sid].blocks) for sid in range(16)}
        tables, host, joined = [], [], {}
        for s, rows in enumerate(sched):
            t0 = time.perf_counter()
            if s == J:
                for slot in plan.leave_slots.tolist():
                    alloc.free(seqs.pop(sched[s - 1][slot][1]).blocks)
                for _, sid, _ in rows:
                    if sid >= 16:
                        sb = SequenceBlocks()
                        sb.ensure_token(plan.seq_ctx(sid) - 1, alloc)
                        seqs[sid] = sb
                        joined[sid] = list(sb.blocks)
            for _, sid, pos in rows:
                seqs[sid].ensure_token(int(pos), alloc)
            tables.append(block_table_array([seqs[sid] for _, sid, _ in rows], stride, poison))
            host.append((time.perf_counter() - t0) * 1e6)
        return np.stack(tables), host, first, joined

    tables, _, _, _ = bookkeeping()
    bt_d = torch.from_numpy(tables).to(dev)
    need = B.pa_append_decode_attention(pool.pool, bt_d[0], stride, pos_d[0], None, k_all[0],
                                        v_all[0], q_all[0], q_rot, H_q, len_d[0], 16, max_len,
                                        scale, out=out, query_workspace=True)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)

    # every step's views, sliced before the timed runs (slicing in the loop is host time that
    # would pace the back-to-back steps)
    views = [(bt_d[s], pos_d[s], k_all[s], v_all[s], q_all[s], len_d[s]) for s in range(steps)]

    def step(s):
        bt_s, pos_s, k_s, v_s, q_s, len_s = views[s]
        B.pa_append_decode_attention(pool.pool, bt_s, stride, pos_s, None, k_s, v_s, q_s, q_rot,
                                     H_q, len_s, 16, max_len, scale, workspace=ws, out=out,
                                     lse=lse)

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    host_us, per_step_us, b2b_us, join_us = [], [], [], []
    for rep in range(reps + 1):  # the first run warms up
        tables_r, host, first, joined = bookkeeping()
        assert np.array_equal(tables_r, tables)  # the same plan gives the same tables
        for sid in range(16):
            write_history(sid, first[sid])
        torch.cuda.synchronize()
        # per-step events, steps issued back to back
        pairs = []
        for s in range(steps):
            if s == J:
                for sid, blocks in joined.items():
                    write_history(sid, blocks)
            a = ev()
            step(s)
            pairs.append((a, ev()))
        torch.cuda.synchronize()
        # the same run as two back-to-back segments around the join
        for sid in range(16):
            write_history(sid, first[sid])
        torch.cuda.synchronize()
        a = ev()
        for s in range(J):
            step(s)
        b = ev()
        for sid, blocks in joined.items():
            write_history(sid, blocks)
        c = ev()
        for s in range(J, steps):
            step(s)
        d = ev()
        torch.cuda.synchronize()
        if rep > 0:
            host_us.extend(host)
            per_step_us.extend(x.elapsed_time(y) * 1e3 for x, y in pairs)
            b2b_us.append((a.elapsed_time(b) + c.elapsed_time(d)) * 1e3 / steps)
            join_us.append(b.elapsed_time(c) * 1e3)
    pct = lambda x, q: round(float(np.percentile(x, q)), 2)  # noqa: E731
    return {"protocol_steps": steps, "protocol_runs": reps,
            "protocol_gpu_us_per_step_back_to_back": round(statistics.median(b2b_us), 2),
            "protocol_gpu_us_per_step_events_median": pct(per_step_us, 50),
            "protocol_gpu_us_per_step_events_p10": pct(per_step_us, 10),
            "protocol_gpu_us_per_step_events_p90": pct(per_step_us, 90),
            "protocol_host_bookkeeping_us_per_step_median": pct(host_us, 50),
            "protocol_host_bookkeeping_us_per_step_p90": pct(host_us, 90),
            "protocol_host_bookkeeping_us_join_step": round(
                statistics.median(host_us[J::steps]), 1),
            "protocol_join_history_upload_gpu_us": round(statistics.median(join_us), 1)}


def main_b16(args):
    """The B=16 lockstep step at the protocol's starting geometry (contexts of seed 1, 32/8 heads,
    D=64, bf16, RoPE theta 1e6): append_kv (keys, values and query rotation) + decode + merge, in
    the paged form and in the right-padded form, and the paged step replayed from a graph (with the
    on-device advance). A step moves ~36 MB and is launch-bound, so the line reports microseconds
    per step, timed over back-to-back steps between one pair of events."""
    import numpy as np
    import torch

    import workloads as W
    from paged_kv_cache_177_amd import binding as B
    from paged_kv_cache_177_amd.runner import PaddedLockstep, PagedStep, to_torch

    torch.cuda.set_device(0)
    dev = "cuda:0"
    plan = W.b16_plan()
    case = W.make_paged_case("b16", plan.seed, plan.n_ctx0, plan.num_q_heads, plan.num_kv_heads,
                             plan.head_dim, plan.dtype, rope_theta=plan.rope_theta)
    kv_bytes = case.kv_bytes()
    stream = torch.cuda.current_stream()
    paged = PagedStep(case, device=dev)

    pc = W.padded_from_paged(case)
    L = PaddedLockstep(pc.dtype, pc.num_q_heads, pc.num_kv_heads, pc.head_dim, pc.batch,
                       pc.seq_cap, rope_theta=pc.rope_theta, rope_max_pos=pc.rope_max_pos,
                       device=dev)
    L.kv.k.copy_(to_torch(pc.k_pad, pc.dtype))
    L.kv.v.copy_(to_torch(pc.v_pad, pc.dtype))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    pos, dest = d(pc.positions), d(pc.dest)
    k_new, v_new = to_torch(pc.k_new, pc.dtype).to(dev), to_torch(pc.v_new, pc.dtype).to(dev)
    q_in = to_torch(pc.q, pc.dtype).to(dev)
    q_rot = torch.empty_like(q_in)
    gs, ge = d(pc.prefix_lens.astype(np.int32)), d(np.full(pc.batch, pc.padded_len, np.int32))
    out = torch.empty((pc.batch, pc.num_q_heads, pc.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((pc.batch, pc.num_q_heads), dtype=torch.float32, device=dev)
    need = B.pa_decode_attention_padded(L.kv.pool, q_rot, pc.num_q_heads, pc.batch, gs, ge,
                                        pc.kv_cols, pc.scale, out=out, query_workspace=True)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)

    def padded_step():
        L.append(pos, dest, k_new, v_new, q_in, q_rot)
        B.pa_decode_attention_padded(L.kv.pool, q_rot, pc.num_q_heads, pc.batch, gs, ge,
                                     pc.kv_cols, pc.scale, workspace=ws if need else None,
                                     out=out, lse=lse)

    def timed(fn, before_timed=None):
        t_w = time.perf_counter()
        done = 0
        while done < args.warmup or time.perf_counter() - t_w < 1.0:
            for _ in range(10):
                fn()
            done += 10
            torch.cuda.synchronize()
        if before_timed is not None:
            before_timed()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / args.steps, a.elapsed_time(b) * 1e3 / args.steps

    def padded_fused_step():
        B.pa_append_decode_attention_padded(L.kv.pool, pos, dest, k_new, v_new, q_in, q_rot,
                                            pc.num_q_heads, gs, ge, pc.kv_cols, pc.batch,
                                            pc.scale, workspace=ws if need else None, out=out,
                                            lse=lse)

    # the step as one fused call (append folded into the decode launch) + the merge, and as the
    # separate calls: the same bits
    wall_paged, ev_paged = timed(paged.fused_step)
    wall_padded, ev_padded = timed(padded_fused_step)
    wall_paged_sep, ev_paged_sep = timed(paged.step)
    wall_padded_sep, ev_padded_sep = timed(padded_step)
    (wall_graph, ev_graph), (wall_g_eager, ev_g_eager) = graph_step_timing(args, plan, timed)
    graph_k = {}
    for k in (4, 16):
        (wg, eg), (we, ee) = graph_step_timing(args, plan, timed, tokens=k)
        graph_k[f"graph_{k}_tokens_us_per_token_events"] = round(eg, 2)
        graph_k[f"graph_{k}_tokens_us_per_token_wall"] = round(wg, 2)
        graph_k[f"graph_{k}_tokens_eager_us_per_token_events"] = round(ee, 2)
    for k in (1, 16):  # the two-kernel token (fused call + add-one kernel), for comparison
        (wg, eg), (we, ee) = graph_step_timing(args, plan, timed, tokens=k, one_launch=False)
        graph_k[f"graph_{k}_tokens_two_kernels_us_per_token_events"] = round(eg, 2)
        graph_k[f"graph_{k}_tokens_two_kernels_eager_us_per_token_events"] = round(ee, 2)
    protocol = b16_protocol_timing(plan)
    out_line = {
        "metric": "B=16 lockstep decode step us (append + decode + merge), paged, bf16",
        "value": round(ev_paged, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_paged / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"b16: B=16 ragged contexts {int(case.n_ctx.min())}.."
                                f"{int(case.n_ctx.max())} (kv_len sum {int(case.kv_lens.sum())}), "
                                f"H_q=32, H_kv=8, D=64, 16-token blocks, RoPE theta 1e6, seed "
                                f"{plan.seed}"),
                   "global_batch": case.batch, "kv_bytes_per_step": kv_bytes,
                   "step": ("append_kv (k, v, q rotation) + decode + lse merge: "
                            "pa_append_decode_attention (one launch: the append folded into "
                            "the split grid, which also merges the splits)")},
        "roofline": {"bound": "hbm", "achieved": round(kv_bytes / (ev_paged * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kv_bytes / (ev_paged * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": "whole step (launch-bound)",
                     "bytes_per_launch": kv_bytes, "avg_launch_us": round(ev_paged, 2)},
        "detail": {"paged_us_per_step_events": round(ev_paged, 2),
                   "paged_us_per_step_wall": round(wall_paged, 2),
                   "padded_us_per_step_events": round(ev_padded, 2),
                   "padded_us_per_step_wall": round(wall_padded, 2),
                   "paged_separate_calls_us_per_step_events": round(ev_paged_sep, 2),
                   "paged_separate_calls_us_per_step_wall": round(wall_paged_sep, 2),
                   "padded_separate_calls_us_per_step_events": round(ev_padded_sep, 2),
                   "padded_separate_calls_us_per_step_wall": round(wall_padded_sep, 2),
                   "graph_us_per_step_events": round(ev_graph, 2),
                   "graph_us_per_step_wall": round(wall_graph, 2),
                   "graph_eager_us_per_step_events": round(ev_g_eager, 2),
                   "graph_eager_us_per_step_wall": round(wall_g_eager, 2),
                   **graph_k,
                   **protocol,
                   "source_hash": kernel_source_hash()},
    }
    if not args.no_cpu_baseline:
        out_line["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(out_line), flush=True)


def main_b128_padded(args):
    """The B=128 step in the right-padded lockstep layout: each row's history in columns
    [0, n_b) of a [128][8][8140][64] bf16 pool, the step's token at the common column 8139, the
    gap [n_b, 8139) never read. One pa_append_decode_attention_padded call per step (append folded
    into the split grid, which merges its own splits); the same K/V bytes as the paged step. The
    paged decode of the same rows runs in the same process for comparison."""
    import numpy as np
    import torch

    import workloads as W
    from paged_kv_cache_177_amd import binding as B
    from paged_kv_cache_177_amd.runner import PaddedLockstep, PagedStep, to_torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = "cuda:0"
    case = W.b128()
    pc = W.padded_from_paged(case)
    kv_bytes = case.kv_bytes()
    stream = torch.cuda.current_stream()
    L = PaddedLockstep(pc.dtype, pc.num_q_heads, pc.num_kv_heads, pc.head_dim, pc.batch,
                       pc.seq_cap, device=dev)
    L.kv.k.copy_(to_torch(pc.k_pad, pc.dtype))
    L.kv.v.copy_(to_torch(pc.v_pad, pc.dtype))
    pc.k_pad = pc.v_pad = None  # host copies no longer needed
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    pos, dest = d(pc.positions), d(pc.dest)
    k_new, v_new = to_torch(pc.k_new, pc.dtype).to(dev), to_torch(pc.v_new, pc.dtype).to(dev)
    q = to_torch(pc.q, pc.dtype).to(dev)
    gs, ge = d(pc.prefix_lens.astype(np.int32)), d(np.full(pc.batch, pc.padded_len, np.int32))
    out = torch.empty((pc.batch, pc.num_q_heads, pc.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((pc.batch, pc.num_q_heads), dtype=torch.float32, device=dev)
    need = B.pa_decode_attention_padded(L.kv.pool, q, pc.num_q_heads, pc.batch, gs, ge,
                                        pc.kv_cols, pc.scale, out=out, query_workspace=True)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    wsa = ws if need else None

    def fused_step():
        B.pa_append_decode_attention_padded(L.kv.pool, pos, dest, k_new, v_new, q, None,
                                            pc.num_q_heads, gs, ge, pc.kv_cols, pc.batch,
                                            pc.scale, workspace=wsa, out=out, lse=lse)

    def decode():
        B.pa_decode_attention_padded(L.kv.pool, q, pc.num_q_heads, pc.batch, gs, ge, pc.kv_cols,
                                     pc.scale, workspace=wsa, out=out, lse=lse)

    def separate_step():
        L.append(pos, dest, k_new, v_new)
        decode()

    def timed(fn):
        t_w = time.perf_counter()
        done = 0
        while done < args.warmup or time.perf_counter() - t_w < 1.0:
            for _ in range(10):
                fn()
            done += 10
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, a.elapsed_time(b) / args.steps

    ms_per_step, step_ev_ms = timed(fused_step)
    sep_ms, sep_ev_ms = timed(separate_step)
    _, dec_avg_ms = timed(decode)

    flush = torch.empty(args.flush_mb * (1 << 20), dtype=torch.uint8, device=dev)
    fl = []
    for _ in range(10):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        decode()
        b.record(stream)
        torch.cuda.synchronize()
        fl.append(a.elapsed_time(b))
    del flush

    # the paged decode of the same rows, timed the same way (same process, same clocks)
    r = PagedStep(case, device=dev)
    r.append()
    _, paged_dec_ms = timed(r.decode)

    achieved = kv_bytes / (dec_avg_ms * 1e-3) / 1e9
    flushed_gbs = kv_bytes / (statistics.median(fl) * 1e-3) / 1e9
    out_line = {
        "metric": METRIC_PADDED,
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"b128 right-padded: B={pc.batch} rows, histories "
                                f"{int(pc.prefix_lens.min())}..{pc.padded_len} columns, padded "
                                f"to {pc.padded_len} + the step's column, H_q={pc.num_q_heads}, "
                                f"H_kv={pc.num_kv_heads}, D={pc.head_dim}, seed {case.seed}"),
                   "global_batch": pc.batch, "kv_bytes_per_step": kv_bytes,
                   "step": ("append_kv + padded decode + lse merge: "
                            "pa_append_decode_attention_padded (one launch)")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "cache": ("warm: decode calls back to back; the flushed figures write "
                               f"{args.flush_mb} MB between single calls"),
                     "achieved_flushed": round(flushed_gbs, 1),
                     "frac_flushed": round(flushed_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": ("pa_decode_attention_padded call (decode_vector_kernel, padded "
                                "split grid merging its own splits)"),
                     "bytes_per_launch": kv_bytes,
                     "avg_launch_us": round(dec_avg_ms * 1e3, 2)},
        "detail": {"us_per_step": round(ms_per_step * 1e3, 2),
                   "us_per_step_events": round(step_ev_ms * 1e3, 2),
                   "us_per_step_separate_calls": round(sep_ms * 1e3, 2),
                   "us_per_step_separate_calls_events": round(sep_ev_ms * 1e3, 2),
                   "decode_us_flushed_median": round(statistics.median(fl) * 1e3, 2),
                   "paged_decode_us_same_run": round(paged_dec_ms * 1e3, 2),
                   "padded_over_paged_decode_time": round(dec_avg_ms / paged_dec_ms, 4),
                   "padded_pool_bytes": int(L.kv.k.numel() * L.kv.k.element_size() * 2),
                   "source_hash": kernel_source_hash(*DECODE_SOURCES)},
    }
    if not args.no_cpu_baseline:
        out_line["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(out_line), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.workload in ("mq", "mq-sparse"):
        main_mq(args)
        return
    if args.workload == "mq-tokenize":
        return main_tokenize(args)
    if args.workload == "b16":
        main_b16(args)
        return
    if args.workload == "b128-padded":
        main_b128_padded(args)
        return

    import numpy as np
    import torch

    import workloads as W
    from paged_kv_cache_177_amd.runner import PagedStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.workload == "b128":
        case = W.b128()
    elif args.workload == "long":
        case = W.long_context()
    else:
        case = W.shard_share(args.workload)
    kv_bytes = case.kv_bytes()
    r = PagedStep(case, device="cuda:0")
    stream = torch.cuda.current_stream()

    # untimed warm-up: at least W steps and at least one second of them (the GPU takes a while to
    # reach its steady clocks; shorter warm-ups measured up to 10% slow)
    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < 1.0:
        for _ in range(10):
            r.fused_step()
        done += 10
        torch.cuda.synchronize()

    def timed_steps(step):
        # back to back with nothing in between (a pair of timing events around every call would
        # add a few microseconds of GPU time to each step)
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ea.record(stream)
        for _ in range(args.steps):
            step()
        eb.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, ea.elapsed_time(eb) / args.steps

    def separate_step():
        r.append()
        r.decode()

    # The timed steps: one pa_append_decode_attention call each (the append folded into the
    # decode launch, then the merge). The same step as separate append and decode calls (the
    # same bits) is timed next, for comparison.
    ms_per_step, step_ev_ms = timed_steps(r.fused_step)
    for _ in range(args.warmup):
        separate_step()
    sep_ms, sep_ev_ms = timed_steps(separate_step)

    # The decode call's duration for the roofline: the same number of decode calls back to back
    # between one pair of events, on the stream they run on.
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ea.record(stream)
    for _ in range(args.steps):
        r.decode()
    eb.record(stream)
    torch.cuda.synchronize()
    dec_avg_ms = ea.elapsed_time(eb) / args.steps

    # The spread over single calls, each between its own pair of events (the events' own cost
    # is inside these figures).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        r.append()
        evs[i][0].record(stream)
        r.decode()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in evs]

    # extra: the append alone, and the append with per-head QK RMSNorm fused in (unit weights),
    # back-to-back calls between one pair of events each
    append_us, append_norm_us = append_timings(r, case, stream)

    # one GPU of four holding a quarter of each row: after the all-gather of the four shares'
    # (out, lse), pa_lse_merge combines them; here the share's own results stand in for the four.
    # Back-to-back calls of so short a kernel are paced by the host's call rate: its own duration
    # comes from the profiler.
    merge_us = None
    if args.workload == "long-sp4":
        from paged_kv_cache_177_amd import binding as B

        n_pairs = case.batch * case.num_q_heads
        parts_o = r.out.reshape(1, n_pairs, case.head_dim).repeat(4, 1, 1).contiguous()
        parts_l = r.lse.reshape(1, n_pairs).repeat(4, 1).contiguous()
        m_out = torch.empty((n_pairs, case.head_dim), dtype=torch.float32, device="cuda:0")
        m_lse = torch.empty((n_pairs,), dtype=torch.float32, device="cuda:0")
        for _ in range(10):
            B.pa_lse_merge(parts_o, parts_l, 4, n_pairs, case.head_dim, m_out, m_lse)
        ma, mb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ma.record(stream)
        for _ in range(args.steps):
            B.pa_lse_merge(parts_o, parts_l, 4, n_pairs, case.head_dim, m_out, m_lse)
        mb.record(stream)
        torch.cuda.synchronize()
        merge_us = ma.elapsed_time(mb) * 1e3 / args.steps

    # extra: decode calls with the last-level cache flushed before each one (outside the events)
    flush = torch.empty(args.flush_mb * (1 << 20), dtype=torch.uint8, device="cuda:0")
    fl = []
    for _ in range(10):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        r.decode()
        b.record(stream)
        torch.cuda.synchronize()
        fl.append(a.elapsed_time(b))
    del flush

    # extra: the practical read ceiling of this GPU, measured in the same run
    ceiling, ceiling_grid = read_ceiling_gbs()

    achieved = kv_bytes / (dec_avg_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash(*DECODE_SOURCES)
    traffic = read_traffic(src_hash) if args.workload == "b128" else None
    out = {
        "metric": (METRIC if args.workload == "b128" else
                   METRIC_LONG if args.workload == "long" else METRIC_SHARE[args.workload]),
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{case.name}: B={case.batch} ragged contexts "
                                f"{int(case.n_ctx.min())}..{int(case.n_ctx.max())} "
                                f"(kv_len sum {int(case.kv_lens.sum())}), H_q={case.num_q_heads}, "
                                f"H_kv={case.num_kv_heads}, D={case.head_dim}, 16-token blocks, "
                                f"shuffled pool of {case.num_blocks} blocks, seed {case.seed}"),
                   "global_batch": case.batch, "kv_bytes_per_step": kv_bytes,
                   "step": ("append_kv + decode + lse merge: pa_append_decode_attention (the "
                            "append folded into the decode launch) + the merge kernel"
                            if args.workload.startswith("long") else
                            "append_kv + decode + lse merge: pa_append_decode_attention (one "
                            "launch: the append folded into the split grid, which also merges "
                            "the splits)")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "cache": ("warm: decode calls back to back; the flushed figures write "
                               f"{args.flush_mb} MB between single calls"),
                     "achieved_flushed": round(kv_bytes / (statistics.median(fl) * 1e-3) / 1e9, 1),
                     "frac_flushed": round(kv_bytes / (statistics.median(fl) * 1e-3) / 1e9
                                           / HBM_PEAK_GBS, 4),
                     "traffic": (round(traffic / (dec_avg_ms * 1e-3) / 1e9, 1)
                                 if traffic is not None else None),
                     "kernel": ("pa_decode_attention call (decode_vector_kernel, split grid "
                                "merging its own splits)") if not args.workload.startswith("long")
                               else ("pa_decode_attention call (decode_vector_kernel, compact "
                                     "grid, + lse_reduce_kernel)"),
                     "bytes_per_launch": kv_bytes,
                     "avg_launch_us": round(dec_avg_ms * 1e3, 2)},
        "detail": {"us_per_step": round(ms_per_step * 1e3, 2),
                   "us_per_step_events": round(step_ev_ms * 1e3, 2),
                   "us_per_step_separate_calls": round(sep_ms * 1e3, 2),
                   "us_per_step_separate_calls_events": round(sep_ev_ms * 1e3, 2),
                   "pct_hbm_peak_step": round(100 * kv_bytes / (ms_per_step * 1e-3) / 1e9
                                              / HBM_PEAK_GBS, 2),
                   "decode_us_single_call_median": round(statistics.median(dec_ms) * 1e3, 2),
                   "decode_us_single_call_p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                   "decode_us_single_call_p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
                   "decode_us_flushed_median": round(statistics.median(fl) * 1e3, 2),
                   "kv_gbs_flushed": round(kv_bytes / (statistics.median(fl) * 1e-3) / 1e9, 1),
                   "traffic_bytes_per_call": traffic,
                   "hbm_read_ceiling_gbs": round(ceiling, 1),
                   "hbm_read_ceiling_grid": ceiling_grid,
                   "decode_pct_of_read_ceiling": round(100 * achieved / ceiling, 1),
                   "append_us": round(append_us, 2),
                   "append_qk_norm_us": round(append_norm_us, 2),
                   "lse_merge_4_parts_us_per_call_events":
                       None if merge_us is None else round(merge_us, 2),
                   "source_hash": src_hash},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case)
    if args.traffic_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
