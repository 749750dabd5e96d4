"""Benchmark of the WKV-7 state-slot hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one decode call of the 256-active-slot workload: a pool of 1024
fp32 state slots, H=32 heads of N=64, one token per active slot with bf16
r,w,k,v,a,b drawn from the synthetic recipe (fresh inputs every step, all
pre-generated in HBM before timing). W untimed steps, then exactly K timed
steps bracketed by device synchronisation. Prints ONE JSON line.

The line carries the decode kernel's roofline (algorithmic bytes per launch
over its average duration, timed with HIP events on the launch stream), the
float64 CPU oracle's rate on a bounded sample of the same workload, and, when
built, a chunked-prefill leg (8 sequences of 4096 tokens, H=32).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = ("WKV-7 tokens/s (decode B slots; prefill) + % of HBM peak / MFMA "
          "util, 1 GPU")
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
N = 64


def decode_bytes_per_token_head(in_bytes: int = 2) -> int:
    """State read + written (fp32), six input vectors, fp32 output."""
    return 2 * 4 * N * N + 6 * N * in_bytes + N * 4


def kernel_sha(names) -> str:
    """Digest of the kernel's source files (a name or a list of names under
    csrc/, in order)."""
    h = hashlib.sha256()
    for name in ([names] if isinstance(names, str) else names):
        with open(os.path.join(ROOT, "linear_attention_rnn_amd", "csrc",
                               name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kind: str, bytes_alg: float):
    """HBM bytes per launch from committed rocprofv3 PMC counters, if they
    were taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kind}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha(t["kernel_src"]):
        return None
    return float(t["hbm_bytes_per_launch"])


# Raw TCC read-request counts by size and write-request counts: the bytes a
# kernel moves between the L2 and the memory side, with no fitted factor.
RAW_READ = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum",
            "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")
RAW_WRITE = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")


def pmc_summary(paths, kernel: str) -> dict:
    """Means per dispatch of the counters in rocprofv3 counter-collection
    CSVs (one or more passes) for kernels whose name contains `kernel`,
    grouped by grid size; with the raw request counts present, the bytes
    read (32/64/128-byte requests) and written (64-byte requests and the
    rest as 32-byte ones) per dispatch."""
    import csv
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    grids = {}
    for path in paths:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if kernel not in row["Kernel_Name"]:
                    continue
                key = (path, int(row["Dispatch_Id"]))
                per[key][row["Counter_Name"]] += float(row["Counter_Value"])
                grids[key] = int(row["Grid_Size"])
    groups = collections.defaultdict(lambda: collections.defaultdict(list))
    distinct = collections.defaultdict(collections.Counter)
    for key, cs in per.items():
        for c, v in cs.items():
            groups[grids[key]][c].append(v)
        if all(c in cs for c in RAW_READ):
            rb = (128 * cs["TCC_EA0_RDREQ_128B_sum"] +
                  64 * cs["TCC_EA0_RDREQ_64B_sum"] +
                  32 * cs["TCC_EA0_RDREQ_32B_sum"])
            distinct[grids[key]][f"read {rb / 2**20:.2f} MiB"] += 1
        if all(c in cs for c in RAW_WRITE):
            wb = (64 * cs["TCC_EA0_WRREQ_64B_sum"] + 32 *
                  (cs["TCC_EA0_WRREQ_sum"] - cs["TCC_EA0_WRREQ_64B_sum"]))
            distinct[grids[key]][f"write {wb / 2**20:.2f} MiB"] += 1
    out = {}
    for g, cs in sorted(groups.items()):
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        m["dispatches"] = max(len(v) for v in cs.values())
        if distinct[g]:
            m["per_dispatch_values"] = dict(distinct[g])
        if all(c in m for c in RAW_READ):
            m["read_bytes"] = (128 * m["TCC_EA0_RDREQ_128B_sum"] +
                               64 * m["TCC_EA0_RDREQ_64B_sum"] +
                               32 * m["TCC_EA0_RDREQ_32B_sum"])
        if all(c in m for c in RAW_WRITE):
            m["write_bytes"] = (64 * m["TCC_EA0_WRREQ_64B_sum"] + 32 *
                                (m["TCC_EA0_WRREQ_sum"] -
                                 m["TCC_EA0_WRREQ_64B_sum"]))
        out[f"grid{g}"] = m
    return out


def run_decode(steps: int, warmup: int, seed: int = 1):
    import torch
    import wkv7_inputs as G
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    n_slots, n_active, H = 1024, 256, 32
    rng = np.random.default_rng(seed)
    ids = rng.permutation(n_slots)[:n_active].astype(np.int32)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    pool = W.wkv7_pool_create(n_slots, H, N)
    try:
        # resident states N(0, 0.1) in every slot
        init = torch.randn((n_slots, H, N, N), device=dev, generator=gen) * 0.1
        W.wkv7_resume(pool, np.arange(n_slots, dtype=np.int32), init)
        del init
        total = steps + warmup
        xs = [G.draw_tokens_device(gen, n_active, H, N, "bf16", dev)
              for _ in range(total)]
        cu = np.arange(n_active + 1, dtype=np.int32)
        o = torch.empty((n_active, H, N), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()
        torch.cuda.synchronize()

        # the batch layout is the same every step: validate it and put it
        # on the device once, then each step only launches the kernel
        plan = W.wkv7_plan_create(pool, ids, cu)

        def step(x):
            W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o, stream=stream)

        for i in range(warmup):
            step(xs[i])
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            step(xs[warmup + i])
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        # one kernel per step, back to back on the stream: the events'
        # span over K launches is the average launch duration (with the
        # gaps between launches, so never below the kernel's own time)
        k_ms = ev0.elapsed_time(ev1) / steps

        # the same steps through wkv7_forward (host-side validation and
        # metadata staging on every call), for reference
        torch.cuda.synchronize()
        f0 = time.perf_counter()
        for i in range(steps):
            x = xs[warmup + i]
            W.wkv7_forward(pool, ids, cu, x["r"], x["w"], x["k"], x["v"],
                           x["a"], x["b"], o, stream=stream)
        torch.cuda.synchronize()
        f1 = time.perf_counter()
        W.wkv7_plan_destroy(plan)
    finally:
        W.wkv7_pool_destroy(pool)
    wall = t1 - t0
    bytes_launch = n_active * H * decode_bytes_per_token_head(2)
    return {
        "tokens": n_active * steps, "wall_s": wall,
        "ms_per_step": wall / steps * 1e3,
        "forward_ms_per_step": (f1 - f0) / steps * 1e3,
        "kernel_ms": float(k_ms),
        "bytes_per_launch": bytes_launch, "n_active": n_active, "H": H,
        "n_slots": n_slots,
    }


def chunk_mfma_flops_per_chunk_head() -> int:
    """MFMA flops the chunked-prefill kernel's fast plan (bf16 inputs) issues
    per 32-token chunk and head, from the instructions in its compiled loop
    body: each of the
    4 t wavefronts issues 18 v_mfma_f32_16x16x32_bf16 (its Gram matrix),
    each of the 4 value wavefronts 24 v_mfma_f32_16x16x32_f16 and one
    v_mfma_f32_16x16x16_f16 (T_10), and the two value wavefronts that build
    T's diagonal blocks 20 v_mfma_f32_16x16x16_f16 between them (16384 and
    8192 flops per instruction)."""
    return 4 * 18 * 16384 + 4 * 24 * 16384 + (4 + 20) * 8192


def chunk_mfma_flops_per_chunk_head_precise() -> int:
    """MFMA flops of the chunked kernel's precise plan per 32-token chunk and
    head, from the instructions its compiled loop issues (383 per chunk and
    head in the SQ counters): the 4 t wavefronts' Gram products as in the
    fast plan, 72 v_mfma_f32_16x16x32_bf16 on each value wavefront (X 18,
    U 6, O 24, the state 24), and T's 23 v_mfma_f32_16x16x16_f16 on the Gram
    wavefront."""
    return 4 * 18 * 16384 + 4 * 72 * 16384 + 23 * 8192


CHUNK_L = 32        # chunk length of the chunked-prefill kernel


def prefill_alg_flops_per_token_head(L: int = CHUNK_L) -> float:
    """Dense flop count of the chunked form per token and head:
    16 L N + 8 N^2 + (2/3) L^2 + N^2 / L."""
    return 16 * L * N + 8 * N * N + (2.0 / 3.0) * L * L + N * N / L


def run_prefill(steps: int, warmup: int, seed: int = 2):
    """8 fresh sequences of 4096 tokens, H=32, bf16 inputs, zero state; one
    step = reset the 8 slots + one forward over the packed batch. The
    forward is timed with HIP events on the launch stream."""
    import torch
    import wkv7_inputs as G
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    n_seq, T, H = 8, 4096, 32
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    x = G.draw_tokens_device(gen, n_seq * T, H, N, "bf16", dev)
    ids = np.arange(n_seq, dtype=np.int32)
    cu = (np.arange(n_seq + 1) * T).astype(np.int32)
    o = torch.empty((n_seq * T, H, N), dtype=torch.float32, device=dev)
    pool = W.wkv7_pool_create(n_seq, H, N)
    stream = torch.cuda.current_stream()
    try:
        plan = W.wkv7_plan_create(pool, ids, cu)

        def step():
            W.wkv7_reset(pool, ids, stream=stream)
            W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o, stream=stream)

        for _ in range(warmup):
            step()
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            W.wkv7_reset(pool, ids, stream=stream)
            ev0[i].record(stream)
            W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o, stream=stream)
            ev1[i].record(stream)
        torch.cuda.synchronize()
        k_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(ev0, ev1)]))
        W.wkv7_plan_destroy(plan)
    finally:
        W.wkv7_pool_destroy(pool)
    tokens = n_seq * T
    chunks = n_seq * (T // CHUNK_L)
    bytes_alg = tokens * H * (6 * N * 2 + N * 4) + n_seq * H * 2 * 4 * N * N
    issued = chunks * H * chunk_mfma_flops_per_chunk_head()
    alg = tokens * H * prefill_alg_flops_per_token_head()
    sec = k_ms * 1e-3
    return {
        "workload": "prefill_b8_t4096_h32_bf16in_f32state",
        "tokens_per_s": tokens / sec,
        "kernel": "chunk_p_kernel (bf16 inputs, chunks of 32 tokens)",
        "kernel_ms": k_ms,
        "hbm": {"achieved": bytes_alg / sec / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": bytes_alg / sec / 1e9 / HBM_PEAK_GBS,
                "bytes_per_launch": bytes_alg,
                "traffic": load_traffic("prefill", bytes_alg)},
        "mfma": {"issued_tflops": issued / sec / 1e12,
                 "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "util": issued / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                 "issued_flops_per_launch": issued,
                 "algorithmic_tflops": alg / sec / 1e12},
        "steps": steps, "warmup": warmup,
    }


def run_prefill_f32(steps: int = 5, warmup: int = 3, seed: int = 2):
    """The 8 x 4096 x H=32 prefill with fp32 inputs, which take the chunked
    kernel's precise plan (chunks of 32, every product from split-bf16
    operands); one step = reset the 8 slots + one plan forward, timed with an
    event pair around the forward."""
    import torch
    import wkv7_inputs as G
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    n_seq, T, H = 8, 4096, 32
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    x = G.draw_tokens_device(gen, n_seq * T, H, N, "f32", dev)
    ids = np.arange(n_seq, dtype=np.int32)
    cu = (np.arange(n_seq + 1) * T).astype(np.int32)
    o = torch.empty((n_seq * T, H, N), dtype=torch.float32, device=dev)
    pool = W.wkv7_pool_create(n_seq, H, N)
    stream = torch.cuda.current_stream()
    try:
        plan = W.wkv7_plan_create(pool, ids, cu)
        times = []
        for i in range(warmup + steps):
            W.wkv7_reset(pool, ids, stream=stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= warmup:
                times.append(e0.elapsed_time(e1))
        W.wkv7_plan_destroy(plan)
    finally:
        W.wkv7_pool_destroy(pool)
    k_ms = float(np.mean(times))
    tokens = n_seq * T
    bytes_alg = tokens * H * (6 * N * 4 + N * 4) + n_seq * H * 2 * 4 * N * N
    issued = (tokens // CHUNK_L) * H * chunk_mfma_flops_per_chunk_head_precise()
    sec = k_ms * 1e-3
    return {"workload": "prefill_b8_t4096_h32_f32in_f32state",
            "kernel": "chunk_p_kernel<fp32, precise> (chunks of 32, "
                      "split-bf16 products)",
            "tokens_per_s": tokens / (k_ms * 1e-3), "kernel_ms": k_ms,
            "hbm": {"achieved": bytes_alg / (k_ms * 1e-3) / 1e9,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": bytes_alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "bytes_per_launch": bytes_alg,
                    "traffic": load_traffic("prefill_f32", bytes_alg)},
            "mfma": {"issued_tflops": issued / sec / 1e12,
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "util": issued / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                     "issued_flops_per_launch": issued},
            "steps": steps, "warmup": warmup}


def _draw_device(gen, T: int, H: int, dtype: str, dev, chunk: int = 16384):
    """Synthetic inputs [T, H, N] drawn on the device in token chunks (the
    float32 temporaries of a whole large batch would be several GB)."""
    import torch
    import wkv7_inputs as G
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {n: torch.empty((T, H, N), dtype=td, device=dev) for n in G.NAMES}
    for t0 in range(0, T, chunk):
        x = G.draw_tokens_device(gen, min(chunk, T - t0), H, N, dtype, dev)
        for n in G.NAMES:
            out[n][t0:t0 + x[n].shape[0]].copy_(x[n])
    return out


def run_small(calls: int = 200, warmup: int = 20, seed: int = 0):
    """The small case: one sequence of 64 tokens, H=2, fp32 inputs, from a
    zeroed slot (64 tokens take the chunked kernel). Launch-bound: reported
    as microseconds per call, through wkv7_forward (host validation and
    metadata staging each call) and through a plan, with no roofline."""
    import torch
    import wkv7_inputs as G
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    H, T = 2, 64
    b = G.make_batch(np.random.default_rng(seed), [0], [T], H, N, G.F32)
    x = {n: b.inputs[n].to(dev) for n in G.NAMES}
    o = torch.empty((T, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    pool = W.wkv7_pool_create(1, H, N)
    out = {"workload": "small_h2_t64_f32in_zero_state"}
    try:
        plan = W.wkv7_plan_create(pool, b.slot_ids, b.cu_seqlens)

        def fwd():
            W.wkv7_forward(pool, b.slot_ids, b.cu_seqlens, x["r"], x["w"],
                           x["k"], x["v"], x["a"], x["b"], o, stream=stream)

        def fwd_plan():
            W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o, stream=stream)

        for name, fn in (("forward", fwd), ("plan", fwd_plan)):
            for _ in range(warmup):
                fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record(stream)
            for _ in range(calls):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            out[f"{name}_us_per_call_wall"] = (t1 - t0) / calls * 1e6
            out[f"{name}_us_per_call_gpu"] = e0.elapsed_time(e1) / calls * 1e3
        # the same plan call captured 50 times into one HIP graph (on torch's
        # capture stream, current inside the block) and replayed
        n_cap, reps = 50, max(1, calls // 50)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(n_cap):
                W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"],
                                    x["v"], x["a"], x["b"], o)
        torch.cuda.synchronize()
        graph.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        out["graph_us_per_call_wall"] = (t1 - t0) / (reps * n_cap) * 1e6
        out["graph_us_per_call_gpu"] = e0.elapsed_time(e1) / (reps * n_cap) * 1e3
        del graph
        W.wkv7_plan_destroy(plan)
    finally:
        W.wkv7_pool_destroy(pool)
    out["calls"] = calls
    return out


def run_short(reps: int = 50, warmup: int = 5, seed: int = 6):
    """Short multi-token sequences: GPU microseconds per plan call on the
    default split (sequential below PREFILL_MIN_LEN tokens) and with every
    sequence forced onto each kernel, for a few (sequence, head) chains
    (8 sequences x H=32, latency-bound) and for many (256 x H=32,
    throughput-bound). bf16 and fp32 inputs, zeroed slots, fresh-drawn
    synthetic tokens."""
    import torch
    import wkv7_inputs as G
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    H = 32
    big = 1 << 30
    out = {"workload": "short_sequences_h32", "unit": "us per call (GPU)",
           "cases": []}
    for dtype in ("bf16", "f32"):
        for nseq, T in ((8, 8), (8, 24), (8, 48), (256, 8), (256, 24)):
            g = torch.Generator(device=dev)
            g.manual_seed(seed)
            x = G.draw_tokens_device(g, nseq * T, H, N, dtype, dev)
            o = torch.empty((nseq * T, H, N), dtype=torch.float32, device=dev)
            ids = np.arange(nseq, dtype=np.int32)
            cu = (np.arange(nseq + 1) * T).astype(np.int32)
            case = {"dtype": dtype, "n_seq": nseq, "T": T}
            for name, min_len in (("default", None), ("sequential", big),
                                  ("chunked", 1)):
                pool = W.wkv7_pool_create(nseq, H, N)
                try:
                    if min_len is not None:
                        W.wkv7_pool_set_option(
                            pool, W.WKV7_OPT_PREFILL_MIN_LEN, min_len)
                    plan = W.wkv7_plan_create(pool, ids, cu)

                    def call():
                        W.wkv7_forward_plan(pool, plan, x["r"], x["w"],
                                            x["k"], x["v"], x["a"], x["b"],
                                            o, stream=stream)
                    for _ in range(warmup):
                        call()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    torch.cuda.synchronize()
                    e0.record(stream)
                    for _ in range(reps):
                        call()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    case[name] = e0.elapsed_time(e1) / reps * 1e3
                    W.wkv7_plan_destroy(plan)
                finally:
                    W.wkv7_pool_destroy(pool)
            out["cases"].append(case)
    return out


def run_decode_cold(steps: int = 20, warmup: int = 3, seed: int = 1):
    """The headline decode batch shape with a new random 256-slot subset of
    the 1024-slot pool every step (the pool's 512 MiB is twice the MALL, so
    a step's slots are mostly not cached from the step before). One plan per
    step, built before timing; one event pair over the K launches."""
    import torch
    import wkv7_inputs as G
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    n_slots, n_active, H = 1024, 256, 32
    rng = np.random.default_rng(seed + 100)
    total = steps + warmup
    id_sets = [rng.permutation(n_slots)[:n_active].astype(np.int32)
               for _ in range(total)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 100)
    pool = W.wkv7_pool_create(n_slots, H, N)
    plans = []
    try:
        init = torch.randn((n_slots, H, N, N), device=dev, generator=gen) * 0.1
        W.wkv7_resume(pool, np.arange(n_slots, dtype=np.int32), init)
        del init
        xs = [G.draw_tokens_device(gen, n_active, H, N, "bf16", dev)
              for _ in range(total)]
        cu = np.arange(n_active + 1, dtype=np.int32)
        o = torch.empty((n_active, H, N), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()
        plans = [W.wkv7_plan_create(pool, ids, cu) for ids in id_sets]

        def step(i):
            x = xs[i]
            W.wkv7_forward_plan(pool, plans[i], x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o, stream=stream)

        for i in range(warmup):
            step(i)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(steps):
            step(warmup + i)
        ev1.record(stream)
        torch.cuda.synchronize()
        k_ms = ev0.elapsed_time(ev1) / steps
    finally:
        for pl in plans:
            W.wkv7_plan_destroy(pl)
        W.wkv7_pool_destroy(pool)
    bytes_launch = n_active * H * decode_bytes_per_token_head(2)
    gbs = bytes_launch / (k_ms * 1e-3) / 1e9
    return {
        "workload": "decode_b256_h32_pool1024_bf16in_f32state_new_subset_each_step",
        "tokens_per_s": n_active / (k_ms * 1e-3), "kernel_ms": k_ms,
        "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": bytes_launch},
        "steps": steps, "warmup": warmup,
    }


def run_decode_large(steps: int = 20, warmup: int = 3, seed: int = 4):
    """The large-pool decode step: 1024 random slots of a 4096-slot pool,
    H=64 (1 GiB of active state, four times the MALL), fresh bf16 inputs
    every step, launched through a plan; one event pair over the K steps."""
    import torch
    import wkv7_inputs as G
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    n_slots, n_active, H = 4096, 1024, 64
    ids = np.random.default_rng(seed).permutation(n_slots)[:n_active].astype(
        np.int32)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    pool = W.wkv7_pool_create(n_slots, H, N)
    try:
        init = torch.randn((n_active, H, N, N), device=dev, generator=gen) * 0.1
        W.wkv7_resume(pool, ids, init)
        del init
        xs = [G.draw_tokens_device(gen, n_active, H, N, "bf16", dev)
              for _ in range(steps + warmup)]
        cu = np.arange(n_active + 1, dtype=np.int32)
        o = torch.empty((n_active, H, N), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()
        plan = W.wkv7_plan_create(pool, ids, cu)
        for i in range(warmup):
            x = xs[i]
            W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o, stream=stream)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(steps):
            x = xs[warmup + i]
            W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o, stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        k_ms = ev0.elapsed_time(ev1) / steps
        W.wkv7_plan_destroy(plan)
        # hibernate 256 of the touched slots into pinned host memory and
        # resume them (1 MiB per slot; DMA over PCIe)
        hib_ids = ids[:256]
        host = torch.empty((256, H, N, N), dtype=torch.float32,
                           pin_memory=True)
        hib_bytes = host.numel() * 4
        t_h, t_r = [], []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e2 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            W.wkv7_hibernate(pool, hib_ids, host, stream=stream)
            e1.record(stream)
            W.wkv7_resume(pool, hib_ids, host, stream=stream)
            e2.record(stream)
            torch.cuda.synchronize()
            t_h.append(e0.elapsed_time(e1))
            t_r.append(e1.elapsed_time(e2))
        del host
    finally:
        W.wkv7_pool_destroy(pool)
    bytes_launch = n_active * H * decode_bytes_per_token_head(2)
    gbs = bytes_launch / (k_ms * 1e-3) / 1e9
    hib = {"slots": 256, "bytes": hib_bytes,
           "hibernate_GBps": hib_bytes / (min(t_h) * 1e-3) / 1e9,
           "resume_GBps": hib_bytes / (min(t_r) * 1e-3) / 1e9,
           "hibernate_ms": min(t_h), "resume_ms": min(t_r),
           "note": "pinned host memory, best of 3"}
    return {
        "hibernate_resume": hib,
        "workload": "decode_b1024_h64_pool4096_bf16in_f32state",
        "tokens_per_s": n_active / (k_ms * 1e-3), "kernel_ms": k_ms,
        "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": bytes_launch,
                "traffic": load_traffic("decode_large", bytes_launch)},
        "steps": steps, "warmup": warmup,
    }


def run_prefill_ragged(steps: int = 3, warmup: int = 3, seed: int = 4):
    """32 fresh sequences with lengths integer-uniform in [128, 8192], H=64,
    bf16 inputs; one step = reset the 32 slots + one plan forward (timed
    with an event pair around the forward)."""
    import torch
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    H, n_seq = 64, 32
    lens = np.random.default_rng(seed).integers(128, 8193, size=n_seq)
    T = int(lens.sum())
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    x = _draw_device(gen, T, H, "bf16", dev)
    ids = np.arange(n_seq, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o = torch.empty((T, H, N), dtype=torch.float32, device=dev)
    pool = W.wkv7_pool_create(n_seq, H, N)
    stream = torch.cuda.current_stream()
    try:
        plan = W.wkv7_plan_create(pool, ids, cu)
        times = []
        for i in range(warmup + steps):
            W.wkv7_reset(pool, ids, stream=stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= warmup:
                times.append(e0.elapsed_time(e1))
        W.wkv7_plan_destroy(plan)
    finally:
        W.wkv7_pool_destroy(pool)
    k_ms = float(np.mean(times))
    sec = k_ms * 1e-3
    bytes_alg = T * H * (6 * N * 2 + N * 4) + n_seq * H * 2 * 4 * N * N
    chunks = int(sum((int(n) + CHUNK_L - 1) // CHUNK_L for n in lens))
    issued = chunks * H * chunk_mfma_flops_per_chunk_head()
    return {
        "workload": "prefill_32ragged_128to8192_h64_bf16in_f32state",
        "tokens": T, "tokens_per_s": T / sec, "kernel_ms": k_ms,
        "hbm": {"achieved": bytes_alg / sec / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": bytes_alg / sec / 1e9 / HBM_PEAK_GBS,
                "bytes_per_launch": bytes_alg},
        "mfma": {"issued_tflops": issued / sec / 1e12,
                 "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "util": issued / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS},
        "steps": steps, "warmup": warmup,
    }


def run_mixed(steps: int = 10, warmup: int = 2, seed: int = 3,
              segment_len: int = 0):
    """The 12-layer RWKV-X-0.2B-shaped stack (H=12, one 128-slot pool per
    layer): per layer and step 64 decode tokens plus 4 fresh prefills of
    512, 1024, 2048 and 2048 tokens in one packed call (the prefill slots
    are reset first); fresh inputs per layer and step; one event pair over
    the K steps of 12 layers. segment_len > 0 turns on segment-parallel
    prefill with segments of that many tokens."""
    import torch
    import wkv7_inputs as G
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    n_layers, n_slots, H = 12, 128, 12
    prefill_lens = [512, 1024, 2048, 2048]
    perm = np.random.default_rng(seed).permutation(n_slots).astype(np.int32)
    dec_ids, pre_ids = perm[:64], perm[64:68]
    ids = np.concatenate([dec_ids, pre_ids])
    lens = [1] * 64 + prefill_lens
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    pools, plans = [], []
    stream = torch.cuda.current_stream()
    try:
        for _ in range(n_layers):
            pool = W.wkv7_pool_create(n_slots, H, N)
            pools.append(pool)
            W.wkv7_pool_set_option(pool, W.WKV7_OPT_SEGMENT_LEN, segment_len)
            init = torch.randn((64, H, N, N), device=dev, generator=gen) * 0.1
            W.wkv7_resume(pool, dec_ids, init)
            plans.append(W.wkv7_plan_create(pool, ids, cu))
        xs = [[G.draw_tokens_device(gen, T, H, N, "bf16", dev)
               for _ in range(n_layers)] for _ in range(steps + warmup)]
        o = torch.empty((T, H, N), dtype=torch.float32, device=dev)

        def step(i):
            for li in range(n_layers):
                x = xs[i][li]
                W.wkv7_reset(pools[li], pre_ids, stream=stream)
                W.wkv7_forward_plan(pools[li], plans[li], x["r"], x["w"],
                                    x["k"], x["v"], x["a"], x["b"], o,
                                    stream=stream)

        for i in range(warmup):
            step(i)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(steps):
            step(warmup + i)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
    finally:
        for pl in plans:
            W.wkv7_plan_destroy(pl)
        for pool in pools:
            W.wkv7_pool_destroy(pool)
    bytes_layer = (64 * H * decode_bytes_per_token_head(2)
                   + sum(prefill_lens) * H * (6 * N * 2 + N * 4)
                   + 4 * H * 2 * 4 * N * N)
    return {
        "workload": "mixed_12layers_h12_64decode_4prefill_bf16in",
        "segment_len": segment_len,
        "tokens_per_step": T, "ms_per_step": ms,
        "tokens_per_s": T / (ms * 1e-3),
        "layer_tokens_per_s": n_layers * T / (ms * 1e-3),
        "hbm": {"achieved": n_layers * bytes_layer / (ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": n_layers * bytes_layer / (ms * 1e-3) / 1e9
                / HBM_PEAK_GBS},
        "steps": steps, "warmup": warmup,
    }


def run_prefill_long(T: int = 32768, H: int = 32, steps: int = 3,
                     warmup: int = 2, seed: int = 6, segment_len: int = 4096):
    """One fresh sequence of T tokens at H=32 (the time to prefill one long
    prompt): H chains only, so most CUs would idle; timed unsplit and with
    segment-parallel prefill (segments of segment_len tokens), each step a
    reset + one plan forward timed with an event pair."""
    import torch
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    x = _draw_device(gen, T, H, "bf16", dev)
    o = torch.empty((T, H, N), dtype=torch.float32, device=dev)
    ids = np.zeros(1, dtype=np.int32)
    cu = np.array([0, T], dtype=np.int32)
    stream = torch.cuda.current_stream()
    out = {"workload": f"prefill_1x{T}_h{H}_bf16in_f32state",
           "segment_len": segment_len}
    for name, seg in (("unsplit", 0), ("segmented", segment_len)):
        pool = W.wkv7_pool_create(1, H, N)
        try:
            W.wkv7_pool_set_option(pool, W.WKV7_OPT_SEGMENT_LEN, seg)
            plan = W.wkv7_plan_create(pool, ids, cu)
            times = []
            for i in range(warmup + steps):
                W.wkv7_reset(pool, ids, stream=stream)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"],
                                    x["v"], x["a"], x["b"], o, stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                if i >= warmup:
                    times.append(e0.elapsed_time(e1))
            W.wkv7_plan_destroy(plan)
        finally:
            W.wkv7_pool_destroy(pool)
        ms = float(np.mean(times))
        out[name] = {"ms": ms, "tokens_per_s": T / (ms * 1e-3)}
    return out


INT8_MFMA_PEAK_TOPS = 5000.0


def run_q8_proj(steps: int = 50, warmup: int = 5, seed: int = 5):
    """The INT8 projections upstream of the recurrence in decode: the six
    weight matrices r, w, k, v, a, b of a C=2048 layer stacked into one
    [12288, 2048] int8 matrix (quantized once, outside the timed region);
    a step quantizes the B input rows (bf16) and runs the INT8 product,
    through wkv7_q8_linear (one launch for up to four tokens) and, for
    reference, through wkv7_q8_quantize + wkv7_q8_matmul. B=256 (the decode
    batch) and B=1 (one sequence's matrix-vector product), each timed with
    one event pair over K steps."""
    import torch
    from linear_attention_rnn_amd import wkv7 as W

    dev = torch.device("cuda:0")
    C = 2048
    O = 6 * C
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    w = (torch.randn((O, C), device=dev, generator=gen) / C ** 0.5).to(
        torch.bfloat16)
    wq = torch.empty((O, C), dtype=torch.int8, device=dev)
    ws = torch.empty(O, dtype=torch.float32, device=dev)
    W.wkv7_q8_quantize(w, wq, ws)
    stream = torch.cuda.current_stream()
    out = {}
    for B in (256, 1):
        xs = [torch.randn((B, C), device=dev, generator=gen).to(torch.bfloat16)
              for _ in range(8)]
        xq = torch.empty((B, C), dtype=torch.int8, device=dev)
        xsc = torch.empty(B, dtype=torch.float32, device=dev)
        y = torch.empty((B, O), dtype=torch.float32, device=dev)

        def step_two(i):
            W.wkv7_q8_quantize(xs[i % 8], xq, xsc, stream=stream)
            W.wkv7_q8_matmul(wq, ws, xq, xsc, y, stream=stream)

        def step(i):                    # one call (one launch for B <= 4)
            W.wkv7_q8_linear(wq, ws, xs[i % 8], xq, xsc, y, stream=stream)

        def timed(fn):
            for i in range(warmup):
                fn(i)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(steps):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps * 1e3

        us_two = timed(step_two)
        us = timed(step)
        # the same steps replayed from a captured HIP graph (no host launch
        # cost between kernels: the GPU's own rate for these short kernels)
        n_cap = 20
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_cap):
                W.wkv7_q8_linear(wq, ws, xs[i % 8], xq, xsc, y)
        torch.cuda.synchronize()
        graph.replay()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        reps = max(1, steps // n_cap)
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(reps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        us_graph = g0.elapsed_time(g1) / (reps * n_cap) * 1e3
        del graph
        ops = 2.0 * B * O * C
        nbytes = O * C + 4 * O + B * C * 2 + B * C + 4 * B + 4 * B * O
        out[f"b{B}"] = {
            "us_per_step": us, "two_calls_us_per_step": us_two,
            "graph_us_per_step": us_graph,
            "tops": ops / (us * 1e-6) / 1e12,
            "mfma_frac": ops / (us * 1e-6) / 1e12 / INT8_MFMA_PEAK_TOPS,
            "hbm_gbs": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_step": nbytes,
        }
    return {"workload": "q8_proj_c2048_stacked6_bf16in", "peak_int8_tops":
            INT8_MFMA_PEAK_TOPS, **out, "steps": steps, "warmup": warmup}


def run_ceilings(reps: int = 10):
    """What the chip sustains, measured with the probe library: uint4
    streaming copies over the decode legs' state sizes (in place, as the
    decode kernel reads and rewrites its slots; the large one also with
    non-temporal loads and stores, and source to destination) and matrix-core
    loops. Copy rates count bytes read plus bytes written; each figure is
    the best over a few launch shapes, timed with one event pair around
    `reps` back-to-back launches after a warm-up."""
    import torch
    from linear_attention_rnn_amd import hw_probe as P

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn, n=reps):
        fn()
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    def copy_gbs(src, dst, nbytes, nt):
        best = 0.0
        for blocks in (1024, 2048, 4096, 8192):
            t = timed(lambda: P.hwprobe_copy(src, dst, nbytes, nt, blocks,
                                             stream))
            best = max(best, 2 * nbytes / t / 1e9)
        return best

    out = {"unit_copy": "GB/s (read + written)", "unit_mfma": "TFLOP/s"}
    small = 128 << 20           # the headline decode's active state
    big = 1 << 30               # the large-pool decode's active state
    a = torch.empty(big // 4, dtype=torch.float32, device=dev).normal_()
    out["copy_inplace_128MiB"] = copy_gbs(a, a, small, False)
    out["copy_inplace_1GiB"] = copy_gbs(a, a, big, False)
    out["copy_inplace_1GiB_nt"] = copy_gbs(a, a, big, True)
    # 128 MiB windows of a 512 MiB buffer, a different window each launch:
    # no reuse between launches. The cold decode leg reads a random quarter
    # of its 512 MiB pool per step, which overlaps the previous step's slots
    # by a quarter on average, so it can exceed this figure; it is reported
    # against the published peak only.
    win = [a[i * (small // 4):(i + 1) * (small // 4)] for i in range(4)]
    best = 0.0
    for blocks in (2048, 8192):
        k = {"i": 0}

        def rot():
            w = win[k["i"] % 4]
            k["i"] += 1
            P.hwprobe_copy(w, w, small, False, blocks, stream)
        best = max(best, 2 * small / timed(rot, 12) / 1e9)
    out["copy_inplace_128MiB_rotating_512MiB"] = best
    b = torch.empty_like(a)
    out["copy_1GiB_nt"] = copy_gbs(a, b, big, True)
    out["torch_copy_1GiB"] = 2 * big / timed(lambda: b.copy_(a)) / 1e9
    del b
    # PCIe: one contiguous 256 MiB DMA each way with pinned host memory
    host = torch.empty(64 << 20, dtype=torch.float32, pin_memory=True)
    dsub = a[:64 << 20]
    out["pcie_d2h_256MiB"] = (256 << 20) / timed(
        lambda: host.copy_(dsub, non_blocking=True), 3) / 1e9
    out["pcie_h2d_256MiB"] = (256 << 20) / timed(
        lambda: dsub.copy_(host, non_blocking=True), 3) / 1e9
    out["unit_pcie"] = "GB/s (one direction)"
    del a, host, dsub
    blocks = 1024               # four workgroups of four wavefronts per CU
    res = torch.empty(blocks * P.WAVES_PER_BLOCK, dtype=torch.float32,
                      device=dev)
    for kind, key, iters in ((P.MFMA_BF16, "mfma_bf16_16x16x32", 20000),
                             (P.MFMA_I8, "mfma_i8_16x16x64", 20000),
                             (P.MFMA_I8_32, "mfma_i8_32x32x32", 10000)):
        ops = {}

        def run():
            ops["n"] = P.hwprobe_mfma(kind, blocks, iters, res, stream)
        t = timed(run, 3)
        out[key] = ops["n"] / t / 1e12
    out["hbm_ceiling_decode"] = out["copy_inplace_128MiB"]
    out["hbm_ceiling_decode_large"] = max(out["copy_inplace_1GiB"],
                                          out["copy_inplace_1GiB_nt"])
    return out


def _with_ceiling(obj: dict, achieved: float, ceiling: float) -> dict:
    obj["measured_ceiling"] = ceiling
    obj["frac_of_measured"] = achieved / ceiling
    return obj


def _oracle_decode_slice(lo: int, hi: int, seed: int, seconds: float,
                         barrier=None, queue=None):
    """Whole decode steps of slots lo..hi of the 256-slot H=32 batch through
    the float64 oracle, one BLAS thread, until `seconds` of compute have
    passed (input generation is not timed). Returns (tokens, seconds)."""
    from threadpoolctl import threadpool_limits
    import wkv7_inputs as G
    from oracle import wkv7_decode_batch

    with threadpool_limits(1):
        wl = G.cfg_decode(seed=seed)
        S = G.as_f64(wl.init_states[lo:hi])
        ids = wl.batch.slot_ids
        # one untimed step first (the state's pages are touched there)
        b = G.decode_step_inputs(seed, 10**6, ids, wl.H, wl.N)
        _, S = wkv7_decode_batch(S, {k: v[lo:hi]
                                     for k, v in b.inputs64().items()})
        if barrier is not None:
            barrier.wait()
        n_steps, t_used = 0, 0.0
        while t_used < seconds:
            b = G.decode_step_inputs(seed, n_steps, ids, wl.H, wl.N)
            x = {k: v[lo:hi] for k, v in b.inputs64().items()}
            t0 = time.perf_counter()
            _, S = wkv7_decode_batch(S, x)
            t_used += time.perf_counter() - t0
            n_steps += 1
    res = ((hi - lo) * n_steps, t_used)
    if queue is not None:
        queue.put(res)
    return res


HOST_SHARE = 16   # CPU threads one GPU's jobs may use on the GPU host


def _host_cores() -> int:
    """Cores of this process's CPU set, at most HOST_SHARE."""
    return max(1, min(HOST_SHARE, len(os.sched_getaffinity(0))))


def _numpy_oracle_decode(seconds: float, seed: int, cores: int) -> dict:
    """The numpy float64 oracle on whole decode steps of the 256-slot, H=32
    batch: one core, then the slots split over `cores` worker processes
    running at once (the rate is the sum of the workers' rates)."""
    import multiprocessing as mp

    tok1, t1 = _oracle_decode_slice(0, 256, seed, seconds)
    out = {"single_core_value": tok1 / t1, "value": tok1 / t1, "cores": 1,
           "steps_single_core": tok1 // 256, "seconds_single_core": t1}
    if cores > 1:
        ctx = mp.get_context("spawn")
        barrier, queue = ctx.Barrier(cores), ctx.Queue()
        bounds = np.linspace(0, 256, cores + 1).astype(int)
        procs = [ctx.Process(target=_oracle_decode_slice,
                             args=(int(bounds[i]), int(bounds[i + 1]), seed,
                                   seconds, barrier, queue))
                 for i in range(cores)]
        for p in procs:
            p.start()
        res = []
        try:
            for _ in procs:
                res.append(queue.get(timeout=120))
        except Exception:            # a worker failed: keep the one-core rate
            res = []
        for p in procs:
            p.join(timeout=30)
            if p.is_alive():
                p.terminate()
                p.join(timeout=10)
        if len(res) == cores and all(p.exitcode == 0 for p in procs):
            out["value"] = sum(t / s for t, s in res)
            out["cores"] = cores
    return out


def _rate(fn, units: float, budget: float):
    """Run fn() until `budget` seconds have passed (at least once); returns
    (units per second, calls, seconds)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= budget:
            return units * n / dt, n, dt


def cpu_baseline(seconds: float, seed: int = 1) -> dict:
    """The CPU oracles, timed on this host in the same run, on bounded
    samples of every workload.

    Headline: the plain-C float64 oracle (oracle/wkv7_ref.c) on whole decode
    steps of the 256-slot H=32 batch, independent heads on one thread per
    core (value), and on one thread (single_core_value). Per workload: the
    same oracle's tokens per second on a sample of that workload with the
    workload's own shapes and input recipe. Beside it, the numpy float64
    oracle on the decode batch, on one core and on one worker process per
    core. Input generation is not timed."""
    import torch
    import wkv7_inputs as G
    from oracle import wkv7_cref as C
    from oracle import wkv7_sequence

    cores = _host_cores()
    budget = max(0.25, seconds / 20.0)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)

    def draw(T, H):
        return G.draw_tokens_device(gen, T, H, N, "bf16", "cpu")

    per = {}
    # small: one sequence of 64 tokens, H=2, fp32 inputs, zero state
    wl = G.cfg_small(seed=0)
    x0, x0_64 = wl.batch.inputs, wl.batch.inputs64()

    def small_c():
        C.run_heads(np.zeros((2, N, N)), x0, 64, 2, N, threads=1)

    def small_np():
        wkv7_sequence(np.zeros((2, N, N)), **x0_64)

    r_c, n_c, t_c = _rate(small_c, 1, budget)
    r_n, n_n, t_n = _rate(small_np, 1, budget)
    per["small_h2_t64_f32in"] = {"us_per_call_1core": 1e6 / r_c,
                                 "us_per_call_1core_numpy": 1e6 / r_n,
                                 "tokens_per_s_1core": 64 * r_c}
    # decode: 256 slots x H=32, one token each, states N(0, 0.1)
    S1 = np.ascontiguousarray(
        np.random.default_rng(seed).normal(0, 0.1, (256 * 32, N, N)))
    xd = draw(256, 32)
    dec_1, _, _ = _rate(lambda: C.run_heads(S1, xd, 1, 256 * 32, N,
                                            threads=1), 256, budget)
    dec_n, n_dec, t_dec = _rate(lambda: C.run_heads(S1, xd, 1, 256 * 32, N,
                                                    threads=cores),
                                256, budget)
    per["decode_b256_h32_bf16in"] = {"tokens_per_s": dec_n,
                                     "tokens_per_s_1core": dec_1}
    _progress(f"cpu baseline: decode {dec_1:.0f} tokens/s on one thread, "
              f"{dec_n:.0f} on {cores}")
    # prefill: 8 x 4096 tokens, H=32, zero state; a sample of 2 sequences
    xp = [draw(4096, 32) for _ in range(2)]

    def prefill():
        for x in xp:
            C.run_heads(np.zeros((32, N, N)), x, 4096, 32, N, threads=cores)

    r, _, _ = _rate(prefill, 2 * 4096, budget)
    per["prefill_b8_t4096_h32_bf16in"] = {
        "tokens_per_s": r, "sample": "2 of the 8 sequences of 4096 tokens"}
    # mixed stack: one layer (64 decode slots + prefills 512, 1024, 2048,
    # 2048) at H=12; a 12-layer step is 12 such layers
    xm_d = draw(64, 12)
    xm_p = [draw(T, 12) for T in (512, 1024, 2048, 2048)]
    Sm = np.ascontiguousarray(
        np.random.default_rng(seed + 1).normal(0, 0.1, (64 * 12, N, N)))

    def mixed_layer():
        C.run_heads(Sm, xm_d, 1, 64 * 12, N, threads=cores)
        for x in xm_p:
            C.run_heads(np.zeros((12, N, N)), x, x["r"].shape[0], 12, N,
                        threads=cores)

    r, _, _ = _rate(mixed_layer, 5696, budget)
    per["mixed_12layers_h12_bf16in"] = {"layer_tokens_per_s": r,
                                        "tokens_per_s": r / 12,
                                        "sample": "one of the 12 layers"}
    # large pool decode: 1024 slots x H=64
    S4 = np.ascontiguousarray(
        np.random.default_rng(seed + 2).normal(0, 0.1, (1024 * 64, N, N)))
    x4 = draw(1024, 64)
    r, _, _ = _rate(lambda: C.run_heads(S4, x4, 1, 1024 * 64, N,
                                        threads=cores), 1024, budget)
    per["decode_b1024_h64_bf16in"] = {"tokens_per_s": r}
    del S4
    # large pool prefill: 4 of the 32 ragged sequences (lengths from the
    # same draw as the GPU leg), H=64
    lens = np.random.default_rng(4).integers(128, 8193, size=32)[:4]
    x4p = [draw(int(T), 64) for T in lens]

    def ragged():
        for x in x4p:
            C.run_heads(np.zeros((64, N, N)), x, x["r"].shape[0], 64, N,
                        threads=cores)

    r, _, _ = _rate(ragged, float(lens.sum()), budget)
    per["prefill_32ragged_128to8192_h64_bf16in"] = {
        "tokens_per_s": r,
        "sample": f"4 of the 32 sequences ({int(lens.sum())} tokens)"}
    _progress("cpu baseline: per-workload oracle rates done")
    npy = _numpy_oracle_decode(budget * 2, seed, cores)
    _progress(f"cpu baseline: numpy oracle {npy['single_core_value']:.0f} "
              f"tokens/s on one core")
    model = _cpu_model()
    return {
        "value": dec_n, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "single_core_value": dec_1,
        "sample": (f"decode steps of the 256-slot H=32 batch, plain-C "
                   f"float64 oracle, heads split over {cores} threads; "
                   f"{n_dec} steps in {t_dec:.1f} s"),
        "cpu_model": model,
        "host_cpus_in_affinity": len(os.sched_getaffinity(0)),
        "per_workload": per,
        "numpy_oracle": npy,
    }


def _cpu_model() -> str:
    """Model name with family/model/stepping (some hosts report only the
    vendor line), from /proc/cpuinfo."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    info.setdefault(k.strip(), v.strip())
                if not line.strip() and info:
                    break
    except OSError:
        return "unknown CPU"
    name = info.get("model name", "unknown CPU")
    return (f"{name} (family {info.get('cpu family', '?')}, model "
            f"{info.get('model', '?')}, stepping {info.get('stepping', '?')}"
            f", {info.get('cpu MHz', '?')} MHz)")


def _progress(msg: str) -> None:
    """One line per finished leg on stderr (stdout carries only the JSON
    line), so that a long run shows it is alive. Python's cyclic garbage
    collector is off while legs run (a full collection inside a timed loop
    of short calls shows up as host time per call, as timeit avoids too);
    it runs here, between legs."""
    gc.collect()
    print(f"bench.py: {msg}", file=sys.stderr, flush=True)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--legs",
                    default="decode,prefill,decode_cold,decode_large,"
                            "prefill_f32,prefill_ragged,mixed,prefill_long,"
                            "q8_proj,small,short,ceilings",
                    help="comma list of legs to run (default: all of them; a "
                         "subset when profiling one kernel)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                    help="summarise rocprofv3 counter CSVs (no GPU use) for "
                         "--kernel and exit; with --traffic-out, write the "
                         "traffic record the bench reports for --grid")
    ap.add_argument("--kernel", default="seq_kernel")
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--src", default="",
                    help="comma list of the kernel's source files (csrc/)")
    ap.add_argument("--workload", default="")
    ap.add_argument("--traffic-out", default="")
    args = ap.parse_args(argv)
    if args.pmc_summary:
        summ = pmc_summary(args.pmc_summary, args.kernel)
        print(json.dumps(summ, indent=1))
        if args.traffic_out:
            m = summ[f"grid{args.grid}"]
            src = args.src.split(",")
            rec = {"kernel": args.kernel, "kernel_src": src,
                   "kernel_sha": kernel_sha(src), "workload": args.workload,
                   "grid": args.grid, "counters_per_dispatch": m,
                   "read_bytes_per_launch": m["read_bytes"],
                   "write_bytes_per_launch": m["write_bytes"],
                   "hbm_bytes_per_launch": m["read_bytes"] + m["write_bytes"]}
            with open(args.traffic_out, "w") as f:
                json.dump(rec, f, indent=1)
        return 0
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not "
              "supported (slots shard across GPUs with no exchange, but no "
              "multi-GPU run is built)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    gc.collect()
    gc.disable()

    legs = set(args.legs.split(","))
    if legs == {"prefill"}:
        print(json.dumps({"prefill": run_prefill(args.prefill_steps, 20)}),
              flush=True)
        return 0
    if legs == {"q8_proj"}:
        print(json.dumps({"q8_proj": run_q8_proj()}), flush=True)
        return 0
    if legs == {"short"}:
        print(json.dumps({"short": run_short()}), flush=True)
        return 0
    if legs <= {"mixed", "prefill_long"}:
        out = {}
        if "mixed" in legs:
            out["mixed"] = run_mixed()
            out["mixed_segmented"] = run_mixed(segment_len=512)
        if "prefill_long" in legs:
            out["prefill_long"] = run_prefill_long()
        print(json.dumps(out), flush=True)
        return 0
    d = run_decode(args.steps, args.warmup)
    _progress(f"decode: {d['kernel_ms'] * 1e3:.1f} us per launch")
    achieved = d["bytes_per_launch"] / (d["kernel_ms"] * 1e-3) / 1e9
    traffic = load_traffic("decode", d["bytes_per_launch"])
    line = {
        "metric": METRIC,
        "value": d["tokens"] / d["wall_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": d["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode_b256_h32_pool1024_bf16in_f32state",
            "n_slots": d["n_slots"], "active_slots": d["n_active"],
            "H": d["H"], "N": N, "input_dtype": "bf16",
            "state_dtype": "f32", "output_dtype": "f32",
            "launch": "wkv7_forward_plan (metadata validated and uploaded "
                      "once)",
            "forward_api_ms_per_step": d["forward_ms_per_step"],
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": "seq_kernel<bf16> (decode)",
            "kernel_ms": d["kernel_ms"],
            "timing": "HIP events around the K timed launches / K",
            "bytes_per_launch": d["bytes_per_launch"],
        },
    }
    if not args.no_prefill and "prefill" in legs:
        line["prefill"] = run_prefill(args.prefill_steps, 20)
        _progress("prefill done")
    if "decode_large" in legs:
        line["decode_large"] = run_decode_large()
        _progress("decode_large done")
    if "decode_cold" in legs:
        line["decode_cold"] = run_decode_cold()
        _progress("decode_cold done")
    if "small" in legs:
        line["small"] = run_small()
        _progress("small done")
    if "short" in legs:
        line["short"] = run_short()
        _progress("short done")
    if not args.no_prefill and "prefill_f32" in legs:
        line["prefill_f32"] = run_prefill_f32()
        _progress("prefill_f32 done")
    if not args.no_prefill and "prefill_ragged" in legs:
        line["prefill_ragged"] = run_prefill_ragged()
        _progress("prefill_ragged done")
    if "mixed" in legs:
        line["mixed"] = run_mixed()
        line["mixed_segmented"] = run_mixed(segment_len=512)
        _progress("mixed done")
    if not args.no_prefill and "prefill_long" in legs:
        line["prefill_long"] = run_prefill_long()
        _progress("prefill_long done")
    if "q8_proj" in legs:
        line["q8_proj"] = run_q8_proj()
        _progress("q8_proj done")
    if "ceilings" in legs:
        c = run_ceilings()
        _progress("ceilings done")
        line["ceilings"] = c
        _with_ceiling(line["roofline"], achieved, c["hbm_ceiling_decode"])
        if "prefill" in line:
            m = line["prefill"]["mfma"]
            _with_ceiling(m, m["issued_tflops"], c["mfma_bf16_16x16x32"])
        if "decode_large" in line:
            h = line["decode_large"]["hbm"]
            _with_ceiling(h, h["achieved"], c["hbm_ceiling_decode_large"])
        if "q8_proj" in line:
            q = line["q8_proj"]
            # the tiled product runs on v_mfma_i32_32x32x32_i8
            q["measured_int8_tops"] = c["mfma_i8_32x32x32"]
            for k, v in q.items():
                if isinstance(v, dict) and "tops" in v:
                    v["mfma_frac_of_measured"] = v["tops"] / c["mfma_i8_32x32x32"]
        if "decode_large" in line:
            hr = line["decode_large"]["hibernate_resume"]
            hr["pcie_d2h_contiguous_GBps"] = c["pcie_d2h_256MiB"]
            hr["pcie_h2d_contiguous_GBps"] = c["pcie_h2d_256MiB"]
    if not args.no_cpu_baseline:
        _progress("cpu baseline (oracle) running")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        _progress("cpu baseline done")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
