#!/usr/bin/env python3
"""Benchmark of the batched GQA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  The timed workload is the LLaMA-2-70B-shaped 80-layer
decode step with 256 sequences (contexts 512..1536, KV blocks of 16, untied
LM head of 32,000), bf16, replayed as one captured hipGraph per step:
``value`` is decode tokens/s (256 x steps / seconds) with every input
already resident in HBM.

Also reported (each kernel timed live with HIP events on the stream it runs
on, behind a queued busy-wait kernel so host launch gaps do not count):
  * ``roofline``: the step's dominant kernel (the paged decode attention)
    against the HBM peak, with its calibrated counter traffic and its share
    of the measured read ceiling; ``gemm_roofline``: the step's gate-up
    projection at 256 rows against the bf16 MFMA peak;
  * ``step``, ``kernels``, ``clock``: the step's runs, eager time, HBM floor,
    the nano-batch overlap against the unsplit step, per-kernel rates, and
    the shader clock while it replays; ``corun_interference``: the co-run
    profile P(R) of its gate-up projection beside its attention;
  * ``qwen05b_b32_ctx512``, ``qwen05b_b1_ctx512``, ``batch_sweep``,
    ``bucketed_capture``: the Qwen2.5-0.5B-shaped 24-layer step at batch 32
    and 1 (context 512) and under the continuous-batching mix (batch 1..256,
    contexts 128..2048, fragmented tables, a graph per batch size);
  * ``dense_batch``, ``dense_attention_roofline``, ``dense_gemm_roofline``:
    the LLaMA-2-70B-shaped layer at the 2048-token dense batch -- decode
    attention (512 rows x context 1024) against the HBM peak, the four
    projections against the bf16 MFMA peak, the layer step serial and under
    the nano-batch schedules, and the co-run profile;
  * ``hbm_read_ceiling``: the library's streaming read over 4 GiB (the read
    rate a kernel reaches here); ``torch_copy_rate``: a plain device copy;
  * ``cpu_baseline``: the CPU oracle timed on the host (bounded sample).
"""
from __future__ import annotations

import argparse
import faulthandler
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from decode_step_06_amd import ns  # noqa: E402
from decode_step_06_amd import roofline as rf  # noqa: E402
from decode_step_06_amd.configs import WORKLOADS  # noqa: E402
from decode_step_06_amd.inputs import gen_batch, gen_weights  # noqa: E402
from decode_step_06_amd.runner import (DeviceWeights, alloc_sequences, blocks_for, create_engine,  # noqa: E402
                                       fill_past, fill_past_random_on_device)

HEADLINE = "llama70b_80l_b256"
SMALL = "qwen05b_b32_ctx512"


def decode_sched(**kw):
    """Schedule of the decode-only workloads (one row per sequence): RoPE and
    the cache write fused into the attention kernel."""
    return ns.make_sched(fuse_rope_attention=True, **kw)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def busy(stream, ms=30):
    """Queue a bounded busy-wait kernel so the launches after it are all
    enqueued before the GPU reaches them."""
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(ms * 1e-3 * 2.0e9))


def time_launches(fn, n, stream, reps=3):
    """Average device time per launch of fn(i) over n back-to-back launches
    (HIP events on `stream`); median over reps."""
    out = []
    for _ in range(reps):
        busy(stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        e1.synchronize()
        out.append(e0.elapsed_time(e1) / n * 1e-3)
    return statistics.median(out)


def read_ceiling(stream, nbytes=4 << 30, n=10):
    """Achievable HBM read rate: the library's streaming read (ns_read_stream:
    every byte once, 16-byte non-temporal loads) over a 4 GiB buffer, beside
    the 8 TB/s datasheet figure and the attention's bytes per second."""
    src = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(ns.NS_READ_STREAM_WORDS, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()  # the buffers were written on torch's stream

    def launch(i):
        ns.ns_read_stream(src.data_ptr(), nbytes, sink.data_ptr(), ns.NS_READ_STREAM_WORDS, stream)

    for i in range(3):
        launch(i)
    t = time_launches(launch, n, stream)
    del src, sink
    torch.cuda.synchronize()
    gbs = nbytes / t / 1e9
    return {"kernel": "read_stream_kernel (ns_read_stream)", "bytes_per_launch": nbytes, "avg_launch_us": t * 1e6,
            "gbs": gbs, "frac_of_peak": gbs / rf.HBM_PEAK_GBS}


def copy_ceiling(stream, nbytes=1 << 30, n=10):
    """Achievable HBM rate of a plain device copy (torch's copy kernel, 1 GiB
    read + 1 GiB written per launch) beside the 8 TB/s datasheet figure.  Run
    after the library's kernels, so that the 256 MiB calibration copy stays
    the largest copy before them in a profiled run."""
    src = torch.empty(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    def launch(i):
        with torch.cuda.stream(stream):
            dst.copy_(src)

    for i in range(3):
        launch(i)
    t = time_launches(launch, n, stream)
    del src, dst
    torch.cuda.synchronize()
    return {"bytes_per_copy": 2 * nbytes, "gbs": 2 * nbytes / t / 1e9, "frac_of_peak": 2 * nbytes / t / 1e9 / rf.HBM_PEAK_GBS}


# ---------------------------------------------------------------- the timed step
def setup_step(wname):
    w = WORKLOADS[wname]
    shape = w.model
    log(f"[bench] generating {wname} inputs (seeded)")
    weights = gen_weights(shape, seed=w.seeds["weights"])
    b = gen_batch(w)
    maxb = blocks_for(b.seq_lens)
    h = create_engine(shape, DeviceWeights.from_numpy(shape, weights), b.num_blocks, b.n_seqs, maxb, b.n_rows,
                      b.free_order, decode_sched())
    alloc_sequences(h, b.seq_lens)
    fill_past(h, b.past_seq, b.past_pos, b.past_k, b.past_v)
    return w, weights, b, h, maxb


def run_step_bench(h, b, steps, warmup, warm_seconds, stream):
    shape = h.shape
    out = torch.empty((b.n_rows, shape.vocab or shape.hidden), device="cuda")
    nb = ns.Batch(b.row_seq, b.row_pos, b.tokens)
    g = ns.ns_graph_capture(h.eng, b.n_rows, out.data_ptr(), stream)
    try:
        # eager step once (launch count), then sustained warm-up for the clock
        ns.ns_decode_step(h.eng, nb, out.data_ptr(), stream)
        stream.synchronize()
        launches = ns.ns_engine_last_launches(h.eng)
        t_end = time.time() + warm_seconds
        while time.time() < t_end:
            for _ in range(20):
                ns.ns_graph_replay(g, nb, stream)
            stream.synchronize()
        for _ in range(warmup):
            ns.ns_graph_replay(g, nb, stream)
        stream.synchronize()
        runs = []
        for _ in range(2):  # timed twice; disagreement over 15% is flagged
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                ns.ns_graph_replay(g, nb, stream)
            stream.synchronize()
            torch.cuda.synchronize()
            runs.append((time.perf_counter() - t0) / steps)
        # eager steps for the fixed per-step cost (eager - graph)
        for _ in range(3):
            ns.ns_decode_step(h.eng, nb, out.data_ptr(), stream)
        stream.synchronize()
        t0 = time.perf_counter()
        n_eager = max(5, steps // 4)
        for _ in range(n_eager):
            ns.ns_decode_step(h.eng, nb, out.data_ptr(), stream)
        stream.synchronize()
        eager = (time.perf_counter() - t0) / n_eager
    finally:
        ns.ns_graph_destroy(g)
    return runs, eager, launches


# ---------------------------------------------------------------- greedy decoding
def greedy_loop(h, b, stream, steps=100):
    """Greedy decoding at the step's batch (the 0.5B-shaped step at 32 rows):
    the device argmax alone, and a
    loop of steps whose tokens come from the previous step's argmax, either
    on the device (graph replay + ns_sample_greedy, token ids fed back
    through token_ids_dev: no host round trip) or through the host (replay,
    copy the logits back, argmax in numpy, upload the tokens)."""
    V, T = h.shape.vocab, b.n_rows
    out = torch.empty((T, V), device="cuda")
    tok_dev = torch.zeros((T,), dtype=torch.int32, device="cuda")
    res = {"argmax_us": time_launches(lambda i: ns.ns_sample_greedy(out.data_ptr(), T, V, tok_dev.data_ptr(), stream),
                                      50, stream) * 1e6}
    g = ns.ns_graph_capture(h.eng, T, out.data_ptr(), stream)
    try:
        first = ns.Batch(b.row_seq, b.row_pos, b.tokens)
        fed = ns.Batch(b.row_seq, b.row_pos, tokens_dev=tok_dev)
        ns.ns_graph_replay(g, first, stream)
        ns.ns_sample_greedy(out.data_ptr(), T, V, tok_dev.data_ptr(), stream)
        stream.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            ns.ns_graph_replay(g, fed, stream)
            ns.ns_sample_greedy(out.data_ptr(), T, V, tok_dev.data_ptr(), stream)
        stream.synchronize()
        res["device_feedback_ms_per_step"] = (time.perf_counter() - t0) / steps * 1e3
        host = np.empty((T, V), dtype=np.float32)
        tok = b.tokens
        t0 = time.perf_counter()
        n_host = max(10, steps // 4)
        for _ in range(n_host):
            ns.ns_graph_replay(g, ns.Batch(b.row_seq, b.row_pos, tok), stream)
            stream.synchronize()
            host[:] = out.cpu().numpy()
            tok = np.argmax(host, axis=1).astype(np.int32)
        res["host_feedback_ms_per_step"] = (time.perf_counter() - t0) / n_host * 1e3
    finally:
        ns.ns_graph_destroy(g)
    res["device_feedback_tokens_per_s"] = T / (res["device_feedback_ms_per_step"] * 1e-3)
    return res


# ---------------------------------------------------------------- kernels of the step
def step_kernels(h, b, stream, reps=5):
    """Per-kernel device time inside the real step: an eager serial step with
    the engine's profiling on records a HIP event after every launch on the
    step's stream (a busy-wait kernel queued first keeps host launch gaps out
    of the timing).  Returns per class: launches per step, mean us per
    launch, algorithmic bytes (and FLOPs) per launch."""
    s = h.shape
    L, H, F, V, T = s.n_layers, s.hidden, s.ffn, s.vocab, b.n_rows
    DQ = s.n_q_heads * s.head_dim
    out = torch.empty((T, V or H), device="cuda")
    nb = ns.Batch(b.row_seq, b.row_pos, b.tokens)
    ns.ns_engine_profile(h.eng, True)
    per = {}
    try:
        for _ in range(reps):
            busy(stream)
            ns.ns_decode_step(h.eng, nb, out.data_ptr(), stream)
            kinds, us = ns.ns_engine_profile_read(h.eng)
            for k, u in zip(kinds, us):
                per.setdefault(k, []).append(u)
    finally:
        ns.ns_engine_profile(h.eng, False)
    ctx = (b.row_pos + 1).astype(np.int64)
    work = {  # algorithmic bytes (and FLOPs) per launch
        "qkv_proj": (rf.gemm_bytes(T, s.qkv_dim, H, 2, "store"), rf.gemm_flops(T, s.qkv_dim, H)),
        "o_proj": (rf.gemm_bytes(T, H, DQ, 2, "resid"), rf.gemm_flops(T, H, DQ)),
        "gate_up_proj": (rf.gemm_bytes(T, F, H, 2, "silu"), rf.gemm_flops(T, F, H, True)),
        "down_proj": (rf.gemm_bytes(T, H, F, 2, "resid"), rf.gemm_flops(T, H, F)),
        "lm_head": (rf.gemm_bytes(T, V, H, 2, "store"), rf.gemm_flops(T, V, H)),
        "attention": (int(rf.attention_bytes(s, ctx)), int(rf.attention_flops(s, ctx))),
    }
    res = {}
    for k, us in per.items():
        n = len(us) // reps
        mean = float(np.mean(us))
        r = {"launches_per_step": n, "us_per_launch": mean, "us_per_step": mean * n}
        if k in work:
            nbytes, fl = work[k]
            r.update(bytes_per_launch=nbytes, gbs=nbytes / (mean * 1e-6) / 1e9,
                     tflops=fl / (mean * 1e-6) / 1e12)
        res[k] = r
    return res


ORDER_ITEMS = 1024  # work items from which the engine takes attention rows longest context first


def attention_isolated(h, b, maxb, stream, n=400):
    """The step's attention (the layers' caches in turn, the step's rows and
    block tables, the engine's launch shape and row order) launched n times
    back to back on `stream`: HIP events around the loop give its average
    launch duration -- the figure a kernel trace of this run reports for these
    launches."""
    s = h.shape
    nd = b.n_rows
    order = np.arange(nd)
    if nd * s.n_kv_heads >= ORDER_ITEMS:  # as the engine orders them (the op takes rows as given)
        order = np.argsort(-(b.row_pos.astype(np.int64)), kind="stable")
    rowb = torch.from_numpy(b.row_seq[order].astype(np.int32)).cuda()
    pos = torch.from_numpy(b.row_pos[order].astype(np.int32)).cuda()
    bt = torch.from_numpy(ns.ns_kv_block_table(h.kv, b.n_seqs, maxb).copy()).cuda()
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    q_att = torch.randn((nd, s.n_kv_heads, s.head_dim // 8, s.group, 8), generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty((nd, s.n_q_heads * s.head_dim), device="cuda", dtype=torch.bfloat16)
    wsb = ns.ns_op_attention_ws_bytes(h.desc, nd, maxb)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

    # the launches cycle through the layers' caches (as the step does), so
    # they stream from HBM rather than re-reading one layer's K/V from the
    # last-level cache
    layer_bytes = 2 * h.num_blocks * s.n_kv_heads * 16 * s.head_dim * 2
    bases = [h.kv_mem.data_ptr() + l * layer_bytes for l in range(s.n_layers)]

    def launch(i):
        ns.ns_op_attention(h.desc, nd, q_att.data_ptr(), bases[i % len(bases)], h.num_blocks, rowb.data_ptr(),
                           pos.data_ptr(), bt.data_ptr(), maxb, o.data_ptr(), ws.data_ptr(), wsb, 0, stream)

    for i in range(20):
        launch(i)
    stream.synchronize()
    t = time_launches(launch, n, stream, reps=3)
    nbytes = int(rf.attention_bytes(s, (b.row_pos + 1).astype(np.int64)))
    return {"us": t * 1e6, "bytes": nbytes, "gbs": nbytes / t / 1e9, "launches": n * 3 + 20}


def step_slab_rows(rows):
    """Rows of a slab block of a bf16 step's activations for an engine of
    `rows` rows (odd, at least rows), and whether a step of that many rows
    keeps them K-slab-major (more than 16 rows) -- the engine's choices."""
    return rows | 1, rows > 16


def slab_input(A):
    """A [M, K] bf16 input in the layout a step of M rows gives its
    projections: (tensor, rows per slab block), K-slab-major with an odd block
    of rows above 16 rows, else row-major (rows per block 0)."""
    M, K = A.shape
    r, packed = step_slab_rows(M)
    if not packed:
        return A.contiguous(), 0
    pad = torch.cat([A, torch.zeros((r - M, K), dtype=A.dtype, device=A.device)])
    out = torch.empty_like(pad)
    ns.ns_pack_weight(pad.data_ptr(), out.data_ptr(), r, K)
    return out, r


def step_gemm(epi, M, N, K, A_in, B, C, stream):
    """One projection launch in the step's layouts: A_in from slab_input, B
    the engine's K-slab-major weights, C fp32 [M, N] (store / residual) or,
    for SwiGLU, a bf16 buffer of slab_output's size."""
    A, a_rows = A_in
    if a_rows:
        ns.ns_op_gemm_slab(epi, M, N, K, A.data_ptr(), a_rows, B, C.data_ptr(), a_rows, stream)
    else:
        ns.ns_op_gemm_packed(ns.NS_BF16, epi, M, N, K, A.data_ptr(), B, C.data_ptr(), stream)


def slab_output(M, N):
    """A bf16 SwiGLU output buffer large enough for step_gemm's layout."""
    r, packed = step_slab_rows(M)
    return torch.empty(((N + 31) // 32 * 32 * (r if packed else M),), device="cuda", dtype=torch.bfloat16)


def gate_up_isolated(h, b, stream, n=400):
    """The step's gate-up projection (the layers' K-slab-major weights in
    turn, a [rows, H] bf16 input and the SwiGLU output in the layouts the step
    keeps them in: the same kernel and launch shape as in the step) launched
    n times back to back on `stream`."""
    s = h.shape
    T, H, F = b.n_rows, s.hidden, s.ffn
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    A = slab_input(torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16))
    C = slab_output(T, F)
    # the launches cycle through the layers' weights (as the step does), so
    # they stream from HBM rather than from the last-level cache
    wgu = [lw["wgu"].data_ptr() for lw in h.weights.t["layers"]]

    def launch(i):
        step_gemm(ns.NS_EPI_SILU, T, F, H, A, wgu[i % len(wgu)], C, stream)

    for i in range(20):
        launch(i)
    stream.synchronize()
    t = time_launches(launch, n, stream, reps=3)
    nbytes = rf.gemm_bytes(T, F, H, 2, "silu")
    return {"us": t * 1e6, "bytes": nbytes, "gbs": nbytes / t / 1e9, "launches": n * 3 + 20}


def recorded_traffic(name):
    """HBM bytes per launch from the committed counter summary of kernel
    `name`, if the kernel's source is unchanged since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = os.path.join(ROOT, kv.get("source", ""))
    if not os.path.isfile(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("source_sha256"):
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


# ---------------------------------------------------------------- co-run interference P(R)
CORUN_CAPS = tuple(range(16, 257, 16))   # attention workgroup caps: 1/16 .. all of the 256 CUs


def corun_launches(t_gemm_us, t_attn_us, n_gemm):
    """Attention launches that keep the second stream busy about as long as
    n_gemm projection launches keep the first (at least one)."""
    if t_gemm_us <= 0 or t_attn_us <= 0 or n_gemm < 1:
        raise ValueError("solo times and the launch count must be positive")
    return max(1, int(round(n_gemm * t_gemm_us / t_attn_us)))


def corun_profile(gemm, attn, gemm_flops, attn_bytes, caps=CORUN_CAPS, n_gemm=4):
    """NanoFlow's interference profile P(R) on one GPU ("The part that is
    harder than it looks": the share R of the GPU given to the memory-bound
    op, and each op's throughput when the two co-run).  `gemm(stream)` and
    `attn(stream, cap)` enqueue one launch of the projection and of the paged
    attention (capped at `cap` workgroups, a persistent grid: the share R =
    cap / 256 CUs).  For each cap: the attention alone, then both together on
    two streams released by one event (the attention launched as often as
    keeps its stream busy as long as the projection's), each stream timed
    from the release to its last launch with HIP events.  P_gemm and P_attn
    are the co-run throughputs over the solo ones (uncapped); their sum over
    1 is what overlapping gains over running the two one after the other."""
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()

    def solo(fn, stream, n):
        for _ in range(2):
            fn(stream)
        stream.synchronize()
        return time_launches(lambda i: fn(stream), n, stream) * 1e6

    t_g = solo(gemm, sa, n_gemm)
    t_a0 = solo(lambda st: attn(st, 0), sb, 8)
    rows = []
    for cap in caps:
        t_a = solo(lambda st: attn(st, cap), sb, 8)
        n_a = corun_launches(t_g, t_a, n_gemm)
        busy(sa)
        e0 = torch.cuda.Event(enable_timing=True)
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(sa)
        sb.wait_event(e0)
        for _ in range(n_gemm):
            gemm(sa)
        ea.record(sa)
        for _ in range(n_a):
            attn(sb, cap)
        eb.record(sb)
        sa.synchronize()
        sb.synchronize()
        tg_co = e0.elapsed_time(ea) * 1e3 / n_gemm
        ta_co = e0.elapsed_time(eb) * 1e3 / n_a
        p_g, p_a = t_g / tg_co, t_a0 / ta_co
        rows.append({"cap": cap, "share": cap / 256.0, "attn_solo_us": t_a, "attn_corun_us": ta_co,
                     "gemm_corun_us": tg_co, "p_gemm": p_g, "p_attn": p_a, "p_sum": p_g + p_a})
    best = max(rows, key=lambda r: r["p_sum"])
    return {"gemm_solo_us": t_g, "gemm_tflops_solo": gemm_flops / t_g / 1e6, "attn_solo_us": t_a0,
            "attn_gbs_solo": attn_bytes / t_a0 / 1e3, "curve": rows, "best_cap": best["cap"],
            "best_p_sum": best["p_sum"]}


# ---------------------------------------------------------------- the dense-batch layer
def dense_batch(stream, steps=10):
    """LLaMA-2-70B-shaped layer at the 2048-token dense batch (device-drawn
    weights and cache): attention and projection roofline fractions, and the
    layer step serial vs nano-batch overlapped (graph replays)."""
    w = WORKLOADS["llama70b_layer_t2048"]
    s = w.model
    log("[bench] dense batch: llama70b layer, 2048 rows")
    b = gen_batch(w, with_past=False)
    maxb = blocks_for(b.seq_lens)
    dw = DeviceWeights.random_on_device(s, seed=0)
    h = create_engine(s, dw, b.num_blocks, b.n_seqs, maxb, b.n_rows, b.free_order, None, nan_poison=False)
    res = {}
    try:
        alloc_sequences(h, b.seq_lens)
        fill_past_random_on_device(h, b.past_seq, b.past_pos, seed=4)
        H, F, DQ, T = s.hidden, s.ffn, s.n_q_heads * s.head_dim, b.n_rows
        lw = dw.t["layers"][0]
        A = torch.randn((T, max(H, F, DQ)), device="cuda").to(torch.bfloat16)
        C32 = torch.empty((T, max(s.qkv_dim, H)), device="cuda")
        Cb = torch.empty((T, F), device="cuda", dtype=torch.bfloat16)
        # the whole layer step first: serial vs nano-batched with overlap (the
        # isolated kernels below are then the last launches of their kernels,
        # for the counter summaries)
        x = torch.randn((T, H), device="cuda")
        out = torch.empty((T, H), device="cuda")
        nb = ns.Batch(b.row_seq, b.row_pos, None, x)
        def nano(overlap=True, **kw):
            return ns.make_sched(nano_rows=w.nano_splits, qkv_rows=(512,) * w.qkv_splits, overlap=overlap,
                                 prefill_tiles=True, **kw)

        # the interference profile P(R): the gate-up projection at 2048 rows
        # against the decode attention of the 512 decode rows (context 1024)
        # capped at R workgroups, on two streams
        nd = w.n_decode
        rowb = torch.arange(nd, dtype=torch.int32, device="cuda")
        pos = torch.from_numpy(b.row_pos[:nd].astype(np.int32)).cuda()
        bt = torch.from_numpy(ns.ns_kv_block_table(h.kv, b.n_seqs, maxb)[:nd].copy()).cuda()
        q_att = torch.randn((nd, s.n_kv_heads, s.head_dim // 8, s.group, 8), device="cuda").to(torch.bfloat16)
        o = torch.empty((nd, DQ), device="cuda", dtype=torch.bfloat16)
        wsb = ns.ns_op_attention_ws_bytes(h.desc, nd, maxb)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        ab = rf.attention_bytes(s, [w.decode_ctx] * nd)
        Cb2 = torch.empty_like(Cb)

        def attn_op(st, cap):
            ns.ns_op_attention(h.desc, nd, q_att.data_ptr(), h.kv_mem.data_ptr(), h.num_blocks, rowb.data_ptr(),
                               pos.data_ptr(), bt.data_ptr(), maxb, o.data_ptr(), ws.data_ptr(), wsb, cap, st)

        def gu_op(st):
            ns.ns_op_gemm_packed(ns.NS_BF16, ns.NS_EPI_SILU, T, F, H, A.data_ptr(), lw["wgu"].data_ptr(),
                                 Cb2.data_ptr(), st)

        res["corun"] = corun_profile(gu_op, attn_op, rf.gemm_flops(T, F, H, True), ab)
        # nano-batched variants: the split alone on one stream (the cost of
        # smaller projection launches); overlapped in row order; decode rows'
        # attention queued last with the prompt nano-batch's projections
        # first; that with the attention capped at a number of workgroups
        for label, sched in (("serial", ns.make_sched(prefill_tiles=True)),
                             ("serial_decode_kernel_only", ns.make_sched()),
                             ("nano_split_no_overlap", nano(overlap=False)),
                             ("nano_overlap", nano()),
                             ("nano_overlap_decode_first", nano(decode_rows_first=True)),
                             ("nano_overlap_decode_first_cap256", nano(decode_rows_first=True, attn_wg_cap=256)),
                             ("nano_overlap_decode_first_cap128", nano(decode_rows_first=True, attn_wg_cap=128)),
                             # other split sizes: two halves; the decode rows alone against the
                             # prompt chunks (512/1536); the pages' 768/1280 at QKV as well
                             ("nano_overlap_1024_1024", ns.make_sched(nano_rows=(1024, 1024), overlap=True,
                                                                      prefill_tiles=True)),
                             ("nano_overlap_512_1536_decode_first",
                              ns.make_sched(nano_rows=(512, 1536), overlap=True, prefill_tiles=True,
                                            decode_rows_first=True)),
                             ("nano_overlap_768_1280_qkv_same",
                              ns.make_sched(nano_rows=w.nano_splits, overlap=True, prefill_tiles=True)),
                             # the split with the attention capped at the P(R) profile's best share
                             ("nano_overlap_1024_1024_cap_best",
                              ns.make_sched(nano_rows=(1024, 1024), overlap=True, prefill_tiles=True,
                                            attn_wg_cap=res["corun"]["best_cap"]))):
            ns.ns_engine_set_sched(h.eng, sched)
            g = ns.ns_graph_capture(h.eng, T, out.data_ptr(), stream)
            try:
                for _ in range(3):
                    ns.ns_graph_replay(g, nb, stream)
                stream.synchronize()
                t = time_launches(lambda i: ns.ns_graph_replay(g, nb, stream), steps, stream)
            finally:
                ns.ns_graph_destroy(g)
            res[f"layer_step_ms_{label}"] = t * 1e3
        best = min((k for k in res if k.startswith("layer_step_ms_nano_overlap")), key=lambda k: res[k])
        res["layer_best_nano_schedule"] = best[len("layer_step_ms_"):]
        # the schedule search's choice over every variant timed (serial included)
        chosen = min((k for k in res if k.startswith("layer_step_ms_")), key=lambda k: res[k])
        res["chosen_schedule"] = chosen[len("layer_step_ms_"):]
        res["layer_tokens_per_s_nano"] = T / (res[best] * 1e-3)
        res["layer_tokens_per_s_serial"] = T / (res["layer_step_ms_serial"] * 1e-3)
        # sustained GEMM work before the isolated timings: the clock ramps up
        # under load
        t_end = time.time() + 1.5
        while time.time() < t_end:
            ns.ns_op_gemm_packed(ns.NS_BF16, ns.NS_EPI_SILU, T, F, H, A.data_ptr(), lw["wgu"].data_ptr(),
                                 Cb.data_ptr(), stream=stream)
            stream.synchronize()
        # the shader clock under this GEMM's sustained load (the MFMA peak
        # scales with it)
        res["clock_during_gate_up_gemm"] = sample_clock(
            lambda: [ns.ns_op_gemm_packed(ns.NS_BF16, ns.NS_EPI_SILU, T, F, H, A.data_ptr(), lw["wgu"].data_ptr(),
                                          Cb.data_ptr(), stream=stream) for _ in range(800)], stream)
        gem = {}
        for name, epi, N, K, Bw, C in (("qkv_proj", ns.NS_EPI_STORE, s.qkv_dim, H, lw["wqkv"], C32),
                                       ("o_proj", ns.NS_EPI_RESID, H, DQ, lw["wo"], C32),
                                       ("gate_up_proj", ns.NS_EPI_SILU, F, H, lw["wgu"], Cb),
                                       ("down_proj", ns.NS_EPI_RESID, H, F, lw["wdown"], C32)):
            # the engine's weights (K-slab-major) and the step's layouts of
            # the input and the SwiGLU output, as the step runs them
            Ak = slab_input(A[:, :K])
            Ck = slab_output(T, N) if epi == ns.NS_EPI_SILU else C
            t = time_launches(lambda i: step_gemm(epi, T, N, K, Ak, Bw.data_ptr(), Ck, stream), 5, stream)
            fl = rf.gemm_flops(T, N, K, epi == ns.NS_EPI_SILU)
            gem[name] = dict(us=t * 1e6, tflops=fl / t / 1e12, frac=fl / t / 1e12 / rf.BF16_PEAK_TFLOPS)
        tot_fl = sum(rf.gemm_flops(T, N, K, sw) for N, K, sw in ((s.qkv_dim, H, False), (H, DQ, False),
                                                                 (F, H, True), (H, F, False)))
        tot_t = sum(v["us"] for v in gem.values()) * 1e-6
        res["gemm"] = gem
        res["gemm_tflops"] = tot_fl / tot_t / 1e12
        res["gemm_mfma_frac"] = res["gemm_tflops"] / rf.BF16_PEAK_TFLOPS
        # decode attention: the 512 decode rows at context 1024
        t = time_launches(lambda i: ns.ns_op_attention(h.desc, nd, q_att.data_ptr(), h.kv_mem.data_ptr(),
                                                       h.num_blocks, rowb.data_ptr(), pos.data_ptr(), bt.data_ptr(),
                                                       maxb, o.data_ptr(), ws.data_ptr(), wsb, 0, stream), 5, stream)
        ab = rf.attention_bytes(s, [w.decode_ctx] * nd)
        res["attention"] = dict(us=t * 1e6, gbs=ab / t / 1e9, hbm_frac=ab / t / 1e9 / rf.HBM_PEAK_GBS, bytes=ab)
    finally:
        h.destroy()
        torch.cuda.synchronize()
    return res


# ---------------------------------------------------------------- batch sweep
SWEEP = (1, 8, 32, 64, 128, 256)


def _graph_rate(h, b, stream, steps, warm_seconds, sched=None):
    """Device time per replay of the step's graph (median of 3 timings of
    `steps` back-to-back replays)."""
    if sched is not None:
        ns.ns_engine_set_sched(h.eng, sched)
    out = torch.empty((b.n_rows, h.shape.vocab or h.shape.hidden), device="cuda")
    nb = ns.Batch(b.row_seq, b.row_pos, b.tokens)
    g = ns.ns_graph_capture(h.eng, b.n_rows, out.data_ptr(), stream)
    try:
        t_end = time.time() + warm_seconds
        while time.time() < t_end:
            ns.ns_graph_replay(g, nb, stream)
            stream.synchronize()
        return time_launches(lambda i: ns.ns_graph_replay(g, nb, stream), steps, stream)
    finally:
        ns.ns_graph_destroy(g)


def _step_row(h, b, t, stream):
    s = h.shape
    ctx = (b.row_pos + 1).astype(np.int64)
    sb = rf.step_bytes(s, ctx)
    kern = step_kernels(h, b, stream, reps=3)
    att = kern.get("attention", {})
    tot = sum(v["us_per_step"] for v in kern.values())
    return {"tokens_per_s": b.n_rows / t, "ms_per_step": t * 1e3, "mean_ctx": float(ctx.mean()),
            "algorithmic_bytes": sb, "hbm_floor_ms": rf.floor_seconds(sb) * 1e3,
            "step_hbm_frac": sb / t / 1e9 / rf.HBM_PEAK_GBS,
            "attention_gbs": att.get("gbs"), "attention_hbm_frac": (att.get("gbs") or 0) / rf.HBM_PEAK_GBS,
            "attention_share_of_step": att.get("us_per_step", 0) / tot if tot else None,
            "kernels_per_step": sum(v["launches_per_step"] for v in kern.values())}


def batch_sweep(stream, dw, steps=100, warm_seconds=1.0):
    """Qwen2.5-0.5B-shaped 24-layer step under the continuous-batching mix:
    batch 1..256, contexts uniform in 128..2048, fragmented block tables, one
    graph captured per batch size."""
    res = {}
    for B in SWEEP:
        w = WORKLOADS[f"qwen05b_mix_b{B}"]
        b = gen_batch(w, with_past=False)
        maxb = blocks_for(b.seq_lens)
        log(f"[bench] batch sweep B={B}")
        h = create_engine(w.model, dw, b.num_blocks, b.n_seqs, maxb, b.n_rows, b.free_order, decode_sched(),
                          nan_poison=False)
        try:
            alloc_sequences(h, b.seq_lens)
            fill_past_random_on_device(h, b.past_seq, b.past_pos, seed=w.seeds["kv"])
            t = _graph_rate(h, b, stream, steps, warm_seconds)
            res[str(B)] = _step_row(h, b, t, stream)
        finally:
            h.destroy()
            torch.cuda.synchronize()
    return res


BUCKETS = (1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 192, 256)


def bucket_capture(stream, dw, steps=50):
    """Bucketed capture for the continuous-batching mix (Qwen2.5-0.5B-shaped,
    24 layers, up to 256 rows): capture time and device memory of one graph
    per bucket, and what padding costs -- a batch replayed on the next
    bucket up against a graph captured for its exact size."""
    w = WORKLOADS["qwen05b_mix_b256"]
    b = gen_batch(w, with_past=False)
    maxb = blocks_for(b.seq_lens)
    log("[bench] bucketed capture")
    h = create_engine(w.model, dw, b.num_blocks, b.n_seqs, maxb, b.n_rows, b.free_order, decode_sched(),
                      nan_poison=False)
    res = {"buckets": list(BUCKETS)}
    try:
        alloc_sequences(h, b.seq_lens)
        fill_past_random_on_device(h, b.past_seq, b.past_pos, seed=w.seeds["kv"])
        out = torch.empty((b.n_rows, w.model.vocab), device="cuda")
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        t0 = time.perf_counter()
        gs = ns.ns_graph_set_capture(h.eng, BUCKETS, out.data_ptr(), stream)
        torch.cuda.synchronize()
        res["capture_ms_total"] = (time.perf_counter() - t0) * 1e3
        res["capture_ms_per_graph"] = res["capture_ms_total"] / len(BUCKETS)
        try:
            # graph memory is committed at the first launch: replay each once
            for bk in BUCKETS:
                nb = ns.Batch(b.row_seq[:bk], b.row_pos[:bk], b.tokens[:bk])
                ns.ns_graph_set_replay(gs, nb, stream)
            torch.cuda.synchronize()
            res["device_mem_mb"] = (free0 - torch.cuda.mem_get_info()[0]) / 2 ** 20
            pad = {}
            for n in (33, 100, 200):
                nb = ns.Batch(b.row_seq[:n], b.row_pos[:n], b.tokens[:n])
                used = ns.ns_graph_set_replay(gs, nb, stream)
                t_pad = time_launches(lambda i: ns.ns_graph_set_replay(gs, nb, stream), steps, stream)
                g = ns.ns_graph_capture(h.eng, n, out.data_ptr(), stream)
                try:
                    t_exact = time_launches(lambda i: ns.ns_graph_replay(g, nb, stream), steps, stream)
                finally:
                    ns.ns_graph_destroy(g)
                pad[str(n)] = {"bucket": used, "padded_ms": t_pad * 1e3, "exact_ms": t_exact * 1e3,
                               "padding_overhead": t_pad / t_exact - 1.0}
            res["padding"] = pad
        finally:
            ns.ns_graph_set_destroy(gs)
    finally:
        h.destroy()
        torch.cuda.synchronize()
    return res


# ---------------------------------------------------------------- GPU clock
def gfx_clock_reader():
    """A function returning the shader clock (MHz) of the GPU torch uses, read
    from the amd-smi metrics on the host, or None when it cannot be read."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        hdl = handles[0]
        if len(handles) > 1:
            bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            for x in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(x)
                if bus is not None and int(bdf.split(":")[1], 16) == bus:
                    hdl = x
    except Exception:
        return None

    def read():
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(hdl)
        except Exception:
            return None
        cur = m.get("current_gfxclks")
        if isinstance(cur, (list, tuple)):
            vals = [v for v in cur if isinstance(v, (int, float)) and 0 < v < 10000]
            if vals:
                return float(np.mean(vals))
        for k in ("average_gfxclk_frequency", "current_gfxclk"):
            v = m.get(k)
            if isinstance(v, (int, float)) and 0 < v < 10000:
                return float(v)
        return None
    return read


def sample_clock(enqueue, stream, seconds=0.8):
    """Shader clock while the GPU runs the work `enqueue()` queues (a second
    or more of graph replays): sampled on the host every 50 ms."""
    read = gfx_clock_reader()
    if read is None:
        return None
    enqueue()
    time.sleep(0.2)
    vals = []
    t_end = time.time() + seconds
    while time.time() < t_end:
        v = read()
        if v is not None:
            vals.append(v)
        time.sleep(0.05)
    stream.synchronize()
    if not vals:
        return None
    return {"mhz_median": float(np.median(vals)), "mhz_min": float(min(vals)), "mhz_max": float(max(vals)),
            "samples": len(vals), "source": "amd-smi gpu metrics (shader clock), while the timed launches run"}


# ---------------------------------------------------------------- the headline: 80-layer 70B step
def llama80(args, stream):
    """LLaMA-2-70B-shaped 80-layer decode step, 256 sequences at contexts
    uniform in 512..1536, weights (138 GB) and cache (88 GB) drawn on the
    device: the whole step replayed as one hipGraph (the unsplit schedule),
    with and without the two-way nano-batch overlap; the paged attention and
    the gate-up projection launched alone over the layers' caches and
    weights for their rooflines."""
    w = WORKLOADS[HEADLINE]
    s = w.model
    torch.cuda.empty_cache()
    b = gen_batch(w, with_past=False, pool_slack=1.02)
    maxb = blocks_for(b.seq_lens)
    log("[bench] llama70b 80 layers: drawing weights and cache on the device")
    t0 = time.time()
    dw = DeviceWeights.random_on_device(s, seed=w.seeds["weights"])
    h = create_engine(s, dw, b.num_blocks, b.n_seqs, maxb, b.n_rows, b.free_order, decode_sched(), nan_poison=False)
    res = {"weights_gb": dw.bytes() / 1e9, "kv_pool_gb": h.kv_mem.numel() / 1e9}
    try:
        alloc_sequences(h, b.seq_lens)
        fill_past_random_on_device(h, b.past_seq, b.past_pos, seed=w.seeds["kv"])
        torch.cuda.synchronize()
        res["setup_s"] = time.time() - t0
        log("[bench] llama70b 80 layers: timing graph replays")
        res["runs"], res["eager"], res["launches"] = run_step_bench(h, b, args.steps, args.warmup, args.warm_seconds,
                                                                    stream)
        out = torch.empty((b.n_rows, s.vocab), device="cuda")
        nb = ns.Batch(b.row_seq, b.row_pos, b.tokens)
        g = ns.ns_graph_capture(h.eng, b.n_rows, out.data_ptr(), stream)
        try:
            res["clock"] = sample_clock(lambda: [ns.ns_graph_replay(g, nb, stream) for _ in range(25)], stream)
        finally:
            ns.ns_graph_destroy(g)
        res["kernels"] = step_kernels(h, b, stream, reps=2)
        res["nano_ms"] = _graph_rate(h, b, stream, max(5, args.steps // 2), 1.0,
                                     decode_sched(nano_rows=w.nano_splits, overlap=True)) * 1e3
        ns.ns_engine_set_sched(h.eng, decode_sched())
        res["corun"] = llama80_corun(h, b, maxb)
        # last, so that a kernel trace of this run ends with these launches
        res["att"] = attention_isolated(h, b, maxb, stream, n=100)
        res["gu"] = gate_up_isolated(h, b, stream, n=100)
    finally:
        h.destroy()
        del dw
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return w, b, res


def llama80_corun(h, b, maxb):
    """P(R) at the 80-layer step's shapes: the gate-up projection at 256 rows
    (layer 0's weights, 940 MB, streamed from HBM every launch) against the
    step's paged attention over layer 0's cache (1.1 GB)."""
    s = h.shape
    T, H, F = b.n_rows, s.hidden, s.ffn
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    A = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    C = torch.empty((T, F), device="cuda", dtype=torch.bfloat16)
    wgu = h.weights.t["layers"][0]["wgu"]
    rowb = torch.from_numpy(b.row_seq.astype(np.int32)).cuda()
    pos = torch.from_numpy(b.row_pos.astype(np.int32)).cuda()
    bt = torch.from_numpy(ns.ns_kv_block_table(h.kv, b.n_seqs, maxb).copy()).cuda()
    q_att = torch.randn((T, s.n_kv_heads, s.head_dim // 8, s.group, 8), generator=g,
                        device="cuda").to(torch.bfloat16)
    o = torch.empty((T, s.n_q_heads * s.head_dim), device="cuda", dtype=torch.bfloat16)
    wsb = ns.ns_op_attention_ws_bytes(h.desc, T, maxb)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def attn_op(st, cap):
        ns.ns_op_attention(h.desc, T, q_att.data_ptr(), h.kv_mem.data_ptr(), h.num_blocks, rowb.data_ptr(),
                           pos.data_ptr(), bt.data_ptr(), maxb, o.data_ptr(), ws.data_ptr(), wsb, cap, st)

    def gu_op(st):
        ns.ns_op_gemm_packed(ns.NS_BF16, ns.NS_EPI_SILU, T, F, H, A.data_ptr(), wgu.data_ptr(), C.data_ptr(), st)

    return corun_profile(gu_op, attn_op, rf.gemm_flops(T, F, H, True),
                         rf.attention_bytes(s, (b.row_pos + 1).tolist()))


# ---------------------------------------------------------------- the small model's decode steps
def small_step(stream, wname, steps, warm_seconds, detail):
    """The Qwen2.5-0.5B-shaped 24-layer step at one batch (graph replay);
    with `detail`, also per-kernel times, the two-way nano split, the
    separate RoPE kernel, greedy decoding and the rooflines of the gate-up
    GEMV and the attention (isolated launches)."""
    w, weights, b, h, maxb = setup_step(wname)
    res = {}
    try:
        runs, eager, launches = run_step_bench(h, b, steps, 5, warm_seconds, stream)
        step_s = runs[-1]
        sb = rf.step_bytes(w.model, (b.row_pos + 1).tolist())
        res = {"tokens_per_s": b.n_rows / step_s, "ms_per_step": step_s * 1e3,
               "runs_ms": [r * 1e3 for r in runs], "runs_disagree_over_15pct": bool(max(runs) > 1.15 * min(runs)),
               "eager_ms": eager * 1e3, "fixed_cost_ms": (eager - step_s) * 1e3, "kernels_per_step": launches,
               "algorithmic_bytes": sb, "hbm_floor_ms": rf.floor_seconds(sb) * 1e3,
               "step_hbm_frac": sb / step_s / 1e9 / rf.HBM_PEAK_GBS}
        if detail:
            kern = step_kernels(h, b, stream)
            res["kernels"] = kern
            if w.nano_splits:
                res["nano_overlap_ms"] = _graph_rate(h, b, stream, steps, 1.0,
                                                     decode_sched(nano_rows=w.nano_splits, overlap=True)) * 1e3
                res["nano_split"] = list(w.nano_splits)
            res["separate_rope_kernel_ms"] = _graph_rate(h, b, stream, steps, 1.0, ns.make_sched()) * 1e3
            ns.ns_engine_set_sched(h.eng, decode_sched())
            res["greedy_decoding"] = greedy_loop(h, b, stream)
            att = attention_isolated(h, b, maxb, stream)
            gu = gate_up_isolated(h, b, stream)
            tot = sum(v["us_per_step"] for v in kern.values())
            res["gate_up_roofline"] = {
                "kernel": "gate-up projection + SwiGLU (gemv_bf16_kernel)", "bound": "hbm",
                "achieved": gu["gbs"], "peak": rf.HBM_PEAK_GBS, "unit": "GB/s", "frac": gu["gbs"] / rf.HBM_PEAK_GBS,
                "traffic": recorded_traffic("gemm_gate_up_qwen05b_b32"), "bytes_per_launch": gu["bytes"],
                "avg_launch_us": gu["us"], "isolated_launches": gu["launches"],
                "share_of_step": kern["gate_up_proj"]["us_per_step"] / tot}
            res["attention_roofline"] = {
                "kernel": "paged decode attention (attn_mfma_kernel)", "bound": "hbm", "achieved": att["gbs"],
                "peak": rf.HBM_PEAK_GBS, "unit": "GB/s", "frac": att["gbs"] / rf.HBM_PEAK_GBS,
                "traffic": recorded_traffic("attention_qwen05b_b32_ctx512"), "bytes_per_launch": att["bytes"],
                "avg_launch_us": att["us"], "isolated_launches": att["launches"],
                "share_of_step": kern["attention"]["us_per_step"] / tot}
    finally:
        h.destroy()
        torch.cuda.synchronize()
    return res, h.weights


# ---------------------------------------------------------------- CPU oracle
def oracle_step_seconds(shape, b, maxb, gen, min_seconds=0.0):
    """Wall time of the oracle in its float32 mode for one decode step of a
    workload: one layer over all of the batch's rows (its attention over each
    row's cached context through the block tables), times the layer count,
    plus the final norm and LM head.  The layer runs at least 3 times and
    until `min_seconds` of it have passed (at most 50), and its median counts
    (each run writes the same cache slots, so the work is the same).  The
    oracle gets inputs of its own, of the workload's shapes and
    distributions, drawn with torch's generator `gen` on the device and copied
    to the host (nothing read back from the library).  Returns (seconds,
    seconds of the one layer, seconds of the head, layer runs, seconds of all
    layer runs)."""
    from dataclasses import replace

    from decode_step_06_amd.inputs import GAIN_STD, WEIGHT_STD, weight_names
    from oracle import decoder as od
    from oracle import kvcache as okv

    def draw(shp, std=1.0, mean=0.0):
        t = torch.randn(shp, generator=gen, device="cuda") * std + mean
        return t.to(torch.bfloat16).float().cpu().numpy()

    lw = {n: draw(sh, GAIN_STD, 1.0) if n.endswith("norm") else draw(sh, WEIGHT_STD) for n, sh in weight_names(shape)}
    alloc = okv.BlockAllocator(b.num_blocks, b.free_order, b.n_seqs, maxb)
    for q, n in enumerate(b.seq_lens):
        alloc.alloc(q, int(n))
    tables = alloc.table_rows()
    cache = od.OracleKV(1, b.num_blocks, shape.n_kv_heads, shape.head_dim, dtype=np.float32)
    P = len(b.past_seq)
    od.fill_past(cache, tables, b.past_seq, b.past_pos, [draw((P, shape.n_kv_heads, shape.head_dim))],
                 [draw((P, shape.n_kv_heads, shape.head_dim))])
    x = draw((b.n_rows, shape.hidden))
    one = od.Oracle(replace(shape, n_layers=1, vocab=0, tied=False), {"layers": [lw]}, precision="f32")
    runs = []
    while len(runs) < 3 or (sum(runs) < min_seconds and len(runs) < 50):
        t0 = time.perf_counter()
        y = one.step(cache, tables, b.row_seq, b.row_pos, x=x)
        runs.append(time.perf_counter() - t0)
    t_layer = statistics.median(runs)
    t_head = 0.0
    if shape.vocab:
        head = od.Oracle(shape, {"final_norm": draw((shape.hidden,), GAIN_STD, 1.0),
                                 "lm_head": draw((shape.vocab, shape.hidden), WEIGHT_STD)}, precision="f32")
        t0 = time.perf_counter()
        head.head(y)
        t_head = time.perf_counter() - t0
    return t_layer * shape.n_layers + t_head, t_layer, t_head, len(runs), sum(runs)


def cpu_baseline(full=False):
    """The oracle (float32 mode) timed on this host's cores: the headline's
    80-layer step from one of its layers (256 rows) and its LM head, and the
    0.5B-shaped step at batch 32; with `full`, also the continuous-batching
    mix at each batch size and the 2048-row 70B-shaped layer."""
    log("[bench] cpu_baseline: timing the oracle (float32)")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    cores = len(os.sched_getaffinity(0))
    w = WORKLOADS[HEADLINE]
    b = gen_batch(w, with_past=False, pool_slack=1.02)
    t, tl, th, nr, tr = oracle_step_seconds(w.model, b, blocks_for(b.seq_lens), gen, min_seconds=8.0)
    out = {"value": b.n_rows / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"one of the 80 layers of {HEADLINE} over all {b.n_rows} rows, run {nr} times ({tr:.1f} s; "
                     f"median {tl:.2f} s), plus the final norm and LM head ({th:.1f} s), float32 numpy; the step "
                     f"time is 80 x the layer's median + the head",
           "threads_env": os.environ.get("OMP_NUM_THREADS")}
    other = [SMALL] + ([f"qwen05b_mix_b{B}" for B in SWEEP] + ["llama70b_layer_t2048"] if full else [])
    extra = {}
    for name in other:
        wo = WORKLOADS[name]
        bo = gen_batch(wo, with_past=False)
        t, tl, th, nr, _ = oracle_step_seconds(wo.model, bo, blocks_for(bo.seq_lens), gen, min_seconds=1.0)
        extra[name] = {"tokens_per_s": bo.n_rows / t, "step_s": t, "layer_s": tl, "head_s": th, "layer_runs": nr}
    out["other_workloads"] = extra
    return out


def _jsonable(o):
    if isinstance(o, (np.integer,)):
        return int(o)
    if isinstance(o, (np.floating,)):
        return float(o)
    if isinstance(o, float):
        return o
    raise TypeError(type(o))


def _rounded(o, nd=4):
    if isinstance(o, dict):
        return {k: _rounded(v, nd) for k, v in o.items()}
    if isinstance(o, (list, tuple)):
        return [_rounded(v, nd) for v in o]
    if isinstance(o, (float, np.floating)):
        return float(f"{float(o):.{nd + 2}g}")
    if isinstance(o, np.integer):
        return int(o)
    return o


def _leg(fn, *a, **kw):
    try:
        return json.loads(json.dumps(fn(*a, **kw), default=_jsonable))
    except Exception as e:  # report, do not hide
        log(f"[bench] {fn.__name__} failed: {e!r}")
        return {"error": repr(e)}


def dense_rooflines(d):
    """The 2048-row layer's attention (HBM) and projections (MFMA) as roofline
    entries of their own, from the dense leg's isolated launches."""
    if not isinstance(d, dict) or "attention" not in d or "gemm" not in d:
        return {}
    a, g = d["attention"], d["gemm"]
    return {"dense_attention_roofline": {
                "workload": "llama70b_layer_t2048: 512 decode rows at context 1024", "bound": "hbm",
                "achieved": a["gbs"], "peak": rf.HBM_PEAK_GBS, "unit": "GB/s", "frac": a["hbm_frac"],
                "traffic": recorded_traffic("attention_llama70b_b512_ctx1024"), "bytes_per_launch": a["bytes"],
                "avg_launch_us": a["us"]},
            "dense_gemm_roofline": {
                "workload": "llama70b_layer_t2048: QKV, O, gate-up and down projections at 2048 rows", "bound": "mfma",
                "achieved": d["gemm_tflops"], "peak": rf.BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": d["gemm_mfma_frac"], "gate_up_traffic": recorded_traffic("gemm_gate_up_llama70b_t2048"),
                "per_projection_us": {k: v["us"] for k, v in g.items()},
                "clock_during_gate_up_gemm": d.get("clock_during_gate_up_gemm")}}


def dense_leg_isolated():
    """The dense-batch leg in a child process of its own.  Once, in a run of
    several legs, the leg ended the process with a host segmentation fault
    (no GPU fault reported, cause not found); run apart, such a crash costs
    this leg's entries instead of the whole line.  The child's log and any
    fault trace go to this process's stderr; its JSON comes back on stdout."""
    # the leg takes about a minute; a child that hangs must not hold the line
    return run_child_leg([sys.executable, os.path.abspath(__file__), "--child-leg", "dense"], "dense-batch",
                         timeout=600)


def run_child_leg(cmd, name, timeout=1200):
    """Run `cmd` as a child process and return the JSON object on the last
    line of its stdout, or {"error": ...} when it times out, exits with a
    nonzero status (a signal shows as a negative one) or prints no JSON."""
    try:
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=timeout)
    except subprocess.TimeoutExpired:
        return {"error": f"{name} child process timed out after {timeout} s"}
    if r.returncode != 0:
        return {"error": f"{name} child process exited with status {r.returncode}"}
    try:
        out = json.loads(r.stdout.strip().splitlines()[-1])
    except (IndexError, ValueError) as e:
        return {"error": f"{name} child process printed no result: {e!r}"}
    return out if isinstance(out, dict) else {"error": f"{name} child process printed a non-object"}


def _small_legs(args, stream, result):
    """The 0.5B-shaped step at 32 rows (then at 1 row with the 'b1' leg), and
    the batch sweep and bucketed capture over its weights."""
    if args.no_small:
        return

    def small(detail, wname):
        res, dw = small_step(stream, wname, 200, 8.0 if detail else 3.0, detail)
        return res, dw
    sm, dw = small(True, SMALL)
    result[SMALL] = _rounded(json.loads(json.dumps(sm, default=_jsonable)))
    if not args.no_b1:
        result["qwen05b_b1_ctx512"] = _rounded(_leg(lambda: small(False, "qwen05b_b1_ctx512")[0]))
    if not args.no_sweep:
        result["batch_sweep"] = _rounded(_leg(batch_sweep, stream, dw))
        result["bucketed_capture"] = _rounded(_leg(bucket_capture, stream, dw))
    del dw
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-seconds", type=float, default=8.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-full", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-small", action="store_true")
    ap.add_argument("--legs", default="headline,small,b1,sweep,dense,cpu",
                    help="comma list of legs to run (profiling runs take one); without 'headline' the line "
                         "carries only the legs run and no value")
    ap.add_argument("--child-leg", choices=["dense"], default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()
    faulthandler.enable()  # a native crash prints the Python frames it happened under
    legs = set(args.legs.split(","))
    args.no_small = args.no_small or "small" not in legs
    args.no_b1 = "b1" not in legs
    args.no_sweep = args.no_sweep or "sweep" not in legs
    args.no_dense = args.no_dense or "dense" not in legs
    args.no_cpu_baseline = args.no_cpu_baseline or "cpu" not in legs
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the decode step is built and measured on a single MI355X "
              "(no sharding, no collectives); --gpus must be 1.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ns.lib()
    stream = torch.cuda.Stream()
    # a plain device copy of known size: calibrates the HBM byte counters
    # (FETCH_SIZE / WRITE_SIZE) of a profiled run of this same command
    calib_bytes = 256 << 20
    calib_src = torch.ones(calib_bytes // 4, device="cuda")
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    if args.child_leg == "dense":  # run by dense_leg_isolated
        print(json.dumps(_rounded(_leg(dense_batch, stream)), default=_jsonable), flush=True)
        return
    if "headline" not in legs:
        result = {"metric": "decode tokens/s @1 GPU; attn HBM GB/s and GEMM MFMA % of peak", "value": None,
                  "legs": sorted(legs)}
        _small_legs(args, stream, result)
        if not args.no_dense:
            result["dense_batch"] = _rounded(_leg(dense_batch, stream))
            result.update(dense_rooflines(result["dense_batch"]))
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = _rounded(cpu_baseline(args.cpu_baseline_full))
        print(json.dumps(result, default=_jsonable), flush=True)
        return
    w, b, r = llama80(args, stream)
    s = w.model
    runs = r["runs"]
    step_s = runs[-1]
    ctx = (b.row_pos + 1).tolist()
    sb = rf.step_bytes(s, ctx)
    kern = r["kernels"]
    tot = sum(v["us_per_step"] for v in kern.values())
    att, gu = r["att"], r["gu"]
    # dominant kernel: the paged decode attention (4 wavefronts per (row, KV
    # head) item over whole contexts, no combine launch), the kernel with the
    # largest share of the step's device time in the kernel trace of this
    # command; HBM-bound.  Its average launch duration from back-to-back
    # launches over the layers' caches (events on the launching stream).
    roof = {"kernel": "paged decode attention (attn_mfma_kernel, whole contexts)", "bound": "hbm",
            "achieved": round(att["gbs"], 1), "peak": rf.HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(att["gbs"] / rf.HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic("attention_llama70b_80l_b256"),
            "bytes_per_launch": att["bytes"], "avg_launch_us": round(att["us"], 3),
            "isolated_launches": att["launches"],
            "in_step_event_interval_us": round(kern["attention"]["us_per_launch"], 3),
            "share_of_step": round(kern["attention"]["us_per_step"] / tot, 3)}
    T, H, F = b.n_rows, s.hidden, s.ffn
    gfl = rf.gemm_flops(T, F, H, True)
    gemm_roof = {"kernel": "gate-up projection + SwiGLU at 256 rows (gemm_big_kernel)", "bound": "mfma",
                 "achieved": round(gfl / (gu["us"] * 1e-6) / 1e12, 1), "peak": rf.BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(gfl / (gu["us"] * 1e-6) / 1e12 / rf.BF16_PEAK_TFLOPS, 4),
                 "hbm_gbs": round(gu["gbs"], 1), "hbm_frac": round(gu["gbs"] / rf.HBM_PEAK_GBS, 4),
                 "flops_per_launch": gfl, "bytes_per_launch": gu["bytes"], "avg_launch_us": round(gu["us"], 3),
                 "isolated_launches": gu["launches"],
                 # back-to-back launches hold the matrix cores busy without a
                 # pause and run at a lower clock than the step's, where the
                 # memory-bound kernels come between them
                 "in_step_event_interval_us": round(kern["gate_up_proj"]["us_per_launch"], 3),
                 "in_step_tflops": round(gfl / (kern["gate_up_proj"]["us_per_launch"] * 1e-6) / 1e12, 1),
                 "share_of_step": round(kern["gate_up_proj"]["us_per_step"] / tot, 3)}
    result = {
        "metric": "decode tokens/s @1 GPU; attn HBM GB/s and GEMM MFMA % of peak",
        "value": round(b.n_rows / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and cached context, drawn on the device)",
        "config": {"workload": w.name, "batch": b.n_rows, "context": "uniform 512..1536", "layers": s.n_layers,
                   "hidden": s.hidden, "heads": f"{s.n_q_heads}q/{s.n_kv_heads}kv", "vocab": s.vocab,
                   "kv_block": 16, "mode": "hipGraph replay of the whole step", "parallelism": "single GPU"},
        "roofline": roof,
        "gemm_roofline": gemm_roof,
        "calibration_copy_bytes": calib_bytes,
        "step": _rounded({"runs_ms": [x * 1e3 for x in runs], "runs_disagree_over_15pct": max(runs) > 1.15 * min(runs),
                          "eager_ms": r["eager"] * 1e3, "fixed_cost_ms": (r["eager"] - step_s) * 1e3,
                          "kernels_per_step": r["launches"], "algorithmic_bytes": sb,
                          "hbm_floor_ms": rf.floor_seconds(sb) * 1e3,
                          "step_hbm_frac": sb / step_s / 1e9 / rf.HBM_PEAK_GBS,
                          "nano_overlap_ms": r["nano_ms"], "nano_split": list(w.nano_splits),
                          "chosen_schedule": "unsplit" if step_s * 1e3 <= r["nano_ms"] else "nano_overlap",
                          "warm_seconds": args.warm_seconds, "weights_gb": r["weights_gb"],
                          "kv_pool_gb": r["kv_pool_gb"], "setup_s": r["setup_s"]}),
        "clock": _rounded(r["clock"]),
        "corun_interference": _rounded(r["corun"]),
        "kernels": _rounded(kern),
    }
    del r
    _small_legs(args, stream, result)
    if not args.no_dense:
        torch.cuda.empty_cache()
        result["dense_batch"] = _rounded(dense_leg_isolated())
        result.update(dense_rooflines(result["dense_batch"]))
    result["torch_copy_rate"] = _rounded(copy_ceiling(stream))
    result["hbm_read_ceiling"] = _rounded(read_ceiling(stream))
    rc = result["hbm_read_ceiling"]["gbs"]
    for key in ("roofline", "dense_attention_roofline"):
        if key in result:
            result[key]["frac_of_read_ceiling"] = round(result[key]["achieved"] / rc, 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _rounded(cpu_baseline(args.cpu_baseline_full))
    print(json.dumps(result, default=_jsonable), flush=True)


if __name__ == "__main__":
    main()
