"""Shared setup for the GPU parity tests: run a workload through the C ABI
and through the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

from decode_step_06_amd import ns
from decode_step_06_amd.configs import ModelShape, Workload
from decode_step_06_amd.inputs import Batch, gen_batch, gen_weights
from decode_step_06_amd.runner import (DeviceWeights, alloc_sequences, blocks_for, create_engine, fill_past)
from oracle import decoder as od
from oracle import kvcache as okv


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


# Tolerances (relative L2, max abs) over an output.
#  bf16: the bound for bf16 activations -- one layer, or one kernel, given the
#        same inputs on both sides.
#  bf16_stack: a whole multi-layer stack.  GPU and oracle round to bf16 at
#        the same storage points, but from fp32 vs fp64 values, so some
#        roundings land on neighbouring bf16 values; such differences are
#        re-rounded at every later storage point and compound with depth
#        until they reach the size of bf16 rounding noise itself.  With
#        relative RMS rounding noise 2^-8 / sqrt(3) ~ 2.3e-3 per storage point
#        on the residual path and 2L + 1 = 49 such points in 24 layers, the
#        compounded bound is 2.3e-3 * sqrt(49) ~ 1.6e-2; max abs scales alike
#        (2e-2 * 7 / 2, rounded to 6e-2).
#  f32: fp32 models at fp32 accuracy.
def stack_tol(n_layers):
    """(rel L2, max abs) for an n-layer bf16 stack: 2.3e-3 and 8.6e-3 per
    square root of the 2L + 1 residual-path storage points."""
    r = float(np.sqrt(2 * n_layers + 1))
    return 2.3e-3 * r, 8.6e-3 * r


TOL = {"bf16": (5e-3, 2e-2), "bf16_stack": stack_tol(24), "bf16_stack80": stack_tol(80), "f32": (1e-5, 1e-5)}


def assert_close(gpu, ref, dtype, what=""):
    """Relative L2 and max abs error.  The max-abs bound is stated for
    unit-scale activations: when the reference's RMS exceeds 1 (e.g. a
    LLaMA-70B-shaped layer, whose down projection sums 28672 products) the
    bound scales with it."""
    r, m = rel_l2(gpu, ref), max_abs(gpu, ref)
    tr, tm = TOL[dtype]
    scale = max(1.0, float(np.sqrt(np.mean(np.square(np.asarray(ref, np.float64))))))
    tm = tm * scale
    say(f"  parity {what}: rel_l2={r:.3e} (<= {tr:g}) max_abs={m:.3e} (<= {tm:g}, output rms scale {scale:.2f})")
    assert np.isfinite(np.asarray(gpu)).all(), "non-finite GPU output"
    assert r <= tr and m <= tm, f"{what}: rel_l2 {r:.3e}, max_abs {m:.3e}"


class Case:
    """A workload set up on the device (weights, KV manager, cached context)."""

    def __init__(self, w: Workload, weights=None, batch: Batch = None, sched=None, max_tokens=None, maxb=None,
                 n_layers=None):
        self.w = w
        self.shape: ModelShape = w.model
        self.weights = weights if weights is not None else gen_weights(self.shape, seed=w.seeds["weights"])
        self.batch = batch if batch is not None else gen_batch(w)
        b = self.batch
        self.maxb = maxb or blocks_for(b.seq_lens)
        self.max_tokens = max_tokens or b.n_rows
        self.dw = DeviceWeights.from_numpy(self.shape, self.weights)
        self.h = create_engine(self.shape, self.dw, b.num_blocks, b.n_seqs, self.maxb, self.max_tokens,
                               b.free_order, sched)
        alloc_sequences(self.h, b.seq_lens)
        fill_past(self.h, b.past_seq, b.past_pos, b.past_k, b.past_v)
        self.x_dev = None if b.x is None else torch.from_numpy(b.x).cuda()

    @property
    def out_cols(self):
        return self.shape.vocab or self.shape.hidden

    def ns_batch(self, rows=None):
        b = self.batch
        sel = slice(None) if rows is None else rows
        x = None if self.x_dev is None else self.x_dev[sel].contiguous()
        return ns.Batch(b.row_seq[sel], b.row_pos[sel], None if b.tokens is None else b.tokens[sel], x)

    def step(self, stream=None, rows=None):
        nb = self.ns_batch(rows)
        n = nb.seq.shape[0]
        out = torch.full((n, self.out_cols), float("nan"), device="cuda")
        ns.ns_decode_step(self.h.eng, nb, out.data_ptr(), stream)
        torch.cuda.synchronize()
        return out

    def reset_cache(self):
        """Re-poison and re-fill the cache (a step writes its rows' K/V)."""
        from decode_step_06_amd.runner import nan_fill_
        nan_fill_(self.h.kv_mem, self.shape)
        b = self.batch
        fill_past(self.h, b.past_seq, b.past_pos, b.past_k, b.past_v)

    def tables(self):
        return ns.ns_kv_block_table(self.h.kv, self.batch.n_seqs, self.maxb)

    def close(self):
        self.h.destroy()
        torch.cuda.synchronize()


def oracle_run(shape, weights, batch: Batch, maxb, nano_splits=None, emulate=None):
    alloc = okv.BlockAllocator(batch.num_blocks, batch.free_order, batch.n_seqs, maxb)
    for s, n in enumerate(batch.seq_lens):
        alloc.alloc(s, int(n))
    tables = alloc.table_rows()
    cache = od.OracleKV(shape.n_layers, batch.num_blocks, shape.n_kv_heads, shape.head_dim)
    od.fill_past(cache, tables, batch.past_seq, batch.past_pos, batch.past_k, batch.past_v)
    orc = od.Oracle(shape, weights, emulate_bf16=emulate)
    out = orc.step(cache, tables, batch.row_seq, batch.row_pos, tokens=batch.tokens, x=batch.x,
                   nano_splits=nano_splits)
    return out, cache, tables


def sample_rows(n, k=6):
    """k rows spread over a batch of n, always the first and the last."""
    return sorted(set(np.linspace(0, n - 1, min(k, n)).round().astype(int).tolist()))


def oracle_sampled(shape, weights, batch: Batch, rows, keep, kept_k, kept_v, emulate=None):
    """The oracle on a sample of rows.  Rows are independent, so the sampled
    rows' outputs need only their own sequences' cached context: the sampled
    sequences get a compact pool of their own (attention reads a sequence's
    positions in logical order, whatever blocks hold them), filled with the
    kept past K/V (``keep`` masks batch.past_seq / past_pos)."""
    rows = np.asarray(rows)
    seqs = sorted({int(batch.row_seq[r]) for r in rows})
    cid = {s: i for i, s in enumerate(seqs)}
    lens = [int(batch.seq_lens[s]) for s in seqs]
    blocks = [-(-n // okv.BLOCK) for n in lens]
    nblk = sum(blocks)
    alloc = okv.BlockAllocator(nblk, np.arange(nblk, dtype=np.int32), len(seqs), max(blocks))
    for i, n in enumerate(lens):
        alloc.alloc(i, n)
    tables = alloc.table_rows()
    cache = od.OracleKV(shape.n_layers, nblk, shape.n_kv_heads, shape.head_dim)
    ps = np.array([cid[int(s)] for s in batch.past_seq[keep]], dtype=np.int32)
    od.fill_past(cache, tables, ps, batch.past_pos[keep], kept_k, kept_v)
    orc = od.Oracle(shape, weights, emulate_bf16=emulate)
    rs = np.array([cid[int(batch.row_seq[r])] for r in rows], dtype=np.int32)
    tok = None if batch.tokens is None else batch.tokens[rows]
    x = None if batch.x is None else batch.x[rows]
    return orc.step(cache, tables, rs, batch.row_pos[rows], tokens=tok, x=x)


# ---------------------------------------------------------------- teacher-forced per-layer parity
def one_layer_shape(shape: ModelShape) -> ModelShape:
    """Layer l of a stack on its own: one layer, no vocabulary (hidden state in
    and out)."""
    from dataclasses import replace
    return replace(shape, name=shape.name + "_1layer", n_layers=1, vocab=0, tied=False)


class LayerChain:
    """Layer l of a stack run alone on the GPU: a one-layer engine without a
    vocabulary over the stack's weights of layer l and layer l's part of the
    stack's KV memory (a stack's cache is its layers' regions back to back),
    with a KV manager that holds the same block tables.  Each call runs one
    eager step of that engine in the schedule given."""

    def __init__(self, h, b: Batch, sched, stream):
        import ctypes
        self._ct = ctypes
        self.h, self.b, self.sched, self.stream = h, b, sched, stream
        self.shape1 = one_layer_shape(h.shape)
        self.desc1 = ns.model_desc(self.shape1)
        self.kv1 = ns.ns_kv_create(self.desc1, h.num_blocks, h.max_seqs, h.max_blocks, b.free_order)
        for s, n in enumerate(b.seq_lens):
            ns.ns_kv_alloc(self.kv1, s, int(n))
        t1 = ns.ns_kv_block_table(self.kv1, h.max_seqs, h.max_blocks)
        t0 = ns.ns_kv_block_table(h.kv, h.max_seqs, h.max_blocks)
        assert np.array_equal(t0, t1), "one-layer KV manager holds other block tables"
        self.layer_bytes = ns.ns_kv_bytes(self.desc1, h.num_blocks)
        assert self.layer_bytes * h.shape.n_layers == h.kv_mem.numel()
        self.ws_bytes = ns.ns_workspace_bytes(self.desc1, h.max_tokens, h.max_blocks)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")

    def run(self, layer: int, x: torch.Tensor) -> torch.Tensor:
        """Layer `layer` of the stack on the fp32 hidden state x [T, H]."""
        lw = self.h.weights.t["layers"][layer]
        names = ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wdown")
        arrs = {n: (self._ct.c_void_p * 1)(lw[n].data_ptr()) for n in names}
        w = ns.ns_weights(*[arrs[n] for n in names], None, None, None)
        eng = ns.ns_engine_create(self.desc1, w, self.kv1, self.h.kv_mem.data_ptr() + layer * self.layer_bytes,
                                  self.layer_bytes, self.ws.data_ptr(), self.ws_bytes, self.h.max_tokens, self.sched)
        try:
            x = x.contiguous()
            out = torch.full_like(x, float("nan"))
            ns.ns_decode_step(eng, ns.Batch(self.b.row_seq, self.b.row_pos, None, x), out.data_ptr(), self.stream)
            self.stream.synchronize()
        finally:
            ns.ns_engine_destroy(eng)
        return out

    def head(self, x: torch.Tensor) -> torch.Tensor:
        """Final RMSNorm + LM head of the stack on the fp32 hidden state x."""
        s, t = self.h.shape, self.h.weights.t
        T = x.shape[0]
        hf = torch.empty((T, s.hidden), dtype=torch.bfloat16, device="cuda")
        logits = torch.full((T, s.vocab), float("nan"), device="cuda")
        ns.ns_op_rmsnorm(ns.NS_BF16, T, s.hidden, x.contiguous().data_ptr(), t["final_norm"].data_ptr(), s.rms_eps,
                         hf.data_ptr(), self.stream)
        ns.ns_op_gemm_packed(ns.NS_BF16, ns.NS_EPI_STORE, T, s.vocab, s.hidden, hf.data_ptr(),
                             t["lm_head"].data_ptr(), logits.data_ptr(), self.stream)
        self.stream.synchronize()
        return logits

    def close(self):
        if self.kv1:
            ns.ns_kv_destroy(self.kv1)
            self.kv1 = None


def check_layer(out, ref, x_in, what, ref32=None, max_abs_bound=None):
    """The bound for bf16 activations on a layer's output hidden state and on
    its change (the layer's attention and MLP contributions): relative L2 <=
    5e-3, and max abs <= 2e-2.

    ``ref32``: the oracle's float32-arithmetic run of the same layer (same
    bf16 storage points) on the same rows.  Two correct fp32 implementations
    of these storage points differ wherever a value lands on the other side of
    a bf16 rounding boundary, and such a difference scales with the
    activation: on hidden states of RMS well above 1 (a LLaMA-70B-shaped
    layer, RMS about 7.6) the oracle's own float32 run is more than 2e-2 from
    its float64 run at the worst element.  The max-abs bound is then 1.5 times
    that measured distance; the relative L2 bound never moves.

    ``max_abs_bound``: a max-abs bound the caller sets instead (a stack's
    layers checked against one bound pooled over all of them); returns
    (rel_l2, max_abs, change rel_l2, the oracle's own f32-vs-f64 max abs)."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    x_in = np.asarray(x_in, np.float64)
    assert np.isfinite(out).all(), f"{what}: non-finite GPU output"
    r, m = rel_l2(out, ref), max_abs(out, ref)
    rd = rel_l2(out - x_in, ref - x_in)
    tr, tm = TOL["bf16"]
    extra = ""
    d32 = 0.0
    if ref32 is not None:
        d32 = max_abs(ref32, ref)
        tm = max(tm, 1.5 * d32)
        extra = f" (oracle f32 vs f64: rel_l2={rel_l2(ref32, ref):.2e} max_abs={d32:.2e})"
    if max_abs_bound is not None:
        tm = max_abs_bound
    say(f"  {what}: rel_l2={r:.2e} max_abs={m:.2e} change rel_l2={rd:.2e}{extra}")
    assert r <= tr and m <= tm and rd <= tr, f"{what}: rel_l2 {r:.3e} max_abs {m:.3e} change rel_l2 {rd:.3e}"
    return r, m, rd, d32


def oracle_one_layer(shape, lw, tables, num_blocks, past_seq, past_pos, past_k_l, past_v_l, row_seq, row_pos, x,
                     precision="f64", emulate=None):
    """The oracle's layer alone (bf16 storage points for a bf16 model) on
    hidden input x, with that layer's cached context."""
    s1 = one_layer_shape(shape)
    ft = np.float64 if precision == "f64" else np.float32
    cache = od.OracleKV(1, num_blocks, shape.n_kv_heads, shape.head_dim, dtype=ft)
    od.fill_past(cache, tables, past_seq, past_pos, [past_k_l], [past_v_l])
    out = od.Oracle(s1, {"layers": [lw]}, emulate_bf16=emulate, precision=precision).step(
        cache, tables, row_seq, row_pos, x=np.asarray(x, ft))
    return out.astype(np.float64)
