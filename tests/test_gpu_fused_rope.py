"""RoPE and the cache write of each row's own K/V fused into the bf16
attention kernel (ns_sched.fuse_rope_attention), for steps whose rows belong
to distinct sequences.  It computes the same bits as the separate
RoPE/cache-write kernel followed by attention: the outputs and the whole KV
cache after the step are compared bit for bit, in every launch shape of the
attention kernel that fuses it (8 and 4 wavefronts per work item, split
contexts, head_dim 64 and 128; from 2048 work items on the engine keeps the
separate kernel), eager and graph-replayed, nano-batched with overlap.
The fused step also matches the oracle, and a batch that repeats a sequence
is rejected with no side effects."""
import numpy as np
import pytest
import torch

from decode_step_06_amd import ns
from decode_step_06_amd.configs import ModelShape, Workload
from gpu_helpers import Case, assert_close, oracle_run, say

pytestmark = pytest.mark.gpu

SMALL = ModelShape("small", 2, 256, 8, 2, 64, 512, 1000, True, "bf16")
SMALL_H = ModelShape("small_h", 2, 256, 8, 2, 64, 512, 0, False, "bf16")
QWEN1 = ModelShape("qwen1", 1, 896, 14, 2, 64, 512, 0, False, "bf16")       # 7 query heads per KV head
LLAMA1 = ModelShape("llama1", 1, 1024, 8, 1, 128, 512, 0, False, "bf16")    # head_dim 128, 8 per KV head
KV8 = ModelShape("kv8", 1, 512, 16, 8, 64, 256, 0, False, "bf16")          # 8 KV heads, 2 query heads each

CASES = {
    # rows x KV heads <= 256: 8 wavefronts per item
    "small-8waves": Workload("f8", SMALL, 6, ctx_range=(1, 200)),
    # <= 2047 items: 4 wavefronts (split-K QKV slices: steps of <= 256 rows)
    "small-4waves": Workload("f4", SMALL_H, 200, ctx_range=(1, 40)),
    # more than 256 rows: the unsplit QKV projection's fp32 result
    "small-4waves-300rows": Workload("f4b", SMALL_H, 300, ctx_range=(1, 40)),
    # 1024 items of 8 KV heads: 4 wavefronts
    "kv8-4waves": Workload("f1", KV8, 128, ctx_range=(1, 70)),
    # 2048..4095 items: 4 wavefronts, where the engine keeps the separate
    # kernel (with slices)
    "kv8-4waves-2048items": Workload("f1", KV8, 256, ctx_range=(1, 70)),
    # >= 4096 items: one wavefront per item, separate kernel (with slices and
    # with the unsplit projection)
    "kv8-1wave": Workload("f1c", KV8, 512, ctx_range=(1, 40)),
    "small-1wave-2100rows": Workload("f1b", SMALL_H, 2100, ctx_range=(1, 24)),
    # contexts past 8 passes of 8 wavefronts: split into partitions + combine
    "qwen-split": Workload("fs", QWEN1, 3, ctx_range=(4100, 5000)),
    "llama-d128": Workload("fl", LLAMA1, 5, ctx_range=(1, 300)),
}


def _kv_bytes(c):
    torch.cuda.synchronize()
    return c.h.kv_mem.view(torch.uint8).clone()


@pytest.mark.parametrize("name", list(CASES))
def test_fused_rope_attention_is_bit_exact(name):
    w = CASES[name]
    c = Case(w)
    try:
        say(f"case {name}: {c.batch.n_rows} rows, contexts {int(c.batch.row_pos.min()) + 1}.."
            f"{int(c.batch.row_pos.max()) + 1}")
        ref = c.step().cpu()
        n_ref = ns.ns_engine_last_launches(c.h.eng)
        ref_kv = _kv_bytes(c)
        ns.ns_engine_set_sched(c.h.eng, ns.make_sched(fuse_rope_attention=True))
        c.reset_cache()
        got = c.step().cpu()
        fused = c.batch.n_rows * w.model.n_kv_heads < 2048
        assert ns.ns_engine_last_launches(c.h.eng) == n_ref - (w.model.n_layers if fused else 0)
        torch.testing.assert_close(got, ref, rtol=0, atol=0)
        assert torch.equal(_kv_bytes(c), ref_kv), "cache after the fused step differs"
        # a captured graph of the fused step replays the same bits
        out = torch.empty_like(got).cuda()
        stream = torch.cuda.Stream()
        g = ns.ns_graph_capture(c.h.eng, c.batch.n_rows, out.data_ptr(), stream)
        try:
            for _ in range(2):
                c.reset_cache()
                ns.ns_graph_replay(g, c.ns_batch(), stream)
                stream.synchronize()
                torch.testing.assert_close(out.cpu(), ref, rtol=0, atol=0)
        finally:
            ns.ns_graph_destroy(g)
    finally:
        c.close()


def test_fused_rope_attention_nano_overlap_launch_count_and_oracle():
    w = CASES["small-8waves"]
    c = Case(w)
    try:
        ref = c.step().cpu()
        n_ref = ns.ns_engine_last_launches(c.h.eng)
        ns.ns_engine_set_sched(c.h.eng, ns.make_sched(nano_rows=(2, 4), qkv_rows=(3, 3), overlap=True,
                                                      fuse_rope_attention=True))
        c.reset_cache()
        got = c.step().cpu()
        torch.testing.assert_close(got, ref, rtol=0, atol=0)
        ns.ns_engine_set_sched(c.h.eng, ns.make_sched(fuse_rope_attention=True))
        c.reset_cache()
        got = c.step().cpu().numpy()
        n_fused = ns.ns_engine_last_launches(c.h.eng)
        say(f"  kernels per step: {n_ref} separate, {n_fused} fused")
        assert n_fused == n_ref - w.model.n_layers
        orc, _, _ = oracle_run(w.model, c.weights, c.batch, c.maxb)
        assert_close(got, orc, "bf16", "fused RoPE/attention step vs oracle")
    finally:
        c.close()


def test_fused_rope_attention_rejects_repeated_sequences():
    w = Workload("fr", SMALL, 3, ctx_range=(5, 60), prefill_chunks=(4,))
    c = Case(w, sched=ns.make_sched(fuse_rope_attention=True))
    try:
        before = _kv_bytes(c)
        out = torch.full((c.batch.n_rows, c.out_cols), 7.0, device="cuda")
        with pytest.raises(ns.NSError) as ei:
            ns.ns_decode_step(c.h.eng, c.ns_batch(), out.data_ptr(), None)
        assert ei.value.code == ns.NS_EINVAL
        assert "more than one row" in str(ei.value)
        assert torch.equal(_kv_bytes(c), before)
        assert bool((out == 7.0).all())
        # the decode rows alone are accepted
        c.step(rows=slice(0, 3))
        # and the option excludes prefill tiles
        with pytest.raises(ns.NSError):
            ns.ns_engine_set_sched(c.h.eng, ns.make_sched(fuse_rope_attention=True, prefill_tiles=True))
    finally:
        c.close()
