"""The Qwen2.5-0.5B-shaped continuous-batching mix at full size: batch 1, 8,
32, 64, 128 and 256, contexts uniform in 128..2048, fragmented block tables,
one hipGraph captured per batch size -- the launch configuration the
benchmark times.  Each replay is checked bit-exactly against an eager step,
and a sample of rows against the oracle."""
import numpy as np
import pytest
import torch

from decode_step_06_amd import ns
from decode_step_06_amd.configs import QWEN05B, WORKLOADS
from decode_step_06_amd.inputs import gen_batch, gen_weights
from decode_step_06_amd.runner import (DeviceWeights, alloc_sequences, blocks_for, create_engine,
                                       fill_past_random_on_device)
from gpu_helpers import assert_close, oracle_sampled, sample_rows, say

pytestmark = pytest.mark.gpu

SWEEP = (1, 8, 32, 64, 128, 256)


@pytest.fixture(scope="module")
def qwen():
    weights = gen_weights(QWEN05B, seed=0)
    # the oracle's copy in float64 once (it would widen every matrix per call)
    w64 = {"layers": [{k: v.astype(np.float64) for k, v in lw.items()} for lw in weights["layers"]],
           "final_norm": weights["final_norm"].astype(np.float64)}
    w64["embed"] = weights["embed"].astype(np.float64)
    w64["lm_head"] = w64["embed"]
    dw = DeviceWeights.from_numpy(QWEN05B, weights)
    yield w64, dw
    del dw
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", SWEEP)
def test_mix_graph_per_batch_size_matches_eager_and_oracle(qwen, B):
    w64, dw = qwen
    w = WORKLOADS[f"qwen05b_mix_b{B}"]
    b = gen_batch(w, with_past=False)
    rows = sample_rows(b.n_rows)
    seqs = sorted({int(b.row_seq[r]) for r in rows})
    keep = np.isin(b.past_seq, seqs)
    maxb = blocks_for(b.seq_lens)
    say(f"mix B={B}: 24 layers, contexts {int(b.seq_lens.min())}..{int(b.seq_lens.max())}, "
        f"pool {b.num_blocks} blocks (fragmented), sampled rows {rows}")
    # the benchmark's schedule for these decode batches: RoPE and the cache
    # write fused into attention
    h = create_engine(QWEN05B, dw, b.num_blocks, b.n_seqs, maxb, b.n_rows, b.free_order,
                      ns.make_sched(fuse_rope_attention=True))
    stream = torch.cuda.Stream()
    try:
        alloc_sequences(h, b.seq_lens)
        kept_k, kept_v = fill_past_random_on_device(h, b.past_seq, b.past_pos, seed=w.seeds["kv"], keep=keep)
        nb = ns.Batch(b.row_seq, b.row_pos, b.tokens)
        out_g = torch.full((b.n_rows, QWEN05B.vocab), float("nan"), device="cuda")
        out_e = torch.full_like(out_g, float("nan"))
        g = ns.ns_graph_capture(h.eng, b.n_rows, out_g.data_ptr(), stream)
        try:
            ns.ns_graph_replay(g, nb, stream)
            stream.synchronize()
            # a step rewrites its own rows' K/V with the same values, so an
            # eager step after the replay sees the same cache
            ns.ns_decode_step(h.eng, nb, out_e.data_ptr(), stream)
            stream.synchronize()
            assert torch.equal(out_g, out_e), "graph replay differs from the eager step"
            got = out_g[rows].cpu().numpy()
        finally:
            ns.ns_graph_destroy(g)
    finally:
        h.destroy()
        torch.cuda.synchronize()
    ref = oracle_sampled(QWEN05B, w64, b, rows, keep, kept_k, kept_v)
    assert_close(got, ref, "bf16_stack", f"mix B={B} logits of sampled rows")
    agree = (np.argmax(got, 1) == np.argmax(ref, 1)).mean()
    say(f"  argmax agreement {agree:.3f} over {len(rows)} rows")
