"""The LLaMA-2-70B-shaped layer at the dense-batch size (2048 rows: 512
decode rows at context 1024, then three fresh prefill chunks of 512),
nano-batched 768/1280 with four QKV nano-ops and attention overlapped on the
second stream, in the launch configuration the benchmark times.  The oracle
computes sampled rows one by one."""
import numpy as np
import pytest
import torch

from decode_step_06_amd import ns
from decode_step_06_amd.configs import WORKLOADS
from decode_step_06_amd.inputs import gen_batch, gen_weights
from gpu_helpers import Case, assert_close, say
from oracle import decoder as od
from oracle import kvcache as okv

pytestmark = pytest.mark.gpu

SAMPLE_ROWS = [0, 1, 255, 511,                 # decode rows (context 1024)
               512, 513, 812, 1023,            # first prefill chunk: positions 0, 1, 300, 511
               1024 + 17, 1536 + 511]          # later chunks


@pytest.mark.parametrize("prefill_tiles", [True, False], ids=["prefill-tiles", "decode-kernel-only"])
def test_llama70b_layer_dense_batch_sampled_rows(prefill_tiles):
    w = WORKLOADS["llama70b_layer_t2048"]
    shape = w.model
    say("layer llama70b_layer_t2048: generating inputs")
    weights = gen_weights(shape, seed=0)
    b = gen_batch(w)
    sched = ns.make_sched(nano_rows=w.nano_splits, qkv_rows=(512,) * w.qkv_splits, overlap=True,
                          prefill_tiles=prefill_tiles)
    c = Case(w, weights=weights, batch=b, sched=sched)
    try:
        say("  GPU step")
        got = c.step().cpu().numpy()
        assert np.isfinite(got).all()
        say("  oracle for sampled rows")
        orc = od.Oracle(shape, weights)
        alloc = okv.BlockAllocator(b.num_blocks, b.free_order, b.n_seqs, c.maxb)
        for s, n in enumerate(b.seq_lens):
            alloc.alloc(s, int(n))
        tables = alloc.table_rows()
        np.testing.assert_array_equal(c.tables(), np.array(tables, dtype=np.int32))
        x = b.x.astype(np.float64)
        q, k, v = orc.qkv(0, x, b.row_pos)          # every row's K/V enters the cache
        slots = okv.slot_map(tables, b.row_seq, b.row_pos)
        # cached context of the decode rows plus this step's K/V, by slot
        kcache, vcache = {}, {}
        psl = okv.slot_map(tables, b.past_seq, b.past_pos)
        for i, s in enumerate(psl):
            kcache[s] = b.past_k[0][i]
            vcache[s] = b.past_v[0][i]
        for i, s in enumerate(slots):
            kcache[s] = k[i]
            vcache[s] = v[i]
        if prefill_tiles:
            # decode rows' attention queued last, prompt nano-batch's projections
            # first: the same work in another order, bit-exact
            ns.ns_engine_set_sched(c.h.eng, ns.make_sched(nano_rows=w.nano_splits, qkv_rows=(512,) * w.qkv_splits,
                                                          overlap=True, prefill_tiles=True, decode_rows_first=True))
            c.reset_cache()
            np.testing.assert_array_equal(c.step().cpu().numpy(), got)
        rows = np.array(SAMPLE_ROWS)
        o = np.zeros((len(rows), shape.n_q_heads, shape.head_dim))
        for j, t in enumerate(rows):
            s, p = int(b.row_seq[t]), int(b.row_pos[t])
            sl = [okv.slot_of(tables[s], i) for i in range(p + 1)]
            keys = np.stack([kcache[z] for z in sl]).astype(np.float64)
            vals = np.stack([vcache[z] for z in sl]).astype(np.float64)
            o[j], _ = od.attention_row(q[t], keys, vals, shape.group)
        o = od.round_bf16(o.reshape(len(rows), -1))
        ref = orc.post_attention(0, x[rows], o)
        assert_close(got[rows], ref, "bf16", "llama70b layer, sampled rows")
    finally:
        c.close()
