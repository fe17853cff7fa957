"""Teacher-forced per-layer parity through the whole Qwen2.5-0.5B-shaped
stack (24 layers, tied 151,936-row head).

Layer l of the stack runs alone on the GPU (a one-layer engine over the
stack's weights of layer l and that layer's part of the stack's KV memory),
fed the GPU's own output of layer l - 1; the first layer gets the embedding
rows of the step's tokens.  The oracle's layer l gets the same input.  Every
layer's output hidden state and its change must be within the bound for bf16
activations (relative L2 <= 5e-3, max abs <= 2e-2, unscaled), and so must the
final norm + full-vocabulary LM head over the GPU's last hidden state.  The
engines run in the launch configuration the benchmark times for these
batches (RoPE and the cache write fused into attention)."""
import numpy as np
import pytest
import torch

from decode_step_06_amd import ns
from decode_step_06_amd.configs import WORKLOADS
from decode_step_06_amd.inputs import gen_batch, gen_weights
from decode_step_06_amd.runner import DeviceWeights, alloc_sequences, blocks_for, create_engine, fill_past
from gpu_helpers import LayerChain, check_layer, oracle_one_layer, say
from oracle import decoder as od
from oracle import kvcache as okv

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(300)
@pytest.mark.parametrize("wname", ["qwen05b_b32_ctx512", "qwen05b_b1_ctx512", "qwen05b_mix_b64"])
def test_qwen_stack_every_layer_and_head_teacher_forced(wname):
    w = WORKLOADS[wname]
    shape = w.model
    weights = gen_weights(shape, seed=w.seeds["weights"])
    b = gen_batch(w)
    maxb = blocks_for(b.seq_lens)
    sched = ns.make_sched(fuse_rope_attention=True)
    say(f"{wname}: {b.n_rows} rows, contexts {int(b.seq_lens.min())}..{int(b.seq_lens.max())}, "
        f"{shape.n_layers} layers teacher-forced")
    h = create_engine(shape, DeviceWeights.from_numpy(shape, weights), b.num_blocks, b.n_seqs, maxb, b.n_rows,
                      b.free_order, sched)
    stream = torch.cuda.Stream()
    chain = None
    try:
        alloc_sequences(h, b.seq_lens)
        fill_past(h, b.past_seq, b.past_pos, b.past_k, b.past_v)
        alloc = okv.BlockAllocator(b.num_blocks, b.free_order, b.n_seqs, maxb)
        for s, n in enumerate(b.seq_lens):
            alloc.alloc(s, int(n))
        tables = alloc.table_rows()
        chain = LayerChain(h, b, sched, stream)
        x = torch.from_numpy(np.ascontiguousarray(weights["embed"][b.tokens])).cuda()
        worst = [0.0, 0.0, 0.0]
        for layer in range(shape.n_layers):
            x_in = x.cpu().numpy()
            x = chain.run(layer, x)
            ref = oracle_one_layer(shape, weights["layers"][layer], tables, b.num_blocks, b.past_seq, b.past_pos,
                                   b.past_k[layer], b.past_v[layer], b.row_seq, b.row_pos, x_in)
            res = check_layer(x.cpu().numpy(), ref, x_in, f"layer {layer}")
            worst = [max(a, c) for a, c in zip(worst, res)]
        logits = chain.head(x).cpu().numpy()
        ref = od.Oracle(shape, weights).head(x.cpu().numpy().astype(np.float64))
        check_layer(logits, ref, np.zeros_like(ref), "final norm + LM head")
        agree = (np.argmax(logits, 1) == np.argmax(ref, 1)).mean()
        say(f"  worst layer: rel_l2={worst[0]:.2e} max_abs={worst[1]:.2e} change rel_l2={worst[2]:.2e}; "
            f"head argmax agreement {agree:.3f}")
        assert agree == 1.0
    finally:
        if chain is not None:
            chain.close()
        h.destroy()
        torch.cuda.synchronize()
