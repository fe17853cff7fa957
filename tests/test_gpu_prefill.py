"""The MFMA prefill-tile attention through the C ABI: rows forming tiles of
32 consecutive positions of one sequence (prompt chunks, with and without
cached context before them) mixed with decode rows and ragged remainders,
against the oracle's attention per row."""
import numpy as np
import pytest
import torch

from decode_step_06_amd import ns
from decode_step_06_amd.configs import ModelShape
from gpu_helpers import rel_l2, say
from oracle import decoder as od

pytestmark = pytest.mark.gpu

SHAPES = [
    ModelShape("llama-attn", 1, 8192, 64, 8, 128, 64, 0, False, "bf16"),
    ModelShape("qwen-attn", 1, 896, 14, 2, 64, 64, 0, False, "bf16"),
]


def _run(shape, ctx, rows, seed):
    """ctx: tokens cached per sequence (all positions written); rows: list of
    (sequence, position).  Returns the GPU output [n, nq, d] and the oracle's."""
    rng = np.random.default_rng(seed)
    nkv, d, G, E = shape.n_kv_heads, shape.head_dim, shape.group, 8
    S = len(ctx)
    maxb = max(-(-c // 16) for c in ctx)
    nb = sum(-(-c // 16) for c in ctx) + 2
    order = np.random.default_rng(seed + 7).permutation(nb)
    btab = -np.ones((S, maxb), np.int32)
    k = 0
    for s, c in enumerate(ctx):
        for j in range(-(-c // 16)):
            btab[s, j] = order[k]
            k += 1
    kphys = torch.full((nb, nkv, d // E, 16, E), float("nan"), dtype=torch.bfloat16)
    vphys = torch.full((nb, nkv, 16, d), float("nan"), dtype=torch.bfloat16)
    K, V = [], []
    for s, c in enumerate(ctx):
        kk = torch.from_numpy(rng.standard_normal((c, nkv, d)).astype(np.float32)).to(torch.bfloat16)
        vv = torch.from_numpy(rng.standard_normal((c, nkv, d)).astype(np.float32)).to(torch.bfloat16)
        K.append(kk)
        V.append(vv)
        for p in range(c):
            blk, tok = int(btab[s, p // 16]), p % 16
            kphys[blk, :, :, tok, :] = kk[p].reshape(nkv, d // E, E)
            vphys[blk, :, tok, :] = vv[p]
    vphys = vphys.transpose(2, 3).contiguous()  # bf16 cache: each V block stored [d][16]
    kv = torch.cat([kphys.reshape(-1).view(torch.uint8), vphys.reshape(-1).view(torch.uint8)]).cuda()
    n = len(rows)
    q = torch.from_numpy(rng.standard_normal((n, shape.n_q_heads, d)).astype(np.float32)).to(torch.bfloat16)
    q_att = q.reshape(n, nkv, G, d // E, E).permute(0, 1, 3, 2, 4).contiguous().cuda()
    seq = np.array([r[0] for r in rows], np.int32)
    pos = np.array([r[1] for r in rows], np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    rowb, posd, bt = dev(seq), dev(pos), dev(btab)
    out = torch.full((n, shape.n_q_heads * d), float("nan"), dtype=torch.bfloat16, device="cuda")
    desc = ns.model_desc(shape)
    wsb = ns.ns_op_attention_ws_bytes(desc, n, maxb)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    ns.ns_op_attention_prefill(desc, n, q_att.data_ptr(), kv.data_ptr(), nb, rowb.data_ptr(), posd.data_ptr(), bt.data_ptr(),
                       maxb, out.data_ptr(), ws.data_ptr(), wsb, 0)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().reshape(n, shape.n_q_heads, d)
    ref = np.stack([od.attention_row(q[i].double().numpy(), K[s][:p + 1].double().numpy(),
                                     V[s][:p + 1].double().numpy(), G)[0] for i, (s, p) in enumerate(rows)])
    return got, ref


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_prefill_tiles_match_oracle(shape):
    # seq 0: chunk of 64 after 236 cached positions (2 tiles); seq 1: fresh
    # chunk of 32 (1 tile); seq 2: fresh chunk of 45 (1 tile + 13 rows for the
    # decode kernel); seq 3: one decode row; then a short mixed tail
    ctx = [300, 32, 45, 700, 90]
    rows = [(0, p) for p in range(236, 300)] + [(1, p) for p in range(32)] + [(2, p) for p in range(45)]
    rows += [(3, 699)] + [(4, p) for p in range(70, 90)]
    say(f"prefill tiles {shape.name}: {len(rows)} rows")
    got, ref = _run(shape, ctx, rows, seed=5)
    for i in range(len(rows)):
        assert rel_l2(got[i], ref[i]) < 4e-3, (i, rows[i], rel_l2(got[i], ref[i]))


def test_prefill_tile_at_context_start_single_key_rows():
    """The first row of a fresh chunk sees only its own key: its output is V
    of that key for every head (rounded to bf16 at the store)."""
    shape = SHAPES[0]
    rows = [(0, p) for p in range(32)]
    got, ref = _run(shape, [32], rows, seed=6)
    np.testing.assert_allclose(got[0], ref[0], rtol=0, atol=0)
    for i in range(32):
        assert rel_l2(got[i], ref[i]) < 4e-3


def test_engine_step_with_prefill_tiles():
    """A 2-layer bf16 stack (head_dim 64, 4 query heads per KV head) over 32
    decode rows and two fresh prompt chunks (64 and 40 rows: three tiles and
    a remainder): with prefill tiles the step matches the oracle, the
    decode-kernel-only step within rounding, and a graph replay the eager
    step bit for bit; with a nano-batch split (at a multiple of 32 rows, so
    the tiles stay where they were) the overlapped step equals the serial
    one bit for bit and the oracle within the bound."""
    from decode_step_06_amd.configs import Workload
    from gpu_helpers import Case, assert_close, oracle_run
    shape = ModelShape("small-pf", 2, 256, 8, 2, 64, 512, 1000, True, "bf16")
    w = Workload("small_pf", shape, 32, ctx_range=(1, 200), prefill_chunks=(64, 40))
    c = Case(w, sched=ns.make_sched(prefill_tiles=True))
    try:
        say("engine step with prefill tiles: 32 decode rows + chunks of 64 and 40")
        tiles = c.step().cpu().numpy()
        ref, _, _ = oracle_run(shape, c.weights, c.batch, c.maxb)
        assert_close(tiles, ref, "bf16", "prefill tiles vs oracle")
        ns.ns_engine_set_sched(c.h.eng, ns.make_sched())
        c.reset_cache()
        plain = c.step().cpu().numpy()
        # fp16 probabilities on one side, fp32 on the other, and every bf16
        # storage point after it: the two agree to the same bound as each does
        # to the oracle
        assert_close(tiles, plain, "bf16", "prefill tiles vs decode kernel only")
        runs = {}
        for name, sched in (("serial", ns.make_sched(prefill_tiles=True)),
                            ("split", ns.make_sched(nano_rows=(64, 72), prefill_tiles=True)),
                            ("split-overlap", ns.make_sched(nano_rows=(64, 72), overlap=True, prefill_tiles=True))):
            ns.ns_engine_set_sched(c.h.eng, sched)
            c.reset_cache()
            eager = c.step().cpu().numpy()
            c.reset_cache()
            nb = c.ns_batch()
            out = torch.full((c.batch.n_rows, shape.vocab), float("nan"), device="cuda")
            st = torch.cuda.Stream()
            g = ns.ns_graph_capture(c.h.eng, c.batch.n_rows, out.data_ptr(), st)
            try:
                ns.ns_graph_replay(g, nb, st)
                st.synchronize()
            finally:
                ns.ns_graph_destroy(g)
            np.testing.assert_array_equal(out.cpu().numpy(), eager, err_msg=f"{name}: graph vs eager")
            runs[name] = eager
        np.testing.assert_array_equal(runs["serial"], tiles)
        # the second stream changes the order of launches, not their results
        np.testing.assert_array_equal(runs["split-overlap"], runs["split"])
        assert_close(runs["split"], ref, "bf16", "split step with prefill tiles vs oracle")
    finally:
        c.close()
