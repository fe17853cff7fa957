"""The attention entry point that allocates nothing (ns_op_attention_static:
split-context partials in a static device array) against the same op with a
caller workspace (ns_op_attention), through the C ABI: two calls in a row,
the second with a smaller batch, both with contexts split across work items
(so the partials are used), bit for bit."""
import numpy as np
import pytest
import torch

from decode_step_06_amd import ns
from decode_step_06_amd.configs import LLAMA70B
from gpu_helpers import one_layer_shape, say

pytestmark = pytest.mark.gpu


def _case(n_rows, ctx_lo, ctx_hi, seed):
    """n_rows decode rows of the LLaMA-70B-shaped layer (8 KV heads, 8 query
    heads each, head_dim 128) with contexts in [ctx_lo, ctx_hi], fragmented
    block tables and a random bf16 cache."""
    shape = one_layer_shape(LLAMA70B)
    desc = ns.model_desc(shape)
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, n_rows)
    nblk = [int(-(-c // 16)) for c in ctx]
    maxb = max(nblk)
    total = sum(nblk) + 3
    perm = rng.permutation(total).astype(np.int32)
    btab = np.full((n_rows, maxb), -1, np.int32)
    at = 0
    for r, n in enumerate(nblk):
        btab[r, :n] = perm[at:at + n]
        at += n
    kv_bytes = ns.ns_kv_bytes(desc, total)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    kv = (torch.randn(kv_bytes // 2, generator=g, device="cuda")).to(torch.bfloat16)
    d, G, nkv = shape.head_dim, shape.group, shape.n_kv_heads
    q = torch.randn((n_rows, nkv, d // 8, G, 8), generator=g, device="cuda").to(torch.bfloat16)
    return dict(desc=desc, n=n_rows, ctx=ctx, maxb=maxb, total=total, kv=kv, q=q,
                bseq=torch.arange(n_rows, dtype=torch.int32, device="cuda"),
                pos=torch.from_numpy((ctx - 1).astype(np.int32)).cuda(),
                btab=torch.from_numpy(btab).cuda(), out_cols=shape.n_q_heads * d)


def _run(c, static):
    out = torch.full((c["n"], c["out_cols"]), float("nan"), device="cuda", dtype=torch.bfloat16)
    args = (c["desc"], c["n"], c["q"].data_ptr(), c["kv"].data_ptr(), c["total"], c["bseq"].data_ptr(),
            c["pos"].data_ptr(), c["btab"].data_ptr(), c["maxb"], out.data_ptr())
    if static:
        ns.ns_op_attention_static(*args, 0)
    else:
        wsb = ns.ns_op_attention_ws_bytes(c["desc"], c["n"], c["maxb"])
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        ns.ns_op_attention(*args, ws.data_ptr(), wsb, 0)
    torch.cuda.synchronize()
    return out


def test_static_scratch_attention_matches_workspace_attention_twice():
    big = _case(64, 4000, 8192, 1)     # 512 work items of 4 wavefronts, contexts in two parts
    small = _case(4, 5000, 8192, 2)    # 32 work items of 8 wavefronts, contexts in two parts
    for c in (big, small):
        need = ns.ns_op_attention_ws_bytes(c["desc"], c["n"], c["maxb"])
        assert 0 < need <= ns.NS_ATTENTION_STATIC_SCRATCH_BYTES
        say(f"  {c['n']} rows, contexts {int(c['ctx'].min())}..{int(c['ctx'].max())}: partials {need} bytes")
    s_big = _run(big, True)
    s_small = _run(small, True)     # the second call, on a smaller input, reuses the array
    w_big = _run(big, False)
    w_small = _run(small, False)
    assert torch.isfinite(s_big.float()).all() and torch.isfinite(s_small.float()).all()
    assert torch.equal(s_big, w_big)
    assert torch.equal(s_small, w_small)
    # and once more on the first input after the second: the array keeps no state that matters
    assert torch.equal(_run(big, True), w_big)
