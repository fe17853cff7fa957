"""Kernel-level parity on the GPU, through the C ABI: the dense projection
against a float64 reference of the same product, and paged attention against
the oracle (plus its exact special cases)."""
import numpy as np
import pytest
import torch

from decode_step_06_amd import ns
from decode_step_06_amd.configs import ModelShape
from gpu_helpers import max_abs, rel_l2, say
from oracle import decoder as od

pytestmark = pytest.mark.gpu


def _bf16_grid(a):
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)


# (2000, 8100, 512): 256 x 256 tiles over 8 row tiles, the ping-pong kernel,
# with ragged last row and column tiles
GEMM_SHAPES = [(1, 64, 64), (5, 130, 96), (16, 896, 896), (17, 1152, 896), (32, 300, 128), (33, 256, 4864),
               (64, 64, 256), (100, 520, 160), (130, 384, 512), (257, 640, 1024), (32, 896, 4864),
               (1, 896, 4864), (32, 4864, 896), (8, 1000, 1024), (192, 1300, 1056), (2000, 8100, 512)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("epi", [ns.NS_EPI_STORE, ns.NS_EPI_RESID, ns.NS_EPI_SILU])
def test_gemm_bf16_matches_float64(M, N, K, epi):
    say(f"gemm bf16 M={M} N={N} K={K} epi={epi}")
    rng = np.random.default_rng(M * 7 + N + K + epi)
    A = _bf16_grid(rng.standard_normal((M, K)))
    Bn = 2 * N if epi == ns.NS_EPI_SILU else N
    B = _bf16_grid(rng.standard_normal((Bn, K)) * 0.05)
    ref = A.double() @ B.double().T
    if epi == ns.NS_EPI_SILU:
        g, u = ref[:, :N], ref[:, N:]
        ref = g / (1 + torch.exp(-g)) * u
        C = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    else:
        C0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32))
        C = C0.cuda().clone()
        if epi == ns.NS_EPI_RESID:
            ref = ref + C0.double()
    Ad, Bd = A.cuda(), B.cuda()
    C_in = C.clone()
    ns.ns_op_gemm(ns.NS_BF16, epi, M, N, K, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr())
    torch.cuda.synchronize()
    got = C.double().cpu().numpy()
    # deterministic: a second call gives the same bits
    C2 = C_in.clone()
    ns.ns_op_gemm(ns.NS_BF16, epi, M, N, K, Ad.data_ptr(), Bd.data_ptr(), C2.data_ptr())
    torch.cuda.synchronize()
    assert torch.equal(C2.cpu(), C.cpu())
    ref = ref.numpy()
    # fp32 accumulation of K products (and a final bf16 rounding for SwiGLU)
    tol = 4e-3 if epi == ns.NS_EPI_SILU else 1e-5
    assert rel_l2(got, ref) < tol, (rel_l2(got, ref), max_abs(got, ref))


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES + [(2048, 1024, 8192), (256, 896, 4864), (128, 1152, 896)])
@pytest.mark.parametrize("epi", [ns.NS_EPI_STORE, ns.NS_EPI_SILU])
def test_gemm_kslab_major_weights_equal_row_major(M, N, K, epi):
    """The engine's K-slab-major weights give the row-major result bit for
    bit (same kernels, same accumulation order; only the addressing of B
    differs), at every regime: weight streaming, split tiles, big tiles."""
    from decode_step_06_amd.runner import pack_kslab_host
    say(f"gemm packed B M={M} N={N} K={K} epi={epi}")
    rng = np.random.default_rng(M + 3 * N + K + epi)
    A = _bf16_grid(rng.standard_normal((M, K))).cuda()
    Bn = 2 * N if epi == ns.NS_EPI_SILU else N
    Bh = _bf16_grid(rng.standard_normal((Bn, K)) * 0.05)
    Bp = torch.from_numpy(pack_kslab_host(Bh.view(torch.int16).numpy())).view(torch.bfloat16).cuda()
    # the device packer agrees with the host reordering
    Bd = Bh.cuda()
    Bq = torch.empty_like(Bd)
    ns.ns_pack_weight(Bd.data_ptr(), Bq.data_ptr(), Bn, K)
    torch.cuda.synchronize()
    assert torch.equal(Bq.view(torch.int16), Bp.view(torch.int16))
    dt = torch.bfloat16 if epi == ns.NS_EPI_SILU else torch.float32
    C1 = torch.zeros((M, N), dtype=dt, device="cuda")
    C2 = torch.zeros((M, N), dtype=dt, device="cuda")
    ns.ns_op_gemm(ns.NS_BF16, epi, M, N, K, A.data_ptr(), Bd.data_ptr(), C1.data_ptr())
    ns.ns_op_gemm_packed(ns.NS_BF16, epi, M, N, K, A.data_ptr(), Bp.data_ptr(), C2.data_ptr())
    torch.cuda.synchronize()
    assert torch.equal(C1.cpu(), C2.cpu())


SLAB_SHAPES = [(1, 64, 64), (5, 160, 96), (17, 1152, 896), (33, 256, 4864), (64, 64, 256), (100, 512, 160),
               (130, 384, 512), (256, 896, 4864), (257, 640, 1024), (32, 4864, 896), (300, 512, 1024),
               (2048, 1024, 8192)]


@pytest.mark.parametrize("M,N,K", SLAB_SHAPES)
@pytest.mark.parametrize("epi", [ns.NS_EPI_STORE, ns.NS_EPI_RESID, ns.NS_EPI_SILU])
def test_gemm_slab_layouts_equal_row_major(M, N, K, epi):
    """The projections as a bf16 step runs them -- A and the SwiGLU output
    K-slab-major with slab blocks of more rows than the launch's (an odd
    count), the weights K-slab-major -- give the row-major result bit for bit
    in every regime, read only A's first M rows of each block and leave the
    output blocks' other rows untouched."""
    from decode_step_06_amd.runner import pack_kslab_host
    say(f"gemm slab layouts M={M} N={N} K={K} epi={epi}")
    rng = np.random.default_rng(7 * M + N + K + epi)
    a_rows, c_rows = M | 1 if M % 2 == 0 else M + 2, M + 3
    A = _bf16_grid(rng.standard_normal((M, K))).cuda()
    # rows past M hold values that would change the result if read
    Apad = torch.cat([A, _bf16_grid(rng.standard_normal((a_rows - M, K)) * 1e3).cuda()])
    As = torch.empty_like(Apad)
    ns.ns_pack_weight(Apad.data_ptr(), As.data_ptr(), a_rows, K)
    Bn = 2 * N if epi == ns.NS_EPI_SILU else N
    Bp = torch.from_numpy(pack_kslab_host(_bf16_grid(rng.standard_normal((Bn, K)) * 0.05).view(torch.int16).numpy()))
    Bp = Bp.view(torch.bfloat16).cuda()
    if epi == ns.NS_EPI_SILU:
        ref = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
        sentinel = torch.tensor(12345.0, dtype=torch.bfloat16)
        got = torch.full((N // 32 * c_rows * 32,), float(sentinel), dtype=torch.bfloat16, device="cuda")
    else:
        ref = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).cuda()
        got = ref.clone()
    ns.ns_op_gemm_packed(ns.NS_BF16, epi, M, N, K, A.data_ptr(), Bp.data_ptr(), ref.data_ptr())
    ns.ns_op_gemm_slab(epi, M, N, K, As.data_ptr(), a_rows, Bp.data_ptr(), got.data_ptr(), c_rows)
    torch.cuda.synchronize()
    if epi == ns.NS_EPI_SILU:
        blocks = got.cpu().view(N // 32, c_rows, 32)
        unpacked = blocks[:, :M, :].permute(1, 0, 2).reshape(M, N)
        assert torch.equal(unpacked.view(torch.int16), ref.cpu().view(torch.int16))
        assert torch.equal(blocks[:, M:, :], torch.full_like(blocks[:, M:, :], float(sentinel)))
    else:
        assert torch.equal(got.cpu(), ref.cpu())


def test_gemm_slab_rejects_bad_arguments():
    x = torch.zeros((64 * 64,), dtype=torch.bfloat16, device="cuda")
    for args in ((3, 4, 32, 64, 4), (ns.NS_EPI_STORE, 4, 32, 48, 4), (ns.NS_EPI_STORE, 4, 32, 64, 3),
                 (ns.NS_EPI_SILU, 4, 48, 64, 4)):
        epi, M, N, K, a_rows = args
        with pytest.raises(ns.NSError):
            ns.ns_op_gemm_slab(epi, M, N, K, x.data_ptr(), a_rows, x.data_ptr(), x.data_ptr(), M)
    with pytest.raises(ns.NSError):  # the SwiGLU output's blocks must hold M rows
        ns.ns_op_gemm_slab(ns.NS_EPI_SILU, 4, 32, 64, x.data_ptr(), 4, x.data_ptr(), x.data_ptr(), 3)


def test_pack_weight_rejects_bad_shapes():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros_like(x)
    for args in ((x.data_ptr(), x.data_ptr(), 4, 64), (x.data_ptr(), y.data_ptr(), 4, 48),
                 (x.data_ptr(), y.data_ptr(), 0, 64), (0, y.data_ptr(), 4, 64)):
        with pytest.raises(ns.NSError):
            ns.ns_pack_weight(*args)
    with pytest.raises(ns.NSError):  # the packed layout is bf16 only
        ns.ns_op_gemm_packed(ns.NS_F32, ns.NS_EPI_STORE, 4, 4, 64, x.data_ptr(), x.data_ptr(), y.data_ptr())


@pytest.mark.parametrize("epi", [ns.NS_EPI_STORE, ns.NS_EPI_RESID, ns.NS_EPI_SILU])
def test_gemm_f32_matches_float64(epi):
    rng = np.random.default_rng(epi)
    M, N, K = 7, 45, 70
    A = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    Bn = 2 * N if epi == ns.NS_EPI_SILU else N
    B = torch.from_numpy(rng.standard_normal((Bn, K)).astype(np.float32))
    ref = A.double() @ B.double().T
    C0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32))
    if epi == ns.NS_EPI_SILU:
        ref = ref[:, :N] / (1 + torch.exp(-ref[:, :N])) * ref[:, N:]
    elif epi == ns.NS_EPI_RESID:
        ref = ref + C0.double()
    C = C0.cuda().clone()
    Ad, Bd = A.cuda(), B.cuda()   # keep the device copies alive across the call
    ns.ns_op_gemm(ns.NS_F32, epi, M, N, K, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr())
    torch.cuda.synchronize()
    assert rel_l2(C.double().cpu().numpy(), ref.numpy()) < 1e-6


def test_gemm_rejects_unsupported_k():
    A = torch.zeros((4, 40), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ns.NSError) as ei:
        ns.ns_op_gemm(ns.NS_BF16, 0, 4, 4, 40, A.data_ptr(), A.data_ptr(), A.data_ptr())
    assert ei.value.code == ns.NS_ESHAPE


# ---------------------------------------------------------------- attention
def _attn_setup(shape: ModelShape, ctx, seed, shuffle=True, nan_poison=True):
    """Cache and queries for rows (one per sequence) with the given context
    lengths; returns device buffers and the logical host copies."""
    rng = np.random.default_rng(seed)
    nkv, d, G = shape.n_kv_heads, shape.head_dim, shape.group
    E = 8 if shape.dtype == "bf16" else 4
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    S = len(ctx)
    maxb = max(-(-c // 16) for c in ctx)
    nb = sum(-(-c // 16) for c in ctx) + 3
    # the block order comes from its own generator so the data are the same either way
    order = np.random.default_rng(seed + 1000).permutation(nb) if shuffle else np.arange(nb)
    btab = -np.ones((S, maxb), np.int32)
    k = 0
    for s, c in enumerate(ctx):
        for j in range(-(-c // 16)):
            btab[s, j] = order[k]
            k += 1
    desc = ns.model_desc(shape)
    kvb = ns.ns_kv_bytes(desc, nb) // shape.n_layers
    # physical layout (documented in ns.h), built on the host: unused slots NaN
    fill = float("nan") if nan_poison else 0.0
    kphys = torch.full((nb, nkv, d // E, 16, E), fill, dtype=dt)
    # V: token rows for fp32, each block transposed ([d][16]) for bf16
    vphys = torch.full((nb, nkv, 16, d), fill, dtype=dt)
    K, V = {}, {}
    for s, c in enumerate(ctx):
        kk = torch.from_numpy(rng.standard_normal((c, nkv, d)).astype(np.float32)).to(dt)
        vv = torch.from_numpy(rng.standard_normal((c, nkv, d)).astype(np.float32)).to(dt)
        K[s], V[s] = kk, vv
        for p in range(c):
            blk, tok = int(btab[s, p // 16]), p % 16
            kphys[blk, :, :, tok, :] = kk[p].reshape(nkv, d // E, E)
            vphys[blk, :, tok, :] = vv[p]
    if shape.dtype == "bf16":
        vphys = vphys.transpose(2, 3).contiguous()
    kv = torch.cat([kphys.reshape(-1).view(torch.uint8), vphys.reshape(-1).view(torch.uint8)]).cuda()
    assert kv.numel() == kvb
    q = torch.from_numpy(rng.standard_normal((S, shape.n_q_heads, d)).astype(np.float32)).to(dt)
    # attention layout [S][nkv][d/E][G][E]
    q_att = q.reshape(S, nkv, G, d // E, E).permute(0, 1, 3, 2, 4).contiguous()
    return dict(desc=desc, kv=kv, nb=nb, btab=btab, maxb=maxb, K=K, V=V, q=q, q_att=q_att, dt=dt)


def _attn_run(shape, st, ctx, wg_cap=0):
    S = len(ctx)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    rowb, pos, bt = dev(np.arange(S)), dev(np.array(ctx) - 1), dev(st["btab"])
    out = torch.full((S, shape.n_q_heads * shape.head_dim), float("nan"), dtype=st["dt"], device="cuda")
    wsb = ns.ns_op_attention_ws_bytes(st["desc"], S, st["maxb"])
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    qa = st["q_att"].cuda()
    ns.ns_op_attention(st["desc"], S, qa.data_ptr(), st["kv"].data_ptr(), st["nb"], rowb.data_ptr(),
                       pos.data_ptr(), bt.data_ptr(), st["maxb"], out.data_ptr(), ws.data_ptr(), wsb, wg_cap)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().reshape(S, shape.n_q_heads, shape.head_dim)


ATTN_SHAPES = [
    ModelShape("qwen-attn", 1, 896, 14, 2, 64, 64, 0, False, "bf16"),
    ModelShape("llama-attn", 1, 8192, 64, 8, 128, 64, 0, False, "bf16"),
    ModelShape("tiny-attn", 1, 128, 4, 1, 32, 64, 0, False, "f32"),
]


@pytest.mark.parametrize("shape", ATTN_SHAPES, ids=lambda s: s.name)
def test_attention_matches_oracle_ragged(shape):
    ctx = [1, 2, 15, 16, 17, 63, 64, 65, 130, 511, 700]
    if shape.n_kv_heads == 8:
        ctx = [1, 17, 64, 300, 1024]
    say(f"attention {shape.name} ctx={ctx}")
    st = _attn_setup(shape, ctx, seed=1)
    got = _attn_run(shape, st, ctx)
    for s, c in enumerate(ctx):
        ref, _ = od.attention_row(st["q"][s].double().numpy(), st["K"][s].double().numpy(),
                                  st["V"][s].double().numpy(), shape.group)
        tol = 4e-3 if shape.dtype == "bf16" else 1e-5   # output stored in bf16
        assert rel_l2(got[s], ref) < tol, (s, c, rel_l2(got[s], ref))


@pytest.mark.parametrize("shape", ATTN_SHAPES[:2], ids=lambda s: s.name)
def test_attention_single_cached_token_returns_v_exactly(shape):
    ctx = [1] * 5
    st = _attn_setup(shape, ctx, seed=2)
    got = _attn_run(shape, st, ctx)
    for s in range(5):
        for h in range(shape.n_q_heads):
            np.testing.assert_array_equal(got[s, h], st["V"][s][0, h // shape.group].float().numpy())


def test_attention_shuffled_table_equals_identity_bit_exact():
    shape = ATTN_SHAPES[0]
    ctx = [37, 300, 64, 129]
    a = _attn_run(shape, _attn_setup(shape, ctx, seed=3, shuffle=True), ctx)
    b = _attn_run(shape, _attn_setup(shape, ctx, seed=3, shuffle=False), ctx)
    np.testing.assert_array_equal(a, b)


def test_attention_workgroup_cap_is_bit_exact():
    shape = ATTN_SHAPES[1]
    ctx = [100, 1024, 333, 5]
    st = _attn_setup(shape, ctx, seed=4)
    a = _attn_run(shape, st, ctx, wg_cap=0)
    b = _attn_run(shape, st, ctx, wg_cap=7)
    np.testing.assert_array_equal(a, b)


def test_attention_kv_load_policy_is_bit_exact():
    """A layer region of 512 MiB or more takes the cache with non-temporal
    loads, a smaller one with ordinary loads: the same cache placed in both
    gives the same bits."""
    shape = ATTN_SHAPES[1]
    ctx = [1, 16, 17, 200, 1024, 777, 64, 65, 1500, 3]
    st = _attn_setup(shape, ctx, seed=6)
    small = _attn_run(shape, st, ctx)
    per_block = ns.ns_kv_bytes(st["desc"], 1) // shape.n_layers  # K + V bytes of one block
    nb_big = -(-(512 << 20) // per_block)
    assert nb_big > st["nb"] and nb_big * per_block >= 512 << 20 > st["nb"] * per_block
    half, half_big = st["nb"] * per_block // 2, nb_big * per_block // 2
    big = torch.zeros(nb_big * per_block, dtype=torch.uint8, device="cuda")
    big[:half] = st["kv"][:half]                       # K blocks
    big[half_big:half_big + half] = st["kv"][half:]    # V blocks
    say(f"attention load policy: {st['nb']} blocks ({st['nb'] * per_block >> 20} MiB) vs {nb_big} blocks")
    large = _attn_run(shape, dict(st, kv=big, nb=nb_big), ctx)
    assert np.isfinite(small).all()
    np.testing.assert_array_equal(small, large)


# Launch shapes the engine picks from the batch: 8 wavefronts per work item
# for few items, 4 up to 4095 items, 1 from 4096, and a split context with
# the combine launch for a long context at a small batch.
@pytest.mark.parametrize("shape_i,n_rows,ctx_hi", [(0, 300, 300), (0, 1100, 80), (0, 2100, 60), (0, 1, 9000),
                                                   (1, 1, 4100)],
                         ids=["qwen-300rows-4waves", "qwen-1100rows-4waves", "qwen-2100rows-1wave",
                              "qwen-ctx9000-split", "llama-ctx4100-split"])
def test_attention_launch_shapes_match_oracle(shape_i, n_rows, ctx_hi):
    shape = ATTN_SHAPES[shape_i]
    rng = np.random.default_rng(11 + n_rows)
    ctx = [ctx_hi] if n_rows == 1 else [int(c) for c in rng.integers(1, ctx_hi + 1, n_rows)]
    say(f"attention launch shape {shape.name} rows={n_rows} ctx<={ctx_hi}")
    st = _attn_setup(shape, ctx, seed=5)
    got = _attn_run(shape, st, ctx)
    for s, c in enumerate(ctx):
        ref, _ = od.attention_row(st["q"][s].double().numpy(), st["K"][s].double().numpy(),
                                  st["V"][s].double().numpy(), shape.group)
        assert rel_l2(got[s], ref) < 4e-3, (s, c, rel_l2(got[s], ref))   # output stored in bf16
