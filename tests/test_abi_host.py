"""The C-ABI library on the CPU: it loads, exports every entry point that
include/ns.h declares, and its host-only KV block manager and slot map match
the oracle bit for bit (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from decode_step_06_amd import ns
from decode_step_06_amd.configs import QWEN05B, TINY, LLAMA70B
from oracle import kvcache as okv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "ns.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(ns_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_entry_point():
    L = ns.lib()
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
        assert n in ns.SIGNATURES, f"{n} missing from the binding"
    assert sorted(ns.SIGNATURES) == names


def test_kv_bytes_and_workspace_sizes():
    d = ns.model_desc(QWEN05B)
    # K and V, 24 layers, 2 KV heads x 64 dims x 16 slots x bf16 per block
    assert ns.ns_kv_bytes(d, 10) == 24 * 2 * 10 * 2 * 16 * 64 * 2
    assert ns.ns_workspace_bytes(d, 32, 128) > 32 * 896 * 4
    bad = ns.model_desc(QWEN05B)
    bad.head_dim = 48
    assert ns.ns_kv_bytes(bad, 10) == 0


def _random_ops(rng, n_ops, max_seqs, nb):
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        s = int(rng.integers(0, max_seqs))
        if r < 0.75:
            ops.append(("alloc", s, int(rng.integers(0, 16 * 9))))
        else:
            ops.append(("free", s, 0))
    return ops


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_kv_manager_matches_oracle_bit_exact(seed):
    rng = np.random.default_rng(seed)
    nb, max_seqs, maxb = 40, 6, 8
    order = rng.permutation(nb).astype(np.int32)
    desc = ns.model_desc(TINY)
    kv = ns.ns_kv_create(desc, nb, max_seqs, maxb, order)
    ref = okv.BlockAllocator(nb, order, max_seqs, maxb)
    try:
        for op, s, n in _random_ops(rng, 300, max_seqs, nb):
            if op == "alloc":
                try:
                    ref.alloc(s, n)
                    want = None
                except okv.NoBlocks:
                    want = ns.NS_ENOBLOCKS
                except okv.BadShape:
                    want = ns.NS_ESHAPE
                if want is None:
                    ns.ns_kv_alloc(kv, s, n)
                else:
                    with pytest.raises(ns.NSError) as ei:
                        ns.ns_kv_alloc(kv, s, n)
                    assert ei.value.code == want
            else:
                ref.free_seq(s)
                ns.ns_kv_free_seq(kv, s)
            got = ns.ns_kv_block_table(kv, max_seqs, maxb)
            np.testing.assert_array_equal(got, np.array(ref.table_rows(), dtype=np.int32))
            assert ns.ns_kv_num_free(kv) == len(ref.free)
        # slot map over every allocated position, plus padding rows
        tabs = ref.table_rows()
        seq, pos = [], []
        for s in range(max_seqs):
            cap = ns.ns_kv_capacity(kv, s)
            for p in range(cap):
                seq.append(s)
                pos.append(p)
        seq += [-1, -1]
        pos += [0, 5]
        got = ns.ns_slot_map(kv, seq, pos)
        np.testing.assert_array_equal(got, np.array(okv.slot_map(tabs, seq, pos), dtype=np.int32))
    finally:
        ns.ns_kv_destroy(kv)


def test_kv_manager_workload_tables_match_oracle():
    from decode_step_06_amd.configs import WORKLOADS
    from decode_step_06_amd.inputs import gen_batch
    w = WORKLOADS["qwen05b_mix_b64"]
    b = gen_batch(w, with_past=False)
    maxb = 128
    desc = ns.model_desc(w.model)
    kv = ns.ns_kv_create(desc, b.num_blocks, b.n_seqs, maxb, b.free_order)
    ref = okv.BlockAllocator(b.num_blocks, b.free_order, b.n_seqs, maxb)
    try:
        for s, n in enumerate(b.seq_lens):
            ns.ns_kv_alloc(kv, s, int(n))
            ref.alloc(s, int(n))
        np.testing.assert_array_equal(ns.ns_kv_block_table(kv, b.n_seqs, maxb), np.array(ref.table_rows()))
        np.testing.assert_array_equal(ns.ns_slot_map(kv, b.row_seq, b.row_pos),
                                      np.array(okv.slot_map(ref.table_rows(), b.row_seq, b.row_pos)))
    finally:
        ns.ns_kv_destroy(kv)


def test_kv_error_paths_have_no_side_effects():
    desc = ns.model_desc(TINY)
    with pytest.raises(ns.NSError) as ei:
        ns.ns_kv_create(desc, 4, 2, 2, [0, 1, 1, 3])          # not a permutation
    assert ei.value.code == ns.NS_EINVAL
    kv = ns.ns_kv_create(desc, 4, 2, 3, None)
    try:
        ns.ns_kv_alloc(kv, 0, 33)                              # 3 blocks: 0 1 2
        before = ns.ns_kv_block_table(kv, 2, 3).copy()
        for args, code in [((1, 17), ns.NS_ENOBLOCKS), ((1, 49), ns.NS_ESHAPE), ((2, 1), ns.NS_EINVAL),
                           ((-1, 1), ns.NS_EINVAL), ((0, -5), ns.NS_EINVAL)]:
            with pytest.raises(ns.NSError) as ei:
                ns.ns_kv_alloc(kv, *args)
            assert ei.value.code == code
            np.testing.assert_array_equal(ns.ns_kv_block_table(kv, 2, 3), before)
        assert ns.ns_kv_num_free(kv) == 1
        # slot map: validation before any output
        out = np.full(3, 99, dtype=np.int32)
        rc = ns.lib().ns_slot_map(kv, 3, np.array([0, 0, 1], np.int32).ctypes.data_as(ns._PI),
                                  np.array([0, 47, 0], np.int32).ctypes.data_as(ns._PI),
                                  out.ctypes.data_as(ns._PI))
        assert rc == ns.NS_ESHAPE and (out == 99).all()        # seq 1 holds no blocks
        with pytest.raises(ns.NSError) as ei:
            ns.ns_slot_map(kv, [0], [48])
        assert ei.value.code == ns.NS_ESHAPE
        assert "position 48" in str(ei.value)
    finally:
        ns.ns_kv_destroy(kv)


def test_engine_create_rejects_bad_arguments_without_a_gpu():
    desc = ns.model_desc(LLAMA70B)
    kv = ns.ns_kv_create(desc, 8, 2, 4, None)
    try:
        w = ns.ns_weights()
        out = ctypes.c_void_p()
        rc = ns.lib().ns_engine_create(ctypes.byref(desc), ctypes.byref(w), kv, None, 0, None, 0, 16, None,
                                       ctypes.byref(out))
        assert rc == ns.NS_EINVAL
        assert "null" in ns.lib().ns_last_error().decode()
    finally:
        ns.ns_kv_destroy(kv)
    assert ns.lib().ns_engine_destroy(None) == ns.NS_OK   # releasing no engine is a no-op
    # the slab-layout projection checks its arguments before any launch (the
    # pointers below are never dereferenced)
    L, fake = ns.lib(), 4096
    assert L.ns_op_gemm_slab(3, 4, 32, 64, fake, 4, fake, fake, 4, None) == ns.NS_EINVAL      # epilogue
    assert L.ns_op_gemm_slab(ns.NS_EPI_STORE, -1, 32, 64, fake, 4, fake, fake, 4, None) == ns.NS_EINVAL
    assert L.ns_op_gemm_slab(ns.NS_EPI_STORE, 0, 32, 64, None, 0, None, None, 0, None) == ns.NS_OK  # empty
    assert L.ns_op_gemm_slab(ns.NS_EPI_STORE, 4, 32, 64, None, 4, fake, fake, 4, None) == ns.NS_EINVAL
    assert L.ns_op_gemm_slab(ns.NS_EPI_STORE, 4, 32, 48, fake, 4, fake, fake, 4, None) == ns.NS_ESHAPE
    assert L.ns_op_gemm_slab(ns.NS_EPI_STORE, 4, 32, 64, fake, 3, fake, fake, 4, None) == ns.NS_EINVAL  # a_rows
    assert L.ns_op_gemm_slab(ns.NS_EPI_SILU, 4, 48, 64, fake, 4, fake, fake, 4, None) == ns.NS_EINVAL   # N % 32
    assert L.ns_op_gemm_slab(ns.NS_EPI_SILU, 4, 32, 64, fake, 4, fake, fake, 3, None) == ns.NS_EINVAL   # c_rows
    rc = ns.lib().ns_op_gemm(ns.NS_BF16, 0, 4, 4, 30, None, None, None, None)
    assert rc == ns.NS_EINVAL  # null matrices are checked first
    bad = ns.model_desc(TINY)
    bad.n_q_heads, bad.n_kv_heads = 5, 2       # heads do not group evenly
    kvp = ctypes.c_void_p()
    assert ns.lib().ns_kv_create(ctypes.byref(bad), 4, 1, 1, None, ctypes.byref(kvp)) == ns.NS_EINVAL


def test_schedule_options_are_validated_without_a_gpu():
    """ns_sched is checked before anything else of the engine: flags must be
    0 or 1, RoPE fused into attention excludes prefill tiles, and the
    CU-masked second stream is switched off."""
    desc = ns.model_desc(LLAMA70B)
    kv = ns.ns_kv_create(desc, 8, 2, 4, None)
    try:
        w = ns.ns_weights()
        out = ctypes.c_void_p()
        for sched, msg in ((ns.make_sched(fuse_rope_attention=True, prefill_tiles=True), "exclude each other"),
                           (ns.make_sched(overlap=True, cu_mask_frac=0.4), "cu_mask_frac is disabled"),
                           (ns.make_sched(decode_rows_first=True), None),
                           (ns.make_sched(fuse_rope_attention=True), None)):
            rc = ns.lib().ns_engine_create(ctypes.byref(desc), ctypes.byref(w), kv, None, 0, None, 0, 16,
                                           ctypes.byref(sched), ctypes.byref(out))
            assert rc == ns.NS_EINVAL
            err = ns.lib().ns_last_error().decode()
            # a valid schedule gets past the check and fails on the null weights
            assert (msg in err) if msg else ("null" in err)
        bad = ns.make_sched()
        bad.decode_rows_first = 2
        rc = ns.lib().ns_engine_create(ctypes.byref(desc), ctypes.byref(w), kv, None, 0, None, 0, 16,
                                       ctypes.byref(bad), ctypes.byref(out))
        assert rc == ns.NS_EINVAL and "decode_rows_first" in ns.lib().ns_last_error().decode()
    finally:
        ns.ns_kv_destroy(kv)


def test_op_rmsnorm_validates_before_enqueue():
    L = ns.lib()
    assert L.ns_op_rmsnorm(7, 4, 8, None, None, 1e-6, None, None) == ns.NS_EINVAL   # bad dtype
    assert L.ns_op_rmsnorm(ns.NS_BF16, 4, 0, None, None, 1e-6, None, None) == ns.NS_EINVAL  # hidden 0
    assert L.ns_op_rmsnorm(ns.NS_BF16, 4, 8, None, None, -1.0, None, None) == ns.NS_EINVAL  # eps < 0
    assert L.ns_op_rmsnorm(ns.NS_BF16, 4, 8, None, None, 1e-6, None, None) == ns.NS_EINVAL  # null pointers
