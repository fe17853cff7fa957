"""ctypes binding of the C ABI in ``include/ns.h`` (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of the decode step: all device work runs in the HIP library.  The
library must have been built (``python -m decode_step_06_amd.build``); if it
is missing, loading raises instead of falling back to anything else.
Non-zero status codes raise ``NSError`` carrying ``ns_last_error()``.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libns.so")

NS_OK, NS_EINVAL, NS_ENOBLOCKS, NS_ESHAPE, NS_ESTATE, NS_EHIP = 0, -1, -2, -3, -4, -5
NS_F32, NS_BF16 = 0, 1
NS_EPI_STORE, NS_EPI_RESID, NS_EPI_SILU = 0, 1, 2
BLOCK_SIZE = 16

STATUS_NAMES = {0: "NS_OK", -1: "NS_EINVAL", -2: "NS_ENOBLOCKS", -3: "NS_ESHAPE", -4: "NS_ESTATE", -5: "NS_EHIP"}


class NSError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


class ns_model_desc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("tied", C.c_int32), ("rms_eps", C.c_float),
                ("rope_base", C.c_float), ("dtype", C.c_int32)]


class ns_weights(C.Structure):
    _fields_ = [("attn_norm", C.POINTER(C.c_void_p)), ("wqkv", C.POINTER(C.c_void_p)),
                ("wo", C.POINTER(C.c_void_p)), ("mlp_norm", C.POINTER(C.c_void_p)),
                ("wgu", C.POINTER(C.c_void_p)), ("wdown", C.POINTER(C.c_void_p)),
                ("final_norm", C.c_void_p), ("embed", C.c_void_p), ("lm_head", C.c_void_p)]


class ns_sched(C.Structure):
    _fields_ = [("n_nano", C.c_int32), ("nano_rows", C.c_int32 * 4), ("n_qkv", C.c_int32),
                ("qkv_rows", C.c_int32 * 4), ("overlap", C.c_int32), ("attn_wg_cap", C.c_int32),
                ("cu_mask_frac", C.c_float), ("prefill_tiles", C.c_int32),
                ("decode_rows_first", C.c_int32), ("fuse_rope_attention", C.c_int32)]


class ns_batch(C.Structure):
    _fields_ = [("n_tok", C.c_int32), ("token_ids", C.POINTER(C.c_int32)), ("hidden_in", C.c_void_p),
                ("seq", C.POINTER(C.c_int32)), ("pos", C.POINTER(C.c_int32)), ("token_ids_dev", C.c_void_p)]


_P = C.c_void_p
_I = C.c_int32
_PI = C.POINTER(C.c_int32)
# name -> (restype, argtypes); exactly the entry points of include/ns.h
SIGNATURES = {
    "ns_last_error": (C.c_char_p, []),
    "ns_kv_bytes": (C.c_size_t, [C.POINTER(ns_model_desc), _I]),
    "ns_kv_create": (C.c_int, [C.POINTER(ns_model_desc), _I, _I, _I, _PI, C.POINTER(_P)]),
    "ns_kv_alloc": (C.c_int, [_P, _I, _I]),
    "ns_kv_free_seq": (C.c_int, [_P, _I]),
    "ns_kv_block_table": (C.c_int, [_P, _PI]),
    "ns_kv_capacity": (C.c_int, [_P, _I, _PI]),
    "ns_kv_num_free": (C.c_int, [_P, _PI]),
    "ns_kv_destroy": (None, [_P]),
    "ns_slot_map": (C.c_int, [_P, _I, _PI, _PI, _PI]),
    "ns_workspace_bytes": (C.c_size_t, [C.POINTER(ns_model_desc), _I, _I]),
    "ns_engine_create": (C.c_int, [C.POINTER(ns_model_desc), C.POINTER(ns_weights), _P, _P, C.c_size_t, _P,
                                   C.c_size_t, _I, C.POINTER(ns_sched), C.POINTER(_P)]),
    "ns_engine_destroy": (C.c_int, [_P]),
    "ns_engine_set_sched": (C.c_int, [_P, C.POINTER(ns_sched)]),
    "ns_decode_step": (C.c_int, [_P, C.POINTER(ns_batch), _P, _P]),
    "ns_graph_capture": (C.c_int, [_P, _I, _P, _P, C.POINTER(_P)]),
    "ns_graph_replay": (C.c_int, [_P, C.POINTER(ns_batch), _P]),
    "ns_graph_destroy": (None, [_P]),
    "ns_sample_greedy": (C.c_int, [_P, _I, _I, _P, _P]),
    "ns_read_stream": (C.c_int, [_P, C.c_size_t, _P, C.c_size_t, _P]),
    "ns_graph_set_capture": (C.c_int, [_P, _PI, _I, _P, _P, C.POINTER(_P)]),
    "ns_graph_set_replay": (C.c_int, [_P, C.POINTER(ns_batch), _P, _PI]),
    "ns_graph_set_destroy": (None, [_P]),
    "ns_kv_scatter": (C.c_int, [_P, _I, _I, _P, _P, _P, _P]),
    "ns_kv_gather": (C.c_int, [_P, _I, _I, _P, _P, _P, _P]),
    "ns_engine_last_launches": (C.c_int, [_P, _PI]),
    "ns_engine_profile": (C.c_int, [_P, _I]),
    "ns_engine_profile_read": (C.c_int, [_P, _I, _PI, C.POINTER(C.c_float), _PI]),
    "ns_op_gemm": (C.c_int, [_I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "ns_op_gemm_packed": (C.c_int, [_I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "ns_op_gemm_slab": (C.c_int, [_I, _I, _I, _I, _P, _I, _P, _P, _I, _P]),
    "ns_pack_weight": (C.c_int, [_P, _P, _I, _I, _P]),
    "ns_op_rmsnorm": (C.c_int, [_I, _I, _I, _P, _P, C.c_float, _P, _P]),
    "ns_op_attention_ws_bytes": (C.c_size_t, [C.POINTER(ns_model_desc), _I, _I]),
    "ns_op_attention": (C.c_int, [C.POINTER(ns_model_desc), _I, _P, _P, _I, _P, _P, _P, _I, _P, _P, C.c_size_t,
                                  _I, _P]),
    "ns_op_attention_prefill": (C.c_int, [C.POINTER(ns_model_desc), _I, _P, _P, _I, _P, _P, _P, _I, _P, _P,
                                          C.c_size_t, _I, _P]),
    "ns_op_attention_static": (C.c_int, [C.POINTER(ns_model_desc), _I, _P, _P, _I, _P, _P, _P, _I, _P, _I, _P]),
}

_LIB: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """Load the built HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decode_step_06_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(rc: int) -> None:
    if rc != NS_OK:
        raise NSError(rc, lib().ns_last_error().decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_PI)


def model_desc(shape) -> ns_model_desc:
    """Descriptor from a model shape (configs.ModelShape)."""
    return ns_model_desc(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                         shape.ffn, shape.vocab, int(shape.tied), shape.rms_eps, shape.rope_base,
                         NS_BF16 if shape.dtype == "bf16" else NS_F32)


def make_sched(nano_rows: Sequence[int] = (), qkv_rows: Sequence[int] = (), overlap: bool = False,
               attn_wg_cap: int = 0, cu_mask_frac: float = 0.0, prefill_tiles: bool = False,
               decode_rows_first: bool = False, fuse_rope_attention: bool = False) -> ns_sched:
    s = ns_sched()
    s.n_nano = len(nano_rows)
    for i, r in enumerate(nano_rows):
        s.nano_rows[i] = int(r)
    s.n_qkv = len(qkv_rows)
    for i, r in enumerate(qkv_rows):
        s.qkv_rows[i] = int(r)
    s.overlap = int(bool(overlap))
    s.attn_wg_cap = int(attn_wg_cap)
    s.cu_mask_frac = float(cu_mask_frac)
    s.prefill_tiles = int(bool(prefill_tiles))
    s.decode_rows_first = int(bool(decode_rows_first))
    s.fuse_rope_attention = int(bool(fuse_rope_attention))
    return s


# ---------------------------------------------------------------- KV manager
def ns_kv_bytes(desc: ns_model_desc, num_blocks: int) -> int:
    return int(lib().ns_kv_bytes(C.byref(desc), num_blocks))


def ns_kv_create(desc: ns_model_desc, num_blocks: int, max_seqs: int, max_blocks_per_seq: int,
                 free_order=None) -> C.c_void_p:
    out = C.c_void_p()
    fo = None if free_order is None else _i32(free_order)
    _check(lib().ns_kv_create(C.byref(desc), num_blocks, max_seqs, max_blocks_per_seq,
                              None if fo is None else _ptr(fo), C.byref(out)))
    return out


def ns_kv_alloc(kv, seq: int, n_tokens: int) -> None:
    _check(lib().ns_kv_alloc(kv, seq, n_tokens))


def ns_kv_free_seq(kv, seq: int) -> None:
    _check(lib().ns_kv_free_seq(kv, seq))


def ns_kv_block_table(kv, max_seqs: int, max_blocks_per_seq: int) -> np.ndarray:
    out = np.empty((max_seqs, max_blocks_per_seq), dtype=np.int32)
    _check(lib().ns_kv_block_table(kv, _ptr(out)))
    return out


def ns_kv_capacity(kv, seq: int) -> int:
    v = C.c_int32()
    _check(lib().ns_kv_capacity(kv, seq, C.byref(v)))
    return v.value


def ns_kv_num_free(kv) -> int:
    v = C.c_int32()
    _check(lib().ns_kv_num_free(kv, C.byref(v)))
    return v.value


def ns_kv_destroy(kv) -> None:
    lib().ns_kv_destroy(kv)


def ns_slot_map(kv, seq, pos) -> np.ndarray:
    s, p = _i32(seq), _i32(pos)
    out = np.full(s.shape[0], -7, dtype=np.int32)
    _check(lib().ns_slot_map(kv, s.shape[0], _ptr(s), _ptr(p), _ptr(out)))
    return out


# ---------------------------------------------------------------- engine
def ns_workspace_bytes(desc: ns_model_desc, max_tokens: int, max_blocks_per_seq: int) -> int:
    return int(lib().ns_workspace_bytes(C.byref(desc), max_tokens, max_blocks_per_seq))


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


class Batch:
    """Host arrays of one step kept alive for the duration of a call."""

    def __init__(self, seq, pos, tokens=None, hidden_in=None, tokens_dev=None):
        self.seq = _i32(seq)
        self.pos = _i32(pos)
        self.tokens = None if tokens is None else _i32(tokens)
        self.hidden_in = hidden_in  # device tensor (fp32 [n, H]) or None
        self.tokens_dev = tokens_dev  # device int32 tensor [n] (on-device token feedback) or None
        self.c = ns_batch(self.seq.shape[0], None if self.tokens is None else _ptr(self.tokens),
                          None if hidden_in is None else hidden_in.data_ptr(), _ptr(self.seq), _ptr(self.pos),
                          None if tokens_dev is None else tokens_dev.data_ptr())


def ns_engine_create(desc, weights: ns_weights, kv, kv_dev: int, kv_bytes: int, ws_dev: int, ws_bytes: int,
                     max_tokens: int, sched: Optional[ns_sched] = None) -> C.c_void_p:
    out = C.c_void_p()
    _check(lib().ns_engine_create(C.byref(desc), C.byref(weights), kv, kv_dev, kv_bytes, ws_dev, ws_bytes,
                                  max_tokens, None if sched is None else C.byref(sched), C.byref(out)))
    return out


def ns_engine_destroy(eng) -> None:
    _check(lib().ns_engine_destroy(eng))


def ns_engine_set_sched(eng, sched: ns_sched) -> None:
    _check(lib().ns_engine_set_sched(eng, C.byref(sched)))


def ns_decode_step(eng, batch: Batch, out_dev: int, stream=None) -> None:
    _check(lib().ns_decode_step(eng, C.byref(batch.c), out_dev, _stream_ptr(stream)))


def ns_graph_set_capture(eng, buckets, out_dev: int, stream) -> C.c_void_p:
    b = _i32(buckets)
    gs = C.c_void_p()
    _check(lib().ns_graph_set_capture(eng, _ptr(b), len(b), out_dev, _stream_ptr(stream), C.byref(gs)))
    return gs


def ns_graph_set_replay(gs, batch: Batch, stream) -> int:
    used = C.c_int32(0)
    _check(lib().ns_graph_set_replay(gs, C.byref(batch.c), _stream_ptr(stream), C.byref(used)))
    return used.value


def ns_graph_set_destroy(gs) -> None:
    lib().ns_graph_set_destroy(gs)


def ns_sample_greedy(logits_dev: int, n_rows: int, vocab: int, tokens_dev: int, stream=None) -> None:
    _check(lib().ns_sample_greedy(logits_dev, n_rows, vocab, tokens_dev, _stream_ptr(stream)))


NS_READ_STREAM_WORDS = 2048


def ns_read_stream(src_dev: int, nbytes: int, sink_dev: int, sink_words: int, stream=None) -> None:
    _check(lib().ns_read_stream(src_dev, nbytes, sink_dev, sink_words, _stream_ptr(stream)))


def ns_graph_capture(eng, bucket: int, out_dev: int, stream) -> C.c_void_p:
    g = C.c_void_p()
    _check(lib().ns_graph_capture(eng, bucket, out_dev, _stream_ptr(stream), C.byref(g)))
    return g


def ns_graph_replay(graph, batch: Batch, stream) -> None:
    _check(lib().ns_graph_replay(graph, C.byref(batch.c), _stream_ptr(stream)))


def ns_graph_destroy(graph) -> None:
    lib().ns_graph_destroy(graph)


def ns_kv_scatter(eng, layer: int, n: int, slots_dev: int, k_dev: int, v_dev: int, stream=None) -> None:
    _check(lib().ns_kv_scatter(eng, layer, n, slots_dev, k_dev, v_dev, _stream_ptr(stream)))


def ns_kv_gather(eng, layer: int, n: int, slots_dev: int, k_dev: int, v_dev: int, stream=None) -> None:
    _check(lib().ns_kv_gather(eng, layer, n, slots_dev, k_dev, v_dev, _stream_ptr(stream)))


def ns_engine_last_launches(eng) -> int:
    v = C.c_int32()
    _check(lib().ns_engine_last_launches(eng, C.byref(v)))
    return v.value


KERNEL_CLASSES = ["embed", "rope_table", "rmsnorm", "qkv_proj", "rope_kv_write", "attention", "o_proj",
                  "gate_up_proj", "down_proj", "lm_head", "copy_out"]


def ns_engine_profile(eng, enable: bool) -> None:
    _check(lib().ns_engine_profile(eng, int(bool(enable))))


def ns_engine_profile_read(eng, cap: int = 8192):
    kinds = np.zeros(cap, dtype=np.int32)
    us = np.zeros(cap, dtype=np.float32)
    n = C.c_int32()
    _check(lib().ns_engine_profile_read(eng, cap, _ptr(kinds), us.ctypes.data_as(C.POINTER(C.c_float)),
                                        C.byref(n)))
    m = min(n.value, cap)
    return [KERNEL_CLASSES[k] for k in kinds[:m]], us[:m].astype(np.float64)


# ---------------------------------------------------------------- single kernels
def ns_op_gemm(dtype: int, epi: int, M: int, N: int, K: int, A: int, B: int, Cp: int, stream=None) -> None:
    _check(lib().ns_op_gemm(dtype, epi, M, N, K, A, B, Cp, _stream_ptr(stream)))


def ns_op_gemm_packed(dtype: int, epi: int, M: int, N: int, K: int, A: int, B: int, Cp: int, stream=None) -> None:
    _check(lib().ns_op_gemm_packed(dtype, epi, M, N, K, A, B, Cp, _stream_ptr(stream)))


def ns_op_gemm_slab(epi: int, M: int, N: int, K: int, A: int, a_rows: int, B: int, Cp: int, c_rows: int,
                    stream=None) -> None:
    _check(lib().ns_op_gemm_slab(epi, M, N, K, A, a_rows, B, Cp, c_rows, _stream_ptr(stream)))


def ns_op_rmsnorm(dtype: int, n_rows: int, hidden: int, x: int, gain: int, eps: float, out: int, stream=None) -> None:
    _check(lib().ns_op_rmsnorm(dtype, n_rows, hidden, x, gain, eps, out, _stream_ptr(stream)))


def ns_pack_weight(src: int, dst: int, rows: int, cols: int, stream=None) -> None:
    _check(lib().ns_pack_weight(src, dst, rows, cols, _stream_ptr(stream)))


def ns_op_attention_ws_bytes(desc, n_rows: int, max_blocks_per_seq: int) -> int:
    return int(lib().ns_op_attention_ws_bytes(C.byref(desc), n_rows, max_blocks_per_seq))


def ns_op_attention(desc, n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab, max_blocks_per_seq, out,
                    ws, ws_bytes, wg_cap=0, stream=None) -> None:
    _check(lib().ns_op_attention(C.byref(desc), n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab,
                                 max_blocks_per_seq, out, ws, ws_bytes, wg_cap, _stream_ptr(stream)))


def ns_op_attention_prefill(desc, n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab, max_blocks_per_seq,
                            out, ws, ws_bytes, wg_cap=0, stream=None) -> None:
    _check(lib().ns_op_attention_prefill(C.byref(desc), n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab,
                                         max_blocks_per_seq, out, ws, ws_bytes, wg_cap, _stream_ptr(stream)))


NS_ATTENTION_STATIC_SCRATCH_BYTES = 5 << 20  # include/ns.h


def ns_op_attention_static(desc, n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab, max_blocks_per_seq,
                           out, wg_cap=0, stream=None) -> None:
    _check(lib().ns_op_attention_static(C.byref(desc), n_rows, q_att, kv_layer, num_blocks, row_bseq, row_pos, btab,
                                        max_blocks_per_seq, out, wg_cap, _stream_ptr(stream)))
