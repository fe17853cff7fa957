"""Seeded synthetic inputs for the decode step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle take what it
returns, so the two sides see bit-identical inputs.

Recipe (all draws from numpy ``Generator(PCG64(seed))``):

* weights (seed 0): matrices N(0, 0.02); RMSNorm gains 1 + 0.1 N(0, 1) (so a
  dropped gain changes the output by far more than the tolerance); drawn in
  the order layer 0..L-1 (attn_norm, wqkv, wo, mlp_norm, wgu, wdown), then
  final_norm, embedding, LM head.  Rounded to bf16 (round-to-nearest-even)
  for bf16 models, so both sides see the same representable values.
* token ids / hidden input (seed 1): ids uniform in [0, V); hidden rows N(0, 1).
* context lengths (seed 2): uniform over the workload's inclusive range.
* block free order (seed 3): a uniform random permutation of the pool
  ("fragmented" block tables).
* past K/V (seed 4): N(0, 1), bf16-rounded for bf16 models, for positions
  0..ctx-2 of every decode sequence, layer by layer.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .configs import BLOCK_SIZE, ModelShape, Workload

WEIGHT_STD = 0.02
GAIN_STD = 0.1


def _round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even), as float32.

    Input preparation only (the drawn values are put on the storage grid).
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _to_grid(a: np.ndarray, model: ModelShape) -> np.ndarray:
    return _round_bf16(a) if model.dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def weight_names(model: ModelShape):
    """Per-layer weight names and shapes, in draw order."""
    H, F, Dq = model.hidden, model.ffn, model.n_q_heads * model.head_dim
    return [("attn_norm", (H,)), ("wqkv", (model.qkv_dim, H)), ("wo", (H, Dq)),
            ("mlp_norm", (H,)), ("wgu", (2 * F, H)), ("wdown", (H, F))]


def gen_weights(model: ModelShape, seed: int = 0, n_layers: Optional[int] = None) -> dict:
    """All weights as float32 numpy arrays (row-major [out, in] for matrices;
    ``wgu`` is the gate rows stacked over the up rows)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L = model.n_layers if n_layers is None else n_layers

    def mat(shape):
        return _to_grid(rng.standard_normal(shape, dtype=np.float32) * np.float32(WEIGHT_STD), model)

    def gain(shape):
        return _to_grid(np.float32(1.0) + rng.standard_normal(shape, dtype=np.float32)
                        * np.float32(GAIN_STD), model)

    layers = []
    for _ in range(L):
        lw = {}
        for name, shape in weight_names(model):
            lw[name] = gain(shape) if name.endswith("norm") else mat(shape)
        layers.append(lw)
    out = {"layers": layers, "final_norm": None, "embed": None, "lm_head": None}
    if model.vocab:
        out["final_norm"] = gain((model.hidden,))
        out["embed"] = mat((model.vocab, model.hidden))
        out["lm_head"] = out["embed"] if model.tied else mat((model.vocab, model.hidden))
    return out


@dataclass
class Batch:
    """One step's rows, sequences, pool and cached context."""
    seq_lens: np.ndarray      # [S] tokens each sequence holds after this step
    row_seq: np.ndarray       # [T] int32 sequence of each row
    row_pos: np.ndarray       # [T] int32 position of each row
    tokens: Optional[np.ndarray]  # [T] int32 token ids (models with a vocabulary)
    x: Optional[np.ndarray]       # [T, H] float32 hidden input (models without one)
    num_blocks: int
    free_order: np.ndarray    # [NB] int32 initial free-list order
    past_seq: np.ndarray      # [P] int32 sequence of each cached (past) position
    past_pos: np.ndarray      # [P] int32 position of each cached (past) position
    past_k: List[np.ndarray]  # per layer [P, n_kv, d] float32
    past_v: List[np.ndarray]

    @property
    def n_rows(self) -> int:
        return int(self.row_seq.shape[0])

    @property
    def n_seqs(self) -> int:
        return int(self.seq_lens.shape[0])


def blocks_needed(n_tokens: int) -> int:
    return -(-int(n_tokens) // BLOCK_SIZE)


def gen_batch(w: Workload, n_layers: Optional[int] = None, with_past: bool = True,
              pool_slack: float = 1.25) -> Batch:
    model = w.model
    L = model.n_layers if n_layers is None else n_layers
    s = w.seeds
    if w.ctx_range is not None:
        lo, hi = w.ctx_range
        ctx = np.random.Generator(np.random.PCG64(s["ctx"])).integers(lo, hi + 1, size=w.n_decode)
    else:
        ctx = np.full(w.n_decode, int(w.decode_ctx), dtype=np.int64)
    seq_lens = np.concatenate([ctx, np.array(w.prefill_chunks, dtype=np.int64)]).astype(np.int32)
    row_seq, row_pos = [], []
    for i in range(w.n_decode):
        row_seq.append(i)
        row_pos.append(int(ctx[i]) - 1)
    for c, n in enumerate(w.prefill_chunks):
        for p in range(n):
            row_seq.append(w.n_decode + c)
            row_pos.append(p)
    row_seq = np.array(row_seq, dtype=np.int32)
    row_pos = np.array(row_pos, dtype=np.int32)

    need = sum(blocks_needed(n) for n in seq_lens)
    nb = w.num_blocks if w.num_blocks is not None else max(need, int(np.ceil(need * pool_slack)) + 1)
    if w.shuffle_blocks:
        free_order = np.random.Generator(np.random.PCG64(s["perm"])).permutation(nb).astype(np.int32)
    else:
        free_order = np.arange(nb, dtype=np.int32)

    rng_x = np.random.Generator(np.random.PCG64(s["x"]))
    T = row_seq.shape[0]
    tokens = x = None
    if model.vocab:
        tokens = rng_x.integers(0, model.vocab, size=T).astype(np.int32)
    else:
        x = rng_x.standard_normal((T, model.hidden), dtype=np.float32)

    past_seq = np.concatenate([np.full(int(c) - 1, i, dtype=np.int32) for i, c in enumerate(ctx)]) \
        if w.n_decode else np.zeros(0, np.int32)
    past_pos = np.concatenate([np.arange(int(c) - 1, dtype=np.int32) for c in ctx]) \
        if w.n_decode else np.zeros(0, np.int32)
    past_k, past_v = [], []
    if with_past:
        rng_kv = np.random.Generator(np.random.PCG64(s["kv"]))
        shape = (past_seq.shape[0], model.n_kv_heads, model.head_dim)
        for _ in range(L):
            past_k.append(_to_grid(rng_kv.standard_normal(shape, dtype=np.float32), model))
            past_v.append(_to_grid(rng_kv.standard_normal(shape, dtype=np.float32), model))
    return Batch(seq_lens, row_seq, row_pos, tokens, x, nb, free_order, past_seq, past_pos,
                 past_k, past_v)
