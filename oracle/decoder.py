"""Oracle: one batched decode iteration of a pre-norm GQA transformer stack.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy, float64.

What the step computes comes from the pages' description of the decode path:

* page "gpu-waiting-not-working" (nanoserve notes), changes table in section
  "What I changed because of it": RMSNorm at two places per layer, RoPE whose
  cos/sin depend only on the positions (so one table serves every layer),
  grouped-query attention that reads each KV head for its whole group of
  query heads (no expanded K/V copy), and a paged KV cache addressed through
  per-sequence block tables;
* page "NanoFlow: LLM Serving Is Compute Bound, and Your GPU Is Half Idle",
  table in section "Four resource classes, one serialized queue": the dense
  projections KQV, O, Up, Gate, Down, decode attention, and LayerNorm/RoPE;
  section "Nano-batching: manufacturing independence": rows of the dense batch
  are independent, so a split batch computes the same thing.

The pages name these operators but do not define them; the definitions used
are the standard LLaMA / Qwen2 ones (the readings are listed with the design
notes): RMSNorm y = x / sqrt(mean(x^2) + eps) * g; rotate-half RoPE with
inverse frequencies base^(-2j/d); softmax attention with scale 1/sqrt(d) over
the sequence's cached prefix including the current token, query head h reading
KV head h // G; SwiGLU act = silu(gate) * up; pre-norm residual blocks; no
biases; a final RMSNorm and LM head giving float32 logits.

Storage points (``emulate_bf16``): a bf16 model stores these values as bf16
(round to nearest, ties to even), and the oracle rounds at exactly these
points: weights and embedding (already on the grid in the inputs), normalised
activations, rotated q, the K/V written to the cache, the attention output,
and the SwiGLU activation.  The residual stream and the logits stay wide.

Precision (``precision``): "f64" (the default) computes every value in
float64 and is the mode every parity check uses; "f32" is the same code on
float32 arrays (angles still in float64), for timing the oracle as a CPU
baseline only.
"""
from __future__ import annotations

import math

import numpy as np

from .kvcache import BLOCK, slot_of


# ---------------------------------------------------------------- bf16 grid
def round_bf16(a):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bf16 keeps 8 significant bits and float32's exponent range: for |v| in
    [2^e, 2^(e+1)) the spacing is 2^(e-7); below 2^-126 the spacing is fixed at
    2^-133 (subnormals).  Values beyond the largest finite bf16 become inf.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.array(a, copy=True)
    fin = np.isfinite(a) & (a != 0)
    v = a[fin]
    _, e = np.frexp(np.abs(v))          # |v| = m * 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, -126)          # |v| in [2^e, 2^(e+1)), clamped to the normal range
    step = np.ldexp(1.0, e - 7)
    r = np.rint(v / step) * step         # rint: ties to even
    bf16_max = np.ldexp(float(2 ** 8 - 1), 127 - 7)
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def _store(a, emulate, ft=np.float64):
    return (round_bf16(a) if emulate else np.asarray(a, dtype=np.float64)).astype(ft, copy=False)


# ---------------------------------------------------------------- operators
def rmsnorm(x, gain, eps, ft=np.float64):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gain."""
    x = np.asarray(x, dtype=ft)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=ft)


def linear(x, w, ft=np.float64):
    """y = x W^T with W stored row-major as [out, in] (no bias)."""
    return np.asarray(x, dtype=ft) @ np.asarray(w, dtype=ft).T


def rope_angles(pos, head_dim, base):
    """Rotation angles [T, d/2]: pos * base^(-2j/d), j = 0..d/2-1.

    One table per step: the angles depend only on the positions, never on the
    layer (nanoserve notes, changes table, "RoPE cos/sin computed once").
    """
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(base), -2.0 * j / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def apply_rope(x, angles, ft=np.float64):
    """Rotate-half RoPE: the pair (j, j + d/2) of each head turns by angle j.

    x: [T, heads, d]; angles: [T, d/2].
    """
    x = np.asarray(x, dtype=ft)
    half = x.shape[-1] // 2
    c = np.cos(angles).astype(ft)[:, None, :]
    s = np.sin(angles).astype(ft)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def attention_row(q, keys, values, group):
    """Softmax attention of one row's query heads over its context.

    q: [nq, d]; keys, values: [n, nkv, d] (positions 0..n-1 of the sequence).
    Query head h reads KV head h // group.  Returns (o [nq, d], p [nq, n]).
    """
    nq, d = q.shape
    n = keys.shape[0]
    o = np.zeros((nq, d), dtype=q.dtype)
    probs = np.zeros((nq, n), dtype=q.dtype)
    if n == 0:
        return o, probs
    for h in range(nq):
        g = h // group
        scores = keys[:, g, :] @ q[h] / math.sqrt(d)
        w = np.exp(scores - scores.max())
        w = w / w.sum()
        probs[h] = w
        o[h] = w @ values[:, g, :]
    return o, probs


# ---------------------------------------------------------------- KV cache
class OracleKV:
    """Logical paged cache: per layer K, V of shape [num_blocks * 16, nkv, d].

    Slots nobody wrote hold NaN, so reading one shows up in every output it
    touches.
    """

    def __init__(self, n_layers, num_blocks, n_kv, head_dim, block=BLOCK, dtype=np.float64):
        n = num_blocks * block
        self.block = block
        self.k = [np.full((n, n_kv, head_dim), np.nan, dtype=dtype) for _ in range(n_layers)]
        self.v = [np.full((n, n_kv, head_dim), np.nan, dtype=dtype) for _ in range(n_layers)]

    def write(self, layer, slots, k, v):
        """Cache write at each row's slot (slot < 0: padding row, nothing written)."""
        for i, s in enumerate(slots):
            if s >= 0:
                self.k[layer][s] = k[i]
                self.v[layer][s] = v[i]

    def gather(self, layer, table_row, n):
        """Positions 0..n-1 of a sequence, read through its block table."""
        slots = [slot_of(table_row, p, self.block) for p in range(n)]
        return self.k[layer][slots], self.v[layer][slots]


# ---------------------------------------------------------------- the step
class Oracle:
    """Plain decode step.  ``model`` needs the attributes of a model shape
    (n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, rms_eps,
    rope_base, dtype); ``weights`` is the dict of float arrays described in
    the input generator (per-layer attn_norm, wqkv, wo, mlp_norm, wgu, wdown;
    final_norm, embed, lm_head)."""

    def __init__(self, model, weights, emulate_bf16=None, precision="f64"):
        self.m = model
        self.w = weights
        self.emulate = (model.dtype == "bf16") if emulate_bf16 is None else bool(emulate_bf16)
        assert precision in ("f64", "f32")
        self.ft = np.float64 if precision == "f64" else np.float32

    # -- pieces, each one step of the layer --------------------------------
    def embed(self, tokens):
        return np.asarray(self.w["embed"])[np.asarray(tokens)].astype(self.ft)

    def qkv(self, layer, x, pos):
        """Pre-attention half up to the cache write: norm, QKV projection, RoPE."""
        m, lw, ft = self.m, self.w["layers"][layer], self.ft
        nq, nkv, d = m.n_q_heads, m.n_kv_heads, m.head_dim
        h = _store(rmsnorm(x, lw["attn_norm"], m.rms_eps, ft), self.emulate, ft)
        y = linear(h, lw["wqkv"], ft)
        T = x.shape[0]
        q = y[:, : nq * d].reshape(T, nq, d)
        k = y[:, nq * d: (nq + nkv) * d].reshape(T, nkv, d)
        v = y[:, (nq + nkv) * d:].reshape(T, nkv, d)
        ang = rope_angles(pos, d, m.rope_base)
        q = _store(apply_rope(q, ang, ft), self.emulate, ft)
        k = _store(apply_rope(k, ang, ft), self.emulate, ft)
        v = _store(v, self.emulate, ft)
        return q, k, v

    def attend(self, layer, cache, tables, q, row_seq, row_pos):
        m = self.m
        T = q.shape[0]
        o = np.zeros((T, m.n_q_heads, m.head_dim), dtype=self.ft)
        for t in range(T):
            s = int(row_seq[t])
            if s < 0:
                continue
            n = int(row_pos[t]) + 1
            keys, values = cache.gather(layer, tables[s], n)
            o[t], _ = attention_row(q[t], keys, values, m.n_q_heads // m.n_kv_heads)
        return _store(o.reshape(T, -1), self.emulate, self.ft)

    def post_attention(self, layer, x, o):
        """O projection + residual, then the SwiGLU MLP + residual."""
        m, lw, ft = self.m, self.w["layers"][layer], self.ft
        x = x + linear(o, lw["wo"], ft)
        h2 = _store(rmsnorm(x, lw["mlp_norm"], m.rms_eps, ft), self.emulate, ft)
        gu = linear(h2, lw["wgu"], ft)
        F = m.ffn
        act = _store(silu(gu[:, :F]) * gu[:, F:], self.emulate, ft)
        return x + linear(act, lw["wdown"], ft)

    def head(self, x):
        m, ft = self.m, self.ft
        hf = _store(rmsnorm(x, self.w["final_norm"], m.rms_eps, ft), self.emulate, ft)
        return linear(hf, self.w["lm_head"], ft)

    # -- whole step --------------------------------------------------------
    def step(self, cache, tables, row_seq, row_pos, tokens=None, x=None, nano_splits=None):
        """One decode iteration over all rows; returns logits [T, V] (models
        with a vocabulary) or the final hidden state [T, H].

        ``nano_splits``: row counts of nano-batches.  Each layer then runs the
        norm/QKV/RoPE/cache-write part nano-batch by nano-batch (in row order)
        and afterwards attention and the rest nano-batch by nano-batch; rows
        are independent, so the result equals the unsplit step (NanoFlow
        review, "Nano-batching: manufacturing independence").
        """
        m = self.m
        row_seq = np.asarray(row_seq)
        row_pos = np.asarray(row_pos)
        T = row_seq.shape[0]
        if x is None:
            x = self.embed(tokens)
        x = np.array(x, dtype=self.ft)
        bounds = [0]
        for n in (nano_splits or [T]):
            bounds.append(bounds[-1] + int(n))
        assert bounds[-1] == T, "nano splits must cover the batch"
        parts = [slice(bounds[i], bounds[i + 1]) for i in range(len(bounds) - 1)]
        slots = [-1 if s < 0 else slot_of(tables[int(s)], int(p), cache.block)
                 for s, p in zip(row_seq, row_pos)]
        for layer in range(m.n_layers):
            qs = {}
            for r in parts:
                q, k, v = self.qkv(layer, x[r], row_pos[r])
                cache.write(layer, slots[r], k, v)
                qs[r.start] = q
            for r in parts:
                o = self.attend(layer, cache, tables, qs[r.start], row_seq[r], row_pos[r])
                x[r] = self.post_attention(layer, x[r], o)
        if m.vocab:
            return self.head(x)
        return x


def fill_past(cache, tables, past_seq, past_pos, past_k, past_v):
    """Write the already-cached context (positions before this step) into the
    oracle cache through the block tables."""
    slots = [slot_of(tables[int(s)], int(p), cache.block) for s, p in zip(past_seq, past_pos)]
    dt = cache.k[0].dtype if cache.k else np.float64
    for layer in range(len(past_k)):
        cache.write(layer, slots, np.asarray(past_k[layer], dtype=dt), np.asarray(past_v[layer], dtype=dt))
