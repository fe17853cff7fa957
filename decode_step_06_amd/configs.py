"""Model shapes and workloads of the batched GQA decode step.

Pure data: sizes, counts and seeds, no arithmetic of the method.  Every
workload is synthetic and seeded; the shapes follow the pages' workloads:

* ``tiny``: a single fp32 decoder layer (hidden 128, 4 query / 1 KV head,
  head_dim 32, SwiGLU 256), used to check every step at a size the oracle
  runs in milliseconds.
* ``qwen05b``: the Qwen2.5-0.5B shape that the page "gpu-waiting-not-working"
  (nanoserve notes, section "The number that didn't fit") profiles: 24 layers,
  hidden 896, 14 query / 2 KV heads (the 7x grouping of its changes table),
  head_dim 64, FFN 4864, vocabulary 151936 with the LM head tied to the
  embedding (its 943 MiB of fp16 weights only add up with a tied head).
* ``llama70b``: the LLaMA-2-70B shape that the page "NanoFlow: LLM Serving Is
  Compute Bound, and Your GPU Is Half Idle" costs out (hidden 8192, 64 query /
  8 KV heads, head_dim 128, FFN 28672, 80 layers, vocabulary 32000, untied).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

BLOCK_SIZE = 16  # KV slots per cache block


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int            # 0: no embedding / LM head (hidden state in, hidden state out)
    tied: bool            # LM head shares the embedding matrix
    dtype: str            # "f32" or "bf16": storage type of weights and activations
    rms_eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


TINY = ModelShape("tiny", 1, 128, 4, 1, 32, 256, 0, False, "f32")
QWEN05B = ModelShape("qwen05b", 24, 896, 14, 2, 64, 4864, 151936, True, "bf16")
LLAMA70B_LAYER = ModelShape("llama70b_layer", 1, 8192, 64, 8, 128, 28672, 0, False, "bf16")
LLAMA70B = ModelShape("llama70b", 80, 8192, 64, 8, 128, 28672, 32000, False, "bf16")


@dataclass(frozen=True)
class Workload:
    """One batch of rows for one step.

    ``decode_ctx``: context lengths of the decode sequences (each decodes one
    token at position ctx-1; the earlier ctx-1 positions are already cached).
    ``ctx_range``: when set, decode context lengths are drawn uniformly from
    this inclusive range instead.
    ``prefill_chunks``: fresh sequences whose first ``n`` tokens are all in
    this step (positions 0..n-1), placed after the decode rows.
    """
    name: str
    model: ModelShape
    n_decode: int
    decode_ctx: Optional[int] = None
    ctx_range: Optional[Tuple[int, int]] = None
    prefill_chunks: Tuple[int, ...] = ()
    num_blocks: Optional[int] = None   # pool size; None: exactly what the batch needs plus slack
    shuffle_blocks: bool = True        # free list in a seeded random order (fragmented tables)
    nano_splits: Tuple[int, ...] = ()  # row counts of the nano-batches (empty: one batch)
    qkv_splits: int = 1                # nano-ops at the QKV projection
    seeds: dict = field(default_factory=lambda: dict(weights=0, x=1, ctx=2, perm=3, kv=4))

    @property
    def n_rows(self) -> int:
        return self.n_decode + sum(self.prefill_chunks)


WORKLOADS = {
    "tiny_b4": Workload("tiny_b4", TINY, 4, ctx_range=(5, 40), num_blocks=16),
    "qwen05b_b1_ctx512": Workload("qwen05b_b1_ctx512", QWEN05B, 1, decode_ctx=512),
    "qwen05b_b32_ctx512": Workload("qwen05b_b32_ctx512", QWEN05B, 32, decode_ctx=512,
                                   nano_splits=(16, 16)),
    "llama70b_layer_t2048": Workload("llama70b_layer_t2048", LLAMA70B_LAYER, 512, decode_ctx=1024,
                                     prefill_chunks=(512, 512, 512), nano_splits=(768, 1280),
                                     qkv_splits=4),
    "llama70b_80l_b256": Workload("llama70b_80l_b256", LLAMA70B, 256, ctx_range=(512, 1536),
                                  nano_splits=(128, 128)),
}
for _b in (1, 8, 32, 64, 128, 256):
    WORKLOADS[f"qwen05b_mix_b{_b}"] = Workload(f"qwen05b_mix_b{_b}", QWEN05B, _b,
                                               ctx_range=(128, 2048))


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return replace(w, **kw)
