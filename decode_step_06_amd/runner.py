"""Device-side setup around the C ABI: weight upload, KV memory, engine.

Marshalling only -- torch supplies device memory and streams, the HIP
library does every step of the decode path.  Used by the tests and the
benchmark.  Unused KV memory is filled with NaN so that a read of a slot
nobody wrote poisons every output it touches.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import ns
from .configs import BLOCK_SIZE, ModelShape


def torch_dtype(shape: ModelShape):
    return torch.bfloat16 if shape.dtype == "bf16" else torch.float32


def nan_fill_(buf: torch.Tensor, shape: ModelShape) -> None:
    """Fill a raw uint8 buffer with quiet NaNs of the model's element type."""
    if shape.dtype == "bf16":
        buf.view(torch.int16).fill_(0x7FC0)
    else:
        buf.view(torch.int32).fill_(0x7FC00000)


PACKED = ("wqkv", "wo", "wgu", "wdown")  # K-slab-major in bf16 models (see ns_weights)


def pack_kslab_host(w: np.ndarray) -> np.ndarray:
    """Row-major [R, K] -> the K-slab-major layout (same bytes, reordered)."""
    R, K = w.shape
    return np.ascontiguousarray(w.reshape(R, K // 32, 32).transpose(1, 0, 2)).reshape(R, K)


def unpack_kslab(t: torch.Tensor, R: int, K: int) -> torch.Tensor:
    """K-slab-major device tensor -> row-major [R, K] (a copy)."""
    return t.reshape(K // 32, R, 32).permute(1, 0, 2).reshape(R, K).contiguous()


class DeviceWeights:
    """Weights as device tensors plus the ns_weights struct pointing at them.
    In bf16 models the projection matrices are held K-slab-major, as the
    engine reads them."""

    def __init__(self, shape: ModelShape, tensors: dict):
        self.shape = shape
        self.t = tensors
        L = shape.n_layers

        def arr(name):
            return (C_void_p_array(L))(*[tensors["layers"][l][name].data_ptr() for l in range(L)])

        self._arrays = {n: arr(n) for n in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wdown")}
        a = self._arrays
        self.c = ns.ns_weights(a["attn_norm"], a["wqkv"], a["wo"], a["mlp_norm"], a["wgu"], a["wdown"],
                               tensors["final_norm"].data_ptr() if tensors["final_norm"] is not None else None,
                               tensors["embed"].data_ptr() if tensors["embed"] is not None else None,
                               tensors["lm_head"].data_ptr() if tensors["lm_head"] is not None else None)

    @classmethod
    def from_numpy(cls, shape: ModelShape, w: dict, device="cuda"):
        dt = torch_dtype(shape)

        def up(a):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)

        pk = shape.dtype == "bf16"
        layers = [{k: up(pack_kslab_host(v) if (pk and k in PACKED) else v) for k, v in lw.items()}
                  for lw in w["layers"]]
        emb = up(w["embed"])
        lm_src = w["embed"] if shape.tied else w["lm_head"]
        if lm_src is None:
            lm = None
        elif pk:  # K-slab-major (a tied model's head is a packed copy of the embedding)
            lm = up(pack_kslab_host(lm_src))
        else:
            lm = emb if shape.tied else up(lm_src)
        return cls(shape, {"layers": layers, "final_norm": up(w["final_norm"]), "embed": emb, "lm_head": lm})

    @classmethod
    def random_on_device(cls, shape: ModelShape, seed: int = 0, device="cuda"):
        """Same distributions as the seeded host generator, drawn on the device
        with torch's generator (for shapes too large to draw on the host)."""
        from .inputs import GAIN_STD, WEIGHT_STD, weight_names
        dt = torch_dtype(shape)
        g = torch.Generator(device=device)
        g.manual_seed(seed)

        def mat(shp):
            return (torch.randn(shp, generator=g, device=device, dtype=torch.float32) * WEIGHT_STD).to(dt)

        def gain(shp):
            return (1.0 + torch.randn(shp, generator=g, device=device, dtype=torch.float32) * GAIN_STD).to(dt)

        def packed(shp):  # drawn row-major, stored K-slab-major
            a = mat(shp)
            if shape.dtype != "bf16":
                return a
            out = torch.empty_like(a)
            ns.ns_pack_weight(a.data_ptr(), out.data_ptr(), shp[0], shp[1])
            torch.cuda.synchronize()
            return out

        layers = []
        for _ in range(shape.n_layers):
            layers.append({n: (gain(s) if n.endswith("norm") else packed(s) if n in PACKED else mat(s))
                           for n, s in weight_names(shape)})
        fn = emb = lm = None
        if shape.vocab:
            fn = gain((shape.hidden,))
            emb = mat((shape.vocab, shape.hidden))
            if shape.dtype != "bf16":
                lm = emb if shape.tied else mat((shape.vocab, shape.hidden))
            elif shape.tied:  # a packed copy of the embedding
                lm = torch.empty_like(emb)
                ns.ns_pack_weight(emb.data_ptr(), lm.data_ptr(), shape.vocab, shape.hidden)
                torch.cuda.synchronize()
            else:
                lm = packed((shape.vocab, shape.hidden))
        return cls(shape, {"layers": layers, "final_norm": fn, "embed": emb, "lm_head": lm})

    def logical_layer(self, l: int) -> dict:
        """Layer l's weights as row-major device tensors (copies)."""
        from .inputs import weight_names
        shapes = dict(weight_names(self.shape))
        out = {}
        for k, v in self.t["layers"][l].items():
            if k in PACKED and self.shape.dtype == "bf16":
                out[k] = unpack_kslab(v, *shapes[k])
            else:
                out[k] = v
        return out

    def logical_lm_head(self) -> torch.Tensor:
        """The LM head as a row-major [V, H] device tensor."""
        lm = self.t["lm_head"]
        if self.shape.dtype == "bf16":
            return unpack_kslab(lm, self.shape.vocab, self.shape.hidden)
        return lm

    def bytes(self) -> int:
        seen, total = set(), 0
        for lw in self.t["layers"]:
            for v in lw.values():
                total += v.numel() * v.element_size()
        for k in ("final_norm", "embed", "lm_head"):
            v = self.t[k]
            if v is not None and v.data_ptr() not in seen:
                seen.add(v.data_ptr())
                total += v.numel() * v.element_size()
        return total


def C_void_p_array(n):
    import ctypes
    return ctypes.c_void_p * n


@dataclass
class EngineHandle:
    shape: ModelShape
    desc: ns.ns_model_desc
    kv: object
    eng: object
    weights: DeviceWeights
    kv_mem: torch.Tensor
    ws: torch.Tensor
    num_blocks: int
    max_seqs: int
    max_blocks: int
    max_tokens: int

    def destroy(self):
        if self.eng:
            ns.ns_engine_destroy(self.eng)
            self.eng = None
        if self.kv:
            ns.ns_kv_destroy(self.kv)
            self.kv = None


def create_engine(shape: ModelShape, weights: DeviceWeights, num_blocks: int, max_seqs: int, max_blocks: int,
                  max_tokens: int, free_order=None, sched: Optional[ns.ns_sched] = None, device="cuda",
                  nan_poison: bool = True) -> EngineHandle:
    desc = ns.model_desc(shape)
    kv = ns.ns_kv_create(desc, num_blocks, max_seqs, max_blocks, free_order)
    kv_bytes = ns.ns_kv_bytes(desc, num_blocks)
    kv_mem = torch.empty(kv_bytes, dtype=torch.uint8, device=device)
    if nan_poison:
        nan_fill_(kv_mem, shape)
    ws_bytes = ns.ns_workspace_bytes(desc, max_tokens, max_blocks)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    eng = ns.ns_engine_create(desc, weights.c, kv, kv_mem.data_ptr(), kv_bytes, ws.data_ptr(), ws_bytes,
                              max_tokens, sched)
    return EngineHandle(shape, desc, kv, eng, weights, kv_mem, ws, num_blocks, max_seqs, max_blocks, max_tokens)


def fill_past(h: EngineHandle, past_seq, past_pos, past_k: List, past_v: List, device="cuda") -> None:
    """Write already-cached context (host arrays, logical [n, nkv, d] per
    layer) into the device cache through the engine's scatter entry point."""
    n = int(len(past_seq))
    if n == 0:
        return
    slots = ns.ns_slot_map(h.kv, past_seq, past_pos)
    slots_d = torch.from_numpy(slots).to(device)
    dt = torch_dtype(h.shape)
    for layer in range(len(past_k)):
        k = torch.from_numpy(np.ascontiguousarray(past_k[layer])).to(device=device, dtype=dt)
        v = torch.from_numpy(np.ascontiguousarray(past_v[layer])).to(device=device, dtype=dt)
        ns.ns_kv_scatter(h.eng, layer, n, slots_d.data_ptr(), k.data_ptr(), v.data_ptr())
    torch.cuda.synchronize()


def fill_past_random_on_device(h: EngineHandle, past_seq, past_pos, seed: int = 4, device="cuda",
                               chunk: int = 1 << 16, keep=None):
    """Past K/V ~ N(0, 1) drawn on the device (large workloads), scattered
    layer by layer in chunks of positions.

    ``keep``: optional boolean mask over the past positions; the drawn values
    (on the model's storage grid) of the kept positions are copied back as
    float32 host arrays and returned as (k_layers, v_layers), so a checker can
    rebuild the same context for a sample of sequences without reading the
    cache back through the library."""
    n = int(len(past_seq))
    s = h.shape
    kept_k = [[] for _ in range(s.n_layers)]
    kept_v = [[] for _ in range(s.n_layers)]
    if n == 0:
        return (kept_k, kept_v) if keep is not None else None
    slots = torch.from_numpy(ns.ns_slot_map(h.kv, past_seq, past_pos)).to(device)
    dt = torch_dtype(h.shape)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    keep_t = torch.from_numpy(np.asarray(keep, dtype=bool)).to(device) if keep is not None else None
    for layer in range(s.n_layers):
        for c0 in range(0, n, chunk):
            m = min(chunk, n - c0)
            k = torch.randn((m, s.n_kv_heads, s.head_dim), generator=g, device=device).to(dt)
            v = torch.randn((m, s.n_kv_heads, s.head_dim), generator=g, device=device).to(dt)
            ns.ns_kv_scatter(h.eng, layer, m, slots[c0:].data_ptr(), k.data_ptr(), v.data_ptr())
            if keep_t is not None:
                sel = keep_t[c0:c0 + m]
                kept_k[layer].append(k[sel].float().cpu().numpy())
                kept_v[layer].append(v[sel].float().cpu().numpy())
    torch.cuda.synchronize()
    if keep is None:
        return None
    return ([np.concatenate(a) for a in kept_k], [np.concatenate(a) for a in kept_v])


def alloc_sequences(h: EngineHandle, seq_lens) -> None:
    for s, n in enumerate(seq_lens):
        ns.ns_kv_alloc(h.kv, s, int(n))


def blocks_for(seq_lens) -> int:
    return int(max(-(-int(n) // BLOCK_SIZE) for n in seq_lens))
