"""Seeded synthetic inputs and workload shapes.

This module is shared by the product tests, the benchmark and the oracle
checks.  It holds no attention arithmetic: it only draws i.i.d. standard
normal tensors, rounds them to bfloat16 when asked, and names the workload
shapes.

The workloads stand in for the pages' datasets (egocentric / Kinetics video
clips and long visual contexts of multimodal LLMs), which are not available:
tokens are i.i.d. N(0, 1) at the attention shapes those models produce.
Sequence lengths follow the cube partition N = (T/t)(H/h)(W/w) of
"Training a Large Video Model on a Single Machine in a Day", §3 "Video
Transformer"; the long-KV cross-attention shape is the setting of the
LV-XAttn abstract (small query block, large key/value blocks).

Seeding is per head, so any (b, h) slice can be regenerated on its own:
tensor t of head (b, h) in workload c uses numpy's PCG64 with seed
(4c + t) * 2**20 + b*H + h, drawing standard_normal((N, d), float32).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}


@dataclass(frozen=True)
class Workload:
    cid: int          # seed namespace
    name: str
    B: int
    H: int
    Nq: int
    Nkv: int
    d: int
    dtype: str        # "f32" or "bf16"
    chunks: int = 1   # KV chunks merged through the log-sum-exp

    @property
    def scale(self) -> float:
        # 1/sqrt(d), rounded to fp32: both the kernels and the oracle use
        # exactly this value.
        return float(np.float32(1.0 / np.sqrt(self.d)))

    @property
    def units(self) -> int:
        """B*H*Nq*Nkv*d: the forward is 4 units of flops, the backward 10."""
        return self.B * self.H * self.Nq * self.Nkv * self.d


WORKLOADS = {
    # 8 frames at 112x112 with 2x16x16 tubelets: 4*7*7 = 196 tokens
    "tiny_f32": Workload(1, "tiny_f32", 1, 2, 196, 196, 64, "f32"),
    # 16 frames at 224x224 with 2x16x16 tubelets: 8*14*14 = 1568 tokens
    "vit_b": Workload(2, "vit_b", 32, 12, 1568, 1568, 64, "bf16"),
    "vit_l": Workload(3, "vit_l", 16, 16, 1568, 1568, 64, "bf16"),
    # 16 frames at 224x224 with 2x14x14 tubelets: 8*16*16 = 2048 tokens
    "vit_h14": Workload(4, "vit_h14", 8, 16, 2048, 2048, 80, "bf16"),
    # 128 text tokens against 256 frames x 128 visual tokens, 8 KV chunks
    "xattn": Workload(5, "xattn", 4, 32, 128, 32768, 128, "bf16", chunks=8),
    # The ViT-B clips above (32 clips, 8 x 14 x 14 tubelet grid, 12 heads,
    # d = 64) under divided space-time attention: temporal attention over the
    # 8 time steps of each of the 32 * 196 spatial positions, and spatial
    # attention over the 196 positions of each of the 32 * 8 time steps
    # (sequences flattened into the batch axis).
    "vit_b_temporal": Workload(6, "vit_b_temporal", 32 * 196, 12, 8, 8, 64, "bf16"),
    "vit_b_spatial": Workload(7, "vit_b_spatial", 32 * 8, 12, 196, 196, 64, "bf16"),
}


@dataclass(frozen=True)
class PackedWorkload:
    """Variable-length sequences packed along one token axis ([T, H, d]),
    each attending to itself.  Sequence s, head h draws its rows like head
    (b = s, h) of a dense workload with the same cid."""
    cid: int
    name: str
    H: int
    d: int
    lens: tuple       # tokens per sequence (queries = keys)
    dtype: str = "bf16"
    chunks: int = 1

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))

    @property
    def tokens(self) -> int:
        return int(sum(self.lens))

    @property
    def units(self) -> int:
        """sum over sequences of n*n*d, times H (the dense B*H*Nq*Nkv*d)."""
        return self.H * self.d * int(sum(n * n for n in self.lens))

    @property
    def cu(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int32)


PACKED_WORKLOADS = {
    # Mixed image / video batch packed instead of padded (the sequence
    # packing of the NeMo video-model page): ViT-B clips of 16, 8 and 4
    # frames (8, 4, 2 tubelet steps of 14 x 14) and single images, eight of
    # each, 12 heads, d = 64.
    "vit_b_packed": PackedWorkload(8, "vit_b_packed", 12, 64, (1568, 784, 392, 196) * 8),
}


def packed_tensor(w: PackedWorkload, tensor: str) -> np.ndarray:
    """The packed [T, H, d] tensor: sequence s, head h at rows cu[s]..cu[s+1]."""
    cu = w.cu
    out = np.empty((w.tokens, w.H, w.d), dtype=np.float32)
    for s, n in enumerate(w.lens):
        for h in range(w.H):
            out[cu[s]:cu[s + 1], h] = head_tensor(w.cid, tensor, s, h, w.H, n, w.d, w.dtype)
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def head_seed(cid: int, tensor: str, b: int, h: int, H: int) -> int:
    return (cid * 4 + TENSOR_IDS[tensor]) * (1 << 20) + b * H + h


def head_tensor(cid: int, tensor: str, b: int, h: int, H: int, n: int, d: int,
                dtype: str) -> np.ndarray:
    """One head's [n, d] slice of tensor `tensor`, as fp32 values."""
    g = np.random.Generator(np.random.PCG64(head_seed(cid, tensor, b, h, H)))
    x = g.standard_normal((n, d), dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def full_tensor(cid: int, tensor: str, B: int, H: int, n: int, d: int,
                dtype: str, out: np.ndarray | None = None) -> np.ndarray:
    """The whole [B, H, n, d] tensor (concatenation of the per-head slices)."""
    if out is None:
        out = np.empty((B, H, n, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h] = head_tensor(cid, tensor, b, h, H, n, d, dtype)
    return out


def workload_head(w: Workload, b: int, h: int) -> dict:
    """q, k, v, do of head (b, h) as fp32 arrays."""
    return {
        "q": head_tensor(w.cid, "q", b, h, w.H, w.Nq, w.d, w.dtype),
        "k": head_tensor(w.cid, "k", b, h, w.H, w.Nkv, w.d, w.dtype),
        "v": head_tensor(w.cid, "v", b, h, w.H, w.Nkv, w.d, w.dtype),
        "do": head_tensor(w.cid, "do", b, h, w.H, w.Nq, w.d, w.dtype),
    }


def random_case(seed: int, B: int, H: int, Nq: int, Nkv: int, d: int,
                dtype: str = "bf16", q_mult: float = 1.0) -> dict:
    """A small ad-hoc case (tests): q, k, v, do as [B, H, N, d] fp32 arrays.

    q_mult multiplies q before rounding; powers of two keep bf16 values exact
    and make the softmax peaky (a stress case for the running maximum).
    """
    g = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, n in (("q", Nq), ("k", Nkv), ("v", Nkv), ("do", Nq)):
        x = g.standard_normal((B, H, n, d), dtype=np.float32)
        if name == "q":
            x = x * np.float32(q_mult)
        out[name] = round_to_bf16(x) if dtype == "bf16" else x
    return out
