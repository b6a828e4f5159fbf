"""Seeded synthetic workloads for one rank's share of a Ulysses attention layer.

This module is shared by the tests, the smoke check and the bench. It holds the
configuration shapes and the seeded input generators, and nothing of the method's
arithmetic: no permute, no attention, no gradient. Both the CPU oracle and the
GPU path consume the exact bytes produced here.

Source of the shapes: the pages describe a Ulysses layer in which each of P GPUs
holds a contiguous chunk of tokens with all heads ("Ulysses Sequence Parallelism:
Training with Million-Token Contexts", section on how it works, steps 1-3), and the
benchmark workload is Qwen3-4B at 64K tokens with SP=4 (same page, throughput
section). UPipe's 32B-class share (tilnote.io commentary, section on activation
memory) gives the chunked case. Values are random normal: trained weights and the
Gutenberg dataset are not available and attention cost depends only on shapes and
document lengths.

Recipe (also stated in the design doc):
  * every global tensor [s, H, d] is drawn in row chunks of CHUNK_ROWS rows; chunk c
    of tensor `name` comes from numpy.random.default_rng([seed, TENSOR_ID[name], c])
    .standard_normal(..., float32), times `amp`, then rounded to bf16 (round to
    nearest even) or kept as fp32. Any row range can therefore be regenerated
    without drawing the rest of the tensor.
  * rank p holds rows [p*s_l, (p+1)*s_l) of each global tensor (contiguous chunks).
  * packed documents: lengths from their own default_rng(seed).geometric(1/mean) until
    their sum reaches s, the last one truncated to fit; cu_seqlens = running sums.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK_ROWS = 4096
TENSOR_ID = {"q": 1, "k": 2, "v": 3, "do": 4}


@dataclass(frozen=True)
class Config:
    name: str
    P: int            # simulated ranks (SP size)
    s_l: int          # tokens per rank
    Hq: int           # global q heads
    Hkv: int          # global kv heads
    d: int            # head dim
    dtype: str        # "bf16" or "f32"
    amp: float = 1.0  # inputs are amp * N(0, 1)
    causal: bool = True
    packed_mean: float | None = None     # mean document length when packed
    chunk_heads: tuple = field(default_factory=tuple)  # q heads per chunk (UPipe)

    @property
    def s(self) -> int:
        return self.P * self.s_l

    @property
    def Hq_l(self) -> int:
        return self.Hq // self.P

    @property
    def Hkv_l(self) -> int:
        return self.Hkv // self.P

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def esize(self) -> int:
        return 2 if self.dtype == "bf16" else 4


WORKLOADS = {
    # tiny fp32 case: 2 ranks x 256 tokens, 4 q / 4 kv heads, d 64, inputs 0.5*N(0,1)
    "tiny_f32": Config("tiny_f32", P=2, s_l=256, Hq=4, Hkv=4, d=64, dtype="f32", amp=0.5),
    # Qwen3-4B-shaped SP=4 share at 8K tokens
    "qwen_8k": Config("qwen_8k", P=4, s_l=2048, Hq=32, Hkv=8, d=128, dtype="bf16"),
    # mid-size shares of the same model at 16K and 32K tokens (grids of one to two rounds)
    "qwen_16k": Config("qwen_16k", P=4, s_l=4096, Hq=32, Hkv=8, d=128, dtype="bf16"),
    "qwen_32k": Config("qwen_32k", P=4, s_l=8192, Hq=32, Hkv=8, d=128, dtype="bf16"),
    # the 64K headline share: 8 q / 2 kv heads after the all-to-all
    "qwen_64k": Config("qwen_64k", P=4, s_l=16384, Hq=32, Hkv=8, d=128, dtype="bf16"),
    # packed SFT batch at 98304 tokens, documents of mean length 6000
    "packed_96k": Config("packed_96k", P=4, s_l=24576, Hq=32, Hkv=8, d=128, dtype="bf16",
                         packed_mean=6000.0),
    # one rank's share of a million-token sequence: 8 ranks of 131072 tokens, 16 q / 8 kv heads
    "million": Config("million", P=8, s_l=131072, Hq=16, Hkv=8, d=128, dtype="bf16"),
    # UPipe headwise-chunked share, 32B-shaped SP=8 at 262144 tokens
    "upipe_256k": Config("upipe_256k", P=8, s_l=32768, Hq=64, Hkv=8, d=128, dtype="bf16",
                         chunk_heads=(1, 2)),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even), returned as a uint16 bit array."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw element bits (uint16 bf16 / uint32 fp32) -> float64 values."""
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float32).astype(np.float64)


def gen_rows(cfg: Config, name: str, row0: int, row1: int, seed: int = 0) -> np.ndarray:
    """Rows [row0, row1) of the global tensor `name` ([s, H, d]) as raw bits.

    bf16 -> uint16 bits, f32 -> uint32 bits."""
    H = cfg.Hq if name in ("q", "do") else cfg.Hkv
    amp = 1.0 if name == "do" else cfg.amp
    parts = []
    c0, c1 = row0 // CHUNK_ROWS, (row1 - 1) // CHUNK_ROWS
    for c in range(c0, c1 + 1):
        lo, hi = c * CHUNK_ROWS, min((c + 1) * CHUNK_ROWS, cfg.s)
        rng = np.random.default_rng([seed, TENSOR_ID[name], c])
        x = rng.standard_normal((hi - lo, H, cfg.d), dtype=np.float32)
        if amp != 1.0:
            x *= np.float32(amp)
        a, b = max(lo, row0) - lo, min(hi, row1) - lo
        x = x[a:b]
        parts.append(to_bf16_bits(x) if cfg.dtype == "bf16" else x.view(np.uint32).copy())
    return np.concatenate(parts, axis=0) if len(parts) > 1 else parts[0]


def gen_global(cfg: Config, name: str, seed: int = 0) -> np.ndarray:
    return gen_rows(cfg, name, 0, cfg.s, seed)


def shards_of(glob: np.ndarray, P: int) -> list:
    """Split a global [s, H, d] tensor into P contiguous token shards (rank p: rows p*s_l..)."""
    s_l = glob.shape[0] // P
    return [np.ascontiguousarray(glob[p * s_l:(p + 1) * s_l]) for p in range(P)]


def head_slice(glob: np.ndarray, P: int, rank: int) -> np.ndarray:
    """The [s, H/P, d] head shard of rank `rank` taken straight from the global tensor."""
    Hl = glob.shape[1] // P
    return np.ascontiguousarray(glob[:, rank * Hl:(rank + 1) * Hl])


def doc_lengths(s: int, mean: float, seed: int = 0) -> list:
    """Packed document lengths: geometric(1/mean) draws (support >= 1) from their own
    default_rng(seed) stream until they cover s; the last one is truncated to fit."""
    rng = np.random.default_rng(seed)
    out, tot = [], 0
    while tot < s:
        n = int(rng.geometric(1.0 / mean))
        n = min(n, s - tot)
        out.append(n)
        tot += n
    return out


def cu_seqlens_of(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def cu_seqlens_for(cfg: Config, seed: int = 0):
    if cfg.packed_mean is None:
        return None
    return cu_seqlens_of(doc_lengths(cfg.s, cfg.packed_mean, seed))


def torch_from_bits(bits: np.ndarray, dtype: str, device="cpu") -> torch.Tensor:
    """Wrap raw bits as a torch tensor of the element type (bf16 or fp32), no rounding."""
    if dtype == "bf16":
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(bits.view(np.float32))
    return t.to(device)


def bits_from_torch(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    raise TypeError(t.dtype)
