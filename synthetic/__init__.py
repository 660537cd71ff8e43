"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path.

This module only draws numbers and describes shapes. It holds none of the
attention, merge or relayout arithmetic, so the oracle and the GPU library stay
independent: both read the very same bits from here.

Recipe (one CPU ``torch.Generator`` per workload, seed ``1000 + workload id``,
the shared-seed practice of the Context parallelism guide (diffusers), Ring
Attention example): Q, K, V are drawn in that order as fp32 N(0, 1) over the
whole sequence, shape ``[1][S][H][D]``, then rounded to bf16 (round to nearest
even) for the bf16 workloads. A Ulysses rank's input is the same full-sequence
tensor viewed as ``[P][1][S/P][H][D]`` (P contiguous sequence shards).

Shapes follow the workloads the pages benchmark: FLUX 1024x1024 (4096 image +
512 text tokens) and 1008x1008 (63x63 + 512 = 4481 tokens, which only Ulysses
Anything splits over 4 ranks), Qwen-Image 1536x1536 (96x96 latent + 256 text
tokens), a Wan video of 21x30x52 latent patches, and a 128K-token causal LLM.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype and how the sequence is split."""

    wid: int
    name: str
    S: int  # total sequence length
    H: int  # total heads
    D: int  # head dim
    dtype: torch.dtype
    causal: bool
    P: int  # ring degree (ring workloads) or Ulysses degree (Ulysses workloads)
    kind: str  # "ring", "ulysses", "ulysses_anything", "kv_gather" or "unified"
    # ring: K/V chunk lengths in sequence order; ulysses_anything: tokens per rank;
    # unified: ring segment lengths (each spread over P / len(chunk_lens) Ulysses ranks)
    chunk_lens: Tuple[int, ...] = ()

    @property
    def seed(self) -> int:
        return 1000 + self.wid

    @property
    def H_local(self) -> int:
        return self.H // self.P

    @property
    def S_local(self) -> int:
        return self.S // self.P

    @property
    def head_counts(self) -> Tuple[int, ...]:
        """Heads per Ulysses rank (contiguous groups, the first H mod P get one more)."""
        return even_split(self.H, self.P)

    def chunk_starts(self) -> List[int]:
        starts, acc = [], 0
        for n in self.chunk_lens:
            starts.append(acc)
            acc += n
        return starts


def even_split(S: int, P: int) -> Tuple[int, ...]:
    """Split S tokens into P contiguous chunks; the first S mod P chunks get one more."""
    base, extra = divmod(S, P)
    return tuple(base + (1 if c < extra else 0) for c in range(P))


TINY = Workload(1, "tiny-ring-fp32", S=256, H=2, D=64, dtype=torch.float32, causal=False,
                P=4, kind="ring", chunk_lens=(64, 64, 64, 64))
TINY_RELAYOUT_P = 2
FLUX_RING = Workload(2, "flux-1024-ring4-rank0", S=4608, H=24, D=128, dtype=torch.bfloat16,
                     causal=False, P=4, kind="ring", chunk_lens=(1152, 1152, 1152, 1152))
QWEN_ULYSSES = Workload(3, "qwen-image-1536-ulysses4-rank0", S=9472, H=24, D=128,
                        dtype=torch.bfloat16, causal=False, P=4, kind="ulysses")
WAN_ULYSSES = Workload(4, "wan-21x30x52-ulysses8-rank0", S=32760, H=40, D=128,
                       dtype=torch.bfloat16, causal=False, P=8, kind="ulysses")
LLM_ULYSSES = Workload(5, "llm-128k-causal-ulysses8-rank0", S=131072, H=32, D=128,
                       dtype=torch.bfloat16, causal=True, P=8, kind="ulysses")
LLM_RING_ANYTHING = Workload(5, "llm-ring-anything-4099", S=4099, H=32, D=128,
                             dtype=torch.bfloat16, causal=True, P=4, kind="ring",
                             chunk_lens=even_split(4099, 4))

# FLUX at 1008x1008: 63x63 latent patches + 512 text tokens = 4481, which no
# Ulysses degree of 4 divides (the Ulysses Anything case of the diffusers guide)
FLUX_ANYTHING = Workload(6, "flux-1008-ulysses-anything4-rank0", S=63 * 63 + 512, H=24, D=128,
                         dtype=torch.bfloat16, causal=False, P=4, kind="ulysses_anything",
                         chunk_lens=even_split(63 * 63 + 512, 4))

# Wan 21x30x52 over a K/V-gather degree of 4 (the fastest tested topology for
# Wan2.2 on the SGLang Diffusion page): rank r keeps its query shard and
# attends to the K/V gathered from all 4 shards
WAN_KV_GATHER = Workload(7, "wan-21x30x52-kvgather4-rank0", S=32760, H=40, D=128,
                         dtype=torch.bfloat16, causal=False, P=4, kind="kv_gather",
                         chunk_lens=even_split(32760, 4))

# FLUX 1024x1024 on 4 ranks as Ulysses 2 x ring 2 (the unified mode of the
# diffusers guide's 4-GPU benchmark): 2 ring segments of 2304 tokens, each
# spread over 2 Ulysses ranks
FLUX_UNIFIED = Workload(8, "flux-1024-unified-u2r2-rank0", S=4608, H=24, D=128,
                        dtype=torch.bfloat16, causal=False, P=4, kind="unified",
                        chunk_lens=(2304, 2304))

WORKLOADS = {w.name: w for w in (TINY, FLUX_RING, QWEN_ULYSSES, WAN_ULYSSES, LLM_ULYSSES,
                                 LLM_RING_ANYTHING, FLUX_ANYTHING, WAN_KV_GATHER, FLUX_UNIFIED)}


def ring_order(rank: int, P: int) -> List[int]:
    """Chunk visit order of ring rank ``rank``: its own chunk, then r-1, r-2, ... mod P."""
    return [(rank - t) % P for t in range(P)]


def draw(shape: Sequence[int], dtype: torch.dtype, gen: torch.Generator) -> torch.Tensor:
    """fp32 N(0,1) draw, rounded to ``dtype`` (round to nearest even for bf16)."""
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def make_qkv(w: Workload, S: Optional[int] = None, H: Optional[int] = None,
             scale_q: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Full-sequence Q, K, V on the CPU, each ``[1][S][H][D]``, seeded by the workload.

    ``S``/``H`` override the sequence length / head count (smaller parity cases
    with the same recipe). ``scale_q`` multiplies Q before rounding, for the
    peaky-softmax stress input.
    """
    S = w.S if S is None else S
    H = w.H if H is None else H
    gen = torch.Generator().manual_seed(w.seed)
    out = []
    for i in range(3):
        x = torch.randn((1, S, H, w.D), generator=gen, dtype=torch.float32)
        if i == 0 and scale_q != 1.0:
            x = x * scale_q
        out.append(x if w.dtype == torch.float32 else x.to(w.dtype))
    return out[0], out[1], out[2]


def make_tensor(shape: Sequence[int], dtype: torch.dtype, seed: int) -> torch.Tensor:
    """A seeded N(0,1) tensor of any shape (parity cases of assorted sizes)."""
    return draw(shape, dtype, torch.Generator().manual_seed(seed))


def random_bits(shape: Sequence[int], itemsize: int, seed: int) -> torch.Tensor:
    """Random raw bit patterns (uint16 or int32 words) for bit-exact copy tests.

    Every pattern is possible, so NaN payloads, infinities, denormals and -0
    all occur.
    """
    gen = torch.Generator().manual_seed(seed)
    if itemsize == 2:
        return torch.randint(0, 1 << 16, tuple(shape), generator=gen, dtype=torch.int32).to(
            torch.int16)
    if itemsize == 4:
        return torch.randint(-(1 << 31), 1 << 31, tuple(shape), generator=gen,
                             dtype=torch.int64).to(torch.int32)
    raise ValueError("itemsize must be 2 or 4")


def random_splits(S: int, P: int, seed: int, min_len: int = 1) -> Tuple[int, ...]:
    """P positive chunk lengths summing to S, drawn from a seeded generator."""
    if P * min_len > S:
        raise ValueError("cannot split")
    gen = torch.Generator().manual_seed(seed)
    cuts = torch.randperm(S - P * min_len + P - 1, generator=gen)[: P - 1].sort().values.tolist()
    lens, prev = [], -1
    for c in cuts + [S - P * min_len + P - 1]:
        lens.append(c - prev - 1 + min_len)
        prev = c
    return tuple(lens)
