"""Named workloads for query-guided chunk-sparse attention.

Each preset fixes the shapes, the selection budget and the synthetic-data recipe of one
workload: four decode shapes (a tiny case, a Llama-3.2-1B-shaped and a Llama-3.1-8B-shaped
cache, and a two-level gist-of-gist cache at 512K tokens) and one block-sparse causal prefill
with the SAS gate.  The method follows "Simplified Sparse Attention via Gist Tokens"
(gist scoring, section 3.2; selective unfolding, section 3.3; gist-of-gist, section 3.5) and
"SAS: Simple Attention Sparsification" (abstract: log-form softmax gate, always-kept current
block).  Values here are sizes only; nothing in this module computes.
"""
from dataclasses import dataclass, field, replace
from typing import Optional


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int          # batch
    Hq: int         # query heads
    Hkv: int        # key/value heads (GQA: query head h reads KV head h // (Hq // Hkv))
    d: int          # head dim
    N: int          # tokens in cache, current token included
    C: int          # chunk size == page size
    g: int          # gist tokens per chunk
    k: int          # chunks selected (historical), the current chunk is always kept
    gate: int = 0   # 0: none, 1: SAS log-softmax gate on selected raw tokens
    levels: int = 1
    J: int = 0      # chunks per level-2 group
    k2: int = 0     # level-2 groups selected
    n_plant: int = 0        # query-aligned chunks per (batch, KV head)
    plant_groups: int = 0   # levels=2: planted chunks are spread over this many groups
    paged: bool = False     # random page table (else identity)
    shift: float = 0.5      # planted keys get +shift * unit(sum of the group's queries)
    gist_noise: float = 0.1  # std of the noise added to gist means

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def M(self) -> int:
        return -(-self.N // self.C)

    @property
    def H(self) -> int:
        """Historical (selectable) chunks: all but the current one."""
        return self.M - 1

    @property
    def nG(self) -> int:
        return -(-self.H // self.J) if self.levels == 2 else 0

    @property
    def cur_len(self) -> int:
        return self.N - (self.M - 1) * self.C

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    T: int
    blk: int
    k: int
    gate: int = 1

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def nb(self) -> int:
        return self.T // self.blk

    def with_(self, **kw) -> "PrefillConfig":
        return replace(self, **kw)


# Tiny decode: one KV head, 64 chunks of 64 tokens, one gist per chunk, top-4.
TINY = DecodeConfig("tiny_decode_4k", B=1, Hq=4, Hkv=1, d=64, N=4096, C=64, g=1, k=4,
                    n_plant=4)
# Llama-3.2-1B-shaped decode at 32K tokens, 8 gists per 64-token chunk (8x compression).
LLAMA1B = DecodeConfig("llama32_1b_decode_32k", B=8, Hq=32, Hkv=8, d=64, N=32768, C=64, g=8,
                       k=8, n_plant=16)
# Llama-3.1-8B-shaped decode at 128K tokens, 4 gists per 128-token chunk (32x), SAS gate,
# paged KV with one chunk per page and a random page table.
LLAMA8B = DecodeConfig("llama31_8b_decode_128k", B=16, Hq=32, Hkv=8, d=128, N=131072, C=128,
                       g=4, k=16, gate=1, n_plant=32, paged=True)
# Two-level gist-of-gist decode at 512K tokens: level-2 gists summarise 16 chunks,
# top-4 groups, then top-32 chunks among their 64.
HSSA = DecodeConfig("hssa_decode_512k", B=4, Hq=32, Hkv=8, d=128, N=524288, C=128, g=4, k=32,
                    levels=2, J=16, k2=4, n_plant=32, plant_groups=4)
# Block-sparse causal prefill (SAS training-form forward) at 16K tokens, 64-token blocks.
@dataclass(frozen=True)
class GistPrefillConfig:
    """SSA gist-masked prefill: M chunks of L raw tokens, each followed by its g gist tokens."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    M: int
    L: int
    g: int

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def W(self) -> int:
        """Positions per chunk (raw tokens, then gists)."""
        return self.L + self.g

    @property
    def Tp(self) -> int:
        """Positions of the interleaved sequence."""
        return self.M * self.W

    def with_(self, **kw) -> "GistPrefillConfig":
        return replace(self, **kw)


PREFILL = PrefillConfig("sas_prefill_16k", B=1, Hq=32, Hkv=8, d=128, T=16384, blk=64, k=16,
                        gate=1)

# SSA gist-masked prefill of 16K raw tokens with the Llama-3.1-8B head layout: 128 chunks of
# 128 tokens, 4 gists each (32x compression), 16,896 positions in the interleaved sequence.
GIST_PREFILL = GistPrefillConfig("ssa_gist_prefill_16k", B=1, Hq=32, Hkv=8, d=128, M=128, L=128,
                                 g=4)

DECODE_CONFIGS = {c.name: c for c in (TINY, LLAMA1B, LLAMA8B, HSSA)}
PREFILL_CONFIGS = {PREFILL.name: PREFILL}
GIST_PREFILL_CONFIGS = {GIST_PREFILL.name: GIST_PREFILL}
# Index of each preset in the published list of workloads (seed = 1000 * index + instance).
CONFIG_INDEX = {TINY.name: 1, LLAMA1B.name: 2, LLAMA8B.name: 3, HSSA.name: 4, PREFILL.name: 5,
                GIST_PREFILL.name: 6}


def seed_for(name: str, instance: int = 0) -> int:
    return 1000 * CONFIG_INDEX.get(name, 9) + instance
