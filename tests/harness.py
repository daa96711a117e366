"""Glue between the seeded generator and the CPU oracle (tests only)."""
import numpy as np
import torch

import oracle
from top_chunk_sparse_amd.synth import DecodeInputs, PrefillInputs, bf16_bits


def host(t):
    return None if t is None else bf16_bits(t)


def oracle_decode(inp: DecodeInputs, **kw) -> "oracle.DecodeResult":
    c = inp.cfg
    args = dict(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, N=c.N, C_=c.C, g=c.g, k=c.k, gate=c.gate,
                levels=c.levels, J=c.J, k2=c.k2,
                q=host(inp.q), k_pages=host(inp.k_pages), v_pages=host(inp.v_pages),
                page_table=inp.page_table.cpu().numpy().astype(np.int32),
                gist_k=host(inp.gist_k), gist_v=host(inp.gist_v),
                gist2_k=host(inp.gist2_k), gist2_v=host(inp.gist2_v))
    args.update(kw)
    return oracle.decode(**args)


def oracle_prefill(inp: PrefillInputs, **kw) -> "oracle.PrefillResult":
    c = inp.cfg
    args = dict(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, T=c.T, blk=c.blk, k=c.k, gate=c.gate,
                q=host(inp.q), k_=host(inp.k), v=host(inp.v),
                S=inp.S.cpu().numpy().astype(np.float32))
    args.update(kw)
    return oracle.prefill(**args)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()
