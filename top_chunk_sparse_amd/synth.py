"""Seeded synthetic inputs for the chunk-sparse attention workloads.

This module only draws and lays out data; it holds none of the attention or selection
arithmetic.  Both the HIP path and the CPU oracle consume the exact bf16 bytes it produces.

Recipe (decode):
  * q, K, V ~ N(0, 1) in fp32, rounded to bf16 (round-to-nearest-even).
  * Planted chunks: per (batch, KV head) a set of distinct historical chunks; every key of a
    planted chunk gets ``shift * u`` added in fp32 before rounding, where u is the unit vector
    of the sum of the group's query heads (read back from bf16).
  * Gist t of chunk c = mean over the t-th sub-block of C/g tokens of the stored (bf16) keys
    (values) + N(0, noise^2), rounded to bf16.  Gists exist for historical chunks only.
  * Level-2 gist t of group r = mean over the group's chunks of gist t + N(0, noise^2).
  * Paged KV: physical layout [P][Hkv][C][d] with one chunk per page; the page table maps
    (batch, chunk) to a page, a random permutation of all pages when ``paged``.
Recipe (prefill): q, K, V ~ N(0, 1) -> bf16; selector scores S ~ N(0, 1) fp32 of shape
[B][Hkv][nb][nb] (entries on or above the diagonal are left random on purpose).
Recipe (SSA gist-masked prefill): the interleaved sequence of M chunks, each L raw tokens then
g gist tokens; q, K, V ~ N(0, 1) -> bf16 at every position (raw and gist alike: the kernel's
work does not depend on what the gists learned).
Recipe (prefill gradients): upstream dout ~ N(0, 1) -> bf16 [B][Hq][T][d] and dlse ~ N(0, 1)
fp32 [B][Hq][T], drawn from a generator seeded apart from the forward inputs.

Random values depend on the device the generator runs on (torch's CPU and GPU generators
differ); a given (config, seed, device) always yields identical bytes.
"""
from dataclasses import dataclass
from typing import Optional, List

import torch

from .configs import DecodeConfig, GistPrefillConfig, PrefillConfig


@dataclass
class DecodeInputs:
    cfg: DecodeConfig
    q: torch.Tensor            # bf16 [B][Hq][d]
    k_pages: torch.Tensor      # bf16 [P][Hkv][C][d]
    v_pages: torch.Tensor      # bf16 [P][Hkv][C][d]
    page_table: torch.Tensor   # int32 [B][max_chunks]
    gist_k: torch.Tensor       # bf16 [B][Hkv][M-1][g][d]
    gist_v: torch.Tensor
    gist2_k: Optional[torch.Tensor]  # bf16 [B][Hkv][nG][g][d] or None
    gist2_v: Optional[torch.Tensor]
    planted: torch.Tensor      # int64 [B][Hkv][n_plant], ascending chunk ids

    @property
    def num_pages(self) -> int:
        return self.k_pages.shape[0]


@dataclass
class PrefillInputs:
    cfg: PrefillConfig
    q: torch.Tensor   # bf16 [B][Hq][T][d]
    k: torch.Tensor   # bf16 [B][Hkv][T][d]
    v: torch.Tensor   # bf16 [B][Hkv][T][d]
    S: torch.Tensor   # fp32 [B][Hkv][nb][nb]


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _pick_planted(cfg: DecodeConfig, gen, device) -> torch.Tensor:
    """Distinct historical chunk ids per (b, kv); never the current chunk."""
    B, Hkv, H = cfg.B, cfg.Hkv, cfg.H
    n = min(cfg.n_plant, H)
    out = torch.empty((B, Hkv, n), dtype=torch.int64)
    for b in range(B):
        for kv in range(Hkv):
            if cfg.levels == 2 and cfg.plant_groups > 0 and n > 0:
                full = H // cfg.J                     # groups holding J chunks
                ng = min(cfg.plant_groups, full)
                per = n // ng
                groups = torch.randperm(full, generator=gen, device=device)[:ng].cpu()
                ids = []
                for r in groups.tolist():
                    within = torch.randperm(cfg.J, generator=gen, device=device)[:per].cpu()
                    ids += [r * cfg.J + w for w in within.tolist()]
                ids = ids + [ids[-1]] * (n - len(ids))   # n divisible by ng in every preset
                out[b, kv] = torch.tensor(sorted(ids))
            else:
                out[b, kv] = torch.randperm(H, generator=gen, device=device)[:n].cpu().sort().values
    return out


def make_decode(cfg: DecodeConfig, seed: int, device="cpu", max_chunks: Optional[int] = None,
                extra_pages: int = 0) -> DecodeInputs:
    """Draw one decode instance.  ``max_chunks`` pads the page-table rows (stride >= M);
    ``extra_pages`` appends unused pages to the pool (filled with noise)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, Hq, Hkv, d, C, g, M = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.C, cfg.g, cfg.M
    G, H = cfg.G, cfg.H
    assert Hq % Hkv == 0 and C % g == 0 and cfg.N >= 1
    mc = M if max_chunks is None else max_chunks
    assert mc >= M

    q = _randn((B, Hq, d), gen, device).to(torch.bfloat16)
    planted = _pick_planted(cfg, gen, device)

    P = B * M + extra_pages
    if cfg.paged:
        perm = torch.randperm(P, generator=gen, device=device).to(torch.int32)
    else:
        perm = torch.arange(P, device=device, dtype=torch.int32)
    page_table = torch.full((B, mc), -1, dtype=torch.int32, device=device)
    page_table[:, :M] = perm[: B * M].view(B, M)

    k_pages = torch.empty((P, Hkv, C, d), dtype=torch.bfloat16, device=device)
    v_pages = torch.empty((P, Hkv, C, d), dtype=torch.bfloat16, device=device)
    gist_k = torch.empty((B, Hkv, H, g, d), dtype=torch.bfloat16, device=device)
    gist_v = torch.empty((B, Hkv, H, g, d), dtype=torch.bfloat16, device=device)

    # Unit vector of the summed group queries, read back from the stored bf16 q.
    qs = q.float().view(B, Hkv, G, d).sum(2)
    u = qs / qs.norm(dim=-1, keepdim=True).clamp_min(1e-30)

    for b in range(B):
        kb = _randn((Hkv, M, C, d), gen, device)
        vb = _randn((Hkv, M, C, d), gen, device)
        for kv in range(Hkv):
            ids = planted[b, kv].to(device)
            if ids.numel():
                kb[kv, ids] += cfg.shift * u[b, kv]
        kb = kb.to(torch.bfloat16)
        vb = vb.to(torch.bfloat16)
        # The current chunk's tail beyond N holds no tokens; zero it so it is inert.
        if cfg.cur_len < C:
            kb[:, M - 1, cfg.cur_len:] = 0
            vb[:, M - 1, cfg.cur_len:] = 0
        pages = page_table[b, :M].long()
        k_pages[pages] = kb.permute(1, 0, 2, 3)
        v_pages[pages] = vb.permute(1, 0, 2, 3)
        if H > 0:
            sub = C // g
            km = kb[:, :H].float().view(Hkv, H, g, sub, d).mean(3)
            vm = vb[:, :H].float().view(Hkv, H, g, sub, d).mean(3)
            gist_k[b] = (km + cfg.gist_noise * _randn(km.shape, gen, device)).to(torch.bfloat16)
            gist_v[b] = (vm + cfg.gist_noise * _randn(vm.shape, gen, device)).to(torch.bfloat16)
        del kb, vb
    if extra_pages:
        k_pages[B * M:] = _randn((extra_pages, Hkv, C, d), gen, device).to(torch.bfloat16)
        v_pages[B * M:] = _randn((extra_pages, Hkv, C, d), gen, device).to(torch.bfloat16)

    gist2_k = gist2_v = None
    if cfg.levels == 2:
        nG, J = cfg.nG, cfg.J
        gist2_k = torch.empty((B, Hkv, nG, g, d), dtype=torch.bfloat16, device=device)
        gist2_v = torch.empty((B, Hkv, nG, g, d), dtype=torch.bfloat16, device=device)
        for r in range(nG):
            lo, hi = r * J, min(H, (r + 1) * J)
            mk = gist_k[:, :, lo:hi].float().mean(2)
            mv = gist_v[:, :, lo:hi].float().mean(2)
            gist2_k[:, :, r] = (mk + cfg.gist_noise * _randn(mk.shape, gen, device)).to(torch.bfloat16)
            gist2_v[:, :, r] = (mv + cfg.gist_noise * _randn(mv.shape, gen, device)).to(torch.bfloat16)

    return DecodeInputs(cfg, q, k_pages, v_pages, page_table, gist_k, gist_v, gist2_k, gist2_v,
                        planted)


def make_prefill(cfg: PrefillConfig, seed: int, device="cpu") -> PrefillInputs:
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, Hq, Hkv, d, T, nb = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.T, cfg.nb
    assert T % cfg.blk == 0
    q = _randn((B, Hq, T, d), gen, device).to(torch.bfloat16)
    k = _randn((B, Hkv, T, d), gen, device).to(torch.bfloat16)
    v = _randn((B, Hkv, T, d), gen, device).to(torch.bfloat16)
    S = _randn((B, Hkv, nb, nb), gen, device)
    return PrefillInputs(cfg, q, k, v, S)


@dataclass
class GistPrefillInputs:
    cfg: GistPrefillConfig
    q: torch.Tensor            # bf16 [B][Hq][T'][d], T' = M (L + g)
    k: torch.Tensor            # bf16 [B][Hkv][T'][d]
    v: torch.Tensor


def make_gist_prefill(cfg: GistPrefillConfig, seed: int, device="cpu") -> GistPrefillInputs:
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = _randn((cfg.B, cfg.Hq, cfg.Tp, cfg.d), gen, device).to(torch.bfloat16)
    k = _randn((cfg.B, cfg.Hkv, cfg.Tp, cfg.d), gen, device).to(torch.bfloat16)
    v = _randn((cfg.B, cfg.Hkv, cfg.Tp, cfg.d), gen, device).to(torch.bfloat16)
    return GistPrefillInputs(cfg, q, k, v)


def make_prefill_grads(cfg: PrefillConfig, seed: int, device="cpu"):
    """Upstream gradients (dout bf16 [B][Hq][T][d], dlse fp32 [B][Hq][T]) for a backward call."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 7919)
    dout = _randn((cfg.B, cfg.Hq, cfg.T, cfg.d), gen, device).to(torch.bfloat16)
    dlse = _randn((cfg.B, cfg.Hq, cfg.T), gen, device)
    return dout, dlse


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor (exact bit pattern)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
