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


# ---------------------------------------------------------------------------------------
# GPU-vs-oracle parity (decode)
# ---------------------------------------------------------------------------------------
GAP_EXCUSE = 1e-5     # relative score gap at the k-th boundary below which a mismatch is excused
OUT_TOL = 1e-2        # max-abs tolerance on out and lse (bf16 inputs, fp32 accumulation)


def boundary_gap(scores: np.ndarray, k: int) -> float:
    """Relative gap between the k-th and (k+1)-th largest finite scores (inf if no boundary)."""
    s = np.sort(scores[np.isfinite(scores)])[::-1]
    if k <= 0 or k >= len(s):
        return float("inf")
    a, b = s[k - 1], s[k]
    return float((a - b) / max(abs(a), abs(b), 1.0))


def check_decode(inp: DecodeInputs, call, ref=None, units=None, tol=OUT_TOL, report=None):
    """Compare one finished GPU decode call with the oracle.  Returns a dict of statistics.
    Selected indices must match exactly except where the oracle's boundary gap is below
    GAP_EXCUSE; such units are counted and compared against the oracle run on the GPU's
    selection instead."""
    c = inp.cfg
    G = c.G
    if ref is None:
        ref = oracle_decode(inp, k=call.p.k, units=units, scale=float(call.p.scale))
    all_units = list(range(c.B * c.Hkv)) if units is None else list(units)
    gsel = call.sel.cpu().numpy()
    gout = call.out.cpu().double().numpy()
    glse = call.lse.cpu().double().numpy()
    ggrp = call.sel_groups.cpu().numpy() if call.sel_groups is not None else None
    excused = []
    k = call.p.k
    for u in all_units:
        b, kv = divmod(u, c.Hkv)
        ok = np.array_equal(gsel[b, kv], ref.sel[b, kv])
        if c.levels == 2:
            ok = ok and np.array_equal(ggrp[b, kv], ref.sel_groups[b, kv])
        if ok:
            continue
        gaps = []
        if c.levels == 2:
            gaps.append(boundary_gap(ref.group_scores[b, kv], c.k2))
        gaps.append(boundary_gap(ref.chunk_scores[b, kv], k))
        assert min(gaps) < GAP_EXCUSE, (
            f"unit {u}: selection differs (gpu {gsel[b, kv].tolist()} vs oracle "
            f"{ref.sel[b, kv].tolist()}) with boundary gap {min(gaps):.3g}")
        excused.append(u)
    if excused:
        forced = np.ascontiguousarray(gsel.astype(np.int32))
        fg = np.ascontiguousarray(ggrp.astype(np.int32)) if ggrp is not None else None
        ref2 = oracle_decode(inp, k=k, units=excused, forced_sel=forced, forced_groups=fg,
                             scale=float(call.p.scale))
        for u in excused:
            b, kv = divmod(u, c.Hkv)
            ref.out[b, kv * G:(kv + 1) * G] = ref2.out[b, kv * G:(kv + 1) * G]
            ref.lse[b, kv * G:(kv + 1) * G] = ref2.lse[b, kv * G:(kv + 1) * G]
    rows = [(u // c.Hkv, (u % c.Hkv) * G + h) for u in all_units for h in range(G)]
    bi = np.array([r[0] for r in rows])
    hi = np.array([r[1] for r in rows])
    err_out = np.abs(gout[bi, hi] - ref.out[bi, hi]).max()
    err_lse = np.abs(glse[bi, hi] - ref.lse[bi, hi]).max()
    stats = dict(units=len(all_units), excused=len(excused), max_abs_out=float(err_out),
                 max_abs_lse=float(err_lse))
    scored_units = [u for u in all_units if not (c.levels == 2 and u in excused)]
    if call.chunk_scores is not None and c.H > 0 and scored_units:
        gs = call.chunk_scores.cpu().double().numpy()
        ub = np.array([u // c.Hkv for u in scored_units])
        uk = np.array([u % c.Hkv for u in scored_units])
        a, r_ = gs[ub, uk], ref.chunk_scores[ub, uk]
        fin = np.isfinite(r_)
        assert (np.isfinite(a) == fin).all(), "chunk_scores: scored set differs"
        if fin.any():
            stats["max_abs_score"] = float(np.abs(a[fin] - r_[fin]).max())
    if report is not None:
        report.update(stats)
    assert err_out <= tol and err_lse <= tol, stats
    return stats
