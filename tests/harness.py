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


def oracle_prefill_backward(inp: PrefillInputs, dout, dlse, **kw) -> "oracle.PrefillGrads":
    c = inp.cfg
    args = dict(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, T=c.T, blk=c.blk, k=c.k, gate=c.gate,
                q=host(inp.q), k_=host(inp.k), v=host(inp.v),
                S=inp.S.cpu().numpy().astype(np.float32), dout=host(dout),
                dlse=None if dlse is None else dlse.cpu().numpy().astype(np.float32))
    args.update(kw)
    return oracle.prefill_backward(**args)


def oracle_gist_prefill(inp, **kw):
    c = inp.cfg
    args = dict(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, M=c.M, L=c.L, g=c.g, q=host(inp.q),
                k_=host(inp.k), v=host(inp.v))
    args.update(kw)
    return oracle.gist_prefill(**args)


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


def top_p_margin(scores: np.ndarray, p: float, k: int) -> float:
    """Distance of the running share from p at the top-p cut (fp64, rank order): the cut is a
    floating-point decision, so a selection that differs only where the running share is
    within GAP_EXCUSE of p is excused (and counted)."""
    s = scores[np.isfinite(scores)]
    if p >= 1.0 or len(s) == 0:
        return float("inf")
    order = np.lexsort((np.arange(len(s)), -s))
    m = s.max()
    share = np.exp(s[order] - (m + np.log(np.exp(s - m).sum())))
    cum = np.cumsum(share)
    r = int(np.argmax(cum >= p)) if (cum >= p).any() else len(s) - 1
    if r >= k:
        return float("inf")   # the cap decided, not the share
    near = [abs(cum[r] - p)]
    if r > 0:
        near.append(abs(cum[r - 1] - p))
    return float(min(near))


def check_decode(inp: DecodeInputs, call, ref=None, units=None, tol=OUT_TOL, report=None):
    """Compare one finished GPU decode call with the oracle.  Returns a dict of statistics.
    Selected indices must match exactly except where the oracle's boundary gap is below
    GAP_EXCUSE; such units are counted and compared against the oracle run on the GPU's
    selection instead."""
    c = inp.cfg
    G = c.G
    gmode = "selected" if getattr(call, "gist_mode", 0) == 1 else True
    top_p = float(call.p.top_p)
    heads = int(getattr(call, "head_select", 0))
    adaptive = int(getattr(call, "adaptive_k", 0))
    if ref is None:
        ref = oracle_decode(inp, k=call.p.k, units=units, scale=float(call.p.scale),
                            gists_in_softmax=gmode, top_p=top_p, head_select=heads,
                            adaptive_k=adaptive)
    all_units = list(range(c.B * c.Hkv)) if units is None else list(units)
    gsel = call.sel.cpu().numpy()
    gout = call.out.cpu().double().numpy()
    glse = call.lse.cpu().double().numpy()
    ggrp = call.sel_groups.cpu().numpy() if call.sel_groups is not None else None
    excused = []
    k, k2 = call.p.k, c.k2
    if adaptive:   # the boundary sits at the selected count, min(cap, budget), at each level
        budget = oracle.adaptive_k_budget(N=c.N, C_=c.C, Hq=c.Hq, Hkv=c.Hkv, levels=c.levels,
                                          J=c.J)
        k, k2 = min(k, budget), min(k2, budget)
    for u in all_units:
        b, kv = divmod(u, c.Hkv)
        ok = np.array_equal(gsel[b, kv], ref.sel[b, kv])
        if c.levels == 2:
            ok = ok and np.array_equal(ggrp[b, kv], ref.sel_groups[b, kv])
        if ok:
            continue
        gaps = []
        if c.levels == 2:
            gaps.append(boundary_gap(ref.group_scores[b, kv], k2))
        if heads:   # every head's own boundary decides its part of the union
            gaps += [boundary_gap(ref.chunk_scores[b, kv * G + h], k) for h in range(G)]
        elif top_p > 0:
            ke_ref = int((ref.sel[b, kv] >= 0).sum())
            gaps.append(boundary_gap(ref.chunk_scores[b, kv], ke_ref))
            gaps.append(top_p_margin(ref.chunk_scores[b, kv], top_p, k))
        else:
            gaps.append(boundary_gap(ref.chunk_scores[b, kv], k))
        assert min(gaps) < GAP_EXCUSE, (
            f"unit {u}: selection differs (gpu {gsel[b, kv].tolist()} vs oracle "
            f"{ref.sel[b, kv].tolist()}) with boundary gap {min(gaps):.3g}")
        excused.append(u)
    if excused:
        forced = np.ascontiguousarray(gsel.astype(np.int32))
        fg = np.ascontiguousarray(ggrp.astype(np.int32)) if ggrp is not None else None
        ref2 = oracle_decode(inp, k=call.p.k, units=excused, forced_sel=forced, forced_groups=fg,
                             scale=float(call.p.scale), gists_in_softmax=gmode,
                             head_select=heads)
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
        rs = ref.chunk_scores
        if heads:   # one row per query head: view as [B][Hkv][G * H]
            gs = gs.reshape(c.B, c.Hkv, -1)
            rs = rs.reshape(c.B, c.Hkv, -1)
        ub = np.array([u // c.Hkv for u in scored_units])
        uk = np.array([u % c.Hkv for u in scored_units])
        a, r_ = gs[ub, uk], rs[ub, uk]
        fin = np.isfinite(r_)
        assert (np.isfinite(a) == fin).all(), "chunk_scores: scored set differs"
        if fin.any():
            stats["max_abs_score"] = float(np.abs(a[fin] - r_[fin]).max())
    if report is not None:
        report.update(stats)
    assert err_out <= tol and err_lse <= tol, stats
    return stats


# ---------------------------------------------------------------------------------------
# GPU-vs-oracle parity (prefill)
# ---------------------------------------------------------------------------------------
def check_prefill_selection(inp: PrefillInputs, gsel: np.ndarray, k: int):
    """Property check of the block selection on every (b, kv, i) row, any size: ascending,
    in range, -1 padded to min(k, i) entries, and the chosen set is a top set of S[i][j < i]
    under (score desc, index asc) -- every chosen score beats every unchosen one, and a tie
    at the boundary goes to the lower index.  Returns the number of rows checked."""
    c = inp.cfg
    S = inp.S.cpu().numpy().astype(np.float32)
    nb = c.nb
    gsel = gsel.reshape(c.B * c.Hkv, nb, k)
    S = S.reshape(c.B * c.Hkv, nb, nb)
    for i in range(nb):
        ke = min(k, i)
        rows = gsel[:, i, :]
        assert (rows[:, ke:] == -1).all(), f"block {i}: padding"
        if ke == 0:
            continue
        chosen = rows[:, :ke]
        assert ((chosen >= 0) & (chosen < i)).all(), f"block {i}: index out of range"
        assert (np.diff(chosen, axis=1) > 0).all(), f"block {i}: not ascending"
        if ke == i:
            continue
        s_i = S[:, i, :i]
        mask = np.zeros((len(rows), i), bool)
        np.put_along_axis(mask, chosen.astype(np.int64), True, axis=1)
        ch_min = np.where(mask, s_i, np.inf).min(axis=1)
        un_max = np.where(mask, -np.inf, s_i).max(axis=1)
        assert (ch_min >= un_max).all(), f"block {i}: a better block was left out"
        tie = ch_min == un_max
        for u in np.nonzero(tie)[0]:
            v = ch_min[u]
            hi_ch = np.nonzero(mask[u] & (s_i[u] == v))[0].max()
            lo_un = np.nonzero(~mask[u] & (s_i[u] == v))[0].min()
            assert hi_ch < lo_un, f"block {i} unit {u}: tie not broken to the lower index"
    return c.B * c.Hkv * nb


def check_prefill(inp: PrefillInputs, call, blocks=None, tol=OUT_TOL, report=None):
    """Compare one finished GPU prefill call with the oracle on the query blocks ``blocks``
    (flat ids unit * nb + i; all when None).  The selection must match the oracle's exactly:
    both sides rank the same fp32 selector scores S[i][j < i] (ties to the lower j), so no
    boundary is excused."""
    c = inp.cfg
    G, nb, blk = c.G, c.nb, c.blk
    k = call.p.k
    allb = np.arange(c.B * c.Hkv * nb) if blocks is None else np.asarray(blocks, np.int64)
    ref = oracle_prefill(inp, k=k, blocks=None if blocks is None else allb.astype(np.int32),
                         scale=float(call.p.scale))
    gout = call.out.cpu().numpy()
    glse = call.lse.cpu().numpy()
    if k > 0:
        gsel = call.sel.cpu().numpy()
        for x in allb:
            u, i = divmod(int(x), nb)
            b, kv = divmod(u, c.Hkv)
            assert np.array_equal(gsel[b, kv, i], ref.sel[b, kv, i]), (
                f"block {x}: selection differs (gpu {gsel[b, kv, i].tolist()} vs oracle "
                f"{ref.sel[b, kv, i].tolist()})")
    err_out = err_lse = 0.0
    for x in allb:
        u, i = divmod(int(x), nb)
        b, kv = divmod(u, c.Hkv)
        hs, ts = slice(kv * G, (kv + 1) * G), slice(i * blk, (i + 1) * blk)
        err_out = max(err_out, float(np.abs(gout[b, hs, ts] - ref.out[b, hs, ts]).max()))
        err_lse = max(err_lse, float(np.abs(glse[b, hs, ts] - ref.lse[b, hs, ts]).max()))
    stats = dict(blocks=len(allb), excused=0, max_abs_out=err_out, max_abs_lse=err_lse)
    if report is not None:
        report.update(stats)
    assert err_out <= tol and err_lse <= tol, stats
    return stats
