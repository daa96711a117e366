"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin ties the oracle to something the pages or the mathematics fix:
  * textbook dense attention (torch scaled_dot_product_attention in float64) for the special
    cases that reduce to it: every chunk selected, no chunk selected, full causal prefill;
  * closed forms: pooled chunk score of identical logits, the SAS gate with equal scores
    (gamma = -log|H|), softmax-set sizes (SSA appendix B.1 counts k gist + kL raw tokens);
  * invariants: softmax weights sum to one with the gate inside the softmax (SAS abstract),
    permuting unselected chunks changes nothing, lse is consistent with the weights;
  * library routines for the selection rule: numpy stable argsort (lowest index on ties);
  * brute force: a separate numpy evaluation that materialises the token set.
The functions named pin_* take no fixtures so that test_oracle_mutants.py can re-run them
against deliberately broken copies of the oracle.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from top_chunk_sparse_amd.configs import DecodeConfig, PrefillConfig
from top_chunk_sparse_amd.configs import GistPrefillConfig
from top_chunk_sparse_amd.synth import (make_decode, make_gist_prefill, make_prefill,
                                        make_prefill_grads)
from harness import (oracle_decode, oracle_gist_prefill, oracle_prefill, oracle_prefill_backward,
                     f64)

TOL = 1e-12

SMALL = DecodeConfig("pin_small", B=2, Hq=4, Hkv=2, d=16, N=21 * 8 + 5, C=8, g=2, k=3,
                     n_plant=3, paged=True)
SMALL_G1 = DecodeConfig("pin_g1", B=1, Hq=2, Hkv=2, d=16, N=30 * 8, C=8, g=1, k=4, n_plant=2)
SMALL_L2 = DecodeConfig("pin_l2", B=1, Hq=4, Hkv=1, d=16, N=37 * 8 + 3, C=8, g=2, k=5,
                        levels=2, J=4, k2=2, n_plant=4, plant_groups=2, paged=True)
PF = PrefillConfig("pin_prefill", B=1, Hq=4, Hkv=2, d=16, T=8 * 10, blk=8, k=3, gate=1)


# ----------------------------------------------------------------------------------------
# brute force (numpy, independent of oracle.c)
# ----------------------------------------------------------------------------------------
def _lse(x):
    x = np.asarray(x, dtype=np.float64).ravel()
    m = x.max()
    return m + math.log(np.exp(x - m).sum())


def _logical_kv(inp):
    """K/V as [B][Hkv][M][C][d] float64, through the page table."""
    c = inp.cfg
    pt = inp.page_table.cpu().numpy()[:, : c.M]
    kp, vp = f64(inp.k_pages), f64(inp.v_pages)
    K = kp[pt].transpose(0, 2, 1, 3, 4)
    V = vp[pt].transpose(0, 2, 1, 3, 4)
    return K, V


def brute_decode(inp, gists=True, top_p=0.0, head_select=False):
    c = inp.cfg
    G, H, sig = c.G, c.H, 1.0 / math.sqrt(c.d)
    q = f64(inp.q)
    K, V = _logical_kv(inp)
    gk, gv = f64(inp.gist_k), f64(inp.gist_v)
    out = np.zeros((c.B, c.Hq, c.d))
    lse = np.zeros((c.B, c.Hq))
    sels = np.full((c.B, c.Hkv, G * c.k if head_select else c.k), -1, np.int32)
    for b in range(c.B):
        for kv in range(c.Hkv):
            qg = q[b, kv * G:(kv + 1) * G]
            Ks, Vs, bias = [], [], []
            if c.levels == 2:
                g2k, g2v = f64(inp.gist2_k)[b, kv], f64(inp.gist2_v)[b, kv]
                s2 = np.array([_lse(sig * qg @ g2k[r].T) for r in range(c.nG)])
                order = sorted(range(c.nG), key=lambda r: (-s2[r], r))
                groups = sorted(order[: c.k2])
                cand = [x for r in groups for x in range(r * c.J, min((r + 1) * c.J, H))]
                if gists is True:
                    Ks += [g2k.reshape(-1, c.d)]
                    Vs += [g2v.reshape(-1, c.d)]
                    bias += [0.0] * (c.nG * c.g)
                if gists == "selected":
                    Ks += [g2k[r] for r in groups]
                    Vs += [g2v[r] for r in groups]
                    bias += [0.0] * (len(groups) * c.g)
            else:
                cand = list(range(H))
            s = {x: _lse(sig * qg @ gk[b, kv, x].T) for x in cand}
            order = sorted(cand, key=lambda x: (-s[x], x))
            r = len(order)
            if 0.0 < top_p < 1.0:
                shares = np.exp(np.array([s[x] for x in order]) - _lse([s[x] for x in cand]))
                r = int(np.argmax(np.cumsum(shares) >= top_p)) + 1
            sel = sorted(order[: min(c.k, r)])
            if head_select:   # every head's own top-k by its own score; the union
                union = set()
                for h in range(G):
                    sh = {x: _lse(sig * gk[b, kv, x] @ qg[h]) for x in cand}
                    union |= set(sorted(cand, key=lambda x: (-sh[x], x))[: c.k])
                sel = sorted(union)
            sels[b, kv, : len(sel)] = sel
            lse_s = _lse([s[x] for x in cand]) if cand else 0.0
            if gists is True:
                for x in cand:
                    Ks.append(gk[b, kv, x])
                    Vs.append(gv[b, kv, x])
                    bias += [0.0] * c.g
            if gists == "selected":
                for x in sel:
                    Ks.append(gk[b, kv, x])
                    Vs.append(gv[b, kv, x])
                    bias += [0.0] * c.g
            for x in sel:
                Ks.append(K[b, kv, x])
                Vs.append(V[b, kv, x])
                bias += [(s[x] - lse_s) if c.gate else 0.0] * c.C
            Ks.append(K[b, kv, H, : c.cur_len])
            Vs.append(V[b, kv, H, : c.cur_len])
            bias += [0.0] * c.cur_len
            Kt, Vt, bt = np.concatenate(Ks), np.concatenate(Vs), np.array(bias)
            for h in range(G):
                lam = sig * Kt @ qg[h] + bt
                m = lam.max()
                w = np.exp(lam - m)
                out[b, kv * G + h] = w @ Vt / w.sum()
                lse[b, kv * G + h] = m + math.log(w.sum())
    return out, lse, sels


def brute_prefill(inp):
    c = inp.cfg
    G, nb, blk, sig = c.G, c.nb, c.blk, 1.0 / math.sqrt(c.d)
    q, K, V, S = f64(inp.q), f64(inp.k), f64(inp.v), inp.S.double().numpy()
    out = np.zeros(q.shape)
    lse = np.zeros(q.shape[:3])
    for b in range(c.B):
        for kv in range(c.Hkv):
            for i in range(nb):
                row = S[b, kv, i, :i]
                sel = sorted(sorted(range(i), key=lambda j: (-row[j], j))[: c.k])
                ls = _lse(row) if i > 0 else 0.0
                for h in range(kv * G, (kv + 1) * G):
                    for r in range(blk):
                        p = i * blk + r
                        idx = [u for j in sel for u in range(j * blk, (j + 1) * blk)]
                        bias = [(row[j] - ls) if c.gate else 0.0 for j in sel for _ in range(blk)]
                        idx += list(range(i * blk, p + 1))
                        bias += [0.0] * (r + 1)
                        lam = sig * K[b, kv, idx] @ q[b, h, p] + np.array(bias)
                        m = lam.max()
                        w = np.exp(lam - m)
                        out[b, h, p] = w @ V[b, kv, idx] / w.sum()
                        lse[b, h, p] = m + math.log(w.sum())
    return out, lse


# ----------------------------------------------------------------------------------------
# textbook attention helper (float64 SDPA)
# ----------------------------------------------------------------------------------------
def sdpa(qv, Kt, Vt, bias=None):
    """softmax(q K^T / sqrt(d) + bias) V for one query vector; also returns the natural log
    normaliser computed by torch.logsumexp."""
    qt = torch.from_numpy(np.asarray(qv, np.float64))[None, None, None]
    kt = torch.from_numpy(np.asarray(Kt, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(Vt, np.float64))[None, None]
    mask = None if bias is None else torch.from_numpy(np.asarray(bias, np.float64))[None, None, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)[0, 0, 0].numpy()
    lam = (kt[0, 0] @ qt[0, 0, 0]) / math.sqrt(qt.shape[-1])
    if mask is not None:
        lam = lam + mask[0, 0, 0]
    return o, float(torch.logsumexp(lam, 0))


# ----------------------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------------------
def pin_brute_force_decode():
    for cfg in (SMALL, SMALL.with_(gate=1), SMALL_G1, SMALL_L2):
        inp = make_decode(cfg, seed=11, max_chunks=cfg.M + 3, extra_pages=2)
        r = oracle_decode(inp)
        o, l, s = brute_decode(inp)
        assert np.array_equal(r.sel, s), cfg.name
        assert np.abs(r.out - o).max() < TOL, cfg.name
        assert np.abs(r.lse - l).max() < TOL, cfg.name


def pin_k_all_is_dense():
    """Every chunk selected: softmax over the whole cache (all gists + every raw token) is
    textbook attention; without gists it is dense attention over the N raw tokens."""
    cfg = SMALL.with_(k=SMALL.H, B=1)
    inp = make_decode(cfg, seed=5)
    K, V = _logical_kv(inp)
    q, gk, gv = f64(inp.q), f64(inp.gist_k), f64(inp.gist_v)
    for gists in (True, False):
        r = oracle_decode(inp, gists_in_softmax=gists)
        assert np.array_equal(r.sel[0, 0], np.arange(cfg.H))
        for h in range(cfg.Hq):
            kv = h // cfg.G
            raw_k = K[0, kv].reshape(-1, cfg.d)[: cfg.N]
            raw_v = V[0, kv].reshape(-1, cfg.d)[: cfg.N]
            if gists:
                raw_k = np.concatenate([gk[0, kv].reshape(-1, cfg.d), raw_k])
                raw_v = np.concatenate([gv[0, kv].reshape(-1, cfg.d), raw_v])
            o, l = sdpa(q[0, h], raw_k, raw_v)
            assert np.abs(r.out[0, h] - o).max() < TOL
            assert abs(r.lse[0, h] - l) < TOL


def pin_k_zero_is_gists_plus_current():
    for gate in (0, 1):
        cfg = SMALL.with_(k=0, gate=gate, B=1)
        inp = make_decode(cfg, seed=6)
        K, V = _logical_kv(inp)
        q, gk, gv = f64(inp.q), f64(inp.gist_k), f64(inp.gist_v)
        r = oracle_decode(inp)
        for h in range(cfg.Hq):
            kv = h // cfg.G
            kt = np.concatenate([gk[0, kv].reshape(-1, cfg.d), K[0, kv, cfg.H, : cfg.cur_len]])
            vt = np.concatenate([gv[0, kv].reshape(-1, cfg.d), V[0, kv, cfg.H, : cfg.cur_len]])
            o, l = sdpa(q[0, h], kt, vt)
            assert np.abs(r.out[0, h] - o).max() < TOL
            assert abs(r.lse[0, h] - l) < TOL


def pin_weights_sum_to_one_and_reconstruct():
    for gate in (0, 1):
        cfg = SMALL.with_(gate=gate, B=1)
        inp = make_decode(cfg, seed=7)
        cap = cfg.H * cfg.g + cfg.k * cfg.C + cfg.C
        r = oracle_decode(inp, weights_cap=cap)
        K, V = _logical_kv(inp)
        gv = f64(inp.gist_v)
        for h in range(cfg.Hq):
            kv = h // cfg.G
            n = r.n_tokens[0, h]
            w = r.weights[0, h, :n]
            assert abs(w.sum() - 1.0) < TOL
            assert (w > 0).all()
            # token order: gists (chunk, t), selected chunks ascending, current chunk
            vt = [gv[0, kv].reshape(-1, cfg.d)]
            vt += [V[0, kv, c] for c in r.sel[0, kv] if c >= 0]
            vt += [V[0, kv, cfg.H, : cfg.cur_len]]
            assert np.abs(w @ np.concatenate(vt) - r.out[0, h]).max() < TOL


def pin_permutation_invariance():
    cfg = SMALL.with_(gate=1)
    inp = make_decode(cfg, seed=8)
    r = oracle_decode(inp)
    rng = np.random.default_rng(0)
    pt = inp.page_table.clone()
    gk, gv = inp.gist_k.clone(), inp.gist_v.clone()
    for b in range(cfg.B):
        # one permutation per batch row, over chunks no KV head of that row selected
        chosen = set(r.sel[b].ravel().tolist())
        free = [c for c in range(cfg.H) if c not in chosen]
        perm = rng.permutation(free)
        pt[b, free] = inp.page_table[b, perm]
        gk[b, :, free] = inp.gist_k[b, :, perm]
        gv[b, :, free] = inp.gist_v[b, :, perm]
    from dataclasses import replace
    inp2 = replace(inp, page_table=pt, gist_k=gk, gist_v=gv)
    r2 = oracle_decode(inp2)
    assert np.array_equal(r.sel, r2.sel)
    assert np.abs(r.out - r2.out).max() < TOL
    assert np.abs(r.lse - r2.lse).max() < TOL


def pin_selection_single_gist_single_head():
    """G = g = 1: the chunk score is sigma q . Kg and the choice is numpy's stable argsort."""
    inp = make_decode(SMALL_G1, seed=9)
    r = oracle_decode(inp)
    q, gk = f64(inp.q), f64(inp.gist_k)
    for kv in range(SMALL_G1.Hkv):
        s = gk[0, kv, :, 0] @ q[0, kv] / math.sqrt(SMALL_G1.d)
        assert np.abs(r.chunk_scores[0, kv] - s).max() < TOL
        want = np.sort(np.argsort(-s, kind="stable")[: SMALL_G1.k])
        assert np.array_equal(r.sel[0, kv], want)


def pin_pooled_score_closed_form():
    """Identical queries in a group and identical gists in a chunk: the G*g logits all equal
    x_c, so the pooled log-sum-exp is x_c + log(G*g)."""
    cfg = SMALL.with_(B=1, Hkv=1, Hq=4)
    inp = make_decode(cfg, seed=10)
    inp.q[0, 1:] = inp.q[0, 0]
    inp.gist_k[0, 0, :, 1:] = inp.gist_k[0, 0, :, :1]
    r = oracle_decode(inp)
    x = f64(inp.gist_k)[0, 0, :, 0] @ f64(inp.q)[0, 0] / math.sqrt(cfg.d)
    assert np.abs(r.chunk_scores[0, 0] - (x + math.log(cfg.G * cfg.g))).max() < TOL


def pin_pooled_score_dominant_term():
    """One gist logit far above the rest: the pooled score tends to that logit."""
    cfg = SMALL.with_(B=1, Hkv=1, Hq=2, g=2)
    inp = make_decode(cfg, seed=12)
    q = f64(inp.q)[0]
    inp.gist_k.zero_()
    c = 5
    inp.gist_k[0, 0, c, 1] = torch.from_numpy(q[1] * 8.0).to(torch.bfloat16)
    r = oracle_decode(inp)
    g = f64(inp.gist_k)[0, 0, c]
    logits = np.sort((q @ g.T).ravel() / math.sqrt(cfg.d))
    big, second = logits[-1], logits[-2]
    # max <= LSE <= max + log(1 + (n-1) e^(second-max))
    gap = r.chunk_scores[0, 0, c] - big
    assert 0 <= gap <= math.log1p((cfg.G * cfg.g - 1) * math.exp(second - big)) + 1e-12
    assert gap < 1e-6
    others = np.delete(r.chunk_scores[0, 0], c)
    assert np.abs(others - math.log(cfg.G * cfg.g)).max() < TOL   # all-zero gists: logits 0


def pin_tie_break_lowest_index():
    cfg = SMALL.with_(B=1, k=3)
    inp = make_decode(cfg, seed=13)
    # chunks 2, 6, 9, 14 get the same (largest) gists -> exact ties; lowest three win
    for c in (6, 9, 14):
        inp.gist_k[0, :, c] = inp.gist_k[0, :, 2]
    for kv in range(cfg.Hkv):
        G = cfg.G
        qs = inp.q[0, kv * G:(kv + 1) * G].float().sum(0)
        inp.gist_k[0, kv, 2] = (qs * 3).to(torch.bfloat16)
        for c in (6, 9, 14):
            inp.gist_k[0, kv, c] = inp.gist_k[0, kv, 2]
    r = oracle_decode(inp)
    for kv in range(cfg.Hkv):
        assert r.sel[0, kv].tolist() == [2, 6, 9]


def pin_gate_equal_scores_closed_form():
    """All historical chunks score the same: the SAS gate is -log|H| on every selected raw
    token, ties go to the lowest indices, so the result is textbook attention with a
    constant additive bias of -log|H| on chunks 0..k-1."""
    cfg = SMALL.with_(B=1, gate=1, k=3)
    inp = make_decode(cfg, seed=14)
    inp.gist_k[0, :, :] = inp.gist_k[0, :, :1]
    r = oracle_decode(inp)
    K, V = _logical_kv(inp)
    q, gk, gv = f64(inp.q), f64(inp.gist_k), f64(inp.gist_v)
    gamma = -math.log(cfg.H)
    for h in range(cfg.Hq):
        kv = h // cfg.G
        assert r.sel[0, kv].tolist() == list(range(cfg.k))
        kt = np.concatenate([gk[0, kv].reshape(-1, cfg.d), K[0, kv, : cfg.k].reshape(-1, cfg.d),
                             K[0, kv, cfg.H, : cfg.cur_len]])
        vt = np.concatenate([gv[0, kv].reshape(-1, cfg.d), V[0, kv, : cfg.k].reshape(-1, cfg.d),
                             V[0, kv, cfg.H, : cfg.cur_len]])
        bias = np.zeros(len(kt))
        bias[cfg.H * cfg.g: cfg.H * cfg.g + cfg.k * cfg.C] = gamma
        o, l = sdpa(q[0, h], kt, vt, bias)
        assert np.abs(r.out[0, h] - o).max() < TOL
        assert abs(r.lse[0, h] - l) < TOL


def pin_token_counts():
    """Softmax-set sizes: (M-1) g gists + k_eff C raw + the current chunk; raw tokens only
    without gists; at two levels nG g + |candidates| g + k_eff C + current."""
    cfg = SMALL.with_(B=1)
    inp = make_decode(cfg, seed=15)
    r = oracle_decode(inp)
    assert (r.n_tokens == cfg.H * cfg.g + cfg.k * cfg.C + cfg.cur_len).all()
    r = oracle_decode(inp, gists_in_softmax=False)
    assert (r.n_tokens == cfg.k * cfg.C + cfg.cur_len).all()
    r = oracle_decode(inp, k=cfg.H + 5)
    assert (r.n_tokens == cfg.H * cfg.g + cfg.H * cfg.C + cfg.cur_len).all()
    inp2 = make_decode(SMALL_L2, seed=15)
    r2 = oracle_decode(inp2)
    c2 = SMALL_L2
    cand = sum(min(c2.H, (g + 1) * c2.J) - g * c2.J for g in r2.sel_groups[0, 0])
    assert (r2.n_tokens == c2.nG * c2.g + cand * c2.g + c2.k * c2.C + c2.cur_len).all()
    # the pages' per-step count: k selected gists + k*L raw when the set is k*(1 + L) (g = 1)
    assert oracle.token_count(N=8 * 10, C_=8, g=1, k_eff=3, gists_in_softmax=False) == 3 * 8 + 8


def pin_two_level_everything_selected_is_dense():
    c = SMALL_L2.with_(k2=SMALL_L2.nG, k=SMALL_L2.H)
    inp = make_decode(c, seed=16)
    r = oracle_decode(inp)
    K, V = _logical_kv(inp)
    q = f64(inp.q)
    for h in range(c.Hq):
        kt = np.concatenate([f64(inp.gist2_k)[0, 0].reshape(-1, c.d),
                             f64(inp.gist_k)[0, 0].reshape(-1, c.d),
                             K[0, 0].reshape(-1, c.d)[: c.N]])
        vt = np.concatenate([f64(inp.gist2_v)[0, 0].reshape(-1, c.d),
                             f64(inp.gist_v)[0, 0].reshape(-1, c.d),
                             V[0, 0].reshape(-1, c.d)[: c.N]])
        o, l = sdpa(q[0, h], kt, vt)
        assert np.abs(r.out[0, h] - o).max() < TOL
        assert abs(r.lse[0, h] - l) < TOL


def pin_two_level_all_groups_same_choice_as_one_level():
    c = SMALL_L2.with_(k2=SMALL_L2.nG)
    inp = make_decode(c, seed=17)
    r2 = oracle_decode(inp)
    r1 = oracle_decode(inp, levels=1, J=0, k2=0, gist2_k=None, gist2_v=None)
    assert np.array_equal(r1.sel, r2.sel)
    assert np.abs(r1.chunk_scores - r2.chunk_scores).max() < TOL


def pin_two_level_group_selection():
    """Level-2 selection on group scores with one gist and one head reduces to argsort."""
    c = SMALL_L2.with_(Hq=1, g=1, n_plant=2, plant_groups=1)
    inp = make_decode(c, seed=18)
    r = oracle_decode(inp)
    s2 = f64(inp.gist2_k)[0, 0, :, 0] @ f64(inp.q)[0, 0] / math.sqrt(c.d)
    assert np.abs(r.group_scores[0, 0] - s2).max() < TOL
    assert np.array_equal(r.sel_groups[0, 0], np.sort(np.argsort(-s2, kind="stable")[: c.k2]))
    members = {x for gr in r.sel_groups[0, 0] for x in range(gr * c.J, min(c.H, (gr + 1) * c.J))}
    assert set(r.sel[0, 0].tolist()) <= members
    assert np.isinf(r.chunk_scores[0, 0, [x for x in range(c.H) if x not in members]]).all()


def pin_brute_force_prefill():
    for gate in (0, 1):
        cfg = PF.with_(gate=gate)
        inp = make_prefill(cfg, seed=19)
        r = oracle_prefill(inp)
        o, l = brute_prefill(inp)
        assert np.abs(r.out - o).max() < TOL
        assert np.abs(r.lse - l).max() < TOL


def pin_prefill_dense_causal():
    """Gate off and k >= blocks: textbook causal attention (is_causal)."""
    cfg = PF.with_(gate=0, k=PF.nb)
    inp = make_prefill(cfg, seed=20)
    r = oracle_prefill(inp)
    q, k, v = (torch.from_numpy(f64(t)) for t in (inp.q, inp.k, inp.v))
    G = cfg.G
    k = k.repeat_interleave(G, 1)
    v = v.repeat_interleave(G, 1)
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()
    assert np.abs(r.out - o).max() < TOL
    lam = (q @ k.transpose(-1, -2)) / math.sqrt(cfg.d)
    lam = lam.masked_fill(torch.ones(cfg.T, cfg.T, dtype=torch.bool).triu(1), float("-inf"))
    assert np.abs(r.lse - torch.logsumexp(lam, -1).numpy()).max() < TOL


def pin_prefill_gate_block_bias():
    """Gate on and every earlier block kept: causal attention with an additive block bias of
    log_softmax over the selector row (torch.log_softmax), 0 on the diagonal block."""
    cfg = PF.with_(gate=1, k=PF.nb)
    inp = make_prefill(cfg, seed=21)
    r = oracle_prefill(inp)
    q, k, v = (torch.from_numpy(f64(t)) for t in (inp.q, inp.k, inp.v))
    G, nb, blk = cfg.G, cfg.nb, cfg.blk
    S = inp.S.double()
    for kv in range(cfg.Hkv):
        bias = torch.full((cfg.T, cfg.T), float("-inf"), dtype=torch.float64)
        for i in range(nb):
            rows = slice(i * blk, (i + 1) * blk)
            if i > 0:
                ls = torch.log_softmax(S[0, kv, i, :i], 0)
                bias[rows, : i * blk] = ls.repeat_interleave(blk)[None]
            bias[rows, rows] = torch.zeros(blk, blk, dtype=torch.float64).masked_fill(
                torch.ones(blk, blk, dtype=torch.bool).triu(1), float("-inf"))
        for h in range(kv * G, (kv + 1) * G):
            o = F.scaled_dot_product_attention(q[0, h][None], k[0, kv][None], v[0, kv][None],
                                               attn_mask=bias[None])[0].numpy()
            assert np.abs(r.out[0, h] - o).max() < TOL


def pin_prefill_selection_argsort():
    inp = make_prefill(PF.with_(k=3), seed=22)
    r = oracle_prefill(inp)
    S = inp.S.numpy()
    for kv in range(PF.Hkv):
        for i in range(PF.nb):
            want = np.sort(np.argsort(-S[0, kv, i, :i], kind="stable")[: min(3, i)])
            got = r.sel[0, kv, i]
            assert np.array_equal(got[: len(want)], want)
            assert (got[len(want):] == -1).all()


def pin_selected_gists_brute_force():
    """Token set of the selected chunks' gists + their raw tokens + the current chunk ("SSA",
    section 3.3), against the independent numpy evaluation, gate off and on."""
    for cfg in (SMALL, SMALL.with_(gate=1), SMALL_G1):
        inp = make_decode(cfg, seed=13, max_chunks=cfg.M + 1, extra_pages=1)
        r = oracle_decode(inp, gists_in_softmax="selected")
        o, l, s_ = brute_decode(inp, gists="selected")
        assert np.array_equal(r.sel, s_), cfg.name
        assert np.abs(r.out - o).max() < TOL, cfg.name
        assert np.abs(r.lse - l).max() < TOL, cfg.name


def pin_selected_gists_k_all_equals_all_gists():
    """With every chunk selected the selected-gist set is the whole cache again."""
    for gate in (0, 1):
        cfg = SMALL.with_(k=SMALL.H, gate=gate)
        inp = make_decode(cfg, seed=14)
        a = oracle_decode(inp, gists_in_softmax=True)
        b = oracle_decode(inp, gists_in_softmax="selected")
        assert np.abs(a.out - b.out).max() < TOL and np.abs(a.lse - b.lse).max() < TOL


def pin_selected_gists_k_zero_is_current_chunk():
    """No chunk selected: only the current chunk's raw tokens remain (textbook attention)."""
    cfg = SMALL.with_(k=0, B=1)
    inp = make_decode(cfg, seed=15)
    K, V = _logical_kv(inp)
    q = f64(inp.q)
    r = oracle_decode(inp, gists_in_softmax="selected")
    for h in range(cfg.Hq):
        kv = h // cfg.G
        o, l = sdpa(q[0, h], K[0, kv, cfg.H, : cfg.cur_len], V[0, kv, cfg.H, : cfg.cur_len])
        assert np.abs(r.out[0, h] - o).max() < TOL
        assert abs(r.lse[0, h] - l) < TOL


def pin_selected_gists_token_count_and_weights():
    """|V_t| = k (g + C) + |current chunk|, which is the page's k (1 + L) at g = 1 plus the
    current chunk; the weights sum to one with the gate inside the softmax."""
    assert oracle.token_count(N=100, C_=8, g=1, k_eff=4, gists_in_softmax="selected") == 4 * 9 + 4
    assert oracle.token_count(N=96, C_=8, g=3, k_eff=5, gists_in_softmax="selected") == 5 * 11 + 8
    cfg = SMALL.with_(gate=1, B=1)
    inp = make_decode(cfg, seed=16)
    cap = cfg.k * (cfg.g + cfg.C) + cfg.C
    r = oracle_decode(inp, gists_in_softmax="selected", weights_cap=cap)
    for h in range(cfg.Hq):
        n = r.n_tokens[0, h]
        assert n == cfg.k * (cfg.g + cfg.C) + cfg.cur_len
        w = r.weights[0, h, :n]
        assert abs(w.sum() - 1.0) < TOL and (w > 0).all()


def pin_selected_gists_two_level_brute_force():
    """Two levels, selected summaries: the chosen groups' meta-gists + the chosen chunks' gists
    and raw tokens + the current chunk ("SSA", section B.2: each level contributes its selected
    summaries and the bottom level the raw tokens), against the numpy evaluation."""
    for cfg in (SMALL_L2, SMALL_L2.with_(g=1, Hq=2, k2=3, k=7), SMALL_L2.with_(B=2, Hkv=2, J=3)):
        inp = make_decode(cfg, seed=21, max_chunks=cfg.M + 1, extra_pages=1)
        r = oracle_decode(inp, gists_in_softmax="selected")
        o, l, s_ = brute_decode(inp, gists="selected")
        assert np.array_equal(r.sel, s_), cfg.name
        assert np.abs(r.out - o).max() < TOL, cfg.name
        assert np.abs(r.lse - l).max() < TOL, cfg.name


def pin_selected_gists_two_level_everything_selected_is_dense():
    """Every group and every chunk chosen: the two-level selected set is the whole cache with
    all meta-gists and gists again (textbook attention over that set)."""
    c = SMALL_L2.with_(k2=SMALL_L2.nG, k=SMALL_L2.H)
    inp = make_decode(c, seed=22)
    r = oracle_decode(inp, gists_in_softmax="selected")
    K, V = _logical_kv(inp)
    q = f64(inp.q)
    kt = np.concatenate([f64(inp.gist2_k)[0, 0].reshape(-1, c.d),
                         f64(inp.gist_k)[0, 0].reshape(-1, c.d), K[0, 0].reshape(-1, c.d)[: c.N]])
    vt = np.concatenate([f64(inp.gist2_v)[0, 0].reshape(-1, c.d),
                         f64(inp.gist_v)[0, 0].reshape(-1, c.d), V[0, 0].reshape(-1, c.d)[: c.N]])
    for h in range(c.Hq):
        o, l = sdpa(q[0, h], kt, vt)
        assert np.abs(r.out[0, h] - o).max() < TOL
        assert abs(r.lse[0, h] - l) < TOL


def pin_selected_gists_two_level_count_and_weights():
    """|V_t| = k2 g + k (g + C) + |current chunk| at two levels; weights sum to one."""
    assert oracle.token_count(N=100, C_=8, g=2, k_eff=4, levels=2, J=3, k2_eff=2,
                              gists_in_softmax="selected") == 2 * 2 + 4 * 10 + 4
    c = SMALL_L2
    inp = make_decode(c, seed=23)
    cap = c.k2 * c.g + c.k * (c.g + c.C) + c.C
    r = oracle_decode(inp, gists_in_softmax="selected", weights_cap=cap)
    for h in range(c.Hq):
        n = r.n_tokens[0, h]
        assert n == c.k2 * c.g + c.k * (c.g + c.C) + c.cur_len
        w = r.weights[0, h, :n]
        assert abs(w.sum() - 1.0) < TOL and (w > 0).all()
    # a chosen group's meta-gists are present: an exact reconstruction of the output from the
    # weights over the materialised set, meta-gists first in chosen-group order
    K, V = _logical_kv(inp)
    g2v, gv = f64(inp.gist2_v)[0, 0], f64(inp.gist_v)[0, 0]
    groups, sel = r.sel_groups[0, 0], r.sel[0, 0]
    vt = np.concatenate([g2v[groups].reshape(-1, c.d)] +
                        [np.concatenate([gv[x], V[0, 0, x]]) for x in sel] +
                        [V[0, 0, c.H, : c.cur_len]])
    for h in range(c.Hq):
        n = r.n_tokens[0, h]
        assert np.abs(r.weights[0, h, :n] @ vt - r.out[0, h]).max() < 1e-10


def pin_head_select_brute_force():
    """Per-head selection (SSA appendix A: each head selects on its own, the union is unfolded
    into the shared KV) against the numpy evaluation, with every gist and with the selected
    gists; the per-head scores against their definition."""
    for cfg, gm in ((SMALL, True), (SMALL.with_(Hq=8, k=2), "selected"), (SMALL_G1, True),
                    (SMALL.with_(Hq=8, g=1, k=4), True)):
        inp = make_decode(cfg, seed=31, max_chunks=cfg.M + 1, extra_pages=1)
        r = oracle_decode(inp, head_select=1, gists_in_softmax=gm)
        o, l, s_ = brute_decode(inp, gists=gm, head_select=True)
        assert r.sel.shape[-1] == cfg.G * cfg.k
        assert np.array_equal(r.sel, s_), cfg.name
        assert np.abs(r.out - o).max() < TOL, cfg.name
        assert np.abs(r.lse - l).max() < TOL, cfg.name
        q, gk = f64(inp.q), f64(inp.gist_k)
        for b in range(cfg.B):
            for h in range(cfg.Hq):
                want = [_lse(gk[b, h // cfg.G, x] @ q[b, h] / math.sqrt(cfg.d)) for x in range(cfg.H)]
                assert np.abs(r.chunk_scores[b, h] - want).max() < TOL


def pin_head_select_one_head_per_group_is_kv_select():
    """G = 1: a head's own score is the pooled score, so per-head selection is the KV-head
    selection."""
    cfg = SMALL.with_(Hq=2, Hkv=2)
    inp = make_decode(cfg, seed=32)
    a = oracle_decode(inp)
    b = oracle_decode(inp, head_select=1)
    assert np.array_equal(a.sel, b.sel)
    assert np.abs(a.out - b.out).max() < TOL and np.abs(a.lse - b.lse).max() < TOL


def pin_head_select_shared_query():
    """Every head of a group with the same query: the heads pick the same chunks, so the union
    is one head's top-k, which ranks like the pooled score (pooled = own score + log G)."""
    cfg = SMALL.with_(Hq=8)
    inp = make_decode(cfg, seed=33)
    q = inp.q.view(cfg.B, cfg.Hkv, cfg.G, cfg.d)
    q[:] = q[:, :, :1, :].clone()
    a = oracle_decode(inp)
    b = oracle_decode(inp, head_select=1)
    assert np.array_equal(b.sel[..., : cfg.k], a.sel) and (b.sel[..., cfg.k:] == -1).all()
    assert np.abs(a.out - b.out).max() < TOL
    assert np.abs(b.chunk_scores.reshape(cfg.B, cfg.Hkv, cfg.G, -1)[:, :, 0] + math.log(cfg.G)
                  - a.chunk_scores).max() < 1e-10


def pin_head_select_union_bounds_and_dense():
    """k_eff <= |union| <= min(G k, H), ascending; each head's own argsort top-k (g = 1) is in
    the union; with k = all the set is the whole cache (textbook attention)."""
    cfg = SMALL.with_(Hq=8, g=1, k=3, B=1)
    inp = make_decode(cfg, seed=34)
    r = oracle_decode(inp, head_select=1)
    q, gk = f64(inp.q), f64(inp.gist_k)
    for kv in range(cfg.Hkv):
        u = r.sel[0, kv][r.sel[0, kv] >= 0]
        assert cfg.k <= len(u) <= min(cfg.G * cfg.k, cfg.H) and (np.diff(u) > 0).all()
        for h in range(kv * cfg.G, (kv + 1) * cfg.G):
            s = gk[0, kv, :, 0] @ q[0, h]
            assert set(np.argsort(-s, kind="stable")[: cfg.k]) <= set(u.tolist())
    c = SMALL.with_(k=SMALL.H, B=1)
    inp = make_decode(c, seed=35)
    r = oracle_decode(inp, head_select=1)
    K, V = _logical_kv(inp)
    q = f64(inp.q)
    for h in range(c.Hq):
        kv = h // c.G
        kt = np.concatenate([f64(inp.gist_k)[0, kv].reshape(-1, c.d), K[0, kv].reshape(-1, c.d)[: c.N]])
        vt = np.concatenate([f64(inp.gist_v)[0, kv].reshape(-1, c.d), V[0, kv].reshape(-1, c.d)[: c.N]])
        o, l = sdpa(q[0, h], kt, vt)
        assert np.abs(r.out[0, h] - o).max() < TOL and abs(r.lse[0, h] - l) < TOL


def pin_top_p_brute_force():
    """Top-p with a cap of k chunks: the shortest ranked prefix whose share of the softmax over
    all historical chunk scores reaches p, against the numpy evaluation."""
    for cfg, tp in ((SMALL.with_(k=12), 0.3), (SMALL.with_(k=12, gate=1), 0.8),
                    (SMALL_G1.with_(k=25), 0.55), (SMALL.with_(k=2), 0.95)):
        inp = make_decode(cfg, seed=17)
        r = oracle_decode(inp, top_p=tp)
        o, l, s_ = brute_decode(inp, top_p=tp)
        assert np.array_equal(r.sel, s_), (cfg.name, tp)
        assert np.abs(r.out - o).max() < TOL and np.abs(r.lse - l).max() < TOL


def pin_top_p_one_is_top_k():
    cfg = SMALL.with_(k=7, gate=1)
    inp = make_decode(cfg, seed=18)
    a, b = oracle_decode(inp), oracle_decode(inp, top_p=1.0)
    assert np.array_equal(a.sel, b.sel) and np.abs(a.out - b.out).max() == 0.0


def pin_top_p_equal_scores_closed_form():
    """All chunk scores equal: each chunk holds 1/|H| of the mass, so top-p keeps the
    ceil(p |H|) lowest-index chunks (|H| = 21: p = 0.3 -> 7, p = 0.5 -> 11), capped at k;
    a tiny p keeps exactly one chunk."""
    cfg = SMALL.with_(B=1, k=30, N=22 * 8)
    inp = make_decode(cfg, seed=19)
    from dataclasses import replace
    gk = inp.gist_k.clone()
    gk[:] = gk[:, :, :1]
    inp2 = replace(inp, gist_k=gk)
    assert cfg.H == 21
    for tp, want in ((0.3, 7), (0.5, 11), (1e-9, 1)):
        r = oracle_decode(inp2, top_p=tp)
        for kv in range(cfg.Hkv):
            assert r.sel[0, kv].tolist() == list(range(want)) + [-1] * (cfg.k - want), (tp, kv)
    r = oracle_decode(inp2, top_p=0.5, k=4)
    assert r.sel[0, 0].tolist() == [0, 1, 2, 3]


def pin_top_p_two_levels_all_groups_is_one_level():
    """Two levels with every group chosen: the candidates are all historical chunks, so top-p
    keeps what it keeps at one level (the two softmax sets differ by the level-2 gists only)."""
    cfg = SMALL_L2.with_(k=12)
    inp = make_decode(cfg, seed=21)
    kept = set()
    for tp in (0.2, 0.6, 0.97):
        two = oracle_decode(inp, top_p=tp, k2=cfg.nG)
        one = oracle_decode(inp, top_p=tp, levels=1)
        assert np.array_equal(two.sel, one.sel), tp
        kept.add(int((two.sel >= 0).sum()))
    assert len(kept) > 1   # the cut, not only the cap, decides


def pin_top_p_two_levels_one_is_top_k():
    cfg = SMALL_L2.with_(k=6)
    inp = make_decode(cfg, seed=22)
    a, b = oracle_decode(inp), oracle_decode(inp, top_p=1.0)
    assert np.array_equal(a.sel, b.sel) and np.array_equal(a.sel_groups, b.sel_groups)
    assert np.abs(a.out - b.out).max() == 0.0


def pin_top_p_two_levels_over_candidates():
    """Two levels, two of ten groups chosen: the shares are those of the softmax over the
    chosen groups' member chunks, the only chunks scored.  A tiny p keeps the best candidate;
    p = 0.5 keeps the shortest ranked prefix of candidates reaching half their mass (numpy),
    which differs from the prefix over all historical chunks' scores."""
    cfg = SMALL_L2.with_(k=8)
    inp = make_decode(cfg, seed=23)
    r = oracle_decode(inp, top_p=0.5)
    full = oracle_decode(inp, k=cfg.H, levels=1)   # every chunk's score, no groups
    cand = [c for grp in r.sel_groups[0, 0] if grp >= 0
            for c in range(grp * cfg.J, min((grp + 1) * cfg.J, cfg.H))]
    sc = full.chunk_scores[0, 0]
    assert np.array_equal(r.chunk_scores[0, 0][cand], sc[cand])
    assert np.isinf(np.delete(r.chunk_scores[0, 0], cand)).all()

    def prefix(ids, p):
        order = sorted(ids, key=lambda c: (-sc[c], c))
        sh = np.exp(sc[order] - np.logaddexp.reduce(sc[ids]))
        n = int(np.argmax(np.cumsum(sh) >= p)) + 1
        return sorted(order[:min(n, cfg.k)])

    want = prefix(cand, 0.5)
    got = [c for c in r.sel[0, 0].tolist() if c >= 0]
    assert got == want and 1 < len(got) < cfg.k
    assert prefix(list(range(cfg.H)), 0.5) != want
    tiny = oracle_decode(inp, top_p=1e-12)
    best = max(cand, key=lambda c: (sc[c], -c))
    assert tiny.sel[0, 0].tolist() == [best] + [-1] * (cfg.k - 1)


def pin_top_p_tiny_is_argmax():
    cfg = SMALL.with_(k=5)
    inp = make_decode(cfg, seed=20)
    r = oracle_decode(inp, top_p=1e-12)
    full = oracle_decode(inp, k=cfg.H)
    for b in range(cfg.B):
        for kv in range(cfg.Hkv):
            sc = full.chunk_scores[b, kv]
            best = int(np.argmax(sc))   # first maximum: lowest index on ties
            assert r.sel[b, kv].tolist() == [best] + [-1] * (cfg.k - 1)


# ----------------------------------------------------------------------------------------
# adaptive top-k (SSA appendix A).  The appendix names the budget's ingredients and its
# properties but prints no formula and no values, so only those properties are pinned here:
# at least one chunk; grows with the KV positions n_kv; divided among the G heads whose picks
# are unioned; unfolded raw tokens proportional to n_kv with the effective compression L_eff
# = L (one level) or L J (two levels); the same budget at both levels.
# ----------------------------------------------------------------------------------------
def _budget(N, C_, G, levels=1, J=0):
    return oracle.adaptive_k_budget(N=N, C_=C_, Hq=8 * G, Hkv=8, levels=levels, J=J)


def pin_adaptive_k_stated_properties():
    for C_ in (8, 64, 128):
        for levels, J in ((1, 0), (2, 4), (2, 16)):
            l_eff = C_ * (J if levels == 2 else 1)
            for G in (1, 2, 4, 8):
                prev = 0
                for N in sorted({1, 2, C_, C_ + 1, l_eff * G * C_ - 1, l_eff * G * C_,
                                 3 * l_eff * G * C_ + 7, 131072, 524288, 1 << 21}):
                    b = _budget(N, C_, G, levels, J)
                    assert b >= 1, (C_, levels, J, G, N)            # at least one chunk
                    assert b >= prev, (C_, levels, J, G, N)         # grows with n_kv
                    prev = b
                    # the G heads' picks together unfold G k chunks of L tokens: within one
                    # chunk per head of the n_kv / L_eff positions of the compressed cache
                    assert G * (b - 1) * C_ <= N / l_eff < G * b * C_, (C_, levels, J, G, N)
                    # dividing by G: the group's budget, G times its per-head share, stays within
                    # G - 1 chunks of the budget one head alone would get
                    one = _budget(N, C_, 1, levels, J)
                    assert G * (b - 1) <= one - 1 < G * b, (C_, levels, J, G, N)
    # proportional to n_kv: doubling a large cache doubles the unfolded tokens (to one chunk)
    for levels, J in ((1, 0), (2, 16)):
        a, b2 = _budget(1 << 20, 64, 4, levels, J), _budget(1 << 21, 64, 4, levels, J)
        assert abs((b2 - 1) - 2 * (a - 1)) <= 1


def pin_adaptive_k_reduces_to_fixed_k():
    """With the budget b, adaptive decode selects exactly what fixed k = min(cap, b) (and
    k2 = min(k2 cap, b) at two levels) selects, bit for bit, and the same budget serves both
    levels."""
    one = SMALL.with_(gate=1, k=6)                       # b = 173 // (8 * 2 * 8) + 1 = 2
    two = SMALL_L2.with_(N=130 * 8 + 3, k=6, k2=5)       # b = 1043 // (32 * 4 * 8) + 1 = 2
    cases = ((one, {}), (one.with_(k=1), {}), (SMALL.with_(k=5, gate=0), {"head_select": 1}),
             (two, {}), (two.with_(k2=1), {}))
    for cfg, kw in cases:
        inp = make_decode(cfg, seed=41)
        b = _budget(cfg.N, cfg.C, cfg.G, cfg.levels, cfg.J)
        assert b == 2, cfg.name
        r = oracle_decode(inp, adaptive_k=1, **kw)
        k1 = min(cfg.k, b)
        lv = {"k2": min(cfg.k2, b)} if cfg.levels == 2 else {}
        ref = oracle_decode(inp, k=k1, **lv, **kw)
        G = cfg.G if kw.get("head_select") else 1
        assert r.sel.shape[-1] == G * cfg.k      # the caller's stride is kept
        pad = np.full(r.sel.shape, -1, np.int32)
        pad[..., : G * k1] = ref.sel
        assert np.array_equal(r.sel, pad), cfg.name
        assert np.array_equal(r.out, ref.out) and np.array_equal(r.lse, ref.lse), cfg.name
        if cfg.levels == 2:
            gpad = np.full(r.sel_groups.shape, -1, np.int32)
            gpad[..., : lv["k2"]] = ref.sel_groups
            assert np.array_equal(r.sel_groups, gpad), cfg.name
            k2e = min(cfg.k2, b, cfg.nG)
            assert ((r.sel_groups >= 0).sum(-1) == k2e).all()
            if cfg.k2 >= b and cfg.k >= b:       # the same budget at both levels
                assert ((r.sel >= 0).sum(-1) == b).all() and k2e == b
        elif not kw:
            assert ((r.sel >= 0).sum(-1) == min(cfg.k, b, cfg.H)).all()


# ----------------------------------------------------------------------------------------
# prefill backward
# ----------------------------------------------------------------------------------------
PFB = PrefillConfig("pin_prefill_bwd", B=1, Hq=4, Hkv=2, d=16, T=8 * 6, blk=8, k=2, gate=1)


def torch_prefill_grads(inp, dout, dlse, sel):
    """The prefill written densely in torch float64 (a [T][T] mask with the gate bias of every
    chosen block built from log_softmax(S[i][:i])), differentiated by autograd."""
    c = inp.cfg
    G, blk, nb, T = c.G, c.blk, c.nb, c.T
    q = torch.tensor(f64(inp.q), requires_grad=True)
    k = torch.tensor(f64(inp.k), requires_grad=True)
    v = torch.tensor(f64(inp.v), requires_grad=True)
    S = torch.tensor(inp.S.double().numpy(), requires_grad=True)
    bias = torch.full((c.B, c.Hkv, T, T), -math.inf, dtype=torch.float64)
    for b in range(c.B):
        for kv in range(c.Hkv):
            for i in range(nb):
                rows = slice(i * blk, (i + 1) * blk)
                if i > 0 and c.k > 0:
                    g = torch.log_softmax(S[b, kv, i, :i], 0)
                    for j in sel[b, kv, i]:
                        if j >= 0:
                            val = g[j] if c.gate else torch.zeros((), dtype=torch.float64)
                            bias[b, kv, rows, j * blk:(j + 1) * blk] = val
                diag = torch.zeros(blk, blk, dtype=torch.float64)
                diag[torch.triu(torch.ones(blk, blk, dtype=torch.bool), 1)] = -math.inf
                bias[b, kv, rows, rows] = diag
    qg = q.view(c.B, c.Hkv, G, T, c.d)
    lam = torch.matmul(qg, k.unsqueeze(2).transpose(-1, -2)) / math.sqrt(c.d) + bias.unsqueeze(2)
    lse = torch.logsumexp(lam, -1)
    out = torch.matmul(torch.softmax(lam, -1), v.unsqueeze(2))
    loss = (out.reshape(c.B, c.Hq, T, c.d) * torch.tensor(f64(dout))).sum()
    if dlse is not None:
        loss = loss + (lse.reshape(c.B, c.Hq, T) * dlse.double()).sum()
    loss.backward()
    dS = S.grad.numpy() if S.grad is not None else np.zeros(S.shape)   # S unused: no gradient
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), dS


def pin_prefill_backward_autograd():
    """Every gradient against torch autograd of the dense float64 formulation (gate on and off,
    with and without dlse, k = 0)."""
    for cfg, with_dlse in ((PFB, True), (PFB.with_(gate=0), True), (PFB, False),
                           (PFB.with_(k=0), True), (PFB.with_(k=4, Hq=2), True)):
        inp = make_prefill(cfg, seed=41)
        dout, dlse = make_prefill_grads(cfg, seed=41)
        dlse = dlse if with_dlse else None
        r = oracle_prefill_backward(inp, dout, dlse)
        sel = oracle_prefill(inp).sel
        dq, dk, dv, dS = torch_prefill_grads(inp, dout, dlse, sel)
        for name, a, b in (("dq", r.dq, dq), ("dk", r.dk, dk), ("dv", r.dv, dv), ("dS", r.dS, dS)):
            assert np.abs(a - b).max() < 1e-10 * max(1.0, np.abs(b).max()), (cfg.name, name)


def pin_prefill_backward_finite_differences_S():
    """dL/dS against central differences of the oracle forward (L = sum dout . out + sum dlse .
    lse), at entries whose perturbation leaves the selection unchanged."""
    cfg = PFB
    inp = make_prefill(cfg, seed=42)
    dout, dlse = make_prefill_grads(cfg, seed=42)
    r = oracle_prefill_backward(inp, dout, dlse)
    go, gl = f64(dout), dlse.double().numpy()
    base = oracle_prefill(inp)
    S0 = inp.S.clone()
    rng = np.random.default_rng(0)
    checked = 0
    for _ in range(12):
        i = int(rng.integers(1, cfg.nb))
        j = int(rng.integers(0, i))
        kv = int(rng.integers(0, cfg.Hkv))
        vals = []
        for sgn in (1.0, -1.0):
            inp.S = S0.clone()
            inp.S[0, kv, i, j] = float(np.float32(S0[0, kv, i, j].item() + sgn * 2.0 ** -9))
            f = oracle_prefill(inp)
            if not np.array_equal(f.sel, base.sel):
                vals = None
                break
            vals.append(((f.out * go).sum() + (f.lse * gl).sum(), inp.S[0, kv, i, j].item()))
        inp.S = S0
        if vals is None:
            continue
        fd = (vals[0][0] - vals[1][0]) / (vals[0][1] - vals[1][1])
        assert abs(fd - r.dS[0, kv, i, j]) < 1e-5 * max(1.0, abs(fd)), (i, j, fd, r.dS[0, kv, i, j])
        checked += 1
    assert checked >= 8


def pin_prefill_backward_closed_forms():
    """Every query row's weights sum to one, so per KV head the dv rows add up to the group's
    dout rows and the dk rows to sigma * sum dlse * q; with the gate, each dS row sums to zero
    (the log-softmax Jacobian); without it dS is zero."""
    cfg = PFB.with_(k=3)
    inp = make_prefill(cfg, seed=43)
    dout, dlse = make_prefill_grads(cfg, seed=43)
    r = oracle_prefill_backward(inp, dout, dlse)
    go, q = f64(dout), f64(inp.q)
    gl = dlse.double().numpy()
    sig = 1.0 / math.sqrt(cfg.d)
    for kv in range(cfg.Hkv):
        hs = slice(kv * cfg.G, (kv + 1) * cfg.G)
        assert np.abs(r.dv[0, kv].sum(0) - go[0, hs].sum((0, 1))).max() < 1e-9
        want_dk = sig * (gl[0, hs, :, None] * q[0, hs]).sum((0, 1))
        assert np.abs(r.dk[0, kv].sum(0) - want_dk).max() < 1e-9
    assert np.abs(r.dS.sum(-1)).max() < 1e-10
    assert np.abs(np.triu(r.dS[0, 0])).max() == 0.0
    r0 = oracle_prefill_backward(make_prefill(cfg.with_(gate=0), seed=43), dout, dlse)
    assert (r0.dS == 0).all()


# ----------------------------------------------------------------------------------------
# SSA gist-masked prefill
# ----------------------------------------------------------------------------------------
GP = GistPrefillConfig("pin_gist_prefill", B=1, Hq=4, Hkv=2, d=16, M=5, L=6, g=2)


def dense_masked(q, k, v, allowed):
    """Textbook attention of every row over the keys its mask row allows (float64)."""
    lam = q @ k.T / math.sqrt(q.shape[-1])
    lam = np.where(allowed, lam, -np.inf)
    m = lam.max(-1, keepdims=True)
    w = np.exp(lam - m)
    return (w @ v) / w.sum(-1, keepdims=True), (m + np.log(w.sum(-1, keepdims=True)))[:, 0]


def pin_gist_prefill_dense_mask():
    """Against dense attention under the mask of section 3.1, built as a [T'][T'] boolean array
    from chunk ids and gist flags (causal, and same chunk or gist key), G = 1 and 2, g = 1..3."""
    for cfg in (GP, GP.with_(Hq=2, g=1, L=7), GP.with_(g=3, L=4, M=6)):
        inp = make_gist_prefill(cfg, seed=51)
        out, lse = oracle_gist_prefill(inp)
        pos = np.arange(cfg.Tp)
        chunk, gist = pos // cfg.W, (pos % cfg.W) >= cfg.L
        allowed = (pos[None, :] <= pos[:, None]) & ((chunk[None, :] == chunk[:, None]) | gist[None, :])
        q, k, v = f64(inp.q), f64(inp.k), f64(inp.v)
        for h in range(cfg.Hq):
            o, l = dense_masked(q[0, h], k[0, h // cfg.G], v[0, h // cfg.G], allowed)
            assert np.abs(out[0, h] - o).max() < TOL and np.abs(lse[0, h] - l).max() < TOL


def pin_gist_prefill_special_cases():
    """One chunk: causal attention over the chunk (torch sdpa); no gists: each chunk causal on
    its own (block-diagonal)."""
    for cfg in (GP.with_(M=1), GP.with_(g=0)):
        inp = make_gist_prefill(cfg, seed=52)
        out, lse = oracle_gist_prefill(inp)
        q, k, v = (torch.tensor(f64(t)) for t in (inp.q, inp.k, inp.v))
        for h in range(cfg.Hq):
            for c in range(cfg.M):
                rs = slice(c * cfg.W, (c + 1) * cfg.W)
                want = F.scaled_dot_product_attention(q[0, h, rs][None], k[0, h // cfg.G, rs][None],
                                                      v[0, h // cfg.G, rs][None], is_causal=True)[0]
                assert np.abs(out[0, h, rs] - want.numpy()).max() < TOL


def pin_gist_prefill_bottleneck():
    """Later tokens reach a chunk only through its gists: new raw K/V in chunk 1 change no output
    outside chunk 1 (bitwise) but do change chunk 1's own later rows; new gist K/V of chunk 1
    change the outputs of later chunks."""
    cfg = GP
    inp = make_gist_prefill(cfg, seed=53)
    base, _ = oracle_gist_prefill(inp)
    raw = slice(1 * cfg.W, 1 * cfg.W + cfg.L)
    k0, v0 = inp.k.clone(), inp.v.clone()
    inp.k[:, :, raw] = -inp.k[:, :, raw]
    inp.v[:, :, raw] = inp.v[:, :, raw] * 2
    out, _ = oracle_gist_prefill(inp)
    outside = np.r_[0:cfg.W, 2 * cfg.W:cfg.Tp]
    assert np.array_equal(out[:, :, outside], base[:, :, outside])
    assert np.abs(out[:, :, raw] - base[:, :, raw]).max() > 1e-3
    inp.k, inp.v = k0.clone(), v0.clone()
    gist = slice(1 * cfg.W + cfg.L, 2 * cfg.W)
    inp.v[:, :, gist] = inp.v[:, :, gist] * 3
    out, _ = oracle_gist_prefill(inp)
    assert np.array_equal(out[:, :, : 1 * cfg.W + cfg.L], base[:, :, : 1 * cfg.W + cfg.L])
    assert np.abs(out[:, :, 2 * cfg.W:] - base[:, :, 2 * cfg.W:]).max() > 1e-3


PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_forced_selection_matches_free_selection():
    inp = make_decode(SMALL.with_(gate=1), seed=23)
    r = oracle_decode(inp)
    r2 = oracle_decode(inp, forced_sel=np.ascontiguousarray(r.sel))
    assert np.array_equal(r.out, r2.out)
    pin = make_prefill(PF, seed=24)
    p1 = oracle_prefill(pin)
    p2 = oracle_prefill(pin, forced_sel=np.ascontiguousarray(p1.sel))
    assert np.array_equal(p1.out, p2.out)


def test_unit_subset():
    inp = make_decode(SMALL, seed=25)
    r = oracle_decode(inp)
    r2 = oracle_decode(inp, units=[3, 0])
    for u in (0, 3):
        b, kv = divmod(u, SMALL.Hkv)
        G = SMALL.G
        assert np.array_equal(r.out[b, kv * G:(kv + 1) * G], r2.out[b, kv * G:(kv + 1) * G])
    assert np.isnan(r2.out[0, 2]).all()


def test_bad_page_gives_nan():
    inp = make_decode(SMALL, seed=26)
    r = oracle_decode(inp)
    pt = inp.page_table.clone()
    pt[1, r.sel[1, 0, 0]] = 10 ** 6
    from dataclasses import replace
    r2 = oracle_decode(replace(inp, page_table=pt))
    G = SMALL.G
    assert np.isnan(r2.out[1, :G]).all() and np.isnan(r2.lse[1, :G]).all()
    assert not np.isnan(r2.out[0]).any()
