"""Plants plausible mistakes in copies of oracle.c (CPU only) and checks that the pins catch
every one: a dropped term, a wrong sign, a wrong pooling, a reversed tie-break, an off-by-one
window.  The default oracle build is untouched; each mutant is compiled into a temp dir."""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, mutated text) -- each original must occur exactly once
MUTANTS = [
    ("gate_sign", "gamma = s[j] - lse_s;", "gamma = lse_s - s[j];"),
    ("gate_unnormalised", "gamma = s[j] - lse_s;", "gamma = s[j];"),
    ("max_pooling",
     "    double s = logsumexp(l, G * g);\n",
     "    double s = l[0]; for (int x = 1; x < G * g; ++x) if (l[x] > s) s = l[x];\n"),
    ("tie_break_highest", "return (x->c > y->c) - (x->c < y->c);",
     "return (x->c < y->c) - (x->c > y->c);"),
    ("drop_current_chunk", "for (int u = 0; u < cur; ++u) {", "for (int u = 0; u < 0; ++u) {"),
    ("drop_gists", "    if (p->gists_in_softmax == 1) {\n        if (p->levels == 2)\n            for",
     "    if (0) {\n        if (p->levels == 2)\n            for"),
    ("diag_not_causal", "for (int u = i * blk; u <= pos; ++u) {\n                tk[n].k",
     "for (int u = i * blk; u < (i + 1) * blk; ++u) {\n                tk[n].k"),
    ("diag_off_by_one", "for (int u = i * blk; u <= pos; ++u) {\n                tk[n].k",
     "for (int u = i * blk; u < pos; ++u) {\n                tk[n].k"),
    ("prefill_gate_wrong_row", "double gamma = p->gate ? (double)Srow[j] - lse_s : 0.0;",
     "double gamma = p->gate ? (double)io->S[(unit * nb + j) * nb + i] - lse_s : 0.0;"),
    ("scale_missing", "    return sigma * s;\n}", "    return s;\n}"),
    ("lse_log2", "    return m + log(z);\n}\n\ntypedef struct { double s; int c; } scored;",
     "    return m + log2(z);\n}\n\ntypedef struct { double s; int c; } scored;"),
    ("top_k_off_by_one", "    int ke = k < n ? k : n;", "    int ke = k < n ? k - 1 : n;"),
    ("prefill_sees_diagonal_in_selection", "for (int j = 0; j < i; ++j) { s[j]",
     "for (int j = 0; j < i; ++j) { s[j] = (double)Srow[j + 1]; ids[j] = j; } for (int j = 0; j < 0; ++j) { s[j]"),
    ("weights_transposed_v", "o[i] += w * bf(t[x].v[i]);", "o[i] += w * bf(t[x].k[i]);"),
    ("top_p_cap_off_by_one", "    int ke = r < k ? r : k;\n    for (int i = 0; i < ke; ++i) chosen[i] = v[i].c;\n    qsort(chosen, (size_t)ke, sizeof(int), ascending);\n    free(v);\n    return ke;\n}\n\n/* Pooled",
     "    int ke = r < k ? r : k - 1;\n    for (int i = 0; i < ke; ++i) chosen[i] = v[i].c;\n    qsort(chosen, (size_t)ke, sizeof(int), ascending);\n    free(v);\n    return ke;\n}\n\n/* Pooled"),
    ("top_p_unranked", "    qsort(v, (size_t)n, sizeof(scored), by_rank);\n    const double lse = logsumexp(s, n);",
     "    const double lse = logsumexp(s, n);"),
    ("top_p_shares_of_first_half", "    const double lse = logsumexp(s, n);", "    const double lse = logsumexp(s, (n + 1) / 2);"),
    # at two levels top-p silently falls back to the top-k chunk choice
    ("top_p_one_level_only", "    } else if (p->top_p > 0.0) {\n        ke = top_p(",
     "    } else if (p->top_p > 0.0 && p->levels == 1) {\n        ke = top_p("),
    ("selected_gists_first_only", "tk[n].k = gk + ((size_t)c * g + t) * d;",
     "tk[n].k = gk + ((size_t)c * g + 0) * d;"),
    ("selected_gists_gated", "                tk[n].v = gv + ((size_t)c * g + t) * d;\n                tk[n++].bias = 0.0;",
     "                tk[n].v = gv + ((size_t)c * g + t) * d;\n                tk[n++].bias = p->gate ? 0.5 : 0.0;"),
    ("selected_meta_gists_dropped", "        for (int i = 0; i < k2e; ++i)\n            for (int t = 0; t < g; ++t) {",
     "        for (int i = 0; i < 0; ++i)\n            for (int t = 0; t < g; ++t) {"),
    ("selected_meta_gists_by_position", "tk[n].k = g2k + ((size_t)groups[i] * g + t) * d;",
     "tk[n].k = g2k + ((size_t)i * g + t) * d;"),
    ("head_select_first_head_only", "        for (int h = 0; h < G; ++h) {\n            for (int i = 0; i < n_cand; ++i) {\n                sh[i]",
     "        for (int h = 0; h < 1; ++h) {\n            for (int i = 0; i < n_cand; ++i) {\n                sh[i]"),
    ("head_select_pooled_score", "sh[i] = pooled_score(qg + (size_t)h * d, 1,", "sh[i] = pooled_score(qg, G,"),
    ("head_select_last_pick_dropped", "for (int j = 0; j < kh; ++j) in_union[pick[j]] = 1;",
     "for (int j = 0; j + 1 < kh; ++j) in_union[pick[j]] = 1;"),
    ("bwd_drop_D", "const double dl = lam[x] * (dP - D);", "const double dl = lam[x] * dP;"),
    ("bwd_gate_jacobian_sign", "dS[j] = -exp(sc[j] - norm) * tot;", "dS[j] = exp(sc[j] - norm) * tot;"),
    ("bwd_dk_unscaled", "dK[(size_t)key[x] * d + e] += sigma * dl * bf(qr[e]);",
     "dK[(size_t)key[x] * d + e] += dl * bf(qr[e]);"),
    ("bwd_dv_from_dlambda", "dV[(size_t)key[x] * d + e] += lam[x] * bf(gr[e]);",
     "dV[(size_t)key[x] * d + e] += dl * bf(gr[e]);"),
    ("bwd_dlse_ignored", "double D = io->dlse ? -(double)io->dlse[qrow] : 0.0;", "double D = 0.0;"),
    ("bwd_diag_noncausal", "for (int u = i * blk; u <= pos; ++u) {\n                    key[n] = u;",
     "for (int u = i * blk; u < (i + 1) * blk; ++u) {\n                    key[n] = u;"),
    ("gist_prefill_raw_leak", "if (cx == cp || is_gist) {", "if (1) {"),
    ("gist_prefill_no_earlier_gists", "if (cx == cp || is_gist) {", "if (cx == cp) {"),
    ("gist_prefill_first_gist_as_raw", "const int is_gist = (x % W) >= p->L;",
     "const int is_gist = (x % W) > p->L;"),
    ("adaptive_k_no_plus_one", "return (int)((long long)p->N / (l_eff * G * p->C)) + 1;",
     "return (int)((long long)p->N / (l_eff * G * p->C));"),
    ("adaptive_k_not_divided_by_group", "return (int)((long long)p->N / (l_eff * G * p->C)) + 1;",
     "return (int)((long long)p->N / (l_eff * p->C)) + 1;"),
    ("adaptive_k_two_levels_compress_like_one",
     "p->levels == 2 ? (long long)p->C * p->J : (long long)p->C;", "(long long)p->C;"),
    ("adaptive_k_groups_not_adapted", "        if (ka < k2) k2 = ka;\n", ""),
    ("adaptive_k_ignored", "        if (ka < k1) k1 = ka;\n", ""),
]


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/missing"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-w",
                           "-I", os.path.dirname(SRC), "-o", str(so), str(path), "-lm"])
    return str(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    so = _build(tmp_path, name, old, new)
    prev = oracle.swap_library(so)
    caught = []
    try:
        for pin in pins.PINS:
            try:
                pin()
            except Exception:  # any failure of a pin counts as caught
                caught.append(pin.__name__)
    finally:
        oracle.swap_library(None)
        if prev is not None:
            oracle._lib = prev
    assert caught, f"no pin caught mutant {name}"
