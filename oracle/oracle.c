/*
 * oracle.c -- plain, slow CPU reference for query-guided chunk-sparse attention (fp64).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load or call this library.  The GPU path never links, loads or calls it,
 * and it shares no code, header, table or helper with the GPU path.
 *
 * Every quantity is evaluated in double precision from the exact bf16 input values
 * (bf16 -> fp64 is exact).  Nothing is blocked, fused or reordered: each step is the
 * definition written out, one loop per sum.
 *
 * Sources (the pages' own section names):
 *   "Simplified Sparse Attention via Gist Tokens" (SSA):
 *     section 3.2  -- chunks are scored by query-key dot products against learned gist keys;
 *     section 3.3  -- the top-k chunks are selected and their raw tokens are restored
 *                     ("selective unfolding"); unselected chunks stay excluded;
 *     section 3.5, B.2 -- gist-of-gist hierarchy: meta-gists are scored first, lower levels
 *                     only score the candidates exposed by the selected meta-gists;
 *     section 3.1  -- a gist's KV pair can stand in for its chunk's KV.
 *   "SAS: Simple Attention Sparsification" (abstract): the selector's continuous scores enter
 *     the attention logits inside the softmax in log form; the gate is a normalized softmax
 *     over the history; the current block is always kept.
 *
 * Readings where the pages are silent (stated once here, used everywhere below):
 *   - chunk score s_c = log-sum-exp over the G heads of the KV group and the g gists of chunk
 *     c of the gist logits sigma * q_h . Kg[c][t]  (pooled query->gist attention mass in log
 *     form; equals sigma * q . Kg[c] when G = g = 1);
 *   - ranking key: larger score first, then lower chunk index; k_eff = min(k, candidates);
 *   - SAS gate gamma_c = s_c - log sum_{c' historical} exp(s_c') for selected chunks, added to
 *     every raw token of c; gists and the current chunk carry bias 0;
 *   - softmax token set: every scored summary (all historical gists, or at two levels all
 *     meta-gists plus the candidates' gists), the raw tokens of the selected chunks, and the
 *     raw tokens of the current chunk (the last, possibly partial, chunk); in the selected-
 *     summary mode the summaries are only the gists of the selected chunks and, at two
 *     levels, the meta-gists of the selected groups (section B.2);
 *   - per-head selection (appendix A: each head selects its chunks on its own, then the union
 *     is unfolded into the shared KV): head h's score of chunk c is the log-sum-exp of its own
 *     g gist logits, each head takes its top-k by the same ranking key, and every head of the
 *     group attends to the union of the G selections (ascending); no gate is defined for it;
 *   - prefill: per query block i, top-min(k, i) earlier blocks by the selector row S[i][j<i];
 *     gate log_softmax over all j < i; the diagonal block is token-causal with bias 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* bf16 bit pattern -> double, exactly: the bf16 bits are the upper half of an IEEE float. */
static double bf(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* sigma * q . k over d elements. */
static double dotq(const uint16_t* q, const uint16_t* k, int d, double sigma)
{
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += bf(q[i]) * bf(k[i]);
    return sigma * s;
}

/* log(sum_i exp(x_i)), n >= 1, with the maximum factored out. */
static double logsumexp(const double* x, int n)
{
    double m = -INFINITY;
    for (int i = 0; i < n; ++i) if (x[i] > m) m = x[i];
    double z = 0.0;
    for (int i = 0; i < n; ++i) z += exp(x[i] - m);
    return m + log(z);
}

typedef struct { double s; int c; } scored;

/* Larger score first; equal scores: lower index first. */
static int by_rank(const void* a, const void* b)
{
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->c > y->c) - (x->c < y->c);
}

static int ascending(const void* a, const void* b)
{
    int x = *(const int*)a, y = *(const int*)b;
    return (x > y) - (x < y);
}

/* Top-k of n scored items by (score desc, index asc); writes the chosen indices ascending.
 * Returns k_eff = min(k, n). */
static int top_k(const double* s, const int* idx, int n, int k, int* chosen)
{
    scored* v = (scored*)malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; ++i) { v[i].s = s[i]; v[i].c = idx[i]; }
    qsort(v, (size_t)n, sizeof(scored), by_rank);
    int ke = k < n ? k : n;
    if (ke < 0) ke = 0;
    for (int i = 0; i < ke; ++i) chosen[i] = v[i].c;
    qsort(chosen, (size_t)ke, sizeof(int), ascending);
    free(v);
    return ke;
}

/* One token of the softmax set: key row, value row, additive bias. */
typedef struct { const uint16_t* k; const uint16_t* v; double bias; } token;

/* o = sum_x softmax(lambda)_x v_x with lambda_x = sigma q.k_x + bias_x; returns the natural-log
 * normaliser lse = max + log(sum exp(lambda - max)).  Optionally writes the weights. */
static double attend(const uint16_t* q, const token* t, int n, int d, double sigma,
                     double* o, double* w_out)
{
    double* lam = (double*)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int x = 0; x < n; ++x) {
        lam[x] = dotq(q, t[x].k, d, sigma) + t[x].bias;
        if (lam[x] > m) m = lam[x];
    }
    double z = 0.0;
    for (int x = 0; x < n; ++x) z += exp(lam[x] - m);
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    for (int x = 0; x < n; ++x) {
        double w = exp(lam[x] - m) / z;
        if (w_out) w_out[x] = w;
        for (int i = 0; i < d; ++i) o[i] += w * bf(t[x].v[i]);
    }
    free(lam);
    return m + log(z);
}

/* Top-p with a cap: rank n scored items by (score desc, index asc); p_i = exp(s_i - lse) is an
 * item's share of the softmax over all n items.  Keep the shortest ranked prefix whose shares
 * add up to at least p (p >= 1 keeps everything), then at most k of them; indices ascending.
 * Returns the number kept. */
static int top_p(const double* s, const int* idx, int n, double p, int k, int* chosen)
{
    if (n <= 0 || k <= 0) return 0;
    scored* v = (scored*)malloc(sizeof(scored) * (size_t)n);
    for (int i = 0; i < n; ++i) { v[i].s = s[i]; v[i].c = idx[i]; }
    qsort(v, (size_t)n, sizeof(scored), by_rank);
    const double lse = logsumexp(s, n);
    int r = n;
    if (p < 1.0) {
        double mass = 0.0;
        for (int i = 0; i < n; ++i) {
            mass += exp(v[i].s - lse);
            if (mass >= p) { r = i + 1; break; }
        }
    }
    int ke = r < k ? r : k;
    for (int i = 0; i < ke; ++i) chosen[i] = v[i].c;
    qsort(chosen, (size_t)ke, sizeof(int), ascending);
    free(v);
    return ke;
}

/* Pooled chunk score: LSE over the G heads of the group and g gists at `gist` ([g][d]). */
static double pooled_score(const uint16_t* q_group, int G, const uint16_t* gist, int g, int d,
                           double sigma)
{
    double* l = (double*)malloc(sizeof(double) * (size_t)(G * g));
    for (int h = 0; h < G; ++h)
        for (int t = 0; t < g; ++t)
            l[h * g + t] = dotq(q_group + (size_t)h * d, gist + (size_t)t * d, d, sigma);
    double s = logsumexp(l, G * g);
    free(l);
    return s;
}

int or_decode_token_count(const or_decode_shape* p, int k_eff, int n_cand, int k2_eff)
{
    int M = (p->N + p->C - 1) / p->C;
    int H = M - 1;
    int cur = p->N - H * p->C;
    int summaries = 0;
    if (p->gists_in_softmax == 1) {
        if (p->levels == 2) summaries = ((H + p->J - 1) / p->J) * p->g + n_cand * p->g;
        else summaries = H * p->g;
    } else if (p->gists_in_softmax == 2) {
        summaries = k_eff * p->g;   /* each selected chunk brings its own gists */
        if (p->levels == 2) summaries += k2_eff * p->g;   /* and each selected group its own */
    }
    return summaries + k_eff * p->C + cur;
}

/* Adaptive top-k ("SSA", appendix A "More Details on Adaptive Top-k").  The appendix builds
 * one selection budget per routing level from the KV positions available n_kv, the effective
 * compression L_eff (the chunk size L at one level, L * J at two levels), the group size G and
 * L, divides by G because each head selects before the union is unfolded into the shared KV,
 * adds 1 so that at least one chunk is selected, and uses the same budget at both levels.  It
 * does not print the formula.  Reading used here: the compressed cache holds n_kv / L_eff
 * summary positions; the raw tokens unfolded by the G heads together (G * k chunks of L
 * tokens) are to match that count, so k = floor(n_kv / (L_eff * G * L)) + 1, with n_kv = N,
 * the tokens in the cache.  Unfolded tokens then stay proportional to n_kv at every
 * compression ratio.  PARITY UNPINNED against the paper's own (unprinted) formula: only the
 * properties the appendix states are pinned. */
int or_adaptive_k(const or_decode_shape* p)
{
    const long long G = p->Hq / p->Hkv;
    const long long l_eff = p->levels == 2 ? (long long)p->C * p->J : (long long)p->C;
    return (int)((long long)p->N / (l_eff * G * p->C)) + 1;
}

/* Decode for one unit (b, kv). */
static int decode_unit(const or_decode_shape* p, const or_decode_io* io, int b, int kv)
{
    const int G = p->Hq / p->Hkv, d = p->d, g = p->g, C = p->C;
    const int M = (p->N + C - 1) / C, H = M - 1;
    const int cur = p->N - H * C;
    const double sigma = p->scale > 0 ? p->scale : 1.0 / sqrt((double)d);
    const int gcap = p->gist_cap > 0 ? p->gist_cap : H;
    const uint16_t* qg = io->q + ((size_t)b * p->Hq + (size_t)kv * G) * d;
    const uint16_t* gk = io->gist_k + ((size_t)b * p->Hkv + kv) * (size_t)gcap * g * d;
    const uint16_t* gv = io->gist_v + ((size_t)b * p->Hkv + kv) * (size_t)gcap * g * d;
    const int32_t* pt = io->page_table + (size_t)b * p->max_chunks;
    const size_t unit = (size_t)b * p->Hkv + kv;
    /* chunks (k1) and groups (k2) to select; sel and sel_groups keep the strides k and k2 */
    int k1 = p->k, k2 = p->k2;
    if (p->adaptive_k) {
        const int ka = or_adaptive_k(p);
        if (ka < k1) k1 = ka;
        if (ka < k2) k2 = ka;
    }

    /* Candidate chunks: every historical chunk, or at two levels the members of the
     * selected level-2 groups. */
    int* cand = (int*)malloc(sizeof(int) * (size_t)(H > 0 ? H : 1));
    int n_cand = 0;
    int nG = 0, k2e = 0;
    int* groups = NULL;
    const uint16_t *g2k = NULL, *g2v = NULL;
    if (p->levels == 2) {
        nG = (H + p->J - 1) / p->J;
        g2k = io->gist2_k + unit * (size_t)nG * g * d;
        g2v = io->gist2_v + unit * (size_t)nG * g * d;
        double* s2 = (double*)malloc(sizeof(double) * (size_t)(nG > 0 ? nG : 1));
        int* ids = (int*)malloc(sizeof(int) * (size_t)(nG > 0 ? nG : 1));
        groups = (int*)malloc(sizeof(int) * (size_t)(nG > 0 ? nG : 1));
        for (int r = 0; r < nG; ++r) {
            s2[r] = pooled_score(qg, G, g2k + (size_t)r * g * d, g, d, sigma);
            ids[r] = r;
            if (io->group_scores) io->group_scores[unit * nG + r] = s2[r];
        }
        if (io->forced_groups) {
            k2e = 0;
            for (int i = 0; i < p->k2; ++i) {
                int r = io->forced_groups[unit * p->k2 + i];
                if (r >= 0) groups[k2e++] = r;
            }
        } else {
            k2e = top_k(s2, ids, nG, k2, groups);
        }
        if (io->sel_groups)
            for (int i = 0; i < p->k2; ++i)
                io->sel_groups[unit * p->k2 + i] = i < k2e ? groups[i] : -1;
        for (int i = 0; i < k2e; ++i)
            for (int c = groups[i] * p->J; c < (groups[i] + 1) * p->J && c < H; ++c)
                cand[n_cand++] = c;
        free(s2);
        free(ids);
    } else {
        for (int c = 0; c < H; ++c) cand[n_cand++] = c;
    }

    /* Chunk scores over the candidates. */
    double* s = (double*)malloc(sizeof(double) * (size_t)(n_cand > 0 ? n_cand : 1));
    for (int i = 0; i < n_cand; ++i) {
        s[i] = pooled_score(qg, G, gk + (size_t)cand[i] * g * d, g, d, sigma);
    }
    if (io->chunk_scores && !p->head_select) {
        for (int c = 0; c < H; ++c) io->chunk_scores[unit * H + c] = -INFINITY;
        for (int i = 0; i < n_cand; ++i) io->chunk_scores[unit * H + cand[i]] = s[i];
    }

    /* Selection. */
    const int sk = p->head_select ? G * p->k : p->k;   /* entries per unit in sel */
    int* sel = (int*)malloc(sizeof(int) * (size_t)(sk > 0 ? sk : 1));
    int ke = 0;
    if (io->forced_sel) {
        for (int i = 0; i < sk; ++i) {
            int c = io->forced_sel[unit * sk + i];
            if (c >= 0) sel[ke++] = c;
        }
    } else if (p->head_select) {
        /* each head's own score and own top-k; the union, ascending */
        char* in_union = (char*)calloc((size_t)(H > 0 ? H : 1), 1);
        double* sh = (double*)malloc(sizeof(double) * (size_t)(n_cand > 0 ? n_cand : 1));
        int* pick = (int*)malloc(sizeof(int) * (size_t)(p->k > 0 ? p->k : 1));
        for (int h = 0; h < G; ++h) {
            for (int i = 0; i < n_cand; ++i) {
                sh[i] = pooled_score(qg + (size_t)h * d, 1, gk + (size_t)cand[i] * g * d, g, d,
                                     sigma);
                if (io->chunk_scores)
                    io->chunk_scores[(unit * G + h) * (size_t)H + cand[i]] = sh[i];
            }
            const int kh = top_k(sh, cand, n_cand, k1, pick);
            for (int j = 0; j < kh; ++j) in_union[pick[j]] = 1;
        }
        for (int c = 0; c < H; ++c)
            if (in_union[c]) sel[ke++] = c;
        free(pick);
        free(sh);
        free(in_union);
    } else if (p->top_p > 0.0) {
        ke = top_p(s, cand, n_cand, p->top_p, k1, sel);
    } else {
        ke = top_k(s, cand, n_cand, k1, sel);
    }
    if (io->sel)
        for (int i = 0; i < sk; ++i) io->sel[unit * sk + i] = i < ke ? sel[i] : -1;

    /* SAS gate: log of the softmax over all historical chunk scores (one level only). */
    double lse_s = 0.0;
    if (p->gate && n_cand > 0) lse_s = logsumexp(s, n_cand);

    /* Token set. */
    int cap = or_decode_token_count(p, ke, n_cand, k2e);
    token* tk = (token*)malloc(sizeof(token) * (size_t)cap);
    int n = 0;
    if (p->gists_in_softmax == 2 && p->levels == 2)
        /* Selected summaries at the upper level: the meta-gists of the chosen groups
         * ("SSA", B.2: every level contributes its selected summary tokens). */
        for (int i = 0; i < k2e; ++i)
            for (int t = 0; t < g; ++t) {
                tk[n].k = g2k + ((size_t)groups[i] * g + t) * d;
                tk[n].v = g2v + ((size_t)groups[i] * g + t) * d;
                tk[n++].bias = 0.0;
            }
    if (p->gists_in_softmax == 1) {
        if (p->levels == 2)
            for (int r = 0; r < nG; ++r)
                for (int t = 0; t < g; ++t) {
                    tk[n].k = g2k + ((size_t)r * g + t) * d;
                    tk[n].v = g2v + ((size_t)r * g + t) * d;
                    tk[n++].bias = 0.0;
                }
        for (int i = 0; i < n_cand; ++i)
            for (int t = 0; t < g; ++t) {
                tk[n].k = gk + ((size_t)cand[i] * g + t) * d;
                tk[n].v = gv + ((size_t)cand[i] * g + t) * d;
                tk[n++].bias = 0.0;
            }
    }
    int bad_page = 0;
    for (int i = 0; i < ke; ++i) {
        int c = sel[i];
        double gamma = 0.0;
        if (p->gate) {
            for (int j = 0; j < n_cand; ++j) if (cand[j] == c) gamma = s[j] - lse_s;
        }
        if (p->gists_in_softmax == 2)   /* the chunk's gists, unbiased ("SSA", section 3.3) */
            for (int t = 0; t < g; ++t) {
                tk[n].k = gk + ((size_t)c * g + t) * d;
                tk[n].v = gv + ((size_t)c * g + t) * d;
                tk[n++].bias = 0.0;
            }
        int page = pt[c];
        if (page < 0 || page >= p->num_pages) { bad_page = 1; continue; }
        const uint16_t* kr = io->k_pages + ((size_t)page * p->Hkv + kv) * (size_t)C * d;
        const uint16_t* vr = io->v_pages + ((size_t)page * p->Hkv + kv) * (size_t)C * d;
        for (int u = 0; u < C; ++u) {
            tk[n].k = kr + (size_t)u * d;
            tk[n].v = vr + (size_t)u * d;
            tk[n++].bias = gamma;
        }
    }
    {
        int page = pt[H];
        if (page < 0 || page >= p->num_pages) {
            bad_page = 1;
        } else {
            const uint16_t* kr = io->k_pages + ((size_t)page * p->Hkv + kv) * (size_t)C * d;
            const uint16_t* vr = io->v_pages + ((size_t)page * p->Hkv + kv) * (size_t)C * d;
            for (int u = 0; u < cur; ++u) {
                tk[n].k = kr + (size_t)u * d;
                tk[n].v = vr + (size_t)u * d;
                tk[n++].bias = 0.0;
            }
        }
    }

    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    for (int h = 0; h < G; ++h) {
        const size_t row = (size_t)b * p->Hq + (size_t)kv * G + h;
        double* w = io->weights ? io->weights + row * (size_t)io->weights_cap : NULL;
        if (w && n > io->weights_cap) w = NULL;
        double l = attend(io->q + row * d, tk, n, d, sigma, o, w);
        if (bad_page) l = NAN;
        for (int i = 0; i < d; ++i) io->out[row * d + i] = bad_page ? NAN : o[i];
        if (io->lse) io->lse[row] = l;
        if (io->n_tokens) io->n_tokens[row] = n;
    }
    free(o);
    free(tk);
    free(sel);
    free(s);
    free(cand);
    free(groups);
    return 0;
}

int or_decode(const or_decode_shape* p, const or_decode_io* io)
{
    if (!p || !io) return 1;
    if (p->Hkv <= 0 || p->Hq % p->Hkv || p->C <= 0 || p->g <= 0 || p->N < 1) return 2;
    if (p->levels == 2 && (p->J <= 0 || p->gate)) return 3;
    if (p->gists_in_softmax < 0 || p->gists_in_softmax > 2) return 4;
    if (!(p->top_p >= 0.0 && p->top_p <= 1.0)) return 5;
    if (p->head_select < 0 || p->head_select > 1 ||
        (p->head_select && (p->levels != 1 || p->gate || p->top_p > 0.0)))
        return 6;
    if (p->adaptive_k < 0 || p->adaptive_k > 1 || (p->adaptive_k && p->top_p > 0.0)) return 7;
    const int total = p->B * p->Hkv;
    const int n = io->units ? io->n_units : total;
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
    for (int i = 0; i < n; ++i) {
        int u = io->units ? io->units[i] : i;
        rc |= decode_unit(p, io, u / p->Hkv, u % p->Hkv);
    }
    return rc;
}

/* Block-sparse causal prefill for one (b, kv, query block i). */
static void prefill_block(const or_prefill_shape* p, const or_prefill_io* io, int b, int kv, int i)
{
    const int G = p->Hq / p->Hkv, d = p->d, blk = p->blk, nb = p->T / p->blk;
    const double sigma = p->scale > 0 ? p->scale : 1.0 / sqrt((double)d);
    const size_t unit = (size_t)b * p->Hkv + kv;
    const float* Srow = io->S + (unit * nb + i) * nb;

    /* Selection over the strictly earlier blocks j < i. */
    double* s = (double*)malloc(sizeof(double) * (size_t)(i > 0 ? i : 1));
    int* ids = (int*)malloc(sizeof(int) * (size_t)(i > 0 ? i : 1));
    int* sel = (int*)malloc(sizeof(int) * (size_t)(p->k > 0 ? p->k : 1));
    for (int j = 0; j < i; ++j) { s[j] = (double)Srow[j]; ids[j] = j; }
    int ke = 0;
    if (io->forced_sel) {
        const int32_t* f = io->forced_sel + (unit * nb + i) * p->k;
        for (int x = 0; x < p->k; ++x) if (f[x] >= 0) sel[ke++] = f[x];
    } else {
        ke = top_k(s, ids, i, p->k, sel);
    }
    if (io->sel)
        for (int x = 0; x < p->k; ++x) io->sel[(unit * nb + i) * p->k + x] = x < ke ? sel[x] : -1;
    double lse_s = (p->gate && i > 0) ? logsumexp(s, i) : 0.0;

    const uint16_t* K = io->k + unit * (size_t)p->T * d;
    const uint16_t* V = io->v + unit * (size_t)p->T * d;
    token* tk = (token*)malloc(sizeof(token) * (size_t)(ke * blk + blk));
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    for (int h = 0; h < G; ++h) {
        const size_t head = (size_t)b * p->Hq + (size_t)kv * G + h;
        for (int r = 0; r < blk; ++r) {
            const int pos = i * blk + r;
            int n = 0;
            for (int x = 0; x < ke; ++x) {
                int j = sel[x];
                double gamma = p->gate ? (double)Srow[j] - lse_s : 0.0;
                for (int u = j * blk; u < (j + 1) * blk; ++u) {
                    tk[n].k = K + (size_t)u * d;
                    tk[n].v = V + (size_t)u * d;
                    tk[n++].bias = gamma;
                }
            }
            for (int u = i * blk; u <= pos; ++u) {
                tk[n].k = K + (size_t)u * d;
                tk[n].v = V + (size_t)u * d;
                tk[n++].bias = 0.0;
            }
            const size_t qrow = head * (size_t)p->T + pos;
            double l = attend(io->q + qrow * d, tk, n, d, sigma, o, NULL);
            for (int e = 0; e < d; ++e) io->out[qrow * d + e] = o[e];
            if (io->lse) io->lse[qrow] = l;
        }
    }
    free(o);
    free(tk);
    free(sel);
    free(ids);
    free(s);
}

int or_prefill(const or_prefill_shape* p, const or_prefill_io* io)
{
    if (!p || !io) return 1;
    if (p->Hkv <= 0 || p->Hq % p->Hkv || p->blk <= 0 || p->T % p->blk) return 2;
    const int nb = p->T / p->blk;
    const int total = p->B * p->Hkv * nb;
    const int n = io->blocks ? io->n_blocks : total;
#pragma omp parallel for schedule(dynamic, 1)
    for (int x = 0; x < n; ++x) {
        int u = io->blocks ? io->blocks[x] : x;
        int i = u % nb, bk = u / nb;
        prefill_block(p, io, bk / p->Hkv, bk % p->Hkv, i);
    }
    return 0;
}

/* Gradients for one (b, kv): every query block in turn, every head and row of it.
 * For a query row with softmax weights P over its token set and output o:
 *   dP_x = dout . v_x,   D = dout . o - dlse,   dlambda_x = P_x (dP_x - D)
 *   dq += sigma dlambda_x k_x,   dk_x += sigma dlambda_x q,   dv_x += P_x dout
 * (the chain rule through lambda_x = sigma q . k_x + bias_x, the softmax and lse).  The gate
 * bias of chosen block j is gamma_ij = S[i][j] - log sum_{j' < i} exp S[i][j'], so
 *   dgamma_ij = sum of dlambda over every head, row and key of (i, j), and
 *   dS[i][j'] = [j' chosen] dgamma_ij' - softmax(S[i][. < i])_j' sum_j dgamma_ij   (j' < i).
 * The selection itself is piecewise constant in S and contributes nothing. */
static void prefill_backward_unit(const or_prefill_shape* p, const or_prefill_bwd_io* io,
                                  int b, int kv)
{
    const int G = p->Hq / p->Hkv, d = p->d, blk = p->blk, nb = p->T / p->blk;
    const double sigma = p->scale > 0 ? p->scale : 1.0 / sqrt((double)d);
    const size_t unit = (size_t)b * p->Hkv + kv;
    const uint16_t* K = io->k + unit * (size_t)p->T * d;
    const uint16_t* V = io->v + unit * (size_t)p->T * d;
    double* dK = io->dk + unit * (size_t)p->T * d;
    double* dV = io->dv + unit * (size_t)p->T * d;
    for (size_t e = 0; e < (size_t)p->T * d; ++e) dK[e] = dV[e] = 0.0;

    const int n_max = (p->k > 0 ? p->k : 0) * blk + blk;
    double* sc = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    int* id = (int*)malloc(sizeof(int) * (size_t)(nb > 0 ? nb : 1));
    int* chosen = (int*)malloc(sizeof(int) * (size_t)(p->k > 0 ? p->k : 1));
    double* dgam = (double*)malloc(sizeof(double) * (size_t)(p->k > 0 ? p->k : 1));
    int* key = (int*)malloc(sizeof(int) * (size_t)n_max);      /* token -> key position  */
    int* slot = (int*)malloc(sizeof(int) * (size_t)n_max);     /* token -> chosen slot   */
    double* bias = (double*)malloc(sizeof(double) * (size_t)n_max);
    double* lam = (double*)malloc(sizeof(double) * (size_t)n_max);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);

    const int n_i = io->n_blocks > 0 && io->n_blocks < nb ? io->n_blocks : nb;
    for (int i = 0; i < n_i; ++i) {
        const float* Srow = io->S + (unit * nb + i) * nb;
        int ke = 0;
        if (io->forced_sel) {
            const int32_t* f = io->forced_sel + (unit * nb + i) * p->k;
            for (int x = 0; x < p->k; ++x) if (f[x] >= 0) chosen[ke++] = f[x];
        } else {
            for (int j = 0; j < i; ++j) { sc[j] = (double)Srow[j]; id[j] = j; }
            ke = top_k(sc, id, i, p->k, chosen);
        }
        for (int j = 0; j < i; ++j) sc[j] = (double)Srow[j];
        const double norm = (p->gate && i > 0) ? logsumexp(sc, i) : 0.0;
        for (int x = 0; x < ke; ++x) dgam[x] = 0.0;

        for (int h = 0; h < G; ++h) {
            const size_t head = (size_t)b * p->Hq + (size_t)kv * G + h;
            for (int r = 0; r < blk; ++r) {
                const int pos = i * blk + r;
                const size_t qrow = head * (size_t)p->T + pos;
                const uint16_t* qr = io->q + qrow * d;
                const uint16_t* gr = io->dout + qrow * d;
                /* the row's token set: the chosen blocks, then the causal part of block i */
                int n = 0;
                for (int x = 0; x < ke; ++x)
                    for (int u = chosen[x] * blk; u < (chosen[x] + 1) * blk; ++u) {
                        key[n] = u;
                        slot[n] = x;
                        bias[n++] = p->gate ? (double)Srow[chosen[x]] - norm : 0.0;
                    }
                for (int u = i * blk; u <= pos; ++u) {
                    key[n] = u;
                    slot[n] = -1;
                    bias[n++] = 0.0;
                }
                double m = -INFINITY;
                for (int x = 0; x < n; ++x) {
                    lam[x] = dotq(qr, K + (size_t)key[x] * d, d, sigma) + bias[x];
                    if (lam[x] > m) m = lam[x];
                }
                double z = 0.0;
                for (int x = 0; x < n; ++x) z += exp(lam[x] - m);
                const double lse = m + log(z);
                for (int e = 0; e < d; ++e) o[e] = 0.0;
                for (int x = 0; x < n; ++x) {
                    lam[x] = exp(lam[x] - lse);   /* from here on: the weight P_x */
                    for (int e = 0; e < d; ++e) o[e] += lam[x] * bf(V[(size_t)key[x] * d + e]);
                }
                double D = io->dlse ? -(double)io->dlse[qrow] : 0.0;
                for (int e = 0; e < d; ++e) D += bf(gr[e]) * o[e];
                double* dq = io->dq + qrow * d;
                for (int e = 0; e < d; ++e) dq[e] = 0.0;
                for (int x = 0; x < n; ++x) {
                    const uint16_t* kx = K + (size_t)key[x] * d;
                    const uint16_t* vx = V + (size_t)key[x] * d;
                    double dP = 0.0;
                    for (int e = 0; e < d; ++e) dP += bf(gr[e]) * bf(vx[e]);
                    const double dl = lam[x] * (dP - D);
                    for (int e = 0; e < d; ++e) {
                        dq[e] += sigma * dl * bf(kx[e]);
                        dK[(size_t)key[x] * d + e] += sigma * dl * bf(qr[e]);
                        dV[(size_t)key[x] * d + e] += lam[x] * bf(gr[e]);
                    }
                    if (slot[x] >= 0) dgam[slot[x]] += dl;
                }
            }
        }

        /* through the gate to the selector scores */
        double* dS = io->dS + (unit * nb + i) * nb;
        for (int j = 0; j < nb; ++j) dS[j] = 0.0;
        if (p->gate && ke > 0) {
            double tot = 0.0;
            for (int x = 0; x < ke; ++x) tot += dgam[x];
            for (int j = 0; j < i; ++j) dS[j] = -exp(sc[j] - norm) * tot;
            for (int x = 0; x < ke; ++x) dS[chosen[x]] += dgam[x];
        }
    }
    free(o);
    free(lam);
    free(bias);
    free(slot);
    free(key);
    free(dgam);
    free(chosen);
    free(id);
    free(sc);
}

int or_prefill_backward(const or_prefill_shape* p, const or_prefill_bwd_io* io)
{
    if (!p || !io || !io->dout || !io->dq || !io->dk || !io->dv || !io->dS) return 1;
    if (p->Hkv <= 0 || p->Hq % p->Hkv || p->blk <= 0 || p->T % p->blk) return 2;
    const int units = p->B * p->Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) prefill_backward_unit(p, io, u / p->Hkv, u % p->Hkv);
    return 0;
}

/* SSA gist-masked prefill for one query position (section 3.1: chunk tokens attend to their
 * own chunk and to the preceding gist tokens; later tokens reach a chunk only through its
 * gists).  The visible set is enumerated in sequence order, straight from the rule. */
static void gist_prefill_row(const or_gist_prefill_shape* p, const or_gist_prefill_io* io,
                             size_t row, token* tk)
{
    const int W = p->L + p->g;                  /* positions per chunk */
    const size_t Tp = (size_t)p->M * W;
    const int G = p->Hq / p->Hkv, d = p->d;
    const double sigma = p->scale > 0 ? p->scale : 1.0 / sqrt((double)d);
    const size_t bh = row / Tp;
    const int pos = (int)(row % Tp);
    const int b = (int)(bh / p->Hq), h = (int)(bh % p->Hq), kv = h / G;
    const int cp = pos / W;
    const uint16_t* K = io->k + ((size_t)b * p->Hkv + kv) * Tp * d;
    const uint16_t* V = io->v + ((size_t)b * p->Hkv + kv) * Tp * d;
    int n = 0;
    for (int x = 0; x <= pos; ++x) {
        const int cx = x / W;
        const int is_gist = (x % W) >= p->L;
        if (cx == cp || is_gist) {
            tk[n].k = K + (size_t)x * d;
            tk[n].v = V + (size_t)x * d;
            tk[n++].bias = 0.0;
        }
    }
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    const double l = attend(io->q + row * d, tk, n, d, sigma, o, NULL);
    for (int e = 0; e < d; ++e) io->out[row * d + e] = o[e];
    if (io->lse) io->lse[row] = l;
    free(o);
}

int or_gist_prefill(const or_gist_prefill_shape* p, const or_gist_prefill_io* io)
{
    if (!p || !io || !io->q || !io->k || !io->v || !io->out) return 1;
    if (p->Hkv <= 0 || p->Hq % p->Hkv || p->M < 1 || p->L < 1 || p->g < 0 || p->d < 1) return 2;
    const size_t Tp = (size_t)p->M * (p->L + p->g);
    const size_t total = (size_t)p->B * p->Hq * Tp;
    const size_t n = io->rows ? (size_t)io->n_rows : total;
    int rc = 0;
#pragma omp parallel reduction(| : rc)
    {
        token* tk = (token*)malloc(sizeof(token) * Tp);
        if (!tk) rc = 1;
#pragma omp for schedule(dynamic, 64)
        for (size_t x = 0; x < n; ++x) {
            if (!tk) continue;
            const size_t row = io->rows ? (size_t)io->rows[x] : x;
            gist_prefill_row(p, io, row, tk);
        }
        free(tk);
    }
    return rc;
}

int or_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
