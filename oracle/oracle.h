/*
 * oracle.h -- interface of the fp64 CPU reference (test infrastructure only; see oracle.c).
 * All pointers are host pointers.  bf16 tensors are passed as their uint16 bit patterns.
 * Shapes:
 *   q            [B][Hq][d]
 *   k/v_pages    [num_pages][Hkv][C][d]
 *   page_table   [B][max_chunks]         chunk c of batch b lives in page page_table[b][c]
 *   gist_k/v     [B][Hkv][gist_cap][g][d] (gist_cap = 0 means M-1)
 *   gist2_k/v    [B][Hkv][nG][g][d]       nG = ceil((M-1)/J), levels = 2 only
 *   out          [B][Hq][d],  lse [B][Hq]
 *   sel          [B][Hkv][k] ascending, -1 padded ([B][Hkv][G*k] with head_select);
 *   sel_groups   [B][Hkv][k2]
 *   chunk_scores [B][Hkv][M-1] (-inf where a chunk was not scored; [B][Hq][M-1] per query
 *                head with head_select)
 *   group_scores [B][Hkv][nG]
 * Prefill:
 *   q [B][Hq][T][d], k/v [B][Hkv][T][d], S fp32 [B][Hkv][nb][nb], out [B][Hq][T][d], lse [B][Hq][T],
 *   sel [B][Hkv][nb][k].
 * Prefill backward: dout [B][Hq][T][d] (bf16), dlse [B][Hq][T], dq [B][Hq][T][d],
 *   dk/dv [B][Hkv][T][d], dS [B][Hkv][nb][nb].
 */
#ifndef TCS_ORACLE_H
#define TCS_ORACLE_H
#include <stdint.h>

typedef struct {
    int B, Hq, Hkv, d;
    int N, C, g, k;
    int gate;             /* 0 none, 1 SAS log-softmax gate                          */
    int gists_in_softmax; /* 1: every scored summary enters the softmax; 0: raw only;
                             2: only the selected chunks' gists (and, at two levels,
                                the selected groups' meta-gists)                         */
    int levels, J, k2;
    int max_chunks;
    int num_pages;
    int gist_cap;
    double scale;         /* <= 0: 1/sqrt(d)                                          */
    double top_p;         /* 0: top-k; in (0, 1]: shortest ranked prefix with softmax
                             mass >= top_p, at most k chunks (at two levels: over the
                             candidates, with the groups still the top k2)             */
    int head_select;      /* 0: one selection per KV head from the group-pooled score;
                             1: every query head picks its own top-k by its own score and
                                the union is unfolded for the whole group (one level, no
                                gate, no top-p)                                          */
    int adaptive_k;       /* 0: select k chunks (k2 groups).  1: adaptive top-k (SSA
                             appendix A): every level selects min(cap, or_adaptive_k(p))
                             with cap = k for chunks and k2 for groups; no top-p           */
} or_decode_shape;

typedef struct {
    const uint16_t *q, *k_pages, *v_pages;
    const int32_t* page_table;
    const uint16_t *gist_k, *gist_v, *gist2_k, *gist2_v;
    const int32_t* forced_sel;     /* NULL: select by score; else [B][Hkv][k], -1 padded  */
    const int32_t* forced_groups;  /* NULL or [B][Hkv][k2]                                 */
    const int32_t* units;          /* NULL: every (b, kv); else n_units flat ids b*Hkv+kv  */
    int n_units;
    double* out;
    double* lse;
    int32_t* sel;
    int32_t* sel_groups;
    double* chunk_scores;
    double* group_scores;
    double* weights;               /* optional [B][Hq][weights_cap] softmax weights       */
    int weights_cap;
    int32_t* n_tokens;             /* optional [B][Hq] size of the softmax token set       */
} or_decode_io;

typedef struct {
    int B, Hq, Hkv, d, T, blk, k, gate;
    double scale;
} or_prefill_shape;

typedef struct {
    const uint16_t *q, *k, *v;
    const float* S;
    const int32_t* forced_sel;     /* NULL or [B][Hkv][nb][k]                              */
    const int32_t* blocks;         /* NULL: all; else flat ids ((b*Hkv+kv)*nb + i)         */
    int n_blocks;
    double* out;
    double* lse;
    int32_t* sel;
} or_prefill_io;

/* Gradients of the block-sparse causal prefill (same shape and selection as the forward) for
 * the loss L = sum dout . out + sum dlse . lse. */
typedef struct {
    const uint16_t *q, *k, *v;
    const float* S;
    const uint16_t* dout;          /* bf16 [B][Hq][T][d]                                   */
    const float* dlse;             /* NULL (zero) or fp32 [B][Hq][T]                       */
    const int32_t* forced_sel;     /* NULL or [B][Hkv][nb][k]                              */
    double* dq;                    /* [B][Hq][T][d]                                        */
    double* dk;                    /* [B][Hkv][T][d]                                       */
    double* dv;                    /* [B][Hkv][T][d]                                       */
    double* dS;                    /* [B][Hkv][nb][nb]; zero where S has no effect         */
    int n_blocks;                  /* 0: every query block; else only blocks i < n_blocks of
                                      each unit (a timing sample: dk, dv and dS then hold
                                      those blocks' contributions only)                    */
} or_prefill_bwd_io;

/* SSA gist-masked prefill ("Simplified Sparse Attention via Gist Tokens", section 3.1): the
 * sequence interleaves M chunks of L raw tokens, each followed by its g gist tokens
 * (T' = M (L + g) positions).  Position x of chunk c(x) is visible to position p of chunk c(p)
 * iff x <= p and (c(x) == c(p) or x is a gist token): a chunk's own tokens causally, and the
 * gist tokens of every earlier chunk.
 *   q [B][Hq][T'][d], k/v [B][Hkv][T'][d], out [B][Hq][T'][d], lse [B][Hq][T'] */
typedef struct {
    int B, Hq, Hkv, d, M, L, g;
    double scale;                  /* <= 0: 1/sqrt(d) */
} or_gist_prefill_shape;

typedef struct {
    const uint16_t *q, *k, *v;
    const int32_t* rows;           /* NULL: every (b, head, position); else flat ids
                                      ((b * Hq + h) * T' + p)                               */
    int n_rows;
    double* out;
    double* lse;
} or_gist_prefill_io;

int or_gist_prefill(const or_gist_prefill_shape* p, const or_gist_prefill_io* io);
int or_decode(const or_decode_shape* p, const or_decode_io* io);
int or_prefill(const or_prefill_shape* p, const or_prefill_io* io);
int or_prefill_backward(const or_prefill_shape* p, const or_prefill_bwd_io* io);
int or_decode_token_count(const or_decode_shape* p, int k_eff, int n_cand, int k2_eff);
int or_adaptive_k(const or_decode_shape* p);
int or_threads(void);

#endif
