/*
 * tcsparse.h -- C ABI of the MI355X (gfx950) query-guided chunk-sparse attention library
 * (libtcsparse.so).
 *
 * What is computed.
 *   Decode ("Simplified Sparse Attention via Gist Tokens", sections 3.2, 3.3, 3.5 and
 *   appendix B; "SAS: Simple Attention Sparsification", abstract).  For each batch row b and
 *   KV head kv (a "unit"), with G = Hq / Hkv query heads h = kv*G .. kv*G+G-1 reading that
 *   KV head, sigma = scale (0 -> 1/sqrt(d)), M = ceil(N / C) chunks, historical chunks
 *   H = {0 .. M-2} and the current chunk c* = M-1 holding tokens [(M-1)C, N):
 *     1. gist logits l[h][c][t] = sigma * q[b][h] . gist_k[b][kv][c][t] for c in H, t < g
 *        (section 3.2: chunk relevance from query-key products against learned gist keys);
 *     2. chunk score s[c] = log sum_{h, t} exp(l[h][c][t])  (the group's pooled
 *        query->gist attention mass, in log form);
 *     3. sel = the min(k, |H|) chunks with the largest s, equal scores broken toward the lower
 *        chunk index, reported in ascending order (section 3.3: top-k selection);
 *     4. SAS gate (gate_mode = TCS_GATE_SAS): gamma[c] = s[c] - log sum_{c' in H} exp(s[c'])
 *        is added to the logit of every raw token of a selected chunk c (the gate sits inside
 *        the softmax in log form; the current chunk and the gists carry no gate);
 *     5. one softmax per query head over: every historical gist (key gist_k, value gist_v,
 *        bias 0), the raw tokens of every selected chunk (bias gamma or 0), and the raw tokens
 *        of the current chunk (bias 0, always kept):
 *          lambda_x = sigma * q . k_x + bias_x,  out = sum_x softmax(lambda)_x v_x,
 *          lse = log sum_x exp(lambda_x)  (natural log, gate included).
 *   gist_mode = TCS_GISTS_SELECTED replaces "every historical gist" in step 5 by the gists of
 *   the selected chunks only, each next to its chunk's raw tokens: the set section 3.3
 *   describes, in which an unselected chunk contributes nothing.  The scores and the selection
 *   (steps 1-4) are unchanged.
 *   top_p in (0, 1] replaces step 3: rank H as in step 3 and keep the shortest ranked prefix
 *   whose shares p[c] = exp(s[c] - log sum_{c' in H} exp(s[c'])) add up to at least top_p
 *   (top_p = 1 keeps every chunk), at most k of them, reported ascending.  At two levels H is
 *   the candidate set (the chosen groups' member chunks, the only chunks scored) and the
 *   groups are still the top k2.  The pages compare against top-p (SSA figure 2) without
 *   spelling the rule out; this is the reading used here.  The shares are summed in fp32 in rank order, so a selection may differ
 *   from an exact evaluation when the running share crosses top_p within rounding.
 *   select_mode = TCS_SELECT_PER_HEAD (one level, no gate, top_p = 0) replaces steps 2-3 by
 *   per-head selection (appendix A: each head selects its chunks on its own and their union is
 *   unfolded into the shared KV): query head h of the group scores chunk c by
 *   s_h[c] = log sum_t exp(l[h][c][t]), takes its own top min(k, |H|) as in step 3, and every
 *   head of the group attends, in step 5, to the raw tokens of the union U of the G heads'
 *   choices (k_eff <= |U| <= min(G k, |H|)).  sel then holds U ascending with G * k entries per
 *   (b, kv) (-1 padded), and chunk_scores holds s_h, one row per query head.
 *   k_mode = TCS_K_ADAPTIVE (adaptive top-k, appendix A "More Details on Adaptive Top-k")
 *   replaces the fixed counts by one budget per routing level,
 *     k_a = floor(N / (L_eff * G * C)) + 1,   L_eff = C (one level) or C * J (two levels),
 *   so that the raw tokens the G heads' choices unfold together (G k_a chunks of C tokens)
 *   match the N / L_eff summary positions of the compressed cache, and at least one chunk is
 *   kept.  Step 3 then selects min(k, k_a) chunks, and at two levels min(k2, k_a) groups: the
 *   same budget at both levels.  k and k2 stay the strides of sel and sel_groups (entries
 *   past the selection are -1).  The appendix names the budget's ingredients (the KV
 *   positions, the effective compression, the group size and the chunk size, the division by
 *   G for the union of the heads' choices, the +1, the same k at both levels) but not the
 *   formula; the one above is the reading used here.  Not with top_p > 0.
 *   Two levels (levels = 2; section 3.5 and appendix B.2): level-2 gists summarise groups of J
 *   consecutive historical chunks.  The group scores s2[r] (step 2 over gist2_k) pick the top
 *   k2 groups; the member chunks of the chosen groups are the candidates; steps 1-3 run over
 *   the candidates only.  The softmax set is: every level-2 gist, the gists of every
 *   candidate chunk, the raw tokens of the selected chunks and of the current chunk; with
 *   TCS_GISTS_SELECTED it is the level-2 gists of the chosen groups, the gists and raw tokens
 *   of the selected chunks and the current chunk (appendix B.2: every level contributes the
 *   summaries it selected, the lowest level also the raw tokens).  The SAS gate is not defined
 *   for two levels (TCS_ERR_UNSUPPORTED).
 *
 *   Prefill ("SAS: Simple Attention Sparsification", abstract: FlashAttention-style forward
 *   with the gate inside the softmax).  Query block i (blk tokens) of KV head kv keeps the
 *   top min(k, i) earlier blocks j < i by the selector row S[b][kv][i][j] (ties to the lower
 *   j) plus its own (diagonal) block, which is token-causal.  Gate (gate_mode = SAS):
 *   gamma[i][j] = S[i][j] - log sum_{j' < i} exp(S[i][j']) on every key of selected block j;
 *   bias 0 on the diagonal block.  out = softmax(sigma q K^T + bias) V, lse natural log.
 *
 *   SSA gist-masked prefill ("Simplified Sparse Attention via Gist Tokens", section 3.1).  The
 *   sequence interleaves M chunks of L raw tokens, each followed by its g gist tokens
 *   (T' = M (L + g) positions; position p lies in chunk p / (L + g) and is a gist token when
 *   p % (L + g) >= L).  Position x is visible to position p iff x <= p and (x is in p's chunk
 *   or x is a gist token): chunk tokens see their own chunk and every earlier chunk's gists,
 *   and later tokens reach a chunk only through its gists.  out = softmax(sigma q K^T) V over
 *   the visible set, lse natural log.  Section 3.6's key-column permutation (summary columns
 *   first) is how it runs: the gists are gathered into a contiguous prefix each call, and the
 *   visible blocks of a query block are a closed form of its chunk and position, so no mask is
 *   stored and nothing needs sharing across layers.
 *
 *   Prefill backward (the SAS training form: the gate is trained end to end through the
 *   softmax).  Gradients of L = sum dout . out + sum dlse . lse with respect to q, k, v and the
 *   selector scores S, with the selection of the forward (recomputed from S; it is piecewise
 *   constant in S and passes no gradient).  For query row r with weights P over its visible
 *   keys and D_r = dout_r . out_r - dlse_r: dlambda_rx = P_rx (dout_r . v_x - D_r);
 *   dq_r = sigma sum_x dlambda_rx k_x; dk_x = sigma sum_r dlambda_rx q_r; dv_x = sum_r P_rx
 *   dout_r (sums over every query head of the group).  With the gate, g_ij = sum of
 *   dlambda over every head, row and key of (query block i, chosen block j), and
 *   dS[i][j'] = [j' chosen] g_ij' - softmax_{j < i}(S[i][j])_j' sum_j g_ij for j' < i, 0 for
 *   j' >= i; without the gate dS = 0.
 *
 * Layouts (row-major, innermost last).  bf16 = IEEE bfloat16 bit patterns.
 *   q            bf16 [B][Hq][d]
 *   k_pages      bf16 [num_pages][Hkv][C][d]   one page holds one chunk of every KV head
 *   v_pages      bf16 [num_pages][Hkv][C][d]
 *   page_table   int32 [B][max_chunks]          page of chunk c of batch row b
 *   gist_k/v     bf16 [B][Hkv][gist_cap][g][d]  rows c < M-1 are read
 *   gist2_k/v    bf16 [B][Hkv][nG][g][d]        nG = ceil((M-1) / J); levels = 2 only
 *   out          fp32 [B][Hq][d]
 *   lse          fp32 [B][Hq]                   optional (NULL)
 *   sel          int32 [B][Hkv][k]              optional; ascending chunk ids, -1 padded
 *                                               ([B][Hkv][G*k] with TCS_SELECT_PER_HEAD)
 *   sel_groups   int32 [B][Hkv][k2]             optional; levels = 2
 *   chunk_scores fp32 [B][Hkv][M-1]             optional; -inf for chunks not scored
 *                                               ([B][Hq][M-1] with TCS_SELECT_PER_HEAD)
 *   Prefill: q bf16 [B][Hq][T][d]; k, v bf16 [B][Hkv][T][d]; S fp32 [B][Hkv][nb][nb] with
 *   nb = T / blk (entries j >= i are ignored); out fp32 [B][Hq][T][d]; lse fp32 [B][Hq][T]
 *   (optional); sel int32 [B][Hkv][nb][k] (optional, ascending, -1 padded).
 *   Gist prefill: q bf16 [B][Hq][T'][d]; k, v bf16 [B][Hkv][T'][d] (the interleaved
 *   sequence); out fp32 [B][Hq][T'][d]; lse fp32 [B][Hq][T'] (optional).
 *   Prefill backward: out, lse fp32 as the forward wrote them (both required); dout bf16
 *   [B][Hq][T][d]; dlse fp32 [B][Hq][T] (optional: NULL means 0); dq fp32 [B][Hq][T][d];
 *   dk, dv fp32 [B][Hkv][T][d]; dS fp32 [B][Hkv][nb][nb] (optional).
 *
 * Ownership, streams, errors.
 *   All tensor pointers are device pointers owned by the caller, as is the workspace (size
 *   from tcs_*_workspace_size, 256-byte aligned).  The library allocates, frees and
 *   synchronises nothing and keeps no global state; every call only enqueues kernels on
 *   `stream` and returns.  Calls sharing a workspace must be ordered on one stream.
 *   A decode workspace starts with a block of arrival counters and flags, laid out the same
 *   way for every shape, that must read zero when a call starts: zero-fill a new workspace
 *   once (tcs_workspace_init, or any zero fill) before its first call; every completed call
 *   leaves them at zero again, so one workspace (as large as the largest shape needs) serves
 *   calls of any shape in turn.  After a call that returned TCS_ERR_HIP, initialise the
 *   workspace again.
 *   Argument errors return before any device work and leave every output untouched.  A
 *   failed launch returns TCS_ERR_HIP.  Inputs must be finite (NaN/Inf inputs give
 *   unspecified results).  A page id outside [0, num_pages) is never read: the heads of the
 *   affected unit get NaN in out and lse.
 *   k larger than the number of candidates is clamped (that is how "all chunks" is asked
 *   for); k = 0 keeps only the gists and the current chunk (with TCS_GISTS_SELECTED only the
 *   current chunk, plus the chosen groups' level-2 gists at two levels).  Results are
 *   deterministic:
 *   no floating-point atomics; the same inputs give bitwise-identical outputs.
 *
 * Supported shapes: d in {64, 128}; G = Hq / Hkv in {1, 2, 4, 8}; g <= 64; C <= 1024;
 * B * Hkv <= 16384; TCS_GISTS_SELECTED: C + g <= 1024; top_p > 0: k <= 256;
 * TCS_SELECT_PER_HEAD: one level, no gate, top_p = 0, M - 1 <= 65536; TCS_K_ADAPTIVE:
 * top_p = 0; two levels:
 * J * g <= 1024 and min(k2, nG) <= 64; prefill d = 128, blk = 64 and T a multiple of blk; gist
 * prefill d = 128, L a multiple of 64, 1 <= g <= 64 with 64 a multiple of g.
 * Other shapes return TCS_ERR_UNSUPPORTED.
 */
#ifndef TCSPARSE_H
#define TCSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TCS_ABI_VERSION 9

typedef enum {
    TCS_OK = 0,
    TCS_ERR_NULL = 1,         /* a required pointer is NULL                          */
    TCS_ERR_SHAPE = 2,        /* inconsistent or out-of-range sizes                  */
    TCS_ERR_UNSUPPORTED = 3,  /* valid, but not built (see supported shapes above)   */
    TCS_ERR_WORKSPACE = 4,    /* workspace NULL, misaligned or smaller than required  */
    TCS_ERR_HIP = 5,          /* a kernel launch failed                               */
    TCS_ERR_TOO_LARGE = 6     /* needs more than the static scratch of the _noalloc call */
} tcs_status;

enum { TCS_GATE_NONE = 0, TCS_GATE_SAS = 1 };
enum { TCS_GISTS_ALL = 0, TCS_GISTS_SELECTED = 1 };   /* which gists enter the softmax */
enum { TCS_SELECT_KV_HEAD = 0, TCS_SELECT_PER_HEAD = 1 };   /* who selects the chunks      */
enum { TCS_K_FIXED = 0, TCS_K_ADAPTIVE = 1 };   /* how many chunks (groups) are selected  */

typedef struct {
    int32_t struct_size;   /* = sizeof(tcs_decode_params) */
    int32_t B, Hq, Hkv, d;
    int32_t N;             /* tokens in the cache, current token included (>= 1)          */
    int32_t C;             /* chunk size = page size (tokens)                             */
    int32_t g;             /* gists per chunk                                             */
    int32_t k;             /* chunks to select (>= 0; clamped to the candidate count)     */
    int32_t gate_mode;     /* TCS_GATE_NONE or TCS_GATE_SAS                               */
    int32_t gist_mode;     /* TCS_GISTS_ALL or TCS_GISTS_SELECTED                         */
    int32_t levels;        /* 1, or 2 for gist-of-gist routing                            */
    int32_t J;             /* levels = 2: chunks per level-2 group                        */
    int32_t k2;            /* levels = 2: groups to select                                */
    int32_t max_chunks;    /* page_table row stride, >= M                                 */
    int32_t num_pages;     /* pages in k_pages / v_pages                                  */
    int32_t gist_cap;      /* chunk capacity of gist_k/v per (b, kv); 0 means M-1          */
    float scale;           /* logit scale; 0 means 1/sqrt(d)                              */
    float top_p;           /* 0: top-k.  In (0, 1]: top-p with a cap of k                 */
    int32_t select_mode;   /* TCS_SELECT_KV_HEAD or TCS_SELECT_PER_HEAD                   */
    int32_t k_mode;        /* TCS_K_FIXED, or TCS_K_ADAPTIVE: k and k2 become caps         */
} tcs_decode_params;

/* Host-only: bytes of workspace sparse_attn_decode needs for these parameters. */
tcs_status tcs_decode_workspace_size(const tcs_decode_params* p, size_t* bytes);

/* Chunk-sparse decode attention for one decode step of every (b, query head); see above. */
tcs_status sparse_attn_decode(const tcs_decode_params* p,
                              const void* q,
                              const void* k_pages, const void* v_pages,
                              const int32_t* page_table,
                              const void* gist_k, const void* gist_v,
                              const void* gist2_k, const void* gist2_v,
                              float* out, float* lse,
                              int32_t* sel, int32_t* sel_groups, float* chunk_scores,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Profiling variant of sparse_attn_decode: identical work and results, and in addition it
 * has caller-created HIP events (hipEvent_t, passed as void*) recorded at the start and the
 * end of each stage's kernel: events[2 i] and events[2 i + 1] for stage i, taken by the kernel
 * launch itself (hipExtLaunchKernel), so that they bracket that kernel alone; a stage that
 * runs no kernel (nothing to score) records both at that point of `stream`.  levels = 1:
 * stage 0 gist scoring with chunk selection, stage 1 chunk attention with the final merge.
 * levels = 2: stage 0 level-2 scoring with group selection, stage 1 candidate scoring with
 * chunk selection, stage 2 chunk attention with the final merge.  Entries beyond n_events,
 * or NULL entries, are skipped. */
tcs_status sparse_attn_decode_timed(const tcs_decode_params* p,
                                    const void* q,
                                    const void* k_pages, const void* v_pages,
                                    const int32_t* page_table,
                                    const void* gist_k, const void* gist_v,
                                    const void* gist2_k, const void* gist2_v,
                                    float* out, float* lse,
                                    int32_t* sel, int32_t* sel_groups, float* chunk_scores,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    void* const* events, int n_events);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): sparse_attn_decode with no workspace argument.  Its
 * workspace is a static device array of TCS_NOALLOC_SCRATCH_BYTES bytes, one per GPU the
 * library runs on, held until the process ends; its address is looked up once per device on
 * the first call made with that device current.  The call allocates and frees nothing.  Every
 * call clears the array's arrival counters (one small fill kernel on `stream`) and leaves the
 * rest of the array holding the call's intermediates.  Shapes whose workspace
 * (tcs_decode_workspace_size) exceeds TCS_NOALLOC_SCRATCH_BYTES return TCS_ERR_TOO_LARGE
 * before any device work; other argument errors as sparse_attn_decode.  All calls on one GPU
 * share its array: calls that overlap on one GPU (other streams, other threads) race, so
 * order them on one stream.  Results are bitwise those of sparse_attn_decode. */
#define TCS_NOALLOC_SCRATCH_BYTES (16u << 20)
tcs_status sparse_attn_decode_noalloc(const tcs_decode_params* p,
                                      const void* q,
                                      const void* k_pages, const void* v_pages,
                                      const int32_t* page_table,
                                      const void* gist_k, const void* gist_v,
                                      const void* gist2_k, const void* gist2_v,
                                      float* out, float* lse,
                                      int32_t* sel, int32_t* sel_groups, float* chunk_scores,
                                      void* stream);

/* Number of stages sparse_attn_decode_timed brackets with event pairs for these parameters
 * (2 for one level, 3 for two levels), -1 if the parameters are invalid.  Host-only. */
int tcs_decode_stage_count(const tcs_decode_params* p);

/* Zero-fills `workspace_bytes` bytes of a workspace on `stream` (one small kernel; no
 * allocation).  Required once before a new decode workspace is first used. */
tcs_status tcs_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

typedef struct {
    int32_t struct_size;   /* = sizeof(tcs_prefill_params) */
    int32_t B, Hq, Hkv, d;
    int32_t T;             /* tokens (multiple of blk)                                    */
    int32_t blk;           /* block size (64)                                             */
    int32_t k;             /* earlier blocks kept per query block (>= 0)                  */
    int32_t gate_mode;     /* TCS_GATE_NONE or TCS_GATE_SAS                               */
    float scale;           /* 0 means 1/sqrt(d)                                           */
} tcs_prefill_params;

tcs_status tcs_prefill_workspace_size(const tcs_prefill_params* p, size_t* bytes);

/* Block-sparse causal attention forward with the SAS gate; see above. */
tcs_status sparse_attn_prefill(const tcs_prefill_params* p,
                               const void* q, const void* k, const void* v,
                               const float* S,
                               float* out, float* lse, int32_t* sel,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Profiling variant of sparse_attn_prefill (events as in sparse_attn_decode_timed, a pair per
 * stage): stage 0 block selection (no kernel when k = 0), stage 1 the attention forward. */
tcs_status sparse_attn_prefill_timed(const tcs_prefill_params* p,
                                     const void* q, const void* k, const void* v,
                                     const float* S,
                                     float* out, float* lse, int32_t* sel,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events, int n_events);

tcs_status tcs_prefill_backward_workspace_size(const tcs_prefill_params* p, size_t* bytes);

/* Gradients of the block-sparse causal prefill (see above).  q, k, v, S and p must be those of
 * the forward call that produced out and lse.  Every output element is written (dq, dk, dv
 * in full; dS in full when not NULL).  Sums run in a fixed order: the same inputs give the
 * same bits. */
tcs_status sparse_attn_prefill_backward(const tcs_prefill_params* p,
                                        const void* q, const void* k, const void* v,
                                        const float* S, const float* out, const float* lse,
                                        const void* dout, const float* dlse,
                                        float* dq, float* dk, float* dv, float* dS,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* Profiling variant of sparse_attn_prefill_backward (a pair of events per stage, as in
 * sparse_attn_decode_timed): stage 0 block selection, stage 1 the row terms D and the
 * chosen-by lists (one kernel), stage 2 the gradient kernel (dq, dk and dv in one grid),
 * stage 3 the dS kernel (none without dS). */
tcs_status sparse_attn_prefill_backward_timed(const tcs_prefill_params* p,
                                              const void* q, const void* k, const void* v,
                                              const float* S, const float* out,
                                              const float* lse, const void* dout,
                                              const float* dlse, float* dq, float* dk,
                                              float* dv, float* dS, void* workspace,
                                              size_t workspace_bytes, void* stream,
                                              void* const* events, int n_events);

typedef struct {
    int32_t struct_size;   /* = sizeof(tcs_gist_prefill_params) */
    int32_t B, Hq, Hkv, d;
    int32_t M;             /* chunks                                                      */
    int32_t L;             /* raw tokens per chunk                                        */
    int32_t g;             /* gist tokens per chunk (they follow the chunk's raw tokens)  */
    float scale;           /* 0 means 1/sqrt(d)                                           */
} tcs_gist_prefill_params;

tcs_status tcs_gist_prefill_workspace_size(const tcs_gist_prefill_params* p, size_t* bytes);

/* SSA gist-masked prefill forward; see above.  Writes every row of out (and of lse). */
tcs_status sparse_attn_gist_prefill(const tcs_gist_prefill_params* p,
                                    const void* q, const void* k, const void* v,
                                    float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Profiling variant (a pair of events per stage, as in sparse_attn_decode_timed): stage 0 the
 * gist gather, stage 1 the query rows (gist rows and raw rows, one launch). */
tcs_status sparse_attn_gist_prefill_timed(const tcs_gist_prefill_params* p,
                                          const void* q, const void* k, const void* v,
                                          float* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream,
                                          void* const* events, int n_events);

/* Measurement aid, not part of the method: a plain streaming read of `bytes` bytes at `src`
 * (16-byte aligned, a multiple of 16) by one kernel on `stream`, each byte loaded once, the
 * HBM read ceiling the decode kernels' bandwidth is compared with.  `sink` (device memory of
 * TCS_STREAM_READ_BLOCKS 32-bit words) receives one word per workgroup so the loads cannot be
 * elided.  TCS_ERR_NULL for a null pointer, TCS_ERR_SHAPE for misalignment. */
#define TCS_STREAM_READ_BLOCKS 4096
tcs_status tcs_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/* Static string naming a status code. */
const char* tcs_status_str(tcs_status s);

/* TCS_ABI_VERSION of the built library. */
int tcs_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TCSPARSE_H */
