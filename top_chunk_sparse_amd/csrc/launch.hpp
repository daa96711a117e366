// launch.hpp -- internal interface between the C ABI layer (api.cpp) and the kernel
// launchers (decode.hip, prefill.hip).  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tcs {

// Events a launcher has recorded at its kernel's own start and end (hipExtLaunchKernel's
// start and stop events, so that they bracket the kernel alone); null members are skipped.
// A launcher that runs no kernel records both where the kernel would have been.
struct KernelEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Per-slot softmax partial: unnormalised acc[d] plus (running max m, sum l).
struct Partials {
    float* acc;   // [B*Hq][nslots][d]
    float* ml;    // [B*Hq][nslots][2]
    int nslots;
};

// Selection done by the last workgroup of each unit (see select_epilogue).
struct SelectOut {
    int k;                    // items to select per unit (per query head with per-head selection)
    int stride;               // entries per unit in sel / gamma (>= k; G * stride per-head)
    int32_t* sel;             // [units][stride] ascending item ids, -1 padded
    float* gamma;             // [units][stride] SAS gate (log of the softmax over all items) or null
    float* cand_score;        // [units][slices][kcap] per-slice candidates
    int32_t* cand_idx;        // [units][slices][kcap]
    int kcap;                 // min(k, items per slice)
    float* slice_lse;         // [units][slices][2] (max, sum exp) or null
    unsigned* counter;        // [units], zero between calls
    float* fill_scores;       // optional [units][H]: -inf outside the chosen groups (level 2)
    int J, H;
    float top_p;              // > 0: keep the shortest ranked prefix with this share (k <= 256)
    // 1: each slice publishes its list and statistics before its V rows (range mode, at most
    // 256 items a slice), and the unit's first slice to finish merges them: counter[u] then
    // counts published slices in its low half and finished ones in its high half
    int defer;
};

struct GistLaunch {
    const uint16_t* q;
    const uint16_t* gk;
    const uint16_t* gv;
    long long unit_stride;    // elements between consecutive (b, kv) gist blocks
    int B, Hq, Hkv, d, g;
    int nitems;               // range mode: items (chunks or level-2 groups) scored
    int slices;               // grid.x
    int items_per_slice;      // range mode
    const int32_t* groups;    // group mode: [units][k2] chosen level-2 groups
    int J, k2, H;             // group mode
    float sigma;
    float* scores_out;        // optional [units][score_stride], indexed by item id
    int score_stride;
    Partials part;
    int slot0;
    SelectOut selo;
    int scores_only;          // 1: score and select only (no gist softmax partials)
    // range mode, one level: every query head of the group selects its own top-k (score =
    // log-sum-exp of its own g gist logits) and the union is written to selo.sel (G * selo.k
    // entries per unit); scores_out then holds one row per query head
    int heads;
    // group mode with scores_only: slice y's softmax partial covers the g level-2 gist rows of
    // its own group groups[u][y] (the selected-summary set at two levels) when pk is not null
    const uint16_t* pk;
    const uint16_t* pv;
    long long p_unit_stride;  // elements between consecutive (b, kv) level-2 gist blocks
};

struct ChunkLaunch {
    const uint16_t* q;
    const uint16_t* kp;
    const uint16_t* vp;
    const int32_t* page_table;
    int B, Hq, Hkv, d, C, N, M;
    int max_chunks, num_pages;
    const int32_t* sel;       // [units][k]
    const float* gamma;       // [units][k] or null
    int k;                    // stride of sel / gamma
    int kslots;               // selected-chunk slots launched (current chunk is slot kslots)
    int cpw;                  // slot mode: slots streamed per workgroup
    int rpw;                  // > 0: row mode, this many rows of the slots laid end to end
    float sigma;
    Partials part;
    int slot0;
    unsigned* counter;        // [units], zero between calls
    float* out;               // [B*Hq][d]
    float* lse;               // [B*Hq] or null
    // selected-gist token set: each selected chunk's g gist rows join its raw rows
    const uint16_t* gk;       // [units][gist_cap][g][d] or null
    const uint16_t* gv;
    long long gist_stride;    // elements between consecutive units' gists
    int g;
};

hipError_t launch_gist(const GistLaunch& a, hipStream_t s, const KernelEvents& ev = {});
hipError_t launch_chunks(const ChunkLaunch& a, hipStream_t s, const KernelEvents& ev = {});
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_fill(int32_t* p, long long n, int32_t v, hipStream_t s);
hipError_t launch_stream_read(const void* p, size_t bytes, unsigned* sink, int blocks,
                              hipStream_t s);

struct PrefillSelectLaunch {
    const float* S;           // [units][nb][nb]
    int units, nb, k;
    int32_t* sel;             // [units][nb][k]
    float* gamma;             // [units][nb][k] or null
};

struct PrefillLaunch {
    const uint16_t* q;        // [B][Hq][T][d]
    const uint16_t* k;        // [B][Hkv][T][d]
    const uint16_t* v;        // [B][Hkv][T][d]
    int B, Hq, Hkv, d, T, blk, ksel;
    const int32_t* sel;       // [B*Hkv][nb][ksel] ascending, -1 padded (null when ksel == 0)
    const float* gamma;       // [B*Hkv][nb][ksel] or null
    float sigma;
    float* out;               // [B][Hq][T][d]
    float* lse;               // [B][Hq][T] or null
};

// Backward of the block-sparse prefill (gradients of sum dout . out + sum dlse . lse).
struct PrefillBwdLaunch {
    const uint16_t* q;        // [B][Hq][T][d]
    const uint16_t* k;        // [B][Hkv][T][d]
    const uint16_t* v;        // [B][Hkv][T][d]
    const uint16_t* dout;     // [B][Hq][T][d]
    const float* out;         // [B][Hq][T][d] (the forward's output)
    const float* lse;         // [B][Hq][T]    (the forward's natural-log lse)
    const float* dlse;        // [B][Hq][T] or null
    const float* S;           // [B*Hkv][nb][nb]
    int B, Hq, Hkv, d, T, blk, ksel, gate;
    const int32_t* sel;       // [B*Hkv][nb][ksel] ascending, -1 padded (ksel > 0)
    const float* gamma;       // [B*Hkv][nb][ksel] or null (gate off)
    float sigma;
    float* D;                 // [B][Hq][T]: dout . out - dlse
    int32_t* inv_i;           // [B*Hkv][nb][nb]: query blocks i > j that chose key block j
    float* inv_g;             // [B*Hkv][nb][nb]: their gates
    int32_t* inv_n;           // [B*Hkv][nb]: list lengths
    float* dgp;               // [B*Hkv][nb][2][4 * head groups][ksel]: gate-gradient partials
    float* dq;                // [B][Hq][T][d]
    float* dk;                // [B][Hkv][T][d]
    float* dv;                // [B][Hkv][T][d]
    float* dS;                // [B*Hkv][nb][nb] or null
    int w_dkv;                // gradient grid: the leading dk / dv workgroups (set by the launch)
};

// SSA gist-masked prefill over the interleaved sequence (M chunks of L raw + g gist rows).
struct GistPrefillLaunch {
    const uint16_t* q;        // [B][Hq][T'][d], T' = M (L + g)
    const uint16_t* k;        // [B][Hkv][T'][d]
    const uint16_t* v;        // [B][Hkv][T'][d]
    int B, Hq, Hkv, d, M, L, g;
    int Gp;                   // rows of the gathered gist arrays: M g rounded up to 64
    uint16_t* gk;             // [B*Hkv][Gp][d]: every chunk's gist keys, chunk-major, zero pad
    uint16_t* gv;             // [B*Hkv][Gp][d]
    float sigma;
    float* out;               // [B][Hq][T'][d]
    float* lse;               // [B][Hq][T'] or null
    int w_gist_rows;          // set by the launcher: the gist-row workgroups of the row grid
};

hipError_t launch_gist_gather(const GistPrefillLaunch& a, hipStream_t s,
                              const KernelEvents& ev = {});
hipError_t launch_gist_prefill_rows(GistPrefillLaunch a, hipStream_t s,
                                    const KernelEvents& ev = {});
hipError_t launch_prefill_select(const PrefillSelectLaunch& a, hipStream_t s,
                                 const KernelEvents& ev = {});
hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t s, const KernelEvents& ev = {});
hipError_t launch_prefill_bwd_prep(const PrefillBwdLaunch& a, hipStream_t s,
                                   const KernelEvents& ev = {});
hipError_t launch_prefill_bwd_grad(PrefillBwdLaunch a, hipStream_t s,
                                   const KernelEvents& ev = {});
hipError_t launch_prefill_bwd_ds(const PrefillBwdLaunch& a, hipStream_t s,
                                 const KernelEvents& ev = {});

}  // namespace tcs
