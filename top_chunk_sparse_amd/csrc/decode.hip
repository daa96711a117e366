// decode.hip -- gfx950 kernels of the chunk-sparse decode path.
//
//   gist_kernel   scores every historical chunk of a (b, kv) unit against the G query heads of
//                 its group through the chunk's gist keys ("Simplified Sparse Attention via
//                 Gist Tokens", section 3.2), pools them into one log-sum-exp score per chunk,
//                 and -- because gists are tokens of the softmax set themselves -- folds the
//                 same gist rows into per-slice softmax partials with the gist values.  Each
//                 slice publishes its best k items; the unit's top-k (section 3.3; ties to the
//                 lower index) and, with the SAS gate on, the gate log p_c over all historical
//                 scores ("SAS", abstract) are taken from those lists by one slice of the unit:
//                 the last to finish, or -- one routing level, plain top-k, lists published
//                 before the V rows -- the first to finish, so that no gist workgroup waits.
//   chunk_kernel  split-K attention over the selected chunks and the current chunk, read
//                 through the page table (section 3.6: only the selected keys are touched);
//                 with every gist in the token set, the rows of all slots, laid end to end,
//                 are cut into equal runs, one per workgroup; the last workgroup of a unit
//                 merges all partials in a fixed order.
//
// Layout of the work: one 256-thread workgroup streams runs of d-element bf16 rows (gist rows
// or the rows of a page).  A row is read by d/8 lanes with one 16-byte load each, so a wave
// reads 4 (d=128) or 8 (d=64) whole rows per instruction, fully coalesced.  Each run is read
// in two phases: the K rows first (dot products with bf16 dot2 instructions, finished by DPP
// row reductions, logits kept in LDS), then -- with the exact per-head maximum known -- the V
// rows, weighted by exp(logit - max).  Only one phase's registers are live at a time, which
// keeps the kernels at high occupancy for latency hiding.
#include "device.hpp"
#include "launch.hpp"

#include <math.h>

namespace tcs {

constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for empty softmax state
constexpr int kMaxSliceRows = 1024;   // rows (gists, or page rows) one workgroup holds logits for

#ifndef TCS_K_U
#define TCS_K_U 2       // row passes per batch of loads in the K phase (two batches in flight)
#endif
#ifndef TCS_V_U
// row passes per batch of loads in the V phase (two batches in flight).  At 128K tokens 4 beats
// 2 (gist kernel 51.8 -> 49.0 us): the V phase has no logits to compute, so only the depth of
// the loads in flight limits it; 6 and 8 cost occupancy (registers) and lose.
#define TCS_V_U 4
#endif
#ifndef TCS_CK_U
#define TCS_CK_U TCS_K_U   // the same, for the chunk kernel's K phase
#endif
#ifndef TCS_CV_U
#define TCS_CV_U TCS_V_U   // the same, for the chunk kernel's V phase in row mode
#endif
#ifndef TCS_CV_U_SLOTS
// the chunk kernel's V phase in slot mode (selected-gist token set: whole slots plus their gist
// rows), where four passes per batch lose (41.3 -> 48.0 us at 128K) while they win in row mode
#define TCS_CV_U_SLOTS 2
#endif

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// ---------------------------------------------------------------------------------------
// Row streaming for one workgroup (256 threads = 4 waves).
// ---------------------------------------------------------------------------------------
template <int D, int G>
struct RowStream {
    static constexpr int LPR = D / 8;          // lanes per row (16 B each)
    static constexpr int RPW = kWave / LPR;    // rows per wave per pass
    static constexpr int NW = 4;               // waves per workgroup
    static constexpr int RPP = RPW * NW;       // rows per workgroup per pass
    int lrow, part;

    __device__ RowStream() {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        part = lane % LPR;
        lrow = w * RPW + lane / LPR;
    }

    // The 8 query elements this lane multiplies, for each head, as bf16 pairs.
    __device__ void load_q(const uint16_t* qg, uint32_t (&q2)[G][4]) const {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint4 v = ld16(qg + h * D + part * 8);
            q2[h][0] = v.x; q2[h][1] = v.y; q2[h][2] = v.z; q2[h][3] = v.w;
        }
    }

    // Streams rows [0, nrows) in batches of U passes through two register buffers: the next
    // batch's loads are issued before the current batch is used, so a batch is always in
    // flight while the workgroup computes.
    // Rows past the end re-read the last row (their results are discarded): unconditional
    // loads keep the wait counts exact, so waiting for one buffer leaves the other in flight.
    template <int U>
    __device__ __forceinline__ void load_batch(const uint16_t* __restrict__ X, int nrows, int base,
                                               uint4 (&r)[U]) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = min(base + u * RPP + lrow, nrows - 1);
            r[u] = ld16(X + (long long)row * D + part * 8);
        }
    }

    // The first batch of rows, issued early (pre = 1 in the streaming call that follows).
    template <int U>
    __device__ __forceinline__ void prefetch(const uint16_t* __restrict__ X, int nrows,
                                             uint4 (&r)[U]) const {
        if (nrows > 0) load_batch<U>(X, nrows, 0, r);
    }
    // The first two batches (pre = 2).
    template <int U>
    __device__ __forceinline__ void prefetch2(const uint16_t* __restrict__ X, int nrows,
                                              uint4 (&ra)[U], uint4 (&rb)[U]) const {
        if (nrows > 0) load_batch<U>(X, nrows, 0, ra);
        if (nrows > U * RPP) load_batch<U>(X, nrows, U * RPP, rb);
    }

    // pre: how many of the first batches (0, 1 or 2) ra and rb already hold.
    template <int U, class Use>
    __device__ __forceinline__ void stream_rows(const uint16_t* __restrict__ X, int nrows,
                                                Use use, uint4 (&ra)[U], uint4 (&rb)[U],
                                                int pre) const {
        constexpr int STEP = U * RPP;
        auto load = [&](uint4 (&r)[U], int base) __attribute__((always_inline)) {
            load_batch<U>(X, nrows, base, r);
        };
        if (nrows <= 0) return;
        if (pre < 1) load(ra, 0);
        for (int base = 0; base < nrows; base += 2 * STEP) {
            if (base + STEP < nrows && (pre < 2 || base > 0)) load(rb, base + STEP);
            use(ra, base);
            if (base + STEP >= nrows) break;
            if (base + 2 * STEP < nrows) load(ra, base + 2 * STEP);
            use(rb, base + STEP);
        }
    }
    template <int U, class Use>
    __device__ __forceinline__ void stream_rows(const uint16_t* __restrict__ X, int nrows,
                                                Use use, uint4 (&ra)[U], bool pre) const {
        uint4 rb[U];
        stream_rows<U>(X, nrows, use, ra, rb, pre ? 1 : 0);
    }

    // K phase: lg[(row0 + r) * G + h] = sigma * q_h . K[r] + bias for rows r < nrows.
    template <int U>
    __device__ __forceinline__ void logits(const uint32_t (&q2)[G][4], const uint16_t* __restrict__ K, int nrows,
                           float sigma, float bias, float* lg, int row0) const {
        uint4 ra[U];
        stream_rows<U>(K, nrows, [&](const uint4 (&kr)[U], int base) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = base + u * RPP + lrow;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float s = dot2(q2[h][0], kr[u].x, 0.f);
                    s = dot2(q2[h][1], kr[u].y, s);
                    s = dot2(q2[h][2], kr[u].z, s);
                    s = dot2(q2[h][3], kr[u].w, s);
                    s = group_sum<LPR>(s);
                    if (part == 0 && row < nrows) lg[(row0 + row) * G + h] = fmaf(s, sigma, bias);
                }
            }
        }, ra, false);
    }

    // V phase: acc[h][e] += w[(row0 + r) * G + h] * V[r][part*8 + e] for rows r < nrows.
    // pre: the first batch is already in `first` (prefetch); else `first` is scratch space.
    template <int U>
    __device__ __forceinline__ void accumulate(float (&acc)[G][8], const uint16_t* __restrict__ V,
                                               int nrows, const float* w, int row0,
                                               uint4 (&first)[U], bool pre = false) const {
        uint4 second[U];
        accumulate2<U>(acc, V, nrows, w, row0, first, second, pre ? 1 : 0);
    }
    // The same with the second batch too (pre = 2: both prefetched).
    template <int U>
    __device__ __forceinline__ void accumulate2(float (&acc)[G][8], const uint16_t* __restrict__ V,
                                                int nrows, const float* w, int row0,
                                                uint4 (&first)[U], uint4 (&second)[U],
                                                int pre) const {
        stream_rows<U>(V, nrows, [&](const uint4 (&vr)[U], int base) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = base + u * RPP + lrow;
                if (row < nrows) {
                    float vf[8];
                    unpack8(vr[u], vf);
                    const float* wr = w + (row0 + row) * G;
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float wh = wr[h];
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(wh, vf[e], acc[h][e]);
                    }
                }
            }
        }, first, second, pre);
    }

    // Sum the lane groups' accumulators and write one partial per head:
    // acc -> P.acc[(bh0 + h) * nslots + slot][0..D), (M[h], L[h]) -> P.ml[...][0..2).
    // fin must hold NW * G * D floats.
    __device__ __forceinline__ void finish(float (&acc)[G][8], const float* M, const float* L, float* fin,
                           const Partials& P, int bh0, int slot) const {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = lane_groups_sum<LPR>(acc[h][e]);
        if (lane < LPR) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) fin[(w * G + h) * D + part * 8 + e] = acc[h][e];
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < G * D; idx += 256) {
            const int h = idx / D, col = idx % D;
            float a = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) a += fin[(ww * G + h) * D + col];
            const long long o = (long long)(bh0 + h) * P.nslots + slot;
            st_shared_dev(P.acc + o * D + col, a);
            if (col == 0) {
                st_shared_dev(P.ml + o * 2, M[h]);
                st_shared_dev(P.ml + o * 2 + 1, L[h]);
            }
        }
    }
};

// Per-head softmax statistics over the logits of n rows (lg[r * G + h]): M[h] = max, then the
// logits are replaced by exp(logit - M[h]) and L[h] = their sum.  Fixed reduction order.
template <int G>
struct HeadStatsSmem {
    float part[4][G];
    float M[G], L[G];
};

template <int G>
__device__ void head_stats(float* lg, int n, HeadStatsSmem<G>& sm) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float x[G];
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] = -INFINITY;
    for (int r = tid; r < n; r += 256)
#pragma unroll
        for (int h = 0; h < G; ++h) x[h] = fmaxf(x[h], lg[r * G + h]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        x[h] = wave_max(x[h]);
        if (lane == 0) sm.part[w][h] = x[h];
    }
    __syncthreads();
    if (tid < G) {
        float m = fmaxf(fmaxf(sm.part[0][tid], sm.part[1][tid]), fmaxf(sm.part[2][tid], sm.part[3][tid]));
        sm.M[tid] = m > kNegBig ? m : kNegBig;   // no finite logit: keep the state finite
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] = 0.f;
    for (int r = tid; r < n; r += 256)
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float e = __expf(lg[r * G + h] - sm.M[h]);
            lg[r * G + h] = e;
            x[h] += e;
        }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        x[h] = wave_sum(x[h]);
        if (lane == 0) sm.part[w][h] = x[h];
    }
    __syncthreads();
    if (tid < G) sm.L[tid] = (sm.part[0][tid] + sm.part[1][tid]) + (sm.part[2][tid] + sm.part[3][tid]);
    __syncthreads();
}

__device__ __forceinline__ void write_empty_partial(const Partials& P, int bh0, int G, int D,
                                                    int slot, float fill_l, float fill_acc) {
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D, col = idx % D;
        const long long o = (long long)(bh0 + h) * P.nslots + slot;
        st_shared_dev(P.acc + o * D + col, fill_acc);
        if (col == 0) {
            st_shared_dev(P.ml + o * 2, fill_l == fill_l ? kNegBig : 0.f);  // NaN fill: m = 0
            st_shared_dev(P.ml + o * 2 + 1, fill_l);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Selection epilogue shared by the scoring passes.  Each workgroup keeps the best
// min(k, items in its slice) of its slice's items (ascending), stores them with their
// scores, and the last workgroup of the unit to finish merges the slices' lists (which are
// in ascending item order, slice after slice) into the unit's top-k.  Ties go to the lower
// item index at both steps, so the result equals a top-k over all items at once.
// ---------------------------------------------------------------------------------------
struct MergeCand {
    float score[256];
    int32_t idx[256];
};

static_assert(kMaxSliceRows * sizeof(float) >= 4 * 256 * 4, "top-p staging fits the slice scores");

struct TopPSmem {             // the capped top-k of one unit, for the top-p cut (4 KB)
    float score[256];
    int32_t idx[256];
    float share[256];         // by rank
    int rank[256];            // by position
};

// A slice's share of the selection: the statistics of its scores for the gate (max and sum of
// exp) and its best min(k, nitems) items, ascending, with their scores.  `scratch` holds a
// TopkSmem, or only a SmallTopkSmem when nitems <= 256 or k >= nitems.
__device__ __forceinline__ void publish_slice(const SelectOut& so, int u, int slot, int nslices,
                                              const float* s_score, int item0, int nitems,
                                              void* scratch, ReduceSmem& red) {
    const int tid = threadIdx.x;
    const int kc = so.k < nitems ? so.k : nitems;
    float* cs = so.cand_score + ((long long)u * nslices + slot) * so.kcap;
    int32_t* ci = so.cand_idx + ((long long)u * nslices + slot) * so.kcap;
    // slice statistics for the gate: max and sum of exp over this slice's scores
    if (so.slice_lse) {
        float mx = -INFINITY;
        for (int i = tid; i < nitems; i += 256) mx = fmaxf(mx, s_score[i]);
        mx = block_max(mx, red);
        float z = 0.f;
        for (int i = tid; i < nitems; i += 256) z += expf(s_score[i] - mx);
        z = block_sum(z, red);
        if (tid == 0) {
            st_shared_dev(so.slice_lse + ((long long)u * nslices + slot) * 2, mx);
            st_shared_dev(so.slice_lse + ((long long)u * nslices + slot) * 2 + 1, z);
        }
    }
    auto emit = [&](int j, int i) {
        st_shared_dev(cs + j, s_score[i]);
        st_shared_dev(ci + j, (int32_t)(item0 + i));
    };
    auto sc = [&](int i) { return s_score[i]; };
    if (kc == nitems) {
        for (int i = tid; i < nitems; i += 256) emit(i, i);
    } else if (nitems <= 256) {
        small_topk(nitems, so.k, sc, emit, *reinterpret_cast<SmallTopkSmem*>(scratch));
    } else {
        block_topk(nitems, so.k, sc, emit, *reinterpret_cast<TopkSmem*>(scratch));
    }
}

// The unit's selection from every slice's published list, by one workgroup that has seen all
// of them published: the top-k of the candidates (ties to the lower item), the gate, top-p.
__device__ __forceinline__ void merge_selection(const SelectOut& so, int u, int nslices,
                                                int last_items, float* lse_part_lds,
                                                void* scratch, MergeCand& mc, int* s_chosen,
                                                TopPSmem& tps, int* s_keep) {
    const int tid = threadIdx.x;
    const float* ucs = so.cand_score + (long long)u * nslices * so.kcap;
    const int32_t* uci = so.cand_idx + (long long)u * nslices * so.kcap;
    const int ncand = (nslices - 1) * so.kcap + (so.k < last_items ? so.k : last_items);
    const bool staged = ncand <= 256;
    // one round trip for every hand-off value this workgroup needs
    const float* sl = so.slice_lse ? so.slice_lse + (long long)u * nslices * 2 : nullptr;
    float* st = reinterpret_cast<float*>(scratch);     // slice statistics, if they fit
    const bool need_lse = sl != nullptr;   // gate, or top-p shares
    const bool lse_staged = 2 * nslices <= kTopkCache;
    if (staged && tid < ncand) {
        mc.score[tid] = ld_shared_dev(ucs + tid);
        mc.idx[tid] = ld_shared_dev(uci + tid);
    }
    if (need_lse && lse_staged)
        for (int i = tid; i < 2 * nslices; i += 256) st[i] = ld_shared_dev(sl + i);
    __syncthreads();
    float lse = 0.f;
    if (need_lse) {
        auto at = [&](int i) { return lse_staged ? st[i] : ld_shared_dev(sl + i); };
        if (tid == 0) {
            float mx = -INFINITY;
            for (int s = 0; s < nslices; ++s) mx = fmaxf(mx, at(2 * s));
            float z = 0.f;
            for (int s = 0; s < nslices; ++s) z += at(2 * s + 1) * expf(at(2 * s) - mx);
            *lse_part_lds = mx + logf(z);
        }
        __syncthreads();
        lse = *lse_part_lds;
    }
    int32_t* sel = so.sel + (long long)u * so.stride;
    float* gam = so.gamma ? so.gamma + (long long)u * so.stride : nullptr;
    auto score_at = [&](int i) { return staged ? mc.score[i] : ld_shared_dev(ucs + i); };
    const bool top_p = so.top_p > 0.f;
    auto emit2 = [&](int j, int i) {
        const int32_t c = staged ? mc.idx[i] : ld_shared_dev(uci + i);
        if (top_p) {   // held back for the cut below (j < k <= 256)
            tps.idx[j] = c;
            tps.score[j] = score_at(i);
            return;
        }
        sel[j] = c;
        if (gam) gam[j] = score_at(i) - lse;
        if (j < 64) s_chosen[j] = c;
    };
    int ke;
    if (so.k >= ncand) {
        for (int i = tid; i < ncand; i += 256) emit2(i, i);
        ke = ncand;
    } else if (staged) {
        ke = small_topk(ncand, so.k, score_at, emit2, *reinterpret_cast<SmallTopkSmem*>(scratch));
    } else {
        ke = block_topk(ncand, so.k, score_at, emit2, *reinterpret_cast<TopkSmem*>(scratch));
    }
    if (top_p) {
        // The capped top-k (ascending chunk id in tps) is ranked by (score desc, id asc); the
        // shares exp(s - lse) are summed in rank order and the shortest prefix reaching top_p
        // is kept (all of it for top_p = 1), written ascending by chunk id.
        __syncthreads();
        int rank = 0;
        if (tid < ke) {
            const float sj = tps.score[tid];
            for (int i = 0; i < ke; ++i) {
                const float si = tps.score[i];
                rank += (si > sj) || (si == sj && i < tid);
            }
            tps.share[rank] = expf(sj - lse);
            tps.rank[tid] = rank;
        }
        __syncthreads();
        if (tid == 0) {
            int keep = ke;
            if (so.top_p < 1.f) {
                float mass = 0.f;
                for (int r = 0; r < ke; ++r) {
                    mass += tps.share[r];
                    if (mass >= so.top_p) { keep = r + 1; break; }
                }
            }
            *s_keep = keep;
        }
        __syncthreads();
        const int keep = *s_keep;
        if (tid < ke && rank < keep) {
            int pos = 0;   // kept entries before this one in chunk-id order
            for (int i = 0; i < tid; ++i) pos += tps.rank[i] < keep;
            sel[pos] = tps.idx[tid];
            if (gam) gam[pos] = tps.score[tid] - lse;
        }
        ke = keep;
    }
    for (int j = ke + tid; j < so.stride; j += 256) {
        sel[j] = -1;
        if (gam) gam[j] = 0.f;
    }
    if (so.fill_scores) {
        // two-level group pass: chunks outside the chosen groups are never scored
        __syncthreads();
        float* fs = so.fill_scores + (long long)u * so.H;
        for (int c = tid; c < so.H; c += 256) {
            const int r = c / so.J;
            bool in = false;
            for (int j = 0; j < ke && j < 64; ++j) in |= s_chosen[j] == r;
            if (!in) fs[c] = -INFINITY;
        }
    }
}

// Publish, then the last slice of the unit to arrive merges.
__device__ __forceinline__ void select_epilogue(const SelectOut& so, int u, int slot, int nslices,
                                const float* s_score, int item0, int nitems, int last_items,
                                float* lse_part_lds, void* scratch, MergeCand& mc, int* s_flag,
                                int* s_chosen, ReduceSmem& red, TopPSmem& tps, int* s_keep) {
    publish_slice(so, u, slot, nslices, s_score, item0, nitems, scratch, red);
    if (!arrive_last(so.counter + u, (unsigned)nslices, s_flag)) return;
    merge_selection(so, u, nslices, last_items, lse_part_lds, scratch, mc, s_chosen, tps, s_keep);
}

// Per-head selection.  Each slice keeps, for every head h of the group, that head's top-k of
// its items in the hand-off lists [unit][h][slice][kcap] (one head's lists are contiguous).
// The last workgroup of the unit merges each head's lists into that head's top-k, marks the
// chosen chunks in an LDS bitmap over the unit's chunks, and writes the union in ascending
// order, -1 padded to G * k entries.
constexpr int kMaxHeadWords = 2048;   // bitmap words: up to 65536 historical chunks

template <int G>
__device__ __forceinline__ void select_epilogue_heads(const SelectOut& so, int u, int slot,
                                                      int nslices, const float* s_score,
                                                      int item0, int nitems, int last_items,
                                                      void* scratch, MergeCand& mc, int* s_flag,
                                                      unsigned* bits) {
    const int tid = threadIdx.x;
    const int kc = so.k < nitems ? so.k : nitems;
    for (int h = 0; h < G; ++h) {
        const float* sh = s_score + h * nitems;   // this head's scores, [item]
        const long long base = (((long long)u * G + h) * nslices + slot) * so.kcap;
        auto emit = [&](int j, int i) {
            st_shared_dev(so.cand_score + base + j, sh[i]);
            st_shared_dev(so.cand_idx + base + j, (int32_t)(item0 + i));
        };
        auto sc = [&](int i) { return sh[i]; };
        if (kc == nitems) {
            for (int i = tid; i < nitems; i += 256) emit(i, i);
        } else if (nitems <= 256) {
            small_topk(nitems, so.k, sc, emit, *reinterpret_cast<SmallTopkSmem*>(scratch));
        } else {
            block_topk(nitems, so.k, sc, emit, *reinterpret_cast<TopkSmem*>(scratch));
        }
        __syncthreads();   // the next head reuses the top-k scratch
    }
    if (!arrive_last(so.counter + u, (unsigned)nslices, s_flag)) return;

    // ---- last workgroup of the unit: every head's top-k, then the union -------------------
    const int nw = (so.H + 31) >> 5;
    for (int w = tid; w < nw; w += 256) bits[w] = 0u;
    const int ncand = (nslices - 1) * so.kcap + (so.k < last_items ? so.k : last_items);
    const bool staged = ncand <= 256;
    for (int h = 0; h < G; ++h) {
        const long long base = ((long long)u * G + h) * nslices * so.kcap;
        const float* ucs = so.cand_score + base;
        const int32_t* uci = so.cand_idx + base;
        if (staged && tid < ncand) {
            mc.score[tid] = ld_shared_dev(ucs + tid);
            mc.idx[tid] = ld_shared_dev(uci + tid);
        }
        __syncthreads();   // staged candidates (and, for h = 0, the cleared bitmap) visible
        auto score_at = [&](int i) { return staged ? mc.score[i] : ld_shared_dev(ucs + i); };
        auto mark = [&](int, int i) {
            const int32_t c = staged ? mc.idx[i] : ld_shared_dev(uci + i);
            atomicOr(&bits[c >> 5], 1u << (c & 31));
        };
        if (so.k >= ncand) {
            for (int i = tid; i < ncand; i += 256) mark(i, i);
        } else if (staged) {
            small_topk(ncand, so.k, score_at, mark, *reinterpret_cast<SmallTopkSmem*>(scratch));
        } else {
            block_topk(ncand, so.k, score_at, mark, *reinterpret_cast<TopkSmem*>(scratch));
        }
        __syncthreads();   // the next head reuses the staging and the top-k scratch
    }
    // compaction: thread t owns a run of bitmap words; its first position is the number of
    // chosen chunks in the words before its run
    const int sk = G * so.stride;
    int32_t* sel = so.sel + (long long)u * sk;
    const int wpt = (nw + 255) / 256;
    const int w0 = min(tid * wpt, nw), w1 = min(w0 + wpt, nw);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
    const int first = block_exclusive_scan(cnt, reinterpret_cast<SmallTopkSmem*>(scratch)->scan);
    if (tid == 255) *s_flag = first + cnt;   // the union's size
    int pos = first;
    for (int w = w0; w < w1; ++w) {
        unsigned m = bits[w];
        while (m) {
            sel[pos++] = w * 32 + (__ffs(m) - 1);
            m &= m - 1u;
        }
    }
    __syncthreads();
    for (int j = *s_flag + tid; j < sk; j += 256) sel[j] = -1;
}

// ---------------------------------------------------------------------------------------
// gist_kernel: grid (slices, units).  Range mode: slice y covers items (chunks, or level-2
// groups) [y*ips, min((y+1)*ips, nitems)).  Group mode (a.groups != null): slice y covers the
// member chunks of level-2 group groups[u][y].
// ---------------------------------------------------------------------------------------
template <int D, int G>
struct GistSmem {
    union alignas(16) {   // 16-byte aligned: the score pooling reads logits as float4
        float lg[kMaxSliceRows * G];                   // logits, then softmax weights
        float fin[RowStream<D, G>::NW * G * D];
        TopkSmem topk;
        SmallTopkSmem small;
    } x;
    float score[kMaxSliceRows];   // also the top-p staging of the last workgroup
    union {
        MergeCand mc;             // the merging workgroup's staged candidates
        SmallTopkSmem pub;        // deferred selection: the slice top-k, taken before the V rows
    } m;
    HeadStatsSmem<G> hs;
    ReduceSmem red;
    float lse;
    int flag;
    int chosen[64];
    int tp_keep;
};

// Softmax partial of the G heads over `nrows` rows whose logits sit in sm.x.lg (values V, the
// first batch already in vfirst) -> slot `slot`.
template <int D, int G>
__device__ __forceinline__ void fold_rows(GistSmem<D, G>& sm, const Partials& part,
                                          const uint16_t* V, int nrows,
                                          uint4 (&vfirst)[TCS_V_U], uint4 (&vsecond)[TCS_V_U],
                                          int npre, int bh0, int slot) {
    using RS = RowStream<D, G>;
    const RS rs;
    head_stats<G>(sm.x.lg, nrows, sm.hs);
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    rs.template accumulate2<TCS_V_U>(acc, V, nrows, sm.x.lg, 0, vfirst, vsecond, npre);
    __syncthreads();   // weights dead: fin may reuse the space
    rs.finish(acc, sm.hs.M, sm.hs.L, sm.x.fin, part, bh0, slot);
}

// Kernel variants, each its own instantiation so that the others compile as if it did not
// exist.  kGistMeta: the group-mode slices of the selected-summary set at two levels, whose
// softmax tokens are their groups' own level-2 gists (a.pk / a.pv).  kGistHeads: per-head
// selection (a.heads), with the union bitmap in `bits`.
constexpr int kGistPlain = 0, kGistMeta = 1, kGistHeads = 2;

template <int D, int G, int MODE>
__device__ __forceinline__ void gist_item(const GistLaunch& a, GistSmem<D, G>& sm, unsigned* bits,
                                          int y, int u) {
    using RS = RowStream<D, G>;
    const int b = u / a.Hkv, kv = u % a.Hkv;
    const int bh0 = b * a.Hq + kv * G;
    int c0, c1, last_items;
    if (a.groups) {
        const int r = a.groups[(long long)u * a.k2 + y];
        c0 = r * a.J;
        c1 = min(c0 + a.J, a.H);
        const int rl = a.groups[(long long)u * a.k2 + a.slices - 1];
        last_items = min(a.J, a.H - rl * a.J);
    } else {
        c0 = y * a.items_per_slice;
        c1 = min(c0 + a.items_per_slice, a.nitems);
        last_items = a.nitems - (a.slices - 1) * a.items_per_slice;
    }
    const int nit = max(c1 - c0, 0);
    const int nrows = nit * a.g;
    const RS rs;
    const uint16_t* K = a.gk + (long long)u * a.unit_stride + (long long)c0 * a.g * D;
    const uint16_t* V = a.gv + (long long)u * a.unit_stride + (long long)c0 * a.g * D;
    {
        uint32_t q2[G][4];
        rs.load_q(a.q + (long long)bh0 * D, q2);
        rs.template logits<TCS_K_U>(q2, K, nrows, a.sigma, 0.f, sm.x.lg, 0);
    }
    // the first V batch travels while the scores and the softmax statistics are computed
    // (two with the selection published first: pooling, the slice top-k and the statistics)
    uint4 vfirst[TCS_V_U], vsecond[TCS_V_U];
    const int npre = MODE == kGistPlain && a.selo.defer ? 2 : 1;
    if (!a.scores_only) {
        if (npre == 2) rs.template prefetch2<TCS_V_U>(V, nrows, vfirst, vsecond);
        else rs.template prefetch<TCS_V_U>(V, nrows, vfirst);
    }
    __syncthreads();
    const int ng = a.g * G;   // logits per item
    if constexpr (MODE == kGistHeads) {
        // each head's own item scores, [h][item]: log-sum-exp over the item's g gist logits of
        // that head (logit of row t, head h at lg[(item g + t) G + h])
        for (int x = threadIdx.x; x < nit * G; x += 256) {
            const int c = x / G, h = x - c * G;
            const float* l = sm.x.lg + c * ng + h;
            float mx = -INFINITY, z = 0.f;
            for (int t = 0; t < a.g; ++t) mx = fmaxf(mx, l[t * G]);
            for (int t = 0; t < a.g; ++t) z += expf(l[t * G] - mx);
            const float sc = mx + logf(z);
            sm.score[h * nit + c] = sc;
            if (a.scores_out)
                a.scores_out[((long long)u * G + h) * a.score_stride + c0 + c] = sc;
        }
    } else
    // pooled item scores: log-sum-exp over the G heads and g gists of each item
    for (int c = threadIdx.x; c < nit; c += 256) {
        const float* x = sm.x.lg + c * ng;
        float mx = -INFINITY, z = 0.f;
        if (ng % 4 == 0) {   // 16-byte LDS reads, several in flight; same summation order
#pragma unroll 4
            for (int i = 0; i < ng; i += 4) {
                const float4 v = *reinterpret_cast<const float4*>(x + i);
                mx = fmaxf(fmaxf(mx, fmaxf(v.x, v.y)), fmaxf(v.z, v.w));
            }
#pragma unroll 4
            for (int i = 0; i < ng; i += 4) {
                const float4 v = *reinterpret_cast<const float4*>(x + i);
                z += expf(v.x - mx);
                z += expf(v.y - mx);
                z += expf(v.z - mx);
                z += expf(v.w - mx);
            }
        } else {
            for (int i = 0; i < ng; ++i) mx = fmaxf(mx, x[i]);
            for (int i = 0; i < ng; ++i) z += expf(x[i] - mx);
        }
        const float s = mx + logf(z);
        sm.score[c] = s;
        if (a.scores_out) a.scores_out[(long long)u * a.score_stride + c0 + c] = s;
    }
    if constexpr (MODE == kGistPlain) {
        if (a.selo.defer) {
            // Publish this slice's list now, while the first V batch travels; the unit's
            // selection is merged by its first slice to finish (which has seen every list
            // published), so no workgroup waits for another.  The unit's counter word holds
            // the published slices in its low half and the finished ones in its high half.
            __syncthreads();   // every pooled score is in sm.score
            publish_slice(a.selo, u, y, a.slices, sm.score, c0, nit, &sm.m.pub, sm.red);
            unsigned* cnt = a.selo.counter + u;
            const unsigned S = (unsigned)a.slices;
            // count the list once every wave's part of it is out
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            wait_vmem();
            __syncthreads();
            unsigned old_p = 0u;
            if (threadIdx.x == 0) old_p = atomicAdd(cnt, 1u);
            if (!a.scores_only)
                fold_rows<D, G>(sm, a.part, V, nrows, vfirst, vsecond, npre, bh0, a.slot0 + y);
            if (threadIdx.x == 0) {
                const unsigned old_f = atomicAdd(cnt, 1u << 16);
                // the first to finish once every list is out merges; if some slice finished
                // before the last list was out, the slice that put it out merges instead
                const bool merge = ((old_f >> 16) == 0u && (old_f & 0xFFFFu) == S) ||
                                   ((old_p & 0xFFFFu) == S - 1u && (old_p >> 16) != 0u);
                if ((old_f >> 16) == S - 1u) atomicExch(cnt, 0u);   // every slice is through
                sm.flag = merge;
            }
            __syncthreads();
            if (sm.flag) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                merge_selection(a.selo, u, a.slices, last_items, &sm.lse, &sm.x, sm.m.mc,
                                sm.chosen, *reinterpret_cast<TopPSmem*>(sm.score), &sm.tp_keep);
            }
            return;
        }
    }
    if (!a.scores_only) {   // the gists are tokens of the softmax set: fold them in here
        fold_rows<D, G>(sm, a.part, V, nrows, vfirst, vsecond, npre, bh0, a.slot0 + y);
    } else if constexpr (MODE == kGistMeta) {
        // selected summaries at two levels: this group's own level-2 gists are the tokens
        const int r = a.groups[(long long)u * a.k2 + y];
        const long long off = (long long)u * a.p_unit_stride + (long long)r * a.g * D;
        __syncthreads();   // every pooled score has read its logits: lg may be overwritten
        {
            uint32_t q2[G][4];
            rs.load_q(a.q + (long long)bh0 * D, q2);
            rs.template logits<TCS_K_U>(q2, a.pk + off, a.g, a.sigma, 0.f, sm.x.lg, 0);
        }
        rs.template prefetch<TCS_V_U>(a.pv + off, a.g, vfirst);
        __syncthreads();
        fold_rows<D, G>(sm, a.part, a.pv + off, a.g, vfirst, vsecond, 1, bh0, a.slot0 + y);
    }
    __syncthreads();
    if constexpr (MODE == kGistHeads) {
        select_epilogue_heads<G>(a.selo, u, y, a.slices, sm.score, c0, nit, last_items, &sm.x,
                                 sm.m.mc, &sm.flag, bits);
    } else {
        select_epilogue(a.selo, u, y, a.slices, sm.score, c0, nit, last_items, &sm.lse, &sm.x,
                        sm.m.mc, &sm.flag, sm.chosen, sm.red,
                        // the slice scores are dead once the slice's list is out: the unit's
                        // top-p cut reuses their space
                        *reinterpret_cast<TopPSmem*>(sm.score), &sm.tp_keep);
    }
}

template <int D, int G>
struct GistHeadsSmem {
    GistSmem<D, G> base;
    unsigned bits[kMaxHeadWords];
};

template <int D, int G, int MODE>
__global__ void __launch_bounds__(256) gist_kernel(GistLaunch a) {
    if constexpr (MODE == kGistHeads) {
        __shared__ GistHeadsSmem<D, G> sm;
        gist_item<D, G, MODE>(a, sm.base, sm.bits, blockIdx.x, blockIdx.y);
    } else {
        __shared__ GistSmem<D, G> sm;
        gist_item<D, G, MODE>(a, sm, nullptr, blockIdx.x, blockIdx.y);
    }
}

// ---------------------------------------------------------------------------------------
// Fixed-order merge of every slot's partial for the G heads of one unit -> out, lse.  All
// hand-off loads are issued before any is used (one memory round trip when the slots fit).
// ---------------------------------------------------------------------------------------
constexpr int kMergeStage = 1024;   // (head, slot) softmax statistics staged in LDS

template <int G>
struct MergeSmem {
    float w[kMergeStage];    // m, then exp(m - M)
    float l[kMergeStage];
    float M[G], L[G];
};

template <int D, int G>
__device__ __forceinline__ void merge_partials(const Partials& P, int bh0, float* out, float* lse,
                               MergeSmem<G>& sm) {
    const int ns = P.nslots;
    const int tid = threadIdx.x;
    // Thread t owns the column pairs t, t + 256, ... of the unit's G heads (pair p: head
    // 2p / D, columns 2p % D and the next), read with 8-byte loads.  Every load is issued
    // unconditionally, with the slot clamped to the last one (its weight is then zero), so
    // that the whole batch is straight-line code in flight at once.
    constexpr int NP = G * D / 2;
    constexpr int PPT = (NP + 255) / 256;
    constexpr int SB = 32 / PPT;   // slots per batch: the unit's whole set for the usual counts
    const bool staged = G * ns <= kMergeStage;
    unsigned long long v[PPT][SB];
    auto pair_ptr = [&](int q) {
        const int p = min(tid + q * 256, NP - 1);
        const int h = 2 * p / D, col = 2 * p % D;
        return reinterpret_cast<const unsigned long long*>(P.acc + (long long)(bh0 + h) * ns * D +
                                                           col);
    };
    auto load_batch = [&](int s0) {
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            const unsigned long long* b = pair_ptr(q);
#pragma unroll
            for (int j = 0; j < SB; ++j)
                v[q][j] = ld_shared_dev(b + (long long)min(s0 + j, ns - 1) * (D / 2));
        }
    };
    load_batch(0);   // in flight together with the statistics below
    if (staged) {
        for (int i = tid; i < G * ns; i += 256) {
            const unsigned long long ml = ld_shared_dev(reinterpret_cast<const unsigned long long*>(
                P.ml + ((long long)(bh0 + i / ns) * ns + i % ns) * 2));
            sm.w[i] = __uint_as_float((unsigned)ml);
            sm.l[i] = __uint_as_float((unsigned)(ml >> 32));
        }
        __syncthreads();
    }
    auto m_at = [&](int h, int s) {
        return staged ? sm.w[h * ns + s] : ld_shared_dev(P.ml + ((long long)(bh0 + h) * ns + s) * 2);
    };
    auto l_at = [&](int h, int s) {
        return staged ? sm.l[h * ns + s]
                      : ld_shared_dev(P.ml + ((long long)(bh0 + h) * ns + s) * 2 + 1);
    };
    {   // per head: M = max of the slots' m, L = sum of exp(m - M) l; one wave per head
        const int lane = tid & 63;
        for (int h = tid >> 6; h < G; h += 4) {
            float mx = kNegBig;
            for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, m_at(h, s));
            mx = wave_max(mx);
            float L = 0.f;
            for (int s = lane; s < ns; s += 64) L += __expf(m_at(h, s) - mx) * l_at(h, s);
            L = wave_sum(L);
            if (lane == 0) {
                sm.M[h] = mx;
                sm.L[h] = L;
            }
        }
    }
    __syncthreads();
    if (staged) {
        for (int i = tid; i < G * ns; i += 256) sm.w[i] = __expf(sm.w[i] - sm.M[i / ns]);
        __syncthreads();
    }
    float o[PPT][2];
#pragma unroll
    for (int q = 0; q < PPT; ++q) o[q][0] = o[q][1] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += SB) {
        if (s0 > 0) load_batch(s0);
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            const int h = 2 * min(tid + q * 256, NP - 1) / D;
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int s = s0 + j;
                if (s < ns) {
                    const float w = staged ? sm.w[h * ns + s] : __expf(m_at(h, s) - sm.M[h]);
                    o[q][0] = fmaf(w, __uint_as_float((unsigned)v[q][j]), o[q][0]);
                    o[q][1] = fmaf(w, __uint_as_float((unsigned)(v[q][j] >> 32)), o[q][1]);
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
        const int p = tid + q * 256;
        if (p < NP) {
            const int h = 2 * p / D, col = 2 * p % D;
            float* op = out + (long long)(bh0 + h) * D + col;
            op[0] = o[q][0] / sm.L[h];
            op[1] = o[q][1] / sm.L[h];
            if (lse && col == 0) lse[bh0 + h] = sm.M[h] + logf(sm.L[h]);
        }
    }
}

// ---------------------------------------------------------------------------------------
// chunk_kernel: grid (ceil((kslots + 1) / cpw), units).  Workgroup x streams slots
// [x*cpw, (x+1)*cpw): slot j < kslots is selected chunk sel[u][j] (skipped if -1), slot
// kslots is the current chunk (tokens [(M-1)C, N)).  Each chunk's raw tokens carry its gate
// bias.  The last workgroup of a unit merges every partial of the unit's G heads.
// ---------------------------------------------------------------------------------------
constexpr int kMaxCpw = 16;

template <int D, int G>
struct ChunkSmem {
    union {
        float lg[kMaxSliceRows * G];
        float fin[RowStream<D, G>::NW * G * D];
        MergeSmem<G> merge;
    } x;
    HeadStatsSmem<G> hs;
    int page[kMaxCpw];
    float bias[kMaxCpw];
    int rb[kMaxCpw];      // first row of the slot's chunk this workgroup reads
    int rows[kMaxCpw];    // rows read from it
    int lrow[kMaxCpw];    // their place in the logits
    int chunk[kMaxCpw];   // selected chunk of the slot, -1 for the current chunk
    int flag;
};

// Workgroup wx of unit u (nwx workgroups per unit).
template <int D, int G, int CVU>
__device__ __forceinline__ void chunk_item(const ChunkLaunch& a, ChunkSmem<D, G>& sm, int wx,
                                           int u, int nwx) {
    using RS = RowStream<D, G>;
    const int b = u / a.Hkv, kv = u % a.Hkv;
    const int bh0 = b * a.Hq + kv * G;
    const int rows_cur = a.N - (a.M - 1) * a.C;
    // Row mode (rpw > 0): the slots' rows laid end to end -- slot j < kslots is C rows from
    // j C, the current chunk rows_cur rows from kslots C -- and this workgroup takes rows
    // [r0, r1).  Slot mode: whole slots [j0, j0 + nj).
    int j0, nj, r0 = 0, r1 = 0;
    if (a.rpw > 0) {
        r0 = wx * a.rpw;
        r1 = min(a.kslots * a.C + rows_cur, r0 + a.rpw);
        j0 = r0 / a.C;
        nj = (r1 - 1) / a.C - j0 + 1;
    } else {
        j0 = wx * a.cpw;
        nj = min(a.cpw, a.kslots + 1 - j0);
    }
    // this workgroup's chunks: page, gate bias and rows (page -1: none, -2: out of range)
    if (threadIdx.x < nj) {
        const int j = j0 + threadIdx.x;
        int c, rows;
        float bias = 0.f;
        if (j < a.kslots) {
            c = a.sel[(long long)u * a.k + j];
            if (c >= 0 && a.gamma) bias = a.gamma[(long long)u * a.k + j];
            rows = a.C;
        } else {
            c = a.M - 1;
            rows = a.N - (a.M - 1) * a.C;
        }
        int page = -1;
        if (c >= 0) {
            page = a.page_table[(long long)b * a.max_chunks + c];
            if (page < 0 || page >= a.num_pages) page = -2;
        }
        int rb = 0, lrow = threadIdx.x * a.C;
        if (a.rpw > 0) {   // clip the slot's rows to [r0, r1)
            rb = max(r0 - j * a.C, 0);
            rows = min(r1 - j * a.C, rows) - rb;
            lrow = j * a.C + rb - r0;
        }
        sm.page[threadIdx.x] = page;
        sm.bias[threadIdx.x] = bias;
        sm.rb[threadIdx.x] = rb;
        sm.rows[threadIdx.x] = rows;
        sm.lrow[threadIdx.x] = lrow;
        sm.chunk[threadIdx.x] = j < a.kslots ? c : -1;
    }
    // LDS rows: row mode, row r0 + i at i; slot mode, the raw rows of slot jj at [jj C, jj C +
    // rows), then (selected-gist token set) the g gist rows of slot jj at [nj C + jj g, ... + g)
    const int graw = a.rpw > 0 ? r1 - r0 : nj * a.C;
    const int nrows_all = graw + (a.gk ? nj * a.g : 0);
    for (int i = threadIdx.x; i < nrows_all * G; i += 256) sm.x.lg[i] = -INFINITY;
    __syncthreads();
    bool bad = false, any = false;
    for (int jj = 0; jj < nj; ++jj) {
        bad |= sm.page[jj] == -2;
        any |= sm.page[jj] >= 0;
    }
    const RS rs;
    if (bad) {
        write_empty_partial(a.part, bh0, G, D, a.slot0 + wx, NAN, NAN);
    } else if (!any) {
        write_empty_partial(a.part, bh0, G, D, a.slot0 + wx, 0.f, 0.f);
    } else {
        {
            uint32_t q2[G][4];
            rs.load_q(a.q + (long long)bh0 * D, q2);
            for (int jj = 0; jj < nj; ++jj) {
                if (sm.page[jj] < 0) continue;
                const long long off =
                    (((long long)sm.page[jj] * a.Hkv + kv) * a.C + sm.rb[jj]) * D;
                rs.template logits<TCS_CK_U>(q2, a.kp + off, sm.rows[jj], a.sigma, sm.bias[jj],
                                            sm.x.lg, sm.lrow[jj]);
                if (a.gk && sm.chunk[jj] >= 0)
                    rs.template logits<TCS_CK_U>(
                        q2, a.gk + (long long)u * a.gist_stride + (long long)sm.chunk[jj] * a.g * D,
                        a.g, a.sigma, 0.f, sm.x.lg, graw + jj * a.g);
            }
        }
        // the first slot's first V batch travels while the softmax statistics are computed
        int jfirst = 0;
        while (sm.page[jfirst] < 0) ++jfirst;   // `any` holds: some slot has a page
        uint4 vb[CVU];
        rs.template prefetch<CVU>(
            a.vp + (((long long)sm.page[jfirst] * a.Hkv + kv) * a.C + sm.rb[jfirst]) * D,
            sm.rows[jfirst], vb);
        __syncthreads();
        head_stats<G>(sm.x.lg, nrows_all, sm.hs);
        float acc[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
        for (int jj = jfirst; jj < nj; ++jj) {
            if (sm.page[jj] < 0) continue;
            const long long off = (((long long)sm.page[jj] * a.Hkv + kv) * a.C + sm.rb[jj]) * D;
            rs.template accumulate<CVU>(acc, a.vp + off, sm.rows[jj], sm.x.lg, sm.lrow[jj],
                                             vb, jj == jfirst);
            if (a.gk && sm.chunk[jj] >= 0)
                rs.template accumulate<CVU>(
                    acc, a.gv + (long long)u * a.gist_stride + (long long)sm.chunk[jj] * a.g * D,
                    a.g, sm.x.lg, graw + jj * a.g, vb);
        }
        __syncthreads();
        rs.finish(acc, sm.hs.M, sm.hs.L, sm.x.fin, a.part, bh0, a.slot0 + wx);
    }
    if (!arrive_last(a.counter + u, (unsigned)nwx, &sm.flag)) return;
    merge_partials<D, G>(a.part, bh0, a.out, a.lse, sm.x.merge);
}

template <int D, int G, int CVU>
__global__ void __launch_bounds__(256) chunk_kernel(ChunkLaunch a) {
    __shared__ ChunkSmem<D, G> sm;
    chunk_item<D, G, CVU>(a, sm, blockIdx.x, blockIdx.y, gridDim.x);
}

// ---------------------------------------------------------------------------------------
// small fill kernels (workspace initialisation; empty selections)
// ---------------------------------------------------------------------------------------
__global__ void zero_kernel(unsigned* p, long long n) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        p[i] = 0u;
}

__global__ void fill_kernel(int32_t* p, long long n, int32_t v) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        p[i] = v;
}

// Plain streaming read: every 16-byte unit of [p, p + n16) is loaded once (non-temporal, four
// in flight per lane) and folded into one word per workgroup, so that nothing is skipped.  The
// HBM ceiling the decode kernels are measured against.
__global__ void __launch_bounds__(256) stream_read_kernel(const uint16_t* p, long long n16,
                                                          unsigned* sink) {
    // Each workgroup reads one contiguous range, 8 loads of 16 B per thread in flight (a wave
    // covers 8 KB per step): on gfx950 this reads faster than a grid-stride walk of the same
    // bytes (6.2 against 5.6 TB/s for 2 GiB, measured on one box).
    constexpr int U = 8, STEP = 256 * U;
    const long long per = ((n16 + gridDim.x - 1) / gridDim.x + STEP - 1) / STEP * STEP;
    const long long lo = blockIdx.x * per, hi = min(lo + per, n16);
    unsigned acc = 0u;
    for (long long base = lo; base < hi; base += STEP) {
        uint4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long i = base + u * 256 + threadIdx.x;
            r[u] = i < hi ? ld16(p + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
    }
    __shared__ unsigned red[4];
    for (int off = 32; off >= 1; off >>= 1) acc ^= (unsigned)__shfl_xor((int)acc, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_stream_read(const void* p, size_t bytes, unsigned* sink, int blocks,
                              hipStream_t s) {
    const long long n16 = (long long)(bytes / 16);
    if (n16 <= 0) return hipSuccess;
    stream_read_kernel<<<blocks, 256, 0, s>>>((const uint16_t*)p, n16, sink);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
template <int D, int MODE>
static hipError_t gist_d(const GistLaunch& a, hipStream_t s, dim3 grid, const KernelEvents& ev) {
    switch (a.Hq / a.Hkv) {
        case 1: return dispatch(gist_kernel<D, 1, MODE>, grid, dim3(256), 0, s, ev, a);
        case 2: return dispatch(gist_kernel<D, 2, MODE>, grid, dim3(256), 0, s, ev, a);
        case 4: return dispatch(gist_kernel<D, 4, MODE>, grid, dim3(256), 0, s, ev, a);
        case 8: return dispatch(gist_kernel<D, 8, MODE>, grid, dim3(256), 0, s, ev, a);
        default: return hipErrorInvalidValue;
    }
}

template <int MODE>
static hipError_t gist_mode(const GistLaunch& a, hipStream_t s, dim3 grid,
                            const KernelEvents& ev) {
    return a.d == 128 ? gist_d<128, MODE>(a, s, grid, ev) : gist_d<64, MODE>(a, s, grid, ev);
}

hipError_t launch_gist(const GistLaunch& a, hipStream_t s, const KernelEvents& ev) {
    if (a.slices <= 0) return no_kernel(ev, s);
    dim3 grid(a.slices, a.B * a.Hkv);
    if (a.pk) {   // only group mode with scores_only carries level-2 gists for the partials
        if (!a.groups || !a.scores_only || !a.pv || a.heads) return hipErrorInvalidValue;
        return gist_mode<kGistMeta>(a, s, grid, ev);
    }
    if (a.selo.defer && (a.groups || a.heads || a.selo.top_p > 0.f || a.selo.fill_scores ||
                         a.items_per_slice > 256 || a.slices > 0xFFFF))
        return hipErrorInvalidValue;
    if (a.heads) {
        // range mode only; every head's scores of a slice fit the score buffer; the union
        // bitmap covers every chunk
        const int G = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
        if (a.groups || (long long)a.items_per_slice * G > kMaxSliceRows ||
            a.nitems > kMaxHeadWords * 32 || a.selo.H != a.nitems)
            return hipErrorInvalidValue;
        return gist_mode<kGistHeads>(a, s, grid, ev);
    }
    return gist_mode<kGistPlain>(a, s, grid, ev);
}

template <int D, int CVU>
static hipError_t chunk_dv(const ChunkLaunch& a, hipStream_t s, dim3 grid,
                           const KernelEvents& ev) {
    switch (a.Hq / a.Hkv) {
        case 1: return dispatch(chunk_kernel<D, 1, CVU>, grid, dim3(256), 0, s, ev, a);
        case 2: return dispatch(chunk_kernel<D, 2, CVU>, grid, dim3(256), 0, s, ev, a);
        case 4: return dispatch(chunk_kernel<D, 4, CVU>, grid, dim3(256), 0, s, ev, a);
        case 8: return dispatch(chunk_kernel<D, 8, CVU>, grid, dim3(256), 0, s, ev, a);
        default: return hipErrorInvalidValue;
    }
}
template <int D>
static hipError_t chunk_d(const ChunkLaunch& a, hipStream_t s, dim3 grid,
                          const KernelEvents& ev) {
    return a.rpw > 0 ? chunk_dv<D, TCS_CV_U>(a, s, grid, ev)
                     : chunk_dv<D, TCS_CV_U_SLOTS>(a, s, grid, ev);
}

hipError_t launch_chunks(const ChunkLaunch& a, hipStream_t s, const KernelEvents& ev) {
    if (a.cpw < 1 || a.cpw > kMaxCpw || (long long)a.cpw * a.C > kMaxSliceRows)
        return hipErrorInvalidValue;
    int nwx = (a.kslots + 1 + a.cpw - 1) / a.cpw;
    if (a.rpw > 0) {   // row mode: no selected gists; a workgroup spans at most kMaxCpw slots
        const long long R = (long long)a.kslots * a.C + (a.N - (long long)(a.M - 1) * a.C);
        if (a.gk || a.rpw > kMaxSliceRows || (long long)(a.rpw + a.C - 1) / a.C + 1 > kMaxCpw)
            return hipErrorInvalidValue;
        nwx = (int)((R + a.rpw - 1) / a.rpw);
    }
    dim3 grid(nwx, a.B * a.Hkv);
    return a.d == 128 ? chunk_d<128>(a, s, grid, ev) : chunk_d<64>(a, s, grid, ev);
}

hipError_t launch_fill(int32_t* p, long long n, int32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    long long blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    fill_kernel<<<(unsigned)blocks, 256, 0, s>>>(p, n, v);
    return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
    const long long n = (long long)(bytes / sizeof(unsigned));
    if (n <= 0) return hipSuccess;
    long long blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    zero_kernel<<<(unsigned)blocks, 256, 0, s>>>((unsigned*)p, n);
    return hipGetLastError();
}

}  // namespace tcs
