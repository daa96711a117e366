// decode.hip -- gfx950 kernels of the chunk-sparse decode path.
//
//   gist_kernel   scores every historical chunk of a (b, kv) unit against the G query heads of
//                 its group through the chunk's gist keys ("Simplified Sparse Attention via
//                 Gist Tokens", section 3.2), pools them into one log-sum-exp score per chunk,
//                 and -- because gists are tokens of the softmax set themselves -- folds the
//                 same gist rows into per-slice softmax partials with the gist values.  The
//                 last workgroup of a unit to finish merges the slices' candidate lists into
//                 the unit's top-k (section 3.3; ties to the lower index) and, with the SAS
//                 gate on, the gate log p_c over all historical scores ("SAS", abstract).
//   chunk_kernel  split-K attention over the selected chunks and the current chunk, read
//                 through the page table (section 3.6: only the selected keys are touched);
//                 the last workgroup of a unit merges all partials in a fixed order.
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

#include <algorithm>

namespace tcs {

constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for empty softmax state
constexpr int kMaxSliceRows = 1024;   // rows (gists, or page rows) one workgroup holds logits for

#ifndef TCS_K_U
#define TCS_K_U 8       // row passes per batch of loads in the K phase
#endif
#ifndef TCS_V_U
#define TCS_V_U 4       // row passes per batch of loads in the V phase
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

    // A workgroup's rows come in segments (one gist slice, or one page per chunk); segment j
    // has seg.rows(j) rows starting at seg.k(j) / seg.v(j) and owns LDS rows
    // [seg.row0(j), seg.row0(j) + rows).  Each phase walks batches of U row passes, segment
    // after segment, with the next batch's loads issued before the current batch is used.
    template <int U, class Seg>
    __device__ void load_batch(const Seg& seg, int nb, int t, bool v, uint4 (&r)[U]) const {
        const int j = t / nb, b = t - (t / nb) * nb;
        const int rows = seg.rows(j);
        const uint16_t* p = v ? seg.v(j) : seg.k(j);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = (b * U + u) * RPP + lrow;
            r[u] = row < rows ? ld16(p + (long long)row * D + part * 8) : make_uint4(0, 0, 0, 0);
        }
    }

    template <int U, class Seg>
    __device__ void use_k(const uint32_t (&q2)[G][4], const Seg& seg, int nb, int t, float sigma,
                          const uint4 (&r)[U], float* lg) const {
        const int j = t / nb, b = t - (t / nb) * nb;
        const int rows = seg.rows(j), row0 = seg.row0(j);
        const float bias = seg.bias(j);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = (b * U + u) * RPP + lrow;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float s = dot2(q2[h][0], r[u].x, 0.f);
                s = dot2(q2[h][1], r[u].y, s);
                s = dot2(q2[h][2], r[u].z, s);
                s = dot2(q2[h][3], r[u].w, s);
                s = group_sum<LPR>(s);
                if (part == 0 && row < rows) lg[(row0 + row) * G + h] = fmaf(s, sigma, bias);
            }
        }
    }

    template <int U, class Seg>
    __device__ void use_v(const Seg& seg, int nb, int t, const uint4 (&r)[U], const float* w,
                          float (&acc)[G][8]) const {
        const int j = t / nb, b = t - (t / nb) * nb;
        const int rows = seg.rows(j), row0 = seg.row0(j);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = (b * U + u) * RPP + lrow;
            if (row < rows) {
                float vf[8];
                unpack8(r[u], vf);
                const float* wr = w + (row0 + row) * G;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float wh = wr[h];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(wh, vf[e], acc[h][e]);
                }
            }
        }
    }

    // K phase over all segments: lg[(row0 + r) * G + h] = sigma * q_h . K[r] + bias.
    template <int U, class Seg>
    __device__ void logits(const uint32_t (&q2)[G][4], const Seg& seg, int nseg, int max_rows,
                           float sigma, float* lg) const {
        const int nb = (max_rows + U * RPP - 1) / (U * RPP);
        const int total = nseg * nb;
        if (total <= 0) return;
        uint4 b0[U], b1[U];
        load_batch<U>(seg, nb, 0, false, b0);
        for (int t = 0; t < total; t += 2) {
            if (t + 1 < total) load_batch<U>(seg, nb, t + 1, false, b1);
            use_k<U>(q2, seg, nb, t, sigma, b0, lg);
            if (t + 1 < total) {
                if (t + 2 < total) load_batch<U>(seg, nb, t + 2, false, b0);
                use_k<U>(q2, seg, nb, t + 1, sigma, b1, lg);
            }
        }
    }

    // V phase over all segments, weights w[(row0 + r) * G + h]; b0 holds batch 0, loaded by
    // the caller with load_batch (so its latency can overlap other work).
    template <int U, class Seg>
    __device__ void accumulate(const Seg& seg, int nseg, int max_rows, const float* w,
                               uint4 (&b0)[U], float (&acc)[G][8]) const {
        const int nb = (max_rows + U * RPP - 1) / (U * RPP);
        const int total = nseg * nb;
        uint4 b1[U];
        for (int t = 0; t < total; t += 2) {
            if (t + 1 < total) load_batch<U>(seg, nb, t + 1, true, b1);
            use_v<U>(seg, nb, t, b0, w, acc);
            if (t + 1 < total) {
                if (t + 2 < total) load_batch<U>(seg, nb, t + 2, true, b0);
                use_v<U>(seg, nb, t + 1, b1, w, acc);
            }
        }
    }

    // Sum the lane groups' accumulators and write one partial per head:
    // acc -> P.acc[(bh0 + h) * nslots + slot][0..D), (M[h], L[h]) -> P.ml[...][0..2).
    // fin must hold NW * G * D floats.
    __device__ void finish(float (&acc)[G][8], const float* M, const float* L, float* fin,
                           const Partials& P, int bh0, int slot) const {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
        for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
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
__device__ __forceinline__ void head_stats(float* lg, int n, HeadStatsSmem<G>& sm) {
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
// Selection shared by the scoring passes, in two steps.  select_publish (every workgroup,
// right after its scores are known): keep the best min(k, items in the slice) of the slice's
// items (ascending), hand them off with their scores, and count the workgroup in; the
// atomic's result is only looked at later, so its latency hides under the V stream.
// select_merge (the workgroup that arrived last, at its end): merge the slices' lists --
// ascending item order, slice after slice -- into the unit's top-k.  Ties go to the lower item
// index at both steps, so the result equals a top-k over all items at once.
// ---------------------------------------------------------------------------------------
struct MergeCand {
    float score[256];
    int32_t idx[256];
};

constexpr int kStagedSlices = 128;   // slice statistics the merge stages in LDS

struct SelectSmem {
    TopkSmem topk;
    SmallTopkSmem small;
    ReduceSmem red;
    MergeCand mc;
    float slse[2 * kStagedSlices];
    float lse;
    int flag;
    int chosen[64];
};

// Returns, in thread 0, the arrival counter's value before this workgroup's increment.
__device__ __forceinline__ unsigned select_publish(const SelectOut& so, int u, int slot, int nslices,
                                   const float* s_score, int item0, int nitems, SelectSmem& ss) {
    const int tid = threadIdx.x;
    const int kc = so.k < nitems ? so.k : nitems;
    float* cs = so.cand_score + ((long long)u * nslices + slot) * so.kcap;
    int32_t* ci = so.cand_idx + ((long long)u * nslices + slot) * so.kcap;
    // slice statistics for the gate: max and sum of exp over this slice's scores
    if (so.slice_lse) {
        float mx = -INFINITY;
        for (int i = tid; i < nitems; i += 256) mx = fmaxf(mx, s_score[i]);
        mx = block_max(mx, ss.red);
        float z = 0.f;
        for (int i = tid; i < nitems; i += 256) z += expf(s_score[i] - mx);
        z = block_sum(z, ss.red);
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
        small_topk(nitems, so.k, sc, emit, ss.small);
    } else {
        block_topk(nitems, so.k, sc, emit, ss.topk);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    wait_vmem();                      // this wave's hand-off stores have completed
    __syncthreads();
    unsigned old = 0;
    if (tid == 0) old = atomicAdd(so.counter + u, 1u);
    return old;
}

// All threads call this with the counter value select_publish returned.  True in the
// workgroup that arrived last (which also returns the counter to zero).
__device__ __forceinline__ bool select_is_last(const SelectOut& so, int u, int nslices, unsigned old,
                               SelectSmem& ss) {
    if (threadIdx.x == 0) {
        const bool last = old == (unsigned)nslices - 1u;
        if (last) atomicExch(so.counter + u, 0u);
        ss.flag = last;
    }
    __syncthreads();
    const bool last = ss.flag != 0;
    if (last) {
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    return last;
}

// The last workgroup merges the slices' candidates into sel (and the gate), written with
// hand-off stores so that workgroups of the same kernel may read them.
__device__ __forceinline__ void select_merge(const SelectOut& so, int u, int nslices, int last_items,
                             SelectSmem& ss) {
    const int tid = threadIdx.x;
    const float* ucs = so.cand_score + (long long)u * nslices * so.kcap;
    const int32_t* uci = so.cand_idx + (long long)u * nslices * so.kcap;
    const int ncand = (nslices - 1) * so.kcap + (so.k < last_items ? so.k : last_items);
    const bool staged = ncand <= 256;
    // one round trip for every hand-off value this workgroup needs
    const float* sl = so.slice_lse ? so.slice_lse + (long long)u * nslices * 2 : nullptr;
    const bool gate = sl && so.gamma;
    const bool lse_staged = nslices <= kStagedSlices;
    if (staged && tid < ncand) {
        ss.mc.score[tid] = ld_shared_dev(ucs + tid);
        ss.mc.idx[tid] = ld_shared_dev(uci + tid);
    }
    if (gate && lse_staged)
        for (int i = tid; i < 2 * nslices; i += 256) ss.slse[i] = ld_shared_dev(sl + i);
    __syncthreads();
    float lse = 0.f;
    if (gate) {
        auto at = [&](int i) { return lse_staged ? ss.slse[i] : ld_shared_dev(sl + i); };
        if (tid == 0) {
            float mx = -INFINITY;
            for (int s = 0; s < nslices; ++s) mx = fmaxf(mx, at(2 * s));
            float z = 0.f;
            for (int s = 0; s < nslices; ++s) z += at(2 * s + 1) * expf(at(2 * s) - mx);
            ss.lse = mx + logf(z);
        }
        __syncthreads();
        lse = ss.lse;
    }
    int32_t* sel = so.sel + (long long)u * so.k;
    float* gam = so.gamma ? so.gamma + (long long)u * so.k : nullptr;
    auto score_at = [&](int i) { return staged ? ss.mc.score[i] : ld_shared_dev(ucs + i); };
    auto emit2 = [&](int j, int i) {
        const int32_t c = staged ? ss.mc.idx[i] : ld_shared_dev(uci + i);
        st_shared_dev(sel + j, c);
        if (gam) st_shared_dev(gam + j, score_at(i) - lse);
        if (j < 64) ss.chosen[j] = c;
    };
    int ke;
    if (so.k >= ncand) {
        for (int i = tid; i < ncand; i += 256) emit2(i, i);
        ke = ncand;
    } else if (staged) {
        ke = small_topk(ncand, so.k, score_at, emit2, ss.small);
    } else {
        ke = block_topk(ncand, so.k, score_at, emit2, ss.topk);
    }
    for (int j = ke + tid; j < so.k; j += 256) {
        st_shared_dev(sel + j, (int32_t)-1);
        if (gam) st_shared_dev(gam + j, 0.f);
    }
    if (so.fill_scores) {
        // two-level group pass: chunks outside the chosen groups are never scored
        __syncthreads();
        float* fs = so.fill_scores + (long long)u * so.H;
        for (int c = tid; c < so.H; c += 256) {
            const int r = c / so.J;
            bool in = false;
            for (int j = 0; j < ke && j < 64; ++j) in |= ss.chosen[j] == r;
            if (!in) fs[c] = -INFINITY;
        }
    }
}

// Bounded wait until *flag != 0 (thread 0 polls, the workgroup waits at a barrier).  Returns
// false if the flag did not come up within `limit` polls; the caller then poisons its result
// instead of waiting on.
__device__ __forceinline__ bool wait_flag(const unsigned* flag, unsigned limit, int* s_ok) {
    if (threadIdx.x == 0) {
        unsigned n = 0;
        int ok = 1;
        while (ld_shared_dev(flag) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++n >= limit) { ok = 0; break; }
        }
        *s_ok = ok;
    }
    __syncthreads();
    const bool ok = *s_ok != 0;
    wait_vmem();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return ok;
}

// Raise *flag after this workgroup's hand-off stores have completed.
__device__ __forceinline__ void raise_flag(unsigned* flag) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0) st_shared_dev(flag, 1u);
}

// One contiguous run of gist rows (K and V), LDS rows from 0.
struct GistSeg {
    const uint16_t* kp;
    const uint16_t* vp;
    int n;
    __device__ const uint16_t* k(int) const { return kp; }
    __device__ const uint16_t* v(int) const { return vp; }
    __device__ int rows(int) const { return n; }
    __device__ int row0(int) const { return 0; }
    __device__ float bias(int) const { return 0.f; }
};

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
    constexpr int PPT = (G * D + 255) / 256;   // (head, column) outputs per thread
#ifndef TCS_MERGE_SB
#define TCS_MERGE_SB 32
#endif
    constexpr int SB = TCS_MERGE_SB / PPT;     // slots whose values one batch holds
    const bool staged = G * ns <= kMergeStage;
    float v[PPT][SB];
    auto load_batch = [&](int s0) {
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            const int p = tid + q * 256;
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int s = s0 + j;
                v[q][j] = (p < G * D && s < ns)
                              ? ld_shared_dev(P.acc + ((long long)(bh0 + p / D) * ns + s) * D + p % D)
                              : 0.f;
            }
        }
    };
    load_batch(0);   // in flight together with the statistics below
    if (staged) {
        for (int i = tid; i < G * ns; i += 256) {
            const float* ml = P.ml + ((long long)(bh0 + i / ns) * ns + i % ns) * 2;
            sm.w[i] = ld_shared_dev(ml);
            sm.l[i] = ld_shared_dev(ml + 1);
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
    if (tid < G) {
        float mx = kNegBig;
        for (int s = 0; s < ns; ++s) mx = fmaxf(mx, m_at(tid, s));
        float L = 0.f;
        for (int s = 0; s < ns; ++s) L += __expf(m_at(tid, s) - mx) * l_at(tid, s);
        sm.M[tid] = mx;
        sm.L[tid] = L;
    }
    __syncthreads();
    if (staged) {
        for (int i = tid; i < G * ns; i += 256) sm.w[i] = __expf(sm.w[i] - sm.M[i / ns]);
        __syncthreads();
    }
    float o[PPT];
#pragma unroll
    for (int q = 0; q < PPT; ++q) o[q] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += SB) {
        if (s0 > 0) load_batch(s0);
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            const int p = tid + q * 256;
            if (p < G * D) {
                const int h = p / D;
#pragma unroll
                for (int j = 0; j < SB; ++j) {
                    const int s = s0 + j;
                    if (s < ns) {
                        const float w = staged ? sm.w[h * ns + s] : __expf(m_at(h, s) - sm.M[h]);
                        o[q] = fmaf(w, v[q][j], o[q]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
        const int p = tid + q * 256;
        if (p < G * D) {
            const int h = p / D, col = p % D;
            out[(long long)(bh0 + h) * D + col] = o[q] / sm.L[h];
            if (lse && col == 0) lse[bh0 + h] = sm.M[h] + logf(sm.L[h]);
        }
    }
}

// Final merge: which counter, how many arrivals, and where the result goes.
struct FinalMerge {
    unsigned* counter;    // [units]
    unsigned total;       // arrivals per unit
    float* out;
    float* lse;
    unsigned* ready;      // persistent kernel: the selection flags to lower again, else null
};

// ---------------------------------------------------------------------------------------
// gist item: one slice of a unit.  Range mode: slice y covers items (chunks, or level-2
// groups) [y*ips, min((y+1)*ips, nitems)).  Group mode (a.groups != null): slice y covers the
// member chunks of level-2 group groups[u][y].  With `fm` the slice also counts towards the
// unit's final merge (persistent kernel), and `ready` is raised once the selection is made.
// ---------------------------------------------------------------------------------------
template <int D, int G>
struct GistSmem {
    union {
        float lg[kMaxSliceRows * G];                   // logits, then softmax weights
        float fin[RowStream<D, G>::NW * G * D];
        MergeSmem<G> merge;
    } x;
    float score[kMaxSliceRows];
    HeadStatsSmem<G> hs;
    SelectSmem ss;
    int flag;
};

// The chunks (or level-2 groups) of slice y of unit u.
struct SliceRange {
    int c0, nit, nrows, last_items;
};

__device__ __forceinline__ SliceRange slice_range(const GistLaunch& a, int u, int y) {
    SliceRange r;
    int c1;
    if (a.groups) {
        const int g = ld_shared_dev(a.groups + (long long)u * a.k2 + y);
        r.c0 = g * a.J;
        c1 = min(r.c0 + a.J, a.H);
        const int gl = ld_shared_dev(a.groups + (long long)u * a.k2 + a.slices - 1);
        r.last_items = min(a.J, a.H - gl * a.J);
    } else {
        r.c0 = y * a.items_per_slice;
        c1 = min(r.c0 + a.items_per_slice, a.nitems);
        r.last_items = a.nitems - (a.slices - 1) * a.items_per_slice;
    }
    r.nit = max(c1 - r.c0, 0);
    r.nrows = r.nit * a.g;
    return r;
}

template <int D>
__device__ __forceinline__ GistSeg gist_seg(const GistLaunch& a, int u, const SliceRange& r) {
    return GistSeg{a.gk + (long long)u * a.unit_stride + (long long)r.c0 * a.g * D,
                   a.gv + (long long)u * a.unit_stride + (long long)r.c0 * a.g * D, r.nrows};
}

// Scoring part of a gist item: logits of the slice's gist keys (LDS), pooled item scores,
// and the selection hand-off.  Returns (thread 0) the selection counter's old value.
template <int D, int G>
__device__ __forceinline__ unsigned gist_front(const GistLaunch& a, int u, int y,
                                               const SliceRange& r, GistSmem<D, G>& sm) {
    using RS = RowStream<D, G>;
    const int bh0 = (u / a.Hkv) * a.Hq + (u % a.Hkv) * G;
    const RS rs;
    const GistSeg seg = gist_seg<D>(a, u, r);
    {
        uint32_t q2[G][4];
        rs.load_q(a.q + (long long)bh0 * D, q2);
        rs.template logits<TCS_K_U>(q2, seg, 1, r.nrows, a.sigma, sm.x.lg);
    }
    __syncthreads();
    // pooled item scores: log-sum-exp over the G heads and g gists of each item
    for (int c = threadIdx.x; c < r.nit; c += 256) {
        const float* x = sm.x.lg + c * a.g * G;
        float mx = -INFINITY;
        for (int i = 0; i < a.g * G; ++i) mx = fmaxf(mx, x[i]);
        float z = 0.f;
        for (int i = 0; i < a.g * G; ++i) z += expf(x[i] - mx);
        const float sc = mx + logf(z);
        sm.score[c] = sc;
        if (a.scores_out) a.scores_out[(long long)u * a.score_stride + r.c0 + c] = sc;
    }
    __syncthreads();
    return select_publish(a.selo, u, y, a.slices, sm.score, r.c0, r.nit, sm.ss);
}

// Whole gist item (scoring, selection, then the V rows of the slice) for the separate-kernel
// path.
template <int D, int G>
__device__ __forceinline__ void gist_item(const GistLaunch& a, int u, int y, GistSmem<D, G>& sm) {
    using RS = RowStream<D, G>;
    const int bh0 = (u / a.Hkv) * a.Hq + (u % a.Hkv) * G;
    const SliceRange r = slice_range(a, u, y);
    const unsigned old = gist_front<D, G>(a, u, y, r, sm);
    const RS rs;
    const GistSeg seg = gist_seg<D>(a, u, r);
    uint4 vb[TCS_V_U];
    rs.template load_batch<TCS_V_U>(seg, (r.nrows + TCS_V_U * RS::RPP - 1) / (TCS_V_U * RS::RPP),
                                    0, true, vb);   // first V batch in flight from here on
    if (select_is_last(a.selo, u, a.slices, old, sm.ss)) select_merge(a.selo, u, a.slices, r.last_items, sm.ss);
    head_stats<G>(sm.x.lg, r.nrows, sm.hs);
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    rs.template accumulate<TCS_V_U>(seg, 1, r.nrows, sm.x.lg, vb, acc);
    __syncthreads();   // weights dead: fin may reuse the space
    rs.finish(acc, sm.hs.M, sm.hs.L, sm.x.fin, a.part, bh0, a.slot0 + y);
}

// Persistent-kernel K item: scoring and selection, then the slice's softmax weights and
// statistics go to the stash for its V item, and the slice's flag is raised.
template <int D, int G>
__device__ __forceinline__ void gist_k_item(const GistLaunch& a, const FusedCtl& ctl, int u,
                                            int y, GistSmem<D, G>& sm) {
    const SliceRange r = slice_range(a, u, y);
    const unsigned old = gist_front<D, G>(a, u, y, r, sm);
    head_stats<G>(sm.x.lg, r.nrows, sm.hs);
    const long long sl = (long long)u * a.slices + y;
    float* w = ctl.wstash + sl * ctl.stash_rows * G;
    for (int i = threadIdx.x; i < r.nrows * G; i += 256) st_shared_dev(w + i, sm.x.lg[i]);
    if (threadIdx.x < G) {
        st_shared_dev(ctl.sstash + (sl * G + threadIdx.x) * 2, sm.hs.M[threadIdx.x]);
        st_shared_dev(ctl.sstash + (sl * G + threadIdx.x) * 2 + 1, sm.hs.L[threadIdx.x]);
    }
    raise_flag(ctl.kdone + sl);
    if (select_is_last(a.selo, u, a.slices, old, sm.ss)) {
        select_merge(a.selo, u, a.slices, r.last_items, sm.ss);
        raise_flag(ctl.ready + u);
    }
}

// Persistent-kernel V item: the V rows of a slice, weighted by the stashed softmax weights,
// into the slice's partial; counts towards the unit's final merge.
template <int D, int G>
__device__ __forceinline__ void gist_v_item(const GistLaunch& a, const FusedCtl& ctl,
                                            const FinalMerge& fm, int u, int y,
                                            GistSmem<D, G>& sm) {
    using RS = RowStream<D, G>;
    const int bh0 = (u / a.Hkv) * a.Hq + (u % a.Hkv) * G;
    const SliceRange r = slice_range(a, u, y);
    const RS rs;
    const GistSeg seg = gist_seg<D>(a, u, r);
    uint4 vb[TCS_V_U];
    rs.template load_batch<TCS_V_U>(seg, (r.nrows + TCS_V_U * RS::RPP - 1) / (TCS_V_U * RS::RPP),
                                    0, true, vb);   // independent of the wait below
    const long long sl = (long long)u * a.slices + y;
    const bool ok = wait_flag(ctl.kdone + sl, ctl.spin_limit, &sm.flag);
    const float* w = ctl.wstash + sl * ctl.stash_rows * G;
    for (int i = threadIdx.x; i < r.nrows * G; i += 256) sm.x.lg[i] = ld_shared_dev(w + i);
    if (threadIdx.x < G) {
        sm.hs.M[threadIdx.x] = ld_shared_dev(ctl.sstash + (sl * G + threadIdx.x) * 2);
        sm.hs.L[threadIdx.x] = ld_shared_dev(ctl.sstash + (sl * G + threadIdx.x) * 2 + 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        st_shared_dev(ctl.kdone + sl, 0u);    // this item is the flag's only reader
        if (!ok) atomicOr(ctl.error, 1u);
    }
    if (!ok) {
        write_empty_partial(a.part, bh0, G, D, a.slot0 + y, NAN, NAN);
    } else {
        float acc[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
        rs.template accumulate<TCS_V_U>(seg, 1, r.nrows, sm.x.lg, vb, acc);
        __syncthreads();   // weights dead: fin may reuse the space
        rs.finish(acc, sm.hs.M, sm.hs.L, sm.x.fin, a.part, bh0, a.slot0 + y);
    }
    __syncthreads();
    if (arrive_last(fm.counter + u, fm.total, &sm.flag)) {
        merge_partials<D, G>(a.part, bh0, fm.out, fm.lse, sm.x.merge);
        st_shared_dev(fm.ready + u, 0u);
    }
}

// gist_kernel: grid (slices, units), one gist item per workgroup (two-level routing).
template <int D, int G>
__global__ void __launch_bounds__(256) gist_kernel(GistLaunch a) {
    __shared__ GistSmem<D, G> sm;
    gist_item<D, G>(a, blockIdx.y, blockIdx.x, sm);
}

// ---------------------------------------------------------------------------------------
// chunk_kernel: grid (ceil((kslots + 1) / cpw), units).  Workgroup x streams slots
// [x*cpw, (x+1)*cpw): slot j < kslots is selected chunk sel[u][j] (skipped if -1), slot
// kslots is the current chunk (tokens [(M-1)C, N)).  Each chunk's raw tokens carry its gate
// bias.  The last workgroup of a unit merges every partial of the unit's G heads.
// ---------------------------------------------------------------------------------------
constexpr int kMaxCpw = 16;

struct PageSegs {
    const uint16_t* kp;
    const uint16_t* vp;
    long long slab;           // elements per (page, kv head) slab: C * d
    int kv_off;               // kv * C * d
    int hkv;
    int C;
    const int* page;          // LDS: page of each chunk (< 0: no rows)
    const int* nrows;
    const float* gbias;
    __device__ long long off(int j) const {
        return ((long long)page[j] * hkv) * slab + kv_off;
    }
    __device__ const uint16_t* k(int j) const { return kp + (page[j] >= 0 ? off(j) : 0); }
    __device__ const uint16_t* v(int j) const { return vp + (page[j] >= 0 ? off(j) : 0); }
    __device__ int rows(int j) const { return page[j] >= 0 ? nrows[j] : 0; }
    __device__ int row0(int j) const { return j * C; }
    __device__ float bias(int j) const { return gbias[j]; }
};

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
    int rows[kMaxCpw];
    int flag;
};

// chunk item: workgroup wx of unit u streams chunk slots [wx*cpw, (wx+1)*cpw).  In the
// persistent kernel (`wait` non-null) it first waits for the unit's selection.
template <int D, int G>
__device__ __forceinline__ void chunk_item(const ChunkLaunch& a, int u, int wx, ChunkSmem<D, G>& sm,
                           const FinalMerge fm, const unsigned* wait, unsigned spin_limit,
                           unsigned* error) {
    using RS = RowStream<D, G>;
    const int b = u / a.Hkv, kv = u % a.Hkv;
    const int bh0 = b * a.Hq + kv * G;
    const int j0 = wx * a.cpw, nj = min(a.cpw, a.kslots + 1 - j0);
    bool stalled = false;
    if (wait && !wait_flag(wait + u, spin_limit, &sm.flag)) {
        stalled = true;
        if (threadIdx.x == 0) atomicOr(error, 1u);
    }
    // this workgroup's chunks: page, gate bias and row count (page -1: none, -2: unusable)
    if (threadIdx.x < nj) {
        const int j = j0 + threadIdx.x;
        int c, rows;
        float bias = 0.f;
        if (j < a.kslots) {
            c = ld_shared_dev(a.sel + (long long)u * a.k + j);
            if (c >= 0 && a.gamma) bias = ld_shared_dev(a.gamma + (long long)u * a.k + j);
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
        sm.page[threadIdx.x] = stalled ? -2 : page;
        sm.bias[threadIdx.x] = bias;
        sm.rows[threadIdx.x] = rows;
    }
    for (int i = threadIdx.x; i < nj * a.C * G; i += 256) sm.x.lg[i] = -INFINITY;
    __syncthreads();
    bool bad = false, any = false;
    for (int jj = 0; jj < nj; ++jj) {
        bad |= sm.page[jj] == -2;
        any |= sm.page[jj] >= 0;
    }
    const RS rs;
    const PageSegs seg{a.kp, a.vp, (long long)a.C * D, kv * a.C * D, a.Hkv, a.C,
                       sm.page, sm.rows, sm.bias};
    if (bad) {
        write_empty_partial(a.part, bh0, G, D, a.slot0 + wx, NAN, NAN);
    } else if (!any) {
        write_empty_partial(a.part, bh0, G, D, a.slot0 + wx, 0.f, 0.f);
    } else {
        {
            uint32_t q2[G][4];
            rs.load_q(a.q + (long long)bh0 * D, q2);
            rs.template logits<TCS_K_U>(q2, seg, nj, a.C, a.sigma, sm.x.lg);
        }
        uint4 vb[TCS_V_U];
        rs.template load_batch<TCS_V_U>(seg, (a.C + TCS_V_U * RS::RPP - 1) / (TCS_V_U * RS::RPP),
                                        0, true, vb);   // first V batch in flight from here on
        __syncthreads();
        head_stats<G>(sm.x.lg, nj * a.C, sm.hs);
        float acc[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
        rs.template accumulate<TCS_V_U>(seg, nj, a.C, sm.x.lg, vb, acc);
        __syncthreads();
        rs.finish(acc, sm.hs.M, sm.hs.L, sm.x.fin, a.part, bh0, a.slot0 + wx);
    }
    __syncthreads();
    if (!arrive_last(fm.counter + u, fm.total, &sm.flag)) return;
    merge_partials<D, G>(a.part, bh0, fm.out, fm.lse, sm.x.merge);
    if (fm.ready) st_shared_dev(fm.ready + u, 0u);
}

// chunk_kernel: grid (chunk workgroups per unit, units).
template <int D, int G>
__global__ void __launch_bounds__(256) chunk_kernel(ChunkLaunch a) {
    __shared__ ChunkSmem<D, G> sm;
    const FinalMerge fm{a.counter, gridDim.x, a.out, a.lse, nullptr};
    chunk_item<D, G>(a, blockIdx.y, blockIdx.x, sm, fm, nullptr, 0u, nullptr);
}

// ---------------------------------------------------------------------------------------
// fused_kernel: the whole one-level decode in one launch of one workgroup per work item.
// Units are dealt round-robin to nq queues, nq dividing the unit count, so every queue has
// the same list length: first the K item of every gist slice of its units (scoring and
// selection), then the V item of every slice (which waits for its own K item), then every
// chunk workgroup of its units (unit-major each) -- so the scoring of all units, on which
// the selections depend, is read first.  Workgroup w belongs to queue w % nq -- interleaved, so that
// workgroups starting early take the gist tickets of every queue -- and takes the next
// ticket of its queue when it starts running and does that item.  A V item waits (bounded) for
// its K item, a chunk item for its unit's selection, which the K items publish; K items never
// wait, and within a queue every K ticket is taken -- by a workgroup that is already running --
// before any other ticket, so each wait has a running producer whatever order the hardware
// starts workgroups in.  Spreading the tickets over nq counters keeps the ticket atomics from
// serialising on one address.  The unit's final merge runs in whichever of its items
// finishes last; the last item of a queue returns the queue's counters to zero.
// ---------------------------------------------------------------------------------------
template <int D, int G>
union FusedSmem {
    GistSmem<D, G> g;
    ChunkSmem<D, G> c;
};

template <int D, int G>
__global__ void __launch_bounds__(256) fused_kernel(GistLaunch g, ChunkLaunch c, FusedCtl ctl) {
    __shared__ FusedSmem<D, G> sm;
    __shared__ int s_item;
    const int units = g.B * g.Hkv;
    const int ncw = (c.kslots + 1 + c.cpw - 1) / c.cpw;
    const int nq = ctl.nq;                          // divides units
    const int q = blockIdx.x % nq;
    const int uq = units / nq;                      // units of each queue
    const int nk = uq * g.slices;                   // K items, then as many V items, then chunks
    const int nitems = 2 * nk + uq * ncw;
    if (threadIdx.x == 0) s_item = (int)atomicAdd(ctl.queue + q, 1u);
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(s_item);   // uniform: scalar branch
    const FinalMerge fm{ctl.done, (unsigned)(g.slices + ncw), c.out, c.lse, ctl.ready};
    if (t < nk) {
        gist_k_item<D, G>(g, ctl, q + (t / g.slices) * nq, t % g.slices, sm.g);
    } else if (t < 2 * nk) {
        const int v = t - nk;
        gist_v_item<D, G>(g, ctl, fm, q + (v / g.slices) * nq, v % g.slices, sm.g);
    } else if (t < nitems) {
        const int ci = t - 2 * nk;
        chunk_item<D, G>(c, q + (ci / ncw) * nq, ci % ncw, sm.c, fm, ctl.ready, ctl.spin_limit,
                         ctl.error);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = atomicAdd(ctl.queue + nq + q, 1u);
        if (old == (unsigned)nitems - 1u) {   // every ticket of this queue is taken and done
            atomicExch(ctl.queue + q, 0u);
            atomicExch(ctl.queue + nq + q, 0u);
        }
    }
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

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
template <int D>
static hipError_t gist_d(const GistLaunch& a, hipStream_t s, dim3 grid) {
    switch (a.Hq / a.Hkv) {
        case 1: gist_kernel<D, 1><<<grid, 256, 0, s>>>(a); break;
        case 2: gist_kernel<D, 2><<<grid, 256, 0, s>>>(a); break;
        case 4: gist_kernel<D, 4><<<grid, 256, 0, s>>>(a); break;
        case 8: gist_kernel<D, 8><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gist(const GistLaunch& a, hipStream_t s) {
    if (a.slices <= 0) return hipSuccess;
    dim3 grid(a.slices, a.B * a.Hkv);
    return a.d == 128 ? gist_d<128>(a, s, grid) : gist_d<64>(a, s, grid);
}

template <int D>
static hipError_t chunk_d(const ChunkLaunch& a, hipStream_t s, dim3 grid) {
    switch (a.Hq / a.Hkv) {
        case 1: chunk_kernel<D, 1><<<grid, 256, 0, s>>>(a); break;
        case 2: chunk_kernel<D, 2><<<grid, 256, 0, s>>>(a); break;
        case 4: chunk_kernel<D, 4><<<grid, 256, 0, s>>>(a); break;
        case 8: chunk_kernel<D, 8><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_chunks(const ChunkLaunch& a, hipStream_t s) {
    if (a.cpw < 1 || a.cpw > kMaxCpw || (long long)a.cpw * a.C > kMaxSliceRows)
        return hipErrorInvalidValue;
    dim3 grid((a.kslots + 1 + a.cpw - 1) / a.cpw, a.B * a.Hkv);
    return a.d == 128 ? chunk_d<128>(a, s, grid) : chunk_d<64>(a, s, grid);
}

template <int D>
static hipError_t fused_d(const FusedLaunch& a, hipStream_t s, int grid) {
    switch (a.g.Hq / a.g.Hkv) {
        case 1: fused_kernel<D, 1><<<grid, 256, 0, s>>>(a.g, a.c, a.ctl); break;
        case 2: fused_kernel<D, 2><<<grid, 256, 0, s>>>(a.g, a.c, a.ctl); break;
        case 4: fused_kernel<D, 4><<<grid, 256, 0, s>>>(a.g, a.c, a.ctl); break;
        case 8: fused_kernel<D, 8><<<grid, 256, 0, s>>>(a.g, a.c, a.ctl); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fused(const FusedLaunch& a, hipStream_t s) {
    const ChunkLaunch& c = a.c;
    if (c.cpw < 1 || c.cpw > kMaxCpw || (long long)c.cpw * c.C > kMaxSliceRows || a.g.slices < 1)
        return hipErrorInvalidValue;
    const long long units = (long long)a.g.B * a.g.Hkv;
    const long long items = 2 * units * a.g.slices + units * ((c.kslots + 1 + c.cpw - 1) / c.cpw);
    if (items > 0x7fffffffLL || a.ctl.nq < 1 || units % a.ctl.nq) return hipErrorInvalidValue;
    return a.g.d == 128 ? fused_d<128>(a, s, (int)items) : fused_d<64>(a, s, (int)items);
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
