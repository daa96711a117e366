// decode.hip -- gfx950 kernels of the chunk-sparse decode path.
//
//   gist_kernel    scores every historical chunk of a (b, kv) unit against the G query heads
//                  of its group through the chunk's gist keys ("Simplified Sparse Attention
//                  via Gist Tokens", section 3.2), pools them into one log-sum-exp score per
//                  chunk, and -- because gists are themselves tokens of the softmax set --
//                  folds the same gist rows into per-slice softmax partials with the gist
//                  values.
//   select_kernel  top-k chunk choice per unit (section 3.3), lowest index on ties, plus the
//                  SAS log-softmax gate over all historical scores ("SAS", abstract).
//   chunk_kernel   split-K attention over the selected chunks and the current chunk, read
//                  through the page table (section 3.6: only the selected keys are touched).
//   combine_kernel merges every partial of a query head in a fixed order.
//
// Layout of the work: one 256-thread workgroup streams a run of d-element bf16 rows (gist
// rows or one page's rows).  A row is read by d/8 lanes with one 16-byte load each, so a
// wave reads 4 (d=128) or 8 (d=64) whole rows per instruction, fully coalesced.  The row
// dot products are finished with DPP row reductions, softmax state is kept per lane group,
// and groups are merged once at the end (shuffles within a wave, LDS across waves).
#include "device.hpp"
#include "launch.hpp"

#include <math.h>

namespace tcs {

constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for empty softmax state

template <int D, int G>
struct RowAttn {
    static constexpr int LPR = D / 8;          // lanes per row (16 B each)
    static constexpr int RPW = kWave / LPR;    // rows per wave per pass
    static constexpr int NW = 4;               // waves per workgroup
    static constexpr int RPP = RPW * NW;       // rows per workgroup per pass

    float q[G][8];
    float m[G], l[G], acc[G][8];
    int lrow, part;

    __device__ void init(const uint16_t* qg /* [G][D] of this unit */) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        part = lane % LPR;
        lrow = w * RPW + lane / LPR;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            uint4 v = ld16(qg + h * D + part * 8);
            unpack8(v, q[h]);
            m[h] = kNegBig;
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
        }
    }

    // Stream rows [0, nrows) of K/V (row stride D).  logit = sigma * q.k + bias.
    // If lds_logits is given, the logit (without bias) of row r for head h goes to
    // lds_logits[r * G + h].
    template <int U>
    __device__ void run(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                        int nrows, float sigma, float bias, float* lds_logits) {
        for (int base = 0; base < nrows; base += U * RPP) {
            uint4 kr[U], vr[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = base + u * RPP + lrow;
                if (row < nrows) {
                    kr[u] = ld16(K + (long long)row * D + part * 8);
                    vr[u] = ld16(V + (long long)row * D + part * 8);
                } else {
                    kr[u] = make_uint4(0, 0, 0, 0);
                    vr[u] = make_uint4(0, 0, 0, 0);
                }
            }
            float x[U][G];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kf[8];
                unpack8(kr[u], kf);
                const int row = base + u * RPP + lrow;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float s = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) s = fmaf(q[h][e], kf[e], s);
                    s = group_sum<LPR>(s) * sigma;
                    if (lds_logits && part == 0 && row < nrows) lds_logits[row * G + h] = s;
                    x[u][h] = row < nrows ? s + bias : -INFINITY;
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float mx = m[h];
#pragma unroll
                for (int u = 0; u < U; ++u) mx = fmaxf(mx, x[u][h]);
                const float sc = __expf(m[h] - mx);
                l[h] *= sc;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= sc;
                m[h] = mx;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vf[8];
                unpack8(vr[u], vf);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float w = __expf(x[u][h] - m[h]);
                    l[h] += w;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(w, vf[e], acc[h][e]);
                }
            }
        }
    }

    // Merge the lane groups of the workgroup and write one partial per head:
    // pacc[(bh0 + h) * nslots + slot][0..D), pml[... ][0..2).
    // lds must hold NW * G * (D + 2) floats.
    __device__ void finish(float* lds, const Partials& P, int bh0, int slot) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        // within the wave: lanes part + r * LPR, r = 0 .. RPW-1
#pragma unroll
        for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float mo = __shfl_xor(m[h], off);
                const float lo = __shfl_xor(l[h], off);
                const float mx = fmaxf(m[h], mo);
                const float a = __expf(m[h] - mx), b = __expf(mo - mx);
                l[h] = l[h] * a + lo * b;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float ao = __shfl_xor(acc[h][e], off);
                    acc[h][e] = acc[h][e] * a + ao * b;
                }
                m[h] = mx;
            }
        }
        float* lacc = lds;                    // [NW][G][D]
        float* lml = lds + NW * G * D;        // [NW][G][2]
        if (lane < LPR) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) lacc[(w * G + h) * D + part * 8 + e] = acc[h][e];
        }
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                lml[(w * G + h) * 2] = m[h];
                lml[(w * G + h) * 2 + 1] = l[h];
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < G * D; idx += 256) {
            const int h = idx / D, col = idx % D;
            float mx = kNegBig;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, lml[(ww * G + h) * 2]);
            float a = 0.f, s = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const float f = __expf(lml[(ww * G + h) * 2] - mx);
                a += f * lacc[(ww * G + h) * D + col];
                s += f * lml[(ww * G + h) * 2 + 1];
            }
            const long long o = (long long)(bh0 + h) * P.nslots + slot;
            st_shared_dev(P.acc + o * D + col, a);
            if (col == 0) {
                st_shared_dev(P.ml + o * 2, mx);
                st_shared_dev(P.ml + o * 2 + 1, s);
            }
        }
    }
};

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

constexpr int kMaxSliceRows = 1024;

// ---------------------------------------------------------------------------------------
// Selection epilogue shared by the scoring passes.  Each workgroup keeps the best
// min(k, items in its slice) of its slice's items (ascending), stores them with their
// scores, and the last workgroup of the unit to finish merges the slices' lists (which are
// in ascending item order, slice after slice) into the unit's top-k.  Ties go to the lower
// item index at both steps, so the result equals a top-k over all items at once.
// ---------------------------------------------------------------------------------------
__device__ void select_epilogue(const SelectOut& so, int u, int slot, int nslices,
                                const float* s_score, int item0, int nitems, int last_items,
                                float* lse_part_lds, void* scratch, int* s_flag, int* s_chosen,
                                ReduceSmem& red) {
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
    if (!arrive_last(so.counter + u, (unsigned)nslices, s_flag)) return;

    // ---- last workgroup of the unit: merge ------------------------------------------------
    const float* ucs = so.cand_score + (long long)u * nslices * so.kcap;
    const int32_t* uci = so.cand_idx + (long long)u * nslices * so.kcap;
    const int ncand = (nslices - 1) * so.kcap + (so.k < last_items ? so.k : last_items);
    float lse = 0.f;
    if (so.slice_lse && so.gamma) {
        // every slice's (max, sum exp) loaded at once, then merged in slice order
        const float* sl = so.slice_lse + (long long)u * nslices * 2;
        float* st = reinterpret_cast<float*>(scratch);     // 2 * nslices floats if they fit
        const bool staged = 2 * nslices <= kTopkCache;
        if (staged)
            for (int i = tid; i < 2 * nslices; i += 256) st[i] = ld_shared_dev(sl + i);
        __syncthreads();
        auto at = [&](int i) { return staged ? st[i] : ld_shared_dev(sl + i); };
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
    int32_t* sel = so.sel + (long long)u * so.k;
    float* gam = so.gamma ? so.gamma + (long long)u * so.k : nullptr;
    auto emit2 = [&](int j, int i) {
        const int32_t c = ld_shared_dev(uci + i);
        sel[j] = c;
        if (gam) gam[j] = ld_shared_dev(ucs + i) - lse;
        if (j < 64) s_chosen[j] = c;
    };
    auto sc2 = [&](int i) { return ld_shared_dev(ucs + i); };
    int ke;
    if (so.k >= ncand) {
        for (int i = tid; i < ncand; i += 256) emit2(i, i);
        ke = ncand;
    } else if (ncand <= 256) {
        ke = small_topk(ncand, so.k, sc2, emit2, *reinterpret_cast<SmallTopkSmem*>(scratch));
    } else {
        ke = block_topk(ncand, so.k, sc2, emit2, *reinterpret_cast<TopkSmem*>(scratch));
    }
    for (int j = ke + tid; j < so.k; j += 256) {
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

// ---------------------------------------------------------------------------------------
// gist_kernel: grid (slices, units).  Range mode: slice y covers items (chunks, or level-2
// groups) [y*ips, min((y+1)*ips, nitems)).  Group mode (a.groups != null): slice y covers the
// member chunks of level-2 group groups[u][y].  Streams the slice's gist rows once: logits
// for the G heads, pooled item scores, the gist softmax partial, then the selection epilogue.
// ---------------------------------------------------------------------------------------
template <int D, int G>
struct GistSmem {
    union {
        float logits[kMaxSliceRows * G];
        float fin[RowAttn<D, G>::NW * G * (D + 2)];
        TopkSmem topk;
        SmallTopkSmem small;
    } x;
    float score[kMaxSliceRows];
    ReduceSmem red;
    float lse;
    int flag;
    int chosen[64];
};

template <int D, int G>
__global__ void __launch_bounds__(256) gist_kernel(GistLaunch a) {
    using RA = RowAttn<D, G>;
    __shared__ GistSmem<D, G> sm;
    const int y = blockIdx.x, u = blockIdx.y;
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
    RA ra;
    ra.init(a.q + (long long)bh0 * D);
    const uint16_t* K = a.gk + (long long)u * a.unit_stride + (long long)c0 * a.g * D;
    const uint16_t* V = a.gv + (long long)u * a.unit_stride + (long long)c0 * a.g * D;
    ra.template run<4>(K, V, nrows, a.sigma, 0.f, sm.x.logits);
    __syncthreads();
    // pooled item scores: log-sum-exp over the G heads and g gists of each item
    for (int c = threadIdx.x; c < nit; c += 256) {
        const float* x = sm.x.logits + c * a.g * G;
        float mx = -INFINITY;
        for (int i = 0; i < a.g * G; ++i) mx = fmaxf(mx, x[i]);
        float z = 0.f;
        for (int i = 0; i < a.g * G; ++i) z += expf(x[i] - mx);
        const float s = mx + logf(z);
        sm.score[c] = s;
        if (a.scores_out) a.scores_out[(long long)u * a.score_stride + c0 + c] = s;
    }
    __syncthreads();
    ra.finish(sm.x.fin, a.part, bh0, a.slot0 + y);
    __syncthreads();
    select_epilogue(a.selo, u, y, a.slices, sm.score, c0, nit, last_items, &sm.lse, &sm.x,
                    &sm.flag, sm.chosen, sm.red);
}

// ---------------------------------------------------------------------------------------
// chunk_kernel: grid (kslots + 1, units).  Slot j < kslots: selected chunk sel[u][j] (an
// empty partial for -1); slot kslots: the current chunk (tokens [(M-1)C, N)).  The last
// workgroup of a unit merges every partial of the unit's G heads in slot order.
// ---------------------------------------------------------------------------------------
constexpr int kMergeStage = 1024;   // (head, slot) softmax statistics staged in LDS

template <int G>
struct MergeSmem {
    float w[kMergeStage];    // m, then exp(m - M)
    float l[kMergeStage];
    float M[G], L[G];
};

// Fixed-order merge of every slot's partial for the G heads of one unit -> out, lse.
// All hand-off loads of a batch are issued before any is used, so the merge costs a few
// memory round trips rather than one per slot.
template <int D, int G>
__device__ void merge_partials(const Partials& P, int bh0, float* out, float* lse,
                               MergeSmem<G>& sm) {
    const int ns = P.nslots;
    const int tid = threadIdx.x;
    const bool staged = G * ns <= kMergeStage;
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
    constexpr int PPT = (G * D + 255) / 256;   // (head, column) outputs per thread
    constexpr int SB = PPT <= 2 ? 16 : 8;      // slots per batch of loads
    float o[PPT];
#pragma unroll
    for (int q = 0; q < PPT; ++q) o[q] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += SB) {
        float v[PPT][SB];
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

// ---------------------------------------------------------------------------------------
// chunk_kernel: grid (ceil((kslots + 1) / cpw), units).  Workgroup x streams slots
// [x*cpw, (x+1)*cpw): slot j < kslots is selected chunk sel[u][j] (skipped if -1), slot
// kslots is the current chunk (tokens [(M-1)C, N)).  Each chunk's raw tokens carry its gate
// bias.  The last workgroup of a unit merges every partial of the unit's G heads.
// ---------------------------------------------------------------------------------------
template <int D, int G>
struct ChunkSmem {
    union {
        float fin[RowAttn<D, G>::NW * G * (D + 2)];
        MergeSmem<G> merge;
    } x;
    int flag;
};

template <int D, int G>
__global__ void __launch_bounds__(256) chunk_kernel(ChunkLaunch a) {
    using RA = RowAttn<D, G>;
    __shared__ ChunkSmem<D, G> sm;
    const int wx = blockIdx.x, u = blockIdx.y;
    const int b = u / a.Hkv, kv = u % a.Hkv;
    const int bh0 = b * a.Hq + kv * G;
    RA ra;
    ra.init(a.q + (long long)bh0 * D);
    bool bad_page = false;
    const int j0 = wx * a.cpw, j1 = min(j0 + a.cpw, a.kslots + 1);
    for (int j = j0; j < j1; ++j) {
        int c, nrows;
        float bias = 0.f;
        if (j < a.kslots) {
            c = a.sel[(long long)u * a.k + j];
            if (c >= 0 && a.gamma) bias = a.gamma[(long long)u * a.k + j];
            nrows = a.C;
        } else {
            c = a.M - 1;
            nrows = a.N - (a.M - 1) * a.C;
        }
        if (c < 0) continue;
        const int page = a.page_table[(long long)b * a.max_chunks + c];
        if (page < 0 || page >= a.num_pages) {
            bad_page = true;
            continue;
        }
        const long long off = ((long long)page * a.Hkv + kv) * a.C * D;
        ra.template run<4>(a.kp + off, a.vp + off, nrows, a.sigma, bias, nullptr);
    }
    if (bad_page)
        write_empty_partial(a.part, bh0, G, D, a.slot0 + wx, NAN, NAN);
    else
        ra.finish(sm.x.fin, a.part, bh0, a.slot0 + wx);
    if (!arrive_last(a.counter + u, (unsigned)gridDim.x, &sm.flag)) return;
    merge_partials<D, G>(a.part, bh0, a.out, a.lse, sm.x.merge);
}

// ---------------------------------------------------------------------------------------
// zero_kernel: clears a workspace region (used once per workspace, before its first call).
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
    if (a.cpw < 1) return hipErrorInvalidValue;
    dim3 grid((a.kslots + 1 + a.cpw - 1) / a.cpw, a.B * a.Hkv);
    return a.d == 128 ? chunk_d<128>(a, s, grid) : chunk_d<64>(a, s, grid);
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
