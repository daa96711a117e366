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
            P.acc[o * D + col] = a;
            if (col == 0) {
                P.ml[o * 2] = mx;
                P.ml[o * 2 + 1] = s;
            }
        }
    }
};

__device__ __forceinline__ void write_empty_partial(const Partials& P, int bh0, int G, int D,
                                                    int slot, float fill_l, float fill_acc) {
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D, col = idx % D;
        const long long o = (long long)(bh0 + h) * P.nslots + slot;
        P.acc[o * D + col] = fill_acc;
        if (col == 0) {
            P.ml[o * 2] = fill_l == fill_l ? kNegBig : 0.f;   // NaN fill: m = 0, l = NaN
            P.ml[o * 2 + 1] = fill_l;
        }
    }
}

constexpr int kMaxSliceRows = 1024;

// ---------------------------------------------------------------------------------------
// gist_kernel: grid (slices, units).  Range mode: slice y covers chunks
// [y*cps, min((y+1)*cps, nchunks)).  Group mode (a.groups != null): slice y covers the members
// of level-2 group r = groups[u][y] (chunks [r*J, min((r+1)*J, H))); scores are written at the
// compact candidate position y*J + offset.
// ---------------------------------------------------------------------------------------
template <int D, int G>
__global__ void __launch_bounds__(256) gist_kernel(GistLaunch a) {
    using RA = RowAttn<D, G>;
    __shared__ float s_logits[kMaxSliceRows * G];
    __shared__ float s_fin[RA::NW * G * (D + 2)];
    const int y = blockIdx.x, u = blockIdx.y;
    const int b = u / a.Hkv, kv = u % a.Hkv;
    const int bh0 = b * a.Hq + kv * G;
    int c0, c1, spos;
    if (a.groups) {
        const int r = a.groups[(long long)u * a.k2 + y];
        if (r < 0) {
            write_empty_partial(a.part, bh0, G, D, a.slot0 + y, 0.f, 0.f);
            return;
        }
        c0 = r * a.J;
        c1 = min(c0 + a.J, a.H);
        spos = y * a.J;
    } else {
        c0 = y * a.chunks_per_slice;
        c1 = min(c0 + a.chunks_per_slice, a.nchunks);
        spos = c0;
    }
    const int nch = max(c1 - c0, 0);
    const int nrows = nch * a.g;
    RA ra;
    ra.init(a.q + (long long)bh0 * D);
    const uint16_t* K = a.gk + (long long)u * a.unit_stride + (long long)c0 * a.g * D;
    const uint16_t* V = a.gv + (long long)u * a.unit_stride + (long long)c0 * a.g * D;
    ra.template run<4>(K, V, nrows, a.sigma, 0.f, s_logits);
    __syncthreads();
    // pooled chunk scores: log-sum-exp over the G heads and g gists of each chunk
    for (int c = threadIdx.x; c < nch; c += 256) {
        const float* x = s_logits + (long long)c * a.g * G;
        float mx = -INFINITY;
        for (int i = 0; i < a.g * G; ++i) mx = fmaxf(mx, x[i]);
        float z = 0.f;
        for (int i = 0; i < a.g * G; ++i) z += expf(x[i] - mx);
        a.scores[(long long)u * a.score_stride + spos + c] = mx + logf(z);
    }
    ra.finish(s_fin, a.part, bh0, a.slot0 + y);
}

// ---------------------------------------------------------------------------------------
// select_kernel: grid (units).  Top-k over a unit's scores and the SAS gate.
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) select_kernel(SelectLaunch a) {
    __shared__ TopkSmem sm;
    __shared__ ReduceSmem red;
    __shared__ int s_groups[64];
    __shared__ int s_ncand;
    const int u = blockIdx.x;
    const float* s = a.scores + (long long)u * a.score_stride;
    int n = a.n;
    if (a.groups) {
        // candidates: members of the chosen groups, in ascending group order
        if (threadIdx.x == 0) {
            int cnt = 0, ng = 0;
            for (int y = 0; y < a.k2; ++y) {
                const int r = a.groups[(long long)u * a.k2 + y];
                if (y < 64) s_groups[y] = r;
                if (r >= 0) { ng = y + 1; cnt = y * a.J + min(a.J, a.H - r * a.J); }
            }
            (void)ng;
            s_ncand = cnt;
        }
        __syncthreads();
        n = s_ncand;
        if (a.chunk_scores_out) {
            float* cs = a.chunk_scores_out + (long long)u * a.H;
            for (int c = threadIdx.x; c < a.H; c += 256) cs[c] = -INFINITY;
            __syncthreads();
            for (int p = threadIdx.x; p < n; p += 256) {
                const int r = s_groups[p / a.J];
                cs[r * a.J + p % a.J] = s[p];
            }
        }
    }
    int32_t* sel = a.sel + (long long)u * a.k;
    float* gam = a.gamma ? a.gamma + (long long)u * a.k : nullptr;
    float lse = 0.f;
    if (gam && n > 0) {
        float mx = -INFINITY;
        for (int i = threadIdx.x; i < n; i += 256) mx = fmaxf(mx, s[i]);
        mx = block_max(mx, red);
        float z = 0.f;
        for (int i = threadIdx.x; i < n; i += 256) z += expf(s[i] - mx);
        z = block_sum(z, red);
        lse = mx + logf(z);
    }
    const int J = a.J;
    const bool gm = a.groups != nullptr;
    const int ke = block_topk(
        n, a.k, [&](int i) { return s[i]; },
        [&](int j, int i) {
            const int c = gm ? s_groups[i / J] * J + i % J : i;
            sel[j] = c;
            if (gam) gam[j] = s[i] - lse;
        },
        sm);
    for (int j = max(ke, 0) + threadIdx.x; j < a.k; j += 256) {
        sel[j] = -1;
        if (gam) gam[j] = 0.f;
    }
}

// ---------------------------------------------------------------------------------------
// chunk_kernel: grid (kslots + 1, units).  Slot j < kslots: selected chunk sel[u][j] (an
// empty partial for -1); slot kslots: the current chunk (tokens [(M-1)C, N)).
// ---------------------------------------------------------------------------------------
template <int D, int G>
__global__ void __launch_bounds__(256) chunk_kernel(ChunkLaunch a) {
    using RA = RowAttn<D, G>;
    __shared__ float s_fin[RA::NW * G * (D + 2)];
    const int j = blockIdx.x, u = blockIdx.y;
    const int b = u / a.Hkv, kv = u % a.Hkv;
    const int bh0 = b * a.Hq + kv * G;
    int c, nrows;
    float bias = 0.f;
    if (j < a.kslots) {
        c = a.sel[(long long)u * a.k + j];
        if (c < 0) {
            write_empty_partial(a.part, bh0, G, D, a.slot0 + j, 0.f, 0.f);
            return;
        }
        if (a.gamma) bias = a.gamma[(long long)u * a.k + j];
        nrows = a.C;
    } else {
        c = a.M - 1;
        nrows = a.N - (a.M - 1) * a.C;
    }
    const int page = a.page_table[(long long)b * a.max_chunks + c];
    if (page < 0 || page >= a.num_pages) {
        write_empty_partial(a.part, bh0, G, D, a.slot0 + j, NAN, NAN);
        return;
    }
    const long long off = ((long long)page * a.Hkv + kv) * a.C * D;
    RA ra;
    ra.init(a.q + (long long)bh0 * D);
    ra.template run<4>(a.kp + off, a.vp + off, nrows, a.sigma, bias, nullptr);
    ra.finish(s_fin, a.part, bh0, a.slot0 + j);
}

// ---------------------------------------------------------------------------------------
// combine_kernel: grid (B*Hq), block D.  Fixed-order merge of all slots.
// ---------------------------------------------------------------------------------------
__global__ void combine_kernel(CombineLaunch a) {
    const int bh = blockIdx.x, col = threadIdx.x;
    const int ns = a.part.nslots, D = a.d;
    const float* ml = a.part.ml + (long long)bh * ns * 2;
    const float* acc = a.part.acc + (long long)bh * ns * D;
    float mx = kNegBig;
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, ml[2 * s]);
    float L = 0.f, o = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float f = __expf(ml[2 * s] - mx);
        L += f * ml[2 * s + 1];
        o += f * acc[(long long)s * D + col];
    }
    a.out[(long long)bh * D + col] = o / L;
    if (a.lse && col == 0) a.lse[bh] = mx + logf(L);
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
    dim3 grid(a.slices, a.B * a.Hkv);
    if (a.slices <= 0) return hipSuccess;
    return a.d == 128 ? gist_d<128>(a, s, grid) : gist_d<64>(a, s, grid);
}

hipError_t launch_select(const SelectLaunch& a, hipStream_t s) {
    if (a.k <= 0 || a.units <= 0) return hipSuccess;
    select_kernel<<<a.units, 256, 0, s>>>(a);
    return hipGetLastError();
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
    dim3 grid(a.kslots + 1, a.B * a.Hkv);
    return a.d == 128 ? chunk_d<128>(a, s, grid) : chunk_d<64>(a, s, grid);
}

hipError_t launch_combine(const CombineLaunch& a, hipStream_t s) {
    combine_kernel<<<a.BH, a.d, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace tcs
