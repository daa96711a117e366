// gist_prefill.hip -- gfx950 kernels of the SSA gist-masked prefill ("Simplified Sparse
// Attention via Gist Tokens", sections 3.1 and 3.6).
#include "device.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"

#include <math.h>

namespace tcs {

// =============================================================================================
// SSA gist-masked prefill ("Simplified Sparse Attention via Gist Tokens", section 3.1: chunk
// tokens see their own chunk and the preceding gist tokens; later tokens reach a chunk only
// through its gists).  Section 3.6's key-column permutation puts the summary columns first:
// gist_gather_kernel copies every chunk's g gist K/V rows into one contiguous array, after
// which the keys a raw query block sees are two dense runs -- the gist prefix [0, c g) and the
// causal part of its own chunk -- and every other key block is skipped.  The block list is a
// closed form of (chunk, block), so no mask is stored.
//   gist_prefill_mfma_kernel<false>  raw query rows: the forward's MFMA machinery over the
//                             diagonal block (token-causal), the chunk's earlier raw blocks and
//                             the gist prefix blocks (the last one cut at column c g).
//   gist_prefill_mfma_kernel<true>   gist query rows, in gathered order: gist t of chunk c is
//                             gathered row c g + t and sees the gathered gists up to itself --
//                             causal attention over the gathered gists -- plus its own chunk's
//                             L raw rows, one block list per 32-row tile: gist blocks up to the
//                             tile's diagonal, then the raw blocks of the chunks the tile spans,
//                             each visible only to its chunk's rows.
// =============================================================================================

__global__ void __launch_bounds__(256) gist_gather_kernel(GistPrefillLaunch a) {
    const int nrb = a.Gp / kPBlk;
    const int unit = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    const int W = a.L + a.g;
    const size_t Tp = (size_t)a.M * W;
    const uint16_t* ks = a.k + (size_t)unit * Tp * kPD;
    const uint16_t* vs = a.v + (size_t)unit * Tp * kPD;
    uint16_t* kd = a.gk + ((size_t)unit * a.Gp + (size_t)rb * kPBlk) * kPD;
    uint16_t* vd = a.gv + ((size_t)unit * a.Gp + (size_t)rb * kPBlk) * kPD;
#pragma unroll
    for (int x = 0; x < 4; ++x) {   // 64 rows x 256 B = 1024 16-byte pieces per array
        const int piece = x * 256 + threadIdx.x;
        const int r = piece >> 4, col = (piece & 15) * 8;
        const int gi = rb * kPBlk + r;   // gist index: chunk gi / g, gist gi % g
        uint4 kx = make_uint4(0u, 0u, 0u, 0u), vx = kx;
        if (gi < a.M * a.g) {
            const size_t src = ((size_t)(gi / a.g) * W + a.L + gi % a.g) * kPD + col;
            kx = *reinterpret_cast<const uint4*>(ks + src);
            vx = *reinterpret_cast<const uint4*>(vs + src);
        }
        *reinterpret_cast<uint4*>(kd + (size_t)r * kPD + col) = kx;
        *reinterpret_cast<uint4*>(vd + (size_t)r * kPD + col) = vx;
    }
}

// Workgroup bid0 of a grid of Wg workgroups of one row kind.  tile_a and tile_b are the
// kernel's two block buffers (distinct LDS objects, K then V of one block each): blocks are
// copied global -> LDS directly, and the loop is unrolled by two so that every copy and operand
// read names its buffer, as in the SAS forward.
template <bool GROWS>
__device__ __forceinline__ void gist_prefill_rows(const GistPrefillLaunch& a, int bid0, int Wg,
                                                  char* tile_a, char* tile_b) {
    const int G = a.Hq / a.Hkv;
    const int nhg = (G + 3) >> 2;
    const int nrb = a.L / kPBlk;                 // raw blocks per chunk
    // query blocks per (unit, head group): raw blocks of every chunk, or 64-row blocks of the
    // gathered gists
    const int nq = GROWS ? a.Gp / kPBlk : a.M * nrb;
    const int W = a.L + a.g;
    const size_t Tp = (size_t)a.M * W;
    // XCD-contiguous ranges as in the forward; within a range the last chunks (longest gist
    // prefix) first, the two row halves of a block side by side
    int bid = bid0;
    if ((Wg & 7) == 0) bid = (bid & 7) * (Wg >> 3) + (bid >> 3);
    const int rh = bid & 1;
    const int qb = nq - 1 - (bid >> 1) % nq;
    const int rest = (bid >> 1) / nq;
    const int hg = rest % nhg;
    const int unit = rest / nhg;
    const int b = unit / a.Hkv, kv = unit % a.Hkv;
    const int ngtot = a.M * a.g;                 // gathered gist rows
    // raw rows: chunk c, block rb.  Gist rows: gathered rows R0 .. R0 + 31 of chunks
    // c_lo .. c_hi.
    const int c = GROWS ? 0 : qb / nrb, rb = GROWS ? 0 : qb % nrb;
    const int R0 = GROWS ? qb * kPBlk + 32 * rh : 0;
    if (GROWS && R0 >= ngtot) return;            // padding rows only (uniform per workgroup)
    const int c_lo = GROWS ? R0 / a.g : 0;
    const int c_hi = GROWS ? min(R0 + 31, ngtot - 1) / a.g : 0;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int head = hg * 4 + w;
    const bool active = head < G;

    const uint16_t* kraw = a.k + ((size_t)unit * Tp + (size_t)c * W) * kPD;   // chunk c's rows
    const uint16_t* vraw = a.v + ((size_t)unit * Tp + (size_t)c * W) * kPD;
    const uint16_t* kgst = a.gk + (size_t)unit * a.Gp * kPD;
    const uint16_t* vgst = a.gv + (size_t)unit * a.Gp * kPD;
    const int ngist = c * a.g;                         // raw rows: visible gist columns
    const int nbg = (ngist + kPBlk - 1) / kPBlk;       // raw rows: gist prefix blocks
    const int last_valid = ngist - (nbg - 1) * kPBlk;  // columns of the last gist block
    // Raw rows, block t: 0 = the diagonal (raw block rb, token-causal), 1..rb = raw blocks
    // 0..rb-1, rb+1.. = gist prefix blocks.  Gist rows, block t: 0..qb = gathered gist blocks
    // (qb is the diagonal, causal in gathered order), then raw block u = t - qb - 1 of chunk
    // c_lo + u / nrb.
    const int nblk = GROWS ? qb + 1 + (c_hi - c_lo + 1) * nrb : 1 + rb + nbg;
    auto blk_row = [&](int t) -> size_t {   // first row of block t in its array
        if (GROWS) {
            if (t <= qb) return (size_t)t * kPBlk;
            const int u = t - qb - 1;
            return (size_t)(c_lo + u / nrb) * W + (size_t)(u % nrb) * kPBlk;
        }
        return t == 0 ? (size_t)rb * kPBlk : t <= rb ? (size_t)(t - 1) * kPBlk
                                                     : (size_t)(t - 1 - rb) * kPBlk;
    };
    auto in_gathered = [&](int t) { return GROWS ? t <= qb : t > rb; };
    const uint16_t* kall = a.k + (size_t)unit * Tp * kPD;   // the interleaved rows of the unit
    const uint16_t* vall = a.v + (size_t)unit * Tp * kPD;
    auto kblock = [&](int t) -> const uint16_t* {
        return (in_gathered(t) ? kgst : GROWS ? kall : kraw) + blk_row(t) * kPD;
    };
    auto vblock = [&](int t) -> const uint16_t* {
        return (in_gathered(t) ? vgst : GROWS ? vall : vraw) + blk_row(t) * kPD;
    };

    const CopyOffsets gk = copy_offsets(kSwzK, w, lane), gv = copy_offsets(kSwzV, w, lane);
    auto dma = [&](int t, char* buf) {   // block t: K tile at buf, V tile at buf + kPTile
        const char* kc = reinterpret_cast<const char*>(kblock(t));
        const char* vc = reinterpret_cast<const char*>(vblock(t));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            __builtin_amdgcn_global_load_lds(kc + gk.c[c], (lds_void*)(buf + (4 * c + w) * 1024),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(vc + gv.c[c],
                                             (lds_void*)(buf + kPTile + (4 * c + w) * 1024), 16,
                                             0, 0);
        }
    };
    dma(0, tile_a);

    // this lane's query row: raw row 64 rb + 32 rh + c32 of chunk c, or gathered gist row
    // r = R0 + c32 (clamped for loading when r is padding; nothing is written for it)
    const int r = R0 + c32;
    const bool row_ok = !GROWS || r < ngtot;
    const int rq = GROWS ? min(r, ngtot - 1) : 0;
    const int rchunk = GROWS ? rq / a.g : c;
    const size_t qpos = GROWS ? (size_t)rchunk * W + a.L + rq % a.g
                              : (size_t)c * W + (size_t)rb * kPBlk + 32 * rh + c32;
    const size_t qrow = (size_t)(b * a.Hq + kv * G + (active ? head : 0)) * Tp + qpos;
    bf16x8 qf[8];
    if constexpr (!GROWS) {   // raw rows: the wave's 32 rows are consecutive positions
        load_q_operand(a.q + (qrow - c32) * kPD, tile_b + w * kQRowsLds, lane, qf);
    } else {
        const uint16_t* qp = a.q + qrow * kPD + 8 * h;
#pragma unroll
        for (int kd = 0; kd < 8; ++kd) qf[kd] = *reinterpret_cast<const bf16x8*>(qp + 16 * kd);
    }

    const int koff0 = c32 * 64 + (((0 + h) ^ swz_k(c32)) << 4);
    const int koff1 = c32 * 64 + (((2 + h) ^ swz_k(c32)) << 4);
    const int g16 = lane >> 4, L16 = lane & 15, rr = L16 >> 2, cc = L16 & 3;
    const int voff = (4 * h + rr) * 64 + (((2 * (g16 & 1) + (cc >> 1)) ^ swz_v(rr)) << 4) +
                     ((cc & 1) << 3);

    const float cs = a.sigma * kLog2e;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m = 0.f, l = 0.f;
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

    // block t is in cur; the copy of block t + 1 goes into nxt once every wave is past block
    // t - 1 (which was in nxt); first: t == 0
    auto block = [&](int t, bool first, const char* cur, char* nxt) {
        wait_vmem_lds();   // this wave's part of block t has landed
        __syncthreads();   // and every wave's; every wave is done with nxt
        if (t + 1 < nblk) dma(t + 1, nxt);
        if (active) {
            const bool half = !GROWS && first && rh == 0;
            const int cut = (!GROWS && t == nblk - 1 && t > rb) ? last_valid : kPBlk;
            const char* kt = cur;
            const char* vt = cur + kPTile + voff;
            f32x16 s[2];
            s[0] = s[1] = f32x16{};
            if (half) qk_product<1>(kt, koff0, koff1, qf, s);
            else qk_product<2>(kt, koff0, koff1, qf, s);
            bf16x8 va[4][4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if (half && st >= 2) break;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) va[st][dt] = v_operand(vt, dt, st);
            }
            if constexpr (GROWS) {
                // gathered gist blocks: causal in gathered order on the diagonal block; a raw
                // block: visible only to the rows of its chunk
                const bool own = t <= qb || c_lo + (t - qb - 1) / nrb == rchunk;
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = 32 * x + 8 * (e >> 2) + 4 * h + (e & 3);
                        if (!own || (t == qb && t * kPBlk + key > rq)) s[x][e] = -INFINITY;
                    }
            } else {
                const int q = 32 * rh + c32;
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = 32 * x + 8 * (e >> 2) + 4 * h + (e & 3);
                        if ((first && key > q) || key >= cut) s[x][e] = -INFINITY;
                    }
            }
            float mx = s[0][0];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[x][e]);
            mx = pair_max(mx);
            // a raw block of another chunk leaves a gist row without keys: no update
            const float mb = mx == -INFINITY ? m : mx * cs;
            if (first) {
                m = mb;
            } else if (__builtin_amdgcn_ballot_w64(mb > m + kRescaleSlack)) {
                const float mn = fmaxf(m, mb);
                const float al = __builtin_amdgcn_exp2f(m - mn);
                m = mn;
                l *= al;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] *= al;
            }
            const float off = -m;
            float sum = 0.f;
            auto p_step = [&](int st) {
                bf16x8 pv;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pv[e] = (__bf16)__builtin_amdgcn_exp2f(s[st >> 1][8 * (st & 1) + e] * cs + off);
                sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 0, 1), ones, sum, false);
                sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 2, 3), ones, sum, false);
                sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 4, 5), ones, sum, false);
                sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 6, 7), ones, sum, false);
                return pv;
            };
            auto pv_mfma = [&](int st, const bf16x8& pst) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[st][dt], pst, o[dt], 0, 0, 0);
            };
            if (half) {
                const bf16x8 p0 = p_step(0);
                const bf16x8 p1 = p_step(1);
                pv_mfma(0, p0);
                pv_mfma(1, p1);
            } else {
                const bf16x8 p0 = p_step(0);
                const bf16x8 p1 = p_step(1);
                pv_mfma(0, p0);
                const bf16x8 p2 = p_step(2);
                pv_mfma(1, p1);
                const bf16x8 p3 = p_step(3);
                pv_mfma(2, p2);
                pv_mfma(3, p3);
            }
            l += sum;
        }
    };
    block(0, true, tile_a, tile_b);
    for (int t = 1; t < nblk; t += 2) {
        block(t, false, tile_b, tile_a);
        if (t + 1 < nblk) block(t + 1, false, tile_a, tile_b);
    }
    if constexpr (!GROWS) {
        // raw rows: a wave's 32 rows are consecutive positions, stored as whole rows
        __syncthreads();   // every wave is done with the last block's tiles
        if (!active) return;
        const float lt = pair_sum(l);
        store_rows_f32(o, 1.f / lt, (w < 2 ? tile_a : tile_b) + (w & 1) * kORowsLds,
                       a.out + (qrow - c32) * kPD, lane);
        if (a.lse && h == 0) a.lse[qrow] = (m + log2f(lt)) * kLn2;
        return;
    }
    if (!active || !row_ok) return;
    const float lt = pair_sum(l);
    const float inv = 1.f / lt;
    float* op = a.out + qrow * kPD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            float4 v;
            v.x = o[dt][4 * e4 + 0] * inv;
            v.y = o[dt][4 * e4 + 1] * inv;
            v.z = o[dt][4 * e4 + 2] * inv;
            v.w = o[dt][4 * e4 + 3] * inv;
            *reinterpret_cast<float4*>(op + 32 * dt + 8 * e4 + 4 * h) = v;
        }
    if (a.lse && h == 0) a.lse[qrow] = (m + log2f(lt)) * kLn2;
}

// One launch for both row kinds: the gist rows' workgroups first (few, with long block lists:
// on their own they fill half the CUs), then the raw rows' workgroups, which take every CU
// slot the gist rows leave.  The gist-row share is a multiple of 8, so both shares keep the
// XCD-contiguous ranges.
__global__ void __launch_bounds__(256, 2) gist_prefill_mfma_kernel(GistPrefillLaunch a) {
    __shared__ __align__(16) char tile_a[2 * kPTile];
    __shared__ __align__(16) char tile_b[2 * kPTile];
    const int wg = a.w_gist_rows;
    if ((int)blockIdx.x < wg) gist_prefill_rows<true>(a, blockIdx.x, wg, tile_a, tile_b);
    else gist_prefill_rows<false>(a, blockIdx.x - wg, gridDim.x - wg, tile_a, tile_b);
}

static hipError_t gist_check(const GistPrefillLaunch& a) {
    if (a.d != kPD || a.L % kPBlk || a.g < 1 || a.g > kPBlk || kPBlk % a.g || a.Hkv <= 0 ||
        a.Hq % a.Hkv || a.Gp % kPBlk || a.Gp < a.M * a.g)
        return hipErrorNotSupported;
    return hipSuccess;
}

hipError_t launch_gist_gather(const GistPrefillLaunch& a, hipStream_t s,
                              const KernelEvents& ev) {
    hipError_t e = gist_check(a);
    if (e != hipSuccess) return e;
    const long long W = (long long)a.B * a.Hkv * (a.Gp / kPBlk);
    if (W <= 0) return no_kernel(ev, s);
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    return dispatch(gist_gather_kernel, dim3((unsigned)W), dim3(256), 0, s, ev, a);
}

hipError_t launch_gist_prefill_rows(GistPrefillLaunch a, hipStream_t s, const KernelEvents& ev) {
    hipError_t e = gist_check(a);
    if (e != hipSuccess) return e;
    const int G = a.Hq / a.Hkv;
    const long long Wr = 2LL * a.B * a.Hkv * a.M * (a.L / kPBlk) * ((G + 3) / 4);
    const long long Wgs = 2LL * a.B * a.Hkv * (a.Gp / kPBlk) * ((G + 3) / 4);
    if (Wr + Wgs <= 0) return no_kernel(ev, s);
    if (Wr + Wgs > 0x7fffffffLL) return hipErrorNotSupported;
    a.w_gist_rows = (int)Wgs;
    return dispatch(gist_prefill_mfma_kernel, dim3((unsigned)(Wr + Wgs)), dim3(256), 0, s, ev, a);
}

}  // namespace tcs
