// prefill.hip -- gfx950 kernels of the block-sparse causal prefill (SAS training-form
// forward, "SAS: Simple Attention Sparsification", abstract: the selector's scores enter the
// attention logits inside the softmax in log form, on a FlashAttention-style forward).
//
//   prefill_select_kernel  per (b, kv, query block i): top-min(k, i) earlier blocks by the
//                          selector row S[i][j < i] (lowest j on ties), ascending, and the
//                          gate log_softmax_j(S[i][j < i]) for the chosen blocks.
//   prefill_fwd_kernel     per (b, kv, query block i, group of up to 4 query heads): online
//                          softmax attention of the block's 64 query rows over its diagonal
//                          block (token-causal) and each chosen earlier block (fully visible,
//                          logit + gate), with bf16 MFMA for both products.
#include "device.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"

#include <math.h>

namespace tcs {

__global__ void __launch_bounds__(256) prefill_select_kernel(PrefillSelectLaunch a) {
    __shared__ TopkSmem sm;
    __shared__ ReduceSmem red;
    const int row = blockIdx.x;                 // (unit * nb + i)
    const int i = row % a.nb;
    const float* s = a.S + (long long)row * a.nb;   // S[unit][i][0..nb)
    int32_t* sel = a.sel + (long long)row * a.k;
    float* gam = a.gamma ? a.gamma + (long long)row * a.k : nullptr;
    float lse = 0.f;
    if (gam && i > 0) {
        float mx = -INFINITY;
        for (int j = threadIdx.x; j < i; j += 256) mx = fmaxf(mx, s[j]);
        mx = block_max(mx, red);
        float z = 0.f;
        for (int j = threadIdx.x; j < i; j += 256) z += expf(s[j] - mx);
        z = block_sum(z, red);
        lse = mx + logf(z);
    }
    int ke;
    if (a.k >= i) {   // every earlier block is chosen: no ranking needed
        for (int j = threadIdx.x; j < i; j += 256) {
            sel[j] = j;
            if (gam) gam[j] = s[j] - lse;
        }
        ke = i;
    } else {
        ke = block_topk(
            i, a.k, [&](int j) { return s[j]; },
            [&](int x, int j) {
                sel[x] = j;
                if (gam) gam[x] = s[j] - lse;
            },
            sm);
    }
    for (int x = ke + threadIdx.x; x < a.k; x += 256) {
        sel[x] = -1;
        if (gam) gam[x] = 0.f;
    }
}

// The same selection with one wave per query block, for rows of at most 256 candidates (four
// per lane, candidate j on lane j % 64, register j / 64): no workgroup barrier anywhere.
// The k-th largest ordered key T is found bit by bit from the top (a bit is kept when at
// least k keys reach the prefix with it set), counted with ballots; every key above T is
// taken, then the keys equal to T in ascending position until k are taken.  Positions are
// written in ascending order: a chosen candidate's slot is the number of chosen ones before
// it, from the ballots' prefix counts.
__global__ void __launch_bounds__(256) prefill_select_wave_kernel(PrefillSelectLaunch a) {
    const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);   // (unit * nb + i)
    if (row >= a.units * a.nb) return;                          // wave-uniform, no barriers
    const int lane = threadIdx.x & 63;
    const int i = row % a.nb;
    const float* s = a.S + (long long)row * a.nb;   // S[unit][i][0..nb)
    int32_t* sel = a.sel + (long long)row * a.k;
    float* gam = a.gamma ? a.gamma + (long long)row * a.k : nullptr;
    float v[4];
    bool ok[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int j = 64 * m + lane;
        ok[m] = j < i;
        v[m] = ok[m] ? s[j] : 0.f;
    }
    float lse = 0.f;
    if (gam && i > 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < 4; ++m) mx = fmaxf(mx, ok[m] ? v[m] : -INFINITY);
        mx = wave_max(mx);
        float z = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) z += ok[m] ? expf(v[m] - mx) : 0.f;
        z = wave_sum(z);
        lse = mx + logf(z);
    }
    const unsigned long long below = (1ull << lane) - 1ull;   // lanes before this one
    if (a.k >= i) {   // every earlier block is chosen: no ranking needed
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if (ok[m]) {
                const int j = 64 * m + lane;
                sel[j] = j;
                if (gam) gam[j] = v[m] - lse;
            }
    } else {
        const int ke = a.k;   // < i
        uint32_t key[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) key[m] = ordered_key(v[m]);
        auto count_ge = [&](uint32_t t) {
            int c = 0;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok[m] && key[m] >= t));
            return c;
        };
        uint32_t T = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            if (count_ge(cand) >= ke) T = cand;
        }
        int gt = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            gt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok[m] && key[m] > T));
        const int take_eq = ke - gt;   // >= 1: at least ke keys reach T, fewer exceed it
        int base = 0, eq_base = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const unsigned long long eqm = __builtin_amdgcn_ballot_w64(ok[m] && key[m] == T);
            const bool tie_taken =
                ((eqm >> lane) & 1ull) && eq_base + __builtin_popcountll(eqm & below) < take_eq;
            const bool take = (ok[m] && key[m] > T) || tie_taken;
            const unsigned long long tm = __builtin_amdgcn_ballot_w64(take);
            if (take) {
                const int pos = base + __builtin_popcountll(tm & below);
                const int j = 64 * m + lane;
                sel[pos] = j;
                if (gam) gam[pos] = v[m] - lse;
            }
            base += __builtin_popcountll(tm);
            eq_base += __builtin_popcountll(eqm);
        }
    }
    const int ke = a.k < i ? a.k : i;
    for (int x = ke + lane; x < a.k; x += 64) {
        sel[x] = -1;
        if (gam) gam[x] = 0.f;
    }
}

hipError_t launch_prefill_select(const PrefillSelectLaunch& a, hipStream_t s,
                                 const KernelEvents& ev) {
    if (a.units <= 0 || a.nb <= 0 || a.k <= 0) return no_kernel(ev, s);
    if (a.nb <= 257) {   // at most 256 candidates per row
        const long long rows = (long long)a.units * a.nb;
        return dispatch(prefill_select_wave_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256),
                        0, s, ev, a);
    }
    return dispatch(prefill_select_kernel, dim3(a.units * a.nb), dim3(256), 0, s, ev, a);
}

// ---- block-sparse forward ------------------------------------------------------------------
//
// Workgroup: 4 waves for one (unit, query block i, row half rh, group of up to 4 heads); wave w
// owns query head 4*hg + w and the 32 query rows 32*rh .. 32*rh + 31 of block i.  Two
// workgroups share a CU (at most 256 registers per lane each), so the matrix work of one and
// the softmax of the other overlap on every SIMD.  All products are
// v_mfma_f32_32x32x16_bf16 (A: 32x16, lane l holds row l%32, k = 8*(l/32)..+7; B: 16x32, lane
// l holds column l%32, same k; D: 32x32, lane l holds column l%32, rows 8*i + 4*(l/32) + j in
// register 4*i + j).
//
//   S^T = K * Q^T   64 keys x 32 queries: a lane owns one query column, so the running max and
//                   sum of a query row live in the lane pair (l, l ^ 32).
//   O^T += V^T P^T  128 dims x 32 queries: the B operand (P^T) is the S^T accumulator of the
//                   same lane rounded to bf16; the A operand (V^T) is read from row-major V in
//                   LDS with the transposing ds_read_b64_tr_b16.
//
// LDS tile of one 64 x 128 block (K or V): four sub-tiles of 32 dims, each 64 rows x 64 B, so
// every operand address is one per-lane base plus a compile-time offset.  Within a 64-byte
// sub-row the 16-byte unit u of row r is stored at u ^ swz(r): for K, ((r >> 1) & 3) ^
// ((r >> 3) & 1) puts the 16 rows that one 128-bit read serves per cycle (and each half of
// them) on distinct banks; for V, (r & 2) keeps the 4 rows x 32 B of a transposing read on
// distinct banks.  Blocks are double buffered and copied global -> LDS directly (no staging
// registers): the two buffers are distinct LDS objects and the block loop is unrolled by two,
// so every copy and operand read names its buffer and the compiler's wait counting lets the
// operand reads of one buffer run while the next block's copy into the other is in flight.

__global__ void __launch_bounds__(256, 2) prefill_fwd_kernel(PrefillLaunch a) {
    __shared__ __align__(16) char tile_a[2 * kPTile];   // K then V of one block
    __shared__ __align__(16) char tile_b[2 * kPTile];
    __shared__ int ring_j[kRing];
    __shared__ float ring_g[kRing];
    const int G = a.Hq / a.Hkv;
    const int nb = a.T / kPBlk;
    const int nhg = (G + 3) >> 2;
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous range of
    // (unit, head group, block, row half) so one KV head's blocks stay in one L2.  Within a
    // range the query blocks run from last to first, the longest (most earlier blocks) first,
    // and the two row halves of a block run side by side, reading the same K/V blocks.
    int bid = blockIdx.x;
    const int W = gridDim.x;
    if ((W & 7) == 0) bid = (bid & 7) * (W >> 3) + (bid >> 3);
    const int rh = bid & 1;
    const int i = nb - 1 - (bid >> 1) % nb;
    const int rest = (bid >> 1) / nb;
    const int hg = rest % nhg;
    const int unit = rest / nhg;
    const int b = unit / a.Hkv, kv = unit % a.Hkv;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int head = hg * 4 + w;
    const bool active = head < G;

    const uint16_t* kbase = a.k + (size_t)unit * a.T * kPD;
    const uint16_t* vbase = a.v + (size_t)unit * a.T * kPD;

    const int ke = a.ksel > 0 ? min(a.ksel, i) : 0;
    const int32_t* selrow = a.sel ? a.sel + ((size_t)unit * nb + i) * a.ksel : nullptr;
    const float* grow = a.gamma ? a.gamma + ((size_t)unit * nb + i) * a.ksel : nullptr;

    // The chosen blocks and their gates pass through a ring of kRing entries in LDS, refilled
    // kRing / 2 entries at a time well ahead of use.
    auto fill_ring = [&](int x0) {   // entries x0 .. x0 + kRing/2 - 1 (those < ke)
        const int x = x0 + threadIdx.x;
        if (threadIdx.x < kRing / 2 && x < ke) {
            ring_j[x & (kRing - 1)] = min(max(selrow[x], 0), i - 1);
            ring_g[x & (kRing - 1)] = grow ? grow[x] * kLog2e : 0.f;
        }
    };
    fill_ring(0);
    fill_ring(kRing / 2);

    // Block 0 of the list is the diagonal block; blocks 1..ke are the chosen earlier ones.
    // Block j's K tile goes to buf, its V tile to buf + kPTile; chunk c of wave w is the 1 KB
    // at (4 c + w) KB of each.
    const CopyOffsets gk = copy_offsets(kSwzK, w, lane), gv = copy_offsets(kSwzV, w, lane);
    auto dma = [&](int j, char* buf) {
        const char* kc = reinterpret_cast<const char*>(kbase + (size_t)j * kPBlk * kPD);
        const char* vc = reinterpret_cast<const char*>(vbase + (size_t)j * kPBlk * kPD);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            __builtin_amdgcn_global_load_lds(kc + gk.c[c], (lds_void*)(buf + (4 * c + w) * 1024),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(vc + gv.c[c],
                                             (lds_void*)(buf + kPTile + (4 * c + w) * 1024), 16,
                                             0, 0);
        }
    };
    dma(i, tile_a);

    // Q^T operand: qf[kd] = Q[32 rh + c32][16 kd + 8 h .. +7] of this wave's head.
    const size_t qrow = ((size_t)(b * a.Hq + kv * G + (active ? head : 0)) * a.T +
                         (size_t)i * kPBlk + 32 * rh + c32);
    bf16x8 qf[8];   // read whole through this wave's 8 KB of tile_b (free until block 1)
    load_q_operand(a.q + (qrow - c32) * kPD, tile_b + w * kQRowsLds, lane, qf);

    // Per-lane LDS offsets (bytes) of the operand reads; everything else is an immediate.
    //   K: row r = 32 x + c32, d = 16 kd + 8 h: sub-tile kd / 2, unit (2 (kd & 1) + h) ^ swz.
    const int koff0 = c32 * 64 + (((0 + h) ^ swz_k(c32)) << 4);
    const int koff1 = c32 * 64 + (((2 + h) ^ swz_k(c32)) << 4);
    //   V (transposing read, 16-lane group g, lane L = 4 rr + cc of the group): row
    //   16 st + 8 rho + 4 h + rr, sub-tile dt, unit (2 (g & 1) + (cc >> 1)) ^ swz, half cc & 1.
    const int g = lane >> 4, L = lane & 15, rr = L >> 2, cc = L & 3;
    const int voff = (4 * h + rr) * 64 + (((2 * (g & 1) + (cc >> 1)) ^ swz_v(rr)) << 4) + ((cc & 1) << 3);


    const float cs = a.sigma * kLog2e;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m = 0.f, l = 0.f;
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

    // block t is in cur; the copy of block t + 1 goes into nxt once every wave is past block
    // t - 1 (which was in nxt)
    auto block = [&](int t, bool first, const char* cur, char* nxt) {   // first: t == 0
        wait_vmem_lds();   // this wave's part of block t has landed
        __syncthreads();   // and every wave's; every wave is done with nxt
        const float bias = first ? 0.f
                                 : __int_as_float(__builtin_amdgcn_readfirstlane(
                                       __float_as_int(ring_g[(t - 1) & (kRing - 1)])));
        if (t < ke) dma(__builtin_amdgcn_readfirstlane(ring_j[t & (kRing - 1)]), nxt);
        // Iteration t reads entries t - 1 and t.  Past this iteration's barrier every entry
        // below t is dead, so at t = 1 + n kRing/2 (n >= 1) the slots of entries
        // t - 1 - kRing/2 .. t - 2 take entries t - 1 + kRing/2 .. t - 2 + kRing, first read
        // kRing/2 - 1 iterations later.
        if (t > kRing / 2 && ((t - 1) & (kRing / 2 - 1)) == 0 && t - 1 + kRing / 2 < ke)
            fill_ring(t - 1 + kRing / 2);
        if (active) {
            // On the diagonal block, rows of the first half see only keys 0..31.
            const bool half = first && rh == 0;
            const char* kt = cur;
            const char* vt = cur + kPTile + voff;

            // ---- S^T = K Q^T ----
            f32x16 s[2];
            s[0] = s[1] = f32x16{};
            if (half) qk_product<1>(kt, koff0, koff1, qf, s);
            else qk_product<2>(kt, koff0, koff1, qf, s);
            // V operands are read now; their latency hides under the softmax.
            bf16x8 va[4][4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if (half && st >= 2) break;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) va[st][dt] = v_operand(vt, dt, st);
            }

            // ---- online softmax (log2 domain) ----
            if (first) {   // diagonal block: key row r sees query row q only if r <= q
                const int q = 32 * rh + c32;
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = 32 * x + 8 * (e >> 2) + 4 * h + (e & 3);
                        if (key > q) s[x][e] = -INFINITY;
                    }
            }
            float mx = s[0][0];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[x][e]);
            mx = pair_max(mx);
            const float mb = mx * cs + bias;
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
            const float off = bias - m;
            float sum = 0.f;
            auto p_step = [&](int st) {   // P^T for key step st (bf16) and its row-sum share
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
            // ---- O^T += V^T P^T, the products of one key step overlapping the exponentials of
            // the next ----
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
                // 4 products of step 0 against the 8 exponentials (+ arithmetic) of step 2
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
                }
                pv_mfma(1, p1);
                const bf16x8 p3 = p_step(3);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 2);
                }
                pv_mfma(2, p2);
                pv_mfma(3, p3);
            }
            l += sum;
        }
    };
    block(0, true, tile_a, tile_b);
    for (int t = 1; t <= ke; t += 2) {
        block(t, false, tile_b, tile_a);
        if (t + 1 <= ke) block(t + 1, false, tile_a, tile_b);
    }
    // ---- epilogue: O = O^T / l, lse = m + log2 l (back to natural log) ----
    __syncthreads();   // every wave is done with the last block's tiles
    if (!active) return;
    const float lt = pair_sum(l);
    const float inv = 1.f / lt;
    store_rows_f32(o, inv, (w < 2 ? tile_a : tile_b) + (w & 1) * kORowsLds,
                   a.out + (qrow - c32) * kPD, lane);
    if (a.lse && h == 0) a.lse[qrow] = (m + log2f(lt)) * kLn2;
}

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t s, const KernelEvents& ev) {
    if (a.d != kPD || a.blk != kPBlk || a.T % kPBlk) return hipErrorNotSupported;
    const int G = a.Hq / a.Hkv;
    const long long W = 2LL * a.B * a.Hkv * (a.T / kPBlk) * ((G + 3) / 4);
    if (W <= 0) return no_kernel(ev, s);
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    return dispatch(prefill_fwd_kernel, dim3((unsigned)W), dim3(256), 0, s, ev, a);
}

}  // namespace tcs
