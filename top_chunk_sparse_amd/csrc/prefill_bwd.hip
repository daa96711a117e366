// prefill_bwd.hip -- gfx950 kernels of the block-sparse causal prefill backward (SAS
// training form: the gate is trained end to end through the softmax).
#include "device.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"

#include <math.h>

namespace tcs {

// =============================================================================================
// Backward: gradients of L = sum dout . out + sum dlse . lse.  For a query row with softmax
// weights P over its visible keys and D = dout . out - dlse, the logit gradient of key x is
// dS_x = P_x (dout . v_x - D); then dq = sigma sum_x dS_x k_x, dk_x = sigma sum_rows dS_x q,
// dv_x = sum_rows P_x dout, and the gate gradient of chosen block j of query block i is the sum
// of dS over every (head, row, key) of (i, j), which reaches S through the log-softmax gate.
// P is recomputed from the forward's lse, so no running max is needed.  Every sum is taken in
// a fixed order (no floating-point atomics): the same inputs give the same bits.
//
//   prefill_bwd_prep_kernel     one grid: per key block j the query blocks i > j that chose
//                               it, ascending, with their gates (the first workgroups); then D
//                               for every query row.
//   prefill_bwd_dq_kernel       the forward's work split (unit, i, row half, head group): per
//                               visible block S^T = K Q^T and dP^T = V dO^T, dS^T = P^T (dP^T - D),
//                               dQ^T += K^T dS^T, and the block's sum of dS^T (gate partial).
//   prefill_bwd_dkv_kernel      per (unit, key block j), two waves per 32 keys: for each head
//                               and each query block that sees j, one wave forms S = Q K^T, P
//                               and dV^T += dO^T P, the other dP = dO V^T, dS and
//                               dK^T += Q^T dS, with a lane per key, in registers.
//   prefill_bwd_ds_kernel       per (unit, i): dS[i][j'] = [j' chosen] dg_ij' -
//                               softmax(S[i][. < i])_j' sum_j dg_ij.
// =============================================================================================

// D of 16 * kPrepU consecutive query rows per workgroup: 16 lanes per row, 16 rows per pass,
// the loads of all passes issued before the first sum (read once: non-temporal).
constexpr int kPrepU = 4;

__device__ __forceinline__ void prep_rows(const PrefillBwdLaunch& a, long long wg) {
    const long long rows = (long long)a.B * a.Hq * a.T;
    const int l16 = threadIdx.x & 15;
    const long long r0 = wg * (16 * kPrepU) + (threadIdx.x >> 4);
    u32x4 g[kPrepU], o0[kPrepU], o1[kPrepU];
#pragma unroll
    for (int u = 0; u < kPrepU; ++u) {
        const long long row = min(r0 + 16 * u, rows - 1);   // in bounds; the store is guarded
        g[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(a.dout + row * kPD + l16 * 8));
        o0[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(a.out + row * kPD + l16 * 8));
        o1[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(a.out + row * kPD + l16 * 8 + 4));
    }
#pragma unroll
    for (int u = 0; u < kPrepU; ++u) {
        const long long row = r0 + 16 * u;
        float x = bf16_lo(g[u].x) * __uint_as_float(o0[u].x) +
                  bf16_hi(g[u].x) * __uint_as_float(o0[u].y) +
                  bf16_lo(g[u].y) * __uint_as_float(o0[u].z) +
                  bf16_hi(g[u].y) * __uint_as_float(o0[u].w) +
                  bf16_lo(g[u].z) * __uint_as_float(o1[u].x) +
                  bf16_hi(g[u].z) * __uint_as_float(o1[u].y) +
                  bf16_lo(g[u].w) * __uint_as_float(o1[u].z) +
                  bf16_hi(g[u].w) * __uint_as_float(o1[u].w);
        x += __shfl_xor(x, 8, 16);
        x += __shfl_xor(x, 4, 16);
        x += __shfl_xor(x, 2, 16);
        x += __shfl_xor(x, 1, 16);
        if (l16 == 0 && row < rows) a.D[row] = x - (a.dlse ? a.dlse[row] : 0.f);
    }
}

// Per key block j (row = unit * nb + j): the query blocks i > j that chose j, ascending, with
// the gate of that choice, compacted by a workgroup scan over i.
__device__ __forceinline__ void inverse_lists(const PrefillBwdLaunch& a, int wg, ScanSmem& scan,
                                              int& total) {
    const int nb = a.T / kPBlk;
    const int unit = wg / nb, j = wg % nb;
    const long long row = (long long)unit * nb + j;
    int base = 0;
    for (int i0 = j + 1; i0 < nb; i0 += 256) {
        const int i = i0 + threadIdx.x;
        int slot = -1;
        if (i < nb && a.ksel > 0) {
            const int32_t* sr = a.sel + ((long long)unit * nb + i) * a.ksel;
            const int ke = min(a.ksel, i);
            for (int x = 0; x < ke; ++x) slot = sr[x] == j ? x : slot;
        }
        const int f = slot >= 0 ? 1 : 0;
        const int pos = base + block_exclusive_scan(f, scan);
        if (f) {
            a.inv_i[row * nb + pos] = i;
            a.inv_g[row * nb + pos] =
                a.gamma ? a.gamma[((long long)unit * nb + i) * a.ksel + slot] : 0.f;
        }
        if (threadIdx.x == 255) total = pos + f;
        __syncthreads();
        base = total;
        __syncthreads();
    }
    if (threadIdx.x == 0) a.inv_n[row] = base;
}

// One grid for both: the inverse lists' workgroups first (few and latency-bound), then the D
// rows' (bandwidth-bound), which start as the first lists finish.  (Spread evenly through the
// grid instead, the lists' workgroups made the launch slower.)
__global__ void __launch_bounds__(256) prefill_bwd_prep_kernel(PrefillBwdLaunch a) {
    __shared__ ScanSmem scan;
    __shared__ int total;
    const int n_inv = a.B * a.Hkv * (a.T / kPBlk);
    if ((int)blockIdx.x < n_inv)
        inverse_lists(a, blockIdx.x, scan, total);
    else
        prep_rows(a, (long long)blockIdx.x - n_inv);
}

// Two workgroups per CU (one would leave one wave per SIMD with nothing to hide its latency),
// so 256 registers per lane.  Blocks are copied global -> LDS directly (no staging registers)
// into two buffers that are distinct LDS objects, the block loop unrolled by two so that every
// copy and every operand read names its buffer: the compiler's wait counting then lets the
// operand reads of one buffer run while the next block's copy into the other is in flight.
// The registers this frees hold the dO^T operand for the whole loop.
//
// One dq item: workgroup bid of the W dq workgroups.  tile_a and tile_b (each 2 kPTile bytes)
// are two distinct LDS objects of the calling kernel; ring_j and ring_g hold kRing entries.
// The XCD-contiguous ranges below take bid's XCD as bid % 8, which holds in the gradient grid
// when the dk / dv workgroups ahead of it are a multiple of 8 (8 KV heads or B Hkv nb % 8 == 0;
// otherwise only the L2 grouping is lost).
__device__ __forceinline__ void bwd_dq_item(const PrefillBwdLaunch& a, int bid, const int W,
                                            char* tile_a, char* tile_b, int* ring_j,
                                            float* ring_g) {
    const int G = a.Hq / a.Hkv;
    const int nb = a.T / kPBlk;
    const int nhg = (G + 3) >> 2;
    if ((W & 7) == 0) bid = (bid & 7) * (W >> 3) + (bid >> 3);
    const int rh = bid & 1;
    const int i = nb - 1 - (bid >> 1) % nb;
    const int rest = (bid >> 1) / nb;
    const int hg = rest % nhg;
    const int unit = rest / nhg;
    const int b = unit / a.Hkv, kv = unit % a.Hkv;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int head = hg * 4 + w;
    const bool active = head < G;

    const uint16_t* kbase = a.k + (size_t)unit * a.T * kPD;
    const uint16_t* vbase = a.v + (size_t)unit * a.T * kPD;
    const int ke = a.ksel > 0 ? min(a.ksel, i) : 0;
    const int32_t* selrow = a.sel ? a.sel + ((size_t)unit * nb + i) * a.ksel : nullptr;
    const float* grow = a.gamma ? a.gamma + ((size_t)unit * nb + i) * a.ksel : nullptr;
    auto fill_ring = [&](int x0) {
        const int x = x0 + threadIdx.x;
        if (threadIdx.x < kRing / 2 && x < ke) {
            ring_j[x & (kRing - 1)] = min(max(selrow[x], 0), i - 1);
            ring_g[x & (kRing - 1)] = grow ? grow[x] * kLog2e : 0.f;
        }
    };
    fill_ring(0);
    fill_ring(kRing / 2);

    // K tiles in the transposable layout (read as K and as K^T), V tiles in the row layout;
    // block j's K tile at buf, its V tile at buf + kPTile, chunk c of wave w the 1 KB at
    // (4 c + w) KB of each
    const CopyOffsets gk = copy_offsets(kSwzT, w, lane), gv = copy_offsets(kSwzK, w, lane);
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

    const size_t qrow = ((size_t)(b * a.Hq + kv * G + (active ? head : 0)) * a.T +
                         (size_t)i * kPBlk + 32 * rh + c32);
    // Q^T and dO^T operands of this lane's query row, both for the whole loop, read whole
    // through this wave's 8 KB of tile_b (free until the first block copy into it)
    char* stage = tile_b + w * kQRowsLds;
    bf16x8 qf[8], gf[8];
    load_q_operand(a.q + (qrow - c32) * kPD, stage, lane, qf);
    load_q_operand(a.dout + (qrow - c32) * kPD, stage, lane, gf);
    const float lse2 = a.lse[qrow] * kLog2e;
    const float Dq = a.D[qrow];

    const int koff0 = c32 * 64 + (((0 + h) ^ swz_t(c32)) << 4);
    const int koff1 = c32 * 64 + (((2 + h) ^ swz_t(c32)) << 4);
    const int voff0 = c32 * 64 + (((0 + h) ^ swz_k(c32)) << 4);
    const int voff1 = c32 * 64 + (((2 + h) ^ swz_k(c32)) << 4);
    const TrOffsets toff = tr_offsets_t(lane);

    const float cs = a.sigma * kLog2e;
    float* dg = a.dgp + ((((size_t)unit * nb + i) * 2 + rh) * (size_t)(nhg * 4) + head) * a.ksel;
    f32x16 dq[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dq[dt] = f32x16{};

    // block t is in cur; the copy of block t + 1 goes into nxt once every wave is past block
    // t - 1 (which was in nxt)
    auto block = [&](int t, char* cur, char* nxt) {
        wait_vmem_lds();   // this wave's part of block t has landed
        __syncthreads();   // and every wave's; every wave is done with nxt
        const float bias = t > 0 ? __int_as_float(__builtin_amdgcn_readfirstlane(
                                       __float_as_int(ring_g[(t - 1) & (kRing - 1)])))
                                 : 0.f;
        if (t < ke) dma(__builtin_amdgcn_readfirstlane(ring_j[t & (kRing - 1)]), nxt);
        if (t > kRing / 2 && ((t - 1) & (kRing / 2 - 1)) == 0 && t - 1 + kRing / 2 < ke)
            fill_ring(t - 1 + kRing / 2);
        if (active) {
            const bool half = (t == 0) && rh == 0;   // diagonal, first row half: keys 0..31
            const char* kt = cur;
            const char* vt = cur + kPTile;
            f32x16 s[2], dp[2];
            s[0] = s[1] = dp[0] = dp[1] = f32x16{};
            if (half) {
                qk_product<1>(kt, koff0, koff1, qf, s);
                qk_product<1>(vt, voff0, voff1, gf, dp);
            } else {
                qk_product<2>(kt, koff0, koff1, qf, s);
                qk_product<2>(vt, voff0, voff1, gf, dp);
            }
            const int q = 32 * rh + c32;
            const float off = bias - lse2;
            float gsum = 0.f;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = 32 * x + 8 * (e >> 2) + 4 * h + (e & 3);
                    float p = __builtin_amdgcn_exp2f(s[x][e] * cs + off);
                    if (t == 0 && key > q) p = 0.f;
                    const float d = p * (dp[x][e] - Dq);
                    dp[x][e] = d;
                    gsum += d;
                }
            if (t > 0) {
                gsum = wave_sum(gsum);
                if (lane == 0) dg[t - 1] = gsum;
            }
            // dQ^T += K^T dS^T over the block's keys (16 per step)
            const char* ktlo = kt + toff.lo;
            const char* kthi = kt + toff.hi;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if (half && st >= 2) break;
                bf16x8 db;
#pragma unroll
                for (int e = 0; e < 8; ++e) db[e] = (__bf16)dp[st >> 1][8 * (st & 1) + e];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        t_operand(ktlo, kthi, dt, st), db, dq[dt], 0, 0, 0);
            }
        }
    };
    for (int t = 0; t <= ke; t += 2) {
        block(t, tile_a, tile_b);
        if (t + 1 <= ke) block(t + 1, tile_b, tile_a);
    }
    __syncthreads();   // every wave is done with the last block's tiles
    if (!active) return;
    // the output through this wave's 16 KB: waves 0, 1 in tile_a, waves 2, 3 in tile_b
    store_rows_f32(dq, a.sigma, (w < 2 ? tile_a : tile_b) + (w & 1) * kORowsLds,
                   a.dq + (qrow - c32) * kPD, lane);
}

// dk / dv: a workgroup of four waves per (unit, key block j).  Wave w works on keys
// 32 kh .. 32 kh + 31 of the block (kh = w & 1) in one of two roles, so that each wave holds
// one key-row operand and one accumulator set and two workgroups fit on a CU:
//   role A (w < 2): S = Q K^T, P = exp2(S - lse) (token-causal on the diagonal block),
//                   dV^T += dO^T P;
//   role B (w >= 2): dP = dO V^T, dS = P (dP - D) with the P that role A left in LDS,
//                   dK^T += Q^T dS.
// Every (head, query block) pair that sees j is one item; the four waves share its Q and dO
// tiles, and the next item's tiles are copied global -> LDS directly while the current one is
// computed (two LDS buffers, distinct objects, the loop unrolled by two as in the dq kernel).  An item has two phases: the S / dP products (with the exponentials of
// role A), a barrier, then the dV / dK products.  Both roles accumulate in registers to the
// end of the list.
constexpr int kBwdBuf = 2 * kPTile + 2 * kPBlk * 4;   // Q tile, dO tile, lse2 and D of 64 rows
constexpr int kBwdP = 4 * 64 * 16;                    // P of 32 keys x 64 rows, fp16

// One dk / dv item: workgroup bid of the B Hkv nb dk / dv workgroups.  buf_a and buf_b (each
// kBwdBuf bytes: two pair buffers, distinct LDS objects of the calling kernel, see the dq
// item), pshare (2 kBwdP bytes: the P hand-over) and the two list slots.
__device__ __forceinline__ void bwd_dkv_item(const PrefillBwdLaunch& a, const int bid,
                                             char* buf_a, char* buf_b, char* pshare,
                                             int* slot_i, float* slot_g) {
    const int G = a.Hq / a.Hkv;
    const int nb = a.T / kPBlk;
    const int units = a.B * a.Hkv;
    // key-block major: the blocks that most query blocks choose (low j) start first, and with
    // eight KV heads each XCD keeps one head's queries in its L2
    const int j = bid / units;
    const int unit = bid % units;
    const int b = unit / a.Hkv, kv = unit % a.Hkv;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int kh = w & 1;
    const bool roleA = w < 2;

    // K^T (role A) or V^T (role B) operand of this lane's key row, kept for the whole kernel
    const size_t kfirst = (size_t)unit * a.T + (size_t)j * kPBlk + 32 * kh;
    bf16x8 kvf[8];
    {
        const uint16_t* kp = (roleA ? a.k : a.v) + (kfirst + c32) * kPD + 8 * h;
#pragma unroll
        for (int kd = 0; kd < 8; ++kd) kvf[kd] = *reinterpret_cast<const bf16x8*>(kp + 16 * kd);
    }
    // Q and dO tiles are stored in the transposable layout and read both row-major (the S / dP
    // products) and transposed (the dV / dK products).
    const int qoff0 = c32 * 64 + (((0 + h) ^ swz_t(c32)) << 4);
    const int qoff1 = c32 * 64 + (((2 + h) ^ swz_t(c32)) << 4);
    const TrOffsets toff = tr_offsets_t(lane);
    const size_t lrow = (size_t)unit * nb + j;
    const int nlist = 1 + a.inv_n[lrow];     // the diagonal block, then the choosers
    const int nitems = G * nlist;             // (head, query block) pairs, head-major
    const float cs = a.sigma * kLog2e;
    const int key = 32 * kh + c32;            // this lane's key row within block j
    // P of this key half: step st of lane l at (64 st + l) * 16 bytes, the same lane and step
    // layout in which role B holds dP, so the hand-over needs no shuffle
    char* pbuf = pshare + kh * kBwdP + lane * 16;
    const CopyOffsets gk = copy_offsets(kSwzT, w, lane), gv = gk;

    // (head, query block) pair it: head it / nlist; list position t = it % nlist: query block j
    // itself (t = 0), then the choosers of j in ascending order.  A pair's query block and
    // gate come from LDS slot it & 1: the lists are read two pairs ahead, with the tiles of the
    // next pair, and thread 0 writes the slot with the tiles at the end of an iteration, so no
    // list read waits in the loop.
    int xi = 0;        // raw list entries of a pair (loaded by every thread from one address)
    float xg = 0.f;
    auto list_load = [&](int it) {
        const size_t e = lrow * nb + max(it % nlist - 1, 0);
        xi = a.inv_i[e];
        xg = a.inv_g[e];
    };
    auto list_store = [&](int it, int sl) {   // pair it's query block and gate (log2 units)
        const bool first = it % nlist == 0;
        slot_i[sl] = first ? j : xi;
        slot_g[sl] = first ? 0.f : xg * kLog2e;
    };
    auto qrow_of = [&](int it, int i) {
        return (size_t)(b * a.Hq + kv * G + it / nlist) * a.T + (size_t)i * kPBlk;
    };
    // a pair's Q and dO tiles straight into LDS buffer buf (Q at buf, dO at buf + kPTile; chunk
    // c of wave w is the 1 KB at (4 c + w) KB of each); its rows' lse (threads 0..63) and D
    // (threads 64..127) go through registers (xl) and are stored after the pair's products
    auto dma = [&](size_t qrow0, char* buf) {
        const char* qc = reinterpret_cast<const char*>(a.q + qrow0 * kPD);
        const char* gc = reinterpret_cast<const char*>(a.dout + qrow0 * kPD);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            __builtin_amdgcn_global_load_lds(qc + gk.c[c], (lds_void*)(buf + (4 * c + w) * 1024),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(gc + gv.c[c],
                                             (lds_void*)(buf + kPTile + (4 * c + w) * 1024), 16,
                                             0, 0);
        }
    };
    float xl = 0.f;
    auto rows_load = [&](size_t qrow0) {
        if (tid < 2 * kPBlk) xl = tid < kPBlk ? a.lse[qrow0 + tid] : a.D[qrow0 + tid - kPBlk];
    };
    auto rows_store = [&](char* buf) {
        if (tid < 2 * kPBlk) reinterpret_cast<float*>(buf + 2 * kPTile)[tid] = xl;
    };

    f32x16 acc[4];   // role A: dV^T, role B: dK^T (32 dims per tile x 32 keys)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

    // pair 0 is (head 0, block j); pair 1's list entry goes to its slot before the loop
    int i_cur = j;
    float bias_cur = 0.f;
    list_load(min(1, nitems - 1));
    rows_load(qrow_of(0, j));
    dma(qrow_of(0, j), buf_a);
    rows_store(buf_a);
    if (tid == 0) list_store(min(1, nitems - 1), 1);

    // pair it is in cur; pair it + 1 is copied into nxt once every wave is past pair it - 1
    // (which was in nxt)
    auto pair = [&](int it, const char* cur, char* nxt) {
        wait_vmem_lds();   // this wave's part of pair it has landed
        __syncthreads();   // and every wave's; slot it & 1 is written; nxt is free
        const bool diag = i_cur == j;
        const float bias = bias_cur;
        int i_nx = 0;
        float bias_nx = 0.f;
        if (it + 1 < nitems) {
            i_nx = __builtin_amdgcn_readfirstlane(slot_i[(it + 1) & 1]);
            bias_nx = __int_as_float(
                __builtin_amdgcn_readfirstlane(__float_as_int(slot_g[(it + 1) & 1])));
            list_load(min(it + 2, nitems - 1));   // before the copy: their waits leave the copy
            rows_load(qrow_of(it + 1, i_nx));
            dma(qrow_of(it + 1, i_nx), nxt);
        }

        // ---- phase 1: S = Q K^T (A) or dP = dO V^T (B); lane: key, rows: queries ----
        f32x16 s[2];
        s[0] = s[1] = f32x16{};
        // (offsets on cur rather than a select of two pointers keep the reads' LDS object
        // visible to the compiler's wait counting)
        // the rows' lse (A) or D (B), read ahead of the products so that they have landed by
        // the time the products are done
        float4 rs[2][4];
        {
            const float* rsl = reinterpret_cast<const float*>(cur + 2 * kPTile +
                                                              (roleA ? 0 : kPBlk * 4));
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4)
                    rs[x][e4] = *reinterpret_cast<const float4*>(rsl + 32 * x + 8 * e4 + 4 * h);
        }
        __builtin_amdgcn_sched_barrier(0);
        qk_product<2>(cur + (roleA ? 0 : kPTile), qoff0, qoff1, kvf, s);
        bf16x8 ob[4];   // the B operands of phase 2: P (A) or dS (B), 16 query rows per step
        if (roleA) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int q0 = 32 * x + 8 * e4 + 4 * h;   // query rows q0 .. q0 + 3
                    const float4 lq = rs[x][e4];
                    const float lv[4] = {lq.x, lq.y, lq.z, lq.w};
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int e = 4 * e4 + jj;
                        float p = __builtin_amdgcn_exp2f(
                            fmaf(s[x][e], cs, fmaf(-lv[jj], kLog2e, bias)));
                        if (diag && key > q0 + jj) p = 0.f;   // diagonal block: token-causal
                        s[x][e] = p;
                    }
                }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                half8 ph;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ob[st][e] = (__bf16)s[st >> 1][8 * (st & 1) + e];
                    ph[e] = (_Float16)s[st >> 1][8 * (st & 1) + e];
                }
                *reinterpret_cast<half8*>(pbuf + st * 1024) = ph;
            }
        }
        lds_handoff_barrier();   // P of this item is in LDS (the next pair's copy flies on)
        if (!roleA) {
            half8 ph[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) ph[st] = *reinterpret_cast<const half8*>(pbuf + st * 1024);
            __builtin_amdgcn_sched_barrier(0);   // all four reads in flight before the first use
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const float4 dd = rs[x][e4];
                    const float dv4[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int e = 4 * e4 + jj;   // step 2 x + e / 8, element e % 8
                        const float p = (float)ph[2 * x + (e >> 3)][e & 7];
                        s[x][e] = p * (s[x][e] - dv4[jj]);
                    }
                }
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int e = 0; e < 8; ++e) ob[st][e] = (__bf16)s[st >> 1][8 * (st & 1) + e];
        }

        // ---- phase 2: dV^T += dO^T P (A) or dK^T += Q^T dS (B), 16 query rows per step ----
        const char* tt = cur + (roleA ? kPTile : 0);
        const char* tlo = tt + toff.lo;
        const char* thi = tt + toff.hi;
        // the transposing operand reads run a step ahead of the products (left to itself the
        // compiler read each product's operand just before it and waited for it there)
        bf16x8 opr[2][4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) opr[0][dt] = t_operand(tlo, thi, dt, 0);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (st + 1 < 4) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) opr[(st + 1) & 1][dt] = t_operand(tlo, thi, dt, st + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opr[st & 1][dt], ob[st], acc[dt],
                                                                  0, 0, 0);
        }
        if (it + 1 < nitems) {
            rows_store(nxt);
            if (tid == 0) list_store(min(it + 2, nitems - 1), it & 1);
            i_cur = i_nx;
            bias_cur = bias_nx;
        }
    };
    for (int it = 0; it < nitems; it += 2) {
        pair(it, buf_a, buf_b);
        if (it + 1 < nitems) pair(it + 1, buf_b, buf_a);
    }

    // this wave's 32 key rows: dV = dV^T (A) or dK = sigma dK^T (B); lane: key row, registers:
    // dims
    __syncthreads();   // every wave is done with the last pair's tiles
    store_rows_f32(acc, roleA ? 1.f : a.sigma, (w < 2 ? buf_a : buf_b) + (w & 1) * kORowsLds,
                   (roleA ? a.dv : a.dk) + kfirst * kPD, lane);
}

// dq and dk / dv in one grid.  Neither reads what the other writes (both take the row terms D
// and the chosen-by lists of the prep pass), so no workgroup waits for another.  The dk / dv
// workgroups come first: they are the long items (the most-chosen key blocks lead), and the
// shorter dq workgroups then fill the CU slots they leave, so neither part's tail runs on an
// otherwise idle GPU and one launch boundary goes.  Both parts use the same LDS objects, so the
// kernel keeps two workgroups per CU.
static_assert(kBwdBuf >= 2 * kPTile, "a dk / dv pair buffer holds a dq K / V block");
static_assert(2 * kBwdP >= kRing * (int)(sizeof(int) + sizeof(float)), "dq block-list ring");
__global__ void __launch_bounds__(256, 2) prefill_bwd_grad_kernel(PrefillBwdLaunch a) {
    __shared__ __align__(16) char buf_a[kBwdBuf];
    __shared__ __align__(16) char buf_b[kBwdBuf];
    __shared__ __align__(16) char pshare[2 * kBwdP];   // dk / dv: P hand-over; dq: block list
    __shared__ int slot_i[2];
    __shared__ float slot_g[2];
    const int wk = a.w_dkv;
    if ((int)blockIdx.x < wk) {
        bwd_dkv_item(a, blockIdx.x, buf_a, buf_b, pshare, slot_i, slot_g);
    } else {
        bwd_dq_item(a, blockIdx.x - wk, gridDim.x - wk, buf_a, buf_b,
                    reinterpret_cast<int*>(pshare),
                    reinterpret_cast<float*>(pshare + kRing * sizeof(int)));
    }
}

__global__ void __launch_bounds__(256) prefill_bwd_ds_kernel(PrefillBwdLaunch a) {
    __shared__ ReduceSmem red;
    const int G = a.Hq / a.Hkv;
    const int nb = a.T / kPBlk;
    const int nh = 4 * ((G + 3) >> 2);
    const long long row = blockIdx.x;   // unit * nb + i
    const int i = (int)(row % nb);
    float* out = a.dS + row * nb;
    const int ke = a.ksel > 0 ? min(a.ksel, i) : 0;
    if (!a.gate || ke == 0) {
        for (int j = threadIdx.x; j < nb; j += 256) out[j] = 0.f;
        return;
    }
    const int32_t* sr = a.sel + row * a.ksel;
    auto dg_of = [&](int x) {   // the chosen slot's gate gradient: row halves, then heads
        float v = 0.f;
        for (int rh = 0; rh < 2; ++rh)
            for (int hd = 0; hd < G; ++hd) v += a.dgp[((row * 2 + rh) * nh + hd) * a.ksel + x];
        return v;
    };
    float part = 0.f;
    for (int x = threadIdx.x; x < ke; x += 256) part += dg_of(x);
    const float tot = block_sum(part, red);
    const float* srow = a.S + row * nb;
    float mx = -INFINITY;
    for (int j = threadIdx.x; j < i; j += 256) mx = fmaxf(mx, srow[j]);
    mx = block_max(mx, red);
    float z = 0.f;
    for (int j = threadIdx.x; j < i; j += 256) z += expf(srow[j] - mx);
    z = block_sum(z, red);
    const float lse = mx + logf(z);
    for (int j = threadIdx.x; j < nb; j += 256) {
        float v = 0.f;
        if (j < i) {
            v = -expf(srow[j] - lse) * tot;
            int lo = 0, hi = ke;   // the chosen list is ascending
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (sr[mid] < j) lo = mid + 1;
                else hi = mid;
            }
            if (lo < ke && sr[lo] == j) v += dg_of(lo);
        }
        out[j] = v;
    }
}

static hipError_t bwd_check(const PrefillBwdLaunch& a) {
    if (a.d != kPD || a.blk != kPBlk || a.T % kPBlk || a.Hkv <= 0 || a.Hq % a.Hkv)
        return hipErrorNotSupported;
    return hipSuccess;
}

hipError_t launch_prefill_bwd_prep(const PrefillBwdLaunch& a, hipStream_t s,
                                   const KernelEvents& ev) {
    hipError_t e = bwd_check(a);
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.B * a.Hq * a.T;
    const long long g1 = (rows + 16 * kPrepU - 1) / (16 * kPrepU);   // D rows
    const long long g2 = (long long)a.B * a.Hkv * (a.T / kPBlk);      // inverse lists
    if (g1 + g2 > 0x7fffffffLL) return hipErrorNotSupported;
    if (g1 + g2 <= 0) return no_kernel(ev, s);
    return dispatch(prefill_bwd_prep_kernel, dim3((unsigned)(g1 + g2)), dim3(256), 0, s, ev, a);
}

hipError_t launch_prefill_bwd_grad(PrefillBwdLaunch a, hipStream_t s, const KernelEvents& ev) {
    hipError_t e = bwd_check(a);
    if (e != hipSuccess) return e;
    const int G = a.Hq / a.Hkv;
    const long long Wq = 2LL * a.B * a.Hkv * (a.T / kPBlk) * ((G + 3) / 4);   // dq
    const long long Wk = (long long)a.B * a.Hkv * (a.T / kPBlk);               // dk / dv
    if (Wq + Wk <= 0) return no_kernel(ev, s);
    if (Wq + Wk > 0x7fffffffLL) return hipErrorNotSupported;
    a.w_dkv = (int)Wk;
    return dispatch(prefill_bwd_grad_kernel, dim3((unsigned)(Wq + Wk)), dim3(256), 0, s, ev, a);
}

hipError_t launch_prefill_bwd_ds(const PrefillBwdLaunch& a, hipStream_t s,
                                 const KernelEvents& ev) {
    hipError_t e = bwd_check(a);
    if (e != hipSuccess) return e;
    const long long W = (long long)a.B * a.Hkv * (a.T / kPBlk);
    if (!a.dS || W <= 0) return no_kernel(ev, s);
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    return dispatch(prefill_bwd_ds_kernel, dim3((unsigned)W), dim3(256), 0, s, ev, a);
}

}  // namespace tcs
