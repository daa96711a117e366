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
//   prefill_bwd_prep_kernel     D for every query row.
//   prefill_bwd_inverse_kernel  per key block j: the query blocks i > j that chose it,
//                               ascending, with their gates.
//   prefill_bwd_dq_kernel       the forward's work split (unit, i, row half, head group): per
//                               visible block S^T = K Q^T and dP^T = V dO^T, dS^T = P^T (dP^T - D),
//                               dQ^T += K^T dS^T, and the block's sum of dS^T (gate partial).
//   prefill_bwd_dkv_kernel      per (unit, key block j), a wave per 32 keys: for each head and
//                               each query block that sees j, S = Q K^T and dP = dO V^T with a
//                               lane per key, dV^T += dO^T P and dK^T += Q^T dS, in registers.
//   prefill_bwd_ds_kernel       per (unit, i): dS[i][j'] = [j' chosen] dg_ij' -
//                               softmax(S[i][. < i])_j' sum_j dg_ij.
// =============================================================================================

__global__ void __launch_bounds__(256) prefill_bwd_prep_kernel(PrefillBwdLaunch a) {
    const long long rows = (long long)a.B * a.Hq * a.T;
    const long long row = ((long long)blockIdx.x * 256 + threadIdx.x) >> 4;
    const int l16 = threadIdx.x & 15;
    if (row >= rows) return;   // whole 16-lane groups leave together
    const uint4 g = *reinterpret_cast<const uint4*>(a.dout + row * kPD + l16 * 8);
    const float4 o0 = *reinterpret_cast<const float4*>(a.out + row * kPD + l16 * 8);
    const float4 o1 = *reinterpret_cast<const float4*>(a.out + row * kPD + l16 * 8 + 4);
    float x = bf16_lo(g.x) * o0.x + bf16_hi(g.x) * o0.y + bf16_lo(g.y) * o0.z +
              bf16_hi(g.y) * o0.w + bf16_lo(g.z) * o1.x + bf16_hi(g.z) * o1.y +
              bf16_lo(g.w) * o1.z + bf16_hi(g.w) * o1.w;
    x += __shfl_xor(x, 8, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 1, 16);
    if (l16 == 0) a.D[row] = x - (a.dlse ? a.dlse[row] : 0.f);
}

__global__ void __launch_bounds__(256) prefill_bwd_inverse_kernel(PrefillBwdLaunch a) {
    __shared__ ScanSmem scan;
    __shared__ int total;
    const int nb = a.T / kPBlk;
    const int unit = blockIdx.x / nb, j = blockIdx.x % nb;
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

// Two workgroups per CU (one would leave one wave per SIMD with nothing to hide its latency),
// so 256 registers per lane: the dO^T operand is re-read for every block from L1 / L2 rather
// than held for the whole loop, which keeps the kernel free of spills.
__global__ void __launch_bounds__(256, 2) prefill_bwd_dq_kernel(PrefillBwdLaunch a) {
    extern __shared__ __align__(16) char lds[];
    const int G = a.Hq / a.Hkv;
    const int nb = a.T / kPBlk;
    const int nhg = (G + 3) >> 2;
    int bid = blockIdx.x;
    const int W = gridDim.x;
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
    int* ring_j = reinterpret_cast<int*>(lds + kPLds);
    float* ring_g = reinterpret_cast<float*>(lds + kPLds + kRing * 4);
    auto fill_ring = [&](int x0) {
        const int x = x0 + threadIdx.x;
        if (threadIdx.x < kRing / 2 && x < ke) {
            ring_j[x & (kRing - 1)] = min(max(selrow[x], 0), i - 1);
            ring_g[x & (kRing - 1)] = grow ? grow[x] * kLog2e : 0.f;
        }
    };
    fill_ring(0);
    fill_ring(kRing / 2);

    // K tiles in the transposable layout (read as K and as K^T), V tiles in the row layout.
    const CopyOffsets gk = copy_offsets(true, w, lane), gv = copy_offsets(false, w, lane);
    uint4 sk0, sk1, sk2, sk3, sv0, sv1, sv2, sv3;
    TCS_STAGE_LOAD(kbase + (size_t)i * kPBlk * kPD, vbase + (size_t)i * kPBlk * kPD);

    const size_t qrow = ((size_t)(b * a.Hq + kv * G + (active ? head : 0)) * a.T +
                         (size_t)i * kPBlk + 32 * rh + c32);
    bf16x8 qf[8];   // Q^T operand of this lane's query row (dO^T is re-read per block)
    const uint16_t* gp = a.dout + qrow * kPD + 8 * h;
    {
        const uint16_t* qp = a.q + qrow * kPD + 8 * h;
#pragma unroll
        for (int kd = 0; kd < 8; ++kd) qf[kd] = *reinterpret_cast<const bf16x8*>(qp + 16 * kd);
    }
    const float lse2 = a.lse[qrow] * kLog2e;
    const float Dq = a.D[qrow];
    TCS_STAGE_STORE(lds, lds + 2 * kPTile);

    const int koff0 = c32 * 64 + (((0 + h) ^ swz_v(c32)) << 4);
    const int koff1 = c32 * 64 + (((2 + h) ^ swz_v(c32)) << 4);
    const int voff0 = c32 * 64 + (((0 + h) ^ swz_k(c32)) << 4);
    const int voff1 = c32 * 64 + (((2 + h) ^ swz_k(c32)) << 4);
    const int toff = tr_offset(lane);
    wait_vmem();

    const float cs = a.sigma * kLog2e;
    float* dg = a.dgp + ((((size_t)unit * nb + i) * 2 + rh) * (size_t)(nhg * 4) + head) * a.ksel;
    f32x16 dq[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dq[dt] = f32x16{};

    for (int t = 0; t <= ke; ++t) {
        __syncthreads();
        const int buf = t & 1;
        const float bias = t > 0 ? __int_as_float(__builtin_amdgcn_readfirstlane(
                                       __float_as_int(ring_g[(t - 1) & (kRing - 1)])))
                                 : 0.f;
        if (t < ke) {
            const int jn = __builtin_amdgcn_readfirstlane(ring_j[t & (kRing - 1)]);
            TCS_STAGE_LOAD(kbase + (size_t)jn * kPBlk * kPD, vbase + (size_t)jn * kPBlk * kPD);
        }
        if (t > kRing / 2 && ((t - 1) & (kRing / 2 - 1)) == 0 && t - 1 + kRing / 2 < ke)
            fill_ring(t - 1 + kRing / 2);
        if (active) {
            const bool half = (t == 0) && rh == 0;   // diagonal, first row half: keys 0..31
            const char* kt = lds + buf * kPTile;
            const char* vt = lds + (2 + buf) * kPTile;
            bf16x8 gf[8];   // dO^T operand (L1 / L2 resident across the blocks)
#pragma unroll
            for (int kd = 0; kd < 8; ++kd) gf[kd] = *reinterpret_cast<const bf16x8*>(gp + 16 * kd);
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
            const char* ktT = kt + toff;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if (half && st >= 2) break;
                bf16x8 db;
#pragma unroll
                for (int e = 0; e < 8; ++e) db[e] = (__bf16)dp[st >> 1][8 * (st & 1) + e];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(ktT, dt, st), db,
                                                                     dq[dt], 0, 0, 0);
            }
        }
        if (t < ke) TCS_STAGE_STORE(lds + (buf ^ 1) * kPTile, lds + (2 + (buf ^ 1)) * kPTile);
    }
    if (!active) return;
    float* op = a.dq + qrow * kPD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            float4 v;
            v.x = dq[dt][4 * e4 + 0] * a.sigma;
            v.y = dq[dt][4 * e4 + 1] * a.sigma;
            v.z = dq[dt][4 * e4 + 2] * a.sigma;
            v.w = dq[dt][4 * e4 + 3] * a.sigma;
            *reinterpret_cast<float4*>(op + 32 * dt + 8 * e4 + 4 * h) = v;
        }
}

// dk / dv: a workgroup of two waves per (unit, key block j); wave w owns keys 32 w .. 32 w + 31
// of the block and accumulates their dK^T and dV^T over every (head, query block) pair that
// sees j, in registers, to the end.  The two waves share each pair's Q and dO tiles; the next
// pair's tiles travel into registers while the current pair is computed (two LDS buffers).
constexpr int kBwdBuf = 2 * kPTile + 2 * kPBlk * 4;   // Q tile, dO tile, lse2 and D of 64 rows
constexpr int kBwdDkvLds = 2 * kBwdBuf;

__global__ void __launch_bounds__(128, 1) prefill_bwd_dkv_kernel(PrefillBwdLaunch a) {
    extern __shared__ __align__(16) char lds[];
    const int G = a.Hq / a.Hkv;
    const int nb = a.T / kPBlk;
    const int units = a.B * a.Hkv;
    // key-block major: the blocks that most query blocks choose (low j) start first, and with
    // eight KV heads each XCD keeps one head's queries in its L2
    const int j = blockIdx.x / units;
    const int unit = blockIdx.x % units;
    const int b = unit / a.Hkv, kv = unit % a.Hkv;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int h = lane >> 5, c32 = lane & 31;

    // K^T and V^T operands of this lane's key row (kept for the whole kernel)
    const size_t kfirst = (size_t)unit * a.T + (size_t)j * kPBlk + 32 * w;
    bf16x8 kf[8], vf[8];
    {
        const uint16_t* kp = a.k + (kfirst + c32) * kPD + 8 * h;
        const uint16_t* vp = a.v + (kfirst + c32) * kPD + 8 * h;
#pragma unroll
        for (int kd = 0; kd < 8; ++kd) {
            kf[kd] = *reinterpret_cast<const bf16x8*>(kp + 16 * kd);
            vf[kd] = *reinterpret_cast<const bf16x8*>(vp + 16 * kd);
        }
    }
    const int qoff0 = c32 * 64 + (((0 + h) ^ swz_v(c32)) << 4);
    const int qoff1 = c32 * 64 + (((2 + h) ^ swz_v(c32)) << 4);
    const int toff = tr_offset(lane);
    const size_t lrow = (size_t)unit * nb + j;
    const int nlist = 1 + a.inv_n[lrow];     // the diagonal block, then the choosers
    const int nitems = G * nlist;             // (head, query block) pairs, head-major
    const float cs = a.sigma * kLog2e;
    const int key = 32 * w + c32;             // this lane's key row within block j
    // Tile slot c * 128 + tid (c < 8) of a 64-row block: sub-tile c / 2, row 32 (c % 2) +
    // tid / 4, stored unit tid % 4 holding source unit (tid % 4) ^ swz_v(row), swz_v(row) =
    // (tid >> 2) & 2; thread tid's source offset is the same for every c but for the row and
    // sub-tile terms.
    const int src_t = (tid >> 2) * kPD * 2 + (((tid & 3) ^ ((tid >> 2) & 2)) << 4);

    // (head, query block) pair it: head it / nlist; query block j itself first, then the
    // choosers of j in ascending order
#define TCS_BWD_ITEM(it, i, bias, qrow0)                                                        \
    do {                                                                                        \
        const int hd_ = (it) / nlist, t_ = (it) - hd_ * nlist;                                  \
        i = t_ == 0 ? j : a.inv_i[lrow * nb + t_ - 1];                                          \
        bias = t_ == 0 ? 0.f : a.inv_g[lrow * nb + t_ - 1] * kLog2e;                            \
        qrow0 = (size_t)(b * a.Hq + kv * G + hd_) * a.T + (size_t)i * kPBlk;                    \
    } while (0)
    // staged copy of a pair's Q and dO tiles (8 + 8 chunks of 16 B per thread) and of its
    // rows' lse2 (threads 0..63) or D (threads 64..127)
#define TCS_BWD_LOAD(qrow0)                                                                     \
    do {                                                                                        \
        const char* qs_ = reinterpret_cast<const char*>(a.q + (qrow0) * kPD) + src_t;           \
        const char* gs_ = reinterpret_cast<const char*>(a.dout + (qrow0) * kPD) + src_t;        \
        xq0 = *reinterpret_cast<const uint4*>(qs_ + 0 * 8192 + 0 * 64);                         \
        xq1 = *reinterpret_cast<const uint4*>(qs_ + 1 * 8192 + 0 * 64);                         \
        xq2 = *reinterpret_cast<const uint4*>(qs_ + 0 * 8192 + 1 * 64);                         \
        xq3 = *reinterpret_cast<const uint4*>(qs_ + 1 * 8192 + 1 * 64);                         \
        xq4 = *reinterpret_cast<const uint4*>(qs_ + 0 * 8192 + 2 * 64);                         \
        xq5 = *reinterpret_cast<const uint4*>(qs_ + 1 * 8192 + 2 * 64);                         \
        xq6 = *reinterpret_cast<const uint4*>(qs_ + 0 * 8192 + 3 * 64);                         \
        xq7 = *reinterpret_cast<const uint4*>(qs_ + 1 * 8192 + 3 * 64);                         \
        xg0 = *reinterpret_cast<const uint4*>(gs_ + 0 * 8192 + 0 * 64);                         \
        xg1 = *reinterpret_cast<const uint4*>(gs_ + 1 * 8192 + 0 * 64);                         \
        xg2 = *reinterpret_cast<const uint4*>(gs_ + 0 * 8192 + 1 * 64);                         \
        xg3 = *reinterpret_cast<const uint4*>(gs_ + 1 * 8192 + 1 * 64);                         \
        xg4 = *reinterpret_cast<const uint4*>(gs_ + 0 * 8192 + 2 * 64);                         \
        xg5 = *reinterpret_cast<const uint4*>(gs_ + 1 * 8192 + 2 * 64);                         \
        xg6 = *reinterpret_cast<const uint4*>(gs_ + 0 * 8192 + 3 * 64);                         \
        xg7 = *reinterpret_cast<const uint4*>(gs_ + 1 * 8192 + 3 * 64);                         \
        xl = tid < 64 ? a.lse[(qrow0) + tid] * kLog2e : a.D[(qrow0) + tid - 64];                \
    } while (0)
#define TCS_BWD_STORE(buf)                                                                      \
    do {                                                                                        \
        char* d_ = (buf) + tid * 16;                                                            \
        *reinterpret_cast<uint4*>(d_ + 0 * 2048) = xq0;                                         \
        *reinterpret_cast<uint4*>(d_ + 1 * 2048) = xq1;                                         \
        *reinterpret_cast<uint4*>(d_ + 2 * 2048) = xq2;                                         \
        *reinterpret_cast<uint4*>(d_ + 3 * 2048) = xq3;                                         \
        *reinterpret_cast<uint4*>(d_ + 4 * 2048) = xq4;                                         \
        *reinterpret_cast<uint4*>(d_ + 5 * 2048) = xq5;                                         \
        *reinterpret_cast<uint4*>(d_ + 6 * 2048) = xq6;                                         \
        *reinterpret_cast<uint4*>(d_ + 7 * 2048) = xq7;                                         \
        *reinterpret_cast<uint4*>(d_ + kPTile + 0 * 2048) = xg0;                                \
        *reinterpret_cast<uint4*>(d_ + kPTile + 1 * 2048) = xg1;                                \
        *reinterpret_cast<uint4*>(d_ + kPTile + 2 * 2048) = xg2;                                \
        *reinterpret_cast<uint4*>(d_ + kPTile + 3 * 2048) = xg3;                                \
        *reinterpret_cast<uint4*>(d_ + kPTile + 4 * 2048) = xg4;                                \
        *reinterpret_cast<uint4*>(d_ + kPTile + 5 * 2048) = xg5;                                \
        *reinterpret_cast<uint4*>(d_ + kPTile + 6 * 2048) = xg6;                                \
        *reinterpret_cast<uint4*>(d_ + kPTile + 7 * 2048) = xg7;                                \
        reinterpret_cast<float*>((buf) + 2 * kPTile)[tid] = xl;                                 \
    } while (0)
    uint4 xq0, xq1, xq2, xq3, xq4, xq5, xq6, xq7, xg0, xg1, xg2, xg3, xg4, xg5, xg6, xg7;
    float xl;   // thread < 64: lse2 of row tid; thread >= 64: D of row tid - 64

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dk[dt] = dv[dt] = f32x16{};

    int i_cur;
    float bias_cur;
    size_t qrow_cur;
    TCS_BWD_ITEM(0, i_cur, bias_cur, qrow_cur);
    TCS_BWD_LOAD(qrow_cur);
    TCS_BWD_STORE(lds);
    wait_vmem();
    for (int it = 0; it < nitems; ++it) {
        __syncthreads();   // buffer it & 1 is filled; both waves are done with the other one
        const char* qt = lds + (it & 1) * kBwdBuf;
        const char* gt = qt + kPTile;
        const float* l2 = reinterpret_cast<const float*>(gt + kPTile);
        const float* Dl = l2 + kPBlk;
        const bool diag = i_cur == j;
        const float bias = bias_cur;
        int i_nx = 0;
        float bias_nx = 0.f;
        size_t qrow_nx = 0;
        if (it + 1 < nitems) {
            TCS_BWD_ITEM(it + 1, i_nx, bias_nx, qrow_nx);
            TCS_BWD_LOAD(qrow_nx);
        }

        f32x16 s[2], dp[2];
        s[0] = s[1] = dp[0] = dp[1] = f32x16{};
        qk_product<2>(qt, qoff0, qoff1, kf, s);    // S = Q K^T (lane: key; rows: queries)
        qk_product<2>(gt, qoff0, qoff1, vf, dp);   // dP = dO V^T
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int q0 = 32 * x + 8 * e4 + 4 * h;   // query rows q0 .. q0 + 3
                const float4 lq = *reinterpret_cast<const float4*>(l2 + q0);
                const float4 dd = *reinterpret_cast<const float4*>(Dl + q0);
                const float lv[4] = {lq.x, lq.y, lq.z, lq.w};
                const float dv4[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int e = 4 * e4 + jj;
                    float p = __builtin_amdgcn_exp2f(s[x][e] * cs + bias - lv[jj]);
                    if (diag && key > q0 + jj) p = 0.f;   // diagonal block: token-causal
                    s[x][e] = p;
                    dp[x][e] = p * (dp[x][e] - dv4[jj]);
                }
            }
        // dV^T += dO^T P and dK^T += Q^T dS over the block's queries (16 per step)
        const char* gtT = gt + toff;
        const char* qtT = qt + toff;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            bf16x8 pb, db;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pb[e] = (__bf16)s[st >> 1][8 * (st & 1) + e];
                db[e] = (__bf16)dp[st >> 1][8 * (st & 1) + e];
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(gtT, dt, st), pb,
                                                                 dv[dt], 0, 0, 0);
                dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(qtT, dt, st), db,
                                                                 dk[dt], 0, 0, 0);
            }
        }
        if (it + 1 < nitems) {
            TCS_BWD_STORE(lds + ((it + 1) & 1) * kBwdBuf);
            i_cur = i_nx;
            bias_cur = bias_nx;
            qrow_cur = qrow_nx;
        }
    }

    // this wave's 32 key rows: dK = sigma dK^T, dV = dV^T (lane: key row; registers: dims)
    float* kp = a.dk + (kfirst + c32) * kPD;
    float* vp = a.dv + (kfirst + c32) * kPD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            float4 x, y;
            x.x = dk[dt][4 * e4 + 0] * a.sigma; x.y = dk[dt][4 * e4 + 1] * a.sigma;
            x.z = dk[dt][4 * e4 + 2] * a.sigma; x.w = dk[dt][4 * e4 + 3] * a.sigma;
            y.x = dv[dt][4 * e4 + 0]; y.y = dv[dt][4 * e4 + 1];
            y.z = dv[dt][4 * e4 + 2]; y.w = dv[dt][4 * e4 + 3];
            *reinterpret_cast<float4*>(kp + 32 * dt + 8 * e4 + 4 * h) = x;
            *reinterpret_cast<float4*>(vp + 32 * dt + 8 * e4 + 4 * h) = y;
        }
#undef TCS_BWD_ITEM
#undef TCS_BWD_LOAD
#undef TCS_BWD_STORE
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

hipError_t launch_prefill_bwd_prep(const PrefillBwdLaunch& a, hipStream_t s) {
    hipError_t e = bwd_check(a);
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.B * a.Hq * a.T;
    const long long g1 = (rows * 16 + 255) / 256;
    const long long g2 = (long long)a.B * a.Hkv * (a.T / kPBlk);
    if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return hipErrorNotSupported;
    if (g1 > 0) prefill_bwd_prep_kernel<<<(unsigned)g1, 256, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (g2 > 0) prefill_bwd_inverse_kernel<<<(unsigned)g2, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_prefill_bwd_dq(const PrefillBwdLaunch& a, hipStream_t s) {
    hipError_t e = bwd_check(a);
    if (e != hipSuccess) return e;
    const int G = a.Hq / a.Hkv;
    const long long W = 2LL * a.B * a.Hkv * (a.T / kPBlk) * ((G + 3) / 4);
    if (W <= 0) return hipSuccess;
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    e = hipFuncSetAttribute((const void*)prefill_bwd_dq_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kPLdsAll);
    if (e != hipSuccess) return e;
    prefill_bwd_dq_kernel<<<(unsigned)W, 256, kPLdsAll, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_prefill_bwd_dkv(const PrefillBwdLaunch& a, hipStream_t s) {
    hipError_t e = bwd_check(a);
    if (e != hipSuccess) return e;
    const long long W = (long long)a.B * a.Hkv * (a.T / kPBlk);
    if (W <= 0) return hipSuccess;
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    e = hipFuncSetAttribute((const void*)prefill_bwd_dkv_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kBwdDkvLds);
    if (e != hipSuccess) return e;
    prefill_bwd_dkv_kernel<<<(unsigned)W, 128, kBwdDkvLds, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_prefill_bwd_ds(const PrefillBwdLaunch& a, hipStream_t s) {
    hipError_t e = bwd_check(a);
    if (e != hipSuccess || !a.dS) return e;
    const long long W = (long long)a.B * a.Hkv * (a.T / kPBlk);
    if (W <= 0) return hipSuccess;
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    prefill_bwd_ds_kernel<<<(unsigned)W, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace tcs
