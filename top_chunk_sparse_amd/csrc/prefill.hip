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
    const int ke = block_topk(
        i, a.k, [&](int j) { return s[j]; },
        [&](int x, int j) {
            sel[x] = j;
            if (gam) gam[x] = s[j] - lse;
        },
        sm);
    for (int x = ke + threadIdx.x; x < a.k; x += 256) {
        sel[x] = -1;
        if (gam) gam[x] = 0.f;
    }
}

hipError_t launch_prefill_select(const PrefillSelectLaunch& a, hipStream_t s) {
    if (a.units <= 0 || a.nb <= 0 || a.k <= 0) return hipSuccess;
    prefill_select_kernel<<<a.units * a.nb, 256, 0, s>>>(a);
    return hipGetLastError();
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
// distinct banks.  Blocks are double buffered: the next block's global loads are issued into
// registers at the top of an iteration and written to the other LDS buffer at its end.  (A
// direct global-to-LDS copy would save those registers, but the compiler then cannot count
// LDS reads precisely and makes every operand read wait for all earlier ones.)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kPD = 128;                     // head dim
constexpr int kPBlk = 64;                    // block rows
constexpr int kPSub = 64 * 64;               // bytes per 32-dim sub-tile (64 rows x 64 B)
constexpr int kPTile = 4 * kPSub;            // bytes per K or V block
constexpr int kRing = 128;                   // entries of the chosen-block ring (power of 2)
constexpr int kPLds = 4 * kPTile;            // K0 K1 V0 V1
constexpr int kPLdsAll = kPLds + kRing * 8;  // + the ring (block ids, gates)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;         // log2 units a stale running max may lag

__device__ __forceinline__ int swz_k(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_v(int r) { return r & 2; }

// Copy one block (64 rows x 128 bf16, rows contiguous in global memory) into an LDS tile.
// Slot s (16 B) of the tile is sub-tile s / 256, row (s / 4) % 64, stored unit s % 4.  Wave w
// issues instruction c for slots (4 c + w) * 64 + lane, i.e. sub-tile c, row 16 w + lane / 4,
// so a lane's source offset is the same for all four instructions but for c * 64 bytes.
struct CopyOffsets { uint32_t c[4]; };   // per-lane source byte offsets, one per chunk

// A block (64 rows x 128 bf16, rows contiguous in global memory) is copied through registers:
// each thread moves four 16-byte chunks of K and four of V.  Chunk c of wave w is tile slot
// s = (4 c + w) * 64 + lane: sub-tile c, row 16 w + lane / 4, stored unit lane % 4, so the
// LDS writes of one instruction are 1 KB contiguous and a lane's source offsets differ only by
// c * 64 bytes.
__device__ __forceinline__ CopyOffsets copy_offsets(bool is_v, int w, int lane) {
    const int r = 16 * w + (lane >> 2);
    const int lu = (lane & 3) ^ (is_v ? swz_v(r) : swz_k(r));
    CopyOffsets o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o.c[c] = (uint32_t)(r * kPD * 2 + c * 64 + lu * 16);
    return o;
}

// Staged copy of one block: eight 16-byte chunks per thread, held in named registers.
#define TCS_STAGE_LOAD(kb, vb)                                                                  \
    do {                                                                                        \
        const char* kc_ = reinterpret_cast<const char*>(kb);                                    \
        const char* vc_ = reinterpret_cast<const char*>(vb);                                    \
        sk0 = *reinterpret_cast<const uint4*>(kc_ + gk.c[0]);                                   \
        sk1 = *reinterpret_cast<const uint4*>(kc_ + gk.c[1]);                                   \
        sk2 = *reinterpret_cast<const uint4*>(kc_ + gk.c[2]);                                   \
        sk3 = *reinterpret_cast<const uint4*>(kc_ + gk.c[3]);                                   \
        sv0 = *reinterpret_cast<const uint4*>(vc_ + gv.c[0]);                                   \
        sv1 = *reinterpret_cast<const uint4*>(vc_ + gv.c[1]);                                   \
        sv2 = *reinterpret_cast<const uint4*>(vc_ + gv.c[2]);                                   \
        sv3 = *reinterpret_cast<const uint4*>(vc_ + gv.c[3]);                                   \
    } while (0)
#define TCS_STAGE_STORE(ktile, vtile)                                                           \
    do {                                                                                        \
        char* kd_ = (ktile) + w * 1024 + lane * 16;                                             \
        char* vd_ = (vtile) + w * 1024 + lane * 16;                                             \
        *reinterpret_cast<uint4*>(kd_ + 0 * 4096) = sk0;                                        \
        *reinterpret_cast<uint4*>(kd_ + 1 * 4096) = sk1;                                        \
        *reinterpret_cast<uint4*>(kd_ + 2 * 4096) = sk2;                                        \
        *reinterpret_cast<uint4*>(kd_ + 3 * 4096) = sk3;                                        \
        *reinterpret_cast<uint4*>(vd_ + 0 * 4096) = sv0;                                        \
        *reinterpret_cast<uint4*>(vd_ + 1 * 4096) = sv1;                                        \
        *reinterpret_cast<uint4*>(vd_ + 2 * 4096) = sv2;                                        \
        *reinterpret_cast<uint4*>(vd_ + 3 * 4096) = sv3;                                        \
    } while (0)

// max / sum of a value over the lane pair (l, l ^ 32), identical in both lanes: one
// v_permlane32_swap exchanges the two 32-lane halves.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// V^T operand of (dim tile dt, key step st): two transposing reads of 4 rows each.
__device__ __forceinline__ bf16x8 v_operand(const char* vt, int dt, int st) {
    const char* ap = vt + dt * kPSub + st * 1024;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)ap);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ap + 512));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S^T (keys NX * 32 x 32 queries) = K Q^T from the K tile kt.  Eight operand reads ahead,
// then one read per product, so each product waits only for its own operand.
template <int NX>
__device__ __forceinline__ void qk_product(const char* kt, int koff0, int koff1,
                                           const bf16x8 (&qf)[8], f32x16 (&s)[2]) {
    bf16x8 kr[8][NX];
#pragma unroll
    for (int kd = 0; kd < 8; ++kd)
#pragma unroll
        for (int x = 0; x < NX; ++x)
            kr[kd][x] = *reinterpret_cast<const bf16x8*>(
                kt + (kd >> 1) * kPSub + ((kd & 1) ? koff1 : koff0) + x * 32 * 64);
#pragma unroll
    for (int kd = 0; kd < 8; ++kd)
#pragma unroll
        for (int x = 0; x < NX; ++x)
            s[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[kd][x], qf[kd], s[x], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int x = 0; x < 8 * NX - 8; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
}

__global__ void __launch_bounds__(256, 2) prefill_fwd_kernel(PrefillLaunch a) {
    extern __shared__ __align__(16) char lds[];
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
    // LDS: K tiles at [0, 2 kPTile), V tiles at [2 kPTile, 4 kPTile), then the ring.

    const int ke = a.ksel > 0 ? min(a.ksel, i) : 0;
    const int32_t* selrow = a.sel ? a.sel + ((size_t)unit * nb + i) * a.ksel : nullptr;
    const float* grow = a.gamma ? a.gamma + ((size_t)unit * nb + i) * a.ksel : nullptr;

    // The chosen blocks and their gates pass through a ring of kRing entries in LDS, refilled
    // kRing / 2 entries at a time well ahead of use.
    int* ring_j = reinterpret_cast<int*>(lds + kPLds);
    float* ring_g = reinterpret_cast<float*>(lds + kPLds + kRing * 4);
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
    const CopyOffsets gk = copy_offsets(false, w, lane), gv = copy_offsets(true, w, lane);
    uint4 sk0, sk1, sk2, sk3, sv0, sv1, sv2, sv3;
    TCS_STAGE_LOAD(kbase + (size_t)i * kPBlk * kPD, vbase + (size_t)i * kPBlk * kPD);

    // Q^T operand: qf[kd] = Q[32 rh + c32][16 kd + 8 h .. +7] of this wave's head.
    const size_t qrow = ((size_t)(b * a.Hq + kv * G + (active ? head : 0)) * a.T +
                         (size_t)i * kPBlk + 32 * rh + c32);
    bf16x8 qf[8];
    {
        const uint16_t* qp = a.q + qrow * kPD + 8 * h;
#pragma unroll
        for (int kd = 0; kd < 8; ++kd) qf[kd] = *reinterpret_cast<const bf16x8*>(qp + 16 * kd);
    }
    TCS_STAGE_STORE(lds, lds + 2 * kPTile);

    // Per-lane LDS offsets (bytes) of the operand reads; everything else is an immediate.
    //   K: row r = 32 x + c32, d = 16 kd + 8 h: sub-tile kd / 2, unit (2 (kd & 1) + h) ^ swz.
    const int koff0 = c32 * 64 + (((0 + h) ^ swz_k(c32)) << 4);
    const int koff1 = c32 * 64 + (((2 + h) ^ swz_k(c32)) << 4);
    //   V (transposing read, 16-lane group g, lane L = 4 rr + cc of the group): row
    //   16 st + 8 rho + 4 h + rr, sub-tile dt, unit (2 (g & 1) + (cc >> 1)) ^ swz, half cc & 1.
    const int g = lane >> 4, L = lane & 15, rr = L >> 2, cc = L & 3;
    const int voff = (4 * h + rr) * 64 + (((2 * (g & 1) + (cc >> 1)) ^ swz_v(rr)) << 4) + ((cc & 1) << 3);

    // The query operands must have landed before the loop: otherwise the compiler's wait
    // counting at the loop head cannot tell them from the next block's loads and makes every
    // iteration's first products wait for that block's global loads.
    wait_vmem();

    const float cs = a.sigma * kLog2e;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m = 0.f, l = 0.f;
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

    for (int t = 0; t <= ke; ++t) {
        // Block t is in buffer t & 1; every wave is done with buffer (t + 1) & 1.
        __syncthreads();
        const int buf = t & 1;
        const float bias = t > 0 ? __int_as_float(__builtin_amdgcn_readfirstlane(
                                       __float_as_int(ring_g[(t - 1) & (kRing - 1)])))
                                 : 0.f;
        if (t < ke) {
            const int jn = __builtin_amdgcn_readfirstlane(ring_j[t & (kRing - 1)]);
            TCS_STAGE_LOAD(kbase + (size_t)jn * kPBlk * kPD, vbase + (size_t)jn * kPBlk * kPD);
        }
        // Iteration t reads entries t - 1 and t.  Past this iteration's barrier every entry
        // below t is dead, so at t = 1 + n kRing/2 (n >= 1) the slots of entries
        // t - 1 - kRing/2 .. t - 2 take entries t - 1 + kRing/2 .. t - 2 + kRing, first read
        // kRing/2 - 1 iterations later.
        if (t > kRing / 2 && ((t - 1) & (kRing / 2 - 1)) == 0 && t - 1 + kRing / 2 < ke)
            fill_ring(t - 1 + kRing / 2);
        if (active) {
            // On the diagonal block, rows of the first half see only keys 0..31.
            const bool half = (t == 0) && rh == 0;
            const char* kt = lds + buf * kPTile;
            const char* vt = lds + (2 + buf) * kPTile + voff;

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
            if (t == 0) {   // diagonal block: key row r sees query row q only if r <= q
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
            if (t == 0) {
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
        if (t < ke) TCS_STAGE_STORE(lds + (buf ^ 1) * kPTile, lds + (2 + (buf ^ 1)) * kPTile);
    }
    if (!active) return;

    // ---- epilogue: O = O^T / l, lse = m + log2 l (back to natural log) ----
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

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t s) {
    if (a.d != kPD || a.blk != kPBlk || a.T % kPBlk) return hipErrorNotSupported;
    const int G = a.Hq / a.Hkv;
    const long long W = 2LL * a.B * a.Hkv * (a.T / kPBlk) * ((G + 3) / 4);
    if (W <= 0) return hipSuccess;
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    // the dynamic LDS (tiles + ring) is above the 64 KB default limit; set on every call (no
    // library state, and it holds for whichever device is current)
    const hipError_t e = hipFuncSetAttribute((const void*)prefill_fwd_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kPLdsAll);
    if (e != hipSuccess) return e;
    prefill_fwd_kernel<<<(unsigned)W, 256, kPLdsAll, s>>>(a);
    return hipGetLastError();
}

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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// s_waitcnt lgkmcnt(0) with vmcnt / expcnt left free (gfx9 encoding)
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

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

// Per-lane LDS offset of the transposing operand reads (the forward's V^T pattern) in a tile
// stored in the transposable layout.
__device__ __forceinline__ int tr_offset(int lane) {
    const int h = lane >> 5, g = lane >> 4, L = lane & 15, rr = L >> 2, cc = L & 3;
    return (4 * h + rr) * 64 + (((2 * (g & 1) + (cc >> 1)) ^ swz_v(rr)) << 4) + ((cc & 1) << 3);
}

__global__ void __launch_bounds__(256, 1) prefill_bwd_dq_kernel(PrefillBwdLaunch a) {
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
    bf16x8 qf[8], gf[8];   // Q^T and dO^T operands of this lane's query row
    {
        const uint16_t* qp = a.q + qrow * kPD + 8 * h;
        const uint16_t* gp = a.dout + qrow * kPD + 8 * h;
#pragma unroll
        for (int kd = 0; kd < 8; ++kd) {
            qf[kd] = *reinterpret_cast<const bf16x8*>(qp + 16 * kd);
            gf[kd] = *reinterpret_cast<const bf16x8*>(gp + 16 * kd);
        }
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

template <bool GROWS>
__global__ void __launch_bounds__(256, 2) gist_prefill_mfma_kernel(GistPrefillLaunch a) {
    extern __shared__ __align__(16) char lds[];
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
    int bid = blockIdx.x;
    const int Wg = gridDim.x;
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

    const CopyOffsets gk = copy_offsets(false, w, lane), gv = copy_offsets(true, w, lane);
    uint4 sk0, sk1, sk2, sk3, sv0, sv1, sv2, sv3;
    TCS_STAGE_LOAD(kblock(0), vblock(0));

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
    {
        const uint16_t* qp = a.q + qrow * kPD + 8 * h;
#pragma unroll
        for (int kd = 0; kd < 8; ++kd) qf[kd] = *reinterpret_cast<const bf16x8*>(qp + 16 * kd);
    }
    TCS_STAGE_STORE(lds, lds + 2 * kPTile);

    const int koff0 = c32 * 64 + (((0 + h) ^ swz_k(c32)) << 4);
    const int koff1 = c32 * 64 + (((2 + h) ^ swz_k(c32)) << 4);
    const int g16 = lane >> 4, L16 = lane & 15, rr = L16 >> 2, cc = L16 & 3;
    const int voff = (4 * h + rr) * 64 + (((2 * (g16 & 1) + (cc >> 1)) ^ swz_v(rr)) << 4) +
                     ((cc & 1) << 3);
    wait_vmem();

    const float cs = a.sigma * kLog2e;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m = 0.f, l = 0.f;
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

    for (int t = 0; t < nblk; ++t) {
        __syncthreads();
        const int buf = t & 1;
        if (t + 1 < nblk) TCS_STAGE_LOAD(kblock(t + 1), vblock(t + 1));
        if (active) {
            const bool half = !GROWS && (t == 0) && rh == 0;
            const int cut = (!GROWS && t == nblk - 1 && t > rb) ? last_valid : kPBlk;
            const char* kt = lds + buf * kPTile;
            const char* vt = lds + (2 + buf) * kPTile + voff;
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
                        if ((t == 0 && key > q) || key >= cut) s[x][e] = -INFINITY;
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
            if (t == 0) {
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
        if (t + 1 < nblk) TCS_STAGE_STORE(lds + (buf ^ 1) * kPTile, lds + (2 + (buf ^ 1)) * kPTile);
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

static hipError_t gist_check(const GistPrefillLaunch& a) {
    if (a.d != kPD || a.L % kPBlk || a.g < 1 || a.g > kPBlk || kPBlk % a.g || a.Hkv <= 0 ||
        a.Hq % a.Hkv || a.Gp % kPBlk || a.Gp < a.M * a.g)
        return hipErrorNotSupported;
    return hipSuccess;
}

hipError_t launch_gist_gather(const GistPrefillLaunch& a, hipStream_t s) {
    hipError_t e = gist_check(a);
    if (e != hipSuccess) return e;
    const long long W = (long long)a.B * a.Hkv * (a.Gp / kPBlk);
    if (W <= 0) return hipSuccess;
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    gist_gather_kernel<<<(unsigned)W, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_gist_prefill_raw(const GistPrefillLaunch& a, hipStream_t s) {
    hipError_t e = gist_check(a);
    if (e != hipSuccess) return e;
    const int G = a.Hq / a.Hkv;
    const long long W = 2LL * a.B * a.Hkv * a.M * (a.L / kPBlk) * ((G + 3) / 4);
    if (W <= 0) return hipSuccess;
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    e = hipFuncSetAttribute((const void*)gist_prefill_mfma_kernel<false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kPLds);
    if (e != hipSuccess) return e;
    gist_prefill_mfma_kernel<false><<<(unsigned)W, 256, kPLds, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_gist_prefill_gists(const GistPrefillLaunch& a, hipStream_t s) {
    hipError_t e = gist_check(a);
    if (e != hipSuccess) return e;
    const int G = a.Hq / a.Hkv;
    const long long W = 2LL * a.B * a.Hkv * (a.Gp / kPBlk) * ((G + 3) / 4);
    if (W <= 0) return hipSuccess;
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    e = hipFuncSetAttribute((const void*)gist_prefill_mfma_kernel<true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kPLds);
    if (e != hipSuccess) return e;
    gist_prefill_mfma_kernel<true><<<(unsigned)W, 256, kPLds, s>>>(a);
    return hipGetLastError();
}

}  // namespace tcs
