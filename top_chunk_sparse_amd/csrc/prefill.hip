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
// Workgroup: 4 waves, wave w owns query head 4*hg + w of the KV group and the 64 rows of query
// block i.  All products use v_mfma_f32_32x32x16_bf16 (A: 32x16, lane l holds row l%32,
// k = 8*(l/32)..+7; B: 16x32, lane l holds column l%32, same k; D: 32x32, lane l holds
// column l%32, rows 8*i + 4*(l/32) + j in register 4*i + j).
//
//   S^T = K * Q^T   64 keys x 64 queries per wave: a lane owns whole query columns, so the
//                   running max / sum of a query row live in one lane pair (l, l ^ 32).
//   O^T += V^T P^T  128 dims x 64 queries: the B operand (P^T) is the S^T accumulator of the
//                   same lane, converted to bf16; the A operand (V^T) comes from row-major V
//                   in LDS through the transposing read ds_read_b64_tr_b16.
//
// K and V blocks (64 rows x 256 B) are copied straight into LDS (global_load_lds_dwordx4),
// double buffered: the next block's copy is in flight while the current one is consumed.  The
// 16-byte unit u of row r is stored at unit u ^ swz(r) so that both the K reads (8 rows per
// bank sweep) and the transposing V reads (4 rows x 32 B) are free of bank conflicts.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kPD = 128;                     // head dim
constexpr int kPBlk = 64;                    // block rows
constexpr int kPRow = kPD * 2;               // bytes per K / V row
constexpr int kPTile = kPBlk * kPRow;        // bytes per K or V block
constexpr int kPLds = 4 * kPTile;            // K0 K1 V0 V1
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;         // log2 units a stale running max may lag

__device__ __forceinline__ int swz_k(int r) { return r & 7; }
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 1; }

// Copy one block (64 rows x 128 bf16, rows contiguous) into an LDS tile.  Each wave issues 4
// instructions of 64 x 16 B; slot s of the tile is row s/16, stored unit s%16.
template <bool IS_V>
__device__ __forceinline__ void copy_block(const uint16_t* src, char* tile, int w, int lane) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int slot0 = (c * 4 + w) * 64;
        const int slot = slot0 + lane;
        const int r = slot >> 4;
        const int lu = (slot & 15) ^ (IS_V ? swz_v(r) : swz_k(r));
        __builtin_amdgcn_global_load_lds(src + r * kPD + lu * 8, (lds_void*)(tile + slot0 * 16),
                                         16, 0, 0);
    }
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__global__ void __launch_bounds__(256) prefill_fwd_kernel(PrefillLaunch a) {
    extern __shared__ __align__(16) char lds[];
    const int G = a.Hq / a.Hkv;
    const int nb = a.T / kPBlk;
    const int nhg = (G + 3) >> 2;
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous range of
    // (unit, head group, block) so one KV head's blocks stay in one L2.  Within a range the
    // query blocks run from last to first, the longest (most earlier blocks) first.
    int bid = blockIdx.x;
    const int W = gridDim.x;
    if ((W & 7) == 0) bid = (bid & 7) * (W >> 3) + (bid >> 3);
    const int i = nb - 1 - bid % nb;
    const int rest = bid / nb;
    const int hg = rest % nhg;
    const int unit = rest / nhg;
    const int b = unit / a.Hkv, kv = unit % a.Hkv;

    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int head = hg * 4 + w;
    const bool active = head < G;

    const uint16_t* kbase = a.k + (size_t)unit * a.T * kPD;
    const uint16_t* vbase = a.v + (size_t)unit * a.T * kPD;
    // LDS: K tiles at [0, 2 kPTile), V tiles at [2 kPTile, 4 kPTile).

    const int ke = a.ksel > 0 ? min(a.ksel, i) : 0;
    const int32_t* selrow = a.sel ? a.sel + ((size_t)unit * nb + i) * a.ksel : nullptr;
    const float* grow = a.gamma ? a.gamma + ((size_t)unit * nb + i) * a.ksel : nullptr;

    // Block 0 of the list is the diagonal block; blocks 1..ke are the chosen earlier ones.
    copy_block<false>(kbase + (size_t)i * kPBlk * kPD, lds, w, lane);
    copy_block<true>(vbase + (size_t)i * kPBlk * kPD, lds + 2 * kPTile, w, lane);

    // Q^T operand: q[qt][kd] = Q[32 qt + c32][16 kd + 8 h .. +7] of this wave's head.
    const size_t qrow0 = ((size_t)(b * a.Hq + kv * G + (active ? head : 0)) * a.T + (size_t)i * kPBlk);
    bf16x8 qf[2][8];
    {
        const uint16_t* qp = a.q + qrow0 * kPD;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int kd = 0; kd < 8; ++kd)
                qf[qt][kd] = *reinterpret_cast<const bf16x8*>(qp + (32 * qt + c32) * kPD + 16 * kd + 8 * h);
    }

    const float cs = a.sigma * kLog2e;
    f32x16 o[4][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) o[dt][qt] = f32x16{};
    float m[2] = {0.f, 0.f}, l[2] = {0.f, 0.f};

    int jn = 0;          // block of list entry t + 1
    float gn = 0.f;      // its gate (log2 units)
    if (ke > 0) {
        jn = min(max(selrow[0], 0), i - 1);
        gn = grow ? grow[0] * kLog2e : 0.f;
    }
    float gcur = 0.f;

    for (int t = 0; t <= ke; ++t) {
        wait_vmem();
        __syncthreads();
        const int buf = t & 1;
        if (t < ke) {
            copy_block<false>(kbase + (size_t)jn * kPBlk * kPD, lds + (buf ^ 1) * kPTile, w, lane);
            copy_block<true>(vbase + (size_t)jn * kPBlk * kPD, lds + (2 + (buf ^ 1)) * kPTile, w, lane);
        }
        const float bias = gcur;
        gcur = gn;
        if (t + 1 < ke) {
            jn = min(max(selrow[t + 1], 0), i - 1);
            gn = grow ? grow[t + 1] * kLog2e : 0.f;
        }
        if (!active) continue;

        // ---- S^T = K Q^T ----
        const char* kt = lds + buf * kPTile;
        f32x16 s[2][2];
#pragma unroll
        for (int x = 0; x < 2; ++x) s[x][0] = s[x][1] = f32x16{};
#pragma unroll
        for (int kd = 0; kd < 8; ++kd) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = 32 * x + c32;
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
                    kt + r * kPRow + (((2 * kd + h) ^ swz_k(r)) << 4));
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    s[x][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qt][kd], s[x][qt], 0, 0, 0);
            }
        }

        // ---- online softmax (log2 domain) ----
        if (t == 0) {   // diagonal block: key row r sees query column c only if r <= c
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = 32 * x + 8 * (e >> 2) + 4 * h + (e & 3);
                        if (key > 32 * qt + c32) s[x][qt][e] = -INFINITY;
                    }
        }
        float mb[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            float mx = s[0][qt][0];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[x][qt][e]);
            mx = fmaxf(mx, xor32(mx));
            mb[qt] = mx * cs + bias;
        }
        if (t == 0) {
            m[0] = mb[0];
            m[1] = mb[1];
        } else {
            const bool need = (mb[0] > m[0] + kRescaleSlack) || (mb[1] > m[1] + kRescaleSlack);
            if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const float mn = fmaxf(m[qt], mb[qt]);
                    const float al = __builtin_amdgcn_exp2f(m[qt] - mn);
                    m[qt] = mn;
                    l[qt] *= al;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) o[dt][qt] *= al;
                }
            }
        }
        bf16x8 p[4][2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const float off = bias - m[qt];
            float sum = 0.f;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    bf16x8 pv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pe = __builtin_amdgcn_exp2f(s[x][qt][8 * hf + e] * cs + off);
                        sum += pe;
                        pv[e] = (__bf16)pe;
                    }
                    p[2 * x + hf][qt] = pv;
                }
            l[qt] += sum;
        }

        // ---- O^T += V^T P^T ----
        const char* vt = lds + (2 + buf) * kPTile;
        const int g = lane >> 4, L = lane & 15;
        const int rr = L >> 2, cc = L & 3;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                s16x4 part[2];
#pragma unroll
                for (int rho = 0; rho < 2; ++rho) {
                    const int r = 16 * st + 8 * rho + 4 * h + rr;
                    const int lu = 4 * dt + 2 * (g & 1) + (cc >> 1);
                    const char* ap = vt + r * kPRow + ((lu ^ swz_v(r)) << 4) + ((cc & 1) << 3);
                    part[rho] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)ap);
                }
                const s16x8 va16 = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
                const bf16x8 va = __builtin_bit_cast(bf16x8, va16);
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[st][qt], o[dt][qt], 0, 0, 0);
            }
        }
    }
    if (!active) return;

    // ---- epilogue: O = O^T / l, lse = m + log2 l (back to natural log) ----
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const float lt = l[qt] + xor32(l[qt]);
        const float inv = 1.f / lt;
        const size_t row = qrow0 + 32 * qt + c32;
        float* op = a.out + row * kPD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                float4 v;
                v.x = o[dt][qt][4 * e4 + 0] * inv;
                v.y = o[dt][qt][4 * e4 + 1] * inv;
                v.z = o[dt][qt][4 * e4 + 2] * inv;
                v.w = o[dt][qt][4 * e4 + 3] * inv;
                *reinterpret_cast<float4*>(op + 32 * dt + 8 * e4 + 4 * h) = v;
            }
        if (a.lse && h == 0) a.lse[row] = (m[qt] + log2f(lt)) * kLn2;
    }
}

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t s) {
    if (a.d != kPD || a.blk != kPBlk || a.T % kPBlk) return hipErrorNotSupported;
    const int G = a.Hq / a.Hkv;
    const long long W = (long long)a.B * a.Hkv * (a.T / kPBlk) * ((G + 3) / 4);
    if (W <= 0) return hipSuccess;
    if (W > 0x7fffffffLL) return hipErrorNotSupported;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_fwd_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kPLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    prefill_fwd_kernel<<<(unsigned)W, 256, kPLds, s>>>(a);
    return hipGetLastError();
}

}  // namespace tcs
