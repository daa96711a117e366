// mfma_tiles.hpp -- the bf16 MFMA tile machinery shared by the prefill kernels (forward,
// backward, SSA gist-masked prefill): 64-row K / V tiles in LDS with their swizzles, the
// staged global -> register -> LDS copy, the operand reads (row-major and transposing), the
// S^T = K Q^T product and the lane-pair reductions.  The layout itself is described with the
// forward kernel (prefill.hip).  Internal; not part of the ABI.
#pragma once
#include "device.hpp"

namespace tcs {

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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// s_waitcnt lgkmcnt(0) with vmcnt / expcnt left free (gfx9 encoding)
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Per-lane LDS offset of the transposing operand reads (the forward's V^T pattern) in a tile
// stored in the transposable layout.
__device__ __forceinline__ int tr_offset(int lane) {
    const int h = lane >> 5, g = lane >> 4, L = lane & 15, rr = L >> 2, cc = L & 3;
    return (4 * h + rr) * 64 + (((2 * (g & 1) + (cc >> 1)) ^ swz_v(rr)) << 4) + ((cc & 1) << 3);
}

}  // namespace tcs
