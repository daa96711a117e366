// device.hpp -- gfx950 device helpers shared by the decode and prefill kernels:
// bf16 unpacking, DPP row reductions, order-preserving float keys, block-wide scans and the
// deterministic top-k used for chunk / block selection.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tcs {

constexpr int kWave = 64;

// ---- bf16 -------------------------------------------------------------------------------
// A dword holds two bf16 values; each is the upper half of an fp32.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

#ifndef TCS_NT_LOADS
#define TCS_NT_LOADS 1   // stream K/V rows with non-temporal loads (read once)
#endif

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
#if TCS_NT_LOADS
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *reinterpret_cast<const uint4*>(p);
#endif
}

// ---- DPP ----------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR (8 or 16) lanes; every lane of a group receives the same,
// bitwise-identical sum (each step adds a lane's value to its partner's, a commutative pair).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LPR == 8 || LPR == 16, "LPR");
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: partner lane ^ 1
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: partner lane ^ 2
    x += dpp<0x141>(x);   // row_half_mirror: the other quad of the 8-lane half
    if constexpr (LPR == 16) x += dpp<0x140>(x);  // row_mirror: the other half of the row
    return x;
}

// Sum over the lanes l, l + LPR, l + 2 LPR, ... of a wave (the same position in every
// LPR-lane group); every such lane receives the same bits.  Steps: lanes l ^ 8 (LPR = 8;
// DPP row_ror:8 swaps the halves of a 16-lane row), then l ^ 16 and l ^ 32 (v_permlane16_swap
// and v_permlane32_swap, whose two results are the lower lane's value, then the upper one's).
template <int LPR>
__device__ __forceinline__ float lane_groups_sum(float x) {
    static_assert(LPR == 8 || LPR == 16, "LPR");
    if constexpr (LPR == 8) x += dpp<0x128>(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- ordered keys -----------------------------------------------------------------------
// Monotone map fp32 -> uint32 (a < b  <=>  key(a) < key(b)); -0 is folded onto +0.
__device__ __forceinline__ uint32_t ordered_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- block scans (blockDim.x == 256) ------------------------------------------------------
struct ScanSmem { int w[4]; };

// Inclusive prefix sum over the 64 lanes of a wave, all lanes active: DPP row shifts by 1, 2,
// 4 and 8 lanes within each 16-lane row (lanes shifted in from outside the row add 0), then
// row_bcast:15 adds the last lane of rows 0 and 2 to rows 1 and 3, and row_bcast:31 the last
// lane of row 1 to rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return x;
}

__device__ __forceinline__ int block_exclusive_scan(int v, ScanSmem& sm) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int x = wave_inclusive_scan(v);
    if (lane == 63) sm.w[w] = x;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < w; ++i) before += sm.w[i];
    __syncthreads();
    return before + x - v;
}

struct ReduceSmem { float v[4]; };

// Whole-wave reductions: DPP steps within each 16-lane row (every lane of a row ends with
// the same bits: each step combines a lane with its partner, a commutative pair), then the
// four rows' values are read with readlane and combined in a fixed order.  All 64 lanes must
// be active.
__device__ __forceinline__ float lane_value(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)),
                 fmaxf(lane_value(x, 32), lane_value(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}
// Fixed-order block reductions (deterministic).  Every thread gets the result.
__device__ __forceinline__ float block_max(float x, ReduceSmem& sm) {
    x = wave_max(x);
    if ((threadIdx.x & 63) == 0) sm.v[threadIdx.x >> 6] = x;
    __syncthreads();
    float r = fmaxf(fmaxf(sm.v[0], sm.v[1]), fmaxf(sm.v[2], sm.v[3]));
    __syncthreads();
    return r;
}
__device__ __forceinline__ float block_sum(float x, ReduceSmem& sm) {
    x = wave_sum(x);
    if ((threadIdx.x & 63) == 0) sm.v[threadIdx.x >> 6] = x;
    __syncthreads();
    float r = (sm.v[0] + sm.v[1]) + (sm.v[2] + sm.v[3]);
    __syncthreads();
    return r;
}

// ---- deterministic block top-k ------------------------------------------------------------
// Chooses the min(k, n) largest of n fp32 scores, equal scores going to the lower position,
// and writes the chosen positions in ascending order.  Radix select on the ordered 32-bit
// key finds the threshold key T (the k_eff-th largest); every key > T is taken, then the
// lowest positions holding T until k_eff are reached.  256 threads.
constexpr int kTopkCache = 4096;   // keys staged in LDS; larger n re-reads global memory

struct TopkSmem {
    unsigned hist[256];
    uint32_t keys[kTopkCache];
    int digit;
    unsigned above;
    uint32_t band[4], bor[4];
    ScanSmem scan;
};

// score(i) -> fp32 score of position i; emit(j, i) is called once for the j-th chosen position
// (j ascending with i).  Returns k_eff.
template <class ScoreFn, class EmitFn>
__device__ int block_topk(int n, int k, ScoreFn score, EmitFn emit, TopkSmem& sm) {
    const int tid = threadIdx.x;
    const int ke = k < n ? k : n;
    if (ke <= 0) return 0;
    const bool cached = n <= kTopkCache;
    if (cached)
        for (int i = tid; i < n; i += 256) sm.keys[i] = ordered_key(score(i));
    __syncthreads();
    auto key_at = [&](int i) -> uint32_t { return cached ? sm.keys[i] : ordered_key(score(i)); };

    // Bytes shared by every key need no histogram pass: start at the first byte that differs.
    uint32_t kand = 0xFFFFFFFFu, kor = 0u;
    for (int i = tid; i < n; i += 256) {
        const uint32_t key = key_at(i);
        kand &= key;
        kor |= key;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        kand &= (uint32_t)__shfl_xor((int)kand, off);
        kor |= (uint32_t)__shfl_xor((int)kor, off);
    }
    if ((tid & 63) == 0) { sm.band[tid >> 6] = kand; sm.bor[tid >> 6] = kor; }
    __syncthreads();
    kand = sm.band[0] & sm.band[1] & sm.band[2] & sm.band[3];
    kor = sm.bor[0] | sm.bor[1] | sm.bor[2] | sm.bor[3];
    __syncthreads();
    const uint32_t diff = kand ^ kor;
    int start = -8;
    uint32_t mask = 0xFFFFFFFFu;
    if (diff) {
        start = ((31 - __clz(diff)) / 8) * 8;
        mask = start == 24 ? 0u : (0xFFFFFFFFu << (start + 8));
    }
    uint32_t prefix = kand & mask;
    unsigned remaining = (unsigned)ke;
    for (int shift = start; shift >= 0; shift -= 8) {
        sm.hist[tid] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += 256) {
            uint32_t key = key_at(i);
            if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            const unsigned c0 = sm.hist[4 * tid], c1 = sm.hist[4 * tid + 1];
            const unsigned c2 = sm.hist[4 * tid + 2], c3 = sm.hist[4 * tid + 3];
            const unsigned tot = c0 + c1 + c2 + c3;
            unsigned S = tot;  // inclusive suffix sum over lanes >= tid
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                unsigned o = __shfl_down(S, off);
                if (tid + off < 64) S += o;
            }
            const unsigned above = S - tot;  // keys whose digit is above this lane's bins
            if (above < remaining && remaining <= S) {
                unsigned a = above;
                int dg;
                if (a + c3 >= remaining) dg = 4 * tid + 3;
                else if (a += c3, a + c2 >= remaining) dg = 4 * tid + 2;
                else if (a += c2, a + c1 >= remaining) dg = 4 * tid + 1;
                else { a += c1; dg = 4 * tid; }
                sm.digit = dg;
                sm.above = a;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sm.digit << shift;
        mask |= 255u << shift;
        remaining -= sm.above;
        __syncthreads();
    }
    const uint32_t T = prefix;
    // Ordered compaction over contiguous per-thread ranges.
    const int per = (n + 255) / 256;
    const int lo = tid * per < n ? tid * per : n;
    const int hi = lo + per < n ? lo + per : n;
    int gt = 0, eq = 0;
    for (int i = lo; i < hi; ++i) {
        uint32_t key = key_at(i);
        gt += key > T;
        eq += key == T;
    }
    const int eq_before = block_exclusive_scan(eq, sm.scan);
    int take_eq = (int)remaining - eq_before;
    take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
    int pos = block_exclusive_scan(gt + take_eq, sm.scan);
    int taken = 0;
    for (int i = lo; i < hi; ++i) {
        uint32_t key = key_at(i);
        bool take = key > T;
        if (key == T && taken < take_eq) { take = true; ++taken; }
        if (take) emit(pos++, i);
    }
    __syncthreads();
    return ke;
}


// ---- small exact top-k by rank counting -------------------------------------------------
// n <= 256 candidates, candidate i owned by thread i, given in ascending index order.  The
// ranking key is (ordered score, then lower position first); candidate i is chosen iff fewer
// than k_eff candidates outrank it, and is emitted at its position among the chosen ones,
// which keeps the output ascending.
struct SmallTopkSmem {
    alignas(16) unsigned long long key[256];
    ScanSmem scan;
};

template <class ScoreFn, class EmitFn>
__device__ int small_topk(int n, int k, ScoreFn score, EmitFn emit, SmallTopkSmem& sm) {
    const int t = threadIdx.x;
    const int ke = k < n ? k : n;
    if (ke <= 0) return 0;
    // keys padded with zeros to a multiple of 8: every real key is nonzero (its low word is
    // ~t), so a pad never outranks one
    const int np = (n + 7) & ~7;
    unsigned long long mine = 0ull;
    if (t < np) {
        if (t < n)
            mine = ((unsigned long long)ordered_key(score(t)) << 32) | (0xFFFFFFFFu - (unsigned)t);
        sm.key[t] = mine;
    }
    __syncthreads();
    bool take = false;
    if (t < n) {
        int rank = 0;
        typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
        // 8 keys per step in four 16-byte reads, several steps in flight
#pragma unroll 4
        for (int j = 0; j < np; j += 8) {
            const u64x2 a0 = *reinterpret_cast<const u64x2*>(&sm.key[j]);
            const u64x2 a1 = *reinterpret_cast<const u64x2*>(&sm.key[j + 2]);
            const u64x2 a2 = *reinterpret_cast<const u64x2*>(&sm.key[j + 4]);
            const u64x2 a3 = *reinterpret_cast<const u64x2*>(&sm.key[j + 6]);
            rank += (a0.x > mine) + (a0.y > mine) + (a1.x > mine) + (a1.y > mine) +
                    (a2.x > mine) + (a2.y > mine) + (a3.x > mine) + (a3.y > mine);
        }
        take = rank < ke;
    }
    // position among the chosen: chosen lanes below in this wave (ballot), then earlier waves
    const unsigned long long m = __ballot(take);
    const int below = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    if ((t & 63) == 0) sm.scan.w[t >> 6] = __popcll(m);
    __syncthreads();
    int pos = below;
    for (int i = 0; i < (t >> 6); ++i) pos += sm.scan.w[i];
    if (take) emit(pos, t);
    __syncthreads();
    return ke;
}

// ---- cross-workgroup hand-off ---------------------------------------------------------------
// On gfx950 each XCD has its own L2, and an agent-scope fence writes back and invalidates the
// whole L2 -- far too slow to run in every workgroup.  Data handed from one workgroup to
// another inside a kernel therefore travels through agent-scope relaxed atomic stores and
// loads, which are performed at the device coherence point, and the fences below only order
// (wait for outstanding memory operations); they make nothing visible by themselves.
template <class T>
__device__ __forceinline__ void st_shared_dev(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_shared_dev(const T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt vmcnt(0) with expcnt / lgkmcnt left free (gfx9 encoding)
__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
}

// s_waitcnt vmcnt(0) lgkmcnt(0): this wave's global -> LDS copies have landed and its own LDS
// stores are done.  Written out before the barrier of a copy loop rather than left to
// __syncthreads(): at a loop header the compiler's wait for the LDS stores of the previous
// iteration (reached over the back edge) has been seen to go missing next to an explicit
// vmcnt wait, so that other waves could pass the barrier and read them early.
__device__ __forceinline__ void wait_vmem_lds() {
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0x0 << 8));
}

// Every workgroup of a unit calls arrive_last() after writing its hand-off data with
// st_shared_dev; exactly one -- the last to arrive -- gets true and may then read the others'
// data with ld_shared_dev.  The last workgroup returns the counter to zero, so a zeroed
// counter stays zeroed between calls.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned total, int* s_flag) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    wait_vmem();                      // this wave's stores have reached the coherence point
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = atomicAdd(counter, 1u);
        const bool last = old == total - 1u;
        if (last) atomicExch(counter, 0u);
        *s_flag = last;
    }
    __syncthreads();
    const bool last = *s_flag != 0;
    // The counter was read before the barrier, so every load issued from here on follows it;
    // the reset above needs no wait (the kernel's end drains it).
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return last;
}

// ---- launches --------------------------------------------------------------------------------
// Launch kernel(a) on s; with an event of ev set, through hipExtLaunchKernel, which records
// the events at the kernel's own start and end.
template <class A, class E>
inline hipError_t dispatch(void (*kernel)(A), dim3 grid, dim3 block, uint32_t shmem,
                           hipStream_t s, const E& ev, const A& a) {
    if (ev.start || ev.stop) {
        void* args[] = {const_cast<A*>(&a)};
        return hipExtLaunchKernel((const void*)kernel, grid, block, args, shmem, s, ev.start,
                                  ev.stop, 0);
    }
    kernel<<<grid, block, shmem, s>>>(a);
    return hipGetLastError();
}

// A launcher that runs no kernel records ev's events back to back.
template <class E>
inline hipError_t no_kernel(const E& ev, hipStream_t s) {
    hipError_t e = hipSuccess;
    if (ev.start) e = hipEventRecord(ev.start, s);
    if (e == hipSuccess && ev.stop) e = hipEventRecord(ev.stop, s);
    return e;
}

}  // namespace tcs
