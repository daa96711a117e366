// api.cpp -- the C ABI of libtcsparse.so (declared in include/tcsparse.h): argument checks,
// workspace carving and the launch sequence.  Everything here is host code; no call
// allocates, frees or synchronises, and argument errors return before any device work.
#include "tcsparse.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "api_internal.hpp"
#include "launch.hpp"

namespace {

using tcs::Partials;

constexpr size_t kAlign = 256;

// Every decode workspace starts with a block of arrival counters laid out the same way for
// every shape, so that one zeroed workspace serves calls of any shape in turn: each call
// leaves every counter it used at zero.  Units are (batch row, KV head) pairs.
constexpr int kMaxUnits = 16384;
constexpr size_t kCntSelect1 = 0;                         // selection arrivals (chunk pass)
constexpr size_t kCntSelect2 = kCntSelect1 + kMaxUnits;   // level-2 group pass
constexpr size_t kCntChunk = kCntSelect2 + kMaxUnits;     // chunk attention final merge
constexpr size_t kCounterWords = kCntChunk + kMaxUnits;
constexpr int kMaxSliceRows = 1024;   // rows one gist workgroup holds logits for (LDS)
#ifndef TCS_TARGET_WORKGROUPS
#define TCS_TARGET_WORKGROUPS 1024
#endif
constexpr int kTargetWorkgroups = TCS_TARGET_WORKGROUPS;   // grid size the passes aim for
#ifndef TCS_CHUNK_TARGET_WORKGROUPS
#define TCS_CHUNK_TARGET_WORKGROUPS 1024
#endif
constexpr int kChunkTargetWorkgroups = TCS_CHUNK_TARGET_WORKGROUPS;   // chunk-attention grid
constexpr int kMaxTopPK = 256;   // top-p: the capped top-k is ranked in one workgroup's LDS
constexpr int kMinSliceRows = 64;
constexpr int kMaxHeadSelectChunks = 65536;   // per-head selection: union bitmap held in LDS

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Events of the profiling entry points: events[2 i] and events[2 i + 1] are recorded by the
// launch of stage i at its kernel's own start and end (hipExtLaunchKernel); entries past
// n_events or null are skipped.
struct StageEvents {
    void* const* ev;
    int n;
    int stage = 0;
    tcs::KernelEvents next() {
        tcs::KernelEvents k;
        const int i = 2 * stage++;
        if (ev && i < n && ev[i]) k.start = (hipEvent_t)ev[i];
        if (ev && i + 1 < n && ev[i + 1]) k.stop = (hipEvent_t)ev[i + 1];
        return k;
    }
};

bool supported_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

// Split `nchunks` chunks of `g` rows into slices for the gist kernel: enough workgroups to
// fill the GPU, at least kMinSliceRows rows each, at most kMaxSliceRows.
void plan_slices(long long units, int nchunks, int g, int* slices, int* cps) {
    if (nchunks <= 0) { *slices = 0; *cps = 1; return; }
    long long want = (kTargetWorkgroups + units - 1) / units;
    if (want < 1) want = 1;
    long long c = (nchunks + want - 1) / want;
    long long cmin = (kMinSliceRows + g - 1) / g;
    if (c < cmin) c = cmin;
    long long cmax = kMaxSliceRows / g;
    if (c > cmax) c = cmax;
    if (c < 1) c = 1;
    *cps = (int)c;
    *slices = (int)((nchunks + c - 1) / c);
}

struct DecodePlan {
    int G, M, H, nG, k2e, S1, cps1, S2, cps2, kslots, cpw, rpw, nwx, nslots, kcap1, kcap2;
    int sk;   // entries per unit in sel: k, or G * k with per-head selection
    int ku, k2u;   // chunks and groups selected: k and k2, or min(cap, budget) when adaptive
    // one level, one list per slice, no top-p, at most 256 candidates per unit: the slices
    // publish their lists before their V rows and the first to finish merges them
    bool defer1;
    float sigma;
    // workspace offsets (bytes)
    size_t off_cnt, off_cs1, off_ci1, off_lse1, off_cs2, off_ci2, off_sel, off_gamma, off_gsel,
        off_acc, off_ml, total;
};

tcs_status plan_decode(const tcs_decode_params* p, DecodePlan* pl) {
    if (!p) return TCS_ERR_NULL;
    if (p->struct_size != (int32_t)sizeof(tcs_decode_params)) return TCS_ERR_SHAPE;
    if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->d < 1 || p->N < 1 || p->C < 1 || p->g < 1 ||
        p->k < 0 || p->num_pages < 1)
        return TCS_ERR_SHAPE;
    if (p->Hq % p->Hkv) return TCS_ERR_SHAPE;
    if (p->levels != 1 && p->levels != 2) return TCS_ERR_SHAPE;
    if (p->gate_mode != TCS_GATE_NONE && p->gate_mode != TCS_GATE_SAS) return TCS_ERR_SHAPE;
    if (p->gist_mode != TCS_GISTS_ALL && p->gist_mode != TCS_GISTS_SELECTED) return TCS_ERR_SHAPE;
    if (!(p->scale >= 0.f) || std::isinf(p->scale)) return TCS_ERR_SHAPE;
    if (!(p->top_p >= 0.f && p->top_p <= 1.f)) return TCS_ERR_SHAPE;
    if (p->select_mode != TCS_SELECT_KV_HEAD && p->select_mode != TCS_SELECT_PER_HEAD)
        return TCS_ERR_SHAPE;
    if (p->k_mode != TCS_K_FIXED && p->k_mode != TCS_K_ADAPTIVE) return TCS_ERR_SHAPE;
    const int G = p->Hq / p->Hkv;
    const long long units = (long long)p->B * p->Hkv;
    const int M = (int)(((long long)p->N + p->C - 1) / p->C);
    const int H = M - 1;
    if (p->max_chunks < M) return TCS_ERR_SHAPE;
    if (p->gist_cap != 0 && p->gist_cap < H) return TCS_ERR_SHAPE;
    if (units > kMaxUnits) return TCS_ERR_UNSUPPORTED;
    if (p->d != 64 && p->d != 128) return TCS_ERR_UNSUPPORTED;
    if (!supported_group(G)) return TCS_ERR_UNSUPPORTED;
    if (p->g > 64 || p->C > kMaxSliceRows) return TCS_ERR_UNSUPPORTED;
    const bool sel_gists = p->gist_mode == TCS_GISTS_SELECTED;
    if (sel_gists && p->C + p->g > kMaxSliceRows) return TCS_ERR_UNSUPPORTED;
    if (p->top_p > 0.f && p->k > kMaxTopPK) return TCS_ERR_UNSUPPORTED;
    const bool heads = p->select_mode == TCS_SELECT_PER_HEAD;
    if (heads && (p->levels != 1 || p->gate_mode != TCS_GATE_NONE || p->top_p > 0.f ||
                  H > kMaxHeadSelectChunks))
        return TCS_ERR_UNSUPPORTED;
    if (p->k_mode == TCS_K_ADAPTIVE && p->top_p > 0.f) return TCS_ERR_UNSUPPORTED;
    if (p->levels == 2 && p->J < 1) return TCS_ERR_SHAPE;
    // Adaptive top-k ("Simplified Sparse Attention via Gist Tokens", appendix A): one budget
    // per routing level, floor(N / (L_eff G C)) + 1 with L_eff = C (one level) or C J (two);
    // both levels select min(cap, budget).  Otherwise k and k2 as given.
    pl->ku = p->k;
    pl->k2u = p->k2;
    if (p->k_mode == TCS_K_ADAPTIVE) {
        const long long l_eff = (long long)p->C * (p->levels == 2 ? p->J : 1);
        const long long budget = (long long)p->N / (l_eff * G * p->C) + 1;
        pl->ku = (int)std::min<long long>(p->k, budget);
        pl->k2u = (int)std::min<long long>(p->k2, budget);
    }
    pl->G = G;
    pl->M = M;
    pl->H = H;
    pl->sigma = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->d);
    int ksel;
    if (p->levels == 2) {
        if (p->J < 1 || p->k2 < 0) return TCS_ERR_SHAPE;
        if (p->gate_mode != TCS_GATE_NONE) return TCS_ERR_UNSUPPORTED;
        if ((long long)p->J * p->g > kMaxSliceRows) return TCS_ERR_UNSUPPORTED;
        pl->nG = (H + p->J - 1) / p->J;
        pl->k2e = pl->k2u < pl->nG ? pl->k2u : pl->nG;
        if (pl->k2e > 64) return TCS_ERR_UNSUPPORTED;   // chosen groups held in LDS
        plan_slices(units, pl->nG, p->g, &pl->S2, &pl->cps2);
        pl->S1 = 0;
        pl->cps1 = 1;
        const long long ncand = (long long)pl->k2e * p->J;
        ksel = (int)(pl->ku < ncand ? pl->ku : ncand);
        pl->kcap2 = pl->k2u < pl->cps2 ? pl->k2u : pl->cps2;
        pl->kcap1 = pl->ku < p->J ? pl->ku : p->J;
    } else {
        pl->nG = 0;
        pl->k2e = 0;
        pl->S2 = 0;
        pl->cps2 = 1;
        // per-head selection keeps G scores per chunk of a slice in LDS
        plan_slices(units, H, heads ? std::max(p->g, G) : p->g, &pl->S1, &pl->cps1);
        ksel = pl->ku < H ? pl->ku : H;
        pl->kcap2 = 0;
        pl->kcap1 = pl->ku < pl->cps1 ? pl->ku : pl->cps1;
        if (heads) ksel = (int)std::min<long long>((long long)G * ksel, H);   // union size bound
    }
    pl->defer1 = false;
    if (p->levels == 1 && !heads && p->top_p == 0.f && pl->S1 > 0 && pl->ku >= 1) {
        const long long last_items = H - (long long)(pl->S1 - 1) * pl->cps1;
        const long long ncand =
            (long long)(pl->S1 - 1) * pl->kcap1 + std::min<long long>(pl->ku, last_items);
        if (ncand <= 256 && pl->cps1 <= 256) {
            pl->defer1 = true;
        }
    }
    pl->kslots = ksel;
    pl->sk = heads ? G * p->k : p->k;
    // chunk attention: enough workgroups to fill the GPU, one or more chunks each
    long long cpw = units * (ksel + 1) / kChunkTargetWorkgroups;
    const long long slot_rows = p->C + (sel_gists ? p->g : 0);   // rows a slot holds in LDS
    const long long cpw_max = std::min<long long>(16, kMaxSliceRows / slot_rows);
    // At least two slots per workgroup once there are enough of them: a workgroup's fixed costs
    // (dispatch, query load, partial write, arrival) then pay for twice the bytes.
    const long long cpw_min = units * (ksel + 1) >= 512 ? 2 : 1;
    pl->cpw = (int)std::max<long long>(std::min(cpw_min, cpw_max), std::min(cpw, cpw_max));
    pl->rpw = 0;
    pl->nwx = (ksel + 1 + pl->cpw - 1) / pl->cpw;
    if (!sel_gists) {
        // Row mode: the slots' rows laid end to end and cut into equal runs, so that the grid
        // comes to about kChunkTargetWorkgroups equal workgroups (a CU then holds whole
        // workgroups of equal work) of at least cpw_min chunks' rows each.
        const long long R = (long long)ksel * p->C + (p->N - (long long)(M - 1) * p->C);
        long long rpw = (units * R + kChunkTargetWorkgroups - 1) / kChunkTargetWorkgroups;
        rpw = std::max<long long>(rpw, std::min(cpw_min, cpw_max) * p->C);
        rpw = (rpw + 15) / 16 * 16;
        rpw = std::min<long long>(rpw, std::min<long long>(kMaxSliceRows, 15LL * p->C));
        pl->rpw = (int)rpw;
        pl->nwx = (int)((R + rpw - 1) / rpw);
    }
    // softmax partial slots per query head: gist slices and level-2 slices (none with selected
    // gists), one per chosen level-2 group (its members' gists, or with selected gists its own
    // level-2 gists), then the chunk-attention workgroups
    pl->nslots = (sel_gists ? 0 : pl->S1 + pl->S2) + pl->k2e + pl->nwx;
    const long long BH = (long long)p->B * p->Hq;
    const long long s1 = p->levels == 2 ? pl->k2e : pl->S1;     // slices of the chunk pass
    auto n1 = [](long long x) { return x > 0 ? x : 1; };
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    pl->off_cnt = take(sizeof(unsigned) * kCounterWords);
    const long long nl = heads ? G : 1;   // candidate lists per slice: one per selecting head
    pl->off_cs1 = take(sizeof(float) * (size_t)n1(units * nl * s1 * pl->kcap1));
    pl->off_ci1 = take(sizeof(int32_t) * (size_t)n1(units * nl * s1 * pl->kcap1));
    pl->off_lse1 = take(sizeof(float) * (size_t)n1(units * s1 * 2));
    pl->off_cs2 = take(sizeof(float) * (size_t)n1(units * pl->S2 * pl->kcap2));
    pl->off_ci2 = take(sizeof(int32_t) * (size_t)n1(units * pl->S2 * pl->kcap2));
    pl->off_sel = take(sizeof(int32_t) * (size_t)n1(units * pl->sk));
    pl->off_gamma = take(sizeof(float) * (size_t)n1(units * p->k));
    pl->off_gsel = take(sizeof(int32_t) * (size_t)n1(units * p->k2));
    pl->off_acc = take(sizeof(float) * (size_t)(BH * pl->nslots * p->d));
    pl->off_ml = take(sizeof(float) * (size_t)(BH * pl->nslots * 2));
    pl->total = off;
    return TCS_OK;
}

struct PrefillPlan {
    int G, nb;
    float sigma;
    size_t off_sel, off_gamma, total;
};

tcs_status plan_prefill(const tcs_prefill_params* p, PrefillPlan* pl) {
    if (!p) return TCS_ERR_NULL;
    if (p->struct_size != (int32_t)sizeof(tcs_prefill_params)) return TCS_ERR_SHAPE;
    if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->d < 1 || p->T < 1 || p->blk < 1 || p->k < 0)
        return TCS_ERR_SHAPE;
    if (p->Hq % p->Hkv || p->T % p->blk) return TCS_ERR_SHAPE;
    if (p->gate_mode != TCS_GATE_NONE && p->gate_mode != TCS_GATE_SAS) return TCS_ERR_SHAPE;
    if (!(p->scale >= 0.f) || std::isinf(p->scale)) return TCS_ERR_SHAPE;
    const int G = p->Hq / p->Hkv;
    if (p->d != 128 || p->blk != 64 || !supported_group(G)) return TCS_ERR_UNSUPPORTED;
    const long long units = (long long)p->B * p->Hkv;
    pl->G = G;
    pl->nb = p->T / p->blk;
    if (units * pl->nb > INT_MAX / 2) return TCS_ERR_UNSUPPORTED;
    pl->sigma = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->d);
    const int kk = p->k > 0 ? p->k : 1;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    pl->off_sel = take(sizeof(int32_t) * (size_t)(units * pl->nb * kk));
    pl->off_gamma = take(sizeof(float) * (size_t)(units * pl->nb * kk));
    pl->total = off;
    return TCS_OK;
}

struct PrefillBwdPlan {
    PrefillPlan f;
    size_t off_D, off_inv_i, off_inv_g, off_inv_n, off_dgp, total;
};

tcs_status plan_prefill_backward(const tcs_prefill_params* p, PrefillBwdPlan* pl) {
    tcs_status st = plan_prefill(p, &pl->f);
    if (st != TCS_OK) return st;
    const long long units = (long long)p->B * p->Hkv;
    const long long nb = pl->f.nb;
    const long long nh = 4LL * ((pl->f.G + 3) / 4);
    const long long kk = p->k > 0 ? p->k : 1;
    size_t off = pl->f.total;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    pl->off_D = take(sizeof(float) * (size_t)((long long)p->B * p->Hq * p->T));
    pl->off_inv_i = take(sizeof(int32_t) * (size_t)(units * nb * nb));
    pl->off_inv_g = take(sizeof(float) * (size_t)(units * nb * nb));
    pl->off_inv_n = take(sizeof(int32_t) * (size_t)(units * nb));
    pl->off_dgp = take(sizeof(float) * (size_t)(units * nb * 2 * nh * kk));
    pl->total = off;
    return TCS_OK;
}

struct GistPrefillPlan {
    int G, Gp;
    float sigma;
    size_t off_gk, off_gv, total;
};

tcs_status plan_gist_prefill(const tcs_gist_prefill_params* p, GistPrefillPlan* pl) {
    if (!p) return TCS_ERR_NULL;
    if (p->struct_size != (int32_t)sizeof(tcs_gist_prefill_params)) return TCS_ERR_SHAPE;
    if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->d < 1 || p->M < 1 || p->L < 1 || p->g < 1)
        return TCS_ERR_SHAPE;
    if (p->Hq % p->Hkv) return TCS_ERR_SHAPE;
    if (!(p->scale >= 0.f) || std::isinf(p->scale)) return TCS_ERR_SHAPE;
    const int G = p->Hq / p->Hkv;
    if (p->d != 128 || p->L % 64 || p->g > 64 || 64 % p->g || !supported_group(G))
        return TCS_ERR_UNSUPPORTED;
    const long long Tp = (long long)p->M * (p->L + p->g);
    if (Tp > INT_MAX / 2 || (long long)p->B * p->Hq * Tp > (1LL << 40)) return TCS_ERR_UNSUPPORTED;
    pl->G = G;
    pl->Gp = (int)(((long long)p->M * p->g + 63) / 64 * 64);
    pl->sigma = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->d);
    const size_t rows = (size_t)p->B * p->Hkv * pl->Gp;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    pl->off_gk = take(sizeof(uint16_t) * rows * p->d);
    pl->off_gv = take(sizeof(uint16_t) * rows * p->d);
    pl->total = off;
    return TCS_OK;
}

tcs_status check_ws(void* ws, size_t have, size_t need) {
    if (have < need) return TCS_ERR_WORKSPACE;
    if (need > 0 && (!ws || ((uintptr_t)ws % kAlign))) return TCS_ERR_WORKSPACE;
    return TCS_OK;
}

}  // namespace

extern "C" {

int tcs_abi_version(void) { return TCS_ABI_VERSION; }

const char* tcs_status_str(tcs_status s) {
    // callers may pass any int (the C enum is an int); read it as one, never as the C++ enum,
    // whose values outside the declared ones are undefined
    int code;
    std::memcpy(&code, &s, sizeof code);
    switch (code) {
        case TCS_OK: return "ok";
        case TCS_ERR_NULL: return "null pointer argument";
        case TCS_ERR_SHAPE: return "invalid sizes";
        case TCS_ERR_UNSUPPORTED: return "unsupported configuration";
        case TCS_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case TCS_ERR_HIP: return "HIP kernel launch failed";
        case TCS_ERR_TOO_LARGE: return "shape needs more than the static scratch of the no-alloc entry point";
    }
    return "unknown status";
}

tcs_status tcs_decode_workspace_size(const tcs_decode_params* p, size_t* bytes) {
    if (!bytes) return TCS_ERR_NULL;
    DecodePlan pl;
    tcs_status st = plan_decode(p, &pl);
    if (st != TCS_OK) return st;
    *bytes = pl.total;
    return TCS_OK;
}

}  // extern "C"

namespace tcs {

tcs_status decode_check(const tcs_decode_params* p, const void* q, const void* k_pages,
                        const void* v_pages, const int32_t* page_table, const void* gist_k,
                        const void* gist_v, const void* gist2_k, const void* gist2_v,
                        const float* out, size_t* workspace_bytes) {
    DecodePlan pl;
    tcs_status st = plan_decode(p, &pl);
    if (st != TCS_OK) return st;
    if (!q || !k_pages || !v_pages || !page_table || !out) return TCS_ERR_NULL;
    if (pl.H > 0 && (!gist_k || !gist_v)) return TCS_ERR_NULL;
    if (p->levels == 2 && pl.nG > 0 && (!gist2_k || !gist2_v)) return TCS_ERR_NULL;
    *workspace_bytes = pl.total;
    return TCS_OK;
}

size_t decode_counter_bytes() { return sizeof(unsigned) * kCounterWords; }

tcs_status decode_impl(const tcs_decode_params* p, const void* q, const void* k_pages,
                       const void* v_pages, const int32_t* page_table, const void* gist_k,
                       const void* gist_v, const void* gist2_k, const void* gist2_v, float* out,
                       float* lse, int32_t* sel, int32_t* sel_groups, float* chunk_scores,
                       void* workspace, size_t workspace_bytes, void* stream,
                       void* const* events, int n_events) {
    size_t need = 0;
    tcs_status st = decode_check(p, q, k_pages, v_pages, page_table, gist_k, gist_v, gist2_k,
                                 gist2_v, out, &need);
    if (st != TCS_OK) return st;
    DecodePlan pl;
    plan_decode(p, &pl);
    st = check_ws(workspace, workspace_bytes, pl.total);
    if (st != TCS_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    StageEvents clk{events, n_events};
    char* ws = (char*)workspace;
    const int units = p->B * p->Hkv;
    const int cap = p->gist_cap > 0 ? p->gist_cap : pl.H;
    unsigned* cnt = (unsigned*)(ws + pl.off_cnt);
    Partials part{(float*)(ws + pl.off_acc), (float*)(ws + pl.off_ml), pl.nslots};
    int32_t* sel_p = sel ? sel : (int32_t*)(ws + pl.off_sel);
    float* gamma = p->gate_mode == TCS_GATE_SAS ? (float*)(ws + pl.off_gamma) : nullptr;
    hipError_t e = hipSuccess;
    int slot = 0;

    tcs::GistLaunch ga{};
    ga.q = (const uint16_t*)q;
    ga.B = p->B; ga.Hq = p->Hq; ga.Hkv = p->Hkv; ga.d = p->d; ga.g = p->g;
    ga.sigma = pl.sigma;
    ga.part = part;
    ga.J = p->J; ga.k2 = p->k2; ga.H = pl.H;

    tcs::SelectOut chunk_sel{};   // the pass that chooses chunks
    chunk_sel.k = pl.ku;
    chunk_sel.stride = p->k;
    chunk_sel.sel = sel_p;
    chunk_sel.cand_score = (float*)(ws + pl.off_cs1);
    chunk_sel.cand_idx = (int32_t*)(ws + pl.off_ci1);
    chunk_sel.kcap = pl.kcap1;
    chunk_sel.J = p->J;
    chunk_sel.H = pl.H;

    bool chunks_chosen = false;
    if (p->levels == 1) {
        chunk_sel.gamma = gamma;
        // the log-sum-exp over every historical score: for the gate and for top-p's shares
        chunk_sel.slice_lse = (gamma || p->top_p > 0.f) ? (float*)(ws + pl.off_lse1) : nullptr;
        chunk_sel.top_p = p->top_p;
        chunk_sel.counter = cnt;
        chunk_sel.defer = pl.defer1;
        ga.gk = (const uint16_t*)gist_k;
        ga.gv = (const uint16_t*)gist_v;
        ga.unit_stride = (long long)cap * p->g * p->d;
        ga.nitems = pl.H;
        ga.slices = pl.S1;
        ga.items_per_slice = pl.cps1;
        ga.groups = nullptr;
        ga.scores_out = chunk_scores;
        ga.score_stride = pl.H;
        ga.slot0 = slot;
        ga.selo = chunk_sel;
        ga.scores_only = p->gist_mode == TCS_GISTS_SELECTED;
        ga.heads = p->select_mode == TCS_SELECT_PER_HEAD;
        e = tcs::launch_gist(ga, s, clk.next());
        if (e != hipSuccess) return TCS_ERR_HIP;
        if (!ga.scores_only) slot += pl.S1;
        chunks_chosen = pl.S1 > 0;
    } else {
        int32_t* gsel = sel_groups ? sel_groups : (int32_t*)(ws + pl.off_gsel);
        // level 2: every group, choosing k2 of them
        tcs::SelectOut gs{};
        gs.k = pl.k2u;
        gs.stride = p->k2;
        gs.sel = gsel;
        gs.cand_score = (float*)(ws + pl.off_cs2);
        gs.cand_idx = (int32_t*)(ws + pl.off_ci2);
        gs.kcap = pl.kcap2;
        gs.counter = cnt + kCntSelect2;
        gs.fill_scores = chunk_scores;
        gs.J = p->J;
        gs.H = pl.H;
        ga.gk = (const uint16_t*)gist2_k;
        ga.gv = (const uint16_t*)gist2_v;
        ga.unit_stride = (long long)pl.nG * p->g * p->d;
        ga.nitems = pl.nG;
        ga.slices = pl.S2;
        ga.items_per_slice = pl.cps2;
        ga.groups = nullptr;
        ga.scores_out = nullptr;
        ga.score_stride = 0;
        ga.slot0 = slot;
        ga.selo = gs;
        ga.scores_only = p->gist_mode == TCS_GISTS_SELECTED;
        e = tcs::launch_gist(ga, s, clk.next());
        if (e != hipSuccess) return TCS_ERR_HIP;
        if (!ga.scores_only) slot += pl.S2;
        if (pl.S2 == 0 && sel_groups && p->k2 > 0) {
            e = tcs::launch_fill(sel_groups, (long long)units * p->k2, -1, s);
            if (e != hipSuccess) return TCS_ERR_HIP;
        }

        // level 1: the member chunks of the chosen groups; top-p's shares are taken over them
        chunk_sel.gamma = nullptr;
        chunk_sel.slice_lse = p->top_p > 0.f ? (float*)(ws + pl.off_lse1) : nullptr;
        chunk_sel.top_p = p->top_p;
        chunk_sel.counter = cnt;
        ga.gk = (const uint16_t*)gist_k;
        ga.gv = (const uint16_t*)gist_v;
        ga.unit_stride = (long long)cap * p->g * p->d;
        ga.nitems = pl.H;
        ga.slices = pl.k2e;
        ga.items_per_slice = p->J;
        ga.groups = gsel;
        ga.scores_out = chunk_scores;
        ga.score_stride = pl.H;
        ga.slot0 = slot;
        ga.selo = chunk_sel;
        if (ga.scores_only) {   // the chosen groups' level-2 gists are the slices' tokens
            ga.pk = (const uint16_t*)gist2_k;
            ga.pv = (const uint16_t*)gist2_v;
            ga.p_unit_stride = (long long)pl.nG * p->g * p->d;
        }
        e = tcs::launch_gist(ga, s, clk.next());
        if (e != hipSuccess) return TCS_ERR_HIP;
        slot += pl.k2e;
        chunks_chosen = pl.k2e > 0;
    }
    if (!chunks_chosen && pl.sk > 0) {
        // no scoring pass ran (no historical chunk, or no group chosen): nothing is selected
        e = tcs::launch_fill(sel_p, (long long)units * pl.sk, -1, s);
        if (e != hipSuccess) return TCS_ERR_HIP;
    }

    tcs::ChunkLaunch ca{};
    ca.q = (const uint16_t*)q;
    ca.kp = (const uint16_t*)k_pages;
    ca.vp = (const uint16_t*)v_pages;
    ca.page_table = page_table;
    ca.B = p->B; ca.Hq = p->Hq; ca.Hkv = p->Hkv; ca.d = p->d; ca.C = p->C; ca.N = p->N;
    ca.M = pl.M; ca.max_chunks = p->max_chunks; ca.num_pages = p->num_pages;
    ca.sel = sel_p; ca.gamma = gamma; ca.k = pl.sk; ca.kslots = pl.kslots; ca.cpw = pl.cpw;
    ca.rpw = pl.rpw;
    ca.sigma = pl.sigma; ca.part = part; ca.slot0 = slot;
    ca.counter = cnt + kCntChunk;
    ca.out = out;
    ca.lse = lse;
    if (p->gist_mode == TCS_GISTS_SELECTED) {
        ca.gk = (const uint16_t*)gist_k;
        ca.gv = (const uint16_t*)gist_v;
        ca.gist_stride = (long long)cap * p->g * p->d;
        ca.g = p->g;
    }
    e = tcs::launch_chunks(ca, s, clk.next());
    if (e != hipSuccess) return TCS_ERR_HIP;
    return TCS_OK;
}

}  // namespace tcs

extern "C" {

tcs_status sparse_attn_decode(const tcs_decode_params* p, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* page_table, const void* gist_k,
                              const void* gist_v, const void* gist2_k, const void* gist2_v,
                              float* out, float* lse, int32_t* sel, int32_t* sel_groups,
                              float* chunk_scores, void* workspace, size_t workspace_bytes,
                              void* stream) {
    return tcs::decode_impl(p, q, k_pages, v_pages, page_table, gist_k, gist_v, gist2_k, gist2_v, out,
                       lse, sel, sel_groups, chunk_scores, workspace, workspace_bytes, stream,
                       nullptr, 0);
}

tcs_status sparse_attn_decode_timed(const tcs_decode_params* p, const void* q,
                                    const void* k_pages, const void* v_pages,
                                    const int32_t* page_table, const void* gist_k,
                                    const void* gist_v, const void* gist2_k, const void* gist2_v,
                                    float* out, float* lse, int32_t* sel, int32_t* sel_groups,
                                    float* chunk_scores, void* workspace, size_t workspace_bytes,
                                    void* stream, void* const* events, int n_events) {
    if (n_events < 0) return TCS_ERR_SHAPE;
    return tcs::decode_impl(p, q, k_pages, v_pages, page_table, gist_k, gist_v, gist2_k, gist2_v, out,
                       lse, sel, sel_groups, chunk_scores, workspace, workspace_bytes, stream,
                       events, n_events);
}

int tcs_decode_stage_count(const tcs_decode_params* p) {
    DecodePlan pl;
    if (plan_decode(p, &pl) != TCS_OK) return -1;
    return p->levels == 2 ? 3 : 2;
}

tcs_status tcs_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (workspace_bytes == 0) return TCS_OK;
    if (!workspace || ((uintptr_t)workspace % kAlign)) return TCS_ERR_WORKSPACE;
    if (tcs::launch_zero(workspace, workspace_bytes, (hipStream_t)stream) != hipSuccess)
        return TCS_ERR_HIP;
    return TCS_OK;
}

tcs_status tcs_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
    if (bytes == 0) return TCS_OK;
    if (!src || !sink) return TCS_ERR_NULL;
    if ((uintptr_t)src % 16 || bytes % 16) return TCS_ERR_SHAPE;
    if (tcs::launch_stream_read(src, bytes, (unsigned*)sink, TCS_STREAM_READ_BLOCKS,
                                (hipStream_t)stream) != hipSuccess)
        return TCS_ERR_HIP;
    return TCS_OK;
}

tcs_status tcs_prefill_workspace_size(const tcs_prefill_params* p, size_t* bytes) {
    if (!bytes) return TCS_ERR_NULL;
    PrefillPlan pl;
    tcs_status st = plan_prefill(p, &pl);
    if (st != TCS_OK) return st;
    *bytes = pl.total;
    return TCS_OK;
}

static tcs_status prefill_impl(const tcs_prefill_params* p, const void* q, const void* k,
                               const void* v, const float* S, float* out, float* lse,
                               int32_t* sel, void* workspace, size_t workspace_bytes,
                               void* stream, void* const* events, int n_events) {
    PrefillPlan pl;
    tcs_status st = plan_prefill(p, &pl);
    if (st != TCS_OK) return st;
    if (!q || !k || !v || !out || (!S && p->k > 0) || (!S && p->gate_mode == TCS_GATE_SAS))
        return TCS_ERR_NULL;
    st = check_ws(workspace, workspace_bytes, pl.total);
    if (st != TCS_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    StageEvents clk{events, n_events};
    char* ws = (char*)workspace;
    const int units = p->B * p->Hkv;
    const int kk = p->k > 0 ? p->k : 0;
    int32_t* sel_p = sel ? sel : (int32_t*)(ws + pl.off_sel);
    float* gamma = p->gate_mode == TCS_GATE_SAS ? (float*)(ws + pl.off_gamma) : nullptr;
    {   // with k = 0 no selection kernel runs (its events are still recorded)
        tcs::PrefillSelectLaunch ps{S, units, pl.nb, kk, sel_p, gamma};
        if (tcs::launch_prefill_select(ps, s, clk.next()) != hipSuccess) return TCS_ERR_HIP;
    }
    tcs::PrefillLaunch pa{};
    pa.q = (const uint16_t*)q;
    pa.k = (const uint16_t*)k;
    pa.v = (const uint16_t*)v;
    pa.B = p->B; pa.Hq = p->Hq; pa.Hkv = p->Hkv; pa.d = p->d; pa.T = p->T; pa.blk = p->blk;
    pa.ksel = kk;
    pa.sel = kk > 0 ? sel_p : nullptr;
    pa.gamma = kk > 0 ? gamma : nullptr;
    pa.sigma = pl.sigma;
    pa.out = out;
    pa.lse = lse;
    hipError_t e = tcs::launch_prefill(pa, s, clk.next());
    if (e == hipErrorNotSupported) return TCS_ERR_UNSUPPORTED;
    if (e != hipSuccess) return TCS_ERR_HIP;
    return TCS_OK;
}

tcs_status tcs_gist_prefill_workspace_size(const tcs_gist_prefill_params* p, size_t* bytes) {
    if (!bytes) return TCS_ERR_NULL;
    GistPrefillPlan pl;
    tcs_status st = plan_gist_prefill(p, &pl);
    if (st != TCS_OK) return st;
    *bytes = pl.total;
    return TCS_OK;
}

static tcs_status gist_prefill_impl(const tcs_gist_prefill_params* p, const void* q,
                                    const void* k, const void* v, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    void* const* events, int n_events) {
    GistPrefillPlan pl;
    tcs_status st = plan_gist_prefill(p, &pl);
    if (st != TCS_OK) return st;
    if (!q || !k || !v || !out) return TCS_ERR_NULL;
    st = check_ws(workspace, workspace_bytes, pl.total);
    if (st != TCS_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    StageEvents clk{events, n_events};
    char* ws = (char*)workspace;
    tcs::GistPrefillLaunch a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.d = p->d; a.M = p->M; a.L = p->L; a.g = p->g;
    a.Gp = pl.Gp;
    a.gk = (uint16_t*)(ws + pl.off_gk);
    a.gv = (uint16_t*)(ws + pl.off_gv);
    a.sigma = pl.sigma;
    a.out = out;
    a.lse = lse;
    hipError_t e = tcs::launch_gist_gather(a, s, clk.next());
    if (e == hipSuccess) e = tcs::launch_gist_prefill_rows(a, s, clk.next());
    if (e == hipErrorNotSupported) return TCS_ERR_UNSUPPORTED;
    return e == hipSuccess ? TCS_OK : TCS_ERR_HIP;
}

tcs_status sparse_attn_gist_prefill(const tcs_gist_prefill_params* p, const void* q,
                                    const void* k, const void* v, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    return gist_prefill_impl(p, q, k, v, out, lse, workspace, workspace_bytes, stream, nullptr, 0);
}

tcs_status sparse_attn_gist_prefill_timed(const tcs_gist_prefill_params* p, const void* q,
                                          const void* k, const void* v, float* out, float* lse,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* const* events, int n_events) {
    if (n_events < 0) return TCS_ERR_SHAPE;
    return gist_prefill_impl(p, q, k, v, out, lse, workspace, workspace_bytes, stream, events,
                             n_events);
}

tcs_status tcs_prefill_backward_workspace_size(const tcs_prefill_params* p, size_t* bytes) {
    if (!bytes) return TCS_ERR_NULL;
    PrefillBwdPlan pl;
    tcs_status st = plan_prefill_backward(p, &pl);
    if (st != TCS_OK) return st;
    *bytes = pl.total;
    return TCS_OK;
}

static tcs_status prefill_backward_impl(const tcs_prefill_params* p, const void* q,
                                        const void* k, const void* v, const float* S,
                                        const float* out, const float* lse, const void* dout,
                                        const float* dlse, float* dq, float* dk, float* dv,
                                        float* dS, void* workspace, size_t workspace_bytes,
                                        void* stream, void* const* events, int n_events) {
    PrefillBwdPlan pl;
    tcs_status st = plan_prefill_backward(p, &pl);
    if (st != TCS_OK) return st;
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv ||
        (!S && (p->k > 0 || p->gate_mode == TCS_GATE_SAS || dS)))
        return TCS_ERR_NULL;
    st = check_ws(workspace, workspace_bytes, pl.total);
    if (st != TCS_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    StageEvents clk{events, n_events};
    char* ws = (char*)workspace;
    const int units = p->B * p->Hkv;
    const int kk = p->k > 0 ? p->k : 0;
    int32_t* sel = (int32_t*)(ws + pl.f.off_sel);
    float* gamma = p->gate_mode == TCS_GATE_SAS ? (float*)(ws + pl.f.off_gamma) : nullptr;
    {   // with k = 0 no selection kernel runs (its events are still recorded)
        tcs::PrefillSelectLaunch ps{S, units, pl.f.nb, kk, sel, gamma};
        if (tcs::launch_prefill_select(ps, s, clk.next()) != hipSuccess) return TCS_ERR_HIP;
    }
    tcs::PrefillBwdLaunch a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.dout = (const uint16_t*)dout;
    a.out = out;
    a.lse = lse;
    a.dlse = dlse;
    a.S = S;
    a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.d = p->d; a.T = p->T; a.blk = p->blk;
    a.ksel = kk;
    a.gate = p->gate_mode == TCS_GATE_SAS;
    a.sel = kk > 0 ? sel : nullptr;
    a.gamma = kk > 0 ? gamma : nullptr;
    a.sigma = pl.f.sigma;
    a.D = (float*)(ws + pl.off_D);
    a.inv_i = (int32_t*)(ws + pl.off_inv_i);
    a.inv_g = (float*)(ws + pl.off_inv_g);
    a.inv_n = (int32_t*)(ws + pl.off_inv_n);
    a.dgp = (float*)(ws + pl.off_dgp);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dS = dS;
    hipError_t e = tcs::launch_prefill_bwd_prep(a, s, clk.next());
    if (e == hipSuccess) e = tcs::launch_prefill_bwd_grad(a, s, clk.next());
    if (e == hipSuccess) e = tcs::launch_prefill_bwd_ds(a, s, clk.next());
    if (e == hipErrorNotSupported) return TCS_ERR_UNSUPPORTED;
    return e == hipSuccess ? TCS_OK : TCS_ERR_HIP;
}

tcs_status sparse_attn_prefill_backward(const tcs_prefill_params* p, const void* q,
                                        const void* k, const void* v, const float* S,
                                        const float* out, const float* lse, const void* dout,
                                        const float* dlse, float* dq, float* dk, float* dv,
                                        float* dS, void* workspace, size_t workspace_bytes,
                                        void* stream) {
    return prefill_backward_impl(p, q, k, v, S, out, lse, dout, dlse, dq, dk, dv, dS,
                                 workspace, workspace_bytes, stream, nullptr, 0);
}

tcs_status sparse_attn_prefill_backward_timed(const tcs_prefill_params* p, const void* q,
                                              const void* k, const void* v, const float* S,
                                              const float* out, const float* lse,
                                              const void* dout, const float* dlse, float* dq,
                                              float* dk, float* dv, float* dS, void* workspace,
                                              size_t workspace_bytes, void* stream,
                                              void* const* events, int n_events) {
    if (n_events < 0) return TCS_ERR_SHAPE;
    return prefill_backward_impl(p, q, k, v, S, out, lse, dout, dlse, dq, dk, dv, dS,
                                 workspace, workspace_bytes, stream, events, n_events);
}

tcs_status sparse_attn_prefill(const tcs_prefill_params* p, const void* q, const void* k,
                               const void* v, const float* S, float* out, float* lse,
                               int32_t* sel, void* workspace, size_t workspace_bytes,
                               void* stream) {
    return prefill_impl(p, q, k, v, S, out, lse, sel, workspace, workspace_bytes, stream,
                        nullptr, 0);
}

tcs_status sparse_attn_prefill_timed(const tcs_prefill_params* p, const void* q, const void* k,
                                     const void* v, const float* S, float* out, float* lse,
                                     int32_t* sel, void* workspace, size_t workspace_bytes,
                                     void* stream, void* const* events, int n_events) {
    if (n_events < 0) return TCS_ERR_SHAPE;
    return prefill_impl(p, q, k, v, S, out, lse, sel, workspace, workspace_bytes, stream, events,
                        n_events);
}

}  // extern "C"
