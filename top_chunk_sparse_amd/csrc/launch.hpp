// launch.hpp -- internal interface between the C ABI layer (api.cpp) and the kernel
// launchers (decode.hip, prefill.hip).  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tcs {

// Per-slot softmax partial: unnormalised acc[d] plus (running max m, sum l).
struct Partials {
    float* acc;   // [B*Hq][nslots][d]
    float* ml;    // [B*Hq][nslots][2]
    int nslots;
};

struct GistLaunch {
    const uint16_t* q;
    const uint16_t* gk;
    const uint16_t* gv;
    long long unit_stride;    // elements between consecutive (b, kv) gist blocks
    int B, Hq, Hkv, d, g;
    int nchunks;              // chunks (or level-2 groups) in the scored range
    int slices;               // grid.x: slices of the range (range mode) or k2 (group mode)
    int chunks_per_slice;     // range mode
    const int32_t* groups;    // group mode: [units][k2] selected groups (-1 padded)
    int J, k2, H;             // group mode
    float sigma;
    float* scores;            // [units][score_stride]
    int score_stride;
    Partials part;
    int slot0;
};

struct SelectLaunch {
    int units;
    const float* scores;      // [units][score_stride]
    int score_stride;
    int n;                    // scores per unit (range mode)
    int k;                    // slots per unit in sel
    int32_t* sel;             // [units][k]
    float* gamma;             // [units][k] or null (SAS gate)
    // group mode (two-level candidates): position p -> chunk groups[u][p / J]*J + p % J
    const int32_t* groups;
    int J, k2, H;
    float* chunk_scores_out;  // optional [units][H]: candidates' scores, -inf elsewhere
};

struct ChunkLaunch {
    const uint16_t* q;
    const uint16_t* kp;
    const uint16_t* vp;
    const int32_t* page_table;
    int B, Hq, Hkv, d, C, N, M;
    int max_chunks, num_pages;
    const int32_t* sel;       // [units][k]
    const float* gamma;       // [units][k] or null
    int k;                    // stride of sel / gamma
    int kslots;               // selected-chunk slots launched (current chunk is slot kslots)
    float sigma;
    Partials part;
    int slot0;
};

struct CombineLaunch {
    Partials part;
    int BH, d;
    float* out;
    float* lse;
};

hipError_t launch_gist(const GistLaunch& a, hipStream_t s);
hipError_t launch_select(const SelectLaunch& a, hipStream_t s);
hipError_t launch_chunks(const ChunkLaunch& a, hipStream_t s);
hipError_t launch_combine(const CombineLaunch& a, hipStream_t s);

struct PrefillSelectLaunch {
    const float* S;           // [units][nb][nb]
    int units, nb, k;
    int32_t* sel;             // [units][nb][k]
    float* gamma;             // [units][nb][k] or null
};

struct PrefillLaunch {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    int B, Hq, Hkv, d, T, blk, ksel;
    const int32_t* sel;       // [B*Hkv][nb][ksel]
    const float* gamma;       // [B*Hkv][nb][ksel] or null
    float sigma;
    float* out;
    float* lse;
};

hipError_t launch_prefill_select(const PrefillSelectLaunch& a, hipStream_t s);
hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t s);

}  // namespace tcs
