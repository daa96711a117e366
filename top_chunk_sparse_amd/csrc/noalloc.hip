// noalloc.hip -- sparse_attn_decode_noalloc: the decode entry point for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The workspace the decode kernels need (arrival counters, per-slice candidate
// lists, softmax partials) lives in a static device array of fixed size, one copy per GPU,
// held until the process ends.  Nothing here allocates or frees.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.hpp"
#include "launch.hpp"

// The array's name is a host-side stand-in in host code; only the address returned by
// hipGetSymbolAddress (one per device) is ever handed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[TCS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per device with that
// device current.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    DeviceScratch& d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        void* ptr = nullptr;
        d.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        d.ptr = d.err == hipSuccess ? ptr : nullptr;
    });
    return d.ptr;
}

}  // namespace

extern "C" tcs_status sparse_attn_decode_noalloc(const tcs_decode_params* p, const void* q,
                                                 const void* k_pages, const void* v_pages,
                                                 const int32_t* page_table, const void* gist_k,
                                                 const void* gist_v, const void* gist2_k,
                                                 const void* gist2_v, float* out, float* lse,
                                                 int32_t* sel, int32_t* sel_groups,
                                                 float* chunk_scores, void* stream) {
    size_t need = 0;
    tcs_status st = tcs::decode_check(p, q, k_pages, v_pages, page_table, gist_k, gist_v,
                                      gist2_k, gist2_v, out, &need);
    if (st != TCS_OK) return st;
    if (need > (size_t)TCS_NOALLOC_SCRATCH_BYTES) return TCS_ERR_TOO_LARGE;
    void* ws = scratch_on_current_device();
    if (!ws) return TCS_ERR_HIP;
    // The counter block must read zero when a call starts; a call that failed may have left it
    // dirty, so it is cleared on every call (a fill kernel, not a memset).
    if (tcs::launch_zero(ws, tcs::decode_counter_bytes(), (hipStream_t)stream) != hipSuccess)
        return TCS_ERR_HIP;
    return tcs::decode_impl(p, q, k_pages, v_pages, page_table, gist_k, gist_v, gist2_k, gist2_v,
                            out, lse, sel, sel_groups, chunk_scores, ws,
                            (size_t)TCS_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0);
}
