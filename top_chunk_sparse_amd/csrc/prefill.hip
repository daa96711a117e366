// prefill.hip -- gfx950 kernels of the block-sparse causal prefill (SAS training-form
// forward, "SAS: Simple Attention Sparsification", abstract: the selector's scores enter the
// attention logits inside the softmax in log form, on a FlashAttention-style forward).
//
//   prefill_select_kernel  per (b, kv, query block i): top-min(k, i) earlier blocks by the
//                          selector row S[i][j < i] (lowest j on ties), ascending, and the
//                          gate log_softmax_j(S[i][j < i]) for the chosen blocks.
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

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t s) {
    (void)a;
    (void)s;
    return hipErrorNotSupported;
}

}  // namespace tcs
