// api_internal.hpp -- the decode entry point's body, shared by the C ABI functions in api.cpp
// and the allocation-free variant in noalloc.hip.  Internal; not part of the ABI.
#pragma once
#include <stddef.h>

#include "tcsparse.h"

namespace tcs {

// Host-side checks of a decode call (parameters, required pointers) and the workspace bytes
// it needs; no device work.
tcs_status decode_check(const tcs_decode_params* p, const void* q, const void* k_pages,
                        const void* v_pages, const int32_t* page_table, const void* gist_k,
                        const void* gist_v, const void* gist2_k, const void* gist2_v,
                        const float* out, size_t* workspace_bytes);

// Bytes of the arrival-counter block at the start of every decode workspace (the same for
// every shape); it must read zero when a call starts.
size_t decode_counter_bytes();

// sparse_attn_decode / sparse_attn_decode_timed on a caller-provided workspace.
tcs_status decode_impl(const tcs_decode_params* p, const void* q, const void* k_pages,
                       const void* v_pages, const int32_t* page_table, const void* gist_k,
                       const void* gist_v, const void* gist2_k, const void* gist2_v, float* out,
                       float* lse, int32_t* sel, int32_t* sel_groups, float* chunk_scores,
                       void* workspace, size_t workspace_bytes, void* stream,
                       void* const* events, int n_events);

}  // namespace tcs
