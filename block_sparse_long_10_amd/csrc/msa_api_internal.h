// Host-side pieces of the C ABI shared between its source files.
#pragma once

#include "msa.h"
#include "msa_launch.h"

namespace msa {

// Records msg as the text of msa_last_error() and returns st.
msa_status set_error(msa_status st, const char* msg);

// msa_decode / msa_decode_append on a given workspace (append may be null):
// validation, then the index launch and the attention launch.
msa_status decode_impl(const msa_params* params, const msa_paged_kv* kv, const void* q,
                       const void* idx_q, const int32_t* seq_lens, int32_t batch,
                       int32_t max_seq_len, float* out, int32_t* sel, void* workspace,
                       size_t workspace_bytes, void* stream, const DecodeAppend* append);

}  // namespace msa
