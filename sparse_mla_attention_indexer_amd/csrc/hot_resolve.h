// hot_resolve.h — limits and launcher of the hot-buffer resolve (hybrid offload).
#pragma once

#include "smla_internal.h"

namespace smla {

// Selections per request (n_q * top_k) and hot slots per request (the pages' default buffer is
// twice top-k, 4,096 rows at k = 2,048).
constexpr int HOT_MAX_SEL = 8192;
constexpr int HOT_MAX_SLOTS = 4096;

hipError_t launch_hot_resolve(const void* table, int32_t batch, const int32_t* idx, int32_t top_k,
                              const int32_t* resident_from, const int32_t* hot_base,
                              int32_t n_slots, int32_t* hot_tok, int32_t* hot_age, int32_t step,
                              const void* host_rows, int64_t host_n_rows, const int64_t* host_row0,
                              int32_t row_bytes, void* kv, int32_t* idx_out, int32_t* n_copied,
                              hipStream_t s);

}  // namespace smla
