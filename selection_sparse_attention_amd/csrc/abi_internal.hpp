// Host-side pieces of the C ABI shared between its source files.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/sparse_attn.h"

namespace sa {

// Validation, workspace carving and launch of the decode entry point
// (workspace protocol as in sparse_attn.h).
int32_t decode_entry(const sa_params* p, const sa_buffers* b, void* ws, size_t* ws_bytes,
                     void* stream);

}  // namespace sa
