// Internal declarations shared by the host checks and the launchers.
#pragma once

#include "../../include/gdn_conv.h"
#include "../../include/gdn_spec.h"
#include "../../include/gdn_bench.h"

namespace gdn {

// Sets the thread-local reason and returns `st`.
gdn_status fail(gdn_status st, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
void clear_error();
int dtype_size(int32_t dtype);
gdn_status check_layer(const gdn_layer* layer);
gdn_status check_pool(const gdn_state_pool* pool);
gdn_status check_conv_layer(const gdn_conv_layer* layer);
gdn_status check_conv_cache(const gdn_conv_cache* cache, const gdn_conv_layer* layer);

}  // namespace gdn
