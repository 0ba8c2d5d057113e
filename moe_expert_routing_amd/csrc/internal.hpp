// internal.hpp - declarations shared by the library's translation units.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_route.h"

namespace moe {

// Host-side validation of a routing call (no device access). Returns MOE_OK
// and the output id space in *e_out, or a negative moe_status.
int validate_route_call(const float *logits, const float *bias, int32_t T,
                        const moe_route_params *prm, int32_t off, int32_t cnt,
                        const moe_route_outputs *o, const void *workspace, size_t ws_bytes,
                        int *e_out);

}  // namespace moe
