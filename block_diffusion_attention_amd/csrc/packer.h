// Host packer: replay rows from captured states, largest-cost-first group assignment.
#pragma once
#include <stdint.h>

#include <string>

#include "../../include/bd_attn.h"

namespace bdattn {

// Validates desc and fills *out (caller-owned arrays). On error returns a
// non-OK status, sets *err and leaves the outputs unspecified.
bd_attn_status build_pack(const bd_pack_desc* desc, bd_pack_out* out, std::string* err);

}  // namespace bdattn
