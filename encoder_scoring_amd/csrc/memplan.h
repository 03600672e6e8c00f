// Offset planning of a pass's intermediate tensors (memplan.cpp).
#pragma once

#include <cstdint>
#include <vector>

namespace es {

// One tensor of a pass: bytes, and the first and last step that touches it.
struct Usage {
  int64_t bytes;
  int32_t first, last;
};

// Offsets (aligned to `align`, a power of two) such that records whose step
// intervals meet never share bytes; returns the bytes the arena needs.
int64_t plan_arena(const std::vector<Usage> &u, int64_t align, std::vector<int64_t> &offset);

}  // namespace es
