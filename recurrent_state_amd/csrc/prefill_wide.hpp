// MFMA prefill for wide feature sets (n = 4, 5 at d_k = 16, d_v = 64): feature blocks, float32 matrix cores.
#pragma once

#include "launch.hpp"

namespace taylor {

bool prefill_wide_has(int nt, int dk, int dv);
long long prefill_wide_ws_bytes(const Shape& s, int BH, int N);
int prefill_wide_launch(const PrefillArgs& a);

}  // namespace taylor
