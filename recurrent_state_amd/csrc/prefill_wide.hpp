// Feature-block MFMA prefill (d_k = 16, d_v = 64): n = 4, 5 for any input type, n = 1..3 for float32
// inputs; float32 matrix cores.
#pragma once

#include "launch.hpp"

namespace taylor {

bool prefill_wide_has(int nt, int dk, int dv, int dtype);
long long prefill_wide_ws_bytes(const Shape& s, int BH, const SeqMap& seq);
int prefill_wide_launch(const PrefillArgs& a);

}  // namespace taylor
