// Pipelined bfloat16 MFMA prefill (gfx950) for d_k = 16, d_v = 64, n = 1..3.
#pragma once

#include "launch.hpp"

namespace taylor {

bool prefill_mfma_has(int nt, int dk, int dv, int dtype);
long long prefill_mfma_ws_bytes(const Shape& s, int BH, const SeqMap& seq);
int prefill_mfma_launch(const PrefillArgs& a);

}  // namespace taylor
