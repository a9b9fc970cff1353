// Per-token coefficients of the expanded-softmax readout (d_k = 16, d_v = 64, orders 1 and 2).
#pragma once

#include "launch.hpp"

namespace taylor {

// Where the readout that follows takes its pieces and prefixes from, and where the coefficients go.
struct CenteredPlan {
  int L;               // piece length of the readout's plan
  long long nslot;     // slots per workspace row
  const float* slots;  // exclusive prefixes (after the scan) when multi, else unused
  int multi;           // 1: prefixes in slots; 0: each pair is one piece starting from a.state (or zero)
  const float* zc;     // per chunk of CH tokens (SeqMap::chunk_index): z of the piece's tokens before it
  int CH;              // chunk length of zc (32 or 64), dividing L
  float4* coef;        // [token-heads] (gamma_0, gamma_1, gamma_2, 0)
};

int centered_coef_launch(const PrefillArgs& a, const CenteredPlan& p);

}  // namespace taylor
