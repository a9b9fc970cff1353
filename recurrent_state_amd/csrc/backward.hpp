// Backward of truncated-kernel causal attention (d_k = 16, d_v = 64, n = 1..5).
#pragma once

#include "launch.hpp"

namespace taylor {

struct BwdArgs {
  Shape s;
  const void *q, *k, *v;
  const float *o, *g;  // forward outputs and their gradient
  const float* state;  // the forward call's incoming state, or null (empty history)
  float* dstate;       // in: gradient of the final state (or null: zero); out: of the incoming state
  float *dq, *dk, *dv;
  void* ws;
  int BH, N;
  hipStream_t stream;
};

struct BwdPlan {
  int L, nseg;  // segment length (a multiple of the 16-token chunk) and segments per pair
};

bool backward_has(int nt, int dk, int dv);
long long backward_ws_bytes(const Shape& s, int BH, int N);
int backward_launch(const BwdArgs& a);

// n = 4, 5 (backward_wide.hip): feature blocks with per-block partial gradients.
long long backward_wide_ws_bytes(const Shape& s, int BH, int N);
int backward_wide_launch(const BwdArgs& a);

}  // namespace taylor
