// Internal launch interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace taylor {

struct Shape {
  int nt;       // Taylor terms
  int dk, dv;   // head dims
  int dtype;    // 0 = float32, 1 = bfloat16 inputs
  float scale;  // score scale
  long long W;       // feature width
  long long stride;  // floats per head block in the state
};

struct DecodeArgs {
  Shape s;
  const void *q, *k, *v;
  float* o;
  float* state;
  int BH;
  hipStream_t stream;
};

struct PrefillArgs {
  Shape s;
  const void *q, *k, *v;
  float* o;        // may be null (state-only)
  float* state;    // may be null (start from zero, discard)
  void* ws;        // workspace
  int BH, N, C;    // heads, tokens, chunk
  hipStream_t stream;
};

// Each returns 0 on success, -2 if the shape has no compiled kernel, -3 on a launch error.
int decode_launch(const DecodeArgs& a);
bool decode_has(int nt, int dk, int dv);

int state_zero_launch(float* state, long long count, hipStream_t stream);

// Exclusive prefix over `nseg` consecutive state blocks per head in `ws` (seeded with `state` when
// non-null, else zero); the total is written to `state` when non-null.  Only the first `elems`
// floats of each block are touched.
int seg_scan_launch(float* ws, float* state, int BH, int nseg, long long stride, long long elems, bool write_prefix,
                    hipStream_t stream);

// Portable prefill path (any compiled (n, d_k, d_v), chunk 64 or 128), VALU float32.
bool prefill_generic_has(int nt, int dk, int dv, int C);
long long prefill_generic_ws_bytes(const Shape& s, int BH, int N, int C);
int prefill_generic_launch(const PrefillArgs& a);

}  // namespace taylor
