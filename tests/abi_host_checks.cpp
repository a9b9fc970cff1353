// Host-side checks of the C ABI's validation, sizing and table export, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the library (tests/test_host_sanitizers.py links it
// against an instrumented build of api.cpp).  Every call here either returns before any HIP call or
// needs no device: the program runs on a machine without a GPU.  Buffers handed to the table export are
// heap blocks of exactly the size the call may write, so a write past the end is reported by ASan; the
// size queries are called at the edges of their ranges, so a signed overflow is reported by UBSan.
// Exit status 0 when every expectation holds; the failing line is printed otherwise.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../include/taylor_attn.h"

static int g_fail = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static taylor_config cfg(int n, int dk, int dv, int chunk = 0, float scale = 1.0f, int dt = TAYLOR_F32,
                         int readout = TAYLOR_READOUT_KERNEL) {
  taylor_config c;
  c.n_terms = n;
  c.d_k = dk;
  c.d_v = dv;
  c.chunk = chunk;
  c.scale = scale;
  c.in_dtype = dt;
  c.readout = readout;
  return c;
}

static long long binom(long long a, long long b) {
  long long r = 1;
  for (long long i = 1; i <= b; ++i) r = r * (a - b + i) / i;
  return r;
}

// An aligned address that is never dereferenced: it only reaches calls rejected for another reason.
static void* const FAKE = reinterpret_cast<void*>(uintptr_t(1) << 20);
static void* const MIS = reinterpret_cast<void*>((uintptr_t(1) << 20) + 4);

static void feature_width_and_sizes() {
  for (int n = 1; n <= 6; ++n)
    for (int d = 1; d <= 16; ++d) {
      long long w = 0;
      for (int m = 0; m < n; ++m) w += binom(d + m - 1, m);
      EXPECT(taylor_feature_width(n, d) == w);
    }
  // edges: the width overflows int long before n = 64 at d = 4096, and is rejected, not wrapped
  EXPECT(taylor_feature_width(64, 4096) == TAYLOR_ERR_INVALID_ARG);
  EXPECT(taylor_feature_width(3, 4096) == 1 + 4096 + 4096 * 4097 / 2);
  EXPECT(taylor_feature_width(0, 16) == TAYLOR_ERR_INVALID_ARG);
  EXPECT(taylor_feature_width(3, 0) == TAYLOR_ERR_INVALID_ARG);
  EXPECT(taylor_feature_width(3, 4097) == TAYLOR_ERR_INVALID_ARG);
  EXPECT(taylor_feature_width(65, 1) == TAYLOR_ERR_INVALID_ARG);
  EXPECT(taylor_feature_width(-2147483647 - 1, -2147483647 - 1) == TAYLOR_ERR_INVALID_ARG);

  taylor_config c = cfg(3, 16, 64);
  EXPECT(taylor_state_elems(&c) == 153 * 65);
  EXPECT(taylor_state_stride(&c) >= 153 * 65 && taylor_state_stride(&c) % 4 == 0);
  EXPECT(taylor_state_elems(nullptr) == TAYLOR_ERR_INVALID_ARG);
  taylor_config huge = cfg(5, 4096, 65536);
  EXPECT(taylor_state_elems(&huge) == TAYLOR_ERR_INVALID_ARG);  // W itself exceeds int
  taylor_config nan_scale = cfg(3, 16, 64, 0, NAN);
  EXPECT(taylor_state_elems(&nan_scale) == TAYLOR_ERR_INVALID_ARG);

  // workspace queries at the edges of the sizes: rejected or sized, never an overflowed product
  const int big = 2147483647;
  EXPECT(taylor_prefill_workspace_bytes(&c, big, big, big) < 0);
  EXPECT(taylor_prefill_workspace_bytes(&c, 1, big, 64) < 0);
  EXPECT(taylor_prefill_workspace_bytes(&c, 1, 1, big) != 0);
  EXPECT(taylor_prefill_workspace_bytes(&c, -1, 1, 64) == TAYLOR_ERR_INVALID_ARG);
  EXPECT(taylor_prefill_workspace_bytes(&c, 1, 8, 4096) > 0);
  EXPECT(taylor_prefill_backward_workspace_bytes(&c, big, big, big) < 0);
  EXPECT(taylor_prefill_backward_workspace_bytes(&c, 4, 16, 8192) > 0);
  const int64_t tmax = INT64_MAX;
  EXPECT(taylor_prefill_varlen_workspace_bytes(&c, big, big, big, tmax) < 0);
  EXPECT(taylor_prefill_varlen_workspace_bytes(&c, 4, 2, 100, 401) == TAYLOR_ERR_INVALID_ARG);
  EXPECT(taylor_prefill_varlen_workspace_bytes(&c, 4, 2, 100, 300) >= 0);
  for (int n = 1; n <= 5; ++n) {
    taylor_config b = cfg(n, 16, 64, 0, 1.0f, TAYLOR_BF16);
    EXPECT(taylor_supported(&b) == TAYLOR_OK);
    EXPECT(taylor_prefill_chunk(&b) > 0);
    EXPECT(taylor_prefill_workspace_bytes(&b, 4, 16, 8192) >= 0);
  }
  for (int s = -3; s <= 3; ++s) EXPECT(taylor_status_string(s) != nullptr);
}

static void monomial_tables() {
  for (int n = 1; n <= 5; ++n)
    for (int d = 1; d <= 16; ++d) {
      const int W = taylor_feature_width(n, d);
      const int width = n - 1 > 1 ? n - 1 : 1;
      // exactly W rows: ASan reports any write past them
      int32_t* idx = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * W * width));
      double* coef = static_cast<double*>(std::malloc(sizeof(double) * W));
      EXPECT(taylor_monomial_table(n, d, idx, coef, (size_t)W) == W);
      // every row: non-decreasing coordinates in [0, d), -1 padding after them, coefficient 1/sqrt(alpha!)
      int prev_order = 0;
      for (int a = 0; a < W; ++a) {
        int m = 0;
        while (m < width && idx[a * width + m] >= 0) ++m;
        for (int p = m; p < width; ++p) EXPECT(idx[a * width + p] == -1);
        for (int p = 0; p < m; ++p) EXPECT(idx[a * width + p] < d && (p == 0 || idx[a * width + p - 1] <= idx[a * width + p]));
        EXPECT(m >= prev_order);
        prev_order = m;
        double fact = 1.0;
        int run = 1;
        for (int p = 1; p <= m; ++p) {
          if (p < m && idx[a * width + p] == idx[a * width + p - 1]) {
            ++run;
            fact *= run;
          } else {
            run = 1;
          }
        }
        EXPECT(std::fabs(coef[a] - 1.0 / std::sqrt(fact)) <= 1e-15);
      }
      EXPECT(taylor_monomial_table(n, d, idx, coef, (size_t)W - 1) == TAYLOR_ERR_INVALID_ARG);
      EXPECT(taylor_monomial_table(n, d, nullptr, coef, (size_t)W) == W);
      EXPECT(taylor_monomial_table(n, d, idx, nullptr, (size_t)W) == W);
      std::free(idx);
      std::free(coef);
    }
  EXPECT(taylor_monomial_table(0, 16, nullptr, nullptr, 0) == TAYLOR_ERR_INVALID_ARG);
  EXPECT(taylor_monomial_table(9, 16, nullptr, nullptr, 1u << 30) == TAYLOR_ERR_INVALID_ARG);
}

static void entry_point_validation() {
  const int E = TAYLOR_ERR_INVALID_ARG, U = TAYLOR_ERR_UNSUPPORTED;
  taylor_config c = cfg(3, 16, 64, 64);
  taylor_config bad_chunk = cfg(3, 16, 64, 96);
  taylor_config seven = cfg(7, 16, 64);
  taylor_config bad_dtype = cfg(3, 16, 64, 0, 1.0f, 5);
  taylor_config bad_readout = cfg(3, 16, 64, 0, 1.0f, TAYLOR_F32, 9);
  float* F = static_cast<float*>(FAKE);
  float* M = static_cast<float*>(MIS);

  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, F, F, FAKE, 1, 1, 64, nullptr, nullptr) == E);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, nullptr, nullptr, FAKE, 1, 1, 64, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, F, F, FAKE, -1, 1, 64, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill(MIS, FAKE, FAKE, F, F, FAKE, 1, 1, 64, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, M, F, FAKE, 1, 1, 64, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, F, F, nullptr, 1, 1, 64, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, F, F, FAKE, 1, 1, 64, &bad_chunk, nullptr) == U);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, F, F, FAKE, 1, 1, 64, &seven, nullptr) == U);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, F, F, FAKE, 1, 1, 64, &bad_dtype, nullptr) == E);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, F, F, FAKE, 1, 1, 64, &bad_readout, nullptr) == E);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, F, F, FAKE, 2147483647, 2147483647, 2147483647, &c, nullptr) < 0);
  EXPECT(taylor_attn_prefill(FAKE, FAKE, FAKE, F, F, nullptr, 1, 1, 0, &c, nullptr) == TAYLOR_OK);  // no launch

  EXPECT(taylor_attn_prefill_into(FAKE, FAKE, FAKE, F, M, F, FAKE, 1, 1, 64, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill_into(FAKE, FAKE, FAKE, F, F, F + 4, FAKE, 2, 2, 64, &c, nullptr) == E);  // overlap
  EXPECT(taylor_attn_prefill_into(FAKE, FAKE, FAKE, F, F, F, nullptr, 1, 1, 64, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill_into(FAKE, FAKE, FAKE, F, F, F, nullptr, 0, 4, 64, &c, nullptr) == TAYLOR_OK);

  taylor_config f5 = cfg(5, 16, 64, 0, 1.0f, TAYLOR_F32);
  EXPECT(taylor_attn_prefill_into_static(FAKE, FAKE, FAKE, F, nullptr, F, 1, 16, 16384, &f5, nullptr) == E);
  EXPECT(taylor_attn_prefill_into_static(FAKE, FAKE, FAKE, F, nullptr, F, 1, 1, 64, nullptr, nullptr) == E);

  int32_t* cu = static_cast<int32_t*>(FAKE);
  EXPECT(taylor_attn_prefill_varlen(FAKE, FAKE, FAKE, F, F, FAKE, cu, 4, 2, 100, 401, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill_varlen(FAKE, FAKE, FAKE, F, F, FAKE, nullptr, 4, 2, 100, 300, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill_varlen(FAKE, FAKE, FAKE, F, F, FAKE, cu, -4, 2, 100, 300, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill_varlen(FAKE, FAKE, FAKE, F, F, nullptr, nullptr, 4, 2, 100, 0, &c, nullptr) == TAYLOR_OK);
  EXPECT(taylor_attn_prefill_varlen_into(FAKE, FAKE, FAKE, F, M, F, FAKE, cu, 4, 2, 100, 300, &c, nullptr) == E);

  EXPECT(taylor_attn_prefill_backward(FAKE, FAKE, FAKE, F, F, F, F, F, F, F, FAKE, -1, 1, 64, &c, nullptr) == E);
  EXPECT(taylor_attn_prefill_backward(FAKE, FAKE, FAKE, F, F, F, F, F, F, F, FAKE, 1, 1, 64, nullptr, nullptr) == E);
  EXPECT(taylor_attn_prefill_backward(FAKE, FAKE, FAKE, F, F, F, F, F, F, F, FAKE, 1, 1, 64, &seven, nullptr) == U);

  EXPECT(taylor_attn_decode_step(FAKE, FAKE, FAKE, F, F, 1, 1, nullptr, nullptr) == E);
  EXPECT(taylor_attn_decode_step(MIS, FAKE, FAKE, F, F, 1, 1, &c, nullptr) == E);
  EXPECT(taylor_attn_decode_step(FAKE, FAKE, FAKE, F, M, 1, 1, &c, nullptr) == E);
  EXPECT(taylor_attn_decode_step(FAKE, FAKE, FAKE, F, F, -1, 1, &c, nullptr) == E);
  EXPECT(taylor_attn_decode_step(FAKE, FAKE, FAKE, F, F, 1, 1, &seven, nullptr) == U);

  EXPECT(taylor_state_init(F, -1, 1, &c, nullptr) == E);
  EXPECT(taylor_state_init(M, 1, 1, &c, nullptr) == E);
  EXPECT(taylor_state_init(F, 1, 1, nullptr, nullptr) == E);
}

int main() {
  feature_width_and_sizes();
  monomial_tables();
  entry_point_validation();
  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host ABI checks passed\n");
  return 0;
}
