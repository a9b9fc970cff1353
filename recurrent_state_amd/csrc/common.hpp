// Shared compile-time tables and device helpers for the Taylor-attention kernels (gfx950).
//
// The monomial features follow "Expanding Attention: A Taylor-Series Route to
// Linear-Time Transformers with a Fixed Number of Recurrent States" (Huang,
// arXiv:2610.20637), Abstract: the m-th Taylor term (s^m/m!) is an inner
// product of m-th tensor powers, and by symmetry only binom(d+m-1, m) distinct
// monomials remain.  Feature alpha of order m is x^alpha / sqrt(alpha!), which
// puts the multiplicity m!/alpha! and the 1/m! of the Taylor term half on each
// side, so <phi_m(q), phi_m(k)> = (q.k)^m / m!.
//
// Feature order: orders m = 0..n-1 ascending; within an order, non-decreasing
// coordinate tuples (i_1 <= ... <= i_m) in lexicographic order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace taylor {

constexpr int kMaxTerms = 5;  // orders 0..4: coordinate tuples of length <= 4

constexpr long long binom(int n, int k) {
  if (k < 0 || k > n) return 0;
  long long r = 1;
  for (int i = 1; i <= k; ++i) r = r * (n - k + i) / i;
  return r;
}

// W = sum_{m<n} binom(d+m-1, m).
constexpr long long feature_width_ll(int n_terms, int d) {
  long long w = 0;
  for (int m = 0; m < n_terms; ++m) w += binom(d + m - 1, m);
  return w;
}

// Enumerates the features of (n_terms, d) in table order and calls
// f(index, order m, coordinates t[0..m-1], alpha!) for each.  Used both at
// compile time (the device tables) and at run time (the host export), so the
// two cannot disagree.
template <class F>
__host__ __device__ constexpr int for_each_monomial(int n_terms, int d, F&& f) {
  int a = 0;
  for (int m = 0; m < n_terms; ++m) {
    int t[kMaxTerms] = {0, 0, 0, 0, 0};
    while (true) {
      int af = 1, run = 1;
      for (int p = 1; p < m; ++p) {
        run = (t[p] == t[p - 1]) ? run + 1 : 1;
        af *= run;
      }
      f(a, m, t, af);
      ++a;
      int p = m - 1;  // advance to the next non-decreasing tuple
      while (p >= 0 && t[p] == d - 1) --p;
      if (p < 0) break;
      ++t[p];
      for (int r = p + 1; r < m; ++r) t[r] = t[p];
    }
  }
  return a;
}

// Compile-time monomial table for (n_terms, d).  coord[a] lists the coordinates
// of feature a (-1 padded); afact[a] = alpha! = prod_i alpha_i!, which for
// orders <= 4 is one of 1, 2, 4, 6, 24.
template <int NT, int DK>
struct Monomials {
  static_assert(NT >= 1 && NT <= kMaxTerms, "1..5 Taylor terms");
  static constexpr int W = (int)feature_width_ll(NT, DK);
  int8_t coord[W][4];
  uint8_t order[W];
  uint8_t afact[W];
  constexpr Monomials() : coord{}, order{}, afact{} {
    for_each_monomial(NT, DK, [this](int a, int m, const int* t, int af) {
      for (int p = 0; p < 4; ++p) coord[a][p] = (int8_t)(p < m ? t[p] : -1);
      order[a] = (uint8_t)m;
      afact[a] = (uint8_t)af;
    });
  }
};

// 1/sqrt(alpha!) rounded to float32, for the alpha! values orders <= 4 produce.
__host__ __device__ constexpr float coef_of_afact(int afact) {
  return afact == 1   ? 1.0f
         : afact == 2 ? (float)0.70710678118654752440
         : afact == 4 ? 0.5f
         : afact == 6 ? (float)0.40824829046386301637
                      : (float)0.20412414523193150819;  // 24
}

template <int NT, int DK>
__constant__ Monomials<NT, DK> kMono = Monomials<NT, DK>();

// phi_a(x) for x in LDS or registers (float32): coefficient times the product of its coordinates.
template <int NT, int DK>
__device__ __forceinline__ float feature_at(const float* x, int a) {
  const Monomials<NT, DK>& T = kMono<NT, DK>;
  float f = coef_of_afact(T.afact[a]);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = T.coord[a][p];
    if (p < NT - 1 && c >= 0) f *= x[c];
  }
  return f;
}

// Element loads: float32 as is, bfloat16 (stored as raw uint16) widened exactly.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// K_n(s) = sum_{m<n} s^m/m! by Horner's rule: 1 + s(1 + s/2(1 + s/3(...))).
template <int NT>
__device__ __forceinline__ float taylor_kernel(float s) {
  float acc = 1.0f;
#pragma unroll
  for (int m = NT - 1; m >= 1; --m) acc = fmaf(acc * s, 1.0f / (float)m, 1.0f);
  return acc;
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
__device__ __forceinline__ float4 fma4(float s, float4 a, float4 c) {
  return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z), fmaf(s, a.w, c.w));
}

}  // namespace taylor
