// Compile-time monomial features of a register-resident coordinate vector (the MFMA prefill kernels).
//
// Feature A of order m is x^alpha / sqrt(alpha!) ("Expanding Attention", Huang, arXiv:2610.20637,
// Abstract: the m-th Taylor term is an inner product of symmetric tensor powers); its coordinates and
// coefficient are fixed at compile time from the table order of common.hpp, so each feature costs
// one multiplication per coordinate and no table lookup.
#pragma once

#include "common.hpp"

namespace taylor {

template <int NT, int DK>
struct FeatureTable {
  static constexpr Monomials<NT, DK> T{};
  static constexpr int W = Monomials<NT, DK>::W;
};

// Feature A of x (float32 registers); zero for A >= W (padding rows of a feature block).
template <int NT, int DK, int A>
__device__ __forceinline__ float feature_ct(const float (&x)[DK]) {
  if constexpr (A >= FeatureTable<NT, DK>::W) {
    return 0.f;
  } else {
    constexpr int c0 = FeatureTable<NT, DK>::T.coord[A][0];
    constexpr int c1 = FeatureTable<NT, DK>::T.coord[A][1];
    constexpr int c2 = FeatureTable<NT, DK>::T.coord[A][2];
    constexpr int c3 = FeatureTable<NT, DK>::T.coord[A][3];
    constexpr float cf = coef_of_afact(FeatureTable<NT, DK>::T.afact[A]);
    float f = cf;
    if constexpr (c0 >= 0) f *= x[c0];
    if constexpr (c1 >= 0) f *= x[c1];
    if constexpr (c2 >= 0) f *= x[c2];
    if constexpr (c3 >= 0) f *= x[c3];
    return f;
  }
}

// Calls f(std::integral_constant<int, I>{}) for the I in [LO, HI) equal to i (i uniform across the
// wavefront, so the search is a few scalar branches).
template <int LO, int HI, class F>
__device__ __forceinline__ void dispatch_index(int i, F&& f) {
  if constexpr (HI - LO == 1) {
    f(std::integral_constant<int, LO>{});
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (i < MID)
      dispatch_index<LO, MID>(i, f);
    else
      dispatch_index<MID, HI>(i, f);
  }
}

}  // namespace taylor
