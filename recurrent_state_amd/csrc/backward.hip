// Backward of truncated-kernel causal attention (gfx950): dq, dk, dv and the gradient of the incoming
// state; float32 matrix cores, and for bfloat16 inputs bfloat16 matrix cores on exact products.
//
// The forward is the method of "Expanding Attention" (Huang, arXiv:2610.20637), Abstract; the pages
// give no gradients, so they are derived here.  With w_ij = K_n(s_ij), s_ij = a_i . k_j, a = sigma q,
// den_i = sum_{j<=i} w_ij (plus phi(a_i) . z0 from an incoming state) and g_i = dL/do_i, write
// gh_i = g_i / den_i and delta_i = g_i . o_i / den_i.  Then
//     dw_ij = gh_i . v_j - delta_i,   ds_ij = dw_ij K_{n-1}(s_ij)
//     dv_j = sum_{i>=j} w_ij gh_i,   dq_i = sigma sum_{j<=i} ds_ij k_j,   dk_j = sigma sum_{i>=j} ds_ij q_i.
// Across chunks the sums factor through states.  The forward states S, z of the tokens before a
// chunk give, for its tokens,
//     dq_i += sigma J_phi(a_i)^T (S gh_i - delta_i z),
// and reverse-time states G_S = sum_{i later} phi(a_i) gh_i^T, G_z = -sum_{i later} phi(a_i) delta_i
// (the gradient of the state at that point) give
//     dv_j += G_S^T phi(k_j),   dk_j += J_phi(k_j)^T (G_S v_j + G_z).
// G at the start of the call is the incoming state's gradient; a gradient for the final state seeds
// G at the end.  J_phi is the Jacobian of the monomial features (orders <= 2 here: n <= 3; n = 4, 5
// run on feature blocks in backward_wide.hip).
//
// Passes over segments of L tokens (one workgroup of 8 wavefronts per segment, 64-token chunks):
//   1. state pass: the S, z increments of each segment;
//   2. forward scan: exclusive prefixes, seeded with the incoming state;
//   3. pass A (chunks in order): den, gh, delta (kept for pass B), dq, the segment's G increments;
//   4. reverse scan of the G increments, seeded with the final state's gradient (its total is the
//      incoming state's gradient);
//   5. pass B (chunks in reverse): dv, dk.
//
// Layout.  Features are split into 16-row tiles; wavefront w owns tiles w and w + 8 and keeps their
// rows of S and G in float32 MFMA accumulators for the whole segment, transposed (the lane holding
// feature f = 16 ft + l16 and value columns d = 16 dt + 4 lg + r), which is exactly the A operand of a
// product that contracts over d (S gh in pass A, G v in pass B).  The feature operands of the state
// updates are formed as the products are issued: each lane's feature is fixed, so phi_f(x_t) is a
// coefficient times two entries of the row of x_t, whose columns 16 and 17 hold ones (orders 0 and 1)
// and 18 a zero (padding features); nothing of phi is stored.  Intra-chunk score tiles stay in
// registers from the scores to the products that consume them: in pass A a tile [key j][query i] is
// the A operand of ds k over j; in pass B a tile [query i][key j] is the A operand of w^T gh and
// ds^T a over i.  dv in pass B contracts G over the features, so the owners copy G into LDS once per
// chunk and every wavefront reads it for two 16x16 tiles of dv.  The feature Jacobians run with one
// lane per token over the wavefront's own (compile-time) features; each wavefront leaves its partial
// dq (dk) rows in its own LDS rows, summed after the chunk.
//
// bfloat16 inputs.  v is exact in bfloat16, and so is the hi + lo pair of a feature without its
// coefficient (x_c0 x_c1 has at most 16 significant bits).  S += phi(K)^T V (state pass, pass A) then runs
// as two 16x16x16 bfloat16 MFMAs per 16 tokens with the same float32 products, the coefficient applied
// once (pass A keeps S_f / cf_f in its accumulators); G v (pass B) takes G as three bfloat16 terms
// (hi and mid in one 16x16x32 MFMA, lo in a second)
// (24 significant bits) against exact v.
#include <type_traits>
#include <utility>

#include "backward.hpp"
#include "features.hpp"

namespace taylor {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kDK = 16, kDV = 64;
constexpr int kC = 64;  // tokens per chunk
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLR = 20;  // a, k rows: 16 coordinates, two ones, two zeros
constexpr int kLV = 68;  // 64-wide rows and feature-major rows
constexpr int kOne0 = 16, kOne1 = 17, kZero = 18;
constexpr int kLP = 17;  // row stride of a wavefront's partial dq (dk) rows: 64 x 17 floats = its 16 rows

template <int NT>
struct BG {
  static constexpr int W = FeatureTable<NT, kDK>::W;
  static constexpr int NFT = (W + 15) / 16;                       // feature tiles
  static constexpr int WP = 16 * NFT;                             // padded features
  static constexpr int NU = (NFT + kWaves - 1) / kWaves;          // tiles per wavefront, at most
  static constexpr int NWF = NFT < kWaves ? NFT : kWaves;         // wavefronts owning tiles
  static constexpr int YR = WP > 16 * kWaves ? WP : 16 * kWaves;  // rows of a feature-major buffer
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// Two floats split into bfloat16 pairs hi = bf16(x), lo = bf16(x - hi) (nearest even).  For a product
// of two bfloat16 values (at most 16 significant bits) hi + lo is exact.
__device__ __forceinline__ void split_bf16x2(float a, float b, bf16x2& hi, bf16x2& lo) {
  hi = __builtin_convertvector(f32x2{a, b}, bf16x2);
  const uint32_t u = __builtin_bit_cast(uint32_t, hi);
  lo = __builtin_convertvector(f32x2{a - __uint_as_float(u << 16), b - __uint_as_float(u & 0xffff0000u)}, bf16x2);
}
// Four floats as three bfloat16 terms hi + mid + lo (each the nearest bfloat16 of what the previous
// terms leave): 24 significant bits, a float32 value to within a unit of its last place.
__device__ __forceinline__ void split3(const f32x4& x, bf16x4& h, bf16x4& m, bf16x4& l) {
  bf16x2 hh[2], mm[2], ll[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float a = x[2 * p], b = x[2 * p + 1];
    hh[p] = __builtin_convertvector(f32x2{a, b}, bf16x2);
    const uint32_t uh = __builtin_bit_cast(uint32_t, hh[p]);
    const float ra = a - __uint_as_float(uh << 16), rb = b - __uint_as_float(uh & 0xffff0000u);
    mm[p] = __builtin_convertvector(f32x2{ra, rb}, bf16x2);
    const uint32_t um = __builtin_bit_cast(uint32_t, mm[p]);
    ll[p] = __builtin_convertvector(f32x2{ra - __uint_as_float(um << 16), rb - __uint_as_float(um & 0xffff0000u)},
                                    bf16x2);
  }
  h = bf16x4{hh[0][0], hh[0][1], hh[1][0], hh[1][1]};
  m = bf16x4{mm[0][0], mm[0][1], mm[1][0], mm[1][1]};
  l = bf16x4{ll[0][0], ll[0][1], ll[1][0], ll[1][1]};
}

// c + a0 b0 + a1 b1 as one 16x16x32 MFMA: lane group g supplies k = 8g..8g+7 of both operands, so the
// two 4-element halves pair up as the two products.  On gfx950 it takes the cycles of one 16x16x16.
__device__ __forceinline__ f32x4 mfma_bf16_pair(bf16x4 a0, bf16x4 a1, bf16x4 b0, bf16x4 b1, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                  __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), c, 0, 0, 0);
}
__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Feature f as (row offset c0) | (row offset c1) << 8: phi_f(x) = cf x[c0] x[c1] on an extended row.
template <int NT>
__device__ __forceinline__ int feature_code(int f) {
  if (f >= BG<NT>::W) return kZero | (kZero << 8);
  const Monomials<NT, kDK>& T = kMono<NT, kDK>;
  const int m = T.order[f];
  const int c0 = m == 0 ? kOne0 : T.coord[f][0];
  const int c1 = m == 0 ? kOne1 : (m == 1 ? kOne0 : T.coord[f][1]);
  return c0 | (c1 << 8);
}
struct LaneF {
  int o0, o1;
  float cf;  // 1/sqrt(2) for x_c^2 (and the zero padding), else 1
};
__device__ __forceinline__ LaneF unpack(int code) {
  LaneF r;
  r.o0 = code & 255;
  r.o1 = code >> 8;
  r.cf = r.o0 == r.o1 ? 0.70710678118654752f : 1.f;
  return r;
}
__device__ __forceinline__ float phi(const float* row, const LaneF& f) { return f.cf * row[f.o0] * row[f.o1]; }

// Element loads: pairs of q, k coordinates, eight-column slices of v (and of g, o, gh: float32).
__device__ __forceinline__ void ld2(const float* p, float (&x)[2]) {
  const f32x2 t = *reinterpret_cast<const f32x2*>(p);
  x[0] = t[0];
  x[1] = t[1];
}
__device__ __forceinline__ void ld2(const uint16_t* p, float (&x)[2]) {
  const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
  x[0] = __uint_as_float(u << 16);
  x[1] = __uint_as_float(u & 0xffff0000u);
}
__device__ __forceinline__ void ld8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}
__device__ __forceinline__ void ld8(const uint16_t* p, float (&x)[8]) {
  const uint4 t = *reinterpret_cast<const uint4*>(p);
  const uint32_t wd[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    x[2 * h] = __uint_as_float(wd[h] << 16);
    x[2 * h + 1] = __uint_as_float(wd[h] & 0xffff0000u);
  }
}

// LDS rows of one chunk.
struct Rows {
  float (*ax)[kLR];  // a = sigma q, extended (null in the state pass)
  float (*kx)[kLR];  // k, extended
  float (*v)[kLV];
  float (*g)[kLV];  // g (pass A) or gh (pass B)
  float* go;        // g . o per token (pass A)
  float* delta;     // delta per token (pass B)
  uint16_t (*vt)[kC + 8] = nullptr;  // bfloat16 inputs: V^T as raw bfloat16 (the exact products' operand)
  uint16_t (*vb)[kDV + 8] = nullptr;  // bfloat16 inputs: V rows as raw bfloat16
};

// One thread's share of a chunk's inputs, loaded a chunk ahead and stored to LDS when the chunk starts,
// so that the global loads of the next chunk are in flight while one is computed.  Thread tid takes
// token tid / 8: coordinates 2 (tid % 8) and + 1 of q and k, columns 8 (tid % 8) .. + 7 of v, g, o,
// gh.  Tokens past the end read the chunk's first row (no conditional load) and store zeros.
// MODE 0: k, v (state pass); 1: q, k, v, g, o (pass A); 2: q, k, v, gh, delta (pass B).
template <typename E, int MODE>
struct Pre {
  float qa[2], kk[2], vv[8], gg[8], oo[8], dl;
  __device__ __forceinline__ void load(const E* q, const E* k, const E* v, const float* g, const float* o,
                                       const float* dlt, long long tok0, int nv, int tid) {
    const int t = tid >> 3, c = tid & 7;
    const long long row = tok0 + (t < nv ? t : 0);
    ld2(k + row * kDK + 2 * c, kk);
    if constexpr (MODE != 0) ld2(q + row * kDK + 2 * c, qa);
    ld8(v + row * kDV + 8 * c, vv);
    if constexpr (MODE != 0) ld8(g + row * kDV + 8 * c, gg);
    if constexpr (MODE == 1) ld8(o + row * kDV + 8 * c, oo);
    if constexpr (MODE == 2) dl = dlt[tok0 + (tid < nv ? tid : 0)];
  }
  __device__ __forceinline__ void store(const Rows& R, int nv, float scale, int tid) const {
    const int t = tid >> 3, c = tid & 7;
    const bool ok = t < nv;
    const float one = ok ? 1.f : 0.f;
    *reinterpret_cast<f32x2*>(&R.kx[t][2 * c]) = f32x2{ok ? kk[0] : 0.f, ok ? kk[1] : 0.f};
    if (c == 0) *reinterpret_cast<f32x4*>(&R.kx[t][kDK]) = f32x4{one, one, 0.f, 0.f};
    if constexpr (MODE != 0) {
      *reinterpret_cast<f32x2*>(&R.ax[t][2 * c]) = f32x2{ok ? scale * qa[0] : 0.f, ok ? scale * qa[1] : 0.f};
      if (c == 0) *reinterpret_cast<f32x4*>(&R.ax[t][kDK]) = f32x4{one, one, 0.f, 0.f};
    }
    if (R.vt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) R.vt[8 * c + e][t] = ok ? (uint16_t)(__float_as_uint(vv[e]) >> 16) : (uint16_t)0;
    }
    if (R.vb) {
      uint32_t wd[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        wd[h] = ok ? (__float_as_uint(vv[2 * h]) >> 16) | (__float_as_uint(vv[2 * h + 1]) & 0xffff0000u) : 0u;
      *reinterpret_cast<uint4*>(&R.vb[t][8 * c]) = uint4{wd[0], wd[1], wd[2], wd[3]};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<f32x4*>(&R.v[t][8 * c + 4 * h]) =
          ok ? f32x4{vv[4 * h], vv[4 * h + 1], vv[4 * h + 2], vv[4 * h + 3]} : zero4();
      if constexpr (MODE != 0)
        *reinterpret_cast<f32x4*>(&R.g[t][8 * c + 4 * h]) =
            ok ? f32x4{gg[4 * h], gg[4 * h + 1], gg[4 * h + 2], gg[4 * h + 3]} : zero4();
    }
    if constexpr (MODE == 1) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(gg[e], oo[e], s);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      if (c == 0) R.go[t] = ok ? s : 0.f;
    }
    if constexpr (MODE == 2)
      if (tid < kC) R.delta[tid] = tid < nv ? dl : 0.f;
  }
};

// Feature of wavefront WW's share at position I (slot I / 16 is tile WW + 8 (I / 16)), or -1.
template <int NT, int WW, int I>
constexpr int own_feature() {
  constexpr int ft = WW + kWaves * (I / 16);
  constexpr int F = 16 * ft + I % 16;
  return (ft < BG<NT>::NFT && F < BG<NT>::W) ? F : -1;
}

// out += J_phi(x)^T y over wavefront WW's features, y_F = ycol[F * kLV] (orders <= 2): order 1 feature
// e_c adds y to out[c]; order 2 feature cf x_c0 x_c1 adds cf y x_c1 to out[c0] and cf y x_c0 to out[c1].
template <int NT, int WW>
__device__ __forceinline__ void own_vjp(const float (&x)[kDK], const float* ycol, float (&out)[kDK]) {
  using FT = FeatureTable<NT, kDK>;
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (([&] {
       constexpr int F = own_feature<NT, WW, I>();
       if constexpr (F >= 0) {
         constexpr int m = FT::T.order[F];
         if constexpr (m == 1) {
           out[FT::T.coord[F][0]] += ycol[F * kLV];
         } else if constexpr (m == 2) {
           constexpr int c0 = FT::T.coord[F][0], c1 = FT::T.coord[F][1];
           constexpr float cf = coef_of_afact(FT::T.afact[F]);
           const float t = cf * ycol[F * kLV];
           out[c0] = fmaf(t, x[c1], out[c0]);
           out[c1] = fmaf(t, x[c0], out[c1]);
         }
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, 16 * BG<NT>::NU>{});
}

// Sum over wavefront WW's features of phi_F(x) z_F.
template <int NT, int WW>
__device__ __forceinline__ float own_dot(const float (&x)[kDK], const float* z) {
  float acc = 0.f;
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (([&] {
       constexpr int F = own_feature<NT, WW, I>();
       if constexpr (F >= 0) acc = fmaf(feature_ct<NT, kDK, F>(x), z[F], acc);
     }()),
     ...);
  }(std::make_integer_sequence<int, 16 * BG<NT>::NU>{});
  return acc;
}

__device__ __forceinline__ void load_coords(const float* row, float (&x)[kDK]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(row + 4 * u);
    x[4 * u] = t[0];
    x[4 * u + 1] = t[1];
    x[4 * u + 2] = t[2];
    x[4 * u + 3] = t[3];
  }
}

// Runs f with the number of feature-tile slots this wavefront owns as a compile-time constant, so
// that the per-slot work of a phase has no branches inside its unrolled loops.
template <int NU, class F>
__device__ __forceinline__ void with_slots(bool two, F&& f) {
  if constexpr (NU > 1) {
    if (two)
      f(std::integral_constant<int, 2>{});
    else
      f(std::integral_constant<int, 1>{});
  } else {
    f(std::integral_constant<int, 1>{});
  }
}

// acc[u][dt] += sum over the chunk's tokens t of A[t][16 dt + l16] sw(t) phi_f(x_t), f the lane's feature
// of slot u (the transposed state tiles), and zs[u] += sum_t phi_f(x_t) zw(t) over this lane's tokens,
// for the first NA slots.  Tokens of the contraction: t = 16 qq + 4 lg + r at step (qq, r).
template <int NA, int UNR = 2, int NU, class SW, class ZW>
__device__ __forceinline__ void state_update(f32x4 (&acc)[NU][4], float (&zs)[NU], const float (*A)[kLV],
                                             const float (*X)[kLR], const LaneF (&lf)[NU], int l16, int lg, SW sw,
                                             ZW zw) {
#pragma unroll UNR
  for (int qq = 0; qq < 4; ++qq)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * qq + 4 * lg + r;
      const float s = sw(t), z = zw(t);
      float b[NA];
#pragma unroll
      for (int u = 0; u < NA; ++u) {
        const float p = phi(&X[t][0], lf[u]);
        b[u] = p * s;
        zs[u] = fmaf(p, z, zs[u]);
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const float a = A[t][16 * dt + l16];
#pragma unroll
        for (int u = 0; u < NA; ++u) acc[u][dt] = mfma(a, b[u], acc[u][dt]);
      }
    }
}

// bfloat16 inputs: acc[u][dt] += sum_t v[t][16 dt + l16] p_f(k_t) over the chunk's tokens, where
// p_f = x[c0] x[c1] is the feature without its coefficient (applied by the caller), a product of two
// bfloat16 values and so exactly hi + lo in bfloat16: two 16x16x16 bfloat16 MFMAs per 16 tokens give
// the float32 products exactly.  zs[u] += sum_t p_f(k_t) over this lane's tokens.  Tokens of the
// contraction at step qq: k = 4 lg + j <-> t = 16 qq + 4 lg + j.
template <int NA, int NU>
__device__ __forceinline__ void state_update_bf16(f32x4 (&acc)[NU][4], float (&zs)[NU], const uint16_t (*VT)[kC + 8],
                                                  const float (*X)[kLR], const LaneF (&lf)[NU], int l16, int lg) {
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int t0 = 16 * qq + 4 * lg;
    bf16x4 bh[NA], bl[NA];
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = X[t0 + j][lf[u].o0] * X[t0 + j][lf[u].o1];
        zs[u] += p[j];
      }
      bf16x2 h0, l0, h1, l1;
      split_bf16x2(p[0], p[1], h0, l0);
      split_bf16x2(p[2], p[3], h1, l1);
      bh[u] = bf16x4{h0[0], h0[1], h1[0], h1[1]};
      bl[u] = bf16x4{l0[0], l0[1], l1[0], l1[1]};
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const i16x4 a = *reinterpret_cast<const i16x4*>(&VT[16 * dt + l16][t0]);
#pragma unroll
      for (int u = 0; u < NA; ++u) {
        const bf16x4 ab = __builtin_bit_cast(bf16x4, a);
        acc[u][dt] = mfma_bf16_pair(ab, ab, bh[u], bl[u], acc[u][dt]);
      }
    }
  }
}

// Sum of the eight wavefronts' partial rows (dq or dk) of a finished chunk, times `mul`.
__device__ __forceinline__ void reduce_rows(const float (*buf)[kLV], float* out, long long tok0, int nv, float mul,
                                            int tid) {
  for (int e = tid; e < kC * kDK; e += kThreads) {
    const int i = e >> 4, d = e & 15;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) s += (&buf[16 * ww][0])[i * kLP + d];
    if (i < nv) out[(tok0 + i) * kDK + d] = mul * s;
  }
}

// dv tiles (jw, 2 hw + e) of a chunk: lane element r is dv[16 jw + 4 lg + r][16 (2 hw + e) + l16].
__device__ __forceinline__ void store_dv(const f32x4 (&t)[2], float* dv, long long tok0, int nv, int jw, int hw, int l16,
                                         int lg) {
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * jw + 4 * lg + r;
      if (j < nv) dv[(tok0 + j) * kDV + 16 * (2 * hw + e) + l16] = t[e][r];
    }
}

// ---------------------------------------------------------------------------------------------------
// 1. State pass: S, z increments of each segment.

struct SmemS {
  alignas(16) float kx[kC][kLR];
  alignas(16) float v[kC][kLV];
  alignas(16) uint16_t vt[kDV][kC + 8];  // bfloat16 inputs
};

template <int NT, typename E>
__global__ __launch_bounds__(kThreads) void bwd_state_kernel(const E* __restrict__ k, const E* __restrict__ v,
                                                             float* __restrict__ sslots, SeqMap seq, int L,
                                                             long long nslot, long long stride) {
  using G = BG<NT>;
  constexpr int W = G::W, NU = G::NU;
  __shared__ SmemS sm;
  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool BF = std::is_same_v<E, uint16_t>;
  const Rows R{nullptr, sm.kx, sm.v, nullptr, nullptr, nullptr, BF ? sm.vt : nullptr};
  LaneF lf[NU];
  bool has[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    lf[u] = unpack(feature_code<NT>(16 * (w + kWaves * u) + l16));
    has[u] = w + kWaves * u < G::NFT;
  }
  const bool two = NU > 1 && has[NU - 1];  // a second feature tile

  for_each_piece<false>(seq, blockIdx.x, blockIdx.y, L, nslot, [&](const SeqPiece& pc) __attribute__((always_inline)) {
    f32x4 st[NU][4];
    float zs[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      zs[u] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) st[u][dt] = zero4();
    }
    const int nch = (pc.n + kC - 1) / kC;
    auto nv_of = [&](int c) { return min(kC, pc.n - c * kC); };
    auto tok_of = [&](int c) { return pc.tok + (long long)c * kC; };
    Pre<E, 0> pre;
    pre.load(nullptr, k, v, nullptr, nullptr, nullptr, tok_of(0), nv_of(0), tid);
    for (int c = 0; c < nch; ++c) {
      pre.store(R, nv_of(c), 1.f, tid);
      const int cn = c + 1 < nch ? c + 1 : c;  // the last chunk reloads itself (no conditional load)
      pre.load(nullptr, k, v, nullptr, nullptr, nullptr, tok_of(cn), nv_of(cn), tid);
      __syncthreads();
      if (has[0]) {
        // S^T += V^T phi(K), z += sum phi(k)
        with_slots<NU>(two, [&](auto NAc) __attribute__((always_inline)) {
          if constexpr (BF)
            state_update_bf16<decltype(NAc)::value>(st, zs, sm.vt, sm.kx, lf, l16, lg);
          else
            state_update<decltype(NAc)::value, 4>(st, zs, sm.v, sm.kx, lf, l16, lg, [](int) { return 1.f; },
                                                  [](int) { return 1.f; });
        });
      }
      __syncthreads();
    }
    float* slot = sslots + pc.slot * stride;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int f = 16 * (w + kWaves * u) + l16;
      float z = zs[u];
      z += __shfl_xor(z, 16);
      z += __shfl_xor(z, 32);
      if constexpr (BF) {
        // the feature coefficient, left out of the products
        z *= lf[u].cf;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) st[u][dt] *= lf[u].cf;
      }
      if (has[u] && f < W) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(slot + (long long)f * kDV + 16 * dt + 4 * lg) = st[u][dt];
        if (lg == 0) slot[(long long)W * kDV + f] = z;
      }
    }
  });
}

// ---------------------------------------------------------------------------------------------------
// 3. Pass A: den, gh, delta, dq and the segment's G increments.

template <int NT>
struct SmemA {
  using G = BG<NT>;
  alignas(16) float y[G::YR][kLV];  // Y^T rows of each owner, then each wavefront's partial dq rows
  alignas(16) float ax[kC][kLR];
  alignas(16) float kx[kC][kLR];
  alignas(16) float v[kC][kLV];
  alignas(16) float g[kC][kLV];
  float denp[kWaves][kC];  // phi(a_i) . z over each owner's features
  float inv[kC], delta[kC], go[kC];
  float zt[G::WP];  // z before the chunk
  alignas(16) uint16_t vt[kDV][kC + 8];  // bfloat16 inputs
};

// Query-row tile of the intra-chunk work in pass A, by wavefront: waves 2, 3, 6, 7 own one feature
// tile each (0 and 1 own two), and the heavier rows go where the SIMD's other wavefront carries less.
__device__ __forceinline__ int row_of_wave(int w) {
  switch (w) {
    case 2: return 3;
    case 3: return 2;
    case 6: return 0;
    case 7: return 1;
    default: return -1;
  }
}

template <int NT, typename E>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                          const E* __restrict__ v, const float* __restrict__ g,
                                                          const float* __restrict__ o,
                                                          const float* __restrict__ sslots,
                                                          float* __restrict__ gslots, float* __restrict__ ghat,
                                                          float* __restrict__ dlt, float* __restrict__ dq,
                                                          SeqMap seq, int L, long long nslot, long long stride,
                                                          float scale) {
  using G = BG<NT>;
  constexpr int W = G::W, NU = G::NU;
  __shared__ SmemA<NT> sm;
  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = row_of_wave(w);
  // bfloat16 inputs: S += phi(K)^T V on exact bfloat16 products; the registers then hold S_f / cf_f
  // (cf_f the feature's coefficient), which the S gh product multiplies back
  constexpr bool BF = std::is_same_v<E, uint16_t>;
  const Rows R{sm.ax, sm.kx, sm.v, sm.g, sm.go, nullptr, BF ? sm.vt : nullptr};
  LaneF lf[NU];
  bool has[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    lf[u] = unpack(feature_code<NT>(16 * (w + kWaves * u) + l16));
    has[u] = w + kWaves * u < G::NFT;
  }
  const bool two = NU > 1 && has[NU - 1];  // a second feature tile
  float* part = &sm.y[16 * w][0];  // this wavefront's partial dq rows [token][coordinate]

  for_each_piece<false>(seq, blockIdx.x, blockIdx.y, L, nslot, [&](const SeqPiece& pc) __attribute__((always_inline)) {
    const float* sslot = sslots + pc.slot * stride;
    float* gslot = gslots + pc.slot * stride;
    f32x4 st[NU][4], gt[NU][4];
    float zf[NU], gzs[NU];  // z (one feature per lane) and this lane's share of sum phi(a) delta
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int f = 16 * (w + kWaves * u) + l16;
      const bool fv = has[u] && f < W;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        st[u][dt] = fv ? *reinterpret_cast<const f32x4*>(sslot + (long long)f * kDV + 16 * dt + 4 * lg) : zero4();
        if constexpr (BF) st[u][dt] *= 1.0f / lf[u].cf;
        gt[u][dt] = zero4();
      }
      zf[u] = fv ? sslot[(long long)W * kDV + f] : 0.f;
      gzs[u] = 0.f;
    }
    for (int f = tid; f < G::WP; f += kThreads) sm.zt[f] = f < W ? sslot[(long long)W * kDV + f] : 0.f;
    const int nch = (pc.n + kC - 1) / kC;
    auto nv_of = [&](int c) { return min(kC, pc.n - c * kC); };
    auto tok_of = [&](int c) { return pc.tok + (long long)c * kC; };
    Pre<E, 1> pre;
    pre.load(q, k, v, g, o, nullptr, tok_of(0), nv_of(0), tid);
    for (int c = 0; c < nch; ++c) {
      const int nv = nv_of(c);
      const long long tok0 = tok_of(c);
      pre.store(R, nv, scale, tid);
      if (c > 0) reduce_rows(sm.y, dq, tok_of(c - 1), nv_of(c - 1), scale, tid);
      const int cn = c + 1 < nch ? c + 1 : c;
      pre.load(q, k, v, g, o, nullptr, tok_of(cn), nv_of(cn), tid);
      __syncthreads();

      // Owners: phi(a_i) . z over their features, the part of den from before the chunk.
      if (has[0]) {
        dispatch_index<0, kWaves>(w, [&](auto WI) {
          constexpr int WW = decltype(WI)::value;
          if constexpr (WW < G::NWF) {
            float x[kDK];
            load_coords(&sm.ax[l][0], x);
            sm.denp[WW][l] = own_dot<NT, WW>(x, sm.zt);
          }
        });
      }
      // Row owners: scores [key j][query i] for key tiles jt <= row, weights, K_{n-1}, row sums.
      f32x4 kp[4];
      float dsum = 0.f;
      if (row >= 0) {
        const f32x4 aa = *reinterpret_cast<const f32x4*>(&sm.ax[16 * row + l16][4 * lg]);
        const int i = 16 * row + l16;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          kp[jt] = zero4();
          if (jt <= row) {
            const f32x4 ka = *reinterpret_cast<const f32x4*>(&sm.kx[16 * jt + l16][4 * lg]);
            f32x4 sc = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) sc = mfma(ka[s], aa[s], sc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * jt + 4 * lg + r;
              const bool ok = j <= i && i < nv;
              dsum += ok ? taylor_kernel<NT>(sc[r]) : 0.f;
              float d = 0.f;
              if constexpr (NT > 1) d = taylor_kernel<NT - 1>(sc[r]);
              kp[jt][r] = ok ? d : 0.f;
            }
          }
        }
        dsum += __shfl_xor(dsum, 16);
        dsum += __shfl_xor(dsum, 32);
      }
      __syncthreads();

      // Row owners: den, 1/den and delta of their 16 queries.
      float iv = 0.f, dl = 0.f;
      if (row >= 0) {
        const int i = 16 * row + l16;
        float den = dsum;
#pragma unroll
        for (int ww = 0; ww < G::NWF; ++ww) den += sm.denp[ww][i];
        iv = i < nv ? 1.0f / den : 0.f;
        dl = sm.go[i] * iv;
        if (lg == 0) {
          sm.inv[i] = iv;
          sm.delta[i] = dl;
        }
      }
      __syncthreads();

      if (has[0]) {
        with_slots<NU>(two, [&](auto NAc) __attribute__((always_inline)) {
          constexpr int NA = decltype(NAc)::value;
          // Y^T = S^T-tiles x g / den_i - z delta_i (S, z before the chunk) into the owner's rows
          float zp[NA][4];  // z[16 ft + 4 lg + r]
#pragma unroll
          for (int u = 0; u < NA; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) zp[u][r] = __shfl(zf[u], 4 * lg + r);
#pragma unroll 1
          for (int it = 0; it < 4; ++it) {
            f32x4 yr[NA];
#pragma unroll
            for (int u = 0; u < NA; ++u) yr[u] = zero4();
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              const f32x4 gv = *reinterpret_cast<const f32x4*>(&sm.g[16 * it + l16][16 * dt + 4 * lg]);
#pragma unroll
              for (int u = 0; u < NA; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) yr[u] = mfma(BF ? st[u][dt][r] * lf[u].cf : st[u][dt][r], gv[r], yr[u]);
            }
            const int i = 16 * it + l16;
            const float ivi = sm.inv[i], dli = sm.delta[i];
#pragma unroll
            for (int u = 0; u < NA; ++u)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                sm.y[16 * (w + kWaves * u) + 4 * lg + r][i] = yr[u][r] * ivi - zp[u][r] * dli;
          }
          // S^T += V^T phi(K), z += sum phi(k)
          float zs[NU];
#pragma unroll
          for (int u = 0; u < NU; ++u) zs[u] = 0.f;
          if constexpr (BF)
            state_update_bf16<NA>(st, zs, sm.vt, sm.kx, lf, l16, lg);
          else
            state_update<NA>(st, zs, sm.v, sm.kx, lf, l16, lg, [](int) { return 1.f; }, [](int) { return 1.f; });
#pragma unroll
          for (int u = 0; u < NA; ++u) {
            float z = zs[u];
            z += __shfl_xor(z, 16);
            z += __shfl_xor(z, 32);
            zf[u] += BF ? lf[u].cf * z : z;
            if (lg == 0) sm.zt[16 * (w + kWaves * u) + l16] = zf[u];
          }
          // G^T += g^T (phi(a) / den), and this lane's share of sum phi(a) delta
          state_update<NA>(gt, gzs, sm.g, sm.ax, lf, l16, lg, [&](int i) { return sm.inv[i]; },
                           [&](int i) { return sm.delta[i]; });
        });
        wave_fence();
        // J_phi(a_i)^T Y_i over the owner's features, one lane per query
        dispatch_index<0, kWaves>(w, [&](auto WI) {
          constexpr int WW = decltype(WI)::value;
          if constexpr (WW < G::NWF) {
            float x[kDK], out[kDK];
            load_coords(&sm.ax[l][0], x);
#pragma unroll
            for (int d = 0; d < kDK; ++d) out[d] = 0.f;
            own_vjp<NT, WW>(x, &sm.y[0][l], out);
            wave_fence();
#pragma unroll
            for (int d = 0; d < kDK; ++d) part[l * kLP + d] = out[d];
          }
        });
      } else {
#pragma unroll
        for (int d = 0; d < kDK; ++d) part[l * kLP + d] = 0.f;
      }
      if (row >= 0) {
        const int i = 16 * row + l16;
        // gh and delta for pass B
        if (i < nv) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x4 gv = *reinterpret_cast<const f32x4*>(&sm.g[i][16 * lg + 4 * e]);
            *reinterpret_cast<f32x4*>(ghat + (tok0 + i) * kDV + 16 * lg + 4 * e) = gv * iv;
          }
          if (lg == 0) dlt[tok0 + i] = dl;
        }
        // dw^T = v gh^T - delta, ds^T = dw^T K_{n-1}, dq += ds k over the key tiles jt <= row
        f32x4 gq[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) gq[qq] = *reinterpret_cast<const f32x4*>(&sm.g[i][16 * qq + 4 * lg]);
        f32x4 dqi = zero4();
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          if (jt <= row) {
            f32x4 dw = zero4();
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.v[16 * jt + l16][16 * qq + 4 * lg]);
#pragma unroll
              for (int r = 0; r < 4; ++r) dw = mfma(av[r], gq[qq][r], dw);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float ds = (dw[r] * iv - dl) * kp[jt][r];
              dqi = mfma(ds, sm.kx[16 * jt + 4 * lg + r][l16], dqi);
            }
          }
        }
        wave_fence();
#pragma unroll
        for (int r = 0; r < 4; ++r) part[(16 * row + 4 * lg + r) * kLP + l16] += dqi[r];
      }
      __syncthreads();
    }
    reduce_rows(sm.y, dq, tok_of(nch - 1), nv_of(nch - 1), scale, tid);
    // the segment's G increments
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int f = 16 * (w + kWaves * u) + l16;
      float z = gzs[u];
      z += __shfl_xor(z, 16);
      z += __shfl_xor(z, 32);
      if (has[u] && f < W) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(gslot + (long long)f * kDV + 16 * dt + 4 * lg) = gt[u][dt];
        if (lg == 0) gslot[(long long)W * kDV + f] = -z;
      }
    }
  });
}

// ---------------------------------------------------------------------------------------------------
// 5. Pass B: dv, dk, chunks in reverse, G (the gradient of the state after the chunk) in the owners'
// accumulators, seeded with the segment's suffix from the reverse scan.

template <int NT>
struct SmemB {
  using G = BG<NT>;
  alignas(16) float z[G::YR][kLV];   // Z^T rows of each owner, then each wavefront's partial dk rows
  alignas(16) float gm[G::WP][kLV];  // G [f][d], copied by the owners at the chunk start
  alignas(16) float ax[kC][kLR];
  alignas(16) float kx[kC][kLR];
  alignas(16) float v[kC][kLV];
  alignas(16) float gh[kC][kLV];
  float delta[kC];
  int code[G::WP];
  alignas(16) uint16_t vb[kC][kDV + 8];  // bfloat16 inputs
};

template <int NT, typename E>
__global__ __launch_bounds__(kThreads) void bwd_dkv_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                           const E* __restrict__ v,
                                                           const float* __restrict__ gslots,
                                                           const float* __restrict__ ghat,
                                                           const float* __restrict__ dlt, float* __restrict__ dk,
                                                           float* __restrict__ dv, SeqMap seq, int L,
                                                           long long nslot, long long stride, float scale) {
  using G = BG<NT>;
  constexpr int W = G::W, NU = G::NU, NFT = G::NFT;
  __shared__ SmemB<NT> sm;
  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // dv tiles (key tile jw, value tiles 2 hw and 2 hw + 1) with the intra-chunk part of key tile jw;
  // the wavefronts with hw = 1 also take dw, ds and ds^T a of that key tile.  The pairing puts the
  // heavy key tiles on the SIMDs whose other wavefront owns fewer feature tiles.
  const int jw = (0x23231010 >> (4 * w)) & 15, hw = (w >> 1) & 1;
  constexpr bool BF = std::is_same_v<E, uint16_t>;
  const Rows R{sm.ax, sm.kx, sm.v, sm.gh, nullptr, sm.delta, nullptr, BF ? sm.vb : nullptr};
  LaneF lf[NU];
  bool has[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    lf[u] = unpack(feature_code<NT>(16 * (w + kWaves * u) + l16));
    has[u] = w + kWaves * u < NFT;
  }
  const bool two = NU > 1 && has[NU - 1];  // a second feature tile
  for (int f = tid; f < G::WP; f += kThreads) sm.code[f] = feature_code<NT>(f);
  float* part = &sm.z[16 * w][0];  // this wavefront's partial dk rows [token][coordinate]

  for_each_piece<false>(seq, blockIdx.x, blockIdx.y, L, nslot, [&](const SeqPiece& pc) __attribute__((always_inline)) {
    const float* gslot = gslots + pc.slot * stride;
    f32x4 gt[NU][4];
    float gzf[NU];  // G_z, one feature per lane
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int f = 16 * (w + kWaves * u) + l16;
      const bool fv = has[u] && f < W;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        gt[u][dt] = fv ? *reinterpret_cast<const f32x4*>(gslot + (long long)f * kDV + 16 * dt + 4 * lg) : zero4();
      gzf[u] = fv ? gslot[(long long)W * kDV + f] : 0.f;
    }
    const int nch = (pc.n + kC - 1) / kC;
    auto nv_of = [&](int c) { return min(kC, pc.n - c * kC); };
    auto tok_of = [&](int c) { return pc.tok + (long long)c * kC; };
    Pre<E, 2> pre;
    pre.load(q, k, v, ghat, nullptr, dlt, tok_of(nch - 1), nv_of(nch - 1), tid);
    for (int c = nch - 1; c >= 0; --c) {
      const int nv = nv_of(c);
      const long long tok0 = tok_of(c);
      pre.store(R, nv, scale, tid);
      if (c < nch - 1) reduce_rows(sm.z, dk, tok_of(c + 1), nv_of(c + 1), 1.f, tid);
      if (has[0]) {
        with_slots<NU>(two, [&](auto NAc) __attribute__((always_inline)) {
#pragma unroll
          for (int u = 0; u < decltype(NAc)::value; ++u)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
              *reinterpret_cast<f32x4*>(&sm.gm[16 * (w + kWaves * u) + l16][16 * dt + 4 * lg]) = gt[u][dt];
        });
      }
      const int cn = c > 0 ? c - 1 : c;  // the first chunk reloads itself (no conditional load)
      pre.load(q, k, v, ghat, nullptr, dlt, tok_of(cn), nv_of(cn), tid);
      __syncthreads();

      if (has[0]) {
        with_slots<NU>(two, [&](auto NAc) __attribute__((always_inline)) {
          constexpr int NA = decltype(NAc)::value;
          // Z^T = G^T-tiles x v + G_z into the owner's rows
          if constexpr (BF) {
            // v is exact in bfloat16 and G enters as three bfloat16 terms: the lane's four accumulator
            // elements of value tile dt are its A operand of a 16-deep product over the value index
            f32x4 zt[NA][4];
#pragma unroll
            for (int u = 0; u < NA; ++u)
#pragma unroll
              for (int jt = 0; jt < 4; ++jt) zt[u][jt] = zero4();
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              bf16x4 gs3[NA][3];
#pragma unroll
              for (int u = 0; u < NA; ++u) split3(gt[u][dt], gs3[u][0], gs3[u][1], gs3[u][2]);
#pragma unroll
              for (int jt = 0; jt < 4; ++jt) {
                const bf16x4 vv = *reinterpret_cast<const bf16x4*>(&sm.vb[16 * jt + l16][16 * dt + 4 * lg]);
                // (hi, mid) and (lo, 0) as the k-halves of two 16x16x32 MFMAs against (v, v): only
                // 16x16x32s chain on zt (a 16x16x16 reading a 16x16x32 result right after it is a
                // pairing that gives wrong sums on gfx950)
#pragma unroll
                for (int u = 0; u < NA; ++u) {
                  zt[u][jt] = mfma_bf16_pair(gs3[u][0], gs3[u][1], vv, vv, zt[u][jt]);
                  zt[u][jt] = mfma_bf16_pair(gs3[u][2], bf16x4{}, vv, vv, zt[u][jt]);
                }
              }
            }
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
              for (int u = 0; u < NA; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  sm.z[16 * (w + kWaves * u) + 4 * lg + r][16 * jt + l16] = zt[u][jt][r] + __shfl(gzf[u], 4 * lg + r);
          } else {
#pragma unroll 1
            for (int jt = 0; jt < 4; ++jt) {
              f32x4 zt[NA];
#pragma unroll
              for (int u = 0; u < NA; ++u) zt[u] = zero4();
#pragma unroll
              for (int dt = 0; dt < 4; ++dt) {
                const f32x4 vv = *reinterpret_cast<const f32x4*>(&sm.v[16 * jt + l16][16 * dt + 4 * lg]);
#pragma unroll
                for (int u = 0; u < NA; ++u)
#pragma unroll
                  for (int r = 0; r < 4; ++r) zt[u] = mfma(gt[u][dt][r], vv[r], zt[u]);
              }
#pragma unroll
              for (int u = 0; u < NA; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  sm.z[16 * (w + kWaves * u) + 4 * lg + r][16 * jt + l16] = zt[u][r] + __shfl(gzf[u], 4 * lg + r);
            }
          }
          // G^T += gh^T phi(a), G_z -= phi(a)^T delta
          float gs[NU];
#pragma unroll
          for (int u = 0; u < NU; ++u) gs[u] = 0.f;
          state_update<NA, BF ? 2 : 4>(gt, gs, sm.gh, sm.ax, lf, l16, lg, [](int) { return 1.f; },
                           [&](int i) { return sm.delta[i]; });
#pragma unroll
          for (int u = 0; u < NA; ++u) {
            float z = gs[u];
            z += __shfl_xor(z, 16);
            z += __shfl_xor(z, 32);
            gzf[u] -= z;
          }
        });
        wave_fence();
        // J_phi(k_j)^T Z_j over the owner's features, one lane per key
        dispatch_index<0, kWaves>(w, [&](auto WI) {
          constexpr int WW = decltype(WI)::value;
          if constexpr (WW < G::NWF) {
            float x[kDK], out[kDK];
            load_coords(&sm.kx[l][0], x);
#pragma unroll
            for (int d = 0; d < kDK; ++d) out[d] = 0.f;
            own_vjp<NT, WW>(x, &sm.z[0][l], out);
            wave_fence();
#pragma unroll
            for (int d = 0; d < kDK; ++d) part[l * kLP + d] = out[d];
          }
        });
      } else {
#pragma unroll
        for (int d = 0; d < kDK; ++d) part[l * kLP + d] = 0.f;
      }

      // dv tiles (jw, 2 hw + e): phi(K) G over all features (the copy in LDS), plus w^T gh in the chunk
      f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll 2
      for (int qq = 0; qq < NFT; ++qq)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * qq + 4 * lg + r;
          const float a = phi(&sm.kx[16 * jw + l16][0], unpack(sm.code[f]));
#pragma unroll
          for (int e = 0; e < 2; ++e) acc[e] = mfma(a, sm.gm[f][16 * (2 * hw + e) + l16], acc[e]);
        }
      const f32x4 kb = *reinterpret_cast<const f32x4*>(&sm.kx[16 * jw + l16][4 * lg]);
      const int j = 16 * jw + l16;
      f32x4 dki = zero4();
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        if (it >= jw) {
          const f32x4 aa = *reinterpret_cast<const f32x4*>(&sm.ax[16 * it + l16][4 * lg]);
          f32x4 sc = zero4();
#pragma unroll
          for (int s = 0; s < 4; ++s) sc = mfma(aa[s], kb[s], sc);  // [query i][key j]
          f32x4 wt, kp;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * it + 4 * lg + r;
            const bool ok = j <= i && i < nv;
            wt[r] = ok ? taylor_kernel<NT>(sc[r]) : 0.f;
            float d = 0.f;
            if constexpr (NT > 1) d = taylor_kernel<NT - 1>(sc[r]);
            kp[r] = ok ? d : 0.f;
          }
#pragma unroll
          for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[e] = mfma(wt[r], sm.gh[16 * it + 4 * lg + r][16 * (2 * hw + e) + l16], acc[e]);
          if (hw) {
            f32x4 dw = zero4();
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const f32x4 ga = *reinterpret_cast<const f32x4*>(&sm.gh[16 * it + l16][16 * qq + 4 * lg]);
              const f32x4 vb = *reinterpret_cast<const f32x4*>(&sm.v[j][16 * qq + 4 * lg]);
#pragma unroll
              for (int r = 0; r < 4; ++r) dw = mfma(ga[r], vb[r], dw);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 16 * it + 4 * lg + r;
              const float ds = (dw[r] - sm.delta[i]) * kp[r];
              dki = mfma(ds, sm.ax[i][l16], dki);
            }
          }
        }
      }
      store_dv(acc, dv, tok0, nv, jw, hw, l16, lg);
      if (hw) {
        wave_fence();
#pragma unroll
        for (int r = 0; r < 4; ++r) part[(16 * jw + 4 * lg + r) * kLP + l16] += dki[r];
      }
      __syncthreads();
    }
    reduce_rows(sm.z, dk, tok_of(0), nv_of(0), 1.f, tid);
  });
}

// Exclusive prefix over each pair's slots in token order, seeded with `seed` (null: zero; not
// modified).  grid = (ceil(elems / 256), pairs).
__global__ __launch_bounds__(256) void bwd_scan_kernel(float* __restrict__ ws, const float* __restrict__ seed,
                                                       long long nslot, long long stride, long long elems,
                                                       SeqMap seq, int L) {
  const long long e = blockIdx.x * 256ll + threadIdx.x;
  if (e >= elems) return;
  const long long bh = blockIdx.y;
  long long first;
  int n;
  seq.pair_slots(bh, nslot, L, first, n);
  float run = seed ? seed[bh * stride + e] : 0.f;
  float* p = ws + first * stride + e;
  for (int s = 0; s < n; ++s) {
    const float t = s + 1 < n ? p[s * stride] : 0.f;  // the last increment enters no prefix
    p[s * stride] = run;
    run += t;
  }
}

// Exclusive suffix over each pair's slots (reverse token order), seeded with dstate (null: zero); the
// total goes back to dstate.
__global__ __launch_bounds__(256) void bwd_rscan_kernel(float* __restrict__ ws, float* __restrict__ dstate,
                                                        long long nslot, long long stride, long long elems,
                                                        SeqMap seq, int L) {
  const long long e = blockIdx.x * 256ll + threadIdx.x;
  if (e >= elems) return;
  const long long bh = blockIdx.y;
  long long first;
  int n;
  seq.pair_slots(bh, nslot, L, first, n);
  float run = dstate ? dstate[bh * stride + e] : 0.f;
  float* p = ws + first * stride + e;
  for (int s = n - 1; s >= 0; --s) {
    const float t = p[s * stride];
    p[s * stride] = run;
    run += t;
  }
  if (dstate) dstate[bh * stride + e] = run;
}

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Segments: about 256 workgroups (one per CU: the LDS holds a chunk's rows and the feature-major
// buffers), never more than the chunks: the count up to ceil(256 / BH) with the fewest rounds of 256
// workgroups times chunks per segment (ties: fewer).
BwdPlan plan_for(int BH, int N) {
  const int nchunk = cdiv(N, kC);
  long long hi = (256 + BH - 1) / BH;
  if (hi > nchunk) hi = nchunk;
  long long want = 1, cost = -1;
  for (long long S = 1; S <= hi; ++S) {
    const long long c = (((long long)BH * S + 255) / 256) * ((nchunk + S - 1) / S);
    if (cost < 0 || c < cost) cost = c, want = S;
  }
  BwdPlan p;
  p.L = cdiv(nchunk, want) * kC;
  p.nseg = cdiv(N, p.L);
  return p;
}

template <int NT, typename E>
int bwd_run(const BwdArgs& a) {
  const BwdPlan p = plan_for(a.BH, a.N);
  const SeqMap seq{nullptr, 0, a.BH, 1, a.N, 0};
  const long long slots = (long long)a.BH * p.nseg * a.s.stride;
  float* ws = (float*)a.ws;
  float* sslots = ws;
  float* gslots = sslots + slots;
  float* ghat = gslots + slots;
  float* dlt = ghat + (long long)a.BH * a.N * kDV;
  const E* q = (const E*)a.q;
  const E* k = (const E*)a.k;
  const E* v = (const E*)a.v;
  const dim3 grid(p.nseg, a.BH), block(kThreads);
  const long long elems = BG<NT>::W * (long long)(kDV + 1);
  const dim3 sgrid(cdiv(elems, 256), a.BH), sblock(256);
  // the state pass feeds only the prefixes of later segments: with one segment per pair the scan alone
  // seeds it with the incoming state (its increment is never read)
  if (p.nseg > 1) bwd_state_kernel<NT, E><<<grid, block, 0, a.stream>>>(k, v, sslots, seq, p.L, p.nseg, a.s.stride);
  bwd_scan_kernel<<<sgrid, sblock, 0, a.stream>>>(sslots, a.state, p.nseg, a.s.stride, elems, seq, p.L);
  bwd_dq_kernel<NT, E><<<grid, block, 0, a.stream>>>(q, k, v, a.g, a.o, sslots, gslots, ghat, dlt, a.dq, seq, p.L,
                                                     p.nseg, a.s.stride, a.s.scale);
  bwd_rscan_kernel<<<sgrid, sblock, 0, a.stream>>>(gslots, a.dstate, p.nseg, a.s.stride, elems, seq, p.L);
  bwd_dkv_kernel<NT, E><<<grid, block, 0, a.stream>>>(q, k, v, gslots, ghat, dlt, a.dk, a.dv, seq, p.L, p.nseg,
                                                      a.s.stride, a.s.scale);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

bool backward_has(int nt, int dk, int dv) { return dk == kDK && dv == kDV && nt >= 1 && nt <= 5; }

long long backward_ws_bytes(const Shape& s, int BH, int N) {
  if (s.nt >= 4) return backward_wide_ws_bytes(s, BH, N);
  if (BH == 0 || N == 0) return 0;
  const BwdPlan p = plan_for(BH, N);
  return (2 * (long long)BH * p.nseg * s.stride + (long long)BH * N * (kDV + 1)) * 4;
}

int backward_launch(const BwdArgs& a) {
  if (!backward_has(a.s.nt, a.s.dk, a.s.dv)) return -2;
  if (a.s.nt >= 4) return backward_wide_launch(a);
  switch (a.s.nt) {
    case 1: return a.s.dtype == 0 ? bwd_run<1, float>(a) : bwd_run<1, uint16_t>(a);
    case 2: return a.s.dtype == 0 ? bwd_run<2, float>(a) : bwd_run<2, uint16_t>(a);
    default: return a.s.dtype == 0 ? bwd_run<3, float>(a) : bwd_run<3, uint16_t>(a);
  }
}

}  // namespace taylor
