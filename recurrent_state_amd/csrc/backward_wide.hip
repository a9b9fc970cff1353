// Backward of truncated-kernel causal attention at n = 4, 5 (W = 969, 4,845 features; d_k = 16,
// d_v = 64), gfx950: dq, dk, dv and the gradient of the incoming state, float32 arithmetic.
//
// The forward is the method of "Expanding Attention" (Huang, arXiv:2610.20637), Abstract; the
// gradients are derived from that definition (the derivation is in backward.hip's header).  With
// a = sigma q, den_i the normaliser of token i, gh_i = g_i / den_i and delta_i = g_i . o_i / den_i:
//     dq_i = sigma J_phi(a_i)^T (S gh_i - delta_i z) + intra-chunk terms   (forward states S, z),
//     dv_j = G_S^T phi(k_j),  dk_j = J_phi(k_j)^T (G_S v_j + G_z) + intra   (reverse states G).
// At n = 4, 5 neither S nor G fits on chip, but every term is a sum over features of terms that each
// involve one feature row: the work splits over blocks of 16 NW features (NW = 4 at n = 4, 8 at n = 5),
// one workgroup of NW wavefronts per (sequence-head pair, block) walking all chunks of the pair, and partial results per block are
// summed in block order by small reduction kernels.  den is such a sum too, and it is needed before
// gh exists; but every term of dq carries the factor 1 / den_i, so the forward walk computes den's
// block parts and dq * den together and the first reduction divides:
//   pass A (chunks in order): den parts phi_B(a_i) . z_B, and J_phi_B(a_i)^T (S_B g_i - z_B (g_i . o_i));
//          the last block adds the intra-chunk parts;
//   reduce 1: den, dq = sigma sum / den, gh and delta per token;
//   pass B (chunks in reverse; G seeded with the final state's gradient): dv and dk parts; the last block
//          adds the intra-chunk parts; the block's G at the start is the incoming state's gradient;
//   reduce 2: dk, dv.
// Wavefront w owns the block's 16-feature tile w: it keeps that tile of S (pass A) or
// G_S (pass B) in float32 MFMA accumulators, transposed (lane feature 16 w + lane % 16, value columns
// 16 dt + 4 (lane / 16) + r), which is the A operand of a product over value columns (S g, G v); it
// expands its own features of the chunk's k and a into LDS (lanes 0..31 from k, lanes 32..63 from a,
// the same compile-time code on both halves), and runs their den part, z or G_z update and feature
// Jacobian (one lane per token).  Only two things cross wavefronts: the per-token sums of the eight
// tiles' Jacobian rows and den parts, and in pass B dv, a product over all the block's features, for
// which each wavefront leaves its G tile in LDS once per chunk.  Barriers per chunk: two in pass A,
// three in pass B (plus two in the last block for the intra-chunk terms).  All products run as float32
// 16x16x4 MFMAs; LDS row strides keep each product's operand reads on distinct banks.
#include <type_traits>
#include <utility>

#include "backward.hpp"
#include "features.hpp"

namespace taylor {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDK = 16, kDV = 64;
constexpr int kC = 32;  // tokens per chunk
constexpr int kLX = 20;           // a, k rows (16 coordinates; 16-byte aligned)
constexpr int kLT = kC + 4;       // rows indexed by feature or value column, columns by token (36)
constexpr int kLR = kDV + 16;     // token rows of 64 values read as [token][16 x + lane % 16] (80)
constexpr int kLGS = kDV + 16;    // pass B's shared G_S rows, read as [feature][16 x + lane % 16] (80)
constexpr int kLG = 68;           // gh (64), delta, padding per token in the workspace

// One 16-feature tile per wavefront: NW wavefronts, FB = 16 NW features per block (n = 4: 4 and 64, so
// that 16 heads make 256 workgroups; n = 5: 8 and 128).
template <int NT>
struct WB {
  static constexpr int W = FeatureTable<NT, kDK>::W;
  static constexpr int NW = NT == 4 ? 4 : 8;
  static constexpr int FB = 16 * NW;
  static constexpr int NB = (W + FB - 1) / FB;  // blocks
  static constexpr int TH = 64 * NW;            // threads
  static constexpr int RT = kC / (4 * NW);      // rounds of 16-thread token groups over a chunk
};

// Field order: the arrays that the unrolled per-tile code addresses with constant offsets (the rows
// of k, a, y, the features, z) come first, inside the 64 KB that an LDS instruction's offset field
// reaches from one base register; placed beyond it, every such access needed a base register of its
// own, hoisted out of the chunk loop, and they spilled.
template <int NW>
struct SmemA {
  static constexpr int FB = 16 * NW, LS = FB + 16;
  alignas(16) float xa[kC][kLX];   // a = sigma q
  alignas(16) float xk[kC][kLX];   // k
  alignas(16) float zz[FB];        // z of the block's features
  alignas(16) float go[kC];        // g . o
  alignas(16) float y[FB][kLT];    // S_f . g_t - z_f (g_t . o_t), feature-major
  alignas(16) float pk[kC][LS];    // phi_f(k_t), the block's features (wavefront w: columns 16w..)
  alignas(16) float pa[kC][LS];    // phi_f(a_t)
  alignas(16) float dred[NW][kC];  // per-tile den parts
  alignas(16) float dintra[kC];        // intra-chunk den (last block)
  float part[NW + 1][kC][kDK + 1];  // per-tile Jacobian rows; [NW]: intra-chunk rows (last block)
  float wm[kC][kC + 1];            // intra-chunk weights [query][key] (last block)
  float dm[kC][kC + 1];            // intra-chunk score gradients times den (last block)
  alignas(16) float v[kC][kLR];    // v rows
  alignas(16) float gt[kDV][kLT];  // g^T
};

template <int NW>
struct SmemB {
  static constexpr int FB = 16 * NW, LS = FB + 16, LQ = FB + 4;
  alignas(16) float xa[kC][kLX];
  alignas(16) float xk[kC][kLX];
  alignas(16) float zz[FB];         // G_z of the block's features
  alignas(16) float go[kC];         // delta
  alignas(16) float y[FB][kLT];     // G_S v_t + G_z, feature-major
  alignas(16) float pk[kC][LQ];     // phi_f(k_t)
  alignas(16) float pa[kC][LS];     // phi_f(a_t)
  float part[NW + 1][kC][kDK + 1];
  float wm[kC][kC + 1];
  float dm[kC][kC + 1];
  alignas(16) float vt[kDV][kLT];   // v^T
  alignas(16) float gh[kC][kLR];    // gh rows
  alignas(16) float gs[FB][kLGS];   // G_S rows of the block (each wavefront's tile, once per chunk)
};

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Orders this wavefront's LDS accesses before and after it (the compiler keeps them in program order;
// the hardware executes a wavefront's LDS instructions in order).
__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The wavefront's feature slot fb * NW + w, opaque to the optimiser at each use: otherwise the
// comparisons of the dispatch tree are hoisted out of the chunk loop and their hundreds of results
// spill.
template <int NW>
__device__ __forceinline__ int slot_of(int fb, int w) {
  int sel = fb * NW + w;
  asm volatile("" : "+s"(sel));
  return sel;
}

__device__ __forceinline__ float ldx(const void* p, long long i, bool bf16) {
  return bf16 ? __uint_as_float((uint32_t)(static_cast<const uint16_t*>(p)[i]) << 16) : static_cast<const float*>(p)[i];
}

// One thread's share of a chunk's inputs, loaded a chunk ahead into registers: for token t, coordinate c
// of q and k, value columns 4c .. 4c + 3 of v and of g, o (pass A) or gh
// (pass B, with delta in o4[0])).  Rows past the end of the pair are zero.
struct ChunkIn {
  float q1, k1;
  f32x4 v4, g4, o4;
};

__device__ __forceinline__ f32x4 ld4(const void* p, long long i, bool bf16) {
  if (bf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
  }
  return *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
}

// pass A: q, k, v, g, o of tokens tok0 .. tok0 + nv - 1
__device__ __forceinline__ void load_a(ChunkIn& in, const void* q, const void* k, const void* v, const float* g,
                                       const float* o, long long tok0, int nv, bool bf16, int t, int c) {
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  in = ChunkIn{0.f, 0.f, z4, z4, z4};
  if (t < nv) {
    const long long r = tok0 + t;
    in.q1 = ldx(q, r * kDK + c, bf16);
    in.k1 = ldx(k, r * kDK + c, bf16);
    in.v4 = ld4(v, r * kDV + 4 * c, bf16);
    in.g4 = *reinterpret_cast<const f32x4*>(g + r * kDV + 4 * c);
    in.o4 = *reinterpret_cast<const f32x4*>(o + r * kDV + 4 * c);
  }
}

// pass B: q, k, v and gh, delta of tokens tok0 .. tok0 + nv - 1
__device__ __forceinline__ void load_b(ChunkIn& in, const void* q, const void* k, const void* v, const float* ghd,
                                       long long tok0, int nv, bool bf16, int t, int c) {
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  in = ChunkIn{0.f, 0.f, z4, z4, z4};
  if (t < nv) {
    const long long r = tok0 + t;
    in.q1 = ldx(q, r * kDK + c, bf16);
    in.k1 = ldx(k, r * kDK + c, bf16);
    in.v4 = ld4(v, r * kDV + 4 * c, bf16);
    in.g4 = *reinterpret_cast<const f32x4*>(ghd + r * kLG + 4 * c);
    if (c == 0) in.o4[0] = ghd[r * kLG + kDV];
  }
}

// The chunk's rows into LDS (token t, coordinate c and value columns 4c .. 4c + 3).  Pass A: a = sigma q, k, v rows, g^T
// and g . o per token (a sum over the token's 16 lanes); pass B: a, k, v^T, gh rows and delta.
template <class SM>
__device__ __forceinline__ void store_a(SM& sm, const ChunkIn& in, float scale, int t, int c) {
  sm.xa[t][c] = scale * in.q1;
  sm.xk[t][c] = in.k1;
  *reinterpret_cast<f32x4*>(&sm.v[t][4 * c]) = in.v4;
#pragma unroll
  for (int e = 0; e < 4; ++e) sm.gt[4 * c + e][t] = in.g4[e];
  float p = (in.g4[0] * in.o4[0] + in.g4[1] * in.o4[1]) + (in.g4[2] * in.o4[2] + in.g4[3] * in.o4[3]);
  p += __shfl_xor(p, 8, 16);
  p += __shfl_xor(p, 4, 16);
  p += __shfl_xor(p, 2, 16);
  p += __shfl_xor(p, 1, 16);
  if (c == 0) sm.go[t] = p;
}

template <class SM>
__device__ __forceinline__ void store_b(SM& sm, const ChunkIn& in, float scale, int t, int c) {
  sm.xa[t][c] = scale * in.q1;
  sm.xk[t][c] = in.k1;
#pragma unroll
  for (int e = 0; e < 4; ++e) sm.vt[4 * c + e][t] = in.v4[e];
  *reinterpret_cast<f32x4*>(&sm.gh[t][4 * c]) = in.g4;
  if (c == 0) sm.go[t] = in.o4[0];
}

// Wavefront w's 16 features F0 = 16 (fb * 8 + w) .. of the chunk's tokens: lanes 0..31 from k into pk,
// lanes 32..63 from a into pa (token l % 32).  A token past the end has zero rows, so only its
// constant feature is masked.
template <int NT, int F0, class SM>
__device__ __forceinline__ void expand_tile(SM& sm, int l, int nv) {
  constexpr int L0 = F0 % SM::FB;
  const int t = l & 31;
  const float* xr = l < 32 ? &sm.xk[t][0] : &sm.xa[t][0];
  float x[kDK];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const f32x4 x4 = *reinterpret_cast<const f32x4*>(xr + 4 * u);
    x[4 * u] = x4[0], x[4 * u + 1] = x4[1], x[4 * u + 2] = x4[2], x[4 * u + 3] = x4[3];
  }
  float f[16];
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((f[I] = feature_ct<NT, kDK, F0 + I>(x)), ...);
  }(std::make_integer_sequence<int, 16>{});
  if constexpr (F0 == 0) f[0] = t < nv ? 1.f : 0.f;
  float* dst = l < 32 ? &sm.pk[t][L0] : &sm.pa[t][L0];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    *reinterpret_cast<f32x4*>(dst + 4 * u) = f32x4{f[4 * u], f[4 * u + 1], f[4 * u + 2], f[4 * u + 3]};
}

// d += y * grad phi_A(x): feature A = cf x_c0 x_c1 ... (coordinates repeat for powers, so adding the
// product of the other coordinates once per occurrence gives alpha_c x^(alpha - e_c)).
template <int NT, int A>
__device__ __forceinline__ void feature_vjp(const float (&x)[kDK], float y, float (&d)[kDK]) {
  if constexpr (A < FeatureTable<NT, kDK>::W) {
    constexpr int m = FeatureTable<NT, kDK>::T.order[A];
    constexpr int c0 = FeatureTable<NT, kDK>::T.coord[A][0];
    constexpr int c1 = FeatureTable<NT, kDK>::T.coord[A][1];
    constexpr int c2 = FeatureTable<NT, kDK>::T.coord[A][2];
    constexpr int c3 = FeatureTable<NT, kDK>::T.coord[A][3];
    constexpr float cf = coef_of_afact(FeatureTable<NT, kDK>::T.afact[A]);
    if constexpr (m == 1) {
      d[c0] = fmaf(cf, y, d[c0]);
    } else if constexpr (m == 2) {
      const float cy = cf * y;
      d[c0] = fmaf(cy, x[c1], d[c0]);
      d[c1] = fmaf(cy, x[c0], d[c1]);
    } else if constexpr (m == 3) {
      const float cy = cf * y;
      d[c0] = fmaf(cy, x[c1] * x[c2], d[c0]);
      d[c1] = fmaf(cy, x[c0] * x[c2], d[c1]);
      d[c2] = fmaf(cy, x[c0] * x[c1], d[c2]);
    } else if constexpr (m == 4) {
      const float cy = cf * y;
      const float p01 = x[c0] * x[c1], p23 = x[c2] * x[c3];
      d[c0] = fmaf(cy, x[c1] * p23, d[c0]);
      d[c1] = fmaf(cy, x[c0] * p23, d[c1]);
      d[c2] = fmaf(cy, p01 * x[c3], d[c2]);
      d[c3] = fmaf(cy, p01 * x[c2], d[c3]);
    }
  }
}

// One lane per token t (< 32): J_phi(x_t)^T y[., t] over the wavefront's 16 features F0 .., into its
// row of part.
template <int NT, int F0, class SM>
__device__ __forceinline__ void jacobian_tile(SM& sm, int w, int t, const float* xr) {
  constexpr int L0 = F0 % SM::FB;
  float x[kDK], d[kDK];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const f32x4 x4 = *reinterpret_cast<const f32x4*>(xr + 4 * u);
    x[4 * u] = x4[0], x[4 * u + 1] = x4[1], x[4 * u + 2] = x4[2], x[4 * u + 3] = x4[3];
  }
#pragma unroll
  for (int c = 0; c < kDK; ++c) d[c] = 0.f;
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((feature_vjp<NT, F0 + I>(x, sm.y[L0 + I][t], d)), ...);
  }(std::make_integer_sequence<int, 16>{});
#pragma unroll
  for (int c = 0; c < kDK; ++c) sm.part[w][t][c] = d[c];
}

// The last block, intra-chunk: wm[i][j] = K_n(s_ij), dm[i][j] = (u_i . v_j - go_i) K_{n-1}(s_ij) for key
// j <= query i (zero above the diagonal), u = g (pass A) or gh (pass B).  Waves 0..3 take the four
// 16x16 tiles; u_i . v_j from u rows given as [d][i] (pass A: g^T) or [i][d] (pass B: gh) and v as
// [j][d] (pass A) or [d][j] (pass B).
template <int NT, bool PASS_A, class SM>
__device__ __forceinline__ void intra_weights(SM& sm, int w, int i16, int lg) {
  if (w >= 4) return;
  const int it = w >> 1, jt = w & 1;
  f32x4 sc = {0.f, 0.f, 0.f, 0.f}, uv = {0.f, 0.f, 0.f, 0.f};
  if (jt <= it) {
#pragma unroll
    for (int s = 0; s < 4; ++s) sc = mfma(sm.xa[16 * it + i16][4 * s + lg], sm.xk[16 * jt + i16][4 * s + lg], sc);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if constexpr (PASS_A)
        uv = mfma(sm.gt[4 * s + lg][16 * it + i16], sm.v[16 * jt + i16][4 * s + lg], uv);
      else
        uv = mfma(sm.gh[16 * it + i16][4 * s + lg], sm.vt[4 * s + lg][16 * jt + i16], uv);
    }
  }
  // sc[r], uv[r]: query i = 16 it + 4 lg + r, key j = 16 jt + i16
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * it + 4 * lg + r, j = 16 * jt + i16;
    const bool ok = j <= i;
    sm.wm[i][j] = ok ? taylor_kernel<NT>(sc[r]) : 0.f;
    sm.dm[i][j] = ok ? (uv[r] - sm.go[i]) * taylor_kernel<NT - 1>(sc[r]) : 0.f;
  }
}

// Pass A: one workgroup per (block, pair), chunks in order.  Writes per token: den_part[block] and
// p16[block] = sigma J_phi_B(a)^T (S_B g - z_B (g . o)) (the last block: plus the intra-chunk parts).
template <int NT>
__global__ __launch_bounds__(WB<NT>::TH) void bwdw_a_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                            const void* __restrict__ v, const float* __restrict__ g,
                                                            const float* __restrict__ o,
                                                            const float* __restrict__ state,
                                                            float* __restrict__ den_part, float* __restrict__ p16,
                                                            int N, long long stride, float scale, int bf16,
                                                            long long T) {
  using P = WB<NT>;
  constexpr int W = P::W, NB = P::NB, NW = P::NW, RT = P::RT;
  __shared__ SmemA<NW> sm;
  const int tid = threadIdx.x, l = tid & 63, i16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fb = blockIdx.x;
  const long long bh = blockIdx.y;
  const int f0 = fb * P::FB + 16 * w;  // the wavefront's first feature
  const int t0 = tid >> 4, c16 = tid & 15;  // the thread's token group (rounds of 4 NW tokens) and coordinate
  const bool intra = fb == NB - 1;          // the block that adds the intra-chunk parts
  const bool real = f0 < W;                 // the tile holds real features (else S, y stay unused zeros)
  // S^T tile: lane holds S[f0 + i16][16 dt + 4 lg + r] in Sa[dt][r]
  f32x4 Sa[4];
  {
    const bool ok = state && f0 + i16 < W;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      Sa[dt] = ok ? *reinterpret_cast<const f32x4*>(state + bh * stride + (long long)(f0 + i16) * kDV + 16 * dt + 4 * lg)
                  : f32x4{0.f, 0.f, 0.f, 0.f};
    if (l < 16) sm.zz[16 * w + l] = (state && f0 + l < W) ? state[bh * stride + (long long)W * kDV + f0 + l] : 0.f;
  }
  const int nch = (N + kC - 1) / kC;
  const bool bf = bf16 != 0;
  ChunkIn in[RT];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int u = 0; u < RT; ++u)
      load_a(in[u], q, k, v, g, o, bh * N + (long long)c * kC, min(kC, N - c * kC), bf, t0 + 4 * NW * u, c16);
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int u = 0; u < RT; ++u) store_a(sm, in[u], scale, t0 + 4 * NW * u, c16);
  };
  load_chunk(0);
  store_chunk();
  if (nch > 1) load_chunk(1);
  for (int c = 0; c < nch; ++c) {
    const int nv = min(kC, N - c * kC);
    const long long tok0 = bh * N + (long long)c * kC;
    __syncthreads();  // the chunk's rows are in LDS
    dispatch_index<0, NB * NW>(slot_of<NW>(fb, w), [&](auto I) { expand_tile<NT, decltype(I)::value * 16>(sm, l, nv); });
    wave_fence();
    // y = S g - z (g . o) over the tile's features (S, z before this chunk)
    if (real) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc = mfma(Sa[dt][r], sm.gt[16 * dt + 4 * lg + r][16 * tt + i16], acc);
        // acc[r]: feature 16 w + 4 lg + r, token 16 tt + i16
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * w + 4 * lg + r, t = 16 * tt + i16;
          sm.y[f][t] = acc[r] - sm.zz[f] * sm.go[t];
        }
      }
    }
    if (l < kC) {
      // den part of token l over the tile's features
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 pv = *reinterpret_cast<const f32x4*>(&sm.pa[l][16 * w + 4 * u]);
        const f32x4 zv = *reinterpret_cast<const f32x4*>(&sm.zz[16 * w + 4 * u]);
        acc = fmaf(pv[0], zv[0], acc);
        acc = fmaf(pv[1], zv[1], acc);
        acc = fmaf(pv[2], zv[2], acc);
        acc = fmaf(pv[3], zv[3], acc);
      }
      sm.dred[w][l] = acc;
    }
    wave_fence();
    // S^T += V^T phi(K) over the tile's features, z += phi(K)^T 1
    if (real) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int s = 0; s < kC / 4; ++s) Sa[dt] = mfma(sm.v[4 * s + lg][16 * dt + i16], sm.pk[4 * s + lg][16 * w + i16], Sa[dt]);
    }
    if (l < 16) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < kC; ++t) acc += sm.pk[t][16 * w + l];
      sm.zz[16 * w + l] += acc;
    }
    if (l < kC)
      dispatch_index<0, NB * NW>(slot_of<NW>(fb, w), [&](auto I) { jacobian_tile<NT, decltype(I)::value * 16>(sm, w, l, &sm.xa[l][0]); });
    if (intra) {
      intra_weights<NT, true>(sm, w, i16, lg);
      __syncthreads();
      if (w < 2) {
        // sum_j dm[i][j] k_j over the chunk: rows 16 w .. 16 w + 15
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kC / 4; ++s) acc = mfma(sm.dm[16 * w + i16][4 * s + lg], sm.xk[4 * s + lg][i16], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.part[NW][16 * w + 4 * lg + r][i16] = acc[r];
      } else if (w == 2 && l < kC) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < kC; ++j) acc += sm.wm[l][j];
        sm.dintra[l] = acc;
      }
    }
    __syncthreads();  // the tiles' parts are in LDS; the chunk's rows are free
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int t = t0 + 4 * NW * u;
      if (t < nv) {
        float s = 0.f;
#pragma unroll
        for (int x = 0; x < NW; ++x) s += sm.part[x][t][c16];
        if (intra) s += sm.part[NW][t][c16];
        p16[((long long)fb * T + tok0 + t) * kDK + c16] = scale * s;
        if (c16 == 0) {
          float dn = 0.f;
#pragma unroll
          for (int x = 0; x < NW; ++x) dn += sm.dred[x][t];
          if (intra) dn += sm.dintra[t];
          den_part[(long long)fb * T + tok0 + t] = dn;
        }
      }
    }
    if (c + 1 < nch) {
      store_chunk();
      if (c + 2 < nch) load_chunk(c + 2);
    }
  }
}

// Sums over the NB blocks of a per-token array of block parts [NB][T][4 * Q] (Q float4s per token), in
// block order, with eight blocks' loads in flight together.
__device__ __forceinline__ f32x4 block_sum4(const float* __restrict__ parts, long long T, int NB, long long tok,
                                            int q4, int Q) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int kB = 8;
  int b = 0;
  for (; b + kB <= NB; b += kB) {
    f32x4 x[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u)
      x[u] = *reinterpret_cast<const f32x4*>(parts + (((long long)(b + u) * T + tok) * Q + q4) * 4);
#pragma unroll
    for (int u = 0; u < kB; ++u) acc = acc + x[u];
  }
  for (; b < NB; ++b) acc = acc + *reinterpret_cast<const f32x4*>(parts + (((long long)b * T + tok) * Q + q4) * 4);
  return acc;
}

__device__ __forceinline__ float block_sum1(const float* __restrict__ parts, long long T, int NB, long long tok) {
  float acc = 0.f;
  constexpr int kB = 8;
  int b = 0;
  for (; b + kB <= NB; b += kB) {
    float x[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) x[u] = parts[(long long)(b + u) * T + tok];
#pragma unroll
    for (int u = 0; u < kB; ++u) acc += x[u];
  }
  for (; b < NB; ++b) acc += parts[(long long)b * T + tok];
  return acc;
}

// Reduce 1, 16 threads per token (thread j: dq coordinates 4j..4j+3 for j < 4, and g, o columns
// 4j..4j+3): den = sum of the block parts, dq = p16 sum / den, gh = g / den, delta = g . o / den.
__global__ __launch_bounds__(256) void bwdw_r1_kernel(const float* __restrict__ den_part, const float* __restrict__ p16,
                                                      const float* __restrict__ g, const float* __restrict__ o,
                                                      float* __restrict__ ghd, float* __restrict__ dq, int NB,
                                                      long long T) {
  const long long tok = blockIdx.x * 16ll + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  if (tok >= T) return;  // the 16 threads of a token leave together
  const float den = block_sum1(den_part, T, NB, tok);
  const f32x4 gv = *reinterpret_cast<const f32x4*>(g + tok * kDV + 4 * j);
  const f32x4 ov = *reinterpret_cast<const f32x4*>(o + tok * kDV + 4 * j);
  float go = (gv[0] * ov[0] + gv[1] * ov[1]) + (gv[2] * ov[2] + gv[3] * ov[3]);
  go += __shfl_xor(go, 8, 16);
  go += __shfl_xor(go, 4, 16);
  go += __shfl_xor(go, 2, 16);
  go += __shfl_xor(go, 1, 16);
  *reinterpret_cast<f32x4*>(ghd + tok * kLG + 4 * j) = f32x4{gv[0] / den, gv[1] / den, gv[2] / den, gv[3] / den};
  if (j == 0) ghd[tok * kLG + kDV] = go / den;
  if (j < kDK / 4) {
    const f32x4 sq = block_sum4(p16, T, NB, tok, j, kDK / 4);
    *reinterpret_cast<f32x4*>(dq + tok * kDK + 4 * j) = f32x4{sq[0] / den, sq[1] / den, sq[2] / den, sq[3] / den};
  }
}

// Pass B: one workgroup per (block, pair), chunks in reverse.  Writes per token the dv and dk parts of
// the block (the last block: plus the intra-chunk parts), and the block's rows of the incoming state's
// gradient.
template <int NT>
__global__ __launch_bounds__(WB<NT>::TH) void bwdw_b_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                            const void* __restrict__ v, const float* __restrict__ ghd,
                                                            float* __restrict__ dstate, float* __restrict__ p16,
                                                            float* __restrict__ pdv, int N, long long stride,
                                                            float scale, int bf16, long long T) {
  using P = WB<NT>;
  constexpr int W = P::W, NB = P::NB, NW = P::NW, RT = P::RT, FB = P::FB;
  constexpr int ND = 8 / NW;  // 16x16 tiles of the chunk's dv per wavefront (8 tiles: 2 token x 4 column)
  __shared__ SmemB<NW> sm;
  const int tid = threadIdx.x, l = tid & 63, i16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fb = blockIdx.x;
  const long long bh = blockIdx.y;
  const int f0 = fb * FB + 16 * w;
  const int t0 = tid >> 4, c16 = tid & 15;
  const bool intra = fb == NB - 1;  // the block that adds the intra-chunk parts
  const bool real = f0 < W;         // the tile holds real features (else G_S, y stay unused zeros)
  // steps of 4 features of the last block with a real one among them (its padding is zero in pk)
  constexpr int kLastSteps = (W - (NB - 1) * FB + 3) / 4;
  // G_S^T tile: lane holds G_S[f0 + i16][16 dt + 4 lg + r] in Ga[dt][r]
  f32x4 Ga[4];
  {
    const bool ok = dstate && f0 + i16 < W;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      Ga[dt] = ok ? *reinterpret_cast<const f32x4*>(dstate + bh * stride + (long long)(f0 + i16) * kDV + 16 * dt + 4 * lg)
                  : f32x4{0.f, 0.f, 0.f, 0.f};
    if (l < 16) sm.zz[16 * w + l] = (dstate && f0 + l < W) ? dstate[bh * stride + (long long)W * kDV + f0 + l] : 0.f;
  }
  auto put_tile = [&]() {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(&sm.gs[16 * w + i16][16 * dt + 4 * lg]) = Ga[dt];
  };
  const int nch = (N + kC - 1) / kC;
  const bool bf = bf16 != 0;
  ChunkIn in[RT];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int u = 0; u < RT; ++u)
      load_b(in[u], q, k, v, ghd, bh * N + (long long)c * kC, min(kC, N - c * kC), bf, t0 + 4 * NW * u, c16);
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int u = 0; u < RT; ++u) store_b(sm, in[u], scale, t0 + 4 * NW * u, c16);
  };
  load_chunk(nch - 1);
  store_chunk();
  put_tile();
  if (nch > 1) load_chunk(nch - 2);
  for (int c = nch - 1; c >= 0; --c) {
    const int nv = min(kC, N - c * kC);
    const long long tok0 = bh * N + (long long)c * kC;
    __syncthreads();  // the chunk's rows and every G_S tile are in LDS
    dispatch_index<0, NB * NW>(slot_of<NW>(fb, w), [&](auto I) { expand_tile<NT, decltype(I)::value * 16>(sm, l, nv); });
    __syncthreads();  // every tile's phi(K) is in LDS
    // dv parts = phi_B(K) G_S (G of the later tokens) over all the block's features: the wavefront's
    // tiles u = w, w + NW of the eight (token tile u / 4, column tile u % 4)
    f32x4 dva[ND];
    auto dv_parts = [&](auto nsteps) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < ND; ++e) {
        const int u = w + NW * e, tt = u >> 2, dt = u & 3;
        dva[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int s = 0; s < decltype(nsteps)::value; ++s)
          dva[e] = mfma(sm.pk[16 * tt + i16][4 * s + lg], sm.gs[4 * s + lg][16 * dt + i16], dva[e]);
      }
    };
    if (intra)
      dv_parts(std::integral_constant<int, kLastSteps>{});
    else
      dv_parts(std::integral_constant<int, FB / 4>{});
    __builtin_amdgcn_sched_barrier(0);
    // y = G_S v + G_z over the tile's features
    if (real) {
#pragma unroll
      for (int ut = 0; ut < 2; ++ut) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc = mfma(Ga[dt][r], sm.vt[16 * dt + 4 * lg + r][16 * ut + i16], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * w + 4 * lg + r;
          sm.y[f][16 * ut + i16] = acc[r] + sm.zz[f];
        }
      }
    }
    wave_fence();
    __builtin_amdgcn_sched_barrier(0);
    // G_S^T += gh^T phi(A), G_z -= phi(A)^T delta over the tile's features
    if (real) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int s = 0; s < kC / 4; ++s) Ga[dt] = mfma(sm.gh[4 * s + lg][16 * dt + i16], sm.pa[4 * s + lg][16 * w + i16], Ga[dt]);
    }
    if (l < 16) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < kC; ++t) acc = fmaf(sm.pa[t][16 * w + l], sm.go[t], acc);
      sm.zz[16 * w + l] -= acc;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (l < kC)
      dispatch_index<0, NB * NW>(slot_of<NW>(fb, w), [&](auto I) { jacobian_tile<NT, decltype(I)::value * 16>(sm, w, l, &sm.xk[l][0]); });
    if (intra) {
      intra_weights<NT, false>(sm, w, i16, lg);
      __syncthreads();
      // dv_j += sum_i wm[i][j] gh_i (the wavefront's dv tiles); dk_j += sum_i dm[i][j] a_i (waves 0, 1)
#pragma unroll
      for (int e = 0; e < ND; ++e) {
        const int u = w + NW * e, tt = u >> 2, dt = u & 3;
#pragma unroll
        for (int s = 0; s < kC / 4; ++s) dva[e] = mfma(sm.wm[4 * s + lg][16 * tt + i16], sm.gh[4 * s + lg][16 * dt + i16], dva[e]);
      }
      if (w < 2) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kC / 4; ++s) acc = mfma(sm.dm[4 * s + lg][16 * w + i16], sm.xa[4 * s + lg][i16], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.part[NW][16 * w + 4 * lg + r][i16] = acc[r];
      }
    }
    __syncthreads();  // the tiles' parts are in LDS; the chunk's rows and G_S tiles are free
#pragma unroll
    for (int e = 0; e < ND; ++e) {
      const int u = w + NW * e, tt = u >> 2, dt = u & 3;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * lg + r;
        if (t < nv) pdv[((long long)fb * T + tok0 + t) * kDV + 16 * dt + i16] = dva[e][r];
      }
    }
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int t = t0 + 4 * NW * u;
      if (t < nv) {
        float s = 0.f;
#pragma unroll
        for (int x = 0; x < NW; ++x) s += sm.part[x][t][c16];
        if (intra) s += sm.part[NW][t][c16];
        p16[((long long)fb * T + tok0 + t) * kDK + c16] = s;
      }
    }
    if (c > 0) {
      store_chunk();
      put_tile();
      if (c > 1) load_chunk(c - 2);
    }
  }
  if (dstate) {
    if (f0 + i16 < W) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<f32x4*>(dstate + bh * stride + (long long)(f0 + i16) * kDV + 16 * dt + 4 * lg) = Ga[dt];
    }
    if (l < 16 && f0 + l < W) dstate[bh * stride + (long long)W * kDV + f0 + l] = sm.zz[16 * w + l];
  }
}

// Reduce 2, 16 threads per token (thread j: dv columns 4j..4j+3, and dk coordinates 4j..4j+3 for
// j < 4): dk, dv = sums of the block parts in block order.
__global__ __launch_bounds__(256) void bwdw_r2_kernel(const float* __restrict__ p16, const float* __restrict__ pdv,
                                                      float* __restrict__ dk, float* __restrict__ dv, int NB,
                                                      long long T) {
  const long long tok = blockIdx.x * 16ll + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  if (tok >= T) return;
  *reinterpret_cast<f32x4*>(dv + tok * kDV + 4 * j) = block_sum4(pdv, T, NB, tok, j, kDV / 4);
  if (j < kDK / 4) *reinterpret_cast<f32x4*>(dk + tok * kDK + 4 * j) = block_sum4(p16, T, NB, tok, j, kDK / 4);
}

// Workspace (floats): gh and delta [T][68], then dv parts [NB][T][64], dq / dk parts [NB][T][16]
// (pass A's are consumed by reduce 1 before pass B writes its own), den parts [NB][T].
template <int NT>
long long bwdw_ws_floats(long long T) {
  return T * kLG + (long long)WB<NT>::NB * T * (kDV + kDK + 1);
}

template <int NT>
int bwdw_run(const BwdArgs& a) {
  constexpr int NB = WB<NT>::NB;
  const long long T = (long long)a.BH * a.N;
  float* ghd = (float*)a.ws;
  float* pdv = ghd + T * kLG;
  float* p16 = pdv + NB * T * kDV;
  float* den_part = p16 + NB * T * kDK;
  const int bf = a.s.dtype != 0;
  const dim3 grid(NB, a.BH), block(WB<NT>::TH);
  const dim3 rgrid((unsigned)((T + 15) / 16)), rblock(256);
  bwdw_a_kernel<NT><<<grid, block, 0, a.stream>>>(a.q, a.k, a.v, a.g, a.o, a.state, den_part, p16, a.N, a.s.stride,
                                                  a.s.scale, bf, T);
  bwdw_r1_kernel<<<rgrid, rblock, 0, a.stream>>>(den_part, p16, a.g, a.o, ghd, a.dq, NB, T);
  bwdw_b_kernel<NT><<<grid, block, 0, a.stream>>>(a.q, a.k, a.v, ghd, a.dstate, p16, pdv, a.N, a.s.stride, a.s.scale,
                                                  bf, T);
  bwdw_r2_kernel<<<rgrid, rblock, 0, a.stream>>>(p16, pdv, a.dk, a.dv, NB, T);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

long long backward_wide_ws_bytes(const Shape& s, int BH, int N) {
  if (BH == 0 || N == 0) return 0;
  const long long T = (long long)BH * N;
  return 4 * (s.nt == 4 ? bwdw_ws_floats<4>(T) : bwdw_ws_floats<5>(T));
}

int backward_wide_launch(const BwdArgs& a) { return a.s.nt == 4 ? bwdw_run<4>(a) : bwdw_run<5>(a); }

}  // namespace taylor
