// Backward of truncated-kernel causal attention at n = 4, 5 (W = 969, 4,845 features; d_k = 16,
// d_v = 64), gfx950: dq, dk, dv and the gradient of the incoming state, float32 arithmetic.
//
// The forward is the method of "Expanding Attention" (Huang, arXiv:2610.20637), Abstract; the
// gradients are derived from that definition (the derivation is in backward.hip's header).  With
// a = sigma q, den_i the normaliser of token i, gh_i = g_i / den_i and delta_i = g_i . o_i / den_i:
//     dq_i = sigma J_phi(a_i)^T (S gh_i - delta_i z) + intra-chunk terms   (forward states S, z),
//     dv_j = G_S^T phi(k_j),  dk_j = J_phi(k_j)^T (G_S v_j + G_z) + intra   (reverse states G).
// At n = 4, 5 neither S nor G fits on chip, but every term is a sum over features of terms that each
// involve one feature row: the work splits over blocks of FB features (64 at n = 4, 128 at n = 5),
// one workgroup per (sequence-head pair, block) walking all chunks of the pair, and partial results
// per block are summed in block order by small reduction kernels.  den is such a sum too, and it is
// needed before gh exists; but every term of dq carries the factor 1 / den_i, so the forward walk
// computes den's block parts and dq * den together and the first reduction divides:
//   pass A (chunks in order; S, z of the block in LDS): den parts phi_B(a_i) . z_B, and
//          J_phi_B(a_i)^T (S_B g_i - z_B (g_i . o_i)); block 0 adds the intra-chunk parts;
//   reduce 1: den, dq = sigma sum / den, gh and delta per token;
//   pass B (chunks in reverse; G_S, G_z of the block in LDS, seeded with the final state's
//          gradient): dv and dk parts; block 0 adds the intra-chunk parts; the block's G at the
//          start is the incoming state's gradient;
//   reduce 2: dk, dv.
// All products over tokens, features and value columns run as float32 16x16x4 MFMAs with operands
// read from LDS; the features of a chunk are expanded once per pass into LDS (lanes 0..31 from k,
// lanes 32..63 from a, the same compile-time code on both halves), and the feature Jacobians run one
// lane per token over each wavefront's compile-time features.
#include <type_traits>
#include <utility>

#include "backward.hpp"
#include "features.hpp"

namespace taylor {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDK = 16, kDV = 64;
constexpr int kC = 32;  // tokens per chunk
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLX = 20;      // a, k rows (16 coordinates; 16-byte aligned, 20 mod 64 banks)
constexpr int kLY = kC + 4;  // feature-major rows of Y
constexpr int kLG = 68;      // gh (64), delta, padding per token in the workspace

template <int NT>
struct WB {
  static constexpr int W = FeatureTable<NT, kDK>::W;
  static constexpr int FB = NT == 4 ? 64 : 128;  // features per block
  static constexpr int NB = (W + FB - 1) / FB;   // blocks
  static constexpr int FW = FB / kWaves;         // features per wavefront in expansions and Jacobians
  static constexpr int NFT = FB / 16;            // 16-row feature tiles per block
  static constexpr int LP = FB + 4;              // token-major feature rows
};

// Row strides are chosen per pass so that the MFMA operand reads of each pass's main products hit 64
// distinct banks or at most two lanes per bank: an operand read [16 x + lane % 16][4 s + lane / 16]
// wants a stride of 4 mod 64, a read [4 s + lane / 16][16 x + lane % 16] one of 16 mod 64 (8 mod 64
// serves both at two lanes per bank).
template <int NT, bool A>
struct WBSmem {
  using P = WB<NT>;
  static constexpr int LPK = P::FB + (A ? 16 : 4);  // pass A reads phi(K) by token rows, pass B by feature
  static constexpr int LPA = P::FB + (A ? 4 : 16);
  static constexpr int LST = A ? 68 : 72;
  static constexpr int LVV = A ? 80 : 68;
  static constexpr int LGG = A ? 68 : 80;
  alignas(16) float pk[kC][LPK];   // phi_f(k_t) of the block's features
  alignas(16) float pa[kC][LPA];   // phi_f(a_t)
  alignas(16) float st[P::FB][LST];  // S rows (pass A) or G_S rows (pass B) of the block
  alignas(16) float y[P::FB][kLY];   // per feature and token: the vector the Jacobian contracts
  alignas(16) float v[kC][LVV];      // v rows
  alignas(16) float gg[kC][LGG];     // g rows (pass A) or gh rows (pass B)
  alignas(16) float xa[kC][kLX];     // a = sigma q
  alignas(16) float xk[kC][kLX];     // k
  float part[kWaves + 1][kC][kDK + 1];  // per-wavefront Jacobian rows; [kWaves]: intra-chunk rows
  float wm[kC][kC + 1];              // intra-chunk weights [query][key] (block 0)
  float dm[kC][kC + 1];              // intra-chunk score gradients (times den in pass A)
  float zz[P::FB];                   // z (pass A) or G_z (pass B) of the block
  float go[kC];                      // g . o (pass A) or delta (pass B)
  float dred[16][kC];                // pass A: 16 partial sums of each token's den part
  float dintra[kC];                  // pass A: intra-chunk den (block 0)
};

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The wavefront's feature slot fb * kWaves + w, opaque to the optimiser at each use: otherwise the
// comparisons of the dispatch tree are hoisted out of the chunk loop and their hundreds of results
// spill.
__device__ __forceinline__ int slot_of(int fb, int w) {
  int sel = fb * kWaves + w;
  asm volatile("" : "+s"(sel));
  return sel;
}

__device__ __forceinline__ float ldx(const void* p, long long i, bool bf16) {
  return bf16 ? __uint_as_float((uint32_t)(static_cast<const uint16_t*>(p)[i]) << 16) : static_cast<const float*>(p)[i];
}

// One thread's share of a chunk's inputs, loaded a chunk ahead into registers (thread t = tid / 16,
// c = tid % 16: coordinate c of q and k, value columns 4c .. 4c + 3 of v and of g, o (pass A) or gh
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
                                       const float* o, long long tok0, int nv, bool bf16, int tid) {
  const int t = tid >> 4, c = tid & 15;
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
                                       long long tok0, int nv, bool bf16, int tid) {
  const int t = tid >> 4, c = tid & 15;
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

// The chunk's rows into LDS: a = sigma q, k, v, g (or gh); go = g . o per token (pass A, a sum over
// the 16 lanes of the token) or delta (pass B).
template <bool PASS_A, class SM>
__device__ __forceinline__ void store_chunk(SM& sm, const ChunkIn& in, float scale, int tid) {
  const int t = tid >> 4, c = tid & 15;
  sm.xa[t][c] = scale * in.q1;
  sm.xk[t][c] = in.k1;
  *reinterpret_cast<f32x4*>(&sm.v[t][4 * c]) = in.v4;
  *reinterpret_cast<f32x4*>(&sm.gg[t][4 * c]) = in.g4;
  if constexpr (PASS_A) {
    float p = (in.g4[0] * in.o4[0] + in.g4[1] * in.o4[1]) + (in.g4[2] * in.o4[2] + in.g4[3] * in.o4[3]);
    p += __shfl_xor(p, 8, 16);
    p += __shfl_xor(p, 4, 16);
    p += __shfl_xor(p, 2, 16);
    p += __shfl_xor(p, 1, 16);
    if (c == 0) sm.go[t] = p;
  } else {
    if (c == 0) sm.go[t] = in.o4[0];
  }
}

// Features F0 .. F0 + FW - 1 of the chunk's tokens: lanes 0..31 from k into pk, lanes 32..63 from a
// into pa (token l % 32).  A token past the end has zero rows, so only its constant feature is masked.
template <int NT, int F0, class SM>
__device__ __forceinline__ void expand_w(SM& sm, int l, int nv) {
  using P = WB<NT>;
  constexpr int L0 = F0 % P::FB;
  const int t = l & 31;
  const float* xr = l < 32 ? &sm.xk[t][0] : &sm.xa[t][0];
  float x[kDK];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const f32x4 x4 = *reinterpret_cast<const f32x4*>(xr + 4 * u);
    x[4 * u] = x4[0], x[4 * u + 1] = x4[1], x[4 * u + 2] = x4[2], x[4 * u + 3] = x4[3];
  }
  float f[P::FW];
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((f[I] = feature_ct<NT, kDK, F0 + I>(x)), ...);
  }(std::make_integer_sequence<int, P::FW>{});
  if constexpr (F0 == 0) f[0] = t < nv ? 1.f : 0.f;
  float* dst = l < 32 ? &sm.pk[t][L0] : &sm.pa[t][L0];
#pragma unroll
  for (int u = 0; u < P::FW / 4; ++u)
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

// One lane per token t (< 32): J_phi(x_t)^T y[., t] over the wavefront's features F0 .. F0 + FW - 1,
// into its row of part.
template <int NT, int F0, class SM>
__device__ __forceinline__ void jacobian_w(SM& sm, int w, int t, bool of_a) {
  using P = WB<NT>;
  constexpr int L0 = F0 % P::FB;
  const float* xr = of_a ? &sm.xa[t][0] : &sm.xk[t][0];
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
  }(std::make_integer_sequence<int, P::FW>{});
#pragma unroll
  for (int c = 0; c < kDK; ++c) sm.part[w][t][c] = d[c];
}

// Block 0, intra-chunk: wm[i][j] = K_n(s_ij), dm[i][j] = (gg_i . v_j - go_i) K_{n-1}(s_ij) for key
// j <= query i (zero above the diagonal).  Waves 0..3 take the four 16x16 tiles.
template <int NT, class SM>
__device__ __forceinline__ void intra_weights(SM& sm, int w, int i16, int lg) {
  if (w >= 4) return;
  const int it = w >> 1, jt = w & 1;
  f32x4 sc = {0.f, 0.f, 0.f, 0.f}, gv = {0.f, 0.f, 0.f, 0.f};
  if (jt <= it) {
#pragma unroll
    for (int s = 0; s < 4; ++s) sc = mfma(sm.xa[16 * it + i16][4 * s + lg], sm.xk[16 * jt + i16][4 * s + lg], sc);
#pragma unroll
    for (int s = 0; s < 16; ++s) gv = mfma(sm.gg[16 * it + i16][4 * s + lg], sm.v[16 * jt + i16][4 * s + lg], gv);
  }
  // sc[r], gv[r]: query i = 16 it + 4 lg + r, key j = 16 jt + i16
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * it + 4 * lg + r, j = 16 * jt + i16;
    const bool ok = j <= i;
    sm.wm[i][j] = ok ? taylor_kernel<NT>(sc[r]) : 0.f;
    sm.dm[i][j] = ok ? (gv[r] - sm.go[i]) * taylor_kernel<NT - 1>(sc[r]) : 0.f;
  }
}

// Pass A: one workgroup per (block, pair), chunks in order.  Writes per token: den_part[block] and
// p16[block] = J_phi_B(a)^T (S_B g - z_B (g . o)) (block 0: plus the intra-chunk parts), both times
// the factors described in the file comment (sigma applied here, 1 / den in reduce 1).
template <int NT>
__global__ __launch_bounds__(kThreads) void bwdw_a_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                          const void* __restrict__ v, const float* __restrict__ g,
                                                          const float* __restrict__ o, const float* __restrict__ state,
                                                          float* __restrict__ den_part, float* __restrict__ p16,
                                                          int N, long long stride, float scale, int bf16,
                                                          long long T) {
  using P = WB<NT>;
  constexpr int FB = P::FB, NFT = P::NFT, W = P::W;
  __shared__ WBSmem<NT, true> sm;
  const int tid = threadIdx.x, l = tid & 63, i16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fb = blockIdx.x;
  const long long bh = blockIdx.y;
  const int f0 = fb * FB;
  for (int e = tid; e < FB * kDV; e += kThreads) {
    const int f = e >> 6, dd = e & 63;
    sm.st[f][dd] = (state && f0 + f < W) ? state[bh * stride + (long long)(f0 + f) * kDV + dd] : 0.f;
  }
  for (int f = tid; f < FB; f += kThreads)
    sm.zz[f] = (state && f0 + f < W) ? state[bh * stride + (long long)W * kDV + f0 + f] : 0.f;
  const int nch = (N + kC - 1) / kC;
  const bool bf = bf16 != 0;
  ChunkIn in;
  load_a(in, q, k, v, g, o, bh * N, min(kC, N), bf, tid);
  for (int c = 0; c < nch; ++c) {
    const int nv = min(kC, N - c * kC);
    const long long tok0 = bh * N + (long long)c * kC;
    __syncthreads();  // the previous chunk's readers are done
    store_chunk<true>(sm, in, scale, tid);
    if (c + 1 < nch) load_a(in, q, k, v, g, o, tok0 + kC, min(kC, N - (c + 1) * kC), bf, tid);
    __syncthreads();
    dispatch_index<0, P::NB * kWaves>(slot_of(fb, w), [&](auto I) { expand_w<NT, decltype(I)::value * P::FW>(sm, l, nv); });
    __syncthreads();
    // Y = S g - z (g . o), feature-major (S, z before this chunk)
    for (int u = w; u < 2 * NFT; u += kWaves) {
      const int ft = u >> 1, tt = u & 1;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s) acc = mfma(sm.st[16 * ft + i16][4 * s + lg], sm.gg[16 * tt + i16][4 * s + lg], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * ft + 4 * lg + r, t = 16 * tt + i16;
        sm.y[f][t] = acc[r] - sm.zz[f] * sm.go[t];
      }
    }
    {
      // den part of token t: phi_B(a_t) . z_B, in 16 partial sums over features p, p + 16, ...
      const int t = tid & 31, p = tid >> 5;
      float acc = 0.f;
#pragma unroll
      for (int f = p; f < FB; f += 16) acc = fmaf(sm.pa[t][f], sm.zz[f], acc);
      sm.dred[p][t] = acc;
    }
    __syncthreads();
    // S += phi_B(K)^T V, z += phi_B(K)^T 1
    for (int u = w; u < 4 * NFT; u += kWaves) {
      const int ft = u >> 2, dt = u & 3;
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sm.st[16 * ft + 4 * lg + r][16 * dt + i16];
#pragma unroll
      for (int s = 0; s < kC / 4; ++s) acc = mfma(sm.pk[4 * s + lg][16 * ft + i16], sm.v[4 * s + lg][16 * dt + i16], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.st[16 * ft + 4 * lg + r][16 * dt + i16] = acc[r];
    }
    for (int f = tid; f < FB; f += kThreads) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < kC; ++t) acc += sm.pk[t][f];
      sm.zz[f] += acc;
    }
    if (l < 32)
      dispatch_index<0, P::NB * kWaves>(slot_of(fb, w), [&](auto I) { jacobian_w<NT, decltype(I)::value * P::FW>(sm, w, l, true); });
    __syncthreads();
    if (fb == 0) {
      intra_weights<NT>(sm, w, i16, lg);
      __syncthreads();
      if (w < 2) {
        // sum_j dm[i][j] k_j over the chunk: rows 16 w .. 16 w + 15
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kC / 4; ++s) acc = mfma(sm.dm[16 * w + i16][4 * s + lg], sm.xk[4 * s + lg][i16], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.part[kWaves][16 * w + 4 * lg + r][i16] = acc[r];
      } else if (w == 2 && l < kC) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < kC; ++j) acc += sm.wm[l][j];
        sm.dintra[l] = acc;
      }
      __syncthreads();
    }
    {
      const int t = tid >> 4, cc = tid & 15;
      if (t < nv) {
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < kWaves; ++u) s += sm.part[u][t][cc];
        if (fb == 0) s += sm.part[kWaves][t][cc];
        p16[((long long)fb * T + tok0 + t) * kDK + cc] = scale * s;
        if (cc == 0) {
          float dn = 0.f;
#pragma unroll
          for (int p = 0; p < 16; ++p) dn += sm.dred[p][t];
          if (fb == 0) dn += sm.dintra[t];
          den_part[(long long)fb * T + tok0 + t] = dn;
        }
      }
    }
  }
}

// Reduce 1, one wavefront per token: den = sum of the block parts (block order), dq = p16 sum / den,
// gh = g / den, delta = g . o / den.
__global__ __launch_bounds__(256) void bwdw_r1_kernel(const float* __restrict__ den_part, const float* __restrict__ p16,
                                                      const float* __restrict__ g, const float* __restrict__ o,
                                                      float* __restrict__ ghd, float* __restrict__ dq, int NB,
                                                      long long T) {
  const long long tok = blockIdx.x * 4ll + (threadIdx.x >> 6);
  const int d = threadIdx.x & 63;
  if (tok >= T) return;
  float den = 0.f;
  for (int b = 0; b < NB; ++b) den += den_part[(long long)b * T + tok];
  const float gv = g[tok * kDV + d];
  float go = gv * o[tok * kDV + d];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) go += __shfl_xor(go, m, 64);
  ghd[tok * kLG + d] = gv / den;
  if (d == 0) ghd[tok * kLG + kDV] = go / den;
  if (d < kDK) {
    float s = 0.f;
    for (int b = 0; b < NB; ++b) s += p16[((long long)b * T + tok) * kDK + d];
    dq[tok * kDK + d] = s / den;
  }
}

// Pass B: one workgroup per (block, pair), chunks in reverse.  Writes per token the dv and dk parts of
// the block (block 0: plus the intra-chunk parts), and the block's rows of the incoming state's
// gradient.
template <int NT>
__global__ __launch_bounds__(kThreads) void bwdw_b_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                          const void* __restrict__ v, const float* __restrict__ ghd,
                                                          float* __restrict__ dstate, float* __restrict__ p16,
                                                          float* __restrict__ pdv, int N, long long stride,
                                                          float scale, int bf16, long long T) {
  using P = WB<NT>;
  constexpr int FB = P::FB, NFT = P::NFT, W = P::W;
  __shared__ WBSmem<NT, false> sm;
  const int tid = threadIdx.x, l = tid & 63, i16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fb = blockIdx.x;
  const long long bh = blockIdx.y;
  const int f0 = fb * FB;
  for (int e = tid; e < FB * kDV; e += kThreads) {
    const int f = e >> 6, dd = e & 63;
    sm.st[f][dd] = (dstate && f0 + f < W) ? dstate[bh * stride + (long long)(f0 + f) * kDV + dd] : 0.f;
  }
  for (int f = tid; f < FB; f += kThreads)
    sm.zz[f] = (dstate && f0 + f < W) ? dstate[bh * stride + (long long)W * kDV + f0 + f] : 0.f;
  const int nch = (N + kC - 1) / kC;
  const int tt = w >> 2, dt = w & 3;  // this wavefront's 16x16 tile of the chunk's dv
  const bool bf = bf16 != 0;
  ChunkIn in;
  load_b(in, q, k, v, ghd, bh * N + (long long)(nch - 1) * kC, N - (nch - 1) * kC, bf, tid);
  for (int c = nch - 1; c >= 0; --c) {
    const int nv = min(kC, N - c * kC);
    const long long tok0 = bh * N + (long long)c * kC;
    __syncthreads();
    store_chunk<false>(sm, in, scale, tid);
    if (c > 0) load_b(in, q, k, v, ghd, tok0 - kC, kC, bf, tid);
    __syncthreads();
    dispatch_index<0, P::NB * kWaves>(slot_of(fb, w), [&](auto I) { expand_w<NT, decltype(I)::value * P::FW>(sm, l, nv); });
    __syncthreads();
    // dv part = phi_B(K) G_S (G of the later tokens); Y = G_S v + G_z, feature-major
    f32x4 dva = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int s = 0; s < FB / 4; ++s) dva = mfma(sm.pk[16 * tt + i16][4 * s + lg], sm.st[4 * s + lg][16 * dt + i16], dva);
    for (int u = w; u < 2 * NFT; u += kWaves) {
      const int ft = u >> 1, ut = u & 1;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s) acc = mfma(sm.st[16 * ft + i16][4 * s + lg], sm.v[16 * ut + i16][4 * s + lg], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * ft + 4 * lg + r;
        sm.y[f][16 * ut + i16] = acc[r] + sm.zz[f];
      }
    }
    __syncthreads();
    // G_S += phi_B(A)^T gh, G_z -= phi_B(A)^T delta
    for (int u = w; u < 4 * NFT; u += kWaves) {
      const int ft = u >> 2, ud = u & 3;
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sm.st[16 * ft + 4 * lg + r][16 * ud + i16];
#pragma unroll
      for (int s = 0; s < kC / 4; ++s) acc = mfma(sm.pa[4 * s + lg][16 * ft + i16], sm.gg[4 * s + lg][16 * ud + i16], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.st[16 * ft + 4 * lg + r][16 * ud + i16] = acc[r];
    }
    for (int f = tid; f < FB; f += kThreads) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < kC; ++t) acc = fmaf(sm.pa[t][f], sm.go[t], acc);
      sm.zz[f] -= acc;
    }
    if (l < 32)
      dispatch_index<0, P::NB * kWaves>(slot_of(fb, w), [&](auto I) { jacobian_w<NT, decltype(I)::value * P::FW>(sm, w, l, false); });
    __syncthreads();
    if (fb == 0) {
      intra_weights<NT>(sm, w, i16, lg);
      __syncthreads();
      // dv_j += sum_i wm[i][j] gh_i (the same tile as dva); dk_j += sum_i dm[i][j] a_i (waves 0, 1)
#pragma unroll
      for (int s = 0; s < kC / 4; ++s) dva = mfma(sm.wm[4 * s + lg][16 * tt + i16], sm.gg[4 * s + lg][16 * dt + i16], dva);
      if (w < 2) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kC / 4; ++s) acc = mfma(sm.dm[4 * s + lg][16 * w + i16], sm.xa[4 * s + lg][i16], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.part[kWaves][16 * w + 4 * lg + r][i16] = acc[r];
      }
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tt + 4 * lg + r;
      if (t < nv) pdv[((long long)fb * T + tok0 + t) * kDV + 16 * dt + i16] = dva[r];
    }
    {
      const int t = tid >> 4, cc = tid & 15;
      if (t < nv) {
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < kWaves; ++u) s += sm.part[u][t][cc];
        if (fb == 0) s += sm.part[kWaves][t][cc];
        p16[((long long)fb * T + tok0 + t) * kDK + cc] = s;
      }
    }
  }
  __syncthreads();
  if (dstate) {
    for (int e = tid; e < FB * kDV; e += kThreads) {
      const int f = e >> 6, dd = e & 63;
      if (f0 + f < W) dstate[bh * stride + (long long)(f0 + f) * kDV + dd] = sm.st[f][dd];
    }
    for (int f = tid; f < FB; f += kThreads)
      if (f0 + f < W) dstate[bh * stride + (long long)W * kDV + f0 + f] = sm.zz[f];
  }
}

// Reduce 2, one wavefront per token: dk, dv = sums of the block parts in block order.
__global__ __launch_bounds__(256) void bwdw_r2_kernel(const float* __restrict__ p16, const float* __restrict__ pdv,
                                                      float* __restrict__ dk, float* __restrict__ dv, int NB,
                                                      long long T) {
  const long long tok = blockIdx.x * 4ll + (threadIdx.x >> 6);
  const int d = threadIdx.x & 63;
  if (tok >= T) return;
  float s = 0.f;
  for (int b = 0; b < NB; ++b) s += pdv[((long long)b * T + tok) * kDV + d];
  dv[tok * kDV + d] = s;
  if (d < kDK) {
    float e = 0.f;
    for (int b = 0; b < NB; ++b) e += p16[((long long)b * T + tok) * kDK + d];
    dk[tok * kDK + d] = e;
  }
}

// Workspace (floats): gh and delta [T][68], then dv parts [NB][T][64], dq / dk parts [NB][T][16]
// (pass A's are consumed by reduce 1 before pass B writes its own), den parts [NB][T].
template <int NT>
long long bwdw_ws_floats(long long T) {
  return T * kLG + (long long)WB<NT>::NB * T * (kDV + kDK + 1);
}

template <int NT>
int bwdw_run(const BwdArgs& a) {
  using P = WB<NT>;
  const long long T = (long long)a.BH * a.N;
  float* ghd = (float*)a.ws;
  float* pdv = ghd + T * kLG;
  float* p16 = pdv + P::NB * T * kDV;
  float* den_part = p16 + P::NB * T * kDK;
  const int bf = a.s.dtype != 0;
  const dim3 grid(P::NB, a.BH), block(kThreads);
  const dim3 rgrid((unsigned)((T + 3) / 4)), rblock(256);
  bwdw_a_kernel<NT><<<grid, block, 0, a.stream>>>(a.q, a.k, a.v, a.g, a.o, a.state, den_part, p16, a.N, a.s.stride,
                                                  a.s.scale, bf, T);
  bwdw_r1_kernel<<<rgrid, rblock, 0, a.stream>>>(den_part, p16, a.g, a.o, ghd, a.dq, P::NB, T);
  bwdw_b_kernel<NT><<<grid, block, 0, a.stream>>>(a.q, a.k, a.v, ghd, a.dstate, p16, pdv, a.N, a.s.stride, a.s.scale,
                                                  bf, T);
  bwdw_r2_kernel<<<rgrid, rblock, 0, a.stream>>>(p16, pdv, a.dk, a.dv, P::NB, T);
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
