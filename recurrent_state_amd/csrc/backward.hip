// Backward of truncated-kernel causal attention (gfx950): dq, dk, dv and the gradient of the incoming
// state, float32 matrix cores.
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
// G at the end.  J_phi is the Jacobian of the monomial features (orders <= 2 here: n <= 3).
//
// Passes over segments of L tokens (one workgroup of 8 wavefronts per segment, 16-token chunks,
// the running state in LDS, float32 16x16x4 MFMAs with operands read from LDS):
//   1. state pass: the S, z increments of each segment;
//   2. forward scan: exclusive prefixes, seeded with the incoming state;
//   3. pass A (chunks in order): den, gh, delta (kept for pass B), dq, the segment's G increments;
//   4. reverse scan of the G increments, seeded with the final state's gradient (its total is the
//      incoming state's gradient);
//   5. pass B (chunks in reverse): dv, dk.
#include <type_traits>
#include <utility>

#include "backward.hpp"
#include "features.hpp"

namespace taylor {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDK = 16, kDV = 64;
constexpr int kC = 16;  // tokens per chunk
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLR = kDK + 4;  // LDS row strides (floats): 16-wide rows,
constexpr int kLV = kDV + 4;  // 64-wide rows,
constexpr int kLC = kC + 4;   // [query][key] tiles

template <int NT>
struct BG {
  static constexpr int W = FeatureTable<NT, kDK>::W;
  static constexpr int WP = (W + 15) / 16 * 16;  // features padded to 16-row tiles
  static constexpr int FPW = WP / kWaves;         // features per wavefront (expansion, Jacobian)
  static constexpr int LF = WP + 4;
  static constexpr int NFT = WP / 16;             // feature tiles
  static constexpr int NTILE = NFT * (kDV / 16);  // 16x16 tiles of a state
  static constexpr int TPW = (NTILE + kWaves - 1) / kWaves;
};

template <int NT>
struct BSmem {
  using G = BG<NT>;
  alignas(16) float st[G::WP][kLV];  // S (pass A) or G_S (pass B); rows past W stay zero
  float zt[G::WP];                   // z or G_z
  alignas(16) float phia[kC][G::LF];
  alignas(16) float phik[kC][G::LF];
  alignas(16) float ar[kC][kLR];  // a = sigma q
  alignas(16) float kr[kC][kLR];
  alignas(16) float vr[kC][kLV];
  alignas(16) float gr[kC][kLV];  // g, then gh
  float wt[kC][kLC], kp[kC][kLC], ds[kC][kLC];  // [query i][key j]
  alignas(16) float y[kC][G::LF];
  float dpart[kWaves][kC][kDK + 1];
  float den[kC], delta[kC], go[kC];  // go: g . o
};

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const uint16_t* p) { return __uint_as_float(((uint32_t)*p) << 16); }

// acc += A B over K (a multiple of 4), one 16x16 output tile: a(m, k) and b(k, n) read LDS (m, n in
// 0..15).  Lane (l16, lg) holds D[4lg + r][l16] in element r.
template <int K, class FA, class FB>
__device__ __forceinline__ f32x4 mm(f32x4 acc, int l16, int lg, FA a, FB b) {
#pragma unroll
  for (int k = 0; k < K; k += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(l16, k + lg), b(k + lg, l16), acc, 0, 0, 0);
  return acc;
}

// Features of wavefront w's share [w FPW, (w+1) FPW) for the chunk's tokens: lanes 0..15 phi(k) of
// token l, lanes 16..31 phi(a) of token l - 16 (WITH_A).  Tokens past the end have zero rows; their
// constant feature is zeroed too.
template <int NT, bool WITH_A>
__device__ __forceinline__ void expand(BSmem<NT>& sm, int w, int l, int nv) {
  using G = BG<NT>;
  if (l >= (WITH_A ? 2 * kC : kC)) return;
  const int t = l & (kC - 1);
  const bool is_a = l >= kC;
  float x[kDK];
#pragma unroll
  for (int d = 0; d < kDK; ++d) x[d] = is_a ? sm.ar[t][d] : sm.kr[t][d];
  float* dst = is_a ? &sm.phia[t][0] : &sm.phik[t][0];
  const bool valid = t < nv;
  dispatch_index<0, kWaves>(w, [&](auto WI) {
    constexpr int F0 = decltype(WI)::value * G::FPW;
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (([&] {
         constexpr int F = F0 + I;
         float f = feature_ct<NT, kDK, F>(x);
         if constexpr (F == 0) f = valid ? 1.f : 0.f;
         dst[F] = f;
       }()),
       ...);
    }(std::make_integer_sequence<int, G::FPW>{});
  });
}

// out += J_phi(x)^T y over wavefront w's share of the features (orders <= 2): order 1 feature e_c
// adds y to out[c]; order 2 feature c * x_c0 x_c1 adds c y x_c1 to out[c0] and c y x_c0 to out[c1].
template <int NT>
__device__ __forceinline__ void feature_vjp(int w, const float (&x)[kDK], const float* y, float (&out)[kDK]) {
  using G = BG<NT>;
  using FT = FeatureTable<NT, kDK>;
  dispatch_index<0, kWaves>(w, [&](auto WI) {
    constexpr int F0 = decltype(WI)::value * G::FPW;
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (([&] {
         constexpr int F = F0 + I;
         if constexpr (F < G::W) {
           constexpr int m = FT::T.order[F];
           if constexpr (m == 1) {
             out[FT::T.coord[F][0]] += y[F];
           } else if constexpr (m == 2) {
             constexpr int c0 = FT::T.coord[F][0], c1 = FT::T.coord[F][1];
             constexpr float cf = coef_of_afact(FT::T.afact[F]);
             const float t = cf * y[F];
             out[c0] = fmaf(t, x[c1], out[c0]);
             out[c1] = fmaf(t, x[c0], out[c1]);
           }
         }
       }()),
       ...);
    }(std::make_integer_sequence<int, G::FPW>{});
  });
}

// One thread's share of a chunk's input rows, loaded a chunk ahead (registers) and stored to LDS when
// the chunk starts, so the global loads of chunk c+1 are in flight while chunk c is computed.
// Element tid of k (tid < 256) or of a = sigma q (tid >= 256); elements tid and tid + 512 of v and of
// g (pass A) or gh (pass B), and of o (pass A: g . o is reduced per token at the store); delta
// (pass B, tid < 16).  Rows past the end are zero.  MODE 0: k, v; 1: pass A; 2: pass B.
template <typename E, int MODE>
struct Pre {
  float kq, v[2], g[2], o[2], dl;
  __device__ __forceinline__ void load(const E* q, const E* k, const E* vg, const float* gg, const float* og,
                                       const float* dlt, long long tok0, int nv, float scale, int tid) {
    // every load reads a valid row (tokens past the end read the chunk's first) and is masked after,
    // so no load is conditional
    const int e = tid & 255, i = e / kDK, d = e % kDK;
    const bool ok = i < nv;
    const long long rk = (tok0 + (ok ? i : 0)) * kDK + d;
    float x = 0.f;
    if (tid < 256)
      x = ld(k + rk);
    else if (MODE != 0)
      x = scale * ld(q + rk);
    kq = ok ? x : 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = (tid >> 6) + 8 * u, c = tid & 63;
      const bool okt = t < nv;
      const long long r = (tok0 + (okt ? t : 0)) * kDV + c;
      const float xv = ld(vg + r);
      v[u] = okt ? xv : 0.f;
      if constexpr (MODE != 0) {
        const float xg = gg[r];
        g[u] = okt ? xg : 0.f;
      } else {
        g[u] = 0.f;
      }
      if constexpr (MODE == 1) {
        const float xo = og[r];
        o[u] = okt ? xo : 0.f;
      } else {
        o[u] = 0.f;
      }
    }
    dl = 0.f;
    if constexpr (MODE == 2) {
      const float xd = dlt[tok0 + (tid < kC && tid < nv ? tid : 0)];
      dl = (tid < kC && tid < nv) ? xd : 0.f;
    }
  }
  template <int NT>
  __device__ __forceinline__ void store(BSmem<NT>& sm, int tid) const {
    const int e = tid & 255, i = e / kDK, d = e % kDK;
    if (tid < 256)
      sm.kr[i][d] = kq;
    else if (MODE != 0)
      sm.ar[i][d] = kq;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = (tid >> 6) + 8 * u, c = tid & 63;
      sm.vr[t][c] = v[u];
      if constexpr (MODE != 0) sm.gr[t][c] = g[u];
      if constexpr (MODE == 1) {
        float go = g[u] * o[u];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) go += __shfl_xor(go, off);
        if (c == 0) sm.go[t] = go;
      }
    }
    if (MODE == 2 && tid < kC) sm.delta[tid] = dl;
  }
};

// Wavefront 0: the chunk's weights w_ij = K_n(s_ij) and K_{n-1}(s_ij) for keys j <= i (zero else),
// then ds_ij = (gh_i . v_j - delta_i) K_{n-1}(s_ij).  Needs gh, delta.
template <int NT>
__device__ __forceinline__ void weights(BSmem<NT>& sm, int l16, int lg, int nv) {
  const f32x4 sc = mm<kDK>(f32x4{0.f, 0.f, 0.f, 0.f}, l16, lg, [&](int m, int kk) { return sm.kr[m][kk]; },
                           [&](int kk, int n) { return sm.ar[n][kk]; });
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 4 * lg + r, i = l16;  // D[key j][query i]
    const bool ok = j <= i && j < nv;
    const float s = sc[r];
    sm.wt[i][j] = ok ? taylor_kernel<NT>(s) : 0.f;
    float d = 0.f;
    if constexpr (NT > 1) d = taylor_kernel<NT - 1>(s);
    sm.kp[i][j] = ok ? d : 0.f;
  }
}

template <int NT>
__device__ __forceinline__ void dscores(BSmem<NT>& sm, int l16, int lg) {
  const f32x4 dw = mm<kDV>(f32x4{0.f, 0.f, 0.f, 0.f}, l16, lg, [&](int m, int kk) { return sm.gr[m][kk]; },
                           [&](int kk, int n) { return sm.vr[n][kk]; });
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * lg + r, j = l16;  // D[query i][key j]
    sm.ds[i][j] = (dw[r] - sm.delta[i]) * sm.kp[i][j];
  }
}

// Pass 1 (MODE 0: S, z increments of each segment) and pass A (MODE 1).  grid = (segments, pairs).
template <int NT, typename E, int MODE>
__global__ __launch_bounds__(kThreads) void bwd_forward_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                               const E* __restrict__ v, const float* __restrict__ g,
                                                               const float* __restrict__ o,
                                                               float* __restrict__ sslots,
                                                               float* __restrict__ gslots,
                                                               float* __restrict__ ghat, float* __restrict__ dlt,
                                                               float* __restrict__ dq, SeqMap seq, int L,
                                                               long long nslot, long long stride, float scale) {
  using G = BG<NT>;
  constexpr int W = G::W, WP = G::WP;
  __shared__ BSmem<NT> sm;
  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  for_each_piece<false>(seq, blockIdx.x, blockIdx.y, L, nslot, [&](const SeqPiece& pc) __attribute__((always_inline)) {
    float* sslot = sslots + pc.slot * stride;
    float* gslot = gslots + pc.slot * stride;
    // the running S, z: zero (increments) or the segment's prefix
    for (int e = tid; e < WP * kDV; e += kThreads) {
      const int f = e / kDV, d = e % kDV;
      sm.st[f][d] = (MODE == 1 && f < W) ? sslot[(long long)f * kDV + d] : 0.f;
    }
    for (int f = tid; f < WP; f += kThreads) sm.zt[f] = (MODE == 1 && f < W) ? sslot[(long long)W * kDV + f] : 0.f;
    f32x4 gacc[G::TPW];  // G_S increments, tiles w, w + 8, ...
#pragma unroll
    for (int u = 0; u < G::TPW; ++u) gacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    float gz = 0.f;  // G_z increment of feature tid
    const int nch = (pc.n + kC - 1) / kC;
    auto nv_of = [&](int c) { return min(kC, pc.n - c * kC); };
    auto tok_of = [&](int c) { return pc.tok + (long long)c * kC; };
    Pre<E, MODE> pre;
    pre.load(q, k, v, g, o, nullptr, tok_of(0), nv_of(0), scale, tid);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      const int nv = nv_of(c);
      const long long tok0 = tok_of(c);
      pre.store(sm, tid);
      const int cn = c + 1 < nch ? c + 1 : c;  // the last chunk reloads itself (no conditional load)
      pre.load(q, k, v, g, o, nullptr, tok_of(cn), nv_of(cn), scale, tid);
      __syncthreads();
      expand<NT, MODE == 1>(sm, w, l, nv);
      __syncthreads();
      if constexpr (MODE == 1) {
        if (w == 0) {
          weights<NT>(sm, l16, lg, nv);
        } else if (w == 1) {
          // phi(a_i) . z over the tokens before the chunk: 4 lanes per token
          float acc = 0.f;
          for (int f = lg; f < WP; f += 4) acc = fmaf(sm.phia[l16][f], sm.zt[f], acc);
          acc += __shfl_xor(acc, 16);
          acc += __shfl_xor(acc, 32);
          if (lg == 0) sm.den[l16] = acc;
        }
        __syncthreads();
        // gh, delta: wavefront w takes tokens 2w, 2w + 1, lane = value column
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int t = 2 * w + u;
          float dn = sm.den[t];
#pragma unroll
          for (int j = 0; j < kC; ++j) dn += sm.wt[t][j];
          const float gv = sm.gr[t][l];
          const bool ok = t < nv;
          const float inv = ok ? 1.0f / dn : 0.f;
          const float gh = gv * inv, dl = sm.go[t] * inv;
          sm.gr[t][l] = gh;
          if (l == 0) sm.delta[t] = dl;
          if (ok) {
            ghat[(tok0 + t) * kDV + l] = gh;
            if (l == 0) dlt[tok0 + t] = dl;
          }
        }
        __syncthreads();
        if (w == 0) dscores<NT>(sm, l16, lg);
        // Y = gh S^T - delta z^T, feature tiles w, w + 8, ...
        for (int t = w; t < G::NFT; t += kWaves) {
          const f32x4 yv = mm<kDV>(f32x4{0.f, 0.f, 0.f, 0.f}, l16, lg, [&](int m, int kk) { return sm.gr[m][kk]; },
                                   [&](int kk, int n) { return sm.st[16 * t + n][kk]; });
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * lg + r, f = 16 * t + l16;
            sm.y[i][f] = yv[r] - sm.delta[i] * sm.zt[f];
          }
        }
        __syncthreads();
        // dq: the Jacobian over this wavefront's features (lanes 0..15 = tokens), and (wavefront 0)
        // the intra-chunk sum_j ds_ij k_j into wt
        if (l < kC) {
          float x[kDK], out[kDK];
#pragma unroll
          for (int d = 0; d < kDK; ++d) {
            x[d] = sm.ar[l][d];
            out[d] = 0.f;
          }
          feature_vjp<NT>(w, x, &sm.y[l][0], out);
#pragma unroll
          for (int d = 0; d < kDK; ++d) sm.dpart[w][l][d] = out[d];
        }
        if (w == 0) {
          const f32x4 di = mm<kC>(f32x4{0.f, 0.f, 0.f, 0.f}, l16, lg, [&](int m, int kk) { return sm.ds[m][kk]; },
                                  [&](int kk, int n) { return sm.kr[kk][n]; });
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.wt[4 * lg + r][l16] = di[r];
        }
        __syncthreads();
        if (tid < kC * kDK) {
          const int i = tid / kDK, d = tid % kDK;
          float s = sm.wt[i][d];
#pragma unroll
          for (int ww = 0; ww < kWaves; ++ww) s += sm.dpart[ww][i][d];
          if (i < nv) dq[(tok0 + i) * kDK + d] = scale * s;
        }
      }
      // S += phi(K)^T V, z += sum phi(k); pass A also G_S += phi(A)^T gh, G_z -= phi(A)^T delta
#pragma unroll
      for (int u = 0; u < G::TPW; ++u) {
        const int t = w + u * kWaves;
        if (t < G::NTILE) {
          const int ft = t / (kDV / 16), dt = t % (kDV / 16);
          f32x4 acc;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = sm.st[16 * ft + 4 * lg + r][16 * dt + l16];
          acc = mm<kC>(acc, l16, lg, [&](int m, int kk) { return sm.phik[kk][16 * ft + m]; },
                       [&](int kk, int n) { return sm.vr[kk][16 * dt + n]; });
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.st[16 * ft + 4 * lg + r][16 * dt + l16] = acc[r];
          if constexpr (MODE == 1)
            gacc[u] = mm<kC>(gacc[u], l16, lg, [&](int m, int kk) { return sm.phia[kk][16 * ft + m]; },
                             [&](int kk, int n) { return sm.gr[kk][16 * dt + n]; });
        }
      }
      if (tid < WP) {
        float sz = 0.f, sg = 0.f;
#pragma unroll
        for (int j = 0; j < kC; ++j) {
          sz += sm.phik[j][tid];
          if constexpr (MODE == 1) sg = fmaf(sm.phia[j][tid], sm.delta[j], sg);
        }
        sm.zt[tid] += sz;
        gz -= sg;
      }
      __syncthreads();
    }
    if constexpr (MODE == 0) {
      for (int e = tid; e < W * kDV; e += kThreads) sslot[e] = sm.st[e / kDV][e % kDV];
      for (int f = tid; f < W; f += kThreads) sslot[(long long)W * kDV + f] = sm.zt[f];
    } else {
#pragma unroll
      for (int u = 0; u < G::TPW; ++u) {
        const int t = w + u * kWaves;
        if (t < G::NTILE) {
          const int ft = t / (kDV / 16), dt = t % (kDV / 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int f = 16 * ft + 4 * lg + r;
            if (f < W) gslot[(long long)f * kDV + 16 * dt + l16] = gacc[u][r];
          }
        }
      }
      if (tid < W) gslot[(long long)W * kDV + tid] = gz;
    }
    __syncthreads();
  });
}

// Pass B: chunks in reverse, the running G (the gradient of the state after the chunk) in LDS,
// seeded with the segment's suffix from the reverse scan.  grid = (segments, pairs).
template <int NT, typename E>
__global__ __launch_bounds__(kThreads) void bwd_reverse_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                               const E* __restrict__ v,
                                                               const float* __restrict__ gslots,
                                                               const float* __restrict__ ghat,
                                                               const float* __restrict__ dlt, float* __restrict__ dk,
                                                               float* __restrict__ dv, SeqMap seq, int L,
                                                               long long nslot, long long stride, float scale) {
  using G = BG<NT>;
  constexpr int W = G::W, WP = G::WP;
  __shared__ BSmem<NT> sm;
  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  for_each_piece<false>(seq, blockIdx.x, blockIdx.y, L, nslot, [&](const SeqPiece& pc) __attribute__((always_inline)) {
    const float* gslot = gslots + pc.slot * stride;
    for (int e = tid; e < WP * kDV; e += kThreads) {
      const int f = e / kDV, d = e % kDV;
      sm.st[f][d] = f < W ? gslot[(long long)f * kDV + d] : 0.f;
    }
    for (int f = tid; f < WP; f += kThreads) sm.zt[f] = f < W ? gslot[(long long)W * kDV + f] : 0.f;
    const int nch = (pc.n + kC - 1) / kC;
    auto nv_of = [&](int c) { return min(kC, pc.n - c * kC); };
    auto tok_of = [&](int c) { return pc.tok + (long long)c * kC; };
    Pre<E, 2> pre;
    pre.load(q, k, v, ghat, nullptr, dlt, tok_of(nch - 1), nv_of(nch - 1), scale, tid);
    __syncthreads();
    for (int c = nch - 1; c >= 0; --c) {
      const int nv = nv_of(c);
      const long long tok0 = tok_of(c);
      pre.store(sm, tid);
      const int cn = c > 0 ? c - 1 : c;  // the first chunk reloads itself (no conditional load)
      pre.load(q, k, v, ghat, nullptr, dlt, tok_of(cn), nv_of(cn), scale, tid);
      __syncthreads();
      expand<NT, true>(sm, w, l, nv);
      __syncthreads();
      if (w == 0) {
        weights<NT>(sm, l16, lg, nv);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        dscores<NT>(sm, l16, lg);
      }
      __syncthreads();
      if (w < kDV / 16) {
        // dv, value tile dt = w: sum_{i>=j} w_ij gh_i (intra) + phi(k_j)^T G_S
        const int dt = w;
        f32x4 acc = mm<kC>(f32x4{0.f, 0.f, 0.f, 0.f}, l16, lg, [&](int m, int kk) { return sm.wt[kk][m]; },
                           [&](int kk, int n) { return sm.gr[kk][16 * dt + n]; });
        acc = mm<WP>(acc, l16, lg, [&](int m, int kk) { return sm.phik[m][kk]; },
                     [&](int kk, int n) { return sm.st[kk][16 * dt + n]; });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 4 * lg + r;
          if (j < nv) dv[(tok0 + j) * kDV + 16 * dt + l16] = acc[r];
        }
      } else {
        // Z = V G_S^T + G_z, feature tiles w - 4, w, w + 4, ...
        for (int t = w - kDV / 16; t < G::NFT; t += kWaves - kDV / 16) {
          const f32x4 zv = mm<kDV>(f32x4{0.f, 0.f, 0.f, 0.f}, l16, lg, [&](int m, int kk) { return sm.vr[m][kk]; },
                                   [&](int kk, int n) { return sm.st[16 * t + n][kk]; });
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.y[4 * lg + r][16 * t + l16] = zv[r] + sm.zt[16 * t + l16];
        }
      }
      __syncthreads();
      // dk: the Jacobian over this wavefront's features (lanes 0..15 = tokens), and (wavefront 0) the
      // intra-chunk sum_{i>=j} ds_ij a_i into wt
      if (l < kC) {
        float x[kDK], out[kDK];
#pragma unroll
        for (int d = 0; d < kDK; ++d) {
          x[d] = sm.kr[l][d];
          out[d] = 0.f;
        }
        feature_vjp<NT>(w, x, &sm.y[l][0], out);
#pragma unroll
        for (int d = 0; d < kDK; ++d) sm.dpart[w][l][d] = out[d];
      }
      if (w == 0) {
        const f32x4 di = mm<kC>(f32x4{0.f, 0.f, 0.f, 0.f}, l16, lg, [&](int m, int kk) { return sm.ds[kk][m]; },
                                [&](int kk, int n) { return sm.ar[kk][n]; });
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.wt[4 * lg + r][l16] = di[r];
      }
      __syncthreads();
      if (tid < kC * kDK) {
        const int j = tid / kDK, d = tid % kDK;
        float s = sm.wt[j][d];
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) s += sm.dpart[ww][j][d];
        if (j < nv) dk[(tok0 + j) * kDK + d] = s;
      }
      // G_S += phi(A)^T gh, G_z -= phi(A)^T delta
#pragma unroll
      for (int u = 0; u < G::TPW; ++u) {
        const int t = w + u * kWaves;
        if (t < G::NTILE) {
          const int ft = t / (kDV / 16), dt = t % (kDV / 16);
          f32x4 acc;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = sm.st[16 * ft + 4 * lg + r][16 * dt + l16];
          acc = mm<kC>(acc, l16, lg, [&](int m, int kk) { return sm.phia[kk][16 * ft + m]; },
                       [&](int kk, int n) { return sm.gr[kk][16 * dt + n]; });
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.st[16 * ft + 4 * lg + r][16 * dt + l16] = acc[r];
        }
      }
      if (tid < WP) {
        float sg = 0.f;
#pragma unroll
        for (int i = 0; i < kC; ++i) sg = fmaf(sm.phia[i][tid], sm.delta[i], sg);
        sm.zt[tid] -= sg;
      }
      __syncthreads();
    }
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
    const float t = p[s * stride];
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

// Segments: about 256 workgroups (one per CU: the LDS holds the running state), never more than the
// chunks.
BwdPlan plan_for(int BH, int N) {
  const int nchunk = cdiv(N, kC);
  long long want = (256 + BH - 1) / BH;
  if (want < 1) want = 1;
  if (want > nchunk) want = nchunk;
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
  bwd_forward_kernel<NT, E, 0><<<grid, block, 0, a.stream>>>(q, k, v, nullptr, nullptr, sslots, nullptr, nullptr,
                                                              nullptr, nullptr, seq, p.L, p.nseg, a.s.stride,
                                                              a.s.scale);
  bwd_scan_kernel<<<sgrid, sblock, 0, a.stream>>>(sslots, a.state, p.nseg, a.s.stride, elems, seq, p.L);
  bwd_forward_kernel<NT, E, 1><<<grid, block, 0, a.stream>>>(q, k, v, a.g, a.o, sslots, gslots, ghat, dlt, a.dq, seq,
                                                              p.L, p.nseg, a.s.stride, a.s.scale);
  bwd_rscan_kernel<<<sgrid, sblock, 0, a.stream>>>(gslots, a.dstate, p.nseg, a.s.stride, elems, seq, p.L);
  bwd_reverse_kernel<NT, E><<<grid, block, 0, a.stream>>>(q, k, v, gslots, ghat, dlt, a.dk, a.dv, seq, p.L, p.nseg,
                                                          a.s.stride, a.s.scale);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

bool backward_has(int nt, int dk, int dv) { return dk == kDK && dv == kDV && nt >= 1 && nt <= 3; }

long long backward_ws_bytes(const Shape& s, int BH, int N) {
  if (BH == 0 || N == 0) return 0;
  const BwdPlan p = plan_for(BH, N);
  return (2 * (long long)BH * p.nseg * s.stride + (long long)BH * N * (kDV + 1)) * 4;
}

int backward_launch(const BwdArgs& a) {
  if (!backward_has(a.s.nt, a.s.dk, a.s.dv)) return -2;
  switch (a.s.nt) {
    case 1: return a.s.dtype == 0 ? bwd_run<1, float>(a) : bwd_run<1, uint16_t>(a);
    case 2: return a.s.dtype == 0 ? bwd_run<2, float>(a) : bwd_run<2, uint16_t>(a);
    default: return a.s.dtype == 0 ? bwd_run<3, float>(a) : bwd_run<3, uint16_t>(a);
  }
}

}  // namespace taylor
