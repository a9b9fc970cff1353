// MFMA chunked prefill for wide feature sets: d_k = 16, d_v = 64, n = 4, 5 (W = 969, 4,845), gfx950.
//
// "Expanding Attention" (Huang, arXiv:2610.20637), Abstract: with exp truncated to n Taylor terms and
// each term factorised into symmetric tensor-power features, the causal history is n additive states,
// so prefill is chunk-local work plus a scan of chunk states.  Per chunk c, with V1 = [V | 1]:
//     O_c  = phi(s Q_c) S_{<c}  +  tril(K_n(s Q_c K_c^T)) V1_c,      S += phi(K_c)^T V1_c,
//     o    = O_c[:, :d_v] / O_c[:, d_v].
// At n = 4, 5 the state (W x 65 floats per head, up to 1.26 MB) fits neither registers nor LDS.  But
// each feature row of S evolves on its own (S_f += phi_f(K_c)^T V1_c involves only features f), and the
// readout phi(sQ) S_{<c} = sum_f phi_f(sQ) S_{f,<c} is a sum over feature blocks f.  So the work is split
// over (segment, head, block of 128 features):
//   * a workgroup of 4 wavefronts walks the chunks of its segment for one feature block; wave w keeps
//     value columns 16w..16w+15 of the block's state slice in MFMA accumulator registers and the block's
//     z lives in LDS;
//   * per chunk all four waves expand the block's features of the chunk's k and sq rows into LDS (one
//     token per lane, 32 features per wave, coordinates fixed at compile time per block), then each wave
//     runs the float32 16x16x4 MFMAs of its columns: readout with S_{<c}, then the state update;
//   * the block's partial numerators phi_f(sQ) S_{f,<c} and partial denominators phi_f(sQ) z_{f,<c} go
//     to a workspace; block 0 also adds the intra-chunk term; a reduction kernel sums the blocks in
//     order and divides.
// Segments, when (head, block) pairs alone do not fill the chip: a state pass writes each segment's
// increment, the scan turns them into exclusive prefixes and the readout pass starts from them.  With
// one segment the readout pass starts from the incoming state and writes the final state itself.
// bfloat16 inputs are widened to float32 on load; all matrix work and accumulation is float32.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "features.hpp"
#include "prefill_wide.hpp"

namespace taylor {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDK = 16, kDV = 64;
constexpr int kCS = 64;          // tokens per chunk
constexpr int kFB = 128;         // features per block
constexpr int kSub = kFB / 4;    // features per wave in the expansion
constexpr int kNAT = kFB / 16;   // 16-row tiles of the block's state slice
constexpr int kNIT = kCS / 16;   // 16-token tiles of a chunk
constexpr int kPairs = kNIT * (kNIT + 1) / 2;
constexpr int kThreads = 256;
constexpr int kLS = kCS + 4;     // phi(K)^T and V^T row stride in floats (68 = 4 mod 64 banks)
constexpr int kLQ = kFB + 4;     // phi(sQ) row stride in floats (132 = 4 mod 64 banks)

template <int NT>
constexpr int n_blocks() {
  return (FeatureTable<NT, kDK>::W + kFB - 1) / kFB;
}

template <bool READOUT>
struct WideSmem {
  static constexpr int RQ = READOUT ? kCS : 1;
  static constexpr int RP = READOUT ? kPairs : 1;
  alignas(16) float phikt[kFB][kLS];  // phi_f(k_j), feature-major
  alignas(16) float vt[kDV][kLS];     // V^T
  alignas(16) float phiq[RQ][kLQ];    // phi_f(s q_i), token-major
  alignas(16) float kr[RQ][kDK];      // block 0: raw k rows (scores)
  alignas(16) float qr[RQ][kDK];      // block 0: raw q rows
  alignas(16) f32x4 a[RP][64];        // block 0: score tiles in MFMA B-operand lane order
  alignas(16) float z[kFB];           // the block's z_{<c}
  float den_part[READOUT ? 4 : 1][RQ];
  float den_intra[RP][16];
};

// Where a workgroup's starting state comes from and where its results go (see the file comment).
struct WideIO {
  float* slots;        // nseg > 1: [heads][nseg][stride] prefixes (readout) or increments (state pass)
  float* state;        // nseg == 1: incoming / final state [heads][stride], or null
  float* part_num;     // [blocks][heads * N][d_v] partial numerators
  float* part_den;     // [blocks][heads * N] partial denominators
  long long stride;
  int nseg;
  int BH;
};

// One token's 16 coordinates from 64 bytes (float32) or 32 bytes (bfloat16) of registers.
template <typename E>
struct Row16;
template <>
struct Row16<float> {
  f32x4 p[4];
  __device__ __forceinline__ void load(const float* src) {
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = *reinterpret_cast<const f32x4*>(src + 4 * u);
  }
  __device__ __forceinline__ void unpack(float (&x)[kDK], float s) const {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * u + r] = s * p[u][r];
  }
};
template <>
struct Row16<__bf16> {
  uint4 p[2];
  __device__ __forceinline__ void load(const __bf16* src) {
    p[0] = *reinterpret_cast<const uint4*>(src);
    p[1] = *reinterpret_cast<const uint4*>(src + 8);
  }
  __device__ __forceinline__ void unpack(float (&x)[kDK], float s) const {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t w[4] = {p[u].x, p[u].y, p[u].z, p[u].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[8 * u + 2 * h] = s * __uint_as_float(w[h] << 16);
        x[8 * u + 2 * h + 1] = s * __uint_as_float(w[h] & 0xffff0000u);
      }
    }
  }
};

// Wave w's 16 value columns of one token (v row slice) from registers.
template <typename E>
struct Vals16 {
  Row16<E> r;
  __device__ __forceinline__ void load(const E* src) { r.load(src); }
  __device__ __forceinline__ void unpack(float (&x)[16]) const { r.unpack(x, 1.0f); }
};

// The chunk inputs one lane holds in flight: k and q rows of token l, and wave w's 16 values of it.
template <typename E, bool READOUT>
struct WideIn {
  Row16<E> k, q;
  Vals16<E> v;
  __device__ __forceinline__ void load(const E* qg, const E* kg, const E* vg, long long tok0, int nv, int l,
                                       int w) {
    const long long row = tok0 + (l < nv ? l : 0);  // tokens past the end read a valid row, masked later
    k.load(kg + row * kDK);
    if constexpr (READOUT) q.load(qg + row * kDK);
    v.load(vg + row * kDV + 16 * w);
  }
};

// Expansion of the block's features of token l: wave sub-block F0 .. F0 + kSub - 1 (global indices).
template <int NT, bool READOUT, int F0>
__device__ __forceinline__ void expand_wave(WideSmem<READOUT>& sm, int w, int l, const float (&xk)[kDK],
                                            const float (&xq)[kDK], bool valid) {
  constexpr int L0 = F0 % kFB;  // row of the first feature inside the block
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((sm.phikt[L0 + I][l] = (F0 + I == 0) ? (valid ? 1.f : 0.f) : feature_ct<NT, kDK, F0 + I>(xk)), ...);
  }(std::make_integer_sequence<int, kSub>{});
  if constexpr (READOUT) {
    float den = 0.f;
    [&]<int... P>(std::integer_sequence<int, P...>) {
      (([&] {
         const f32x4 f = {feature_ct<NT, kDK, F0 + 4 * P>(xq), feature_ct<NT, kDK, F0 + 4 * P + 1>(xq),
                          feature_ct<NT, kDK, F0 + 4 * P + 2>(xq), feature_ct<NT, kDK, F0 + 4 * P + 3>(xq)};
         *reinterpret_cast<f32x4*>(&sm.phiq[l][L0 + 4 * P]) = f;
         const f32x4 zz = *reinterpret_cast<const f32x4*>(&sm.z[L0 + 4 * P]);
         den = fmaf(f[0], zz[0], den);
         den = fmaf(f[1], zz[1], den);
         den = fmaf(f[2], zz[2], den);
         den = fmaf(f[3], zz[3], den);
       }()),
       ...);
    }(std::make_integer_sequence<int, kSub / 4>{});
    sm.den_part[w][l] = den;
  }
}

// One segment of L tokens, one feature block; grid = (segments, heads, blocks).
template <int NT, typename E, bool READOUT>
__global__ __launch_bounds__(kThreads) void prefill_wide_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                                const E* __restrict__ v, WideIO io, int N, int L,
                                                                float scale) {
  constexpr int W = FeatureTable<NT, kDK>::W;
  constexpr int NB = n_blocks<NT>();
  __shared__ WideSmem<READOUT> sm;

  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = 16 * w + l16;  // value column of this lane in the MFMA tiles
  const int seg = blockIdx.x, fb = blockIdx.z;
  const long long bh = blockIdx.y;
  const int f0 = fb * kFB;
  const int t_begin = seg * L, t_end = min(N, t_begin + L);
  const long long hbase = bh * (long long)N;
  const bool intra = READOUT && fb == 0;  // block 0 also carries the intra-chunk term

  // starting state of this block: rows f0 .. f0 + kFB - 1 (zero past W)
  const float* init = nullptr;
  if (io.nseg > 1) {
    if (READOUT) init = io.slots + (bh * io.nseg + seg) * io.stride;
  } else if (READOUT && io.state) {
    init = io.state + bh * io.stride;
  }
  f32x4 Srun[kNAT];
#pragma unroll
  for (int t = 0; t < kNAT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = f0 + 16 * t + 4 * lg + r;
      Srun[t][r] = (init && a < W) ? init[(long long)a * kDV + col] : 0.f;
    }
  if (tid < kFB) sm.z[tid] = (init && f0 + tid < W) ? init[(long long)W * kDV + f0 + tid] : 0.f;

  WideIn<E, READOUT> in;
  in.load(q, k, v, hbase + t_begin, min(kCS, t_end - t_begin), l, w);

  for (int c0 = t_begin; c0 < t_end; c0 += kCS) {
    const int nv = min(kCS, t_end - c0);
    const long long tok0 = hbase + c0;
    const bool valid = l < nv;

    // ---- expansion of this chunk into LDS ----
    __syncthreads();  // previous chunk's MFMAs and z update are done with LDS
    {
      float xk[kDK], xq[kDK];
      in.k.unpack(xk, valid ? 1.0f : 0.0f);  // a token past the end has a zero k row
      if constexpr (READOUT) in.q.unpack(xq, scale);
      dispatch_index<0, NB * 4>(fb * 4 + w, [&](auto I) {
        expand_wave<NT, READOUT, decltype(I)::value * kSub>(sm, w, l, xk, xq, valid);
      });
      float vv[16];
      in.v.unpack(vv);
#pragma unroll
      for (int c = 0; c < 16; ++c) sm.vt[16 * w + c][l] = valid ? vv[c] : 0.f;
      if (intra && w == 0) {
        float xr[kDK];
        in.q.unpack(xr, 1.0f);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          *reinterpret_cast<f32x4*>(&sm.kr[l][4 * u]) = f32x4{xk[4 * u], xk[4 * u + 1], xk[4 * u + 2], xk[4 * u + 3]};
          *reinterpret_cast<f32x4*>(&sm.qr[l][4 * u]) = f32x4{xr[4 * u], xr[4 * u + 1], xr[4 * u + 2], xr[4 * u + 3]};
        }
      }
    }
    __syncthreads();
    if (c0 + kCS < t_end) in.load(q, k, v, tok0 + kCS, min(kCS, t_end - c0 - kCS), l, w);

    // ---- matrix work of wave w (value columns 16w..16w+15) ----
    f32x4 O[READOUT ? kNIT : 1];
    if constexpr (READOUT) {
      if (intra) {
        // score tiles (key tile jt <= query tile it) of this wave's pairs, and their column sums
        for (int p = w; p < kPairs; p += 4) {
          int it = 0;
          while ((it + 1) * (it + 2) / 2 <= p) ++it;
          const int jt = p - it * (it + 1) / 2;
          const f32x4 ak = *reinterpret_cast<const f32x4*>(&sm.kr[16 * jt + l16][4 * lg]);
          const f32x4 bq = *reinterpret_cast<const f32x4*>(&sm.qr[16 * it + l16][4 * lg]);
          f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < 4; ++r) sc = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[r], bq[r], sc, 0, 0, 0);
          // sc[r] = k_j . q_i with j = 16jt + 4lg + r, i = 16it + l16
          f32x4 wt;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * jt + 4 * lg + r, i = 16 * it + l16;
            wt[r] = (jt < it || j <= i) ? taylor_kernel<NT>(scale * sc[r]) : 0.f;
          }
          sm.a[p][l] = wt;
          f32x4 cs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < 4; ++r) cs = __builtin_amdgcn_mfma_f32_16x16x4f32(1.0f, wt[r], cs, 0, 0, 0);
          if (lg == 0) sm.den_intra[p][l16] = cs[0];  // sum over the 16 keys for query 16it + l16
        }
      }
      // readout: O[it][r] = (phi_f(sQ) S_{f,<c})[token 16it + l16][column 16w + 4lg + r]
#pragma unroll
      for (int it = 0; it < kNIT; ++it) O[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kNAT; ++t)
#pragma unroll
        for (int it = 0; it < kNIT; ++it) {
          const f32x4 bq = *reinterpret_cast<const f32x4*>(&sm.phiq[16 * it + l16][16 * t + 4 * lg]);
#pragma unroll
          for (int r = 0; r < 4; ++r) O[it] = __builtin_amdgcn_mfma_f32_16x16x4f32(Srun[t][r], bq[r], O[it], 0, 0, 0);
        }
    }
    // state update: Srun[t] += phi_f(K)^T[16t.., chunk] V[chunk, columns]
#pragma unroll
    for (int jb = 0; jb < kCS / 16; ++jb) {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(&sm.vt[col][16 * jb + 4 * lg]);
#pragma unroll
      for (int t = 0; t < kNAT; ++t) {
        const f32x4 ak = *reinterpret_cast<const f32x4*>(&sm.phikt[16 * t + l16][16 * jb + 4 * lg]);
#pragma unroll
        for (int r = 0; r < 4; ++r) Srun[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[r], bv[r], Srun[t], 0, 0, 0);
      }
    }
    // z_{<c+1} = z_{<c} + row sums of phi_f(K)^T (tokens past the end are zero rows)
    if (tid < kFB) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kCS; j += 4) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sm.phikt[tid][j]);
        acc += (x4[0] + x4[1]) + (x4[2] + x4[3]);
      }
      sm.z[tid] += acc;
    }
    if constexpr (READOUT) {
      if (intra) {
        __syncthreads();  // every wave's score tiles and their sums are visible
#pragma unroll
        for (int it = 0; it < kNIT; ++it)
          for (int jt = 0; jt <= it; ++jt) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.vt[col][16 * jt + 4 * lg]);
            const f32x4 bw = sm.a[it * (it + 1) / 2 + jt][l];
#pragma unroll
            for (int r = 0; r < 4; ++r) O[it] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r], bw[r], O[it], 0, 0, 0);
          }
      }
      // partial numerators of this block (columns 16w + 4lg .. + 3 of token 16it + l16)
      float* pn = io.part_num + ((long long)fb * io.BH * N + tok0) * kDV;
#pragma unroll
      for (int it = 0; it < kNIT; ++it) {
        const int i = 16 * it + l16;
        if (i < nv) *reinterpret_cast<f32x4*>(pn + (long long)i * kDV + 16 * w + 4 * lg) = O[it];
      }
      // partial denominators: wave w writes tokens 16w .. 16w + 15
      if (lg == 0) {
        const int i = 16 * w + l16;
        float d = ((sm.den_part[0][i] + sm.den_part[1][i]) + sm.den_part[2][i]) + sm.den_part[3][i];
        if (intra)
          for (int jt = 0; jt <= w; ++jt) d += sm.den_intra[w * (w + 1) / 2 + jt][l16];
        if (i < nv) io.part_den[(long long)fb * io.BH * N + tok0 + i] = d;
      }
    }
  }

  // state pass: the segment's increment; single-segment readout: the final state
  float* dst = nullptr;
  if (!READOUT)
    dst = io.slots + (bh * io.nseg + seg) * io.stride;
  else if (io.nseg == 1 && io.state)
    dst = io.state + bh * io.stride;
  if (dst) {
#pragma unroll
    for (int t = 0; t < kNAT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = f0 + 16 * t + 4 * lg + r;
        if (a < W) dst[(long long)a * kDV + col] = Srun[t][r];
      }
    __syncthreads();  // the last chunk's z update is complete
    if (tid < kFB && f0 + tid < W) dst[(long long)W * kDV + f0 + tid] = sm.z[tid];
  }
}

// o[token][c] = sum_blocks num / sum_blocks den, blocks in order; 16 threads per token.
__global__ __launch_bounds__(256) void wide_reduce_kernel(const float* __restrict__ num,
                                                          const float* __restrict__ den, float* __restrict__ o,
                                                          long long tokens, int nb) {
  const long long e = blockIdx.x * 256ll + threadIdx.x;
  const long long tok = e >> 4;
  const int g = (int)(e & 15);
  if (tok >= tokens) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float d = 0.f;
  for (int b = 0; b < nb; ++b) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(num + ((long long)b * tokens + tok) * kDV + 4 * g);
    acc = acc + x;
    d += den[(long long)b * tokens + tok];
  }
  *reinterpret_cast<f32x4*>(o + tok * kDV + 4 * g) = f32x4{acc[0] / d, acc[1] / d, acc[2] / d, acc[3] / d};
}

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Segments per head: enough (segment, head, block) workgroups to cover the chip once.
int wide_segments(int BH, int nb, int nchunk, bool outputs) {
  const long long target = outputs ? 256 : 1024;
  long long want = (target + (long long)BH * nb - 1) / ((long long)BH * nb);
  if (want < 1) want = 1;
  if (want > nchunk) want = nchunk;
  return (int)want;
}

struct WideLayout {
  int nseg, L;
  long long slot_floats, part_floats;
};

template <int NT>
WideLayout wide_layout(const Shape& s, int BH, int N, bool outputs) {
  constexpr int NB = n_blocks<NT>();
  const int nchunk = cdiv(N, kCS);
  WideLayout lay;
  lay.L = cdiv(nchunk, wide_segments(BH, NB, nchunk, outputs)) * kCS;
  lay.nseg = cdiv(N, lay.L);
  // slots are needed for several segments, and always for a state-only call (the scan sums them)
  lay.slot_floats = (lay.nseg > 1 || !outputs) ? (long long)BH * lay.nseg * s.stride : 0;
  lay.part_floats = outputs ? (long long)NB * BH * N * (kDV + 1) : 0;
  return lay;
}

long long round_up(long long x, long long m) { return (x + m - 1) / m * m; }

template <int NT, typename E>
int wide_run(const PrefillArgs& a) {
  constexpr int NB = n_blocks<NT>();
  const bool outputs = a.o != nullptr;
  const WideLayout lay = wide_layout<NT>(a.s, a.BH, a.N, outputs);
  float* ws = (float*)a.ws;
  float* slots = ws;
  float* part_num = ws + round_up(lay.slot_floats, 64);
  float* part_den = part_num + (long long)NB * a.BH * a.N * kDV;
  const E* q = (const E*)a.q;
  const E* k = (const E*)a.k;
  const E* v = (const E*)a.v;
  const long long elems = FeatureTable<NT, kDK>::W * (long long)(kDV + 1);
  const dim3 grid(lay.nseg, a.BH, NB), block(kThreads);
  if (!outputs || lay.nseg > 1) {
    const WideIO io{slots, nullptr, nullptr, nullptr, a.s.stride, lay.nseg, a.BH};
    prefill_wide_kernel<NT, E, false><<<grid, block, 0, a.stream>>>(q, k, v, io, a.N, lay.L, a.s.scale);
    if (hipGetLastError() != hipSuccess) return -3;
    if (seg_scan_launch(slots, a.state, a.BH, lay.nseg, a.s.stride, elems, outputs, a.stream)) return -3;
    if (!outputs) return 0;
  }
  const WideIO io{slots, lay.nseg == 1 ? a.state : nullptr, part_num, part_den, a.s.stride, lay.nseg, a.BH};
  prefill_wide_kernel<NT, E, true><<<grid, block, 0, a.stream>>>(q, k, v, io, a.N, lay.L, a.s.scale);
  if (hipGetLastError() != hipSuccess) return -3;
  const long long tokens = (long long)a.BH * a.N;
  wide_reduce_kernel<<<dim3((unsigned)cdiv(tokens * 16, 256)), dim3(256), 0, a.stream>>>(part_num, part_den, a.o,
                                                                                          tokens, NB);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

bool prefill_wide_has(int nt, int dk, int dv) { return dk == kDK && dv == kDV && (nt == 4 || nt == 5); }

// An upper bound over both uses (with and without outputs): the query does not know which follows.
long long prefill_wide_ws_bytes(const Shape& s, int BH, int N) {
  auto bytes = [](const WideLayout& lay) { return (round_up(lay.slot_floats, 64) + lay.part_floats) * 4; };
  if (s.nt == 4) return std::max(bytes(wide_layout<4>(s, BH, N, true)), bytes(wide_layout<4>(s, BH, N, false)));
  return std::max(bytes(wide_layout<5>(s, BH, N, true)), bytes(wide_layout<5>(s, BH, N, false)));
}

int prefill_wide_launch(const PrefillArgs& a) {
  if (!prefill_wide_has(a.s.nt, a.s.dk, a.s.dv)) return -2;
  if (a.s.nt == 4) return a.s.dtype == 0 ? wide_run<4, float>(a) : wide_run<4, __bf16>(a);
  return a.s.dtype == 0 ? wide_run<5, float>(a) : wide_run<5, __bf16>(a);
}

}  // namespace taylor
