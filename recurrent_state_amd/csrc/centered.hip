// Per-token coefficients of the expanded-softmax readout (gfx950).
//
// Su Jianlin, kexue.fm translation 11814, "Calculating the Gradient" and "Linear Attention": softmax
// over the scores x_j = q . k_j, expanded about their mean and truncated after the first or second
// power, is linear attention over moment sums.  For query i with a = sigma q_i and the keys j <= i,
// write c = sum_j 1, d1 = sum_j (a . k_j), d2 = sum_j (a . k_j)^2 / 2 and u = d1 / c.  Expanding the
// centred powers gives weights that are a polynomial in the raw score s_ij = a . k_j,
//     order 1:  p_ij = ((1 - u) + s_ij) / c
//     order 2:  p_ij = ((1 - u + u^2 - d2/c) + (1 - u) s_ij + s_ij^2 / 2) / c,
// so o_i = sum_m gamma_m P_m with P_m = sum_j s_ij^m / m! v_j = phi_m(a)^T S_m (the same states as the
// truncated-kernel method at n = order + 1) and per-token gammas.  c, d1 and d2 are
// phi_m(a) . z_m over the inclusive prefix, m = 0, 1, 2.
//
// This kernel computes (gamma_0, gamma_1, gamma_2, 0) for every token; the readout kernels then scale
// phi_m(a) by gamma_m, weight the intra-chunk pairs by gamma_0 + gamma_1 s + gamma_2 s^2/2 and skip the
// normaliser.  It walks the pieces of the readout's plan, one 64-token chunk per wavefront and no
// dependence between chunks: z before a chunk is the piece's prefix (its slot after the scan) plus
// the z of the piece's earlier tokens, which the state pass wrote per chunk.  Lane = token for the
// inter-chunk dot products (compile-time feature coordinates, z by scalar loads); the intra-chunk
// power sums come from 16x16 score tiles (float32 MFMA, key rows by query columns), reduced over the
// key rows and handed to the token lanes through LDS.
#include <type_traits>
#include <utility>

#include "centered.hpp"
#include "features.hpp"

namespace taylor {
namespace {

constexpr int kDK = 16, kDV = 64;
constexpr int kCH = 64;     // tokens per chunk
constexpr int kWaves = 8;   // one chunk per wavefront at a time
constexpr int kThreads = 64 * kWaves;
constexpr int kLD = kDK + 1;  // LDS row stride of the staged q, k rows

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row `row` of a [*][16] input matrix, widened to float32.
__device__ __forceinline__ void load_row(const float* p, long long row, float (&x)[kDK]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p + row * kDK + 4 * u);
    x[4 * u] = t[0];
    x[4 * u + 1] = t[1];
    x[4 * u + 2] = t[2];
    x[4 * u + 3] = t[3];
  }
}
__device__ __forceinline__ void load_row(const uint16_t* p, long long row, float (&x)[kDK]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint4 t = *reinterpret_cast<const uint4*>(p + row * kDK + 8 * u);
    const uint32_t wd[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      x[8 * u + 2 * h] = __uint_as_float(wd[h] << 16);
      x[8 * u + 2 * h + 1] = __uint_as_float(wd[h] & 0xffff0000u);
    }
  }
}

template <int NT>
__device__ __forceinline__ float4 gammas(float c, float d1, float d2) {
  const float ic = 1.0f / c, u = d1 * ic;
  if constexpr (NT == 2) return make_float4((1.0f - u) * ic, ic, 0.f, 0.f);
  return make_float4((1.0f - u + u * u - d2 * ic) * ic, (1.0f - u) * ic, ic, 0.f);
}

template <int NT, typename E, bool PACKED>
__global__ __launch_bounds__(kThreads) void centered_coef_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                                 const float* __restrict__ slots,
                                                                 const float* __restrict__ state, int multi,
                                                                 const float* __restrict__ zc, SeqMap seq, int L,
                                                                 long long nslot, long long stride, float scale,
                                                                 float4* __restrict__ coef) {
  using FT = FeatureTable<NT, kDK>;
  constexpr int W = FT::W;
  __shared__ float ks[kWaves][kCH][kLD], as[kWaves][kCH][kLD];
  __shared__ float intra[kWaves][3][kCH];
  __shared__ __align__(16) float zs[kWaves][(W + 3) / 4 * 4];

  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long bx = blockIdx.x, by = blockIdx.y;

  for_each_piece<PACKED>(seq, bx, by, L, nslot, [&](const SeqPiece& pc) __attribute__((always_inline)) {
    const float* pre = multi ? slots + pc.slot * stride : (state ? state + pc.pair * stride : nullptr);
    const long long ci0 = seq.chunk_index(pc, 0, kCH);
    const int nch = (pc.n + kCH - 1) / kCH;
    for (int c = w; c < nch; c += kWaves) {
      const int nv = min(kCH, pc.n - c * kCH);
      const long long tok0 = pc.tok + (long long)c * kCH;
      const float* zrow = zc + (ci0 + c) * W;
      float a[kDK], x[kDK];
      const long long row = tok0 + (l < nv ? l : 0);
      load_row(q, row, a);
      load_row(k, row, x);
#pragma unroll
      for (int d = 0; d < kDK; ++d) {
        a[d] = l < nv ? scale * a[d] : 0.f;
        as[w][l][d] = a[d];
        ks[w][l][d] = l < nv ? x[d] : 0.f;
      }
      // z before the chunk = the piece's prefix + z of the piece's earlier tokens, staged in LDS
      for (int f = l; f < W; f += 64) zs[w][f] = (pre ? pre[(long long)W * kDV + f] : 0.f) + zrow[f];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // inter-chunk: phi_f(a) z_f, summed by order
      float p[3] = {0.f, 0.f, 0.f};
      [&]<int... F>(std::integer_sequence<int, F...>) {
        (([&] {
           constexpr int m = FT::T.order[F];
           p[m] = fmaf(feature_ct<NT, kDK, F>(a), zs[w][F], p[m]);
         }()),
         ...);
      }(std::make_integer_sequence<int, W>{});
      // intra-chunk: score tiles (key rows 16jt + 4lg + r, query column 16it + l16), keys j <= i
#pragma unroll
      for (int it = 0; it < kCH / 16; ++it) {
        float t0 = 0.f, t1 = 0.f, t2 = 0.f;
#pragma unroll
        for (int jt = 0; jt <= it; ++jt) {
          f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            sc = __builtin_amdgcn_mfma_f32_16x16x4f32(ks[w][16 * jt + l16][4 * s4 + lg], as[w][16 * it + l16][4 * s4 + lg],
                                                      sc, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * jt + 4 * lg + r, i = 16 * it + l16;
            if (j <= i && j < nv) {
              t0 += 1.0f;
              t1 += sc[r];
              t2 = fmaf(0.5f * sc[r], sc[r], t2);
            }
          }
        }
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
          t0 += __shfl_xor(t0, off);
          t1 += __shfl_xor(t1, off);
          t2 += __shfl_xor(t2, off);
        }
        if (lg == 0) {
          intra[w][0][16 * it + l16] = t0;
          intra[w][1][16 * it + l16] = t1;
          intra[w][2][16 * it + l16] = t2;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (l < nv)
        coef[tok0 + l] = gammas<NT>(p[0] + intra[w][0][l], p[1] + intra[w][1][l], p[2] + intra[w][2][l]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  });
}

template <int NT, typename E>
int coef_run(const PrefillArgs& a, const CenteredPlan& p) {
  const dim3 grid((unsigned)a.seq.grid_x(p.L), (unsigned)a.seq.grid_y(a.BH)), block(kThreads);
  auto kern = a.seq.packed ? centered_coef_kernel<NT, E, true> : centered_coef_kernel<NT, E, false>;
  kern<<<grid, block, 0, a.stream>>>((const E*)a.q, (const E*)a.k, p.slots, a.state_in, p.multi ? 1 : 0, p.zc, a.seq,
                                     p.L, p.nslot, a.s.stride, a.s.scale, p.coef);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

int centered_coef_launch(const PrefillArgs& a, const CenteredPlan& p) {
  if (a.s.dk != kDK || a.s.dv != kDV || p.CH != kCH || p.L % kCH) return -2;
  if (a.s.nt == 2) return a.s.dtype == 0 ? coef_run<2, float>(a, p) : coef_run<2, uint16_t>(a, p);
  if (a.s.nt == 3) return a.s.dtype == 0 ? coef_run<3, float>(a, p) : coef_run<3, uint16_t>(a, p);
  return -2;
}

}  // namespace taylor
