// Decode step and state initialisation (gfx950).
//
// "Expanding Attention" (Huang, arXiv:2610.20637), Abstract: each of the n
// recurrent states is updated by one rank-one outer product per token, at a
// cost independent of the context length.  Per (b, h) one decode step is
//     S += phi(k_t) v_t^T,  z += phi(k_t)          (rank-one update)
//     o_t = (phi(s*q_t)^T S) / (phi(s*q_t)^T z)     (readout)
// which streams the W x (d_v+1) float32 state once: every element is read,
// updated and written back, and the readout is folded into the same pass, so
// the step moves 2 * 4 * W * (d_v+1) bytes per head and is bound by HBM.
//
// Layout per head block: S [W][d_v] row-major, then z [W], padded to a
// multiple of 4 floats.  A workgroup owns one head.  Thread t handles the
// float4 column group t % (d_v/4) of rows t / (d_v/4), t / (d_v/4) + 256/(d_v/4),
// ...: a wavefront reads 64 consecutive float4s (1 KiB) per row batch, fully
// coalesced, and each thread keeps a fixed 4-column slice of the readout
// numerator, reduced at the end with cross-lane shuffles and one LDS pass.
// All row loads of a batch are issued before any update, so every thread has
// up to 12 x 16 B in flight; the first batch is requested before the features
// are formed.
#include "common.hpp"
#include "launch.hpp"

namespace taylor {
namespace {

constexpr int kDecodeThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// A state row piece, read with the nontemporal hint: each element is read once per step, and the
// hint measured 2% faster with the state in the last-level cache (64 x 16 heads, 41 MB) and 9%
// faster above it (512 x 16 heads, 326 MB) than plain loads.  (Nontemporal stores as well, or
// instead, were slower at one size or the other.)
__device__ __forceinline__ float4 load_stream(const float* p) {
  const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(x[0], x[1], x[2], x[3]);
}

// Order of feature a in the table (orders ascend: 1 feature of order 0, then d_k of order 1, ...);
// used at n <= 3 only.
template <int DK>
__device__ __forceinline__ int order_of(int a) {
  return a == 0 ? 0 : a <= DK ? 1 : 2;
}

// CENT: the softmax expanded about the mean score (Su Jianlin, kexue.fm translation 11814, "Linear
// Attention"), order n - 1: with d_m = phi_m(a) . z_m over the inclusive history (a = sigma q),
// c = d_0 and u = d_1 / c, the output is sum_m gamma_m phi_m(a)^T S_m with
//     order 1: gamma = ((1 - u) / c, 1 / c)
//     order 2: gamma = ((1 - u + u^2 - d_2 / c) / c, (1 - u) / c, 1 / c)
// and no normaliser (the weights sum to one).  The d_m are reduced first, phi(a) is scaled by the
// gammas, and the state pass below runs unchanged.
template <int NT, int DK, int DV, typename T, bool CENT>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                const T* __restrict__ v, float* __restrict__ o,
                                                                float* __restrict__ state, long long stride,
                                                                float scale) {
  constexpr int W = Monomials<NT, DK>::W;
  constexpr int CG = DV / 4;  // float4 column groups per S row
  static_assert(DV % 4 == 0 && CG <= 64 && (CG & (CG - 1)) == 0, "d_v/4 must be a power of two <= 64");
  constexpr int RSTEP = kDecodeThreads / CG;  // rows covered by the workgroup per row slot
  constexpr int ROWS = (W + RSTEP - 1) / RSTEP;
  constexpr int RB = ROWS < 12 ? ROWS : 12;  // rows held in registers per batch
  constexpr int NWAVE = kDecodeThreads / 64;

  __shared__ float s_q[DK], s_k[DK];
  __shared__ __align__(16) float s_v[DV];
  __shared__ float s_phik[W], s_phiq[W];
  __shared__ float4 s_red[NWAVE][CG];
  __shared__ float s_redz[NWAVE];
  __shared__ float s_redm[NWAVE][3];

  const int tid = threadIdx.x;
  const long long h = blockIdx.x;
  float* S = state + h * stride;
  float* z = S + (long long)W * DV;
  const int cg = tid % CG;
  const int r0 = tid / CG;

  // The first batch of state rows (and z) is requested before anything else, so the state
  // stream is already in flight while q, k, v arrive and the features are formed.
  float4 buf[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    const int r = r0 + u * RSTEP;
    if (r < W) buf[u] = load_stream(S + (long long)r * DV + cg * 4);
  }
  const float z0 = tid < W ? z[tid] : 0.f;

  if (tid < DK) {
    s_q[tid] = scale * to_f32(q[h * DK + tid]);
    s_k[tid] = to_f32(k[h * DK + tid]);
  }
  if (tid < DV) s_v[tid] = to_f32(v[h * DV + tid]);
  __syncthreads();
  for (int a = tid; a < W; a += kDecodeThreads) {
    s_phiq[a] = feature_at<NT, DK>(s_q, a);
    s_phik[a] = feature_at<NT, DK>(s_k, a);
  }
  __syncthreads();
  if constexpr (CENT) {
    static_assert(NT == 2 || NT == 3, "orders 1 and 2");
    static_assert(W <= kDecodeThreads, "one feature per thread");
    float dm[3] = {0.f, 0.f, 0.f};
    const int m = order_of<DK>(tid);
    if (tid < W) dm[m] = s_phiq[tid] * (z0 + s_phik[tid]);
#pragma unroll
    for (int j = 0; j < 3; ++j)
      for (int off = 1; off < 64; off <<= 1) dm[j] += __shfl_xor(dm[j], off);
    if ((tid & 63) == 0)
#pragma unroll
      for (int j = 0; j < 3; ++j) s_redm[tid >> 6][j] = dm[j];
    __syncthreads();
    float d[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWAVE; ++w)
#pragma unroll
      for (int j = 0; j < 3; ++j) d[j] += s_redm[w][j];
    const float ic = 1.0f / d[0], u = d[1] * ic;
    const float g[3] = {NT == 2 ? (1.0f - u) * ic : (1.0f - u + u * u - d[2] * ic) * ic,
                        NT == 2 ? ic : (1.0f - u) * ic, ic};
    if (tid < W) s_phiq[tid] *= g[m];
    __syncthreads();
  }

  const float4 vv = *reinterpret_cast<const float4*>(s_v + cg * 4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int base = r0; base < W; base += RSTEP * RB) {
    if (base != r0) {
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int r = base + u * RSTEP;
        if (r < W) buf[u] = load_stream(S + (long long)r * DV + cg * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int r = base + u * RSTEP;
      if (r < W) {
        const float4 nv = fma4(s_phik[r], vv, buf[u]);
        acc = fma4(s_phiq[r], nv, acc);
        *reinterpret_cast<float4*>(S + (long long)r * DV + cg * 4) = nv;
      }
    }
  }
  float accz = 0.f;
  if (tid < W) {
    const float nz = z0 + s_phik[tid];
    z[tid] = nz;
    accz = s_phiq[tid] * nz;
  }
  for (int a = tid + kDecodeThreads; a < W; a += kDecodeThreads) {
    const float nz = z[a] + s_phik[a];
    z[a] = nz;
    accz = fmaf(s_phiq[a], nz, accz);
  }

  for (int off = CG; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  for (int off = 1; off < 64; off <<= 1) accz += __shfl_xor(accz, off);
  const int lane = tid & 63, wave = tid >> 6;
  if (lane < CG) s_red[wave][lane] = acc;
  if (lane == 0) s_redz[wave] = accz;
  __syncthreads();
  if (tid < CG) {
    float4 t = s_red[0][tid];
    float den = s_redz[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) {
      t = add4(t, s_red[w][tid]);
      den += s_redz[w];
    }
    if constexpr (CENT)
      *reinterpret_cast<float4*>(o + h * DV + tid * 4) = t;
    else
      *reinterpret_cast<float4*>(o + h * DV + tid * 4) = make_float4(t.x / den, t.y / den, t.z / den, t.w / den);
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ p, long long n4) {
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += (long long)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(256) void copy_kernel(float4* __restrict__ d, const float4* __restrict__ s, long long n4) {
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) d[i] = s[i];
}

template <int NT, int DK, int DV, bool CENT>
int decode_go(const DecodeArgs& a) {
  const dim3 grid(a.BH), block(kDecodeThreads);
  if (a.s.dtype == 0)
    decode_kernel<NT, DK, DV, float, CENT><<<grid, block, 0, a.stream>>>(
        (const float*)a.q, (const float*)a.k, (const float*)a.v, a.o, a.state, a.s.stride, a.s.scale);
  else
    decode_kernel<NT, DK, DV, uint16_t, CENT><<<grid, block, 0, a.stream>>>(
        (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.o, a.state, a.s.stride, a.s.scale);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// The expanded-softmax readout is compiled for n = 2, 3 at d_k = 16, d_v = 64.
template <int NT, int DK, int DV>
constexpr bool has_centered() {
  return (NT == 2 || NT == 3) && DK == 16 && DV == 64;
}

template <int NT, int DK, int DV>
int decode_run(const DecodeArgs& a) {
  if (a.s.readout == 1) {
    if constexpr (has_centered<NT, DK, DV>())
      return decode_go<NT, DK, DV, true>(a);
    else
      return -2;
  }
  return decode_go<NT, DK, DV, false>(a);
}

using DecodeFn = int (*)(const DecodeArgs&);

template <int DK, int DV>
DecodeFn decode_pick(int nt) {
  switch (nt) {
    case 1: return decode_run<1, DK, DV>;
    case 2: return decode_run<2, DK, DV>;
    case 3: return decode_run<3, DK, DV>;
    case 4: return decode_run<4, DK, DV>;
    case 5: return decode_run<5, DK, DV>;
  }
  return nullptr;
}

DecodeFn decode_find(int nt, int dk, int dv) {
  if (dk == 4 && dv == 4) return decode_pick<4, 4>(nt);
  if (dk == 8 && dv == 32) return decode_pick<8, 32>(nt);
  if (dk == 16 && dv == 64) return decode_pick<16, 64>(nt);
  if (dk == 16 && dv == 128) return decode_pick<16, 128>(nt);
  return nullptr;
}

}  // namespace

bool decode_has(int nt, int dk, int dv) { return decode_find(nt, dk, dv) != nullptr; }

int decode_launch(const DecodeArgs& a) {
  DecodeFn f = decode_find(a.s.nt, a.s.dk, a.s.dv);
  return f ? f(a) : -2;
}

int state_copy_launch(float* dst, const float* src, long long count, hipStream_t stream) {
  const long long n4 = count / 4;
  long long blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  copy_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(reinterpret_cast<float4*>(dst),
                                                                 reinterpret_cast<const float4*>(src), n4);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int state_zero_launch(float* state, long long count, hipStream_t stream) {
  const long long n4 = count / 4;
  long long blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(reinterpret_cast<float4*>(state), n4);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace taylor
