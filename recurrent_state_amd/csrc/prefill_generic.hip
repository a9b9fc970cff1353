// Portable chunked prefill (gfx950, float32 vector ALU): any compiled (n, d_k, d_v).
//
// "Expanding Attention" (Huang, arXiv:2610.20637), Abstract: the states are
// additive across chunks, so prefill is chunk-local work plus a parallel scan.
// For a chunk c of C tokens starting at token c*C,
//     out_i = phi(s*q_i)^T S_{<c}  +  sum_{c*C <= j <= i} K_n(s q_i.k_j) [v_j | 1]
//     o_i   = out_i[:d_v] / out_i[d_v]
// where S_{<c} = S_init + sum_{c' < c} dS_{c'} and dS_c = sum_{j in c} phi(k_j) [v_j | 1]^T.
//
// Three launches:
//   1. seg_state  -- dS for segments of L tokens (L = C when outputs are wanted,
//                    larger for a state-only pass), one feature block per workgroup;
//   2. seg_scan   -- exclusive prefix over segments (+ the incoming state), the
//                    total written back to the state;
//   3. readout    -- per chunk: the inter-chunk term from the prefix plus the
//                    quadratic intra-chunk term, then the division.
// This path keeps every intermediate in float32 and favours clarity; the
// d_k = 16, d_v = 64 shapes also have an MFMA path.
#include "common.hpp"
#include "launch.hpp"

namespace taylor {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 64;  // token sub-block held in LDS
constexpr int kFB = 32;  // feature block
constexpr int kJB = 32;  // key block of the intra-chunk score tile

template <int W>
constexpr int n_feature_blocks() { return (W + kFB - 1) / kFB; }

// dS for one segment of tokens and one block of kFB features.
// grid = (segments, heads, feature blocks).  Output rows fb*kFB.. of the
// segment's slot in the workspace: S rows [W][DV] then z [W].
template <int NT, int DK, int DV, typename T>
__global__ __launch_bounds__(kThreads) void seg_state_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                             float* __restrict__ ws, int N, int L, int nseg,
                                                             long long stride) {
  constexpr int W = Monomials<NT, DK>::W;
  constexpr int CG = DV / 4;
  constexpr int P4 = (kFB * CG + kThreads - 1) / kThreads;
  __shared__ float s_k[kTB][DK];
  __shared__ __align__(16) float s_v[kTB][DV];
  __shared__ float s_phi[kTB][kFB + 1];

  const int tid = threadIdx.x;
  const int seg = blockIdx.x;
  const long long bh = blockIdx.y;
  const int fb0 = blockIdx.z * kFB;
  const int t0 = seg * L;
  const int t1 = min(N, t0 + L);
  const T* kb = k + bh * (long long)N * DK;
  const T* vb = v + bh * (long long)N * DV;

  float4 acc[P4];
#pragma unroll
  for (int u = 0; u < P4; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  float accz = 0.f;

  for (int j0 = t0; j0 < t1; j0 += kTB) {
    const int nj = min(kTB, t1 - j0);
    __syncthreads();
    for (int e = tid; e < kTB * DK; e += kThreads) {
      const int j = e / DK, c = e % DK;
      s_k[j][c] = j < nj ? to_f32(kb[(long long)(j0 + j) * DK + c]) : 0.f;
    }
    for (int e = tid; e < kTB * DV; e += kThreads) {
      const int j = e / DV, c = e % DV;
      s_v[j][c] = j < nj ? to_f32(vb[(long long)(j0 + j) * DV + c]) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < kTB * kFB; e += kThreads) {
      const int j = e / kFB, a = e % kFB;
      s_phi[j][a] = (j < nj && fb0 + a < W) ? feature_at<NT, DK>(s_k[j], fb0 + a) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < P4; ++u) {
      const int p = tid + u * kThreads;
      if (p < kFB * CG) {
        const int a = p / CG, cg = p % CG;
        for (int j = 0; j < nj; ++j)
          acc[u] = fma4(s_phi[j][a], *reinterpret_cast<const float4*>(&s_v[j][cg * 4]), acc[u]);
      }
    }
    if (tid < kFB)
      for (int j = 0; j < nj; ++j) accz += s_phi[j][tid];
  }

  float* out = ws + (bh * nseg + seg) * stride;
#pragma unroll
  for (int u = 0; u < P4; ++u) {
    const int p = tid + u * kThreads;
    if (p < kFB * CG) {
      const int a = p / CG, cg = p % CG;
      if (fb0 + a < W) *reinterpret_cast<float4*>(out + (long long)(fb0 + a) * DV + cg * 4) = acc[u];
    }
  }
  if (tid < kFB && fb0 + tid < W) out[(long long)W * DV + fb0 + tid] = accz;
}

// Exclusive prefix over the segments of each (sequence, head) pair, seeded with the incoming state
// (`seed`, null: zero); the total goes to `total` (null: discarded; may be `seed`).
// grid = (ceil(elems/256), pairs).
__global__ __launch_bounds__(kThreads) void seg_scan_kernel(float* __restrict__ ws, const float* seed, float* total,
                                                            long long nslot, long long stride, long long elems,
                                                            int write_prefix, SeqMap seq, int L) {
  const long long e = blockIdx.x * (long long)kThreads + threadIdx.x;
  const long long bh = blockIdx.y;
  if (e >= elems) {
    // the padding after S and z of the final state: zero, whatever the array held before
    if (total && e < stride) total[bh * stride + e] = 0.f;
    return;
  }
  long long first;
  int n;
  seq.pair_slots(bh, nslot, L, first, n);
  float run = seed ? seed[bh * stride + e] : 0.f;
  float* w = ws + first * stride + e;
  // eight slots at a time: their loads are all in flight before the first add (the walk over a pair's
  // slots is otherwise one memory round trip per slot); the sums stay in slot order
  constexpr int kBatch = 8;
  int s = 0;
  for (; s + kBatch <= n; s += kBatch) {
    float t[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) t[u] = w[(s + u) * stride];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (write_prefix) w[(s + u) * stride] = run;
      run += t[u];
    }
  }
  for (; s < n; ++s) {
    const float t = w[s * stride];
    if (write_prefix) w[s * stride] = run;
    run += t;
  }
  if (total) total[bh * stride + e] = run;
}

// Outputs of one chunk.  grid = (chunks, heads).  The chunk's exclusive prefix
// state sits in its workspace slot.  Thread pair p = (token i, column group cg)
// accumulates a float4 numerator slice and its own copy of the denominator.
template <int NT, int DK, int DV, int C, typename T>
__global__ __launch_bounds__(kThreads) void readout_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const float* __restrict__ ws,
                                                           float* __restrict__ o, int N, int nchunk,
                                                           long long stride, float scale) {
  constexpr int W = Monomials<NT, DK>::W;
  constexpr int CG = DV / 4;
  constexpr int PP = (C * CG + kThreads - 1) / kThreads;
  __shared__ float s_q[C][DK];
  __shared__ float s_k[C][DK];
  __shared__ __align__(16) float s_v[C][DV];
  __shared__ float s_phiq[C][kFB + 1];
  __shared__ __align__(16) float s_S[kFB][DV];
  __shared__ float s_z[kFB];
  __shared__ float s_A[C][kJB + 1];

  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const long long bh = blockIdx.y;
  const int i0 = c * C;
  const int nc = min(C, N - i0);
  const long long tok0 = bh * (long long)N + i0;

  for (int e = tid; e < C * DK; e += kThreads) {
    const int i = e / DK, d = e % DK;
    const bool ok = i < nc;
    s_q[i][d] = ok ? scale * to_f32(q[(tok0 + i) * DK + d]) : 0.f;
    s_k[i][d] = ok ? to_f32(k[(tok0 + i) * DK + d]) : 0.f;
  }
  for (int e = tid; e < C * DV; e += kThreads) {
    const int i = e / DV, d = e % DV;
    s_v[i][d] = i < nc ? to_f32(v[(tok0 + i) * DV + d]) : 0.f;
  }

  float4 acc[PP];
  float den[PP];
#pragma unroll
  for (int u = 0; u < PP; ++u) {
    acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    den[u] = 0.f;
  }

  // Inter-chunk term: phi(s*q_i)^T S_{<c}, one feature block at a time.
  const float* pre = ws + (bh * nchunk + c) * stride;
  for (int fb0 = 0; fb0 < W; fb0 += kFB) {
    __syncthreads();
    for (int e = tid; e < kFB * CG; e += kThreads) {
      const int a = e / CG, cg = e % CG;
      *reinterpret_cast<float4*>(&s_S[a][cg * 4]) =
          fb0 + a < W ? *reinterpret_cast<const float4*>(pre + (long long)(fb0 + a) * DV + cg * 4)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < kFB) s_z[tid] = fb0 + tid < W ? pre[(long long)W * DV + fb0 + tid] : 0.f;
    for (int e = tid; e < C * kFB; e += kThreads) {
      const int i = e / kFB, a = e % kFB;
      s_phiq[i][a] = (i < nc && fb0 + a < W) ? feature_at<NT, DK>(s_q[i], fb0 + a) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PP; ++u) {
      const int p = tid + u * kThreads;
      const int i = p / CG, cg = p % CG;
      if (p < C * CG && i < nc) {
        for (int a = 0; a < kFB; ++a) {
          const float f = s_phiq[i][a];
          acc[u] = fma4(f, *reinterpret_cast<const float4*>(&s_S[a][cg * 4]), acc[u]);
          den[u] = fmaf(f, s_z[a], den[u]);
        }
      }
    }
  }

  // Intra-chunk term: the causal truncated kernel over the chunk's own keys.
  for (int jb0 = 0; jb0 < nc; jb0 += kJB) {
    __syncthreads();
    for (int e = tid; e < C * kJB; e += kThreads) {
      const int i = e / kJB, jj = e % kJB;
      const int j = jb0 + jj;
      float w = 0.f;
      if (i < nc && j <= i) {
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < DK; ++d) s = fmaf(s_q[i][d], s_k[j][d], s);
        w = taylor_kernel<NT>(s);
      }
      s_A[i][jj] = w;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PP; ++u) {
      const int p = tid + u * kThreads;
      const int i = p / CG, cg = p % CG;
      if (p < C * CG && i < nc && i >= jb0) {
        const int jend = min(kJB, i - jb0 + 1);
        for (int jj = 0; jj < jend; ++jj) {
          const float w = s_A[i][jj];
          acc[u] = fma4(w, *reinterpret_cast<const float4*>(&s_v[jb0 + jj][cg * 4]), acc[u]);
          den[u] += w;
        }
      }
    }
  }

#pragma unroll
  for (int u = 0; u < PP; ++u) {
    const int p = tid + u * kThreads;
    const int i = p / CG, cg = p % CG;
    if (p < C * CG && i < nc) {
      const float d = den[u];
      *reinterpret_cast<float4*>(o + (tok0 + i) * DV + cg * 4) =
          make_float4(acc[u].x / d, acc[u].y / d, acc[u].z / d, acc[u].w / d);
    }
  }
}

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

int seg_scan_launch(float* ws, const float* seed, float* total, int BH, long long nslot, long long stride,
                    long long elems, bool write_prefix, const SeqMap& seq, int L, hipStream_t stream) {
  seg_scan_kernel<<<dim3(cdiv(total ? stride : elems, kThreads), BH), dim3(kThreads), 0, stream>>>(
      ws, seed, total, nslot, stride, elems, write_prefix ? 1 : 0, seq, L);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

namespace {

// Segments for a state-only pass: enough workgroups to fill the chip, never more than the chunks.
int state_only_segments(int BH, int nfb, int nchunk) {
  long long want = (4096 + (long long)BH * nfb - 1) / ((long long)BH * nfb);
  if (want < 1) want = 1;
  if (want > nchunk) want = nchunk;
  return (int)want;
}

template <int NT, int DK, int DV, typename T>
int generic_run(const PrefillArgs& a) {
  constexpr int W = Monomials<NT, DK>::W;
  constexpr int nfb = n_feature_blocks<W>();
  const int nchunk = cdiv(a.N, a.C);
  const int nseg = a.o ? nchunk : state_only_segments(a.BH, nfb, nchunk);
  const int L = cdiv(nchunk, nseg) * a.C;
  const int nseg_used = cdiv(a.N, L);
  float* ws = (float*)a.ws;
  const long long elems = (long long)W * (DV + 1);

  seg_state_kernel<NT, DK, DV, T><<<dim3(nseg_used, a.BH, nfb), dim3(kThreads), 0, a.stream>>>(
      (const T*)a.k, (const T*)a.v, ws, a.N, L, nseg_used, a.s.stride);
  if (hipGetLastError() != hipSuccess) return -3;
  if (seg_scan_launch(ws, a.state_in, a.state, a.BH, nseg_used, a.s.stride, elems, a.o != nullptr, a.seq, L,
                      a.stream))
    return -3;
  if (a.o) {
    if (a.C == 64)
      readout_kernel<NT, DK, DV, 64, T><<<dim3(nchunk, a.BH), dim3(kThreads), 0, a.stream>>>(
          (const T*)a.q, (const T*)a.k, (const T*)a.v, ws, a.o, a.N, nchunk, a.s.stride, a.s.scale);
    else
      readout_kernel<NT, DK, DV, 128, T><<<dim3(nchunk, a.BH), dim3(kThreads), 0, a.stream>>>(
          (const T*)a.q, (const T*)a.k, (const T*)a.v, ws, a.o, a.N, nchunk, a.s.stride, a.s.scale);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

template <int NT, int DK, int DV>
int generic_dtype(const PrefillArgs& a) {
  return a.s.dtype == 0 ? generic_run<NT, DK, DV, float>(a) : generic_run<NT, DK, DV, uint16_t>(a);
}

using PrefillFn = int (*)(const PrefillArgs&);

template <int DK, int DV>
PrefillFn generic_pick(int nt) {
  switch (nt) {
    case 1: return generic_dtype<1, DK, DV>;
    case 2: return generic_dtype<2, DK, DV>;
    case 3: return generic_dtype<3, DK, DV>;
    case 4: return generic_dtype<4, DK, DV>;
    case 5: return generic_dtype<5, DK, DV>;
  }
  return nullptr;
}

PrefillFn generic_find(int nt, int dk, int dv) {
  if (dk == 4 && dv == 4) return generic_pick<4, 4>(nt);
  if (dk == 8 && dv == 32) return generic_pick<8, 32>(nt);
  if (dk == 16 && dv == 64) return generic_pick<16, 64>(nt);
  return nullptr;
}

}  // namespace

bool prefill_generic_has(int nt, int dk, int dv, int C) {
  return (C == 64 || C == 128) && generic_find(nt, dk, dv) != nullptr;
}

long long prefill_generic_ws_bytes(const Shape& s, int BH, int N, int C) {
  const long long nchunk = (N + C - 1) / C;
  return (long long)BH * nchunk * s.stride * 4;
}

int prefill_generic_launch(const PrefillArgs& a) {
  if (!prefill_generic_has(a.s.nt, a.s.dk, a.s.dv, a.C)) return -2;
  return generic_find(a.s.nt, a.s.dk, a.s.dv)(a);
}

}  // namespace taylor
