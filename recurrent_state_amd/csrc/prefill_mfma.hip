// MFMA chunked prefill for d_k = 16, d_v = 64, n = 1..3 (gfx950 matrix cores).
//
// "Expanding Attention" (Huang, arXiv:2610.20637), Abstract: with the kernel
// exp(s) truncated to n Taylor terms and each term factorised into symmetric
// tensor-power features, the causal history is n additive states, so prefill
// is chunk-local work plus a scan of chunk states.  Per chunk c of C tokens:
//     O_c   = phi(s Q_c) S_{<c}  +  tril(K_n(s Q_c K_c^T)) V_c      (numerators)
//     den_c = phi(s Q_c) z_{<c}  +  rowsum(tril(K_n(s Q_c K_c^T)))
//     S    += phi(K_c)^T V_c,   z += phi(K_c)^T 1
//
// Work split (one workgroup = 4 wavefronts walks a segment of consecutive chunks):
//   * The running state S_{<c} (W_p x 64 floats, W_p = W rounded up to 32) lives
//     in MFMA accumulator registers for the whole segment.  Wave w owns value
//     columns 16w..16w+15, so neither the state update nor the readout needs a
//     cross-wave reduction.
//   * Readout phi(sQ) S: the accumulator tile layout (4 consecutive feature rows
//     per lane) is used directly as the MFMA A operand.  The k-slot order this
//     implies is absorbed by storing phi(sQ) in LDS with the same permutation of
//     features inside each 32-block, so S never round-trips through LDS.  For
//     bfloat16 inputs S is split as S = hi + lo (two bfloat16 MFMAs) so that the
//     state keeps float32 accuracy in the readout.
//   * Intra-chunk scores s Q K^T use the 16x16x16 MFMA with the key block as rows;
//     its accumulator layout is exactly the B-operand layout of the next MFMA
//     (V^T times scores), so scores go through registers -> LDS once and are
//     shared by the 4 waves.  Horner's rule for K_n and the causal mask are
//     applied in registers.
//   * The normaliser z and the inter-chunk denominator are float32 vector work
//     (z is a column sum of phi(K), the denominator a dot product per token).
//
// Two launches of this kernel bracket the scan: a state-only pass writes each
// segment's dS to the workspace, the scan turns those into exclusive prefixes,
// and the readout pass starts each segment from its prefix.
//
// bfloat16 inputs: q, k, v, phi and the scores enter the MFMAs as bfloat16;
// S, z, all accumulation and the outputs are float32.  float32 inputs: every
// MFMA is the float32 16x16x4 one.
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "prefill_mfma.hpp"

namespace taylor {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDK = 16, kDV = 64, kThreads = 256;

template <int NT>
struct Geo {
  static constexpr Monomials<NT, kDK> T{};
  static constexpr int W = Monomials<NT, kDK>::W;
  static constexpr int WP = (W + 31) / 32 * 32;  // features padded to 32-wide MFMA k-blocks
  static constexpr int NAT = WP / 16;            // 16-row feature tiles of the state
  static constexpr int NKB = WP / 32;            // 32-wide feature k-blocks
};

// Feature A of x (float32 registers), coordinates and coefficient fixed at compile time.
template <int NT, int A>
__device__ __forceinline__ float feat(const float (&x)[kDK]) {
  if constexpr (A >= Geo<NT>::W) {
    return 0.f;
  } else {
    constexpr int c0 = Geo<NT>::T.coord[A][0];
    constexpr int c1 = Geo<NT>::T.coord[A][1];
    constexpr int c2 = Geo<NT>::T.coord[A][2];
    constexpr int c3 = Geo<NT>::T.coord[A][3];
    constexpr float cf = coef_of_afact(Geo<NT>::T.afact[A]);
    float f = cf;
    if constexpr (c0 >= 0) f *= x[c0];
    if constexpr (c1 >= 0) f *= x[c1];
    if constexpr (c2 >= 0) f *= x[c2];
    if constexpr (c3 >= 0) f *= x[c3];
    return f;
  }
}

// bfloat16 path: position s of a phi(sQ) row holds feature slot_feature(s), the k-slot order of the
// accumulator-fed A operand (lane group g holds features 4g..4g+3 and 16+4g..16+4g+3 of each 32-block).
__host__ __device__ constexpr int slot_feature_bf16(int s) {
  const int kb = s / 32, r32 = s % 32, g = r32 / 8, r = r32 % 8;
  return 32 * kb + (r < 4 ? g * 4 + r : 16 + g * 4 + (r - 4));
}
template <bool BF16>
__host__ __device__ constexpr int slot_feature(int s) {
  return BF16 ? slot_feature_bf16(s) : s;
}

template <int NT, int CS, bool BF16>
struct Smem {
  using E = typename std::conditional<BF16, __bf16, float>::type;
  static constexpr int WP = Geo<NT>::WP;
  static constexpr int PADE = BF16 ? 8 : 4;  // row padding (elements) against LDS bank conflicts
  static constexpr int LQ = WP + PADE;       // phi(sQ) row stride
  static constexpr int LK = CS + PADE;       // phi(K)^T and V^T row stride
  static constexpr int NIT = CS / 16;
  static constexpr int NPAIR = NIT * (NIT + 1) / 2;
  using ATile = typename std::conditional<BF16, bf16x4, f32x4>::type;
  alignas(16) E q[CS][kDK];
  alignas(16) E k[CS][kDK];
  alignas(16) E vt[kDV][LK];
  alignas(16) E phiq[CS][LQ];
  alignas(16) E phikt[WP][LK];
  alignas(16) ATile a[NPAIR][64];  // score tiles in MFMA B-operand lane order
  float den_intra[NPAIR][16];
  float den_part[kThreads / CS][CS];
  float z[2][WP];  // running normaliser, in phi(sQ) slot order, double-buffered per chunk
  float den[CS];
};

__device__ __forceinline__ int pair_index(int jt, int it) { return it * (it + 1) / 2 + jt; }

__device__ __forceinline__ void load_row16(const float* src, float (&x)[kDK], float scale) {
#pragma unroll
  for (int d = 0; d < kDK; ++d) x[d] = scale * src[d];
}
__device__ __forceinline__ void load_row16(const __bf16* src, float (&x)[kDK], float scale) {
#pragma unroll
  for (int d = 0; d < kDK; ++d) x[d] = scale * (float)src[d];
}

// Rows [G*R, G*R + R) of phi(K_c)^T for token j (R = W_p/4; wave G of 4).
template <int NT, int CS, bool BF16, int G>
__device__ __forceinline__ void phik_rows(Smem<NT, CS, BF16>& sm, int j, const float (&x)[kDK], bool valid) {
  using S = Smem<NT, CS, BF16>;
  constexpr int R = Geo<NT>::WP / 4;
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((sm.phikt[G * R + I][j] = (typename S::E)(valid ? feat<NT, G * R + I>(x) : 0.f)), ...);
  }(std::make_integer_sequence<int, R>{});
}

// Slots [G*R, G*R + R) of the phi(sQ) row of token i, in 8-slot groups (16-byte stores for bfloat16).
template <int NT, int CS, bool BF16, int G>
__device__ __forceinline__ void phiq_slots(Smem<NT, CS, BF16>& sm, int i, const float (&x)[kDK]) {
  constexpr int R = Geo<NT>::WP / 4;
  if constexpr (BF16) {
    [&]<int... P>(std::integer_sequence<int, P...>) {
      (([&] {
         constexpr int s0 = G * R + 8 * P;
         bf16x8 v;
         v[0] = (__bf16)feat<NT, slot_feature_bf16(s0 + 0)>(x);
         v[1] = (__bf16)feat<NT, slot_feature_bf16(s0 + 1)>(x);
         v[2] = (__bf16)feat<NT, slot_feature_bf16(s0 + 2)>(x);
         v[3] = (__bf16)feat<NT, slot_feature_bf16(s0 + 3)>(x);
         v[4] = (__bf16)feat<NT, slot_feature_bf16(s0 + 4)>(x);
         v[5] = (__bf16)feat<NT, slot_feature_bf16(s0 + 5)>(x);
         v[6] = (__bf16)feat<NT, slot_feature_bf16(s0 + 6)>(x);
         v[7] = (__bf16)feat<NT, slot_feature_bf16(s0 + 7)>(x);
         *reinterpret_cast<bf16x8*>(&sm.phiq[i][s0]) = v;
       }()),
       ...);
    }(std::make_integer_sequence<int, R / 8>{});
  } else {
    [&]<int... P>(std::integer_sequence<int, P...>) {
      (([&] {
         constexpr int s0 = G * R + 4 * P;
         f32x4 v;
         v[0] = feat<NT, s0 + 0>(x);
         v[1] = feat<NT, s0 + 1>(x);
         v[2] = feat<NT, s0 + 2>(x);
         v[3] = feat<NT, s0 + 3>(x);
         *reinterpret_cast<f32x4*>(&sm.phiq[i][s0]) = v;
       }()),
       ...);
    }(std::make_integer_sequence<int, R / 4>{});
  }
}

template <int NT, int CS, bool BF16>
__device__ __forceinline__ void features(Smem<NT, CS, BF16>& sm, int w, int l, int nv, float scale, bool readout) {
#pragma unroll
  for (int tt = 0; tt < CS / 64; ++tt) {
    const int j = l + 64 * tt;
    float x[kDK];
    load_row16(&sm.k[j][0], x, 1.0f);
    const bool valid = j < nv;
    switch (w) {
      case 0: phik_rows<NT, CS, BF16, 0>(sm, j, x, valid); break;
      case 1: phik_rows<NT, CS, BF16, 1>(sm, j, x, valid); break;
      case 2: phik_rows<NT, CS, BF16, 2>(sm, j, x, valid); break;
      default: phik_rows<NT, CS, BF16, 3>(sm, j, x, valid); break;
    }
    if (readout) {
      load_row16(&sm.q[j][0], x, scale);
      switch (w) {
        case 0: phiq_slots<NT, CS, BF16, 0>(sm, j, x); break;
        case 1: phiq_slots<NT, CS, BF16, 1>(sm, j, x); break;
        case 2: phiq_slots<NT, CS, BF16, 2>(sm, j, x); break;
        default: phiq_slots<NT, CS, BF16, 3>(sm, j, x); break;
      }
    }
  }
}

// One segment of L tokens per workgroup; grid = (segments, heads).
// READOUT = false: accumulate the segment's dS, z and write them to its workspace slot.
// READOUT = true : start from the exclusive prefix in the slot and write the outputs.
template <int NT, int CS, bool BF16, bool READOUT>
__global__ __launch_bounds__(kThreads) void prefill_mfma_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv, const void* __restrict__ vv, float* __restrict__ o,
    float* __restrict__ ws, int N, int L, int nseg, long long stride, float scale) {
  using G = Geo<NT>;
  using SM = Smem<NT, CS, BF16>;
  using E = typename SM::E;
  constexpr int W = G::W, WP = G::WP, NAT = G::NAT, NKB = G::NKB;
  constexpr int NIT = CS / 16;
  constexpr int EPP = 16 / sizeof(E);  // elements per 16-byte piece
  static_assert(CS == 64 || CS == 128, "chunk of 64 or 128 tokens");
  __shared__ SM sm;

  const E* q = reinterpret_cast<const E*>(qv);
  const E* k = reinterpret_cast<const E*>(kv);
  const E* v = reinterpret_cast<const E*>(vv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int seg = blockIdx.x;
  const long long bh = blockIdx.y;
  const int t_begin = seg * L, t_end = min(N, t_begin + L);
  const long long hbase = bh * (long long)N;
  float* slot = ws + (bh * nseg + seg) * stride;

  // Running state: Srun[t][r] = S[16t + 4lg + r][16w + l16].
  f32x4 Srun[NAT];
#pragma unroll
  for (int t = 0; t < NAT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = 16 * t + 4 * lg + r;
      Srun[t][r] = (READOUT && a < W) ? slot[(long long)a * kDV + 16 * w + l16] : 0.f;
    }
  for (int s = tid; s < WP; s += kThreads) {
    const int a = slot_feature<BF16>(s);
    sm.z[0][s] = (READOUT && a < W) ? slot[(long long)W * kDV + a] : 0.f;
  }
  int zb = 0;

  // bfloat16 readout operands: S = hi + lo, in the A-operand k-slot order.
  bf16x8 Shi[BF16 && READOUT ? NKB : 1], Slo[BF16 && READOUT ? NKB : 1];
  auto split_state = [&]() {
    if constexpr (BF16 && READOUT) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float x = r < 4 ? Srun[2 * kb][r] : Srun[2 * kb + 1][r - 4];
          const __bf16 hi = (__bf16)x;
          Shi[kb][r] = hi;
          Slo[kb][r] = (__bf16)(x - (float)hi);
        }
    }
  };
  split_state();

  for (int c0 = t_begin; c0 < t_end; c0 += CS) {
    const int nv = min(CS, t_end - c0);
    const long long tok0 = hbase + c0;

    // ---- A1: chunk inputs to LDS (q, k rows as is; v transposed) ----
    {
      constexpr int PR = kDK / EPP;  // 16-byte pieces per q/k row
      for (int p = tid; p < CS * PR; p += kThreads) {
        const int row = p / PR, pc = p % PR;
        uint4 zq = make_uint4(0, 0, 0, 0), zk = zq;
        if (row < nv) {
          zk = *reinterpret_cast<const uint4*>(k + (tok0 + row) * kDK + pc * EPP);
          if (READOUT) zq = *reinterpret_cast<const uint4*>(q + (tok0 + row) * kDK + pc * EPP);
        }
        *reinterpret_cast<uint4*>(&sm.k[row][pc * EPP]) = zk;
        if (READOUT) *reinterpret_cast<uint4*>(&sm.q[row][pc * EPP]) = zq;
      }
      constexpr int PV = kDV / EPP;  // 16-byte pieces per v row
      for (int p = tid; p < CS * PV; p += kThreads) {
        const int j = p % CS, pc = p / CS;
        union {
          uint4 u;
          E e[EPP];
        } buf;
        buf.u = make_uint4(0, 0, 0, 0);
        if (j < nv) buf.u = *reinterpret_cast<const uint4*>(v + (tok0 + j) * kDV + pc * EPP);
#pragma unroll
        for (int r = 0; r < EPP; ++r) sm.vt[pc * EPP + r][j] = buf.e[r];
      }
    }
    __syncthreads();

    // ---- A2: features phi(K_c)^T (and phi(sQ_c)) ----
    features<NT, CS, BF16>(sm, w, l, nv, scale, READOUT);
    __syncthreads();

    // ---- B: normaliser, inter denominators, scores, readout ----
    if (tid < WP) {
      const int a = slot_feature<BF16>(tid);
      float acc = 0.f;
      if constexpr (BF16) {
#pragma unroll
        for (int j = 0; j < CS; j += 8) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(&sm.phikt[a][j]);
#pragma unroll
          for (int r = 0; r < 8; ++r) acc += (float)x[r];
        }
      } else {
#pragma unroll
        for (int j = 0; j < CS; j += 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.phikt[a][j]);
          acc += (x[0] + x[1]) + (x[2] + x[3]);
        }
      }
      sm.z[zb ^ 1][tid] = sm.z[zb][tid] + acc;
    }

    f32x4 O[READOUT ? NIT : 1];
    if constexpr (READOUT) {
      // inter-chunk denominators: phi(sq_i) . z_{<c}, split over kThreads/CS parts
      {
        constexpr int P = kThreads / CS, SPP = WP / P;
        const int i = tid % CS, part = tid / CS;
        float acc = 0.f;
        for (int s = part * SPP; s < (part + 1) * SPP; s += EPP) {
          if constexpr (BF16) {
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(&sm.phiq[i][s]);
#pragma unroll
            for (int r = 0; r < 8; ++r) acc = fmaf((float)x[r], sm.z[zb][s + r], acc);
          } else {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.phiq[i][s]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc = fmaf(x[r], sm.z[zb][s + r], acc);
          }
        }
        sm.den_part[part][i] = acc;
      }
      // intra-chunk scores for the (key tile jt <= query tile it) pairs of this wave
      for (int p = w; p < SM::NPAIR; p += 4) {
        int it = 0;
        while ((it + 1) * (it + 2) / 2 <= p) ++it;
        const int jt = p - it * (it + 1) / 2;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF16) {
          const bf16x4 av = *reinterpret_cast<const bf16x4*>(&sm.k[16 * jt + l16][4 * lg]);
          const bf16x4 bv = *reinterpret_cast<const bf16x4*>(&sm.q[16 * it + l16][4 * lg]);
          sc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, av), __builtin_bit_cast(i16x4, bv),
                                                         sc, 0, 0, 0);
        } else {
          const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.k[16 * jt + l16][4 * lg]);
          const f32x4 bv = *reinterpret_cast<const f32x4*>(&sm.q[16 * it + l16][4 * lg]);
#pragma unroll
          for (int r = 0; r < 4; ++r) sc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r], bv[r], sc, 0, 0, 0);
        }
        // sc[r] = k_j . q_i with j = 16jt + 4lg + r, i = 16it + l16
        typename SM::ATile tile;
        float dsum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * jt + 4 * lg + r, i = 16 * it + l16;
          float wgt = j <= i ? taylor_kernel<NT>(scale * sc[r]) : 0.f;
          if constexpr (BF16) {
            tile[r] = (__bf16)wgt;
            dsum += (float)tile[r];
          } else {
            tile[r] = wgt;
            dsum += wgt;
          }
        }
        sm.a[p][l] = tile;
        dsum += __shfl_xor(dsum, 16);
        dsum += __shfl_xor(dsum, 32);
        if (lg == 0) sm.den_intra[p][l16] = dsum;
      }
      // readout: O[it][r] = (phi(sQ) S)[token 16it + l16][column 16w + 4lg + r]
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF16) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&sm.phiq[16 * it + l16][32 * kb + 8 * lg]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Shi[kb], bq, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Slo[kb], bq, acc, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int t = 0; t < NAT; ++t) {
            const f32x4 bq = *reinterpret_cast<const f32x4*>(&sm.phiq[16 * it + l16][16 * t + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Srun[t][r], bq[r], acc, 0, 0, 0);
          }
        }
        O[it] = acc;
      }
    }
    __syncthreads();

    // ---- C: denominators, intra-chunk PV, state update ----
    if constexpr (READOUT) {
      if (tid < CS) {
        const int i = tid, it = i / 16;
        float d = 0.f;
#pragma unroll
        for (int part = 0; part < kThreads / CS; ++part) d += sm.den_part[part][i];
        for (int jt = 0; jt <= it; ++jt) d += sm.den_intra[pair_index(jt, it)][i % 16];
        sm.den[i] = d;
      }
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        for (int jt = 0; jt <= it; ++jt) {
          const int p = pair_index(jt, it);
          if constexpr (BF16) {
            const bf16x4 av = *reinterpret_cast<const bf16x4*>(&sm.vt[16 * w + l16][16 * jt + 4 * lg]);
            const bf16x4 bv = sm.a[p][l];
            O[it] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, av),
                                                              __builtin_bit_cast(i16x4, bv), O[it], 0, 0, 0);
          } else {
            const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.vt[16 * w + l16][16 * jt + 4 * lg]);
            const f32x4 bv = sm.a[p][l];
#pragma unroll
            for (int r = 0; r < 4; ++r) O[it] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r], bv[r], O[it], 0, 0, 0);
          }
        }
      }
    }
    // state update: Srun[t] += phi(K)^T[16t.., chunk] V[chunk, 16w..]
    if constexpr (BF16) {
#pragma unroll
      for (int jb = 0; jb < CS / 32; ++jb) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&sm.vt[16 * w + l16][32 * jb + 8 * lg]);
#pragma unroll
        for (int t = 0; t < NAT; ++t) {
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&sm.phikt[16 * t + l16][32 * jb + 8 * lg]);
          Srun[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bv, Srun[t], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int jb = 0; jb < CS / 16; ++jb) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(&sm.vt[16 * w + l16][16 * jb + 4 * lg]);
#pragma unroll
        for (int t = 0; t < NAT; ++t) {
          const f32x4 ak = *reinterpret_cast<const f32x4*>(&sm.phikt[16 * t + l16][16 * jb + 4 * lg]);
#pragma unroll
          for (int r = 0; r < 4; ++r) Srun[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[r], bv[r], Srun[t], 0, 0, 0);
        }
      }
    }
    __syncthreads();

    // ---- D: outputs, next readout operands ----
    if constexpr (READOUT) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int i = 16 * it + l16;
        if (i < nv) {
          const float d = sm.den[i];
          f32x4 r = O[it];
          *reinterpret_cast<f32x4*>(o + (tok0 + i) * kDV + 16 * w + 4 * lg) =
              f32x4{r[0] / d, r[1] / d, r[2] / d, r[3] / d};
        }
      }
      split_state();
    }
    zb ^= 1;
  }

  if constexpr (!READOUT) {
#pragma unroll
    for (int t = 0; t < NAT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = 16 * t + 4 * lg + r;
        if (a < W) slot[(long long)a * kDV + 16 * w + l16] = Srun[t][r];
      }
    if (tid < WP) {
      const int a = slot_feature<BF16>(tid);
      if (a < W) slot[(long long)W * kDV + a] = sm.z[zb][tid];
    }
  }
}

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Segments per head: enough workgroups to cover the chip about twice, never more than the chunks.
int n_segments(int BH, int nchunk) {
  long long want = (512 + BH - 1) / BH;
  if (want < 1) want = 1;
  if (want > nchunk) want = nchunk;
  return (int)want;
}

template <int NT, int CS, bool BF16>
int run(const PrefillArgs& a) {
  const int nchunk = cdiv(a.N, CS);
  const int nseg0 = n_segments(a.BH, nchunk);
  const int L = cdiv(nchunk, nseg0) * CS;
  const int nseg = cdiv(a.N, L);
  float* ws = (float*)a.ws;
  const long long elems = Geo<NT>::W * (long long)(kDV + 1);
  const dim3 grid(nseg, a.BH), block(kThreads);
  prefill_mfma_kernel<NT, CS, BF16, false>
      <<<grid, block, 0, a.stream>>>(a.q, a.k, a.v, nullptr, ws, a.N, L, nseg, a.s.stride, a.s.scale);
  if (hipGetLastError() != hipSuccess) return -3;
  if (seg_scan_launch(ws, a.state, a.BH, nseg, a.s.stride, elems, a.o != nullptr, a.stream)) return -3;
  if (a.o) {
    prefill_mfma_kernel<NT, CS, BF16, true>
        <<<grid, block, 0, a.stream>>>(a.q, a.k, a.v, a.o, ws, a.N, L, nseg, a.s.stride, a.s.scale);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

// This path walks 64-token chunks whatever the configured chunk (64 or 128): a 128-token chunk
// needs more registers than a wavefront has for the readout (the outputs do not depend on the
// chunk length beyond rounding), and 64 keeps two workgroups per CU for bfloat16 inputs.
constexpr int kChunk = 64;

template <int NT>
int run_dtype(const PrefillArgs& a) {
  return a.s.dtype == 1 ? run<NT, kChunk, true>(a) : run<NT, kChunk, false>(a);
}

}  // namespace

bool prefill_mfma_has(int nt, int dk, int dv, int C) {
  return dk == kDK && dv == kDV && nt >= 1 && nt <= 3 && (C == 64 || C == 128);
}

long long prefill_mfma_ws_bytes(const Shape& s, int BH, int N, int C) {
  const int CS = kChunk;
  const int nchunk = cdiv(N, CS);
  const int nseg0 = n_segments(BH, nchunk);
  const int L = cdiv(nchunk, nseg0) * CS;
  return (long long)BH * cdiv(N, L) * s.stride * 4;
}

int prefill_mfma_launch(const PrefillArgs& a) {
  if (!prefill_mfma_has(a.s.nt, a.s.dk, a.s.dv, a.C)) return -2;
  switch (a.s.nt) {
    case 1: return run_dtype<1>(a);
    case 2: return run_dtype<2>(a);
    default: return run_dtype<3>(a);
  }
}

}  // namespace taylor
