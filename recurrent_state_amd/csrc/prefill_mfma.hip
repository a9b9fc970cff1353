// Pipelined bfloat16 chunked prefill for d_k = 16, d_v = 64, n = 1..3 (gfx950 matrix cores).
//
// "Expanding Attention" (Huang, arXiv:2610.20637), Abstract: with the kernel
// exp(s) truncated to n Taylor terms and each term factorised into symmetric
// tensor-power features, the causal history is n additive states, so prefill
// is chunk-local work plus a scan of chunk states.  Per chunk c of C tokens,
// with V1 = [V | 1] (the value columns plus the normaliser column):
//     O_c  = phi(s Q_c) S_{<c}  +  tril(K_n(s Q_c K_c^T)) V1_c     ([numerators | denominator])
//     S   += phi(K_c)^T V1_c                                        (state and normaliser z)
//     o    = O_c[:, :d_v] / O_c[:, d_v]
//
// One workgroup walks a segment of consecutive 64-token chunks with the running state S_{<c} of the
// segment in MFMA accumulator registers; two launches bracket the scan: a state-only pass writes
// each segment's (S, z) increment to the workspace, the scan turns those into exclusive prefixes,
// and the readout pass starts each segment from its prefix.  Where one segment per (sequence, head)
// pair is estimated faster (short prompts, many pairs), the readout pass alone runs, from the
// incoming state to the final one.  q, k, v, phi and the score weights
// enter bfloat16 MFMAs; S and the weights are split as bfloat16 hi + lo where they meet the MFMAs
// (float32 accuracy for the state), and all accumulation and the outputs are float32.  (float32
// inputs run on the feature-block kernels of prefill_wide.hip.)
#include <algorithm>
#include <atomic>
#include <cstddef>
#include <chrono>
#include <type_traits>
#include <utility>

#include "centered.hpp"
#include "features.hpp"
#include "lds_layout.hpp"
#include "lookback.hpp"
#include "prefill_mfma.hpp"

namespace taylor {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bfloat16 (nearest even) by one conversion instruction.
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) { return __builtin_convertvector(f32x2{a, b}, bf16x2); }

// Splits x = (a, b) into bfloat16 pairs hi = bf16(x), lo = bf16(x - hi), so hi + lo carries x to
// about 16 significant bits.
__device__ __forceinline__ void split_bf16x2(float a, float b, bf16x2& hi, bf16x2& lo) {
  hi = to_bf16x2(a, b);
  const uint32_t u = __builtin_bit_cast(uint32_t, hi);
  lo = to_bf16x2(a - __uint_as_float(u << 16), b - __uint_as_float(u & 0xffff0000u));
}
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDK = 16, kDV = 64;

template <int NT>
struct Geo {
  static constexpr int W = FeatureTable<NT, kDK>::W;
  static constexpr int WP = (W + 31) / 32 * 32;  // features padded to 32-wide MFMA k-blocks
  static constexpr int NAT = WP / 16;            // 16-row feature tiles of the state
  static constexpr int NKB = WP / 32;            // 32-wide feature k-blocks
};

// Feature A of x (float32 registers), coordinates and coefficient fixed at compile time.
template <int NT, int A>
__device__ __forceinline__ float feat(const float (&x)[kDK]) {
  return feature_ct<NT, kDK, A>(x);
}

// bfloat16 path: position s of a phi(sQ) row holds feature slot_feature(s), the k-slot order of the
// accumulator-fed A operand (lane group g holds features 4g..4g+3 and 16+4g..16+4g+3 of each 32-block).
__host__ __device__ constexpr int slot_feature_bf16(int s) {
  const int kb = s / 32, r32 = s % 32, g = r32 / 8, r = r32 % 8;
  return 32 * kb + (r < 4 ? g * 4 + r : 16 + g * 4 + (r - 4));
}

// The slot of feature f in a phi(sQ) row (the inverse of slot_feature_bf16).
__host__ __device__ constexpr int feature_slot_bf16(int f) {
  const int kb = f / 32, f32 = f % 32, hi = f32 >= 16, u = f32 % 16;
  return 32 * kb + 8 * (u / 4) + 4 * hi + u % 4;
}

__device__ __forceinline__ int pair_index(int jt, int it) { return it * (it + 1) / 2 + jt; }

// x where ok holds, else zero, selected word by word (a select of the whole vector would take the
// operands' addresses and move them to scratch memory).
__device__ __forceinline__ uint4 keep_if(bool ok, uint4 x) {
  return make_uint4(ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u);
}

// ------------------------------------------------------------------------------------------------
// Pipelined bfloat16 prefill: 8 wavefronts per workgroup, one barrier per chunk.
//
// Waves 0..3 ("consumers") own value columns 16w..16w+15 and run the MFMAs of chunk c:
// the readout phi(sQ_c) S_{<c} (state kept in accumulator registers, split hi + lo), the
// denominators phi(sQ_c) z_{<c} (z as hi + lo, one more product per readout operand), the
// intra-chunk product V^T tril(K_n(s K Q^T)), the state update phi(K_c)^T V_c, and the
// output division.  Waves 4..7 ("producers") meanwhile prepare chunk c+1 in the other half
// of a double-buffered LDS area: phi(K)^T rows, phi(sQ) rows (slot-permuted), V^T, the
// intra-chunk score tiles (16x16x16 MFMA + Horner + causal mask, stored as bfloat16 hi + lo
// so the intra-chunk weights keep float32 accuracy) with their row sums (the intra-chunk
// denominator part), and z_{<c+1} (kept in LDS in float32, each producer owning a quarter of the
// features, and handed to the consumers as hi + lo).  Producers read their inputs straight
// from global memory, issued a whole chunk ahead.  The single barrier per chunk both hands
// buffer c+1 to the consumers and returns buffer c to the producers.  The feature work per
// token (vector ALU) and the LDS traffic of the operands bound this kernel; the matrix work
// is a fraction of it.
// ------------------------------------------------------------------------------------------------
constexpr int kPipeConsumers = 4;  // one per 16 value columns
constexpr int kRankMax = 512;      // ragged one-pass batches up to this many sequences run longest first
constexpr int kPipeProducers = 4;
constexpr int kPipeThreads = 64 * (kPipeConsumers + kPipeProducers);
constexpr int kPipeChunk = kMfmaChunk;
constexpr int kPipePairs = 10;  // (key tile <= query tile) pairs of 16-token tiles in a chunk

template <int NT, bool READOUT>
struct PipeSmem {
  static constexpr int WP = Geo<NT>::WP;
  // Unpadded rows, 16-byte slots swizzled within each row (swz_kv, swz_q): every access the kernels
  // make of the three tiles below is free of LDS bank conflicts.
  static constexpr int RQ = READOUT ? kPipeChunk : 1;
  static constexpr int RP = READOUT ? kPipePairs : 1;
  alignas(16) __bf16 vt[2][kDV][kPipeChunk];
  alignas(16) __bf16 phikt[2][WP][kPipeChunk];
  alignas(16) __bf16 phiq[2][RQ][WP];
  alignas(16) bf16x4 a[2][RP][64];    // score tiles, high bfloat16 part
  alignas(16) bf16x4 alo[2][RP][64];  // score tiles, low part (w - hi), so hi + lo keeps float32 accuracy
  // z_{<c} as bfloat16 hi (row 0) and lo (row 1) in phi(sQ) slot order: the A operand of the
  // denominator phi(sQ) z, one more matrix-core product of the readout (truncated-kernel readout)
  alignas(16) __bf16 zop[2][2][READOUT ? WP : 8];
  float den_part[2][kPipeProducers][RQ];  // expanded-softmax readout: gamma_0 of each token
  float den_intra[2][RP][16];
  float z[2][WP];  // z_{<c} for chunk parity c & 1, natural feature order
};

// Producer split: producer g owns phi(K)^T rows [g*RK, g*RK + RK) and phi(sQ) 8-slot groups
// [g*RG, g*RG + RG) (clipped to the padded width); it also keeps z for its rows, writes value
// columns [g*VC, g*VC + VC) of V^T and computes score tiles g, g + kPipeProducers, ...
template <int NT>
struct PipeSplit {
  static constexpr int WP = Geo<NT>::WP;
  static constexpr int RK = ((WP + kPipeProducers - 1) / kPipeProducers + 1) / 2 * 2;
  static constexpr int NG = WP / 8;
  static constexpr int RG = (NG + kPipeProducers - 1) / kPipeProducers;
  static constexpr int VC = kDV / kPipeProducers;
};

// LDS layout of the bfloat16 tiles (lds_layout.hpp): unpadded rows, 16-byte slots swizzled by row.
static_assert(kPipeChunk == 64, "phi(K)^T and V^T rows are 128 bytes: 8 slots of 8 tokens");
__device__ __forceinline__ int kv_bf16(int r, int t) { return kv_off<2>(r, t); }
template <int NT>
__device__ __forceinline__ int swz_q(int r) { return swz_tok<Geo<NT>::WP / 8>(r); }

// phi(K)^T rows are written two rows at a time as whole dwords: lane j holds (row r, row r+1) of
// token j; lanes j and j^1 swap those pairs (a quad permutation), then the even lane stores row r of
// tokens j, j+1 and the odd lane row r+1 of tokens j-1, j.  For even r, swz_kv(r + 1) = swz_kv(r) ^ 4,
// so the odd lanes flip bit 2 of their slot once, here.
struct PairStore {
  char* base;    // the lane's row (r or r + 1) and dword within its slot
  int slot;      // the lane's slot before the row's swizzle
  uint32_t sel;  // v_perm_b32(partner, own) bytes: even -> (own.lo, partner.lo), odd -> (partner.hi, own.hi)
  __device__ __forceinline__ PairStore(__bf16* tile, int j) {
    const bool odd = j & 1;
    base = reinterpret_cast<char*>(tile) + (odd ? 128 : 0) + 4 * ((j >> 1) & 3);
    slot = (j >> 3) ^ (odd ? 4 : 0);
    sel = odd ? 0x03020706u : 0x05040100u;
  }
  template <int R>  // even row of the pair
  __device__ __forceinline__ void store(uint32_t own) const {
    static_assert(R % 2 == 0, "rows are written in pairs from an even row");
    const uint32_t partner = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    *reinterpret_cast<uint32_t*>(base + R * 128 + 16 * (slot ^ swz_kv(R))) = __builtin_amdgcn_perm(partner, own, sel);
  }
};

// A token past the end has a zero k row, so all its features are zero except the constant one.
template <int NT, bool READOUT, int G>
__device__ __forceinline__ void pipe_phik_rows(PipeSmem<NT, READOUT>& sm, int b, int j, const float (&x)[kDK],
                                               bool valid) {
  using SP = PipeSplit<NT>;
  static_assert(SP::RK % 2 == 0, "rows are written in pairs");
  const PairStore ps(&sm.phikt[b][0][0], j);
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (([&] {
       constexpr int r0 = G * SP::RK + 2 * I, r1 = r0 + 1;
       if constexpr (r0 < SP::WP) {
         float f0;
         if constexpr (r0 == 0)
           f0 = valid ? 1.f : 0.f;
         else
           f0 = feat<NT, r0>(x);
         ps.store<r0>(__builtin_bit_cast(uint32_t, to_bf16x2(f0, feat<NT, r1>(x))));
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, SP::RK / 2>{});
}

// Order of feature A (0 for the padding slots past the table, whose features are zero).
template <int NT, int A>
constexpr int feature_order() {
  if constexpr (A < Geo<NT>::W)
    return FeatureTable<NT, kDK>::T.order[A];
  else
    return 0;
}

// Feature A of x, scaled by its order's coefficient in CENT mode (expanded-softmax readout).  There
// the constant feature is left out (zero): its term gamma_0 S_{<c} row 0 is added by the consumers
// in float32, since a bfloat16 gamma_0 would carry a 2^-9 relative error into the largest term of the
// output (the truncated-kernel readout shares its feature roundings with its normaliser; this one
// has none).
template <int NT, bool CENT, int A>
__device__ __forceinline__ float qfeat(const float (&x)[kDK], const f32x4& cq) {
  if constexpr (CENT && A == 0)
    return 0.f;
  else if constexpr (CENT)
    return feat<NT, A>(x) * cq[feature_order<NT, A>()];
  else
    return feat<NT, A>(x);
}

// Writes this wave's phi(sQ) groups of token j (CENT: the features scaled by the token's coefficients
// gamma_m).
template <int NT, bool READOUT, bool CENT, int G>
__device__ __forceinline__ void pipe_phiq_groups(PipeSmem<NT, READOUT>& sm, int b, int j, const float (&x)[kDK],
                                                 const f32x4& cq) {
  using SP = PipeSplit<NT>;
  [&]<int... P>(std::integer_sequence<int, P...>) {
    (([&] {
       constexpr int grp = G * SP::RG + P;
       if constexpr (grp < SP::NG) {
         constexpr int s0 = grp * 8;
         uint32_t v[4];
         [&]<int... R>(std::integer_sequence<int, R...>) {
           ((v[R] = __builtin_bit_cast(uint32_t,
                                       to_bf16x2(qfeat<NT, CENT, slot_feature_bf16(s0 + 2 * R)>(x, cq),
                                                 qfeat<NT, CENT, slot_feature_bf16(s0 + 2 * R + 1)>(x, cq)))),
            ...);
         }(std::make_integer_sequence<int, 4>{});
         *reinterpret_cast<uint4*>(reinterpret_cast<char*>(&sm.phiq[b][j][0]) + 16 * (grp ^ swz_q<NT>(j))) =
             make_uint4(v[0], v[1], v[2], v[3]);
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, SP::RG>{});
}

// Query tile and key tile of intra-chunk score pair p (pairs ordered by query tile, then key tile).
constexpr int pair_it(int p) {
  int it = 0;
  while ((it + 1) * (it + 2) / 2 <= p) ++it;
  return it;
}
constexpr int pair_jt(int p) { return p - pair_it(p) * (pair_it(p) + 1) / 2; }

// Score pairs of producer G: G, G + kPipeProducers, ...
template <int G>
constexpr int producer_pairs() {
  return G < kPipePairs ? (kPipePairs - G + kPipeProducers - 1) / kPipeProducers : 0;
}

// Producer G's inputs for one chunk, loaded a chunk ahead of use (lane = token j of the chunk).  CENT
// (expanded-softmax readout) adds the coefficients of the lane's token and of each score tile's
// query column.
template <bool READOUT, bool CENT, int G>
struct PipeIn {
  static constexpr int NS = READOUT ? producer_pairs<G>() : 0;
  static constexpr int NVP = kDV / kPipeProducers / 8;  // 16-byte pieces of v per producer lane
  static_assert(NVP * 8 * kPipeProducers == kDV, "value columns split evenly over producers");
  uint4 k[2], q[READOUT ? 2 : 1], v[NVP];
  uint2 sk[NS > 0 ? NS : 1], sq[NS > 0 ? NS : 1];  // score MFMA operands of this producer's tiles
  f32x4 cq, csq[CENT && NS > 0 ? NS : 1];

  // Tokens past the end read the chunk's first row (always valid), so every load is an
  // unconditional global load whose result is not touched until it is used a chunk later.  Only
  // k needs masking (its features enter S and z) and that happens at unpack time; q, v and the
  // score operands of such tokens never reach a stored output (causal mask, output guard).
  __device__ __forceinline__ void load(const __bf16* qg, const __bf16* kg, const __bf16* vg, const float* cf,
                                       long long tok0, int nv, int l) {
    const long long row = tok0 + (l < nv ? l : 0);
    if constexpr (CENT) cq = *reinterpret_cast<const f32x4*>(cf + 4 * row);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      k[u] = *reinterpret_cast<const uint4*>(kg + row * kDK + 8 * u);
      if constexpr (READOUT) q[u] = *reinterpret_cast<const uint4*>(qg + row * kDK + 8 * u);
    }
#pragma unroll
    for (int u = 0; u < NVP; ++u) v[u] = *reinterpret_cast<const uint4*>(vg + row * kDV + 8 * (NVP * G + u));
    const int l16 = l & 15, lg = l >> 4;
    [&]<int... S>(std::integer_sequence<int, S...>) {
      (([&] {
         constexpr int p = G + kPipeProducers * S;
         const int rk = 16 * pair_jt(p) + l16, rq = 16 * pair_it(p) + l16;
         sk[S] = *reinterpret_cast<const uint2*>(kg + (tok0 + (rk < nv ? rk : 0)) * kDK + 4 * lg);
         sq[S] = *reinterpret_cast<const uint2*>(qg + (tok0 + (rq < nv ? rq : 0)) * kDK + 4 * lg);
         if constexpr (CENT) csq[S] = *reinterpret_cast<const f32x4*>(cf + 4 * (tok0 + (rq < nv ? rq : 0)));
       }()),
       ...);
    }(std::make_integer_sequence<int, NS>{});
  }
};

__device__ __forceinline__ void unpack_row16(const uint4 (&r)[2], float (&x)[kDK], float scale) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t w[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      x[8 * u + 2 * h] = scale * __uint_as_float(w[h] << 16);
      x[8 * u + 2 * h + 1] = scale * __uint_as_float(w[h] & 0xffff0000u);
    }
  }
}

// Producer wave G prepares chunk data in buffer b (chunk parity), with z_{<chunk} in z[b].
template <int NT, bool READOUT, bool CENT, int G>
__device__ __forceinline__ void pipe_produce(PipeSmem<NT, READOUT>& sm, const PipeIn<READOUT, CENT, G>& in, int b,
                                             int l, int nv, float scale, float* zrow) {
  using SP = PipeSplit<NT>;
  constexpr int WP = Geo<NT>::WP;
  const int l16 = l & 15, lg = l >> 4;
  if constexpr (!READOUT && CENT) {
    // state pass before an expanded-softmax readout: z of the piece's tokens before this chunk, into
    // this chunk's row of the per-chunk array (the coefficient kernel adds the piece's prefix)
    const int row = G * SP::RK + l;
    if (l < SP::RK && row < Geo<NT>::W) zrow[row] = sm.z[b][row];
  }
  {
    float x[kDK];
    const bool valid = l < nv;  // a token past the end has a zero k row
    const uint4 kr[2] = {keep_if(valid, in.k[0]), keep_if(valid, in.k[1])};
    unpack_row16(kr, x, 1.0f);
    pipe_phik_rows<NT, READOUT, G>(sm, b, l, x, valid);
  }
  if constexpr (READOUT && !CENT) {
    // z_{<chunk} of this wave's rows (written by the same lanes in the previous phase) as the
    // consumers' denominator operand: hi + lo keeps about 16 significant bits
    const int row = G * SP::RK + l;
    if (l < SP::RK && row < WP) {
      const float zr = sm.z[b][row];
      const __bf16 hi = (__bf16)zr;
      const int s = feature_slot_bf16(row);
      sm.zop[b][0][s] = hi;
      sm.zop[b][1][s] = (__bf16)(zr - (float)hi);
    }
  }
  if constexpr (READOUT) {
    float x[kDK];
    unpack_row16(in.q, x, scale);
    pipe_phiq_groups<NT, READOUT, CENT, G>(sm, b, l, x, in.cq);
    if constexpr (CENT && G == 0)
      sm.den_part[b][0][l] = in.cq[0];  // gamma_0 of token l, for the consumers' constant-feature term
  }
  // V^T: this producer's value columns of token l (16-bit stores: the dword pairing measured no
  // faster here)
#pragma unroll
  for (int u = 0; u < PipeIn<READOUT, CENT, G>::NVP; ++u) {
    const uint32_t w[4] = {in.v[u].x, in.v[u].y, in.v[u].z, in.v[u].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int c = SP::VC * G + 8 * u + 2 * h;
      char* vt = reinterpret_cast<char*>(&sm.vt[b][0][0]);
      *reinterpret_cast<uint16_t*>(vt + kv_bf16(c, l)) = (uint16_t)(w[h] & 0xffffu);
      *reinterpret_cast<uint16_t*>(vt + kv_bf16(c + 1, l)) = (uint16_t)(w[h] >> 16);
    }
  }
  if constexpr (READOUT) {
    // intra-chunk score tiles of this wave's pairs, and their row sums (denominator part)
    [&]<int... S>(std::integer_sequence<int, S...>) {
      (([&] {
         constexpr int p = G + kPipeProducers * S, it = pair_it(p), jt = pair_jt(p);
         f32x4 sc = {0.f, 0.f, 0.f, 0.f};
         sc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, in.sk[S]),
                                                        __builtin_bit_cast(i16x4, in.sq[S]), sc, 0, 0, 0);
         float wgt[4];
#pragma unroll
         for (int r = 0; r < 4; ++r) {
           const int j = 16 * jt + 4 * lg + r, i = 16 * it + l16;
           const float s = scale * sc[r];
           // CENT: gamma_0 + gamma_1 s + gamma_2 s^2 / 2 of query i (gamma_2 = 0 at order 1)
           float poly;
           if constexpr (CENT)
             poly = fmaf(s, fmaf(0.5f * s, in.csq[S][2], in.csq[S][1]), in.csq[S][0]);
           else
             poly = taylor_kernel<NT>(s);
           wgt[r] = (jt < it || j <= i) ? poly : 0.f;
         }
         bf16x2 h0, l0, h1, l1;
         split_bf16x2(wgt[0], wgt[1], h0, l0);
         split_bf16x2(wgt[2], wgt[3], h1, l1);
         const bf16x4 hi = {h0[0], h0[1], h1[0], h1[1]}, lo = {l0[0], l0[1], l1[0], l1[1]};
         sm.a[b][p][l] = hi;
         sm.alo[b][p][l] = lo;
         if constexpr (!CENT) {
           // column sums over the 16 key rows, as ones^T (hi + lo): every row of the product holds them
           const bf16x8 ones = __builtin_bit_cast(bf16x8, i16x8{0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80,
                                                                 0x3f80, 0x3f80});
           const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
           // hi and lo in the two halves of k: one 16x16x32 MFMA sums both
           const f32x4 cs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
               ones, __builtin_shufflevector(hi, lo, 0, 1, 2, 3, 4, 5, 6, 7), zero, 0, 0, 0);
           if (lg == 0) sm.den_intra[b][p][l16] = cs[0];
         }
       }()),
       ...);
    }(std::make_integer_sequence<int, PipeIn<READOUT, CENT, G>::NS>{});
  }
  // z_{<next} = z_{<this} + column sums of this wave's phi(K)^T rows (read back from LDS: the
  // rows were written by this same wave above, and a wave's LDS accesses complete in order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int row = G * SP::RK + l;
  if (l < SP::RK && row < WP) {
    float acc = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int t = 0; t < kPipeChunk; t += 8) {
      const bf16x8 x8 = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(&sm.phikt[b][0][0]) + kv_bf16(row, t));
#pragma unroll
      for (int h = 0; h < 4; ++h) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x8[2 * h], x8[2 * h + 1]}, ones, acc, false);
    }
    sm.z[b ^ 1][row] = sm.z[b][row] + acc;
  }
}

// Producer G over one segment of nch chunks.  Phase c (consumers on chunk c) prepares chunk c+1
// in buffer (c+1) & 1 and issues the loads of chunk c+2; the two register sets a and b alternate
// so no loaded value is copied.  The steady-state loop has no conditional load or produce (every
// load issued in it is consumed in it), so the compiler's memory-counter waits stay exact; the
// last one to three phases are peeled.  z starts from src (null: zero) and ends in dst (null: not
// written).  Executes exactly 2 + nch barriers.
template <int NT, bool READOUT, bool CENT, int G, bool COH = false>
__device__ __forceinline__ void pipe_producer(PipeSmem<NT, READOUT>& sm, const __bf16* q, const __bf16* k,
                                              const __bf16* v, const float* cf, const float* src, float* dst,
                                              float* zc0, long long tok_base, int n_tok, int nch, int l,
                                              float scale, float* keep = nullptr) {
  using SP = PipeSplit<NT>;
  constexpr int W = Geo<NT>::W, WP = Geo<NT>::WP, CS = kPipeChunk;
  auto nv_of = [&](int c) { return min(CS, n_tok - c * CS); };
  auto tok_of = [&](int c) { return tok_base + (long long)c * CS; };
  auto zrow = [&](int c) { return CENT && !READOUT ? zc0 + (long long)c * W : nullptr; };
  // z prefix of this producer's rows
  const int row = G * SP::RK + l;
  if (l < SP::RK && row < WP) sm.z[0][row] = (src && row < W) ? src[(long long)W * kDV + row] : 0.f;
  PipeIn<READOUT, CENT, G> pa, pb;
  pa.load(q, k, v, cf, tok_of(0), nv_of(0), l);
  __syncthreads();  // z prefix visible to every producer
  if (nch > 1) pb.load(q, k, v, cf, tok_of(1), nv_of(1), l);
  pipe_produce<NT, READOUT, CENT, G>(sm, pa, 0, l, nv_of(0), scale, zrow(0));
  __syncthreads();  // chunk 0 ready
  int c = 0;
  for (; c + 3 < nch; c += 2) {
    pa.load(q, k, v, cf, tok_of(c + 2), nv_of(c + 2), l);
    pipe_produce<NT, READOUT, CENT, G>(sm, pb, (c + 1) & 1, l, nv_of(c + 1), scale, zrow(c + 1));
    __syncthreads();
    pb.load(q, k, v, cf, tok_of(c + 3), nv_of(c + 3), l);
    pipe_produce<NT, READOUT, CENT, G>(sm, pa, c & 1, l, nv_of(c + 2), scale, zrow(c + 2));
    __syncthreads();
  }
  // nch - c phases remain (1 to 3); chunks c+1 and c+2 may still need preparing
  if (c + 2 < nch) pa.load(q, k, v, cf, tok_of(c + 2), nv_of(c + 2), l);
  if (c + 1 < nch) pipe_produce<NT, READOUT, CENT, G>(sm, pb, (c + 1) & 1, l, nv_of(c + 1), scale, zrow(c + 1));
  __syncthreads();
  if (c + 1 < nch) {
    if (c + 2 < nch) pipe_produce<NT, READOUT, CENT, G>(sm, pa, c & 1, l, nv_of(c + 2), scale, zrow(c + 2));
    __syncthreads();
    if (c + 2 < nch) __syncthreads();
  }
  if (dst && l < SP::RK && row < W) {
    put_state<COH>(dst + (long long)W * kDV + row, sm.z[nch & 1][row]);
    if (keep) keep[W * kDV + row] = sm.z[nch & 1][row];
  }
}

// Consumer wave w (value columns 16w..16w+15) over one piece: the running state starts from src
// (null: zero; a generic pointer, so it may sit in LDS), the outputs go to o (READOUT), and the state
// at the piece's end goes to dst (null: not written; `pad`: dst is a final state, whose padding after
// z is zeroed too).  Executes exactly 2 + nch barriers, like the producers.
template <int NT, bool READOUT, bool CENT, bool COH = false>
__device__ __forceinline__ void pipe_consumer(PipeSmem<NT, READOUT>& sm, const SeqPiece& pc, const float* src,
                                              float* dst, bool pad, float* __restrict__ o, long long stride,
                                              int w, int tid, float* keep = nullptr) {
  constexpr int W = Geo<NT>::W, NAT = Geo<NT>::NAT, NKB = Geo<NT>::NKB;
  constexpr int CS = kPipeChunk, NIT = CS / 16;
  const int l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int nch = (pc.n + CS - 1) / CS;

  // ---- consumers: wave w owns value columns 16w..16w+15 ----
  f32x4 Srun[NAT];
#pragma unroll
  for (int t = 0; t < NAT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = 16 * t + 4 * lg + r;
      Srun[t][r] = (src && a < W) ? src[(long long)a * kDV + 16 * w + l16] : 0.f;
    }
  __syncthreads();
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int b = c & 1;
    const int nv = min(CS, pc.n - c * CS);
    const long long tok0 = pc.tok + (long long)c * CS;
    const float srow0 = Srun[0][0];  // S_{<c}[0][16w + l16] on lanes 0..15 (CENT)
    f32x4 O[READOUT ? NIT : 1];
    // denominators phi(sQ) z_{<c}: operand rows 0..7 carry z hi, rows 8..15 z lo, so result rows 0..7
    // (lanes 0..31) hold the hi part and rows 8..15 (lanes 32..63) the lo part of each token's sum
    constexpr bool DEN = READOUT && !CENT;
    f32x4 Dz[DEN ? NIT : 1];
    if constexpr (READOUT) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) O[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (DEN)
#pragma unroll
        for (int it = 0; it < NIT; ++it) Dz[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      // readout with S_{<c} = hi + lo, one 32-feature k-block at a time
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        bf16x2 h[4], lw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4& src = Srun[2 * kb + (r >> 1)];
          split_bf16x2(src[2 * (r & 1)], src[2 * (r & 1) + 1], h[r], lw[r]);
        }
        const bf16x8 hi = {h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
        const bf16x8 lo = {lw[0][0], lw[0][1], lw[1][0], lw[1][1], lw[2][0], lw[2][1], lw[3][0], lw[3][1]};
        bf16x8 za;
        if constexpr (DEN) za = *reinterpret_cast<const bf16x8*>(&sm.zop[b][l16 >> 3][32 * kb + 8 * lg]);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const bf16x8 bq = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(&sm.phiq[b][16 * it + l16][0]) +
                                                             64 * kb + 16 * (lg ^ swz_q<NT>(l16)));
          O[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bq, O[it], 0, 0, 0);
          O[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bq, O[it], 0, 0, 0);
          if constexpr (DEN) Dz[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za, bq, Dz[it], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // bound the operands in flight (register budget)
      }
      // intra-chunk V^T x scores (weights as hi + lo)
#pragma unroll
      for (int it = 0; it < NIT; ++it)
#pragma unroll
        for (int jt = 0; jt <= it; ++jt) {
          const bf16x4 av = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const char*>(&sm.vt[b][0][0]) +
                                                             kv_bf16(16 * w + l16, 16 * jt + 4 * lg));
          const bf16x4 bh = sm.a[b][pair_index(jt, it)][l];
          const bf16x4 bl = sm.alo[b][pair_index(jt, it)][l];
          // V^T (hi + lo) as one 16x16x32 MFMA: the halves of k pair av with bh and av with bl
          O[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(av, av, 0, 1, 2, 3, 4, 5, 6, 7),
                                                         __builtin_shufflevector(bh, bl, 0, 1, 2, 3, 4, 5, 6, 7), O[it],
                                                         0, 0, 0);
        }
    }
    // state update
#pragma unroll
    for (int jb = 0; jb < CS / 32; ++jb) {
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(&sm.vt[b][0][0]) +
                                                         kv_bf16(16 * w + l16, 32 * jb + 8 * lg));
#pragma unroll
      for (int t = 0; t < NAT; ++t) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(&sm.phikt[b][0][0]) +
                                                           kv_bf16(16 * t + l16, 32 * jb + 8 * lg));
        Srun[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bv, Srun[t], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (READOUT) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int i = 16 * it + l16;
        float d = 1.f;  // the expanded-softmax readout has no normaliser
        if constexpr (!CENT) {
          // hi part (lanes 0..31) + lo part (lanes 32..63) of the token's phi(sq) . z: after the swap one
          // register holds lanes 0..31's values in both halves and the other lanes 32..63's, so their
          // sum is the same in lanes l and l ^ 32 (v_permlane32_swap: no LDS round trip)
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(Dz[it][0]), __float_as_uint(Dz[it][0]),
                                                           false, false);
          d = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
#pragma unroll
          for (int jt = 0; jt <= it; ++jt) d += sm.den_intra[b][pair_index(jt, it)][l16];
        } else {
          // + gamma_0(i) S_{<c}[0][16w + 4lg + r]: row 0 of columns 16w + 4lg .. lives on lanes 4lg ..
          const float g0 = sm.den_part[b][0][i];
#pragma unroll
          for (int r = 0; r < 4; ++r) O[it][r] = fmaf(g0, __shfl(srow0, 4 * lg + r), O[it][r]);
        }
        if (i < nv) {
          const float inv = CENT ? 1.0f : __builtin_amdgcn_rcpf(d);
          const f32x4 r = O[it];
          *reinterpret_cast<f32x4*>(o + (tok0 + i) * kDV + 16 * w + 4 * lg) =
              f32x4{r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv};
        }
      }
    }
    __syncthreads();
  }

  if (dst) {
#pragma unroll
    for (int t = 0; t < NAT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = 16 * t + 4 * lg + r;
        if (a < W) {
          put_state<COH>(dst + (long long)a * kDV + 16 * w + l16, Srun[t][r]);
          if (keep) keep[a * kDV + 16 * w + l16] = Srun[t][r];
        }
      }
    if (pad && w == 0)  // the padding after z
      for (long long e = (long long)W * (kDV + 1) + l; e < stride; e += 64) dst[e] = 0.f;
  }
}

// The producer waves (w >= kPipeConsumers) over one piece, each on its own compile-time role.
template <int NT, bool READOUT, bool CENT, bool COH = false>
__device__ __forceinline__ void pipe_producers(PipeSmem<NT, READOUT>& sm, int w, const __bf16* q, const __bf16* k,
                                               const __bf16* v, const float* cf, const float* src, float* dst,
                                               float* zc0, long long tok, int n, int l, float scale,
                                               float* keep = nullptr) {
  const int nch = (n + kPipeChunk - 1) / kPipeChunk;
  static_assert(kPipeProducers <= 8, "dispatch below lists up to 8 producers");
#define TAYLOR_PRODUCER(G_)                                                                              \
  case G_:                                                                                             \
    if constexpr (G_ < kPipeProducers)                                                                 \
      pipe_producer<NT, READOUT, CENT, G_, COH>(sm, q, k, v, cf, src, dst, zc0, tok, n, nch, l, scale, keep); \
    break;
  switch (w - kPipeConsumers) {
    TAYLOR_PRODUCER(0)
    TAYLOR_PRODUCER(1)
    TAYLOR_PRODUCER(2)
    TAYLOR_PRODUCER(3)
    TAYLOR_PRODUCER(4)
    TAYLOR_PRODUCER(5)
    TAYLOR_PRODUCER(6)
    TAYLOR_PRODUCER(7)
    default: break;
  }
#undef TAYLOR_PRODUCER
}

template <int NT, bool READOUT, bool PACKED, bool CENT>
__global__ __launch_bounds__(kPipeThreads) void prefill_pipe_kernel(const __bf16* __restrict__ q,
                                                                    const __bf16* __restrict__ k,
                                                                    const __bf16* __restrict__ v,
                                                                    const float* __restrict__ cf,
                                                                    float* __restrict__ o, float* __restrict__ ws,
                                                                    float* __restrict__ zc, const float* sin,
                                                                    float* sout, int direct, SeqMap seq, int L,
                                                                    long long nslot, long long stride, float scale) {
  using G = Geo<NT>;
  using SM = PipeSmem<NT, READOUT>;
  constexpr int W = G::W;
  __shared__ SM sm;

  // The role is taken from a wave-uniform scalar so each wave runs only its own loops; both roles
  // walk the same pieces and execute exactly 2 + nch barriers per piece.  Pieces follow one
  // another in LDS without an extra barrier: a piece's last barrier orders every read of its
  // buffers before the next piece's first writes, and the z rows each producer rewrites at a
  // piece's start are its own.
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long bx = blockIdx.x, by = blockIdx.y;
  // Where a piece's state starts and ends.  Segments: the readout pass starts from its prefix slot and
  // the state pass writes its increment to the slot.  Direct (one segment per pair): the piece starts
  // from the incoming state (null: empty history) and writes the final state (null: discarded), with
  // no state pass and no scan; in place is safe, each value being read and written by one lane.
  auto state_src = [&](const SeqPiece& pc) -> const float* {
    if (direct) return sin ? sin + pc.pair * stride : nullptr;
    return READOUT ? ws + pc.slot * stride : nullptr;
  };
  auto state_dst = [&](const SeqPiece& pc) -> float* {
    if (direct) return sout ? sout + pc.pair * stride : nullptr;
    return READOUT ? nullptr : ws + pc.slot * stride;
  };
  // The pieces of this workgroup.  Ragged batches in one pass: grid (sequence, head), the whole
  // sequence as one piece; an empty one only has its state carried over (by the consumer waves, with
  // no barrier, every value by one thread).
  // direct & 2 (ragged, at most kRankMax sequences): pairs are taken longest first — workgroup i in
  // launch order walks the (i / H)-th longest sequence (ties: lower index first) of head i % H, so the
  // last workgroups to start are the shortest and the CUs finish together.  Each workgroup ranks the
  // lengths itself (B comparisons per thread), so the host asks for it only where the walks are long.
  long long pb = bx, ph = by;
  if constexpr (PACKED) {
    if ((direct & 2) && seq.B <= kRankMax) {
      __shared__ int lens[kRankMax];
      __shared__ int pick;
      const long long lin = bx + by * (long long)gridDim.x;
      const int r = (int)(lin / seq.H);
      ph = lin - (long long)r * seq.H;
      if (tid < seq.B) {
        const long long c0 = seq.off(tid), c1 = seq.off(tid + 1);
        lens[tid] = c1 > c0 ? (int)(c1 - c0) : 0;
      }
      __syncthreads();
      if (tid < seq.B) {
        const int me = lens[tid];
        int rank = 0;
        for (int u = 0; u < seq.B; ++u) rank += (lens[u] > me) || (lens[u] == me && u < tid);
        if (rank == r) pick = tid;
      }
      __syncthreads();
      pb = pick;
    }
  }
  auto walk = [&](bool consumer, auto&& f) __attribute__((always_inline)) {
    if (PACKED && direct) {
      const SeqPiece pc = seq.whole_piece(pb, ph);
      if (pc.n > 0) {
        f(pc);
      } else if (consumer) {
        const float* src = state_src(pc);
        float* dst = state_dst(pc);
        if (dst)
          for (long long e = tid; e < stride; e += 64 * kPipeConsumers)
            dst[e] = (src && e < (long long)W * (kDV + 1)) ? src[e] : 0.f;
      }
    } else {
      for_each_piece<PACKED>(seq, bx, by, L, nslot, f);
    }
  };
  if (w >= kPipeConsumers) {
    walk(false, [&](const SeqPiece& pc) __attribute__((always_inline)) {
      pipe_producers<NT, READOUT, CENT>(sm, w, q, k, v, cf, state_src(pc), state_dst(pc),
                                        zc ? zc + seq.chunk_index(pc, 0, kPipeChunk) * W : nullptr, pc.tok, pc.n, l,
                                        scale);
    });
    return;
  }

  walk(true, [&](const SeqPiece& pc) __attribute__((always_inline)) {
    pipe_consumer<NT, READOUT, CENT>(sm, pc, state_src(pc), state_dst(pc), direct != 0, o, stride, w, tid);
  });
}

// ------------------------------------------------------------------------------------------------
// Single-pass prefill over segments (equal lengths, the truncated-kernel readout): the state pass,
// the scan and the readout pass of the split form in one launch, with a decoupled look-back between
// the segments of a (sequence, head) pair ("Expanding Attention", Abstract: the states add across
// chunks, so prefill admits a parallel scan).  Workgroup (x, pair) walks segment x:
//   1. its state sum over the segment, written to its slot and published at once with a flag
//      (segment 0 starts from the incoming state, so its sum is already the inclusive prefix);
//   2. the exclusive prefix: the flags of segments x-1, x-2, ... are read back until an inclusive one
//      is found, and the published sums from there on are added in segment order; the inclusive
//      prefix (exclusive + its own sum) is then published in turn, so later segments stop at this one;
//   3. the readout walk from the exclusive prefix (staged in LDS); the last segment writes the final
//      state at its end and needs no state sum of its own (nobody reads it).
// Flags, tags and the bounded waits are those of lookback.hpp.
// ------------------------------------------------------------------------------------------------

// The elements of a state block (S rows then z).
template <int NT>
struct StateSlice {
  static constexpr long long E = (long long)Geo<NT>::W * (kDV + 1);
};

template <int NT>
__global__ __launch_bounds__(kPipeThreads) void prefill_pipe_fused_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v, float* __restrict__ o,
    float* __restrict__ agg, float* __restrict__ incl, unsigned long long* flags, const float* sin, float* sout,
    int N, int L, long long stride, float scale, unsigned long long tag) {
  using SM1 = PipeSmem<NT, true>;
  using SM0 = PipeSmem<NT, false>;
  using SL = StateSlice<NT>;
  static_assert(sizeof(SM0) <= sizeof(SM1), "the state walk's LDS fits in the readout's");
  static_assert(SL::E * sizeof(float) <= sizeof(SM1::phiq), "the starting state fits where phi(sQ) goes");
  __shared__ SM1 sm;
  __shared__ unsigned long long seen;
  SM0& sm0 = *reinterpret_cast<SM0*>(&sm);
  float* pre = reinterpret_cast<float*>(&sm.phiq[0][0][0]);  // the segment's starting state, between phases
  // the segment's own sum, kept in LDS at the end of the state walk (where V^T and phi(K)^T were; only
  // the producers' z rows, further on, are still read then)
  float* own = reinterpret_cast<float*>(&sm);
  static_assert(SL::E * sizeof(float) <= offsetof(SM0, phiq), "the kept sum lies before the walk's z rows");

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int x = blockIdx.x, nseg = gridDim.x;
  const long long pair = blockIdx.y, slot = pair * nseg + x;
  const SeqPiece pc{pair * N + (long long)x * L, min(L, N - x * L), slot, pair};
  const bool last = x == nseg - 1;
  const float* sin_p = sin ? sin + pair * stride : nullptr;

  // 1. the segment's state sum (not needed from the last segment)
  if (!last) {
    const float* src = x == 0 ? sin_p : nullptr;
    float* dst = (x == 0 ? incl : agg) + slot * stride;
    if (w >= kPipeConsumers)
      pipe_producers<NT, false, false, true>(sm0, w, q, k, v, nullptr, src, dst, nullptr, pc.tok, pc.n, l, scale,
                                             own);
    else
      pipe_consumer<NT, false, false, true>(sm0, pc, src, dst, false, nullptr, stride, w, tid, own);
  }
  // The sum of a middle segment is published at once (segment 0's as its inclusive prefix), so later
  // segments need not wait for its look-back.  Publishing: the sums were stored through to the point of coherence (agent-scope
  // stores); every wave waits until its stores are acknowledged, then, after the barrier, one thread
  // stores the flag.  Readers load the flag and then the sums from the point of coherence too, so no
  // cache is written back or invalidated on either side.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // also: the state walk's last LDS reads (z rows for dst) are done before `pre` is written
  if (!last && tid == 0)  // segment 0's sum is already its inclusive prefix
    __hip_atomic_store(flags + slot, tag | (x == 0 ? kFlagIncl : kFlagAgg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // 2. the exclusive prefix into `pre`, and the inclusive one published
  lookback_prefix<SL::E, kPipeThreads>(pre, own, sin_p, agg, incl, flags, slot, x, last, stride, tag, seen, tid);

  // 3. the readout walk from `pre` (a generic pointer into LDS; every read of it precedes the walk's
  // first barrier, after which the pipeline reuses that LDS)
  float* dst = last && sout ? sout + pair * stride : nullptr;
  if (w >= kPipeConsumers)
    pipe_producers<NT, true, false>(sm, w, q, k, v, nullptr, pre, dst, nullptr, pc.tok, pc.n, l, scale);
  else
    pipe_consumer<NT, true, false>(sm, pc, pre, dst, dst != nullptr, o, stride, w, tid);
}

// Clears the flags of a call recorded into a graph (tag 0), before its single-pass kernel.
__global__ void clear_flags_kernel(unsigned long long* flags, long long n) {
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i < n) flags[i] = 0;
}

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }
long long round_up(long long x, long long m) { return (x + m - 1) / m * m; }

// Segments per pair: S <= ceil(target / BH) and <= nchunk, the one with the fewest rounds of `target`
// workgroups times chunks per segment (ceil(target / BH) itself can spill a second round: 100 pairs
// take two segments, not three).
int n_segments(int BH, int nchunk, int target) {
  long long hi = (target + BH - 1) / BH;
  if (hi > nchunk) hi = nchunk;
  int best = 1;
  long long cost = -1;
  for (int S = 1; S <= hi; ++S) {  // rounds of `target` workgroups x chunks per segment; ties: fewer
    const long long c = (((long long)BH * S + target - 1) / target) * ((nchunk + S - 1) / S);
    if (cost < 0 || c < cost) cost = c, best = S;
  }
  return best;
}

// One workgroup per CU (double-buffered LDS): about 256 workgroups in total.
constexpr int kSegTargetPipe = 256;

// Piece length and slots.  Equal lengths: about kSegTargetPipe workgroups, each pair cut into
// equal segments.  Ragged: ranges of the packed token axis of about total / kSegTargetPipe
// token-heads each (a multiple of the chunk).  Either may instead run in one pass per pair.
struct PipePlan {
  int L;            // piece (segment or range) length
  long long nslot;  // workspace slots per row
  bool direct;      // one segment per pair, read and written in one pass (no state pass, no scan)
  bool longest_first;  // ragged, one pass: the longest sequences first (ranked in the kernel)
};

// Equal lengths run in one pass (one segment per pair) when that is estimated faster than S segments:
// a chunk costs about kReadoutChunk in the readout pass and kStateChunk in the state pass (tenths of a
// microsecond), the split form's state pass, scan and two more launches add about kSplitFixed, and a
// form with more workgroups than CUs runs in rounds of one workgroup per CU.  One pass:
// rounds(BH) * nchunk * kReadoutChunk; segments: rounds(BH * S) * ceil(nchunk / S) * (kStateChunk +
// kReadoutChunk) + kSplitFixed.  The figures are fits to both forms timed at n = 3, bfloat16, 64 to
// 256 pairs, N = 128 to 8192.
constexpr int kReadoutChunk = 23, kStateChunk = 11, kSplitFixed = 150;
bool one_pass_faster(int BH, int nchunk, int segs) {
  const long long one = (long long)cdiv(BH, kSegTargetPipe) * nchunk * kReadoutChunk;
  const long long split = (long long)cdiv((long long)BH * segs, kSegTargetPipe) * cdiv(nchunk, segs) *
                              (kStateChunk + kReadoutChunk) + kSplitFixed;
  return one < split;
}

PipePlan pipe_plan(int BH, const SeqMap& seq, bool direct_ok) {
  PipePlan p;
  p.direct = p.longest_first = false;
  if (seq.packed) {
    // floor(target / H) ranges per head at most, so ranges x heads never spill a second round
    const long long ranges = std::max<long long>(1, kSegTargetPipe / std::max(1, seq.H));
    const long long per = std::max<long long>(1, (seq.T + ranges - 1) / ranges);
    p.L = (int)std::min<long long>((per + kPipeChunk - 1) / kPipeChunk * kPipeChunk, 1 << 30);
    // One pass per (sequence, head) pair against the balanced ranges: chunks per CU (half a chunk of
    // ragged tail per sequence) for both, plus, for pairs dealt to CUs in launch order, about half the
    // longest pair's walk as the tail of the last CU to finish.
    const long long nch_max = cdiv(seq.N, kPipeChunk);
    const long long per_cu = cdiv((seq.T + 32LL * seq.B) / kPipeChunk * seq.H, kSegTargetPipe);
    p.direct = direct_ok && kReadoutChunk * std::max(nch_max, per_cu + nch_max / 2) <
                                (kStateChunk + kReadoutChunk) * per_cu + kSplitFixed;
    p.longest_first = p.direct && seq.B <= kRankMax && seq.B <= 16 * nch_max;
  } else {
    const int nchunk = cdiv(seq.N, kPipeChunk);
    const int segs = n_segments(BH, nchunk, kSegTargetPipe);
    p.direct = direct_ok && one_pass_faster(BH, nchunk, segs);
    p.L = (p.direct ? nchunk : cdiv(nchunk, segs)) * kPipeChunk;
  }
  p.nslot = seq.row_slots(p.L);
  return p;
}

// The kernel for a call (the expanded-softmax readout exists for n = 2, 3; its state pass also writes
// the per-chunk z rows).
template <int NT, bool READOUT>
auto pipe_kernel_for(bool packed, bool cent) {
  if constexpr (NT == 2 || NT == 3) {
    if (cent) return packed ? prefill_pipe_kernel<NT, READOUT, true, true> : prefill_pipe_kernel<NT, READOUT, false, true>;
  }
  return packed ? prefill_pipe_kernel<NT, READOUT, true, false> : prefill_pipe_kernel<NT, READOUT, false, false>;
}

// The single-pass form applies to equal lengths split into segments, with the truncated-kernel
// readout, where the whole grid is one round of one workgroup per CU.
bool fused_form(const PipePlan& p, const SeqMap& seq, int BH, int readout) {
  const long long nseg = seq.grid_x(p.L);
  return !p.direct && !seq.packed && readout != 1 && nseg > 1 && nseg * BH <= kFusedMaxGrid;
}

template <int NT>
int run_pipe(const PrefillArgs& a) {
  const PipePlan p = pipe_plan(a.BH, a.seq, a.s.readout != 1);
  const bool cent = a.s.readout == 1 && a.o;
  float* ws = (float*)a.ws;
  // workspace: slots | coefficients (4 per token-head) | z before each chunk (W per chunk)
  float* coef = ws + round_up(a.seq.rows(a.BH) * p.nslot * a.s.stride, 64);
  float* zc = coef + round_up(4 * a.seq.tokens(a.BH), 64);
  const long long elems = Geo<NT>::W * (long long)(kDV + 1);
  const dim3 grid((unsigned)(p.direct && a.seq.packed ? a.seq.B : a.seq.grid_x(p.L)), (unsigned)a.seq.grid_y(a.BH)),
      block(kPipeThreads);
  const __bf16* q = (const __bf16*)a.q;
  const __bf16* k = (const __bf16*)a.k;
  const __bf16* v = (const __bf16*)a.v;
  if (p.direct) {
    // one pass: the readout (or, for a state-only call, the state walk) from the incoming state to the
    // final one; a state-only call that discards the state has nothing to do
    if (!a.o && !a.state) return 0;
    if (a.o)
      pipe_kernel_for<NT, true>(a.seq.packed, false)<<<grid, block, 0, a.stream>>>(
          q, k, v, nullptr, a.o, ws, nullptr, a.state_in, a.state, p.longest_first ? 3 : 1, a.seq, p.L, p.nslot,
          a.s.stride, a.s.scale);
    else
      pipe_kernel_for<NT, false>(a.seq.packed, false)<<<grid, block, 0, a.stream>>>(
          q, k, v, nullptr, nullptr, ws, nullptr, a.state_in, a.state, p.longest_first ? 3 : 1, a.seq, p.L,
          p.nslot, a.s.stride, a.s.scale);
    return hipGetLastError() == hipSuccess ? 0 : -3;
  }
  if (a.o && fused_form(p, a.seq, a.BH, a.s.readout)) {
    // single pass: state sums, look-back and readout in one launch (slots: sums | inclusive | flags)
    const long long slots = (long long)grid.x * grid.y;
    float* incl = ws + round_up(slots * a.s.stride, 64);
    unsigned long long* flags = reinterpret_cast<unsigned long long*>(incl + round_up(slots * a.s.stride, 64));
    unsigned long long tag = 0;
    if (stream_recording(a.stream)) {
      clear_flags_kernel<<<dim3((unsigned)cdiv(slots, 256)), dim3(256), 0, a.stream>>>(flags, slots);
      if (hipGetLastError() != hipSuccess) return -3;
    } else {
      tag = lookback_tag();
    }
    prefill_pipe_fused_kernel<NT><<<grid, block, 0, a.stream>>>(q, k, v, a.o, ws, incl, flags, a.state_in, a.state,
                                                                 a.seq.N, p.L, a.s.stride, a.s.scale, tag);
    return hipGetLastError() == hipSuccess ? 0 : -3;
  }
  pipe_kernel_for<NT, false>(a.seq.packed, cent)<<<grid, block, 0, a.stream>>>(
      q, k, v, nullptr, nullptr, ws, cent ? zc : nullptr, nullptr, nullptr, 0, a.seq, p.L, p.nslot, a.s.stride,
      a.s.scale);
  if (hipGetLastError() != hipSuccess) return -3;
  if (seg_scan_launch(ws, a.state_in, a.state, a.BH, p.nslot, a.s.stride, elems, a.o != nullptr, a.seq, p.L,
                      a.stream))
    return -3;
  if (a.o) {
    if (cent) {
      // per-token coefficients from the prefixes the readout starts from
      const CenteredPlan cp{p.L, p.nslot, ws, 1, zc, kPipeChunk, reinterpret_cast<float4*>(coef)};
      if (const int rc = centered_coef_launch(a, cp)) return rc;
    }
    pipe_kernel_for<NT, true>(a.seq.packed, cent)<<<grid, block, 0, a.stream>>>(
        q, k, v, cent ? coef : nullptr, a.o, ws, nullptr, nullptr, nullptr, 0, a.seq, p.L, p.nslot, a.s.stride,
        a.s.scale);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

}  // namespace

// Tags of the single-pass kernels (lookback.hpp): one process-wide counter, started at a time-derived
// value.
unsigned long long lookback_tag() {
  static std::atomic<unsigned long long> counter{
      (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9e3779b97f4a7c15ull};
  unsigned long long t = counter.fetch_add(1, std::memory_order_relaxed) & ((1ull << 62) - 1);
  return (t ? t : 1) << 2;
}

// bfloat16 inputs at d_k = 16, d_v = 64, n = 1..3.  The kernel walks 64-token chunks whatever the
// configured chunk (64 or 128); the outputs do not depend on the chunk length beyond rounding.
bool prefill_mfma_has(int nt, int dk, int dv, int dtype) { return dk == kDK && dv == kDV && nt >= 1 && nt <= 3 && dtype == 1; }

long long prefill_mfma_ws_bytes(const Shape& s, int BH, const SeqMap& seq) {
  const PipePlan p = pipe_plan(BH, seq, s.readout != 1);
  const long long slots = round_up(seq.rows(BH) * p.nslot * s.stride, 64);
  if (fused_form(p, seq, BH, s.readout)) return (2 * slots + seq.rows(BH) * p.nslot * 2) * 4;  // + 8-byte flags
  if (s.readout != 1) return slots * 4;
  return (slots + round_up(4 * seq.tokens(BH), 64) + seq.chunk_count(BH, kPipeChunk) * s.W) * 4;
}

int prefill_mfma_launch(const PrefillArgs& a) {
  if (!prefill_mfma_has(a.s.nt, a.s.dk, a.s.dv, a.s.dtype)) return -2;
  switch (a.s.nt) {
    case 1: return run_pipe<1>(a);
    case 2: return run_pipe<2>(a);
    default: return run_pipe<3>(a);
  }
}

}  // namespace taylor
