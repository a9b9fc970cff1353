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
// over (segment, head, block of FB features; FB = 64 at n = 4, 160 at n = 5), one workgroup of 8
// wavefronts each:
//   * waves 0..3 ("consumers") own value columns 16w..16w+15 of the block's state slice, kept in MFMA
//     accumulator registers, and run only float32 16x16x4 MFMAs on chunk c: the readout with S_{<c}, the
//     intra-chunk PV (the last block, whose padding tiles past W are skipped), the state update;
//   * waves 4..7 ("producers") meanwhile prepare chunk c+1 in the other half of a double-buffered LDS
//     area: producer g expands features g*FB/4 .. of the block for the chunk's 32 tokens (lanes 0..31
//     from k into phi(K)^T, lanes 32..63 from sq into phi(sQ), the same compile-time code on both
//     halves), writes its V^T columns, its part of the denominators phi_f(sq) . z_{f,<c} and updates the
//     block's z rows it owns; for the last block producers 0..2 also build the three intra-chunk score tiles and
//     their column sums.  Their inputs are global loads issued a chunk ahead, in two alternating register
//     sets;
//   * one barrier per chunk; each block writes partial numerators and denominators per token to a
//     workspace and a reduction kernel sums the blocks in order and divides.
// Segments, when (head, block) pairs alone do not fill the chip: a state pass writes each segment's
// increment, the scan turns them into exclusive prefixes and the readout pass starts from them.  With
// one segment the readout pass starts from the incoming state and writes the final state itself.
// bfloat16 inputs are widened to float32 on load; all matrix work and accumulation is float32.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "centered.hpp"
#include "features.hpp"
#include "prefill_wide.hpp"

namespace taylor {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDK = 16, kDV = 64;
constexpr int kCS = kWideChunk;  // tokens per chunk
constexpr int kProd = 4;         // producer waves, FB / 4 features each
constexpr int kCons = 4;         // consumer waves, 16 value columns each
constexpr int kThreads = 64 * (kProd + kCons);
constexpr int kNIT = kCS / 16;   // 16-token tiles of a chunk
constexpr int kPairs = kNIT * (kNIT + 1) / 2;  // (key tile <= query tile) pairs
constexpr int kLS = kCS + 4;     // phi(K)^T and V^T row stride in floats (36: conflict-free 16-byte reads)
static_assert(kPairs <= kProd, "one score tile per producer");

// Features per block: one block holds all features at n <= 3 (16, 32, 160 for W = 1, 17, 153: the
// outputs are then final and written directly); 64 at n = 4 (16 blocks: enough (head, block)
// workgroups at few heads without a state pass); 160 at n = 5 (31 blocks: 16 heads make 496
// workgroups, two rounds of one per CU, where 128-feature blocks made 608, three rounds; 20% less
// partial-output traffic too).
template <int NT>
constexpr int block_features() {
  return NT == 1 ? 16 : NT == 2 ? 32 : NT == 3 ? 160 : NT == 4 ? 64 : 160;
}
template <int NT>
constexpr int n_blocks() {
  return (FeatureTable<NT, kDK>::W + block_features<NT>() - 1) / block_features<NT>();
}
// The block that also carries the intra-chunk term (score tiles, their PV and column sums): the last
// one, whose features past W are padding (9 of 64 real at n = 4, 45 of 160 at n = 5), so that its
// consumers run only the 16-feature tiles holding real features and the extra term lands on the
// lightest block instead of adding to a full one.
template <int NT>
constexpr int intra_block() {
  return n_blocks<NT>() - 1;
}
// 16-feature tiles of the last block that hold real features (all of them at n <= 3: one block).
template <int NT>
constexpr int last_block_tiles() {
  return (FeatureTable<NT, kDK>::W - intra_block<NT>() * block_features<NT>() + 15) / 16;
}

constexpr int pair_it(int p) {
  int it = 0;
  while ((it + 1) * (it + 2) / 2 <= p) ++it;
  return it;
}
constexpr int pair_jt(int p) { return p - pair_it(p) * (pair_it(p) + 1) / 2; }

template <bool READOUT, int FB>
struct WideSmem {
  static constexpr int RQ = READOUT ? kCS : 1;
  static constexpr int RP = READOUT ? kPairs : 1;
  static constexpr int LQ = FB + 4;      // phi(sQ) row stride in floats (4 mod 64 banks)
  alignas(16) float phikt[2][FB][kLS];   // phi_f(k_j), feature-major
  alignas(16) float vt[2][kDV][kLS];     // V^T
  alignas(16) float phiq[2][RQ][LQ];     // phi_f(s q_i), token-major
  alignas(16) f32x4 a[2][RP][64];        // block 0: score tiles in MFMA B-operand lane order
  alignas(16) float z[FB];               // the block's z_{<c}; producer g owns rows g*FB/4 .. + FB/4
  float den_part[2][kProd][RQ];          // phi_f(s q_i) . z_{f,<c} over each producer's features
  float den_intra[2][RP][16];            // column sums of the score tiles
};

// Where a workgroup's starting state comes from and where its results go (see the file comment).
struct WideIO {
  float* slots;        // several segments per pair: workspace slots (placed as SeqMap describes) of
                       // prefixes (readout) or increments (state pass)
  float* state;        // one segment per pair: the final state [pairs][stride], or null
  const float* state_in;  // one segment per pair: the incoming state, or null (may equal state)
  float* part_num;     // [blocks][token-heads][d_v] partial numerators
  float* part_den;     // [blocks][token-heads] partial denominators
  float* out;          // a single block: the outputs [token-heads][d_v]
  long long stride;
  long long nslot;     // slots per workspace row
  long long tokens;    // token-heads of the call
  int multi;           // several segments per pair (grid x > 1)
  const float* coef;   // expanded-softmax readout: [token-heads] (gamma_0, gamma_1, gamma_2, 0), else null
  float* zc;           // its state pass: z of the piece before each 64 tokens (SeqMap::chunk_index)
};

// n consecutive elements (n a multiple of 4) of one token row, widened to float32 on unpack.
template <typename E, int NE>
struct Piece;
template <int NE>
struct Piece<float, NE> {
  f32x4 p[NE / 4];
  __device__ __forceinline__ void load(const float* src) {
#pragma unroll
    for (int u = 0; u < NE / 4; ++u) p[u] = *reinterpret_cast<const f32x4*>(src + 4 * u);
  }
  __device__ __forceinline__ float get(int i) const { return p[i / 4][i % 4]; }
};
template <int NE>
struct Piece<__bf16, NE> {
  uint32_t p[NE / 2];
  __device__ __forceinline__ void load(const __bf16* src) {
    if constexpr (NE % 8 == 0) {
#pragma unroll
      for (int u = 0; u < NE / 8; ++u) {
        const uint4 t = *reinterpret_cast<const uint4*>(src + 8 * u);
        p[4 * u] = t.x;
        p[4 * u + 1] = t.y;
        p[4 * u + 2] = t.z;
        p[4 * u + 3] = t.w;
      }
    } else {
      const uint2 t = *reinterpret_cast<const uint2*>(src);
      p[0] = t.x;
      p[1] = t.y;
    }
  }
  __device__ __forceinline__ float get(int i) const {
    return __uint_as_float(i % 2 == 0 ? p[i / 2] << 16 : p[i / 2] & 0xffff0000u);
  }
};

// One producer lane's inputs for one chunk: a k row (lanes 0..31) or a q row (lanes 32..63) of token
// l % 32, the lane's 8 values of that token, and its score-tile operands (used by block 0 only).  For
// the expanded-softmax readout (CENT) also the coefficients of the lane's token and of its score
// column's query token.
template <typename E, bool CENT>
struct WideIn {
  Piece<E, kDK> row;
  Piece<E, 8> v;
  Piece<E, 4> sk, sq;
  f32x4 cq, csq;
  __device__ __forceinline__ void load(const E* qg, const E* kg, const E* vg, const float* cf, long long tok0, int nv,
                                       int l, int g, bool readout) {
    const int tk = l & 31, h = l >> 5;
    const long long r = tok0 + (tk < nv ? tk : 0);  // tokens past the end read a valid row, masked later
    row.load((readout && h ? qg : kg) + r * kDK);
    v.load(vg + r * kDV + 16 * g + 8 * h);
    if (readout) {
      const int p = g < kPairs ? g : 0;
      const int l16 = l & 15, lg = l >> 4;
      const int rk = 16 * pair_jt(p) + l16, rq = 16 * pair_it(p) + l16;
      sk.load(kg + (tok0 + (rk < nv ? rk : 0)) * kDK + 4 * lg);
      sq.load(qg + (tok0 + (rq < nv ? rq : 0)) * kDK + 4 * lg);
      if constexpr (CENT) {
        cq = *reinterpret_cast<const f32x4*>(cf + 4 * r);
        csq = *reinterpret_cast<const f32x4*>(cf + 4 * (tok0 + (rq < nv ? rq : 0)));
      }
    }
  }
};

// Order of feature A (0 for the padding rows past the table, whose features are zero).
template <int NT, int A>
constexpr int feature_order() {
  if constexpr (A < FeatureTable<NT, kDK>::W)
    return FeatureTable<NT, kDK>::T.order[A];
  else
    return 0;
}

// Producer g's features of its FP = FB / 4 block rows for one token: lanes 0..31 from k into
// phi(K)^T, lanes 32..63 from sq into phi(sQ) (plus their part of the denominators; CENT: each scaled
// by its order's coefficient gamma_m of the token, and no denominator).  F0 = first global feature.
template <int NT, bool READOUT, bool CENT, int FB, int F0>
__device__ __forceinline__ void expand_rows(WideSmem<READOUT, FB>& sm, int b, int g, int l, const float (&x)[kDK],
                                            bool valid, const f32x4& cq) {
  constexpr int FP = FB / kProd;
  constexpr int L0 = F0 % FB;  // first block row of this producer
  const int tk = l & 31;
  float f[FP];
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((f[I] = feature_ct<NT, kDK, F0 + I>(x)), ...);
  }(std::make_integer_sequence<int, FP>{});
  if (l < 32) {
    if constexpr (F0 == 0) f[0] = valid ? 1.f : 0.f;  // the constant feature of a token past the end
#pragma unroll
    for (int i = 0; i < FP; ++i) sm.phikt[b][L0 + i][tk] = f[i];
  } else if constexpr (READOUT && CENT) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((f[I] *= cq[feature_order<NT, F0 + I>()]), ...);
    }(std::make_integer_sequence<int, FP>{});
#pragma unroll
    for (int u = 0; u < FP / 4; ++u)
      *reinterpret_cast<f32x4*>(&sm.phiq[b][tk][L0 + 4 * u]) = f32x4{f[4 * u], f[4 * u + 1], f[4 * u + 2], f[4 * u + 3]};
  } else if constexpr (READOUT) {
    float den = 0.f;
#pragma unroll
    for (int u = 0; u < FP / 4; ++u) {
      *reinterpret_cast<f32x4*>(&sm.phiq[b][tk][L0 + 4 * u]) = f32x4{f[4 * u], f[4 * u + 1], f[4 * u + 2], f[4 * u + 3]};
      const f32x4 zz = *reinterpret_cast<const f32x4*>(&sm.z[L0 + 4 * u]);
      den = fmaf(f[4 * u], zz[0], den);
      den = fmaf(f[4 * u + 1], zz[1], den);
      den = fmaf(f[4 * u + 2], zz[2], den);
      den = fmaf(f[4 * u + 3], zz[3], den);
    }
    sm.den_part[b][g][tk] = den;
  }
}

// Producer g prepares the chunk in buffer b from its inputs.
template <int NT, typename E, bool READOUT, bool CENT, bool OPAQUE>
__device__ __forceinline__ void wide_produce(WideSmem<READOUT, block_features<NT>()>& sm, const WideIn<E, CENT>& in,
                                             int b, int fb, int g, int l, int nv, float scale, float* zrow) {
  constexpr int NB = n_blocks<NT>(), FB = block_features<NT>(), FP = FB / kProd;
  const int tk = l & 31, h = l >> 5, l16 = l & 15, lg = l >> 4;
  const bool valid = tk < nv;
  if constexpr (!READOUT && CENT) {
    // state pass before an expanded-softmax readout (one block): z of the piece before this chunk,
    // at every other chunk (the coefficient kernel works on 64 tokens)
    const int row = FP * g + l;
    if (zrow && l < FP && row < FeatureTable<NT, kDK>::W) zrow[row] = sm.z[row];
  }
  {
    float x[kDK];
    // k rows of tokens past the end are zero (their features vanish except the constant one)
    const float sx = (READOUT && h) ? scale : (valid ? 1.0f : 0.0f);
#pragma unroll
    for (int d = 0; d < kDK; ++d) x[d] = sx * in.row.get(d);
    // OPAQUE: the slot is opaque to the optimiser here: otherwise the comparisons of the dispatch
    // tree are hoisted out of the chunk loop, and their results occupy scalar registers that spill
    // (for the ragged kernels, whose piece loop surrounds the chunk loop, hoisting them costs less)
    int slot = fb * kProd + g;
    if constexpr (OPAQUE) asm volatile("" : "+s"(slot));
    dispatch_index<0, NB * kProd>(slot, [&](auto I) {
      expand_rows<NT, READOUT, CENT, FB, decltype(I)::value * FP>(sm, b, g, l, x, valid, in.cq);
    });
  }
  // V^T: columns 16g + 8h .. + 7 of token tk
#pragma unroll
  for (int c = 0; c < 8; ++c) sm.vt[b][16 * g + 8 * h + c][tk] = valid ? in.v.get(c) : 0.f;
  if constexpr (READOUT) {
    if (fb == intra_block<NT>() && g < kPairs) {
      // score tile of pair g and its column sums (16 keys per query column)
      const int it = pair_it(g), jt = pair_jt(g);
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) sc = __builtin_amdgcn_mfma_f32_16x16x4f32(in.sk.get(r), in.sq.get(r), sc, 0, 0, 0);
      // sc[r] = k_j . q_i with j = 16jt + 4lg + r, i = 16it + l16
      f32x4 wt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jt + 4 * lg + r, i = 16 * it + l16;
        const float s = scale * sc[r];
        // CENT: gamma_0 + gamma_1 s + gamma_2 s^2 / 2 of query i (gamma_2 = 0 at order 1)
        const float poly = CENT ? fmaf(s, fmaf(0.5f * s, in.csq[2], in.csq[1]), in.csq[0]) : taylor_kernel<NT>(s);
        wt[r] = (jt < it || j <= i) ? poly : 0.f;
      }
      sm.a[b][g][l] = wt;
      if constexpr (!CENT) {
        f32x4 cs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) cs = __builtin_amdgcn_mfma_f32_16x16x4f32(1.0f, wt[r], cs, 0, 0, 0);
        if (lg == 0) sm.den_intra[b][g][l16] = cs[0];
      }
    }
  }
  // z_{<next} = z + row sums of this producer's phi(K)^T rows (written by this wave above; a wave's
  // LDS accesses complete in order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (l < FP) {
    const int row = FP * g + l;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kCS; j += 4) {
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sm.phikt[b][row][j]);
      acc += (x4[0] + x4[1]) + (x4[2] + x4[3]);
    }
    sm.z[row] += acc;
  }
}

// Where a piece's block starts from (init: its prefix, or the incoming state when a pair is one
// piece; null: zero) and where its state goes (the piece's increment in the state pass; the final
// state when a pair is one piece; null: nowhere).
template <bool READOUT>
__device__ __forceinline__ void piece_state(const WideIO& io, const SeqPiece& pc, const float*& init, float*& dst) {
  init = nullptr;
  dst = nullptr;
  if (io.multi) {
    if (READOUT) init = io.slots + pc.slot * io.stride;
  } else if (READOUT && io.state_in) {
    init = io.state_in + pc.pair * io.stride;
  }
  if (!READOUT)
    dst = io.slots + pc.slot * io.stride;
  else if (!io.multi && io.state)
    dst = io.state + pc.pair * io.stride;
}

// Producer wave g's walk over one piece of block fb: z starts from init (null: zero) and ends in dst
// (null: not written).  Executes exactly 2 + nch barriers, like the consumers.
template <int NT, typename E, bool READOUT, bool CENT, bool OPAQUE>
__device__ __forceinline__ void wide_producer_piece(WideSmem<READOUT, block_features<NT>()>& sm, const WideIO& io,
                                                    const SeqMap& seq, const SeqPiece& pc, const float* init,
                                                    float* dst, const E* q, const E* k, const E* v, int fb, int g,
                                                    int l, float scale) {
  constexpr int W = FeatureTable<NT, kDK>::W;
  constexpr int FB = block_features<NT>(), FP = FB / kProd;
  const int f0 = fb * FB;
  const int nch = (pc.n + kCS - 1) / kCS;
  auto nv_of = [&](int c) { return min(kCS, pc.n - c * kCS); };
  auto tok_of = [&](int c) { return pc.tok + (long long)c * kCS; };
  auto zrow = [&](int c) {
    return CENT && !READOUT && c % 2 == 0
               ? io.zc + (seq.chunk_index(pc, 0, 2 * kCS) + c / 2) * FeatureTable<NT, kDK>::W
               : nullptr;
  };
  if (l < FP) {
    const int a = f0 + FP * g + l;
    sm.z[FP * g + l] = (init && a < W) ? init[(long long)W * kDV + a] : 0.f;
  }
  WideIn<E, CENT> pa, pb;
  pa.load(q, k, v, io.coef, tok_of(0), nv_of(0), l, g, READOUT);
  __syncthreads();
  if (nch > 1) pb.load(q, k, v, io.coef, tok_of(1), nv_of(1), l, g, READOUT);
  wide_produce<NT, E, READOUT, CENT, OPAQUE>(sm, pa, 0, fb, g, l, nv_of(0), scale, zrow(0));
  __syncthreads();  // chunk 0 ready
  int c = 0;
  for (; c + 3 < nch; c += 2) {
    pa.load(q, k, v, io.coef, tok_of(c + 2), nv_of(c + 2), l, g, READOUT);
    wide_produce<NT, E, READOUT, CENT, OPAQUE>(sm, pb, (c + 1) & 1, fb, g, l, nv_of(c + 1), scale, zrow(c + 1));
    __syncthreads();
    pb.load(q, k, v, io.coef, tok_of(c + 3), nv_of(c + 3), l, g, READOUT);
    wide_produce<NT, E, READOUT, CENT, OPAQUE>(sm, pa, c & 1, fb, g, l, nv_of(c + 2), scale, zrow(c + 2));
    __syncthreads();
  }
  // nch - c phases remain (1 to 3); chunks c+1 and c+2 may still need preparing
  if (c + 2 < nch) pa.load(q, k, v, io.coef, tok_of(c + 2), nv_of(c + 2), l, g, READOUT);
  if (c + 1 < nch) wide_produce<NT, E, READOUT, CENT, OPAQUE>(sm, pb, (c + 1) & 1, fb, g, l, nv_of(c + 1), scale, zrow(c + 1));
  __syncthreads();
  if (c + 1 < nch) {
    if (c + 2 < nch) wide_produce<NT, E, READOUT, CENT, OPAQUE>(sm, pa, c & 1, fb, g, l, nv_of(c + 2), scale, zrow(c + 2));
    __syncthreads();
    if (c + 2 < nch) __syncthreads();
  }
  if (dst && l < FP) {
    const int a = f0 + FP * g + l;
    if (a < W) dst[(long long)W * kDV + a] = sm.z[FP * g + l];
  }
  // the padding after S and z: zero, whatever the array held before
  if (dst && fb == 0 && g == 0 && l < io.stride - (long long)W * (kDV + 1)) dst[(long long)W * (kDV + 1) + l] = 0.f;
}

// Consumer wave w's walk over one piece of block fb (value columns 16w..16w+15): the running state
// starts from init and ends in dst as for the producers; the outputs (READOUT) go to io.out (one
// block) or to the block's partial numerators and denominators.
template <int NT, typename E, bool READOUT, bool CENT>
__device__ __forceinline__ void wide_consumer_piece(WideSmem<READOUT, block_features<NT>()>& sm, const WideIO& io,
                                                    const SeqPiece& pc, const float* init, float* dst, int fb,
                                                    int w, int tid) {
  constexpr int W = FeatureTable<NT, kDK>::W;
  constexpr int FB = block_features<NT>(), NAT = FB / 16;
  const int l = tid & 63, l16 = l & 15, lg = l >> 4;
  const int f0 = fb * FB;
  const int nch = (pc.n + kCS - 1) / kCS;
  auto nv_of = [&](int c) { return min(kCS, pc.n - c * kCS); };
  auto tok_of = [&](int c) { return pc.tok + (long long)c * kCS; };

  // ---- consumers: wave w owns value columns 16w..16w+15 ----
  const int col = 16 * w + l16;
  const bool intra = READOUT && fb == intra_block<NT>();  // the last block also carries the intra-chunk term
  // the last block's tiles past W hold zero features and a zero state: it runs only the others
  constexpr int NLAST = last_block_tiles<NT>();
  const bool short_block = NLAST < NAT && fb == intra_block<NT>();
  f32x4 Srun[NAT];
#pragma unroll
  for (int t = 0; t < NAT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = f0 + 16 * t + 4 * lg + r;
      Srun[t][r] = (init && a < W) ? init[(long long)a * kDV + col] : 0.f;
    }
  __syncthreads();
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int b = c & 1;
    const int nv = nv_of(c);
    const long long tok0 = tok_of(c);
    f32x4 O[READOUT ? kNIT : 1];
    // the chunk's matrix work over the first NTL feature tiles of the block
    auto chunk_mfma = [&](auto ntl) __attribute__((always_inline)) {
      constexpr int NTL = decltype(ntl)::value;
      if constexpr (READOUT) {
#pragma unroll
        for (int it = 0; it < kNIT; ++it) O[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        // readout: O[it][r] = (phi_f(sQ) S_{f,<c})[token 16it + l16][column 16w + 4lg + r]
#pragma unroll
        for (int t = 0; t < NTL; ++t)
#pragma unroll
          for (int it = 0; it < kNIT; ++it) {
            const f32x4 bq = *reinterpret_cast<const f32x4*>(&sm.phiq[b][16 * it + l16][16 * t + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) O[it] = __builtin_amdgcn_mfma_f32_16x16x4f32(Srun[t][r], bq[r], O[it], 0, 0, 0);
          }
        if (intra) {
#pragma unroll
          for (int it = 0; it < kNIT; ++it)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) {
              const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.vt[b][col][16 * jt + 4 * lg]);
              const f32x4 bw = sm.a[b][it * (it + 1) / 2 + jt][l];
#pragma unroll
              for (int r = 0; r < 4; ++r) O[it] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r], bw[r], O[it], 0, 0, 0);
            }
        }
      }
      // state update: Srun[t] += phi_f(K)^T[16t.., chunk] V[chunk, columns]
#pragma unroll
      for (int jb = 0; jb < kCS / 16; ++jb) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(&sm.vt[b][col][16 * jb + 4 * lg]);
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
          const f32x4 ak = *reinterpret_cast<const f32x4*>(&sm.phikt[b][16 * t + l16][16 * jb + 4 * lg]);
#pragma unroll
          for (int r = 0; r < 4; ++r) Srun[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[r], bv[r], Srun[t], 0, 0, 0);
        }
      }
    };
    if (short_block)
      chunk_mfma(std::integral_constant<int, NLAST>{});
    else
      chunk_mfma(std::integral_constant<int, NAT>{});
    if constexpr (READOUT && n_blocks<NT>() == 1) {
      // a single block: the outputs are final (columns 16w + 4lg .. + 3 of token 16it + l16); the
      // expanded-softmax readout has no normaliser (its weights already sum to one)
#pragma unroll
      for (int it = 0; it < kNIT; ++it) {
        const int i = 16 * it + l16;
        float d = 1.f;
        if constexpr (!CENT) {
          d = 0.f;
#pragma unroll
          for (int p = 0; p < kProd; ++p) d += sm.den_part[b][p][i];
          for (int jt = 0; jt <= it; ++jt) d += sm.den_intra[b][it * (it + 1) / 2 + jt][l16];
        }
        if (i < nv) {
          const float inv = CENT ? 1.0f : 1.0f / d;
          const f32x4 r = O[it];
          *reinterpret_cast<f32x4*>(io.out + (tok0 + i) * kDV + 16 * w + 4 * lg) =
              f32x4{r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv};
        }
      }
    } else if constexpr (READOUT) {
      // partial numerators of this block (columns 16w + 4lg .. + 3 of token 16it + l16)
      float* pn = io.part_num + ((long long)fb * io.tokens + tok0) * kDV;
#pragma unroll
      for (int it = 0; it < kNIT; ++it) {
        const int i = 16 * it + l16;
        if (i < nv) *reinterpret_cast<f32x4*>(pn + (long long)i * kDV + 16 * w + 4 * lg) = O[it];
      }
      // partial denominators: consumer w < kNIT writes tokens 16w .. 16w + 15
      if (w < kNIT && lg == 0) {
        const int i = 16 * w + l16;
        float d = 0.f;
#pragma unroll
        for (int p = 0; p < kProd; ++p) d += sm.den_part[b][p][i];
        if (intra)
          for (int jt = 0; jt <= w; ++jt) d += sm.den_intra[b][w * (w + 1) / 2 + jt][l16];
        if (i < nv) io.part_den[(long long)fb * io.tokens + tok0 + i] = d;
      }
    }
    __syncthreads();
  }

  if (dst) {
#pragma unroll
    for (int t = 0; t < NAT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = f0 + 16 * t + 4 * lg + r;
        if (a < W) dst[(long long)a * kDV + col] = Srun[t][r];
      }
  }
}

// The pieces of one workgroup (see SeqMap: a segment of one pair, or the pieces of one token
// range of one head), one feature block; grid = (segments or ranges, pairs or heads, blocks).
template <int NT, typename E, bool READOUT, bool PACKED, bool CENT>
__global__ __launch_bounds__(kThreads) void prefill_wide_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                                const E* __restrict__ v, WideIO io, SeqMap seq,
                                                                int L, float scale) {
  __shared__ WideSmem<READOUT, block_features<NT>()> sm;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fb = blockIdx.z;
  const long long bx = blockIdx.x, by = blockIdx.y;
  // Both roles walk the same pieces and execute exactly 2 + nch barriers per piece.  Pieces follow
  // one another in LDS without an extra barrier: a piece's last barrier orders every read of its
  // buffers before the next piece's first writes, and each producer rewrites only its own z rows
  // at a piece's start.
  for_each_piece<PACKED>(seq, bx, by, L, io.nslot, [&](const SeqPiece& pc) __attribute__((always_inline)) {
    const float* init;
    float* dst;
    piece_state<READOUT>(io, pc, init, dst);
    if (w >= kCons)
      wide_producer_piece<NT, E, READOUT, CENT, !PACKED>(sm, io, seq, pc, init, dst, q, k, v, fb, w - kCons, l, scale);
    else
      wide_consumer_piece<NT, E, READOUT, CENT>(sm, io, pc, init, dst, fb, w, tid);
  });
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
  // eight blocks at a time: their loads are in flight together; the sums stay in block order
  constexpr int kBatch = 8;
  int b = 0;
  for (; b + kBatch <= nb; b += kBatch) {
    f32x4 x[kBatch];
    float y[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      x[u] = *reinterpret_cast<const f32x4*>(num + ((long long)(b + u) * tokens + tok) * kDV + 4 * g);
      y[u] = den[(long long)(b + u) * tokens + tok];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      acc = acc + x[u];
      d += y[u];
    }
  }
  for (; b < nb; ++b) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(num + ((long long)b * tokens + tok) * kDV + 4 * g);
    acc = acc + x;
    d += den[(long long)b * tokens + tok];
  }
  *reinterpret_cast<f32x4*>(o + tok * kDV + 4 * g) = f32x4{acc[0] / d, acc[1] / d, acc[2] / d, acc[3] / d};
}

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Workgroups to aim for: with outputs about one per CU (the readout kernel's LDS allows one), for a
// state-only pass four per CU.
long long wide_target(bool outputs) { return outputs ? 256 : 1024; }

// Segments per pair (equal lengths): enough (segment, pair, block) workgroups to cover the chip once —
// the count up to ceil(target / (BH nb)) with the fewest rounds of `target` workgroups times chunks per
// segment (the ceiling alone can spill a second round; ties: fewer segments).
int wide_segments(int BH, int nb, int nchunk, bool outputs) {
  const long long target = wide_target(outputs), units = (long long)BH * nb;
  long long hi = (target + units - 1) / units;
  if (hi > nchunk) hi = nchunk;
  int best = 1;
  long long cost = -1;
  for (int S = 1; S <= hi; ++S) {
    const long long c = ((units * S + target - 1) / target) * ((nchunk + S - 1) / S);
    if (cost < 0 || c < cost) cost = c, best = S;
  }
  return best;
}

long long round_up(long long x, long long m) { return (x + m - 1) / m * m; }

struct WideLayout {
  int L;  // piece (segment or range) length
  long long gx, nslot, slot_floats, part_floats, coef_floats, zc_floats;
  bool multi;  // state pass + scan before the readout (several pieces per pair, or the expanded-softmax
               // readout, whose coefficient kernel reads the per-chunk z the state pass writes)
};

template <int NT>
WideLayout wide_layout(const Shape& s, int BH, const SeqMap& seq, bool outputs) {
  constexpr int NB = n_blocks<NT>();
  WideLayout lay;
  const bool cent = outputs && s.readout == 1;
  const int unit = cent ? 2 * kCS : kCS;  // the coefficient kernel takes 64-token chunks
  if (seq.packed) {
    // ragged: ranges of the packed token axis, about target workgroups over heads and blocks
    const long long target = wide_target(outputs);
    const long long per = std::max<long long>(1, (seq.tokens(BH) * NB + target - 1) / target);
    lay.L = (int)std::min<long long>((per + unit - 1) / unit * unit, 1 << 30);
  } else {
    const int nchunk = cdiv(seq.N, unit);
    lay.L = cdiv(nchunk, wide_segments(BH, NB, nchunk, outputs)) * unit;
  }
  lay.gx = seq.grid_x(lay.L);
  lay.nslot = seq.row_slots(lay.L);
  // ragged batches always take the state pass and the scan, which writes the final state of every
  // (sequence, head) row, empty sequences included (a single range writes only the rows it walks)
  lay.multi = seq.packed || lay.gx > 1 || cent;
  // slots are needed for a state pass, and always for a state-only call (the scan sums them)
  lay.slot_floats = (lay.multi || !outputs) ? seq.rows(BH) * lay.nslot * s.stride : 0;
  lay.part_floats = (outputs && NB > 1) ? (long long)NB * seq.tokens(BH) * (kDV + 1) : 0;
  lay.coef_floats = cent ? 4 * seq.tokens(BH) : 0;
  lay.zc_floats = cent ? seq.chunk_count(BH, 2 * kCS) * FeatureTable<NT, kDK>::W : 0;
  return lay;
}

// The readout or state-pass kernel for a call (the expanded-softmax readout exists for n = 2, 3 with
// float32 inputs).
template <int NT, typename E, bool READOUT>
auto wide_kernel_for(bool packed, bool cent) {
  if constexpr ((NT == 2 || NT == 3) && std::is_same_v<E, float>) {
    if (cent) return packed ? prefill_wide_kernel<NT, E, READOUT, true, true> : prefill_wide_kernel<NT, E, READOUT, false, true>;
  }
  return packed ? prefill_wide_kernel<NT, E, READOUT, true, false> : prefill_wide_kernel<NT, E, READOUT, false, false>;
}

template <int NT, typename E>
int wide_run(const PrefillArgs& a) {
  constexpr int NB = n_blocks<NT>();
  const bool outputs = a.o != nullptr, cent = a.s.readout == 1;
  const WideLayout lay = wide_layout<NT>(a.s, a.BH, a.seq, outputs);
  const long long tokens = a.seq.tokens(a.BH);
  float* ws = (float*)a.ws;
  float* slots = ws;
  float* part_num = ws + round_up(lay.slot_floats, 64);
  float* part_den = part_num + (long long)NB * tokens * kDV;
  float* coef = part_num + round_up(lay.part_floats, 64);
  float* zc = coef + round_up(lay.coef_floats, 64);
  const E* q = (const E*)a.q;
  const E* k = (const E*)a.k;
  const E* v = (const E*)a.v;
  const long long elems = FeatureTable<NT, kDK>::W * (long long)(kDV + 1);
  const int multi = lay.multi;
  const dim3 grid((unsigned)lay.gx, (unsigned)a.seq.grid_y(a.BH), NB), block(kThreads);
  if (!outputs || multi) {
    const bool zpass = cent && outputs;
    const WideIO io{slots, nullptr, nullptr, nullptr, nullptr, nullptr, a.s.stride, lay.nslot, tokens, multi, nullptr,
                    zpass ? zc : nullptr};
    wide_kernel_for<NT, E, false>(a.seq.packed, zpass)<<<grid, block, 0, a.stream>>>(q, k, v, io, a.seq, lay.L,
                                                                                    a.s.scale);
    if (hipGetLastError() != hipSuccess) return -3;
    if (seg_scan_launch(slots, a.state_in, a.state, a.BH, lay.nslot, a.s.stride, elems, outputs, a.seq, lay.L,
                        a.stream))
      return -3;
    if (!outputs) return 0;
  }
  if (cent) {
    // per-token coefficients from the prefixes the readout starts from
    const CenteredPlan cp{lay.L, lay.nslot, slots, multi, zc, 2 * kCS, reinterpret_cast<float4*>(coef)};
    if (const int rc = centered_coef_launch(a, cp)) return rc;
  }
  const WideIO io{slots,  multi ? nullptr : a.state, multi ? nullptr : a.state_in, part_num, part_den, a.o, a.s.stride,
                  lay.nslot, tokens, multi,
                  cent ? coef : nullptr, nullptr};
  wide_kernel_for<NT, E, true>(a.seq.packed, cent)<<<grid, block, 0, a.stream>>>(q, k, v, io, a.seq, lay.L,
                                                                                a.s.scale);
  if (hipGetLastError() != hipSuccess) return -3;
  if (NB == 1) return 0;  // the outputs are final
  wide_reduce_kernel<<<dim3((unsigned)cdiv(tokens * 16, 256)), dim3(256), 0, a.stream>>>(part_num, part_den, a.o,
                                                                                          tokens, NB);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

// n = 4, 5 for either input type; n = 1..3 for float32 inputs (bfloat16 ones have their own kernel).
bool prefill_wide_has(int nt, int dk, int dv, int dtype) {
  return dk == kDK && dv == kDV && (nt == 4 || nt == 5 || (nt >= 1 && nt <= 3 && dtype == 0));
}

// An upper bound over both uses (with and without outputs): the query does not know which follows.
long long prefill_wide_ws_bytes(const Shape& s, int BH, const SeqMap& seq) {
  auto bytes = [](const WideLayout& lay) {
    return (round_up(lay.slot_floats, 64) + round_up(lay.part_floats, 64) + round_up(lay.coef_floats, 64) +
            lay.zc_floats) * 4;
  };
  auto both = [&](auto layout) { return std::max(bytes(layout(true)), bytes(layout(false))); };
  switch (s.nt) {
    case 1: return both([&](bool o) { return wide_layout<1>(s, BH, seq, o); });
    case 2: return both([&](bool o) { return wide_layout<2>(s, BH, seq, o); });
    case 3: return both([&](bool o) { return wide_layout<3>(s, BH, seq, o); });
    case 4: return both([&](bool o) { return wide_layout<4>(s, BH, seq, o); });
    default: return both([&](bool o) { return wide_layout<5>(s, BH, seq, o); });
  }
}

int prefill_wide_launch(const PrefillArgs& a) {
  if (!prefill_wide_has(a.s.nt, a.s.dk, a.s.dv, a.s.dtype)) return -2;
  switch (a.s.nt) {
    case 1: return wide_run<1, float>(a);
    case 2: return wide_run<2, float>(a);
    case 3: return wide_run<3, float>(a);
    case 4: return a.s.dtype == 0 ? wide_run<4, float>(a) : wide_run<4, __bf16>(a);
    default: return a.s.dtype == 0 ? wide_run<5, float>(a) : wide_run<5, __bf16>(a);
  }
}

}  // namespace taylor
