// Internal launch interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace taylor {

// Tokens per chunk walked by the matrix-core prefill kernels (bfloat16 pipeline; float32 feature
// blocks), whatever the configured chunk length.
constexpr int kMfmaChunk = 64;
constexpr int kWideChunk = 32;

struct Shape {
  int nt;       // Taylor terms
  int dk, dv;   // head dims
  int dtype;    // 0 = float32, 1 = bfloat16 inputs
  int readout;  // 0 = truncated kernel, normalised; 1 = softmax expanded about the mean score
  float scale;  // score scale
  long long W;       // feature width
  long long stride;  // floats per head block in the state
};

struct DecodeArgs {
  Shape s;
  const void *q, *k, *v;
  float* o;
  float* state;
  int BH;
  hipStream_t stream;
};

// A run of consecutive tokens of one (sequence, head) pair that a workgroup processes as a unit: it
// starts from the state of the pair's earlier tokens and adds its own tokens' contribution.
struct SeqPiece {
  long long tok;   // index of its first token in q, k, v and o (rows of d_k / d_v values)
  int n;           // tokens, >= 1
  long long slot;  // its workspace slot
  long long pair;  // the (sequence, head) pair b * H + h
};

// Where the tokens of (sequence, head) pair b * H + h live, and how workgroups cut them into pieces
// of at most L tokens, each with one workspace slot of `stride` floats.
//
// Equal lengths (packed == 0): q, k, v, o are [B][H][N][d].  Grid (ceil(N / L), B * H): workgroup
// (x, bh) takes tokens x*L .. of pair bh, slot bh * nslot + x (nslot = ceil(N / L)).
//
// Ragged (packed == 1): the sequences are packed head-major, [H][T][d] with T total tokens, and
// sequence b occupies tokens cu[b] .. cu[b + 1] - 1 of every head.  Grid (ceil(T / L), H):
// workgroup (x, h) takes the token range [x*L, (x+1)*L) of head h, which holds one piece per
// sequence it overlaps (the work is balanced whatever the lengths).  Piece (x, b) uses slot
// h * nslot + x + b: a sequence's pieces lie in consecutive ranges and the next sequence starts
// no earlier than the range where this one ends, so no two pieces share a slot, and
// nslot = floor(T / L) + B + 1 slots per head suffice.  Offsets read from cu are clamped to
// [0, T], so no index leaves its buffer whatever the array holds (the caller guarantees
// 0 = cu[0] <= ... <= cu[B] = T).
struct SeqMap {
  const int32_t* cu;  // device array of B + 1 offsets, read only when packed
  int packed;
  int B, H;
  int N;        // equal lengths: tokens per sequence; ragged: the longest sequence
  long long T;  // ragged: total tokens

  struct Walk {
    int b;  // next sequence to look at
  };

  __device__ __forceinline__ long long off(int b) const {
    const long long c = cu[b];
    return c < 0 ? 0 : (c > T ? T : c);
  }

  // Equal lengths: the one piece of workgroup (x, y); false when the segment is empty.
  __device__ __forceinline__ bool equal_piece(long long x, long long y, int L, long long nslot, SeqPiece& p) const {
    const long long t0 = x * L;
    if (t0 >= N) return false;
    p = SeqPiece{y * N + t0, (int)(N - t0 < L ? N - t0 : L), y * nslot + x, y};
    return true;
  }

  // Ragged: starts the pieces of workgroup (x, y) at the first sequence ending after the range
  // start (binary search; uniform scalar loads).
  __device__ __forceinline__ Walk begin(long long x, int L) const {
    const long long r0 = x * L;
    int lo = 0, hi = B;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (off(mid + 1) > r0)
        hi = mid;
      else
        lo = mid + 1;
    }
    return Walk{lo};
  }

  // Ragged: the next non-empty piece of workgroup (x, y); false when there is none.
  __device__ __forceinline__ bool next(Walk& w, long long x, long long y, int L, long long nslot,
                                       SeqPiece& p) const {
    const long long r0 = x * L, r1 = (r0 + L < T ? r0 + L : T);
    while (w.b < B) {
      const int b = w.b++;
      const long long c0 = off(b), c1n = off(b + 1), c1 = c1n > c0 ? c1n : c0;
      if (c0 >= r1) {
        w.b = B;
        return false;
      }
      const long long p0 = c0 > r0 ? c0 : r0, p1 = c1 < r1 ? c1 : r1;
      if (p1 > p0) {
        p = SeqPiece{y * T + p0, (int)(p1 - p0), y * nslot + x + b, (long long)b * H + y};
        return true;
      }
    }
    return false;
  }

  // Ragged, one pass: the whole of sequence b in head h as one piece (n may be 0).
  __device__ __forceinline__ SeqPiece whole_piece(long long b, long long h) const {
    const long long c0 = off((int)b), c1n = off((int)b + 1), c1 = c1n > c0 ? c1n : c0;
    return SeqPiece{h * T + c0, (int)(c1 - c0), 0, b * H + h};
  }

  // Slots of pair bh's pieces, in token order: first, first + 1, ..., first + count - 1.
  __device__ __forceinline__ void pair_slots(long long bh, long long nslot, int L, long long& first,
                                             int& count) const {
    if (!packed) {
      first = bh * nslot;
      count = (int)((N + (long long)L - 1) / L);
      return;
    }
    const int b = (int)(bh / H);
    const long long h = bh - (long long)b * H;
    const long long c0 = off(b), c1 = off(b + 1);
    first = h * nslot + c0 / L + b;
    count = c1 > c0 ? (int)((c1 - 1) / L - c0 / L + 1) : 0;
  }

  // Index of chunk c (chunks of CH tokens, CH dividing L) of piece p in a per-chunk array: equal
  // lengths, pair * ceil(N / CH) + (the chunk's position in the pair) / CH; ragged, per head
  // floor(position / CH) + b, which keeps consecutive sequences apart as the slots do, with
  // floor(T / CH) + B + 1 entries per head.
  __device__ __forceinline__ long long chunk_index(const SeqPiece& p, int c, int CH) const {
    if (!packed) {
      const long long per = (N + (long long)CH - 1) / CH;
      return p.pair * per + (p.tok - p.pair * (long long)N) / CH + c;
    }
    const long long b = p.pair / H, h = p.pair - b * H;
    return h * (T / CH + B + 1) + (p.tok - h * T) / CH + c + b;
  }
  long long chunk_count(int BH, int CH) const {
    return packed ? (long long)H * (T / CH + B + 1) : (long long)BH * ((N + (long long)CH - 1) / CH);
  }

  // Token-heads covered: the extent of an output or per-token workspace array.
  __host__ __device__ long long tokens(int BH) const { return packed ? (long long)H * T : (long long)BH * N; }
  // Host side: grid and workspace extent for pieces of L tokens.
  long long grid_x(int L) const { return packed ? (T + L - 1) / L : (N + (long long)L - 1) / L; }
  long long grid_y(int BH) const { return packed ? H : BH; }
  long long rows(int BH) const { return packed ? H : BH; }
  long long row_slots(int L) const { return packed ? T / L + B + 1 : grid_x(L); }
};

// Calls f(piece) for each piece of workgroup (x, y), in token order.  PACKED must equal
// seq.packed; the kernels are compiled for both so that equal lengths keep straight-line code.
template <bool PACKED, class F>
__device__ __forceinline__ void for_each_piece(const SeqMap& seq, long long x, long long y, int L, long long nslot,
                                               F&& f) {
  SeqPiece p;
  if constexpr (PACKED) {
    for (SeqMap::Walk w = seq.begin(x, L); seq.next(w, x, y, L, nslot, p);) f(p);
  } else {
    if (seq.equal_piece(x, y, L, nslot, p)) f(p);
  }
}

struct PrefillArgs {
  Shape s;
  const void *q, *k, *v;
  float* o;               // may be null (state-only)
  const float* state_in;  // the history before the call; null: empty
  float* state;           // where the final state goes; null: discarded.  Equal to state_in or disjoint
  void* ws;        // workspace
  int BH, N, C;    // (sequence, head) pairs, tokens per sequence (the longest when ragged), chunk
  SeqMap seq;      // token placement
  hipStream_t stream;
};

// Each returns 0 on success, -2 if the shape has no compiled kernel, -3 on a launch error.
int decode_launch(const DecodeArgs& a);
bool decode_has(int nt, int dk, int dv);

int state_zero_launch(float* state, long long count, hipStream_t stream);

// Exclusive prefix over the pieces of each (sequence, head) pair in `ws` (slots of `stride` floats
// placed as SeqMap describes for pieces of L tokens, `nslot` per row), seeded with `seed` when
// non-null, else zero; the total is written to `total` when non-null (it may be `seed`).  Only the
// first `elems` floats of each slot are touched.
int seg_scan_launch(float* ws, const float* seed, float* total, int BH, long long nslot, long long stride,
                    long long elems, bool write_prefix, const SeqMap& seq, int L, hipStream_t stream);
// dst = src over `count` floats (a multiple of 4; 16-byte aligned).
int state_copy_launch(float* dst, const float* src, long long count, hipStream_t stream);

// Portable prefill path (any compiled (n, d_k, d_v), chunk 64 or 128), VALU float32.
bool prefill_generic_has(int nt, int dk, int dv, int C);
long long prefill_generic_ws_bytes(const Shape& s, int BH, int N, int C);
int prefill_generic_launch(const PrefillArgs& a);

}  // namespace taylor
