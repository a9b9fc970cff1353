// LDS tile layouts of the bfloat16 prefill: unpadded rows whose 16-byte slots are permuted by an XOR
// with bits of the row index, so that the kernel's reads and writes of a tile are free of bank
// conflicts.  (The float32 feature-block kernel keeps padded rows: there the swizzles removed the
// conflicts without a change in time.)
//
// Bank rule of gfx950 (measured: one wavefront with only lanes 0 and x active, their two addresses
// 256 bytes apart, SQ_LDS_BANK_CONFLICT for x = 1..63 at every access width): reads see 64 four-byte
// banks and writes 32.  A 16-byte read serves 16 lanes per cycle, those with the same lane bit 5 and
// the same parity of lane bits 2..4 (lane 0 is served with lanes 1-3, 12-15 and 20-27); an 8- or
// 4-byte read serves 32 consecutive lanes; a 16-byte write 8 consecutive lanes, an 8-byte write 16, a
// 4-byte write 32.  Under this rule padding cannot serve both sides of these tiles (token-major rows
// read as 16 rows x 4 lane groups are conflict-free for strides of 2 mod 4 sixteen-byte slots, and
// written one row per lane for odd strides), while the swizzles below, found by a search over XOR
// permutations against the rule, serve every access the kernels make of them.
#pragma once

namespace taylor {

// Feature-major tiles with 128-byte rows (phi(K)^T and V^T: 64 bfloat16 tokens per row): slot s of row r sits at slot s ^ swz_kv(r).  Conflict-free for 16-byte reads of rows
// 16t + (lane & 15) at slot 4j + (lane >> 4), 8-byte reads of the same rows, 16-byte reads of one row
// per lane (row sums), 4-byte writes of one row per 32 lanes, paired-row 4-byte writes (even lanes
// row r, odd lanes row r + 1) and 2-byte writes.
__host__ __device__ constexpr int swz_kv(int r) {
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2);
}

// Byte offset of element t (of size ES bytes) in row r of such a tile.
template <int ES>
__host__ __device__ constexpr int kv_off(int r, int t) {
  constexpr int per_slot = 16 / ES;
  return r * 128 + 16 * ((t / per_slot) ^ swz_kv(r)) + ES * (t % per_slot);
}

// Token-major tiles (phi(sQ): one row per token, NS 16-byte slots per row): slot s of row r sits at
// s ^ swz_tok<NS>(r), an XOR within an aligned group of 4, 8 or 16 slots.  Conflict-free for 16-byte
// reads of rows 16i + (lane & 15) at slot 4t + (lane >> 4) and 16-byte writes of one row per lane.
template <int NS>
__host__ __device__ constexpr int swz_tok(int r) {
  static_assert(NS % 4 == 0, "rows of whole groups of four slots");
  if constexpr (NS % 16 == 0)
    return r & 15;
  else if constexpr (NS % 8 == 0)
    return r & 7;
  else
    return (r >> 1) & 3;
}

}  // namespace taylor
