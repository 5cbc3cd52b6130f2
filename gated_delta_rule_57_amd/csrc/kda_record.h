// Layout of the per-(chunk, head) record that the intra-chunk kernel writes and the
// inter-chunk kernels read (shared by the prefill and the backward's forward pass).
#pragma once

#include "kda_device.h"

namespace kda {

__host__ __device__ constexpr size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ constexpr size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }

// Per-(chunk, head) record, element offsets for element type E and chunk C.
template <typename E, int C>
struct Rec {
  static constexpr int NRT = C / 16;           // 16-row tiles of the chunk
  static constexpr int NKC = (C + 31) / 32;    // 32-row k-blocks over the chunk
  static constexpr int FR = 64 * 8;            // one fragment block: 64 lanes x 8 elements
  static constexpr size_t WN = 0;                                   // [NRT][4][64][8]   -W
  static constexpr size_t QT = WN + (size_t)NRT * 4 * FR;           // [NRT][4][64][8]   Q e^G
  static constexpr size_t KE = QT + (size_t)NRT * 4 * FR;           // [8][NKC][64][8]   (K e^{g_C-G})^T
  static constexpr size_t PP = KE + (size_t)8 * NKC * FR;           // [NRT][NKC][64][8] P (causal: the
                                                                    // slots above the diagonal are not written)
  static constexpr size_t UU = PP + (size_t)NRT * NKC * FR;         // [8][NRT][64][4]   U, accumulator order
  static constexpr size_t END = UU + (size_t)NRT * 8 * 64 * 4;
  static constexpr size_t GAMMA_BYTES = al256(END * sizeof(E));      // float[128] e^{g_C}
  static constexpr size_t BYTES = al256(GAMMA_BYTES + D * sizeof(float));
};

// Per-(chunk, head) record of the general diagonal-plus-low-rank recurrence
// S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T, element offsets. The first
// five fields play the roles of the KDA record's, so the state pass reads them the
// same way (W below is the matrix of rows w_r = S_{r-1}^T b_r, which takes the
// place of U~):
//   WN   W_b = T (B e^{G^-})       W = U + W_b S_0
//   QT   Q e^G                      O = Q e^G S_0 + P W + M_qk V
//   KE   (A e^{g_C-G})^T            S_C = e^{g_C} S_0 + KE W + KV V
//   PP   P = M_qa
//   UU   U = T M_bk V
// and three more:
//   KV   (K e^{g_C-G})^T            [8][NKC][64][8]
//   VB   V as B fragments           [8 column slabs][NKC][64][8]
//   OI   M_qk V                     [8 column slabs][NRT][64][4], transposed accumulator
//                                   order: lane (m, g) holds row 16 rt + m, columns
//                                   16 ct + 4 g .. + 3
template <typename E, int C>
struct RecD {
  static constexpr int NRT = C / 16;
  static constexpr int NKC = (C + 31) / 32;
  static constexpr int FR = 64 * 8;
  static constexpr size_t WN = 0;
  static constexpr size_t QT = WN + (size_t)NRT * 4 * FR;
  static constexpr size_t KE = QT + (size_t)NRT * 4 * FR;
  static constexpr size_t PP = KE + (size_t)8 * NKC * FR;
  static constexpr size_t UU = PP + (size_t)NRT * NKC * FR;
  static constexpr size_t KV = UU + (size_t)NRT * 8 * 64 * 4;
  static constexpr size_t VB = KV + (size_t)8 * NKC * FR;
  static constexpr size_t OI = VB + (size_t)8 * NKC * FR;
  static constexpr size_t END = OI + (size_t)C * D;
  static constexpr size_t GAMMA_BYTES = al256(END * sizeof(E));
  static constexpr size_t BYTES = al256(GAMMA_BYTES + D * sizeof(float));
};

// The backward's per-chunk 128 x 128 matrices (the state entering each chunk and the
// state gradient at its end) are kept in 16 x 16 tiles in fragment order, the eight
// tiles of a 16-column slab contiguous: element (i, j) at index
//   ((j / 16 * 8 + i / 16) * 64 + i % 16 + 16 * (j % 16 / 4)) * 4 + j % 4.
// A lane's four consecutive columns of one row are contiguous and every tile is one
// contiguous 512-byte (bf16) block, so the serial pass that owns a slab writes 4 KiB
// in a row, and the 32-wide k-block of a fragment over a row (k = column) is two
// blocks: tiles (i / 16, 2 kb) and (i / 16, 2 kb + 1), lane i % 16 + 16 g in both.
__host__ __device__ constexpr size_t state_tile_index(int i, int j) {
  return ((size_t)((j >> 4) * 8 + (i >> 4)) * 64 + (i & 15) + 16 * ((j & 15) >> 2)) * 4 + (j & 3);
}
// The 16 x 128 U~ and dU~ in the same tiles (one row of them): element (i, j), i < 16,
// at ((j / 16) * 64 + i + 16 * (j % 16 / 4)) * 4 + j % 4.
__host__ __device__ constexpr size_t row_tile_index(int i, int j) {
  return ((size_t)(j >> 4) * 64 + (i & 15) + 16 * ((j & 15) >> 2)) * 4 + (j & 3);
}

// The store of one 128 x 16 slab (slab ct: dst = matrix + ct * 2048) in
// state_tile_index order from its eight tiles in accumulator order (stage [rt][lane][4],
// lane (m, g) holding rows 4 g .. 4 g + 3 of column m): four stores, store q covering
// tiles 2q and 2q + 1 (contiguous), lane l writing the pieces of tile lanes 2 (l % 32)
// and 2 (l % 32) + 1 of tile 2q + l / 32. Non-temporal: the data is read back much later.
template <typename E>
__device__ __forceinline__ void store_state_slab(E* __restrict__ dst, const E* __restrict__ stage, int lane) {
  typedef typename Frag<E>::T F8;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const E* tile = stage + (2 * q + (lane >> 5)) * 256;
    F8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // tile lane tl = (mm, gg): row mm, column 4 gg + e % 4
      const int tl = 2 * (lane & 31) + (e >> 2), mm = tl & 15, gg = tl >> 4;
      x[e] = tile[(4 * gg + (e & 3) + 16 * (mm >> 2)) * 4 + (mm & 3)];
    }
    store_nt(reinterpret_cast<F8*>(dst + (size_t)q * 512 + lane * 8), x);
  }
}

}  // namespace kda
