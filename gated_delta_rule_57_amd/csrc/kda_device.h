// Device helpers for the KDA kernels on gfx950 (CDNA4): element types, MFMA
// fragments and the fragment convention shared by the prefill kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int D = 128;  // head dimension (dk = dv)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
// float -> bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return (__bf16)x; }

// Four consecutive elements, as one 8-byte (bf16) or 16-byte (fp32) access.
template <typename E> struct Vec4;
template <> struct Vec4<float> { typedef floatx4 T; };
template <> struct Vec4<__bf16> { typedef bf16x4 T; };

template <typename E>
__device__ __forceinline__ void load4f(const E* p, float out[4]) {
  typename Vec4<E>::T v = *reinterpret_cast<const typename Vec4<E>::T*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = to_f(v[i]);
}
template <typename E>
__device__ __forceinline__ void store4f(E* p, const float in[4]) {
  typename Vec4<E>::T v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = from_f<E>(in[i]);
  *reinterpret_cast<typename Vec4<E>::T*>(p) = v;
}

// ---------------------------------------------------------------------------
// MFMA fragments.
//
// A product D(16x16) += A(16 x 32) * B(32 x 16) over one "k-block" of 32 is done
// with v_mfma_f32_16x16x32_bf16 (one instruction) or with eight
// v_mfma_f32_16x16x4_f32. Lane l = m + 16 g (m = l & 15, g = l >> 4) holds eight
// operand elements in slots s = 0..7:
//     A: A[m][koff(g, s)]       B: B[koff(g, s)][m]
//     koff(g, s) = 4 g + s          for s < 4
//                = 16 + 4 g + s - 4 for s >= 4
// and receives D[4 g + i][m] in accumulator element i (i = 0..3).
// Because A and B use the same (g, s) -> k map, the map only has to be a
// permutation of 0..31; this one is chosen so that two stacked accumulator tiles
// (rows 0..15 and 16..31 of a 32 x 16 result) are, element for element, the B
// fragment of the next product. Results therefore chain from one MFMA into the
// next in registers, with no shuffle and no LDS round trip.
// ---------------------------------------------------------------------------
template <typename E> struct Frag;
template <> struct Frag<__bf16> { typedef bf16x8 T; };
template <> struct Frag<float> { typedef floatx8 T; };

__device__ __forceinline__ int koff(int g, int s) { return s < 4 ? 4 * g + s : 12 + 4 * g + s; }

__device__ __forceinline__ void mma(floatx4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(floatx4& acc, const floatx8& a, const floatx8& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
}

// Two accumulator tiles (rows 0..15 -> slots 0..3, rows 16..31 -> slots 4..7) as a B
// fragment of element type E.
template <typename E>
__device__ __forceinline__ typename Frag<E>::T acc_pair_to_frag(const floatx4& lo, const floatx4& hi) {
  typename Frag<E>::T f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = from_f<E>(lo[i]);
    f[4 + i] = from_f<E>(hi[i]);
  }
  return f;
}

// Fragment whose k runs along a row of a row-major matrix M (row stride ld
// elements): slot s = M[row][kb + koff(g, s)]. Two 4-element reads.
template <typename E>
__device__ __forceinline__ typename Frag<E>::T frag_rowk(const E* M, int ld, int row, int kb, int g) {
  typename Frag<E>::T f;
  const E* p = M + (size_t)row * ld + kb + 4 * g;
  typename Vec4<E>::T a = *reinterpret_cast<const typename Vec4<E>::T*>(p);
  typename Vec4<E>::T b = *reinterpret_cast<const typename Vec4<E>::T*>(p + 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a[i];
    f[4 + i] = b[i];
  }
  return f;
}

// Fragment whose k runs down a column of a row-major matrix M: slot s =
// M[kb + koff(g, s)][col]. Eight strided reads.
template <typename E>
__device__ __forceinline__ typename Frag<E>::T frag_colk(const E* M, int ld, int col, int kb, int g) {
  typename Frag<E>::T f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = M[(size_t)(kb + koff(g, s)) * ld + col];
  return f;
}

// Global fragment store / load: one lane's eight elements, contiguous.
template <typename E>
__device__ __forceinline__ void store_frag(E* p, const typename Frag<E>::T& f) {
  *reinterpret_cast<typename Frag<E>::T*>(p) = f;
}
template <typename E>
__device__ __forceinline__ typename Frag<E>::T load_frag(const E* p) {
  return *reinterpret_cast<const typename Frag<E>::T*>(p);
}

// Ordering helpers for LDS exchanges between the waves of a work-group.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// Per-row factors of a wave's 32 state rows in the accumulator layout (lane (m, g)
// needs rows 16 j + 4 g + i, j = 0, 1, i = 0..3) from one word per lane: lane (m, g)
// loads row row_word_index(m, g) = 16 ((m >> 3) & 1) + 4 g + (m & 3), and the eight
// values it needs come from its own 16-lane row by DPP moves (a rotation by 8 for the
// other j, a quad broadcast for each i), with no memory or LDS traffic.
__device__ __forceinline__ int row_word_index(int m, int g) { return 16 * ((m >> 3) & 1) + 4 * g + (m & 3); }
__device__ __forceinline__ void rows_from_word(float v, int m, floatx4 out[2]) {
  const int own = __builtin_bit_cast(int, v);
  const int other = __builtin_amdgcn_mov_dpp(own, 0x128, 0xF, 0xF, true);  // row_ror:8
  const bool hi = ((m >> 3) & 1) != 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int x = (hi == (j == 1)) ? own : other;  // lane (m, g) now holds row 16 j + 4 g + (m & 3)
    out[j][0] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x00, 0xF, 0xF, true));  // quad lane 0
    out[j][1] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x55, 0xF, 0xF, true));  // quad lane 1
    out[j][2] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xAA, 0xF, 0xF, true));  // quad lane 2
    out[j][3] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xFF, 0xF, 0xF, true));  // quad lane 3
  }
}

// Non-temporal vector store of a 4-element vector (data read back only much later)
template <typename V>
__device__ __forceinline__ void store_nt(V* p, const V& x) {
  typedef unsigned int U __attribute__((ext_vector_type(sizeof(V) / 4)));
  __builtin_nontemporal_store(__builtin_bit_cast(U, x), reinterpret_cast<U*>(p));
}
// Non-temporal vector load of data read once, long after it was written (the
// per-chunk records and states, the inputs of the intra-chunk kernel).
template <typename V>
__device__ __forceinline__ V load_nt(const V* p) {
  typedef unsigned int U __attribute__((ext_vector_type(sizeof(V) / 4)));
  return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const U*>(p)));
}
// s_waitcnt with lgkmcnt(0) and the vector-memory counter left free
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// work-group barrier for LDS exchanges that leaves in-flight global loads alone
__device__ __forceinline__ void lds_barrier() {
  compiler_fence();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// x plus the value of another lane of its 16-lane row, chosen by a DPP control word
// (row-local patterns only, so every lane has a source)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over the 16 lanes of x's row (lanes with equal lane >> 4), in every lane: quad
// swaps xor 1 and xor 2, then the half-row and row mirrors, which pair each quad and
// each half-row with the other one. DPP moves, no trip through the LDS unit.
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_add<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_add<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_add<0x141>(x);  // row_half_mirror
  return dpp_add<0x140>(x);  // row_mirror
}

// x + (x of the lane 16 apart within each half-wave), with no trip through the LDS
// unit: gfx950's v_permlane16_swap exchanges the odd 16-lane rows of one register with
// the even rows of another, so on two copies of x it leaves rows (x0, x0, x2, x2) in
// one and (x1, x1, x3, x3) in the other, and their sum is the pair sum in every lane
__device__ __forceinline__ float xor16_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x + (x of the lane 32 apart), by v_permlane32_swap (the upper 32 lanes of one register
// with the lower 32 of another) on two copies of x
__device__ __forceinline__ float xor32_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// X^T Y for 16 x 16 fp32 matrices both held in accumulator layout (lane (n, g),
// element i: row 4 g + i of column n): k-step i pairs row 4 g + i of X (as the A
// operand's column) with row 4 g + i of Y (the B operand), on fp32 MFMA.
__device__ __forceinline__ floatx4 mm16_tn(const floatx4& x, const floatx4& y) {
  floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(x[i], y[i], c, 0, 0, 0);
  return c;
}

// (I + A)^{-1} of a strictly lower-triangular 16 x 16 fp32 block A (row-major at a,
// row stride lda, zeros on and above the diagonal), returned in accumulator layout.
// With N = -A nilpotent (N^16 = 0), (I + A)^{-1} = sum_{k<16} N^k =
// (I + N)(I + N^2)(I + N^4)(I + N^8): eight 16 x 16 products on fp32 MFMA (powers
// formed with their transposes, so that every product finds its operands in
// accumulator layout), in place of a 16-step row-by-row substitution on 16 lanes. Its
// rounding grows with the powers' entries, so the bf16-operand paths use it.
__device__ __forceinline__ floatx4 unit_lower_inverse16(const float* a, int lda, int lane) {
  const int n = lane & 15, g = lane >> 4;
  floatx4 N, Nt;
  const floatx4 arow = *reinterpret_cast<const floatx4*>(a + n * lda + 4 * g);  // A[n][4g + i]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    N[i] = -a[(4 * g + i) * lda + n];  // N[4g + i][n]
    Nt[i] = -arow[i];                  // N^T[4g + i][n] = N[n][4g + i]
  }
  auto plus_i = [&](floatx4 x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] += (4 * g + i == n) ? 1.f : 0.f;
    return x;
  };
  const floatx4 N2 = mm16_tn(Nt, N), N2t = mm16_tn(N, Nt);      // N N, (N N)^T
  const floatx4 N4 = mm16_tn(N2t, N2), N4t = mm16_tn(N2, N2t);  // N^4, (N^4)^T
  const floatx4 N8 = mm16_tn(N4t, N4);
  const floatx4 E1t = plus_i(Nt), E2 = plus_i(N2), E4 = plus_i(N4), E8 = plus_i(N8);
  const floatx4 R1t = mm16_tn(E2, E1t);  // ((I + N)(I + N^2))^T
  const floatx4 R2t = mm16_tn(E4, R1t);  // ((I + N)(I + N^2)(I + N^4))^T
  return mm16_tn(R2t, E8);
}

}  // namespace kda
