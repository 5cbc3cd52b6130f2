// Backward pass of the KDA chunk form on gfx950: gradients of
//     L = sum_t <o_t, do_t> + sum_n <S_final[n], dS_final[n]>
// with respect to q, k, v, log_alpha, beta and the initial state. The pages present
// the chunked WY / UT form as what makes KDA efficient to train ("From GPT-2 to Kimi
// K3" digest, section "DeltaNet 병렬화 -- 청크 단위 학습"; GeekNews "Kimi Linear" summary,
// section "청크 단위 병렬 알고리듬"); these are the derivatives of that map.
//
// Per chunk of C = 16 tokens (rows r, s), with S0 the state entering the chunk and
// G the in-chunk cumulative log decay (per channel), the forward is
//     A = tril_strict(diag(beta) (K e^G)(K e^-G)^T),  T = (I + A)^-1
//     W = T diag(beta) K e^G,  U = T diag(beta) V,  U~ = U - W S0
//     P = tril((Q e^G)(K e^-G)^T),  O = (Q e^G) S0 + P U~
//     S_C = e^{g_C} o S0 + (K e^{g_C - G})^T U~ .
// Its reverse, given dO and dS_C (the gradient at the chunk's end):
//     dU~ = P^T dO + (K e^{g_C-G}) dS_C
//     dS0 = (Q e^G)^T dO + e^{g_C} o dS_C - W^T dU~            (carried to the chunk before)
//     X1 = dO S0^T,  X2 = dU~ S0^T,  X3 = U~ dS_C^T,  dgamma = rowsum(dS_C o S0)
//     dP = tril(dO U~^T),  dW = -X2,  dU = dU~
//     dT = dW (diag(beta) K e^G)^T + dU (diag(beta) V)^T,  dA = -T^T dT T^T (strictly lower)
// and from there to q, k, v, beta and G through the element-wise decay factors, then
// dlog_alpha = reverse cumulative sum of dG over the chunk's rows.
//
// Kernels, in launch order:
//   the forward's chunk plan at 16-token chunks (plan_kernel);
//   bwd_local_kernel   one work-group per (chunk, head): W, Q e^G, K e^{g_C-G}, P and
//                      e^{g_C}, in the fragment order the reverse state pass reads,
//                      and the record the forward state pass reads (-W, its
//                      (K e^{g_C-G})^T, U = T diag(beta) V and e^{g_C}; kda_record.h);
//   fwd_state_kernel   the forward state pass (inter16_body), four compute waves
//                      and a store wave per (sequence, head, 16-column slab): keeps
//                      the state entering every chunk and U~;
//   bwd_state_kernel   the reverse state pass (bwd_state_body), four compute waves
//                      and a store wave per (sequence, head, 16-column slab), over
//                      the chunks in reverse
//                      with the 128 x 16 fp32 slab of the state gradient in
//                      accumulator registers: keeps dS_C and dU~ per chunk and writes
//                      the initial-state gradient;
//   bwd_chunk_kernel   one work-group per (chunk, head): everything local to the
//                      chunk. X1, X2, X3 and dgamma are bf16 (or fp32) MFMA products
//                      whose operands come straight from global memory (dO by rows;
//                      the states, state gradients, U~ and dU~ in 16 x 16 tiles);
//                      dT, dB_K, dB_V and the decay-weighted sums over the chunk's rows
//                      are MFMAs too, on operands built in LDS; 16 x 16 algebra (T,
//                      dA) and the element-wise terms run on the VALU in fp32.
// In-chunk decays (log2 units) are factored around a per-channel reference in the
// middle of the chunk's decay range, so both factors stay within 2^(+-60) while the
// range is at most 120; a chunk with a wider range in any channel evaluates every
// term as 2^-|g_r - g_s| instead (exponent <= 0 for any input meeting the
// log_alpha <= 0 precondition).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_device.h"
#include "kda_inter16.h"
#include "kda_internal.h"
#include "kda_record.h"

namespace kda {
namespace {

constexpr int BC = BWD_CHUNK;
static_assert(BC == 16, "the backward kernels are written for 16-token chunks");
constexpr int LDP = D + 4;  // row stride of the fp32 [16][128] LDS matrices: rows 4 apart fall
                            // 16 banks apart, so accumulator-layout reads are conflict-free
constexpr int LDS16 = BC + 1;
// row stride of the [16][128] k and q LDS matrices by element type: bf16 rows 144
// elements (72 words) apart put four consecutive rows 8 banks apart, so a wave reading
// 16 consecutive channels of 4 rows touches 32 distinct banks
template <typename E> struct LdsStride { static constexpr int v = LDP; };
template <> struct LdsStride<__bf16> { static constexpr int v = D + 16; };
constexpr float LOG2E_B = 1.4426950408889634f;

__host__ __device__ constexpr size_t bal256(size_t x) { return (x + 255) & ~(size_t)255; }

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// sum over the 16 lanes l with equal l >> 4 (one row of the element-wise phases)
__device__ __forceinline__ float sum16(float x) { return row16_sum(x); }

// Per-(head, chunk) record for the reverse state pass, in the MFMA operand order
// reverse state pass consumes (lane l = m + 16 g; the fragment convention of
// kda_device.h, chunk rows padded to 32 with zeros):
//   WT   [4 w][64][2 j][4]  slot s of the A fragment of (-W)^T for channel tile
//                           rt = 2w + j: -W[4g+s][16rt+m] (the two tiles that wave w of
//                           the reverse pass uses are one 8-element piece per lane)
//   QTT  [4 w][64][2 j][4]  the same for (Q e^G)^T
//   KEF  [4 kb][64][8]  A fragment of K e^{g_C-G} (rows m, channels 32 kb + koff(g, s))
//   PT   [64][4]        A fragment of P^T: P[4g+s][m]
//   GAM  float[128]     e^{g_C}
template <typename E>
struct BRec {
  static constexpr size_t WT = 0;
  static constexpr size_t QTT = WT + (size_t)8 * 64 * 4 * sizeof(E);
  static constexpr size_t KEF = QTT + (size_t)8 * 64 * 4 * sizeof(E);
  static constexpr size_t PT = KEF + (size_t)4 * 64 * 8 * sizeof(E);
  static constexpr size_t GAM = bal256(PT + (size_t)64 * 4 * sizeof(E));
  static constexpr size_t BYTES = bal256(GAM + D * 4);
};

// Element-wise phases: thread t owns row r = t >> 4. It loads channels
// c0 .. c0 + 7 (c0 = 8 (t & 15)) from global memory, and computes on channels
// ch(i) = (t & 15) + 16 i, i = 0..7: the sixteen lanes of a row then touch sixteen
// consecutive words of any LDS row, one per bank, and the four rows of a wave read
// the same words of another row (a broadcast) in the loops over the chunk's rows.
struct RowMap {
  int r, c0, cg;
  __device__ RowMap(int t) : r(t >> 4), c0(8 * (t & 15)), cg(t & 15) {}
  __device__ int ch(int i) const { return cg + 16 * i; }
};

// Loads eight consecutive values of row r (zeros past len) as fp32.
template <typename E>
__device__ __forceinline__ void load8(const E* base, size_t row_stride, int r, int len, int c0, float out[8]) {
  if (r < len) {
    load4f(base + (size_t)r * row_stride + c0, out);
    load4f(base + (size_t)r * row_stride + c0 + 4, out + 4);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = 0.f;
  }
}

// Copies eight consecutive values of row r (zeros past len) to dst, as KT.
template <typename E, typename KT>
__device__ __forceinline__ void copy8(const E* base, size_t row_stride, int r, int len, int c0, KT* dst) {
  if constexpr (std::is_same<E, KT>::value) {
    typedef typename Vec4<E>::T V4;
    V4 a, b;
    if (r < len) {
      a = *reinterpret_cast<const V4*>(base + (size_t)r * row_stride + c0);
      b = *reinterpret_cast<const V4*>(base + (size_t)r * row_stride + c0 + 4);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = b[i] = from_f<E>(0.f);
    }
    *reinterpret_cast<V4*>(dst) = a;
    *reinterpret_cast<V4*>(dst + 4) = b;
  } else {
    float x[8];
    load8(base, row_stride, r, len, c0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = x[i];
  }
}

// The state-independent part shared by both per-chunk kernels: q, k rows, the
// log2-unit decay cumsum G, the per-channel reference b, M_rs = sum_i k_ri k_si
// 2^(G_ri - G_si) for s < r, optionally P_rs = sum_i q_ri k_si 2^(G_ri - G_si) for
// s <= r, and T = (I + A)^-1 with A_rs = beta_r M_rs. Ends with a barrier.
//
// Decay factoring: with R = G_0 - G_15 (per channel, >= 0) and b = (G_0 + G_15) / 2,
// 2^(G_r - G_s) = 2^(G_r - b) 2^(b - G_s) with both factors in [2^(-R/2), 2^(R/2)], so
// a decay-weighted sum over the chunk's rows is a plain product of factored
// operands (an MFMA) whose every term, masked ones included, stays finite while
// R <= FACTOR_MAX_RANGE. A chunk with a wider range in any channel ("exact") takes
// the element-wise path, 2^-|G_r - G_s| per term.
constexpr float FACTOR_MAX_RANGE = 120.f;

// KT: element type of the k and q copies (the input type keeps them exact and halves
// their LDS in bf16; the gradient kernel keeps fp32 copies)
template <typename KT>
struct LocalLds {
  KT K[BC][LdsStride<KT>::v], Q[BC][LdsStride<KT>::v];
  float G[BC][LDP];
  float M[BC][LDS16], T[BC][LDS16], Pm[BC][LDS16];
  float beta[BC];
  float bref[D];
  alignas(16) float Ta[BC][20];  // diag(beta) M, the operand of the MFMA inverse (16-byte rows)
  int exact;
};

// Fragment over row 16 nt + m of a tiled matrix, k running over columns
// 32 kb + koff(g, s): slots 0..3 come from tile (nt, 2 kb) and 4..7 from tile
// (nt, 2 kb + 1), lane m + 16 g in both, so each is one contiguous load per wave.
// TS: tile (r, t) starts at element (t * TS + r) * 256 (state_tile_index: TS = 8;
// row_tile_index, one row of tiles: TS = 1, nt = 0).
template <typename E, int TS, bool NT = false>
__device__ __forceinline__ typename Frag<E>::T tile_frag(const E* __restrict__ M, int nt, int kb, int lane) {
  typedef typename Vec4<E>::T V4;
  const V4* plo = reinterpret_cast<const V4*>(M + ((size_t)(2 * kb * TS + nt) * 64 + lane) * 4);
  const V4* phi = reinterpret_cast<const V4*>(M + ((size_t)((2 * kb + 1) * TS + nt) * 64 + lane) * 4);
  const V4 lo = NT ? load_nt(plo) : *plo;
  const V4 hi = NT ? load_nt(phi) : *phi;
  typename Frag<E>::T f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = lo[i];
    f[4 + i] = hi[i];
  }
  return f;
}

// Fragments over the chunk's rows (k < 16; slots 4..7, rows 16..31, are zero):
// A operand, row m: slot s = f(4 g + s); B operand, column m: slot s = f(4 g + s).
template <typename E, typename F>
__device__ __forceinline__ typename Frag<E>::T rows_frag(int g, F f) {
  typename Frag<E>::T x;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    x[s] = from_f<E>(f(4 * g + s));
    x[4 + s] = from_f<E>(0.f);
  }
  return x;
}

// The chunk inputs local_forward starts from, as this thread loads them (row RowMap(t).r,
// channels c0 .. c0 + 7; rows past len read the chunk's first row and are zeroed when
// stored; beta of row t < 16): loaded apart from their use, so that a kernel can issue
// them together with its other loads.
template <typename E>
struct LocalIn {
  typename Vec4<E>::T k[2], q[2];
  floatx4 la[2];
  float beta;
};
template <typename E>
__device__ __forceinline__ void local_load(LocalIn<E>& in, const E* __restrict__ q, const E* __restrict__ k,
                                           const float* __restrict__ log_alpha, const float* __restrict__ beta,
                                           int tok0, int len, int h, int H, int t) {
  typedef typename Vec4<E>::T V4;
  const size_t HD = (size_t)H * D;
  const RowMap rm(t);
  const size_t off = (size_t)tok0 * HD + (size_t)h * D + (size_t)(rm.r < len ? rm.r : 0) * HD + rm.c0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    in.k[u] = *reinterpret_cast<const V4*>(k + off + 4 * u);
    in.q[u] = *reinterpret_cast<const V4*>(q + off + 4 * u);
    in.la[u] = *reinterpret_cast<const floatx4*>(log_alpha + off + 4 * u);
  }
  in.beta = 0.f;
  if (t < BC && t < len) in.beta = beta[(size_t)(tok0 + t) * H + h];
}

// TM_IN: T and M are given (this thread's element (t / 16, t % 16) of each, as
// bwd_local_kernel stored them) and are put in LDS instead of being formed again.
template <typename E, bool WANT_P, typename KT, bool TM_IN = false>
__device__ void local_forward_in(LocalLds<KT>& L, const LocalIn<E>& in, int len, int t, float t_in = 0.f,
                                 float m_in = 0.f) {
  typedef typename Frag<E>::T FragT;
  const RowMap rm(t);
  const int lane = t & 63, w = t >> 6, m = lane & 15, g = lane >> 4;
  if constexpr (TM_IN) {
    L.T[t >> 4][t & 15] = t_in;
    L.M[t >> 4][t & 15] = m_in;
  }
  {
    const bool valid = rm.r < len;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = rm.c0 + 4 * u + i;
        L.K[rm.r][c] = valid ? from_f<KT>(to_f(in.k[u][i])) : from_f<KT>(0.f);
        L.Q[rm.r][c] = valid ? from_f<KT>(to_f(in.q[u][i])) : from_f<KT>(0.f);
        L.G[rm.r][c] = valid ? in.la[u][i] : 0.f;
      }
    if (t < BC) L.beta[t] = in.beta;
    if (t == 0) L.exact = 0;
  }
  __syncthreads();
  if (t < D) {  // cumulative log2 decay down the chunk, one channel per thread
    float run = 0.f, g0 = 0.f;
#pragma unroll
    for (int r = 0; r < BC; ++r) {
      run += L.G[r][t] * LOG2E_B;
      L.G[r][t] = run;
      if (r == 0) g0 = run;
    }
    L.bref[t] = 0.5f * (g0 + run);
    if (g0 - run > FACTOR_MAX_RANGE) L.exact = 1;
  }
  __syncthreads();
  if constexpr (TM_IN) return;
  if (!L.exact) {
    if (w == 0) {  // M (and P) as factored products over the 128 channels
      floatx4 pk = {0.f, 0.f, 0.f, 0.f}, pq = pk;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        FragT lk, rk, lq;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int ch = 32 * kb + koff(g, s);
          const float kv = to_f(L.K[m][ch]), d = L.G[m][ch] - L.bref[ch];
          lk[s] = from_f<E>(kv * exp2_hw(d));
          rk[s] = from_f<E>(kv * exp2_hw(-d));
          if constexpr (WANT_P) lq[s] = from_f<E>(to_f(L.Q[m][ch]) * exp2_hw(d));
        }
        mma(pk, lk, rk);  // lane (m, g): sum_ch Lk[4g+i][ch] Rk[m][ch]
        if constexpr (WANT_P) mma(pq, lq, rk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        L.M[r][m] = m < r ? pk[i] : 0.f;
        if constexpr (WANT_P) L.Pm[r][m] = m <= r ? pq[i] : 0.f;
      }
    }
  } else {
    float kr[8], qr[8], gr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kr[i] = to_f(L.K[rm.r][rm.ch(i)]);
      qr[i] = to_f(L.Q[rm.r][rm.ch(i)]);
      gr[i] = L.G[rm.r][rm.ch(i)];
    }
#pragma unroll
    for (int s = 0; s < BC; ++s) {
      float pk = 0.f, pq = 0.f;
      if (s <= rm.r) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float ks = to_f(L.K[s][rm.ch(i)]) * exp2_hw(gr[i] - L.G[s][rm.ch(i)]);  // exponent <= 0
          pk += kr[i] * ks;
          if constexpr (WANT_P) pq += qr[i] * ks;
        }
      }
      pk = sum16(pk);
      if constexpr (WANT_P) pq = sum16(pq);
      if ((t & 15) == 0) {
        L.M[rm.r][s] = s < rm.r ? pk : 0.f;
        if constexpr (WANT_P) L.Pm[rm.r][s] = s <= rm.r ? pq : 0.f;
      }
    }
  }
  __syncthreads();
  if constexpr (std::is_same<E, __bf16>::value) {
    // T = (I + A)^-1 by the power product on fp32 MFMA (kda_device.h), one wave: A =
    // diag(beta) M to Ta, then T from it in accumulator layout (lane (m, g) holds rows
    // 4 g .. 4 g + 3 of column m); the wave's LDS accesses run in order
    if (w == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) L.Ta[4 * g + i][m] = L.beta[4 * g + i] * L.M[4 * g + i][m];
      const floatx4 tb = unit_lower_inverse16(&L.Ta[0][0], 20, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) L.T[4 * g + i][m] = tb[i];
    }
  } else if (t < BC) {  // T = (I + A)^-1 by forward substitution, one column per thread, in registers
    const int cc = t;
    float tc[BC];
#pragma unroll
    for (int r = 0; r < BC; ++r) {
      float x = r == cc ? 1.f : 0.f;  // rows above cc stay exactly 0
#pragma unroll
      for (int s = 0; s < r; ++s) x -= L.beta[r] * L.M[r][s] * tc[s];
      tc[r] = x;
      L.T[r][cc] = x;
    }
  }
  __syncthreads();
}

template <typename E, bool WANT_P, typename KT>
__device__ void local_forward(LocalLds<KT>& L, const E* __restrict__ q, const E* __restrict__ k,
                              const float* __restrict__ log_alpha, const float* __restrict__ beta, int tok0, int len,
                              int h, int H, int t) {
  LocalIn<E> in;
  local_load(in, q, k, log_alpha, beta, tok0, len, h, H, t);
  local_forward_in<E, WANT_P>(L, in, len, t);
}

// ---------------------------------------------------------------------------
// bwd_local_kernel: the backward record of one (chunk, head), and the chunk's record
// for the forward state pass. W = T diag(beta) K e^G is one MFMA per 16-channel tile;
// its accumulator layout is the fragment order of the backward record, so W, Q e^G and
// P leave as one 8-byte store per lane and tile. The forward record takes W the other
// way round (the same MFMA with its operands swapped gives W^T, whose accumulator
// layout is the forward record's -W fragment), U = T diag(beta) V likewise in its
// accumulator order, and (K e^{g_C-G})^T as one lane's whole fragment slot.
// ---------------------------------------------------------------------------
template <typename E>
__global__ void __launch_bounds__(256) bwd_local_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                        const E* __restrict__ v,
                                                        const float* __restrict__ log_alpha,
                                                        const float* __restrict__ beta,
                                                        const int32_t* __restrict__ total_chunks,
                                                        const int2* __restrict__ info, int H, int mc,
                                                        char* __restrict__ brec, char* __restrict__ records,
                                                        float* __restrict__ tm) {
  using BR = BRec<E>;
  using RC = Rec<E, BC>;
  typedef typename Frag<E>::T FragT;
  typedef typename Vec4<E>::T V4;
  __shared__ LocalLds<E> L;
  const int c = blockIdx.x / H, h = blockIdx.x - c * H;
  if (c >= *total_chunks) return;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, m = lane & 15, g = lane >> 4;
  const int2 inf = info[c];
  const int tok0 = inf.x, len = inf.y;
  LocalIn<E> lin;
  local_load(lin, q, k, log_alpha, beta, tok0, len, h, H, t);
  // v as the B operand of U = T diag(beta) V for value tiles 2w and 2w + 1: lane (m, g)
  // takes rows 4g .. 4g + 3 of column 16 ct + m (rows past len zeroed where used),
  // issued after the local forward's loads so that its first wait does not wait for them
  E vv[2][4];
  {
    const size_t HD = (size_t)H * D;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 4 * g + s;
        vv[j][s] = v[(size_t)(tok0 + (r < len ? r : 0)) * HD + (size_t)h * D + 16 * (2 * w + j) + m];
      }
  }
  local_forward_in<E, true>(L, lin, len, t);
  {  // T and M for the gradient kernel, which would otherwise form them again
    float* tmc = tm + ((size_t)h * mc + c) * 2 * BC * BC;
    tmc[t] = L.T[t >> 4][t & 15];
    tmc[BC * BC + t] = L.M[t >> 4][t & 15];
  }

  char* rb = brec + ((size_t)h * mc + c) * BR::BYTES;
  E* wt = reinterpret_cast<E*>(rb + BR::WT);
  E* qtt = reinterpret_cast<E*>(rb + BR::QTT);
  E* kef = reinterpret_cast<E*>(rb + BR::KEF);
  const FragT ta = rows_frag<E>(g, [&](int u) { return L.T[m][u]; });  // A: row m of T
  FragT wf, qf;  // channel tiles 2w and 2w + 1, one piece per lane
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int nt = 2 * w + j, ch = 16 * nt + m;
    floatx4 wacc = {0.f, 0.f, 0.f, 0.f};
    mma(wacc, ta, rows_frag<E>(g, [&](int u) { return L.beta[u] * to_f(L.K[u][ch]) * exp2_hw(L.G[u][ch]); }));
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // element i: row 4g+i, channel ch
      const int r = 4 * g + i;
      const float gr = L.G[r][ch];
      wf[4 * j + i] = from_f<E>(-wacc[i]);
      qf[4 * j + i] = from_f<E>(to_f(L.Q[r][ch]) * exp2_hw(gr));
    }
  }
  store_frag<E>(wt + ((size_t)w * 64 + lane) * 8, wf);
  store_frag<E>(qtt + ((size_t)w * 64 + lane) * 8, qf);
  {  // K e^{g_C-G} as the A fragment of k-block w: lane (m, g) builds its whole slot (row
     // m, channels 32 w + koff(g, s)), so each wave writes 1 KiB contiguously
    FragT kf;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int ch = 32 * w + koff(g, s);
      kf[s] = from_f<E>(to_f(L.K[m][ch]) * exp2_hw(L.G[BC - 1][ch] - L.G[m][ch]));
    }
    store_frag<E>(kef + ((size_t)w * 64 + lane) * 8, kf);
  }
  if (w == 0) {
    V4 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = from_f<E>(L.Pm[4 * g + i][m]);
    *reinterpret_cast<V4*>(reinterpret_cast<E*>(rb + BR::PT) + (size_t)lane * 4) = pv;
  }
  // the forward state pass's record
  char* fb = records + ((size_t)h * mc + c) * RC::BYTES;
  E* fr = reinterpret_cast<E*>(fb);
  {
    FragT wn, ke[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ct = 2 * w + j, ch = 16 * ct + m;
      // W^T tile: lane (m, g), element i = W[row m][channel 16 ct + 4 g + i]
      floatx4 wt = {0.f, 0.f, 0.f, 0.f};
      mma(wt, rows_frag<E>(g, [&](int u) { return L.beta[u] * to_f(L.K[u][ch]) * exp2_hw(L.G[u][ch]); }), ta);
      // U tile: element i = U[row 4 g + i][value column 16 ct + m]
      FragT bv;  // B operand: slot s = beta_u V[u][16 ct + m], u = 4 g + s (k = 16..31 zero)
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const int u = 4 * g + s2;
        bv[s2] = from_f<E>(u < len ? L.beta[u] * to_f(vv[j][s2]) : 0.f);
        bv[4 + s2] = from_f<E>(0.f);
      }
      floatx4 uacc = {0.f, 0.f, 0.f, 0.f};
      mma(uacc, ta, bv);
      const float uo[4] = {uacc[0], uacc[1], uacc[2], uacc[3]};
      store4f(fr + RC::UU + ((size_t)ct * 64 + lane) * 4, uo);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wn[4 * j + i] = from_f<E>(-wt[i]);
        // (K e^{g_C-G})^T over channel tile ct: rows 4 g + i (rows 16.. of the k-block are zero)
        const int r = 4 * g + i;
        ke[j][i] = from_f<E>(to_f(L.K[r][ch]) * exp2_hw(L.G[BC - 1][ch] - L.G[r][ch]));
        ke[j][4 + i] = from_f<E>(0.f);
      }
      store_frag<E>(fr + RC::KE + ((size_t)ct * 64 + lane) * 8, ke[j]);
    }
    store_frag<E>(fr + RC::WN + ((size_t)w * 64 + lane) * 8, wn);  // k-block w: tiles 2w, 2w + 1
  }
  if (t < D) {
    const float gc = exp2_hw(L.G[BC - 1][t]);
    reinterpret_cast<float*>(rb + BR::GAM)[t] = gc;
    reinterpret_cast<float*>(fb + RC::GAMMA_BYTES)[t] = gc;
  }
}

// ---------------------------------------------------------------------------
// The reverse state pass (bwd_state_body): four waves per (sequence, head,
// 16-column slab), chunks in reverse. Wave w keeps dS rows 32w + 16j + 4g + i (j = 0, 1), column 16ct + m, in
// Lm[j], the layout whose pair is a B fragment over its 32 rows. Per chunk, wave w
// forms its k-block's part of dU~ = P^T dO + (K e^{g_C-G}) dS (P^T dO once, in wave
// 0), the parts are summed through LDS behind one barrier that leaves global loads
// in flight, and each wave updates its own rows. Work-group ids are dealt so that
// the eight slabs of a head share one XCD's L2. As in the forward pass, a fifth wave
// stores the per-chunk dS_C and dU~ from LDS, so that no compute wave waits on store
// acknowledgements when it waits for its next operands.
// ---------------------------------------------------------------------------
constexpr int STATE_TOUCH_AHEAD = 4;

template <typename E>
__device__ __forceinline__ void bwd_state_body(int b, const char* __restrict__ brec,
                                               const int32_t* __restrict__ chunk_off, const int2* __restrict__ info,
                                               const E* __restrict__ dout, const float* __restrict__ d_final,
                                               float* __restrict__ d_initial, E* __restrict__ dstates,
                                               E* __restrict__ dut, int N, int H, int mc) {
  using BR = BRec<E>;
  typedef typename Frag<E>::T FragT;
  typedef typename Vec4<E>::T V4;
  // four elements kept as raw 32-bit words while loading (packed bf16 vectors in a
  // struct otherwise end up in scratch)
  typedef unsigned int RawV __attribute__((ext_vector_type(sizeof(V4) / 4)));
  typedef unsigned int RawV2 __attribute__((ext_vector_type(2 * sizeof(V4) / 4)));
  __shared__ floatx4 xp[2][4][64];  // dU~ parts, by chunk parity
  // by chunk parity: dS at the chunk's end, tile rt (rows 16 rt ..) of the slab at
  // [rt][lane][4] in accumulator order (lane (m, g) holds rows 4g .. 4g+3 of column m),
  // and dU~ the same way
  __shared__ __attribute__((aligned(16))) E stg_s[2][8 * 64 * 4];
  __shared__ __attribute__((aligned(16))) E stg_u[2][64 * 4];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int xcd = b & 7, rest = b >> 3;
  const int ct = rest & 7, slot = rest >> 3;
  const int u = slot * 8 + xcd;
  if (u >= N * H) return;  // uniform over the work-group
  const int n = u / H, h = u - n * H;
  const size_t HD = (size_t)H * D;
  const int c_begin = chunk_off[n], c_end = chunk_off[n + 1];

  if (w == 4) {
    // the store wave: one barrier per chunk, as the compute waves, and one after the
    // last. After the barrier of the chunk i-th from the end, that chunk's dS_C and the
    // dU~ of the chunk after it are in LDS until the next barrier but one. For dU~
    // lane (m, g) stores row m, columns 16 ct + 4 g .. + 3, reading the four values
    // from lanes 4 g .. 4 g + 3, slot m % 4, of the accumulator order.
    auto gather = [&](const E* tile) {
      V4 x;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) x[s4] = tile[(4 * g + s4 + 16 * (m >> 2)) * 4 + (m & 3)];
      return x;
    };
    E* dut_h = dut + (size_t)h * mc * BC * D + ((size_t)ct * 64 + lane) * 4;
    for (int i = 0; c_end - 1 - i >= c_begin; ++i) {
      lds_barrier();
      const int c = c_end - 1 - i;
      store_state_slab(dstates + ((size_t)h * mc + c) * D * D + (size_t)ct * 2048, stg_s[i & 1], lane);
      if (i > 0) store_nt(reinterpret_cast<V4*>(dut_h + (size_t)(c + 1) * BC * D), gather(stg_u[(i - 1) & 1]));
    }
    lds_barrier();
    if (c_end > c_begin)
      store_nt(reinterpret_cast<V4*>(dut_h + (size_t)c_begin * BC * D), gather(stg_u[(c_end - c_begin - 1) & 1]));
    return;
  }

  const size_t sbase = (size_t)u * D * D + (size_t)(32 * w + 4 * g) * D + 16 * ct + m;
  // first token and end of the sequence: chunk c starts at seq_t0 + (c - c_begin) BC
  int seq_t0 = 0, seq_t1 = 0;
  if (c_end > c_begin) {
    const int2 first = info[c_begin], last = info[c_end - 1];
    seq_t0 = first.x;
    seq_t1 = last.x + last.y;
  }

  floatx4 Lm[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    Lm[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (d_final) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Lm[j][i] = d_final[sbase + (size_t)(16 * j + i) * D];
    }
  }
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // slots 0..3 from a 4-vector, slots 4..7 (chunk rows 16..31) zero
  auto half_frag = [](const RawV& raw) {
    const V4 x = __builtin_bit_cast(V4, raw);
    FragT f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f[s] = x[s];
      f[4 + s] = from_f<E>(0.f);
    }
    return f;
  };

  // a stage holds what the loads return (four elements as raw 32-bit words):
  // building fragments at load time would make the wave wait for the data one step
  // early; they are built where they are used. grad_o comes as one 4-element piece
  // per lane, row lane / 4, columns 16 ct + 4 (lane % 4) .. + 3, and is regrouped
  // into the fragment's columns by lane permutes (four scalar loads per lane, one per
  // row, cost a sixth of the kernel's time).
  constexpr int RW = (int)(sizeof(V4) / 4);
  struct Stage {
    unsigned wt[2][RW], qt[2][RW], pt[RW], dow[RW];
    FragT ke;
    float gw;  // e^{g_C} of row 32w + row_word_index(m, g)
  };
  auto raw_frag = [&](const unsigned* r) {
    RawV x;
#pragma unroll
    for (int i = 0; i < RW; ++i) x[i] = r[i];
    return half_frag(x);
  };
  auto load = [&](Stage& st, int c) {
    const char* rb = brec + ((size_t)h * mc + c) * BR::BYTES;
    const E* wt = reinterpret_cast<const E*>(rb + BR::WT);
    const E* qt = reinterpret_cast<const E*>(rb + BR::QTT);
    {  // channel tiles 2w and 2w + 1: one piece per lane
      const RawV2 a = *reinterpret_cast<const RawV2*>(wt + ((size_t)w * 64 + lane) * 8);
      const RawV2 q = *reinterpret_cast<const RawV2*>(qt + ((size_t)w * 64 + lane) * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < RW; ++i) {
          st.wt[j][i] = a[j * RW + i];
          st.qt[j][i] = q[j * RW + i];
        }
    }
    st.ke = load_frag<E>(reinterpret_cast<const E*>(rb + BR::KEF) + ((size_t)w * 64 + lane) * 8);
    if (w == 0) {  // P^T dO is formed by wave 0 only (w is uniform over the wave)
      const RawV p4 = *reinterpret_cast<const RawV*>(reinterpret_cast<const E*>(rb + BR::PT) + (size_t)lane * 4);
#pragma unroll
      for (int i = 0; i < RW; ++i) st.pt[i] = p4[i];
    }
    const float* gam = reinterpret_cast<const float*>(rb + BR::GAM);
    st.gw = gam[32 * w + row_word_index(m, g)];
    // the chunk's tokens follow from the sequence's (no address waits on a load);
    // rows past len read row 0 and are zeroed
    const int tok0 = seq_t0 + (c - c_begin) * BC, len = min(BC, seq_t1 - tok0);
    const int r = lane >> 2;
    const RawV d = *reinterpret_cast<const RawV*>(dout + (size_t)(tok0 + (r < len ? r : 0)) * HD + (size_t)h * D +
                                                  16 * ct + 4 * (lane & 3));
#pragma unroll
    for (int i = 0; i < RW; ++i) st.dow[i] = r < len ? d[i] : 0u;
  };

  // B fragment of dO over the chunk rows: lane (m, g) takes row 4g + s, column m from
  // lane (4g + s) * 4 + m / 4, element m % 4 (all 64 lanes active)
  auto do_frag = [&](const Stage& st) {
    FragT f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int src = ((4 * g + s) * 4 + (m >> 2)) * 4;  // byte address of the source lane
      unsigned v[RW];
#pragma unroll
      for (int i = 0; i < RW; ++i) v[i] = (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)st.dow[i]);
      if constexpr (RW == 2) {  // bf16: two elements per word
        const unsigned wd = (m & 2) ? v[1] : v[0];
        f[s] = __builtin_bit_cast(E, (unsigned short)((m & 1) ? (wd >> 16) : (wd & 0xffffu)));
      } else {
        const unsigned lo = (m & 1) ? v[1] : v[0], hi = (m & 1) ? v[3] : v[2];
        f[s] = __builtin_bit_cast(E, (m & 2) ? hi : lo);
      }
      f[4 + s] = from_f<E>(0.f);
    }
    return f;
  };
  // the dO fragment of the chunk computed next, permuted one chunk early (after the
  // barrier of the chunk before it), where its latency overlaps that chunk's work
  FragT dOn;

  auto compute = [&](const Stage& st, int c, int buf, const Stage& nx) {
    const FragT dOb = dOn;
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // this wave's two tiles of the gradient at the chunk's end, to LDS
      V4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = from_f<E>(Lm[j][i]);
      *reinterpret_cast<V4*>(&stg_s[buf][((2 * w + j) * 64 + lane) * 4]) = x;
    }
    // this wave's part of dU~ = P^T dO + (K e^{g_C-G}) dS
    floatx4 dp4 = zero4;
    if (w == 0) mma(dp4, raw_frag(st.pt), dOb);
    mma(dp4, st.ke, acc_pair_to_frag<E>(Lm[0], Lm[1]));
    xp[buf][w][lane] = dp4;
    lds_barrier();
    dOn = do_frag(nx);
    const floatx4 du = xp[buf][0][lane] + xp[buf][1][lane] + xp[buf][2][lane] + xp[buf][3][lane];
    if (w == 0) {  // dU~ to LDS, for the store wave after the next barrier
      V4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = from_f<E>(du[i]);
      *reinterpret_cast<V4*>(&stg_u[buf][lane * 4]) = x;
    }
    const FragT dUb = acc_pair_to_frag<E>(du, zero4);
    // dS0_w = e^{g_C} o dS_w + (Q e^G)^T_w dO + (-W)^T_w dU~
    floatx4 gm[2];
    rows_from_word(st.gw, m, gm);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      Lm[j] = gm[j] * Lm[j];
      mma(Lm[j], raw_frag(st.qt[j]), dOb);
      mma(Lm[j], raw_frag(st.wt[j]), dUb);
    }
  };

  // L2 touch STATE_TOUCH_AHEAD chunks beyond the register stage: each line of the
  // record and of the chunk's grad_o rows is read (one word) by one of the head's 32
  // waves, so the real loads hit in L2 (the words are XOR-folded into tacc, stored
  // only by a never-taken branch). No address here depends on a load: that would make
  // the wave wait.
  constexpr int LINES = (int)(BR::BYTES / 128);
  constexpr int ROW_LINES = D * (int)sizeof(E) / 128;  // lines of one grad_o row of a head
  constexpr int DO_PER_WAVE = BC * ROW_LINES / 32;     // grad_o lines each wave touches
  static_assert(BR::BYTES % 128 == 0 && LINES <= 32 * (64 - DO_PER_WAVE), "one touch per lane");
  // the last DO_PER_WAVE lanes touch grad_o; lanes past the record's last line touch
  // that line again (an unconditional load is never merged with an old value)
  const int do_line = (ct * 4 + w) * DO_PER_WAVE + (63 - lane);
  const bool touch_do = lane >= 64 - DO_PER_WAVE;
  const int touch_line = min((ct * 4 + w) + 32 * lane, LINES - 1);
  unsigned tacc = 0u;
  auto touch = [&](int c) {
    const int tok0 = seq_t0 + (c - c_begin) * BC, len = min(BC, seq_t1 - tok0);
    const int r = do_line / ROW_LINES;
    const unsigned* p =
        touch_do ? reinterpret_cast<const unsigned*>(dout + (size_t)(tok0 + (r < len ? r : 0)) * HD + (size_t)h * D +
                                                     (do_line % ROW_LINES) * (128 / (int)sizeof(E)))
                 : reinterpret_cast<const unsigned*>(brec + ((size_t)h * mc + c) * BR::BYTES +
                                                     (size_t)touch_line * 128);
    return *p;
  };

  // four named stages, three chunks of operands in flight: step r of an iteration
  // loads chunk c - 3 into the stage consumed one step earlier (past the start, the
  // first chunk again: every step issues the same loads)
  Stage sa, sb, sc, sd;
  if (c_begin < c_end) {
    load(sa, c_end - 1);
    load(sb, max(c_end - 2, c_begin));
    load(sc, max(c_end - 3, c_begin));
    dOn = do_frag(sa);
  }
  for (int c0 = c_end - 1; c0 >= c_begin; c0 -= 4) {
    // the iteration's four chunks: the first step touches the four beyond the touch
    // distance; the words are folded in after the last step (none lives across the
    // back edge, where a register copy would wait for it)
    load(sd, max(c0 - 3, c_begin));
    const unsigned t0 = touch(max(c0 - 3 - STATE_TOUCH_AHEAD, c_begin));
    const unsigned t1 = touch(max(c0 - 4 - STATE_TOUCH_AHEAD, c_begin));
    const unsigned t2 = touch(max(c0 - 5 - STATE_TOUCH_AHEAD, c_begin));
    const unsigned t3 = touch(max(c0 - 6 - STATE_TOUCH_AHEAD, c_begin));
    compute(sa, c0, 0, sb);
    load(sa, max(c0 - 4, c_begin));
    if (c0 - 1 >= c_begin) compute(sb, c0 - 1, 1, sc);
    load(sb, max(c0 - 5, c_begin));
    if (c0 - 2 >= c_begin) compute(sc, c0 - 2, 0, sd);
    load(sc, max(c0 - 6, c_begin));
    if (c0 - 3 >= c_begin) compute(sd, c0 - 3, 1, sa);
    tacc ^= t0 ^ t1 ^ t2 ^ t3;
  }
  lds_barrier();  // the store wave's last one: dU~ of the first chunk
  // mc is never negative (the host sizes it from the shapes), so this never stores
  if (mc < 0 && tacc == 0u) dut[lane] = from_f<E>(0.f);
  if (d_initial) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) d_initial[sbase + (size_t)(16 * j + i) * D] = Lm[j][i];
  }
}

// The two serial state passes run as separate launches, one work-group per CU each.
// Run side by side in one launch (one work-group of each per CU) they take longer
// than one after the other: each already saturates a per-CU resource.
template <typename E>
__global__ void __launch_bounds__(320) fwd_state_kernel(const char* __restrict__ records,
                                                        const int32_t* __restrict__ chunk_off,
                                                        const int2* __restrict__ info,
                                                        const float* __restrict__ initial_state, int N, int H, int mc,
                                                        E* __restrict__ states, E* __restrict__ ut) {
  inter16_body<E, false>(blockIdx.x, records, chunk_off, info, initial_state, nullptr, nullptr, N, H, mc, states,
                         ut);
}

template <typename E>
__global__ void __launch_bounds__(320) bwd_state_kernel(const char* __restrict__ brec,
                                                        const int32_t* __restrict__ chunk_off,
                                                        const int2* __restrict__ info, const E* __restrict__ dout,
                                                        const float* __restrict__ d_final,
                                                        float* __restrict__ d_initial, E* __restrict__ dstates,
                                                        E* __restrict__ dut, int N, int H, int mc) {
  bwd_state_body<E>(blockIdx.x, brec, chunk_off, info, dout, d_final, d_initial, dstates, dut, N, H, mc);
}

// ---------------------------------------------------------------------------
// bwd_chunk_kernel: the gradients of one (chunk, head). After the state products,
// wave w owns channels 32 w .. 32 w + 31 (two 16-channel tiles) and works in the
// MFMA accumulator layout: lane (m, g), element i is row 4 g + i, channel 16 nt + m.
// dB_K = T^T dW, dB_V = T^T dU and the four decay-weighted sums over the chunk's
// rows are MFMAs on factored operands (element-wise on the exact path).
// ---------------------------------------------------------------------------
struct ChunkLds {
  LocalLds<float> L;
  float V[BC][LDP];
  float dU[BC][LDP];  // dU~
  float X2[BC][LDP];  // dU~ S0^T
  float dP[BC][LDS16], dT[BC][LDS16], dA[BC][LDS16];
  float dTp[4][BC][LDS16];
  float dgam[D];
  float dbp[4][BC];
};

template <typename E>
__device__ __forceinline__ typename Frag<E>::T zero_frag() {
  typename Frag<E>::T f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = from_f<E>(0.f);
  return f;
}

template <typename E>
__global__ void __launch_bounds__(256, 2) bwd_chunk_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, const E* __restrict__ dout, const E* __restrict__ states,
    const E* __restrict__ dstates, const E* __restrict__ ut, const E* __restrict__ dut,
    const float* __restrict__ tm, const int32_t* __restrict__ total_chunks, const int2* __restrict__ info, int H,
    int mc, E* __restrict__ dq,
    E* __restrict__ dk, E* __restrict__ dv, float* __restrict__ dlog_alpha, float* __restrict__ dbeta) {
  typedef typename Frag<E>::T FragT;
  __shared__ ChunkLds S;
  LocalLds<float>& L = S.L;
  const int c = blockIdx.x / H, h = blockIdx.x - c * H;
  if (c >= *total_chunks) return;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, m = lane & 15, g = lane >> 4;
  const int2 inf = info[c];
  const int tok0 = inf.x, len = inf.y;
  const size_t HD = (size_t)H * D;
  const size_t rowbase = (size_t)tok0 * HD + (size_t)h * D;
  const size_t cix = (size_t)h * mc + c;
  const E* S0 = states + cix * D * D;
  const E* dSC = dstates + cix * D * D;
  const E* Ut = ut + cix * BC * D;
  const E* dUt = dut + cix * BC * D;
  const RowMap rm(t);

  // Every global load of the chunk is issued here, before anything waits for one: the
  // local forward's inputs, the v and dU~ rows, and (bf16: they fit in registers) the
  // operands of the state products, so the chunk pays one memory latency, not three.
  // (raw loads, converted where they are stored: a conversion next to its load would
  // wait for it, and for every load issued before it)
  typedef typename Vec4<E>::T V4;
  LocalIn<E> lin;
  local_load(lin, q, k, log_alpha, beta, tok0, len, h, H, t);
  const float t_in = tm[cix * 2 * BC * BC + t], m_in = tm[cix * 2 * BC * BC + BC * BC + t];  // T, M (bwd_local)
  V4 xv[2], xdu[2];
  {
    const size_t vo = rowbase + (size_t)(rm.r < len ? rm.r : 0) * HD + rm.c0;  // rows past len zeroed below
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      xv[u] = *reinterpret_cast<const V4*>(v + vo + 4 * u);
      xdu[u] = *reinterpret_cast<const V4*>(dUt + row_tile_index(rm.r, rm.c0 + 4 * u));
    }
  }
  constexpr bool HOIST = std::is_same<E, __bf16>::value;
  // state-product operands: rows of dO, U~ and dU~ (A), and the 16 x 16 tiles of S0 and
  // dS_C over row 16 nt + m, columns 32 kb + koff(g, s) (B; tiles (nt, 2 kb), (nt, 2 kb + 1))
  FragT a1[4], a2[4], a3[4], bsf[2][4], bdf[2][4];
  auto load_ops = [&] {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      a1[kb] = m < len ? frag_rowk<E>(dout + rowbase, (int)HD, m, 32 * kb, g) : zero_frag<E>();
      a2[kb] = tile_frag<E, 1>(dUt, 0, kb, lane);
      a3[kb] = tile_frag<E, 1>(Ut, 0, kb, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bsf[j][kb] = tile_frag<E, 8, true>(S0, 2 * w + j, kb, lane);
        bdf[j][kb] = tile_frag<E, 8, true>(dSC, 2 * w + j, kb, lane);
      }
    }
  };
  if constexpr (HOIST) load_ops();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    S.V[rm.r][rm.c0 + i] = rm.r < len ? to_f(xv[i >> 2][i & 3]) : 0.f;
    S.dU[rm.r][rm.c0 + i] = to_f(xdu[i >> 2][i & 3]);
  }
  local_forward_in<E, false, float, true>(L, lin, len, t, t_in, m_in);

  // ---- state products: wave w forms channel tiles 2w and 2w+1 of
  //      X1 = dO S0^T, X2 = dU~ S0^T, X3 = U~ dS_C^T, and dgamma = rowsum(dS_C o S0)
  floatx4 x1r[2], x3r[2];
  {
    if constexpr (!HOIST) load_ops();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nt = 2 * w + j;
      floatx4 x1 = {0.f, 0.f, 0.f, 0.f}, x2 = x1, x3 = x1;
      float dg = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const FragT bs = bsf[j][kb];
        const FragT bd = bdf[j][kb];
        mma(x1, a1[kb], bs);
        mma(x2, a2[kb], bs);
        mma(x3, a3[kb], bd);
#pragma unroll
        for (int s = 0; s < 8; ++s) dg += to_f(bs[s]) * to_f(bd[s]);
      }
      dg = xor32_sum(xor16_sum(dg));
      if (g == 0) S.dgam[16 * nt + m] = dg;
      x1r[j] = x1;
      x3r[j] = x3;
#pragma unroll
      for (int i = 0; i < 4; ++i) S.X2[4 * g + i][16 * nt + m] = x2[i];
    }
    if (w == 0) {  // dP = tril(dO U~^T)
      floatx4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(p, a1[kb], tile_frag<E, 1>(Ut, 0, kb, lane));
#pragma unroll
      for (int i = 0; i < 4; ++i) S.dP[4 * g + i][m] = m <= 4 * g + i ? p[i] : 0.f;
    }
  }
  __syncthreads();

  // ---- dT = (dW (K e^G)^T + dU V^T) diag(beta), dW = -X2: wave w sums channels
  //      32w .. 32w+31 (one MFMA pair), the four partials are added below
  {
    FragT ax, bk, au, bv;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int ch = 32 * w + koff(g, s);
      ax[s] = from_f<E>(-S.X2[m][ch]);
      bk[s] = from_f<E>(to_f(L.K[m][ch]) * exp2_hw(L.G[m][ch]));
      au[s] = from_f<E>(S.dU[m][ch]);
      bv[s] = from_f<E>(S.V[m][ch]);
    }
    floatx4 p = {0.f, 0.f, 0.f, 0.f};
    mma(p, ax, bk);
    mma(p, au, bv);
#pragma unroll
    for (int i = 0; i < 4; ++i) S.dTp[w][4 * g + i][m] = p[i];
  }
  __syncthreads();
  {
    const int r = t >> 4, s = t & 15;
    const float a = S.dTp[0][r][s] + S.dTp[1][r][s] + S.dTp[2][r][s] + S.dTp[3][r][s];
    S.dT[r][s] = s < r ? a * L.beta[s] : 0.f;  // only the strictly lower part of T varies
  }
  __syncthreads();
  // ---- dA = -T^T dT T^T, strictly lower: Y = dT T^T into dA, then -T^T Y into dT --
  {
    const int r = t >> 4, s = t & 15;
    float y = 0.f;
#pragma unroll
    for (int u = 0; u < BC; ++u) y += S.dT[r][u] * L.T[s][u];
    S.dA[r][s] = y;
  }
  __syncthreads();
  {
    const int r = t >> 4, s = t & 15;
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < BC; ++u) a -= L.T[u][r] * S.dA[u][s];
    __syncthreads();
    S.dT[r][s] = s < r ? a : 0.f;  // dT now holds dA
  }
  __syncthreads();

  // ---- per element (row 4g+i, channel 16nt+m): dq, dk, dv, dG, dbeta partials ----
  const bool exact = L.exact != 0;
  const FragT aTt = rows_frag<E>(g, [&](int u) { return L.T[u][m]; });                   // T^T, row m
  const FragT adA = rows_frag<E>(g, [&](int u) { return S.dT[m][u]; });                  // dA
  const FragT adAt = rows_frag<E>(g, [&](int u) { return L.beta[u] * S.dT[u][m]; });     // (diag(beta) dA)^T
  const FragT adP = rows_frag<E>(g, [&](int u) { return S.dP[m][u]; });                  // dP
  const FragT adPt = rows_frag<E>(g, [&](int u) { return S.dP[u][m]; });                 // dP^T
  float dbr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ch = 16 * (2 * w + j) + m;
    const float bch = L.bref[ch];
    floatx4 dbk = {0.f, 0.f, 0.f, 0.f}, dbv = dbk, ra = dbk, rp = dbk, rat = dbk, rpt = dbk;
    mma(dbk, aTt, rows_frag<E>(g, [&](int u) { return S.X2[u][ch]; }));  // T^T X2 = -dB_K
    mma(dbv, aTt, rows_frag<E>(g, [&](int u) { return S.dU[u][ch]; }));  // T^T dU = dB_V
    if (!exact) {
      const FragT brk = rows_frag<E>(g, [&](int u) { return to_f(L.K[u][ch]) * exp2_hw(bch - L.G[u][ch]); });
      mma(ra, adA, brk);
      mma(rp, adP, brk);
      mma(rat, adAt, rows_frag<E>(g, [&](int u) { return to_f(L.K[u][ch]) * exp2_hw(L.G[u][ch] - bch); }));
      mma(rpt, adPt, rows_frag<E>(g, [&](int u) { return to_f(L.Q[u][ch]) * exp2_hw(L.G[u][ch] - bch); }));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = L.G[4 * g + i][ch] - bch;
        const float lr = exp2_hw(d), rr = exp2_hw(-d);
        ra[i] *= lr;
        rp[i] *= lr;
        rat[i] *= rr;
        rpt[i] *= rr;
      }
    } else {
      // T, dA strictly lower and dP lower: row u < r only feeds the sums along row r,
      // row u > r only those down column r, both weighted 2^-|G_r - G_u|
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        const float gr = L.G[r][ch];
        for (int u = 0; u < BC; ++u) {
          const float f = exp2_hw(-fabsf(gr - L.G[u][ch]));
          const float ku = to_f(L.K[u][ch]) * f;
          ra[i] += S.dT[r][u] * ku;
          rp[i] += S.dP[r][u] * ku;
          rat[i] += L.beta[u] * S.dT[u][r] * ku;
          rpt[i] += S.dP[u][r] * to_f(L.Q[u][ch]) * f;
        }
      }
    }
    const float gl = L.G[BC - 1][ch];
    float dgr[4], kexs = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      const float gr = L.G[r][ch], er = exp2_hw(gr), el = exp2_hw(gl - gr);
      const float kr = to_f(L.K[r][ch]), qr = to_f(L.Q[r][ch]), br = L.beta[r];
      const float bk_ = -dbk[i], bv_ = dbv[i], x1 = x1r[j][i], x3 = x3r[j][i];
      const float dqv = x1 * er + rp[i];
      const float dkv = br * bk_ * er + br * ra[i] + rat[i] + rpt[i] + x3 * el;
      const float kex = x3 * kr * el;
      dgr[i] = x1 * qr * er + rp[i] * qr + br * bk_ * kr * er + br * ra[i] * kr - rat[i] * kr - rpt[i] * kr - kex;
      dbr[i] += bk_ * kr * er + bv_ * S.V[r][ch];
      kexs += kex;
      if (r < len) {
        const size_t o = rowbase + (size_t)r * HD + ch;
        dq[o] = from_f<E>(dqv);
        dk[o] = from_f<E>(dkv);
        dv[o] = from_f<E>(br * bv_);
      }
    }
    // dlog_alpha = reverse cumulative sum of dG over the rows (4 per lane, lanes
    // m + 16 g in order), plus the terms of g_C (the last row): sum_r K e^{g_C-G}
    // terms and dgamma e^{g_C}, which every row's sum includes
    const float blk = dgr[0] + dgr[1] + dgr[2] + dgr[3];
    kexs = xor32_sum(xor16_sum(kexs));
    // the row blocks below this lane's (lanes m + 16 gg, gg > g), by lane swaps: the
    // other row of this row's pair, then the other pair's sum
    float above;
    {
      const unsigned u = __float_as_uint(blk);
      const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // rows 2p, 2p + 1
      const float e0 = __uint_as_float(r16[0]), e1 = __uint_as_float(r16[1]);
      const unsigned ps = __float_as_uint(e0 + e1);
      const auto r32 = __builtin_amdgcn_permlane32_swap(ps, ps, false, false);  // pairs 0 and 1
      above = ((g & 1) ? 0.f : e1) + (g < 2 ? __uint_as_float(r32[1]) : 0.f);
    }
    float run = above + kexs + S.dgam[ch] * exp2_hw(gl);
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      run += dgr[i];
      const int r = 4 * g + i;
      if (r < len) dlog_alpha[rowbase + (size_t)r * HD + ch] = run;
    }
  }
  // dbeta = sum over channels of (dB_K o K e^G + dB_V o V) + sum_s dA_rs M_rs
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = row16_sum(dbr[i]);
    if (m == 0) S.dbp[w][4 * g + i] = x;
  }
  __syncthreads();
  if (t < len) {
    float am = 0.f;
    for (int s = 0; s < t; ++s) am += S.dT[t][s] * L.M[t][s];
    dbeta[(size_t)(tok0 + t) * H + h] = S.dbp[0][t] + S.dbp[1][t] + S.dbp[2][t] + S.dbp[3][t] + am;
  }
}

}  // namespace

size_t backward_record_bytes(int dtype) { return dtype == 0 ? BRec<__bf16>::BYTES : BRec<float>::BYTES; }

BackwardWs backward_ws_layout(int B, int T, int H, int num_seqs, bool varlen, int dtype) {
  const int64_t mc = max_chunks(B, T, num_seqs, varlen, BC);
  const size_t es = dtype == 0 ? 2 : 4;
  BackwardWs l;
  l.fwd = prefill_ws_layout(B, T, H, num_seqs, varlen, BC, dtype);
  l.off_brec = bal256(l.fwd.total);
  l.off_states = l.off_brec + (size_t)mc * H * backward_record_bytes(dtype);
  l.off_dstates = l.off_states + bal256((size_t)mc * H * D * D * es);
  l.off_ut = l.off_dstates + bal256((size_t)mc * H * D * D * es);
  l.off_dut = l.off_ut + bal256((size_t)mc * H * BC * D * es);
  l.off_tm = l.off_dut + bal256((size_t)mc * H * BC * D * es);
  l.total = l.off_tm + bal256((size_t)mc * H * 2 * BC * BC * sizeof(float));
  return l;
}

namespace {
template <typename E>
hipError_t launch_backward_typed(const void* q, const void* k, const void* v, const float* log_alpha,
                                 const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                                 int num_seqs, const void* dout, const float* d_final, void* dq, void* dk, void* dv,
                                 float* dlog_alpha, float* dbeta, float* d_initial, int B, int T, int H,
                                 void* workspace, hipStream_t stream) {
  const bool varlen = cu_seqlens != nullptr;
  const int N = varlen ? num_seqs : B;
  const int64_t mc = max_chunks(B, T, num_seqs, varlen, BC);
  const BackwardWs l = backward_ws_layout(B, T, H, num_seqs, varlen, std::is_same<E, float>::value ? 1 : 0);
  char* ws = reinterpret_cast<char*>(workspace);
  const int32_t* chunk_off = reinterpret_cast<const int32_t*>(ws + l.fwd.off_chunk_off);
  const int2* info = reinterpret_cast<const int2*>(ws + l.fwd.off_info);
  char* brec = ws + l.off_brec;
  E* states = reinterpret_cast<E*>(ws + l.off_states);
  E* dstates = reinterpret_cast<E*>(ws + l.off_dstates);
  E* ut = reinterpret_cast<E*>(ws + l.off_ut);
  E* dut = reinterpret_cast<E*>(ws + l.off_dut);
  float* tm = reinterpret_cast<float*>(ws + l.off_tm);
  trace_begin(stream);
  hipError_t e = launch_plan(cu_seqlens, N, T, varlen ? T : N * T, BC, mc,
                             reinterpret_cast<int32_t*>(ws + l.fwd.off_chunk_off),
                             reinterpret_cast<int2*>(ws + l.fwd.off_info), stream);
  trace_mark(stream, 0);
  if (e != hipSuccess) return e;
  char* records = ws + l.fwd.off_records;
  if (mc > 0) {
    hipLaunchKernelGGL(bwd_local_kernel<E>, dim3((unsigned)(mc * H)), dim3(256), 0, stream, (const E*)q,
                       (const E*)k, (const E*)v, log_alpha, beta, chunk_off + N, info, H, (int)mc, brec, records,
                       tm);
    e = hipGetLastError();
    trace_mark(stream, 5);
    if (e != hipSuccess) return e;
  }
  const int64_t slots = ((int64_t)N * H + 7) / 8;
  if (slots > 0) {
    hipLaunchKernelGGL(fwd_state_kernel<E>, dim3((unsigned)(slots * 64)), dim3(320), 0, stream, records, chunk_off,
                       info, initial_state, N, H, (int)mc, states, ut);
    e = hipGetLastError();
    trace_mark(stream, 2);
    if (e != hipSuccess) return e;
  }
  if (slots > 0) {
    hipLaunchKernelGGL(bwd_state_kernel<E>, dim3((unsigned)(slots * 64)), dim3(320), 0, stream, brec, chunk_off,
                       info, (const E*)dout, d_final, d_initial, dstates, dut, N, H, (int)mc);
    e = hipGetLastError();
    trace_mark(stream, 6);
    if (e != hipSuccess) return e;
  }
  if (mc > 0) {
    hipLaunchKernelGGL(bwd_chunk_kernel<E>, dim3((unsigned)(mc * H)), dim3(256), 0, stream, (const E*)q,
                       (const E*)k, (const E*)v, log_alpha, beta, (const E*)dout, states, dstates, ut, dut, tm,
                       chunk_off + N, info, H, (int)mc, (E*)dq, (E*)dk, (E*)dv, dlog_alpha, dbeta);
    e = hipGetLastError();
    trace_mark(stream, 7);
  }
  return e;
}
}  // namespace

size_t backward_workspace_bytes(int B, int T, int H, int num_seqs, bool varlen, int dtype) {
  return backward_ws_layout(B, T, H, num_seqs, varlen, dtype).total;
}

hipError_t launch_backward(int dtype, const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                           const void* dout, const float* d_final, void* dq, void* dk, void* dv, float* dlog_alpha,
                           float* dbeta, float* d_initial, int B, int T, int H, void* workspace,
                           hipStream_t stream) {
  if (dtype == 0)
    return launch_backward_typed<__bf16>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, dout,
                                         d_final, dq, dk, dv, dlog_alpha, dbeta, d_initial, B, T, H, workspace,
                                         stream);
  return launch_backward_typed<float>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, dout, d_final,
                                      dq, dk, dv, dlog_alpha, dbeta, d_initial, B, T, H, workspace, stream);
}

}  // namespace kda
