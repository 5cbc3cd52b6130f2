// Backward pass of the KDA chunk form on gfx950: gradients of
//     L = sum_t <o_t, do_t> + sum_n <S_final[n], dS_final[n]>
// with respect to q, k, v, log_alpha, beta and the initial state. The pages present
// the chunked WY / UT form as what makes KDA efficient to train ("From GPT-2 to Kimi
// K3" digest, section on chunked computation; GeekNews "Kimi Linear" summary,
// section "청크 단위 병렬화"); these are the derivatives of that map.
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
//   the forward at 16-token chunks (plan, intra_kernel, inter_kernel) keeping, per
//     (head, chunk), the state entering the chunk and U~;
//   bwd_local_kernel   one work-group per (chunk, head): W, Q e^G, K e^{g_C-G}, P and
//                      e^{g_C} in plain row-major form;
//   bwd_state_kernel   one wave per (sequence, head, 16-column slab), serial over the
//                      chunks in reverse, the 128 x 16 fp32 slab of the state
//                      gradient in accumulator registers: keeps dS_C and dU~ per chunk,
//                      writes the initial-state gradient;
//   bwd_chunk_kernel   one work-group per (chunk, head): everything local to the
//                      chunk. X1, X2, X3 and dgamma are bf16 (or fp32) MFMA products
//                      whose operands come straight from row-major global memory; the
//                      16 x 16 matrices and the decay-weighted sums run on the VALU in
//                      fp32.
// In-chunk decays are evaluated per element as 2^(g_r - g_s) with r >= s, so every
// exponent is <= 0 for any input that meets the log_alpha <= 0 precondition: no
// factoring or overflow guard is needed at 16 rows.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int BC = BWD_CHUNK;
static_assert(BC == 16, "the backward kernels are written for 16-token chunks");
constexpr int LDP = D;  // row stride of the fp32 [16][128] LDS matrices (see RowMap)
constexpr int LDS16 = BC + 1;
constexpr float LOG2E_B = 1.4426950408889634f;

__host__ __device__ constexpr size_t bal256(size_t x) { return (x + 255) & ~(size_t)255; }

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// sum over the 16 lanes l with equal l >> 4 (one row of the element-wise phases)
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 1);
  return x;
}

// Per-(head, chunk) record for the reverse state pass, in the MFMA operand order
// bwd_state_kernel consumes (lane l = m + 16 g; the fragment convention of
// kda_device.h, chunk rows padded to 32 with zeros):
//   WT   [8 rt][64][4]  slot s of the A fragment of (-W)^T, channel tile rt: -W[4g+s][16rt+m]
//   QTT  [8 rt][64][4]  the same for (Q e^G)^T
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

// (row, channel) of a 16 x 128 chunk matrix -> element index in the A fragment of its
// transpose (tile rt = channel / 16: lane (channel % 16) + 16 (row / 4), slot row % 4)
__device__ __forceinline__ int tfrag_index(int row, int ch) { return ((ch >> 4) * 64 + (row >> 2) * 16 + (ch & 15)) * 4 + (row & 3); }
// (row, channel) -> element index in the A fragment of the matrix itself (k = channel)
__device__ __forceinline__ int afrag_index(int row, int ch) {
  const int kb = ch >> 5, ko = ch & 31;
  const int gg = ko < 16 ? ko >> 2 : (ko - 16) >> 2;
  const int ss = ko < 16 ? ko & 3 : 4 + ((ko - 16) & 3);
  return (kb * 64 + gg * 16 + row) * 8 + ss;
}

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

// The state-independent part shared by both per-chunk kernels: q, k (and v) rows,
// the log2-unit decay cumsum G, M_rs = sum_i k_ri k_si 2^(G_ri - G_si) for s < r,
// optionally P_rs = sum_i q_ri k_si 2^(G_ri - G_si) for s <= r, and T = (I + A)^-1
// with A_rs = beta_r M_rs. Ends with a barrier.
struct LocalLds {
  float K[BC][LDP], Q[BC][LDP], G[BC][LDP];
  float M[BC][LDS16], T[BC][LDS16], Pm[BC][LDS16];
  float beta[BC];
};

template <typename E, bool WANT_P>
__device__ void local_forward(LocalLds& L, const E* __restrict__ q, const E* __restrict__ k,
                              const float* __restrict__ log_alpha, const float* __restrict__ beta, int tok0, int len,
                              int h, int H, int t) {
  const size_t HD = (size_t)H * D;
  const RowMap rm(t);
  {
    const size_t base = (size_t)tok0 * HD + (size_t)h * D;
    float x[8];
    load8(k + base, HD, rm.r, len, rm.c0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) L.K[rm.r][rm.c0 + i] = x[i];
    load8(q + base, HD, rm.r, len, rm.c0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) L.Q[rm.r][rm.c0 + i] = x[i];
    load8(log_alpha + base, HD, rm.r, len, rm.c0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) L.G[rm.r][rm.c0 + i] = x[i];
    if (t < BC) L.beta[t] = t < len ? beta[(size_t)(tok0 + t) * H + h] : 0.f;
  }
  __syncthreads();
  if (t < D) {  // cumulative log2 decay down the chunk, one channel per thread
    float run = 0.f;
#pragma unroll
    for (int r = 0; r < BC; ++r) {
      run += L.G[r][t] * LOG2E_B;
      L.G[r][t] = run;
    }
  }
  __syncthreads();
  {
    float kr[8], qr[8], gr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kr[i] = L.K[rm.r][rm.ch(i)];
      qr[i] = L.Q[rm.r][rm.ch(i)];
      gr[i] = L.G[rm.r][rm.ch(i)];
    }
#pragma unroll
    for (int s = 0; s < BC; ++s) {
      float pk = 0.f, pq = 0.f;
      if (s <= rm.r) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float ks = L.K[s][rm.ch(i)] * exp2_hw(gr[i] - L.G[s][rm.ch(i)]);  // exponent <= 0
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
  if (t < BC) {  // T = (I + A)^-1 by forward substitution, one column per thread, in registers
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

// ---------------------------------------------------------------------------
// bwd_local_kernel: the backward record of one (chunk, head).
// ---------------------------------------------------------------------------
template <typename E>
__global__ void __launch_bounds__(256) bwd_local_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                        const float* __restrict__ log_alpha,
                                                        const float* __restrict__ beta,
                                                        const int32_t* __restrict__ total_chunks,
                                                        const int2* __restrict__ info, int H, int mc,
                                                        char* __restrict__ brec) {
  using BR = BRec<E>;
  __shared__ LocalLds L;
  const int c = blockIdx.x / H, h = blockIdx.x - c * H;
  if (c >= *total_chunks) return;
  const int t = threadIdx.x;
  const int2 inf = info[c];
  local_forward<E, true>(L, q, k, log_alpha, beta, inf.x, inf.y, h, H, t);

  char* rb = brec + ((size_t)h * mc + c) * BR::BYTES;
  E* wt = reinterpret_cast<E*>(rb + BR::WT);
  E* qtt = reinterpret_cast<E*>(rb + BR::QTT);
  E* kef = reinterpret_cast<E*>(rb + BR::KEF);
  const RowMap rm(t);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = rm.ch(i);
    const float gr = L.G[rm.r][ch];
    float acc = 0.f;
    for (int s = 0; s <= rm.r; ++s) acc += L.T[rm.r][s] * L.beta[s] * L.K[s][ch] * exp2_hw(L.G[s][ch]);
    wt[tfrag_index(rm.r, ch)] = from_f<E>(-acc);
    qtt[tfrag_index(rm.r, ch)] = from_f<E>(L.Q[rm.r][ch] * exp2_hw(gr));
    kef[afrag_index(rm.r, ch)] = from_f<E>(L.K[rm.r][ch] * exp2_hw(L.G[BC - 1][ch] - gr));
  }
  {  // P^T fragment: thread t = (row r, column m) of P
    const int r = t >> 4, mm = t & 15;
    reinterpret_cast<E*>(rb + BR::PT)[((r >> 2) * 16 + mm) * 4 + (r & 3)] = from_f<E>(L.Pm[r][mm]);
  }
  if (t < D) reinterpret_cast<float*>(rb + BR::GAM)[t] = exp2_hw(L.G[BC - 1][t]);
}

// ---------------------------------------------------------------------------
// bwd_state_kernel: one wave per (sequence, head, 16-column slab), chunks in
// reverse. Lane (m, g) keeps dS[16 rt + 4 g + i][16 ct + m] in Lm[rt][i], the layout
// of the forward state kernel, so Lm pairs are B fragments as they stand. Work-group
// ids are dealt so that the eight slabs of a head share one XCD's L2.
// ---------------------------------------------------------------------------
constexpr int STATE_TOUCH_AHEAD = 4;

template <typename E>
__global__ void __launch_bounds__(64) bwd_state_kernel(const char* __restrict__ brec,
                                                       const int32_t* __restrict__ chunk_off,
                                                       const int2* __restrict__ info, const E* __restrict__ dout,
                                                       const float* __restrict__ d_final, float* __restrict__ d_initial,
                                                       E* __restrict__ dstates, E* __restrict__ dut, int N, int H,
                                                       int mc) {
  using BR = BRec<E>;
  typedef typename Frag<E>::T FragT;
  typedef typename Vec4<E>::T V4;
  // four elements kept as raw 32-bit words in the register stage (packed bf16
  // vectors in a struct array otherwise end up in scratch)
  typedef unsigned int RawV __attribute__((ext_vector_type(sizeof(V4) / 4)));
  constexpr int XW = 16 + 16 / (int)sizeof(E);  // LDS row stride (elements): 16 columns + 16 bytes
  constexpr int VE = 16 / (int)sizeof(E);       // elements per 16-byte store
  __shared__ __attribute__((aligned(16))) E xs[D * XW];
  __shared__ __attribute__((aligned(16))) float xg[D];

  const int b = blockIdx.x;
  const int xcd = b & 7, rest = b >> 3;
  const int ct = rest & 7, slot = rest >> 3;
  const int u = slot * 8 + xcd;
  if (u >= N * H) return;
  const int n = u / H, h = u - n * H;
  const int lane = threadIdx.x, m = lane & 15, g = lane >> 4;
  const size_t HD = (size_t)H * D;
  const size_t sbase = (size_t)u * D * D + 16 * ct + m;

  floatx4 Lm[8];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    Lm[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (d_final) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Lm[rt][i] = d_final[sbase + (size_t)(16 * rt + 4 * g + i) * D];
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

  // operands are kept as whole fragments (chunk rows 16..31 zero): a stage of
  // half-width vectors gets merged into wide loads that keep it out of registers
  struct Stage {
    FragT wt[8], qt[8], pt, dov;
    FragT ke[4];
    floatx4 gm;
    int2 inf;
  };
  const int c_begin = chunk_off[n], c_end = chunk_off[n + 1];
  auto load = [&](Stage& st, int c) {
    const char* rb = brec + ((size_t)h * mc + c) * BR::BYTES;
    const E* wt = reinterpret_cast<const E*>(rb + BR::WT);
    const E* qt = reinterpret_cast<const E*>(rb + BR::QTT);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      st.wt[rt] = half_frag(*reinterpret_cast<const RawV*>(wt + ((size_t)rt * 64 + lane) * 4));
      st.qt[rt] = half_frag(*reinterpret_cast<const RawV*>(qt + ((size_t)rt * 64 + lane) * 4));
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      st.ke[kb] = load_frag<E>(reinterpret_cast<const E*>(rb + BR::KEF) + ((size_t)kb * 64 + lane) * 8);
    st.pt = half_frag(*reinterpret_cast<const RawV*>(reinterpret_cast<const E*>(rb + BR::PT) + (size_t)lane * 4));
    st.gm = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(rb + BR::GAM) + 4 * (lane & 31));
    const int2 inf = info[c];
    st.inf = inf;
    V4 d;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int row = 4 * g + s;
      d[s] = row < inf.y ? dout[(size_t)(inf.x + row) * HD + (size_t)h * D + 16 * ct + m] : from_f<E>(0.f);
    }
    st.dov = half_frag(__builtin_bit_cast(RawV, d));
  };

  auto compute = [&](const Stage& st, int c) {
    {  // the gradient at the chunk's end, for the per-chunk kernel, as 16-byte row pieces
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[(16 * rt + 4 * g + i) * XW + m] = from_f<E>(Lm[rt][i]);
      __syncthreads();
      E* dp = dstates + ((size_t)h * mc + c) * D * D + 16 * ct;
#pragma unroll
      for (int j = 0; j < 2 * (int)sizeof(E); ++j) {
        const int piece = lane + 64 * j, row = piece / (16 / VE), col = (piece % (16 / VE)) * VE;
        *reinterpret_cast<uint4*>(dp + (size_t)row * D + col) = *reinterpret_cast<const uint4*>(&xs[row * XW + col]);
      }
      __syncthreads();
    }
    const FragT dOb = st.dov;  // B fragment of dO over the chunk rows
    // dU~ = P^T dO + (K e^{g_C-G}) dS_C
    floatx4 du = zero4;
    mma(du, st.pt, dOb);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mma(du, st.ke[kb], acc_pair_to_frag<E>(Lm[2 * kb], Lm[2 * kb + 1]));
    {
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[(4 * g + i) * XW + m] = from_f<E>(du[i]);
      if (lane < 32) *reinterpret_cast<floatx4*>(&xg[4 * lane]) = st.gm;
      __syncthreads();
      if (lane < 16 * (16 / VE)) {
        const int row = lane / (16 / VE), col = (lane % (16 / VE)) * VE;
        *reinterpret_cast<uint4*>(dut + ((size_t)h * mc + c) * BC * D + (size_t)row * D + 16 * ct + col) =
            *reinterpret_cast<const uint4*>(&xs[row * XW + col]);
      }
    }
    const FragT dUb = acc_pair_to_frag<E>(du, zero4);
    // dS0 = e^{g_C} o dS_C + (Q e^G)^T dO + (-W)^T dU~
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      const floatx4 gv = *reinterpret_cast<const floatx4*>(&xg[16 * rt + 4 * g]);
      Lm[rt] = gv * Lm[rt];
      mma(Lm[rt], st.qt[rt], dOb);
      mma(Lm[rt], st.wt[rt], dUb);
    }
    __syncthreads();
  };

  // L2 touch STATE_TOUCH_AHEAD chunks beyond the register stage: the head's eight
  // slab waves each read one word of every eighth record line, so the real loads
  // hit in L2 (the words are XOR-folded into tacc, stored only by a never-taken
  // branch). No address here depends on a load: that would make the wave wait.
  constexpr int LINES = (int)(BR::BYTES / 128);
  static_assert(BR::BYTES % 128 == 0 && LINES <= 8 * 64, "one touch per lane");
  const int touch_line = ct + 8 * lane;
  unsigned tacc = 0u;
  auto touch = [&](int c) {
    unsigned x = 0u;
    if (touch_line < LINES)
      x = *reinterpret_cast<const unsigned*>(brec + ((size_t)h * mc + c) * BR::BYTES + (size_t)touch_line * 128);
    return x;
  };

  // two named stages: each step loads chunk c - 1 into the stage consumed one step
  // earlier (past the start, the first chunk again: every step issues the same loads)
  Stage sa, sb;
  unsigned ta = 0u, tb = 0u;
  if (c_begin < c_end) load(sa, c_end - 1);
  for (int c0 = c_end - 1; c0 >= c_begin; c0 -= 2) {
    load(sb, max(c0 - 1, c_begin));
    ta = touch(max(c0 - 1 - STATE_TOUCH_AHEAD, c_begin));
    compute(sa, c0);
    tacc ^= tb;
    load(sa, max(c0 - 2, c_begin));
    tb = touch(max(c0 - 2 - STATE_TOUCH_AHEAD, c_begin));
    if (c0 - 1 >= c_begin) compute(sb, c0 - 1);
    tacc ^= ta;
  }
  // mc is never negative (the host sizes it from the shapes), so this never stores
  if (mc < 0 && tacc == 0u) dut[lane] = from_f<E>(0.f);
  if (d_initial) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) d_initial[sbase + (size_t)(16 * rt + 4 * g + i) * D] = Lm[rt][i];
  }
}

// ---------------------------------------------------------------------------
// bwd_chunk_kernel: the gradients of one (chunk, head).
// ---------------------------------------------------------------------------
struct ChunkLds {
  LocalLds L;
  float V[BC][LDP];
  float dU[BC][LDP];                   // dU~; later the per-row KE terms of dG
  float X1[BC][LDP], X2[BC][LDP], X3[BC][LDP];  // X2 is later dG
  float dP[BC][LDS16], dT[BC][LDS16], dA[BC][LDS16];
  float dgam[D];
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
    const int32_t* __restrict__ total_chunks, const int2* __restrict__ info, int H, int mc, E* __restrict__ dq,
    E* __restrict__ dk, E* __restrict__ dv, float* __restrict__ dlog_alpha, float* __restrict__ dbeta) {
  typedef typename Frag<E>::T FragT;
  __shared__ ChunkLds S;
  LocalLds& L = S.L;
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

  {
    float x[8];
    load8(v + rowbase, HD, rm.r, len, rm.c0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) S.V[rm.r][rm.c0 + i] = x[i];
    load8(dUt, D, rm.r, BC, rm.c0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) S.dU[rm.r][rm.c0 + i] = x[i];
  }
  local_forward<E, false>(L, q, k, log_alpha, beta, tok0, len, h, H, t);

  // ---- state products: wave w forms channel tiles 2w and 2w+1 of
  //      X1 = dO S0^T, X2 = dU~ S0^T, X3 = U~ dS_C^T, and dgamma = rowsum(dS_C o S0)
  {
    FragT a1[4], a2[4], a3[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      a1[kb] = m < len ? frag_rowk<E>(dout + rowbase, (int)HD, m, 32 * kb, g) : zero_frag<E>();
      a2[kb] = frag_rowk<E>(dUt, D, m, 32 * kb, g);
      a3[kb] = frag_rowk<E>(Ut, D, m, 32 * kb, g);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nt = 2 * w + j;
      floatx4 x1 = {0.f, 0.f, 0.f, 0.f}, x2 = x1, x3 = x1;
      float dg = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const FragT bs = frag_rowk<E>(S0, D, 16 * nt + m, 32 * kb, g);
        const FragT bd = frag_rowk<E>(dSC, D, 16 * nt + m, 32 * kb, g);
        mma(x1, a1[kb], bs);
        mma(x2, a2[kb], bs);
        mma(x3, a3[kb], bd);
#pragma unroll
        for (int s = 0; s < 8; ++s) dg += to_f(bs[s]) * to_f(bd[s]);
      }
      dg += __shfl_xor(dg, 16);
      dg += __shfl_xor(dg, 32);
      if (g == 0) S.dgam[16 * nt + m] = dg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        S.X1[4 * g + i][16 * nt + m] = x1[i];
        S.X2[4 * g + i][16 * nt + m] = x2[i];
        S.X3[4 * g + i][16 * nt + m] = x3[i];
      }
    }
    if (w == 0) {  // dP = tril(dO U~^T)
      floatx4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(p, a1[kb], frag_rowk<E>(Ut, D, m, 32 * kb, g));
#pragma unroll
      for (int i = 0; i < 4; ++i) S.dP[4 * g + i][m] = m <= 4 * g + i ? p[i] : 0.f;
    }
  }
  __syncthreads();

  // ---- dT = dW (diag(beta) K e^G)^T + dU (diag(beta) V)^T, dW = -X2 -------------
  {
    float x2r[8], dur[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x2r[i] = S.X2[rm.r][rm.ch(i)];
      dur[i] = S.dU[rm.r][rm.ch(i)];
    }
#pragma unroll
    for (int s = 0; s < BC; ++s) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ch = rm.ch(i);
        acc += -x2r[i] * L.K[s][ch] * exp2_hw(L.G[s][ch]) + dur[i] * S.V[s][ch];
      }
      acc = sum16(acc) * L.beta[s];
      if ((t & 15) == 0) S.dT[rm.r][s] = s < rm.r ? acc : 0.f;  // only the strictly lower part of T varies
    }
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

  // ---- per (row, 8 channels): dv, dbeta, dq, dk and dG --------------------------
  const int r = rm.r;
  float dqv[8], dkv[8], dgv[8], kex[8];
  {
    const float br = L.beta[r];
    float dbk[8], dbv[8], kr[8], qr[8], gr[8];
    float ra[8], rp[8], rat[8], rpt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dbk[i] = dbv[i] = ra[i] = rp[i] = rat[i] = rpt[i] = 0.f;
      kr[i] = L.K[r][rm.ch(i)];
      qr[i] = L.Q[r][rm.ch(i)];
      gr[i] = L.G[r][rm.ch(i)];
    }
    // One pass over the chunk's rows s. T is lower (T[s][r] = 0 for s < r), dA
    // strictly lower and dP lower, so row s < r only feeds the sums along row r
    // (ra, rp: weights e^{g_r - g_s}) and row s > r only those down column r
    // (rat, rpt: weights e^{g_s - g_r}); with g non-increasing both weights are
    // 2^-|g_r - g_s|, and the other side's coefficients are exact zeros.
#pragma unroll 2
    for (int s = 0; s < BC; ++s) {
      const float tsr = L.T[s][r];
      const float a_rs = S.dT[r][s], p_rs = S.dP[r][s];                  // dA, dP along row r
      const float a_sr = L.beta[s] * S.dT[s][r], p_sr = S.dP[s][r];      // down column r
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ch = rm.ch(i);
        dbk[i] -= tsr * S.X2[s][ch];  // dB_K = T^T dW
        dbv[i] += tsr * S.dU[s][ch];  // dB_V = T^T dU
        const float ks = L.K[s][ch], qs = L.Q[s][ch];
        const float f = exp2_hw(-fabsf(gr[i] - L.G[s][ch]));
        ra[i] += a_rs * ks * f;
        rp[i] += p_rs * ks * f;
        rat[i] += a_sr * ks * f;
        rpt[i] += p_sr * qs * f;
      }
    }
    float dbeta_part = 0.f, dvv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ch = rm.ch(i);
      const float eg = exp2_hw(gr[i]);
      const float el = exp2_hw(L.G[BC - 1][ch] - gr[i]);
      dbeta_part += dbk[i] * kr[i] * eg + dbv[i] * S.V[r][ch];
      dvv[i] = br * dbv[i];
      const float x1 = S.X1[r][ch], x3 = S.X3[r][ch];
      dqv[i] = x1 * eg + rp[i];
      dkv[i] = br * dbk[i] * eg + br * ra[i] + rat[i] + rpt[i] + x3 * el;
      kex[i] = x3 * kr[i] * el;
      dgv[i] = x1 * qr[i] * eg + rp[i] * qr[i] + br * dbk[i] * kr[i] * eg + br * ra[i] * kr[i] - rat[i] * kr[i] -
               rpt[i] * kr[i] - kex[i];
    }
    dbeta_part = sum16(dbeta_part);
    if ((t & 15) == 0 && r < len) {
      float am = 0.f;
      for (int s = 0; s < r; ++s) am += S.dT[r][s] * L.M[r][s];
      dbeta[(size_t)(tok0 + r) * H + h] = dbeta_part + am;
    }
    if (r < len) {
      const size_t ro = rowbase + (size_t)r * HD;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dv[ro + rm.ch(i)] = from_f<E>(dvv[i]);
        dq[ro + rm.ch(i)] = from_f<E>(dqv[i]);
        dk[ro + rm.ch(i)] = from_f<E>(dkv[i]);
      }
    }
  }
  __syncthreads();  // every read of X2 and dU is done
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    S.X2[r][rm.ch(i)] = dgv[i];
    S.dU[r][rm.ch(i)] = kex[i];
  }
  __syncthreads();
  if (t < D) {  // g_C = G at the last row: its gradient gathers the K e^{g_C-G} and e^{g_C} terms
    float extra = S.dgam[t] * exp2_hw(L.G[BC - 1][t]);
#pragma unroll
    for (int rr = 0; rr < BC; ++rr) extra += S.dU[rr][t];
    float run = extra;
    for (int rr = BC - 1; rr >= 0; --rr) {
      run += S.X2[rr][t];
      if (rr < len) dlog_alpha[rowbase + (size_t)rr * HD + t] = run;
    }
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
  l.total = l.off_dut + bal256((size_t)mc * H * BC * D * es);
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
  const int dtype = std::is_same<E, float>::value ? 1 : 0;

  trace_begin(stream);
  hipError_t e = launch_forward_states(dtype, q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, B, T,
                                       H, workspace, states, ut, stream);
  if (e != hipSuccess) return e;
  if (mc > 0) {
    hipLaunchKernelGGL(bwd_local_kernel<E>, dim3((unsigned)(mc * H)), dim3(256), 0, stream, (const E*)q,
                       (const E*)k, log_alpha, beta, chunk_off + N, info, H, (int)mc, brec);
    e = hipGetLastError();
    trace_mark(stream, 5);
    if (e != hipSuccess) return e;
  }
  const int64_t slots = ((int64_t)N * H + 7) / 8;
  if (slots > 0) {
    hipLaunchKernelGGL(bwd_state_kernel<E>, dim3((unsigned)(slots * 64)), dim3(64), 0, stream, brec, chunk_off,
                       info, (const E*)dout, d_final, d_initial, dstates, dut, N, H, (int)mc);
    e = hipGetLastError();
    trace_mark(stream, 6);
    if (e != hipSuccess) return e;
  }
  if (mc > 0) {
    hipLaunchKernelGGL(bwd_chunk_kernel<E>, dim3((unsigned)(mc * H)), dim3(256), 0, stream, (const E*)q,
                       (const E*)k, (const E*)v, log_alpha, beta, (const E*)dout, states, dstates, ut, dut,
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
