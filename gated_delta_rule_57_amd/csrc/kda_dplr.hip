// Chunked forward of the general diagonal-plus-low-rank (DPLR) recurrence on gfx950
//
//     S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T ,   o_t = S_t^T q_t
//
// the comparison point for KDA's chunk kernel (GeekNews "Kimi Linear" summary,
// section "일반 DPLR보다 줄어든 연산량": KDA and a general DPLR transition both allow
// fine-grained decay, but KDA ties the transition's two low-rank vectors to the key,
// which halves the secondary C x C matrices per chunk and drops three matrix
// products). Here the two vectors are free, so every chunk needs all four.
//
// Chunk form (rows r, s; g = inclusive and g^- = g - log_alpha exclusive cumulative
// log-decay per channel; S_0 the state entering the chunk; w_r = S_{r-1}^T b_r):
//   M_ba = tril_strict sum_c b_rc a_sc e^{g^-_rc - g_sc}     M_bk: k_s in place of a_s
//   M_qa = tril        sum_c q_rc a_sc e^{g_rc - g_sc}       M_qk: k_s in place of a_s
//   T    = (I - M_ba)^{-1}                                    forward substitution
//   W_b  = T (B e^{G^-}) ,  U = T M_bk V                      W = U + W_b S_0
//   O    = (Q e^G) S_0 + M_qa W + M_qk V
//   S_C  = Diag(e^{g_C}) S_0 + (A e^{g_C-G})^T W + (K e^{g_C-G})^T V
// (unrolling w_r inside the chunk gives (I - M_ba) W = (B e^{G^-}) S_0 + M_bk V).
//
// dplr_intra_kernel computes everything that does not depend on the state, one
// work-group per (chunk, head), into a record (RecD) whose first five fields play
// the roles of the KDA record's; the 64-token inter kernels, instantiated with the
// DPLR flag, then run the serial state pass exactly as for KDA plus the two
// V-terms. In-chunk decay uses the same sub-chunk factoring as the KDA intra
// kernel, in log2 units with reference points b_0 = 0, b_I = g[16 I - 1]: for a
// block (I, J <= I), 2^(x_r - g_s) = 2^(x_r - b_I) 2^(b_I - b_{J+1}) 2^(b_{J+1} - g_s)
// with x = g for the q rows and x = g^- for the b rows; g^-_r <= b_I holds for r in
// sub-chunk I, so both row factors stay <= 1. A chunk whose diagonal range
// b_I - b_{I+1} exceeds 120 for some channel takes an exact path that sums every
// entry on the VALU with 2^(x_r - g_s), exponent <= 0.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_inter64.h"
#include "kda_record.h"

namespace kda {

namespace {

constexpr int DC = 64;                      // chunk length
constexpr int DWAVES = 8;                   // waves per intra-chunk work-group
constexpr int DTHREADS = 64 * DWAVES;
constexpr float DP_LOG2E = 1.4426950408889634f;
constexpr float DP_RANGE_LIMIT = 120.f;     // log2 units

__host__ __device__ constexpr size_t dmax(size_t a, size_t b) { return a > b ? a : b; }
__device__ __forceinline__ float dexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Shared-memory plan (byte offsets). Phase A builds the factored operands and the
// four C x C matrices; phase B reuses the space for T and the chunk products.
template <typename E>
struct DSmem {
  static constexpr int C = DC;
  static constexpr int NSUB = C / 16;
  static constexpr int LD = D + 8;   // row stride of [rows][128] E matrices
  static constexpr int GLD = D + 4;  // row stride of fp32 [rows][128] matrices
  static constexpr int LDC = C + 4;  // row stride of the fp32 C x C matrix
  static constexpr int LDK = C + 8;  // row stride of E C x C matrices
  // phase A: the cumulative sum, then (factored path) the row operands over it
  static constexpr size_t G = 0;                                        // float[C][GLD] inclusive log2 cumsum
  static constexpr size_t LB = 0;                                       // E[C][LD]  b_r 2^(g^-_r - b_I)
  static constexpr size_t LQ = LB + al16((size_t)C * LD * sizeof(E));   // E[C][LD]  q_r 2^(g_r - b_I)
  static constexpr size_t RA = LQ + al16((size_t)C * LD * sizeof(E));   // float[C][GLD]  a_s 2^(b_{J+1} - g_s)
  static constexpr size_t RK = RA + al16((size_t)C * GLD * 4);          // float[C][GLD]  k_s 2^(b_{J+1} - g_s)
  static constexpr size_t A_END = RK + al16((size_t)C * GLD * 4);
  static_assert(G + (size_t)C * GLD * 4 <= RA, "the right operands are written while the cumsum is read");
  // phase B
  static constexpr size_t MA = 0;                                       // float[C][LDC]  -M_ba, strictly lower
  static constexpr size_t TD = MA + al16((size_t)C * LDC * 4);          // float[NSUB][16][20] diagonal blocks of T
  static constexpr size_t TB = TD + al16((size_t)NSUB * 16 * 20 * 4);   // E[C][LDK]  T
  static constexpr size_t KT = TB + al16((size_t)C * LDK * sizeof(E));  // E[C][LD]   B e^{G^-}
  static constexpr size_t VV = KT + al16((size_t)C * LD * sizeof(E));   // E[C][LD]   V
  static constexpr size_t MB = VV + al16((size_t)C * LD * sizeof(E));   // E[C][LDK]  M_bk
  static constexpr size_t MQ = MB + al16((size_t)C * LDK * sizeof(E));  // E[C][LDK]  M_qk
  static constexpr size_t YY = MB;                                      // E[C][LD]   M_bk V, once MB and MQ are read
  static constexpr size_t B_END = MQ + al16((size_t)C * LDK * sizeof(E));
  static_assert(YY + (size_t)C * LD * sizeof(E) <= B_END, "M_bk V fits where M_bk and M_qk were");
  // tables that live through every phase
  static constexpr size_t BND = dmax(A_END, B_END);                     // float[NSUB+1][D] b_I
  static constexpr int NBLK = NSUB * (NSUB + 1) / 2;
  static constexpr int NSCALE = NBLK + NSUB;
  static constexpr size_t SCL = BND + (size_t)(NSUB + 1) * D * 4;       // float[NSCALE][D]
  static constexpr size_t FLAG = SCL + (size_t)NSCALE * D * 4;          // int[NSUB]
  static constexpr size_t TOTAL = al16(FLAG + 4 * NSUB);
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one gfx950 CU");
};

// Which 16 x 16 block (I, J <= I) of the four C x C matrices wave w forms in its
// bi-th slot (bi < 2). The blocks J = 2 kb and 2 kb + 1 of a block row fill one
// 16-byte slot of P per lane, so they go to the same wave and P leaves as whole
// slots: waves 0-3 take the pairs of block rows 1-3, waves 4 and 5 the single blocks
// (0, 0) and (2, 2). The two slots wholly above the diagonal are never read and
// not written.
__device__ __forceinline__ bool dwave_block(int w, int bi, int& I, int& J) {
  if (w < 4) {  // (1,0) (1,1) | (2,0) (2,1) | (3,0) (3,1) | (3,2) (3,3)
    I = w < 3 ? w + 1 : 3;
    J = (w < 3 ? 0 : 2) + bi;
    return true;
  }
  I = J = 2 * (w - 4);  // (0,0) | (2,2)
  return bi == 0 && w < 6;
}

}  // namespace

// ---------------------------------------------------------------------------
// Intra-chunk kernel: one work-group of 8 waves per (chunk, head); its LDS plan
// allows one work-group per CU, so the eight waves (two per SIMD) are what hides
// latency. Thread t owns channels 4 (t & 31) .. + 3 of rows (t >> 5) + 16 i in the
// element-wise phases. The four C x C matrices are computed transposed, one
// 16 x 16 block (I, J <= I) per wave at a time (lane (m, g), element ii = entry
// (16 I + m, 16 J + 4 g + ii)); wave w takes value columns 16 w .. 16 w + 15 in B3.
// Phases (barriers in between):
//   P1  loads of q, k, v, a, b and log_alpha; log2 cumulative sum, sub-chunk
//       boundaries and block scales, range flags
//   P2  Q e^G to the record; B e^{G^-} kept; factored row operands to LDS
//   P3  M_ba, M_bk, M_qa, M_qk by MFMA; M_qa, (A e^{g_C-G})^T, (K e^{g_C-G})^T to the record
//   B0  -M_ba (fp32), M_bk, M_qk, B e^{G^-}, V to LDS
//   B1  diagonal 16 x 16 blocks of T = (I - M_ba)^{-1} by forward substitution
//   B2  off-diagonal blocks of T by fp32 MFMA
//   B3  V fragments and M_qk V to the record; M_bk V to LDS; W_b = T (B e^{G^-}) and
//       U = T (M_bk V) to the record
// ---------------------------------------------------------------------------
template <typename E>
__global__ void __launch_bounds__(DTHREADS) dplr_intra_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                         const E* __restrict__ v, const E* __restrict__ a,
                                                         const E* __restrict__ b, const float* __restrict__ log_alpha,
                                                         const int32_t* __restrict__ total_chunks,
                                                         const int2* __restrict__ info, int H, int mc,
                                                         char* __restrict__ records) {
  using SM = DSmem<E>;
  using RC = RecD<E, DC>;
  typedef typename Frag<E>::T FragT;
  typedef typename Vec4<E>::T V4;
  constexpr int C = DC, NSUB = SM::NSUB, LD = SM::LD, GLD = SM::GLD, LDC = SM::LDC, LDK = SM::LDK;
  constexpr int NRT = C / 16, NKC = C / 32, RG = DTHREADS / 32, RPT = C / RG;
  constexpr int NBLK = SM::NBLK, BPW = (NBLK + DWAVES - 1) / DWAVES;
  static_assert(DWAVES == D / 16 && NSUB == 4 && BPW == 2, "the wave assignment below is for 8 waves, C = 64");

  __shared__ __attribute__((aligned(16))) char smem[SM::TOTAL];
  float* sG = reinterpret_cast<float*>(smem + SM::G);
  float* sBnd = reinterpret_cast<float*>(smem + SM::BND);
  float* sScl = reinterpret_cast<float*>(smem + SM::SCL);
  int* sFlag = reinterpret_cast<int*>(smem + SM::FLAG);

  const int c = blockIdx.x / H, h = blockIdx.x - c * H;  // heads fastest, as in the KDA intra kernel
  if (c >= *total_chunks) return;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, m = lane & 15, g = lane >> 4;
  const int ch0 = 4 * (t & 31), rbase = t >> 5;
  const int2 inf = info[c];
  const int tok0 = inf.x, len = inf.y;
  const size_t HD = (size_t)H * D;
  char* rec_base = records + ((size_t)h * mc + c) * RC::BYTES;
  E* rec = reinterpret_cast<E*>(rec_base);
  float* rec_gamma = reinterpret_cast<float*>(rec_base + RC::GAMMA_BYTES);

  // ---- P1: all loads in flight (rows past len read row 0 and are zeroed at use) --
  //      the decays first, behind a compiler fence: memory counters count in issue
  //      order, so the decay phases then wait for the decays only
  V4 qv[RPT], kv[RPT], vv[RPT], av[RPT], bv[RPT];
  floatx4 la[RPT];
  auto row_off = [&](int i) {
    const int r = rbase + RG * i;
    return (size_t)(tok0 + (r < len ? r : 0)) * HD + (size_t)h * D + ch0;
  };
#pragma unroll
  for (int i = 0; i < RPT; ++i) la[i] = *reinterpret_cast<const floatx4*>(log_alpha + row_off(i));
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const size_t off = row_off(i);
    qv[i] = *reinterpret_cast<const V4*>(q + off);
    kv[i] = *reinterpret_cast<const V4*>(k + off);
    vv[i] = *reinterpret_cast<const V4*>(v + off);
    av[i] = *reinterpret_cast<const V4*>(a + off);
    bv[i] = *reinterpret_cast<const V4*>(b + off);
  }
  auto val = [&](const V4& x, int i, int j) { return rbase + RG * i < len ? to_f(x[j]) : 0.f; };
  if (t < NSUB) sFlag[t] = 0;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rbase + RG * i;
    *reinterpret_cast<floatx4*>(sG + r * GLD + ch0) = r < len ? la[i] * DP_LOG2E : floatx4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  {  // cumulative sum over the rows per channel: NP row ranges, then the carries
    constexpr int NP = DTHREADS / D, PR = C / NP;
    const int chn = t & (D - 1), part = t / D;
    float x[PR];
#pragma unroll
    for (int r = 0; r < PR; ++r) x[r] = sG[(part * PR + r) * GLD + chn];
#pragma unroll
    for (int r = 1; r < PR; ++r) x[r] += x[r - 1];
#pragma unroll
    for (int r = 0; r < PR; ++r) sG[(part * PR + r) * GLD + chn] = x[r];
    __syncthreads();
    float carry = 0.f;
    for (int p2 = 0; p2 < part; ++p2) carry += sG[(p2 * PR + PR - 1) * GLD + chn];
    __syncthreads();  // every carry is read before any range is shifted
#pragma unroll
    for (int r = 0; r < PR; ++r) sG[(part * PR + r) * GLD + chn] = x[r] + carry;
  }
  __syncthreads();
  if (t < D) {
    float bnd[NSUB + 1];
    bnd[0] = 0.f;
#pragma unroll
    for (int I = 1; I <= NSUB; ++I) bnd[I] = sG[(16 * I - 1) * GLD + t];
#pragma unroll
    for (int I = 0; I <= NSUB; ++I) sBnd[I * D + t] = bnd[I];
    rec_gamma[t] = dexp2(bnd[NSUB]);
#pragma unroll
    for (int I = 0; I < NSUB; ++I)
      if (!(bnd[I] - bnd[I + 1] <= DP_RANGE_LIMIT)) atomicOr(&sFlag[I], 1);
#pragma unroll
    for (int I = 0; I < NSUB; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) sScl[(I * (I + 1) / 2 + J) * D + t] = dexp2(bnd[I] - bnd[J + 1]);
#pragma unroll
    for (int J = 0; J < NSUB; ++J) sScl[(NBLK + J) * D + t] = dexp2(bnd[NSUB] - bnd[J + 1]);
  }
  __syncthreads();
  bool exact = false;
#pragma unroll
  for (int I = 0; I < NSUB; ++I) exact |= sFlag[I] != 0;

  // Q e^G to its fragment slot: 4 consecutive channels are half of one lane's fragment
  auto store_qt = [&](int r, const float qt[4]) {
    const int kb = ch0 >> 5, co = ch0 & 31;
    const int fg = (co & 15) >> 2, fh = co >> 4;
    store4f(rec + RC::QT + ((size_t)((r >> 4) * 4 + kb) * 64 + (r & 15) + 16 * fg) * 8 + 4 * fh, qt);
  };
  // (A e^{g_C-G})^T and (K e^{g_C-G})^T as transposed fragments, whole 16-byte slots:
  // item (channel, 4-row group fg, k-block kb) holds rows 32 kb + 4 fg + j and
  // 32 kb + 16 + 4 fg + j; 16 consecutive items fill 256 contiguous bytes.
  // ends(s, ch, ae, ke) gives both values of chunk row s.
  auto emit_ends = [&](auto ends) {
    for (int it = t; it < D * NKC * 4; it += DTHREADS) {
      const int ch = it & (D - 1), fg = (it >> 7) & 3, kb = it >> 9;
      floatx4 alo, ahi, klo, khi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a0, k0, a1, k1;
        ends(32 * kb + 4 * fg + j, ch, a0, k0);
        ends(32 * kb + 16 + 4 * fg + j, ch, a1, k1);
        alo[j] = a0;
        klo[j] = k0;
        ahi[j] = a1;
        khi[j] = k1;
      }
      const size_t slot = ((size_t)((ch >> 4) * NKC + kb) * 64 + (ch & 15) + 16 * fg) * 8;
      store_frag<E>(rec + RC::KE + slot, acc_pair_to_frag<E>(alo, ahi));
      store_frag<E>(rec + RC::KV + slot, acc_pair_to_frag<E>(klo, khi));
    }
  };
  // P = M_qa in whole slots: an even block waits in p_lo for its odd partner unless it
  // is the last of its block row
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  floatx4 p_lo = zero4;
  auto emit_p = [&](int I, int J, const floatx4& acc) {
    floatx4 pv;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) pv[ii] = (16 * J + 4 * g + ii <= 16 * I + m) ? acc[ii] : 0.f;
    E* dst = rec + RC::PP + ((size_t)(I * NKC + (J >> 1)) * 64 + lane) * 8;
    if (J & 1)
      store_frag<E>(dst, acc_pair_to_frag<E>(p_lo, pv));
    else if (J == I)
      store_frag<E>(dst, acc_pair_to_frag<E>(pv, zero4));
    else
      p_lo = pv;
  };

  float bt[RPT][4];  // B e^{G^-}, kept for phase B
  floatx4 aBA[BPW], aBK[BPW], aQA[BPW], aQK[BPW];
  if (!exact) {
    // ---- P2 (factored) ------------------------------------------------------------
    E* sLB = reinterpret_cast<E*>(smem + SM::LB);
    E* sLQ = reinterpret_cast<E*>(smem + SM::LQ);
    float* sRA = reinterpret_cast<float*>(smem + SM::RA);
    float* sRK = reinterpret_cast<float*>(smem + SM::RK);
    V4 lbv[RPT], lqv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + RG * i, I = r >> 4;
      const floatx4 gr = *reinterpret_cast<const floatx4*>(sG + r * GLD + ch0);
      const floatx4 gx = r > 0 ? *reinterpret_cast<const floatx4*>(sG + (r - 1) * GLD + ch0)
                               : floatx4{0.f, 0.f, 0.f, 0.f};
      const floatx4 b0 = *reinterpret_cast<const floatx4*>(sBnd + I * D + ch0);
      const floatx4 b1 = *reinterpret_cast<const floatx4*>(sBnd + (I + 1) * D + ch0);
      float qt[4];
      floatx4 ra, rk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float qq = val(qv[i], i, j), bb = val(bv[i], i, j), aa = val(av[i], i, j), kk = val(kv[i], i, j);
        qt[j] = qq * dexp2(gr[j]);                       // exponents <= 0 throughout
        bt[i][j] = bb * dexp2(gx[j]);
        lbv[i][j] = from_f<E>(bb * dexp2(gx[j] - b0[j]));
        lqv[i][j] = from_f<E>(qq * dexp2(gr[j] - b0[j]));
        const float rs = dexp2(b1[j] - gr[j]);
        ra[j] = aa * rs;
        rk[j] = kk * rs;
      }
      *reinterpret_cast<floatx4*>(sRA + r * GLD + ch0) = ra;
      *reinterpret_cast<floatx4*>(sRK + r * GLD + ch0) = rk;
      store_qt(r, qt);
    }
    __syncthreads();  // every thread has its decays; the row operands overwrite the cumsum
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + RG * i;
      *reinterpret_cast<V4*>(sLB + r * LD + ch0) = lbv[i];
      *reinterpret_cast<V4*>(sLQ + r * LD + ch0) = lqv[i];
    }
    __syncthreads();
    // ---- P3 (factored): block (I, J) = lhs_I diag(2^(b_I - b_{J+1})) rhs_J^T ------------
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      aBA[bi] = aBK[bi] = aQA[bi] = aQK[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      int I, J;
      if (!dwave_block(w, bi, I, J)) break;
      const int rrow = 16 * I + m, srow = 16 * J + m;
      const float* scl = sScl + (size_t)(I * (I + 1) / 2 + J) * D;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        FragT flb, flq, fra, frk;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ch = 32 * kb + 16 * hh + 4 * g;
          const V4 lb4 = *reinterpret_cast<const V4*>(sLB + rrow * LD + ch);
          const V4 lq4 = *reinterpret_cast<const V4*>(sLQ + rrow * LD + ch);
          const floatx4 ra4 = *reinterpret_cast<const floatx4*>(sRA + srow * GLD + ch);
          const floatx4 rk4 = *reinterpret_cast<const floatx4*>(sRK + srow * GLD + ch);
          const floatx4 sc = *reinterpret_cast<const floatx4*>(scl + ch);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            flb[4 * hh + j] = lb4[j];
            flq[4 * hh + j] = lq4[j];
            fra[4 * hh + j] = from_f<E>(ra4[j] * sc[j]);
            frk[4 * hh + j] = from_f<E>(rk4[j] * sc[j]);
          }
        }
        mma(aBA[bi], fra, flb);
        mma(aBK[bi], frk, flb);
        mma(aQA[bi], fra, flq);
        mma(aQK[bi], frk, flq);
      }
      emit_p(I, J, aQA[bi]);
    }
    // (A e^{g_C-G})^T and (K e^{g_C-G})^T: rhs_s 2^(g_C - b_{J+1})
    emit_ends([&](int s, int ch, float& ae, float& ke) {
      const float f = sScl[(NBLK + (s >> 4)) * D + ch];
      ae = sRA[s * GLD + ch] * f;
      ke = sRK[s * GLD + ch] * f;
    });
  } else {
    // ---- P2 (exact) ---------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + RG * i;
      const floatx4 gr = *reinterpret_cast<const floatx4*>(sG + r * GLD + ch0);
      const floatx4 gx = r > 0 ? *reinterpret_cast<const floatx4*>(sG + (r - 1) * GLD + ch0)
                               : floatx4{0.f, 0.f, 0.f, 0.f};
      float qt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qt[j] = val(qv[i], i, j) * dexp2(gr[j]);
        bt[i][j] = val(bv[i], i, j) * dexp2(gx[j]);
      }
      store_qt(r, qt);
    }
    // ---- P3 (exact): every entry summed over the channels with 2^(x_r - g_s) ------
    const E* qh = q + (size_t)tok0 * HD + (size_t)h * D;
    const E* kh = k + (size_t)tok0 * HD + (size_t)h * D;
    const E* ah = a + (size_t)tok0 * HD + (size_t)h * D;
    const E* bh = b + (size_t)tok0 * HD + (size_t)h * D;
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      aBA[bi] = aBK[bi] = aQA[bi] = aQK[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      int I, J;
      if (!dwave_block(w, bi, I, J)) break;
      const int r = 16 * I + m;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int s = 16 * J + 4 * g + ii;
        float ba = 0.f, bk = 0.f, qa = 0.f, qk = 0.f;
        if (s <= r && r < len) {
          for (int ch = 0; ch < D; ++ch) {
            const float gs = sG[s * GLD + ch];
            const float asc = to_f(ah[(size_t)s * HD + ch]), ksc = to_f(kh[(size_t)s * HD + ch]);
            const float qrc = to_f(qh[(size_t)r * HD + ch]);
            const float ein = dexp2(sG[r * GLD + ch] - gs);
            qa += qrc * asc * ein;
            qk += qrc * ksc * ein;
            if (s < r) {
              const float brc = to_f(bh[(size_t)r * HD + ch]);
              const float eex = dexp2(sG[(r - 1) * GLD + ch] - gs);
              ba += brc * asc * eex;
              bk += brc * ksc * eex;
            }
          }
        }
        aBA[bi][ii] = ba;
        aBK[bi][ii] = bk;
        aQA[bi][ii] = qa;
        aQK[bi][ii] = qk;
      }
      emit_p(I, J, aQA[bi]);
    }
    emit_ends([&](int s, int ch, float& ae, float& ke) {
      const float f = s < len ? dexp2(sBnd[NSUB * D + ch] - sG[s * GLD + ch]) : 0.f;
      ae = s < len ? to_f(ah[(size_t)s * HD + ch]) * f : 0.f;
      ke = s < len ? to_f(kh[(size_t)s * HD + ch]) * f : 0.f;
    });
  }
  __syncthreads();  // phase A buffers are dead from here on

  float* sA = reinterpret_cast<float*>(smem + SM::MA);
  float* sTd = reinterpret_cast<float*>(smem + SM::TD);
  E* sTb = reinterpret_cast<E*>(smem + SM::TB);
  E* sKt = reinterpret_cast<E*>(smem + SM::KT);
  E* sV = reinterpret_cast<E*>(smem + SM::VV);
  E* sMB = reinterpret_cast<E*>(smem + SM::MB);
  E* sMQ = reinterpret_cast<E*>(smem + SM::MQ);
  E* sY = reinterpret_cast<E*>(smem + SM::YY);

  // ---- B0: -M_ba (fp32), M_bk, M_qk (E), masked; B e^{G^-} and V -----------------------
#pragma unroll
  for (int bi = 0; bi < BPW; ++bi) {
    int I, J;
    if (!dwave_block(w, bi, I, J)) break;
    const int r = 16 * I + m;
    floatx4 ma;
    float mb[4], mq[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int s = 16 * J + 4 * g + ii;
      ma[ii] = s < r ? -aBA[bi][ii] : 0.f;
      mb[ii] = s < r ? aBK[bi][ii] : 0.f;
      mq[ii] = s <= r ? aQK[bi][ii] : 0.f;
    }
    *reinterpret_cast<floatx4*>(sA + r * LDC + 16 * J + 4 * g) = ma;
    store4f(sMB + r * LDK + 16 * J + 4 * g, mb);
    store4f(sMQ + r * LDK + 16 * J + 4 * g, mq);
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rbase + RG * i;
    float vr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vr[j] = val(vv[i], i, j);
    store4f(sKt + r * LD + ch0, bt[i]);
    store4f(sV + r * LD + ch0, vr);
  }
  // T, M_bk and M_qk above the diagonal blocks are zero
  for (int e = t; e < C * C; e += DTHREADS) {
    const int r = e / C, s = e % C;
    if ((s >> 4) > (r >> 4)) {
      sTb[r * LDK + s] = from_f<E>(0.f);
      sMB[r * LDK + s] = from_f<E>(0.f);
      sMQ[r * LDK + s] = from_f<E>(0.f);
    }
  }
  __syncthreads();

  // ---- B1: diagonal blocks T_II = (I + A_II)^{-1}, A = -M_ba (lane j = column j) -----
  if (w < NSUB && lane < 16) {
    const int j = lane, o0 = 16 * w;
    float col[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) x -= sA[(o0 + r) * LDC + o0 + s] * col[s];
      col[r] = x;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sTd[(w * 16 + r) * 20 + j] = col[r];
      sTb[(o0 + r) * LDK + o0 + j] = from_f<E>(col[r]);
    }
  }
  __syncthreads();

  // ---- B2: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, block column J per wave ------------
  if (w < NSUB - 1) {
    const int J = w;
    floatx4 Tcol[NSUB];
#pragma unroll
    for (int K = 0; K < NSUB; ++K) {
      Tcol[K] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (K == J)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) Tcol[K][ii] = sTd[(K * 16 + 4 * g + ii) * 20 + m];
    }
#pragma unroll
    for (int I = 1; I < NSUB; ++I) {
      if (I <= J) continue;
      floatx4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < I; ++K) {
        if (K < J) continue;
        const floatx4 av4 = *reinterpret_cast<const floatx4*>(sA + (16 * I + m) * LDC + 16 * K + 4 * g);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) X = __builtin_amdgcn_mfma_f32_16x16x4f32(av4[jj], Tcol[K][jj], X, 0, 0, 0);
      }
      const floatx4 tii = *reinterpret_cast<const floatx4*>(sTd + (I * 16 + m) * 20 + 4 * g);
      floatx4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tii[jj], X[jj], Y, 0, 0, 0);
      Tcol[I] = -Y;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sTb[(16 * I + 4 * g + ii) * LDK + 16 * J + m] = from_f<E>(-Y[ii]);
    }
  }

  // ---- B3a: V fragments and M_qk V to the record; M_bk V in registers ----------------
  const int ct = w;  // this wave's 16 value columns
  floatx4 yk[NRT];
  {
    FragT bV[NKC];
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) {
      bV[kb] = frag_colk(sV, LD, 16 * ct + m, 32 * kb, g);
      store_frag<E>(rec + RC::VB + ((size_t)(ct * NKC + kb) * 64 + lane) * 8, bV[kb]);
    }
    floatx4 ao[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      yk[rt] = ao[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= (rt >> 1); ++kb) {  // both matrices are lower triangular
        mma(yk[rt], frag_rowk(sMB, LDK, 16 * rt + m, 32 * kb, g), bV[kb]);  // (M_bk V)[16 rt + 4 g + ii][16 ct + m]
        mma(ao[rt], bV[kb], frag_rowk(sMQ, LDK, 16 * rt + m, 32 * kb, g));  // (M_qk V)[16 rt + m][16 ct + 4 g + ii]
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {  // accumulator order per (slab, row tile): 512 contiguous bytes
      const float oo[4] = {ao[rt][0], ao[rt][1], ao[rt][2], ao[rt][3]};
      store4f(rec + RC::OI + ((size_t)(ct * NRT + rt) * 64 + lane) * 4, oo);
    }
  }
  __syncthreads();  // M_bk and M_qk are read; T is complete
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) sY[(16 * rt + 4 * g + ii) * LD + 16 * ct + m] = from_f<E>(yk[rt][ii]);
  __syncthreads();

  // ---- B3b: W_b = T (B e^{G^-}) (computed transposed, fragment order) and U = T (M_bk V).
  //      Wave w takes the slab pair 2 (w & 3), 2 (w & 3) + 1 and the row tiles
  //      2 (w >> 2), 2 (w >> 2) + 1, so both halves of a W_b slot come from one wave.
  {
    const int ct0 = 2 * (w & 3), rt0 = 2 * (w >> 2);
    FragT bK[2][NKC], bY[2][NKC];
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) {
        bK[cl][kb] = frag_colk(sKt, LD, 16 * (ct0 + cl) + m, 32 * kb, g);
        bY[cl][kb] = frag_colk(sY, LD, 16 * (ct0 + cl) + m, 32 * kb, g);
      }
#pragma unroll
    for (int rl = 0; rl < 2; ++rl) {
      const int rt = rt0 + rl;
      floatx4 aw[2] = {zero4, zero4}, au[2] = {zero4, zero4};
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) {
        if (kb > (rt >> 1)) break;  // T is lower triangular (rt is uniform over the wave)
        const FragT aT = frag_rowk(sTb, LDK, 16 * rt + m, 32 * kb, g);
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
          mma(aw[cl], bK[cl][kb], aT);  // lane (m, g): W_b[16 rt + m][16 (ct0 + cl) + 4 g + ii]
          mma(au[cl], aT, bY[cl][kb]);  // lane (m, g): U[16 rt + 4 g + ii][16 (ct0 + cl) + m]
        }
      }
      store_frag<E>(rec + RC::WN + ((size_t)(rt * 4 + (w & 3)) * 64 + lane) * 8, acc_pair_to_frag<E>(aw[0], aw[1]));
#pragma unroll
      for (int cl = 0; cl < 2; ++cl) {
        const float uo[4] = {au[cl][0], au[cl][1], au[cl][2], au[cl][3]};
        store4f(rec + RC::UU + ((size_t)((ct0 + cl) * NRT + rt) * 64 + lane) * 4, uo);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
size_t dplr_record_bytes(int dtype) { return dtype == 0 ? RecD<__bf16, DC>::BYTES : RecD<float, DC>::BYTES; }

PrefillWs dplr_ws_layout(int B, int T, int H, int num_seqs, bool varlen, int dtype) {
  return plan_ws_layout(B, T, H, num_seqs, varlen, DC, dplr_record_bytes(dtype));
}

size_t dplr_workspace_bytes(int B, int T, int H, int num_seqs, bool varlen, int dtype) {
  return dplr_ws_layout(B, T, H, num_seqs, varlen, dtype).total;
}

namespace {
template <typename E>
hipError_t launch_dplr_typed(const void* q, const void* k, const void* v, const void* a, const void* b,
                             const float* log_alpha, const float* initial_state, const int32_t* cu_seqlens, int N,
                             void* o, float* final_state, int T, int H, int64_t mc, const PrefillWs& l, char* ws,
                             hipStream_t stream) {
  int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + l.off_chunk_off);
  int2* info = reinterpret_cast<int2*>(ws + l.off_info);
  char* records = ws + l.off_records;
  trace_begin(stream);
  const int total_tokens = cu_seqlens ? T : N * T;
  hipError_t e = launch_plan(cu_seqlens, N, T, total_tokens, DC, mc, chunk_off, info, stream);
  trace_mark(stream, 0);
  if (e != hipSuccess) return e;
  if (mc > 0) {
    hipLaunchKernelGGL(dplr_intra_kernel<E>, dim3((unsigned)(mc * H)), dim3(DTHREADS), 0, stream, (const E*)q,
                       (const E*)k, (const E*)v, (const E*)a, (const E*)b, log_alpha, chunk_off + N, info, H, (int)mc,
                       records);
    e = hipGetLastError();
    trace_mark(stream, 1);
    if (e != hipSuccess) return e;
  }
  const int64_t slots = ((int64_t)N * H + 7) / 8;
  if (slots > 0) {
    if constexpr (std::is_same<E, __bf16>::value) {
      hipLaunchKernelGGL((inter_wg_kernel<INTER_LOOKAHEAD, true>), dim3((unsigned)(slots * 64)), dim3(256), 0,
                         stream, records, chunk_off, cu_seqlens, T, total_tokens, initial_state, final_state,
                         (__bf16*)o, N, H, (int)mc);
    } else {
      hipLaunchKernelGGL((inter_kernel<E, DC, true>), dim3((unsigned)(slots * 64)), dim3(64), 0, stream, records,
                         chunk_off, info, initial_state, final_state, (E*)o, N, H, (int)mc);
    }
    e = hipGetLastError();
    trace_mark(stream, 2);
  }
  return e;
}
}  // namespace

hipError_t launch_dplr(int dtype, const void* q, const void* k, const void* v, const void* a, const void* b,
                       const float* log_alpha, const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                       void* o, float* final_state, int B, int T, int H, void* workspace, hipStream_t stream) {
  const bool varlen = cu_seqlens != nullptr;
  const int N = varlen ? num_seqs : B;
  const PrefillWs l = dplr_ws_layout(B, T, H, num_seqs, varlen, dtype);
  const int64_t mc = max_chunks(B, T, num_seqs, varlen, DC);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == 0)
    return launch_dplr_typed<__bf16>(q, k, v, a, b, log_alpha, initial_state, cu_seqlens, N, o, final_state, T, H,
                                     mc, l, ws, stream);
  return launch_dplr_typed<float>(q, k, v, a, b, log_alpha, initial_state, cu_seqlens, N, o, final_state, T, H, mc,
                                  l, ws, stream);
}

}  // namespace kda
