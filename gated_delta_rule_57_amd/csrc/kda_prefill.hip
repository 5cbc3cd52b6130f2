// Chunked KDA prefill on gfx950: chunk plan, intra-chunk kernel, inter-chunk
// state-and-output kernel.
//
// Method (GeekNews "Kimi Linear" summary, section "청크 단위 병렬 알고리듬";
// "From GPT-2 to Kimi K3" digest, section "DeltaNet 병렬화 -- 청크 단위 학습"):
// each sequence is cut into chunks of C tokens. Inside a chunk (rows r, s;
// g_r = sum_{j<=r} log_alpha_j per channel; S_0 the state entering the chunk):
//   A    = tril_strict(beta (K e^G)(K e^-G)^T)           decay-weighted key products
//   T    = (I + A)^{-1}                                   forward substitution (UT transform)
//   W    = T diag(beta)(K e^G) ,  U = T diag(beta) V      WY factors
//   U~   = U - W S_0
//   P    = tril((Q e^G)(K e^-G)^T)                        causal in-chunk scores
//   O    = (Q e^G) S_0 + P U~
//   S_C  = Diag(e^{g_C}) S_0 + (K e^{g_C - G})^T U~
// The diagonal-plus-low-rank transition has both low-rank factors tied to k, so a
// chunk needs only the two C x C matrices A and P (section "일반 DPLR보다 줄어든
// 연산량").
//
// Kernels (all launched on the caller's stream):
//   plan_kernel   cu_seqlens (or B fixed-length rows) -> per-sequence first chunk and
//                 per-chunk (first token, length).
//   intra_kernel  one work-group per (chunk, head), fully parallel: everything that
//                 does not depend on the state -- G, A, T, W, U, Q e^G, P,
//                 K e^{g_C-G}, e^{g_C} -- written to a per-(chunk, head) record in
//                 the MFMA fragment order the next kernel consumes.
//   inter kernels one work-group per (sequence, head, 16 value columns), serial over
//                 the sequence's chunks with its 128 x 16 slab of the fp32 state held in
//                 accumulator registers: U~, O and the state update chain from one
//                 MFMA to the next without leaving registers. The value columns of
//                 S evolve independently, which is what makes the slab split exact.
//                 inter_wg_kernel (bf16, 64-token chunks) and inter16_kernel
//                 (16-token chunks) spread a slab over four waves and have each
//                 record line pulled into L2 by one wave of the head a few chunks
//                 ahead; inter_kernel (fp32, 64-token chunks) uses one wave.
//
// In-chunk decay (the pages note that fine-grained decay makes the in-chunk
// division numerically delicate): everything is done in log2 units (x = log2 alpha)
// and the chunk's rows are grouped in sub-chunks of 16. Every exponent is kept a
// sum of the decays it spans, never the difference of two long cumulative sums, so
// fp32 rounding stays relative to the exponent itself:
//   loc_r = x over rows [first row of r's sub-chunk, r]    (running sum, <= 0)
//   suf_s = x over rows (s, last row of s's sub-chunk]     (reverse running sum, <= 0)
//   R_I   = x over sub-chunk I;  b_I = R_0 + ... + R_{I-1}
// For an A / P block (I, J), r in sub-chunk I and s in sub-chunk J <= I:
//   gh_r - gh_s = loc_r + E_IJ + suf_s,  E_IJ = R_{J+1} + ... + R_{I-1}, E_II = -R_I
// The first and last terms belong to one row each, so they are applied once per row
// (lhs_r = x_r 2^(loc_r), x = k for A, q for P; rhs_s = k_s 2^(suf_s)); 2^(E_IJ) is a
// per-channel scale of the block, <= 1 off the diagonal and 2^(-R_I) on it. When
// -R_I exceeds 120 for some sub-chunk, the chunk instead takes an exact path whose
// operands are built per block from the raw inputs, and that diagonal block is
// summed on the VALU with 2^(gh_r - gh_s) per element, the exponent taken as
// loc_r - loc_s or suf_s - suf_r, whichever subtracts the smaller sum; no factor can
// overflow for any input. Q e^G, K e^G (exponent b_I + loc_r), K e^{g_C-G}
// (suf_s + E_{J,n}) and e^{g_C} only need exponents <= 0 and are taken directly.
#include <algorithm>
#include <type_traits>

#include "kda_device.h"
#include "kda_fusion_dev.h"
#include "kda_internal.h"
#include "kda_inter16.h"
#include "kda_inter64.h"
#include "kda_record.h"

namespace kda {

namespace {

constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float DIAG_RANGE_LIMIT = 120.f;  // log2 units
// A bf16 64-token chunk whose total decay stays within this range (log2 units) in every
// channel takes the direct form: x_r 2^(gh_r) >= x_r 2^-96 stays a normal number for any
// component above 2^-30, and k_s 2^(-gh_s) <= 2^96 is far from overflow
constexpr float DIRECT_RANGE_LIMIT = 96.f;

// decay granularity (kda_fusion.gate_kind): one per key channel (KDA), one per
// (token, head) (Gated DeltaNet), none (DeltaNet)
constexpr int GATE_CHANNEL = 0, GATE_HEAD = 1, GATE_NONE = 2;

__host__ __device__ constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Shared-memory plan of the intra-chunk kernel (byte offsets). Phase A buffers are
// dead once the A / P blocks are formed; phase B buffers reuse the same space.
template <typename E, int C>
struct Smem {
  static constexpr int NSUB = C / 16;
  static constexpr int CK = C < 32 ? 32 : C;   // chunk rows padded to whole k-blocks
  static constexpr int NKC = CK / 32;
  static constexpr int LD = D + 8;             // row stride of [rows][128] E matrices
  static constexpr int GLD = D + 4;            // row stride of the fp32 decay cumsum
  static constexpr int LDC = C + 4;            // row stride of the fp32 A matrix
  static constexpr int LDK = CK + 8;           // row stride of E matrices indexed by chunk row
  // phase A: per-channel decays. G holds the log2 decays, then their running sums
  // inside each sub-chunk (loc); SUF the reverse running sums (suf). Scalar gates
  // keep their row sums at G and raw k and q at K and Q.
  static constexpr size_t G = 0;                                          // float[C][GLD]
  static constexpr size_t K = G + al16((size_t)C * GLD * 4);              // E[C][LD]
  static constexpr size_t Q = K + al16((size_t)C * LD * sizeof(E));       // E[C][LD]
  static constexpr size_t A_END = Q + al16((size_t)C * LD * sizeof(E));
  // phase A, factored path: loc (at G) is replaced by the per-row factored operands
  // once every thread holds its own decays in registers; suf sits where the right
  // operands go (RR) and each thread replaces its own entries
  static constexpr size_t LK = 0;                                         // E[C][LD]     k_r 2^(loc_r)
  static constexpr size_t LQ = LK + al16((size_t)C * LD * sizeof(E));     // E[C][LD]     q_r 2^(loc_r)
  static constexpr size_t RR = LQ + al16((size_t)C * LD * sizeof(E));     // float[C][GLD] k_s 2^(suf_s)
  static constexpr size_t SUF = RR;                                       // float[C][GLD] suf
  static constexpr size_t F_END = RR + al16((size_t)C * GLD * 4);
  static_assert(G + (size_t)C * GLD * 4 <= RR, "the suffix sums must not overlap the prefix sums");
  // phase B: A, diagonal blocks of T, T diag(beta), K e^G, V
  static constexpr size_t MA = 0;                                         // float[C][LDC]
  static constexpr size_t TD = MA + al16((size_t)C * LDC * 4);            // float[NSUB][16][20]
  static constexpr size_t TB = TD + al16((size_t)NSUB * 16 * 20 * 4);     // E[C][LDK]
  static constexpr size_t KT = TB + al16((size_t)C * LDK * sizeof(E));    // E[CK][LD]
  static constexpr size_t VV = KT + al16((size_t)CK * LD * sizeof(E));    // E[CK][LD]
  static constexpr size_t B_END = VV + al16((size_t)CK * LD * sizeof(E));
  // tables that live through every phase
  static constexpr size_t BND = cmax(cmax(A_END, F_END), B_END);  // float[NSUB+1][D] b_I
  // per-channel block scales 2^(b_I - b_{J+1}): entry I (I + 1) / 2 + J for the A / P
  // block (I, J <= I), entry NBLK + J for (chunk end, J)
  static constexpr int NBLK = NSUB * (NSUB + 1) / 2;
  static constexpr int NSCALE = NBLK + NSUB;
  static constexpr size_t SCL = BND + (size_t)(NSUB + 1) * D * 4;  // float[NSCALE][D]
  static constexpr size_t BETA = SCL + (size_t)NSCALE * D * 4;     // float[CK]
  static constexpr size_t NRM = BETA + (size_t)CK * 4;            // float[2][CK] prologue scales of k, q
  static constexpr size_t FLAG = NRM + (size_t)2 * CK * 4;        // int[NSUB + 1]: range flags, direct-form flag
  static constexpr size_t GAM = al16(FLAG + 4 * (NSUB + 1));      // float[D] e^{g_C} (direct form)
  static constexpr size_t TOTAL = GAM + (size_t)D * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one gfx950 CU");
};

// Which 16 x 16 block (I, J <= I) of A and P wave w forms in its bi-th slot. The two
// blocks J = 2 kb and 2 kb + 1 of a block row I fill one 16-byte fragment slot of P
// per lane, so they go to the same wave, one after the other, and P leaves the
// kernel as whole slots (half-slot stores cost the kernel several percent). With
// four sub-chunks the waves take 3, 3, 2 and 2 blocks, as a round-robin split would.
template <int NSUB>
__device__ __forceinline__ bool wave_block(int w, int bi, int& I, int& J) {
  if constexpr (NSUB == 1) {
    I = J = 0;
    return w == 0 && bi == 0;
  } else {
    static_assert(NSUB == 4, "block assignment for 16- and 64-token chunks");
    if (bi < 2) {  // (1,0) (1,1) | (2,0) (2,1) | (3,0) (3,1) | (3,2) (3,3)
      I = w < 3 ? w + 1 : 3;
      J = (w < 3 ? 0 : 2) + bi;
      return true;
    }
    I = J = 2 * w;  // (0,0) | (2,2)
    return bi == 2 && w < 2;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Chunk plan. One work-group of 1024 threads. Sequence n is rows [start, end) of
// the packed token axis; it owns chunks [chunk_off[n], chunk_off[n+1]).
// info[c] = (first token, number of tokens) of chunk c.
// Sequence bounds are clamped to [0, total_tokens] and the chunk count to the
// workspace's capacity, so cu_seqlens that break their precondition give
// unspecified results but never an access outside the buffers.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) plan_kernel(const int32_t* __restrict__ cu_seqlens, int N, int T,
                                                    int total_tokens, int C, int capacity,
                                                    int32_t* __restrict__ chunk_off, int2* __restrict__ info) {
  __shared__ int s_scan[1024];
  __shared__ int s_carry;
  const int t = threadIdx.x;

  auto clampt = [&](int x) { return min(max(x, 0), total_tokens); };
  auto seq_start = [&](int n) { return cu_seqlens ? clampt(cu_seqlens[n]) : n * T; };
  auto seq_end = [&](int n) { return cu_seqlens ? clampt(cu_seqlens[n + 1]) : (n + 1) * T; };
  if (t == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int n = base + t;
    int cnt = 0;
    if (n < N) {
      const int len = seq_end(n) - seq_start(n);
      cnt = len > 0 ? (len + C - 1) / C : 0;
    }
    s_scan[t] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int x = t >= off ? s_scan[t - off] : 0;
      __syncthreads();
      s_scan[t] += x;
      __syncthreads();
    }
    const int carry = s_carry;
    if (n < N) chunk_off[n] = min(carry + s_scan[t] - cnt, capacity);
    __syncthreads();
    if (t == 1023) s_carry = min(carry + s_scan[1023], capacity);
    __syncthreads();
  }
  const int total = s_carry;
  if (t == 0) chunk_off[N] = total;
  __syncthreads();
  for (int c = t; c < total; c += 1024) {
    // the largest n with chunk_off[n] <= c; empty sequences are skipped because they
    // share their offset with the next sequence
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (chunk_off[mid] <= c) lo = mid;
      else hi = mid - 1;
    }
    const int tok0 = seq_start(lo) + (c - chunk_off[lo]) * C;
    const int len = min(C, seq_end(lo) - tok0);
    info[c] = make_int2(tok0, len);
  }
}

// ---------------------------------------------------------------------------
// Intra-chunk kernel: one work-group (4 waves) per (chunk, head).
//
// Thread t owns channels 4 (t & 31) .. + 3 of rows (t >> 5) + 8 i in the
// element-wise phases. MFMA products that feed the record are taken in the
// orientation whose accumulator layout already is the fragment layout the
// inter-chunk kernel reads (see kda_device.h): P and -W are computed transposed,
// so each lane stores its four accumulator values as one 8-byte write, with no
// transposition through LDS. Phases (barriers in between):
//   P1  load the chunk (all loads issued before any is waited on); log2 decays
//   P1b cumulative sum over the rows, sub-chunk boundaries, fallback flags
//   P2  Q e^G to the record; K e^G kept in registers; raw q, k to LDS
//   P3  A and P blocks by MFMA (operands built from k, q and G on the fly),
//       P and K e^{g_C-G} to the record
//   B0  beta-scaled, masked A to LDS; K e^G and V to LDS
//   B1  diagonal 16 x 16 blocks of T = (I + A)^{-1} by forward substitution
//   B2  off-diagonal blocks of T, one block column per wave, by fp32 MFMA
//   B3  W = T diag(beta) K e^G (stored as -W) and U = T diag(beta) V
// ---------------------------------------------------------------------------
template <typename E, int C, int GATE>
__global__ void __launch_bounds__(256) intra_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                    const E* __restrict__ v, const float* __restrict__ log_alpha,
                                                    const float* __restrict__ beta,
                                                    int32_t* __restrict__ chunk_off, int2* __restrict__ info,
                                                    int N, int uni_T, int H, int mc, char* __restrict__ records,
                                                    Fusion fu) {
  using SM = Smem<E, C>;
  using RC = Rec<E, C>;
  typedef typename Frag<E>::T FragT;
  typedef typename Vec4<E>::T V4;
  constexpr int NSUB = SM::NSUB, CK = SM::CK, NKC = SM::NKC, LD = SM::LD, GLD = SM::GLD, LDC = SM::LDC,
                LDK = SM::LDK;
  constexpr int NRT = C / 16;
  constexpr int RPT = C / 8;  // rows per thread in element-wise phases

  __shared__ __attribute__((aligned(16))) char smem[SM::TOTAL];
  float* sG = reinterpret_cast<float*>(smem + SM::G);
  E* sK = reinterpret_cast<E*>(smem + SM::K);
  E* sQ = reinterpret_cast<E*>(smem + SM::Q);
  float* sA = reinterpret_cast<float*>(smem + SM::MA);
  float* sTd = reinterpret_cast<float*>(smem + SM::TD);
  E* sTb = reinterpret_cast<E*>(smem + SM::TB);
  E* sKt = reinterpret_cast<E*>(smem + SM::KT);
  E* sV = reinterpret_cast<E*>(smem + SM::VV);
  float* sBnd = reinterpret_cast<float*>(smem + SM::BND);
  float* sBeta = reinterpret_cast<float*>(smem + SM::BETA);
  int* sFlag = reinterpret_cast<int*>(smem + SM::FLAG);
  float* sNrm = reinterpret_cast<float*>(smem + SM::NRM);

  // heads vary fastest over the work-group ids: the work-groups in flight together
  // cover whole token rows of q, k, v and the gates, not one head's 256-byte pieces
  const int c = blockIdx.x / H, h = blockIdx.x - c * H;
  const int t = threadIdx.x;
  int tok0, len;
  if (uni_T > 0) {
    // N sequences of uni_T tokens, no plan kernel: the chunk table is arithmetic (the
    // grid covers it exactly), and head 0's work-groups write it for the state kernels
    // that run after this one
    const int ncs = (uni_T + C - 1) / C;
    const int n = c / ncs, jc = c - n * ncs;
    tok0 = n * uni_T + jc * C;
    len = min(C, uni_T - jc * C);
    if (h == 0 && t == 0) {
      info[c] = make_int2(tok0, len);
      if (jc == 0) chunk_off[n] = c;
      if (c == 0) chunk_off[N] = N * ncs;
    }
  } else {
    if (c >= chunk_off[N]) return;
    const int2 inf = info[c];
    tok0 = inf.x;
    len = inf.y;
  }
  const int lane = t & 63, w = t >> 6, m = lane & 15, g = lane >> 4;
  const int cq = t & 31, ch0 = 4 * cq, rbase = t >> 5;
  const size_t HD = (size_t)H * D;
  char* rec_base = records + ((size_t)h * mc + c) * RC::BYTES;  // head-major: a head's chunks are contiguous
  E* rec = reinterpret_cast<E*>(rec_base);
  float* rec_gamma = reinterpret_cast<float*>(rec_base + RC::GAMMA_BYTES);

  // ---- P1: every load of the chunk in flight at once (rows past len read row 0 and
  //          are zeroed), then log2-domain decays into sG ----------------------------
  // The decays and beta are issued first and k, q, v after a compiler fence: memory
  // counters count in issue order, so the decay phases wait for the decays only, and
  // k, q, v (raw, converted where first used) land while those phases run.
  float kr[RPT][4], qr[RPT][4], vr[RPT][4];
  typename Vec4<E>::T kraw[RPT], qraw[RPT], vraw[RPT];
  floatx4 la[RPT];
  auto row_off = [&](int i) {
    const int r = rbase + 8 * i;
    return (size_t)(tok0 + (r < len ? r : 0)) * HD + (size_t)h * D + ch0;
  };
  if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) la[i] = load_nt(reinterpret_cast<const floatx4*>(log_alpha + row_off(i)));
  }
  float braw = 0.f, lraw = 0.f;
  if (t < CK && t < len) {
    braw = beta[(size_t)(tok0 + t) * H + h];
    if constexpr (GATE == GATE_HEAD) lraw = log_alpha[(size_t)(tok0 + t) * H + h];
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const size_t off = row_off(i);
    kraw[i] = load_nt(reinterpret_cast<const typename Vec4<E>::T*>(k + off));
    qraw[i] = load_nt(reinterpret_cast<const typename Vec4<E>::T*>(q + off));
    vraw[i] = load_nt(reinterpret_cast<const typename Vec4<E>::T*>(v + off));
  }
  float la_row = 0.f;  // scalar gate: log decay of row t (t < CK), natural-log units
  if (t < CK) {
    float bt = 0.f;
    if (t < len) {
      bt = braw;
      if (fu.beta_preactivation) bt = sigmoid_f(bt);
      if constexpr (GATE == GATE_HEAD) {
        la_row = lraw;
        if (fu.gate_preactivation) la_row = -softplus_f(la_row);
      }
    }
    sBeta[t] = bt;
  }
  if (t <= NSUB) sFlag[t] = 0;
  // Rows past len are zeroed and (prologue on raw inputs) q and k rows L2-normalised
  // where they are first needed, after the decay phases: nothing before the first
  // barrier waits for the q, k and v loads. A row's 128 channels are spread over the
  // 32 lanes of one half-wave (4 each), so its squared norm is a half-wave sum.
  auto prep_rows = [&] {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      asm volatile("" : "+v"(kraw[i]), "+v"(qraw[i]), "+v"(vraw[i]));  // converted here, not earlier
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kr[i][j] = to_f(kraw[i][j]);
        qr[i][j] = to_f(qraw[i][j]);
        vr[i][j] = to_f(vraw[i][j]);
      }
    }
    if (fu.normalize_qk) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sk += kr[i][j] * kr[i][j];
          sq += qr[i][j] * qr[i][j];
        }
        const float ik = rsqrtf(half_wave_sum(sk) + fu.qk_eps), iq = rsqrtf(half_wave_sum(sq) + fu.qk_eps);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kr[i][j] *= ik;
          qr[i][j] *= iq;
        }
        if (GATE == GATE_CHANNEL && cq == 0) {  // the row's scales, for the exact path's reloads of raw k and q
          sNrm[rbase + 8 * i] = ik;
          sNrm[CK + rbase + 8 * i] = iq;
        }
      }
    } else if (GATE == GATE_CHANNEL && cq == 0) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        sNrm[rbase + 8 * i] = 1.f;
        sNrm[CK + rbase + 8 * i] = 1.f;
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + 8 * i;
      const bool valid = r < len;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kr[i][j] = valid ? kr[i][j] : 0.f;
        qr[i][j] = valid ? qr[i][j] : 0.f;
        vr[i][j] = valid ? vr[i][j] : 0.f;
      }
    }
  };
  constexpr int NBLK = SM::NBLK;
  constexpr int BPW = (NBLK + 3) / 4;
  static_assert(NBLK <= 10, "wave_block covers up to four sub-chunks");
  // P to the record in whole 16-byte slots: block (I, J) is half of slot (I, J / 2);
  // an even block waits in p_lo for its odd partner unless it is the last of its row
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
  // (K e^{g_C - G})^T to the record: item (channel, 4-row group fg, k-block kb) is one
  // lane's whole slot, rows 32 kb + 4 fg + j and 32 kb + 16 + 4 fg + j; 16 consecutive
  // items fill 256 contiguous bytes. kval(s, ch) gives the value of chunk row s < C.
  auto emit_ke = [&](auto kval) {
    for (int it = t; it < D * NKC * 4; it += 256) {
      const int ch = it & (D - 1), fg = (it >> 7) & 3, kb = it >> 9;
      floatx4 lo, hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s0 = 32 * kb + 4 * fg + j, s1 = s0 + 16;
        lo[j] = s0 < C ? kval(s0, ch) : 0.f;
        hi[j] = s1 < C ? kval(s1, ch) : 0.f;
      }
      store_frag<E>(rec + RC::KE + ((size_t)((ch >> 4) * NKC + kb) * 64 + (ch & 15) + 16 * fg) * 8,
                    acc_pair_to_frag<E>(lo, hi));
    }
  };
  float ktr[RPT][4];
  floatx4 accA[BPW], accP[BPW];
  if constexpr (GATE == GATE_CHANNEL) {
  if (fu.gate_preactivation) {  // log alpha = -softplus(a), kept in natural-log units here
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) la[i][j] = -softplus_f(la[i][j]);
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rbase + 8 * i;
    floatx4 l2 = r < len ? la[i] * LOG2E_F : floatx4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<floatx4*>(sG + r * GLD + ch0) = l2;
  }
  __syncthreads();
  float* sSuf = reinterpret_cast<float*>(smem + SM::SUF);
  {  // ---- P1b: per channel and sub-chunk, running sums of the log2 decays from the
     //      sub-chunk's first row (loc, over the decays at sG) and to its last row
     //      (suf, to sSuf); the two halves of the work-group take half the sub-chunks
    const int chn = t & 127, half = t >> 7;
    constexpr int SPH = NSUB >= 2 ? NSUB / 2 : 1;
    if (NSUB >= 2 || half == 0) {
#pragma unroll
      for (int u = 0; u < SPH; ++u) {
        const int r0 = 16 * (half * SPH + u);
        float x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = sG[(r0 + j) * GLD + chn];
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          acc += x[j];
          sG[(r0 + j) * GLD + chn] = acc;
        }
        acc = 0.f;
#pragma unroll
        for (int j = 15; j >= 0; --j) {
          sSuf[(r0 + j) * GLD + chn] = acc;
          acc += x[j];
        }
      }
    }
  }
  __syncthreads();
  float* sScl = reinterpret_cast<float*>(smem + SM::SCL);
  if (t < D) {
    float R[NSUB], bnd[NSUB + 1];
    bnd[0] = 0.f;
#pragma unroll
    for (int I = 0; I < NSUB; ++I) {
      R[I] = sG[(16 * I + 15) * GLD + t];
      bnd[I + 1] = bnd[I] + R[I];
    }
#pragma unroll
    for (int I = 0; I <= NSUB; ++I) sBnd[I * D + t] = bnd[I];
    rec_gamma[t] = fast_exp2(bnd[NSUB]);
    reinterpret_cast<float*>(smem + SM::GAM)[t] = fast_exp2(bnd[NSUB]);
#pragma unroll
    for (int I = 0; I < NSUB; ++I)
      if (!(-R[I] <= DIAG_RANGE_LIMIT)) atomicOr(&sFlag[I], 1);
    if (!(-bnd[NSUB] <= DIRECT_RANGE_LIMIT)) atomicOr(&sFlag[NSUB], 1);
    // block scales 2^(E_IJ): sums of the whole sub-chunks strictly between J and I
    // (<= 1), 2^(-R_I) on the diagonal (used only while -R_I <= the limit); then
    // 2^(R_{J+1} + ... + R_{n-1}) for the chunk end
#pragma unroll
    for (int I = 0; I < NSUB; ++I) {
      float e = 0.f;
#pragma unroll
      for (int J = I - 1; J >= 0; --J) {
        sScl[(I * (I + 1) / 2 + J) * D + t] = fast_exp2(e);
        e += R[J];
      }
      sScl[(I * (I + 1) / 2 + I) * D + t] = fast_exp2(-R[I]);
    }
    float e = 0.f;
#pragma unroll
    for (int J = NSUB - 1; J >= 0; --J) {
      sScl[(SM::NBLK + J) * D + t] = fast_exp2(e);
      e += R[J];
    }
  }
  __syncthreads();
  bool exact = false;  // some diagonal block exceeds the range limit: per-element path
#pragma unroll
  for (int I = 0; I < NSUB; ++I) exact |= sFlag[I] != 0;
  // the whole chunk within the direct range (implies !exact: -R_I <= -b_n <= the range)
  constexpr bool HAS_DIRECT = std::is_same<E, __bf16>::value && C == 64;
  const bool direct = HAS_DIRECT && sFlag[NSUB] == 0;
  prep_rows();

  if (direct) {
    // ---- P2 (direct): the chunk's decay is within the direct range, so
    //      2^(gh_r - gh_s) = 2^(gh_r) 2^(-gh_s) splits with no scale table:
    //      lhs_r = x_r 2^(gh_r) (x = k, q: also K e^G and Q e^G), rhs_s = k_s 2^(-gh_s),
    //      gh = b_I + loc ------------------------------------------------------------
    E* sLK = reinterpret_cast<E*>(smem + SM::LK);
    E* sLQ = reinterpret_cast<E*>(smem + SM::LQ);
    E* sRK = reinterpret_cast<E*>(smem + SM::RR);  // E[C][LD], inside RR
    V4 lkv[RPT], lqv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + 8 * i, I = r >> 4;
      const floatx4 loc = *reinterpret_cast<const floatx4*>(sG + r * GLD + ch0);
      const floatx4 b0 = *reinterpret_cast<const floatx4*>(sBnd + I * D + ch0);
      float qt[4];
      V4 rk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gh = b0[j] + loc[j];
        const float eg = fast_exp2(gh);  // >= 2^-96
        qt[j] = qr[i][j] * eg;
        ktr[i][j] = kr[i][j] * eg;
        lkv[i][j] = from_f<E>(ktr[i][j]);
        lqv[i][j] = from_f<E>(qt[j]);
        rk[j] = from_f<E>(kr[i][j] * fast_exp2(-gh));  // <= 2^96 |k|
      }
      *reinterpret_cast<V4*>(sRK + r * LD + ch0) = rk;
    }
    __syncthreads();  // every thread has its decays; the left operands overwrite the cumsum
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + 8 * i;
      *reinterpret_cast<V4*>(sLK + r * LD + ch0) = lkv[i];
      *reinterpret_cast<V4*>(sLQ + r * LD + ch0) = lqv[i];
    }
    __syncthreads();
    // ---- P3 (direct): the blocks straight from the operands; entries above the
    //      diagonal (up to 2^96 |x| |k|) are dropped where A and P are taken
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      accA[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      accP[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      int I, J;
      if (!wave_block<NSUB>(w, bi, I, J)) break;
      const int rrow = 16 * I + m, srow = 16 * J + m;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        FragT lk, lq, rhs;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ch = 32 * kb + 16 * hh + 4 * g;
          const V4 a = *reinterpret_cast<const V4*>(sLK + rrow * LD + ch);
          const V4 bq = *reinterpret_cast<const V4*>(sLQ + rrow * LD + ch);
          const V4 rv = *reinterpret_cast<const V4*>(sRK + srow * LD + ch);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            lk[4 * hh + j] = a[j];
            lq[4 * hh + j] = bq[j];
            rhs[4 * hh + j] = rv[j];
          }
        }
        mma(accA[bi], rhs, lk);
        mma(accP[bi], rhs, lq);
        // lq is Q e^G of row tile I, k-block kb in the record's slot order: the wave
        // with the tile's J = 0 block stores it, 1 KiB contiguous per instruction
        if (J == 0) store_frag<E>(rec + RC::QT + ((size_t)(I * 4 + kb) * 64 + lane) * 8, lq);
      }
      emit_p(I, J, accP[bi]);
    }
    // (K e^{g_C - G})^T = rhs_s 2^(g_C) to the record
    const float* sGam = reinterpret_cast<const float*>(smem + SM::GAM);
    emit_ke([&](int s, int ch) { return to_f(sRK[s * LD + ch]) * sGam[ch]; });
  } else if (!exact) {
    // ---- P2 (factored path): Q e^G to the record, K e^G kept for B0, and per row
    //      the operands of every A / P block:
    //        lhs_r = x_r 2^(loc_r)    (x = k or q)
    //        rhs_s = k_s 2^(suf_s)
    //      both with exponents <= 0. Block (I, J) is lhs_I diag(2^(E_IJ)) rhs_J^T,
    //      the per-channel scale taken from the table above. rhs_s replaces suf_s in
    //      place (each thread its own entries).
    E* sLK = reinterpret_cast<E*>(smem + SM::LK);
    E* sLQ = reinterpret_cast<E*>(smem + SM::LQ);
    float* sRR = reinterpret_cast<float*>(smem + SM::RR);
    V4 lkv[RPT], lqv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + 8 * i, I = r >> 4;
      const floatx4 loc = *reinterpret_cast<const floatx4*>(sG + r * GLD + ch0);
      const floatx4 suf = *reinterpret_cast<const floatx4*>(sSuf + r * GLD + ch0);
      const floatx4 b0 = *reinterpret_cast<const floatx4*>(sBnd + I * D + ch0);
      float qt[4];
      floatx4 rr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float kk = kr[i][j], qq = qr[i][j];
        const float eg = fast_exp2(b0[j] + loc[j]);  // exponent <= 0
        const float pl = fast_exp2(loc[j]);          // exponent <= 0
        qt[j] = qq * eg;
        ktr[i][j] = kk * eg;
        lkv[i][j] = from_f<E>(kk * pl);
        lqv[i][j] = from_f<E>(qq * pl);
        rr[j] = kk * fast_exp2(suf[j]);             // exponent <= 0
      }
      *reinterpret_cast<floatx4*>(sRR + r * GLD + ch0) = rr;
      const int kb = ch0 >> 5, co = ch0 & 31;
      const int fg = (co & 15) >> 2, fh = co >> 4;
      store4f(rec + RC::QT + ((size_t)((r >> 4) * 4 + kb) * 64 + (r & 15) + 16 * fg) * 8 + 4 * fh, qt);
    }
    __syncthreads();  // every thread has its decays; the left operands overwrite the cumsum
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + 8 * i;
      *reinterpret_cast<V4*>(sLK + r * LD + ch0) = lkv[i];
      *reinterpret_cast<V4*>(sLQ + r * LD + ch0) = lqv[i];
    }
    __syncthreads();

    // ---- P3 (factored path): one 16 x 16 block (I, J <= I) per wave at a time,
    //      computed transposed as in the exact path ------------------------------
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      accA[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      accP[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      int I, J;
      if (!wave_block<NSUB>(w, bi, I, J)) break;
      const int rrow = 16 * I + m, srow = 16 * J + m;
      const float* scl = sScl + (size_t)(I * (I + 1) / 2 + J) * D;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        FragT lk, lq, rhs;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ch = 32 * kb + 16 * hh + 4 * g;
          const V4 a = *reinterpret_cast<const V4*>(sLK + rrow * LD + ch);
          const V4 bq = *reinterpret_cast<const V4*>(sLQ + rrow * LD + ch);
          const floatx4 rv = *reinterpret_cast<const floatx4*>(sRR + srow * GLD + ch);
          const floatx4 sc = *reinterpret_cast<const floatx4*>(scl + ch);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            lk[4 * hh + j] = a[j];
            lq[4 * hh + j] = bq[j];
            rhs[4 * hh + j] = from_f<E>(rv[j] * sc[j]);
          }
        }
        mma(accA[bi], rhs, lk);
        mma(accP[bi], rhs, lq);
      }
      emit_p(I, J, accP[bi]);
    }
    // (K e^{g_C - G})^T = rhs_s 2^(g_C - b_{J+1}) to the record
    emit_ke([&](int s, int ch) { return sRR[s * GLD + ch] * sScl[(NBLK + (s >> 4)) * D + ch]; });
  } else {
    // ---- P2 (exact path): Q e^G straight to its fragment slot (4 consecutive channels are half of a
    //          lane's fragment); K e^G kept for B0. loc and suf stay in LDS for P3,
    //          which takes raw q and k from global memory (the rows just loaded) --------
  #pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + 8 * i, I = r >> 4;
      const floatx4 loc = *reinterpret_cast<const floatx4*>(sG + r * GLD + ch0);
      const floatx4 b0 = *reinterpret_cast<const floatx4*>(sBnd + I * D + ch0);
      float qt[4];
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float eg = fast_exp2(b0[j] + loc[j]);  // exponent <= 0
        qt[j] = qr[i][j] * eg;
        ktr[i][j] = kr[i][j] * eg;
      }
      const int kb = ch0 >> 5, co = ch0 & 31;
      const int fg = (co & 15) >> 2, fh = co >> 4;
      store4f(rec + RC::QT + ((size_t)((r >> 4) * 4 + kb) * 64 + (r & 15) + 16 * fg) * 8 + 4 * fh, qt);
    }
    // raw (prologue-scaled) k (which 0) or q (which 1) of chunk row r, channels ch .. ch + 3;
    // zero past len
    auto raw4 = [&](int which, int r, int ch, float out[4]) {
      if (r < len) {
        load4f((which ? q : k) + (size_t)(tok0 + r) * HD + (size_t)h * D + ch, out);
        const float f = sNrm[which * CK + r];
  #pragma unroll
        for (int j = 0; j < 4; ++j) out[j] *= f;
      } else {
  #pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = 0.f;
      }
    };

    // ---- P3: A and P, one 16 x 16 block (I, J <= I) per wave at a time. Computed
    //          transposed: lane (m, g), element ii holds entry (r = 16 I + m,
    //          s = 16 J + 4 g + ii). lhs_r = x_r 2^(loc_r) (x = k or q),
    //          rhs_s = k_s 2^(suf_s) 2^(E_IJ). -------------------------------------------
  #pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      accA[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      accP[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      int I, J;
      if (!wave_block<NSUB>(w, bi, I, J)) break;
      if (J == I && sFlag[I]) {
        // element-wise path: 2^(gh_r - gh_s) with exponent <= 0 for every kept entry,
        // as loc_r - loc_s or suf_s - suf_r, whichever subtracts the smaller sum
        const int r = 16 * I + m;
        float sa[4] = {0.f, 0.f, 0.f, 0.f}, sp[4] = {0.f, 0.f, 0.f, 0.f};
        for (int ch = 0; ch < D; ch += 4) {
          float kk[4], qq[4];
          raw4(0, r, ch, kk);
          raw4(1, r, ch, qq);
          const floatx4 lr = *reinterpret_cast<const floatx4*>(sG + r * GLD + ch);
          const floatx4 fr = *reinterpret_cast<const floatx4*>(sSuf + r * GLD + ch);
  #pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int s = 16 * J + 4 * g + ii;
            if (s > r) continue;
            float ks[4];
            raw4(0, s, ch, ks);
            const floatx4 ls = *reinterpret_cast<const floatx4*>(sG + s * GLD + ch);
            const floatx4 fs = *reinterpret_cast<const floatx4*>(sSuf + s * GLD + ch);
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float ex = fabsf(ls[j]) <= fabsf(fr[j]) ? lr[j] - ls[j] : fs[j] - fr[j];
              const float kd = ks[j] * fast_exp2(ex);
              sa[ii] += kk[j] * kd;
              sp[ii] += qq[j] * kd;
            }
          }
        }
  #pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          accA[bi][ii] = sa[ii];
          accP[bi][ii] = sp[ii];
        }
      } else {
        const int rrow = 16 * I + m, srow = 16 * J + m;
        const float* scl = sScl + (size_t)(I * (I + 1) / 2 + J) * D;
  #pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          FragT lk, lq, rhs;
  #pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int ch = 32 * kb + 16 * hh + 4 * g;
            float kk[4], qq[4], ks[4];
            raw4(0, rrow, ch, kk);
            raw4(1, rrow, ch, qq);
            raw4(0, srow, ch, ks);
            const floatx4 lr = *reinterpret_cast<const floatx4*>(sG + rrow * GLD + ch);
            const floatx4 fs = *reinterpret_cast<const floatx4*>(sSuf + srow * GLD + ch);
            const floatx4 sc = *reinterpret_cast<const floatx4*>(scl + ch);
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float pl = fast_exp2(lr[j]);
              lk[4 * hh + j] = from_f<E>(kk[j] * pl);
              lq[4 * hh + j] = from_f<E>(qq[j] * pl);
              rhs[4 * hh + j] = from_f<E>(ks[j] * fast_exp2(fs[j]) * sc[j]);
            }
          }
          mma(accA[bi], rhs, lk);
          mma(accP[bi], rhs, lq);
        }
      }
      emit_p(I, J, accP[bi]);
    }
    // (K e^{g_C - G})^T to the record: k_s 2^(suf_s) 2^(R_{J+1} + ... + R_{n-1})
    emit_ke([&](int s, int ch) {
      const float ks = s < len ? to_f(k[(size_t)(tok0 + s) * HD + (size_t)h * D + ch]) * sNrm[s] : 0.f;
      return ks * fast_exp2(sSuf[s * GLD + ch]) * sScl[(NBLK + (s >> 4)) * D + ch];
    });
  }
  } else {
    // ---- scalar gate: one decay per (token, head) (GATE_HEAD), or none (GATE_NONE).
    //      The decay of a row pair is the scalar 2^(gh_r - gh_s), exponent <= 0 for
    //      s <= r, so the raw products k k^T and q k^T are scaled per element after
    //      the MFMA and no factoring or fallback is needed ------------------------
    float* sGs = sG;        // float[CK]: running sums of the row decays (log2) from row 0
    float* sGf = sG + 64;   // float[CK]: running sums over the rows after s to the chunk end
    if (w == 0) {           // one wave holds every row (CK <= 64)
      float x = 0.f;
      if constexpr (GATE == GATE_HEAD) x = la_row * LOG2E_F;  // zero past len
      float f = __shfl_down(x, 1, 64);
      if (lane == 63) f = 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64), z = __shfl_down(f, off, 64);
        if (lane >= off) x += y;
        if (lane + off < 64) f += z;
      }
      if (lane < CK) {
        sGs[lane] = x;
        sGf[lane] = f;
      }
    }
    __syncthreads();
    const float gC = sGs[C - 1];
    if (t < D) rec_gamma[t] = fast_exp2(gC);
    prep_rows();
    // ---- P2 (scalar): Q e^G to the record, K e^G kept for B0, raw q, k to LDS --
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rbase + 8 * i;
      const float eg = GATE == GATE_NONE ? 1.f : fast_exp2(sGs[r]);
      float qt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qt[j] = qr[i][j] * eg;
        ktr[i][j] = kr[i][j] * eg;
      }
      store4f(sK + r * LD + ch0, kr[i]);
      store4f(sQ + r * LD + ch0, qr[i]);
      const int kb = ch0 >> 5, co = ch0 & 31;
      const int fg = (co & 15) >> 2, fh = co >> 4;
      store4f(rec + RC::QT + ((size_t)((r >> 4) * 4 + kb) * 64 + (r & 15) + 16 * fg) * 8 + 4 * fh, qt);
    }
    __syncthreads();
    // ---- P3 (scalar): raw block products, then the pair decay per element ------
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      accA[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      accP[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
      int I, J;
      if (!wave_block<NSUB>(w, bi, I, J)) break;
      const int rrow = 16 * I + m, srow = 16 * J + m;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        FragT lk, lq, rhs;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ch = 32 * kb + 16 * hh + 4 * g;
          const V4 a = *reinterpret_cast<const V4*>(sK + rrow * LD + ch);
          const V4 bq = *reinterpret_cast<const V4*>(sQ + rrow * LD + ch);
          const V4 bs = *reinterpret_cast<const V4*>(sK + srow * LD + ch);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            lk[4 * hh + j] = a[j];
            lq[4 * hh + j] = bq[j];
            rhs[4 * hh + j] = bs[j];
          }
        }
        mma(accA[bi], rhs, lk);
        mma(accP[bi], rhs, lq);
      }
      const int r = rrow;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int s = 16 * J + 4 * g + ii;
        // 2^(gh_r - gh_s) from whichever running sums subtract the smaller total
        const float ex = fabsf(sGs[s]) <= fabsf(sGf[r]) ? sGs[r] - sGs[s] : sGf[s] - sGf[r];
        const float f = s <= r ? (GATE == GATE_NONE ? 1.f : fast_exp2(ex)) : 0.f;
        accA[bi][ii] *= f;
        accP[bi][ii] *= f;
      }
      emit_p(I, J, accP[bi]);
    }
    // (K e^{g_C - G})^T to the record
    emit_ke([&](int s, int ch) { return to_f(sK[s * LD + ch]) * (GATE == GATE_NONE ? 1.f : fast_exp2(sGf[s])); });
  }
  __syncthreads();  // phase A buffers are dead from here on

  // ---- B0: A (row r scaled by beta_r, strictly lower) to LDS; K e^G and V ----------
#pragma unroll
  for (int bi = 0; bi < BPW; ++bi) {
    int I, J;
    if (!wave_block<NSUB>(w, bi, I, J)) break;
    const int r = 16 * I + m;
    const float br = sBeta[r];
    floatx4 a;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) a[ii] = (16 * J + 4 * g + ii < r) ? br * accA[bi][ii] : 0.f;
    *reinterpret_cast<floatx4*>(sA + r * LDC + 16 * J + 4 * g) = a;
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rbase + 8 * i;
    store4f(sKt + r * LD + ch0, ktr[i]);
    store4f(sV + r * LD + ch0, vr[i]);
  }
  if (CK > C) {
    const float z[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r = C + rbase; r < CK; r += 8) {
      store4f(sKt + r * LD + ch0, z);
      store4f(sV + r * LD + ch0, z);
    }
  }
  // T diag(beta) above the diagonal blocks and in the k padding is zero
  for (int e = t; e < C * CK; e += 256) {
    const int r = e / CK, s = e % CK;
    if ((s >> 4) > (r >> 4)) sTb[r * LDK + s] = from_f<E>(0.f);
  }
  __syncthreads();

  // ---- B1: diagonal blocks T_II = (I + A_II)^{-1}: bf16 operands by the power
  //      product on MFMA (all 64 lanes), fp32 row by row (lane j = column j) ---------
  if constexpr (std::is_same<E, __bf16>::value) {
    if (w < NSUB) {
      const int o0 = 16 * w;
      const floatx4 tb = unit_lower_inverse16(sA + o0 * LDC + o0, LDC, lane);
      const float bn = sBeta[o0 + m];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 4 * g + ii;
        sTd[(w * 16 + r) * 20 + m] = tb[ii];
        sTb[(o0 + r) * LDK + o0 + m] = from_f<E>(tb[ii] * bn);
      }
    }
  } else if (w < NSUB && lane < 16) {
    const int j = lane, o0 = 16 * w;
    float col[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float val = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) val -= sA[(o0 + r) * LDC + o0 + s] * col[s];
      col[r] = val;
    }
    const float bj = sBeta[o0 + j];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sTd[(w * 16 + r) * 20 + j] = col[r];
      sTb[(o0 + r) * LDK + o0 + j] = from_f<E>(col[r] * bj);
    }
  }
  __syncthreads();

  // ---- B2: off-diagonal blocks of T, block column J per wave:
  //          T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, in fp32 MFMA ------------------------
  if (w < NSUB - 1) {
    const int J = w;
    floatx4 Tcol[NSUB];  // T_KJ in accumulator layout, K = J .. I-1 (compile-time indices only)
#pragma unroll
    for (int K = 0; K < NSUB; ++K) {
      Tcol[K] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (K == J)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) Tcol[K][ii] = sTd[(K * 16 + 4 * g + ii) * 20 + m];
    }
    const float bm = sBeta[16 * J + m];
#pragma unroll
    for (int I = 1; I < NSUB; ++I) {
      if (I <= J) continue;
      floatx4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < I; ++K) {
        if (K < J) continue;
        const floatx4 a = *reinterpret_cast<const floatx4*>(sA + (16 * I + m) * LDC + 16 * K + 4 * g);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) X = __builtin_amdgcn_mfma_f32_16x16x4f32(a[jj], Tcol[K][jj], X, 0, 0, 0);
      }
      const floatx4 tii = *reinterpret_cast<const floatx4*>(sTd + (I * 16 + m) * 20 + 4 * g);
      floatx4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tii[jj], X[jj], Y, 0, 0, 0);
      Tcol[I] = -Y;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sTb[(16 * I + 4 * g + ii) * LDK + 16 * J + m] = from_f<E>(-Y[ii] * bm);
    }
  }
  __syncthreads();

  // ---- B3: W (computed transposed, stored as -W in fragment order) and U, two
  //      16-column slabs per wave. T is block lower triangular, so row tile rt needs
  //      k-blocks kb <= rt / 2 only. A slab's products are all issued before its
  //      stores, so their MFMA latencies overlap. The wave's two slabs are the two
  //      halves of its -W slots, so each slot leaves as one 16-byte store after the
  //      second slab. ---------------------------------------------------------------------
  floatx4 aw[2][NRT];
#pragma unroll
  for (int cl = 0; cl < 2; ++cl) {
    const int ct = 2 * w + cl;
    FragT bK[NKC], bV[NKC];
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) {
      bK[kb] = frag_colk(sKt, LD, 16 * ct + m, 32 * kb, g);
      bV[kb] = frag_colk(sV, LD, 16 * ct + m, 32 * kb, g);
    }
    floatx4 au[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      aw[cl][rt] = au[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= (rt >> 1); ++kb) {
        const FragT aT = frag_rowk(sTb, LDK, 16 * rt + m, 32 * kb, g);
        mma(aw[cl][rt], bK[kb], aT);  // lane (m, g): W[16 rt + m][16 ct + 4 g + ii]
        mma(au[rt], aT, bV[kb]);      // lane (m, g): U[16 rt + 4 g + ii][16 ct + m]
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const float uo[4] = {au[rt][0], au[rt][1], au[rt][2], au[rt][3]};
      store4f(rec + RC::UU + ((size_t)(ct * NRT + rt) * 64 + lane) * 4, uo);
    }
  }
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
    store_frag<E>(rec + RC::WN + ((size_t)(rt * 4 + w) * 64 + lane) * 8, acc_pair_to_frag<E>(-aw[0][rt], -aw[1][rt]));
}

// Inter-chunk kernel for 16-token chunks (the body and its description are in
// kda_inter16.h).
template <typename E>
__global__ void __launch_bounds__(256) inter16_kernel(const char* __restrict__ records,
                                                      const int32_t* __restrict__ chunk_off,
                                                      const int2* __restrict__ info,
                                                      const float* __restrict__ initial_state,
                                                      float* __restrict__ final_state, E* __restrict__ o, int N, int H,
                                                      int mc) {
  inter16_body<E, true>(blockIdx.x, records, chunk_off, info, initial_state, final_state, o, N, H, mc, nullptr,
                        nullptr);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int64_t max_chunks(int B, int T, int num_seqs, bool varlen, int chunk) {
  const int64_t per = ((int64_t)T + chunk - 1) / chunk;
  return varlen ? per + num_seqs : (int64_t)B * per;
}

size_t chunk_record_bytes(int dtype, int chunk) {
  if (dtype == 0) return chunk == 16 ? Rec<__bf16, 16>::BYTES : Rec<__bf16, 64>::BYTES;
  return chunk == 16 ? Rec<float, 16>::BYTES : Rec<float, 64>::BYTES;
}

PrefillWs plan_ws_layout(int B, int T, int H, int num_seqs, bool varlen, int chunk, size_t record_bytes) {
  const int N = varlen ? num_seqs : B;
  const int64_t mc = max_chunks(B, T, num_seqs, varlen, chunk);
  PrefillWs l;
  l.off_chunk_off = 0;
  l.off_info = al256((size_t)(N + 1) * sizeof(int32_t));
  l.off_records = l.off_info + al256((size_t)mc * sizeof(int2));
  l.total = l.off_records + (size_t)mc * H * record_bytes;
  return l;
}

PrefillWs prefill_ws_layout(int B, int T, int H, int num_seqs, bool varlen, int chunk, int dtype) {
  return plan_ws_layout(B, T, H, num_seqs, varlen, chunk, chunk_record_bytes(dtype, chunk));
}

hipError_t launch_plan(const int32_t* cu_seqlens, int N, int T, int total_tokens, int chunk, int64_t mc,
                       int32_t* chunk_off, int2* info, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, N, T, total_tokens, chunk, (int)mc,
                     chunk_off, info);
  return hipGetLastError();
}

namespace {
using WsLayout = PrefillWs;
inline WsLayout ws_layout(int B, int T, int H, int num_seqs, bool varlen, int chunk, int dtype) {
  return prefill_ws_layout(B, T, H, num_seqs, varlen, chunk, dtype);
}

template <typename E, int C>
hipError_t launch_typed(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                        const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                        float* final_state, int T, int H, int64_t mc, const WsLayout& l, char* ws,
                        const Fusion& fusion, hipStream_t stream) {
  int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + l.off_chunk_off);
  int2* info = reinterpret_cast<int2*>(ws + l.off_info);
  char* records = ws + l.off_records;
  trace_begin(stream);
  const int total_tokens = cu_seqlens ? T : N * T;
  // A batch of equal sequences needs no plan kernel: the intra-chunk kernel writes the
  // chunk table itself (uni_T). Packed sequences, and calls with no chunks (whose state
  // kernels still read the table), run the plan first.
  const int uni_T = (!cu_seqlens && mc > 0) ? T : 0;
  hipError_t e = hipSuccess;
  if (uni_T == 0) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, N, T, total_tokens, C, (int)mc,
                       chunk_off, info);
    e = hipGetLastError();
    trace_mark(stream, 0);
    if (e != hipSuccess) return e;
  }
  if (mc > 0) {
    auto* kern = fusion.gate_kind == GATE_HEAD   ? intra_kernel<E, C, GATE_HEAD>
                 : fusion.gate_kind == GATE_NONE ? intra_kernel<E, C, GATE_NONE>
                                                 : intra_kernel<E, C, GATE_CHANNEL>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(mc * H)), dim3(256), 0, stream, (const E*)q, (const E*)k,
                       (const E*)v, log_alpha, beta, chunk_off, info, N, uni_T, H, (int)mc, records, fusion);
    e = hipGetLastError();
    trace_mark(stream, 1);
    if (e != hipSuccess) return e;
  }
  const int64_t units = (int64_t)N * H;
  const int64_t slots = (units + 7) / 8;
  if constexpr (std::is_same<E, __bf16>::value && C == 64) {
    if (slots > 0 && prefill_kernels(0, 64, fusion.prefill_path, mc, H) == KERNELS_RECORD_SEG) {
      // segment-parallel full-width state kernels on the records (output epilogue fused in)
      int B = cu_seqlens ? 1 : N;
      const SegWs sl =
          seg_ws_layout(B, T, H, cu_seqlens ? N : 0, cu_seqlens != nullptr, false, fusion.out_gate != nullptr);
      return launch_state_seg(records, chunk_off, mc, cu_seqlens, N, T, H, initial_state, final_state, o, fusion,
                              ws + al256(l.total), sl, stream);
    }
  }
  if (slots > 0) {
    if constexpr (std::is_same<E, __bf16>::value && C == 64) {
      hipLaunchKernelGGL(inter_wg_kernel<INTER_LOOKAHEAD>, dim3((unsigned)(slots * 64)), dim3(256), 0, stream,
                         records, chunk_off, cu_seqlens, T, total_tokens, initial_state, final_state, (__bf16*)o, N,
                         H, (int)mc);
    } else if constexpr (C == 16) {
      hipLaunchKernelGGL(inter16_kernel<E>, dim3((unsigned)(slots * 64)), dim3(256), 0, stream, records, chunk_off,
                         info, initial_state, final_state, (E*)o, N, H, (int)mc);
    } else {
      hipLaunchKernelGGL((inter_kernel<E, C>), dim3((unsigned)(slots * 64)), dim3(64), 0, stream, records,
                         chunk_off, info, initial_state, final_state, (E*)o, N, H, (int)mc);
    }
    e = hipGetLastError();
    trace_mark(stream, 2);
    if (e != hipSuccess) return e;
  }
  if (fusion.out_gate) {
    const int64_t rows = (int64_t)(cu_seqlens ? T : (int64_t)N * T) * H;
    e = launch_output_norm_gate(std::is_same<E, float>::value ? 1 : 0, o, fusion.out_gate, fusion.norm_weight, o,
                                rows, fusion.norm_eps, stream);
  }
  return e;
}
}  // namespace

size_t prefill_workspace_bytes(int B, int T, int H, int num_seqs, bool varlen, int chunk, int dtype, int path) {
  const int kern = prefill_kernels(dtype, chunk, path, max_chunks(B, T, num_seqs, varlen, chunk), H);
  // the plans with and without the output epilogue differ: room for either
  auto seg_bytes = [&](bool single) {
    return std::max(seg_ws_layout(B, T, H, num_seqs, varlen, single, false).total,
                    seg_ws_layout(B, T, H, num_seqs, varlen, single, true).total);
  };
  if (kern == KERNELS_SINGLE) return seg_bytes(true);
  const size_t rec = ws_layout(B, T, H, num_seqs, varlen, chunk, dtype).total;
  if (kern == KERNELS_RECORD_SEG) return al256(rec) + seg_bytes(false);
  return rec;
}

hipError_t launch_prefill(int dtype, int chunk, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta, const float* initial_state,
                          const int32_t* cu_seqlens, int num_seqs, void* o, float* final_state, int B,
                          int T, int H, const Fusion& fusion, void* workspace, hipStream_t stream) {
  const bool varlen = cu_seqlens != nullptr;
  const int kern = prefill_kernels(dtype, chunk, fusion.prefill_path, max_chunks(B, T, num_seqs, varlen, chunk), H);
  if (kern == KERNELS_SINGLE)
    return launch_prefill_seg(q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, o, final_state, B, T,
                              H, fusion, workspace, stream);
  const int N = varlen ? num_seqs : B;
  const WsLayout l = ws_layout(B, T, H, num_seqs, varlen, chunk, dtype);
  const int64_t mc = max_chunks(B, T, num_seqs, varlen, chunk);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == 0) {
    if (chunk == 16)
      return launch_typed<__bf16, 16>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, N, o, final_state, T, H,
                                      mc, l, ws, fusion, stream);
    return launch_typed<__bf16, 64>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, N, o, final_state, T, H,
                                    mc, l, ws, fusion, stream);
  }
  if (chunk == 16)
    return launch_typed<float, 16>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, N, o, final_state, T, H,
                                   mc, l, ws, fusion, stream);
  return launch_typed<float, 64>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, N, o, final_state, T, H, mc,
                                 l, ws, fusion, stream);
}

}  // namespace kda
