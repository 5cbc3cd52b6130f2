// Segment-parallel single-pass chunked prefill for bf16 q/k/v and 64-token chunks.
//
// Method (GeekNews "Kimi Linear" summary, section "청크 단위 병렬 알고리듬";
// "From GPT-2 to Kimi K3" digest, section "DeltaNet 병렬화 -- 청크 단위 학습"):
// per chunk (rows r, s; g_r = sum_{j<=r} log_alpha_j per channel; S_0 the state
// entering the chunk)
//   A    = tril_strict(beta (K e^G)(K e^-G)^T),  T = (I + A)^{-1}
//   W    = T diag(beta)(K e^G),  U = T diag(beta) V
//   U~   = U - W S_0,  P = tril((Q e^G)(K e^-G)^T)
//   O    = (Q e^G) S_0 + P U~,   S_C = Diag(e^{g_C}) S_0 + (K e^{g_C-G})^T U~
// Each chunk is an affine map of the state, S_C = M S_0 + B with
//   M = Diag(e^{g_C}) - (K e^{g_C-G})^T W ,   B = (K e^{g_C-G})^T U,
// and a run of chunks composes to one such map.
//
// Design. One work-group of eight waves owns a whole (sequence, head) segment of
// consecutive chunks and the full 128 x 128 fp32 state. For every chunk it forms
// the chunk's matrices in LDS from q, k, v, the gates and beta, then advances the
// state in registers, so nothing but the inputs, the outputs and a few states per
// segment goes through HBM. A sequence is cut into a first segment of `l0` chunks
// and further segments of `lseg` chunks so that enough work-groups run at once:
//   pass A  segment 0 of a sequence runs the output pass from the initial state
//           and writes the state at its end; every middle segment composes its
//           chunk maps into (M, B) (state columns from the identity and from zero);
//   scan    per (sequence, head, 16 state columns): S_in(j) = M_{j-1} S_in(j-1) + B_{j-1};
//   pass B  segments 1.. run the output pass from their entry state; the last one
//           writes the final state.
// The two passes each have about one work-group per (sequence, head, segment), so
// the segment length is chosen to give about as many work-groups as compute units.
// In pass A the first segments write outputs while the others only compose maps,
// which costs less per chunk, so the first segment is shorter (l0 = a fixed share of
// lseg, per kernel set) and both kinds of work-group finish together.
//
// In-chunk decay: everything in log2 units; rows are grouped in sub-chunks of 16
// with b_I the cumulative decay before sub-chunk I. Decays inside a sub-chunk are
// kept as local prefix sums loc_r = gh_r - b_I and sub-chunk totals R_I, so no
// exponent is formed as the difference of two long sums. For an A / P block
// (I, J <= I), r in I, s in J:
//   2^(gh_r - gh_s) = 2^(loc_r) * 2^(b_I - b_{J+1}) * 2^(R_J - loc_s)
// The outer factors have exponents <= 0 and belong to one row each; the middle one
// is a per-channel block scale, <= 1 off the diagonal and 2^(-R_I) on it. When
// -R_I exceeds 120 for some sub-chunk, its diagonal block is summed element-wise
// with 2^(loc_r - loc_s) (exponent <= 0 for every kept entry) instead, so no factor
// can overflow or underflow into the result for any input.
#include <type_traits>

#include "kda_device.h"
#include "kda_fusion_dev.h"
#include "kda_internal.h"
#include "kda_record.h"

namespace kda {

namespace {

constexpr int SC = 64;           // chunk length
constexpr int NSUBC = 4;         // 16-row sub-chunks per chunk
constexpr int NTHR = 512;        // threads per work-group (eight waves)
constexpr float L2E = 1.4426950408889634f;
constexpr float SUB_RANGE_LIMIT = 120.f;  // log2 units
// A chunk whose total decay stays within this range (log2 units) in every channel
// takes the direct form: x_r 2^(gh_r) >= x_r 2^-96 stays a normal number for any
// component above 2^-30, and k_s 2^(-gh_s) <= 2^96 is far from overflow
constexpr float DIRECT_RANGE_LIMIT = 96.f;
constexpr int G_CHANNEL = 0, G_HEAD = 1, G_NONE = 2;
constexpr int ST = D * D;        // floats in one 128 x 128 state

__host__ __device__ constexpr size_t smax(size_t a, size_t b) { return a > b ? a : b; }

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS plan (byte offsets). The scratch region is reused phase by phase; the chain
// operands live from the phase that writes them to the end of the chunk's state step.
struct SegSmem {
  static constexpr int LD = D + 8;     // bf16 [64][LD]
  static constexpr int GLD = D + 4;    // fp32 [64][GLD]
  static constexpr int LDC = SC + 4;   // fp32 [64][LDC]
  static constexpr int LDK = SC + 8;   // bf16 [64][LDK]
  // phase A, factored: local decay prefix (G), overwritten by the left operands
  static constexpr size_t G = 0;                                    // float[64][GLD]
  static constexpr size_t LK = 0;                                   // bf16[64][LD]  k_r 2^(loc_r)
  static constexpr size_t LQ = LK + al16((size_t)SC * LD * 2);      // bf16[64][LD]  q_r 2^(loc_r)
  static constexpr size_t RR = LQ + al16((size_t)SC * LD * 2);      // float[64][GLD] k_s 2^(R_J - loc_s)
  static constexpr size_t A_END = RR + al16((size_t)SC * GLD * 4);
  static_assert(G + (size_t)SC * GLD * 4 <= RR, "the right operands must not overlap the decay prefix");
  // phase A, exact: the prefix stays, raw k and q beside it
  static constexpr size_t XK = al16((size_t)SC * GLD * 4);          // bf16[64][LD]
  static constexpr size_t XQ = XK + al16((size_t)SC * LD * 2);      // bf16[64][LD]
  static constexpr size_t X_END = XQ + al16((size_t)SC * LD * 2);
  // phase B
  static constexpr size_t MA = 0;                                   // float[64][LDC] beta-scaled A
  static constexpr size_t TD = MA + al16((size_t)SC * LDC * 4);     // float[4][16][20] diagonal blocks of T
  static constexpr size_t TB = TD + al16((size_t)NSUBC * 16 * 20 * 4);  // bf16[64][LDK] T diag(beta)
  static constexpr size_t KT = TB + al16((size_t)SC * LDK * 2);     // bf16[64][LD] K e^G
  static constexpr size_t VV = KT + al16((size_t)SC * LD * 2);      // bf16[64][LD] V
  static constexpr size_t B_END = VV + al16((size_t)SC * LD * 2);
  static constexpr size_t SCR = smax(smax(A_END, X_END), B_END);
  // tables
  static constexpr int NBLK = NSUBC * (NSUBC + 1) / 2;             // A / P blocks (I, J <= I)
  static constexpr size_t BND = SCR;                                // float[5][128] b_I
  static constexpr size_t RS = BND + (size_t)(NSUBC + 1) * D * 4;   // float[4][128] R_I
  static constexpr size_t SCL = RS + (size_t)NSUBC * D * 4;         // float[NBLK + 4][128] block scales
  static constexpr size_t BETA = SCL + (size_t)(NBLK + NSUBC) * D * 4;  // float[64]
  static constexpr size_t GS = BETA + SC * 4;                       // float[64] scalar-gate cumsum
  static constexpr size_t FLAG = GS + SC * 4;                       // int[8]: sub-chunk range flags, direct-form flag
  // chain operands, in MFMA fragment order (kda_device.h)
  static constexpr size_t CW = al16(FLAG + 32);                     // bf16[4 rt][4 kb][64][8]  -W
  static constexpr size_t CQ = CW + 16384;                          // bf16[4 rt][4 kb][64][8]  Q e^G
  static constexpr size_t CK = CQ + 16384;                          // bf16[8 rt][2 kb][64][8]  (K e^{g_C-G})^T
  static constexpr size_t CP = CK + 16384;                          // bf16[4 rt][2 kb][64][8]  P
  static constexpr size_t CG = CP + 8192;                           // float[128] e^{g_C}
  static constexpr size_t ON = CG + D * 4;                          // float[4][64] output row sums
  static constexpr size_t NW = ON + 4 * SC * 4;                     // float[128] output norm weight
  static constexpr size_t TOTAL = NW + D * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one gfx950 CU");
};

// Which A / P block (I, J <= I) wave w forms in slot bi. The two blocks J = 2 kb and
// 2 kb + 1 of block row I fill one fragment slot of P, so they go to one wave.
__device__ __forceinline__ bool seg_block(int w, int bi, int& I, int& J) {
  if (w < 4) {  // (1,0)(1,1) | (2,0)(2,1) | (3,0)(3,1) | (3,2)(3,3)
    I = w < 3 ? w + 1 : 3;
    J = (w < 3 ? 0 : 2) + bi;
    return true;
  }
  I = J = (w == 4) ? 0 : 2;  // (0,0) | (2,2)
  return bi == 0 && w < 6;
}

// What a work-group does with its segment.
enum PassKind { PASS_OUT = 0, PASS_MAP = 1 };

struct SegArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const float* log_alpha;
  const float* beta;
  const float* initial_state;
  float* final_state;
  __bf16* o;
  const int32_t* cu_seqlens;
  int T;             // tokens per sequence (fixed-length batches)
  int total_tokens;  // tokens in the packed axis
  int N, H, lseg, l0;      // chunks per segment after the first, and in the first
  const int32_t* seg_off;  // [N + 1]
  const int2* seg_info;    // [segments] (sequence, index in sequence)
  float* seg_in;           // [segments][H][128 * 128] state entering the segment
  float* seg_map;          // [segments][H][2][128 * 128] (M, B) of the segment
  Fusion fu;
  // record-fed passes only: the per-(chunk, head) records (head-major) and the chunk plan
  const char* records;
  const int32_t* chunk_off;  // [N + 1]
  int mc;
};

// Raw inputs of one chunk as this thread loads them: rows rbase + 16 i (i = the row's
// sub-chunk), channels ch0 .. ch0 + 3; beta (and the scalar gate) of row t < 64.
struct InRegs {
  bf16x4 k[4], q[4], v[4];
  floatx4 la[4];
  float bt, lah;
};

// Loads of one part of a chunk's inputs into this thread's registers. Rows past the
// chunk's end read row 0 (zeroed where used).
// Per-chunk scalar base pointers (uniform over the work-group) and 32-bit lane offsets,
// so a load costs no 64-bit address arithmetic. Rows past the chunk's end read row 0
// (zeroed where used).
template <int GATE>
__device__ __forceinline__ void load_gate(const SegArgs& a, InRegs& x, int tok0, int len, int h, int t) {
  const int HD = a.H * D;
  const int rbase = t >> 5, ch0 = 4 * (t & 31);
  if constexpr (GATE == G_CHANNEL) {
    const float* base = a.log_alpha + (size_t)tok0 * HD + (size_t)h * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + 16 * i;
      x.la[i] = *reinterpret_cast<const floatx4*>(base + (unsigned)((r < len ? r : 0) * HD + ch0));
    }
  }
  if (t < SC) {
    const unsigned ro = (unsigned)((t < len ? t : 0) * a.H);
    x.bt = (a.beta + (size_t)tok0 * a.H + h)[ro];
    if constexpr (GATE == G_HEAD) x.lah = (a.log_alpha + (size_t)tok0 * a.H + h)[ro];
  }
}
template <int PASS>
__device__ __forceinline__ void load_kq(const SegArgs& a, InRegs& x, int tok0, int len, int h, int t) {
  const int HD = a.H * D;
  const int rbase = t >> 5, ch0 = 4 * (t & 31);
  const size_t base = (size_t)tok0 * HD + (size_t)h * D;
  const __bf16* kb = a.k + base;
  const __bf16* qb = a.q + base;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rbase + 16 * i;
    const unsigned off = (unsigned)((r < len ? r : 0) * HD + ch0);
    x.k[i] = *reinterpret_cast<const bf16x4*>(kb + off);
    if constexpr (PASS == PASS_OUT) x.q[i] = *reinterpret_cast<const bf16x4*>(qb + off);
  }
}
__device__ __forceinline__ void load_v(const SegArgs& a, InRegs& x, int tok0, int len, int h, int t) {
  const int HD = a.H * D;
  const int rbase = t >> 5, ch0 = 4 * (t & 31);
  const __bf16* vb = a.v + (size_t)tok0 * HD + (size_t)h * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rbase + 16 * i;
    x.v[i] = *reinterpret_cast<const bf16x4*>(vb + (unsigned)((r < len ? r : 0) * HD + ch0));
  }
}

// Where a state step finds the chunk's operands (LDS, MFMA fragment order; the same
// layout as the per-chunk record of kda_record.h) and its partner exchange buffers.
struct ChainOps {
  const bf16x8* cW;  // [4 rt][4 kb] -W
  const bf16x8* cQ;  // [4 rt][4 kb] Q e^G
  const bf16x8* cK;  // [8 rt][2 kb] (K e^{g_C-G})^T
  const bf16x8* cP;  // [4 rt][2 kb] P (slots above the diagonal unused)
  const float* cG;   // [128] e^{g_C}
  bf16x8* xS;        // [4 groups][2 halves][2 kb][2 ct] state halves as B fragments; a
                     // wave's U~ half goes over its partner's slot once read
  float* sON;        // [4 groups][64] output row sums (epilogue)
};

// One chunk of the output pass for wave half hr (see seg_pass): U~ = U - W S,
// O = (Q e^G) S + P U~, S <- Diag(e^{g_C}) S + (K e^{g_C-G})^T U~, with the output
// RMSNorm and gate when fu.out_gate is set. S holds the wave's key rows 64 hr ..
// 64 hr + 63 of columns col0 .. col0 + 31; au the U rows 32 hr .. of the same
// columns. Two work-group barriers (three with the epilogue).
// `mid` runs between the two barriers (the record-fed passes stage the next chunk's
// operands there).
// hr is a run-time (wave-uniform) value, not a template argument: both wave halves run
// one copy of the code, so loads issued in `mid` or for the next chunk's gate land in
// the same registers for every wave and stay in flight across the loop's back edge (two
// inlined copies would be merged by register copies that wait for every load).
// The output epilogue's gate values of one chunk (len >= 1 tokens from tok0) for wave
// half hr: rows 32 hr + 16 j + m, one 16-byte load of 8 consecutive columns per row
// (col0 + 4 g .. for even g, col0 + 4 g + 12 .. for odd g: the same columns the lane
// writes of o); rows past len read the chunk's first row. The epilogue trades halves
// between lanes g and g ^ 1 where it uses them. Only the passes instantiated for an
// output gate call it, and they call it on every path, so its loads are never merged
// with a path without them.
typedef bf16x8 GateRegs[2];
__device__ __forceinline__ void load_out_gate(GateRegs& zv, const Fusion& fu, size_t HD, int h, int tok0,
                                              int len, int w, int lane) {
  const int m = lane & 15, g = lane >> 4, col0 = 32 * (w & 3), hr = w >> 2;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 32 * hr + 16 * j + m, rr = row < len ? row : 0;
    zv[j] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(fu.out_gate) + (size_t)(tok0 + rr) * HD +
                                             (size_t)h * D + col0 + 4 * g + ((g & 1) ? 12 : 0));
  }
}

// OG: the output epilogue runs (fu.out_gate is set). zv holds this chunk's gate values
// on entry (see load_out_gate); with PF it holds the next chunk's (next_len tokens from
// tok0 + 64; this chunk's again if there is none) on return, so each load has a whole
// step to land. nw holds the norm weight of columns col0 + 16 c + 4 g .. + 3.
template <bool OG, bool PF, typename Mid>
__device__ __forceinline__ void out_state_step(floatx4 (&S)[4][2], const floatx4 (&au)[2][2], const ChainOps& op,
                                               const Fusion& fu, __bf16* __restrict__ o, size_t HD, int h, int tok0,
                                               int len, int next_len, GateRegs& zv, const floatx4 (&nw)[2],
                                               int w, int lane, Mid&& mid) {
  const int hr = w >> 2, ho = 1 - hr;
  const int m = lane & 15, g = lane >> 4;
  const int c4 = w & 3, col0 = 32 * c4;
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // the state's rows as operand fragments: own k-blocks 2 hr + j, the partner's 2 ho + j
  bf16x8 Sown[2][2], Spar[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      Sown[j][c] = acc_pair_to_frag<__bf16>(S[2 * j][c], S[2 * j + 1][c]);
      op.xS[((c4 * 2 + hr) * 4 + j * 2 + c) * 64 + lane] = Sown[j][c];
    }
  // U~ = U - W S and O^T = S^T (Q e^G)^T for chunk rows 32 hr .. 32 hr + 31 (row tiles
  // rt = 2 hr + j); the own key rows first, the partner's after the exchange
  floatx4 Ut[2][2], xt[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      Ut[j][c] = au[c][j];
      xt[j][c] = zero4;
    }
  auto state_products = [&](int kb, const bf16x8 (&sb)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rt = 2 * hr + j;
      const bf16x8 wf = op.cW[(rt * 4 + kb) * 64 + lane];
      const bf16x8 qf = op.cQ[(rt * 4 + kb) * 64 + lane];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        mma(Ut[j][c], wf, sb[c]);
        mma(xt[j][c], sb[c], qf);
      }
    }
  };
  state_products(2 * hr, Sown[0]);
  state_products(2 * hr + 1, Sown[1]);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int c = 0; c < 2; ++c) Spar[j][c] = op.xS[((c4 * 2 + ho) * 4 + j * 2 + c) * 64 + lane];
  mid();
  state_products(2 * ho, Spar[0]);
  state_products(2 * ho + 1, Spar[1]);
  // U~ rows 32 hr .. as the operand fragment of k-block hr, for both waves of the pair:
  // written over the partner's state slot, which only this wave reads and has read
  bf16x8 Uown[2], Upar[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    Uown[c] = acc_pair_to_frag<__bf16>(Ut[0][c], Ut[1][c]);
    op.xS[((c4 * 2 + ho) * 4 + c) * 64 + lane] = Uown[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 2; ++c) Upar[c] = op.xS[((c4 * 2 + hr) * 4 + c) * 64 + lane];
  // U~ by k-block: rows 0 .. 31 and 32 .. 63 of the chunk
  bf16x8 U0[2], U1[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    U0[c] = hr ? Upar[c] : Uown[c];
    U1[c] = hr ? Uown[c] : Upar[c];
  }
  // O^T += U~^T P^T, causal k-blocks only: k-block 0 for every row tile, k-block 1 for
  // the row tiles of the second half
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rt = 2 * hr + j;
    const bf16x8 pf0 = op.cP[(rt * 2 + 0) * 64 + lane];
#pragma unroll
    for (int c = 0; c < 2; ++c) mma(xt[j][c], U0[c], pf0);
    if (hr) {
      const bf16x8 pf1 = op.cP[(rt * 2 + 1) * 64 + lane];
#pragma unroll
      for (int c = 0; c < 2; ++c) mma(xt[j][c], U1[c], pf1);
    }
  }
  // S = Diag(e^{g_C}) S + (K e^{g_C-G})^T U~ for key rows 64 hr ..
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rt = 4 * hr + j;
    const floatx4 gv = *reinterpret_cast<const floatx4*>(op.cG + 16 * rt + 4 * g);
    const bf16x8 k0 = op.cK[(rt * 2 + 0) * 64 + lane], k1 = op.cK[(rt * 2 + 1) * 64 + lane];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      S[j][c] = gv * S[j][c];
      mma(S[j][c], k0, U0[c]);
      mma(S[j][c], k1, U1[c]);
    }
  }
  if constexpr (OG) {
    // RMSNorm over the row's 128 values (four column groups hold 32 each) times the gate
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += xt[j][c][i] * xt[j][c][i];
      ss = xor32_sum(xor16_sum(ss));  // over the lanes of equal m
      if (g == 0) op.sON[c4 * SC + 32 * hr + 16 * j + m] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 32 * hr + 16 * j + m;
      float tot = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) tot += op.sON[q4 * SC + row];
      const float inv = rsqrtf(tot * (1.f / D) + fu.norm_eps);
      // the lane loaded 8 consecutive columns (see load_out_gate): it keeps the half of
      // its own 16-column tile and trades the other with lane g ^ 1
      const bool godd = (g & 1) != 0;
      typedef unsigned u32x4g __attribute__((ext_vector_type(4)));
      const u32x4g zu = __builtin_bit_cast(u32x4g, zv[j]);
      const unsigned give0 = godd ? zu[0] : zu[2], give1 = godd ? zu[1] : zu[3];
      const auto r0 = __builtin_amdgcn_permlane16_swap(give0, give0, false, false);
      const auto r1 = __builtin_amdgcn_permlane16_swap(give1, give1, false, false);
      const unsigned got0 = godd ? r0[0] : r0[1], got1 = godd ? r1[0] : r1[1];
      typedef unsigned u32x2g __attribute__((ext_vector_type(2)));
      const u32x2g keep = godd ? u32x2g{zu[2], zu[3]} : u32x2g{zu[0], zu[1]}, got = {got0, got1};
      const bf16x4 zc[2] = {__builtin_bit_cast(bf16x4, godd ? got : keep), __builtin_bit_cast(bf16x4, godd ? keep : got)};
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) xt[j][c][i] = xt[j][c][i] * inv * nw[c][i] * sigmoid_f((float)zc[c][i]);
    }
    if constexpr (PF) {  // one load on every path: a select of the chunk, not a branch around it
      // the gate values are used up before the loads that overwrite them are issued (see
      // the record prefetch of the record-fed passes)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < 2; ++c) asm volatile("" : "+v"(xt[j][c])::"memory");
      const bool nx = next_len > 0;
      load_out_gate(zv, fu, HD, h, nx ? tok0 + SC : tok0, nx ? next_len : len, w, lane);
    }
  }
  // Each lane writes 8 consecutive columns of its row as one 16-byte store: lanes g and
  // g ^ 1 (16 lanes apart) trade the half they do not write, so even g writes columns
  // 4 g .. 4 g + 7 of the first 16-column tile and odd g columns 4 g + 12 .. 4 g + 19
  // (the second tile), and a row's 64 bytes leave in one instruction.
  const bool godd = (g & 1) != 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const floatx4 keep = godd ? xt[j][1] : xt[j][0], give = godd ? xt[j][0] : xt[j][1];
    bf16x4 kb4, gb4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kb4[i] = (__bf16)keep[i];
      gb4[i] = (__bf16)give[i];
    }
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 gu = __builtin_bit_cast(u32x2, gb4);
    const auto r0 = __builtin_amdgcn_permlane16_swap(gu[0], gu[0], false, false);
    const auto r1 = __builtin_amdgcn_permlane16_swap(gu[1], gu[1], false, false);
    const u32x2 ru = {godd ? r0[0] : r0[1], godd ? r1[0] : r1[1]};
    const bf16x4 rb4 = __builtin_bit_cast(bf16x4, ru);
    bf16x8 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ov[i] = godd ? rb4[i] : kb4[i];
      ov[4 + i] = godd ? kb4[i] : rb4[i];
    }
    const int row = 32 * hr + 16 * j + m;
    if (row < len)
      *reinterpret_cast<bf16x8*>(o + (size_t)(tok0 + row) * HD + (size_t)h * D + col0 + 4 * g + (godd ? 12 : 0)) = ov;
  }
}

// One chunk of the map pass (see seg_pass): wave w carries 32 columns of [M | B]
// over all key rows; waves 4-7 (the B columns) add their U rows au. No barrier.
__device__ __forceinline__ void map_state_step(floatx4 (&S)[8][2], const floatx4 (&au)[2][4], const ChainOps& op,
                                               int w, int lane) {
  const int g = lane >> 4;
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  bf16x8 Sb[4][2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int c = 0; c < 2; ++c) Sb[kb][c] = acc_pair_to_frag<__bf16>(S[2 * kb][c], S[2 * kb + 1][c]);
  floatx4 Ut[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      Ut[rt][c] = w >= 4 ? au[c][rt] : zero4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(Ut[rt][c], op.cW[(rt * 4 + kb) * 64 + lane], Sb[kb][c]);
    }
  bf16x8 Ub[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c = 0; c < 2; ++c) Ub[kb][c] = acc_pair_to_frag<__bf16>(Ut[2 * kb][c], Ut[2 * kb + 1][c]);
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    const floatx4 gv = *reinterpret_cast<const floatx4*>(op.cG + 16 * rt + 4 * g);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      S[rt][c] = gv * S[rt][c];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(S[rt][c], op.cK[(rt * 2 + kb) * 64 + lane], Ub[kb][c]);
    }
  }
}

// The output norm weight of this wave's columns col0 + 16 c + 4 g .. + 3, held for the
// whole pass (zero when there is no epilogue).
template <bool LOAD>
__device__ __forceinline__ void load_norm_weight(floatx4 (&nw)[2], const Fusion& fu, int w, int lane) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    nw[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (LOAD) nw[c] = *reinterpret_cast<const floatx4*>(fu.norm_weight + 32 * (w & 3) + 16 * c + 4 * (lane >> 4));
  }
}

// State initialisation and store of a pass: S[j][c] holds rows row0 + 16 j + 4 g + i of
// column col0 + 16 c + m (output pass: row0 = 64 (w >> 2), NRS = 4; map pass: row0 = 0,
// NRS = 8, the M columns (waves 0-3) start at the identity).
template <int NRS, bool OUTP>
__device__ __forceinline__ void init_state(floatx4 (&S)[NRS][2], const float* __restrict__ init, int w, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const int col0 = 32 * (w & 3), row0 = OUTP ? 64 * (w >> 2) : 0;
#pragma unroll
  for (int j = 0; j < NRS; ++j)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      S[j][c] = floatx4{0.f, 0.f, 0.f, 0.f};
      const int col = col0 + 16 * c + m;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + 16 * j + 4 * g + i;
        if constexpr (OUTP) {
          if (init) S[j][c][i] = init[row * D + col];
        } else {
          if (w < 4 && row == col) S[j][c][i] = 1.f;
        }
      }
    }
}
template <int NRS, bool OUTP>
__device__ __forceinline__ void store_state(const floatx4 (&S)[NRS][2], float* __restrict__ out, int w, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const int col0 = 32 * (w & 3), row0 = OUTP ? 64 * (w >> 2) : 0;
  float* dst = out;
  if constexpr (!OUTP) dst += (w >= 4) ? ST : 0;
#pragma unroll
  for (int j = 0; j < NRS; ++j)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(row0 + 16 * j + 4 * g + i) * D + col0 + 16 * c + m] = S[j][c][i];
}

// ---------------------------------------------------------------------------
// One pass over a segment: `nchunks` chunks from token `tok_begin` of a sequence
// ending at `tok_end`.
//   PASS_OUT: state from `init` (NULL: zeros); writes o; state at the end to `out`
//             (NULL: not written).
//   PASS_MAP: waves 0-3 carry the columns of M from the identity with U = 0, waves
//             4-7 the columns of B from zero; (M, B) to `out` ([2][128 * 128]).
// Output pass: waves c and c + 4 (c = w & 3) share state and output columns 32 c ..
// 32 c + 31; wave half r = w >> 2 keeps the state's key rows 64 r .. 64 r + 63 and forms
// the chunk's rows 32 r .. 32 r + 31 of U~ and O, so it reads only its halves of W,
// Q e^G and (K e^{g_C-G})^T. The partner's half of the state (as bf16 operand
// fragments) and the other 32 rows of U~ cross through LDS. Map pass: wave w owns
// 32 columns of [M | B] over all key rows.
// ---------------------------------------------------------------------------
template <int GATE, int PASS, bool OG>
__device__ void seg_pass(const SegArgs& a, char* smem, int h, int tok_begin, int tok_end, int nchunks,
                         const float* __restrict__ init, float* __restrict__ out) {
  using SM = SegSmem;
  constexpr int LD = SM::LD, GLD = SM::GLD, LDC = SM::LDC, LDK = SM::LDK, NBLK = SM::NBLK;
  constexpr bool OUTP = PASS == PASS_OUT;
  constexpr int NRS = OUTP ? 4 : 8;  // 16-row state tiles per wave (two 16-column tiles)
  const Fusion& fu = a.fu;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t HD = (size_t)a.H * D;

  float* sG = reinterpret_cast<float*>(smem + SM::G);
  __bf16* sLK = reinterpret_cast<__bf16*>(smem + SM::LK);
  __bf16* sLQ = reinterpret_cast<__bf16*>(smem + SM::LQ);
  float* sRR = reinterpret_cast<float*>(smem + SM::RR);
  __bf16* sXK = reinterpret_cast<__bf16*>(smem + SM::XK);
  __bf16* sXQ = reinterpret_cast<__bf16*>(smem + SM::XQ);
  float* sA = reinterpret_cast<float*>(smem + SM::MA);
  float* sTd = reinterpret_cast<float*>(smem + SM::TD);
  __bf16* sTb = reinterpret_cast<__bf16*>(smem + SM::TB);
  __bf16* sKt = reinterpret_cast<__bf16*>(smem + SM::KT);
  __bf16* sV = reinterpret_cast<__bf16*>(smem + SM::VV);
  float* sBnd = reinterpret_cast<float*>(smem + SM::BND);
  float* sR = reinterpret_cast<float*>(smem + SM::RS);
  float* sScl = reinterpret_cast<float*>(smem + SM::SCL);
  float* sBeta = reinterpret_cast<float*>(smem + SM::BETA);
  float* sGs = reinterpret_cast<float*>(smem + SM::GS);
  int* sFlag = reinterpret_cast<int*>(smem + SM::FLAG);
  bf16x8* cK = reinterpret_cast<bf16x8*>(smem + SM::CK);
  bf16x8* cP = reinterpret_cast<bf16x8*>(smem + SM::CP);
  float* cG = reinterpret_cast<float*>(smem + SM::CG);
  __bf16* cWe = reinterpret_cast<__bf16*>(smem + SM::CW);
  __bf16* cQe = reinterpret_cast<__bf16*>(smem + SM::CQ);

  floatx4 S[NRS][2];
  init_state<NRS, OUTP>(S, init, w, lane);
  // the output norm weight waits in LDS (registers are tight here); the first chunk's
  // barriers order its store before the epilogue reads it
  if (OG && OUTP && threadIdx.x < D / 4)
    reinterpret_cast<floatx4*>(smem + SM::NW)[threadIdx.x] = reinterpret_cast<const floatx4*>(fu.norm_weight)[threadIdx.x];
  const ChainOps ops{reinterpret_cast<const bf16x8*>(smem + SM::CW), reinterpret_cast<const bf16x8*>(smem + SM::CQ),
                     reinterpret_cast<const bf16x8*>(smem + SM::CK), reinterpret_cast<const bf16x8*>(smem + SM::CP),
                     reinterpret_cast<const float*>(smem + SM::CG), reinterpret_cast<bf16x8*>(smem + SM::G),
                     reinterpret_cast<float*>(smem + SM::ON)};

  // x holds the inputs of the chunk being processed; the decays and k, q are reloaded
  // with the next chunk's as soon as they have been consumed, so the loads overlap the
  // rest of the chunk without a second register copy; v is loaded at the start of its
  // own chunk
  InRegs x;
  if (nchunks > 0) {
    const int l0 = min(SC, tok_end - tok_begin);
    load_gate<GATE>(a, x, tok_begin, l0, h, threadIdx.x);
    load_kq<PASS>(a, x, tok_begin, l0, h, threadIdx.x);
  }

  for (int ci = 0; ci < nchunks; ++ci) {
    // Lane indices are re-derived from an opaque copy of the thread id in every
    // iteration: otherwise the compiler hoists hundreds of lane-dependent addresses
    // out of the loop and spills them.
    int t_opaque = threadIdx.x;
    asm volatile("" : "+v"(t_opaque));
    const int t = t_opaque;
    const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), m = lane & 15, g = lane >> 4;
    const int cq = t & 31, ch0 = 4 * cq, rbase = t >> 5;
    const int tok0 = tok_begin + SC * ci;
    const int len = min(SC, tok_end - tok0);
    const int tokn = tok_begin + SC * min(ci + 1, nchunks - 1);  // the next chunk (this one again at the end)
    const int lenn = min(SC, tok_end - tokn);
    // ---- S0: log2 decays, beta -------------------------------------------------------
    bool vrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vrow[i] = rbase + 16 * i < len;
    float la_row = 0.f;
    if (t < SC) {
      float bt = 0.f;
      if (t < len) {
        bt = x.bt;
        if (fu.beta_preactivation) bt = sigmoid_f(bt);
        if constexpr (GATE == G_HEAD) {
          la_row = x.lah;
          if (fu.gate_preactivation) la_row = -softplus_f(la_row);
        }
      }
      sBeta[t] = bt;
    }
    if (t <= NSUBC) sFlag[t] = 0;
    if constexpr (GATE == G_CHANNEL) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        floatx4 l2 = {0.f, 0.f, 0.f, 0.f};
        if (vrow[i]) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float la = fu.gate_preactivation ? -softplus_f(x.la[i][j]) : x.la[i][j];
            l2[j] = la * L2E;
          }
        }
        *reinterpret_cast<floatx4*>(sG + (rbase + 16 * i) * GLD + ch0) = l2;
      }
    } else if constexpr (GATE == G_HEAD) {
      if (t < SC) sGs[t] = la_row * L2E;  // zero past len
    }
    load_gate<GATE>(a, x, tokn, lenn, h, t);
    // v of this chunk: first used after the decay and A / P phases, so its load has
    // them to land, and it does not hold registers across the state step
    load_v(a, x, tok0, len, h, t);
    __syncthreads();
    // k and q of this thread's rows, L2-normalised (prologue) and zeroed past the
    // chunk's end; taken where the decay operands are formed, then reloaded with the
    // next chunk's
    float kr[4][4], qr[4][4];
    auto take_kq = [&]() {
      // k and q are used from here on, not from the top of the chunk: a wait for them
      // there would also wait for the previous chunk's output stores
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        asm volatile("" : "+v"(x.k[i]));
        if constexpr (OUTP) asm volatile("" : "+v"(x.q[i]));
      }
      float ik[4] = {1.f, 1.f, 1.f, 1.f}, iq[4] = {1.f, 1.f, 1.f, 1.f};
      if (fu.normalize_qk) {  // a row's 128 channels are the 32 lanes of one half-wave
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sk = 0.f, sq = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float kk = (float)x.k[i][j];
            sk += kk * kk;
            if constexpr (OUTP) {
              const float qq = (float)x.q[i][j];
              sq += qq * qq;
            }
          }
          ik[i] = rsqrtf(half_wave_sum(sk) + fu.qk_eps);
          if constexpr (OUTP) iq[i] = rsqrtf(half_wave_sum(sq) + fu.qk_eps);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kr[i][j] = vrow[i] ? (float)x.k[i][j] * ik[i] : 0.f;
          qr[i][j] = (OUTP && vrow[i]) ? (float)x.q[i][j] * iq[i] : 0.f;
        }
      load_kq<PASS>(a, x, tokn, lenn, h, t);
    };

    float ktr[4][4];  // K e^G of this thread's rows
    floatx4 accA[2], accP[2];
    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    floatx4 p_lo = zero4;
    // P to its fragment slots, causal entries only: block (I, J) is half of slot (I, J / 2)
    auto emit_p = [&](int I, int J, const floatx4& acc) {
      floatx4 pv;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) pv[ii] = (16 * J + 4 * g + ii <= 16 * I + m) ? acc[ii] : 0.f;
      bf16x8* dst = cP + (I * 2 + (J >> 1)) * 64 + lane;
      if (J & 1)
        *dst = acc_pair_to_frag<__bf16>(p_lo, pv);
      else if (J == I)
        *dst = acc_pair_to_frag<__bf16>(pv, zero4);
      else
        p_lo = pv;
    };
    // (K e^{g_C - G})^T to its fragment slots: item (channel, 4-row group fg, k-block kb)
    // is one lane's whole slot; kval(s, ch) is the value of chunk row s
    auto emit_ke = [&](auto kval) {
#pragma unroll
      for (int q = 0; q < D * 2 * 4 / NTHR; ++q) {
        const int it = t + q * NTHR;
        const int ch = it & (D - 1), fg = (it >> 7) & 3, kb = it >> 9;
        floatx4 lo, hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo[j] = kval(32 * kb + 4 * fg + j, ch);
          hi[j] = kval(32 * kb + 16 + 4 * fg + j, ch);
        }
        cK[((ch >> 4) * 2 + kb) * 64 + (ch & 15) + 16 * fg] = acc_pair_to_frag<__bf16>(lo, hi);
      }
    };
    // Q e^G: four consecutive channels of row r are half of one fragment slot
    auto q_slot = [&](int r) {
      const int kb = ch0 >> 5, co = ch0 & 31;
      return cQe + ((size_t)((r >> 4) * 4 + kb) * 64 + (r & 15) + 16 * ((co & 15) >> 2)) * 8 + 4 * (co >> 4);
    };

    if constexpr (GATE == G_CHANNEL) {
      {  // ---- P1b: local prefix over each sub-chunk's 16 rows, per channel; totals R_I
        const int chn = t & (D - 1), I = t >> 7;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = sG[(16 * I + r) * GLD + chn];
#pragma unroll
        for (int r = 1; r < 16; ++r) x[r] += x[r - 1];
#pragma unroll
        for (int r = 0; r < 16; ++r) sG[(16 * I + r) * GLD + chn] = x[r];
        sR[I * D + chn] = x[15];
      }
      __syncthreads();
      if (t < D) {  // ---- tables: b_I, block scales, e^{g_C}, range flags
        float R[NSUBC], b[NSUBC + 1];
#pragma unroll
        for (int I = 0; I < NSUBC; ++I) R[I] = sR[I * D + t];
        b[0] = 0.f;
#pragma unroll
        for (int I = 0; I < NSUBC; ++I) b[I + 1] = b[I] + R[I];
#pragma unroll
        for (int I = 0; I <= NSUBC; ++I) sBnd[I * D + t] = b[I];
        cG[t] = ex2(b[NSUBC]);
#pragma unroll
        for (int I = 0; I < NSUBC; ++I)
          if (!(-R[I] <= SUB_RANGE_LIMIT)) atomicOr(&sFlag[I], 1);
        if (!(-b[NSUBC] <= DIRECT_RANGE_LIMIT)) atomicOr(&sFlag[NSUBC], 1);
        // 2^(b_I - b_{J+1}): the sum of the whole sub-chunks strictly between J and I,
        // or 2^(-R_I) on the diagonal
#pragma unroll
        for (int I = 0; I < NSUBC; ++I)
#pragma unroll
          for (int J = 0; J <= I; ++J) {
            float e = 0.f;
            if (J == I) {
              e = -R[I];
            } else {
#pragma unroll
              for (int K = J + 1; K < I; ++K) e += R[K];
            }
            sScl[(I * (I + 1) / 2 + J) * D + t] = ex2(e);
          }
        // 2^(g_C - b_{J+1})
#pragma unroll
        for (int J = 0; J < NSUBC; ++J) {
          float e = 0.f;
#pragma unroll
          for (int K = J + 1; K < NSUBC; ++K) e += R[K];
          sScl[(NBLK + J) * D + t] = ex2(e);
        }
      }
      __syncthreads();
      bool exact = false;
#pragma unroll
      for (int I = 0; I < NSUBC; ++I) exact |= sFlag[I] != 0;
      const bool direct = sFlag[NSUBC] == 0;  // implies !exact: -R_I <= -b_4 <= the direct range

      take_kq();
      if (direct) {
        // ---- P2 (direct): the whole chunk's decay is within the direct range, so
        //      2^(gh_r - gh_s) = 2^(gh_r) 2^(-gh_s) splits with no scale table:
        //      lhs_r = x_r 2^(gh_r) (x = k, q; also K e^G and Q e^G), rhs_s = k_s 2^(-gh_s),
        //      gh = b_I + loc --------------------------------------------------------
        __bf16* sRK = reinterpret_cast<__bf16*>(smem + SM::RR);  // bf16[64][LD], inside RR
        bf16x4 lkv[4], lqv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + 16 * i;
          const floatx4 loc = *reinterpret_cast<const floatx4*>(sG + r * GLD + ch0);
          const floatx4 bI = *reinterpret_cast<const floatx4*>(sBnd + i * D + ch0);
          float qt[4];
          bf16x4 rk;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gh = bI[j] + loc[j];
            const float eg = ex2(gh);  // >= 2^-96
            qt[j] = qr[i][j] * eg;
            ktr[i][j] = kr[i][j] * eg;
            lkv[i][j] = (__bf16)ktr[i][j];
            lqv[i][j] = (__bf16)qt[j];
            rk[j] = (__bf16)(kr[i][j] * ex2(-gh));  // <= 2^96
          }
          *reinterpret_cast<bf16x4*>(sRK + r * LD + ch0) = rk;
          if constexpr (OUTP) store4f(q_slot(r), qt);
        }
        __syncthreads();  // every thread has its decays: the left operands overwrite the prefix
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + 16 * i;
          *reinterpret_cast<bf16x4*>(sLK + r * LD + ch0) = lkv[i];
          if constexpr (OUTP) *reinterpret_cast<bf16x4*>(sLQ + r * LD + ch0) = lqv[i];
        }
        __syncthreads();
        // ---- P3 (direct): the blocks straight from the bf16 operands; entries above
        //      the diagonal (up to 2^96) are dropped by selection where A and P are taken
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
          accA[bi] = accP[bi] = zero4;
          int I, J;
          if (!seg_block(w, bi, I, J)) break;
          const int rrow = 16 * I + m, srow = 16 * J + m;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            bf16x8 lk, lq, rhs;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int ch = 32 * kb + 16 * hh + 4 * g;
              const bf16x4 xa = *reinterpret_cast<const bf16x4*>(sLK + rrow * LD + ch);
              const bf16x4 xr = *reinterpret_cast<const bf16x4*>(sRK + srow * LD + ch);
              bf16x4 xq;
              if constexpr (OUTP) xq = *reinterpret_cast<const bf16x4*>(sLQ + rrow * LD + ch);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                lk[4 * hh + j] = xa[j];
                if constexpr (OUTP) lq[4 * hh + j] = xq[j];
                rhs[4 * hh + j] = xr[j];
              }
            }
            mma(accA[bi], rhs, lk);
            if constexpr (OUTP) mma(accP[bi], rhs, lq);
          }
          if constexpr (OUTP) emit_p(I, J, accP[bi]);
        }
        // (K e^{g_C - G})^T = rhs_s 2^(g_C)
        emit_ke([&](int s, int ch) { return (float)sRK[s * LD + ch] * cG[ch]; });
      } else if (!exact) {
        // ---- P2 (factored): Q e^G to its slots, K e^G kept, and per row
        //      lhs_r = x_r 2^(loc_r) (x = k, q) and rhs_s = k_s 2^(R_J - loc_s) --------
        bf16x4 lkv[4], lqv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + 16 * i;
          const floatx4 loc = *reinterpret_cast<const floatx4*>(sG + r * GLD + ch0);
          const floatx4 bI = *reinterpret_cast<const floatx4*>(sBnd + i * D + ch0);
          const floatx4 RI = *reinterpret_cast<const floatx4*>(sR + i * D + ch0);
          float qt[4];
          floatx4 rr;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float eg = ex2(bI[j] + loc[j]);  // exponent <= 0
            const float pl = ex2(loc[j]);          // exponent <= 0
            qt[j] = qr[i][j] * eg;
            ktr[i][j] = kr[i][j] * eg;
            lkv[i][j] = (__bf16)(kr[i][j] * pl);
            lqv[i][j] = (__bf16)(qr[i][j] * pl);
            rr[j] = kr[i][j] * ex2(RI[j] - loc[j]);  // exponent <= 0
          }
          *reinterpret_cast<floatx4*>(sRR + r * GLD + ch0) = rr;
          if constexpr (OUTP) store4f(q_slot(r), qt);
        }
        __syncthreads();  // every thread has its decays: the left operands overwrite the prefix
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + 16 * i;
          *reinterpret_cast<bf16x4*>(sLK + r * LD + ch0) = lkv[i];
          if constexpr (OUTP) *reinterpret_cast<bf16x4*>(sLQ + r * LD + ch0) = lqv[i];
        }
        __syncthreads();
        // ---- P3 (factored): blocks computed transposed: lane (m, g), element ii holds
        //      entry (r = 16 I + m, s = 16 J + 4 g + ii) -----------------------------
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
          accA[bi] = accP[bi] = zero4;
          int I, J;
          if (!seg_block(w, bi, I, J)) break;
          const int rrow = 16 * I + m, srow = 16 * J + m;
          const float* scl = sScl + (I * (I + 1) / 2 + J) * D;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            bf16x8 lk, lq, rhs;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int ch = 32 * kb + 16 * hh + 4 * g;
              const bf16x4 xa = *reinterpret_cast<const bf16x4*>(sLK + rrow * LD + ch);
              const floatx4 rv = *reinterpret_cast<const floatx4*>(sRR + srow * GLD + ch);
              const floatx4 sc = *reinterpret_cast<const floatx4*>(scl + ch);
              bf16x4 xq;
              if constexpr (OUTP) xq = *reinterpret_cast<const bf16x4*>(sLQ + rrow * LD + ch);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                lk[4 * hh + j] = xa[j];
                if constexpr (OUTP) lq[4 * hh + j] = xq[j];
                rhs[4 * hh + j] = (__bf16)(rv[j] * sc[j]);
              }
            }
            mma(accA[bi], rhs, lk);
            if constexpr (OUTP) mma(accP[bi], rhs, lq);
          }
          if constexpr (OUTP) emit_p(I, J, accP[bi]);
        }
        emit_ke([&](int s, int ch) { return sRR[s * GLD + ch] * sScl[(NBLK + (s >> 4)) * D + ch]; });
      } else {
        // ---- P2 (exact): raw k, q beside the prefix; Q e^G and K e^G as above ------
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + 16 * i;
          const floatx4 loc = *reinterpret_cast<const floatx4*>(sG + r * GLD + ch0);
          const floatx4 bI = *reinterpret_cast<const floatx4*>(sBnd + i * D + ch0);
          float qt[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float eg = ex2(bI[j] + loc[j]);
            qt[j] = qr[i][j] * eg;
            ktr[i][j] = kr[i][j] * eg;
          }
          store4f(sXK + r * LD + ch0, kr[i]);
          store4f(sXQ + r * LD + ch0, qr[i]);
          if constexpr (OUTP) store4f(q_slot(r), qt);
        }
        __syncthreads();
        // ---- P3 (exact): a flagged diagonal block element-wise with 2^(loc_r - loc_s);
        //      every other block from lhs_r = x_r 2^(loc_r) and
        //      rhs_s = k_s 2^(b_I - gh_s) = k_s 2^(R_J + ... + R_{I-1} - loc_s)
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
          accA[bi] = accP[bi] = zero4;
          int I, J;
          if (!seg_block(w, bi, I, J)) break;
          if (J == I && sFlag[I]) {
            const int r = 16 * I + m;
#pragma unroll 1
            for (int ii = 0; ii < 4; ++ii) {
              const int s = 16 * J + 4 * g + ii;
              float sa = 0.f, sp = 0.f;
              if (s <= r) {
#pragma unroll 1
                for (int ch = 0; ch < D; ++ch) {
                  const float ks = (float)sXK[s * LD + ch] * ex2(sG[r * GLD + ch] - sG[s * GLD + ch]);
                  sa += (float)sXK[r * LD + ch] * ks;
                  sp += (float)sXQ[r * LD + ch] * ks;
                }
              }
              accA[bi][ii] = sa;
              accP[bi][ii] = sp;
            }
          } else {
            const int rrow = 16 * I + m, srow = 16 * J + m;
#pragma unroll 1
            for (int kb = 0; kb < 4; ++kb) {
              bf16x8 lk, lq, rhs;
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                const int ch = 32 * kb + 16 * hh + 4 * g;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const float lr = sG[rrow * GLD + ch + j], ls = sG[srow * GLD + ch + j];
                  // b_I - gh_s = (b_I - b_J) - loc_s; on the diagonal (unflagged, so
                  // -R_I <= the limit) this is -loc_s <= 120
                  float e = -ls;
                  for (int K = J; K < I; ++K) e += sR[K * D + ch + j];
                  const float pl = ex2(lr);
                  lk[4 * hh + j] = (__bf16)((float)sXK[rrow * LD + ch + j] * pl);
                  lq[4 * hh + j] = (__bf16)((float)sXQ[rrow * LD + ch + j] * pl);
                  rhs[4 * hh + j] = (__bf16)((float)sXK[srow * LD + ch + j] * ex2(e));
                }
              }
              mma(accA[bi], rhs, lk);
              if constexpr (OUTP) mma(accP[bi], rhs, lq);
            }
          }
          if constexpr (OUTP) emit_p(I, J, accP[bi]);
        }
        // (K e^{g_C - G})^T = k_s 2^(b_4 - b_J - loc_s), exponent <= 0
        emit_ke([&](int s, int ch) {
          const int J = s >> 4;
          float e = -sG[s * GLD + ch];
          for (int K = J; K < NSUBC; ++K) e += sR[K * D + ch];
          return (float)sXK[s * LD + ch] * ex2(e);
        });
      }
    } else {
      // ---- scalar gate (one decay per row) or none: raw k k^T and q k^T by MFMA, then
      //      the pair decay 2^(gh_r - gh_s) per element, exponent <= 0 where kept ------
      if (w == 0) {
        float x = 0.f;
        if constexpr (GATE == G_HEAD) x = sGs[lane];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off, 64);
          if (lane >= off) x += y;
        }
        if constexpr (GATE == G_HEAD) sGs[lane] = x;
      }
      __syncthreads();
      const float gC = GATE == G_NONE ? 0.f : sGs[SC - 1];
      take_kq();
      if (t < D) cG[t] = GATE == G_NONE ? 1.f : ex2(gC);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rbase + 16 * i;
        const float eg = GATE == G_NONE ? 1.f : ex2(sGs[r]);
        float qt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qt[j] = qr[i][j] * eg;
          ktr[i][j] = kr[i][j] * eg;
        }
        store4f(sXK + r * LD + ch0, kr[i]);
        store4f(sXQ + r * LD + ch0, qr[i]);
        if constexpr (OUTP) store4f(q_slot(r), qt);
      }
      __syncthreads();
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        accA[bi] = accP[bi] = zero4;
        int I, J;
        if (!seg_block(w, bi, I, J)) break;
        const int rrow = 16 * I + m, srow = 16 * J + m;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          bf16x8 lk, lq, rhs;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int ch = 32 * kb + 16 * hh + 4 * g;
            const bf16x4 xa = *reinterpret_cast<const bf16x4*>(sXK + rrow * LD + ch);
            const bf16x4 xq = *reinterpret_cast<const bf16x4*>(sXQ + rrow * LD + ch);
            const bf16x4 xs = *reinterpret_cast<const bf16x4*>(sXK + srow * LD + ch);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              lk[4 * hh + j] = xa[j];
              lq[4 * hh + j] = xq[j];
              rhs[4 * hh + j] = xs[j];
            }
          }
          mma(accA[bi], rhs, lk);
          if constexpr (OUTP) mma(accP[bi], rhs, lq);
        }
        const int r = rrow;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int s = 16 * J + 4 * g + ii;
          const float f = s <= r ? (GATE == G_NONE ? 1.f : ex2(sGs[r] - sGs[s])) : 0.f;
          accA[bi][ii] *= f;
          accP[bi][ii] *= f;
        }
        if constexpr (OUTP) emit_p(I, J, accP[bi]);
      }
      emit_ke([&](int s, int ch) {
        return (float)sXK[s * LD + ch] * (GATE == G_NONE ? 1.f : ex2(gC - sGs[s]));
      });
    }
    __syncthreads();  // phase A buffers are dead from here on

    // ---- B0: beta-scaled strictly lower A; K e^G and V; zero T above its diagonal blocks
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      int I, J;
      if (!seg_block(w, bi, I, J)) break;
      const int r = 16 * I + m;
      const float br = sBeta[r];
      floatx4 av;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) av[ii] = (16 * J + 4 * g + ii < r) ? br * accA[bi][ii] : 0.f;
      *reinterpret_cast<floatx4*>(sA + r * LDC + 16 * J + 4 * g) = av;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + 16 * i;
      store4f(sKt + r * LD + ch0, ktr[i]);
      bf16x4 vv = x.v[i];
      if (!vrow[i]) vv = bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
      *reinterpret_cast<bf16x4*>(sV + r * LD + ch0) = vv;
    }
    {  // the products read T's blocks (0, 1) and (2, 3) above the diagonal: zero them
      const int blk = t >> 8, e = t & 255;
      sTb[(32 * blk + (e >> 4)) * LDK + 32 * blk + 16 + (e & 15)] = (__bf16)0.f;
    }
    __syncthreads();

    // ---- B1: diagonal blocks T_II = (I + A_II)^{-1} by the power product on fp32
    //      MFMA, one wave per block ---------------------------------------------------
    if (w < NSUBC) {
      const int o0 = 16 * w;
      const floatx4 tb = unit_lower_inverse16(sA + o0 * LDC + o0, LDC, lane);
      const float bn = sBeta[o0 + m];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 4 * g + ii;
        sTd[(w * 16 + r) * 20 + m] = tb[ii];
        sTb[(o0 + r) * LDK + o0 + m] = (__bf16)(tb[ii] * bn);
      }
    }
    __syncthreads();

    // ---- B2: off-diagonal blocks T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ (fp32 MFMA) --
    if (w < NSUBC - 1) {
      const int J = w;
      floatx4 Tcol[NSUBC];
#pragma unroll
      for (int K = 0; K < NSUBC; ++K) {
        Tcol[K] = zero4;
        if (K == J)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) Tcol[K][ii] = sTd[(K * 16 + 4 * g + ii) * 20 + m];
      }
      const float bm = sBeta[16 * J + m];
#pragma unroll
      for (int I = 1; I < NSUBC; ++I) {
        if (I <= J) continue;
        floatx4 X = zero4;
#pragma unroll
        for (int K = 0; K < I; ++K) {
          if (K < J) continue;
          const floatx4 av = *reinterpret_cast<const floatx4*>(sA + (16 * I + m) * LDC + 16 * K + 4 * g);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) X = __builtin_amdgcn_mfma_f32_16x16x4f32(av[jj], Tcol[K][jj], X, 0, 0, 0);
        }
        const floatx4 tii = *reinterpret_cast<const floatx4*>(sTd + (I * 16 + m) * 20 + 4 * g);
        floatx4 Y = zero4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tii[jj], X[jj], Y, 0, 0, 0);
        Tcol[I] = -Y;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sTb[(16 * I + 4 * g + ii) * LDK + 16 * J + m] = (__bf16)(-Y[ii] * bm);
      }
    }
    __syncthreads();

    // ---- B3: W (transposed, stored as -W fragments) and U. Output pass: wave (c, r)
    //      forms both for rows 32 r .. 32 r + 31 and columns 32 c .. 32 c + 31 and keeps
    //      its U. Map pass: waves 0-3 form W slabs 2 w, 2 w + 1 (all rows); waves 4-7
    //      the U slabs of their B columns. T is block lower triangular, so row tile rt
    //      needs k-blocks kb <= rt / 2 only. ----------------------------------------
    constexpr int NUR = OUTP ? 2 : 4;  // row tiles of U a wave keeps
    floatx4 au[2][NUR];
    {
      const int hr = w >> 2;
      const bool do_w = OUTP || w < 4, do_u = OUTP || w >= 4;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ct = 2 * (w & 3) + c;
        bf16x8 bK[2], bV[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (OUTP && kb > hr) continue;
          if (do_w) bK[kb] = frag_colk(sKt, LD, 16 * ct + m, 32 * kb, g);
          if (do_u) bV[kb] = frag_colk(sV, LD, 16 * ct + m, 32 * kb, g);
        }
#pragma unroll
        for (int j = 0; j < NUR; ++j) {
          const int rt = OUTP ? 2 * hr + j : j;
          floatx4 aw = zero4;
          au[c][j] = zero4;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (kb > (rt >> 1)) continue;
            const bf16x8 aT = frag_rowk(sTb, LDK, 16 * rt + m, 32 * kb, g);
            if (do_w) mma(aw, bK[kb], aT);       // lane (m, g): W[16 rt + m][16 ct + 4 g + ii]
            if (do_u) mma(au[c][j], aT, bV[kb]);  // lane (m, g): U[16 rt + 4 g + ii][16 ct + m]
          }
          if (do_w) {
            const float wn[4] = {-aw[0], -aw[1], -aw[2], -aw[3]};
            store4f(cWe + ((size_t)(rt * 4 + (ct >> 1)) * 64 + lane) * 8 + 4 * (ct & 1), wn);
          }
        }
      }
    }
    __syncthreads();

    // ---- the state step (the exchange buffers of the output pass reuse the scratch
    //      region, dead until the next chunk's decay phase) ----------------------------
    if constexpr (OUTP) {
      // the output gate values are loaded at the step (registers here are too tight to
      // hold the next chunk's across the chunk's matrix phases)
      GateRegs zv;
      floatx4 nw[2];
      if constexpr (OG) {
        load_out_gate(zv, fu, HD, h, tok0, len, w, lane);
#pragma unroll
        for (int c = 0; c < 2; ++c)
          nw[c] = *reinterpret_cast<const floatx4*>(smem + SM::NW + 4 * (32 * (w & 3) + 16 * c + 4 * g));
      }
      out_state_step<OG, false>(S, au, ops, fu, a.o, HD, h, tok0, len, 0, zv, nw, w, lane, [] {});
    } else {
      map_state_step(S, au, ops, w, lane);
    }
  }

  if (out) store_state<NRS, OUTP>(S, out, w, lane);
}

// ---------------------------------------------------------------------------
// The same passes fed by the per-chunk records of the intra-chunk kernel (kda_record.h)
// instead of forming each chunk's matrices in the work-group: the record's fragment
// region (-W, Q e^G, (K e^{g_C-G})^T, P; the map pass takes -W and (K e^{g_C-G})^T
// only) is copied into LDS as it is laid out, each wave takes its U tiles into
// registers, and the next chunk's record is loaded into registers while the current
// one is used. Records are read once per work-group, so a head's segment reads each of
// its records from HBM once.
// ---------------------------------------------------------------------------
struct RecSmem {
  static constexpr size_t STAGE = 57344 + D * 4;                      // -W, Q e^G, K, P, then e^{g_C}
  static constexpr size_t CW = 0, CQ = 16384, CK = 32768, CP = 49152, CG = 57344;  // within a stage
  static constexpr size_t XS = 2 * STAGE;                            // bf16x8[4][2][2][2][64]
  static constexpr size_t ON = XS + 32768;                           // float[4][64]
  static constexpr size_t TOTAL = ON + 4 * SC * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one gfx950 CU");
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int PASS>
struct RecRegs {
  static constexpr int NCOPY = PASS == PASS_OUT ? 7 : 4;  // 16-byte pieces of the fragment region per thread
  static constexpr int NU = PASS == PASS_OUT ? 2 : 4;     // row tiles of U per column tile
  u32x4 d[NCOPY];
  u32x4 gm;
  bf16x4 u[2][NU];
};

template <int PASS>
__device__ __forceinline__ void load_record(RecRegs<PASS>& x, const char* __restrict__ rb, int t) {
  using RC = Rec<__bf16, 64>;
  const u32x4* src = reinterpret_cast<const u32x4*>(rb);
  const int w = t >> 6, lane = t & 63;
#pragma unroll
  for (int q = 0; q < RecRegs<PASS>::NCOPY; ++q) {
    // output pass: pieces 0 .. 3583 (-W, Q e^G, K, P); map pass: -W (0 .. 1023) and
    // (K e^{g_C-G})^T (2048 .. 3071)
    const int piece = PASS == PASS_OUT ? t + NTHR * q : (q < 2 ? t + NTHR * q : 2048 + t + NTHR * (q - 2));
    x.d[q] = load_nt(src + piece);
  }
  if (t < 32) x.gm = load_nt(reinterpret_cast<const u32x4*>(rb + RC::GAMMA_BYTES) + t);
  const bf16x4* uu = reinterpret_cast<const bf16x4*>(rb + RC::UU * 2);
  const int c4 = w & 3, hr = w >> 2;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int j = 0; j < RecRegs<PASS>::NU; ++j) {
      const int ct = 2 * c4 + c, rt = PASS == PASS_OUT ? 2 * hr + j : j;
      if (PASS == PASS_OUT || w >= 4) x.u[c][j] = load_nt(uu + (ct * 4 + rt) * 64 + lane);
    }
}

template <int PASS, bool OG>
__device__ void rec_pass(const SegArgs& a, char* smem, int h, int c_first, int tok_begin, int tok_end, int nchunks,
                         const float* __restrict__ init, float* __restrict__ out) {
  using RS = RecSmem;
  using RC = Rec<__bf16, 64>;
  constexpr bool OUTP = PASS == PASS_OUT;
  constexpr int NRS = OUTP ? 4 : 8, NU = RecRegs<PASS>::NU;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t HD = (size_t)a.H * D;
  const char* head_rec = a.records + (size_t)h * a.mc * RC::BYTES;
  floatx4 S[NRS][2];
  init_state<NRS, OUTP>(S, init, w, lane);
  floatx4 nw[2];
  load_norm_weight<OG && OUTP>(nw, a.fu, w, lane);
  auto stage_ops = [&](int b) {
    char* st = smem + b * RS::STAGE;
    return ChainOps{reinterpret_cast<const bf16x8*>(st + RS::CW), reinterpret_cast<const bf16x8*>(st + RS::CQ),
                    reinterpret_cast<const bf16x8*>(st + RS::CK), reinterpret_cast<const bf16x8*>(st + RS::CP),
                    reinterpret_cast<const float*>(st + RS::CG), reinterpret_cast<bf16x8*>(smem + RS::XS),
                    reinterpret_cast<float*>(smem + RS::ON)};
  };
  // x holds the record of the chunk after the one being formed: it is copied into the
  // other LDS stage in the middle of the current chunk, and its U tiles are taken for
  // the next chunk, then x is loaded with the record two chunks ahead
  RecRegs<PASS> x;
  floatx4 au[2][NU];
  auto take = [&](int t, int b) {
    char* st = smem + b * RS::STAGE;
    u32x4* dst = reinterpret_cast<u32x4*>(st);
#pragma unroll
    for (int q = 0; q < RecRegs<PASS>::NCOPY; ++q) {
      const int piece = OUTP ? t + NTHR * q : (q < 2 ? t + NTHR * q : 2048 + t + NTHR * (q - 2));
      dst[piece] = x.d[q];
    }
    if (t < 32) reinterpret_cast<u32x4*>(st + RS::CG)[t] = x.gm;
  };
  auto take_u = [&](floatx4 (&u)[2][NU], int w_) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < NU; ++j) {
        u[c][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (OUTP || w_ >= 4)
#pragma unroll
          for (int i = 0; i < 4; ++i) u[c][j][i] = (float)x.u[c][j][i];
      }
  };
  GateRegs zv;  // output gate values of the chunk being stepped (epilogue)
  if (nchunks > 0) {
    if constexpr (OUTP && OG) {
      const int l0 = min(SC, tok_end - tok_begin);
      load_out_gate(zv, a.fu, HD, h, tok_begin, l0, w, lane);
    }
    load_record<PASS>(x, head_rec + (size_t)c_first * RC::BYTES, threadIdx.x);
    take(threadIdx.x, 0);
    take_u(au, w);
    load_record<PASS>(x, head_rec + (size_t)(c_first + min(1, nchunks - 1)) * RC::BYTES, threadIdx.x);
    __syncthreads();
  }
  for (int ci = 0; ci < nchunks; ++ci) {
    int t_opaque = threadIdx.x;
    asm volatile("" : "+v"(t_opaque));
    const int t = t_opaque;
    const int lane_ = t & 63, w_ = __builtin_amdgcn_readfirstlane(t >> 6);
    const int tok0 = tok_begin + SC * ci;
    const int len = min(SC, tok_end - tok0);
    const int b = ci & 1;
    const ChainOps ops = stage_ops(b);
    floatx4 au_next[2][NU];
    // stage the next chunk (the last one again at the end) and load the one after it
    auto mid = [&] {
      take(t, b ^ 1);
      take_u(au_next, w_);
      // the U tiles are converted before the loads that overwrite x are issued, so the
      // loads can land in x's own registers (a conversion moved past them would keep the
      // old x live, and the loop would then copy the loaded registers, waiting for them)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < NU; ++j) asm volatile("" : "+v"(au_next[c][j])::"memory");
      load_record<PASS>(x, head_rec + (size_t)(c_first + min(ci + 2, nchunks - 1)) * RC::BYTES, t);
    };
    if constexpr (OUTP) {
      const int next_len = ci + 1 < nchunks ? min(SC, tok_end - tok0 - SC) : 0;
      out_state_step<OG, true>(S, au, ops, a.fu, a.o, HD, h, tok0, len, next_len, zv, nw, w_, lane_, mid);
    } else {
      mid();
      map_state_step(S, au, ops, w_, lane_);
      __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < NU; ++j) au[c][j] = au_next[c][j];
  }
  if (out) store_state<NRS, OUTP>(S, out, w, lane);
}

// Token range of sequence n, clamped to the packed axis.
__device__ __forceinline__ void seq_range(const SegArgs& a, int n, int& s0, int& s1) {
  if (a.cu_seqlens) {
    s0 = min(max(a.cu_seqlens[n], 0), a.total_tokens);
    s1 = min(max(a.cu_seqlens[n + 1], 0), a.total_tokens);
    s1 = max(s1, s0);
  } else {
    s0 = n * a.T;
    s1 = s0 + a.T;
  }
}

// Pass A (SECOND = false) or pass B (SECOND = true): one work-group per (segment,
// head), heads varying fastest so that the work-groups in flight together read
// whole token rows.
template <int GATE, bool SECOND, bool OG>
__global__ void __launch_bounds__(NTHR) seg_pass_kernel(SegArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[SegSmem::TOTAL];
  const int s = blockIdx.x / a.H, h = blockIdx.x - s * a.H;
  if (s >= a.seg_off[a.N]) return;
  const int2 si = a.seg_info[s];
  const int n = si.x, j = si.y;
  const int ns = a.seg_off[n + 1] - a.seg_off[n];
  int s0, s1;
  seq_range(a, n, s0, s1);
  const int nc = (s1 - s0 + SC - 1) / SC;
  const int c0 = j == 0 ? 0 : a.l0 + (j - 1) * a.lseg;
  const int cnt = max(0, min(j == 0 ? a.l0 : a.lseg, nc - c0));
  const int tb = s0 + c0 * SC;
  const size_t uh = (size_t)n * a.H + h;
  const size_t sh = (size_t)s * a.H + h;
  if constexpr (!SECOND) {
    if (j == 0) {
      const float* init = a.initial_state ? a.initial_state + uh * ST : nullptr;
      float* out = ns == 1 ? (a.final_state ? a.final_state + uh * ST : nullptr) : a.seg_in + (sh + a.H) * ST;
      seg_pass<GATE, PASS_OUT, OG>(a, smem, h, tb, s1, cnt, init, out);
    } else if (j < ns - 1) {
      seg_pass<GATE, PASS_MAP, OG>(a, smem, h, tb, s1, cnt, nullptr, a.seg_map + sh * 2 * ST);
    }
  } else {
    if (j == 0) return;
    float* out = (j == ns - 1 && a.final_state) ? a.final_state + uh * ST : nullptr;
    seg_pass<GATE, PASS_OUT, OG>(a, smem, h, tb, s1, cnt, a.seg_in + sh * ST, out);
  }
}

// Record-fed pass A / pass B, one work-group per (segment, head) as seg_pass_kernel.
template <bool SECOND, bool OG>
__global__ void __launch_bounds__(NTHR) rec_seg_kernel(SegArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[RecSmem::TOTAL];
  const int s = blockIdx.x / a.H, h = blockIdx.x - s * a.H;
  if (s >= a.seg_off[a.N]) return;
  const int2 si = a.seg_info[s];
  const int n = si.x, j = si.y;
  const int ns = a.seg_off[n + 1] - a.seg_off[n];
  int s0, s1;
  seq_range(a, n, s0, s1);
  const int c_seq = a.chunk_off[n];
  const int nc = a.chunk_off[n + 1] - c_seq;
  const int c0 = j == 0 ? 0 : a.l0 + (j - 1) * a.lseg;
  const int cnt = max(0, min(j == 0 ? a.l0 : a.lseg, nc - c0));
  const int tb = s0 + c0 * SC;
  const size_t uh = (size_t)n * a.H + h;
  const size_t sh = (size_t)s * a.H + h;
  if constexpr (!SECOND) {
    if (j == 0) {
      const float* init = a.initial_state ? a.initial_state + uh * ST : nullptr;
      float* out = ns == 1 ? (a.final_state ? a.final_state + uh * ST : nullptr) : a.seg_in + (sh + a.H) * ST;
      rec_pass<PASS_OUT, OG>(a, smem, h, c_seq + c0, tb, s1, cnt, init, out);
    } else if (j < ns - 1) {
      rec_pass<PASS_MAP, OG>(a, smem, h, c_seq + c0, tb, s1, cnt, nullptr, a.seg_map + sh * 2 * ST);
    }
  } else {
    if (j == 0) return;
    float* out = (j == ns - 1 && a.final_state) ? a.final_state + uh * ST : nullptr;
    rec_pass<PASS_OUT, OG>(a, smem, h, c_seq + c0, tb, s1, cnt, a.seg_in + sh * ST, out);
  }
}

// Entry states of segments 2.. of each sequence: S_in(j) = M_{j-1} S_in(j-1) + B_{j-1},
// in fp32 (fp32 MFMA). One work-group of four waves per (sequence, head, 16 state
// columns); wave w forms rows 32 w .. 32 w + 31. Lane (m, q) holds M[row m][16 kb + 4 q ..
// + 3] as one 16-byte load, so MFMA step (kb, e) pairs k = 16 kb + 4 q + e on both
// operands; the next step's M and B rows are loaded while the current one is formed,
// and the state slab is double-buffered in LDS (one barrier per step).
__global__ void __launch_bounds__(256) seg_scan_kernel(const int32_t* __restrict__ seg_off, int N, int H,
                                                       float* __restrict__ seg_in,
                                                       const float* __restrict__ seg_map) {
  __shared__ float sl[2][D][17];
  const int u = blockIdx.x >> 3, slab = blockIdx.x & 7;
  if (u >= N * H) return;
  const int n = u / H, h = u - n * H;
  const int sb = seg_off[n], ns = seg_off[n + 1] - sb;
  if (ns < 3) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, m = lane & 15, q = lane >> 4;
  const int c0 = 16 * slab;
  {
    const float* src = seg_in + ((size_t)(sb + 1) * H + h) * ST;
    for (int e = t; e < D * 16; e += 256) sl[0][e >> 4][e & 15] = src[(e >> 4) * D + c0 + (e & 15)];
  }
  floatx4 mv[2][8], bv[2];
  auto load_map = [&](int j) {
    const float* Mp = seg_map + ((size_t)(sb + j - 1) * H + h) * 2 * ST;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int rt = 2 * w + r;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        mv[r][kb] = *reinterpret_cast<const floatx4*>(Mp + (size_t)(16 * rt + m) * D + 16 * kb + 4 * q);
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[r][i] = Mp[ST + (size_t)(16 * rt + 4 * q + i) * D + c0 + m];
    }
  };
  load_map(2);
  __syncthreads();
  for (int j = 2; j < ns; ++j) {
    const int cur = j & 1, nxt = cur ^ 1;  // sl[cur] holds S_in(j - 1); S_in(j) goes to sl[nxt]
    floatx4 acc[2] = {bv[0], bv[1]};
    floatx4 a[2][8];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) a[r][kb] = mv[r][kb];
    if (j + 1 < ns) load_map(j + 1);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float b = sl[cur][16 * kb + 4 * q + e][m];
#pragma unroll
        for (int r = 0; r < 2; ++r) acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r][kb][e], b, acc[r], 0, 0, 0);
      }
    float* dst = seg_in + ((size_t)(sb + j) * H + h) * ST;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * (2 * w + r) + 4 * q + i;
        sl[nxt][row][m] = acc[r][i];
        dst[(size_t)row * D + c0 + m] = acc[r][i];
      }
    __syncthreads();
  }
}

// Segment plan: per sequence its chunk count nc and segment count (one when nc <= l0,
// else 1 + ceil((nc - l0) / lseg)); seg_off = exclusive prefix of the segment counts (clamped to the table's
// capacity), seg_info[s] = (sequence, index within it). One work-group of 1024.
__global__ void __launch_bounds__(1024) seg_plan_kernel(const int32_t* __restrict__ cu_seqlens, int N, int T,
                                                        int total_tokens, int lseg, int l0, int capacity,
                                                        int32_t* __restrict__ seg_off, int2* __restrict__ seg_info) {
  __shared__ int s_scan[1024];
  __shared__ int s_carry;
  const int t = threadIdx.x;
  auto clampt = [&](int x) { return min(max(x, 0), total_tokens); };
  if (t == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int n = base + t;
    int cnt = 0;
    if (n < N) {
      int len = T;
      if (cu_seqlens) len = max(0, clampt(cu_seqlens[n + 1]) - clampt(cu_seqlens[n]));
      const int nc = (len + SC - 1) / SC;
      cnt = nc <= l0 ? 1 : 1 + (nc - l0 + lseg - 1) / lseg;
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
    if (n < N) seg_off[n] = min(carry + s_scan[t] - cnt, capacity);
    __syncthreads();
    if (t == 1023) s_carry = min(carry + s_scan[1023], capacity);
    __syncthreads();
  }
  const int total = s_carry;
  if (t == 0) seg_off[N] = total;
  __syncthreads();
  for (int s = t; s < total; s += 1024) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg_off[mid] <= s) lo = mid;
      else hi = mid - 1;
    }
    seg_info[s] = make_int2(lo, s - seg_off[lo]);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int seg_chunks_per_segment(int64_t mc, int N, int H, int first_pct) {
  // about SEG_TARGET_GROUPS work-groups per pass: the segments after the first number
  // (mc - N l0) / lseg per head, with l0 = first_pct % of lseg, so
  // lseg = mc H / (SEG_TARGET_GROUPS + N H first_pct / 100), rounded up
  const int64_t den = (int64_t)SEG_TARGET_GROUPS * 100 + (int64_t)N * H * first_pct;
  int64_t l = (mc * H * 100 + den - 1) / den;
  if (l < SEG_MIN_CHUNKS) l = SEG_MIN_CHUNKS;
  if (l > mc) l = mc > 0 ? mc : 1;
  return (int)l;
}

int seg_first_chunks(int lseg, int first_pct) {
  const int l0 = (lseg * first_pct + 99) / 100;
  return l0 < 1 ? 1 : l0;
}

SegWs seg_ws_layout_for(int lseg, int l0, int64_t msg, int N, int H) {
  SegWs l;
  l.lseg = lseg;
  l.l0 = l0;
  l.max_segments = msg;
  l.off_seg_off = 0;
  l.off_seg_info = al256((size_t)(N + 1) * sizeof(int32_t));
  l.off_seg_in = l.off_seg_info + al256((size_t)msg * sizeof(int2));
  l.off_seg_map = l.off_seg_in + al256((size_t)msg * H * ST * sizeof(float));
  l.total = l.off_seg_map + al256((size_t)msg * H * 2 * ST * sizeof(float));
  return l;
}

SegWs seg_ws_layout(int B, int T, int H, int num_seqs, bool varlen, bool single, bool gated) {
  const int N = varlen ? num_seqs : B;
  const int64_t mc = max_chunks(B, T, num_seqs, varlen, SC);
  const int pct = single ? (gated ? SEG_FIRST_PCT_SINGLE_GATED : SEG_FIRST_PCT_SINGLE)
                         : (gated ? SEG_FIRST_PCT_RECORD_GATED : SEG_FIRST_PCT_RECORD);
  const int lseg = seg_chunks_per_segment(mc, N, H, pct);
  const int l0 = seg_first_chunks(lseg, pct);
  // a sequence of nc chunks has 1 + ceil((nc - l0) / lseg) segments (one if nc <= l0):
  // exactly that for N sequences of T tokens; at most 2 + (nc - l0) / lseg each when
  // packed, so 2 N + ceil(mc / lseg) over all
  int64_t msg;
  if (!varlen) {
    const int64_t nc = ((int64_t)T + SC - 1) / SC;
    msg = (int64_t)N * (nc <= l0 ? 1 : 1 + (nc - l0 + lseg - 1) / lseg);
  } else {
    msg = 2 * (int64_t)N + (mc + lseg - 1) / lseg;
  }
  return seg_ws_layout_for(lseg, l0, msg, N, H);
}

namespace {
template <int GATE, bool OG>
hipError_t launch_seg_typed(const SegArgs& a, int64_t msg, bool any_multi, hipStream_t stream) {
  const unsigned grid = (unsigned)(msg * a.H);
  hipLaunchKernelGGL((seg_pass_kernel<GATE, false, OG>), dim3(grid), dim3(NTHR), 0, stream, a);
  hipError_t e = hipGetLastError();
  trace_mark(stream, 8);
  if (e != hipSuccess || !any_multi) return e;
  hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)((int64_t)a.N * a.H * 8)), dim3(256), 0, stream, a.seg_off,
                     a.N, a.H, a.seg_in, a.seg_map);
  e = hipGetLastError();
  trace_mark(stream, 9);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((seg_pass_kernel<GATE, true, OG>), dim3(grid), dim3(NTHR), 0, stream, a);
  e = hipGetLastError();
  trace_mark(stream, 10);
  return e;
}
}  // namespace

hipError_t launch_state_seg(const char* records, const int32_t* chunk_off, int64_t mc, const int32_t* cu_seqlens,
                            int N, int T, int H, const float* initial_state, float* final_state, void* o,
                            const Fusion& fusion, void* seg_workspace, const SegWs& l, hipStream_t stream) {
  const int lseg = l.lseg;
  const int64_t max_segments = l.max_segments;
  char* ws = reinterpret_cast<char*>(seg_workspace);
  SegArgs a{};
  a.initial_state = initial_state;
  a.final_state = final_state;
  a.o = reinterpret_cast<__bf16*>(o);
  a.cu_seqlens = cu_seqlens;
  a.T = T;
  a.total_tokens = cu_seqlens ? T : N * T;
  a.N = N;
  a.H = H;
  a.lseg = lseg;
  a.l0 = l.l0;
  a.seg_off = reinterpret_cast<int32_t*>(ws + l.off_seg_off);
  a.seg_info = reinterpret_cast<int2*>(ws + l.off_seg_info);
  a.seg_in = reinterpret_cast<float*>(ws + l.off_seg_in);
  a.seg_map = reinterpret_cast<float*>(ws + l.off_seg_map);
  a.fu = fusion;
  a.records = records;
  a.chunk_off = chunk_off;
  a.mc = (int)mc;
  hipLaunchKernelGGL(seg_plan_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, N, T, a.total_tokens, lseg, l.l0,
                     (int)max_segments, const_cast<int32_t*>(a.seg_off), const_cast<int2*>(a.seg_info));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(max_segments * H);
  const bool og = fusion.out_gate != nullptr;
  if (og) hipLaunchKernelGGL((rec_seg_kernel<false, true>), dim3(grid), dim3(NTHR), 0, stream, a);
  else hipLaunchKernelGGL((rec_seg_kernel<false, false>), dim3(grid), dim3(NTHR), 0, stream, a);
  e = hipGetLastError();
  trace_mark(stream, 8);
  if (e != hipSuccess || (int64_t)l.l0 >= mc) return e;
  hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)((int64_t)N * H * 8)), dim3(256), 0, stream, a.seg_off, N, H,
                     a.seg_in, a.seg_map);
  e = hipGetLastError();
  trace_mark(stream, 9);
  if (e != hipSuccess) return e;
  if (og) hipLaunchKernelGGL((rec_seg_kernel<true, true>), dim3(grid), dim3(NTHR), 0, stream, a);
  else hipLaunchKernelGGL((rec_seg_kernel<true, false>), dim3(grid), dim3(NTHR), 0, stream, a);
  e = hipGetLastError();
  trace_mark(stream, 10);
  return e;
}

hipError_t launch_prefill_seg(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                              int num_seqs, void* o, float* final_state, int B, int T, int H, const Fusion& fusion,
                              void* workspace, hipStream_t stream) {
  const bool varlen = cu_seqlens != nullptr;
  const int N = varlen ? num_seqs : B;
  const SegWs l = seg_ws_layout(B, T, H, num_seqs, varlen, true, fusion.out_gate != nullptr);
  const int64_t mc = max_chunks(B, T, num_seqs, varlen, SC);
  char* ws = reinterpret_cast<char*>(workspace);
  SegArgs a;
  a.q = reinterpret_cast<const __bf16*>(q);
  a.k = reinterpret_cast<const __bf16*>(k);
  a.v = reinterpret_cast<const __bf16*>(v);
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.initial_state = initial_state;
  a.final_state = final_state;
  a.o = reinterpret_cast<__bf16*>(o);
  a.cu_seqlens = cu_seqlens;
  a.T = T;
  a.total_tokens = varlen ? T : N * T;
  a.N = N;
  a.H = H;
  a.lseg = l.lseg;
  a.l0 = l.l0;
  a.seg_off = reinterpret_cast<int32_t*>(ws + l.off_seg_off);
  a.seg_info = reinterpret_cast<int2*>(ws + l.off_seg_info);
  a.seg_in = reinterpret_cast<float*>(ws + l.off_seg_in);
  a.seg_map = reinterpret_cast<float*>(ws + l.off_seg_map);
  a.fu = fusion;
  trace_begin(stream);
  hipLaunchKernelGGL(seg_plan_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, N, T, a.total_tokens, l.lseg, l.l0,
                     (int)l.max_segments, const_cast<int32_t*>(a.seg_off), const_cast<int2*>(a.seg_info));
  hipError_t e = hipGetLastError();
  trace_mark(stream, 0);
  if (e != hipSuccess) return e;
  // some sequence can have more than one segment unless one segment holds every chunk
  const bool any_multi = (int64_t)l.l0 < mc;
  const bool og = fusion.out_gate != nullptr;
  if (fusion.gate_kind == G_HEAD)
    return og ? launch_seg_typed<G_HEAD, true>(a, l.max_segments, any_multi, stream)
              : launch_seg_typed<G_HEAD, false>(a, l.max_segments, any_multi, stream);
  if (fusion.gate_kind == G_NONE)
    return og ? launch_seg_typed<G_NONE, true>(a, l.max_segments, any_multi, stream)
              : launch_seg_typed<G_NONE, false>(a, l.max_segments, any_multi, stream);
  return og ? launch_seg_typed<G_CHANNEL, true>(a, l.max_segments, any_multi, stream)
            : launch_seg_typed<G_CHANNEL, false>(a, l.max_segments, any_multi, stream);
}

}  // namespace kda
