// The inter-chunk kernels of 64-token chunks: one work-group per (sequence, head,
// 16 value columns), serial over the sequence's chunks with the 128 x 16 slab of
// the fp32 state in accumulator registers. Shared by the KDA prefill and the
// general diagonal-plus-low-rank (DPLR) forward, which differ only in a few extra
// record terms (the DP template flag).
#pragma once

#include <type_traits>

#include "kda_device.h"
#include "kda_record.h"

namespace kda {

// ---------------------------------------------------------------------------
// Inter-chunk kernel: one wave per (sequence, head, 16-column slab), serial over
// the sequence's chunks. Work-group ids are laid out so that the eight slabs of
// one (sequence, head) land on the same XCD (ids are dealt to the 8 XCDs round
// robin), where they share that XCD's L2 copy of the chunk records.
// With DP set it runs the general diagonal-plus-low-rank recurrence from RecD
// records: W = U + W_b S takes the place of U~, O gains M_qk V and the state
// update gains (K e^{g_C-G})^T V.
// ---------------------------------------------------------------------------
template <typename E, int C, bool DP = false>
__global__ void __launch_bounds__(64) inter_kernel(const char* __restrict__ records,
                                                   const int32_t* __restrict__ chunk_off,
                                                   const int2* __restrict__ info,
                                                   const float* __restrict__ initial_state,
                                                   float* __restrict__ final_state, E* __restrict__ o, int N,
                                                   int H, int mc) {
  using RC = typename std::conditional<DP, RecD<E, C>, Rec<E, C>>::type;
  typedef typename Frag<E>::T FragT;
  constexpr int NRT = RC::NRT, NKC = RC::NKC;

  const int b = blockIdx.x;
  const int xcd = b & 7, rest = b >> 3;
  const int ct = rest & 7, slot = rest >> 3;
  const int u = slot * 8 + xcd;
  if (u >= N * H) return;
  const int n = u / H, h = u - n * H;
  const int lane = threadIdx.x, m = lane & 15, g = lane >> 4;
  const size_t HD = (size_t)H * D;
  const size_t sbase = (size_t)u * D * D + 16 * ct + m;

  floatx4 S[8];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) S[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (initial_state) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[rt][i] = initial_state[sbase + (size_t)(16 * rt + 4 * g + i) * D];
  }

  const int c_begin = chunk_off[n], c_end = chunk_off[n + 1];
  for (int c = c_begin; c < c_end; ++c) {
    const char* rb = records + ((size_t)h * mc + c) * RC::BYTES;
    const E* rec = reinterpret_cast<const E*>(rb);
    const float* gam = reinterpret_cast<const float*>(rb + RC::GAMMA_BYTES);
    const int2 inf = info[c];

    FragT Sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Sb[kb] = acc_pair_to_frag<E>(S[2 * kb], S[2 * kb + 1]);

    // U~ = U - W S  (the record holds -W; for DP, W = U + W_b S with W_b held)
    floatx4 Ut[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      float u4[4];
      load4f(rec + RC::UU + ((size_t)(ct * NRT + rt) * 64 + lane) * 4, u4);
      Ut[rt] = floatx4{u4[0], u4[1], u4[2], u4[3]};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        mma(Ut[rt], load_frag<E>(rec + RC::WN + ((size_t)(rt * 4 + kb) * 64 + lane) * 8), Sb[kb]);
    }
    // (Q e^G) S
    floatx4 X[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      X[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        mma(X[rt], load_frag<E>(rec + RC::QT + ((size_t)(rt * 4 + kb) * 64 + lane) * 8), Sb[kb]);
    }
    FragT Ub[NKC];
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb)
      Ub[kb] = acc_pair_to_frag<E>(Ut[2 * kb], (2 * kb + 1 < NRT) ? Ut[2 * kb + 1] : floatx4{0.f, 0.f, 0.f, 0.f});
    // O = (Q e^G) S + P U~, causal: row tile rt needs k-blocks <= rt / 2
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
      for (int kb = 0; kb <= (rt >> 1); ++kb)
        mma(X[rt], load_frag<E>(rec + RC::PP + ((size_t)(rt * NKC + kb) * 64 + lane) * 8), Ub[kb]);
      if constexpr (DP) {
#pragma unroll
        for (int i = 0; i < 4; ++i)  // row 16 rt + 4 g + i, column 16 ct + m of the transposed tile
          X[rt][i] += to_f(rec[RC::OI + ((size_t)(ct * NRT + rt) * 64 + 4 * g + i + 16 * (m >> 2)) * 4 + (m & 3)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * rt + 4 * g + i;
        if (row < inf.y) o[(size_t)(inf.x + row) * HD + (size_t)h * D + 16 * ct + m] = from_f<E>(X[rt][i]);
      }
    }
    // S = Diag(e^{g_C}) S + (K e^{g_C - G})^T U~   (DP: + (K e^{g_C-G})^T V)
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      const floatx4 gv = *reinterpret_cast<const floatx4*>(gam + 16 * rt + 4 * g);
      S[rt] = gv * S[rt];
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) {
        mma(S[rt], load_frag<E>(rec + RC::KE + ((size_t)(rt * NKC + kb) * 64 + lane) * 8), Ub[kb]);
        if constexpr (DP)
          mma(S[rt], load_frag<E>(rec + RC::KV + ((size_t)(rt * NKC + kb) * 64 + lane) * 8),
              load_frag<E>(rec + RC::VB + ((size_t)(ct * NKC + kb) * 64 + lane) * 8));
      }
    }
  }
  if (final_state) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) final_state[sbase + (size_t)(16 * rt + 4 * g + i) * D] = S[rt][i];
  }
}

// ---------------------------------------------------------------------------
// Inter-chunk kernel, bf16 records of 64-token chunks, four waves per (sequence,
// head, 16-column slab). The work of one chunk is split over the four SIMDs of a
// CU, wave w taking
//   U~ rows 16w..16w+15          U~_w = U_w - W_w S         (4 MFMAs)
//   O  rows 16w..16w+15          O_w  = (Q e^G)_w S + P_w U~ (5-6 MFMAs)
//   state rows 32w..32w+31       S_w <- e^{g_C} S_w + (K e^{g_C-G})^T_w U~ (4 MFMAs)
// so that every record fragment is read by exactly one wave, straight from global
// memory into registers. The waves exchange two small bf16 operands per chunk
// through LDS: each wave's 32 state rows as one 1 KiB B fragment (all waves need
// the whole S for U~ and O), and each wave's 16 rows of U~ (all waves need the
// whole U~ for the state update and O). Loads run LA chunks ahead of the compute,
// in registers. O is formed transposed (operands of the MFMA swapped), which puts
// four consecutive output columns of one row in each lane: one 8-byte store per
// lane, no staging.
// With DP set it runs the general diagonal-plus-low-rank recurrence from RecD
// records (W = U + W_b S in place of U~, O += M_qk V, S_w += (K e^{g_C-G})^T_w V).
// ---------------------------------------------------------------------------
namespace {
// chunks of record data in flight ahead of the one being computed
constexpr int INTER_LOOKAHEAD = 1;
// chunks beyond the lookahead whose record lines are pulled into L2 ahead of use
constexpr int INTER_TOUCH_AHEAD = 4;

// gw: e^{g_C} of state row 32 w + row_word_index(m, g) (spread to the lane's eight
// rows by DPP moves where it is used)
template <bool DP> struct InterStage {
  bf16x8 wn[4], qt[4], ke[4], pp[2];
  bf16x4 uu;
  float gw;
};
template <> struct InterStage<true> {
  bf16x8 wn[4], qt[4], ke[4], pp[2], kv[4], vb[2];
  bf16x4 uu, oi;
  float gw;
};

}  // namespace

template <int LA, bool DP = false>
__global__ void __launch_bounds__(256) inter_wg_kernel(const char* __restrict__ records,
                                                       const int32_t* __restrict__ chunk_off,
                                                       const int32_t* __restrict__ cu_seqlens, int T,
                                                       int total_tokens, const float* __restrict__ initial_state,
                                                       float* __restrict__ final_state, __bf16* __restrict__ o,
                                                       int N, int H, int mc) {
  using RC = typename std::conditional<DP, RecD<__bf16, 64>, Rec<__bf16, 64>>::type;
  static_assert(RC::NRT == 4 && RC::NKC == 2, "layout below assumes 64-token chunks");
  __shared__ __attribute__((aligned(16))) bf16x8 xS[4 * 64];  // state B fragments, k-block kb = 32 rows
  __shared__ __attribute__((aligned(16))) bf16x8 xU[2 * 64];  // U~ B fragments, k-block kb = 32 chunk rows

  const int b = blockIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int xcd = b & 7, rest = b >> 3;
  const int ct = rest & 7, slot = rest >> 3;
  const int u = slot * 8 + xcd;
  if (u >= N * H) return;  // uniform over the work-group
  const int n = u / H, h = u - n * H;
  const size_t HD = (size_t)H * D;

  int s_start, s_end;
  if (cu_seqlens) {
    s_start = min(max(cu_seqlens[n], 0), total_tokens);
    s_end = min(max(cu_seqlens[n + 1], 0), total_tokens);
  } else {
    s_start = n * T;
    s_end = s_start + T;
  }

  // state rows 32w + 16j + 4g + i, column 16ct + m
  const size_t sidx = (size_t)u * D * D + (size_t)(32 * w + 4 * g) * D + 16 * ct + m;
  floatx4 Sw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    Sw[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (initial_state) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Sw[j][i] = initial_state[sidx + (size_t)(16 * j + i) * D];
    }
  }

  const int c_begin = chunk_off[n], c_end = chunk_off[n + 1];
  const char* head_records = records + (size_t)h * mc * RC::BYTES;
  const int lo16 = lane * 16;
  auto load = [&](InterStage<DP>& st, int c) {
    const char* rb = head_records + (size_t)c * RC::BYTES;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      st.wn[kb] = *reinterpret_cast<const bf16x8*>(rb + (RC::WN * 2) + (4 * w + kb) * 1024 + lo16);
      st.qt[kb] = *reinterpret_cast<const bf16x8*>(rb + (RC::QT * 2) + (4 * w + kb) * 1024 + lo16);
      st.ke[kb] = *reinterpret_cast<const bf16x8*>(rb + (RC::KE * 2) + (4 * w + kb) * 1024 + lo16);
    }
    // P is causal: rows 0..31 (waves 0 and 1) have no second k-block, and those slots
    // are neither written nor read (w is uniform over the wave)
    st.pp[0] = *reinterpret_cast<const bf16x8*>(rb + (RC::PP * 2) + (2 * w) * 1024 + lo16);
    if (w >= 2) st.pp[1] = *reinterpret_cast<const bf16x8*>(rb + (RC::PP * 2) + (2 * w + 1) * 1024 + lo16);
    st.uu = *reinterpret_cast<const bf16x4*>(rb + (RC::UU * 2) + ((ct * 4 + w) * 64 + lane) * 8);
    if constexpr (DP) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        st.kv[kb] = *reinterpret_cast<const bf16x8*>(rb + (RC::KV * 2) + (4 * w + kb) * 1024 + lo16);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        st.vb[kb] = *reinterpret_cast<const bf16x8*>(rb + (RC::VB * 2) + (2 * ct + kb) * 1024 + lo16);
      st.oi = *reinterpret_cast<const bf16x4*>(rb + (RC::OI * 2) + ((ct * 4 + w) * 64 + lane) * 8);
    }
    st.gw = reinterpret_cast<const float*>(rb + RC::GAMMA_BYTES)[32 * w + row_word_index(m, g)];
  };

  auto compute = [&](const InterStage<DP>& st, int c) {
    // this wave's 32 state rows as a B fragment, for every wave
    xS[w * 64 + lane] = acc_pair_to_frag<__bf16>(Sw[0], Sw[1]);
    lds_barrier();
    bf16x8 Sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Sb[kb] = xS[kb * 64 + lane];
    // U~_w = U_w - W_w S  (the record holds -W; for DP, W_w = U_w + W_b,w S)
    floatx4 ut = floatx4{(float)st.uu[0], (float)st.uu[1], (float)st.uu[2], (float)st.uu[3]};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mma(ut, st.wn[kb], Sb[kb]);
    {
      bf16x4 uh;
#pragma unroll
      for (int i = 0; i < 4; ++i) uh[i] = (__bf16)ut[i];
      // rows 16w + 4g + i are slots 4 (w & 1) + i of k-block w >> 1
      *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(xU) + ((w >> 1) * 64 + lane) * 16 + (w & 1) * 8) = uh;
    }
    // e^{g_C} S_w, ahead of the barrier
    floatx4 gm[2];
    rows_from_word(st.gw, m, gm);
#pragma unroll
    for (int j = 0; j < 2; ++j) Sw[j] = gm[j] * Sw[j];
    lds_barrier();
    bf16x8 Ub[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Ub[kb] = xU[kb * 64 + lane];
    // O_w^T = S^T (Q e^G)_w^T : lane (m, g) holds row 16w + m, columns 4g..4g+3
    floatx4 xt = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mma(xt, Sb[kb], st.qt[kb]);
    // S_w += (K e^{g_C-G})^T_w U~
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        mma(Sw[j], st.ke[2 * j + kb], Ub[kb]);
        if constexpr (DP) mma(Sw[j], st.kv[2 * j + kb], st.vb[kb]);
      }
    // O_w^T += U~^T P_w^T, causal k-blocks only
    mma(xt, Ub[0], st.pp[0]);
    if (w >= 2) mma(xt, Ub[1], st.pp[1]);
    if constexpr (DP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) xt[i] += (float)st.oi[i];
    }
    const int tok0 = s_start + (c - c_begin) * 64;
    const int row = 16 * w + m;
    if (row < s_end - tok0) {
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = (__bf16)xt[i];
      *reinterpret_cast<bf16x4*>(o + (size_t)(tok0 + row) * HD + (size_t)h * D + 16 * ct + 4 * g) = ov;
    }
  };

  // L2 touch. The eight slab work-groups of a head read every record line, and
  // without help all eight wait out the same DRAM fill together, which caps each
  // CU's request rate. So each line of chunk c + LA + INTER_TOUCH_AHEAD is first
  // read (one dword) by a single wave of the head, spread over its 32 waves, and
  // the eight real reads of it then hit in L2. The words are XOR-folded into
  // tacc, which only a never-taken branch stores: that keeps the loads alive
  // without making any step wait for them before the next one.
  constexpr int REC_LINES = (int)(RC::BYTES / 128);
  static_assert(RC::BYTES % 128 == 0 && REC_LINES <= 32 * 64, "one touch per lane per line");
  // lanes past the record's last line touch that line again: the load stays
  // unconditional, so its destination register is never merged with an old value
  const int touch_line = min((ct * 4 + w) + 32 * lane, REC_LINES - 1);
  // Each loop iteration covers TOUCH_STEPS chunks: its first step touches the next
  // TOUCH_STEPS chunks beyond the touch distance, and the words are folded in after
  // its last step. No touched word lives across the loop's back edge, where a
  // register copy would have to wait for it.
  constexpr int TOUCH_STEPS = 4;
  static_assert(TOUCH_STEPS % (LA + 1) == 0, "steps per loop iteration");
  unsigned tacc = 0u;

  InterStage<DP> st[LA + 1];
#pragma unroll
  for (int r = 0; r < LA; ++r)
    if (c_begin < c_end) load(st[r], min(c_begin + r, c_end - 1));
  for (int c0 = c_begin; c0 < c_end; c0 += TOUCH_STEPS) {
    unsigned tv[TOUCH_STEPS];
#pragma unroll
    for (int r = 0; r < TOUCH_STEPS; ++r) {
      const int c = c0 + r;
      // the stage consumed one step earlier takes chunk c + LA; past the end the
      // final record is loaded again, so every step issues the same loads and the
      // register stages rotate without leaving the loop body
      load(st[(r + LA) % (LA + 1)], min(c + LA, c_end - 1));
      if (r == 0) {
#pragma unroll
        for (int j = 0; j < TOUCH_STEPS; ++j)
          tv[j] = *reinterpret_cast<const unsigned*>(
              head_records + (size_t)min(c0 + LA + INTER_TOUCH_AHEAD + j, c_end - 1) * RC::BYTES +
              (size_t)touch_line * 128);
      }
      if (c < c_end) compute(st[r % (LA + 1)], c);
    }
#pragma unroll
    for (int j = 0; j < TOUCH_STEPS; ++j) tacc ^= tv[j];
  }
  // total_tokens is never negative (the host rejects it), so this never stores
  if (total_tokens < 0 && tacc == 0u) o[lane] = (__bf16)0.f;
  if (final_state) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) final_state[sidx + (size_t)(16 * j + i) * D] = Sw[j][i];
  }
}

}  // namespace kda
