// Inter-chunk state pass for 16-token chunks (bf16 or fp32 records), shared by the
// chunk-16 prefill and the backward's forward state pass.
#pragma once

#include "kda_device.h"
#include "kda_record.h"

namespace kda {

// ---------------------------------------------------------------------------
// Inter-chunk kernel for 16-token chunks: four waves per (sequence, head, 16-column
// slab), wave w keeping state rows 32w .. 32w+31. Per chunk, wave w forms its
// k-block's part of U~ = U - W S (and of (Q e^G) S), the four parts are summed
// through LDS behind one barrier that leaves global loads in flight, and each wave
// updates its own rows. The next chunk's fragments are loaded into registers while
// the current one is computed, and each record line is touched in L2 a few chunks
// ahead by one wave of the head.
// The backward's forward pass keeps the state entering every chunk and U~. Their
// stores go out through a fifth wave: the four compute waves put their accumulator
// registers into LDS (one 8-byte write per 16 x 16 tile and lane), and after the
// chunk's barrier the store wave reads them back transposed and writes whole 16 x 16
// tiles (non-temporal: only the gradient kernel reads them back). On this
// architecture stores count in the same in-order counter as loads, so a compute
// wave that stored would wait on its own store acknowledgements each time it waits
// for the next chunk's operands.
// ---------------------------------------------------------------------------
constexpr int INTER16_LOOKAHEAD = 3;
constexpr int INTER16_TOUCH_AHEAD = 4;

// The body of one work-group with work-group index b, laid out like the 64-token
// kernel: b & 7 selects the XCD, (b >> 3) & 7 the slab, b >> 6 the (sequence, head)
// group. Called by inter16_kernel (WANT_O: 256 threads, o non-null, states and ut
// null) and by the backward's forward state pass (!WANT_O: 320 threads, the fifth
// wave storing states and ut, both non-null; Q e^G and P are neither loaded nor
// touched in L2, which leaves fewer than half of the bytes per chunk).
template <typename E, bool WANT_O>
__device__ __forceinline__ void inter16_body(int b, const char* __restrict__ records,
                                             const int32_t* __restrict__ chunk_off, const int2* __restrict__ info,
                                             const float* __restrict__ initial_state, float* __restrict__ final_state,
                                             E* __restrict__ o, int N, int H, int mc, E* __restrict__ states,
                                             E* __restrict__ ut) {
  using RC = Rec<E, 16>;
  typedef typename Frag<E>::T FragT;
  static_assert(RC::NRT == 1 && RC::NKC == 1, "16-token chunks");
  typedef typename Vec4<E>::T V4;
  constexpr bool SW = !WANT_O;  // a store wave (wave 4) writes the states and U~
  __shared__ floatx4 xp[2][4][64];  // U~ parts, by chunk parity
  __shared__ floatx4 xq[WANT_O ? 2 : 1][4][WANT_O ? 64 : 1];  // (Q e^G) S parts
  // by chunk parity: the state entering the chunk, tile rt (rows 16 rt ..) of the slab
  // at [rt][lane][4] in accumulator order (lane (m, g) holds rows 4g .. 4g+3 of column
  // m), and U~ the same way
  __shared__ __attribute__((aligned(16))) E stg_s[SW ? 2 : 1][SW ? 8 * 64 * 4 : 4];
  __shared__ __attribute__((aligned(16))) E stg_u[SW ? 2 : 1][SW ? 64 * 4 : 4];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int xcd = b & 7, rest = b >> 3;
  const int ct = rest & 7, slot = rest >> 3;
  const int u = slot * 8 + xcd;
  if (u >= N * H) return;  // uniform over the work-group
  const int n = u / H, h = u - n * H;
  const size_t HD = (size_t)H * D;
  const int c_begin = chunk_off[n], c_end = chunk_off[n + 1];

  if constexpr (SW) {
   if (w == 4) {
    // the store wave: one barrier per chunk, as the compute waves, and one after the
    // last. After the barrier of the chunk i-th from the start, that chunk's state
    // and the previous chunk's U~ are in LDS until the next barrier but one. For U~
    // lane (m, g) stores row m, columns 16 ct + 4 g .. + 3, reading the four values
    // from lanes 4 g .. 4 g + 3, slot m % 4, of the accumulator order.
    auto gather = [&](const E* tile) {
      V4 x;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) x[s4] = tile[(4 * g + s4 + 16 * (m >> 2)) * 4 + (m & 3)];
      return x;
    };
    E* ut_h = ut + (size_t)h * mc * 16 * D + ((size_t)ct * 64 + lane) * 4;
    for (int i = 0; c_begin + i < c_end; ++i) {
      lds_barrier();
      const int c = c_begin + i;
      store_state_slab(states + ((size_t)h * mc + c) * D * D + (size_t)ct * 2048, stg_s[i & 1], lane);
      if (i > 0) store_nt(reinterpret_cast<V4*>(ut_h + (size_t)(c - 1) * 16 * D), gather(stg_u[(i - 1) & 1]));
    }
    lds_barrier();
    if (c_end > c_begin)
      store_nt(reinterpret_cast<V4*>(ut_h + (size_t)(c_end - 1) * 16 * D), gather(stg_u[(c_end - c_begin - 1) & 1]));
    return;
   }
  }

  // state rows 32w + 16j + 4g + i, column 16ct + m
  const size_t sbase = (size_t)u * D * D + (size_t)(32 * w + 4 * g) * D + 16 * ct + m;

  floatx4 S[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    S[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (initial_state) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[j][i] = initial_state[sbase + (size_t)(16 * j + i) * D];
    }
  }

  // a stage holds what the loads return, unconverted: converting at load time would
  // make the wave wait for the data one step early
  struct Stage {
    FragT wn, qt, ke[2], pp;
    typename Vec4<E>::T uu;
    float gw;  // e^{g_C} of row 32w + row_word_index(m, g)
    int2 inf;
  };
  auto load = [&](Stage& st, int c) {
    const char* rb = records + ((size_t)h * mc + c) * RC::BYTES;
    const E* rec = reinterpret_cast<const E*>(rb);
    st.wn = load_frag<E>(rec + RC::WN + ((size_t)w * 64 + lane) * 8);
    if constexpr (WANT_O) {
      st.qt = load_frag<E>(rec + RC::QT + ((size_t)w * 64 + lane) * 8);
      if (w == 1) st.pp = load_frag<E>(rec + RC::PP + (size_t)lane * 8);  // used by wave 1 only
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) st.ke[j] = load_frag<E>(rec + RC::KE + ((size_t)(2 * w + j) * 64 + lane) * 8);
    if (w == 0)  // U is added by wave 0 only (w is uniform over the wave)
      st.uu = *reinterpret_cast<const typename Vec4<E>::T*>(rec + RC::UU + ((size_t)ct * 64 + lane) * 4);
    const float* gam = reinterpret_cast<const float*>(rb + RC::GAMMA_BYTES);
    st.gw = gam[32 * w + row_word_index(m, g)];
    st.inf = info[c];
  };

  auto compute = [&](const Stage& st, int c, int buf) {
    const FragT Sb = acc_pair_to_frag<E>(S[0], S[1]);  // k-block w of the state
    if constexpr (SW) {  // this wave's two tiles of the state entering the chunk, to LDS
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        V4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = from_f<E>(S[j][i]);
        *reinterpret_cast<V4*>(&stg_s[buf][((2 * w + j) * 64 + lane) * 4]) = x;
      }
    }
    // parts over this wave's 32 state rows: U - W S (U added once, by wave 0) and (Q e^G) S
    floatx4 up = w == 0 ? floatx4{to_f(st.uu[0]), to_f(st.uu[1]), to_f(st.uu[2]), to_f(st.uu[3])}
                        : floatx4{0.f, 0.f, 0.f, 0.f};
    mma(up, st.wn, Sb);
    xp[buf][w][lane] = up;
    if constexpr (WANT_O) {
      floatx4 xpart = {0.f, 0.f, 0.f, 0.f};
      mma(xpart, st.qt, Sb);
      xq[buf][w][lane] = xpart;
    }
    lds_barrier();
    const floatx4 Ut = xp[buf][0][lane] + xp[buf][1][lane] + xp[buf][2][lane] + xp[buf][3][lane];
    if constexpr (SW) {
      if (w == 0) {  // U~ to LDS, for the store wave after the next barrier
        V4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = from_f<E>(Ut[i]);
        *reinterpret_cast<V4*>(&stg_u[buf][lane * 4]) = x;
      }
    }
    const FragT Ub = acc_pair_to_frag<E>(Ut, floatx4{0.f, 0.f, 0.f, 0.f});
    if constexpr (WANT_O) {
      if (w == 1) {  // O = (Q e^G) S + P U~
        floatx4 X = xq[buf][0][lane] + xq[buf][1][lane] + xq[buf][2][lane] + xq[buf][3][lane];
        mma(X, st.pp, Ub);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * g + i;
          if (row < st.inf.y) o[(size_t)(st.inf.x + row) * HD + (size_t)h * D + 16 * ct + m] = from_f<E>(X[i]);
        }
      }
    }
    // S_w = Diag(e^{g_C}) S_w + (K e^{g_C - G})^T_w U~
    floatx4 gm[2];
    rows_from_word(st.gw, m, gm);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      S[j] = gm[j] * S[j];
      mma(S[j], st.ke[j], Ub);
    }
  };

  // L2 touch INTER16_TOUCH_AHEAD chunks beyond the register stage: each line of the
  // record that the loads above read is read first (one word) by one of the head's 32
  // waves, so the real loads hit in L2 (the words are XOR-folded into tacc, stored
  // only by a never-taken branch). Without the output only the W, K e^{g_C-G}, U and
  // e^{g_C} lines are needed.
  constexpr int LINES = (int)(RC::BYTES / 128);
  static_assert(RC::BYTES % 128 == 0 && LINES <= 32 * 64, "one touch per lane");
  constexpr int WN_L = (int)((RC::QT - RC::WN) * sizeof(E) / 128);
  constexpr int KE_L = (int)((RC::PP - RC::KE) * sizeof(E) / 128);
  constexpr int UU_L = (int)(RC::GAMMA_BYTES / 128) - (int)(RC::UU * sizeof(E) / 128);
  constexpr int NEED = WANT_O ? LINES : WN_L + KE_L + UU_L + (LINES - (int)(RC::GAMMA_BYTES / 128));
  static_assert((RC::QT * sizeof(E)) % 128 == 0 && (RC::KE * sizeof(E)) % 128 == 0 &&
                (RC::PP * sizeof(E)) % 128 == 0 && (RC::UU * sizeof(E)) % 128 == 0, "line-aligned parts");
  // lanes past the last needed line touch that line again (an unconditional load is
  // never merged with an old value)
  const int tl = min((ct * 4 + w) + 32 * lane, NEED - 1);
  const int touch_line = WANT_O ? tl
                         : tl < WN_L        ? tl
                         : tl < WN_L + KE_L ? (int)(RC::KE * sizeof(E) / 128) + (tl - WN_L)
                                            : (int)(RC::UU * sizeof(E) / 128) + (tl - WN_L - KE_L);
  // each loop iteration covers four chunks: its first step touches the next four
  // beyond the touch distance and the words are folded in after its last step, so
  // no touched word lives across the back edge (where a copy would wait for it)
  unsigned tacc = 0u;

  // INTER16_LOOKAHEAD chunks of operands in flight in registers
  constexpr int LA = INTER16_LOOKAHEAD;
  static_assert(4 % (LA + 1) == 0, "four steps per loop iteration");
  Stage st[LA + 1];
#pragma unroll
  for (int r = 0; r < LA; ++r)
    if (c_begin < c_end) load(st[r], min(c_begin + r, c_end - 1));
  for (int c0 = c_begin; c0 < c_end; c0 += 4) {
    unsigned tv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = c0 + r;
      // the stage consumed one step earlier takes chunk c + LA (past the end, the
      // last chunk again: every step issues the same loads)
      load(st[(r + LA) % (LA + 1)], min(c + LA, c_end - 1));
      if (r == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          tv[j] = *reinterpret_cast<const unsigned*>(
              records + ((size_t)h * mc + min(c0 + LA + INTER16_TOUCH_AHEAD + j, c_end - 1)) * RC::BYTES +
              (size_t)touch_line * 128);
      }
      if (c < c_end) compute(st[r % (LA + 1)], c, r & 1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) tacc ^= tv[j];
  }
  if constexpr (SW) lds_barrier();  // the store wave's last one: U~ of the last chunk
  // mc is never negative (the host sizes it from the shapes), so this never stores
  if (mc < 0 && tacc == 0u) o[lane] = from_f<E>(0.f);
  if (final_state) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) final_state[sbase + (size_t)(16 * j + i) * D] = S[j][i];
  }
}

}  // namespace kda
