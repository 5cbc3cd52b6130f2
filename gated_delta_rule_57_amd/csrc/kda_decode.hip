// Single-token KDA decode step on gfx950.
//
// One new token per (sequence, head) against a persisted 128 x 128 fp32 state,
// updated in place. The recurrence (GeekNews "Kimi Linear" summary, section
// "Kimi Delta Attention의 세밀한 메모리 제어"; "From GPT-2 to Kimi K3" digest,
// sections "DeltaNet -- 유한한 캐시의 덮어쓰기" and "Kimi Linear (KDA) -- 채널별
// 세밀한 게이팅"), expanded so that the state is read once and written once:
//     S' = Diag(alpha) S ; r = S'^T k ; p = S'^T q ; u = beta (v - r)
//     S  = S' + k u^T    ; o = S^T q = p + (k^T q) u
// Work is bound by HBM: 64 KiB read + 64 KiB written per (sequence, head),
// against ~7 flops per state element. Each work-group owns one state: 256 threads,
// thread (rg, cg) holds rows 16 rg .. 16 rg + 15 and columns 4 cg .. 4 cg + 3 in
// registers (16 float4 loads, streamed with non-temporal hints because the state
// of a batch is larger than the last-level cache and is not reused within a step).
#include "kda_device.h"
#include "kda_fusion_dev.h"
#include "kda_internal.h"

namespace kda {

template <typename E>
__global__ void __launch_bounds__(256) decode_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                     const E* __restrict__ v,
                                                     const float* __restrict__ log_alpha,
                                                     const float* __restrict__ beta,
                                                     float* __restrict__ state, E* __restrict__ o, Fusion fu) {
  __shared__ float s_ka[D];      // alpha_i k_i
  __shared__ float s_qa[D];      // alpha_i q_i
  __shared__ float s_alpha[D];
  __shared__ float s_k[D];
  __shared__ float s_red[2][3];  // per wave of the first two: k.k, q.q, k.q
  __shared__ floatx4 s_part[8][32][2];  // per row group: partial r and p for 4 columns

  const int t = threadIdx.x;
  const size_t nh = blockIdx.x;
  const int cg = t & 31, rg = t >> 5;
  float* S = state + nh * (size_t)(D * D);

  // Issue the state loads first: they are the bulk of the traffic.
  floatx4 srow[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    srow[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(S + (size_t)(16 * rg + i) * D + 4 * cg));

  // k^T k, q^T q and k^T q over the 128 channels: wave-level reductions in waves 0
  // and 1, combined through LDS
  float kk = 0.f, qq = 0.f, a = 0.f;
  if (t < D) {
    // decay: per key channel, one per (sequence, head), or none (alpha = 1)
    float la = 0.f;
    if (fu.gate_kind == 0) la = log_alpha[nh * D + t];
    else if (fu.gate_kind == 1) la = log_alpha[nh];
    if (fu.gate_kind != 2 && fu.gate_preactivation) la = -softplus_f(la);
    a = __expf(la);
    kk = to_f(k[nh * D + t]);
    qq = to_f(q[nh * D + t]);
    // wave sums by DPP inside 16-lane rows and lane swaps across them (no LDS trips)
    const float pk = xor32_sum(xor16_sum(row16_sum(kk * kk)));
    const float pq = xor32_sum(xor16_sum(row16_sum(qq * qq)));
    const float pkq = xor32_sum(xor16_sum(row16_sum(kk * qq)));
    if ((t & 63) == 0) {
      s_red[t >> 6][0] = pk;
      s_red[t >> 6][1] = pq;
      s_red[t >> 6][2] = pkq;
    }
  }
  __syncthreads();
  // prologue on raw inputs: L2-normalise k and q
  float ik = 1.f, iq = 1.f;
  if (fu.normalize_qk) {
    ik = rsqrtf(s_red[0][0] + s_red[1][0] + fu.qk_eps);
    iq = rsqrtf(s_red[0][1] + s_red[1][1] + fu.qk_eps);
  }
  const float kq = (s_red[0][2] + s_red[1][2]) * ik * iq;
  if (t < D) {
    kk *= ik;
    qq *= iq;
    s_alpha[t] = a;
    s_k[t] = kk;
    s_ka[t] = a * kk;
    s_qa[t] = a * qq;
  }
  __syncthreads();

  floatx4 r = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float ka = s_ka[16 * rg + i], qa = s_qa[16 * rg + i];
    r += ka * srow[i];
    p += qa * srow[i];
  }
  s_part[rg][cg][0] = r;
  s_part[rg][cg][1] = p;
  __syncthreads();

  floatx4 rs = {0.f, 0.f, 0.f, 0.f}, ps = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rs += s_part[j][cg][0];
    ps += s_part[j][cg][1];
  }
  float vv[4];
  load4f(v + nh * D + 4 * cg, vv);
  const float b = fu.beta_preactivation ? sigmoid_f(beta[nh]) : beta[nh];
  floatx4 u, out;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    u[jj] = b * (vv[jj] - rs[jj]);
    out[jj] = ps[jj] + kq * u[jj];
  }
  if (rg == 0) {
    float ov[4] = {out[0], out[1], out[2], out[3]};
    if (fu.out_gate) {
      // epilogue: RMSNorm over the 128 outputs (the 32 lanes of this half-wave hold
      // them all), times the weight and the sigmoid output gate
      const float inv = rsqrtf(half_wave_sum(ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3]) *
                               (1.f / D) + fu.norm_eps);
      float z[4];
      load4f(reinterpret_cast<const E*>(fu.out_gate) + nh * D + 4 * cg, z);
      const floatx4 wv = *reinterpret_cast<const floatx4*>(fu.norm_weight + 4 * cg);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) ov[jj] = ov[jj] * inv * wv[jj] * sigmoid_f(z[jj]);
    }
    store4f(o + nh * D + 4 * cg, ov);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = s_alpha[16 * rg + i], kk = s_k[16 * rg + i];
    floatx4 nv = a * srow[i] + kk * u;
    __builtin_nontemporal_store(nv, reinterpret_cast<floatx4*>(S + (size_t)(16 * rg + i) * D + 4 * cg));
  }
}

hipError_t launch_decode(int dtype, const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, float* state, void* o, int N, int H, const Fusion& fusion,
                         hipStream_t stream) {
  const size_t units = (size_t)N * H;
  if (units == 0) return hipSuccess;
  dim3 grid((unsigned)units), block(256);
  trace_begin(stream);
  if (dtype == 0)
    hipLaunchKernelGGL(decode_kernel<__bf16>, grid, block, 0, stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, log_alpha, beta, state, (__bf16*)o, fusion);
  else
    hipLaunchKernelGGL(decode_kernel<float>, grid, block, 0, stream, (const float*)q, (const float*)k,
                       (const float*)v, log_alpha, beta, state, (float*)o, fusion);
  hipError_t e = hipGetLastError();
  trace_mark(stream, 3);
  return e;
}

}  // namespace kda
