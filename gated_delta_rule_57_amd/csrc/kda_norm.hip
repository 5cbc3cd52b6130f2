// Output epilogue of the KDA layer on gfx950: per-head RMSNorm times a sigmoid
// output gate (GeekNews "Kimi Linear" summary, section "Kimi Linear 모델 구성":
// a per-head RMSNorm and a data-dependent output gate come before the output
// projection), for the rows of a prefill output.
//
//   out[r][:] = o[r][:] / sqrt(mean_j o[r][j]^2 + eps) * weight[:] * sigmoid(gate[r][:])
//
// One row = one (token, head), 128 values. Sixteen lanes own a row, eight values
// per lane (one 16-byte load of bf16), so the mean square is a 16-lane sum; a
// work-group of 256 threads covers 16 rows. HBM-bound: o and gate are read once
// and out written once.
#include "kda_device.h"
#include "kda_fusion_dev.h"
#include "kda_internal.h"

namespace kda {

template <typename E>
__global__ void __launch_bounds__(256) output_norm_gate_kernel(const E* __restrict__ o, const E* __restrict__ gate,
                                                               const float* __restrict__ weight, E* out,
                                                               int64_t rows, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = 8 * (threadIdx.x & 15);
  // rows past the end read row 0 and store nothing, so every lane takes part in the sum
  const size_t base = (size_t)(row < rows ? row : 0) * D + c;
  float x[8], z[8];
  load4f(o + base, x);
  load4f(o + base + 4, x + 4);
  load4f(gate + base, z);
  load4f(gate + base + 4, z + 4);
  const floatx4 w0 = *reinterpret_cast<const floatx4*>(weight + c);
  const floatx4 w1 = *reinterpret_cast<const floatx4*>(weight + c + 4);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
  ss = row16_sum(ss);
  const float inv = rsqrtf(ss * (1.f / D) + eps);
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = x[j] * inv * (j < 4 ? w0[j] : w1[j - 4]) * sigmoid_f(z[j]);
  if (row < rows) {
    store4f(out + base, y);
    store4f(out + base + 4, y + 4);
  }
}

hipError_t launch_output_norm_gate(int dtype, const void* o, const void* gate, const float* weight, void* out,
                                   int64_t rows, float eps, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = (rows + 15) / 16;
  if (dtype == 0)
    hipLaunchKernelGGL(output_norm_gate_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const __bf16*)o, (const __bf16*)gate, weight, (__bf16*)out, rows, eps);
  else
    hipLaunchKernelGGL(output_norm_gate_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float*)o, (const float*)gate, weight, (float*)out, rows, eps);
  hipError_t e = hipGetLastError();
  trace_mark(stream, 4);
  return e;
}

}  // namespace kda
