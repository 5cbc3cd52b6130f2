// Device helpers for the layer prologue and epilogue around the KDA recurrence
// (GeekNews "Kimi Linear" summary, section "Kimi Linear 모델 구성": L2-normalised
// q and k, a GDN/Mamba-like decay function for the per-channel gate, a per-head
// RMSNorm and a data-dependent output gate). Readings where the page is silent
// are documented with kda_fusion in include/kda.h.
#pragma once

#include <hip/hip_runtime.h>

#include "kda_device.h"

namespace kda {

// log2(1 + 2^y) without overflow, from the hardware exp2 and log2: max(y, 0) +
// log2(1 + 2^-|y|). The argument of log2 is in (1, 2], where it is accurate; a
// term 2^-|y| below half an ulp of 1 is dropped, an absolute error < 2^-24.
__device__ __forceinline__ float softplus2_f(float y) {
  return fmaxf(y, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(y)));
}

// log(1 + e^x) = ln2 * log2(1 + 2^(x log2 e))
__device__ __forceinline__ float softplus_f(float x) {
  return 0.6931471805599453f * softplus2_f(x * 1.4426950408889634f);
}

// 1 / (1 + e^-x) without overflow
__device__ __forceinline__ float sigmoid_f(float x) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
  const float r = __builtin_amdgcn_rcpf(1.f + e);
  return x >= 0.f ? r : e * r;
}

// sum over the 32 lanes that share (lane & 32), i.e. one half of the wave: the 16-lane
// row sums (row16_sum, by DPP), then the two rows of the half added
__device__ __forceinline__ float half_wave_sum(float x) { return xor16_sum(row16_sum(x)); }

}  // namespace kda
