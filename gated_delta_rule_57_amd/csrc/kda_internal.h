// Internal interface between the C ABI layer (kda_api.hip) and the kernel
// launchers. Not installed; callers use include/kda.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Tracing hooks (see kda_timing_enable in include/kda.h): trace_begin before a
// call's first launch, trace_mark(kernel id) after each launch. No-ops unless
// timing is enabled.
void trace_begin(hipStream_t stream);
void trace_mark(hipStream_t stream, int kernel_id);

// The layer's prologue (on raw q, k, gate and beta inputs) and epilogue (output
// RMSNorm times a sigmoid gate), as described for kda_fusion in include/kda.h.
// Passed to kernels by value; all-zero = the plain recurrence.
struct Fusion {
  int normalize_qk;
  float qk_eps;
  int gate_preactivation;
  int beta_preactivation;
  const void* out_gate;      // nullable; o's layout and dtype
  const float* norm_weight;  // [128], with out_gate
  float norm_eps;
  int gate_kind;             // 0: per channel, 1: per (token, head), 2: none
};

// dtype: 0 = bf16, 1 = fp32 (the kda_dtype values).
hipError_t launch_decode(int dtype, const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, float* state, void* o, int N, int H, const Fusion& fusion,
                         hipStream_t stream);

// out = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate), rows of 128 values; out may equal o.
hipError_t launch_output_norm_gate(int dtype, const void* o, const void* gate, const float* weight, void* out,
                                   int64_t rows, float eps, hipStream_t stream);

// Upper bound on the number of chunks of a batch: B sequences of T tokens, or
// num_seqs packed sequences totalling T tokens.
int64_t max_chunks(int B, int T, int num_seqs, bool varlen, int chunk);

// Bytes of one per-(chunk, head) record written by the intra-chunk kernel.
size_t chunk_record_bytes(int dtype, int chunk);

// Workspace bytes for a prefill call.
size_t prefill_workspace_bytes(int B, int T, int H, int num_seqs, bool varlen, int chunk, int dtype);

hipError_t launch_prefill(int dtype, int chunk, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta, const float* initial_state,
                          const int32_t* cu_seqlens, int num_seqs, void* o, float* final_state, int B,
                          int T, int H, const Fusion& fusion, void* workspace, hipStream_t stream);

// Byte offsets of a prefill workspace: chunk plan (chunk_off [N+1], info [mc]
// int2) and the per-(head, chunk) records.
struct PrefillWs {
  size_t off_chunk_off, off_info, off_records, total;
};
PrefillWs prefill_ws_layout(int B, int T, int H, int num_seqs, bool varlen, int chunk, int dtype);
// The same layout for records of record_bytes each.
PrefillWs plan_ws_layout(int B, int T, int H, int num_seqs, bool varlen, int chunk, size_t record_bytes);

// The chunk plan: per-sequence first chunk (chunk_off [N+1]) and per-chunk (first
// token, length) (info [mc]) for chunks of the given length.
hipError_t launch_plan(const int32_t* cu_seqlens, int N, int T, int total_tokens, int chunk, int64_t mc,
                       int32_t* chunk_off, int2* info, hipStream_t stream);

// Chunk length of the backward pass.
constexpr int BWD_CHUNK = 16;

// Backward workspace: the forward's (at BWD_CHUNK), then the backward records, the
// chunk-entry states, the chunk-end state gradients, U~ and dU~ per (head, chunk).
struct BackwardWs {
  PrefillWs fwd;
  size_t off_brec, off_states, off_dstates, off_ut, off_dut, total;
};
BackwardWs backward_ws_layout(int B, int T, int H, int num_seqs, bool varlen, int dtype);
size_t backward_workspace_bytes(int B, int T, int H, int num_seqs, bool varlen, int dtype);

// Gradients of the plain recurrence (see kda_chunk_bwd in include/kda.h).
hipError_t launch_backward(int dtype, const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                           const void* dout, const float* d_final, void* dq, void* dk, void* dv, float* dlog_alpha,
                           float* dbeta, float* d_initial, int B, int T, int H, void* workspace,
                           hipStream_t stream);

// The first part of the forward pass at BWD_CHUNK-token chunks, for the backward:
// the chunk plan and the per-(head, chunk) records, in a workspace laid out by
// prefill_ws_layout(..., BWD_CHUNK, dtype). The backward launches the forward
// state pass (chunk-entry states and U~) itself.
hipError_t launch_forward_records(int dtype, const void* q, const void* k, const void* v, const float* log_alpha,
                                  const float* beta, const int32_t* cu_seqlens, int num_seqs, int B, int T, int H,
                                  void* workspace, hipStream_t stream);

// The general diagonal-plus-low-rank forward (see kda_dplr_chunk_fwd in
// include/kda.h), 64-token chunks.
size_t dplr_workspace_bytes(int B, int T, int H, int num_seqs, bool varlen, int dtype);
hipError_t launch_dplr(int dtype, const void* q, const void* k, const void* v, const void* a, const void* b,
                       const float* log_alpha, const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                       void* o, float* final_state, int B, int T, int H, void* workspace, hipStream_t stream);

}  // namespace kda
