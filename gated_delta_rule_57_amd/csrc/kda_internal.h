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
  int prefill_path;          // kda_prefill_path: 0 automatic, 1 record + slab state, 2 single pass,
                             // 3 record + segment-parallel state
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

// Workspace bytes for a prefill call on the given path (Fusion::prefill_path).
size_t prefill_workspace_bytes(int B, int T, int H, int num_seqs, bool varlen, int chunk, int dtype, int path = 0);

// The kernels a prefill runs, from its dtype, chunk and Fusion::prefill_path
// (kda_prefill_path in include/kda.h). Only bf16 with 64-token chunks has a choice.
enum PrefillKernels {
  KERNELS_RECORD_SLAB = 0,  // intra-chunk records, state kernels per 16 value columns
  KERNELS_RECORD_SEG = 1,   // intra-chunk records, segment-parallel full-width state kernels
  KERNELS_SINGLE = 2        // segment-parallel single pass, no records
};
// The automatic path takes the segment-parallel state kernels when the prefill has at
// least SEG_MIN_CHUNK_HEADS (chunk, head) pairs, counting the chunk bound of a packed
// batch: below that a slab work-group per (sequence, head, 16 value columns) leaves the
// chip's CUs free for one serial walk each, and the segment scan and short segments
// cost more (1 x 4K tokens x 32 heads: 0.155 against 0.189 ms); above it the slab
// work-groups share CUs and walk their chains in turn (8 x 4K x 32 heads: 1.14 against
// 0.87 ms; 1024 x 64 tokens x 32 heads: 4.75 against 3.26 ms; measured on MI355X).
constexpr int64_t SEG_MIN_CHUNK_HEADS = 4096;
inline int prefill_kernels(int dtype, int chunk, int path, int64_t max_chunks, int H) {
  if (dtype != 0 || chunk != 64) return KERNELS_RECORD_SLAB;
  if (path == 1) return KERNELS_RECORD_SLAB;
  if (path == 2) return KERNELS_SINGLE;
  if (path == 3) return KERNELS_RECORD_SEG;
  return max_chunks * H >= SEG_MIN_CHUNK_HEADS ? KERNELS_RECORD_SEG : KERNELS_RECORD_SLAB;
}

// Segment-parallel passes (kda_seg.hip): about SEG_TARGET_GROUPS work-groups per
// pass, segments of at least SEG_MIN_CHUNKS chunks.
constexpr int SEG_TARGET_GROUPS = 256;
constexpr int SEG_MIN_CHUNKS = 1;
// The first segment of a sequence is this share (percent) of the later ones: in pass
// A its work-groups write outputs while the others only compose maps (record-fed: a
// map chunk moves about 0.55 of an output chunk's bytes; single pass: about 0.8 of its
// work), so both finish together. With the output epilogue (RMSNorm and gate) an
// output chunk costs more (record-fed: it also reads the gate, about 1.3 times the time
// of a plain one; single pass: about 1.17 times), so the first segment is shorter.
constexpr int SEG_FIRST_PCT_RECORD = 55;
constexpr int SEG_FIRST_PCT_SINGLE = 80;
constexpr int SEG_FIRST_PCT_RECORD_GATED = 42;
constexpr int SEG_FIRST_PCT_SINGLE_GATED = 70;
int seg_chunks_per_segment(int64_t max_chunks, int N, int H, int first_pct);
int seg_first_chunks(int lseg, int first_pct);
// Workspace: segment offsets [N+1] int32, segment table [segments] int2, entry
// states [segments][H][128*128] fp32, segment maps [segments][H][2][128*128] fp32.
struct SegWs {
  int lseg, l0;  // chunks per segment after the first, and in the first
  int64_t max_segments;
  size_t off_seg_off, off_seg_info, off_seg_in, off_seg_map, total;
};
// single: the plan of the single pass (else the record-fed kernels); gated: with the
// output epilogue
SegWs seg_ws_layout(int B, int T, int H, int num_seqs, bool varlen, bool single, bool gated);
SegWs seg_ws_layout_for(int lseg, int l0, int64_t max_segments, int N, int H);
// The single pass: every step of the prefill for bf16, 64-token chunks.
hipError_t launch_prefill_seg(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                              int num_seqs, void* o, float* final_state, int B, int T, int H, const Fusion& fusion,
                              void* workspace, hipStream_t stream);
// The segment-parallel state kernels fed by bf16 64-token records (segment plan, first
// pass, scan, second pass), with the output epilogue of `fusion` fused in.
hipError_t launch_state_seg(const char* records, const int32_t* chunk_off, int64_t mc, const int32_t* cu_seqlens,
                            int N, int T, int H, const float* initial_state, float* final_state, void* o,
                            const Fusion& fusion, void* seg_workspace, const SegWs& plan, hipStream_t stream);

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
// chunk-entry states, the chunk-end state gradients, U~ and dU~, and T and M (two
// fp32 16 x 16 matrices) per (head, chunk).
struct BackwardWs {
  PrefillWs fwd;
  size_t off_brec, off_states, off_dstates, off_ut, off_dut, off_tm, total;
};
BackwardWs backward_ws_layout(int B, int T, int H, int num_seqs, bool varlen, int dtype);
size_t backward_workspace_bytes(int B, int T, int H, int num_seqs, bool varlen, int dtype);

// Gradients of the plain recurrence (see kda_chunk_bwd in include/kda.h).
hipError_t launch_backward(int dtype, const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                           const void* dout, const float* d_final, void* dq, void* dk, void* dv, float* dlog_alpha,
                           float* dbeta, float* d_initial, int B, int T, int H, void* workspace,
                           hipStream_t stream);

// The general diagonal-plus-low-rank forward (see kda_dplr_chunk_fwd in
// include/kda.h), 64-token chunks.
size_t dplr_workspace_bytes(int B, int T, int H, int num_seqs, bool varlen, int dtype);
hipError_t launch_dplr(int dtype, const void* q, const void* k, const void* v, const void* a, const void* b,
                       const float* log_alpha, const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                       void* o, float* final_state, int B, int T, int H, void* workspace, hipStream_t stream);

}  // namespace kda
