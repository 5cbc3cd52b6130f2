/*
 * kda.h -- C ABI of libkda.so: Kimi Delta Attention (KDA) forward on AMD MI355X (gfx950).
 *
 * KDA is the delta-rule linear-attention recurrence with a per-channel forget gate.
 * Per sequence and head, token by token,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T ,   o_t = S_t^T q_t ,
 *
 * with S in R^{dk x dv}, alpha_t = exp(log_alpha_t) one decay per key channel and
 * beta_t one write strength per (token, head). The output reads the state after its
 * own token's update. Sources (web pages on the method):
 *   - "From GPT-2 to Kimi K3" digest, sections "DeltaNet -- 유한한 캐시의 덮어쓰기"
 *     (read with the key, subtract, write the difference back along the key),
 *     "Gated DeltaNet -- 망각을 더하다" (a decay alpha in [0,1]; 1 = pure delta rule)
 *     and "Kimi Linear (KDA) -- 채널별 세밀한 게이팅" (the scalar becomes Diag(alpha));
 *   - GeekNews "Kimi Linear" summary, sections "Kimi Delta Attention의 세밀한 메모리
 *     제어" (per-channel diagonal gate, DPLR transition tied to k), "청크 단위 병렬
 *     알고리듬" (chunkwise WY/UT algorithm, forward substitution) and "Kimi Linear
 *     모델 구성" (L2-normalised q and k; head dimension 128).
 *
 * Common conventions
 *   - Every pointer passed to a compute entry point is a DEVICE pointer on the
 *     current HIP device, owned by the caller. The library keeps no pointer after it
 *     returns. Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream); buffers must stay alive until that stream has finished.
 *   - All argument checks run on the host before any HIP call and return a status;
 *     nothing is ever thrown across the ABI. A device fault surfaces at the caller's
 *     next synchronisation of the stream.
 *   - dk = dv = 128 only (the head dimension the pages use for all experiments);
 *     any other value returns KDA_ERR_UNSUPPORTED.
 *   - q, k, v and o have dtype `dtype` (KDA_BF16 or KDA_FP32). log_alpha, beta,
 *     initial_state, final_state and the decode state are always float32.
 *   - Every tensor pointer must be 16-byte aligned, except beta and cu_seqlens (4
 *     bytes) and the workspace (256 bytes); KDA_ERR_INVALID_ARG otherwise.
 *   - Value preconditions (documented, not checked): q and k are L2-normalised per
 *     (token, head) by the caller; log_alpha is finite and <= 0; beta is in [0, 1]
 *     (unless the kda_fusion prologue below derives them from raw inputs).
 *     Outside them the result is unspecified but every kernel still terminates.
 *   - No scale is applied to q.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 5

/* Element type of q, k, v and o. */
typedef enum { KDA_BF16 = 0, KDA_FP32 = 1 } kda_dtype;

/* Return codes of every entry point. */
typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = -1, /* null required pointer, bad shape, misalignment, bad cu_seqlens use */
  KDA_ERR_UNSUPPORTED = -2, /* dk/dv != 128, chunk not in {16, 64}, unknown dtype */
  KDA_ERR_WORKSPACE = -3,   /* caller workspace smaller than kda_chunk_fwd_workspace_size() */
  KDA_ERR_DEVICE = -4       /* a HIP call failed; kda_last_error() holds its message */
} kda_status;

/* Version of this ABI (KDA_ABI_VERSION of the built library). */
int kda_abi_version(void);

/* Static text for a status code. */
const char *kda_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char *kda_last_error(void);

/*
 * Bytes of device workspace kda_chunk_fwd needs for this problem (an upper bound
 * that does not depend on the sequence lengths inside cu_seqlens). Returns 0 for
 * arguments kda_chunk_fwd would reject. With cu_seqlens, pass B = 1 and num_seqs =
 * its number of sequences; without, num_seqs is ignored (B sequences of T tokens).
 */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int num_seqs, int chunk, int dtype);

/*
 * Chunked prefill: runs the recurrence over whole sequences.
 *
 * The chunkwise algorithm (GeekNews "Kimi Linear" summary, section "청크 단위 병렬
 * 알고리듬"; "From GPT-2 to Kimi K3" digest, section "DeltaNet 병렬화 -- 청크 단위
 * 학습"): each sequence is cut into chunks of `chunk` tokens from its own start (the
 * last one may be partial); each chunk's decay-weighted A = tril(beta (K e^G)(K e^-G)^T)
 * is inverted as I + A by forward substitution into the WY factors, and the fp32
 * state is carried across the chunks of each sequence while the outputs are written.
 * For bf16 with 64-token chunks the default state step is segment-parallel: a
 * work-group owns a run of chunks of one (sequence, head) and the whole 128 x 128
 * state, reading each chunk's record once; the middle runs of a long sequence first
 * compose their chunk maps (the state is an affine function of the state entering a
 * run), a short scan gives every run its entry state, then the runs write their
 * outputs. kda_fusion.prefill_path selects the other kernel sets (see
 * kda_prefill_path). The result does not depend on `chunk` or the path except for
 * rounding.
 *
 *   q, k        [B, T, H, dk]  dtype      o          [B, T, H, dv]  dtype (written)
 *   v           [B, T, H, dv]  dtype      log_alpha  [B, T, H, dk]  float32
 *   beta        [B, T, H]      float32
 *   initial_state [N, H, dk, dv] float32 or NULL (zeros); S[i][j] = key channel i, value channel j
 *   final_state   [N, H, dk, dv] float32 or NULL (not written); may equal initial_state
 *   cu_seqlens  int32 [num_seqs + 1] or NULL. With it, B must be 1 and sequence n is
 *               tokens [cu_seqlens[n], cu_seqlens[n+1]) of the T packed tokens; the
 *               entries must be non-decreasing with cu_seqlens[0] = 0 and
 *               cu_seqlens[num_seqs] = T (a precondition: it lives on the device and
 *               is not read by the host). Zero-length sequences are allowed
 *               (final = initial). Without it, N = B sequences of T tokens.
 *   chunk       16 or 64.
 *   workspace   device buffer of at least kda_chunk_fwd_workspace_size() bytes, or
 *               NULL: the library then allocates and frees it in stream order. It
 *               holds one record per (chunk, head) (1.16 KB per token and head in
 *               bf16) and, on the segment-parallel paths, three 128 x 128 fp32 states
 *               per (segment, head) (about 60 MiB at 128K tokens x 32 heads; the single
 *               pass needs only these).
 * T = 0 (or B = 0) is a valid call that copies initial_state to final_state (zeros
 * if initial_state is NULL). `o` must not alias any input. Size limits, each
 * KDA_ERR_INVALID_ARG: B*T below 2^31 - 64 tokens, N*H below 2^25 (sequence, head)
 * pairs, and (chunks, bounded by B*ceil(T/chunk) or ceil(T/chunk) + num_seqs) * H
 * below 2^31.
 */
int kda_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                  const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                  int num_seqs, void *o, float *final_state, int B, int T, int H, int dk,
                  int dv, int chunk, int dtype, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * One decode step for N independent sequences: the recurrence applied to a single
 * new token per (sequence, head), on a persisted state updated in place. It reads
 * and writes each 128 x 128 fp32 state once.
 *
 *   q, k        [N, H, dk] dtype      v, o  [N, H, dv] dtype (o written)
 *   log_alpha   [N, H, dk] float32    beta  [N, H]     float32
 *   state       [N, H, dk, dv] float32, in/out
 * N = 0 is a valid no-op. `o` must not alias any input or the state.
 */
int kda_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                    const float *beta, float *state, void *o, int N, int H, int dk, int dv,
                    int dtype, void *stream);

/*
 * The layer's prologue and epilogue, fused around the recurrence. The Kimi Linear
 * layer (GeekNews "Kimi Linear" summary, section "Kimi Linear 모델 구성") L2-normalises
 * each head's query and key for eigenvalue stability, takes the per-channel decay
 * from a GDN/Mamba-like decay function of a low-rank projection, and applies a
 * per-head RMSNorm and a data-dependent output gate before the output projection.
 * Readings where the page is silent (the same as the oracle's):
 *   normalize_qk        q and k are raw: each (token, head) row x becomes
 *                       x / sqrt(sum_i x_i^2 + qk_eps)           (qk_eps >= 0)
 *   gate_preactivation  log_alpha holds a pre-activation a: log alpha = -softplus(a)
 *   beta_preactivation  beta holds a pre-activation b: beta = sigmoid(b)
 *   out_gate            NULL, or z with o's layout and dtype: each output row becomes
 *                       o / sqrt(mean_j o_j^2 + norm_eps) * norm_weight * sigmoid(z)
 *                       (norm_weight: float32 [dv], shared by the heads, 16-byte
 *                       aligned, required with out_gate; norm_eps >= 0)
 *   prefill_path        a kda_prefill_path value, see below
 * Zero-initialised = the plain recurrence on the automatic path. The prologue runs
 * inside the kernels that read q, k, log_alpha and beta. The prefill epilogue runs
 * inside the segment-parallel state kernels, whose work-groups hold whole output rows;
 * with the slab state kernels (KDA_PATH_RECORD, other dtypes and chunks) it is one
 * more pass over o (a row's dv values are spread over work-groups there). The decode
 * epilogue runs inside the decode kernel.
 */
typedef struct kda_fusion {
  int normalize_qk;
  float qk_eps;
  int gate_preactivation;
  int beta_preactivation;
  const void *out_gate;
  const float *norm_weight;
  float norm_eps;
  int gate_kind;    /* a kda_gate value, see below */
  int prefill_path; /* a kda_prefill_path value, see below */
} kda_fusion;

/*
 * Which kernels a prefill runs (kda_fusion.prefill_path). Only bf16 with 64-token
 * chunks has a choice; every other dtype and chunk runs the record path.
 *   KDA_PATH_AUTO         an intra-chunk kernel writes a record per (chunk, head); when
 *                         the call has at least 4096 (chunk, head) pairs (counting the
 *                         chunk bound ceil(T / 64) + num_seqs of a packed batch) the
 *                         segment-parallel full-width state kernels read each record
 *                         once per sequence segment, otherwise the KDA_PATH_RECORD state
 *                         kernels run (the default; the faster of the two at each size)
 *   KDA_PATH_RECORD       the same records; the state kernel runs one work-group per
 *                         (sequence, head, 16 value columns) over the whole sequence,
 *                         the structure kda_dplr_chunk_fwd also has
 *   KDA_PATH_SINGLE_PASS  no records: the segment-parallel work-groups form each
 *                         chunk's matrices themselves (the middle segments twice),
 *                         with the least HBM traffic and a workspace of a few states
 *                         per (segment, head)
 *   KDA_PATH_RECORD_SEGMENTED  the records and the segment-parallel state kernels at
 *                         any size
 * All of them compute the same recurrence.
 */
typedef enum {
  KDA_PATH_AUTO = 0,
  KDA_PATH_RECORD = 1,
  KDA_PATH_SINGLE_PASS = 2,
  KDA_PATH_RECORD_SEGMENTED = 3
} kda_prefill_path;

/*
 * Decay granularity (kda_fusion.gate_kind). The pages trace KDA back through two
 * special cases ("From GPT-2 to Kimi K3" digest, sections "DeltaNet -- 유한한 캐시의
 * 덮어쓰기" and "Gated DeltaNet -- 망각을 더하다"; GeekNews "Kimi Linear" summary,
 * section "선형 어텐션에서 Gated DeltaNet까지"): Gated DeltaNet has one scalar decay per
 * (token, head) and DeltaNet none (alpha = 1). They run on dedicated paths that need
 * no per-channel decay factoring:
 *   KDA_GATE_CHANNEL  log_alpha [.., H, dk], one decay per key channel (KDA; the default)
 *   KDA_GATE_HEAD     log_alpha [.., H], one decay per (token, head), 4-byte aligned
 *   KDA_GATE_NONE     alpha = 1; log_alpha is not read and may be NULL
 * gate_preactivation applies to the gate that is read.
 */
typedef enum { KDA_GATE_CHANNEL = 0, KDA_GATE_HEAD = 1, KDA_GATE_NONE = 2 } kda_gate;

/*
 * kda_chunk_fwd with the prologue / epilogue of `fusion` (NULL = kda_chunk_fwd).
 * All other arguments, the workspace and the errors are those of kda_chunk_fwd;
 * a bad fusion field (negative eps, out_gate without norm_weight, misalignment)
 * returns KDA_ERR_INVALID_ARG. With out_gate, o receives the gated, normalised output.
 */
int kda_chunk_fwd_fused(const void *q, const void *k, const void *v, const float *log_alpha,
                        const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                        int num_seqs, void *o, float *final_state, int B, int T, int H, int dk,
                        int dv, int chunk, int dtype, const kda_fusion *fusion, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Workspace bytes of kda_chunk_fwd_fused with this `fusion` (its prefill_path decides);
 * 0 for arguments the call would reject. */
size_t kda_chunk_fwd_fused_workspace_size(int B, int T, int H, int num_seqs, int chunk, int dtype,
                                          const kda_fusion *fusion);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments and
 * results as kda_chunk_fwd without the workspace; nothing is allocated. The kernels'
 * scratch is a static device array of KDA_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU
 * the library runs on holds from the first call until the process ends; its address
 * is looked up once per device. bf16 with 64-token chunks runs the single-pass
 * kernels (KDA_PATH_SINGLE_PASS), whose scratch is a few 128 x 128 fp32 states per
 * (segment, head): about 60 MiB at 128K tokens x 32 heads; fp32 and 16-token chunks
 * run the record path, whose scratch grows with B*T*H (kda_chunk_fwd_fused_workspace_size
 * with that prefill_path gives the need of any configuration). A configuration that
 * needs more than the array holds returns KDA_ERR_WORKSPACE before any HIP call.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other host threads) race.
 * With kda_timing_enable on, the timing records still create host-side events.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *log_alpha,
                          const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                          int num_seqs, void *o, float *final_state, int B, int T, int H, int dk,
                          int dv, int chunk, int dtype, void *stream);

/* kda_decode_step with the prologue / epilogue of `fusion` (NULL = kda_decode_step). */
int kda_decode_step_fused(const void *q, const void *k, const void *v, const float *log_alpha,
                          const float *beta, float *state, void *o, int N, int H, int dk, int dv,
                          int dtype, const kda_fusion *fusion, void *stream);

/*
 * The output epilogue on its own: for each of `rows` rows of dv values,
 * out = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate). o, gate and out have
 * dtype `dtype` and the same [rows, dv] layout; weight is float32 [dv]; out may
 * equal o (in place), gate must not alias out. dv = 128 only; rows = 0 is a no-op.
 */
int kda_output_norm_gate(const void *o, const void *gate, const float *weight, void *out, int64_t rows,
                         int dv, float eps, int dtype, void *stream);

/*
 * Backward of kda_chunk_fwd (the plain recurrence, no kda_fusion): the gradients of
 *
 *     L = sum over tokens of <o_t, grad_o_t> + sum over sequences of <final_state, grad_final_state>
 *
 * with respect to q, k, v, log_alpha, beta and initial_state. The pages present
 * the chunked WY / UT form as what makes KDA efficient to train ("From GPT-2 to
 * Kimi K3" digest, section "DeltaNet 병렬화 -- 청크 단위 학습"; GeekNews "Kimi Linear" summary,
 * section "청크 단위 병렬 알고리듬"). It recomputes the forward internally (16-token
 * chunks, keeping each chunk's entry state), runs the state gradient backwards
 * through the chunks, then forms every chunk's gradients in parallel.
 *
 *   q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, B, T, H, dk,
 *               dv, dtype: as kda_chunk_fwd (the inputs of the forward call).
 *   grad_o             [B, T, H, dv]  dtype, required when B*T > 0
 *   grad_final_state   [N, H, dk, dv] float32, or NULL for zeros
 *   grad_q, grad_k     [B, T, H, dk]  dtype (written)
 *   grad_v             [B, T, H, dv]  dtype (written)
 *   grad_log_alpha     [B, T, H, dk]  float32 (written)
 *   grad_beta          [B, T, H]      float32 (written)
 *   grad_initial_state [N, H, dk, dv] float32 (written), or NULL
 *   workspace          at least kda_chunk_bwd_workspace_size() bytes (256-byte
 *                      aligned), or NULL: allocated and freed in stream order. It
 *                      holds two 128 x 128 matrices in dtype per (16-token chunk,
 *                      head): 64 KiB (bf16) per 16 tokens and head.
 * Alignment: 16 bytes for every tensor except beta, grad_beta and cu_seqlens (4).
 * The written gradients must not alias any input. Returns KDA_OK,
 * KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED (dk or dv != 128, bad dtype),
 * KDA_ERR_WORKSPACE or KDA_ERR_DEVICE, with the same checks as kda_chunk_fwd.
 * T = 0 (or B = 0) writes grad_initial_state = grad_final_state (zeros if NULL).
 */
size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int num_seqs, int dtype);
int kda_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                  const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                  int num_seqs, const void *grad_o, const float *grad_final_state, void *grad_q,
                  void *grad_k, void *grad_v, float *grad_log_alpha, float *grad_beta,
                  float *grad_initial_state, int B, int T, int H, int dk, int dv, int dtype,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Chunked forward of the general diagonal-plus-low-rank (DPLR) recurrence, the
 * comparison point the GeekNews "Kimi Linear" summary measures KDA's chunk kernel
 * against (section "일반 DPLR보다 줄어든 연산량": KDA ties the DPLR transition's two
 * low-rank vectors to the key, which halves the secondary C x C matrices per chunk
 * and removes three matrix products). The pages do not write the general form out;
 * this is the rank-one reading, per sequence and head, token by token:
 *
 *     S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T ,   o_t = S_t^T q_t
 *
 * KDA is the case a_t = -beta_t k_t, b_t = alpha_t * k_t with written key beta_t k_t.
 *
 *   q, k, a, b   [B, T, H, dk]  dtype
 *   v, o         [B, T, H, dv]  dtype (o written)
 *   log_alpha    [B, T, H, dk]  float32, alpha_t = exp(log_alpha_t)
 *   initial_state, final_state, cu_seqlens, num_seqs, B, T, H, dk, dv, dtype,
 *   workspace, stream: as kda_chunk_fwd, with kda_dplr_chunk_fwd_workspace_size().
 *   chunk        64 only (KDA_ERR_UNSUPPORTED otherwise).
 * Alignment: 16 bytes for every tensor except cu_seqlens (4). o must not alias an
 * input; final_state may equal initial_state. Value preconditions (documented,
 * not checked): log_alpha finite and <= 0, and the transitions keep the state
 * finite. Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED,
 * KDA_ERR_WORKSPACE or KDA_ERR_DEVICE. Timing ids as kda_chunk_fwd (plan, intra,
 * inter).
 */
size_t kda_dplr_chunk_fwd_workspace_size(int B, int T, int H, int num_seqs, int dtype);
int kda_dplr_chunk_fwd(const void *q, const void *k, const void *v, const void *a, const void *b,
                       const float *log_alpha, const float *initial_state, const int32_t *cu_seqlens,
                       int num_seqs, void *o, float *final_state, int B, int T, int H, int dk, int dv,
                       int chunk, int dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Per-kernel timing, a tracing aid. While enabled, every kda_chunk_fwd, kda_chunk_bwd,
 * kda_dplr_chunk_fwd and kda_decode_step call records HIP events on its stream before its first kernel
 * and after each kernel it launches, so the durations are measured on the stream
 * the kernels run on (the fused variants and kda_output_norm_gate included). Kernel
 * ids: KDA_KERNEL_PLAN (chunk or segment plan), KDA_KERNEL_INTRA (intra-chunk),
 * KDA_KERNEL_INTER (inter-chunk state and output), KDA_KERNEL_DECODE,
 * KDA_KERNEL_OUTNORM (output RMSNorm and gate), for kda_chunk_bwd, whose internal
 * forward reports its plan and state pass under KDA_KERNEL_PLAN and KDA_KERNEL_INTER,
 * KDA_KERNEL_BWD_LOCAL (per-chunk records of both state passes), KDA_KERNEL_BWD_STATE
 * (state gradient through the chunks) and
 * KDA_KERNEL_BWD_CHUNK (per-chunk gradients), and for the segment-parallel prefill
 * KDA_KERNEL_SEG_FIRST (first segments' outputs and the middle segments' maps),
 * KDA_KERNEL_SEG_SCAN (segment entry states) and KDA_KERNEL_SEG_SECOND (the other
 * segments' outputs).
 *
 * kda_timing_enable(1) starts recording (and discards anything recorded before);
 * kda_timing_enable(0) stops. kda_timing_read() waits for the recorded events,
 * writes for each kernel id < n the total milliseconds and the launch count since
 * the last enable/read into total_ms[id] and launches[id] (either may be NULL),
 * and clears the record. Returns KDA_OK, KDA_ERR_INVALID_ARG for n < 0, or
 * KDA_ERR_DEVICE. Recording is process-wide and serialised by a lock; the events
 * cost a few microseconds per launch.
 */
#define KDA_KERNEL_PLAN 0
#define KDA_KERNEL_INTRA 1
#define KDA_KERNEL_INTER 2
#define KDA_KERNEL_DECODE 3
#define KDA_KERNEL_OUTNORM 4
#define KDA_KERNEL_BWD_LOCAL 5
#define KDA_KERNEL_BWD_STATE 6
#define KDA_KERNEL_BWD_CHUNK 7
#define KDA_KERNEL_SEG_FIRST 8
#define KDA_KERNEL_SEG_SCAN 9
#define KDA_KERNEL_SEG_SECOND 10
#define KDA_NUM_KERNELS 11

int kda_timing_enable(int on);
int kda_timing_read(double *total_ms, int *launches, int n);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
