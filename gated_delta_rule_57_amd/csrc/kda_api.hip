// C ABI of libkda.so (declared in include/kda.h): argument validation on the
// host, workspace handling and dispatch to the kernel launchers. Every check runs
// before the first HIP call, so every error path can be exercised without a GPU.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>
#include <vector>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return KDA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shared checks of the prefill arguments; returns KDA_OK or a status with the
// reason recorded.
int check_prefill(int B, int T, int H, int num_seqs, bool varlen, int dk, int dv, int chunk, int dtype) {
  if (dtype != KDA_BF16 && dtype != KDA_FP32) return fail(KDA_ERR_UNSUPPORTED, "dtype %d is not KDA_BF16 or KDA_FP32", dtype);
  if (dk != 128 || dv != 128) return fail(KDA_ERR_UNSUPPORTED, "dk=%d dv=%d: only 128 is supported", dk, dv);
  if (chunk != 16 && chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk=%d: only 16 and 64 are supported", chunk);
  if (B < 0 || T < 0) return fail(KDA_ERR_INVALID_ARG, "B=%d T=%d must be >= 0", B, T);
  if (H <= 0) return fail(KDA_ERR_INVALID_ARG, "H=%d must be > 0", H);
  if (varlen) {
    if (B != 1) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens requires B == 1 (got B=%d)", B);
    if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs=%d must be >= 0", num_seqs);
    if (num_seqs == 0 && T > 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs=0 with T=%d tokens", T);
  }
  // token indices are int32 on the device; element offsets are 64-bit
  if ((int64_t)B * T > (int64_t)INT32_MAX - 64) return fail(KDA_ERR_INVALID_ARG, "B*T=%lld is too large", (long long)B * T);
  if ((int64_t)(varlen ? num_seqs : B) * H > (int64_t)INT32_MAX / 64)
    return fail(KDA_ERR_INVALID_ARG, "too many (sequence, head) pairs");
  // the intra-chunk kernel runs one work-group per (chunk, head) on a 1-D grid
  if (kda::max_chunks(B, T, num_seqs, varlen, chunk) * H > (int64_t)INT32_MAX)
    return fail(KDA_ERR_INVALID_ARG, "too many (chunk, head) pairs");
  return KDA_OK;
}

// ---- per-kernel timing (tracing aid) ------------------------------------------
struct TraceRec {
  hipStream_t stream;
  int kernel;  // -1: start of a call
  hipEvent_t ev;
};
std::mutex g_trace_mu;
bool g_trace_on = false;
std::vector<TraceRec> g_trace;
std::vector<hipEvent_t> g_event_pool;

void trace_record(hipStream_t s, int kernel) {
  std::lock_guard<std::mutex> lock(g_trace_mu);
  if (!g_trace_on) return;
  hipEvent_t ev;
  if (!g_event_pool.empty()) {
    ev = g_event_pool.back();
    g_event_pool.pop_back();
  } else if (hipEventCreate(&ev) != hipSuccess) {
    return;
  }
  if (hipEventRecord(ev, s) != hipSuccess) {
    g_event_pool.push_back(ev);
    return;
  }
  g_trace.push_back({s, kernel, ev});
}

void trace_clear_locked() {
  for (auto& r : g_trace) g_event_pool.push_back(r.ev);
  g_trace.clear();
}

}  // namespace

namespace kda {
void trace_begin(hipStream_t stream) { trace_record(stream, -1); }
void trace_mark(hipStream_t stream, int kernel_id) { trace_record(stream, kernel_id); }
}  // namespace kda

extern "C" {

int kda_timing_enable(int on) {
  std::lock_guard<std::mutex> lock(g_trace_mu);
  trace_clear_locked();
  g_trace_on = on != 0;
  return ok();
}

int kda_timing_read(double* total_ms, int* launches, int n) {
  if (n < 0) return fail(KDA_ERR_INVALID_ARG, "n=%d must be >= 0", n);
  std::lock_guard<std::mutex> lock(g_trace_mu);
  for (int i = 0; i < n; ++i) {
    if (total_ms) total_ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  int status = KDA_OK;
  if (!g_trace.empty()) {
    hipError_t e = hipEventSynchronize(g_trace.back().ev);
    for (size_t i = 0; e == hipSuccess && i < g_trace.size(); ++i) e = hipEventSynchronize(g_trace[i].ev);
    if (e != hipSuccess) {
      status = fail(KDA_ERR_DEVICE, "hipEventSynchronize: %s", hipGetErrorString(e));
    } else {
      for (size_t i = 0; i < g_trace.size(); ++i) {
        const TraceRec& r = g_trace[i];
        if (r.kernel < 0) continue;
        // the previous event recorded on the same stream opens this kernel's interval
        for (size_t j = i; j-- > 0;) {
          if (g_trace[j].stream != r.stream) continue;
          float ms = 0.f;
          if (hipEventElapsedTime(&ms, g_trace[j].ev, r.ev) == hipSuccess && r.kernel < n) {
            if (total_ms) total_ms[r.kernel] += ms;
            if (launches) launches[r.kernel] += 1;
          }
          break;
        }
      }
    }
  }
  trace_clear_locked();
  return status == KDA_OK ? ok() : status;
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: unsupported configuration";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace too small";
    case KDA_ERR_DEVICE: return "KDA_ERR_DEVICE: HIP runtime error";
    default: return "unknown kda status";
  }
}

const char* kda_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {
int check_fusion(const kda_fusion* f) {
  if (!f) return KDA_OK;
  if (!(f->qk_eps >= 0.f) || !(f->norm_eps >= 0.f))
    return fail(KDA_ERR_INVALID_ARG, "qk_eps and norm_eps must be >= 0");
  if (f->gate_kind < KDA_GATE_CHANNEL || f->gate_kind > KDA_GATE_NONE)
    return fail(KDA_ERR_INVALID_ARG, "gate_kind %d is not a kda_gate", f->gate_kind);
  if (f->prefill_path < KDA_PATH_AUTO || f->prefill_path > KDA_PATH_RECORD_SEGMENTED)
    return fail(KDA_ERR_INVALID_ARG, "prefill_path %d is not a kda_prefill_path", f->prefill_path);
  if (f->out_gate) {
    if (!f->norm_weight) return fail(KDA_ERR_INVALID_ARG, "out_gate needs norm_weight");
    if (!aligned(f->out_gate, 16) || !aligned(f->norm_weight, 16))
      return fail(KDA_ERR_INVALID_ARG, "out_gate and norm_weight must be 16-byte aligned");
  }
  return KDA_OK;
}

kda::Fusion to_internal(const kda_fusion* f) {
  kda::Fusion u{};
  if (f) {
    u.normalize_qk = f->normalize_qk != 0;
    u.qk_eps = f->qk_eps;
    u.gate_preactivation = f->gate_preactivation != 0;
    u.beta_preactivation = f->beta_preactivation != 0;
    u.out_gate = f->out_gate;
    u.norm_weight = f->out_gate ? f->norm_weight : nullptr;
    u.norm_eps = f->norm_eps;
    u.gate_kind = f->gate_kind;
    u.prefill_path = f->prefill_path;
  }
  return u;
}
}  // namespace

extern "C" {

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int num_seqs, int chunk, int dtype) {
  // Without cu_seqlens, num_seqs is ignored; with it the caller passes B = 1.
  const bool varlen = num_seqs > 0 && B == 1;
  if (check_prefill(B, T, H, varlen ? num_seqs : 0, varlen, 128, 128, chunk, dtype) != KDA_OK) return 0;
  return kda::prefill_workspace_bytes(B, T, H, num_seqs, varlen, chunk, dtype, KDA_PATH_AUTO);
}

size_t kda_chunk_fwd_fused_workspace_size(int B, int T, int H, int num_seqs, int chunk, int dtype,
                                          const kda_fusion* fusion) {
  const bool varlen = num_seqs > 0 && B == 1;
  if (check_prefill(B, T, H, varlen ? num_seqs : 0, varlen, 128, 128, chunk, dtype) != KDA_OK) return 0;
  if (check_fusion(fusion) != KDA_OK) return 0;
  return kda::prefill_workspace_bytes(B, T, H, num_seqs, varlen, chunk, dtype,
                                      fusion ? fusion->prefill_path : KDA_PATH_AUTO);
}


}  // extern "C"

namespace {
// The prefill behind kda_chunk_fwd, kda_chunk_fwd_fused and kda_chunk_fwd_noalloc.
// With `scratch` set (and workspace NULL) the kernels use that buffer of
// `scratch_bytes` and nothing is allocated; a configuration that needs more returns
// KDA_ERR_WORKSPACE before any HIP call. `get_scratch` is then called once the
// arguments are checked and returns the current device's buffer.
int prefill_impl(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                 const float* initial_state, const int32_t* cu_seqlens, int num_seqs, void* o, float* final_state,
                 int B, int T, int H, int dk, int dv, int chunk, int dtype, const kda_fusion* fusion, void* workspace,
                 size_t workspace_bytes, int (*get_scratch)(void**), size_t scratch_bytes, void* stream) {
  const bool varlen = cu_seqlens != nullptr;
  int st = check_prefill(B, T, H, num_seqs, varlen, dk, dv, chunk, dtype);
  if (st != KDA_OK) return st;
  st = check_fusion(fusion);
  if (st != KDA_OK) return st;
  const int gate = fusion ? fusion->gate_kind : KDA_GATE_CHANNEL;
  const int64_t tokens = (int64_t)B * T;
  if (tokens > 0) {
    if (!q || !k || !v || !beta || !o || (!log_alpha && gate != KDA_GATE_NONE))
      return fail(KDA_ERR_INVALID_ARG, "q, k, v, log_alpha (unless gate_kind is KDA_GATE_NONE), beta and o must be "
                                       "non-null when B*T > 0");
  }
  const void* ptrs[] = {q, k, v, o, initial_state, final_state};
  const char* names[] = {"q", "k", "v", "o", "initial_state", "final_state"};
  for (int i = 0; i < 6; ++i)
    if (ptrs[i] && !aligned(ptrs[i], 16)) return fail(KDA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  if (gate != KDA_GATE_NONE && log_alpha && !aligned(log_alpha, gate == KDA_GATE_HEAD ? 4 : 16))
    return fail(KDA_ERR_INVALID_ARG, "log_alpha is not %d-byte aligned", gate == KDA_GATE_HEAD ? 4 : 16);
  if (beta && !aligned(beta, 4)) return fail(KDA_ERR_INVALID_ARG, "beta is not 4-byte aligned");
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens is not 4-byte aligned");
  if (workspace && !aligned(workspace, 256)) return fail(KDA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const int N = varlen ? num_seqs : B;
  if (N == 0) return ok();
  const int path = fusion ? fusion->prefill_path : KDA_PATH_AUTO;
  const size_t need = kda::prefill_workspace_bytes(B, T, H, num_seqs, varlen, chunk, dtype, path);
  if (workspace && workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if (get_scratch && need > scratch_bytes)
    return fail(KDA_ERR_WORKSPACE, "this prefill needs %zu bytes of scratch; the static scratch holds %zu", need,
                scratch_bytes);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = workspace;
  bool allocated = false;
  if (!ws && get_scratch) {
    const int st2 = get_scratch(&ws);
    if (st2 != KDA_OK) return st2;
  } else if (!ws) {
    hipError_t e = hipMallocAsync(&ws, need, s);
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "hipMallocAsync(%zu): %s", need, hipGetErrorString(e));
    allocated = true;
  }
  hipError_t e = kda::launch_prefill(dtype, chunk, q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, o,
                                     final_state, B, T, H, to_internal(fusion), ws, s);
  if (allocated) {
    hipError_t e2 = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

// Scratch of kda_chunk_fwd_noalloc. Each GPU the library runs on holds its own copy
// until the process ends. In host code the array's name is only a host-side stand-in:
// host code uses the per-device address from hipGetSymbolAddress, never the name.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// The current device's address of `scratch`, looked up once per device (with that
// device current) and kept.
int current_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(KDA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                SCRATCH_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KDA_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}
}  // namespace

extern "C" {

int kda_chunk_fwd_fused(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                        const float* initial_state, const int32_t* cu_seqlens, int num_seqs, void* o,
                        float* final_state, int B, int T, int H, int dk, int dv, int chunk, int dtype,
                        const kda_fusion* fusion, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, o, final_state, B, T, H, dk, dv,
                      chunk, dtype, fusion, workspace, workspace_bytes, nullptr, 0, stream);
}

int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                          const float* initial_state, const int32_t* cu_seqlens, int num_seqs, void* o,
                          float* final_state, int B, int T, int H, int dk, int dv, int chunk, int dtype, void* stream) {
  kda_fusion f{};
  f.gate_kind = KDA_GATE_CHANNEL;
  f.prefill_path = (dtype == KDA_BF16 && chunk == 64) ? KDA_PATH_SINGLE_PASS : KDA_PATH_AUTO;
  return prefill_impl(q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, o, final_state, B, T, H, dk, dv,
                      chunk, dtype, &f, nullptr, 0, current_scratch, KDA_NOALLOC_SCRATCH_BYTES, stream);
}

size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int num_seqs, int dtype) {
  const bool varlen = num_seqs > 0 && B == 1;
  if (check_prefill(B, T, H, varlen ? num_seqs : 0, varlen, 128, 128, kda::BWD_CHUNK, dtype) != KDA_OK) return 0;
  return kda::backward_workspace_bytes(B, T, H, num_seqs, varlen, dtype);
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int num_seqs, const void* grad_o,
                  const float* grad_final_state, void* grad_q, void* grad_k, void* grad_v, float* grad_log_alpha,
                  float* grad_beta, float* grad_initial_state, int B, int T, int H, int dk, int dv, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const bool varlen = cu_seqlens != nullptr;
  int st = check_prefill(B, T, H, num_seqs, varlen, dk, dv, kda::BWD_CHUNK, dtype);
  if (st != KDA_OK) return st;
  const int64_t tokens = (int64_t)B * T;
  if (tokens > 0) {
    if (!q || !k || !v || !log_alpha || !beta || !grad_o || !grad_q || !grad_k || !grad_v || !grad_log_alpha ||
        !grad_beta)
      return fail(KDA_ERR_INVALID_ARG, "q, k, v, log_alpha, beta, grad_o and the five token gradients must be "
                                       "non-null when B*T > 0");
  }
  const void* ptrs[] = {q, k, v, log_alpha, grad_o, grad_q, grad_k, grad_v, grad_log_alpha, initial_state,
                        grad_final_state, grad_initial_state};
  const char* names[] = {"q", "k", "v", "log_alpha", "grad_o", "grad_q", "grad_k", "grad_v", "grad_log_alpha",
                         "initial_state", "grad_final_state", "grad_initial_state"};
  for (int i = 0; i < 12; ++i)
    if (ptrs[i] && !aligned(ptrs[i], 16)) return fail(KDA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  if (beta && !aligned(beta, 4)) return fail(KDA_ERR_INVALID_ARG, "beta is not 4-byte aligned");
  if (grad_beta && !aligned(grad_beta, 4)) return fail(KDA_ERR_INVALID_ARG, "grad_beta is not 4-byte aligned");
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens is not 4-byte aligned");
  if (workspace && !aligned(workspace, 256)) return fail(KDA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const int N = varlen ? num_seqs : B;
  if (N == 0) return ok();
  const size_t need = kda::backward_workspace_bytes(B, T, H, num_seqs, varlen, dtype);
  if (workspace && workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = workspace;
  if (!ws) {
    hipError_t e = hipMallocAsync(&ws, need, s);
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "hipMallocAsync(%zu): %s", need, hipGetErrorString(e));
  }
  hipError_t e = kda::launch_backward(dtype, q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, grad_o,
                                      grad_final_state, grad_q, grad_k, grad_v, grad_log_alpha, grad_beta,
                                      grad_initial_state, B, T, H, ws, s);
  if (!workspace) {
    hipError_t e2 = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "backward launch: %s", hipGetErrorString(e));
  return ok();
}

size_t kda_dplr_chunk_fwd_workspace_size(int B, int T, int H, int num_seqs, int dtype) {
  const bool varlen = num_seqs > 0 && B == 1;
  if (check_prefill(B, T, H, varlen ? num_seqs : 0, varlen, 128, 128, 64, dtype) != KDA_OK) return 0;
  return kda::dplr_workspace_bytes(B, T, H, num_seqs, varlen, dtype);
}

int kda_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const void* b,
                       const float* log_alpha, const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                       void* o, float* final_state, int B, int T, int H, int dk, int dv, int chunk, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const bool varlen = cu_seqlens != nullptr;
  if (chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk=%d: the DPLR forward supports 64 only", chunk);
  int st = check_prefill(B, T, H, num_seqs, varlen, dk, dv, chunk, dtype);
  if (st != KDA_OK) return st;
  const int64_t tokens = (int64_t)B * T;
  if (tokens > 0 && (!q || !k || !v || !a || !b || !log_alpha || !o))
    return fail(KDA_ERR_INVALID_ARG, "q, k, v, a, b, log_alpha and o must be non-null when B*T > 0");
  const void* ptrs[] = {q, k, v, a, b, log_alpha, o, initial_state, final_state};
  const char* names[] = {"q", "k", "v", "a", "b", "log_alpha", "o", "initial_state", "final_state"};
  for (int i = 0; i < 9; ++i)
    if (ptrs[i] && !aligned(ptrs[i], 16)) return fail(KDA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens is not 4-byte aligned");
  if (workspace && !aligned(workspace, 256)) return fail(KDA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const int N = varlen ? num_seqs : B;
  if (N == 0) return ok();
  const size_t need = kda::dplr_workspace_bytes(B, T, H, num_seqs, varlen, dtype);
  if (workspace && workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = workspace;
  if (!ws) {
    hipError_t e = hipMallocAsync(&ws, need, s);
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "hipMallocAsync(%zu): %s", need, hipGetErrorString(e));
  }
  hipError_t e = kda::launch_dplr(dtype, q, k, v, a, b, log_alpha, initial_state, cu_seqlens, num_seqs, o,
                                  final_state, B, T, H, ws, s);
  if (!workspace) {
    hipError_t e2 = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "DPLR launch: %s", hipGetErrorString(e));
  return ok();
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int num_seqs, void* o,
                  float* final_state, int B, int T, int H, int dk, int dv, int chunk, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return kda_chunk_fwd_fused(q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs, o, final_state, B, T, H,
                             dk, dv, chunk, dtype, nullptr, workspace, workspace_bytes, stream);
}

int kda_decode_step_fused(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                          float* state, void* o, int N, int H, int dk, int dv, int dtype, const kda_fusion* fusion,
                          void* stream) {
  if (dtype != KDA_BF16 && dtype != KDA_FP32) return fail(KDA_ERR_UNSUPPORTED, "dtype %d is not KDA_BF16 or KDA_FP32", dtype);
  if (dk != 128 || dv != 128) return fail(KDA_ERR_UNSUPPORTED, "dk=%d dv=%d: only 128 is supported", dk, dv);
  if (N < 0) return fail(KDA_ERR_INVALID_ARG, "N=%d must be >= 0", N);
  if (H <= 0) return fail(KDA_ERR_INVALID_ARG, "H=%d must be > 0", H);
  if ((int64_t)N * H > (int64_t)INT32_MAX) return fail(KDA_ERR_INVALID_ARG, "N*H is too large");
  int st = check_fusion(fusion);
  if (st != KDA_OK) return st;
  if (N == 0) return ok();
  const int gate = fusion ? fusion->gate_kind : KDA_GATE_CHANNEL;
  const void* ptrs[] = {q, k, v, log_alpha, beta, state, o};
  const char* names[] = {"q", "k", "v", "log_alpha", "beta", "state", "o"};
  for (int i = 0; i < 7; ++i) {
    const bool is_gate = i == 3;
    if (is_gate && gate == KDA_GATE_NONE) continue;
    if (!ptrs[i]) return fail(KDA_ERR_INVALID_ARG, "%s must be non-null", names[i]);
    const size_t need = (i == 4 || (is_gate && gate == KDA_GATE_HEAD)) ? 4 : 16;
    if (!aligned(ptrs[i], need)) return fail(KDA_ERR_INVALID_ARG, "%s is not %zu-byte aligned", names[i], need);
  }
  hipError_t e = kda::launch_decode(dtype, q, k, v, log_alpha, beta, state, o, N, H, to_internal(fusion),
                                    reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

int kda_decode_step(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                    float* state, void* o, int N, int H, int dk, int dv, int dtype, void* stream) {
  return kda_decode_step_fused(q, k, v, log_alpha, beta, state, o, N, H, dk, dv, dtype, nullptr, stream);
}

int kda_output_norm_gate(const void* o, const void* gate, const float* weight, void* out, int64_t rows, int dv,
                         float eps, int dtype, void* stream) {
  if (dtype != KDA_BF16 && dtype != KDA_FP32) return fail(KDA_ERR_UNSUPPORTED, "dtype %d is not KDA_BF16 or KDA_FP32", dtype);
  if (dv != 128) return fail(KDA_ERR_UNSUPPORTED, "dv=%d: only 128 is supported", dv);
  if (rows < 0) return fail(KDA_ERR_INVALID_ARG, "rows=%lld must be >= 0", (long long)rows);
  if (rows > ((int64_t)1 << 34)) return fail(KDA_ERR_INVALID_ARG, "rows=%lld is too large", (long long)rows);
  if (!(eps >= 0.f)) return fail(KDA_ERR_INVALID_ARG, "eps must be >= 0");
  if (rows == 0) return ok();
  const void* ptrs[] = {o, gate, weight, out};
  const char* names[] = {"o", "gate", "weight", "out"};
  for (int i = 0; i < 4; ++i) {
    if (!ptrs[i]) return fail(KDA_ERR_INVALID_ARG, "%s must be non-null", names[i]);
    if (!aligned(ptrs[i], 16)) return fail(KDA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  if (gate == out) return fail(KDA_ERR_INVALID_ARG, "gate must not alias out");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  kda::trace_begin(s);
  hipError_t e = kda::launch_output_norm_gate(dtype, o, gate, weight, out, rows, eps, s);
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "output norm launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
