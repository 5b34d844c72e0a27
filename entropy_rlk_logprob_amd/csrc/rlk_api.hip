// C-ABI host layer: argument validation, workspace sizing, device check, launches.
// Validation never touches the device and happens before anything is launched; there is
// no fallback route -- an unsupported case is an error.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "rlk_launch.hpp"
#include "rlk_logprob.h"
#include "rlk_state.hpp"

namespace {

static_assert(sizeof(rlk_row_state) == sizeof(rlk::WireState) &&
                  alignof(rlk_row_state) == alignof(rlk::WireState),
              "rlk_row_state is the wire state");

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

constexpr double kLog2e = 1.44269504088896340735992468100189214;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxVocab = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxVocabLinear = int64_t(1) << 26;
constexpr int64_t kMaxHidden = int64_t(1) << 20;
// Comparison: the block count (ceil(T / 4096)) stays a valid grid size.
constexpr int64_t kMaxCompareTokens = int64_t(1) << 40;
// Row strides of the fused path: 256 rows x stride stays within 32-bit tile offsets.
constexpr int64_t kMaxLdLinear = int64_t(1) << 22;

rlk_status check_device() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return RLK_ERR_UNSUPPORTED_DEVICE;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return RLK_ERR_UNSUPPORTED_DEVICE;
  if (dev >= kMaxDevices) return RLK_ERR_UNSUPPORTED_DEVICE;
  int st = g_device_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return RLK_ERR_UNSUPPORTED_DEVICE;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_ok[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? RLK_OK : RLK_ERR_UNSUPPORTED_DEVICE;
}

bool valid_splits(int32_t s) { return s == 1 || s == 2 || s == 4 || s == 8; }

bool valid_temperature(float t) { return std::isfinite(t) && t > 0.0f; }

size_t logits_ws_bytes(int64_t T, int32_t S) {
  return S > 1 ? (size_t)S * (size_t)T * sizeof(rlk::WireState) : 0;
}

// Backward workspace: the forward's shard states, then one root state per row.
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t backward_root_offset(int64_t T, int32_t S) { return align256(logits_ws_bytes(T, S)); }
size_t backward_ws_bytes(int64_t T, int32_t S) {
  return T == 0 ? 0 : backward_root_offset(T, S) + (size_t)T * sizeof(rlk::WireState);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shared validation of the logits-path calls.
rlk_status validate_logits(const void* logits, int64_t ld, int64_t T, int64_t V,
                           float temperature, int32_t S, void* ws, size_t ws_bytes) {
  if (T < 0 || T > kMaxRows || V < 1 || V > kMaxVocab || ld < V) return RLK_ERR_INVALID_ARGUMENT;
  if (T > 0 && !logits) return RLK_ERR_INVALID_ARGUMENT;
  if (!valid_temperature(temperature) || !valid_splits(S)) return RLK_ERR_INVALID_ARGUMENT;
  const size_t need = logits_ws_bytes(T, S);
  if (need > 0 && (!ws || !aligned(ws, 256))) {
    if (ws && !aligned(ws, 256)) return RLK_ERR_INVALID_ARGUMENT;
    return RLK_ERR_WORKSPACE_TOO_SMALL;
  }
  if (ws_bytes < need) return RLK_ERR_WORKSPACE_TOO_SMALL;
  return RLK_OK;
}

// logits_f32 or logits_bf16 (exactly one non-null) in the same [T, ld] row-major layout.
rlk_status run_logits(const float* logits_f32, const uint16_t* logits_bf16, int64_t ld, int64_t T,
                      int64_t V, const int64_t* targets, float temperature, int32_t S, float* lp,
                      float* ent, rlk_row_state* states, void* ws, void* stream) {
  rlk::LogitsArgs a;
  a.X = logits_f32;
  a.Xh = logits_bf16;
  a.ld = ld;
  a.T = T;
  a.V = V;
  a.Vc = rlk::chunk_cols(V);
  a.targets = targets;
  a.beta = 1.0 / (double)temperature;
  a.c = (float)(kLog2e / (double)temperature);
  a.S = S;
  a.vec = logits_f32 ? (aligned(logits_f32, 16) && ld % 4 == 0)
                     : (aligned(logits_bf16, 8) && ld % 4 == 0);
  a.lp = lp;
  a.ent = ent;
  a.ws = static_cast<rlk::WireState*>(ws);
  a.root = reinterpret_cast<rlk::WireState*>(states);
  const hipError_t e = rlk::launch_logits_path(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

// Shared validation of the fused forward calls (everything but the workspace); *need gets
// the workspace bytes the call needs.
rlk_status validate_linear(const uint16_t* hidden_bf16, int64_t ld_hidden,
                           const uint16_t* weight_bf16, int64_t ld_weight, int64_t n_tokens,
                           int64_t hidden_dim, int64_t vocab, const int64_t* target_ids,
                           float temperature, int32_t vocab_splits, const float* logprob_out,
                           const rlk_row_state* row_states_out, size_t* need) {
  *need = 0;
  if (n_tokens < 0 || n_tokens > kMaxRows || vocab < 1 || vocab > kMaxVocabLinear)
    return RLK_ERR_INVALID_ARGUMENT;
  if (hidden_dim < 64 || hidden_dim > kMaxHidden || hidden_dim % 64 != 0)
    return RLK_ERR_INVALID_ARGUMENT;
  if (ld_hidden < hidden_dim || ld_weight < hidden_dim || ld_hidden % 8 != 0 ||
      ld_weight % 8 != 0 || ld_hidden > kMaxLdLinear || ld_weight > kMaxLdLinear)
    return RLK_ERR_INVALID_ARGUMENT;
  if (!valid_temperature(temperature) || !valid_splits(vocab_splits))
    return RLK_ERR_INVALID_ARGUMENT;
  if (n_tokens == 0) return RLK_OK;
  if (!hidden_bf16 || !weight_bf16 || !target_ids || !logprob_out)
    return RLK_ERR_INVALID_ARGUMENT;
  if (row_states_out && !aligned(row_states_out, 8)) return RLK_ERR_INVALID_ARGUMENT;
  if (!aligned(hidden_bf16, 16) || !aligned(weight_bf16, 16)) return RLK_ERR_INVALID_ARGUMENT;
  *need = rlk::linear_workspace_layout(n_tokens, vocab, vocab_splits).total;
  return RLK_OK;
}

rlk_status run_linear(const uint16_t* hidden_bf16, int64_t ld_hidden, const uint16_t* weight_bf16,
                      int64_t ld_weight, int64_t n_tokens, int64_t hidden_dim, int64_t vocab,
                      const int64_t* target_ids, float temperature, int32_t vocab_splits,
                      float* logprob_out, float* entropy_out, rlk_row_state* row_states_out,
                      void* workspace, void* stream) {
  rlk::LinearArgs a;
  a.H = hidden_bf16;
  a.W = weight_bf16;
  a.ldh = ld_hidden;
  a.ldw = ld_weight;
  a.T = n_tokens;
  a.d = hidden_dim;
  a.V = vocab;
  a.Vc = rlk::chunk_cols(vocab);
  a.targets = target_ids;
  a.beta = 1.0 / (double)temperature;
  a.c = (float)(kLog2e / (double)temperature);
  a.S = vocab_splits;
  a.lp = logprob_out;
  a.ent = entropy_out;
  a.ws = workspace;
  a.root = reinterpret_cast<rlk::WireState*>(row_states_out);
  const hipError_t e = rlk::launch_linear_path(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

// Workspace of rlk_linear_logprob_noalloc: one static device array, which every GPU the
// library runs on holds (its own copy) until the process ends.  Host code never uses the
// array's name as an address (it is a host-side stand-in there): each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current.  The fused
// forward writes every byte of the workspace it reads, so nothing needs clearing between
// calls.
__device__ __align__(256) unsigned char scratch[RLK_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

rlk_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return RLK_ERR_UNSUPPORTED_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return RLK_ERR_HIP;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return RLK_OK;
}

}  // namespace

extern "C" {

size_t rlk_workspace_bytes(int op, int64_t n_tokens, int64_t vocab, int64_t hidden,
                           int32_t vocab_splits) {
  if (op == RLK_OP_COMPARE) {
    if (n_tokens < 0 || n_tokens > kMaxCompareTokens) return RLK_WORKSPACE_INVALID;
    return rlk::compare_workspace_bytes(n_tokens);
  }
  if (n_tokens < 0 || n_tokens > kMaxRows || vocab < 1 || !valid_splits(vocab_splits))
    return RLK_WORKSPACE_INVALID;
  switch (op) {
    case RLK_OP_FROM_LOGITS:
    case RLK_OP_ENTROPY:
      if (vocab > kMaxVocab) return RLK_WORKSPACE_INVALID;
      return logits_ws_bytes(n_tokens, vocab_splits);
    case RLK_OP_BACKWARD_FROM_LOGITS:
      if (vocab > kMaxVocab) return RLK_WORKSPACE_INVALID;
      return backward_ws_bytes(n_tokens, vocab_splits);
    case RLK_OP_LINEAR_BACKWARD:
      if (vocab > kMaxVocabLinear || hidden < 64 || hidden > kMaxHidden || hidden % 64 != 0)
        return RLK_WORKSPACE_INVALID;
      return n_tokens == 0
                 ? 0
                 : rlk::linear_backward_layout(n_tokens, vocab, hidden, vocab_splits).total;
    case RLK_OP_LINEAR:
      if (vocab > kMaxVocabLinear || hidden < 0) return RLK_WORKSPACE_INVALID;
      return n_tokens == 0 ? 0 : rlk::linear_workspace_layout(n_tokens, vocab, vocab_splits).total;
    default:
      return RLK_WORKSPACE_INVALID;
  }
}

rlk_status rlk_logprob_from_logits_with_states(const float* logits, int64_t ld_logits,
                                               int64_t n_tokens, int64_t vocab,
                                               const int64_t* target_ids, float temperature,
                                               int32_t vocab_splits, float* logprob_out,
                                               float* entropy_out,
                                               rlk_row_state* row_states_out, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  if (n_tokens > 0 && (!target_ids || !logprob_out)) return RLK_ERR_INVALID_ARGUMENT;
  if (row_states_out && !aligned(row_states_out, 8)) return RLK_ERR_INVALID_ARGUMENT;
  rlk_status s = validate_logits(logits, ld_logits, n_tokens, vocab, temperature, vocab_splits,
                                 workspace, workspace_bytes);
  if (s != RLK_OK) return s;
  if (n_tokens == 0) return RLK_OK;
  s = check_device();
  if (s != RLK_OK) return s;
  return run_logits(logits, nullptr, ld_logits, n_tokens, vocab, target_ids, temperature,
                    vocab_splits, logprob_out, entropy_out, row_states_out, workspace, stream);
}

rlk_status rlk_logprob_from_logits(const float* logits, int64_t ld_logits, int64_t n_tokens,
                                   int64_t vocab, const int64_t* target_ids, float temperature,
                                   int32_t vocab_splits, float* logprob_out, float* entropy_out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return rlk_logprob_from_logits_with_states(logits, ld_logits, n_tokens, vocab, target_ids,
                                             temperature, vocab_splits, logprob_out,
                                             entropy_out, nullptr, workspace, workspace_bytes,
                                             stream);
}

rlk_status rlk_logprob_from_logits_bf16(const uint16_t* logits, int64_t ld_logits,
                                        int64_t n_tokens, int64_t vocab,
                                        const int64_t* target_ids, float temperature,
                                        int32_t vocab_splits, float* logprob_out,
                                        float* entropy_out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (n_tokens > 0 && (!target_ids || !logprob_out)) return RLK_ERR_INVALID_ARGUMENT;
  rlk_status s = validate_logits(logits, ld_logits, n_tokens, vocab, temperature, vocab_splits,
                                 workspace, workspace_bytes);
  if (s != RLK_OK) return s;
  if (n_tokens == 0) return RLK_OK;
  s = check_device();
  if (s != RLK_OK) return s;
  return run_logits(nullptr, logits, ld_logits, n_tokens, vocab, target_ids, temperature,
                    vocab_splits, logprob_out, entropy_out, nullptr, workspace, stream);
}

rlk_status rlk_entropy_bf16(const uint16_t* logits, int64_t ld_logits, int64_t n_tokens,
                            int64_t vocab, float temperature, int32_t vocab_splits,
                            float* entropy_out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (n_tokens > 0 && !entropy_out) return RLK_ERR_INVALID_ARGUMENT;
  rlk_status s = validate_logits(logits, ld_logits, n_tokens, vocab, temperature, vocab_splits,
                                 workspace, workspace_bytes);
  if (s != RLK_OK) return s;
  if (n_tokens == 0) return RLK_OK;
  s = check_device();
  if (s != RLK_OK) return s;
  return run_logits(nullptr, logits, ld_logits, n_tokens, vocab, nullptr, temperature,
                    vocab_splits, nullptr, entropy_out, nullptr, workspace, stream);
}

rlk_status rlk_entropy(const float* logits, int64_t ld_logits, int64_t n_tokens, int64_t vocab,
                       float temperature, int32_t vocab_splits, float* entropy_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (n_tokens > 0 && !entropy_out) return RLK_ERR_INVALID_ARGUMENT;
  rlk_status s = validate_logits(logits, ld_logits, n_tokens, vocab, temperature, vocab_splits,
                                 workspace, workspace_bytes);
  if (s != RLK_OK) return s;
  if (n_tokens == 0) return RLK_OK;
  s = check_device();
  if (s != RLK_OK) return s;
  return run_logits(logits, nullptr, ld_logits, n_tokens, vocab, nullptr, temperature,
                    vocab_splits, nullptr, entropy_out, nullptr, workspace, stream);
}

rlk_status rlk_linear_logprob_with_states(const uint16_t* hidden_bf16, int64_t ld_hidden,
                                          const uint16_t* weight_bf16, int64_t ld_weight,
                                          int64_t n_tokens, int64_t hidden_dim, int64_t vocab,
                                          const int64_t* target_ids, float temperature,
                                          int32_t vocab_splits, float* logprob_out,
                                          float* entropy_out, rlk_row_state* row_states_out,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream) {
  size_t need = 0;
  rlk_status s = validate_linear(hidden_bf16, ld_hidden, weight_bf16, ld_weight, n_tokens,
                                 hidden_dim, vocab, target_ids, temperature, vocab_splits,
                                 logprob_out, row_states_out, &need);
  if (s != RLK_OK) return s;
  if (n_tokens == 0) return RLK_OK;
  if (workspace && !aligned(workspace, 256)) return RLK_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < need) return RLK_ERR_WORKSPACE_TOO_SMALL;
  s = check_device();
  if (s != RLK_OK) return s;
  return run_linear(hidden_bf16, ld_hidden, weight_bf16, ld_weight, n_tokens, hidden_dim, vocab,
                    target_ids, temperature, vocab_splits, logprob_out, entropy_out,
                    row_states_out, workspace, stream);
}

rlk_status rlk_linear_logprob(const uint16_t* hidden_bf16, int64_t ld_hidden,
                              const uint16_t* weight_bf16, int64_t ld_weight, int64_t n_tokens,
                              int64_t hidden_dim, int64_t vocab, const int64_t* target_ids,
                              float temperature, int32_t vocab_splits, float* logprob_out,
                              float* entropy_out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return rlk_linear_logprob_with_states(hidden_bf16, ld_hidden, weight_bf16, ld_weight, n_tokens,
                                        hidden_dim, vocab, target_ids, temperature, vocab_splits,
                                        logprob_out, entropy_out, nullptr, workspace,
                                        workspace_bytes, stream);
}

rlk_status rlk_linear_logprob_noalloc(const uint16_t* hidden_bf16, int64_t ld_hidden,
                                      const uint16_t* weight_bf16, int64_t ld_weight,
                                      int64_t n_tokens, int64_t hidden_dim, int64_t vocab,
                                      const int64_t* target_ids, float temperature,
                                      int32_t vocab_splits, float* logprob_out,
                                      float* entropy_out, void* stream) {
  size_t need = 0;
  rlk_status s = validate_linear(hidden_bf16, ld_hidden, weight_bf16, ld_weight, n_tokens,
                                 hidden_dim, vocab, target_ids, temperature, vocab_splits,
                                 logprob_out, nullptr, &need);
  if (s != RLK_OK) return s;
  if (n_tokens == 0) return RLK_OK;
  if (need > (size_t)RLK_NOALLOC_SCRATCH_BYTES) return RLK_ERR_WORKSPACE_TOO_SMALL;
  s = check_device();
  if (s != RLK_OK) return s;
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != RLK_OK) return s;
  return run_linear(hidden_bf16, ld_hidden, weight_bf16, ld_weight, n_tokens, hidden_dim, vocab,
                    target_ids, temperature, vocab_splits, logprob_out, entropy_out, nullptr, ws,
                    stream);
}

const char* rlk_status_string(rlk_status status) {
  switch (status) {
    case RLK_OK: return "ok";
    case RLK_ERR_INVALID_ARGUMENT: return "invalid argument";
    case RLK_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case RLK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RLK_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* rlk_backend_id(void) { return "rlk.logprob.strict.gfx950.v1"; }

rlk_status rlk_logprob_compare(const float* train_logprob, const float* rollout_logprob,
                               const uint8_t* active_mask, int64_t n_tokens,
                               rlk_compare_result* result, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (n_tokens < 0 || n_tokens > kMaxCompareTokens || !result || !aligned(result, 8))
    return RLK_ERR_INVALID_ARGUMENT;
  if (n_tokens > 0 && (!train_logprob || !rollout_logprob)) return RLK_ERR_INVALID_ARGUMENT;
  const size_t need = rlk::compare_workspace_bytes(n_tokens);
  if (need > 0) {
    if (!workspace) return RLK_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, 256)) return RLK_ERR_INVALID_ARGUMENT;
  }
  if (workspace_bytes < need) return RLK_ERR_WORKSPACE_TOO_SMALL;
  rlk_status s = check_device();
  if (s != RLK_OK) return s;
  const hipError_t e = rlk::launch_compare(train_logprob, rollout_logprob, active_mask, n_tokens,
                                           workspace, result, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

rlk_status rlk_logprob_backward_from_logits(const float* logits, int64_t ld_logits,
                                            int64_t n_tokens, int64_t vocab,
                                            const int64_t* target_ids, float temperature,
                                            int32_t vocab_splits, const float* grad_logprob,
                                            const float* grad_entropy,
                                            const rlk_row_state* row_states, float* grad_logits,
                                            int64_t ld_grad, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  if (n_tokens < 0 || n_tokens > kMaxRows || vocab < 1 || vocab > kMaxVocab || ld_logits < vocab ||
      ld_grad < vocab)
    return RLK_ERR_INVALID_ARGUMENT;
  if (n_tokens > 0 && (!logits || !grad_logits || (grad_logprob && !target_ids)))
    return RLK_ERR_INVALID_ARGUMENT;
  if (grad_logits == logits && ld_grad != ld_logits) return RLK_ERR_INVALID_ARGUMENT;
  if (row_states && !aligned(row_states, 8)) return RLK_ERR_INVALID_ARGUMENT;
  if (!valid_temperature(temperature) || !valid_splits(vocab_splits))
    return RLK_ERR_INVALID_ARGUMENT;
  const size_t need = backward_ws_bytes(n_tokens, vocab_splits);
  if (need > 0) {
    if (!workspace) return RLK_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, 256)) return RLK_ERR_INVALID_ARGUMENT;
  }
  if (workspace_bytes < need) return RLK_ERR_WORKSPACE_TOO_SMALL;
  if (n_tokens == 0) return RLK_OK;
  rlk_status s = check_device();
  if (s != RLK_OK) return s;
  rlk::LogitsArgs a;
  a.X = logits;
  a.Xh = nullptr;
  a.ld = ld_logits;
  a.T = n_tokens;
  a.V = vocab;
  a.Vc = rlk::chunk_cols(vocab);
  a.targets = target_ids;
  a.beta = 1.0 / (double)temperature;
  a.c = (float)(kLog2e / (double)temperature);
  a.S = vocab_splits;
  a.vec = aligned(logits, 16) && ld_logits % 4 == 0;
  a.lp = nullptr;
  a.ent = nullptr;
  char* ws = static_cast<char*>(workspace);
  a.ws = reinterpret_cast<rlk::WireState*>(ws);
  a.root = row_states ? reinterpret_cast<rlk::WireState*>(const_cast<rlk_row_state*>(row_states))
                      : reinterpret_cast<rlk::WireState*>(ws + backward_root_offset(n_tokens,
                                                                                   vocab_splits));
  const bool vec = a.vec && aligned(grad_logits, 16) && ld_grad % 4 == 0;
  const hipError_t e =
      rlk::launch_logits_backward(a, grad_logprob, grad_entropy, grad_logits, ld_grad, vec,
                                  row_states != nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

rlk_status rlk_linear_logprob_backward(const uint16_t* hidden_bf16, int64_t ld_hidden,
                                       const uint16_t* weight_bf16, int64_t ld_weight,
                                       int64_t n_tokens, int64_t hidden_dim, int64_t vocab,
                                       const int64_t* target_ids, float temperature,
                                       int32_t vocab_splits, const float* grad_logprob,
                                       const float* grad_entropy,
                                       const rlk_row_state* row_states, float* grad_hidden,
                                       int64_t ld_grad_hidden, float* grad_weight,
                                       int64_t ld_grad_weight, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (n_tokens < 0 || n_tokens > kMaxRows || vocab < 1 || vocab > kMaxVocabLinear)
    return RLK_ERR_INVALID_ARGUMENT;
  if (hidden_dim < 64 || hidden_dim > kMaxHidden || hidden_dim % 64 != 0)
    return RLK_ERR_INVALID_ARGUMENT;
  if (ld_hidden < hidden_dim || ld_weight < hidden_dim || ld_hidden % 8 != 0 ||
      ld_weight % 8 != 0 || ld_hidden > kMaxLdLinear || ld_weight > kMaxLdLinear)
    return RLK_ERR_INVALID_ARGUMENT;
  if ((grad_hidden && ld_grad_hidden < hidden_dim) || (grad_weight && ld_grad_weight < hidden_dim))
    return RLK_ERR_INVALID_ARGUMENT;
  if (!valid_temperature(temperature) || !valid_splits(vocab_splits))
    return RLK_ERR_INVALID_ARGUMENT;
  if (n_tokens > 0) {
    if (!hidden_bf16 || !weight_bf16 || (grad_logprob && !target_ids))
      return RLK_ERR_INVALID_ARGUMENT;
    if (row_states && !aligned(row_states, 8)) return RLK_ERR_INVALID_ARGUMENT;
    if (!aligned(hidden_bf16, 16) || !aligned(weight_bf16, 16)) return RLK_ERR_INVALID_ARGUMENT;
    const size_t need =
        rlk::linear_backward_layout(n_tokens, vocab, hidden_dim, vocab_splits).total;
    if (workspace && !aligned(workspace, 256)) return RLK_ERR_INVALID_ARGUMENT;
    if (!workspace || workspace_bytes < need) return RLK_ERR_WORKSPACE_TOO_SMALL;
  }
  if (!grad_hidden && !grad_weight) return RLK_OK;
  rlk_status s = check_device();
  if (s != RLK_OK) return s;
  if (n_tokens == 0) {
    // The gradient of an empty sum: grad_weight is all zeros (grad_hidden has no rows).
    if (!grad_weight) return RLK_OK;
    const hipError_t e = rlk::launch_zero_f32(grad_weight, ld_grad_weight, vocab, hidden_dim,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RLK_OK : RLK_ERR_HIP;
  }
  rlk::LinearArgs a;
  a.H = hidden_bf16;
  a.W = weight_bf16;
  a.ldh = ld_hidden;
  a.ldw = ld_weight;
  a.T = n_tokens;
  a.d = hidden_dim;
  a.V = vocab;
  a.Vc = rlk::chunk_cols(vocab);
  a.targets = target_ids;
  a.beta = 1.0 / (double)temperature;
  a.c = (float)(kLog2e / (double)temperature);
  a.S = vocab_splits;
  a.lp = nullptr;
  a.ent = nullptr;
  a.ws = workspace;
  a.root = nullptr;
  const hipError_t e =
      rlk::launch_linear_backward(a, grad_logprob, grad_entropy, grad_hidden, ld_grad_hidden,
                                  grad_weight, ld_grad_weight,
                                  reinterpret_cast<const rlk::WireState*>(row_states),
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

}  // extern "C"
