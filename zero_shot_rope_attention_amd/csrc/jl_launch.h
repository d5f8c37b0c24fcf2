// Host-side launch interface between the C ABI (jl_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jl {

// kModeBifocal corrects the keys tile by tile inside the attention kernel;
// kModeBifocalPre first writes the corrected keys of the whole cache to a
// workspace (one elementwise pass) and stages them like plain keys.
enum PrefillMode : int { kModePlain = 0, kModeBifocal = 1, kModePasses = 2, kModeBifocalPre = 3, kModeSliding = 4 };

// Everything a prefill launch needs; validated by the caller.
struct PrefillProblem {
  const void* q;
  const void* k;
  const void* v;
  void* out;        // bf16 [B, n_q, Hq, D]       (plain / bifocal)
  float* lse;       // fp32 [B, Hq, n_q] or null  (plain / bifocal)
  float* out_abc;   // fp32 [3, B, n_q, Hq, D]    (passes)
  float* lse_abc;   // fp32 [3, B, Hq, n_q]       (passes)
  void* kg;         // bf16 [B, n_kv, Hkv, D] corrected keys (bifocal, precorrected)
  int32_t batch, n_q, n_kv, n_q_heads, n_kv_heads;
  int32_t group;         // g(s); 1 for plain
  int32_t local_window;  // W, already clamped to <= n_kv
  double rope_base;
  float softmax_scale;   // > 0
};

hipError_t launch_prefill(PrefillMode mode, const PrefillProblem& p, hipStream_t stream);

struct DecodeProblem {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* seq_lens;   // device [B] keys per sequence, or null: every sequence holds n_kv keys
  int32_t batch, n_kv, n_q_heads, n_kv_heads;  // n_kv: cache positions per sequence
  int64_t pretrained_window;  // L (bifocal); g(s) is taken per sequence in the kernels
  int32_t local_window;       // W (clamped to each sequence's length in the kernels)
  double rope_base;
  float softmax_scale;
  void* workspace;
  bool sliding = false;  // plain attention over the newest min(W, s) keys only (bifocal must be false)
};

// Number of key chunks the decode splits a cache of n_kv keys into (upper bound
// over every local window), and the workspace bytes that many chunks need.
int32_t decode_max_splits(int32_t batch, int32_t n_kv, int32_t n_kv_heads);
size_t decode_workspace_bytes(int32_t batch, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads);

hipError_t launch_decode(bool bifocal, const DecodeProblem& p, hipStream_t stream);

}  // namespace jl
