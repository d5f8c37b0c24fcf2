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

// Long-range schedules: where a remote query at p and a remote key at j are
// moved before their score is taken (positions a_q(p), a_k(j)).
//  kSchedGrouped:    a_q(p) = floor(p/g), a_k(j) = floor(j/g), g the smallest
//                    integer with floor((s-1)/g) <= L-1.
//  kSchedSeam:       a_q(p) = floor(p/g) + W - floor(W/g), a_k(j) = floor(j/g):
//                    remote distances continue the local ones at the seam; g the
//                    smallest integer keeping every shifted distance <= L-1.
//  kSchedFractional: a_q(p) = p/l, a_k(j) = j/l, l = max(1, (s-1)/(L-1)).
// The kernels see every schedule as integer grouping: a group factor g, a query
// shift, and a rate multiplying theta.  The fractional schedule is g = 2^30
// (floor(p/g) = 0 for every position, so c(p) = -p) with rate 1 - 1/l: the
// correction rot(x_p, -p (1 - 1/l) theta) moves x_p from p to p/l.
enum Schedule : int32_t { kSchedGrouped = 0, kSchedSeam = 1, kSchedFractional = 2 };
constexpr int32_t kFracGroup = 1 << 30;  // positions must stay below it

// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1 (which overflows
// int32 for a near 2^31).
__host__ __device__ inline int32_t ceil_div(int32_t a, int32_t b) { return a > 0 ? (a - 1) / b + 1 : 0; }

// Group factor of a sequence of s >= 1 keys (1: the base model, no remote key
// is moved).  Seam needs w < big_l whenever s > big_l.
__host__ __device__ inline int32_t sched_group(int32_t s, int64_t big_l, int32_t w, int32_t sched) {
  if ((int64_t)s <= big_l) return 1;
  const int32_t l32 = (int32_t)big_l;  // big_l < s here
  if (sched == kSchedFractional) return kFracGroup;
  if (sched != kSchedSeam) return (s - 1) / l32 + 1;
  // smallest g with floor((s-1)/g) - floor(w/g) <= r, r = L-1-w.  Since
  // floor(D/g) <= floor((s-1)/g) - floor(w/g) <= floor(D/g) + 1 with D = s-1-w,
  // no g <= D/(r+1) qualifies, and g = D/r + 1 (r >= 1) or g = s (r = 0) does:
  // the search starts at the lower bound and takes few steps unless r is small.
  const int32_t d = s - 1 - w, r = l32 - 1 - w;
  if (d < 0) return 1;
  int32_t g = d / (r + 1) + 1;
  while (g < s && (s - 1) / g - w / g > r) ++g;  // g = s always qualifies when r >= 0
  return g;
}

__host__ __device__ inline int32_t sched_q_shift(int32_t g, int32_t w, int32_t sched) {
  return (sched == kSchedSeam && g > 1) ? w - w / g : 0;
}

// Factor on theta for the corrections: 1 - 1/l = (s - L)/(s - 1) for the
// fractional schedule at s > L, else 1.
__host__ __device__ inline double sched_rate(int32_t s, int64_t big_l, int32_t sched) {
  if (sched != kSchedFractional || (int64_t)s <= big_l) return 1.0;
  return (double)((int64_t)s - big_l) / (double)(s - 1);
}

// Everything a prefill launch needs; validated by the caller.
struct PrefillProblem {
  const void* q;
  const void* k;
  const void* v;
  void* out;        // bf16 [B, n_q, Hq, D]       (plain / bifocal)
  float* lse;       // fp32 [B, Hq, n_q] or null  (plain / bifocal)
  float* out_abc;   // fp32 [3, B, n_q, Hq, D]    (passes; null: out/lse take the merged result)
  float* lse_abc;   // fp32 [3, B, Hq, n_q]       (passes)
  void* kg;         // bf16 [B, n_kv, Hkv, D] corrected keys (bifocal, precorrected)
  int32_t batch, n_q, n_kv, n_q_heads, n_kv_heads;
  int32_t group;         // g(s); 1 for plain
  int32_t local_window;  // W, already clamped to <= n_kv
  double rope_base;
  float softmax_scale;   // > 0
  int32_t q_shift = 0;   // added to c(p) of the queries (seam schedule)
  double rate = 1.0;     // factor on theta for the corrections (fractional schedule)
  // Variable-length batches (plain and precorrected bifocal modes only): q, out
  // packed [total_q, Hq, D] with sequence b's rows cu_q[b] .. cu_q[b+1]-1 (device
  // [B+1]); kv_lens (device [B]) keys per sequence in caches of n_kv rows; lse
  // [Hq, total_q]; n_q the longest query count.  g, the shift and the rate are then
  // taken per sequence in the kernels from the fields below (group, q_shift and
  // rate are not used).
  const int32_t* cu_q = nullptr;
  const int32_t* kv_lens = nullptr;
  int32_t total_q = 0;
  int32_t schedule = kSchedGrouped;
  int64_t pretrained_window = 1;
  // Explicit query positions (plain and precorrected bifocal modes, uniform
  // batches): device int32 [n_q], nondecreasing, in [0, n_kv); null: n_kv - n_q + i.
  const int32_t* q_pos = nullptr;
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
  int32_t schedule = kSchedGrouped;  // long-range schedule, taken per sequence in the kernels
  // Paged cache: k and v are pools [n_pages, page_size, Hkv, D]; position j of
  // sequence b in page block_table[b * pages_per_seq + j / page_size] (device);
  // page_size a power of two >= 32, n_kv = pages_per_seq * page_size, seq_lens set.
  const int32_t* block_table = nullptr;
  int32_t pages_per_seq = 0, page_size = 0, n_pages = 0;
};

// Number of key chunks the decode splits a cache of n_kv keys into (upper bound
// over every local window), and the workspace bytes that many chunks need.
int32_t decode_max_splits(int32_t batch, int32_t n_kv, int32_t n_kv_heads);
size_t decode_workspace_bytes(int32_t batch, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads);

hipError_t launch_decode(bool bifocal, const DecodeProblem& p, hipStream_t stream);

// The allocation-free decode's workspace: a device array of this many bytes per
// GPU (its address on the current device in *ptr).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

// Per-head RMSNorm of the query and key heads, RoPE at the tokens' positions
// n_kv - n_new + i, and the append of keys and values to the caches.
struct NormRopeProblem {
  const void* qkv;      // bf16 [B * n_new, (Hq + 2 Hkv) D]: query heads, then key heads, then value heads
  const void* gamma_q;  // bf16 [D]
  const void* gamma_k;  // bf16 [D]
  void* q;              // bf16 [B * n_new, Hq, D]  normalised, rotated queries
  void* k_cache;        // bf16 [B, n_kv, Hkv, D]   rows n_kv - n_new .. n_kv - 1 written
  void* v_cache;        // bf16 [B, n_kv, Hkv, D]
  int32_t batch, n_new, n_kv, n_q_heads, n_kv_heads;
  float eps;
  double rope_base;
};
hipError_t launch_norm_rope(const NormRopeProblem& p, hipStream_t stream);

// Row-major y[m, n] = x[m, k] w[n, k]^T in bf16 with fp32 accumulation: the
// library's weight-streaming kernel for up to 8 rows, rocBLAS otherwise, whose
// scratch is gemm_ws (kGemmWorkspaceBytes of device memory from the caller).
constexpr size_t kGemmWorkspaceBytes = size_t(32) << 20;
hipError_t launch_gemm_xwt(const void* x, const void* w, void* y, int64_t m, int64_t n, int64_t k,
                           void* gemm_ws, size_t gemm_ws_bytes, hipStream_t stream);

}  // namespace jl
