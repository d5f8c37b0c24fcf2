// C ABI of the bifocal-attention library: argument validation, g(s), launch
// planning and error reporting.  Declarations and contracts: include/jl_bifocal.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "jl_bifocal.h"
#include "jl_launch.h"

namespace {

thread_local char g_err[512] = "";

jl_status fail(jl_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

jl_status ok() {
  g_err[0] = '\0';
  return JL_OK;
}

constexpr int32_t kMaxKvHeads = 65536;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Elements of a [b, n, h, 128] tensor, or -1 on int64 overflow.
int64_t elements(int64_t b, int64_t n, int64_t h) {
  const int64_t lim = INT64_C(1) << 55;
  if (b > lim / n) return -1;
  int64_t x = b * n;
  if (x > lim / h) return -1;
  x *= h;
  if (x > lim / 128) return -1;
  return x * 128;
}

// One query of the HIP runtime per process: is there a usable device?
jl_status device_check() {
  static std::atomic<int> state{-1};  // -1 unknown, 0 none, 1 present (callers may race to fill it)
  int st = state.load(std::memory_order_relaxed);
  if (st < 0) {
    int count = 0;
    st = (hipGetDeviceCount(&count) == hipSuccess && count > 0) ? 1 : 0;
    state.store(st, std::memory_order_relaxed);
  }
  if (st == 0) return fail(JL_ERR_DEVICE, "no HIP device available");
  return JL_OK;
}

jl_status check_pointer(const void* p, const char* name, bool nullable = false) {
  if (!p) return nullable ? JL_OK : fail(JL_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(JL_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return JL_OK;
}

struct Shape {
  int32_t batch, n_q, n_kv, hq, hkv, head_dim;
};

jl_status check_shape(const Shape& s) {
  if (s.batch < 1 || s.n_q < 1 || s.n_kv < 1 || s.hq < 1 || s.hkv < 1 || s.head_dim < 1)
    return fail(JL_ERR_INVALID_ARG, "sizes must be >= 1 (batch=%d n_q=%d n_kv=%d Hq=%d Hkv=%d D=%d)", s.batch,
                s.n_q, s.n_kv, s.hq, s.hkv, s.head_dim);
  if (s.n_q > s.n_kv) return fail(JL_ERR_INVALID_ARG, "n_q (%d) > n_kv (%d)", s.n_q, s.n_kv);
  if (s.hq % s.hkv) return fail(JL_ERR_INVALID_ARG, "n_q_heads (%d) %% n_kv_heads (%d) != 0", s.hq, s.hkv);
  if (s.head_dim != 128) return fail(JL_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", s.head_dim);
  // 64 key rows of one head stride must stay within a 32-bit buffer range
  if (s.hkv > kMaxKvHeads)
    return fail(JL_ERR_UNSUPPORTED, "n_kv_heads %d unsupported (at most %d)", s.hkv, kMaxKvHeads);
  if (elements(s.batch, s.n_q, s.hq) < 0 || elements(s.batch, s.n_kv, s.hkv) < 0)
    return fail(JL_ERR_UNSUPPORTED, "tensor sizes overflow 64-bit element offsets");
  return JL_OK;
}

jl_status check_windows(int64_t big_l, int64_t w, double base) {
  if (big_l < 1) return fail(JL_ERR_INVALID_ARG, "pretrained_window must be >= 1 (got %lld)", (long long)big_l);
  if (w < 1) return fail(JL_ERR_INVALID_ARG, "local_window must be >= 1 (got %lld)", (long long)w);
  if (w > big_l)
    return fail(JL_ERR_INVALID_ARG, "local_window (%lld) > pretrained_window (%lld)", (long long)w,
                (long long)big_l);
  if (!(base > 1.0) || !std::isfinite(base)) return fail(JL_ERR_INVALID_ARG, "rope_base must be finite and > 1");
  return JL_OK;
}

jl_status check_scale(float scale, float* out) {
  if (std::isnan(scale) || std::isinf(scale)) return fail(JL_ERR_INVALID_ARG, "softmax_scale is not finite");
  *out = scale > 0.0f ? scale : 1.0f / std::sqrt(128.0f);
  return JL_OK;
}

jl_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(JL_ERR_DEVICE, "HIP launch error: %s", hipGetErrorString(e));
  return ok();
}

#define JL_TRY(expr)                \
  do {                              \
    jl_status st_ = (expr);         \
    if (st_ != JL_OK) return st_;   \
  } while (0)

jl_status prefill_common(const void* q, const void* k, const void* v, const Shape& s, float scale_in,
                         float* scale) {
  JL_TRY(check_pointer(q, "q"));
  JL_TRY(check_pointer(k, "k"));
  JL_TRY(check_pointer(v, "v"));
  JL_TRY(check_shape(s));
  JL_TRY(check_scale(scale_in, scale));
  return JL_OK;
}

}  // namespace

extern "C" {

const char* jl_last_error(void) { return g_err; }

int64_t jl_group_factor(int64_t seq_len, int64_t pretrained_window) {
  if (seq_len < 1 || pretrained_window < 1) return 0;
  // smallest g with (s - 1) / g <= L - 1  <=>  s <= g L  <=>  g = ceil(s / L)
  const int64_t g = seq_len / pretrained_window + (seq_len % pretrained_window != 0);
  return g < 1 ? 1 : g;
}

// Explicit query positions: NULL (the newest rows) or a 4-byte-aligned device array.
static jl_status check_positions(const int32_t* q_pos, bool nullable) {
  if (!q_pos) return nullable ? JL_OK : fail(JL_ERR_INVALID_ARG, "q_pos is NULL");
  if (reinterpret_cast<uintptr_t>(q_pos) % 4 != 0) return fail(JL_ERR_INVALID_ARG, "q_pos is not 4-byte aligned");
  return JL_OK;
}

jl_status jl_plain_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int32_t* q_pos, int32_t batch, int32_t n_q, int32_t n_kv, int32_t n_q_heads,
                           int32_t n_kv_heads, int32_t head_dim, float softmax_scale, void* stream) {
  float scale;
  const Shape s{batch, n_q, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(prefill_common(q, k, v, s, softmax_scale, &scale));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_positions(q_pos, true));
  JL_TRY(device_check());
  jl::PrefillProblem p{q, k, v, out, lse, nullptr, nullptr, nullptr, batch, n_q, n_kv, n_q_heads, n_kv_heads, 1, 1,
                       2.0, scale};
  p.q_pos = q_pos;
  return launched(jl::launch_prefill(jl::kModePlain, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_sliding_prefill(const void* q, const void* k, const void* v, void* out, float* lse, int32_t batch,
                             int32_t n_q, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                             int64_t local_window, float softmax_scale, void* stream) {
  float scale;
  const Shape s{batch, n_q, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(prefill_common(q, k, v, s, softmax_scale, &scale));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  if (local_window < 1) return fail(JL_ERR_INVALID_ARG, "local_window must be >= 1 (got %lld)", (long long)local_window);
  JL_TRY(device_check());
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  jl::PrefillProblem p{q, k, v, out, lse, nullptr, nullptr, nullptr, batch, n_q, n_kv, n_q_heads, n_kv_heads, 1, w,
                       2.0, scale};
  return launched(jl::launch_prefill(jl::kModeSliding, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_bifocal_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                             const int32_t* q_pos, int32_t batch, int32_t n_q, int32_t n_kv, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window, int64_t local_window,
                             double rope_base, float softmax_scale, void* stream) {
  float scale;
  const Shape s{batch, n_q, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(prefill_common(q, k, v, s, softmax_scale, &scale));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_positions(q_pos, true));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(device_check());
  const int64_t g = jl_group_factor(n_kv, pretrained_window);
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  const jl::PrefillMode mode = g == 1 ? jl::kModePlain : jl::kModeBifocal;
  jl::PrefillProblem p{q, k, v, out, lse, nullptr, nullptr, nullptr, batch, n_q, n_kv, n_q_heads, n_kv_heads,
                       (int32_t)g, w, rope_base, scale};
  p.q_pos = q_pos;
  return launched(jl::launch_prefill(mode, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_bifocal_prefill_passes(const void* q, const void* k, const void* v, float* out_abc, float* lse_abc,
                                    int32_t batch, int32_t n_q, int32_t n_kv, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                    int64_t local_window, double rope_base, float softmax_scale, void* stream) {
  float scale;
  const Shape s{batch, n_q, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(prefill_common(q, k, v, s, softmax_scale, &scale));
  JL_TRY(check_pointer(out_abc, "out_abc"));
  JL_TRY(check_pointer(lse_abc, "lse_abc"));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(device_check());
  const int64_t g = jl_group_factor(n_kv, pretrained_window);
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  jl::PrefillProblem p{q, k, v, nullptr, nullptr, out_abc, lse_abc, nullptr, batch, n_q, n_kv, n_q_heads,
                       n_kv_heads, (int32_t)g, w, rope_base, scale};
  return launched(jl::launch_prefill(jl::kModePasses, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_bifocal_prefill_three_pass(const void* q, const void* k, const void* v, void* out, float* lse,
                                        int32_t batch, int32_t n_q, int32_t n_kv, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                        int64_t local_window, double rope_base, float softmax_scale, void* stream) {
  float scale;
  const Shape s{batch, n_q, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(prefill_common(q, k, v, s, softmax_scale, &scale));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(device_check());
  const int64_t g = jl_group_factor(n_kv, pretrained_window);
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  // no per-pass buffers: the passes kernel writes the merged output and lse
  jl::PrefillProblem p{q, k, v, out, lse, nullptr, nullptr, nullptr, batch, n_q, n_kv, n_q_heads, n_kv_heads,
                       (int32_t)g, w, rope_base, scale};
  return launched(jl::launch_prefill(jl::kModePasses, p, static_cast<hipStream_t>(stream)));
}

size_t jl_bifocal_prefill_workspace_size(int32_t batch, int32_t n_kv, int32_t n_kv_heads, int32_t head_dim) {
  if (batch < 1 || n_kv < 1 || n_kv_heads < 1 || head_dim != 128) return 0;
  const int64_t e = elements(batch, n_kv, n_kv_heads);
  if (e < 0) return 0;
  return (size_t)e * 2;
}

jl_status jl_bifocal_prefill_ws(const void* q, const void* k, const void* v, void* out, float* lse, int32_t batch,
                                int32_t n_q, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                int64_t pretrained_window, int64_t local_window, double rope_base,
                                float softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
  float scale;
  const Shape s{batch, n_q, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(prefill_common(q, k, v, s, softmax_scale, &scale));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  const int64_t g = jl_group_factor(n_kv, pretrained_window);
  if (g > 1) {
    JL_TRY(check_pointer(workspace, "workspace"));
    const size_t need = jl_bifocal_prefill_workspace_size(batch, n_kv, n_kv_heads, head_dim);
    if (workspace_bytes < need)
      return fail(JL_ERR_WORKSPACE, "workspace_bytes %zu < required %zu", workspace_bytes, need);
  }
  JL_TRY(device_check());
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  const jl::PrefillMode mode = g == 1 ? jl::kModePlain : jl::kModeBifocalPre;
  jl::PrefillProblem p{q, k, v, out, lse, nullptr, nullptr, g == 1 ? nullptr : workspace, batch, n_q, n_kv,
                       n_q_heads, n_kv_heads, (int32_t)g, w, rope_base, scale};
  return launched(jl::launch_prefill(mode, p, static_cast<hipStream_t>(stream)));
}

size_t jl_bifocal_decode_workspace_size(int32_t batch, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t head_dim) {
  if (batch < 1 || n_kv < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim != 128) return 0;
  return jl::decode_workspace_bytes(batch, n_kv, n_q_heads, n_kv_heads);
}

static jl_status decode_common(const void* q, const void* k, const void* v, void* out, float* lse, const Shape& s,
                               float scale_in, float* scale, void* workspace, size_t workspace_bytes) {
  JL_TRY(check_pointer(q, "q"));
  JL_TRY(check_pointer(k, "k_cache"));
  JL_TRY(check_pointer(v, "v_cache"));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_shape(s));
  if (s.hq / s.hkv > 16)
    return fail(JL_ERR_UNSUPPORTED, "decode supports at most 16 query heads per KV head (got %d)", s.hq / s.hkv);
  JL_TRY(check_scale(scale_in, scale));
  JL_TRY(check_pointer(workspace, "workspace"));
  const size_t need = jl::decode_workspace_bytes(s.batch, s.n_kv, s.hq, s.hkv);
  if (workspace_bytes < need)
    return fail(JL_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes,
                need);
  return JL_OK;
}

jl_status jl_plain_decode(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                          int32_t batch, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                          float softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
  float scale;
  const Shape s{batch, 1, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(decode_common(q, k_cache, v_cache, out, lse, s, softmax_scale, &scale, workspace, workspace_bytes));
  JL_TRY(device_check());
  jl::DecodeProblem p{q, k_cache, v_cache, out, lse, nullptr, batch, n_kv, n_q_heads, n_kv_heads, 1, 0, 2.0, scale,
                      workspace};
  return launched(jl::launch_decode(false, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_bifocal_decode(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                            int32_t batch, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            int64_t pretrained_window, int64_t local_window, double rope_base, float softmax_scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
  float scale;
  const Shape s{batch, 1, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(decode_common(q, k_cache, v_cache, out, lse, s, softmax_scale, &scale, workspace, workspace_bytes));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(device_check());
  const int64_t g = jl_group_factor(n_kv, pretrained_window);
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  jl::DecodeProblem p{q, k_cache, v_cache, out, lse, nullptr, batch, n_kv, n_q_heads, n_kv_heads, pretrained_window,
                      w, rope_base, scale, workspace};
  return launched(jl::launch_decode(g > 1, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                    int32_t batch, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, int64_t pretrained_window, int64_t local_window,
                                    double rope_base, float softmax_scale, void* stream) {
  float scale;
  const Shape s{batch, 1, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(check_pointer(q, "q"));
  JL_TRY(check_pointer(k_cache, "k_cache"));
  JL_TRY(check_pointer(v_cache, "v_cache"));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_shape(s));
  if (s.hq / s.hkv > 16)
    return fail(JL_ERR_UNSUPPORTED, "decode supports at most 16 query heads per KV head (got %d)", s.hq / s.hkv);
  JL_TRY(check_scale(softmax_scale, &scale));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  const size_t need = jl::decode_workspace_bytes(batch, n_kv, n_q_heads, n_kv_heads);
  if (need > jl::kDecodeScratchBytes)
    return fail(JL_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of decode workspace, more than the %zu the allocation-free entry point "
                "holds; use jl_bifocal_decode with a workspace",
                need, jl::kDecodeScratchBytes);
  JL_TRY(device_check());
  void* ws = nullptr;
  const hipError_t e = jl::decode_scratch(&ws);
  if (e != hipSuccess) return fail(JL_ERR_DEVICE, "device workspace address: %s", hipGetErrorString(e));
  const int64_t g = jl_group_factor(n_kv, pretrained_window);
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  jl::DecodeProblem p{q, k_cache, v_cache, out, lse, nullptr, batch, n_kv, n_q_heads, n_kv_heads, pretrained_window,
                      w, rope_base, scale, ws};
  return launched(jl::launch_decode(g > 1, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_sliding_decode(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                            int32_t batch, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            int64_t local_window, float softmax_scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
  float scale;
  const Shape s{batch, 1, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(decode_common(q, k_cache, v_cache, out, lse, s, softmax_scale, &scale, workspace, workspace_bytes));
  if (local_window < 1) return fail(JL_ERR_INVALID_ARG, "local_window must be >= 1 (got %lld)", (long long)local_window);
  JL_TRY(device_check());
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  jl::DecodeProblem p{q, k_cache, v_cache, out, lse, nullptr, batch, n_kv, n_q_heads, n_kv_heads, 1, w, 2.0, scale,
                      workspace};
  p.sliding = true;
  return launched(jl::launch_decode(false, p, static_cast<hipStream_t>(stream)));
}

static jl_status check_seq_lens(const int32_t* seq_lens) {
  if (!seq_lens) return fail(JL_ERR_INVALID_ARG, "seq_lens is NULL");
  if (reinterpret_cast<uintptr_t>(seq_lens) % 4 != 0) return fail(JL_ERR_INVALID_ARG, "seq_lens is not 4-byte aligned");
  return JL_OK;
}

jl_status jl_plain_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                 const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim, float softmax_scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  float scale;
  const Shape s{batch, 1, max_seq_len, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(decode_common(q, k_cache, v_cache, out, lse, s, softmax_scale, &scale, workspace, workspace_bytes));
  JL_TRY(check_seq_lens(seq_lens));
  JL_TRY(device_check());
  jl::DecodeProblem p{q, k_cache, v_cache, out, lse, seq_lens, batch, max_seq_len, n_q_heads, n_kv_heads, 1, 0, 2.0,
                      scale, workspace};
  return launched(jl::launch_decode(false, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_bifocal_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                   const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                   int64_t local_window, double rope_base, float softmax_scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  float scale;
  const Shape s{batch, 1, max_seq_len, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(decode_common(q, k_cache, v_cache, out, lse, s, softmax_scale, &scale, workspace, workspace_bytes));
  JL_TRY(check_seq_lens(seq_lens));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(device_check());
  // g(s_b) is taken per sequence in the kernels; a sequence with g = 1 is computed as plain attention
  const int32_t w = (int32_t)(local_window < max_seq_len ? local_window : max_seq_len);
  jl::DecodeProblem p{q, k_cache, v_cache, out, lse, seq_lens, batch, max_seq_len, n_q_heads, n_kv_heads,
                      pretrained_window, w, rope_base, scale, workspace};
  return launched(jl::launch_decode(true, p, static_cast<hipStream_t>(stream)));
}

static_assert(JL_SCHED_GROUPED == jl::kSchedGrouped && JL_SCHED_SEAM == jl::kSchedSeam &&
                  JL_SCHED_FRACTIONAL == jl::kSchedFractional,
              "schedule numbers of the C ABI and the kernels");

static jl_status check_schedule(int32_t schedule, int64_t big_l, int64_t w, int64_t n_kv) {
  if (schedule == jl::kSchedGrouped) return JL_OK;
  if (schedule == jl::kSchedSeam) {
    if (w >= big_l)
      return fail(JL_ERR_INVALID_ARG, "the seam-shifted schedule needs local_window (%lld) < pretrained_window (%lld)",
                  (long long)w, (long long)big_l);
    return JL_OK;
  }
  if (schedule == jl::kSchedFractional) {
    if (big_l < 2) return fail(JL_ERR_INVALID_ARG, "the fractional schedule needs pretrained_window >= 2");
    if (n_kv >= jl::kFracGroup)
      return fail(JL_ERR_UNSUPPORTED, "the fractional schedule supports at most %d keys", jl::kFracGroup - 1);
    return JL_OK;
  }
  return fail(JL_ERR_INVALID_ARG, "unknown schedule %d", (int)schedule);
}

double jl_schedule_factor(int64_t seq_len, int64_t pretrained_window, int64_t local_window, int32_t schedule) {
  if (seq_len < 1 || seq_len > 0x7fffffff || pretrained_window < 1 || local_window < 1 ||
      local_window > pretrained_window)
    return 0.0;
  if (check_schedule(schedule, pretrained_window, local_window, seq_len) != JL_OK) return 0.0;
  if (schedule == jl::kSchedFractional)
    return seq_len <= pretrained_window ? 1.0 : (double)(seq_len - 1) / (double)(pretrained_window - 1);
  const int32_t w = (int32_t)(local_window < seq_len ? local_window : seq_len);
  return (double)jl::sched_group((int32_t)seq_len, pretrained_window, w, schedule);
}

jl_status jl_bifocal_prefill_sched(const void* q, const void* k, const void* v, void* out, float* lse, int32_t batch,
                                   int32_t n_q, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int64_t pretrained_window, int64_t local_window,
                                   double rope_base, int32_t schedule, float softmax_scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  float scale;
  const Shape s{batch, n_q, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(prefill_common(q, k, v, s, softmax_scale, &scale));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(check_schedule(schedule, pretrained_window, local_window, n_kv));
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  const int32_t g = jl::sched_group(n_kv, pretrained_window, w, schedule);
  // a workspace selects the two-launch form (corrected keys written first); none, the single kernel
  const bool two_launch = workspace != nullptr || workspace_bytes != 0;
  if (g > 1 && two_launch) {
    JL_TRY(check_pointer(workspace, "workspace"));
    const size_t need = jl_bifocal_prefill_workspace_size(batch, n_kv, n_kv_heads, head_dim);
    if (workspace_bytes < need)
      return fail(JL_ERR_WORKSPACE, "workspace_bytes %zu < required %zu", workspace_bytes, need);
  }
  JL_TRY(device_check());
  const jl::PrefillMode mode = g == 1 ? jl::kModePlain : (two_launch ? jl::kModeBifocalPre : jl::kModeBifocal);
  jl::PrefillProblem p{q, k, v, out, lse, nullptr, nullptr, mode == jl::kModeBifocalPre ? workspace : nullptr, batch,
                       n_q, n_kv, n_q_heads, n_kv_heads, g, w, rope_base, scale};
  p.q_shift = jl::sched_q_shift(g, w, schedule);
  p.rate = jl::sched_rate(n_kv, pretrained_window, schedule);
  return launched(jl::launch_prefill(mode, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_bifocal_decode_sched(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                  const int32_t* seq_lens, int32_t batch, int32_t n_kv, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                  int64_t local_window, double rope_base, int32_t schedule, float softmax_scale,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  float scale;
  const Shape s{batch, 1, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(decode_common(q, k_cache, v_cache, out, lse, s, softmax_scale, &scale, workspace, workspace_bytes));
  if (seq_lens) JL_TRY(check_seq_lens(seq_lens));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(check_schedule(schedule, pretrained_window, local_window, n_kv));
  JL_TRY(device_check());
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  // uniform lengths with g = 1 run the plain kernel; otherwise g, the shift and the
  // rate are taken per sequence in the kernels
  const bool bif = seq_lens != nullptr || jl::sched_group(n_kv, pretrained_window, w, schedule) > 1;
  jl::DecodeProblem p{q, k_cache, v_cache, out, lse, seq_lens, batch, n_kv, n_q_heads, n_kv_heads, pretrained_window,
                      w, rope_base, scale, workspace};
  p.schedule = schedule;
  return launched(jl::launch_decode(bif, p, static_cast<hipStream_t>(stream)));
}

static jl_status prefill_varlen_common(const void* q, const void* k, const void* v, void* out,
                                       const int32_t* cu_seqlens_q, const int32_t* seq_lens, int32_t batch,
                                       int32_t total_q, int32_t max_q, int32_t max_seq_len, int32_t hq, int32_t hkv,
                                       int32_t head_dim, float scale_in, float* scale) {
  JL_TRY(check_pointer(q, "q"));
  JL_TRY(check_pointer(k, "k_cache"));
  JL_TRY(check_pointer(v, "v_cache"));
  JL_TRY(check_pointer(out, "out"));
  if (!cu_seqlens_q || reinterpret_cast<uintptr_t>(cu_seqlens_q) % 4 != 0)
    return fail(JL_ERR_INVALID_ARG, "cu_seqlens_q is NULL or not 4-byte aligned");
  JL_TRY(check_seq_lens(seq_lens));
  if (total_q < 1) return fail(JL_ERR_INVALID_ARG, "total_q must be >= 1 (got %d)", total_q);
  const Shape s{batch, max_q, max_seq_len, hq, hkv, head_dim};
  JL_TRY(check_shape(s));
  if (elements(total_q, 1, hq) < 0) return fail(JL_ERR_UNSUPPORTED, "tensor sizes overflow 64-bit element offsets");
  JL_TRY(check_scale(scale_in, scale));
  return JL_OK;
}

jl_status jl_bifocal_prefill_varlen(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* seq_lens, int32_t batch,
                                    int32_t total_q, int32_t max_q, int32_t max_seq_len, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                    int64_t local_window, double rope_base, int32_t schedule, float softmax_scale,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  float scale;
  JL_TRY(prefill_varlen_common(q, k_cache, v_cache, out, cu_seqlens_q, seq_lens, batch, total_q, max_q, max_seq_len,
                               n_q_heads, n_kv_heads, head_dim, softmax_scale, &scale));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(check_schedule(schedule, pretrained_window, local_window, max_seq_len));
  // a workspace selects the two-launch form (corrected keys written first); none, the single kernel
  const bool two_launch = workspace != nullptr || workspace_bytes != 0;
  if (two_launch) {
    JL_TRY(check_pointer(workspace, "workspace"));
    const size_t need = jl_bifocal_prefill_workspace_size(batch, max_seq_len, n_kv_heads, head_dim);
    if (workspace_bytes < need)
      return fail(JL_ERR_WORKSPACE, "workspace_bytes %zu < required %zu", workspace_bytes, need);
  }
  JL_TRY(device_check());
  // the factor, the shift and the rate are taken per sequence in the kernels
  const int32_t w = (int32_t)(local_window < max_seq_len ? local_window : max_seq_len);
  jl::PrefillProblem p{q, k_cache, v_cache, out, lse, nullptr, nullptr, two_launch ? workspace : nullptr, batch,
                       max_q, max_seq_len, n_q_heads, n_kv_heads, 1, w, rope_base, scale};
  p.cu_q = cu_seqlens_q;
  p.kv_lens = seq_lens;
  p.total_q = total_q;
  p.schedule = schedule;
  p.pretrained_window = pretrained_window;
  return launched(
      jl::launch_prefill(two_launch ? jl::kModeBifocalPre : jl::kModeBifocal, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_plain_prefill_varlen(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                  const int32_t* cu_seqlens_q, const int32_t* seq_lens, int32_t batch,
                                  int32_t total_q, int32_t max_q, int32_t max_seq_len, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, float softmax_scale, void* stream) {
  float scale;
  JL_TRY(prefill_varlen_common(q, k_cache, v_cache, out, cu_seqlens_q, seq_lens, batch, total_q, max_q, max_seq_len,
                               n_q_heads, n_kv_heads, head_dim, softmax_scale, &scale));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(device_check());
  jl::PrefillProblem p{q, k_cache, v_cache, out, lse, nullptr, nullptr, nullptr, batch, max_q, max_seq_len,
                       n_q_heads, n_kv_heads, 1, 1, 2.0, scale};
  p.cu_q = cu_seqlens_q;
  p.kv_lens = seq_lens;
  p.total_q = total_q;
  return launched(jl::launch_prefill(jl::kModePlain, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_bifocal_prefill_positions(const void* q, const void* k, const void* v, void* out, float* lse,
                                       const int32_t* q_pos, int32_t batch, int32_t n_q, int32_t n_kv,
                                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                       int64_t pretrained_window, int64_t local_window, double rope_base,
                                       int32_t schedule, float softmax_scale, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  float scale;
  const Shape s{batch, n_q, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(prefill_common(q, k, v, s, softmax_scale, &scale));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_positions(q_pos, false));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(check_schedule(schedule, pretrained_window, local_window, n_kv));
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  const int32_t g = jl::sched_group(n_kv, pretrained_window, w, schedule);
  // a workspace selects the two-launch form (corrected keys written first); none, the single kernel
  const bool two_launch = workspace != nullptr || workspace_bytes != 0;
  if (g > 1 && two_launch) {
    JL_TRY(check_pointer(workspace, "workspace"));
    const size_t need = jl_bifocal_prefill_workspace_size(batch, n_kv, n_kv_heads, head_dim);
    if (workspace_bytes < need)
      return fail(JL_ERR_WORKSPACE, "workspace_bytes %zu < required %zu", workspace_bytes, need);
  }
  JL_TRY(device_check());
  const jl::PrefillMode mode = g == 1 ? jl::kModePlain : (two_launch ? jl::kModeBifocalPre : jl::kModeBifocal);
  jl::PrefillProblem p{q, k, v, out, lse, nullptr, nullptr, mode == jl::kModeBifocalPre ? workspace : nullptr, batch,
                       n_q, n_kv, n_q_heads, n_kv_heads, g, w, rope_base, scale};
  p.q_shift = jl::sched_q_shift(g, w, schedule);
  p.rate = jl::sched_rate(n_kv, pretrained_window, schedule);
  p.q_pos = q_pos;
  return launched(jl::launch_prefill(mode, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_plain_prefill_positions(const void* q, const void* k, const void* v, void* out, float* lse,
                                     const int32_t* q_pos, int32_t batch, int32_t n_q, int32_t n_kv,
                                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float softmax_scale,
                                     void* stream) {
  float scale;
  const Shape s{batch, n_q, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(prefill_common(q, k, v, s, softmax_scale, &scale));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(lse, "lse", true));
  JL_TRY(check_positions(q_pos, false));
  JL_TRY(device_check());
  jl::PrefillProblem p{q, k, v, out, lse, nullptr, nullptr, nullptr, batch, n_q, n_kv, n_q_heads, n_kv_heads, 1, 1,
                       2.0, scale};
  p.q_pos = q_pos;
  return launched(jl::launch_prefill(jl::kModePlain, p, static_cast<hipStream_t>(stream)));
}

static jl_status paged_common(const int32_t* block_table, const int32_t* seq_lens, int32_t n_pages,
                              int32_t page_size, int32_t pages_per_seq, int32_t n_kv_heads, int32_t* n_kv) {
  if (!block_table || reinterpret_cast<uintptr_t>(block_table) % 4 != 0)
    return fail(JL_ERR_INVALID_ARG, "block_table is NULL or not 4-byte aligned");
  JL_TRY(check_seq_lens(seq_lens));
  if (page_size < 32 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
    return fail(JL_ERR_INVALID_ARG, "page_size must be a power of two in [32, 2^20] (got %d)", page_size);
  if (n_pages < 1 || pages_per_seq < 1)
    return fail(JL_ERR_INVALID_ARG, "n_pages and pages_per_seq must be >= 1 (got %d, %d)", n_pages, pages_per_seq);
  const int64_t nkv = (int64_t)pages_per_seq * page_size;
  if (nkv > 0x7fffffff) return fail(JL_ERR_UNSUPPORTED, "pages_per_seq * page_size exceeds 2^31 - 1");
  if (elements(n_pages, page_size, n_kv_heads) < 0)
    return fail(JL_ERR_UNSUPPORTED, "the page pool overflows 64-bit element offsets");
  *n_kv = (int32_t)nkv;
  return JL_OK;
}

jl_status jl_bifocal_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* out, float* lse,
                                  const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                  int32_t n_pages, int32_t page_size, int32_t pages_per_seq, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int64_t pretrained_window,
                                  int64_t local_window, double rope_base, int32_t schedule, float softmax_scale,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  int32_t n_kv = 0;
  JL_TRY(paged_common(block_table, seq_lens, n_pages, page_size, pages_per_seq, n_kv_heads, &n_kv));
  float scale;
  const Shape s{batch, 1, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(decode_common(q, k_pages, v_pages, out, lse, s, softmax_scale, &scale, workspace, workspace_bytes));
  JL_TRY(check_windows(pretrained_window, local_window, rope_base));
  JL_TRY(check_schedule(schedule, pretrained_window, local_window, n_kv));
  JL_TRY(device_check());
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  jl::DecodeProblem p{q, k_pages, v_pages, out, lse, seq_lens, batch, n_kv, n_q_heads, n_kv_heads,
                      pretrained_window, w, rope_base, scale, workspace};
  p.schedule = schedule;
  p.block_table = block_table;
  p.pages_per_seq = pages_per_seq;
  p.page_size = page_size;
  p.n_pages = n_pages;
  return launched(jl::launch_decode(true, p, static_cast<hipStream_t>(stream)));
}

jl_status jl_plain_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* out, float* lse,
                                const int32_t* block_table, const int32_t* seq_lens, int32_t batch, int32_t n_pages,
                                int32_t page_size, int32_t pages_per_seq, int32_t n_q_heads, int32_t n_kv_heads,
                                int32_t head_dim, float softmax_scale, void* workspace, size_t workspace_bytes,
                                void* stream) {
  int32_t n_kv = 0;
  JL_TRY(paged_common(block_table, seq_lens, n_pages, page_size, pages_per_seq, n_kv_heads, &n_kv));
  float scale;
  const Shape s{batch, 1, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(decode_common(q, k_pages, v_pages, out, lse, s, softmax_scale, &scale, workspace, workspace_bytes));
  JL_TRY(device_check());
  jl::DecodeProblem p{q, k_pages, v_pages, out, lse, seq_lens, batch, n_kv, n_q_heads, n_kv_heads, 1, 0, 2.0, scale,
                      workspace};
  p.block_table = block_table;
  p.pages_per_seq = pages_per_seq;
  p.page_size = page_size;
  p.n_pages = n_pages;
  return launched(jl::launch_decode(false, p, static_cast<hipStream_t>(stream)));
}

// Workspace of the attention layer: projected q/k/v, rotated queries, the
// attention output, the attention's own workspace (chunk partials for the
// decode; the prefill needs none) and the library GEMM's scratch, each
// 256-byte aligned.
struct LayerWorkspace {
  size_t qkv, q, attn, attn_ws, gemm_ws, total;
};
static bool layer_workspace(int32_t batch, int32_t n_new, int32_t n_kv, int32_t hq, int32_t hkv, LayerWorkspace* l) {
  const int64_t e_qkv = elements(batch, n_new, (int64_t)hq + 2 * (int64_t)hkv);
  const int64_t e_q = elements(batch, n_new, hq);
  if (e_qkv < 0 || e_q < 0 || elements(batch, n_kv, hkv) < 0) return false;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  l->qkv = 0;
  l->q = up((size_t)e_qkv * 2);
  l->attn = l->q + up((size_t)e_q * 2);
  l->attn_ws = l->attn + up((size_t)e_q * 2);
  const size_t aw = n_new == 1 ? jl::decode_workspace_bytes(batch, n_kv, hq, hkv) : 0;
  l->gemm_ws = l->attn_ws + up(aw);
  l->total = l->gemm_ws + jl::kGemmWorkspaceBytes;
  return true;
}

size_t jl_qwen3_layer_workspace_size(int32_t batch, int32_t n_new, int32_t n_kv, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t head_dim) {
  if (batch < 1 || n_new < 1 || n_kv < n_new || n_q_heads < 1 || n_kv_heads < 1 || head_dim != 128 ||
      n_q_heads % n_kv_heads != 0)
    return 0;
  LayerWorkspace l;
  return layer_workspace(batch, n_new, n_kv, n_q_heads, n_kv_heads, &l) ? l.total : 0;
}

jl_status jl_qwen3_attention_layer(const void* x, const void* w_qkv, const void* q_norm_weight,
                                   const void* k_norm_weight, const void* w_o, void* out, void* k_cache,
                                   void* v_cache, int32_t batch, int32_t n_new, int32_t n_kv, int32_t hidden,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float rms_eps,
                                   int32_t attention, int64_t pretrained_window, int64_t local_window,
                                   double rope_base, int32_t schedule, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  const Shape s{batch, n_new, n_kv, n_q_heads, n_kv_heads, head_dim};
  JL_TRY(check_pointer(x, "x"));
  JL_TRY(check_pointer(w_qkv, "w_qkv"));
  JL_TRY(check_pointer(q_norm_weight, "q_norm_weight"));
  JL_TRY(check_pointer(k_norm_weight, "k_norm_weight"));
  JL_TRY(check_pointer(w_o, "w_o"));
  JL_TRY(check_pointer(out, "out"));
  JL_TRY(check_pointer(k_cache, "k_cache"));
  JL_TRY(check_pointer(v_cache, "v_cache"));
  JL_TRY(check_shape(s));
  if (hidden < 1) return fail(JL_ERR_INVALID_ARG, "hidden must be >= 1 (got %d)", hidden);
  if (!(rms_eps >= 0.0f) || std::isinf(rms_eps)) return fail(JL_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (attention != JL_LAYER_PLAIN && attention != JL_LAYER_BIFOCAL)
    return fail(JL_ERR_INVALID_ARG, "unknown attention kind %d", (int)attention);
  const bool bif_req = attention == JL_LAYER_BIFOCAL;
  if (bif_req) {
    JL_TRY(check_windows(pretrained_window, local_window, rope_base));
    JL_TRY(check_schedule(schedule, pretrained_window, local_window, n_kv));
  } else if (!(rope_base > 1.0) || !std::isfinite(rope_base)) {
    return fail(JL_ERR_INVALID_ARG, "rope_base must be finite and > 1");
  }
  const int64_t t = (int64_t)batch * n_new;
  const int64_t n_qkv = ((int64_t)n_q_heads + 2 * (int64_t)n_kv_heads) * 128;
  if (t > 0x7fffffff || n_qkv > 0x7fffffff || (int64_t)n_q_heads * 128 > 0x7fffffff ||
      elements(t, hidden, 1) < 0)
    return fail(JL_ERR_UNSUPPORTED, "layer sizes exceed the 32-bit GEMM dimensions");
  LayerWorkspace l;
  if (!layer_workspace(batch, n_new, n_kv, n_q_heads, n_kv_heads, &l))
    return fail(JL_ERR_UNSUPPORTED, "tensor sizes overflow 64-bit element offsets");
  JL_TRY(check_pointer(workspace, "workspace"));
  if (workspace_bytes < l.total)
    return fail(JL_ERR_WORKSPACE, "workspace_bytes %zu < required %zu", workspace_bytes, l.total);
  JL_TRY(device_check());

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* qkv = ws + l.qkv;
  void* q = ws + l.q;
  void* attn = ws + l.attn;
  void* attn_ws = ws + l.attn_ws;
  void* gemm_ws = ws + l.gemm_ws;
  const float scale = 1.0f / std::sqrt(128.0f);
  const int32_t w = (int32_t)(local_window < n_kv ? local_window : n_kv);
  const int32_t g = bif_req ? jl::sched_group(n_kv, pretrained_window, w, schedule) : 1;
  const bool bif = bif_req && g > 1;

  hipError_t e = jl::launch_gemm_xwt(x, w_qkv, qkv, t, n_qkv, hidden, gemm_ws, jl::kGemmWorkspaceBytes, st);
  if (e != hipSuccess) return launched(e);
  jl::NormRopeProblem nr{qkv, q_norm_weight, k_norm_weight, q, k_cache, v_cache, batch, n_new, n_kv, n_q_heads,
                         n_kv_heads, rms_eps, rope_base};
  e = jl::launch_norm_rope(nr, st);
  if (e != hipSuccess) return launched(e);
  if (n_new == 1) {
    jl::DecodeProblem p{q, k_cache, v_cache, attn, nullptr, nullptr, batch, n_kv, n_q_heads, n_kv_heads,
                        bif ? pretrained_window : 1, bif ? w : 0, rope_base, scale, attn_ws};
    p.schedule = bif ? schedule : jl::kSchedGrouped;
    e = jl::launch_decode(bif, p, st);
  } else {
    // the single-kernel bifocal prefill: keys corrected in LDS, no workspace
    jl::PrefillProblem p{q, k_cache, v_cache, attn, nullptr, nullptr, nullptr, nullptr, batch,
                         n_new, n_kv, n_q_heads, n_kv_heads, bif ? g : 1, bif ? w : 1, rope_base, scale};
    if (bif) {
      p.q_shift = jl::sched_q_shift(g, w, schedule);
      p.rate = jl::sched_rate(n_kv, pretrained_window, schedule);
    }
    e = jl::launch_prefill(bif ? jl::kModeBifocal : jl::kModePlain, p, st);
  }
  if (e != hipSuccess) return launched(e);
  return launched(
      jl::launch_gemm_xwt(attn, w_o, out, t, hidden, (int64_t)n_q_heads * 128, gemm_ws, jl::kGemmWorkspaceBytes, st));
}

}  // extern "C"
