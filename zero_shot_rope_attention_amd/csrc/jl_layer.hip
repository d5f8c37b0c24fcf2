// Pieces of a Qwen3-shaped attention layer around the attention kernels: the
// per-head RMSNorm + RoPE + cache append that turns the projected q/k/v into the
// attention's inputs, and the projections themselves (rocBLAS bf16 GEMMs, and a
// weight-streaming kernel of our own for the few tokens of a decode step).
//
// The method runs inside Qwen3 models (seventnews.com, "Empirical results that
// challenge the status quo"); a layer of them projects the hidden states to
// query, key and value heads, normalises the query and key heads, rotates them
// at the tokens' original positions (the cache keeps those positions: ResearchPod
// transcript, cache exchange), attends, and projects back.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <cmath>

#include "jl_device.h"
#include "jl_launch.h"

namespace jl {
namespace {

constexpr int kHeadThreads = 16;                 // threads per head: 4 pairs (d, d + 64) each
constexpr int kNormThreads = 256;                // 16 heads per workgroup
constexpr int kHeadsPerGroup = kNormThreads / kHeadThreads;

struct NormRopeArgs {
  const uint16_t* qkv;     // [T, (Hq + 2 Hkv) D], T = B * n_new tokens
  const uint16_t* gamma_q;  // [D]
  const uint16_t* gamma_k;  // [D]
  uint16_t* q;             // [T, Hq, D]
  uint16_t* k_cache;       // [B, n_kv, Hkv, D]
  uint16_t* v_cache;       // [B, n_kv, Hkv, D]
  int64_t n_heads_total;   // T * (Hq + 2 Hkv)
  int32_t n_new, n_kv, hq, hkv;
  float eps;
  double theta_rev[kHalfD];  // theta_d / (2 pi)
};

// One head of one token per 16 threads.  Thread l holds d = 4l .. 4l+3 and the
// partners d + 64, so the rotate-half pairs never leave the thread; the sum of
// squares is reduced across the 16 threads.  Values are read once and written
// once (the kernel is bound by those bytes).
__global__ __launch_bounds__(kNormThreads) void norm_rope_kernel(const NormRopeArgs a) {
  const int64_t head = (int64_t)blockIdx.x * kHeadsPerGroup + (threadIdx.x / kHeadThreads);
  const int l = threadIdx.x % kHeadThreads;
  if (head >= a.n_heads_total) return;  // whole 16-thread groups leave together
  const int per_tok = a.hq + 2 * a.hkv;
  const int64_t t = head / per_tok;
  const int h = (int)(head % per_tok);
  const int b = (int)(t / a.n_new);
  const int p = a.n_kv - a.n_new + (int)(t % a.n_new);  // the token's original position

  const uint16_t* src = a.qkv + head * kD;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(src + 4 * l);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(src + kHalfD + 4 * l);
  const int kv_h = h < a.hq ? 0 : (h < a.hq + a.hkv ? h - a.hq : h - a.hq - a.hkv);
  const int64_t cache_row = (((int64_t)b * a.n_kv + p) * a.hkv + kv_h) * kD;
  if (h >= a.hq + a.hkv) {  // a value head: appended as it is
    *reinterpret_cast<u32x2*>(a.v_cache + cache_row + 4 * l) = lo;
    *reinterpret_cast<u32x2*>(a.v_cache + cache_row + kHalfD + 4 * l) = hi;
    return;
  }
  float x1[4] = {bf_lo(lo[0]), bf_hi(lo[0]), bf_lo(lo[1]), bf_hi(lo[1])};
  float x2[4] = {bf_lo(hi[0]), bf_hi(hi[0]), bf_lo(hi[1]), bf_hi(hi[1])};
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
#pragma unroll
  for (int m = 1; m < kHeadThreads; m <<= 1) ss += __shfl_xor(ss, m, kHeadThreads);
  const float r = 1.0f / sqrtf(ss * (1.0f / kD) + a.eps);
  const bool is_q = h < a.hq;
  const uint16_t* gam = is_q ? a.gamma_q : a.gamma_k;
  const u32x2 g_lo = *reinterpret_cast<const u32x2*>(gam + 4 * l);
  const u32x2 g_hi = *reinterpret_cast<const u32x2*>(gam + kHalfD + 4 * l);
  const float g1[4] = {bf_lo(g_lo[0]), bf_hi(g_lo[0]), bf_lo(g_lo[1]), bf_hi(g_lo[1])};
  const float g2[4] = {bf_lo(g_hi[0]), bf_hi(g_hi[0]), bf_lo(g_hi[1]), bf_hi(g_hi[1])};
  float y1[4], y2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2 cs = rot_cs(p, a.theta_rev[4 * l + e]);  // p theta_d, reduced in fp64
    const float u1 = x1[e] * r * g1[e], u2 = x2[e] * r * g2[e];
    y1[e] = u1 * cs.x - u2 * cs.y;
    y2[e] = u2 * cs.x + u1 * cs.y;
  }
  const u32x2 o_lo = {pack_bf16(y1[0], y1[1]), pack_bf16(y1[2], y1[3])};
  const u32x2 o_hi = {pack_bf16(y2[0], y2[1]), pack_bf16(y2[2], y2[3])};
  uint16_t* dst = is_q ? a.q + (t * a.hq + h) * kD : a.k_cache + cache_row;
  *reinterpret_cast<u32x2*>(dst + 4 * l) = o_lo;
  *reinterpret_cast<u32x2*>(dst + kHalfD + 4 * l) = o_hi;
}

// y[t, r] = sum_k x[t, k] w[r, k] for a handful of tokens (a decode step): the
// product reads every weight once, so it is bound by the weight bytes, and a
// wave per kGemvRows output rows streams them with 16-byte loads while every
// lane keeps the tokens' matching 8 elements beside them.  Dot products of bf16
// pairs accumulate in fp32 (v_dot2), then a 64-lane reduction per output.
constexpr int kGemvMaxTokens = 8;
constexpr int kGemvRows = 4;
constexpr int kGemvWaves = 4;

template <int T>
__global__ __launch_bounds__(kGemvWaves * 64) void gemv_xwt_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ w,
                                                                    uint16_t* __restrict__ y, int n, int k) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * kGemvWaves + wave) * kGemvRows;
  if (row0 >= n) return;  // whole waves leave together
  const uint16_t* wr[kGemvRows];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r) wr[r] = w + (int64_t)min(row0 + r, n - 1) * k;
  float acc[kGemvRows][T];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[r][t] = 0.0f;
#pragma unroll 2
  for (int k0 = 8 * lane; k0 < k; k0 += 512) {
    u32x4 wv[kGemvRows], xv[T];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) wv[r] = *reinterpret_cast<const u32x4*>(wr[r] + k0);
#pragma unroll
    for (int t = 0; t < T; ++t) xv[t] = *reinterpret_cast<const u32x4*>(x + (int64_t)t * k + k0);
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // each element is copied out first: bit_cast of a vector element in place
          // reads element 0 whatever the index (hipcc's front end)
          const uint32_t wp = wv[r][e], xp = xv[t][e];
          acc[r][t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp), __builtin_bit_cast(bf16x2, xp),
                                                      acc[r][t], false);
        }
  }
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float v = acc[r][t];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      acc[r][t] = v;
    }
  if (lane < T) {
    // lane t writes token t's rows
#pragma unroll
    for (int t = 0; t < T; ++t)
      if (t == lane)
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r)
          if (row0 + r < n) {
            const uint32_t pk = pack_bf16(acc[r][t], 0.0f);
            y[(int64_t)t * n + row0 + r] = (uint16_t)(pk & 0xffffu);
          }
  }
}

template <int T>
hipError_t launch_gemv(const void* x, const void* w, void* y, int n, int k, hipStream_t stream) {
  const int per_block = kGemvRows * kGemvWaves;
  const int blocks = (n + per_block - 1) / per_block;
  hipLaunchKernelGGL((gemv_xwt_kernel<T>), dim3(blocks), dim3(kGemvWaves * 64), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), static_cast<uint16_t*>(y), n,
                     k);
  return hipGetLastError();
}

// rocBLAS handles of the calling thread, one per device: created on first use,
// destroyed when the thread exits.
struct ThreadHandles {
  static constexpr int kMaxDevices = 64;
  rocblas_handle h[kMaxDevices] = {};
  ~ThreadHandles() {
    for (rocblas_handle& x : h)
      if (x) rocblas_destroy_handle(x);
  }
};

rocblas_handle thread_handle() {
  thread_local ThreadHandles handles;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= ThreadHandles::kMaxDevices) return nullptr;
  rocblas_handle& h = handles.h[dev];
  if (!h && rocblas_create_handle(&h) != rocblas_status_success) h = nullptr;
  return h;
}

}  // namespace

hipError_t launch_norm_rope(const NormRopeProblem& p, hipStream_t stream) {
  NormRopeArgs a;
  a.qkv = static_cast<const uint16_t*>(p.qkv);
  a.gamma_q = static_cast<const uint16_t*>(p.gamma_q);
  a.gamma_k = static_cast<const uint16_t*>(p.gamma_k);
  a.q = static_cast<uint16_t*>(p.q);
  a.k_cache = static_cast<uint16_t*>(p.k_cache);
  a.v_cache = static_cast<uint16_t*>(p.v_cache);
  a.n_new = p.n_new;
  a.n_kv = p.n_kv;
  a.hq = p.n_q_heads;
  a.hkv = p.n_kv_heads;
  a.eps = p.eps;
  a.n_heads_total = (int64_t)p.batch * p.n_new * (p.n_q_heads + 2 * p.n_kv_heads);
  const double two_pi = 6.283185307179586476925286766559;
  for (int d = 0; d < kHalfD; ++d) a.theta_rev[d] = std::pow(p.rope_base, -2.0 * d / kD) / two_pi;
  const int64_t blocks = (a.n_heads_total + kHeadsPerGroup - 1) / kHeadsPerGroup;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(norm_rope_kernel, dim3((unsigned)blocks), dim3(kNormThreads), 0, stream, a);
  return hipGetLastError();
}

// Row-major y[m, n] = x[m, k] w[n, k]^T, bf16 in and out, fp32 accumulation.
// In rocBLAS's column-major terms that is y^T (n x m) = w (op T of the k x n
// column-major view) times x^T (k x m).
hipError_t launch_gemm_xwt(const void* x, const void* w, void* y, int64_t m, int64_t n, int64_t k,
                           void* gemm_ws, size_t gemm_ws_bytes, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  if (m > 0x7fffffff || n > 0x7fffffff || k > 0x7fffffff) return hipErrorInvalidValue;
  // a few tokens (decode): the weight-streaming kernel above; 16-byte rows need k % 8 == 0
  const bool aligned = (reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w)) % 16 == 0 && k % 8 == 0;
  if (m <= kGemvMaxTokens && aligned) {
    switch (m) {
      case 1: return launch_gemv<1>(x, w, y, (int)n, (int)k, stream);
      case 2: return launch_gemv<2>(x, w, y, (int)n, (int)k, stream);
      case 3: return launch_gemv<3>(x, w, y, (int)n, (int)k, stream);
      case 4: return launch_gemv<4>(x, w, y, (int)n, (int)k, stream);
      case 5: return launch_gemv<5>(x, w, y, (int)n, (int)k, stream);
      case 6: return launch_gemv<6>(x, w, y, (int)n, (int)k, stream);
      case 7: return launch_gemv<7>(x, w, y, (int)n, (int)k, stream);
      default: return launch_gemv<8>(x, w, y, (int)n, (int)k, stream);
    }
  }
  rocblas_handle h = thread_handle();
  if (!h) return hipErrorInvalidValue;
  if (rocblas_set_stream(h, stream) != rocblas_status_success) return hipErrorInvalidValue;
  // the GEMM's scratch is the caller's memory: rocBLAS allocates none for it
  if (rocblas_set_workspace(h, gemm_ws, gemm_ws_bytes) != rocblas_status_success) return hipErrorInvalidValue;
  const float alpha = 1.0f, beta = 0.0f;
  const rocblas_status st =
      rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)n, (rocblas_int)m,
                      (rocblas_int)k, &alpha, w, rocblas_datatype_bf16_r, (rocblas_int)k, x, rocblas_datatype_bf16_r,
                      (rocblas_int)k, &beta, y, rocblas_datatype_bf16_r, (rocblas_int)n, y, rocblas_datatype_bf16_r,
                      (rocblas_int)n, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success) return hipErrorLaunchFailure;
  return hipGetLastError();
}

}  // namespace jl
