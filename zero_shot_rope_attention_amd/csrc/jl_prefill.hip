// Fused bifocal prefill for gfx950 (MI355X).
//
// One workgroup owns a block of query rows for `hpw` query heads that share a KV
// head (GQA), and sweeps the causal key range once in tiles of 64 keys.  Each
// tile of K (as cached, at original positions) and V is staged in LDS once and
// used by every wave; in the bifocal modes the same staging step also writes the
// corrected keys k^g_j = rot(k_j, c(j) theta) next to them, so the correction
// rotation is computed on the fly, once per tile, and never stored in HBM
// (ResearchPod transcript, cache exchange: original positions in the cache,
// remapping applied at lookup).  Queries are corrected once, in registers.
//
// Each wave owns 32 query rows of one head and computes, per tile,
//   S^T = K Q^T   (MFMA; A = keys from LDS, B = query fragment in registers)
//   O^T += V^T P^T (MFMA; A = V^T from LDS, B = probabilities in registers)
// so that every lane holds one query row's scores, softmax state and output
// columns, and no transposition of P or of the running statistics is needed.
//
// Modes
//   kModePlain   : causal attention on the cached vectors (base model).
//   kModeBifocal : the inclusion-exclusion merge of the three passes of the
//                  method (ResearchPod summary, 2nd paragraph; Abstract).  The
//                  passes are evaluated with one shared running maximum.  With a
//                  shared maximum pass B's and pass C's probabilities on a local
//                  key are bit-identical, so B - C leaves exactly B's remote keys,
//                  and since PV is linear the merged numerator
//                  sum_X sign_X P_X V = (P_A + P_B - P_C) V needs one accumulator:
//                  local keys carry base-RoPE scores, remote keys grouped scores.
//   kModePasses  : the three passes with their own maxima and accumulators,
//                  each normalised on its own key set and written out with its
//                  log-sum-exp (pass A local/base, B causal/grouped, C
//                  local/grouped; ResearchPod transcript, prefill exchange).
#include "jl_device.h"
#include "jl_launch.h"

namespace jl {
namespace {

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  float* out_abc;
  float* lse_abc;
  int32_t batch, n_q, n_kv, hq, hkv;
  int32_t grp;        // Hq / Hkv
  int32_t hpw;        // query heads per workgroup
  int32_t bm;         // query rows per workgroup
  int32_t n_qblocks;  // ceil(n_q / bm)
  int32_t n_units;    // batch * Hkv * (grp / hpw)
  int32_t g;          // group factor g(s)
  int32_t w;          // local window
  float inv_g;
  float scale_log2;   // softmax scale * log2(e)
  double theta_rev[kHalfD];  // theta_d / (2 pi)
};

// Swizzled 16-byte chunk of a 256-byte K row: spreads the 32 rows one MFMA
// operand read touches (key permutation below) over all 64 LDS banks.
__device__ __forceinline__ int k_chunk(int row, int chunk) {
  return chunk ^ ((row & 7) | ((row & 16) >> 1));
}
// Byte offset of 16-byte chunk `c` (8 keys) in row d of the transposed V tile.
__device__ __forceinline__ int vt_offset(int d, int c) { return d * (kBN * 2) + ((c ^ ((d >> 1) & 7)) << 4); }

// Key (within a 32-key block) that MFMA row m of S^T stands for.  With this
// permutation, lane half h holds keys 16h .. 16h+15 of the block in output
// registers 0..15, so a lane's probabilities form B operands of O^T = V^T P^T
// directly (8 consecutive keys per operand).
__device__ __forceinline__ int perm_key(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

__device__ __forceinline__ float elem(const u32x4& u, int e) {
  uint32_t w = u[e >> 1];
  return (e & 1) ? bf_hi(w) : bf_lo(w);
}

// S^T tile (64 keys x 32 query rows) from a K tile in LDS and the query fragment.
__device__ __forceinline__ void qk_tile(const uint8_t* kbuf, const bf16x8 (&qf)[8], int lane, f32x16 (&s)[2]) {
  const int h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * kb + perm_key(lane & 31);
    const uint8_t* rp = kbuf + row * 256;
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(rp + (k_chunk(row, 2 * kk + h) << 4));
      acc = mfma32(as_bf16x8(a), qf[kk], acc);
    }
    s[kb] = acc;
  }
}

template <int MODE, int NW>
__global__ __launch_bounds__(NW * 64, 1) void prefill_kernel(const PrefillArgs a) {
  constexpr int NT = NW * 64;
  constexpr bool kGrouped = MODE != kModePlain;
  constexpr int NS = (MODE == kModePasses) ? 3 : 1;

  __shared__ __attribute__((aligned(16))) uint8_t s_k[kBN * 256];
  __shared__ __attribute__((aligned(16))) uint8_t s_kg[kGrouped ? kBN * 256 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_vt[kD * kBN * 2];
  __shared__ f32x2 s_tdelta[kGrouped ? 65 * kHalfD : 1];  // E(-u theta_d), u = 0..64
  __shared__ f32x2 s_base[kGrouped ? 2 * kHalfD : 1];     // E(c(j0) theta_d), double-buffered

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int n = lane & 31;

  // Workgroup -> (unit, query block).  Dispatch places consecutive workgroups
  // on consecutive XCDs; when possible every XCD keeps one KV head, so the
  // workgroups resident on an XCD stream the same K/V tiles through its L2.
  // Within a unit the longest (last) query blocks go first.
  int unit, rank;
  {
    const int id = blockIdx.x;
    if ((a.n_units & 7) == 0) {
      const int slot = id >> 3;
      unit = (id & 7) + 8 * (slot / a.n_qblocks);
      rank = slot % a.n_qblocks;
    } else {
      unit = id / a.n_qblocks;
      rank = id % a.n_qblocks;
    }
  }
  const int qb = a.n_qblocks - 1 - rank;
  const int n_hg = a.grp / a.hpw;
  const int hg = unit % n_hg;
  const int bk = unit / n_hg;
  const int kvh = bk % a.hkv;
  const int b = bk / a.hkv;
  const int hq = kvh * a.grp + hg * a.hpw + (wave % a.hpw);
  const int row0_wg = qb * a.bm;
  const int row0 = row0_wg + (wave / a.hpw) * 32;
  const int pos_off = a.n_kv - a.n_q;
  const int last_row_wg = min(a.n_q, row0_wg + a.bm) - 1;
  const int kend = pos_off + last_row_wg + 1;  // keys 0 .. kend-1 are visible to some row
  const int ntiles = (kend + kBN - 1) / kBN;

  const bool wave_rows = row0 < a.n_q;
  const int wp_lo = pos_off + row0;
  const int wp_hi = pos_off + min(a.n_q, row0 + 32) - 1;
  const int my_row = row0 + n;
  const bool row_ok = my_row < a.n_q;
  const int my_p = row_ok ? pos_off + my_row : -1;  // -1: no causal key at all

  const int64_t q_rs = (int64_t)a.hq * kD;
  const int64_t kv_rs = (int64_t)a.hkv * kD;
  const uint16_t* kbase = a.k + (int64_t)b * a.n_kv * kv_rs + (int64_t)kvh * kD;
  const uint16_t* vbase = a.v + (int64_t)b * a.n_kv * kv_rs + (int64_t)kvh * kD;

  // ---- query fragments (B operand of S^T): row my_row, d = 16kk + 8h + e ----
  bf16x8 qf[8];
  bf16x8 qg[8];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.n_q + (row_ok ? my_row : 0)) * q_rs + (int64_t)hq * kD;
    u32x4 raw[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      raw[kk] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0};
      qf[kk] = as_bf16x8(raw[kk]);
    }
    if constexpr (kGrouped) {
      // q^g = rot(q, c(p) theta), rounded to bf16
      const long long cq = row_ok ? (long long)(my_p / a.g) - my_p : 0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 lo, hi;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float y1[2], y2[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int e = 2 * e2 + t;
            const int d = 16 * kk + 8 * h + e;
            const f32x2 cs = rot_cs(cq, a.theta_rev[d]);
            const float x1 = elem(raw[kk], e), x2 = elem(raw[kk + 4], e);
            y1[t] = x1 * cs.x - x2 * cs.y;
            y2[t] = x2 * cs.x + x1 * cs.y;
          }
          lo[e2] = pack_bf16(y1[0], y1[1]);
          hi[e2] = pack_bf16(y2[0], y2[1]);
        }
        qg[kk] = as_bf16x8(lo);
        qg[kk + 4] = as_bf16x8(hi);
      }
    }
  }

  if constexpr (kGrouped) {
    for (int idx = tid; idx < 65 * kHalfD; idx += NT)
      s_tdelta[idx] = rot_cs(-(long long)(idx >> 6), a.theta_rev[idx & 63]);
    if (tid < kHalfD) s_base[tid] = f32x2{1.0f, 0.0f};  // tile 0: c(0) = 0
  }

  float m_run[NS], l_run[NS];
  f32x16 acc[NS][4];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    m_run[s] = kNegBig;
    l_run[s] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[s][nb] = f32x16{};
  }

  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kBN;

    // ---- stage K (and corrected K) ----
    // item: key kt, 16-byte chunks c and c+8 (the two halves of 8 rotate-half pairs)
    bool need_grp = false;
    int r_mod = 0;
    if constexpr (MODE == kModeBifocal) need_grp = (j0 <= kend - 1 - a.w);  // some remote key
    if constexpr (MODE == kModePasses) need_grp = true;
    if constexpr (kGrouped) r_mod = j0 % a.g;
    const f32x2* base_cur = s_base + (t & 1) * kHalfD;
    for (int id = tid; id < kBN * 8; id += NT) {
      const int kt = id >> 3;
      const int c = id & 7;
      const int j = j0 + kt;
      u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (j < a.n_kv) {
        const uint16_t* kp = kbase + (int64_t)j * kv_rs + 8 * c;
        lo = *reinterpret_cast<const u32x4*>(kp);
        hi = *reinterpret_cast<const u32x4*>(kp + kHalfD);
      }
      *reinterpret_cast<u32x4*>(s_k + kt * 256 + (k_chunk(kt, c) << 4)) = lo;
      *reinterpret_cast<u32x4*>(s_k + kt * 256 + (k_chunk(kt, c + 8) << 4)) = hi;
      if constexpr (kGrouped) {
        if (need_grp) {
          // c(j) = c(j0) - u with u = kt - floor((r + kt) / g), r = j0 mod g
          const int u = kt - small_div(r_mod + kt, a.g, a.inv_g);
          const f32x2* td = s_tdelta + u * kHalfD + 8 * c;
          const f32x2* bs = base_cur + 8 * c;
          u32x4 glo, ghi;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            float y1[2], y2[2];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
              const int e = 2 * e2 + q2;
              const f32x2 cs = cmul(bs[e], td[e]);
              const float x1 = elem(lo, e), x2 = elem(hi, e);
              y1[q2] = x1 * cs.x - x2 * cs.y;
              y2[q2] = x2 * cs.x + x1 * cs.y;
            }
            glo[e2] = pack_bf16(y1[0], y1[1]);
            ghi[e2] = pack_bf16(y2[0], y2[1]);
          }
          *reinterpret_cast<u32x4*>(s_kg + kt * 256 + (k_chunk(kt, c) << 4)) = glo;
          *reinterpret_cast<u32x4*>(s_kg + kt * 256 + (k_chunk(kt, c + 8) << 4)) = ghi;
        }
      }
    }
    // ---- stage V transposed: item = keys (2kp, 2kp+1) x d chunk dc ----
    for (int id = tid; id < (kBN / 2) * 16; id += NT) {
      const int kp = id >> 4;
      const int dc = id & 15;
      const int j = j0 + 2 * kp;
      u32x4 va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
      if (j < a.n_kv) va = *reinterpret_cast<const u32x4*>(vbase + (int64_t)j * kv_rs + 8 * dc);
      if (j + 1 < a.n_kv) vb = *reinterpret_cast<const u32x4*>(vbase + (int64_t)(j + 1) * kv_rs + 8 * dc);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wa = va[e >> 1], wb = vb[e >> 1];
        const uint32_t val = (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
        const int d = 8 * dc + e;
        *reinterpret_cast<uint32_t*>(s_vt + vt_offset(d, kp >> 2) + ((kp & 3) << 2)) = val;
      }
    }
    // ---- rotation base for the next tile ----
    if constexpr (kGrouped) {
      if (tid < kHalfD && t + 1 < ntiles) {
        const int j1 = j0 + kBN;
        s_base[((t + 1) & 1) * kHalfD + tid] = rot_cs((long long)(j1 / a.g) - j1, a.theta_rev[tid]);
      }
    }
    __syncthreads();

    // ---- per-wave compute ----
    if (wave_rows && j0 <= wp_hi) {
      bool use_base = true, use_grp = false;
      if constexpr (MODE == kModeBifocal) {
        use_grp = (j0 <= wp_hi - a.w);                 // a remote key for some row of the wave
        use_base = (j0 + kBN - 1 >= wp_lo - a.w + 1);  // a local key for some row of the wave
      }
      if constexpr (MODE == kModePasses) {
        use_grp = true;
        use_base = true;
      }
      f32x16 sb[2], sg[2];
      if (use_base) qk_tile(s_k, qf, lane, sb);
      if constexpr (kGrouped) {
        if (use_grp) qk_tile(s_kg, qg, lane, sg);
      }

      // scores in log2 units per state; keys j = j0 + 32kb + 16h + i
      float x[NS][2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dist = my_p - (j0 + 32 * kb + 16 * h + i);
          const bool causal = dist >= 0;
          if constexpr (MODE == kModePlain) {
            x[0][kb][i] = causal ? sb[kb][i] * a.scale_log2 : -INFINITY;
          } else if constexpr (MODE == kModeBifocal) {
            const bool local = causal && dist < a.w;
            const float v = local ? (use_base ? sb[kb][i] : 0.0f) : (use_grp ? sg[kb][i] : 0.0f);
            x[0][kb][i] = causal ? v * a.scale_log2 : -INFINITY;
          } else {
            const bool local = causal && dist < a.w;
            x[0][kb][i] = local ? sb[kb][i] * a.scale_log2 : -INFINITY;
            x[1][kb][i] = causal ? sg[kb][i] * a.scale_log2 : -INFINITY;
            x[NS - 1][kb][i] = local ? sg[kb][i] * a.scale_log2 : -INFINITY;
          }
        }
      }

      // online softmax per state
      uint32_t pk[NS][2][8];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float mloc = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, x[s][kb][i]);
        mloc = fmaxf(mloc, swap_halves(mloc));
        const float m_new = fmaxf(m_run[s], mloc);
        const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_new);
        m_run[s] = m_new;
        float psum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i2 = 0; i2 < 8; ++i2) {
            const float p0 = __builtin_amdgcn_exp2f(x[s][kb][2 * i2] - m_new);
            const float p1 = __builtin_amdgcn_exp2f(x[s][kb][2 * i2 + 1] - m_new);
            psum += p0 + p1;
            pk[s][kb][i2] = pack_bf16(p0, p1);
          }
        }
        l_run[s] = l_run[s] * alpha + psum;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[s][nb] *= alpha;
      }

      // O^T += V^T P^T over 4 steps of 16 keys: step (kb, half) uses keys
      // 32kb + 16h + 8half + e, which are output registers 8half + e of block kb.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int c = 4 * kb + 2 * h + half;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int d = 32 * nb + n;
            const u32x4 vf = *reinterpret_cast<const u32x4*>(s_vt + vt_offset(d, c));
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              const u32x4 pf = {pk[s][kb][4 * half + 0], pk[s][kb][4 * half + 1], pk[s][kb][4 * half + 2],
                                pk[s][kb][4 * half + 3]};
              acc[s][nb] = mfma32(as_bf16x8(vf), as_bf16x8(pf), acc[s][nb]);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds row my_row, columns d = 32nb + 8(i/4) + 4h + (i%4) ----
  if (!row_ok) return;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float lt = l_run[s] + swap_halves(l_run[s]);
    const bool empty = !(lt > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / lt;
    const float lse_v = empty ? -INFINITY : (m_run[s] + __builtin_log2f(lt)) * kLn2;
    if constexpr (MODE == kModePasses) {
      float* o = a.out_abc + ((((int64_t)s * a.batch + b) * a.n_q + my_row) * a.hq + hq) * kD;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          float4 val = {acc[s][nb][4 * i4] * inv, acc[s][nb][4 * i4 + 1] * inv, acc[s][nb][4 * i4 + 2] * inv,
                        acc[s][nb][4 * i4 + 3] * inv};
          *reinterpret_cast<float4*>(o + 32 * nb + 8 * i4 + 4 * h) = val;
        }
      if (h == 0) a.lse_abc[(((int64_t)s * a.batch + b) * a.hq + hq) * a.n_q + my_row] = lse_v;
    } else {
      uint16_t* o = a.out + (((int64_t)b * a.n_q + my_row) * a.hq + hq) * kD;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          u32x2 val = {pack_bf16(acc[s][nb][4 * i4] * inv, acc[s][nb][4 * i4 + 1] * inv),
                       pack_bf16(acc[s][nb][4 * i4 + 2] * inv, acc[s][nb][4 * i4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(o + 32 * nb + 8 * i4 + 4 * h) = val;
        }
      if (a.lse && h == 0) a.lse[((int64_t)b * a.hq + hq) * a.n_q + my_row] = lse_v;
    }
  }
}

template <int MODE, int NW>
hipError_t launch_mode(const PrefillProblem& p, hipStream_t stream) {
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.out = static_cast<uint16_t*>(p.out);
  a.lse = p.lse;
  a.out_abc = p.out_abc;
  a.lse_abc = p.lse_abc;
  a.batch = p.batch;
  a.n_q = p.n_q;
  a.n_kv = p.n_kv;
  a.hq = p.n_q_heads;
  a.hkv = p.n_kv_heads;
  a.grp = p.n_q_heads / p.n_kv_heads;
  int hpw = 1;
  for (int c = NW; c > 1; c >>= 1)
    if (a.grp % c == 0) {
      hpw = c;
      break;
    }
  a.hpw = hpw;
  a.bm = 32 * NW / hpw;
  a.n_qblocks = (p.n_q + a.bm - 1) / a.bm;
  a.n_units = p.batch * p.n_kv_heads * (a.grp / hpw);
  a.g = p.group;
  a.w = p.local_window;
  a.inv_g = 1.0f / (float)p.group;
  a.scale_log2 = p.softmax_scale * 1.4426950408889634f;
  const double two_pi = 6.283185307179586476925286766559;
  for (int d = 0; d < kHalfD; ++d) a.theta_rev[d] = std::pow(p.rope_base, -2.0 * d / kD) / two_pi;
  const long long blocks = (long long)a.n_units * a.n_qblocks;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<MODE, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(PrefillMode mode, const PrefillProblem& p, hipStream_t stream) {
  switch (mode) {
    case kModePlain: return launch_mode<kModePlain, 8>(p, stream);
    case kModeBifocal: return launch_mode<kModeBifocal, 8>(p, stream);
    case kModePasses: return launch_mode<kModePasses, 4>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace jl
