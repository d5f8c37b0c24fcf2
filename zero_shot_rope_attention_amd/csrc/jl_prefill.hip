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
#include <type_traits>

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
  const uint16_t* kg;  // corrected keys of the whole cache (precorrected mode)
  int32_t batch, n_q, n_kv, hq, hkv;
  int32_t grp;        // Hq / Hkv
  int32_t hpw;        // query heads per workgroup
  int32_t bm;         // query rows per workgroup
  int32_t n_qblocks;  // ceil(n_q / bm)
  int32_t n_units;    // batch * Hkv * (grp / hpw)
  int32_t g;          // group factor g(s)
  int32_t w;          // local window
  int32_t q_shift;    // added to c(p) of the queries: the seam shift W - floor(W/g), else 0
  float inv_g;
  float scale_log2;   // softmax scale * log2(e)
  double theta_rev[kHalfD];  // theta_d / (2 pi)
  // variable-length batches (the VARLEN kernels only): sequence b has the packed
  // query rows cu_q[b] .. cu_q[b+1]-1 and kv_lens[b] cached keys; n_q is then the
  // longest query count, n_kv the cache's rows per sequence, and the group factor,
  // query shift and rate are taken per sequence from big_l, w and sched
  const int32_t* cu_q;
  const int32_t* kv_lens;
  int32_t total_q;
  int32_t sched;
  int64_t big_l;
  // explicit query positions (the QPOS kernels only): row i sits at q_pos[i],
  // nondecreasing, shared by the batch; otherwise row i sits at n_kv - n_q + i
  const int32_t* q_pos;
};

// Swizzled 16-byte chunk of a 256-byte K row: spreads the 32 rows one MFMA
// operand read touches (key permutation below) over all 64 LDS banks.
__device__ __forceinline__ int k_chunk(int row, int chunk) {
  return chunk ^ ((row & 7) | ((row & 16) >> 1));
}
// V tiles are kept row-major (key rows of 256 bytes); 16-byte chunk c of key row
// r is stored at chunk c ^ 4(r % 4), which makes the transposed reads of the
// PV operand (4 keys x 64 bytes per half-wave) hit all 64 LDS banks once.
__device__ __forceinline__ int v_chunk(int row, int chunk) { return chunk ^ ((row & 3) << 2); }

// Rows of the single kernel's small-angle table (-u theta_d in revolutions)
// are padded by 16 bytes, so that the 16 lanes of a 16-byte read (two keys,
// eight chunks) fall on different banks when their u differ by one.
constexpr int kUangStride = kHalfD + 4;

// Key (within a 32-key block) that MFMA row m of S^T stands for.  With this
// permutation, lane half h holds keys 16h .. 16h+15 of the block in output
// registers 0..15, so a lane's probabilities form B operands of O^T = V^T P^T
// directly (8 consecutive keys per operand).
__device__ __forceinline__ int perm_key(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

__device__ __forceinline__ float elem(const u32x4& u, int e) {
  uint32_t w = u[e >> 1];
  return (e & 1) ? bf_hi(w) : bf_lo(w);
}

// Lane-constant LDS byte offsets of the MFMA operands within a tile.  The
// swizzles only depend on a key row's low bits, which are the same for every
// row a lane touches, so everything else is an immediate offset.
struct LaneOffsets {
  int k[8];  // K fragment of step kk (key block 0; block 1 is +32 rows)
  int v[4];  // V^T fragment of column block nb (keys 4r + j/4 of the lane group)
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
  LaneOffsets o;
  const int h = lane >> 5;
  const int row = perm_key(lane & 31);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) o.k[kk] = row * 256 + (k_chunk(row, 2 * kk + h) << 4);
  const int j = lane & 15;
  const int key = 16 * h + (j >> 2);
  const int dcol = 16 * ((lane >> 4) & 1) + 4 * (j & 3);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) o.v[nb] = key * 256 + (v_chunk(key, (32 * nb + dcol) >> 3) << 4) + ((dcol & 7) << 1);
  return o;
}

// The same offsets from two words: the swizzles only flip address bits 5-7 (K:
// fragment kk is fragment 0 with kk in bits 5-7) and 6-7 (V: column block nb
// is block 0 with nb in bits 6-7), and tile buffers are 16 KB aligned, so the
// flips commute with adding a buffer's base.
struct LaneBase {
  uint32_t k0, v0;
};
__device__ __forceinline__ LaneBase lane_base(int lane) {
  const LaneOffsets o = lane_offsets(lane);
  return LaneBase{(uint32_t)o.k[0], (uint32_t)o.v[0]};
}
__device__ __forceinline__ LaneOffsets lane_expand(const LaneBase& b) {
  LaneOffsets o;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) o.k[kk] = (int)(b.k0 ^ ((uint32_t)kk << 5));
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) o.v[nb] = (int)(b.v0 ^ ((uint32_t)nb << 6));
  return o;
}

// Byte offsets of K fragment kk and V^T column block nb, from either form.
__device__ __forceinline__ int k_off(const LaneOffsets& o, int kk) { return o.k[kk]; }
__device__ __forceinline__ int v_off(const LaneOffsets& o, int nb) { return o.v[nb]; }
__device__ __forceinline__ int k_off(const LaneBase& b, int kk) { return (int)(b.k0 ^ ((uint32_t)kk << 5)); }
__device__ __forceinline__ int v_off(const LaneBase& b, int nb) { return (int)(b.v0 ^ ((uint32_t)nb << 6)); }

// S^T of one 32-key block (rows kbuf .. kbuf + 32 keys) against the query fragment.
// kLean: each step's operand is read in that step (a scheduling barrier after
// every product), for code outside the hot loop where registers are short.
template <bool kLean = false, class LO>
__device__ __forceinline__ f32x16 qk_block(const uint8_t* kbuf, const LO& lo, const bf16x8 (&q)[8]) {
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    acc = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(kbuf + k_off(lo, kk))), q[kk], acc);
    if constexpr (kLean) __builtin_amdgcn_sched_barrier(0);
  }
  return acc;
}

// S^T tile (64 keys x 32 query rows) from a K tile in LDS and the query
// fragment; the two 32-key blocks accumulate side by side.
template <bool kLean = false, class LO>
__device__ __forceinline__ void qk_tile(const uint8_t* kbuf, const LO& lo, const bf16x8 (&qf)[8], f32x16 (&s)[2]) {
  f32x16 acc0 = {}, acc1 = {};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(kbuf + k_off(lo, kk));
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(kbuf + k_off(lo, kk) + 32 * 256);
    acc0 = mfma32(as_bf16x8(a0), qf[kk], acc0);
    acc1 = mfma32(as_bf16x8(a1), qf[kk], acc1);
    if constexpr (kLean) __builtin_amdgcn_sched_barrier(0);
  }
  s[0] = acc0;
  s[1] = acc1;
}

// Direct HBM -> LDS staging of a 64-key tile (16 KB) of V, or of K as cached:
// 16 wave-instructions of 1 KB (4 key rows each), split over the NW waves.
// Lane l fills physical chunk l % 16 of row 4 i + l / 16 and so fetches the
// logical chunk that the swizzle maps there.  Rows past n_kv re-read the last
// key (finite data whose probabilities are exactly zero).
template <int NW, bool kIsK>
__device__ __forceinline__ void dma_tile(uint8_t* lds_tile, const uint16_t* base, int64_t kv_rs, int n_kv, int j0,
                                         int wave, int lane) {
#pragma unroll
  for (int r = 0; r < 16 / NW; ++r) {
    const int blk = wave + r * NW;
    const int row = 4 * blk + (lane >> 4);
    const int pc = lane & 15;
    const int c = kIsK ? k_chunk(row, pc) : v_chunk(row, pc);
    const int j = min(j0 + row, n_kv - 1);
    lds_dma16(base + (int64_t)j * kv_rs + 8 * c, lds_tile + blk * 1024);
  }
}

// Registers holding one thread's share of a K tile between its global load and
// its LDS store (the load of tile t+2 is in flight while tile t is computed):
// key kt, chunks c and c+8, i.e. both halves of 8 rotate-half pairs.
template <int ITEMS>
struct KRegs {
  u32x4 lo[ITEMS], hi[ITEMS];
};

template <int NT>
__device__ __forceinline__ void load_k(KRegs<512 / NT>& r, const uint16_t* kbase, int64_t kv_rs, int n_kv, int j0,
                                       int tid) {
#pragma unroll
  for (int it = 0; it < 512 / NT; ++it) {
    const int id = tid + it * NT;
    const int kt = id >> 3, c = id & 7;
    const int j = min(j0 + kt, n_kv - 1);
    const uint16_t* kp = kbase + (int64_t)j * kv_rs + 8 * c;
    r.lo[it] = *reinterpret_cast<const u32x4*>(kp);
    r.hi[it] = *reinterpret_cast<const u32x4*>(kp + kHalfD);
  }
}

// Registers -> LDS: K as cached and K corrected by c(j) theta.
template <int NT>
__device__ __forceinline__ void store_k(const KRegs<512 / NT>& r, uint8_t* sk, uint8_t* skg, const f32x2* s_tdelta,
                                        const f32x2* base, int j0, int g, float inv_g, int tid) {
  const int r_mod = j0 % g;
#pragma unroll
  for (int it = 0; it < 512 / NT; ++it) {
    const int id = tid + it * NT;
    const int kt = id >> 3, c = id & 7;
    *reinterpret_cast<u32x4*>(sk + kt * 256 + (k_chunk(kt, c) << 4)) = r.lo[it];
    *reinterpret_cast<u32x4*>(sk + kt * 256 + (k_chunk(kt, c + 8) << 4)) = r.hi[it];
    // c(j) = c(j0) - u with u = kt - floor((r + kt) / g), r = j0 mod g
    const int u = kt - small_div(r_mod + kt, g, inv_g);
    const f32x2* td = s_tdelta + u * kHalfD + 8 * c;
    const f32x2* bs = base + 8 * c;
    u32x4 glo, ghi;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      float y1[2], y2[2];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int e = 2 * e2 + q2;
        const f32x2 cs = cmul(bs[e], td[e]);
        const float x1 = elem(r.lo[it], e), x2 = elem(r.hi[it], e);
        const f32x2 yr = rot_pair(x1, x2, cs.x, cs.y);
        y1[q2] = yr.x;
        y2[q2] = yr.y;
      }
      glo[e2] = pack_bf16(y1[0], y1[1]);
      ghi[e2] = pack_bf16(y2[0], y2[1]);
    }
    *reinterpret_cast<u32x4*>(skg + kt * 256 + (k_chunk(kt, c) << 4)) = glo;
    *reinterpret_cast<u32x4*>(skg + kt * 256 + (k_chunk(kt, c + 8) << 4)) = ghi;
  }
}

// Raw scores q.k of one wave's 32 query rows against one 64-key tile; masked
// entries are -inf.  Lane (h, n) gets row n, keys j0 + 32kb + 16h + i.
// kInterior: every key of the tile is causal for every row of the workgroup and,
// in the bifocal mode, remote for every row -- no masks, grouped scores only.
template <int MODE, bool kInterior, int NS, bool kLean = false, class LO>
__device__ __forceinline__ void tile_scores(const uint8_t* sk, const uint8_t* skg, const LO& lo,
                                            const bf16x8 (&qf)[8], const bf16x8 (&qg)[8], int lane, int j0,
                                            int my_p, int w, bool use_base, bool use_grp, float (&x)[NS][2][16]) {
  const int h = lane >> 5;
  if constexpr (kInterior) {
    f32x16 sc[2];
    qk_tile(MODE == kModePlain ? sk : skg, lo, MODE == kModePlain ? qf : qg, sc);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[0][kb][i] = sc[kb][i];
  } else if constexpr (MODE == kModePlain) {
    f32x16 sb[2];
    qk_tile<kLean>(sk, lo, qf, sb);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        x[0][kb][i] = (my_p - (j0 + 32 * kb + 16 * h + i) >= 0) ? sb[kb][i] : -INFINITY;
  } else if constexpr (MODE == kModeBifocal) {
    // remote keys take grouped scores, local keys base scores; one 32-key block
    // at a time, so that only one block's products of each kind are live
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (use_grp) {
        const f32x16 sg = qk_block<kLean>(skg + kb * 32 * 256, lo, qg);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[0][kb][i] = (my_p - (j0 + 32 * kb + 16 * h + i) >= 0) ? sg[i] : -INFINITY;
        __builtin_amdgcn_sched_barrier(0);
      }
      if (use_base) {
        const f32x16 sb = qk_block<kLean>(sk + kb * 32 * 256, lo, qf);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dist = my_p - (j0 + 32 * kb + 16 * h + i);
          const bool local = dist >= 0 && dist < w;
          const float other = use_grp ? x[0][kb][i] : -INFINITY;
          x[0][kb][i] = local ? sb[i] : other;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    f32x16 sb[2], sg[2];
    qk_tile(sk, lo, qf, sb);
    qk_tile(skg, lo, qg, sg);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int dist = my_p - (j0 + 32 * kb + 16 * h + i);
        const bool causal = dist >= 0;
        const bool local = causal && dist < w;
        x[0][kb][i] = local ? sb[kb][i] : -INFINITY;
        x[1][kb][i] = causal ? sg[kb][i] : -INFINITY;
        x[NS - 1][kb][i] = local ? sg[kb][i] : -INFINITY;
      }
  }
}

// Online softmax, first half: running maximum and (rarely) the rescale.
// Scores stay in raw units: p = 2^(c (x - m)), c = scale * log2(e).  The
// maximum m used in the exponent is only raised, and the accumulators
// rescaled, when a row's maximum exceeds it by more than 8 / c (so p <= 2^8);
// the decision is taken for the whole wave, so most tiles skip it.  Any m
// gives the same normalised result: numerator and denominator share it.
template <int NS>
__device__ __forceinline__ void softmax_max(const float (&x)[NS][2][16], float (&m_run)[NS], float (&l_run)[NS],
                                            f32x16 (&acc)[NS][4], float scale_log2) {
  const float thr = 8.0f / scale_log2;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, x[s][kb][i]);
    mloc = half_max(mloc);
    if (__builtin_amdgcn_ballot_w64(mloc > m_run[s] + thr)) {
      const float m_new = fmaxf(m_run[s], mloc);
      const float alpha = __builtin_amdgcn_exp2f((m_run[s] - m_new) * scale_log2);
      m_run[s] = m_new;
      l_run[s] *= alpha;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[s][nb] *= alpha;
    }
  }
}

// Online softmax, second half: probabilities (bf16 pairs) and row sums.
// kF32Sum: the sums add the fp32 probabilities, so the normaliser (and the lse)
// carry fp32 rounding only.  Otherwise they add the bf16-rounded probabilities,
// the weights the P V product applies, in one v_dot2 per pair (fewer VALU
// instructions, which the single-kernel bifocal mode is bound by); the lse then
// carries the probabilities' bf16 rounding, a relative error of at most 2^-8 in
// the normaliser.
template <int NS, bool kF32Sum>
__device__ __forceinline__ void softmax_exp(const float (&x)[NS][2][16], const float (&m_run)[NS],
                                            float (&l_run)[NS], float scale_log2, uint32_t (&pk)[NS][2][8]) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float mc = -m_run[s] * scale_log2;
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[s][kb][2 * i2], scale_log2, mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[s][kb][2 * i2 + 1], scale_log2, mc));
        pk[s][kb][i2] = pack_bf16(p0, p1);
        if constexpr (kF32Sum) psum += p0 + p1;
        else psum = add_bf16_pair(pk[s][kb][i2], psum);
      }
    }
    l_run[s] += psum;
  }
}

// O^T += V^T P^T over 4 steps of 16 keys: step (kb, half) uses keys
// 32kb + 16h + 8half + e, which are output registers 8half + e of block kb.
// O^T += V^T P^T over 4 steps of 16 keys: step (kb, half) uses keys
// 32kb + 16h + 8half + e, which are output registers 8half + e of block kb.
// The V^T operand (lane (n, h): d = 32nb + n, 8 keys) comes from two
// transposed reads of the row-major V tile: lane j of each 16-lane group reads
// 4 values of d at key 4r + j/4 (r = 0, 1), columns 4(j % 4) .. 4(j % 4) + 3.
template <int NS, bool kLean = false, class LO = LaneOffsets>
__device__ __forceinline__ void pv_tile(const uint8_t* sv, const LO& lo, const uint32_t (&pk)[NS][2][8],
                                        f32x16 (&acc)[NS][4]) {
  const lds_byte* vp[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) vp[nb] = lds_opaque(lds_ptr(sv) + v_off(lo, nb));
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    const int kb = step >> 1, half = step & 1;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const u32x2 t0 = lds_read_tr16(vp[nb] + (32 * kb + 8 * half) * 256);
      const u32x2 t1 = lds_read_tr16(vp[nb] + (32 * kb + 8 * half + 4) * 256);
      const u32x4 vf = {t0.x, t0.y, t1.x, t1.y};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 pf = {pk[s][kb][4 * half + 0], pk[s][kb][4 * half + 1], pk[s][kb][4 * half + 2],
                          pk[s][kb][4 * half + 3]};
        acc[s][nb] = mfma32(as_bf16x8(vf), as_bf16x8(pf), acc[s][nb]);
      }
      if constexpr (kLean) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Software pipeline over key tiles (one barrier per tile).  Iteration t:
//   global loads of tile t+2 -> registers          (in flight during the rest)
//   softmax maximum / rescale on the scores of tile t (computed last iteration)
//   scores of tile t+1 (QK MFMAs)  | probabilities of tile t (VALU)
//   O += P V for tile t (PV MFMAs)  | registers of tile t+2 -> LDS (VALU: the
//                                     correction rotation, V transposition)
//   barrier
// K tiles are double-buffered (t+1 read, t+2 written), V tiles triple-buffered
// (t read, t+1 waiting, t+2 written).
template <int MODE, int NW>
__global__ __launch_bounds__(NW * 64, 1) void prefill_kernel(const PrefillArgs a) {
  constexpr int NT = NW * 64;
  constexpr bool kGrouped = MODE != kModePlain;
  constexpr int NS = (MODE == kModePasses) ? 3 : 1;
  constexpr int kTileBytes = kBN * 256;

  __shared__ __attribute__((aligned(16))) uint8_t s_k[2 * kTileBytes];                  // K as cached
  __shared__ __attribute__((aligned(16))) uint8_t s_kg[kGrouped ? 2 * kTileBytes : 16];  // corrected K
  __shared__ __attribute__((aligned(16))) uint8_t s_v[3 * kTileBytes];                  // V row-major
  __shared__ f32x2 s_tdelta[kGrouped ? 65 * kHalfD : 1];  // E(-u theta_d), u = 0..64
  __shared__ f32x2 s_base[kGrouped ? 3 * kHalfD : 1];     // E(c(j0) theta_d) of tile u at u % 3

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;

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
  const int my_row = row0 + (lane & 31);
  const bool row_ok = my_row < a.n_q;
  const int my_p = row_ok ? pos_off + my_row : -1;  // -1: no causal key at all

  const int64_t q_rs = (int64_t)a.hq * kD;
  const int64_t kv_rs = (int64_t)a.hkv * kD;
  const uint16_t* kbase = a.k + (int64_t)b * a.n_kv * kv_rs + (int64_t)kvh * kD;
  const uint16_t* vbase = a.v + (int64_t)b * a.n_kv * kv_rs + (int64_t)kvh * kD;

  KRegs<512 / NT> kregs;
  if constexpr (kGrouped) load_k<NT>(kregs, kbase, kv_rs, a.n_kv, 0, tid);

  // ---- query fragments (B operand of S^T): row my_row, d = 16kk + 8h + e ----
  bf16x8 qf[8];
  bf16x8 qg[8];
  const uint16_t* qrow = a.q + ((int64_t)b * a.n_q + (row_ok ? my_row : 0)) * q_rs + (int64_t)hq * kD;
  auto qraw_reload = [&](int kk) -> u32x4 {
    return row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0};
  };
  {
    u32x4 raw[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      raw[kk] = qraw_reload(kk);
      qf[kk] = as_bf16x8(raw[kk]);
    }
    if constexpr (kGrouped) {
      // q^g = rot(q, c(p) theta), rounded to bf16
      const long long cq = row_ok ? (long long)(my_p / a.g) - my_p + a.q_shift : 0;
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
            const f32x2 yr = rot_pair(x1, x2, cs.x, cs.y);
            y1[t] = yr.x;
            y2[t] = yr.y;
          }
          lo[e2] = pack_bf16(y1[0], y1[1]);
          hi[e2] = pack_bf16(y2[0], y2[1]);
        }
        qg[kk] = as_bf16x8(lo);
        qg[kk + 4] = as_bf16x8(hi);
      }
    }
  }

  auto base_angles = [&](int tt, int slot) {  // E(c(j0) theta_d) of tile tt, by threads 0..63
    const int j = tt * kBN;
    s_base[slot * kHalfD + tid] = rot_cs((long long)(j / a.g) - j, a.theta_rev[tid]);
  };
  // Tile tt into LDS: V (and, plain, K) by direct copies issued here; in the
  // bifocal modes K comes from registers loaded earlier, corrected on the way.
  auto dma = [&](int tt, int ks, int vs) {
    dma_tile<NW, false>(s_v + vs * kTileBytes, vbase, kv_rs, a.n_kv, tt * kBN, wave, lane);
    if constexpr (!kGrouped) dma_tile<NW, true>(s_k + ks * kTileBytes, kbase, kv_rs, a.n_kv, tt * kBN, wave, lane);
  };
  auto stage_k = [&](int tt, int ks, int vs) {
    if constexpr (kGrouped)
      store_k<NT>(kregs, s_k + ks * kTileBytes, s_kg + ks * kTileBytes, s_tdelta, s_base + vs * kHalfD, tt * kBN,
                  a.g, a.inv_g, tid);
  };

  if constexpr (kGrouped) {
    for (int idx = tid; idx < 65 * kHalfD; idx += NT)
      s_tdelta[idx] = rot_cs(-(long long)(idx >> 6), a.theta_rev[idx & 63]);
    if (tid < kHalfD)
      for (int t = 0; t < 3; ++t) base_angles(min(t, ntiles - 1), t);
    __syncthreads();
  }
  dma(0, 0, 0);
  stage_k(0, 0, 0);
  if (ntiles > 1) {
    dma(1, 1, 1);
    if constexpr (kGrouped) load_k<NT>(kregs, kbase, kv_rs, a.n_kv, kBN, tid);
    stage_k(1, 1, 1);
  }
  wait_vmem();

  float m_run[NS], l_run[NS];
  f32x16 acc[NS][4];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    m_run[s] = kNegBig;
    l_run[s] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[s][nb] = f32x16{};
  }

  // Interior tiles: causal for every row of the workgroup and (bifocal) remote
  // for every row: keys j <= P0 - W with P0 the first row's position.
  const int p0_wg = pos_off + row0_wg;
  int n_interior = 0;
  if constexpr (MODE == kModePlain) n_interior = min(ntiles, max(0, (p0_wg + 1) / kBN));
  if constexpr (MODE == kModeBifocal) n_interior = min(ntiles, max(0, (p0_wg - a.w + 1) / kBN));

  const LaneOffsets lofs = lane_offsets(lane);
  auto wave_uses = [&](int t) { return wave_rows && t * kBN <= wp_hi; };
  auto scores = [&](int t, auto interior_tag, float (&xs)[NS][2][16]) {
    constexpr bool kInt = decltype(interior_tag)::value;
    const int j0 = t * kBN;
    bool use_base = true, use_grp = false;
    if constexpr (MODE == kModeBifocal) {
      use_grp = (j0 <= wp_hi - a.w);                 // a remote key for some row of the wave
      use_base = (j0 + kBN - 1 >= wp_lo - a.w + 1);  // a local key for some row of the wave
    }
    if constexpr (MODE == kModePasses) use_grp = true;
    tile_scores<MODE, kInt, NS>(s_k + (t & 1) * kTileBytes, s_kg + (kGrouped ? (t & 1) * kTileBytes : 0), lofs, qf,
                                qg, lane, j0, my_p, a.w, use_base, use_grp, xs);
  };

  __syncthreads();

  // Scores of the current tile live in xa or xb; steps alternate the two so
  // that no copy is needed (the loops are unrolled by two).
  float xa[NS][2][16], xb[NS][2][16];
  if (wave_uses(0)) {
    if (n_interior > 0) scores(0, std::true_type{}, xa);
    else scores(0, std::false_type{}, xa);
  }

  auto step = [&](int t, auto next_interior_tag, float (&x_cur)[NS][2][16], float (&x_next)[NS][2][16]) {
    constexpr bool kNextInterior = decltype(next_interior_tag)::value;
    // Loads and staging run unconditionally (the tile index is clamped at the
    // end: re-staging the last tile into free slots is harmless), which keeps
    // the whole step in one basic block apart from the rare rescale.
    const int t2 = min(t + 2, ntiles - 1);
    dma(t2, t & 1, (t + 2) % 3);
    if constexpr (kGrouped) {
      load_k<NT>(kregs, kbase, kv_rs, a.n_kv, t2 * kBN, tid);
      // rotation base of tile t+3 (its slot was last read while staging tile t)
      if (tid < kHalfD) base_angles(min(t + 3, ntiles - 1), (t + 3) % 3);
    }
    // interior steps: every wave with rows uses tiles t and t+1
    const bool act = kNextInterior || wave_uses(t);
    if (act) softmax_max<NS>(x_cur, m_run, l_run, acc, a.scale_log2);
    // region 1: QK MFMAs of tile t+1 beside the exponentials of tile t
    uint32_t pk[NS][2][8];
    if (kNextInterior || (t + 1 < ntiles && wave_uses(t + 1))) scores(t + 1, next_interior_tag, x_next);
    if (act) softmax_exp<NS, true>(x_cur, m_run, l_run, a.scale_log2, pk);
    __builtin_amdgcn_sched_barrier(0);
    // region 2: PV MFMAs of tile t beside the staging of tile t+2
    if (act) pv_tile<NS>(s_v + (t % 3) * kTileBytes, lofs, pk, acc);
    stage_k(t2, t & 1, (t + 2) % 3);
    wait_vmem();
    __syncthreads();
  };

  // interior steps: t = 0 .. n_interior-2 (tile t+1 is interior)
  int t = 0;
  const int t_int_end = max(0, n_interior - 1);
  for (; t + 1 < t_int_end; t += 2) {
    step(t, std::true_type{}, xa, xb);
    step(t + 1, std::true_type{}, xb, xa);
  }
  bool in_b = false;  // current scores in xb?
  if (t < t_int_end) {
    step(t, std::true_type{}, xa, xb);
    ++t;
    in_b = true;
  }
  if constexpr (MODE == kModeBifocal) {
    // the base-RoPE query fragment is only needed from the band on
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = as_bf16x8(qraw_reload(kk));
  }
  if (!in_b) {
    for (; t + 1 < ntiles; t += 2) {
      step(t, std::false_type{}, xa, xb);
      step(t + 1, std::false_type{}, xb, xa);
    }
    if (t < ntiles) step(t, std::false_type{}, xa, xb);
  } else {
    for (; t + 1 < ntiles; t += 2) {
      step(t, std::false_type{}, xb, xa);
      step(t + 1, std::false_type{}, xa, xb);
    }
    if (t < ntiles) step(t, std::false_type{}, xb, xa);
  }

  // ---- epilogue: lane holds row my_row, columns d = 32nb + 8(i/4) + 4h + (i%4) ----
  if (!row_ok) return;
  if constexpr (MODE == kModePasses) {
    if (!a.out_abc) {
      // Merged output (no per-pass buffers): the inclusion-exclusion of the three
      // passes A (local keys, base scores), B (causal keys, grouped scores) and C
      // (local keys, grouped scores), each weighted by its own normaliser.  In
      // log2 units lse_X = m_X tau log2(e) + log2 l_X; with M the largest lse,
      // e_X = 2^(m_X tau log2(e) - M) scales pass X's unnormalised sums, so
      //   Z = e_A l_A + e_B l_B - e_C l_C,  O = (e_A acc_A + e_B acc_B - e_C acc_C) / Z,
      //   lse = (M + log2 Z) ln 2.
      // Each l_X is the sum over the row's two lane halves (a cross-lane reduction).
      float lt[NS], ml[NS], e[NS];
      float mx = -INFINITY;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        lt[s] = half_sum(l_run[s]);
        ml[s] = m_run[s] * a.scale_log2;
        if (lt[s] > 0.0f) mx = fmaxf(mx, ml[s] + __builtin_log2f(lt[s]));
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) e[s] = lt[s] > 0.0f ? __builtin_amdgcn_exp2f(ml[s] - mx) : 0.0f;
      const float z = __builtin_fmaf(e[0], lt[0], __builtin_fmaf(e[1], lt[1], -e[2] * lt[2]));
      const float inv = 1.0f / z;
      const float c0 = e[0] * inv, c1 = e[1] * inv, c2 = -e[2] * inv;
      auto merged = [&](int nb, int i) {
        return __builtin_fmaf(acc[0][nb][i], c0, __builtin_fmaf(acc[1][nb][i], c1, acc[2][nb][i] * c2));
      };
      uint16_t* o = a.out + (((int64_t)b * a.n_q + my_row) * a.hq + hq) * kD;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          u32x2 val = {pack_bf16(merged(nb, 4 * i4), merged(nb, 4 * i4 + 1)),
                       pack_bf16(merged(nb, 4 * i4 + 2), merged(nb, 4 * i4 + 3))};
          *reinterpret_cast<u32x2*>(o + 32 * nb + 8 * i4 + 4 * h) = val;
        }
      if (a.lse && h == 0) a.lse[((int64_t)b * a.hq + hq) * a.n_q + my_row] = (mx + __builtin_log2f(z)) * kLn2;
      return;
    }
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float lt = half_sum(l_run[s]);
    const bool empty = !(lt > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / lt;
    const float lse_v = empty ? -INFINITY : (m_run[s] * a.scale_log2 + __builtin_log2f(lt)) * kLn2;
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

// ---------------------------------------------------------------------------
// Ping-pong prefill (plain and bifocal).
//
// Waves 0-3 (group A) and 4-7 (group B) -- one of each per SIMD -- run the same
// per-tile program half a tile apart, separated by workgroup barriers:
//     A: | M(0) | V(0) | M(1) | V(1) | ...
//     B: |  --  | M(0) | V(0) | M(1) | ...
// M(k) is the MFMA phase (S = QK^T of tile k, O += P V of tile k-1) and V(k)
// the VALU phase (softmax of tile k, staging of half a future tile), so in
// every phase one wave of each SIMD keeps the matrix cores busy while the
// other works on the vector ALUs.  Tile t is staged from registers loaded one
// phase earlier: its key half 32..63 by group B in V(t-2), its half 0..31 by
// group A in V(t-1).  K and corrected K are double-buffered, V triple-buffered.
// ---------------------------------------------------------------------------

// One group's half (32 keys) of a tile in registers: one K item (key, chunks
// c and c+8 -- both halves of 8 rotate-half pairs) and two 16-byte V chunks.
// K items: runs of 8 lanes read the 8 chunk pairs of one key (coalesced rows).
__device__ __forceinline__ int half_tile_key(int gtid) { return gtid >> 3; }
__device__ __forceinline__ int half_tile_chunk(int gtid) { return gtid & 7; }
struct HalfTile {
  u32x4 klo, khi, v0, v1;
};

// Staging loads go through buffer resources built per tile (scalar registers:
// base = key j0 of this head, range = the keys that exist), so each lane only
// keeps constant byte offsets and rows past n_kv read as zeros (finite, and
// their probabilities are exactly zero).  The range check covers the VGPR
// offset plus the instruction offset but not the scalar offset, so every row
// offset is carried in a VGPR.
struct StageOffsets {
  uint32_t k;   // K item: key kt, chunk c (and c + 8 at +128 bytes)
  uint32_t v0;  // V chunk of row `row`
  uint32_t v1;  // the same chunk of row + 16
};

__device__ __forceinline__ StageOffsets stage_offsets(int64_t kv_rs, int half, int gtid) {
  StageOffsets o;
  const uint32_t row_bytes = (uint32_t)(kv_rs * 2);
  o.k = (uint32_t)(32 * half + half_tile_key(gtid)) * row_bytes + 16u * (uint32_t)half_tile_chunk(gtid);
  o.v0 = (uint32_t)(32 * half + (gtid >> 4)) * row_bytes + 16u * (uint32_t)(gtid & 15);
  o.v1 = o.v0 + 16u * row_bytes;
  return o;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* head_base, int64_t kv_rs, int n_kv,
                                                            int j0) {
  const int rows = min(kBN, n_kv - j0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(head_base + (int64_t)j0 * kv_rs), (short)0,
                                           (int)(rows * kv_rs * 2), 0x00020000);
}

__device__ __forceinline__ void load_half(HalfTile& r, const uint16_t* kbase, const uint16_t* vbase, int64_t kv_rs,
                                          int n_kv, int j0, const StageOffsets& so) {
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase, kv_rs, n_kv, j0);
  const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vbase, kv_rs, n_kv, j0);
  r.klo = __builtin_amdgcn_raw_buffer_load_b128(rk, so.k, 0, 0);
  r.khi = __builtin_amdgcn_raw_buffer_load_b128(rk, so.k + 128, 0, 0);
  r.v0 = __builtin_amdgcn_raw_buffer_load_b128(rv, so.v0, 0, 0);
  r.v1 = __builtin_amdgcn_raw_buffer_load_b128(rv, so.v1, 0, 0);
}

__device__ __forceinline__ void load_k_only(HalfTile& r, const uint16_t* kbase, int64_t kv_rs, int n_kv, int j0,
                                            const StageOffsets& so) {
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase, kv_rs, n_kv, j0);
  r.klo = __builtin_amdgcn_raw_buffer_load_b128(rk, so.k, 0, 0);
  r.khi = __builtin_amdgcn_raw_buffer_load_b128(rk, so.k + 128, 0, 0);
}
__device__ __forceinline__ void store_k_only(const HalfTile& r, uint8_t* sk, int half, int gtid) {
  const int kt = 32 * half + half_tile_key(gtid), c = half_tile_chunk(gtid);
  *reinterpret_cast<u32x4*>(sk + kt * 256 + (k_chunk(kt, c) << 4)) = r.klo;
  *reinterpret_cast<u32x4*>(sk + kt * 256 + (k_chunk(kt, c + 8) << 4)) = r.khi;
}

// Registers -> LDS: the group's half of a tile, K (as staged) and V.
__device__ __forceinline__ void store_half(const HalfTile& r, uint8_t* sk, uint8_t* sv, int half, int gtid) {
  {
    const int row = 32 * half + (gtid >> 4), c = gtid & 15;
    *reinterpret_cast<u32x4*>(sv + row * 256 + (v_chunk(row, c) << 4)) = r.v0;
    *reinterpret_cast<u32x4*>(sv + (row + 16) * 256 + (v_chunk(row + 16, c) << 4)) = r.v1;
  }
  const int kt = 32 * half + half_tile_key(gtid), c = half_tile_chunk(gtid);
  *reinterpret_cast<u32x4*>(sk + kt * 256 + (k_chunk(kt, c) << 4)) = r.klo;
  *reinterpret_cast<u32x4*>(sk + kt * 256 + (k_chunk(kt, c + 8) << 4)) = r.khi;
}


// Interior MFMA phase: S = K Q^T of tile k (16 MFMAs, two 32-key blocks) and,
// when kPV, O^T += V^T P^T of tile k-1 (16 MFMAs), issued alternately.  The
// LDS operands of step i + kDist are read while the MFMAs of step i run (a
// ring of kDist + 1 operand sets), and the order is pinned so the compiler does
// not hoist all 48 reads ahead of the matrix work.
// `hook(i)` runs at step i = 0..15 (a constant once unrolled), in the same
// scheduling region as that step's two MFMAs, so the work it adds issues in
// the matrix cores' shadow.
struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

template <bool kPV, typename Hook = NoHook, int kDist = 2>
__device__ __forceinline__ void mphase_interior(const uint8_t* kbuf, const uint8_t* vbuf, const LaneOffsets& lo,
                                                const bf16x8 (&q)[8], const uint32_t (&pk)[1][2][8],
                                                f32x16 (&sc)[2], f32x16 (&acc)[1][4], const Hook& hook = Hook()) {
  auto read_k = [&](int i) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(kbuf + lo.k[i >> 1] + (i & 1) * (32 * 256));
  };
  const lds_byte* vp[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) vp[nb] = kPV ? lds_opaque(lds_ptr(vbuf) + lo.v[nb]) : nullptr;
  auto read_v = [&](int i) -> u32x4 {
    const int st = i >> 2, nb = i & 3;
    const int kb = st >> 1, half = st & 1;
    const u32x2 t0 = lds_read_tr16(vp[nb] + (32 * kb + 8 * half) * 256);
    const u32x2 t1 = lds_read_tr16(vp[nb] + (32 * kb + 8 * half + 4) * 256);
    return u32x4{t0.x, t0.y, t1.x, t1.y};
  };
  u32x4 kr[kDist + 1], vr[kDist + 1];
#pragma unroll
  for (int i = 0; i < kDist; ++i) {
    kr[i] = read_k(i);
    if constexpr (kPV) vr[i] = read_v(i);
  }
  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + kDist < 16) {
      kr[(i + kDist) % (kDist + 1)] = read_k(i + kDist);
      if constexpr (kPV) vr[(i + kDist) % (kDist + 1)] = read_v(i + kDist);
    }
    const bf16x8 ka = as_bf16x8(kr[i % (kDist + 1)]);
    if (i & 1) s1 = mfma32(ka, q[i >> 1], s1);
    else s0 = mfma32(ka, q[i >> 1], s0);
    if constexpr (kPV) {
      const int st = i >> 2, nb = i & 3;
      const int kb = st >> 1, half = st & 1;
      const u32x4 pf = {pk[0][kb][4 * half], pk[0][kb][4 * half + 1], pk[0][kb][4 * half + 2],
                        pk[0][kb][4 * half + 3]};
      acc[0][nb] = mfma32(as_bf16x8(vr[i % (kDist + 1)]), as_bf16x8(pf), acc[0][nb]);
    }
    hook(i);
    __builtin_amdgcn_sched_barrier(0);
  }
  sc[0] = s0;
  sc[1] = s1;
}

// A workgroup barrier that orders this wave's LDS reads and writes (lgkmcnt)
// but not its direct V copies still in flight, which __syncthreads would wait
// for; the "memory" clobber keeps the compiler from moving memory accesses
// across it.  Each V copy is waited for by its own wave (the key loads issued
// after it) before the barrier that ends the next MFMA phase, two phases
// before the tile is first read.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt not waited for
  asm volatile("s_barrier" ::: "memory");
}

// mphase_interior for the single-kernel bifocal prefill: operands read one
// step ahead and addressed from the lane's two base offsets (LaneBase), which
// keeps ten registers free for the staging work the hook adds.
template <typename Hook>
__device__ __forceinline__ void mphase_compact(const uint8_t* kbuf, const uint8_t* vbuf, const LaneBase& lb,
                                               const bf16x8 (&q)[8], const uint32_t (&pk)[1][2][8],
                                               f32x16 (&sc)[2], f32x16 (&acc)[1][4], const Hook& hook) {
  const uint32_t kb = (uint32_t)(uintptr_t)lds_ptr(kbuf) + lb.k0;
  auto read_k = [&](int i) -> u32x4 {
    const lds_byte* p = (const lds_byte*)(uintptr_t)(kb ^ ((uint32_t)(i >> 1) << 5));
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p + (i & 1) * (32 * 256));
  };
  const uint32_t vb = (uint32_t)(uintptr_t)lds_ptr(vbuf) + lb.v0;
  const lds_byte* vp[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) vp[nb] = lds_opaque((const lds_byte*)(uintptr_t)(vb ^ ((uint32_t)nb << 6)));
  auto read_v = [&](int i) -> u32x4 {
    const int st = i >> 2, nb = i & 3;
    const int kbk = st >> 1, half = st & 1;
    const u32x2 t0 = lds_read_tr16(vp[nb] + (32 * kbk + 8 * half) * 256);
    const u32x2 t1 = lds_read_tr16(vp[nb] + (32 * kbk + 8 * half + 4) * 256);
    return u32x4{t0.x, t0.y, t1.x, t1.y};
  };
  u32x4 kr[2], vr[2];
  kr[0] = read_k(0);
  vr[0] = read_v(0);
  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + 1 < 16) {
      kr[(i + 1) & 1] = read_k(i + 1);
      vr[(i + 1) & 1] = read_v(i + 1);
    }
    const bf16x8 ka = as_bf16x8(kr[i & 1]);
    if (i & 1) s1 = mfma32(ka, q[i >> 1], s1);
    else s0 = mfma32(ka, q[i >> 1], s0);
    const int st = i >> 2, nb = i & 3;
    const int kbk = st >> 1, half = st & 1;
    const u32x4 pf = {pk[0][kbk][4 * half], pk[0][kbk][4 * half + 1], pk[0][kbk][4 * half + 2],
                      pk[0][kbk][4 * half + 3]};
    acc[0][nb] = mfma32(as_bf16x8(vr[i & 1]), as_bf16x8(pf), acc[0][nb]);
    hook(i);
    __builtin_amdgcn_sched_barrier(0);
  }
  sc[0] = s0;
  sc[1] = s1;
}

// One sequence of a variable-length batch, as the prefill kernel sees it.
struct SeqView {
  int n_q, n_kv, n_qblocks, g, q_shift;
  int64_t q0;   // first packed query row
  double rate;  // factor on theta (fractional schedule)
};

template <int MODE, bool VARLEN = false, bool QPOS = false>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(const PrefillArgs a) {
  static_assert(MODE == kModePlain || MODE == kModeBifocalPre || MODE == kModeSliding,
                "ping-pong kernel: plain, bifocal with corrected keys staged, or sliding window "
                "(the single-kernel bifocal form is prefill_fused_kernel)");
  static_assert(!(VARLEN || QPOS) || MODE == kModePlain || MODE == kModeBifocalPre,
                "variable-length batches and explicit positions: plain or bifocal");
  static_assert(!(VARLEN && QPOS), "explicit positions are for uniform batches");
  constexpr bool kSliding = MODE == kModeSliding;   // base scores on the window's keys only
  constexpr bool kGrouped = MODE != kModePlain && !kSliding;  // grouped scores on remote keys
  constexpr bool kPre = MODE == kModeBifocalPre;    // keys corrected beforehand (a.kg)
  constexpr int kTileBytes = kBN * 256;

  __shared__ __attribute__((aligned(16))) uint8_t s_k[2 * kTileBytes];                  // K as cached
  __shared__ __attribute__((aligned(16))) uint8_t s_kg[kGrouped ? 2 * kTileBytes : 16];  // corrected K
  __shared__ __attribute__((aligned(16))) uint8_t s_v[3 * kTileBytes];                  // V row-major

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: group A, 1: group B
  const int gtid = tid & 255;
  const int h = lane >> 5;

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
  // The sequence's sizes.  Uniform batches read them from the arguments where they
  // are used (the accessors below), variable-length batches from the sequence's
  // entries, clamped: lengths outside the contract give an unspecified result,
  // never an access out of range.
  SeqView sv{};
  if constexpr (VARLEN) {
    const int bv = unit / (a.grp / a.hpw) / a.hkv;
    sv.n_kv = min(max(a.kv_lens[bv], 1), a.n_kv);
    sv.q0 = min(max(a.cu_q[bv], 0), a.total_q);
    sv.n_q = min(min(max(a.cu_q[bv + 1] - sv.q0, 0), a.total_q - sv.q0), min(a.n_q, sv.n_kv));
    sv.n_qblocks = (sv.n_q + a.bm - 1) / a.bm;
    if (rank >= sv.n_qblocks) return;  // a shorter sequence: no query block here
    if constexpr (MODE == kModeBifocal || MODE == kModeBifocalPre) {
      sv.g = sched_group(sv.n_kv, a.big_l, a.w, a.sched);
      sv.q_shift = sched_q_shift(sv.g, a.w, a.sched);
      sv.rate = sched_rate(sv.n_kv, a.big_l, a.sched);
    }
  }
  // (macros, not lambdas: a lambda capturing the kernel's argument block by
  // reference makes the compiler copy it to private memory)
#define SEQ_N_Q (VARLEN ? sv.n_q : a.n_q)
#define SEQ_N_KV (VARLEN ? sv.n_kv : a.n_kv)
#define SEQ_G (VARLEN ? sv.g : a.g)
#define SEQ_Q_SHIFT (VARLEN ? sv.q_shift : a.q_shift)
#define SEQ_THETA(d) (VARLEN ? a.theta_rev[d] * sv.rate : a.theta_rev[d])
  const int qb = (VARLEN ? sv.n_qblocks : a.n_qblocks) - 1 - rank;
  const int n_hg = a.grp / a.hpw;
  const int hg = unit % n_hg;
  const int bk = unit / n_hg;
  const int kvh = bk % a.hkv;
  const int b = bk / a.hkv;
#define SEQ_Q0 (VARLEN ? sv.q0 : (int64_t)b * a.n_q)
  const int hq = kvh * a.grp + hg * a.hpw + (wave % a.hpw);
  const int row0_wg = qb * a.bm;
  const int row0 = row0_wg + (wave / a.hpw) * 32;
  const int pos_off = SEQ_N_KV - SEQ_N_Q;
  // position of query row r: explicit positions are clamped into the context
  // (positions outside the contract give an unspecified result, never an access
  // out of range); tiles are classified from the first and last rows' positions
#define SEQ_POS(r) (QPOS ? min(max(a.q_pos[(r)], 0), SEQ_N_KV - 1) : pos_off + (r))
  const int last_row_wg = min(SEQ_N_Q, row0_wg + a.bm) - 1;
  const int kend = QPOS ? SEQ_POS(last_row_wg) + 1 : pos_off + last_row_wg + 1;
  const int ntiles = (kend + kBN - 1) / kBN;

  const bool wave_rows = row0 < SEQ_N_Q;
  const int wp_lo = QPOS ? SEQ_POS(min(row0, SEQ_N_Q - 1)) : pos_off + row0;
  const int wp_hi = QPOS ? SEQ_POS(min(SEQ_N_Q, row0 + 32) - 1) : pos_off + min(SEQ_N_Q, row0 + 32) - 1;
  const int my_row = row0 + (lane & 31);
  const bool row_ok = my_row < SEQ_N_Q;
  const int my_p = row_ok ? (QPOS ? SEQ_POS(my_row) : pos_off + my_row) : -1;

  const int64_t q_rs = (int64_t)a.hq * kD;
  const int64_t kv_rs = (int64_t)a.hkv * kD;
  const uint16_t* kbase = a.k + (int64_t)b * a.n_kv * kv_rs + (int64_t)kvh * kD;
  const uint16_t* vbase = a.v + (int64_t)b * a.n_kv * kv_rs + (int64_t)kvh * kD;
  const uint16_t* kgbase = kPre ? a.kg + (int64_t)b * a.n_kv * kv_rs + (int64_t)kvh * kD : nullptr;

  // tile kinds of this workgroup's rows [p0, p1] (see the tile program below)
  const int p0_wg = QPOS ? SEQ_POS(row0_wg) : pos_off + row0_wg;
  int n_interior = 0;
  if constexpr (MODE == kModePlain) n_interior = min(ntiles, max(0, (p0_wg + 1) / kBN));
  if constexpr (kGrouped) n_interior = min(ntiles, max(0, (p0_wg - a.w + 1) / kBN));
  // sliding window: the sweep starts at the first tile holding a key inside
  // some row's window; the tiles before it are never read.  t0 is 0 otherwise.
  const int t0 = kSliding ? min(ntiles - 1, max(0, (p0_wg - a.w + 1) / kBN)) : 0;
  if constexpr (kSliding) n_interior = t0;
  // first tile whose causal keys are local for every row of the workgroup
  int t_local = n_interior;
  if constexpr (kGrouped || kSliding) {
    const int first_all_local = (QPOS ? SEQ_POS(last_row_wg) : pos_off + last_row_wg) - a.w + 1;
    t_local = first_all_local <= 0 ? 0 : (first_all_local + kBN - 1) / kBN;
    t_local = min(ntiles, max(n_interior, t_local));
  }
  // precorrected mode: interior tiles stage the corrected keys (into s_kg) in
  // place of the cached ones, edge tiles both, local tiles the cached ones
  auto k_src = [&](int t) { return (kPre && t < n_interior) ? kgbase : kbase; };
  auto k_dst = [&](int t) { return ((kPre && t < n_interior) ? s_kg : s_k) + (t & 1) * kTileBytes; };

  HalfTile regs;
  const StageOffsets soff = stage_offsets(kv_rs, grp, gtid);
  load_half(regs, k_src(t0), vbase, kv_rs, SEQ_N_KV, t0 * kBN, soff);

  bf16x8 qf[8];
  bf16x8 qg[8];
  {
    const uint16_t* qrow = a.q + (SEQ_Q0 + (row_ok ? my_row : 0)) * q_rs + (int64_t)hq * kD;
    u32x4 raw[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      raw[kk] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0};
      qf[kk] = as_bf16x8(raw[kk]);
    }
    if constexpr (kGrouped) {
      const long long cq = row_ok ? (long long)(my_p / SEQ_G) - my_p + SEQ_Q_SHIFT : 0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 lo, hi;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float y1[2], y2[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int e = 2 * e2 + t;
            const f32x2 cs = rot_cs(cq, SEQ_THETA(16 * kk + 8 * h + e));
            const float x1 = elem(raw[kk], e), x2 = elem(raw[kk + 4], e);
            const f32x2 yr = rot_pair(x1, x2, cs.x, cs.y);
            y1[t] = yr.x;
            y2[t] = yr.y;
          }
          lo[e2] = pack_bf16(y1[0], y1[1]);
          hi[e2] = pack_bf16(y2[0], y2[1]);
        }
        qg[kk] = as_bf16x8(lo);
        qg[kk + 4] = as_bf16x8(hi);
      }
    }
  }

  auto store = [&](int tt) {
    if constexpr (kPre) {
      store_half(regs, k_dst(tt), s_v + (tt % 3) * kTileBytes, grp, gtid);
      if (tt >= n_interior && tt < t_local) {  // edge tile: the corrected keys too
        HalfTile kgr;
        load_k_only(kgr, kgbase, kv_rs, SEQ_N_KV, tt * kBN, soff);
        store_k_only(kgr, s_kg + (tt & 1) * kTileBytes, grp, gtid);
      }
    } else {
      store_half(regs, s_k + (tt & 1) * kTileBytes, s_v + (tt % 3) * kTileBytes, grp, gtid);
    }
  };

  // ---- prologue: tiles 0 and 1, each group its half ----
  store(t0);
  __syncthreads();
  if (ntiles > t0 + 1) {
    load_half(regs, k_src(t0 + 1), vbase, kv_rs, SEQ_N_KV, (t0 + 1) * kBN, soff);
    store(t0 + 1);
  }

  const LaneOffsets lofs = lane_offsets(lane);
  float m_run[1] = {kNegBig}, l_run[1] = {0.0f};
  f32x16 acc[1][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[0][nb] = f32x16{};

  // tile t holds a key this wave's rows attend to (sliding: inside some row's window)
  auto uses = [&](int t) {
    return wave_rows && t * kBN <= wp_hi && (!kSliding || t * kBN + kBN - 1 >= wp_lo - a.w + 1);
  };

  float xs[1][2][16];
  uint32_t pk[1][2][8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 8; ++i) pk[0][kb][i] = 0u;
  const int ahead = grp == 0 ? 1 : 2;  // A stages tile k+1, B tile k+2

  __syncthreads();
  if (grp == 1) __syncthreads();  // group B runs one phase behind

  // One tile of the ping-pong program: phase M(k), barrier, phase V(k), barrier.
  // Tile kinds: kInterior (all keys causal and, bifocal, remote for every row
  // of the workgroup: grouped scores, no masks), kEdge (bifocal: keys local for
  // some rows and remote for others: both score kinds), kLocalFree (precorrected
  // bifocal and sliding window: every key causal and local for every row: base
  // scores, no masks, the interior tiles' interleaved MFMA phase) and kLocal (every causal
  // key local for every row: base scores with the causal mask).  Only the one
  // or two edge tiles of a sweep keep both query fragments live.
  constexpr int kInterior = 0, kEdge = 1, kLocal = 2, kLocalFree = 3;
  auto tile = [&](int k, auto kind_tag) {
    constexpr int kKind = decltype(kind_tag)::value;
    // the wave in its MFMA phase goes first when both waves of a SIMD can issue
    __builtin_amdgcn_s_setprio(2);
    const int tt = k + ahead;
    const bool do_stage = tt < ntiles && tt >= t0 + 2;
    // plain and precorrected: the staging loads fly during the MFMA phase; fused
    // bifocal: they are issued at the start of the VALU phase, so that the 16
    // registers they fill are not live across the MFMA phase, where that kernel
    // has none left
    if (do_stage) load_half(regs, k_src(tt), vbase, kv_rs, SEQ_N_KV, tt * kBN, soff);
    const uint8_t* sk = s_k + (k & 1) * kTileBytes;
    const uint8_t* skg = s_kg + (kGrouped ? (k & 1) * kTileBytes : 0);
    // V of tile k-1 (at the first tile the probabilities are zero and that
    // tile's finite V is read instead, which adds exactly nothing)
    const uint8_t* svp = s_v + ((k > t0 ? k - 1 : t0) % 3) * kTileBytes;
    if constexpr (kKind == kInterior || kKind == kLocalFree) {
      constexpr bool kG = kGrouped && kKind == kInterior;  // grouped scores on remote tiles only
      f32x16 sc[2];
      mphase_interior<true>(kG ? skg : sk, svp, lofs, kG ? qg : qf, pk, sc, acc);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) xs[0][kb][i] = sc[kb][i];
    } else {
      const int j0 = k * kBN;
      if (uses(k)) {
        if constexpr (kKind == kEdge) {
          // sliding window: keys outside every window are masked, not grouped
          const bool use_grp = !kSliding && (j0 <= wp_hi - a.w);
          const bool use_base = (j0 + kBN - 1 >= wp_lo - a.w + 1);
          tile_scores<kModeBifocal, false, 1>(sk, skg, lofs, qf, qg, lane, j0, my_p, a.w, use_base, use_grp, xs);
        } else {
          tile_scores<kModePlain, false, 1>(sk, skg, lofs, qf, qg, lane, j0, my_p, a.w, true, false, xs);
        }
      }
      if (k > t0 && uses(k - 1)) pv_tile<1>(svp, lofs, pk, acc);
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    // the row maxima belong to this phase: left to itself the compiler hoists
    // them above the barrier, where the MFMA wave would first wait for its last
    // products instead of reaching the barrier as soon as they are issued
    {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(xs[0][kb][i]));
    }
    // ---- V(k): softmax of tile k, staging ----
    if (kKind == kInterior || kKind == kLocalFree || uses(k)) {
      softmax_max<1>(xs, m_run, l_run, acc, a.scale_log2);
      // plain and sliding windows: fp32 sums (the lse carries fp32 rounding only).
      // Bifocal on corrected keys: the sums of the bf16-rounded probabilities, the
      // weights P V applies, as in the single kernel, so that every output is a
      // convex combination of value rows (an fp32 sum against bf16 weights adds an
      // error of up to 2^-8 |out|, which shows on rows with few keys)
      softmax_exp<1, MODE != kModeBifocalPre>(xs, m_run, l_run, a.scale_log2, pk);
      if constexpr (MODE == kModeBifocalPre) {
        // with only bf16 sums nothing in this phase consumes the probabilities,
        // and the compiler would sink their exponentials into the next MFMA
        // phase (measured ≈ 3% slower): they are formed here
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(pk[0][kb][i]));
      }
    }
    // the scores are dead once the probabilities exist: keep the staging after
    __builtin_amdgcn_sched_barrier(0);
    if (do_stage) {
      if constexpr (kKind == kLocal || kKind == kLocalFree)  // every later tile is local: no corrected keys
        store_half(regs, s_k + (tt & 1) * kTileBytes, s_v + (tt % 3) * kTileBytes, grp, gtid);
      else
        store(tt);
    }
    __syncthreads();
  };

  int k = t0;
  if constexpr (!kSliding)
    for (; k < n_interior; ++k) tile(k, std::integral_constant<int, kInterior>{});
  if constexpr (kGrouped) {
    // the base-RoPE query fragment is only needed from the band on
    const uint16_t* qrow = a.q + (SEQ_Q0 + (row_ok ? my_row : 0)) * q_rs + (int64_t)hq * kD;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = as_bf16x8(row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0});
  }
  if constexpr (kGrouped || kSliding)
    for (; k < t_local; ++k) tile(k, std::integral_constant<int, kEdge>{});
  if constexpr (kPre || kSliding) {
    // local tiles below the workgroup's first row need no mask, as in plain mode
    const int t_free = min(ntiles, max(k, (p0_wg + 1) / kBN));
    if constexpr (kPre) {
      // the base query fragment afresh: the copy from before the edge tiles, where
      // both fragments are live, is partly held in scratch by then
      const uint16_t* qrow = a.q + (SEQ_Q0 + (row_ok ? my_row : 0)) * q_rs + (int64_t)hq * kD;
      asm volatile("" : "+v"(qrow));
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        qf[kk] = as_bf16x8(row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0});
    }
    for (; k < t_free; ++k) tile(k, std::integral_constant<int, kLocalFree>{});
  }
  for (; k < ntiles; ++k) tile(k, std::integral_constant<int, kLocal>{});
  if (uses(ntiles - 1)) pv_tile<1>(s_v + ((ntiles - 1) % 3) * kTileBytes, lofs, pk, acc);
  if (grp == 0) __syncthreads();

  // ---- epilogue: lane holds row my_row, columns d = 32nb + 8(i/4) + 4h + (i%4) ----
  if (!row_ok) return;
  const float lt = half_sum(l_run[0]);
  const float inv = 1.0f / lt;
  const float lse_v = (m_run[0] * a.scale_log2 + __builtin_log2f(lt)) * kLn2;
  uint16_t* o = a.out + ((SEQ_Q0 + my_row) * a.hq + hq) * kD;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      u32x2 val = {pack_bf16(acc[0][nb][4 * i4] * inv, acc[0][nb][4 * i4 + 1] * inv),
                   pack_bf16(acc[0][nb][4 * i4 + 2] * inv, acc[0][nb][4 * i4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(o + 32 * nb + 8 * i4 + 4 * h) = val;
    }
  if (a.lse && h == 0) {
    // lse: [B, Hq, n_q] for uniform batches, [Hq, total_q] over the packed rows otherwise
    if constexpr (VARLEN) a.lse[(int64_t)hq * a.total_q + sv.q0 + my_row] = lse_v;
    else a.lse[((int64_t)b * a.hq + hq) * a.n_q + my_row] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// Single-kernel bifocal prefill: the keys are corrected tile by tile in LDS.
//
// The ping-pong of prefill_pp_kernel (waves 0-3 and 4-7 half a tile apart, one
// group in its MFMA phase while the other is in its VALU phase), with the
// staging of the next key tile moved into the MFMA phase: the correction
// rotation of its keys, its LDS writes and the loads of the tile after it are
// spread over the steps of the MFMA sequence.  A wave issues about one
// instruction per 4-5 cycles whatever its kind, so a VALU phase holding both
// the softmax and the rotation outlasts the other group's MFMA phase, whose
// wave leaves most of its own issue slots idle between MFMAs.  The keys'
// angles themselves (the tile's rotation base plus each key's small-angle
// table entry) are formed in the VALU phase before, which has slack.
//
// A key's angle c(j) theta_d = c(j0) theta_d - u theta_d, u = j - j0 - (floor(j
// / g) - floor(j0 / g)) < 64: the tile's base angle (exact integer c(j0), fp64
// reduction, one wave per group per tile) plus a small-angle table entry, both
// in revolutions, then the hardware cosine and sine.
//
// Tile program of each group for tile k:
//   M(k): S = K^g Q^T of tile k and O^T += V^T P^T of tile k-1 (MFMA), and the
//         group's half of tile k+1's keys into LDS (corrected, and as cached
//         for band tiles), then its half of tile k+2: the V rows copied
//         straight from memory into LDS, the keys loaded into registers.
//   V(k): the softmax of tile k, then tile k+3's rotation base and each
//         thread's 8 key angles of tile k+2.
// Tile k+1's keys are written in M(k) by both groups into the K / K^g buffers
// of tile k-1, last read in M(k-1) of both groups.  V rows sit in four slots
// (tile & 3): tile k+2's copies land in the slot of tile k-2, last read in
// M(k-1), and are complete (each wave waits for them with its key loads in
// M(k+1)) two phases before M(k+3) first reads them; the loop's barriers wait
// for LDS operations only, so the copies stay in flight across them.  Rotation
// bases sit in four slots per group (tile & 3): tile k+3's is written in V(k)
// into the slot of tile k-1, whose angles were formed in V(k-3), and read in
// V(k+1), after the barriers between.  Staging past the
// last tile re-stages the last one into slots no later phase reads, so the
// loop has no branches.
// ---------------------------------------------------------------------------
template <bool VARLEN = false, bool QPOS = false>
__global__ __launch_bounds__(512, 1) void prefill_fused_kernel(const PrefillArgs a) {
  static_assert(!(VARLEN && QPOS), "explicit positions are for uniform batches");
  constexpr int kTileBytes = kBN * 256;
  // tile buffers, 16 KB aligned (LaneBase): K as cached (band tiles) x 2 and
  // corrected K x 2; V row-major x 4 (tile t in slot t & 3), an object of its
  // own, so that the compiler waits for the copies into it only before V reads
  __shared__ __attribute__((aligned(16384))) uint8_t s_tiles[4 * kTileBytes];
  __shared__ __attribute__((aligned(16384))) uint8_t s_vt[4 * kTileBytes];
  uint8_t* const s_k = s_tiles;
  uint8_t* const s_kg = s_tiles + 2 * kTileBytes;
  uint8_t* const s_v = s_vt;
  __shared__ __attribute__((aligned(16))) float s_uang[64 * kUangStride];  // -u theta_d in revolutions, u < 64
  __shared__ __attribute__((aligned(16))) float s_base[8 * kHalfD];        // c(j0) theta_d, revolutions: [group][tile & 3]
  __shared__ double s_theta[kHalfD];                                        // theta_d / (2 pi)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: group A, 1: group B
  const int gtid = tid & 255;
  const int h = lane >> 5;

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
  SeqView sv{};
  if constexpr (VARLEN) {
    const int bv = unit / (a.grp / a.hpw) / a.hkv;
    sv.n_kv = min(max(a.kv_lens[bv], 1), a.n_kv);
    sv.q0 = min(max(a.cu_q[bv], 0), a.total_q);
    sv.n_q = min(min(max(a.cu_q[bv + 1] - sv.q0, 0), a.total_q - sv.q0), min(a.n_q, sv.n_kv));
    sv.n_qblocks = (sv.n_q + a.bm - 1) / a.bm;
    if (rank >= sv.n_qblocks) return;  // a shorter sequence: no query block here
    sv.g = sched_group(sv.n_kv, a.big_l, a.w, a.sched);
    sv.q_shift = sched_q_shift(sv.g, a.w, a.sched);
    sv.rate = sched_rate(sv.n_kv, a.big_l, a.sched);
  }
  const int qb = (VARLEN ? sv.n_qblocks : a.n_qblocks) - 1 - rank;
  const int n_hg = a.grp / a.hpw;
  const int hg = unit % n_hg;
  const int bk = unit / n_hg;
  const int kvh = bk % a.hkv;
  const int b = bk / a.hkv;
  const int hq = kvh * a.grp + hg * a.hpw + (wave % a.hpw);
  const int row0_wg = qb * a.bm;
  const int row0 = row0_wg + (wave / a.hpw) * 32;
  const int pos_off = SEQ_N_KV - SEQ_N_Q;
  const int last_row_wg = min(SEQ_N_Q, row0_wg + a.bm) - 1;
  const int kend = QPOS ? SEQ_POS(last_row_wg) + 1 : pos_off + last_row_wg + 1;
  const int ntiles = (kend + kBN - 1) / kBN;

  const bool wave_rows = row0 < SEQ_N_Q;
  const int wp_lo = QPOS ? SEQ_POS(min(row0, SEQ_N_Q - 1)) : pos_off + row0;
  const int wp_hi = QPOS ? SEQ_POS(min(SEQ_N_Q, row0 + 32) - 1) : pos_off + min(SEQ_N_Q, row0 + 32) - 1;
  const int my_row = row0 + (lane & 31);
  const bool row_ok = my_row < SEQ_N_Q;
  const int my_p = row_ok ? (QPOS ? SEQ_POS(my_row) : pos_off + my_row) : -1;
  const int w = a.w;
  const int g = SEQ_G;
  const float scale_log2 = a.scale_log2;

  const int64_t q_rs = (int64_t)a.hq * kD;
  const int64_t kv_rs = (int64_t)a.hkv * kD;
  const int n_kv = SEQ_N_KV;
  const uint16_t* kbase = a.k + (int64_t)b * a.n_kv * kv_rs + (int64_t)kvh * kD;
  const uint16_t* vbase = a.v + (int64_t)b * a.n_kv * kv_rs + (int64_t)kvh * kD;

  // tile kinds: interior (every key remote for every row of the workgroup:
  // grouped scores, no masks), edge (both score kinds), local (every causal key
  // local for every row: base scores with the causal mask)
  const int p0_wg = QPOS ? SEQ_POS(row0_wg) : pos_off + row0_wg;
  const int n_interior = min(ntiles, max(0, (p0_wg - w + 1) / kBN));
  int t_local;
  {
    const int first_all_local = (QPOS ? SEQ_POS(last_row_wg) : pos_off + last_row_wg) - w + 1;
    t_local = first_all_local <= 0 ? 0 : (first_all_local + kBN - 1) / kBN;
    t_local = min(ntiles, max(n_interior, t_local));
  }
  // local tiles below the workgroup's first row (every key causal for every
  // row) need no mask: they run the interior tiles' code on the keys staged
  // with a zero rotation (so exactly as cached) and the base-RoPE query
  const int t_free = min(ntiles, max(t_local, (p0_wg + 1) / kBN));

  // tables first, while few values are live
  if (tid < kHalfD) s_theta[tid] = SEQ_THETA(tid);
#pragma unroll 1
  for (int idx = tid; idx < 64 * kHalfD; idx += 512)
    s_uang[(idx >> 6) * kUangStride + (idx & 63)] = rev_reduce(-(idx >> 6), SEQ_THETA(idx & 63));

  // V rows go from memory straight into their LDS slot: this wave's 8 rows of
  // the group's half of a tile, two 16-byte copies per lane (lane l: row 4r +
  // l / 16, LDS position l % 16, so it fetches chunk v_chunk(row, l % 16))
  typedef __attribute__((address_space(3))) void lds_void;
  auto copy_v = [&](int tt, const __amdgpu_buffer_rsrc_t rv) {
    int t = lane;  // offsets formed here rather than kept live
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 32 * grp + 8 * (wave & 3) + 4 * r + (t >> 4);
      const uint32_t vo = (uint32_t)row * (uint32_t)(kv_rs * 2) + 16u * (uint32_t)v_chunk(row, t & 15);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (lds_void*)(s_v + (tt & 3) * kTileBytes + (32 * grp + 8 * (wave & 3) + 4 * r) * 256), 16, (int)vo,
          0, 0, 0);
    }
  };
  HalfTile regs;
  const StageOffsets soff = stage_offsets(kv_rs, grp, gtid);
  copy_v(0, tile_rsrc(vbase, kv_rs, n_kv, 0));
  load_k_only(regs, kbase, kv_rs, n_kv, 0, soff);

  // this lane's share of its query row as stored (the address made opaque, so
  // that the loads stay where they are written)
  auto load_qraw = [&](u32x4 (&raw)[8]) {
    const uint16_t* qrow = a.q + (SEQ_Q0 + (row_ok ? my_row : 0)) * q_rs + (int64_t)hq * kD + 8 * h;
    asm volatile("" : "+v"(qrow));
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      raw[kk] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk) : u32x4{0, 0, 0, 0};
  };
  // q^g = rot(q, c(p) theta), rounded to bf16
  auto correct_q = [&](const u32x4 (&raw)[8], bf16x8 (&dst)[8]) {
    const long long cq = row_ok ? (long long)(my_p / g) - my_p + SEQ_Q_SHIFT : 0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 lo, hi;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float y1[2], y2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int e = 2 * e2 + t;
          const f32x2 cs = rot_cs(cq, SEQ_THETA(16 * kk + 8 * h + e));
          const f32x2 yr = rot_pair(elem(raw[kk], e), elem(raw[kk + 4], e), cs.x, cs.y);
          y1[t] = yr.x;
          y2[t] = yr.y;
        }
        lo[e2] = pack_bf16(y1[0], y1[1]);
        hi[e2] = pack_bf16(y2[0], y2[1]);
      }
      dst[kk] = as_bf16x8(lo);
      dst[kk + 4] = as_bf16x8(hi);
    }
  };
  // the query fragment: corrected (interior and edge tiles), then base-RoPE
  // (local tiles; edge tiles read that one afresh)
  bf16x8 qg[8];
  {
    u32x4 raw[8];
    load_qraw(raw);
    correct_q(raw, qg);
  }

  // ---- staging of this group's half of tile tt: 16 steps, run one per MFMA
  // step of an interior tile's MFMA phase, or back to back otherwise: the keys
  // as cached where needed (step 0), one corrected pair on every odd step (its
  // angle formed in the VALU phase before), and at step 15 the corrected keys'
  // LDS writes and the next tile's V copies and key loads.  Spreading the
  // rotations over the phase measured about 1% faster than eight consecutive
  // steps ----
  // this thread: key kt = 32 grp + gtid / 8 of the tile, rotate-half pairs 8c .. 8c+7
  const int kc = half_tile_chunk(gtid);
  // LDS byte offset of this thread's K rows within a tile (kept live: it is
  // cheaper than forming it twice per tile): chunks c and c + 8 differ in bit
  // 3 of the swizzled chunk only (offset ^ 128)
  const uint32_t kw0 = (uint32_t)((32 * grp + half_tile_key(gtid)) * 256 +
                                  (k_chunk(32 * grp + half_tile_key(gtid), half_tile_chunk(gtid)) << 4));
  const uint32_t ug = (uint32_t)g;
  // floor(n / g) for the n = r + kt < g + 64 of the rotation table index,
  // without a division or a branch: the high word of n * ceil(2^32 / g), exact
  // while n g < 2^32 (the error n (ceil(2^32/g) - 2^32/g) / 2^32 < 1/g stays
  // below the gap of n/g to the next integer), for 2 <= g <= kMagicMaxG; n for
  // g = 1 (magic 0, n added once); (n >= g) above (magic 0, n < 2g)
  constexpr uint32_t kMagicMaxG = 65472;  // (g + 63) g < 2^32
  const uint32_t g_magic = (g > 1 && ug <= kMagicMaxG) ? (uint32_t)((0x100000000ull + ug - 1) / ug) : 0u;
  const uint32_t g_one = g == 1 ? 1u : 0u;
  const uint32_t g_cmp = ug > kMagicMaxG ? ug : 0xffffffffu;
  auto floor_div_g = [&](uint32_t n) -> uint32_t {
    return __umulhi(n, g_magic) + n * g_one + (n >= g_cmp ? 1u : 0u);
  };
  // the same with g = 1's scalars for local tiles (zero rotation: u = 0)
  auto floor_div_sel = [&](uint32_t n, bool zero) -> uint32_t {
    const uint32_t gm = zero ? 0u : g_magic, go = zero ? 1u : g_one, gc = zero ? 0xffffffffu : g_cmp;
    return __umulhi(n, gm) + n * go + (n >= gc ? 1u : 0u);
  };
  // per-tile scalars, advanced once per tile: the tile whose loads and key
  // angles are prepared next (ld_t, its j0 = 64 ld_t, ld_r = j0 mod g, ld_q =
  // floor(j0 / g)); ld_t stops at the last tile (staging past it re-stages the
  // last tile into unread slots)
  const uint32_t r64 = (uint32_t)kBN % ug, q64 = (uint32_t)kBN / ug;
  int ld_t = 0;
  uint32_t ld_r = 0, ld_q = 0;
  const uint16_t* ld_k = kbase;  // the tile's first K and V rows
  const uint16_t* ld_v = vbase;
  auto advance_ld = [&]() {
    if (ld_t < ntiles - 1) {
      ++ld_t;
      ld_k += kBN * kv_rs;
      ld_v += kBN * kv_rs;
      ld_r += r64;
      ld_q += q64;
      if (ld_r >= ug) {
        ld_r -= ug;
        ++ld_q;
      }
    }
  };
  float ang8[8];  // this thread's 8 key angles (revolutions) for the tile staged next
  float ylo[2], yhi[2];
  // rotation base of tile tt (clamped to the last tile) into slot tt & 3, by
  // the group's first 64 threads; q = floor(64 t / g)
  auto base_angles = [&](int tt, int t_c, uint32_t q_c) {
    int t = gtid;  // the address formed here rather than kept live
    asm volatile("" : "+v"(t));
    s_base[(4 * grp + (tt & 3)) * kHalfD + t] = rev_reduce((int)q_c - t_c * kBN, s_theta[t]);
  };
  // the tile after ld_t (clamped), one tile ahead of the angle preparation
  auto base_ahead = [&](int tt) {
    const bool more = ld_t < ntiles - 1;
    const int t1 = more ? ld_t + 1 : ld_t;
    const uint32_t q1 = ld_q + (more ? q64 + (ld_r + r64 >= ug ? 1u : 0u) : 0u);
    // local tiles: base 0 (c = q - 64 t is zeroed)
    base_angles(tt, t1, t1 >= t_local ? (uint32_t)(t1 * kBN) : q1);
  };
  // kRot: tile tt needs corrected keys; kCached: it needs the keys as cached
  auto stage_step = [&](int tt, int i, auto rot_tag, auto cached_tag) {
    constexpr bool kRot = decltype(rot_tag)::value, kCached = decltype(cached_tag)::value;
    if constexpr (kRot) {
      if (i & 1) {  // pair e = (i - 1) / 2 on every other step: c(j0) theta_d - u theta_d
        const int e = i >> 1;
        const float ang = ang8[e];
        const f32x2 cs = {__builtin_amdgcn_cosf(ang), __builtin_amdgcn_sinf(ang)};
        const f32x2 yr = rot_pair(elem(regs.klo, e), elem(regs.khi, e), cs.x, cs.y);
        ylo[e & 1] = yr.x;
        yhi[e & 1] = yr.y;
        if (e & 1) {
          // pairs e-1 and e came from word e/2 of each half: the corrected pair
          // replaces it in place (the keys as cached, where needed, are already
          // in LDS)
          regs.klo[e >> 1] = pack_bf16(ylo[0], ylo[1]);
          regs.khi[e >> 1] = pack_bf16(yhi[0], yhi[1]);
        }
      }
      if (i == 15) {
        uint8_t* skg = s_kg + (tt & 1) * kTileBytes;
        *reinterpret_cast<u32x4*>(skg + kw0) = regs.klo;
        *reinterpret_cast<u32x4*>(skg + (kw0 ^ 128u)) = regs.khi;
      }
    }
    if constexpr (kCached) {
      if (i == 0) {  // before the rotation overwrites them
        uint8_t* sk = s_k + (tt & 1) * kTileBytes;
        *reinterpret_cast<u32x4*>(sk + kw0) = regs.klo;
        *reinterpret_cast<u32x4*>(sk + (kw0 ^ 128u)) = regs.khi;
      }
    }
    if (i == 15) {
      // last, after any reload of the phase (a reload issued after these loads
      // would wait for them); the lane's load offsets are formed here rather
      // than kept live through the loop
      int t = gtid;
      asm volatile("" : "+v"(t));
      // buffer resources over the tile's rows that exist (rows past n_kv read zeros)
      const int nbytes = (int)(min(kBN, n_kv - ld_t * kBN) * kv_rs * 2);
      copy_v(tt + 1, __builtin_amdgcn_make_buffer_rsrc((void*)ld_v, (short)0, nbytes, 0x00020000));
      const StageOffsets so = stage_offsets(kv_rs, grp, t);
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)ld_k, (short)0, nbytes, 0x00020000);
      regs.klo = __builtin_amdgcn_raw_buffer_load_b128(rk, so.k, 0, 0);
      regs.khi = __builtin_amdgcn_raw_buffer_load_b128(rk, so.k + 128, 0, 0);
    }
  };
  // this thread's 8 key angles for tile tt, whose j0 mod g is r: the tile's
  // rotation base (slot tt & 3) plus the small-angle row of c(j) = c(j0) - u,
  // u = kt - floor((r + kt) / g)
  auto angle_row = [&](int tt, uint32_t r) {
    int t = gtid;  // kt formed here rather than kept live
    asm volatile("" : "+v"(t));
    const int key = 32 * grp + half_tile_key(t);
    const bool zero = min(tt, ntiles - 1) >= t_local;  // a local tile: u = 0, base 0
    const int u = key - (int)floor_div_sel((zero ? 0u : r) + (uint32_t)key, zero);
    const float* ua = s_uang + u * kUangStride + 8 * kc;
    const float* bs = s_base + (4 * grp + (tt & 3)) * kHalfD + 8 * kc;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const f32x4 uv = *reinterpret_cast<const f32x4*>(ua + 4 * b);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bs + 4 * b);
#pragma unroll
      for (int e = 0; e < 4; ++e) ang8[4 * b + e] = bv[e] + uv[e];
    }
  };
  // after the staging of a tile: the next one's scalars
  auto next_stage = [&]() {
    advance_ld();
  };
  constexpr int kStageSteps = 16;
  using TT = std::true_type;
  using FF = std::false_type;

  // ---- prologue: the rotation bases of tiles 0-2, tile 0 staged, the loads
  // and the key angles of tile 1 ----
  __syncthreads();  // theta table
  if (gtid < 64) {  // rotation bases of tiles 0, 1, 2
#pragma unroll 1
    for (int t = 0; t < 3; ++t) {
      const int t_c = min(t, ntiles - 1);
      base_angles(t, t_c, t_c >= t_local ? (uint32_t)(t_c * kBN) : (uint32_t)(t_c * kBN) / ug);
    }
  }
  advance_ld();  // the prologue's loads are tile 1's
  __syncthreads();
  angle_row(0, 0u);
#pragma unroll
  for (int i = 0; i < kStageSteps; ++i) {
    if (n_interior > 0 || (t_local == 0 && t_free > 0)) stage_step(0, i, TT{}, FF{});
    else if (t_local > 0) stage_step(0, i, TT{}, TT{});
    else stage_step(0, i, FF{}, TT{});
  }
  angle_row(1, ld_r);
  next_stage();

  const LaneBase lbase = lane_base(lane);
  float m_run[1] = {kNegBig}, l_run[1] = {0.0f};
  f32x16 acc[1][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[0][nb] = f32x16{};
  auto uses = [&](int t) { return wave_rows && t * kBN <= wp_hi; };
  float xs[1][2][16];
  uint32_t pk[1][2][8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 8; ++i) pk[0][kb][i] = 0u;

  __syncthreads();
  if (grp == 1) __syncthreads();  // group B runs one phase behind

  constexpr int kInterior = 0, kEdge = 1, kLocal = 2;

  // tile k of kind KK, staging tile k + 1 of kind KT
  auto tile = [&](int k, auto kk_tag, auto kt_tag) {
    constexpr int KK = decltype(kk_tag)::value, KT = decltype(kt_tag)::value;
    using RotT = std::integral_constant<bool, KT != kLocal>;
    using CachedT = std::integral_constant<bool, KT != kInterior>;
    __builtin_amdgcn_s_setprio(2);
    const uint8_t* sk = s_k + (k & 1) * kTileBytes;
    const uint8_t* skg = s_kg + (k & 1) * kTileBytes;
    // V of tile k-1 (at tile 0 the probabilities are zero and tile 0's finite V is read)
    const uint8_t* svp = s_v + ((k > 0 ? k - 1 : 0) & 3) * kTileBytes;
    if constexpr (KK == kInterior) {
      f32x16 sc[2];
      auto hook = [&](int i) {
        if (i < kStageSteps) stage_step(k + 1, i, RotT{}, CachedT{});
      };
      // operands read one step ahead: the staging work makes a step long enough
      // to cover the LDS latency, and the two registers sets saved are needed.
      // (Unmasked local tiles come here too: their keys were staged into the
      // corrected buffer with a zero rotation, and qg then holds the base query.)
      mphase_compact(skg, svp, lbase, qg, pk, sc, acc, hook);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) xs[0][kb][i] = sc[kb][i];
    } else {
      const int j0 = k * kBN;
      if (uses(k)) {
        if constexpr (KK == kEdge) {
          const bool use_grp = j0 <= wp_hi - w;
          const bool use_base = j0 + kBN - 1 >= wp_lo - w + 1;
          // an edge tile (one or two per workgroup) reads the base-RoPE query
          // fragment afresh: it and the corrected one do not both fit in
          // registers across the band
          bf16x8 qfe[8];
          {
            u32x4 raw[8];
            load_qraw(raw);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) qfe[kk] = as_bf16x8(raw[kk]);
          }
          tile_scores<kModeBifocal, false, 1, true>(sk, skg, lbase, qfe, qg, lane, j0, my_p, w, use_base, use_grp,
                                                    xs);
        } else {
          tile_scores<kModePlain, false, 1>(sk, skg, lbase, qg, qg, lane, j0, my_p, w, true, false, xs);  // qg: base-RoPE by then
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (k > 0 && uses(k - 1)) pv_tile<1, KK == kEdge>(svp, lbase, pk, acc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kStageSteps; ++i) stage_step(k + 1, i, RotT{}, CachedT{});
    }
    lds_barrier();
    __builtin_amdgcn_s_setprio(0);
    // the row maxima belong to the VALU phase (the MFMA wave reaches the barrier
    // as soon as its last products are issued)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(xs[0][kb][i]));
    // ---- V(k): softmax of tile k ----
    if (KK == kInterior || uses(k)) {
      softmax_max<1>(xs, m_run, l_run, acc, scale_log2);
      softmax_exp<1, false>(xs, m_run, l_run, scale_log2, pk);
    }
    // tile k+3's rotation base, by the group's first wave, and for tile k+2,
    // staged in the next MFMA phase, each thread's 8 key angles (its r is
    // ld_r).  This phase has slack; in the MFMA phase the table reads and the
    // additions measured about 1% slower
    if (gtid < 64) base_ahead(k + 3);
    angle_row(k + 2, ld_r);
    next_stage();
    lds_barrier();
  };

  // tile k+1's kind decides its staging: corrected keys (interior tiles, and
  // unmasked local tiles with a zero rotation), both kinds (edge) or the keys
  // as cached (masked local tiles)
  using KI = std::integral_constant<int, kInterior>;
  using KE = std::integral_constant<int, kEdge>;
  using KL = std::integral_constant<int, kLocal>;
  int k = 0;
  for (; k + 1 < n_interior; ++k) tile(k, KI{}, KI{});
  if (k < n_interior) {
    if (k + 1 < t_local) tile(k, KI{}, KE{});
    else if (k + 1 < t_free) tile(k, KI{}, KI{});
    else tile(k, KI{}, KL{});
    ++k;
  }
  for (; k < t_local; ++k) {
    if (k + 1 < t_local) tile(k, KE{}, KE{});
    else if (k + 1 < t_free) tile(k, KE{}, KI{});
    else tile(k, KE{}, KL{});
  }
  // from here on the query fragment is the base-RoPE one (the corrected one is dead)
  {
    u32x4 raw[8];
    load_qraw(raw);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qg[kk] = as_bf16x8(raw[kk]);
  }
  for (; k + 1 < t_free; ++k) tile(k, KI{}, KI{});
  if (k < t_free) {
    tile(k, KI{}, KL{});
    ++k;
  }
  for (; k < ntiles; ++k) tile(k, KL{}, KL{});
  // the V copies of the tiles staged past the last are still in flight: none
  // may land after the workgroup ends
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (uses(ntiles - 1)) pv_tile<1>(s_v + ((ntiles - 1) & 3) * kTileBytes, lane_expand(lbase), pk, acc);
  if (grp == 0) __syncthreads();

  // ---- epilogue: lane holds row my_row, columns d = 32nb + 8(i/4) + 4h + (i%4) ----
  if (!row_ok) return;
  const float lt = half_sum(l_run[0]);
  const float inv = 1.0f / lt;
  const float lse_v = (m_run[0] * scale_log2 + __builtin_log2f(lt)) * kLn2;
  uint16_t* o = a.out + ((SEQ_Q0 + my_row) * a.hq + hq) * kD;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      u32x2 val = {pack_bf16(acc[0][nb][4 * i4] * inv, acc[0][nb][4 * i4 + 1] * inv),
                   pack_bf16(acc[0][nb][4 * i4 + 2] * inv, acc[0][nb][4 * i4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(o + 32 * nb + 8 * i4 + 4 * h) = val;
    }
  if (a.lse && h == 0) {
    if constexpr (VARLEN) a.lse[(int64_t)hq * a.total_q + sv.q0 + my_row] = lse_v;
    else a.lse[((int64_t)b * a.hq + hq) * a.n_q + my_row] = lse_v;
  }
}

#undef SEQ_N_Q
#undef SEQ_POS
#undef SEQ_N_KV
#undef SEQ_G
#undef SEQ_Q_SHIFT
#undef SEQ_THETA
#undef SEQ_Q0

// ---------------------------------------------------------------------------
// Corrected keys of the whole cache, for the precorrected mode:
// k^g_j = rot(k_j, c(j) theta), c(j) = floor(j / g) - j, written in the layout
// of k.  Thread (row, c) handles rotate-half pairs 8c .. 8c+7 of one cached key
// row for every KV head: the 8 angles are reduced in fp64 once and reused.
// ---------------------------------------------------------------------------
struct CorrectArgs {
  const uint16_t* k;
  uint16_t* kg;
  int64_t rows;  // batch * n_kv
  int32_t n_kv, hkv, g;
  double theta_rev[kHalfD];
  // variable-length batches: keys per sequence (rows past them are skipped), with
  // g and the rate taken per sequence; null for uniform batches
  const int32_t* kv_lens;
  int64_t big_l;
  int32_t w, sched;
};

template <bool VARLEN>
__global__ __launch_bounds__(256) void correct_keys_kernel(const CorrectArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int c = threadIdx.x & 7;
  if (row >= a.rows) return;
  const int j = (int)(row % a.n_kv);
  f32x2 cs[8];
  if constexpr (VARLEN) {
    const int s_b = min(max(a.kv_lens[row / a.n_kv], 1), a.n_kv);
    if (j >= s_b) return;  // past the sequence's keys: never read
    const int g = sched_group(s_b, a.big_l, a.w, a.sched);
    const double rate = sched_rate(s_b, a.big_l, a.sched);
    const long long cj = (long long)(j / g) - j;
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[e] = rot_cs(cj, a.theta_rev[8 * c + e] * rate);
  } else {
    const long long cj = (long long)(j / a.g) - j;
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[e] = rot_cs(cj, a.theta_rev[8 * c + e]);
  }
  for (int hh = 0; hh < a.hkv; ++hh) {
    const int64_t base = (row * a.hkv + hh) * kD + 8 * c;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(a.k + base);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(a.k + base + kHalfD);
    u32x4 glo, ghi;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      float y1[2], y2[2];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int e = 2 * e2 + q2;
        const float x1 = elem(lo, e), x2 = elem(hi, e);
        const f32x2 yr = rot_pair(x1, x2, cs[e].x, cs[e].y);
        y1[q2] = yr.x;
        y2[q2] = yr.y;
      }
      glo[e2] = pack_bf16(y1[0], y1[1]);
      ghi[e2] = pack_bf16(y2[0], y2[1]);
    }
    *reinterpret_cast<u32x4*>(a.kg + base) = glo;
    *reinterpret_cast<u32x4*>(a.kg + base + kHalfD) = ghi;
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
  a.kg = static_cast<const uint16_t*>(p.kg);
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
  a.q_shift = p.q_shift;
  a.inv_g = 1.0f / (float)p.group;
  a.cu_q = p.cu_q;
  a.kv_lens = p.kv_lens;
  a.total_q = p.total_q;
  a.sched = p.schedule;
  a.big_l = p.pretrained_window;
  a.q_pos = p.q_pos;
  if ((p.cu_q || p.q_pos) && !(MODE == kModePlain || MODE == kModeBifocal || MODE == kModeBifocalPre))
    return hipErrorInvalidValue;
  if (p.cu_q && p.q_pos) return hipErrorInvalidValue;
  a.scale_log2 = p.softmax_scale * 1.4426950408889634f;
  // theta_d / (2 pi), times the schedule's rate (1 but for the fractional one)
  const double two_pi = 6.283185307179586476925286766559;
  for (int d = 0; d < kHalfD; ++d) a.theta_rev[d] = std::pow(p.rope_base, -2.0 * d / kD) / two_pi * p.rate;
  const long long blocks = (long long)a.n_units * a.n_qblocks;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if constexpr (MODE == kModeBifocalPre) {
    CorrectArgs c;
    c.k = a.k;
    c.kg = static_cast<uint16_t*>(p.kg);
    c.rows = (int64_t)p.batch * p.n_kv;
    c.n_kv = p.n_kv;
    c.hkv = p.n_kv_heads;
    c.g = p.group;
    for (int d = 0; d < kHalfD; ++d) c.theta_rev[d] = a.theta_rev[d];
    c.kv_lens = p.kv_lens;
    c.big_l = p.pretrained_window;
    c.w = p.local_window;
    c.sched = p.schedule;
    const long long cblocks = (c.rows + 31) / 32;
    if (cblocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (p.kv_lens)
      hipLaunchKernelGGL(correct_keys_kernel<true>, dim3((unsigned)cblocks), dim3(256), 0, stream, c);
    else
      hipLaunchKernelGGL(correct_keys_kernel<false>, dim3((unsigned)cblocks), dim3(256), 0, stream, c);
  }
  if constexpr (MODE == kModePasses)
    hipLaunchKernelGGL((prefill_kernel<MODE, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  else if constexpr (MODE == kModeBifocal) {
    if (p.cu_q)
      hipLaunchKernelGGL((prefill_fused_kernel<true>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
    else if (p.q_pos)
      hipLaunchKernelGGL((prefill_fused_kernel<false, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_fused_kernel<>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  } else if constexpr (MODE == kModePlain || MODE == kModeBifocalPre) {
    if (p.cu_q)
      hipLaunchKernelGGL((prefill_pp_kernel<MODE, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
    else if (p.q_pos)
      hipLaunchKernelGGL((prefill_pp_kernel<MODE, false, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                         a);
    else
      hipLaunchKernelGGL((prefill_pp_kernel<MODE>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  } else
    hipLaunchKernelGGL((prefill_pp_kernel<MODE>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(PrefillMode mode, const PrefillProblem& p, hipStream_t stream) {
  switch (mode) {
    case kModePlain: return launch_mode<kModePlain, 8>(p, stream);
    case kModeBifocal: return launch_mode<kModeBifocal, 8>(p, stream);
    case kModePasses: return launch_mode<kModePasses, 4>(p, stream);
    case kModeBifocalPre: return launch_mode<kModeBifocalPre, 8>(p, stream);
    case kModeSliding: return launch_mode<kModeSliding, 8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace jl
