// Split-K bifocal decode for gfx950 (MI355X): one new query per sequence
// against a KV cache that keeps original positions (ResearchPod transcript,
// cache exchange: the cache is never rewritten; the correction is applied at
// lookup).
//
// At one query (position p = s - 1) the local keys are the contiguous suffix
// [s - W, s) and the remote keys the prefix [0, s - W).  Pass B minus pass C of
// the inclusion-exclusion merge then covers exactly the remote prefix with
// grouped scores, and pass A the local suffix with base scores, so the merged
// softmax is the combination of two disjoint partial softmaxes.  The cache is
// cut into chunks that never straddle s - W; every chunk yields a partial
// (normalised output, log-sum-exp) and a second kernel merges the partials.
//
// Per workgroup: one KV head, its G query heads, one chunk of up to 1024 keys
// (2 waves x up to 512 keys, each wave streaming its keys in 32-key blocks with
// the next block in flight; shorter caches use shorter waves so that about one
// full round of workgroups remains).  Two-wave workgroups, four per CU, keep the merge at
// the end of one workgroup from idling a large share of the CU's loads.
// Per wave and block:
//   S^T = K Q^T   (MFMA; A = key fragments loaded straight from HBM, 16-byte
//                  loads; remote keys are rotated in registers by the
//                  correction relative to the query's, each lane holding both
//                  halves of its rotate-half pairs)
//   O^T += V^T P^T (MFMA; V transposed through a per-wave LDS tile)
#include <atomic>
#include <cmath>

#include "jl_device.h"
#include "jl_launch.h"

namespace jl {
namespace {

constexpr int kWaves = 2;
constexpr int kMaxBlocksPerWave = 16;  // 512 keys per wave at most
// Enough workgroups for one full round at four per CU on 256 CUs.
constexpr int64_t kTargetWorkgroups = 1024;
// Workgroups of this kernel resident on one CU: the heads interleaved per chunk.
constexpr int kOrderHeads = 4;
constexpr int kMaxGroup = 16;  // query heads per KV head handled by one workgroup

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  float* part_o;    // [B, Hq, n_wg, D]
  float* part_lse;  // [B, Hq, n_wg]
  const int32_t* seq_lens;  // [B] keys held by each sequence, or null: every sequence holds n_kv
  int32_t batch, n_kv, hq, hkv, grp;  // n_kv: cache positions per sequence (the cache's stride)
  int64_t pretrained_window;          // L
  int32_t local_window;               // W (clamped to each sequence's length)
  int32_t n_wg;        // chunk slots per sequence (grid x; the partials' row stride)
  int32_t nb;          // 32-key blocks per wave (even, 2..16)
  int32_t kpw;         // keys per wave = 32 nb; a chunk is kWaves * kpw keys
  int32_t order_ncu;   // > 0: workgroup order interleaves heads with this stride (the CU count); 0: chunk-major
  int32_t sliding;     // 1: sliding window, only the newest min(W, s) keys (plain kernel)
  int32_t sched;       // long-range schedule (Schedule), per sequence
  float scale_log2;
  double theta_rev[kHalfD];
  // Paged caches (the PAGED kernels only): k and v are pools of n_pages pages of
  // 2^page_shift positions each ([n_pages, page, Hkv, D]); position j of sequence b
  // sits in page block_table[b * pages_per_seq + (j >> page_shift)].  n_kv is then
  // pages_per_seq pages' worth of positions.
  const int32_t* block_table;
  int32_t pages_per_seq, page_shift, n_pages;
};

// How one sequence of s keys is cut: g = g(s) of the schedule for the bifocal
// kernel (1 for plain); with g > 1 the remote prefix [0, s - min(W, s)) is cut into n_rem
// chunks of kpg keys and the local suffix into the rest, so that no chunk
// straddles the boundary; with g = 1 every chunk is local (base scores).
// A sliding window (plain attention over the newest min(W, s) keys) has no
// remote chunk at all: only the suffix is cut, with base scores.
struct SeqSplit {
  int g, remote_end, n_rem, n_chunks;
};
__device__ __forceinline__ SeqSplit seq_split(int s, bool bif, int64_t big_l, int w_req, int kpg, bool sliding,
                                              int sched) {
  SeqSplit r;
  r.g = bif ? sched_group(s, big_l, w_req, sched) : 1;
  const int w = min(w_req, s);
  r.remote_end = (r.g > 1 || sliding) ? s - w : 0;
  r.n_rem = sliding ? 0 : ceil_div(r.remote_end, kpg);
  r.n_chunks = r.n_rem + ceil_div(s - r.remote_end, kpg);
  return r;
}

// Keys of sequence b: seq_lens[b] clamped into [1, n_kv] (a length outside the
// contract gives an unspecified result, never an access outside the cache).
__device__ __forceinline__ int seq_length(const int32_t* seq_lens, int b, int n_kv) {
  return seq_lens ? min(max(seq_lens[b], 1), n_kv) : n_kv;
}

__device__ __forceinline__ int perm_key(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

__device__ __forceinline__ float elem(const u32x4& u, int e) {
  uint32_t w = u[e >> 1];
  return (e & 1) ? bf_hi(w) : bf_lo(w);
}


// V tiles in LDS: row-major, 256-byte key rows, chunk c of row r stored at c ^ 4(r % 4)
__device__ __forceinline__ int v_chunk(int row, int chunk) { return chunk ^ ((row & 3) << 2); }

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

constexpr int kBlk = 32;              // keys per MFMA block
constexpr int kVmemPerBlock = 16;     // 8 K loads + 8 V copies per block and lane
constexpr int kVBlockBytes = kBlk * 256;

// Two waves per SIMD (<= 256 VGPRs): four workgroups per CU.
// PAGED: the cache is a pool of pages (see DecodeArgs).  Chunks then start at
// multiples of the chunk size rather than at the local window's start, so that
// every 32-key block lies in one page (pages hold a power of two >= 32
// positions); the one chunk holding both remote and local keys turns its local
// keys by a zero angle, which leaves them exactly as cached.
template <bool BIF, bool PAGED = false>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_kernel(
    const DecodeArgs a) {
  // per-wave V blocks, double-buffered; two separate objects so that the
  // compiler can tell which direct copy a transposed read waits for
  __shared__ __attribute__((aligned(16))) uint8_t s_v0[kWaves][kVBlockBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_v1[kWaves][kVBlockBytes];
  __shared__ float s_fb[kWaves][kHalfD];  // per wave: (c(ws) - c(p)) theta_d / (2 pi), reduced to [-1/2, 1/2]
  __shared__ float s_th[kWaves][kHalfD];  // theta_d / (2 pi) times the schedule's rate
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_l[kWaves][kMaxGroup];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int n = lane & 31;
  // Workgroup order.  Workgroups are dealt to the CUs in id order, so ids
  // order_ncu apart share a CU.  When the shape allows it, such ids take
  // different KV heads of one chunk: the heads of a key row are interleaved in
  // memory, and rows read by all their heads at about the same time stream
  // faster (3 us of 93 at 128K) than rows whose heads are read far apart.
  int sp, bh;
  {
    const int i = blockIdx.x;
    if (a.order_ncu > 0) {
      const int slot = i % a.order_ncu, round = i / a.order_ncu;
      const int item = slot + a.order_ncu * (round / kOrderHeads);  // over n_wg x (B*Hkv / kOrderHeads)
      bh = round % kOrderHeads + kOrderHeads * (item / a.n_wg);
      sp = item % a.n_wg;
    } else {
      sp = i % a.n_wg;
      bh = i / a.n_wg;
    }
  }
  const int b = bh / a.hkv;
  const int kvh = bh % a.hkv;

  const int kpg = kWaves * a.kpw;
  const int s_len = seq_length(a.seq_lens, b, a.n_kv);
  const SeqSplit sq = seq_split(s_len, BIF, a.pretrained_window, a.local_window, kpg, a.sliding != 0, a.sched);
  int ks, ke;
  bool remote = false;
  int first_local = 0;  // PAGED: keys from here on take base scores
  if constexpr (PAGED) {
    if (sp >= ceil_div(s_len, kpg)) return;  // a shorter sequence of the batch: no chunk here
    ks = sp * kpg;
    ke = min(s_len, ks + kpg);
    first_local = (BIF && sq.g > 1) ? s_len - min(a.local_window, s_len) : 0;
    remote = BIF && ks < first_local;
  } else {
    if (sp >= sq.n_chunks) return;  // a shorter sequence of the batch: no chunk here
    if (sp < sq.n_rem) {
      ks = sp * kpg;
      ke = min(sq.remote_end, ks + kpg);
      remote = BIF;
    } else {
      ks = sq.remote_end + (sp - sq.n_rem) * kpg;
      ke = min(s_len, ks + kpg);
    }
  }
  const int ws = ks + wave * a.kpw;
  const int we = min(ke, ws + a.kpw);

  const int64_t kv_rs = (int64_t)a.hkv * kD;
  const uint16_t* kbase = a.k + (PAGED ? 0 : (int64_t)b * a.n_kv * kv_rs) + (int64_t)kvh * kD;
  const uint16_t* vbase = a.v + (PAGED ? 0 : (int64_t)b * a.n_kv * kv_rs) + (int64_t)kvh * kD;
  // PAGED: the pages of this wave's keys (at most 17), one per lane, loaded before
  // anything else: every block's address needs its page.  Entries are clamped into
  // the pool (a table outside the contract gives an unspecified result, never an
  // access out of range).
  int pt_first = 0, pt_page = 0;
  if constexpr (PAGED) {
    pt_first = ws >> a.page_shift;
    const int idx = min(pt_first + lane, a.pages_per_seq - 1);
    pt_page = min(max(a.block_table[(int64_t)b * a.pages_per_seq + idx], 0), a.n_pages - 1);
  }
  // row of key jb in the cache (PAGED: in the pool)
  auto cache_row = [&](int jb) -> int64_t {
    if constexpr (PAGED) {
      // a wave with no keys of its own re-reads the chunk's last key, which may sit in
      // an earlier page than the wave's start: clamp the lane index into the table
      const int pg = __builtin_amdgcn_readlane(pt_page, max((jb >> a.page_shift) - pt_first, 0));
      return ((int64_t)pg << a.page_shift) + (jb & ((1 << a.page_shift) - 1));
    } else {
      return jb;
    }
  };

  // ---- per-block loads: K fragment into registers (key j0 + perm_key(n),
  // d = 16kk + 8h + e), V rows into this wave's LDS buffer by direct copies ----
  // Each block builds buffer resources over the (at most 32) rows it may
  // touch, from jb = its first row clamped into the wave's range; rows past the
  // range re-read the wave's last key (we - 1 >= ks always), so every offset
  // stays below 32 rows.  Buffer (MUBUF) loads rather than FLAT ones: while a
  // FLAT-encoded LDS copy is in flight the compiler can only wait for every
  // load, never for the older ones alone.
  const uint32_t row_bytes = (uint32_t)kv_rs * 2u;  // <= 16 MiB (n_kv_heads <= 65536)
  typedef __attribute__((address_space(3))) void lds_void;
  // The block's rows, its byte count and so its buffer resource are the same for
  // the whole wave; readfirstlane states it, or the compiler wraps every buffer
  // load in a loop over the distinct resources it cannot rule out.
  auto rsrc_for = [&](const uint16_t* base, int jb, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + cache_row(jb) * kv_rs), (short)0, (int)nbytes,
                                             0x00020000);
  };
  auto issue_k = [&](int blk, u32x4 (&kr)[8]) {
    const int j0 = ws + blk * kBlk;
    const int jb = __builtin_amdgcn_readfirstlane(min(j0, we - 1));
    const uint32_t nbytes = (uint32_t)__builtin_amdgcn_readfirstlane(min(kBlk, we - jb) * (int)row_bytes);
    const __amdgpu_buffer_rsrc_t krs = rsrc_for(kbase, jb, nbytes);
    const uint32_t ko = (uint32_t)(min(j0 + perm_key(n), we - 1) - jb) * row_bytes + 16u * (uint32_t)h;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kr[kk] = __builtin_amdgcn_raw_buffer_load_b128(krs, ko + 32u * kk, 0, 0);
  };
  auto issue_v = [&](int blk, int buf) {
    const int j0 = ws + blk * kBlk;
    const int jb = __builtin_amdgcn_readfirstlane(min(j0, we - 1));
    const uint32_t nbytes = (uint32_t)__builtin_amdgcn_readfirstlane(min(kBlk, we - jb) * (int)row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = rsrc_for(vbase, jb, nbytes);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = 4 * r + (lane >> 4);
      const int c = v_chunk(row, lane & 15);
      const uint32_t vo = (uint32_t)(min(j0 + row, we - 1) - jb) * row_bytes + 16u * (uint32_t)c;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(buf ? &s_v1[wave][r * 1024] : &s_v0[wave][r * 1024]),
                                               16, (int)vo, 0, 0, 0);
    }
  };
  auto issue = [&](int blk, u32x4 (&kr)[8], int buf) {
    issue_k(blk, kr);
    issue_v(blk, buf);
  };
  u32x4 ka[8], kb[8];

  // Loads in the order they are needed: this lane's angle-table entries and
  // query fragment first (tiny), then the first two key/value blocks, so that
  // waiting for the former never waits for the stream.
  double th64 = 0.0;
  if (BIF) th64 = a.theta_rev[lane];  // unconditional within the instantiation: keeps the wait for it exact
  const bool col_ok = n < a.grp;
  const uint16_t* qrow = a.q + ((int64_t)b * a.hq + kvh * a.grp + (col_ok ? n : 0)) * kD;
  u32x4 qraw[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qraw[kk] = col_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0};
  issue(0, ka, 0);
  issue(1, kb, 1);
  // Everything below reads data loaded above; waiting for block 0 (and so for
  // the older table and query loads) explicitly keeps the wait exact.
  wait_vmem_at_most<kVmemPerBlock>();
  __builtin_amdgcn_sched_barrier(0);

  // query fragment (B operand of S^T): column n = query head kvh*G + n (n < G),
  // as stored; its correction is folded into the keys' angle below
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk] = as_bf16x8(qraw[kk]);

  // Remote keys.  Rotations in the same planes commute and are orthogonal, so
  // the grouped score rot(q, c_q(p) theta) . rot(k_j, c(j) theta) equals
  // q . rot(k_j, (c(j) - c_q(p)) theta): only the key turns, by
  //   (c(j) - c_q(p)) theta_d = (c(ws) - c_q(p)) theta_d - u(j) theta_d,
  //   u = t - floor((r + t)/g), t = j - ws, r = ws mod g,
  // with c(j) = floor(j/g) - j, c_q(p) = c(p) + the schedule's query shift, and
  // theta times the schedule's rate (fractional: g = 2^30 makes u = t).
  // The wave's part is reduced in fp64 once; the per-key part u theta_d
  // (u < 512, the longest wave) is exact enough in fp32, and the sum (below 82 revolutions) lies
  // inside the domain of the hardware sine and cosine, which reduce it exactly.
  int r_s = 0;
  const float inv_g = 1.0f / (float)sq.g;
  if (BIF && remote) {
    const int p = s_len - 1;  // the query's position
    const long long cq = (long long)(p / sq.g) - p + sched_q_shift(sq.g, a.local_window, a.sched);
    const long long cb = ((long long)(ws / sq.g) - ws) - cq;
    r_s = ws % sq.g;
    const double th = th64 * sched_rate(s_len, a.pretrained_window, a.sched);
    const double r = (double)cb * th;
    s_fb[wave][lane] = (float)(r - __builtin_rint(r));
    s_th[wave][lane] = (float)th;
    __builtin_amdgcn_wave_barrier();
  }

  // lane-constant part of the transposed V reads (see the prefill kernel)
  const int jl = lane & 15;
  const int vkey = 16 * h + (jl >> 2);
  const int dcol = 16 * ((lane >> 4) & 1) + 4 * (jl & 3);
  int voff[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) voff[nb] = vkey * 256 + (v_chunk(vkey, (32 * nb + dcol) >> 3) << 4) + ((dcol & 7) << 1);

  float m_run = kNegBig, l_run = 0.0f;
  const float thr = 8.0f / a.scale_log2;
  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x16{};

  auto process = [&](int blk, u32x4 (&kr)[8], int buf, bool more, int next_blk) {
    const int j0 = ws + blk * kBlk;
    // block blk's loads are older than the (up to) 16 of block blk+1
    if (more) wait_vmem_at_most<kVmemPerBlock>();
    else wait_vmem_at_most<0>();
    __builtin_amdgcn_sched_barrier(0);  // nothing that reads the block may move above the wait
    if (BIF && remote) {
      const int t = j0 + perm_key(n) - ws;
      // PAGED: a local key of the chunk that holds both kinds turns by zero
      const float on = (PAGED && (j0 + perm_key(n) >= first_local)) ? 0.0f : 1.0f;
      const float uf = (float)(t - small_div(r_s + t, sq.g, inv_g)) * on;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float4 fb0 = *reinterpret_cast<const float4*>(&s_fb[wave][16 * kk + 8 * h]);
        const float4 fb1 = *reinterpret_cast<const float4*>(&s_fb[wave][16 * kk + 8 * h + 4]);
        const float4 th0 = *reinterpret_cast<const float4*>(&s_th[wave][16 * kk + 8 * h]);
        const float4 th1 = *reinterpret_cast<const float4*>(&s_th[wave][16 * kk + 8 * h + 4]);
        const float fbv[8] = {fb0.x, fb0.y, fb0.z, fb0.w, fb1.x, fb1.y, fb1.z, fb1.w};
        const float thv[8] = {th0.x, th0.y, th0.z, th0.w, th1.x, th1.y, th1.z, th1.w};
        u32x4 lo, hi;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float y1[2], y2[2];
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            const int e = 2 * e2 + q2;
            const float rev = (PAGED ? fbv[e] * on : fbv[e]) - uf * thv[e];  // angle in revolutions
            const float co = __builtin_amdgcn_cosf(rev);
            const float si = __builtin_amdgcn_sinf(rev);
            const float x1 = elem(kr[kk], e), x2 = elem(kr[kk + 4], e);
            const f32x2 yr = rot_pair(x1, x2, co, si);
            y1[q2] = yr.x;
            y2[q2] = yr.y;
          }
          lo[e2] = pack_bf16(y1[0], y1[1]);
          hi[e2] = pack_bf16(y2[0], y2[1]);
        }
        kr[kk] = lo;
        kr[kk + 4] = hi;
      }
    }
    f32x16 s = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = mfma32(as_bf16x8(kr[kk]), qf[kk], s);
    // Bifocal: the key registers are free once S is formed, so the next key
    // fragment is requested before the softmax rather than after the block (the
    // rotation lengthens every block).  Plain keeps both requests after the block.
    if (BIF && next_blk >= 0) issue_k(next_blk, kr);

    // online softmax (lazy rescale, as in the prefill): lane = head n, keys j0 + 16h + i
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (j0 + 16 * h + i >= we) s[i] = -INFINITY;
      mloc = fmaxf(mloc, s[i]);
    }
    mloc = half_max(mloc);
    if (__builtin_amdgcn_ballot_w64(mloc > m_run + thr)) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb] *= alpha;
    }
    const float mc = -m_run * a.scale_log2;
    uint32_t pk[8];
    float psum = 0.0f;
#pragma unroll
    for (int i2 = 0; i2 < 8; ++i2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i2], a.scale_log2, mc));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i2 + 1], a.scale_log2, mc));
      pk[i2] = pack_bf16(p0, p1);
      psum += p0 + p1;  // fp32 probabilities: the normaliser carries fp32 rounding only
    }
    l_run += psum;
    // O^T += V^T P^T: keys 16h + 8half + e
    const uint8_t* sv = buf ? &s_v1[wave][0] : &s_v0[wave][0];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x4 pf = {pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]};
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const u32x2 t0 = lds_read_tr16(sv + voff[nb] + (8 * half) * 256);
        const u32x2 t1 = lds_read_tr16(sv + voff[nb] + (8 * half + 4) * 256);
        const u32x4 vf = {t0.x, t0.y, t1.x, t1.y};
        acc[nb] = mfma32(as_bf16x8(vf), as_bf16x8(pf), acc[nb]);
      }
    }
  };

  // Blocks in pairs (the two register/LDS buffers alternate), every load
  // issued unconditionally (blocks past the end of the wave's range re-read
  // its last key and are masked out entirely), so that the wait on the
  // prefetched block is exact: only block b+1's loads are newer than block b's
  // (block b+2's are issued after that wait).
  const int n_blocks = a.nb;  // even and >= 2
#pragma unroll 1
  for (int blk = 0; blk < n_blocks - 2; blk += 2) {
    process(blk, ka, 0, true, blk + 2);
    __builtin_amdgcn_wave_barrier();  // the V buffer is free again once its reads returned
    if (!BIF) issue_k(blk + 2, ka);
    issue_v(blk + 2, 0);
    process(blk + 1, kb, 1, true, blk + 3);
    __builtin_amdgcn_wave_barrier();
    if (!BIF) issue_k(blk + 3, kb);
    issue_v(blk + 3, 1);
  }
  process(n_blocks - 2, ka, 0, true, -1);
  process(n_blocks - 1, kb, 1, false, -1);

  // ---- merge the waves' partial softmaxes of this chunk ----
  const float lt = half_sum(l_run);
  __syncthreads();  // every wave is done with its V buffers
  float* red = reinterpret_cast<float*>(&s_v0[0][0]);  // [wave][G][D] fp32, at most the 16 KiB of s_v0
  if (n < a.grp) {
    if (h == 0) {
      s_m[wave][n] = m_run * a.scale_log2;  // log2 units
      s_l[wave][n] = lt;
    }
    float* dst = red + ((size_t)wave * a.grp + n) * kD;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4*>(dst + 32 * nb + 8 * i4 + 4 * h) =
            float4{acc[nb][4 * i4], acc[nb][4 * i4 + 1], acc[nb][4 * i4 + 2], acc[nb][4 * i4 + 3]};
  }
  __syncthreads();
  for (int item = tid; item < a.grp * kD; item += kWaves * 64) {
    const int hh = item / kD, d = item % kD;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (s_l[w][hh] > 0.0f) mx = fmaxf(mx, s_m[w][hh]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (!(s_l[w][hh] > 0.0f)) continue;
      const float sc = __builtin_amdgcn_exp2f(s_m[w][hh] - mx);
      lsum += s_l[w][hh] * sc;
      o += red[((size_t)w * a.grp + hh) * kD + d] * sc;
    }
    const int64_t bh = (int64_t)b * a.hq + kvh * a.grp + hh;
    a.part_o[(bh * a.n_wg + sp) * kD + d] = o / lsum;
    if (d == 0) a.part_lse[bh * a.n_wg + sp] = (mx + __builtin_log2f(lsum)) * kLn2;
  }
}

// Merge the per-chunk partials of one (sequence, query head): lse-weighted sum.
// 256 threads = 8 chunk lanes x 32 threads, each thread owning 4 of the 128
// output columns.  A chunk lane takes every 8th partial; all of a round's loads
// (up to 16 partials per thread) are issued together and merged with a running
// maximum, so a whole head costs one memory round trip per 128 partials.  The
// 8 lanes are then merged through LDS.
constexpr int kCombineThreads = 256;
constexpr int kCombineLanes = kCombineThreads / 32;
constexpr int kCombineBatch = 16;
struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  uint16_t* out;
  float* lse;
  const int32_t* seq_lens;
  int32_t n_kv, hq, n_wg, local_window, kpg, bif, sliding, sched, paged;
  int64_t pretrained_window;
};
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(const CombineArgs ca) {
  __shared__ float4 s_o[kCombineLanes][32];
  __shared__ float s_m[kCombineLanes];
  __shared__ float s_l[kCombineLanes];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int cl = tid >> 5, c4 = tid & 31;
  const int s_len = seq_length(ca.seq_lens, (int)(bh / ca.hq), ca.n_kv);
  const int n_wg = ca.paged ? ceil_div(s_len, ca.kpg)
                            : seq_split(s_len, ca.bif != 0, ca.pretrained_window, ca.local_window, ca.kpg,
                                        ca.sliding != 0, ca.sched).n_chunks;
  const float* pl = ca.part_lse + bh * ca.n_wg;  // rows of ca.n_wg slots, the first n_wg filled
  const float* po = ca.part_o + bh * ca.n_wg * kD + 4 * c4;
  uint16_t* out = ca.out;
  float* lse = ca.lse;
  float m = -INFINITY, l = 0.0f;
  float4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = cl; s0 < n_wg; s0 += kCombineLanes * kCombineBatch) {
    float lv[kCombineBatch];
    float4 x[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const int s = s0 + kCombineLanes * i;
      const bool ok = s < n_wg;
      lv[i] = ok ? pl[s] : -INFINITY;
      x[i] = ok ? *reinterpret_cast<const float4*>(po + (int64_t)s * kD) : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // lv[0] belongs to partial s0 < n_wg, whose chunk is non-empty: mx is finite
    float mx = m;
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) mx = fmaxf(mx, lv[i]);
    const float sc = __expf(m - mx);  // 0 on the first round (m = -inf)
    l *= sc;
    o.x *= sc;
    o.y *= sc;
    o.z *= sc;
    o.w *= sc;
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const float w = __expf(lv[i] - mx);  // 0 for the padding entries
      l += w;
      o.x += w * x[i].x;
      o.y += w * x[i].y;
      o.z += w * x[i].z;
      o.w += w * x[i].w;
    }
    m = mx;
  }
  s_o[cl][c4] = o;
  if (c4 == 0) {
    s_m[cl] = m;
    s_l[cl] = l;
  }
  __syncthreads();
  if (tid < 32) {
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < kCombineLanes; ++g)
      if (s_l[g] > 0.0f) mx = fmaxf(mx, s_m[g]);
    float ws = 0.0f;
    float4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < kCombineLanes; ++g) {
      if (!(s_l[g] > 0.0f)) continue;  // a lane with no partials (n_wg < 8)
      const float sc = __expf(s_m[g] - mx);
      const float4 x = s_o[g][tid];
      ws += s_l[g] * sc;
      t.x += x.x * sc;
      t.y += x.y * sc;
      t.z += x.z * sc;
      t.w += x.w * sc;
    }
    const float inv = 1.0f / ws;
    const u32x2 pk = {pack_bf16(t.x * inv, t.y * inv), pack_bf16(t.z * inv, t.w * inv)};
    *reinterpret_cast<u32x2*>(out + bh * kD + 4 * tid) = pk;
    if (lse && tid == 0) lse[bh] = mx + __logf(ws);
  }
}

}  // namespace

// Blocks per wave: the longest waves (fewest partials) that still give about
// one full round of workgroups; shorter caches get shorter waves.
int32_t decode_blocks_per_wave(int32_t batch, int32_t n_kv, int32_t n_kv_heads) {
  int32_t nb = kMaxBlocksPerWave;
  while (nb > 2) {
    const int64_t chunk = (int64_t)kWaves * kBlk * nb;
    if ((int64_t)batch * n_kv_heads * ((n_kv + chunk - 1) / chunk) >= kTargetWorkgroups) break;
    nb -= 2;
  }
  return nb;
}

int32_t decode_max_splits(int32_t batch, int32_t n_kv, int32_t n_kv_heads) {
  const int32_t chunk = kWaves * kBlk * decode_blocks_per_wave(batch, n_kv, n_kv_heads);
  return ceil_div(n_kv, chunk) + 1;
}

size_t decode_workspace_bytes(int32_t batch, int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads) {
  const size_t rows = (size_t)batch * n_q_heads * decode_max_splits(batch, n_kv, n_kv_heads);
  return rows * kD * sizeof(float) + rows * sizeof(float);
}

// Device-resident workspace of the allocation-free decode entry point: one copy
// per GPU, kept until the process ends.  Host code uses only the address
// returned by hipGetSymbolAddress (the array's name is a host-side stand-in).
// It holds chunk partials only, each written before it is read within a call,
// so nothing in it has to start at zero; calls that overlap on one GPU share it
// and race.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];  // per device, filled on first use
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    // with device dev current; racing callers get the same address
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

// CUs of the current device (queried once per device; 0 if unknown).
static int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0: not queried yet; -1: unknown
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    v = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : -1;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

hipError_t launch_decode(bool bifocal, const DecodeProblem& p, hipStream_t stream) {
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.out = static_cast<uint16_t*>(p.out);
  a.lse = p.lse;
  a.batch = p.batch;
  a.n_kv = p.n_kv;
  a.hq = p.n_q_heads;
  a.hkv = p.n_kv_heads;
  a.grp = p.n_q_heads / p.n_kv_heads;
  if (a.grp > kMaxGroup) return hipErrorInvalidValue;
  a.seq_lens = p.seq_lens;
  a.sliding = p.sliding ? 1 : 0;
  if (p.sliding && bifocal) return hipErrorInvalidValue;
  const bool paged = p.block_table != nullptr;
  a.block_table = p.block_table;
  a.pages_per_seq = p.pages_per_seq;
  a.n_pages = p.n_pages;
  a.page_shift = 0;
  if (paged) {
    // pages of a power of two >= 32 positions, lengths per sequence, no window-only mode
    if (p.sliding || !p.seq_lens || p.page_size < kBlk || (p.page_size & (p.page_size - 1)) != 0 || p.n_pages < 1 ||
        (int64_t)p.pages_per_seq * p.page_size != p.n_kv)
      return hipErrorInvalidValue;
    while ((1 << a.page_shift) < p.page_size) ++a.page_shift;
  }
  a.pretrained_window = bifocal ? p.pretrained_window : 1;
  a.local_window = (bifocal || p.sliding) ? p.local_window : 0;
  a.sched = bifocal ? p.schedule : kSchedGrouped;
  a.nb = decode_blocks_per_wave(p.batch, p.n_kv, p.n_kv_heads);
  if (p.sliding) {
    // chunks sized for the window's keys, if their count fits the workspace bound
    const int32_t w = p.local_window < p.n_kv ? p.local_window : p.n_kv;
    const int32_t nb_w = decode_blocks_per_wave(p.batch, w, p.n_kv_heads);
    const int32_t chunk_w = kWaves * kBlk * nb_w;
    if (ceil_div(w, chunk_w) <= decode_max_splits(p.batch, p.n_kv, p.n_kv_heads)) a.nb = nb_w;
  }
  a.kpw = kBlk * a.nb;
  const int32_t chunk = kWaves * a.kpw;
  if (paged) {
    // chunks start at multiples of the chunk: at most ceil(n_kv / chunk) per sequence
    a.n_wg = ceil_div(p.n_kv, chunk);
  } else if (p.seq_lens) {
    // any length up to n_kv fits (the cut at the local window's start may add one chunk)
    a.n_wg = decode_max_splits(p.batch, p.n_kv, p.n_kv_heads);
  } else if (p.sliding) {
    const int32_t w = p.local_window < p.n_kv ? p.local_window : p.n_kv;
    a.n_wg = ceil_div(w, chunk);
  } else {
    // every sequence holds n_kv keys: exactly its chunks (the kernels' cut, on the host)
    const int32_t g = bifocal ? sched_group(p.n_kv, a.pretrained_window, a.local_window, a.sched) : 1;
    const int32_t remote_end = g > 1 ? p.n_kv - (p.local_window < p.n_kv ? p.local_window : p.n_kv) : 0;
    const int32_t n_rem = ceil_div(remote_end, chunk);
    a.n_wg = n_rem + ceil_div(p.n_kv - remote_end, chunk);
  }
  a.scale_log2 = p.softmax_scale * 1.4426950408889634f;
  // theta_d / (2 pi) for this RoPE base, kept per thread for the next call
  thread_local double cached_base = 0.0;
  thread_local double cached_rev[kHalfD];
  if (cached_base != p.rope_base) {
    const double two_pi = 6.283185307179586476925286766559;
    for (int d = 0; d < kHalfD; ++d) cached_rev[d] = std::pow(p.rope_base, -2.0 * d / kD) / two_pi;
    cached_base = p.rope_base;
  }
  for (int d = 0; d < kHalfD; ++d) a.theta_rev[d] = cached_rev[d];
  const size_t rows = (size_t)p.batch * p.n_q_heads * decode_max_splits(p.batch, p.n_kv, p.n_kv_heads);
  a.part_o = static_cast<float*>(p.workspace);
  a.part_lse = a.part_o + rows * kD;
  // partials: rows of n_wg chunk slots per (sequence, query head)
  // head-interleaved order when it is a bijection on the grid: B*Hkv a multiple of
  // kOrderHeads and the grid a whole number of kOrderHeads rounds over the CUs
  const int64_t n_bh = (int64_t)p.batch * p.n_kv_heads;
  const int64_t n_grid = (int64_t)a.n_wg * n_bh;
  const int ncu = device_cu_count();
  a.order_ncu = (ncu > 0 && n_bh % kOrderHeads == 0 && n_grid % ((int64_t)ncu * kOrderHeads) == 0) ? ncu : 0;
  if (n_grid > 0x7fffffff) return hipErrorInvalidValue;
  if (paged && bifocal)
    hipLaunchKernelGGL((decode_split_kernel<true, true>), dim3((unsigned)n_grid), dim3(kWaves * 64), 0, stream, a);
  else if (paged)
    hipLaunchKernelGGL((decode_split_kernel<false, true>), dim3((unsigned)n_grid), dim3(kWaves * 64), 0, stream, a);
  else if (bifocal)
    hipLaunchKernelGGL((decode_split_kernel<true>), dim3((unsigned)n_grid), dim3(kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<false>), dim3((unsigned)n_grid), dim3(kWaves * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CombineArgs ca;
  ca.part_o = a.part_o;
  ca.part_lse = a.part_lse;
  ca.out = a.out;
  ca.lse = a.lse;
  ca.seq_lens = a.seq_lens;
  ca.n_kv = a.n_kv;
  ca.hq = a.hq;
  ca.n_wg = a.n_wg;
  ca.local_window = a.local_window;
  ca.kpg = chunk;
  ca.bif = bifocal ? 1 : 0;
  ca.sliding = a.sliding;
  ca.sched = a.sched;
  ca.paged = paged ? 1 : 0;
  ca.pretrained_window = a.pretrained_window;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(p.batch * p.n_q_heads), dim3(kCombineThreads), 0, stream, ca);
  return hipGetLastError();
}

}  // namespace jl
