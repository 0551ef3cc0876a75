// Chunked KDA prefill on gfx950 matrix cores, with the state checkpoint exported inside the
// same pass ("vLLM lifts Kimi K3 throughput by up to 2.8x", section "KDA checkpoints stay
// inside the prefill").
//
// Chunked (WY/UT) form of the gated delta rule, for one head and one chunk of C tokens
// (rows r, s) entered with state S (d x d, fp32). With G_r = sum_{t<=r} log2 a_t per key
// channel:
//     A_kk[r,s] = sum_i k_ri k_si 2^(G_ri - G_si)  (s < r),  A_qk likewise with q_r (s <= r)
//     T  = (I + Diag(b) A_kk)^-1 Diag(b)
//     X  = V - Kt S          Kt_r = k_r 2^(G_r)
//     W  = T X               (the delta-rule innovations of the chunk)
//     O  = Qt S + A_qk W     Qt_r = q_r 2^(G_r)
//     S' = Diag(2^(G_C)) S + Kbar^T W,    Kbar_s = k_s 2^(G_C - G_s)
// Derivation: write each step as S_r = Diag(a_r) S_{r-1} + k_r w_r^T and unroll over the chunk.
//
// Design for MI355X: everything that does not depend on S (decays, Kt, Qt, Kbar, A_qk, T,
// 2^(G_C)) is computed for every (chunk, head) at once by chunk_prep_kernel, which fills the
// GPU whatever the batch shape; the sequential part left for state_pass_kernel is three
// small matrix products per chunk (X, W, then O and S'), so the per-chunk latency of a long
// sequence is a few hundred MFMA cycles instead of the whole chunk computation.
//   * chunk_prep_kernel writes each chunk's operands as fp16 16x32 A-operand fragments of
//     v_mfma_f32_16x16x32_f16 in lane order (one 1 KiB fragment = 64 lanes x 16 bytes), so the
//     state pass copies a chunk's 60.5 KiB block into LDS with coalesced 16-byte loads and
//     reads every fragment with one conflict-free ds_read_b128 per lane.
//   * state_pass_kernel keeps the state S in fp32 MFMA accumulators for the whole sequence.
//     The accumulator tiles of S, X and W become B operands of the next product in registers:
//     fp16 conversion plus two lane-half swaps (v_permlane32_swap, v_permlane16_swap) per
//     pair of 16-row tiles; no LDS round trip and no barrier inside the chain.
//   * fp16 operands (same rate as bf16, 3 more mantissa bits) keep the chunked form within
//     2e-3 of the sequential fp64 result; bf16 operands do not (5e-3 in emulation).
//   * decay factors are products of a over row ranges inside a chunk, formed by
//     multiplication: every factor is at most 1 except the column factor of the diagonal
//     16x16 blocks of A_kk / A_qk, the inverse of the block's 16-token decay. That factor is
//     used only for key channels whose block decay is at least 2^-12 (so it stays <= 4096 in
//     fp16); a channel that decays faster within a block is left out of that block's diagonal
//     products and its terms k_r k_s prod_{s<t<=r} a_t are added in fp32 from the raw inputs,
//     exact for any decay (reported as KDA_DEVERR_DECAY_RANGE, informational).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"

// Workspace of kda_prefill_noalloc, for callers that cannot allocate device memory: every GPU
// the library runs on holds one copy until the process ends. Host code never uses this name as
// an address (it is a host-side stand-in there): prefill_scratch looks the device address up.
static __device__ __align__(256) char scratch[kda::PREFILL_SCRATCH_BYTES];

namespace kda {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

constexpr int PD = PREFILL_D;     // head dim (dk = dv)
constexpr int PC = PREFILL_CHUNK; // chunk
constexpr int PNB = PC / 16;      // 16-row blocks per chunk
constexpr int NPAIR = PNB * (PNB + 1) / 2;
constexpr int P16 = PD + 8;       // row pitch (halves) of [.][PD] fp16 arrays
constexpr int PC16 = PC + 8;      // row pitch (halves) of [.][PC] fp16 arrays
// Smallest 16-token decay of a key channel whose diagonal-block terms go through the fp16
// factorisation (column factor <= 2^12); below it the block's terms of that channel are
// evaluated exactly in fp32.
constexpr float DIAG_DECAY_MIN = 1.f / 4096.f;   // 2^-12
constexpr int LDS_PER_CU = 160 * 1024;   // gfx950: LDS of one CU, the most one work-group may hold

// ---- per-(chunk, head) operand block --------------------------------------------------------
// A fragment holds a 16 x 32 fp16 tile A[16][32] as the A operand of v_mfma_f32_16x16x32_f16:
// lane L = l16 + 16 * lq owns A[l16][8 lq .. 8 lq + 7] at bytes 16 L .. 16 L + 15.
constexpr int FRAG = 1024;
constexpr int OFF_KT = 0;             // -Kt:    f = 4 rt + kk  (token tile rt, channel block kk)
constexpr int OFF_QT = 16 * FRAG;     // Qt:     same
constexpr int OFF_KB = 32 * FRAG;     // Kbar^T: f = 2 rt + kk  (channel tile rt < 8, token block kk)
constexpr int OFF_T = 48 * FRAG;      // T:      f = tri_frag(rt, kk), token block kk <= rt / 2
constexpr int OFF_AQ = 54 * FRAG;     // A_qk:   same
constexpr int OFF_GAM = 60 * FRAG;    // 2^(G_C), fp32 [PD]
constexpr int BLOCK_BYTES = 60 * FRAG + 4 * PD;   // 61952, a multiple of 256
static_assert(BLOCK_BYTES == PREFILL_BLOCK_BYTES, "operand block size shared with the host plan");

// Lower-triangular 64x64 operands keep only the fragments with kk <= rt / 2:
// (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
__host__ __device__ constexpr int tri_frag(int rt, int kk) { return rt < 2 ? rt : 2 * rt - 2 + kk; }

__device__ __forceinline__ int frag_lane_byte(int row, int k) {   // byte of A[row][k] in its fragment
  return ((row & 15) + 16 * ((k & 31) >> 3)) * 16 + (k & 7) * 2;
}

__device__ __forceinline__ f4 mfma32(half8 a, half8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(half4 a, half4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 ld8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }
// fp32 -> fp16 (round to nearest even) as packed conversions (v_cvt_pk_f16_f32)
__device__ __forceinline__ half4 to_h4(f4 x) { return __builtin_convertvector(x, half4); }

// Work-group barrier for LDS hand-offs: waits for this wave's LDS operations only; global
// loads and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Lane exchanges inside groups of four lanes (DPP quad_perm: a VALU operand modifier, no
// LDS round trip): value of lane l ^ 1 and of lane l ^ 2.
__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Raw buffer resource over [base, base + bytes): loads beyond return 0, stores beyond are
// dropped by the hardware, so ragged chunk tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ---- plan: chunk offsets, checkpoint offsets and the longest-first order -----------------
// choff[i] = sum_{j<i} ceil(len_j / PC) (n_seq + 1 entries), ckoff[i] = sum_{j<i} floor(len_j /
// ckpt_interval), order[rank] = index of the sequence with that rank in descending length
// (ties: lower index first).
constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_MAX_SORT = 8192;

__global__ __launch_bounds__(PLAN_THREADS) void prefill_plan_kernel(const int32_t* __restrict__ cu,
                                                                  int n_seq, int ckpt_interval,
                                                                  int32_t* __restrict__ choff,
                                                                  int32_t* __restrict__ ckoff,
                                                                  int32_t* __restrict__ order) {
  __shared__ int32_t len_s[PLAN_MAX_SORT];
  __shared__ int32_t part_c[PLAN_THREADS], part_k[PLAN_THREADS];
  const int t = threadIdx.x;
  const int per = (n_seq + PLAN_THREADS - 1) / PLAN_THREADS;
  const int j0 = t * per, j1 = min(n_seq, j0 + per);
  int sc = 0, sk = 0;
  for (int j = j0; j < j1; ++j) {
    const int len = cu[j + 1] - cu[j];
    sc += seq_chunks(len, PC, ckpt_interval);
    sk += ckpt_interval > 0 ? len / ckpt_interval : 0;
  }
  // inclusive scan of the per-thread sums over the work-group (Hillis-Steele)
  part_c[t] = sc;
  part_k[t] = sk;
  __syncthreads();
  for (int off = 1; off < PLAN_THREADS; off <<= 1) {
    const int vc = t >= off ? part_c[t - off] : 0, vk = t >= off ? part_k[t - off] : 0;
    __syncthreads();
    part_c[t] += vc;
    part_k[t] += vk;
    __syncthreads();
  }
  if (t == PLAN_THREADS - 1) choff[n_seq] = part_c[t];
  sc = part_c[t] - sc;   // exclusive
  sk = part_k[t] - sk;
  for (int j = j0; j < j1; ++j) {
    const int len = cu[j + 1] - cu[j];
    choff[j] = sc;
    ckoff[j] = sk;
    sc += seq_chunks(len, PC, ckpt_interval);
    sk += ckpt_interval > 0 ? len / ckpt_interval : 0;
  }
  if (n_seq > PLAN_MAX_SORT) {
    for (int j = t; j < n_seq; j += PLAN_THREADS) order[j] = j;
    return;
  }
  for (int j = t; j < n_seq; j += PLAN_THREADS) len_s[j] = cu[j + 1] - cu[j];
  __syncthreads();
  for (int j = t; j < n_seq; j += PLAN_THREADS) {
    const int lj = len_s[j];
    int rj = 0;
    for (int k = 0; k < n_seq; ++k) {
      const int lk = len_s[k];
      rj += (lk > lj) || (lk == lj && k < j);
    }
    order[rj] = j;
  }
}

// A batch of at most 64 sequences is planned inside chunk_prep_kernel instead (one lane per
// sequence), which saves the plan kernel's launch: lane i gets sequence i's length, chunk count
// and exclusive chunk / checkpoint offsets.
constexpr int PLAN_INLINE_MAX = PREFILL_PLAN_INLINE_MAX;
struct LanePlan {
  int len, nch, choff, ckoff, n_ck;
};
__device__ __forceinline__ LanePlan lane_plan(const int32_t* cu, int n_seq, int interval, int lane) {
  LanePlan q{0, 0, 0, 0, 0};
  if (lane < n_seq) {
    q.len = cu[lane + 1] - cu[lane];
    q.nch = seq_chunks(q.len, PC, interval);
    q.n_ck = interval > 0 ? q.len / interval : 0;
  }
  int c = q.nch, k = q.n_ck;   // inclusive scans over the wave
  for (int off = 1; off < 64; off <<= 1) {
    const int cc = __shfl_up(c, off), kk = __shfl_up(k, off);
    if (lane >= off) {
      c += cc;
      k += kk;
    }
  }
  q.choff = c - q.nch;
  q.ckoff = k - q.n_ck;
  return q;
}

// ---- chunk_prep_kernel: the S-independent part of one (chunk, head) -------------------------
constexpr int PNW = 8;            // waves per work-group
constexpr int PNT = 64 * PNW;

struct PrepLds {
  _Float16 ka[PC][P16];      // rows of block P times 2^(G - G_start(P))     (A operand, A_kk)
  _Float16 qa[PC][P16];      // q likewise                                   (A operand, A_qk)
  _Float16 f16[PC][P16];     // F_s = k_s 2^(G_end(block of s) - G_s)
  float ldg[PNB][16][16];    // diagonal blocks of Diag(b) A_kk (strictly lower), fp32
  _Float16 loff[PC][PC16];   // Diag(b) A_kk below the diagonal blocks, fp16
  union {
    float part[PC / 4][PD];  // products of a over each group of 4 rows
    float nd[PC][16];        // diagonal 16x16 blocks of (I + Diag(b) A_kk)^-1
  } u4;
  float bp[PNB][PD];         // decay over each block: 2^(G_end(P) - G_start(P))
  _Float16 xvh[NPAIR][PD];   // 2^(G_start(P) - G_end(Q)) per pair, fp16
  float b[PC];
  uint32_t xmask[PNB][PD / 32];   // channels whose block decay is below DIAG_DECAY_MIN
};

// pair index p = P(P+1)/2 + Q for Q <= P
__device__ __forceinline__ int pair_p(int p) { return p >= 6 ? 3 : (p >= 3 ? 2 : (p >= 1 ? 1 : 0)); }

// Column block Q of T = N Diag(b), N = (I + Diag(b) A_kk)^-1, from the diagonal inverses:
// N_PQ = -N_PP sum_{Q<=R<P} L_PR N_RQ, 16x16x16 fp16 products with fp32 accumulation. The
// accumulator layout of a 16x16x16 product equals its B-operand layout, so N_RQ stays in
// registers from one product to the next. T blocks go straight to their fragments.
template <int Q>
__device__ __forceinline__ void t_column(const PrepLds& L, char* blk, int l16, int lq) {
  f4 nq[PNB];
#pragma unroll
  for (int e = 0; e < 4; ++e) nq[Q][e] = L.u4.nd[16 * Q + 4 * lq + e][l16];
  const float bq = L.b[16 * Q + l16];
  auto put = [&](int Pb, const f4& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * Pb + 4 * lq + e, col = 16 * Q + l16;
      *reinterpret_cast<_Float16*>(blk + OFF_T + tri_frag(Pb, col >> 5) * FRAG + frag_lane_byte(row, col)) =
          (_Float16)(v[e] * bq);
    }
  };
  put(Q, nq[Q]);
#pragma unroll
  for (int Pb = Q + 1; Pb < PNB; ++Pb) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int R = Q; R < Pb; ++R) {
      const half4 lr = *reinterpret_cast<const half4*>(&L.loff[16 * Pb + l16][16 * R + 4 * lq]);
      acc = mfma16(lr, to_h4(nq[R]), acc);
    }
    const f4 np = *reinterpret_cast<const f4*>(&L.u4.nd[16 * Pb + l16][4 * lq]);
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    nq[Pb] = -mfma16(to_h4(np), to_h4(acc), zero);
    put(Pb, nq[Pb]);
  }
}

// One work-group per (chunk, head): blockIdx.x = global chunk index * H + head. Thread t
// owns key rows 4m .. 4m+3 (m = t / 32) and key channels 4cq .. 4cq+3 (cq = t % 32) in the
// staging and operand phases. For batches of at most PLAN_INLINE_MAX sequences every wave plans
// the batch itself and work-group 0 writes the plan arrays for the state pass; larger batches
// read choff from the plan kernel.
__global__ __launch_bounds__(PNT, 2) void chunk_prep_kernel(PoolView P, PrefillLaunch A,
                                                            int32_t* __restrict__ choff,
                                                            int32_t* __restrict__ ckoff,
                                                            int32_t* __restrict__ order,
                                                            char* __restrict__ blocks) {
  __shared__ PrepLds L;
  const int H = P.H, h = blockIdx.x % H, gc = blockIdx.x / H;
  int si, c;
  if (A.n_seq <= PLAN_INLINE_MAX) {
    const int lane = (int)threadIdx.x & 63;
    const LanePlan q = lane_plan(A.cu_seqlens, A.n_seq, A.ckpt_interval, lane);
    // the sequence whose chunk range holds gc (every chunk of the grid lies in one)
    const uint64_t hit = __ballot(lane < A.n_seq && q.choff <= gc && gc < q.choff + q.nch);
    si = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
    c = gc - __shfl(q.choff, si);
    if (blockIdx.x == 0 && threadIdx.x < 64 && lane < A.n_seq) {
      choff[lane] = q.choff;
      ckoff[lane] = q.ckoff;
      if (lane == A.n_seq - 1) choff[A.n_seq] = q.choff + q.nch;
      int rank = 0;   // descending length, ties: lower index first
      for (int k = 0; k < A.n_seq; ++k) {
        const int lk = __shfl(q.len, k);
        rank += (lk > q.len) || (lk == q.len && k < lane);
      }
      order[rank] = lane;
    }
  } else {
    // the last i with choff[i] <= gc (binary search, uniform)
    int lo_i = 0, hi_i = A.n_seq - 1;
    while (lo_i < hi_i) {
      const int mid = (lo_i + hi_i + 1) >> 1;
      if (choff[mid] <= gc) lo_i = mid; else hi_i = mid - 1;
    }
    si = lo_i;
    c = gc - choff[si];
  }
  int t0, n;
  chunk_span(c, A.cu_seqlens[si + 1] - A.cu_seqlens[si], PC, A.ckpt_interval, &t0, &n);
  const int tok0 = A.cu_seqlens[si] + t0;
  char* blk = blocks + (size_t)blockIdx.x * BLOCK_BYTES;
  const size_t hstride = (size_t)H * PD;

  const int t = threadIdx.x, w = t >> 6, l = t & 63, l16 = l & 15, lq = l >> 4;
  const int m4 = t >> 5, c4 = (t & 31) * 4, Pm = m4 >> 2, mq = m4 & 3;

  // ---- raw rows; padded rows (r >= n) have k = q = 0, a = 1, b = 0 ---------------------------
  uint2 kr4[4], qr4[4];
  f4 cpre[4], dsuf[3];   // cpre[i] = a_0..a_i, dsuf[i] = a_{i+1}..a_3 over the thread's rows
  {
    f4 av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * m4 + i;
      uint2 kk = make_uint2(0, 0), qq = make_uint2(0, 0);
      float4 a = make_float4(1.f, 1.f, 1.f, 1.f);
      if (r < n) {
        const size_t off = (size_t)(tok0 + r) * hstride + (size_t)h * PD + c4;
        kk = *reinterpret_cast<const uint2*>(A.t.k + off);
        qq = *reinterpret_cast<const uint2*>(A.t.q + off);
        a = *reinterpret_cast<const float4*>(A.t.a + off);
      }
      kr4[i] = kk;
      qr4[i] = qq;
      av[i] = f4{a.x, a.y, a.z, a.w};
    }
    cpre[0] = av[0];
    cpre[1] = cpre[0] * av[1];
    cpre[2] = cpre[1] * av[2];
    cpre[3] = cpre[2] * av[3];
    dsuf[2] = av[3];
    dsuf[1] = av[2] * av[3];
    dsuf[0] = av[1] * dsuf[1];
    *reinterpret_cast<f4*>(&L.u4.part[m4][c4]) = cpre[3];
  }
  if (t < PC) L.b[t] = t < n ? A.t.b[(size_t)(tok0 + t) * H + h] : 0.f;
  if (t < PNB * PD / 32) (&L.xmask[0][0])[t] = 0u;
  __syncthreads();

  // ---- decayed fp16 operands: Ka/Qa (rows of block P times 2^(G - G_start(P))), F (times
  //      2^(G_end(P) - G)) to LDS; Kt/Qt (times 2^G) straight to their fragments. Every
  //      factor is at most 1. ---------------------------------------------------------------
  {
    // Products of the row-group decays: gsp over the blocks before this one (a wave-uniform
    // loop), then the four groups of this block: pre before the thread's rows, post after.
    f4 gsp = {1.f, 1.f, 1.f, 1.f};
    for (int mm = 0; mm < 4 * Pm; ++mm) gsp *= *reinterpret_cast<const f4*>(&L.u4.part[mm][c4]);
    f4 blk4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) blk4[q] = *reinterpret_cast<const f4*>(&L.u4.part[4 * Pm + q][c4]);
    const f4 one = {1.f, 1.f, 1.f, 1.f};
    const f4 p01 = blk4[0] * blk4[1], p23 = blk4[2] * blk4[3];
    const f4 pre = mq == 0 ? one : (mq == 1 ? blk4[0] : (mq == 2 ? p01 : p01 * blk4[2]));
    const f4 post = mq == 3 ? one : (mq == 2 ? blk4[3] : (mq == 1 ? p23 : blk4[1] * p23));
    if (mq == 3) {
      const f4 bpv = p01 * p23;   // decay over the whole block
      *reinterpret_cast<f4*>(&L.bp[Pm][c4]) = bpv;
      if (Pm == PNB - 1) *reinterpret_cast<f4*>(blk + OFF_GAM + 4 * c4) = gsp * bpv;
      uint32_t fast = 0;   // the thread's four channels (one 32-channel word) that decay fast
#pragma unroll
      for (int e = 0; e < 4; ++e) fast |= (bpv[e] < DIAG_DECAY_MIN ? 1u : 0u) << ((c4 + e) & 31);
      if (fast) {
        atomicOr(&L.xmask[Pm][c4 >> 5], fast);
        atomicOr(P.err, (uint32_t)KDA_DEVERR_DECAY_RANGE);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * m4 + i;
      const float kr[4] = {__uint_as_float(kr4[i].x << 16), __uint_as_float(kr4[i].x & 0xffff0000u),
                           __uint_as_float(kr4[i].y << 16), __uint_as_float(kr4[i].y & 0xffff0000u)};
      const float qr[4] = {__uint_as_float(qr4[i].x << 16), __uint_as_float(qr4[i].x & 0xffff0000u),
                           __uint_as_float(qr4[i].y << 16), __uint_as_float(qr4[i].y & 0xffff0000u)};
      const f4 e1 = pre * cpre[i];                                   // 2^(G_r - G_start(P))
      const f4 e2 = i == 3 ? post : post * dsuf[i < 3 ? i : 0];     // 2^(G_end(P) - G_r)
      f4 ka, qa, kt, qt, fv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ka[e] = kr[e] * e1[e];
        qa[e] = qr[e] * e1[e];
        kt[e] = -(ka[e] * gsp[e]);   // stored negated: X = V + (-Kt) S
        qt[e] = qa[e] * gsp[e];
        fv[e] = kr[e] * e2[e];
      }
      *reinterpret_cast<half4*>(&L.ka[r][c4]) = to_h4(ka);
      *reinterpret_cast<half4*>(&L.qa[r][c4]) = to_h4(qa);
      *reinterpret_cast<half4*>(&L.f16[r][c4]) = to_h4(fv);
      const int fo = (4 * (r >> 4) + (c4 >> 5)) * FRAG + frag_lane_byte(r, c4);
      *reinterpret_cast<half4*>(blk + OFF_KT + fo) = to_h4(kt);
      *reinterpret_cast<half4*>(blk + OFF_QT + fo) = to_h4(qt);
    }
  }
  __syncthreads();

  // ---- A_kk, A_qk block pairs on matrix cores. Waves 0-3: diagonal pair (w, w), then the
  //      inverse of that block by forward substitution (the wave's own LDS writes, no barrier
  //      needed). Waves 4-7: the six off-diagonal pairs; waves 6-7 also Kbar^T and the zero
  //      blocks above the diagonal inside the T / A_qk fragments. ---------------------------
  {
    int pa, pb;
    switch (w) {
      case 0: pa = 0; pb = -1; break;
      case 1: pa = 2; pb = -1; break;
      case 2: pa = 5; pb = -1; break;
      case 3: pa = 9; pb = -1; break;
      case 4: pa = 1; pb = 7; break;
      case 5: pa = 3; pb = 8; break;
      case 6: pa = 4; pb = -1; break;
      default: pa = 6; pb = -1; break;
    }
    for (int pi = 0; pi < 2; ++pi) {
      const int p = pi == 0 ? pa : pb;
      if (p < 0) break;
      const int Pb = pair_p(p), Q = p - Pb * (Pb + 1) / 2;
      {   // this pair's column factor, two channels per lane (read back by this wave only):
          // the decay between the end of block Q and the start of block P, or the inverse
          // decay of the block when P = Q
        const int i0 = 2 * l;
        float z0, z1;
        if (Pb == Q) {   // 0 for the fast-decaying channels: their terms are added exactly below
          const uint32_t fast = L.xmask[Q][i0 >> 5] >> (i0 & 31);
          z0 = fast & 1u ? 0.f : __builtin_amdgcn_rcpf(L.bp[Q][i0]);
          z1 = fast & 2u ? 0.f : __builtin_amdgcn_rcpf(L.bp[Q][i0 + 1]);
        } else {
          z0 = 1.f;
          z1 = 1.f;
          for (int R = Q + 1; R < Pb; ++R) {
            z0 *= L.bp[R][i0];
            z1 *= L.bp[R][i0 + 1];
          }
        }
        L.xvh[p][i0] = (_Float16)z0;
        L.xvh[p][i0 + 1] = (_Float16)z1;
      }
      f4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < PD / 32; ++kk) {
        const int c = 32 * kk + 8 * lq;
        // k_s 2^(G_start(P) - G_s) = F_s 2^(G_start(P) - G_end(Q)), packed fp16 products
        const half8 bb = ld8(&L.f16[16 * Q + l16][c]) * ld8(&L.xvh[p][c]);
        akk = mfma32(ld8(&L.ka[16 * Pb + l16][c]), bb, akk);
        aqk = mfma32(ld8(&L.qa[16 * Pb + l16][c]), bb, aqk);
      }
      if (Pb == Q) {
        // Channels whose decay over this block is below DIAG_DECAY_MIN: their terms
        // k_r k_s prod_{s<t<=r} a_t (A_kk, s < r) and q_r k_s prod_{s<t<=r} a_t (A_qk, s <= r)
        // in fp32 from the raw inputs, for this lane's rows 4 lq + e and column s. Padded rows
        // (past the chunk) read k = q = 0 and a = 1, as everywhere in this kernel.
        const int s = l16, nb = n - 16 * Pb;   // rows of this block inside the chunk
        const size_t blk0 = (size_t)(tok0 + 16 * Pb) * hstride + (size_t)h * PD;
#pragma unroll 1
        for (int wd = 0; wd < PD / 32; ++wd) {
          uint32_t msk = (uint32_t)__builtin_amdgcn_readfirstlane((int)L.xmask[Q][wd]);
          while (msk) {
            const int i = 32 * wd + __builtin_ctz(msk);
            msk &= msk - 1;
            const float* ac = A.t.a + blk0 + i;
            float run = 1.f, dec[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int tt = 0; tt < 16; ++tt, ac += hstride) {
              const float a_t = tt < nb ? *ac : 1.f;
              if (tt > s) run *= a_t;
              if ((tt >> 2) == lq) dec[0] = (tt & 3) == 0 ? run : dec[0];
              if ((tt >> 2) == lq) dec[1] = (tt & 3) == 1 ? run : dec[1];
              if ((tt >> 2) == lq) dec[2] = (tt & 3) == 2 ? run : dec[2];
              if ((tt >> 2) == lq) dec[3] = (tt & 3) == 3 ? run : dec[3];
            }
            const float ks = s < nb ? bf2f(A.t.k[blk0 + (size_t)s * hstride + i]) : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * lq + e;
              const size_t off = blk0 + (size_t)r * hstride + i;
              const float kr = r < nb ? bf2f(A.t.k[off]) : 0.f, qr = r < nb ? bf2f(A.t.q[off]) : 0.f;
              const float w = ks * dec[e];
              if (r > s) akk[e] = __builtin_fmaf(kr, w, akk[e]);
              if (r >= s) aqk[e] = __builtin_fmaf(qr, w, aqk[e]);
            }
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = 16 * Pb + 4 * lq + e, ss = 16 * Q + l16;
        const float lv = L.b[rr] * akk[e];
        if (Pb == Q)
          L.ldg[Pb][4 * lq + e][l16] = ss < rr ? lv : 0.f;
        else
          L.loff[rr][ss] = (_Float16)lv;
        *reinterpret_cast<_Float16*>(blk + OFF_AQ + tri_frag(Pb, ss >> 5) * FRAG + frag_lane_byte(rr, ss)) =
            (_Float16)(ss <= rr ? aqk[e] : 0.f);
      }
    }
    if (w < PNB) {
      {   // inverse of the diagonal block w by forward substitution. Column j = l / 4 runs on
          // four lanes; lane q = l % 4 keeps x_s for s = q (mod 4) in xs[s / 4] and sums
          // those terms (the block stores zeros on and above its diagonal, and xs starts at 0,
          // so not-yet-computed terms add nothing); a butterfly gives all four lanes the sum.
        const int Pb = w, j = l >> 2, q = l & 3;
        // the lane's coefficients L[r][4k + q] (k <= (r - 1) / 4), loaded before the chain
        float lv[16][4];
#pragma unroll
        for (int r = 1; r < 16; ++r)
#pragma unroll
          for (int k = 0; k <= (r - 1) / 4; ++k) lv[r][k] = L.ldg[Pb][r][4 * k + q];
        float x[16], xs[4] = {0.f, 0.f, 0.f, 0.f};
        x[0] = j == 0 ? 1.f : 0.f;
        if (q == 0) xs[0] = x[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) {
          float part = 0.f;
#pragma unroll
          for (int k = 0; k <= (r - 1) / 4; ++k) part = __builtin_fmaf(lv[r][k], xs[k], part);
          float tot = part + quad_xor1(part);
          tot = tot + quad_xor2(tot);
          x[r] = (r == j ? 1.f : 0.f) - tot;
          if ((r & 3) == q) xs[r >> 2] = x[r];
        }
        if (q == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) L.u4.nd[16 * Pb + r][j] = x[r];
        }
      }
    } else if (w >= PNB + 2) {
      const int tt = t - (PNB + 2) * 64;   // 0 .. 127
      // Kbar^T = (F * z)^T, z = decay from the end of block Q to the end of the chunk: the 8
      // tokens s0 .. s0+7 of channel i are one lane's 16 bytes of fragment (i / 16, s0 / 32)
      for (int it = tt; it < PD * (PC / 8); it += 128) {
        const int i = it % PD, s0 = (it / PD) * 8, Q = s0 >> 4;
        float zf = 1.f;
        for (int R = Q + 1; R < PNB; ++R) zf *= L.bp[R][i];
        const _Float16 z = (_Float16)zf;
        half8 fk;
#pragma unroll
        for (int e = 0; e < 8; ++e) fk[e] = L.f16[s0 + e][i];
        *reinterpret_cast<half8*>(blk + OFF_KB + (2 * (i >> 4) + (s0 >> 5)) * FRAG + frag_lane_byte(i, s0)) =
            fk * z;
      }
      // blocks (0,1) and (2,3) lie above the diagonal inside fragments (0,0) and (2,1) of T
      // and A_qk: lanes 32..63, the second half of each fragment
      {
        const int which = tt >> 5, u = tt & 31;   // 4 half-fragments x 32 lanes x 16 bytes
        const int base = (which & 1 ? OFF_AQ : OFF_T) + (which & 2 ? tri_frag(2, 1) : 0) * FRAG + FRAG / 2;
        *reinterpret_cast<uint4*>(blk + base + 16 * u) = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __syncthreads();

  // ---- waves 0-3: T column blocks -----------------------------------------------------------
  switch (w) {
    case 0: t_column<0>(L, blk, l16, lq); break;
    case 1: t_column<1>(L, blk, l16, lq); break;
    case 2: t_column<2>(L, blk, l16, lq); break;
    case 3: t_column<3>(L, blk, l16, lq); break;
    default: break;
  }
}

// ---- state_pass_kernel: the sequential part ---------------------------------------------

typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

// LDS image of one chunk for a work-group with VSW value columns: the operand block, then
// V[64][VSW] bf16 rows. With more load-issuing threads than V units, the threads past the
// last unit repeat the loads of the first ones (same bytes to the same place).
template <int VSW, int NT>
struct StateBuf {
  static constexpr int BYTES = BLOCK_BYTES + PC * VSW * 2;
  static constexpr int VROW_UNITS = VSW / 8;          // 16-byte units per V row
  static constexpr int VUNITS = PC * VROW_UNITS;
  static constexpr int NV = (VUNITS + NT - 1) / NT;   // V units per load-issuing thread
  static_assert((NV * NT) % VUNITS == 0, "V rows split evenly over the threads");
};

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane i of
// the wave writes lds_wave_base + 16 i. lds_wave_base must be wave-uniform. Issued as inline
// assembly so that the compiler does not put a full vmcnt(0) wait in front of every later LDS
// read; completion is awaited explicitly (vm_wait) before the barrier that publishes the
// buffer. M0 is saved and restored around the load; one wait state separates the M0 write
// from the load that reads it.
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(lds_wave_base)
      : "memory");
}
// 4 bytes per lane (global_load_lds_dword): lane i writes lds_wave_base + 4 i. Used only to
// bring lines into L2 ahead of their LDS-direct loads; the LDS bytes it writes are never read.
__device__ __forceinline__ void lds_dma4(const void* gsrc, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(lds_wave_base)
      : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Accumulator tiles lo (rows 0..15) and hi (rows 16..31) of a 32-row k block -> the fp16
// B operand of v_mfma_f32_16x16x32_f16 (lane group g holds k rows 8g .. 8g+7). Lane group g of
// an accumulator tile holds rows 4g .. 4g+3; the two swaps move rows across lane halves so
// that every group ends with 8 consecutive rows. The same registers are the A operand of
// the transposed product (A[l16][8 lq + i] with rows and columns exchanged).
__device__ __forceinline__ half8 acc_pair_to_b(f4 lo, f4 hi) {
  const half4 a = to_h4(lo), b = to_h4(hi);
  const u2v au = __builtin_bit_cast(u2v, a), bu = __builtin_bit_cast(u2v, b);
  // first value: lanes 0-31 keep rows 0..7 of lo, lanes 32-63 take rows 0..7 of hi;
  // second value: rows 8..15 of lo (lanes 0-31) and of hi (lanes 32-63)
  const auto s01 = __builtin_amdgcn_permlane32_swap(au[0], bu[0], false, false);
  const auto s23 = __builtin_amdgcn_permlane32_swap(au[1], bu[1], false, false);
  // per 16-lane row: the first value gets the lower four rows, the second the upper four
  const auto t01 = __builtin_amdgcn_permlane16_swap(s01[0], s01[1], false, false);
  const auto t23 = __builtin_amdgcn_permlane16_swap(s23[0], s23[1], false, false);
  const u4v r = {t01[0], t23[0], t01[1], t23[1]};
  return __builtin_bit_cast(half8, r);
}

// The LDS-direct loads of one chunk, in three groups, each issued as soon as the previous
// chunk in the same buffer has no reader left for that part:
//   kv()  : -Kt and the work-group's V columns   (read by X)
//   qta() : Qt, T and A_qk                       (read by W and O)
//   kbg() : Kbar^T and 2^(G_C)                   (read by the state update)
// Fragment units are t + NT j of each part (NT load-issuing threads). Rows past the sequence
// re-read its last row of V: their T columns and Kbar rows are zero, so any finite value there
// drops out, and O rows past the sequence are never stored.
template <int VSW, int NT>
struct StateFetch {
  using SB = StateBuf<VSW, NT>;
  static constexpr int PART = 16 * FRAG / 16 / NT;           // units per thread of Kt, Qt, Kbar^T
  static constexpr int TRI = 12 * FRAG / 16 / NT;            // units per thread of T and A_qk
  static_assert(PART * NT * 16 == 16 * FRAG && TRI * NT * 16 == 12 * FRAG, "even split");
  static constexpr int N_KV = PART + SB::NV, N_QTA = PART + TRI;
  const char* bsrc;          // operand block of the chunk
  const uint16_t* vsrc;      // V[token 0 of the chunk][head][col0]
  uint32_t buf;              // LDS buffer
  int n, hstr, t, rot;
  __device__ __forceinline__ StateFetch(const char* blk0, const PrefillLaunch& A, int c, int H, int lo,
                                        int len, int h, int col0, int t_, uint32_t buf_)
      : bsrc(blk0 + (size_t)c * H * BLOCK_BYTES),
        buf(buf_),
        hstr(H * PD),
        t(t_),
        rot((col0 / VSW) * 128) {
    int t0;
    chunk_span(c, len, PC, A.ckpt_interval, &t0, &n);
    vsrc = A.t.v + (size_t)(lo + t0) * H * PD + (size_t)h * PD + col0;
  }
  // Units t + NT j of a part of `count` units per thread, whole waves of 64 consecutive units
  // per instruction. The slices of one head (which read the same block on one XCD at about the
  // same time) start at different 2 KiB offsets of the part, spreading their requests over the
  // L2 channels (2.5% on one 8192-token prompt at 16-column slices).
  __device__ __forceinline__ void units(int off, int count) const {
    const int total = NT * count, sh = rot % total, l = t & 63;
#pragma unroll
    for (int j = 0; j < count; ++j) {
      int u0 = (t - l) + NT * j + sh;
      if (u0 >= total) u0 -= total;
      lds_dma16(bsrc + off + 16 * (u0 + l), (uint32_t)__builtin_amdgcn_readfirstlane((int)(buf + off + 16 * u0)));
    }
  }
  __device__ __forceinline__ void kv() const {
    units(OFF_KT, PART);
#pragma unroll
    for (int j = 0; j < SB::NV; ++j) {
      const int u = (t + NT * j) % SB::VUNITS, r = u / SB::VROW_UNITS, q = u % SB::VROW_UNITS;
      // the destination is uniform per wave: unit u lands at 16 u, and the wave's units are
      // consecutive (NT and VUNITS are multiples of 64)
      const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane((int)(buf + BLOCK_BYTES + 16 * (u - (t & 63))));
      lds_dma16(vsrc + (size_t)min(r, n - 1) * hstr + 8 * q, dst);
    }
  }
  __device__ __forceinline__ void qta() const {
    units(OFF_QT, PART);
    units(OFF_T, TRI);
  }
  __device__ __forceinline__ void kbg() const {
    units(OFF_KB, PART);
    if (t < 32) lds_dma16(bsrc + OFF_GAM + 16 * t, buf + OFF_GAM);
  }
};

// One work-group per (sequence, head, slice of VSW value columns). Work-groups run longest
// sequence first and all slices of a head sit on one XCD (shared L2 for the operand blocks).
// CW compute waves, each owning TPW 16-column tiles of the state (VSW = 16 CW TPW), and LW
// load waves that issue every LDS-direct load and wait for it, so the compute waves never stall
// on vector-memory issue. Per chunk every compute wave reads all 60 KiB of the chunk's
// fragments from LDS (a wave drains about 35 bytes per cycle, a CU 128), and each fragment
// feeds TPW products.
//
// Load schedule, buffer c & 1 holding chunk c, one barrier before each group's first use:
//   BX (before X):     -Kt / V of chunk c have landed;         then Kbar^T / 2^(G_C) of c + 1 load
//   BW (before W):     Qt / T / A_qk of chunk c have landed;  then -Kt / V of chunk c + 2 load
//   BS (before S'):    Kbar^T / 2^(G_C) of chunk c landed;     then Qt / T / A_qk of c + 2 load
// Each group reloads into the buffer right after the barrier that follows its last reader, so
// every group has about 1.6-1.75 chunks of lead. A load wave waits before each barrier until
// only the operations issued after the awaited group are pending (the four groups that follow
// it in issue order; the prologue issues kv(0), qta(0), kbg(0), kv(1), qta(1), which gives the
// same counts from chunk 0 on). Lanes 0-31 of load wave 0 also load 2^(G_C) in each kbg group:
// the counts leave that load out, so that wave waits for slightly more than it needs.
// A state-pass work-group has SCW compute waves (one per 16-column tile of a 128-column slice)
// and SLW load waves; a work-group on a narrower slice ends its surplus compute waves at once
// (a barrier counts only the waves still running), except wave SCW - 1, the prefetch wave.
constexpr int SCW = PD / 16;
constexpr int SLW = 4;

// L2 prefetch. The LDS-direct loads of a chunk wait on HBM (the operand blocks and the V rows
// are not in L2 when their group is issued, ~1.7 chunks ahead of use), and the chain's pace is
// set by that latency. Below 128 columns the last compute-wave position (wave SCW - 1) has no
// state tile and becomes a prefetch wave: after the first barrier of chunk c it touches every
// 128-byte line of chunk c + PF's operand block and of its 64 V rows (all columns of the head),
// split over the head's slices, with 4-byte LDS-direct loads into a 256-byte LDS area nobody
// reads. It never waits for them (its vmcnt is its own), so the load waves then find the lines
// in L2: one 8192-token prompt at 16-column slices, state pass 200 -> 183 us. The prefetched
// chunks of the four heads an XCD holds at 16 columns take ~1.5 MiB of its 4 MiB L2; at 32
// columns and wider (more heads per XCD) the prefetch measured no gain and is left off.
constexpr int PF_LINES = BLOCK_BYTES / 128 + 2 * PC;        // 484 block lines + 128 V lines
constexpr int PF_INSTR = (PF_LINES + 63) / 64;               // 10 wave instructions per chunk
static_assert(BLOCK_BYTES % 128 == 0, "whole lines");
constexpr int PF_LDS = 256;                                  // the prefetch wave's LDS area
__host__ __device__ constexpr int prefetch_distance(int vsw) { return vsw == 16 ? 4 : 0; }

// The pass of (sequence, head) chain hg (rank hg / H by length, head hg % H) over value
// columns [VSW vs, VSW (vs + 1)), on the work-group's LDS (two chunk images of StateBuf<VSW>).
template <int VSW>
__device__ __forceinline__ void state_pass_body(const PoolView& P, const PrefillLaunch& A,
                                                const int32_t* __restrict__ choff,
                                                const int32_t* __restrict__ ckoff,
                                                const int32_t* __restrict__ order,
                                                const char* __restrict__ blocks, int hg, int vs,
                                                int wave, char* lds_base, uint32_t pf_lds) {
  constexpr int TPW = 1;                    // 16-column tiles per compute wave
  constexpr int LW = SLW;
  constexpr int NTL = 64 * LW;              // load-issuing threads
  using SB = StateBuf<VSW, NTL>;
  using SF = StateFetch<VSW, NTL>;
  constexpr int N_KBG = SF::PART;           // without the 2^(G_C) load
  constexpr int WAIT_BX = SF::N_QTA + N_KBG + SF::N_KV + SF::N_QTA;
  constexpr int WAIT_BW = N_KBG + SF::N_KV + SF::N_QTA + N_KBG;
  constexpr int WAIT_BS = SF::N_KV + SF::N_QTA + N_KBG + SF::N_KV;
  static_assert(WAIT_BX <= 63 && WAIT_BW <= 63 && WAIT_BS <= 63, "vmcnt holds at most 63");
  const int H = P.H, h = hg % H, si = order[hg / H];
  // Load waves are waves SCW .. SCW + LW - 1; t and w index within a role. Below 128 columns
  // wave SCW - 1 prefetches (it is past the compute waves).
  const bool loads = wave >= SCW;
  const int w = loads ? wave - SCW : wave, t = (int)threadIdx.x - 64 * (wave - w),
            l = t & 63, l16 = l & 15, lq = l >> 4;

  const int lo = A.cu_seqlens[si], len = A.cu_seqlens[si + 1] - lo;
  const int nch = seq_chunks(len, PC, A.ckpt_interval);
  int ck = A.ckpt_interval > 0 ? ckoff[si] : 0;
  const int init = A.init_slot ? A.init_slot[si] : -1;
  const bool has_init = init >= 0 && init < P.num_slots;
  const size_t per = (size_t)H * PD * PD, hoff = (size_t)h * PD * PD;
  const int col0 = vs * VSW;                  // first column of the work-group
  const int cw = 16 * TPW * w;                // first column of the wave, within the slice
  const int colw = col0 + cw;
  const int hst2 = H * PD * 2;
  const char* blk0 = blocks + ((size_t)choff[si] * H + h) * BLOCK_BYTES;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds_base, lds1 = lds0 + SB::BYTES;
  const int64_t pos0 = has_init ? P.meta[init].pos : 0;
  const int nlast = nch - 1;
  auto sf = [&](int c) __attribute__((always_inline)) {   // past the last chunk: repeat it
    return SF(blk0, A, min(c, nlast), H, lo, len, h, col0, t, (c & 1) ? lds1 : lds0);
  };
  if (!loads && wave >= VSW / 16) {
    // ---- prefetch wave (VSW < 128) --------------------------------------------------------------
    constexpr int PF = prefetch_distance(VSW), NVS = PD / VSW;
    if constexpr (PF > 0) {
      auto prefetch = [&](int cc) __attribute__((always_inline)) {
        if (cc > nlast) return;
        int t0, n;
        chunk_span(cc, len, PC, A.ckpt_interval, &t0, &n);
        const char* b = blk0 + (size_t)cc * H * BLOCK_BYTES;
        const char* vrow =
            reinterpret_cast<const char*>(A.t.v + (size_t)(lo + t0) * H * PD + (size_t)h * PD);
        for (int j = vs; j < PF_INSTR; j += NVS) {
          const int x = 64 * j + l;   // line x: block lines, then V rows (two lines each)
          const char* a;
          if (x < BLOCK_BYTES / 128) {
            a = b + 128 * x;
          } else {
            const int y = min(x - BLOCK_BYTES / 128, 2 * PC - 1);
            a = vrow + (size_t)min(y >> 1, n - 1) * hst2 + 128 * (y & 1);
          }
          lds_dma4(a, pf_lds);
        }
      };
      for (int c = 2; c < PF; ++c) prefetch(c);
      for (int c = 0; c < nch; ++c) {
        lds_barrier();   // BX
        prefetch(c + PF);
        lds_barrier();   // BW
        lds_barrier();   // BS
      }
      vm_wait<0>();
      if (A.out_slot[si] >= 0 && A.out_slot[si] < P.num_slots) __syncthreads();
    }
    return;
  }
  if (loads) {
    // ---- load waves ------------------------------------------------------------------------
    if (nch > 0) {
      const SF f0 = sf(0), f1 = sf(1);
      f0.kv();
      f0.qta();
      f0.kbg();
      f1.kv();
      f1.qta();
    }
    for (int c = 0; c < nch; ++c) {
      vm_wait<WAIT_BX>();
      lds_barrier();   // BX
      sf(c + 1).kbg();
      vm_wait<WAIT_BW>();
      lds_barrier();   // BW
      sf(c + 2).kv();
      vm_wait<WAIT_BS>();
      lds_barrier();   // BS
      sf(c + 2).qta();
    }
    vm_wait<0>();   // the last (repeated) loads land before the work-group ends
    if (A.out_slot[si] >= 0 && A.out_slot[si] < P.num_slots) __syncthreads();
    return;
  }

  // ---- compute waves ---------------------------------------------------------------------------
  // S tiles (tile j, row tile rt) in accumulator layout: rows 16 rt + 4 lq + e, column
  // colw + 16 j + l16. Element (j, rt, e) sits at byte svo + (e PD + 16 j) 4 + 16 PD 4 rt of the
  // head's 128 x 128 fp32 matrix: one lane offset, the rest in the instruction's immediate and
  // scalar offsets (no per-element address registers). Without an init slot the buffer range
  // is empty and every load returns 0; all loads are in flight together.
  const int svo = ((4 * lq) * PD + colw + l16) * 4;
  f4 S[TPW][8];
  {
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(P.state + (has_init ? (size_t)init * per + hoff : 0), has_init ? PD * PD * 4 : 0);
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          S[j][rt][e] = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(rs, svo + (e * PD + 16 * j) * 4, rt * 16 * PD * 4, 0));
  }
  auto store_state = [&](int slot) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(P.state + (size_t)slot * per + hoff, PD * PD * 4);
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[j][rt][e]), rd, svo + (e * PD + 16 * j) * 4,
                                                rt * 16 * PD * 4, 0);
  };

  for (int c = 0; c < nch; ++c) {
    int t0, n;
    chunk_span(c, len, PC, A.ckpt_interval, &t0, &n);
    const int tok0 = lo + t0;
    const char* buf = lds_base + (c & 1) * SB::BYTES;
    const _Float16* bh = reinterpret_cast<const _Float16*>(buf);
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(buf + BLOCK_BYTES);
    auto frag = [&](int off, int f) __attribute__((always_inline)) {
      return ld8(bh + (off + f * FRAG) / 2 + 8 * l);
    };

    // S -> B operands (channel blocks kk = 0..3); no LDS involved, ahead of the barrier
    half8 sB[TPW][4], xB[TPW][2], wB[TPW][2];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sB[j][kk] = acc_pair_to_b(S[j][2 * kk], S[j][2 * kk + 1]);
    lds_barrier();   // BX: -Kt and V of this chunk have landed

    // Every phase streams its fragments in small groups: the reads of group g + 1 are issued
    // before the products of group g, with scheduling fences between, so the compiler neither
    // hoists a whole phase's reads (register pressure) nor sinks them into short read / wait /
    // product runs; each group's wait counts down over the reads issued after it.
#define KDA_FENCE() __builtin_amdgcn_sched_barrier(0)
    // X = V + (-Kt) S: the accumulators start from V; groups of four -Kt fragments (one
    // channel block kk, all token tiles)
    {
      f4 X[TPW][4];
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            X[j][rt][e] = __uint_as_float((uint32_t)vb[(16 * rt + 4 * lq + e) * VSW + cw + 16 * j + l16] << 16);
      half8 a[2][4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) a[0][rt] = frag(OFF_KT, 4 * rt);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < 3) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) a[(kk + 1) & 1][rt] = frag(OFF_KT, 4 * rt + kk + 1);
        }
        KDA_FENCE();
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int j = 0; j < TPW; ++j) X[j][rt] = mfma32(a[kk & 1][rt], sB[j][kk], X[j][rt]);
        KDA_FENCE();
      }
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) xB[j][kk] = acc_pair_to_b(X[j][2 * kk], X[j][2 * kk + 1]);
    }
    lds_barrier();   // BW: Qt, T and A_qk of this chunk have landed; -Kt and V are free

    // W = T X (T is zero above the diagonal: token blocks kk <= rt / 2), then
    // O^T = S^T Qt^T + W^T A_qk^T: the operands of O = Qt S + A_qk W with their roles swapped.
    // An accumulator tile then holds O[token 16 rt + l16][columns 4 lq .. 4 lq + 3 of its
    // 16-column tile], stored as 8 bf16 bytes; rows >= n fall outside the buffer range.
    {
      half8 tf[6], q[6], b[2][4];
#pragma unroll
      for (int f = 0; f < 6; ++f) tf[f] = frag(OFF_T, f);
#pragma unroll
      for (int f = 0; f < 6; ++f) q[f] = frag(OFF_AQ, f);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) b[0][kk] = frag(OFF_QT, kk);
      KDA_FENCE();
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        f4 W[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          W[rt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk <= rt / 2; ++kk) W[rt] = mfma32(tf[tri_frag(rt, kk)], xB[j][kk], W[rt]);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) wB[j][kk] = acc_pair_to_b(W[2 * kk], W[2 * kk + 1]);
      }
      KDA_FENCE();
      const __amdgpu_buffer_rsrc_t ro =
          buffer_rsrc(A.t.o + (size_t)tok0 * H * PD + (size_t)h * PD + colw, (uint32_t)(n * hst2));
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (rt < 3) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) b[(rt + 1) & 1][kk] = frag(OFF_QT, 4 * (rt + 1) + kk);
        }
        KDA_FENCE();
        f4 O[TPW];
#pragma unroll
        for (int j = 0; j < TPW; ++j) O[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int j = 0; j < TPW; ++j) O[j] = mfma32(sB[j][kk], b[rt & 1][kk], O[j]);
#pragma unroll
        for (int kk = 0; kk <= rt / 2; ++kk)
#pragma unroll
          for (int j = 0; j < TPW; ++j) O[j] = mfma32(wB[j][kk], q[tri_frag(rt, kk)], O[j]);
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          const u2v ob = __builtin_bit_cast(u2v, __builtin_convertvector(O[j], bf4));
          __builtin_amdgcn_raw_buffer_store_b64(ob, ro, (16 * rt + l16) * hst2 + 32 * j + 8 * lq, 0, 0);
        }
        KDA_FENCE();
      }
    }
    lds_barrier();   // BS: Kbar^T and 2^(G_C) of this chunk have landed; Qt, T, A_qk are free

    // S <- Diag(2^(G_C)) S + Kbar^T W, in groups of two channel tiles
    {
      const float* gam = reinterpret_cast<const float*>(buf + OFF_GAM);
      half8 kb[2][4];
      f4 g[2][2];
      auto rd = [&](int gi, half8* kbp, f4* gp) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kbp[i] = frag(OFF_KB, 4 * gi + i);   // channel tiles 2gi, 2gi+1
#pragma unroll
        for (int i = 0; i < 2; ++i) gp[i] = *reinterpret_cast<const f4*>(gam + 16 * (2 * gi + i) + 4 * lq);
      };
      rd(0, kb[0], g[0]);
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        if (gi < 3) rd(gi + 1, kb[(gi + 1) & 1], g[(gi + 1) & 1]);
        KDA_FENCE();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rt = 2 * gi + i;
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            S[j][rt] *= g[gi & 1][i];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) S[j][rt] = mfma32(kb[gi & 1][2 * i + kk], wB[j][kk], S[j][rt]);
          }
        }
        KDA_FENCE();
      }
    }
#undef KDA_FENCE

    // ---- checkpoint export inside the pass -------------------------------------------------
    const int done = t0 + n;
    if (A.ckpt_interval > 0 && done % A.ckpt_interval == 0) {
      // uniform index: a scalar load through the constant address space (no vector-memory
      // wait behind the chunk's in-flight loads)
      typedef const __attribute__((address_space(4))) int32_t* cptr;
      const int dst = ((cptr)(uintptr_t)A.ckpt_slot)[ck++];
      if (dst >= 0 && dst < P.num_slots) {
        store_state(dst);
        if (t == 0 && h == 0 && vs == 0) {
          kda_slot_meta mm{pos0 + done, 0, 0, 0, 0};
          P.meta[dst] = mm;
        }
      }
    }
  }

  const int out = A.out_slot[si];
  if (out >= 0 && out < P.num_slots) {
    __syncthreads();   // the init slot may be the out slot: every read of it is done
    store_state(out);
    if (t == 0 && h == 0 && vs == 0) {
      kda_slot_meta mm{pos0 + len, 0, 0, 0, 0};
      P.meta[out] = mm;
    }
  }
}

// Work-group bid of the pass: its group g in the width plan (groups run longest sequences
// first), then within the group the slices of a head sit on one XCD (block index mod 8) so that
// they share L2 for the operand blocks.
__global__ __launch_bounds__(64 * (SCW + SLW)) void state_pass_kernel(PoolView P, PrefillLaunch A,
                                                                     const int32_t* __restrict__ choff,
                                                                     const int32_t* __restrict__ ckoff,
                                                                     const int32_t* __restrict__ order,
                                                                     const char* __restrict__ blocks) {
  __shared__ __attribute__((aligned(16))) char lds[2 * StateBuf<PD, 64 * SLW>::BYTES];
  extern __shared__ __attribute__((aligned(16))) char state_pass_dyn[];   // PF_LDS bytes used
  const StatePlan& sp = A.plan;
  const int bid = blockIdx.x;
  int g = 0;
  while (g + 1 < sp.n_groups && bid >= sp.wg_begin[g + 1]) ++g;
  const int vsw = sp.vsw[g], nvs = PD / vsw, r0 = g > 0 ? sp.rank_end[g - 1] : 0;
  const int lb = bid - sp.wg_begin[g], xcd = lb & 7, m = lb >> 3;
  const int hgl = (m / nvs) * 8 + xcd;
  if (hgl >= (sp.rank_end[g] - r0) * P.H) return;
  // the wave index is uniform: derived addresses (buffer descriptors among them) stay scalar
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (wave < SCW && wave >= vsw / 16 && !(wave == SCW - 1 && prefetch_distance(vsw) > 0)) return;
  const int hg = r0 * P.H + hgl, vs = m % nvs;
  const uint32_t pf = (uint32_t)(uintptr_t)state_pass_dyn;
  switch (vsw) {
    case 16: state_pass_body<16>(P, A, choff, ckoff, order, blocks, hg, vs, wave, lds, pf); break;
    case 32: state_pass_body<32>(P, A, choff, ckoff, order, blocks, hg, vs, wave, lds, pf); break;
    case 64: state_pass_body<64>(P, A, choff, ckoff, order, blocks, hg, vs, wave, lds, pf); break;
    default: state_pass_body<128>(P, A, choff, ckoff, order, blocks, hg, vs, wave, lds, pf); break;
  }
}

// ---- d = 16: the chunked form of one (sequence, head) in one wave -------------------------------
// With d = 16 and chunk 16 a chunk's operands are single 16 x 16 tiles, so a wave keeps the whole
// chunked form on chip -- no operand blocks, no workspace -- and runs every product on
// v_mfma_f32_16x16x4_f32 (fp32 operands and accumulation). Lane L = i16 + 16 g:
//   * as an A / B operand at step s of a K = 16 product it holds element (i16, 4 g + s): row i16
//     of A, column i16 of B, index 4 g + s of the contracted dimension;
//   * as an accumulator it holds rows 4 g .. 4 g + 3 of column i16 -- which is exactly the B
//     operand of the next product, so the state S (rows = key channels), X and W pass from one
//     product to the next in registers.
// Per chunk (decays from the chunk start, D_r = prod_{t<=r} a_t, E_s = prod_{t>s} a_t):
//   A_kk = (K D)(K / D)^T (s < r), A_qk = (Q D)(K / D)^T (s <= r), T = (I + Diag(b) A_kk)^-1 Diag(b),
//   X = V - (K D) S, W = T X, O = (Q D) S + A_qk W, S' = Diag(D_15) S + (K E)^T W.
// A key channel whose decay over the chunk is below 2^-60 (where 1 / D could leave the fp32
// range) takes no part in the factored A products; its terms k_r k_s prod_{s<t<=r} a_t are added
// exactly from the raw inputs instead (KDA_DEVERR_DECAY_RANGE, informational).
constexpr int SD = 16;                          // head dim of this form
constexpr int SC = 16;                          // its chunk
constexpr float SMALL_CHUNK_DECAY_MIN = 0x1p-60f;

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// value of lane l - N (row_shr) or l + N (row_shl) inside the lane's 16-lane row, 1 past its ends
template <int CTRL>
__device__ __forceinline__ float row_shift_or_one(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), CTRL, 0xF, 0xF, false));
}

struct SmallLds {
  float m[3][SC][SC + 1];   // Diag(b) A_kk, then T; A_qk; K E (token-major)
  float b[SC];
};

__global__ __launch_bounds__(64) void prefill_small_kernel(PoolView P, PrefillLaunch A) {
  __shared__ SmallLds L;
  const int H = P.H, h = blockIdx.x % H, si = blockIdx.x / H;
  const int l = threadIdx.x, i16 = l & 15, g = l >> 4;
  const int lo = A.cu_seqlens[si], len = A.cu_seqlens[si + 1] - lo;
  const int nch = seq_chunks(len, SC, A.ckpt_interval);
  int ck = 0;   // first checkpoint entry of this sequence
  if (A.ckpt_interval > 0)
    for (int j = 0; j < si; ++j) ck += (A.cu_seqlens[j + 1] - A.cu_seqlens[j]) / A.ckpt_interval;
  const int init = A.init_slot ? A.init_slot[si] : -1;
  const bool has_init = init >= 0 && init < P.num_slots;
  const size_t per = (size_t)H * SD * SD, hoff = (size_t)h * SD * SD, hs = (size_t)H * SD;
  const int64_t pos0 = has_init ? P.meta[init].pos : 0;
  f4 S;   // S[4 g + e][i16]
#pragma unroll
  for (int e = 0; e < 4; ++e) S[e] = has_init ? P.state[init * per + hoff + (4 * g + e) * SD + i16] : 0.f;

  for (int c = 0; c < nch; ++c) {
    int t0, n;
    chunk_span(c, len, SC, A.ckpt_interval, &t0, &n);
    const size_t base = (size_t)(lo + t0) * hs + (size_t)h * SD;   // token 0 of the chunk, this head
    // row i16, channels 4 g .. 4 g + 3; padded rows: k = q = v = 0, a = 1, b = 0
    const bool live = i16 < n;
    f4 av = {1.f, 1.f, 1.f, 1.f}, kv = {0.f, 0.f, 0.f, 0.f}, qv = kv;
    if (live) {
      const float4 a4 = *reinterpret_cast<const float4*>(A.t.a + base + (size_t)i16 * hs + 4 * g);
      av = f4{a4.x, a4.y, a4.z, a4.w};
      const uint2 kw = *reinterpret_cast<const uint2*>(A.t.k + base + (size_t)i16 * hs + 4 * g);
      const uint2 qw = *reinterpret_cast<const uint2*>(A.t.q + base + (size_t)i16 * hs + 4 * g);
      kv = f4{bf2f(kw.x & 0xffffu), bf2f(kw.x >> 16), bf2f(kw.y & 0xffffu), bf2f(kw.y >> 16)};
      qv = f4{bf2f(qw.x & 0xffffu), bf2f(qw.x >> 16), bf2f(qw.y & 0xffffu), bf2f(qw.y >> 16)};
    }
    f4 X;   // starts as V[4 g + e][i16]
#pragma unroll
    for (int e = 0; e < 4; ++e) X[e] = 4 * g + e < n ? bf2f(A.t.v[base + (size_t)(4 * g + e) * hs + i16]) : 0.f;
    if (g == 0) L.b[i16] = live ? A.t.b[(size_t)(lo + t0 + i16) * H + h] : 0.f;

    // decays down the rows (the lanes of each 16-lane row): inclusive prefix D, exclusive suffix E
    f4 Dp, Es;
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx) {
      float d = av[sidx];
      d *= row_shift_or_one<0x111>(d);
      d *= row_shift_or_one<0x112>(d);
      d *= row_shift_or_one<0x114>(d);
      d *= row_shift_or_one<0x118>(d);
      Dp[sidx] = d;
      float e = row_shift_or_one<0x101>(av[sidx]);
      e *= row_shift_or_one<0x101>(e);
      e *= row_shift_or_one<0x102>(e);
      e *= row_shift_or_one<0x104>(e);
      e *= row_shift_or_one<0x108>(e);
      Es[sidx] = e;
    }
    // the chunk's decay of channel 4 g + s (row 15 of this lane group)
    f4 gam;
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx) gam[sidx] = __shfl(Dp[sidx], 16 * g + 15);
    uint32_t fast = 0;   // channels (bit = channel) below SMALL_CHUNK_DECAY_MIN
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx) {
      const uint64_t bal = __ballot(i16 == 0 && gam[sidx] < SMALL_CHUNK_DECAY_MIN);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) fast |= (uint32_t)((bal >> (16 * gg)) & 1u) << (4 * gg + sidx);
    }
    fast = (uint32_t)__builtin_amdgcn_readfirstlane((int)fast);
    if (fast && l == 0) atomicOr(P.err, (uint32_t)KDA_DEVERR_DECAY_RANGE);

    f4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = akk;
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx) {
      const float ki = (fast >> (4 * g + sidx)) & 1u ? 0.f : kv[sidx] / Dp[sidx];
      akk = mfma4(kv[sidx] * Dp[sidx], ki, akk);
      aqk = mfma4(qv[sidx] * Dp[sidx], ki, aqk);
    }
    if (fast) {   // exact terms of the fast channels: column i16, rows 4 g + e
      const size_t cb = (size_t)(lo + t0) * hs + (size_t)h * SD;
      uint32_t msk = fast;
      while (msk) {
        const int ch = __builtin_ctz(msk);
        msk &= msk - 1;
        float run = 1.f, dec[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int tt = 0; tt < SC; ++tt) {
          const float a_t = tt < n ? A.t.a[cb + (size_t)tt * hs + ch] : 1.f;
          if (tt > i16) run *= a_t;
          if ((tt >> 2) == g) dec[0] = (tt & 3) == 0 ? run : dec[0];
          if ((tt >> 2) == g) dec[1] = (tt & 3) == 1 ? run : dec[1];
          if ((tt >> 2) == g) dec[2] = (tt & 3) == 2 ? run : dec[2];
          if ((tt >> 2) == g) dec[3] = (tt & 3) == 3 ? run : dec[3];
        }
        const float ks = i16 < n ? bf2f(A.t.k[cb + (size_t)i16 * hs + ch]) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float kr = r < n ? bf2f(A.t.k[cb + (size_t)r * hs + ch]) : 0.f;
          const float qr = r < n ? bf2f(A.t.q[cb + (size_t)r * hs + ch]) : 0.f;
          const float wgt = ks * dec[e];
          if (r > i16) akk[e] = __builtin_fmaf(kr, wgt, akk[e]);
          if (r >= i16) aqk[e] = __builtin_fmaf(qr, wgt, aqk[e]);
        }
      }
    }
    __syncthreads();   // b landed; the previous chunk's readers of m[] are done
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * g + e;
      L.m[0][r][i16] = i16 < r ? L.b[r] * akk[e] : 0.f;   // Diag(b) A_kk, strictly lower
      L.m[1][r][i16] = i16 <= r ? aqk[e] : 0.f;           // A_qk, lower
    }
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx) L.m[2][i16][4 * g + sidx] = kv[sidx] * Es[sidx];   // K E
    __syncthreads();
    // T = (I + Diag(b) A_kk)^-1 Diag(b): lanes 0..15 each solve one column j by forward
    // substitution, then scale it by b_j; written over Diag(b) A_kk row by row (row r is read
    // only by rows after it, and each lane works on its own column)
    if (l < SC) {
      const int j = l;
      float x[SC];
#pragma unroll
      for (int r = 0; r < SC; ++r) {
        float acc = r == j ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) acc = __builtin_fmaf(-L.m[0][r][m], x[m], acc);
        x[r] = acc;
      }
      const float bj = L.b[j];
#pragma unroll
      for (int r = 0; r < SC; ++r) L.m[0][r][j] = x[r] * bj;
    }
    __syncthreads();

    // X = V - (K D) S; W = T X; O = (Q D) S + A_qk W; S' = Diag(gamma) S + (K E)^T W
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx) X = mfma4(-(kv[sidx] * Dp[sidx]), S[sidx], X);
    f4 W = {0.f, 0.f, 0.f, 0.f}, O = W;
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx) W = mfma4(L.m[0][i16][4 * g + sidx], X[sidx], W);
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx) {
      O = mfma4(qv[sidx] * Dp[sidx], S[sidx], O);
      O = mfma4(L.m[1][i16][4 * g + sidx], W[sidx], O);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * g + e;
      if (r < n) A.t.o[base + (size_t)r * hs + i16] = (uint16_t)(pack_bf2(O[e], 0.f) & 0xffffu);
    }
    f4 Sn;
#pragma unroll
    for (int e = 0; e < 4; ++e) Sn[e] = S[e] * __shfl(Dp[e], 16 * g + 15);   // gamma of row 4 g + e
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx) Sn = mfma4(L.m[2][4 * g + sidx][i16], W[sidx], Sn);
    S = Sn;

    const int done = t0 + n;
    if (A.ckpt_interval > 0 && done % A.ckpt_interval == 0) {
      const int dst = A.ckpt_slot[ck++];
      if (dst >= 0 && dst < P.num_slots) {
#pragma unroll
        for (int e = 0; e < 4; ++e) P.state[dst * per + hoff + (4 * g + e) * SD + i16] = S[e];
        if (l == 0 && h == 0) {
          kda_slot_meta mm{pos0 + done, 0, 0, 0, 0};
          P.meta[dst] = mm;
        }
      }
    }
  }
  const int out = A.out_slot[si];
  if (out >= 0 && out < P.num_slots) {
#pragma unroll
    for (int e = 0; e < 4; ++e) P.state[out * per + hoff + (4 * g + e) * SD + i16] = S[e];
    if (l == 0 && h == 0) {
      kda_slot_meta mm{pos0 + len, 0, 0, 0, 0};
      P.meta[out] = mm;
    }
  }
}


hipError_t launch_state(const PoolView& p, const PrefillLaunch& a, const int32_t* choff,
                        const int32_t* ckoff, const int32_t* order, const char* blocks, hipStream_t s) {
  const int nb = a.plan.wg_begin[a.plan.n_groups];
  if (nb <= 0) return hipSuccess;
  // The rest of the CU's LDS is requested too (unused), so that no other work-group shares a CU
  // with a state-pass work-group: in a mixed batch the decode and verify kernels on the side
  // stream then run on the CUs the pass leaves free instead of slowing its sequential chain.
  constexpr int lds_static = 2 * StateBuf<PD, 64 * SLW>::BYTES;
  static_assert(lds_static + PF_LDS <= LDS_PER_CU, "state pass LDS image and prefetch area");
  hipLaunchKernelGGL(state_pass_kernel, dim3(nb), dim3(64 * (SCW + SLW)), LDS_PER_CU - lds_static, s, p,
                     a, choff, ckoff, order, blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t prefill_scratch(void** out) {
  // Device address of `scratch` on the current device, looked up once per device (each GPU
  // holds its own copy at its own address) and kept for later calls.
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* per_device[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    per_device[dev] = ptr;
  }
  *out = per_device[dev];
  return hipSuccess;
}

hipError_t launch_prefill(const PoolView& p, const PrefillLaunch& a, hipStream_t s) {
  if (a.n_seq <= 0) return hipSuccess;
  if (p.dk == SD && a.chunk == SC) {
    hipLaunchKernelGGL(prefill_small_kernel, dim3((unsigned)(a.n_seq * p.H)), dim3(64), 0, s, p, a);
    return hipGetLastError();
  }
  if (p.dk != PD || a.chunk != PC) return hipErrorInvalidValue;
  char* ws = static_cast<char*>(a.workspace);
  int32_t* choff = reinterpret_cast<int32_t*>(ws);
  int32_t* ckoff = choff + (a.n_seq + 1);
  int32_t* order = ckoff + a.n_seq;
  char* blocks = ws + prefill_plan_bytes(a.n_seq);
  hipError_t e = hipSuccess;
  if (a.n_seq > PLAN_INLINE_MAX || a.n_chunks == 0) {
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, s, a.cu_seqlens, a.n_seq,
                       a.ckpt_interval, choff, ckoff, order);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_chunks > 0) {
    hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)(a.n_chunks * p.H)), dim3(PNT), 0, s, p, a,
                       choff, ckoff, order, blocks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_state(p, a, choff, ckoff, order, blocks, s);
}

}  // namespace kda
