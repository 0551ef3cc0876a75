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
// Design for MI355X:
//   * one work-group (8 waves, two per SIMD) per (sequence, head, slice of VS value columns).
//     Value columns of S evolve independently, so slices need no exchange; the launcher picks
//     VS in {16, 32, 64, 128} so that sequences x heads x slices stays within two rounds of
//     CUs (a lone 8192-token prompt at 32 heads runs 8 slices per head, a batch of 6 prompts
//     2 slices), and work-groups start longest sequence first. The S-independent part
//     (A_kk, A_qk, T) is recomputed per slice.
//   * all contractions run on v_mfma_f32_16x16x32_f16 / 16x16x16f16 with fp32 accumulation.
//     fp16 operands (same rate as bf16, 3 more mantissa bits) keep the chunked form within
//     2e-3 of the sequential fp64 result; bf16 operands do not (5e-3 in emulation). The state
//     stays fp32 in MFMA accumulator registers across chunks; only operand copies are fp16.
//   * every exponential factor is at most 1 except the column factor of the diagonal 16x16
//     blocks of A_kk / A_qk, bounded by the 16-token decay of the block; beyond 2^14 on any
//     channel the kernel flags KDA_DEVERR_DECAY_RANGE.
//   * the next chunk's q/k/a/v/b are loaded into registers while the current chunk computes.
//   * block ids are mapped so that all slices of one head run on the same XCD and share its L2.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int PD = 128;           // head dim (dk = dv)
constexpr int PC = 64;            // chunk
constexpr int PNB = PC / 16;      // 16-row blocks per chunk
constexpr int PNW = 8;            // waves per work-group
constexpr int PNT = 64 * PNW;
constexpr int P16 = PD + 8;       // row pitch (halves) of [.][PD] fp16 arrays
constexpr int PG = PD + 4;        // row pitch (floats) of the G array (16-row fragment reads hit
                                  // every LDS bank exactly four times)
constexpr int PC16 = PC + 8;      // row pitch (halves) of [.][PC] fp16 arrays
constexpr int PL = PC + 8;        // row pitch (floats) of the fp32 [PC][PC] array
constexpr int NPAIR = PNB * (PNB + 1) / 2;
constexpr float DIAG_LOG2_LIMIT = 14.f;

template <int VS>
struct PfLds {
  _Float16 kt[PC][P16];      // Kt = k 2^G (fp16)
  _Float16 qt[PC][P16];      // Qt = q 2^G (fp16)
  union {
    struct {                 // A-operands of A_kk / A_qk: rows of block P times 2^(G - G_start(P))
      _Float16 ka[PC][P16];
      _Float16 qa[PC][P16];
    } a;
    _Float16 s16t[VS][P16];  // S^T (fp16 operand copy)
  } u1;
  _Float16 kbt[PD][PC16];    // Kbar^T
  union {
    float l32[PC][PL];       // Diag(b) A_kk, strictly lower
    _Float16 x16t[VS][PC16]; // X^T
  } u2;
  union {
    _Float16 f16[PC][P16];   // F_s = k_s 2^(G_end(block of s) - G_s)
    _Float16 w16t[VS][PC16]; // W^T
  } u3;
  _Float16 aqk[PC][PC16];    // A_qk, zero above the diagonal
  _Float16 t16[PC][PC16];    // T, zero above the diagonal
  union {
    float part[PC / 4][PD];  // sums of log2 a over each group of 4 rows
    float nd[PC][16];        // diagonal 16x16 blocks of (I + Diag(b) A_kk)^-1
  } u4;
  float ge[PNB][PD];         // G at the last row of each block
  _Float16 xvh[NPAIR][PD];   // 2^(G_start(P) - G_end(Q)) per pair, fp16
  float gam[PD];             // 2^(G_C)
  float b[PC];
};

__device__ __forceinline__ f4 mfma32(half8 a, half8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(half4 a, half4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// Decay factors use the hardware exp2 / log2 (the fast path of HIP's math library): a result
// below 2^-126 flushes to zero, which only drops contributions already below fp32 resolution.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __log2f(x); }

__device__ __forceinline__ half8 ld8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }
__device__ __forceinline__ void ld_f8(const float* p, float (&f)[8]) {
  f4 x = *reinterpret_cast<const f4*>(p), y = *reinterpret_cast<const f4*>(p + 4);
  f[0] = x[0]; f[1] = x[1]; f[2] = x[2]; f[3] = x[3]; f[4] = y[0]; f[5] = y[1]; f[6] = y[2]; f[7] = y[3];
}
__device__ __forceinline__ void unpack8(const _Float16* raw, float (&f)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(raw);
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(ws[e] << 16);
    f[2 * e + 1] = __uint_as_float(ws[e] & 0xffff0000u);
  }
}
// fp32 -> fp16 (round to nearest even) as packed conversions (v_cvt_pk_f16_f32)
__device__ __forceinline__ half4 to_h4(f4 x) { return __builtin_convertvector(x, half4); }

// Work-group barrier for LDS hand-offs inside the chunk loop: waits for this wave's LDS
// operations only. Global loads (the next chunk's prefetch) and stores (outputs, checkpoints)
// stay in flight across it; no wave of the work-group reads what another wave stores to global
// memory in the loop, and the loop never reads a register before its load has been waited on.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Index of the sequence with the given rank in descending length order (ties: lower index
// first). Uniform across the work-group; O(n_seq^2), used once per work-group.
__device__ __forceinline__ int seq_by_rank(const int32_t* cu, int n_seq, int rank) {
  if (n_seq > 256) return rank;
  for (int j = 0; j < n_seq; ++j) {
    const int lj = cu[j + 1] - cu[j];
    int rj = 0;
    for (int k = 0; k < n_seq; ++k) {
      const int lk = cu[k + 1] - cu[k];
      rj += (lk > lj) || (lk == lj && k < j);
    }
    if (rj == rank) return j;
  }
  return rank;
}

// pair index p = P(P+1)/2 + Q for Q <= P
__device__ __forceinline__ int pair_p(int p) { return p >= 6 ? 3 : (p >= 3 ? 2 : (p >= 1 ? 1 : 0)); }

// Column block Q of T = N Diag(b), N = (I + Diag(b) A_kk)^-1, from the diagonal inverses:
// N_PQ = -N_PP sum_{Q<=R<P} L_PR N_RQ, 16x16x16 fp16 products with fp32 accumulation. The
// accumulator layout of a 16x16x16 product equals its B-operand layout, so N_RQ stays in
// registers from one product to the next.
template <int Q, class Lds>
__device__ __forceinline__ void t_column(Lds& L, int l16, int lq) {
  f4 nq[PNB];
#pragma unroll
  for (int e = 0; e < 4; ++e) nq[Q][e] = L.u4.nd[16 * Q + 4 * lq + e][l16];
  const float bq = L.b[16 * Q + l16];
#pragma unroll
  for (int e = 0; e < 4; ++e) L.t16[16 * Q + 4 * lq + e][16 * Q + l16] = (_Float16)(nq[Q][e] * bq);
#pragma unroll
  for (int Pb = Q + 1; Pb < PNB; ++Pb) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int R = Q; R < Pb; ++R) {
      const f4 lr = *reinterpret_cast<const f4*>(&L.u2.l32[16 * Pb + l16][16 * R + 4 * lq]);
      acc = mfma16(to_h4(lr), to_h4(nq[R]), acc);
    }
    const f4 np = *reinterpret_cast<const f4*>(&L.u4.nd[16 * Pb + l16][4 * lq]);
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    nq[Pb] = -mfma16(to_h4(np), to_h4(acc), zero);
#pragma unroll
    for (int e = 0; e < 4; ++e) L.t16[16 * Pb + 4 * lq + e][16 * Q + l16] = (_Float16)(nq[Pb][e] * bq);
  }
}

// Raw inputs of one chunk, held in registers between chunks (prefetch). Thread t owns key
// rows 4m .. 4m+3 (m = t / 32) and key channels 4cq .. 4cq+3 (cq = t % 32): a row of 32
// threads reads 256 contiguous bytes of q / k and 512 of a.
template <int VS>
struct Stage {
  static constexpr int NCT = VS / 16;
  static constexpr int NXT = (4 * NCT + PNW - 1) / PNW;   // X tiles per wave
  uint2 k[4], q[4];       // 4 bf16 each
  float4 a[4];
  uint32_t v[NXT][4];     // V of the wave's X tiles: bf16 bits, rows 4*lq+e (kept unpacked so
                          // that nothing waits on these loads before the next chunk)
  float b;
};

template <int VS>
__device__ __forceinline__ void load_stage(Stage<VS>& st, const PrefillLaunch& A, size_t tok0, int n,
                                           int h, int H, int col0, int t, int w, int l16, int lq) {
  constexpr int NCT = VS / 16;
  const size_t hstride = (size_t)H * PD;
  const int m = t >> 5, c4 = (t & 31) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * m + i;
    uint2 kk = make_uint2(0, 0), qq = make_uint2(0, 0);
    float4 av = make_float4(1.f, 1.f, 1.f, 1.f);
    if (r < n) {
      const size_t off = (tok0 + r) * hstride + (size_t)h * PD + c4;
      kk = *reinterpret_cast<const uint2*>(A.t.k + off);
      qq = *reinterpret_cast<const uint2*>(A.t.q + off);
      av = *reinterpret_cast<const float4*>(A.t.a + off);
    }
    st.k[i] = kk;
    st.q[i] = qq;
    st.a[i] = av;
  }
#pragma unroll
  for (int j = 0; j < Stage<VS>::NXT; ++j) {
    const int it = w + PNW * j;
    if (it < 4 * NCT) {
      const int rt = it & 3, ct = it >> 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * lq + e;
        st.v[j][e] = r < n ? A.t.v[(tok0 + r) * hstride + (size_t)h * PD + col0 + 16 * ct + l16] : 0u;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) st.v[j][e] = 0u;
    }
  }
  st.b = (t < n) ? A.t.b[(tok0 + t) * H + h] : 0.f;
}

template <int VS>
__global__ __launch_bounds__(PNT) void prefill_chunk_kernel(PoolView P, PrefillLaunch A, int n_hg) {
  constexpr int NVS = PD / VS, NCT = VS / 16;
  constexpr int NS = 8 * NCT / PNW;                       // S tiles per wave
  constexpr int NXT = Stage<VS>::NXT;
  static_assert(8 * NCT % PNW == 0, "S tiles must divide among the waves");
  __shared__ PfLds<VS> L;
  const int bid = blockIdx.x, xcd = bid & 7, m = bid >> 3;
  const int vs = m % NVS, hg = (m / NVS) * 8 + xcd;
  if (hg >= n_hg) return;
  // Work-groups are dispatched in block order: sequence rank 0 (the longest; ties by index)
  // first, so the longest recurrences start before the short ones fill the remaining CUs.
  const int H = P.H, h = hg % H;
  const int si = seq_by_rank(A.cu_seqlens, A.n_seq, hg / H);
  const int t = threadIdx.x, w = t >> 6, l = t & 63, l16 = l & 15, lq = l >> 4;

  const int lo = A.cu_seqlens[si], hi = A.cu_seqlens[si + 1], len = hi - lo;
  int ck = 0;
  if (A.ckpt_interval > 0)
    for (int j = 0; j < si; ++j) ck += (A.cu_seqlens[j + 1] - A.cu_seqlens[j]) / A.ckpt_interval;
  const int init = A.init_slot ? A.init_slot[si] : -1;
  const bool has_init = init >= 0 && init < P.num_slots;
  const size_t per = (size_t)H * PD * PD, hoff = (size_t)h * PD * PD;
  const int col0 = vs * VS;
  const size_t hstride = (size_t)H * PD;

  // State slice in accumulator layout. Wave w owns S tiles it = w + PNW*j: row tile
  // it % 8 (key channels 16*rt + 4*lq + e), column tile it / 8 (col0 + 16*ct + l16).
  f4 S[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int it = w + PNW * j, rt = it & 7, ct = it >> 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + 4 * lq + e;
      S[j][e] = has_init ? P.state[init * per + hoff + (size_t)row * PD + col0 + 16 * ct + l16] : 0.f;
    }
  }
  const int64_t pos0 = has_init ? P.meta[init].pos : 0;

  // T and A_qk are lower triangular; their upper blocks stay zero for the whole kernel.
  for (int i = t; i < PC * PC16; i += PNT) {
    (&L.aqk[0][0])[i] = (_Float16)0.f;
    (&L.t16[0][0])[i] = (_Float16)0.f;
  }

  Stage<VS> st;
  if (len > 0) load_stage<VS>(st, A, (size_t)lo, min(PC, len), h, H, col0, t, w, l16, lq);

  for (int c0 = 0; c0 < len; c0 += PC) {
    const int n = min(PC, len - c0);
    const size_t tok0 = (size_t)(lo + c0);
    lds_barrier();   // previous chunk's readers are done with every array below
    // Lane indices re-derived through an opaque copy each chunk: LDS addresses are then
    // recomputed per chunk instead of being hoisted out of the loop, where they would hold
    // about a hundred VGPRs for the whole kernel.
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int t = tid, l = t & 63, l16 = l & 15, lq = l >> 4;

    // ---- G = cumulative log2 a over the chunk's rows, per key channel: in registers over
    //      the thread's 4 rows, then one exchange of the 16 row-group sums through LDS ------
    const int m4 = t >> 5, c4 = (t & 31) * 4, Pm = m4 >> 2;
    uint2 kcur[4], qcur[4];
    f4 Gl[4];
    {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc += f4{flog2(st.a[i].x), flog2(st.a[i].y), flog2(st.a[i].z), flog2(st.a[i].w)};
        Gl[i] = acc;
        kcur[i] = st.k[i];
        qcur[i] = st.q[i];
      }
      *reinterpret_cast<f4*>(&L.u4.part[m4][c4]) = acc;
    }
    if (t < PC) L.b[t] = st.b;
    uint32_t vcur[NXT][4];
#pragma unroll
    for (int j = 0; j < NXT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) vcur[j][e] = st.v[j][e];
    // prefetch the next chunk while this one computes
    if (c0 + PC < len) load_stage<VS>(st, A, tok0 + PC, min(PC, len - c0 - PC), h, H, col0, t, w, l16, lq);
    lds_barrier();

    // ---- decayed fp16 operands from registers: Ka/Qa (rows of block P times 2^(G - G_start(P))),
    //      F (times 2^(G_end(P) - G)), Kt/Qt (times 2^G); every factor is <= 1. Each thread sums
    //      the row-group totals in the same order, so G at a block's last row equals G_end. ------
    {
      // Row-group sums in increasing order: whole blocks before this one (a wave-uniform
      // loop), then the four groups of this block. gs = G before the block, pre = G before
      // the thread's rows, gend = G at the block's last row; every thread of a block adds the
      // same terms in the same order, so G at a block's last row equals gend exactly.
      f4 gs = {0.f, 0.f, 0.f, 0.f};
      for (int mm = 0; mm < 4 * Pm; ++mm) gs += *reinterpret_cast<const f4*>(&L.u4.part[mm][c4]);
      f4 blk[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) blk[q] = *reinterpret_cast<const f4*>(&L.u4.part[4 * Pm + q][c4]);
      const int mq = m4 & 3;
      const f4 s1 = gs + blk[0], s2 = s1 + blk[1], s3 = s2 + blk[2];
      const f4 pre = mq == 0 ? gs : (mq == 1 ? s1 : (mq == 2 ? s2 : s3));
      const f4 gend = s3 + blk[3];
      if ((m4 & 3) == 3) {
        *reinterpret_cast<f4*>(&L.ge[Pm][c4]) = gend;
        if (Pm == PNB - 1)
          *reinterpret_cast<f4*>(&L.gam[c4]) = f4{fexp2(gend[0]), fexp2(gend[1]), fexp2(gend[2]), fexp2(gend[3])};
        const f4 dec = gs - gend;   // log2 of the inverse decay of this block, >= 0
        if (dec[0] > DIAG_LOG2_LIMIT || dec[1] > DIAG_LOG2_LIMIT || dec[2] > DIAG_LOG2_LIMIT ||
            dec[3] > DIAG_LOG2_LIMIT)
          atomicOr(P.err, (uint32_t)KDA_DEVERR_DECAY_RANGE);
      }
      const f4 y = {fexp2(gs[0]), fexp2(gs[1]), fexp2(gs[2]), fexp2(gs[3])};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * m4 + i;
        const float kr[4] = {__uint_as_float(kcur[i].x << 16), __uint_as_float(kcur[i].x & 0xffff0000u),
                             __uint_as_float(kcur[i].y << 16), __uint_as_float(kcur[i].y & 0xffff0000u)};
        const float qr[4] = {__uint_as_float(qcur[i].x << 16), __uint_as_float(qcur[i].x & 0xffff0000u),
                             __uint_as_float(qcur[i].y << 16), __uint_as_float(qcur[i].y & 0xffff0000u)};
        f4 ka, qa, kt, qt, fv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float G = pre[e] + Gl[i][e];
          const float e1 = fexp2(G - gs[e]);
          ka[e] = kr[e] * e1;
          qa[e] = qr[e] * e1;
          kt[e] = ka[e] * y[e];
          qt[e] = qa[e] * y[e];
          fv[e] = kr[e] * fexp2(gend[e] - G);
        }
        *reinterpret_cast<half4*>(&L.u1.a.ka[r][c4]) = to_h4(ka);
        *reinterpret_cast<half4*>(&L.u1.a.qa[r][c4]) = to_h4(qa);
        *reinterpret_cast<half4*>(&L.kt[r][c4]) = to_h4(kt);
        *reinterpret_cast<half4*>(&L.qt[r][c4]) = to_h4(qt);
        *reinterpret_cast<half4*>(&L.u3.f16[r][c4]) = to_h4(fv);
      }
    }
    lds_barrier();

    // ---- A_kk, A_qk block pairs on matrix cores. Waves 0-3: diagonal pair (w, w), then the
    //      inverse of that block by forward substitution (the wave's own LDS writes, no
    //      barrier needed). Waves 4-7: the six off-diagonal pairs; waves 6-7 also Kbar^T. -----
    {
      // pair index p = P(P+1)/2 + Q: diagonal pairs 0, 2, 5, 9; off-diagonal 1, 3, 4, 6, 7, 8
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
        {   // this pair's column factor, two channels per lane (read back by this wave only)
          const int i0 = 2 * l;
          const float g0 = Pb > 0 ? L.ge[Pb - 1][i0] : 0.f, g1 = Pb > 0 ? L.ge[Pb - 1][i0 + 1] : 0.f;
          L.xvh[p][i0] = (_Float16)fexp2(g0 - L.ge[Q][i0]);
          L.xvh[p][i0 + 1] = (_Float16)fexp2(g1 - L.ge[Q][i0 + 1]);
        }
        f4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < PD / 32; ++kk) {
          const int c = 32 * kk + 8 * lq;
          // k_s 2^(G_start(P) - G_s) = F_s 2^(G_start(P) - G_end(Q)), packed fp16 products
          const half8 bb = ld8(&L.u3.f16[16 * Q + l16][c]) * ld8(&L.xvh[p][c]);
          akk = mfma32(ld8(&L.u1.a.ka[16 * Pb + l16][c]), bb, akk);
          aqk = mfma32(ld8(&L.u1.a.qa[16 * Pb + l16][c]), bb, aqk);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 16 * Pb + 4 * lq + e, ss = 16 * Q + l16;
          L.u2.l32[rr][ss] = ss < rr ? L.b[rr] * akk[e] : 0.f;
          L.aqk[rr][ss] = (_Float16)(ss <= rr ? aqk[e] : 0.f);
        }
      }
      if (w < PNB) {
        {   // inverse of the diagonal block w by forward substitution. Column j = l / 4 runs on
            // four lanes; lane q = l % 4 keeps x_s for s = q (mod 4) in xs[s / 4] and sums
            // those terms (the block stores zeros on and above its diagonal, and xs starts at 0,
            // so not-yet-computed terms add nothing); a butterfly gives all four lanes the sum.
          const int Pb = w, j = l >> 2, q = l & 3;
          float x[16], xs[4] = {0.f, 0.f, 0.f, 0.f};
          x[0] = j == 0 ? 1.f : 0.f;
          if (q == 0) xs[0] = x[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) {
            float part = 0.f;
#pragma unroll
            for (int k = 0; k <= (r - 1) / 4; ++k)
              part = __builtin_fmaf(L.u2.l32[16 * Pb + r][16 * Pb + 4 * k + q], xs[k], part);
            float tot = part + __shfl_xor(part, 1);
            tot = tot + __shfl_xor(tot, 2);
            x[r] = (r == j ? 1.f : 0.f) - tot;
            if ((r & 3) == q) xs[r >> 2] = x[r];
          }
          if (q == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) L.u4.nd[16 * Pb + r][j] = x[r];
          }
        }
      } else if (w >= PNB + 2) {   // Kbar^T = (F * zv)^T
        for (int it = t - (PNB + 2) * 64; it < PD * (PC / 8); it += (PNW - PNB - 2) * 64) {
          const int i = it % PD, s0 = (it / PD) * 8, Q = s0 >> 4;
          const _Float16 z = (_Float16)fexp2(L.ge[PNB - 1][i] - L.ge[Q][i]);
          half8 fk;
#pragma unroll
          for (int e = 0; e < 8; ++e) fk[e] = L.u3.f16[s0 + e][i];
          *reinterpret_cast<half8*>(&L.kbt[i][s0]) = fk * z;
        }
      }
    }
    lds_barrier();

    // ---- waves 0-3: T column blocks; then every wave: fp16 copy of its S^T tiles --------
    if (w < PNB) {
      switch (w) {
        case 0: t_column<0>(L, l16, lq); break;
        case 1: t_column<1>(L, l16, lq); break;
        case 2: t_column<2>(L, l16, lq); break;
        default: t_column<3>(L, l16, lq); break;
      }
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int it = w + PNW * j, rt = it & 7, ct = it >> 3;
      *reinterpret_cast<half4*>(&L.u1.s16t[16 * ct + l16][16 * rt + 4 * lq]) = to_h4(S[j]);
    }
    lds_barrier();

    // ---- X = V - Kt S --------------------------------------------------------------------
#pragma unroll
    for (int j = 0; j < NXT; ++j) {
      const int it = w + PNW * j;
      if (it < 4 * NCT) {
        const int rt = it & 3, ct = it >> 2;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < PD / 32; ++kk)
          acc = mfma32(ld8(&L.kt[16 * rt + l16][32 * kk + 8 * lq]),
                       ld8(&L.u1.s16t[16 * ct + l16][32 * kk + 8 * lq]), acc);
        f4 xv;
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[e] = __uint_as_float(vcur[j][e] << 16) - acc[e];
        *reinterpret_cast<half4*>(&L.u2.x16t[16 * ct + l16][16 * rt + 4 * lq]) = to_h4(xv);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();

    // ---- W = T X (T is zero above the diagonal) --------------------------------------------
#pragma unroll
    for (int j = 0; j < NXT; ++j) {
      const int it = w + PNW * j;
      if (it < 4 * NCT) {
        const int rt = it & 3, ct = it >> 2;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk <= (rt >> 1); ++kk)
          acc = mfma32(ld8(&L.t16[16 * rt + l16][32 * kk + 8 * lq]),
                       ld8(&L.u2.x16t[16 * ct + l16][32 * kk + 8 * lq]), acc);
        *reinterpret_cast<half4*>(&L.u3.w16t[16 * ct + l16][16 * rt + 4 * lq]) = to_h4(acc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();

    // ---- O = Qt S + A_qk W; S <- Diag(gamma) S + Kbar^T W -------------------------------------
#pragma unroll
    for (int j = 0; j < NXT; ++j) {
      const int it = w + PNW * j;
      if (it < 4 * NCT) {
        const int rt = it & 3, ct = it >> 2;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < PD / 32; ++kk)
          acc = mfma32(ld8(&L.qt[16 * rt + l16][32 * kk + 8 * lq]),
                       ld8(&L.u1.s16t[16 * ct + l16][32 * kk + 8 * lq]), acc);
        for (int kk = 0; kk <= (rt >> 1); ++kk)
          acc = mfma32(ld8(&L.aqk[16 * rt + l16][32 * kk + 8 * lq]),
                       ld8(&L.u3.w16t[16 * ct + l16][32 * kk + 8 * lq]), acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * lq + e;
          if (r < n) A.t.o[(tok0 + r) * hstride + (size_t)h * PD + col0 + 16 * ct + l16] = (uint16_t)f2bf(acc[e]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int it = w + PNW * j, rt = it & 7, ct = it >> 3;
#pragma unroll
      for (int e = 0; e < 4; ++e) S[j][e] *= L.gam[16 * rt + 4 * lq + e];
#pragma unroll
      for (int kk = 0; kk < PC / 32; ++kk)
        S[j] = mfma32(ld8(&L.kbt[16 * rt + l16][32 * kk + 8 * lq]),
                      ld8(&L.u3.w16t[16 * ct + l16][32 * kk + 8 * lq]), S[j]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- checkpoint export inside the pass -------------------------------------------------
    const int done = c0 + n;
    if (A.ckpt_interval > 0 && done % A.ckpt_interval == 0) {
      const int dst = A.ckpt_slot[ck++];
      if (dst >= 0 && dst < P.num_slots) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int it = w + PNW * j, rt = it & 7, ct = it >> 3;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = 16 * rt + 4 * lq + e;
            P.state[dst * per + hoff + (size_t)row * PD + col0 + 16 * ct + l16] = S[j][e];
          }
        }
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
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int it = w + PNW * j, rt = it & 7, ct = it >> 3;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + 4 * lq + e;
        P.state[out * per + hoff + (size_t)row * PD + col0 + 16 * ct + l16] = S[j][e];
      }
    }
    if (t == 0 && h == 0 && vs == 0) {
      kda_slot_meta mm{pos0 + len, 0, 0, 0, 0};
      P.meta[out] = mm;
    }
  }
}

int device_cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
    else
      cus = 256;
  }
  return cus;
}

template <int VS>
hipError_t launch_vs(const PoolView& p, const PrefillLaunch& a, int n_hg, hipStream_t s) {
  const int blocks = ((n_hg + 7) / 8) * 8 * (PD / VS);
  hipLaunchKernelGGL(prefill_chunk_kernel<VS>, dim3(blocks), dim3(PNT), 0, s, p, a, n_hg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PoolView& p, const PrefillLaunch& a, hipStream_t s) {
  if (p.dk != PD || a.chunk != PC) return launch_prefill_recurrent(p, a, s);
  // One work-group per CU (LDS-bound). The per-chunk latency of a chain depends little on
  // the slice width (the S-independent part dominates), so split value columns as long as
  // the grid stays within two rounds of CUs; work-groups start longest sequence first.
  const int n_hg = a.n_seq * p.H, cus = device_cu_count();
  if (n_hg * 8 <= 2 * cus) return launch_vs<16>(p, a, n_hg, s);
  if (n_hg * 4 <= 2 * cus) return launch_vs<32>(p, a, n_hg, s);
  if (n_hg * 2 <= 2 * cus) return launch_vs<64>(p, a, n_hg, s);
  return launch_vs<128>(p, a, n_hg, s);
}

}  // namespace kda
