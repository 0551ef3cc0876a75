// KDA single-token kernels on gfx950: decode, speculative verify, ReplaySSM commit and
// rollback, plus the slot reset / checkpoint copies.
//
// The token update is the gated delta rule with per-key-channel decay (the pages name the
// KDA state -- "vLLM lifts Kimi K3 throughput by up to 2.8x", section "Kimi K3 stresses the
// whole stack" -- but print no formula):
//     S' = Diag(a) S;  u = S'^T k;  p = S'^T q;  delta = b (v - u)
//     S  = S' + k delta^T;  o = S^T q = p + (k . q) delta
// Each (sequence, head, value-column slice) work-group streams its fp32 state tile in once with
// 16-byte loads, keeps it in VGPRs for every position it processes, and writes it back at most
// once: decode is HBM-bound (about 0.9 flop per byte); verify and commit of a few sequences are
// bound by the chain of positions instead (one wave per SIMD stepping one position after
// another).
//
// Thread layout (StepCfg): a work-group owns VS value columns of one head. Thread t holds
// RPT consecutive key rows x 4 consecutive columns (one float4 per row). The reductions over
// key rows (u, p and k.q) go first through the thread's own rows, then a butterfly across
// the lanes of a wave that hold the same columns (DPP and lane-swap instructions), then
// across waves through LDS in wave order. Decode and commit (and verify of more than 16
// positions, and the direct per-draft scheme) use the same layout and the same step function,
// so a commit that replays n positions yields the state bit-for-bit equal to n decode calls.
// Verify of up to 16 positions at d = 128 writes no state and solves its positions together in
// WY form instead (verify_wy_kernel).
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <int D>
struct StepCfg;

template <>
struct StepCfg<128> {
  static constexpr int D = 128, VS = 32, RPT = 8;
  static constexpr int TPR = VS / 4, NRG = D / RPT, NT = NRG * TPR, NW = NT / 64;
};

template <>
struct StepCfg<16> {
  static constexpr int D = 16, VS = 16, RPT = 1;
  static constexpr int TPR = VS / 4, NRG = D / RPT, NT = NRG * TPR, NW = NT / 64;
};

template <class C>
struct StepIn {
  uint32_t kw[(C::RPT + 1) / 2];   // raw bf16 of k rows
  uint32_t vw[2];                  // raw bf16 of the thread's 4 value columns
  float k[C::RPT], q[C::RPT], a[C::RPT], v[4];
  float b;
};

// Cross-wave reduction scratch: two buffers so one barrier per step suffices.
template <class C>
struct StepLds {
  float red[2][C::NW][2 * C::VS + 4];
};

// x + the value of lane l ^ 8 (DPP row_ror:8 inside each 16-lane row: a VALU operand
// modifier, no LDS round trip).
__device__ __forceinline__ float add_xor8(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}

// x + the value of lane l ^ 16 / l ^ 32. With both operands equal, v_permlane16_swap returns
// (row 2r, row 2r) and (row 2r + 1, row 2r + 1) of x for each pair of 16-lane rows, and
// v_permlane32_swap the lower and the upper half-wave: the sum of the pair is the same in both
// lanes of a pair.
__device__ __forceinline__ float add_xor16(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Sum over the lanes of a wave that hold the same value columns (lanes l ^ TPR, l ^ 2 TPR, ..).
// Each level adds a lane and its partner, so both lanes of a pair get the same bits.
template <class C>
__device__ __forceinline__ float rows_sum(float x) {
  if constexpr (C::TPR == 8) {
    return add_xor32(add_xor16(add_xor8(x)));
  } else {
#pragma unroll
    for (int m = C::TPR; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
  }
}

// One position of the rule on the thread's RPT x 4 tile. WITH_O also produces o for the
// thread's 4 columns (valid in every thread).
template <class C, bool WITH_O>
__device__ __forceinline__ void step(float (&S)[C::RPT][4], const StepIn<C>& in,
                                     StepLds<C>& lds, int buf, float (&o)[4]) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, cg = t % C::TPR;
#pragma unroll
  for (int r = 0; r < C::RPT; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) S[r][c] = S[r][c] * in.a[r];
  float u[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
  for (int r = 0; r < C::RPT; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u[c] = __builtin_fmaf(S[r][c], in.k[r], u[c]);
      if constexpr (WITH_O) p[c] = __builtin_fmaf(S[r][c], in.q[r], p[c]);
    }
  if constexpr (WITH_O) {
#pragma unroll
    for (int r = 0; r < C::RPT; ++r) kq = __builtin_fmaf(in.k[r], in.q[r], kq);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u[c] = rows_sum<C>(u[c]);
    if constexpr (WITH_O) p[c] = rows_sum<C>(p[c]);
  }
  if constexpr (WITH_O) kq = rows_sum<C>(kq);
  if constexpr (C::NW > 1) {
    float* red = lds.red[buf][w];
    if (lane < C::TPR) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        red[cg * 4 + c] = u[c];
        if constexpr (WITH_O) red[C::VS + cg * 4 + c] = p[c];
      }
      if (WITH_O && lane == 0) red[2 * C::VS] = kq;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u[c] = lds.red[buf][0][cg * 4 + c];
      if constexpr (WITH_O) p[c] = lds.red[buf][0][C::VS + cg * 4 + c];
    }
    if constexpr (WITH_O) kq = lds.red[buf][0][2 * C::VS];
#pragma unroll
    for (int ww = 1; ww < C::NW; ++ww) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u[c] = u[c] + lds.red[buf][ww][cg * 4 + c];
        if constexpr (WITH_O) p[c] = p[c] + lds.red[buf][ww][C::VS + cg * 4 + c];
      }
      if constexpr (WITH_O) kq = kq + lds.red[buf][ww][2 * C::VS];
    }
  }
  float dl[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) dl[c] = in.b * (in.v[c] - u[c]);
#pragma unroll
  for (int r = 0; r < C::RPT; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) S[r][c] = __builtin_fmaf(in.k[r], dl[c], S[r][c]);
  if constexpr (WITH_O) {
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = __builtin_fmaf(kq, dl[c], p[c]);
  }
}

// Raw inputs of one position as loaded: k, a (and q) rows r0..r0+RPT-1 and v columns
// c0..c0+3. Loops over positions fetch position j + 1 while position j is stepped, so only
// the first position's load latency is exposed.
template <class C>
struct StepRaw {
  uint32_t kw[(C::RPT + 1) / 2], qw[(C::RPT + 1) / 2], vw[2];
  float a[C::RPT];
  float b;
};

template <class C, bool WITH_Q>
__device__ __forceinline__ void fetch_in(StepRaw<C>& r, const uint16_t* q, const uint16_t* k,
                                         const uint16_t* v, const float* a, const float* b,
                                         int r0, int c0) {
  load_bf16_raw<C::RPT>(k + r0, r.kw);
  if constexpr (WITH_Q) load_bf16_raw<C::RPT>(q + r0, r.qw);
  load_f32<C::RPT>(a + r0, r.a);
  load_bf16_raw<4>(v + c0, r.vw);
  r.b = *b;
}

template <class C, bool WITH_Q>
__device__ __forceinline__ void unpack_in(StepIn<C>& in, const StepRaw<C>& r) {
#pragma unroll
  for (int i = 0; i < (C::RPT + 1) / 2; ++i) in.kw[i] = r.kw[i];
  unpack_bf16<C::RPT>(r.kw, in.k);
  if constexpr (WITH_Q) unpack_bf16<C::RPT>(r.qw, in.q);
#pragma unroll
  for (int i = 0; i < C::RPT; ++i) in.a[i] = r.a[i];
  in.vw[0] = r.vw[0];
  in.vw[1] = r.vw[1];
  unpack_bf16<4>(r.vw, in.v);
  in.b = r.b;
}

template <class C, bool WITH_Q>
__device__ __forceinline__ void load_in(StepIn<C>& in, const uint16_t* q, const uint16_t* k,
                                        const uint16_t* v, const float* a, const float* b,
                                        int r0, int c0) {
  StepRaw<C> r;
  fetch_in<C, WITH_Q>(r, q, k, v, a, b, r0, c0);
  unpack_in<C, WITH_Q>(in, r);
}

template <class C>
__device__ __forceinline__ void load_state(float (&S)[C::RPT][4], const float* Sp, int r0, int c0) {
#pragma unroll
  for (int r = 0; r < C::RPT; ++r) {
    float4 x = *reinterpret_cast<const float4*>(Sp + (size_t)(r0 + r) * C::D + c0);
    S[r][0] = x.x; S[r][1] = x.y; S[r][2] = x.z; S[r][3] = x.w;
  }
}

template <class C>
__device__ __forceinline__ void store_state(const float (&S)[C::RPT][4], float* Sp, int r0, int c0) {
#pragma unroll
  for (int r = 0; r < C::RPT; ++r)
    *reinterpret_cast<float4*>(Sp + (size_t)(r0 + r) * C::D + c0) =
        make_float4(S[r][0], S[r][1], S[r][2], S[r][3]);
}

__device__ __forceinline__ int wrap(int x, int R) { return ((x % R) + R) % R; }

// Ring entry j after entry `base` (0 <= base < R, 0 <= j <= R): one compare, no division.
__device__ __forceinline__ int ring_at(int base, int j, int R) {
  const int e = base + j;
  return e >= R ? e - R : e;
}

typedef uint32_t u2v __attribute__((ext_vector_type(2)));

// 8-byte stores through a buffer resource over [base, base + bytes) whose lanes opt out with
// an offset past the range (the hardware drops them): every wave issues the same store
// instructions whatever its lanes' roles, so a loop that prefetches its next position's inputs
// before these stores waits only for those loads (a fixed count of later operations), not for
// the stores to retire.
struct MaskedStore {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t oob;
  __device__ __forceinline__ MaskedStore(const void* base, uint32_t bytes)
      : rs(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000)),
        oob(bytes) {}
  __device__ __forceinline__ void b64(bool on, uint32_t byte_off, const uint32_t (&w)[2]) const {
    __builtin_amdgcn_raw_buffer_store_b64(u2v{w[0], w[1]}, rs, on ? byte_off : oob, 0, 0);
  }
};

// An empty use of every state register: the compiler places the wait for the state loads here,
// before a loop over positions, instead of at their first use inside the loop, where it would
// also wait for the next position's prefetched inputs on every iteration.
template <class C>
__device__ __forceinline__ void state_ready(const float (&S)[C::RPT][4]) {
#pragma unroll
  for (int r = 0; r < C::RPT; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" ::"v"(S[r][c]));
}

// Steps positions 0..n-1 (n >= 1) with the next position's inputs in flight. The inputs
// alternate between two register buffers and the loop covers two positions per trip, so no
// buffer is ever copied: one buffer carried around the loop would be moved into place on every
// trip, and those moves wait for the loads in flight. Both positions of a trip issue the same
// memory operations whatever n is -- a fetch past the end re-reads position n - 1, and for an
// odd n the trip's second position is a padding position j = n, where `body` must neither step
// nor store anything visible -- so the compiler can count the operations issued after each
// buffer's loads and waits for those loads only. The state and the first position's inputs are
// waited for at once: nothing is in flight when the loop is entered, so the waits inside it
// follow the loop's own pattern.
template <class C, bool WITH_Q, class Fetch, class Body>
__device__ __forceinline__ void stepped_positions(int n, float (&S)[C::RPT][4], const float* Sp, int r0,
                                                  int c0, Fetch&& fetch, Body&& body) {
  StepRaw<C> b0, b1;
  fetch(b0, 0);
  load_state<C>(S, Sp, r0, c0);
  __builtin_amdgcn_s_waitcnt(0);   // position 0 needs both
  state_ready<C>(S);
  auto one = [&](int j, const StepRaw<C>& cur, StepRaw<C>& nxt) {
    StepIn<C> in;
    unpack_in<C, WITH_Q>(in, cur);
    fetch(nxt, j + 1 < n ? j + 1 : n - 1);
    body(j, in);
  };
  for (int j = 0; j < n; j += 2) {
    one(j, b0, b1);
    one(j + 1, b1, b0);
  }
}

// Slot indices of a decode or commit batch of at most SLOT_ARG_MAX sequences, by value among the
// kernel arguments (decode_kernel<D, true>, commit_kernel<D, true>; larger batches read the
// device array). The kernel's arguments are loaded before anything else, so the state tile's
// address then waits for no load of its own (decode of 16 sequences, cold, by events: 21.8 ->
// 21.2 us).
struct SlotArg {
  int32_t id[SLOT_ARG_MAX];
};

// grid: (H * (D / VS), B); block (vs, h) with vs fastest in x, the sequence bi in y (no kernel
// argument is needed to find bi, so its slot index loads with the arguments).
template <int D, bool BY_VALUE>
__global__ __launch_bounds__(StepCfg<D>::NT) void decode_kernel(PoolView P, StepTensors T, SlotArg sa,
                                                                const int32_t* __restrict__ slots) {
  using C = StepCfg<D>;
  __shared__ StepLds<C> lds;
  constexpr int NVS = D / C::VS;
  const int vs = blockIdx.x % NVS, h = blockIdx.x / NVS, bi = blockIdx.y;
  const int slot = BY_VALUE ? sa.id[bi] : slots[bi];
  if (slot < 0 || slot >= P.num_slots) {
    if (threadIdx.x == 0 && h == 0 && vs == 0) atomicOr(P.err, DEVERR_SLOT_RANGE);
    return;
  }
  const int t = threadIdx.x, cg = t % C::TPR, rg = t / C::TPR;
  const int r0 = rg * C::RPT, c0 = vs * C::VS + cg * 4;
  float* Sp = P.state + ((size_t)slot * P.H + h) * D * D;
  float S[C::RPT][4];
  load_state<C>(S, Sp, r0, c0);
  const size_t row = (size_t)bi * P.H + h;
  StepIn<C> in;
  load_in<C, true>(in, T.q + row * D, T.k + row * D, T.v + row * D, T.a + row * D, T.b + row, r0, c0);
  float o[4];
  step<C, true>(S, in, lds, 0, o);
  store_state<C>(S, Sp, r0, c0);
  if (rg == 0) {
    uint32_t ow[2] = {pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3])};
    store_bf16_raw<4>(T.o + row * D + c0, ow);
  }
  if (t == 0 && h == 0 && vs == 0) P.meta[slot].pos += 1;
}

// The ring append of a verify: the entries are the verify's own inputs (k, v, a, b of each
// position), so extra work-groups of the same launch, one per (sequence, head), copy them while
// the stepping work-groups run; the loop over positions then stores only its outputs (the five
// masked ring stores per position cost ~1.7 us of that loop at 4 sequences). Entry j of the head
// goes to ring entry ring_at(head, j, R), as the replay at commit reads it.
template <int D>
__device__ __forceinline__ void ring_append(const PoolView& P, const StepTensors& T, int n_pos, int bi, int h,
                                            int slot, int head) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  constexpr int CPP = D / 2;                       // 16-byte pieces per position: k D/8, v D/8, a D/4
  constexpr int NB = 4;                            // pieces per thread in flight together
  const int t = threadIdx.x, R = P.R, total = n_pos * CPP, nt = blockDim.x;
  auto src_of = [&](int x) -> const u4* {
    const int j = x / CPP, u = x % CPP;
    const size_t src = ((size_t)bi * n_pos + j) * P.H + h;
    if (u < D / 8) return reinterpret_cast<const u4*>(T.k + src * D) + u;
    if (u < D / 4) return reinterpret_cast<const u4*>(T.v + src * D) + (u - D / 8);
    return reinterpret_cast<const u4*>(T.a + src * D) + (u - D / 4);
  };
  auto dst_of = [&](int x) -> u4* {
    const int j = x / CPP, u = x % CPP;
    const size_t dst = ((size_t)slot * R + ring_at(head, j, R)) * P.H + h;
    if (u < D / 8) return reinterpret_cast<u4*>(P.ring_k + dst * D) + u;
    if (u < D / 4) return reinterpret_cast<u4*>(P.ring_v + dst * D) + (u - D / 8);
    return reinterpret_cast<u4*>(P.ring_a + dst * D) + (u - D / 4);
  };
  // NB loads issued before their stores: the inputs and the ring never overlap, and the stores
  // would otherwise hold each next load back (one memory round trip per piece)
  for (int x0 = t; x0 < total; x0 += NB * nt) {
    u4 buf[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int x = x0 + i * nt;
      buf[i] = *src_of(x < total ? x : x0);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int x = x0 + i * nt;
      if (x < total) *dst_of(x) = buf[i];
    }
  }
  for (int j = t; j < n_pos; j += nt)
    P.ring_b[((size_t)slot * R + ring_at(head, j, R)) * P.H + h] = T.b[((size_t)bi * n_pos + j) * P.H + h];
}

// Speculative verify: n_pos positions on a register copy; outputs + ring appends only. Grid:
// B * H * (D / VS) stepping work-groups, then B * H ring-append work-groups.
template <int D>
__global__ __launch_bounds__(StepCfg<D>::NT) void verify_kernel(PoolView P, StepTensors T, int n_pos,
                                                                const int32_t* __restrict__ slots) {
  using C = StepCfg<D>;
  __shared__ StepLds<C> lds;
  constexpr int NVS = D / C::VS;
  const int n_step = gridDim.x / (NVS + 1) * NVS;   // stepping work-groups; the rest append
  if ((int)blockIdx.x >= n_step) {
    const int hb = blockIdx.x - n_step, h = hb % P.H, bi = hb / P.H;
    const int slot = slots[bi];
    if (slot < 0 || slot >= P.num_slots) return;     // flagged by the stepping work-groups
    ring_append<D>(P, T, n_pos, bi, h, slot, wrap(P.meta[slot].ring_head, P.R));
    return;
  }
  const int vs = blockIdx.x % NVS, h = (blockIdx.x / NVS) % P.H, bi = blockIdx.x / (NVS * P.H);
  const int slot = slots[bi];
  if (slot < 0 || slot >= P.num_slots) {
    if (threadIdx.x == 0 && h == 0 && vs == 0) atomicOr(P.err, DEVERR_SLOT_RANGE);
    return;
  }
  const int t = threadIdx.x, rg = t / C::TPR;
  const int r0 = rg * C::RPT, c0 = vs * C::VS + (t % C::TPR) * 4;
  const int R = P.R;
  const int head = wrap(P.meta[slot].ring_head, R);
  const float* Sp = P.state + ((size_t)slot * P.H + h) * D * D;
  float S[C::RPT][4];
  auto fetch = [&](StepRaw<C>& r, int j) {
    const size_t row = ((size_t)bi * n_pos + j) * P.H + h;
    fetch_in<C, true>(r, T.q + row * D, T.k + row * D, T.v + row * D, T.a + row * D, T.b + row, r0, c0);
  };
  // outputs of this sequence and head (rows j of n_pos): a byte range small enough for 32-bit
  // buffer offsets
  const size_t HD = (size_t)P.H * D;
  const MaskedStore so(T.o + ((size_t)bi * n_pos * P.H + h) * D, (uint32_t)(n_pos * HD * 2));
  const bool out_lane = rg == 0;
  stepped_positions<C, true>(n_pos, S, Sp, r0, c0, fetch, [&](int j, const StepIn<C>& in) {
    const bool live = j < n_pos;   // false only at the padding position
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    if (live) step<C, true>(S, in, lds, j & 1, o);
    const uint32_t ow[2] = {pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3])};
    so.b64(live && out_lane, (uint32_t)((size_t)j * HD + c0) * 2, ow);
  });
  if (t == 0 && h == 0 && vs == 0) {
    P.meta[slot].v_base = head;
    P.meta[slot].v_npos = n_pos;
    P.meta[slot].pending = n_pos;
  }
}

// ---- verify of up to 16 positions in WY form (d = 128) -------------------------------------
// Unrolling the step over the verify's positions j = 0 .. P-1 from the committed state S (G_j =
// a_0 ... a_j per key channel, delta_j the step's b_j (v_j - u_j)):
//   S_j = Diag(G_j) S + sum_{m<=j} Diag(G_j / G_m) k_m delta_m^T, so
//   delta_j = b_j (v_j - S^T (G_j k_j) - sum_{m<j} A[j][m] delta_m),  A[j][m]  = sum_i k_j k_m G_j / G_m
//   o_j     = S^T (G_j q_j) + sum_{m<=j} Aq[j][m] delta_m,              Aq[j][m] = sum_i q_j k_m G_j / G_m
// (G_j / G_m = a_{m+1} ... a_j): Delta = T (V - (G K) S) with T = (I + Diag(b) A)^-1 Diag(b) and
// O = (G Q) S + Aq Delta. No position waits for the one before it: the products run on fp32
// matrix cores (v_mfma_f32_16x16x4_f32), and only the 16 x 16 inverse is sequential. A key
// channel whose decay over the P positions is below 2^-60 (k_m / G_m could leave the fp32 range)
// takes no part in the factored A products; its terms are added exactly from the raw inputs.
// Work-group: (sequence, head, 64 value columns), four waves of one 16-column tile each; waves
// 0-1 also compute the key channels' decays and the two key-channel halves of A, waves 2-3 stage
// V and compute the halves of Aq, and wave 0 the inverse (while the others compute their tiles'
// P and R). As in verify_kernel the launch ends with B * H ring-append work-groups, and no state
// is written.
typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int VCP = 16;                 // positions of the WY verify (at most)
constexpr int VC_COLS = 64;             // value columns per work-group
constexpr int VC_NCS = 128 / VC_COLS;   // work-groups per (sequence, head)
constexpr int VC_NT = 256;
constexpr float VC_DECAY_MIN = 0x1p-60f;
static_assert(VCP * 128 / 2 <= 4 * VC_NT, "one ring-append batch per thread");

struct VerifyLds {
  float gk[VCP][132];          // G_j k_j  (rows j >= P zero)
  float gq[VCP][132];          // G_j q_j
  float ki[VCP][132];          // k_m / G_m, zero on fast channels
  float at[2][VCP][VCP];       // A halves (waves 0, 1), row-major
  float aq[2][VCP][VCP + 1];   // Aq halves (waves 2, 3)
  float tm[VCP][VCP + 1];      // T
  float v[VCP][VC_COLS];       // V of the work-group's columns
  float b[VCP];
  uint64_t fast[2];            // key channels decaying below VC_DECAY_MIN
};

// the value of lane `src` of each group of four lanes, to all four (DPP quad_perm)
__device__ __forceinline__ float quad_bcast(float x, int src) {
  const int v = __float_as_int(x);
  switch (src) {
    case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, false));
  }
}

__device__ __forceinline__ f4v mfma4(float a, float b, f4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Ring append of the WY verify (n_pos <= 16): every input piece is loaded before the slot and
// its ring head are awaited, then stored (one memory round trip for the copy).
__device__ __forceinline__ void ring_append_wy(const PoolView& P, const StepTensors& T, int np, int bi, int h,
                                               const int32_t* __restrict__ slots) {
  constexpr int D = 128, CPP = D / 2;   // 16-byte pieces per position: k D/8, v D/8, a D/4
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const int t = threadIdx.x, total = np * CPP;
  auto piece = [&](int x, int& u) -> size_t {   // row of piece x, u its index in the row
    u = x % CPP;
    return (size_t)(x / CPP);
  };
  u4 buf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int u;
    const size_t j = piece(min(t + VC_NT * i, total - 1), u);
    const size_t src = ((size_t)bi * np + j) * P.H + h;
    buf[i] = u < D / 8   ? reinterpret_cast<const u4*>(T.k + src * D)[u]
             : u < D / 4 ? reinterpret_cast<const u4*>(T.v + src * D)[u - D / 8]
                         : reinterpret_cast<const u4*>(T.a + src * D)[u - D / 4];
  }
  const float bb = T.b[((size_t)bi * np + min(t, np - 1)) * P.H + h];
  const int slot = slots[bi];
  if (slot < 0 || slot >= P.num_slots) return;   // flagged by the WY work-groups
  const int R = P.R, head = wrap(P.meta[slot].ring_head, R);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = t + VC_NT * i;
    if (x < total) {
      int u;
      const size_t j = piece(x, u);
      const size_t dst = ((size_t)slot * R + ring_at(head, (int)j, R)) * P.H + h;
      if (u < D / 8)
        reinterpret_cast<u4*>(P.ring_k + dst * D)[u] = buf[i];
      else if (u < D / 4)
        reinterpret_cast<u4*>(P.ring_v + dst * D)[u - D / 8] = buf[i];
      else
        reinterpret_cast<u4*>(P.ring_a + dst * D)[u - D / 4] = buf[i];
    }
  }
  if (t < np) P.ring_b[((size_t)slot * R + ring_at(head, t, R)) * P.H + h] = bb;
}

__global__ __launch_bounds__(VC_NT) void verify_wy_kernel(PoolView P, StepTensors T, int n_pos,
                                                          const int32_t* __restrict__ slots) {
  constexpr int D = 128;
  __shared__ VerifyLds L;
  // the wave index is uniform: the role branches below are scalar
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, i16 = l & 15, g = l >> 4;
  const int np = n_pos;
  const size_t HD = (size_t)P.H * D;
  const int n_wy = gridDim.x / (VC_NCS + 1) * VC_NCS;   // WY work-groups; the rest append
  if ((int)blockIdx.x >= n_wy) {
    const int hb = blockIdx.x - n_wy;
    ring_append_wy(P, T, np, hb / P.H, hb % P.H, slots);
    return;
  }
  const int cs = blockIdx.x % VC_NCS, h = (blockIdx.x / VC_NCS) % P.H, bi = blockIdx.x / (VC_NCS * P.H);
  const int ct = 16 * w, c0 = cs * VC_COLS + ct;   // the wave's tile (in the slice, in the head)
  // Every input load is issued before any is used, and before the slot index (which the state
  // tile's address needs) is awaited: waves 0-1 the positions' k, q and a of key channel i = t
  // (rows past P re-read row P - 1 and are masked), waves 2-3 the V columns and b. The bf16
  // words are converted only once all loads are issued, so no load waits on an earlier one.
  constexpr int NV = VCP * VC_COLS / 128;   // V values per thread of waves 2-3
  uint32_t kw[VCP], qw[VCP], vw[NV];
  float ar[VCP], bv = 0.f;
  if (w < 2) {
#pragma unroll
    for (int j = 0; j < VCP; ++j) {
      const size_t row = ((size_t)bi * np + min(j, np - 1)) * HD + (size_t)h * D + t;
      kw[j] = T.k[row];
      qw[j] = T.q[row];
      ar[j] = T.a[row];
    }
  } else {
    const int u = t - D;
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int e = u + 128 * x, j = e / VC_COLS, c = e % VC_COLS;
      vw[x] = T.v[((size_t)bi * np + min(j, np - 1)) * HD + (size_t)h * D + cs * VC_COLS + c];
    }
    bv = T.b[((size_t)bi * np + min(u % VCP, np - 1)) * P.H + h];
  }
  const int slot = slots[bi];
  if (slot < 0 || slot >= P.num_slots) {
    if (t == 0 && h == 0 && cs == 0) atomicOr(P.err, DEVERR_SLOT_RANGE);
    return;
  }
  // the wave's state tile as the B operand of the K = 128 products (K index 32 g + s):
  // sv[s] = S[32 g + s][c0 + i16]
  float sv[32];
  {
    const float* Sp = P.state + ((size_t)slot * P.H + h) * D * D + c0 + i16;
#pragma unroll
    for (int s = 0; s < 32; ++s) sv[s] = Sp[(size_t)(32 * g + s) * D];
  }
  // keeps the compiler from merging the role branches (which would place the slot read and the
  // state loads after the first use of the inputs: two memory round trips instead of one)
  asm volatile("" ::: "memory");
  if (w < 2) {
    // key channel i = t: running decay over the positions, the decayed rows and k / G
    const int i = t;
    float G = 1.f, gmin = 1.f;
#pragma unroll
    for (int j = 0; j < VCP; ++j) {
      const bool live = j < np;
      const float kr = live ? bf2f(kw[j]) : 0.f, qr = live ? bf2f(qw[j]) : 0.f;
      G = live ? G * ar[j] : G;
      gmin = fminf(gmin, G);
      L.gk[j][i] = G * kr;
      L.gq[j][i] = G * qr;
      ar[j] = kr * __builtin_amdgcn_rcpf(G);   // k / G, stored below unless the channel is fast
    }
    const bool fast = !(gmin >= VC_DECAY_MIN);   // NaN decays take the exact path too
#pragma unroll
    for (int j = 0; j < VCP; ++j) L.ki[j][i] = fast ? 0.f : ar[j];
    const uint64_t m = __ballot(fast);
    if (l == 0) L.fast[w] = m;
  } else {
    const int u = t - D;
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int e = u + 128 * x, j = e / VC_COLS, c = e % VC_COLS;
      L.v[j][c] = j < np ? bf2f(vw[x]) : 0.f;
    }
    if (u < VCP) L.b[u] = u < np ? bv : 0.f;
  }
  __syncthreads();

  // products with K = 128 on the wave's tile, K index 32 g + s
  auto tile_product = [&](const float(*X)[132]) __attribute__((always_inline)) {
    f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 8; ++s4) {
      const f4v xa = *reinterpret_cast<const f4v*>(&X[i16][32 * g + 4 * s4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma4(xa[e], sv[4 * s4 + e], acc);
    }
    return acc;
  };
  {
    // A (waves 0-1) and Aq (waves 2-3) over key channels [64 (w & 1), 64 (w & 1) + 64): the
    // 16 x 16 results of [16 x 64] x [64 x 16], K index 64 (w & 1) + 16 g + s
    const float(*X)[132] = w < 2 ? L.gk : L.gq;
    const int kb = 64 * (w & 1) + 16 * g;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const f4v xa = *reinterpret_cast<const f4v*>(&X[i16][kb + 4 * s4]);
      const f4v ka = *reinterpret_cast<const f4v*>(&L.ki[i16][kb + 4 * s4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma4(xa[e], ka[e], acc);
    }
    if ((w & 1) == 0 && (L.fast[0] | L.fast[1])) {
      // exact terms of the fast channels: element (j, m) = (4 g + e, i16)
      for (int wd = 0; wd < 2; ++wd) {
        uint64_t fm = L.fast[wd];
        while (fm) {
          const int i = 64 * wd + __builtin_ctzll(fm);
          fm &= fm - 1;
          const int m = i16;
          const float km = m < np ? bf2f(T.k[((size_t)bi * np + m) * HD + (size_t)h * D + i]) : 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * g + e;
            if (j < np && m < np && (w == 0 ? j > m : j >= m)) {
              float prod = 1.f;
              for (int tt = m + 1; tt <= j; ++tt) prod *= T.a[((size_t)bi * np + tt) * HD + (size_t)h * D + i];
              const size_t rj = ((size_t)bi * np + j) * HD + (size_t)h * D + i;
              const float xj = w == 0 ? bf2f(T.k[rj]) : bf2f(T.q[rj]);
              acc[e] = __builtin_fmaf(xj * km, prod, acc[e]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (w < 2)
        L.at[w][4 * g + e][i16] = acc[e];
      else
        L.aq[w - 2][4 * g + e][i16] = acc[e];
    }
  }
  __syncthreads();
  if (w == 0) {
    // T = (I + Diag(b) A)^-1 Diag(b) by forward substitution, column m = l / 4 on the four lanes
    // of a quad: lane q keeps the running sums of rows j = 4 k + q. Step r: x_r = [r = m] -
    // acc_r on the lane that holds row r, broadcast to its quad (DPP), then every row j > r
    // takes b_j A[j][r] x_r. The coefficients (zero unless j > r; A is zero on rows and columns
    // past P) are read once, up front.
    const int m = l >> 2, q = l & 3;
    f4v lr[4][4];   // lr[k][c][e] = b_j A[j][4 c + e] for j = 4 k + q > 4 c + e, else 0
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = 4 * k + q;
      const float bj = L.b[j];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f4v a = *reinterpret_cast<const f4v*>(&L.at[0][j][4 * c]) + *reinterpret_cast<const f4v*>(&L.at[1][j][4 * c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) lr[k][c][e] = j > 4 * c + e ? bj * a[e] : 0.f;
      }
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f}, xv[VCP];
#pragma unroll
    for (int r = 0; r < VCP; ++r) {
      const float own = (r == m ? 1.f : 0.f) - acc[r >> 2];   // x_r on lane q = r % 4
      xv[r] = quad_bcast(own, r & 3);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = __builtin_fmaf(lr[k][r >> 2][r & 3], xv[r], acc[k]);
    }
    // lane q stores rows 4 k + q (no store inside the chain: it would wait on the reads above)
    const float bm = L.b[m];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x = q == 0 ? xv[4 * k] : q == 1 ? xv[4 * k + 1] : q == 2 ? xv[4 * k + 2] : xv[4 * k + 3];
      L.tm[4 * k + q][m] = x * bm;
    }
  }
  // P = (G K) S and R = (G Q) S on the wave's tile (wave 0 after the inverse, the others
  // meanwhile)
  const f4v pa = tile_product(L.gk), ra = tile_product(L.gq);
  __syncthreads();
  {
    // Delta = T (V - P), O = R + Aq Delta on the wave's tile: K = 16 with index 4 g + s, so the
    // accumulator tiles (rows 4 g + e) are the B operands as they stand
    f4v xv, dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) xv[e] = L.v[4 * g + e][ct + i16] - pa[e];
#pragma unroll
    for (int s = 0; s < 4; ++s) dv = mfma4(L.tm[i16][4 * g + s], xv[s], dv);
    f4v ov = ra;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int m = 4 * g + s;
      const float aq = i16 >= m ? L.aq[0][i16][m] + L.aq[1][i16][m] : 0.f;
      ov = mfma4(aq, dv[s], ov);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * g + e;
      if (j < np)
        T.o[((size_t)bi * np + j) * HD + (size_t)h * D + c0 + i16] = (uint16_t)(pack_bf2(ov[e], 0.f) & 0xffffu);
    }
  }
  if (t == 0 && h == 0 && cs == 0) {
    P.meta[slot].v_base = wrap(P.meta[slot].ring_head, P.R);
    P.meta[slot].v_npos = n_pos;
    P.meta[slot].pending = n_pos;
  }
}

// ReplaySSM commit: replay 1 + n_accepted ring entries into the slot, store once. Grid and slot
// ids as for decode_kernel (the sequence in y; ids by value for up to SLOT_ARG_MAX sequences).
template <int D, bool BY_VALUE>
__global__ __launch_bounds__(StepCfg<D>::NT) void commit_kernel(PoolView P, SlotArg sa,
                                                                const int32_t* __restrict__ slots,
                                                                const int32_t* __restrict__ n_acc) {
  using C = StepCfg<D>;
  __shared__ StepLds<C> lds;
  constexpr int NVS = D / C::VS;
  const int vs = blockIdx.x % NVS, h = blockIdx.x / NVS, bi = blockIdx.y;
  const int slot = BY_VALUE ? sa.id[bi] : slots[bi];
  if (slot < 0 || slot >= P.num_slots) {
    if (threadIdx.x == 0 && h == 0 && vs == 0) atomicOr(P.err, DEVERR_SLOT_RANGE);
    return;
  }
  const int t = threadIdx.x, cg = t % C::TPR, rg = t / C::TPR;
  const int r0 = rg * C::RPT, c0 = vs * C::VS + cg * 4;
  const int R = P.R;
  const int vb = wrap(P.meta[slot].v_base, R);
  int vn = P.meta[slot].v_npos;
  vn = vn < 1 ? 1 : (vn > R ? R : vn);
  int na = n_acc[bi];
  const bool bad = na < 0 || na > vn - 1;
  na = na < 0 ? 0 : (na > vn - 1 ? vn - 1 : na);
  const int n = 1 + na;
  float* Sp = P.state + ((size_t)slot * P.H + h) * D * D;
  float S[C::RPT][4];
  auto fetch = [&](StepRaw<C>& r, int j) {
    const size_t e = ((size_t)slot * R + (size_t)ring_at(vb, j, R)) * P.H + h;
    fetch_in<C, false>(r, nullptr, P.ring_k + e * D, P.ring_v + e * D, P.ring_a + e * D, P.ring_b + e,
                       r0, c0);
  };
  stepped_positions<C, false>(n, S, Sp, r0, c0, fetch, [&](int j, const StepIn<C>& in) {
    float o[4];
    if (j < n) step<C, false>(S, in, lds, j & 1, o);   // j == n: padding position
  });
  store_state<C>(S, Sp, r0, c0);
  if (t == 0 && h == 0 && vs == 0) {
    P.meta[slot].ring_head = ring_at(vb, n, R);
    P.meta[slot].pos += n;
    P.meta[slot].pending = 0;
    if (bad) atomicOr(P.err, (uint32_t)KDA_DEVERR_NACC_RANGE);
  }
}

// Direct per-draft state checkpointing, the scheme ReplaySSM is weighed against ("vLLM lifts
// Kimi K3 throughput by up to 2.8x", section "ReplaySSM shrinks rollback state"): verify
// writes the state after every position j to draft[bi][j] ([B][n_pos][H][D][D] fp32) instead
// of appending ring entries; the outputs are those of verify_kernel (same step code, same
// order). The ring is untouched.
template <int D>
__global__ __launch_bounds__(StepCfg<D>::NT) void verify_direct_kernel(PoolView P, StepTensors T, int n_pos,
                                                                       const int32_t* __restrict__ slots,
                                                                       float* __restrict__ draft) {
  using C = StepCfg<D>;
  __shared__ StepLds<C> lds;
  constexpr int NVS = D / C::VS;
  const int vs = blockIdx.x % NVS, h = (blockIdx.x / NVS) % P.H, bi = blockIdx.x / (NVS * P.H);
  const int slot = slots[bi];
  if (slot < 0 || slot >= P.num_slots) {
    if (threadIdx.x == 0 && h == 0 && vs == 0) atomicOr(P.err, DEVERR_SLOT_RANGE);
    return;
  }
  const int t = threadIdx.x, cg = t % C::TPR, rg = t / C::TPR;
  const int r0 = rg * C::RPT, c0 = vs * C::VS + cg * 4;
  const float* Sp = P.state + ((size_t)slot * P.H + h) * D * D;
  float S[C::RPT][4];
  load_state<C>(S, Sp, r0, c0);
  auto fetch = [&](StepRaw<C>& r, int j) {
    const size_t row = ((size_t)bi * n_pos + j) * P.H + h;
    fetch_in<C, true>(r, T.q + row * D, T.k + row * D, T.v + row * D, T.a + row * D, T.b + row, r0, c0);
  };
  StepRaw<C> nxt;
  fetch(nxt, 0);
  state_ready<C>(S);
  for (int j = 0; j < n_pos; ++j) {
    const size_t row = ((size_t)bi * n_pos + j) * P.H + h;
    StepIn<C> in;
    unpack_in<C, true>(in, nxt);
    if (j + 1 < n_pos) fetch(nxt, j + 1);
    float o[4];
    step<C, true>(S, in, lds, j & 1, o);
    if (rg == 0) {
      uint32_t ow[2] = {pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3])};
      store_bf16_raw<4>(T.o + row * D + c0, ow);
    }
    store_state<C>(S, draft + row * D * D, r0, c0);
  }
  if (t == 0 && h == 0 && vs == 0) {
    P.meta[slot].v_base = wrap(P.meta[slot].ring_head, P.R);
    P.meta[slot].v_npos = n_pos;
    P.meta[slot].pending = n_pos;
  }
}

// Direct commit: the slot's state becomes draft[bi][n_accepted] (the state after 1 +
// n_accepted positions); pos advances by 1 + n_accepted, the ring pointer stays. n_accepted
// outside [0, v_npos - 1] is clamped and flagged as in commit_kernel.
template <int D>
__global__ __launch_bounds__(StepCfg<D>::NT) void commit_direct_kernel(PoolView P, const int32_t* __restrict__ slots,
                                                                       const int32_t* __restrict__ n_acc,
                                                                       const float* __restrict__ draft, int n_pos) {
  using C = StepCfg<D>;
  constexpr int NVS = D / C::VS;
  const int vs = blockIdx.x % NVS, h = (blockIdx.x / NVS) % P.H, bi = blockIdx.x / (NVS * P.H);
  const int slot = slots[bi];
  if (slot < 0 || slot >= P.num_slots) {
    if (threadIdx.x == 0 && h == 0 && vs == 0) atomicOr(P.err, DEVERR_SLOT_RANGE);
    return;
  }
  const int t = threadIdx.x, cg = t % C::TPR, rg = t / C::TPR;
  const int r0 = rg * C::RPT, c0 = vs * C::VS + cg * 4;
  int vn = P.meta[slot].v_npos;
  vn = vn < 1 ? 1 : (vn > n_pos ? n_pos : vn);
  int na = n_acc[bi];
  const bool bad = na < 0 || na > vn - 1;
  na = na < 0 ? 0 : (na > vn - 1 ? vn - 1 : na);
  float S[C::RPT][4];
  load_state<C>(S, draft + (((size_t)bi * n_pos + na) * P.H + h) * D * D, r0, c0);
  store_state<C>(S, P.state + ((size_t)slot * P.H + h) * D * D, r0, c0);
  if (t == 0 && h == 0 && vs == 0) {
    P.meta[slot].pos += 1 + na;
    P.meta[slot].pending = 0;
    if (bad) atomicOr(P.err, (uint32_t)KDA_DEVERR_NACC_RANGE);
  }
}

__global__ void rollback_kernel(PoolView P, int B, const int32_t* __restrict__ slots) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B) return;
  const int slot = slots[i];
  if (slot < 0 || slot >= P.num_slots) {
    atomicOr(P.err, DEVERR_SLOT_RANGE);
    return;
  }
  P.meta[slot].pending = 0;
}

// Zero (src < 0) or copy one slot's state; block 0 thread 0 also writes dst's metadata.
__global__ void slot_fill_kernel(PoolView P, int src, int dst, size_t n4) {
  const size_t per = (size_t)P.H * P.dk * P.dv;
  float4* d = reinterpret_cast<float4*>(P.state + (size_t)dst * per);
  const float4* s = src >= 0 ? reinterpret_cast<const float4*>(P.state + (size_t)src * per) : nullptr;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    d[i] = s ? s[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    kda_slot_meta m;
    m.pos = src >= 0 ? P.meta[src].pos : 0;
    m.ring_head = 0; m.pending = 0; m.v_base = 0; m.v_npos = 0;
    P.meta[dst] = m;
  }
}

__global__ void clear_word_kernel(uint32_t* w) { *w = 0u; }

template <int D>
int step_blocks(const PoolView& p, int B) { return B * p.H * (D / StepCfg<D>::VS); }

}  // namespace

hipError_t launch_decode(const PoolView& p, const StepTensors& t, int32_t B, const int32_t* h_slots,
                         const int32_t* d_slots, hipStream_t s) {
  SlotArg sa{};
  const bool by_value = B <= SLOT_ARG_MAX;
  if (by_value)
    for (int32_t i = 0; i < B; ++i) sa.id[i] = h_slots[i];
  const dim3 g128(step_blocks<128>(p, 1), B), g16(step_blocks<16>(p, 1), B);
  if (p.dk == 128 && by_value)
    hipLaunchKernelGGL((decode_kernel<128, true>), g128, dim3(StepCfg<128>::NT), 0, s, p, t, sa, d_slots);
  else if (p.dk == 128)
    hipLaunchKernelGGL((decode_kernel<128, false>), g128, dim3(StepCfg<128>::NT), 0, s, p, t, sa, d_slots);
  else if (by_value)
    hipLaunchKernelGGL((decode_kernel<16, true>), g16, dim3(StepCfg<16>::NT), 0, s, p, t, sa, d_slots);
  else
    hipLaunchKernelGGL((decode_kernel<16, false>), g16, dim3(StepCfg<16>::NT), 0, s, p, t, sa, d_slots);
  return hipGetLastError();
}

hipError_t launch_verify(const PoolView& p, const StepTensors& t, int32_t B, int32_t n_pos,
                         const int32_t* d_slots, hipStream_t s) {
  if (p.dk == 128 && n_pos <= VCP)
    hipLaunchKernelGGL(verify_wy_kernel, dim3(B * p.H * (VC_NCS + 1)), dim3(VC_NT), 0, s, p, t, n_pos, d_slots);
  else if (p.dk == 128)
    hipLaunchKernelGGL(verify_kernel<128>, dim3(step_blocks<128>(p, B) + B * p.H), dim3(StepCfg<128>::NT), 0, s, p,
                       t, n_pos, d_slots);
  else
    hipLaunchKernelGGL(verify_kernel<16>, dim3(step_blocks<16>(p, B) + B * p.H), dim3(StepCfg<16>::NT), 0, s, p, t,
                       n_pos, d_slots);
  return hipGetLastError();
}

hipError_t launch_commit(const PoolView& p, int32_t B, const int32_t* h_slots, const int32_t* d_slots,
                         const int32_t* d_n_acc, hipStream_t s) {
  SlotArg sa{};
  const bool by_value = B <= SLOT_ARG_MAX;
  if (by_value)
    for (int32_t i = 0; i < B; ++i) sa.id[i] = h_slots[i];
  const dim3 g128(step_blocks<128>(p, 1), B), g16(step_blocks<16>(p, 1), B);
  if (p.dk == 128 && by_value)
    hipLaunchKernelGGL((commit_kernel<128, true>), g128, dim3(StepCfg<128>::NT), 0, s, p, sa, d_slots, d_n_acc);
  else if (p.dk == 128)
    hipLaunchKernelGGL((commit_kernel<128, false>), g128, dim3(StepCfg<128>::NT), 0, s, p, sa, d_slots, d_n_acc);
  else if (by_value)
    hipLaunchKernelGGL((commit_kernel<16, true>), g16, dim3(StepCfg<16>::NT), 0, s, p, sa, d_slots, d_n_acc);
  else
    hipLaunchKernelGGL((commit_kernel<16, false>), g16, dim3(StepCfg<16>::NT), 0, s, p, sa, d_slots, d_n_acc);
  return hipGetLastError();
}

hipError_t launch_verify_direct(const PoolView& p, const StepTensors& t, int32_t B, int32_t n_pos,
                                const int32_t* d_slots, float* draft, hipStream_t s) {
  if (p.dk == 128)
    hipLaunchKernelGGL(verify_direct_kernel<128>, dim3(step_blocks<128>(p, B)), dim3(StepCfg<128>::NT), 0, s, p, t,
                       n_pos, d_slots, draft);
  else
    hipLaunchKernelGGL(verify_direct_kernel<16>, dim3(step_blocks<16>(p, B)), dim3(StepCfg<16>::NT), 0, s, p, t,
                       n_pos, d_slots, draft);
  return hipGetLastError();
}

hipError_t launch_commit_direct(const PoolView& p, int32_t B, const int32_t* d_slots, const int32_t* d_n_acc,
                                const float* draft, int32_t n_pos, hipStream_t s) {
  if (p.dk == 128)
    hipLaunchKernelGGL(commit_direct_kernel<128>, dim3(step_blocks<128>(p, B)), dim3(StepCfg<128>::NT), 0, s, p,
                       d_slots, d_n_acc, draft, n_pos);
  else
    hipLaunchKernelGGL(commit_direct_kernel<16>, dim3(step_blocks<16>(p, B)), dim3(StepCfg<16>::NT), 0, s, p,
                       d_slots, d_n_acc, draft, n_pos);
  return hipGetLastError();
}

hipError_t launch_rollback(const PoolView& p, int32_t B, const int32_t* d_slots, hipStream_t s) {
  hipLaunchKernelGGL(rollback_kernel, dim3((B + 63) / 64), dim3(64), 0, s, p, B, d_slots);
  return hipGetLastError();
}

static hipError_t launch_fill(const PoolView& p, int src, int dst, hipStream_t s) {
  const size_t n4 = (size_t)p.H * p.dk * p.dv / 4;
  int blocks = (int)((n4 + 255) / 256);
  blocks = blocks > 1024 ? 1024 : blocks;
  hipLaunchKernelGGL(slot_fill_kernel, dim3(blocks), dim3(256), 0, s, p, src, dst, n4);
  return hipGetLastError();
}

hipError_t launch_slot_reset(const PoolView& p, int32_t slot, hipStream_t s) { return launch_fill(p, -1, slot, s); }

hipError_t launch_slot_copy(const PoolView& p, int32_t src, int32_t dst, hipStream_t s) {
  return launch_fill(p, src, dst, s);
}

hipError_t launch_clear_word(uint32_t* w, hipStream_t s) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, s, w);
  return hipGetLastError();
}

}  // namespace kda
