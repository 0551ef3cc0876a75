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
// across waves through LDS in wave order. Decode, verify and commit use the same layout and
// the same step function, so a commit that replays n positions yields the state bit-for-bit
// equal to n decode calls.
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

// grid: B * H * (D / VS); block (bi, h, vs) with vs fastest.
template <int D>
__global__ __launch_bounds__(StepCfg<D>::NT) void decode_kernel(PoolView P, StepTensors T,
                                                                const int32_t* __restrict__ slots) {
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
  const int t = threadIdx.x, R = P.R, total = n_pos * CPP;
  for (int x = t; x < total; x += blockDim.x) {
    const int j = x / CPP, u = x % CPP;
    const size_t src = ((size_t)bi * n_pos + j) * P.H + h, dst = ((size_t)slot * R + ring_at(head, j, R)) * P.H + h;
    if (u < D / 8)
      reinterpret_cast<u4*>(P.ring_k + dst * D)[u] = reinterpret_cast<const u4*>(T.k + src * D)[u];
    else if (u < D / 4)
      reinterpret_cast<u4*>(P.ring_v + dst * D)[u - D / 8] = reinterpret_cast<const u4*>(T.v + src * D)[u - D / 8];
    else
      reinterpret_cast<u4*>(P.ring_a + dst * D)[u - D / 4] = reinterpret_cast<const u4*>(T.a + src * D)[u - D / 4];
  }
  for (int j = t; j < n_pos; j += blockDim.x)
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

// ReplaySSM commit: replay 1 + n_accepted ring entries into the slot, store once.
template <int D>
__global__ __launch_bounds__(StepCfg<D>::NT) void commit_kernel(PoolView P, const int32_t* __restrict__ slots,
                                                                const int32_t* __restrict__ n_acc) {
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

hipError_t launch_decode(const PoolView& p, const StepTensors& t, int32_t B, const int32_t* d_slots,
                         hipStream_t s) {
  if (p.dk == 128)
    hipLaunchKernelGGL(decode_kernel<128>, dim3(step_blocks<128>(p, B)), dim3(StepCfg<128>::NT), 0, s, p, t, d_slots);
  else
    hipLaunchKernelGGL(decode_kernel<16>, dim3(step_blocks<16>(p, B)), dim3(StepCfg<16>::NT), 0, s, p, t, d_slots);
  return hipGetLastError();
}

hipError_t launch_verify(const PoolView& p, const StepTensors& t, int32_t B, int32_t n_pos,
                         const int32_t* d_slots, hipStream_t s) {
  if (p.dk == 128)
    hipLaunchKernelGGL(verify_kernel<128>, dim3(step_blocks<128>(p, B) + B * p.H), dim3(StepCfg<128>::NT), 0, s, p,
                       t, n_pos, d_slots);
  else
    hipLaunchKernelGGL(verify_kernel<16>, dim3(step_blocks<16>(p, B) + B * p.H), dim3(StepCfg<16>::NT), 0, s, p, t,
                       n_pos, d_slots);
  return hipGetLastError();
}

hipError_t launch_commit(const PoolView& p, int32_t B, const int32_t* d_slots, const int32_t* d_n_acc,
                         hipStream_t s) {
  if (p.dk == 128)
    hipLaunchKernelGGL(commit_kernel<128>, dim3(step_blocks<128>(p, B)), dim3(StepCfg<128>::NT), 0, s, p, d_slots, d_n_acc);
  else
    hipLaunchKernelGGL(commit_kernel<16>, dim3(step_blocks<16>(p, B)), dim3(StepCfg<16>::NT), 0, s, p, d_slots, d_n_acc);
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
