// Internal interface between the host-side pool logic (kda_pool.cpp) and the HIP kernels.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Device-side view of a pool: raw pointers and geometry, passed by value to launchers.
struct PoolView {
  float* state;             // [num_slots][H][dk][dv]
  uint16_t* ring_k;         // bf16 [num_slots][R][H][dk]
  uint16_t* ring_v;         // bf16 [num_slots][R][H][dv]
  float* ring_a;            // [num_slots][R][H][dk]
  float* ring_b;            // [num_slots][R][H]
  kda_slot_meta* meta;      // [num_slots]
  uint32_t* err;            // device error word
  int32_t num_slots, H, dk, dv, R;
};

struct StepTensors {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;   // bf16 bits
  const float* a; const float* b;
  uint16_t* o;
};

// Geometry of the chunked prefill at d = 128, shared by the kernels and the host plan: head
// dim, chunk, bytes of one (chunk, head) operand block in the workspace, and the largest batch
// whose plan the operand kernel computes itself.
constexpr int PREFILL_D = 128;
constexpr int PREFILL_CHUNK = 64;
constexpr int PREFILL_BLOCK_BYTES = 60 * 1024 + 4 * PREFILL_D;
constexpr int PREFILL_PLAN_INLINE_MAX = 64;

// Width plan of the prefill's sequential pass: the sequences ranked rank_end[g - 1] ..
// rank_end[g] - 1 by length (rank_end[-1] = 0) run in work-groups of vsw[g] value columns
// (16, 32, 64 or 128), work-groups wg_begin[g] .. wg_begin[g + 1] - 1 (each group a multiple of
// 8), groups in rank order so that the longest sequences' work-groups are dispatched first.
struct StatePlan {
  int32_t n_groups;
  int32_t rank_end[4], vsw[4], wg_begin[5];
};

struct PrefillLaunch {
  StepTensors t;
  int32_t n_seq, n_tok, chunk, ckpt_interval;
  const int32_t* cu_seqlens;   // device
  const int32_t* init_slot;    // device or nullptr
  const int32_t* out_slot;     // device
  const int32_t* ckpt_slot;    // device or nullptr
  int32_t max_len;             // longest sequence (host-known), sizes the grid
  int64_t n_chunks;            // sum over sequences of ceil(len / chunk) (host-known)
  void* workspace;             // device, at least prefill_workspace_bytes(...) bytes
  StatePlan plan;              // from plan_state_pass (host lengths)
};

// Decode and commit take the host copy of the slot indices too: a batch of at most SLOT_ARG_MAX
// sequences passes them by value among the kernel arguments.
constexpr int SLOT_ARG_MAX = 64;
hipError_t launch_decode(const PoolView& p, const StepTensors& t, int32_t B, const int32_t* h_slots,
                         const int32_t* d_slots, hipStream_t s);
hipError_t launch_verify(const PoolView& p, const StepTensors& t, int32_t B, int32_t n_pos,
                         const int32_t* d_slots, hipStream_t s);
hipError_t launch_commit(const PoolView& p, int32_t B, const int32_t* h_slots, const int32_t* d_slots,
                         const int32_t* d_n_accepted, hipStream_t s);
hipError_t launch_rollback(const PoolView& p, int32_t B, const int32_t* d_slots,
                           hipStream_t s);
// Direct per-draft checkpoints: verify writes every position's state to draft
// ([B][n_pos][H][dk][dv] fp32); commit copies draft[b][n_accepted[b]] into the slot.
hipError_t launch_verify_direct(const PoolView& p, const StepTensors& t, int32_t B, int32_t n_pos,
                                const int32_t* d_slots, float* draft, hipStream_t s);
hipError_t launch_commit_direct(const PoolView& p, int32_t B, const int32_t* d_slots,
                                const int32_t* d_n_acc, const float* draft, int32_t n_pos,
                                hipStream_t s);
hipError_t launch_slot_reset(const PoolView& p, int32_t slot, hipStream_t s);
hipError_t launch_slot_copy(const PoolView& p, int32_t src, int32_t dst, hipStream_t s);
hipError_t launch_clear_word(uint32_t* w, hipStream_t s);
hipError_t launch_prefill(const PoolView& p, const PrefillLaunch& a, hipStream_t s);
// Width plan for the sequential pass of a prefill with host lengths h_cu[0..n_seq]. Long
// chains take narrow slices (a chunk's latency falls with fewer compute waves sharing a CU's
// LDS), short ones wide slices (fewer work-groups, each CU-cheaper per column), chosen by a
// latency / CU-time model of the pass; beyond 64 sequences one width for all.
StatePlan plan_state_pass(const int32_t* h_cu, int n_seq, int H);
// Device workspace the prefill of n_seq sequences with n_chunks chunks in total needs (0 for
// d = 16, whose chunked form keeps every chunk on chip): the plan arrays, then the operand
// blocks.
size_t prefill_workspace_bytes(int dk, int chunk, int H, int n_seq, int64_t n_chunks);
size_t prefill_plan_bytes(int n_seq);
// Scratch of the allocation-free prefill: a file-scope device array of this many bytes in the
// prefill's code object; prefill_scratch returns its address on the current device (looked up
// once per device).
constexpr size_t PREFILL_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t prefill_scratch(void** out);

// Chunking of one sequence of len tokens with checkpoints every `interval` tokens (0: none).
// Every checkpoint position ends a chunk ("vLLM lifts Kimi K3 throughput by up to 2.8x",
// section "KDA checkpoints stay inside the prefill": the export happens inside the pass rather
// than by splitting the prefill), so an interval that is not a multiple of the chunk splits
// each interval into ceil(interval / chunk) chunks, the last one short; otherwise chunks are
// chunk tokens from the sequence start and only the last one may be short.
__host__ __device__ inline int seq_chunks(int len, int chunk, int interval) {
  if (interval <= 0 || interval % chunk == 0) return (len + chunk - 1) / chunk;
  const int per = (interval + chunk - 1) / chunk, full = len / interval, rem = len % interval;
  return full * per + (rem + chunk - 1) / chunk;
}
// First token (relative to the sequence start) and token count of chunk c.
__host__ __device__ inline void chunk_span(int c, int len, int chunk, int interval, int* t0, int* n) {
  if (interval <= 0 || interval % chunk == 0) {
    *t0 = chunk * c;
    *n = len - *t0 < chunk ? len - *t0 : chunk;
    return;
  }
  const int per = (interval + chunk - 1) / chunk, seg = c / per, j = c % per;
  const int seg_len = len - seg * interval < interval ? len - seg * interval : interval;
  *t0 = seg * interval + chunk * j;
  *n = seg_len - chunk * j < chunk ? seg_len - chunk * j : chunk;
}

// Shapes the kernels are instantiated for.
inline bool supported_dim(int d) { return d == 16 || d == 128; }
inline int prefill_chunk_for(int d) { return d == 16 ? 16 : 64; }

}  // namespace kda
