/*
 * kda.h -- C ABI of the MI355X (gfx950) engine for the Kimi Delta Attention (KDA)
 * fixed-size recurrent-state update.
 *
 * What is computed. The pages describe KDA as recurrent layers that keep a fixed-size state
 * per head instead of a token-growing KV cache ("vLLM brings day-0 support to Moonshot's
 * Kimi K3", section "Confirmed"; "vLLM lifts Kimi K3 throughput by up to 2.8x", section
 * "Kimi K3 stresses the whole stack"). They print no equation; this library computes the
 * gated delta rule with per-key-channel decay. Per head, with S a dk x dv fp32 matrix:
 *
 *     S_t = Diag(a_t) S_{t-1} - b_t k_t (k_t^T Diag(a_t) S_{t-1}) + b_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller. The library allocates and
 *     frees no device memory, creates no stream or event, and synchronises only in
 *     kda_read_device_error: the prefill workspace and the side stream and events of a mixed
 *     batch are the caller's too.
 *   - Token tensors are dense row-major: q, k [n][H][dk] bf16; v [n][H][dv] bf16;
 *     a [n][H][dk] fp32 (decay in (0,1)); b [n][H] fp32; o [n][H][dv] bf16.
 *     Device pointers must be 16-byte aligned.
 *   - Slot state is fp32 [num_slots][H][dk][dv] (row = key channel, column = value channel).
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on it only, apart
 *     from the part of a mixed batch forked to the caller's side stream and joined back to
 *     `stream`.
 *   - Every call returns a kda_status; kda_last_error() gives a message for the last failure
 *     on the calling thread. A call rejected by its checks (any status but KDA_EHIP) enqueues
 *     no device work and changes no host state. KDA_EHIP means a HIP runtime call failed; part
 *     of the call's work may have been enqueued by then.
 *   - One pool is driven from one host thread at a time.
 *   - Apart from kda_read_device_error, a call enqueues only kernel launches (and, for a mixed
 *     batch with a side stream, the event record / wait pairs of its fork and join), so it can
 *     be captured into a HIP graph; replaying the graph repeats the device work only (the
 *     host-side slot states change once, at capture).
 *   - Supported shapes: dk == dv in {16, 128}; prefill chunk 16 (dk 16) or 64 (dk 128).
 *     Both prefill shapes run the chunked form on the matrix cores.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_EINVAL = -1,        /* bad pointer, size, alignment or slot id                  */
  KDA_ENOSLOT = -2,       /* pool exhausted                                           */
  KDA_ESTATE = -3,        /* slot in the wrong state (free / idle / pending)          */
  KDA_EUNSUPPORTED = -4,  /* shape or parameter this build does not instantiate       */
  KDA_EWORKSPACE = -5,    /* workspace missing or too small                           */
  KDA_EHIP = -6           /* a HIP runtime call failed                                */
} kda_status;

/* Device error bits, accumulated in the pool's device error word. */
#define KDA_DEVERR_NACC_RANGE 1u   /* commit got n_accepted outside [0, verified-1]; clamped */
#define KDA_DEVERR_SLOT_RANGE 2u   /* a device slot array held an id outside the pool; skipped */
#define KDA_DEVERR_DECAY_RANGE 4u  /* prefill, informational: a key channel decayed below 2^-12
                                      within a 16-token block; that block's diagonal terms of the
                                      channel were evaluated exactly in fp32 (slower path, same
                                      accuracy) instead of through fp16 factors               */

/* Pool geometry. ring_cap = positions a verify may hold (1 + max drafts), 1..64. */
typedef struct {
  int32_t num_slots, num_heads, dk, dv, ring_cap;
} kda_pool_desc;

/* Per-slot metadata kept in device memory (array of num_slots, 24 bytes each). */
typedef struct {
  int64_t pos;        /* tokens folded into the slot's state                          */
  int32_t ring_head;  /* ring entry where the next verify starts writing              */
  int32_t pending;    /* positions verified and not yet committed (0 = idle)          */
  int32_t v_base;     /* ring_head at the last verify                                 */
  int32_t v_npos;     /* positions written by the last verify                         */
} kda_slot_meta;

typedef struct kda_pool kda_pool;   /* opaque host object owned by the library */

/* ---- sizes of the caller-owned device buffers ------------------------------------------ */
/* state: num_slots*H*dk*dv*4 bytes.                                                         */
size_t kda_state_bytes(const kda_pool_desc* desc);
/* ReplaySSM ring, four sections, each 256-byte aligned, for every (slot, entry, head):
 *   k bf16 [slot][ring_cap][H][dk] | v bf16 [..][dv] | a fp32 [..][dk] | b fp32 [slot][ring_cap][H]
 * kda_ring_layout writes the byte offsets of the four sections into offsets[0..3].          */
size_t kda_ring_bytes(const kda_pool_desc* desc);
kda_status kda_ring_layout(const kda_pool_desc* desc, size_t offsets[4]);
/* meta: kda_slot_meta[num_slots], then a uint32 device error word at
 * kda_meta_error_offset(). The caller zero-fills the buffer before kda_pool_create.          */
size_t kda_meta_bytes(const kda_pool_desc* desc);
size_t kda_meta_error_offset(const kda_pool_desc* desc);

/* ---- pool and slots (prefix-cache slot pool: "Kimi K3 is here: efficient day-0 support on
 * vLLM", summary: one hybrid cache manages recurrent KDA state beside paged KV) ------------ */
/* Validates desc and the three buffers and builds the free list. Host only; no device work.
 * EINVAL on null/misaligned pointers or bad sizes, EUNSUPPORTED on dk/dv not instantiated.  */
kda_status kda_pool_create(const kda_pool_desc* desc, void* state, void* ring, void* meta,
                           kda_pool** out);
/* Frees the host object only (no device call, no synchronisation): the device buffers stay the
 * caller's, and work already enqueued on them is the caller's to wait for.                    */
kda_status kda_pool_destroy(kda_pool* pool);
/* Allocates the lowest free slot index. ENOSLOT when none is free. Host only; the slot's
 * device state is whatever it last held -- call kda_slot_reset or write it by prefill.      */
kda_status kda_slot_alloc(kda_pool* pool, int32_t* slot_out);
/* EINVAL if the slot is not live; ESTATE if it has a pending verify.                       */
kda_status kda_slot_free(kda_pool* pool, int32_t slot);
/* Zeroes a live idle slot's state and metadata (one fill kernel, no memset node).           */
kda_status kda_slot_reset(kda_pool* pool, int32_t slot, void* stream);
/* Copies the state and pos of live idle slot src into live idle slot dst (dst ring pointer
 * and pending cleared): a prefix-cache block export outside a prefill ("vLLM lifts Kimi K3
 * throughput by up to 2.8x", section "KDA checkpoints stay inside the prefill").             */
kda_status kda_slot_checkpoint(kda_pool* pool, int32_t src, int32_t dst, void* stream);

/* ---- chunked prefill with in-pass checkpoint export ------------------------------------
 * ("vLLM lifts Kimi K3 throughput by up to 2.8x", section "KDA checkpoints stay inside the
 * prefill": the recurrent-state checkpoint is exported during the original prefill pass
 * instead of splitting the prefill at the last cacheable block boundary.)
 *
 * Sequence i covers packed tokens [cu_seqlens[i], cu_seqlens[i+1]) of q/k/v/a/b/o. It starts
 * from the state of init_slot[i] (or zeros if init_slot is NULL or init_slot[i] == -1),
 * writes o for every token, writes its final state to out_slot[i] (which may equal
 * init_slot[i]) with pos = init pos + length, and -- when ckpt_interval > 0 -- writes the
 * state after every ckpt_interval of its tokens to the next entry of ckpt_slot
 * (floor(len_i / ckpt_interval) entries per sequence, concatenated in sequence order), each
 * with pos = init pos + boundary. All out and checkpoint slots must be live, idle and
 * distinct, and no init slot may be another sequence's out or checkpoint slot.
 * chunk must be the instantiated chunk for dk. ckpt_interval may be any positive token
 * count: every checkpoint position ends a chunk, so an interval that is not a multiple of
 * the chunk cuts each interval into ceil(interval / chunk) chunks, the last one short.
 * Every h_* array is a host copy of the matching d_* device array (same contents); the host
 * copies drive validation, the device copies drive the kernels. Zero-length sequences are
 * allowed.
 * workspace: device memory, 256-byte aligned, of at least kda_prefill_workspace_bytes(pool,
 * n_tok, n_seq, chunk, ckpt_interval) bytes, owned by the caller and not touched by anything
 * else until the work on `stream` is done (the chunked form at dk 128 stages every chunk's
 * S-independent operands there, 60.5 KiB per chunk and head). A NULL or too small workspace
 * where one is needed returns KDA_EWORKSPACE; the library never allocates one.            */
typedef struct {
  const void* q; const void* k; const void* v;   /* bf16 */
  const float* a; const float* b;
  void* o;                                       /* bf16 */
  int32_t n_seq, n_tok, chunk, ckpt_interval;
  const int32_t* h_cu_seqlens; const int32_t* d_cu_seqlens;   /* [n_seq+1], starts at 0 */
  const int32_t* h_init_slot;  const int32_t* d_init_slot;    /* [n_seq] or NULL        */
  const int32_t* h_out_slot;   const int32_t* d_out_slot;     /* [n_seq]                */
  const int32_t* h_ckpt_slot;  const int32_t* d_ckpt_slot;    /* concat, or NULL        */
  void* workspace; size_t workspace_bytes;
} kda_prefill_args;
/* Workspace bytes that any prefill of n_tok tokens in n_seq sequences with that checkpoint
 * interval needs (an upper bound over length mixes: at most floor(n_tok / chunk) + n_seq
 * chunks, plus floor(n_tok / ckpt_interval) when the interval is not a multiple of the
 * chunk); 0 where none is needed (dk = 16 keeps every chunk on chip) or for n_seq <= 0.    */
size_t kda_prefill_workspace_bytes(const kda_pool* pool, int32_t n_tok, int32_t n_seq,
                                   int32_t chunk, int32_t ckpt_interval);
kda_status kda_prefill(kda_pool* pool, const kda_prefill_args* args, void* stream);
/* ---- prefill without allocation: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation) ---------------
 * kda_prefill with its workspace taken from a scratch area inside the library
 * (KDA_PREFILL_SCRATCH_BYTES per GPU, held from the library's first use on that GPU until the
 * process ends); args->workspace and workspace_bytes are ignored, and the call allocates
 * nothing. A prefill whose workspace need (kda_prefill_workspace_bytes for its lengths)
 * exceeds KDA_PREFILL_SCRATCH_BYTES returns KDA_EWORKSPACE before any device work. Every call
 * on a GPU shares that GPU's scratch, which keeps the last call's contents (a call needs none
 * of them): calls that overlap on one GPU (two streams, two threads) race and must be
 * serialised by the caller. Results are bit-identical to kda_prefill's.                      */
#define KDA_PREFILL_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_prefill_noalloc(kda_pool* pool, const kda_prefill_args* args, void* stream);
/* Width plan of kda_prefill's sequential (inter-chunk) pass for sequences with host lengths
 * h_cu_seqlens[0..n_seq] on the current device (the chunked form, dk = 128): returns the number
 * of groups G (1..4) and fills rank_end[0..G-1] and vsw[0..G-1] (caller arrays of 4): the
 * sequences ranked rank_end[i-1] .. rank_end[i] - 1 by length (longest first, ties: lower index
 * first; rank_end[-1] = 0) run in work-groups of vsw[i] value columns (16, 32, 64 or 128).
 * Long chains take narrow slices, short ones wide slices, by a latency / CU-time model; one
 * group beyond 64 sequences. kda_prefill, kda_prefill_noalloc and the prefill part of
 * kda_mixed_batch all follow this plan. Host only; returns 0 for a null argument or
 * n_seq <= 0.                                                                                */
int32_t kda_prefill_plan(const kda_pool* pool, int32_t n_seq, const int32_t* h_cu_seqlens,
                         int32_t* rank_end, int32_t* vsw);

/* ---- decode and speculative verify ---------------------------------------------------- */
/* Token tensors are [B][n_pos][H][d] (n_pos = 1 for decode); slots[B] are live, idle and
 * distinct; h_slots / d_slots are host / device copies with the same contents.              */
typedef struct {
  const void* q; const void* k; const void* v;   /* bf16 */
  const float* a; const float* b;
  void* o;                                       /* bf16 [B][n_pos][H][dv] */
  int32_t B;
  const int32_t* h_slots; const int32_t* d_slots;
} kda_step_args;

/* One token per sequence against its slot: the state is read once, updated and written
 * back in place; pos += 1. A batch of at most 64 sequences takes its slot indices from
 * h_slots (passed to the kernel by value, so d_slots is not read); larger batches read
 * d_slots. ("Kimi K3 is here: efficient day-0 support on vLLM", summary: fused kernels for
 * KDA decode.)                                                                             */
kda_status kda_decode(kda_pool* pool, const kda_step_args* args, void* stream);

/* Speculative verify of n_pos = 1 + T positions (1 <= n_pos <= ring_cap): computes o for
 * every position from the committed state (at dk = 128 and n_pos <= 16 all positions at once
 * in WY form, otherwise by stepping a register copy of the state), and appends each
 * position's (k, v, a, b) to the slot's ring from ring_head on (mod ring_cap). The committed
 * state is NOT written. Marks the slot pending (v_base = ring_head, v_npos = pending = n_pos).
 * ("vLLM lifts Kimi K3 throughput by up to 2.8x", section "ReplaySSM shrinks rollback state":
 * recent inputs stay in a buffer, the accepted state is rebuilt at commit.)                */
kda_status kda_verify(kda_pool* pool, const kda_step_args* args, int32_t n_pos, void* stream);

/* ReplaySSM commit. d_n_accepted[B] (device, e.g. written by an on-GPU sampler) gives the
 * accepted drafts n per sequence; 1 + n ring entries from v_base are replayed into the slot
 * with the same arithmetic as kda_decode (bit-identical to 1 + n decode calls), the state
 * is written once, ring_head = (v_base + 1 + n) mod ring_cap, pos += 1 + n, pending = 0.
 * n outside [0, v_npos - 1] sets KDA_DEVERR_NACC_RANGE and is clamped. Slots must be pending.
 * As for kda_decode, a batch of at most 64 takes its slot indices from h_slots.              */
kda_status kda_commit(kda_pool* pool, int32_t B, const int32_t* h_slots,
                      const int32_t* d_slots, const int32_t* d_n_accepted, void* stream);

/* Reject every drafted position: only pending is cleared; state, ring_head and pos keep
 * their values ("ReplaySSM shrinks rollback state": a reject only moves the buffer pointer). */
kda_status kda_rollback(kda_pool* pool, int32_t B, const int32_t* h_slots,
                        const int32_t* d_slots, void* stream);

/* ---- direct per-draft state checkpoints (the alternative ReplaySSM is weighed against) ---
 * ("vLLM lifts Kimi K3 throughput by up to 2.8x", section "ReplaySSM shrinks rollback state":
 * the scheme that saves the state at every drafted position, against which the ring is the
 * smaller one.) kda_verify_direct is kda_verify except that, instead of appending ring
 * entries, it writes the state after each of its n_pos positions to draft_states
 * ([B][n_pos][H][dk][dv] fp32, device, 16-byte aligned, caller-owned,
 * kda_draft_state_bytes(...) bytes). Outputs o come from the stepping form: bit-identical to
 * kda_verify's where that steps too (dk = 16, n_pos > 16), equal to its WY form up to
 * rounding otherwise. The ring is untouched; the slot becomes pending a direct commit
 * (v_base = ring_head, v_npos = pending = n_pos); 1 <= n_pos <= ring_cap as for kda_verify.
 * kda_commit_direct then copies
 * draft_states[b][n] (n = d_n_accepted[b], clamped to [0, v_npos - 1] with
 * KDA_DEVERR_NACC_RANGE as in kda_commit) into the slot: the same state kda_commit would
 * build by replay, bit for bit; pos += 1 + n, pending = 0, ring_head unchanged. The commit
 * takes the same draft_states buffer, n_pos and slot order as the verify (EINVAL otherwise);
 * kda_commit refuses slots pending a direct commit and kda_commit_direct slots pending a
 * ring commit (ESTATE); kda_rollback clears either. Draft buffers stay the caller's.     */
size_t kda_draft_state_bytes(const kda_pool_desc* desc, int32_t B, int32_t n_pos);
kda_status kda_verify_direct(kda_pool* pool, const kda_step_args* args, int32_t n_pos,
                             void* draft_states, void* stream);
kda_status kda_commit_direct(kda_pool* pool, int32_t B, const int32_t* h_slots,
                             const int32_t* d_slots, const int32_t* d_n_accepted,
                             const void* draft_states, int32_t n_pos, void* stream);

/* ---- mixed speculative / non-speculative batch ---------------------------------------
 * ("vLLM lifts Kimi K3 throughput by up to 2.8x", section "Small tensor copies leave the hot
 * path": contiguous zero-copy slices and direct output writes instead of index_select /
 * index_copy.) One packed token buffer [prefill tokens | decode tokens | verify tokens]:
 * prefill sequences take the first prefill.n_tok rows (cu_seqlens relative to row 0),
 * n_decode decode tokens follow, then n_verify * n_pos verify tokens ([seq][pos] order).
 * o is written in the same packing, with no gather or scatter; the prefill's token pointers
 * and the step slot arrays of `prefill`, `decode` and `verify` are ignored in favour of the
 * packed ones below. Commit, decode and verify touch only their own slots, so when the batch
 * also has a prefill and the caller gives a side stream they run (in that order) on that side
 * stream while the prefill's kernels run on `stream`: forked by fork_event, recorded on
 * `stream` before the prefill's first kernel, joined by join_event, recorded on the side
 * stream and waited on by `stream` before the call returns. Everything enqueued on `stream`
 * afterwards is ordered after all three parts. side_stream NULL: the three parts run in order
 * on `stream` ahead of the prefill. The side stream (default priority) and both events
 * (timing may be disabled) are the caller's; a call that uses them must not overlap another
 * call using the same events.                                                            */
typedef struct {
  const void* q; const void* k; const void* v;   /* bf16 [n_total][H][d] */
  const float* a; const float* b;
  void* o;                                       /* bf16 [n_total][H][dv] */
  kda_prefill_args prefill;                      /* slot arrays, seqlens, chunk, interval */
  int32_t n_decode;
  const int32_t* h_decode_slots; const int32_t* d_decode_slots;
  int32_t n_verify, n_pos;
  const int32_t* h_verify_slots; const int32_t* d_verify_slots;
  /* ReplaySSM commits of slots pending from an earlier verify (typically the previous
   * step's), as kda_commit with d_n_accepted: they run before this batch's decode and verify,
   * which may name the same slots again; they must not be any prefill slot. 0 = none.   */
  int32_t n_commit;
  const int32_t* h_commit_slots; const int32_t* d_commit_slots;
  const int32_t* d_n_accepted;
  void* side_stream;   /* hipStream_t or NULL                                             */
  void* fork_event;    /* hipEvent_t, required with a side stream                         */
  void* join_event;    /* hipEvent_t, required with a side stream                         */
} kda_mixed_args;
kda_status kda_mixed_batch(kda_pool* pool, const kda_mixed_args* args, void* stream);

/* ---- errors ------------------------------------------------------------------------- */
/* Synchronises `stream`, returns the device error word in *bits_out and clears it.       */
kda_status kda_read_device_error(kda_pool* pool, uint32_t* bits_out, void* stream);
const char* kda_status_string(kda_status status);
const char* kda_last_error(void);

/* Host-side view of a slot: 0 free, 1 idle, 2 pending a ring commit, 3 pending a direct
 * commit; -1 for an id out of range.                                                      */
int32_t kda_slot_host_state(const kda_pool* pool, int32_t slot);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
