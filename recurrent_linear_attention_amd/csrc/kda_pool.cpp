// Host side of the KDA engine: pool geometry, slot free list and idle/pending state
// machine, argument validation, and dispatch to the kernel launchers. The library allocates no
// device memory and creates no stream or event: every device buffer, the prefill workspace, and
// the side stream and events of a mixed batch belong to the caller.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kda_status hip_fail(hipError_t e, const char* what) {
  return fail(KDA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Host slot states; SLOT_ANY_PENDING is only a check argument (either pending state).
enum : uint8_t { SLOT_FREE = 0, SLOT_IDLE = 1, SLOT_PENDING = 2, SLOT_PENDING_DIRECT = 3, SLOT_ANY_PENDING = 4 };

kda_status check_desc(const kda_pool_desc* d) {
  if (!d) return fail(KDA_EINVAL, "null pool descriptor");
  if (d->num_slots <= 0 || d->num_heads <= 0 || d->dk <= 0 || d->dv <= 0)
    return fail(KDA_EINVAL, "pool sizes must be positive");
  if (d->ring_cap < 1 || d->ring_cap > 64) return fail(KDA_EINVAL, "ring_cap must be 1..64");
  if (d->dk != d->dv || !kda::supported_dim(d->dk))
    return fail(KDA_EUNSUPPORTED, "dk = dv in {16, 128} only (got dk=%d dv=%d)", d->dk, d->dv);
  return KDA_OK;
}

void ring_offsets(const kda_pool_desc* d, size_t off[4], size_t* total) {
  size_t per = (size_t)d->num_slots * d->ring_cap * d->num_heads;
  off[0] = 0;
  off[1] = align_up(off[0] + per * d->dk * 2, 256);
  off[2] = align_up(off[1] + per * d->dv * 2, 256);
  off[3] = align_up(off[2] + per * d->dk * 4, 256);
  *total = align_up(off[3] + per * 4, 256);
}

}  // namespace

struct kda_pool {
  kda_pool_desc desc;
  kda::PoolView view;
  std::vector<uint8_t> slot_state;     // SLOT_FREE / SLOT_IDLE / SLOT_PENDING / SLOT_PENDING_DIRECT
  // Direct verify of a slot pending a direct commit: its draft buffer, n_pos and batch index.
  std::vector<const void*> draft_buf;
  std::vector<int32_t> draft_npos, draft_index;
  std::vector<uint32_t> stamp;         // distinctness checks
  uint32_t epoch = 0;

  // Mark-and-check: returns false if a slot repeats within one validation pass.
  void begin_pass() {
    if (++epoch == 0) {
      std::fill(stamp.begin(), stamp.end(), 0u);
      epoch = 1;
    }
  }
  bool mark(int32_t s) {
    if (stamp[s] == epoch) return false;
    stamp[s] = epoch;
    return true;
  }
  bool marked(int32_t s) const { return stamp[s] == epoch; }
};

namespace {

kda_status check_slots(kda_pool* p, int32_t B, const int32_t* h, uint8_t want,
                       bool fresh_pass = true) {
  if (B < 0) return fail(KDA_EINVAL, "negative batch");
  if (B > 0 && !h) return fail(KDA_EINVAL, "null host slot array");
  if (fresh_pass) p->begin_pass();
  for (int32_t i = 0; i < B; ++i) {
    int32_t s = h[i];
    if (s < 0 || s >= p->desc.num_slots || p->slot_state[s] == SLOT_FREE)
      return fail(KDA_EINVAL, "slot %d (entry %d) is not a live slot", s, i);
    const uint8_t st = p->slot_state[s];
    const bool ok = want == SLOT_ANY_PENDING ? (st == SLOT_PENDING || st == SLOT_PENDING_DIRECT) : st == want;
    if (!ok)
      return fail(KDA_ESTATE, "slot %d is %s", s,
                  st == SLOT_PENDING          ? "pending a ring commit (kda_commit / kda_rollback)"
                  : st == SLOT_PENDING_DIRECT ? "pending a direct commit (kda_commit_direct / kda_rollback)"
                                              : "not pending");
    if (!p->mark(s)) return fail(KDA_EINVAL, "slot %d repeats within one call", s);
  }
  return KDA_OK;
}

kda_status check_tensors(const void* q, const void* k, const void* v, const void* a,
                         const void* b, const void* o) {
  if (!q || !k || !v || !a || !b || !o) return fail(KDA_EINVAL, "null token tensor");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(a, 16) ||
      !aligned(o, 16) || !aligned(b, 4))
    return fail(KDA_EINVAL, "token tensors must be 16-byte aligned (b: 4-byte)");
  return KDA_OK;
}

kda::StepTensors tensors(const void* q, const void* k, const void* v, const float* a,
                         const float* b, void* o) {
  return kda::StepTensors{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), a, b, static_cast<uint16_t*>(o)};
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

size_t kda_state_bytes(const kda_pool_desc* d) {
  if (check_desc(d) != KDA_OK) return 0;
  return (size_t)d->num_slots * d->num_heads * d->dk * d->dv * sizeof(float);
}

size_t kda_draft_state_bytes(const kda_pool_desc* d, int32_t B, int32_t n_pos) {
  if (check_desc(d) != KDA_OK || B < 0 || n_pos < 0) return 0;
  return (size_t)B * n_pos * d->num_heads * d->dk * d->dv * sizeof(float);
}

size_t kda_ring_bytes(const kda_pool_desc* d) {
  if (check_desc(d) != KDA_OK) return 0;
  size_t off[4], total;
  ring_offsets(d, off, &total);
  return total;
}

kda_status kda_ring_layout(const kda_pool_desc* d, size_t offsets[4]) {
  kda_status st = check_desc(d);
  if (st != KDA_OK) return st;
  if (!offsets) return fail(KDA_EINVAL, "null offsets");
  size_t total;
  ring_offsets(d, offsets, &total);
  return KDA_OK;
}

size_t kda_meta_error_offset(const kda_pool_desc* d) {
  if (check_desc(d) != KDA_OK) return 0;
  return align_up((size_t)d->num_slots * sizeof(kda_slot_meta), 256);
}

size_t kda_meta_bytes(const kda_pool_desc* d) {
  if (check_desc(d) != KDA_OK) return 0;
  return kda_meta_error_offset(d) + 256;
}

kda_status kda_pool_create(const kda_pool_desc* d, void* state, void* ring, void* meta,
                           kda_pool** out) {
  kda_status st = check_desc(d);
  if (st != KDA_OK) return st;
  if (!out) return fail(KDA_EINVAL, "null output handle");
  if (!state || !ring || !meta) return fail(KDA_EINVAL, "null device buffer");
  if (!aligned(state, 256) || !aligned(ring, 256) || !aligned(meta, 256))
    return fail(KDA_EINVAL, "device buffers must be 256-byte aligned");
  kda_pool* p = new (std::nothrow) kda_pool();
  if (!p) return fail(KDA_EINVAL, "out of host memory");
  p->desc = *d;
  size_t off[4], total;
  ring_offsets(d, off, &total);
  char* r = static_cast<char*>(ring);
  p->view.state = static_cast<float*>(state);
  p->view.ring_k = reinterpret_cast<uint16_t*>(r + off[0]);
  p->view.ring_v = reinterpret_cast<uint16_t*>(r + off[1]);
  p->view.ring_a = reinterpret_cast<float*>(r + off[2]);
  p->view.ring_b = reinterpret_cast<float*>(r + off[3]);
  p->view.meta = static_cast<kda_slot_meta*>(meta);
  p->view.err = reinterpret_cast<uint32_t*>(static_cast<char*>(meta) + kda_meta_error_offset(d));
  p->view.num_slots = d->num_slots;
  p->view.H = d->num_heads;
  p->view.dk = d->dk;
  p->view.dv = d->dv;
  p->view.R = d->ring_cap;
  p->slot_state.assign(d->num_slots, SLOT_FREE);
  p->draft_buf.assign(d->num_slots, nullptr);
  p->draft_npos.assign(d->num_slots, 0);
  p->draft_index.assign(d->num_slots, 0);
  p->stamp.assign(d->num_slots, 0u);
  *out = p;
  return KDA_OK;
}

kda_status kda_pool_destroy(kda_pool* p) {
  if (!p) return fail(KDA_EINVAL, "null pool");
  delete p;
  return KDA_OK;
}

kda_status kda_slot_alloc(kda_pool* p, int32_t* slot_out) {
  if (!p || !slot_out) return fail(KDA_EINVAL, "null argument");
  for (int32_t s = 0; s < p->desc.num_slots; ++s) {
    if (p->slot_state[s] == SLOT_FREE) {
      p->slot_state[s] = SLOT_IDLE;
      *slot_out = s;
      return KDA_OK;
    }
  }
  return fail(KDA_ENOSLOT, "all %d slots are live", p->desc.num_slots);
}

kda_status kda_slot_free(kda_pool* p, int32_t s) {
  if (!p) return fail(KDA_EINVAL, "null pool");
  if (s < 0 || s >= p->desc.num_slots || p->slot_state[s] == SLOT_FREE)
    return fail(KDA_EINVAL, "slot %d is not live", s);
  if (p->slot_state[s] == SLOT_PENDING || p->slot_state[s] == SLOT_PENDING_DIRECT)
    return fail(KDA_ESTATE, "slot %d is pending", s);
  p->slot_state[s] = SLOT_FREE;
  return KDA_OK;
}

int32_t kda_prefill_plan(const kda_pool* p, int32_t n_seq, const int32_t* h_cu, int32_t* rank_end,
                         int32_t* vsw) {
  if (!p || !h_cu || !rank_end || !vsw || n_seq <= 0) return 0;
  const kda::StatePlan sp = kda::plan_state_pass(h_cu, n_seq, p->desc.num_heads);
  for (int32_t g = 0; g < sp.n_groups; ++g) {
    rank_end[g] = sp.rank_end[g];
    vsw[g] = sp.vsw[g];
  }
  return sp.n_groups;
}

int32_t kda_slot_host_state(const kda_pool* p, int32_t s) {
  if (!p || s < 0 || s >= p->desc.num_slots) return -1;
  return p->slot_state[s];
}

kda_status kda_slot_reset(kda_pool* p, int32_t s, void* stream) {
  if (!p) return fail(KDA_EINVAL, "null pool");
  kda_status st = check_slots(p, 1, &s, SLOT_IDLE);
  if (st != KDA_OK) return st;
  hipError_t e = kda::launch_slot_reset(p->view, s, as_stream(stream));
  return e == hipSuccess ? KDA_OK : hip_fail(e, "slot reset launch");
}

kda_status kda_slot_checkpoint(kda_pool* p, int32_t src, int32_t dst, void* stream) {
  if (!p) return fail(KDA_EINVAL, "null pool");
  int32_t pair[2] = {src, dst};
  kda_status st = check_slots(p, 2, pair, SLOT_IDLE);
  if (st != KDA_OK) return st;
  hipError_t e = kda::launch_slot_copy(p->view, src, dst, as_stream(stream));
  return e == hipSuccess ? KDA_OK : hip_fail(e, "slot checkpoint launch");
}

size_t kda_prefill_workspace_bytes(const kda_pool* p, int32_t n_tok, int32_t n_seq,
                                   int32_t chunk, int32_t ckpt_interval) {
  if (!p || n_tok < 0 || n_seq <= 0 || chunk <= 0 || ckpt_interval < 0) return 0;
  // sum_i seq_chunks(len_i) <= floor(n_tok / chunk) + n_seq, plus one more chunk per
  // checkpoint boundary when the interval is not a multiple of the chunk
  int64_t bound = (int64_t)(n_tok / chunk) + n_seq;
  if (ckpt_interval > 0 && ckpt_interval % chunk != 0) bound += n_tok / ckpt_interval;
  return kda::prefill_workspace_bytes(p->desc.dk, chunk, p->desc.num_heads, n_seq, bound);
}

static kda_status validate_prefill(kda_pool* p, const kda_prefill_args* a, bool tensors_needed,
                                   int32_t* max_len, int64_t* n_chunks) {
  if (!p || !a) return fail(KDA_EINVAL, "null argument");
  if (a->n_seq < 0 || a->n_tok < 0) return fail(KDA_EINVAL, "negative n_seq / n_tok");
  if (a->chunk != kda::prefill_chunk_for(p->desc.dk))
    return fail(KDA_EUNSUPPORTED, "chunk %d not instantiated for d=%d (use %d)", a->chunk,
                p->desc.dk, kda::prefill_chunk_for(p->desc.dk));
  if (a->ckpt_interval < 0)
    return fail(KDA_EUNSUPPORTED, "negative checkpoint interval %d", a->ckpt_interval);
  *n_chunks = 0;
  if (a->n_seq == 0) {
    *max_len = 0;
    return a->n_tok == 0 ? KDA_OK : fail(KDA_EINVAL, "tokens without sequences");
  }
  if (tensors_needed) {
    kda_status st = check_tensors(a->q, a->k, a->v, a->a, a->b, a->o);
    if (st != KDA_OK && a->n_tok > 0) return st;
  }
  if (!a->h_cu_seqlens || !a->d_cu_seqlens || !a->h_out_slot || !a->d_out_slot)
    return fail(KDA_EINVAL, "null cu_seqlens / out_slot");
  if ((a->h_init_slot == nullptr) != (a->d_init_slot == nullptr))
    return fail(KDA_EINVAL, "init_slot host and device copies must both be given or both NULL");
  const int32_t* cu = a->h_cu_seqlens;
  if (cu[0] != 0) return fail(KDA_EINVAL, "cu_seqlens[0] must be 0");
  int64_t n_ckpt = 0, nch = 0;
  int32_t mx = 0;
  for (int32_t i = 0; i < a->n_seq; ++i) {
    if (cu[i + 1] < cu[i]) return fail(KDA_EINVAL, "cu_seqlens must be non-decreasing");
    int32_t len = cu[i + 1] - cu[i];
    mx = len > mx ? len : mx;
    nch += kda::seq_chunks(len, a->chunk, a->ckpt_interval);
    if (a->ckpt_interval > 0) n_ckpt += len / a->ckpt_interval;
  }
  if (cu[a->n_seq] != a->n_tok) return fail(KDA_EINVAL, "cu_seqlens[n_seq] != n_tok");
  if (n_ckpt > 0 && (!a->h_ckpt_slot || !a->d_ckpt_slot))
    return fail(KDA_EINVAL, "checkpoint slots required (%lld)", (long long)n_ckpt);
  // out and checkpoint slots: live, idle, all distinct.
  kda_status st = check_slots(p, a->n_seq, a->h_out_slot, SLOT_IDLE);
  if (st != KDA_OK) return st;
  if (n_ckpt > 0) {
    st = check_slots(p, (int32_t)n_ckpt, a->h_ckpt_slot, SLOT_IDLE, /*fresh_pass=*/false);
    if (st != KDA_OK) return st;
  }
  // init slots: -1 or live idle; never another sequence's out slot nor any checkpoint slot.
  if (a->h_init_slot) {
    for (int32_t i = 0; i < a->n_seq; ++i) {
      int32_t s = a->h_init_slot[i];
      if (s == -1) continue;
      if (s < 0 || s >= p->desc.num_slots || p->slot_state[s] == SLOT_FREE)
        return fail(KDA_EINVAL, "init slot %d is not live", s);
      if (p->slot_state[s] != SLOT_IDLE) return fail(KDA_ESTATE, "init slot %d is pending", s);
      if (p->marked(s) && s != a->h_out_slot[i])
        return fail(KDA_EINVAL, "init slot %d is written by this prefill", s);
    }
  }
  *max_len = mx;
  *n_chunks = nch;
  return KDA_OK;
}

// Device workspace of a prefill: the caller's buffer, checked against the need. The library
// never allocates one itself.
static kda_status prefill_workspace(kda_pool* p, const kda_prefill_args* a, int64_t n_chunks,
                                    void** ws) {
  const size_t need =
      kda::prefill_workspace_bytes(p->desc.dk, a->chunk, p->desc.num_heads, a->n_seq, n_chunks);
  *ws = nullptr;
  if (need == 0) return KDA_OK;
  if (!a->workspace)
    return fail(KDA_EWORKSPACE, "no workspace given, this prefill needs %zu bytes", need);
  if (a->workspace_bytes < need)
    return fail(KDA_EWORKSPACE, "workspace of %zu bytes, this prefill needs %zu",
                a->workspace_bytes, need);
  if (!aligned(a->workspace, 256)) return fail(KDA_EINVAL, "workspace must be 256-byte aligned");
  *ws = a->workspace;
  return KDA_OK;
}

static kda_status run_prefill(kda_pool* p, const kda_prefill_args* a, int32_t max_len,
                              int64_t n_chunks, void* ws, void* stream) {
  kda::PrefillLaunch L{tensors(a->q, a->k, a->v, a->a, a->b, a->o), a->n_seq, a->n_tok,
                       a->chunk, a->ckpt_interval, a->d_cu_seqlens, a->d_init_slot,
                       a->d_out_slot, a->d_ckpt_slot, max_len, n_chunks, ws};
  L.plan = kda::plan_state_pass(a->h_cu_seqlens, a->n_seq, p->desc.num_heads);
  hipError_t e = kda::launch_prefill(p->view, L, as_stream(stream));
  return e == hipSuccess ? KDA_OK : hip_fail(e, "prefill launch");
}

kda_status kda_prefill(kda_pool* p, const kda_prefill_args* a, void* stream) {
  int32_t max_len = 0;
  int64_t n_chunks = 0;
  kda_status st = validate_prefill(p, a, true, &max_len, &n_chunks);
  if (st != KDA_OK) return st;
  if (a->n_seq == 0) return KDA_OK;
  void* ws = nullptr;
  st = prefill_workspace(p, a, n_chunks, &ws);
  if (st != KDA_OK) return st;
  return run_prefill(p, a, max_len, n_chunks, ws, stream);
}

static_assert(KDA_PREFILL_SCRATCH_BYTES == kda::PREFILL_SCRATCH_BYTES, "scratch size in the header");

kda_status kda_prefill_noalloc(kda_pool* p, const kda_prefill_args* a, void* stream) {
  int32_t max_len = 0;
  int64_t n_chunks = 0;
  kda_status st = validate_prefill(p, a, true, &max_len, &n_chunks);
  if (st != KDA_OK) return st;
  if (a->n_seq == 0) return KDA_OK;
  const size_t need =
      kda::prefill_workspace_bytes(p->desc.dk, a->chunk, p->desc.num_heads, a->n_seq, n_chunks);
  if (need > kda::PREFILL_SCRATCH_BYTES)
    return fail(KDA_EWORKSPACE,
                "this prefill needs %zu bytes of workspace; kda_prefill_noalloc holds %zu "
                "(split the prefill, or call kda_prefill with a workspace)",
                need, (size_t)kda::PREFILL_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = kda::prefill_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
  }
  return run_prefill(p, a, max_len, n_chunks, ws, stream);
}

kda_status kda_decode(kda_pool* p, const kda_step_args* a, void* stream) {
  if (!p || !a) return fail(KDA_EINVAL, "null argument");
  kda_status st = check_slots(p, a->B, a->h_slots, SLOT_IDLE);
  if (st != KDA_OK) return st;
  if (a->B == 0) return KDA_OK;
  st = check_tensors(a->q, a->k, a->v, a->a, a->b, a->o);
  if (st != KDA_OK) return st;
  if (!a->d_slots) return fail(KDA_EINVAL, "null device slot array");
  hipError_t e = kda::launch_decode(p->view, tensors(a->q, a->k, a->v, a->a, a->b, a->o), a->B,
                                    a->h_slots, a->d_slots, as_stream(stream));
  return e == hipSuccess ? KDA_OK : hip_fail(e, "decode launch");
}

kda_status kda_verify(kda_pool* p, const kda_step_args* a, int32_t n_pos, void* stream) {
  if (!p || !a) return fail(KDA_EINVAL, "null argument");
  if (n_pos < 1 || n_pos > p->desc.ring_cap)
    return fail(KDA_EINVAL, "n_pos %d outside 1..ring_cap (%d)", n_pos, p->desc.ring_cap);
  kda_status st = check_slots(p, a->B, a->h_slots, SLOT_IDLE);
  if (st != KDA_OK) return st;
  if (a->B == 0) return KDA_OK;
  st = check_tensors(a->q, a->k, a->v, a->a, a->b, a->o);
  if (st != KDA_OK) return st;
  if (!a->d_slots) return fail(KDA_EINVAL, "null device slot array");
  hipError_t e = kda::launch_verify(p->view, tensors(a->q, a->k, a->v, a->a, a->b, a->o), a->B,
                                    n_pos, a->d_slots, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "verify launch");
  for (int32_t i = 0; i < a->B; ++i) p->slot_state[a->h_slots[i]] = SLOT_PENDING;
  return KDA_OK;
}

kda_status kda_commit(kda_pool* p, int32_t B, const int32_t* h_slots, const int32_t* d_slots,
                      const int32_t* d_n_accepted, void* stream) {
  if (!p) return fail(KDA_EINVAL, "null pool");
  kda_status st = check_slots(p, B, h_slots, SLOT_PENDING);
  if (st != KDA_OK) return st;
  if (B == 0) return KDA_OK;
  if (!d_slots || !d_n_accepted) return fail(KDA_EINVAL, "null device array");
  hipError_t e = kda::launch_commit(p->view, B, h_slots, d_slots, d_n_accepted, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "commit launch");
  for (int32_t i = 0; i < B; ++i) p->slot_state[h_slots[i]] = SLOT_IDLE;
  return KDA_OK;
}

kda_status kda_rollback(kda_pool* p, int32_t B, const int32_t* h_slots, const int32_t* d_slots,
                        void* stream) {
  if (!p) return fail(KDA_EINVAL, "null pool");
  kda_status st = check_slots(p, B, h_slots, SLOT_ANY_PENDING);
  if (st != KDA_OK) return st;
  if (B == 0) return KDA_OK;
  if (!d_slots) return fail(KDA_EINVAL, "null device slot array");
  hipError_t e = kda::launch_rollback(p->view, B, d_slots, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "rollback launch");
  for (int32_t i = 0; i < B; ++i) p->slot_state[h_slots[i]] = SLOT_IDLE;
  return KDA_OK;
}

kda_status kda_mixed_batch(kda_pool* p, const kda_mixed_args* m, void* stream) {
  if (!p || !m) return fail(KDA_EINVAL, "null argument");
  const int32_t H = p->desc.num_heads, dk = p->desc.dk, dv = p->desc.dv;
  if (m->n_decode < 0 || m->n_verify < 0 || m->n_commit < 0) return fail(KDA_EINVAL, "negative batch");
  if (m->side_stream && (!m->fork_event || !m->join_event))
    return fail(KDA_EINVAL, "a side stream needs its fork and join events");
  if (m->n_verify > 0 && (m->n_pos < 1 || m->n_pos > p->desc.ring_cap))
    return fail(KDA_EINVAL, "n_pos %d outside 1..ring_cap", m->n_pos);
  kda_status st = check_tensors(m->q, m->k, m->v, m->a, m->b, m->o);
  if (st != KDA_OK) return st;
  // Validate every part before launching any of them, so a failure enqueues nothing.
  kda_prefill_args pre = m->prefill;
  pre.q = m->q; pre.k = m->k; pre.v = m->v; pre.a = m->a; pre.b = m->b; pre.o = m->o;
  int32_t max_len = 0;
  int64_t n_chunks = 0;
  st = validate_prefill(p, &pre, false, &max_len, &n_chunks);
  if (st != KDA_OK) return st;
  auto mark_prefill_slots = [&]() {
    p->begin_pass();
    for (int32_t i = 0; i < pre.n_seq; ++i) p->mark(pre.h_out_slot[i]);
    if (pre.ckpt_interval > 0 && pre.h_ckpt_slot) {
      int64_t n_ckpt = 0;
      for (int32_t i = 0; i < pre.n_seq; ++i)
        n_ckpt += (pre.h_cu_seqlens[i + 1] - pre.h_cu_seqlens[i]) / pre.ckpt_interval;
      for (int64_t i = 0; i < n_ckpt; ++i) p->mark(pre.h_ckpt_slot[i]);
    }
    if (pre.h_init_slot)
      for (int32_t i = 0; i < pre.n_seq; ++i)
        if (pre.h_init_slot[i] >= 0) p->mark(pre.h_init_slot[i]);
  };
  // Commit slots: pending a ring commit, distinct from each other and from the prefill's slots
  // (the prefill is not ordered against the side stream).
  mark_prefill_slots();
  st = check_slots(p, m->n_commit, m->h_commit_slots, SLOT_PENDING, false);
  if (st != KDA_OK) return st;
  if (m->n_commit > 0 && (!m->d_commit_slots || !m->d_n_accepted))
    return fail(KDA_EINVAL, "null device commit array");
  if ((m->n_decode > 0 && !m->d_decode_slots) || (m->n_verify > 0 && !m->d_verify_slots))
    return fail(KDA_EINVAL, "null device slot array");
  // Decode and verify slots: idle once the commits are done (they run first, in order on the
  // same stream), distinct from each other and from the prefill's slots. The commit slots are
  // marked idle here; every failure before the first launch marks them pending again, so a
  // rejected call leaves the pool as it was.
  for (int32_t i = 0; i < m->n_commit; ++i) p->slot_state[m->h_commit_slots[i]] = SLOT_IDLE;
  auto keep_pending = [&](kda_status why) {
    for (int32_t i = 0; i < m->n_commit; ++i) p->slot_state[m->h_commit_slots[i]] = SLOT_PENDING;
    return why;
  };
  mark_prefill_slots();
  st = check_slots(p, m->n_decode, m->h_decode_slots, SLOT_IDLE, false);
  if (st == KDA_OK) st = check_slots(p, m->n_verify, m->h_verify_slots, SLOT_IDLE, false);
  if (st != KDA_OK) return keep_pending(st);

  hipStream_t s = as_stream(stream);
  const size_t n_pre = (size_t)pre.n_tok;
  auto part = [&](size_t row) {
    return tensors(static_cast<const uint16_t*>(m->q) + row * H * dk,
                   static_cast<const uint16_t*>(m->k) + row * H * dk,
                   static_cast<const uint16_t*>(m->v) + row * H * dv, m->a + row * H * dk,
                   m->b + row * H, static_cast<uint16_t*>(m->o) + row * H * dv);
  };
  // Commit, decode and verify touch only their own slots (checked distinct from the
  // prefill's above), so they need no order against the prefill: with a prefill in the batch
  // and a side stream given they go to the side stream, in that order, ahead of the prefill's
  // kernels, and the caller's stream waits for them before anything later. They then run beside
  // the prefill's S-independent kernel (whose work-groups leave room on each CU) and are done
  // before its sequential pass starts, which therefore keeps every CU and its width plan.
  struct StepLaunches {
    kda_pool* p;
    const kda_mixed_args* m;
    kda::StepTensors dec, ver;
    hipStream_t s, aux;
    hipEvent_t ev_fork, ev_join;
    bool fork;
    hipError_t run(hipStream_t on) const {
      hipError_t e = hipSuccess;
      if (m->n_commit > 0) {
        e = kda::launch_commit(p->view, m->n_commit, m->h_commit_slots, m->d_commit_slots, m->d_n_accepted, on);
        if (e != hipSuccess) return e;
      }
      if (m->n_decode > 0) {
        e = kda::launch_decode(p->view, dec, m->n_decode, m->h_decode_slots, m->d_decode_slots, on);
        if (e != hipSuccess) return e;
      }
      if (m->n_verify > 0)
        e = kda::launch_verify(p->view, ver, m->n_verify, m->n_pos, m->d_verify_slots, on);
      return e;
    }
    hipError_t forked() const {
      hipError_t e = hipEventRecord(ev_fork, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(aux, ev_fork, 0);
      if (e == hipSuccess) e = run(aux);
      if (e == hipSuccess) e = hipEventRecord(ev_join, aux);
      return e;
    }
  };
  const bool steps = m->n_decode > 0 || m->n_verify > 0 || m->n_commit > 0;
  StepLaunches sl{p, m, part(n_pre), part(n_pre + m->n_decode), s, as_stream(m->side_stream),
                  static_cast<hipEvent_t>(m->fork_event), static_cast<hipEvent_t>(m->join_event),
                  pre.n_seq > 0 && steps && m->side_stream != nullptr};
  hipError_t e = hipSuccess;
  if (pre.n_seq > 0) {
    void* ws = nullptr;
    st = prefill_workspace(p, &pre, n_chunks, &ws);
    if (st != KDA_OK) return keep_pending(st);
    kda::PrefillLaunch L{part(0), pre.n_seq, pre.n_tok, pre.chunk, pre.ckpt_interval,
                         pre.d_cu_seqlens, pre.d_init_slot, pre.d_out_slot, pre.d_ckpt_slot,
                         max_len, n_chunks, ws};
    L.plan = kda::plan_state_pass(pre.h_cu_seqlens, pre.n_seq, H);
    if (sl.fork) {
      e = sl.forked();
      if (e != hipSuccess) return hip_fail(e, "mixed: side stream");
    } else if (steps) {
      e = sl.run(s);
      if (e != hipSuccess) return hip_fail(e, "mixed: commit / decode / verify launch");
    }
    e = kda::launch_prefill(p->view, L, s);
    if (e != hipSuccess) return hip_fail(e, "mixed: prefill launch");
    if (sl.fork) {
      e = hipStreamWaitEvent(s, sl.ev_join, 0);
      if (e != hipSuccess) return hip_fail(e, "mixed: join");
    }
  } else if (steps) {
    e = sl.run(s);
    if (e != hipSuccess) return hip_fail(e, "mixed: commit / decode / verify launch");
  }
  for (int32_t i = 0; i < m->n_verify; ++i) p->slot_state[m->h_verify_slots[i]] = SLOT_PENDING;
  return KDA_OK;
}

kda_status kda_verify_direct(kda_pool* p, const kda_step_args* a, int32_t n_pos, void* draft,
                             void* stream) {
  if (!p || !a) return fail(KDA_EINVAL, "null argument");
  if (n_pos < 1 || n_pos > p->desc.ring_cap)
    return fail(KDA_EINVAL, "n_pos %d outside 1..ring_cap (%d)", n_pos, p->desc.ring_cap);
  kda_status st = check_slots(p, a->B, a->h_slots, SLOT_IDLE);
  if (st != KDA_OK) return st;
  if (a->B == 0) return KDA_OK;
  st = check_tensors(a->q, a->k, a->v, a->a, a->b, a->o);
  if (st != KDA_OK) return st;
  if (!a->d_slots) return fail(KDA_EINVAL, "null device slot array");
  if (!draft || !aligned(draft, 16)) return fail(KDA_EINVAL, "draft states must be 16-byte aligned");
  hipError_t e = kda::launch_verify_direct(p->view, tensors(a->q, a->k, a->v, a->a, a->b, a->o), a->B,
                                           n_pos, a->d_slots, static_cast<float*>(draft), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "direct verify launch");
  for (int32_t i = 0; i < a->B; ++i) {
    const int32_t s = a->h_slots[i];
    p->slot_state[s] = SLOT_PENDING_DIRECT;
    p->draft_buf[s] = draft;
    p->draft_npos[s] = n_pos;
    p->draft_index[s] = i;
  }
  return KDA_OK;
}

kda_status kda_commit_direct(kda_pool* p, int32_t B, const int32_t* h_slots, const int32_t* d_slots,
                             const int32_t* d_n_accepted, const void* draft, int32_t n_pos,
                             void* stream) {
  if (!p) return fail(KDA_EINVAL, "null pool");
  kda_status st = check_slots(p, B, h_slots, SLOT_PENDING_DIRECT);
  if (st != KDA_OK) return st;
  if (B == 0) return KDA_OK;
  if (!d_slots || !d_n_accepted) return fail(KDA_EINVAL, "null device array");
  for (int32_t i = 0; i < B; ++i) {
    const int32_t s = h_slots[i];
    if (p->draft_buf[s] != draft || p->draft_npos[s] != n_pos || p->draft_index[s] != i)
      return fail(KDA_EINVAL,
                  "slot %d (entry %d): draft buffer, n_pos and slot order must match its direct "
                  "verify (entry %d, n_pos %d)", s, i, p->draft_index[s], p->draft_npos[s]);
  }
  hipError_t e = kda::launch_commit_direct(p->view, B, d_slots, d_n_accepted,
                                           static_cast<const float*>(draft), n_pos, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "direct commit launch");
  for (int32_t i = 0; i < B; ++i) {
    p->slot_state[h_slots[i]] = SLOT_IDLE;
    p->draft_buf[h_slots[i]] = nullptr;
  }
  return KDA_OK;
}

kda_status kda_read_device_error(kda_pool* p, uint32_t* bits_out, void* stream) {
  if (!p || !bits_out) return fail(KDA_EINVAL, "null argument");
  hipStream_t s = as_stream(stream);
  uint32_t bits = 0;
  hipError_t e = hipMemcpyAsync(&bits, p->view.err, sizeof bits, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = kda::launch_clear_word(p->view.err, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the device error word");
  *bits_out = bits;
  return KDA_OK;
}

const char* kda_status_string(kda_status st) {
  switch (st) {
    case KDA_OK: return "ok";
    case KDA_EINVAL: return "invalid argument";
    case KDA_ENOSLOT: return "no free slot";
    case KDA_ESTATE: return "slot in the wrong state";
    case KDA_EUNSUPPORTED: return "unsupported shape or parameter";
    case KDA_EWORKSPACE: return "workspace too small";
    case KDA_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
