// Drives the host paths of the KDA C ABI (pools, slots, the idle / pending state machine,
// argument validation, prefill planning, error strings) against the host-only build with the
// HIP stand-ins of hip_stubs.cpp, so that LeakSanitizer sees every pool destroyed and every
// pointer dropped at exit. Test infrastructure: built and run by tests/test_host_sanitizers.py
// under AddressSanitizer, LeakSanitizer and UndefinedBehaviorSanitizer. Exits non-zero on an
// unexpected status.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "kda.h"

namespace {
int failures = 0;
void expect(kda_status got, kda_status want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "%s: got %d (%s), want %d\n", what, (int)got, kda_last_error(), (int)want);
    ++failures;
  }
}
void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }
}  // namespace

int main() {
  const uintptr_t F = 1u << 20;   // 256-aligned placeholder device address, never dereferenced
  for (int round = 0; round < 3; ++round) {
    for (int d : {16, 128}) {
      kda_pool_desc desc{12, 4, d, d, 9};
      kda_pool* p = nullptr;
      expect(kda_pool_create(&desc, fake(F), fake(F), fake(F), &p), KDA_OK, "create");
      std::vector<int32_t> s(12);
      for (int i = 0; i < 12; ++i) expect(kda_slot_alloc(p, &s[i]), KDA_OK, "alloc");
      int32_t extra = -1;
      expect(kda_slot_alloc(p, &extra), KDA_ENOSLOT, "alloc past the end");
      expect(kda_slot_free(p, s[11]), KDA_OK, "free");
      expect(kda_slot_free(p, s[11]), KDA_EINVAL, "free twice");
      // verify -> commit, verify -> rollback, direct verify -> direct commit
      int32_t vs[2] = {s[0], s[1]};
      kda_step_args st{fake(F), fake(F), fake(F), (const float*)fake(F), (const float*)fake(F),
                       fake(F), 2, vs, (const int32_t*)fake(F)};
      expect(kda_verify(p, &st, 5, nullptr), KDA_OK, "verify");
      expect(kda_decode(p, &st, nullptr), KDA_ESTATE, "decode of a pending slot");
      expect(kda_slot_free(p, s[0]), KDA_ESTATE, "free of a pending slot");
      expect(kda_commit(p, 2, vs, (const int32_t*)fake(F), (const int32_t*)fake(F), nullptr), KDA_OK, "commit");
      expect(kda_verify(p, &st, 10, nullptr), KDA_EINVAL, "verify past the ring");
      expect(kda_verify(p, &st, 9, nullptr), KDA_OK, "verify");
      expect(kda_rollback(p, 2, vs, (const int32_t*)fake(F), nullptr), KDA_OK, "rollback");
      expect(kda_verify_direct(p, &st, 3, fake(F), nullptr), KDA_OK, "direct verify");
      expect(kda_commit(p, 2, vs, (const int32_t*)fake(F), (const int32_t*)fake(F), nullptr), KDA_ESTATE,
             "ring commit of a direct verify");
      expect(kda_commit_direct(p, 2, vs, (const int32_t*)fake(F), (const int32_t*)fake(F), fake(F), 3, nullptr),
             KDA_OK, "direct commit");
      expect(kda_decode(p, &st, nullptr), KDA_OK, "decode");
      expect(kda_slot_reset(p, s[2], nullptr), KDA_OK, "reset");
      expect(kda_slot_checkpoint(p, s[2], s[3], nullptr), KDA_OK, "checkpoint");
      // prefill: validation, workspace, plan, noalloc limit
      const int chunk = d == 16 ? 16 : 64;
      int32_t cu[4] = {0, 300, 300, 431}, out[3] = {s[4], s[5], s[6]}, init[3] = {-1, s[2], -1};
      int32_t ck[4] = {s[7], s[8], s[9], s[10]};
      kda_prefill_args pa{};
      pa.q = pa.k = pa.v = pa.o = fake(F);
      pa.a = pa.b = (const float*)fake(F);
      pa.n_seq = 3; pa.n_tok = 431; pa.chunk = chunk; pa.ckpt_interval = 128;
      pa.h_cu_seqlens = cu; pa.d_cu_seqlens = (const int32_t*)fake(F);
      pa.h_init_slot = init; pa.d_init_slot = (const int32_t*)fake(F);
      pa.h_out_slot = out; pa.d_out_slot = (const int32_t*)fake(F);
      pa.h_ckpt_slot = ck; pa.d_ckpt_slot = (const int32_t*)fake(F);
      const size_t need = kda_prefill_workspace_bytes(p, 431, 3, chunk, 128);
      pa.workspace = nullptr;
      expect(kda_prefill(p, &pa, nullptr), d == 16 ? KDA_OK : KDA_EWORKSPACE, "prefill without workspace");
      pa.workspace = fake(F); pa.workspace_bytes = need;
      expect(kda_prefill(p, &pa, nullptr), KDA_OK, "prefill");
      pa.chunk = 32;
      expect(kda_prefill(p, &pa, nullptr), KDA_EUNSUPPORTED, "prefill with a chunk not built");
      pa.chunk = chunk;
      int32_t bad_out[3] = {s[4], s[4], s[6]};
      pa.h_out_slot = bad_out;
      expect(kda_prefill(p, &pa, nullptr), KDA_EINVAL, "repeated out slot");
      pa.h_out_slot = out;
      int32_t ends[4], vsw[4];
      const int32_t groups = kda_prefill_plan(p, 3, cu, ends, vsw);
      if (groups < 1 || groups > 4) { std::fprintf(stderr, "plan groups %d\n", groups); ++failures; }
      if (d == 128) {
        int32_t cu_big[2] = {0, 32768}, out_big[1] = {s[4]};   // 513 chunks x 4 heads > 64 MiB
        kda_prefill_args big = pa;
        big.n_seq = 1; big.n_tok = 32768; big.ckpt_interval = 0;
        big.h_cu_seqlens = cu_big; big.h_out_slot = out_big; big.h_init_slot = nullptr;
        big.d_init_slot = nullptr; big.h_ckpt_slot = nullptr; big.d_ckpt_slot = nullptr;
        expect(kda_prefill_noalloc(p, &big, nullptr), KDA_EWORKSPACE, "noalloc beyond its scratch");
      }
      // mixed batch: overlap rejected, then a valid one with and without a side stream
      kda_mixed_args m{};
      m.q = m.k = m.v = m.o = fake(F);
      m.a = m.b = (const float*)fake(F);
      m.prefill = pa;
      int32_t dec[2] = {s[4], s[3]};
      m.n_decode = 2; m.h_decode_slots = dec; m.d_decode_slots = (const int32_t*)fake(F);
      expect(kda_mixed_batch(p, &m, nullptr), KDA_EINVAL, "mixed: decode slot = prefill out slot");
      m.n_decode = 1; m.h_decode_slots = &s[3];   // idle, not a prefill slot
      m.side_stream = fake(F);
      expect(kda_mixed_batch(p, &m, nullptr), KDA_EINVAL, "mixed: side stream without events");
      m.fork_event = m.join_event = fake(F);
      expect(kda_mixed_batch(p, &m, nullptr), KDA_OK, "mixed with a side stream");
      m.side_stream = m.fork_event = m.join_event = nullptr;
      expect(kda_mixed_batch(p, &m, nullptr), KDA_OK, "mixed without a side stream");
      uint32_t bits = 7;
      expect(kda_read_device_error(p, &bits, nullptr), KDA_OK, "read error word");
      if (bits != 0) ++failures;
      for (int i = 0; i < 11; ++i) kda_slot_free(p, s[i]);
      expect(kda_pool_destroy(p), KDA_OK, "destroy");
    }
    kda_pool_desc bad{0, 4, 128, 128, 9};
    kda_pool* q = nullptr;
    expect(kda_pool_create(&bad, fake(F), fake(F), fake(F), &q), KDA_EINVAL, "create with no slots");
    bad = kda_pool_desc{4, 4, 64, 64, 9};
    expect(kda_pool_create(&bad, fake(F), fake(F), fake(F), &q), KDA_EUNSUPPORTED, "create at d = 64");
  }
  for (int st = -6; st <= 0; ++st) (void)kda_status_string((kda_status)st);
  std::printf("host ABI driver: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
