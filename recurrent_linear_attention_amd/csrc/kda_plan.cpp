// Host-side planning of the chunked prefill (no device code): workspace size, the width plan of
// the sequential pass, and the device's CU count that the plan packs against.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "kda_internal.h"

namespace kda {
namespace {

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

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t prefill_plan_bytes(int n_seq) { return align256(sizeof(int32_t) * (3 * (size_t)n_seq + 1)); }

size_t prefill_workspace_bytes(int dk, int chunk, int H, int n_seq, int64_t n_chunks) {
  if (dk != PREFILL_D || chunk != PREFILL_CHUNK || n_seq <= 0) return 0;
  return prefill_plan_bytes(n_seq) + (size_t)n_chunks * H * PREFILL_BLOCK_BYTES;
}

StatePlan plan_state_pass(const int32_t* h_cu, int n_seq, int H) {
  // Per-chunk latency of one chain (us) with 16, 32, 64 and 128 value columns per work-group,
  // measured on MI355X for the mixed 16384-token batch, plus a work-group's start-up; the pass
  // keeps one work-group per CU, and list scheduling in rank order packs CU-time to ~85%.
  constexpr float LAT[4] = {1.55f, 1.8f, 2.3f, 3.1f};
  constexpr float START = 3.f, PACK = 0.85f;
  constexpr int WIDTH[4] = {16, 32, 64, 128};
  const int cus = device_cu_count();
  auto build = [&](int n_groups, const int* ends, const int* widths) {
    StatePlan sp{};
    sp.n_groups = n_groups;
    int begin = 0, r0 = 0;
    for (int g = 0; g < n_groups; ++g) {
      sp.rank_end[g] = ends[g];
      sp.vsw[g] = widths[g];
      sp.wg_begin[g] = begin;
      begin += ((ends[g] - r0) * H + 7) / 8 * 8 * (PREFILL_D / widths[g]);
      r0 = ends[g];
    }
    sp.wg_begin[n_groups] = begin;
    return sp;
  };
  // one width for all: the narrowest whose grid fits in one round of CUs, else 64 columns
  const int n_hg = n_seq * H;
  const int wu = n_hg * 8 <= cus ? 0 : (n_hg * 4 <= cus ? 1 : 2);
  const int end_all[1] = {n_seq}, w_all[1] = {WIDTH[wu]};
  const StatePlan uniform = build(1, end_all, w_all);
  if (n_seq < 2 || n_seq > PREFILL_PLAN_INLINE_MAX) return uniform;
  // chunk counts in rank order: descending length, ties lower index first (the plan's order)
  int idx[PREFILL_PLAN_INLINE_MAX], nch[PREFILL_PLAN_INLINE_MAX];
  for (int i = 0; i < n_seq; ++i) idx[i] = i;
  auto len = [&](int i) { return h_cu[i + 1] - h_cu[i]; };
  std::stable_sort(idx, idx + n_seq, [&](int x, int y) { return len(x) > len(y); });
  for (int r = 0; r < n_seq; ++r) nch[r] = seq_chunks(len(idx[r]), PREFILL_CHUNK, 0);
  auto predict = [&](const int* wi) {
    float chain = 0.f, cu_time = 0.f;
    int64_t wgs = 0;
    for (int r = 0; r < n_seq; ++r) {
      const float t = nch[r] * LAT[wi[r]] + START;
      const int slices = PREFILL_D / WIDTH[wi[r]];
      chain = std::max(chain, t);
      cu_time += (float)H * slices * t;
      wgs += (int64_t)H * slices;
    }
    return wgs <= cus ? chain : std::max(chain, cu_time / (PACK * cus));
  };
  int wi[PREFILL_PLAN_INLINE_MAX], best[PREFILL_PLAN_INLINE_MAX];
  for (int r = 0; r < n_seq; ++r) wi[r] = wu;
  const float t_uniform = predict(wi);
  float t_best = t_uniform;
  bool found = false;
  // each candidate bounds every chain by one chain's time at one width; each rank then takes
  // the widest slices that stay within it (non-decreasing along the ranks)
  for (int rr = 0; rr < n_seq; ++rr)
    for (int ww = 0; ww < 4; ++ww) {
      const float bound = nch[rr] * LAT[ww] + START;
      bool ok = true;
      for (int r = 0; r < n_seq && ok; ++r) {
        int w = 3;
        while (w >= 0 && nch[r] * LAT[w] + START > bound) --w;
        if (w < 0) ok = false;
        wi[r] = w;
      }
      if (!ok) continue;
      const float t = predict(wi);
      if (t < t_best) {
        t_best = t;
        found = true;
        std::copy(wi, wi + n_seq, best);
      }
    }
  // a different plan only for a clear predicted gain (the model is coarse)
  if (!found || t_best > 0.95f * t_uniform) return uniform;
  int ends[4], widths[4], n_groups = 0;
  for (int r = 0; r < n_seq; ++r) {
    if (n_groups == 0 || WIDTH[best[r]] != widths[n_groups - 1]) {
      if (n_groups == 4) return uniform;
      widths[n_groups++] = WIDTH[best[r]];
    }
    ends[n_groups - 1] = r + 1;
  }
  return build(n_groups, ends, widths);
}

}  // namespace kda
