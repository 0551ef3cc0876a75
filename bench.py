"""Benchmark: one serving step of the KDA engine on the mixed 16384-token batch, plus the
single-purpose workloads the per-kernel targets are quoted on.

A step is the whole hot path over one packed batch -- 6 chunked prefills (lognormal lengths,
16316 tokens), 32 single-token decodes, the ReplaySSM commit of the 4 sequences verified in the
previous step and 4 speculative verifies of 1+8 positions on them, all issued by one
kda_mixed_batch call -- on H=32 heads (one GPU's share), d_k = d_v = 128, a pool of 512 fp32
state slots. Inputs are synthetic and seeded (kda_inputs) and resident in HBM before timing
starts. `value` = tokens per second of the whole step (16384 / step time, wall clock over the
timed steps).

`roofline` describes the dominant part of the step, the chunked prefill (one kda_prefill call:
its chunk_prep and state_pass kernels), timed with HIP events on the stream the library
launches on, in a second pass that issues the step's calls one by one (`kernels`). Every timing
event is made with hipEventDisableSystemFence (TimingEvent), so its record adds no system-scope
cache write-back to the interval it brackets.

`configs` times each call on its own workload, cold: before every timed call a 512 MiB write
evicts the 256 MB Infinity Cache, and a HIP event pair on the call's stream brackets the call
alone (median and p10 / p90 over the iterations; `ms_clean` = the same with a 512 MiB read as
the eviction, which leaves clean lines behind: see Cold; `ms_warm` = back-to-back calls without
an eviction, for contrast):
  * decode_b16: 16 single-token decodes against a 256-slot pool (slots a random permutation);
  * verify_commit_b4: 4 speculative verifies of 1+8 positions, then the ReplaySSM commit of
    the accepted drafts (accepted counts ~ U{0..8});
  * prefill_8192: one 8192-token prompt, chunk 64, the state exported to a checkpoint slot
    every 1024 tokens inside the pass (8 checkpoints) and to the out slot.

`cpu_baseline` runs the CPU oracle (fp64 numpy, test infrastructure) on the mixed step, split
by heads over a process pool of the host's cores, before the GPU is touched.

    python bench.py [--gpus 1] [--steps 100] [--warmup 30]

Before the W warm-up steps the step runs PREWARM_STEPS times untimed (~0.3 s; reported as
`prewarm`): an idle GPU raises its clock only under sustained load, and a few warm-up steps
alone leave the timed steps up to ~10% slow. The timed steps then measure the steady serving
rate.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA tokens/s + achieved HBM GB/s (decode/verify), MFMA % (prefill), 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0      # dense bf16 / fp16
DTYPE = "bf16 q/k/v/o, fp16 matrix-core operands, fp32 state and accumulation"
PREWARM_STEPS = 700             # untimed steps before the warm-up steps (~0.3 s)

# Algorithmic bytes (d = 128, fp32 state, bf16 q/k/v/o, fp32 a and b).
D = 128
C = 64
STATE_B = D * D * 4
TOK_IN_B = 3 * D * 2 + D * 4 + 4            # q, k, v bf16 + a fp32 + b fp32
TOK_OUT_B = D * 2                           # o bf16
RING_ENTRY_B = 2 * D * 2 + D * 4 + 4        # k, v bf16 + a fp32 + b fp32
# Algorithmic flops of the chunked prefill per token-head (triangle-exact): three d x d state
# contractions (6 d^2), the intra-chunk products C (3 d_k + 2 d_v) and the triangular solve
# C^2 / 3. (The kernels need C (2 d_k + 2 d_v) of the middle term: they form W = T (V - Kt S)
# in one triangular product instead of T V and T Kt separately.)
PREFILL_FLOP_TOK_HEAD = 6 * D * D + C * (3 * D + 2 * D) + C * C / 3

# HBM traffic of one prefill call of the mixed step (its two kernels: chunk_prep, which plans a
# batch of this size itself, and state_pass), from rocprofv3 counter passes (FETCH_SIZE and
# WRITE_SIZE, KiB per dispatch) scaled by the counters' reading for a 1 GiB device copy
# (FETCH_SIZE reads half the copied bytes, WRITE_SIZE all of them: factors 2.0 and 1.0). Valid
# only for the kernel source it was measured on (first 16 hex digits of its SHA-256); for any
# other source the bench reports traffic as null.
PREFILL_TRAFFIC = {"source_sha256_16": "eafba37a442e28de", "fetch_scale": 2.0, "write_scale": 1.0,
                   "fetch_kib": {"chunk_prep_kernel": 269337, "state_pass_kernel": 316235},
                   "write_kib": {"chunk_prep_kernel": 501497, "state_pass_kernel": 142818}}


def prefill_traffic_bytes():
    import hashlib
    src = os.path.join(ROOT, "recurrent_linear_attention_amd", "csrc", "kda_prefill.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    t = PREFILL_TRAFFIC
    if sha != t["source_sha256_16"]:
        return None
    return int((sum(t["fetch_kib"].values()) * t["fetch_scale"]
                + sum(t["write_kib"].values()) * t["write_scale"]) * 1024)


def prefill_bytes(n_tok, H, n_out, n_init=0, n_ckpt=0):
    return n_tok * H * (TOK_IN_B + TOK_OUT_B) + (n_out + n_init + n_ckpt) * H * STATE_B


def prefill_flops(n_tok, H):
    return n_tok * H * PREFILL_FLOP_TOK_HEAD


def decode_bytes(B, H):
    return B * H * (2 * STATE_B + TOK_IN_B + TOK_OUT_B)


def verify_bytes(B, P, H):
    return B * H * (STATE_B + P * (TOK_IN_B + TOK_OUT_B + RING_ENTRY_B))


def verify_direct_bytes(B, P, H):
    """Direct per-draft checkpoints: the verify's state read and token traffic plus one state
    write per position (in place of the ring entries)."""
    return B * H * (STATE_B + P * (TOK_IN_B + TOK_OUT_B) + P * STATE_B)


def commit_direct_bytes(B, H):
    return B * H * 2 * STATE_B


def commit_bytes(n_replayed_total, B, H):
    return B * H * 2 * STATE_B + n_replayed_total * H * RING_ENTRY_B


# ----------------------------------------------------------------------------- CPU baseline

_CPU_W = None   # the mixed workload as numpy arrays, set in the parent before the workers fork


def _oracle_step_on_heads(heads):
    """Worker: the CPU oracle on the whole mixed step restricted to `heads` (one thread)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import KDAPool as OPool
    w = _CPU_W
    hs = list(heads)
    npd = {n: (x[:, hs] if x.ndim == 2 else x[:, hs, :]) for n, x in w["tokens"].items()}
    o = OPool(w["n_slots"], len(hs), D, D, w["ring_cap"])
    for _ in range(w["n_slots"]):
        o.alloc()
    ds, vs, ps = w["decode_slots"], w["verify_slots"], w["prefill_slots"]
    o.state[np.concatenate([ds, vs])] = w["states"][:, hs]
    n_pre, nd, P = w["cu_seqlens"][-1], w["n_decode"], w["n_pos"]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        o.prefill({n: x[:n_pre] for n, x in npd.items()}, w["cu_seqlens"],
                  [-1] * len(ps), ps, [], 0)
        o.decode({n: x[n_pre:n_pre + nd] for n, x in npd.items()}, ds)
        o.verify({n: x[n_pre + nd:].reshape((len(vs), P) + x.shape[1:]) for n, x in npd.items()},
                 vs)
        o.commit(vs, w["n_accepted"])
        return time.perf_counter() - t0


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, max_workers: int):
    """The CPU oracle as it stands (fp64 numpy), on the whole mixed step with all heads: the
    (sequence, head) chains are independent, so the heads are split over a pool of worker
    processes, one thread each, one per host core the process may run on (at most
    max_workers). Must run before the GPU is initialised: the workers are forked, and they
    get plain numpy arrays only (torch's thread pools do not survive a fork)."""
    import multiprocessing as mp
    global _CPU_W
    _CPU_W = {**{k: w[k] for k in ("n_slots", "ring_cap", "decode_slots", "verify_slots",
                                   "prefill_slots", "cu_seqlens", "n_decode", "n_pos",
                                   "n_accepted")},
              "tokens": w["tokens"].np, "states": w["states"].double().numpy()}
    H = w["H"]
    n = max(1, min(len(os.sched_getaffinity(0)), max_workers, H))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    parts = [list(range(i, H, n)) for i in range(n)]
    with mp.get_context("fork").Pool(n) as pool:
        pool.map(_oracle_step_on_heads, [[0]] * n)          # workers up, modules imported
        t0 = time.perf_counter()
        per = pool.map(_oracle_step_on_heads, parts)
        wall = time.perf_counter() - t0
    total_tok = int(w["cu_seqlens"][-1]) + w["n_decode"] + w["n_verify"] * w["n_pos"]
    return {"value": round(total_tok / wall, 1), "unit": "tokens/s", "cores": n,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"the whole mixed step (6 prefills, {w['n_decode']} decodes, "
                      f"{w['n_verify']} verifies of 1+{w['n_pos'] - 1}, their commit) on all "
                      f"{H} heads, fp64 numpy, heads split over {n} worker processes (one "
                      f"thread each); wall {wall:.2f} s, {sum(per):.1f} s of CPU time"}


# ----------------------------------------------------------------------------- GPU timing

def _stats(ms):
    import numpy as np
    a = np.asarray(ms)
    return {"ms": round(float(np.median(a)), 5), "ms_p10": round(float(np.percentile(a, 10)), 5),
            "ms_p90": round(float(np.percentile(a, 90)), 5)}


def _bw(bytes_, ms):
    gbs = bytes_ / ms / 1e6
    return {"alg_bytes": int(bytes_), "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def _clean(ms, bytes_):
    """The clean-eviction timing of a call (see Cold): median and its algorithmic GB/s."""
    import numpy as np
    m = float(np.median(np.asarray(ms)))
    gbs = bytes_ / m / 1e6
    return {"ms_clean": round(m, 5), "GBps_clean": round(gbs, 1), "hbm_frac_clean": round(gbs / HBM_PEAK_GBS, 4)}


class TimingEvent:
    """A HIP event for timing, made through the HIP runtime torch loaded with
    hipEventDisableSystemFence: recording it performs no system-scope cache write-back and
    invalidation (which torch's timing events do, for the host's sake, and which would land in
    the timed interval: ~1.7 us on a 16-sequence decode). Same interface as torch.cuda.Event."""
    _hip = None

    def __init__(self, torch, enable_timing=True):
        import ctypes
        if TimingEvent._hip is None:
            from recurrent_linear_attention_amd import _abi
            hip = _abi.hip_runtime()
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self.torch, self._c = torch, ctypes
        self.h = ctypes.c_void_p()
        if TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h), 0x20000000) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self):
        if TimingEvent._hip.hipEventRecord(self.h, self.torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        ms = self._c.c_float()
        if TimingEvent._hip.hipEventElapsedTime(self._c.byref(ms), self.h, end.h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        hip = type(self)._hip   # not the module global, which may be gone at interpreter exit
        if hip is not None and self.h:
            hip.hipEventDestroy(self.h)


class Cold:
    """Times calls cold: before each timed call an untimed pass over 512 MiB on the same stream
    evicts the 256 MB Infinity Cache and the L2s, and an event pair brackets the call alone.
    Two evictions, which bound the call's HBM cost from both sides:
      * dirty (`ms`): a 512 MiB write. The caches are then full of dirty lines, so every line
        the call brings in or writes also writes one of them back: the call pays for its own
        writes, and for write-backs its reads cause (an over-charge of up to its read bytes);
      * clean (`ms_clean`): a 512 MiB read of a buffer nothing writes. The caches hold clean
        lines, so the call's reads cost no write-back, but its own writes may still sit in the
        caches when it ends (an under-charge of up to its write bytes)."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.scratch = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)
        self.clean_src = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
        self.scratch.fill_(0.0)   # pushes clean_src's initial writes out of the caches
        self.n = 0

    def evict(self, clean=False):
        self.n += 1
        if clean:
            self.sink = self.clean_src.sum()
        else:
            self.scratch.fill_(float(self.n))

    def time(self, iters, calls, clean=False):
        """calls: functions run in order each iteration, each timed cold. Returns per-call lists
        of event times (ms)."""
        torch = self.torch
        ev = [[(TimingEvent(torch), TimingEvent(torch))
               for _ in calls] for _ in range(iters)]
        for it in range(iters):
            for j, fn in enumerate(calls):
                self.evict(clean)
                ev[it][j][0].record()
                fn()
                ev[it][j][1].record()
        torch.cuda.synchronize()
        return [[ev[it][j][0].elapsed_time(ev[it][j][1]) for it in range(iters)] for j in range(len(calls))]

    def warm(self, iters, fn):
        torch = self.torch
        e0, e1 = TimingEvent(torch), TimingEvent(torch)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters


def measured_peaks(torch, dev):
    """What this GPU sustains on plain work, beside the published peaks: a 1 GiB device-to-device
    copy (bytes read + written per second) and a 8192^3 bf16 matmul (dense TFLOP/s), each the
    best of 5 timed repeats after a warm-up."""
    src = torch.ones(2**28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0, e1 = TimingEvent(torch), TimingEvent(torch)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return min(out)

    ms_copy = best(lambda: dst.copy_(src))
    ms_mm = best(lambda: torch.matmul(a, b))
    res = {"hbm_spec_GBps": HBM_PEAK_GBS, "mfma_fp16_spec_TFLOPs": MFMA_PEAK_TFLOPS,
           "copy_GBps": round(2 * src.numel() * 4 / ms_copy / 1e6, 1),
           "matmul_bf16_TFLOPs": round(2 * 8192**3 / ms_mm / 1e9, 1)}
    del src, dst, a, b
    return res


def bench_decode(torch, kda, ki, dev, cold, iters):
    w = ki.decode_workload(1)
    H, B = w["H"], w["B"]
    pool = kda.KDAPool(w["n_slots"], H, D, w["ring_cap"], device=dev)
    for _ in range(w["n_slots"]):
        pool.kda_slot_alloc()
    slots = kda.IndexArray(w["slots"], dev)
    pool.state[w["slots"].tolist()] = w["states"].to(dev)
    t = w["tokens"]
    q, k, v, a, b = (x.to(dev).contiguous() for x in (t.q, t.k, t.v, t.a, t.b))
    o = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    call = lambda: pool.kda_decode(q, k, v, a, b, slots, o=o)  # noqa: E731
    for _ in range(5):
        call()
    (ms,) = cold.time(iters, [call])
    (ms_c,) = cold.time(iters, [call], clean=True)
    st = _stats(ms)
    out = {"workload": f"decode: B={B} sequences x 1 token, H={H}, d={D}, pool {w['n_slots']} "
                       "slots (random permutation), fp32 state", **st,
           **_bw(decode_bytes(B, H), st["ms"]), "tokens_per_s": round(B / (st["ms"] / 1e3), 1),
           **_clean(ms_c, decode_bytes(B, H)), "ms_warm": round(cold.warm(iters, call), 5)}
    del pool
    return out


def bench_verify_commit(torch, kda, ki, dev, cold, iters):
    import numpy as np
    w = ki.verify_workload(2)
    H, B, P = w["H"], w["B"], w["n_pos"]
    pool = kda.KDAPool(w["n_slots"], H, D, w["ring_cap"], device=dev)
    for _ in range(w["n_slots"]):
        pool.kda_slot_alloc()
    slots = kda.IndexArray(w["slots"], dev)
    pool.state[w["slots"].tolist()] = w["states"].to(dev)
    t = w["tokens"]
    q, k, v, a, b = (x.to(dev).contiguous() for x in (t.q, t.k, t.v, t.a, t.b))
    o = torch.empty((B, P, H, D), dtype=torch.bfloat16, device=dev)
    na = torch.from_numpy(w["n_accepted"]).to(dev)
    ver = lambda: pool.kda_verify(q, k, v, a, b, slots, o=o)  # noqa: E731
    com = lambda: pool.kda_commit(slots, na)  # noqa: E731
    for _ in range(3):
        ver()
        com()
    ms_v, ms_c = cold.time(iters, [ver, com])
    ms_vc, ms_cc = cold.time(iters, [ver, com], clean=True)
    sv, sc = _stats(ms_v), _stats(ms_c)
    n_rep = int(np.sum(1 + w["n_accepted"]))
    out = {"workload": f"speculative verify of B={B} x 1+{P - 1} positions, then ReplaySSM commit "
                       f"of accepted counts {w['n_accepted'].tolist()} ({n_rep} positions "
                       f"replayed), H={H}, d={D}, pool {w['n_slots']} slots, ring of {w['ring_cap']}",
           "verify": {**sv, **_bw(verify_bytes(B, P, H), sv["ms"]),
                      "positions_per_s": round(B * P / (sv["ms"] / 1e3), 1),
                      **_clean(ms_vc, verify_bytes(B, P, H))},
           "commit": {**sc, **_bw(commit_bytes(n_rep, B, H), sc["ms"]),
                      **_clean(ms_cc, commit_bytes(n_rep, B, H))},
           "committed_tokens_per_s": round(n_rep / ((sv["ms"] + sc["ms"]) / 1e3), 1)}
    del pool
    return out


def bench_verify_schemes(torch, kda, ki, dev, cold, iters, batches=(4, 16, 64)):
    """ReplaySSM ring against direct per-draft checkpoints at several verify batch sizes (1+8
    positions, H = 32): per scheme the cold verify and commit times, the bytes each moves, and
    the memory each needs beside the committed state (ring entries per slot, draft states per
    verifying sequence)."""
    import numpy as np
    out = {}
    for B in batches:
        w = ki.verify_workload(20 + B, B=B, n_slots=max(256, B))
        H, P = w["H"], w["n_pos"]
        pool = kda.KDAPool(w["n_slots"], H, D, w["ring_cap"], device=dev)
        for _ in range(w["n_slots"]):
            pool.kda_slot_alloc()
        slots = kda.IndexArray(w["slots"], dev)
        pool.state[w["slots"].tolist()] = w["states"].to(dev)
        t = w["tokens"]
        q, k, v, a, b = (x.to(dev).contiguous() for x in (t.q, t.k, t.v, t.a, t.b))
        o = torch.empty((B, P, H, D), dtype=torch.bfloat16, device=dev)
        na = torch.from_numpy(w["n_accepted"]).to(dev)
        draft = pool.kda_draft_states(B, P)
        calls = [lambda: pool.kda_verify(q, k, v, a, b, slots, o=o),
                 lambda: pool.kda_commit(slots, na),
                 lambda: pool.kda_verify_direct(q, k, v, a, b, slots, draft_states=draft, o=o),
                 lambda: pool.kda_commit_direct(slots, na, draft)]
        for _ in range(2):
            for fn in calls:
                fn()
        ms = [float(np.median(x)) for x in cold.time(iters, calls)]
        n_rep = int(np.sum(1 + w["n_accepted"]))
        ring_b = verify_bytes(B, P, H) + commit_bytes(n_rep, B, H)
        direct_b = verify_direct_bytes(B, P, H) + commit_direct_bytes(B, H)
        out[f"B{B}"] = {
            "ring": {"verify_ms": round(ms[0], 5), "commit_ms": round(ms[1], 5),
                     "bytes": int(ring_b), "extra_bytes_per_slot": w["ring_cap"] * H * RING_ENTRY_B},
            "direct": {"verify_ms": round(ms[2], 5), "commit_ms": round(ms[3], 5),
                       "bytes": int(direct_b), "extra_bytes_per_sequence": P * H * STATE_B},
            "ring_over_direct_time": round((ms[0] + ms[1]) / (ms[2] + ms[3]), 3)}
        del pool, draft
    return {"workload": "verify of B x 1+8 positions and the commit of the accepted drafts, H=32, "
                        "d=128, ReplaySSM ring against direct per-draft state checkpoints", **out}


def bench_prefix_hit_and_intervals(torch, kda, ki, dev, cold, iters, aligned_ms):
    """The two prefix-cache rows beside the 8192-token prefill (H = 32): checkpoints every 1000
    tokens (not a multiple of the 64-token chunk: every interval gets chunks of its own) against
    every 1024; and a partial hit, a new 8192-token prompt whose first 6144 tokens match a cached
    prompt with checkpoints every 1024 tokens, served as the checkpoint copy into the request's
    slot, the prefill of the remaining 2048 tokens from that slot, then a verify of 1+8 drafts
    and the commit of the accepted ones on the same slot."""
    import numpy as np
    w = ki.prefill_workload(3)
    H, L = w["H"], w["cu_seqlens"][-1]
    pool = kda.KDAPool(w["n_slots"], H, D, w["ring_cap"], device=dev)
    for _ in range(w["n_slots"]):
        pool.kda_slot_alloc()
    t = w["tokens"]
    q, k, v, a, b = (x.to(dev).contiguous() for x in (t.q, t.k, t.v, t.a, t.b))
    o = torch.empty((L, H, D), dtype=torch.bfloat16, device=dev)
    cu, out = kda.IndexArray(w["cu_seqlens"], dev), kda.IndexArray([0], dev)
    # unaligned interval: 8 boundaries at 1000, 2000, ..., 8000
    I_u = 1000
    cks_u = kda.IndexArray(list(range(1, 1 + L // I_u)), dev)
    unal = lambda: pool.kda_prefill(q, k, v, a, b, cu, out, ckpt_slots=cks_u, ckpt_interval=I_u, o=o)  # noqa: E731
    # partial hit: checkpoint slot 9 holds the cached prompt's state after 6144 tokens (its
    # sixth 1024-token checkpoint); the request's slot 10 resumes from it
    hit = kda.prefix_hit(6144, L, 1024)
    cached, req = 9, 10
    pool.kda_prefill(q[:hit], k[:hit], v[:hit], a[:hit], b[:hit], kda.IndexArray([0, hit], dev),
                     kda.IndexArray([cached], dev))
    rest = L - hit
    cu_r, out_r, init_r = (kda.IndexArray([0, rest], dev), kda.IndexArray([req], dev),
                           kda.IndexArray([req], dev))
    o_r = torch.empty((rest, H, D), dtype=torch.bfloat16, device=dev)
    P = 9
    vw = ki.verify_workload(31, B=1, P=P, H=H)
    vt = vw["tokens"]
    vq, vk, vv, va, vb = (x.to(dev).contiguous() for x in (vt.q, vt.k, vt.v, vt.a, vt.b))
    vo = torch.empty((1, P, H, D), dtype=torch.bfloat16, device=dev)
    sl, na = kda.IndexArray([req], dev), torch.from_numpy(vw["n_accepted"]).to(dev)
    calls = [unal,
             lambda: pool.kda_slot_checkpoint(cached, req),
             lambda: pool.kda_prefill(q[hit:], k[hit:], v[hit:], a[hit:], b[hit:], cu_r, out_r,
                                      init_slots=init_r, o=o_r),
             lambda: pool.kda_verify(vq, vk, vv, va, vb, sl, o=vo),
             lambda: pool.kda_commit(sl, na)]
    for _ in range(2):
        for fn in calls:
            fn()
    ms = [float(np.median(x)) for x in cold.time(iters, calls)]
    served = ms[1] + ms[2] + ms[3] + ms[4]
    res = {"workload": "one 8192-token prompt, H=32, d=128: checkpoints every 1000 tokens against "
                       "every 1024; a 6144-token prefix-cache hit (checkpoint copy, prefill of the "
                       "other 2048 tokens from it, verify of 1+8 drafts and commit on the slot)",
           "unaligned_1000_ms": round(ms[0], 5), "aligned_1024_ms": aligned_ms,
           "unaligned_over_aligned": round(ms[0] / aligned_ms, 3),
           "hit": {"cached_tokens": hit, "checkpoint_copy_ms": round(ms[1], 5),
                   "prefill_rest_ms": round(ms[2], 5), "verify_ms": round(ms[3], 5),
                   "commit_ms": round(ms[4], 5), "served_ms": round(served, 5),
                   "full_prefill_ms": aligned_ms, "served_over_full": round(served / aligned_ms, 3)}}
    del pool
    return res


def bench_prefill(torch, kda, ki, dev, cold, iters):
    w = ki.prefill_workload(3)
    H, L, I = w["H"], w["cu_seqlens"][-1], w["ckpt_interval"]
    n_ck = L // I
    pool = kda.KDAPool(w["n_slots"], H, D, w["ring_cap"], device=dev)
    for _ in range(w["n_slots"]):
        pool.kda_slot_alloc()
    t = w["tokens"]
    q, k, v, a, b = (x.to(dev).contiguous() for x in (t.q, t.k, t.v, t.a, t.b))
    o = torch.empty((L, H, D), dtype=torch.bfloat16, device=dev)
    cu, out = kda.IndexArray(w["cu_seqlens"], dev), kda.IndexArray([0], dev)
    cks = kda.IndexArray(list(range(1, 1 + n_ck)), dev)
    call = lambda: pool.kda_prefill(q, k, v, a, b, cu, out, ckpt_slots=cks, ckpt_interval=I, o=o)  # noqa: E731
    for _ in range(3):
        call()
    (ms,) = cold.time(iters, [call])
    (ms_c,) = cold.time(iters, [call], clean=True)
    st = _stats(ms)
    byts, fl = prefill_bytes(L, H, n_out=1, n_ckpt=n_ck), prefill_flops(L, H)
    bw = _bw(byts, st["ms"])
    tf = fl / st["ms"] / 1e9
    res = {"workload": f"prefill: one {L}-token prompt, H={H}, d={D}, chunk {C}, state checkpoint "
                       f"every {I} tokens inside the pass ({n_ck} checkpoints) and at the end",
           **st, **bw, "tokens_per_s": round(L / (st["ms"] / 1e3), 1),
           "alg_flops": int(fl), "alg_TFLOPs": round(tf, 2), "mfma_frac": round(tf / MFMA_PEAK_TFLOPS, 4),
           # the MFMA rate this workload would reach at full HBM bandwidth (arithmetic intensity x
           # 8 TB/s) and the achieved share of it, which equals hbm_frac
           "hbm_bound_TFLOPs": round(fl / byts * HBM_PEAK_GBS / 1e3, 1),
           "frac_of_hbm_bound_ceiling": bw["hbm_frac"], **_clean(ms_c, byts),
           "ms_warm": round(cold.warm(max(iters // 2, 1), call), 5)}
    del pool
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config-iters", type=int, default=50,
                    help="cold timed calls per single-purpose workload")
    ap.add_argument("--cpu-workers", type=int, default=16)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 3 times (a known-size reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n, "repeats": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the KDA hot path shards by heads and sequences "
              "with no exchange, and this build runs on a single MI355X (--gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np

    import kda_inputs as ki

    w = ki.mixed_workload(4)
    cpu = None
    if not args.no_cpu:   # before the GPU is touched: the oracle's workers are forked
        print("bench: CPU oracle baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_workers)

    import torch

    import recurrent_linear_attention_amd as kda
    from recurrent_linear_attention_amd import IndexArray

    H, P = w["H"], w["n_pos"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pool = kda.KDAPool(w["n_slots"], H, D, w["ring_cap"], device=dev)
    for _ in range(w["n_slots"]):
        pool.kda_slot_alloc()
    ds, vs, ps = w["decode_slots"], w["verify_slots"], w["prefill_slots"]
    pool.state[np.concatenate([ds, vs]).tolist()] = w["states"].to(dev)
    tok = w["tokens"]
    q, k, v, a, b = (t.to(dev).contiguous() for t in (tok.q, tok.k, tok.v, tok.a, tok.b))
    o = torch.empty((q.shape[0], H, D), dtype=torch.bfloat16, device=dev)
    cu = IndexArray(w["cu_seqlens"], dev)
    i_ps, i_ds, i_vs = IndexArray(ps, dev), IndexArray(ds, dev), IndexArray(vs, dev)
    na = torch.from_numpy(w["n_accepted"]).to(dev)
    n_pre, nd, nv = int(w["cu_seqlens"][-1]), w["n_decode"], w["n_verify"]
    total_tok = n_pre + nd + nv * P

    # A serving step commits the previous step's verified drafts (ReplaySSM) and then verifies
    # new ones on the same slots: the batch's commit part runs ahead of its verify on the side
    # stream, next to the prefill. The first batch has no earlier verify to commit.
    pool.kda_mixed_batch(q, k, v, a, b, cu, i_ps, i_ds, i_vs, P, o=o)

    def step():
        pool.kda_mixed_batch(q, k, v, a, b, cu, i_ps, i_ds, i_vs, P, o=o, commit_slots=i_vs,
                             n_accepted=na)

    print("bench: mixed step ...", file=sys.stderr, flush=True)
    t_pw = time.perf_counter()
    for _ in range(PREWARM_STEPS):
        step()
    torch.cuda.synchronize()
    s_pre_warm = time.perf_counter() - t_pw
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = TimingEvent(torch), TimingEvent(torch)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_step_dev = e0.elapsed_time(e1) / args.steps
    pool.kda_commit(i_vs, na)   # the last verify: the pool is idle again for the second pass

    # Second timed pass: the same launches issued one by one, bracketed by events.
    sl = lambda t, lo, hi: t[lo:hi]  # noqa: E731
    dq, dk, dv, da, db, do = (sl(t, n_pre, n_pre + nd) for t in (q, k, v, a, b, o))
    vq, vk, vv, va, vb, vo = (sl(t, n_pre + nd, total_tok).reshape((nv, P) + t.shape[1:])
                              for t in (q, k, v, a, b, o))
    pq, pk, pv, pa, pb, po = (sl(t, 0, n_pre) for t in (q, k, v, a, b, o))
    # ... and the direct per-draft checkpoint pair on the same verify slots, the scheme
    # ReplaySSM is weighed against (state written at every verified position)
    names = ["prefill", "decode", "verify", "commit", "verify_direct", "commit_direct"]
    draft = pool.kda_draft_states(nv, P)
    ev = [[TimingEvent(torch) for _ in range(7)] for _ in range(args.steps)]
    for s in range(args.steps):
        E = ev[s]
        E[0].record()
        pool.kda_prefill(pq, pk, pv, pa, pb, cu, i_ps, o=po)
        E[1].record()
        pool.kda_decode(dq, dk, dv, da, db, i_ds, o=do)
        E[2].record()
        pool.kda_verify(vq, vk, vv, va, vb, i_vs, o=vo)
        E[3].record()
        pool.kda_commit(i_vs, na)
        E[4].record()
        pool.kda_verify_direct(vq, vk, vv, va, vb, i_vs, draft_states=draft, o=vo)
        E[5].record()
        pool.kda_commit_direct(i_vs, na, draft)
        E[6].record()
    torch.cuda.synchronize()
    ms = {n: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]))
          for i, n in enumerate(names)}
    n_rep = int(np.sum(1 + w["n_accepted"]))
    byts = {"prefill": prefill_bytes(n_pre, H, len(ps)), "decode": decode_bytes(nd, H),
            "verify": verify_bytes(nv, P, H), "commit": commit_bytes(n_rep, nv, H),
            "verify_direct": verify_direct_bytes(nv, P, H), "commit_direct": commit_direct_bytes(nv, H)}
    kernels = {n: {"ms": round(ms[n], 5), **_bw(byts[n], ms[n])} for n in names}
    pf = prefill_flops(n_pre, H)
    kernels["prefill"]["alg_TFLOPs"] = round(pf / ms["prefill"] / 1e9, 2)
    kernels["prefill"]["mfma_frac"] = round(pf / ms["prefill"] / 1e9 / MFMA_PEAK_TFLOPS, 4)
    pre_gbs = byts["prefill"] / ms["prefill"] / 1e6
    roofline = {"bound": "hbm", "achieved": round(pre_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(pre_gbs / HBM_PEAK_GBS, 4), "traffic": prefill_traffic_bytes(),
                "kernel": "prefill: one kda_prefill call over all sequences of the batch "
                          "(chunk_prep and state_pass kernels, back to back on one stream)",
                "alg_bytes_per_launch": byts["prefill"]}
    del pool

    configs = peaks = None
    if not args.no_configs:
        print("bench: single-purpose workloads (cold) ...", file=sys.stderr, flush=True)
        cold = Cold(torch, dev)
        configs = {"decode_b16": bench_decode(torch, kda, ki, dev, cold, args.config_iters),
                   "verify_commit_b4": bench_verify_commit(torch, kda, ki, dev, cold, args.config_iters),
                   "verify_schemes": bench_verify_schemes(torch, kda, ki, dev, cold,
                                                          max(args.config_iters // 5, 3)),
                   "prefill_8192": bench_prefill(torch, kda, ki, dev, cold, max(args.config_iters // 2, 1))}
        configs["prefix_hit_and_intervals"] = bench_prefix_hit_and_intervals(
            torch, kda, ki, dev, cold, max(args.config_iters // 5, 3), configs["prefill_8192"]["ms"])
        del cold
        peaks = measured_peaks(torch, dev)
        # each HBM-bound figure also as a share of what a plain device copy sustains
        for part in (configs["decode_b16"], configs["verify_commit_b4"]["verify"],
                     configs["verify_commit_b4"]["commit"], configs["prefill_8192"]):
            part["copy_frac"] = round(part["GBps"] / peaks["copy_GBps"], 4)
            part["copy_frac_clean"] = round(part["GBps_clean"] / peaks["copy_GBps"], 4)
        for part in kernels.values():
            part["copy_frac"] = round(part["GBps"] / peaks["copy_GBps"], 4)

    out = {"metric": METRIC, "value": round(total_tok / (ms_step / 1e3), 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "prewarm": {"steps": PREWARM_STEPS, "s": round(s_pre_warm, 3)},
           "ms_per_step": round(ms_step, 4), "ms_per_step_device": round(ms_step_dev, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
           "data": "synthetic (seeded, kda_inputs)",
           "config": {"workload": "mixed varlen batch: 6 prefills (lognormal lengths "
                                  f"{w['lengths']}) + {nd} decodes + ReplaySSM commit of the "
                                  f"previous step's {nv} verifies + {nv} verifies of 1+{P - 1}",
                      "tokens_per_step": total_tok, "heads": H, "d_k": D, "d_v": D,
                      "chunk": C, "pool_slots": w["n_slots"]},
           "roofline": roofline, "cpu_baseline": cpu, "peaks": peaks, "kernels": kernels,
           "configs": configs}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
