"""Benchmark: one serving step of the KDA engine on the mixed 16384-token batch.

A step is the whole hot path over one packed batch -- 6 chunked prefills (lognormal lengths,
16316 tokens), 32 single-token decodes, the ReplaySSM commit of the 4 sequences verified in the
previous step and 4 speculative verifies of 1+8 positions on them, all issued by one
kda_mixed_batch call -- on H=32 heads
(one GPU's share), d_k = d_v = 128, a pool of 512 fp32 state slots. Inputs are synthetic and
seeded (kda_inputs.mixed_workload) and resident in HBM before timing starts.

Prints one JSON line. `value` = tokens per second of the whole step (16384 / step time).
`roofline` describes the dominant part, the chunked prefill (one kda_prefill call: its
chunk_prep and state_pass kernels), timed with HIP events on the stream the library launches
on, in a second timed pass that issues the same calls one by one. `cpu_baseline` times the CPU
oracle on a bounded sample (a subset of heads).

    python bench.py [--gpus 1] [--steps 100] [--warmup 30]

The warm-up steps bring the GPU to its steady clock (the first few dozen steps after start run
~5% slower); the timed steps then measure the steady serving rate.
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

# Algorithmic bytes (d = 128, fp32 state, bf16 q/k/v/o, fp32 a and b).
D = 128
STATE_B = D * D * 4
TOK_IN_B = 3 * D * 2 + D * 4 + 4            # q, k, v bf16 + a fp32 + b fp32
TOK_OUT_B = D * 2                           # o bf16
RING_ENTRY_B = 2 * D * 2 + D * 4 + 4        # k, v bf16 + a fp32 + b fp32


# HBM traffic of one prefill call of the mixed step (its two kernels: chunk_prep, which plans a
# batch of this size itself, and state_pass), from rocprofv3 counter passes (FETCH_SIZE and WRITE_SIZE, KiB per dispatch)
# scaled by the counters' reading for a 1 GiB device copy (FETCH_SIZE reads half the copied
# bytes, WRITE_SIZE all of them: factors 2.0 and 1.0). Valid only for the kernel source it was
# measured on (first 16 hex digits of its SHA-256); for any other source the bench reports
# traffic as null.
PREFILL_TRAFFIC = {"source_sha256_16": "4d34be1df2b4e43e", "fetch_scale": 2.0, "write_scale": 1.0,
                   "fetch_kib": {"chunk_prep_kernel": 269326, "state_pass_kernel": 316202},
                   "write_kib": {"chunk_prep_kernel": 501492, "state_pass_kernel": 142817}}


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


def prefill_flops(n_tok, H, C=64):
    # chunked form, triangle-exact: three d x d state contractions per token (K~S, Q~S,
    # Kbar^T W), four C x C x d triangular products per chunk, the triangular solve.
    return n_tok * H * (6 * D * D + 4 * D * C + C * C / 3)


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


def cpu_baseline(w, heads: int):
    """The CPU oracle as it stands, on the same workload restricted to `heads` heads."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import KDAPool as OPool
    H = w["H"]
    hs = list(range(heads))
    tok = w["tokens"]

    def sub(x):
        return x[:, hs] if x.ndim == 2 else x[:, hs, :]

    npd = {n: sub(x) for n, x in tok.np.items()}
    o = OPool(w["n_slots"], heads, D, D, w["ring_cap"])
    for _ in range(w["n_slots"]):
        o.alloc()
    ds, vs, ps = w["decode_slots"], w["verify_slots"], w["prefill_slots"]
    st = w["states"].double().numpy()[:, hs]
    o.state[np.concatenate([ds, vs])] = st
    n_pre, nd, P = w["cu_seqlens"][-1], w["n_decode"], w["n_pos"]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        o.prefill({n: x[:n_pre] for n, x in npd.items()}, w["cu_seqlens"],
                  [-1] * len(ps), ps, [], 0)
        o.decode({n: x[n_pre:n_pre + nd] for n, x in npd.items()}, ds)
        o.verify({n: x[n_pre + nd:].reshape((len(vs), P) + x.shape[1:]) for n, x in npd.items()},
                 vs)
        o.commit(vs, w["n_accepted"])
        dt = time.perf_counter() - t0
    total_tok = int(w["cu_seqlens"][-1]) + nd + len(vs) * P
    return {"value": total_tok * heads / H / dt, "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"the whole mixed step (prefill, decode, verify, commit) on {heads} of "
                      f"{H} heads, fp64 numpy, one thread; {dt:.1f} s of CPU time, scaled "
                      f"to all {H} heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--no-cpu", action="store_true")
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
    import torch

    import kda_inputs as ki
    import recurrent_linear_attention_amd as kda
    from recurrent_linear_attention_amd import IndexArray

    w = ki.mixed_workload(4)
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
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
    kernels = {n: {"ms": round(ms[n], 5), "alg_bytes": byts[n],
                   "GBps": round(byts[n] / ms[n] / 1e6, 1),
                   "hbm_frac": round(byts[n] / ms[n] / 1e6 / HBM_PEAK_GBS, 4)} for n in names}
    pf = prefill_flops(n_pre, H)
    kernels["prefill"]["alg_TFLOPs"] = round(pf / ms["prefill"] / 1e9, 2)
    kernels["prefill"]["mfma_frac"] = round(pf / ms["prefill"] / 1e9 / MFMA_PEAK_TFLOPS, 4)
    pre_gbs = byts["prefill"] / ms["prefill"] / 1e6
    roofline = {"bound": "hbm", "achieved": round(pre_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(pre_gbs / HBM_PEAK_GBS, 4), "traffic": prefill_traffic_bytes(),
                "kernel": "prefill: one kda_prefill call over all sequences of the batch "
                          "(chunk_prep and state_pass kernels, back to back on one stream)",
                "alg_bytes_per_launch": byts["prefill"]}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_heads)

    out = {"metric": METRIC, "value": round(total_tok / (ms_step / 1e3), 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_step, 4), "ms_per_step_device": round(ms_step_dev, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded, kda_inputs.mixed_workload)",
           "config": {"workload": "mixed varlen batch: 6 prefills (lognormal lengths "
                                  f"{w['lengths']}) + {nd} decodes + ReplaySSM commit of the "
                                  f"previous step's {nv} verifies + {nv} verifies of 1+{P - 1}",
                      "tokens_per_step": total_tok, "heads": H, "d_k": D, "d_v": D,
                      "chunk": 64, "pool_slots": w["n_slots"]},
           "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
