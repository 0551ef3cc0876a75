"""Seeded synthetic inputs for the KDA engine and its CPU oracle.

This module only draws random numbers and rounds them to their storage types. It holds
none of the KDA arithmetic, so the HIP path and the oracle can both take their inputs from
it without sharing any of the method's code.

Distributions (one recipe for every workload):

* q, k ~ N(0, 1), then l2-normalised per (token, head) over the key dimension in float64,
  then rounded to bfloat16 (round-to-nearest-even);
* v ~ N(0, 1), rounded to bfloat16;
* a = sigmoid(N(2, 1)) per (token, head, key channel), float32 -- the per-key-channel decay;
* b = sigmoid(N(0, 1)) per (token, head), float32 -- the delta-rule write strength;
* slot states that a workload needs pre-filled ~ N(0, 1), float32.

Every workload seeds ``numpy.random.default_rng(seed)`` once and draws in a fixed order:
q, k, v, a, b, initial states, slot permutation, accepted-draft counts.

The returned arrays are torch CPU tensors in storage dtype (bf16 / fp32 / int32) plus
float64 numpy copies of exactly the same values for the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "Tokens", "draw_tokens", "draw_states", "lognormal_prefill_lengths",
    "tiny_workload", "decode_workload", "verify_workload", "prefill_workload",
    "mixed_workload", "to_bf16",
]


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """Round float64/float32 values to bfloat16 (RNE) and return a CPU bf16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


@dataclass
class Tokens:
    """Per-token inputs, leading dims ``lead`` (e.g. [N] or [B, P]) then [H, d]."""
    q: torch.Tensor          # bf16 [..., H, dk]
    k: torch.Tensor          # bf16 [..., H, dk]
    v: torch.Tensor          # bf16 [..., H, dv]
    a: torch.Tensor          # fp32 [..., H, dk]
    b: torch.Tensor          # fp32 [..., H]
    np: dict = field(default_factory=dict)   # float64 copies: q, k, v, a, b

    def slice(self, lo: int, hi: int) -> "Tokens":
        t = Tokens(self.q[lo:hi], self.k[lo:hi], self.v[lo:hi], self.a[lo:hi], self.b[lo:hi])
        t.np = {n: arr[lo:hi] for n, arr in self.np.items()}
        return t


def draw_tokens(rng: np.random.Generator, lead: tuple, H: int, dk: int, dv: int) -> Tokens:
    """Draw q, k, v, a, b in that order for ``lead + (H,)`` (token, head) positions."""
    shp = tuple(lead) + (H,)
    q = rng.standard_normal(shp + (dk,))
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True))
    k = rng.standard_normal(shp + (dk,))
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    v = rng.standard_normal(shp + (dv,))
    a = _sigmoid(rng.normal(2.0, 1.0, size=shp + (dk,))).astype(np.float32)
    b = _sigmoid(rng.normal(0.0, 1.0, size=shp)).astype(np.float32)
    t = Tokens(to_bf16(q), to_bf16(k), to_bf16(v), torch.from_numpy(a), torch.from_numpy(b))
    t.np = {"q": _f64(t.q), "k": _f64(t.k), "v": _f64(t.v),
            "a": a.astype(np.float64), "b": b.astype(np.float64)}
    return t


def draw_states(rng: np.random.Generator, n: int, H: int, dk: int, dv: int) -> torch.Tensor:
    """n slot states ~ N(0, 1) in float32, shape [n, H, dk, dv]."""
    return torch.from_numpy(rng.standard_normal((n, H, dk, dv)).astype(np.float32))


def lognormal_prefill_lengths(rng: np.random.Generator, n: int, total: int,
                              mu: float = 7.5, sigma: float = 1.0,
                              lo: int = 256, hi: int = 16384) -> list[int]:
    """Prompt lengths ~ lognormal(mu, sigma), clipped to [lo, hi], rescaled to sum to ``total``.

    Rescaling uses largest-remainder rounding and re-clips at ``lo`` so the packed batch
    fills an exact token budget.
    """
    raw = np.clip(np.rint(rng.lognormal(mu, sigma, size=n)), lo, hi)
    for _ in range(8):
        scaled = raw * (total / raw.sum())
        base = np.floor(scaled).astype(np.int64)
        rem = total - int(base.sum())
        order = np.argsort(-(scaled - base), kind="stable")
        base[order[:rem]] += 1
        if base.min() >= lo:
            return [int(x) for x in base]
        raw = np.maximum(base, lo).astype(np.float64)
    raise ValueError("cannot fit lengths into the token budget")


# --------------------------------------------------------------------------------------
# Workloads.  Each returns a plain dict so that tests, the benchmark and the smoke check
# all drive the library and the oracle with identical arrays.
# --------------------------------------------------------------------------------------

def tiny_workload(seed: int = 0) -> dict:
    """B=1, H=2, d=16: 64-token prefill (chunk 16, checkpoint every 16), then verify 1+4
    drafts with 2 accepted and commit; pool of 8 slots."""
    rng = np.random.default_rng(seed)
    H, d, T, P = 2, 16, 64, 5
    pre = draw_tokens(rng, (T,), H, d, d)
    ver = draw_tokens(rng, (1, P), H, d, d)
    return dict(H=H, dk=d, dv=d, n_slots=8, ring_cap=9, chunk=16, ckpt_interval=16,
                prefill=pre, cu_seqlens=[0, T], verify=ver, n_pos=P, n_accepted=[2])


def decode_workload(seed: int = 1, B: int = 16, H: int = 32, d: int = 128,
                    n_slots: int = 256) -> dict:
    """B single-token decodes against a pool of n_slots states, slots by random permutation."""
    rng = np.random.default_rng(seed)
    tok = draw_tokens(rng, (B,), H, d, d)
    states = draw_states(rng, B, H, d, d)
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    return dict(H=H, dk=d, dv=d, n_slots=n_slots, ring_cap=9, B=B, tokens=tok,
                states=states, slots=slots)


def verify_workload(seed: int = 2, B: int = 4, P: int = 9, H: int = 32, d: int = 128,
                    n_slots: int = 256) -> dict:
    """B sequences verify 1+T = P positions each; accepted drafts ~ U{0..P-1}."""
    rng = np.random.default_rng(seed)
    tok = draw_tokens(rng, (B, P), H, d, d)
    states = draw_states(rng, B, H, d, d)
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    n_acc = rng.integers(0, P, size=B).astype(np.int32)
    return dict(H=H, dk=d, dv=d, n_slots=n_slots, ring_cap=max(9, P), B=B, n_pos=P,
                tokens=tok, states=states, slots=slots, n_accepted=n_acc)


def prefill_workload(seed: int = 3, lengths=(8192,), H: int = 32, d: int = 128,
                     chunk: int = 64, ckpt_interval: int = 1024, n_slots: int = 64,
                     init_states: bool = False) -> dict:
    """Packed varlen prefill; checkpoints every ckpt_interval tokens (0 = none)."""
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    tok = draw_tokens(rng, (int(cu[-1]),), H, d, d)
    states = draw_states(rng, len(lengths), H, d, d) if init_states else None
    return dict(H=H, dk=d, dv=d, n_slots=n_slots, ring_cap=9, chunk=chunk,
                ckpt_interval=ckpt_interval, tokens=tok, cu_seqlens=[int(x) for x in cu],
                init_states=states)


def mixed_workload(seed: int = 4, n_prefill: int = 6, n_decode: int = 32, n_verify: int = 4,
                   P: int = 9, total: int = 16384, H: int = 32, d: int = 128,
                   n_slots: int = 512, chunk: int = 64) -> dict:
    """One packed batch: [prefill tokens | decode tokens | verify tokens], ``total`` tokens."""
    rng = np.random.default_rng(seed)
    n_pre_tok = total - n_decode - n_verify * P
    # lengths come from their own generator so that the token draws keep the fixed order
    lengths = lognormal_prefill_lengths(np.random.default_rng(seed + 1000), n_prefill, n_pre_tok)
    tok = draw_tokens(rng, (total,), H, d, d)
    states = draw_states(rng, n_decode + n_verify, H, d, d)
    perm = rng.permutation(n_slots).astype(np.int32)
    n_acc = rng.integers(0, P, size=n_verify).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return dict(H=H, dk=d, dv=d, n_slots=n_slots, ring_cap=max(9, P), chunk=chunk,
                ckpt_interval=0, tokens=tok, lengths=lengths,
                cu_seqlens=[int(x) for x in cu], n_prefill=n_prefill, n_decode=n_decode,
                n_verify=n_verify, n_pos=P, states=states,
                prefill_slots=perm[:n_prefill],
                decode_slots=perm[n_prefill:n_prefill + n_decode],
                verify_slots=perm[n_prefill + n_decode:n_prefill + n_decode + n_verify],
                n_accepted=n_acc)
