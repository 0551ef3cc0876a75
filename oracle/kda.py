"""CPU oracle for the KDA fixed-size recurrent-state engine (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module. The product path never does: it runs entirely in the HIP library.

What is computed
----------------
The pages ("vLLM lifts Kimi K3 throughput by up to 2.8x", section "Kimi K3 stresses the whole
stack"; "vLLM brings day-0 support to Moonshot's Kimi K3", section "Confirmed") describe Kimi
Delta Attention (KDA) as a recurrent layer whose fixed-size per-head state is updated as
tokens arrive, but they print no equation. This engine takes the gated delta rule with
per-key-channel decay as that update. For one head, with the state S a d_k x d_v matrix,
decay a_t in (0,1)^{d_k}, write strength b_t, key k_t, value v_t and query q_t:

    S_t = Diag(a_t) S_{t-1} - b_t k_t (k_t^T Diag(a_t) S_{t-1}) + b_t k_t v_t^T
    o_t = S_t^T q_t                      (read out from the updated state)

Everything here is float64, one token at a time, in exactly that order. Heads are
independent, so each function below works on any number of leading (sequence, head) axes
with numpy broadcasting; that is batching, not reordering.

The three uses the pages describe are modelled on a pool of state slots:

* prefill with checkpoint export inside the same pass ("vLLM lifts Kimi K3 throughput ...",
  section "KDA checkpoints stay inside the prefill"): the state after every ``interval``
  tokens of a prompt is copied to a cache-block slot while the prefill runs;
* single-token decode against cached per-request state ("Kimi K3 is here: efficient day-0
  support on vLLM", summary and FAQ on prefix caching over KDA state);
* speculative verify with ReplaySSM commit ("vLLM lifts Kimi K3 throughput ...", section
  "ReplaySSM shrinks rollback state"): verify leaves the committed state untouched and keeps
  the drafted inputs in a per-slot ring; commit replays the accepted prefix into the state;
  a reject only moves the ring pointer.
"""
from __future__ import annotations

import numpy as np

# Device error bits, mirrored by the library's error word.
ERR_NACC_RANGE = 1


def kda_step(S, q, k, v, a, b):
    """One token of the gated delta rule. Returns (S_t, o_t).

    Shapes: S [..., dk, dv]; q, k, a [..., dk]; v [..., dv]; b [...].
    """
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    S_dec = a[..., :, None] * S                              # Diag(a_t) S_{t-1}: scale key rows
    u = np.einsum("...ij,...i->...j", S_dec, k)              # k_t^T Diag(a_t) S_{t-1}
    S_new = S_dec + b[..., None, None] * (k[..., :, None] * (v - u)[..., None, :])
    o = np.einsum("...ij,...i->...j", S_new, q)              # S_t^T q_t
    return S_new, o


def kda_scan(S0, q, k, v, a, b, snapshot_every: int = 0):
    """Run kda_step over the token axis 0 of q, k, v, a, b.

    S0 [..., dk, dv]; q [T, ..., dk] etc.  Returns (S_T, O [T, ..., dv], snapshots), where
    ``snapshots`` holds the state after token p (1-based) for every p divisible by
    ``snapshot_every`` (empty if 0).
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    T = q.shape[0]
    O = np.zeros((T,) + S.shape[:-2] + (S.shape[-1],))
    snaps = []
    for t in range(T):
        S, O[t] = kda_step(S, q[t], k[t], v[t], a[t], b[t])
        if snapshot_every and (t + 1) % snapshot_every == 0:
            snaps.append(S.copy())
    return S, O, snaps


class KDAPool:
    """float64 model of the whole engine: state slots, ReplaySSM rings and per-slot metadata.

    Slot metadata mirrors what the library keeps on the device:
      pos        tokens folded into the slot's state;
      ring_head  ring entry where the next verify starts writing;
      pending    number of verified-but-undecided positions (0 = idle);
      v_base     ring_head at the last verify;
      v_npos     positions written by the last verify.
    Host-side bookkeeping: a slot is free or live; a live slot is idle or pending.
    Allocation returns the lowest free index.
    """

    def __init__(self, n_slots: int, H: int, dk: int, dv: int, ring_cap: int):
        self.n_slots, self.H, self.dk, self.dv, self.R = n_slots, H, dk, dv, ring_cap
        self.state = np.zeros((n_slots, H, dk, dv))
        self.ring_k = np.zeros((n_slots, ring_cap, H, dk))
        self.ring_v = np.zeros((n_slots, ring_cap, H, dv))
        self.ring_a = np.zeros((n_slots, ring_cap, H, dk))
        self.ring_b = np.zeros((n_slots, ring_cap, H))
        self.pos = np.zeros(n_slots, np.int64)
        self.ring_head = np.zeros(n_slots, np.int32)
        self.pending = np.zeros(n_slots, np.int32)
        self.v_base = np.zeros(n_slots, np.int32)
        self.v_npos = np.zeros(n_slots, np.int32)
        self.live = np.zeros(n_slots, bool)
        self.direct = np.zeros(n_slots, bool)   # pending a direct commit (not a ring commit)
        self.error_bits = 0

    # ---------------------------------------------------------------- bookkeeping
    def meta(self) -> np.ndarray:
        """[n_slots, 5] int64: pos, ring_head, pending, v_base, v_npos."""
        return np.stack([self.pos, self.ring_head, self.pending, self.v_base,
                         self.v_npos], axis=1).astype(np.int64)

    def alloc(self) -> int:
        free = np.flatnonzero(~self.live)
        if free.size == 0:
            raise LookupError("pool exhausted")
        s = int(free[0])
        self.live[s] = True
        return s

    def _check_idle(self, slots, distinct=True):
        slots = [int(s) for s in slots]
        for s in slots:
            if not (0 <= s < self.n_slots) or not self.live[s]:
                raise ValueError(f"slot {s} is not live")
            if self.pending[s]:
                raise RuntimeError(f"slot {s} has a pending verify")
        if distinct and len(set(slots)) != len(slots):
            raise ValueError("slots repeat within one call")
        return slots

    def _check_pending(self, slots, direct=None):
        """direct: None accepts either kind of pending verify, else the kind it must be."""
        slots = [int(s) for s in slots]
        for s in slots:
            if not (0 <= s < self.n_slots) or not self.live[s]:
                raise ValueError(f"slot {s} is not live")
            if not self.pending[s]:
                raise RuntimeError(f"slot {s} has no pending verify")
            if direct is not None and bool(self.direct[s]) != direct:
                raise RuntimeError(f"slot {s} is pending the other kind of commit")
        if len(set(slots)) != len(slots):
            raise ValueError("slots repeat within one call")
        return slots

    def free(self, s: int):
        self._check_idle([s])
        self.live[s] = False

    def _clear_meta(self, s, pos=0):
        self.pos[s] = pos
        self.ring_head[s] = self.pending[s] = self.v_base[s] = self.v_npos[s] = 0

    def reset(self, s: int):
        """Zero a live idle slot's state and metadata."""
        self._check_idle([s])
        self.state[s] = 0.0
        self._clear_meta(s)

    def checkpoint(self, src: int, dst: int):
        """Copy a live state to another live slot (prefix-cache block export outside prefill)."""
        self._check_idle([src, dst])
        self.state[dst] = self.state[src]
        self._clear_meta(dst, self.pos[src])

    # ---------------------------------------------------------------- the three uses
    def prefill(self, tok: dict, cu_seqlens, init_slot, out_slot, ckpt_slot, interval: int):
        """Packed varlen prefill.

        tok: float64 arrays q, k, a [N, H, dk], v [N, H, dv], b [N, H].
        Sequence i covers tokens cu_seqlens[i]:cu_seqlens[i+1]; it starts from the state of
        init_slot[i] (-1 = zeros), writes its final state to out_slot[i] and, when
        interval > 0, the state after every ``interval`` of its tokens to the next entry of
        ``ckpt_slot`` (floor(len_i / interval) entries per sequence, concatenated).
        Returns O [N, H, dv].
        """
        N = int(cu_seqlens[-1])
        O = np.zeros((N, self.H, self.dv))
        ck = 0
        for i in range(len(cu_seqlens) - 1):
            lo, hi = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
            if init_slot[i] >= 0:
                S0, p0 = self.state[init_slot[i]].copy(), int(self.pos[init_slot[i]])
            else:
                S0, p0 = np.zeros((self.H, self.dk, self.dv)), 0
            S, O[lo:hi], snaps = kda_scan(S0, tok["q"][lo:hi], tok["k"][lo:hi],
                                          tok["v"][lo:hi], tok["a"][lo:hi],
                                          tok["b"][lo:hi], interval)
            for m, snap in enumerate(snaps):
                dst = int(ckpt_slot[ck])
                ck += 1
                self.state[dst] = snap
                self._clear_meta(dst, p0 + (m + 1) * interval)
            self.state[out_slot[i]] = S
            self._clear_meta(out_slot[i], p0 + (hi - lo))
        return O

    def decode(self, tok: dict, slots):
        """One token per sequence: tok arrays [B, H, ...]. Returns o [B, H, dv]."""
        slots = self._check_idle(slots)
        S, o = kda_step(self.state[slots], tok["q"], tok["k"], tok["v"], tok["a"], tok["b"])
        self.state[slots] = S
        self.pos[slots] += 1
        return o

    def verify(self, tok: dict, slots):
        """Verify P = 1+T positions per sequence: tok arrays [B, P, H, ...].

        Steps a copy of the committed state through all P positions, returns o [B, P, H, dv],
        writes the P inputs into the slot's ring from ring_head on, and marks the slot pending.
        The committed state is not written.
        """
        slots = self._check_idle(slots)
        P = tok["q"].shape[1]
        if not 1 <= P <= self.R:
            raise ValueError("positions exceed ring capacity")
        S = self.state[slots].copy()
        O = np.zeros((len(slots), P, self.H, self.dv))
        for j in range(P):
            S, O[:, j] = kda_step(S, tok["q"][:, j], tok["k"][:, j], tok["v"][:, j],
                                  tok["a"][:, j], tok["b"][:, j])
        for n, s in enumerate(slots):
            for j in range(P):
                e = (self.ring_head[s] + j) % self.R
                self.ring_k[s, e] = tok["k"][n, j]
                self.ring_v[s, e] = tok["v"][n, j]
                self.ring_a[s, e] = tok["a"][n, j]
                self.ring_b[s, e] = tok["b"][n, j]
            self.v_base[s] = self.ring_head[s]
            self.v_npos[s] = P
            self.pending[s] = P
        return O

    def commit(self, slots, n_accepted):
        """ReplaySSM commit: replay ring entries v_base .. v_base + n_acc (1 + n_acc positions,
        position 0 being the token sampled at the previous step) into the slot's state, then
        advance ring_head past them. An n_acc outside [0, v_npos - 1] sets ERR_NACC_RANGE and
        is clamped into that range."""
        slots = self._check_pending(slots, direct=False)
        for s, na in zip(slots, n_accepted):
            na = int(na)
            if na < 0 or na > self.v_npos[s] - 1:
                self.error_bits |= ERR_NACC_RANGE
                na = min(max(na, 0), int(self.v_npos[s]) - 1)
            n = 1 + na
            S = self.state[s]
            for j in range(n):
                e = (self.v_base[s] + j) % self.R
                S, _ = kda_step(S, np.zeros(self.dk), self.ring_k[s, e], self.ring_v[s, e],
                                self.ring_a[s, e], self.ring_b[s, e])
            self.state[s] = S
            self.ring_head[s] = (self.v_base[s] + n) % self.R
            self.pos[s] += n
            self.pending[s] = 0

    def rollback(self, slots):
        """Reject every drafted position: only the pending mark is cleared; the state, the
        ring pointer and pos are untouched."""
        slots = self._check_pending(slots)
        for s in slots:
            self.pending[s] = 0
            self.direct[s] = False

    # ------------------------------------------- direct per-draft state checkpoints
    # The scheme the ReplaySSM section weighs the ring against ("vLLM lifts Kimi K3 throughput
    # by up to 2.8x", section "ReplaySSM shrinks rollback state"): verify saves the state at
    # every drafted position, and commit keeps the accepted one.
    def verify_direct(self, tok: dict, slots):
        """Like verify, but returns the state after each position instead of writing the ring:
        (o [B, P, H, dv], states [B, P, H, dk, dv]). The ring is untouched; the slot is marked
        pending a direct commit (v_base = ring_head, v_npos = pending = P)."""
        slots = self._check_idle(slots)
        P = tok["q"].shape[1]
        if not 1 <= P <= self.R:
            raise ValueError("positions exceed ring capacity")
        S = self.state[slots].copy()
        O = np.zeros((len(slots), P, self.H, self.dv))
        states = np.zeros((len(slots), P, self.H, self.dk, self.dv))
        for j in range(P):
            S, O[:, j] = kda_step(S, tok["q"][:, j], tok["k"][:, j], tok["v"][:, j],
                                  tok["a"][:, j], tok["b"][:, j])
            states[:, j] = S
        for s in slots:
            self.v_base[s] = self.ring_head[s]
            self.v_npos[s] = P
            self.pending[s] = P
            self.direct[s] = True
        return O, states

    def commit_direct(self, slots, n_accepted, states):
        """Keep the state after 1 + n_acc positions (states from verify_direct, same slot
        order): pos += 1 + n_acc, pending = 0, ring_head unchanged. n_acc outside
        [0, v_npos - 1] sets ERR_NACC_RANGE and is clamped, as in commit."""
        slots = self._check_pending(slots, direct=True)
        for n, (s, na) in enumerate(zip(slots, n_accepted)):
            na = int(na)
            if na < 0 or na > self.v_npos[s] - 1:
                self.error_bits |= ERR_NACC_RANGE
                na = min(max(na, 0), int(self.v_npos[s]) - 1)
            self.state[s] = states[n, na]
            self.pos[s] += 1 + na
            self.pending[s] = 0
            self.direct[s] = False
