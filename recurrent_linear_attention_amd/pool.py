"""Python binding of the KDA C ABI: the same entry points, taking torch tensors.

Argument marshalling only -- torch provides device memory, streams and events, the library
(``lib/libkda.so``) does all the work. Index arrays given as plain sequences are copied to the
device on torch's current stream, so calls should run on that stream. ``KDAPool`` owns the
caller-side device buffers (state, ReplaySSM ring, metadata, the prefill workspace), the side
stream and events of mixed batches, and the library's pool handle.
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_int32, c_size_t, c_uint32, c_void_p

import numpy as np
import torch

from . import _abi
from ._abi import check, lib

__all__ = ["KDAPool", "IndexArray", "chunk_for"]


def chunk_for(d: int) -> int:
    """The prefill chunk this build instantiates for head dim d."""
    return 16 if d == 16 else 64


def prefix_hit(match_len: int, prompt_len: int, interval: int) -> int:
    """Partial prefix-cache hit over KDA state checkpoints ("Kimi K3 is here: efficient day-0
    support on vLLM", FAQ on prefix caching; "vLLM lifts Kimi K3 throughput by up to 2.8x",
    section "KDA checkpoints stay inside the prefill"): a cached prompt left a state checkpoint
    after every `interval` tokens, and a new prompt shares its first `match_len` tokens. The
    state can resume from the deepest checkpoint inside the shared prefix, but at least one
    prompt token is always prefilled so the step still produces the last prompt token's output.
    Returns the number of prompt tokens the reused checkpoint covers (0: a miss); that
    checkpoint is the (returned // interval - 1)-th of the cached prompt's."""
    if interval <= 0 or prompt_len <= 0:
        return 0
    usable = min(max(match_len, 0), prompt_len - 1)
    return usable // interval * interval


def _stream(stream=None) -> c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return c_void_p(s.cuda_stream)


def _check_draft(t: torch.Tensor, B: int, n_pos: int, H: int, d: int) -> None:
    if (t.dtype != torch.float32 or not t.is_contiguous() or t.device.type != "cuda"
            or tuple(t.shape) != (B, n_pos, H, d, d)):
        raise ValueError(f"draft_states must be a contiguous float32 device tensor of shape "
                         f"{(B, n_pos, H, d, d)}")


def _dev(t: torch.Tensor | None, dtype, name: str) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _ix(values, device) -> "IndexArray":
    return values if isinstance(values, IndexArray) else IndexArray(values, device)


class IndexArray:
    """An int32 index array held twice, as the ABI wants it: a host copy (validation and
    bookkeeping) and a device copy (read by the kernels). Build once and reuse it to keep
    host-to-device copies out of a timed loop."""

    def __init__(self, values, device):
        self.np = np.ascontiguousarray(np.asarray(values, dtype=np.int32).reshape(-1))
        self.dev = torch.from_numpy(self.np).to(device, non_blocking=False)

    def __len__(self):
        return int(self.np.size)

    @property
    def h(self):
        return self.np.ctypes.data if self.np.size else None

    @property
    def d(self):
        return self.dev.data_ptr() if self.np.size else None


class _StreamEvent:
    """A HIP event for ordering streams of one device: created through the HIP runtime torch
    loaded (the one libkda.so binds to) with hipEventDisableTiming | hipEventDisableSystemFence,
    destroyed with its owner."""
    _hip = None
    FLAGS = 0x2 | 0x20000000

    def __init__(self):
        if _StreamEvent._hip is None:
            hip = _abi.hip_runtime()
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(c_void_p), ctypes.c_uint]
            hip.hipEventCreateWithFlags.restype = ctypes.c_int
            hip.hipEventDestroy.argtypes = [c_void_p]
            hip.hipEventDestroy.restype = ctypes.c_int
            _StreamEvent._hip = hip
        h = c_void_p()
        err = _StreamEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), self.FLAGS)
        if err != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({err})")
        self.handle = h.value

    def __del__(self):
        hip = type(self)._hip   # not the module global, which may be gone at interpreter exit
        if getattr(self, "handle", None) and hip is not None:
            hip.hipEventDestroy(self.handle)
            self.handle = None


class KDAPool:
    """A pool of fp32 KDA state slots with per-slot ReplaySSM rings, on one GPU."""

    def __init__(self, num_slots: int, num_heads: int, d: int, ring_cap: int = 9,
                 device: str | torch.device = "cuda"):
        self.device = torch.device(device)
        self.desc = _abi.kda_pool_desc(num_slots, num_heads, d, d, ring_cap)
        self.num_slots, self.H, self.d, self.R = num_slots, num_heads, d, ring_cap
        sb = lib.kda_state_bytes(byref(self.desc))
        if sb == 0:
            raise ValueError(f"unsupported pool geometry (d={d})")
        self.state = torch.zeros((num_slots, num_heads, d, d), dtype=torch.float32,
                                 device=self.device)
        self.ring = torch.zeros(lib.kda_ring_bytes(byref(self.desc)), dtype=torch.uint8,
                                device=self.device)
        self.meta = torch.zeros(lib.kda_meta_bytes(byref(self.desc)), dtype=torch.uint8,
                                device=self.device)
        h = c_void_p()
        check(lib.kda_pool_create(byref(self.desc), self.state.data_ptr(), self.ring.data_ptr(),
                                  self.meta.data_ptr(), byref(h)), "kda_pool_create")
        self.handle = h
        off = (c_size_t * 4)()
        check(lib.kda_ring_layout(byref(self.desc), off), "kda_ring_layout")
        self.ring_offsets = list(off)
        self.err_offset = lib.kda_meta_error_offset(byref(self.desc))
        self._ws = None     # prefill workspace (torch allocation, grown on demand)
        self._side = None   # side stream + fork / join events of mixed batches (created on first use)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            lib.kda_pool_destroy(h)
            self.handle = None

    # ------------------------------------------------------------------ slots
    def kda_slot_alloc(self) -> int:
        s = c_int32()
        check(lib.kda_slot_alloc(self.handle, byref(s)), "kda_slot_alloc")
        return s.value

    def kda_slot_free(self, slot: int) -> None:
        check(lib.kda_slot_free(self.handle, slot), "kda_slot_free")

    def kda_slot_reset(self, slot: int, stream=None) -> None:
        check(lib.kda_slot_reset(self.handle, slot, _stream(stream)), "kda_slot_reset")

    def kda_slot_checkpoint(self, src: int, dst: int, stream=None) -> None:
        check(lib.kda_slot_checkpoint(self.handle, src, dst, _stream(stream)),
              "kda_slot_checkpoint")

    def host_state(self, slot: int) -> int:
        return lib.kda_slot_host_state(self.handle, slot)

    # ------------------------------------------------------------------ helpers
    def _tok_ptrs(self, q, k, v, a, b, o):
        return (_dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"),
                _dev(v, torch.bfloat16, "v"), _dev(a, torch.float32, "a"),
                _dev(b, torch.float32, "b"), _dev(o, torch.bfloat16, "o"))

    def _workspace(self, n_tok: int, n_seq: int, chunk: int, interval: int):
        """Device workspace for a prefill of this size from torch's allocator, kept and grown
        per pool (the library then allocates nothing). Returns (pointer, bytes)."""
        need = lib.kda_prefill_workspace_bytes(self.handle, n_tok, n_seq, chunk, max(interval, 0))
        if need == 0:
            return None, 0
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws.data_ptr(), self._ws.numel()

    def _prefill_struct(self, n_tok, cu, init, out, ckpt, chunk, interval, ptrs):
        args = _abi.kda_prefill_args(*ptrs)
        args.n_seq = cu.np.size - 1
        args.n_tok = n_tok
        args.chunk = chunk
        args.ckpt_interval = interval
        args.workspace, args.workspace_bytes = self._workspace(n_tok, args.n_seq, chunk, interval)
        args.h_cu_seqlens, args.d_cu_seqlens = cu.h, cu.d
        if init is not None:
            args.h_init_slot, args.d_init_slot = init.h, init.d
        args.h_out_slot, args.d_out_slot = out.h, out.d
        if ckpt is not None:
            args.h_ckpt_slot, args.d_ckpt_slot = ckpt.h, ckpt.d
        return args

    # ------------------------------------------------------------------ the three uses
    def kda_prefill(self, q, k, v, a, b, cu_seqlens, out_slots, init_slots=None,
                    ckpt_slots=None, ckpt_interval: int = 0, chunk: int | None = None,
                    o=None, stream=None) -> torch.Tensor:
        """Packed varlen prefill; q, k, a [N, H, d], v [N, H, d], b [N, H]. Returns o."""
        n_tok = q.shape[0]
        if o is None:
            o = torch.empty((n_tok, self.H, self.d), dtype=torch.bfloat16, device=q.device)
        cu = _ix(cu_seqlens, self.device)
        out = _ix(out_slots, self.device)
        init = None if init_slots is None else _ix(init_slots, self.device)
        ckpt = None if ckpt_slots is None or len(ckpt_slots) == 0 else _ix(ckpt_slots, self.device)
        args = self._prefill_struct(n_tok, cu, init, out, ckpt,
                                    chunk or chunk_for(self.d), ckpt_interval,
                                    self._tok_ptrs(q, k, v, a, b, o))
        check(lib.kda_prefill(self.handle, byref(args), _stream(stream)), "kda_prefill")
        return o

    def kda_prefill_noalloc(self, q, k, v, a, b, cu_seqlens, out_slots, o, init_slots=None,
                            ckpt_slots=None, ckpt_interval: int = 0, stream=None) -> torch.Tensor:
        """kda_prefill with the library's scratch as workspace (kda_prefill_noalloc): nothing is
        allocated for the call. o and, to keep the call free of allocations, IndexArray
        arguments are the caller's."""
        n_tok = q.shape[0]
        cu = _ix(cu_seqlens, self.device)
        out = _ix(out_slots, self.device)
        init = None if init_slots is None else _ix(init_slots, self.device)
        ckpt = None if ckpt_slots is None or len(ckpt_slots) == 0 else _ix(ckpt_slots, self.device)
        args = _abi.kda_prefill_args(*self._tok_ptrs(q, k, v, a, b, o))
        args.n_seq, args.n_tok = cu.np.size - 1, n_tok
        args.chunk, args.ckpt_interval = chunk_for(self.d), ckpt_interval
        args.h_cu_seqlens, args.d_cu_seqlens = cu.h, cu.d
        if init is not None:
            args.h_init_slot, args.d_init_slot = init.h, init.d
        args.h_out_slot, args.d_out_slot = out.h, out.d
        if ckpt is not None:
            args.h_ckpt_slot, args.d_ckpt_slot = ckpt.h, ckpt.d
        check(lib.kda_prefill_noalloc(self.handle, byref(args), _stream(stream)), "kda_prefill_noalloc")
        return o

    def _step_args(self, q, k, v, a, b, o, slots):
        s = _ix(slots, self.device)
        args = _abi.kda_step_args(*self._tok_ptrs(q, k, v, a, b, o))
        args.B = s.np.size
        args.h_slots, args.d_slots = s.h, s.d
        return args, s

    def kda_decode(self, q, k, v, a, b, slots, o=None, stream=None) -> torch.Tensor:
        """One token per sequence: q, k, a, v [B, H, d], b [B, H]. Returns o [B, H, d]."""
        if o is None:
            o = torch.empty(q.shape[:-1] + (self.d,), dtype=torch.bfloat16, device=q.device)
        args, keep = self._step_args(q, k, v, a, b, o, slots)
        check(lib.kda_decode(self.handle, byref(args), _stream(stream)), "kda_decode")
        return o

    def kda_verify(self, q, k, v, a, b, slots, o=None, stream=None) -> torch.Tensor:
        """Verify P positions per sequence: q, k, a, v [B, P, H, d], b [B, P, H]."""
        n_pos = q.shape[1]
        if o is None:
            o = torch.empty(q.shape[:-1] + (self.d,), dtype=torch.bfloat16, device=q.device)
        args, keep = self._step_args(q, k, v, a, b, o, slots)
        check(lib.kda_verify(self.handle, byref(args), n_pos, _stream(stream)), "kda_verify")
        return o

    def kda_commit(self, slots, n_accepted: torch.Tensor, stream=None) -> None:
        """n_accepted: device int32 [B] (accepted drafts per sequence)."""
        s = _ix(slots, self.device)
        na = _dev(n_accepted, torch.int32, "n_accepted")
        check(lib.kda_commit(self.handle, s.np.size, s.h, s.d, na, _stream(stream)),
              "kda_commit")

    def kda_draft_states(self, B: int, n_pos: int) -> torch.Tensor:
        """A draft-state buffer for kda_verify_direct: fp32 [B, n_pos, H, d, d] on the pool's
        device (kda_draft_state_bytes bytes)."""
        n = lib.kda_draft_state_bytes(byref(self.desc), B, n_pos)
        if n == 0 and B * n_pos > 0:
            raise ValueError("invalid draft-state geometry")
        return torch.empty((B, n_pos, self.H, self.d, self.d), dtype=torch.float32, device=self.device)

    def kda_verify_direct(self, q, k, v, a, b, slots, draft_states=None, o=None, stream=None):
        """Verify P positions per sequence, writing the state after every position to
        draft_states [B, P, H, d, d] (allocated when None) instead of the ring. Returns
        (o, draft_states)."""
        n_pos = q.shape[1]
        if o is None:
            o = torch.empty(q.shape[:-1] + (self.d,), dtype=torch.bfloat16, device=q.device)
        if draft_states is None:
            draft_states = self.kda_draft_states(q.shape[0], n_pos)
        _check_draft(draft_states, q.shape[0], n_pos, self.H, self.d)
        args, keep = self._step_args(q, k, v, a, b, o, slots)
        check(lib.kda_verify_direct(self.handle, byref(args), n_pos, draft_states.data_ptr(),
                                    _stream(stream)), "kda_verify_direct")
        return o, draft_states

    def kda_commit_direct(self, slots, n_accepted: torch.Tensor, draft_states: torch.Tensor,
                          stream=None) -> None:
        """Commit by copying draft_states[b, n_accepted[b]] (the buffer, position count and slot
        order of the kda_verify_direct call) into each slot."""
        s = _ix(slots, self.device)
        na = _dev(n_accepted, torch.int32, "n_accepted")
        n_pos = draft_states.shape[1]
        _check_draft(draft_states, s.np.size, n_pos, self.H, self.d)
        check(lib.kda_commit_direct(self.handle, s.np.size, s.h, s.d, na, draft_states.data_ptr(),
                                    n_pos, _stream(stream)), "kda_commit_direct")

    def kda_rollback(self, slots, stream=None) -> None:
        s = _ix(slots, self.device)
        check(lib.kda_rollback(self.handle, s.np.size, s.h, s.d, _stream(stream)),
              "kda_rollback")

    def kda_mixed_batch(self, q, k, v, a, b, cu_seqlens, out_slots, decode_slots,
                        verify_slots, n_pos: int, init_slots=None, ckpt_slots=None,
                        ckpt_interval: int = 0, o=None, stream=None, commit_slots=None,
                        n_accepted: torch.Tensor | None = None, fork: bool = True) -> torch.Tensor:
        """One packed batch [prefill tokens | decode tokens | verify tokens ([seq][pos])].
        commit_slots / n_accepted (device int32): ReplaySSM commits of slots pending from an
        earlier verify, run before this batch's decode and verify. fork: run those parts on the
        pool's side stream beside the prefill (False: in order on `stream`, ahead of it)."""
        if o is None:
            o = torch.empty(q.shape[:-1] + (self.d,), dtype=torch.bfloat16, device=q.device)
        ptrs = self._tok_ptrs(q, k, v, a, b, o)
        cu = _ix(cu_seqlens, self.device)
        out = _ix(out_slots, self.device)
        init = None if init_slots is None else _ix(init_slots, self.device)
        ckpt = None if ckpt_slots is None or len(ckpt_slots) == 0 else _ix(ckpt_slots, self.device)
        dec = _ix(decode_slots, self.device)
        ver = _ix(verify_slots, self.device)
        m = _abi.kda_mixed_args(*ptrs)
        m.prefill = self._prefill_struct(int(cu.np[-1]), cu, init, out, ckpt, chunk_for(self.d),
                                         ckpt_interval, (None,) * 6)
        m.n_decode, m.h_decode_slots, m.d_decode_slots = dec.np.size, dec.h, dec.d
        m.n_verify, m.n_pos = ver.np.size, n_pos
        m.h_verify_slots, m.d_verify_slots = ver.h, ver.d
        if commit_slots is not None:
            com = _ix(commit_slots, self.device)
            m.n_commit, m.h_commit_slots, m.d_commit_slots = com.np.size, com.h, com.d
            m.d_n_accepted = _dev(n_accepted, torch.int32, "n_accepted")
        if fork and m.prefill.n_seq > 0 and (m.n_decode or m.n_verify or m.n_commit):
            side, ev_fork, ev_join = self._side_stream()
            m.side_stream, m.fork_event, m.join_event = side.cuda_stream, ev_fork, ev_join
        check(lib.kda_mixed_batch(self.handle, byref(m), _stream(stream)), "kda_mixed_batch")
        return o

    def _side_stream(self):
        """Side stream (default priority, from torch) and fork / join events for mixed batches.
        The events only order two streams of one device, so they are made without timing and
        without the system-scope fence an event record otherwise performs (a cache write-back
        for the host's sake: ~3 us per mixed step)."""
        if self._side is None:
            side = torch.cuda.Stream(device=self.device)
            with torch.cuda.device(self.device):
                evs = [_StreamEvent(), _StreamEvent()]
            self._side = (side, evs)
        side, evs = self._side
        return side, evs[0].handle, evs[1].handle

    def kda_prefill_plan(self, cu_seqlens) -> list:
        """Width plan of kda_prefill's state pass for these sequence boundaries:
        [(rank_end, value_columns), ...] over the sequences ranked by length."""
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        ends, vsw = np.zeros(4, np.int32), np.zeros(4, np.int32)
        n = lib.kda_prefill_plan(self.handle, cu.size - 1, cu.ctypes.data, ends.ctypes.data,
                                 vsw.ctypes.data)
        return [(int(ends[i]), int(vsw[i])) for i in range(n)]

    def kda_read_device_error(self, stream=None) -> int:
        bits = c_uint32()
        check(lib.kda_read_device_error(self.handle, byref(bits), _stream(stream)),
              "kda_read_device_error")
        return bits.value

    # ------------------------------------------------------------------ views for checks
    def meta_array(self) -> np.ndarray:
        """[num_slots, 5] int64: pos, ring_head, pending, v_base, v_npos (synchronous copy)."""
        raw = self.meta[: self.num_slots * 24].cpu().numpy()
        rec = raw.view(np.dtype([("pos", "<i8"), ("ring_head", "<i4"), ("pending", "<i4"),
                                 ("v_base", "<i4"), ("v_npos", "<i4")]))
        return np.stack([rec[f].astype(np.int64) for f in rec.dtype.names], axis=1)

    def ring_tensors(self):
        """Views of the ring sections: k, v bf16 [S, R, H, d]; a fp32 [S, R, H, d]; b [S, R, H]."""
        S, R, H, d = self.num_slots, self.R, self.H, self.d
        n = S * R * H
        o = self.ring_offsets
        k = self.ring[o[0]:o[0] + n * d * 2].view(torch.bfloat16).view(S, R, H, d)
        v = self.ring[o[1]:o[1] + n * d * 2].view(torch.bfloat16).view(S, R, H, d)
        a = self.ring[o[2]:o[2] + n * d * 4].view(torch.float32).view(S, R, H, d)
        b = self.ring[o[3]:o[3] + n * 4].view(torch.float32).view(S, R, H)
        return k, v, a, b
