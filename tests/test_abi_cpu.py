"""CPU-side checks of the C ABI: the library loads and exports every declared symbol, the
size helpers follow the documented layouts, and the host-side pool bookkeeping and argument
validation behave as documented. No call here reaches a kernel launch: pools are created
over placeholder device addresses, and every exercised path fails validation first or is
host-only."""
import ctypes
import os
import re
from ctypes import byref, c_int32, c_size_t, c_void_p

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "recurrent_linear_attention_amd", "lib", "libkda.so")
if not os.path.exists(LIB):   # the library is built, not committed
    import importlib.util   # build.py from its file: the package __init__ loads the library
    _spec = importlib.util.spec_from_file_location(
        "_kda_build", os.path.join(ROOT, "recurrent_linear_attention_amd", "build.py"))
    _b = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(_b)
    _b.build()

from recurrent_linear_attention_amd import _abi  # noqa: E402
from recurrent_linear_attention_amd._abi import lib  # noqa: E402
from oracle import KDAPool as OraclePool  # noqa: E402

FAKE = 1 << 20          # 256-aligned placeholder "device" address, never dereferenced


def header_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(kda_\w+)\s*\(", src))


def test_every_declared_symbol_is_exported_and_bound():
    names = header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(_abi.PROTOTYPES), names ^ set(_abi.PROTOTYPES)


def desc(n=8, H=2, d=16, R=9):
    return _abi.kda_pool_desc(n, H, d, d, R)


def test_size_helpers():
    d = desc(n=256, H=32, d=128, R=9)
    assert lib.kda_state_bytes(byref(d)) == 256 * 32 * 128 * 128 * 4
    off = (c_size_t * 4)()
    assert lib.kda_ring_layout(byref(d), off) == 0
    per = 256 * 9 * 32
    assert off[0] == 0 and off[1] >= per * 128 * 2 and off[2] >= off[1] + per * 128 * 2
    assert off[3] >= off[2] + per * 128 * 4 and all(o % 256 == 0 for o in off)
    assert lib.kda_ring_bytes(byref(d)) >= off[3] + per * 4
    assert lib.kda_meta_error_offset(byref(d)) >= 256 * 24
    assert lib.kda_meta_bytes(byref(d)) >= lib.kda_meta_error_offset(byref(d)) + 4
    assert ctypes.sizeof(_abi.kda_slot_meta) == 24
    assert lib.kda_draft_state_bytes(byref(d), 4, 9) == 4 * 9 * 32 * 128 * 128 * 4
    assert lib.kda_draft_state_bytes(byref(d), -1, 9) == 0
    bad = _abi.kda_pool_desc(8, 2, 64, 64, 9)
    assert lib.kda_state_bytes(byref(bad)) == 0          # d = 64 not instantiated
    assert lib.kda_draft_state_bytes(byref(bad), 1, 1) == 0


class HostPool:
    def __init__(self, n=8, H=2, d=16, R=9):
        self.d = desc(n, H, d, R)
        h = c_void_p()
        assert lib.kda_pool_create(byref(self.d), FAKE, FAKE, FAKE, byref(h)) == 0
        self.h = h

    def __del__(self):
        lib.kda_pool_destroy(self.h)

    def alloc(self):
        s = c_int32()
        st = lib.kda_slot_alloc(self.h, byref(s))
        return st, s.value


def test_pool_create_rejects_bad_arguments():
    h = c_void_p()
    d = desc()
    assert lib.kda_pool_create(byref(d), None, FAKE, FAKE, byref(h)) == _abi.KDA_EINVAL
    assert lib.kda_pool_create(byref(d), FAKE + 4, FAKE, FAKE, byref(h)) == _abi.KDA_EINVAL
    d64 = _abi.kda_pool_desc(8, 2, 64, 64, 9)
    assert lib.kda_pool_create(byref(d64), FAKE, FAKE, FAKE, byref(h)) == _abi.KDA_EUNSUPPORTED
    d0 = _abi.kda_pool_desc(8, 2, 16, 16, 0)
    assert lib.kda_pool_create(byref(d0), FAKE, FAKE, FAKE, byref(h)) == _abi.KDA_EINVAL
    assert b"ring_cap" in lib.kda_last_error()


def test_alloc_free_trace_matches_oracle_model():
    rng = np.random.default_rng(0)
    p, m = HostPool(n=16), OraclePool(16, 1, 2, 2, 3)
    for _ in range(400):
        if rng.random() < 0.55:
            st, s = p.alloc()
            try:
                ms = m.alloc()
                assert st == 0 and s == ms
            except LookupError:
                assert st == _abi.KDA_ENOSLOT
        else:
            s = int(rng.integers(-1, 17))
            st = lib.kda_slot_free(p.h, s)
            try:
                m.free(s)
                assert st == 0
            except (ValueError, IndexError):
                assert st == _abi.KDA_EINVAL
        for s in range(16):
            assert lib.kda_slot_host_state(p.h, s) == int(m.live[s])


def i32(*v):
    return np.array(v, dtype=np.int32)


def step_args(B, slots):
    a = _abi.kda_step_args(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    a.B = B
    a.h_slots = slots.ctypes.data
    a.d_slots = FAKE
    return a


def test_step_validation_errors_launch_nothing():
    p = HostPool()
    s0, s1 = p.alloc()[1], p.alloc()[1]
    dead = i32(5)
    assert lib.kda_decode(p.h, byref(step_args(1, dead)), None) == _abi.KDA_EINVAL
    dup = i32(s0, s0)
    assert lib.kda_decode(p.h, byref(step_args(2, dup)), None) == _abi.KDA_EINVAL
    assert b"repeats" in lib.kda_last_error()
    ok = i32(s0, s1)
    assert lib.kda_verify(p.h, byref(step_args(2, ok)), 10, None) == _abi.KDA_EINVAL
    assert lib.kda_verify(p.h, byref(step_args(2, ok)), 0, None) == _abi.KDA_EINVAL
    # commit / rollback of idle slots: wrong state
    assert lib.kda_commit(p.h, 2, ok.ctypes.data, FAKE, FAKE, None) == _abi.KDA_ESTATE
    assert lib.kda_rollback(p.h, 2, ok.ctypes.data, FAKE, None) == _abi.KDA_ESTATE
    # misaligned token tensor
    a = step_args(2, ok)
    a.q = FAKE + 2
    assert lib.kda_decode(p.h, byref(a), None) == _abi.KDA_EINVAL
    # nothing changed host-side
    assert lib.kda_slot_host_state(p.h, s0) == 1 and lib.kda_slot_host_state(p.h, s1) == 1
    # zero-size batches are no-ops
    assert lib.kda_decode(p.h, byref(step_args(0, ok)), None) == 0
    assert lib.kda_slot_reset(p.h, 7, None) == _abi.KDA_EINVAL
    assert lib.kda_slot_checkpoint(p.h, s0, s0, None) == _abi.KDA_EINVAL


def test_direct_checkpoint_validation_errors_launch_nothing():
    p = HostPool()
    s0, s1 = p.alloc()[1], p.alloc()[1]
    ok = i32(s0, s1)
    # n_pos outside 1..ring_cap, missing / misaligned draft buffer
    assert lib.kda_verify_direct(p.h, byref(step_args(2, ok)), 10, FAKE, None) == _abi.KDA_EINVAL
    assert lib.kda_verify_direct(p.h, byref(step_args(2, ok)), 0, FAKE, None) == _abi.KDA_EINVAL
    assert lib.kda_verify_direct(p.h, byref(step_args(2, ok)), 3, None, None) == _abi.KDA_EINVAL
    assert lib.kda_verify_direct(p.h, byref(step_args(2, ok)), 3, FAKE + 4, None) == _abi.KDA_EINVAL
    dup = i32(s0, s0)
    assert lib.kda_verify_direct(p.h, byref(step_args(2, dup)), 3, FAKE, None) == _abi.KDA_EINVAL
    # a direct commit of idle slots: wrong state
    assert lib.kda_commit_direct(p.h, 2, ok.ctypes.data, FAKE, FAKE, FAKE, 3, None) == _abi.KDA_ESTATE
    assert b"not pending" in lib.kda_last_error()
    # nothing changed host-side; zero-size batches are no-ops
    assert lib.kda_slot_host_state(p.h, s0) == 1 and lib.kda_slot_host_state(p.h, s1) == 1
    assert lib.kda_verify_direct(p.h, byref(step_args(0, ok)), 3, FAKE, None) == 0


def prefill_args(cu, out, init=None, ckpt=None, chunk=16, interval=0):
    a = _abi.kda_prefill_args(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    a.n_seq, a.n_tok, a.chunk, a.ckpt_interval = cu.size - 1, int(cu[-1]), chunk, interval
    a.h_cu_seqlens, a.d_cu_seqlens = cu.ctypes.data, FAKE
    a.h_out_slot, a.d_out_slot = out.ctypes.data, FAKE
    if init is not None:
        a.h_init_slot, a.d_init_slot = init.ctypes.data, FAKE
    if ckpt is not None:
        a.h_ckpt_slot, a.d_ckpt_slot = ckpt.ctypes.data, FAKE
    return a


def test_prefill_validation_errors():
    p = HostPool()
    s = [p.alloc()[1] for _ in range(6)]
    cu, out = i32(0, 40, 64), i32(s[0], s[1])
    # chunk not instantiated / interval not a multiple of the chunk
    assert lib.kda_prefill(p.h, byref(prefill_args(cu, out, chunk=32)), None) == _abi.KDA_EUNSUPPORTED
    assert lib.kda_prefill(p.h, byref(prefill_args(cu, out, interval=-16)), None) == _abi.KDA_EUNSUPPORTED
    # cu_seqlens must start at 0, not decrease, and end at n_tok
    assert lib.kda_prefill(p.h, byref(prefill_args(i32(1, 40, 64), out)), None) == _abi.KDA_EINVAL
    assert lib.kda_prefill(p.h, byref(prefill_args(i32(0, 40, 30), out)), None) == _abi.KDA_EINVAL
    # checkpoints needed (40 // 16 + 24 // 16 = 3) but none given
    assert lib.kda_prefill(p.h, byref(prefill_args(cu, out, interval=16)), None) == _abi.KDA_EINVAL
    # out slots must be distinct; checkpoint slots distinct from out slots
    assert lib.kda_prefill(p.h, byref(prefill_args(cu, i32(s[0], s[0]))), None) == _abi.KDA_EINVAL
    ck = i32(s[2], s[3], s[1])
    assert lib.kda_prefill(p.h, byref(prefill_args(cu, out, ckpt=ck, interval=16)), None) == _abi.KDA_EINVAL
    # an init slot written by another sequence of the same call
    assert lib.kda_prefill(p.h, byref(prefill_args(cu, out, init=i32(s[1], -1))), None) == _abi.KDA_EINVAL
    # a non-live slot anywhere
    assert lib.kda_prefill(p.h, byref(prefill_args(cu, i32(s[0], 7))), None) == _abi.KDA_EINVAL
    # empty prefill is a no-op
    assert lib.kda_prefill(p.h, byref(prefill_args(i32(0), i32())), None) == 0


def test_prefill_workspace_size_and_checks():
    p = HostPool(H=4, d=128)
    s = [p.alloc()[1] for _ in range(3)]
    p16 = HostPool(H=4, d=16)
    # the d = 16 form keeps its chunks on chip and takes no workspace, nor does an empty call
    assert lib.kda_prefill_workspace_bytes(p16.h, 1000, 3, 16, 0) == 0
    assert lib.kda_prefill_workspace_bytes(p.h, 1000, 0, 64, 0) == 0
    # at most floor(1000 / 64) + 3 = 18 chunks, 61,952 bytes per (chunk, head), plus a small plan
    need = lib.kda_prefill_workspace_bytes(p.h, 1000, 3, 64, 0)
    assert 18 * 4 * 61952 <= need < 19 * 4 * 61952
    assert lib.kda_prefill_workspace_bytes(p.h, 1064, 3, 64, 0) > need
    assert lib.kda_prefill_workspace_bytes(p.h, 1000, 4, 64, 0) > need
    # an interval that is a multiple of the chunk adds nothing; any other adds one chunk per
    # boundary: 1000 // 100 = 10 more
    assert lib.kda_prefill_workspace_bytes(p.h, 1000, 3, 64, 128) == need
    assert lib.kda_prefill_workspace_bytes(p.h, 1000, 3, 64, 100) == need + 10 * 4 * 61952
    assert lib.kda_prefill_workspace_bytes(p.h, 1000, 3, 64, -1) == 0
    # lengths 640 + 360 -> 10 + 6 chunks; a too-small or misaligned buffer fails validation
    cu, out = i32(0, 640, 1000), i32(s[0], s[1])
    a = prefill_args(cu, out, chunk=64)
    a.workspace, a.workspace_bytes = FAKE, 16 * 4 * 61952 - 1
    assert lib.kda_prefill(p.h, byref(a), None) == _abi.KDA_EWORKSPACE
    assert b"workspace" in lib.kda_last_error()
    a.workspace, a.workspace_bytes = FAKE + 16, need
    assert lib.kda_prefill(p.h, byref(a), None) == _abi.KDA_EINVAL
    # no workspace at all: rejected, never allocated by the library
    a.workspace, a.workspace_bytes = None, 0
    assert lib.kda_prefill(p.h, byref(a), None) == _abi.KDA_EWORKSPACE
    assert b"no workspace" in lib.kda_last_error()
    a.workspace_bytes = need
    assert lib.kda_prefill(p.h, byref(a), None) == _abi.KDA_EWORKSPACE


def test_prefill_noalloc_rejects_prefills_beyond_its_scratch():
    # one 4096-token prompt at 32 heads needs 65 chunks x 32 x 61,952 bytes > 64 MiB: rejected
    # before any device call, nothing allocated, slots unchanged
    p = HostPool(n=4, H=32, d=128)
    s = [p.alloc()[1] for _ in range(2)]
    a = prefill_args(i32(0, 4096), i32(s[0]), chunk=64)
    assert lib.kda_prefill_workspace_bytes(p.h, 4096, 1, 64, 0) > 64 << 20
    assert lib.kda_prefill_noalloc(p.h, byref(a), None) == _abi.KDA_EWORKSPACE
    assert b"kda_prefill_noalloc holds 67108864" in lib.kda_last_error()
    # argument checks come first, as in kda_prefill
    assert lib.kda_prefill_noalloc(p.h, byref(prefill_args(i32(0, 40), i32(s[0]), chunk=32)), None) \
        == _abi.KDA_EUNSUPPORTED
    assert lib.kda_prefill_noalloc(p.h, byref(prefill_args(i32(0), i32(), chunk=64)), None) == 0
    assert [lib.kda_slot_host_state(p.h, x) for x in s] == [1, 1]


def test_mixed_batch_side_stream_needs_both_events():
    p = HostPool()
    s = [p.alloc()[1] for _ in range(3)]
    m, _keep = mixed_args(i32(0, 32), i32(s[0]), dec=[s[1]])
    m.side_stream, m.fork_event, m.join_event = FAKE, FAKE, None
    assert lib.kda_mixed_batch(p.h, byref(m), None) == _abi.KDA_EINVAL
    assert b"fork and join events" in lib.kda_last_error()
    m.fork_event, m.join_event = None, FAKE
    assert lib.kda_mixed_batch(p.h, byref(m), None) == _abi.KDA_EINVAL
    assert lib.kda_slot_host_state(p.h, s[1]) == 1


def test_mixed_batch_rejects_slot_overlap():
    p = HostPool()
    s = [p.alloc()[1] for _ in range(4)]
    m = _abi.kda_mixed_args(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    cu, out = i32(0, 32), i32(s[0])
    m.prefill = prefill_args(cu, out)
    dec, ver = i32(s[1], s[0]), i32(s[2])
    m.n_decode, m.h_decode_slots, m.d_decode_slots = 2, dec.ctypes.data, FAKE
    m.n_verify, m.n_pos, m.h_verify_slots, m.d_verify_slots = 1, 5, ver.ctypes.data, FAKE
    assert lib.kda_mixed_batch(p.h, byref(m), None) == _abi.KDA_EINVAL
    assert lib.kda_slot_host_state(p.h, s[2]) == 1      # verify slot not marked pending


def test_mixed_batch_commit_part_validation():
    p = HostPool()
    s = [p.alloc()[1] for _ in range(4)]
    m = _abi.kda_mixed_args(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    cu, out = i32(0, 32), i32(s[0])
    m.prefill = prefill_args(cu, out)
    com = i32(s[1])
    m.n_commit, m.h_commit_slots, m.d_commit_slots, m.d_n_accepted = 1, com.ctypes.data, FAKE, FAKE
    # committing an idle slot: wrong state, nothing changes
    assert lib.kda_mixed_batch(p.h, byref(m), None) == _abi.KDA_ESTATE
    assert lib.kda_slot_host_state(p.h, s[1]) == 1
    # a commit slot may not be a prefill slot
    com2 = i32(s[0])
    m.h_commit_slots = com2.ctypes.data
    assert lib.kda_mixed_batch(p.h, byref(m), None) in (_abi.KDA_EINVAL, _abi.KDA_ESTATE)
    m.n_commit = -1
    assert lib.kda_mixed_batch(p.h, byref(m), None) == _abi.KDA_EINVAL


def test_status_strings():
    for st in range(-6, 1):
        assert lib.kda_status_string(st)


def test_prefix_hit_policy():
    from recurrent_linear_attention_amd import prefix_hit
    # (shared prefix, prompt length, checkpoint interval) -> tokens covered by the checkpoint
    cases = [((0, 3000, 1024), 0), ((700, 3000, 1024), 0), ((1023, 3000, 1024), 0),
             ((1024, 3000, 1024), 1024), ((2100, 3000, 1024), 2048), ((3000, 3000, 1024), 2048),
             ((5000, 3000, 1024), 2048), ((2048, 2048, 1024), 1024), ((2049, 2049, 1024), 2048),
             ((64, 65, 64), 64), ((64, 64, 64), 0), ((10, 10, 0), 0), ((-3, 10, 4), 0)]
    for args, want in cases:
        assert prefix_hit(*args) == want, (args, want)


def plan_of(lengths, H=32):
    p = HostPool(n=8, H=H, d=128)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    ends, vsw = np.zeros(4, np.int32), np.zeros(4, np.int32)
    n = lib.kda_prefill_plan(p.h, len(lengths), cu.ctypes.data, ends.ctypes.data, vsw.ctypes.data)
    return [(int(ends[i]), int(vsw[i])) for i in range(n)]


def test_prefill_width_plan():
    """State-pass width plan on a 256-CU part (the CU count this container's library falls
    back to without a device): one width while every chain is about as long as the rest
    (the narrowest whose grid fits in one round of CUs, else 64 columns), narrow slices for
    long chains and 128-column slices for short ones in a lognormal mix; groups cover the
    ranks in order."""
    assert plan_of([8192]) == [(1, 16)]
    assert plan_of([5719, 4580]) == [(2, 32)]
    assert plan_of([2048] * 4) == [(4, 64)]
    assert plan_of([1024] * 8) == [(8, 128)]
    assert plan_of([512] * 32) == [(32, 128)]
    assert plan_of([1423, 1318, 1801, 1475, 4580, 5719]) == [(1, 32), (2, 64), (6, 128)]
    assert plan_of([300, 8000, 200, 100, 50, 10]) == [(1, 32), (6, 128)]
    assert plan_of([100] * 65) == [(65, 64)]                 # beyond 64 sequences: one width
    assert plan_of([0, 0, 0]) == [(3, 64)]                   # no chunk: no gain, one width
    p = HostPool(n=8, H=32, d=128)
    z = np.zeros(4, np.int32)
    assert lib.kda_prefill_plan(p.h, 0, z.ctypes.data, z.ctypes.data, z.ctypes.data) == 0
    assert lib.kda_prefill_plan(p.h, 1, None, z.ctypes.data, z.ctypes.data) == 0


def mixed_args(cu, out, dec=(), ver=(), n_pos=3, com=None, init=None, chunk=16):
    m = _abi.kda_mixed_args(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    keep = []
    m.prefill = prefill_args(cu, out, init=init, chunk=chunk)
    keep += [cu, out, init]
    for name, sl in (("decode", dec), ("verify", ver)):
        arr = i32(*sl)
        keep.append(arr)
        setattr(m, "n_" + name, arr.size)
        setattr(m, "h_" + name + "_slots", arr.ctypes.data if arr.size else None)
        setattr(m, "d_" + name + "_slots", FAKE if arr.size else None)
    m.n_pos = n_pos
    if com is not None:
        arr = i32(*com)
        keep.append(arr)
        m.n_commit, m.h_commit_slots, m.d_commit_slots, m.d_n_accepted = arr.size, arr.ctypes.data, FAKE, FAKE
    return m, keep


def test_mixed_batch_validation_errors_change_nothing():
    """Every part of a mixed batch is validated before anything is launched: slots distinct
    across the prefill (out and init slots), decode and verify parts, commit slots pending,
    n_pos within the ring, device arrays present. A rejected call leaves every slot's host
    state as it was."""
    p = HostPool()
    s = [p.alloc()[1] for _ in range(7)]
    cu, out = i32(0, 20, 33), i32(s[0], s[1])
    states = lambda: [lib.kda_slot_host_state(p.h, x) for x in range(8)]  # noqa: E731
    before = states()
    cases = [
        (mixed_args(cu, out, dec=[s[2], s[1]]), _abi.KDA_EINVAL),            # decode = prefill out
        (mixed_args(cu, out, ver=[s[0]]), _abi.KDA_EINVAL),                  # verify = prefill out
        (mixed_args(cu, out, dec=[s[2]], init=i32(s[3], -1), ver=[s[3]]), _abi.KDA_EINVAL),  # = init
        (mixed_args(cu, out, dec=[s[2]], ver=[s[2]]), _abi.KDA_EINVAL),      # decode = verify
        (mixed_args(cu, out, dec=[s[2], s[2]]), _abi.KDA_EINVAL),            # repeated decode slot
        (mixed_args(cu, out, ver=[s[2]], n_pos=10), _abi.KDA_EINVAL),        # n_pos > ring_cap
        (mixed_args(cu, out, ver=[s[2]], n_pos=0), _abi.KDA_EINVAL),
        (mixed_args(cu, out, dec=[7]), _abi.KDA_EINVAL),                     # not a live slot
        (mixed_args(cu, out, com=[s[4]]), _abi.KDA_ESTATE),                  # commit of an idle slot
        (mixed_args(cu, out, dec=[s[2]], chunk=64), _abi.KDA_EUNSUPPORTED),  # chunk 64 at d = 16
        (mixed_args(i32(0, 20, 10), out, dec=[s[2]]), _abi.KDA_EINVAL),      # cu_seqlens decreasing
    ]
    for i, ((m, _keep), want) in enumerate(cases):
        assert lib.kda_mixed_batch(p.h, byref(m), None) == want, (i, lib.kda_last_error())
        assert states() == before, i
    m, _keep = mixed_args(cu, out, dec=[s[2]])
    m.d_decode_slots = None
    assert lib.kda_mixed_batch(p.h, byref(m), None) == _abi.KDA_EINVAL
    m, _keep = mixed_args(cu, out, ver=[s[2]])
    m.d_verify_slots = None
    assert lib.kda_mixed_batch(p.h, byref(m), None) == _abi.KDA_EINVAL
    assert b"null device slot array" in lib.kda_last_error()
    m, _keep = mixed_args(cu, out, dec=[s[2]])
    m.n_decode = -1
    assert lib.kda_mixed_batch(p.h, byref(m), None) == _abi.KDA_EINVAL
    assert states() == before


@pytest.mark.parametrize("d", [16, 128])
def test_validation_fuzz_rejects_and_keeps_host_state(d):
    """Random prefill, decode, verify, commit and rollback calls, each a valid call with one
    certainly-invalid field drawn at random (slot out of range, free, repeated, or written
    twice; broken cu_seqlens or n_tok; wrong chunk; negative interval; missing or misaligned
    tensor, slot array or workspace; position count out of range; commit or rollback of idle
    slots): every call is refused before any device work (neither OK nor a HIP error), and no
    slot's host state changes. The host-sanitizer test runs this under ASan and UBSan too."""
    rng = np.random.default_rng(4242 + d)
    n, R, chunk = 24, 9, (16 if d == 16 else 64)
    p = HostPool(n=n, H=2, d=d, R=R)
    live = [p.alloc()[1] for _ in range(20)]      # slots 20..23 stay free
    free_slots = [20, 21, 22, 23]
    before = [lib.kda_slot_host_state(p.h, s) for s in range(n)]
    refused = (_abi.KDA_OK, _abi.KDA_EHIP)

    def unchanged():
        assert [lib.kda_slot_host_state(p.h, s) for s in range(n)] == before

    for _ in range(300):
        n_seq = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(0, 300, size=n_seq)]
        lens[0] = max(lens[0], 1)
        interval = int(rng.choice([0, chunk, 100]))
        n_ck = sum(L // interval for L in lens) if interval else 0
        if n_seq + n_ck > 20:
            interval, n_ck = 0, 0
        perm = [int(x) for x in rng.permutation(live)]
        out = i32(*perm[:n_seq])
        ck = i32(*perm[n_seq:n_seq + n_ck]) if n_ck else None
        rest = perm[n_seq + n_ck:]
        init = i32(*[rest[i] if i < len(rest) and rng.random() < 0.5 else -1 for i in range(n_seq)])
        cu = i32(0, *np.cumsum(lens))
        a = prefill_args(cu, out, init, ck, chunk=chunk, interval=interval)
        need = lib.kda_prefill_workspace_bytes(p.h, int(cu[-1]), n_seq, chunk, interval)
        a.workspace, a.workspace_bytes = FAKE, need
        # what these lengths need exactly (the plan arrays, then one block per chunk and head;
        # an interval that is not a multiple of the chunk cuts every interval into
        # ceil(interval / chunk) chunks): kda_prefill_workspace_bytes bounds it from above
        if need:
            per = -(-interval // chunk)
            chunks = sum(-(-L // chunk) if interval % chunk == 0 else
                         (L // interval) * per - (-(L % interval) // chunk) for L in lens)
            exact = -(-4 * (3 * n_seq + 1) // 256) * 256 + chunks * 2 * 61952
            assert exact <= need
        kinds = ["out_range", "out_free", "cu0", "ntok", "chunk", "interval", "null_q",
                 "misaligned_o", "null_cu", "init_free", "init_half"]
        if n_seq >= 2:
            kinds += ["out_dup", "init_other_out", "cu_decrease"]
        if n_ck:
            kinds += ["ck_dup_out", "ck_missing"]
        if need > 0:
            kinds += ["ws_small", "ws_null", "ws_misaligned"]
        kind = kinds[int(rng.integers(0, len(kinds)))]
        if kind == "out_range":
            out[int(rng.integers(0, n_seq))] = int(rng.choice([-2, n, n + 7, 1 << 30]))
        elif kind == "out_free":
            out[int(rng.integers(0, n_seq))] = free_slots[int(rng.integers(0, 4))]
        elif kind == "out_dup":
            out[1] = out[0]
        elif kind == "init_other_out":
            init[1] = out[0]
        elif kind == "init_free":
            init[0] = free_slots[int(rng.integers(0, 4))]
        elif kind == "init_half":
            a.d_init_slot = None
        elif kind == "cu0":
            cu[0] = 1
        elif kind == "cu_decrease":
            cu[1] = cu[2] + 1
        elif kind == "ntok":
            a.n_tok = int(cu[-1]) + int(rng.integers(1, 100))
        elif kind == "chunk":
            a.chunk = chunk * 2
        elif kind == "interval":
            a.ckpt_interval = -int(rng.integers(1, 1000))
        elif kind == "null_q":
            a.q = None
        elif kind == "misaligned_o":
            a.o = FAKE + 8
        elif kind == "null_cu":
            a.h_cu_seqlens = None
        elif kind == "ck_dup_out":
            ck[0] = out[0]
        elif kind == "ck_missing":
            a.h_ckpt_slot = None
        elif kind == "ws_small":
            a.workspace_bytes = exact - 1
        elif kind == "ws_null":
            a.workspace = None
        elif kind == "ws_misaligned":
            a.workspace = FAKE + 16
        st = lib.kda_prefill(p.h, byref(a), None)
        assert st not in refused, (kind, st)
        unchanged()

        B = int(rng.integers(1, 5))
        slots = i32(*[int(x) for x in rng.choice(live, size=B, replace=False)])
        sa = step_args(B, slots)
        kinds = ["range", "free", "b_neg", "null_h", "null_d", "null_q", "misaligned_k",
                 "npos0", "npos_big", "commit_idle", "rollback_idle"] + (["dup"] if B >= 2 else [])
        kind = kinds[int(rng.integers(0, len(kinds)))]
        call = "decode" if kind not in ("npos0", "npos_big") else "verify"
        if kind == "range":
            slots[int(rng.integers(0, B))] = int(rng.choice([-1, n, 1 << 20]))
        elif kind == "free":
            slots[int(rng.integers(0, B))] = free_slots[int(rng.integers(0, 4))]
        elif kind == "dup":
            slots[1] = slots[0]
        elif kind == "b_neg":
            sa.B = -int(rng.integers(1, 5))
        elif kind == "null_h":
            sa.h_slots = None
        elif kind == "null_d":
            sa.d_slots = None
        elif kind == "null_q":
            sa.q = None
        elif kind == "misaligned_k":
            sa.k = FAKE + 4
        if kind == "commit_idle":
            st = lib.kda_commit(p.h, B, slots.ctypes.data, FAKE, FAKE, None)
        elif kind == "rollback_idle":
            st = lib.kda_rollback(p.h, B, slots.ctypes.data, FAKE, None)
        elif call == "verify":
            st = lib.kda_verify(p.h, byref(sa), 0 if kind == "npos0" else R + 1, None)
        elif rng.random() < 0.5:
            st = lib.kda_decode(p.h, byref(sa), None)
        else:
            st = lib.kda_verify(p.h, byref(sa), int(rng.integers(1, R + 1)), None)
        assert st not in refused, (kind, st)
        unchanged()


@pytest.mark.parametrize("d", [16, 128])
def test_mixed_batch_validation_fuzz(d):
    """Random kda_mixed_batch calls, each a valid batch (prompts, decodes, verifies, optional
    side stream) with one certainly-invalid choice drawn at random: a decode or verify slot that
    is also a prefill out or init slot, a decode slot repeated as a verify slot, a commit of idle
    slots, a free or out-of-range step slot, a position count out of range, a side stream with
    a missing event, a null packed tensor or device slot array: every call is refused before
    any device work and no slot's host state changes."""
    rng = np.random.default_rng(777 + d)
    n, R, chunk = 24, 9, (16 if d == 16 else 64)
    p = HostPool(n=n, H=2, d=d, R=R)
    live = [p.alloc()[1] for _ in range(20)]
    before = [lib.kda_slot_host_state(p.h, s) for s in range(n)]
    for _ in range(300):
        perm = [int(x) for x in rng.permutation(live)]
        n_seq, nd, nv = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
        out, dec, ver = perm[:n_seq], perm[n_seq:n_seq + nd], perm[n_seq + nd:n_seq + nd + nv]
        spare = perm[n_seq + nd + nv:]
        init = [spare[0] if rng.random() < 0.5 else -1] + [-1] * (n_seq - 1)
        lens = [int(x) for x in rng.integers(1, 200, size=n_seq)]
        cu = i32(0, *np.cumsum(lens))
        kinds = ["dec_is_out", "ver_is_out", "dec_is_ver", "commit_idle", "dec_free", "ver_range",
                 "npos0", "npos_big", "fork_missing", "join_missing", "null_q", "null_dver"]
        if init[0] >= 0:
            kinds += ["dec_is_init", "ver_is_init"]
        kind = kinds[int(rng.integers(0, len(kinds)))]
        com = None
        n_pos = int(rng.integers(1, R + 1))
        if kind == "dec_is_out":
            dec[0] = out[0]
        elif kind == "ver_is_out":
            ver[0] = out[int(rng.integers(0, n_seq))]
        elif kind == "dec_is_init":
            dec[0] = init[0]
        elif kind == "ver_is_init":
            ver[0] = init[0]
        elif kind == "dec_is_ver":
            dec[0] = ver[0]
        elif kind == "commit_idle":
            com = [spare[-1]]
        elif kind == "dec_free":
            dec[0] = int(rng.integers(20, 24))
        elif kind == "ver_range":
            ver[0] = int(rng.choice([-1, n, 1 << 16]))
        elif kind == "npos0":
            n_pos = 0
        elif kind == "npos_big":
            n_pos = R + 1
        m, _keep = mixed_args(cu, i32(*out), dec=dec, ver=ver, n_pos=n_pos, com=com,
                              init=i32(*init), chunk=chunk)
        ws_need = lib.kda_prefill_workspace_bytes(p.h, int(cu[-1]), n_seq, chunk, 0)
        m.prefill.workspace, m.prefill.workspace_bytes = FAKE, ws_need
        if rng.random() < 0.5 or kind in ("fork_missing", "join_missing"):
            m.side_stream, m.fork_event, m.join_event = FAKE, FAKE, FAKE
        if kind == "fork_missing":
            m.fork_event = None
        elif kind == "join_missing":
            m.join_event = None
        elif kind == "null_q":
            m.q = None
        elif kind == "null_dver":
            m.d_verify_slots = None
        st = lib.kda_mixed_batch(p.h, byref(m), None)
        assert st not in (_abi.KDA_OK, _abi.KDA_EHIP), (kind, st)
        assert [lib.kda_slot_host_state(p.h, s) for s in range(n)] == before, kind
