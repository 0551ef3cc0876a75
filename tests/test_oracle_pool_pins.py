"""Pins for the oracle's pool bookkeeping outside the three uses' arithmetic: KDAPool.decode,
KDAPool.reset and KDAPool.checkpoint ("vLLM lifts Kimi K3 throughput by up to 2.8x", section
"ReplaySSM shrinks rollback state": a cache that holds recurrent state must roll back and
resume exactly; "Kimi K3 is here: efficient day-0 support on vLLM", summary: prefix caching
over KDA state).

Each pin is hand-scripted: the expected metadata is written out by hand, and the expected
state comes from a closed form (one step from a zero state is S = b k v^T, o = b (q.k) v; a
no-write step with a = 1, b = 0 leaves S and reads o = S^T q), never from the oracle's own
step function. The mutants at the end plant plausible bookkeeping mistakes in the oracle (on
the CPU only) and check that some pin here fails for each."""
import numpy as np
import pytest

import oracle.kda as ok
from oracle import KDAPool


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _ring_round(p, s, rng, n_pos, n_acc):
    """Drive slot s through one verify of n_pos positions and a commit of n_acc drafts, so its
    metadata holds non-zero ring fields."""
    H, d = p.H, p.dk
    tok = {"q": _unit(rng, (1, n_pos, H, d)), "k": _unit(rng, (1, n_pos, H, d)),
           "v": rng.standard_normal((1, n_pos, H, d)),
           "a": np.full((1, n_pos, H, d), 0.9), "b": np.full((1, n_pos, H), 0.5)}
    p.verify(tok, [s])
    p.commit([s], [n_acc])


def test_decode_advances_pos_and_writes_only_the_named_slots():
    # Slots 1 and 3 decode from a zero state: S = b k v^T and o = b (q.k) v exactly (one step
    # of the rule from S = 0). Slot 2 is live but not named, slot 0 holds a state of its own:
    # neither changes, in state or metadata.
    rng = np.random.default_rng(101)
    H, d = 2, 4
    p = KDAPool(5, H, d, d, 9)
    slots = [p.alloc() for _ in range(4)]
    assert slots == [0, 1, 2, 3]
    p.state[0] = rng.standard_normal((H, d, d))
    p.pos[0], p.pos[2] = 7, 11
    before = p.state.copy()
    q, k = _unit(rng, (2, H, d)), _unit(rng, (2, H, d))
    v = rng.standard_normal((2, H, d))
    a = np.full((2, H, d), 0.8)
    b = np.array([[0.25, 0.5], [0.75, 1.0]])
    o = p.decode({"q": q, "k": k, "v": v, "a": a, "b": b}, [3, 1])
    for n, s in enumerate([3, 1]):
        for h in range(H):
            np.testing.assert_allclose(p.state[s, h], b[n, h] * np.outer(k[n, h], v[n, h]), atol=1e-15)
            np.testing.assert_allclose(o[n, h], b[n, h] * (q[n, h] @ k[n, h]) * v[n, h], atol=1e-15)
    for s in (0, 2, 4):
        assert np.array_equal(p.state[s], before[s])
    assert [tuple(r) for r in p.meta()] == [(7, 0, 0, 0, 0), (1, 0, 0, 0, 0), (11, 0, 0, 0, 0),
                                             (1, 0, 0, 0, 0), (0, 0, 0, 0, 0)]


def test_decode_no_write_step_reads_the_state_and_keeps_ring_fields():
    # a = 1, b = 0: the state is untouched and o = S^T q. A slot with ring fields from an
    # earlier verify / commit keeps them; only pos moves.
    rng = np.random.default_rng(102)
    H, d = 1, 3
    p = KDAPool(2, H, d, d, 9)
    s = p.alloc()
    _ring_round(p, s, rng, n_pos=4, n_acc=2)                 # pos 3, ring_head 3, v_base 0, v_npos 4
    assert tuple(p.meta()[s]) == (3, 3, 0, 0, 4)
    S = p.state[s].copy()
    q = _unit(rng, (1, H, d))
    o = p.decode({"q": q, "k": _unit(rng, (1, H, d)), "v": rng.standard_normal((1, H, d)),
                  "a": np.ones((1, H, d)), "b": np.zeros((1, H))}, [s])
    assert np.array_equal(p.state[s], S)
    np.testing.assert_allclose(o[0, 0], S[0].T @ q[0, 0], atol=1e-15)
    assert tuple(p.meta()[s]) == (4, 3, 0, 0, 4)


def test_decode_refuses_a_pending_slot():
    rng = np.random.default_rng(103)
    p = KDAPool(1, 1, 2, 2, 9)
    s = p.alloc()
    tok = {"q": _unit(rng, (1, 2, 1, 2)), "k": _unit(rng, (1, 2, 1, 2)),
           "v": rng.standard_normal((1, 2, 1, 2)), "a": np.ones((1, 2, 1, 2)), "b": np.ones((1, 2, 1))}
    p.verify(tok, [s])
    step = {n: x[:, 0] for n, x in tok.items()}
    with pytest.raises(RuntimeError):
        p.decode(step, [s])


def test_reset_zeroes_state_and_every_metadata_field():
    rng = np.random.default_rng(104)
    H, d = 2, 3
    p = KDAPool(3, H, d, d, 9)
    s0, s1 = p.alloc(), p.alloc()
    p.state[[s0, s1]] = rng.standard_normal((2, H, d, d))
    _ring_round(p, s1, rng, n_pos=5, n_acc=3)                # pos 4, ring_head 4, v_npos 5
    _ring_round(p, s0, rng, n_pos=2, n_acc=0)                # pos 1, ring_head 1, v_npos 2
    keep = p.state[s0].copy()
    assert tuple(p.meta()[s1]) == (4, 4, 0, 0, 5)
    p.reset(s1)
    assert np.array_equal(p.state[s1], np.zeros((H, d, d)))
    assert tuple(p.meta()[s1]) == (0, 0, 0, 0, 0)
    assert np.array_equal(p.state[s0], keep)                 # the other slot is untouched
    assert tuple(p.meta()[s0]) == (1, 1, 0, 0, 2)


def test_reset_refuses_pending_and_free_slots():
    rng = np.random.default_rng(105)
    p = KDAPool(2, 1, 2, 2, 9)
    s = p.alloc()
    tok = {"q": _unit(rng, (1, 1, 1, 2)), "k": _unit(rng, (1, 1, 1, 2)),
           "v": rng.standard_normal((1, 1, 1, 2)), "a": np.ones((1, 1, 1, 2)), "b": np.ones((1, 1, 1))}
    p.verify(tok, [s])
    with pytest.raises(RuntimeError):
        p.reset(s)
    with pytest.raises(ValueError):
        p.reset(1)                                           # never allocated


def test_checkpoint_copies_state_and_pos_and_clears_destination_ring_fields():
    # src: pos 6, ring_head 6 after two rounds. dst: its own state, pos 2, ring_head 2 and
    # v_npos 3. After checkpoint(src, dst): dst state == src state, dst meta == (6, 0, 0, 0, 0);
    # src keeps everything.
    rng = np.random.default_rng(106)
    H, d = 2, 3
    p = KDAPool(3, H, d, d, 9)
    src, dst = p.alloc(), p.alloc()
    p.state[[src, dst]] = rng.standard_normal((2, H, d, d))
    _ring_round(p, src, rng, n_pos=4, n_acc=3)               # pos 4, ring_head 4
    _ring_round(p, src, rng, n_pos=3, n_acc=1)               # pos 6, ring_head 6, v_base 4, v_npos 3
    _ring_round(p, dst, rng, n_pos=3, n_acc=1)               # pos 2, ring_head 2, v_npos 3
    assert tuple(p.meta()[src]) == (6, 6, 0, 4, 3)
    assert tuple(p.meta()[dst]) == (2, 2, 0, 0, 3)
    S_src = p.state[src].copy()
    p.checkpoint(src, dst)
    assert np.array_equal(p.state[dst], S_src)
    assert np.array_equal(p.state[src], S_src)
    assert tuple(p.meta()[dst]) == (6, 0, 0, 0, 0)
    assert tuple(p.meta()[src]) == (6, 6, 0, 4, 3)


def test_checkpoint_then_decode_matches_decode_of_the_source():
    # A decode on the copy reads the copied state: with a = 1, b = 0 both read o = S^T q.
    rng = np.random.default_rng(107)
    H, d = 1, 4
    p = KDAPool(2, H, d, d, 9)
    src, dst = p.alloc(), p.alloc()
    p.state[src] = rng.standard_normal((H, d, d))
    p.pos[src] = 9
    p.checkpoint(src, dst)
    q = _unit(rng, (1, H, d))
    tok = {"q": q, "k": _unit(rng, (1, H, d)), "v": rng.standard_normal((1, H, d)),
           "a": np.ones((1, H, d)), "b": np.zeros((1, H))}
    o = p.decode(tok, [dst])
    np.testing.assert_allclose(o[0, 0], p.state[src, 0].T @ q[0, 0], atol=1e-15)
    assert tuple(p.meta()[dst]) == (10, 0, 0, 0, 0)


def test_checkpoint_refuses_pending_slots():
    rng = np.random.default_rng(108)
    p = KDAPool(2, 1, 2, 2, 9)
    src, dst = p.alloc(), p.alloc()
    tok = {"q": _unit(rng, (1, 1, 1, 2)), "k": _unit(rng, (1, 1, 1, 2)),
           "v": rng.standard_normal((1, 1, 1, 2)), "a": np.ones((1, 1, 1, 2)), "b": np.ones((1, 1, 1))}
    p.verify(tok, [dst])
    with pytest.raises(RuntimeError):
        p.checkpoint(src, dst)


# ------------------------------------------------------------------ planted mistakes

def _m_decode_no_pos(self, tok, slots):
    slots = self._check_idle(slots)
    S, o = ok.kda_step(self.state[slots], tok["q"], tok["k"], tok["v"], tok["a"], tok["b"])
    self.state[slots] = S
    return o


def _m_decode_slots_reversed(self, tok, slots):
    slots = self._check_idle(slots)
    S, o = ok.kda_step(self.state[slots], tok["q"], tok["k"], tok["v"], tok["a"], tok["b"])
    self.state[slots[::-1]] = S
    self.pos[slots] += 1
    return o


def _m_decode_pos_on_all_live(self, tok, slots):
    slots = self._check_idle(slots)
    S, o = ok.kda_step(self.state[slots], tok["q"], tok["k"], tok["v"], tok["a"], tok["b"])
    self.state[slots] = S
    self.pos[self.live] += 1
    return o


def _m_reset_keeps_meta(self, s):
    self._check_idle([s])
    self.state[s] = 0.0
    self.pos[s] = 0


def _m_reset_keeps_pos(self, s):
    self._check_idle([s])
    self.state[s] = 0.0
    self.ring_head[s] = self.pending[s] = self.v_base[s] = self.v_npos[s] = 0


def _m_checkpoint_keeps_dst_ring(self, src, dst):
    self._check_idle([src, dst])
    self.state[dst] = self.state[src]
    self.pos[dst] = self.pos[src]


def _m_checkpoint_copies_src_ring(self, src, dst):
    self._check_idle([src, dst])
    self.state[dst] = self.state[src]
    for f in ("pos", "ring_head", "pending", "v_base", "v_npos"):
        getattr(self, f)[dst] = getattr(self, f)[src]


def _m_checkpoint_pos_zero(self, src, dst):
    self._check_idle([src, dst])
    self.state[dst] = self.state[src]
    self._clear_meta(dst)


PINS = [test_decode_advances_pos_and_writes_only_the_named_slots,
        test_decode_no_write_step_reads_the_state_and_keeps_ring_fields,
        test_reset_zeroes_state_and_every_metadata_field,
        test_checkpoint_copies_state_and_pos_and_clears_destination_ring_fields,
        test_checkpoint_then_decode_matches_decode_of_the_source]


@pytest.mark.parametrize("method,mutant", [
    ("decode", _m_decode_no_pos), ("decode", _m_decode_slots_reversed),
    ("decode", _m_decode_pos_on_all_live), ("reset", _m_reset_keeps_meta),
    ("reset", _m_reset_keeps_pos), ("checkpoint", _m_checkpoint_keeps_dst_ring),
    ("checkpoint", _m_checkpoint_copies_src_ring), ("checkpoint", _m_checkpoint_pos_zero)])
def test_some_pool_pin_catches_mutant(method, mutant, monkeypatch):
    monkeypatch.setattr(KDAPool, method, mutant)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutant.__name__}"
