"""Pins for the CPU oracle: each test checks the oracle against something other than itself --
a hand-derived example, a closed form, an invariant of the rule, or a special case that
reduces to a textbook result. Chosen so that a dropped term, a wrong sign, a transposed
decay or a pre-update readout fails at least one of them."""
import json
import os

import numpy as np
import pytest

from oracle import KDAPool, kda_chunked, kda_scan, kda_step, ERR_NACC_RANGE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, T, dk, dv, a_mu=2.0):
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    a = 1 / (1 + np.exp(-rng.normal(a_mu, 1.0, (T, dk))))
    b = 1 / (1 + np.exp(-rng.normal(0.0, 1.0, T)))
    return q, k, v, a, b


def test_hand_derived_2x2():
    g = json.load(open(os.path.join(GOLDEN, "hand_2x2.json")))
    S = np.array(g["S0"], float)
    for st, S_ref, o_ref in zip(g["steps"], g["S"], g["o"]):
        S, o = kda_step(S, *(np.array(st[n], float) for n in ("q", "k", "v", "a", "b")))
        np.testing.assert_allclose(S, S_ref, atol=1e-12)
        np.testing.assert_allclose(o, o_ref, atol=1e-12)


def test_scalar_geometric_series():
    # d_k = d_v = 1 with constant a, b, k, v: S_t = c S_{t-1} + e, c = a(1 - b k^2), e = b k v,
    # so from S_0 = 0: S_t = e (1 - c^t) / (1 - c) and o_t = q S_t.
    a, b, k, v, q = 0.9, 0.3, 0.8, -1.7, 0.5
    c, e = a * (1 - b * k * k), b * k * v
    T = 40
    ones = np.ones((T, 1))
    S, O, _ = kda_scan(np.zeros((1, 1)), q * ones, k * ones, v * ones, a * ones, b * np.ones(T))
    t = np.arange(1, T + 1)
    np.testing.assert_allclose(O[:, 0], q * e * (1 - c ** t) / (1 - c), rtol=1e-13)


def test_one_step_from_zero_reads_updated_state():
    rng = np.random.default_rng(1)
    q, k, v, a, b = (x[0] for x in rand_inputs(rng, 1, 5, 3))
    S, o = kda_step(np.zeros((5, 3)), q, k, v, a, b)
    np.testing.assert_allclose(S, b * np.outer(k, v), atol=1e-15)
    np.testing.assert_allclose(o, b * (q @ k) * v, atol=1e-15)


def test_unit_key_readout_writes_value_exactly():
    # a = 1, b = 1, ||k|| = 1: the delta rule makes k_t^T S_t = v_t^T whatever S_{t-1} was.
    rng = np.random.default_rng(2)
    q, k, v, _, _ = rand_inputs(rng, 30, 8, 6)
    S = rng.standard_normal((8, 6))
    for t in range(30):
        S, _ = kda_step(S, q[t], k[t], v[t], np.ones(8), 1.0)
        np.testing.assert_allclose(k[t] @ S, v[t], atol=1e-12)


def test_no_write_keeps_state_and_reads_it():
    rng = np.random.default_rng(3)
    q, k, v, _, _ = rand_inputs(rng, 20, 6, 4)
    S0 = rng.standard_normal((6, 4))
    S, O, _ = kda_scan(S0, q, k, v, np.ones((20, 6)), np.zeros(20))
    assert np.array_equal(S, S0)
    np.testing.assert_allclose(O, q @ S0, atol=1e-14)


def test_pure_decay_scales_key_rows():
    # b = 0: S_T = Diag(prod_t a_t) S_0 -- decay acts on key channels (rows), dk != dv.
    rng = np.random.default_rng(4)
    q, k, v, a, _ = rand_inputs(rng, 25, 7, 3)
    S0 = rng.standard_normal((7, 3))
    S, _, _ = kda_scan(S0, q, k, v, a, np.zeros(25))
    np.testing.assert_allclose(S, np.prod(a, axis=0)[:, None] * S0, rtol=1e-13)


def test_transition_matrix_closed_form():
    # S_t = A_t S_{t-1} + b_t k_t v_t^T with A_t = (I - b_t k_t k_t^T) Diag(a_t), hence
    # S_T = (A_T ... A_1) S_0 + sum_t (A_T ... A_{t+1}) b_t k_t v_t^T.
    rng = np.random.default_rng(5)
    dk, dv, T = 4, 3, 12
    q, k, v, a, b = rand_inputs(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    A = [(np.eye(dk) - b[t] * np.outer(k[t], k[t])) @ np.diag(a[t]) for t in range(T)]
    prod = np.eye(dk)
    acc = np.zeros((dk, dv))
    for t in reversed(range(T)):
        acc += prod @ (b[t] * np.outer(k[t], v[t]))
        prod = prod @ A[t]
    S, O, _ = kda_scan(S0, q, k, v, a, b)
    np.testing.assert_allclose(S, prod @ S0 + acc, atol=1e-13)


def test_orthonormal_keys_overwrite_memory():
    # a = 1, b = 1 and keys forming an orthonormal basis: after d_k writes the state holds
    # exactly sum_t k_t v_t^T and nothing of S_0 survives.
    rng = np.random.default_rng(6)
    dk, dv = 6, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm.T
    V = rng.standard_normal((dk, dv))
    S, _, _ = kda_scan(rng.standard_normal((dk, dv)), K, K, V, np.ones((dk, dk)), np.ones(dk))
    np.testing.assert_allclose(S, K.T @ V, atol=1e-12)


def test_relaxed_kaczmarz_converges_to_least_squares():
    # a = 1, constant b in (0, 2): the step is the relaxed Kaczmarz / Widrow-Hoff projection for
    # X^T k_t = v_t. On a consistent system with keys spanning R^dk it converges to the
    # solution that numpy.linalg.lstsq returns.
    rng = np.random.default_rng(7)
    dk, dv, m = 5, 3, 12
    K = rng.standard_normal((m, dk)); K /= np.linalg.norm(K, axis=1, keepdims=True)
    X = rng.standard_normal((dk, dv))
    V = K @ X
    sweeps = 300
    idx = np.tile(np.arange(m), sweeps)
    T = idx.size
    S, _, _ = kda_scan(np.zeros((dk, dv)), K[idx], K[idx], V[idx], np.ones((T, dk)),
                       np.full(T, 0.7))
    X_ls = np.linalg.lstsq(K, V, rcond=None)[0]
    np.testing.assert_allclose(S, X_ls, atol=1e-10)


def test_superposition_in_state_and_values():
    rng = np.random.default_rng(8)
    q, k, v, a, b = rand_inputs(rng, 40, 6, 4)
    S0 = rng.standard_normal((6, 4))
    S1, O1, _ = kda_scan(S0, q, k, v, a, b)
    S2, O2, _ = kda_scan(S0, q, k, 0 * v, a, b)
    S3, O3, _ = kda_scan(0 * S0, q, k, v, a, b)
    np.testing.assert_allclose(S1, S2 + S3, atol=1e-13)
    np.testing.assert_allclose(O1, O2 + O3, atol=1e-13)


def test_value_columns_and_heads_are_independent():
    rng = np.random.default_rng(9)
    q, k, v, a, b = rand_inputs(rng, 30, 6, 5)
    S0 = rng.standard_normal((6, 5))
    S, O, _ = kda_scan(S0, q, k, v, a, b)
    cols = [1, 3]
    Sc, Oc, _ = kda_scan(S0[:, cols], q, k, v[:, cols], a, b)
    np.testing.assert_allclose(Sc, S[:, cols], atol=1e-14)
    np.testing.assert_allclose(Oc, O[:, cols], atol=1e-14)
    # batched heads equal heads one by one
    q2, k2, v2, a2, b2 = rand_inputs(rng, 30, 6, 5)
    Sh, Oh, _ = kda_scan(np.stack([S0, 2 * S0]), np.stack([q, q2], 1), np.stack([k, k2], 1),
                         np.stack([v, v2], 1), np.stack([a, a2], 1), np.stack([b, b2], 1))
    S_b, O_b, _ = kda_scan(2 * S0, q2, k2, v2, a2, b2)
    np.testing.assert_allclose(Sh[0], S, atol=1e-14)
    np.testing.assert_allclose(Sh[1], S_b, atol=1e-14)
    np.testing.assert_allclose(Oh[:, 1], O_b, atol=1e-14)


@pytest.mark.parametrize("C,T,d", [(4, 37, 6), (8, 64, 16), (16, 64, 16), (64, 150, 32)])
def test_chunked_equals_sequential(C, T, d):
    rng = np.random.default_rng(10 + C)
    q, k, v, a, b = rand_inputs(rng, T, d, d)
    S0 = rng.standard_normal((d, d))
    every = 2 * C
    S, O, sn = kda_scan(S0, q, k, v, a, b, snapshot_every=every)
    Sc, Oc, snc = kda_chunked(S0, q, k, v, a, b, C, snapshot_every=every)
    scale = np.abs(O).max()
    np.testing.assert_allclose(Oc, O, atol=1e-12 * scale)
    np.testing.assert_allclose(Sc, S, atol=1e-12 * np.abs(S).max())
    assert len(sn) == len(snc) == T // every
    for x, y in zip(sn, snc):
        np.testing.assert_allclose(y, x, atol=1e-12 * np.abs(x).max())


def test_transitions_are_contractions():
    # ||(I - b k k^T) Diag(a)||_2 <= max(a) < 1 for b in [0, 1] and unit k: the state of the
    # recurrence stays bounded, which the kernels' fp32 state relies on.
    rng = np.random.default_rng(11)
    _, k, _, a, b = rand_inputs(rng, 200, 16, 16)
    for t in range(200):
        A = (np.eye(16) - b[t] * np.outer(k[t], k[t])) @ np.diag(a[t])
        assert np.linalg.norm(A, 2) <= a[t].max() + 1e-12


# ------------------------------------------------------------------ pool / ReplaySSM model

def _tok(rng, lead, H, d):
    q = rng.standard_normal(lead + (H, d)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal(lead + (H, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return {"q": q, "k": k, "v": rng.standard_normal(lead + (H, d)),
            "a": 1 / (1 + np.exp(-rng.normal(2, 1, lead + (H, d)))),
            "b": 1 / (1 + np.exp(-rng.normal(0, 1, lead + (H,))))}


def test_alloc_lowest_free_first_and_exhaustion():
    p = KDAPool(4, 1, 2, 2, 3)
    assert [p.alloc() for _ in range(4)] == [0, 1, 2, 3]
    with pytest.raises(LookupError):
        p.alloc()
    p.free(2)
    p.free(0)
    assert p.alloc() == 0 and p.alloc() == 2
    with pytest.raises(ValueError):
        p.free(5)


def test_ring_pointer_trace_hand_scripted():
    # R = 9. verify 5 at head 0 -> entries 0..4; commit 2 accepted -> 3 replayed, head 3.
    # verify 9 from head 3 -> entries 3..8,0,1,2; reject -> head stays 3.
    # verify 9 again; commit 8 -> head (3 + 9) % 9 = 3, pos 3 + 9 = 12.
    rng = np.random.default_rng(12)
    p = KDAPool(2, 1, 4, 4, 9)
    s = p.alloc()
    p.verify(_tok(rng, (1, 5), 1, 4), [s])
    assert tuple(p.meta()[s]) == (0, 0, 5, 0, 5)
    p.commit([s], [2])
    assert tuple(p.meta()[s]) == (3, 3, 0, 0, 5)
    tok = _tok(rng, (1, 9), 1, 4)
    p.verify(tok, [s])
    assert tuple(p.meta()[s]) == (3, 3, 9, 3, 9)
    np.testing.assert_array_equal(p.ring_k[s, 0, 0], tok["k"][0, 6, 0])   # wrapped entry
    before = p.state.copy()
    p.rollback([s])
    assert np.array_equal(p.state, before)
    assert tuple(p.meta()[s]) == (3, 3, 0, 3, 9)
    p.verify(tok, [s])
    p.commit([s], [8])
    assert tuple(p.meta()[s]) == (12, 3, 0, 3, 9)
    with pytest.raises(RuntimeError):
        p.commit([s], [0])           # nothing pending


def test_verify_does_not_write_state_and_commit_replays_stepwise():
    rng = np.random.default_rng(13)
    H, d, P = 2, 8, 6
    p = KDAPool(3, H, d, d, 9)
    slots = [p.alloc(), p.alloc()]
    p.state[slots] = rng.standard_normal((2, H, d, d))
    tok = _tok(rng, (2, P), H, d)
    before = p.state.copy()
    O = p.verify(tok, slots)
    assert np.array_equal(p.state, before)
    n_acc = [3, 0]
    p.commit(slots, n_acc)
    for n, s in enumerate(slots):
        S = before[s]
        for j in range(1 + n_acc[n]):
            S, o = kda_step(S, tok["q"][n, j], tok["k"][n, j], tok["v"][n, j],
                            tok["a"][n, j], tok["b"][n, j])
            np.testing.assert_allclose(O[n, j], o, atol=1e-14)
        np.testing.assert_allclose(p.state[s], S, atol=1e-14)


def test_commit_clamps_out_of_range_acceptance():
    rng = np.random.default_rng(14)
    p = KDAPool(1, 1, 4, 4, 9)
    s = p.alloc()
    tok = _tok(rng, (1, 3), 1, 4)
    p.verify(tok, [s])
    p.commit([s], [7])                      # only 3 positions were verified
    assert p.error_bits & ERR_NACC_RANGE
    assert tuple(p.meta()[s])[:3] == (3, 3, 0)


def test_direct_checkpoints_are_the_prefix_states():
    """Direct per-draft checkpoints: the state kept for position j is the sequential scan's
    state after positions 0..j, and the outputs are the ring verify's."""
    rng = np.random.default_rng(21)
    H, d, P = 2, 8, 5
    p, r = KDAPool(3, H, d, d, 9), KDAPool(3, H, d, d, 9)
    slots = [p.alloc(), p.alloc()]
    assert [r.alloc(), r.alloc()] == slots
    S0 = rng.standard_normal((2, H, d, d))
    p.state[slots] = S0
    r.state[slots] = S0
    tok = _tok(rng, (2, P), H, d)
    O, states = p.verify_direct(tok, slots)
    np.testing.assert_array_equal(O, r.verify(tok, slots))
    for n in range(2):
        _, O_scan, snaps = kda_scan(S0[n], *(tok[x][n] for x in "qkvab"), snapshot_every=1)
        np.testing.assert_allclose(O[n], O_scan, atol=1e-14)
        for j in range(P):
            np.testing.assert_allclose(states[n, j], snaps[j], atol=1e-14)
    assert np.array_equal(p.state[slots], S0)                     # committed state untouched
    assert np.array_equal(p.ring_k, np.zeros_like(p.ring_k))       # ring untouched


def test_direct_commit_equals_ring_replay():
    """Keeping the stored state of 1 + n positions == replaying them from the ring; the ring
    pointer moves only in the ring scheme. Out-of-range acceptance clamps in both."""
    rng = np.random.default_rng(22)
    H, d, P = 2, 8, 6
    p, r = KDAPool(3, H, d, d, 9), KDAPool(3, H, d, d, 9)
    slots = [p.alloc(), p.alloc(), p.alloc()]
    assert [r.alloc(), r.alloc(), r.alloc()] == slots
    S0 = rng.standard_normal((3, H, d, d))
    p.state[slots] = S0
    r.state[slots] = S0
    tok = _tok(rng, (3, P), H, d)
    _, states = p.verify_direct(tok, slots)
    r.verify(tok, slots)
    n_acc = [2, 0, 9]                                             # 9 > P - 1: clamped to 5
    p.commit_direct(slots, n_acc, states)
    r.commit(slots, n_acc)
    np.testing.assert_allclose(p.state[slots], r.state[slots], atol=1e-13)
    assert p.error_bits & ERR_NACC_RANGE and r.error_bits & ERR_NACC_RANGE
    assert list(p.pos[slots]) == list(r.pos[slots]) == [3, 1, 6]
    assert list(p.pending[slots]) == [0, 0, 0]
    assert list(p.ring_head[slots]) == [0, 0, 0] and list(r.ring_head[slots]) == [3, 1, 6]


def test_direct_and_ring_commits_do_not_mix():
    rng = np.random.default_rng(23)
    p = KDAPool(2, 1, 4, 4, 9)
    a, b = p.alloc(), p.alloc()
    tok = _tok(rng, (1, 3), 1, 4)
    _, states = p.verify_direct(tok, [a])
    p.verify(tok, [b])
    with pytest.raises(RuntimeError):
        p.commit([a], [0])
    with pytest.raises(RuntimeError):
        p.commit_direct([b], [0], states)
    before = p.state.copy()
    p.rollback([a, b])                                            # either kind rolls back
    assert np.array_equal(p.state, before) and list(p.pending) == [0, 0]
    assert not p.direct.any()


def test_checkpoint_equals_prefix_prefill():
    # The checkpoint exported after m*interval tokens equals the final state of a prefill
    # that stops at that boundary.
    rng = np.random.default_rng(15)
    H, d, T, I = 2, 8, 50, 16
    tok = _tok(rng, (T,), H, d)
    p = KDAPool(8, H, d, d, 9)
    out, c0, c1, c2 = (p.alloc() for _ in range(4))
    O = p.prefill(tok, [0, T], [-1], [out], [c0, c1, c2], I)
    for m, c in enumerate([c0, c1, c2]):
        q = KDAPool(1, H, d, d, 9)
        s = q.alloc()
        cut = {n: x[:(m + 1) * I] for n, x in tok.items()}
        Oq = q.prefill(cut, [0, (m + 1) * I], [-1], [s], [], 0)
        np.testing.assert_allclose(p.state[c], q.state[s], atol=1e-14)
        np.testing.assert_allclose(O[:(m + 1) * I], Oq, atol=1e-14)
        assert p.pos[c] == (m + 1) * I
    assert p.pos[out] == T


def test_prefill_resume_from_slot_equals_one_long_prefill():
    rng = np.random.default_rng(16)
    H, d = 1, 6
    tok = _tok(rng, (40,), H, d)
    p = KDAPool(4, H, d, d, 9)
    s1, s2 = p.alloc(), p.alloc()
    O1 = p.prefill({n: x[:24] for n, x in tok.items()}, [0, 24], [-1], [s1], [], 0)
    O2 = p.prefill({n: x[24:] for n, x in tok.items()}, [0, 16], [s1], [s1], [], 0)
    assert p.pos[s1] == 40
    O = p.prefill(tok, [0, 40], [-1], [s2], [], 0)
    np.testing.assert_allclose(np.concatenate([O1, O2]), O, atol=1e-14)
    np.testing.assert_allclose(p.state[s1], p.state[s2], atol=1e-14)
