"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle on the same
seeded inputs. Outputs within 2e-3 (``parity.rel_bf16``), states within 2e-3 (``parity.rel``),
slot metadata and ring contents bit-exact, rejected drafts leave the state bit-identical.

Workloads: the tiny d=16 case in full; the decode, verify/commit, 8192-token prefill and
mixed 16384-token batch at their full sizes on every head; mid-size ragged prefills in full.
Every comparison is taken over the whole tensor and per (sequence, head), and its measured
errors are logged (tests/parity.py)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kda_inputs as ki  # noqa: E402
import recurrent_linear_attention_amd as kda  # noqa: E402
from oracle import KDAPool as OPool  # noqa: E402
from tests.parity import TOL, check_out, check_state, dev, f64, meta_equal  # noqa: E402


def pools(n_slots, H, d, R=9, alloc=True):
    g, o = kda.KDAPool(n_slots, H, d, R), OPool(n_slots, H, d, d, R)
    if alloc:
        for _ in range(n_slots):
            assert g.kda_slot_alloc() == o.alloc()
    return g, o


def put_states(g, o, slots, states):
    slots = [int(s) for s in slots]
    g.state[slots] = states.to("cuda")
    o.state[slots] = states.double().numpy()
    torch.cuda.synchronize()


def tok_dev(t: ki.Tokens):
    return dev(t.q), dev(t.k), dev(t.v), dev(t.a), dev(t.b)


def ring_check(g, o, slots):
    rk, rv, ra, rb = g.ring_tensors()
    for s in slots:
        np.testing.assert_array_equal(f64(rk[s]), o.ring_k[s])
        np.testing.assert_array_equal(f64(rv[s]), o.ring_v[s])
        np.testing.assert_array_equal(f64(ra[s]), o.ring_a[s])
        np.testing.assert_array_equal(f64(rb[s]), o.ring_b[s])


def device_errors(g) -> int:
    """The pool's device error bits (read and cleared) without the informational bit that
    reports the prefill's exact path for strongly decaying channels, which random gates may
    take (tests that force that path check the bit itself)."""
    return g.kda_read_device_error() & ~kda._abi.KDA_DEVERR_DECAY_RANGE


def heads_np(t: ki.Tokens, heads):
    return {n: x[..., heads, :] if x.ndim >= 3 and n != "b" else x[..., heads]
            for n, x in t.np.items()}


# ----------------------------------------------------------------------------- tiny, d = 16

def test_tiny_prefill_checkpoints_verify_commit():
    w = ki.tiny_workload(0)
    H, d = w["H"], w["dk"]
    g, o = pools(w["n_slots"], H, d, w["ring_cap"])
    out, cks = 0, [1, 2, 3, 4]
    pre = w["prefill"]
    O = g.kda_prefill(*tok_dev(pre), w["cu_seqlens"], [out], ckpt_slots=cks,
                      ckpt_interval=w["ckpt_interval"], chunk=w["chunk"])
    Oo = o.prefill(pre.np, w["cu_seqlens"], [-1], [out], cks, w["ckpt_interval"])
    torch.cuda.synchronize()
    check_out(O, Oo, w["cu_seqlens"], v=pre.np["v"])
    for s in [out] + cks:
        check_state(g.state[s], o.state[s])
    meta_equal(g.meta_array(), o.meta(), [out] + cks)
    # the checkpoint after 64 tokens is the final state: the same bytes
    assert torch.equal(g.state[cks[-1]], g.state[out])

    ver = w["verify"]
    before = g.state.clone()
    Ov = g.kda_verify(*tok_dev(ver), [out])
    Ovo = o.verify(ver.np, [out])
    torch.cuda.synchronize()
    check_out(Ov, Ovo, v=ver.np["v"])
    assert torch.equal(g.state, before)
    ring_check(g, o, [out])
    meta_equal(g.meta_array(), o.meta(), [out])
    assert g.host_state(out) == 2

    na = torch.tensor(w["n_accepted"], dtype=torch.int32, device="cuda")
    g.kda_commit([out], na)
    o.commit([out], w["n_accepted"])
    torch.cuda.synchronize()
    check_state(g.state[out], o.state[out])
    meta_equal(g.meta_array(), o.meta(), [out])
    assert device_errors(g) == 0


# ----------------------------------------------------------------------------- decode

def test_decode_full_size():
    w = ki.decode_workload(1)
    g, o = pools(w["n_slots"], w["H"], w["dk"])
    slots = w["slots"]
    put_states(g, o, slots, w["states"])
    untouched = [s for s in range(w["n_slots"]) if s not in set(slots.tolist())][:8]
    before = g.state[untouched].clone()
    O = g.kda_decode(*tok_dev(w["tokens"]), slots)
    Oo = o.decode(w["tokens"].np, slots)
    torch.cuda.synchronize()
    check_out(O, Oo, v=w["tokens"].np["v"])
    check_state(g.state[slots.tolist()], o.state[slots])
    assert torch.equal(g.state[untouched], before)
    meta_equal(g.meta_array(), o.meta(), range(w["n_slots"]))


@pytest.mark.parametrize("d,B", [(128, 64), (128, 65), (16, 64), (16, 65)])
def test_decode_slot_ids_by_value_and_from_device(d, B):
    """Decode takes the slot ids of a batch of at most 64 sequences by value among the kernel
    arguments and reads the device array for larger batches: both sides of that limit, slots a
    random permutation of a larger pool, against the oracle, untouched slots unchanged."""
    H, n_slots = 4, 96
    rng = np.random.default_rng(640 + B + d)
    g, o = pools(n_slots, H, d)
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    put_states(g, o, slots, ki.draw_states(rng, B, H, d, d))
    untouched = sorted(set(range(n_slots)) - set(slots.tolist()))
    before = g.state[untouched].clone()
    tok = ki.draw_tokens(rng, (B,), H, d, d)
    O = g.kda_decode(*tok_dev(tok), slots)
    Oo = o.decode(tok.np, slots)
    torch.cuda.synchronize()
    check_out(O, Oo, v=tok.np["v"])
    check_state(g.state[slots.tolist()], o.state[slots])
    assert torch.equal(g.state[untouched], before)
    meta_equal(g.meta_array(), o.meta(), range(n_slots))
    assert device_errors(g) == 0


# ----------------------------------------------------------------------------- verify / commit

@pytest.mark.parametrize("d,B", [(128, 64), (128, 65), (16, 65)])
def test_commit_slot_ids_by_value_and_from_device(d, B):
    """Commit takes the slot ids of at most 64 sequences by value among the kernel arguments
    and reads the device array beyond: a verify of 1+2 positions and the commit of random
    accepted counts on both sides of that limit, state and metadata against the oracle."""
    H, n_slots, P = 2, 96, 3
    rng = np.random.default_rng(650 + B + d)
    g, o = pools(n_slots, H, d, R=P)
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    put_states(g, o, slots, ki.draw_states(rng, B, H, d, d))
    tok = ki.draw_tokens(rng, (B, P), H, d, d)
    g.kda_verify(*tok_dev(tok), slots)
    o.verify(tok.np, slots)
    na = rng.integers(0, P, size=B).astype(np.int32)
    g.kda_commit(slots, torch.from_numpy(na).to("cuda"))
    o.commit(slots, na)
    torch.cuda.synchronize()
    check_state(g.state[slots.tolist()], o.state[slots])
    meta_equal(g.meta_array(), o.meta(), range(n_slots))
    assert device_errors(g) == 0


def test_verify_commit_rollback_full_size():
    w = ki.verify_workload(2)
    g, o = pools(w["n_slots"], w["H"], w["dk"], w["ring_cap"])
    slots = w["slots"]
    put_states(g, o, slots, w["states"])
    tok = w["tokens"]
    before = g.state.clone()
    O = g.kda_verify(*tok_dev(tok), slots)
    Oo = o.verify(tok.np, slots)
    torch.cuda.synchronize()
    check_out(O, Oo, v=tok.np["v"])
    assert torch.equal(g.state, before), "verify must not write any state"
    ring_check(g, o, slots)
    meta_equal(g.meta_array(), o.meta(), slots)

    na = torch.from_numpy(w["n_accepted"]).to("cuda")
    g.kda_commit(slots, na)
    o.commit(slots, w["n_accepted"])
    torch.cuda.synchronize()
    check_state(g.state[slots.tolist()], o.state[slots])
    meta_equal(g.meta_array(), o.meta(), slots)

    # replay == stepwise: 1 + n decode calls from the same state give the same bytes
    g2, _ = pools(w["n_slots"], w["H"], w["dk"], w["ring_cap"])
    g2.state.copy_(before)
    for j in range(w["n_pos"]):
        live = [i for i in range(len(slots)) if j <= w["n_accepted"][i]]
        if not live:
            break
        sl = slots[live]
        tj = [dev(x[live, j]) for x in (tok.q, tok.k, tok.v, tok.a, tok.b)]
        g2.kda_decode(*tj, sl)
    torch.cuda.synchronize()
    assert torch.equal(g2.state[slots.tolist()], g.state[slots.tolist()])

    # a full reject: state bit-identical, pointer untouched
    tok2 = ki.draw_tokens(np.random.default_rng(20), (len(slots), 5), w["H"], w["dk"], w["dk"])
    snap = g.state.clone()
    g.kda_verify(*tok_dev(tok2), slots)
    o.verify(tok2.np, slots)
    g.kda_rollback(slots)
    o.rollback(slots)
    torch.cuda.synchronize()
    assert torch.equal(g.state, snap)
    meta_equal(g.meta_array(), o.meta(), slots)
    ring_check(g, o, slots)
    assert device_errors(g) == 0


@pytest.mark.parametrize("d", [128, 16])
@pytest.mark.parametrize("P", [1, 2, 3, 8, 9, 16, 17])
def test_verify_commit_every_position_count(d, P):
    """Verify of P positions (odd counts end the kernels' two-position loop with a padding
    position, even ones do not), then commits accepting P - 1 and 0 drafts on two sequences:
    outputs, ring entries and metadata against the oracle, nothing written past the P entries,
    and the committed states bit-identical to the same positions applied as decode calls."""
    H, R = 4, max(9, P)
    rng = np.random.default_rng(700 + 10 * P + d)
    g, o = pools(8, H, d, R)
    slots = np.array([2, 5], dtype=np.int32)
    st = ki.draw_states(rng, 2, H, d, d)
    put_states(g, o, slots, st)
    tok = ki.draw_tokens(rng, (2, P), H, d, d)
    before = g.state.clone()
    ring_before = [t.clone() for t in g.ring_tensors()]
    O = g.kda_verify(*tok_dev(tok), slots)
    Oo = o.verify(tok.np, slots)
    torch.cuda.synchronize()
    check_out(O, Oo, v=tok.np["v"])
    assert torch.equal(g.state, before), "verify must not write any state"
    ring_check(g, o, slots)
    # ring entries past the P written ones (in ring order from the old head) are untouched
    for t_new, t_old in zip(g.ring_tensors(), ring_before):
        for s_ in slots:
            assert torch.equal(t_new[int(s_)][P:], t_old[int(s_)][P:])
    meta_equal(g.meta_array(), o.meta(), slots)
    na = np.array([P - 1, 0], dtype=np.int32)
    g.kda_commit(slots, torch.from_numpy(na).to("cuda"))
    o.commit(slots, na)
    torch.cuda.synchronize()
    check_state(g.state[slots.tolist()], o.state[slots])
    meta_equal(g.meta_array(), o.meta(), slots)
    g2, _ = pools(8, H, d, R)
    g2.state.copy_(before)
    for j in range(P):
        live = [i for i in range(2) if j <= na[i]]
        tj = [dev(x[live, j]) for x in (tok.q, tok.k, tok.v, tok.a, tok.b)]
        g2.kda_decode(*tj, slots[live])
    torch.cuda.synchronize()
    assert torch.equal(g2.state[slots.tolist()], g.state[slots.tolist()])
    assert device_errors(g) == 0


@pytest.mark.parametrize("P", [9, 16])
def test_verify_under_strong_decay(P):
    """Verify and commit with strongly decaying channels: a = 0.3, 1e-3 and 0 (a full forget of
    the channel) at every position, outputs and committed states against the oracle."""
    H, d = 4, 128
    rng = np.random.default_rng(970 + P)
    g, o = pools(8, H, d, max(9, P))
    slots = np.array([1, 6], dtype=np.int32)
    put_states(g, o, slots, ki.draw_states(rng, 2, H, d, d))
    tok = ki.draw_tokens(rng, (2, P), H, d, d)
    tok.a[:, :, 0, [3, 70]] = 0.3
    tok.a[:, :, 1, [5, 9, 127]] = 1e-3
    tok.a[:, :, 2, 64] = 0.0
    tok.a[:, :, 3, :] = 1e-3
    tok.np["a"] = tok.a.to(torch.float64).numpy()
    O = g.kda_verify(*tok_dev(tok), slots)
    Oo = o.verify(tok.np, slots)
    torch.cuda.synchronize()
    assert torch.isfinite(O.float()).all()
    check_out(O, Oo, v=tok.np["v"])
    na = np.array([P - 1, P // 2], dtype=np.int32)
    g.kda_commit(slots, torch.from_numpy(na).to("cuda"))
    o.commit(slots, na)
    torch.cuda.synchronize()
    check_state(g.state[slots.tolist()], o.state[slots])
    meta_equal(g.meta_array(), o.meta(), slots)
    assert device_errors(g) == 0


@pytest.mark.parametrize("d", [128, 16])
def test_verify_commit_at_ring_capacity(d):
    """The largest ring a pool takes (64 entries): verify of 64 positions, commits accepting 63
    and 0 drafts, against the oracle; the committed states bit-identical to the same positions
    applied as decode calls."""
    H, R, P = 2, 64, 64
    rng = np.random.default_rng(900 + d)
    g, o = pools(6, H, d, R)
    slots = np.array([1, 4], dtype=np.int32)
    put_states(g, o, slots, ki.draw_states(rng, 2, H, d, d))
    tok = ki.draw_tokens(rng, (2, P), H, d, d)
    before = g.state.clone()
    O = g.kda_verify(*tok_dev(tok), slots)
    Oo = o.verify(tok.np, slots)
    torch.cuda.synchronize()
    check_out(O, Oo, v=tok.np["v"])
    assert torch.equal(g.state, before)
    ring_check(g, o, slots)
    na = np.array([P - 1, 0], dtype=np.int32)
    g.kda_commit(slots, torch.from_numpy(na).to("cuda"))
    o.commit(slots, na)
    torch.cuda.synchronize()
    check_state(g.state[slots.tolist()], o.state[slots])
    meta_equal(g.meta_array(), o.meta(), slots)
    g2, _ = pools(6, H, d, R)
    g2.state.copy_(before)
    for j in range(P):
        live = [i for i in range(2) if j <= na[i]]
        tj = [dev(x[live, j]) for x in (tok.q, tok.k, tok.v, tok.a, tok.b)]
        g2.kda_decode(*tj, slots[live])
    torch.cuda.synchronize()
    assert torch.equal(g2.state[slots.tolist()], g.state[slots.tolist()])
    assert device_errors(g) == 0


def test_rule_invariants_at_full_size():
    """Properties of the rule checked on the device at the decode workload's size (16 sequences,
    32 heads, d = 128), independent of the oracle: with b = 0 and a = 1 nothing is written --
    decode, verify + full commit and a resumed prefill leave the state bit-identical; with a = 1,
    b = 1 and a one-hot key e_i, row i of the new state is the value vector."""
    w = ki.decode_workload(1)
    H, d = w["H"], w["dk"]
    g, _ = pools(w["n_slots"], H, d)
    slots = w["slots"]
    g.state[slots.tolist()] = w["states"].to("cuda")
    rng = np.random.default_rng(950)
    B = len(slots)
    # no write: b = 0, a = 1
    tok = ki.draw_tokens(rng, (B,), H, d, d)
    tok.a.fill_(1.0)
    tok.b.zero_()
    before = g.state.clone()
    g.kda_decode(*tok_dev(tok), slots)
    vt = ki.draw_tokens(rng, (B, 9), H, d, d)
    vt.a.fill_(1.0)
    vt.b.zero_()
    g.kda_verify(*tok_dev(vt), slots)
    g.kda_commit(slots, torch.full((B,), 8, dtype=torch.int32, device="cuda"))
    pt = ki.draw_tokens(rng, (300,), H, d, d)
    pt.a.fill_(1.0)
    pt.b.zero_()
    free = [s_ for s_ in range(w["n_slots"]) if s_ not in set(slots.tolist())][:1]
    g.kda_prefill(*tok_dev(pt), [0, 300], free, init_slots=[int(slots[0])])
    torch.cuda.synchronize()
    assert torch.equal(g.state[slots.tolist()], before[slots.tolist()])
    assert torch.equal(g.state[free[0]], before[int(slots[0])])
    # unit-key readout: a = 1, b = 1, k = e_i  =>  S_new[i, :] = v
    tok = ki.draw_tokens(rng, (B,), H, d, d)
    tok.a.fill_(1.0)
    tok.b.fill_(1.0)
    idx = rng.integers(0, d, size=(B, H))
    k = torch.zeros((B, H, d), dtype=torch.bfloat16)
    k[np.arange(B)[:, None], np.arange(H)[None, :], idx] = 1.0
    tok.k = k
    g.kda_decode(*tok_dev(tok), slots)
    torch.cuda.synchronize()
    ib = torch.arange(B, device="cuda")[:, None]
    ih = torch.arange(H, device="cuda")[None, :]
    rows = g.state[slots.tolist()][ib, ih, torch.from_numpy(idx).to("cuda")]
    v = tok.v.float().to("cuda")
    scale = torch.maximum(v.abs().max(), g.state[slots.tolist()].abs().max())
    assert ((rows - v).abs().max() / scale).item() <= 1e-6
    assert device_errors(g) == 0


@pytest.mark.parametrize("d", [128, 16])
@pytest.mark.parametrize("case", ["channels", "heads"])
def test_prefill_strong_decay_matches_oracle(case, d):
    """Key channels that decay fast within a 16-token block take the exact fp32 path of the
    diagonal blocks: a = 0.3, 0.05 and 1e-3 on a few channels of three heads, and 1e-3 on one
    channel for 40 tokens mid-sequence ("channels"), or on every channel of a head ("heads");
    a = 0.6 sits just inside the fp16 factorisation (16-token decay 2.8e-4 >= 2^-12). Outputs,
    checkpoints and final states against the oracle (no NaN can pass), with a resumed sequence;
    the informational flag is raised and reading the error word clears it. At d = 16 (chunk
    16, fp32 factors) the exact path starts below a chunk decay of 2^-60: a = 0.3 stays on the
    factored path there, 0.05 and 1e-3 take the exact one."""
    H, interval = 4, 128
    lengths = [300, 130, 64]
    rng = np.random.default_rng(960 + len(case) + d)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    ch = ([9, 50], [5, 77], [0, 64, 127], [3, 100], 20) if d == 128 else ([3, 9], [5, 12], [0, 7, 15], [3, 10], 2)
    if case == "channels":
        tok.a[:, 0, ch[0]] = 0.6
        tok.a[:, 1, ch[1]] = 0.3
        tok.a[:, 2, ch[2]] = 0.05
        tok.a[:, 3, ch[3]] = 1e-3
        tok.a[100:140, 0, ch[4]] = 1e-3
    else:
        tok.a[:, 0, :] = 0.6
        tok.a[:, 1, :] = 0.3
        tok.a[:, 2, :] = 0.05
        tok.a[:, 3, :] = 1e-3
    tok.np["a"] = tok.a.to(torch.float64).numpy()
    g, o = pools(12, H, d)
    put_states(g, o, [11], ki.draw_states(rng, 1, H, d, d))
    init, out = [-1, 11, -1], [0, 1, 2]
    n_ck = sum(L // interval for L in lengths)
    cks = list(range(3, 3 + n_ck))
    O = g.kda_prefill(*tok_dev(tok), cu, out, init_slots=init, ckpt_slots=cks, ckpt_interval=interval)
    torch.cuda.synchronize()
    Oo = o.prefill(tok.np, cu, init, out, cks, interval)
    assert torch.isfinite(O.float()).all()
    check_out(O, Oo, cu, v=tok.np["v"])
    check_state(g.state[out + cks], o.state[out + cks], "final and checkpoint states")
    meta_equal(g.meta_array(), o.meta(), out + cks)
    assert g.kda_read_device_error() == kda._abi.KDA_DEVERR_DECAY_RANGE
    assert g.kda_read_device_error() == 0


@pytest.mark.parametrize("d", [128, 16])
def test_prefill_unit_key_readout_through_chunks(d):
    """The readout invariant of the rule through the chunked prefill: with a = 1, b = 1 and a
    unit key, k_t^T S_t = v_t^T after every token whatever the state was, so a query equal to
    the key reads o_t = v_t. Keys repeat from a small set of unit vectors that bf16 holds
    exactly (one-hot, or +-1/2 on four channels), across several chunks and a ragged tail, from
    a random initial state; outputs against v itself and against the oracle, states against the
    oracle."""
    H = 4
    lengths = [200, 64, 37]
    rng = np.random.default_rng(961 + d)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = int(cu[-1])
    tok = ki.draw_tokens(rng, (N,), H, d, d)
    keys = np.zeros((12, d))
    for j in range(6):
        keys[j, rng.integers(d)] = 1.0
        keys[6 + j, rng.choice(d, 4, replace=False)] = 0.5 * rng.choice([-1.0, 1.0], 4)
    k = keys[rng.integers(len(keys), size=(N, H))]
    tok.k = ki.to_bf16(k)
    tok.q = tok.k.clone()
    tok.a.fill_(1.0)
    tok.b.fill_(1.0)
    tok.np.update(q=k.copy(), k=k.copy(), a=np.ones((N, H, d)), b=np.ones((N, H)))
    g, o = pools(8, H, d)
    put_states(g, o, [5, 6, 7], ki.draw_states(rng, 3, H, d, d))
    O = g.kda_prefill(*tok_dev(tok), cu, [0, 1, 2], init_slots=[5, 6, 7])
    torch.cuda.synchronize()
    Oo = o.prefill(tok.np, cu, [5, 6, 7], [0, 1, 2], [], 0)
    check_out(O, tok.np["v"], cu, "o against v", v=tok.np["v"])
    check_out(O, Oo, cu, "o against the oracle", v=tok.np["v"])
    check_state(g.state[[0, 1, 2]], o.state[[0, 1, 2]])
    assert device_errors(g) == 0


@pytest.mark.parametrize("d", [128, 16])
def test_direct_per_draft_checkpoints_match_ring_scheme(d):
    """Direct per-draft state checkpoints beside ReplaySSM: the same outputs as the ring
    verify (bit for bit), draft states equal to the oracle's prefix states, and a direct
    commit that leaves the same state bytes as the ring commit's replay; the ring pointer stays.
    Out-of-range acceptance is clamped and flagged; the two pending kinds do not mix."""
    w = ki.verify_workload(2) if d == 128 else ki.verify_workload(7, B=3, P=5, H=2, d=16, n_slots=8)
    P = w["n_pos"]
    g, o = pools(w["n_slots"], w["H"], w["dk"], w["ring_cap"])
    r, _ = pools(w["n_slots"], w["H"], w["dk"], w["ring_cap"])
    slots = w["slots"]
    put_states(g, o, slots, w["states"])
    r.state.copy_(g.state)
    tok = w["tokens"]
    before = g.state.clone()
    meta_before = g.meta_array().copy()
    O, draft = g.kda_verify_direct(*tok_dev(tok), slots)
    Or = r.kda_verify(*tok_dev(tok), slots)
    Oo, states_o = o.verify_direct(tok.np, slots)
    torch.cuda.synchronize()
    # the direct scheme steps position by position (it stores every draft state); the ring verify
    # of up to 16 positions solves them at once in WY form: both against the oracle
    check_out(O, Oo, v=tok.np["v"])
    check_out(Or, Oo, v=tok.np["v"])
    check_state(draft, states_o)
    assert torch.equal(g.state, before), "direct verify must not write any committed state"
    meta_equal(g.meta_array(), o.meta(), slots)
    assert all(g.host_state(int(s)) == 3 for s in slots)
    with pytest.raises(kda.KDAError):           # a ring commit of a slot pending a direct one
        g.kda_commit(slots, torch.zeros(len(slots), dtype=torch.int32, device="cuda"))

    na_np = w["n_accepted"].copy()
    na_np[-1] = P + 3                           # out of range: clamped to P - 1 and flagged
    na = torch.from_numpy(na_np).to("cuda")
    g.kda_commit_direct(slots, na, draft)
    r.kda_commit(slots, na)
    o.commit_direct(slots, na_np, states_o)
    torch.cuda.synchronize()
    assert torch.equal(g.state, r.state), "direct commit must leave the ring commit's state bytes"
    check_state(g.state[slots.tolist()], o.state[slots])
    meta_equal(g.meta_array(), o.meta(), slots)
    m, mr = g.meta_array(), r.meta_array()
    assert np.array_equal(m[slots, 0], mr[slots, 0])                   # pos advanced alike
    assert np.array_equal(m[slots, 1], meta_before[slots, 1])          # ring_head unchanged
    assert g.kda_read_device_error() == 1 and r.kda_read_device_error() == 1

    # a full reject after a direct verify: state bit-identical, pointers untouched
    snap, msnap = g.state.clone(), g.meta_array().copy()
    g.kda_verify_direct(*tok_dev(tok), slots, draft_states=draft)
    g.kda_rollback(slots)
    torch.cuda.synchronize()
    assert torch.equal(g.state, snap)
    m = g.meta_array()
    assert np.array_equal(m[slots, :3], np.stack([msnap[slots, 0], msnap[slots, 1],
                                                  np.zeros(len(slots), np.int64)], axis=1))
    assert all(g.host_state(int(s)) == 1 for s in slots)
    assert device_errors(g) == 0


def test_commit_out_of_range_acceptance_is_clamped_and_flagged():
    w = ki.verify_workload(5, B=2, P=4)
    g, o = pools(16, w["H"], w["dk"], 9)
    slots = np.array([3, 9], dtype=np.int32)
    put_states(g, o, slots, w["states"])
    g.kda_verify(*tok_dev(w["tokens"]), slots)
    o.verify(w["tokens"].np, slots)
    na = [7, -2]
    g.kda_commit(slots, torch.tensor(na, dtype=torch.int32, device="cuda"))
    o.commit(slots, na)
    assert g.kda_read_device_error() == kda._abi.KDA_DEVERR_NACC_RANGE
    assert o.error_bits == kda._abi.KDA_DEVERR_NACC_RANGE
    check_state(g.state[slots.tolist()], o.state[slots])
    meta_equal(g.meta_array(), o.meta(), slots)
    assert g.kda_read_device_error() == 0     # reading clears the word


def test_ring_wraps_over_many_rounds():
    H, d, R = 4, 128, 9
    g, o = pools(8, H, d, R)
    rng = np.random.default_rng(30)
    slots = np.array([1, 6], dtype=np.int32)
    put_states(g, o, slots, ki.draw_states(rng, 2, H, d, d))
    for r in range(6):
        P = int(rng.integers(1, R + 1))
        tok = ki.draw_tokens(rng, (2, P), H, d, d)
        Og = g.kda_verify(*tok_dev(tok), slots)
        Oo = o.verify(tok.np, slots)
        if r % 3 == 2:
            g.kda_rollback(slots)
            o.rollback(slots)
        else:
            na = rng.integers(0, P, size=2).astype(np.int32)
            g.kda_commit(slots, torch.from_numpy(na).to("cuda"))
            o.commit(slots, na)
        torch.cuda.synchronize()
        check_out(Og, Oo, v=tok.np["v"])
    check_state(g.state[slots.tolist()], o.state[slots])
    meta_equal(g.meta_array(), o.meta(), slots)
    ring_check(g, o, slots)


# ----------------------------------------------------------------------------- prefill

@pytest.mark.parametrize("d", [16, 128])
def test_prefill_ragged_with_resume_and_checkpoints(d):
    """Several sequences with ragged lengths (0, 1, chunk-1, chunk, chunk+1, several chunks),
    some resuming from a slot, checkpoint export at every chunk*2 tokens."""
    C = kda.chunk_for(d)
    H = 4
    lengths = [0, 1, C - 1, C, C + 1, 3 * C + 7, 5 * C]
    n = len(lengths)
    g, o = pools(40, H, d)
    rng = np.random.default_rng(40 + d)
    init = [-1, 20, -1, 21, -1, 22, 23]
    put_states(g, o, [20, 21, 22, 23], ki.draw_states(rng, 4, H, d, d))
    out = [0, 1, 2, 21, 4, 5, 6]            # sequence 3 updates its init slot in place
    interval = 2 * C
    n_ck = sum(L // interval for L in lengths)
    cks = list(range(8, 8 + n_ck))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    O = g.kda_prefill(*tok_dev(tok), cu, out, init_slots=init, ckpt_slots=cks,
                      ckpt_interval=interval)
    Oo = o.prefill(tok.np, cu, init, out, cks, interval)
    torch.cuda.synchronize()
    check_out(O, Oo, cu, v=tok.np["v"])
    for s in out + cks:
        check_state(g.state[s], o.state[s])
    meta_equal(g.meta_array(), o.meta(), out + cks)


def _cat(a: ki.Tokens, b: ki.Tokens) -> ki.Tokens:
    t = ki.Tokens(*(torch.cat([getattr(a, n), getattr(b, n)]) for n in "qkvab"))
    t.np = {n: np.concatenate([a.np[n], b.np[n]]) for n in a.np}
    return t


@pytest.mark.parametrize("match,I", [(0, 1024), (700, 1024), (1024, 1024), (2100, 1024),
                                     (3000, 1024), (2100, 1000)])
def test_prefix_cache_hit_then_speculative_decode(match, I):
    """Partial prefix-cache hit with speculative decode: a cached 3000-token prompt left state
    checkpoints every I tokens; a new prompt shares its first `match` tokens. The request
    slot takes the deepest usable checkpoint (prefix_hit), prefills the rest of its prompt from
    that offset in place, then verifies 1+4 drafts and commits 2. State, outputs and pos must
    match the oracle running the whole new prompt from zero."""
    H, d, L = 4, 128, 3000
    g, o = pools(16, H, d)
    rng = np.random.default_rng(70 + match + I)
    cached = ki.draw_tokens(rng, (L,), H, d, d)
    fresh = ki.draw_tokens(rng, (L,), H, d, d)
    prompt = _cat(cached.slice(0, match), fresh.slice(match, L))
    c_out, ck, req = 0, list(range(1, 1 + L // I)), 10
    g.kda_prefill(*tok_dev(cached), [0, L], [c_out], ckpt_slots=ck, ckpt_interval=I)
    hit = kda.prefix_hit(match, L, I)
    rest = prompt.slice(hit, L)
    if hit:
        g.kda_slot_checkpoint(ck[hit // I - 1], req)
        O = g.kda_prefill(*tok_dev(rest), [0, L - hit], [req], init_slots=[req])
    else:
        O = g.kda_prefill(*tok_dev(rest), [0, L], [req])
    drafts = ki.draw_tokens(rng, (1, 5), H, d, d)
    Ov = g.kda_verify(*tok_dev(drafts), [req])
    g.kda_commit([req], torch.tensor([2], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()

    Oo = o.prefill(prompt.np, [0, L], [-1], [req], [], 0)
    Ovo = o.verify(drafts.np, [req])
    o.commit([req], [2])
    check_out(O, Oo[hit:], [0, L - hit], v=rest.np["v"])
    check_out(Ov, Ovo, v=drafts.np["v"])
    check_state(g.state[req], o.state[req])
    m = g.meta_array()
    assert int(m[req, 0]) == L + 3 and int(m[req, 2]) == 0
    meta_equal(m, o.meta(), [req])
    assert device_errors(g) == 0


@pytest.mark.parametrize("d,interval", [(128, 100), (128, 37), (128, 65), (128, 1000), (16, 10), (16, 24)])
def test_prefill_checkpoints_at_unaligned_intervals(d, interval):
    """Checkpoint intervals that are not a multiple of the chunk: every boundary ends a chunk
    inside the pass (short chunks mid-sequence). Ragged lengths, resumed sequences, all
    checkpoints and outputs against the oracle."""
    H = 4
    lengths = [0, 1, interval - 1, interval, interval + 1, 3 * interval + 7, 7 * interval + 3, 64]
    n = len(lengths)
    g, o = pools(64, H, d)
    rng = np.random.default_rng(80 + d + interval)
    init = [-1, 40, -1, 41, -1, 42, -1, 43]
    put_states(g, o, [40, 41, 42, 43], ki.draw_states(rng, 4, H, d, d))
    out = [0, 1, 2, 41, 4, 5, 6, 7]          # sequence 3 updates its init slot in place
    n_ck = sum(L // interval for L in lengths)
    cks = list(range(8, 8 + n_ck))
    assert 8 + n_ck <= 40
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    O = g.kda_prefill(*tok_dev(tok), cu, out, init_slots=init, ckpt_slots=cks,
                      ckpt_interval=interval)
    Oo = o.prefill(tok.np, cu, init, out, cks, interval)
    torch.cuda.synchronize()
    check_out(O, Oo, cu, v=tok.np["v"])
    for s_ in out + cks:
        check_state(g.state[s_], o.state[s_])
    meta_equal(g.meta_array(), o.meta(), out + cks)
    assert device_errors(g) == 0


@pytest.mark.parametrize("H,n_seq,plan", [(4, 7, [(7, 16)]), (32, 2, [(2, 32)]),
                                           (32, 3, [(1, 32), (2, 64), (3, 128)]),
                                           (32, 9, [(9, 128)])])
def test_prefill_every_slice_width(H, n_seq, plan):
    """Small ragged batches whose state pass runs 16-, 32-, 64- and 128-column slices (on a
    256-CU part; the plan the library reports is pinned); each must match the oracle (every
    head, a resumed first sequence, checkpoints)."""
    rng = np.random.default_rng(60 + H + n_seq)
    lengths = [int(x) for x in rng.integers(1, 300, size=n_seq)]
    lengths[0] = 257
    d = 128
    g, _ = pools(32, H, d)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    assert g.kda_prefill_plan(cu) == plan
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    init = [-1] * n_seq
    init[0] = 31
    st = ki.draw_states(rng, 1, H, d, d)
    g.state[31] = st[0].to("cuda")
    out = list(range(n_seq))
    interval = 128
    n_ck = sum(L // interval for L in lengths)
    cks = list(range(n_seq, n_seq + n_ck))
    O = g.kda_prefill(*tok_dev(tok), cu, out, init_slots=init, ckpt_slots=cks, ckpt_interval=interval)
    torch.cuda.synchronize()
    heads = list(range(H))
    o = OPool(32, len(heads), d, d, 9)
    for _ in range(32):
        o.alloc()
    o.state[31] = st[0][heads].double().numpy()
    Oo = o.prefill(heads_np(tok, heads), cu, init, out, cks, interval)
    check_out(O[:, heads], Oo, cu, v=tok.np["v"])
    for s in out + cks:
        check_state(g.state[s][heads], o.state[s])
    meta_equal(g.meta_array(), o.meta(), out + cks)
    assert device_errors(g) == 0


def test_prefill_full_size_all_heads():
    """One 8192-token prompt, 32 heads, chunk 64, checkpoints every 1024 tokens: outputs,
    the eight checkpoints and the final state of every head against the oracle."""
    w = ki.prefill_workload(3)
    H, d = w["H"], w["dk"]
    tok = w["tokens"]
    n_ck = 8192 // w["ckpt_interval"]
    g, _ = pools(64, H, d)
    out, cks = 0, list(range(1, 1 + n_ck))
    O = g.kda_prefill(*tok_dev(tok), w["cu_seqlens"], [out], ckpt_slots=cks,
                      ckpt_interval=w["ckpt_interval"], chunk=w["chunk"])
    torch.cuda.synchronize()
    heads = list(range(H))
    o = OPool(64, len(heads), d, d, 9)
    for _ in range(64):
        o.alloc()
    Oo = o.prefill(heads_np(tok, heads), w["cu_seqlens"], [-1], [out], cks, w["ckpt_interval"])
    check_out(O[:, heads], Oo, w["cu_seqlens"], v=tok.np["v"])
    for s in [out] + cks:
        check_state(g.state[s][heads], o.state[s])
    meta_equal(g.meta_array(), o.meta(), [out] + cks)
    assert torch.isfinite(O.float()).all()


def test_prefill_is_deterministic():
    w = ki.prefill_workload(7, lengths=(700, 300), H=8, ckpt_interval=128)
    tok = w["tokens"]
    res = []
    for _ in range(2):
        g, _ = pools(16, w["H"], w["dk"])
        O = g.kda_prefill(*tok_dev(tok), w["cu_seqlens"], [0, 1], ckpt_slots=list(range(2, 9)),
                          ckpt_interval=128)
        torch.cuda.synchronize()
        res.append((O.clone(), g.state.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


# ----------------------------------------------------------------------------- plan and workspace

@pytest.mark.parametrize("n_seq,H", [(1500, 2), (9000, 1)])
def test_prefill_many_short_sequences(n_seq, H):
    """More sequences than the plan kernel has threads (several per thread in its scan), and
    more than it orders by length (identity order); empty sequences and two-chunk ones among
    them. Oracle per sequence from a zero state."""
    from oracle import kda_scan
    rng = np.random.default_rng(70 + n_seq)
    lengths = rng.choice([0, 1, 2, 3, 65], size=n_seq, p=[0.2, 0.3, 0.2, 0.2, 0.1])
    d = 128
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    g = kda.KDAPool(n_seq, H, d)
    for _ in range(n_seq):
        g.kda_slot_alloc()
    O = g.kda_prefill(*tok_dev(tok), cu, list(range(n_seq)))
    torch.cuda.synchronize()
    t = tok.np
    Oo = np.zeros((int(cu[-1]), H, d))
    sample = set(rng.choice(n_seq, size=40, replace=False).tolist()) | {int(np.argmax(lengths))}
    S_ref = {}
    for i in range(n_seq):
        lo, hi = int(cu[i]), int(cu[i + 1])
        if hi == lo and i not in sample:
            continue
        S, Oi, _ = kda_scan(np.zeros((H, d, d)), t["q"][lo:hi], t["k"][lo:hi], t["v"][lo:hi],
                            t["a"][lo:hi], t["b"][lo:hi])
        Oo[lo:hi] = Oi
        if i in sample:
            S_ref[i] = S
    check_out(O, Oo, cu, v=t["v"])
    for i, S in S_ref.items():
        check_state(g.state[i], S)
    meta = g.meta_array()
    np.testing.assert_array_equal(meta[:, 0], lengths)
    assert device_errors(g) == 0



@pytest.mark.parametrize("n_seq", [63, 64, 65])
def test_prefill_plan_inside_and_outside_the_operand_kernel(n_seq):
    """Up to 64 sequences the operand kernel plans the batch itself (one lane per sequence);
    from 65 on the plan kernel does. Both sides of the boundary, with resumed sequences,
    checkpoints every 128 tokens, ties in length and empty sequences: outputs, final and
    checkpoint states against the oracle, checkpoint metadata exact."""
    rng = np.random.default_rng(900 + n_seq)
    H, d, interval = 2, 128, 128
    lengths = [int(x) for x in rng.choice([0, 5, 64, 130, 300, 700], size=n_seq)]
    lengths[0], lengths[1] = 700, 700    # a tie for the longest
    n_ck = sum(L // interval for L in lengths)
    n_slots = 2 * n_seq + n_ck
    g, o = pools(n_slots, H, d)
    init = [i if i % 3 == 0 else -1 for i in range(n_seq)]
    states = ki.draw_states(rng, n_seq, H, d, d)
    put_states(g, o, range(n_seq), states)
    out = list(range(n_seq, 2 * n_seq))
    cks = list(range(2 * n_seq, n_slots))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    O = g.kda_prefill(*tok_dev(tok), cu, out, init_slots=init, ckpt_slots=cks,
                      ckpt_interval=interval)
    torch.cuda.synchronize()
    Oo = o.prefill(tok.np, cu, init, out, cks, interval)
    check_out(O, Oo, cu, v=tok.np["v"])
    for s_ in out + cks:
        check_state(g.state[s_], o.state[s_])
    meta_equal(g.meta_array(), o.meta(), out + cks)
    assert device_errors(g) == 0


def test_prefill_only_empty_sequences():
    """A batch whose sequences are all empty has no chunk: the plan kernel runs, no operand
    kernel, and the state pass copies each init state (or zero) to its out slot."""
    rng = np.random.default_rng(77)
    H, d = 4, 128
    g, o = pools(8, H, d)
    put_states(g, o, [0, 1], ki.draw_states(rng, 2, H, d, d))
    cu = np.zeros(4, np.int32)
    tok = ki.draw_tokens(rng, (0,), H, d, d)
    g.kda_prefill(*tok_dev(tok), cu, [4, 5, 6], init_slots=[0, -1, 1])
    torch.cuda.synchronize()
    o.prefill(tok.np, cu, [0, -1, 1], [4, 5, 6], [], 0)
    for s_ in (4, 5, 6):
        np.testing.assert_array_equal(f64(g.state[s_]), o.state[s_])
    meta_equal(g.meta_array(), o.meta(), [4, 5, 6])
    assert device_errors(g) == 0

def test_prefill_one_long_and_five_short():
    """One long prompt (not first in the batch) and five short ones at 32 heads: the long one
    starts first and the short ones share the remaining CUs. Checkpoints, a resumed short
    sequence and the outputs must match the oracle."""
    rng = np.random.default_rng(85)
    H, d = 32, 128
    lengths = [600, 3000, 600, 600, 600, 600]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    g, _ = pools(40, H, d)
    st = ki.draw_states(rng, 1, H, d, d)
    g.state[39] = st[0].to("cuda")
    init = [-1, -1, 39, -1, -1, -1]
    out = list(range(6))
    interval = 512
    n_ck = sum(L // interval for L in lengths)
    cks = list(range(6, 6 + n_ck))
    O = g.kda_prefill(*tok_dev(tok), cu, out, init_slots=init, ckpt_slots=cks, ckpt_interval=interval)
    torch.cuda.synchronize()
    heads = list(range(H))
    o = OPool(40, len(heads), d, d, 9)
    for _ in range(40):
        o.alloc()
    o.state[39] = st[0][heads].double().numpy()
    Oo = o.prefill(heads_np(tok, heads), cu, init, out, cks, interval)
    check_out(O[:, heads], Oo, cu, v=tok.np["v"])
    for s_ in out + cks:
        check_state(g.state[s_][heads], o.state[s_])
    meta_equal(g.meta_array(), o.meta(), out + cks)
    assert device_errors(g) == 0



@pytest.mark.parametrize("lengths,plan", [
    ([1024] * 8, [(8, 128)]),
    ([300, 8000, 200, 100, 50, 10], [(1, 32), (6, 128)]),
    ([1423, 1318, 1801, 1475, 4580, 5719], [(1, 32), (2, 64), (6, 128)]),
])
def test_prefill_planned_slice_widths(lengths, plan):
    """Batches whose state pass runs one, two and three groups of slice widths in one launch
    (longest sequences in the narrowest slices, short ones in 128-column work-groups): the
    plan the library reports, and outputs, final and checkpoint states of every head against
    the oracle, with a resumed sequence and checkpoints every 1024 tokens."""
    rng = np.random.default_rng(sum(lengths) % 1000)
    H, d, interval = 32, 128, 1024
    n_seq = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    n_ck = sum(L // interval for L in lengths)
    n_slots = n_seq + n_ck + 1
    g, _ = pools(n_slots, H, d)
    assert g.kda_prefill_plan(cu) == plan
    st = ki.draw_states(rng, 1, H, d, d)
    g.state[n_slots - 1] = st[0].to("cuda")
    init = [-1] * n_seq
    init[n_seq - 1] = n_slots - 1
    out = list(range(n_seq))
    cks = list(range(n_seq, n_seq + n_ck))
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    O = g.kda_prefill(*tok_dev(tok), cu, out, init_slots=init, ckpt_slots=cks, ckpt_interval=interval)
    torch.cuda.synchronize()
    heads = list(range(H))
    o = OPool(n_slots, len(heads), d, d, 9)
    for _ in range(n_slots):
        o.alloc()
    o.state[n_slots - 1] = st[0][heads].double().numpy()
    Oo = o.prefill(heads_np(tok, heads), cu, init, out, cks, interval)
    check_out(O[:, heads], Oo, cu, v=tok.np["v"])
    for s_ in out + cks:
        check_state(g.state[s_][heads], o.state[s_])
    meta_equal(g.meta_array(), o.meta(), out + cks)
    assert device_errors(g) == 0

def test_prefill_without_workspace_is_rejected():
    """workspace = NULL through the C ABI: KDA_EWORKSPACE, nothing launched (outputs and
    states untouched); the same call with the binding's workspace then runs."""
    from ctypes import byref
    from recurrent_linear_attention_amd import _abi
    from recurrent_linear_attention_amd.pool import _ix, _stream
    rng = np.random.default_rng(80)
    H, d = 4, 128
    g = kda.KDAPool(8, H, d)
    for _ in range(8):
        g.kda_slot_alloc()
    cu = np.array([0, 300, 300, 429], dtype=np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    q, k, v, a, b = tok_dev(tok)
    O = torch.zeros((int(cu[-1]), H, d), dtype=torch.bfloat16, device="cuda")
    before = g.state.clone()
    args = g._prefill_struct(int(cu[-1]), _ix(cu, g.device), None, _ix([0, 1, 2], g.device), None,
                             64, 0, g._tok_ptrs(q, k, v, a, b, O))
    args.workspace, args.workspace_bytes = None, 0
    assert _abi.lib.kda_prefill(g.handle, byref(args), _stream(None)) == _abi.KDA_EWORKSPACE
    torch.cuda.synchronize()
    assert not O.any() and torch.equal(g.state, before)
    g.kda_prefill(q, k, v, a, b, cu, [0, 1, 2], o=O)
    torch.cuda.synchronize()
    assert O.float().abs().sum() > 0


def test_mixed_batch_without_side_stream_matches_forked():
    """kda_mixed_batch with no side stream runs commit, decode and verify in order on the
    caller's stream ahead of the prefill; every output, state, ring entry and metadata field is
    bit-identical to the forked schedule on the binding's side stream."""
    H, d, P = 4, 128, 5
    rng = np.random.default_rng(33)
    ds, vs = [3, 4, 9], [6, 7]
    st = ki.draw_states(rng, 5, H, d, d)
    lens = [300, 129, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]) + len(ds) + len(vs) * P,), H, d, d)
    res = []
    for side in (True, False):
        g, o = pools(12, H, d)
        put_states(g, o, ds + vs, st)
        O = g.kda_mixed_batch(*tok_dev(tok), cu, [0, 1, 2], ds, vs, P, fork=side)
        torch.cuda.synchronize()
        res.append((O.clone(), g.state.clone(), [t.clone() for t in g.ring_tensors()], g.meta_array()))
    (O1, S1, R1, M1), (O2, S2, R2, M2) = res
    assert torch.equal(O1, O2)
    assert torch.equal(S1, S2)
    assert all(torch.equal(a_, b_) for a_, b_ in zip(R1, R2))
    assert np.array_equal(M1, M2)


@pytest.mark.parametrize("d,H", [(128, 3), (128, 5), (16, 5), (16, 1)])
def test_odd_head_counts_through_every_path(d, H):
    """Head counts that are not a multiple of the eight XCDs (the state pass rounds each width
    group's grid up and idles the spare work-groups; the step kernels tile heads by slot):
    a mixed batch (three ragged prompts, one resumed, checkpoints; decodes; verifies of 1+4),
    then the verifies' commit and a decode of the committed slots, each against the oracle."""
    P, interval = 5, (128 if d == 128 else 32)
    rng = np.random.default_rng(400 + 10 * H + d)
    lens = [200, 67, 130] if d == 128 else [50, 17, 33]
    ds, vs = [3, 4], [6, 7, 8]
    n_ck = sum(L // interval for L in lens)
    n_slots = 10 + n_ck
    g, o = pools(n_slots, H, d, P)
    put_states(g, o, ds + vs + [9], ki.draw_states(rng, 6, H, d, d))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out, init = [0, 1, 2], [9, -1, -1]
    cks = list(range(10, 10 + n_ck))
    n_pre = int(cu[-1])
    tok = ki.draw_tokens(rng, (n_pre + len(ds) + len(vs) * P,), H, d, d)
    O = g.kda_mixed_batch(*tok_dev(tok), cu, out, ds, vs, P, init_slots=init, ckpt_slots=cks,
                          ckpt_interval=interval)
    torch.cuda.synchronize()
    Op = o.prefill(tok.slice(0, n_pre).np, cu, init, out, cks, interval)
    Od = o.decode(tok.slice(n_pre, n_pre + len(ds)).np, ds)
    vt = {n: x[n_pre + len(ds):].reshape((len(vs), P) + x.shape[1:]) for n, x in tok.np.items()}
    Ov = o.verify(vt, vs)
    check_out(O[:n_pre], Op, cu, v=tok.np["v"][:n_pre])
    check_out(O[n_pre:n_pre + len(ds)], Od, v=tok.np["v"][n_pre:n_pre + len(ds)])
    check_out(O[n_pre + len(ds):].reshape(len(vs), P, H, d), Ov,
              v=tok.np["v"][n_pre + len(ds):].reshape(len(vs), P, H, d))
    for s in out + cks + ds:
        check_state(g.state[s], o.state[s])
    ring_check(g, o, vs)
    meta_equal(g.meta_array(), o.meta(), range(n_slots))
    na = np.array([4, 0, 2], dtype=np.int32)
    g.kda_commit(vs, torch.from_numpy(na).to("cuda"))
    o.commit(vs, na)
    t2 = ki.draw_tokens(rng, (len(vs),), H, d, d)
    O2 = g.kda_decode(*tok_dev(t2), vs)
    O2o = o.decode(t2.np, vs)
    torch.cuda.synchronize()
    check_out(O2, O2o, v=t2.np["v"])
    for s in vs:
        check_state(g.state[s], o.state[s])
    meta_equal(g.meta_array(), o.meta(), range(n_slots))
    assert device_errors(g) == 0


def test_mixed_batch_without_prefill():
    """Only decode and verify parts: they run on the caller's stream, as separate calls would."""
    H, d, P = 4, 128, 5
    g, o = pools(8, H, d)
    rng = np.random.default_rng(90)
    ds, vs = [1, 4, 6], [0, 7]
    put_states(g, o, ds + vs, ki.draw_states(rng, 5, H, d, d))
    tok = ki.draw_tokens(rng, (len(ds) + len(vs) * P,), H, d, d)
    O = g.kda_mixed_batch(*tok_dev(tok), [0], [], ds, vs, P)
    torch.cuda.synchronize()
    Od = o.decode(tok.slice(0, len(ds)).np, ds)
    vt = {n: x[len(ds):].reshape((len(vs), P) + x.shape[1:]) for n, x in tok.np.items()}
    Ov = o.verify(vt, vs)
    check_out(O[:len(ds)], Od, v=tok.np["v"][:len(ds)])
    check_out(O[len(ds):].reshape(len(vs), P, H, d), Ov, v=tok.np["v"][len(ds):].reshape(len(vs), P, H, d))
    check_state(g.state[ds], o.state[ds])
    meta_equal(g.meta_array(), o.meta(), ds + vs)
    ring_check(g, o, vs)


# ----------------------------------------------------------------------------- mixed batch

def test_mixed_batch_full_size():
    """The mixed 16384-token batch (6 prompts, 32 decodes, 4 verifies of 1+8) at 32 heads: every
    part of every head against the oracle, then the verify part's commit."""
    w = ki.mixed_workload(4)
    H, d, P = w["H"], w["dk"], w["n_pos"]
    g, o_all = pools(w["n_slots"], H, d, w["ring_cap"])
    ds, vs, ps = w["decode_slots"], w["verify_slots"], w["prefill_slots"]
    put_states(g, o_all, np.concatenate([ds, vs]), w["states"])
    tok = w["tokens"]
    O = g.kda_mixed_batch(*tok_dev(tok), w["cu_seqlens"], ps, ds, vs, P)
    torch.cuda.synchronize()
    n_pre = w["cu_seqlens"][-1]
    nd = w["n_decode"]
    # decode + verify parts: every head through the oracle
    Od = o_all.decode(tok.slice(n_pre, n_pre + nd).np, ds)
    vt = {n: x[n_pre + nd:].reshape((w["n_verify"], P) + x.shape[1:])
          for n, x in tok.np.items()}
    Ov = o_all.verify(vt, vs)
    check_out(O[n_pre:n_pre + nd], Od, v=tok.np["v"][n_pre:n_pre + nd])
    check_out(O[n_pre + nd:].reshape(w["n_verify"], P, H, d), Ov, v=tok.np["v"][n_pre + nd:].reshape(w["n_verify"], P, H, d))
    check_state(g.state[ds.tolist()], o_all.state[ds])
    meta_equal(g.meta_array(), o_all.meta(), np.concatenate([ds, vs]))
    ring_check(g, o_all, vs)
    # prefill part: every head
    heads = list(range(H))
    o = OPool(w["n_slots"], len(heads), d, d, 9)
    for _ in range(w["n_slots"]):
        o.alloc()
    pre = tok.slice(0, n_pre)
    Op = o.prefill(heads_np(pre, heads), w["cu_seqlens"], [-1] * len(ps), ps, [], 0)
    check_out(O[:n_pre, heads], Op, w["cu_seqlens"], v=tok.np["v"][:n_pre])
    for s in ps:
        check_state(g.state[int(s)][heads], o.state[s])
    # commit the verify part as the next step would
    na = torch.from_numpy(w["n_accepted"]).to("cuda")
    g.kda_commit(vs, na)
    o_all.commit(vs, w["n_accepted"])
    torch.cuda.synchronize()
    check_state(g.state[vs.tolist()], o_all.state[vs])
    assert device_errors(g) == 0



def test_mixed_batch_decode_heavy():
    """A mixed batch whose side-stream work (a commit, 64 decodes and 8 verifies of 1+8)
    outlasts its short prefill's operand kernel, so the state pass runs beside it: every part
    against the oracle, all heads."""
    rng = np.random.default_rng(321)
    H, d, P = 4, 128, 9
    lengths = [65, 1]
    n_dec, n_ver = 64, 8
    n_slots = 2 + n_dec + n_ver
    g, o = pools(n_slots, H, d, R=P)
    ps = np.arange(2)
    ds = np.arange(2, 2 + n_dec)
    vs = np.arange(2 + n_dec, n_slots)
    put_states(g, o, np.concatenate([ds, vs]), ki.draw_states(rng, n_dec + n_ver, H, d, d))
    # a first verify on vs, committed by the batch below ahead of its own verify
    t0 = ki.draw_tokens(rng, (n_ver, P), H, d, d)
    g.kda_verify(*tok_dev(t0), vs)
    o.verify(t0.np, vs)
    na = rng.integers(0, P, size=n_ver).astype(np.int32)
    o.commit(vs, na)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    n_pre = int(cu[-1])
    tok = ki.draw_tokens(rng, (n_pre + n_dec + n_ver * P,), H, d, d)
    O = g.kda_mixed_batch(*tok_dev(tok), cu, ps, ds, vs, P, commit_slots=vs,
                          n_accepted=torch.from_numpy(na).to("cuda"))
    Op = o.prefill(tok.slice(0, n_pre).np, cu, [-1, -1], ps, [], 0)
    Od = o.decode(tok.slice(n_pre, n_pre + n_dec).np, ds)
    vt = {k_: x[n_pre + n_dec:].reshape((n_ver, P) + x.shape[1:]) for k_, x in tok.np.items()}
    Ov = o.verify(vt, vs)
    torch.cuda.synchronize()
    check_out(O[:n_pre], Op, cu, v=tok.np["v"][:n_pre])
    check_out(O[n_pre:n_pre + n_dec], Od, v=tok.np["v"][n_pre:n_pre + n_dec])
    check_out(O[n_pre + n_dec:].reshape(n_ver, P, H, d), Ov, v=tok.np["v"][n_pre + n_dec:].reshape(n_ver, P, H, d))
    for s_ in np.concatenate([ps, ds, vs]):
        check_state(g.state[int(s_)], o.state[s_])
    meta_equal(g.meta_array(), o.meta(), np.arange(n_slots))
    ring_check(g, o, vs)
    assert device_errors(g) == 0


def test_mixed_batch_many_prefills():
    """A mixed batch with 70 prompts (more than the operand kernel plans itself: the plan
    kernel runs on the caller's stream) next to decodes and a verify on the side stream:
    every part against the oracle, all heads (H = 4, short ragged prompts)."""
    rng = np.random.default_rng(123)
    H, d, P = 4, 128, 3
    lengths = [int(x) for x in rng.choice([0, 1, 7, 64, 65, 200], size=70)]
    n_dec, n_ver = 5, 2
    n_slots = 70 + n_dec + n_ver
    g, o = pools(n_slots, H, d, R=P)
    ps = np.arange(70)
    ds = np.arange(70, 70 + n_dec)
    vs = np.arange(70 + n_dec, n_slots)
    put_states(g, o, np.concatenate([ds, vs]), ki.draw_states(rng, n_dec + n_ver, H, d, d))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    n_pre = int(cu[-1])
    tok = ki.draw_tokens(rng, (n_pre + n_dec + n_ver * P,), H, d, d)
    O = g.kda_mixed_batch(*tok_dev(tok), cu, ps, ds, vs, P)
    torch.cuda.synchronize()
    Op = o.prefill(tok.slice(0, n_pre).np, cu, [-1] * 70, ps, [], 0)
    Od = o.decode(tok.slice(n_pre, n_pre + n_dec).np, ds)
    vt = {n: x[n_pre + n_dec:].reshape((n_ver, P) + x.shape[1:]) for n, x in tok.np.items()}
    Ov = o.verify(vt, vs)
    check_out(O[:n_pre], Op, cu, v=tok.np["v"][:n_pre])
    check_out(O[n_pre:n_pre + n_dec], Od, v=tok.np["v"][n_pre:n_pre + n_dec])
    check_out(O[n_pre + n_dec:].reshape(n_ver, P, H, d), Ov, v=tok.np["v"][n_pre + n_dec:].reshape(n_ver, P, H, d))
    for s_ in np.concatenate([ps, ds]):
        check_state(g.state[int(s_)], o.state[s_])
    meta_equal(g.meta_array(), o.meta(), np.arange(n_slots))
    ring_check(g, o, vs)
    assert device_errors(g) == 0

@pytest.mark.parametrize("d", [128, 16])
def test_mixed_batch_commits_previous_verify(d):
    """Two serving steps: the second mixed batch commits the first one's verified drafts (its
    commit part) before verifying the same slots again, next to a new prefill and decodes.
    Every output, state and metadata entry against the oracle applying the same operations in
    order, at d = 128 (chunk 64) and d = 16 (chunk 16)."""
    H, P = 4, 5
    g, o = pools(32, H, d)
    rng = np.random.default_rng(90)
    ds, vs = np.array([3, 7, 11], np.int32), np.array([5, 20], np.int32)
    put_states(g, o, np.concatenate([ds, vs]), ki.draw_states(rng, 5, H, d, d))

    def step(pre_len, out, commit, n_acc):
        cu = np.concatenate([[0], np.cumsum(pre_len)]).astype(np.int32)
        n_pre = int(cu[-1])
        tok = ki.draw_tokens(rng, (n_pre + len(ds) + len(vs) * P,), H, d, d)
        kw = {}
        if commit is not None:
            kw = dict(commit_slots=commit, n_accepted=torch.tensor(n_acc, dtype=torch.int32, device="cuda"))
            o.commit(commit, n_acc)
        O = g.kda_mixed_batch(*tok_dev(tok), cu, out, ds, vs, P, **kw)
        Op = o.prefill(tok.slice(0, n_pre).np, cu, [-1] * len(out), out, [], 0)
        Od = o.decode(tok.slice(n_pre, n_pre + len(ds)).np, ds)
        vt = {n: x[n_pre + len(ds):].reshape((len(vs), P) + x.shape[1:]) for n, x in tok.np.items()}
        Ov = o.verify(vt, vs)
        torch.cuda.synchronize()
        check_out(O[:n_pre], Op, cu, v=tok.np["v"][:n_pre])
        check_out(O[n_pre:n_pre + len(ds)], Od, v=tok.np["v"][n_pre:n_pre + len(ds)])
        check_out(O[n_pre + len(ds):].reshape(len(vs), P, H, d), Ov, v=tok.np["v"][n_pre + len(ds):].reshape(len(vs), P, H, d))

    step([300, 100], [0, 1], None, None)
    step([200, 257], [2, 4], vs, [3, 0])
    touched = [0, 1, 2, 4] + ds.tolist() + vs.tolist()
    for s_ in touched:
        check_state(g.state[s_], o.state[s_])
    meta_equal(g.meta_array(), o.meta(), touched)
    ring_check(g, o, vs)
    assert all(g.host_state(int(s_)) == 2 for s_ in vs)
    assert device_errors(g) == 0


def test_mixed_batches_hand_slots_between_streams():
    """Two mixed batches enqueued back to back with no host synchronisation between them, each
    stream reading what the other wrote in the batch before: the second batch decodes the slots
    the first one prefilled (caller's stream, then side stream: ordered by the fork event),
    resumes prefills from the slots the first one decoded (side stream, then caller's stream:
    ordered by the join event), and commits and re-verifies the first one's verified slot.
    Outputs, states and metadata against the oracle applying the same operations in order."""
    H, d, P = 4, 128, 5
    g, o = pools(32, H, d)
    rng = np.random.default_rng(95)
    ds1, vs1 = [10, 11], [20]
    put_states(g, o, ds1 + vs1, ki.draw_states(rng, 3, H, d, d))

    def cu_of(lens):
        return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)

    def parts(tok, n_pre, nd, nv):
        vt = {n: x[n_pre + nd:].reshape((nv, P) + x.shape[1:]) for n, x in tok.np.items()}
        return tok.slice(0, n_pre).np, tok.slice(n_pre, n_pre + nd).np, vt

    cu1, out1 = cu_of([300, 150]), [0, 1]
    n1 = int(cu1[-1])
    tok1 = ki.draw_tokens(rng, (n1 + len(ds1) + len(vs1) * P,), H, d, d)
    O1 = g.kda_mixed_batch(*tok_dev(tok1), cu1, out1, ds1, vs1, P)
    cu2, init2, out2, ds2, vs2 = cu_of([200, 70]), [10, 11], [12, 13], [0, 1], [20]
    n2 = int(cu2[-1])
    na = [2]
    tok2 = ki.draw_tokens(rng, (n2 + len(ds2) + len(vs2) * P,), H, d, d)
    O2 = g.kda_mixed_batch(*tok_dev(tok2), cu2, out2, ds2, vs2, P, init_slots=init2,
                           commit_slots=vs2, n_accepted=torch.tensor(na, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()

    p1, d1, v1 = parts(tok1, n1, len(ds1), len(vs1))
    Op1, Od1, Ov1 = o.prefill(p1, cu1, [-1, -1], out1, [], 0), o.decode(d1, ds1), o.verify(v1, vs1)
    o.commit(vs2, na)
    p2, d2, v2 = parts(tok2, n2, len(ds2), len(vs2))
    Op2, Od2, Ov2 = o.prefill(p2, cu2, init2, out2, [], 0), o.decode(d2, ds2), o.verify(v2, vs2)
    for O, n, cu, Op, Od, Ov, tok, nd in ((O1, n1, cu1, Op1, Od1, Ov1, tok1, len(ds1)),
                                          (O2, n2, cu2, Op2, Od2, Ov2, tok2, len(ds2))):
        vv = tok.np["v"]
        check_out(O[:n], Op, cu, v=vv[:n])
        check_out(O[n:n + nd], Od, v=vv[n:n + nd])
        check_out(O[n + nd:].reshape(1, P, H, d), Ov, v=vv[n + nd:].reshape(1, P, H, d))
    touched = out1 + ds1 + vs1 + out2
    for s_ in touched:
        check_state(g.state[s_], o.state[s_])
    meta_equal(g.meta_array(), o.meta(), touched)
    ring_check(g, o, vs2)
    assert device_errors(g) == 0


def test_mixed_batch_is_deterministic():
    """The same mixed batch (prefill on the caller's stream, commit / decode / verify on the
    side stream) on two pools with the same contents gives the same bytes: outputs, states,
    ring entries and metadata."""
    H, d, P = 4, 128, 5
    rng = np.random.default_rng(31)
    ds, vs = [3, 4, 9], [6, 7]
    st = ki.draw_states(rng, 5, H, d, d)
    lens = [300, 129, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]) + len(ds) + len(vs) * P,), H, d, d)
    res = []
    for _ in range(2):
        g, o = pools(12, H, d)
        put_states(g, o, ds + vs, st)
        O = g.kda_mixed_batch(*tok_dev(tok), cu, [0, 1, 2], ds, vs, P)
        torch.cuda.synchronize()
        res.append((O.clone(), g.state.clone(), [t.clone() for t in g.ring_tensors()], g.meta_array()))
    (O1, S1, R1, M1), (O2, S2, R2, M2) = res
    assert torch.equal(O1, O2)
    assert torch.equal(S1, S2)
    assert all(torch.equal(a, b) for a, b in zip(R1, R2))
    assert np.array_equal(M1, M2)


def test_mixed_batch_rejected_keeps_commit_pending():
    """A mixed batch rejected after its commit part passed validation (a decode slot that is
    also a prefill out slot) launches nothing: the commit slots stay pending, no state or ring
    entry changes, and the commit then runs as usual."""
    H, d, P = 4, 128, 3
    g, o = pools(8, H, d)
    rng = np.random.default_rng(77)
    vs = np.array([5, 6], dtype=np.int32)
    put_states(g, o, vs, ki.draw_states(rng, 2, H, d, d))
    vt = ki.draw_tokens(rng, (2, P), H, d, d)
    g.kda_verify(*tok_dev(vt), vs)
    o.verify(vt.np, vs)
    torch.cuda.synchronize()
    tok = ki.draw_tokens(rng, (21,), H, d, d)
    na = np.array([1, 2], dtype=np.int32)
    na_dev = torch.from_numpy(na).to("cuda")
    before = g.state.clone()
    ring_before = [t.clone() for t in g.ring_tensors()]
    meta_before = g.meta_array().copy()
    with pytest.raises(kda.KDAError):
        g.kda_mixed_batch(*tok_dev(tok), [0, 20], [1], [1], [], P, commit_slots=vs, n_accepted=na_dev)
    torch.cuda.synchronize()
    assert all(g.host_state(int(s_)) == 2 for s_ in vs)
    assert torch.equal(g.state, before)
    assert all(torch.equal(a, b) for a, b in zip(g.ring_tensors(), ring_before))
    assert np.array_equal(g.meta_array(), meta_before)
    g.kda_commit(vs, na_dev)
    o.commit(vs, na)
    torch.cuda.synchronize()
    check_state(g.state[vs.tolist()], o.state[vs])
    meta_equal(g.meta_array(), o.meta(), vs)
    assert device_errors(g) == 0


# ----------------------------------------------------------------------------- slot ops

def test_slot_reset_and_checkpoint_copy():
    H, d = 4, 128
    g, o = pools(8, H, d)
    rng = np.random.default_rng(50)
    put_states(g, o, [2, 5], ki.draw_states(rng, 2, H, d, d))
    tok = ki.draw_tokens(rng, (2,), H, d, d)
    g.kda_decode(*tok_dev(tok), [2, 5])
    o.decode(tok.np, [2, 5])
    g.kda_slot_checkpoint(2, 7)
    o.checkpoint(2, 7)
    g.kda_slot_reset(5)
    o.reset(5)
    torch.cuda.synchronize()
    assert torch.equal(g.state[7], g.state[2])
    assert not g.state[5].any()
    meta_equal(g.meta_array(), o.meta(), [2, 5, 7])


# ----------------------------------------------------------------------------- large pool

def test_large_pool_high_slot_indices():
    """An 8192-slot pool at H = 32, d = 128 (16 GiB of fp32 state, 2.4 GB of ring): decode,
    verify of 1+8 and its commit, a resumed prefill with in-pass checkpoints, and a slot
    checkpoint copy, on slots whose state lies past 2^31 floats and 2^31 bytes of the pool,
    against the oracle on a compact pool holding the same slots' contents."""
    H, d, n, R = 32, 128, 8192, 9
    g = kda.KDAPool(n, H, d, R)
    for _ in range(n):
        g.kda_slot_alloc()
    dec, ver, pre_init = [8191, 6000, 4100], [8190, 5001], 6001
    pre_out, cks, cp_dst = [8189, 4099], [8100, 8101, 8102], 100
    used = dec + ver + [pre_init] + pre_out + cks + [cp_dst]
    m = {s: i for i, s in enumerate(used)}
    o = OPool(len(used), H, d, d, R)
    for _ in used:
        o.alloc()
    om = lambda slots: [m[s] for s in slots]  # noqa: E731
    rng = np.random.default_rng(8192)
    seeded = dec + ver + [pre_init]
    st = ki.draw_states(rng, len(seeded), H, d, d)
    g.state[seeded] = st.to("cuda")
    o.state[om(seeded)] = st.double().numpy()

    def same_meta(slots):
        np.testing.assert_array_equal(g.meta_array()[slots], o.meta()[om(slots)])

    tok = ki.draw_tokens(rng, (len(dec),), H, d, d)
    O = g.kda_decode(*tok_dev(tok), dec)
    Oo = o.decode(tok.np, om(dec))
    torch.cuda.synchronize()
    check_out(O, Oo, v=tok.np["v"])
    for s in dec:
        check_state(g.state[s], o.state[m[s]])

    P = 9
    vt = ki.draw_tokens(rng, (len(ver), P), H, d, d)
    Ov = g.kda_verify(*tok_dev(vt), ver)
    Ovo = o.verify(vt.np, om(ver))
    torch.cuda.synchronize()
    check_out(Ov, Ovo, v=vt.np["v"])
    na = np.array([8, 3], dtype=np.int32)
    g.kda_commit(ver, torch.from_numpy(na).to("cuda"))
    o.commit(om(ver), na)
    torch.cuda.synchronize()
    for s in ver:
        check_state(g.state[s], o.state[m[s]])

    lens, interval = [700, 300], 256
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pt = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    Op = g.kda_prefill(*tok_dev(pt), cu, pre_out, init_slots=[pre_init, -1], ckpt_slots=cks,
                       ckpt_interval=interval)
    Opo = o.prefill(pt.np, cu, [m[pre_init], -1], om(pre_out), om(cks), interval)
    torch.cuda.synchronize()
    check_out(Op, Opo, cu, v=pt.np["v"])
    for s in pre_out + cks:
        check_state(g.state[s], o.state[m[s]])

    g.kda_slot_checkpoint(8189, cp_dst)
    o.checkpoint(m[8189], m[cp_dst])
    torch.cuda.synchronize()
    assert torch.equal(g.state[cp_dst], g.state[8189])
    same_meta(used)
    assert device_errors(g) == 0


def test_prefill_long_prompt():
    """One 65536-token prompt (1024 chunks in one chain) at H = 8, resumed from a slot, with a
    checkpoint every 8192 tokens: outputs, the 8 checkpoints and the final state of two heads
    against the oracle, every head finite."""
    H, d, L, interval = 8, 128, 65536, 8192
    rng = np.random.default_rng(65536)
    n_ck = L // interval
    g, _ = pools(n_ck + 2, H, d)
    cu = np.array([0, L], dtype=np.int32)
    init, out, cks = n_ck + 1, 0, list(range(1, n_ck + 1))
    st = ki.draw_states(rng, 1, H, d, d)
    g.state[init] = st[0].to("cuda")
    tok = ki.draw_tokens(rng, (L,), H, d, d)
    O = g.kda_prefill(*tok_dev(tok), cu, [out], init_slots=[init], ckpt_slots=cks,
                      ckpt_interval=interval)
    torch.cuda.synchronize()
    assert torch.isfinite(O.float()).all() and torch.isfinite(g.state[[out] + cks]).all()
    heads = [0, 5]
    o = OPool(n_ck + 2, len(heads), d, d, 9)
    for _ in range(n_ck + 2):
        o.alloc()
    o.state[init] = st[0][heads].double().numpy()
    Oo = o.prefill(heads_np(tok, heads), cu, [init], [out], cks, interval)
    check_out(O[:, heads], Oo, cu, v=tok.np["v"][:, heads])
    for s in [out] + cks:
        check_state(g.state[s][heads], o.state[s])
    assert torch.equal(g.state[cks[-1]], g.state[out])   # the last boundary is the prompt's end
    assert device_errors(g) == 0


@pytest.mark.parametrize("seed", range(32))
def test_mixed_batches_random_shapes(seed):
    """Two serving steps of mixed batches with shapes drawn at random: head count 1-8, d = 16
    or 128, 0-4 prompts of 0-300 tokens (some resumed from a slot, checkpoints at a random
    interval), 0-4 decodes, 1-3 verifies of 1-9 positions; the second step commits the first
    one's verifies with random accepted counts and verifies some of those slots again. Every
    output, state, ring entry and metadata field against the oracle after each step."""
    rng = np.random.default_rng(9000 + seed)
    d = int(rng.choice([16, 128]))
    H = int(rng.integers(1, 9))
    P = int(rng.integers(1, 10))
    R = max(P, 9)
    n_slots = 192   # 12 seeded, and per step up to 4 out slots and 72 checkpoint slots
    g, o = pools(n_slots, H, d, R)
    free = list(rng.permutation(n_slots))
    take = lambda n: [int(free.pop()) for _ in range(n)]  # noqa: E731
    seeded = take(12)
    st = ki.draw_states(rng, len(seeded), H, d, d)
    put_states(g, o, seeded, st)
    verify_slots = seeded[:int(rng.integers(1, 4))]
    rest = seeded[len(verify_slots):]

    def step(commit=None):
        n_seq = int(rng.integers(0, 5))
        lens = [int(x) for x in rng.integers(0, 301, size=n_seq)]
        interval = int(rng.choice([0, 16, 37, 64, 100]))
        n_ck = sum(L // interval for L in lens) if interval else 0
        out, cks = take(n_seq), take(n_ck)
        init = [int(rest.pop()) if (rest and rng.random() < 0.5) else -1 for _ in range(n_seq)]
        dec = [s for s in rest[:int(rng.integers(0, 5))]]
        for s in dec:
            rest.remove(s)
        ver = verify_slots if commit is None else [s for s in verify_slots if rng.random() < 0.7] or verify_slots[:1]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        n_pre = int(cu[-1])
        tok = ki.draw_tokens(rng, (n_pre + len(dec) + len(ver) * P,), H, d, d)
        kw = {}
        if commit is not None:
            kw = dict(commit_slots=commit[0], n_accepted=torch.from_numpy(commit[1]).to("cuda"))
            o.commit(commit[0], commit[1])
        O = g.kda_mixed_batch(*tok_dev(tok), cu, out, dec, ver, P, init_slots=init,
                              ckpt_slots=cks, ckpt_interval=interval, **kw)
        torch.cuda.synchronize()
        if n_seq:
            Op = o.prefill(tok.slice(0, n_pre).np, cu, init, out, cks, interval)
            check_out(O[:n_pre], Op, cu, v=tok.np["v"][:n_pre])
        if dec:
            Od = o.decode(tok.slice(n_pre, n_pre + len(dec)).np, dec)
            check_out(O[n_pre:n_pre + len(dec)], Od, v=tok.np["v"][n_pre:n_pre + len(dec)])
        vt = {n: x[n_pre + len(dec):].reshape((len(ver), P) + x.shape[1:]) for n, x in tok.np.items()}
        Ov = o.verify(vt, ver)
        check_out(O[n_pre + len(dec):].reshape(len(ver), P, H, d), Ov,
                  v=tok.np["v"][n_pre + len(dec):].reshape(len(ver), P, H, d))
        for s in out + cks + dec + (commit[0] if commit is not None else []):
            check_state(g.state[s], o.state[s])
        ring_check(g, o, ver)
        meta_equal(g.meta_array(), o.meta(), range(n_slots))
        return ver

    ver1 = step()
    na = rng.integers(0, P, size=len(ver1)).astype(np.int32)
    ver2 = step(commit=(ver1, na))
    g.kda_commit(ver2, torch.from_numpy(np.zeros(len(ver2), dtype=np.int32)).to("cuda"))
    o.commit(ver2, np.zeros(len(ver2), dtype=np.int32))
    torch.cuda.synchronize()
    for s in ver2:
        check_state(g.state[s], o.state[s])
    meta_equal(g.meta_array(), o.meta(), range(n_slots))
    assert device_errors(g) == 0


@pytest.mark.parametrize("seed", range(16))
def test_prefill_random_batches(seed):
    """Prefill batches drawn at random: 1-100 sequences of lognormal lengths (some empty, some
    one chunk, a few thousand tokens), head count 1-8 (so the width plan varies from one width
    for all to several groups, inside and outside the operand kernel's own plan), resumed
    sequences, and a random checkpoint interval (0, aligned or not to the chunk), at d = 128 and
    16: outputs, final and checkpoint states against the oracle, metadata exact. Total work is
    bounded so that the oracle takes about a second."""
    rng = np.random.default_rng(7000 + seed)
    d = 128 if seed % 4 else 16
    H = int(rng.integers(1, 9))
    n_seq = int(rng.choice([1, 2, 5, 9, 40, 64, 65, 100]))
    budget = 24000 // H
    lengths = np.minimum(rng.lognormal(5.0, 1.2, size=n_seq).astype(int), 3000)
    lengths[rng.random(n_seq) < 0.1] = 0
    while lengths.sum() > budget:
        lengths = lengths // 2
    lengths = [int(x) for x in lengths]
    interval = int(rng.choice([0, 64, 128, 100, 37]))
    n_ck = sum(L // interval for L in lengths) if interval else 0
    n_slots = 2 * n_seq + n_ck
    g, o = pools(n_slots, H, d)
    init = [i if rng.random() < 0.3 else -1 for i in range(n_seq)]
    put_states(g, o, range(n_seq), ki.draw_states(rng, n_seq, H, d, d))
    out = list(range(n_seq, 2 * n_seq))
    cks = list(range(2 * n_seq, n_slots))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
    if d == 128:
        plan = g.kda_prefill_plan(cu)
        assert plan[-1][0] == n_seq and all(w in (16, 32, 64, 128) for _, w in plan)
    O = g.kda_prefill(*tok_dev(tok), cu, out, init_slots=init, ckpt_slots=cks,
                      ckpt_interval=interval)
    torch.cuda.synchronize()
    Oo = o.prefill(tok.np, cu, init, out, cks, interval)
    check_out(O, Oo, cu, v=tok.np["v"])
    for s_ in out + cks:
        check_state(g.state[s_], o.state[s_])
    meta_equal(g.meta_array(), o.meta(), range(n_slots))
    assert device_errors(g) == 0


@pytest.mark.parametrize("seed", range(12))
def test_random_operation_sequences(seed):
    """40 pool operations drawn at random over a 10-slot pool, each on slots in the state it
    needs: decode, verify + commit or rollback (ring scheme), verify_direct + commit_direct or
    rollback (whole batches), slot reset, slot checkpoint copy, and a small resumed prefill.
    After every operation its outputs, draft states and touched states are checked against the
    oracle, ring entries and every slot's metadata exactly; the oracle then takes the GPU's
    states, so each operation is checked from identical inputs."""
    rng = np.random.default_rng(5100 + seed)
    d = 16 if seed % 3 == 0 else 128
    H, n, R = int(rng.integers(1, 5)), 10, 9
    g, o = pools(n, H, d, R)
    put_states(g, o, range(n), ki.draw_states(rng, n, H, d, d))
    IDLE, RING, DIRECT = 1, 2, 3
    state = {s: IDLE for s in range(n)}
    npos, direct = {}, []

    def idle(k):
        c = [s for s in range(n) if state[s] == IDLE]
        k = min(k, len(c))
        return [int(x) for x in rng.choice(c, size=k, replace=False)] if k else []

    ran = []

    def sync(slots):
        ran.append(len(slots))
        torch.cuda.synchronize()
        for s in slots:
            check_state(g.state[s], o.state[s])
            o.state[s] = f64(g.state[s])
        meta_equal(g.meta_array(), o.meta(), range(n))

    for _ in range(40):
        op = rng.choice(["decode", "verify", "commit", "rollback", "vdirect", "cdirect",
                         "reset", "copy", "prefill"])
        if op == "decode" and idle(1):
            S = idle(int(rng.integers(1, 4)))
            t = ki.draw_tokens(rng, (len(S),), H, d, d)
            O = g.kda_decode(*tok_dev(t), S)
            check_out(O, o.decode(t.np, S), v=t.np["v"])
            sync(S)
        elif op in ("verify", "vdirect") and idle(1):
            S, P = idle(int(rng.integers(1, 4))), int(rng.integers(1, R + 1))
            t = ki.draw_tokens(rng, (len(S), P), H, d, d)
            if op == "verify":
                O = g.kda_verify(*tok_dev(t), S)
                Oo = o.verify(t.np, S)
                for s in S:
                    state[s], npos[s] = RING, P
            else:
                O, dr = g.kda_verify_direct(*tok_dev(t), S)
                Oo, dro = o.verify_direct(t.np, S)
                torch.cuda.synchronize()
                for b in range(len(S)):
                    for j in range(P):
                        check_state(dr[b, j], dro[b, j])
                for s in S:
                    state[s] = DIRECT
                direct.append((S, P, dr))
            torch.cuda.synchronize()
            check_out(O, Oo, v=t.np["v"])
            if op == "verify":
                ring_check(g, o, S)
            sync(S)
        elif op == "commit" and any(v == RING for v in state.values()):
            S = [s for s in range(n) if state[s] == RING and rng.random() < 0.7] or \
                [s for s in range(n) if state[s] == RING][:1]
            na = np.array([int(rng.integers(0, npos[s])) for s in S], dtype=np.int32)
            g.kda_commit(S, torch.from_numpy(na).to("cuda"))
            o.commit(S, na)
            for s in S:
                state[s] = IDLE
            sync(S)
        elif op == "cdirect" and direct:
            S, P, dr = direct.pop(int(rng.integers(0, len(direct))))
            na = rng.integers(0, P, size=len(S)).astype(np.int32)
            g.kda_commit_direct(S, torch.from_numpy(na).to("cuda"), dr)
            o.commit_direct(S, na, np.stack([f64(dr[b]) for b in range(len(S))]))
            for s in S:
                state[s] = IDLE
            sync(S)
        elif op == "rollback" and (direct or any(v == RING for v in state.values())):
            if direct and rng.random() < 0.5:
                S = direct.pop(int(rng.integers(0, len(direct))))[0]
            else:
                S = [s for s in range(n) if state[s] == RING][:int(rng.integers(1, 4))]
                if not S:
                    S = direct.pop()[0]
            g.kda_rollback(S)
            o.rollback(S)
            for s in S:
                state[s] = IDLE
            sync(S)
        elif op == "reset" and idle(1):
            s = idle(1)[0]
            g.kda_slot_reset(s)
            o.reset(s)
            sync([s])
        elif op == "copy" and len(idle(2)) == 2:
            src, dst = idle(2)
            g.kda_slot_checkpoint(src, dst)
            o.checkpoint(src, dst)
            sync([dst])
        elif op == "prefill" and len(idle(3)) == 3:
            S = idle(3)
            lens = [int(x) for x in rng.integers(0, 150, size=2)]
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            init, out = [S[2], -1], S[:2]
            t = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
            O = g.kda_prefill(*tok_dev(t), cu, out, init_slots=init)
            Oo = o.prefill(t.np, cu, init, out, [], 0)
            torch.cuda.synchronize()
            check_out(O, Oo, cu, v=t.np["v"])
            sync(out)
    assert len(ran) >= 25, f"only {len(ran)} of 40 drawn operations applied"
    assert device_errors(g) == 0


@pytest.mark.parametrize("d", [128, 16])
def test_steps_replayed_from_a_captured_graph(d):
    """Decode, then verify of 1+4 and its commit, captured once into a HIP graph (torch.cuda.graph
    on the binding's calls; slot arrays, accepted counts and outputs built before the capture)
    and replayed four times, with eager work and a synchronisation between replays: after every
    replay the outputs, states, rings and metadata equal, bit for bit, those of a second pool
    that made the same calls eagerly as many times."""
    H, P = 4, 5
    rng = np.random.default_rng(31 + d)
    pools_ = [pools(8, H, d)[0] for _ in range(2)]
    st = ki.draw_states(rng, 8, H, d, d)
    for g in pools_:
        g.state.copy_(st.to("cuda"))
    dec, ver = kda.IndexArray([1, 6], "cuda"), kda.IndexArray([2, 5], "cuda")
    na = torch.tensor([3, 1], dtype=torch.int32, device="cuda")
    td = tok_dev(ki.draw_tokens(rng, (2,), H, d, d))
    tv = tok_dev(ki.draw_tokens(rng, (2, P), H, d, d))
    outs = [(torch.empty((2, H, d), dtype=torch.bfloat16, device="cuda"),
             torch.empty((2, P, H, d), dtype=torch.bfloat16, device="cuda")) for _ in range(2)]

    def calls(g, od, ov):
        g.kda_decode(*td, dec, o=od)
        g.kda_verify(*tv, ver, o=ov)
        g.kda_commit(ver, na)

    eager, graphed = pools_
    calls(graphed, *outs[1])             # once eagerly on both pools before the capture
    calls(eager, *outs[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):        # recorded, not run: both pools stay one step in
        calls(graphed, *outs[1])
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(4):
        graph.replay()
        calls(eager, *outs[0])
        scratch.add_(1.0)                # the program's own eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(outs[1][0], outs[0][0]) and torch.equal(outs[1][1], outs[0][1])
        assert torch.equal(graphed.state, eager.state)
        assert all(torch.equal(a_, b_) for a_, b_ in zip(graphed.ring_tensors(), eager.ring_tensors()))
        assert np.array_equal(graphed.meta_array(), eager.meta_array())
    assert device_errors(graphed) == 0 and device_errors(eager) == 0


def test_mixed_step_replayed_from_a_captured_graph():
    """A serving step through kda_mixed_batch (commit of the previous step's verifies, decodes,
    verifies of 1+4, three prompts; commit, decode and verify forked to the binding's side
    stream and joined back) captured into a HIP graph and replayed three times, with eager work
    and a synchronisation between replays: after every replay outputs, states, rings and
    metadata equal, bit for bit, those of a second pool stepping eagerly."""
    H, d, P = 4, 128, 5
    rng = np.random.default_rng(57)
    st = ki.draw_states(rng, 10, H, d, d)
    lens = [300, 129, 64]
    cu = kda.IndexArray(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), "cuda")
    out, dec, ver = (kda.IndexArray(x, "cuda") for x in ([0, 1, 2], [3, 4], [6, 7]))
    n_tok = sum(lens) + 2 + 2 * P
    tok = tok_dev(ki.draw_tokens(rng, (n_tok,), H, d, d))
    na = torch.tensor([2, 4], dtype=torch.int32, device="cuda")
    pools_ = []
    for _ in range(2):
        g = pools(10, H, d)[0]
        g.state.copy_(st.to("cuda"))
        o = torch.empty((n_tok, H, d), dtype=torch.bfloat16, device="cuda")
        g.kda_mixed_batch(*tok, cu, out, dec, ver, P, o=o)   # first step: nothing to commit
        pools_.append((g, o))
    (eager, oe), (graphed, og) = pools_

    def step(g, o):
        g.kda_mixed_batch(*tok, cu, out, dec, ver, P, o=o, commit_slots=ver, n_accepted=na)

    step(eager, oe)
    step(graphed, og)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(graphed, og)
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        graph.replay()
        step(eager, oe)
        scratch.mul_(0.5)
        torch.cuda.synchronize()
        assert torch.equal(og, oe)
        assert torch.equal(graphed.state, eager.state)
        assert all(torch.equal(a_, b_) for a_, b_ in zip(graphed.ring_tensors(), eager.ring_tensors()))
        assert np.array_equal(graphed.meta_array(), eager.meta_array())
    assert device_errors(graphed) == 0 and device_errors(eager) == 0


def test_readme_python_example_runs():
    """The Python example in README.md runs as printed and leaves the slot metadata it shows."""
    import contextlib
    import io
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    readme = os.path.join(root, "README.md")
    if not os.path.exists(readme):
        pytest.skip("README.md is not in this copy of the tree")
    text = open(readme).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        exec(compile(code, "README.md", "exec"), {})
    line = buf.getvalue().strip().splitlines()[-1]
    assert "torch.Size([1000, 8, 128]) torch.Size([1, 8, 128]) torch.Size([1, 5, 8, 128])" in line
    assert re.sub(r"\s+", " ", line).endswith("[1004 3 0 0 5]"), line
