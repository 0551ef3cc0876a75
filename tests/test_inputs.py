"""The seeded input generators: shapes, dtypes, the normalisation, and the packed-length recipe."""
import numpy as np
import torch

import kda_inputs as ki


def test_tokens_shapes_dtypes_and_normalisation():
    t = ki.draw_tokens(np.random.default_rng(0), (5,), 3, 16, 8)
    assert t.q.dtype == torch.bfloat16 and t.a.dtype == torch.float32
    assert tuple(t.q.shape) == (5, 3, 16) and tuple(t.v.shape) == (5, 3, 8)
    assert tuple(t.b.shape) == (5, 3)
    # q, k are unit vectors before bf16 rounding (relative rounding <= 2^-9 per element)
    n = np.linalg.norm(t.np["k"], axis=-1)
    assert np.all(np.abs(n - 1) < 4e-3)
    assert np.all((t.np["a"] > 0) & (t.np["a"] < 1)) and np.all((t.np["b"] > 0) & (t.np["b"] < 1))
    np.testing.assert_array_equal(t.np["q"], t.q.double().numpy())


def test_seeded_draws_repeat():
    a = ki.decode_workload(seed=1, B=2, H=2, d=16, n_slots=8)
    b = ki.decode_workload(seed=1, B=2, H=2, d=16, n_slots=8)
    assert torch.equal(a["tokens"].q, b["tokens"].q) and np.array_equal(a["slots"], b["slots"])


def test_mixed_lengths_fill_budget():
    w = ki.mixed_workload(H=2, d=16)
    assert sum(w["lengths"]) == 16384 - 32 - 36
    assert min(w["lengths"]) >= 256 and len(w["lengths"]) == 6
    assert len(set(np.concatenate([w["prefill_slots"], w["decode_slots"], w["verify_slots"]]).tolist())) == 42
