"""The allocation-free prefill entry point (kda_prefill_noalloc) against kda_prefill, through
the C ABI: two calls in a row on the same GPU, the second smaller, each bit-identical to
kda_prefill with a workspace of the caller's on a pool with the same contents (same kernels);
an oversized call is rejected and writes nothing."""
from ctypes import byref

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kda_inputs as ki  # noqa: E402
import recurrent_linear_attention_amd as kda  # noqa: E402
from recurrent_linear_attention_amd import _abi  # noqa: E402
from recurrent_linear_attention_amd.pool import _ix, _stream  # noqa: E402
from tests.parity import dev  # noqa: E402


def _pool(H, d, n_slots, states):
    g = kda.KDAPool(n_slots, H, d)
    for _ in range(n_slots):
        g.kda_slot_alloc()
    g.state[: states.shape[0]] = states.to("cuda")
    return g


@pytest.mark.parametrize("d", [128, 16])
def test_prefill_noalloc_matches_prefill(d):
    H, interval = 8, 2 * kda.chunk_for(d)
    rng = np.random.default_rng(4040 + d)
    n_slots = 40
    states = ki.draw_states(rng, 4, H, d, d)
    # the first call the larger one, the second smaller (the scratch keeps the first's bytes)
    for lengths in ([700, 130, 64, 1, 0], [200, 65]):
        n = len(lengths)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        tok = ki.draw_tokens(rng, (int(cu[-1]),), H, d, d)
        q, k, v, a, b = (dev(x) for x in (tok.q, tok.k, tok.v, tok.a, tok.b))
        init = [0] + [-1] * (n - 1)
        out = list(range(4, 4 + n))
        n_ck = sum(L // interval for L in lengths)
        cks = list(range(4 + n, 4 + n + n_ck))
        ref, tst = _pool(H, d, n_slots, states), _pool(H, d, n_slots, states)
        O1 = ref.kda_prefill(q, k, v, a, b, cu, out, init_slots=init, ckpt_slots=cks,
                             ckpt_interval=interval)
        O2 = torch.full_like(O1, float("nan"))
        args = _abi.kda_prefill_args(*tst._tok_ptrs(q, k, v, a, b, O2))
        cu_i, out_i, init_i, ck_i = (_ix(x, tst.device) for x in (cu, out, init, cks))
        args.n_seq, args.n_tok, args.chunk, args.ckpt_interval = n, int(cu[-1]), kda.chunk_for(d), interval
        args.h_cu_seqlens, args.d_cu_seqlens = cu_i.h, cu_i.d
        args.h_init_slot, args.d_init_slot = init_i.h, init_i.d
        args.h_out_slot, args.d_out_slot = out_i.h, out_i.d
        args.h_ckpt_slot, args.d_ckpt_slot = ck_i.h, ck_i.d
        assert _abi.lib.kda_prefill_noalloc(tst.handle, byref(args), _stream(None)) == 0
        torch.cuda.synchronize()
        assert torch.equal(O1, O2)
        assert torch.equal(ref.state, tst.state)
        assert np.array_equal(ref.meta_array(), tst.meta_array())
        assert tst.kda_read_device_error() & ~_abi.KDA_DEVERR_DECAY_RANGE == 0


def test_prefill_noalloc_rejects_an_oversized_prefill():
    H, d, L = 32, 128, 4096
    rng = np.random.default_rng(4041)
    g = _pool(H, d, 4, ki.draw_states(rng, 1, H, d, d))
    tok = ki.draw_tokens(rng, (L,), H, d, d)
    q, k, v, a, b = (dev(x) for x in (tok.q, tok.k, tok.v, tok.a, tok.b))
    O = torch.zeros((L, H, d), dtype=torch.bfloat16, device="cuda")
    before = g.state.clone()
    with pytest.raises(kda.KDAError) as e:
        g.kda_prefill_noalloc(q, k, v, a, b, [0, L], [1], O)
    assert e.value.status == _abi.KDA_EWORKSPACE
    torch.cuda.synchronize()
    assert not O.any() and torch.equal(g.state, before)
