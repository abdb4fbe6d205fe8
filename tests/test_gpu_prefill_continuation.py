"""Prefill continued through the state pool and from intermediate states.

A long sequence prefilled in pieces (each piece starting from the state the
previous one left in the pool) must give exactly the outputs and final state
of one call over the whole sequence, as must a prefill started from an
intermediate state of a longer call: chunk boundaries line up, so the
device arithmetic is the same operation for operation and the comparison is
bitwise.  A batch of two 4096-token rows (fixed layout) is checked against
the oracle on every head.
"""

import numpy as np
import pytest

from linear_attention_03_amd import workloads as wl

import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def _prefill(torch, kda, c, q, k, v, g, b, pool, idx, t0, t1, intermediate=None):
    """Prefill of tokens [t0, t1) of row 0 of case c from pool[idx]."""
    sl = slice(t0, t1)
    return kda.prefill(q[:, sl], k[:, sl], v[:, sl], g[:, sl], b[:, sl], scale=c.scale,
                       initial_state=pool, initial_state_indices=idx, use_qk_l2norm_in_kernel=True,
                       A_log=gu.dev(c.A_log), dt_bias=gu.dev(c.dt_bias), lower_bound=c.lower_bound,
                       beta_is_raw=True, chunk_size=c.chunk_size, intermediate_states=intermediate)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_in_pieces_equals_one_call(dtype):
    import torch
    from linear_attention_03_amd import kda
    T = 8192 if dtype == "bf16" else 1024
    c = wl.prefill_case(seed=90, B=1, T=T, H=16, K=128, V=128, dtype=dtype, slots=4)
    gu.say(f"prefill 1x{T} {dtype} in one call and in pieces")
    q, k, v, g, b = (gu.dev(x, dtype) for x in (c.q, c.k, c.v, c.g, c.beta))
    idx = gu.dev(c.indices, "i32")
    pool_one = gu.dev(c.pool)
    o_one = _prefill(torch, kda, c, q, k, v, g, b, pool_one, idx, 0, T)
    pool_pc = gu.dev(c.pool)
    cuts = [0, T // 4, T // 2, T]                       # pieces of whole chunks
    o_pc = [_prefill(torch, kda, c, q, k, v, g, b, pool_pc, idx, t0, t1) for t0, t1 in zip(cuts, cuts[1:])]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(o_pc, dim=1), o_one), "outputs of the pieces differ from one call"
    assert torch.equal(pool_pc, pool_one), "final state of the pieces differs from one call"


def test_prefill_from_intermediate_state_equals_tail():
    import torch
    from linear_attention_03_amd import kda
    T, C = 2048, 64
    c = wl.prefill_case(seed=91, B=1, T=T, H=16, K=128, V=128, dtype="bf16", slots=4)
    gu.say(f"prefill 1x{T} from intermediate states")
    q, k, v, g, b = (gu.dev(x, "bf16") for x in (c.q, c.k, c.v, c.g, c.beta))
    idx = gu.dev(c.indices, "i32")
    pool = gu.dev(c.pool)
    inter = torch.zeros(kda.prefill_max_chunks(T, C), c.HV, c.V, c.K, device="cuda")
    o_full = _prefill(torch, kda, c, q, k, v, g, b, pool, idx, 0, T, intermediate=inter)
    for ci in (1, 7, 31):
        # the state entering chunk ci, placed in a pool slot of its own
        pool2 = gu.dev(c.pool)
        pool2[int(c.indices[0])] = inter[ci]
        o_tail = _prefill(torch, kda, c, q, k, v, g, b, pool2, idx, ci * C, T)
        torch.cuda.synchronize()
        assert torch.equal(o_tail, o_full[:, ci * C:]), f"tail from chunk {ci} differs"
        assert torch.equal(pool2[int(c.indices[0])], pool[int(c.indices[0])]), f"final state from chunk {ci} differs"


def test_prefill_batch_two_rows_4096():
    c = wl.prefill_case(seed=92, B=2, T=4096, H=16, K=128, V=128, dtype="bf16", slots=5)
    gu.say("prefill 2x4096 bf16, fixed layout")
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name="2x4096")
    assert np.all(np.isfinite(gu.host(o)))
