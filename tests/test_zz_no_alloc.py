"""kda_prefill_noalloc (the prefill with its workspace in the library's
built-in scratch) against kda_prefill, through the C ABI: two calls in a
row, the second with a smaller input, each bit for bit equal to kda_prefill
on the same inputs (same kernels, same arithmetic), and within the oracle's
tolerances; a call whose workspace exceeds the scratch is refused."""

import numpy as np
import pytest

from linear_attention_03_amd import workloads as wl

import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def _noalloc(kda, d, o):
    c = d.c
    return kda.prefill_noalloc(d.q, d.k, d.v, d.g, d.beta, o=o, scale=c.scale, initial_state=d.pool,
                               initial_state_indices=d.idx, use_qk_l2norm_in_kernel=c.use_qk_l2norm,
                               cu_seqlens=d.cu, A_log=d.A_log, dt_bias=d.dt_bias, lower_bound=c.lower_bound,
                               beta_is_raw=c.beta_is_raw, chunk_size=c.chunk_size)


def test_prefill_noalloc_two_calls_match_prefill():
    import torch
    from linear_attention_03_amd import kda
    cases = [
        wl.prefill_case(seed=501, B=1, T=4096, H=16, K=128, V=128, dtype="bf16", slots=4),
        wl.prefill_case(seed=502, B=1, T=430, H=16, K=128, V=128, dtype="bf16", slots=6,
                        lengths=[1, 64, 65, 300]),
    ]
    for c in cases:
        name = f"noalloc T={c.T} N={c.N}"
        gu.say(name)
        ref = gu.PrefillDev(c)
        o_ref = ref.run()
        got = gu.PrefillDev(c)
        o = torch.full_like(o_ref, float("nan"))
        _noalloc(kda, got, o)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"{name}: output differs from kda_prefill"
        assert torch.equal(got.pool.view(torch.int32), ref.pool.view(torch.int32)), f"{name}: state differs"
        gu.check_prefill(c, o, got.pool, name=name)


def test_prefill_noalloc_refuses_oversize():
    import torch
    from linear_attention_03_amd import kda
    c = wl.prefill_case(seed=503, B=1, T=8192, H=16, K=128, V=128, dtype="bf16", slots=2)
    d = gu.PrefillDev(c)
    o = torch.zeros(1, c.T, c.HV, c.V, dtype=torch.bfloat16, device="cuda")
    pool0 = d.pool.clone()
    with pytest.raises(kda.KdaInvalidArgument, match="built-in scratch holds"):
        _noalloc(kda, d, o)
    torch.cuda.synchronize()
    assert torch.equal(d.pool, pool0) and not o.any()
