"""The two-level scan of the matrix-core prefill (run_chunks > 0), through
the C ABI, against the fp64 oracle on every head: runs of 8 and of 3 chunks
at 1 x 4096, slow decay (where the run maps carry the whole state from run
to run and their products decide the result), packed sequences of 0, 1, 64,
65 and longer lengths with intermediate states, grouped heads with the
unbounded gate, a batch of two rows, NaN gate / beta pads, and determinism.
The default (run_chunks = 0) is covered by every other prefill test."""

import numpy as np
import pytest

from linear_attention_03_amd import workloads as wl
from oracle import kda as ok

import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def _run(d, run_chunks, **kw):
    from linear_attention_03_amd import kda
    c = d.c
    return kda.prefill(d.q, d.k, d.v, d.g, d.beta, scale=c.scale, initial_state=d.pool,
                       initial_state_indices=d.idx, use_qk_l2norm_in_kernel=c.use_qk_l2norm,
                       cu_seqlens=d.cu, A_log=d.A_log, dt_bias=d.dt_bias, lower_bound=c.lower_bound,
                       beta_is_raw=c.beta_is_raw, chunk_size=c.chunk_size, run_chunks=run_chunks, **kw)


@pytest.mark.parametrize("L", [8, 3])
def test_runs_1x4096(L):
    c = wl.prefill_case(seed=700 + L, B=1, T=4096, H=16, K=128, V=128, dtype="bf16", slots=4)
    name = f"1x4096 runs of {L} chunks"
    gu.say(name)
    d = gu.PrefillDev(c)
    o = _run(d, L)
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)


@pytest.mark.parametrize("gval", [0.0, -1e-3])
def test_runs_slow_decay(gval):
    """Log-decay 0 / -1e-3 on every channel: nothing is forgotten, so every
    run's entry state is the chain of the run maps M_j (products of 512
    tokens' transitions) applied to the pool state."""
    import torch
    from linear_attention_03_amd import kda
    c = wl.prefill_case(seed=710, B=1, T=4096, H=16, K=128, V=128, dtype="bf16", slots=4)
    g = wl.round_bf16(np.full(c.g.shape, gval, np.float32))
    name = f"1x4096 runs of 8, log-decay {gval}"
    gu.say(name)
    q, k, v, gd, b = (gu.dev(x, "bf16") for x in (c.q, c.k, c.v, g, c.beta))
    pool = gu.dev(c.pool)
    idx = gu.dev(c.indices, "i32")
    o = kda.prefill(q, k, v, gd, b, scale=c.scale, initial_state=pool, initial_state_indices=idx,
                    use_qk_l2norm_in_kernel=True, beta_is_raw=True, chunk_size=64, run_chunks=8)
    torch.cuda.synchronize()
    o_ref, p_ref, _ = ok.prefill(c.q, c.k, c.v, g, c.beta, scale=c.scale, initial_state=c.pool,
                                 initial_state_indices=c.indices, use_qk_l2norm_in_kernel=True, beta_is_raw=True)
    s = int(c.indices[0])
    e_o = gu.check_out(gu.host(o), o_ref, "bf16", f"{name} o")
    e_s = gu.check_state(pool[s].cpu().numpy().astype(np.float64), p_ref[s], "bf16", f"{name} state")
    gu.say(f"{name}: max|do|/max|o| = {e_o:.2e}, state relative Frobenius = {e_s:.2e}")


def test_runs_packed_with_intermediate_states():
    import torch
    from linear_attention_03_amd import kda
    lengths = [700, 0, 1, 64, 65, 2048, 130]
    c = wl.prefill_case(seed=720, B=1, T=sum(lengths), H=16, K=128, V=128, dtype="bf16", lengths=lengths,
                        slots=10)
    n_rows = kda.prefill_max_chunks(c.T, 64, num_seqs=c.N)
    inter = torch.full((n_rows, c.HV, c.V, c.K), float("nan"), device="cuda")
    name = "packed runs of 4 chunks, intermediate states"
    gu.say(name)
    d = gu.PrefillDev(c)
    o = _run(d, 4, intermediate_states=inter)
    torch.cuda.synchronize()
    o_ref, pool_ref, inter_ref = gu.prefill_oracle(c, intermediate=True)
    gu.check_prefill(c, o, d.pool, name=name, o_ref=o_ref, pool_ref=pool_ref)
    got = inter.cpu().numpy()
    n = inter_ref.shape[0]
    assert n == sum((x + 63) // 64 for x in lengths)
    for i in range(n):
        gu.check_state(got[i].astype(np.float64), inter_ref[i], "bf16", f"{name}: chunk {i}")
    assert np.all(np.isnan(got[n:]))


@pytest.mark.parametrize("unbounded", [False, True])
def test_runs_grouped_heads(unbounded):
    c = wl.prefill_case(seed=730 + unbounded, B=1, T=2500, H=4, HV=16, K=128, V=128, dtype="bf16",
                        slots=4, unbounded=unbounded)
    name = f"1x2500 H=4 HV=16 runs of 5, {'unbounded' if unbounded else 'bounded'}"
    gu.say(name)
    d = gu.PrefillDev(c)
    o = _run(d, 5)
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)


def test_runs_batch_two_rows_and_nan_pads_and_determinism():
    import torch
    c = wl.prefill_case(seed=740, B=2, T=1500, H=16, K=128, V=128, dtype="bf16", slots=5)
    name = "2x1500 runs of 7"
    gu.say(name)
    d = gu.PrefillDev(c)
    pool0 = d.pool.clone()
    o = _run(d, 7)
    torch.cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)
    p1 = d.pool.clone()
    d.pool.copy_(pool0)
    o2 = _run(d, 7)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(d.pool, p1), "two-level scan is not deterministic"
    # NaN pads past T in g and beta are never read
    g_pad = np.concatenate([c.g, np.full((2, 64, c.HV, c.K), np.nan, np.float32)], axis=1)
    b_pad = np.concatenate([c.beta, np.full((2, 64, c.HV), np.nan, np.float32)], axis=1)
    d3 = gu.PrefillDev(c, g=g_pad, beta=b_pad)
    o3 = _run(d3, 7)
    torch.cuda.synchronize()
    assert torch.equal(o3.view(torch.int16), o.view(torch.int16))
    assert torch.equal(d3.pool.view(torch.int32), p1.view(torch.int32))
