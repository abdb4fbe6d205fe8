"""Grouped q/k heads (HV a multiple of H) and the unbounded gate (A_log
without lower_bound) on the GPU, through the C ABI, against the fp64
oracle: decode, verify with its replayed commit, and prefill on both the
general and the MFMA path (the unbounded gate's large decays take the
MFMA prep's exact-exponential branch)."""

import numpy as np
import pytest

from linear_attention_03_amd import workloads as wl
from oracle import kda as ok

import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H,HV,K,V", [(2, 4, 64, 128), (1, 4, 128, 64), (4, 4, 32, 32), (2, 8, 128, 128)])
@pytest.mark.parametrize("unbounded", [False, True])
def test_decode_grouped_heads_and_gate(dtype, H, HV, K, V, unbounded):
    c = wl.decode_case(seed=1300 + H + HV + K, B=5, H=H, HV=HV, K=K, V=V, slots=8, dtype=dtype,
                       pad_requests=(2,), unbounded=unbounded)
    name = f"decode H={H} HV={HV} K={K} V={V} {dtype} {'unbounded' if unbounded else 'bounded'}"
    gu.say(name)
    d = gu.DecodeDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    o_ref, pool_ref = gu.decode_oracle(c)
    gu.check_out(gu.host(o), o_ref, dtype, f"{name} o")
    pool = d.pool.cpu().numpy()
    for s in c.indices[c.indices >= 0]:
        gu.check_state(pool[s].astype(np.float64), pool_ref[s], dtype, f"{name} slot {s}")
    assert np.all(gu.host(o)[2] == 0)


def _verify_kw(c):
    return dict(N=c.N, H=c.H, HV=c.HV, K=c.K, V=c.V, scale=c.scale, conv_weight=c.conv_weight,
                conv_state=c.conv_state, initial_state=c.pool, initial_state_indices=c.indices,
                parents=c.parents, activation=c.activation, A_log=c.A_log, dt_bias=c.dt_bias,
                lower_bound=c.lower_bound, beta_is_raw=c.beta_is_raw,
                use_qk_l2norm_in_kernel=c.use_qk_l2norm)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H,HV,K,V", [(2, 4, 64, 64), (1, 2, 128, 128), (2, 8, 32, 64)])
@pytest.mark.parametrize("unbounded", [False, True])
@pytest.mark.parametrize("tree", [False, True])
def test_verify_and_replay_grouped_heads_and_gate(dtype, H, HV, K, V, unbounded, tree):
    import torch
    from linear_attention_03_amd import kda
    c = wl.verify_case(seed=1400 + H + HV + K, B=4, N=6, H=H, HV=HV, K=K, V=V, tree=tree, slots=9,
                       dtype=dtype, pad_requests=(1,), unbounded=unbounded)
    name = f"verify H={H} HV={HV} K={K} V={V} {dtype} {'tree' if tree else 'chain'} {'unbounded' if unbounded else 'bounded'}"
    gu.say(name)
    d = gu.VerifyDev(c)
    o = d.run()
    torch.cuda.synchronize()
    o_ref, snaps_ref = gu.verify_oracle(c)
    gu.check_out(gu.host(o), o_ref, dtype, f"{name} o")
    snaps = d.snaps.cpu().numpy()
    for (s, i), S in snaps_ref.items():
        gu.check_state(snaps[s, i].astype(np.float64), S, dtype, f"{name} snapshot ({s},{i})")
    accepted = np.array([5, 0, -1, 3], np.int32)
    kda.commit_replay(gu.dev(accepted, "i32"), d.mixed, d.a, d.b, N=c.N, H=c.H, HV=c.HV, K=c.K, V=c.V,
                      scale=c.scale, conv_weight=d.w, conv_state=d.cs, initial_state=d.pool,
                      initial_state_indices=d.idx, parents=d.parents, activation=c.activation,
                      A_log=d.A_log, dt_bias=d.dt_bias, lower_bound=c.lower_bound)
    torch.cuda.synchronize()
    pool_ref, cs_ref = ok.commit_replay(accepted, c.mixed_qkv, c.a, c.b, **_verify_kw(c))
    pool = d.pool.cpu().numpy()
    for r, s in enumerate(c.indices):
        if s >= 0 and accepted[r] >= 0:
            gu.check_state(pool[s].astype(np.float64), pool_ref[s], dtype, f"{name} replay slot {s}")
            assert np.array_equal(pool[s].view(np.uint32), snaps[r, accepted[r]].view(np.uint32)), \
                f"{name}: replayed state differs from the snapshot"
    assert np.array_equal(gu.host(d.cs), cs_ref)


@pytest.mark.parametrize("dtype,K,V,C", [("f32", 64, 32, 16), ("f32", 128, 128, 64), ("bf16", 128, 128, 64),
                                          ("bf16", 64, 64, 64)])
@pytest.mark.parametrize("H,HV", [(2, 4), (1, 4)])
@pytest.mark.parametrize("unbounded", [False, True])
def test_prefill_grouped_heads_and_gate(dtype, K, V, C, H, HV, unbounded):
    lengths = [1, 63, 64, 65, 130, 7]
    c = wl.prefill_case(seed=1500 + K + H + HV, B=1, T=sum(lengths), H=H, HV=HV, K=K, V=V, dtype=dtype,
                        chunk_size=C, lengths=lengths, slots=9, unbounded=unbounded)
    name = f"prefill varlen H={H} HV={HV} K={K} V={V} C={C} {dtype} {'unbounded' if unbounded else 'bounded'}"
    gu.say(name)
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)


@pytest.mark.parametrize("unbounded", [False, True])
def test_prefill_grouped_heads_4096(unbounded):
    """The MFMA path at full length: 1 x 4096, 4 q/k heads, 16 value heads."""
    c = wl.prefill_case(seed=1600 + unbounded, B=1, T=4096, H=4, HV=16, K=128, V=128, dtype="bf16",
                        slots=4, unbounded=unbounded)
    name = f"prefill 1x4096 H=4 HV=16 {'unbounded' if unbounded else 'bounded'}"
    gu.say(name)
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)
