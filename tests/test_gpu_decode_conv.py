"""kda_decode_conv (the one-token conv update and the packed decode in one
launch) through the C ABI against the fp64 oracle (conv update then
decode) and against kda_conv_update followed by kda_decode on the conv's
q || k || v output: the conv-state roll bit for bit (both copy inputs),
output and pool within the tolerances (the fused call keeps the conv
output in fp32, the two launches store it in the input dtype), on the
48-request workload and on other shapes, conv widths, grouped heads, the
unbounded gate, padded requests and several steps in a row."""

import numpy as np
import pytest

from linear_attention_03_amd import workloads as wl
from oracle import kda as ok

import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def _case(seed, B, H, HV, K, V, dtype, W=4, bias=False, slots=12, pads=(), unbounded=False, tokens=1):
    d = wl.decode_case(seed=seed, B=B, H=H, HV=HV, K=K, V=V, slots=slots, dtype=dtype, pad_requests=pads,
                       unbounded=unbounded)
    rng = np.random.default_rng(seed + 1000)
    C = d.mixed_qkv.shape[1]
    rnd = (lambda x: wl.round_bf16(x.astype(np.float32))) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    extra = dict(w=rnd(rng.uniform(-0.5, 0.5, (C, W))), bias=rnd(0.1 * rng.standard_normal(C)) if bias else None,
                 cs=rnd(rng.standard_normal((slots, C, W - 1))),
                 cidx=rng.permutation(slots)[:B].astype(np.int32),
                 xs=[d.mixed_qkv] + [rnd(rng.standard_normal(d.mixed_qkv.shape)) for _ in range(tokens - 1)],
                 a_s=[d.a] + [rnd(rng.standard_normal(d.a.shape)) for _ in range(tokens - 1)],
                 b_s=[d.b] + [rnd(rng.standard_normal(d.b.shape)) for _ in range(tokens - 1)])
    return d, extra


def _gate_kw(d, dev):
    return dict(A_log=dev(d.A_log), dt_bias=dev(d.dt_bias), lower_bound=d.lower_bound)


def _run_both(d, e, activation, t=0, state=None):
    """One token through the fused call and through conv_update + decode on
    separate copies; returns both sets of device results."""
    import torch
    from linear_attention_03_amd import kda
    dt = d.dtype
    dev = gu.dev
    x, a, b = dev(e["xs"][t], dt), dev(e["a_s"][t], dt), dev(e["b_s"][t], dt)
    w = dev(e["w"], dt)
    bias = None if e["bias"] is None else dev(e["bias"], dt)
    idx, cidx = dev(d.indices, "i32"), dev(e["cidx"], "i32")
    if state is None:
        state = dict(p1=dev(d.pool), c1=dev(e["cs"], dt), p2=dev(d.pool), c2=dev(e["cs"], dt))
    kw = dict(scale=d.scale, beta_is_raw=d.beta_is_raw, use_qk_l2norm_in_kernel=d.use_qk_l2norm,
              **_gate_kw(d, dev))
    o1 = kda.decode_conv(x, a, b, H=d.H, HV=d.HV, K=d.K, V=d.V, conv_weight=w, conv_bias=bias,
                         conv_state=state["c1"], conv_state_indices=cidx, activation=activation,
                         initial_state=state["p1"], initial_state_indices=idx, **kw)
    # two launches; a padded request's conv slot is passed as padded too
    cidx2 = dev(np.where(d.indices < 0, -1, e["cidx"]).astype(np.int32), "i32")
    y = kda.conv_update(x, conv_weight=w, conv_bias=bias, conv_state=state["c2"], conv_state_indices=cidx2,
                        activation=activation)
    HK = d.H * d.K
    B = x.shape[0]
    o2 = kda.decode(y[:, :HK].view(B, d.H, d.K), y[:, HK:2 * HK].view(B, d.H, d.K),
                    y[:, 2 * HK:].view(B, d.HV, d.V), a, b, initial_state=state["p2"], initial_state_indices=idx,
                    **kw)
    torch.cuda.synchronize()
    return o1, o2, state


def _oracle(d, e, activation, t, pool, cs):
    return ok.decode_conv(e["xs"][t], e["a_s"][t], e["b_s"][t], H=d.H, HV=d.HV, K=d.K, V=d.V, scale=d.scale,
                          conv_weight=e["w"], conv_state=cs, initial_state=pool, initial_state_indices=d.indices,
                          conv_state_indices=e["cidx"], conv_bias=e["bias"], activation=activation,
                          A_log=d.A_log, dt_bias=d.dt_bias, lower_bound=d.lower_bound, beta_is_raw=d.beta_is_raw,
                          use_qk_l2norm_in_kernel=d.use_qk_l2norm)


def _check(d, e, activation, name, tokens=1):
    import torch
    pool_ref, cs_ref = d.pool, e["cs"]
    state = None
    for t in range(tokens):
        o1, o2, state = _run_both(d, e, activation, t, state)
        bits = torch.int16 if d.dtype == "bf16" else torch.int32
        assert torch.equal(state["c1"].view(bits), state["c2"].view(bits)), f"{name} t={t}: conv state differs"
        # consistency with the two launches: their conv output is rounded to
        # the input dtype (relative 2^-9 for bf16), so they agree to that
        # rounding, not to the oracle's 1e-3 state bar (checked below)
        gu.check_out(gu.host(o1), gu.host(o2), d.dtype, f"{name} t={t} o vs two launches")
        live = d.indices[d.indices >= 0]
        e2 = gu.rel_fro(gu.host(state["p1"][live]), gu.host(state["p2"][live]))
        assert e2 <= 1e-2, f"{name} t={t}: pool vs two launches {e2:.3e}"
        o_ref, pool_ref, cs_ref = _oracle(d, e, activation, t, pool_ref, cs_ref)
        gu.check_out(gu.host(o1), o_ref, d.dtype, f"{name} t={t} o")
        pool = state["p1"].cpu().numpy()
        for s in d.indices[d.indices >= 0]:
            gu.check_state(pool[s].astype(np.float64), pool_ref[s], d.dtype, f"{name} t={t} slot {s}")
        # conv state: bit copies of inputs (exact in the input dtype)
        assert np.array_equal(gu.host(state["c1"]), cs_ref), f"{name} t={t}: conv state vs oracle"
    untouched = np.setdiff1d(np.arange(d.pool.shape[0]), d.indices)
    assert np.array_equal(state["p1"].cpu().numpy()[untouched].view(np.uint32), d.pool[untouched].view(np.uint32))
    gu.say(f"{name}: conv state == two launches bit for bit over {tokens} token(s); o and pool within tolerance "
           f"of the two launches and the oracle")


def test_decode_conv_48x1():
    d, e = _case(seed=1700, B=48, H=16, HV=16, K=128, V=128, dtype="bf16", slots=240, pads=(5, 30))
    _check(d, e, "silu", "decode+conv 48x1 bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H,HV,K,V", [(2, 2, 128, 128), (2, 4, 64, 32), (1, 4, 32, 64), (4, 4, 128, 64)])
@pytest.mark.parametrize("W", [2, 3, 4])
def test_decode_conv_shapes_and_widths(dtype, H, HV, K, V, W):
    d, e = _case(seed=1710 + H + HV + K + V + W, B=6, H=H, HV=HV, K=K, V=V, dtype=dtype, W=W, bias=(W == 3),
                 pads=(2,))
    _check(d, e, "none" if W == 2 else "silu", f"decode+conv H={H} HV={HV} K={K} V={V} W={W} {dtype}")


@pytest.mark.parametrize("unbounded", [False, True])
def test_decode_conv_three_steps_grouped(unbounded):
    d, e = _case(seed=1750 + unbounded, B=5, H=2, HV=8, K=128, V=128, dtype="bf16", pads=(1,),
                 unbounded=unbounded, tokens=3)
    _check(d, e, "silu", f"decode+conv 3 steps H=2 HV=8 {'unbounded' if unbounded else 'bounded'}", tokens=3)
