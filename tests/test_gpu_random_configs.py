"""Seeded random combinations of the call options, through the C ABI,
against the fp64 oracle: the fixed sweeps in the other files vary one or two
options at a time; here every case draws all of them at once.

Prefill: dtype, K, V, q/k heads and grouped value heads, chunk 16 or 64,
fixed batch or packed lengths (with runs of 1, 15 .. 17, 63 .. 65, 129
tokens), padded gate / beta rows, the bounded (lower bound -1 .. -10),
unbounded or raw gate, raw or activated beta, in-kernel or host L2 norm.
Decode: the same per-token options, 1 .. 33 requests with padded ones.
Verify: chain, tree or forest drafts of 1 .. 16 tokens, conv with or without
SiLU and bias-free, padded requests, every gate form, then a commit of a
random accepted node per request.  Half the prefill cases also write the
intermediate states, checked chunk by chunk.  q and k reach the
kernels already normalised when the in-kernel norm is off, so the delta
rule stays a contraction as in the served models."""

import dataclasses

import numpy as np
import pytest

from linear_attention_03_amd import workloads as wl

import gpu_util as gu
from test_gpu_decode_verify import run_decode_case, run_verify_case

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def _unit_rows(x, n_heads, dim):
    """x [..., n_heads * dim] (or [..., n_heads, dim]) with every head row
    scaled to unit L2 norm, in float64."""
    shp = x.shape
    y = np.asarray(x, np.float64).reshape(*shp[:-1], n_heads, dim) if shp[-1] == n_heads * dim else \
        np.asarray(x, np.float64)
    y = y / np.maximum(np.linalg.norm(y, axis=-1, keepdims=True), 1e-6)
    return y.reshape(shp)


def _gate(rng):
    kind = rng.choice(["bounded", "unbounded", "raw"])
    lb = float(rng.choice([-1.0, -5.0, -10.0])) if kind == "bounded" else None
    return kind, lb


def _beta_activated(raw):
    return 1.0 / (1.0 + np.exp(-np.asarray(raw, np.float64)))


@pytest.mark.parametrize("case", range(16))
def test_random_prefill(case):
    """Cases 10 .. 15 keep the shape of the matrix-core path (bf16, K = V =
    128, chunk 64) and draw the rest."""
    rng = np.random.default_rng(9100 + case)
    dtype = str(rng.choice(["f32", "bf16"]))
    K, V = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128]))
    H = int(rng.integers(1, 4))
    HV = H * int(rng.choice([1, 2]))
    C = int(rng.choice([16, 64]))
    if case >= 10:
        dtype, K, V, C = "bf16", 128, 128, 64
    pad = int(rng.choice([0, 5]))
    if rng.random() < 0.5:
        lengths = [int(x) for x in rng.choice([1, 15, 16, 17, 63, 64, 65, 100, 129], size=int(rng.integers(2, 5)))]
        c = wl.prefill_case(seed=9200 + case, B=1, T=sum(lengths), H=H, HV=HV, K=K, V=V, dtype=dtype,
                            chunk_size=C, lengths=lengths, pad_rows=pad, slots=8)
        layout = f"packed {lengths}"
    else:
        B, T = int(rng.choice([1, 2])), int(rng.choice([1, 17, 64, 100, 129]))
        c = wl.prefill_case(seed=9200 + case, B=B, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype,
                            chunk_size=C, pad_rows=pad, slots=8)
        layout = f"fixed {B}x{T}"
    kind, lb = _gate(rng)
    kw = {"lower_bound": lb}
    if kind == "unbounded":
        kw["lower_bound"] = None
    elif kind == "raw":
        # the gate tensor is the log-decay itself: -softplus of the drawn values
        kw.update(A_log=None, dt_bias=None,
                  g=wl._as_dtype(-np.logaddexp(0.0, np.asarray(c.g, np.float64)), dtype))
    if rng.random() < 0.5:
        kw.update(beta_is_raw=False, beta=wl._as_dtype(_beta_activated(c.beta), dtype))
    if rng.random() < 0.5:
        kw.update(use_qk_l2norm=False, q=wl._as_dtype(_unit_rows(c.q, H, K), dtype),
                  k=wl._as_dtype(_unit_rows(c.k, H, K), dtype))
    c = dataclasses.replace(c, **kw)
    with_inter = rng.random() < 0.5
    name = (f"random prefill {case}: {layout} H={H} HV={HV} K={K} V={V} C={C} {dtype} gate={kind}"
            f"{'' if lb is None else f' lb={lb}'} beta_raw={c.beta_is_raw} l2norm={c.use_qk_l2norm} pad={pad}"
            f"{' intermediate states' if with_inter else ''}")
    d = gu.PrefillDev(c)
    from linear_attention_03_amd import kda
    path = kda.prefill_path(d.q, d.k, d.v, d.g, d.beta, scale=c.scale, initial_state=d.pool,
                            initial_state_indices=d.idx, use_qk_l2norm_in_kernel=c.use_qk_l2norm, cu_seqlens=d.cu,
                            A_log=d.A_log, dt_bias=d.dt_bias, lower_bound=c.lower_bound,
                            beta_is_raw=c.beta_is_raw, chunk_size=C)
    name += f" ({path} path)"
    gu.say(name)
    torch = gu.torch()
    if not with_inter:
        o = d.run()
        torch.cuda.synchronize()
        gu.check_prefill(c, o, d.pool, name=name)
        return
    rows = (kda.prefill_max_chunks(c.T, C, num_seqs=c.N) if c.cu_seqlens is not None
            else kda.prefill_max_chunks(c.T, C, B=c.B))
    inter = torch.full((rows, c.HV, c.V, c.K), float("nan"), device="cuda")
    o = d.run(intermediate=inter)
    torch.cuda.synchronize()
    o_ref, pool_ref, inter_ref = gu.prefill_oracle(c, intermediate=True)
    gu.check_prefill(c, o, d.pool, name=name, o_ref=o_ref, pool_ref=pool_ref)
    got = inter.cpu().numpy()
    n = inter_ref.shape[0]
    for i in range(n):
        gu.check_state(got[i].astype(np.float64), inter_ref[i], c.dtype, f"{name} chunk {i}")
    assert np.all(np.isnan(got[n:])), f"{name}: an intermediate-state row past the last chunk was written"


@pytest.mark.parametrize("case", range(10))
def test_random_decode(case):
    rng = np.random.default_rng(9300 + case)
    dtype = str(rng.choice(["f32", "bf16"]))
    K, V = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128]))
    H = int(rng.integers(1, 4))
    HV = H * int(rng.choice([1, 2]))
    B = int(rng.choice([1, 7, 33]))
    pads = tuple(int(x) for x in rng.choice(B, size=min(B - 1, 2), replace=False)) if B > 1 else ()
    c = wl.decode_case(seed=9400 + case, B=B, H=H, HV=HV, K=K, V=V, slots=B + 4, dtype=dtype, pad_requests=pads)
    kind, lb = _gate(rng)
    kw = {"lower_bound": lb}
    if kind == "unbounded":
        kw["lower_bound"] = None
    elif kind == "raw":
        kw.update(A_log=None, dt_bias=None, a=wl._as_dtype(-np.logaddexp(0.0, np.asarray(c.a, np.float64)), dtype))
    if rng.random() < 0.5:
        kw.update(beta_is_raw=False, b=wl._as_dtype(_beta_activated(c.b), dtype))
    if rng.random() < 0.5:
        m = np.asarray(c.mixed_qkv, np.float64).copy()
        m[:, :2 * H * K] = _unit_rows(m[:, :2 * H * K], 2 * H, K)
        kw.update(use_qk_l2norm=False, mixed_qkv=wl._as_dtype(m, dtype))
    c = dataclasses.replace(c, **kw)
    run_decode_case(c, f"random decode {case}: B={B} pads={pads} H={H} HV={HV} K={K} V={V} {dtype} gate={kind}"
                       f"{'' if lb is None else f' lb={lb}'} beta_raw={c.beta_is_raw} l2norm={c.use_qk_l2norm}")


@pytest.mark.parametrize("case", range(10))
def test_random_verify(case):
    rng = np.random.default_rng(9500 + case)
    dtype = str(rng.choice(["f32", "bf16"]))
    K, V = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128]))
    H = int(rng.integers(1, 3))
    HV = H * int(rng.choice([1, 2]))
    B = int(rng.choice([1, 3, 9]))
    N = int(rng.integers(1, 17))
    shape = str(rng.choice(["chain", "tree", "forest"]))
    pads = (int(rng.integers(0, B)),) if B > 1 else ()
    c = wl.verify_case(seed=9600 + case, B=B, N=N, H=H, HV=HV, K=K, V=V, tree=shape != "chain",
                       multi_root=shape == "forest", slots=B + 3, dtype=dtype, pad_requests=pads)
    kind, lb = _gate(rng)
    kw = {"lower_bound": lb}
    if kind == "unbounded":
        kw["lower_bound"] = None
    elif kind == "raw":
        kw.update(A_log=None, dt_bias=None, a=wl._as_dtype(-np.logaddexp(0.0, np.asarray(c.a, np.float64)), dtype))
    if rng.random() < 0.5:
        kw.update(beta_is_raw=False, b=wl._as_dtype(_beta_activated(c.b), dtype))
    if rng.random() < 0.3:
        kw["activation"] = "none"
    c = dataclasses.replace(c, **kw)
    name = (f"random verify {case}: B={B} N={N} {shape} pads={pads} H={H} HV={HV} K={K} V={V} {dtype}"
            f" gate={kind}{'' if lb is None else f' lb={lb}'} beta_raw={c.beta_is_raw} act={c.activation}")
    d, _ = run_verify_case(c, name)
    # then commit a random accepted node per request (-1: none), against the
    # oracle's commit of the same snapshots: the pool bit for bit, the conv
    # state rolled along the accepted path
    from linear_attention_03_amd import kda
    from oracle import kda as ok
    accepted = rng.integers(-1, N, size=B).astype(np.int32)
    kda.commit(gu.dev(accepted, "i32"), N=c.N, snapshots=d.snaps, initial_state=d.pool,
               initial_state_indices=d.idx, conv_state=d.cs, mixed_qkv=d.mixed, parents=d.parents)
    gu.torch().cuda.synchronize()
    snaps_host = d.snaps.cpu().numpy()
    pool_ref, cs_ref = ok.commit(accepted, N=c.N, snapshots=snaps_host.astype(np.float64), initial_state=c.pool,
                                 initial_state_indices=c.indices, conv_state=c.conv_state,
                                 mixed_qkv=c.mixed_qkv, parents=c.parents)
    assert np.array_equal(d.pool.cpu().numpy().astype(np.float64), pool_ref), f"{name}: committed pool"
    assert np.array_equal(gu.host(d.cs), cs_ref), f"{name}: committed conv state"
