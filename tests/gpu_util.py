"""Helpers for the GPU parity tests: moving seeded workloads to the device,
running the oracle on the same inputs, and the tolerance checks.

Tolerances (per written tensor): outputs max|do| <= 1e-2 * max|o| and
states relative Frobenius error <= 1e-3 for bfloat16 inputs; for float32
inputs the bars are 1e-4 for both.  Slot and snapshot placement is checked
bit-exactly (untouched slots keep their bytes, NaN sentinels stay NaN).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import kda as ok
from linear_attention_03_amd import workloads as wl

OUT_TOL = {"bf16": 1e-2, "f32": 1e-4}
STATE_TOL = {"bf16": 1e-3, "f32": 1e-4}


def torch():
    import torch as _t
    return _t


def require_gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_03_amd import kda
    kda.lib()          # fails loudly when libkda.so is missing


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(x, dtype="f32"):
    t = torch()
    tt = t.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return tt.to("cuda").to(t.bfloat16)
    if dtype == "i32":
        return tt.to(t.int32).to("cuda")
    return tt.to("cuda").to(t.float32)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_fro(got, ref):
    d = np.linalg.norm((got - ref).ravel())
    n = np.linalg.norm(ref.ravel())
    return d / n if n > 0 else d


def check_out(got, ref, dtype, name):
    err = np.abs(got - ref).max() if ref.size else 0.0
    scale = np.abs(ref).max() if ref.size else 0.0
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert err <= OUT_TOL[dtype] * scale + 1e-30, f"{name}: max|do|={err:.3e} > {OUT_TOL[dtype]}*max|o|={scale:.3e}"
    return err / scale if scale else 0.0


def check_state(got, ref, dtype, name):
    e = rel_fro(got, ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite state"
    assert e <= STATE_TOL[dtype], f"{name}: relative Frobenius error {e:.3e} > {STATE_TOL[dtype]}"
    return e


# ----------------------------------------------------------------- prefill

def prefill_oracle(c: wl.PrefillCase, heads=None, intermediate=False, g=None, beta=None):
    """Oracle prefill of case c restricted to value heads `heads` (all by
    default; a subset passes the q/k head each of them reads)."""
    grp = c.HV // c.H
    if heads is None:
        heads, qk_heads = list(range(c.HV)), list(range(c.H))
    else:
        heads = list(heads)
        qk_heads = [h // grp for h in heads]
    K = c.K
    raw = c.A_log is None                 # the gate tensor already holds the log-decay
    dt = None if raw else c.dt_bias.reshape(c.HV, K)[heads].reshape(-1)
    g = c.g if g is None else g
    beta = c.beta if beta is None else beta
    return ok.prefill(c.q[:, :, qk_heads], c.k[:, :, qk_heads], c.v[:, :, heads], g[:, :, heads],
                      beta[:, :, heads], scale=c.scale, initial_state=c.pool[:, heads],
                      initial_state_indices=c.indices, use_qk_l2norm_in_kernel=c.use_qk_l2norm,
                      cu_seqlens=c.cu_seqlens, A_log=None if raw else c.A_log[heads], dt_bias=dt,
                      lower_bound=c.lower_bound, beta_is_raw=c.beta_is_raw,
                      output_intermediate_states=intermediate, chunk_size=c.chunk_size)


class PrefillDev:
    """Device copies of a prefill case."""

    def __init__(self, c: wl.PrefillCase, g=None, beta=None):
        d = c.dtype
        self.q, self.k, self.v = dev(c.q, d), dev(c.k, d), dev(c.v, d)
        self.g = dev(c.g if g is None else g, d)
        self.beta = dev(c.beta if beta is None else beta, d)
        self.A_log = None if c.A_log is None else dev(c.A_log)       # None: raw gate
        self.dt_bias = None if c.dt_bias is None else dev(c.dt_bias)
        self.pool = dev(c.pool)
        self.idx = dev(c.indices, "i32")
        self.cu = None if c.cu_seqlens is None else dev(c.cu_seqlens, "i32")
        self.c = c

    def run(self, intermediate=None, o=None, workspace=None, stream=None):
        from linear_attention_03_amd import kda
        c = self.c
        return kda.prefill(self.q, self.k, self.v, self.g, self.beta, scale=c.scale,
                           initial_state=self.pool, initial_state_indices=self.idx,
                           use_qk_l2norm_in_kernel=c.use_qk_l2norm, cu_seqlens=self.cu,
                           A_log=self.A_log, dt_bias=self.dt_bias, lower_bound=c.lower_bound,
                           beta_is_raw=c.beta_is_raw, chunk_size=c.chunk_size,
                           intermediate_states=intermediate, o=o, workspace=workspace, stream=stream)


def check_prefill(c, o_dev, pool_dev, heads=None, name="", o_ref=None, pool_ref=None):
    """Compare GPU prefill results with the oracle on `heads`; every slot
    not indexed must be bit-unchanged."""
    heads = list(range(c.HV)) if heads is None else list(heads)
    if o_ref is None:
        o_ref, pool_ref, _ = prefill_oracle(c, heads)
    o = host(o_dev)[:, :, heads]
    err_o = check_out(o, o_ref, c.dtype, f"{name} o")
    pool = pool_dev.cpu().numpy()
    err_s = 0.0
    for s in c.indices:
        err_s = max(err_s, check_state(pool[s][heads].astype(np.float64), pool_ref[s], c.dtype, f"{name} state slot {s}"))
    others = np.setdiff1d(np.arange(c.pool.shape[0]), c.indices)
    assert np.array_equal(pool[others].view(np.uint32), c.pool[others].view(np.uint32)), f"{name}: unindexed slot changed"
    say(f"{name}: max|do|/max|o| = {err_o:.2e}, worst state relative Frobenius = {err_s:.2e}")
    return err_o, err_s


# ----------------------------------------------------------------- decode / verify

class DecodeDev:
    def __init__(self, c: wl.DecodeCase):
        d = c.dtype
        self.mixed = dev(c.mixed_qkv, d)
        HK = c.H * c.K
        B = c.B
        self.q = self.mixed[:, :HK].view(B, c.H, c.K)
        self.k = self.mixed[:, HK:2 * HK].view(B, c.H, c.K)
        self.v = self.mixed[:, 2 * HK:].view(B, c.HV, c.V)
        self.a, self.b = dev(c.a, d), dev(c.b, d)
        self.A_log = None if c.A_log is None else dev(c.A_log)       # None: raw gate
        self.dt_bias = None if c.dt_bias is None else dev(c.dt_bias)
        self.pool = dev(c.pool)
        self.idx = dev(c.indices, "i32")
        self.c = c

    def run(self, o=None, stream=None):
        from linear_attention_03_amd import kda
        c = self.c
        return kda.decode(self.q, self.k, self.v, self.a, self.b, scale=c.scale,
                          initial_state=self.pool, initial_state_indices=self.idx,
                          A_log=self.A_log, dt_bias=self.dt_bias, lower_bound=c.lower_bound,
                          beta_is_raw=c.beta_is_raw, use_qk_l2norm_in_kernel=c.use_qk_l2norm,
                          o=o, stream=stream)


def decode_oracle(c: wl.DecodeCase):
    return ok.decode(c.q(), c.k(), c.v(), c.a, c.b, scale=c.scale, initial_state=c.pool,
                     initial_state_indices=c.indices, A_log=c.A_log, dt_bias=c.dt_bias,
                     lower_bound=c.lower_bound, beta_is_raw=c.beta_is_raw,
                     use_qk_l2norm_in_kernel=c.use_qk_l2norm)


class VerifyDev:
    def __init__(self, c: wl.VerifyCase, snapshot_slots=None):
        t = torch()
        d = c.dtype
        self.mixed = dev(c.mixed_qkv, d)
        self.a, self.b = dev(c.a, d), dev(c.b, d)
        self.w = dev(c.conv_weight, d)
        self.cs = dev(c.conv_state, d)
        self.A_log = None if c.A_log is None else dev(c.A_log)
        self.dt_bias = None if c.dt_bias is None else dev(c.dt_bias)
        self.pool = dev(c.pool)
        self.idx = dev(c.indices, "i32")
        self.parents = None if c.parents is None else dev(c.parents, "i32")
        ns = c.B if snapshot_slots is None else snapshot_slots
        self.snaps = t.full((ns, c.N, c.HV, c.V, c.K), float("nan"), dtype=t.float32, device="cuda")
        self.c = c

    def run(self, o=None, stream=None, snapshot_indices=None):
        from linear_attention_03_amd import kda
        c = self.c
        return kda.verify(self.mixed, self.a, self.b, N=c.N, H=c.H, HV=c.HV, K=c.K, V=c.V,
                          scale=c.scale, conv_weight=self.w, conv_state=self.cs,
                          initial_state=self.pool, initial_state_indices=self.idx,
                          snapshots=self.snaps, parents=self.parents, activation=c.activation,
                          snapshot_indices=snapshot_indices, A_log=self.A_log, dt_bias=self.dt_bias,
                          lower_bound=c.lower_bound, beta_is_raw=c.beta_is_raw,
                          use_qk_l2norm_in_kernel=c.use_qk_l2norm, o=o, stream=stream)


def verify_oracle(c: wl.VerifyCase, snapshot_indices=None):
    return ok.verify(c.mixed_qkv, c.a, c.b, N=c.N, H=c.H, HV=c.HV, K=c.K, V=c.V, scale=c.scale,
                     conv_weight=c.conv_weight, conv_state=c.conv_state, initial_state=c.pool,
                     initial_state_indices=c.indices, parents=c.parents, activation=c.activation,
                     snapshot_indices=snapshot_indices, A_log=c.A_log, dt_bias=c.dt_bias,
                     lower_bound=c.lower_bound, beta_is_raw=c.beta_is_raw,
                     use_qk_l2norm_in_kernel=c.use_qk_l2norm)
