#!/usr/bin/env python3
"""Throughput of the KDA hot path on one MI355X.

One step = one call of every phase on its workload, inputs resident in HBM:
  prefill  1 x 4096 tokens, 16 heads of 128 x 128, bf16, chunk 64
  decode   48 requests x 1 token (packed mixed_qkv), in-place pool update
  verify   48 requests x 6 draft tokens (chain), width-4 causal conv + SiLU,
           one fp32 snapshot per draft token
  commit   48 requests, accepted node drawn once (seeded)
value = tokens per step (4096 + 48 + 288) / seconds per step, from one HIP
graph per step replayed back to back.  The graph has two branches: the
prefill on one, verify -> decode -> commit on the other (the phases serve
disjoint requests); the same step on one stream is reported beside it.

Per-call kernel times come from kda_set_call_events: a call's first kernel
stamps a start event as it begins and its last kernel a stop event as it
ends (hipExtLaunchKernel), so the interval is the call's GPU time without
launch gaps, the quantity rocprofv3's kernel trace reports.  They are taken
  * in the step: every phase of the K timed eager steps (the `phases` entry
    and the `roofline` entry);
  * per workload (`configs`): the five workloads of the benchmark plan
    (tiny float32 prefill, decode 48 x 1, prefill 1 x 4096 / 1 x 8192,
    packed 8192 with padded gate rows, verify 48 x 6 chain and tree) plus
    commit, verify without snapshots, commit by replay and the conv update.
    Each call is timed `--samples` times hot (repeated back to back) and
    cold (a 512 MiB buffer written and another 512 MiB read before each
    call, so that neither the L2 caches nor the 256 MB last-level cache
    hold its inputs or dirty lines), in
    `--sample-procs` processes; medians and 10th / 90th percentiles are
    reported, and HBM fractions use the cold median.
Every enqueue happens behind a GPU spin kernel, so host launch cost never
shows in a timed interval.

Rooflines: decode, verify and commit are bound by HBM (algorithmic bytes /
time against 8 TB/s).  The prefill is below the ridge point as well
(9.2 GFLOP over 86 MB at 1 x 4096), so its roofline fraction is
max(t_HBM, t_MFMA) / t with both raw fractions reported.  `traffic` is the
HBM bytes per call from rocprofv3's FETCH_SIZE and WRITE_SIZE counters, each
scaled by what the same counter reads for a plain copy of known size,
stored in profiles/traffic.json with a hash of the kernel sources (null
once the sources change).

CPU baseline: the fp64 oracle on the host on whole steps of the same
workloads, once on one thread and once over all cores (independent heads
and requests spread over a process pool), with the CPU model stated.

    python bench.py [--steps K] [--warmup W] [--samples S] [--sample-procs P]
                    [--no-cpu-baseline] [--no-configs]
    python bench.py --write-traffic FETCH_DIR WRITE_DIR   (after two --pmc runs)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA tokens/s + µs/call per phase (16 heads×128) on 1 MI355X; % HBM/MFMA peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA, published
F32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COLD_BYTES = 512 << 20          # written before every cold call
COPY_BYTES = 256 << 20          # traffic calibration copy
STEP = ["prefill", "decode", "verify", "commit"]
# The step graph: the prefill on one branch, verify -> decode -> commit on a
# second that forks at the start of the step and joins at its end.  The
# phases work on disjoint requests (pools, conv states, outputs), so they
# may overlap; the prefill's scan leaves half the compute units idle and is
# bound by per-CU operand loads, not by HBM, so the HBM-bound phases fill
# them.  Measured against other orders and splits; this one was fastest.
STEP_BRANCHES = [["prefill"], ["verify", "decode", "commit"]]
TRAFFIC_KERNELS = {"prep_mfma_kernel": "prefill", "scan_mfma_kernel": "prefill",
                   "decode_kernel": "decode", "verify_kernel": "verify", "commit_kernel": "commit"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash():
    d = os.path.join(ROOT, "linear_attention_03_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------- host workloads

class HostWork:
    """Seeded host inputs of every benchmarked call (NumPy)."""

    def __init__(self):
        from linear_attention_03_amd import workloads as wl
        self.wl = wl
        self.p4096 = wl.config2_prefill(4096)
        self.d = wl.config1_decode()
        self.v = wl.config4_verify(tree=False)
        rng = np.random.default_rng(wl.BASE_SEED + 5)
        self.accepted = rng.integers(-1, self.v.N, self.v.B).astype(np.int32)

    def configs(self):
        wl = self.wl
        self.tiny = wl.config0_tiny()
        self.p8192 = wl.config2_prefill(8192)
        self.varlen = wl.config3_varlen(pad_value=1e4)
        self.vtree = wl.config4_verify(tree=True)
        # the 1 x 4096 workload's values as float32 inputs (general path, fp32 matrix tiles)
        import dataclasses
        self.p4096_f32 = dataclasses.replace(self.p4096, dtype="f32", name="prefill 1x4096 fp32")
        # the smaller batches of the pages' decode and verify tables (same shapes otherwise)
        self.d_small = {B: wl.decode_case(seed=wl.BASE_SEED + 20 + B, B=B, H=16, K=128, V=128,
                                          name=f"decode {B}x1 H=16 K=V=128 bf16") for B in (1, 16)}
        self.v_small = {B: wl.verify_case(seed=wl.BASE_SEED + 30 + B, B=B, N=6, H=16, K=128, V=128, tree=False,
                                          name=f"verify {B}x6 chain H=16 K=V=128 bf16 conv4") for B in (1, 16)}


def state_bytes(c):
    return c.HV * c.V * c.K * 4


def prefill_bytes(c):
    """Algorithmic HBM bytes of one prefill: q, k, g (K wide) and v, o (V
    wide) per token and head, beta per token and head, A_log / dt_bias,
    and the state of every sequence read and written once.  Padding rows
    of g and beta are not read and not counted."""
    el = 2 if c.dtype == "bf16" else 4
    T, H, HV, K, V = c.T * c.B, c.H, c.HV, c.K, c.V
    return (T * H * K * 2 * el + T * HV * K * el + T * HV * V * 2 * el + T * HV * el
            + HV * 4 + HV * K * 4 + 2 * c.N * state_bytes(c))


def prefill_flops(c):
    """Per chunk and head 5 C^2 K + 3 * 2 C K V + C^3 / 3 (gated Grams, WY/UT
    products, inter-chunk products); partial chunks counted as full."""
    C = c.chunk_size
    n_chunks = sum(-(-int(n) // C) for n in c.lengths())
    return n_chunks * c.HV * (5 * C * C * c.K + 3 * 2 * C * c.K * c.V + C ** 3 / 3)


def decode_bytes(d):
    bf = 2
    return (d.B * d.mixed_qkv.shape[1] * bf + d.B * d.HV * d.K * bf + d.B * d.HV * bf
            + d.B * d.HV * d.V * bf + d.B * 2 * state_bytes(d))


def verify_bytes(v, snapshots=True):
    bf = 2
    cdim = v.mixed_qkv.shape[1]
    b = (v.B * v.N * (cdim + v.HV * v.K + v.HV) * bf          # mixed_qkv, a, b
         + v.B * cdim * 3 * bf + cdim * 4 * bf                # conv state, weights
         + v.B * v.N * v.HV * v.V * bf                       # o
         + v.B * state_bytes(v))                             # pool read
    return b + (v.B * v.N * state_bytes(v) if snapshots else 0)


def commit_bytes(v, accepted):
    n = int((accepted >= 0).sum())
    return n * 2 * state_bytes(v) + n * v.mixed_qkv.shape[1] * 3 * 2 * 2


def commit_replay_bytes(v, accepted):
    # per accepted request: pool state in and out, its draft inputs and conv
    # state re-read, and the conv roll
    n = int((accepted >= 0).sum())
    cdim = v.mixed_qkv.shape[1]
    return (n * 2 * state_bytes(v) + n * v.N * (cdim + v.HV * v.K + v.HV) * 2
            + n * cdim * 3 * 2 + n * cdim * 3 * 2 * 2)


def conv_state_bytes(d):
    """Conv state read and written (W - 1 = 3 entries per channel) and the
    weights, for one token of every request."""
    C = d.mixed_qkv.shape[1]
    return d.B * C * 3 * 2 * 2 + C * 4 * 2


def conv_update_bytes(d):
    C = d.mixed_qkv.shape[1]
    return d.B * C * (1 + 1 + 3 + 3) * 2 + C * 4 * 2


# ----------------------------------------------------------------- device calls

class Calls:
    """Device-resident inputs and one enqueue function per benchmarked call."""

    def __init__(self, hw: HostWork, with_configs: bool):
        import torch
        from linear_attention_03_amd import kda
        self.torch, self.kda, self.hw = torch, kda, hw
        self.dev = "cuda"
        self.fn, self.info = {}, {}
        self._prefill("prefill", hw.p4096, "prefill 1x4096 bf16")
        self._decode(hw.d)
        self._verify(hw.v, hw.accepted)
        if with_configs:
            self._prefill("prefill_tiny", hw.tiny, "tiny prefill 1x128 H=4 K=V=32 C=16 fp32")
            self._prefill("prefill_8192", hw.p8192, "prefill 1x8192 bf16")
            self._prefill("prefill_varlen", hw.varlen, "packed 8192 (9 sequences), g/beta padded to 12288")
            self._prefill("prefill_f32", hw.p4096_f32, "prefill 1x4096 fp32 inputs (the same values)")
            self._verify_tree(hw.vtree)
            for B, d in hw.d_small.items():
                self._decode_only(f"decode_{B}", d)
            for B, v in hw.v_small.items():
                self._verify_only(f"verify_{B}", v)
        self.scratch = None

    def to(self, x, dt="f32"):
        torch = self.torch
        t = torch.from_numpy(np.ascontiguousarray(x)).to(self.dev)
        return {"bf16": lambda: t.to(torch.bfloat16), "i32": lambda: t.to(torch.int32),
                "f32": lambda: t.float()}[dt]()

    def _add(self, name, fn, **info):
        self.fn[name] = fn
        self.info[name] = info

    def _prefill(self, name, c, what):
        torch, kda = self.torch, self.kda
        dt = c.dtype
        q, k, v, g, b = (self.to(x, dt) for x in (c.q, c.k, c.v, c.g, c.beta))
        A, dtb = self.to(c.A_log), self.to(c.dt_bias)
        pool, idx = self.to(c.pool), self.to(c.indices, "i32")
        cu = None if c.cu_seqlens is None else self.to(c.cu_seqlens, "i32")
        o = torch.empty(c.B, c.T, c.HV, c.V, dtype=q.dtype, device=self.dev)
        args = kda._prefill_args(q, k, v, g, b, o, scale=c.scale, initial_state=pool,
                                 initial_state_indices=idx, use_qk_l2norm_in_kernel=c.use_qk_l2norm,
                                 cu_seqlens=cu, A_log=A, dt_bias=dtb, lower_bound=c.lower_bound,
                                 beta_is_raw=c.beta_is_raw, chunk_size=c.chunk_size, intermediate_states=None)
        ws = torch.empty(max(kda.prefill_workspace_size(args), 1), dtype=torch.uint8, device=self.dev)
        path = kda.prefill_path_of(args)
        # matrix-core path: prep + scan; general path: the fp32-tile prep, the
        # exact prep for the chunks it flagged (not launched for a bounded gate
        # with lower_bound in [-8.75, 0], where no chunk can be flagged), the
        # fp32-tile scan
        bounded_safe = c.A_log is not None and c.lower_bound is not None and -8.75 <= c.lower_bound <= 0.0
        launches = 2 if path == "matrix" or bounded_safe else 3

        def run():
            kda.prefill(q, k, v, g, b, scale=c.scale, initial_state=pool, initial_state_indices=idx,
                        use_qk_l2norm_in_kernel=c.use_qk_l2norm, cu_seqlens=cu, A_log=A, dt_bias=dtb,
                        lower_bound=c.lower_bound, beta_is_raw=c.beta_is_raw, chunk_size=c.chunk_size,
                        o=o, workspace=ws)
        self._add(name, run, workload=what, tokens=c.T * c.B, bytes=prefill_bytes(c), flops=prefill_flops(c),
                  bound="hbm+mfma", launches=launches, path=path,
                  mfma_peak=BF16_MFMA_PEAK_TFLOPS if path == "matrix" else F32_MFMA_PEAK_TFLOPS)

    def _decode(self, d):
        kda = self.kda
        mixed = self.to(d.mixed_qkv, "bf16")
        HK = d.H * d.K
        q = mixed[:, :HK].view(d.B, d.H, d.K)
        k = mixed[:, HK:2 * HK].view(d.B, d.H, d.K)
        v = mixed[:, 2 * HK:].view(d.B, d.HV, d.V)
        a, b = self.to(d.a, "bf16"), self.to(d.b, "bf16")
        A, dtb = self.to(d.A_log), self.to(d.dt_bias)
        pool, idx = self.to(d.pool), self.to(d.indices, "i32")
        o = self.torch.empty(d.B, d.HV, d.V, dtype=self.torch.bfloat16, device=self.dev)

        def run():
            kda.decode(q, k, v, a, b, scale=d.scale, initial_state=pool, initial_state_indices=idx,
                       A_log=A, dt_bias=dtb, lower_bound=d.lower_bound, o=o)
        self._add("decode", run, workload="decode 48x1", tokens=d.B, bytes=decode_bytes(d),
                  bound="hbm", launches=1)
        # conv update of the same 48 requests' token (weights and state drawn like verify's)
        crng = np.random.default_rng(self.hw.wl.BASE_SEED + 6)
        C = d.mixed_qkv.shape[1]
        cw = self.to(self.hw.wl.round_bf16(crng.uniform(-0.5, 0.5, (C, 4)).astype(np.float32)), "bf16")
        ccs = self.to(self.hw.wl.round_bf16(crng.standard_normal((240, C, 3)).astype(np.float32)), "bf16")
        cy = self.torch.empty_like(mixed)

        def conv():
            kda.conv_update(mixed, conv_weight=cw, conv_state=ccs, conv_state_indices=idx, y=cy)
        self._add("conv_update", conv, workload="conv update 48 x 6144 channels, width 4", tokens=d.B,
                  bytes=conv_update_bytes(d), bound="hbm", launches=1)
        # the same decode step with its conv update fused in (own state copies)
        pool2, ccs2 = pool.clone(), ccs.clone()
        o2 = self.torch.empty_like(o)

        def decode_conv():
            kda.decode_conv(mixed, a, b, H=d.H, HV=d.HV, K=d.K, V=d.V, scale=d.scale, conv_weight=cw,
                            conv_state=ccs2, conv_state_indices=idx, initial_state=pool2,
                            initial_state_indices=idx, A_log=A, dt_bias=dtb, lower_bound=d.lower_bound, o=o2)
        self._add("decode_conv", decode_conv, workload="decode 48x1 with the width-4 conv update fused in",
                  tokens=d.B, bytes=decode_bytes(d) + conv_state_bytes(d), bound="hbm", launches=1)

    def _decode_only(self, name, d):
        kda = self.kda
        mixed = self.to(d.mixed_qkv, "bf16")
        HK = d.H * d.K
        q = mixed[:, :HK].view(d.B, d.H, d.K)
        k = mixed[:, HK:2 * HK].view(d.B, d.H, d.K)
        v = mixed[:, 2 * HK:].view(d.B, d.HV, d.V)
        a, b = self.to(d.a, "bf16"), self.to(d.b, "bf16")
        A, dtb = self.to(d.A_log), self.to(d.dt_bias)
        pool, idx = self.to(d.pool), self.to(d.indices, "i32")
        o = self.torch.empty(d.B, d.HV, d.V, dtype=self.torch.bfloat16, device=self.dev)

        def run():
            kda.decode(q, k, v, a, b, scale=d.scale, initial_state=pool, initial_state_indices=idx,
                       A_log=A, dt_bias=dtb, lower_bound=d.lower_bound, o=o)
        self._add(name, run, workload=f"decode {d.B}x1", tokens=d.B, bytes=decode_bytes(d),
                  bound="hbm", launches=1)

    def _verify_only(self, name, v):
        torch, kda = self.torch, self.kda
        x = self._verify_inputs(v)
        snap = torch.empty(v.B, v.N, v.HV, v.V, v.K, dtype=torch.float32, device=self.dev)
        o = torch.empty(v.B * v.N, v.HV, v.V, dtype=torch.bfloat16, device=self.dev)

        def run():
            kda.verify(x["mixed"], x["a"], x["b"], N=v.N, H=v.H, HV=v.HV, K=v.K, V=v.V, scale=v.scale,
                       conv_weight=x["w"], conv_state=x["cs"], initial_state=x["pool"],
                       initial_state_indices=x["idx"], snapshots=snap, A_log=x["A"], dt_bias=x["dt"],
                       lower_bound=v.lower_bound, o=o)
        self._add(name, run, workload=f"verify {v.B}x6 chain, conv width 4 + SiLU, snapshots",
                  tokens=v.B * v.N, bytes=verify_bytes(v), bound="hbm", launches=1)

    def _verify_inputs(self, v):
        return dict(mixed=self.to(v.mixed_qkv, "bf16"), a=self.to(v.a, "bf16"), b=self.to(v.b, "bf16"),
                    w=self.to(v.conv_weight, "bf16"), cs=self.to(v.conv_state, "bf16"),
                    A=self.to(v.A_log), dt=self.to(v.dt_bias), pool=self.to(v.pool),
                    idx=self.to(v.indices, "i32"),
                    parents=None if v.parents is None else self.to(v.parents, "i32"))

    def _verify(self, v, accepted):
        torch, kda = self.torch, self.kda
        x = self._verify_inputs(v)
        snap = torch.empty(v.B, v.N, v.HV, v.V, v.K, dtype=torch.float32, device=self.dev)
        o = torch.empty(v.B * v.N, v.HV, v.V, dtype=torch.bfloat16, device=self.dev)
        acc = self.to(accepted, "i32")
        kw = dict(N=v.N, H=v.H, HV=v.HV, K=v.K, V=v.V, scale=v.scale, conv_weight=x["w"],
                  conv_state=x["cs"], initial_state=x["pool"], initial_state_indices=x["idx"],
                  A_log=x["A"], dt_bias=x["dt"], lower_bound=v.lower_bound)

        def verify():
            kda.verify(x["mixed"], x["a"], x["b"], snapshots=snap, o=o, **kw)

        def commit():
            kda.commit(acc, N=v.N, snapshots=snap, initial_state=x["pool"], initial_state_indices=x["idx"],
                       conv_state=x["cs"], mixed_qkv=x["mixed"])

        def verify_nosnap():
            kda.verify(x["mixed"], x["a"], x["b"], snapshots=None, o=o, **kw)

        def commit_replay():
            kda.commit_replay(acc, x["mixed"], x["a"], x["b"], **kw)

        nacc = int((accepted >= 0).sum())
        self._add("verify", verify, workload="verify 48x6 chain, conv width 4 + SiLU, snapshots",
                  tokens=v.B * v.N, bytes=verify_bytes(v), bound="hbm", launches=1)
        self._add("commit", commit, workload=f"commit 48 requests ({nacc} accepted), snapshot copy + conv roll",
                  tokens=0, bytes=commit_bytes(v, accepted), bound="hbm", launches=1)
        self._add("verify_nosnap", verify_nosnap, workload="verify 48x6 chain, outputs only (commit by replay)",
                  tokens=v.B * v.N, bytes=verify_bytes(v, snapshots=False), bound="hbm", launches=1)
        self._add("commit_replay", commit_replay, workload=f"commit by replay, 48 requests ({nacc} accepted)",
                  tokens=0, bytes=commit_replay_bytes(v, accepted), bound="hbm", launches=2)

    def _verify_tree(self, v):
        torch, kda = self.torch, self.kda
        x = self._verify_inputs(v)
        snap = torch.empty(v.B, v.N, v.HV, v.V, v.K, dtype=torch.float32, device=self.dev)
        o = torch.empty(v.B * v.N, v.HV, v.V, dtype=torch.bfloat16, device=self.dev)

        def run():
            kda.verify(x["mixed"], x["a"], x["b"], N=v.N, H=v.H, HV=v.HV, K=v.K, V=v.V, scale=v.scale,
                       conv_weight=x["w"], conv_state=x["cs"], initial_state=x["pool"],
                       initial_state_indices=x["idx"], snapshots=snap, parents=x["parents"], A_log=x["A"],
                       dt_bias=x["dt"], lower_bound=v.lower_bound, o=o)
        self._add("verify_tree", run, workload="verify 48x6 random tree, conv width 4 + SiLU, snapshots",
                  tokens=v.B * v.N, bytes=verify_bytes(v), bound="hbm", launches=1)

    def copy(self):
        """A plain streaming kernel over COPY_BYTES (each element read once and
        written once): the calibration of the HBM byte counters."""
        torch = self.torch
        if not hasattr(self, "copy_src"):
            self.copy_src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=self.dev)
            self.copy_dst = torch.empty_like(self.copy_src)
        torch.neg(self.copy_src, out=self.copy_dst)

    def evict(self):
        """Leave no line of the next call's inputs in any cache: write
        COLD_BYTES, then read another COLD_BYTES, so that the caches hold
        clean lines of the second buffer.  (After the write alone they would
        hold dirty lines whose write-back would then run inside the timed
        call.)"""
        torch = self.torch
        if self.scratch is None:
            self.scratch = torch.empty(COLD_BYTES // 4, dtype=torch.int32, device=self.dev)
            self.scratch_r = torch.ones(COLD_BYTES // 4, dtype=torch.int32, device=self.dev)
            self.scratch_sum = torch.empty((), dtype=torch.int64, device=self.dev)
        self.scratch.fill_(7)
        torch.sum(self.scratch_r, 0, dtype=torch.int64, out=self.scratch_sum)


# ----------------------------------------------------------------- timing

class Spin:
    """Holds the current stream with a GPU busy-wait while the host enqueues."""

    def __init__(self, torch):
        self.torch = torch
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 10_000_000
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        torch.cuda.synchronize()
        self.rate = n / (e0.elapsed_time(e1) * 1e-3)

    def hold(self, ms):
        self.torch.cuda._sleep(max(int(ms * 1e-3 * self.rate), 1))


class EventPool:
    """Timing events created up front (recorded once so that they exist)."""

    def __init__(self, torch, n):
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.ev:
            e.record()
        torch.cuda.synchronize()


def timed_calls(calls, spin, seq, evs):
    """Enqueue `seq` (a list of (name or None, cold)) behind a spin kernel;
    each named call is stamped with its own call events.  Returns the µs of
    each named call, in order."""
    torch, kda = calls.torch, calls.kda
    n = sum(1 for name, _ in seq if name)
    assert 2 * n <= len(evs.ev)
    torch.cuda.synchronize()
    spin.hold(10.0 + 0.25 * len(seq))
    i = 0
    for name, cold in seq:
        if cold:
            calls.evict()
        if name:
            kda.set_call_events(evs.ev[2 * i], evs.ev[2 * i + 1])
            calls.fn[name]()
            i += 1
    torch.cuda.synchronize()
    return [evs.ev[2 * j].elapsed_time(evs.ev[2 * j + 1]) * 1e3 for j in range(n)]


def time_step_eager(calls, spin, steps, evs):
    seq = [(ph, False) for _ in range(steps) for ph in STEP]
    us = timed_calls(calls, spin, seq, evs)
    per = {ph: us[i::len(STEP)] for i, ph in enumerate(STEP)}
    return per


def time_step_graph(calls, spin, steps, branches):
    """One step captured as a HIP graph (every call enqueues its kernels on
    the capturing stream; the library allocates and synchronises nothing),
    replayed `steps` times back to back behind a spin kernel.  `branches`
    lists the phases of each branch in order: one branch is the one-stream
    step; with two, the second branch forks from the first at the start of
    the step and joins it at the end, so its phases run concurrently with
    the first branch's (the phases touch disjoint pools and buffers)."""
    torch = calls.torch
    side = torch.cuda.Stream()
    other = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def body():
        if len(branches) > 1:
            other.wait_stream(side)
        for ph in branches[0]:
            calls.fn[ph]()
        for br in branches[1:]:
            with torch.cuda.stream(other):
                for ph in br:
                    calls.fn[ph]()
        if len(branches) > 1:
            side.wait_stream(other)

    with torch.cuda.stream(side):
        body()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spin.hold(10.0 + 0.5 * steps)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def sample_configs(calls, spin, names, samples, warmup):
    """Hot and cold samples (µs) of every call in `names`, in batches."""
    evs = EventPool(calls.torch, 2 * 64)
    out = {}
    for name in names:
        for _ in range(warmup):
            calls.fn[name]()
        hot, cold = [], []
        left = samples
        while left > 0:
            n = min(left, 32)
            hot += timed_calls(calls, spin, [(name, False)] * n, evs)
            cold += timed_calls(calls, spin, [(name, True)] * n, evs)
            left -= n
        out[name] = {"hot": hot, "cold": cold}
        log(f"  {name}: hot median {np.median(hot):.2f} us, cold median {np.median(cold):.2f} us")
    return out


def sample_only(args):
    """Child process: per-workload samples only, one JSON line on stdout."""
    import torch
    from linear_attention_03_amd import kda
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    kda.lib()
    hw = HostWork()
    hw.configs()
    calls = Calls(hw, with_configs=True)
    spin = Spin(torch)
    res = sample_configs(calls, spin, list(calls.fn), args.samples, args.warmup)
    print(json.dumps({"samples": res}), flush=True)


# ----------------------------------------------------------------- CPU baseline

def _oracle_step_part(job):
    """One share of an oracle step (run in a pool worker): ('prefill', heads)
    or ('decode' | 'verify', requests)."""
    from threadpoolctl import threadpool_limits
    from oracle import kda as ok
    kind, sel = job
    with threadpool_limits(1):
        if kind == "prefill":
            p = _POOL_HW.p4096
            heads = list(sel)
            dt = p.dt_bias.reshape(p.HV, p.K)[heads].reshape(-1)
            ok.prefill(p.q[:, :, heads], p.k[:, :, heads], p.v[:, :, heads], p.g[:, :, heads],
                       p.beta[:, :, heads], scale=p.scale, initial_state=p.pool[p.indices][:, heads],
                       initial_state_indices=np.arange(1), use_qk_l2norm_in_kernel=True,
                       A_log=p.A_log[heads], dt_bias=dt, lower_bound=p.lower_bound, beta_is_raw=True)
        elif kind == "decode":
            d = _POOL_HW.d
            r = list(sel)
            ok.decode(d.q()[r], d.k()[r], d.v()[r], d.a[r], d.b[r], scale=d.scale, initial_state=d.pool,
                      initial_state_indices=d.indices[r], A_log=d.A_log, dt_bias=d.dt_bias,
                      lower_bound=d.lower_bound)
        else:
            v = _POOL_HW.v
            r = list(sel)
            rows = np.concatenate([np.arange(i * v.N, (i + 1) * v.N) for i in r])
            ok.verify(v.mixed_qkv[rows], v.a[rows], v.b[rows], N=v.N, H=v.H, HV=v.HV, K=v.K, V=v.V,
                      scale=v.scale, conv_weight=v.conv_weight, conv_state=v.conv_state,
                      initial_state=v.pool, initial_state_indices=v.indices[r], A_log=v.A_log,
                      dt_bias=v.dt_bias, lower_bound=v.lower_bound)
    return kind


_POOL_HW = None


def _step_jobs(hw, parts):
    p, d, v = hw.p4096, hw.d, hw.v
    jobs = [("prefill", h) for h in np.array_split(np.arange(p.HV), min(parts, p.HV))]
    jobs += [("decode", r) for r in np.array_split(np.arange(d.B), max(1, parts // 4))]
    jobs += [("verify", r) for r in np.array_split(np.arange(v.B), max(1, parts // 2))]
    return jobs


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(hw, min_seconds=8.0):
    """fp64 oracle over whole steps (prefill 1 x 4096, decode 48 x 1,
    verify 48 x 6 chain), once on one thread and once over every core
    (heads of the prefill and requests of decode / verify spread over a
    process pool; each worker runs the oracle on one thread).  Runs before
    the process touches the GPU."""
    import multiprocessing as mp
    global _POOL_HW
    _POOL_HW = hw
    tokens = hw.p4096.T + hw.d.B + hw.v.B * hw.v.N
    cores = min(os.cpu_count() or 1, 16)
    res = {}
    # one thread: whole steps in this process
    t0, reps = time.perf_counter(), 0
    while time.perf_counter() - t0 < min_seconds:
        for job in _step_jobs(hw, 1):
            _oracle_step_part(job)
        reps += 1
    t1 = time.perf_counter() - t0
    res["one_thread"] = {"value": round(tokens * reps / t1, 1), "steps": reps, "seconds": round(t1, 2)}
    # all cores: the same steps split over a fork pool
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_step_part, _step_jobs(hw, cores)[:cores])      # warm the workers
        t0, reps = time.perf_counter(), 0
        while time.perf_counter() - t0 < min_seconds:
            pool.map(_oracle_step_part, _step_jobs(hw, cores))
            reps += 1
        t2 = time.perf_counter() - t0
    res["all_cores"] = {"value": round(tokens * reps / t2, 1), "steps": reps, "seconds": round(t2, 2),
                        "processes": cores}
    return {"value": res["all_cores"]["value"], "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"fp64 NumPy oracle on whole steps (prefill 1x{hw.p4096.T}, decode 48x1, verify 48x6 "
                       f"chain; commit not timed): {res['all_cores']['steps']} step(s) over {cores} worker "
                       f"processes (heads / requests split), {res['one_thread']['steps']} step(s) on one thread"),
            "one_thread": res["one_thread"], "all_cores": res["all_cores"],
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}


# ----------------------------------------------------------------- traffic

def _counter_means(run_dir, counter):
    """Mean counter value per dispatch (KiB), keyed by the phase whose
    kernel the dispatch ran, from a rocprofv3 --pmc CSV run directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = next((TRAFFIC_KERNELS[m] + ":" + m for m in TRAFFIC_KERNELS if m in name), None)
            if key is None and "neg_kernel" in name:
                key = "copy:copy"
            if key is not None:
                d = (key, r.get("Dispatch_Id", len(per)))
                per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    sums = {}
    for (key, _), val in per.items():
        sums.setdefault(key, []).append(val)
    return {k: float(np.mean(v)) for k, v in sums.items()}, {k: len(v) for k, v in sums.items()}


def write_traffic(fetch_dir, write_dir):
    fetch, nf = _counter_means(fetch_dir, "FETCH_SIZE")
    write, nw = _counter_means(write_dir, "WRITE_SIZE")
    kib = COPY_BYTES / 1024
    f_scale, w_scale = fetch["copy:copy"] / kib, write["copy:copy"] / kib
    out = {"copy_calibration": {"bytes_each_way": COPY_BYTES, "fetch_kib": fetch["copy:copy"],
                                "write_kib": write["copy:copy"], "fetch_factor": f_scale,
                                "write_factor": w_scale}}
    h = source_hash()
    for phase in ("prefill", "decode", "verify", "commit"):
        keys = [k for k in fetch if k.startswith(phase + ":")]
        if not keys or any(k not in write for k in keys):
            continue
        f_b = sum(fetch[k] for k in keys) * 1024 / f_scale       # one dispatch of each kernel per call
        w_b = sum(write[k] for k in keys) * 1024 / w_scale
        out[phase] = {"source_hash": h, "bytes_per_call": round(f_b + w_b), "fetch_bytes": round(f_b),
                      "write_bytes": round(w_b), "dispatches_counted": {k: nf[k] for k in keys},
                      "raw_kib": {k: {"FETCH_SIZE": round(fetch[k]), "WRITE_SIZE": round(write[k])} for k in keys}}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def traffic_for(phase):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    ent = json.load(open(TRAFFIC_FILE)).get(phase)
    if ent and ent.get("source_hash") == source_hash():
        return ent.get("bytes_per_call")
    return None


# ----------------------------------------------------------------- reporting

def pct(x):
    x = np.asarray(x, dtype=np.float64)
    return {"median": round(float(np.median(x)), 2), "p10": round(float(np.percentile(x, 10)), 2),
            "p90": round(float(np.percentile(x, 90)), 2), "mean": round(float(np.mean(x)), 2), "n": int(x.size)}


def roofline_entry(info, us, phase):
    """Roofline of one call at `us` µs per call."""
    t = us * 1e-6
    gbps = info["bytes"] / t / 1e9
    e = {"phase": phase, "us_per_call": round(us, 2), "algorithmic_bytes_per_call": info["bytes"],
         "achieved_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    if info.get("flops"):
        peak = info.get("mfma_peak", BF16_MFMA_PEAK_TFLOPS)
        tf = info["flops"] / t / 1e12
        t_hbm = info["bytes"] / (HBM_PEAK_GBPS * 1e9)
        t_mfma = info["flops"] / (peak * 1e12)
        e.update({"algorithmic_flops_per_call": round(info["flops"]), "achieved_TFLOPs": round(tf, 2),
                  "mfma_frac": round(tf / peak, 4), "mfma_peak_TFLOPs": peak,
                  "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                  "floor_us": round(max(t_hbm, t_mfma) * 1e6, 2),
                  "roofline_frac": round(max(t_hbm, t_mfma) / t, 4)})
    else:
        e.update({"bound": "hbm", "floor_us": round(info["bytes"] / (HBM_PEAK_GBPS * 1e9) * 1e6, 2),
                  "roofline_frac": round(gbps / HBM_PEAK_GBPS, 4)})
    return e


def main():
    if len(sys.argv) == 4 and sys.argv[1] == "--write-traffic":
        write_traffic(sys.argv[2], sys.argv[3])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--samples", type=int, default=64, help="hot and cold samples per workload and process")
    ap.add_argument("--sample-procs", type=int, default=3, help="processes taking per-workload samples")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="time the step only")
    ap.add_argument("--traffic-run", action="store_true",
                    help="step calls and the calibration copy only (rocprofv3 --pmc runs)")
    ap.add_argument("--sample-only", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the one-GPU path only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "libkda's kernels run on one GPU and do not shard across GPUs.", file=sys.stderr)
        sys.exit(2)
    if args.sample_only:
        sample_only(args)
        return

    hw = HostWork()
    with_configs = not (args.no_configs or args.traffic_run)
    cpu = None
    if not args.no_cpu_baseline and not args.traffic_run:
        log("timing the oracle on the host (cpu_baseline), before any GPU use")
        cpu = cpu_baseline(hw)
    child_samples = []
    if with_configs:
        hw.configs()
        for i in range(max(args.sample_procs - 1, 0)):
            log(f"per-workload samples, process {i + 2} of {args.sample_procs}")
            r = subprocess.run([sys.executable, os.path.abspath(__file__), "--sample-only",
                                "--samples", str(args.samples), "--warmup", str(args.warmup)],
                               stdout=subprocess.PIPE, text=True, timeout=600)
            if r.returncode != 0:
                print(f"sampling process failed with exit status {r.returncode}", file=sys.stderr)
                sys.exit(r.returncode or 1)
            child_samples.append(json.loads(r.stdout.strip().splitlines()[-1])["samples"])

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from linear_attention_03_amd import kda
    kda.lib()
    log(f"device {torch.cuda.get_device_name(0)}; building workloads")
    calls = Calls(hw, with_configs=with_configs)
    spin = Spin(torch)
    if args.traffic_run:
        for _ in range(args.steps):
            for ph in STEP:
                calls.fn[ph]()
            calls.copy()
        torch.cuda.synchronize()
        log("traffic run done")
        return
    tokens = hw.p4096.T + hw.d.B + hw.v.B * hw.v.N
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        for ph in STEP:
            calls.fn[ph]()
    torch.cuda.synchronize()
    evs = EventPool(torch, 2 * len(STEP) * args.steps)
    log(f"timing {args.steps} eager steps (call events per phase)")
    per = time_step_eager(calls, spin, args.steps, evs)
    eager_ms = sum(float(np.sum(v)) for v in per.values()) / args.steps / 1e3
    graph_ms = time_step_graph(calls, spin, args.steps, STEP_BRANCHES)
    serial_ms = time_step_graph(calls, spin, args.steps, [STEP])
    log(f"graph: {graph_ms * 1e3:.1f} us/step (two branches), {serial_ms * 1e3:.1f} us/step (one stream); "
        f"kernels in the step {eager_ms * 1e3:.1f} us")

    phases = {}
    for ph in STEP:
        info = calls.info[ph]
        st = pct(per[ph])
        ent = {"workload": info["workload"], "us": st["mean"], "us_median": st["median"],
               "us_p10": st["p10"], "us_p90": st["p90"],
               "tokens_per_s": round(info["tokens"] / (st["mean"] * 1e-6), 1) if info["tokens"] else None}
        ent.update({k: v for k, v in roofline_entry(info, st["mean"], ph).items() if k not in ("phase", "us_per_call")})
        ent["traffic_bytes_per_call"] = traffic_for(ph)
        phases[ph] = ent

    configs = None
    if with_configs:
        log(f"per-workload samples, process 1 of {args.sample_procs}")
        mine = sample_configs(calls, spin, list(calls.fn), args.samples, args.warmup)
        configs = {}
        for name in calls.fn:
            hot = list(mine[name]["hot"]) + [x for c in child_samples for x in c[name]["hot"]]
            cold = list(mine[name]["cold"]) + [x for c in child_samples for x in c[name]["cold"]]
            info = calls.info[name]
            h, c = pct(hot), pct(cold)
            ent = {"workload": info["workload"], "launches": info["launches"], "hot_us": h, "cold_us": c,
                   **({"prefill_path": info["path"]} if "path" in info else {}),
                   "tokens_per_s_cold": round(info["tokens"] / (c["median"] * 1e-6), 1) if info["tokens"] else None,
                   "roofline_cold": roofline_entry(info, c["median"], name)}
            configs[name] = ent

    # the dominant single kernel of the step: the verify launch
    dom = max((ph for ph in STEP if calls.info[ph]["launches"] == 1), key=lambda ph: phases[ph]["us"])
    achieved = phases[dom]["achieved_GBps"]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_for(dom),
                "kernel": "verify_kernel<bf16,128,128,8,chain,snapshots,32 rows>", "phase": dom,
                "algorithmic_bytes_per_call": calls.info[dom]["bytes"], "us_per_call": phases[dom]["us"],
                "timing": "mean kernel time of the call over the timed eager steps (call events)"}
    roofline_phases = {ph: roofline_entry(calls.info[ph], phases[ph]["us"], ph) for ph in STEP}
    out = {
        "metric": METRIC,
        "value": round(tokens / (graph_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(graph_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16/bf16 MFMA operands + fp32 state and accumulation",
        "data": "synthetic",
        "config": {"workload": f"KDA step: prefill 1x{hw.p4096.T} + decode 48x1 + verify 48x6 chain (conv4) + commit",
                   "heads": 16, "head_dim": 128, "inputs": "bf16", "state": "fp32",
                   "prefill_products": "fp16 / bf16 MFMA operands, fp32 accumulation",
                   "decode_verify_math": "fp32", "chunk_size": hw.p4096.chunk_size, "tokens_per_step": tokens,
                   "launch": "one HIP graph per step, replayed back to back: prefill on one branch, "
                             "verify -> decode -> commit on a second (fork at the start, join at the end)"},
        "one_stream_graph_ms_per_step": round(serial_ms, 4),
        "eager_kernel_ms_per_step": round(eager_ms, 4),
        "phases": phases,
        "roofline": roofline,
        "roofline_phases": roofline_phases,
    }
    if configs is not None:
        out["configs"] = configs
        out["configs_method"] = (f"per call: {args.samples} hot (back to back) and {args.samples} cold (512 MiB "
                                 f"written, then 512 MiB read, before each) samples in each of {args.sample_procs} processes; kernel time "
                                 "from call events")
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
