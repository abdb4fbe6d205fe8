#!/usr/bin/env python3
"""Throughput of the KDA hot path on one MI355X.

One step = one call of every phase on its workload, back to back on one
stream, inputs resident in HBM:
  prefill  1 x 4096 tokens, 16 heads of 128 x 128, bf16, chunk 64
  decode   48 requests x 1 token (packed mixed_qkv), in-place pool update
  verify   48 requests x 6 draft tokens (chain), width-4 causal conv + SiLU,
           one fp32 snapshot per draft token
  commit   48 requests, accepted node drawn once (seeded)
value = tokens per step (4096 + 48 + 288) / seconds per step.

Timing: W untimed warmup steps; then a GPU spin kernel holds the stream
while the host enqueues all K steps with HIP events between the phases, so
the events measure back-to-back GPU work with no host gaps.  Per-phase
averages come from those events.  The step is then captured once as a HIP
graph and K replays are timed the same way; `value` and `ms_per_step` come
from the replays (`--eager` keeps the eager figure), `eager_ms_per_step`
reports the other. the roofline entry is for the
single-launch kernel with the largest time.  Its `traffic` is the HBM bytes
per launch from rocprofv3's FETCH_SIZE and WRITE_SIZE counters, each scaled
by what the same counter reads for a plain copy of known size (the `copy`
phase), stored in profiles/traffic.json together with a hash of the kernel
sources so that a stale figure is reported as null.  The oracle (fp64 NumPy, one thread) is timed on a
bounded sample of the same workloads and scaled to the same unit.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --write-traffic FETCH_DIR WRITE_DIR   (after two --pmc runs)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA tokens/s + µs/call per phase (16 heads×128) on 1 MI355X; % HBM/MFMA peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash():
    d = os.path.join(ROOT, "linear_attention_03_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class Workloads:
    """Device-resident inputs of one step."""

    def __init__(self, prefill_T):
        import torch
        from linear_attention_03_amd import kda, workloads as wl
        self.torch, self.kda = torch, kda
        dev = "cuda"

        def to(x, dt="f32"):
            t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
            return {"bf16": lambda: t.to(torch.bfloat16), "i32": lambda: t.to(torch.int32),
                    "f32": lambda: t.float()}[dt]()

        p = wl.config2_prefill(prefill_T)
        self.p = p
        self.pq, self.pk, self.pv = to(p.q, "bf16"), to(p.k, "bf16"), to(p.v, "bf16")
        self.pg, self.pb = to(p.g, "bf16"), to(p.beta, "bf16")
        self.pA, self.pdt = to(p.A_log), to(p.dt_bias)
        self.ppool, self.pidx = to(p.pool), to(p.indices, "i32")
        self.po = torch.empty(1, p.T, p.HV, p.V, dtype=torch.bfloat16, device=dev)
        args = kda._prefill_args(self.pq, self.pk, self.pv, self.pg, self.pb, self.po, scale=p.scale,
                                 initial_state=self.ppool, initial_state_indices=self.pidx,
                                 use_qk_l2norm_in_kernel=True, cu_seqlens=None, A_log=self.pA,
                                 dt_bias=self.pdt, lower_bound=p.lower_bound, beta_is_raw=True,
                                 chunk_size=p.chunk_size, intermediate_states=None)
        self.pws = torch.empty(max(kda.prefill_workspace_size(args), 1), dtype=torch.uint8, device=dev)

        d = wl.config1_decode()
        self.d = d
        self.dmixed = to(d.mixed_qkv, "bf16")
        HK = d.H * d.K
        self.dq = self.dmixed[:, :HK].view(d.B, d.H, d.K)
        self.dk = self.dmixed[:, HK:2 * HK].view(d.B, d.H, d.K)
        self.dv = self.dmixed[:, 2 * HK:].view(d.B, d.HV, d.V)
        self.da, self.db = to(d.a, "bf16"), to(d.b, "bf16")
        self.dA, self.ddt = to(d.A_log), to(d.dt_bias)
        self.dpool, self.didx = to(d.pool), to(d.indices, "i32")
        self.do = torch.empty(d.B, d.HV, d.V, dtype=torch.bfloat16, device=dev)
        # conv update ahead of a decode step: one token of 48 requests over the
        # q || k || v channels, width 4 (weights and state drawn like verify's)
        crng = np.random.default_rng(wl.BASE_SEED + 6)
        C = d.mixed_qkv.shape[1]
        self.cw = to(wl.round_bf16(crng.uniform(-0.5, 0.5, (C, 4)).astype(np.float32)), "bf16")
        self.ccs = to(wl.round_bf16(crng.standard_normal((240, C, 3)).astype(np.float32)), "bf16")
        self.cy = torch.empty_like(self.dmixed)

        v = wl.config4_verify(tree=False)
        self.v = v
        self.vmixed, self.va, self.vb = to(v.mixed_qkv, "bf16"), to(v.a, "bf16"), to(v.b, "bf16")
        self.vw, self.vcs = to(v.conv_weight, "bf16"), to(v.conv_state, "bf16")
        self.vA, self.vdt = to(v.A_log), to(v.dt_bias)
        self.vpool, self.vidx = to(v.pool), to(v.indices, "i32")
        self.vsnap = torch.empty(v.B, v.N, v.HV, v.V, v.K, dtype=torch.float32, device=dev)
        self.vo = torch.empty(v.B * v.N, v.HV, v.V, dtype=torch.bfloat16, device=dev)
        rng = np.random.default_rng(wl.BASE_SEED + 5)
        self.accepted = to(rng.integers(-1, v.N, v.B).astype(np.int32), "i32")
        self.copy_src = self.copy_dst = None

    def copy(self):
        """A plain streaming kernel over COPY_BYTES (each element read once and
        written once, negated so that it is a kernel and not a DMA copy): the
        calibration for the HBM byte counters, never part of a step."""
        if self.copy_src is None:
            n = COPY_BYTES // 4
            self.copy_src = self.torch.ones(n, dtype=self.torch.int32, device="cuda")
            self.copy_dst = self.torch.empty_like(self.copy_src)
        self.torch.neg(self.copy_src, out=self.copy_dst)

    # one call per phase -------------------------------------------------
    def prefill(self):
        p = self.p
        self.kda.prefill(self.pq, self.pk, self.pv, self.pg, self.pb, scale=p.scale,
                         initial_state=self.ppool, initial_state_indices=self.pidx,
                         use_qk_l2norm_in_kernel=True, A_log=self.pA, dt_bias=self.pdt,
                         lower_bound=p.lower_bound, beta_is_raw=True, chunk_size=p.chunk_size,
                         o=self.po, workspace=self.pws)

    def decode(self):
        d = self.d
        self.kda.decode(self.dq, self.dk, self.dv, self.da, self.db, scale=d.scale,
                        initial_state=self.dpool, initial_state_indices=self.didx, A_log=self.dA,
                        dt_bias=self.ddt, lower_bound=d.lower_bound, o=self.do)

    def verify(self):
        v = self.v
        self.kda.verify(self.vmixed, self.va, self.vb, N=v.N, H=v.H, HV=v.HV, K=v.K, V=v.V,
                        scale=v.scale, conv_weight=self.vw, conv_state=self.vcs,
                        initial_state=self.vpool, initial_state_indices=self.vidx,
                        snapshots=self.vsnap, A_log=self.vA, dt_bias=self.vdt,
                        lower_bound=v.lower_bound, o=self.vo)

    def commit(self):
        v = self.v
        self.kda.commit(self.accepted, N=v.N, snapshots=self.vsnap, initial_state=self.vpool,
                        initial_state_indices=self.vidx, conv_state=self.vcs, mixed_qkv=self.vmixed)

    # commit by replay: verify without snapshots, then the replayed commit
    def verify_nosnap(self):
        v = self.v
        self.kda.verify(self.vmixed, self.va, self.vb, N=v.N, H=v.H, HV=v.HV, K=v.K, V=v.V,
                        scale=v.scale, conv_weight=self.vw, conv_state=self.vcs,
                        initial_state=self.vpool, initial_state_indices=self.vidx,
                        snapshots=None, A_log=self.vA, dt_bias=self.vdt,
                        lower_bound=v.lower_bound, o=self.vo)

    def commit_replay(self):
        v = self.v
        self.kda.commit_replay(self.accepted, self.vmixed, self.va, self.vb, N=v.N, H=v.H, HV=v.HV,
                               K=v.K, V=v.V, scale=v.scale, conv_weight=self.vw, conv_state=self.vcs,
                               initial_state=self.vpool, initial_state_indices=self.vidx,
                               A_log=self.vA, dt_bias=self.vdt, lower_bound=v.lower_bound)

    def conv_update(self):
        self.kda.conv_update(self.dmixed, conv_weight=self.cw, conv_state=self.ccs,
                             conv_state_indices=self.didx, y=self.cy)

    # algorithmic bytes / flops per call --------------------------------
    def phase_bytes(self):
        p, d, v = self.p, self.d, self.v
        state = lambda c: c.HV * c.V * c.K * 4                       # noqa: E731
        bf = 2
        prefill = (p.T * p.H * p.K * 3 * bf + p.T * p.H * p.V * bf      # q, k, g ; v
                   + p.T * p.H * bf + p.T * p.HV * p.V * bf             # beta ; o
                   + p.H * p.K * 4 * 2 + 2 * state(p))                 # A_log/dt_bias ; state in + out
        decode = (d.B * d.mixed_qkv.shape[1] * bf + d.B * d.HV * d.K * bf + d.B * d.HV * bf
                  + d.B * d.HV * d.V * bf + d.B * 2 * state(d))
        cdim = v.mixed_qkv.shape[1]
        verify = (v.B * v.N * (cdim + v.HV * v.K + v.HV) * bf          # mixed_qkv, a, b
                  + v.B * cdim * 3 * bf + cdim * 4 * bf                # conv state, weights
                  + v.B * v.N * v.HV * v.V * bf                       # o
                  + v.B * state(v) + v.B * v.N * state(v))            # pool read, snapshots written
        acc = self.accepted.cpu().numpy()
        n_acc = int((acc >= 0).sum())
        commit = n_acc * 2 * state(v) + n_acc * cdim * 3 * bf * 2
        verify_nosnap = verify - v.B * v.N * state(v)
        # replay: per accepted request its pool state in and out, its draft
        # inputs and conv state re-read, and the conv roll
        commit_replay = (n_acc * 2 * state(v) + n_acc * v.N * (cdim + v.HV * v.K + v.HV) * bf
                         + n_acc * cdim * 3 * bf + n_acc * cdim * 3 * bf * 2)
        C = d.mixed_qkv.shape[1]
        conv_update = d.B * C * (1 + 1 + 3 + 3) * bf + C * 4 * bf    # x, y, state in + out; weights
        return {"prefill": prefill, "decode": decode, "verify": verify, "commit": commit,
                "conv_update": conv_update,
                "verify_nosnap": verify_nosnap, "commit_replay": commit_replay, "copy": 2 * COPY_BYTES}

    def prefill_flops(self):
        # per full chunk x head: 5 C^2 K + 3 * 2 C K V + C^3 / 3 (gated Grams, WY/UT
        # products, inter-chunk products); partial chunks counted as full
        p = self.p
        C = p.chunk_size
        n_chunks = -(-p.T // C) * p.B
        return n_chunks * p.H * (5 * C * C * p.K + 3 * 2 * C * p.K * p.V + C ** 3 / 3)


PHASES = ["prefill", "decode", "verify", "commit"]
REPLAY_PHASES = ["verify_nosnap", "commit_replay"]
LAUNCHES = {"prefill": 2, "decode": 1, "verify": 1, "commit": 1, "copy": 1,
            "verify_nosnap": 1, "commit_replay": 2, "conv_update": 1}
KERNEL_NAMES = {"prefill": "prep_mfma_kernel + scan_mfma_kernel", "decode": "decode_kernel",
                "verify": "verify_kernel", "commit": "commit_kernel", "copy": "torch neg (int32)",
                "verify_nosnap": "verify_kernel (no snapshots)",
                "commit_replay": "verify_kernel (replay) + commit_kernel (conv roll)",
                "conv_update": "conv_update_kernel"}
COPY_BYTES = 256 << 20
TOKENS = None


def spin_ms(torch, ms):
    """Hold the current stream for about `ms` milliseconds."""
    cycles = int(ms * 1e-3 * spin_ms.rate)
    torch.cuda._sleep(max(cycles, 1))


def calibrate_spin(torch):
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10_000_000
    e0.record()
    torch.cuda._sleep(n)
    e1.record()
    torch.cuda.synchronize()
    spin_ms.rate = n / (e0.elapsed_time(e1) * 1e-3)


def time_steps(wk, steps, phases):
    torch = wk.torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    spin_ms(torch, 20.0 + 2.0 * steps)
    t_host0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        for i, ph in enumerate(phases):
            getattr(wk, ph)()
            ev[s][i + 1].record()
    t_enqueue = time.perf_counter() - t_host0
    torch.cuda.synchronize()
    per = {ph: [] for ph in phases}
    for s in range(steps):
        for i, ph in enumerate(phases):
            per[ph].append(ev[s][i].elapsed_time(ev[s][i + 1]) * 1e3)   # us
    total_ms = ev[0][0].elapsed_time(ev[-1][-1])
    return total_ms, per, t_enqueue


def time_graph(wk, steps, phases):
    """One step captured as a HIP graph (every call of the step enqueues its
    kernels on the capturing stream; the library allocates and synchronises
    nothing), replayed `steps` times back to back behind a spin kernel."""
    torch = wk.torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for ph in phases:
            getattr(wk, ph)()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for ph in phases:
                getattr(wk, ph)()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spin_ms(torch, 20.0 + 2.0 * steps)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), graph


def cpu_baseline(wk, min_seconds=10.0):
    """fp64 oracle on one host thread over whole steps of the same workloads
    (prefill 1 x T, decode 48 x 1, verify 48 x 6 chain), repeated until at
    least `min_seconds` of CPU work; commit (a copy) is not timed."""
    from threadpoolctl import threadpool_limits
    from oracle import kda as ok
    p, d, v = wk.p, wk.d, wk.v
    reps, spent = 0, 0.0
    with threadpool_limits(1):
        while spent < min_seconds:
            t0 = time.perf_counter()
            ok.prefill(p.q, p.k, p.v, p.g, p.beta, scale=p.scale,
                       initial_state=p.pool[p.indices], initial_state_indices=np.arange(1),
                       use_qk_l2norm_in_kernel=True, A_log=p.A_log, dt_bias=p.dt_bias,
                       lower_bound=p.lower_bound, beta_is_raw=True)
            ok.decode(d.q(), d.k(), d.v(), d.a, d.b, scale=d.scale, initial_state=d.pool,
                      initial_state_indices=d.indices, A_log=d.A_log, dt_bias=d.dt_bias,
                      lower_bound=d.lower_bound)
            ok.verify(v.mixed_qkv, v.a, v.b, N=v.N, H=v.H, HV=v.HV, K=v.K, V=v.V,
                      scale=v.scale, conv_weight=v.conv_weight, conv_state=v.conv_state,
                      initial_state=v.pool, initial_state_indices=v.indices, A_log=v.A_log,
                      dt_bias=v.dt_bias, lower_bound=v.lower_bound)
            spent += time.perf_counter() - t0
            reps += 1
    return {"value": round(TOKENS * reps / spent, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"fp64 NumPy oracle, 1 thread: {reps} whole step(s) (prefill 1x{p.T}, decode 48x1, "
                       f"verify 48x6 chain; commit not timed)"),
            "seconds_measured": round(spent, 2)}


def _counter_means(run_dir, counter):
    """Mean counter value per dispatch (KiB), keyed by the phase whose
    kernel the dispatch ran, from a rocprofv3 --pmc CSV run directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    match = {"prep_mfma_kernel": "prefill", "scan_mfma_kernel": "prefill", "decode_kernel": "decode",
             "verify_kernel": "verify", "commit_kernel": "commit"}
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = next((match[m] for m in match if m in name), None)
            if key is None and "neg_kernel" in name:
                key = "copy"
            if key is not None:
                per.setdefault((key, r.get("Dispatch_Id", len(per))), 0.0)
                per[(key, r.get("Dispatch_Id", len(per)))] += float(r["Counter_Value"])
    sums = {}
    for (key, _), val in per.items():
        sums.setdefault(key, []).append(val)
    return {k: float(np.mean(v)) for k, v in sums.items()}, {k: len(v) for k, v in sums.items()}


def write_traffic(fetch_dir, write_dir):
    fetch, nf = _counter_means(fetch_dir, "FETCH_SIZE")
    write, nw = _counter_means(write_dir, "WRITE_SIZE")
    kib = COPY_BYTES / 1024
    f_scale, w_scale = fetch["copy"] / kib, write["copy"] / kib
    out = {"copy_calibration": {"bytes_each_way": COPY_BYTES, "fetch_kib": fetch["copy"],
                                "write_kib": write["copy"], "fetch_factor": f_scale,
                                "write_factor": w_scale}}
    h = source_hash()
    for k in ("prefill", "decode", "verify", "commit"):
        if k not in fetch or k not in write:
            continue
        # kernel dispatches per call: prefill is two launches (prep, scan)
        f_b = fetch[k] * 1024 / f_scale * LAUNCHES[k]
        w_b = write[k] * 1024 / w_scale * LAUNCHES[k]
        out[k] = {"source_hash": h, "bytes_per_call": round(f_b + w_b), "fetch_bytes": round(f_b),
                  "write_bytes": round(w_b), "dispatches_counted": nf[k]}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def main():
    global TOKENS
    if len(sys.argv) == 4 and sys.argv[1] == "--write-traffic":
        write_traffic(sys.argv[2], sys.argv[3])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prefill-T", type=int, default=4096)
    ap.add_argument("--phases", default=",".join(PHASES), help="comma list (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches only (no graph replay)")
    ap.add_argument("--no-replay", action="store_true", help="skip timing the commit-by-replay path")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the one-GPU path only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the kernels do not shard across GPUs in this build.", file=sys.stderr)
        sys.exit(2)
    phases = [p for p in args.phases.split(",") if p]

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from linear_attention_03_amd import kda
    kda.lib()
    log(f"device {torch.cuda.get_device_name(0)}; building workloads")
    wk = Workloads(args.prefill_T)
    TOKENS = wk.p.T + wk.d.B + wk.v.B * wk.v.N
    calibrate_spin(torch)
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        for ph in phases:
            getattr(wk, ph)()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    total_ms, per, t_enq = time_steps(wk, args.steps, phases)
    torch.cuda.synchronize()
    eager_ms = total_ms / args.steps
    log(f"eager: {eager_ms * 1e3:.1f} us/step (host enqueue {t_enq * 1e3:.1f} ms for all steps)")
    ms_per_step, launch = eager_ms, "eager launches behind a spin kernel"
    if not args.eager:
        graph_ms, _graph = time_graph(wk, args.steps, phases)
        ms_per_step, launch = graph_ms / args.steps, "one HIP graph per step, replayed back to back"
        log(f"graph: {ms_per_step * 1e3:.1f} us/step")

    nbytes = wk.phase_bytes()
    tokens = {"prefill": wk.p.T, "decode": wk.d.B, "verify": wk.v.B * wk.v.N, "commit": 0, "copy": 0,
              "verify_nosnap": wk.v.B * wk.v.N, "commit_replay": 0, "conv_update": wk.d.B}
    replay_out = None
    if not args.no_replay and all(ph in phases for ph in ("verify", "commit")):
        # the alternative verify/commit pair, on the same draft: timed after
        # the step, so that its pool updates do not feed the step's inputs
        log("timing the commit-by-replay pair")
        for _ in range(args.warmup):
            for ph in REPLAY_PHASES:
                getattr(wk, ph)()
        _, per_r, _ = time_steps(wk, args.steps, REPLAY_PHASES)
        per.update(per_r)
        pair_ms = None
        if not args.eager:
            pair_ms, _g = time_graph(wk, args.steps, REPLAY_PHASES)
        replay_out = {"phases": REPLAY_PHASES,
                      "pair_us_graph": round(pair_ms / args.steps * 1e3, 2) if pair_ms else None,
                      "snapshot_pair_us": round(float(np.mean(per["verify"]) + np.mean(per["commit"])), 2),
                      "replay_pair_us": round(float(np.mean(per["verify_nosnap"]) + np.mean(per["commit_replay"])), 2),
                      "accepted_requests": int((wk.accepted >= 0).sum().item())}
    extra = []
    if not args.no_replay and "decode" in phases:
        # the conv update that precedes a decode step (not part of the step)
        log("timing the conv update")
        for _ in range(args.warmup):
            wk.conv_update()
        _, per_c, _ = time_steps(wk, args.steps, ["conv_update"])
        per.update(per_c)
        extra.append("conv_update")
    phase_out = {}
    for ph in list(phases) + (REPLAY_PHASES if replay_out else []) + extra:
        us = float(np.mean(per[ph]))
        gbps = nbytes[ph] / (us * 1e-6) / 1e9
        phase_out[ph] = {"us": round(us, 2), "us_median": round(float(np.median(per[ph])), 2),
                         "tokens_per_s": round(tokens[ph] / (us * 1e-6), 1) if tokens[ph] else None,
                         "algorithmic_MB": round(nbytes[ph] / 1e6, 2), "GBps": round(gbps, 1),
                         "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    if "prefill" in phase_out:
        fl = wk.prefill_flops()
        us = phase_out["prefill"]["us"]
        phase_out["prefill"]["TFLOPs"] = round(fl / (us * 1e-6) / 1e12, 2)
        phase_out["prefill"]["mfma_frac"] = round(fl / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 5)
    # the dominant kernel: the single-launch call with the largest time (the
    # prefill call is two launches, reported in its phase entry)
    single = [ph for ph in phases if LAUNCHES[ph] == 1 and ph != "copy"] or phases
    dom = max(single, key=lambda ph: phase_out[ph]["us"])
    achieved = phase_out[dom]["GBps"]
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tj = json.load(open(TRAFFIC_FILE))
        ent = tj.get(dom)
        if ent and ent.get("source_hash") == source_hash():
            traffic = ent.get("bytes_per_call")
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": KERNEL_NAMES[dom], "phase": dom, "algorithmic_bytes_per_call": nbytes[dom],
                "us_per_call": phase_out[dom]["us"]}

    out = {
        "metric": METRIC,
        "value": round(TOKENS / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"KDA step: prefill 1x{wk.p.T} + decode 48x1 + verify 48x6 chain (conv4) + commit",
                   "heads": 16, "head_dim": 128, "inputs": "bf16", "state": "fp32",
                   "prefill_products": "fp16 / bf16 MFMA operands, fp32 accumulation",
                   "decode_verify_math": "fp32",
                   "chunk_size": wk.p.chunk_size, "tokens_per_step": TOKENS,
                   "phases_timed": phases, "launch": launch},
        "eager_ms_per_step": round(eager_ms, 4),
        "phases": phase_out,
        "roofline": roofline,
    }
    if replay_out:
        out["commit_by_replay"] = replay_out
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (cpu_baseline)")
        out["cpu_baseline"] = cpu_baseline(wk)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
