"""Phases on disjoint requests may run concurrently: prefill on one stream
and the other phases on a second, all on ONE shared state pool (disjoint
slots), captured as one HIP graph with a fork and a join.  Two layouts:
decode -> verify -> commit enqueued before the prefill, and the step graph
of the benchmark (the prefill first, then verify -> decode -> commit on the
second branch).  Every replay (with the pool and conv state reset by eager
copies in between) must equal the one-stream run bit for bit, pool and
outputs."""

import numpy as np
import pytest

from linear_attention_03_amd import workloads as wl

import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


@pytest.mark.parametrize("layout", ["decode_verify_commit_first", "prefill_first_verify_decode_commit"])
def test_prefill_and_other_phases_on_two_streams(layout):
    import torch
    from linear_attention_03_amd import kda
    H, K, V, slots = 4, 128, 128, 40
    perm = np.random.default_rng(2000).permutation(slots).astype(np.int32)
    cp = wl.prefill_case(seed=2001, B=1, T=1024, H=H, K=K, V=V, dtype="bf16", slots=slots)
    cp.indices = perm[:1].copy()
    cd = wl.decode_case(seed=2002, B=16, H=H, K=K, V=V, slots=slots)
    cd.indices = perm[1:17].copy()
    cv = wl.verify_case(seed=2003, B=16, N=6, H=H, K=K, V=V, tree=True, slots=slots)
    cv.indices = perm[17:33].copy()
    pool0 = gu.dev(cp.pool)                                  # the one shared pool
    pdev, ddev, vdev = gu.PrefillDev(cp), gu.DecodeDev(cd), gu.VerifyDev(cv)
    pdev.pool = ddev.pool = vdev.pool = pool0.clone()
    cs0 = vdev.cs.clone()
    acc = gu.dev(np.array([5, -1, 0, 3] * 4, np.int32), "i32")
    po = torch.empty(1, cp.T, H, V, dtype=torch.bfloat16, device="cuda")
    do = torch.empty(cd.B, H, V, dtype=torch.bfloat16, device="cuda")
    vo = torch.empty(cv.B * cv.N, H, V, dtype=torch.bfloat16, device="cuda")
    args = kda._prefill_args(pdev.q, pdev.k, pdev.v, pdev.g, pdev.beta, po, scale=cp.scale,
                             initial_state=pdev.pool, initial_state_indices=pdev.idx,
                             use_qk_l2norm_in_kernel=True, cu_seqlens=None, A_log=pdev.A_log,
                             dt_bias=pdev.dt_bias, lower_bound=cp.lower_bound, beta_is_raw=True,
                             chunk_size=64, intermediate_states=None)
    ws = torch.empty(kda.prefill_workspace_size(args), dtype=torch.uint8, device="cuda")

    def prefill():
        pdev.run(o=po, workspace=ws)

    def commit():
        kda.commit(acc, N=cv.N, snapshots=vdev.snaps, initial_state=vdev.pool, initial_state_indices=vdev.idx,
                   conv_state=vdev.cs, mixed_qkv=vdev.mixed, parents=vdev.parents)

    def chain():
        if layout == "decode_verify_commit_first":
            ddev.run(o=do)
            vdev.run(o=vo)
            commit()
        else:
            vdev.run(o=vo)
            ddev.run(o=do)
            commit()

    def reset():
        pdev.pool.copy_(pool0)
        vdev.cs.copy_(cs0)
        for t in (po, do, vo):
            t.zero_()

    gu.say("concurrent phases: one-stream reference")
    reset()
    prefill()
    chain()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (pdev.pool, vdev.cs, po, do, vo)]

    side, other = torch.cuda.Stream(), torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            other.wait_stream(side)
            if layout == "decode_verify_commit_first":
                with torch.cuda.stream(other):
                    chain()
                prefill()
            else:
                prefill()
                with torch.cuda.stream(other):
                    chain()
            side.wait_stream(other)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        gu.say(f"concurrent phases ({layout}): two-branch graph replay {rep}")
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (pdev.pool, vdev.cs, po, do, vo)
        for name, a, b in zip(("pool", "conv state", "prefill o", "decode o", "verify o"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the one-stream run"
