"""GPU parity of the chunked prefill against the fp64 oracle, through the C
ABI: the tiny float32 case (chunk 16), a length x heads x layout x dtype
sweep (chunk 64, head dim 128), the full 1 x 4096 / 1 x 8192 and packed 8192
workloads on every head, padded gate / beta rows, the T = 1 case before
longer calls, intermediate states on both paths, determinism, graph replay,
a call on a side stream, bf16 views off 16-byte alignment (reported as
and run on the general path), and the general path's fp32-tile preps at
chunk 16 and 64 for every K and V, with and without chunks left to the
exact prep."""

import numpy as np
import pytest

from linear_attention_03_amd import workloads as wl

import gpu_util as gu

pytestmark = pytest.mark.gpu

SWEEP_LENGTHS = [1, 2, 3, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 500, 1023, 2048]


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def test_prefill_tiny_fp32_chunk16():
    c = wl.config0_tiny()
    gu.say(c.name)
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=c.name)
    assert np.all(np.isnan(d.pool[0].cpu().numpy())), "NaN sentinel slot was touched"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H", [1, 4, 16])
def test_prefill_sweep_varlen(dtype, H):
    """All sweep lengths packed into one call (cu_seqlens)."""
    T = sum(SWEEP_LENGTHS)
    c = wl.prefill_case(seed=300 + H, B=1, T=T, H=H, K=128, V=128, dtype=dtype, chunk_size=64,
                        lengths=SWEEP_LENGTHS, slots=40)
    name = f"varlen sweep T={T} H={H} {dtype}"
    gu.say(name)
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", SWEEP_LENGTHS)
def test_prefill_sweep_fixed(dtype, T):
    """Fixed layout, batch 2, every sweep length; heads 1 / 4 / 16 rotate over
    the lengths so every head count meets short, chunk-edge and long cases."""
    H = [1, 4, 16][SWEEP_LENGTHS.index(T) % 3]
    c = wl.prefill_case(seed=400 + T, B=2, T=T, H=H, K=128, V=128, dtype=dtype, chunk_size=64, slots=5)
    name = f"fixed B=2 T={T} H={H} {dtype}"
    gu.say(name)
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)


@pytest.mark.parametrize("K,V,C", [(32, 64, 16), (64, 32, 64), (64, 128, 16), (128, 32, 64), (128, 128, 64)])
def test_prefill_other_head_dims(K, V, C):
    c = wl.prefill_case(seed=450 + K + V + C, B=1, T=150, H=3, K=K, V=V, dtype="bf16", chunk_size=C,
                        lengths=[0, 37, 1, 112], slots=6)
    name = f"K={K} V={V} C={C} varlen with an empty sequence"
    gu.say(name)
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)


@pytest.mark.parametrize("T", [4096, 8192])
def test_prefill_full_fixed(T):
    c = wl.config2_prefill(T)
    gu.say(c.name)
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=c.name)
    assert np.all(np.isfinite(gu.host(o)))


def test_prefill_full_varlen_padded_rows_ignored():
    """Packed 8192 tokens with g / beta padded to 12288 rows: 1e4 pads match
    the oracle, and NaN pads give bitwise identical output and state."""
    import torch
    c = wl.config3_varlen(pad_value=1e4)
    gu.say(c.name)
    d = gu.PrefillDev(c)
    o = d.run()
    torch.cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=c.name)
    g_nan, b_nan = c.g.copy(), c.beta.copy()
    g_nan[:, c.T:] = np.nan
    b_nan[:, c.T:] = np.nan
    gu.say("varlen with NaN pads")
    d2 = gu.PrefillDev(c, g=g_nan, beta=b_nan)
    o2 = d2.run()
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(d.pool.view(torch.int32), d2.pool.view(torch.int32))


@pytest.mark.parametrize("layout", ["fixed", "varlen"])
def test_t1_prefill_then_longer_calls(layout):
    """T = 1 first, then 4096 tokens, then a packed batch; each checked against
    the oracle (the pages' T = 1 trace-specialisation hazard does not exist
    for ahead-of-time kernels, but the behaviour is pinned anyway)."""
    cases = [
        wl.prefill_case(seed=61, B=1, T=1, H=16, K=128, V=128, dtype="bf16", slots=8,
                        lengths=None if layout == "fixed" else [1]),
        wl.prefill_case(seed=62, B=1, T=4096, H=16, K=128, V=128, dtype="bf16", slots=8,
                        lengths=None if layout == "fixed" else [4096]),
        wl.prefill_case(seed=63, B=1, T=700, H=16, K=128, V=128, dtype="bf16", slots=8,
                        lengths=[1, 64, 635]),
    ]
    for c in cases:
        name = f"{layout} T={c.T} N={c.N}"
        gu.say(name)
        d = gu.PrefillDev(c)
        o = d.run()
        gu.torch().cuda.synchronize()
        gu.check_prefill(c, o, d.pool, name=name)


@pytest.mark.parametrize("C", [16, 64])
def test_prefill_intermediate_states(C):
    import torch
    from linear_attention_03_amd import kda
    c = wl.prefill_case(seed=70 + C, B=1, T=300, H=2, K=64, V=64, dtype="f32", chunk_size=C,
                        lengths=[5, 130, 0, 165], slots=6)
    n_rows = kda.prefill_max_chunks(c.T, C, num_seqs=c.N)
    inter = torch.full((n_rows, c.HV, c.V, c.K), float("nan"), device="cuda")
    gu.say(f"intermediate states C={C}")
    d = gu.PrefillDev(c)
    o = d.run(intermediate=inter)
    torch.cuda.synchronize()
    o_ref, pool_ref, inter_ref = gu.prefill_oracle(c, intermediate=True)
    gu.check_prefill(c, o, d.pool, name="intermediate", o_ref=o_ref, pool_ref=pool_ref)
    got = inter.cpu().numpy()
    assert inter_ref.shape[0] == sum((n + C - 1) // C for n in c.lengths())
    for i in range(inter_ref.shape[0]):
        gu.check_state(got[i].astype(np.float64), inter_ref[i], "f32", f"chunk {i}")
    assert np.all(np.isnan(got[inter_ref.shape[0]:]))


def test_prefill_intermediate_states_mfma_path():
    """Intermediate states of the matrix-core path (bf16, chunk 64,
    K = V = 128, 16 heads) element by element against the oracle, packed
    lengths 1, 64, 65 and longer; rows past the last chunk stay untouched."""
    import torch
    from linear_attention_03_amd import kda
    lengths = [1, 64, 65, 130, 7, 300]
    c = wl.prefill_case(seed=75, B=1, T=sum(lengths), H=16, K=128, V=128, dtype="bf16", chunk_size=64,
                        lengths=lengths, slots=9)
    n_rows = kda.prefill_max_chunks(c.T, 64, num_seqs=c.N)
    inter = torch.full((n_rows, c.HV, c.V, c.K), float("nan"), device="cuda")
    gu.say("intermediate states, bf16 chunk 64, 16 heads")
    d = gu.PrefillDev(c)
    o = d.run(intermediate=inter)
    torch.cuda.synchronize()
    o_ref, pool_ref, inter_ref = gu.prefill_oracle(c, intermediate=True)
    gu.check_prefill(c, o, d.pool, name="intermediate mfma", o_ref=o_ref, pool_ref=pool_ref)
    got = inter.cpu().numpy()
    n = sum((x + 63) // 64 for x in lengths)
    assert inter_ref.shape[0] == n
    worst = 0.0
    for i in range(n):
        worst = max(worst, gu.check_state(got[i].astype(np.float64), inter_ref[i], "bf16", f"chunk {i}"))
    assert np.all(np.isnan(got[n:]))
    gu.say(f"intermediate states: worst relative Frobenius {worst:.2e} over {n} chunks")


def test_prefill_scan_claim_matches_shared_launch():
    """A scan grid of at most one block per CU claims its compute units (a
    kernel build whose waves hold the whole register file); a larger grid
    runs the plain build.  Both builds do the same arithmetic, so one
    sequence prefilled alone (claiming launch) and as row 0 of a batch large
    enough for the plain launch must agree bit for bit, outputs and state."""
    import dataclasses
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks_per_seq = 16 * (128 // 16)                 # heads x 16-column slices
    nB = cus // blocks_per_seq + 1                    # past one block per CU
    cb = wl.prefill_case(seed=1700, B=nB, T=320, H=16, K=128, V=128, dtype="bf16", slots=nB + 3)
    c1 = dataclasses.replace(cb, q=cb.q[:1], k=cb.k[:1], v=cb.v[:1], g=cb.g[:1], beta=cb.beta[:1],
                             indices=cb.indices[:1].copy())
    assert 1 * blocks_per_seq <= cus < nB * blocks_per_seq
    gu.say(f"scan claim: 1 sequence ({blocks_per_seq} blocks) against {nB} ({nB * blocks_per_seq} blocks), {cus} CUs")
    d1, db = gu.PrefillDev(c1), gu.PrefillDev(cb)
    o1, ob = d1.run(), db.run()
    torch.cuda.synchronize()
    assert torch.equal(o1[0], ob[0]), "outputs of the claiming and the shared scan launch differ"
    s = int(cb.indices[0])
    assert torch.equal(d1.pool[s], db.pool[s]), "final states of the claiming and the shared scan launch differ"


def test_prefill_on_side_stream_without_workspace():
    """prefill(stream=s) with no o and no workspace: both are allocated for
    stream s, so memory freed when the call returns is not handed to work on
    the current stream while s still uses it.  The current stream meanwhile
    allocates and fills buffers of the workspace's size; every run must equal
    a run on the current stream bit for bit."""
    import torch
    from linear_attention_03_amd import kda
    c = wl.prefill_case(seed=81, B=1, T=2048, H=16, K=128, V=128, dtype="bf16", slots=4)
    d = gu.PrefillDev(c)
    pool0 = d.pool.clone()
    o_tmp = torch.empty(1, c.T, c.HV, c.V, dtype=torch.bfloat16, device="cuda")
    ws_bytes = kda.prefill_workspace_size(kda._prefill_args(
        d.q, d.k, d.v, d.g, d.beta, o_tmp, scale=c.scale, initial_state=d.pool, initial_state_indices=d.idx,
        use_qk_l2norm_in_kernel=True, cu_seqlens=None, A_log=d.A_log, dt_bias=d.dt_bias,
        lower_bound=c.lower_bound, beta_is_raw=True, chunk_size=64, intermediate_states=None))
    gu.say("prefill on the current stream (reference)")
    o_ref = d.run()
    torch.cuda.synchronize()
    pool_ref = d.pool.clone()
    s = torch.cuda.Stream()
    outs = []
    for rep in range(3):
        gu.say(f"prefill on a side stream, run {rep}")
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            d.pool.copy_(pool0)
        o = d.run(stream=s)
        for _ in range(4):
            junk = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            junk.fill_(0xFF)
            del junk
        with torch.cuda.stream(s):
            outs.append((o.clone(), d.pool.clone()))
    torch.cuda.synchronize()
    for o, pool in outs:
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(pool.view(torch.int32), pool_ref.view(torch.int32))


def test_prefill_deterministic_and_graph_replay():
    import torch
    from linear_attention_03_amd import kda
    c = wl.prefill_case(seed=80, B=1, T=1000, H=16, K=128, V=128, dtype="bf16", lengths=[200, 800], slots=4)
    d = gu.PrefillDev(c)
    pool0 = d.pool.clone()
    o = torch.empty(1, c.T, c.HV, c.V, dtype=torch.bfloat16, device="cuda")
    args = kda._prefill_args(d.q, d.k, d.v, d.g, d.beta, o, scale=c.scale, initial_state=d.pool,
                             initial_state_indices=d.idx, use_qk_l2norm_in_kernel=True, cu_seqlens=d.cu,
                             A_log=d.A_log, dt_bias=d.dt_bias, lower_bound=c.lower_bound, beta_is_raw=True,
                             chunk_size=64, intermediate_states=None)
    ws = torch.empty(kda.prefill_workspace_size(args), dtype=torch.uint8, device="cuda")
    gu.say("prefill eager x2")
    d.run(o=o, workspace=ws)
    torch.cuda.synchronize()
    o1, p1 = o.clone(), d.pool.clone()
    d.pool.copy_(pool0)
    d.run(o=o, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(d.pool, p1), "prefill is not deterministic"
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            d.run(o=o, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        gu.say(f"prefill graph replay {rep}")
        d.pool.copy_(pool0)
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o1) and torch.equal(d.pool, p1)


@pytest.mark.parametrize("gval", [0.0, -1e-3, "mixed"])
def test_prefill_slow_decay_state_tolerance(gval):
    """Log-decay at or near zero on every channel (gate given as the
    log-decay itself): every token stays in the state, rounding errors are
    not forgotten and the state grows to tens of times its initial size, the
    hardest case for the state tolerance.  "mixed" alternates chunks of
    log-decay -1e-3 and -1.5, so one call takes both operand precisions of
    the Gram products (narrow and wide in-block decay spans)."""
    import torch
    from linear_attention_03_amd import kda
    from oracle import kda as ok
    c = wl.prefill_case(seed=96, B=1, T=4096, H=16, K=128, V=128, dtype="bf16", slots=4)
    if gval == "mixed":
        per_token = np.where((np.arange(c.g.shape[1]) // 64) % 2 == 0, -1e-3, -1.5).astype(np.float32)
        g = wl.round_bf16(np.broadcast_to(per_token[None, :, None, None], c.g.shape).copy())
    else:
        g = wl.round_bf16(np.full(c.g.shape, gval, np.float32))
    heads = list(range(c.HV))
    gu.say(f"prefill 1x4096 bf16, log-decay {gval} on every channel")
    q, k, v, gd, b = (gu.dev(x, "bf16") for x in (c.q, c.k, c.v, g, c.beta))
    pool = gu.dev(c.pool)
    idx = gu.dev(c.indices, "i32")
    o = kda.prefill(q, k, v, gd, b, scale=c.scale, initial_state=pool, initial_state_indices=idx,
                    use_qk_l2norm_in_kernel=True, beta_is_raw=True, chunk_size=64)
    torch.cuda.synchronize()
    o_ref, p_ref, _ = ok.prefill(c.q[:, :, heads], c.k[:, :, heads], c.v[:, :, heads], g[:, :, heads],
                                 c.beta[:, :, heads], scale=c.scale, initial_state=c.pool[:, heads],
                                 initial_state_indices=c.indices, use_qk_l2norm_in_kernel=True,
                                 beta_is_raw=True)
    s = int(c.indices[0])
    e_o = gu.check_out(gu.host(o)[:, :, heads], o_ref, "bf16", f"log-decay {gval} o")
    e_s = gu.check_state(pool[s][heads].cpu().numpy().astype(np.float64), p_ref[s], "bf16",
                         f"log-decay {gval} state")
    gu.say(f"log-decay {gval}: max|do|/max|o| = {e_o:.2e}, state relative Frobenius = {e_s:.2e}, "
           f"|S| grew {np.linalg.norm(p_ref[s]) / np.linalg.norm(c.pool[s][heads]):.0f}x")


def test_prefill_large_qk_scale_and_wide_decay_spans():
    """q and k of magnitude ~1e5 (the in-kernel L2 norm makes the result
    independent of their scale) with a bounded gate of lower bound -9.5, so
    the in-block decay spans of the Gram factorisation reach ~76: every Gram
    operand must stay finite (they carry the norms, at most e^span each)."""
    import dataclasses
    import torch
    c0 = wl.prefill_case(seed=97, B=1, T=2048, H=16, K=128, V=128, dtype="bf16", slots=4)
    c = dataclasses.replace(c0, q=wl.round_bf16(c0.q * np.float32(1e5)), k=wl.round_bf16(c0.k * np.float32(1e5)),
                            lower_bound=-9.5, name="prefill 1x2048 bf16, |q|,|k| ~ 1e5, lower bound -9.5")
    gu.say(c.name)
    d = gu.PrefillDev(c)
    o = d.run()
    torch.cuda.synchronize()
    assert np.all(np.isfinite(gu.host(o))), "non-finite output"
    gu.check_prefill(c, o, d.pool, name=c.name)


def test_prefill_large_state_and_values():
    """Initial state ~ N(0, 30) and values scaled by 100: the state and the
    corrected values U reach the hundreds to thousands, inside the fp16
    range the matrix-core path states as its precondition; relative errors
    must not depend on that scale."""
    import dataclasses
    import torch
    c0 = wl.prefill_case(seed=98, B=1, T=2048, H=16, K=128, V=128, dtype="bf16", slots=4, pool_std=30.0)
    c = dataclasses.replace(c0, v=wl.round_bf16(c0.v * np.float32(100.0)),
                            name="prefill 1x2048 bf16, state ~ N(0, 30), values x100")
    gu.say(c.name)
    d = gu.PrefillDev(c)
    o = d.run()
    torch.cuda.synchronize()
    assert np.all(np.isfinite(gu.host(o))), "non-finite output"
    gu.check_prefill(c, o, d.pool, name=c.name)


@pytest.mark.parametrize("case", ["values_x1e5_no_decay", "state_3e5"])
def test_prefill_beyond_fp16_range(case):
    """The state and the corrected values U leave the fp16 range (|S| up to
    ~3e5, |U| up to ~4e5): values x 1e5 with log-decay 0 on every channel,
    or an initial state ~ N(0, 3e5) under the bounded gate.  The scan's fp16
    operands are scaled by per-wave powers of two there, so the results stay
    within the tolerances on every head."""
    import dataclasses
    import torch
    c0 = wl.prefill_case(seed=99, B=1, T=2048, H=16, K=128, V=128, dtype="bf16", slots=4)
    if case == "values_x1e5_no_decay":
        c = dataclasses.replace(c0, v=wl.round_bf16(c0.v * np.float32(1e5)), g=np.zeros_like(c0.g), A_log=None,
                                name="prefill 1x2048, values x 1e5, log-decay 0")
    else:
        c = dataclasses.replace(c0, pool=(c0.pool * np.float32(3e5 / 0.02)).astype(np.float32),
                                name="prefill 1x2048, initial state ~ N(0, 3e5)")
    gu.say(c.name)
    q, k, v, g, b = (gu.dev(x, "bf16") for x in (c.q, c.k, c.v, c.g, c.beta))
    pool = gu.dev(c.pool)
    idx = gu.dev(c.indices, "i32")
    kw = dict(A_log=None, dt_bias=None, lower_bound=None) if c.A_log is None else \
        dict(A_log=gu.dev(c.A_log), dt_bias=gu.dev(c.dt_bias), lower_bound=c.lower_bound)
    o = kda_prefill(q, k, v, g, b, c, pool, idx, **kw)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(gu.host(o))), "non-finite output"
    o_ref, p_ref, _ = gu.prefill_oracle(c)
    s = int(c.indices[0])
    assert np.abs(p_ref[s]).max() > 65504 or np.abs(c.pool[s]).max() > 65504
    e_o = gu.check_out(gu.host(o), o_ref, "bf16", f"{c.name} o")
    e_s = gu.check_state(pool[s].cpu().numpy().astype(np.float64), p_ref[s], "bf16", f"{c.name} state")
    gu.say(f"{c.name}: max|S| {np.abs(p_ref[s]).max():.3g}, max|do|/max|o| = {e_o:.2e}, "
           f"state relative Frobenius = {e_s:.2e}")


def kda_prefill(q, k, v, g, b, c, pool, idx, **kw):
    from linear_attention_03_amd import kda
    return kda.prefill(q, k, v, g, b, scale=c.scale, initial_state=pool, initial_state_indices=idx,
                       use_qk_l2norm_in_kernel=True, beta_is_raw=True, chunk_size=64, **kw)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_small_positive_log_decay(dtype):
    """A log-decay given directly (no A_log) with small positive values,
    g ~ U(0, 0.02): the state grows (about e^7 over 700 tokens) instead of
    decaying, the Grams take the exact-exponential branch and the in-chunk
    e^G stay far inside fp16; every head against the oracle."""
    import dataclasses
    import torch
    c0 = wl.prefill_case(seed=120, B=1, T=700, H=16, K=128, V=128, dtype=dtype, slots=4)
    rng = np.random.default_rng(121)
    g = rng.uniform(0.0, 0.02, c0.g.shape).astype(np.float32)
    g = wl.round_bf16(g) if dtype == "bf16" else g
    c = dataclasses.replace(c0, g=g, A_log=None, name=f"prefill 1x700 {dtype}, log-decay ~ U(0, 0.02)")
    gu.say(c.name)
    q, k, v, gd, b = (gu.dev(x, dtype) for x in (c.q, c.k, c.v, c.g, c.beta))
    pool = gu.dev(c.pool)
    idx = gu.dev(c.indices, "i32")
    o = kda_prefill(q, k, v, gd, b, c, pool, idx, A_log=None, dt_bias=None, lower_bound=None)
    torch.cuda.synchronize()
    gu.check_prefill(c, o, pool, name=c.name)


def test_prefill_positive_lower_bound_takes_float32_path():
    """A bounded gate with lower_bound > 0 (positive log-decays up to 0.02)
    on bf16 inputs: routed to the float32 path, results on every head
    within the bf16 tolerances."""
    import dataclasses
    c0 = wl.prefill_case(seed=122, B=1, T=400, H=16, K=128, V=128, dtype="bf16", slots=4)
    c = dataclasses.replace(c0, lower_bound=0.02, name="prefill 1x400 bf16, lower_bound +0.02")
    gu.say(c.name)
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=c.name)


def _offset_view(t, off):
    """A copy of t as a view `off` elements into a wider last dimension, so
    the rows keep their values but not 16-byte alignment."""
    import torch
    shape = list(t.shape)
    buf = torch.zeros(shape[:-1] + [shape[-1] + 8], dtype=t.dtype, device=t.device)
    view = buf[..., off:off + shape[-1]]
    view.copy_(t)
    return view


def test_prefill_misaligned_bf16_view_takes_general_path():
    """bf16 q, k, g and v viewed one element past a 16-byte boundary: the
    path query reports the general float32 path, the call takes it and
    matches the oracle on every head; the aligned tensors report the
    matrix-core path and also match."""
    import torch
    from linear_attention_03_amd import kda
    c = wl.prefill_case(seed=131, B=1, T=300, H=4, HV=8, K=128, V=128, dtype="bf16", slots=4)
    d = gu.PrefillDev(c)
    kw = dict(scale=c.scale, initial_state=d.pool, initial_state_indices=d.idx, use_qk_l2norm_in_kernel=True,
              A_log=d.A_log, dt_bias=d.dt_bias, lower_bound=c.lower_bound, beta_is_raw=True, chunk_size=64)
    assert kda.prefill_path(d.q, d.k, d.v, d.g, d.beta, **kw) == "matrix"
    q, k, g, v = (_offset_view(t, 1) for t in (d.q, d.k, d.g, d.v))
    assert q.data_ptr() % 16 != 0 and torch.equal(q, d.q)
    assert kda.prefill_path(q, k, v, g, d.beta, **kw) == "general"
    name = "prefill 1x300 bf16 H=4 HV=8, rows off 16-byte alignment"
    gu.say(name)
    o_ref, pool_ref, _ = gu.prefill_oracle(c)
    o = kda.prefill(q, k, v, g, d.beta, **kw)
    torch.cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name + " (general path)", o_ref=o_ref, pool_ref=pool_ref)
    d2 = gu.PrefillDev(c)
    o2 = d2.run()
    torch.cuda.synchronize()
    gu.check_prefill(c, o2, d2.pool, name=name + ": aligned copy (matrix path)", o_ref=o_ref, pool_ref=pool_ref)


@pytest.mark.parametrize("K,V,C", [(128, 128, 64), (64, 64, 64), (32, 128, 64), (128, 128, 16), (64, 32, 16)])
def test_prefill_fp32_tiles_mixed_exact_fallback(K, V, C):
    """float32 inputs (the fp32-tile prep) with lower bound -12: some
    chunks' half-block decay spans pass 80 and are flagged to the exact
    prep, the others are not, in one call of packed sequences; every head
    against the oracle at the float32 tolerance."""
    import dataclasses
    import torch
    from linear_attention_03_amd import kda
    lengths = [300, 1, 64, 65, 570]
    c0 = wl.prefill_case(seed=140 + K + V + C, B=1, T=sum(lengths), H=8, K=K, V=V, dtype="f32",
                         lengths=lengths, slots=8, chunk_size=C)
    lb = -12.0 if C == 64 else -40.0
    c = dataclasses.replace(c0, lower_bound=lb, name=f"prefill packed 1000 f32 K={K} V={V} C={C}, lower bound {lb}")
    # the flagged share, from the same gate map as the oracle (spans over half blocks, natural log units)
    raw = c.g[0].astype(np.float64)
    g = c.lower_bound / (1.0 + np.exp(-np.exp(c.A_log)[None, :, None] * (raw + c.dt_bias.reshape(c.HV, c.K)[None])))
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    flagged = total = 0
    for st, n in zip(starts, lengths):
        for c_ in range(0, n, C):
            G = np.cumsum(g[st + c_: st + min(n, c_ + C)], 0)
            G = np.concatenate([G, np.repeat(G[-1:], C - G.shape[0], 0)], 0)
            for h in range(c.HV):
                total += 1
                span = max(max((G[16 * s, h] - G[16 * s + 7, h]).max(), (G[16 * s + 7, h] - G[16 * s + 15, h]).max())
                           for s in range(C // 16))
                flagged += span > 80.0
    gu.say(f"{c.name}: {flagged} of {total} (chunk, head) items past a span of 80")
    assert 0 < flagged < total
    d = gu.PrefillDev(c)
    assert kda.prefill_path(d.q, d.k, d.v, d.g, d.beta, scale=c.scale, initial_state=d.pool,
                            initial_state_indices=d.idx, use_qk_l2norm_in_kernel=True, cu_seqlens=d.cu,
                            A_log=d.A_log, dt_bias=d.dt_bias, lower_bound=c.lower_bound, beta_is_raw=True,
                            chunk_size=C) == "general"
    o = d.run()
    torch.cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=c.name)


@pytest.mark.parametrize("C", [16, 64])
def test_prefill_fp32_tiles_bounded_gate_at_the_no_flag_limit(C):
    """A bounded gate with lower_bound -8.75 (the strongest for which the
    general path launches no exact prep) and raw gates pushed up so most
    log-decays sit near the bound: the widest spans the fp32-tile prep then
    meets (up to 8 rows from a reference row) approach 70 and must still be
    handled by it; every head against the oracle at the float32
    tolerance."""
    import dataclasses
    import torch
    lengths = [300, 1, 64, 65, 570]
    c0 = wl.prefill_case(seed=150 + C, B=1, T=sum(lengths), H=8, K=64, V=64, dtype="f32",
                         lengths=lengths, slots=8, chunk_size=C)
    g = (np.abs(c0.g) + 4.0).astype(np.float32)          # sigmoid near 1: log-decay near the bound
    c = dataclasses.replace(c0, g=g, lower_bound=-8.75, name=f"prefill packed 1000 f32 C={C}, lower bound -8.75")
    gmap = c.lower_bound / (1.0 + np.exp(-np.exp(c.A_log)[None, :, None] * (g[0].astype(np.float64)
                                                                               + c.dt_bias.reshape(c.HV, c.K)[None])))
    gu.say(f"{c.name}: mean log-decay {gmap.mean():.2f}, widest 8-row span {-8 * gmap.min():.1f}")
    assert -8 * gmap.min() > 60.0
    d = gu.PrefillDev(c)
    o = d.run()
    torch.cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=c.name)


def test_prefill_fp32_tiles_intermediate_states():
    """Intermediate states of the general path on fp32 tiles (float32, C = 64,
    K = V = 128: fp32-tile prep and scan) element by element against the
    oracle, packed lengths 1, 64, 65 and longer."""
    import torch
    from linear_attention_03_amd import kda
    lengths = [1, 64, 65, 200, 7]
    c = wl.prefill_case(seed=141, B=1, T=sum(lengths), H=4, K=128, V=128, dtype="f32", chunk_size=64,
                        lengths=lengths, slots=7)
    n_rows = kda.prefill_max_chunks(c.T, 64, num_seqs=c.N)
    inter = torch.full((n_rows, c.HV, c.V, c.K), float("nan"), device="cuda")
    gu.say("intermediate states, f32 chunk 64, K = V = 128")
    d = gu.PrefillDev(c)
    o = d.run(intermediate=inter)
    torch.cuda.synchronize()
    o_ref, pool_ref, inter_ref = gu.prefill_oracle(c, intermediate=True)
    gu.check_prefill(c, o, d.pool, name="intermediate f32 tiles", o_ref=o_ref, pool_ref=pool_ref)
    got = inter.cpu().numpy()
    n = sum((x + 63) // 64 for x in lengths)
    assert inter_ref.shape[0] == n
    for i in range(n):
        gu.check_state(got[i].astype(np.float64), inter_ref[i], "f32", f"chunk {i}")
    assert np.all(np.isnan(got[n:]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [32, 64, 128])
@pytest.mark.parametrize("V", [32, 64, 128])
@pytest.mark.parametrize("C", [16, 64])
def test_prefill_fp32_tiles_every_head_dim(dtype, K, V, C):
    """The general path for every K, V and chunk size (fp32-tile prep and
    scan; bf16 at K = V = 128, C = 64 takes the matrix path instead), packed
    lengths 1, 15, 16, 17, 64, 65 and longer with grouped heads, every head
    against the oracle."""
    lengths = [1, 15, 16, 17, 64, 65, 200]
    c = wl.prefill_case(seed=150 + K + 3 * V + C, B=1, T=sum(lengths), H=2, HV=4, K=K, V=V, dtype=dtype,
                        chunk_size=C, lengths=lengths, slots=9)
    name = f"general path C={C} K={K} V={V} {dtype} packed"
    gu.say(name)
    d = gu.PrefillDev(c)
    o = d.run()
    gu.torch().cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)


@pytest.mark.parametrize("K,V,C", [(64, 64, 64), (32, 128, 64), (128, 64, 16)])
def test_prefill_fp32_tiles_misaligned_rows(K, V, C):
    """bf16 rows one element past a 16-byte boundary on the general path:
    the fp32-tile preps' element-load variants, against the oracle."""
    import torch
    from linear_attention_03_amd import kda
    c = wl.prefill_case(seed=160 + K + V + C, B=1, T=300, H=4, K=K, V=V, dtype="bf16", slots=4, chunk_size=C)
    d = gu.PrefillDev(c)
    kw = dict(scale=c.scale, initial_state=d.pool, initial_state_indices=d.idx, use_qk_l2norm_in_kernel=True,
              A_log=d.A_log, dt_bias=d.dt_bias, lower_bound=c.lower_bound, beta_is_raw=True, chunk_size=C)
    q, k, g, v = (_offset_view(t, 1) for t in (d.q, d.k, d.g, d.v))
    assert q.data_ptr() % 16 != 0
    name = f"prefill 1x300 bf16 K={K} V={V} C={C}, rows off 16-byte alignment"
    gu.say(name)
    o = kda.prefill(q, k, v, g, d.beta, **kw)
    torch.cuda.synchronize()
    gu.check_prefill(c, o, d.pool, name=name)
