"""Pins of the fp64 oracle against things other than itself: closed forms,
a hand-worked exact example, invariants of the delta rule, brute force with
dense transition matrices, the chunked form, textbook convolution and the
pages' contract (errors, padded rows).  CPU only."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import kda as ok
from oracle import chunked as oc
from linear_attention_03_amd import workloads as wl

RTOL_EXACT = 1e-12


def _rand_prefill(rng, B, T, H, K, V, slots=4, lengths=None):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = rng.standard_normal((B, T, H, K))
    beta = rng.standard_normal((B, T, H))
    A_log = rng.uniform(0, np.log(16), H)
    dt = 0.1 * rng.standard_normal(H * K)
    pool = 0.3 * rng.standard_normal((slots, H, V, K))
    if lengths is None:
        idx = rng.permutation(slots)[:B]
        cu = None
    else:
        idx = rng.permutation(slots)[:len(lengths)]
        cu = np.concatenate([[0], np.cumsum(lengths)])
    return dict(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt,
                lower_bound=-5.0, beta_is_raw=True, use_qk_l2norm_in_kernel=True,
                initial_state=pool, initial_state_indices=idx, cu_seqlens=cu,
                scale=K ** -0.5)


# ---------------------------------------------------------------- gate, beta, norm

def test_gate_closed_forms():
    lb = -5.0
    HV, K = 2, 3
    A_log = np.array([0.0, np.log(2.0)])
    dt = np.zeros(HV * K)
    # raw + dt_bias = 0 -> sigmoid(0) = 1/2 for any A_log
    g = ok.activate_gate(np.zeros((HV, K)), A_log, dt, lb)
    np.testing.assert_allclose(g, lb / 2, rtol=0, atol=1e-15)
    # head 0: exp(0) * ln3 -> sigmoid = 3/4 ; head 1: exp(ln2) * ln3/2 = ln3 -> 3/4
    raw = np.array([[np.log(3.0)] * K, [np.log(3.0) / 2] * K])
    np.testing.assert_allclose(ok.activate_gate(raw, A_log, dt, lb), 0.75 * lb, rtol=1e-14)
    # dt_bias is [HV*K], head-major: channel (1, 2) gets ln3 / 2 -> 3/4 there, 1/2 elsewhere
    dt2 = np.zeros(HV * K)
    dt2[1 * K + 2] = np.log(3.0) / 2
    g2 = ok.activate_gate(np.zeros((HV, K)), A_log, dt2, lb)
    expect = np.full((HV, K), lb / 2)
    expect[1, 2] = 0.75 * lb
    np.testing.assert_allclose(g2, expect, rtol=1e-14)
    # saturation: bounded in (lb, 0)
    assert np.allclose(ok.activate_gate(np.full((HV, K), 1e4), A_log, dt, lb), lb)
    assert np.all(ok.activate_gate(np.full((HV, K), -1e4), A_log, dt, lb) == 0.0)
    # no A_log: the gate is used as given
    raw = np.random.default_rng(0).standard_normal((HV, K))
    assert np.array_equal(ok.activate_gate(raw, None, None, None), raw)


def test_unbounded_gate_closed_forms():
    """A_log without lower_bound: g = -exp(A_log) * log(1 + e^(raw + dt))."""
    import math
    HV, K = 2, 3
    A_log = np.array([0.0, np.log(2.0)])
    dt = np.zeros(HV * K)
    ea = np.array([[1.0], [2.0]])
    # raw + dt = 0 -> softplus = ln 2
    np.testing.assert_allclose(ok.activate_gate(np.zeros((HV, K)), A_log, dt, None),
                               -ea * math.log(2.0) * np.ones((HV, K)), rtol=1e-15)
    # raw = ln(e - 1) -> softplus = 1 exactly
    raw = np.full((HV, K), math.log(math.e - 1.0))
    np.testing.assert_allclose(ok.activate_gate(raw, A_log, dt, None), -ea * np.ones((HV, K)), rtol=1e-14)
    # dt_bias shifts the argument per channel: channel (0, 1) at ln 3 -> ln 4
    dt2 = np.zeros(HV * K)
    dt2[1] = math.log(3.0)
    g = ok.activate_gate(np.zeros((HV, K)), A_log, dt2, None)
    assert abs(g[0, 1] + math.log(4.0)) < 1e-15 and abs(g[0, 0] + math.log(2.0)) < 1e-15
    # no floor: large arguments give -exp(A_log) * x; large negative ones vanish
    np.testing.assert_allclose(ok.activate_gate(np.full((HV, K), 1e4), A_log, dt, None), -ea * 1e4 * np.ones((HV, K)), rtol=1e-14)
    tiny = ok.activate_gate(np.full((HV, K), -50.0), A_log, dt, None)
    np.testing.assert_allclose(tiny, -ea * math.exp(-50.0) * np.ones((HV, K)), rtol=1e-12)


def test_grouped_heads_share_qk():
    """H q/k heads, HV = 2H value heads: value heads 2j and 2j+1 read q/k
    head j.  Two value heads of one group given the same v, gate, beta and
    state give the same output bit for bit; the same inputs in value heads
    of different groups do not (their q/k differ)."""
    rng = np.random.default_rng(21)
    B, H, HV, K, V = 2, 2, 4, 8, 4
    q = rng.standard_normal((B, H, K))
    k = rng.standard_normal((B, H, K))
    v = np.repeat(rng.standard_normal((B, 1, V)), HV, axis=1)
    a = np.tile(rng.standard_normal((B, 1, K)), (1, HV, 1)).reshape(B, HV * K)
    b = np.repeat(rng.standard_normal((B, 1)), HV, axis=1)
    pool = np.repeat(0.3 * rng.standard_normal((3, 1, V, K)), HV, axis=1)
    A_log = np.zeros(HV)
    dt = np.zeros(HV * K)
    o, p = ok.decode(q, k, v, a, b, scale=K ** -0.5, initial_state=pool, initial_state_indices=[2, 0],
                     A_log=A_log, dt_bias=dt, lower_bound=-5.0)
    assert np.array_equal(o[:, 0], o[:, 1]) and np.array_equal(o[:, 2], o[:, 3])
    assert np.array_equal(p[:, 0], p[:, 1]) and np.array_equal(p[:, 2], p[:, 3])
    assert np.abs(o[:, 0] - o[:, 2]).max() > 1e-3
    # the same holds through prefill (value heads 2j and 2j+1 share q/k head j)
    T = 5
    qp = rng.standard_normal((1, T, H, K))
    kp = rng.standard_normal((1, T, H, K))
    vp = np.repeat(rng.standard_normal((1, T, 1, V)), HV, axis=2)
    gp = np.repeat(-np.abs(rng.standard_normal((1, T, 1, K))), HV, axis=2)
    bp = np.repeat(rng.uniform(0.1, 0.9, (1, T, 1)), HV, axis=2)
    op, pp, _ = ok.prefill(qp, kp, vp, gp, bp, scale=K ** -0.5, initial_state=pool, initial_state_indices=[1])
    assert np.array_equal(op[:, :, 0], op[:, :, 1]) and np.array_equal(op[:, :, 2], op[:, :, 3])
    assert np.abs(op[:, :, 1] - op[:, :, 2]).max() > 1e-3
    with pytest.raises(ValueError, match="multiple"):
        ok.decode(q, k, v[:, :3], a.reshape(B, HV, K)[:, :3].reshape(B, 3 * K), b[:, :3], scale=1.0,
                  initial_state=pool[:, :3], initial_state_indices=[2, 0])


def test_beta_and_l2norm_closed_forms():
    np.testing.assert_allclose(ok.activate_beta(np.array([0.0, np.log(3.0)]), True), [0.5, 0.75], rtol=1e-15)
    x = np.array([0.3, -2.0])
    assert np.array_equal(ok.activate_beta(x, False), x)
    y = ok.l2_normalize(np.array([[3.0, 4.0]]))
    np.testing.assert_allclose(y, [[0.6, 0.8]], rtol=1e-7)
    z = ok.l2_normalize(np.zeros((1, 4)))
    assert np.all(z == 0.0)


# ---------------------------------------------------------------- exact hand-worked example

def test_hand_worked_two_tokens():
    """K = V = 2, S0 = I.  Token 1: exp(g) = (1/2, 1/4), beta = 1/2, k = e0,
    v = (3, 5), q = e1.  Decay: S = diag(1/2, 1/4); S^T k = (1/2, 0);
    error (5/2, 5); S1 = [[7/4, 5/2], [0, 1/4]]; o1 = S1^T q = (0, 1/4).
    Token 2: g = 0, beta = 1, k = e1, v = (2, -1), q = (1, 1).
    S^T k = (0, 1/4); error (2, -5/4); S2 = [[7/4, 5/2], [2, -1]];
    o2 = (15/4, 3/2).  The pool stores S2^T."""
    F = Fraction
    q = np.array([[[[0.0, 1.0]], [[1.0, 1.0]]]])
    k = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]])
    v = np.array([[[[3.0, 5.0]], [[2.0, -1.0]]]])
    g = np.array([[[[np.log(0.5), np.log(0.25)]], [[0.0, 0.0]]]])
    beta = np.array([[[0.5], [1.0]]])
    pool = np.eye(2)[None, None].copy()      # S0^T = I
    o, new_pool, _ = ok.prefill(q, k, v, g, beta, scale=1.0, initial_state=pool,
                                initial_state_indices=[0])
    o_exp = np.array([[F(0), F(1, 4)], [F(15, 4), F(3, 2)]], dtype=object).astype(float)
    S2 = np.array([[F(7, 4), F(5, 2)], [F(2), F(-1)]], dtype=object).astype(float)
    np.testing.assert_allclose(o[0, :, 0], o_exp, rtol=0, atol=1e-14)
    np.testing.assert_allclose(new_pool[0, 0], S2.T, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- brute force, dense transitions

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_dense_transitions(seed):
    """S_t = (I - beta k k^T) Diag(exp g) S_{t-1} + beta k v^T as explicit
    K x K matrices multiplied out in extended precision."""
    rng = np.random.default_rng(seed)
    T, H, K, V = 7, 2, 3, 4
    c = _rand_prefill(rng, 1, T, H, K, V, slots=2)
    o, pool, _ = ok.prefill(**c)
    ld = np.longdouble
    qn = ok.l2_normalize(c["q"][0]).astype(ld)
    kn = ok.l2_normalize(c["k"][0]).astype(ld)
    gg = ok.activate_gate(c["g"][0], c["A_log"], c["dt_bias"], -5.0).astype(ld)
    bb = ok.sigmoid(c["beta"][0]).astype(ld)
    s = int(c["initial_state_indices"][0])
    for h in range(H):
        S = c["initial_state"][s, h].T.astype(ld)
        for t in range(T):
            kk = kn[t, h][:, None]
            M = (np.eye(K, dtype=ld) - bb[t, h] * (kk @ kk.T)) @ np.diag(np.exp(gg[t, h]))
            S = M @ S + bb[t, h] * kk @ c["v"][0, t, h][None, :].astype(ld)
            ot = c["scale"] * (S.T @ qn[t, h])
            np.testing.assert_allclose(o[0, t, h], ot.astype(np.float64), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(pool[s, h], S.T.astype(np.float64), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants

def test_beta_one_overwrites_key_slot():
    """beta = 1: after each token S_t^T k_t = v_t exactly, for any decay and
    initial state (pins decay-before-correction and the transposition)."""
    rng = np.random.default_rng(3)
    H, K, V = 3, 8, 5
    S = rng.standard_normal((H, K, V))
    for _ in range(6):
        q = ok.l2_normalize(rng.standard_normal((H, K)))
        kr = rng.standard_normal((H, K))
        k = kr / np.linalg.norm(kr, axis=-1, keepdims=True)     # exactly unit keys
        v = rng.standard_normal((H, V))
        g = -rng.uniform(0, 5, (H, K))
        S, _ = ok.kda_step(S, q, k, v, g, np.ones(H), 1.0)
        np.testing.assert_allclose(np.einsum("hkv,hk->hv", S, k), v, rtol=1e-12, atol=1e-12)


def test_beta_zero_is_pure_decay():
    """beta = 0: S_T = Diag(exp(sum g)) S_0 and o_t = scale (Diag(exp G_t) S_0)^T q_t."""
    rng = np.random.default_rng(4)
    T, H, K, V = 9, 2, 4, 3
    c = _rand_prefill(rng, 1, T, H, K, V, slots=3)
    c["beta"] = np.zeros_like(c["beta"])
    c["beta_is_raw"] = False
    o, pool, _ = ok.prefill(**c)
    g = ok.activate_gate(c["g"][0], c["A_log"], c["dt_bias"], -5.0)
    G = np.cumsum(g, axis=0)
    qn = ok.l2_normalize(c["q"][0])
    s = int(c["initial_state_indices"][0])
    S0 = np.transpose(c["initial_state"][s], (0, 2, 1))
    for t in range(T):
        St = np.exp(G[t])[:, :, None] * S0
        np.testing.assert_allclose(o[0, t], c["scale"] * np.einsum("hkv,hk->hv", St, qn[t]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(pool[s], np.transpose(np.exp(G[-1])[:, :, None] * S0, (0, 2, 1)), rtol=1e-12, atol=1e-14)


def test_orthonormal_keys_store_and_recall():
    """g = 0, beta = 1, orthonormal keys, S_0 = 0: S = sum_i k_i v_i^T and a
    query equal to k_j reads back scale * v_j."""
    rng = np.random.default_rng(5)
    K, V, T = 8, 6, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys = Qm[:, :T].T                          # T orthonormal rows
    vals = rng.standard_normal((T, V))
    q = np.zeros((1, T + 1, 1, K))
    k = np.zeros((1, T + 1, 1, K))
    v = np.zeros((1, T + 1, 1, V))
    k[0, :T, 0] = keys
    v[0, :T, 0] = vals
    q[0, T, 0] = keys[2]                        # read with key 2 at the end (k=0, beta=0 there)
    g = np.zeros((1, T + 1, 1, K))
    beta = np.ones((1, T + 1, 1))
    beta[0, T] = 0.0
    pool = np.zeros((1, 1, V, K))
    o, new_pool, _ = ok.prefill(q, k, v, g, beta, scale=0.5, initial_state=pool,
                                initial_state_indices=[0])
    np.testing.assert_allclose(new_pool[0, 0].T, keys.T @ vals, atol=1e-12)
    np.testing.assert_allclose(o[0, T, 0], 0.5 * vals[2], atol=1e-12)


def test_linearity_in_values_and_state():
    rng = np.random.default_rng(6)
    c = _rand_prefill(rng, 1, 11, 2, 4, 4, slots=2)
    o1, p1, _ = ok.prefill(**c)
    c2 = dict(c)
    c2["v"] = 2.5 * c["v"]
    c2["initial_state"] = 2.5 * c["initial_state"]
    o2, p2, _ = ok.prefill(**c2)
    np.testing.assert_allclose(o2, 2.5 * o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p2, 2.5 * p1, rtol=1e-12, atol=1e-13)


def test_ranges_of_preprocessed_inputs():
    c = wl.config0_tiny()
    g = ok.activate_gate(c.g, c.A_log, c.dt_bias, c.lower_bound)
    # (lower_bound, 0) mathematically; the sigmoid saturates to 0 or 1 in floating point
    assert np.all(g <= 0) and np.all(g >= c.lower_bound)
    assert np.any(g < -4.9) and np.any(g > -0.1)
    n = np.linalg.norm(ok.l2_normalize(c.q), axis=-1)
    np.testing.assert_allclose(n, 1.0, rtol=1e-6)


# ---------------------------------------------------------------- chunked form, varlen, T=1

@pytest.mark.parametrize("C", [16, 64])
@pytest.mark.parametrize("lengths", [[1], [15], [16], [17], [64], [65], [130], [3, 64, 1, 40, 100]])
def test_chunked_equals_recurrent(C, lengths):
    rng = np.random.default_rng(len(lengths) * 100 + sum(lengths) + C)
    T = sum(lengths)
    c = _rand_prefill(rng, 1, T, 2, 8, 8, slots=8, lengths=lengths if len(lengths) > 1 else None)
    o_r, p_r, i_r = ok.prefill(**c, output_intermediate_states=True, chunk_size=C)
    o_c, p_c, i_c = oc.prefill_chunked(**c, chunk_size=C, output_intermediate_states=True)
    scale_o = np.abs(o_r).max()
    np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-10 * scale_o)
    np.testing.assert_allclose(p_c, p_r, rtol=0, atol=1e-10 * np.abs(p_r).max())
    assert i_r.shape == i_c.shape
    np.testing.assert_allclose(i_c, i_r, rtol=0, atol=1e-10 * np.abs(p_r).max())


@pytest.mark.parametrize("C", [16, 64])
def test_chunked_equals_recurrent_grouped_heads(C):
    """Two q/k heads shared by four value heads (value head h reads q/k head
    h // 2): the chunked form must expand the groups as the recurrence does;
    indexing v or the state by the q/k head would fail here."""
    rng = np.random.default_rng(31 + C)
    lengths = [5, 70, 33]
    c = _rand_prefill(rng, 1, sum(lengths), 4, 8, 8, slots=6, lengths=lengths)
    c["q"], c["k"] = c["q"][:, :, :2].copy(), c["k"][:, :, :2].copy()
    o_r, p_r, i_r = ok.prefill(**c, output_intermediate_states=True, chunk_size=C)
    o_c, p_c, i_c = oc.prefill_chunked(**c, chunk_size=C, output_intermediate_states=True)
    assert o_c.shape == o_r.shape == (1, sum(lengths), 4, 8)
    np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-10 * np.abs(o_r).max())
    np.testing.assert_allclose(p_c, p_r, rtol=0, atol=1e-10 * np.abs(p_r).max())
    np.testing.assert_allclose(i_c, i_r, rtol=0, atol=1e-10 * np.abs(p_r).max())
    # value heads 0 and 1 share q/k but not v: their outputs differ
    assert not np.allclose(o_r[..., 0, :], o_r[..., 1, :])


def test_chunked_strong_decay_no_overflow():
    """lower_bound -5 over 64 tokens drives cumulative log-decay to -320;
    the chunked form must stay finite and equal to the recurrence."""
    rng = np.random.default_rng(8)
    c = _rand_prefill(rng, 1, 128, 1, 8, 8, slots=2)
    c["g"] = np.full_like(c["g"], 50.0)      # sigmoid -> 1, g -> -5 everywhere
    o_r, p_r, _ = ok.prefill(**c)
    o_c, p_c, _ = oc.prefill_chunked(**c, chunk_size=64)
    assert np.all(np.isfinite(o_c))
    np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-10 * np.abs(o_r).max())


def test_varlen_equals_independent_sequences_and_heads():
    rng = np.random.default_rng(9)
    lengths = [5, 1, 33, 17]
    c = _rand_prefill(rng, 1, sum(lengths), 3, 4, 6, slots=6, lengths=lengths)
    o, pool, _ = ok.prefill(**c)
    cu = c["cu_seqlens"]
    for n in range(len(lengths)):
        for h in range(3):
            sl = slice(cu[n], cu[n + 1])
            s = int(c["initial_state_indices"][n])
            cn = dict(q=c["q"][:, sl, h:h + 1], k=c["k"][:, sl, h:h + 1], v=c["v"][:, sl, h:h + 1],
                      g=c["g"][:, sl, h:h + 1], beta=c["beta"][:, sl, h:h + 1],
                      A_log=c["A_log"][h:h + 1], dt_bias=c["dt_bias"][h * 4:(h + 1) * 4],
                      lower_bound=-5.0, beta_is_raw=True, use_qk_l2norm_in_kernel=True,
                      initial_state=c["initial_state"][s:s + 1, h:h + 1], initial_state_indices=[0],
                      scale=c["scale"])
            on, pn, _ = ok.prefill(**cn)
            np.testing.assert_allclose(o[:, sl, h:h + 1], on, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(pool[s, h], pn[0, 0], rtol=1e-13, atol=1e-15)


def test_single_token_prefill_equals_decode_step():
    dc = wl.decode_case(seed=11, B=3, H=2, K=8, V=4, slots=5, dtype="f32")
    o_d, p_d = ok.decode(dc.q(), dc.k(), dc.v(), dc.a, dc.b, scale=dc.scale,
                         initial_state=dc.pool, initial_state_indices=dc.indices,
                         A_log=dc.A_log, dt_bias=dc.dt_bias, lower_bound=dc.lower_bound)
    for r in range(dc.B):
        o_p, p_p, _ = ok.prefill(dc.q()[r:r + 1, None], dc.k()[r:r + 1, None], dc.v()[r:r + 1, None],
                                 dc.a[r:r + 1, None].reshape(1, 1, dc.HV, dc.K), dc.b[r:r + 1, None],
                                 scale=dc.scale, initial_state=dc.pool,
                                 initial_state_indices=dc.indices[r:r + 1],
                                 A_log=dc.A_log, dt_bias=dc.dt_bias, lower_bound=dc.lower_bound,
                                 beta_is_raw=True, use_qk_l2norm_in_kernel=True)
        np.testing.assert_array_equal(o_p[0, 0], o_d[r])
        s = dc.indices[r]
        np.testing.assert_array_equal(p_p[s], p_d[s])


def test_padded_gate_rows_are_ignored():
    """g / beta rows beyond T (graph-bucket padding) must never be read: 1e4
    and NaN pads give bitwise identical results."""
    base = wl.prefill_case(seed=12, B=1, T=40, H=2, K=8, V=8, dtype="f32",
                           chunk_size=16, lengths=[7, 33], pad_rows=24, pad_value=1e4, slots=4)
    kw = dict(scale=base.scale, initial_state=base.pool, initial_state_indices=base.indices,
              cu_seqlens=base.cu_seqlens, A_log=base.A_log, dt_bias=base.dt_bias,
              lower_bound=base.lower_bound, beta_is_raw=True, use_qk_l2norm_in_kernel=True)
    o1, p1, _ = ok.prefill(base.q, base.k, base.v, base.g, base.beta, **kw)
    g_nan = base.g.copy(); g_nan[:, 40:] = np.nan
    b_nan = base.beta.copy(); b_nan[:, 40:] = np.nan
    o2, p2, _ = ok.prefill(base.q, base.k, base.v, g_nan, b_nan, **kw)
    o3, p3, _ = ok.prefill(base.q, base.k, base.v, base.g[:, :40], base.beta[:, :40], **kw)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2)
    assert np.array_equal(o1, o3) and np.array_equal(p1, p3)


# ---------------------------------------------------------------- contract errors

def test_prefill_contract_errors():
    c = _rand_prefill(np.random.default_rng(13), 1, 8, 1, 4, 4)
    with pytest.raises(ValueError, match="state pool and one slot index"):
        ok.prefill(**{**c, "initial_state": None})
    with pytest.raises(ValueError, match="state pool and one slot index"):
        ok.prefill(**{**c, "initial_state_indices": None})
    with pytest.raises(ValueError, match="g has 7 token rows"):
        ok.prefill(**{**c, "g": c["g"][:, :7]})
    with pytest.raises(ValueError, match="beta has 5 token rows"):
        ok.prefill(**{**c, "beta": c["beta"][:, :5]})
    # longer g / beta are padding: accepted, and rows past T are not read
    pad = dict(c, g=np.concatenate([c["g"], np.full((1, 3, 1, 4), np.nan)], axis=1),
               beta=np.concatenate([c["beta"], np.full((1, 3, 1), np.nan)], axis=1))
    o_pad, p_pad, _ = ok.prefill(**pad)
    o_ref, p_ref, _ = ok.prefill(**c)
    assert np.array_equal(o_pad, o_ref) and np.array_equal(p_pad, p_ref)


def test_decode_contract_errors_and_padding():
    dc = wl.decode_case(seed=14, B=3, H=2, K=8, V=4, slots=5, dtype="f32", pad_requests=(1,))
    kw = dict(scale=dc.scale, initial_state=dc.pool, initial_state_indices=dc.indices,
              A_log=dc.A_log, dt_bias=dc.dt_bias, lower_bound=dc.lower_bound)
    o, p = ok.decode(dc.q(), dc.k(), dc.v(), dc.a, dc.b, **kw)
    assert np.all(o[1] == 0)
    untouched = [s for s in range(5) if s not in dc.indices]
    assert np.array_equal(p[untouched], dc.pool[untouched])
    with pytest.raises(ValueError, match=r"HV\*K"):
        ok.decode(dc.q(), dc.k(), dc.v(), dc.a[:, :-1], dc.b, **kw)
    # key dim 6 (q and k cut to 6 channels, gate and pool to match): refused
    q6, k6 = dc.q()[..., :6], dc.k()[..., :6]
    a6 = dc.a.reshape(3, 2, 8)[..., :6].reshape(3, 12)
    kw6 = {**kw, "initial_state": np.zeros((5, 2, 4, 6)), "dt_bias": dc.dt_bias.reshape(2, 8)[:, :6].reshape(-1)}
    with pytest.raises(ValueError, match="K=6 is not a power of two"):
        ok.decode(q6, k6, dc.v(), a6, dc.b, **kw6)


# ---------------------------------------------------------------- conv, verify, commit

def test_conv_chain_matches_textbook_correlation():
    """Chain drafts: node i's conv output equals np.correlate of each
    channel's sequence (conv_state then tokens 0..i) with its weights."""
    rng = np.random.default_rng(15)
    N, C, W = 6, 5, 4
    x = rng.standard_normal((N, C))
    cs = rng.standard_normal((C, W - 1))
    w = rng.standard_normal((C, W))
    y = ok.causal_conv_draft(x, cs, w, None, np.arange(N) - 1, None)
    for c in range(C):
        seq = np.concatenate([cs[c], x[:, c]])
        ref = np.correlate(seq, w[c], mode="valid")      # ref[n] = sum_j w[j] seq[n + j]
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-14, atol=1e-14)
    ys = ok.causal_conv_draft(x, cs, w, np.ones(C), np.arange(N) - 1, "silu")
    z = y + 1.0
    np.testing.assert_allclose(ys, z / (1 + np.exp(-z)), rtol=1e-14)


def test_conv_update_steps_match_textbook_correlation():
    """T one-token updates from a conv state: step t's output is
    np.correlate of each channel's sequence (conv state, x_0 .. x_t) with its
    weights at the last window, plus the bias; the state keeps the last W-1
    inputs.  A negative index gives zero output and leaves every slot alone."""
    rng = np.random.default_rng(16)
    B, C, W, T, slots = 3, 7, 4, 6, 5
    cs0 = rng.standard_normal((slots, C, W - 1))
    w = rng.standard_normal((C, W))
    bias = rng.standard_normal(C)
    idx = np.array([4, -1, 1])
    xs = rng.standard_normal((T, B, C))
    cs = cs0
    for t in range(T):
        y, cs = ok.conv_update(xs[t], conv_weight=w, conv_state=cs, conv_state_indices=idx,
                               conv_bias=bias, activation=None)
        assert np.all(y[1] == 0)
        for r in (0, 2):
            for c in range(C):
                seq = np.concatenate([cs0[idx[r], c], xs[:t + 1, r, c]])
                ref = np.correlate(seq, w[c], mode="valid")[-1] + bias[c]
                assert abs(y[r, c] - ref) < 1e-13
                np.testing.assert_array_equal(cs[idx[r], c], seq[-(W - 1):])
    for s in (0, 2, 3):
        np.testing.assert_array_equal(cs[s], cs0[s])
    ys, _ = ok.conv_update(xs[0], conv_weight=w, conv_state=cs0, conv_state_indices=idx, conv_bias=bias)
    z, _ = ok.conv_update(xs[0], conv_weight=w, conv_state=cs0, conv_state_indices=idx, conv_bias=bias,
                          activation=None)
    np.testing.assert_allclose(ys, z / (1 + np.exp(-z)), rtol=1e-14)


def _verify_kw(vc):
    return dict(N=vc.N, H=vc.H, HV=vc.HV, K=vc.K, V=vc.V, scale=vc.scale,
                conv_weight=vc.conv_weight, conv_state=vc.conv_state,
                initial_state=vc.pool, initial_state_indices=vc.indices,
                parents=vc.parents, A_log=vc.A_log, dt_bias=vc.dt_bias,
                lower_bound=vc.lower_bound)


def test_verify_chain_snapshots_equal_prefix_states():
    """Chain snapshot i equals the prefill state after tokens 0..i of the
    conv'd inputs; outputs equal the prefill outputs."""
    vc = wl.verify_case(seed=16, B=2, N=5, H=2, K=8, V=4, tree=False, slots=6, dtype="f32")
    o, snaps = ok.verify(vc.mixed_qkv, vc.a, vc.b, **_verify_kw(vc))
    HK = vc.H * vc.K
    for r in range(vc.B):
        rows = slice(r * vc.N, (r + 1) * vc.N)
        y = ok.causal_conv_draft(vc.mixed_qkv[rows], vc.conv_state[vc.indices[r]], vc.conv_weight,
                                 None, np.arange(vc.N) - 1, "silu")
        q = y[:, :HK].reshape(1, vc.N, vc.H, vc.K)
        k = y[:, HK:2 * HK].reshape(1, vc.N, vc.H, vc.K)
        v = y[:, 2 * HK:].reshape(1, vc.N, vc.HV, vc.V)
        g = vc.a[rows].reshape(1, vc.N, vc.HV, vc.K)
        for i in range(vc.N):
            o_p, p_p, _ = ok.prefill(q[:, :i + 1], k[:, :i + 1], v[:, :i + 1], g[:, :i + 1],
                                     vc.b[rows][None, :i + 1], scale=vc.scale,
                                     initial_state=vc.pool, initial_state_indices=vc.indices[r:r + 1],
                                     A_log=vc.A_log, dt_bias=vc.dt_bias, lower_bound=vc.lower_bound,
                                     beta_is_raw=True, use_qk_l2norm_in_kernel=True)
            np.testing.assert_allclose(snaps[(r, i)], p_p[vc.indices[r]], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(o[r * vc.N + i], o_p[0, i], rtol=1e-12, atol=1e-14)


def test_verify_tree_node_equals_chain_along_its_path():
    vc = wl.verify_case(seed=17, B=3, N=6, H=2, K=8, V=4, tree=True, slots=6,
                        dtype="f32", multi_root=True)
    o, snaps = ok.verify(vc.mixed_qkv, vc.a, vc.b, **_verify_kw(vc))
    for r in range(vc.B):
        for i in range(vc.N):
            path = ok.path_to_root(vc.parents[r], i)
            L = len(path)
            rows = [r * vc.N + p for p in path]
            sub = wl.VerifyCase(mixed_qkv=vc.mixed_qkv[rows], a=vc.a[rows], b=vc.b[rows],
                                conv_weight=vc.conv_weight, conv_state=vc.conv_state,
                                A_log=vc.A_log, dt_bias=vc.dt_bias, lower_bound=vc.lower_bound,
                                scale=vc.scale, pool=vc.pool, indices=vc.indices[r:r + 1],
                                parents=None, N=L, H=vc.H, HV=vc.HV, K=vc.K, V=vc.V)
            o_c, s_c = ok.verify(sub.mixed_qkv, sub.a, sub.b, **_verify_kw(sub))
            np.testing.assert_array_equal(snaps[(r, i)], s_c[(0, L - 1)])
            np.testing.assert_array_equal(o[r * vc.N + i], o_c[L - 1])


def test_verify_padded_request_and_readonly_pool():
    vc = wl.verify_case(seed=18, B=3, N=4, H=1, K=4, V=4, tree=True, slots=5,
                        dtype="f32", pad_requests=(2,))
    pool0 = vc.pool.copy()
    cs0 = vc.conv_state.copy()
    o, snaps = ok.verify(vc.mixed_qkv, vc.a, vc.b, **_verify_kw(vc))
    assert np.all(o[2 * vc.N:] == 0)
    assert not any(k[0] == 2 for k in snaps)
    assert np.array_equal(vc.pool, pool0) and np.array_equal(vc.conv_state, cs0)


def test_commit_restores_snapshot_and_continues_the_conv():
    """After committing node a, (i) the pool slot equals snapshot a, and
    (ii) the next draft's conv with the rolled conv state equals the conv
    over the whole history (conv_state, accepted path, next token)."""
    vc = wl.verify_case(seed=19, B=3, N=5, H=1, K=4, V=4, tree=True, slots=5, dtype="f32")
    o, snaps = ok.verify(vc.mixed_qkv, vc.a, vc.b, **_verify_kw(vc))
    snap_arr = np.full((vc.B, vc.N, vc.HV, vc.V, vc.K), np.nan)
    for (s, i), S in snaps.items():
        snap_arr[s, i] = S
    accepted = np.array([3, -1, 0])
    pool, cs = ok.commit(accepted, N=vc.N, snapshots=snap_arr, initial_state=vc.pool,
                         initial_state_indices=vc.indices, conv_state=vc.conv_state,
                         mixed_qkv=vc.mixed_qkv, parents=vc.parents)
    np.testing.assert_array_equal(pool[vc.indices[0]], snap_arr[0, 3])
    np.testing.assert_array_equal(pool[vc.indices[1]], vc.pool[vc.indices[1]])
    np.testing.assert_array_equal(pool[vc.indices[2]], snap_arr[2, 0])
    np.testing.assert_array_equal(cs[vc.indices[1]], vc.conv_state[vc.indices[1]])
    rng = np.random.default_rng(20)
    for r in (0, 2):
        path = ok.path_to_root(vc.parents[r], accepted[r])
        x_next = rng.standard_normal((1, vc.conv_dim))
        y_roll = ok.causal_conv_draft(x_next, cs[vc.indices[r]], vc.conv_weight, None, [-1], None)
        full = np.concatenate([vc.conv_state[vc.indices[r]].T, vc.mixed_qkv[[r * vc.N + p for p in path]], x_next])
        ref = np.array([np.correlate(full[:, c], vc.conv_weight[c], mode="valid")[-1] for c in range(vc.conv_dim)])
        np.testing.assert_allclose(y_roll[0], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("tree", [False, True])
def test_commit_replay_equals_snapshot_commit(tree):
    """Replaying the accepted path from the pool state reaches bit for bit
    the state verify snapshotted for the accepted node (same steps in the
    same order), for chains and trees, every accepted index and none; the
    conv state rolls identically."""
    vc = wl.verify_case(seed=21 + tree, B=4, N=6, H=2, K=8, V=8, tree=tree, slots=6, dtype="f32")
    kw = _verify_kw(vc)
    o, snaps = ok.verify(vc.mixed_qkv, vc.a, vc.b, **kw)
    snap_arr = np.full((vc.B, vc.N, vc.HV, vc.V, vc.K), np.nan)
    for (s, i), S in snaps.items():
        snap_arr[s, i] = S
    for accepted in (np.array([5, -1, 0, 2]), np.array([0, 3, 4, -1]), np.array([-1, -1, 5, 1])):
        pool_s, cs_s = ok.commit(accepted, N=vc.N, snapshots=snap_arr, initial_state=vc.pool,
                                 initial_state_indices=vc.indices, conv_state=vc.conv_state,
                                 mixed_qkv=vc.mixed_qkv, parents=kw.get("parents"))
        pool_r, cs_r = ok.commit_replay(accepted, vc.mixed_qkv, vc.a, vc.b, **kw)
        np.testing.assert_array_equal(pool_r, pool_s)
        np.testing.assert_array_equal(cs_r, cs_s)


def test_decode_conv_steps_equal_prefill_of_convolved_sequence():
    """T successive fused conv + decode steps ([42905] Summary: conv1d update
    and recurrence in one launch) of two requests with grouped heads equal,
    per request, the textbook causal correlation (np.correlate over the
    conv state followed by the tokens, then SiLU) of the whole sequence fed
    to one prefill from the same pool state; the conv state ends as the
    last W-1 inputs.  A padded request changes nothing."""
    rng = np.random.default_rng(41)
    T, B, H, HV, K, V, Wd = 5, 3, 2, 4, 8, 4, 4
    C = 2 * H * K + HV * V
    x = rng.standard_normal((T, B, C))
    a = rng.standard_normal((T, B, HV * K))
    bb = rng.standard_normal((T, B, HV))
    w = rng.uniform(-0.5, 0.5, (C, Wd))
    bias = 0.1 * rng.standard_normal(C)
    cs0 = rng.standard_normal((6, C, Wd - 1))
    pool0 = 0.3 * rng.standard_normal((6, HV, V, K))
    sidx = np.array([4, -1, 1])
    cidx = np.array([2, 3, 5])
    A_log = rng.uniform(0, np.log(16), HV)
    dt = 0.1 * rng.standard_normal(HV * K)
    kw = dict(H=H, HV=HV, K=K, V=V, scale=K ** -0.5, conv_weight=w, conv_bias=bias, A_log=A_log,
              dt_bias=dt, lower_bound=-5.0)
    pool, cs = pool0.copy(), cs0.copy()
    cs[3] = np.nan                      # the padded request's conv slot: never read or written
    outs = []
    for t in range(T):
        o, pool, cs = ok.decode_conv(x[t], a[t], bb[t], conv_state=cs, initial_state=pool,
                                     initial_state_indices=sidx, conv_state_indices=cidx, **kw)
        outs.append(o)
    assert np.all(np.isnan(cs[3])) and all(np.all(o[1] == 0) for o in outs)
    for r in (0, 2):
        hist = np.concatenate([cs0[cidx[r]], x[:, r].T], axis=1)          # [C, W-1+T], oldest first
        y = np.stack([np.correlate(hist[c], w[c], mode="valid") for c in range(C)], axis=1) + bias
        y = y * ok.sigmoid(y)                                             # [T, C]
        HK = H * K
        q = y[:, :HK].reshape(1, T, H, K)
        k = y[:, HK:2 * HK].reshape(1, T, H, K)
        v = y[:, 2 * HK:].reshape(1, T, HV, V)
        o_ref, p_ref, _ = ok.prefill(q, k, v, a[:, r].reshape(1, T, HV, K), bb[:, r].reshape(1, T, HV),
                                     scale=K ** -0.5, initial_state=pool0, initial_state_indices=[sidx[r]],
                                     use_qk_l2norm_in_kernel=True, A_log=A_log, dt_bias=dt, lower_bound=-5.0,
                                     beta_is_raw=True)
        for t in range(T):
            np.testing.assert_allclose(outs[t][r], o_ref[0, t], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(pool[sidx[r]], p_ref[sidx[r]], rtol=1e-11, atol=1e-12)
        np.testing.assert_array_equal(cs[cidx[r]], x[-(Wd - 1):, r].T)
    untouched = [s for s in range(6) if s not in (1, 4)]
    assert np.array_equal(pool[untouched], pool0[untouched])
