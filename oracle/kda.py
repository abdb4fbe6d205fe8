"""Token-by-token fp64 oracle of the KDA recurrence.  TEST INFRASTRUCTURE ONLY.

Sources (cited below by the pull-request number in each page's title)
-------
[42857] "[KDA] Support Helion MTP verification and harden prefill, decode"
        (sglang pull request 42857): Motivation, Modifications, KDA
        microbenchmarks table.
[35197] report on sglang pull request 35197, "fix(kernel) Fix Helion
        small-token prefill bug": implementation breakdown (实现拆解) and key
        code snippets (关键源码片段) of the prefill entry and the packed-decode
        input check.
[42905] "[KDA] Default GLM-5-Next spec verify to the CuTe DSL KDA kernel"
        (sglang pull request 42905): Summary, Results (per-layer target verify).

The pages name the method and its three phases ([42857] Motivation: KDA
prefill, decode and EAGLE/MTP verification) and the argument contract
([35197] key code snippets of the prefill entry and the decode input check)
but print no formula.
The recurrence restated here is the reading taken for the method they name:
per (sequence, head), with the state S of shape [K, V],

    S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
    o_t = scale * S_t^T q_t

evaluated as: decay the rows of S by exp(g_t); subtract the delta-rule
prediction error; read out.  All arithmetic is float64.

State layout: the pool stores S transposed, pool[slot, h, v, k] = S[k, v]
(in [35197]'s decode snippet the pool's last three dims are value heads,
value dim and key dim, in that order).

Readings of points the pages leave open (each is also listed in the design
notes of the repository):
  * gate map  g = lower_bound * sigmoid(exp(A_log[h]) * (raw + dt_bias[h, :]))
    when A_log and lower_bound are given; the pages only name A_log, dt_bias
    and lower_bound ([35197] prefill entry signature) and a bounded gate of -5 ([42857]
    microbenchmarks).  A_log is per head [HV]; dt_bias is [HV*K], matching
    the raw gate width HV*K that [35197]'s decode input check enforces.  Without A_log,
    g is used as given.
  * unbounded gate (A_log without lower_bound; [42857] Motivation names the
    bounded-gate case, which implies the other): the usual KDA gate
    g = -exp(A_log[h]) * softplus(raw + dt_bias[h, :]), softplus(x) =
    log(1 + e^x).  Like the bounded map it is negative and decreasing in
    exp(A_log); it differs in having no floor.
  * grouped heads (H q/k heads, HV value heads, HV a multiple of H; [35197]'s
    decode input check and prefill signature name H and HV separately): value
    head hv reads q/k head hv // (HV / H), so consecutive value heads share
    one q/k head.
  * beta = sigmoid(raw) iff beta_is_raw ([42857] Modifications), else as given.
  * q/k L2 norm over the head dim: x * (sum x^2 + 1e-6)^(-1/2) ([35197] names
    use_qk_l2norm_in_kernel; the epsilon is not on the pages).
  * scale multiplies the read-out after the norm; it is always explicit here.
  * a negative slot index in decode / verify marks a padded request: its
    output is zero and no state is read or written.
  * causal conv (verify): width W (4 in the workloads), weights w[c, j],
    y = sum_j w[c, j] * x_{t-W+1+j} (+ bias), so w[c, W-1] multiplies the
    current token; history runs back along the draft's ancestor path and then
    into conv_state[c, :] (oldest first); activation SiLU or none; the conv
    covers the q || k || v channels of mixed_qkv and the L2 norm follows it
    ([42905] Summary: conv1d + recurrence fused in one launch).
  * tree encoding: parents[b, i] in {-1} U [0, i); -1 attaches to the pool
    state; parents=None means a chain (parent i-1).
  * commit: accepted[b] is the last accepted node (-1: none); the pool slot
    takes that node's snapshot and the conv state rolls along that node's
    path ([42857] review thread: verify, commit a partially accepted prefix,
    verify again).
"""

from __future__ import annotations

import numpy as np

L2_EPS = 1e-6


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def sigmoid(x):
    """Logistic function in float64 (large negative inputs give 0)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def l2_normalize(x, eps=L2_EPS):
    """x * (sum(x^2) + eps)^(-1/2) over the last axis ([35197]: in-kernel q/k L2
    norm, ``use_qk_l2norm_in_kernel``)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def softplus(x):
    """log(1 + e^x) in float64, without overflow for large x."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def activate_gate(raw, A_log, dt_bias, lower_bound):
    """Raw gate [..., HV, K] -> log-decay.

    Bounded (lower_bound given): lower_bound * sigmoid(exp(A_log) (raw + dt)),
    in (lower_bound, 0).  Unbounded (lower_bound None):
    -exp(A_log) * softplus(raw + dt), in (-inf, 0).  Readings of the pages'
    A_log / dt_bias / lower_bound arguments ([35197] prefill entry signature; [42857]
    'bounded gate -5', and its bounded-gate decode).  A_log is None: the
    gate is already a log-decay and is returned unchanged.
    """
    raw = np.asarray(raw, dtype=np.float64)
    if A_log is None:
        return raw
    HV, K = raw.shape[-2:]
    a = np.exp(np.asarray(A_log, dtype=np.float64)).reshape(HV, 1)
    dt = np.zeros((HV, K)) if dt_bias is None else np.asarray(dt_bias, np.float64).reshape(HV, K)
    if lower_bound is None:
        return -a * softplus(raw + dt)
    return float(lower_bound) * sigmoid(a * (raw + dt))


def expand_qk_heads(x, HV):
    """q or k [..., H, K] -> [..., HV, K]: value head hv reads q/k head
    hv // (HV / H) (grouped heads; H == HV is the identity)."""
    H = x.shape[-2]
    if HV % H != 0:
        raise ValueError(f"HV ({HV}) must be a multiple of H ({H})")
    return np.repeat(x, HV // H, axis=-2)


def activate_beta(raw, beta_is_raw):
    """beta = sigmoid(raw) iff beta_is_raw ([42857] Modifications: forward
    beta_is_raw)."""
    raw = np.asarray(raw, dtype=np.float64)
    return sigmoid(raw) if beta_is_raw else raw


def kda_step(S, q, k, v, g, beta, scale):
    """One token of the recurrence for a batch of heads.

    S [H, K, V] (math orientation), q/k [H, K], v [H, V], g [H, K], beta [H].
    Returns the new state and o [H, V].
    """
    S = np.exp(g)[:, :, None] * S                        # Diag(exp g) S
    pred = np.einsum("hkv,hk->hv", S, k)                 # S^T k
    S = S + beta[:, None, None] * k[:, :, None] * (v - pred)[:, None, :]
    o = scale * np.einsum("hkv,hk->hv", S, q)            # scale S^T q
    return S, o


def _pool_to_S(pool_slot):
    # pool[slot] is [HV, V, K] = S^T per head
    return np.transpose(np.asarray(pool_slot, np.float64), (0, 2, 1)).copy()


def _S_to_pool(S):
    return np.transpose(S, (0, 2, 1))


def _sequences(B, T, cu_seqlens):
    """List of (batch row, first token, end token) per sequence ([35197]:
    cu_seqlens packs sequences along q.shape[1])."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    if B != 1:
        raise ValueError("cu_seqlens requires batch size 1")
    if cu[0] != 0 or cu[-1] != T or any(cu[i] > cu[i + 1] for i in range(len(cu) - 1)):
        raise ValueError("cu_seqlens must rise from 0 to T")
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def _token_rows(x, T, name):
    """The first T token rows of a [B, rows, ...] tensor.  Rows past T are
    padding the entry never reads ([35197], prefill entry: gate and beta may
    be longer than q but not shorter)."""
    x = np.asarray(x)
    if x.shape[1] < T:
        raise ValueError(f"{name} has {x.shape[1]} token rows but q has {T}")
    return _f64(x[:, :T])


def prefill(q, k, v, g, beta, *, scale, initial_state, initial_state_indices,
            use_qk_l2norm_in_kernel=False, cu_seqlens=None, A_log=None,
            dt_bias=None, lower_bound=None, beta_is_raw=False,
            output_intermediate_states=False, chunk_size=64):
    """Prefill over fixed-length or packed (cu_seqlens) sequences.

    q, k [B, T, H, K]; v [B, T, HV, V]; g [B, T_g, HV, K] with T_g >= T;
    beta [B, T_b, HV] with T_b >= T; initial_state [slots, HV, V, K];
    initial_state_indices [N].

    Entry contract of [35197] (key code snippets, prefill entry): the call
    works on an indexed state pool only, and g / beta rows at or past T are
    padding that is never read.  Returns (o [B, T, HV, V], new pool,
    intermediates).  The final state of sequence n is written to
    pool[indices[n]].  With output_intermediate_states the state entering
    every chunk of chunk_size tokens is returned, in global chunk order
    ([n_chunks, HV, V, K]).
    """
    if initial_state is None or initial_state_indices is None:
        raise ValueError("prefill: a state pool and one slot index per sequence are required")
    q, k, v = _f64(q), _f64(k), _f64(v)
    T = q.shape[1]
    g, beta = _token_rows(g, T, "g"), _token_rows(beta, T, "beta")
    seqs = _sequences(q.shape[0], T, cu_seqlens)
    slots = [int(x) for x in np.asarray(initial_state_indices)]
    if len(slots) != len(seqs):
        raise ValueError(f"prefill: {len(seqs)} sequences but {len(slots)} slot indices")
    HV, V, K = v.shape[2], v.shape[3], q.shape[3]

    if use_qk_l2norm_in_kernel:
        q, k = l2_normalize(q), l2_normalize(k)
    q, k = expand_qk_heads(q, HV), expand_qk_heads(k, HV)
    g = activate_gate(g, A_log, dt_bias, lower_bound)
    beta = activate_beta(beta, beta_is_raw)

    pool = np.array(initial_state, dtype=np.float64, copy=True)
    o = np.zeros((q.shape[0], T, HV, V))
    inter = []
    for (b, t0, t1), slot in zip(seqs, slots):
        S = _pool_to_S(pool[slot])
        for t in range(t0, t1):
            if output_intermediate_states and (t - t0) % chunk_size == 0:
                inter.append(_S_to_pool(S).copy())
            S, o[b, t] = kda_step(S, q[b, t], k[b, t], v[b, t], g[b, t], beta[b, t], scale)
        pool[slot] = _S_to_pool(S)
    inter = np.stack(inter) if inter else np.zeros((0, HV, V, K))
    return o, pool, (inter if output_intermediate_states else None)


def decode(q, k, v, a, b, *, scale, initial_state, initial_state_indices,
           A_log=None, dt_bias=None, lower_bound=None, beta_is_raw=True,
           use_qk_l2norm_in_kernel=True):
    """Packed one-token decode with an in-place pool update.

    q, k [B, H, K]; v [B, HV, V]; a [B, HV*K] raw gate; b [B, HV] raw beta.
    The input check of [35197] (key code snippets, packed decode) refuses key
    or value head dims that are not powers of two and a raw gate whose width
    is not HV*K; both are restated here.  A request whose slot index is
    negative is padding: o = 0, no state touched.  Returns (o [B, HV, V],
    new pool).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, K = q.shape[0], q.shape[2]
    HV, V = v.shape[1], v.shape[2]
    for name, n in (("K", K), ("V", V)):
        if n < 1 or bin(n).count("1") != 1:
            raise ValueError(f"decode: head dim {name}={n} is not a power of two")
    a = np.asarray(a)
    if a.shape[1] != HV * K:
        raise ValueError(f"decode: raw gate a has {a.shape[1]} columns, HV*K = {HV * K} expected")
    pool = np.array(initial_state, dtype=np.float64, copy=True)
    if pool.shape[-3:] != (HV, V, K):
        raise ValueError(f"decode: pool slots are {pool.shape[-3:]}, ({HV}, {V}, {K}) expected")
    if use_qk_l2norm_in_kernel:
        q, k = l2_normalize(q), l2_normalize(k)
    q, k = expand_qk_heads(q, HV), expand_qk_heads(k, HV)
    g = activate_gate(_f64(a).reshape(B, HV, K), A_log, dt_bias, lower_bound)
    beta = activate_beta(b, beta_is_raw)
    o = np.zeros((B, HV, V))
    for r in range(B):
        s = int(initial_state_indices[r])
        if s < 0:
            continue
        S, o[r] = kda_step(_pool_to_S(pool[s]), q[r], k[r], v[r], g[r], beta[r], scale)
        pool[s] = _S_to_pool(S)
    return o, pool


def path_to_root(parents_row, i):
    """Nodes from the root down to node i (inclusive) of one draft."""
    path = []
    while i >= 0:
        path.append(i)
        i = int(parents_row[i])
    return path[::-1]


def check_parents(parents, N):
    parents = np.asarray(parents)
    for row in parents:
        for i in range(N):
            if not (row[i] == -1 or 0 <= row[i] < i):
                raise ValueError("parents[b, i] must be -1 or an earlier node")


def causal_conv_draft(x, conv_state, weight, bias, parents_row, activation):
    """Depthwise causal conv of every draft node of one request.

    x [N, C] pre-conv inputs of the N draft tokens; conv_state [C, W-1]
    (oldest first); weight [C, W]; bias [C] or None.  For node i the input
    sequence is conv_state followed by the tokens on the path root..i; the
    output is the last window, y = sum_j w[:, j] * window[j] (+ bias), then
    SiLU if activation == 'silu'.  Returns [N, C].
    """
    x = _f64(x)
    N, C = x.shape
    W = weight.shape[1]
    hist = _f64(conv_state).T                        # [W-1, C]
    w = _f64(weight)
    y = np.zeros((N, C))
    for i in range(N):
        seq = np.concatenate([hist, x[path_to_root(parents_row, i)]], axis=0)
        window = seq[-W:]
        y[i] = np.sum(w.T * window, axis=0)
        if bias is not None:
            y[i] += _f64(bias)
    if activation == "silu":
        y = y * sigmoid(y)
    elif activation not in (None, "none"):
        raise ValueError("activation must be 'silu' or None")
    return y


def verify(mixed_qkv, a, b, *, N, H, HV, K, V, scale, conv_weight, conv_state,
           initial_state, initial_state_indices, conv_bias=None,
           conv_state_indices=None, parents=None, activation="silu",
           snapshot_indices=None, num_snapshot_slots=None, A_log=None,
           dt_bias=None, lower_bound=None, beta_is_raw=True,
           use_qk_l2norm_in_kernel=True):
    """Speculative target verify over chain or tree drafts.

    mixed_qkv [B*N, 2*H*K + HV*V] pre-conv tokens (q || k || v channels);
    a [B*N, HV*K] raw gate; b [B*N, HV] raw beta; conv_state [slots, C, W-1].
    Node i of request r starts from its parent's state (the pool state for a
    root) and its state is a per-candidate snapshot ([42857] Modifications: chain
    / tree verification with per-candidate state snapshots).  The pool and
    the conv state are only read.

    Returns (o [B*N, HV, V], snapshots {(snapshot slot, node): [HV, V, K]}).
    """
    mixed = _f64(mixed_qkv)
    BN, C = mixed.shape
    B = BN // N
    if C != 2 * H * K + HV * V:
        raise ValueError("mixed_qkv width must be 2*H*K + HV*V")
    if parents is None:
        parents = np.tile(np.arange(N) - 1, (B, 1))
    check_parents(parents, N)
    sidx = np.arange(B) if snapshot_indices is None else np.asarray(snapshot_indices)
    cidx = np.asarray(initial_state_indices) if conv_state_indices is None else np.asarray(conv_state_indices)
    g_all = activate_gate(_f64(a).reshape(BN, HV, K), A_log, dt_bias, lower_bound)
    beta_all = activate_beta(b, beta_is_raw)
    o = np.zeros((BN, HV, V))
    snaps = {}
    for r in range(B):
        s = int(initial_state_indices[r])
        if s < 0:
            continue
        y = causal_conv_draft(mixed[r * N:(r + 1) * N], conv_state[int(cidx[r])],
                              conv_weight, conv_bias, parents[r], activation)
        q = y[:, :H * K].reshape(N, H, K)
        k = y[:, H * K:2 * H * K].reshape(N, H, K)
        v = y[:, 2 * H * K:].reshape(N, HV, V)
        if use_qk_l2norm_in_kernel:
            q, k = l2_normalize(q), l2_normalize(k)
        q, k = expand_qk_heads(q, HV), expand_qk_heads(k, HV)
        S0 = _pool_to_S(initial_state[s])
        states = []
        for i in range(N):
            p = int(parents[r][i])
            Sp = S0 if p < 0 else states[p]
            Si, o[r * N + i] = kda_step(Sp, q[i], k[i], v[i], g_all[r * N + i],
                                        beta_all[r * N + i], scale)
            states.append(Si)
            snaps[(int(sidx[r]), i)] = _S_to_pool(Si)
    return o, snaps


def commit(accepted, *, N, snapshots, initial_state, initial_state_indices,
           conv_state, mixed_qkv, parents=None, snapshot_indices=None,
           conv_state_indices=None):
    """Commit the accepted node of every request.

    accepted [B] is the index of the last accepted node (-1: none accepted).
    The pool slot takes that node's snapshot; the conv state rolls to the
    last W-1 inputs of conv_state followed by the path root..accepted ([42857]
    review thread: commit a partially accepted prefix between verify rounds).
    snapshots is an array [snap_slots, N, HV, V, K].  Returns (pool, conv_state).
    """
    pool = np.array(initial_state, dtype=np.float64, copy=True)
    cs = np.array(conv_state, dtype=np.float64, copy=True)
    B = len(accepted)
    if parents is None:
        parents = np.tile(np.arange(N) - 1, (B, 1))
    sidx = np.arange(B) if snapshot_indices is None else np.asarray(snapshot_indices)
    cidx = np.asarray(initial_state_indices) if conv_state_indices is None else np.asarray(conv_state_indices)
    mixed = np.asarray(mixed_qkv)
    Wm1 = cs.shape[-1]
    for r in range(B):
        acc = int(accepted[r])
        s = int(initial_state_indices[r])
        if acc < 0 or s < 0:
            continue
        pool[s] = snapshots[int(sidx[r]), acc]
        path = path_to_root(parents[r], acc)
        seq = np.concatenate([cs[int(cidx[r])].T, mixed[r * N + np.array(path)]], axis=0)
        cs[int(cidx[r])] = seq[-Wm1:].T
    return pool, cs


def commit_replay(accepted, mixed_qkv, a, b, *, N, H, HV, K, V, scale, conv_weight,
                  conv_state, initial_state, initial_state_indices, conv_bias=None,
                  conv_state_indices=None, parents=None, activation="silu", A_log=None,
                  dt_bias=None, lower_bound=None, beta_is_raw=True,
                  use_qk_l2norm_in_kernel=True):
    """Commit without per-candidate snapshots (the ReplaySSM direction the
    pages rank above snapshot verify, mechanism not described there):
    verify only reads the pool, and commit replays the recurrence over the
    accepted path root .. accepted[r] from the request's pool state, with
    the conv outputs verify saw (same draft, same conv state).  The conv
    state then rolls exactly as in `commit`.  The arguments are those of
    `verify` plus `accepted`.  Returns (pool, conv_state).
    """
    mixed = _f64(mixed_qkv)
    BN = mixed.shape[0]
    B = BN // N
    pool = np.array(initial_state, dtype=np.float64, copy=True)
    cs = np.array(conv_state, dtype=np.float64, copy=True)
    if parents is None:
        parents = np.tile(np.arange(N) - 1, (B, 1))
    check_parents(parents, N)
    cidx = np.asarray(initial_state_indices) if conv_state_indices is None else np.asarray(conv_state_indices)
    g_all = activate_gate(_f64(a).reshape(BN, HV, K), A_log, dt_bias, lower_bound)
    beta_all = activate_beta(b, beta_is_raw)
    Wm1 = cs.shape[-1]
    for r in range(B):
        acc = int(accepted[r])
        s = int(initial_state_indices[r])
        if acc < 0 or s < 0:
            continue
        y = causal_conv_draft(mixed[r * N:(r + 1) * N], conv_state[int(cidx[r])],
                              conv_weight, conv_bias, parents[r], activation)
        q = y[:, :H * K].reshape(N, H, K)
        k = y[:, H * K:2 * H * K].reshape(N, H, K)
        v = y[:, 2 * H * K:].reshape(N, HV, V)
        if use_qk_l2norm_in_kernel:
            q, k = l2_normalize(q), l2_normalize(k)
        q, k = expand_qk_heads(q, HV), expand_qk_heads(k, HV)
        path = path_to_root(parents[r], acc)
        S = _pool_to_S(initial_state[s])
        for i in path:
            S, _ = kda_step(S, q[i], k[i], v[i], g_all[r * N + i], beta_all[r * N + i], scale)
        pool[s] = _S_to_pool(S)
        seq = np.concatenate([cs[int(cidx[r])].T, mixed[r * N + np.array(path)]], axis=0)
        cs[int(cidx[r])] = seq[-Wm1:].T
    return pool, cs


def conv_update(x, *, conv_weight, conv_state, conv_state_indices, conv_bias=None,
                activation="silu"):
    """One-token depthwise causal conv update, the step before a packed
    decode whose q || k || v channels come out of the conv ([42905] Summary:
    conv1d then recurrence; the same conv reading as causal_conv_draft).

    x [B, C] pre-conv channels of one token per request; conv_state
    [slots, C, W-1] (oldest first); weight [C, W]; bias [C] or None.  For
    request r with s = conv_state_indices[r] >= 0 the window is
    conv_state[s] followed by x[r]; y[r] = sum_j w[:, j] * window[j]
    (+ bias), then SiLU if activation == 'silu'; conv_state[s] keeps the
    window's last W-1 entries.  A negative index: y[r] = 0, no state
    touched.  Returns (y [B, C], conv_state).
    """
    x = _f64(x)
    B, C = x.shape
    cs = np.array(conv_state, dtype=np.float64, copy=True)
    w = _f64(conv_weight)
    y = np.zeros((B, C))
    for r in range(B):
        s = int(conv_state_indices[r])
        if s < 0:
            continue
        window = np.concatenate([cs[s], x[r][:, None]], axis=1)     # [C, W]
        z = np.sum(w * window, axis=1)
        if conv_bias is not None:
            z = z + _f64(conv_bias)
        if activation == "silu":
            z = z * sigmoid(z)
        elif activation not in (None, "none"):
            raise ValueError("activation must be 'silu' or None")
        y[r] = z
        cs[s] = window[:, 1:]
    return y, cs


def decode_conv(mixed_qkv, a, b, *, H, HV, K, V, scale, conv_weight, conv_state,
                initial_state, initial_state_indices, conv_state_indices=None,
                conv_bias=None, activation="silu", A_log=None, dt_bias=None,
                lower_bound=None, beta_is_raw=True, use_qk_l2norm_in_kernel=True):
    """One decode step whose q || k || v come out of the one-token conv
    update ([42905] Summary: the conv1d update and the recurrence in one
    launch): conv_update on the token's pre-conv channels, then decode on
    the q, k and v column ranges of its output.  A request whose state index
    is negative is padding for both: zero output, neither the pool nor the
    conv state touched.  Returns (o [B, HV, V], new pool, new conv_state).
    """
    B = np.asarray(mixed_qkv).shape[0]
    sidx = np.asarray(initial_state_indices)
    cidx = sidx if conv_state_indices is None else np.asarray(conv_state_indices)
    cidx = np.where(sidx < 0, -1, cidx)
    y, cs = conv_update(mixed_qkv, conv_weight=conv_weight, conv_state=conv_state,
                        conv_state_indices=cidx, conv_bias=conv_bias, activation=activation)
    HK = H * K
    q = y[:, :HK].reshape(B, H, K)
    k = y[:, HK:2 * HK].reshape(B, H, K)
    v = y[:, 2 * HK:2 * HK + HV * V].reshape(B, HV, V)
    o, pool = decode(q, k, v, a, b, scale=scale, initial_state=initial_state,
                     initial_state_indices=sidx, A_log=A_log, dt_bias=dt_bias,
                     lower_bound=lower_bound, beta_is_raw=beta_is_raw,
                     use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel)
    return o, pool, cs
