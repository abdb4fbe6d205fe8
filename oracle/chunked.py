"""Chunked (WY / UT) form of the KDA recurrence in float64.
TEST INFRASTRUCTURE ONLY.

It restates, chunk by chunk, the algebra a chunked GPU prefill follows, so a
CPU test can pin that algebra against the token-by-token recurrence in
``oracle.kda``.  No blocking, fusion or reordering beyond these steps.

Per chunk of L <= C tokens of one head, with S the state entering the chunk
([K, V], math orientation) and all products in float64:

  G_r     = sum_{i<=r} g_i                 (in-chunk cumulative log-decay)
  A[r, j] = beta_r sum_c k_rc k_jc exp(G_rc - G_jc)   for j < r, else 0
  P[r, j] = sum_c q_rc k_jc exp(G_rc - G_jc)          for j <= r, else 0
  Tm      = (I + A)^{-1}
  W       = Tm diag(beta) (K * exp(G))
  U'      = Tm diag(beta) V
  U       = U' - W S
  O       = scale ((Q * exp(G)) S + P U)
  S      <- Diag(exp(G_last)) S + (K * exp(G_last - G))^T U

Derivation: write the state after token r as
S_r = Diag(e^{G_r}) S + sum_{j<=r} Diag(e^{G_r - G_j}) k_j u_j^T with
u_r = beta_r (v_r - (Diag(e^{g_r}) S_{r-1})^T k_r); stacking the u_r gives
(I + A) U = diag(beta) V - diag(beta) (K * e^G) S.
"""

from __future__ import annotations

import numpy as np

from . import kda as _kda


def _chunk(S, q, k, v, g, beta, scale):
    """One chunk of one head.  S [K, V]; q, k, g [L, K]; v [L, V]; beta [L]."""
    L = q.shape[0]
    G = np.cumsum(g, axis=0)
    diff = G[:, None, :] - G[None, :, :]                  # [r, j, c] = G_r - G_j
    lower_incl = np.tril(np.ones((L, L), dtype=bool))
    lower_strict = np.tril(np.ones((L, L), dtype=bool), -1)
    E = np.where(lower_incl[:, :, None], np.exp(np.where(lower_incl[:, :, None], diff, 0.0)), 0.0)
    A = beta[:, None] * np.einsum("rc,jc,rjc->rj", k, k, E) * lower_strict
    P = np.einsum("rc,jc,rjc->rj", q, k, E) * lower_incl
    Tm = np.linalg.inv(np.eye(L) + A)
    eG = np.exp(G)
    W = Tm @ (beta[:, None] * (k * eG))
    Up = Tm @ (beta[:, None] * v)
    U = Up - W @ S
    O = scale * ((q * eG) @ S + P @ U)
    S_new = np.exp(G[-1])[:, None] * S + (k * np.exp(G[-1][None, :] - G)).T @ U
    return S_new, O


def prefill_chunked(q, k, v, g, beta, *, scale, chunk_size, initial_state,
                    initial_state_indices, use_qk_l2norm_in_kernel=False,
                    cu_seqlens=None, A_log=None, dt_bias=None,
                    lower_bound=None, beta_is_raw=False,
                    output_intermediate_states=False):
    """Same contract and return value as ``oracle.kda.prefill``, computed
    chunk by chunk.  Chunks restart at every sequence start."""
    if initial_state is None or initial_state_indices is None:
        raise ValueError("prefill: a state pool and one slot index per sequence are required")
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T = q.shape[:2]
    K = q.shape[3]
    HV, V = v.shape[2:]
    g = _kda._token_rows(g, T, "g")
    beta = _kda._token_rows(beta, T, "beta")
    if use_qk_l2norm_in_kernel:
        q, k = _kda.l2_normalize(q), _kda.l2_normalize(k)
    # grouped heads: value head h reads q/k head h // (HV / H)
    q, k = _kda.expand_qk_heads(q, HV), _kda.expand_qk_heads(k, HV)
    g = _kda.activate_gate(g, A_log, dt_bias, lower_bound)
    beta = _kda.activate_beta(beta, beta_is_raw)
    seqs = _kda._sequences(B, T, cu_seqlens)
    idx = [int(x) for x in np.asarray(initial_state_indices)]
    pool = np.array(initial_state, dtype=np.float64, copy=True)
    o = np.zeros((B, T, HV, V))
    inter = []
    C = int(chunk_size)
    for n, (b, t0, t1) in enumerate(seqs):
        S = np.transpose(pool[idx[n]], (0, 2, 1)).copy()   # [HV, K, V]
        for c0 in range(t0, t1, C):
            c1 = min(c0 + C, t1)
            if output_intermediate_states:
                inter.append(np.transpose(S, (0, 2, 1)).copy())
            for h in range(HV):
                S[h], o[b, c0:c1, h] = _chunk(S[h], q[b, c0:c1, h], k[b, c0:c1, h],
                                              v[b, c0:c1, h], g[b, c0:c1, h],
                                              beta[b, c0:c1, h], scale)
        pool[idx[n]] = np.transpose(S, (0, 2, 1))
    inter = np.stack(inter) if inter else np.zeros((0, HV, V, K))
    return o, pool, (inter if output_intermediate_states else None)
