"""Seeded synthetic KDA workloads shared by the tests, the benchmark and the
oracle checks.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic.  Every tensor is a NumPy array.  "bf16" inputs are
float32 arrays whose values are exactly representable in bfloat16 (rounded
here, round-to-nearest-even), so the HIP path (which receives them as
bfloat16) and the float64 oracle see the same numbers.

Workloads follow the pages' microbenchmark shapes ("[KDA] Support Helion MTP
verification and harden prefill, decode", KDA microbenchmarks: 16 heads of
dimension 128, BF16 inputs, FP32 state, bounded gate -5; "[KDA] Default
GLM-5-Next spec verify to the CuTe DSL KDA kernel", Results: 6 draft tokens
per request, conv1d + recurrence) and the serving flags on the first page
(state pool of 240 slots, at most 48 running requests, 8192-token prefill
chunks).  Draw order per workload is fixed and listed in each function.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BASE_SEED = 42
LN16 = math.log(16.0)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); the
    result is returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(np.shape(x))


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


@dataclass
class PrefillCase:
    q: np.ndarray            # [B, T, H, K]
    k: np.ndarray            # [B, T, H, K]
    v: np.ndarray            # [B, T, HV, V]
    g: np.ndarray            # [B, T_g, HV, K] raw gate, T_g >= T
    beta: np.ndarray         # [B, T_b, HV] raw beta, T_b >= T
    A_log: np.ndarray        # [HV] float32
    dt_bias: np.ndarray      # [HV*K] float32
    lower_bound: Optional[float]    # None: unbounded gate
    scale: float
    pool: np.ndarray         # [slots, HV, V, K] float32
    indices: np.ndarray      # [N] int32
    cu_seqlens: Optional[np.ndarray]  # [N+1] int32 or None
    chunk_size: int
    dtype: str               # "bf16" or "f32": q, k, v, g, beta and o
    beta_is_raw: bool = True
    use_qk_l2norm: bool = True
    name: str = ""

    @property
    def B(self): return self.q.shape[0]
    @property
    def T(self): return self.q.shape[1]
    @property
    def H(self): return self.q.shape[2]
    @property
    def K(self): return self.q.shape[3]
    @property
    def HV(self): return self.v.shape[2]
    @property
    def V(self): return self.v.shape[3]
    @property
    def N(self): return len(self.indices)

    def lengths(self):
        if self.cu_seqlens is None:
            return [self.T] * self.B
        return list(np.diff(self.cu_seqlens).astype(int))


def prefill_case(*, seed: int, B: int = 1, T: int, H: int, K: int, V: int,
                 dtype: str = "bf16", chunk_size: int = 64,
                 lengths=None, pad_rows: int = 0, pad_value: float = 1e4,
                 slots: int = 240, pool_std: float = 0.02,
                 zero_pool: bool = False, nan_free_slots: bool = True,
                 HV: Optional[int] = None, unbounded: bool = False,
                 name: str = "") -> PrefillCase:
    """Prefill workload.

    Draw order: q, k [.., H, K], v [.., HV, V], raw g [.., HV, K], raw beta
    (all N(0,1)), A_log ~ U(0, ln 16) [HV], dt_bias ~ N(0, 0.1) [HV*K], pool
    ~ N(0, pool_std) (or zeros), then a permutation of the slots whose first
    N entries are the state indices, then (varlen only) a permutation of
    ``lengths``.  HV defaults to H (grouped heads otherwise); ``unbounded``
    drops the lower bound of the gate.  Rows T .. T+pad_rows-1 of g and beta
    hold ``pad_value`` (pages: gate/beta padded to the graph bucket must be
    ignored).
    """
    HV = H if HV is None else HV
    rng = np.random.default_rng(seed)
    q = _as_dtype(rng.standard_normal((B, T, H, K)), dtype)
    k = _as_dtype(rng.standard_normal((B, T, H, K)), dtype)
    v = _as_dtype(rng.standard_normal((B, T, HV, V)), dtype)
    g = _as_dtype(rng.standard_normal((B, T, HV, K)), dtype)
    beta = _as_dtype(rng.standard_normal((B, T, HV)), dtype)
    A_log = rng.uniform(0.0, LN16, size=HV).astype(np.float32)
    dt_bias = (0.1 * rng.standard_normal(HV * K)).astype(np.float32)
    if zero_pool:
        pool = np.zeros((slots, HV, V, K), np.float32)
    else:
        pool = (pool_std * rng.standard_normal((slots, HV, V, K))).astype(np.float32)
    perm = rng.permutation(slots).astype(np.int32)
    cu = None
    if lengths is not None:
        assert B == 1 and sum(lengths) == T
        lens = np.asarray(lengths)[rng.permutation(len(lengths))]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        n_seq = len(lengths)
    else:
        n_seq = B
    indices = perm[:n_seq].copy()
    if pad_rows:
        gp = np.full((B, pad_rows, HV, K), pad_value, np.float32)
        bp = np.full((B, pad_rows, HV), pad_value, np.float32)
        g = np.concatenate([g, gp], axis=1)
        beta = np.concatenate([beta, bp], axis=1)
    return PrefillCase(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log,
                       dt_bias=dt_bias, lower_bound=None if unbounded else -5.0, scale=K ** -0.5,
                       pool=pool, indices=indices, cu_seqlens=cu,
                       chunk_size=chunk_size, dtype=dtype, name=name)


def config0_tiny() -> PrefillCase:
    """Tiny prefill, float32 everywhere: 1 sequence of 128 tokens, 4 heads of
    32 x 32, chunk 16, zero initial state in slot 1 of a 2-slot pool; slot 0
    holds a NaN sentinel that must stay untouched."""
    c = prefill_case(seed=BASE_SEED + 0, B=1, T=128, H=4, K=32, V=32,
                     dtype="f32", chunk_size=16, slots=2, zero_pool=True,
                     name="tiny T=128 H=4 K=V=32 C=16 fp32")
    c.pool[0] = np.nan
    c.indices = np.array([1], np.int32)
    return c


def config2_prefill(T: int = 4096) -> PrefillCase:
    """Fixed-length prefill: batch 1 x T tokens, 16 heads of 128 x 128, bf16
    inputs, chunk 64, one random slot of a 240-slot fp32 pool."""
    return prefill_case(seed=BASE_SEED + 2, B=1, T=T, H=16, K=128, V=128,
                        dtype="bf16", chunk_size=64,
                        name=f"prefill 1x{T} H=16 K=V=128 C=64 bf16")


VARLEN_LENGTHS = [1, 7, 63, 64, 65, 500, 1023, 2048, 4421]


def config3_varlen(pad_value: float = 1e4) -> PrefillCase:
    """Varlen prefill packed to 8192 tokens (lengths 1, 7, 63, 64, 65, 500,
    1023, 2048 and the remainder 4421, order shuffled by the seed); g and beta
    padded to 12288 rows filled with ``pad_value``."""
    return prefill_case(seed=BASE_SEED + 3, B=1, T=8192, H=16, K=128, V=128,
                        dtype="bf16", chunk_size=64, lengths=VARLEN_LENGTHS,
                        pad_rows=12288 - 8192, pad_value=pad_value,
                        name="varlen 8192 (9 seqs) H=16 K=V=128 C=64 bf16, g/beta padded to 12288")


@dataclass
class DecodeCase:
    mixed_qkv: np.ndarray    # [B, 2*H*K + HV*V] (q || k || v)
    a: np.ndarray            # [B, HV*K] raw gate
    b: np.ndarray            # [B, HV] raw beta
    A_log: np.ndarray
    dt_bias: np.ndarray
    lower_bound: Optional[float]    # None: unbounded gate
    scale: float
    pool: np.ndarray         # [slots, HV, V, K]
    indices: np.ndarray      # [B] int32, negative = padded request
    H: int
    HV: int
    K: int
    V: int
    dtype: str = "bf16"
    beta_is_raw: bool = True
    use_qk_l2norm: bool = True
    name: str = ""

    @property
    def B(self): return self.mixed_qkv.shape[0]

    def q(self):
        return self.mixed_qkv[:, :self.H * self.K].reshape(self.B, self.H, self.K)

    def k(self):
        return self.mixed_qkv[:, self.H * self.K:2 * self.H * self.K].reshape(self.B, self.H, self.K)

    def v(self):
        return self.mixed_qkv[:, 2 * self.H * self.K:].reshape(self.B, self.HV, self.V)


def decode_case(*, seed: int, B: int, H: int, K: int, V: int, slots: int = 240,
                dtype: str = "bf16", pad_requests=(), HV: Optional[int] = None,
                unbounded: bool = False, name: str = "") -> DecodeCase:
    """Packed decode workload.  Draw order: mixed_qkv [B, 2HK + HV V], a,
    b (N(0,1)), A_log ~ U(0, ln 16) [HV], dt_bias ~ N(0, 0.1) [HV*K], pool
    ~ N(0, 0.02), slot permutation (first B entries are the indices).
    Requests listed in ``pad_requests`` get index -1.  HV defaults to H;
    ``unbounded`` drops the lower bound of the gate."""
    HV = H if HV is None else HV
    rng = np.random.default_rng(seed)
    width = 2 * H * K + HV * V
    mixed = _as_dtype(rng.standard_normal((B, width)), dtype)
    a = _as_dtype(rng.standard_normal((B, HV * K)), dtype)
    b = _as_dtype(rng.standard_normal((B, HV)), dtype)
    A_log = rng.uniform(0.0, LN16, size=HV).astype(np.float32)
    dt_bias = (0.1 * rng.standard_normal(HV * K)).astype(np.float32)
    pool = (0.02 * rng.standard_normal((slots, HV, V, K))).astype(np.float32)
    indices = rng.permutation(slots)[:B].astype(np.int32)
    for r in pad_requests:
        indices[r] = -1
    return DecodeCase(mixed_qkv=mixed, a=a, b=b, A_log=A_log, dt_bias=dt_bias,
                      lower_bound=None if unbounded else -5.0, scale=K ** -0.5, pool=pool,
                      indices=indices, H=H, HV=HV, K=K, V=V, dtype=dtype, name=name)


def config1_decode() -> DecodeCase:
    """Packed decode: 48 requests x 1 token, 16 heads of 128 x 128, bf16,
    240-slot fp32 pool, indices = a random subset of the slots."""
    return decode_case(seed=BASE_SEED + 1, B=48, H=16, K=128, V=128,
                       name="decode 48x1 H=16 K=V=128 bf16")


@dataclass
class VerifyCase:
    mixed_qkv: np.ndarray    # [B*N, conv_dim] pre-conv
    a: np.ndarray            # [B*N, HV*K]
    b: np.ndarray            # [B*N, HV]
    conv_weight: np.ndarray  # [conv_dim, W]
    conv_state: np.ndarray   # [slots, conv_dim, W-1], oldest first
    A_log: np.ndarray
    dt_bias: np.ndarray
    lower_bound: Optional[float]    # None: unbounded gate
    scale: float
    pool: np.ndarray         # [slots, HV, V, K]
    indices: np.ndarray      # [B] int32
    parents: Optional[np.ndarray]   # [B, N] int32 or None (chain)
    N: int
    H: int
    HV: int
    K: int
    V: int
    dtype: str = "bf16"
    activation: str = "silu"
    beta_is_raw: bool = True
    use_qk_l2norm: bool = True
    snapshot_slots: int = 0
    snapshot_indices: Optional[np.ndarray] = None
    name: str = ""

    @property
    def B(self): return self.mixed_qkv.shape[0] // self.N

    @property
    def conv_dim(self): return self.mixed_qkv.shape[1]


def random_tree(rng, B: int, N: int, multi_root: bool = False) -> np.ndarray:
    """parents[b, 0] = -1 and parents[b, i] ~ U{0 .. i-1} (or U{-1 .. i-1}
    when multi_root)."""
    p = np.empty((B, N), np.int32)
    for b in range(B):
        p[b, 0] = -1
        for i in range(1, N):
            p[b, i] = rng.integers(-1 if multi_root else 0, i)
    return p


def verify_case(*, seed: int, B: int, N: int, H: int, K: int, V: int,
                tree: bool, width: int = 4, slots: int = 240,
                dtype: str = "bf16", multi_root: bool = False,
                pad_requests=(), HV: Optional[int] = None, unbounded: bool = False,
                name: str = "") -> VerifyCase:
    """Target-verify workload.  Draw order: mixed_qkv [B*N, 2HK + HV V], a,
    b (N(0,1)), conv_weight ~ U(-1/2, 1/2), conv_state ~ N(0,1), A_log ~
    U(0, ln 16) [HV], dt_bias ~ N(0, 0.1) [HV*K], pool ~ N(0, 0.02), slot
    permutation, then (tree only) the parents.  The conv state has one entry
    per pool slot and is indexed by the same slot indices.  HV defaults to
    H; ``unbounded`` drops the lower bound of the gate."""
    HV = H if HV is None else HV
    rng = np.random.default_rng(seed)
    cdim = 2 * H * K + HV * V
    mixed = _as_dtype(rng.standard_normal((B * N, cdim)), dtype)
    a = _as_dtype(rng.standard_normal((B * N, HV * K)), dtype)
    b = _as_dtype(rng.standard_normal((B * N, HV)), dtype)
    w = _as_dtype(rng.uniform(-0.5, 0.5, size=(cdim, width)), dtype)
    cs = _as_dtype(rng.standard_normal((slots, cdim, width - 1)), dtype)
    A_log = rng.uniform(0.0, LN16, size=HV).astype(np.float32)
    dt_bias = (0.1 * rng.standard_normal(HV * K)).astype(np.float32)
    pool = (0.02 * rng.standard_normal((slots, HV, V, K))).astype(np.float32)
    indices = rng.permutation(slots)[:B].astype(np.int32)
    for r in pad_requests:
        indices[r] = -1
    parents = random_tree(rng, B, N, multi_root) if tree else None
    return VerifyCase(mixed_qkv=mixed, a=a, b=b, conv_weight=w, conv_state=cs,
                      A_log=A_log, dt_bias=dt_bias, lower_bound=None if unbounded else -5.0,
                      scale=K ** -0.5, pool=pool, indices=indices,
                      parents=parents, N=N, H=H, HV=HV, K=K, V=V, dtype=dtype,
                      snapshot_slots=B, name=name)


def config4_verify(tree: bool = False) -> VerifyCase:
    """MTP target verify: 48 requests x 6 draft tokens, 16 heads of 128 x
    128, bf16, width-4 causal conv with SiLU, chain or random tree."""
    kind = "tree" if tree else "chain"
    return verify_case(seed=BASE_SEED + 4, B=48, N=6, H=16, K=128, V=128,
                       tree=tree, name=f"verify 48x6 {kind} H=16 K=V=128 bf16 conv4")
