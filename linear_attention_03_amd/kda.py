"""Python binding of libkda (ctypes).  Argument marshalling only: every step
of every phase runs in the HIP kernels of libkda.so; PyTorch supplies device
memory and the current stream.  The functions carry the C-ABI names
(kda_prefill -> prefill, ...).

The library is loaded on first use.  If libkda.so is missing the call fails
with an error naming the build command; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP = 0, 1, 2, 3
KDA_F32, KDA_BF16 = 0, 1
KDA_ACT_NONE, KDA_ACT_SILU = 0, 1
KDA_ARGS_PREFILL, KDA_ARGS_DECODE, KDA_ARGS_VERIFY, KDA_ARGS_COMMIT, KDA_ARGS_CONV_UPDATE = 0, 1, 2, 3, 4
KDA_ARGS_DECODE_CONV = 5

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[libkda status {status}] {message}")
        self.status = status
        self.message = message


class KdaInvalidArgument(KdaError, ValueError):
    pass


class KdaUnsupported(KdaError, NotImplementedError):
    pass


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("dtype", _i32),
        ("B", _i64), ("T", _i64), ("H", _i64), ("HV", _i64), ("K", _i64), ("V", _i64),
        ("chunk_size", _i64),
        ("q", _vp), ("q_stride", _i64 * 3),
        ("k", _vp), ("k_stride", _i64 * 3),
        ("v", _vp), ("v_stride", _i64 * 3),
        ("o", _vp), ("o_stride", _i64 * 3),
        ("g", _vp), ("g_rows", _i64), ("g_stride", _i64 * 3),
        ("beta", _vp), ("beta_rows", _i64), ("beta_stride", _i64 * 2),
        ("A_log", _vp), ("dt_bias", _vp), ("lower_bound", _f32), ("has_lower_bound", _i32),
        ("beta_is_raw", _i32), ("use_qk_l2norm", _i32), ("scale", _f32), ("run_chunks", _i32),
        ("cu_seqlens", _vp), ("num_seqs", _i64),
        ("state_pool", _vp), ("num_slots", _i64), ("state_indices", _vp),
        ("intermediate_states", _vp), ("num_intermediate", _i64),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("dtype", _i32),
        ("B", _i64), ("H", _i64), ("HV", _i64), ("K", _i64), ("V", _i64),
        ("q", _vp), ("q_stride", _i64 * 2),
        ("k", _vp), ("k_stride", _i64 * 2),
        ("v", _vp), ("v_stride", _i64 * 2),
        ("o", _vp), ("o_stride", _i64 * 2),
        ("a", _vp), ("a_stride", _i64), ("a_cols", _i64),
        ("b", _vp), ("b_stride", _i64),
        ("A_log", _vp), ("dt_bias", _vp), ("lower_bound", _f32), ("has_lower_bound", _i32),
        ("beta_is_raw", _i32), ("use_qk_l2norm", _i32), ("scale", _f32), ("reserved0", _i32),
        ("state_pool", _vp), ("num_slots", _i64), ("state_indices", _vp),
    ]


class DecodeConvArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("dtype", _i32),
        ("B", _i64), ("H", _i64), ("HV", _i64), ("K", _i64), ("V", _i64),
        ("mixed_qkv", _vp), ("mixed_stride", _i64),
        ("conv_weight", _vp), ("conv_bias", _vp), ("conv_width", _i64),
        ("conv_activation", _i32), ("reserved0", _i32),
        ("conv_state", _vp), ("num_conv_slots", _i64), ("conv_state_indices", _vp),
        ("o", _vp), ("o_stride", _i64 * 2),
        ("a", _vp), ("a_stride", _i64), ("a_cols", _i64),
        ("b", _vp), ("b_stride", _i64),
        ("A_log", _vp), ("dt_bias", _vp), ("lower_bound", _f32), ("has_lower_bound", _i32),
        ("beta_is_raw", _i32), ("use_qk_l2norm", _i32), ("scale", _f32), ("reserved1", _i32),
        ("state_pool", _vp), ("num_slots", _i64), ("state_indices", _vp),
    ]


class VerifyArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("dtype", _i32),
        ("B", _i64), ("N", _i64), ("H", _i64), ("HV", _i64), ("K", _i64), ("V", _i64),
        ("mixed_qkv", _vp), ("mixed_stride", _i64),
        ("conv_weight", _vp), ("conv_bias", _vp), ("conv_width", _i64),
        ("conv_activation", _i32), ("reserved0", _i32),
        ("conv_state", _vp), ("num_conv_slots", _i64), ("conv_state_indices", _vp),
        ("parents", _vp),
        ("o", _vp), ("o_stride", _i64 * 2),
        ("a", _vp), ("a_stride", _i64), ("a_cols", _i64),
        ("b", _vp), ("b_stride", _i64),
        ("A_log", _vp), ("dt_bias", _vp), ("lower_bound", _f32), ("has_lower_bound", _i32),
        ("beta_is_raw", _i32), ("use_qk_l2norm", _i32), ("scale", _f32), ("reserved1", _i32),
        ("state_pool", _vp), ("num_slots", _i64), ("state_indices", _vp),
        ("snapshots", _vp), ("num_snapshot_slots", _i64), ("snapshot_indices", _vp),
    ]


class ConvUpdateArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("dtype", _i32),
        ("B", _i64), ("conv_dim", _i64), ("conv_width", _i64),
        ("conv_activation", _i32), ("reserved0", _i32),
        ("x", _vp), ("x_stride", _i64), ("y", _vp), ("y_stride", _i64),
        ("conv_weight", _vp), ("conv_bias", _vp),
        ("conv_state", _vp), ("num_conv_slots", _i64), ("conv_state_indices", _vp),
    ]


class CommitArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("dtype", _i32),
        ("B", _i64), ("N", _i64), ("HV", _i64), ("K", _i64), ("V", _i64),
        ("conv_dim", _i64), ("conv_width", _i64),
        ("accepted", _vp), ("parents", _vp),
        ("snapshots", _vp), ("num_snapshot_slots", _i64), ("snapshot_indices", _vp),
        ("state_pool", _vp), ("num_slots", _i64), ("state_indices", _vp),
        ("conv_state", _vp), ("num_conv_slots", _i64), ("conv_state_indices", _vp),
        ("mixed_qkv", _vp), ("mixed_stride", _i64),
    ]


EXPORTS = ["kda_abi_version", "kda_args_size", "kda_last_error", "kda_prefill_workspace_size",
           "kda_prefill", "kda_decode", "kda_verify", "kda_commit", "kda_commit_replay",
           "kda_conv_update", "kda_set_call_events", "kda_prefill_noalloc", "kda_decode_conv",
           "kda_prefill_path"]

_lib = None


def lib():
    """Load libkda.so (once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m linear_attention_03_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        L.kda_abi_version.restype = ctypes.c_int
        L.kda_args_size.restype = ctypes.c_size_t
        L.kda_args_size.argtypes = [ctypes.c_int]
        L.kda_last_error.restype = ctypes.c_char_p
        L.kda_prefill_workspace_size.restype = ctypes.c_int
        L.kda_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.kda_prefill.restype = ctypes.c_int
        L.kda_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _vp, ctypes.c_size_t, _vp]
        L.kda_prefill_path.restype = ctypes.c_int
        L.kda_prefill_path.argtypes = [ctypes.POINTER(PrefillArgs), ctypes.POINTER(ctypes.c_int32)]
        L.kda_decode.restype = ctypes.c_int
        L.kda_decode.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
        L.kda_verify.restype = ctypes.c_int
        L.kda_verify.argtypes = [ctypes.POINTER(VerifyArgs), _vp]
        L.kda_commit.restype = ctypes.c_int
        L.kda_commit.argtypes = [ctypes.POINTER(CommitArgs), _vp]
        L.kda_conv_update.restype = ctypes.c_int
        L.kda_conv_update.argtypes = [ctypes.POINTER(ConvUpdateArgs), _vp]
        L.kda_commit_replay.restype = ctypes.c_int
        L.kda_commit_replay.argtypes = [ctypes.POINTER(VerifyArgs), _vp, _vp]
        L.kda_decode_conv.restype = ctypes.c_int
        L.kda_decode_conv.argtypes = [ctypes.POINTER(DecodeConvArgs), _vp]
        L.kda_prefill_noalloc.restype = ctypes.c_int
        L.kda_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), _vp]
        L.kda_set_call_events.restype = ctypes.c_int
        L.kda_set_call_events.argtypes = [_vp, _vp]
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().kda_abi_version()


def args_size(which: int) -> int:
    return lib().kda_args_size(which)


def last_error() -> str:
    return lib().kda_last_error().decode()


def set_call_events(start, stop):
    """kda_set_call_events: the next call on this thread stamps `start` when
    its first kernel begins and `stop` when its last kernel ends.  start and
    stop are torch.cuda.Event(enable_timing=True) objects already recorded
    once (so that they exist), raw hipEvent_t handles, or None."""
    def handle(e):
        if e is None:
            return None
        return e if isinstance(e, int) else e.cuda_event
    _check(lib().kda_set_call_events(handle(start), handle(stop)))


def _check(status: int):
    if status == KDA_OK:
        return
    msg = last_error()
    if status == KDA_ERR_INVALID_ARGUMENT:
        raise KdaInvalidArgument(status, msg)
    if status == KDA_ERR_UNSUPPORTED:
        raise KdaUnsupported(status, msg)
    raise KdaError(status, msg)


# ----------------------------------------------------------------- marshalling helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"activations must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _inner_contig(t, name):
    if t is not None and t.dim() > 0 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the innermost dimension must be contiguous")


def _same_dtype(ref, *ts):
    for name, t in ts:
        if t is not None and t.dtype != ref.dtype:
            raise TypeError(f"{name} must have dtype {ref.dtype} (got {t.dtype})")


def _f32_opt(t, name):
    torch = _torch()
    if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous float32 tensor")


def _i32_opt(t, name):
    torch = _torch()
    if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous int32 tensor")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return _torch().cuda.current_stream().cuda_stream


def _on_stream(stream):
    """Context under which tensors this binding allocates (outputs, the
    prefill workspace) belong to the stream the kernels run on: the caching
    allocator then reuses their memory only in that stream's order, so a
    block freed when the call returns is never handed to other work while
    the kernels still read or write it."""
    import contextlib
    if stream is None:
        return contextlib.nullcontext()
    torch = _torch()
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream)
    return torch.cuda.stream(stream)


def _gate_fields(args, A_log, dt_bias, lower_bound, beta_is_raw, use_qk_l2norm, scale):
    _f32_opt(A_log, "A_log")
    _f32_opt(dt_bias, "dt_bias")
    args.A_log = _ptr(A_log)
    args.dt_bias = _ptr(dt_bias)
    args.lower_bound = 0.0 if lower_bound is None else float(lower_bound)
    args.has_lower_bound = 0 if lower_bound is None else 1
    args.beta_is_raw = int(bool(beta_is_raw))
    args.use_qk_l2norm = int(bool(use_qk_l2norm))
    args.scale = float(scale)


# ----------------------------------------------------------------- prefill

def _prefill_args(q, k, v, g, beta, o, *, scale, initial_state, initial_state_indices,
                  use_qk_l2norm_in_kernel, cu_seqlens, A_log, dt_bias, lower_bound,
                  beta_is_raw, chunk_size, intermediate_states, run_chunks=0):
    a = PrefillArgs()
    a.struct_size = ctypes.sizeof(PrefillArgs)
    a.dtype = _dtype_code(q)
    _same_dtype(q, ("k", k), ("v", v), ("g", g), ("beta", beta), ("o", o))
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("g", g), ("beta", beta)):
        _inner_contig(t, name)
    B, T, H, K = q.shape
    a.B, a.T, a.H, a.K = B, T, H, K
    a.HV, a.V = v.shape[2], v.shape[3]
    a.chunk_size = int(chunk_size)
    a.run_chunks = int(run_chunks)
    a.q, a.k, a.v, a.o, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(g), _ptr(beta)
    a.q_stride[:] = q.stride()[:3]
    a.k_stride[:] = k.stride()[:3]
    a.v_stride[:] = v.stride()[:3]
    a.o_stride[:] = o.stride()[:3]
    a.g_rows = g.shape[1]
    a.g_stride[:] = g.stride()[:3]
    a.beta_rows = beta.shape[1]
    a.beta_stride[:] = beta.stride()[:2]
    _gate_fields(a, A_log, dt_bias, lower_bound, beta_is_raw, use_qk_l2norm_in_kernel, scale)
    _i32_opt(cu_seqlens, "cu_seqlens")
    _i32_opt(initial_state_indices, "initial_state_indices")
    _f32_opt(initial_state, "initial_state")
    _f32_opt(intermediate_states, "intermediate_states")
    a.cu_seqlens = _ptr(cu_seqlens)
    a.num_seqs = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    a.state_pool = _ptr(initial_state)
    a.num_slots = 0 if initial_state is None else initial_state.shape[0]
    a.state_indices = _ptr(initial_state_indices)
    a.intermediate_states = _ptr(intermediate_states)
    a.num_intermediate = 0 if intermediate_states is None else intermediate_states.shape[0]
    return a


def prefill_workspace_size(args: PrefillArgs) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().kda_prefill_workspace_size(ctypes.byref(args), ctypes.byref(n)))
    return n.value


PREFILL_PATHS = {0: "general", 1: "matrix"}     # kda_prefill_path_t


def prefill_path_of(args: PrefillArgs) -> str:
    """kda_prefill_path on prepared arguments: "matrix" or "general"."""
    n = ctypes.c_int32(-1)
    _check(lib().kda_prefill_path(ctypes.byref(args), ctypes.byref(n)))
    return PREFILL_PATHS[n.value]


def prefill_path(q, k, v, g, beta, *, scale, initial_state, initial_state_indices,
                 use_qk_l2norm_in_kernel=False, cu_seqlens=None, A_log=None, dt_bias=None,
                 lower_bound=None, beta_is_raw=False, chunk_size=64, intermediate_states=None,
                 o=None, run_chunks=0):
    """Which implementation prefill() takes for these tensors ("matrix" or
    "general"), without launching anything."""
    if o is None:
        o = _torch().empty(q.shape[0], q.shape[1], v.shape[2], v.shape[3], dtype=q.dtype, device=q.device)
    a = _prefill_args(q, k, v, g, beta, o, scale=scale, initial_state=initial_state,
                      initial_state_indices=initial_state_indices,
                      use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, cu_seqlens=cu_seqlens,
                      A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound,
                      beta_is_raw=beta_is_raw, chunk_size=chunk_size,
                      intermediate_states=intermediate_states, run_chunks=run_chunks)
    return prefill_path_of(a)


def prefill_max_chunks(T: int, chunk_size: int, B: int = 1, num_seqs: Optional[int] = None) -> int:
    """Rows needed in intermediate_states: B*ceil(T/C) (fixed) or
    floor(T/C) + num_seqs (packed)."""
    if num_seqs is not None:
        return T // chunk_size + num_seqs
    return B * ((T + chunk_size - 1) // chunk_size)


def prefill(q, k, v, g, beta, *, scale, initial_state, initial_state_indices,
            use_qk_l2norm_in_kernel=False, cu_seqlens=None, A_log=None, dt_bias=None,
            lower_bound=None, beta_is_raw=False, chunk_size=64, intermediate_states=None,
            o=None, workspace=None, stream=None, run_chunks=0):
    """kda_prefill.  q, k [B,T,H,K]; v [B,T,HV,V]; g [B,>=T,HV,K];
    beta [B,>=T,HV]; initial_state [slots,HV,V,K] float32 (updated in
    place); initial_state_indices int32 [num_seqs]; run_chunks selects the
    two-level scan's run length (0: library default).  Returns o [B,T,HV,V]."""
    torch = _torch()
    if o is None:
        with _on_stream(stream):
            o = torch.empty(q.shape[0], q.shape[1], v.shape[2], v.shape[3], dtype=q.dtype, device=q.device)
    a = _prefill_args(q, k, v, g, beta, o, scale=scale, initial_state=initial_state,
                      initial_state_indices=initial_state_indices,
                      use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, cu_seqlens=cu_seqlens,
                      A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound,
                      beta_is_raw=beta_is_raw, chunk_size=chunk_size,
                      intermediate_states=intermediate_states, run_chunks=run_chunks)
    need = prefill_workspace_size(a)
    if workspace is None:
        with _on_stream(stream):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().kda_prefill(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(stream)))
    return o


NOALLOC_SCRATCH_BYTES = 128 << 20      # KDA_NOALLOC_SCRATCH_BYTES


def prefill_noalloc(q, k, v, g, beta, *, o, scale, initial_state, initial_state_indices,
                    use_qk_l2norm_in_kernel=False, cu_seqlens=None, A_log=None, dt_bias=None,
                    lower_bound=None, beta_is_raw=False, chunk_size=64, intermediate_states=None,
                    stream=None, run_chunks=0):
    """kda_prefill_noalloc: kda_prefill with its workspace in the library's
    built-in scratch.  Nothing is allocated here either, so the output `o`
    [B,T,HV,V] is required.  Calls that overlap on one device race."""
    a = _prefill_args(q, k, v, g, beta, o, scale=scale, initial_state=initial_state,
                      initial_state_indices=initial_state_indices,
                      use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, cu_seqlens=cu_seqlens,
                      A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound,
                      beta_is_raw=beta_is_raw, chunk_size=chunk_size,
                      intermediate_states=intermediate_states, run_chunks=run_chunks)
    _check(lib().kda_prefill_noalloc(ctypes.byref(a), _stream(stream)))
    return o


# ----------------------------------------------------------------- decode

def decode(q, k, v, a, b, *, scale, initial_state, initial_state_indices, A_log=None,
           dt_bias=None, lower_bound=None, beta_is_raw=True, use_qk_l2norm_in_kernel=True,
           o=None, stream=None):
    """kda_decode.  q, k [B,H,K] and v [B,HV,V] (views of a packed mixed_qkv
    are fine); a [B, HV*K] raw gate; b [B, HV] raw beta; the pool slots
    initial_state[initial_state_indices[r]] are updated in place.
    Returns o [B,HV,V]."""
    torch = _torch()
    if o is None:
        with _on_stream(stream):
            o = torch.empty(v.shape[0], v.shape[1], v.shape[2], dtype=q.dtype, device=q.device)
    d = DecodeArgs()
    d.struct_size = ctypes.sizeof(DecodeArgs)
    d.dtype = _dtype_code(q)
    _same_dtype(q, ("k", k), ("v", v), ("a", a), ("b", b), ("o", o))
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("a", a), ("b", b)):
        _inner_contig(t, name)
    d.B, d.H, d.K = q.shape
    d.HV, d.V = v.shape[1], v.shape[2]
    d.q, d.k, d.v, d.o, d.a, d.b = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(a), _ptr(b)
    d.q_stride[:] = q.stride()[:2]
    d.k_stride[:] = k.stride()[:2]
    d.v_stride[:] = v.stride()[:2]
    d.o_stride[:] = o.stride()[:2]
    d.a_stride, d.a_cols = a.stride(0), a.shape[1]
    d.b_stride = b.stride(0)
    _gate_fields(d, A_log, dt_bias, lower_bound, beta_is_raw, use_qk_l2norm_in_kernel, scale)
    _f32_opt(initial_state, "initial_state")
    _i32_opt(initial_state_indices, "initial_state_indices")
    d.state_pool = _ptr(initial_state)
    d.num_slots = 0 if initial_state is None else initial_state.shape[0]
    d.state_indices = _ptr(initial_state_indices)
    _check(lib().kda_decode(ctypes.byref(d), _stream(stream)))
    return o


def decode_conv(mixed_qkv, a, b, *, H, HV, K, V, scale, conv_weight, conv_state, initial_state,
                initial_state_indices, conv_bias=None, conv_state_indices=None, activation="silu",
                A_log=None, dt_bias=None, lower_bound=None, beta_is_raw=True,
                use_qk_l2norm_in_kernel=True, o=None, stream=None):
    """kda_decode_conv: the conv update of one token per request and the
    packed decode in one launch.  mixed_qkv [B, 2HK+HV*V] pre-conv;
    conv_weight [C, W]; conv_state [slots, C, W-1] (rolled in place);
    a [B, HV*K]; b [B, HV]; the pool slots are updated in place.
    Returns o [B,HV,V]."""
    torch = _torch()
    B = mixed_qkv.shape[0]
    if o is None:
        with _on_stream(stream):
            o = torch.empty(B, HV, V, dtype=mixed_qkv.dtype, device=mixed_qkv.device)
    _same_dtype(mixed_qkv, ("a", a), ("b", b), ("o", o), ("conv_weight", conv_weight),
                ("conv_bias", conv_bias), ("conv_state", conv_state))
    for name, t in (("mixed_qkv", mixed_qkv), ("a", a), ("b", b), ("o", o)):
        _inner_contig(t, name)
    for name, t in (("conv_weight", conv_weight), ("conv_bias", conv_bias), ("conv_state", conv_state)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _i32_opt(conv_state_indices, "conv_state_indices")
    _i32_opt(initial_state_indices, "initial_state_indices")
    _f32_opt(initial_state, "initial_state")
    d = DecodeConvArgs()
    d.struct_size = ctypes.sizeof(DecodeConvArgs)
    d.dtype = _dtype_code(mixed_qkv)
    d.B, d.H, d.HV, d.K, d.V = B, H, HV, K, V
    d.mixed_qkv, d.mixed_stride = _ptr(mixed_qkv), mixed_qkv.stride(0)
    d.conv_weight, d.conv_bias = _ptr(conv_weight), _ptr(conv_bias)
    d.conv_width = conv_weight.shape[1]
    d.conv_activation = KDA_ACT_SILU if activation == "silu" else KDA_ACT_NONE
    d.conv_state, d.num_conv_slots = _ptr(conv_state), conv_state.shape[0]
    d.conv_state_indices = _ptr(conv_state_indices)
    d.o = _ptr(o)
    d.o_stride[:] = o.stride()[:2]
    d.a, d.a_stride, d.a_cols = _ptr(a), a.stride(0), a.shape[1]
    d.b, d.b_stride = _ptr(b), b.stride(0)
    _gate_fields(d, A_log, dt_bias, lower_bound, beta_is_raw, use_qk_l2norm_in_kernel, scale)
    d.state_pool, d.num_slots = _ptr(initial_state), initial_state.shape[0]
    d.state_indices = _ptr(initial_state_indices)
    _check(lib().kda_decode_conv(ctypes.byref(d), _stream(stream)))
    return o


# ----------------------------------------------------------------- verify / commit

def _verify_args(mixed_qkv, a, b, o, *, N, H, HV, K, V, scale, conv_weight, conv_state,
                 initial_state, initial_state_indices, snapshots, conv_bias, conv_state_indices,
                 parents, activation, snapshot_indices, A_log, dt_bias, lower_bound, beta_is_raw,
                 use_qk_l2norm_in_kernel):
    """Marshal the kda_verify_args struct (shared by verify and commit_replay)."""
    BN = mixed_qkv.shape[0]
    w = VerifyArgs()
    w.struct_size = ctypes.sizeof(VerifyArgs)
    w.dtype = _dtype_code(mixed_qkv)
    _same_dtype(mixed_qkv, ("a", a), ("b", b), ("o", o), ("conv_weight", conv_weight),
                ("conv_bias", conv_bias), ("conv_state", conv_state))
    for name, t in (("mixed_qkv", mixed_qkv), ("a", a), ("b", b), ("o", o)):
        if t is not None:
            _inner_contig(t, name)
    for name, t in (("conv_weight", conv_weight), ("conv_bias", conv_bias), ("conv_state", conv_state)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if BN % N:
        raise ValueError("mixed_qkv rows must be a multiple of N")
    w.B, w.N, w.H, w.HV, w.K, w.V = BN // N, N, H, HV, K, V
    w.mixed_qkv, w.mixed_stride = _ptr(mixed_qkv), mixed_qkv.stride(0)
    w.conv_weight, w.conv_bias = _ptr(conv_weight), _ptr(conv_bias)
    w.conv_width = conv_weight.shape[1]
    w.conv_activation = KDA_ACT_SILU if activation == "silu" else KDA_ACT_NONE
    w.conv_state, w.num_conv_slots = _ptr(conv_state), conv_state.shape[0]
    _i32_opt(conv_state_indices, "conv_state_indices")
    _i32_opt(parents, "parents")
    _i32_opt(initial_state_indices, "initial_state_indices")
    _i32_opt(snapshot_indices, "snapshot_indices")
    _f32_opt(initial_state, "initial_state")
    _f32_opt(snapshots, "snapshots")
    w.conv_state_indices = _ptr(conv_state_indices)
    w.parents = _ptr(parents)
    if o is not None:
        w.o = _ptr(o)
        w.o_stride[:] = o.stride()[:2]
    w.a, w.a_stride, w.a_cols = _ptr(a), a.stride(0), a.shape[1]
    w.b, w.b_stride = _ptr(b), b.stride(0)
    _gate_fields(w, A_log, dt_bias, lower_bound, beta_is_raw, use_qk_l2norm_in_kernel, scale)
    w.state_pool, w.num_slots = _ptr(initial_state), initial_state.shape[0]
    w.state_indices = _ptr(initial_state_indices)
    if snapshots is not None:
        w.snapshots, w.num_snapshot_slots = _ptr(snapshots), snapshots.shape[0]
        w.snapshot_indices = _ptr(snapshot_indices)
    return w


def verify(mixed_qkv, a, b, *, N, H, HV, K, V, scale, conv_weight, conv_state,
           initial_state, initial_state_indices, snapshots, conv_bias=None,
           conv_state_indices=None, parents=None, activation="silu",
           snapshot_indices=None, A_log=None, dt_bias=None, lower_bound=None,
           beta_is_raw=True, use_qk_l2norm_in_kernel=True, o=None, stream=None):
    """kda_verify.  mixed_qkv [B*N, 2HK+HV*V] pre-conv; conv_weight [C, W];
    conv_state [slots, C, W-1]; snapshots [snap_slots, N, HV, V, K] float32
    (written), or None for outputs only (commit then by commit_replay); the
    pool is read only.  Returns o [B*N, HV, V]."""
    torch = _torch()
    if o is None:
        with _on_stream(stream):
            o = torch.empty(mixed_qkv.shape[0], HV, V, dtype=mixed_qkv.dtype, device=mixed_qkv.device)
    w = _verify_args(mixed_qkv, a, b, o, N=N, H=H, HV=HV, K=K, V=V, scale=scale, conv_weight=conv_weight,
                     conv_state=conv_state, initial_state=initial_state,
                     initial_state_indices=initial_state_indices, snapshots=snapshots, conv_bias=conv_bias,
                     conv_state_indices=conv_state_indices, parents=parents, activation=activation,
                     snapshot_indices=snapshot_indices, A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound,
                     beta_is_raw=beta_is_raw, use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel)
    _check(lib().kda_verify(ctypes.byref(w), _stream(stream)))
    return o


def conv_update(x, *, conv_weight, conv_state, conv_state_indices, conv_bias=None,
                activation="silu", y=None, stream=None):
    """kda_conv_update.  x [B, C] pre-conv (one token per request);
    conv_weight [C, W]; conv_state [slots, C, W-1] (updated in place);
    conv_state_indices int32 [B].  Returns y [B, C] post-conv (y may be x)."""
    torch = _torch()
    if y is None:
        with _on_stream(stream):
            y = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    _same_dtype(x, ("y", y), ("conv_weight", conv_weight), ("conv_bias", conv_bias), ("conv_state", conv_state))
    _inner_contig(x, "x")
    _inner_contig(y, "y")
    for name, t in (("conv_weight", conv_weight), ("conv_bias", conv_bias), ("conv_state", conv_state)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _i32_opt(conv_state_indices, "conv_state_indices")
    c = ConvUpdateArgs()
    c.struct_size = ctypes.sizeof(ConvUpdateArgs)
    c.dtype = _dtype_code(x)
    c.B, c.conv_dim = x.shape
    c.conv_width = conv_weight.shape[1]
    c.conv_activation = KDA_ACT_SILU if activation == "silu" else KDA_ACT_NONE
    c.x, c.x_stride = _ptr(x), x.stride(0)
    c.y, c.y_stride = _ptr(y), y.stride(0)
    c.conv_weight, c.conv_bias = _ptr(conv_weight), _ptr(conv_bias)
    c.conv_state, c.num_conv_slots = _ptr(conv_state), conv_state.shape[0]
    c.conv_state_indices = _ptr(conv_state_indices)
    _check(lib().kda_conv_update(ctypes.byref(c), _stream(stream)))
    return y


def commit_replay(accepted, mixed_qkv, a, b, *, N, H, HV, K, V, scale, conv_weight, conv_state,
                  initial_state, initial_state_indices, conv_bias=None, conv_state_indices=None,
                  parents=None, activation="silu", A_log=None, dt_bias=None, lower_bound=None,
                  beta_is_raw=True, use_qk_l2norm_in_kernel=True, stream=None):
    """kda_commit_replay.  The arguments of the preceding verify call (its
    snapshots and output aside) and accepted int32 [B] (last accepted node
    or -1).  Updates initial_state and conv_state in place."""
    _i32_opt(accepted, "accepted")
    if accepted is None or accepted.shape[0] * N != mixed_qkv.shape[0]:
        raise ValueError("accepted must be int32 [B] with B*N == mixed_qkv rows")
    w = _verify_args(mixed_qkv, a, b, None, N=N, H=H, HV=HV, K=K, V=V, scale=scale, conv_weight=conv_weight,
                     conv_state=conv_state, initial_state=initial_state,
                     initial_state_indices=initial_state_indices, snapshots=None, conv_bias=conv_bias,
                     conv_state_indices=conv_state_indices, parents=parents, activation=activation,
                     snapshot_indices=None, A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound,
                     beta_is_raw=beta_is_raw, use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel)
    _check(lib().kda_commit_replay(ctypes.byref(w), _ptr(accepted), _stream(stream)))


def commit(accepted, *, N, snapshots, initial_state, initial_state_indices,
           conv_state=None, mixed_qkv=None, parents=None, snapshot_indices=None,
           conv_state_indices=None, stream=None):
    """kda_commit.  accepted int32 [B] (last accepted node or -1).  Updates
    initial_state (and conv_state, when given) in place."""
    c = CommitArgs()
    c.struct_size = ctypes.sizeof(CommitArgs)
    for name, t in (("accepted", accepted), ("parents", parents), ("initial_state_indices", initial_state_indices),
                    ("snapshot_indices", snapshot_indices), ("conv_state_indices", conv_state_indices)):
        _i32_opt(t, name)
    _f32_opt(snapshots, "snapshots")
    _f32_opt(initial_state, "initial_state")
    c.B, c.N = accepted.shape[0], N
    c.HV, c.V, c.K = snapshots.shape[2], snapshots.shape[3], snapshots.shape[4]
    c.accepted, c.parents = _ptr(accepted), _ptr(parents)
    c.snapshots, c.num_snapshot_slots = _ptr(snapshots), snapshots.shape[0]
    c.snapshot_indices = _ptr(snapshot_indices)
    c.state_pool, c.num_slots = _ptr(initial_state), initial_state.shape[0]
    c.state_indices = _ptr(initial_state_indices)
    if conv_state is not None:
        if mixed_qkv is None:
            raise ValueError("mixed_qkv is required to roll the conv state")
        if not conv_state.is_contiguous():
            raise ValueError("conv_state must be contiguous")
        _same_dtype(mixed_qkv, ("conv_state", conv_state))
        _inner_contig(mixed_qkv, "mixed_qkv")
        c.dtype = _dtype_code(mixed_qkv)
        c.conv_dim, c.conv_width = conv_state.shape[1], conv_state.shape[2] + 1
        c.conv_state, c.num_conv_slots = _ptr(conv_state), conv_state.shape[0]
        c.conv_state_indices = _ptr(conv_state_indices)
        c.mixed_qkv, c.mixed_stride = _ptr(mixed_qkv), mixed_qkv.stride(0)
    _check(lib().kda_commit(ctypes.byref(c), _stream(stream)))
