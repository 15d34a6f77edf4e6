"""Thin ctypes binding of libgdn.so: argument marshalling only.

Every step of the scan runs in the HIP kernels behind the C ABI (include/gdn.h).
PyTorch provides device memory and the current HIP stream; nothing here
computes any part of the method, and there is no fallback: if libgdn.so is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = 0, 1, 2, 3
GDN_DTYPE_F32, GDN_DTYPE_BF16 = 0, 1
GDN_HEADS_TILED, GDN_HEADS_GROUPED = 0, 1
GDN_STATE_F32, GDN_STATE_F16, GDN_STATE_BF16 = 0, 1, 2
GDN_OUT_F32, GDN_OUT_F16 = 0, 1
ABI_VERSION = 7
# GDN_STATIC_SCRATCH_BYTES: the largest workspace_bytes of gdn_prefill_static
STATIC_SCRATCH_BYTES = 96 << 20
_STATE_DTYPES = {torch.float32: GDN_STATE_F32, torch.float16: GDN_STATE_F16, torch.bfloat16: GDN_STATE_BF16}
_OUT_DTYPES = {torch.float32: GDN_OUT_F32, torch.float16: GDN_OUT_F16}

EXPORTED_SYMBOLS = ("gdn_prefill_workspace_bytes", "gdn_prefill_segments", "gdn_prefill", "gdn_prefill_static",
                    "gdn_prefill_varlen_workspace_bytes",
                    "gdn_prefill_varlen", "gdn_decode", "gdn_kda_prefill", "gdn_kda_decode",
                    "gdn_gated_rmsnorm", "gdn_qkv_prologue", "gdn_status_string", "gdn_last_error",
                    "gdn_abi_version")


class GdnShape(ctypes.Structure):
    """Mirror of gdn_shape in include/gdn.h."""
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("qkv_dtype", ctypes.c_int),
                ("head_map", ctypes.c_int), ("scale", ctypes.c_float), ("state_dtype", ctypes.c_int),
                ("o_dtype", ctypes.c_int)]


class GdnNorm(ctypes.Structure):
    """Mirror of gdn_norm in include/gdn.h (the optional output norm of prefill and decode)."""
    _fields_ = [("weight", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("eps", ctypes.c_float)]


class GdnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"gdn status {status}: {detail}")
        self.status = status
        self.detail = detail


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libgdn.so (torch is imported first so both share one HIP runtime)."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m gated_delta_rule_56_amd.build`")
    lib = ctypes.CDLL(path)
    P, SZ = ctypes.c_void_p, ctypes.c_size_t
    lib.gdn_prefill_workspace_bytes.restype = SZ
    lib.gdn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(GdnShape)]
    lib.gdn_prefill_segments.restype = ctypes.c_int
    lib.gdn_prefill_segments.argtypes = [ctypes.POINTER(GdnShape), SZ]
    lib.gdn_prefill.restype = ctypes.c_int
    lib.gdn_prefill.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P, P, SZ, ctypes.POINTER(GdnNorm), P]
    lib.gdn_prefill_static.restype = ctypes.c_int
    lib.gdn_prefill_static.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P, SZ, ctypes.POINTER(GdnNorm), P]
    lib.gdn_prefill_varlen_workspace_bytes.restype = SZ
    lib.gdn_prefill_varlen_workspace_bytes.argtypes = [ctypes.POINTER(GdnShape)]
    lib.gdn_prefill_varlen.restype = ctypes.c_int
    lib.gdn_prefill_varlen.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.gdn_kda_prefill.restype = ctypes.c_int
    lib.gdn_kda_prefill.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P, P, SZ, P]
    lib.gdn_kda_decode.restype = ctypes.c_int
    lib.gdn_kda_decode.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P]
    lib.gdn_decode.restype = ctypes.c_int
    lib.gdn_decode.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, ctypes.POINTER(GdnNorm), P]
    lib.gdn_gated_rmsnorm.restype = ctypes.c_int
    lib.gdn_gated_rmsnorm.argtypes = [ctypes.POINTER(GdnShape), P, P, P, ctypes.c_float, P]
    lib.gdn_qkv_prologue.restype = ctypes.c_int
    lib.gdn_qkv_prologue.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, ctypes.c_float, P]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_abi_version.restype = ctypes.c_int
    lib.gdn_abi_version.argtypes = []
    if lib.gdn_abi_version() != ABI_VERSION:  # the structures above would not match the library's
        raise ImportError(f"{path} has ABI version {lib.gdn_abi_version()}, this binding needs {ABI_VERSION}; "
                          "rebuild it")
    if path == LIBRARY:
        _lib = lib
    return lib


def _check(lib, status: int) -> None:
    if status != GDN_OK:
        raise GdnError(status, lib.gdn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev_tensor(t: torch.Tensor, name: str, dtype: torch.dtype) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream_handle(stream) -> Optional[int]:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _norm_arg(weight: Optional[torch.Tensor], gate: Optional[torch.Tensor], eps: float, o_shape, dtype: torch.dtype,
              d: int):
    """The gdn_norm argument (None without a weight): weight [d] float32, gate of o's shape in
    the q/k/v dtype or None."""
    if weight is None:
        if gate is not None:
            raise ValueError("norm_gate needs norm_weight")
        return None
    _dev_tensor(weight, "norm_weight", torch.float32)
    if tuple(weight.shape) != (d,):
        raise ValueError(f"norm_weight must be [{d}]")
    if gate is not None:
        _dev_tensor(gate, "norm_gate", dtype)
        if tuple(gate.shape) != tuple(o_shape):
            raise ValueError(f"norm_gate must have o's shape {tuple(o_shape)}")
    return GdnNorm(weight.data_ptr(), gate.data_ptr() if gate is not None else None, float(eps))


def _norm_ref(n: Optional[GdnNorm]):
    return ctypes.byref(n) if n is not None else None


def _scratch(nbytes: int, device, stream) -> torch.Tensor:
    """A workspace for one call, allocated on the stream the call runs on: the caching
    allocator hands a freed block out again only to work ordered after it on that stream."""
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream(device)):
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def make_shape(batch, seq_len, num_k_heads, num_v_heads, head_dim, chunk, qkv_dtype, head_map, scale,
               state_dtype=GDN_STATE_F32, o_dtype=GDN_OUT_F32):
    return GdnShape(batch, seq_len, num_k_heads, num_v_heads, head_dim, head_dim, chunk,
                    qkv_dtype, head_map, float(scale), state_dtype, o_dtype)


def _out_tensor(o: Optional[torch.Tensor], shape, o_dtype: torch.dtype, device) -> torch.Tensor:
    """The output tensor: o as passed (float32 or float16, of the given shape), else a new one."""
    if o is None:
        if o_dtype not in _OUT_DTYPES:
            raise TypeError("o_dtype must be torch.float32 or torch.float16")
        o = torch.empty(shape, dtype=o_dtype, device=device)
    if not isinstance(o, torch.Tensor) or o.dtype not in _OUT_DTYPES:
        raise TypeError("o must be a float32 or float16 tensor")
    _dev_tensor(o, "o", o.dtype)
    if tuple(o.shape) != tuple(shape):
        raise ValueError(f"o must be {list(shape)}")
    return o


def _state_tensor(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype not in _STATE_DTYPES:
        raise TypeError(f"{name} must be a float32, float16 or bfloat16 tensor")
    return _dev_tensor(t, name, t.dtype)


def _prefill_shape(batch, seq_len, num_k_heads, num_v_heads, head_dim, chunk, dtype, head_map):
    return make_shape(batch, seq_len, num_k_heads, num_v_heads, head_dim, chunk,
                      GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32, head_map, 1.0)


def prefill_workspace_bytes(batch: int, seq_len: int, num_k_heads: int, num_v_heads: int, head_dim: int, *,
                            chunk: int = 64, dtype: torch.dtype = torch.bfloat16,
                            head_map: int = GDN_HEADS_TILED) -> int:
    """gdn_prefill_workspace_bytes: the workspace of the preferred segment count (0: none used)."""
    shape = _prefill_shape(batch, seq_len, num_k_heads, num_v_heads, head_dim, chunk, dtype, head_map)
    return int(load_library().gdn_prefill_workspace_bytes(ctypes.byref(shape)))


def prefill_segments(batch: int, seq_len: int, num_k_heads: int, num_v_heads: int, head_dim: int,
                     workspace_bytes: int, *, chunk: int = 64, dtype: torch.dtype = torch.bfloat16,
                     head_map: int = GDN_HEADS_TILED) -> int:
    """gdn_prefill_segments: the segment count a prefill of this shape runs with this workspace."""
    shape = _prefill_shape(batch, seq_len, num_k_heads, num_v_heads, head_dim, chunk, dtype, head_map)
    return int(load_library().gdn_prefill_segments(ctypes.byref(shape), int(workspace_bytes)))


def _prefill_marshal(q, k, v, g, beta, initial_state, chunk, head_map, scale, o, final_state, write_final_state,
                     state_dtype, o_dtype, norm_weight, norm_gate, norm_eps):
    """Checks and shapes the arguments of gdn_prefill / gdn_prefill_static: returns
    (lib, shape, o, final_state, norm)."""
    lib = load_library()
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, nm, dtype)
    _dev_tensor(g, "g", torch.float32)
    _dev_tensor(beta, "beta", torch.float32)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4:
        raise ValueError("q, k must be [B][Hk][T][d] and v [B][Hv][T][d]")
    B, Hk, T, d = q.shape
    Hv = v.shape[1]
    if v.shape != (B, Hv, T, d) or g.shape != (B, Hv, T) or beta.shape != (B, Hv, T):
        raise ValueError("v must be [B][Hv][T][d] and g, beta [B][Hv][T]")
    given = [t.dtype for t in (initial_state, final_state) if t is not None]
    if given and state_dtype is not None and state_dtype != given[0]:
        raise TypeError(f"state_dtype {state_dtype} differs from the state tensors' {given[0]}")
    sdt = given[0] if given else (state_dtype or torch.float32)
    if sdt not in _STATE_DTYPES or any(t != sdt for t in given):
        raise TypeError("the states must be float32, float16 or bfloat16, both of the same type")
    if initial_state is not None:
        _state_tensor(initial_state, "initial_state")
        if initial_state.shape != (B, Hv, d, d):
            raise ValueError("initial_state must be [B][Hv][d][d]")
    o = _out_tensor(o, (B, Hv, T, d), o_dtype, q.device)
    if final_state is None and write_final_state:
        final_state = torch.empty((B, Hv, d, d), dtype=sdt, device=q.device)
    if final_state is not None:
        _state_tensor(final_state, "final_state")
        if final_state.shape != (B, Hv, d, d):
            raise ValueError("final_state must be [B][Hv][d][d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shape = make_shape(B, T, Hk, Hv, d, chunk,
                       GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32, head_map, scale,
                       _STATE_DTYPES[sdt], _OUT_DTYPES[o.dtype])
    norm = _norm_arg(norm_weight, norm_gate, norm_eps, (B, Hv, T, d), dtype, d)
    return lib, shape, o, final_state, norm


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
            initial_state: Optional[torch.Tensor] = None, *, chunk: int = 64, head_map: int = GDN_HEADS_TILED,
            scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
            final_state: Optional[torch.Tensor] = None, write_final_state: bool = True,
            workspace: Optional[torch.Tensor] = None, state_dtype: Optional[torch.dtype] = None,
            o_dtype: torch.dtype = torch.float32, norm_weight: Optional[torch.Tensor] = None,
            norm_gate: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gdn_prefill on torch tensors.

    q, k [B][Hk][T][d] and v [B][Hv][T][d] (bfloat16 or float32); g, beta [B][Hv][T] float32;
    initial_state [B][Hv][d][d] float32, float16 or bfloat16, or None. Returns (o, final_state). Pass
    final_state=initial_state to update a state in place. The states share one storage type:
    that of the state tensors passed, else state_dtype (default float32). o is float32, or
    float16 (o_dtype, or the type of the o passed). workspace: a uint8 device tensor of at
    any size (prefill_workspace_bytes(...) gives the preferred one; less means fewer segments of
    the sequence run in parallel, see prefill_segments), or None to allocate the preferred size
    for this call. norm_weight [d] float32 (and optionally norm_gate, o's shape in the q/k/v
    dtype) applies the gated RMSNorm to every output row before it is stored (gdn_norm).
    """
    lib, shape, o, final_state, norm = _prefill_marshal(q, k, v, g, beta, initial_state, chunk, head_map, scale, o,
                                                        final_state, write_final_state, state_dtype, o_dtype,
                                                        norm_weight, norm_gate, norm_eps)
    ws = lib.gdn_prefill_workspace_bytes(ctypes.byref(shape))
    if workspace is None:
        workspace = _scratch(ws, q.device, stream) if ws else None
    else:
        _dev_tensor(workspace, "workspace", torch.uint8)
        ws = workspace.numel()  # a smaller workspace than preferred means fewer segments
    _check(lib, lib.gdn_prefill(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(workspace), ws,
                                _norm_ref(norm), _stream_handle(stream)))
    return o, final_state


def prefill_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                   initial_state: Optional[torch.Tensor] = None, *, chunk: int = 64,
                   head_map: int = GDN_HEADS_TILED, scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
                   final_state: Optional[torch.Tensor] = None, write_final_state: bool = True,
                   workspace_bytes: Optional[int] = None, state_dtype: Optional[torch.dtype] = None,
                   o_dtype: torch.dtype = torch.float32, norm_weight: Optional[torch.Tensor] = None,
                   norm_gate: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gdn_prefill_static on torch tensors: prefill() with the library's static device scratch
    as the workspace, workspace_bytes of it (None: the preferred size; at most
    STATIC_SCRATCH_BYTES). The library call allocates nothing; pass o (and final_state, or
    write_final_state=False) to keep this wrapper from allocating them."""
    lib, shape, o, final_state, norm = _prefill_marshal(q, k, v, g, beta, initial_state, chunk, head_map, scale, o,
                                                        final_state, write_final_state, state_dtype, o_dtype,
                                                        norm_weight, norm_gate, norm_eps)
    if workspace_bytes is None:
        workspace_bytes = lib.gdn_prefill_workspace_bytes(ctypes.byref(shape))
    _check(lib, lib.gdn_prefill_static(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(initial_state), _ptr(o), _ptr(final_state), int(workspace_bytes),
                                       _norm_ref(norm), _stream_handle(stream)))
    return o, final_state


def prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                   cu_seqlens: torch.Tensor, initial_state: Optional[torch.Tensor] = None, *, chunk: int = 64,
                   head_map: int = GDN_HEADS_TILED, scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
                   final_state: Optional[torch.Tensor] = None, write_final_state: bool = True,
                   workspace: Optional[torch.Tensor] = None, state_dtype: Optional[torch.dtype] = None,
                   o_dtype: torch.dtype = torch.float32, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gdn_prefill_varlen on torch tensors: B sequences packed along one token axis.

    q, k [Hk][T][d] and v [Hv][T][d] bfloat16; g, beta [Hv][T] float32; cu_seqlens [B + 1]
    int32 on the GPU (0 = cu[0] <= ... <= cu[B] = T); initial_state [B][Hv][d][d] float32 or
    float16, or None. Returns (o [Hv][T][d] float32 or float16 (o_dtype), final_state
    [B][Hv][d][d]).
    """
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, nm, torch.bfloat16)
    _dev_tensor(g, "g", torch.float32)
    _dev_tensor(beta, "beta", torch.float32)
    _dev_tensor(cu_seqlens, "cu_seqlens", torch.int32)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("q, k must be [Hk][T][d], v [Hv][T][d] and cu_seqlens [B + 1]")
    Hk, T, d = q.shape
    Hv = v.shape[0]
    B = cu_seqlens.numel() - 1
    if v.shape != (Hv, T, d) or g.shape != (Hv, T) or beta.shape != (Hv, T):
        raise ValueError("v must be [Hv][T][d] and g, beta [Hv][T]")
    given = [t.dtype for t in (initial_state, final_state) if t is not None]
    if given and state_dtype is not None and state_dtype != given[0]:
        raise TypeError(f"state_dtype {state_dtype} differs from the state tensors' {given[0]}")
    sdt = given[0] if given else (state_dtype or torch.float32)
    if sdt not in _STATE_DTYPES or any(t != sdt for t in given):
        raise TypeError("the states must be float32, float16 or bfloat16, both of the same type")
    if initial_state is not None:
        _state_tensor(initial_state, "initial_state")
        if initial_state.shape != (B, Hv, d, d):
            raise ValueError("initial_state must be [B][Hv][d][d]")
    o = _out_tensor(o, (Hv, T, d), o_dtype, q.device)
    if final_state is None and write_final_state:
        final_state = torch.empty((B, Hv, d, d), dtype=sdt, device=q.device)
    if final_state is not None:
        _state_tensor(final_state, "final_state")
        if final_state.shape != (B, Hv, d, d):
            raise ValueError("final_state must be [B][Hv][d][d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shape = make_shape(B, T, Hk, Hv, d, chunk, GDN_DTYPE_BF16, head_map, scale, _STATE_DTYPES[sdt],
                       _OUT_DTYPES[o.dtype])
    ws = lib.gdn_prefill_varlen_workspace_bytes(ctypes.byref(shape))
    if workspace is None:
        workspace = _scratch(ws, q.device, stream)
    else:
        _dev_tensor(workspace, "workspace", torch.uint8)
    _check(lib, lib.gdn_prefill_varlen(ctypes.byref(shape), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(final_state),
                                       _ptr(workspace), workspace.numel(), _stream_handle(stream)))
    return o, final_state


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
           state: torch.Tensor, *, head_map: int = GDN_HEADS_TILED, scale: Optional[float] = None,
           o: Optional[torch.Tensor] = None, o_dtype: torch.dtype = torch.float32,
           norm_weight: Optional[torch.Tensor] = None, norm_gate: Optional[torch.Tensor] = None,
           norm_eps: float = 1e-6, stream=None) -> torch.Tensor:
    """gdn_decode on torch tensors: q, k [B][Hk][d], v [B][Hv][d], g, beta [B][Hv],
    state [B][Hv][d][d] float32, float16 or bfloat16 (updated in place). Returns o [B][Hv][d] float32 or
    float16 (o_dtype, or the type of the o passed); with norm_weight (and optionally norm_gate
    [B][Hv][d]) the gated RMSNorm of every output row (gdn_norm)."""
    lib = load_library()
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, nm, dtype)
    _dev_tensor(g, "g", torch.float32)
    _dev_tensor(beta, "beta", torch.float32)
    _state_tensor(state, "state")
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3:
        raise ValueError("q, k must be [B][Hk][d] and v [B][Hv][d]")
    B, Hk, d = q.shape
    Hv = v.shape[1]
    if v.shape != (B, Hv, d) or g.shape != (B, Hv) or beta.shape != (B, Hv) or state.shape != (B, Hv, d, d):
        raise ValueError("v [B][Hv][d], g/beta [B][Hv], state [B][Hv][d][d] expected")
    o = _out_tensor(o, (B, Hv, d), o_dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shape = make_shape(B, 1, Hk, Hv, d, 0, GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32,
                       head_map, scale, _STATE_DTYPES[state.dtype], _OUT_DTYPES[o.dtype])
    norm = _norm_arg(norm_weight, norm_gate, norm_eps, (B, Hv, d), dtype, d)
    _check(lib, lib.gdn_decode(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(state), _ptr(o), _norm_ref(norm), _stream_handle(stream)))
    return o


def kda_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                initial_state: Optional[torch.Tensor] = None, *, chunk: int = 32, head_map: int = GDN_HEADS_TILED,
                scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
                final_state: Optional[torch.Tensor] = None, write_final_state: bool = True,
                workspace: Optional[torch.Tensor] = None, state_dtype: Optional[torch.dtype] = None,
                o_dtype: torch.dtype = torch.float32, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gdn_kda_prefill on torch tensors: as ``prefill`` with one log-decay per key channel,
    g [B][Hv][T][dk] float32. bfloat16 with chunk 32 or 64 runs the chunked form (segment-
    parallel within the workspace, None: the preferred size allocated for this call); chunk 16
    or float32 runs token by token."""
    lib = load_library()
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, nm, dtype)
    _dev_tensor(g, "g", torch.float32)
    _dev_tensor(beta, "beta", torch.float32)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4:
        raise ValueError("q, k must be [B][Hk][T][d] and v [B][Hv][T][d]")
    B, Hk, T, d = q.shape
    Hv = v.shape[1]
    if v.shape != (B, Hv, T, d) or g.shape != (B, Hv, T, d) or beta.shape != (B, Hv, T):
        raise ValueError("v must be [B][Hv][T][d], g [B][Hv][T][d] and beta [B][Hv][T]")
    given = [t.dtype for t in (initial_state, final_state) if t is not None]
    sdt = given[0] if given else (state_dtype or torch.float32)
    if sdt not in _STATE_DTYPES or any(t != sdt for t in given):
        raise TypeError("the states must be float32, float16 or bfloat16, both of the same type")
    if initial_state is not None:
        _state_tensor(initial_state, "initial_state")
        if initial_state.shape != (B, Hv, d, d):
            raise ValueError("initial_state must be [B][Hv][d][d]")
    o = _out_tensor(o, (B, Hv, T, d), o_dtype, q.device)
    if final_state is None and write_final_state:
        final_state = torch.empty((B, Hv, d, d), dtype=sdt, device=q.device)
    if final_state is not None:
        _state_tensor(final_state, "final_state")
        if final_state.shape != (B, Hv, d, d):
            raise ValueError("final_state must be [B][Hv][d][d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qdt = GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32
    shape = make_shape(B, T, Hk, Hv, d, chunk, qdt, head_map, scale, _STATE_DTYPES[sdt], _OUT_DTYPES[o.dtype])
    ws = 0
    if dtype == torch.bfloat16 and chunk in (32, 64):
        ws_shape = make_shape(B, T, Hk, Hv, d, 32, qdt, head_map, scale, _STATE_DTYPES[sdt], _OUT_DTYPES[o.dtype])
        ws = lib.gdn_prefill_workspace_bytes(ctypes.byref(ws_shape))
    if workspace is None:
        workspace = _scratch(ws, q.device, stream) if ws else None
    else:
        _dev_tensor(workspace, "workspace", torch.uint8)
        ws = workspace.numel()
    _check(lib, lib.gdn_kda_prefill(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(workspace), ws,
                                    _stream_handle(stream)))
    return o, final_state


def kda_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
               state: torch.Tensor, *, head_map: int = GDN_HEADS_TILED, scale: Optional[float] = None,
               o: Optional[torch.Tensor] = None, o_dtype: torch.dtype = torch.float32, stream=None) -> torch.Tensor:
    """gdn_kda_decode on torch tensors: as ``decode`` with g [B][Hv][d] (one log-decay per key
    channel)."""
    lib = load_library()
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, nm, dtype)
    _dev_tensor(g, "g", torch.float32)
    _dev_tensor(beta, "beta", torch.float32)
    _state_tensor(state, "state")
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3:
        raise ValueError("q, k must be [B][Hk][d] and v [B][Hv][d]")
    B, Hk, d = q.shape
    Hv = v.shape[1]
    if v.shape != (B, Hv, d) or g.shape != (B, Hv, d) or beta.shape != (B, Hv) or state.shape != (B, Hv, d, d):
        raise ValueError("v [B][Hv][d], g [B][Hv][d], beta [B][Hv], state [B][Hv][d][d] expected")
    o = _out_tensor(o, (B, Hv, d), o_dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shape = make_shape(B, 1, Hk, Hv, d, 0, GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32,
                       head_map, scale, _STATE_DTYPES[state.dtype], _OUT_DTYPES[o.dtype])
    _check(lib, lib.gdn_kda_decode(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(state), _ptr(o), _stream_handle(stream)))
    return o


def gated_rmsnorm(o: torch.Tensor, weight: torch.Tensor, gate: Optional[torch.Tensor] = None, *,
                  eps: float = 1e-6, stream=None) -> torch.Tensor:
    """gdn_gated_rmsnorm on torch tensors, in place: every row of the last axis of o
    ([B][Hv][T][dv] from prefill or [B][Hv][dv] from decode, float32 or float16) becomes
    o / sqrt(mean(o^2) + eps) * weight * silu(gate); weight [dv] float32; gate of o's shape in
    bfloat16 or float32, or None for no gate factor. Returns o."""
    lib = load_library()
    if not isinstance(o, torch.Tensor) or o.dtype not in _OUT_DTYPES:
        raise TypeError("o must be a float32 or float16 tensor")
    _dev_tensor(o, "o", o.dtype)
    if o.dim() == 3:
        B, Hv, d = o.shape
        T = 1
    elif o.dim() == 4:
        B, Hv, T, d = o.shape
    else:
        raise ValueError("o must be [B][Hv][T][dv] or [B][Hv][dv]")
    _dev_tensor(weight, "weight", torch.float32)
    if weight.shape != (d,):
        raise ValueError("weight must be [dv]")
    dtype = torch.float32
    if gate is not None:
        dtype = gate.dtype
        if dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("gate must be bfloat16 or float32")
        _dev_tensor(gate, "gate", dtype)
        if gate.shape != o.shape:
            raise ValueError("gate must have the shape of o")
    shape = make_shape(B, T, Hv, Hv, d, 0, GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32,
                       GDN_HEADS_TILED, 1.0, o_dtype=_OUT_DTYPES[o.dtype])
    _check(lib, lib.gdn_gated_rmsnorm(ctypes.byref(shape), _ptr(o), _ptr(gate), _ptr(weight), float(eps),
                                      _stream_handle(stream)))
    return o


def qkv_prologue(x: torch.Tensor, conv_weight: torch.Tensor, conv_state: Optional[torch.Tensor] = None, *,
                 num_k_heads: int, num_v_heads: int, head_dim: int, eps: float = 1e-6,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """gdn_qkv_prologue on torch tensors: x [B][T][(2 Hk + Hv) d] (bfloat16 or float32), conv_weight
    [(2 Hk + Hv) d][4] float32, conv_state [B][3][(2 Hk + Hv) d] float32 (updated in place) or None.
    Returns (q, k, v) in x's dtype: q, k [B][Hk][T][d], v [B][Hv][T][d]."""
    lib = load_library()
    dtype = x.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be bfloat16 or float32")
    _dev_tensor(x, "x", dtype)
    Hk, Hv, d = num_k_heads, num_v_heads, head_dim
    C = (2 * Hk + Hv) * d
    if x.dim() != 3 or x.shape[2] != C:
        raise ValueError("x must be [B][T][(2 Hk + Hv) d]")
    B, T, _ = x.shape
    _dev_tensor(conv_weight, "conv_weight", torch.float32)
    if conv_weight.shape != (C, 4):
        raise ValueError("conv_weight must be [(2 Hk + Hv) d][4]")
    if conv_state is not None:
        _dev_tensor(conv_state, "conv_state", torch.float32)
        if conv_state.shape != (B, 3, C):
            raise ValueError("conv_state must be [B][3][(2 Hk + Hv) d]")
    q = torch.empty((B, Hk, T, d), dtype=dtype, device=x.device)
    k = torch.empty((B, Hk, T, d), dtype=dtype, device=x.device)
    v = torch.empty((B, Hv, T, d), dtype=dtype, device=x.device)
    shape = make_shape(B, T, Hk, Hv, d, 0, GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32,
                       GDN_HEADS_TILED, 1.0)
    _check(lib, lib.gdn_qkv_prologue(ctypes.byref(shape), _ptr(x), _ptr(conv_weight), _ptr(conv_state),
                                     _ptr(q), _ptr(k), _ptr(v), float(eps), _stream_handle(stream)))
    return q, k, v
