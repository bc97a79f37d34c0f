"""libgdn: the bounded-decay gated delta rule on MI355X (gfx950).

A thin binding over the C-ABI in include/gdn.h.  The functions carry the C
names and only marshal arguments: PyTorch tensors supply device memory and
the current stream; every step of the computation runs in the HIP kernels of
libgdn.so.  There is no CPU fallback: the first call raises ImportError when
libgdn.so has not been built (python -m gated_delta_rule_linear_amd.build).
The submodule `inputs` (seeded synthetic inputs) does not need the library.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_HOST_SANITIZE=1 loads the build whose host code (validation, planning,
# launch set-up) carries AddressSanitizer and UndefinedBehaviorSanitizer; its
# kernels are the same.  It needs the sanitizer runtime preloaded
# (tests/run_host_sanitizers.sh).
LIB_PATH = os.path.join(_HERE, "libgdn_hostsan.so" if os.environ.get("GDN_HOST_SANITIZE") == "1" else "libgdn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "gdn.h")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_DOMAIN, GDN_ERR_OOM, GDN_ERR_HIP, GDN_ERR_SCRATCH_LIMIT = range(7)
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20
GDN_F32, GDN_BF16 = 0, 1
GDN_GATE_LOG, GDN_GATE_SCALED_SIGMOID, GDN_GATE_ALPHA_MIN = 0, 1, 2
GDN_TILES_DENSE, GDN_TILES_PAIRS = 0, 1


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status} ({gdn_status_string(status)})")
        self.status = status


_LIB = None


def _load():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m gated_delta_rule_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.gdn_status_string.argtypes = [i32]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_state_bytes.argtypes = [i64, i32, i32, i32]
    lib.gdn_state_bytes.restype = sz
    lib.gdn_state_alloc.argtypes = [i64, i32, i32, i32, ctypes.POINTER(P), P]
    lib.gdn_state_alloc.restype = i32
    lib.gdn_state_free.argtypes = [P, P]
    lib.gdn_state_free.restype = i32
    lib.gdn_prefill_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
    lib.gdn_prefill_workspace_bytes.restype = sz
    lib.gdn_prefill.argtypes = [P, P, P, P, P, P, i32, i64, P, P, P, i32, i32, i32, i32, P, sz, P]
    lib.gdn_prefill.restype = i32
    lib.gdn_prefill_maxlen.argtypes = [P, P, P, P, P, P, i32, i64, i64, P, P, P, i32, i32, i32, i32, P, sz, P]
    lib.gdn_prefill_maxlen.restype = i32
    lib.gdn_prefill_workspace_bytes_maxlen.argtypes = [i64, i32, i64, i32, i32, i32]
    lib.gdn_prefill_workspace_bytes_maxlen.restype = sz
    lib.gdn_prefill_noalloc.argtypes = [P, P, P, P, P, P, i32, i64, P, P, P, i32, i32, i32, i32, P]
    lib.gdn_prefill_noalloc.restype = i32
    lib.gdn_decode.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P]
    lib.gdn_decode.restype = i32
    f32 = ctypes.c_float
    lib.gdn_prefill_logits.argtypes = [P, P, P, P, i32, f32, P, P, i32, i64, P, P, P, i32, i32, i32, i32, P, sz, P]
    lib.gdn_prefill_logits.restype = i32
    lib.gdn_decode_logits.argtypes = [P, P, P, P, i32, f32, P, P, P, i32, i32, i32, i32, i32, P]
    lib.gdn_decode_logits.restype = i32
    lib.gdn_prefill_head_gate.argtypes = [P, P, P, P, P, P, i32, i64, P, P, P, i32, i32, i32, i32, P, sz, P]
    lib.gdn_prefill_head_gate.restype = i32
    lib.gdn_decode_head_gate.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P]
    lib.gdn_decode_head_gate.restype = i32
    lib.gdn_prefill_backward_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.gdn_prefill_backward_workspace_bytes.restype = sz
    lib.gdn_prefill_backward.argtypes = [P, P, P, P, P, P, i32, i64, P, P, P, P, P, P, P, P, P, i32, i32, i32, i32,
                                         P, sz, P]
    lib.gdn_prefill_backward.restype = i32
    lib.gdn_prefill_tiles.argtypes = [P, P, P, P, P, P, i32, i64, P, P, P, i32, i32, i32, i32, i32, P]
    lib.gdn_prefill_tiles.restype = i32
    _LIB = lib
    return lib


def load_library():
    """The ctypes handle of libgdn.so (loaded on first use)."""
    return _load()


def exported_symbols_in_header() -> list:
    """Names of the functions include/gdn.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(gdn_[a-z_0-9]+)\s*\(", text, flags=re.M)


def gdn_status_string(status: int) -> str:
    return _load().gdn_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != GDN_OK:
        raise GdnError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> Optional[ctypes.c_void_p]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context for the tensors a call allocates (outputs, workspace): the stream
    the kernels run on.  The caching allocator then gives a block released here
    back only to later work ordered after those kernels on that stream."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None, dims=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions")


def gdn_state_bytes(num_seqs: int, H: int, dk: int, dv: int) -> int:
    return int(_load().gdn_state_bytes(num_seqs, H, dk, dv))


def gdn_prefill_workspace_bytes(T_total: int, num_seqs: int, H: int, dk: int, dv: int, max_seqlen: int = 0) -> int:
    """Scratch bytes of gdn_prefill (max_seqlen > 0: of gdn_prefill with that bound on the lengths)."""
    if max_seqlen:
        return int(_load().gdn_prefill_workspace_bytes_maxlen(T_total, num_seqs, int(max_seqlen), H, dk, dv))
    return int(_load().gdn_prefill_workspace_bytes(T_total, num_seqs, H, dk, dv))


def gdn_state_alloc(num_seqs: int, H: int, dk: int, dv: int, stream=None) -> int:
    """Zero-filled device state [num_seqs, H, dk, dv] fp32; returns the raw device address."""
    out = ctypes.c_void_p()
    _check(_load().gdn_state_alloc(num_seqs, H, dk, dv, ctypes.byref(out), _stream(stream)), "gdn_state_alloc")
    return int(out.value or 0)


def gdn_state_free(address: int, stream=None) -> None:
    _check(_load().gdn_state_free(ctypes.c_void_p(address), _stream(stream)), "gdn_state_free")


def gdn_prefill(q, k, v, g, beta, cu_seqlens, initial_state=None, final_state=None, o=None, workspace=None,
                output_final_state: bool = True, stream=None, max_seqlen: int = 0):
    """Chunked prefill; returns (o, final_state or None).

    q, k [T, H, dk] and v [T, H, dv] in bf16 or fp32; g [T, H, dk] and beta [T, H]
    in fp32; cu_seqlens int32 [num_seqs + 1] on the device.  final_state may be
    initial_state itself (updated in place).  max_seqlen > 0, a host-side bound on
    the sequence lengths, calls gdn_prefill_maxlen (planning for skewed batches)."""
    _need(q, "q", dims=3)
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    _need(g, "g", torch.float32, 3)
    _need(beta, "beta", torch.float32, 2)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    n = cu_seqlens.shape[0] - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
        if initial_state.shape != (n, H, dk, dv):
            raise ValueError("initial_state must be [num_seqs, H, dk, dv]")
    with _on(stream):
        if o is None:
            o = torch.empty((T, H, dv), dtype=dt, device=q.device)
        _need(o, "o", dt, 3)
        if final_state is None and output_final_state:
            final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device)
        if final_state is not None:
            _need(final_state, "final_state", torch.float32, 4)
        need = gdn_prefill_workspace_bytes(T, n, H, dk, dv, max_seqlen)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        if max_seqlen:
            st = _load().gdn_prefill_maxlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), n, T,
                                            int(max_seqlen), _ptr(initial_state), _ptr(final_state), _ptr(o), H, dk,
                                            dv, _dtype_code(q), _ptr(workspace), ws_bytes, _stream(stream))
            _check(st, "gdn_prefill_maxlen")
        else:
            st = _load().gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), n, T,
                                     _ptr(initial_state), _ptr(final_state), _ptr(o), H, dk, dv, _dtype_code(q),
                                     _ptr(workspace), ws_bytes, _stream(stream))
            _check(st, "gdn_prefill")
    return o, final_state


def gdn_prefill_workspace_bytes_maxlen(T_total: int, num_seqs: int, max_seqlen: int, H: int, dk: int, dv: int) -> int:
    return int(_load().gdn_prefill_workspace_bytes_maxlen(T_total, num_seqs, int(max_seqlen), H, dk, dv))


def gdn_prefill_maxlen(q, k, v, g, beta, cu_seqlens, max_seqlen: int, initial_state=None, final_state=None, o=None,
                       workspace=None, output_final_state: bool = True, stream=None):
    """gdn_prefill with a host-side bound max_seqlen on the sequence lengths (see gdn_prefill)."""
    if max_seqlen < 0:
        raise ValueError("max_seqlen must be >= 0")
    return gdn_prefill(q, k, v, g, beta, cu_seqlens, initial_state=initial_state, final_state=final_state, o=o,
                       workspace=workspace, output_final_state=output_final_state, stream=stream,
                       max_seqlen=max_seqlen)


def gdn_prefill_noalloc(q, k, v, g, beta, cu_seqlens, initial_state=None, final_state=None, o=None,
                        output_final_state: bool = True, stream=None):
    """gdn_prefill with its scratch in the library's fixed device array (no
    workspace, no device allocation by the library).  Pass o (and final_state)
    to allocate nothing here either; calls that overlap on one GPU race on the
    shared array."""
    _need(q, "q", dims=3)
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    _need(g, "g", torch.float32, 3)
    _need(beta, "beta", torch.float32, 2)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    n = cu_seqlens.shape[0] - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
        if initial_state.shape != (n, H, dk, dv):
            raise ValueError("initial_state must be [num_seqs, H, dk, dv]")
    with _on(stream):
        if o is None:
            o = torch.empty((T, H, dv), dtype=dt, device=q.device)
        _need(o, "o", dt, 3)
        if final_state is None and output_final_state:
            final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device)
        if final_state is not None:
            _need(final_state, "final_state", torch.float32, 4)
        st = _load().gdn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), n, T,
                                         _ptr(initial_state), _ptr(final_state), _ptr(o), H, dk, dv,
                                         _dtype_code(q), _stream(stream))
        _check(st, "gdn_prefill_noalloc")
    return o, final_state


def gdn_prefill_head_gate(q, k, v, g, beta, cu_seqlens, initial_state=None, final_state=None, o=None, workspace=None,
                          output_final_state: bool = True, stream=None):
    """gdn_prefill with one fp32 log-decay per (token, head): g [T, H]."""
    _need(q, "q", dims=3)
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    _need(g, "g", torch.float32, 2)
    _need(beta, "beta", torch.float32, 2)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    if k.shape != (T, H, dk) or g.shape != (T, H) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    n = cu_seqlens.shape[0] - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
        if initial_state.shape != (n, H, dk, dv):
            raise ValueError("initial_state must be [num_seqs, H, dk, dv]")
    with _on(stream):
        if o is None:
            o = torch.empty((T, H, dv), dtype=dt, device=q.device)
        _need(o, "o", dt, 3)
        if final_state is None and output_final_state:
            final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device)
        if final_state is not None:
            _need(final_state, "final_state", torch.float32, 4)
        need = gdn_prefill_workspace_bytes(T, n, H, dk, dv)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        st = _load().gdn_prefill_head_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), n, T,
                                           _ptr(initial_state), _ptr(final_state), _ptr(o), H, dk, dv, _dtype_code(q),
                                           _ptr(workspace), ws_bytes, _stream(stream))
        _check(st, "gdn_prefill_head_gate")
    return o, final_state


def gdn_decode_head_gate(q, k, v, g, beta, state, o=None, stream=None):
    """gdn_decode with one fp32 log-decay per (sequence, head): g [N, H]."""
    _need(q, "q", dims=3)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    _need(g, "g", torch.float32, 2)
    _need(beta, "beta", torch.float32, 2)
    _need(state, "state", torch.float32, 4)
    if state.shape != (N, H, dk, dv) or k.shape != (N, H, dk) or g.shape != (N, H) or beta.shape != (N, H):
        raise ValueError("inconsistent shapes")
    with _on(stream):
        if o is None:
            o = torch.empty((N, H, dv), dtype=dt, device=q.device)
        _need(o, "o", dt, 3)
        st = _load().gdn_decode_head_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o), N, H,
                                          dk, dv, _dtype_code(q), _stream(stream))
        _check(st, "gdn_decode_head_gate")
    return o


def gdn_prefill_logits(q, k, v, z, gate, gate_param, beta, cu_seqlens, initial_state=None, final_state=None, o=None,
                       workspace=None, output_final_state: bool = True, stream=None):
    """gdn_prefill with bf16 gate logits z [T, H, dk] and a gdn_gate parameterisation
    (GDN_GATE_SCALED_SIGMOID with g_min, or GDN_GATE_ALPHA_MIN with a_min)."""
    _need(q, "q", dims=3)
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    _need(z, "z", torch.bfloat16, 3)
    _need(beta, "beta", torch.float32, 2)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    if k.shape != (T, H, dk) or z.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    n = cu_seqlens.shape[0] - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
        if initial_state.shape != (n, H, dk, dv):
            raise ValueError("initial_state must be [num_seqs, H, dk, dv]")
    with _on(stream):
        if o is None:
            o = torch.empty((T, H, dv), dtype=dt, device=q.device)
        _need(o, "o", dt, 3)
        if final_state is None and output_final_state:
            final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device)
        if final_state is not None:
            _need(final_state, "final_state", torch.float32, 4)
        need = gdn_prefill_workspace_bytes(T, n, H, dk, dv)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        st = _load().gdn_prefill_logits(_ptr(q), _ptr(k), _ptr(v), _ptr(z), int(gate), float(gate_param), _ptr(beta),
                                        _ptr(cu_seqlens), n, T, _ptr(initial_state), _ptr(final_state), _ptr(o), H, dk,
                                        dv, _dtype_code(q), _ptr(workspace), ws_bytes, _stream(stream))
        _check(st, "gdn_prefill_logits")
    return o, final_state


def gdn_decode_logits(q, k, v, z, gate, gate_param, beta, state, o=None, stream=None):
    """gdn_decode with bf16 gate logits z [N, H, dk]; `state` is updated in place."""
    _need(q, "q", dims=3)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    _need(z, "z", torch.bfloat16, 3)
    _need(beta, "beta", torch.float32, 2)
    _need(state, "state", torch.float32, 4)
    if state.shape != (N, H, dk, dv) or k.shape != (N, H, dk) or z.shape != (N, H, dk) or beta.shape != (N, H):
        raise ValueError("inconsistent shapes")
    with _on(stream):
        if o is None:
            o = torch.empty((N, H, dv), dtype=dt, device=q.device)
        _need(o, "o", dt, 3)
        st = _load().gdn_decode_logits(_ptr(q), _ptr(k), _ptr(v), _ptr(z), int(gate), float(gate_param), _ptr(beta),
                                       _ptr(state), _ptr(o), N, H, dk, dv, _dtype_code(q), _stream(stream))
        _check(st, "gdn_decode_logits")
    return o


def gdn_decode(q, k, v, g, beta, state, o=None, stream=None):
    """One token per sequence; `state` [N, H, dk, dv] fp32 is updated in place. Returns o [N, H, dv]."""
    _need(q, "q", dims=3)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    _need(g, "g", torch.float32, 3)
    _need(beta, "beta", torch.float32, 2)
    _need(state, "state", torch.float32, 4)
    if state.shape != (N, H, dk, dv) or k.shape != (N, H, dk) or g.shape != (N, H, dk) or beta.shape != (N, H):
        raise ValueError("inconsistent shapes")
    with _on(stream):
        if o is None:
            o = torch.empty((N, H, dv), dtype=dt, device=q.device)
        _need(o, "o", dt, 3)
        st = _load().gdn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o), N, H, dk, dv,
                            _dtype_code(q), _stream(stream))
        _check(st, "gdn_decode")
    return o


def gdn_prefill_backward_workspace_bytes(T_total: int, num_seqs: int, H: int, dk: int, dv: int, dtype) -> int:
    """Scratch bytes of gdn_prefill_backward (dtype: torch.bfloat16 or torch.float32)."""
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(_load().gdn_prefill_backward_workspace_bytes(int(T_total), int(num_seqs), int(H), int(dk), int(dv),
                                                            code))


def gdn_prefill_backward(q, k, v, g, beta, cu_seqlens, d_o, initial_state=None, d_final_state=None,
                         want_d_initial_state: bool = True, workspace=None, stream=None):
    """Gradients of gdn_prefill: given dL/do [T, H, dv] (and dL/d final state [N, H, dk, dv] fp32, or None
    for zero) returns (dq, dk, dv, dg, dbeta, d_initial_state); dq, dk, dv have the dtype of q, dg and dbeta
    are fp32, d_initial_state is fp32 [N, H, dk, dv] (None when not wanted)."""
    _need(q, "q", dims=3)
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    _need(d_o, "d_o", dt, 3)
    _need(g, "g", torch.float32, 3)
    _need(beta, "beta", torch.float32, 2)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) or d_o.shape != (T, H, dv) \
            or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    n = cu_seqlens.shape[0] - 1
    for name, s in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if s is not None:
            _need(s, name, torch.float32, 4)
            if s.shape != (n, H, dk, dv):
                raise ValueError(f"{name} must be [num_seqs, H, dk, dv]")
    with _on(stream):
        dq = torch.empty_like(q)
        dkk = torch.empty_like(k)
        dvv = torch.empty_like(v)
        dg = torch.empty_like(g)
        db = torch.empty_like(beta)
        dS0 = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device) if want_d_initial_state else None
        need = gdn_prefill_backward_workspace_bytes(T, n, H, dk, dv, dt)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
        st = _load().gdn_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), n, T,
                                          _ptr(initial_state), _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dkk),
                                          _ptr(dvv), _ptr(dg), _ptr(db), _ptr(dS0), H, dk, dv, _dtype_code(q),
                                          _ptr(workspace), ws_bytes, _stream(stream))
        _check(st, "gdn_prefill_backward")
    return dq, dkk, dvv, dg, db, dS0


def gdn_prefill_tiles(q, k, v, g, beta, cu_seqlens, tile_path, initial_state=None, final_state=None, o=None,
                      output_final_state: bool = True, stream=None):
    """Prefill in 16-token windows with the diagonal-tile path GDN_TILES_DENSE (g in [-5, 0]) or
    GDN_TILES_PAIRS (any finite g <= 0).  Returns (o, final_state)."""
    _need(q, "q", dims=3)
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    _need(g, "g", torch.float32, 3)
    _need(beta, "beta", torch.float32, 2)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    n = cu_seqlens.shape[0] - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
        if initial_state.shape != (n, H, dk, dv):
            raise ValueError("initial_state must be [num_seqs, H, dk, dv]")
    with _on(stream):
        if o is None:
            o = torch.empty((T, H, dv), dtype=dt, device=q.device)
        _need(o, "o", dt, 3)
        if final_state is None and output_final_state:
            final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device)
        if final_state is not None:
            _need(final_state, "final_state", torch.float32, 4)
        st = _load().gdn_prefill_tiles(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), n, T,
                                       _ptr(initial_state), _ptr(final_state), _ptr(o), H, dk, dv, _dtype_code(q),
                                       int(tile_path), _stream(stream))
        _check(st, "gdn_prefill_tiles")
    return o, final_state


__all__ = [
    "gdn_status_string", "gdn_state_bytes", "gdn_state_alloc", "gdn_state_free", "gdn_prefill_workspace_bytes",
    "gdn_prefill", "gdn_prefill_maxlen", "gdn_prefill_workspace_bytes_maxlen", "gdn_prefill_noalloc", "gdn_decode", "gdn_prefill_logits", "gdn_decode_logits", "gdn_prefill_head_gate",
    "gdn_decode_head_gate", "gdn_prefill_backward", "gdn_prefill_backward_workspace_bytes", "gdn_prefill_tiles", "GdnError", "load_library", "LIB_PATH",
    "GDN_GATE_LOG", "GDN_GATE_SCALED_SIGMOID", "GDN_GATE_ALPHA_MIN", "GDN_TILES_DENSE", "GDN_TILES_PAIRS",
]
