"""CPU oracle for the bounded-decay gated delta rule (ctypes over gdn_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this package.  The library under
gated_delta_rule_linear_amd/ never imports it, and it imports nothing from
there.

Every function takes and returns numpy arrays in host memory with the packed
layouts q, k, g [T, H, dk]; v, o [T, H, dv]; beta [T, H]; states
[num_seqs, H, dk, dv]; cu_seqlens [num_seqs + 1] (int32).  Inputs are
converted exactly to the function's float type (a bf16 or fp32 input upcasts
without rounding).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_SRC_BWD = os.path.join(_HERE, "gdn_oracle_backward.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
# With GDN_HOST_SANITIZE=1 the oracle is the AddressSanitizer + UndefinedBehavior-
# Sanitizer build (clang, the runtime of the sanitized libgdn build; see
# tests/run_host_sanitizers.sh).
_SAN_PATH = os.path.join(_HERE, "libgdn_oracle_hostsan.so")
CLANG = "/opt/rocm/llvm/bin/clang"
_lib = None


def _sanitized() -> bool:
    return os.environ.get("GDN_HOST_SANITIZE") == "1"


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile gdn_oracle.c and gdn_oracle_backward.c with gcc into
    oracle/libgdn_oracle.so (sanitize: with clang, AddressSanitizer and
    UndefinedBehaviorSanitizer, into oracle/libgdn_oracle_hostsan.so)."""
    path = _SAN_PATH if sanitize else _LIB_PATH
    if force or not os.path.exists(path):
        tmp = path + f".tmp{os.getpid()}"
        if sanitize:
            cmd = [CLANG, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=undefined", "-shared-libsan", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                   "-Wall", "-Wextra", "-o", tmp, _SRC, _SRC_BWD, "-lm"]
        else:
            cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                   "-Wall", "-Wextra", "-o", tmp, _SRC, _SRC_BWD, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _SAN_PATH if _sanitized() else _LIB_PATH
    if not os.path.exists(path):
        build(force=False, sanitize=_sanitized())
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.gdn_oracle_recurrent_f64.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, P, P, i32]
    lib.gdn_oracle_recurrent_f32.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, P, P, i32]
    lib.gdn_oracle_chunked_f64.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P, i32]
    lib.gdn_oracle_bruteforce_f64.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, P, P]
    lib.gdn_oracle_backward_f64.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, P, P, i32, P, P, P, P, P, P,
                                            i32]
    for f in (lib.gdn_oracle_recurrent_f64, lib.gdn_oracle_recurrent_f32, lib.gdn_oracle_chunked_f64,
              lib.gdn_oracle_bruteforce_f64, lib.gdn_oracle_backward_f64):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _as(x, dt):
    return np.ascontiguousarray(np.asarray(x), dtype=dt)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(q, k, v, g, beta, cu_seqlens, initial_state, dt):
    q, k, v, g, beta = (_as(x, dt) for x in (q, k, v, g, beta))
    cu = _as(cu_seqlens, np.int32)
    T, H, dk = q.shape
    dv = v.shape[2]
    n = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk) and v.shape == (T, H, dv)
    assert beta.shape == (T, H) and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    S0 = None if initial_state is None else _as(initial_state, dt)
    if S0 is not None:
        assert S0.shape == (n, H, dk, dv)
    return q, k, v, g, beta, cu, S0, T, H, dk, dv, n


def recurrent(q, k, v, g, beta, cu_seqlens, initial_state=None, dtype=np.float64, threads=None):
    """Token-by-token recurrence. Returns (o [T,H,dv], final_state [N,H,dk,dv])."""
    dt = np.dtype(dtype)
    q, k, v, g, beta, cu, S0, T, H, dk, dv, n = _prep(q, k, v, g, beta, cu_seqlens, initial_state, dt)
    o = np.zeros((T, H, dv), dt)
    Sf = np.zeros((n, H, dk, dv), dt)
    if threads is None:
        threads = min(os.cpu_count() or 1, max(1, n * H))
    if dt not in (np.float64, np.float32):
        raise ValueError("dtype must be float64 or float32")
    fn = _load().gdn_oracle_recurrent_f64 if dt == np.float64 else _load().gdn_oracle_recurrent_f32
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), n, H, dk, dv, _ptr(S0), _ptr(o),
            _ptr(Sf), int(threads))
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return o, Sf


def chunked(q, k, v, g, beta, cu_seqlens, initial_state=None, chunk=64, threads=None):
    """Chunk-by-chunk fp64 form (local cumulative decay + triangular solve)."""
    q, k, v, g, beta, cu, S0, T, H, dk, dv, n = _prep(q, k, v, g, beta, cu_seqlens, initial_state, np.float64)
    o = np.zeros((T, H, dv))
    Sf = np.zeros((n, H, dk, dv))
    if threads is None:
        threads = min(os.cpu_count() or 1, max(1, n * H))
    rc = _load().gdn_oracle_chunked_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), n, H, dk, dv,
                                        int(chunk), _ptr(S0), _ptr(o), _ptr(Sf), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle chunked form failed ({rc})")
    return o, Sf


def bruteforce(q, k, v, g, beta, cu_seqlens, initial_state=None):
    """Explicit unrolled sums for sequences of at most 16 tokens (fp64)."""
    q, k, v, g, beta, cu, S0, T, H, dk, dv, n = _prep(q, k, v, g, beta, cu_seqlens, initial_state, np.float64)
    o = np.zeros((T, H, dv))
    Sf = np.zeros((n, H, dk, dv))
    rc = _load().gdn_oracle_bruteforce_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), n, H, dk, dv,
                                           _ptr(S0), _ptr(o), _ptr(Sf))
    if rc != 0:
        raise RuntimeError(f"oracle brute force failed ({rc})")
    return o, Sf


def backward(q, k, v, g, beta, cu_seqlens, d_o, initial_state=None, d_final_state=None, interval=64,
             threads=None):
    """Gradients of a loss with the given dL/do [T,H,dv] and dL/d(final state)
    [N,H,dk,dv] (None: zero), in fp64, by the reverse-mode recurrence of
    gdn_oracle_backward.c.  Returns a dict with dq, dk, dg [T,H,dk], dv
    [T,H,dv], dbeta [T,H] and d_initial_state [N,H,dk,dv]."""
    q, k, v, g, beta, cu, S0, T, H, dk, dv, n = _prep(q, k, v, g, beta, cu_seqlens, initial_state, np.float64)
    dO = _as(d_o, np.float64)
    assert dO.shape == (T, H, dv)
    dSf = None if d_final_state is None else _as(d_final_state, np.float64)
    if dSf is not None:
        assert dSf.shape == (n, H, dk, dv)
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)), dg=np.zeros((T, H, dk)),
               dbeta=np.zeros((T, H)), d_initial_state=np.zeros((n, H, dk, dv)))
    if threads is None:
        threads = min(os.cpu_count() or 1, max(1, n * H))
    rc = _load().gdn_oracle_backward_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), n, H, dk, dv,
                                         _ptr(S0), _ptr(dO), _ptr(dSf), int(interval), _ptr(out["dq"]),
                                         _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                                         _ptr(out["d_initial_state"]), int(threads))
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return out


def decode_step(q, k, v, g, beta, state, dtype=np.float64, threads=None):
    """One token per sequence ([N,H,*] inputs) from `state` [N,H,dk,dv]: returns (o, new_state)."""
    N = np.asarray(q).shape[0]
    cu = np.arange(N + 1, dtype=np.int32)
    return recurrent(q, k, v, g, beta, cu, initial_state=state, dtype=dtype, threads=threads)


# Gate parameterisations computed from logits (the values of gdn_gate).
GATE_SCALED_SIGMOID = 1
GATE_ALPHA_MIN = 2


def sigmoid(z):
    """1 / (1 + e^-z) in fp64, without overflow for large |z|."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gates_from_logits(z, gate, p):
    """The log-decay g from logits z, in fp64.

    GATE_SCALED_SIGMOID: g = p * sigmoid(z) with p = g_min -- the lower-bounded
    scaled-sigmoid decay of "Trillion-Parameter MoE Multimodal LLMs: How to
    Evaluate the New Generation", section 3.1, eq. 1 (g_min = -5 there).
    GATE_ALPHA_MIN: g = log(p + (1 - p) * sigmoid(z)) with p = a_min, the
    decay factor alpha = e^g bounded below by a_min.
    """
    s = sigmoid(z)
    if gate == GATE_SCALED_SIGMOID:
        return float(p) * s
    if gate == GATE_ALPHA_MIN:
        return np.log(float(p) + (1.0 - float(p)) * s)
    raise ValueError(f"unknown gate {gate!r}")


def rel_err(x, ref) -> float:
    """max|x - ref| / max|ref| over the whole tensor, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den
