"""Shared pieces of the GPU parity tests: run the library and the oracle on the
same seeded inputs and compare with max|x - ref| / max|ref| per tensor."""

import os
import sys

import numpy as np
import torch

import oracle

# Tolerances of the comparison: fp32 inputs are held to 1e-4 and bf16 inputs to
# 2e-2 (bf16 operands carry 8 significant bits; the fp32 path rounds nothing
# below fp32).
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def to_device(x, device="cuda"):
    """Copy a PrefillInputs to the device (in place of the CPU tensors)."""
    for name in ("q", "k", "v", "g", "beta", "cu_seqlens", "initial_state", "z"):
        t = getattr(x, name)
        if t is not None:
            setattr(x, name, t.to(device).contiguous())
    return x


def oracle_prefill(x, units=None, gate=None):
    """fp64 oracle for the inputs in x (tensors anywhere).  With `units` a list of
    (sequence, head) pairs, only those are computed: returns dict {(n, h): (o, S)}.
    With gate = (kind, p) the log-decay is the oracle's parameterisation of the
    bf16 logits x.z instead of x.g; a 2-D x.g is one gate per (token, head)."""
    cu = x.cu_seqlens.cpu().numpy().astype(np.int32)
    dk = x.q.shape[2]
    if gate:
        gof = lambda a: oracle.gates_from_logits(a(x.z), *gate)
    elif x.g.dim() == 2:  # one gate per (token, head): the same decay on every key channel
        gof = lambda a: np.repeat(a(x.g)[:, :, None], dk, axis=2)
    else:
        gof = lambda a: a(x.g)
    if units is None:
        o, S = oracle.recurrent(np64(x.q), np64(x.k), np64(x.v), gof(np64), np64(x.beta), cu,
                                initial_state=None if x.initial_state is None else np64(x.initial_state))
        return o, S
    res = {}
    for n, h in units:
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda t: np64(t[a:b, h:h + 1])
        S0 = None if x.initial_state is None else np64(x.initial_state[n:n + 1, h:h + 1])
        o, S = oracle.recurrent(sl(x.q), sl(x.k), sl(x.v), gof(sl), np64(x.beta[a:b, h:h + 1]),
                                np.array([0, b - a], np.int32), initial_state=S0)
        res[(n, h)] = (o[:, 0], S[0, 0])
    return res


def rel(x, ref):
    return oracle.rel_err(x, ref)


def assert_close(name, x, ref, tol):
    e = rel(x, ref)
    log(f"  {name}: rel err {e:.3e} (tol {tol:.0e})")
    assert np.isfinite(e) and e <= tol, f"{name}: rel err {e:.3e} > {tol}"
    return e
