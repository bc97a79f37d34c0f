"""Randomised GPU parity: a fixed-seed list of configurations mixing dtype, head
dimensions, head and sequence counts, ragged and empty lengths, the gate forms
(per-channel log-decays of both recipes, bf16 logits, one log-decay per (token,
head)), initial states and the time split (planned, off, or forced segment
lengths), each compared element by element with the fp64 oracle.  Forward and
backward.  The configurations are drawn once, at import, from a seeded
generator, so every run checks the same ones."""

import numpy as np
import pytest
import torch

import gated_delta_rule_linear_amd as gdn
import oracle
from gated_delta_rule_linear_amd import inputs
from helpers import TOL, assert_close, log, np64, oracle_prefill, to_device

pytestmark = pytest.mark.gpu

DIMS = [(128, 128), (64, 64), (64, 128), (128, 64)]


def _lengths(rng, n, hi):
    out = []
    for _ in range(n):
        u = rng.random()
        out.append(0 if u < 0.1 else int(rng.integers(1, 65)) if u < 0.4 else int(rng.integers(65, hi + 1)))
    return out


def _forward_cases(count=60, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        entry = ["prefill", "prefill", "logits", "head_gate"][int(rng.integers(0, 4))]
        # (the logit and per-head gate entry points take bf16 only)
        dtype = torch.bfloat16 if entry in ("logits", "head_gate") or rng.random() < 0.5 else torch.float32
        dk, dv = DIMS[int(rng.integers(0, 4))]
        H = int(rng.integers(1, 7))
        n = int(rng.integers(1, 11))
        cases.append(dict(i=i, entry=entry, dtype=dtype, dk=dk, dv=dv, H=H,
                          lengths=_lengths(rng, n, 700),
                          gate=["amin", "pages"][int(rng.integers(0, 2))],
                          a_min=[0.9, 0.99][int(rng.integers(0, 2))],
                          init=bool(rng.integers(0, 2)),
                          seg=[None, "0", "64", "128", "192"][int(rng.integers(0, 5))],
                          seed=int(rng.integers(0, 1 << 30))))
    return cases


def _backward_cases(count=48, seed=2027):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        dk, dv = DIMS[int(rng.integers(0, 4))]
        cases.append(dict(i=i, dtype=torch.bfloat16 if rng.random() < 0.7 else torch.float32, dk=dk, dv=dv,
                          H=int(rng.integers(1, 5)), lengths=_lengths(rng, int(rng.integers(1, 8)), 300),
                          gate=["amin", "pages"][int(rng.integers(0, 2))], init=bool(rng.integers(0, 2)),
                          final=bool(rng.integers(0, 2)), seg=[None, "0", "64", "128"][int(rng.integers(0, 4))],
                          seed=int(rng.integers(0, 1 << 30))))
    return cases


def _name(c):
    return (f"{c['i']}-{c.get('entry', 'bwd')}-{str(c['dtype'])[6:]}-d{c['dk']}x{c['dv']}-H{c['H']}"
            f"-n{len(c['lengths'])}-{c['gate']}-seg{c['seg']}")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def _segment(monkeypatch, var, seg):
    if seg is None:
        monkeypatch.delenv(var, raising=False)
    else:
        monkeypatch.setenv(var, seg)


@pytest.mark.parametrize("c", _forward_cases(), ids=_name)
def test_random_forward(monkeypatch, c):
    log(f"random forward case {c}")
    _segment(monkeypatch, "GDN_PREFILL_SEGMENT", c["seg"])
    x = inputs.make_prefill_inputs(c["lengths"], c["H"], c["dk"], c["dv"], dtype=c["dtype"], gate=c["gate"],
                                   a_min=c["a_min"], init_state=c["init"], seed=c["seed"],
                                   logits=c["entry"] == "logits", head_gate=c["entry"] == "head_gate")
    if c["entry"] == "logits":
        # the pages' recipe is the scaled sigmoid with g_min = -5; the a_min one its own parameterisation
        kind, p = ((gdn.GDN_GATE_SCALED_SIGMOID, -5.0) if c["gate"] == "pages"
                   else (gdn.GDN_GATE_ALPHA_MIN, c["a_min"]))
        okind = oracle.GATE_SCALED_SIGMOID if c["gate"] == "pages" else oracle.GATE_ALPHA_MIN
        ref_o, ref_S = oracle_prefill(x, gate=(okind, p))
        to_device(x)
        o, S = gdn.gdn_prefill_logits(x.q, x.k, x.v, x.z, kind, p, x.beta, x.cu_seqlens,
                                      initial_state=x.initial_state)
    else:
        ref_o, ref_S = oracle_prefill(x)
        to_device(x)
        call = gdn.gdn_prefill_head_gate if c["entry"] == "head_gate" else gdn.gdn_prefill
        o, S = call(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, TOL[c["dtype"]])
    assert_close("final_state", np64(S), ref_S, TOL[c["dtype"]])


@pytest.mark.parametrize("c", _backward_cases(), ids=_name)
def test_random_backward(monkeypatch, c):
    log(f"random backward case {c}")
    _segment(monkeypatch, "GDN_BACKWARD_SEGMENT", c["seg"])
    H, dk, dv = c["H"], c["dk"], c["dv"]
    x = inputs.make_prefill_inputs(c["lengths"], H, dk, dv, dtype=c["dtype"], gate=c["gate"],
                                   init_state=c["init"], seed=c["seed"])
    d_o, dSf = inputs.make_cotangents(x.T_total, x.num_seqs, H, dk, dv, dtype=c["dtype"], final_state=c["final"],
                                      seed=c["seed"] + 1)
    cu = x.cu_seqlens.cpu().numpy().astype(np.int32)
    ref = oracle.backward(np64(x.q), np64(x.k), np64(x.v), np64(x.g), np64(x.beta), cu, np64(d_o),
                          initial_state=None if x.initial_state is None else np64(x.initial_state),
                          d_final_state=None if dSf is None else np64(dSf))
    to_device(x)
    out = gdn.gdn_prefill_backward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, d_o.cuda(),
                                   initial_state=x.initial_state,
                                   d_final_state=None if dSf is None else dSf.cuda())
    torch.cuda.synchronize()
    for name, got in zip(("dq", "dk", "dv", "dg", "dbeta", "d_initial_state"), out):
        assert_close(name, np64(got), ref[name], TOL[c["dtype"]])
