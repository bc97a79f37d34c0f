"""GPU parity at full workload sizes, in the launch configuration bench.py
times (the split plan the library picks by itself).  The fp64 oracle computes
sampled (sequence, head) units in full — every output token and the final
state of each sampled unit — and the library's result for those units is
compared element by element.  The 2^20-token case is checked on three heads
in full against the fp64 oracle, and on every head against the unsplit
kernel; a skewed batch given without a bound on its lengths, on sampled
units in full and on the long sequence against the bounded plan.  The decode
workload runs all 128 steps over every (sequence, head)
and is compared with the fp64 oracle at every step."""

import os

import numpy as np
import pytest
import torch

import gated_delta_rule_linear_amd as gdn
import oracle
from gated_delta_rule_linear_amd import inputs
from helpers import assert_close, log, np64

pytestmark = pytest.mark.gpu
TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()
    os.environ.pop("GDN_PREFILL_SEGMENT", None)


def _oracle_units(x, units, dtype=np.float64):
    """{(n, h): (o, S)} from the oracle, one call per sequence over its sampled heads."""
    cu = x.cu_seqlens.cpu().numpy()
    by_seq = {}
    for n, h in units:
        by_seq.setdefault(n, []).append(h)
    res = {}
    for n, hs in by_seq.items():
        a, b = int(cu[n]), int(cu[n + 1])
        idx = torch.tensor(hs, device=x.q.device)
        sl = lambda t: t[a:b].index_select(1, idx).to("cpu", torch.float64).numpy()
        S0 = None
        if x.initial_state is not None:
            S0 = x.initial_state[n:n + 1].index_select(1, idx).to("cpu", torch.float64).numpy()
        o, S = oracle.recurrent(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), np.array([0, b - a], np.int32),
                                initial_state=S0, dtype=dtype, threads=min(len(hs), 16))
        for j, h in enumerate(hs):
            res[(n, h)] = (o[:, j], S[0, j])
    return res


def _check_units(x, o, S, units, tol=TOL_BF16):
    cu = x.cu_seqlens.cpu().numpy()
    ref = _oracle_units(x, units)
    for (n, h), (ro, rS) in ref.items():
        a, b = int(cu[n]), int(cu[n + 1])
        assert_close(f"seq {n} head {h}: o", np64(o[a:b, h]), ro, tol)
        assert_close(f"seq {n} head {h}: final state", np64(S[n, h]), rS, tol)


def _run(x):
    T, H, dk = x.q.shape
    dv = x.v.shape[-1]
    n = len(x.lengths)
    ws = gdn.gdn_prefill_workspace_bytes(T, n, H, dk, dv)
    log(f"  T={T} H={H} seqs={n}: workspace {ws} bytes ({'split' if ws else 'whole sequences'})")
    o, S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    return o, S


def test_prefill_64k_as_benchmarked():
    log("prefill_64k: one 65536-token sequence, 32 heads, d 128, bf16")
    x = inputs.make_workload("prefill_64k", seed=0, device="cuda")
    o, S = _run(x)
    _check_units(x, o, S, [(0, 0), (0, 13), (0, 31)])


def test_batch4_t8k():
    log("batch4_t8k: four 8192-token sequences, 32 heads")
    x = inputs.make_workload("batch4_t8k", seed=1, device="cuda")
    o, S = _run(x)
    _check_units(x, o, S, [(0, 0), (1, 7), (2, 20), (3, 31)])


def test_varlen64():
    log("varlen64: 64 sequences of 512..16384 tokens, 32 heads, random initial states")
    x = inputs.make_workload("varlen64", seed=2, device="cuda")
    o, S = _run(x)
    L = x.lengths
    longest, shortest = int(np.argmax(L)), int(np.argmin(L))
    _check_units(x, o, S, [(longest, 3), (shortest, 30), (17, 16), (63, 0)])


@pytest.mark.timeout(600)
def test_skewed64_without_a_bound():
    # 63 sequences of 1,024 tokens and, last, one of 262,144, 32 heads, random initial
    # states: 2,048 units, so sequences of the mean length would need no split, and no
    # bound on the lengths is given; the length-agnostic plan cuts the long sequence
    # into segments of 326,656 / 9 tokens (rounded to 64).  Two heads of the long
    # sequence and two short units in full against the fp64 oracle; the long sequence
    # against gdn_prefill_maxlen's plan on every head.
    log("skewed64 without a bound: 63 x 1024 + 1 x 262144 tokens, 32 heads")
    lens = [1024] * 63 + [262144]
    x = inputs.make_prefill_inputs(lens, 32, 128, 128, dtype=torch.bfloat16, init_state=True, seed=41,
                                   device="cuda")
    T = sum(lens)
    assert gdn.gdn_prefill_workspace_bytes(T, 64, 32, 128, 128) > 9 * 32 * 128 * 128 * 4  # split maps
    o, S = _run(x)
    _check_units(x, o, S, [(63, 0), (63, 31), (0, 5), (62, 17)])
    o2, S2 = gdn.gdn_prefill_maxlen(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, 262144,
                                    initial_state=x.initial_state)
    torch.cuda.synchronize()
    a = T - 262144
    for h in range(32):
        assert_close(f"long sequence head {h}: o vs the bounded plan", np64(o[a:, h]), np64(o2[a:, h]), TOL_BF16)
        assert_close(f"long sequence head {h}: state vs the bounded plan", np64(S[63, h]), np64(S2[63, h]), TOL_BF16)


@pytest.mark.timeout(600)
def test_long_1m():
    log("long_1m: one 2^20-token sequence, 16 heads, a_min 0.99")
    x = inputs.make_workload("long_1m", seed=3, device="cuda")
    o, S = _run(x)
    # every head against the unsplit kernel (one workgroup per head, no time split)
    os.environ["GDN_PREFILL_SEGMENT"] = "0"
    try:
        o1, S1 = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("GDN_PREFILL_SEGMENT", None)
    for h in range(16):
        assert_close(f"head {h}: o split vs unsplit", np64(o[:, h]), np64(o1[:, h]), TOL_BF16)
        assert_close(f"head {h}: state split vs unsplit", np64(S[0, h]), np64(S1[0, h]), TOL_BF16)
    del o1, S1
    # the first, a middle and the last head in full with the fp64 oracle
    ref = _oracle_units(x, [(0, 0), (0, 5), (0, 15)])
    for (_, h), (ro, rS) in ref.items():
        assert_close(f"head {h}: o (fp64 oracle)", np64(o[:, h]), ro, TOL_BF16)
        assert_close(f"head {h}: final state (fp64 oracle)", np64(S[0, h]), rS, TOL_BF16)


@pytest.mark.timeout(600)
def test_decode_512x32_all_128_steps():
    # the decode workload as specified: 512 sequences x 32 heads, one token per step
    # for 128 steps, states updated in place; every output of every step and the
    # final states of all 16384 (sequence, head) units against the fp64 oracle
    N, H, d, steps = 512, 32, 128, 128
    log(f"decode: {N} sequences x {H} heads, d {d}, bf16, {steps} steps")
    S0, draws = inputs.make_decode_steps(N, H, d, d, steps, dtype=torch.bfloat16, seed=4, device="cuda")
    state = S0.clone()
    ref_S = np64(S0)
    worst = 0.0
    for st, dr in enumerate(draws):
        o = gdn.gdn_decode(dr.q, dr.k, dr.v, dr.g, dr.beta, state)
        torch.cuda.synchronize()
        ref_o, ref_S = oracle.decode_step(np64(dr.q), np64(dr.k), np64(dr.v), np64(dr.g), np64(dr.beta), ref_S,
                                          threads=16)
        e = oracle.rel_err(np64(o), ref_o)
        worst = max(worst, e)
        assert np.isfinite(e) and e <= 1e-2, f"step {st}: o rel err {e:.3e}"
        if st % 32 == 31 or st == steps - 1:
            log(f"  step {st}: o rel err {e:.3e} (worst so far {worst:.3e})")
    assert_close("final states, all units", np64(state), ref_S, 1e-5)


@pytest.mark.parametrize("name", ["batch4_t8k", "varlen64"])
def test_backward_full_size_sampled_units(name):
    # the whole workload through gdn_prefill_backward; two (sequence, head) units
    # recomputed by the fp64 oracle's reverse-mode recurrence and compared in full
    log(f"backward full size {name}")
    x = inputs.make_workload(name, seed=0, device="cuda")
    H, dk, dv = x.q.shape[1], x.q.shape[2], x.v.shape[2]
    d_o, dSf = inputs.make_cotangents(x.T_total, x.num_seqs, H, dk, dv, dtype=x.q.dtype, seed=1, device="cuda")
    out = gdn.gdn_prefill_backward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, d_o, initial_state=x.initial_state,
                                   d_final_state=dSf)
    torch.cuda.synchronize()
    cu = x.cu_seqlens.cpu().numpy()
    units = [(0, 0), (x.num_seqs - 1, H - 1)]
    for n, h in units:
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda t: np64(t[a:b, h:h + 1])
        S0 = None if x.initial_state is None else np64(x.initial_state[n:n + 1, h:h + 1])
        ref = oracle.backward(sl(x.q), sl(x.k), sl(x.v), sl(x.g), np64(x.beta[a:b, h:h + 1]),
                              np.array([0, b - a], np.int32), sl(d_o), initial_state=S0,
                              d_final_state=np64(dSf[n:n + 1, h:h + 1]))
        got = {"dq": sl(out[0]), "dk": sl(out[1]), "dv": sl(out[2]), "dg": sl(out[3]),
               "dbeta": np64(out[4][a:b, h:h + 1]), "d_initial_state": np64(out[5][n:n + 1, h:h + 1])}
        log(f"  unit (seq {n}, head {h}), {b - a} tokens")
        for k in got:
            assert_close(k, got[k], ref[k], TOL_BF16)


def test_tiles_pairs_full_size_sampled_units():
    # the position-pair path over the whole four-sequence batch, two units against the oracle
    log("tiles pairs full size batch4_t8k")
    x = inputs.make_workload("batch4_t8k", seed=0, device="cuda")
    o, S = gdn.gdn_prefill_tiles(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, gdn.GDN_TILES_PAIRS)
    torch.cuda.synchronize()
    H = x.q.shape[1]
    units = [(0, 0), (x.num_seqs - 1, H - 1)]
    ref = _oracle_units(x, units)
    cu = x.cu_seqlens.cpu().numpy()
    for (n, h), (ro, rS) in ref.items():
        a, b = int(cu[n]), int(cu[n + 1])
        assert_close(f"o unit ({n},{h})", np64(o[a:b, h]), ro, TOL_BF16)
        assert_close(f"S unit ({n},{h})", np64(S[n, h]), rS, TOL_BF16)
