"""GPU parity of gdn_prefill_tiles (the diagonal-tile comparison) through the
C-ABI against the fp64 oracle: the position-pair path on the unbounded
negative-softplus gate (steep decays that overflow a split of the pair decays
in fp32), both paths on bounded gates, and the two paths against each other."""

import numpy as np
import pytest
import torch

import gated_delta_rule_linear_amd as gdn
from gated_delta_rule_linear_amd import inputs
from helpers import TOL, assert_close, log, np64, oracle_prefill, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def _case(lengths, H, dk, dv, dtype, gate, path, scale=1.0, init=True, seed=0):
    log(f"tiles case lengths={lengths} H={H} dk={dk} dv={dv} {dtype} gate={gate}x{scale} path={path} init={init}")
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype=dtype, gate=gate, init_state=init, seed=seed,
                                   softplus_scale=scale)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    o, S = gdn.gdn_prefill_tiles(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, path, initial_state=x.initial_state)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert_close("o", np64(o), ref_o, tol)
    assert_close("final_state", np64(S), ref_S, tol)
    return x, o, S


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_pairs_unbounded_softplus_gate(dtype, dk, dv):
    # g = -softplus(8 z): steep, unbounded decays
    _case([1, 15, 16, 17, 100, 0, 200], 2, dk, dv, dtype, "softplus", gdn.GDN_TILES_PAIRS, scale=8.0, seed=1)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pairs_softplus_gate_unscaled(dtype):
    _case([300, 77], 3, 128, 128, dtype, "softplus", gdn.GDN_TILES_PAIRS, seed=2)


@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("gate", ["amin", "pages"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_both_paths_bounded_gates(path, gate, dtype):
    _case([1, 15, 16, 17, 130, 0, 64], 2, 128, 128, dtype, gate, path, seed=3)


def test_paths_agree_on_bounded_gates():
    x = inputs.make_prefill_inputs([500, 33], 4, 128, 128, dtype=torch.bfloat16, gate="pages", init_state=True,
                                   seed=4)
    to_device(x)
    od, Sd = gdn.gdn_prefill_tiles(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, gdn.GDN_TILES_DENSE,
                                   initial_state=x.initial_state)
    op, Sp = gdn.gdn_prefill_tiles(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, gdn.GDN_TILES_PAIRS,
                                   initial_state=x.initial_state)
    o, S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o pairs vs dense", np64(op), np64(od), 2e-2)
    assert_close("o pairs vs gdn_prefill", np64(op), np64(o), 2e-2)
    assert_close("S pairs vs dense", np64(Sp), np64(Sd), 2e-2)


def test_pairs_final_state_in_place():
    x = inputs.make_prefill_inputs([40, 70], 2, 64, 64, dtype=torch.bfloat16, gate="softplus", init_state=True,
                                   seed=5, softplus_scale=4.0)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    S = x.initial_state.clone()
    o, _ = gdn.gdn_prefill_tiles(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, gdn.GDN_TILES_PAIRS, initial_state=S,
                                 final_state=S)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, 2e-2)
    assert_close("final_state (in place)", np64(S), ref_S, 2e-2)
