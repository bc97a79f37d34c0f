"""GPU parity of the time-split prefill: sequences cut into segments whose
transitions are computed in parallel, folded, then replayed.  The segment
length is forced with GDN_PREFILL_SEGMENT so that small inputs exercise every
path (non-last segments, ragged last ones, sequences shorter than a segment,
empty sequences, many segments per sequence); results are compared with the
fp64 oracle element by element and with the unsplit kernel."""

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


def _run(x, seg, monkeypatch, **kw):
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", str(seg))
    o, S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, **kw)
    torch.cuda.synchronize()
    return o, S


def _case(monkeypatch, lengths, H, dk, dv, dtype, seg, gate="amin", init=True, seed=0):
    log(f"split case lengths={lengths} H={H} dk={dk} dv={dv} {dtype} seg={seg} gate={gate} init={init} seed={seed}")
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype=dtype, gate=gate, init_state=init, seed=seed)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    o, S = _run(x, seg, monkeypatch, initial_state=x.initial_state)
    assert_close("o", np64(o), ref_o, TOL[dtype])
    assert_close("final_state", np64(S), ref_S, TOL[dtype])
    o1, S1 = _run(x, 0, monkeypatch, initial_state=x.initial_state)
    assert_close("o vs unsplit", np64(o), np64(o1), TOL[dtype])
    assert_close("state vs unsplit", np64(S), np64(S1), TOL[dtype])


def test_split_bf16_ragged(monkeypatch):
    # lengths below, at and above the segment, a zero-length sequence, several segments
    _case(monkeypatch, [1, 255, 256, 257, 0, 700, 64], 3, 128, 128, torch.bfloat16, 256, seed=20)


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, torch.bfloat16), (64, 64, torch.float32)])
def test_split_units_multiple_of_eight(monkeypatch, dk, dv, dtype):
    # 16 (sequence, head) units with initial states: the fold keeps the column
    # blocks of a unit together (the block order for unit counts divisible by 8)
    _case(monkeypatch, [900, 333], 8, dk, dv, dtype, 128, seed=24)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_split_many_units_fold(monkeypatch, dtype):
    # 40 split sequences x 2 heads x 8 column blocks = 640 fold workgroups, more than
    # the 256 compute units: the fold prefetches one step ahead, two workgroups per CU
    _case(monkeypatch, [260 + 7 * i for i in range(40)], 2, 128, 128, dtype, 128, seed=25)


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (64, 64)])
def test_split_head_dims(monkeypatch, dk, dv):
    _case(monkeypatch, [300, 5, 129], 2, dk, dv, torch.bfloat16, 128, seed=21)


def test_split_fp32(monkeypatch):
    _case(monkeypatch, [500, 64, 193], 2, 128, 128, torch.float32, 192, seed=22)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_split_pages_gate(monkeypatch, dtype):
    # chunks beyond the single-reference budget inside the transition pass
    _case(monkeypatch, [400, 130], 2, 128, 128, dtype, 128, gate="pages", seed=23)


def test_split_zero_initial_state(monkeypatch):
    _case(monkeypatch, [390, 77], 2, 128, 128, torch.bfloat16, 128, init=False, seed=24)


def test_split_one_chunk_segments(monkeypatch):
    # ten segments of one chunk each: a fold of nine transitions
    _case(monkeypatch, [640, 65], 2, 128, 128, torch.bfloat16, 64, seed=25)


def test_split_final_state_in_place(monkeypatch):
    # final_state aliases initial_state: segment 0 reads it while the last segment finishes
    x = inputs.make_prefill_inputs([520, 60, 0], 2, 128, 128, dtype=torch.bfloat16, init_state=True, seed=26)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    S = x.initial_state.clone()
    o, S_out = _run(x, 128, monkeypatch, initial_state=S, final_state=S)
    assert S_out.data_ptr() == S.data_ptr()
    assert_close("o", np64(o), ref_o, 2e-2)
    assert_close("final_state (in place)", np64(S), ref_S, 2e-2)
    assert torch.equal(S[2], x.initial_state[2])


def test_split_deterministic(monkeypatch):
    x = inputs.make_prefill_inputs([1000, 300], 4, 128, 128, dtype=torch.bfloat16, init_state=True, seed=27)
    to_device(x)
    o1, S1 = _run(x, 256, monkeypatch, initial_state=x.initial_state)
    o2, S2 = _run(x, 256, monkeypatch, initial_state=x.initial_state)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_split_caller_workspace(monkeypatch):
    # a caller-owned workspace of exactly the reported size, reused twice
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "128")
    x = inputs.make_prefill_inputs([450, 200], 2, 128, 128, dtype=torch.bfloat16, init_state=True, seed=28)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    need = gdn.gdn_prefill_workspace_bytes(x.T_total, 2, 2, 128, 128)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # contents on entry are ignored
    for _ in range(2):
        o, S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state,
                               workspace=ws)
        torch.cuda.synchronize()
        assert_close("o", np64(o), ref_o, 2e-2)
        assert_close("final_state", np64(S), ref_S, 2e-2)


@pytest.mark.parametrize("kind,p,gate", [(gdn.GDN_GATE_SCALED_SIGMOID, -5.0, "pages"),
                                         (gdn.GDN_GATE_ALPHA_MIN, 0.9, "amin")])
def test_split_logits(monkeypatch, kind, p, gate):
    # the logit gate through the transition, fold and replay kernels
    lengths = [1, 255, 256, 257, 0, 700]
    log(f"split logits lengths={lengths} gate={gate}")
    x = inputs.make_prefill_inputs(lengths, 3, 128, 128, dtype=torch.bfloat16, gate=gate, a_min=0.9, init_state=True,
                                   seed=23, logits=True)
    ref_o, ref_S = oracle_prefill(x, gate=(kind, p))
    to_device(x)
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "256")
    o, S = gdn.gdn_prefill_logits(x.q, x.k, x.v, x.z, kind, p, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, TOL[torch.bfloat16])
    assert_close("final_state", np64(S), ref_S, TOL[torch.bfloat16])


@pytest.mark.parametrize("gate", ["amin", "pages"])
def test_split_head_gate(monkeypatch, gate):
    # one gate per (token, head) through the transition, fold and replay kernels
    lengths = [1, 255, 256, 257, 0, 700]
    log(f"split head gate lengths={lengths} gate={gate}")
    x = inputs.make_prefill_inputs(lengths, 3, 128, 128, dtype=torch.bfloat16, gate=gate, a_min=0.9, init_state=True,
                                   seed=24, head_gate=True)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "256")
    o, S = gdn.gdn_prefill_head_gate(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, TOL[torch.bfloat16])
    assert_close("final_state", np64(S), ref_S, TOL[torch.bfloat16])
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "0")
    o1, S1 = gdn.gdn_prefill_head_gate(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o vs unsplit", np64(o), np64(o1), TOL[torch.bfloat16])


def test_maxlen_hint_splits_a_skewed_batch(monkeypatch):
    # one 16,384-token sequence among 31 of 256 tokens, 4 heads: planned from the
    # mean length the batch is not split; with the bound on the lengths the long
    # sequence is cut into segments.  Every unit against the fp64 oracle.
    monkeypatch.delenv("GDN_PREFILL_SEGMENT", raising=False)
    lengths = [256] * 15 + [16384] + [256] * 16
    H, d = 4, 128
    T = sum(lengths)
    assert gdn.gdn_prefill_workspace_bytes(T, len(lengths), H, d, d) == 0
    assert gdn.gdn_prefill_workspace_bytes_maxlen(T, len(lengths), 16384, H, d, d) > 0
    log(f"skewed batch T={T}: workspace with the bound "
        f"{gdn.gdn_prefill_workspace_bytes_maxlen(T, len(lengths), 16384, H, d, d)} bytes")
    x = inputs.make_prefill_inputs(lengths, H, d, d, dtype=torch.bfloat16, init_state=True, seed=26)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    o, S = gdn.gdn_prefill_maxlen(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, 16384, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, TOL[torch.bfloat16])
    assert_close("final_state", np64(S), ref_S, TOL[torch.bfloat16])
    # a bound that is too large or too small changes the plan, not the result
    for bound in (1 << 20, 1024):
        ob, Sb = gdn.gdn_prefill_maxlen(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, bound,
                                        initial_state=x.initial_state)
        torch.cuda.synchronize()
        assert_close(f"o, bound {bound}", np64(ob), ref_o, TOL[torch.bfloat16])
        assert_close(f"final_state, bound {bound}", np64(Sb), ref_S, TOL[torch.bfloat16])
    # under validation, a sequence longer than the bound is a domain error and nothing is written
    monkeypatch.setenv("GDN_VALIDATE", "1")
    oz = torch.full_like(o, 7.0)
    with pytest.raises(gdn.GdnError) as ei:
        gdn.gdn_prefill_maxlen(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, 8192, initial_state=x.initial_state, o=oz)
    assert ei.value.status == gdn.GDN_ERR_DOMAIN
    torch.cuda.synchronize()
    assert torch.all(oz == 7.0)
