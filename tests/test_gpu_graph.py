"""HIP graph capture of the library's calls: gdn_prefill with and without the
time split (the split forks a side stream and joins it back with events),
with the order table of a many-unit batch and with the length-agnostic split,
gdn_prefill_backward with its time split and with the order table, and
gdn_decode.  Each call is
captured once after an eager warm-up, then replayed several times with
unrelated eager work, a host synchronisation and a clearing of the outputs
between replays; every replay must reproduce the eager call's outputs bit for
bit (the kernels are deterministic)."""

import pytest
import torch

import gated_delta_rule_linear_amd as gdn
from gated_delta_rule_linear_amd import inputs
from helpers import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def _graph_check(fn, name, replays=3):
    eager = [t.clone() for t in fn()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    for rep in range(replays):
        junk = torch.randn(1 << 20, device="cuda")
        assert torch.isfinite((junk * 2).sum()).item()  # eager work and a host synchronisation
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"{name}: replay {rep}, output {i} differs from the eager call"
    log(f"  {name}: {replays} replays equal the eager call")


@pytest.mark.parametrize("seg", [128, 0])
def test_prefill_graph(monkeypatch, seg):
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", str(seg))
    log(f"graph: gdn_prefill lengths=[700, 0, 300] H=2 d=128 bf16 segment={seg}")
    x = inputs.make_prefill_inputs([700, 0, 300], 2, 128, 128, dtype=torch.bfloat16, init_state=True, seed=40)
    to_device(x)
    _graph_check(lambda: gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state),
                 f"gdn_prefill segment={seg}")


def test_prefill_graph_longest_first(monkeypatch):
    # 90 sequences x 3 heads = 270 units: the unsplit pass takes them longest first
    # from an order table that a kernel of the call writes
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "0")
    lengths = [(37 * i) % 301 for i in range(90)]
    log(f"graph: gdn_prefill 90 sequences of 0..300 tokens H=3 d=128 bf16, longest first")
    x = inputs.make_prefill_inputs(lengths, 3, 128, 128, dtype=torch.bfloat16, init_state=True, seed=43)
    to_device(x)
    _graph_check(lambda: gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state),
                 "gdn_prefill longest first")


def test_prefill_graph_length_agnostic_split(monkeypatch):
    # 15 sequences of 1,000 tokens and one of 140,000, 32 heads: the mean length needs
    # no split, so the plan splits every sequence longer than T / 9 (the long one, into
    # 9 segments): table, order, split list, maps, first segments, fold and later segments
    monkeypatch.delenv("GDN_PREFILL_SEGMENT", raising=False)
    lengths = [1000] * 15 + [140000]
    log("graph: gdn_prefill 15 x 1000 + 1 x 140000 tokens H=32 d=128 bf16, length-agnostic split")
    x = inputs.make_prefill_inputs(lengths, 32, 128, 128, dtype=torch.bfloat16, init_state=True, seed=44,
                                   device="cuda")
    assert gdn.gdn_prefill_workspace_bytes(x.T_total, 16, 32, 128, 128) > 8 * 32 * 128 * 128 * 4
    _graph_check(lambda: gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state),
                 "gdn_prefill length-agnostic split")


def test_backward_graph_longest_first(monkeypatch):
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "0")
    lengths = [(53 * i) % 201 for i in range(90)]
    log("graph: gdn_prefill_backward 90 sequences of 0..200 tokens H=3 d=128 bf16, longest first")
    x = inputs.make_prefill_inputs(lengths, 3, 128, 128, dtype=torch.bfloat16, init_state=True, seed=45)
    d_o, dSf = inputs.make_cotangents(x.T_total, x.num_seqs, 3, 128, 128, dtype=torch.bfloat16, seed=145)
    to_device(x)
    d_o, dSf = d_o.cuda(), dSf.cuda()
    _graph_check(lambda: gdn.gdn_prefill_backward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, d_o,
                                                  initial_state=x.initial_state, d_final_state=dSf),
                 "gdn_prefill_backward longest first")


def test_backward_graph(monkeypatch):
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "128")
    log("graph: gdn_prefill_backward lengths=[700, 0, 300] H=2 d=128 bf16 segment=128")
    x = inputs.make_prefill_inputs([700, 0, 300], 2, 128, 128, dtype=torch.bfloat16, init_state=True, seed=41)
    d_o, dSf = inputs.make_cotangents(x.T_total, x.num_seqs, 2, 128, 128, dtype=torch.bfloat16, seed=141)
    to_device(x)
    d_o, dSf = d_o.cuda(), dSf.cuda()
    _graph_check(lambda: gdn.gdn_prefill_backward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, d_o,
                                                  initial_state=x.initial_state, d_final_state=dSf),
                 "gdn_prefill_backward segment=128")


def test_decode_graph():
    log("graph: gdn_decode N=64 H=4 d=128 bf16")
    S0, draws = inputs.make_decode_steps(64, 4, 128, 128, 1, dtype=torch.bfloat16, seed=42)
    d = draws[0]
    S0 = S0.cuda()
    q, k, v, g, beta = (t.cuda() for t in (d.q, d.k, d.v, d.g, d.beta))
    state = torch.empty_like(S0)

    def step():
        state.copy_(S0)  # the step updates the state in place: start every replay from S0
        o = gdn.gdn_decode(q, k, v, g, beta, state)
        return o, state

    _graph_check(step, "gdn_decode")
