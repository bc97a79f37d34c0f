"""Stream ordering of the library's calls on streams other than the current one.

  * A prefill on a given stream allocates its outputs and its time-split
    workspace on that stream: while its kernels are still queued behind other
    work there, memory the current stream allocates and fills in the meantime
    cannot be the workspace the call released, so the result is the reference
    result bit for bit.
  * Split prefills on two caller streams at once (each with its own side
    stream) both give the reference result.
"""

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


def _inputs(seed):
    return to_device(inputs.make_prefill_inputs([4096, 1500], 4, 128, 128, dtype=torch.bfloat16, init_state=True,
                                                seed=seed))


def _call(x, stream=None):
    return gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state, stream=stream)


def test_prefill_on_a_non_current_stream_keeps_its_workspace(monkeypatch):
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "512")
    x = _inputs(50)
    ws = gdn.gdn_prefill_workspace_bytes(x.T_total, x.num_seqs, 4, 128, 128)
    assert ws > 0
    ref_o, ref_S = _call(x)
    torch.cuda.synchronize()
    log(f"split prefill on a held-back stream, workspace {ws} bytes")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        torch.cuda._sleep(100_000_000)  # hold the stream back: the prefill's kernels run well after this returns
    o, S = _call(x, stream=s)
    # the current stream allocates and overwrites blocks of the workspace's size meanwhile
    junk = [torch.full((ws // 4 + 64,), float("nan"), device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o, ref_o) and torch.equal(S, ref_S)


def test_split_prefills_on_two_streams_at_once(monkeypatch):
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "512")
    xa, xb = _inputs(51), _inputs(52)
    ra, rb = _call(xa), _call(xb)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for s in (sa, sb):
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        outs.append((_call(xa, stream=sa), _call(xb, stream=sb)))
    torch.cuda.synchronize()
    for rep, (a, b) in enumerate(outs):
        assert torch.equal(a[0], ra[0]) and torch.equal(a[1], ra[1]), f"stream a, call {rep}"
        assert torch.equal(b[0], rb[0]) and torch.equal(b[1], rb[1]), f"stream b, call {rep}"
    log("  two caller streams x 3 split calls each equal the reference")
