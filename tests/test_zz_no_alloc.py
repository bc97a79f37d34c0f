"""gdn_prefill_noalloc, the allocation-free variant of gdn_prefill, through the
C-ABI: on two calls in a row on one GPU (the second smaller, so it reuses the
scratch the first left behind), its outputs equal gdn_prefill's bit for bit
(same kernels and plan; only the scratch address differs) and the fp64
oracle's within the bf16 tolerance on sampled units.  Both calls use the time
split, so the scratch is really used."""

import numpy as np
import pytest
import torch

import gated_delta_rule_linear_amd as gdn
import oracle
from gated_delta_rule_linear_amd import inputs
from helpers import assert_close, log, np64, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def _case(lengths, H, seed):
    x = to_device(inputs.make_prefill_inputs(lengths, H, 128, 128, dtype=torch.bfloat16, init_state=True,
                                             seed=seed))
    ws = gdn.gdn_prefill_workspace_bytes(x.T_total, x.num_seqs, H, 128, 128)
    log(f"lengths {lengths} H {H}: scratch needed {ws} bytes of {gdn.GDN_NOALLOC_SCRATCH_BYTES}")
    assert 0 < ws <= gdn.GDN_NOALLOC_SCRATCH_BYTES
    ref_o, ref_S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    o = torch.full_like(ref_o, float("nan"))
    S = torch.full_like(ref_S, float("nan"))
    torch.cuda.synchronize()
    gdn.gdn_prefill_noalloc(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state,
                            final_state=S, o=o)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o), "o differs from gdn_prefill"
    assert torch.equal(S, ref_S), "final state differs from gdn_prefill"
    cu = x.cu_seqlens.cpu().numpy()
    for n, h in [(0, 0), (x.num_seqs - 1, H - 1)]:
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda t: np64(t[a:b, h:h + 1])
        ro, rS = oracle.recurrent(sl(x.q), sl(x.k), sl(x.v), sl(x.g), np64(x.beta[a:b, h:h + 1]),
                                  np.array([0, b - a], np.int32),
                                  initial_state=np64(x.initial_state[n:n + 1, h:h + 1]))
        assert_close(f"seq {n} head {h}: o", np64(o[a:b, h]), ro[:, 0], 2e-2)
        assert_close(f"seq {n} head {h}: state", np64(S[n, h]), rS[0, 0], 2e-2)


def test_noalloc_two_calls_second_smaller(monkeypatch):
    # the library's own plan: one 16,384-token sequence x 32 heads is split (32 MiB of scratch)
    monkeypatch.delenv("GDN_PREFILL_SEGMENT", raising=False)
    _case([16384], 32, seed=60)
    # then a smaller ragged batch with a forced split, over the scratch the first call left
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "256")
    _case([1000, 0, 333], 4, seed=61)
