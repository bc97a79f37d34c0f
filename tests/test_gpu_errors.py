"""The boundary's error contract on the GPU, through the C-ABI:

  * GDN_VALIDATE=1 turns a log-decay outside [-5, 0] (the pages' bound) and a
    malformed cu_seqlens into GDN_ERR_DOMAIN before any kernel is enqueued:
    the outputs and the states keep the values they had;
  * an allocation the device cannot hold is GDN_ERR_OOM, and the library keeps
    working after it;
  * a NaN in one (sequence, head)'s input reaches that unit's outputs from its
    token on and its final state, and nothing else: every other unit, and the
    unit's own chunks before the token, are bit for bit those of the clean
    run -- with and without the time split, and in the decode step.
"""

import ctypes

import numpy as np
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


def _prefill_into(x, o, S, initial_state=None):
    return gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=initial_state, final_state=S,
                           o=o)


def _expect_domain(fn):
    with pytest.raises(gdn.GdnError) as ei:
        fn()
    assert ei.value.status == gdn.GDN_ERR_DOMAIN, str(ei.value)


@pytest.mark.parametrize("bad", [0.5, -5.5, float("nan"), float("inf")])
def test_validate_rejects_gate_outside_the_bound(monkeypatch, bad):
    monkeypatch.setenv("GDN_VALIDATE", "1")
    x = to_device(inputs.make_prefill_inputs([70, 33], 2, 64, 64, dtype=torch.bfloat16, init_state=True, seed=3))
    x.g[40, 1, 7] = bad
    log(f"g[40, 1, 7] = {bad}")
    o = torch.full_like(x.v, 7.0)
    S = torch.full_like(x.initial_state, 3.0)
    S0 = x.initial_state.clone()
    _expect_domain(lambda: _prefill_into(x, o, S, x.initial_state))
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(S == 3.0), "a rejected call wrote its outputs"
    assert torch.equal(x.initial_state, S0)


def test_validate_accepts_the_bound_endpoints(monkeypatch):
    monkeypatch.setenv("GDN_VALIDATE", "1")
    x = to_device(inputs.make_prefill_inputs([70, 33], 2, 64, 64, dtype=torch.bfloat16, seed=4))
    x.g[::2] = -5.0
    x.g[1::2] = 0.0
    o, S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()


@pytest.mark.parametrize("case", ["decreasing", "short", "long", "nonzero_start"])
def test_validate_rejects_malformed_cu_seqlens(monkeypatch, case):
    monkeypatch.setenv("GDN_VALIDATE", "1")
    x = to_device(inputs.make_prefill_inputs([50, 30, 20], 2, 64, 64, dtype=torch.bfloat16, seed=5))
    cu = {"decreasing": [0, 60, 50, 100], "short": [0, 50, 80, 99], "long": [0, 50, 80, 101],
          "nonzero_start": [1, 50, 80, 100]}[case]
    log(f"cu_seqlens {cu} for T = 100")
    x.cu_seqlens = torch.tensor(cu, dtype=torch.int32, device="cuda")
    o = torch.full_like(x.v, 7.0)
    S = torch.full((3, 2, 64, 64), 3.0, device="cuda")
    _expect_domain(lambda: _prefill_into(x, o, S))
    # the logit entry point checks cu_seqlens the same way
    z = torch.zeros_like(x.q)
    _expect_domain(lambda: gdn.gdn_prefill_logits(x.q, x.k, x.v, z, gdn.GDN_GATE_SCALED_SIGMOID, -5.0, x.beta,
                                                  x.cu_seqlens, final_state=S, o=o))
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(S == 3.0), "a rejected call wrote its outputs"


def test_validate_rejects_decode_gate_outside_the_bound(monkeypatch):
    monkeypatch.setenv("GDN_VALIDATE", "1")
    S0, draws = inputs.make_decode_steps(4, 2, 128, 128, 1, dtype=torch.bfloat16, seed=6, device="cuda")
    dr = draws[0]
    dr.g[2, 1, 100] = 0.25
    state = S0.clone()
    o = torch.full_like(dr.v, 7.0)
    _expect_domain(lambda: gdn.gdn_decode(dr.q, dr.k, dr.v, dr.g, dr.beta, state, o=o))
    torch.cuda.synchronize()
    assert torch.equal(state, S0) and torch.all(o == 7.0)


def test_state_alloc_beyond_the_device_is_oom_and_recoverable():
    lib = gdn.load_library()
    out = ctypes.c_void_p()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # 2^24 sequences x 32 heads x 128 x 128 fp32 = 32 TiB: far beyond one GPU's 288 GB
    st = lib.gdn_state_alloc(1 << 24, 32, 128, 128, ctypes.byref(out), stream)
    assert st == gdn.GDN_ERR_OOM and not out.value
    # the library and the device still work afterwards
    addr = gdn.gdn_state_alloc(2, 3, 64, 64)
    torch.cuda.synchronize()
    host = np.empty(2 * 3 * 64 * 64, np.float32)
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime already loaded (by torch and libgdn)
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    assert hip.hipMemcpy(host.ctypes.data, addr, host.nbytes, 2) == 0  # 2: device to host
    assert not host.any(), "gdn_state_alloc must zero-fill"
    gdn.gdn_state_free(addr)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- NaN propagation

def _nan_case(monkeypatch, dtype, split, tensor):
    lengths = [300, 200]
    H, d = 3, 128 if dtype == torch.bfloat16 else 64
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "64" if split else "0")
    x = to_device(inputs.make_prefill_inputs(lengths, H, d, d, dtype=dtype, init_state=True, seed=7))
    o_c, S_c = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    n, h, t = 0, 1, 150  # sequence 0, head 1, token 150 of 300
    getattr(x, tensor)[t, h, 5] = float("nan")
    o_n, S_n = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    log(f"NaN in {tensor}[{t}, {h}, 5], {dtype}, {'split (64-token segments)' if split else 'unsplit'}")
    return lengths, (n, h, t), (o_c, S_c), (o_n, S_n)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nan_in_key_poisons_its_unit_from_that_token_on(monkeypatch, dtype, split):
    # a key enters the read S'^T k, which mixes every value column: the whole state
    # and every output of the unit from token t on are NaN
    lengths, (n, h, t), (o_c, S_c), (o_n, S_n) = _nan_case(monkeypatch, dtype, split, "k")
    assert not torch.isfinite(o_n[t:lengths[0], h].float()).any()
    assert not torch.isfinite(S_n[n, h]).any()
    # its earlier chunks (64-token boundaries: the chunk of every kernel divides 64) are untouched
    c0 = t // 64 * 64
    assert torch.equal(o_n[:c0, h], o_c[:c0, h])
    # every other unit is bit for bit the clean run
    other = [hh for hh in range(o_c.shape[1]) if hh != h]
    assert torch.equal(o_n[:, other], o_c[:, other])
    assert torch.equal(o_n[lengths[0]:, h], o_c[lengths[0]:, h])
    assert torch.equal(S_n[:, other], S_c[:, other]) and torch.equal(S_n[1, h], S_c[1, h])


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nan_in_value_poisons_its_value_column_from_that_token_on(monkeypatch, dtype, split):
    # value column c of the state depends on column c of v only: a NaN in v[t, h, 5]
    # reaches state column 5 and output column 5 of the unit from token t on, and
    # every other column stays bit for bit the clean run
    lengths, (n, h, t), (o_c, S_c), (o_n, S_n) = _nan_case(monkeypatch, dtype, split, "v")
    assert not torch.isfinite(o_n[t:lengths[0], h, 5].float()).any()
    assert not torch.isfinite(S_n[n, h, :, 5]).any()
    cols = [c for c in range(o_c.shape[2]) if c != 5]
    assert torch.equal(o_n[:, :, cols], o_c[:, :, cols])
    assert torch.equal(S_n[:, :, :, cols], S_c[:, :, :, cols])
    c0 = t // 64 * 64
    assert torch.equal(o_n[:c0, h, 5], o_c[:c0, h, 5])
    other = [hh for hh in range(o_c.shape[1]) if hh != h]
    assert torch.equal(o_n[:, other], o_c[:, other]) and torch.equal(S_n[:, other], S_c[:, other])


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nan_in_query_reaches_only_its_own_output(monkeypatch, dtype, split):
    # q is read only by its own token's output: o_t = S_t^T q_t
    lengths, (n, h, t), (o_c, S_c), (o_n, S_n) = _nan_case(monkeypatch, dtype, split, "q")
    assert not torch.isfinite(o_n[t, h].float()).any()
    keep = torch.ones(o_c.shape[0], dtype=torch.bool, device=o_c.device)
    keep[t] = False
    assert torch.equal(o_n[keep], o_c[keep])
    assert torch.equal(o_n[t, [0, 2]], o_c[t, [0, 2]])
    assert torch.equal(S_n, S_c)


def test_nan_in_decode_reaches_only_its_unit():
    S0, draws = inputs.make_decode_steps(8, 4, 128, 128, 1, dtype=torch.bfloat16, seed=8, device="cuda")
    dr = draws[0]
    s_c = S0.clone()
    o_c = gdn.gdn_decode(dr.q, dr.k, dr.v, dr.g, dr.beta, s_c)
    dr.v[3, 2, 17] = float("nan")
    s_n = S0.clone()
    o_n = gdn.gdn_decode(dr.q, dr.k, dr.v, dr.g, dr.beta, s_n)
    torch.cuda.synchronize()
    # value column 17 of that unit only (o = S^T q and the state's column 17)
    assert not torch.isfinite(o_n[3, 2, 17].float()) and not torch.isfinite(s_n[3, 2, :, 17]).any()
    cols = [c for c in range(128) if c != 17]
    assert torch.equal(o_n[3, 2, cols], o_c[3, 2, cols]) and torch.equal(s_n[3, 2, :, cols], s_c[3, 2, :, cols])
    mask = torch.ones(8, 4, dtype=torch.bool, device="cuda")
    mask[3, 2] = False
    assert torch.equal(o_n[mask], o_c[mask]) and torch.equal(s_n[mask], s_c[mask])
