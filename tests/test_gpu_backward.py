"""GPU parity of gdn_prefill_backward: dq, dk, dv, dg, dbeta and the initial
state's gradient through the C-ABI against the fp64 oracle's reverse-mode
recurrence (oracle.backward, pinned by finite differences and hand-derived
cases in test_oracle_backward_pins.py), element by element on seeded inputs.
Sizes span several 16-token sub-chunks and ragged tails."""

import numpy as np
import pytest
import torch

import gated_delta_rule_linear_amd as gdn
import oracle
from gated_delta_rule_linear_amd import inputs
from helpers import TOL, assert_close, log, np64, to_device

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def _oracle_grads(x, d_o, dSf):
    cu = x.cu_seqlens.cpu().numpy().astype(np.int32)
    return oracle.backward(np64(x.q), np64(x.k), np64(x.v), np64(x.g), np64(x.beta), cu, np64(d_o),
                           initial_state=None if x.initial_state is None else np64(x.initial_state),
                           d_final_state=None if dSf is None else np64(dSf))


def _run(x, d_o, dSf):
    out = gdn.gdn_prefill_backward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, d_o, initial_state=x.initial_state,
                                   d_final_state=dSf)
    torch.cuda.synchronize()
    return dict(zip(NAMES, out))


def _check(got, ref, tol):
    for name in NAMES:
        assert_close(name, np64(got[name]), ref[name], tol)


def _case(lengths, H, dk, dv, dtype, gate="amin", init=True, final=True, seed=0, x=None):
    log(f"backward case lengths={lengths} H={H} dk={dk} dv={dv} {dtype} gate={gate} init={init} final={final}")
    if x is None:
        x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype=dtype, gate=gate, init_state=init, seed=seed)
    d_o, dSf = inputs.make_cotangents(x.T_total, x.num_seqs, H, dk, dv, dtype=dtype, final_state=final,
                                      seed=seed + 100)
    ref = _oracle_grads(x, d_o, dSf)
    to_device(x)
    d_o = d_o.cuda()
    dSf = None if dSf is None else dSf.cuda()
    got = _run(x, d_o, dSf)
    _check(got, ref, TOL[dtype])
    return x, d_o, dSf, got


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_longest_first_order_many_units(dtype, d):
    # 90 sequences of 0 .. 300 tokens x 3 heads: 270 (sequence, head) units, more
    # than the compute units, so both sweeps take the sequences longest first
    # through an order table in the workspace; every gradient of every unit,
    # the initial state's included, against the fp64 oracle
    rng = np.random.default_rng(35)
    lengths = [int(v) for v in rng.integers(0, 301, 90)]
    lengths[7] = lengths[60] = 0
    lengths[88] = 1
    _case(lengths, 3, d, d, dtype, seed=37)


@pytest.mark.timeout(600)
def test_length_agnostic_split_skewed(monkeypatch):
    # 15 sequences of 1,000 tokens and one of 140,000, 32 heads: 512 units, more than
    # the compute units, so the plan cuts every sequence longer than T / 9 tokens (the
    # long one, into 9 segments) and the sweeps take its segments first.  Every
    # gradient against the unsplit pass (one workgroup per (sequence, head)); two short
    # units also against the fp64 oracle.
    monkeypatch.delenv("GDN_BACKWARD_SEGMENT", raising=False)
    lengths = [1000] * 15 + [140000]
    H, d = 32, 128
    log("backward length-agnostic split: 15 x 1000 + 1 x 140000 tokens, 32 heads")
    x = inputs.make_prefill_inputs(lengths, H, d, d, dtype=torch.bfloat16, init_state=True, seed=47)
    d_o, dSf = inputs.make_cotangents(x.T_total, x.num_seqs, H, d, d, dtype=torch.bfloat16, seed=147)
    T = x.T_total
    unsplit_bytes = (T // 16 + 16) * H * d * d * 2
    assert gdn.gdn_prefill_backward_workspace_bytes(T, 16, H, d, d, torch.bfloat16) > unsplit_bytes + (1 << 20)
    to_device(x)
    d_o, dSf = d_o.cuda(), dSf.cuda()
    got = _run(x, d_o, dSf)
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "0")
    ref = _run(x, d_o, dSf)
    for name in NAMES:
        assert_close(f"{name} split vs unsplit", np64(got[name]), np64(ref[name]), TOL[torch.bfloat16])
    # two short units against the oracle, each on its own tokens (units are independent)
    cu = x.cu_seqlens.cpu().numpy()
    for n, h in ((0, 3), (14, 30)):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda t: t[a:b, h:h + 1].cpu()
        sub = inputs.PrefillInputs(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta),
                                   torch.tensor([0, b - a], dtype=torch.int32), [b - a],
                                   x.initial_state[n:n + 1, h:h + 1].cpu())
        r = _oracle_grads(sub, d_o[a:b, h:h + 1].cpu(), dSf[n:n + 1, h:h + 1].cpu())
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            assert_close(f"seq {n} head {h} {name}", np64(got[name][a:b, h:h + 1]), r[name], TOL[torch.bfloat16])
        assert_close(f"seq {n} head {h} d_initial_state", np64(got["d_initial_state"][n:n + 1, h:h + 1]),
                     r["d_initial_state"], TOL[torch.bfloat16])


@pytest.mark.parametrize("seg", [0, 64])
def test_many_short_sequences(monkeypatch, seg):
    # 1,500 sequences of 0 .. 150 tokens x 2 heads, d = 64, fp32: the order tables over
    # several blocks of sequences (without the split, and with 64-token segments, where
    # the segment prefix table orders the sweeps); every gradient against the oracle
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", str(seg))
    rng = np.random.default_rng(61 + seg)
    lengths = [int(v) for v in rng.integers(0, 151, 1500)]
    for i in range(0, 1500, 9):
        lengths[i] = 0
    _case(lengths, 2, 64, 64, torch.float32, seed=62)


def test_small_fp32():
    # one 256-token sequence, 2 heads, d = 64, fp32, zero initial state
    _case([256], 2, 64, 64, torch.float32, init=False)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_bf16_ragged(dk, dv):
    _case([1, 15, 16, 17, 63, 0, 130], 3, dk, dv, torch.bfloat16, seed=1)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_fp32_ragged(dk, dv):
    _case([1, 15, 16, 17, 63, 0, 130], 2, dk, dv, torch.float32, seed=2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pages_gate(dtype):
    # g = -5 sigmoid(z): about -40 per 16 tokens, the range the window reference is built for
    _case([320, 100], 2, 128, 128, dtype, gate="pages", seed=3)


def test_no_initial_state_no_final_gradient():
    _case([200, 33], 2, 128, 128, torch.bfloat16, init=False, final=False, seed=4)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gate_endpoints_and_beta_extremes(dtype):
    # g exactly -5 and exactly 0 on alternating 16-token blocks, beta in {0, 1}
    lengths = [96, 50]
    x = inputs.make_prefill_inputs(lengths, 2, 64, 64, dtype=dtype, gate="pages", init_state=True, seed=5)
    T = x.T_total
    blk = (torch.arange(T) // 16) % 2
    x.g = torch.where(blk[:, None, None] == 0, torch.tensor(-5.0), torch.tensor(0.0)).expand(T, 2, 64).contiguous()
    x.beta = (torch.arange(T * 2).reshape(T, 2) % 3 != 0).to(torch.float32)
    _case(lengths, 2, 64, 64, dtype, x=x, seed=5)


def test_deterministic():
    x = inputs.make_prefill_inputs([300, 77], 2, 128, 128, dtype=torch.bfloat16, init_state=True, seed=6)
    d_o, dSf = inputs.make_cotangents(x.T_total, x.num_seqs, 2, 128, 128, seed=106)
    to_device(x)
    d_o, dSf = d_o.cuda(), dSf.cuda()
    a = _run(x, d_o, dSf)
    b = _run(x, d_o, dSf)
    for name in NAMES:
        assert torch.equal(a[name], b[name]), name


def test_without_initial_state_gradient_output():
    x = inputs.make_prefill_inputs([40], 1, 64, 64, dtype=torch.bfloat16, init_state=True, seed=7)
    d_o, dSf = inputs.make_cotangents(x.T_total, 1, 1, 64, 64, seed=107)
    ref = _oracle_grads(x, d_o, dSf)
    to_device(x)
    out = gdn.gdn_prefill_backward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, d_o.cuda(),
                                   initial_state=x.initial_state, d_final_state=dSf.cuda(),
                                   want_d_initial_state=False)
    torch.cuda.synchronize()
    assert out[5] is None
    for name, t in zip(NAMES[:5], out[:5]):
        assert_close(name, np64(t), ref[name], TOL[torch.bfloat16])


def test_pages_gate_long_sequences(monkeypatch):
    # the pages' gate g = -5 sigmoid(z) over a few thousand tokens: every window
    # needs its middle reference (about -40 per 16 tokens); one sweep per
    # (sequence, head) (the planner would split these few units)
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "0")
    _case([2048, 1000], 4, 128, 128, torch.bfloat16, gate="pages", seed=8)


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_bf16_rectangular_longer(dk, dv):
    _case([777, 64, 1300], 3, dk, dv, torch.bfloat16, seed=9)


# ---- time split: each sequence cut into segments of GDN_BACKWARD_SEGMENT
# tokens, with the transitions, both folds and the per-segment sweeps


@pytest.mark.parametrize("seg,dk,dv,dtype", [(64, 128, 128, torch.bfloat16), (64, 64, 64, torch.float32),
                                             (128, 64, 128, torch.bfloat16), (64, 128, 64, torch.bfloat16),
                                             (192, 128, 128, torch.float32), (64, 64, 64, torch.bfloat16)])
def test_split_ragged(monkeypatch, seg, dk, dv, dtype):
    # empty sequences, sequences of one, two and many segments, ragged last segments (129 and 130
    # tokens end in last segments of one and two tokens at seg = 64); bf16 with d_k = d_v takes the
    # reverse maps' offsets from the transition pass's q^, the other cases from adjoint-only sweeps
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", str(seg))
    _case([1, 15, 16, 17, 63, 0, 130, 700, 128, 129], 3, dk, dv, dtype, seed=10)


def test_split_pages_gate_long(monkeypatch):
    # eight segments per sequence under the pages' steep gate
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "256")
    _case([2048, 1000], 4, 128, 128, torch.bfloat16, gate="pages", seed=11)


def test_split_units_multiple_of_eight_rectangular(monkeypatch):
    # 16 units, d_k != d_v: both folds with the column blocks of a unit together
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "128")
    _case([700, 257], 8, 64, 128, torch.bfloat16, seed=14)


def test_split_no_initial_state_no_final_gradient(monkeypatch):
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "64")
    _case([200, 0, 33], 2, 128, 128, torch.bfloat16, init=False, final=False, seed=12)


def test_split_many_units_fold(monkeypatch):
    # 40 split sequences x 2 heads: both folds with more workgroups (640) than compute units,
    # which prefetch one step ahead, two workgroups per CU
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "128")
    _case([260 + 7 * i for i in range(40)], 2, 128, 128, torch.bfloat16, seed=16)


def test_split_matches_unsplit_bf16(monkeypatch):
    # bf16 with d_k = d_v: the split with q^ against the unsplit call, within the bf16 tolerance
    x = inputs.make_prefill_inputs([900, 300], 2, 128, 128, dtype=torch.bfloat16, init_state=True, seed=15)
    d_o, dSf = inputs.make_cotangents(x.T_total, x.num_seqs, 2, 128, 128, dtype=torch.bfloat16, seed=115)
    to_device(x)
    d_o, dSf = d_o.cuda(), dSf.cuda()
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "0")
    a = _run(x, d_o, dSf)
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "128")
    b = _run(x, d_o, dSf)
    for name in NAMES:
        assert_close(name, np64(b[name]), np64(a[name]), TOL[torch.bfloat16])


def test_split_matches_unsplit(monkeypatch):
    # the same call with and without the split agrees to rounding (fp32)
    x = inputs.make_prefill_inputs([900, 300], 2, 64, 64, dtype=torch.float32, init_state=True, seed=13)
    d_o, dSf = inputs.make_cotangents(x.T_total, x.num_seqs, 2, 64, 64, dtype=torch.float32, seed=113)
    to_device(x)
    d_o, dSf = d_o.cuda(), dSf.cuda()
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "0")
    a = _run(x, d_o, dSf)
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "128")
    b = _run(x, d_o, dSf)
    for name in NAMES:
        assert_close(name, np64(b[name]), np64(a[name]), TOL[torch.float32])
