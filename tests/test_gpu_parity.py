"""GPU parity: gdn_prefill and gdn_decode through the C-ABI against the fp64
oracle, element by element, on seeded inputs.  Sizes span several chunks and
ragged tails; the full-size workloads are checked on sampled (sequence, head)
units in test_gpu_fullsize.py."""

import math

import numpy as np
import pytest
import torch

import gated_delta_rule_linear_amd as gdn
import oracle
from gated_delta_rule_linear_amd import inputs
from helpers import TOL, assert_close, log, np64, oracle_prefill, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def _prefill_case(lengths, H, dk, dv, dtype, gate="amin", a_min=0.9, init=True, seed=0):
    log(f"case lengths={lengths} H={H} dk={dk} dv={dv} {dtype} gate={gate} init={init} seed={seed}")
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype=dtype, gate=gate, a_min=a_min, init_state=init,
                                   seed=seed)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    o, S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert_close("o", np64(o), ref_o, tol)
    assert_close("final_state", np64(S), ref_S, tol)
    return x, o, S


def test_small_fp32_single_sequence():
    # one 256-token sequence, 2 heads, d = 64, fp32, zero initial state
    _prefill_case([256], 2, 64, 64, torch.float32, init=False)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_bf16_ragged(dk, dv):
    _prefill_case([1, 63, 64, 65, 130, 0, 200], 3, dk, dv, torch.bfloat16, seed=1)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_fp32_ragged(dk, dv):
    _prefill_case([1, 63, 64, 65, 130, 0, 200], 2, dk, dv, torch.float32, seed=2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pages_gate_forces_subtiles(dtype):
    # g = -5 sigmoid(z): a chunk's total log-decay reaches about -80 (32 tokens)
    # or -160 (64 tokens), beyond the single-reference budget, so every chunk
    # takes the per-16-token-block middle reference
    _prefill_case([320, 320], 4, 128, 128, dtype, gate="pages", seed=3)


@pytest.mark.parametrize("gate", ["amin", "pages"])
def test_bf16_single_role_kernel(monkeypatch, gate):
    # the single-role bf16 kernel (64-token chunks), selected by GDN_PREFILL_KERNEL=seq
    monkeypatch.setenv("GDN_PREFILL_KERNEL", "seq")
    lengths = [1, 63, 64, 65, 130, 0, 200] if gate == "amin" else [320, 320]
    _prefill_case(lengths, 3, 128, 128, torch.bfloat16, gate=gate, seed=5)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gate_endpoints_and_beta_extremes(dtype):
    # g exactly -5 on even chunks and exactly 0 on odd chunks, beta in {0, 1},
    # lengths {0, 1, 63, 64, 65}
    lengths = [0, 1, 63, 64, 65]
    H, d = 2, 128
    x = inputs.make_prefill_inputs(lengths, H, d, d, dtype=dtype, init_state=True, seed=4)
    cu = x.cu_seqlens.tolist()
    for n in range(len(lengths)):
        for t in range(cu[n], cu[n + 1]):
            x.g[t] = -5.0 if ((t - cu[n]) // 64) % 2 == 0 else 0.0
    x.beta.copy_((torch.arange(x.T_total)[:, None] + torch.arange(H)[None, :]) % 2 == 0)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    o, S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, TOL[dtype])
    assert_close("final_state", np64(S), ref_S, TOL[dtype])


def test_scalar_gate_special_case():
    # all channels of g equal (a per-head gate)
    x = inputs.make_prefill_inputs([190, 77], 2, 128, 128, dtype=torch.bfloat16, init_state=True, seed=5)
    x.g.copy_(x.g[:, :, :1].expand_as(x.g))
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    o, S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, 2e-2)
    assert_close("final_state", np64(S), ref_S, 2e-2)


def test_write_then_read_on_gpu():
    # unit keys, beta = 1: querying with the key just written returns its value
    x = inputs.make_prefill_inputs([128, 50], 2, 128, 128, dtype=torch.float32, gate="pages", init_state=True,
                                   seed=6)
    x.beta.fill_(1.0)
    x.q = x.k.clone()
    to_device(x)
    o, _ = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o vs v", np64(o), np64(x.v), 1e-4)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_longest_first_order_many_units(monkeypatch, dtype, d):
    # 90 sequences of 0 .. 600 tokens x 3 heads: 270 (sequence, head) units, more
    # than the 256 compute units, so the pass over whole sequences takes them
    # longest first through an order table in the workspace.  Every unit
    # against the fp64 oracle, initial and final states included (each
    # workgroup must still read and write its own unit's states).
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "0")
    rng = np.random.default_rng(31)
    lengths = [int(v) for v in rng.integers(0, 601, 90)]
    lengths[3] = lengths[50] = 0
    lengths[89] = 1
    H = 3
    assert gdn.gdn_prefill_workspace_bytes(sum(lengths), len(lengths), H, d, d) == 512  # int32 [90], rounded
    assert gdn.gdn_prefill_workspace_bytes(sum(lengths[:85]), 85, H, d, d) == 0  # 255 units: no table
    _prefill_case(lengths, H, d, d, dtype, seed=33)


@pytest.mark.parametrize("seg", [0, 64])
def test_many_short_sequences(monkeypatch, seg):
    # 3,000 sequences of 0 .. 40 tokens (a tenth of them empty) x 2 heads, d = 64, fp32:
    # the order kernel and the segment table walk several blocks of sequences.  With
    # 64-token segments a second batch, 1,500 sequences of 0 .. 300 tokens, has most of
    # them split.  Every unit against the oracle, both states included.
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", str(seg))
    rng = np.random.default_rng(51 + seg)
    lengths = [int(v) for v in rng.integers(0, 41, 3000)]
    for i in range(0, 3000, 10):
        lengths[i] = 0
    _prefill_case(lengths, 2, 64, 64, torch.float32, seed=52)
    if seg:
        lengths = [int(v) for v in rng.integers(0, 301, 1500)]
        _prefill_case(lengths, 2, 64, 64, torch.float32, seed=53)


def test_split_prefill_equals_whole():
    x = inputs.make_prefill_inputs([300], 2, 128, 128, dtype=torch.bfloat16, init_state=True, seed=7)
    to_device(x)
    o, S = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    for a in (64, 100):
        cu1 = torch.tensor([0, a], dtype=torch.int32, device="cuda")
        cu2 = torch.tensor([0, 300 - a], dtype=torch.int32, device="cuda")
        sl = lambda t, lo, hi: t[lo:hi].contiguous()
        o1, S1 = gdn.gdn_prefill(sl(x.q, 0, a), sl(x.k, 0, a), sl(x.v, 0, a), sl(x.g, 0, a), sl(x.beta, 0, a), cu1,
                                 initial_state=x.initial_state)
        o2, S2 = gdn.gdn_prefill(sl(x.q, a, 300), sl(x.k, a, 300), sl(x.v, a, 300), sl(x.g, a, 300),
                                 sl(x.beta, a, 300), cu2, initial_state=S1)
        torch.cuda.synchronize()
        assert_close(f"split at {a}: o", np64(torch.cat([o1, o2])), np64(o), 2e-2)
        assert_close(f"split at {a}: S", np64(S2), np64(S), 2e-2)


def test_final_state_in_place_and_zero_length():
    x = inputs.make_prefill_inputs([70, 0, 5], 2, 64, 64, dtype=torch.bfloat16, init_state=True, seed=8)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    S = x.initial_state.clone()
    o, S_out = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=S, final_state=S)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    assert_close("o", np64(o), ref_o, 2e-2)
    assert_close("final_state (in place)", np64(S), ref_S, 2e-2)
    assert torch.equal(S[1], x.initial_state[1])  # zero-length sequence keeps its state


def test_deterministic():
    x = inputs.make_prefill_inputs([500, 33], 4, 128, 128, dtype=torch.bfloat16, init_state=True, seed=9)
    to_device(x)
    o1, S1 = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    o2, S2 = gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_decode_steps(dtype, dk, dv):
    N, H, steps = 5, 3, 6
    log(f"decode N={N} H={H} dk={dk} dv={dv} {dtype}")
    S0, draws = inputs.make_decode_steps(N, H, dk, dv, steps, dtype=dtype, seed=10)
    ref_S = np64(S0)
    state = S0.cuda()
    for st, d in enumerate(draws):
        ref_o, ref_S = oracle.decode_step(np64(d.q), np64(d.k), np64(d.v), np64(d.g), np64(d.beta), ref_S)
        o = gdn.gdn_decode(d.q.cuda(), d.k.cuda(), d.v.cuda(), d.g.cuda(), d.beta.cuda(), state)
        torch.cuda.synchronize()
        tol = 1e-5 if dtype == torch.float32 else 1e-2
        assert_close(f"step {st} o", np64(o), ref_o, tol)
    assert_close("state", np64(state), ref_S, 1e-5)


def test_one_token_prefill_equals_decode():
    N, H, d = 4, 2, 128
    S0, draws = inputs.make_decode_steps(N, H, d, d, 1, dtype=torch.bfloat16, seed=11)
    dr = draws[0]
    state = S0.cuda().contiguous()
    o_dec = gdn.gdn_decode(dr.q.cuda(), dr.k.cuda(), dr.v.cuda(), dr.g.cuda(), dr.beta.cuda(), state)
    cu = torch.arange(N + 1, dtype=torch.int32, device="cuda")
    o_pre, S_pre = gdn.gdn_prefill(dr.q.cuda(), dr.k.cuda(), dr.v.cuda(), dr.g.cuda(), dr.beta.cuda(), cu,
                                   initial_state=S0.cuda())
    torch.cuda.synchronize()
    assert_close("o", np64(o_pre), np64(o_dec), 1e-2)
    assert_close("S", np64(S_pre), np64(state), 1e-2)


def test_prefill_then_decode_handoff():
    # prefill of T tokens followed by decode steps equals one prefill of T + steps tokens
    H, d, T, steps = 2, 128, 130, 3
    x = inputs.make_prefill_inputs([T + steps], H, d, d, dtype=torch.bfloat16, init_state=True, seed=12)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o, S = gdn.gdn_prefill(x.q[:T].contiguous(), x.k[:T].contiguous(), x.v[:T].contiguous(), x.g[:T].contiguous(),
                           x.beta[:T].contiguous(), cu, initial_state=x.initial_state)
    outs = [o]
    for t in range(T, T + steps):
        sl = lambda z: z[t:t + 1].contiguous()
        outs.append(gdn.gdn_decode(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), S))
    torch.cuda.synchronize()
    assert_close("o", np64(torch.cat(outs)), ref_o, 2e-2)
    assert_close("S", np64(S), ref_S, 2e-2)


def test_state_alloc_is_zeroed():
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    nbytes = gdn.gdn_state_bytes(3, 2, 64, 128)
    p = gdn.gdn_state_alloc(3, 2, 64, 128)
    torch.cuda.synchronize()
    try:
        host = (ctypes.c_char * nbytes)()
        assert hip.hipMemcpy(ctypes.addressof(host), ctypes.c_void_p(p), nbytes, 2) == 0  # device to host
        assert not any(bytes(host))
    finally:
        gdn.gdn_state_free(p)
        torch.cuda.synchronize()


# ---------------------------------------------------------------- gates from bf16 logits

LOGIT_GATES = [("pages", gdn.GDN_GATE_SCALED_SIGMOID, -5.0), ("amin", gdn.GDN_GATE_ALPHA_MIN, 0.9)]


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
@pytest.mark.parametrize("gate,kind,p", LOGIT_GATES)
def test_prefill_logits(gate, kind, p, dk, dv):
    # the log-decay computed in the kernel from bf16 logits; the oracle applies
    # its own fp64 parameterisation to the same logits
    lengths = [1, 63, 64, 65, 130, 0, 200]
    log(f"logits case lengths={lengths} H=3 dk={dk} dv={dv} gate={gate} p={p}")
    x = inputs.make_prefill_inputs(lengths, 3, dk, dv, dtype=torch.bfloat16, gate=gate, a_min=0.9, init_state=True,
                                   seed=6, logits=True)
    ref_o, ref_S = oracle_prefill(x, gate=(kind, p))
    to_device(x)
    o, S = gdn.gdn_prefill_logits(x.q, x.k, x.v, x.z, kind, p, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, TOL[torch.bfloat16])
    assert_close("final_state", np64(S), ref_S, TOL[torch.bfloat16])


@pytest.mark.parametrize("gate,kind,p", LOGIT_GATES)
def test_decode_logits(gate, kind, p):
    N, H, d, steps = 5, 3, 128, 4
    log(f"decode logits N={N} H={H} d={d} gate={gate}")
    S0, draws = inputs.make_decode_steps(N, H, d, d, steps, dtype=torch.bfloat16, gate=gate, a_min=0.9, seed=12,
                                         logits=True)
    ref_S = np64(S0)
    state = S0.cuda()
    for st, dr in enumerate(draws):
        g = oracle.gates_from_logits(np64(dr.z), kind, p)
        ref_o, ref_S = oracle.decode_step(np64(dr.q), np64(dr.k), np64(dr.v), g, np64(dr.beta), ref_S)
        o = gdn.gdn_decode_logits(dr.q.cuda(), dr.k.cuda(), dr.v.cuda(), dr.z.cuda(), kind, p, dr.beta.cuda(), state)
        torch.cuda.synchronize()
        assert_close(f"step {st} o", np64(o), ref_o, 1e-2)
    assert_close("state", np64(state), ref_S, 1e-5)


# ---------------------------------------------------------------- one gate per (token, head)

@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("gate", ["amin", "pages"])
def test_prefill_head_gate(gate, dk, dv):
    # the oracle runs the per-channel recurrence with the gate repeated over
    # the key channels (pinned against the scalar-gate recurrence on the CPU)
    lengths = [1, 63, 64, 65, 130, 0, 200]
    log(f"head-gate case lengths={lengths} H=3 dk={dk} dv={dv} gate={gate}")
    x = inputs.make_prefill_inputs(lengths, 3, dk, dv, dtype=torch.bfloat16, gate=gate, a_min=0.9, init_state=True,
                                   seed=7, head_gate=True)
    assert x.g.shape == (sum(lengths), 3)
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    o, S = gdn.gdn_prefill_head_gate(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, TOL[torch.bfloat16])
    assert_close("final_state", np64(S), ref_S, TOL[torch.bfloat16])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_head_gate(dtype):
    N, H, d, steps = 5, 3, 128, 4
    log(f"decode head gate N={N} H={H} d={d} {dtype}")
    S0, draws = inputs.make_decode_steps(N, H, d, d, steps, dtype=dtype, seed=13, head_gate=True)
    ref_S = np64(S0)
    state = S0.cuda()
    for st, dr in enumerate(draws):
        g = np.repeat(np64(dr.g)[:, :, None], d, axis=2)
        ref_o, ref_S = oracle.decode_step(np64(dr.q), np64(dr.k), np64(dr.v), g, np64(dr.beta), ref_S)
        o = gdn.gdn_decode_head_gate(dr.q.cuda(), dr.k.cuda(), dr.v.cuda(), dr.g.cuda(), dr.beta.cuda(), state)
        torch.cuda.synchronize()
        assert_close(f"step {st} o", np64(o), ref_o, 1e-5 if dtype == torch.float32 else 1e-2)
    assert_close("state", np64(state), ref_S, 1e-5)


def test_head_gate_endpoints_and_beta_extremes():
    # one gate per (token, head): exactly -5 on even 64-token blocks and 0 on
    # odd ones (a 32-token chunk at -5 spans e^-160, which underflows fp32 in
    # e^{G_t}: the true contribution lies far below bf16 resolution), beta in
    # {0, 1}, lengths {0, 1, 63, 64, 65, 300}
    lengths = [0, 1, 63, 64, 65, 300]
    H, d = 2, 128
    x = inputs.make_prefill_inputs(lengths, H, d, d, dtype=torch.bfloat16, init_state=True, seed=4, head_gate=True)
    cu = x.cu_seqlens.tolist()
    for n in range(len(lengths)):
        for t in range(cu[n], cu[n + 1]):
            x.g[t] = -5.0 if ((t - cu[n]) // 64) % 2 == 0 else 0.0
    x.beta.copy_((torch.arange(x.T_total)[:, None] + torch.arange(H)[None, :]) % 2 == 0)
    log(f"head-gate endpoints lengths={lengths}")
    ref_o, ref_S = oracle_prefill(x)
    to_device(x)
    o, S = gdn.gdn_prefill_head_gate(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state)
    torch.cuda.synchronize()
    assert_close("o", np64(o), ref_o, TOL[torch.bfloat16])
    assert_close("final_state", np64(S), ref_S, TOL[torch.bfloat16])
