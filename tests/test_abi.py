"""The C-ABI library on the host, without a GPU: it loads, exports every entry
point include/gdn.h declares, and rejects bad arguments with the documented
status codes before touching any memory or the device."""

import ctypes

import pytest

import gated_delta_rule_linear_amd as gdn

OK, INVALID, UNSUPPORTED, DOMAIN, OOM, HIPERR = range(6)
BAD = ctypes.c_void_p(0x1001)  # misaligned; never dereferenced because validation rejects it first
NUL = None


@pytest.fixture(scope="module")
def lib():
    return gdn.load_library()


def test_exports_every_declared_symbol(lib):
    names = gdn.exported_symbols_in_header()
    assert set(names) == {"gdn_status_string", "gdn_state_bytes", "gdn_state_alloc", "gdn_state_free",
                          "gdn_prefill_workspace_bytes", "gdn_prefill", "gdn_decode", "gdn_prefill_logits",
                          "gdn_decode_logits", "gdn_prefill_head_gate", "gdn_decode_head_gate",
                          "gdn_prefill_backward_workspace_bytes", "gdn_prefill_backward", "gdn_prefill_tiles",
                          "gdn_prefill_noalloc", "gdn_prefill_maxlen", "gdn_prefill_workspace_bytes_maxlen"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    seen = set()
    for code in range(7):
        s = gdn.gdn_status_string(code)
        assert s and s not in seen
        seen.add(s)
    assert gdn.gdn_status_string(99) == "unknown status"


def test_state_bytes():
    assert gdn.gdn_state_bytes(512, 32, 128, 128) == 512 * 32 * 128 * 128 * 4
    assert gdn.gdn_state_bytes(0, 32, 128, 128) == 0
    assert gdn.gdn_state_bytes(-1, 32, 128, 128) == 0
    # 2^62 * 32 * 128 * 128 * 4 = 2^83 bytes: saturates instead of wrapping to 0
    assert gdn.gdn_state_bytes(1 << 62, 32, 128, 128) == 2 ** 64 - 1


def _prefill(lib, q=NUL, cu=NUL, n=1, T=10, H=4, dk=64, dv=64, dt=1, o=NUL, S0=NUL, Sf=NUL, ws=NUL, wsb=0):
    return lib.gdn_prefill(q, q, q, q, q, cu, n, T, S0, Sf, o, H, dk, dv, dt, ws, wsb, None)


def test_prefill_argument_errors(lib):
    assert _prefill(lib) == INVALID                       # null pointers with T > 0
    assert _prefill(lib, dk=96) == UNSUPPORTED
    assert _prefill(lib, dv=32) == UNSUPPORTED
    assert _prefill(lib, dt=7) == UNSUPPORTED
    assert _prefill(lib, n=-1) == INVALID
    assert _prefill(lib, T=-5) == INVALID
    assert _prefill(lib, H=0) == INVALID
    assert _prefill(lib, n=0, T=3) == INVALID              # tokens but no sequence
    assert _prefill(lib, q=BAD, cu=BAD) == INVALID         # misaligned
    assert _prefill(lib, n=0, T=0) == OK                   # nothing to do, nothing touched


def test_decode_argument_errors(lib):
    def dec(p=NUL, N=4, H=2, dk=128, dv=128, dt=1):
        return lib.gdn_decode(p, p, p, p, p, p, p, N, H, dk, dv, dt, None)
    assert dec() == INVALID
    assert dec(dk=100) == UNSUPPORTED
    assert dec(dt=3) == UNSUPPORTED
    assert dec(N=-1) == INVALID
    assert dec(H=0) == INVALID
    assert dec(p=BAD) == INVALID
    assert dec(N=0) == OK


def test_state_alloc_argument_errors(lib):
    out = ctypes.c_void_p()
    assert lib.gdn_state_alloc(4, 2, 64, 64, None, None) == INVALID
    assert lib.gdn_state_alloc(4, 2, 48, 64, ctypes.byref(out), None) == UNSUPPORTED
    assert lib.gdn_state_alloc(-1, 2, 64, 64, ctypes.byref(out), None) == INVALID
    assert lib.gdn_state_alloc(0, 2, 64, 64, ctypes.byref(out), None) == OK and not out.value
    assert lib.gdn_state_free(None, None) == OK


def test_state_alloc_overflowing_size_is_oom_without_a_device_call(lib):
    # the size check comes before any HIP call, so this runs without a GPU
    out = ctypes.c_void_p(1234)
    assert lib.gdn_state_alloc(1 << 62, 32, 128, 128, ctypes.byref(out), None) == OOM
    assert not out.value
    assert lib.gdn_state_alloc((1 << 63) - 1, 1, 64, 64, ctypes.byref(out), None) == OOM


ORDER_TABLE_64 = 256  # int32 [64], rounded up to 256 bytes


def _al(x):
    return (x + 255) // 256 * 256


def _prefill_ws(T, n, H, dk, dv, seg):
    # the layout of gdn_prefill's workspace for segments of seg tokens (0: no
    # split): M and N slots of the T // seg non-last segments, the int32 table
    # [n + 1], the list of split sequences (at most min(n, T // (seg + 1))),
    # then the int32 order table [n] when it is kept
    b = 0
    if seg > 0:
        fs = T // seg
        b = _al(fs * H * dk * dk * 4) + _al(fs * H * dk * dv * 4) + _al((n + 1) * 4) + \
            _al(max(min(n, T // (seg + 1)), 1) * 4)
    if n > 1 and (seg > 0 or n * H > 256):
        b += _al(n * 4)
    return b


def _agnostic_seg(T, H):
    # the length-agnostic split of a batch with more units than compute units:
    # segments of T / (256 / H + 1) tokens, rounded up to a multiple of 64
    pmax = 256 // H + 1
    return (-(-T // pmax) + 63) // 64 * 64


def test_unit_order_table(monkeypatch):
    # the order table (int32 [num_seqs], 256-byte rounded) is kept when the split
    # runs with more than one sequence, or when (sequence, head) units outnumber
    # the 256 compute units; a single sequence or a batch that starts at once has none
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "0")
    assert gdn.gdn_prefill_workspace_bytes(10000, 8, 32, 128, 128) == 0      # 256 units
    assert gdn.gdn_prefill_workspace_bytes(10000, 9, 32, 128, 128) == 256    # 288 units
    assert gdn.gdn_prefill_workspace_bytes(10 ** 6, 65, 32, 128, 128) == 512  # int32 [65]
    assert gdn.gdn_prefill_workspace_bytes(10 ** 6, 1, 512, 128, 128) == 0   # one sequence
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "1024")
    one = gdn.gdn_prefill_workspace_bytes(4096, 1, 2, 64, 64)
    assert gdn.gdn_prefill_workspace_bytes(4096, 2, 2, 64, 64) == one + 256


def test_workspace_bound_needs_no_lengths():
    # the bound is a function of the arguments alone
    a = gdn.gdn_prefill_workspace_bytes(65536, 1, 32, 128, 128)
    b = gdn.gdn_prefill_workspace_bytes(65536, 1, 32, 128, 128)
    assert a == b and a >= 0


def test_time_split_plan(monkeypatch):
    monkeypatch.delenv("GDN_PREFILL_SEGMENT", raising=False)
    # one 65,536-token sequence x 32 heads: 32 workgroups would leave most CUs idle -> split
    assert gdn.gdn_prefill_workspace_bytes(65536, 1, 32, 128, 128) > 0
    # 64 sequences of ~8K tokens x 32 heads: 2048 workgroups already, so sequences of the
    # mean length need no split; the length-agnostic plan splits any sequence longer than
    # 540000 / 9 tokens (none, if the lengths are near the mean)
    assert _agnostic_seg(540000, 32) == 60032
    assert gdn.gdn_prefill_workspace_bytes(540000, 64, 32, 128, 128) == _prefill_ws(540000, 64, 32, 128, 128, 60032)
    # ... but not when the segment would be shorter than 16,384 tokens
    assert gdn.gdn_prefill_workspace_bytes(100000, 64, 32, 128, 128) == ORDER_TABLE_64
    # nor with more than 128 heads (fewer than three segments), nor for one sequence
    assert gdn.gdn_prefill_workspace_bytes(10 ** 7, 4, 256, 64, 64) == _al(4 * 4)
    assert gdn.gdn_prefill_workspace_bytes(540000, 1, 512, 64, 64) == 0
    # short sequences are never split
    assert gdn.gdn_prefill_workspace_bytes(256, 1, 2, 64, 64) == 0
    assert gdn.gdn_prefill_workspace_bytes(0, 3, 2, 64, 64) == 0


def test_time_split_plan_with_a_bound_on_the_lengths(monkeypatch):
    monkeypatch.delenv("GDN_PREFILL_SEGMENT", raising=False)
    # one 262,144-token sequence among 63 of 1,024 tokens, 32 heads: 2,048 units, so the
    # mean-length plan does not split; the bound on the lengths cuts the long sequence
    T, n, H = 262144 + 63 * 1024, 64, 32
    assert gdn.gdn_prefill_workspace_bytes(T, n, H, 128, 128) == _prefill_ws(T, n, H, 128, 128, _agnostic_seg(T, H))
    assert gdn.gdn_prefill_workspace_bytes_maxlen(T, n, 262144, H, 128, 128) > ORDER_TABLE_64
    # a bound of 0 is gdn_prefill's plan; balanced batches plan as without a bound
    for args in ((65536, 1, 32), (32768, 4, 32), (540000, 64, 32), (T, n, H)):
        assert gdn.gdn_prefill_workspace_bytes_maxlen(args[0], args[1], 0, args[2], 128, 128) == \
            gdn.gdn_prefill_workspace_bytes(*args, 128, 128)
    assert gdn.gdn_prefill_workspace_bytes_maxlen(32768, 4, 8192, 32, 128, 128) == \
        gdn.gdn_prefill_workspace_bytes(32768, 4, 32, 128, 128)
    # uniform lengths up to the bound: nothing to gain from a split
    assert gdn.gdn_prefill_workspace_bytes_maxlen(540000, 64, 16384, 32, 128, 128) == ORDER_TABLE_64
    assert gdn.gdn_prefill_workspace_bytes_maxlen(T, n, -1, H, 128, 128) == 0


def test_maxlen_argument_errors(lib):
    p = ctypes.c_void_p(0x10000)
    st = lib.gdn_prefill_maxlen(p, p, p, p, p, p, 1, 10, -1, None, None, p, 4, 64, 64, 1, None, 0, None)
    assert st == INVALID


def test_time_split_workspace_layout(monkeypatch):
    # forced 8192-token segments: 8 full segments -> at most 8 non-last ones per
    # 65,536 tokens; each (slot, head) holds M (d_k x d_k) and N (d_k x d_v) in
    # fp32, each area rounded up to 256 bytes, then the int32 table [n + 1] and,
    # with more than one sequence, the int32 order table [n]
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "8192")
    assert gdn.gdn_prefill_workspace_bytes(65536, 1, 32, 128, 64) == \
        8 * 32 * 128 * 128 * 4 + 8 * 32 * 128 * 64 * 4 + 256 + 256
    assert gdn.gdn_prefill_workspace_bytes(65535, 3, 2, 64, 64) == 7 * 2 * 64 * 64 * 4 * 2 + 256 + 256 + 256
    for args in ((65536, 1, 32, 128, 64), (65535, 3, 2, 64, 64), (10 ** 6, 300, 1, 64, 64)):
        assert gdn.gdn_prefill_workspace_bytes(*args) == _prefill_ws(*args, 8192)
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "100")  # rounded up to 128
    assert gdn.gdn_prefill_workspace_bytes(1000, 1, 1, 64, 64) == 7 * 64 * 64 * 4 * 2 + 256 + 256
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "0")
    assert gdn.gdn_prefill_workspace_bytes(65536, 1, 32, 128, 128) == 0


def test_short_workspace_rejected(lib, monkeypatch):
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "64")
    p = ctypes.c_void_p(0x10000)  # aligned; never dereferenced because validation rejects the call first
    need = gdn.gdn_prefill_workspace_bytes(1000, 1, 2, 64, 64)
    assert need > 0
    assert _prefill(lib, q=p, cu=p, o=p, T=1000, H=2, ws=NUL, wsb=0) == INVALID
    assert _prefill(lib, q=p, cu=p, o=p, T=1000, H=2, ws=p, wsb=need - 1) == INVALID


def _prefill_logits(lib, gate=1, p=-5.0, q=NUL, cu=NUL, n=1, T=10, H=4, dk=64, dv=64, dt=1):
    return lib.gdn_prefill_logits(q, q, q, q, gate, p, q, cu, n, T, NUL, NUL, q, H, dk, dv, dt, NUL, 0, None)


def _decode_logits(lib, gate=1, p=-5.0, q=NUL, cu=NUL, N=2, H=4, dk=64, dv=64, dt=1):
    return lib.gdn_decode_logits(q, q, q, q, gate, p, q, q, q, N, H, dk, dv, dt, None)


def test_logit_gate_argument_errors(lib):
    # gate kind, then its parameter's range (g must stay in [-5, 0]), then the
    # dtype (bf16 only), all before any pointer is looked at
    for f in (_prefill_logits, _decode_logits):
        assert f(lib, gate=0) == INVALID                    # GDN_GATE_LOG is not a logit gate
        assert f(lib, gate=3) == INVALID
        assert f(lib, gate=1, p=-5.5) == DOMAIN             # g_min below -5
        assert f(lib, gate=1, p=0.5) == DOMAIN              # g_min above 0
        assert f(lib, gate=2, p=0.005) == DOMAIN            # a_min below e^-5
        assert f(lib, gate=2, p=1.5) == DOMAIN
        assert f(lib, gate=1, p=float("nan")) == DOMAIN
        assert f(lib, gate=1, p=-5.0, dt=0) == UNSUPPORTED  # fp32 inputs
        assert f(lib, gate=2, p=0.9) == INVALID             # valid gate, then null pointers
        assert f(lib, gate=1, p=-5.0, q=BAD, cu=BAD) == INVALID
    assert _prefill_logits(lib, n=0, T=0) == OK
    assert _decode_logits(lib, N=0) == OK


def test_head_gate_argument_errors(lib):
    P = ctypes.c_void_p(0x10000)  # aligned; never dereferenced because validation rejects the call first
    pre = lambda q=NUL, g=NUL, dt=1, n=1, T=10: lib.gdn_prefill_head_gate(q, q, q, g, q, q, n, T, NUL, NUL, q, 4, 64,
                                                                         64, dt, NUL, 0, None)
    dec = lambda q=NUL, g=NUL, dt=1, N=2: lib.gdn_decode_head_gate(q, q, q, g, q, q, q, N, 4, 64, 64, dt, None)
    assert pre(dt=0) == UNSUPPORTED            # prefill: bf16 only
    assert pre() == INVALID                    # null pointers
    assert pre(q=P, g=NUL) == INVALID          # null gates
    assert pre(q=P, g=ctypes.c_void_p(0x10002)) == INVALID  # gates misaligned
    assert pre(n=0, T=0) == OK
    assert dec() == INVALID
    assert dec(q=P, g=NUL) == INVALID
    assert dec(N=0) == OK


def _backward(lib, p=NUL, cu=NUL, n=1, T=10, H=4, dk=64, dv=64, dt=1, ws=NUL, wsb=0):
    return lib.gdn_prefill_backward(p, p, p, p, p, cu, n, T, NUL, p, NUL, p, p, p, p, p, NUL, H, dk, dv, dt, ws, wsb,
                                    None)


def test_backward_workspace_bytes(lib):
    f = lib.gdn_prefill_backward_workspace_bytes
    # one state per 16-token sub-chunk and head, in the input dtype
    assert f(1024, 2, 4, 128, 128, 1) == (1024 // 16 + 2) * 4 * 128 * 128 * 2
    assert f(1000, 3, 2, 64, 128, 0) == (1000 // 16 + 3) * 2 * 64 * 128 * 4
    assert f(-1, 1, 1, 64, 64, 1) == 0
    assert f(16, 1, 1, 64, 64, 9) == 0


def _backward_ws(T, n, H, dk, dv, bf16, seg):
    # checkpoints, then with a time split of segment length seg the forward
    # pass's split workspace (M, N of the T // seg non-last segment slots, the
    # segment table, the split list) and one d_k x d_v fp32 gradient per segment slot; without
    # it, the int32 order table [n] when more than one sequence gives more
    # (sequence, head) units than the 256 compute units
    al = lambda x: (x + 255) // 256 * 256
    ck = al((T // 16 + n) * H * dk * dv * (2 if bf16 else 4))
    if seg == 0:
        return ck + (al(n * 4) if n > 1 and n * H > 256 else 0)
    fs = T // seg
    pre = al(fs * H * dk * dk * 4) + al(fs * H * dk * dv * 4) + al((n + 1) * 4) + al(max(min(n, T // (seg + 1)), 1) * 4)
    # bf16 with d_k = d_v (the reverse maps' offsets from the transition pass): the last
    # segment's d_k x d_k fp32 transition per split-list entry and head, and the bf16
    # q^ buffer [T, H, d_k]
    qmaps = al(min(n, T // (seg + 1)) * H * dk * dk * 4) + al(T * H * dk * 2) if bf16 and dk == dv else 0
    # with more than one sequence, the order table [n] and the segment prefix table [n + 1]
    order = al(n * 4) + al((n + 1) * 4) if n > 1 else 0
    return ck + al(pre) + al((T // seg + n) * H * dk * dv * 4) + qmaps + order


def test_backward_workspace_bytes_split(lib, monkeypatch):
    f = lib.gdn_prefill_backward_workspace_bytes
    monkeypatch.delenv("GDN_BACKWARD_SEGMENT", raising=False)
    # few (sequence, head) units over long sequences: segments for about 512 workgroups
    assert f(32768, 4, 32, 128, 128, 1) == _backward_ws(32768, 4, 32, 128, 128, True, 2048)
    assert f(65536, 1, 16, 128, 128, 1) == _backward_ws(65536, 1, 16, 128, 128, True, 2048)
    assert f(1 << 20, 1, 16, 128, 128, 1) == _backward_ws(1 << 20, 1, 16, 128, 128, True, 32768)
    # enough units to fill the chip, or sequences too short for three segments: no split
    assert f(65536, 8, 32, 128, 128, 1) == _backward_ws(65536, 8, 32, 128, 128, True, 0)
    # more units than compute units: the length-agnostic split (sequences longer than
    # T / (256 / H + 1) tokens are cut), when that segment is at least 16,384 tokens
    T = 262144 + 63 * 1024
    assert f(T, 64, 32, 128, 128, 1) == _backward_ws(T, 64, 32, 128, 128, True, _agnostic_seg(T, 32))
    assert f(100000, 64, 32, 128, 128, 1) == _backward_ws(100000, 64, 32, 128, 128, True, 0)
    assert f(65536, 9, 32, 128, 128, 1) == _backward_ws(65536, 9, 32, 128, 128, True, 0)
    assert _backward_ws(65536, 9, 32, 128, 128, True, 0) == _backward_ws(65536, 8, 32, 128, 128, True, 0) \
        + 32 * 128 * 128 * 2 + 256  # one more sequence's checkpoint slot per head, and the order table
    assert f(1024, 4, 32, 128, 128, 1) == _backward_ws(1024, 4, 32, 128, 128, True, 0)
    # forced length, rounded up to a multiple of 64; 0 turns the split off
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "200")
    assert f(1000, 3, 2, 64, 128, 0) == _backward_ws(1000, 3, 2, 64, 128, False, 256)
    monkeypatch.setenv("GDN_BACKWARD_SEGMENT", "0")
    assert f(32768, 4, 32, 128, 128, 1) == _backward_ws(32768, 4, 32, 128, 128, True, 0)


def test_backward_argument_errors(lib):
    assert _backward(lib) == INVALID                      # null pointers with T > 0
    assert _backward(lib, dk=96) == UNSUPPORTED
    assert _backward(lib, dv=32) == UNSUPPORTED
    assert _backward(lib, dt=7) == UNSUPPORTED
    assert _backward(lib, n=-1) == INVALID
    assert _backward(lib, H=0) == INVALID
    assert _backward(lib, n=0, T=3) == INVALID
    assert _backward(lib, p=BAD, cu=BAD) == INVALID       # misaligned
    assert _backward(lib, n=0, T=0) == OK                 # nothing to do


def _tiles(lib, p=NUL, cu=NUL, n=1, T=10, H=4, dk=64, dv=64, dt=1, path=0):
    return lib.gdn_prefill_tiles(p, p, p, p, p, cu, n, T, NUL, NUL, p, H, dk, dv, dt, path, None)


def test_tiles_argument_errors(lib):
    assert _tiles(lib) == INVALID                         # null pointers with T > 0
    assert _tiles(lib, path=2) == INVALID                 # unknown tile path
    assert _tiles(lib, dk=96) == UNSUPPORTED
    assert _tiles(lib, dt=7) == UNSUPPORTED
    assert _tiles(lib, H=0) == INVALID
    assert _tiles(lib, p=BAD, cu=BAD, path=1) == INVALID  # misaligned
    assert _tiles(lib, n=0, T=0, path=1) == OK


def test_noalloc_rejects_a_call_beyond_its_scratch(lib, monkeypatch):
    # 2^22 tokens in 64-token segments x 32 heads: the split maps need far more than the fixed
    # scratch, so the call is refused before any device call (the pointers are never read)
    monkeypatch.setenv("GDN_PREFILL_SEGMENT", "64")
    T, n, H = 1 << 22, 1, 32
    assert gdn.gdn_prefill_workspace_bytes(T, n, H, 128, 128) > gdn.GDN_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(0x10000)
    st = lib.gdn_prefill_noalloc(p, p, p, p, p, p, n, T, None, p, p, H, 128, 128, 1, None)
    assert st == gdn.GDN_ERR_SCRATCH_LIMIT
    assert "scratch" in gdn.gdn_status_string(st)
    assert lib.gdn_prefill_noalloc(p, p, p, p, p, p, -1, T, None, p, p, H, 128, 128, 1, None) == INVALID
