"""Throughput of the gated delta rule on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one gdn_prefill call over the prefill workload: one sequence of
65,536 tokens, 32 heads, d_k = d_v = 128, bf16 q/k/v, fp32 gates
(alpha = 0.9 + 0.1 sigmoid(N(0,1))), zero initial state, final state written.
W untimed steps, then exactly K steps bracketed by device synchronisation and
timed with HIP events on the stream the kernels run on.  `value` is tokens per
second of that workload.

The decode step (512 sequences x 32 heads, one token each, fp32 state updated
in place) is timed in the same run over K calls and reported under "decode"
as achieved HBM bandwidth.

"roofline" prices one gdn_prefill call against MI355X's 8 TB/s HBM with the
algorithmic bytes of the layer (q, k, v, o in bf16, g and beta in fp32, the
final state).  The call is a short sequence of kernels on one stream (for this
workload: segment table, segment transitions, fold, replay of every segment);
its duration is measured with HIP events around the calls on that stream.
"traffic" is the HBM bytes the rocprofv3 counters FETCH_SIZE and WRITE_SIZE
read for those kernels, scaled by what the same counters read for a plain
copy of known size (profiles/traffic.json; null when the kernel sources have
changed since).  "cpu_baseline" is the fp32 oracle on the host cores over the
same workload.  One JSON line is printed.

    python bench.py --copy-calibration 1073741824

runs only a device-to-device copy of that many bytes (three times), the
reference for scaling the counters.

    python bench.py --summarize-pmc <dir>/bench_counter_collection.csv ...

summarises rocprofv3 --pmc output per kernel and grid (matrix-core and VALU
busy, LDS bank conflicts, instruction counts, clock) without a GPU.

Two more legs follow in the same run, each on four 8,192-token sequences x
32 heads and reported in objects of their own: "tile_paths" times
gdn_prefill_tiles with dense window products and with position-pair decays
(the diagonal-tile comparison), and "backward" times gdn_prefill_backward
with its own roofline, sampled parity and host-oracle baseline.
--no-tiles / --no-backward skip them.

"gate_variants" times the gate forms of NEXT f1 (bf16 logits, gate computed in the
kernel) and f4 (one log-decay per (token, head)) on the prefill_64k and decode
shapes, with their rooflines and sampled parity.  --no-gates skips them.

"workloads" times gdn_prefill on the other prefill shapes: 64 packed
sequences of 512..16,384 tokens with random initial states (varlen64), one
2^20-token sequence x 16 heads (long_1m), and a skewed batch of 63 sequences
of 1,024 tokens plus one of 262,144 (skewed64, with and without the bound on
the lengths of gdn_prefill_maxlen), each with its roofline, sampled parity and
a host-oracle baseline on a stated sample, after --workload-warmup (10)
untimed calls; and gdn_prefill_backward on varlen64 and skewed64
(varlen64_backward, skewed64_backward) with its roofline and sampled parity.  --no-workloads skips them.  "device" gives
the GPU's compute-unit count and clock as the runtime reports them, beside
the published peaks the fractions use.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (H=32,d=128,T=64K bf16) + decode HBM GB/s; % of roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published (no sparsity)
KERNEL_SOURCES = ["gdn_prefill.hip", "gdn_decode.hip", "gdn_mfma.h", "gdn_device.h", "gdn_api.cpp", "gdn_kernels.h",
                  "gdn_fold.h", "gdn_segunit.h"]
BACKWARD_SOURCES = ["gdn_backward.hip", "gdn_backward.h", "gdn_tile16.h", "gdn_mfma.h", "gdn_device.h",
                    "gdn_api_backward.cpp", "gdn_prefill.hip", "gdn_kernels.h", "gdn_fold.h", "gdn_segunit.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
BF16_CHUNK = 32  # the bf16 prefill kernel's chunk length (tokens)
# dense bf16 matrix-core flops per clock and CU on CDNA4: the published 2.5 PFLOP/s
# at 256 CUs and 2.4 GHz (2.5e15 / (256 * 2.4e9) = 4069, i.e. 2048 FMA)
BF16_FLOP_PER_CLK_CU = 4096


def prefill_bytes(T_tokens: int, H: int, dk: int, dv: int, n_seqs: int, elt: int = 2, init_state: bool = False,
                  gate_bytes=None):
    """Algorithmic HBM bytes of one prefill launch: every input read once, every output written once
    (gate_bytes per (token, head): 4 d_k for fp32 per-channel log-decays by default; 2 d_k for bf16
    logits, 4 for one log-decay per (token, head))."""
    per_head_token = elt * (2 * dk + dv) + (4 * dk if gate_bytes is None else gate_bytes) + 4 + elt * dv
    states = n_seqs * H * dk * dv * 4 * (2 if init_state else 1)
    return T_tokens * H * per_head_token + states


def prefill_flops(T_tokens: int, H: int, dk: int, dv: int, C: int = BF16_CHUNK):
    """Algorithmic flops of one prefill launch with the causal intra-chunk tiles counted dense:
    three d_k x d_v state contractions per token (Q~S, W S, K_dec^T U), the two Gram products and
    the P U and W, U~ products inside the chunk, and the C^3/3 triangular solve spread over C tokens."""
    per = 6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3
    return T_tokens * H * per


def backward_bytes(T_tokens: int, H: int, dk: int, dv: int, n_seqs: int, elt: int = 2, init_state: bool = False,
                   d_final: bool = True):
    """Algorithmic HBM bytes of one backward launch: q, k, v, dL/do, g, beta read once; dq, dk, dv, dg,
    dbeta written once; per (sequence, head) the initial state and dL/d(final state) read and the initial
    state's gradient written.  (The checkpoints the kernels keep are the implementation's, not counted.)"""
    per_head_token = elt * (2 * dk + 2 * dv) + 4 * dk + 4 + elt * (2 * dk + dv) + 4 * dk + 4
    states = n_seqs * H * dk * dv * 4 * (1 + (1 if init_state else 0) + (1 if d_final else 0))
    return T_tokens * H * per_head_token + states


def backward_flops(T_tokens: int, H: int, dk: int, dv: int, C: int = 16):
    """Matrix-core flops of one backward launch as the kernels form it, per 16-token sub-chunk: nine
    state-sized products (forward replay k~ S and k^T U; in the gradient pass k~ S, k^ dS, q~^T dO,
    k~^T dR, and the three key-channel products with the state rows) and twelve token-pair products
    (16 x 16 over d_k or d_v, or over the 16 tokens), spread over C tokens."""
    per = 9 * 2 * dk * dv + 12 * 2 * C * max(dk, dv)
    return T_tokens * H * per


def decode_bytes(N: int, H: int, dk: int, dv: int, elt: int = 2, gate_bytes=None):
    """Algorithmic HBM bytes of one decode launch: state read and written, token vectors read, o written
    (gate_bytes as for prefill_bytes)."""
    per = 8 * dk * dv + elt * (2 * dk + dv) + (4 * dk if gate_bytes is None else gate_bytes) + 4 + elt * dv
    return N * H * per


def source_hash(files=None) -> str:
    h = hashlib.sha256()
    for f in files or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_linear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def device_info():
    """The GPU as the runtime reports it: name, architecture, compute units, peak
    engine clock (rocminfo), memory; and the dense bf16 matrix peak those imply."""
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count,
            "hbm_bytes": props.total_memory, "max_clock_mhz": None}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=120).stdout
        arch = props.gcnArchName.split(":")[0]
        for block in out.split("*******"):
            if re.search(rf"Name:\s+{arch}\b", block):
                m = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", block)
                if m:
                    info["max_clock_mhz"] = int(m.group(1))
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if info["max_clock_mhz"]:
        info["bf16_mfma_peak_tflops_from_cus_and_clock"] = (
            info["compute_units"] * info["max_clock_mhz"] * 1e6 * BF16_FLOP_PER_CLK_CU / 1e12)
    info["published_peaks"] = {"hbm_gbs": HBM_PEAK_GBS, "bf16_mfma_tflops": MFMA_BF16_PEAK_TFLOPS}
    return info


def measured_counters(kernel: str):
    """Matrix-core and VALU busy fractions of `kernel` from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_hash") != source_hash():
        return None
    return {k: v for k, v in e.items() if k != "source_hash"}


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_hash") != source_hash(BACKWARD_SOURCES if kernel == "backward" else None):
        return None
    return e.get("bytes_per_launch")


def time_loop(fn, steps: int, warmup: int, stream):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per call


def summarize_pmc(paths):
    """Per (kernel, grid size): mean duration and counters of a rocprofv3 --pmc
    run (counter_collection.csv files), with MI355X's derived figures:
    matrix-core busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x
    1024 SIMDs); VALU busy = SQ_ACTIVE_INST_VALU / (256 CUs x GRBM_GUI_ACTIVE per
    XCD); LDS bank-conflict share = SQ_LDS_BANK_CONFLICT / (256 x the same);
    GRBM_GUI_ACTIVE is summed over the 8 XCDs in the CSV, so it is divided by 8;
    clock = those cycles / duration."""
    import csv
    import collections

    def short(n):
        m = re.search(r"(prefill_ws_kernel|prefill_seq_kernel|seg_fold_kernel|seg_table_kernel|decode_kernel|"
                      r"bwd_\w+_kernel|tile_prefill_kernel|seq_order_kernel)", n)
        if not m:
            return n[:40]
        k = m.group(0)
        if k in ("prefill_ws_kernel", "prefill_seq_kernel"):  # transition maps or outputs (template MAP)
            k += "<map" if re.search(r"kernelILi\d+ELi\d+ELb1", n) else "<out"
            gm = re.search(r"prefill_ws_kernelILi\d+ELi\d+ELb[01]ELi\d+ELi(\d)E", n)  # gate mode
            k += {"1": ",logits", "2": ",head gate"}.get(gm.group(1), "") if gm else ""
            k += ",q^" if re.search(r"prefill_ws_kernelILi\d+ELi\d+ELb1ELi2ELi0ELb1E", n) else ""  # backward's maps
            k += ",checkpoints" if re.search(r"prefill_ws_kernelILi\d+ELi\d+ELb1ELi1ELi0ELb0ELb1E", n) else ""
            k += ">"
        elif k == "bwd_grad_kernel":  # adjoint only or full (template DONLY)
            k += "<adjoint-only>" if re.search(r"ELb1EE", n) else "<full>"
        return k

    per = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                k = (short(r["Kernel_Name"]), int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
                per[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
                dur[k][(p, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = {}
    for k in sorted(per, key=lambda k: -sum(dur[k].values())):
        c = {n: sum(v) / len(v) for n, v in per[k].items()}
        ns = sum(dur[k].values()) / len(dur[k])
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / 8
        e = {"dispatches": len(dur[k]), "mean_us": ns / 1e3, "clock_ghz": cyc / ns if ns else None}
        if cyc:
            for name, ctr, den in (("mfma_busy", "SQ_VALU_MFMA_BUSY_CYCLES", 1024), ("valu_busy", "SQ_ACTIVE_INST_VALU", 256),
                                   ("lds_bank_conflict", "SQ_LDS_BANK_CONFLICT", 256)):
                if ctr in c:
                    e[name] = c[ctr] / (den * cyc)
        for n in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAVES"):
            if n in c:
                e[n] = c[n]
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            e["mfma_bf16_flops"] = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        out[f"{k[0]} workgroups={k[1]}"] = e
    print(json.dumps(out, indent=1))


def copy_calibration(nbytes: int):
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "calls": 3}), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        return ""


def cpu_baseline(x, n_seqs: int, what: str):
    """fp32 oracle on the host over the first `n_seqs` sequences of x (every head):
    tokens/s of that sample."""
    import oracle

    oracle.build(force=False)
    H = x.q.shape[1]
    cu = x.cu_seqlens[:n_seqs + 1].to("cpu", torch.int64).numpy()
    tokens = int(cu[-1])
    sl = lambda t: t[:tokens].to("cpu", torch.float32).numpy()
    S0 = None if x.initial_state is None else x.initial_state[:n_seqs].to("cpu", torch.float32).numpy()
    units = n_seqs * H
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    threads = max(1, min(os.cpu_count() or 1, units, share))
    t0 = time.perf_counter()
    oracle.recurrent(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), cu.astype(np.int32), initial_state=S0,
                     dtype=np.float32, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}: {tokens} tokens x {H} heads, fp32 sequential recurrence (OpenMP over "
                      f"(sequence, head) units), {dt:.2f} s wall; host {_cpu_model() or 'unknown CPU'}, "
                      f"{os.cpu_count()} logical CPUs visible"}


def prefix_view(x, tokens: int):
    """The first `tokens` tokens of a one-sequence workload, as a one-sequence workload."""
    from gated_delta_rule_linear_amd.inputs import PrefillInputs

    cu = torch.tensor([0, tokens], dtype=torch.int32)
    return PrefillInputs(x.q[:tokens], x.k[:tokens], x.v[:tokens], x.g[:tokens], x.beta[:tokens], cu, [tokens],
                         x.initial_state, None)


def prefill_leg(gdn, name, x, steps, warmup, stream, cpu: bool, cpu_seqs: int, cpu_what: str, cpu_x=None,
                max_seqlen: int = 0):
    """Time gdn_prefill over the workload x (every output written, final state included;
    max_seqlen > 0: gdn_prefill_maxlen with that bound); sampled parity of sequence 0,
    head 0 (first 2048 tokens) against the fp64 oracle."""
    import oracle

    T, H, dk = x.q.shape
    dv = x.v.shape[2]
    n = x.num_seqs
    o = torch.empty((T, H, dv), dtype=x.q.dtype, device=x.q.device)
    S = torch.empty((n, H, dk, dv), dtype=torch.float32, device=x.q.device)
    ws_bytes = gdn.gdn_prefill_workspace_bytes(T, n, H, dk, dv, max_seqlen)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.q.device) if ws_bytes else None

    def step():
        gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, initial_state=x.initial_state, final_state=S,
                        o=o, workspace=ws, stream=stream, max_seqlen=max_seqlen)

    ms = time_loop(step, steps, warmup, stream)
    init = x.initial_state is not None
    pbytes = prefill_bytes(T, H, dk, dv, n, init_state=init)
    pflops = prefill_flops(T, H, dk, dv)
    gbs = pbytes / (ms / 1e3) / 1e9
    cu = x.cu_seqlens.to("cpu", torch.int64).numpy()
    tk = int(min(2048, cu[1]))
    s0 = None if not init else x.initial_state[:1, :1].to("cpu", torch.float64).numpy()
    ro, _ = oracle.recurrent(*(t[:tk, :1].to("cpu", torch.float64).numpy() for t in (x.q, x.k, x.v, x.g)),
                             x.beta[:tk, :1].to("cpu", torch.float64).numpy(), np.array([0, tk], np.int32),
                             initial_state=s0)
    leg = {"workload": name, "num_seqs": n, "T": T, "H": H, "d_k": dk, "d_v": dv, "initial_state": init,
           "max_seqlen_hint": max_seqlen, "workspace_bytes": ws_bytes, "steps": steps, "warmup": warmup,
           "ms_per_step": ms,
           "tokens_per_s": T / (ms / 1e3),
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": pbytes},
           "mfma": {"algorithmic_flops_per_launch": pflops, "chunk": BF16_CHUNK,
                    "frac": pflops / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
           "parity": {"o_rel_err_seq0_head0_first_tokens": oracle.rel_err(
               o[:tk, :1].to("cpu", torch.float64).numpy(), ro), "tokens": tk}}
    del o, S, ws
    if cpu:
        leg["cpu_baseline"] = cpu_baseline(cpu_x if cpu_x is not None else x, cpu_seqs, cpu_what)
    return leg


def gate_variants_leg(gdn, inputs, x, o, S, ws, N, Hd, d, steps, warmup, stream):
    """gdn_prefill_logits (GDN_GATE_ALPHA_MIN, a_min = 0.9, on bf16 logits) and
    gdn_prefill_head_gate on the prefill_64k shape (same q, k, v, beta, same plan and
    workspace), and gdn_decode_logits / gdn_decode_head_gate on the decode shape: time,
    algorithmic bytes, roofline; sampled parity of the prefill variants (head 0, first
    2048 tokens) against the fp64 oracle with its own gate parameterisation."""
    import oracle

    T, H, dk = x.q.shape
    dv = x.v.shape[2]
    gen = torch.Generator(device=x.q.device)
    gen.manual_seed(7)
    # logits z ~ N(0,1) in bf16: the kernel computes g = log(0.9 + 0.1 sigmoid(z)) per channel
    z = torch.randn((T, H, dk), generator=gen, device=x.q.device).to(torch.bfloat16)
    # one log-decay per (token, head) in [-5, 0]
    gh = (-5.0 * torch.sigmoid(torch.randn((T, H), generator=gen, device=x.q.device))).float()
    tk = 2048
    sl = lambda t: t[:tk, :1].to("cpu", torch.float64).numpy()
    res = {"workload": "prefill_64k and decode_512x32 with the other gate forms", "steps": steps, "warmup": warmup}

    def prefill_variant(name, call, gbytes, g_ref):
        ms = time_loop(call, steps, warmup, stream)
        b = prefill_bytes(T, H, dk, dv, 1, gate_bytes=gbytes)
        ro, _ = oracle.recurrent(sl(x.q), sl(x.k), sl(x.v), g_ref, sl(x.beta), np.array([0, tk], np.int32))
        gbs = b / (ms / 1e3) / 1e9
        res[name] = {"ms_per_step": ms, "tokens_per_s": T / (ms / 1e3), "algorithmic_bytes_per_launch": b,
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": gbs / HBM_PEAK_GBS},
                     "parity_o_rel_err_head0_first2048": oracle.rel_err(o[:tk, :1].to("cpu", torch.float64).numpy(),
                                                                         ro)}

    prefill_variant("prefill_logits",
                    lambda: gdn.gdn_prefill_logits(x.q, x.k, x.v, z, gdn.GDN_GATE_ALPHA_MIN, 0.9, x.beta, x.cu_seqlens,
                                                   final_state=S, o=o, workspace=ws, stream=stream),
                    2 * dk, oracle.gates_from_logits(sl(z), oracle.GATE_ALPHA_MIN, 0.9))
    prefill_variant("prefill_head_gate",
                    lambda: gdn.gdn_prefill_head_gate(x.q, x.k, x.v, gh, x.beta, x.cu_seqlens, final_state=S, o=o,
                                                      workspace=ws, stream=stream),
                    4, np.repeat(gh[:tk, :1].to("cpu", torch.float64).numpy()[:, :, None], dk, axis=2))
    del z, gh
    for name, kw, gbytes in (("decode_logits", {"logits": True}, 2 * dk), ("decode_head_gate", {"head_gate": True}, 4)):
        S0, draws = inputs.make_decode_steps(N, Hd, d, d, max(1, min(steps + warmup, 32)), dtype=torch.bfloat16,
                                             seed=0, device=x.q.device, **kw)
        st = S0.contiguous()
        od = torch.empty((N, Hd, d), dtype=torch.bfloat16, device=x.q.device)
        it = [0]

        def dstep():
            dr = draws[it[0] % len(draws)]
            it[0] += 1
            if name == "decode_logits":
                gdn.gdn_decode_logits(dr.q, dr.k, dr.v, dr.z, gdn.GDN_GATE_ALPHA_MIN, 0.9, dr.beta, st, o=od,
                                      stream=stream)
            else:
                gdn.gdn_decode_head_gate(dr.q, dr.k, dr.v, dr.g, dr.beta, st, o=od, stream=stream)

        ms = time_loop(dstep, steps, warmup, stream)
        b = decode_bytes(N, Hd, d, d, gate_bytes=gbytes)
        gbs = b / (ms / 1e3) / 1e9
        res[name] = {"ms_per_step": ms, "algorithmic_bytes_per_launch": b,
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": gbs / HBM_PEAK_GBS}}
        del S0, draws, st, od
    return res


def backward_leg(gdn, name, x, steps, warmup, stream):
    """Time gdn_prefill_backward over the workload x (every gradient written, the initial
    state's included; dL/do ~ N(0,1), dL/d(final state) ~ 0.02 N(0,1)); sampled parity of
    sequence 0, head 0 (its whole length) against the fp64 oracle."""
    import oracle
    from gated_delta_rule_linear_amd import inputs

    T, H, dk = x.q.shape
    dv = x.v.shape[2]
    n = x.num_seqs
    d_o, dSf = inputs.make_cotangents(T, n, H, dk, dv, dtype=x.q.dtype, seed=1, device=x.q.device)
    wsb = gdn.gdn_prefill_backward_workspace_bytes(T, n, H, dk, dv, x.q.dtype)
    ws = torch.empty(wsb, dtype=torch.uint8, device=x.q.device)
    out = []

    def step():
        out[:] = gdn.gdn_prefill_backward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, d_o,
                                          initial_state=x.initial_state, d_final_state=dSf, workspace=ws,
                                          stream=stream)

    ms = time_loop(step, steps, warmup, stream)
    init = x.initial_state is not None
    bbytes = backward_bytes(T, H, dk, dv, n, init_state=init)
    gbs = bbytes / (ms / 1e3) / 1e9
    cu = x.cu_seqlens.to("cpu", torch.int64).numpy()
    L0 = int(cu[1])
    su = lambda t: t[:L0, :1].to("cpu", torch.float64).numpy()
    ref = oracle.backward(su(x.q), su(x.k), su(x.v), su(x.g), su(x.beta), np.array([0, L0], np.int32), su(d_o),
                          initial_state=None if not init else x.initial_state[:1, :1].to("cpu", torch.float64).numpy(),
                          d_final_state=dSf[:1, :1].to("cpu", torch.float64).numpy())
    par = max(oracle.rel_err(su(gt), ref[nm]) for gt, nm in zip(out[:5], ("dq", "dk", "dv", "dg", "dbeta")))
    leg = {"workload": name + " backward", "num_seqs": n, "T": T, "H": H, "d_k": dk, "d_v": dv,
           "initial_state": init, "workspace_bytes": wsb, "steps": steps, "warmup": warmup, "ms_per_step": ms,
           "tokens_per_s": T / (ms / 1e3),
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": bbytes},
           "parity_max_rel_err_seq0_head0": par, "parity_tokens": L0}
    del out[:], ws, d_o, dSf
    return leg


def cpu_backward_baseline(x, d_o, dSf, tokens: int, heads: int):
    """The oracle's reverse-mode recurrence (fp64, OpenMP over heads) on the host for the first
    `tokens` tokens of the first `heads` heads of sequence 0."""
    import oracle

    oracle.build(force=False)
    sl = lambda t: t[:tokens, :heads].to("cpu", torch.float64).numpy()
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    threads = max(1, min(os.cpu_count() or 1, heads, share))
    t0 = time.perf_counter()
    oracle.backward(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), np.array([0, tokens], np.int32), sl(d_o),
                    d_final_state=dSf[:1, :heads].to("cpu", torch.float64).numpy(), threads=threads)
    dt = time.perf_counter() - t0
    return {"value": tokens * heads / dt / x.q.shape[1], "unit": "tokens/s (all heads)", "cores": threads,
            "kind": "oracle",
            "sample": f"first {tokens} tokens of sequence 0, {heads} of {x.q.shape[1]} heads, fp64 reverse-mode "
                      f"recurrence (checkpoints every 64 tokens, OpenMP over heads), {dt:.2f} s wall; value is "
                      f"head-tokens/s divided by the {x.q.shape[1]} heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-tokens", type=int, default=65536)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=10)
    ap.add_argument("--no-tiles", action="store_true")
    ap.add_argument("--tiles-steps", type=int, default=10)
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV", help="summarise rocprofv3 --pmc CSVs and exit")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--no-gates", action="store_true")
    ap.add_argument("--workload-steps", type=int, default=10)
    ap.add_argument("--workload-warmup", type=int, default=10)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build runs the layer on a single MI355X "
              f"(asked for --gpus {args.gpus}); sharding across GPUs is described in DESIGN.md.", file=sys.stderr)
        sys.exit(2)

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import gated_delta_rule_linear_amd as gdn
    from gated_delta_rule_linear_amd import inputs

    gdn.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---- prefill workload
    T, H, d = 65536, 32, 128
    x = inputs.make_workload("prefill_64k", seed=0, device=dev)
    xf = x
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    S = torch.empty((1, H, d, d), dtype=torch.float32, device=dev)
    ws_bytes = gdn.gdn_prefill_workspace_bytes(T, 1, H, d, d)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None

    def step():
        gdn.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, final_state=S, o=o, workspace=ws, stream=stream)

    ms = time_loop(step, args.steps, args.warmup, stream)
    tokens_per_s = T / (ms / 1e3)
    pbytes = prefill_bytes(T, H, d, d, 1)
    achieved = pbytes / (ms / 1e3) / 1e9
    pflops = prefill_flops(T, H, d, d)
    tflops = pflops / (ms / 1e3) / 1e12

    # sampled parity on the timed inputs: head 0, first 2048 tokens
    import oracle

    tk = 2048
    ro, _ = oracle.recurrent(*(t[:tk, :1].to("cpu", torch.float64).numpy() for t in (x.q, x.k, x.v, x.g)),
                             x.beta[:tk, :1].to("cpu", torch.float64).numpy(), np.array([0, tk], np.int32))
    parity = oracle.rel_err(o[:tk, :1].to("cpu", torch.float64).numpy(), ro)

    # ---- decode workload
    N, Hd = 512, 32
    S0, draws = inputs.make_decode_steps(N, Hd, d, d, max(1, min(args.steps + args.warmup, 32)),
                                         dtype=torch.bfloat16, seed=0, device=dev)
    state = S0.contiguous()
    od = torch.empty((N, Hd, d), dtype=torch.bfloat16, device=dev)
    it = [0]

    def dstep():
        dr = draws[it[0] % len(draws)]
        it[0] += 1
        gdn.gdn_decode(dr.q, dr.k, dr.v, dr.g, dr.beta, state, o=od, stream=stream)

    dms = time_loop(dstep, args.steps, args.warmup, stream)
    dbytes = decode_bytes(N, Hd, d, d)
    dgbs = dbytes / (dms / 1e3) / 1e9

    # ---- the other gate forms (NEXT f1: bf16 logits with the gate computed in the kernel; f4: one
    # log-decay per (token, head)) on the same prefill and decode shapes
    gates = None
    if not args.no_gates:
        gates = gate_variants_leg(gdn, inputs, x, o, S, ws, N, Hd, d, args.steps, args.warmup, stream)

    del o
    torch.cuda.empty_cache()
    xb = inputs.make_workload("batch4_t8k", seed=0, device=dev)
    Tb, nb = xb.T_total, xb.num_seqs

    # ---- diagonal-tile paths: the same batch through gdn_prefill_tiles with dense window products and
    # with position-pair decays (bounded gates, so both are valid), then gdn_prefill; and the pair path on
    # the unbounded negative-softplus gate
    tiles = None
    if not args.no_tiles:
        ob = torch.empty_like(xb.v)
        tbytes = prefill_bytes(Tb, H, d, d, nb)

        def tiles_step(path, xx):
            return lambda: gdn.gdn_prefill_tiles(xx.q, xx.k, xx.v, xx.g, xx.beta, xx.cu_seqlens, path, o=ob,
                                                 output_final_state=False, stream=stream)

        tms_dense = time_loop(tiles_step(gdn.GDN_TILES_DENSE, xb), args.tiles_steps, 3, stream)
        tms_pairs = time_loop(tiles_step(gdn.GDN_TILES_PAIRS, xb), args.tiles_steps, 3, stream)
        tms_prefill = time_loop(lambda: gdn.gdn_prefill(xb.q, xb.k, xb.v, xb.g, xb.beta, xb.cu_seqlens, o=ob,
                                                        output_final_state=False, stream=stream),
                                args.tiles_steps, 3, stream)
        xs = inputs.make_prefill_inputs([8192] * 4, H, d, d, dtype=torch.bfloat16, gate="softplus", seed=0,
                                        device=dev)
        tms_soft = time_loop(tiles_step(gdn.GDN_TILES_PAIRS, xs), args.tiles_steps, 3, stream)
        del xs
        frac = lambda ms: tbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS
        tiles = {"workload": "batch4_t8k forward, 16-token windows", "steps": args.tiles_steps, "warmup": 3,
                 "dense_window_products_ms": tms_dense, "position_pairs_ms": tms_pairs,
                 "position_pairs_over_dense": tms_pairs / tms_dense,
                 "position_pairs_softplus_gate_ms": tms_soft, "gdn_prefill_ms": tms_prefill,
                 "hbm_frac": {"dense": frac(tms_dense), "pairs": frac(tms_pairs), "gdn_prefill": frac(tms_prefill)},
                 "algorithmic_bytes_per_launch": tbytes}
        del ob

    # ---- backward workload: four 8192-token sequences, 32 heads (a training batch)
    bwd = None
    if not args.no_backward:
        d_o, dSf = inputs.make_cotangents(Tb, nb, H, d, d, dtype=torch.bfloat16, seed=1, device=dev)
        grads = [torch.empty_like(t) for t in (xb.q, xb.k, xb.v, xb.g, xb.beta)]
        dS0 = torch.empty((nb, H, d, d), dtype=torch.float32, device=dev)
        bws = torch.empty(gdn.gdn_prefill_backward_workspace_bytes(Tb, nb, H, d, d, torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        lib = gdn.load_library()
        ptr = lambda t: t.data_ptr()

        def bstep():
            st = lib.gdn_prefill_backward(ptr(xb.q), ptr(xb.k), ptr(xb.v), ptr(xb.g), ptr(xb.beta),
                                          ptr(xb.cu_seqlens), nb, Tb, None, ptr(d_o), ptr(dSf), ptr(grads[0]),
                                          ptr(grads[1]), ptr(grads[2]), ptr(grads[3]), ptr(grads[4]), ptr(dS0),
                                          H, d, d, gdn.GDN_BF16, ptr(bws), bws.numel(), stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"gdn_prefill_backward: {st}")

        bms = time_loop(bstep, args.backward_steps, 3, stream)
        bbytes = backward_bytes(Tb, H, d, d, nb)
        bflops = backward_flops(Tb, H, d, d)
        bgbs = bbytes / (bms / 1e3) / 1e9
        # sampled parity: sequence 0, head 0, whole sequence (a gradient depends on every later token)
        su = lambda t: t[:8192, :1].to("cpu", torch.float64).numpy()
        ref = oracle.backward(su(xb.q), su(xb.k), su(xb.v), su(xb.g), su(xb.beta), np.array([0, 8192], np.int32),
                              su(d_o), d_final_state=dSf[:1, :1].to("cpu", torch.float64).numpy())
        bpar = max(oracle.rel_err(su(gt), ref[nm]) for gt, nm in zip(grads, ("dq", "dk", "dv", "dg", "dbeta")))
        bwd = {"workload": "batch4_t8k backward", "num_seqs": nb, "T": Tb, "H": H, "d_k": d, "d_v": d,
               "workspace_bytes": bws.numel(),
               "ms_per_step": bms, "steps": args.backward_steps, "warmup": 3, "tokens_per_s": Tb / (bms / 1e3),
               "roofline": {"bound": "hbm", "achieved": bgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": bgbs / HBM_PEAK_GBS, "traffic": measured_traffic("backward"),
                            "kernel": "gdn_prefill_backward call (time split planned for 128 units: "
                                      "seg_table, prefill_ws_kernel<128,128,map,q^>, seg_fold, "
                                      "bwd_dpass_kernel<128,128>, bwd_fold_rev_q_kernel, "
                                      "prefill_ws_kernel<128,128,map,checkpoints>, "
                                      "bwd_grad_kernel<bf16,128,128,full>)",
                            "algorithmic_bytes_per_launch": bbytes},
               "mfma": {"flops_per_launch": bflops, "achieved": bflops / (bms / 1e3) / 1e12,
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": bflops / (bms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
               "parity_max_rel_err_seq0_head0": bpar}
        if not args.no_cpu:
            bwd["cpu_baseline"] = cpu_backward_baseline(xb, d_o, dSf, 8192, 16)

    # ---- the other prefill workloads: varlen64 and long_1m
    workloads = None
    if not args.no_workloads:
        del xb
        torch.cuda.empty_cache()
        workloads = {}
        xv = inputs.make_workload("varlen64", seed=0, device=dev)
        # host sample: the first sequences up to ~65,536 tokens (whole sequences, their initial states)
        cuv = xv.cu_seqlens.to("cpu", torch.int64).numpy()
        nv = max(1, int(np.searchsorted(cuv, 65536, side="right")) - 1)
        ww = args.workload_warmup
        workloads["varlen64"] = prefill_leg(gdn, "varlen64", xv, args.workload_steps, ww, stream, not args.no_cpu,
                                            nv, f"the first {nv} of 64 sequences")
        if not args.no_backward:
            workloads["varlen64_backward"] = backward_leg(gdn, "varlen64", xv, max(3, args.workload_steps // 2),
                                                          3, stream)
        del xv
        torch.cuda.empty_cache()
        xl = inputs.make_workload("long_1m", seed=0, device=dev)
        workloads["long_1m"] = prefill_leg(gdn, "long_1m", xl, args.workload_steps, ww, stream,
                                           not args.no_cpu, 1, "the first 131072 of 1048576 tokens",
                                           cpu_x=prefix_view(xl, 131072))
        del xl
        torch.cuda.empty_cache()
        # a skewed packed batch: 63 sequences of 1,024 tokens and one of 262,144, 32 heads;
        # gdn_prefill plans from the mean length, gdn_prefill_maxlen from the bound on the lengths
        lens = [1024] * 63 + [262144]
        xs = inputs.make_prefill_inputs(lens, 32, d, d, dtype=torch.bfloat16, seed=5, device=dev)
        plain = prefill_leg(gdn, "skewed64", xs, args.workload_steps, ww, stream, False, 0, "")
        hinted = prefill_leg(gdn, "skewed64", xs, args.workload_steps, ww, stream, not args.no_cpu, 63,
                             "the 63 sequences of 1,024 tokens", max_seqlen=max(lens))
        hinted["without_hint_ms_per_step"] = plain["ms_per_step"]
        hinted["without_hint_roofline_frac"] = plain["roofline"]["frac"]
        hinted["speedup_from_hint"] = plain["ms_per_step"] / hinted["ms_per_step"]
        workloads["skewed64"] = hinted
        if not args.no_backward:
            workloads["skewed64_backward"] = backward_leg(gdn, "skewed64", xs, 3, 1, stream)
        del xs
        torch.cuda.empty_cache()

    traffic = measured_traffic("prefill")
    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_64k", "num_seqs": 1, "T": T, "H": H, "d_k": d, "d_v": d,
                   "gates": "alpha=0.9+0.1*sigmoid(N(0,1)) per key channel", "initial_state": "zero",
                   "chunk": 32, "workspace_bytes": ws_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gdn_prefill call (seg_table; prefill_ws_kernel<128,128,out> of segment 0 on a side "
                               "stream beside prefill_ws_kernel<128,128,map>; seg_fold; "
                               "prefill_ws_kernel<128,128,out> of segments 1-8)",
                     "algorithmic_bytes_per_launch": pbytes},
        "decode": {"workload": "decode_512x32", "N": N, "H": Hd, "d_k": d, "d_v": d, "ms_per_step": dms,
                   "tokens_per_s": N / (dms / 1e3), "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": dgbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": dbytes,
                   "traffic": measured_traffic("decode")},
        "mfma": {"algorithmic_flops_per_launch": pflops, "chunk": BF16_CHUNK, "achieved": tflops,
                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                 "counters": measured_counters("prefill")},
        "attainable_roofline_frac": max(pflops / (MFMA_BF16_PEAK_TFLOPS * 1e12), pbytes / (HBM_PEAK_GBS * 1e9))
                                    / (ms / 1e3),
        "parity": {"prefill_o_rel_err_head0_first2048": parity},
    }
    if gates is not None:
        res["gate_variants"] = gates
    if tiles is not None:
        res["tile_paths"] = tiles
    if bwd is not None:
        res["backward"] = bwd
    if workloads is not None:
        res["workloads"] = workloads
    res["device"] = device_info()
    if not args.no_cpu:
        xc = xf if args.cpu_tokens >= T else prefix_view(xf, args.cpu_tokens)
        what = "the whole 65536-token sequence" if args.cpu_tokens >= T else f"the first {args.cpu_tokens} tokens"
        res["cpu_baseline"] = cpu_baseline(xc, 1, what)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
