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

Two more legs follow in the same run, each on four 8,192-token sequences x
32 heads and reported in objects of their own: "tile_paths" times
gdn_prefill_tiles with dense window products and with position-pair decays
(the diagonal-tile comparison), and "backward" times gdn_prefill_backward
with its own roofline, sampled parity and host-oracle baseline.
--no-tiles / --no-backward skip them.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
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
                  "gdn_fold.h"]
BACKWARD_SOURCES = ["gdn_backward.hip", "gdn_backward.h", "gdn_tile16.h", "gdn_mfma.h", "gdn_device.h",
                    "gdn_api_backward.cpp", "gdn_prefill.hip", "gdn_kernels.h", "gdn_fold.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def prefill_bytes(T_tokens: int, H: int, dk: int, dv: int, n_seqs: int, elt: int = 2, init_state: bool = False):
    """Algorithmic HBM bytes of one prefill launch: every input read once, every output written once."""
    per_head_token = elt * (2 * dk + dv) + 4 * dk + 4 + elt * dv
    states = n_seqs * H * dk * dv * 4 * (2 if init_state else 1)
    return T_tokens * H * per_head_token + states


def prefill_flops(T_tokens: int, H: int, dk: int, dv: int, C: int = 64):
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


def decode_bytes(N: int, H: int, dk: int, dv: int, elt: int = 2):
    """Algorithmic HBM bytes of one decode launch: state read and written, token vectors read, o written."""
    per = 8 * dk * dv + elt * (2 * dk + dv) + 4 * dk + 4 + elt * dv
    return N * H * per


def source_hash(files=None) -> str:
    h = hashlib.sha256()
    for f in files or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_linear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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


def copy_calibration(nbytes: int):
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "calls": 3}), flush=True)


def cpu_baseline(x, tokens: int):
    """fp32 oracle on the host over the first `tokens` tokens of every head."""
    import oracle

    oracle.build(force=False)
    H = x.q.shape[1]
    sl = lambda t: t[:tokens].to("cpu", torch.float32).numpy()
    args = [sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), np.array([0, tokens], np.int32)]
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    threads = max(1, min(os.cpu_count() or 1, H, share))
    t0 = time.perf_counter()
    oracle.recurrent(*args, dtype=np.float32, threads=threads)
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    whole = "the whole 65536-token sequence" if tokens >= x.q.shape[0] else f"the first {tokens} tokens"
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{whole}, all {H} heads, fp32 sequential recurrence (OpenMP over heads), {dt:.2f} s wall; "
                      f"host {model or 'unknown CPU'}, {os.cpu_count()} logical CPUs visible"}


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
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build runs the layer on a single MI355X "
              f"(asked for --gpus {args.gpus}); sharding across GPUs is described in DESIGN.md.", file=sys.stderr)
        sys.exit(2)

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
                                      "seg_table, prefill_ws_kernel<128,128,map>, seg_fold, "
                                      "bwd_grad_kernel<bf16,128,128,adjoint-only>, bwd_fold_rev_kernel, "
                                      "bwd_states_kernel<bf16,128,128>, bwd_grad_kernel<bf16,128,128,full>)",
                            "algorithmic_bytes_per_launch": bbytes},
               "mfma": {"flops_per_launch": bflops, "achieved": bflops / (bms / 1e3) / 1e12,
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": bflops / (bms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
               "parity_max_rel_err_seq0_head0": bpar}
        if not args.no_cpu:
            bwd["cpu_baseline"] = cpu_backward_baseline(xb, d_o, dSf, 2048, 16)

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
        "mfma": {"algorithmic_flops_per_launch": pflops, "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS},
        "attainable_roofline_frac": max(pflops / (MFMA_BF16_PEAK_TFLOPS * 1e12), pbytes / (HBM_PEAK_GBS * 1e9))
                                    / (ms / 1e3),
        "parity": {"prefill_o_rel_err_head0_first2048": parity},
    }
    if tiles is not None:
        res["tile_paths"] = tiles
    if bwd is not None:
        res["backward"] = bwd
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(xf, min(args.cpu_tokens, T))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
