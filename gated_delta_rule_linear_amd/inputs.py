"""Seeded synthetic inputs for the gated delta-rule layer.

This module draws random tensors and nothing else: it holds none of the
layer's arithmetic, and both the GPU path and the CPU oracle consume what it
returns.  The draw order is fixed so a seed names one input set:

  1. per-sequence lengths (packed variable-length batches only),
  2. q, k, v, the beta logits, the decay logits,
  3. the initial states (when asked for),
  4. decode draws, one block per step, in step order.
The backward pass's incoming gradients (make_cotangents) come from a
generator of their own.

Distributions
  q, k   N(0, 1) per element, L2-normalised over the key channels of each
         (token, head) in fp32, then cast to the working dtype (RNE).
  v      N(0, 1), cast to the working dtype.
  beta   sigmoid(N(0, 1)), fp32, one value per (token, head).
  g      log-decay per (token, head, key channel), fp32.  Two recipes:
           "amin":  alpha = a_min + (1 - a_min) * sigmoid(N(0,1)), g = log(alpha)
           "pages": g = g_min * sigmoid(N(0,1)) with g_min = -5, the lower-bounded
                    scaled-sigmoid decay of the bounded-decay articles
                    ("Lower-Bounded Decay Parameterization", eq. 1 of
                    "Trillion-Parameter MoE Multimodal LLMs: How to Evaluate the
                    New Generation", section 3.1).
           "softplus": g = -softplus(s * N(0,1)), the unbounded negative-softplus
                    gate the bounded form replaces (same articles); s = softplus_scale
                    (1 by default; larger values give steep decays, down to about
                    -4s per token)
  S0     0.02 * N(0, 1), fp32, layout [num_seqs, H, d_k, d_v].
  g      (head_gate=True) one log-decay per (token, head), [T_total, H], same recipes.
  z      (logits=True) the decay logits N(0,1) themselves, cast to bf16 (RNE),
         for the entry points that compute the gate in the kernel; g is still
         the recipe applied to the fp32 logits.

Layouts: q, k, g are [T_total, H, d_k]; v is [T_total, H, d_v]; beta is
[T_total, H]; sequences are packed back to back and described by int32
cu_seqlens of length num_seqs + 1.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import torch

G_MIN = -5.0


@dataclasses.dataclass
class PrefillInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    cu_seqlens: torch.Tensor  # int32, on the same device as the tensors
    lengths: list
    initial_state: Optional[torch.Tensor]
    z: Optional[torch.Tensor] = None  # bf16 decay logits [T, H, dk] (logits=True)

    @property
    def T_total(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_seqs(self) -> int:
        return len(self.lengths)


@dataclasses.dataclass
class DecodeStep:
    q: torch.Tensor  # [N, H, dk]
    k: torch.Tensor
    v: torch.Tensor  # [N, H, dv]
    g: torch.Tensor  # [N, H, dk] fp32
    beta: torch.Tensor  # [N, H] fp32
    z: Optional[torch.Tensor] = None  # bf16 decay logits [N, H, dk] (logits=True)


def make_generator(seed: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def draw_lengths(gen: torch.Generator, n: int, lo: int, hi: int) -> list:
    """n sequence lengths uniform on [lo, hi] (both ends included)."""
    dev = gen.device
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen, device=dev).cpu()]


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def _draw_qkv(gen, shape_k, shape_v, dtype, device):
    q = _unit_rows(torch.randn(shape_k, generator=gen, device=device, dtype=torch.float32)).to(dtype)
    k = _unit_rows(torch.randn(shape_k, generator=gen, device=device, dtype=torch.float32)).to(dtype)
    v = torch.randn(shape_v, generator=gen, device=device, dtype=torch.float32).to(dtype)
    return q, k, v


def _draw_gates(gen, shape_beta, shape_g, gate: str, a_min: float, device, softplus_scale: float = 1.0):
    beta = torch.sigmoid(torch.randn(shape_beta, generator=gen, device=device, dtype=torch.float32))
    z = torch.randn(shape_g, generator=gen, device=device, dtype=torch.float32)
    if gate == "amin":
        alpha = a_min + (1.0 - a_min) * torch.sigmoid(z)
        g = torch.log(alpha)
    elif gate == "pages":
        g = G_MIN * torch.sigmoid(z)
    elif gate == "softplus":
        g = -torch.nn.functional.softplus(softplus_scale * z)
    else:
        raise ValueError(f"unknown gate recipe {gate!r}")
    return beta, g.contiguous(), z


def make_prefill_inputs(lengths: Sequence[int], H: int, dk: int, dv: int, dtype=torch.bfloat16,
                        gate: str = "amin", a_min: float = 0.9, init_state: bool = False,
                        seed: int = 0, device="cpu", gen: Optional[torch.Generator] = None,
                        logits: bool = False, head_gate: bool = False,
                        softplus_scale: float = 1.0) -> PrefillInputs:
    """Packed prefill inputs for the given sequence lengths (draw order above)."""
    if gen is None:
        gen = make_generator(seed, device)
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    q, k, v = _draw_qkv(gen, (T, H, dk), (T, H, dv), dtype, device)
    beta, g, z = _draw_gates(gen, (T, H), (T, H) if head_gate else (T, H, dk), gate, a_min, device,
                             softplus_scale)
    zb = z.to(torch.bfloat16) if logits else None
    del z
    S0 = None
    if init_state:
        S0 = 0.02 * torch.randn((len(lengths), H, dk, dv), generator=gen, device=device, dtype=torch.float32)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return PrefillInputs(q, k, v, g, beta, cu.to(device), lengths, S0, zb)


def make_decode_steps(N: int, H: int, dk: int, dv: int, steps: int, dtype=torch.bfloat16,
                      gate: str = "amin", a_min: float = 0.9, seed: int = 0, device="cpu",
                      gen: Optional[torch.Generator] = None, logits: bool = False, head_gate: bool = False):
    """Initial states (0.02*N(0,1)) followed by `steps` one-token draws for N sequences."""
    if gen is None:
        gen = make_generator(seed, device)
    S0 = 0.02 * torch.randn((N, H, dk, dv), generator=gen, device=device, dtype=torch.float32)
    out = []
    for _ in range(steps):
        q, k, v = _draw_qkv(gen, (N, H, dk), (N, H, dv), dtype, device)
        beta, g, z = _draw_gates(gen, (N, H), (N, H) if head_gate else (N, H, dk), gate, a_min, device)
        out.append(DecodeStep(q, k, v, g, beta, z.to(torch.bfloat16) if logits else None))
    return S0, out


def make_cotangents(T: int, num_seqs: int, H: int, dk: int, dv: int, dtype=torch.bfloat16,
                    final_state: bool = True, seed: int = 0, device="cpu",
                    gen: Optional[torch.Generator] = None):
    """Gradients flowing into the layer's outputs, for the backward pass:
    dL/do ~ N(0, 1) [T, H, dv] cast to dtype (RNE), and dL/d(final state)
    ~ 0.02 * N(0, 1) [num_seqs, H, dk, dv] fp32 (None when final_state is False),
    drawn in that order."""
    if gen is None:
        gen = make_generator(seed, device)
    d_o = torch.randn((T, H, dv), generator=gen, device=device, dtype=torch.float32).to(dtype)
    dSf = None
    if final_state:
        dSf = 0.02 * torch.randn((num_seqs, H, dk, dv), generator=gen, device=device, dtype=torch.float32)
    return d_o, dSf


# Named workloads.  Each entry: how to build its inputs from a generator.
WORKLOADS = {
    # fp32 parity case: one sequence of 256 tokens, 2 heads, d = 64.
    "small_fp32": dict(lengths=[256], H=2, dk=64, dv=64, dtype=torch.float32, gate="amin", a_min=0.9,
                       init_state=False),
    # four 8192-token sequences, 32 heads, d = 128, bf16.
    "batch4_t8k": dict(lengths=[8192] * 4, H=32, dk=128, dv=128, dtype=torch.bfloat16, gate="amin",
                       a_min=0.9, init_state=False),
    # one 65536-token sequence, 32 heads, d = 128, bf16 (the prefill throughput workload).
    "prefill_64k": dict(lengths=[65536], H=32, dk=128, dv=128, dtype=torch.bfloat16, gate="amin",
                        a_min=0.9, init_state=False),
    # one 2^20-token sequence, 16 heads, slow decay.
    "long_1m": dict(lengths=[1 << 20], H=16, dk=128, dv=128, dtype=torch.bfloat16, gate="amin",
                    a_min=0.99, init_state=False),
}


def make_varlen64_inputs(seed: int = 0, device="cpu", n_seqs: int = 64, lo: int = 512, hi: int = 16384,
                         H: int = 32, dk: int = 128, dv: int = 128, dtype=torch.bfloat16,
                         logits: bool = False, head_gate: bool = False) -> PrefillInputs:
    """64 packed sequences with lengths uniform on [512, 16384], random initial states."""
    gen = make_generator(seed, device)
    lengths = draw_lengths(gen, n_seqs, lo, hi)
    return make_prefill_inputs(lengths, H, dk, dv, dtype=dtype, gate="amin", a_min=0.9, init_state=True,
                               device=device, gen=gen, logits=logits, head_gate=head_gate)


def make_workload(name: str, seed: int = 0, device="cpu", logits: bool = False,
                  head_gate: bool = False) -> PrefillInputs:
    if name == "varlen64":
        return make_varlen64_inputs(seed=seed, device=device, logits=logits, head_gate=head_gate)
    spec = dict(WORKLOADS[name])
    return make_prefill_inputs(seed=seed, device=device, logits=logits, head_gate=head_gate, **spec)
