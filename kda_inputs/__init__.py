"""Seeded synthetic inputs for KDA prefill and decode.

This module is the one thing the HIP path's tests and the oracle share: it
draws random tensors and nothing else.  It holds none of the method's
arithmetic and imports neither the oracle nor the native binding.

Recipe (the workloads the library is measured on; there is no dataset):

* q, k ~ N(0, 1), then L2-normalised per (token, head) in fp32 before the
  single quantisation to the I/O dtype;
* v ~ N(0, 1);
* beta = sigmoid(N(0, 1)), one value per (token, head);
* g = -softplus(N(mu, 1)) * s per (token, head, key channel), so g <= 0;
* initial state ~ N(0, std^2) in fp32 (or zeros), one per (sequence, head);
* output-gate pre-activations z ~ N(0, 2^2) (own generator and seed);
* front end (own generator and seed): raw q, k, v as above but not
  normalised; conv weights N(0, 1/W); conv states N(0, 1); low-rank gate
  factors a ~ N(0, 1), b ~ N(0, 1/r) (so a b^T ~ N(0, 1)), bias N(0, s^2);
* varlen batches draw integer lengths uniformly in [lo, hi] (both ends
  inclusive) on the CPU generator before any tensor, so the packing does not
  depend on the device.

Draw order for prefill: [lengths], q, k, v, beta logits, g logits, initial
state.  Decode: initial state, then per step q, k, v, beta logits, g logits.
All draws are fp32 from one ``torch.Generator`` seeded with ``seed`` on the
device the tensors are made on, then quantised once.  The same quantised bytes
go to the GPU library and (upcast exactly to fp32 on the host) to the oracle.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import torch


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    lens: tuple            # sequence lengths; () means "draw varlen lengths"
    heads: int
    d: int
    io_dtype: str          # "bf16" or "fp32"
    g_mu: float = 0.0      # g = -softplus(N(g_mu, 1)) * g_scale
    g_scale: float = 1.0
    s0_std: Optional[float] = None   # None: zero initial state
    varlen_n: int = 0      # >0: draw this many lengths uniformly in [lo, hi]
    varlen_lo: int = 0
    varlen_hi: int = 0
    seed: int = 0


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    n_seqs: int
    heads: int
    d: int
    io_dtype: str
    steps: int
    g_mu: float = 0.0
    g_scale: float = 0.5
    s0_std: float = 0.02
    seed: int = 3


#: The five workloads.  Index = seed.
CONFIGS: Dict[int, object] = {
    0: PrefillConfig("tiny prefill T=256 H=2 d=64 fp32", (256,), 2, 64, "fp32",
                     g_mu=0.0, g_scale=1.0, s0_std=None, seed=0),
    1: PrefillConfig("single-sequence prefill T=8192 H=32 d=128 bf16", (8192,), 32, 128,
                     "bf16", g_mu=0.0, g_scale=0.5, s0_std=0.02, seed=1),
    2: PrefillConfig("varlen prefill 64 seqs U[1024,32768] H=32 d=128 bf16", (), 32, 128,
                     "bf16", g_mu=0.0, g_scale=0.5, s0_std=0.02, varlen_n=64,
                     varlen_lo=1024, varlen_hi=32768, seed=2),
    3: DecodeConfig("decode 256 seqs H=32 d=128 bf16 tokens fp32 state, 100 steps",
                    256, 32, 128, "bf16", 100, g_mu=0.0, g_scale=0.5, s0_std=0.02, seed=3),
    4: PrefillConfig("million-token prefill T=1048576 H=16 d=128 bf16", (1 << 20,), 16, 128,
                     "bf16", g_mu=-2.0, g_scale=1.0, s0_std=0.02, seed=4),
}


def torch_dtype(io_dtype: str) -> torch.dtype:
    if io_dtype == "bf16":
        return torch.bfloat16
    if io_dtype == "fp32":
        return torch.float32
    raise ValueError(f"unknown io dtype {io_dtype!r}")


def draw_lengths(n: int, lo: int, hi: int, seed: int) -> List[int]:
    """Integer lengths uniform in [lo, hi], drawn on the CPU generator."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return torch.randint(lo, hi + 1, (n,), generator=gen).tolist()


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    # input recipe: unit-norm q/k rows (fp32) before quantisation
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def _randn(shape, gen, device) -> torch.Tensor:
    """fp32 N(0,1) of ``shape`` (drawn in one call per tensor)."""
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_prefill(T_lens, heads: int, d: int, io_dtype: str = "bf16", *,
                 g_mu: float = 0.0, g_scale: float = 1.0, s0_std: Optional[float] = None,
                 seed: int = 0, device="cpu", packed_cu: bool = True,
                 d_v: Optional[int] = None, scalar_gate: bool = False) -> dict:
    """Draw one prefill batch.

    ``T_lens`` is a list of sequence lengths (packed back to back).  Returns a
    dict with q, k, g ``[T,H,d]``, v ``[T,H,d_v]``, beta ``[T,H]`` in the I/O
    dtype, ``initial_state`` ``[N,H,d,d_v]`` fp32 (or None), ``cu_seqlens`` int32
    ``[N+1]`` (or None when ``packed_cu`` is False and all lengths are equal),
    and the lengths.  ``scalar_gate``: g is ``[T,H]`` (one decay per token and
    head) instead of ``[T,H,d]``.
    """
    d_v = d if d_v is None else d_v
    lens = [int(x) for x in T_lens]
    T = sum(lens)
    N = len(lens)
    dt = torch_dtype(io_dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = _unit_rows(_randn((T, heads, d), gen, device)).to(dt)
    k = _unit_rows(_randn((T, heads, d), gen, device)).to(dt)
    v = _randn((T, heads, d_v), gen, device).to(dt)
    beta = torch.sigmoid(_randn((T, heads), gen, device)).to(dt)
    g = (-torch.nn.functional.softplus(_randn((T, heads) if scalar_gate else (T, heads, d),
                                              gen, device) + g_mu) * g_scale).to(dt)
    s0 = None
    if s0_std is not None:
        s0 = _randn((N, heads, d, d_v), gen, device) * s0_std
    cu = None
    if packed_cu or len(set(lens)) > 1:
        c = [0]
        for L in lens:
            c.append(c[-1] + L)
        cu = torch.tensor(c, dtype=torch.int32, device=device)
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=s0, cu_seqlens=cu,
                lens=lens, heads=heads, d=d, d_v=d_v, io_dtype=io_dtype)


def make_config_prefill(cfg_id: int, device="cpu") -> dict:
    cfg = CONFIGS[cfg_id]
    assert isinstance(cfg, PrefillConfig)
    if cfg.varlen_n:
        lens = draw_lengths(cfg.varlen_n, cfg.varlen_lo, cfg.varlen_hi, cfg.seed)
    else:
        lens = list(cfg.lens)
    return make_prefill(lens, cfg.heads, cfg.d, cfg.io_dtype, g_mu=cfg.g_mu,
                        g_scale=cfg.g_scale, s0_std=cfg.s0_std, seed=cfg.seed,
                        device=device, packed_cu=bool(cfg.varlen_n))


def make_decode(n_seqs: int, heads: int, d: int, io_dtype: str = "bf16", steps: int = 1,
                *, g_mu: float = 0.0, g_scale: float = 0.5, s0_std: float = 0.02,
                seed: int = 3, device="cpu", scalar_gate: bool = False) -> dict:
    """Draw a decode workload: one fp32 state per (sequence, head) and ``steps``
    batches of one token per sequence.  Per-step tensors are stacked on a
    leading step axis: q, k, g ``[steps,N,H,d]``, v ``[steps,N,H,d]``,
    beta ``[steps,N,H]``."""
    dt = torch_dtype(io_dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    state = _randn((n_seqs, heads, d, d), gen, device) * s0_std
    qs, ks, vs, bs, gs = [], [], [], [], []
    for _ in range(steps):
        qs.append(_unit_rows(_randn((n_seqs, heads, d), gen, device)).to(dt))
        ks.append(_unit_rows(_randn((n_seqs, heads, d), gen, device)).to(dt))
        vs.append(_randn((n_seqs, heads, d), gen, device).to(dt))
        bs.append(torch.sigmoid(_randn((n_seqs, heads), gen, device)).to(dt))
        gshape = (n_seqs, heads) if scalar_gate else (n_seqs, heads, d)
        gs.append((-torch.nn.functional.softplus(_randn(gshape, gen, device)
                                                 + g_mu) * g_scale).to(dt))
    return dict(state=state, q=torch.stack(qs), k=torch.stack(ks), v=torch.stack(vs),
                beta=torch.stack(bs), g=torch.stack(gs), n_seqs=n_seqs, heads=heads,
                d=d, io_dtype=io_dtype, steps=steps)


def make_config_decode(cfg_id: int = 3, device="cpu", steps: Optional[int] = None) -> dict:
    cfg = CONFIGS[cfg_id]
    assert isinstance(cfg, DecodeConfig)
    return make_decode(cfg.n_seqs, cfg.heads, cfg.d, cfg.io_dtype,
                       cfg.steps if steps is None else steps, g_mu=cfg.g_mu,
                       g_scale=cfg.g_scale, s0_std=cfg.s0_std, seed=cfg.seed,
                       device=device)


def make_out_gate(shape, io_dtype: str = "bf16", *, std: float = 2.0, seed: int = 7,
                  device="cpu") -> torch.Tensor:
    """Output-gate pre-activations z ~ N(0, std^2) of the given shape ([T, H, d_v]
    per value channel or [T, H] per head), drawn from their own generator."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return (_randn(tuple(shape), gen, device) * std).to(torch_dtype(io_dtype))


def make_front_end(n_tokens: int, n_seqs: int, heads: int, d: int, io_dtype: str = "bf16", *,
                   width: int = 4, rank: int = 64, bias_std: float = 0.0, seed: int = 11,
                   device="cpu") -> dict:
    """Front-end tensors, drawn from their own generator in this order: conv
    weights ``[3, H, W, d]`` ~ N(0, 1/W); conv state ``[N, 3, W-1, H, d]`` ~
    N(0, 1); gate factors a ``[T, r]`` ~ N(0, 1) and b ``[H, d, r]`` ~ N(0, 1/r),
    so a b^T ~ N(0, 1) like the g logits of the plain recipe; bias ``[H, d]``
    fp32 ~ N(0, bias_std^2) (None when bias_std is 0)."""
    dt = torch_dtype(io_dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    if width > 0:
        out["conv_weight"] = (_randn((3, heads, width, d), gen, device) / width ** 0.5).to(dt)
        out["conv_state"] = _randn((n_seqs, 3, max(width - 1, 0), heads, d), gen, device).to(dt)
    if rank > 0:
        out["gate_a"] = _randn((n_tokens, rank), gen, device).to(dt)
        out["gate_b"] = (_randn((heads, d, rank), gen, device) / rank ** 0.5).to(dt)
        out["gate_bias"] = (_randn((heads, d), gen, device) * bias_std) if bias_std else None
    return out


def seeded_heads(n_heads: int, count: int, seed: int) -> List[int]:
    """The first ``count`` entries of a seeded permutation of the heads (the
    subset the oracle is run on for the long workloads); seed = config + 100."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return sorted(torch.randperm(n_heads, generator=gen)[:count].tolist())
