"""GPU parity under strong and extreme decay.

The retention alpha = exp(g) is per key channel, so some channels forget within
a token or two while others keep their memory ("From KV Cache to Depth
Attention: The Bottlenecks Kimi K3 Had to Break", Technical Details, KDA
bullet).  Inside a 64-token chunk the prefill factors its decay ratios around
16-token block boundaries; a block whose total decay in some channel exceeds
2^64 has its diagonal products computed exactly instead.  These cases drive
both paths (and the switch between them) against the fp64 oracle, on the same
quantised inputs, at the usual bar: max abs error 2e-2 (bf16 I/O) and 1e-4
(fp32 I/O), with every output finite.
"""

import math
import sys

import numpy as np
import pytest
import torch

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

TOL = {"bf16": 2e-2, "fp32": 1e-4}
LENS = [1, 63, 64, 65, 0, 127, 200]
IO_D = [("bf16", 128), ("bf16", 64), ("fp32", 64)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return None if t is None else t.detach().float().cpu().numpy()


def maxerr(a, b):
    a = np.asarray(a, np.float64)
    return float(np.max(np.abs(a - np.asarray(b, np.float64)))) if a.size else 0.0


@pytest.fixture(scope="module")
def lib():
    import linear_attention_recurrence_06_amd as kda
    kda.load_library()
    return kda


def check_prefill(lib, oracle, inp, label, g_oracle=None):
    out, fin = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["initial_state"], inp["cu_seqlens"],
                                     num_seqs=len(inp["lens"]))
    torch.cuda.synchronize()
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].cpu().numpy()
    g_ref = host(inp["g"]) if g_oracle is None else g_oracle
    o_ref, f_ref = oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), g_ref,
                                  host(inp["beta"]), cu_seqlens=cu,
                                  initial_state=host(inp["initial_state"]),
                                  n_seqs=len(inp["lens"]))
    o_gpu, f_gpu = host(out), host(fin)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(f_gpu)), f"{label}: non-finite"
    eo, ef = maxerr(o_gpu, o_ref), maxerr(f_gpu, f_ref)
    tol = TOL[inp["io_dtype"]]
    say(f"[{label}] err_out={eo:.3e} err_state={ef:.3e} max|o|={np.abs(o_ref).max():.2f} tol={tol}")
    assert eo <= tol and ef <= tol


def base(io, d, seed, lens=LENS, H=2, scalar_gate=False):
    from kda_inputs import make_prefill
    return make_prefill(lens, H, d, io, g_scale=0.5, s0_std=0.02, seed=seed, device="cuda",
                        scalar_gate=scalar_gate)


@pytest.mark.parametrize("gval", [-8.0, -30.0])
@pytest.mark.parametrize("io,d", IO_D)
def test_uniform_strong_decay(lib, oracle, io, d, gval):
    """Every channel of every token at g = -8 or -30: each block's decay is far
    past the factored range (16 * 8 / ln 2 = 185 in log2 units)."""
    inp = base(io, d, seed=301)
    inp["g"] = torch.full_like(inp["g"], gval)
    check_prefill(lib, oracle, inp, f"g={gval} {io} d={d}")


@pytest.mark.parametrize("io,d", IO_D)
def test_decay_spikes(lib, oracle, io, d):
    """The usual gate with 1% of its (token, channel) entries at -100: single
    tokens that wipe one channel, inside otherwise long memories."""
    inp = base(io, d, seed=302)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(303)
    spike = torch.rand(inp["g"].shape, generator=gen, device="cuda") < 0.01
    inp["g"] = torch.where(spike, torch.full_like(inp["g"], -100.0), inp["g"])
    assert int(spike.sum()) > 0
    check_prefill(lib, oracle, inp, f"1% at -100 {io} d={d}")


@pytest.mark.parametrize("blocks", [(1,), (0, 3), (2,)])
def test_mixed_blocks(lib, oracle, blocks):
    """Strong decay (g = -12) only on the tokens of the given 16-token blocks of
    every chunk: those blocks take the exact diagonal path, the others the
    factored one, in the same chunk."""
    inp = base("bf16", 128, seed=304, lens=[320], H=3)
    t = torch.arange(320, device="cuda") % 64 // 16
    hit = torch.zeros_like(t, dtype=torch.bool)
    for b in blocks:
        hit |= t == b
    inp["g"] = torch.where(hit[:, None, None], torch.full_like(inp["g"], -12.0), inp["g"])
    check_prefill(lib, oracle, inp, f"g=-12 in blocks {blocks}")


@pytest.mark.parametrize("gval", [-2.70, -2.85])
def test_factored_range_edge(lib, oracle, gval):
    """Uniform g just inside (-2.70: 62.3 in log2 units per block) and just past
    (-2.85: 65.8) the factored range."""
    for io, d in IO_D:
        inp = base(io, d, seed=305)
        inp["g"] = torch.full_like(inp["g"], gval)
        check_prefill(lib, oracle, inp, f"g={gval} {io} d={d}")


def test_infinite_decay(lib, oracle):
    """g = -inf (a retention of exactly zero) on a few tokens: outputs stay
    finite and match the oracle, whose exp(-inf) is 0."""
    inp = base("bf16", 128, seed=306)
    g = inp["g"].clone()
    g[5] = -math.inf
    g[70, :, :16] = -math.inf
    g[130, 1] = -math.inf
    inp["g"] = g
    check_prefill(lib, oracle, inp, "g=-inf on some tokens")


def test_scalar_gate_strong_decay(lib, oracle):
    """The per-head gate g [T, H] at -30 on every other token."""
    inp = base("bf16", 128, seed=307, scalar_gate=True)
    g = inp["g"].clone()
    g[::2] = -30.0
    inp["g"] = g
    d = inp["q"].shape[2]
    g_full = np.repeat(host(g)[:, :, None], d, axis=2)
    check_prefill(lib, oracle, inp, "per-head gate, -30 on every other token", g_oracle=g_full)


@pytest.mark.parametrize("io,d", IO_D)
def test_low_rank_gate_strong_decay(lib, oracle, io, d):
    """The front end's low-rank gate with biases of +25 on half the key channels,
    so its computed g = -softplus(a b^T + bias) sits near -25 there."""
    from kda_inputs import make_front_end
    H = 2
    inp = base(io, d, seed=308, H=H)
    T, N = sum(LENS), len(LENS)
    fe = make_front_end(T, N, H, d, io, width=0, rank=64, bias_std=1.0, seed=309,
                        device="cuda")
    bias = fe["gate_bias"].clone()
    bias[:, ::2] += 25.0
    out, fin, _, _ = lib.kda_chunk_prefill_ex(
        inp["q"], inp["k"], inp["v"], None, inp["beta"], inp["initial_state"],
        inp["cu_seqlens"], gate_a=fe["gate_a"], gate_b=fe["gate_b"], gate_bias=bias)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].cpu().numpy()
    g_ref = oracle.low_rank_gate(host(fe["gate_a"]), host(fe["gate_b"]), host(bias))
    assert g_ref.min() < -20
    o_ref, f_ref = oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), g_ref,
                                  host(inp["beta"]), cu_seqlens=cu,
                                  initial_state=host(inp["initial_state"]), n_seqs=N)
    o_gpu, f_gpu = host(out), host(fin)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(f_gpu))
    eo, ef = maxerr(o_gpu, o_ref), maxerr(f_gpu, f_ref)
    say(f"[low-rank gate, +25 bias, {io} d={d}] err_out={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL[io] and ef <= TOL[io]


def test_decode_strong_decay(lib, oracle):
    """Decode steps with g at -30 on every channel of half the sequences and
    1% spikes at -100 elsewhere."""
    from kda_inputs import make_decode
    w = make_decode(6, 3, 128, "bf16", steps=3, seed=310, device="cuda")
    st = w["state"].clone()
    st_ref = host(w["state"]).astype(np.float64)
    for s in range(3):
        g = w["g"][s].clone()
        g[::2] = -30.0
        g[1, 0, ::100] = -100.0
        o = lib.kda_decode_step(w["q"][s], w["k"][s], w["v"][s], g, w["beta"][s], st)
        torch.cuda.synchronize()
        o_ref = oracle.decode_step(host(w["q"][s]), host(w["k"][s]), host(w["v"][s]),
                                   host(g), host(w["beta"][s]), st_ref)
        assert np.all(np.isfinite(host(o)))
        assert maxerr(host(o), o_ref) <= TOL["bf16"]
    assert maxerr(host(st), st_ref) <= TOL["bf16"]
