"""The per-head (scalar) forget gate: g is [T, H] (decode [N, H]), one decay per
token and head shared by every key channel ("Kimi K3: The Manos, The Mythos,
The Legendos", bullet on KDA as online learning: the scalar forget gate that
KDA refines into a diagonal one).  By definition it is the per-channel gate
with all channels equal, so the reference is the fp64 oracle fed g broadcast
over the channels (the oracle's scalar-gate pin, P7b, checks that case against
a geometric series)."""

import sys

import numpy as np
import pytest
import torch

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().float().cpu().numpy()


def maxerr(a, b):
    a = np.asarray(a, np.float64)
    return float(np.max(np.abs(a - np.asarray(b, np.float64)))) if a.size else 0.0


@pytest.fixture(scope="module")
def lib():
    import linear_attention_recurrence_06_amd as kda
    kda.load_library()
    return kda


def broadcast(g, d):
    return g.unsqueeze(-1).expand(*g.shape, d).contiguous()


@pytest.mark.parametrize("io,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_scalar_gate_prefill(lib, oracle, io, d):
    from kda_inputs import make_prefill
    lens = [1, 63, 64, 65, 0, 127, 129, 300]
    inp = make_prefill(lens, 3, d, io, g_scale=0.5, s0_std=0.02, seed=51, device="cuda",
                       scalar_gate=True)
    assert inp["g"].shape == (sum(lens), 3)
    out, fin = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["initial_state"], inp["cu_seqlens"])
    torch.cuda.synchronize()
    gb = broadcast(inp["g"], d)
    o_ref, f_ref = oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(gb),
                                  host(inp["beta"]), cu_seqlens=inp["cu_seqlens"].cpu().numpy(),
                                  initial_state=host(inp["initial_state"]), n_seqs=len(lens))
    eo, ef = maxerr(host(out), o_ref), maxerr(host(fin), f_ref)
    say(f"scalar gate prefill {io} d={d}: err_out={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL[io] and ef <= TOL[io]
    # the same computation as the per-channel path on the broadcast gate, bit for bit
    o2, f2 = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], gb, inp["beta"],
                                   inp["initial_state"], inp["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(fin, f2)


def test_scalar_gate_prefill_full_size(lib, oracle):
    """T=8192, H=32, d=128 bf16 with g [T, H]: every head against the oracle."""
    from kda_inputs import make_prefill
    inp = make_prefill([8192], 32, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=52,
                       device="cuda", scalar_gate=True)
    out, fin = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["initial_state"], None)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]),
                                  host(broadcast(inp["g"], 128)), host(inp["beta"]),
                                  initial_state=host(inp["initial_state"]))
    eo, ef = maxerr(host(out), o_ref), maxerr(host(fin), f_ref)
    say(f"scalar gate T=8192: err_out={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("io,d", [("bf16", 128), ("fp32", 64)])
def test_scalar_gate_decode(lib, oracle, io, d):
    from kda_inputs import make_decode
    w = make_decode(6, 4, d, io, steps=3, seed=53, device="cuda", scalar_gate=True)
    assert w["g"].shape == (3, 6, 4)
    st = w["state"].clone()
    st_ref = host(w["state"]).astype(np.float64)
    for s in range(3):
        o = lib.kda_decode_step(w["q"][s], w["k"][s], w["v"][s], w["g"][s], w["beta"][s], st)
        torch.cuda.synchronize()
        o_ref = oracle.decode_step(host(w["q"][s]), host(w["k"][s]), host(w["v"][s]),
                                   host(broadcast(w["g"][s], d)), host(w["beta"][s]), st_ref)
        assert maxerr(host(o), o_ref) <= TOL[io]
    assert maxerr(host(st), st_ref) <= TOL[io]
