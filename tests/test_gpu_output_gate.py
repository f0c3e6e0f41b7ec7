"""The output forget gate fused into the output write: out = o * sigmoid(z), z
per value channel ([T, H, d_v]) or per head ([T, H]) ("Kimi K3: The Manos, The
Mythos, The Legendos", bullet on stability details).  The reference is the fp64
oracle's read-out passed through the oracle's gate (``apply_output_gate``,
pinned by closed-form values of the logistic function); the gate must leave the
state path, final states and checkpoints, bit for bit as without it."""

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


LENS = [1, 63, 64, 65, 0, 127, 129, 300]


@pytest.mark.parametrize("io,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
@pytest.mark.parametrize("per_head", [False, True])
def test_gated_prefill_matches_oracle(lib, oracle, io, d, per_head):
    from kda_inputs import make_out_gate, make_prefill
    say(f"gated prefill {io} d={d} per_head={per_head}")
    H = 3
    inp = make_prefill(LENS, H, d, io, g_scale=0.5, s0_std=0.02, seed=61, device="cuda")
    T = sum(LENS)
    z = make_out_gate((T, H) if per_head else (T, H, d), io, seed=62, device="cuda")
    out, fin, ck, _ = lib.kda_chunk_prefill_ex(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                            inp["initial_state"], inp["cu_seqlens"],
                                            out_gate_z=z)
    torch.cuda.synchronize()
    assert ck is None
    o_ref, f_ref = oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["g"]),
                                  host(inp["beta"]), cu_seqlens=inp["cu_seqlens"].cpu().numpy(),
                                  initial_state=host(inp["initial_state"]), n_seqs=len(LENS))
    o_ref = oracle.apply_output_gate(o_ref, host(z))
    eo, ef = maxerr(host(out), o_ref), maxerr(host(fin), f_ref)
    say(f"  err_out={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL[io] and ef <= TOL[io]
    # the gate touches the output only: the final state is the ungated call's
    o0, f0 = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   inp["initial_state"], inp["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(fin, f0)


def test_gate_at_zero_halves_the_output(lib):
    """sigmoid(0) = 1/2: a zero z scales the ungated output by exactly one half
    (a power of two commutes with the final rounding)."""
    from kda_inputs import make_prefill
    inp = make_prefill(LENS, 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=63, device="cuda")
    T = sum(LENS)
    z = torch.zeros((T, 2, 128), dtype=torch.bfloat16, device="cuda")
    out, _, _, _ = lib.kda_chunk_prefill_ex(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                         inp["initial_state"], inp["cu_seqlens"], out_gate_z=z)
    o0, _ = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                  inp["initial_state"], inp["cu_seqlens"])
    torch.cuda.synchronize()
    torch.testing.assert_close(out.float(), o0.float() * 0.5, rtol=1e-6, atol=0)


def test_gate_with_checkpoints(lib, oracle):
    """Both options at once: checkpoints and final states equal the ungated
    call's bit for bit; the output matches the gated oracle."""
    from kda_inputs import make_out_gate, make_prefill
    H, d = 4, 128
    inp = make_prefill(LENS, H, d, "bf16", g_scale=0.5, s0_std=0.02, seed=64, device="cuda")
    T = sum(LENS)
    z = make_out_gate((T, H, d), "bf16", seed=65, device="cuda")
    out, fin, ck, _ = lib.kda_chunk_prefill_ex(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                            inp["initial_state"], inp["cu_seqlens"],
                                            out_gate_z=z, checkpoint_interval=1)
    o0, f0, ck0 = lib.kda_chunk_prefill_checkpoints(inp["q"], inp["k"], inp["v"], inp["g"],
                                                    inp["beta"], inp["initial_state"],
                                                    inp["cu_seqlens"], checkpoint_interval=1)
    torch.cuda.synchronize()
    assert ck.shape == ck0.shape and ck.shape[0] > 0
    assert torch.equal(ck, ck0) and torch.equal(fin, f0)
    o_ref, _ = oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["g"]),
                              host(inp["beta"]), cu_seqlens=inp["cu_seqlens"].cpu().numpy(),
                              initial_state=host(inp["initial_state"]), n_seqs=len(LENS))
    eo = maxerr(host(out), oracle.apply_output_gate(o_ref, host(z)))
    say(f"gated prefill with checkpoints: err_out={eo:.3e}")
    assert eo <= TOL["bf16"]


def test_gated_prefill_full_size(lib, oracle):
    """T=8192, H=32, d=128 bf16, per-channel z, in the launch configuration the
    benchmark times: every head against the gated oracle."""
    from kda_inputs import make_out_gate, make_prefill
    say("gated prefill T=8192 H=32 d=128")
    inp = make_prefill([8192], 32, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=66,
                       device="cuda")
    z = make_out_gate((8192, 32, 128), "bf16", seed=67, device="cuda")
    out, fin, _, _ = lib.kda_chunk_prefill_ex(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                           inp["initial_state"], None, out_gate_z=z)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["g"]),
                                  host(inp["beta"]), initial_state=host(inp["initial_state"]))
    eo = maxerr(host(out), oracle.apply_output_gate(o_ref, host(z)))
    ef = maxerr(host(fin), f_ref)
    say(f"  err_out={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("io,d", [("bf16", 128), ("fp32", 64)])
@pytest.mark.parametrize("per_head", [False, True])
def test_gated_decode_matches_oracle(lib, oracle, io, d, per_head):
    from kda_inputs import make_decode, make_out_gate
    N, H, steps = 6, 4, 3
    w = make_decode(N, H, d, io, steps=steps, seed=68, device="cuda")
    z = make_out_gate((steps, N, H) if per_head else (steps, N, H, d), io, seed=69,
                      device="cuda")
    st = w["state"].clone()
    st_plain = w["state"].clone()
    st_ref = host(w["state"]).astype(np.float64)
    for s in range(steps):
        o = lib.kda_decode_step_ex(w["q"][s], w["k"][s], w["v"][s], w["g"][s], w["beta"][s], st,
                                   out_gate_z=z[s])
        lib.kda_decode_step(w["q"][s], w["k"][s], w["v"][s], w["g"][s], w["beta"][s], st_plain)
        torch.cuda.synchronize()
        o_ref = oracle.decode_step(host(w["q"][s]), host(w["k"][s]), host(w["v"][s]),
                                   host(w["g"][s]), host(w["beta"][s]), st_ref)
        e = maxerr(host(o), oracle.apply_output_gate(o_ref, host(z[s])))
        say(f"gated decode {io} d={d} per_head={per_head} step {s}: err={e:.3e}")
        assert e <= TOL[io]
    assert maxerr(host(st), st_ref) <= TOL[io]
    assert torch.equal(st, st_plain)
