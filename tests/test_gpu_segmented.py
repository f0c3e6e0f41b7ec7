"""GPU tests of the segmented prefill: a long sequence with few heads is cut
into P + 1 segments.  A first pass of the fused kernel runs segment 0 with its
outputs from the initial state and forms the state maps S_end = M S_start + b
of segments 1..P-1 (b from the zero state, M from the identity with V = 0); a
scan composes them into the start states of segments 2..P; a second pass runs
segments 1..P from their start states with their outputs.

* Parity with the fp64 oracle at the bf16 bar (max abs error 2e-2, every
  output finite): one ragged sequence (P = 4, the last segment ending in a
  partial chunk), packed sequences with empty segments and an
  empty sequence, equal lengths without cu_seqlens, decay strong
  enough for the exact diagonal products, channels of all three decay
  regimes, no initial and no final state, P = 64 (the most).
* Agreement with the two-kernel path within twice that bar where the oracle
  would be slow: the automatic choice on a 262,144-token sequence with 8 heads.
* Bitwise: two runs of the same call, the library-allocated workspace, a
  workspace of just the bytes the call's path uses (segmented, fused and
  two-kernel), the final state written over the initial state on a side
  stream, and graph replays of the segmented and the fused path.

KDA_PREFILL_PATH=segmented forces the path and KDA_PREFILL_SEGMENTS sets P.
"""

import sys

import numpy as np
import pytest
import torch

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

TOL = 2e-2


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


def args_of(inp):
    return (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"],
            inp["cu_seqlens"])


def run(lib, monkeypatch, inp, path, segments=None, **kw):
    monkeypatch.setenv("KDA_PREFILL_PATH", path)
    if segments is None:
        monkeypatch.delenv("KDA_PREFILL_SEGMENTS", raising=False)
    else:
        monkeypatch.setenv("KDA_PREFILL_SEGMENTS", str(segments))
    out, fin = lib.kda_chunk_prefill(*args_of(inp), num_seqs=len(inp["lens"]), **kw)
    torch.cuda.synchronize()
    return out, fin


def near_split(lib, monkeypatch, inp, label, segments=None, **kw):
    """The segmented path, checked against the two-kernel path within 2 TOL."""
    o_s, f_s = run(lib, monkeypatch, inp, "split", **kw)
    o_g, f_g = run(lib, monkeypatch, inp, "segmented", segments, **kw)
    eo = maxerr(host(o_g), host(o_s))
    ef = maxerr(host(f_g), host(f_s)) if f_g is not None else 0.0
    say(f"[{label}] segmented vs split: out {eo:.3e} state {ef:.3e}")
    assert torch.isfinite(o_g.float()).all()
    assert (f_g is None) == (f_s is None)
    assert f_g is None or torch.isfinite(f_g).all()
    assert eo <= 2 * TOL and ef <= 2 * TOL
    return o_g, f_g


def oracle_check(oracle, inp, out, fin, label):
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].cpu().numpy()
    o_ref, f_ref = oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["g"]),
                                  host(inp["beta"]), cu_seqlens=cu,
                                  initial_state=host(inp["initial_state"]),
                                  n_seqs=len(inp["lens"]))
    eo = maxerr(host(out), o_ref)
    ef = maxerr(host(fin), f_ref) if fin is not None else 0.0
    say(f"[{label}] oracle err_out={eo:.3e} err_state={ef:.3e} tol={TOL}")
    assert eo <= TOL and ef <= TOL


def test_ragged_sequence(lib, oracle, monkeypatch):
    """16,421 tokens (257 chunks, the last partial) x 2 heads, P = 4: segment
    0 of 57 chunks, then four of 50 (the last ending in the partial chunk)."""
    from kda_inputs import make_prefill
    inp = make_prefill([16421], 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=601,
                       device="cuda")
    out, fin = near_split(lib, monkeypatch, inp, "ragged", segments=4)
    oracle_check(oracle, inp, out, fin, "ragged")


def test_packed_sequences(lib, oracle, monkeypatch):
    """Four packed sequences of 200, 20,000, 0 and 9,000 tokens, P = 8, cut
    into 9 segments each on the device: the short one leaves segment 0 and
    four others empty (their maps M = I, b = 0) and the empty one keeps its
    initial state."""
    from kda_inputs import make_prefill
    lens = [200, 20000, 0, 9000]
    inp = make_prefill(lens, 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=610, device="cuda")
    assert inp["cu_seqlens"] is not None
    out, fin = near_split(lib, monkeypatch, inp, "packed", segments=8)
    oracle_check(oracle, inp, out, fin, "packed")
    assert torch.equal(fin[2], inp["initial_state"][2])


def test_equal_lengths_without_cu(lib, oracle, monkeypatch):
    """Three 8,192-token sequences without cu_seqlens, P = 3."""
    from kda_inputs import make_prefill
    inp = make_prefill([8192] * 3, 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=602,
                       device="cuda", packed_cu=False)
    assert inp["cu_seqlens"] is None
    out, fin = near_split(lib, monkeypatch, inp, "equal lengths", segments=3)
    oracle_check(oracle, inp, out, fin, "equal lengths")


@pytest.mark.parametrize("g_value", [-8.0, -30.0])
def test_strong_decay(lib, oracle, monkeypatch, g_value):
    """Blocks past the factored range in every channel, plus 1% of gates at
    -100: the maps' linear parts then decay to zero within a segment."""
    from kda_inputs import make_prefill
    inp = make_prefill([6000], 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=603,
                       device="cuda")
    g = torch.full_like(inp["g"], g_value)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(604)
    g[torch.rand(g.shape, generator=gen, device="cuda") < 0.01] = -100.0
    inp["g"] = g
    out, fin = near_split(lib, monkeypatch, inp, f"g={g_value}", segments=4)
    oracle_check(oracle, inp, out, fin, f"g={g_value}")


def test_mixed_decay_forms(lib, oracle, monkeypatch):
    """Key channels in the three decay regimes side by side, and long-retention
    channels (g near zero) whose state carries across every segment."""
    from kda_inputs import make_prefill
    inp = make_prefill([12800], 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=605,
                       device="cuda")
    g = inp["g"].float().clone()
    g[:, :, 32:64] = -2.0
    g[:, :, 64:96] = -8.0
    g[:, :, 96:128] = -0.001
    inp["g"] = g.to(inp["g"].dtype)
    out, fin = near_split(lib, monkeypatch, inp, "mixed decay", segments=5)
    oracle_check(oracle, inp, out, fin, "mixed decay")


def test_no_initial_no_final_state(lib, oracle, monkeypatch):
    from kda_inputs import make_prefill
    inp = make_prefill([9000], 2, 128, "bf16", g_scale=0.5, s0_std=None, seed=606,
                       device="cuda")
    assert inp["initial_state"] is None
    out, fin = near_split(lib, monkeypatch, inp, "no states", segments=4,
                          output_final_state=False)
    assert fin is None
    oracle_check(oracle, inp, out, None, "no states")


def test_two_chains_per_pass(lib, oracle, monkeypatch):
    """9,000 tokens x 2 heads with P = 2: segment 0 beside a single map in the
    first pass, a one-step scan, segments 1 and 2 in the second."""
    from kda_inputs import make_prefill
    inp = make_prefill([9000], 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=614,
                       device="cuda")
    out, fin = near_split(lib, monkeypatch, inp, "P = 2", segments=2)
    oracle_check(oracle, inp, out, fin, "P = 2")


def test_auto_choice_many_heads(lib, monkeypatch):
    """8,192 tokens x 96 heads: where the fused kernel would run a chain per CU,
    the automatic choice on a 256-CU device is P = 2; checked against the
    two-kernel path and bitwise against the forced path."""
    from kda_inputs import make_prefill
    inp = make_prefill([8192], 96, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=615,
                       device="cuda")
    o_a, f_a = run(lib, monkeypatch, inp, "auto")
    o_s, f_s = run(lib, monkeypatch, inp, "split")
    eo, ef = maxerr(host(o_a), host(o_s)), maxerr(host(f_a), host(f_s))
    say(f"[auto 8,192 x 96] vs split: out {eo:.3e} state {ef:.3e}")
    assert torch.isfinite(o_a.float()).all() and torch.isfinite(f_a).all()
    assert eo <= 2 * TOL and ef <= 2 * TOL
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        o_g, f_g = run(lib, monkeypatch, inp, "segmented", 2)
        assert torch.equal(o_g, o_a) and torch.equal(f_g, f_a)


def test_sixty_four_segments(lib, oracle, monkeypatch):
    """32,768 tokens x 2 heads with P = 64: an empty segment 0 and 64 of 8
    chunks; the scan composes the most maps a call can have."""
    from kda_inputs import make_prefill
    inp = make_prefill([32768], 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=611,
                       device="cuda")
    out, fin = near_split(lib, monkeypatch, inp, "64 segments", segments=64)
    oracle_check(oracle, inp, out, fin, "64 segments")


def test_in_place_on_a_side_stream(lib, monkeypatch):
    """final_state aliasing initial_state, called on a side stream that alone
    is synchronised: the same results as the call with separate states."""
    from kda_inputs import make_prefill
    inp = make_prefill([16421], 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=612,
                       device="cuda")
    o_ref, f_ref = run(lib, monkeypatch, inp, "segmented", 4)
    st = inp["initial_state"].clone()
    out = torch.empty_like(o_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], st, None,
                              out, st, stream=side)
    side.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(st, f_ref)


def test_auto_choice_long_sequence(lib, monkeypatch):
    """262,144 tokens x 8 heads: 8 chains, so on a 256-CU device the automatic
    choice cuts the sequence into 32 segments of 128 chunks (256 chains);
    checked against the two-kernel path, bitwise against the forced path with
    the same count, and bitwise from run to run."""
    from kda_inputs import make_prefill
    inp = make_prefill([262144], 8, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=607,
                       device="cuda")
    o_a, f_a = run(lib, monkeypatch, inp, "auto")
    o_s, f_s = run(lib, monkeypatch, inp, "split")
    eo, ef = maxerr(host(o_a), host(o_s)), maxerr(host(f_a), host(f_s))
    say(f"[auto 262,144 x 8] vs split: out {eo:.3e} state {ef:.3e}")
    assert torch.isfinite(o_a.float()).all() and torch.isfinite(f_a).all()
    assert eo <= 2 * TOL and ef <= 2 * TOL
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    o_g, f_g = run(lib, monkeypatch, inp, "segmented", min(64, cus // 8))
    assert torch.equal(o_g, o_a) and torch.equal(f_g, f_a)
    o_2, f_2 = run(lib, monkeypatch, inp, "segmented", min(64, cus // 8))
    assert torch.equal(o_2, o_g) and torch.equal(f_2, f_g)


def test_path_choice(lib, monkeypatch):
    """The rule on a 256-CU device: P = one chain per CU in each pass (at most
    64), lowered until segments hold at least 12 chunks; taken with P >= 2
    whose chains fill 3/4 of the CUs, or with P >= 16, or where the fused
    kernel (a chain per 3 CUs at d = 128) would take the call."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the thresholds below are for 256 compute units")
    monkeypatch.delenv("KDA_PREFILL_PATH", raising=False)
    monkeypatch.delenv("KDA_PREFILL_SEGMENTS", raising=False)
    K = lib.kda
    path = lambda T, N, H, packed=False, io=K.KDA_BF16, d=128: lib.kda_prefill_path(
        lib.make_dims(T, N, H, d, d, io), packed)
    SEG, FUSED, SPLIT = K.KDA_PATH_SEGMENTED, K.KDA_PATH_FUSED, K.KDA_PATH_SPLIT
    assert path(1 << 20, 1, 16) == (SEG, 16)         # the million-token workload
    assert path(8192, 1, 32) == (SEG, 8)             # the 8,192-token workload: 14-chunk segments
    assert path(1007721, 64, 32, packed=True)[0] == FUSED   # the packed headline: 2,048 chains
    assert path(1 << 19, 1, 8) == (SEG, 32)
    assert path(1 << 18, 1, 4) == (SEG, 64)          # at most 64
    assert path(1 << 20, 1, 64) == (SEG, 4)
    assert path(1 << 16, 1, 48) == (SEG, 5)          # 240 chains
    assert path(1 << 16, 1, 80) == (SEG, 3)
    assert path(4 * 4096, 4, 20, packed=True) == (SEG, 3)   # 16-chunk segments
    assert path(1 << 16, 1, 86) == (SEG, 2)          # where the fused kernel would run
    assert path(1 << 20, 1, 128) == (SEG, 2)
    assert path(1 << 16, 1, 160)[0] == FUSED         # P = 1
    assert path(2048, 1, 128)[0] == FUSED            # P = 2 would leave 11-chunk segments
    assert path(1 << 16, 1, 1) == (SEG, 64)          # 16-chunk segments
    assert path(1 << 14, 1, 16) == (SEG, 16)
    assert path(4096, 1, 32)[0] == SPLIT             # P = 4 at most: 128 chains
    assert path(8192, 1, 16)[0] == SPLIT             # P = 8 at most: 128 chains
    assert path(8192, 1, 4)[0] == SPLIT
    assert path(1 << 20, 2, 8)[0] == SEG             # equal lengths, no cu
    assert path(1 << 20, 2, 8, packed=True)[0] == SEG  # cut on the device
    assert path(1 << 20, 1, 16, packed=True) == (SEG, 16)   # cu = [0, T]
    assert path(1 << 20, 1, 16, io=K.KDA_FP32)[0] == K.KDA_PATH_PIPELINED  # bf16 only
    assert path(1 << 20, 1, 16, d=64)[0] == K.KDA_PATH_PIPELINED    # d = 128 only
    assert path(1 << 16, 1, 86, d=64)[0] == SPLIT    # d = 64: the fused kernel from 128
    monkeypatch.setenv("KDA_PREFILL_PATH", "split")
    assert path(1 << 20, 1, 16)[0] == K.KDA_PATH_PIPELINED
    monkeypatch.setenv("KDA_PREFILL_PATH", "segmented")
    monkeypatch.setenv("KDA_PREFILL_SEGMENTS", "4")
    assert path(16421, 1, 2) == (K.KDA_PATH_SEGMENTED, 4)


def test_library_workspace(lib, monkeypatch):
    """No workspace given: the library allocates the index areas and the maps."""
    from kda_inputs import make_prefill
    inp = make_prefill([16421], 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=608,
                       device="cuda")
    o_w, f_w = run(lib, monkeypatch, inp, "segmented", 4)
    o_l, f_l = run(lib, monkeypatch, inp, "segmented", 4, library_workspace=True)
    assert torch.equal(o_l, o_w) and torch.equal(f_l, f_w)


@pytest.mark.parametrize("lens,heads,path", [([16384], 32, 3), ([4096] * 16, 32, 2),
                                             ([300, 65], 3, 0)])
def test_path_workspace(lib, monkeypatch, lens, heads, path):
    """A workspace of exactly kda_prefill_path_workspace_bytes (the segmented
    path: index areas and maps; the fused kernel: index areas; the two-kernel
    path: everything) gives the results of the full-size workspace bitwise; a
    byte less is rejected."""
    from kda_inputs import make_prefill
    monkeypatch.delenv("KDA_PREFILL_PATH", raising=False)
    monkeypatch.delenv("KDA_PREFILL_SEGMENTS", raising=False)
    K = lib.kda
    n, T = len(lens), sum(lens)
    dims = lib.make_dims(T, n, heads, 128, 128, K.KDA_BF16)
    full = lib.kda_prefill_workspace_bytes(dims)
    need = lib.kda_prefill_path_workspace_bytes(dims, n > 1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus == 256:
        assert lib.kda_prefill_path(dims, n > 1)[0] == path
    assert 0 < need <= full and (need == full) == (path == 0)
    say(f"[path workspace {n} x {lens[0]} x {heads}] {need} of {full} bytes")
    inp = make_prefill(lens, heads, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=613,
                       device="cuda", packed_cu=n > 1)
    ws_full = torch.empty(full, dtype=torch.uint8, device="cuda")
    o_f, f_f = lib.kda_chunk_prefill(*args_of(inp), num_seqs=n, workspace=ws_full)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_p, f_p = lib.kda_chunk_prefill(*args_of(inp), num_seqs=n, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_f) and torch.equal(f_p, f_f)
    with pytest.raises(lib.KDAError) as e:
        lib.kda_chunk_prefill(*args_of(inp), num_seqs=n, workspace=ws[:need - 1])
    assert e.value.status == K.KDA_ERR_WORKSPACE
    fp32 = lib.make_dims(T, n, heads, 128, 128, K.KDA_FP32)
    assert lib.kda_prefill_path_workspace_bytes(fp32, n > 1) == lib.kda_prefill_workspace_bytes(fp32)


@pytest.mark.parametrize("path,lens,heads,segments", [("segmented", [16421], 2, 4),
                                                      ("fused", [300, 64, 1000, 5], 4, None)])
def test_replayed_from_a_graph(lib, monkeypatch, path, lens, heads, segments):
    """The segmented and fused paths captured into a graph (every launch on
    the capturing stream, the chain counter zeroed by a kernel, not a memset)
    and replayed three times with eager work in between: every replay equals
    the eager call bit for bit."""
    from kda_inputs import make_prefill
    inp = make_prefill(lens, heads, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=609,
                       device="cuda")
    o_ref, f_ref = run(lib, monkeypatch, inp, path, segments)
    dims = lib.make_dims(sum(lens), len(lens), heads, 128, 128, lib.kda.KDA_BF16)
    ws = torch.empty(lib.kda_prefill_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    out, fin = torch.empty_like(o_ref), torch.empty_like(f_ref)
    call = lambda: lib.kda_chunk_prefill(*args_of(inp), out, fin, num_seqs=len(lens), workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(fin, f_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        fin.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say(f"[{path}] graph replay {rep}")
        assert torch.equal(out, o_ref) and torch.equal(fin, f_ref)
