"""Pipelined prefill of one long sequence.

When a single sequence is long (at least 4 segments of 1,024 chunks) and its
recurrence workgroups (one per head and 16-column tile) leave compute units
idle, the library prepares later chunks on a second stream while the
recurrence works through earlier ones.  The arithmetic per chunk is the same,
so every result must equal, bit for bit, the single-launch path.  The same
tokens take that path when packed as a two-sequence batch whose second sequence
is empty: with more than one sequence the library never pipelines.

Also checked: the call's results are ordered on the caller's stream (a side
stream, synchronised alone), the state handed between segments goes through
the workspace when no final state is asked for, and final_state may alias
initial_state.  Its parity with the oracle follows from that bitwise equality
and the single-launch path's parity tests.  The bf16 d = 128 sequences here
would otherwise take the segmented path, so each test sets
KDA_PREFILL_PATH=split.
"""

import sys

import pytest
import torch

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

# 4,097 chunks: the shortest pipelined length (4 segments) plus a partial chunk
T_PIPE = 4 * 1024 * 64 + 37


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def two_kernel_path(monkeypatch):
    """The bf16 d = 128 sequences below would otherwise be segmented: these
    tests are about the two-kernel path (set per test; the rule test below
    clears it)."""
    monkeypatch.setenv("KDA_PREFILL_PATH", "split")
    monkeypatch.delenv("KDA_PREFILL_SEGMENTS", raising=False)


@pytest.fixture(scope="module")
def lib():
    import linear_attention_recurrence_06_amd as kda
    kda.load_library()
    return kda


def two_seq(inp, T):
    """The packed form of the same tokens: cu = [0, T, T] (an empty second
    sequence) and its initial state slot appended."""
    cu = torch.tensor([0, T, T], dtype=torch.int32, device="cuda")
    s0 = inp["initial_state"]
    s0_2 = torch.cat([s0, torch.randn_like(s0)]) if s0 is not None else None
    return cu, s0_2


@pytest.mark.parametrize("io,d,H,packed,scalar", [("bf16", 128, 2, False, False),
                                                  ("fp32", 64, 3, False, False),
                                                  ("bf16", 128, 3, True, False),
                                                  ("bf16", 64, 2, False, True)])
def test_pipelined_equals_single_launch(lib, io, d, H, packed, scalar):
    """packed: the one sequence given through cu_seqlens = [0, T] (the chunk
    index path); scalar: the per-head gate g [T, H]."""
    from kda_inputs import make_prefill
    inp = make_prefill([T_PIPE], H, d, io, g_scale=0.5, s0_std=0.02, seed=201, device="cuda",
                       scalar_gate=scalar)
    say(f"pipeline {io} d={d} H={H} T={T_PIPE} packed={packed} scalar_gate={scalar}")
    cu1 = torch.tensor([0, T_PIPE], dtype=torch.int32, device="cuda") if packed else None
    E = lib.kda.KDA_BF16 if io == "bf16" else lib.kda.KDA_FP32
    # the call is pipelined (4 segments); the two-sequence form is not
    assert lib.kda_prefill_pipeline_segments(lib.make_dims(T_PIPE, 1, H, d, d, E)) == 4
    assert lib.kda_prefill_pipeline_segments(lib.make_dims(T_PIPE, 2, H, d, d, E)) == 0
    o_p, f_p = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["initial_state"], cu1)
    cu, s0_2 = two_seq(inp, T_PIPE)
    o_r, f_r = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     s0_2, cu)
    # no final state: the segments hand the state over through the workspace
    o_n, f_n = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["initial_state"], cu1, output_final_state=False)
    torch.cuda.synchronize()
    assert f_n is None
    assert torch.equal(o_p, o_r) and torch.equal(f_p, f_r[:1])
    assert torch.equal(o_n, o_r)
    assert torch.equal(f_r[1:], s0_2[1:])  # the empty sequence keeps its state


def test_pipelined_all_options(lib):
    """Front end (W = 4 + SiLU, rank-64 gate), output gate per channel and a
    checkpoint every 512 chunks, pipelined (the sequence given through
    cu_seqlens = [0, T]) against single-launch."""
    from kda_inputs import make_front_end, make_out_gate, make_prefill
    H, d, T = 2, 128, T_PIPE
    inp = make_prefill([T], H, d, "bf16", g_scale=0.5, s0_std=0.02, seed=202, device="cuda")
    fe = make_front_end(T, 1, H, d, "bf16", width=4, rank=64, bias_std=0.3, seed=203,
                        device="cuda")
    z = make_out_gate((T, H, d), "bf16", seed=204, device="cuda")
    common = dict(out_gate_z=z, checkpoint_interval=512, conv_weight=fe["conv_weight"],
                  conv_silu=True, output_conv_state=True, gate_a=fe["gate_a"],
                  gate_b=fe["gate_b"], gate_bias=fe["gate_bias"])
    cu1 = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o_p, f_p, ck_p, cs_p = lib.kda_chunk_prefill_ex(
        inp["q"], inp["k"], inp["v"], None, inp["beta"], inp["initial_state"], cu1,
        conv_state_in=fe["conv_state"], **common)
    cu, s0_2 = two_seq(inp, T)
    cs_in2 = torch.cat([fe["conv_state"], torch.randn_like(fe["conv_state"].float())
                        .to(fe["conv_state"].dtype)])
    o_r, f_r, ck_r, cs_r = lib.kda_chunk_prefill_ex(
        inp["q"], inp["k"], inp["v"], None, inp["beta"], s0_2, cu,
        conv_state_in=cs_in2, **common)
    torch.cuda.synchronize()
    say(f"pipeline all options: checkpoints {ck_p.shape[0]}")
    assert ck_p.shape[0] == (T + 63) // 64 // 512 == ck_r.shape[0]
    assert torch.equal(o_p, o_r) and torch.equal(f_p, f_r[:1])
    assert torch.equal(ck_p, ck_r)
    assert torch.equal(cs_p, cs_r[:1])


def test_pipeline_segment_rule(lib, monkeypatch):
    """Segments as documented: min(16, chunks / 1024) when that is at least 4,
    for one sequence whose H * d / 16 recurrence workgroups leave CUs idle and
    that neither the fused nor the segmented path takes (fp32 I/O below, which
    neither takes)."""
    monkeypatch.delenv("KDA_PREFILL_PATH", raising=False)
    K = lib.kda
    seg = lambda T, N, H, d=128, io=K.KDA_FP32: lib.kda_prefill_pipeline_segments(
        lib.make_dims(T, N, H, d, d, io))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert seg(4095 * 64, 1, 2) == 0                  # 4,095 chunks
    assert seg(4095 * 64 + 1, 1, 2) == 4              # 4,096 chunks (the last one partial)
    assert seg(8191 * 64, 1, 2) == 7                  # 8,191 chunks: 7 whole 1,024-chunk segments
    # the million-token workload: segmented instead (bf16, on 256 CUs), so
    # not pipelined; with fp32 I/O it is
    if cus == 256:
        assert seg(1 << 20, 1, 16, io=K.KDA_BF16) == 0
    assert seg(1 << 20, 1, 16) == (16 if 16 * 8 < cus else 0)
    assert seg(1 << 22, 1, 2) == 16                   # at most 16 segments
    assert seg(8192, 1, 32) == 0                      # the 8,192-token workload: too short
    assert seg(1 << 20, 1, cus // 8) == 0             # the recurrence fills every CU
    assert seg(1 << 20, 2, 2) == 0                    # more than one sequence
    assert seg(1 << 20, 1, 2, 96) == -1               # rejected descriptor


def test_pipelined_in_place_and_on_a_side_stream(lib):
    """final_state aliasing initial_state, called on a side stream that alone is
    synchronised: the results are complete and match the default-stream call."""
    from kda_inputs import make_prefill
    H, d, T = 2, 128, T_PIPE
    inp = make_prefill([T], H, d, "bf16", g_scale=0.5, s0_std=0.02, seed=205, device="cuda")
    o_ref, f_ref = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                         inp["initial_state"], None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    st = inp["initial_state"].clone()
    out = torch.empty_like(o_ref)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], st, None,
                              out, st, stream=side)
        # work queued after the call on the same stream sees its results
        total = out.float().sum()
    side.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(st, f_ref)
    assert float(total) == float(o_ref.float().sum())


@pytest.mark.parametrize("T,H", [(8192 + 37, 4), (T_PIPE, 2)])
def test_prefill_replayed_from_a_graph(lib, T, H):
    """A prefill captured into a graph (on a stream under capture the call is
    not pipelined: it launches only on that stream) and replayed three times,
    with eager work in between: every replay equals the eager call bit for bit."""
    from kda_inputs import make_prefill
    d = 128
    inp = make_prefill([T], H, d, "bf16", g_scale=0.5, s0_std=0.02, seed=206, device="cuda")
    o_ref, f_ref = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                         inp["initial_state"], None)
    torch.cuda.synchronize()
    dims = lib.make_dims(T, 1, H, d, d, lib.kda.KDA_BF16)
    ws = torch.empty(lib.kda_prefill_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(o_ref)
    fin = torch.empty_like(f_ref)
    call = lambda: lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                         inp["initial_state"], None, out, fin, workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        fin.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say(f"graph replay {rep}: T={T} H={H}")
        assert torch.equal(out, o_ref) and torch.equal(fin, f_ref)
