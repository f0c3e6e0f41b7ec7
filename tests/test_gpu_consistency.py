"""GPU properties of the HIP path that hold at any size, and option coverage.

* determinism: the same call twice gives the same bytes;
* a NULL initial state is the zero state, bit for bit;
* final_state may alias initial_state (in-place resume) with the same result;
* splitting a sequence at a chunk boundary and resuming from the final state
  reproduces the unsplit run bit for bit (the chunk partition is the same); a
  split inside a chunk agrees within the parity tolerance;
* the prefill of T tokens and T decode steps agree (two independent kernels);
* a non-finite value in one sequence leaves every other sequence untouched;
* scale != 1 and qk_l2norm = 0, odd head counts, many short sequences, against
  the fp64 oracle;
* checkpointed prefill: every intermediate state against the oracle's final
  state of that prefix, bitwise equal to a prefill of the prefix alone, and the
  outputs unchanged.
* decode steps captured into a graph and replayed over fresh tokens equal the
  same steps run eagerly, bit for bit.
"""

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


def prefill(lib, inp, **kw):
    out, fin = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp.get("initial_state"), inp.get("cu_seqlens"),
                                     num_seqs=len(inp["lens"]), **kw)
    torch.cuda.synchronize()
    return out, fin


def oracle_prefill(oracle, inp, **kw):
    s0 = inp.get("initial_state")
    cu = inp.get("cu_seqlens")
    return oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["g"]),
                          host(inp["beta"]), cu_seqlens=None if cu is None else cu.cpu().numpy(),
                          initial_state=None if s0 is None else host(s0),
                          n_seqs=len(inp["lens"]), **kw)


def slice_tokens(inp, t0, t1, s0):
    """One sequence made of tokens [t0, t1) of a single-sequence batch."""
    return dict(q=inp["q"][t0:t1].contiguous(), k=inp["k"][t0:t1].contiguous(),
                v=inp["v"][t0:t1].contiguous(), g=inp["g"][t0:t1].contiguous(),
                beta=inp["beta"][t0:t1].contiguous(), initial_state=s0, cu_seqlens=None,
                lens=[t1 - t0])


# ----------------------------------------------------------------------------- bitwise properties
@pytest.mark.parametrize("io,d", [("bf16", 128), ("fp32", 64)])
def test_prefill_deterministic(lib, io, d):
    from kda_inputs import make_prefill
    say(f"determinism io={io} d={d}")
    inp = make_prefill([1000, 700, 64, 3], 4, d, io, g_scale=0.5, s0_std=0.02, seed=31,
                       device="cuda")
    o1, f1 = prefill(lib, inp)
    o2, f2 = prefill(lib, inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_decode_deterministic(lib):
    from kda_inputs import make_decode
    w = make_decode(7, 5, 128, "bf16", steps=2, seed=32, device="cuda")
    outs = []
    for _ in range(2):
        st = w["state"].clone()
        o = [lib.kda_decode_step(w["q"][s], w["k"][s], w["v"][s], w["g"][s], w["beta"][s], st)
             for s in range(2)]
        torch.cuda.synchronize()
        outs.append((torch.stack(o), st))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_null_initial_state_is_zero_state(lib):
    from kda_inputs import make_prefill
    inp = make_prefill([300, 65], 3, 128, "bf16", g_scale=0.5, s0_std=None, seed=33,
                       device="cuda")
    assert inp["initial_state"] is None
    o_null, f_null = prefill(lib, inp)
    inp["initial_state"] = torch.zeros(2, 3, 128, 128, device="cuda")
    o_zero, f_zero = prefill(lib, inp)
    assert torch.equal(o_null, o_zero) and torch.equal(f_null, f_zero)


def test_final_state_may_alias_initial_state(lib):
    from kda_inputs import make_prefill
    inp = make_prefill([257, 64, 1], 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=34,
                       device="cuda")
    o_ref, f_ref = prefill(lib, inp)
    st = inp["initial_state"].clone()
    inp["initial_state"] = st
    o, f = prefill(lib, inp, final_state=st)
    assert f.data_ptr() == st.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(st, f_ref)


def test_split_at_chunk_boundary_is_exact(lib):
    """Tokens [0, 128) then [128, 300) resumed from the first part's final
    state equal one pass over [0, 300), bit for bit."""
    from kda_inputs import make_prefill
    inp = make_prefill([300], 4, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=35, device="cuda")
    o_full, f_full = prefill(lib, inp)
    a = slice_tokens(inp, 0, 128, inp["initial_state"])
    o_a, f_a = prefill(lib, a)
    b = slice_tokens(inp, 128, 300, f_a)
    o_b, f_b = prefill(lib, b)
    assert torch.equal(torch.cat([o_a, o_b]), o_full)
    assert torch.equal(f_b, f_full)


@pytest.mark.parametrize("io,d", [("bf16", 128), ("fp32", 64)])
def test_split_inside_chunk_resumes(lib, oracle, io, d):
    """A split at token 130 (inside a chunk) changes the chunk partition; both
    halves, chained through the final state, agree with the oracle's one pass."""
    from kda_inputs import make_prefill
    inp = make_prefill([300], 3, d, io, g_scale=0.5, s0_std=0.02, seed=36, device="cuda")
    a = slice_tokens(inp, 0, 130, inp["initial_state"])
    o_a, f_a = prefill(lib, a)
    b = slice_tokens(inp, 130, 300, f_a)
    o_b, f_b = prefill(lib, b)
    o_ref, f_ref = oracle_prefill(oracle, inp)
    eo = maxerr(host(torch.cat([o_a, o_b])), o_ref)
    ef = maxerr(host(f_b), f_ref)
    say(f"split at 130 {io} d={d}: err_out={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL[io] and ef <= TOL[io]


@pytest.mark.parametrize("io,d", [("bf16", 128), ("fp32", 64)])
def test_prefill_matches_decode_steps(lib, io, d):
    """The chunked prefill over T tokens and T single-token decode steps (the
    token-by-token form, a separate kernel) reach the same outputs and state."""
    from kda_inputs import make_prefill
    lens = [150, 64, 1]
    inp = make_prefill(lens, 3, d, io, g_scale=0.5, s0_std=0.02, seed=37, device="cuda")
    o_p, f_p = prefill(lib, inp)
    o_d = torch.empty_like(o_p)
    starts = np.cumsum([0] + lens)
    for n, L in enumerate(lens):
        st = inp["initial_state"][n:n + 1].clone()
        for t in range(starts[n], starts[n] + L):
            sl = lambda x: x[t:t + 1].contiguous()
            o_d[t:t + 1] = lib.kda_decode_step(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]),
                                               sl(inp["g"]), sl(inp["beta"]), st)
        torch.cuda.synchronize()
        ef = maxerr(host(st[0]), host(f_p[n]))
        assert ef <= TOL[io], f"sequence {n}: state differs by {ef}"
    eo = maxerr(host(o_d), host(o_p))
    say(f"prefill vs decode {io} d={d}: out diff {eo:.3e}")
    assert eo <= TOL[io]


def test_nonfinite_input_stays_in_its_sequence(lib):
    """A NaN in one sequence's values and a +inf in another's keys leave every
    other sequence's outputs and states exactly as in the clean run."""
    from kda_inputs import make_prefill
    lens = [200, 130, 64, 77]
    inp = make_prefill(lens, 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=38, device="cuda")
    o_ref, f_ref = prefill(lib, inp)
    bad = dict(inp)
    bad["v"] = inp["v"].clone()
    bad["k"] = inp["k"].clone()
    bad["v"][200 + 70, 1, 5] = float("nan")       # sequence 1
    bad["k"][330 + 10, 0, 0] = float("inf")       # sequence 2
    o, f = prefill(lib, bad)
    for n, (t0, t1) in enumerate([(0, 200), (394, 471)]):
        assert torch.equal(o[t0:t1], o_ref[t0:t1])
    assert torch.equal(f[0], f_ref[0]) and torch.equal(f[3], f_ref[3])
    # heads are independent too: sequence 1's head 0 never saw the NaN
    assert torch.equal(o[200:330, 0], o_ref[200:330, 0])


# ----------------------------------------------------------------------------- options vs oracle
@pytest.mark.parametrize("io,d", [("bf16", 128), ("fp32", 64)])
def test_scale_and_no_l2norm(lib, oracle, io, d):
    """scale = 0.25 on q̄ and qk_l2norm = 0 (q, k used as given: the recipe
    already draws unit rows, so the recurrence stays contractive)."""
    from kda_inputs import make_prefill
    inp = make_prefill([190, 64], 2, d, io, g_scale=0.5, s0_std=0.02, seed=39, device="cuda")
    for scale, l2 in ((0.25, True), (1.0, False), (0.5, False)):
        o, f = prefill(lib, inp, scale=scale, qk_l2norm=l2)
        o_ref, f_ref = oracle_prefill(oracle, inp, scale=scale, l2norm=l2)
        eo, ef = maxerr(host(o), o_ref), maxerr(host(f), f_ref)
        say(f"scale={scale} l2norm={l2} {io} d={d}: err_out={eo:.3e} err_state={ef:.3e}")
        assert eo <= TOL[io] and ef <= TOL[io]


def test_decode_scale_and_no_l2norm(lib, oracle):
    from kda_inputs import make_decode
    w = make_decode(4, 3, 128, "bf16", steps=3, seed=40, device="cuda")
    for scale, l2 in ((0.25, True), (0.5, False)):
        st = w["state"].clone()
        st_ref = host(w["state"]).astype(np.float64)
        for s in range(3):
            o = lib.kda_decode_step(w["q"][s], w["k"][s], w["v"][s], w["g"][s], w["beta"][s],
                                    st, scale=scale, qk_l2norm=l2)
            torch.cuda.synchronize()
            o_ref = oracle.decode_step(host(w["q"][s]), host(w["k"][s]), host(w["v"][s]),
                                       host(w["g"][s]), host(w["beta"][s]), st_ref,
                                       scale=scale, l2norm=l2)
            assert maxerr(host(o), o_ref) <= TOL["bf16"]
        assert maxerr(host(st), st_ref) <= TOL["bf16"]


@pytest.mark.parametrize("heads", [1, 5])
def test_odd_head_counts(lib, oracle, heads):
    from kda_inputs import make_prefill
    inp = make_prefill([129, 260], heads, 128, "bf16", g_scale=0.5, s0_std=0.02,
                       seed=41 + heads, device="cuda")
    o, f = prefill(lib, inp)
    o_ref, f_ref = oracle_prefill(oracle, inp)
    assert maxerr(host(o), o_ref) <= TOL["bf16"] and maxerr(host(f), f_ref) <= TOL["bf16"]


def test_many_short_sequences(lib, oracle):
    """300 packed sequences of 0..130 tokens (many single-chunk and empty
    sequences, more sequences than compute units)."""
    from kda_inputs import make_prefill
    rng = np.random.default_rng(43)
    lens = rng.integers(0, 131, size=300).tolist()
    lens[5] = 0
    lens[6] = 1
    inp = make_prefill(lens, 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=43, device="cuda")
    o, f = prefill(lib, inp)
    o_ref, f_ref = oracle_prefill(oracle, inp)
    eo, ef = maxerr(host(o), o_ref), maxerr(host(f), f_ref)
    say(f"300 short sequences ({sum(lens)} tokens): err_out={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
    # the empty sequence returns its initial state unchanged
    assert torch.equal(f[5], inp["initial_state"][5])


@pytest.mark.parametrize("d,n_seqs", [(128, 600), (64, 520)])
def test_wide_column_tiles(lib, oracle, monkeypatch, d, n_seqs):
    """Enough chains (sequences x 4 heads >= 2,048 / (d / 64)) that the
    recurrence takes 64-column tiles: ragged packed sequences of 0..200 tokens
    against the oracle.  This many chains would take the fused kernel, so the
    two-kernel path is forced (its checkpoint and output-gate variants are
    checked bit for bit against its plain result)."""
    monkeypatch.setenv("KDA_PREFILL_PATH", "split")
    from kda_inputs import make_prefill
    rng = np.random.default_rng(44 + d)
    lens = rng.integers(0, 201, size=n_seqs).tolist()
    lens[3] = 0
    inp = make_prefill(lens, 4, d, "bf16", g_scale=0.5, s0_std=0.02, seed=44, device="cuda")
    o, f = prefill(lib, inp)
    o_ref, f_ref = oracle_prefill(oracle, inp)
    eo, ef = maxerr(host(o), o_ref), maxerr(host(f), f_ref)
    say(f"{n_seqs} sequences x 4 heads d={d} ({sum(lens)} tokens): err_out={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
    assert torch.equal(f[3], inp["initial_state"][3])
    # checkpoints (the checkpointing 64-column kernel): every prefix state against
    # the oracle, and the plain outputs unchanged bit for bit
    out_c, fin_c, ck = lib.kda_chunk_prefill_checkpoints(
        inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"],
        inp["cu_seqlens"], checkpoint_interval=1)
    torch.cuda.synchronize()
    ref = _prefix_oracle_states(oracle, inp, lens, 1)
    assert ck.shape[0] == ref.shape[0] > 0
    assert maxerr(host(ck), ref) <= TOL["bf16"]
    assert torch.equal(out_c, o) and torch.equal(fin_c, f)
    # the output gate (which keeps 32-column tiles) against the oracle's gated read-out
    from kda_inputs import make_out_gate
    z = make_out_gate((sum(lens), 4), "bf16", seed=45, device="cuda")
    out_g, fin_g, _, _ = lib.kda_chunk_prefill_ex(
        inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"],
        inp["cu_seqlens"], out_gate_z=z)
    torch.cuda.synchronize()
    assert maxerr(host(out_g), oracle.apply_output_gate(o_ref, host(z))) <= TOL["bf16"]
    assert torch.equal(fin_g, f)


# ----------------------------------------------------------------------------- checkpoints
def _prefix_oracle_states(oracle, inp, lens, interval, heads=None):
    """Oracle final states of every checkpointed prefix: sequence n, prefix
    64 * interval * (j + 1) tokens, for each such length strictly inside n."""
    cu = np.cumsum([0] + list(lens))
    hs = list(range(inp["q"].shape[1])) if heads is None else list(heads)
    sel = lambda x: host(x[:, hs].contiguous())
    q, k, v, g = sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["g"])
    b = host(inp["beta"][:, hs].contiguous())
    s0 = None if inp["initial_state"] is None else host(inp["initial_state"][:, hs].contiguous())
    pieces, plens, init = [], [], []
    for n, L in enumerate(lens):
        step = 64 * interval
        P = step
        while P < L:
            pieces.append(slice(cu[n], cu[n] + P))
            plens.append(P)
            init.append(n)
            P += step
    if not pieces:
        return np.zeros((0, len(hs), q.shape[2], v.shape[2]))
    cat = lambda x: np.concatenate([x[sl] for sl in pieces], axis=0)
    pcu = np.cumsum([0] + plens).astype(np.int32)
    ps0 = None if s0 is None else s0[init]
    _, fin = oracle.prefill(cat(q), cat(k), cat(v), cat(g), cat(b), cu_seqlens=pcu,
                            initial_state=ps0, n_seqs=len(plens))
    return fin


@pytest.mark.parametrize("io,d", [("bf16", 128), ("fp32", 64)])
@pytest.mark.parametrize("interval", [1, 2, 3])
def test_checkpoints_match_oracle_prefixes(lib, oracle, io, d, interval):
    from kda_inputs import make_prefill
    lens = [1, 63, 64, 65, 0, 127, 128, 129, 300, 700]
    inp = make_prefill(lens, 3, d, io, g_scale=0.5, s0_std=0.02, seed=44, device="cuda")
    out, fin, ck = lib.kda_chunk_prefill_checkpoints(
        inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"],
        inp["cu_seqlens"], checkpoint_interval=interval)
    torch.cuda.synchronize()
    ref = _prefix_oracle_states(oracle, inp, lens, interval)
    assert ck.shape[0] == ref.shape[0] > 0
    e = maxerr(host(ck), ref)
    say(f"checkpoints {io} d={d} interval={interval}: {ck.shape[0]} states, err {e:.3e}")
    assert e <= TOL[io]
    # the plain call's results are unchanged, bit for bit
    o2, f2 = prefill(lib, inp)
    assert torch.equal(out, o2) and torch.equal(fin, f2)


def test_checkpoint_is_the_prefix_final_state(lib):
    """A checkpoint is bitwise the final state of a prefill of that prefix."""
    from kda_inputs import make_prefill
    inp = make_prefill([1000], 4, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=45, device="cuda")
    _, _, ck = lib.kda_chunk_prefill_checkpoints(
        inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"], None,
        checkpoint_interval=4)
    torch.cuda.synchronize()
    assert ck.shape[0] == 3  # after 256, 512, 768 tokens
    for j in range(3):
        P = 256 * (j + 1)
        _, f = prefill(lib, slice_tokens(inp, 0, P, inp["initial_state"]))
        assert torch.equal(ck[j], f[0]), f"checkpoint {j}"


def test_checkpoints_config1(lib, oracle):
    """T=8192, H=32: a checkpoint every 16 chunks (7 states per head); 2 seeded
    heads against the oracle's prefix states."""
    from kda_inputs import make_config_prefill, seeded_heads
    inp = make_config_prefill(1, device="cuda")
    out, fin, ck = lib.kda_chunk_prefill_checkpoints(
        inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"], None,
        checkpoint_interval=16)
    torch.cuda.synchronize()
    hs = seeded_heads(32, 2, 101)
    ref = _prefix_oracle_states(oracle, inp, [8192], 16, heads=hs)
    e = maxerr(host(ck[:, hs].contiguous()), ref)
    say(f"config1 checkpoints: {ck.shape[0]} states, err {e:.3e}")
    assert ck.shape[0] == 7 and e <= TOL["bf16"]


def test_decode_steps_replayed_from_a_graph(lib):
    """Four decode steps captured into a graph once (static token buffers, the
    state advanced in place) and replayed for three rounds of fresh tokens, with
    eager copies in between: every round's outputs and state equal the same
    steps run eagerly, bit for bit."""
    from kda_inputs import make_decode
    N, H, d, steps, rounds = 8, 4, 128, 4, 3
    w = make_decode(N, H, d, "bf16", steps=steps * rounds, seed=41, device="cuda")
    # eager reference
    st_ref = w["state"].clone()
    o_ref = []
    for s in range(steps * rounds):
        o_ref.append(lib.kda_decode_step(w["q"][s], w["k"][s], w["v"][s], w["g"][s],
                                         w["beta"][s], st_ref))
    torch.cuda.synchronize()
    # static buffers for one round
    bufs = {n: w[n][:steps].clone() for n in ("q", "k", "v", "g", "beta")}
    outs = torch.empty((steps, N, H, d), dtype=torch.bfloat16, device="cuda")
    st = w["state"].clone()

    def round_():
        for s in range(steps):
            lib.kda_decode_step(bufs["q"][s], bufs["k"][s], bufs["v"][s], bufs["g"][s],
                                bufs["beta"][s], st, outs[s])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        round_()                       # warm-up outside the graph (advances a scratch state)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    st.copy_(w["state"])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_()
    torch.cuda.synchronize()
    st.copy_(w["state"])               # capture does not run the steps
    for r in range(rounds):
        for n in bufs:
            bufs[n].copy_(w[n][r * steps:(r + 1) * steps])
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(outs[s], o_ref[r * steps + s]), f"round {r} step {s}"
        say(f"decode graph round {r}: outputs equal")
    assert torch.equal(st, st_ref)


def test_stream_given_as_a_handle(lib):
    """The binding takes a stream as a torch stream or as a raw handle (0 for the
    null stream): the same results either way, with the internal workspace kept
    alive for the stream the call ran on."""
    from kda_inputs import make_prefill
    inp = make_prefill([300, 77], 2, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=46, device="cuda")
    o_ref, f_ref = prefill(lib, inp)
    side = torch.cuda.Stream()
    for handle in (0, side.cuda_stream):
        torch.cuda.synchronize()
        o, f = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["initial_state"], inp["cu_seqlens"], stream=handle)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(f, f_ref), f"stream handle {handle}"
