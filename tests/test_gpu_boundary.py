"""GPU tests of the boundary's supported range, through the C ABI:

* fp32 I/O at d_k = d_v = 128 against the fp64 oracle (tolerance 1e-4);
* a prefill given no workspace (the library allocates one on the stream),
  bitwise equal to the same call with a caller workspace;
* launches split along the grid's y dimension: a prefill with more than 65,535
  chunk slots (on the two-kernel path, forced, and on the fused kernel its
  chain count picks) and a decode step over more than 65,535 sequences,
  against the oracle.
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
    return None if t is None else t.detach().float().cpu().numpy()


def maxerr(a, b):
    a = np.asarray(a, np.float64)
    return float(np.max(np.abs(a - np.asarray(b, np.float64)))) if a.size else 0.0


@pytest.fixture(scope="module")
def lib():
    import linear_attention_recurrence_06_amd as kda
    kda.load_library()
    return kda


def check(lib, oracle, inp, label, heads=None):
    out, fin = lib.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["initial_state"], inp["cu_seqlens"],
                                     num_seqs=len(inp["lens"]))
    torch.cuda.synchronize()
    hs = list(range(inp["q"].shape[1])) if heads is None else list(heads)
    sel = lambda x: host(x[:, hs].contiguous())
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].cpu().numpy()
    s0 = None if inp["initial_state"] is None else host(inp["initial_state"][:, hs].contiguous())
    o_ref, f_ref = oracle.prefill(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["g"]),
                                  sel(inp["beta"]), cu_seqlens=cu, initial_state=s0,
                                  n_seqs=len(inp["lens"]))
    o_gpu, f_gpu = host(out[:, hs]), host(fin[:, hs])
    eo, ef = maxerr(o_gpu, o_ref), maxerr(f_gpu, f_ref)
    tol = TOL[inp["io_dtype"]]
    say(f"[{label}] err_out={eo:.3e} err_state={ef:.3e} tol={tol}")
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(f_gpu))
    assert eo <= tol and ef <= tol
    return out, fin


def test_fp32_d128_ragged(lib, oracle):
    from kda_inputs import make_prefill
    inp = make_prefill([1, 63, 64, 65, 0, 127, 128, 129, 300], 3, 128, "fp32", g_scale=0.5,
                       s0_std=0.02, seed=401, device="cuda")
    check(lib, oracle, inp, "fp32 d=128 ragged")


def test_fp32_d128_long(lib, oracle):
    """8,192 tokens x 4 heads, fp32 I/O, d = 128."""
    from kda_inputs import make_prefill
    inp = make_prefill([8192], 4, 128, "fp32", g_scale=0.5, s0_std=0.02, seed=402,
                       device="cuda")
    check(lib, oracle, inp, "fp32 d=128 T=8192 H=4")


def test_fp32_d128_strong_decay_and_decode(lib, oracle):
    """fp32 d = 128 through the exact diagonal path (g = -8), then decode steps
    from its final state."""
    from kda_inputs import make_decode, make_prefill
    inp = make_prefill([200, 77], 2, 128, "fp32", g_scale=0.5, s0_std=0.02, seed=403,
                       device="cuda")
    inp["g"] = torch.full_like(inp["g"], -8.0)
    _, fin = check(lib, oracle, inp, "fp32 d=128 g=-8")
    w = make_decode(2, 2, 128, "fp32", steps=2, seed=404, device="cuda")
    st = fin.clone()
    st_ref = host(fin).astype(np.float64)
    for s in range(2):
        o = lib.kda_decode_step(w["q"][s], w["k"][s], w["v"][s], w["g"][s], w["beta"][s], st)
        torch.cuda.synchronize()
        o_ref = oracle.decode_step(host(w["q"][s]), host(w["k"][s]), host(w["v"][s]),
                                   host(w["g"][s]), host(w["beta"][s]), st_ref)
        assert maxerr(host(o), o_ref) <= TOL["fp32"]
    assert maxerr(host(st), st_ref) <= TOL["fp32"]


@pytest.mark.parametrize("lens,heads", [([300, 1, 700], 4), ([1 << 18], 16)])
def test_library_workspace_equals_caller_workspace(lib, lens, heads):
    """workspace NULL: the library allocates it on the stream (hipMallocAsync /
    hipFreeAsync).  Results are bitwise those of a caller workspace; the second
    shape (one 262,144-token sequence, 16 heads) takes the segmented path."""
    from kda_inputs import make_prefill
    inp = make_prefill(lens, heads, 128, "bf16", g_scale=0.5, s0_std=0.02, seed=405,
                       device="cuda", packed_cu=len(lens) > 1)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"],
            inp["cu_seqlens"])
    o1, f1 = lib.kda_chunk_prefill(*args, num_seqs=len(lens))
    o2, f2 = lib.kda_chunk_prefill(*args, num_seqs=len(lens), library_workspace=True)
    s = torch.cuda.Stream()
    # the side stream starts after the inputs exist (torch made them on the
    # current stream)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o3, f3 = lib.kda_chunk_prefill(*args, num_seqs=len(lens), library_workspace=True,
                                       stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    assert torch.equal(o1, o3) and torch.equal(f1, f3)


@pytest.mark.parametrize("path", ["split", "auto"])
def test_prefill_more_than_65535_chunk_slots(lib, oracle, monkeypatch, path):
    """65,600 one-token sequences plus one of 1,000 tokens: 66,641 chunk slots,
    so the preparation is launched in two grid ranges (the two-kernel path,
    forced: its 131,202 chains would take the fused kernel, which the second
    case runs)."""
    from kda_inputs import make_prefill
    if path == "split":
        monkeypatch.setenv("KDA_PREFILL_PATH", "split")
    else:
        monkeypatch.delenv("KDA_PREFILL_PATH", raising=False)
    lens = [1] * 65600 + [1000]
    inp = make_prefill(lens, 2, 64, "bf16", g_scale=0.5, s0_std=0.02, seed=406, device="cuda")
    check(lib, oracle, inp, f"66,641 chunk slots, {path}")


def test_decode_more_than_65535_sequences(lib, oracle):
    """One decode step over 66,000 sequences (two grid ranges)."""
    from kda_inputs import make_decode
    w = make_decode(66000, 1, 64, "bf16", steps=1, seed=407, device="cuda")
    st = w["state"].clone()
    st_ref = host(w["state"]).astype(np.float64)
    o = lib.kda_decode_step(w["q"][0], w["k"][0], w["v"][0], w["g"][0], w["beta"][0], st)
    torch.cuda.synchronize()
    o_ref = oracle.decode_step(host(w["q"][0]), host(w["k"][0]), host(w["v"][0]),
                               host(w["g"][0]), host(w["beta"][0]), st_ref)
    eo, es = maxerr(host(o), o_ref), maxerr(host(st), st_ref)
    say(f"[decode 66,000 sequences] err_out={eo:.3e} err_state={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
