"""The no-allocation prefill (kda_chunk_prefill_noalloc, for callers that
cannot allocate device memory) against kda_chunk_prefill with a caller
workspace: the same kernels on the same inputs, so the outputs and final
states must be bitwise equal.  Two calls in a row, the second smaller, so the
second runs on the array the first left behind.  Named to run last: it shares
the library's per-device array with nothing else in the suite."""

import sys

import pytest
import torch

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import linear_attention_recurrence_06_amd as kda
    kda.load_library()
    return kda


def run_pair(lib, inp):
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"],
            inp["cu_seqlens"])
    N = len(inp["lens"])
    o_ref, f_ref = lib.kda_chunk_prefill(*args, num_seqs=N)
    out = torch.empty_like(o_ref)
    fin = torch.empty_like(f_ref)
    lib.kda_chunk_prefill_noalloc(*args, out=out, final_state=fin, num_seqs=N)
    torch.cuda.synchronize()
    return o_ref, f_ref, out, fin


@pytest.mark.parametrize("io,d,lens,heads", [
    ("bf16", 128, [8192], 32),          # segmented: 8 chains per head in each pass
    ("fp32", 64, [8192], 8),            # the two-kernel path
    ("bf16", 128, [4096] * 16, 32),     # the fused kernel: 512 chains
    ("bf16", 128, [16384], 32),         # segmented, 28-chunk segments
])
def test_noalloc_equals_prefill_twice(lib, io, d, lens, heads):
    """The last two need far less of the array than kda_prefill_workspace_bytes
    (2.3 GiB and 0.6 GiB, past the array): the fused path uses only the
    index areas, the segmented path those and its state maps."""
    from kda_inputs import make_prefill
    big = make_prefill(lens, heads, d, io, g_scale=0.5, s0_std=0.02, seed=501, device="cuda",
                       packed_cu=len(lens) > 1)
    small = make_prefill([65, 1, 300], 3, d, io, g_scale=0.5, s0_std=0.02, seed=502,
                         device="cuda")
    for label, inp in (("first call", big), ("second, smaller call", small)):
        o_ref, f_ref, out, fin = run_pair(lib, inp)
        say(f"noalloc {io} d={d} {label}: tokens={sum(inp['lens'])} heads={inp['q'].shape[1]}")
        assert torch.equal(out, o_ref), label
        assert torch.equal(fin, f_ref), label


def test_noalloc_rejects_past_its_array(lib):
    """fp32 I/O takes the two-kernel path, whose records for 16,384 tokens x 32
    heads at d = 128 do not fit the array."""
    from kda_inputs import make_prefill
    inp = make_prefill([16384], 32, 128, "fp32", seed=503, device="cuda", packed_cu=False)
    dims = lib.make_dims(16384, 1, 32, 128, 128, lib.kda.KDA_FP32)
    assert lib.kda_prefill_workspace_bytes(dims) > lib.kda.KDA_NOALLOC_SCRATCH_BYTES
    out = torch.empty_like(inp["v"])
    with pytest.raises(lib.KDAError) as e:
        lib.kda_chunk_prefill_noalloc(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                      out=out)
    assert e.value.status == lib.kda.KDA_ERR_WORKSPACE
