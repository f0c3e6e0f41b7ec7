"""C ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, sizes workspaces, and rejects bad arguments with the
documented status codes before touching the device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_06_amd as pkg
    from linear_attention_recurrence_06_amd import build
    if not os.path.exists(pkg.kda.LIB_PATH):
        build.build(verbose=False)
    pkg.load_library()
    return pkg.kda


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_][a-z0-9_]*\s*\*?\s*(kda_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_and_library_agree(kda):
    names = declared_functions()
    assert set(names) >= {"kda_chunk_prefill", "kda_decode_step",
                          "kda_prefill_workspace_bytes", "kda_status_string", "kda_version"}
    lib = kda.load_library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kda.h but not exported"
    assert set(kda.EXPORTED) == set(names)


def test_status_strings(kda):
    for code, name in enumerate(["KDA_OK", "KDA_ERR_INVALID_ARG", "KDA_ERR_UNSUPPORTED",
                                 "KDA_ERR_MISALIGNED", "KDA_ERR_WORKSPACE", "KDA_ERR_HIP"]):
        assert kda.status_string(code) == name
    assert kda.load_library().kda_version() >= 10000


def test_workspace_bytes(kda):
    d = kda.make_dims(8192, 1, 32, 128, 128, kda.KDA_BF16)
    ws = kda.kda_prefill_workspace_bytes(d)
    # chunk index and checkpoint index (N+1 int32 each) and one (token, length)
    # descriptor per chunk slot, each padded to 256 B, then per (chunk slot,
    # head): W, Qhat, U (64x128), Kprime^T (128x64), M (64x64) bf16 and 128 fp32
    rec = (4 * 64 * 128 + 64 * 64) * 2 + 128 * 4
    slots = 8192 // 64 + 1
    desc = -(-slots * 8 // 256) * 256
    # plus, for one sequence, the fp32 state of every head (handed between the
    # segments of a pipelined call)
    assert ws == 2 * 256 + desc + rec * slots * 32 + 32 * 128 * 128 * 4
    d2 = kda.make_dims(8192, 2, 32, 128, 128, kda.KDA_BF16)
    slots2 = 8192 // 64 + 2
    desc2 = -(-slots2 * 8 // 256) * 256
    assert kda.kda_prefill_workspace_bytes(d2) == 2 * 256 + desc2 + rec * slots2 * 32
    # a rejected descriptor has no pipeline segment count and no path
    assert kda.kda_prefill_pipeline_segments(kda.make_dims(64, 1, 1, 96, 96, kda.KDA_BF16)) == -1
    assert kda.kda_prefill_path(kda.make_dims(64, 1, 1, 96, 96, kda.KDA_BF16))[0] == -1
    assert kda.kda_prefill_path_workspace_bytes(kda.make_dims(64, 1, 1, 96, 96, kda.KDA_BF16)) == 0
    # unsupported descriptors size to 0
    assert kda.kda_prefill_workspace_bytes(kda.make_dims(64, 1, 1, 96, 96, kda.KDA_BF16)) == 0
    # fp32 I/O at d = 128: the same record with 4-byte elements
    rec4 = (4 * 64 * 128 + 64 * 64) * 4 + 128 * 4
    d4 = kda.make_dims(8192, 2, 32, 128, 128, kda.KDA_FP32)
    assert kda.kda_prefill_workspace_bytes(d4) == 2 * 256 + desc2 + rec4 * slots2 * 32


FAKE = 1 << 40  # 16-byte aligned addresses the validation only compares, never dereferences


def prefill_call(kda, dims, **over):
    lib = kda.load_library()
    T, H, D = dims.total_tokens, dims.num_heads, dims.d_k
    E = 2 if dims.io_dtype == kda.KDA_BF16 else 4
    big = max(T * H * D * E, 1) + 4096
    ptr = {"q": FAKE, "k": FAKE + big, "v": FAKE + 2 * big, "g": FAKE + 3 * big,
           "beta": FAKE + 4 * big, "s0": None, "cu": None, "out": FAKE + 5 * big,
           "fin": None, "ws": FAKE + 6 * big}
    ptr.update(over)
    wsb = over.get("ws_bytes", kda.kda_prefill_workspace_bytes(dims))
    return lib.kda_chunk_prefill(ctypes.byref(dims), ptr["q"], ptr["k"], ptr["v"], ptr["g"],
                                 ptr["beta"], ptr["s0"], ptr["cu"], ptr["out"], ptr["fin"],
                                 ptr["ws"], wsb, None)


def test_prefill_validation(kda):
    d = kda.make_dims(256, 2, 4, 128, 128, kda.KDA_BF16)
    assert prefill_call(kda, d, q=None) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(kda, d, out=None) == kda.KDA_ERR_INVALID_ARG
    # (no workspace is valid -- the library allocates one on the stream -- so a
    # NULL workspace is only ever combined here with another error: a call that
    # passed validation would launch on these fake addresses)
    assert prefill_call(kda, d, ws=None, q=None) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(kda, d, ws=None, q=FAKE + 8) == kda.KDA_ERR_MISALIGNED
    # smaller than any path uses (the fused kernel's index areas, 768 bytes
    # here): rejected without asking the device; a plain bf16 call is otherwise
    # sized by its path, which needs the device
    assert prefill_call(kda, d, ws_bytes=512) == kda.KDA_ERR_WORKSPACE
    # the workspace must not overlap an input (the kernels write it)
    big = 256 * 4 * 128 * 2 + 4096
    assert prefill_call(kda, d, ws=FAKE + 3 * big + 256) == kda.KDA_ERR_INVALID_ARG   # over g
    assert prefill_call(kda, d, ws=FAKE - 4096) == kda.KDA_ERR_INVALID_ARG            # over q
    assert prefill_call(kda, d, s0=FAKE + 6 * big + 1024) == kda.KDA_ERR_INVALID_ARG  # S0 in it
    assert prefill_call(kda, d, q=FAKE + 8) == kda.KDA_ERR_MISALIGNED
    assert prefill_call(kda, d, beta=FAKE * 4 + 1) == kda.KDA_ERR_MISALIGNED
    assert prefill_call(kda, d, out=FAKE + 64) == kda.KDA_ERR_INVALID_ARG   # overlaps q
    bad = kda.make_dims(256, 2, 4, 96, 96, kda.KDA_BF16)
    assert prefill_call(kda, bad) == kda.KDA_ERR_UNSUPPORTED
    bad = kda.make_dims(256, 2, 4, 64, 128, kda.KDA_BF16)
    assert prefill_call(kda, bad) == kda.KDA_ERR_UNSUPPORTED
    bad = kda.make_dims(256, 2, 4, 128, 128, 7)
    assert prefill_call(kda, bad) == kda.KDA_ERR_UNSUPPORTED
    bad = kda.make_dims(256, 2, 4, 128, 128, kda.KDA_BF16, chunk=32)
    assert prefill_call(kda, bad) == kda.KDA_ERR_UNSUPPORTED
    bad = kda.make_dims(255, 2, 4, 128, 128, kda.KDA_BF16)   # uneven split without cu_seqlens
    assert prefill_call(kda, bad) == kda.KDA_ERR_INVALID_ARG
    # the supported range: T_total <= 2^31 - 1, H <= 65536
    bad = kda.make_dims(1 << 31, 1, 1, 128, 128, kda.KDA_BF16)
    assert prefill_call(kda, bad) == kda.KDA_ERR_UNSUPPORTED
    assert kda.kda_prefill_workspace_bytes(bad) == 0
    bad = kda.make_dims(64, 1, 65537, 128, 128, kda.KDA_BF16)
    assert prefill_call(kda, bad) == kda.KDA_ERR_UNSUPPORTED
    assert kda.kda_prefill_workspace_bytes(kda.make_dims(64, 1, 65536, 64, 64, kda.KDA_BF16)) > 0
    # final_state may be the same buffer as initial_state, but not a shifted view of it
    s = FAKE * 8
    assert prefill_call(kda, d, s0=s, fin=s + 64) == kda.KDA_ERR_INVALID_ARG
    # an empty batch is a no-op
    e = kda.make_dims(0, 0, 4, 128, 128, kda.KDA_BF16)
    assert prefill_call(kda, e) == kda.KDA_OK


def test_decode_validation(kda):
    lib = kda.load_library()
    d = kda.make_dims(8, 8, 2, 128, 128, kda.KDA_BF16)
    n = 8 * 2 * 128 * 2 + 4096
    args = [FAKE, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, FAKE + 4 * n, FAKE + 8 * n, FAKE + 5 * n]
    call = lambda a, dd=d: lib.kda_decode_step(ctypes.byref(dd), *a, None)
    assert call([None] + args[1:]) == kda.KDA_ERR_INVALID_ARG
    a = list(args); a[5] = FAKE + 8 * n + 4          # state must be 16-byte aligned
    assert call(a) == kda.KDA_ERR_MISALIGNED
    a = list(args); a[6] = args[0]                  # out overlaps q
    assert call(a) == kda.KDA_ERR_INVALID_ARG
    bad = kda.make_dims(9, 8, 2, 128, 128, kda.KDA_BF16)   # decode needs T == N
    assert call(args, bad) == kda.KDA_ERR_INVALID_ARG
    assert call(args, kda.make_dims(0, 0, 2, 128, 128, kda.KDA_BF16)) == kda.KDA_OK


def test_checkpoint_count(kda):
    """floor((ceil(len / 64) - 1) / interval) states per non-empty sequence."""
    d = kda.make_dims(8192, 1, 32, 128, 128, kda.KDA_BF16)
    assert kda.kda_checkpoint_count(d, None, 1) == 127
    assert kda.kda_checkpoint_count(d, None, 16) == 7
    assert kda.kda_checkpoint_count(d, None, 128) == 0
    lens = [1, 63, 64, 65, 0, 127, 128, 129, 300]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    dv = kda.make_dims(cu[-1], len(lens), 3, 128, 128, kda.KDA_BF16)
    chunks = [-(-L // 64) for L in lens]
    for interval in (1, 2, 3):
        expect = sum((c - 1) // interval for c in chunks if c > 0)
        assert kda.kda_checkpoint_count(dv, cu, interval) == expect
    assert kda.kda_checkpoint_count(dv, cu, 0) == -1
    assert kda.kda_checkpoint_count(kda.make_dims(100, 3, 1, 128, 128, kda.KDA_BF16), None, 1) == -1


def test_checkpoint_validation(kda):
    lib = kda.load_library()
    d = kda.make_dims(1024, 2, 4, 128, 128, kda.KDA_BF16)
    T, H, D = 1024, 4, 128
    big = T * H * D * 2 + 4096
    base = dict(q=FAKE, k=FAKE + big, v=FAKE + 2 * big, g=FAKE + 3 * big, beta=FAKE + 4 * big,
                out=FAKE + 5 * big, ws=FAKE + 6 * big, ck=FAKE + 20 * big)
    wsb = kda.kda_prefill_workspace_bytes(d)

    def call(interval, **over):
        p = dict(base)
        p.update(over)
        return lib.kda_chunk_prefill_checkpoints(
            ctypes.byref(d), p["q"], p["k"], p["v"], p["g"], p["beta"], None, None, p["out"],
            None, interval, p["ck"], p["ws"], wsb, None)

    assert call(0) == kda.KDA_ERR_INVALID_ARG
    assert call(-3) == kda.KDA_ERR_INVALID_ARG
    assert call(1, ck=None) == kda.KDA_ERR_INVALID_ARG
    assert call(1, ck=FAKE + 20 * big + 2) == kda.KDA_ERR_MISALIGNED
    # equal lengths: the checkpoint buffer (2 seqs x 7 states x 4 heads x 64 KiB) must
    # not overlap the output
    assert call(1, ck=FAKE + 5 * big + 64) == kda.KDA_ERR_INVALID_ARG


def test_gate_field_and_validation(kda):
    # the descriptor as laid out in include/kda.h: int64 + nine 4-byte fields, 8-aligned
    assert ctypes.sizeof(kda.kda_dims) == 48
    assert kda.kda_dims.gate.offset == 40
    d = kda.make_dims(1024, 1, 2, 128, 128, kda.KDA_BF16, gate=2)
    assert kda.kda_prefill_workspace_bytes(d) == 0
    assert prefill_call(kda, d) == kda.KDA_ERR_INVALID_ARG
    # the per-head gate reads g element by element: 2-byte alignment is enough
    d1 = kda.make_dims(1024, 1, 2, 128, 128, kda.KDA_BF16, gate=kda.KDA_GATE_HEAD)
    assert kda.kda_prefill_workspace_bytes(d1) == kda.kda_prefill_workspace_bytes(
        kda.make_dims(1024, 1, 2, 128, 128, kda.KDA_BF16))
    assert prefill_call(kda, d1, g=FAKE + 3 * (1024 * 2 * 128 * 2 + 4096) + 2,
                        ws_bytes=1024) == kda.KDA_ERR_WORKSPACE
    assert prefill_call(kda, d1, g=FAKE + 3 * (1024 * 2 * 128 * 2 + 4096) + 1) == \
        kda.KDA_ERR_MISALIGNED


def test_options_layout(kda):
    # the option structs as laid out in include/kda.h
    assert ctypes.sizeof(kda.kda_prefill_options) == 32
    assert kda.kda_prefill_options.checkpoints.offset == 8
    assert kda.kda_prefill_options.out_gate_z.offset == 16
    assert kda.kda_prefill_options.front_end.offset == 24
    assert ctypes.sizeof(kda.kda_decode_options) == 24
    assert kda.kda_decode_options.out_gate_z.offset == 8
    assert kda.kda_decode_options.front_end.offset == 16
    assert ctypes.sizeof(kda.kda_front_end) == 64
    assert kda.kda_front_end.conv_weight.offset == 8
    assert kda.kda_front_end.gate_rank.offset == 32
    assert kda.kda_front_end.gate_a.offset == 40
    assert kda.kda_front_end.gate_bias.offset == 56


def test_output_gate_validation(kda):
    lib = kda.load_library()
    d = kda.make_dims(1024, 2, 4, 128, 128, kda.KDA_BF16)
    T, H, D = 1024, 4, 128
    big = T * H * D * 2 + 4096
    base = dict(q=FAKE, k=FAKE + big, v=FAKE + 2 * big, g=FAKE + 3 * big, beta=FAKE + 4 * big,
                out=FAKE + 5 * big, ws=FAKE + 6 * big, z=FAKE + 30 * big, fin=None)
    wsb = kda.kda_prefill_workspace_bytes(d)

    def call(og, interval=0, null_opts=False, **over):
        p = dict(base, wsb=wsb)
        p.update(over)
        o = kda.kda_prefill_options(interval, og, None, p["z"])
        return lib.kda_chunk_prefill_ex(
            ctypes.byref(d), p["q"], p["k"], p["v"], p["g"], p["beta"], None, None, p["out"],
            p["fin"], None if null_opts else ctypes.byref(o), p["ws"], p["wsb"], None)

    assert call(3) == kda.KDA_ERR_INVALID_ARG
    assert call(-1) == kda.KDA_ERR_INVALID_ARG
    assert call(kda.KDA_OUT_GATE_CHANNEL, z=None) == kda.KDA_ERR_INVALID_ARG
    assert call(kda.KDA_OUT_GATE_HEAD, z=FAKE + 30 * big + 1) == kda.KDA_ERR_MISALIGNED
    # z is read element by element: 2-byte alignment is enough for bf16
    assert call(kda.KDA_OUT_GATE_CHANNEL, z=FAKE + 30 * big + 2, wsb=1024) == kda.KDA_ERR_WORKSPACE
    # z (an input) must not overlap out: T*H*d_v elements per channel, T*H per head
    assert call(kda.KDA_OUT_GATE_CHANNEL, z=FAKE + 5 * big - 64) == kda.KDA_ERR_INVALID_ARG
    assert call(kda.KDA_OUT_GATE_HEAD, z=FAKE + 5 * big - T * H * 2 + 2) == \
        kda.KDA_ERR_INVALID_ARG
    assert call(kda.KDA_OUT_GATE_CHANNEL, z=FAKE + 5 * big - T * H * 2) == \
        kda.KDA_ERR_INVALID_ARG
    # nor the final state
    assert call(kda.KDA_OUT_GATE_CHANNEL, fin=FAKE + 30 * big + 256) == kda.KDA_ERR_INVALID_ARG
    # with no gate, z is ignored (NULL options mean "no options"); such a call
    # may take the fused path, so only a workspace below its 768 bytes is
    # rejected without the device
    assert call(kda.KDA_OUT_GATE_NONE, z=None, wsb=512) == kda.KDA_ERR_WORKSPACE
    assert call(0, null_opts=True, wsb=512) == kda.KDA_ERR_WORKSPACE
    # an empty batch is a no-op even with a gate and no z
    e = kda.make_dims(0, 0, 4, 128, 128, kda.KDA_BF16)
    o = kda.kda_prefill_options(0, kda.KDA_OUT_GATE_CHANNEL, None, None)
    assert lib.kda_chunk_prefill_ex(ctypes.byref(e), None, None, None, None, None, None, None,
                                    None, None, ctypes.byref(o), FAKE, 0, None) == kda.KDA_OK


def test_decode_output_gate_validation(kda):
    lib = kda.load_library()
    d = kda.make_dims(8, 8, 2, 128, 128, kda.KDA_BF16)
    n = 8 * 2 * 128 * 2 + 4096
    args = [FAKE, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, FAKE + 4 * n, FAKE + 8 * n, FAKE + 5 * n]
    z = FAKE + 12 * n

    def call(og, zz=z, a=args):
        o = kda.kda_decode_options(og, 0, zz, None)
        return lib.kda_decode_step_ex(ctypes.byref(d), *a, ctypes.byref(o), None)

    assert call(5) == kda.KDA_ERR_INVALID_ARG
    assert call(kda.KDA_OUT_GATE_HEAD, None) == kda.KDA_ERR_INVALID_ARG
    assert call(kda.KDA_OUT_GATE_CHANNEL, z + 1) == kda.KDA_ERR_MISALIGNED
    assert call(kda.KDA_OUT_GATE_CHANNEL, args[6] + 64) == kda.KDA_ERR_INVALID_ARG  # overlaps out
    a = list(args); a[5] = FAKE + 8 * n + 4
    assert call(kda.KDA_OUT_GATE_CHANNEL, z, a) == kda.KDA_ERR_MISALIGNED
    assert call(kda.KDA_OUT_GATE_HEAD, args[5] + 4096) == kda.KDA_ERR_INVALID_ARG  # in the state


def test_front_end_validation(kda):
    lib = kda.load_library()
    d = kda.make_dims(1024, 2, 4, 128, 128, kda.KDA_BF16)
    T, H, D = 1024, 4, 128
    big = T * H * D * 2 + 4096
    base = dict(q=FAKE, k=FAKE + big, v=FAKE + 2 * big, g=FAKE + 3 * big, beta=FAKE + 4 * big,
                out=FAKE + 5 * big, ws=FAKE + 6 * big)
    wsb = kda.kda_prefill_workspace_bytes(d)
    W0, A0, B0, S0, S1 = (FAKE + 40 * big, FAKE + 41 * big, FAKE + 42 * big, FAKE + 43 * big,
                          FAKE + 44 * big)

    def fe(**over):
        f = dict(conv_width=4, conv_silu=1, conv_weight=W0, conv_state_in=S0, conv_state_out=S1,
                 gate_rank=64, reserved=0, gate_a=A0, gate_b=B0, gate_bias=None)
        f.update(over)
        return kda.kda_front_end(**f)

    def call(f, **over):
        p = dict(base, wsb=wsb)
        p.update(over)
        o = kda.kda_prefill_options(0, 0, None, None, ctypes.pointer(f) if f else None)
        return lib.kda_chunk_prefill_ex(ctypes.byref(over.get("dims", d)), p["q"], p["k"], p["v"],
                                        p["g"], p["beta"], None, None, p["out"], None,
                                        ctypes.byref(o), p["ws"], p["wsb"], None)

    INV, MIS, WS = kda.KDA_ERR_INVALID_ARG, kda.KDA_ERR_MISALIGNED, kda.KDA_ERR_WORKSPACE
    # a valid front end (low-rank gate, so g NULL) reaches the workspace check
    assert call(fe(), g=None, wsb=1024) == WS
    # with a low-rank gate g must be NULL; without one it is required
    assert call(fe()) == INV
    assert call(fe(gate_rank=0, gate_a=None, gate_b=None), g=None) == INV
    assert call(fe(gate_rank=0, gate_a=None, gate_b=None), wsb=1024) == WS
    assert call(None, g=None) == INV
    for bad in (dict(conv_width=5), dict(conv_width=-1), dict(conv_silu=2), dict(reserved=1),
                dict(gate_rank=48), dict(gate_rank=256), dict(conv_weight=None),
                dict(gate_a=None), dict(gate_b=None)):
        assert call(fe(**bad), g=None) == INV, bad
    # the low-rank gate is per channel: not with the per-head gate descriptor
    dh = kda.make_dims(1024, 2, 4, 128, 128, kda.KDA_BF16, gate=kda.KDA_GATE_HEAD)
    assert call(fe(), g=None, dims=dh) == INV
    # alignment: 16 bytes for the tensors, 4 for the bias
    for name, val in (("conv_weight", W0 + 8), ("conv_state_in", S0 + 8),
                      ("conv_state_out", S1 + 8), ("gate_a", A0 + 8), ("gate_b", B0 + 8),
                      ("gate_bias", FAKE + 45 * big + 2)):
        assert call(fe(**{name: val}), g=None) == MIS, name
    # conv states are not read or written at width 1, so they are not checked
    assert call(fe(conv_width=1, conv_state_in=S0 + 8, conv_state_out=S1 + 8), g=None,
                wsb=1024) == WS
    # the conv state output must not overlap an input or another output
    assert call(fe(conv_state_out=base["q"] + 64), g=None) == INV
    assert call(fe(conv_state_out=base["out"] + 64), g=None) == INV
    assert call(fe(conv_state_out=S0 + 64), g=None) == INV
    assert call(fe(conv_state_out=A0), g=None) == INV
    # out must not overlap the front end's inputs
    assert call(fe(), g=None, out=W0) == INV
    assert call(fe(), g=None, out=B0 - 64) == INV


def test_decode_front_end_validation(kda):
    lib = kda.load_library()
    d = kda.make_dims(8, 8, 2, 128, 128, kda.KDA_BF16)
    n = 8 * 2 * 128 * 2 + 4096
    args = [FAKE, FAKE + n, FAKE + 2 * n, None, FAKE + 4 * n, FAKE + 8 * n, FAKE + 5 * n]
    W0, A0, B0, S0 = FAKE + 20 * n, FAKE + 21 * n, FAKE + 22 * n, FAKE + 23 * n

    def call(a=args, **over):
        f = dict(conv_width=3, conv_silu=0, conv_weight=W0, conv_state_in=S0, conv_state_out=S0,
                 gate_rank=32, reserved=0, gate_a=A0, gate_b=B0, gate_bias=None)
        f.update(over)
        fe = kda.kda_front_end(**f)
        o = kda.kda_decode_options(0, 0, None, ctypes.pointer(fe))
        return lib.kda_decode_step_ex(ctypes.byref(d), *a, ctypes.byref(o), None)

    INV, MIS = kda.KDA_ERR_INVALID_ARG, kda.KDA_ERR_MISALIGNED
    # (the in-place conv state is allowed; a misaligned recurrent state stops the call)
    a = list(args); a[5] = FAKE + 8 * n + 4
    assert call(a) == MIS
    assert call(conv_state_out=S0 + 64) == INV      # partial overlap with the input state
    assert call(conv_state_out=args[6]) == INV      # the conv state over out
    assert call(gate_rank=0, gate_a=None, gate_b=None) == INV  # no gate at all
    assert call(gate_a=A0 + 4) == MIS


def test_noalloc_validation(kda):
    """The no-allocation prefill rejects sizes past its per-device array and bad
    arguments before touching the device (every call here is rejected: a call
    that passed validation would launch on these fake addresses).  The size
    check needs no device where only the two-kernel path applies (fp32 I/O);
    a bf16 call is sized by the path the device's CU count picks."""
    lib = kda.load_library()
    cap = 320 << 20
    fits = kda.make_dims(8192, 1, 32, 128, 128, kda.KDA_BF16)
    assert kda.kda_prefill_workspace_bytes(fits) <= cap
    too_big = kda.make_dims(16384, 1, 32, 128, 128, kda.KDA_FP32)
    assert kda.kda_prefill_workspace_bytes(too_big) > cap
    T, H, D = 16384, 32, 128
    big = T * H * D * 4 + 4096
    p = [FAKE, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, FAKE + 4 * big, None, None,
         FAKE + 5 * big, None]
    call = lambda dd, a: lib.kda_chunk_prefill_noalloc(ctypes.byref(dd), *a, None)
    assert call(too_big, p) == kda.KDA_ERR_WORKSPACE
    assert call(kda.make_dims(256, 1, 4, 96, 96, kda.KDA_BF16), p) == kda.KDA_ERR_UNSUPPORTED
    a = list(p); a[0] = None
    assert call(fits, a) == kda.KDA_ERR_INVALID_ARG
    a = list(p); a[7] = FAKE + 64                     # out over q
    assert call(fits, a) == kda.KDA_ERR_INVALID_ARG
    a = list(p); a[1] = FAKE + big + 8                # k misaligned
    assert call(fits, a) == kda.KDA_ERR_MISALIGNED
