"""Python binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the stream; there
is no CPU path.  If libkda.so is missing or fails to load, every call raises.

    out, final = kda_chunk_prefill(q, k, v, g, beta, initial_state, cu_seqlens)
    out = kda_decode_step(q, k, v, g, beta, state)        # state updated in place

Layouts (contiguous, token-major): q, k, g ``[T, H, d_k]``; v, out ``[T, H, d_v]``;
beta ``[T, H]``; states ``[N, H, d_k, d_v]`` float32; cu_seqlens int32 ``[N+1]``.
A g of shape ``[T, H]`` (decode ``[N, H]``) selects the per-head (scalar) gate.
q, k, v, g, beta share one dtype (bfloat16 or float32), which is also out's.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_MISALIGNED, \
    KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(6)
KDA_BF16, KDA_FP32 = 0, 1
KDA_GATE_CHANNEL, KDA_GATE_HEAD = 0, 1
KDA_PATH_SPLIT, KDA_PATH_PIPELINED, KDA_PATH_FUSED, KDA_PATH_SEGMENTED = range(4)

#: every symbol include/kda.h declares
EXPORTED = ("kda_prefill_workspace_bytes", "kda_chunk_prefill", "kda_checkpoint_count",
            "kda_chunk_prefill_checkpoints", "kda_chunk_prefill_ex", "kda_decode_step",
            "kda_decode_step_ex", "kda_status_string", "kda_version",
            "kda_prefill_pipeline_segments", "kda_chunk_prefill_noalloc", "kda_prefill_path",
            "kda_prefill_path_workspace_bytes")

#: bytes of the per-device array kda_chunk_prefill_noalloc uses as its workspace
KDA_NOALLOC_SCRATCH_BYTES = 320 << 20


class kda_dims(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("qk_l2norm", ctypes.c_int32),
        ("gate", ctypes.c_int32),
    ]


KDA_OUT_GATE_NONE, KDA_OUT_GATE_CHANNEL, KDA_OUT_GATE_HEAD = 0, 1, 2


class kda_front_end(ctypes.Structure):
    _fields_ = [
        ("conv_width", ctypes.c_int32),
        ("conv_silu", ctypes.c_int32),
        ("conv_weight", ctypes.c_void_p),
        ("conv_state_in", ctypes.c_void_p),
        ("conv_state_out", ctypes.c_void_p),
        ("gate_rank", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("gate_a", ctypes.c_void_p),
        ("gate_b", ctypes.c_void_p),
        ("gate_bias", ctypes.c_void_p),
    ]


class kda_prefill_options(ctypes.Structure):
    _fields_ = [
        ("checkpoint_interval", ctypes.c_int32),
        ("out_gate", ctypes.c_int32),
        ("checkpoints", ctypes.c_void_p),
        ("out_gate_z", ctypes.c_void_p),
        ("front_end", ctypes.POINTER(kda_front_end)),
    ]


class kda_decode_options(ctypes.Structure):
    _fields_ = [
        ("out_gate", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("out_gate_z", ctypes.c_void_p),
        ("front_end", ctypes.POINTER(kda_front_end)),
    ]


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkda.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m linear_attention_recurrence_06_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(kda_dims)
    lib.kda_prefill_workspace_bytes.argtypes = [D]
    lib.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_prefill.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.kda_chunk_prefill.restype = ctypes.c_int
    lib.kda_checkpoint_count.argtypes = [D, P, ctypes.c_int32]
    lib.kda_checkpoint_count.restype = ctypes.c_int64
    lib.kda_chunk_prefill_checkpoints.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_int32,
                                                  P, P, ctypes.c_size_t, P]
    lib.kda_chunk_prefill_checkpoints.restype = ctypes.c_int
    lib.kda_chunk_prefill_ex.argtypes = [D, P, P, P, P, P, P, P, P, P,
                                         ctypes.POINTER(kda_prefill_options), P,
                                         ctypes.c_size_t, P]
    lib.kda_chunk_prefill_ex.restype = ctypes.c_int
    lib.kda_decode_step_ex.argtypes = [D, P, P, P, P, P, P, P,
                                       ctypes.POINTER(kda_decode_options), P]
    lib.kda_decode_step_ex.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [D, P, P, P, P, P, P, P, P]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int
    lib.kda_prefill_pipeline_segments.argtypes = [D]
    lib.kda_prefill_pipeline_segments.restype = ctypes.c_int32
    lib.kda_prefill_path.argtypes = [D, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.kda_prefill_path.restype = ctypes.c_int32
    lib.kda_prefill_path_workspace_bytes.argtypes = [D, ctypes.c_int32]
    lib.kda_prefill_path_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_prefill_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
    lib.kda_chunk_prefill_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_FP32
    raise TypeError(f"unsupported I/O dtype {t.dtype}; use bfloat16 or float32")


def _stream_handle(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(need: int, device, stream) -> torch.Tensor:
    """The call's internal workspace.  torch hands freed memory on to later
    work of the stream it was allocated on, so a workspace used on another
    stream is recorded on that stream: its memory is not reused before the
    call's kernels there are done."""
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if stream is not None:
        if isinstance(stream, torch.cuda.Stream):
            s = stream
        elif int(stream) == 0:   # the null stream
            s = torch.cuda.default_stream(device)
        else:
            s = torch.cuda.ExternalStream(int(stream), device=device)
        if s != torch.cuda.current_stream(device):
            ws.record_stream(s)
    return ws


def make_dims(total_tokens: int, num_seqs: int, num_heads: int, d_k: int, d_v: int,
              io_dtype: int, scale: float = 1.0, qk_l2norm: bool = True,
              chunk: int = 64, gate: int = KDA_GATE_CHANNEL) -> kda_dims:
    return kda_dims(int(total_tokens), int(num_seqs), int(num_heads), int(d_k), int(d_v),
                    int(chunk), int(io_dtype), float(scale), 1 if qk_l2norm else 0, int(gate))


def _gate(g: torch.Tensor, lead) -> int:
    """KDA_GATE_HEAD when g has no key-channel axis ([T, H] / [N, H])."""
    return KDA_GATE_HEAD if g.dim() == len(lead) else KDA_GATE_CHANNEL


def kda_prefill_workspace_bytes(dims: kda_dims) -> int:
    return int(load_library().kda_prefill_workspace_bytes(ctypes.byref(dims)))


def kda_prefill_path_workspace_bytes(dims: kda_dims, packed: bool = False) -> int:
    """Bytes of workspace a plain prefill of these sizes uses on the current
    device (the path's own need; 0 for a rejected descriptor)."""
    return int(load_library().kda_prefill_path_workspace_bytes(ctypes.byref(dims),
                                                               int(bool(packed))))


def kda_prefill_pipeline_segments(dims: kda_dims) -> int:
    """Segments a prefill of these sizes is pipelined into on the current
    device (0: one launch of each kernel or another path; -1: rejected
    descriptor)."""
    return int(load_library().kda_prefill_pipeline_segments(ctypes.byref(dims)))


def kda_prefill_path(dims: kda_dims, packed: bool = False):
    """(path, segments) a plain prefill of these sizes takes on the current
    device: path one of KDA_PATH_*, or -1 for a rejected descriptor."""
    seg = ctypes.c_int32(0)
    path = int(load_library().kda_prefill_path(ctypes.byref(dims), int(bool(packed)),
                                               ctypes.byref(seg)))
    return path, int(seg.value)


def _check_tensor(name, t, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def kda_chunk_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None,
                      final_state: Optional[torch.Tensor] = None, *,
                      num_seqs: Optional[int] = None, scale: float = 1.0,
                      qk_l2norm: bool = True, workspace: Optional[torch.Tensor] = None,
                      output_final_state: bool = True, library_workspace: bool = False,
                      stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked KDA prefill over packed sequences (see include/kda.h).

    Returns ``(out, final_state)``; ``final_state`` is None when
    ``output_final_state`` is False and none was passed.  Without
    ``cu_seqlens`` the T tokens form ``num_seqs`` (default 1) equal sequences.
    The workspace is ``workspace``, else one allocated here with torch, else
    (``library_workspace=True``) none: the library then allocates it
    stream-ordered on ``stream``.
    """
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    dt = q.dtype
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        _check_tensor("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    gate = _gate(g, (T, H))
    for name, t, shp in (("q", q, (T, H, dk)), ("k", k, (T, H, dk)),
                         ("g", g, (T, H) if gate else (T, H, dk)),
                         ("v", v, (T, H, dv)), ("beta", beta, (T, H))):
        _check_tensor(name, t, shp, dt, dev)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((T, H, dv), dtype=dt, device=dev)
    else:
        _check_tensor("out", out, (T, H, dv), dt, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check_tensor("final_state", final_state, (N, H, dk, dv), torch.float32, dev)
    dims = make_dims(T, N, H, dk, dv, _io_dtype(q), scale, qk_l2norm, gate=gate)
    if workspace is None and not library_workspace:
        # what this call's path uses (the fused and segmented paths need out
        # aligned to 16 bytes; otherwise the two-kernel workspace)
        if out.data_ptr() % 16 == 0:
            with torch.cuda.device(dev):
                need = kda_prefill_path_workspace_bytes(dims, cu_seqlens is not None)
        else:
            need = kda_prefill_workspace_bytes(dims)
        workspace = _workspace(need, dev, stream)
    rc = lib.kda_chunk_prefill(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                               _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens), _ptr(out),
                               _ptr(final_state), _ptr(workspace),
                               0 if workspace is None else workspace.numel(),
                               _stream_handle(stream, dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_prefill")
    return out, final_state


def kda_chunk_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              g: torch.Tensor, beta: torch.Tensor,
                              initial_state: Optional[torch.Tensor] = None,
                              cu_seqlens: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None,
                              final_state: Optional[torch.Tensor] = None, *,
                              num_seqs: Optional[int] = None, scale: float = 1.0,
                              qk_l2norm: bool = True, stream=None):
    """The prefill through kda_chunk_prefill_noalloc (include/kda.h): the library
    uses its per-device array as the workspace and allocates nothing.  ``out``
    and ``final_state`` must be given (this wrapper allocates nothing either).
    Returns ``(out, final_state)``."""
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    dt = q.dtype
    if out is None:
        raise ValueError("kda_chunk_prefill_noalloc: pass out (nothing is allocated here)")
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        _check_tensor("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    gate = _gate(g, (T, H))
    for name, t, shp in (("q", q, (T, H, dk)), ("k", k, (T, H, dk)),
                         ("g", g, (T, H) if gate else (T, H, dk)),
                         ("v", v, (T, H, dv)), ("beta", beta, (T, H)), ("out", out, (T, H, dv))):
        _check_tensor(name, t, shp, dt, dev)
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _check_tensor(name, t, (N, H, dk, dv), torch.float32, dev)
    dims = make_dims(T, N, H, dk, dv, _io_dtype(q), scale, qk_l2norm, gate=gate)
    rc = lib.kda_chunk_prefill_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
                                       _ptr(out), _ptr(final_state),
                                       _stream_handle(stream, dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_prefill_noalloc")
    return out, final_state


def kda_checkpoint_count(dims: kda_dims, host_cu_seqlens=None, checkpoint_interval: int = 1) -> int:
    """Number of intermediate states a checkpointed prefill writes (host
    cu_seqlens: any int sequence, or None for equal lengths)."""
    lib = load_library()
    if host_cu_seqlens is None:
        return int(lib.kda_checkpoint_count(ctypes.byref(dims), None, int(checkpoint_interval)))
    arr = (ctypes.c_int32 * len(host_cu_seqlens))(*[int(x) for x in host_cu_seqlens])
    return int(lib.kda_checkpoint_count(ctypes.byref(dims), arr, int(checkpoint_interval)))


def kda_chunk_prefill_checkpoints(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  g: torch.Tensor, beta: torch.Tensor,
                                  initial_state: Optional[torch.Tensor] = None,
                                  cu_seqlens: Optional[torch.Tensor] = None,
                                  out: Optional[torch.Tensor] = None,
                                  final_state: Optional[torch.Tensor] = None, *,
                                  checkpoint_interval: int,
                                  checkpoints: Optional[torch.Tensor] = None,
                                  host_cu_seqlens=None, num_seqs: Optional[int] = None,
                                  scale: float = 1.0, qk_l2norm: bool = True,
                                  workspace: Optional[torch.Tensor] = None,
                                  output_final_state: bool = True, stream=None):
    """Chunked prefill that also returns intermediate states (include/kda.h,
    kda_chunk_prefill_checkpoints).  Returns ``(out, final_state, checkpoints)``
    with checkpoints ``[C, H, d_k, d_v]`` float32: sequence n's states after
    each ``64 * checkpoint_interval`` of its tokens, strictly inside it.  Sizing
    needs the lengths on the host: pass ``host_cu_seqlens`` or they are copied
    from ``cu_seqlens``."""
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    dt = q.dtype
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        _check_tensor("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
        if host_cu_seqlens is None:
            host_cu_seqlens = cu_seqlens.cpu().tolist()
    else:
        N = 1 if num_seqs is None else int(num_seqs)
        host_cu_seqlens = None
    gate = _gate(g, (T, H))
    for name, t, shp in (("q", q, (T, H, dk)), ("k", k, (T, H, dk)),
                         ("g", g, (T, H) if gate else (T, H, dk)),
                         ("v", v, (T, H, dv)), ("beta", beta, (T, H))):
        _check_tensor(name, t, shp, dt, dev)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((T, H, dv), dtype=dt, device=dev)
    else:
        _check_tensor("out", out, (T, H, dv), dt, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check_tensor("final_state", final_state, (N, H, dk, dv), torch.float32, dev)
    dims = make_dims(T, N, H, dk, dv, _io_dtype(q), scale, qk_l2norm, gate=gate)
    C = kda_checkpoint_count(dims, host_cu_seqlens, checkpoint_interval)
    if C < 0:
        raise KDAError(KDA_ERR_INVALID_ARG, "kda_checkpoint_count")
    if checkpoints is None:
        checkpoints = torch.empty((max(C, 1), H, dk, dv), dtype=torch.float32, device=dev)
    elif checkpoints.shape[0] < C or tuple(checkpoints.shape[1:]) != (H, dk, dv):
        raise ValueError(f"checkpoints must be [>= {C}, {H}, {dk}, {dv}] float32")
    need = kda_prefill_workspace_bytes(dims)
    if workspace is None:
        workspace = _workspace(need, dev, stream)
    rc = lib.kda_chunk_prefill_checkpoints(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(initial_state), _ptr(cu_seqlens), _ptr(out), _ptr(final_state),
        int(checkpoint_interval), _ptr(checkpoints), _ptr(workspace), workspace.numel(),
        _stream_handle(stream, dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_prefill_checkpoints")
    return out, final_state, checkpoints[:C]


def kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, state: torch.Tensor,
                    out: Optional[torch.Tensor] = None, *, scale: float = 1.0,
                    qk_l2norm: bool = True, stream=None) -> torch.Tensor:
    """One KDA decode step (one token per sequence); ``state`` [N,H,d_k,d_v]
    float32 is advanced in place.  Returns ``out`` [N,H,d_v]."""
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    dt = q.dtype
    gate = _gate(g, (N, H))
    for name, t, shp in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)),
                         ("g", g, (N, H) if gate else (N, H, dk)),
                         ("v", v, (N, H, dv)), ("beta", beta, (N, H))):
        _check_tensor(name, t, shp, dt, dev)
    _check_tensor("state", state, (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _check_tensor("out", out, (N, H, dv), dt, dev)
    dims = make_dims(N, N, H, dk, dv, _io_dtype(q), scale, qk_l2norm, gate=gate)
    rc = lib.kda_decode_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                             _ptr(beta), _ptr(state), _ptr(out), _stream_handle(stream, dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_decode_step")
    return out


def _out_gate(z: Optional[torch.Tensor], lead, dv: int, dt, dev) -> int:
    if z is None:
        return KDA_OUT_GATE_NONE
    if z.dim() == len(lead):
        _check_tensor("out_gate_z", z, tuple(lead), dt, dev)
        return KDA_OUT_GATE_HEAD
    _check_tensor("out_gate_z", z, tuple(lead) + (dv,), dt, dev)
    return KDA_OUT_GATE_CHANNEL


def _front_end(lead, N: int, H: int, d: int, dt, dev, conv_weight, conv_silu, conv_state_in,
               conv_state_out, gate_a, gate_b, gate_bias):
    """Checks the front-end tensors and builds the kda_front_end descriptor
    (None without a front end)."""
    if conv_weight is None and gate_a is None:
        return None
    fe = kda_front_end()
    if conv_weight is not None:
        W = conv_weight.shape[2]
        _check_tensor("conv_weight", conv_weight, (3, H, W, d), dt, dev)
        fe.conv_width = W
        fe.conv_silu = 1 if conv_silu else 0
        fe.conv_weight = _ptr(conv_weight)
        for name, t in (("conv_state_in", conv_state_in), ("conv_state_out", conv_state_out)):
            if t is not None:
                _check_tensor(name, t, (N, 3, W - 1, H, d), dt, dev)
        fe.conv_state_in = _ptr(conv_state_in)
        fe.conv_state_out = _ptr(conv_state_out)
    if gate_a is not None:
        r = gate_a.shape[-1]
        _check_tensor("gate_a", gate_a, tuple(lead) + (r,), dt, dev)
        _check_tensor("gate_b", gate_b, (H, d, r), dt, dev)
        if gate_bias is not None:
            _check_tensor("gate_bias", gate_bias, (H, d), torch.float32, dev)
        fe.gate_rank = r
        fe.gate_a = _ptr(gate_a)
        fe.gate_b = _ptr(gate_b)
        fe.gate_bias = _ptr(gate_bias)
    return fe


def kda_chunk_prefill_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         g: Optional[torch.Tensor], beta: torch.Tensor,
                         initial_state: Optional[torch.Tensor] = None,
                         cu_seqlens: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None,
                         final_state: Optional[torch.Tensor] = None, *,
                         out_gate_z: Optional[torch.Tensor] = None,
                         checkpoint_interval: int = 0,
                         checkpoints: Optional[torch.Tensor] = None,
                         conv_weight: Optional[torch.Tensor] = None, conv_silu: bool = False,
                         conv_state_in: Optional[torch.Tensor] = None,
                         conv_state_out: Optional[torch.Tensor] = None,
                         output_conv_state: bool = False,
                         gate_a: Optional[torch.Tensor] = None,
                         gate_b: Optional[torch.Tensor] = None,
                         gate_bias: Optional[torch.Tensor] = None,
                         host_cu_seqlens=None, num_seqs: Optional[int] = None,
                         scale: float = 1.0, qk_l2norm: bool = True,
                         workspace: Optional[torch.Tensor] = None,
                         output_final_state: bool = True, stream=None):
    """Chunked prefill with options (include/kda.h, kda_chunk_prefill_ex):
    checkpoints; the output gate out = o * sigmoid(z) (z ``[T,H,d_v]`` per
    channel or ``[T,H]`` per head); the front end (q, k, v raw projections
    convolved with ``conv_weight [3,H,W,d]``, optional SiLU, conv states
    ``[N,3,W-1,H,d]``; g = -softplus(gate_a gate_b^T + gate_bias) with
    ``gate_a [T,r]``, ``gate_b [H,d,r]``, ``gate_bias [H,d]`` fp32, g None).
    Returns ``(out, final_state, checkpoints, conv_state_out)`` (None where not
    asked for)."""
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    dt = q.dtype
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        _check_tensor("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    gate = _gate(g, (T, H)) if g is not None else KDA_GATE_CHANNEL
    for name, t, shp in (("q", q, (T, H, dk)), ("k", k, (T, H, dk)),
                         ("v", v, (T, H, dv)), ("beta", beta, (T, H))):
        _check_tensor(name, t, shp, dt, dev)
    if g is not None:
        _check_tensor("g", g, (T, H) if gate else (T, H, dk), dt, dev)
    og = _out_gate(out_gate_z, (T, H), dv, dt, dev)
    if conv_weight is not None and conv_state_out is None and output_conv_state:
        W = conv_weight.shape[2]
        conv_state_out = torch.empty((N, 3, W - 1, H, dk), dtype=dt, device=dev)
    fe = _front_end((T,), N, H, dk, dt, dev, conv_weight, conv_silu, conv_state_in,
                    conv_state_out, gate_a, gate_b, gate_bias)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((T, H, dv), dtype=dt, device=dev)
    else:
        _check_tensor("out", out, (T, H, dv), dt, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check_tensor("final_state", final_state, (N, H, dk, dv), torch.float32, dev)
    dims = make_dims(T, N, H, dk, dv, _io_dtype(q), scale, qk_l2norm, gate=gate)
    C = 0
    if checkpoint_interval:
        if cu_seqlens is not None and host_cu_seqlens is None:
            host_cu_seqlens = cu_seqlens.cpu().tolist()
        C = kda_checkpoint_count(dims, host_cu_seqlens if cu_seqlens is not None else None,
                                 checkpoint_interval)
        if C < 0:
            raise KDAError(KDA_ERR_INVALID_ARG, "kda_checkpoint_count")
        if checkpoints is None:
            checkpoints = torch.empty((max(C, 1), H, dk, dv), dtype=torch.float32, device=dev)
    opts = kda_prefill_options(int(checkpoint_interval), og, _ptr(checkpoints), _ptr(out_gate_z),
                               ctypes.pointer(fe) if fe is not None else None)
    need = kda_prefill_workspace_bytes(dims)
    if workspace is None:
        workspace = _workspace(need, dev, stream)
    rc = lib.kda_chunk_prefill_ex(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens), _ptr(out),
                                  _ptr(final_state), ctypes.byref(opts), _ptr(workspace),
                                  workspace.numel(), _stream_handle(stream, dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_prefill_ex")
    return out, final_state, (checkpoints[:C] if checkpoint_interval else None), conv_state_out


def kda_decode_step_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       g: Optional[torch.Tensor], beta: torch.Tensor, state: torch.Tensor,
                       out: Optional[torch.Tensor] = None, *,
                       out_gate_z: Optional[torch.Tensor] = None,
                       conv_weight: Optional[torch.Tensor] = None, conv_silu: bool = False,
                       conv_state: Optional[torch.Tensor] = None,
                       gate_a: Optional[torch.Tensor] = None,
                       gate_b: Optional[torch.Tensor] = None,
                       gate_bias: Optional[torch.Tensor] = None,
                       scale: float = 1.0, qk_l2norm: bool = True, stream=None) -> torch.Tensor:
    """One decode step with options: the output gate (z ``[N,H,d_v]`` or
    ``[N,H]``) and/or the front end (``conv_state [N,3,W-1,H,d]`` advanced in
    place; ``gate_a [N,r]``)."""
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    dt = q.dtype
    gate = _gate(g, (N, H)) if g is not None else KDA_GATE_CHANNEL
    for name, t, shp in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)),
                         ("v", v, (N, H, dv)), ("beta", beta, (N, H))):
        _check_tensor(name, t, shp, dt, dev)
    if g is not None:
        _check_tensor("g", g, (N, H) if gate else (N, H, dk), dt, dev)
    _check_tensor("state", state, (N, H, dk, dv), torch.float32, dev)
    og = _out_gate(out_gate_z, (N, H), dv, dt, dev)
    fe = _front_end((N,), N, H, dk, dt, dev, conv_weight, conv_silu, conv_state, conv_state,
                    gate_a, gate_b, gate_bias)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _check_tensor("out", out, (N, H, dv), dt, dev)
    dims = make_dims(N, N, H, dk, dv, _io_dtype(q), scale, qk_l2norm, gate=gate)
    opts = kda_decode_options(og, 0, _ptr(out_gate_z),
                              ctypes.pointer(fe) if fe is not None else None)
    rc = lib.kda_decode_step_ex(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(state), _ptr(out), ctypes.byref(opts),
                                _stream_handle(stream, dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_decode_step_ex")
    return out
