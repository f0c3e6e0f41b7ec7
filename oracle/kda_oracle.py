"""KDA oracle: plain fp64 CPU reference for the Kimi Delta Attention recurrence.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  The product path
(the HIP library behind ``include/kda.h`` and its Python binding) never imports
it, shares no code with it and has no CPU fallback.

Two independent formulations live here, both in fp64:

* ``prefill`` / ``decode_step`` / ``chunked`` call ``kda_oracle.c`` (plain C,
  token-by-token recurrence; the chunk form is a second formulation used only
  to pin the chunk algebra).
* ``naive_expansion`` is numpy: the closed-form unrolling of the recurrence,
  S_t = Phi(t,0) S_0 + sum_{s<=t} Phi(t,s) beta_s k_s v_s^T with
  Phi(t,s) = A_t ... A_{s+1} and A_s = (I - beta_s k_s k_s^T) Diag(exp g_s),
  built from explicit d_k x d_k matrix products (O(T^2) products; tiny inputs
  only).

The recurrence is the delta rule with a diagonal (per-channel) gate described
on "From KV Cache to Depth Attention: The Bottlenecks Kimi K3 Had to Break",
Technical Details, Kimi Delta Attention bullet, and "Kimi K3: The Manos, The
Mythos, The Legendos", bullets on KDA as online learning and on the stability
details (L2-normalised queries and keys).

``short_conv`` and ``low_rank_gate`` (numpy) are the front end that may
produce q, k, v and g from raw projections: a short causal convolution per
channel and g = -softplus(a b^T + bias).

``apply_output_gate`` (numpy) is the output forget gate that may follow the
read-out: out * sigmoid(z), z per value channel or per head.

Inputs are float32 numpy arrays holding the exact upcast of what the GPU path
reads (bf16 -> fp32 is exact), token-major: q, k, g ``[T, H, d_k]``,
v ``[T, H, d_v]``, beta ``[T, H]``; states ``[N, H, d_k, d_v]``.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

#: default epsilon inside the L2-norm square root: x / sqrt(sum x^2 + EPS)
EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile ``kda_oracle.c`` into ``oracle/libkda_oracle.so`` with gcc.

    No fast-math and no FP contraction, so every operation rounds as written.
    """
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-o", tmp, _SRC, "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    D = ctypes.c_double
    I = ctypes.c_int
    lib.kda_oracle_prefill.argtypes = [I64, P, I64, I64, I64, P, P, P, P, P, P,
                                       D, D, I, P, P, I]
    lib.kda_oracle_prefill.restype = I
    lib.kda_oracle_chunked.argtypes = [I64, P, I64, I64, I64, P, P, P, P, P, P,
                                       D, D, I, I64, P, P, I]
    lib.kda_oracle_chunked.restype = I
    lib.kda_oracle_decode_step.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P,
                                           D, D, I, P, I]
    lib.kda_oracle_decode_step.restype = I
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily route this module's calls to another build of the oracle
    source (the test suite uses it to check that planted mistakes are caught)."""
    global _lib
    saved = _lib
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


def default_threads() -> int:
    """Host threads the oracle uses by default: every core this process may use."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f32(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float32)
    return a


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cu(cu_seqlens, T: int, n_seqs: Optional[int]) -> np.ndarray:
    if cu_seqlens is None:
        n = 1 if n_seqs is None else int(n_seqs)
        if n == 0:
            return np.zeros(1, dtype=np.int64)
        assert T % n == 0, "without cu_seqlens, T must split evenly into n_seqs"
        return np.arange(n + 1, dtype=np.int64) * (T // n)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    assert cu.ndim == 1 and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    return cu


def _run(fn_name: str, q, k, v, g, beta, cu_seqlens, initial_state, n_seqs,
         scale, eps, l2norm, threads, chunk=None) -> Tuple[np.ndarray, np.ndarray]:
    lib = _load()
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and beta.shape == (T, H)
    cu = _cu(cu_seqlens, T, n_seqs)
    N = cu.shape[0] - 1
    s0 = None
    if initial_state is not None:
        s0 = _f32(initial_state)
        assert s0.shape == (N, H, dk, dv)
    out = np.zeros((T, H, dv), dtype=np.float64)
    fin = np.zeros((N, H, dk, dv), dtype=np.float64)
    threads = default_threads() if threads is None else int(threads)
    args = [N, _ptr(cu), H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(s0), float(scale), float(eps), int(bool(l2norm))]
    if chunk is not None:
        args.append(int(chunk))
    args += [_ptr(out), _ptr(fin), threads]
    rc = getattr(lib, fn_name)(*args)
    if rc != 0:
        raise RuntimeError(f"{fn_name} failed with code {rc}")
    return out, fin


def prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, n_seqs=None,
            scale: float = 1.0, eps: float = EPS, l2norm: bool = True,
            threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token fp64 recurrence over packed sequences.

    Returns ``(out [T,H,d_v], final_state [N,H,d_k,d_v])`` as float64.
    ``cu_seqlens`` (int, ``[N+1]``) delimits the sequences; without it the T
    tokens form ``n_seqs`` (default 1) equal-length sequences.
    """
    return _run("kda_oracle_prefill", q, k, v, g, beta, cu_seqlens, initial_state,
                n_seqs, scale, eps, l2norm, threads)


def chunked(q, k, v, g, beta, chunk: int, cu_seqlens=None, initial_state=None,
            n_seqs=None, scale: float = 1.0, eps: float = EPS, l2norm: bool = True,
            threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The same function through the fp64 chunk-wise WY form (chunk >= 1)."""
    return _run("kda_oracle_chunked", q, k, v, g, beta, cu_seqlens, initial_state,
                n_seqs, scale, eps, l2norm, threads, chunk=chunk)


def decode_step(q, k, v, g, beta, state: np.ndarray, scale: float = 1.0,
                eps: float = EPS, l2norm: bool = True,
                threads: Optional[int] = None) -> np.ndarray:
    """One token per sequence.  ``state`` (float64 ``[N,H,d_k,d_v]``, C-contiguous)
    is updated in place; returns ``out [N,H,d_v]`` as float64."""
    lib = _load()
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    N, H, dk = q.shape
    dv = v.shape[2]
    assert state.dtype == np.float64 and state.flags.c_contiguous
    assert state.shape == (N, H, dk, dv)
    out = np.zeros((N, H, dv), dtype=np.float64)
    threads = default_threads() if threads is None else int(threads)
    rc = lib.kda_oracle_decode_step(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(state), float(scale), float(eps),
                                    1 if l2norm else 0, _ptr(out), threads)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_decode_step failed with code {rc}")
    return out


def apply_output_gate(out, z) -> np.ndarray:
    """Output forget gate on the attention read-out, in fp64.

    "Kimi K3: The Manos, The Mythos, The Legendos", stability-details bullet,
    lists a per-head output forget gate.  Read here as the usual sigmoid gate:
    out' = out * sigmoid(z) with z a caller-supplied pre-activation, either one
    value per value channel (z shaped like ``out``, ``[..., d_v]``) or one value
    per head (z ``[...]``, broadcast over the d_v channels).
    """
    o = np.asarray(out, dtype=np.float64)
    zz = np.asarray(z, dtype=np.float64)
    if zz.shape == o.shape[:-1]:
        zz = zz[..., None]
    assert zz.shape[:-1] == o.shape[:-1] and zz.shape[-1] in (1, o.shape[-1])
    return o * (1.0 / (1.0 + np.exp(-zz)))


def _seq_bounds(cu_seqlens, T: int, n_seqs: Optional[int]) -> np.ndarray:
    return _cu(cu_seqlens, T, n_seqs)


def short_conv(x, weight, cu_seqlens=None, n_seqs=None, state=None, silu: bool = False):
    """Short causal depthwise convolution over each sequence's tokens, in fp64.

    "Kimi K3: The Manos, The Mythos, The Legendos", stability-details bullet,
    names short convolutions on q, k and v for local dependencies; the reading
    taken here is the plain one: per channel, an FIR filter of width W over the
    current token and the W-1 before it, within the sequence,
        y_t[c] = sum_{j=0}^{W-1} weight[c][j] * x_{t-(W-1)+j}[c],
    optionally followed by SiLU (y * sigmoid(y)).  Tokens before a sequence's
    start are the rows of its conv state (state[n][j] is token start-(W-1)+j),
    or zero without one.

    x ``[T, H, d]``; weight ``[H, d, W]``; state ``[N, W-1, H, d]`` or None.
    Returns ``(y [T, H, d], final_state [N, W-1, H, d])``, the final state
    holding each sequence's last W-1 input rows (continuing from its state
    when the sequence is shorter than W-1).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    T, H, d = x.shape
    W = w.shape[2]
    assert w.shape == (H, d, W) and W >= 1
    cu = _seq_bounds(cu_seqlens, T, n_seqs)
    N = cu.shape[0] - 1
    st = np.zeros((N, W - 1, H, d)) if state is None else np.asarray(state, dtype=np.float64)
    assert st.shape == (N, W - 1, H, d)
    y = np.zeros((T, H, d))
    fin = np.zeros((N, W - 1, H, d))
    for n in range(N):
        b, e = int(cu[n]), int(cu[n + 1])
        ext = np.concatenate([st[n], x[b:e]], axis=0)  # ext[i] is token b-(W-1)+i
        for t in range(e - b):
            acc = np.zeros((H, d))
            for j in range(W):
                acc += w[:, :, j] * ext[t + j]
            y[b + t] = acc
        fin[n] = ext[ext.shape[0] - (W - 1):]
    if silu:
        y = y / (1.0 + np.exp(-y))
    return y, fin


def low_rank_gate(a, b, bias=None):
    """Decay gate from a low-rank projection, in fp64.

    "Kimi K3: The Manos, The Mythos, The Legendos", stability-details bullet,
    names low-rank decay gates.  Read as: the layer's hidden state is projected
    to rank r (``a [T, r]``, a projection outside this path), then up to every
    head's key channels by ``b [H, d_k, r]`` (plus an optional per-channel
    ``bias [H, d_k]``), and the log-retention is g = -softplus(a b^T + bias),
    which is <= 0 as the recurrence needs.  Returns g ``[T, H, d_k]``.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    z = np.einsum("tj,hcj->thc", a, b)
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)[None]
    return -np.logaddexp(0.0, z)


def naive_expansion(q, k, v, g, beta, initial_state=None, scale: float = 1.0,
                    eps: float = EPS, l2norm: bool = True):
    """Closed-form unrolling of one sequence (numpy fp64, tiny inputs only).

    q, k, g ``[T, d_k]``; v ``[T, d_v]``; beta ``[T]``; initial_state ``[d_k, d_v]``.
    Builds every transition A_s = (I - beta_s k_s k_s^T) Diag(exp g_s) as an
    explicit matrix and every product Phi(t, s) = A_t ... A_{s+1}, then
    S_t = Phi(t, 0) S_0 + sum_{s=1..t} Phi(t, s) beta_s k_s v_s^T, o_t = S_t^T q_t.
    Returns ``(out [T, d_v], states [T, d_k, d_v])``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, dk = q.shape
    dv = v.shape[1]
    if l2norm:
        q = q / np.sqrt((q * q).sum(axis=1, keepdims=True) + eps)
        k = k / np.sqrt((k * k).sum(axis=1, keepdims=True) + eps)
    q = q * scale
    S0 = np.zeros((dk, dv)) if initial_state is None else \
        np.asarray(initial_state, dtype=np.float64)
    eye = np.eye(dk)
    trans = [(eye - beta[s] * np.outer(k[s], k[s])) @ np.diag(np.exp(g[s]))
             for s in range(T)]

    def phi(t, s):
        """Phi(t, s) = A_t A_{t-1} ... A_{s+1} (0-based token indices t, s; s < t
        means tokens s+1..t).  Phi(t, t) = I."""
        m = eye.copy()
        for r in range(s + 1, t + 1):
            m = trans[r] @ m
        return m

    outs = np.zeros((T, dv))
    states = np.zeros((T, dk, dv))
    for t in range(T):
        St = phi(t, -1) @ S0
        for s in range(t + 1):
            St = St + phi(t, s) @ (beta[s] * np.outer(k[s], v[s]))
        states[t] = St
        outs[t] = St.T @ q[t]
    return outs, states
