"""ctypes front of the fp64 C oracle (``gdn_oracle.c``) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It never touches the HIP library.

Arrays cross as numpy arrays.  io tensors (qkv, a, b, conv_w, conv_state)
are either ``uint16`` bf16 bit patterns or ``float32``; everything the
oracle produces is ``float64`` except the conv tails, which are bit copies of
io tensors.  The arithmetic itself is documented in ``gdn_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("num_k_heads", ctypes.c_int64), ("num_v_heads", ctypes.c_int64),
                ("head_k_dim", ctypes.c_int64), ("head_v_dim", ctypes.c_int64),
                ("conv_kernel", ctypes.c_int64), ("start_pos", ctypes.c_int64),
                ("ckpt_interval", ctypes.c_int64), ("io_bf16", ctypes.c_int32),
                ("round_conv", ctypes.c_int32), ("q_scale", ctypes.c_double),
                ("l2_eps", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        D = ctypes.POINTER(_Dims)
        _lib.oracle_layer.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_int64, P, P, P]
        _lib.oracle_layer.restype = ctypes.c_int
        _lib.oracle_conv_tail.argtypes = [D, P, P, P, P]
        _lib.oracle_conv_tail.restype = ctypes.c_int
        _lib.oracle_frontend.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P]
        _lib.oracle_frontend.restype = ctypes.c_int
        _lib.oracle_core.argtypes = [D, P, P, P, P, P, P, P, P]
        _lib.oracle_core.restype = ctypes.c_int
        _lib.oracle_ckpt_count.argtypes = [D]
        _lib.oracle_ckpt_count.restype = ctypes.c_int64
        for name in ("rounding_to_bf16", "oracle_softplus", "oracle_sigmoid", "oracle_silu"):
            getattr(_lib, name).argtypes = [ctypes.c_double]
            getattr(_lib, name).restype = ctypes.c_double
        _lib.oracle_l2_normalize.argtypes = [P, ctypes.c_int64, ctypes.c_double, ctypes.c_double]
        _lib.oracle_l2_normalize.restype = None
        _lib.oracle_output_gate.argtypes = [ctypes.c_int64, ctypes.c_int64, P, P, P, ctypes.c_double, P]
        _lib.oracle_output_gate.restype = None
        _lib.oracle_gate_g.argtypes = [ctypes.c_double] * 3
        _lib.oracle_gate_g.restype = ctypes.c_double
        _lib.oracle_num_threads.restype = ctypes.c_int
        _lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


@dataclass
class Dims:
    batch: int
    seq_len: int
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int
    head_v_dim: int
    conv_kernel: int = 4
    start_pos: int = 0
    ckpt_interval: int = 0
    io_bf16: bool = True
    round_conv: bool = True
    q_scale: float = 1.0
    l2_eps: float = 1e-6

    @property
    def conv_dim(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    def c(self) -> _Dims:
        return _Dims(self.batch, self.seq_len, self.num_k_heads, self.num_v_heads,
                     self.head_k_dim, self.head_v_dim, self.conv_kernel, self.start_pos,
                     self.ckpt_interval, int(self.io_bf16), int(self.round_conv),
                     float(self.q_scale), float(self.l2_eps))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _io(x, dims: Dims, shape):
    """Check an io tensor: uint16 (bf16 bits) or float32, C-contiguous, of shape."""
    if x is None:
        return None
    want = np.uint16 if dims.io_bf16 else np.float32
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError(f"io tensor must be {want.__name__}, got {x.dtype}")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"shape {x.shape} != {shape}")
    return x


def _f32(x, shape):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"shape {x.shape} != {shape}")
    return x


def ckpt_count(dims: Dims) -> int:
    return int(lib().oracle_ckpt_count(ctypes.byref(dims.c())))


def layer(dims: Dims, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in=None, S0=None,
          heads=None, want_ckpt=False):
    """Front end + recurrence for the selected value heads.

    Returns dict(out [B, L, nsel, d_v], S [B, nsel, d_k, d_v], ckpt_S
    [n_ckpt, B, nsel, d_k, d_v] or None), all float64.
    """
    B, L, Hv = dims.batch, dims.seq_len, dims.num_v_heads
    dk, dv, K = dims.head_k_dim, dims.head_v_dim, dims.conv_kernel
    qkv = _io(qkv, dims, (B, L, dims.conv_dim))
    a = _io(a, dims, (B, L, Hv))
    b = _io(b, dims, (B, L, Hv))
    conv_w = _io(conv_w, dims, (dims.conv_dim, K))
    conv_state_in = _io(conv_state_in, dims, (B, dims.conv_dim, K - 1))
    A_log = _f32(A_log, (Hv,))
    dt_bias = _f32(dt_bias, (Hv,))
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, dtype=np.float64)
        if S0.shape != (B, Hv, dk, dv):
            raise ValueError(f"S0 shape {S0.shape}")
    if heads is None:
        hs, nsel = None, Hv
    else:
        hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
        nsel = int(hs.size)
    out = np.zeros((B, L, nsel, dv), np.float64)
    S = np.zeros((B, nsel, dk, dv), np.float64)
    ck = None
    if want_ckpt:
        ck = np.zeros((ckpt_count(dims), B, nsel, dk, dv), np.float64)
    rc = lib().oracle_layer(ctypes.byref(dims.c()), _ptr(qkv), _ptr(a), _ptr(b), _ptr(conv_w),
                            _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_in), _ptr(S0),
                            _ptr(hs), nsel, _ptr(out), _ptr(S), _ptr(ck))
    if rc != 0:
        raise ValueError("oracle_layer rejected its arguments")
    return {"out": out, "S": S, "ckpt_S": ck}


def conv_tail(dims: Dims, qkv, conv_state_in=None, want_ckpt=False):
    """Carried conv state after the call (and at each checkpoint): bit copies."""
    B, L, K = dims.batch, dims.seq_len, dims.conv_kernel
    qkv = _io(qkv, dims, (B, L, dims.conv_dim))
    conv_state_in = _io(conv_state_in, dims, (B, dims.conv_dim, K - 1))
    dt = np.uint16 if dims.io_bf16 else np.float32
    tail = np.zeros((B, dims.conv_dim, K - 1), dt)
    ck = np.zeros((ckpt_count(dims), B, dims.conv_dim, K - 1), dt) if want_ckpt else None
    lib().oracle_conv_tail(ctypes.byref(dims.c()), _ptr(qkv), _ptr(conv_state_in), _ptr(tail),
                           _ptr(ck))
    return tail, ck


def frontend(dims: Dims, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in=None):
    """Materialised front end: q_hat, k_hat [B,L,Hk,dk], v [B,L,Hv,dv], g, beta [B,L,Hv]."""
    B, L, Hk, Hv = dims.batch, dims.seq_len, dims.num_k_heads, dims.num_v_heads
    dk, dv, K = dims.head_k_dim, dims.head_v_dim, dims.conv_kernel
    qkv = _io(qkv, dims, (B, L, dims.conv_dim))
    a = _io(a, dims, (B, L, Hv))
    b = _io(b, dims, (B, L, Hv))
    conv_w = _io(conv_w, dims, (dims.conv_dim, K))
    conv_state_in = _io(conv_state_in, dims, (B, dims.conv_dim, K - 1))
    A_log = _f32(A_log, (Hv,))
    dt_bias = _f32(dt_bias, (Hv,))
    q = np.zeros((B, L, Hk, dk))
    k = np.zeros((B, L, Hk, dk))
    v = np.zeros((B, L, Hv, dv))
    g = np.zeros((B, L, Hv))
    beta = np.zeros((B, L, Hv))
    rc = lib().oracle_frontend(ctypes.byref(dims.c()), _ptr(qkv), _ptr(a), _ptr(b), _ptr(conv_w),
                               _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_in), _ptr(q), _ptr(k),
                               _ptr(v), _ptr(g), _ptr(beta))
    if rc != 0:
        raise ValueError("oracle_frontend rejected its arguments")
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta}


def core(q, k, v, g, beta, S0=None):
    """The recurrence alone on given features (fp64).

    q, k [B,L,Hk,dk]; v [B,L,Hv,dv]; g, beta [B,L,Hv]; S0 [B,Hv,dk,dv] or None.
    Returns (out [B,L,Hv,dv], S [B,Hv,dk,dv]).
    """
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    g = np.ascontiguousarray(g, np.float64)
    beta = np.ascontiguousarray(beta, np.float64)
    B, L, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, L) and g.shape == beta.shape == (B, L, Hv)
    dims = Dims(B, L, Hk, Hv, dk, dv)
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, np.float64)
        assert S0.shape == (B, Hv, dk, dv)
    out = np.zeros((B, L, Hv, dv))
    S = np.zeros((B, Hv, dk, dv))
    rc = lib().oracle_core(ctypes.byref(dims.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(S0), _ptr(out), _ptr(S))
    if rc != 0:
        raise ValueError("oracle_core rejected its arguments")
    return out, S


def round_bf16(x: float) -> float:
    return float(lib().rounding_to_bf16(float(x)))


def softplus(x: float) -> float:
    return float(lib().oracle_softplus(float(x)))


def sigmoid(x: float) -> float:
    return float(lib().oracle_sigmoid(float(x)))


def silu(x: float) -> float:
    return float(lib().oracle_silu(float(x)))


def gate_g(A_log: float, a: float, dt_bias: float) -> float:
    return float(lib().oracle_gate_g(float(A_log), float(a), float(dt_bias)))


def l2_normalize(x, eps: float = 1e-6, scale: float = 1.0):
    y = np.array(x, dtype=np.float64, copy=True).ravel()
    lib().oracle_l2_normalize(_ptr(y), y.size, float(eps), float(scale))
    return y


def output_gate(o, z, w, eps: float = 1e-6):
    """RMSNormGated over the last axis: y = w * o / sqrt(mean(o^2) + eps) *
    silu(z), fp64.  o, z [..., n] (any numbers; io tensors converted by the
    caller), w [n]."""
    o = np.ascontiguousarray(o, np.float64)
    z = np.ascontiguousarray(z, np.float64)
    w = np.ascontiguousarray(w, np.float64)
    n = o.shape[-1]
    assert z.shape == o.shape and w.shape == (n,)
    y = np.zeros_like(o)
    lib().oracle_output_gate(o.size // n if n else 0, n, _ptr(o), _ptr(z), _ptr(w), float(eps), _ptr(y))
    return y
