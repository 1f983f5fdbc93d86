"""Thin Python binding of libgdn.so (the C ABI in include/gdn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the stream.  If
the library is missing this module raises on import -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with "
                      "`python -m linear_attention_recurrence_causal_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EALIAS, GDN_ESPACE, GDN_EHIP = range(6)
GDN_F32, GDN_BF16 = 0, 1
GDN_PRECISION_DEFAULT, GDN_PRECISION_HILO = 0, 1


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.gdn_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


class _Config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_k_heads", ctypes.c_int32),
                ("num_v_heads", ctypes.c_int32), ("head_k_dim", ctypes.c_int32),
                ("head_v_dim", ctypes.c_int32), ("conv_kernel", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("q_scale", ctypes.c_float), ("l2_eps", ctypes.c_float), ("precision", ctypes.c_int32)]


class CkptEntry(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_int64), ("position", ctypes.c_int64),
                ("conv_offset", ctypes.c_uint64), ("rec_offset", ctypes.c_uint64)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_CFG = ctypes.POINTER(_Config)
_lib.gdn_status_string.argtypes = [ctypes.c_int32]
_lib.gdn_status_string.restype = ctypes.c_char_p
_lib.gdn_version.restype = ctypes.c_int32
GDN_VERSION = 200   # the header this binding's structures mirror
if _lib.gdn_version() != GDN_VERSION:
    raise ImportError(f"{_LIB_PATH} is version {_lib.gdn_version()}, this binding expects {GDN_VERSION}: rebuild")
_lib.gdn_state_checkpoint.argtypes = [_CFG, _I64, _I64, _I64, ctypes.POINTER(CkptEntry), _I64,
                                      ctypes.POINTER(_I64), ctypes.POINTER(_U64)]
_lib.gdn_state_checkpoint.restype = ctypes.c_int32
_lib.gdn_prefill_workspace_bytes.argtypes = [_CFG, _I64, ctypes.POINTER(_U64)]
_lib.gdn_prefill_workspace_bytes.restype = ctypes.c_int32
_lib.gdn_prefill_chunked.argtypes = [_CFG, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _U64, _I64, _P, _U64, _P]
_lib.gdn_prefill_chunked.restype = ctypes.c_int32
_lib.gdn_prefill_chunked_noalloc.argtypes = [_CFG, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _U64, _I64, _P]
_lib.gdn_prefill_chunked_noalloc.restype = ctypes.c_int32
NOALLOC_SCRATCH_BYTES = 64 << 20
_lib.gdn_decode_step.argtypes = [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.gdn_decode_multi.argtypes = [_CFG, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P]
_lib.gdn_decode_multi.restype = ctypes.c_int32
_lib.gdn_decode_step.restype = ctypes.c_int32
_lib.gdn_decode_gated.argtypes = [_CFG, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  ctypes.c_float, _P, _P, _P, _P]
_lib.gdn_decode_gated.restype = ctypes.c_int32
_lib.gdn_output_gate.argtypes = [_CFG, _I64, _P, _P, _P, ctypes.c_float, _P, _P]
_lib.gdn_output_gate.restype = ctypes.c_int32
_I64P = ctypes.POINTER(_I64)
_lib.gdn_prefill_varlen_workspace_bytes.argtypes = [_CFG, _I64P, _I64P, ctypes.POINTER(_U64)]
_lib.gdn_prefill_varlen_workspace_bytes.restype = ctypes.c_int32
_lib.gdn_prefill_varlen.argtypes = [_CFG, _I64P, _I64P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _U64, _I64, _P, _U64, _P]
_lib.gdn_prefill_varlen.restype = ctypes.c_int32
_lib.gdn_ckpt_lookup.argtypes = [_CFG, _I64, _I64, ctypes.c_int32, ctypes.POINTER(CkptEntry)]
_lib.gdn_ckpt_lookup.restype = ctypes.c_int32

lib = _lib


@dataclass(frozen=True)
class Config:
    """Mirror of ``gdn_config``."""
    batch: int
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int = 128
    head_v_dim: int = 128
    conv_kernel: int = 4
    chunk: int = 64
    io_dtype: int = GDN_BF16
    q_scale: float = 1.0
    l2_eps: float = 1e-6
    precision: int = GDN_PRECISION_DEFAULT

    @property
    def conv_dim(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    @property
    def torch_io(self) -> torch.dtype:
        return torch.bfloat16 if self.io_dtype == GDN_BF16 else torch.float32

    def c(self) -> _Config:
        return _Config(self.batch, self.num_k_heads, self.num_v_heads, self.head_k_dim,
                       self.head_v_dim, self.conv_kernel, self.chunk, self.io_dtype,
                       self.q_scale, self.l2_eps, self.precision)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype, device, stream):
    """A tensor the call allocates for its outputs or workspace.

    Ordering contract: the call's kernels run on ``stream`` (the current
    stream when None).  The tensor is allocated while that stream is current,
    so the caching allocator hands out a block whose earlier users were all on
    that stream, and the kernels that write it are ordered after them.  Reuse
    of the block by other streams afterwards follows torch's usual rule for a
    tensor that belongs to ``stream``."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _check(t, name, shape, dtype, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def state_checkpoint(cfg: Config, start_pos: int, seq_len: int, interval: int):
    """Checkpoint plan: (list of CkptEntry, buffer_bytes)."""
    count, nbytes = _I64(0), _U64(0)
    st = _lib.gdn_state_checkpoint(ctypes.byref(cfg.c()), start_pos, seq_len, interval, None, 0,
                                   ctypes.byref(count), ctypes.byref(nbytes))
    if st != GDN_OK:
        raise GdnError(st, "gdn_state_checkpoint")
    arr = (CkptEntry * max(count.value, 1))()
    st = _lib.gdn_state_checkpoint(ctypes.byref(cfg.c()), start_pos, seq_len, interval, arr,
                                   count.value, ctypes.byref(count), ctypes.byref(nbytes))
    if st != GDN_OK:
        raise GdnError(st, "gdn_state_checkpoint")
    return list(arr)[: count.value], nbytes.value


def prefill_workspace_bytes(cfg: Config, seq_len: int) -> int:
    n = _U64(0)
    st = _lib.gdn_prefill_workspace_bytes(ctypes.byref(cfg.c()), seq_len, ctypes.byref(n))
    if st != GDN_OK:
        raise GdnError(st, "gdn_prefill_workspace_bytes")
    return n.value


def _prefill_buffers(cfg: Config, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in, rec_state_in,
                     ckpt_buf, out, conv_state_out, rec_state_out, stream):
    """Shape checks of a prefill call and the outputs (allocated with torch
    when not given); returns (L, out, conv_state_out, rec_state_out,
    ckpt_bytes)."""
    B, Hv, dk, dv = cfg.batch, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim
    L = qkv.shape[1]
    io = cfg.torch_io
    _check(qkv, "qkv", (B, L, cfg.conv_dim), io)
    _check(a, "a", (B, L, Hv), io)
    _check(b, "b", (B, L, Hv), io)
    _check(conv_w, "conv_w", (cfg.conv_dim, cfg.conv_kernel), io)
    _check(A_log, "A_log", (Hv,), torch.float32)
    _check(dt_bias, "dt_bias", (Hv,), torch.float32)
    _check(conv_state_in, "conv_state_in", (B, cfg.conv_dim, cfg.conv_kernel - 1), io, True)
    _check(rec_state_in, "rec_state_in", (B, Hv, dk, dv), torch.float32, True)
    dev = qkv.device
    if out is None:
        out = _empty((B, L, Hv, dv), io, dev, stream)
    if conv_state_out is None:
        conv_state_out = _empty((B, cfg.conv_dim, cfg.conv_kernel - 1), io, dev, stream)
    if rec_state_out is None:
        rec_state_out = _empty((B, Hv, dk, dv), torch.float32, dev, stream)
    _check(out, "out", (B, L, Hv, dv), io)
    _check(conv_state_out, "conv_state_out", (B, cfg.conv_dim, cfg.conv_kernel - 1), io)
    _check(rec_state_out, "rec_state_out", (B, Hv, dk, dv), torch.float32)
    ck_bytes = 0
    if ckpt_buf is not None:
        if not ckpt_buf.is_cuda or not ckpt_buf.is_contiguous():
            raise ValueError("ckpt_buf must be a contiguous device tensor")
        ck_bytes = ckpt_buf.numel() * ckpt_buf.element_size()
    return L, out, conv_state_out, rec_state_out, ck_bytes


def prefill_chunked(cfg: Config, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in=None,
                    rec_state_in=None, *, start_pos: int = 0, ckpt_interval: int = 0,
                    ckpt_buf=None, out=None, conv_state_out=None, rec_state_out=None,
                    workspace="auto", stream=None):
    """Chunked prefill; returns (out, conv_state_out, rec_state_out).

    Outputs not passed in are allocated with torch.  ``ckpt_buf`` is a uint8
    device tensor of at least ``state_checkpoint(...)[1]`` bytes.
    ``workspace``: "auto" allocates ``prefill_workspace_bytes`` (two-pass
    path, whole call in one segment); a contiguous uint8 device tensor is used
    as given (any size; below one chunk's worth the fused path runs); None
    runs the fused single-pass kernel.
    """
    L, out, conv_state_out, rec_state_out, ck_bytes = _prefill_buffers(
        cfg, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in, rec_state_in, ckpt_buf, out,
        conv_state_out, rec_state_out, stream)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
        ws = prefill_workspace_bytes(cfg, L)
        wsbuf = _empty(ws, torch.uint8, qkv.device, stream) if ws else None
    elif workspace is None:
        ws, wsbuf = 0, None
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws, wsbuf = workspace.numel() * workspace.element_size(), workspace
    st = _lib.gdn_prefill_chunked(
        ctypes.byref(cfg.c()), L, start_pos, _ptr(qkv), _ptr(a), _ptr(b), _ptr(conv_w),
        _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_in), _ptr(conv_state_out),
        _ptr(rec_state_in), _ptr(rec_state_out), _ptr(out), _ptr(ckpt_buf), ck_bytes,
        ckpt_interval, _ptr(wsbuf), ws, _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_prefill_chunked")
    return out, conv_state_out, rec_state_out


def prefill_chunked_noalloc(cfg: Config, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in=None,
                            rec_state_in=None, *, start_pos: int = 0, ckpt_interval: int = 0,
                            ckpt_buf=None, out=None, conv_state_out=None, rec_state_out=None,
                            stream=None):
    """gdn_prefill_chunked_noalloc: the two-pass prefill on the library's
    static scratch array (no workspace, nothing allocated by the call; the
    outputs are allocated here only when not passed in).  Returns (out,
    conv_state_out, rec_state_out)."""
    L, out, conv_state_out, rec_state_out, ck_bytes = _prefill_buffers(
        cfg, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in, rec_state_in, ckpt_buf, out,
        conv_state_out, rec_state_out, stream)
    st = _lib.gdn_prefill_chunked_noalloc(
        ctypes.byref(cfg.c()), L, start_pos, _ptr(qkv), _ptr(a), _ptr(b), _ptr(conv_w),
        _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_in), _ptr(conv_state_out),
        _ptr(rec_state_in), _ptr(rec_state_out), _ptr(out), _ptr(ckpt_buf), ck_bytes,
        ckpt_interval, _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_prefill_chunked_noalloc")
    return out, conv_state_out, rec_state_out


def decode_step(cfg: Config, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in=None,
                rec_state_in=None, *, out=None, conv_state_out=None, rec_state_out=None,
                stream=None):
    """One recurrent step; returns (out, conv_state_out, rec_state_out).

    ``rec_state_out`` may be ``rec_state_in`` (in-place update)."""
    B, Hv, dk, dv = cfg.batch, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim
    io = cfg.torch_io
    _check(qkv, "qkv", (B, cfg.conv_dim), io)
    _check(a, "a", (B, Hv), io)
    _check(b, "b", (B, Hv), io)
    _check(conv_w, "conv_w", (cfg.conv_dim, cfg.conv_kernel), io)
    _check(A_log, "A_log", (Hv,), torch.float32)
    _check(dt_bias, "dt_bias", (Hv,), torch.float32)
    _check(conv_state_in, "conv_state_in", (B, cfg.conv_dim, cfg.conv_kernel - 1), io, True)
    _check(rec_state_in, "rec_state_in", (B, Hv, dk, dv), torch.float32, True)
    dev = qkv.device
    if out is None:
        out = _empty((B, Hv, dv), io, dev, stream)
    if conv_state_out is None:
        conv_state_out = _empty((B, cfg.conv_dim, cfg.conv_kernel - 1), io, dev, stream)
    if rec_state_out is None:
        rec_state_out = _empty((B, Hv, dk, dv), torch.float32, dev, stream)
    _check(out, "out", (B, Hv, dv), io)
    _check(conv_state_out, "conv_state_out", (B, cfg.conv_dim, cfg.conv_kernel - 1), io)
    _check(rec_state_out, "rec_state_out", (B, Hv, dk, dv), torch.float32)
    st = _lib.gdn_decode_step(ctypes.byref(cfg.c()), _ptr(qkv), _ptr(a), _ptr(b), _ptr(conv_w),
                              _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_in),
                              _ptr(conv_state_out), _ptr(rec_state_in), _ptr(rec_state_out),
                              _ptr(out), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_step")
    return out, conv_state_out, rec_state_out


MAX_DECODE_TOKENS = 8


def decode_multi(cfg: Config, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in=None,
                 rec_state_in=None, *, out=None, conv_state_out=None, rec_state_out=None,
                 rec_snapshots=None, conv_snapshots=None, snapshots=False, stream=None):
    """T consecutive tokens per sequence in one call (qkv [B, T, conv_dim]);
    returns (out [B, T, H_v, d_v], conv_state_out, rec_state_out,
    rec_snapshots, conv_snapshots).  ``snapshots=True`` allocates the
    per-token state snapshots ([T, B, H_v, d_k, d_v] and [T, B, conv_dim,
    K-1]); otherwise they are None unless passed in."""
    B, Hv, dk, dv = cfg.batch, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim
    io = cfg.torch_io
    if qkv.dim() != 3:
        raise ValueError(f"qkv must be [B, T, conv_dim], got {tuple(qkv.shape)}")
    T = qkv.shape[1]
    _check(qkv, "qkv", (B, T, cfg.conv_dim), io)
    _check(a, "a", (B, T, Hv), io)
    _check(b, "b", (B, T, Hv), io)
    _check(conv_w, "conv_w", (cfg.conv_dim, cfg.conv_kernel), io)
    _check(A_log, "A_log", (Hv,), torch.float32)
    _check(dt_bias, "dt_bias", (Hv,), torch.float32)
    _check(conv_state_in, "conv_state_in", (B, cfg.conv_dim, cfg.conv_kernel - 1), io, True)
    _check(rec_state_in, "rec_state_in", (B, Hv, dk, dv), torch.float32, True)
    dev = qkv.device
    if out is None:
        out = _empty((B, T, Hv, dv), io, dev, stream)
    if conv_state_out is None:
        conv_state_out = _empty((B, cfg.conv_dim, cfg.conv_kernel - 1), io, dev, stream)
    if rec_state_out is None:
        rec_state_out = _empty((B, Hv, dk, dv), torch.float32, dev, stream)
    if snapshots and rec_snapshots is None:
        rec_snapshots = _empty((T, B, Hv, dk, dv), torch.float32, dev, stream)
    if snapshots and conv_snapshots is None:
        conv_snapshots = _empty((T, B, cfg.conv_dim, cfg.conv_kernel - 1), io, dev, stream)
    _check(out, "out", (B, T, Hv, dv), io)
    _check(conv_state_out, "conv_state_out", (B, cfg.conv_dim, cfg.conv_kernel - 1), io)
    _check(rec_state_out, "rec_state_out", (B, Hv, dk, dv), torch.float32)
    _check(rec_snapshots, "rec_snapshots", (T, B, Hv, dk, dv), torch.float32, True)
    _check(conv_snapshots, "conv_snapshots", (T, B, cfg.conv_dim, cfg.conv_kernel - 1), io, True)
    st = _lib.gdn_decode_multi(ctypes.byref(cfg.c()), T, _ptr(qkv), _ptr(a), _ptr(b), _ptr(conv_w),
                               _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_in), _ptr(conv_state_out),
                               _ptr(rec_state_in), _ptr(rec_state_out), _ptr(out), _ptr(rec_snapshots),
                               _ptr(conv_snapshots), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_multi")
    return out, conv_state_out, rec_state_out, rec_snapshots, conv_snapshots


GATE_EPS = 1e-6


def output_gate(cfg: Config, o, z, norm_w, eps: float = GATE_EPS, *, y=None, stream=None):
    """RMSNormGated of the core output: y = norm_w * o / sqrt(mean(o^2) + eps)
    * silu(z) per token and value head over d_v.  o, z: [..., H_v, d_v] (any
    leading token axes, contiguous); y may be o or z (in place).  Returns y."""
    Hv, dv = cfg.num_v_heads, cfg.head_v_dim
    io = cfg.torch_io
    if o is None or o.dim() < 2 or tuple(o.shape[-2:]) != (Hv, dv):
        raise ValueError(f"o must be [..., {Hv}, {dv}]")
    shape = tuple(o.shape)
    rows = o.numel() // (Hv * dv)
    _check(o, "o", shape, io)
    _check(z, "z", shape, io)
    _check(norm_w, "norm_w", (dv,), io)
    if y is None:
        y = _empty(shape, io, o.device, stream)
    _check(y, "y", shape, io)
    st = _lib.gdn_output_gate(ctypes.byref(cfg.c()), rows, _ptr(o), _ptr(z), _ptr(norm_w), eps, _ptr(y),
                              _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_output_gate")
    return y


def decode_gated(cfg: Config, qkv, a, b, conv_w, A_log, dt_bias, z, norm_w, conv_state_in=None,
                 rec_state_in=None, *, eps: float = GATE_EPS, y=None, out=None, want_out=False,
                 conv_state_out=None, rec_state_out=None, rec_snapshots=None, conv_snapshots=None,
                 snapshots=False, stream=None):
    """decode_multi with the output gate fused in (qkv [B, T, conv_dim], z
    [B, T, H_v, d_v]); returns (y, out, conv_state_out, rec_state_out,
    rec_snapshots, conv_snapshots).  The ungated out is written only if
    passed in or ``want_out``; otherwise it is None."""
    B, Hv, dk, dv = cfg.batch, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim
    io = cfg.torch_io
    if qkv.dim() != 3:
        raise ValueError(f"qkv must be [B, T, conv_dim], got {tuple(qkv.shape)}")
    T = qkv.shape[1]
    _check(qkv, "qkv", (B, T, cfg.conv_dim), io)
    _check(a, "a", (B, T, Hv), io)
    _check(b, "b", (B, T, Hv), io)
    _check(conv_w, "conv_w", (cfg.conv_dim, cfg.conv_kernel), io)
    _check(A_log, "A_log", (Hv,), torch.float32)
    _check(dt_bias, "dt_bias", (Hv,), torch.float32)
    _check(z, "z", (B, T, Hv, dv), io)
    _check(norm_w, "norm_w", (dv,), io)
    _check(conv_state_in, "conv_state_in", (B, cfg.conv_dim, cfg.conv_kernel - 1), io, True)
    _check(rec_state_in, "rec_state_in", (B, Hv, dk, dv), torch.float32, True)
    dev = qkv.device
    if y is None:
        y = _empty((B, T, Hv, dv), io, dev, stream)
    if out is None and want_out:
        out = _empty((B, T, Hv, dv), io, dev, stream)
    if conv_state_out is None:
        conv_state_out = _empty((B, cfg.conv_dim, cfg.conv_kernel - 1), io, dev, stream)
    if rec_state_out is None:
        rec_state_out = _empty((B, Hv, dk, dv), torch.float32, dev, stream)
    if snapshots and rec_snapshots is None:
        rec_snapshots = _empty((T, B, Hv, dk, dv), torch.float32, dev, stream)
    if snapshots and conv_snapshots is None:
        conv_snapshots = _empty((T, B, cfg.conv_dim, cfg.conv_kernel - 1), io, dev, stream)
    _check(y, "y", (B, T, Hv, dv), io)
    _check(out, "out", (B, T, Hv, dv), io, True)
    _check(conv_state_out, "conv_state_out", (B, cfg.conv_dim, cfg.conv_kernel - 1), io)
    _check(rec_state_out, "rec_state_out", (B, Hv, dk, dv), torch.float32)
    _check(rec_snapshots, "rec_snapshots", (T, B, Hv, dk, dv), torch.float32, True)
    _check(conv_snapshots, "conv_snapshots", (T, B, cfg.conv_dim, cfg.conv_kernel - 1), io, True)
    st = _lib.gdn_decode_gated(ctypes.byref(cfg.c()), T, _ptr(qkv), _ptr(a), _ptr(b), _ptr(conv_w),
                               _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_in), _ptr(conv_state_out),
                               _ptr(rec_state_in), _ptr(rec_state_out), _ptr(out), _ptr(z), _ptr(norm_w),
                               eps, _ptr(y), _ptr(rec_snapshots), _ptr(conv_snapshots), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode_gated")
    return y, out, conv_state_out, rec_state_out, rec_snapshots, conv_snapshots


def _i64_array(xs):
    xs = [int(x) for x in xs]
    return (_I64 * max(1, len(xs)))(*xs)


def prefill_varlen_workspace_bytes(cfg: Config, cu_seqlens, start_pos) -> int:
    n = _U64(0)
    st = _lib.gdn_prefill_varlen_workspace_bytes(ctypes.byref(cfg.c()), _i64_array(cu_seqlens),
                                                 _i64_array(start_pos), ctypes.byref(n))
    if st != GDN_OK:
        raise GdnError(st, "gdn_prefill_varlen_workspace_bytes")
    return n.value


def prefill_varlen(cfg: Config, cu_seqlens, start_pos, qkv, a, b, conv_w, A_log, dt_bias,
                   conv_state_in=None, rec_state_in=None, *, ckpt_interval: int = 0, ckpt_buf=None,
                   out=None, conv_state_out=None, rec_state_out=None, workspace="auto", stream=None):
    """cfg.batch sequences packed along the token axis: cu_seqlens [B + 1] and
    start_pos [B] are host sequences of ints; qkv [T, conv_dim], a, b [T, H_v];
    returns (out [T, H_v, d_v], conv_state_out, rec_state_out).
    ``workspace``: "auto" allocates prefill_varlen_workspace_bytes, else a
    contiguous uint8 device tensor (at least one chunk per sequence of a
    group of 64)."""
    B, Hv, dk, dv = cfg.batch, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim
    cu = [int(x) for x in cu_seqlens]
    sp = [int(x) for x in start_pos]
    if len(cu) != B + 1 or len(sp) != B:
        raise ValueError(f"cu_seqlens needs {B + 1} entries and start_pos {B}")
    T = cu[-1]
    io = cfg.torch_io
    _check(qkv, "qkv", (T, cfg.conv_dim), io)
    _check(a, "a", (T, Hv), io)
    _check(b, "b", (T, Hv), io)
    _check(conv_w, "conv_w", (cfg.conv_dim, cfg.conv_kernel), io)
    _check(A_log, "A_log", (Hv,), torch.float32)
    _check(dt_bias, "dt_bias", (Hv,), torch.float32)
    _check(conv_state_in, "conv_state_in", (B, cfg.conv_dim, cfg.conv_kernel - 1), io, True)
    _check(rec_state_in, "rec_state_in", (B, Hv, dk, dv), torch.float32, True)
    dev = qkv.device
    if out is None:
        out = _empty((T, Hv, dv), io, dev, stream)
    if conv_state_out is None:
        conv_state_out = _empty((B, cfg.conv_dim, cfg.conv_kernel - 1), io, dev, stream)
    if rec_state_out is None:
        rec_state_out = _empty((B, Hv, dk, dv), torch.float32, dev, stream)
    _check(out, "out", (T, Hv, dv), io)
    _check(conv_state_out, "conv_state_out", (B, cfg.conv_dim, cfg.conv_kernel - 1), io)
    _check(rec_state_out, "rec_state_out", (B, Hv, dk, dv), torch.float32)
    ck_bytes = 0
    if ckpt_buf is not None:
        if not ckpt_buf.is_cuda or not ckpt_buf.is_contiguous():
            raise ValueError("ckpt_buf must be a contiguous device tensor")
        ck_bytes = ckpt_buf.numel() * ckpt_buf.element_size()
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto' or a uint8 device tensor")
        ws = max(prefill_varlen_workspace_bytes(cfg, cu, sp), 256)
        wsbuf = _empty(ws, torch.uint8, dev, stream)
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws, wsbuf = workspace.numel() * workspace.element_size(), workspace
    st = _lib.gdn_prefill_varlen(
        ctypes.byref(cfg.c()), _i64_array(cu), _i64_array(sp), _ptr(qkv), _ptr(a), _ptr(b), _ptr(conv_w),
        _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_in), _ptr(conv_state_out), _ptr(rec_state_in),
        _ptr(rec_state_out), _ptr(out), _ptr(ckpt_buf), ck_bytes, ckpt_interval, _ptr(wsbuf), ws,
        _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_prefill_varlen")
    return out, conv_state_out, rec_state_out


def ckpt_lookup(cfg: Config, interval: int, cached_tokens: int, seq_index: int = 0) -> CkptEntry:
    """The checkpoint to resume a request from after a prefix hit of
    ``cached_tokens`` tokens (slot -1: none, start a new request)."""
    e = CkptEntry()
    st = _lib.gdn_ckpt_lookup(ctypes.byref(cfg.c()), interval, cached_tokens, seq_index, ctypes.byref(e))
    if st != GDN_OK:
        raise GdnError(st, "gdn_ckpt_lookup")
    return e
