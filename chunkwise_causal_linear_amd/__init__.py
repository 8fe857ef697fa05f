"""Chunkwise causal linear attention for MI355X (gfx950): thin Python binding.

Every step of the computation runs in the HIP library ``lib/libfla_linattn.so``
(C ABI: include/fla_linattn.h).  This module only marshals torch tensors into
pointers, sizes and flags, and raises when the library is missing or a call fails.
There is no CPU fallback.

torch is imported before the library is loaded so that the HIP runtime torch ships
(soname libamdhip64.so.7) is the one the library binds to: one runtime per process,
shared streams and device pointers.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libfla_linattn.so")

FLA_OK, FLA_ERR_INVALID_ARG, FLA_ERR_UNSUPPORTED, FLA_ERR_DEVICE, FLA_ERR_SCRATCH = 0, -1, -2, -3, -4
FLA_BF16 = 1 << 0
FLA_DECAY_GAMMA = 1 << 1
FLA_DECAY_GATE = 1 << 2
FLA_PHI_ELU1 = 1 << 3
FLA_NORMALIZE = 1 << 4
FLA_DECAY_TOKEN = 1 << 5
FLA_LAYOUT_BTHD = 1 << 6

EXPORTED = ("fla_linattn_fwd", "fla_linattn_fwd_segments", "fla_linattn_step",
            "fla_status_string", "fla_linattn_segments_for", "fla_linattn_bwd",
            "fla_linattn_fwd_varlen", "fla_linattn_bwd_varlen", "fla_gdn_fwd",
            "fla_probe_stream", "fla_probe_mfma", "fla_probe_mfma_flops",
            "fla_linattn_fwd_noalloc", "fla_linattn_fwd_proj", "fla_probe_chunk_pattern")
PROBE_READ, PROBE_COPY, PROBE_MIX5 = 0, 1, 2

_lib = None


class FlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def load_library():
    """Load the HIP library (raises ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                          "(python -m chunkwise_causal_linear_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, u32, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int
    lib.fla_linattn_fwd.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, u32, p]
    lib.fla_linattn_fwd.restype = c_int
    lib.fla_linattn_fwd_segments.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64,
                                             u32, i64, p]
    lib.fla_linattn_fwd_segments.restype = c_int
    lib.fla_linattn_step.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, u32, p]
    lib.fla_linattn_step.restype = c_int
    lib.fla_status_string.argtypes = [c_int]
    lib.fla_status_string.restype = ctypes.c_char_p
    lib.fla_linattn_segments_for.argtypes = [i64, i64, i64, i64, i64, i64, u32,
                                             ctypes.POINTER(i64)]
    lib.fla_linattn_segments_for.restype = c_int
    lib.fla_linattn_bwd.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64,
                                    i64, u32, p]
    lib.fla_linattn_bwd.restype = c_int
    lib.fla_linattn_fwd_varlen.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64,
                                           u32, p]
    lib.fla_linattn_fwd_varlen.restype = c_int
    lib.fla_linattn_bwd_varlen.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p, p, i64, i64, i64,
                                           i64, i64, i64, u32, p]
    lib.fla_linattn_bwd_varlen.restype = c_int
    lib.fla_gdn_fwd.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, u32, p]
    lib.fla_gdn_fwd.restype = c_int
    lib.fla_linattn_fwd_noalloc.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64,
                                            u32, p]
    lib.fla_linattn_fwd_noalloc.restype = c_int
    lib.fla_linattn_fwd_proj.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64,
                                         i64, u32, p]
    lib.fla_linattn_fwd_proj.restype = c_int
    lib.fla_probe_stream.argtypes = [p, p, i64, c_int, p]
    lib.fla_probe_stream.restype = c_int
    lib.fla_probe_mfma.argtypes = [p, i64, i64, p]
    lib.fla_probe_mfma.restype = c_int
    lib.fla_probe_mfma_flops.argtypes = [i64, i64]
    lib.fla_probe_mfma_flops.restype = ctypes.c_double
    lib.fla_probe_chunk_pattern.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, p]
    lib.fla_probe_chunk_pattern.restype = c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fla_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensors(q: torch.Tensor, same_dtype=(), fp32=(), extra=()) -> None:
    """Host-side checks shared by every call: every tensor is contiguous (a strided view
    such as q[:, :, t] would be read as if it were dense); q is bf16 or fp32; tensors in
    same_dtype have q's dtype; fp32 tensors (decays, states) are float32; all live on q's
    device, a GPU.  None entries are skipped."""
    tensors = [t for t in (q, *same_dtype, *fp32, *extra) if t is not None]
    for t in tensors:
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (got a strided view)")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"q must be bfloat16 or float32, got {q.dtype}")
    for t in same_dtype:
        if t is not None and t.dtype != q.dtype:
            raise ValueError(f"k, v, out and upstream gradients must have q's dtype {q.dtype}, "
                             f"got {t.dtype}")
    for t in fp32:
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"decays and states must be float32, got {t.dtype}")
    if not q.is_cuda:
        raise ValueError("tensors must be on the GPU")
    for t in tensors:
        if t.device != q.device:
            raise ValueError(f"all tensors must be on {q.device}, got one on {t.device}")


def flags_for(dtype: torch.dtype, decay_kind: str, phi_elu1: bool, normalize: bool) -> int:
    f = FLA_BF16 if dtype == torch.bfloat16 else 0
    f |= {"none": 0, "gamma": FLA_DECAY_GAMMA, "gate": FLA_DECAY_GATE,
          "token": FLA_DECAY_TOKEN}[decay_kind]
    if phi_elu1:
        f |= FLA_PHI_ELU1
    if normalize:
        f |= FLA_NORMALIZE
    return f


def _decay_kind(decay: Optional[torch.Tensor], decay_kind: Optional[str]) -> str:
    if decay_kind is not None:
        return decay_kind
    if decay is None:
        return "none"
    return {1: "gamma", 3: "token"}.get(decay.dim(), "gate")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: Optional[torch.Tensor] = None,
        *, decay_kind: Optional[str] = None, init_state: Optional[torch.Tensor] = None,
        out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
        want_final: bool = True, chunk: int = 64, phi_elu1: bool = False,
        normalize: bool = False, n_segments: Optional[int] = None, layout: str = "bhtd",
        noalloc: bool = False, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise forward.  q, k [B,H,T,dk]; v [B,H,T,dv] (bf16 or fp32, on the GPU);
    decay: gamma [H], gate [B,H,T,dk] or per-token scalar [B,H,T] (fp32); init/final state
    fp32 [B,H,dk,dv(+1)].  layout="bthd": token-major q, k [B,T,H,dk], v and out
    [B,T,H,dv], gate [B,T,H,dk], per-token decay [B,T,H].
    noalloc=True calls fla_linattn_fwd_noalloc (workspace from the library's static scratch
    array; automatic segment count only).
    Returns (out, final_state)."""
    if layout == "bthd":
        B, T, H, dk = q.shape
    elif layout == "bhtd":
        B, H, T, dk = q.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    dv = v.shape[-1]
    kind = _decay_kind(decay, decay_kind)
    ncol = dv + (1 if normalize else 0)
    if out is None:
        out = torch.empty((B, T, H, dv) if layout == "bthd" else (B, H, T, dv), dtype=q.dtype,
                          device=q.device)
    if final_state is None and want_final:
        final_state = torch.empty((B, H, dk, ncol), dtype=torch.float32, device=q.device)
    _check_tensors(q, (k, v, out), (decay, init_state, final_state))
    flags = flags_for(q.dtype, kind, phi_elu1, normalize)
    if layout == "bthd":
        flags |= FLA_LAYOUT_BTHD
    lib = load_library()
    if noalloc:
        if n_segments is not None:
            raise ValueError("the no-allocation entry point chooses the segment count itself")
        rc = lib.fla_linattn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(decay),
                                         _ptr(init_state), _ptr(out), _ptr(final_state), B, H,
                                         T, dk, dv, chunk, flags, _stream(stream))
    elif n_segments is None:
        rc = lib.fla_linattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(init_state),
                                 _ptr(out), _ptr(final_state), B, H, T, dk, dv, chunk, flags,
                                 _stream(stream))
    else:
        rc = lib.fla_linattn_fwd_segments(_ptr(q), _ptr(k), _ptr(v), _ptr(decay),
                                          _ptr(init_state), _ptr(out), _ptr(final_state), B, H,
                                          T, dk, dv, chunk, flags, int(n_segments),
                                          _stream(stream))
    if rc != FLA_OK:
        raise FlaError("fla_linattn_fwd", rc)
    return out, final_state


def step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor,
         decay: Optional[torch.Tensor] = None, *, decay_kind: Optional[str] = None,
         out: Optional[torch.Tensor] = None, phi_elu1: bool = False, normalize: bool = False,
         stream=None) -> torch.Tensor:
    """One decoding token: q, k [B,H,dk]; v [B,H,dv]; state fp32 [B,H,dk,dv(+1)] updated in
    place; decay gamma [H], gate [B,H,dk] or per-token scalar [B,H].  Returns out [B,H,dv]."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    if decay_kind is None:
        decay_kind = ("none" if decay is None
                      else {1: "gamma", 2: "token"}.get(decay.dim(), "gate"))
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _check_tensors(q, (k, v, out), (decay, state))
    flags = flags_for(q.dtype, decay_kind, phi_elu1, normalize)
    rc = load_library().fla_linattn_step(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(state),
                                         _ptr(out), B, H, dk, dv, flags, _stream(stream))
    if rc != FLA_OK:
        raise FlaError("fla_linattn_step", rc)
    return out


def segments_for(B, H, T, dk, dv, chunk, flags) -> int:
    n = ctypes.c_int64(0)
    rc = load_library().fla_linattn_segments_for(B, H, T, dk, dv, chunk, flags, ctypes.byref(n))
    if rc != FLA_OK:
        raise FlaError("fla_linattn_segments_for", rc)
    return int(n.value)


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
        decay: Optional[torch.Tensor] = None, *, decay_kind: Optional[str] = None,
        init_state: Optional[torch.Tensor] = None, dfinal: Optional[torch.Tensor] = None,
        want_dgate: bool = True, want_dinit: bool = True, chunk: int = 64,
        phi_elu1: bool = False, layout: str = "bhtd", stream=None):
    """Chunkwise backward.  Inputs as in ``fwd`` (no normaliser); dout laid out like v in
    q's dtype; dfinal fp32 [B,H,dk,dv] or None.  Returns (dq, dk, dv, dgate, dinit): dgate
    is shaped like the gate / per-token decay (None for gamma, no decay, or not wanted);
    dinit fp32 [B,H,dk,dv] (None if not wanted).  layout="bthd": token-major tensors as in
    ``fwd``."""
    if layout == "bthd":
        B, T, H, dk = q.shape
    elif layout == "bhtd":
        B, H, T, dk = q.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    dv = v.shape[-1]
    kind = _decay_kind(decay, decay_kind)
    _check_tensors(q, (k, v, dout), (decay, init_state, dfinal))
    dq, dkk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dgate = None
    if want_dgate and kind in ("gate", "token"):
        dgate = torch.empty_like(decay, dtype=torch.float32)
    dinit = None
    if want_dinit:
        dinit = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    flags = flags_for(q.dtype, kind, phi_elu1, False) | (FLA_LAYOUT_BTHD if layout == "bthd" else 0)
    rc = load_library().fla_linattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(init_state),
                                        _ptr(dout), _ptr(dfinal), _ptr(dq), _ptr(dkk), _ptr(dvv),
                                        _ptr(dgate), _ptr(dinit), B, H, T, dk, dv, chunk, flags,
                                        _stream(stream))
    if rc != FLA_OK:
        raise FlaError("fla_linattn_bwd", rc)
    return dq, dkk, dvv, dgate, dinit


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
               decay: Optional[torch.Tensor] = None, *, decay_kind: Optional[str] = None,
               init_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               final_state: Optional[torch.Tensor] = None, want_final: bool = True,
               chunk: int = 64, phi_elu1: bool = False, normalize: bool = False,
               stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward over packed sequences.  q, k [total,H,dk]; v [total,H,dv]; cu_seqlens int64
    [N+1] on the GPU (sequence s = tokens cu[s]..cu[s+1]-1); decay: gamma [H], gate
    [total,H,dk] or per-token [total,H]; states fp32 [N,H,dk,dv(+1)].  Returns (out, final)."""
    total, H, dk = q.shape
    dv = v.shape[-1]
    n = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int64 or n < 1:
        raise ValueError("cu_seqlens must be an int64 tensor of N + 1 offsets")
    if decay_kind is None:
        decay_kind = ("none" if decay is None
                      else {1: "gamma", 2: "token"}.get(decay.dim(), "gate"))
    ncol = dv + (1 if normalize else 0)
    if out is None:
        out = torch.empty((total, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and want_final:
        final_state = torch.empty((n, H, dk, ncol), dtype=torch.float32, device=q.device)
    _check_tensors(q, (k, v, out), (decay, init_state, final_state), (cu_seqlens,))
    flags = flags_for(q.dtype, decay_kind, phi_elu1, normalize) | FLA_LAYOUT_BTHD
    rc = load_library().fla_linattn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(decay),
                                               _ptr(init_state), _ptr(out), _ptr(final_state),
                                               _ptr(cu_seqlens), n, total, H, dk, dv, chunk,
                                               flags, _stream(stream))
    if rc != FLA_OK:
        raise FlaError("fla_linattn_fwd_varlen", rc)
    return out, final_state


def bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
               cu_seqlens: torch.Tensor, decay: Optional[torch.Tensor] = None, *,
               decay_kind: Optional[str] = None, init_state: Optional[torch.Tensor] = None,
               dfinal: Optional[torch.Tensor] = None, want_dgate: bool = True,
               want_dinit: bool = True, chunk: int = 64, phi_elu1: bool = False, stream=None):
    """Backward over packed sequences (the gradients of ``fwd_varlen``).  Tensors as in
    ``fwd_varlen``; dout [total,H,dv]; dfinal fp32 [N,H,dk,dv] or None.  Returns
    (dq, dk, dv, dgate, dinit) as ``bwd`` does, dinit [N,H,dk,dv]."""
    total, H, dk = q.shape
    dv = v.shape[-1]
    n = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int64 or n < 1:
        raise ValueError("cu_seqlens must be an int64 tensor of N + 1 offsets")
    if decay_kind is None:
        decay_kind = ("none" if decay is None
                      else {1: "gamma", 2: "token"}.get(decay.dim(), "gate"))
    _check_tensors(q, (k, v, dout), (decay, init_state, dfinal), (cu_seqlens,))
    dq, dkk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dgate = None
    if want_dgate and decay_kind in ("gate", "token"):
        dgate = torch.empty_like(decay, dtype=torch.float32)
    dinit = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device) if want_dinit else None
    flags = flags_for(q.dtype, decay_kind, phi_elu1, False) | FLA_LAYOUT_BTHD
    rc = load_library().fla_linattn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(decay),
                                               _ptr(init_state), _ptr(dout), _ptr(dfinal),
                                               _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dgate),
                                               _ptr(dinit), _ptr(cu_seqlens), n, total, H, dk,
                                               dv, chunk, flags, _stream(stream))
    if rc != FLA_OK:
        raise FlaError("fla_linattn_bwd_varlen", rc)
    return dq, dkk, dvv, dgate, dinit


def fwd_proj(x: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor, H: int,
             decay: Optional[torch.Tensor] = None, *, decay_kind: Optional[str] = None,
             init_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
             final_state: Optional[torch.Tensor] = None, want_final: bool = True,
             chunk: int = 64, phi_elu1: bool = False, normalize: bool = False,
             stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Projections + feature map + forward: x [B,T,hidden]; w_q, w_k [hidden,H*dk]; w_v
    [hidden,H*dv] (x's dtype); decay gamma [H], gate [B,T,H,dk] or per-token [B,T,H].
    Returns (out [B,T,H,dv], final_state [B,H,dk,dv(+1)])."""
    B, T, hidden = x.shape
    dk = w_q.shape[1] // H
    dv = w_v.shape[1] // H
    if w_q.shape != (hidden, H * dk) or w_k.shape != w_q.shape or w_v.shape != (hidden, H * dv):
        raise ValueError("projection shapes: w_q, w_k [hidden, H*dk], w_v [hidden, H*dv]")
    if decay_kind is None:
        decay_kind = ("none" if decay is None
                      else {1: "gamma", 3: "token"}.get(decay.dim(), "gate"))
    ncol = dv + (1 if normalize else 0)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=x.dtype, device=x.device)
    if final_state is None and want_final:
        final_state = torch.empty((B, H, dk, ncol), dtype=torch.float32, device=x.device)
    _check_tensors(x, (w_q, w_k, w_v, out), (decay, init_state, final_state))
    flags = flags_for(x.dtype, decay_kind, phi_elu1, normalize) | FLA_LAYOUT_BTHD
    rc = load_library().fla_linattn_fwd_proj(_ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                                             _ptr(decay), _ptr(init_state), _ptr(out),
                                             _ptr(final_state), B, T, hidden, H, dk, dv, chunk,
                                             flags, _stream(stream))
    if rc != FLA_OK:
        raise FlaError("fla_linattn_fwd_proj", rc)
    return out, final_state


def gdn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
            beta: torch.Tensor, *, init_state: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
            want_final: bool = True, chunk: int = 64,
            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated delta rule forward.  q, k [B,H,T,dk]; v [B,H,T,dv] (bf16 or fp32); alpha, beta
    fp32 [B,H,T]; states fp32 [B,H,dk,dv].  Returns (out, final_state)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if final_state is None and want_final:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    _check_tensors(q, (k, v, out), (alpha, beta, init_state, final_state))
    flags = FLA_BF16 if q.dtype == torch.bfloat16 else 0
    rc = load_library().fla_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(init_state), _ptr(out), _ptr(final_state), B, H, T, dk,
                                     dv, chunk, flags, _stream(stream))
    if rc != FLA_OK:
        raise FlaError("fla_gdn_fwd", rc)
    return out, final_state


def probe_stream(src: torch.Tensor, dst: torch.Tensor, nbytes: int, pattern: int,
                 stream=None) -> None:
    """One pass of the HBM streaming probe (include/fla_probe.h): PROBE_READ reads nbytes
    of src (dst gets one word per workgroup), PROBE_COPY copies nbytes, PROBE_MIX5 reads
    5/6 and writes 1/6 of nbytes."""
    for t in (src, dst):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("probe buffers must be contiguous device tensors")
    rc = load_library().fla_probe_stream(_ptr(src), _ptr(dst), int(nbytes), int(pattern),
                                         _stream(stream))
    if rc != 0:
        raise FlaError("fla_probe_stream", rc)


def probe_chunk_pattern(q: torch.Tensor, k: torch.Tensor, gate: torch.Tensor, v: torch.Tensor,
                        out: torch.Tensor, stream=None) -> None:
    """One launch of the forward pass's access-pattern probe (include/fla_probe.h): q, k
    bf16 [B,H,T,128], gate fp32 [B,H,T,128], v and out bf16 [B,H,T,dv]."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    for t in (q, k, gate, v, out):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("probe tensors must be contiguous device tensors")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype or \
            out.dtype != q.dtype or gate.dtype != torch.float32:
        raise ValueError("q, k, v, out must be bf16 and the gate fp32")
    if k.shape != q.shape or gate.shape != q.shape or v.shape[:3] != q.shape[:3] or \
            out.shape != v.shape:
        raise ValueError("shapes must be q, k, gate [B,H,T,128] and v, out [B,H,T,dv]")
    rc = load_library().fla_probe_chunk_pattern(_ptr(q), _ptr(k), _ptr(gate), _ptr(v),
                                                _ptr(out), B, H, T, dk, dv, _stream(stream))
    if rc != 0:
        raise FlaError("fla_probe_chunk_pattern", rc)


def probe_mfma(out: torch.Tensor, workgroups: int, iters: int, stream=None) -> float:
    """One launch of the bf16 MFMA probe; returns the dense FLOPs it performs.
    out: fp32 device tensor of at least 4 * workgroups elements."""
    if out.dtype != torch.float32 or out.numel() < 4 * workgroups or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor of 4 * workgroups elements")
    lib = load_library()
    rc = lib.fla_probe_mfma(_ptr(out), int(workgroups), int(iters), _stream(stream))
    if rc != 0:
        raise FlaError("fla_probe_mfma", rc)
    return float(lib.fla_probe_mfma_flops(int(workgroups), int(iters)))
