"""Python binding of the gated delta-rule C-ABI (include/gdn.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs are allocated with torch, and raw device pointers plus torch's
current HIP stream are handed to ``gdn_prefill`` / ``gdn_decode_step`` in
``libgdn_mi355x.so`` (and the per-key-channel variants ``gdn_kda_prefill`` /
``gdn_kda_decode_step``).  Every step of the computation runs in the library's HIP
kernels; there is no fallback: if the library is missing or the tensors are not
on a GPU the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

from .build import LIB_PATH

GDN_F32 = 0
GDN_BF16 = 1
GDN_F16 = 2
# input prologue flags (gdn_prologue_flags)
PROLOGUE_QK_L2NORM = 1
PROLOGUE_BETA_SIGMOID = 2
PROLOGUE_G_SOFTPLUS = 4
PROLOGUE_ALL = 7
D = 128
CHUNK = 64

_lib = None


class GDNError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load the built HIP library (never builds it)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m linear_attention_chunked_gdn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, fp, ip, i32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32
    lib.gdn_prefill.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32, i32,
                                ctypes.c_int, vp, fp, vp]
    lib.gdn_prefill.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, i32, i32, i32, i32, i32, ctypes.c_int,
                                    vp, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    p32 = ctypes.POINTER(ctypes.c_int32)
    lib.gdn_prefill_plan.argtypes = [i32, i32, i32, ctypes.c_int, p32, p32, p32, p32]
    lib.gdn_prefill_plan.restype = ctypes.c_int
    lib.gdn_prefill_fused.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32, i32,
                                      ctypes.c_int, ctypes.c_uint32, vp, fp, vp]
    lib.gdn_prefill_fused.restype = ctypes.c_int
    lib.gdn_decode_step_fused.argtypes = [vp, vp, vp, fp, fp, fp, i32, i32, i32, i32, i32, ctypes.c_int,
                                          ctypes.c_uint32, vp, vp]
    lib.gdn_decode_step_fused.restype = ctypes.c_int
    lib.gdn_kda_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_kda_workspace_size.restype = ctypes.c_int
    lib.gdn_kda_prefill.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32, i32,
                                    ctypes.c_int, vp, ctypes.c_size_t, vp, fp, vp]
    lib.gdn_kda_prefill.restype = ctypes.c_int
    lib.gdn_prefill_split_workspace_size.argtypes = lib.gdn_kda_workspace_size.argtypes
    lib.gdn_prefill_split_workspace_size.restype = ctypes.c_int
    lib.gdn_prefill_split.argtypes = lib.gdn_kda_prefill.argtypes
    lib.gdn_prefill_split.restype = ctypes.c_int
    lib.gdn_prefill_split_noalloc.argtypes = lib.gdn_prefill.argtypes
    lib.gdn_prefill_split_noalloc.restype = ctypes.c_int
    lib.gdn_prefill_split_fused.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32, i32,
                                            ctypes.c_int, ctypes.c_uint32, vp, ctypes.c_size_t, vp, fp, vp]
    lib.gdn_prefill_split_fused.restype = ctypes.c_int
    lib.gdn_prefill_seg_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_prefill_seg_workspace_size.restype = ctypes.c_int
    lib.gdn_prefill_seg_choose.argtypes = [i32, i32, i32, i32, p32]
    lib.gdn_prefill_seg_choose.restype = ctypes.c_int
    lib.gdn_prefill_seg.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32, i32, i32,
                                    ctypes.c_int, vp, ctypes.c_size_t, vp, fp, vp]
    lib.gdn_prefill_seg.restype = ctypes.c_int
    lib.gdn_kda_prefill_seg.argtypes = lib.gdn_prefill_seg.argtypes
    lib.gdn_kda_prefill_seg.restype = ctypes.c_int
    lib.gdn_kda_decode_step.argtypes = lib.gdn_decode_step.argtypes
    lib.gdn_kda_decode_step.restype = ctypes.c_int
    lib.gdn_prefill_auto_plan.argtypes = [i32, i32, i32, ctypes.c_int, ctypes.c_uint32, p32, p32,
                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_prefill_auto_plan.restype = ctypes.c_int
    lib.gdn_prefill_auto.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32,
                                     ctypes.c_int, ctypes.c_uint32, vp, ctypes.c_size_t, vp, fp, vp]
    lib.gdn_prefill_auto.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(lib, status: int, what: str):
    if status != 0:
        name = lib.gdn_status_string(status).decode()
        detail = lib.gdn_last_error().decode()
        raise GDNError(status, f"{what}: {name}: {detail}")


def _io_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return GDN_F16
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v must be bfloat16, float16 or float32, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fits(t, dtype, shape, device) -> bool:
    return (isinstance(t, torch.Tensor) and t.dtype == dtype and t.shape == shape and t.device == device
            and t.is_contiguous())


def _decode_call(lib, fn, name: str, q, k, v, g, g_shape, beta, state, out, extra=()):
    """The decode steps' marshalling, kept short (a serving loop calls it once per token):
    one combined check of every tensor (the detailed one only when it fails), raw
    pointers as integers, and no device switch when q's device is already current."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"gdn.{name} runs on the GPU only; q is on {dev}")
    io = _io_code(q)
    B, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    if out is None:
        out = torch.empty((B, Hv, Dv), dtype=q.dtype, device=dev)
    checks = ((k, "k", q.dtype, (B, Hk, Dk)), (v, "v", q.dtype, (B, Hv, Dv)),
              (g, "g", torch.float32, g_shape(B, Hv, Dk)), (beta, "beta", torch.float32, (B, Hv)),
              (state, "state", torch.float32, (B, Hv, Dv, Dk)), (out, "out", q.dtype, (B, Hv, Dv)))
    if not (q.is_contiguous() and all(_fits(t, dt, sh, dev) for t, _, dt, sh in checks)):
        if not q.is_contiguous():
            raise ValueError("q must be contiguous")
        for t, nm, dt, sh in checks:
            _need(t, nm, dt, sh, dev)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), state.data_ptr(),
            B, Hk, Hv, Dk, Dv, io) + tuple(extra)
    if dev.index == torch.cuda.current_device():
        st = fn(*args, out.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    else:
        with torch.cuda.device(dev):
            st = fn(*args, out.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    if st != 0:
        _check(lib, st, name)
    return out


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
            beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
            cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = CHUNK,
            output_final_state: bool = True, out: Optional[torch.Tensor] = None,
            final_state: Optional[torch.Tensor] = None, prologue: int = 0, lib=None
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Packed chunked prefill.  q, k: [T, Hk, 128]; v: [T, Hv, 128] (bf16, fp16 or fp32,
    all the same); g, beta: [T, Hv] fp32; initial_state: [N, Hv, 128, 128] fp32 or None;
    cu_seqlens: [N+1] int32 on the device, or None for one sequence.  Returns
    (o [T, Hv, 128], final_state [N, Hv, 128, 128] fp32 or None).  A nonzero
    ``prologue`` (PROLOGUE_* flags) calls gdn_prefill_fused: q, k, g, beta are then the
    values before those steps."""
    lib = lib or load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn.prefill runs on the GPU only; q is on " + str(dev))
    io = _io_code(q)
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _need(q, "q", q.dtype, (T, Hk, Dk), dev)
    _need(k, "k", q.dtype, (T, Hk, Dk), dev)
    _need(v, "v", q.dtype, (T, Hv, Dv), dev)
    _need(g, "g", torch.float32, (T, Hv), dev)
    _need(beta, "beta", torch.float32, (T, Hv), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, Hv, Dv, Dk), dev)
    if out is None:
        out = torch.empty((T, Hv, Dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (T, Hv, Dv), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, Hv, Dv, Dk), dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        if prologue:
            st = lib.gdn_prefill_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                       _ptr(cu_seqlens), N, T, Hk, Hv, Dk, Dv, chunk_size, io, prologue,
                                       _ptr(out), _ptr(final_state), ctypes.c_void_p(stream))
        else:
            st = lib.gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                 _ptr(cu_seqlens), N, T, Hk, Hv, Dk, Dv, chunk_size, io, _ptr(out),
                                 _ptr(final_state), ctypes.c_void_p(stream))
    _check(lib, st, "gdn_prefill_fused" if prologue else "gdn_prefill")
    return out, final_state


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                beta: torch.Tensor, state: torch.Tensor, out: Optional[torch.Tensor] = None,
                prologue: int = 0, lib=None) -> torch.Tensor:
    """One token per sequence; ``state`` [B, Hv, 128, 128] fp32 is updated in place.
    q, k: [B, Hk, 128]; v: [B, Hv, 128]; g, beta: [B, Hv].  Returns o [B, Hv, 128].
    A nonzero ``prologue`` calls gdn_decode_step_fused."""
    lib = lib or load_library()
    if prologue:
        return _decode_call(lib, lib.gdn_decode_step_fused, "gdn_decode_step_fused", q, k, v, g,
                            lambda B, Hv, Dk: (B, Hv), beta, state, out, extra=(int(prologue),))
    return _decode_call(lib, lib.gdn_decode_step, "gdn_decode_step", q, k, v, g, lambda B, Hv, Dk: (B, Hv),
                        beta, state, out)


def kda_workspace_size(N: int, T: int, Hv: int, chunk_size: int = CHUNK, lib=None) -> int:
    """Workspace bytes gdn_kda_prefill needs for N sequences, T packed tokens, Hv heads."""
    lib = lib or load_library()
    n = ctypes.c_size_t()
    _check(lib, lib.gdn_kda_workspace_size(N, T, Hv, chunk_size, ctypes.byref(n)), "gdn_kda_workspace_size")
    return int(n.value)


def kda_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = CHUNK,
                output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                final_state: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                lib=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Packed chunked prefill with one decay per key channel: as ``prefill`` except
    g: [T, Hv, 128] fp32 and q, k, v bf16 or fp16.  ``workspace`` (a uint8 device tensor
    of at least ``kda_workspace_size`` bytes) is allocated here when not given."""
    return _prefill_ws("gdn_kda_prefill", kda_workspace_size, True, q, k, v, g, beta, initial_state,
                       cu_seqlens, chunk_size, output_final_state, out, final_state, workspace, lib)


def _prefill_ws(fn: str, size_fn, per_channel: bool, q, k, v, g, beta, initial_state, cu_seqlens,
                chunk_size, output_final_state, out, final_state, workspace, lib, extra=(),
                extra_after_io: bool = False):
    """The entry points that take a caller-owned workspace (gdn_kda_prefill, gdn_prefill_split,
    gdn_prefill_split_fused, gdn_prefill_seg, gdn_prefill_auto: chunk_size None, it has no
    such argument); ``extra`` holds further integer arguments,
    which size_fn takes too: after chunk_size (the segment count), or after io_dtype with
    extra_after_io (the prologue flags)."""
    lib = lib or load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"{fn} runs on the GPU only; q is on " + str(dev))
    io = _io_code(q)
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _need(q, "q", q.dtype, (T, Hk, Dk), dev)
    _need(k, "k", q.dtype, (T, Hk, Dk), dev)
    _need(v, "v", q.dtype, (T, Hv, Dv), dev)
    _need(g, "g", torch.float32, (T, Hv, Dk) if per_channel else (T, Hv), dev)
    _need(beta, "beta", torch.float32, (T, Hv), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, Hv, Dv, Dk), dev)
    if out is None:
        out = torch.empty((T, Hv, Dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (T, Hv, Dv), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, Hv, Dv, Dk), dev)
    need = size_fn(N, T, Hv, chunk_size, *extra, lib=lib)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on " + str(dev))
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        pre, post = ((), extra) if extra_after_io else (extra, ())
        chunk = () if chunk_size is None else (chunk_size,)   # gdn_prefill_auto has none
        st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                              _ptr(cu_seqlens), N, T, Hk, Hv, Dk, Dv, *chunk, *pre, io, *post, _ptr(workspace),
                              workspace.numel(), _ptr(out), _ptr(final_state), ctypes.c_void_p(stream))
    _check(lib, st, fn)
    return out, final_state


def prefill_split_workspace_size(N: int, T: int, Hv: int, chunk_size: int = CHUNK, lib=None) -> int:
    """Workspace bytes gdn_prefill_split needs for N sequences, T packed tokens, Hv heads."""
    lib = lib or load_library()
    n = ctypes.c_size_t()
    _check(lib, lib.gdn_prefill_split_workspace_size(N, T, Hv, chunk_size, ctypes.byref(n)),
           "gdn_prefill_split_workspace_size")
    return int(n.value)


def prefill_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = CHUNK,
                  output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  prologue: int = 0, lib=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``prefill`` in two launches (gdn_prefill_split): q, k, v bf16 or fp16; ``workspace``
    (a uint8 device tensor of at least ``prefill_split_workspace_size`` bytes) is allocated
    here when not given.  A nonzero ``prologue`` (PROLOGUE_* flags) calls
    gdn_prefill_split_fused: q, k, g, beta are then the raw inputs of those steps."""
    if prologue:
        size_fn = lambda N, T, Hv, C, _p, lib=None: prefill_split_workspace_size(N, T, Hv, C, lib=lib)  # noqa: E731
        return _prefill_ws("gdn_prefill_split_fused", size_fn, False, q, k, v, g, beta, initial_state,
                           cu_seqlens, chunk_size, output_final_state, out, final_state, workspace, lib,
                           extra=(int(prologue),), extra_after_io=True)
    return _prefill_ws("gdn_prefill_split", prefill_split_workspace_size, False, q, k, v, g, beta,
                       initial_state, cu_seqlens, chunk_size, output_final_state, out, final_state,
                       workspace, lib)


NOALLOC_SCRATCH_BYTES = 96 << 20   # GDN_NOALLOC_SCRATCH_BYTES


def prefill_split_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                          cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = CHUNK,
                          output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                          final_state: Optional[torch.Tensor] = None, lib=None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``prefill_split`` without a workspace (gdn_prefill_split_noalloc): the library's
    static per-GPU scratch stands in for it.  Pass ``out`` (and ``final_state``) to make
    the call allocate nothing at all; sizes beyond NOALLOC_SCRATCH_BYTES of workspace
    raise GDNError."""
    lib = lib or load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_prefill_split_noalloc runs on the GPU only; q is on " + str(dev))
    io = _io_code(q)
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _need(q, "q", q.dtype, (T, Hk, Dk), dev)
    _need(k, "k", q.dtype, (T, Hk, Dk), dev)
    _need(v, "v", q.dtype, (T, Hv, Dv), dev)
    _need(g, "g", torch.float32, (T, Hv), dev)
    _need(beta, "beta", torch.float32, (T, Hv), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, Hv, Dv, Dk), dev)
    if out is None:
        out = torch.empty((T, Hv, Dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (T, Hv, Dv), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, Hv, Dv, Dk), dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.gdn_prefill_split_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                           _ptr(cu_seqlens), N, T, Hk, Hv, Dk, Dv, chunk_size, io, _ptr(out),
                                           _ptr(final_state), ctypes.c_void_p(stream))
    _check(lib, st, "gdn_prefill_split_noalloc")
    return out, final_state


def prefill_seg_workspace_size(N: int, T: int, Hv: int, chunk_size: int = CHUNK, segments: int = 1,
                               lib=None) -> int:
    """Workspace bytes gdn_prefill_seg needs for N sequences, T packed tokens, Hv heads and
    ``segments`` segments per sequence."""
    lib = lib or load_library()
    n = ctypes.c_size_t()
    _check(lib, lib.gdn_prefill_seg_workspace_size(N, T, Hv, chunk_size, segments, ctypes.byref(n)),
           "gdn_prefill_seg_workspace_size")
    return int(n.value)


def prefill_seg_choose(N: int, T: int, Hv: int, chunk_size: int = CHUNK, lib=None) -> int:
    """gdn_prefill_seg_choose: the segment count for these sizes on the current device."""
    lib = lib or load_library()
    n = ctypes.c_int32()
    _check(lib, lib.gdn_prefill_seg_choose(N, T, Hv, chunk_size, ctypes.byref(n)), "gdn_prefill_seg_choose")
    return int(n.value)


def prefill_seg(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = CHUNK,
                segments: Optional[int] = None, output_final_state: bool = True,
                out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, lib=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``prefill_split`` with each sequence's recurrence run as ``segments`` concurrent
    segments (gdn_prefill_seg); ``segments`` defaults to ``prefill_seg_choose``'s count."""
    lib = lib or load_library()
    if segments is None:
        N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
        with torch.cuda.device(q.device):
            segments = prefill_seg_choose(N, q.shape[0], v.shape[1], chunk_size, lib=lib)
    return _prefill_ws("gdn_prefill_seg", prefill_seg_workspace_size, False, q, k, v, g, beta,
                       initial_state, cu_seqlens, chunk_size, output_final_state, out, final_state,
                       workspace, lib, extra=(int(segments),))


def kda_prefill_seg(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                    cu_seqlens: Optional[torch.Tensor] = None, segments: Optional[int] = None,
                    output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                    final_state: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    lib=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``kda_prefill`` with each sequence's recurrence run as ``segments`` concurrent
    segments (gdn_kda_prefill_seg; g: [T, Hv, 128]); ``segments`` defaults to
    ``prefill_seg_choose``'s count."""
    lib = lib or load_library()
    if segments is None:
        N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
        with torch.cuda.device(q.device):
            segments = prefill_seg_choose(N, q.shape[0], v.shape[1], CHUNK, lib=lib)
    return _prefill_ws("gdn_kda_prefill_seg", prefill_seg_workspace_size, True, q, k, v, g, beta,
                       initial_state, cu_seqlens, CHUNK, output_final_state, out, final_state,
                       workspace, lib, extra=(int(segments),))


def kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, state: torch.Tensor, out: Optional[torch.Tensor] = None,
                    lib=None) -> torch.Tensor:
    """One token per sequence with one decay per key channel: as ``decode_step`` except
    g: [B, Hv, 128] fp32."""
    lib = lib or load_library()
    return _decode_call(lib, lib.gdn_kda_decode_step, "gdn_kda_decode_step", q, k, v, g,
                        lambda B, Hv, Dk: (B, Hv, Dk), beta, state, out)


PATH_ONE_LAUNCH, PATH_SPLIT, PATH_SEG = 0, 1, 2
PATH_NAMES = {PATH_ONE_LAUNCH: "one_launch", PATH_SPLIT: "split", PATH_SEG: "seg"}


def prefill_auto_plan(N: int, T: int, Hv: int, io_dtype: int = GDN_BF16, prologue: int = 0, lib=None) -> dict:
    """gdn_prefill_auto_plan: the path gdn_prefill_auto takes on the current device for these
    sizes ("one_launch", "split" or "seg"), its segment count and workspace bytes."""
    lib = lib or load_library()
    path, seg, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_size_t()
    _check(lib, lib.gdn_prefill_auto_plan(N, T, Hv, io_dtype, prologue, ctypes.byref(path), ctypes.byref(seg),
                                          ctypes.byref(n)), "gdn_prefill_auto_plan")
    return {"path": PATH_NAMES[path.value], "segments": seg.value, "workspace_bytes": int(n.value)}


def prefill_auto(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                 beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                 cu_seqlens: Optional[torch.Tensor] = None, output_final_state: bool = True,
                 out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, prologue: int = 0, lib=None
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``prefill`` through the fastest path for these sizes (gdn_prefill_auto).  A workspace
    of ``prefill_auto_plan(...)["workspace_bytes"]`` bytes is allocated here when not
    given."""
    lib = lib or load_library()
    if q.device.type != "cuda":
        raise ValueError("gdn_prefill_auto runs on the GPU only; q is on " + str(q.device))
    if workspace is None:   # the library checks a given workspace's size itself
        N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
        with torch.cuda.device(q.device):
            need = prefill_auto_plan(N, q.shape[0], v.shape[1], _io_code(q), prologue, lib=lib)["workspace_bytes"]
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    size_fn = lambda N, T, Hv, C, _p, lib=None: 0  # noqa: E731
    return _prefill_ws("gdn_prefill_auto", size_fn, False, q, k, v, g, beta, initial_state, cu_seqlens,
                       None, output_final_state, out, final_state, workspace, lib, extra=(int(prologue),),
                       extra_after_io=True)


def prefill_plan(N: int, Hv: int, io_dtype: int = GDN_BF16, lib=None) -> dict:
    """Launch shape of gdn_prefill for these sizes (host only, launches nothing)."""
    lib = lib or load_library()
    dvs, wg, lds, thr = (ctypes.c_int32() for _ in range(4))
    st = lib.gdn_prefill_plan(N, Hv, D, io_dtype, ctypes.byref(dvs), ctypes.byref(wg), ctypes.byref(lds),
                              ctypes.byref(thr))
    _check(lib, st, "gdn_prefill_plan")
    return dict(dv_per_workgroup=dvs.value, workgroups=wg.value, lds_bytes=lds.value,
                threads_per_workgroup=thr.value)
