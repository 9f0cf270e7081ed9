"""Helpers shared by the GPU tests, the smoke check and the bench: moving seeded inputs
to the device, and the tolerance checks.

Tolerances (the acceptance bar for this path):
  * fp32 I/O: max |x - x_oracle| <= 1e-3, for outputs and final states separately;
  * bf16 I/O (fp32 accumulation and state): error / rms(x_oracle) <= 2e-2, outputs and
    final states each against their own RMS.  The final state is stored in fp32 and
    the bound applies to max |x - x_oracle|.  The outputs are stored in bf16, and
    rounding the exact result to bf16 alone already moves the largest outputs by more
    than 2e-2 * rms (the outputs' max/rms ratio is about 15), so for them the bound
    applies to the kernel's own error: max_i (|x_i - x_oracle_i| - |x_i| / 255) where
    |x_i| / 255 bounds the round-to-nearest-even storage rounding of the kernel's fp32
    result y_i (|y - bf16(y)| <= 2^-8 |y| and |y| <= |x| / (1 - 2^-8)).
  * fp16 I/O: the same bar as bf16, with the fp16 storage allowance |x_i| / 2047 + 2^-25
    (|y - fp16(y)| <= 2^-11 |y| for normal values, at most 2^-25 below the normal range).
NMSE = sum (x - x_ref)^2 / sum x_ref^2 and the plain max |x - x_ref| / rms are
reported beside them.
"""
from __future__ import annotations

import numpy as np
import torch

TOL_F32_ABS = 1e-3
TOL_BF16_REL_RMS = 2e-2
TOL_16BIT_REL_RMS = TOL_BF16_REL_RMS

TORCH_IO = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def to_device(x, device="cuda"):
    """Seeded numpy inputs -> device tensors in the storage types the library takes."""
    io = TORCH_IO[x.io]

    def t(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)

    d = dict(q=t(x.q, io), k=t(x.k, io), v=t(x.v, io), g=t(x.g, torch.float32),
             beta=t(x.beta, torch.float32),
             cu_seqlens=t(x.cu_seqlens, torch.int32) if x.N > 1 else None,
             initial_state=None if x.initial_state is None else t(x.initial_state, torch.float32))
    return d


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def storage_allowance(got: np.ndarray, storage) -> np.ndarray:
    """Bound on |y - round(y)| for the kernel's fp32 result y behind each stored value
    got (storage: None / False = not rounded, 'bf16' or True, 'f16')."""
    if storage in ("bf16", True):
        return np.abs(got) / 255.0
    if storage == "f16":
        return np.abs(got) / 2047.0 + 2.0 ** -25
    return np.zeros_like(got)


def error_stats(got: np.ndarray, ref: np.ndarray, storage=None) -> dict:
    """storage: the storage rounding to allow for, as in storage_allowance."""
    diff = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    mx = float(diff.max()) if diff.size else 0.0
    kernel_err = diff - storage_allowance(got, storage)
    kmx = float(max(kernel_err.max(), 0.0)) if diff.size else 0.0
    den = float(np.sum(ref ** 2))
    return dict(max_abs=mx, rms_ref=rms, rel_rms=(mx / rms if rms > 0 else mx),
                kernel_rel_rms=(kmx / rms if rms > 0 else kmx),
                nmse=(float(np.sum(diff ** 2)) / den if den > 0 else float(np.sum(diff ** 2))),
                finite=bool(np.all(np.isfinite(got))))


def check_pair(name: str, a: np.ndarray, b: np.ndarray, io: str, stored=True) -> float:
    """Two kernels' results for the same inputs: each is within the tolerance of the exact
    result, so they differ by at most twice the tolerance, beside both storage roundings
    (stored: whether a and b were stored in io)."""
    st = io if (stored and io != "f32") else None
    diff = np.abs(a - b) - storage_allowance(a, st) - storage_allowance(b, st)
    rms = float(np.sqrt(np.mean(b ** 2))) if b.size else 0.0
    err = float(max(diff.max(), 0.0)) if diff.size else 0.0
    print(f"  {name}: (|a - b| - roundings) max={err:.3e} rms={rms:.3e}", flush=True)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), f"{name}: non-finite values"
    if io == "f32":
        assert err <= 2 * TOL_F32_ABS, f"{name}: {err:.3e} > 2 x {TOL_F32_ABS}"
    else:
        assert err <= 2 * TOL_BF16_REL_RMS * rms, f"{name}: {err / rms:.3e} of rms > 2 x {TOL_BF16_REL_RMS}"
    return err


def check(name: str, got: np.ndarray, ref: np.ndarray, io: str, stored=None) -> dict:
    """stored: the 16-bit type `got` was stored in, or None / False (default: io
    when io is 16-bit and the name does not mention a state)."""
    if stored is None:
        stored = io if io != "f32" and "state" not in name else None
    s = error_stats(got, ref, storage=stored)
    print(f"  {name}: max_abs={s['max_abs']:.3e} rms_ref={s['rms_ref']:.3e} "
          f"max/rms={s['rel_rms']:.3e} kernel/rms={s['kernel_rel_rms']:.3e} "
          f"nmse={s['nmse']:.3e}", flush=True)
    assert s["finite"], f"{name}: non-finite values"
    if io == "f32":
        assert s["max_abs"] <= TOL_F32_ABS, f"{name}: max abs {s['max_abs']:.3e} > {TOL_F32_ABS}"
    else:
        if s["rms_ref"] == 0.0:
            assert s["max_abs"] == 0.0, f"{name}: reference is zero, got {s['max_abs']:.3e}"
        else:
            assert s["kernel_rel_rms"] <= TOL_BF16_REL_RMS, (
                f"{name}: error / rms {s['kernel_rel_rms']:.3e} > {TOL_BF16_REL_RMS}")
    return s
