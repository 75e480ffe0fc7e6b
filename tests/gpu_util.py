"""Shared helpers of the GPU parity tests (host side only)."""
import numpy as np
import torch

from synth import bf16_bits_to_f32

# tolerances of the sparse-attention outputs and gradients
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 2e-2
FP32_REL_L2 = 1e-5
FP32_MAX_ABS = 1e-5


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy fp32 -> cuda float32; numpy uint16 (bf16 bits) -> cuda bf16."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).cuda()
    if a.dtype == np.float64:
        return torch.from_numpy(a).cuda()
    if a.dtype in (np.int32, np.int64):
        return torch.from_numpy(a.astype(np.int32)).cuda()
    raise TypeError(a.dtype)


def widen(a: np.ndarray) -> np.ndarray:
    """Storage buffer -> fp64 (exact)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def err_stats(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)
    return rel, float(np.abs(diff).max()) if diff.size else 0.0


def assert_close(got, ref, bf16: bool, what: str = ""):
    rel, mx = err_stats(got, ref)
    rl, ma = (BF16_REL_L2, BF16_MAX_ABS) if bf16 else (FP32_REL_L2, FP32_MAX_ABS)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert rel <= rl and mx <= ma, f"{what}: rel L2 {rel:.3e} max-abs {mx:.3e}"
    return rel, mx
