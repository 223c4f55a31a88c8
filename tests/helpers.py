"""Shared test helpers: tensor <-> oracle-array conversion and tolerances.

Conversions only; no quantization arithmetic lives here.
"""
import numpy as np
import torch


def to_oracle(t: torch.Tensor) -> np.ndarray:
    """Device/CPU tensor -> numpy in the oracle's convention (f32 as float32,
    bf16/f16 as uint16 bits, int32 codes as uint32, u8 as uint8)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def from_bits(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    if dtype in (torch.bfloat16, torch.float16):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dtype)
    if dtype == torch.int32:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32))
    return torch.from_numpy(np.ascontiguousarray(a))


ORACLE_DT = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


def normwise_rel_err(y_gpu: torch.Tensor, y_ref: np.ndarray) -> float:
    """max|y - y_ref| / max|y_ref| over the whole output."""
    y = y_gpu.detach().float().cpu().double().numpy()
    den = np.abs(y_ref).max()
    num = np.abs(y - y_ref).max()
    return float(num / den) if den > 0 else float(num)


def tolerance(dtype: torch.dtype, K: int) -> float:
    """Matmul acceptance: normwise 1e-5*sqrt(K) for fp32 outputs, 2e-2 for
    16-bit outputs (fp32 accumulation in both cases)."""
    return 1e-5 * np.sqrt(K) if dtype == torch.float32 else 2e-2
