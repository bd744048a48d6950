"""Helpers for the GPU parity tests: moving 16-bit bit patterns between NumPy and torch."""
import numpy as np
import torch

DEV = "cuda"
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def bits_to_dev(bits_u16: np.ndarray, dt: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).view(TDT[dt]).to(DEV)


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u32_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(DEV)


def dev_to_u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def u8_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def out_bits_or_f32(t: torch.Tensor, dt: str) -> np.ndarray:
    """fp32 outputs as float32 arrays, 16-bit outputs as bit patterns (what oracle.round_f32_to returns)."""
    return t.cpu().numpy() if dt == "f32" else dev_to_bits(t)


def same_values(a: np.ndarray, b: np.ndarray) -> bool:
    """Bitwise equality of two float32 (or uint16 bit-pattern) arrays, treating all NaNs as equal."""
    if a.dtype == np.float32:
        na, nb = np.isnan(a), np.isnan(b)
        return bool(np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))
    return bool(np.array_equal(a, b))
