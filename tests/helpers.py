"""Test helpers: move stored numpy arrays (float32 / bf16 bit patterns) to and from the GPU."""
import numpy as np
import torch


def to_dev(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    if dtype == "bf16":
        a = np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16)
        return torch.from_numpy(a).to(device).view(torch.bfloat16)
    raise ValueError(dtype)


def from_dev(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float32:
        return t.detach().cpu().numpy()
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype in (torch.int64, torch.uint64):
        return t.detach().cpu().numpy().view(np.uint64)
    raise ValueError(t.dtype)


def bits_to_dev(words: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words, dtype=np.uint64).view(np.int64)).to(device)


def sdtype(t: torch.Tensor) -> str:
    return "f32" if t.dtype == torch.float32 else "bf16"


def ulp_distance(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """Distance in units in the last place between two stored arrays of one type."""
    if dtype == "f32":
        ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
        ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
        sign = np.int64(1) << 31
    else:
        ia = np.asarray(a, np.uint16).astype(np.int64)
        ib = np.asarray(b, np.uint16).astype(np.int64)
        sign = np.int64(1) << 15
    # map sign-magnitude encodings onto a monotone integer line
    ia = np.where(ia & sign, -(ia & (sign - 1)), ia & (sign - 1))
    ib = np.where(ib & sign, -(ib & (sign - 1)), ib & (sign - 1))
    return np.abs(ia - ib)


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(x, np.float64) - ref) / (den if den > 0 else 1.0))
