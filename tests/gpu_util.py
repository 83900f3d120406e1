"""Helpers shared by the GPU tests (host-side marshalling only)."""
import numpy as np


def to_dev(bits: np.ndarray, device="cuda"):
    """bf16 bit patterns (numpy uint16) -> CUDA bfloat16 tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev_strided(bits: np.ndarray, ld: int, device="cuda"):
    """A row-strided view (leading dimension ld >= cols) holding bits."""
    import torch
    rows, cols = bits.shape
    buf = np.full((rows, ld), 0x7FC0, dtype=np.uint16)   # NaN padding: must never be read
    buf[:, :cols] = bits
    t = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).to(device)
    return t[:, :cols]


def host_u8(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.uint8)


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))
