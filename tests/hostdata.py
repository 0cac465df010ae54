"""Host-side conversions between torch tensors and the oracle's numpy inputs."""
import numpy as np
import torch


def to_oracle(t):
    """torch tensor (any device) -> numpy array in the oracle's encoding:
    float32 stays float32, bfloat16 becomes its uint16 bit patterns."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.int32, torch.int64, torch.uint8):
        return t.numpy()
    raise TypeError(t.dtype)


def bf16_bits_to_f64(a):
    """uint16 bf16 bit patterns -> float64 values."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(a):
    """Round float32 to bf16 (nearest-even) and return uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)
