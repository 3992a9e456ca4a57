"""Upload of stored inputs to GPU memory as torch tensors (plumbing only:
the bytes are passed through unchanged)."""
import numpy as np

from .gen import Tensor


def dev(t, device="cuda"):
    """Upload a stored input (a `Tensor` or a raw numpy array) as a torch
    tensor of the matching dtype: uint16 bf16 bits -> bfloat16, uint8 e4m3
    codes -> float8_e4m3fn, anything else as it is."""
    import torch
    raw = t.raw if isinstance(t, Tensor) else t
    if raw.dtype == np.uint16:
        return torch.from_numpy(raw.view(np.int16)).to(device).view(torch.bfloat16)
    if raw.dtype == np.uint8:
        return torch.from_numpy(raw).to(device).view(torch.float8_e4m3fn)
    return torch.from_numpy(np.ascontiguousarray(raw)).to(device)
