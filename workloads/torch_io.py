"""Moving workload arrays to and from device tensors (reinterpretation only).

Array conventions: float32 / float16 as themselves; uint16 holds bfloat16
bits (device dtype torch.bfloat16); uint8 holds E4M3FN codes (kept as uint8
on the device, which libpa's binding reads as fp8 E4M3FN).
"""

import numpy as np
import torch


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def widen_to_f64(t: torch.Tensor) -> np.ndarray:
    """A device output (float32 / float16 / bfloat16) as float64 values."""
    return t.detach().cpu().to(torch.float64).numpy()
