"""Helpers shared by the tests: storage views for the oracle and error metrics."""
import numpy as np
import torch


def np_storage(t: torch.Tensor) -> np.ndarray:
    """A stored tensor as the oracle reads it: float32, bf16 bits (uint16), E4M3 codes or packed
    E2M1 codes (uint8)."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.float32, torch.uint8):
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def exact64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a stored float tensor (fp32, bf16 and E4M3 all embed in fp64)."""
    return t.detach().cpu().to(torch.float64).numpy()


def rel_err(got, ref) -> float:
    """max |got - ref| / RMS(ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)
