"""Small conversions between torch tensors and the oracle's numpy layouts
(bf16 as uint16 bit patterns, e4m3 as uint8 codes)."""
import numpy as np
import torch


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def f64(t) -> np.ndarray:
    """Exact fp64 values of a float tensor (bf16/fp32) or numpy array."""
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def e4m3_f64(codes) -> np.ndarray:
    """fp64 values of e4m3 codes through torch's float8_e4m3fn dtype."""
    c = torch.as_tensor(np.asarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()
