"""What an fp8 (E4M3FN) pool holds, computed with torch's float8_e4m3fn cast
and widening instead of the oracle's codec, so that the oracle's fp8 paths
can be pinned against a library routine (glossary page "PagedAttention",
related techniques: the 8-bit KV cache; one fp32 scale per pool, stored
code * scale = value)."""
import numpy as np
import torch


def codes(x: torch.Tensor, scale: float) -> np.ndarray:
    """E4M3FN codes of fp32(x) * fp32(1 / scale) by torch's cast (round to
    nearest even).  torch turns magnitudes past 464 into NaN where the cache
    saturates, so the scaled inputs must stay below that."""
    inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32)
    y = x.float() * inv
    assert float(y.abs().max()) < 464.0
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def dequant(x: torch.Tensor, scale: float) -> np.ndarray:
    """The value the pool holds for x: its code widened by torch, times the
    pool's fp32 scale (fp64; exact, as a code has 4 significant bits and the
    scale 24)."""
    c = torch.from_numpy(codes(x, scale)).view(torch.float8_e4m3fn)
    return c.to(torch.float64).numpy() * float(np.float32(scale))
