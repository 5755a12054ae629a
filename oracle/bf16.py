"""bf16 bit patterns -> float64, exactly (test infrastructure only).

A bf16 value is the top 16 bits of an IEEE binary32; shifting the pattern
left by 16 gives that binary32, which float64 holds exactly.
"""
import numpy as np


def widen(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
