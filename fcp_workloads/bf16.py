"""bfloat16 encoding of float32 draws (round to nearest, ties to even) and exact widening."""
import numpy as np


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even.

    Inputs are finite N(0,1) draws; NaN/Inf inputs are not expected and not special-cased.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (exact)."""
    return bf16_bits_to_f32(b).astype(np.float64)
