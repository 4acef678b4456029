"""Host-side helpers for the tests: bit-pattern views of torch tensors."""
import numpy as np
import torch


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits8(t: torch.Tensor) -> np.ndarray:
    """float8_e4m3fn tensor -> numpy uint8 codes (host copy)."""
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def from_bits16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def bf16_f64(a: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns with torch (a library routine, not the oracle)."""
    return from_bits16(a).double().numpy()


def e4m3_f64(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double().numpy()
