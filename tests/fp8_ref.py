"""Independent reading of the FP8 block-scaled expert layout for the oracle's
pins: torch's float8_e4m3fn conversion decodes the codes; the 128 x 128 block
scales are expanded with numpy."""
import numpy as np
import torch


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def dequant_dense(codes: np.ndarray, bscales: np.ndarray) -> np.ndarray:
    """[E][out][in] weights: e4m3(code) * scale of the (out/128, in/128) block."""
    s = np.repeat(np.repeat(bscales.astype(np.float64), 128, axis=1), 128, axis=2)
    return e4m3_decode(codes) * s


def random_codes(rng, shape) -> np.ndarray:
    """Uniform E4M3 codes without the two NaN codes."""
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c
