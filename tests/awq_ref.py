"""An independent numpy reading of the AWQ W4A16 g32 GEMM layout, used by the
tests to pack known integer codes and to unpack whole tensors at once.

Layout (AWQ-g32 card, "Checkpoint": asymmetric W4A16, group size 32, integer
zero point, GEMM packing; the nibble order within a word is the commonly
documented GEMM interleave and is a reading, not stated on the pages):
    qweight [E][in][out/8] int32   nibble j of word c = code of column 8c + PERM[j]
    qzeros  [E][in/32][out/8] int32 same nibble order, one zero per (group, column)
    scales  [E][in/32][out] fp16
    w[e][o][i] = (code - zero) * scale
"""
import numpy as np

PERM = np.array([0, 2, 4, 6, 1, 3, 5, 7])


def pack_nibbles(vals: np.ndarray) -> np.ndarray:
    """[..., out] integers 0..15 -> [..., out/8] int32 words."""
    *lead, out = vals.shape
    v = vals.reshape(*lead, out // 8, 8).astype(np.uint64)
    word = np.zeros((*lead, out // 8), np.uint64)
    for j in range(8):
        word |= v[..., PERM[j]] << np.uint64(4 * j)
    return word.astype(np.uint32).view(np.int32)


def unpack_nibbles(words: np.ndarray) -> np.ndarray:
    """[..., out/8] int32 words -> [..., out] integers 0..15."""
    w = np.asarray(words).view(np.uint32).astype(np.uint64)
    *lead, n8 = w.shape
    out = np.zeros((*lead, n8, 8), np.int64)
    for j in range(8):
        out[..., PERM[j]] = (w >> np.uint64(4 * j)) & np.uint64(15)
    return out.reshape(*lead, n8 * 8)


def dequant_dense(qweight, qzeros, scales) -> np.ndarray:
    """Whole projection as dense fp64 [E][out][in]."""
    q = unpack_nibbles(qweight)                       # [E][in][out]
    z = np.repeat(unpack_nibbles(qzeros), 32, axis=1)  # [E][in][out]
    s = np.repeat(np.asarray(scales, np.uint16).view(np.float16).astype(np.float64), 32, axis=1)
    return np.transpose((q - z) * s, (0, 2, 1))


def to_output_major(qweight: np.ndarray) -> np.ndarray:
    """AWQ codes [E][in][out/8] -> the same codes output-major [E][out][in/8]:
    word w of output column o holds inputs 8w..8w+7, input 8w + j in nibble j."""
    q = unpack_nibbles(qweight)                       # [E][in][out]
    E, I, O = q.shape
    qt = np.transpose(q, (0, 2, 1)).reshape(E, O, I // 8, 8).astype(np.uint64)
    word = np.zeros((E, O, I // 8), np.uint64)
    for j in range(8):
        word |= qt[..., j] << np.uint64(4 * j)
    return word.astype(np.uint32).view(np.int32)
