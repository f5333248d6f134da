"""Plain CPU definition of the block-quantized weight formats (numpy).

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this package.

Source: "Rockchip NPU sidecars" (audio.cpp docs), section "The talker is the
only DRAM-bound candidate": the Talker's matmuls ship as GGUF Q8_0 (32 int8
weights and one fp16 scale per block, 34 bytes) and re-quantized to Q4_K
they move 47% fewer bytes for 23% less time.  The pages name the formats
but not their rounding; the readings taken here (each listed in the design
notes):

* a block is 32 consecutive weights of one row (along the input dimension);
* int8 form: d = max|w| / 127, q = round(w / d) rounded half away from zero,
  clamped to [-127, 127], q = 0 when d = 0; the scale is stored as IEEE fp16
  (round to nearest even) and a weight reads back as fp16(d) * q;
* 4-bit form: the same with 7 in place of 127 (q in [-7, 7]), stored as the
  nibble q + 8, two weights per byte: weight 2i in the low nibble of byte i,
  weight 2i+1 in the high nibble.  18 bytes per 32 weights, the byte rate of
  Q4_K (144 bytes per 256).

The decisions (the code of each weight) are taken in float32 -- the division
w / d and the rounding -- the precision a GPU kernel takes them in.
"""

from __future__ import annotations

import numpy as np

BLOCK = 32
Q8, Q4 = "q8", "q4"
QMAX = {Q8: 127, Q4: 7}


def _round_half_away(v: np.ndarray) -> np.ndarray:
    """Nearest integer, halves away from zero, exact for float32 input (the
    fraction is computed exactly; no 'add 0.5' rounding step)."""
    a = np.abs(v)
    f = np.floor(a)
    r = np.where(a - f >= np.float32(0.5), f + 1, f)
    return np.copysign(r, v)


def block_scales(w: np.ndarray, fmt: str) -> np.ndarray:
    """float32 d per block: max |w| over the block / QMAX."""
    n, k = w.shape
    assert k % BLOCK == 0
    b = np.abs(np.asarray(w, np.float32)).reshape(n, k // BLOCK, BLOCK)
    return (b.max(axis=2) / np.float32(QMAX[fmt])).astype(np.float32)


def quantize(w: np.ndarray, fmt: str):
    """Quantize rows of w ([N, K] float32 values, K a multiple of 32).
    Returns (codes, scales): codes int8 [N, K] for Q8, uint8 [N, K/2] for Q4
    (nibbles q + 8, pairs as in the module notes); scales uint16 [N, K/32],
    the fp16 bit patterns of d."""
    w = np.asarray(w, np.float32)
    n, k = w.shape
    d = block_scales(w, fmt)
    dd = np.repeat(d, BLOCK, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (w / dd).astype(np.float32)
    q = np.where(dd > 0, _round_half_away(ratio), 0)
    q = np.clip(q, -QMAX[fmt], QMAX[fmt]).astype(np.int32)
    scales = d.astype(np.float16).view(np.uint16)
    if fmt == Q8:
        return q.astype(np.int8), scales
    nib = (q + 8).astype(np.uint8)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, scales


def codes_of(codes: np.ndarray, fmt: str, k: int) -> np.ndarray:
    """Signed codes q [N, K] from the stored form."""
    if fmt == Q8:
        return codes.astype(np.int32)
    lo = (codes & 0x0F).astype(np.int32) - 8
    hi = (codes >> 4).astype(np.int32) - 8
    q = np.empty((codes.shape[0], k), np.int32)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return q


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str, k: int) -> np.ndarray:
    """float64 [N, K] weights fp16(d) * q (exact: an 11-bit scale times a
    code of at most 8 bits)."""
    d = scales.view(np.float16).astype(np.float64)
    return codes_of(codes, fmt, k) * np.repeat(d, BLOCK, axis=1)


def bytes_per_weight(fmt: str) -> float:
    """Stored bytes per weight: codes plus one fp16 scale per block."""
    code_bits = 8 if fmt == Q8 else 4
    return (BLOCK * code_bits / 8 + 2) / BLOCK
