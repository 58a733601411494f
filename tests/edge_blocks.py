"""Adversarial weight blocks for parity tests (input generation only, no arithmetic of
the method).

Every code a block may hold is drawn: all 256 byte values, so Q8_0 meets -128 (byte
0x80) and Q4_0 every nibble. Scales are the binary16 edge values, each with both
signs (a negative scale flips every weight of its block):

  1.0 (0x3C00), the smallest subnormal 2^-24 (0x0001), the largest subnormal
  (0x03FF), the smallest normal 2^-14 (0x0400), an inexact third (0x3555), zero
  (0x0000 and 0x8000), and the largest scale the leg allows.

The largest scale: on the f32 leg 65504 (0x7BFF), whose products d*q are exact in f32.
On the f16 leg the weight is RNE_fp16(d*q) and must stay finite, |d*q| <= 65504:
Q4_0 codes give |q - 8| <= 8, so d = 8188 (0x6FFF, 8 * 8188 = 65504); Q8_0 codes give
|q| <= 128, so d = 511.75 (0x5FFF, 128 * 511.75 = 65504). Larger scales would turn
weights into infinities, which the f16 leg does not define.

Row r takes scale magnitude SCALES[r % len] in every block, so that each output
column measures one scale on its own (a row of mixed magnitudes is dominated by its
largest blocks in the normalised error); the rows past the first len(SCALES) * 2
mix magnitudes block by block. Signs are drawn per block.
"""
import numpy as np

from quantized_weight_prefill_gguf_amd import synth

COMMON = [0x3C00, 0x0001, 0x03FF, 0x0400, 0x3555, 0x0000]
TOP = {("f32", synth.Q4_0): 0x7BFF, ("f32", synth.Q8_0): 0x7BFF,
       ("f16", synth.Q4_0): 0x6FFF, ("f16", synth.Q8_0): 0x5FFF}


def scales(leg, qtype):
    """Scale magnitudes (binary16 bits, sign clear) for this leg and block type."""
    return COMMON + [TOP[(leg, qtype)]]


def weight(qtype, rows, k, leg, seed):
    """uint8 blocks [rows * (k/32) * block_bytes] of adversarial blocks."""
    B = synth.BLOCK_BYTES[qtype]
    nb = k // 32
    rng = np.random.default_rng([seed, 7, qtype])
    W = rng.integers(0, 256, size=(rows, nb, B), dtype=np.uint8)
    mags = np.array(scales(leg, qtype), np.uint16)
    L = len(mags)
    per_row = mags[np.arange(rows) % L][:, None] * np.ones((1, nb), np.uint16)
    mixed = np.arange(rows) >= 2 * L
    per_row[mixed] = mags[rng.integers(0, L, size=(int(mixed.sum()), nb))]
    sign = rng.integers(0, 2, size=(rows, nb)).astype(np.uint16) << 15
    d = (per_row | sign).astype(np.uint16)
    W[:, :, 0] = d & 0xFF
    W[:, :, 1] = d >> 8
    return W.reshape(-1)
