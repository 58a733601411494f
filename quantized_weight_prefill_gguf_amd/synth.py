"""Seeded synthetic inputs: weights, activations, residuals and their GGUF encoding.

This module generates inputs only. It holds none of the method's arithmetic (no
block decode, no GEMM, no epilogue); both the GPU path and the CPU oracle consume
the bytes and arrays it returns.

Draws: ``numpy.random.default_rng([seed, workload_id, tensor_id])`` with
tensor ids W (or W_gate) = 0, W_up = 1, W_down = 2, X = 3, R = 4, row scale = 5.
Weights are float64 N(0, 0.02) cast to f32; X and R are f32 N(0, 1).

Quantizers (GGUF block formats, 32 elements per block, fp16 scale little-endian in
bytes 0-1):

* Q8_0 (34 B): d16 = RNE_fp16(amax / 127) with the division in f32,
  q = clamp(round_half_away(w / d16), -127, 127) as int8 in bytes 2-33.
* Q4_0 (18 B): m = the element of largest magnitude (first on ties),
  d16 = RNE_fp16(m / -8), q = clamp(round_half_away(w / d16) + 8, 0, 15);
  element j < 16 is the low nibble of byte 2+j, element j >= 16 the high nibble of
  byte 2+(j-16).
* An all-zero block gets d16 = +0 and q = 0 (Q8_0) or 8 (Q4_0).

numpy's float32 -> float16 cast is IEEE round-to-nearest-even.
"""
import numpy as np

Q4_0, Q8_0 = 0, 1
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34}
QTYPE_NAMES = {"q4_0": Q4_0, "q8_0": Q8_0}

TENSOR_W, TENSOR_W_UP, TENSOR_W_DOWN, TENSOR_X, TENSOR_R, TENSOR_ROWSCALE = range(6)


def rng_for(seed, workload_id, tensor_id):
    return np.random.default_rng([seed, workload_id, tensor_id])


def weights_f32(rows, k, seed=0, workload_id=0, tensor_id=TENSOR_W, std=0.02):
    """f32 [rows][k] drawn as float64 N(0, std) then cast."""
    g = rng_for(seed, workload_id, tensor_id)
    return g.normal(0.0, std, size=(rows, k)).astype(np.float32)


def activations(T, k, seed=0, workload_id=0, tensor_id=TENSOR_X, row_scale=False):
    """f32 [T][k] N(0, 1); with row_scale each row is multiplied by s_t ~ U[0.5, 2]."""
    g = rng_for(seed, workload_id, tensor_id)
    X = g.standard_normal(size=(T, k), dtype=np.float32)
    if row_scale:
        s = rng_for(seed, workload_id, TENSOR_ROWSCALE).uniform(0.5, 2.0, size=T)
        X = (X * s.astype(np.float32)[:, None]).astype(np.float32)
    return X


def _round_half_away(v):
    # v is exactly representable in float64; |v| + 0.5 is exact there.
    v = v.astype(np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def quantize_q8_0(w):
    """f32 [rows][k] -> Q8_0 blocks as uint8 [rows * (k/32) * 34]."""
    w = np.ascontiguousarray(w, np.float32)
    rows, k = w.shape
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    blk = w.reshape(rows, k // 32, 32)
    amax = np.max(np.abs(blk), axis=2)
    d32 = (amax / np.float32(127.0)).astype(np.float32)
    d16 = d32.astype(np.float16)
    zero = amax == 0
    d16 = np.where(zero, np.float16(0.0), d16)
    dd = d16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(zero[..., None], np.float32(0.0), blk / np.where(dd == 0, np.float32(1), dd))
    q = np.clip(_round_half_away(v.astype(np.float32)), -127, 127).astype(np.int8)
    out = np.empty((rows, k // 32, 34), np.uint8)
    out[..., 0:2] = d16.view(np.uint16)[..., None].view(np.uint8).reshape(rows, k // 32, 2)
    out[..., 2:] = q.view(np.uint8)
    return out.reshape(-1)


def quantize_q4_0(w):
    """f32 [rows][k] -> Q4_0 blocks as uint8 [rows * (k/32) * 18]."""
    w = np.ascontiguousarray(w, np.float32)
    rows, k = w.shape
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    blk = w.reshape(rows, k // 32, 32)
    idx = np.argmax(np.abs(blk), axis=2)  # first index on ties
    m = np.take_along_axis(blk, idx[..., None], axis=2)[..., 0]
    d32 = (m / np.float32(-8.0)).astype(np.float32)
    d16 = d32.astype(np.float16)
    zero = m == 0
    d16 = np.where(zero, np.float16(0.0), d16)
    dd = d16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(zero[..., None], np.float32(0.0), blk / np.where(dd == 0, np.float32(1), dd))
    q = np.clip(_round_half_away(v.astype(np.float32)) + 8, 0, 15).astype(np.uint8)
    q = np.where(zero[..., None], np.uint8(8), q)
    out = np.empty((rows, k // 32, 18), np.uint8)
    out[..., 0:2] = d16.view(np.uint16)[..., None].view(np.uint8).reshape(rows, k // 32, 2)
    out[..., 2:] = (q[..., :16] | (q[..., 16:] << 4)).astype(np.uint8)
    return out.reshape(-1)


def quantize(qtype, w):
    return quantize_q4_0(w) if qtype == Q4_0 else quantize_q8_0(w)


def quantized_weight(qtype, rows, k, seed=0, workload_id=0, tensor_id=TENSOR_W):
    """Blocks of an N(0, 0.02) [rows][k] weight."""
    return quantize(qtype, weights_f32(rows, k, seed, workload_id, tensor_id))


def gate_up_weight(qtype, n, k, seed=0, workload_id=0):
    """One buffer of 2n rows: the gate weight's n rows, then the up weight's."""
    g = quantized_weight(qtype, n, k, seed, workload_id, TENSOR_W)
    u = quantized_weight(qtype, n, k, seed, workload_id, TENSOR_W_UP)
    return np.concatenate([g, u])


def zero_q4_0(rows, k):
    """All-zero Q4_0 weight: scale 1.0 (0x3C00) and every nibble 8."""
    out = np.empty((rows, k // 32, 18), np.uint8)
    out[..., 0] = 0x00
    out[..., 1] = 0x3C
    out[..., 2:] = 0x88
    return out.reshape(-1)
