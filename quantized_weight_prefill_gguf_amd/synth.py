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

* F16: the weight rounded to binary16, little-endian, 32 values (64 bytes) per
  block.
* Q4_K / Q5_K (256 weights, 144 / 176 B): per 32-weight sub-block j, an affine
  code range from min(0, min w) to max w over 2^b - 1 steps (b = 4 or 5); the
  super-block's d and dmin are the largest sub-block step and offset over 63
  (binary16), the sub-block's 6-bit s_j, m_j their ratios to those (rounded), and
  q = clamp(round((w + dmin m_j) / (d s_j)), 0, 2^b - 1).
* Q6_K (256 weights, 210 B): per 16-weight sub-block a step amax / 31, d the
  largest step over 127 (binary16), sc_j = round(step / d) as int8, and
  q = clamp(round(w / (d sc_j)) + 32, 0, 63).
* IQ4_XS (256 weights, 136 B): per 32-weight sub-block a step amax / 127, d the
  largest step over 31 (binary16), the sub-block's 6-bit scale ls = 32 +
  round(step / d), and each weight's code the index of the nearest of the 16 grid
  values to w / (d (ls - 32)).
  These encoders are test-input generators, not llama.cpp's quantizers; any valid
  block serves the parity tests. Byte layouts: GGUF's, as the oracle restates them.

numpy's float32 -> float16 cast is IEEE round-to-nearest-even.
"""
import numpy as np

Q4_0, Q8_0, F16, Q4_K, Q5_K, Q6_K, IQ4_XS = 0, 1, 2, 3, 4, 5, 6
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, F16: 64, Q4_K: 144, Q5_K: 176, Q6_K: 210, IQ4_XS: 136}
BLOCK_ELEMS = {Q4_0: 32, Q8_0: 32, F16: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256, IQ4_XS: 256}
QTYPE_NAMES = {"q4_0": Q4_0, "q8_0": Q8_0, "f16": F16, "q4_k": Q4_K, "q5_k": Q5_K, "q6_k": Q6_K,
               "iq4_xs": IQ4_XS}

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


def quantize_f16(w):
    """f32 [rows][k] -> binary16 little-endian, uint8 [rows * k * 2]."""
    w = np.ascontiguousarray(w, np.float32)
    if w.shape[1] % 32:
        raise ValueError("k must be a multiple of 32")
    return w.astype(np.float16).view(np.uint8).reshape(-1).copy()


def _fp16_bits(v):
    return np.asarray(v, np.float32).astype(np.float16).view(np.uint16)


def pack_k_scales(s, m):
    """6-bit scales s and mins m [..., 8] -> the 12 packed bytes of a Q4_K / Q5_K
    super-block: sub-blocks 0-3 in the low 6 bits of bytes j (scale) and j + 4
    (min); sub-blocks 4-7 split into low nibbles (byte j + 4: scale low, min high)
    and top 2 bits (bits 6-7 of bytes j - 4 and j)."""
    s = np.asarray(s, np.uint8)
    m = np.asarray(m, np.uint8)
    out = np.zeros(s.shape[:-1] + (12,), np.uint8)
    for j in range(4):
        out[..., j] = (s[..., j] & 63) | ((s[..., j + 4] >> 4) << 6)
        out[..., j + 4] = (m[..., j] & 63) | ((m[..., j + 4] >> 4) << 6)
        out[..., j + 8] = (s[..., j + 4] & 15) | ((m[..., j + 4] & 15) << 4)
    return out


def _quantize_kaffine(w, bits):
    w = np.ascontiguousarray(w, np.float32)
    rows, k = w.shape
    if k % 256:
        raise ValueError("k must be a multiple of 256")
    nq = (1 << bits) - 1
    sb = w.reshape(rows, k // 256, 8, 32)
    lo = np.minimum(sb.min(axis=3), 0.0).astype(np.float32)
    hi = sb.max(axis=3).astype(np.float32)
    step = (hi - lo) / np.float32(nq)
    off = -lo
    d16 = _fp16_bits(step.max(axis=2) / np.float32(63))
    dm16 = _fp16_bits(off.max(axis=2) / np.float32(63))
    d = d16.view(np.float16).astype(np.float32)[..., None]
    dm = dm16.view(np.float16).astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sj = np.where(d > 0, np.clip(_round_half_away(step / np.where(d > 0, d, 1)), 0, 63), 0).astype(np.uint8)
        mj = np.where(dm > 0, np.clip(_round_half_away(off / np.where(dm > 0, dm, 1)), 0, 63), 0).astype(np.uint8)
        a = (d * sj.astype(np.float32))[..., None]
        b = (dm * mj.astype(np.float32))[..., None]
        q = np.where(a > 0, np.clip(_round_half_away((sb + b) / np.where(a > 0, a, 1)), 0, nq), 0).astype(np.uint8)
    return rows, k, d16, dm16, pack_k_scales(sj, mj), q.reshape(rows, k // 256, 256)


def quantize_q4_k(w):
    """f32 [rows][k] -> Q4_K super-blocks, uint8 [rows * (k/256) * 144]."""
    rows, k, d16, dm16, sc, q = _quantize_kaffine(w, 4)
    out = np.zeros((rows, k // 256, 144), np.uint8)
    out[..., 0:2] = d16[..., None].view(np.uint8).reshape(rows, k // 256, 2)
    out[..., 2:4] = dm16[..., None].view(np.uint8).reshape(rows, k // 256, 2)
    out[..., 4:16] = sc
    g = q.reshape(rows, k // 256, 4, 2, 32)     # [p][upper][l]
    out[..., 16:144] = (g[..., 0, :] | (g[..., 1, :] << 4)).reshape(rows, k // 256, 128)
    return out.reshape(-1)


def quantize_q5_k(w):
    """f32 [rows][k] -> Q5_K super-blocks, uint8 [rows * (k/256) * 176]."""
    rows, k, d16, dm16, sc, q = _quantize_kaffine(w, 5)
    out = np.zeros((rows, k // 256, 176), np.uint8)
    out[..., 0:2] = d16[..., None].view(np.uint8).reshape(rows, k // 256, 2)
    out[..., 2:4] = dm16[..., None].view(np.uint8).reshape(rows, k // 256, 2)
    out[..., 4:16] = sc
    hb = (q >> 4).reshape(rows, k // 256, 8, 32)  # element 32 b + l -> bit b of qh[l]
    qh = np.zeros((rows, k // 256, 32), np.uint8)
    for b in range(8):
        qh |= (hb[..., b, :] << b).astype(np.uint8)
    out[..., 16:48] = qh
    g = (q & 15).reshape(rows, k // 256, 4, 2, 32)
    out[..., 48:176] = (g[..., 0, :] | (g[..., 1, :] << 4)).reshape(rows, k // 256, 128)
    return out.reshape(-1)


def quantize_q6_k(w):
    """f32 [rows][k] -> Q6_K super-blocks, uint8 [rows * (k/256) * 210]."""
    w = np.ascontiguousarray(w, np.float32)
    rows, k = w.shape
    if k % 256:
        raise ValueError("k must be a multiple of 256")
    sb = w.reshape(rows, k // 256, 16, 16)
    step = (np.abs(sb).max(axis=3) / np.float32(31)).astype(np.float32)
    d16 = _fp16_bits(step.max(axis=2) / np.float32(127))
    d = d16.view(np.float16).astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d > 0, np.clip(_round_half_away(step / np.where(d > 0, d, 1)), -128, 127), 0).astype(np.int8)
        a = (d * sc.astype(np.float32))[..., None]
        q = np.where(a != 0, np.clip(_round_half_away(sb / np.where(a != 0, a, 1)) + 32, 0, 63), 32)
    q = q.astype(np.uint8).reshape(rows, k // 256, 2, 4, 32)   # [half][quarter][l]
    out = np.zeros((rows, k // 256, 210), np.uint8)
    ql = np.zeros((rows, k // 256, 2, 64), np.uint8)
    ql[..., 0:32] = (q[..., 0, :] & 15) | ((q[..., 2, :] & 15) << 4)
    ql[..., 32:64] = (q[..., 1, :] & 15) | ((q[..., 3, :] & 15) << 4)
    qh = ((q[..., 0, :] >> 4) | ((q[..., 1, :] >> 4) << 2) | ((q[..., 2, :] >> 4) << 4)
          | ((q[..., 3, :] >> 4) << 6)).astype(np.uint8)
    out[..., 0:128] = ql.reshape(rows, k // 256, 128)
    out[..., 128:192] = qh.reshape(rows, k // 256, 64)
    out[..., 192:208] = sc.view(np.uint8)
    out[..., 208:210] = d16[..., None].view(np.uint8).reshape(rows, k // 256, 2)
    return out.reshape(-1)


# The 16 values an IQ4_XS code selects (GGUF's IQ4_NL grid), in code order.
_IQ4_GRID = np.array([-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113],
                     np.float32)


def quantize_iq4_xs(w):
    """f32 [rows][k] -> IQ4_XS super-blocks, uint8 [rows * (k/256) * 136]."""
    w = np.ascontiguousarray(w, np.float32)
    rows, k = w.shape
    if k % 256:
        raise ValueError("k must be a multiple of 256")
    nsb = k // 256
    sb = w.reshape(rows, nsb, 8, 32)
    step = (np.abs(sb).max(axis=3) / np.float32(127)).astype(np.float32)
    d16 = _fp16_bits(step.max(axis=2) / np.float32(31))
    d = d16.view(np.float16).astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.where(d > 0, np.clip(_round_half_away(step / np.where(d > 0, d, 1)), 0, 31), 0)
    ls = (m + 32).astype(np.uint32)
    dl = (d * m.astype(np.float32))[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(dl > 0, sb / np.where(dl > 0, dl, 1), 0).astype(np.float32)
    mids = (_IQ4_GRID[1:] + _IQ4_GRID[:-1]) / 2
    code = np.searchsorted(mids, v).astype(np.uint8)          # [rows][nsb][8][32]
    out = np.zeros((rows, nsb, 136), np.uint8)
    out[..., 0:2] = d16[..., None].view(np.uint8).reshape(rows, nsb, 2)
    sh = np.zeros((rows, nsb), np.uint32)
    for b in range(8):
        sh |= ((ls[..., b] >> 4) & 3) << (2 * b)
    out[..., 2] = (sh & 0xFF).astype(np.uint8)
    out[..., 3] = (sh >> 8).astype(np.uint8)
    for i in range(4):
        out[..., 4 + i] = ((ls[..., 2 * i] & 15) | ((ls[..., 2 * i + 1] & 15) << 4)).astype(np.uint8)
    out[..., 8:136] = (code[..., 0:16] | (code[..., 16:32] << 4)).reshape(rows, nsb, 128)
    return out.reshape(-1)


QUANTIZERS = {Q4_0: quantize_q4_0, Q8_0: quantize_q8_0, F16: quantize_f16, Q4_K: quantize_q4_k,
              Q5_K: quantize_q5_k, Q6_K: quantize_q6_k, IQ4_XS: quantize_iq4_xs}


def quantize(qtype, w):
    return QUANTIZERS[qtype](w)


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
