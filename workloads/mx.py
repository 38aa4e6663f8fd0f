"""OCP MX (block-scaled FP8, E4M3 elements) encoding of bf16 weights.

Input preparation for the low-precision expert-weight path: it turns the
seeded bf16 expert weights into E4M3 element codes and E8M0 scale codes.
It only encodes.  The oracle decodes the codes with its own code, and the
HIP path with the gfx950 scaled conversion instruction, so neither shares
arithmetic with the other through this module.

Encoding of one block of 32 consecutive values V along a row (OCP
Microscaling Formats specification v1.0, conversion from higher precision,
with the E4M3 element type):
  * amax = max |V|.  An all-zero block gets scale code 127 (2^0).
  * shared exponent = floor(log2(amax)) - 8 (8 is the largest E4M3 normal
    exponent), clamped to [-127, 127]; scale code = shared exponent + 127.
  * each element is V / 2^shared, rounded to the nearest E4M3 value (ties to
    even mantissa), magnitudes above 448 (the largest E4M3 normal) clamped
    to 448; the sign is kept, also for zero.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_EMAX = 8
E4M3_MAX = 448.0


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def encode_e4m3(y: np.ndarray) -> np.ndarray:
    """Round float64 values to E4M3 codes (ties to even, saturating at 448)."""
    y = np.asarray(y, np.float64)
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.minimum(np.abs(y), E4M3_MAX)
    code = np.zeros(a.shape, np.uint8)
    nz = a > 0
    _, ex = np.frexp(np.where(nz, a, 1.0))
    e = ex.astype(np.int64) - 1                   # a = 1.f x 2^e
    normal = nz & (e >= -6)
    # normals: 3 mantissa bits, a carry to the next binade when rounding up
    mant = np.where(normal, a / np.ldexp(1.0, np.where(normal, e, 0)), 1.0)
    m = np.rint((mant - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    ncode = ((e + 7) << 3) | m
    # subnormals: a = m x 2^-9, m in 0..8 (8 becomes the smallest normal, code 8)
    sm = np.rint(a * 512.0).astype(np.int64)
    code = np.where(normal, ncode, np.where(nz, sm, 0)).astype(np.uint8)
    return code | sign


def encode_mx(bits: np.ndarray):
    """bf16 bit patterns [..., K] (K a multiple of 32) -> (E4M3 codes
    [..., K] uint8, E8M0 scale codes [..., K/32] uint8)."""
    v = bf16_bits_to_f64(bits)
    shp = v.shape
    assert shp[-1] % BLOCK == 0
    blk = v.reshape(shp[:-1] + (shp[-1] // BLOCK, BLOCK))
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.clip(ex.astype(np.int64) - 1 - E4M3_EMAX, -127, 127)
    shared = np.where(amax > 0, shared, 0)
    scale_code = (shared + 127).astype(np.uint8)
    y = blk / np.ldexp(1.0, shared)[..., None]
    codes = encode_e4m3(y).reshape(shp)
    return codes, scale_code


def encode_mx_rows(bits: np.ndarray):
    """encode_mx over the leading axis in slices (threads, bounded memory):
    the same codes as encode_mx on the whole array."""
    from concurrent.futures import ThreadPoolExecutor

    from . import _threads
    bits = np.asarray(bits, np.uint16)
    if bits.ndim < 2 or bits.size <= (1 << 22):
        return encode_mx(bits)
    codes = np.empty(bits.shape, np.uint8)
    scales = np.empty(bits.shape[:-1] + (bits.shape[-1] // BLOCK,), np.uint8)

    def one(i):
        codes[i], scales[i] = encode_mx(bits[i])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(bits.shape[0])))
    return codes, scales


def mx_layer(layer: dict) -> dict:
    """The expert weights of a layer (w13, w2, ws13, ws2) in MX form, each as
    (codes, scale codes); other tensors are shared with the bf16 layer."""
    out = {}
    for name in ("w13", "w2", "ws13", "ws2"):
        w = layer.get(name)
        out[name] = None if w is None else encode_mx_rows(w)
    return out
