"""OCP 8-bit floating point, E4M3 encoding: decoding (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The key cache of the fp8 variant stores each key element as one byte in the
E4M3 encoding of the OCP 8-bit floating point specification (OFP8, v1.0):
bit 7 is the sign, bits 6..3 the exponent field E (bias 7), bits 2..0 the
mantissa field M.

* E = 0: subnormal, value (M / 8) * 2^-6 (so M = 0 is a signed zero);
* 1 <= E <= 15: normal, value (1 + M / 8) * 2^(E - 7);
* E = 15 and M = 7: NaN (this encoding has no infinities), so the largest
  finite magnitude is (1 + 6/8) * 2^8 = 448.

The caller's cache stores K = k_scale[b, h_kv] * decode(K8) with one fp32
scale per (sequence, KV head); the oracle decodes every byte exactly into fp64
and multiplies by that scale.
"""

import numpy as np


def e4m3_value(code):
    """Exact value of one E4M3 byte (float; NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# value of every code, in code order
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode(codes):
    """fp64 values of an array of E4M3 bytes (any integer dtype, same shape)."""
    return E4M3_TABLE[np.asarray(codes).astype(np.uint8)]


def dequantize(K8, k_scale):
    """K = k_scale[b, h_kv] * decode(K8[b, h_kv, j, i]) in fp64.

    K8: (B, H_kv, max_n_k, d) bytes; k_scale: (B, H_kv) fp32.
    """
    return decode(K8) * np.asarray(k_scale, dtype=np.float64)[:, :, None, None]
