"""FP8 KV cache: E4M3 codes and the cache write / decode over them (oracle;
test infrastructure only).

The pages do not define a quantised cache; they only note that decode is
bound by the bytes moved ("vLLM Architecture, Memory and Benchmarks Deep
Dive", section 1: a memory-bandwidth problem) and that the cache size scales
with the bytes per element b in M_KV = 2*L*H_KV*d_head*T*b ("Optimizing LLM
Inference", KV-cache section). The format is therefore a stated choice:

* OCP E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 holds subnormals (m * 2^-9); no infinities; 0x7F and 0xFF
  are NaN; the largest finite magnitude is 1.75 * 2^8 = 448.
* Encoding rounds to nearest with ties to even; magnitudes beyond 448
  saturate to +-448; NaN encodes as 0x7F.
* One scale per pool and call: the stored code of x is encode(fp32(x) /
  fp32(scale)), the quotient rounded to fp32 as the kernel computes it
  (the quotient decides an integer code, so both sides form it in the same
  precision); the cache then holds decode(code) * scale.
* Pool layouts: the key pool is [num_blocks][H_KV][block_size][d] like the
  BF16 pools; the value pool stores each block transposed,
  [num_blocks][H_KV][d][block_size] (the token index fastest), so that the
  tokens of one channel are adjacent. The block table and the slot of a
  token (block * block_size + offset) mean the same for both.
"""

import numpy as np

from . import attention

E4M3_MAX = 448.0


def decode_e4m3(codes):
    """float64 values of E4M3FN codes (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def encode_e4m3(values):
    """E4M3FN codes (uint8) of float values: round to nearest even,
    saturate beyond 448, NaN -> 0x7F."""
    v = np.asarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    flat_v, flat_o = v.reshape(-1), out.reshape(-1)
    for i, x in enumerate(flat_v.tolist()):
        if x != x:
            flat_o[i] = 0x7F
            continue
        s = 0x80 if np.signbit(x) else 0
        a = abs(x)
        if a >= E4M3_MAX:
            flat_o[i] = s | 0x7E
            continue
        if a < 2.0 ** -6:                       # subnormal range: steps of 2^-9
            m = int(np.rint(a / 2.0 ** -9))     # exact quotient, ties to even
            flat_o[i] = s | m                   # m == 8 is the smallest normal, 0x08
            continue
        e = int(np.floor(np.log2(a)))
        if 2.0 ** e > a:                        # guard the log2 rounding
            e -= 1
        elif 2.0 ** (e + 1) <= a:
            e += 1
        m = int(np.rint((a / 2.0 ** e - 1.0) * 8.0))
        if m == 8:                              # rounded up to the next power of two
            e, m = e + 1, 0
        if e + 7 > 15 or (e + 7 == 15 and m == 7):
            flat_o[i] = s | 0x7E                # rounding reached past 448
            continue
        flat_o[i] = s | ((e + 7) << 3) | m
    return out


def quantize(x, scale):
    """Codes of x under a pool scale: encode(fp32(x) / fp32(scale))."""
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return encode_e4m3(q.astype(np.float64))


def dequantize(codes, scale):
    return decode_e4m3(codes) * float(np.float32(scale))


def value_rows(value_codes):
    """A value code pool in the key pools' row layout [nb][H][bs][d]."""
    return np.ascontiguousarray(np.swapaxes(value_codes, 2, 3))


def value_pool(rows):
    """Inverse of value_rows: [nb][H][bs][d] rows to the value pool layout."""
    return np.ascontiguousarray(np.swapaxes(rows, 2, 3))


def cache_write(key_codes, value_codes, key, value, slot_mapping, block_size, k_scale, v_scale):
    """The slot-mapped write of attention.cache_write, storing the codes of
    key / k_scale and value / v_scale in copies of the two code pools (the
    value pool in its transposed block layout)."""
    kc, vr = attention.cache_write(key_codes, value_rows(value_codes), quantize(key, k_scale),
                                   quantize(value, v_scale), slot_mapping, block_size)
    return kc, value_pool(vr)


def decode(query, key_codes, value_codes, block_tables, context_lens, block_size, scale, k_scale,
           v_scale):
    """Decode attention over the dequantised cache (attention.decode)."""
    return attention.decode(query, dequantize(key_codes, k_scale),
                            dequantize(value_rows(value_codes), v_scale), block_tables,
                            context_lens, block_size, scale)


def decode_partitions(query, key_codes, value_codes, block_tables, context_lens, block_size,
                      scale, k_scale, v_scale, partition_size, seqs=None, heads=None):
    """attention.decode_partitions over the dequantised cache."""
    return attention.decode_partitions(query, dequantize(key_codes, k_scale),
                                       dequantize(value_rows(value_codes), v_scale), block_tables,
                                       context_lens, block_size, scale, partition_size,
                                       seqs=seqs, heads=heads)
