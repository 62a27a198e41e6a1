"""Oracle: an 8-bit floating-point (E4M3) KV cache, written plainly.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

The pages only name the option: "10 Serving Engines" lists a KV-cache
precision flag (``--kv-cache-dtype``) that takes effect where the engine and
its kernels support it.  They fix no format, rounding or scale, so every
step below is a reading (parity partly unpinned by the pages):

* Format: OCP 8-bit E4M3 ("e4m3fn") -- sign, 4 exponent bits (bias 7), 3
  mantissa bits; exponent field 0 is subnormal (value m/8 * 2^-6); no
  infinities; S.1111.111 is NaN, so the largest finite magnitude is
  1.75 * 2^8 = 448.
* Scale: one float per cache (k_scale, v_scale), chosen by the caller.  The
  stored code of an element x is E4M3(x * (1/scale)), the product taken in
  float32 (the precision the kernel decides the code in), rounded to the
  nearest E4M3 value with ties to an even mantissa, and saturated to +-448.
  The attention reads code * scale.
* Everything else (layout, slots, block tables, the attention itself) is as
  for the 16/32-bit caches: one byte per element instead of two or four.
"""

import math

import numpy as np

from oracle.attention import attend, to_f64

E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of one E4M3 code (0..255) as a Python float; NaN for S.1111.111.

    OCP E4M3: e = bits 6..3, m = bits 2..0; e == 0 -> (m / 8) * 2^-6,
    otherwise (1 + m / 8) * 2^(e - 7).
    """
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_encode(v):
    """E4M3 code of a float (already scaled): saturate to +-448, then round
    to the nearest representable value, ties to an even mantissa.

    Below 2^-6 the grid is the subnormal step 2^-9 (code = multiples of the
    step; 8 steps = 2^-6 is the smallest normal code, 0x08).  From 2^-6 up,
    a binade [2^e, 2^(e+1)) holds 8 values 2^(e-3) apart; rounding up out of
    the binade gives the first value of the next.  Python's round() rounds
    halves to even, and every division here is by a power of two (exact).
    """
    v = float(v)
    if v != v:
        return 0x7F
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = min(abs(v), E4M3_MAX)
    if a < 2.0 ** -6:
        return sign | int(round(a / 2.0 ** -9))
    frac, exp2 = math.frexp(a)          # a = frac * 2^exp2, frac in [0.5, 1)
    e = exp2 - 1                        # a in [2^e, 2^(e+1))
    n = int(round(a / 2.0 ** (e - 3)))  # 8 .. 16
    if n == 16:
        e, n = e + 1, 8
    return sign | ((e + 7) << 3) | (n - 8)


def quantize(x, inv_scale):
    """Codes (uint8 array) of float32 values x scaled by inv_scale: the
    product is rounded to float32 first, as the kernel computes it."""
    prod = np.asarray(x, dtype=np.float32) * np.float32(inv_scale)
    flat = [e4m3_encode(float(p)) for p in prod.ravel()]
    return np.asarray(flat, dtype=np.uint8).reshape(prod.shape)


def dequantize(codes, scale):
    """float64 values code * scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[codes] * float(scale)


def store_kv(k_cache, v_cache, k, v, slot_mapping, k_inv_scale, v_inv_scale,
             src_dtype):
    """Quantise new K/V rows and scatter them (copies of the code caches).

    As ``attention.store_kv`` (ModelRunner page, sections 2 and 5: row t goes
    to flat slot slot_mapping[t], a negative slot writes nothing), with each
    element stored as its E4M3 code.  k, v: [T, Hkv, D] of ``src_dtype``
    (bf16 bits or float32); the caches: uint8 [NB, bs, Hkv, D].  A slot
    past the cache is a precondition violation and raises IndexError, as in
    ``attention.store_kv``.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    num_blocks, bs = k_out.shape[0], k_out.shape[1]
    k32 = to_f64(k, src_dtype).astype(np.float32)   # exact: inputs are f32/bf16
    v32 = to_f64(v, src_dtype).astype(np.float32)
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        if slot >= num_blocks * bs:
            raise IndexError(f"slot {slot} outside the cache")
        k_out[slot // bs, slot % bs] = quantize(k32[t], k_inv_scale)
        v_out[slot // bs, slot % bs] = quantize(v32[t], v_inv_scale)
    return k_out, v_out


def decode_attention(q, k_codes, v_codes, block_tables, context_lens, scale,
                     k_scale, v_scale, q_dtype, seqs=None):
    """Decode attention over an E4M3 cache: the same definition as
    ``attention.decode_attention`` with K = code * k_scale and V = code *
    v_scale (gathered through the block table, Warmup Guide Chapter 3)."""
    q64 = to_f64(q, q_dtype)
    b_count, hq, d = q64.shape
    bs, hkv = k_codes.shape[1], k_codes.shape[2]
    group = hq // hkv
    out = np.zeros((b_count, hq, d), dtype=np.float64)
    for b in (range(b_count) if seqs is None else seqs):
        length = int(context_lens[b])
        if length == 0:
            continue
        kc = np.empty((length, hkv, d), dtype=np.uint8)
        vc = np.empty((length, hkv, d), dtype=np.uint8)
        for t in range(length):
            blk = int(block_tables[b][t // bs])
            if blk < 0 or blk >= k_codes.shape[0]:
                raise IndexError(f"block id {blk} outside the pool")
            kc[t] = k_codes[blk, t % bs]
            vc[t] = v_codes[blk, t % bs]
        keys = dequantize(kc, k_scale)
        values = dequantize(vc, v_scale)
        for h in range(hq):
            g = h // group
            o, _ = attend(q64[b, h][None, :], keys[:, g, :], values[:, g, :],
                          scale, [length])
            out[b, h] = o[0]
    return out
