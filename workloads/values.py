"""Seeded tensor values: N(0, 1) normals, optionally rounded to bfloat16.

Values are drawn with a ``torch.Generator`` seeded explicitly, on the device
the tensor lives on (the CPU for small checks, the GPU for full-size pools so
that gigabytes of inputs take a second rather than minutes).  The oracle never
re-derives values from a seed: it reads a host copy of the very tensors the
kernels read.
"""

import torch

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(dtype):
    return _TORCH_DTYPE[dtype]


def _generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_values(shape, dtype, seed, device="cpu", chunk_elems=1 << 28):
    """A tensor of N(0,1) values of the given element type ("f32"/"bf16").

    Drawn in float32 and cast (round to nearest even for bfloat16), in chunks
    along the first dimension so the float32 staging stays bounded.
    """
    out = torch.empty(shape, dtype=_TORCH_DTYPE[dtype], device=device)
    g = _generator(seed, device)
    flat = out.view(-1)
    n = flat.numel()
    pos = 0
    while pos < n:
        m = min(chunk_elems, n - pos)
        flat[pos:pos + m] = torch.randn(m, generator=g, device=device,
                                        dtype=torch.float32).to(out.dtype)
        pos += m
    return out


def fill_pool(num_blocks, block_size, num_kv_heads, head_dim, dtype, seed,
              device="cpu"):
    """K and V caches [num_blocks, block_size, Hkv, D], every slot N(0,1)."""
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    k = make_values(shape, dtype, seed, device)
    v = make_values(shape, dtype, seed + 7919, device)
    return k, v


def make_codes(shape, seed, device="cpu", chunk_elems=1 << 26):
    """A uint8 tensor of 8-bit float (E4M3) codes for a synthetic 8-bit
    cache: random sign and mantissa, the 4-bit exponent field drawn around
    the field value 7 (magnitudes near 1, spread over a few binades), and no
    NaN code (field 15 with mantissa 7 becomes mantissa 6).  Bit fields
    only -- no rounding or scaling is done here.  Drawn on ``device`` in
    chunks."""
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    g = _generator(seed, device)
    flat = out.view(-1)
    n = flat.numel()
    pos = 0
    while pos < n:
        m = min(chunk_elems, n - pos)
        sign = torch.randint(0, 2, (m,), generator=g, device=device,
                             dtype=torch.int32)
        exp = (torch.randn(m, generator=g, device=device) * 1.5 + 6.5) \
            .round().clamp(0, 15).to(torch.int32)
        man = torch.randint(0, 8, (m,), generator=g, device=device,
                            dtype=torch.int32)
        man = torch.where((exp == 15) & (man == 7), torch.full_like(man, 6), man)
        flat[pos:pos + m] = ((sign << 7) | (exp << 3) | man).to(torch.uint8)
        pos += m
    return out


def fill_pool_codes(num_blocks, block_size, num_kv_heads, head_dim, seed,
                    device="cpu"):
    """8-bit (E4M3 code) K and V caches [num_blocks, block_size, Hkv, D]."""
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    return (make_codes(shape, seed, device),
            make_codes(shape, seed + 7919, device))


def poison_unused(k_cache, v_cache, valid_mask):
    """Overwrite every (block, offset) that no sequence keeps with NaN, so a
    kernel that reads outside a context -- or masks by multiplying with zero
    -- shows NaN in its output.  ``valid_mask`` is a bool array
    [num_blocks, block_size] (numpy or torch)."""
    mask = torch.as_tensor(valid_mask, device=k_cache.device)
    bad = ~mask
    k_cache[bad] = float("nan")
    v_cache[bad] = float("nan")
    return k_cache, v_cache


def host_bits(t):
    """Host numpy copy of a tensor's raw element bits: uint16 for bfloat16,
    float32 for float32 (the form the oracle reads)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")
