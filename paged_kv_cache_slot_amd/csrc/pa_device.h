// Device helpers shared by the gfx950 kernels of libpa.
//
// Element types: float, and bfloat16 carried as its raw 16 bits (uint16_t).
// A bfloat16 is the high half of a float32, so widening is a shift; packed
// pairs of bfloat16 in one dword feed v_dot2_f32_bf16 directly.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<float> {
  static constexpr int kBytes = 4;
};
template <>
struct ElemTraits<bf16_t> {
  static constexpr int kBytes = 2;
};

// Low / high bfloat16 of a packed dword, widened exactly to float.
__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bfloat16 pair (low = lo), round to nearest even, one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Pack the low (high) bfloat16 halves of two dwords: result low half from
// x, high half from y.
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// dot of two packed bfloat16 pairs, accumulated in float (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc,
                                         false);
}

// DPP quad permutations: lane i of each group of 4 reads lane perm[i].
// Control byte = sel0 | sel1 << 2 | sel2 << 4 | sel3 << 6.
constexpr int kQuadSwap1 = 0xB1;  // [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7 - i in each 8 lanes
constexpr int kRowMirror = 0x140;      // lane i <-> 15 - i in each 16 lanes

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}

// Sum over the 4 lanes of a quad; every lane of the quad gets the total.
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp_f32<kQuadSwap1>(x);
  x += dpp_f32<kQuadSwap2>(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// 2^x (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// float <-> IEEE binary16 bits (v_cvt_f16_f32 rounds to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Partial results of a split (partitioned) attention row with bfloat16 I/O
// are stored normalised, o = acc / l, as binary16: half the bytes of fp32,
// and interleaved partial writes slow the K/V read stream far beyond their
// own size.  A partial with |o| >= 2^15 somewhere is stored as o * 2^-16
// and flagged by storing its sum l negated; the merge undoes both.
constexpr float kPartialBig = 32768.f;
constexpr float kPartialShrink = 1.f / 65536.f;
constexpr float kPartialGrow = 65536.f;
constexpr float kHalfMax = 65504.f;

__device__ __forceinline__ uint16_t partial_f16(float o, bool big) {
  const float v = big ? o * kPartialShrink : o;
  return f32_to_f16(fminf(fmaxf(v, -kHalfMax), kHalfMax));
}

// Log-sum-exp merge of n partial results of one output element.  Partial
// k has a reference max m_k (base-2 logits), a sum l_k and an unnormalised
// output a_k; the result is sum_k 2^(m_k - m) a_k / sum_k 2^(m_k - m) l_k
// with m the largest m_k, or 0 when no partial saw a key.  load(k, m, l, a)
// fetches partial k.  The loads of a group of kGroup partials are issued
// together (one memory round trip per group): slots past n load partial
// n - 1 again, unconditionally, and are then masked out.  The group's max
// becomes the reference, rescaling what earlier groups summed.  With
// n <= kGroup this is the plain two-pass merge: max over all, then
// weighted sums.  (m, l, o) may start as a partial already in registers.
template <int kGroup, typename LoadFn>
__device__ __forceinline__ float merge_partials(int n, LoadFn load,
                                                float m = -INFINITY,
                                                float l = 0.f, float o = 0.f) {
  for (int i0 = 0; i0 < n; i0 += kGroup) {
    float mv[kGroup], sv[kGroup], av[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const bool in = i0 + u < n;
      load(in ? i0 + u : n - 1, mv[u], sv[u], av[u]);
      mv[u] = in ? mv[u] : -INFINITY;
      sv[u] = in ? sv[u] : 0.f;
      av[u] = in ? av[u] : 0.f;
    }
    float gm = m;
#pragma unroll
    for (int u = 0; u < kGroup; ++u) gm = fmaxf(gm, mv[u]);
    if (gm == -INFINITY) continue;          // nothing visible yet
    if (gm > m) {
      const float a = m == -INFINITY ? 0.f : fast_exp2(m - gm);
      l *= a;
      o *= a;
      m = gm;
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      if (i0 + u < n) {
        const float w = fast_exp2(mv[u] - m);
        l = fmaf(w, sv[u], l);
        o = fmaf(w, av[u], o);
      }
    }
  }
  return (m == -INFINITY || !(l > 0.f)) ? 0.f : o / l;
}

// Two E4M3 codes (bytes 0-1, or 2-3 with kHigh, of w) -> two bfloat16, and
// eight codes (bytes of lo, then hi) -> eight bfloat16 (exact; E4M3 values
// are a subset of bfloat16's).
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  return make_uint4(e4m3x2_to_bf16<false>(lo), e4m3x2_to_bf16<true>(lo),
                    e4m3x2_to_bf16<false>(hi), e4m3x2_to_bf16<true>(hi));
}

// 16-byte global load / store.
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
// 16-byte load marked non-temporal: streamed data used once.
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// Word 3 of a raw (unswizzled, untyped) gfx9 buffer resource.
constexpr int kBufferRsrcWord3 = 0x00020000;
// Cache-policy bits of a buffer load: non-temporal (streamed, used once).
constexpr int kCacheNT = 2;

// A bounds-checked view of one cache block: a buffer resource whose size is
// the bytes of the block's valid tokens.  Loads past that size return zeros
// without touching memory, so a block past the context, a block id outside
// the pool and the slots past the context of a partial block all read as
// zero, and every load instruction can be issued unconditionally.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const char* base,
                                                            int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes,
                                           kBufferRsrcWord3);
}
__device__ __forceinline__ uint4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r,
                                             uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCacheNT);
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace pa
