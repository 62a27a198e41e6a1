// store_kv: scatter new K/V rows into their physical cache slots.
//
// Row t of k and of v (num_kv_heads * head_dim elements, row_bytes bytes) is
// copied whole to flat slot slot_mapping[t]; a negative slot is batch padding
// and writes nothing ("3.6 ModelRunner, CUDA Graph, and benchmarks", sections
// 2 and 5).  Pure data movement: HBM-bound at 2 * row_bytes read + written
// per row, or launch-bound for the few hundred rows of one decode step.
//
// Mapping: the flat space of (row, 16-byte vector) is covered by threads,
// consecutive threads on consecutive 16-byte vectors of a row, so every wave
// reads and writes whole contiguous rows (coalesced on both sides even though
// destination rows are scattered).  Each thread moves one vector of K and the
// same vector of V.  Addresses are 64-bit: a cache pool exceeds 2^31 bytes.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void store_kv_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int64_t num_tokens,
    int64_t vecs_per_row, int64_t num_slots) {
  const int64_t total = num_tokens * vecs_per_row;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x +
                   threadIdx.x;
       i < total; i += stride) {
    const int64_t t = i / vecs_per_row;
    const int64_t e = i - t * vecs_per_row;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    const uint4 kv = k[i];
    const uint4 vv = v[i];
    k_cache[slot * vecs_per_row + e] = kv;
    v_cache[slot * vecs_per_row + e] = vv;
  }
}

hipError_t launch_store_kv(const void* k, const void* v, void* k_cache,
                           void* v_cache, const int32_t* slot_mapping,
                           int64_t num_tokens, int64_t row_bytes,
                           int64_t num_slots, hipStream_t stream) {
  const int64_t vecs = row_bytes / 16;
  const int64_t total = num_tokens * vecs;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  // Enough waves to cover the chip several times over; beyond that the
  // grid-stride loop takes the rest.
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(store_kv_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(threads), 0, stream,
                     reinterpret_cast<const uint4*>(k),
                     reinterpret_cast<const uint4*>(v),
                     reinterpret_cast<uint4*>(k_cache),
                     reinterpret_cast<uint4*>(v_cache), slot_mapping,
                     num_tokens, vecs, num_slots);
  return hipGetLastError();
}

// Quantising store (E4M3 cache).  The pages only name a cache-precision
// option ("10 Serving Engines", the --kv-cache-dtype flag); the format taken
// is OCP E4M3 with one scale per cache: element x is stored as the code of
// x * inv_scale (float32 product), rounded to nearest even by the hardware
// conversion and saturated to +-448 first (the conversion itself would turn
// an overflow into NaN).  Each thread converts 8 elements of one row: one
// 16-byte (bf16) or two 16-byte (fp32) loads and one 8-byte store per cache.
__device__ __forceinline__ float sat_e4m3(float x) {
  return x != x ? x : fminf(fmaxf(x, -448.f), 448.f);
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), w, true);
  return static_cast<uint32_t>(w);
}

template <bool kBf16Src>
__device__ __forceinline__ uint2 quant8(const char* src, float inv_scale) {
  float x[8];
  if constexpr (kBf16Src) {
    const uint4 r = *reinterpret_cast<const uint4*>(src);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16) * inv_scale;
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u) * inv_scale;
    }
  } else {
    const uint4 r0 = *reinterpret_cast<const uint4*>(src);
    const uint4 r1 = *reinterpret_cast<const uint4*>(src + 16);
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(w[i]) * inv_scale;
  }
  return make_uint2(e4m3x4(x[0], x[1], x[2], x[3]), e4m3x4(x[4], x[5], x[6], x[7]));
}

template <bool kBf16Src>
__global__ __launch_bounds__(256) void store_kv_fp8_kernel(
    const char* __restrict__ k, const char* __restrict__ v,
    uint2* __restrict__ k_cache, uint2* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int64_t num_tokens,
    int64_t groups_per_row, int64_t num_slots, float k_inv_scale,
    float v_inv_scale) {
  constexpr int kSrcBytes = kBf16Src ? 16 : 32;   // source bytes of 8 elements
  const int64_t total = num_tokens * groups_per_row;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < total; i += stride) {
    const int64_t t = i / groups_per_row;
    const int64_t e = i - t * groups_per_row;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    const uint2 kq = quant8<kBf16Src>(k + i * kSrcBytes, k_inv_scale);
    const uint2 vq = quant8<kBf16Src>(v + i * kSrcBytes, v_inv_scale);
    k_cache[slot * groups_per_row + e] = kq;
    v_cache[slot * groups_per_row + e] = vq;
  }
}

hipError_t launch_store_kv_fp8(const void* k, const void* v, void* k_cache,
                               void* v_cache, const int32_t* slot_mapping,
                               int64_t num_tokens, int64_t row_elems,
                               int64_t num_slots, bool bf16_src,
                               float k_inv_scale, float v_inv_scale,
                               hipStream_t stream) {
  const int64_t groups = row_elems / 8;
  const int64_t total = num_tokens * groups;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) return hipSuccess;
  auto kc = reinterpret_cast<uint2*>(k_cache);
  auto vc = reinterpret_cast<uint2*>(v_cache);
  auto ks = static_cast<const char*>(k);
  auto vs = static_cast<const char*>(v);
  if (bf16_src)
    hipLaunchKernelGGL(store_kv_fp8_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(threads), 0, stream, ks, vs, kc, vc, slot_mapping,
                       num_tokens, groups, num_slots, k_inv_scale, v_inv_scale);
  else
    hipLaunchKernelGGL(store_kv_fp8_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(threads), 0, stream, ks, vs, kc, vc, slot_mapping,
                       num_tokens, groups, num_slots, k_inv_scale, v_inv_scale);
  return hipGetLastError();
}

}  // namespace pa
