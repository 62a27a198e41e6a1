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

}  // namespace pa
