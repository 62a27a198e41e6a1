// copy_blocks: copy whole cache blocks, the data side of copy-on-write.
//
// For each pair (src, dst) of block_pairs, block dst of the K cache and of
// the V cache becomes a bit-for-bit copy of block src ("Warmup Guide --
// Inference Serving Internals", Chapter 4: a sequence about to write into a
// block other sequences also hold first copies that one block and writes
// into its private copy).  A pair with an id outside [0, num_blocks), or
// with src == dst, copies nothing.
//
// Mapping: grid (pair, slice of a block, cache).  Each workgroup moves one
// 16 KiB slice of one block of one cache: 256 threads x 4 16-byte vectors,
// consecutive threads on consecutive vectors, so reads and writes are whole
// contiguous lines.  The pair's ids are read by scalar loads (uniform over
// the workgroup).  Pure data movement: HBM-bound at 2 * block_bytes read and
// 2 * block_bytes written per pair.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kVecsPerThread = 4;
constexpr int64_t kSliceBytes = kThreads * kVecsPerThread * 16;   // 16 KiB

__device__ __forceinline__ int load_uniform_pair(const int32_t* pairs,
                                                 int64_t i) {
#if defined(__HIP_DEVICE_COMPILE__)
  return ((const __attribute__((address_space(4))) int32_t*)pairs)[i];
#else
  return pairs[i];
#endif
}

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ block_pairs, int64_t block_bytes,
    int64_t num_blocks) {
  const int64_t pair = blockIdx.x;
  const int src = load_uniform_pair(block_pairs, 2 * pair);
  const int dst = load_uniform_pair(block_pairs, 2 * pair + 1);
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks ||
      src == dst)
    return;   // uniform
  char* cache = blockIdx.z == 0 ? k_cache : v_cache;
  const char* from = cache + static_cast<int64_t>(src) * block_bytes;
  char* to = cache + static_cast<int64_t>(dst) * block_bytes;
  const int64_t base = static_cast<int64_t>(blockIdx.y) * kSliceBytes;
  uint4 v[kVecsPerThread];
#pragma unroll
  for (int u = 0; u < kVecsPerThread; ++u) {
    const int64_t off = base + (static_cast<int64_t>(u) * kThreads + threadIdx.x) * 16;
    v[u] = off < block_bytes ? ld16_nt(from + off) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kVecsPerThread; ++u) {
    const int64_t off = base + (static_cast<int64_t>(u) * kThreads + threadIdx.x) * 16;
    if (off < block_bytes) st16(to + off, v[u]);
  }
}

}  // namespace

hipError_t launch_copy_blocks(void* k_cache, void* v_cache,
                              const int32_t* block_pairs, int64_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks,
                              hipStream_t stream) {
  const int64_t slices = (block_bytes + kSliceBytes - 1) / kSliceBytes;
  if (slices > 65535 || num_pairs > 0x7fffffff) return hipErrorNotSupported;
  dim3 grid(static_cast<unsigned>(num_pairs), static_cast<unsigned>(slices), 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, stream,
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache),
                     block_pairs, block_bytes, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
