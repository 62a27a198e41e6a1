// Helpers of the MFMA tile kernels (varlen prefill and the small-row path):
// LDS DMA of cache rows, explicit memory-counter waits, LDS transpose reads,
// lane-half exchange, the clamped extent of one varlen sequence, and the
// longest-first counting sort their schedules use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

constexpr int kTileBlock = 16;   // tokens per cache block

// A wave-uniform int32 that stays constant for the whole kernel (a block id),
// read through the constant address space so it arrives by a scalar load
// counted by lgkmcnt.  Read as a vector load it would be counted by vmcnt,
// and each wait for it would also wait for every DMA load issued before.
__device__ __forceinline__ int load_uniform_i32(const int32_t* base, int idx) {
#if defined(__HIP_DEVICE_COMPILE__)
  return ((const __attribute__((address_space(4))) int32_t*)base)[idx];
#else
  return base[idx];
#endif
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l's bytes land at lds + 16 l; `lds` must be
// the same for the whole wave (it goes to M0).  Completion is counted by
// vmcnt.  Issued from inline assembly: the compiler cannot tell which LDS
// bytes the load writes and, seeing the builtin, would wait for it before
// the next LDS read of any buffer -- which would make the prefetch of later
// tiles wait for the current one.  The caller orders the loads against LDS
// reads with explicit vmcnt waits (and barriers where other waves read).
// The source is base + off: base uniform (an SGPR pair), off this lane's
// 32-bit byte offset.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const unsigned m0 = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds)));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(m0) : "memory", "m0");
#else
  (void)base;
  (void)off;
  (void)lds;
#endif
}

// Wait until at most N vector memory loads of this lane are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
#endif
}

// Wait until this wave's LDS reads and writes (and scalar loads) are done.
__device__ __forceinline__ void wait_lgkm() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
}

// Workgroup barrier after this wave's LDS reads have completed.  Unlike
// __syncthreads it does not also wait for every vector load in flight (the
// prefetched K/V tiles).
__device__ __forceinline__ void lds_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
}

// LDS transpose read (ds_read_b64_tr_b16).  In each group of 16 lanes, if
// lane s reads the four 16-bit values M[s][0..3] at its address, lane i
// receives M[4k + i/4][i % 4] for k = 0..3 (checked on gfx950).
// (The host compilation pass has no LDS address space; it only needs the
// declaration.)
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(p));
  return __builtin_bit_cast(uint2, r);
#else
  (void)p;
  return make_uint2(0, 0);
#endif
}

// The value lane l ^ 32 holds (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float swap_halves(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
#else
  return x;
#endif
}

// Query rows and cached keys of varlen sequence b, clamped so that no index
// leaves the buffers: rows q0 .. q0 + lq - 1 of q, keys 0 .. lk - 1.
struct SeqExtent {
  int q0, lq, lk;
};
__device__ __forceinline__ SeqExtent seq_extent(const int32_t* cu_q,
                                                const int32_t* cu_k, int b,
                                                int max_q, int max_k,
                                                int64_t total_q,
                                                int max_blocks) {
  int q0 = cu_q[b];
  int lq = cu_q[b + 1] - q0;
  int lk = cu_k[b + 1] - cu_k[b];
  q0 = q0 < 0 ? 0 : q0;
  lq = lq < 0 ? 0 : (lq > max_q ? max_q : lq);
  if (q0 + lq > total_q) lq = static_cast<int>(total_q - q0 < 0 ? 0 : total_q - q0);
  lk = lk < 0 ? 0 : (lk > max_k ? max_k : lk);
  if (lk > max_blocks * kTileBlock) lk = max_blocks * kTileBlock;
  return {q0, lq, lk};
}

// Longest-first order of n work items, by one workgroup of kThreads
// threads: a counting sort over kBins weight bins in LDS (`bins`, kBins
// ints; `wave_sum`, kThreads / 64 ints), heaviest bin first.  weight(item)
// must lie in [0, kBins).  Items of equal weight land in any order.  The
// bins of each thread's first kRegItems items stay in registers between the
// two passes, so their inputs are read once.
template <int kThreads, int kBins, int kRegItems, typename WeightFn>
__device__ __forceinline__ void longest_first_order(int n, WeightFn weight,
                                                    int32_t* order, int* bins,
                                                    int* wave_sum) {
  static_assert(kBins % kThreads == 0, "bins per thread");
  constexpr int kBinsPerThread = kBins / kThreads;
  const int tid = threadIdx.x;
  int mybin[kRegItems];
#pragma unroll
  for (int k = 0; k < kRegItems; ++k) {
    const int item = tid + k * kThreads;
    mybin[k] = item < n ? weight(item) : 0;
  }
  for (int i = tid; i < kBins; i += kThreads) bins[i] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kRegItems; ++k)
    if (tid + k * kThreads < n) atomicAdd(&bins[mybin[k]], 1);
  for (int item = tid + kRegItems * kThreads; item < n; item += kThreads)
    atomicAdd(&bins[weight(item)], 1);
  __syncthreads();
  // Exclusive prefix from the heaviest bin down: a scan inside each wave,
  // then the totals of the waves before it.
  int cnt[kBinsPerThread];
  int mine = 0;
#pragma unroll
  for (int k = 0; k < kBinsPerThread; ++k) {
    cnt[k] = bins[kBins - 1 - (kBinsPerThread * tid + k)];
    mine += cnt[k];
  }
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  int incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off *= 2) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wave_sum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_sum[w];
  int start = before + incl - mine;
#pragma unroll
  for (int k = 0; k < kBinsPerThread; ++k) {
    bins[kBins - 1 - (kBinsPerThread * tid + k)] = start;
    start += cnt[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kRegItems; ++k) {
    const int item = tid + k * kThreads;
    if (item < n) order[atomicAdd(&bins[mybin[k]], 1)] = item;
  }
  for (int item = tid + kRegItems * kThreads; item < n; item += kThreads)
    order[atomicAdd(&bins[weight(item)], 1)] = item;
}

// Rank of this workgroup's work item in the longest-first order, found by
// the workgroup itself when there are at most as many items as threads
// (no plan kernel): heaviest first, equal weights by index.  `s_w` is LDS
// scratch of round_up(n, 4) + 1 ints.  Returns the item of rank `rank`
// (-1 if none).  Every thread of the workgroup must call it.
template <int kThreads, typename WeightFn>
__device__ __forceinline__ int inline_ranked_item(int n, int rank,
                                                  WeightFn weight, int* s_w) {
  const int tid = threadIdx.x;
  int* s_item = s_w + kThreads + 4;
  const int n4 = (n + 3) & ~3;
  int w = -1;
  if (tid < n) w = weight(tid);
  if (tid < n4) s_w[tid] = w;               // padding -1: lighter than any item
  if (tid == 0) *s_item = -1;
  __syncthreads();
  if (tid < n) {
    int r = 0;
    for (int j = 0; j < n4; j += 4) {
      const int4 x = *reinterpret_cast<const int4*>(s_w + j);
      r += (x.x > w || (x.x == w && j < tid)) ? 1 : 0;
      r += (x.y > w || (x.y == w && j + 1 < tid)) ? 1 : 0;
      r += (x.z > w || (x.z == w && j + 2 < tid)) ? 1 : 0;
      r += (x.w > w || (x.w == w && j + 3 < tid)) ? 1 : 0;
    }
    if (r == rank) *s_item = tid;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_item);
}

}  // namespace pa
