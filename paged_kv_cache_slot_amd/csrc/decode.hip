// Paged decode attention for gfx950: split-context partitions + merge.
//
// What it computes (the pages name the kernel, "3.6 ModelRunner, CUDA Graph,
// and benchmarks" section 2, and the block-table walk, "Warmup Guide --
// Inference Serving Internals" Chapter 3): for sequence b with context
// length L and query head h,
//     out[b,h] = softmax_j(scale * q[b,h] . K_b[j]) V_b[j],   j < L,
// K_b[j] being row j % 16 of physical block block_tables[b][j / 16], KV head
// h / G.
//
// Design (MI355X-first; the work is an HBM stream, ~2 FLOP per byte):
//  * one workgroup (4 waves) per (partition of P tokens, KV head, sequence):
//    every K/V byte of a KV head is read once for all G query heads of its
//    group;
//  * pass 1, QK: 4 lanes per token, 16 tokens (one block) per wave step;
//    each lane holds a quarter of the row in 16-byte chunks, dots against q
//    kept in registers with v_dot2_f32_bf16 (bf16) or FMA (fp32), and the 4
//    partial sums are combined with two DPP quad permutes -- no LDS traffic
//    for the reduction;
//  * the partition's logits (G x P floats) sit in LDS; the exact partition
//    max is known before any exponent, so each partition needs one exp per
//    logit and no rescaling;
//  * pass 2, PV: lanes own head dimensions and walk the block's tokens, so
//    every V load is a contiguous row segment; the weights come from LDS as
//    broadcasts;
//  * the 4 waves' partial outputs are summed through LDS; a partition writes
//    (max, sum, unnormalised output) to the workspace, and a second small
//    kernel merges the partitions with log-sum-exp weights.  With a single
//    partition the first kernel writes the final output itself.
//  * masking is by predicate only: tokens at or past L, and tokens of a
//    block id outside the pool, take no part (never multiplied by zero), so
//    garbage or NaN in unused slots cannot leak into the output.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kBlock = 16;           // tokens per cache block
constexpr int kWaves = 4;            // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D, int G, int P>
struct DecodeShape {
  static constexpr int kElem = ElemTraits<T>::kBytes;
  static constexpr int kRow = D * kElem;     // bytes of one (token, KV head)
  static constexpr int kChunks = kRow / 64;  // 16-byte chunks per QK lane
  static constexpr int kBlocks = P / kBlock; // blocks per partition
  // PV layout: each lane owns kPvVec contiguous bytes of a row.
  static constexpr int kPvVec = kRow >= 256 ? kRow / 64 : 4;
  static constexpr int kPvLanes = kRow / kPvVec;   // lanes per token
  static constexpr int kPvSlots = kWave / kPvLanes;  // tokens per wave step
  static constexpr int kPvElems = kPvVec / kElem;
  static constexpr int kPvSteps = kBlock / kPvSlots;
  static_assert(kRow % 64 == 0, "row must split into 4 lanes x 16 bytes");
  static_assert(kPvSlots >= 1 && kBlock % kPvSlots == 0, "PV layout");
  static_assert(P % (kBlock * kWaves) == 0, "partition shape");
};

// Partial dot products of one 16-byte chunk of K with the matching chunk of
// each query head.
template <typename T, int G>
struct ChunkDot;

template <int G>
struct ChunkDot<bf16_t, G> {
  static __device__ __forceinline__ void run(const uint4& k, const uint4* q,
                                             float* s) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = s[h];
      a = dot2_bf16(k.x, q[h].x, a);
      a = dot2_bf16(k.y, q[h].y, a);
      a = dot2_bf16(k.z, q[h].z, a);
      a = dot2_bf16(k.w, q[h].w, a);
      s[h] = a;
    }
  }
};

template <int G>
struct ChunkDot<float, G> {
  static __device__ __forceinline__ void run(const uint4& k, const uint4* q,
                                             float* s) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = s[h];
      a = fmaf(__uint_as_float(k.x), __uint_as_float(q[h].x), a);
      a = fmaf(__uint_as_float(k.y), __uint_as_float(q[h].y), a);
      a = fmaf(__uint_as_float(k.z), __uint_as_float(q[h].z), a);
      a = fmaf(__uint_as_float(k.w), __uint_as_float(q[h].w), a);
      s[h] = a;
    }
  }
};

// Load kPvVec bytes of V and widen to kPvElems floats.
template <typename T, int kVec>
struct PvLoad;

template <>
struct PvLoad<bf16_t, 4> {
  typedef uint32_t raw_t;
  static __device__ __forceinline__ raw_t load(const char* p) {
    return *reinterpret_cast<const uint32_t*>(p);
  }
  static __device__ __forceinline__ void widen(raw_t r, float* v) {
    v[0] = bf16_lo(r);
    v[1] = bf16_hi(r);
  }
};

template <>
struct PvLoad<float, 4> {
  typedef uint32_t raw_t;
  static __device__ __forceinline__ raw_t load(const char* p) {
    return *reinterpret_cast<const uint32_t*>(p);
  }
  static __device__ __forceinline__ void widen(raw_t r, float* v) {
    v[0] = __uint_as_float(r);
  }
};

template <>
struct PvLoad<float, 8> {
  typedef uint2 raw_t;
  static __device__ __forceinline__ raw_t load(const char* p) {
    return *reinterpret_cast<const uint2*>(p);
  }
  static __device__ __forceinline__ void widen(raw_t r, float* v) {
    v[0] = __uint_as_float(r.x);
    v[1] = __uint_as_float(r.y);
  }
};

template <typename T>
__device__ __forceinline__ void store_out(T* out, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* out, float x) {
  *out = x;
}
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t* out, float x) {
  out->bits = f32_to_bf16_rne(x);
}

struct DecodeParams {
  void* out;
  const void* q;
  const char* k_cache;
  const char* v_cache;
  int64_t num_blocks;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int max_context_len;
  int num_heads;
  int num_kv_heads;
  float scale_log2;  // scale * log2(e): logits live in the base-2 domain
  float* ws_max;     // [B, Hq, NP]   (multi-partition only)
  float* ws_sum;     // [B, Hq, NP]
  float* ws_acc;     // [B, Hq, NP, D]
  int num_partitions;
};

__device__ __forceinline__ int clamp_len(const DecodeParams& p, int b) {
  int len = p.context_lens[b];
  len = len < 0 ? 0 : len;
  len = len > p.max_context_len ? p.max_context_len : len;
  const int cap = p.max_blocks_per_seq * kBlock;
  return len > cap ? cap : len;
}

template <typename T, int D, int G, int P>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(
    DecodeParams p) {
  using S = DecodeShape<T, D, G, P>;
  __shared__ int s_blk[S::kBlocks];
  __shared__ float s_logit[G * P];
  __shared__ float s_red[kWaves][G];
  __shared__ float s_acc[kWaves * S::kPvSlots][G][D];
  __shared__ float s_m[G], s_l[G];

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const bool single = p.num_partitions == 1;

  const int len = clamp_len(p, b);
  const int t0 = part * P;
  const int head0 = kvh * G;
  const int64_t row_stride = static_cast<int64_t>(p.num_kv_heads) * S::kRow;

  if (t0 >= len) {
    // Nothing to attend.  A single-partition launch owns the output row and
    // writes zeros for an empty context (batch padding); otherwise the merge
    // pass never reads this partition.
    if (single && part == 0) {
      T* out = reinterpret_cast<T*>(p.out) +
               (static_cast<int64_t>(b) * p.num_heads + head0) * D;
      for (int i = tid; i < G * D; i += kThreads) store_out<T>(out + i, 0.f);
    }
    return;
  }
  const int ntok = min(P, len - t0);
  const int nblk = (ntok + kBlock - 1) / kBlock;

  // Block ids of this partition (only the ones the context covers).
  if (tid < nblk) {
    s_blk[tid] = p.block_tables[static_cast<int64_t>(b) * p.max_blocks_per_seq +
                                t0 / kBlock + tid];
  }

  // ---- pass 1: logits -------------------------------------------------
  const int tok = lane >> 2;      // token inside the block
  const int quarter = lane & 3;   // which quarter of the row
  uint4 qreg[S::kChunks][G];
  {
    const char* qbase = reinterpret_cast<const char*>(p.q) +
                        (static_cast<int64_t>(b) * p.num_heads + head0) *
                            S::kRow;
#pragma unroll
    for (int c = 0; c < S::kChunks; ++c)
#pragma unroll
      for (int h = 0; h < G; ++h)
        qreg[c][h] = ld16(qbase + h * S::kRow + (c * 4 + quarter) * 16);
  }
  __syncthreads();

  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;

  auto load_k = [&](int j, uint4* kr, bool& ok) {
    const int blk = s_blk[j];
    const int t = j * kBlock + tok;
    ok = t < ntok && blk >= 0 && blk < p.num_blocks;
#pragma unroll
    for (int c = 0; c < S::kChunks; ++c) kr[c] = make_uint4(0, 0, 0, 0);
    if (ok) {
      const char* row = p.k_cache +
                        (static_cast<int64_t>(blk) * kBlock + tok) * row_stride +
                        static_cast<int64_t>(kvh) * S::kRow;
#pragma unroll
      for (int c = 0; c < S::kChunks; ++c)
        kr[c] = ld16(row + (c * 4 + quarter) * 16);
    }
  };

  {
    uint4 cur[S::kChunks], nxt[S::kChunks];
    bool cur_ok = false, nxt_ok = false;
    int j = wave;
    if (j < nblk) load_k(j, cur, cur_ok);
    for (; j < nblk; j += kWaves) {
      if (j + kWaves < nblk) load_k(j + kWaves, nxt, nxt_ok);
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
      for (int c = 0; c < S::kChunks; ++c)
        ChunkDot<T, G>::run(cur[c], &qreg[c][0], s);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float v = quad_sum(s[h]) * p.scale_log2;
        s[h] = cur_ok ? v : -INFINITY;
        mloc[h] = fmaxf(mloc[h], s[h]);
        if ((h & 3) == quarter) s_logit[h * P + j * kBlock + tok] = s[h];
      }
#pragma unroll
      for (int c = 0; c < S::kChunks; ++c) cur[c] = nxt[c];
      cur_ok = nxt_ok;
    }
  }

  // Partition max per head: wave, then workgroup.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = wave_max(mloc[h]);
    if (lane == 0) s_red[wave][h] = m;
  }
  __syncthreads();
  float mpart[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = s_red[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_red[w][h]);
    mpart[h] = m;
  }
  __syncthreads();

  // Weights 2^(s - m) in place, and their sums.  Slots of masked tokens
  // inside the last block hold -inf and become 0; a head whose every token
  // was masked (all block ids invalid) has m = -inf and gets all-zero
  // weights and a zero sum.
  const int nslot = nblk * kBlock;
  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float acc = 0.f;
    const bool live = mpart[h] != -INFINITY;
    for (int t = tid; t < nslot; t += kThreads) {
      float* ptr = &s_logit[h * P + t];
      const float w = (live && t < ntok) ? fast_exp2(*ptr - mpart[h]) : 0.f;
      *ptr = w;
      acc += w;
    }
    acc = wave_sum(acc);
    if (lane == 0) s_red[wave][h] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l += s_red[w][h];
    lsum[h] = l;
  }

  // ---- pass 2: weighted sum of V ---------------------------------------
  using L = PvLoad<T, S::kPvVec>;
  const int pv_slot = lane / S::kPvLanes;
  const int pv_lane = lane % S::kPvLanes;
  float acc[G][S::kPvElems];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < S::kPvElems; ++e) acc[h][e] = 0.f;

  for (int j = wave; j < nblk; j += kWaves) {
    const int blk = s_blk[j];
    if (blk < 0 || blk >= p.num_blocks) continue;  // uniform over the wave
    const int nvalid = min(kBlock, ntok - j * kBlock);
    const char* base = p.v_cache + static_cast<int64_t>(blk) * kBlock * row_stride +
                       static_cast<int64_t>(kvh) * S::kRow + pv_lane * S::kPvVec;
    typename L::raw_t vr[S::kPvSteps];
#pragma unroll
    for (int st = 0; st < S::kPvSteps; ++st) {
      const int i = st * S::kPvSlots + pv_slot;
      if (i < nvalid) vr[st] = L::load(base + i * row_stride);
    }
#pragma unroll
    for (int st = 0; st < S::kPvSteps; ++st) {
      const int i = st * S::kPvSlots + pv_slot;
      if (i < nvalid) {
        float v[S::kPvElems];
        L::widen(vr[st], v);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float w = s_logit[h * P + j * kBlock + i];
#pragma unroll
          for (int e = 0; e < S::kPvElems; ++e) acc[h][e] = fmaf(w, v[e], acc[h][e]);
        }
      }
    }
  }

  // Sum the partial outputs of all waves (and token slots) through LDS.
  if (tid == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[h] = mpart[h];
      s_l[h] = lsum[h];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < S::kPvElems; ++e)
      s_acc[wave * S::kPvSlots + pv_slot][h][pv_lane * S::kPvElems + e] = acc[h][e];
  __syncthreads();

  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D;
    const int d = i % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves * S::kPvSlots; ++w) o += s_acc[w][h][d];
    const int64_t head = static_cast<int64_t>(b) * p.num_heads + head0 + h;
    if (single) {
      const float l = s_l[h];
      T* out = reinterpret_cast<T*>(p.out) + head * D + d;
      store_out<T>(out, l > 0.f ? o / l : 0.f);
    } else {
      const int64_t slot = head * p.num_partitions + part;
      p.ws_acc[slot * D + d] = o;
      if (d == 0) {
        p.ws_max[slot] = s_m[h];
        p.ws_sum[slot] = s_l[h];
      }
    }
  }
}

// Merge the partitions of one (sequence, query head): weights 2^(m_p - m*)
// rescale each partition's sum and output; the result is their ratio.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeParams p,
                                                         int partition_tokens) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int len = clamp_len(p, b);
  const int np = (len + partition_tokens - 1) / partition_tokens;
  const int64_t head = static_cast<int64_t>(b) * p.num_heads + h;
  T* out = reinterpret_cast<T*>(p.out) + head * D + d;
  const float* mx = p.ws_max + head * p.num_partitions;
  const float* sm = p.ws_sum + head * p.num_partitions;
  const float* ac = p.ws_acc + head * p.num_partitions * D + d;
  float m = -INFINITY;
  for (int i = 0; i < np; ++i) m = fmaxf(m, mx[i]);
  if (np == 0 || m == -INFINITY) {
    store_out<T>(out, 0.f);
    return;
  }
  float l = 0.f, o = 0.f;
  for (int i = 0; i < np; ++i) {
    const float w = fast_exp2(mx[i] - m);
    l = fmaf(w, sm[i], l);
    o = fmaf(w, ac[static_cast<int64_t>(i) * D], o);
  }
  store_out<T>(out, l > 0.f ? o / l : 0.f);
}

template <typename T, int D, int G, int P>
hipError_t launch_typed(const DecodeParams& prm, int num_seqs, int num_kv_heads,
                        int num_heads, hipStream_t stream) {
  dim3 grid(prm.num_partitions, num_kv_heads, num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, G, P>), grid,
                     dim3(kThreads), 0, stream, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || prm.num_partitions == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(num_heads, num_seqs),
                     dim3(D), 0, stream, prm, P);
  return hipGetLastError();
}

template <typename T, int D, int P>
hipError_t dispatch_group(const DecodeParams& prm, int num_seqs,
                          int num_kv_heads, int num_heads, hipStream_t s) {
  switch (num_heads / num_kv_heads) {
    case 1: return launch_typed<T, D, 1, P>(prm, num_seqs, num_kv_heads, num_heads, s);
    case 2: return launch_typed<T, D, 2, P>(prm, num_seqs, num_kv_heads, num_heads, s);
    case 4: return launch_typed<T, D, 4, P>(prm, num_seqs, num_kv_heads, num_heads, s);
    case 8: return launch_typed<T, D, 8, P>(prm, num_seqs, num_kv_heads, num_heads, s);
    default: return hipErrorInvalidValue;
  }
}

constexpr int kPartitionTokens = 512;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

DecodePlan plan_decode(int num_seqs, int num_heads, int num_kv_heads,
                       int head_dim, int max_context_len) {
  (void)num_kv_heads;
  DecodePlan plan{};
  plan.partition_tokens = kPartitionTokens;
  int np = (max_context_len + kPartitionTokens - 1) / kPartitionTokens;
  plan.num_partitions = np < 1 ? 1 : np;
  if (plan.num_partitions == 1) {
    plan.workspace_bytes = 0;
    return plan;
  }
  const size_t slots = static_cast<size_t>(num_seqs) * num_heads *
                       plan.num_partitions;
  plan.off_max = 0;
  plan.off_sum = align256(slots * sizeof(float));
  plan.off_acc = plan.off_sum + align256(slots * sizeof(float));
  plan.workspace_bytes =
      plan.off_acc + align256(slots * static_cast<size_t>(head_dim) * sizeof(float));
  return plan;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan,
                         hipStream_t stream) {
  DecodeParams prm{};
  prm.out = a.out;
  prm.q = a.q;
  prm.k_cache = static_cast<const char*>(a.k_cache);
  prm.v_cache = static_cast<const char*>(a.v_cache);
  prm.num_blocks = a.num_blocks;
  prm.block_tables = a.block_tables;
  prm.max_blocks_per_seq = a.max_blocks_per_seq;
  prm.context_lens = a.context_lens;
  prm.max_context_len = a.max_context_len;
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  prm.scale_log2 = a.scale * kLog2e;
  prm.num_partitions = plan.num_partitions;
  if (plan.num_partitions > 1) {
    char* ws = static_cast<char*>(a.workspace);
    prm.ws_max = reinterpret_cast<float*>(ws + plan.off_max);
    prm.ws_sum = reinterpret_cast<float*>(ws + plan.off_sum);
    prm.ws_acc = reinterpret_cast<float*>(ws + plan.off_acc);
  }
  constexpr int P = kPartitionTokens;
  if (a.bf16) {
    if (a.head_dim == 128)
      return dispatch_group<bf16_t, 128, P>(prm, a.num_seqs, a.num_kv_heads, a.num_heads, stream);
    return dispatch_group<bf16_t, 64, P>(prm, a.num_seqs, a.num_kv_heads, a.num_heads, stream);
  }
  if (a.head_dim == 128)
    return dispatch_group<float, 128, P>(prm, a.num_seqs, a.num_kv_heads, a.num_heads, stream);
  return dispatch_group<float, 64, P>(prm, a.num_seqs, a.num_kv_heads, a.num_heads, stream);
}

}  // namespace pa
