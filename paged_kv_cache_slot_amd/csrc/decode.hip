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
//    group; wave w takes blocks w, w+4, ... of the partition;
//  * access pattern: 16 lanes cover one 256-byte (token, KV head) row, so
//    every wave load instruction reads whole 128-byte lines of 4 rows; loads
//    are non-temporal (each byte is used once) and address a wave-uniform
//    block base held in SGPRs plus per-lane offsets fixed for the whole
//    kernel; the next block is loaded while the current one is consumed;
//  * pass 1, QK: each lane dots its 8 dimensions of 4 tokens against q held
//    in registers (v_dot2_f32_bf16 for bf16, FMA for fp32); the 16 partial
//    sums of a row are combined with four DPP steps (two quad swaps, half
//    mirror, mirror) -- no LDS round trip for the reduction;
//  * the partition's logits sit in LDS token-major; the exact partition max
//    is known before any exponent, so each logit takes one exp and nothing
//    is rescaled; the first V block is already in flight during the softmax;
//  * pass 2, PV: same lane layout; each lane accumulates its 8 dimensions
//    over its tokens with weights read from LDS as broadcasts; rows of a wave
//    are summed with lane shuffles and the 4 waves through LDS;
//  * a partition writes (max, sum, unnormalised output) to the workspace and
//    a second small kernel merges the partitions with log-sum-exp weights;
//    with a single partition the first kernel writes the output itself;
//  * masking is by select only: tokens at or past L and blocks whose id is
//    outside the pool contribute weight 0 *and* value 0 (loaded values are
//    replaced, never multiplied by zero), so NaN or garbage in unused slots
//    cannot reach the output.  Every slot of a valid block is in bounds, so
//    whole blocks are loaded without per-token branches.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kBlock = 16;           // tokens per cache block
constexpr int kWaves = 4;            // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;

// How a wave covers one 16-token block of one KV head: kLpr lanes share a
// row (token), each lane takes kCpl 16-byte chunks of it, and one load
// instruction covers kRpi rows.  Every instruction reads whole 128-byte
// lines (kLpr * 16 >= 128).
template <int kRow, int kMaxLpr>
struct BlockLayout {
  static constexpr int kChunksPerRow = kRow / 16;
  static constexpr int kLpr = kChunksPerRow < kMaxLpr ? kChunksPerRow : kMaxLpr;
  static constexpr int kRpi = kWave / kLpr;          // rows per instruction
  static constexpr int kCpl = kChunksPerRow / kLpr;  // chunks per lane per row
  static constexpr int kTpl = kBlock / kRpi;         // tokens per lane
  static_assert(kLpr * 16 >= 128, "whole cache lines per instruction");
};

template <typename T, int D, int G, int P>
struct DecodeShape {
  static constexpr int kElem = ElemTraits<T>::kBytes;
  static constexpr int kRow = D * kElem;          // bytes of one (token, KV head)
  static constexpr int kEpc = 16 / kElem;         // elements per 16-byte chunk
  static constexpr int kBlocks = P / kBlock;      // blocks per partition
  using K = BlockLayout<kRow, 8>;    // QK: 8 lanes per row, short reductions
  using V = BlockLayout<kRow, 16>;   // PV: 16 lanes per row, few accumulators
  // bf16 PV runs on v_dot2 over token pairs (i, i + 1 of a lane's tokens).
  static constexpr bool kPairPv = sizeof(T) == 2 && V::kTpl % 2 == 0;
  static constexpr int kPairsPerBlock = kBlock / 2;
  // Register cap that keeps 5 waves per SIMD for the bf16 shapes that fit
  // without spilling; the others keep what the compiler needs.
  static constexpr int kMinWaves = (sizeof(T) == 2 && G <= 4) ? 5 : 1;
  static_assert(kRow % 128 == 0, "rows must be whole 128-byte lines");
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

// Widen one 16-byte chunk to floats.
template <typename T>
struct Widen;
template <>
struct Widen<bf16_t> {
  static __device__ __forceinline__ void run(const uint4& c, float* v) {
    v[0] = bf16_lo(c.x); v[1] = bf16_hi(c.x);
    v[2] = bf16_lo(c.y); v[3] = bf16_hi(c.y);
    v[4] = bf16_lo(c.z); v[5] = bf16_hi(c.z);
    v[6] = bf16_lo(c.w); v[7] = bf16_hi(c.w);
  }
};
template <>
struct Widen<float> {
  static __device__ __forceinline__ void run(const uint4& c, float* v) {
    v[0] = __uint_as_float(c.x); v[1] = __uint_as_float(c.y);
    v[2] = __uint_as_float(c.z); v[3] = __uint_as_float(c.w);
  }
};

// Sum over the kLpr lanes of a DPP row group (kLpr = 4, 8 or 16); every
// lane of the group gets the total.
template <int kLpr>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_f32<kQuadSwap1>(x);
  x += dpp_f32<kQuadSwap2>(x);
  if (kLpr >= 8) x += dpp_f32<kRowHalfMirror>(x);
  if (kLpr == 16) x += dpp_f32<kRowMirror>(x);
  return x;
}


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
__global__ __launch_bounds__(kThreads) __attribute__((
    amdgpu_waves_per_eu(DecodeShape<T, D, G, P>::kMinWaves, 8))) void
decode_partition_kernel(
    DecodeParams p) {
  using S = DecodeShape<T, D, G, P>;
  using KL = typename S::K;
  using VL = typename S::V;
  __shared__ int s_blk[S::kBlocks];
  __shared__ float s_w[P * G];        // logits, then fp32 weights: [t][h]
  __shared__ uint32_t s_wp[S::kPairPv ? P / 2 * G : 1];  // bf16 weight pairs
  __shared__ float s_red[kWaves][G];
  __shared__ float s_acc[kWaves][G][D];
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
  const int row_stride = p.num_kv_heads * S::kRow;   // bytes per slot
  const int64_t blk_bytes = static_cast<int64_t>(kBlock) * row_stride;

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

  // Wave-uniform block base (SGPRs).  An id outside the pool reads block 0
  // and the whole block is then ignored.
  auto block_base = [&](const char* cache, int j, bool& ok) {
    int blk = __builtin_amdgcn_readfirstlane(s_blk[j]);
    ok = blk >= 0 && blk < p.num_blocks;
    blk = ok ? blk : 0;
    return cache + static_cast<int64_t>(blk) * blk_bytes;
  };
  // Tokens of block j that lie inside the context (uniform).
  auto valid_in = [&](int j) { return min(kBlock, ntok - j * kBlock); };

  // ---- pass 1: logits -----------------------------------------------------
  // Lane (krs, ke): token i * KL::kRpi + krs, chunks cc * KL::kLpr + ke.
  const int krs = lane / KL::kLpr;
  const int ke = lane % KL::kLpr;
  uint32_t koff[KL::kTpl][KL::kCpl];
#pragma unroll
  for (int i = 0; i < KL::kTpl; ++i)
#pragma unroll
    for (int cc = 0; cc < KL::kCpl; ++cc)
      koff[i][cc] = (i * KL::kRpi + krs) * row_stride + kvh * S::kRow +
                    (cc * KL::kLpr + ke) * 16;
  uint4 qreg[KL::kCpl][G];
  {
    const char* qbase = reinterpret_cast<const char*>(p.q) +
                        (static_cast<int64_t>(b) * p.num_heads + head0) * S::kRow;
#pragma unroll
    for (int cc = 0; cc < KL::kCpl; ++cc)
#pragma unroll
      for (int h = 0; h < G; ++h)
        qreg[cc][h] = ld16(qbase + h * S::kRow + (cc * KL::kLpr + ke) * 16);
  }
  __syncthreads();

  auto load_k = [&](int j, uint4 (*r)[KL::kCpl], bool& ok) {
    const char* base = block_base(p.k_cache, j, ok);
#pragma unroll
    for (int i = 0; i < KL::kTpl; ++i)
#pragma unroll
      for (int cc = 0; cc < KL::kCpl; ++cc) r[i][cc] = ld16_nt(base + koff[i][cc]);
  };

  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;

  auto logits = [&](int j, const uint4 (*kr)[KL::kCpl], bool ok) {
    const int nvalid = ok ? valid_in(j) : 0;
#pragma unroll
    for (int i = 0; i < KL::kTpl; ++i) {
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
      for (int cc = 0; cc < KL::kCpl; ++cc) ChunkDot<T, G>::run(kr[i][cc], qreg[cc], s);
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = row_sum<KL::kLpr>(s[h]) * p.scale_log2;
      const int tb = i * KL::kRpi + krs;       // token inside the block
      if (nvalid < kBlock) {                   // uniform: partial or bad block
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = tb < nvalid ? s[h] : -INFINITY;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) mloc[h] = fmaxf(mloc[h], s[h]);
      if (ke == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_w[(j * kBlock + tb) * G + h] = s[h];
      }
    }
  };
  {
    uint4 ka[KL::kTpl][KL::kCpl], kb[KL::kTpl][KL::kCpl];
    bool oka = false, okb = false;
    int j = wave;
    if (j < nblk) load_k(j, ka, oka);
    while (j < nblk) {
      if (j + kWaves < nblk) load_k(j + kWaves, kb, okb);
      logits(j, ka, oka);
      j += kWaves;
      if (j >= nblk) break;
      if (j + kWaves < nblk) load_k(j + kWaves, ka, oka);
      logits(j, kb, okb);
      j += kWaves;
    }
  }

  // ---- first V block in flight; softmax over the partition ---------------
  // Lane (vrs, ve): token i * VL::kRpi + vrs, chunks cc * VL::kLpr + ve.
  const int vrs = lane / VL::kLpr;
  const int ve = lane % VL::kLpr;
  uint32_t voff[VL::kTpl][VL::kCpl];
#pragma unroll
  for (int i = 0; i < VL::kTpl; ++i)
#pragma unroll
    for (int cc = 0; cc < VL::kCpl; ++cc)
      voff[i][cc] = (i * VL::kRpi + vrs) * row_stride + kvh * S::kRow +
                    (cc * VL::kLpr + ve) * 16;
  auto load_v = [&](int j, uint4 (*r)[VL::kCpl], bool& ok) {
    const char* base = block_base(p.v_cache, j, ok);
#pragma unroll
    for (int i = 0; i < VL::kTpl; ++i)
#pragma unroll
      for (int cc = 0; cc < VL::kCpl; ++cc) r[i][cc] = ld16_nt(base + voff[i][cc]);
  };
  uint4 va[VL::kTpl][VL::kCpl], vb[VL::kTpl][VL::kCpl];
  bool vok_a = false, vok_b = false;
  if (wave < nblk) load_v(wave, va, vok_a);

#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = wave_max(mloc[h]);
    if (lane == 0) s_red[wave][h] = m;
  }
  __syncthreads();
  if (tid < G) {
    float m = s_red[0][tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_red[w][tid]);
    s_m[tid] = m;
  }
  __syncthreads();
  {
    // Weights 2^(s - m); masked slots (-inf) become 0, and a head whose
    // every token was masked (m = -inf) gets all-zero weights.  kThreads is a
    // multiple of G, so each thread always works on the same head.
    const int h = tid % G;
    const float m = s_m[h];
    float acc_l = 0.f;
    auto weight = [&](float x) {
      return (m == -INFINITY || x == -INFINITY) ? 0.f : fast_exp2(x - m);
    };
    if constexpr (S::kPairPv) {
      // Pair q of block j joins the lane's tokens t and t + VL::kRpi of the
      // PV layout; the pair is stored as two bfloat16 (low = t).
      for (int i = tid; i < nblk * S::kPairsPerBlock * G; i += kThreads) {
        const int pr = i / G;
        const int j = pr / S::kPairsPerBlock;
        const int q = pr % S::kPairsPerBlock;
        const int ta = j * kBlock + (q / VL::kRpi) * 2 * VL::kRpi + q % VL::kRpi;
        const float wa = weight(s_w[ta * G + h]);
        const float wb = weight(s_w[(ta + VL::kRpi) * G + h]);
        s_wp[i] = static_cast<uint32_t>(f32_to_bf16_rne(wa)) |
                  (static_cast<uint32_t>(f32_to_bf16_rne(wb)) << 16);
        acc_l += wa + wb;
      }
    } else {
      for (int i = tid; i < nblk * kBlock * G; i += kThreads) {
        const float w = weight(s_w[i]);
        s_w[i] = w;
        acc_l += w;
      }
    }
#pragma unroll
    for (int o = kWave / 2; o >= G; o >>= 1) acc_l += __shfl_xor(acc_l, o, kWave);
    if (lane < G) s_red[wave][lane] = acc_l;
  }
  __syncthreads();
  if (tid < G) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l += s_red[w][tid];
    s_l[tid] = l;
  }

  // ---- pass 2: weighted sum of V -----------------------------------------
  float acc[G][VL::kCpl][S::kEpc];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int cc = 0; cc < VL::kCpl; ++cc)
#pragma unroll
      for (int x = 0; x < S::kEpc; ++x) acc[h][cc][x] = 0.f;

  auto accumulate = [&](int j, uint4 (*vr)[VL::kCpl], bool ok) {
    if (!ok) return;  // uniform: a block outside the pool adds nothing
    const int nvalid = valid_in(j);
    if (nvalid < kBlock) {
      // Partial last block: replace slots past the context by zeros (they
      // may hold anything, NaN included); their weights are 0 as well.
#pragma unroll
      for (int i = 0; i < VL::kTpl; ++i)
#pragma unroll
        for (int cc = 0; cc < VL::kCpl; ++cc)
          if (i * VL::kRpi + vrs >= nvalid) vr[i][cc] = make_uint4(0, 0, 0, 0);
    }
    if constexpr (S::kPairPv) {
#pragma unroll
      for (int pi = 0; pi < VL::kTpl / 2; ++pi) {
        const int q = pi * VL::kRpi + vrs;     // pair index inside the block
        uint32_t wp[G];
#pragma unroll
        for (int h = 0; h < G; ++h) wp[h] = s_wp[(j * S::kPairsPerBlock + q) * G + h];
#pragma unroll
        for (int cc = 0; cc < VL::kCpl; ++cc) {
          const uint4 x = vr[2 * pi][cc];
          const uint4 y = vr[2 * pi + 1][cc];
          const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
          const uint32_t ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            const uint32_t lo = pack_lo(xs[dw], ys[dw]);
            const uint32_t hi = pack_hi(xs[dw], ys[dw]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              acc[h][cc][2 * dw] = dot2_bf16(lo, wp[h], acc[h][cc][2 * dw]);
              acc[h][cc][2 * dw + 1] = dot2_bf16(hi, wp[h], acc[h][cc][2 * dw + 1]);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < VL::kTpl; ++i) {
        const int t = j * kBlock + i * VL::kRpi + vrs;
        float w[G];
#pragma unroll
        for (int h = 0; h < G; ++h) w[h] = s_w[t * G + h];
#pragma unroll
        for (int cc = 0; cc < VL::kCpl; ++cc) {
          float v[S::kEpc];
          Widen<T>::run(vr[i][cc], v);
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int x = 0; x < S::kEpc; ++x)
              acc[h][cc][x] = fmaf(w[h], v[x], acc[h][cc][x]);
        }
      }
    }
  };
  {
    int j = wave;
    while (j < nblk) {
      if (j + kWaves < nblk) load_v(j + kWaves, vb, vok_b);
      accumulate(j, va, vok_a);
      j += kWaves;
      if (j >= nblk) break;
      if (j + kWaves < nblk) load_v(j + kWaves, va, vok_a);
      accumulate(j, vb, vok_b);
      j += kWaves;
    }
  }

  // Sum the row groups of the wave (same dimensions, different tokens) with
  // shuffles, then the waves through LDS.
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int cc = 0; cc < VL::kCpl; ++cc)
#pragma unroll
      for (int x = 0; x < S::kEpc; ++x) {
        float a = acc[h][cc][x];
#pragma unroll
        for (int o = VL::kLpr; o < kWave; o <<= 1) a += __shfl_xor(a, o, kWave);
        acc[h][cc][x] = a;
      }
  if (vrs == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int cc = 0; cc < VL::kCpl; ++cc)
#pragma unroll
        for (int x = 0; x < S::kEpc; ++x)
          s_acc[wave][h][(cc * VL::kLpr + ve) * S::kEpc + x] = acc[h][cc][x];
  }
  __syncthreads();

  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D;
    const int d = i % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += s_acc[w][h][d];
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

#ifndef PA_DECODE_PARTITION
#define PA_DECODE_PARTITION 512
#endif
constexpr int kPartitionTokens = PA_DECODE_PARTITION;

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
