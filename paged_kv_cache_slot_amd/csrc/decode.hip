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
//  * one workgroup (4 waves) per (partition, KV head, sequence): every K/V
//    byte of a KV head is read once for all G query heads of its group;
//  * a partition is walked in chunks of 512 tokens (the chunk's logits sit
//    in LDS); wave w takes blocks w, w+4, ... of each chunk.  The running
//    max and sum carry from chunk to chunk and the output so far is
//    rescaled when the max grows, so a partition of several chunks writes
//    one partial result.  Partial writes interleaved with the K/V read
//    stream cost HBM read bandwidth far beyond their own bytes, so the plan
//    takes the longest partitions that still leave enough workgroups;
//  * the 1-D grid runs KV head fastest, then sequence, then partition.  The
//    dispatcher sends workgroup i to XCD i % 8, so this spreads every
//    sequence and partition evenly over the 8 XCDs (a partition-fastest grid
//    gave partition p of every sequence to XCD p % 8 and left the XCD with
//    the always-full first partitions the last to finish);
//  * access pattern: 8 (QK) or 16 (PV) lanes cover one 256-byte (token,
//    KV head) row, so every load instruction reads whole 128-byte lines;
//    loads are non-temporal buffer loads (each byte is used once) through a
//    per-block buffer resource sized to the block's valid tokens: slots
//    past the context and blocks outside the pool read as zeros without a
//    memory access, so every load is issued unconditionally and the wait
//    before each step is a fixed count; the next block is in flight while
//    the current one is consumed;
//  * a wave's block ids come with one vector load (lane s holds step s's
//    id) and reach SGPRs by readlane;
//  * pass 1, QK: each lane dots its dimensions of its tokens against q held
//    in registers (v_dot2_f32_bf16 for bf16, FMA for fp32); the partial sums
//    of a row are combined with DPP steps -- no LDS round trip;
//  * the chunk's exact max is known before any exponent, so each logit takes
//    one exp; the first V block is already in flight during the softmax;
//  * pass 2, PV: each lane accumulates its 8 dimensions over its tokens
//    (v_dot2 over token pairs for bf16, with bf16 weight pairs from LDS);
//    rows of a wave are summed with lane shuffles and the 4 waves through
//    LDS;
//  * a partition writes (max, sum, unnormalised output) to the workspace and
//    a second small kernel merges the partitions with log-sum-exp weights;
//    with a single partition the first kernel writes the output itself;
//  * masking: tokens at or past L and blocks whose id is outside the pool
//    get logit -inf (weight 0) and read V as zeros, so NaN or garbage in
//    unused slots cannot reach the output.
#include <math.h>

#include <mutex>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_tile.h"

namespace pa {

namespace {

constexpr int kBlock = 16;           // tokens per cache block
constexpr int kWaves = 4;            // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kBf16PairOne = 0x3F803F80u;   // (1.0, 1.0) as bfloat16

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

// F8: the cache holds E4M3 codes (one byte per element) and q / out are
// bfloat16.  The kernel then runs the bfloat16 layout on a virtual bf16 row
// (kRow): each lane loads the codes of its virtual chunks (8 codes per
// 16-byte virtual chunk) and widens them to bfloat16 right before use.
template <typename T, int D, int G, int C, bool F8 = false>
struct DecodeShape {
  static constexpr int kElem = ElemTraits<T>::kBytes;
  static constexpr int kRow = D * kElem;          // bytes of one (token, KV head) as T
  static constexpr int kCacheRow = F8 ? D : kRow; // bytes of it in the cache
  static constexpr int kEpc = 16 / kElem;         // elements per 16-byte chunk
  static constexpr int kBlocks = C / kBlock;      // blocks per chunk
  using K = BlockLayout<kRow, 8>;    // QK: 8 lanes per row, short reductions
  using V = BlockLayout<kRow, 16>;   // PV: 16 lanes per row, few accumulators
  // bf16 PV runs on v_dot2 over token pairs (i, i + 1 of a lane's tokens).
  static constexpr bool kPairPv = sizeof(T) == 2 && V::kTpl % 2 == 0;
  static constexpr int kPairsPerBlock = kBlock / 2;
  // Register floor per SIMD for bf16: 5 waves (96 VGPRs) with G <= 2, 3
  // waves (168) with G = 4.  The chunk loop keeps the output accumulators
  // live through the QK pass; a tighter cap for G = 4 made the compiler
  // spill (measured slower).
  static constexpr int kMinWaves =
      sizeof(T) == 2 ? (G <= 2 ? 5 : (G <= 4 ? 3 : 1)) : 1;
  // Blocks each wave has in flight: the next block's K (or V) is loaded
  // while the current one is consumed.  Deeper prefetch was measured and
  // gains nothing.
  static constexpr int kDepth = 2;
  static_assert(kCacheRow % 128 == 0, "rows must be whole 128-byte lines");
  static_assert(!F8 || sizeof(T) == 2, "E4M3 cache with bfloat16 q / out");
  static_assert(C % (kBlock * kWaves) == 0, "chunk shape");
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
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  float scale_log2;  // scale * log2(e): logits live in the base-2 domain
  float* ws_max;     // [B, Hq, ws_stride]   (multi-partition only)
  float* ws_sum;     // [B, Hq, ws_stride]; negative: partial stored scaled
  float* ws_acc;     // [B, Hq, ws_stride, D]: fp32 acc (fp32 I/O)
  uint16_t* ws_acc_h;  // same memory: binary16 acc / l (bfloat16 I/O)
  int num_partitions;
  int partition_tokens;  // tokens per partition, a multiple of the chunk
  int ws_stride;         // partial slots per (sequence, head) >= num_partitions
  // Shared-prefix (cascade) decode: the partitions cover tokens
  // [start_b, L_b) with start_b = prefix_lens[b] rounded down to a block;
  // slots num_partitions .. + ceil(start_b / prefix_chunk_tokens) - 1 hold
  // the prefix partials, which the merge adds.  Null for plain decode.
  const int32_t* prefix_lens;
  int prefix_chunk_tokens;
  int prefix_chunks;     // prefix slots per (sequence, head)
  int force_partials;    // write partials even with one partition
  // Shared-prefix decode whose suffixes fit one partition: the partition
  // kernel merges the prefix partials (complete before it starts) with its
  // own result and writes the output; no suffix partial, no merge kernel.
  int merge_prefix;
  float v_scale;         // output factor (E4M3 cache: V = code * v_scale)
  // Longest-first schedule (null: natural order): entry r is the (part *
  // num_seqs + b) item workgroups r * Hkv .. r * Hkv + Hkv - 1 take.
  const int32_t* order;
  // Longest-first without a plan kernel (plain decode, at most 64
  // sequences): each wave ranks its item itself (ranked_item).
  int inline_rank;
  // Host side only: `order` was written by an earlier kernel on the same
  // stream (the shared-prefix pass), so no plan kernel runs.
  int order_ready;
};

// First token of the partitions: 0, or the block-aligned shared prefix.
__device__ __forceinline__ int suffix_start(const DecodeParams& p, int b,
                                            int len) {
  if (p.prefix_lens == nullptr) return 0;
  int st = p.prefix_lens[b];
  st = st < 0 ? 0 : (st > len ? len : st);
  return st - st % kBlock;
}

// Prefix partials of a sequence whose partitions start at `start`.
__device__ __forceinline__ int prefix_partials(const DecodeParams& p, int start) {
  if (start <= 0 || p.prefix_chunks <= 0) return 0;
  const int n = (start + p.prefix_chunk_tokens - 1) / p.prefix_chunk_tokens;
  return n > p.prefix_chunks ? p.prefix_chunks : n;
}

__device__ __forceinline__ int clamp_len(const DecodeParams& p, int b) {
  int len = p.context_lens[b];
  len = len < 0 ? 0 : len;
  len = len > p.max_context_len ? p.max_context_len : len;
  const int cap = p.max_blocks_per_seq * kBlock;
  return len > cap ? cap : len;
}

// The item of rank r in a longest-first order of the (sequence, partition)
// items, found by one wave from the context lengths of at most 64
// sequences (lane b holds sequence b's), with the length of the item's
// sequence; item -1 past the last non-empty one.  Full partitions come
// first (sequence-major), then each sequence's last, partial one by
// decreasing length (ties by sequence), then the empty ones.  Every lane of
// the wave must call it; the result is wave-uniform.
struct RankedItem {
  int item, len;
};
__device__ __forceinline__ RankedItem ranked_item(const DecodeParams& p, int r) {
  const int lane = __lane_id();
  const int pt = p.partition_tokens;
  const int len = lane < p.num_seqs ? clamp_len(p, lane) : 0;
  const int full = min(len / pt, p.num_partitions);
  int incl = full;                                   // inclusive scan of `full`
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  const int num_full = __shfl(incl, kWave - 1, kWave);
  if (r < num_full) {
    const uint64_t m = __ballot(incl > r && incl - full <= r);
    const int b = __ffsll(static_cast<unsigned long long>(m)) - 1;
    const int part = r - __builtin_amdgcn_readlane(incl - full, b);
    return {part * p.num_seqs + b, __builtin_amdgcn_readlane(len, b)};
  }
  // A partial last partition has len % pt tokens (len <= num_partitions * pt).
  const int w = (lane < p.num_seqs && len % pt != 0) ? len % pt : -1;
  if (r - num_full >= __popcll(__ballot(w >= 0))) return {-1, 0};   // empty
  int rank = 0;
#pragma unroll 1
  for (int k = 0; k < kWave; ++k) {                  // uniform
    const int wk = __builtin_amdgcn_readlane(w, k);
    rank += (wk > w || (wk == w && k < lane)) ? 1 : 0;
  }
  const uint64_t m = __ballot(w >= 0 && rank == r - num_full);
  if (m == 0) return {-1, 0};
  const int b = __ffsll(static_cast<unsigned long long>(m)) - 1;
  const int lb = __builtin_amdgcn_readlane(len, b);
  return {(lb / pt) * p.num_seqs + b, lb};
}

__device__ __forceinline__ uint2 buf_ld8_nt(__amdgpu_buffer_rsrc_t r,
                                            uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCacheNT);
  return make_uint2(v[0], v[1]);
}

// Merged output of one (sequence, query head) at dimension d: weights
// 2^(m_p - m*) rescale each partial's sum and output; the result is their
// ratio.  Slots 0 .. np - 1 hold this call's partitions, slots
// num_partitions .. num_partitions + npre - 1 the prefix partials; (m0,
// l0, o0) is a partial already in registers (empty by default).
template <typename T, int D>
__device__ __forceinline__ float merge_head(const DecodeParams& p, int64_t head,
                                            int d, int np, int npre,
                                            float m0 = -INFINITY, float l0 = 0.f,
                                            float o0 = 0.f) {
  const float* mx = p.ws_max + head * p.ws_stride;
  const float* sm = p.ws_sum + head * p.ws_stride;
  const float* ac = p.ws_acc + head * p.ws_stride * D + d;
  const uint16_t* ach = p.ws_acc_h + head * p.ws_stride * D + d;
  auto slot = [&](int i) { return i < np ? i : p.num_partitions + (i - np); };
  // Partial k as (sum l, unnormalised output l * o): fp32 acc for fp32 I/O,
  // binary16 o (scaled by 2^-16 where l is stored negated) for bfloat16.
  return merge_partials<8>(np + npre, [&](int i, float& m, float& l, float& acc)
                                          __attribute__((always_inline)) {
    const int k = slot(i);
    m = mx[k];
    const float lraw = sm[k];
    if constexpr (sizeof(T) == 2) {
      const float o = f16_to_f32(ach[static_cast<int64_t>(k) * D]);
      l = fabsf(lraw);
      acc = l * (lraw < 0.f ? o * kPartialGrow : o);
    } else {
      l = lraw;
      acc = ac[static_cast<int64_t>(k) * D];
    }
  }, m0, l0, o0);
}

// The same merge (merge_partials, one group) over up to kPre prefix
// partials already in registers: maxima pm, stored sums pl (negative: the
// output is stored scaled), binary16 outputs po; (m, l, o) is this
// partition's partial.  Slots past n are dropped by index.
template <int kPre>
__device__ __forceinline__ float merge_prefetched(int n, const float (&pm)[kPre],
                                                  const float (&pl)[kPre],
                                                  const uint16_t (&po)[kPre], float m,
                                                  float l, float o) {
  float mv[kPre], sv[kPre], av[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const bool in = u < n;
    const float lr = fabsf(pl[u]);
    const float ov = f16_to_f32(po[u]);
    mv[u] = in ? pm[u] : -INFINITY;
    sv[u] = in ? lr : 0.f;
    av[u] = in ? lr * (pl[u] < 0.f ? ov * kPartialGrow : ov) : 0.f;
  }
  float gm = m;
#pragma unroll
  for (int u = 0; u < kPre; ++u) gm = fmaxf(gm, mv[u]);
  if (gm != -INFINITY) {
    if (gm > m) {
      const float a = m == -INFINITY ? 0.f : fast_exp2(m - gm);
      l *= a;
      o *= a;
      m = gm;
    }
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      if (u < n) {
        const float w = fast_exp2(mv[u] - m);
        l = fmaf(w, sv[u], l);
        o = fmaf(w, av[u], o);
      }
    }
  }
  return (m == -INFINITY || !(l > 0.f)) ? 0.f : o / l;
}

template <typename T, int D, int G, int C, bool F8>
__global__ __launch_bounds__(kThreads) __attribute__((
    amdgpu_waves_per_eu(DecodeShape<T, D, G, C, F8>::kMinWaves, 8))) void
decode_partition_kernel(
    DecodeParams p) {
  using S = DecodeShape<T, D, G, C, F8>;
  using KL = typename S::K;
  using VL = typename S::V;
  constexpr int kSteps = S::kBlocks / kWaves;  // blocks per wave per chunk
  constexpr int kDepth = S::kDepth;
  __shared__ float s_w[C * G];        // chunk logits, then fp32 weights: [t][h]
  __shared__ uint32_t s_wp[S::kPairPv ? C / 2 * G : 1];  // bf16 weight pairs
  __shared__ float s_rmax[kWaves][G];
  __shared__ float s_rsum[kWaves][G];
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[G];
  __shared__ float s_mrun[G], s_lrun[G];   // running max and sum per head

  // Workgroup i runs on XCD i % 8.  KV head varies fastest, then sequence,
  // then partition: every XCD gets the same mix of heads, sequences and
  // partitions (a partition-fastest order would hand partition p of every
  // sequence to XCD p % 8 -- the always-full first partitions to one XCD,
  // the mostly empty last ones to another), and the full early partitions
  // are dispatched before the sparse late ones.
  const int kvh = blockIdx.x % p.num_kv_heads;
  int rest = blockIdx.x / p.num_kv_heads;
  int ranked_len = -1;
  if (p.inline_rank) {
    const RankedItem it = ranked_item(p, rest);
    if (it.item < 0) return;                                          // uniform
    rest = __builtin_amdgcn_readfirstlane(it.item);
    ranked_len = __builtin_amdgcn_readfirstlane(it.len);
  } else if (p.order != nullptr) {
    rest = load_uniform_i32(p.order, rest);
    if (rest < 0 || rest >= p.num_seqs * p.num_partitions) return;   // uniform
  }
  const int b = rest % p.num_seqs;
  const int part = rest / p.num_seqs;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const bool single = p.num_partitions == 1 && !p.force_partials;

  const int len = ranked_len >= 0 ? ranked_len : clamp_len(p, b);
  const int t0 = suffix_start(p, b, len) + part * p.partition_tokens;
  const int head0 = kvh * G;
  const int row_stride = p.num_kv_heads * S::kCacheRow;   // bytes per slot
  const int64_t blk_bytes = static_cast<int64_t>(kBlock) * row_stride;

  if (t0 >= len) {
    // Nothing to attend.  A single-partition launch owns the output row and
    // writes zeros for an empty context (batch padding); with the prefix
    // merge the output is the prefix partials' alone; otherwise the merge
    // pass never reads this partition.
    if (part == 0 && (single || p.merge_prefix)) {
      const int npre = single ? 0 : prefix_partials(p, t0);
      for (int i = tid; i < G * D; i += kThreads) {
        const int64_t head = static_cast<int64_t>(b) * p.num_heads + head0 + i / D;
        const float o = npre > 0 ? merge_head<T, D>(p, head, i % D, 0, npre) : 0.f;
        store_out<T>(reinterpret_cast<T*>(p.out) + head * D + i % D, o * p.v_scale);
      }
    }
    return;
  }
  const int part_end = min(len, t0 + p.partition_tokens);
  const int32_t* brow = p.block_tables +
                        static_cast<int64_t>(b) * p.max_blocks_per_seq;

  // Shared-prefix decode whose suffix is this one partition (bf16, one head
  // per wave, at most kPre prefix partials): the prefix pass finished before
  // this kernel started, so the loads of the partials this partition merges
  // with at the end go out now, ahead of the K/V stream, instead of after
  // it.  Wave w holds head head0 + w's; maxima and sums are uniform.  Only
  // the shapes with registers to spare (3 waves per SIMD, G = 4): at 5
  // waves per SIMD the G <= 2 shapes would spill.
  constexpr bool kPrefetch = sizeof(T) == 2 && !F8 && G == 4 && G <= kWaves;
  constexpr int kPre = 8;
  constexpr int kDpl = D / kWave;   // output dimensions per lane
  float pre_m[kPre], pre_l[kPre];
  uint16_t pre_o[kDpl][kPre];
  int npre_held = -1;               // partials held in registers (-1: none)
  if constexpr (kPrefetch) {
    if (p.merge_prefix && wave < G) {
      const int npre = prefix_partials(p, t0);
      if (npre >= 1 && npre <= kPre) {
        const int64_t slot0 =
            (static_cast<int64_t>(b) * p.num_heads + head0 + wave) * p.ws_stride +
            p.num_partitions;
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
          const int64_t slot = slot0 + (k < npre ? k : npre - 1);
          pre_m[k] = p.ws_max[slot];
          pre_l[k] = p.ws_sum[slot];
#pragma unroll
          for (int e = 0; e < kDpl; ++e)
            pre_o[e][k] = p.ws_acc_h[slot * D + e * kWave + lane];
        }
        npre_held = npre;
      }
    }
  }

  // Running softmax state of the partition (max and sum per head) lives in
  // LDS; each lane keeps its share of the unnormalised output.
  if (tid < G) {
    s_mrun[tid] = -INFINITY;
    s_lrun[tid] = 0.f;
  }
  float acc[G][VL::kCpl][S::kEpc];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int cc = 0; cc < VL::kCpl; ++cc)
#pragma unroll
      for (int x = 0; x < S::kEpc; ++x) acc[h][cc][x] = 0.f;

  // The partition is walked in chunks of C tokens whose logits fit in LDS.
  // Each chunk: logits, the chunk max, weights against the running max, and
  // the weighted sum of V; the output so far is rescaled when the max grows.
  // A partition of several chunks writes one partial result instead of one
  // per chunk: partial writes interleaved with the K/V stream cost HBM
  // read bandwidth far beyond their own size.
  for (int tc0 = t0; tc0 < part_end; tc0 += C) {
    const int ntok = min(C, part_end - tc0);
    const int nblk = (ntok + kBlock - 1) / kBlock;
    // The lane-dependent offsets below are recomputed in every chunk (a few
    // integer ops): hoisted out of the loop, the per-step addresses of the
    // unrolled steps would all stay live in registers and spill.
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    // Lane (krs, ke) of the QK layout: token i * KL::kRpi + krs of a block,
    // chunks cc * KL::kLpr + ke of its row.
    const int krs = ln / KL::kLpr;
    const int ke = ln % KL::kLpr;
    // (F8: lane ke's virtual chunks are ke * kCpl + cc, whose codes are
    // one contiguous 8 * kCpl-byte piece of the row.)
    uint32_t koff[KL::kTpl][KL::kCpl];
#pragma unroll
    for (int i = 0; i < KL::kTpl; ++i)
#pragma unroll
      for (int cc = 0; cc < KL::kCpl; ++cc)
        koff[i][cc] = F8 ? (i * KL::kRpi + krs) * row_stride + kvh * S::kCacheRow +
                               ke * (8 * KL::kCpl)
                         : (i * KL::kRpi + krs) * row_stride + kvh * S::kRow +
                               (cc * KL::kLpr + ke) * 16;
    // Lane (vrs, ve) of the PV layout.
    const int vrs = ln / VL::kLpr;
    const int ve = ln % VL::kLpr;
    uint32_t voff[VL::kTpl][VL::kCpl];
#pragma unroll
    for (int i = 0; i < VL::kTpl; ++i)
#pragma unroll
      for (int cc = 0; cc < VL::kCpl; ++cc)
        voff[i][cc] = F8 ? (i * VL::kRpi + vrs) * row_stride + kvh * S::kCacheRow +
                               (cc * VL::kLpr + ve) * 8
                         : (i * VL::kRpi + vrs) * row_stride + kvh * S::kRow +
                               (cc * VL::kLpr + ve) * 16;

    // q of the group's heads, in the QK lane layout.  Loaded again for every
    // chunk (the lines stay in cache) rather than held across the chunk
    // loop, where it would cost 32 registers during the PV pass.
    uint4 qreg[KL::kCpl][G];
    {
      const char* qbase = reinterpret_cast<const char*>(p.q) +
                          (static_cast<int64_t>(b) * p.num_heads + head0) * S::kRow;
#pragma unroll
      for (int cc = 0; cc < KL::kCpl; ++cc)
#pragma unroll
        for (int h = 0; h < G; ++h)
          qreg[cc][h] = ld16(qbase + h * S::kRow +
                             (F8 ? ke * KL::kCpl + cc : cc * KL::kLpr + ke) * 16);
    }

    // Step s of a wave covers block j = wave + s * kWaves of the chunk.  One
    // vector load brings the wave's block ids (lane s holds step s's id);
    // each step takes its id into SGPRs with a readlane.  Valid tokens of a
    // block: 0 past nblk or for an id outside the pool.
    const int32_t* btab = brow + tc0 / kBlock;
    int my_id = 0;
    if (lane < kSteps && wave + lane * kWaves < nblk) my_id = btab[wave + lane * kWaves];
    int blk_off[kSteps];   // block id, 0 standing in for a bad one (uniform)
    int nval[kSteps];      // valid tokens of the block (uniform)
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int j = wave + s * kWaves;
      const int blk = __builtin_amdgcn_readlane(my_id, s);
      const bool ok = j < nblk && blk >= 0 && blk < p.num_blocks;
      nval[s] = ok ? min(kBlock, ntok - j * kBlock) : 0;
      blk_off[s] = ok ? blk : 0;
    }
    auto rsrc = [&](const char* cache, int s) {
      return block_rsrc(cache + static_cast<int64_t>(blk_off[s]) * blk_bytes,
                        nval[s] * row_stride);
    };

    // ---- pass 1: logits ---------------------------------------------------
    uint4 kr[kSteps][KL::kTpl][KL::kCpl];
    uint4 kr8[kSteps][KL::kTpl];          // F8: the codes of both chunks
    static_assert(!F8 || KL::kCpl == 2, "E4M3 K: two virtual chunks per lane");
    auto load_k = [&](int s) {
      const auto r = rsrc(p.k_cache, s);
#pragma unroll
      for (int i = 0; i < KL::kTpl; ++i) {
        if constexpr (F8) {
          kr8[s][i] = buf_ld16_nt(r, koff[i][0]);
        } else {
#pragma unroll
          for (int cc = 0; cc < KL::kCpl; ++cc) kr[s][i][cc] = buf_ld16_nt(r, koff[i][cc]);
        }
      }
    };
    auto k_chunk = [&](int s, int i, int cc) __attribute__((always_inline)) {
      if constexpr (F8) {
        return cc == 0 ? e4m3x8_to_bf16(kr8[s][i].x, kr8[s][i].y)
                       : e4m3x8_to_bf16(kr8[s][i].z, kr8[s][i].w);
      } else {
        return kr[s][i][cc];
      }
    };
    float mloc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
    auto logits = [&](int s) {
      const int j = wave + s * kWaves;
      const int nvalid = nval[s];
#pragma unroll
      for (int i = 0; i < KL::kTpl; ++i) {
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h] = 0.f;
#pragma unroll
        for (int cc = 0; cc < KL::kCpl; ++cc) ChunkDot<T, G>::run(k_chunk(s, i, cc), qreg[cc], sc);
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h] = row_sum<KL::kLpr>(sc[h]) * p.scale_log2;
        const int tb = i * KL::kRpi + krs;     // token inside the block
        if (nvalid < kBlock) {                 // uniform: partial or bad block
#pragma unroll
          for (int h = 0; h < G; ++h) sc[h] = tb < nvalid ? sc[h] : -INFINITY;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) mloc[h] = fmaxf(mloc[h], sc[h]);
        if (ke == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) s_w[(j * kBlock + tb) * G + h] = sc[h];
        }
      }
    };
    // kDepth - 1 blocks ahead: every load is issued unconditionally (past
    // the context it reads nothing), so the wait before each step is a fixed
    // count.
#pragma unroll
    for (int s = 0; s < kDepth - 1 && s < kSteps; ++s) load_k(s);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (wave + s * kWaves >= nblk) break;
      if (s + kDepth - 1 < kSteps) load_k(s + kDepth - 1);
      // Keep the prefetch here: without a memory clobber the compiler may
      // sink a load down to the step that uses it.
      __asm__ volatile("" ::: "memory");
      logits(s);
    }

    // ---- first V blocks in flight; softmax over the chunk -----------------
    uint4 vr[kSteps][VL::kTpl][VL::kCpl];
    uint2 vr8[kSteps][VL::kTpl];          // F8: the codes of the chunk
    static_assert(!F8 || VL::kCpl == 1, "E4M3 V: one virtual chunk per lane");
    auto load_v = [&](int s) {
      const auto r = rsrc(p.v_cache, s);
#pragma unroll
      for (int i = 0; i < VL::kTpl; ++i) {
        if constexpr (F8) {
          vr8[s][i] = buf_ld8_nt(r, voff[i][0]);
        } else {
#pragma unroll
          for (int cc = 0; cc < VL::kCpl; ++cc) vr[s][i][cc] = buf_ld16_nt(r, voff[i][cc]);
        }
      }
    };
    auto v_chunk = [&](int s, int i, int cc) __attribute__((always_inline)) {
      if constexpr (F8) {
        (void)cc;
        return e4m3x8_to_bf16(vr8[s][i].x, vr8[s][i].y);
      } else {
        return vr[s][i][cc];
      }
    };
#pragma unroll
    for (int s = 0; s < kDepth - 1 && s < kSteps; ++s) load_v(s);

#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m = wave_max(mloc[h]);
      if (lane == 0) s_rmax[wave][h] = m;
    }
    __syncthreads();
    if (tid < G) {
      float m = s_rmax[0][tid];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_rmax[w][tid]);
      s_m[tid] = m;
    }
    __syncthreads();
    // New running max per head and the factor that rescales what the
    // previous chunks accumulated (1 when the max did not move, including
    // the all-masked -inf case; 0 for the first chunk, whose acc is 0).
    float m_new[G], alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m_old = s_mrun[h];
      m_new[h] = fmaxf(m_old, s_m[h]);
      alpha[h] = m_new[h] == m_old ? 1.f : fast_exp2(m_old - m_new[h]);
    }
    {
      // Weights 2^(s - m); masked slots (-inf) become 0, and a head whose
      // every token was masked (m = -inf) gets all-zero weights.  kThreads
      // is a multiple of G, so each thread always works on the same head.
      const int h = tid % G;
      const float m = m_new[h];
      float acc_l = 0.f;
      auto weight = [&](float x) {
        return (m == -INFINITY || x == -INFINITY) ? 0.f : fast_exp2(x - m);
      };
      if constexpr (S::kPairPv) {
        // Pair q of block j joins the lane's tokens t and t + VL::kRpi of
        // the PV layout; the pair is stored as two bfloat16 (low = t).
        for (int i = tid; i < nblk * S::kPairsPerBlock * G; i += kThreads) {
          const int pr = i / G;
          const int j = pr / S::kPairsPerBlock;
          const int q = pr % S::kPairsPerBlock;
          const int ta = j * kBlock + (q / VL::kRpi) * 2 * VL::kRpi + q % VL::kRpi;
          const float wa = weight(s_w[ta * G + h]);
          const float wb = weight(s_w[(ta + VL::kRpi) * G + h]);
          const uint32_t wp = static_cast<uint32_t>(f32_to_bf16_rne(wa)) |
                              (static_cast<uint32_t>(f32_to_bf16_rne(wb)) << 16);
          s_wp[i] = wp;
          // The sum takes the rounded weights P V uses (one dot2 against
          // a pair of bfloat16 ones), so numerator and denominator agree.
          acc_l = dot2_bf16(wp, kBf16PairOne, acc_l);
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
      if (lane < G) s_rsum[wave][lane] = acc_l;
    }
    __syncthreads();
    // Every thread has read the old running max; thread h moves head h's
    // state on (the next readers come after the next chunk's barriers).
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (tid == h) {
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) l += s_rsum[w][h];
        s_lrun[h] = s_lrun[h] * alpha[h] + l;
        s_mrun[h] = m_new[h];
      }
#pragma unroll
      for (int cc = 0; cc < VL::kCpl; ++cc)
#pragma unroll
        for (int x = 0; x < S::kEpc; ++x) acc[h][cc][x] *= alpha[h];
    }

    // ---- pass 2: weighted sum of V ---------------------------------------
    // Slots past the context read as zeros (see block_rsrc) and have weight
    // 0, so NaN or garbage there cannot reach the sums.
    auto accumulate = [&](int s) {
      const int j = wave + s * kWaves;
      if constexpr (S::kPairPv) {
#pragma unroll
        for (int pi = 0; pi < VL::kTpl / 2; ++pi) {
          const int q = pi * VL::kRpi + vrs;   // pair index inside the block
          uint32_t wp[G];
#pragma unroll
          for (int h = 0; h < G; ++h) wp[h] = s_wp[(j * S::kPairsPerBlock + q) * G + h];
#pragma unroll
          for (int cc = 0; cc < VL::kCpl; ++cc) {
            // pr[2 dw] = (token 0, token 1) of dimension 2 dw, pr[2 dw + 1]
            // of dimension 2 dw + 1, as bfloat16 pairs.
            uint32_t pr[8];
            if constexpr (F8) {
              // Interleave the two tokens' codes first (one byte permute per
              // four codes), then each conversion yields a pair directly.
              const uint2 a = vr8[s][2 * pi];
              const uint2 c = vr8[s][2 * pi + 1];
              const uint32_t il[4] = {__builtin_amdgcn_perm(c.x, a.x, 0x05010400u),
                                      __builtin_amdgcn_perm(c.x, a.x, 0x07030602u),
                                      __builtin_amdgcn_perm(c.y, a.y, 0x05010400u),
                                      __builtin_amdgcn_perm(c.y, a.y, 0x07030602u)};
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                pr[2 * k] = e4m3x2_to_bf16<false>(il[k]);
                pr[2 * k + 1] = e4m3x2_to_bf16<true>(il[k]);
              }
            } else {
              const uint4 x = v_chunk(s, 2 * pi, cc);
              const uint4 y = v_chunk(s, 2 * pi + 1, cc);
              const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
              const uint32_t ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
              for (int dw = 0; dw < 4; ++dw) {
                pr[2 * dw] = pack_lo(xs[dw], ys[dw]);
                pr[2 * dw + 1] = pack_hi(xs[dw], ys[dw]);
              }
            }
#pragma unroll
            for (int dw = 0; dw < 4; ++dw) {
              const uint32_t lo = pr[2 * dw];
              const uint32_t hi = pr[2 * dw + 1];
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
            Widen<T>::run(v_chunk(s, i, cc), v);
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
              for (int x = 0; x < S::kEpc; ++x)
                acc[h][cc][x] = fmaf(w[h], v[x], acc[h][cc][x]);
          }
        }
      }
    };
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (wave + s * kWaves >= nblk) break;
      if (s + kDepth - 1 < kSteps) load_v(s + kDepth - 1);
      __asm__ volatile("" ::: "memory");
      accumulate(s);
    }
    // The fp32 path reads its weights from s_w, which the next chunk's
    // logits overwrite.
    if constexpr (!S::kPairPv) {
      if (tc0 + C < part_end) __syncthreads();
    }
  }

  // Sum the row groups of the wave (same dimensions, different tokens) with
  // shuffles, then the waves through LDS.
  const int vrs = lane / VL::kLpr;
  const int ve = lane % VL::kLpr;
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

  // Head h is written by wave h % kWaves (lanes cover its D dimensions), so
  // a per-head decision is one wave vote.
#pragma unroll
  for (int h = wave; h < G; h += kWaves) {
    const int64_t head = static_cast<int64_t>(b) * p.num_heads + head0 + h;
    const float l = s_lrun[h];
    float ov[D / kWave];
#pragma unroll
    for (int e = 0; e < D / kWave; ++e) {
      ov[e] = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) ov[e] += s_acc[w][h][e * kWave + lane];
    }
    if (single) {
      T* out = reinterpret_cast<T*>(p.out) + head * D;
#pragma unroll
      for (int e = 0; e < D / kWave; ++e)
        store_out<T>(out + e * kWave + lane, l > 0.f ? ov[e] / l * p.v_scale : 0.f);
      continue;
    }
    if (p.merge_prefix) {
      // This partition (the whole suffix) joins the prefix partials.
      T* out = reinterpret_cast<T*>(p.out) + head * D;
      if (kPrefetch && npre_held >= 0) {   // h == wave: one head per wave
#pragma unroll
        for (int e = 0; e < D / kWave; ++e)
          store_out<T>(out + e * kWave + lane,
                       merge_prefetched<kPre>(npre_held, pre_m, pre_l, pre_o[e],
                                              s_mrun[h], l, ov[e]) * p.v_scale);
        continue;
      }
      const int npre = prefix_partials(p, t0);
#pragma unroll
      for (int e = 0; e < D / kWave; ++e)
        store_out<T>(out + e * kWave + lane,
                     merge_head<T, D>(p, head, e * kWave + lane, 0, npre, s_mrun[h], l,
                                      ov[e]) * p.v_scale);
      continue;
    }
    const int64_t slot = head * p.ws_stride + part;
    if constexpr (sizeof(T) == 2) {
      // Normalised binary16 partial (see kPartialBig).
      bool big = false;
#pragma unroll
      for (int e = 0; e < D / kWave; ++e) {
        ov[e] = l > 0.f ? ov[e] / l : 0.f;
        big = big || fabsf(ov[e]) >= kPartialBig;
      }
      big = __any(big);
#pragma unroll
      for (int e = 0; e < D / kWave; ++e)
        p.ws_acc_h[slot * D + e * kWave + lane] = partial_f16(ov[e], big);
      if (lane == 0) {
        p.ws_max[slot] = s_mrun[h];
        p.ws_sum[slot] = big ? -l : l;
      }
    } else {
#pragma unroll
      for (int e = 0; e < D / kWave; ++e) p.ws_acc[slot * D + e * kWave + lane] = ov[e];
      if (lane == 0) {
        p.ws_max[slot] = s_mrun[h];
        p.ws_sum[slot] = l;
      }
    }
  }
}

// The same for plain decode with at most 8 partitions: every slot's loads
// are issued together with the context length's, not after it.  Slots past
// the sequence's partitions hold stale values from other calls; they are
// dropped by index (selects, never arithmetic on them).
template <typename T, int D>
__device__ __forceinline__ float merge_head_all(const DecodeParams& p, int64_t head,
                                                int d, int b) {
  constexpr int kMax = 8;
  const float* mx = p.ws_max + head * p.ws_stride;
  const float* sm = p.ws_sum + head * p.ws_stride;
  // All loads first, in one round trip: the outputs per slot (clamped to
  // the partitions), then maxima and sums as 8 contiguous slots (two wide
  // scalar loads; past this head's partitions they are the next head's
  // slots, or the next workspace array after the last head -- inside the
  // workspace), then the context length.
  uint16_t oh[kMax];
  float of[kMax];
#pragma unroll
  for (int u = 0; u < kMax; ++u) {
    const int k = u < p.num_partitions ? u : p.num_partitions - 1;
    if constexpr (sizeof(T) == 2)
      oh[u] = p.ws_acc_h[(head * p.ws_stride + k) * D + d];
    else
      of[u] = p.ws_acc[(head * p.ws_stride + k) * D + d];
  }
  // Read as vector loads (an opaque per-lane zero offset): all of them are
  // counted by vmcnt and issue together with the outputs'.
  int z = 0;
  __asm__ volatile("" : "+v"(z));
  float mv[kMax], lr[kMax];
#pragma unroll
  for (int u = 0; u < kMax; ++u) {
    mv[u] = mx[u + z];
    lr[u] = sm[u + z];
  }
  const int len = clamp_len(p, b);
  // Scheduling fence: every load above issues before the arithmetic below.
  __builtin_amdgcn_sched_barrier(0);
  float lv[kMax], av[kMax];
#pragma unroll
  for (int u = 0; u < kMax; ++u) {
    if constexpr (sizeof(T) == 2) {
      const float o = f16_to_f32(oh[u]);
      lv[u] = fabsf(lr[u]);
      av[u] = lv[u] * (lr[u] < 0.f ? o * kPartialGrow : o);
    } else {
      lv[u] = lr[u];
      av[u] = of[u];
    }
  }
  int np = (len + p.partition_tokens - 1) / p.partition_tokens;
  np = np > p.num_partitions ? p.num_partitions : np;
  float gm = -INFINITY;
#pragma unroll
  for (int u = 0; u < kMax; ++u) gm = fmaxf(gm, u < np ? mv[u] : -INFINITY);
  if (gm == -INFINITY) return 0.f;
  float l = 0.f, o = 0.f;
#pragma unroll
  for (int u = 0; u < kMax; ++u) {
    const bool in = u < np;
    const float w = in ? fast_exp2(mv[u] - gm) : 0.f;
    l = fmaf(w, in ? lv[u] : 0.f, l);
    o = fmaf(w, in ? av[u] : 0.f, o);
  }
  return l > 0.f ? o / l : 0.f;
}

// Merge pass: one workgroup per (query head, sequence), one thread per
// dimension.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeParams p) {
  const int partition_tokens = p.partition_tokens;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  if (p.prefix_lens == nullptr && p.num_partitions <= 8) {
    const int64_t head = static_cast<int64_t>(b) * p.num_heads + h;
    store_out<T>(reinterpret_cast<T*>(p.out) + head * D + d,
                 merge_head_all<T, D>(p, head, d, b) * p.v_scale);
    return;
  }
  const int len = clamp_len(p, b);
  const int start = suffix_start(p, b, len);
  int np = (len - start + partition_tokens - 1) / partition_tokens;
  np = np > p.num_partitions ? p.num_partitions : np;   // bound violated
  const int64_t head = static_cast<int64_t>(b) * p.num_heads + h;
  T* out = reinterpret_cast<T*>(p.out) + head * D + d;
  store_out<T>(out, merge_head<T, D>(p, head, d, np, prefix_partials(p, start)) * p.v_scale);
}

// Longest-first schedule of the (sequence, partition) items: one workgroup
// counts the items per token count (in 16-token bins, the last bin shared
// by everything longer), then writes them longest first.  With contexts of
// mixed lengths the partial and empty partitions otherwise start last and
// leave the tail of the grid to a few long ones.  Items of equal weight
// land in any order; the results do not depend on the schedule.
constexpr int kPlanThreads = 1024;
constexpr int kPlanBins = 1024;

__device__ __forceinline__ int plan_bin(const DecodeParams& p, int item) {
  const int b = item % p.num_seqs;
  const int part = item / p.num_seqs;
  const int len = clamp_len(p, b);
  int n = len - suffix_start(p, b, len) - part * p.partition_tokens;
  n = n < 0 ? 0 : (n > p.partition_tokens ? p.partition_tokens : n);
  const int bin = (n + kBlock - 1) / kBlock;
  return bin < kPlanBins ? bin : kPlanBins - 1;
}

// Items of the first kPlanRegItems rounds keep their bin in registers, so
// the second pass does not load the context lengths again.
constexpr int kPlanRegItems = 4;

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(
    DecodeParams p, int32_t* __restrict__ order) {
  __shared__ int bins[kPlanBins];
  __shared__ int wave_sum[kPlanThreads / kWave];
  longest_first_order<kPlanThreads, kPlanBins, kPlanRegItems>(
      p.num_seqs * p.num_partitions, [&](int item) { return plan_bin(p, item); },
      order, bins, wave_sum);
}

template <typename T, int D, int G, int C, bool F8>
hipError_t launch_typed(const DecodeParams& prm, int num_seqs, int num_kv_heads,
                        int num_heads, hipStream_t stream) {
  const int64_t wgs = static_cast<int64_t>(prm.num_partitions) * num_kv_heads * num_seqs;
  if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(wgs));
  if (prm.order != nullptr && !prm.order_ready) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream,
                       prm, const_cast<int32_t*>(prm.order));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_partition_kernel<T, D, G, C, F8>), grid,
                     dim3(kThreads), 0, stream, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (prm.num_partitions == 1 && !prm.force_partials) ||
      prm.merge_prefix)
    return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(num_heads, num_seqs),
                     dim3(D), 0, stream, prm);
  return hipGetLastError();
}

template <typename T, int D, int C, bool F8 = false>
hipError_t dispatch_group(const DecodeParams& prm, int num_seqs,
                          int num_kv_heads, int num_heads, hipStream_t s) {
  switch (num_heads / num_kv_heads) {
    case 1: return launch_typed<T, D, 1, C, F8>(prm, num_seqs, num_kv_heads, num_heads, s);
    case 2: return launch_typed<T, D, 2, C, F8>(prm, num_seqs, num_kv_heads, num_heads, s);
    case 4: return launch_typed<T, D, 4, C, F8>(prm, num_seqs, num_kv_heads, num_heads, s);
    case 8: return launch_typed<T, D, 8, C, F8>(prm, num_seqs, num_kv_heads, num_heads, s);
    default: return hipErrorInvalidValue;
  }
}

// Tokens per chunk: the logits of one chunk sit in LDS.
constexpr int kChunkTokens = 512;
// A partition spans one or more chunks.  Fewer, longer partitions write
// fewer partial results (which slow the K/V stream far beyond their own
// bytes) but leave fewer workgroups to balance; the plan takes the longest
// partitions that still give at least this many workgroups.
constexpr int64_t kTargetWorkgroups = 8192;
constexpr int kMaxChunksPerPartition = 16;
// Prefix pass of the shared-prefix decode: about this many workgroups.
constexpr int64_t kPrefixTargetWorkgroups = 128;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// The longest-first schedule pays for its plan kernel (a few microseconds)
// only on grids of several partitions and well over one wave of
// workgroups.  Appends the order array to a multi-partition plan's
// workspace; returns whether the plan uses one.
constexpr int64_t kOrderMinWorkgroups = 4096;
constexpr int kInlineRankSeqs = kWave;
bool plan_order(DecodePlan& plan, int num_seqs, int num_kv_heads) {
  const int64_t wgs = static_cast<int64_t>(num_seqs) * num_kv_heads * plan.num_partitions;
  plan.use_order = plan.num_partitions > 1 && wgs >= kOrderMinWorkgroups;
  if (plan.use_order && plan.workspace_bytes > 0) {
    plan.off_order = plan.workspace_bytes;
    plan.workspace_bytes += align256(static_cast<size_t>(num_seqs) *
                                     plan.num_partitions * sizeof(int32_t));
  }
  return plan.use_order;
}

hipError_t dispatch_decode(const DecodeParams& prm, const DecodeArgs& a,
                           hipStream_t stream) {
  constexpr int P = kChunkTokens;
  if (a.fp8_cache) {   // E4M3 cache, bf16 q / out, head_dim 128 (checked by the caller)
    return dispatch_group<bf16_t, 128, P, true>(prm, a.num_seqs, a.num_kv_heads,
                                                a.num_heads, stream);
  }
  if (a.bf16) {
    if (a.head_dim == 128)
      return dispatch_group<bf16_t, 128, P>(prm, a.num_seqs, a.num_kv_heads, a.num_heads, stream);
    return dispatch_group<bf16_t, 64, P>(prm, a.num_seqs, a.num_kv_heads, a.num_heads, stream);
  }
  if (a.head_dim == 128)
    return dispatch_group<float, 128, P>(prm, a.num_seqs, a.num_kv_heads, a.num_heads, stream);
  return dispatch_group<float, 64, P>(prm, a.num_seqs, a.num_kv_heads, a.num_heads, stream);
}

}  // namespace

DecodePlan plan_decode(int num_seqs, int num_heads, int num_kv_heads,
                       int head_dim, int max_context_len) {
  DecodePlan plan{};
  const int64_t groups = static_cast<int64_t>(num_seqs) * num_kv_heads;
  auto parts = [&](int tokens) {
    const int np = (max_context_len + tokens - 1) / tokens;
    return np < 1 ? 1 : np;
  };
  int chunks = 1;
  while (chunks < kMaxChunksPerPartition &&
         groups * parts(kChunkTokens * chunks * 2) >= kTargetWorkgroups)
    chunks *= 2;
  plan.partition_tokens = kChunkTokens * chunks;
  plan.num_partitions = parts(plan.partition_tokens);
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
  // Up to 64 sequences each wave ranks its own item (no plan kernel, no
  // order array; it costs a workgroup the one load its context length
  // costs anyway); larger batches get the plan kernel.
  if (num_seqs <= kInlineRankSeqs)
    plan.inline_rank = true;
  else
    plan_order(plan, num_seqs, num_kv_heads);
  return plan;
}

// Shared-prefix plan: the suffix partitions as for plain decode (over the
// longest suffix), plus prefix partials of prefix_chunk_tokens keys each.
// The chunk length aims at ~128 (256-row M-tile, key chunk) pieces of the
// prefix pass in all -- ~128 workgroups of the fp32 shapes, ~256 of the
// bf16 group-mode kernel, whose M-tiles hold 128 rows -- and is at least
// two 64-key tiles.  More, shorter chunks would shorten the pass but give
// every suffix workgroup more partials to merge.
SharedPrefixPlan plan_shared_prefix(int num_seqs, int num_heads,
                                    int num_kv_heads, int head_dim,
                                    int max_suffix_len, int max_prefix_len,
                                    int num_groups, int max_group_size) {
  SharedPrefixPlan plan{};
  plan.suffix = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim,
                            max_suffix_len);
  const int g = num_heads / num_kv_heads;
  const int64_t mtiles = (static_cast<int64_t>(max_group_size) * g + 255) / 256;
  const int64_t per_chunk = static_cast<int64_t>(num_groups) * mtiles * num_kv_heads;
  int64_t want = per_chunk > 0 ? (kPrefixTargetWorkgroups + per_chunk - 1) / per_chunk : 1;
  want = want < 1 ? 1 : want;
  int64_t ct = (max_prefix_len + want - 1) / want;
  ct = (ct + 63) / 64 * 64;
  ct = ct < 128 ? 128 : ct;
  plan.prefix_chunk_tokens = static_cast<int>(ct);
  plan.prefix_chunks = max_prefix_len > 0
                           ? static_cast<int>((max_prefix_len + ct - 1) / ct)
                           : 0;
  plan.total_slots = plan.suffix.num_partitions + plan.prefix_chunks;
  const size_t slots = static_cast<size_t>(num_seqs) * num_heads * plan.total_slots;
  plan.off_max = 0;
  plan.off_sum = align256(slots * sizeof(float));
  plan.off_acc = plan.off_sum + align256(slots * sizeof(float));
  plan.workspace_bytes =
      plan.off_acc + align256(slots * static_cast<size_t>(head_dim) * sizeof(float));
  plan.suffix.off_order = 0;
  plan.suffix.use_order = false;
  plan.suffix.inline_rank = false;   // the items start at the shared prefix
  // When the prefix pass runs, its last workgroup writes the suffix
  // schedule for free (the pass is on the critical path anyway); the suffix
  // workgroups then start longest first even with one partition, where
  // natural order left the longest suffixes to start late.  Otherwise the
  // plain-decode rule (a plan kernel for large multi-partition grids).
  plan.order_in_prefix = num_groups > 0 && max_group_size > 0 && plan.prefix_chunks > 0;
  if (plan.order_in_prefix) plan.suffix.use_order = true;
  else plan_order(plan.suffix, num_seqs, num_kv_heads);
  if (plan.suffix.use_order) {
    plan.suffix.off_order = plan.workspace_bytes;
    plan.workspace_bytes += align256(static_cast<size_t>(num_seqs) *
                                     plan.suffix.num_partitions * sizeof(int32_t));
  }
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
  prm.num_seqs = a.num_seqs;
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  prm.scale_log2 = a.scale * a.k_scale * kLog2e;
  prm.v_scale = a.v_scale;
  prm.num_partitions = plan.num_partitions;
  prm.partition_tokens = plan.partition_tokens;
  prm.ws_stride = plan.num_partitions;
  if (plan.num_partitions > 1) {
    char* ws = static_cast<char*>(a.workspace);
    prm.ws_max = reinterpret_cast<float*>(ws + plan.off_max);
    prm.ws_sum = reinterpret_cast<float*>(ws + plan.off_sum);
    prm.ws_acc = reinterpret_cast<float*>(ws + plan.off_acc);
    prm.ws_acc_h = reinterpret_cast<uint16_t*>(ws + plan.off_acc);
    if (plan.use_order) prm.order = reinterpret_cast<int32_t*>(ws + plan.off_order);
    prm.inline_rank = plan.inline_rank ? 1 : 0;
  }
  return dispatch_decode(prm, a, stream);
}

// Workspace of the no-allocation decode: a file-scope device array, of which
// every GPU that loads the library holds its own copy for the life of the
// process.  Host code never uses its name as an address (on the host it is
// only a stand-in for the symbol); the device address comes from
// hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = stream == nullptr ? hipGetDevice(&dev)
                                   : hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    // Look the symbol up with the stream's device current: each device has
    // its own copy of the array at its own address.
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_suffix(const DecodeArgs& a, const SharedPrefixPlan& plan,
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
  prm.num_seqs = a.num_seqs;
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  prm.scale_log2 = a.scale * a.k_scale * kLog2e;
  prm.v_scale = a.v_scale;
  prm.num_partitions = plan.suffix.num_partitions;
  prm.partition_tokens = plan.suffix.partition_tokens;
  prm.ws_stride = plan.total_slots;
  prm.prefix_lens = a.prefix_lens;
  prm.prefix_chunk_tokens = plan.prefix_chunk_tokens;
  prm.prefix_chunks = plan.prefix_chunks;
  prm.force_partials = 1;
  prm.merge_prefix = plan.suffix.num_partitions == 1 ? 1 : 0;
  char* ws = static_cast<char*>(a.workspace);
  prm.ws_max = reinterpret_cast<float*>(ws + plan.off_max);
  prm.ws_sum = reinterpret_cast<float*>(ws + plan.off_sum);
  prm.ws_acc = reinterpret_cast<float*>(ws + plan.off_acc);
  prm.ws_acc_h = reinterpret_cast<uint16_t*>(ws + plan.off_acc);
  if (plan.suffix.use_order) {
    prm.order = reinterpret_cast<int32_t*>(ws + plan.suffix.off_order);
    prm.order_ready = plan.order_in_prefix ? 1 : 0;
  }
  return dispatch_decode(prm, a, stream);
}

}  // namespace pa
