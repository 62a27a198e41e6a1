// Varlen chunked-prefill attention for gfx950, K/V read through block
// tables, QK^T and PV on MFMA.
//
// What it computes ("3.6 ModelRunner, CUDA Graph, and benchmarks", section 2,
// prepare_prefill; "10 Serving Engines", section 10.3): sequence b owns query
// rows cu_q[b] .. cu_q[b+1]-1 (Lq of them) and its first Lk = cu_k[b+1] -
// cu_k[b] cached tokens as keys; with the causal mask query row i sits at
// position Lk - Lq + i (a chunk continues after its history) and sees keys
// 0 .. Lk - Lq + i.  out = softmax(scale * q K^T) V per row and head.
//
// Design (MI355X-first; this is the dense contraction of the path):
//  * one workgroup per (M-tile, KV head, sequence): 8 waves and 256 rows
//    for bf16 (and fp32 with D = 64), 4 waves and 128 rows for fp32 with
//    D = 128; the G query heads of a KV head are packed into M (row m =
//    position m / G, head m % G), so a K/V tile loaded once serves all of
//    them and all waves;
//  * a one-workgroup plan kernel first sorts the (sequence, M-tile) items
//    by the key tiles they read, into the workspace, and workgroups take
//    them heaviest first: with mixed history lengths the longest items no
//    longer start late and set the tail;
//  * per 64-key tile the workgroup gathers K and V through the block table
//    straight into LDS with DMA loads (global_load_lds_dwordx4, issued from
//    inline assembly; one wave-uniform block lookup per 1 KiB load; 16-byte
//    chunks XOR-swizzled by row) into a ring of stages: tile kt + 2 is in
//    flight while tile kt is computed, with one barrier per tile;
//  * each wave computes S^T = K Q^T for its 32 rows with
//    v_mfma_f32_32x32x16_bf16 (fp32 I/O: v_mfma_f32_32x32x2_f32), Q^T held
//    in registers as the B operand.  In the accumulator layout every lane
//    owns one query row, so the online softmax is per lane plus one
//    exchange between the two lane halves (v_permlane32_swap), and the
//    probabilities already sit in the B-operand layout of O^T += V^T P^T --
//    no shuffles or LDS round trip for P; the V^T operand comes straight
//    from the row-major V tile through LDS transpose reads
//    (ds_read_b64_tr_b16);
//  * the softmax is VALU work next to the MFMAs and sets the pace, so its
//    common path is short: bf16 weights are taken against the running
//    reference max without a max scan, and the row sum over the packed
//    weights costs one dot2 per pair; the exact step (max scan, rescale of
//    O) runs on a row's first tile and when the max grows by more than 2^8;
//  * masking is by select: keys past the causal limit or past Lk get weight
//    exactly 0, and V rows past Lk are zeroed in LDS on the one tile that
//    crosses Lk (a NaN there would survive a multiplication by zero); only
//    tiles that cross the causal diagonal or Lk evaluate the mask.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_tile.h"

namespace pa {

namespace {

constexpr int kBlock = 16;         // tokens per cache block
constexpr int kMinBM = 128;        // fewest M rows per workgroup (any shape)
constexpr int kBN = 64;            // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));

// MFMA flavour per element type.  Operand layout of the 32x32xK shapes
// (checked on gfx950): lane l holds A[l % 32][(l / 32) * kPer + e] and
// B[(l / 32) * kPer + e][l % 32]; accumulator register r of lane l is
// C[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32].
template <typename T>
struct Mma;

template <>
struct Mma<bf16_t> {
  static constexpr int kK = 16;    // contraction length per instruction
  static constexpr int kPer = 8;   // elements per lane per operand
  typedef uint4 op_t;              // 8 packed bfloat16
  static __device__ __forceinline__ f32x16_v run(op_t a, op_t b, f32x16_v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8_v, a), __builtin_bit_cast(bf16x8_v, b), c,
        0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static constexpr int kK = 2;
  static constexpr int kPer = 1;
  typedef float op_t;
  static __device__ __forceinline__ f32x16_v run(op_t a, op_t b, f32x16_v c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <typename T, int D, bool kGroup = false>
struct PrefillShape {
  static constexpr int kElem = ElemTraits<T>::kBytes;
  static constexpr int kRow = D * kElem;                  // bytes per key row
  static constexpr int kChunks = kRow / 16;               // 16-byte chunks
  static constexpr bool kBf16 = sizeof(T) == 2;
  // K and V tiles: [kBN rows][kRow], rows unpadded; chunk p of row r holds
  // the row's chunk p ^ swizzle(r), so the lanes of one operand read touch
  // different banks: r % kChunks for K (32 rows, one chunk each), and
  // ((r % 4) << 2) for V (the transpose reads take 4 rows x 2 chunks per
  // 16 lanes).  Both are filled by LDS DMA (global_load_lds_dwordx4) into
  // a ring of kStages stages.
  static constexpr int kTile = kBN * kRow;
  // Where a wave fits in 256 registers (two per SIMD), 8 waves share each
  // K/V tile: 256 M rows per workgroup halve the gather traffic per row,
  // and with one workgroup per CU the LDS holds three K/V stages (tile
  // kt + 2 in flight while tile kt is computed).  fp32 with D = 128 needs
  // one wave per SIMD: 4 waves, two stages (128 KiB).
  // bf16 group mode (shared-prefix partials, a few key tiles per
  // workgroup, too few workgroups of 256 rows to fill the chip): 4 waves
  // and 128 rows, two stages (64 KiB), two workgroups per CU.
  static constexpr bool kSmallGroup = kGroup && kBf16;
  static constexpr int kWaves = kSmallGroup ? 4 : ((kBf16 || D == 64) ? 8 : 4);
  static constexpr int kStages = kWaves == 8 ? 3 : 2;
  static constexpr size_t kLds = 2 * kStages * static_cast<size_t>(kTile);
  static constexpr int kOccupancy = (kWaves == 8 || kSmallGroup) ? 2 : 1;   // waves per SIMD
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kBM = kWaves * 32;                 // M rows per workgroup
  static constexpr int kRowsPerDma = 1024 / kRow;         // rows per 1 KiB DMA
  static constexpr int kDmaPerWave = kTile / 1024 / kWaves;
  static constexpr int kLoadsPerTile = 2 * kDmaPerWave;   // per lane, K and V
  static constexpr int kQSteps = D / Mma<T>::kK;          // MFMAs per S tile
  static constexpr int kPvSteps = kBN / Mma<T>::kK;       // MFMAs per O tile
  static constexpr int kDTiles = D / 32;                  // O^T M-tiles
  static_assert(kTile % (1024 * kWaves) == 0, "tile DMA split");
  static_assert(kLds <= 160 * 1024, "LDS per CU");
  static_assert(kStages * kLoadsPerTile <= 63, "vmcnt range");
  static_assert(kBlock % (kDmaPerWave * kRowsPerDma) == 0,
                "a wave's DMA rows of a tile lie in one cache block");
  static_assert(kBlock % kRowsPerDma == 0, "a DMA load stays in one block");
};

struct PrefillParams {
  int mtiles;                // M-tiles per (sequence, KV head)
  int num_seqs;
  const int32_t* order;      // work items, heaviest first (null: see rank_inline)
  int rank_inline;           // no order: 1 = each workgroup ranks the items
                             // itself (at most one per thread), 0 = natural
  void* out;
  const char* q;
  int64_t total_q;
  const char* k_cache;
  const char* v_cache;
  int64_t num_blocks;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int max_seqlen_q;
  int max_seqlen_k;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  int num_heads;
  int num_kv_heads;
  float scale_log2;
  int causal;
  // Shared-prefix partials (group mode, the kGroup kernel): item b =
  // group * chunks + chunk; the group's members are query rows groups[2g]
  // .. + groups[2g + 1] - 1, its keys the first prefix_lens[groups[2g]]
  // tokens (rounded down to a block) of that first member's table,
  // non-causal, tiles chunk * chunk_tiles .. + chunk_tiles - 1.  Output:
  // partials in the decode workspace layout, slot slot0 + chunk of each
  // (row, head).
  const int32_t* groups;
  const int32_t* prefix_lens;
  int chunk_tiles;
  int chunks;
  float* ws_max;
  float* ws_sum;       // negative: the partial is stored scaled (bf16 I/O)
  float* ws_acc;       // fp32 acc (fp32 I/O)
  uint16_t* ws_acc_h;  // same memory: binary16 acc / sum (bfloat16 I/O)
  int ws_stride;
  int slot0;
  // Group mode: one more workgroup, the grid's last, writes the suffix
  // pass's schedule instead of a partial (null: none).  Entry r of
  // suffix_order is the (partition * order_seqs + b) item the suffix kernel's
  // workgroups r * Hkv .. r * Hkv + Hkv - 1 take, longest first; the weight
  // of an item is its suffix tokens in that partition, as the suffix kernel
  // clamps them (context_lens[b] to order_max_len and the block table,
  // starting at prefix_lens[b] rounded down to a block).
  int32_t* suffix_order;
  const int32_t* context_lens;
  int order_seqs;
  int order_parts;
  int order_part_tokens;
  int order_max_len;
};

// Keys an M-tile reads: the causal limit of its last row, or all lk.
__device__ __forceinline__ int tile_key_end(const SeqExtent& e, int g, int m0,
                                            int bm, int causal) {
  const int i_last = min(e.lq - 1, (m0 + bm - 1) / g);
  int kend = e.lk;
  if (causal) kend = min(e.lk, e.lk - e.lq + i_last + 1);
  return kend < 0 ? 0 : kend;
}

// Work of a (sequence, M-tile) item, the key of the longest-first order:
// the key tiles it reads plus one for its fixed cost; 0 for an M-tile past
// the sequence's rows.  Capped at kPlanBins - 1 (the plan kernel's bins).
constexpr int kPlanBins = 4096;
__device__ __forceinline__ int item_weight(const SeqExtent& e, int item,
                                           int mtiles, int bm, int group,
                                           int causal) {
  const int m0 = (item % mtiles) * bm;
  if (m0 >= e.lq * group) return 0;
  const int w = (tile_key_end(e, group, m0, bm, causal) + kBN - 1) / kBN + 1;
  return w < kPlanBins ? w : kPlanBins - 1;
}

// Weight bin of suffix item `item` (16-token bins, the last one shared by
// everything longer) for the suffix pass's longest-first schedule.
constexpr int kSuffixBins = 1024;
__device__ __forceinline__ int suffix_bin(const PrefillParams& p, int item) {
  const int b = item % p.order_seqs;
  const int part = item / p.order_seqs;
  int len = p.context_lens[b];
  len = len < 0 ? 0 : (len > p.order_max_len ? p.order_max_len : len);
  const int cap = p.max_blocks_per_seq * kBlock;
  len = len > cap ? cap : len;
  int st = p.prefix_lens[b];
  st = st < 0 ? 0 : (st > len ? len : st);
  st -= st % kBlock;
  int n = len - st - part * p.order_part_tokens;
  n = n < 0 ? 0 : (n > p.order_part_tokens ? p.order_part_tokens : n);
  const int bin = (n + kBlock - 1) / kBlock;
  return bin < kSuffixBins ? bin : kSuffixBins - 1;
}

template <int kChunks>
__device__ __forceinline__ int k_swz(int row) { return row % kChunks; }
template <int kChunks>
__device__ __forceinline__ int v_swz(int row) {
  return ((row % 4) << 2) & (kChunks - 1);
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]),
                                             pack_bf16x2(v[2], v[3]));
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// Weights exp2(scale * s - max) of one lane's 32 logits (two S^T tiles),
// rounded to bfloat16 and packed as the B operands of the four PV steps
// (step q: registers (q % 2) * 8 .. + 7 of tile q / 2); returns their sum,
// taken over the rounded values.
__device__ __forceinline__ float bf16_weights(const f32x16_v (&s)[2], float scale,
                                              float neg_max, uint4 (&pb)[4]) {
  const bf16x2_v ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  float sum[2] = {0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = (q % 2) * 8 + 2 * k;
      const float e0 = fast_exp2(fmaf(s[q / 2][r], scale, neg_max));
      const float e1 = fast_exp2(fmaf(s[q / 2][r + 1], scale, neg_max));
      w[k] = pack_bf16x2(e0, e1);
      sum[q / 2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w[k]),
                                                   ones, sum[q / 2], false);
    }
    pb[q] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return sum[0] + sum[1];
}

// Two waves per SIMD (8-wave shapes): one wave's softmax overlaps the
// other's MFMAs.  fp32 with D = 128 runs one wave per SIMD: no register cap
// there (it would only spill).
// kGroup: the shared-prefix partials (group mode), a kernel of its own, so
// that the varlen kernel carries none of its code.  It requests the first
// block ids and the Q rows before the prefix length arrives (neither
// depends on it).
template <typename T, int D, int G, bool kGroup>
__global__ __launch_bounds__((PrefillShape<T, D, kGroup>::kThreads)) __attribute__((amdgpu_waves_per_eu(
    PrefillShape<T, D, kGroup>::kOccupancy, PrefillShape<T, D, kGroup>::kOccupancy))) void
prefill_kernel(PrefillParams p) {
  using S = PrefillShape<T, D, kGroup>;
  using M = Mma<T>;
  typedef typename M::op_t op_t;
  extern __shared__ __align__(16) char smem[];
  // [K stage 0 .. kStages - 1][V stage 0 .. kStages - 1]

  // Workgroup lin takes work item order[lin / Hkv] (a (sequence, M-tile)
  // pair; the plan kernel lists them heaviest first, so the longest ones
  // start first and short ones fill the tail) for KV head lin % Hkv.  The
  // dispatcher deals workgroups to the 8 XCDs round robin (id % 8), each
  // with its own L2; with Hkv a multiple of 8 every M-tile of one (sequence,
  // KV head) group, which all read the same K/V tiles, runs on one XCD.
  const int lin = blockIdx.x;
  if (kGroup && p.suffix_order != nullptr && lin == static_cast<int>(gridDim.x) - 1) {
    // The suffix pass's schedule (it starts after this kernel ends), built
    // beside the prefix partials instead of by a plan kernel of its own.
    // LDS: the bins, then the wave totals.
    int* bins = reinterpret_cast<int*>(smem);
    longest_first_order<S::kThreads, kSuffixBins, 2>(
        p.order_seqs * p.order_parts, [&](int it) { return suffix_bin(p, it); },
        p.suffix_order, bins, bins + kSuffixBins);
    return;
  }
  const int kvh = lin % p.num_kv_heads;
  const int rank = lin / p.num_kv_heads;
  const int tid = threadIdx.x;
  int item = rank;
  if (p.order != nullptr) {
    item = load_uniform_i32(p.order, rank);
  } else if (p.rank_inline) {
    // Few items (at most one per thread): the workgroup finds the item of
    // rank `rank` itself, in the same order the plan kernel would give
    // (heaviest first, equal weights by index), without that kernel's
    // launch.  Scratch: the last V stage, which no DMA writes before the
    // tile loop's first barrier.
    int* s_w = reinterpret_cast<int*>(
        smem + (2 * S::kStages - 1) * static_cast<size_t>(S::kTile));
    auto weight = [&](int it) {
      const SeqExtent e = seq_extent(p.cu_q, p.cu_k, it / p.mtiles, p.max_seqlen_q,
                                     p.max_seqlen_k, p.total_q, p.max_blocks_per_seq);
      return item_weight(e, it, p.mtiles, S::kBM, G, p.causal);
    };
    item = inline_ranked_item<S::kThreads>(p.num_seqs * p.mtiles, rank, weight, s_w);
  }
  if (item < 0 || item >= p.num_seqs * p.mtiles) return;   // uniform
  const int b = item / p.mtiles;
  const int mtile = item % p.mtiles;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int j = lane % 32;                   // this lane's row inside the wave
  const int hh = lane / 32;                  // lane half

  SeqExtent ext;
  int kt0 = 0;              // first key tile of this workgroup
  int chunk = 0;            // group mode: which prefix partial
  int table_row = b;        // block-table row of the keys
  if constexpr (kGroup) {
    const int g = b / p.chunks;
    chunk = b % p.chunks;
    int first = p.groups[2 * g];
    int cnt = p.groups[2 * g + 1];
    first = first < 0 ? 0 : first;
    cnt = cnt < 0 ? 0 : (cnt > p.max_seqlen_q ? p.max_seqlen_q : cnt);
    if (first >= p.total_q) cnt = 0;
    else if (first + cnt > p.total_q) cnt = static_cast<int>(p.total_q - first);
    ext = {first, cnt, 0};   // keys: the prefix length, loaded below
    kt0 = chunk * p.chunk_tiles;
    table_row = first;
  } else {
    ext = seq_extent(p.cu_q, p.cu_k, b, p.max_seqlen_q, p.max_seqlen_k,
                     p.total_q, p.max_blocks_per_seq);
  }
  const int q0 = ext.q0;
  const int lq = ext.lq;
  const int mrows = lq * G;
  const int m0 = mtile * S::kBM;
  if (m0 >= mrows) return;                   // uniform over the workgroup

  // This lane's row: M row m -> query position i, head h.
  const int m = m0 + wave * 32 + j;
  const bool row_ok = m < mrows;
  const int i_pos = row_ok ? m / G : 0;
  const int h = m % G;

  // Q^T as the B operand: lane (j, hh) holds dims s * kK + hh * kPer + e.
  op_t qb[S::kQSteps];
  auto load_q = [&]() __attribute__((always_inline)) {
    const char* qrow = p.q + ((static_cast<int64_t>(q0) + i_pos) * p.num_heads +
                              kvh * G + h) * S::kRow;
#pragma unroll
    for (int s = 0; s < S::kQSteps; ++s) {
      if constexpr (S::kBf16) {
        qb[s] = row_ok ? ld16(qrow + (s * M::kK + hh * M::kPer) * 2)
                       : make_uint4(0, 0, 0, 0);
      } else {
        qb[s] = row_ok ? *reinterpret_cast<const float*>(qrow + (s * M::kK + hh) * 4)
                       : 0.f;
      }
    }
  };
  // A wave's rows of a tile lie in one cache block: block wave_blk of the
  // tile's blocks.
  const int wave_blk = wave * S::kDmaPerWave * S::kRowsPerDma / kBlock;
  const int32_t* btab = p.block_tables +
                        static_cast<int64_t>(table_row) * p.max_blocks_per_seq;
  // Group mode: the ids of the first kStages tiles' blocks, requested with
  // the Q rows before the prefix length is known (clamped to the table row
  // instead of the context; a tile past the context reads block 0 anyway).
  int blk_pre[S::kStages];
  if constexpr (kGroup) {
    load_q();
#pragma unroll
    for (int st = 0; st < S::kStages; ++st)
      blk_pre[st] = p.max_blocks_per_seq > 0
                        ? load_uniform_i32(btab, min((kt0 + st) * (kBN / kBlock) + wave_blk,
                                                     p.max_blocks_per_seq - 1))
                        : 0;
    int pl = lq > 0 ? p.prefix_lens[q0] : 0;
    pl = pl < 0 ? 0 : (pl > p.max_seqlen_k ? p.max_seqlen_k : pl);
    if (pl > p.max_blocks_per_seq * kBlock) pl = p.max_blocks_per_seq * kBlock;
    pl -= pl % kBlock;
    ext.lk = pl;
  }
  const int lk = ext.lk;

  // Key tiles this workgroup reads: kt0 .. kt0 + ntiles - 1.
  int ntiles = (tile_key_end(ext, G, m0, S::kBM, p.causal) + kBN - 1) / kBN;
  if constexpr (kGroup) {
    ntiles = min(ntiles - kt0, p.chunk_tiles);
    if (ntiles <= 0) return;   // past this group's prefix: never merged
  }

  // Last key this row may see.
  const int lim = row_ok ? (p.causal ? lk - lq + i_pos : lk - 1) : lk - 1;
  // Smallest limit of the wave: tiles entirely below it need no mask.
  const int wave_m0 = m0 + wave * 32;
  const int wave_lim = p.causal ? lk - lq + min(wave_m0 / G, lq - 1) : lk - 1;

  if constexpr (!kGroup) load_q();

  // Q must have arrived before the tile loop: a wait for it inside the loop
  // would also wait for the K/V loads in flight there.
#pragma unroll
  for (int s = 0; s < S::kQSteps; ++s) {
    if constexpr (S::kBf16)
      asm volatile("" :: "v"(qb[s].x), "v"(qb[s].y), "v"(qb[s].z), "v"(qb[s].w));
    else
      asm volatile("" :: "v"(qb[s]));
  }

  const int64_t row_stride = static_cast<int64_t>(p.num_kv_heads) * S::kRow;
  const int64_t blk_bytes = row_stride * kBlock;
  const int nblk_ctx = (lk + kBlock - 1) / kBlock;   // blocks the context owns

  // DMA load q of this wave moves tile rows r0 .. r0 + kRowsPerDma - 1 (one
  // cache block); lane l's 16 bytes land at byte 16 l of that 1 KiB and hold
  // chunk pos ^ (r % kChunks) of row r.  The per-lane source offset inside a
  // block is the same for every tile.
  uint32_t dma_k_off[S::kDmaPerWave], dma_v_off[S::kDmaPerWave];
#pragma unroll
  for (int q = 0; q < S::kDmaPerWave; ++q) {
    const int byte = (wave * S::kDmaPerWave + q) * 1024 + lane * 16;
    const int r = byte / S::kRow;
    const int pos = (byte % S::kRow) / 16;
    const int64_t row_base = (r % kBlock) * row_stride + kvh * S::kRow;
    dma_k_off[q] = static_cast<uint32_t>(row_base + (pos ^ k_swz<S::kChunks>(r)) * 16);
    dma_v_off[q] = static_cast<uint32_t>(row_base + (pos ^ v_swz<S::kChunks>(r)) * 16);
  }
  // Every lane issues exactly kLoadsPerTile loads per tile, so that the
  // waits below count tiles.  A wave's rows of a tile lie in one cache
  // block, whose id (a scalar load) is fetched one tile ahead of its use.
  // Rows of blocks past the context, or with an id outside the pool, are
  // read from block 0 instead: they are past Lk (masked by select in S,
  // zeroed in V) or the block table is invalid.
  // (Only called with ntiles >= 1, so the context owns a block; the load
  // is unconditional, from a clamped index, so that nothing waits for it
  // before its use one iteration later.)
  auto block_id = [&](int kt) __attribute__((always_inline)) {
    return load_uniform_i32(btab, min(kt * (kBN / kBlock) + wave_blk, nblk_ctx - 1));
  };
  auto dma_tile = [&](int kt, int blk, char* kbuf, char* vbuf) __attribute__((always_inline)) {
    const bool in_ctx = kt * (kBN / kBlock) + wave_blk < nblk_ctx;   // uniform
    blk = in_ctx && blk >= 0 && blk < p.num_blocks ? blk : 0;
    const int64_t base = static_cast<int64_t>(blk) * blk_bytes;
#pragma unroll
    for (int q = 0; q < S::kDmaPerWave; ++q) {
      const int ii = wave * S::kDmaPerWave + q;
      dma16(p.k_cache + base, dma_k_off[q], kbuf + ii * 1024);
      dma16(p.v_cache + base, dma_v_off[q], vbuf + ii * 1024);
    }
  };

  // LDS read offsets, fixed for the whole kernel.  K (A operand of S^T):
  // lane (j, hh) reads row t * 32 + j, chunk (s * kK + hh * kPer) / 8 (bf16)
  // -- for t = 1 the row is 32 further and the swizzle the same.
  const int kswz = k_swz<S::kChunks>(j);   // rows t * 32 + j: same swizzle
  // V^T (A operand of O^T, bf16): transpose reads over rows
  // 16 s + 4 hh + 8 half + i / 4 and dimensions dt * 32 + 16 * g16 +
  // 4 * (i % 4), with g16 = (lane / 16) % 2, i = lane % 16.  The row's
  // swizzle does not depend on s (16 s is a multiple of kChunks' period).
  const int li = lane % 16;
  const int g16 = (lane / 16) % 2;

  f32x16_v oacc[S::kDTiles];
#pragma unroll
  for (int t = 0; t < S::kDTiles; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float run_max = -INFINITY;   // reference max of this row (scaled, log2)
  float run_sum = 0.f;         // this lane half's share of the row sum

  auto compute = [&](int kt, const char* s_k, char* s_v) {
    // V rows past Lk hold whatever the pool has there (NaN in a poisoned
    // test pool); P is 0 there, but 0 * NaN is NaN, so zero them.
    const int kbase = kt * kBN;
    if (kbase + kBN > lk) {
      for (int i = tid; i < kBN * S::kChunks; i += S::kThreads) {
        const int r = i / S::kChunks;
        if (kbase + r >= lk)
          *reinterpret_cast<uint4*>(s_v + r * S::kRow + (i % S::kChunks) * 16) =
              make_uint4(0, 0, 0, 0);
      }
      __syncthreads();
    }

    // ---- S^T = K Q^T: two 32-key M-tiles, their MFMAs interleaved so
    // consecutive MFMAs never wait on each other's accumulator.
    f32x16_v sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
    {
      const char* krow0 = s_k + j * S::kRow;
      const char* krow1 = s_k + (32 + j) * S::kRow;
      // operands read in batches of up to 8 steps, ahead of their MFMAs
      constexpr int kBatch = S::kQSteps < 8 ? S::kQSteps : 8;
#pragma unroll
      for (int s0 = 0; s0 < S::kQSteps; s0 += kBatch) {
        op_t a0[kBatch], a1[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int s = s0 + u;
          if constexpr (S::kBf16) {
            const int c = ((s * M::kK + hh * M::kPer) / 8) ^ kswz;   // chunk
            a0[u] = *reinterpret_cast<const uint4*>(krow0 + c * 16);
            a1[u] = *reinterpret_cast<const uint4*>(krow1 + c * 16);
          } else {
            const int e = s * M::kK + hh;                          // element
            const int off = ((e / 4) ^ kswz) * 16 + (e % 4) * 4;
            a0[u] = *reinterpret_cast<const float*>(krow0 + off);
            a1[u] = *reinterpret_cast<const float*>(krow1 + off);
          }
        }
        // (the fence keeps the compiler from moving the reads back next
        // to their MFMAs, one LDS latency per MFMA pair)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          sacc[0] = M::run(a0[u], qb[s0 + u], sacc[0]);
          sacc[1] = M::run(a1[u], qb[s0 + u], sacc[1]);
        }
      }
    }

    // ---- online softmax for this lane's row ---------------------------
    // Logits stay raw; scale * log2(e) > 0 enters through one FMA with the
    // (scaled) running max.  Masked keys: raw -inf -> weight exactly 0.
    const bool need_mask = kbase + kBN - 1 > wave_lim || kbase + kBN > lk;
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kpos = kbase + t * 32 + (r / 4) * 8 + hh * 4 + r % 4;
          sacc[t][r] = kpos <= lim ? sacc[t][r] : -INFINITY;
        }
    }
    uint4 pb[4];   // bf16: packed weights, the B operand of each PV step
    if constexpr (S::kBf16) {
      // Fast path: weights against the current reference max, without a
      // max scan.  The row sum is taken over the rounded weights (the ones
      // the PV product uses), two per dot2.  A lane whose share of the sum
      // stays <= 2^13 had every weight <= 2^13: nothing overflows.  If all
      // its weights are <= 2^8 the check passes, so the exact path below
      // runs only on a row's first tile and where its max grows by > 2^8.
      float psum = bf16_weights(sacc, p.scale_log2,
                                run_max == -INFINITY ? 0.f : -run_max, pb);
      const bool exact = run_max == -INFINITY || !(psum <= 8192.f);
      if (__any(exact)) {
        float tmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[t][r]);
        tmax = fmaxf(tmax, swap_halves(tmax)) * p.scale_log2;
        const bool grow = tmax > run_max + 8.f;
        if (__any(grow)) {
          const float new_max = grow ? tmax : run_max;
          const float alpha = run_max == -INFINITY ? 0.f : fast_exp2(run_max - new_max);
          run_max = new_max;
          run_sum *= alpha;
#pragma unroll
          for (int t = 0; t < S::kDTiles; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
        }
        psum = bf16_weights(sacc, p.scale_log2,
                            run_max == -INFINITY ? 0.f : -run_max, pb);
      }
      run_sum += psum;
    } else {
      float tmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[t][r]);
      tmax = fmaxf(tmax, swap_halves(tmax)) * p.scale_log2;
      // The reference max moves only when it would grow by more than 2^8:
      // weights stay <= 256 and the rescale of O is skipped on most tiles.
      // Any reference gives the same O / l; this one keeps every term finite.
      const bool grow = tmax > run_max + 8.f;
      if (__any(grow)) {
        const float new_max = grow ? tmax : run_max;
        const float alpha = run_max == -INFINITY ? 0.f : fast_exp2(run_max - new_max);
        run_max = new_max;
        run_sum *= alpha;
#pragma unroll
        for (int t = 0; t < S::kDTiles; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      }
      // A row that has seen no visible key yet keeps max -inf and weights 0.
      const float neg_max = run_max == -INFINITY ? 0.f : -run_max;
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(fmaf(sacc[t][r], p.scale_log2, neg_max));
          sacc[t][r] = pr;
          psum += pr;
        }
      run_sum += psum;
    }

    // ---- O^T += V^T P^T -------------------------------------------------
#pragma unroll
    for (int s = 0; s < S::kPvSteps; ++s) {
      op_t bop;
      if constexpr (S::kBf16) {
        // keys (2s + e/4) * 8 + hh * 4 + e % 4 of the tile: accumulator
        // registers (s % 2) * 8 .. + 7 of S^T M-tile s / 2.
        bop = pb[s];
      } else {
        // step s covers keys (r/4) * 8 + hh * 4 + r % 4 (+ 32 for M-tile 1)
        // with r = s % 16: one probability per lane.
        bop = sacc[s / 16][s % 16];
      }
      // All D tiles' V^T operands of this key step are read before their
      // MFMAs (fenced as above).
      op_t av[S::kDTiles];
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt) {
        op_t a;
        if constexpr (S::kBf16) {
          // keys 16 s + 4 hh + 0..3 (first half) and + 8 (second half) of
          // dimension dt * 32 + j: two transpose reads.
          const int dim0 = dt * 32 + 16 * g16 + 4 * (li % 4);
          const int row_a = 16 * s + 4 * hh + li / 4;
          const int row_b = row_a + 8;
          const int ca = (dim0 / 8) ^ v_swz<S::kChunks>(row_a);
          const int cb = (dim0 / 8) ^ v_swz<S::kChunks>(row_b);
          const uint2 lo = lds_read_tr16(s_v + row_a * S::kRow + ca * 16 + (dim0 % 8) * 2);
          const uint2 hi = lds_read_tr16(s_v + row_b * S::kRow + cb * 16 + (dim0 % 8) * 2);
          a = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          const int r = s % 16;
          const int key = (s / 16) * 32 + (r / 4) * 8 + hh * 4 + r % 4;
          const int dim = dt * 32 + j;
          a = *reinterpret_cast<const float*>(
              s_v + key * S::kRow + ((dim / 4) ^ v_swz<S::kChunks>(key)) * 16 + (dim % 4) * 4);
        }
        av[dt] = a;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt) oacc[dt] = M::run(av[dt], bop, oacc[dt]);
    }
  };

  // K/V stages: tile kt lives in stage kt % kStages.  Tiles up to
  // kt + kStages - 2 are in flight when tile kt is waited for; after the
  // barrier every wave's loads of tile kt have landed and every wave is
  // done reading tile kt - 1, whose stage then takes tile kt + kStages - 1.
  auto kbuf = [&](int st) __attribute__((always_inline)) { return smem + st * S::kTile; };
  auto vbuf = [&](int st) __attribute__((always_inline)) {
    return smem + (S::kStages + st) * S::kTile;
  };
  // Local tile i is key tile kt0 + i and lives in stage i % kStages.
#pragma unroll
  for (int st = 0; st < S::kStages - 1; ++st)
    if (st < ntiles)
      dma_tile(kt0 + st, kGroup ? blk_pre[st] : block_id(kt0 + st), kbuf(st), vbuf(st));
  int next_blk = ntiles > 0 ? (kGroup ? blk_pre[S::kStages - 1]
                                      : block_id(kt0 + S::kStages - 1))
                            : 0;
  for (int it = 0; it < ntiles; ++it) {
    const int ahead = min(S::kStages - 2, ntiles - 1 - it);   // tiles after it in flight
    if (S::kStages >= 3 && ahead >= 1)
      wait_vm<(S::kStages >= 3 ? S::kLoadsPerTile : 0)>();
    else
      wait_vm<0>();
    lds_barrier();
    const int nt = it + S::kStages - 1;
    if (nt < ntiles) {
      dma_tile(kt0 + nt, next_blk, kbuf(nt % S::kStages), vbuf(nt % S::kStages));
      next_blk = block_id(kt0 + nt + 1);
    }
    const int st = it % S::kStages;
    compute(kt0 + it, kbuf(st), vbuf(st));
  }

  // ---- normalise and write: lane (j, hh) holds dims (r/4)*8 + hh*4 + r%4
  // of each 32-dim tile for its row.
  const float total = run_sum + swap_halves(run_sum);
  if (!row_ok) return;
  if constexpr (kGroup) {
    // A partial: its output (bf16 I/O: normalised, binary16; fp32 I/O: the
    // unnormalised fp32 sum), its reference max and its sum.
    const int64_t slot =
        ((static_cast<int64_t>(q0) + i_pos) * p.num_heads + kvh * G + h) *
            p.ws_stride + p.slot0 + chunk;
    if constexpr (S::kBf16) {
      const float inv = total > 0.f ? 1.f / total : 0.f;
      float big = 0.f;
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) big = fmaxf(big, fabsf(oacc[dt][r] * inv));
      const bool is_big = fmaxf(big, swap_halves(big)) >= kPartialBig;   // whole row
      uint16_t* acc = p.ws_acc_h + slot * D;
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint16_t hv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) hv[u] = partial_f16(oacc[dt][g4 * 4 + u] * inv, is_big);
          *reinterpret_cast<uint2*>(acc + dt * 32 + g4 * 8 + hh * 4) =
              make_uint2(hv[0] | (static_cast<uint32_t>(hv[1]) << 16),
                         hv[2] | (static_cast<uint32_t>(hv[3]) << 16));
        }
      if (hh == 0) {
        p.ws_max[slot] = run_max;
        p.ws_sum[slot] = is_big ? -total : total;
      }
    } else {
      float* acc = p.ws_acc + slot * D;
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<float4*>(acc + dt * 32 + g4 * 8 + hh * 4) =
              make_float4(oacc[dt][g4 * 4], oacc[dt][g4 * 4 + 1],
                          oacc[dt][g4 * 4 + 2], oacc[dt][g4 * 4 + 3]);
      if (hh == 0) {
        p.ws_max[slot] = run_max;
        p.ws_sum[slot] = total;
      }
    }
    return;
  }
  const float inv = total > 0.f ? 1.f / total : 0.f;
  T* orow = reinterpret_cast<T*>(p.out) +
            ((static_cast<int64_t>(q0) + i_pos) * p.num_heads + kvh * G + h) * D;
#pragma unroll
  for (int dt = 0; dt < S::kDTiles; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = oacc[dt][g4 * 4 + u] * inv;
      store4<T>(orow + dt * 32 + g4 * 8 + hh * 4, v);
    }
}

// Longest-first schedule.  One workgroup weighs every (sequence, M-tile)
// item by the key tiles it reads (plus one for its fixed cost; 0 for an
// M-tile past the sequence's rows) and writes the items to `order` by
// descending weight: a counting sort over weight bins in LDS (weights past
// the last bin share it).  Items of equal weight land in any order; the
// attention results do not depend on the schedule.
constexpr int kPlanThreads = 1024;

struct PlanParams {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int num_seqs;
  int mtiles;
  int bm;                    // M rows per workgroup
  int group;
  int max_seqlen_q;
  int max_seqlen_k;
  int64_t total_q;
  int max_blocks_per_seq;
  int causal;
};

__device__ __forceinline__ int plan_bin(const PlanParams& q, int item) {
  const SeqExtent e = seq_extent(q.cu_q, q.cu_k, item / q.mtiles, q.max_seqlen_q,
                                 q.max_seqlen_k, q.total_q, q.max_blocks_per_seq);
  return item_weight(e, item, q.mtiles, q.bm, q.group, q.causal);
}

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(
    PlanParams q, int32_t* __restrict__ order) {
  __shared__ int bins[kPlanBins];
  __shared__ int wave_sum[kPlanThreads / kWave];
  longest_first_order<kPlanThreads, kPlanBins, 1>(
      q.num_seqs * q.mtiles, [&](int item) { return plan_bin(q, item); }, order,
      bins, wave_sum);
}

int m_tiles(int max_seqlen_q, int group, int bm) {
  return static_cast<int>((static_cast<int64_t>(max_seqlen_q) * group + bm - 1) / bm);
}

template <typename T, int D, int G, bool kGroup>
hipError_t launch_kernel(const PrefillParams& pr, int64_t wgs, hipStream_t stream) {
  using S = PrefillShape<T, D, kGroup>;
  const size_t lds = S::kLds;
  if (lds > 65536) {
    static bool raised = false;   // once per kernel instantiation
    if (!raised) {
      hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&prefill_kernel<T, D, G, kGroup>),
          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  hipLaunchKernelGGL((prefill_kernel<T, D, G, kGroup>), dim3(static_cast<unsigned>(wgs)),
                     dim3(S::kThreads), lds, stream, pr);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_typed(const PrefillParams& prm, const PrefillArgs& a,
                        hipStream_t stream) {
  using S = PrefillShape<T, D>;
  const int mtiles = m_tiles(a.max_seqlen_q, G, S::kBM);
  const int64_t items = static_cast<int64_t>(a.num_seqs) * mtiles;
  const int64_t wgs = items * a.num_kv_heads;
  if (wgs > 0x7fffffff) return hipErrorNotSupported;
  const size_t lds = S::kLds;
  PrefillParams pr = prm;
  pr.mtiles = mtiles;
  pr.num_seqs = a.num_seqs;
  pr.order = nullptr;
  pr.rank_inline = 0;
  if (items <= S::kThreads) {
    pr.rank_inline = 1;   // ranked inside the attention kernel
  } else if (a.workspace != nullptr &&
             a.workspace_bytes >= static_cast<size_t>(items) * sizeof(int32_t)) {
    PlanParams q{};
    q.cu_q = a.cu_seqlens_q;
    q.cu_k = a.cu_seqlens_k;
    q.num_seqs = a.num_seqs;
    q.mtiles = mtiles;
    q.bm = S::kBM;
    q.group = G;
    q.max_seqlen_q = a.max_seqlen_q;
    q.max_seqlen_k = a.max_seqlen_k;
    q.total_q = a.total_q;
    q.max_blocks_per_seq = a.max_blocks_per_seq;
    q.causal = a.causal ? 1 : 0;
    int32_t* order = static_cast<int32_t*>(a.workspace);
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0,
                       stream, q, order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    pr.order = order;
  }
  (void)lds;
  return launch_kernel<T, D, G, false>(pr, wgs, stream);
}

// Shared-prefix partials: group mode of the same kernel, natural order;
// with plan.order_in_prefix one more workgroup writes the suffix schedule.
template <typename T, int D, int G>
hipError_t launch_prefix_typed(const PrefillParams& prm, const PrefixArgs& a,
                               const SharedPrefixPlan& plan, hipStream_t stream) {
  using S = PrefillShape<T, D, true>;
  if (a.num_groups <= 0 || plan.prefix_chunks <= 0 || a.max_group_size <= 0)
    return hipSuccess;
  PrefillParams pr = prm;
  pr.mtiles = m_tiles(a.max_group_size, G, S::kBM);
  const int64_t items = static_cast<int64_t>(a.num_groups) * plan.prefix_chunks;
  const int64_t wgs = items * pr.mtiles * a.num_kv_heads;
  if (items > 0x7fffffff || wgs + 1 > 0x7fffffff) return hipErrorNotSupported;
  pr.num_seqs = static_cast<int>(items);
  pr.order = nullptr;
  pr.rank_inline = 0;
  pr.chunk_tiles = plan.prefix_chunk_tokens / kBN;
  pr.chunks = plan.prefix_chunks;
  if (!plan.order_in_prefix) return launch_kernel<T, D, G, true>(pr, wgs, stream);
  static_assert(kSuffixBins % S::kThreads == 0, "bins per thread");
  static_assert((kSuffixBins + S::kThreads / kWave) * sizeof(int) <= S::kLds,
                "schedule LDS");
  pr.suffix_order = reinterpret_cast<int32_t*>(static_cast<char*>(a.workspace) +
                                               plan.suffix.off_order);
  pr.context_lens = a.context_lens;
  pr.order_seqs = a.num_seqs;
  pr.order_parts = plan.suffix.num_partitions;
  pr.order_part_tokens = plan.suffix.partition_tokens;
  pr.order_max_len = a.max_context_len;
  return launch_kernel<T, D, G, true>(pr, wgs + 1, stream);
}

template <typename T, int D>
hipError_t dispatch_group(const PrefillParams& prm, const PrefillArgs& a, int g,
                          hipStream_t s) {
  switch (g) {
    case 1: return launch_typed<T, D, 1>(prm, a, s);
    case 2: return launch_typed<T, D, 2>(prm, a, s);
    case 4: return launch_typed<T, D, 4>(prm, a, s);
    case 8: return launch_typed<T, D, 8>(prm, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t dispatch_prefix(const PrefillParams& prm, const PrefixArgs& a,
                           const SharedPrefixPlan& plan, hipStream_t s) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_prefix_typed<T, D, 1>(prm, a, plan, s);
    case 2: return launch_prefix_typed<T, D, 2>(prm, a, plan, s);
    case 4: return launch_prefix_typed<T, D, 4>(prm, a, plan, s);
    case 8: return launch_prefix_typed<T, D, 8>(prm, a, plan, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// The schedule: one int32 per (sequence, M-tile) item, counted for the
// smallest M-tile of any shape and the G the launch dispatches on
// (num_heads / num_kv_heads).
size_t prefill_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads,
                               int head_dim, int max_seqlen_q, int max_seqlen_k) {
  const int g = num_heads / num_kv_heads;
  if (g < 1) return 0;
  const int64_t items = static_cast<int64_t>(num_seqs) * m_tiles(max_seqlen_q, g, kMinBM);
  const size_t tiles = static_cast<size_t>((items * 4 + 255) / 256 * 256);
  // The small-row path (bfloat16 only; the size does not depend on the
  // element type) may take these sizes: room for its partials too.
  const VerifyPlan vp = plan_verify(num_seqs, num_heads, num_kv_heads, head_dim,
                                    max_seqlen_q, max_seqlen_k);
  return vp.use && vp.workspace_bytes > tiles ? vp.workspace_bytes : tiles;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  PrefillParams prm{};
  prm.out = a.out;
  prm.q = static_cast<const char*>(a.q);
  prm.total_q = a.total_q;
  prm.k_cache = static_cast<const char*>(a.k_cache);
  prm.v_cache = static_cast<const char*>(a.v_cache);
  prm.num_blocks = a.num_blocks;
  prm.cu_q = a.cu_seqlens_q;
  prm.cu_k = a.cu_seqlens_k;
  prm.max_seqlen_q = a.max_seqlen_q;
  prm.max_seqlen_k = a.max_seqlen_k;
  prm.block_tables = a.block_tables;
  prm.max_blocks_per_seq = a.max_blocks_per_seq;
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  prm.scale_log2 = a.scale * kLog2e;
  prm.causal = a.causal ? 1 : 0;
  const int g = a.num_heads / a.num_kv_heads;
  if (a.bf16) {
    const VerifyPlan vp = plan_verify(a.num_seqs, a.num_heads, a.num_kv_heads,
                                      a.head_dim, a.max_seqlen_q, a.max_seqlen_k);
    if (vp.use) return launch_verify(a, vp, stream);
    if (a.head_dim == 128) return dispatch_group<bf16_t, 128>(prm, a, g, stream);
    return dispatch_group<bf16_t, 64>(prm, a, g, stream);
  }
  if (a.head_dim == 128) return dispatch_group<float, 128>(prm, a, g, stream);
  return dispatch_group<float, 64>(prm, a, g, stream);
}

hipError_t launch_prefix_partials(const PrefixArgs& a,
                                  const SharedPrefixPlan& plan,
                                  hipStream_t stream) {
  PrefillParams prm{};
  prm.q = static_cast<const char*>(a.q);
  prm.total_q = a.num_seqs;
  prm.k_cache = static_cast<const char*>(a.k_cache);
  prm.v_cache = static_cast<const char*>(a.v_cache);
  prm.num_blocks = a.num_blocks;
  prm.max_seqlen_q = a.max_group_size;
  prm.max_seqlen_k = a.max_prefix_len;
  prm.block_tables = a.block_tables;
  prm.max_blocks_per_seq = a.max_blocks_per_seq;
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  prm.scale_log2 = a.scale * kLog2e;
  prm.causal = 0;
  prm.groups = a.groups;
  prm.prefix_lens = a.prefix_lens;
  char* ws = static_cast<char*>(a.workspace);
  prm.ws_max = reinterpret_cast<float*>(ws + plan.off_max);
  prm.ws_sum = reinterpret_cast<float*>(ws + plan.off_sum);
  prm.ws_acc = reinterpret_cast<float*>(ws + plan.off_acc);
  prm.ws_acc_h = reinterpret_cast<uint16_t*>(ws + plan.off_acc);
  prm.ws_stride = plan.total_slots;
  prm.slot0 = plan.suffix.num_partitions;
  if (a.bf16) {
    if (a.head_dim == 128) return dispatch_prefix<bf16_t, 128>(prm, a, plan, stream);
    return dispatch_prefix<bf16_t, 64>(prm, a, plan, stream);
  }
  if (a.head_dim == 128) return dispatch_prefix<float, 128>(prm, a, plan, stream);
  return dispatch_prefix<float, 64>(prm, a, plan, stream);
}

}  // namespace pa
