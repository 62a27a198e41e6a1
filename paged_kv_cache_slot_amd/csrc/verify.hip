// Varlen attention of a few query rows per sequence over a paged context --
// the shape of a speculative-decoding verify pass, and of large decode
// batches (one row per sequence) -- for gfx950, bfloat16 (the decode route
// also over an 8-bit E4M3 cache).
//
// What it computes: exactly what the varlen prefill computes (sequence b
// owns query rows cu_q[b] .. cu_q[b+1]-1, Lq of them, and its first Lk
// cached tokens as keys; causal row i sees keys 0 .. Lk - Lq + i), for
// launches whose packed rows per KV head, G * max Lq, are at most 64.  In a
// verify pass the target model runs once over the k proposed positions of
// every sequence ("Warmup Guide -- Inference Serving Internals", Chapter 7,
// the scheme; "10 Serving Engines", sections 10.6.1-10.6.2: the gamma
// proposed tokens are verified in one target pass): Lq = k + 1 rows per
// sequence, each a decode row one position further, over a long cache.
//
// Design (MI355X-first).  Like decode this is an HBM stream -- every K/V
// byte of a KV head serves only G * Lq rows -- but with up to 64 rows per
// KV head the dot products belong on MFMA:
//  * a work item is (sequence, partition, KV head), taken by a workgroup of
//    4 waves; the G * Lq rows of a KV head are packed into NT tiles of 16
//    (row m = position m / G, head m % G), so one K/V byte loaded serves all
//    of them;
//  * persistent workgroups, one per CU, draw (sequence, partition, KV head)
//    tickets from a counter in the workspace, longest items first (a plan
//    kernel orders them): the 8 XCDs of the chip stream at different rates
//    (~0.72 to ~0.85 TB/s each, measured), and the dispatcher's fixed round
//    robin share per XCD would leave the fast XCDs idle for the last ~15 %
//    of the launch;
//  * wave w streams cache blocks w, w + 4, ... of its partition with 16-byte
//    bounds-checked buffer loads into registers, kDepth blocks ahead, and
//    writes each block to its own LDS stage (16-byte chunks XOR-swizzled by
//    row; E4M3 codes widened to bfloat16 on the way) right before computing
//    it; waves never wait for each other inside the loop.  Every loop step
//    issues its loads (past the wave's last block they are sized to
//    nothing), so each wait for a block counts exactly the blocks loaded
//    after it.  Loads into registers stream faster than LDS DMA here (~6.7
//    against ~6.3 TB/s measured on this access pattern);
//  * with one row tile and an even number of KV heads a work item takes
//    two adjacent KV heads: each token's read is then one 512-byte piece,
//    which streams at the chip's full read rate (~7.2 TB/s measured, 6.7
//    for 256-byte pieces);
//  * per block and head: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16
//    keys from LDS, all four fragments read before the MFMAs; B = Q^T held
//    in registers), online softmax per lane (a lane holds
//    four keys of one row), O^T += V^T P^T with v_mfma_f32_16x16x16_bf16
//    (A = V^T by LDS transpose reads, B = P^T taken straight from the S^T
//    accumulators, whose layout is already the B operand's);
//  * the softmax reference max moves only when a logit exceeds it by more
//    than 2^8 (exact rescale of O then); otherwise weights are taken
//    against it directly, so most blocks need no cross-lane max;
//  * the four waves' (max, sum, O) are combined through LDS at the end; a
//    single partition writes the output, several write binary16 partials
//    that a merge kernel combines with log-sum-exp weights;
//  * masking by select: keys past a row's causal limit or past Lk, and the
//    keys of a block whose id lies outside the pool, get weight exactly 0;
//    V rows past Lk and such blocks arrive as zeros from the bounds-checked
//    loads (a NaN there would survive a multiplication by zero).
#include <math.h>

#include <atomic>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_tile.h"

namespace pa {

namespace {

constexpr int kBlock = kTileBlock;   // tokens per cache block
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kBf16PairOne = 0x3F803F80u;   // (1.0, 1.0) as bfloat16

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

// Operand layouts of the 16x16 shapes: lane l holds A[l % 16][k(l / 16, e)]
// and B[k(l / 16, e)][l % 16] (the same k for both); accumulator register
// r of lane l is C[4 (l / 16) + r][l % 16].  For 16x16x16, k(g, e) = 4 g +
// e, which is what lets the S^T accumulators feed the PV step as B.
__device__ __forceinline__ f32x4_v mfma_qk(uint4 a, uint4 b, f32x4_v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                 __builtin_bit_cast(bf16x8_v, b),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_v mfma_pv(uint2 a, uint2 b, f32x4_v c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16_t, a),
                                                   __builtin_bit_cast(v4i16_t, b),
                                                   c, 0, 0, 0);
}

// HP KV heads per work item: their rows are adjacent in every cache row, so
// one item reads HP * 2D contiguous bytes per token (HP * D with an 8-bit
// E4M3 cache, F8, whose codes are widened to bfloat16 on the way to LDS).
template <int D, int NT, int HP, bool F8 = false>
struct VerifyShape {
  static constexpr int kRow = D * 2;                   // bytes of one head's row in LDS
  static constexpr int kChunks = kRow / 16;            // 16-byte chunks per head row
  static constexpr int kPiece = HP * kRow;             // LDS bytes per token
  static constexpr int kSrcPiece = F8 ? HP * D : kPiece;   // cache bytes per token
  static constexpr int kBlockBytes = kBlock * kPiece;  // one block of the HP heads in LDS
  static constexpr int kLoads = kBlock * kSrcPiece / 1024;   // 16-byte loads per lane, K or V
  static constexpr int kStage = 2 * kBlockBytes;       // K block, then V block
  static constexpr int kRows = NT * 16;                // packed query rows per head
  static constexpr int kQBytes = HP * kRows * kRow;    // [head][row][kRow]
  // Four row tiles: Q^T stays in LDS (in registers it would not leave room
  // for the accumulators and the blocks in flight without spilling).
  static constexpr bool kQInLds = NT == 4;
  // Blocks in flight per wave (registers: 2 * kLoads uint4 each), the most
  // that fit beside the accumulators without spilling.  E4M3 blocks take
  // half the registers but keep the same depth: deeper (twice as many
  // blocks) measured slower, the register pressure serialising the LDS
  // reads.
  static constexpr int kDepth =
      NT == 4 ? (D == 128 ? 1 : 2) : (HP == 2 && D == 128 ? 2 : 3);
  static constexpr int kQSteps = D / 32;               // QK MFMAs per row tile
  static constexpr int kDTiles = D / 16;               // O^T tiles per row tile
  // LDS: [stage of wave 0 .. 3][Q rows (kQInLds)]; the combine reuses it:
  // each wave's O as fp32 rows padded by 16 bytes (so the 16 rows a lane
  // group writes fall in different banks), then (max, sum) per row; rows
  // of head h of the item after those of head h - 1.
  static constexpr size_t kQOff = static_cast<size_t>(kWaves) * kStage;
  static constexpr int kORow = D * 4 + 16;
  static constexpr int kAllRows = HP * kRows;
  static constexpr size_t kCombine =
      static_cast<size_t>(kWaves) * kAllRows * kORow + kWaves * kAllRows * 8;
  static constexpr int kTpr = D / 8;                   // combine threads per row
  static constexpr int kRowsPerPass = kThreads / kTpr;
  // The next ticket, broadcast through LDS past the combine area (written
  // and read outside the loop).
  static constexpr size_t kTicket = kCombine;
  static constexpr size_t kLoopLds = kQOff + (kQInLds ? kQBytes : 0);
  static constexpr size_t kLds = kLoopLds > kCombine + 16 ? kLoopLds : kCombine + 16;
  static_assert(kBlock * kSrcPiece % 1024 == 0, "1 KiB per load instruction");
  static_assert(kLds <= 160 * 1024, "LDS per CU");
  static_assert(!kQInLds || HP == 1, "four row tiles take one head");
};

// 16-byte chunk swizzles, XOR on the chunk index inside each 256-byte bank
// period, per row of a K/V stage (kPiece bytes; chunk p = head * kChunks +
// chunk).  K: 16 lanes read one chunk of 16 consecutive rows; V: 16 lanes
// read two adjacent chunks of 4 rows each (transpose reads), 64 lanes 16
// rows.  With rows of >= 256 bytes every row starts a bank period; with
// 128-byte rows two rows share one.
template <int kPiece>
__device__ __forceinline__ int k_swz(int row) {
  return kPiece >= 256 ? row % 16 : (row / 2) % (kPiece / 16);
}
template <int kPiece>
__device__ __forceinline__ int v_swz(int row) {
  return kPiece >= 256 ? 2 * (row % 8) : 2 * ((row / 2) % (kPiece / 32));
}

struct VerifyParams {
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
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  float scale_log2;
  int causal;
  int partition_tokens;      // keys per partition (a multiple of 64)
  int num_partitions;
  // Work items (partition * num_seqs + b), heaviest first, from the plan
  // kernel.  With HP KV heads per ticket, ticket t is item order[t / (Hkv /
  // HP)] for KV heads HP * (t % (Hkv / HP)) ..; the workgroups draw tickets
  // from `counter` (zeroed by the plan kernel).
  const int32_t* order;
  int* counter;
  int num_tickets;
  int heads_per_item;
  // Decode (one query row per sequence): row b of q, keys 0 .. L_b - 1 with
  // L_b = context_lens[b]; cu_q / cu_k are not read then.
  const int32_t* context_lens;
  // Partials (num_partitions > 1): slot ((b * max_seqlen_q + i) * Hq + h) *
  // num_partitions + partition.
  float* ws_max;
  float* ws_sum;             // negative: the partial is stored scaled
  uint16_t* ws_acc_h;        // binary16 acc / sum, D per slot
  float v_scale;             // output factor (E4M3 cache: V = code * v_scale)
};

// Keys of sequence extent e that partition `part` reads: [key0, key1).  The
// last row sees every key, so the partition ends at Lk.
__device__ __forceinline__ int partition_blocks(const VerifyParams& p,
                                                const SeqExtent& e, int part) {
  const int key0 = part * p.partition_tokens;
  const int key1 = min(e.lk, key0 + p.partition_tokens);
  return key1 > key0 ? (key1 + kBlock - 1) / kBlock - key0 / kBlock : 0;
}

__device__ __forceinline__ SeqExtent verify_extent(const VerifyParams& p, int b) {
  if (p.context_lens != nullptr) {
    int lk = p.context_lens[b];
    lk = lk < 0 ? 0 : (lk > p.max_seqlen_k ? p.max_seqlen_k : lk);
    if (lk > p.max_blocks_per_seq * kBlock) lk = p.max_blocks_per_seq * kBlock;
    return {b, 1, lk};
  }
  return seq_extent(p.cu_q, p.cu_k, b, p.max_seqlen_q, p.max_seqlen_k, p.total_q,
                    p.max_blocks_per_seq);
}

// Weight of a work item for the longest-first order: its blocks (capped
// at kPlanBins - 1); 0 for a sequence without query rows.
constexpr int kPlanBins = 1024;
__device__ __forceinline__ int item_weight(const VerifyParams& p, int item) {
  const int b = item % p.num_seqs;
  const SeqExtent e = verify_extent(p, b);
  if (e.lq == 0) return 0;
  const int w = partition_blocks(p, e, item / p.num_seqs);
  return w < kPlanBins ? w : kPlanBins - 1;
}

// One work ticket: (sequence, partition, HP KV heads).  Returns the next
// ticket, drawn while the combine runs (no DMA in flight then).
template <int D, int G, int NT, int HP, bool F8>
__device__ __forceinline__ int verify_item(const VerifyParams& p, int ticket, char* smem) {
  using S = VerifyShape<D, NT, HP, F8>;
  constexpr int kP = S::kPiece;
  const int tid = threadIdx.x;
  int* s_ticket = reinterpret_cast<int*>(smem + S::kTicket);
  auto next_ticket = [&]() __attribute__((always_inline)) {
    if (tid == 0) *s_ticket = atomicAdd(p.counter, 1);
    __syncthreads();
    return *s_ticket;
  };
  // The tickets of one item are consecutive: workgroups running at the same
  // time read adjacent pieces of the same cache rows.
  const int groups = p.num_kv_heads / HP;
  const int kvh0 = (ticket % groups) * HP;
  const int n_items = p.num_seqs * p.num_partitions;
  const int item = load_uniform_i32(p.order, ticket / groups);
  if (item < 0 || item >= n_items) return next_ticket();   // uniform
  const int part = item / p.num_seqs;
  const int b = item % p.num_seqs;
  const SeqExtent ext = verify_extent(p, b);
  const int q0 = ext.q0, lq = ext.lq, lk = ext.lk;
  if (lq == 0) return next_ticket();
  // Several partitions: one past Lk is never merged.  A single partition
  // always writes its rows (zeros where a row sees no key).
  const int nblk = partition_blocks(p, ext, part);
  if (nblk == 0 && p.num_partitions > 1) return next_ticket();
  const int kb0 = part * p.partition_tokens / kBlock;

  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int j = lane % 16;     // row (of a row tile) / key (of a block) of this lane
  const int g = lane / 16;     // lane group: keys 4g .. 4g + 3 of S^T
  const int nbw = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;

  constexpr int kSrc = S::kSrcPiece;
  const int64_t row_stride = static_cast<int64_t>(p.num_kv_heads) * (kSrc / HP);
  const int64_t blk_bytes = row_stride * kBlock;
  const int32_t* btab = p.block_tables + static_cast<int64_t>(b) * p.max_blocks_per_seq;
  const int nblk_ctx = (lk + kBlock - 1) / kBlock;

  // ---- load offsets.  Load u of a block brings rows r = (1024 u + 16 l)
  // / kSrc of the block.  bfloat16: lane l's 16 bytes go to slot pos of row
  // r in the stage and are the piece's chunk pos ^ swizzle(r).  E4M3: lane
  // l's 16 codes are chunk pos of the code row; widened they are bfloat16
  // chunks 2 pos and 2 pos + 1, which go to slots (2 pos) ^ swizzle(r) and
  // (2 pos + 1) ^ swizzle(r) (the swizzles keep a chunk pair together in one
  // 256-byte bank period).
  uint32_t k_src[S::kLoads], v_src[S::kLoads];
#pragma unroll
  for (int u = 0; u < S::kLoads; ++u) {
    const int byte = u * 1024 + lane * 16;
    const int r = byte / kSrc;
    const int pos = (byte % kSrc) / 16;
    const int64_t base = r * row_stride + kvh0 * (kSrc / HP);
    if constexpr (F8) {
      k_src[u] = static_cast<uint32_t>(base + pos * 16);
      v_src[u] = k_src[u];
    } else {
      k_src[u] = static_cast<uint32_t>(base + (pos ^ k_swz<kP>(r)) * 16);
      v_src[u] = static_cast<uint32_t>(base + (pos ^ v_swz<kP>(r)) * 16);
    }
  }
  // Block ids are scalar loads (wave-uniform indices), clamped to the
  // partition's last block (steps past the wave's last block load nothing).
  // An empty partition (a single-partition item with Lk = 0) reads no id:
  // its clamped index would lie before the row.
  const int kb_last = kb0 + nblk - 1;
  auto block_id = [&](int jb) __attribute__((always_inline)) {
    return nblk > 0 ? load_uniform_i32(btab, min(kb0 + wave + kWaves * jb, kb_last)) : 0;
  };
  constexpr int kL = S::kLoads;
  uint4 rb[S::kDepth][2 * kL];   // blocks in flight: K loads, then V loads
  // Step jb's block (id blk) through bounds-checked views of its valid
  // tokens: rows past the context, a step past the wave's last block and a
  // block id outside the pool read as zeros without touching memory.
  // Returns 1 for an id outside the pool (whose keys are then masked).
  auto load_block = [&](int jb, int blk, uint4 (&r)[2 * kL]) __attribute__((always_inline)) {
    const bool in_pool = blk >= 0 && blk < p.num_blocks;
    const int kbj = kb0 + wave + kWaves * jb;
    const int ntok = jb < nbw && in_pool ? min(kBlock, lk - kbj * kBlock) : 0;
    const int64_t off = static_cast<int64_t>(in_pool ? blk : 0) * blk_bytes;
    const int bytes = ntok * static_cast<int>(row_stride);
    const auto rk = block_rsrc(p.k_cache + off, bytes);
    const auto rv = block_rsrc(p.v_cache + off, bytes);
#pragma unroll
    for (int u = 0; u < kL; ++u) {
      r[u] = buf_ld16_nt(rk, k_src[u]);
      r[kL + u] = buf_ld16_nt(rv, v_src[u]);
    }
    return in_pool ? 0 : 1;
  };
  char* st = smem + wave * S::kStage;   // this wave's stage
  auto store_block = [&](const uint4 (&r)[2 * kL]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kL; ++u) {
      if constexpr (F8) {
        const int byte = u * 1024 + lane * 16;
        const int row = byte / kSrc;
        const int pos = (byte % kSrc) / 16;
        char* kr = st + row * kP;
        char* vr = st + S::kBlockBytes + row * kP;
        const int kx = k_swz<kP>(row), vx = v_swz<kP>(row);
        *reinterpret_cast<uint4*>(kr + ((2 * pos) ^ kx) * 16) = e4m3x8_to_bf16(r[u].x, r[u].y);
        *reinterpret_cast<uint4*>(kr + ((2 * pos + 1) ^ kx) * 16) = e4m3x8_to_bf16(r[u].z, r[u].w);
        *reinterpret_cast<uint4*>(vr + ((2 * pos) ^ vx) * 16) =
            e4m3x8_to_bf16(r[kL + u].x, r[kL + u].y);
        *reinterpret_cast<uint4*>(vr + ((2 * pos + 1) ^ vx) * 16) =
            e4m3x8_to_bf16(r[kL + u].z, r[kL + u].w);
      } else {
        *reinterpret_cast<uint4*>(st + u * 1024 + lane * 16) = r[u];
        *reinterpret_cast<uint4*>(st + S::kBlockBytes + u * 1024 + lane * 16) = r[kL + u];
      }
    }
  };
  // ---- Q^T, the B operand of S^T: lane (g, j) holds dimensions 32 s + 8 g
  // .. + 7 of row 16 n + j of head hp; rows past G * Lq repeat row 0
  // (finite values, results never written).  In registers, or (four row
  // tiles) in LDS, where wave w writes row tile w.  Its loads go out ahead
  // of the first K/V blocks.
  uint4 qb[S::kQInLds ? 1 : HP][S::kQSteps][S::kQInLds ? 1 : NT];
  char* qlds = smem + S::kQOff;
  const char* qbase = p.q + static_cast<int64_t>(q0) * p.num_heads * S::kRow;
  auto q_row = [&](int hp, int m) __attribute__((always_inline)) {
    const int mm = m < G * lq ? m : 0;
    return qbase + ((mm / G) * p.num_heads + (kvh0 + hp) * G + mm % G) * S::kRow;
  };
  if constexpr (S::kQInLds) {
    const char* qrow = q_row(0, wave * 16 + j);
#pragma unroll
    for (int s = 0; s < S::kQSteps; ++s) qb[0][s][0] = ld16(qrow + (32 * s + 8 * g) * 2);
  } else {
#pragma unroll
    for (int hp = 0; hp < HP; ++hp)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const char* qrow = q_row(hp, n * 16 + j);
#pragma unroll
        for (int s = 0; s < S::kQSteps; ++s) qb[hp][s][n] = ld16(qrow + (32 * s + 8 * g) * 2);
      }
  }
  __asm__ volatile("" ::: "memory");

  // ---- prologue: blocks 0 .. kDepth - 1 in flight, all kDepth loads
  // issued (past the wave's last block they read nothing).  Q has then
  // arrived once at most the K/V loads are outstanding: the explicit waits
  // (on both paths) say so, and spare the loop's uses of Q a wait for every
  // load in flight.
  int bad[S::kDepth];   // per block in flight: its id is outside the pool
  if (nbw > 0) {
#pragma unroll
    for (int d = 0; d < S::kDepth; ++d) bad[d] = load_block(d, block_id(d), rb[d]);
    constexpr int kKV = S::kDepth * 2 * kL;
    static_assert(kKV < 64, "vmcnt is six bits");
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((kKV & 15) | (7 << 4) | (15 << 8) | ((kKV >> 4) << 14));
  } else {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0): Q only
  }
  if constexpr (!S::kQInLds) {
#pragma unroll
    for (int hp = 0; hp < HP; ++hp)
#pragma unroll
      for (int s = 0; s < S::kQSteps; ++s)
#pragma unroll
        for (int n = 0; n < NT; ++n)
          __asm__ volatile("" : "+v"(qb[hp][s][n].x), "+v"(qb[hp][s][n].y),
                                "+v"(qb[hp][s][n].z), "+v"(qb[hp][s][n].w));
  }
  int next_id = block_id(S::kDepth);
  if constexpr (S::kQInLds) {
    const int m = wave * 16 + j;
#pragma unroll
    for (int s = 0; s < S::kQSteps; ++s)
      *reinterpret_cast<uint4*>(qlds + m * S::kRow + ((4 * s + g) ^ k_swz<S::kRow>(m)) * 16) =
          qb[0][s][0];
    __syncthreads();
  }
  auto q_op = [&](int hp, int s, int n) __attribute__((always_inline)) {
    if constexpr (S::kQInLds) {
      const int m = n * 16 + j;
      return *reinterpret_cast<const uint4*>(qlds + m * S::kRow +
                                             ((4 * s + g) ^ k_swz<S::kRow>(m)) * 16);
    } else {
      return qb[hp][s][n];
    }
  };

  // Row constants: the last key each of this lane's rows may see.
  int lim[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int m = n * 16 + j;
    lim[n] = (p.causal && m < G * lq) ? lk - lq + m / G : lk - 1;
  }
  const int min_lim = p.causal ? lk - lq : lk - 1;   // over the real rows

  // LDS read offsets inside a stage.  K (A of S^T): row j, chunk hp *
  // kChunks + 4 s + g.
  const int k_off = j * kP;
  const int k_x = k_swz<kP>(j) * 16;
  // V^T (A of O^T, transpose reads): lane (g, s') reads row 4 g + s' / 4,
  // dimensions 16 dt + 4 (s' % 4) .. + 3 of head hp; lane (g, i) receives
  // V[4 g + e][16 dt + i] for e = 0..3.  The swizzle is even, so it keeps
  // the chunk pair (2 dt, 2 dt + 1) together.
  const int v_row = 4 * g + j / 4;
  const int v_off = S::kBlockBytes + v_row * kP + ((j % 4) / 2) * 16 + (j % 2) * 8;
  const int v_x = v_swz<kP>(v_row) * 16;

  f32x4_v oacc[HP][S::kDTiles][NT];
  float run_max[HP][NT], run_sum[HP][NT];
#pragma unroll
  for (int hp = 0; hp < HP; ++hp)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt) oacc[hp][dt][n] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      run_max[hp][n] = -INFINITY;   // reference max of the row (scaled, log2)
      run_sum[hp][n] = 0.f;         // this lane's share of the row sum
    }

  // (V rows past Lk arrive as zeros, so P V never meets stale values.)
  auto compute = [&](int kb, int bad_blk) __attribute__((always_inline)) {
    const int kbase = kb * kBlock;
    const bool masked = bad_blk || kbase + kBlock - 1 > min_lim || kbase + kBlock > lk;
#pragma unroll
    for (int hp = 0; hp < HP; ++hp) {
      // ---- S^T = K Q^T
      f32x4_v sacc[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) sacc[n] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      // All of the head's K fragments are read before its MFMAs (the fence
      // keeps the compiler from interleaving them again): one LDS latency
      // per head instead of one per MFMA.
      uint4 ka[S::kQSteps];
#pragma unroll
      for (int s = 0; s < S::kQSteps; ++s)
        ka[s] = *reinterpret_cast<const uint4*>(
            st + k_off + (((hp * S::kChunks + 4 * s + g) * 16) ^ k_x));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < S::kQSteps; ++s) {
#pragma unroll
        for (int n = 0; n < NT; ++n) sacc[n] = mfma_qk(ka[s], q_op(hp, s, n), sacc[n]);
      }
      // ---- mask: key 4 g + r of the block against each row's limit
      if (masked) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sacc[n][r] = !bad_blk && kbase + 4 * g + r <= lim[n] ? sacc[n][r] : -INFINITY;
      }
      // ---- online softmax.  Fast path: weights against the reference
      // max, summed over the bfloat16-rounded values the PV step uses; a
      // lane share <= 2^13 means every weight is.  The exact path (max over
      // the row's 16 keys, rescale of O) runs on a row's first visible
      // block and where its max grows by more than 2^8.
      uint2 pb[NT];
      float psum[NT];
      auto weights = [&](int n) __attribute__((always_inline)) {
        const float neg = run_max[hp][n] == -INFINITY ? 0.f : -run_max[hp][n];
        const float w0 = fast_exp2(fmaf(sacc[n][0], p.scale_log2, neg));
        const float w1 = fast_exp2(fmaf(sacc[n][1], p.scale_log2, neg));
        const float w2 = fast_exp2(fmaf(sacc[n][2], p.scale_log2, neg));
        const float w3 = fast_exp2(fmaf(sacc[n][3], p.scale_log2, neg));
        pb[n] = make_uint2(pack_bf16x2(w0, w1), pack_bf16x2(w2, w3));
        psum[n] = dot2_bf16(pb[n].y, kBf16PairOne, dot2_bf16(pb[n].x, kBf16PairOne, 0.f));
      };
      bool exact = false;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        weights(n);
        exact = exact || run_max[hp][n] == -INFINITY || !(psum[n] <= 8192.f);
      }
      if (__any(exact)) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          float t = fmaxf(fmaxf(sacc[n][0], sacc[n][1]), fmaxf(sacc[n][2], sacc[n][3]));
          t = fmaxf(t, __shfl_xor(t, 16, kWave));
          t = fmaxf(t, swap_halves(t)) * p.scale_log2;
          const bool grow = t > run_max[hp][n] + 8.f;
          if (__any(grow)) {
            const float nm = grow ? t : run_max[hp][n];
            const float alpha =
                run_max[hp][n] == -INFINITY ? 0.f : fast_exp2(run_max[hp][n] - nm);
            run_max[hp][n] = nm;
            run_sum[hp][n] *= alpha;
#pragma unroll
            for (int dt = 0; dt < S::kDTiles; ++dt) oacc[hp][dt][n] *= alpha;
            weights(n);
          }
        }
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) run_sum[hp][n] += psum[n];
      // ---- O^T += V^T P^T
      // (the V^T fragments likewise, all before the MFMAs)
      uint2 va[S::kDTiles];
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt)
        va[dt] = lds_read_tr16(st + v_off + (((hp * S::kChunks + 2 * dt) * 16) ^ v_x));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt) {
#pragma unroll
        for (int n = 0; n < NT; ++n) oacc[hp][dt][n] = mfma_pv(va[dt], pb[n], oacc[hp][dt][n]);
      }
    }
  };

  // ---- main loop: block jb arrives in rb[jb % kDepth]; it goes to the
  // wave's LDS stage, the block kDepth further on is loaded into the freed
  // registers, and the stage is computed.  (LDS operations of one wave run
  // in order: the stores of block jb + 1 follow the reads of block jb.)
  // Every step stores and issues its loads, also the last group's steps
  // past the wave's last block (whose loads read nothing and which compute
  // nothing): with no load skipped, every wait for a block counts exactly
  // the kDepth - 1 blocks loaded after it.
  for (int jb0 = 0; jb0 < nbw; jb0 += S::kDepth) {
#pragma unroll
    for (int d = 0; d < S::kDepth; ++d) {
      const int jb = jb0 + d;
      const int bad_blk = bad[d];
      store_block(rb[d]);
      bad[d] = load_block(jb + S::kDepth, next_id, rb[d]);
      next_id = block_id(jb + S::kDepth + 1);
      // keep the loads here: the compiler may otherwise sink them to
      // their use
      __asm__ volatile("" ::: "memory");
      if (jb < nbw) compute(kb0 + wave + kWaves * jb, bad_blk);
    }
  }

  // ---- combine the four waves.  Every wave is past its loop (and so past
  // its last LDS read of the stages and of Q) after this barrier.
  float total[HP][NT];
#pragma unroll
  for (int hp = 0; hp < HP; ++hp)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float t = run_sum[hp][n] + __shfl_xor(run_sum[hp][n], 16, kWave);
      total[hp][n] = t + swap_halves(t);
    }
  __syncthreads();
  int next = 0;
  if (tid == 0) next = atomicAdd(p.counter, 1);
  float2* ml = reinterpret_cast<float2*>(smem + kWaves * S::kAllRows * S::kORow);
  {
    char* ow = smem + static_cast<size_t>(wave) * S::kAllRows * S::kORow;
#pragma unroll
    for (int hp = 0; hp < HP; ++hp)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int m = hp * S::kRows + n * 16 + j;
#pragma unroll
        for (int dt = 0; dt < S::kDTiles; ++dt)
          *reinterpret_cast<float4*>(ow + m * S::kORow + (dt * 16 + 4 * g) * 4) =
              make_float4(oacc[hp][dt][n][0], oacc[hp][dt][n][1], oacc[hp][dt][n][2],
                          oacc[hp][dt][n][3]);
        if (g == 0) ml[wave * S::kAllRows + m] = make_float2(run_max[hp][n], total[hp][n]);
      }
  }
  __syncthreads();
  const int c = tid % S::kTpr;   // dimensions 8 c .. 8 c + 7
#pragma unroll
  for (int r0 = 0; r0 < S::kAllRows; r0 += S::kRowsPerPass) {
    const int rr = r0 + tid / S::kTpr;   // head rr / kRows of the item, row rr % kRows
    const int m = rr % S::kRows;
    if (rr >= S::kAllRows || m >= G * lq) continue;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, ml[w * S::kAllRows + rr].x);
    float l = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float2 st = ml[w * S::kAllRows + rr];
        const float a = fast_exp2(st.x - mx);   // 0 for a wave that saw nothing
        l = fmaf(a, st.y, l);
        const char* src = smem + static_cast<size_t>(w) * S::kAllRows * S::kORow +
                          rr * S::kORow + c * 32;
        const float4 x = *reinterpret_cast<const float4*>(src);
        const float4 y = *reinterpret_cast<const float4*>(src + 16);
        o[0] = fmaf(a, x.x, o[0]); o[1] = fmaf(a, x.y, o[1]);
        o[2] = fmaf(a, x.z, o[2]); o[3] = fmaf(a, x.w, o[3]);
        o[4] = fmaf(a, y.x, o[4]); o[5] = fmaf(a, y.y, o[5]);
        o[6] = fmaf(a, y.z, o[6]); o[7] = fmaf(a, y.w, o[7]);
      }
    }
    const float inv = (l > 0.f ? 1.f / l : 0.f) * p.v_scale;
    const int i = m / G;
    const int head = (kvh0 + rr / S::kRows) * G + m % G;
    if (p.num_partitions == 1) {
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) +
                       ((static_cast<int64_t>(q0) + i) * p.num_heads + head) * D + c * 8;
      *reinterpret_cast<uint4*>(orow) =
          make_uint4(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                     pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv));
    } else {
      // A partial: normalised output as binary16 (scaled by 2^-16, sum
      // negated, when some |o| of the row reaches 2^15), max, sum.
      float big = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) big = fmaxf(big, fabsf(o[e] * inv));
#pragma unroll
      for (int x = 1; x < S::kTpr; x *= 2) big = fmaxf(big, __shfl_xor(big, x, kWave));
      const bool is_big = big >= kPartialBig;
      const int64_t slot =
          ((static_cast<int64_t>(b) * p.max_seqlen_q + i) * p.num_heads + head) *
              p.num_partitions + part;
      uint16_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = partial_f16(o[e] * inv, is_big);
      *reinterpret_cast<uint4*>(p.ws_acc_h + slot * D + c * 8) =
          make_uint4(h[0] | (static_cast<uint32_t>(h[1]) << 16),
                     h[2] | (static_cast<uint32_t>(h[3]) << 16),
                     h[4] | (static_cast<uint32_t>(h[5]) << 16),
                     h[6] | (static_cast<uint32_t>(h[7]) << 16));
      if (c == 0) {
        p.ws_max[slot] = mx;
        p.ws_sum[slot] = is_big ? -l : l;
      }
    }
  }
  if (tid == 0) *s_ticket = next;
  __syncthreads();
  return *s_ticket;
}

// Persistent workgroups (as many as fit on the chip at once) draw tickets
// until none are left: the XCDs of one chip do not stream at the same rate,
// and a fixed share of the work per XCD (the dispatcher deals workgroups to
// the XCDs round robin) would leave the fast ones idle at the end.
template <int D, int G, int NT, int HP, bool F8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
verify_kernel(VerifyParams p) {
  using S = VerifyShape<D, NT, HP, F8>;
  extern __shared__ __align__(16) char smem[];
  int* s_ticket = reinterpret_cast<int*>(smem + S::kTicket);
  if (threadIdx.x == 0) *s_ticket = atomicAdd(p.counter, 1);
  __syncthreads();
  int t = *s_ticket;
  while (t < p.num_tickets) {
    __syncthreads();   // every thread has read the ticket
    t = verify_item<D, G, NT, HP, F8>(p, __builtin_amdgcn_readfirstlane(t), smem);
  }
}


// Merge the partitions of one (sequence, row, query head): row i of
// sequence b reads the partitions that hold a key it sees.
template <int D>
__global__ __launch_bounds__(D) void verify_merge_kernel(VerifyParams p) {
  const int h = blockIdx.x % p.num_heads;
  const int rest = blockIdx.x / p.num_heads;
  const int i = rest % p.max_seqlen_q;
  const int b = rest / p.max_seqlen_q;
  const int d = threadIdx.x;
  const SeqExtent e = verify_extent(p, b);
  if (i >= e.lq) return;
  int kend = p.causal ? e.lk - e.lq + i + 1 : e.lk;
  kend = kend < 0 ? 0 : kend;
  int np = (kend + p.partition_tokens - 1) / p.partition_tokens;
  np = np > p.num_partitions ? p.num_partitions : np;
  const int64_t slot0 =
      ((static_cast<int64_t>(b) * p.max_seqlen_q + i) * p.num_heads + h) * p.num_partitions;
  const float o = merge_partials<8>(np, [&](int k, float& m, float& l, float& acc)
                                            __attribute__((always_inline)) {
    const int64_t s = slot0 + k;
    const float lraw = p.ws_sum[s];
    const float ov = f16_to_f32(p.ws_acc_h[s * D + d]);
    m = p.ws_max[s];
    l = fabsf(lraw);
    acc = l * (lraw < 0.f ? ov * kPartialGrow : ov);
  });
  uint16_t* out = reinterpret_cast<uint16_t*>(p.out) +
                  ((static_cast<int64_t>(e.q0) + i) * p.num_heads + h) * D + d;
  *out = f32_to_bf16_rne(o);
}

constexpr int kPlanThreads = 1024;

// The longest-first order of the work items, and a zero ticket counter.
__global__ __launch_bounds__(kPlanThreads) void verify_plan_kernel(
    VerifyParams p, int32_t* __restrict__ order) {
  __shared__ int bins[kPlanBins];
  __shared__ int wave_sum[kPlanThreads / kWave];
  if (threadIdx.x == 0) *p.counter = 0;
  longest_first_order<kPlanThreads, kPlanBins, 4>(
      p.num_seqs * p.num_partitions, [&](int item) { return item_weight(p, item); },
      order, bins, wave_sum);
}

template <int D, int G, int NT, int HP, bool F8>
hipError_t launch_nt(const VerifyParams& prm, const VerifyPlan& plan, hipStream_t s) {
  using S = VerifyShape<D, NT, HP, F8>;
  static bool raised = false;   // once per kernel instantiation
  if (!raised) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&verify_kernel<D, G, NT, HP, F8>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(S::kLds));
    if (e != hipSuccess) return e;
    raised = true;
  }
  // As many workgroups as the chip holds at once (fewer for a small launch).
  const int64_t slots = device_cus();
  const int64_t wgs = prm.num_tickets < slots ? prm.num_tickets : slots;
  hipLaunchKernelGGL(verify_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, prm,
                     const_cast<int32_t*>(prm.order));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_kernel<D, G, NT, HP, F8>), dim3(static_cast<unsigned>(wgs)),
                     dim3(kThreads), S::kLds, s, prm);
  e = hipGetLastError();
  if (e != hipSuccess || plan.num_partitions == 1) return e;
  const int64_t merges = static_cast<int64_t>(prm.num_seqs) * prm.max_seqlen_q *
                         prm.num_heads;
  hipLaunchKernelGGL((verify_merge_kernel<D>), dim3(static_cast<unsigned>(merges)),
                     dim3(D), 0, s, prm);
  return hipGetLastError();
}

// An E4M3 cache comes only with one query row per sequence (the decode
// route): one row tile.
template <int D, int G, bool F8>
hipError_t launch_g(const VerifyParams& prm, const VerifyPlan& plan, hipStream_t s) {
  if constexpr (F8) {
    if (plan.row_tiles != 1) return hipErrorInvalidValue;
    return plan.heads_per_item == 2 ? launch_nt<D, G, 1, 2, true>(prm, plan, s)
                                    : launch_nt<D, G, 1, 1, true>(prm, plan, s);
  } else {
    switch (plan.row_tiles) {
      case 1: return plan.heads_per_item == 2 ? launch_nt<D, G, 1, 2, false>(prm, plan, s)
                                              : launch_nt<D, G, 1, 1, false>(prm, plan, s);
      case 2: return launch_nt<D, G, 2, 1, false>(prm, plan, s);
      case 4: return launch_nt<D, G, 4, 1, false>(prm, plan, s);
      default: return hipErrorInvalidValue;
    }
  }
}

template <int D, bool F8 = false>
hipError_t launch_d(const VerifyParams& prm, const VerifyPlan& plan, int g,
                    hipStream_t s) {
  switch (g) {
    case 1: return launch_g<D, 1, F8>(prm, plan, s);
    case 2: return launch_g<D, 2, F8>(prm, plan, s);
    case 4: return launch_g<D, 4, F8>(prm, plan, s);
    case 8: return launch_g<D, 8, F8>(prm, plan, s);
    default: return hipErrorInvalidValue;
  }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Partitions: few enough that most launches need no merge, enough tickets
// (~4 per workgroup slot) that a small batch still balances over the chip.
constexpr int64_t kTargetWorkgroups = 1024;
constexpr int kMinPartitionTokens = 256;

}  // namespace

int device_cus() {
  constexpr int kMaxDeviceIds = 64;
  static std::atomic<int> cus[kMaxDeviceIds];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDeviceIds) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

VerifyPlan plan_verify(int num_seqs, int num_heads, int num_kv_heads,
                       int head_dim, int max_seqlen_q, int max_seqlen_k) {
  VerifyPlan plan{};
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
    return plan;
  const int g = num_heads / num_kv_heads;
  const int64_t rows = static_cast<int64_t>(g) * max_seqlen_q;
  if ((g != 1 && g != 2 && g != 4 && g != 8) || (head_dim != 64 && head_dim != 128) ||
      max_seqlen_q <= 0 || rows > 64 || max_seqlen_k <= 0)
    return plan;
  plan.use = true;
  plan.row_tiles = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  // Two KV heads per work item (512-byte reads at D = 128) where the
  // registers allow: one row tile.
  plan.heads_per_item = (num_kv_heads % 2 == 0 && plan.row_tiles == 1) ? 2 : 1;
  const int64_t groups = static_cast<int64_t>(num_seqs) * (num_kv_heads / plan.heads_per_item);
  int64_t parts = groups >= kTargetWorkgroups
                      ? 1
                      : (kTargetWorkgroups + groups - 1) / groups;
  int64_t tokens = (max_seqlen_k + parts - 1) / parts;
  tokens = (tokens + 63) / 64 * 64;
  if (tokens < kMinPartitionTokens) tokens = kMinPartitionTokens;
  plan.partition_tokens = static_cast<int>(tokens);
  plan.num_partitions = static_cast<int>((max_seqlen_k + tokens - 1) / tokens);
  size_t bytes = 0;
  if (plan.num_partitions > 1) {
    const size_t slots = static_cast<size_t>(num_seqs) * max_seqlen_q * num_heads *
                         plan.num_partitions;
    plan.off_max = 0;
    plan.off_sum = align256(slots * sizeof(float));
    plan.off_acc = plan.off_sum + align256(slots * sizeof(float));
    bytes = plan.off_acc + align256(slots * static_cast<size_t>(head_dim) * 2);
  }
  const int64_t items = static_cast<int64_t>(num_seqs) * plan.num_partitions;
  plan.off_order = bytes;
  bytes += align256(static_cast<size_t>(items) * sizeof(int32_t));
  plan.off_counter = bytes;
  bytes += 256;
  plan.workspace_bytes = bytes;
  return plan;
}

namespace {

hipError_t launch_plan(VerifyParams& prm, const VerifyPlan& plan, void* workspace,
                       int head_dim, bool fp8_cache, hipStream_t stream) {
  const int64_t tickets = static_cast<int64_t>(prm.num_seqs) * plan.num_partitions *
                          (prm.num_kv_heads / plan.heads_per_item);
  const int64_t merges = static_cast<int64_t>(prm.num_seqs) * prm.max_seqlen_q * prm.num_heads;
  if (tickets > 0x7fffffff || merges > 0x7fffffff) return hipErrorNotSupported;
  prm.partition_tokens = plan.partition_tokens;
  prm.num_partitions = plan.num_partitions;
  char* ws = static_cast<char*>(workspace);
  if (plan.num_partitions > 1) {
    prm.ws_max = reinterpret_cast<float*>(ws + plan.off_max);
    prm.ws_sum = reinterpret_cast<float*>(ws + plan.off_sum);
    prm.ws_acc_h = reinterpret_cast<uint16_t*>(ws + plan.off_acc);
  }
  prm.order = reinterpret_cast<const int32_t*>(ws + plan.off_order);
  prm.counter = reinterpret_cast<int*>(ws + plan.off_counter);
  prm.num_tickets = static_cast<int>(tickets);
  prm.heads_per_item = plan.heads_per_item;
  const int g = prm.num_heads / prm.num_kv_heads;
  if (fp8_cache) {
    if (head_dim != 128) return hipErrorNotSupported;
    return launch_d<128, true>(prm, plan, g, stream);
  }
  if (head_dim == 128) return launch_d<128>(prm, plan, g, stream);
  return launch_d<64>(prm, plan, g, stream);
}

}  // namespace

hipError_t launch_verify_decode(const DecodeArgs& a, const VerifyPlan& plan,
                                hipStream_t stream) {
  VerifyParams prm{};
  prm.out = a.out;
  prm.q = static_cast<const char*>(a.q);
  prm.total_q = a.num_seqs;
  prm.k_cache = static_cast<const char*>(a.k_cache);
  prm.v_cache = static_cast<const char*>(a.v_cache);
  prm.num_blocks = a.num_blocks;
  prm.context_lens = a.context_lens;
  prm.max_seqlen_q = 1;
  prm.max_seqlen_k = a.max_context_len;
  prm.block_tables = a.block_tables;
  prm.max_blocks_per_seq = a.max_blocks_per_seq;
  prm.num_seqs = a.num_seqs;
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  // E4M3 cache: K = code * k_scale joins the logit scale, V = code *
  // v_scale the output (both 1 otherwise).
  prm.scale_log2 = a.scale * a.k_scale * kLog2e;
  prm.v_scale = a.v_scale;
  prm.causal = 1;
  return launch_plan(prm, plan, a.workspace, a.head_dim, a.fp8_cache, stream);
}

hipError_t launch_verify(const PrefillArgs& a, const VerifyPlan& plan,
                         hipStream_t stream) {
  VerifyParams prm{};
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
  prm.num_seqs = a.num_seqs;
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  prm.scale_log2 = a.scale * kLog2e;
  prm.v_scale = 1.f;
  prm.causal = a.causal ? 1 : 0;
  return launch_plan(prm, plan, a.workspace, a.head_dim, false, stream);
}

}  // namespace pa
