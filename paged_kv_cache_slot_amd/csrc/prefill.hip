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
//  * one workgroup (4 waves) per (M-tile of 128 rows, KV head, sequence);
//    the G query heads of a KV head are packed into M (row m = position
//    m / G, head m % G), so a K/V tile loaded once serves all of them;
//  * per 64-key tile the workgroup gathers K (row-major) and V (transposed)
//    through the block table into padded LDS, the next tile's global loads
//    in flight while the current one is computed;
//  * each wave computes S^T = K Q^T for its 32 rows with
//    v_mfma_f32_32x32x16_bf16 (fp32 I/O: v_mfma_f32_32x32x2_f32), Q^T held
//    in registers as the B operand.  In the accumulator layout every lane
//    owns one query row, so the online softmax (running max, rescale, sum)
//    is per lane plus one exchange between the two lane halves, and the
//    probabilities already sit in the B-operand layout of O^T += V^T P^T --
//    no shuffles or LDS round trip for P;
//  * masking is by select: keys past the causal limit or past Lk get weight
//    exactly 0, and V rows past Lk are zeroed in LDS (a NaN there would
//    survive a multiplication by zero);
//  * only tiles that cross the causal diagonal or Lk evaluate the mask; the
//    running max moves lazily, so O is rescaled on few tiles.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kBlock = 16;         // tokens per cache block
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBM = 128;           // M rows (query row x head) per workgroup
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

template <typename T, int D>
struct PrefillShape {
  static constexpr int kElem = ElemTraits<T>::kBytes;
  static constexpr int kRow = D * kElem;                  // bytes per key row
  static constexpr int kChunks = kRow / 16;               // 16-byte chunks
  static constexpr bool kBf16 = sizeof(T) == 2;
  // K tile, row-major, rows padded so 32 lanes reading one column of 32
  // different rows spread over the banks.
  static constexpr int kKPitch = kRow + 16;
  // V tile: bf16 transposed [D][kBN keys] (MFMA A operand wants 8 keys of
  // one dimension per lane); fp32 row-major (one element per lane).
  static constexpr int kVPitch = kBf16 ? kBN * 2 + 8 : kRow + 16;
  static constexpr int kVBytes = kBf16 ? D * kVPitch : kBN * kVPitch;
  static constexpr int kQSteps = D / Mma<T>::kK;          // MFMAs per S tile
  static constexpr int kPvSteps = kBN / Mma<T>::kK;       // MFMAs per O tile
  static constexpr int kDTiles = D / 32;                  // O^T M-tiles
  // Tile staging: thread t moves chunk column t % kChunks of kKpt
  // consecutive keys (kKpt = kLoadsPerThread), so a bf16 thread can write
  // its 8 dims x kKpt keys of V^T as 8 runs of kKpt keys.
  static constexpr int kLoadsPerThread = kBN * kChunks / kThreads;
  static constexpr int kKpt = kLoadsPerThread;
  static_assert(kBN * kChunks % kThreads == 0, "tile load split");
  static_assert(kThreads % kChunks == 0, "chunk columns per thread");
  static_assert(!kBf16 || kKpt == 2 || kKpt == 4, "bf16 V^T write width");
};

struct PrefillParams {
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
};

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

// Two waves per SIMD: one wave's softmax and LDS traffic overlap the other's
// MFMAs.  Every shape fits the 256-register budget without spilling.
template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillParams p) {
  using S = PrefillShape<T, D>;
  using M = Mma<T>;
  typedef typename M::op_t op_t;
  extern __shared__ __align__(16) char smem[];
  char* s_k = smem;                          // [kBN][kKPitch]
  char* s_v = smem + kBN * S::kKPitch;       // see PrefillShape

  const int mtile = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int j = lane % 32;                   // this lane's row inside the wave
  const int hh = lane / 32;                  // lane half

  // Sequence extent, clamped so no index leaves the buffers.
  int q0 = p.cu_q[b];
  int lq = p.cu_q[b + 1] - q0;
  int lk = p.cu_k[b + 1] - p.cu_k[b];
  q0 = q0 < 0 ? 0 : q0;
  lq = lq < 0 ? 0 : (lq > p.max_seqlen_q ? p.max_seqlen_q : lq);
  if (q0 + lq > p.total_q) lq = static_cast<int>(p.total_q - q0 < 0 ? 0 : p.total_q - q0);
  lk = lk < 0 ? 0 : (lk > p.max_seqlen_k ? p.max_seqlen_k : lk);
  if (lk > p.max_blocks_per_seq * kBlock) lk = p.max_blocks_per_seq * kBlock;
  const int mrows = lq * G;
  const int m0 = mtile * kBM;
  if (m0 >= mrows) return;                   // uniform over the workgroup

  // Key range this workgroup needs.
  const int i_last = min(lq - 1, (m0 + kBM - 1) / G);
  int kend = lk;
  if (p.causal) kend = min(lk, lk - lq + i_last + 1);
  kend = kend < 0 ? 0 : kend;
  const int ntiles = (kend + kBN - 1) / kBN;

  // This lane's row: M row m -> query position i, head h.
  const int m = m0 + wave * 32 + j;
  const bool row_ok = m < mrows;
  const int i_pos = row_ok ? m / G : 0;
  const int h = m % G;
  // Last key this row may see.
  const int lim = row_ok ? (p.causal ? lk - lq + i_pos : lk - 1) : lk - 1;
  // Smallest limit of the wave: tiles entirely below it need no mask.
  const int wave_m0 = m0 + wave * 32;
  const int wave_lim = p.causal ? lk - lq + min(wave_m0 / G, lq - 1) : lk - 1;

  // Q^T as the B operand: lane (j, hh) holds dims s * kK + hh * kPer + e.
  op_t qb[S::kQSteps];
  {
    const char* qrow = p.q + ((static_cast<int64_t>(q0) + i_pos) * p.num_heads +
                              kvh * G + h) * S::kRow;
#pragma unroll
    for (int s = 0; s < S::kQSteps; ++s) {
      if constexpr (S::kBf16) {
        qb[s] = row_ok ? ld16(qrow + (s * M::kK + hh * M::kPer) * 2)
                       : make_uint4(0, 0, 0, 0);
      } else {
        qb[s] = row_ok ? *reinterpret_cast<const float*>(
                             qrow + (s * M::kK + hh) * 4)
                       : 0.f;
      }
    }
  }

  const int64_t row_stride = static_cast<int64_t>(p.num_kv_heads) * S::kRow;
  const int32_t* btab = p.block_tables +
                        static_cast<int64_t>(b) * p.max_blocks_per_seq;

  // Tile staging (see PrefillShape): thread t owns chunk column c of keys
  // kg * kKpt .. kg * kKpt + kKpt - 1 of the tile.
  const int st_c = tid % S::kChunks;
  const int st_k0 = (tid / S::kChunks) * S::kKpt;
  uint4 kst[S::kKpt], vst[S::kKpt];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int u = 0; u < S::kKpt; ++u) {
      const int kpos = kt * kBN + st_k0 + u;
      kst[u] = make_uint4(0, 0, 0, 0);
      vst[u] = make_uint4(0, 0, 0, 0);
      if (kpos < lk) {
        const int blk = btab[kpos / kBlock];
        if (blk >= 0 && blk < p.num_blocks) {
          const int64_t off = (static_cast<int64_t>(blk) * kBlock + kpos % kBlock) *
                                  row_stride + static_cast<int64_t>(kvh) * S::kRow +
                              st_c * 16;
          kst[u] = ld16(p.k_cache + off);
          vst[u] = ld16(p.v_cache + off);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < S::kKpt; ++u)
      *reinterpret_cast<uint4*>(s_k + (st_k0 + u) * S::kKPitch + st_c * 16) = kst[u];
    if constexpr (S::kBf16) {
      // transpose kKpt keys x 8 dims in registers: dim 2w (2w+1) of key u is
      // the low (high) half of dword w of vst[u].
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t x[S::kKpt];
#pragma unroll
        for (int u = 0; u < S::kKpt; ++u)
          x[u] = w == 0 ? vst[u].x : w == 1 ? vst[u].y : w == 2 ? vst[u].z : vst[u].w;
        char* lo_row = s_v + (st_c * 8 + 2 * w) * S::kVPitch + st_k0 * 2;
        char* hi_row = lo_row + S::kVPitch;
        if constexpr (S::kKpt == 4) {
          *reinterpret_cast<uint2*>(lo_row) =
              make_uint2(pack_lo(x[0], x[1]), pack_lo(x[2], x[3]));
          *reinterpret_cast<uint2*>(hi_row) =
              make_uint2(pack_hi(x[0], x[1]), pack_hi(x[2], x[3]));
        } else {
          *reinterpret_cast<uint32_t*>(lo_row) = pack_lo(x[0], x[1]);
          *reinterpret_cast<uint32_t*>(hi_row) = pack_hi(x[0], x[1]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < S::kKpt; ++u)
        *reinterpret_cast<uint4*>(s_v + (st_k0 + u) * S::kVPitch + st_c * 16) = vst[u];
    }
  };

  f32x16_v oacc[S::kDTiles];
#pragma unroll
  for (int t = 0; t < S::kDTiles; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float run_max = -INFINITY;   // reference max of this row (scaled, log2)
  float run_sum = 0.f;         // this lane half's share of the row sum

  if (ntiles > 0) load_tile(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();           // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (kt + 1 < ntiles) load_tile(kt + 1);

    // ---- S^T = K Q^T: two 32-key M-tiles ------------------------------
    f32x16_v sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
      const char* krow = s_k + (t * 32 + j) * S::kKPitch;
#pragma unroll
      for (int s = 0; s < S::kQSteps; ++s) {
        op_t a;
        if constexpr (S::kBf16) {
          a = *reinterpret_cast<const uint4*>(krow + (s * M::kK + hh * M::kPer) * 2);
        } else {
          a = *reinterpret_cast<const float*>(krow + (s * M::kK + hh) * 4);
        }
        sacc[t] = M::run(a, qb[s], sacc[t]);
      }
    }

    // ---- online softmax for this lane's row ---------------------------
    // Logits stay raw; scale * log2(e) > 0 enters through one FMA with the
    // (scaled) running max.  Masked keys: raw -inf -> weight exactly 0.
    const int kbase = kt * kBN;
    const bool need_mask = kbase + kBN - 1 > wave_lim || kbase + kBN > lk;
    float tmax = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kpos = kbase + t * 32 + (r / 4) * 8 + hh * 4 + r % 4;
          sacc[t][r] = kpos <= lim ? sacc[t][r] : -INFINITY;
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[t][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave)) * p.scale_log2;
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

    // ---- O^T += V^T P^T -------------------------------------------------
#pragma unroll
    for (int s = 0; s < S::kPvSteps; ++s) {
      op_t bop;
      if constexpr (S::kBf16) {
        // keys (2s + e/4) * 8 + hh * 4 + e % 4 of the tile: accumulator
        // registers (s % 2) * 8 .. + 7 of S^T M-tile s / 2.
        const int t = s / 2;
        const int r0 = (s % 2) * 8;
        bop.x = pack_bf16x2(sacc[t][r0 + 0], sacc[t][r0 + 1]);
        bop.y = pack_bf16x2(sacc[t][r0 + 2], sacc[t][r0 + 3]);
        bop.z = pack_bf16x2(sacc[t][r0 + 4], sacc[t][r0 + 5]);
        bop.w = pack_bf16x2(sacc[t][r0 + 6], sacc[t][r0 + 7]);
      } else {
        // step s covers keys (r/4) * 8 + hh * 4 + r % 4 (+ 32 for M-tile 1)
        // with r = s % 16: one probability per lane.
        bop = sacc[s / 16][s % 16];
      }
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt) {
        const int dim = dt * 32 + j;
        op_t a;
        if constexpr (S::kBf16) {
          const char* vt = s_v + dim * S::kVPitch;
          const uint2 lo = *reinterpret_cast<const uint2*>(vt + (s * 16 + hh * 4) * 2);
          const uint2 hi = *reinterpret_cast<const uint2*>(vt + (s * 16 + 8 + hh * 4) * 2);
          a = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          const int r = s % 16;
          const int key = (s / 16) * 32 + (r / 4) * 8 + hh * 4 + r % 4;
          a = *reinterpret_cast<const float*>(s_v + key * S::kVPitch + dim * 4);
        }
        oacc[dt] = M::run(a, bop, oacc[dt]);
      }
    }
  }

  // ---- normalise and write: lane (j, hh) holds dims (r/4)*8 + hh*4 + r%4
  // of each 32-dim tile for its row.
  const float total = run_sum + __shfl_xor(run_sum, 32, kWave);
  if (!row_ok) return;
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

template <typename T, int D, int G>
hipError_t launch_typed(const PrefillParams& prm, int num_seqs, int max_seqlen_q,
                        int num_kv_heads, hipStream_t stream) {
  using S = PrefillShape<T, D>;
  const int mtiles = (max_seqlen_q * G + kBM - 1) / kBM;
  const size_t lds = static_cast<size_t>(kBN) * S::kKPitch + S::kVBytes;
  if (lds > 65536) {
    static bool raised = false;   // once per kernel instantiation
    if (!raised) {
      hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&prefill_kernel<T, D, G>),
          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  hipLaunchKernelGGL((prefill_kernel<T, D, G>), dim3(mtiles, num_kv_heads, num_seqs),
                     dim3(kThreads), lds, stream, prm);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_group(const PrefillParams& prm, int g, int num_seqs,
                          int max_seqlen_q, int num_kv_heads, hipStream_t s) {
  switch (g) {
    case 1: return launch_typed<T, D, 1>(prm, num_seqs, max_seqlen_q, num_kv_heads, s);
    case 2: return launch_typed<T, D, 2>(prm, num_seqs, max_seqlen_q, num_kv_heads, s);
    case 4: return launch_typed<T, D, 4>(prm, num_seqs, max_seqlen_q, num_kv_heads, s);
    case 8: return launch_typed<T, D, 8>(prm, num_seqs, max_seqlen_q, num_kv_heads, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t prefill_workspace_bytes(int, int, int, int, int, int) { return 0; }

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
    if (a.head_dim == 128)
      return dispatch_group<bf16_t, 128>(prm, g, a.num_seqs, a.max_seqlen_q, a.num_kv_heads, stream);
    return dispatch_group<bf16_t, 64>(prm, g, a.num_seqs, a.max_seqlen_q, a.num_kv_heads, stream);
  }
  if (a.head_dim == 128)
    return dispatch_group<float, 128>(prm, g, a.num_seqs, a.max_seqlen_q, a.num_kv_heads, stream);
  return dispatch_group<float, 64>(prm, g, a.num_seqs, a.max_seqlen_q, a.num_kv_heads, stream);
}

}  // namespace pa
