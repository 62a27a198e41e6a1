// C ABI of libpa: host-side validation of scalar arguments, then dispatch to
// the kernel launchers.  Declarations and the contract live in include/pa.h.
#include "../../include/pa.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include "pa_internal.h"

namespace {

constexpr int32_t kAbiVersion = 1;

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int elem_bytes(pa_dtype dtype) { return dtype == PA_BF16 ? 2 : 4; }

bool dtype_ok(pa_dtype dtype) { return dtype == PA_F32 || dtype == PA_BF16; }

bool group_ok(int32_t num_heads, int32_t num_kv_heads) {
  if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return false;
  const int g = num_heads / num_kv_heads;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

// Shared checks of the attention entry points.
pa_status check_attention(int32_t block_size, int32_t num_seqs,
                          int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t max_blocks_per_seq,
                          int64_t num_blocks, pa_dtype dtype) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq < 0 || num_blocks < 0 || block_size <= 0)
    return PA_ERR_SHAPE;
  if (num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 16) return PA_ERR_UNSUPPORTED;
  if (!group_ok(num_heads, num_kv_heads)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size is negative or inconsistent";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: head_dim, block_size, GQA ratio, dtype or "
             "alignment not supported";
    case PA_ERR_WORKSPACE:
      return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: kernel launch failed";
    case PA_ERR_SCRATCH_LIMIT:
      return "PA_ERR_SCRATCH_LIMIT: these sizes need more workspace than the "
             "library's static 32 MiB decode scratch holds; call pa_decode "
             "with a workspace instead";
  }
  return "PA_ERR_?: unknown status";
}

int32_t pa_abi_version(void) { return kAbiVersion; }

pa_status pa_store_kv(const void* k, const void* v, void* k_cache,
                      void* v_cache, const int32_t* slot_mapping,
                      int64_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int64_t num_slots, pa_dtype dtype,
                      void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_slots < 0)
    return PA_ERR_SHAPE;
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  const int64_t row_bytes =
      static_cast<int64_t>(num_kv_heads) * head_dim * elem_bytes(dtype);
  if (row_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  hipError_t e = pa::launch_store_kv(k, v, k_cache, v_cache, slot_mapping,
                                     num_tokens, row_bytes, num_slots,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache,
                         const int32_t* block_pairs, int64_t num_pairs,
                         int64_t block_bytes, int64_t num_blocks,
                         void* stream) {
  if (num_pairs < 0 || block_bytes < 0 || num_blocks < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0 || block_bytes == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return PA_ERR_NULL;
  if (block_bytes % 16 != 0 || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, block_pairs,
                                        num_pairs, block_bytes, num_blocks,
                                        static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

namespace {

// Which kernel a decode call runs.  A decode (bf16 q, bf16 or E4M3 cache)
// that the decode kernel would split into partitions runs on the small-row
// attention kernel (one query row per sequence) when that kernel's plan
// needs no partitions -- a batch with >= 1024 (sequence, KV head pair) work
// items -- or partitions of >= 2048 tokens: it streams the cache faster
// (8B-shaped step 744 -> 688 us; 8-bit cache 415-448 -> 356-360 us; 192
// sequences of U[256, 8192] in 2 partitions 550 -> 502 us; 48-160-sequence
// batches with 2-8 partitions of 2,752-4,096 tokens 2-22 % faster).  With
// shorter partitions its per-item start and combine weigh more (64
// sequences in 4 partitions of 1,024: 102.6 -> 107.3 us; 128 sequences in
// 2 of 1,280: 128 -> 152 us), so those, every decode without partitions
// and every fp32 decode run on the decode kernel.
constexpr int kRowsMinPartitionTokens = 2048;

struct DecodeRoute {
  pa::DecodePlan decode;
  pa::VerifyPlan rows;
  bool use_rows;
  size_t bytes;   // workspace the chosen kernel needs
};

DecodeRoute route_decode(int num_seqs, int num_heads, int num_kv_heads,
                         int head_dim, int max_context_len, bool bf16) {
  DecodeRoute r{};
  r.decode = pa::plan_decode(num_seqs, num_heads, num_kv_heads, head_dim,
                             max_context_len);
  r.rows = pa::plan_verify(num_seqs, num_heads, num_kv_heads, head_dim, 1,
                           max_context_len);
  r.use_rows = bf16 && r.decode.workspace_bytes > 0 && r.rows.use &&
               (r.rows.num_partitions == 1 ||
                r.rows.partition_tokens >= kRowsMinPartitionTokens);
  r.bytes = r.use_rows ? r.rows.workspace_bytes : r.decode.workspace_bytes;
  return r;
}

}  // namespace

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len <= 0)
    return 0;
  // Either element type: the larger of the two kernels' needs.
  const DecodeRoute f = route_decode(num_seqs, num_heads, num_kv_heads, head_dim,
                                     max_context_len, false);
  const DecodeRoute b = route_decode(num_seqs, num_heads, num_kv_heads, head_dim,
                                     max_context_len, true);
  return f.bytes > b.bytes ? f.bytes : b.bytes;
}

pa_status pa_decode(void* out, const void* q, const void* k_cache,
                    const void* v_cache, int64_t num_blocks,
                    int32_t block_size, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t max_context_len, int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, float scale, void* workspace,
                    size_t workspace_bytes, pa_dtype dtype, void* stream) {
  pa_status st = check_attention(block_size, num_seqs, num_heads, num_kv_heads,
                                 head_dim, max_blocks_per_seq, num_blocks,
                                 dtype);
  if (st != PA_OK) return st;
  if (max_context_len < 0) return PA_ERR_SHAPE;
  if (!(scale > 0.f) || !std::isfinite(scale)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !context_lens) return PA_ERR_NULL;
  if (max_context_len > 0 && (!k_cache || !v_cache || !block_tables))
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  const DecodeRoute route = route_decode(num_seqs, num_heads, num_kv_heads,
                                         head_dim, max_context_len, dtype == PA_BF16);
  if (route.bytes > 0 && (!workspace || workspace_bytes < route.bytes))
    return PA_ERR_WORKSPACE;
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.scale = scale;
  a.workspace = workspace;
  a.bf16 = dtype == PA_BF16;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = route.use_rows ? pa::launch_verify_decode(a, route.rows, hs)
                                : pa::launch_decode(a, route.decode, hs);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_seqlen_q <= 0 || max_seqlen_k <= 0)
    return 0;
  return pa::prefill_workspace_bytes(num_seqs, num_heads, num_kv_heads,
                                     head_dim, max_seqlen_q, max_seqlen_k);
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache,
                            const void* v_cache, int64_t num_blocks,
                            int32_t block_size, const int32_t* block_tables,
                            int32_t max_blocks_per_seq,
                            const int32_t* context_lens,
                            int32_t max_context_len, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, float scale, pa_dtype dtype,
                            void* stream) {
  pa_status st = check_attention(block_size, num_seqs, num_heads, num_kv_heads,
                                 head_dim, max_blocks_per_seq, num_blocks,
                                 dtype);
  if (st != PA_OK) return st;
  if (max_context_len < 0) return PA_ERR_SHAPE;
  if (!(scale > 0.f) || !std::isfinite(scale)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !context_lens) return PA_ERR_NULL;
  if (max_context_len > 0 && (!k_cache || !v_cache || !block_tables))
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  const DecodeRoute route = route_decode(num_seqs, num_heads, num_kv_heads,
                                         head_dim, max_context_len, dtype == PA_BF16);
  if (route.bytes > pa::kDecodeScratchBytes) return PA_ERR_SCRATCH_LIMIT;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  if (route.bytes > 0 && pa::decode_scratch(s, &scratch) != hipSuccess)
    return PA_ERR_LAUNCH;
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.scale = scale;
  a.workspace = scratch;
  a.bf16 = dtype == PA_BF16;
  hipError_t e = route.use_rows ? pa::launch_verify_decode(a, route.rows, s)
                                : pa::launch_decode(a, route.decode, s);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_prefill_varlen(void* out, const void* q, int64_t total_q,
                            const void* k_cache, const void* v_cache,
                            int64_t num_blocks, int32_t block_size,
                            const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, float scale, int32_t causal,
                            void* workspace, size_t workspace_bytes,
                            pa_dtype dtype, void* stream) {
  pa_status st = check_attention(block_size, num_seqs, num_heads, num_kv_heads,
                                 head_dim, max_blocks_per_seq, num_blocks,
                                 dtype);
  if (st != PA_OK) return st;
  if (total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return PA_ERR_SHAPE;
  if (!(scale > 0.f) || !std::isfinite(scale)) return PA_ERR_SHAPE;
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PA_OK;
  if (!out || !q || !cu_seqlens_q || !cu_seqlens_k) return PA_ERR_NULL;
  if (max_seqlen_k > 0 && (!k_cache || !v_cache || !block_tables))
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  const size_t need = pa_prefill_workspace_bytes(
      num_seqs, num_heads, num_kv_heads, head_dim, max_seqlen_q, max_seqlen_k);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return PA_ERR_WORKSPACE;
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.total_q = total_q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.max_seqlen_q = max_seqlen_q;
  a.max_seqlen_k = max_seqlen_k;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.scale = scale;
  a.causal = causal != 0;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.bf16 = dtype == PA_BF16;
  hipError_t e = pa::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

size_t pa_decode_shared_prefix_workspace_bytes(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t max_suffix_len, int32_t max_prefix_len,
    int32_t num_groups, int32_t max_group_size) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_suffix_len < 0 || max_prefix_len < 0 || num_groups < 0 ||
      max_group_size < 0 || num_heads % num_kv_heads != 0)
    return 0;
  return pa::plan_shared_prefix(num_seqs, num_heads, num_kv_heads, head_dim,
                                max_suffix_len, max_prefix_len, num_groups,
                                max_group_size)
      .workspace_bytes;
}

pa_status pa_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* prefix_lens, int32_t max_suffix_len,
    int32_t max_prefix_len, const int32_t* groups, int32_t num_groups,
    int32_t max_group_size, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, float scale, void* workspace,
    size_t workspace_bytes, pa_dtype dtype, void* stream) {
  pa_status st = check_attention(block_size, num_seqs, num_heads, num_kv_heads,
                                 head_dim, max_blocks_per_seq, num_blocks,
                                 dtype);
  if (st != PA_OK) return st;
  if (max_suffix_len < 0 || max_prefix_len < 0 || num_groups < 0 ||
      max_group_size < 0)
    return PA_ERR_SHAPE;
  const int64_t max_len = static_cast<int64_t>(max_suffix_len) + max_prefix_len;
  if (max_len > 0x7fffffff) return PA_ERR_SHAPE;
  if (!(scale > 0.f) || !std::isfinite(scale)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !context_lens || !prefix_lens) return PA_ERR_NULL;
  if (max_len > 0 && (!k_cache || !v_cache || !block_tables))
    return PA_ERR_NULL;
  if (num_groups > 0 && !groups) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  const pa::SharedPrefixPlan plan = pa::plan_shared_prefix(
      num_seqs, num_heads, num_kv_heads, head_dim, max_suffix_len,
      max_prefix_len, num_groups, max_group_size);
  if (!workspace || workspace_bytes < plan.workspace_bytes)
    return PA_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  pa::PrefixArgs pre{};
  pre.q = q;
  pre.k_cache = k_cache;
  pre.v_cache = v_cache;
  pre.num_blocks = num_blocks;
  pre.block_tables = block_tables;
  pre.max_blocks_per_seq = max_blocks_per_seq;
  pre.prefix_lens = prefix_lens;
  pre.context_lens = context_lens;
  pre.max_context_len = static_cast<int>(max_len);
  pre.groups = groups;
  pre.num_groups = num_groups;
  pre.max_group_size = max_group_size;
  pre.max_prefix_len = max_prefix_len;
  pre.num_seqs = num_seqs;
  pre.num_heads = num_heads;
  pre.num_kv_heads = num_kv_heads;
  pre.head_dim = head_dim;
  pre.scale = scale;
  pre.workspace = workspace;
  pre.bf16 = dtype == PA_BF16;
  hipError_t e = pa::launch_prefix_partials(pre, plan, s);
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = static_cast<int>(max_len);
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.scale = scale;
  a.workspace = workspace;
  a.bf16 = dtype == PA_BF16;
  a.prefix_lens = prefix_lens;
  e = pa::launch_decode_suffix(a, plan, s);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_store_kv_fp8(const void* k, const void* v, void* k_cache,
                          void* v_cache, const int32_t* slot_mapping,
                          int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int64_t num_slots,
                          pa_dtype src_dtype, float k_scale, float v_scale,
                          void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_slots < 0)
    return PA_ERR_SHAPE;
  if (!(k_scale > 0.f) || !std::isfinite(k_scale) || !(v_scale > 0.f) ||
      !std::isfinite(v_scale))
    return PA_ERR_SHAPE;
  if (!dtype_ok(src_dtype)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (row_elems % 8 != 0) return PA_ERR_UNSUPPORTED;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  hipError_t e = pa::launch_store_kv_fp8(
      k, v, k_cache, v_cache, slot_mapping, num_tokens, row_elems, num_slots,
      src_dtype == PA_BF16, 1.0f / k_scale, 1.0f / v_scale,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_decode_fp8(void* out, const void* q, const void* k_cache,
                        const void* v_cache, int64_t num_blocks,
                        int32_t block_size, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t max_context_len, int32_t num_seqs,
                        int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, float scale, float k_scale,
                        float v_scale, void* workspace, size_t workspace_bytes,
                        void* stream) {
  pa_status st = check_attention(block_size, num_seqs, num_heads, num_kv_heads,
                                 head_dim, max_blocks_per_seq, num_blocks,
                                 PA_BF16);
  if (st != PA_OK) return st;
  if (head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (max_context_len < 0) return PA_ERR_SHAPE;
  if (!(scale > 0.f) || !std::isfinite(scale) || !(k_scale > 0.f) ||
      !std::isfinite(k_scale) || !(v_scale > 0.f) || !std::isfinite(v_scale))
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !context_lens) return PA_ERR_NULL;
  if (max_context_len > 0 && (!k_cache || !v_cache || !block_tables))
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  // Same route as a bfloat16 cache: large batches on the small-row kernel.
  const DecodeRoute route = route_decode(num_seqs, num_heads, num_kv_heads,
                                         head_dim, max_context_len, true);
  if (route.bytes > 0 && (!workspace || workspace_bytes < route.bytes))
    return PA_ERR_WORKSPACE;
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.scale = scale;
  a.workspace = workspace;
  a.bf16 = true;
  a.fp8_cache = true;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = route.use_rows ? pa::launch_verify_decode(a, route.rows, hs)
                                : pa::launch_decode(a, route.decode, hs);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
