// Internal launch interface between the C ABI (api.cpp) and the kernel
// translation units.  Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Compute units of the current device (looked up once per device).
int device_cus();

// ---- store -------------------------------------------------------------
hipError_t launch_store_kv(const void* k, const void* v, void* k_cache,
                           void* v_cache, const int32_t* slot_mapping,
                           int64_t num_tokens, int64_t row_bytes,
                           int64_t num_slots, hipStream_t stream);

// Quantising store into E4M3 caches: row t (num_kv_heads * head_dim
// elements of bf16 or fp32) goes to flat slot slot_mapping[t] as the codes
// of x * inv_scale (per cache), saturated to +-448.
hipError_t launch_store_kv_fp8(const void* k, const void* v, void* k_cache,
                               void* v_cache, const int32_t* slot_mapping,
                               int64_t num_tokens, int64_t row_elems,
                               int64_t num_slots, bool bf16_src,
                               float k_inv_scale, float v_inv_scale,
                               hipStream_t stream);

// ---- block copy (copy-on-write) -----------------------------------------
hipError_t launch_copy_blocks(void* k_cache, void* v_cache,
                              const int32_t* block_pairs, int64_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks,
                              hipStream_t stream);

// ---- decode ------------------------------------------------------------
struct DecodePlan {
  int partition_tokens;  // tokens per context partition (multiple of 512)
  int num_partitions;    // ceil(max_context_len / partition_tokens), >= 1
  size_t workspace_bytes;
  size_t off_max, off_sum, off_acc;  // byte offsets inside the workspace
  bool use_order;        // longest-first schedule of (sequence, partition)
  size_t off_order;      // its int32 [num_seqs * num_partitions] array
  bool inline_rank;      // longest first, each workgroup ranking its own item
};

DecodePlan plan_decode(int num_seqs, int num_heads, int num_kv_heads,
                       int head_dim, int max_context_len);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  int64_t num_blocks;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int max_context_len;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int head_dim;
  float scale;
  void* workspace;
  bool bf16;
  const int32_t* prefix_lens = nullptr;   // shared-prefix decode only
  // E4M3 cache (q / out bf16): K = code * k_scale, V = code * v_scale.
  bool fp8_cache = false;
  float k_scale = 1.f;
  float v_scale = 1.f;
};

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan,
                         hipStream_t stream);

// Size of the library's static decode scratch array (one per GPU, kept
// until the process ends): the workspace of pa_decode_noalloc.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;

// Device address of the static scratch array on the device `stream`
// belongs to (the current device for the null stream).  The address is
// looked up once per device, with that device current, and cached.
hipError_t decode_scratch(hipStream_t stream, void** ptr);

// ---- shared-prefix (cascade) decode ------------------------------------
struct SharedPrefixPlan {
  DecodePlan suffix;         // partitions over [prefix, L_b) (workspace unused)
  int prefix_chunk_tokens;   // keys per prefix partial, multiple of 64
  int prefix_chunks;         // prefix partial slots per (sequence, head)
  int total_slots;           // suffix.num_partitions + prefix_chunks
  // The prefix pass runs, and its last workgroup writes the suffix pass's
  // longest-first schedule at suffix.off_order (no plan kernel).
  bool order_in_prefix;
  size_t workspace_bytes;
  size_t off_max, off_sum, off_acc;  // [B, Hq, total_slots] (acc: x D)
};

SharedPrefixPlan plan_shared_prefix(int num_seqs, int num_heads,
                                    int num_kv_heads, int head_dim,
                                    int max_suffix_len, int max_prefix_len,
                                    int num_groups, int max_group_size);

// Suffix pass + merge of a shared-prefix decode: a.prefix_lens set,
// a.max_context_len the bound of L_b.  Writes the suffix partials and then
// merges them with the prefix partials already in the workspace.
hipError_t launch_decode_suffix(const DecodeArgs& a,
                                const SharedPrefixPlan& plan,
                                hipStream_t stream);

// Prefix pass: for each group, the attention of every member's query rows
// over the group's shared prefix keys, in chunks, as partials (unnormalised
// output, reference max, sum) in slots suffix.num_partitions + chunk.
struct PrefixArgs {
  const void* q;             // [num_seqs, Hq, D]
  const void* k_cache;
  const void* v_cache;
  int64_t num_blocks;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* prefix_lens;   // [num_seqs]
  const int32_t* context_lens;  // [num_seqs]: for the suffix schedule
  int max_context_len;          // the suffix pass's bound on context_lens
  const int32_t* groups;        // [num_groups, 2]: first sequence, count
  int num_groups;
  int max_group_size;
  int max_prefix_len;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int head_dim;
  float scale;
  void* workspace;
  bool bf16;
};

hipError_t launch_prefix_partials(const PrefixArgs& a,
                                  const SharedPrefixPlan& plan,
                                  hipStream_t stream);

// ---- prefill -----------------------------------------------------------
struct PrefillArgs {
  void* out;
  const void* q;
  int64_t total_q;
  const void* k_cache;
  const void* v_cache;
  int64_t num_blocks;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int max_seqlen_q;
  int max_seqlen_k;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int head_dim;
  float scale;
  bool causal;
  void* workspace;
  size_t workspace_bytes;
  bool bf16;
};

size_t prefill_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads,
                               int head_dim, int max_seqlen_q,
                               int max_seqlen_k);

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Small-row path of the varlen prefill (bfloat16): used when the packed
// rows per KV head, G * max_seqlen_q, are at most 64 (a verify pass, a
// one-row chunk).  Split-context partitions over the keys, merged when
// there are several; a plan kernel orders the work longest first and
// persistent workgroups draw it from a counter in the workspace.
struct VerifyPlan {
  bool use;              // these sizes take the small-row path
  int row_tiles;         // 16-row tiles per KV head: 1, 2 or 4
  int heads_per_item;    // KV heads one workgroup takes at a time: 1 or 2
  int partition_tokens;  // keys per partition (multiple of 64)
  int num_partitions;    // >= 1
  size_t workspace_bytes;
  size_t off_max, off_sum, off_acc;  // partials (num_partitions > 1)
  size_t off_order;      // int32 [num_seqs * num_partitions], longest first
  size_t off_counter;    // int32 ticket counter
};

VerifyPlan plan_verify(int num_seqs, int num_heads, int num_kv_heads,
                       int head_dim, int max_seqlen_q, int max_seqlen_k);

hipError_t launch_verify(const PrefillArgs& a, const VerifyPlan& plan,
                         hipStream_t stream);

// bfloat16 decode on the same kernel: one query row per sequence, keys
// 0 .. context_lens[b] - 1.  The plan is plan_verify(num_seqs, num_heads,
// num_kv_heads, head_dim, 1, max_context_len).
hipError_t launch_verify_decode(const DecodeArgs& a, const VerifyPlan& plan,
                                hipStream_t stream);

}  // namespace pa
