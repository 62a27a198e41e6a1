/*
 * pa.h -- C ABI of libpa, the MI355X (gfx950) paged KV-cache hot path.
 *
 * Operations over a block-table-indexed KV cache:
 *
 *   pa_store_kv        scatter new K/V rows into their physical slots
 *   pa_copy_blocks     copy whole blocks (the data side of copy-on-write)
 *   pa_decode_shared_prefix  decode where groups of sequences share leading
 *                      blocks: the shared keys are read once per group
 *   pa_store_kv_fp8, pa_decode_fp8  the same over an 8-bit (E4M3) cache
 *   pa_decode          one query row per sequence against its paged context
 *   pa_prefill_varlen  packed variable-length (chunked) prefill, causal,
 *                      history read through block tables
 *
 * Sources.  The data contract follows "3.6 ModelRunner, CUDA Graph, and
 * benchmarks" (a source reading of nano-vllm): section 2 (prepare_prefill /
 * prepare_decode: slot_mapping, cu_seqlens_q / cu_seqlens_k, max_seqlen_q /
 * max_seqlen_k, context_lens, -1 padded block_tables), section 3 (the
 * per-step attention context), section 4 (the cache tensor layout) and
 * section 5 (padding: slot -1 writes nothing, context length 0 reads
 * nothing, stale block-table entries are never read).  Paging itself is the
 * "Warmup Guide -- Inference Serving Internals", Chapter 3.  The attention
 * each row computes is out = softmax(scale * q K^T) V (the pages name the
 * kernels but do not write the formula out).
 *
 * Layouts (all row-major, contiguous, element type `pa_dtype`):
 *   q, out (decode)        [num_seqs, num_heads, head_dim]
 *   q, out (prefill)       [total_q, num_heads, head_dim], sequences packed
 *                          end to end as cu_seqlens_q says
 *   k, v (store)           [num_tokens, num_kv_heads, head_dim]
 *   k_cache, v_cache       [num_blocks, block_size, num_kv_heads, head_dim],
 *                          i.e. flat [num_slots, num_kv_heads, head_dim] with
 *                          slot = block_id * block_size + offset
 *   block_tables           int32 [num_seqs, max_blocks_per_seq]; row b lists
 *                          sequence b's physical blocks in logical order;
 *                          entries past ceil(len / block_size) are padding
 *                          (-1 or stale) and are never read
 *
 * GQA: query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Pointers.  Every tensor pointer is a device pointer, 16-byte aligned.  The
 * caller owns every buffer; the library never allocates, frees, or keeps a
 * pointer after the call returns.  Scratch space is a caller-provided
 * workspace sized by the *_workspace_bytes queries -- except for
 * pa_decode_noalloc, which uses a static scratch array the library holds on
 * each GPU (see there).
 *
 * Streams.  Every call only enqueues work on `stream` (a hipStream_t; NULL
 * is the default stream) and returns; it never synchronises, allocates or
 * copies to the host, so it can be captured in a HIP graph.  Ordering
 * between calls (store before attend) is the caller's, by stream order.
 *
 * Errors.  Host-side checks of the scalar arguments return a status code;
 * nothing aborts and nothing throws across the ABI.  Device-side data
 * (slots, block ids, lengths, cu_seqlens) are preconditions -- see each
 * call -- but the kernels clamp or skip values that would address memory
 * outside the buffers described by the scalar arguments, so a violated
 * precondition gives wrong numbers, never an out-of-bounds access.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,         /* a required pointer is NULL                    */
  PA_ERR_SHAPE = 2,        /* a size is negative / inconsistent             */
  PA_ERR_UNSUPPORTED = 3,  /* head_dim, block_size, GQA ratio, dtype or
                              pointer alignment not supported               */
  PA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than the query says */
  PA_ERR_LAUNCH = 5,       /* the HIP runtime rejected a kernel launch      */
  PA_ERR_SCRATCH_LIMIT = 6 /* pa_decode_noalloc: the sizes need more than the
                              static scratch holds                          */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* pa_status_string(pa_status status);

/* ABI version of this header; bumps on any signature change. */
int32_t pa_abi_version(void);

/*
 * pa_store_kv -- write new K/V rows into the cache at their slots.
 *
 * For every t in [0, num_tokens): if slot_mapping[t] >= 0, the whole row
 * k[t] (num_kv_heads * head_dim elements) is copied bit for bit to flat slot
 * slot_mapping[t] of k_cache, and v[t] likewise to v_cache.  A negative slot
 * (batch padding) writes nothing.  ModelRunner page, sections 2 and 5.
 *
 *   k, v          device, [num_tokens, num_kv_heads, head_dim]
 *   k_cache,
 *   v_cache       device, [num_slots, num_kv_heads, head_dim] (any block size)
 *   slot_mapping  device int32 [num_tokens]
 *   num_slots     num_blocks * block_size of the cache
 *
 * Preconditions: non-negative slots are distinct (a duplicate leaves one of
 * the rows, unspecified which).  Slots >= num_slots are skipped.
 * Requires num_kv_heads * head_dim * element size to be a multiple of 16.
 * num_tokens == 0 is a no-op returning PA_OK.
 */
pa_status pa_store_kv(const void* k, const void* v, void* k_cache,
                      void* v_cache, const int32_t* slot_mapping,
                      int64_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int64_t num_slots, pa_dtype dtype,
                      void* stream);

/*
 * pa_copy_blocks -- copy whole cache blocks, bit for bit.
 *
 * For every i in [0, num_pairs): block block_pairs[2i + 1] (destination) of
 * k_cache and of v_cache becomes a copy of block block_pairs[2i] (source).
 * This is the data side of copy-on-write: a sequence about to write into a
 * block that other sequences also hold copies that one block into a fresh
 * block, lowers the shared block's reference count and writes into its copy
 * ("Warmup Guide -- Inference Serving Internals", Chapter 4).  The
 * reference counts and block tables are host metadata, not this call's.
 *
 *   k_cache, v_cache  device, [num_blocks, block_bytes bytes] each (any
 *                     block size, head count, head_dim or element type)
 *   block_pairs       device int32 [num_pairs, 2]: (source, destination)
 *   block_bytes       bytes of one block of one cache, a multiple of 16
 *
 * A pair with an id outside [0, num_blocks), or with source == destination,
 * copies nothing.  Preconditions: destinations are distinct and no block is
 * both a source and a destination in the same call (the copies run in
 * parallel; a chain or a repeated destination leaves unspecified contents).
 * num_pairs == 0 or block_bytes == 0 is a no-op returning PA_OK;
 * PA_ERR_UNSUPPORTED for block_bytes above 1 GiB or unaligned pointers.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache,
                         const int32_t* block_pairs, int64_t num_pairs,
                         int64_t block_bytes, int64_t num_blocks,
                         void* stream);

/*
 * Bytes of workspace pa_decode needs for these sizes, either element type
 * (the larger need of the two; 0 when one context partition covers
 * max_context_len and no merge pass is needed, and 0 for a non-positive
 * size, which pa_decode rejects).  The workspace holds the partitions'
 * partial results and, for large grids of more than 64 sequences, a
 * longest-first work order (and a work counter) that a one-workgroup plan
 * kernel writes at the start of each call (every call rewrites them, so
 * calls that share a workspace on one stream are safe).  Up to 64
 * sequences the workgroups find their place in that order themselves.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len);

/*
 * pa_decode -- decode attention over a paged cache.
 *
 * For sequence b with L = context_lens[b] (the count includes the token being
 * decoded, whose K/V the caller stored first) and each query head h:
 *   out[b, h] = softmax_j(scale * q[b, h] . K_b[j]) V_b[j],  j in [0, L)
 * where K_b[j] is k_cache[block_tables[b, j / block_size], j % block_size,
 * h / G] and G = num_heads / num_kv_heads.  L == 0 (batch padding) gives a
 * zero row.  ModelRunner page, section 2 (prepare_decode) and section 5.
 *
 * Split-context: the context is cut into fixed partitions processed in
 * parallel, each keeping its own running max and sum; a second pass merges
 * the partitions (the merge is skipped when one partition covers
 * max_context_len).  A large bf16 batch (one the decode kernel would split
 * into partitions, with >= 1024 (sequence, KV-head-pair) work items) runs
 * instead on the kernel of pa_prefill_varlen's small-row path (one query
 * row per sequence, MFMA dot products, persistent workgroups, no
 * partitions); all other calls run on the decode kernel (vector dot
 * products).  Both compute the same softmax; results agree to rounding.
 *
 *   out, q         device, [num_seqs, num_heads, head_dim]
 *   k_cache,
 *   v_cache        device, [num_blocks, block_size, num_kv_heads, head_dim]
 *   block_tables   device int32 [num_seqs, max_blocks_per_seq]
 *   context_lens   device int32 [num_seqs]
 *   max_context_len  host-known upper bound of context_lens (sizes the grid
 *                  without a device-to-host copy)
 *   workspace      device, >= pa_decode_workspace_bytes(...) bytes (may be
 *                  NULL when that is 0); contents on entry do not matter
 *
 * Supported: head_dim in {64, 128}; block_size == 16; num_heads /
 * num_kv_heads in {1, 2, 4, 8}; dtype F32 or BF16 (fp32 accumulation,
 * bf16 output rounded to nearest even); scale positive and finite
 * (PA_ERR_SHAPE otherwise; it is 1/sqrt(head_dim) in practice).
 * Preconditions: context_lens[b] <= max_context_len and
 * <= max_blocks_per_seq * block_size (larger values are clamped); the first
 * ceil(L / block_size) block ids of row b lie in [0, num_blocks) (an id
 * outside that range contributes nothing).
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache,
                    const void* v_cache, int64_t num_blocks,
                    int32_t block_size, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t max_context_len, int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, float scale, void* workspace,
                    size_t workspace_bytes, pa_dtype dtype, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, kernels and arguments as
 * pa_decode, without the workspace.  The partial results and the schedule
 * go to a static scratch array of 32 MiB (33,554,432 bytes) that the
 * library holds on each GPU it runs on until the process ends.  The call
 * allocates nothing; on its first call on a device it looks up that
 * device's array address once (hipGetSymbolAddress).
 *
 * Limit: calls whose kernel needs more than 33,554,432 bytes of workspace
 * return PA_ERR_SCRATCH_LIMIT and launch nothing.  For fp32 that need is
 * pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
 * max_context_len) (256 sequences x 32 query heads of head_dim 128 at
 * max_context_len 8192 need about 17 MB); a bf16 call that runs on the
 * small-row kernel needs only its schedule (4 bytes per sequence), which
 * the same query bounds.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (nothing needs to start at zero: each call writes what
 * it reads).  Calls that overlap on one GPU -- on different streams, or
 * from different host threads without stream ordering -- race on the
 * array and give wrong results; calls in order on one stream are safe.
 * Other arguments, errors and supported shapes: as pa_decode.
 */
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache,
                            const void* v_cache, int64_t num_blocks,
                            int32_t block_size, const int32_t* block_tables,
                            int32_t max_blocks_per_seq,
                            const int32_t* context_lens,
                            int32_t max_context_len, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, float scale, pa_dtype dtype,
                            void* stream);

/* Bytes of workspace pa_prefill_varlen needs for these sizes: the work
 * schedule, one int32 per (sequence, 128-row M-tile) item (0 when
 * max_seqlen_k is 0).  Written and read by each call when there are more
 * work items than one attention workgroup has threads; with fewer, every
 * workgroup ranks the items itself and the workspace is not touched.  Its
 * contents between calls mean nothing.  Calls that share a workspace on
 * one stream are safe; calls on different streams need their own. */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k);

/*
 * pa_prefill_varlen -- varlen (chunked) prefill attention, K/V read from the
 * paged cache.
 *
 * Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 * (Lq rows) and Lk = cu_seqlens_k[b+1] - cu_seqlens_k[b] keys, the first Lk
 * tokens of its block table (history and this step's tokens, which the
 * caller stored first).  With causal != 0 query row i sits at absolute
 * position Lk - Lq + i and sees keys 0 .. Lk - Lq + i (bottom-right
 * alignment: a chunk continues after its cached history); otherwise every
 * row sees all Lk keys.  ModelRunner page, section 2 (prepare_prefill), and
 * "10 Serving Engines", section 10.3 (chunked prefill).
 *
 *   out, q          device, [total_q, num_heads, head_dim]
 *   cu_seqlens_q/k  device int32 [num_seqs + 1], non-decreasing, from 0
 *   max_seqlen_q/k  host-known upper bounds of Lq / Lk
 *   block_tables    device int32 [num_seqs, max_blocks_per_seq]
 *   workspace       device, >= pa_prefill_workspace_bytes(...) bytes
 *
 * Supported: as pa_decode.  Preconditions: Lq <= Lk when causal; Lq <=
 * max_seqlen_q, Lk <= max_seqlen_k and <= max_blocks_per_seq * block_size
 * (larger values are clamped); rows past total_q are never touched.
 */
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
                            pa_dtype dtype, void* stream);

/* Bytes of workspace pa_decode_shared_prefix needs for these sizes (> 0
 * whenever num_seqs > 0): partial results, one slot per suffix partition and
 * per prefix chunk, for each (sequence, query head), and the suffix pass's
 * schedule (one int32 per (sequence, suffix partition)) where it uses one. */
size_t pa_decode_shared_prefix_workspace_bytes(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t max_suffix_len, int32_t max_prefix_len,
    int32_t num_groups, int32_t max_group_size);

/*
 * pa_decode_shared_prefix -- decode attention, same result as pa_decode, for
 * batches where groups of sequences share their leading cache blocks.
 *
 * Sharing: sequences that start with the same tokens hold the same physical
 * blocks for them, stored once ("Warmup Guide -- Inference Serving
 * Internals", Chapter 4, prefix sharing by reference counts).  pa_decode
 * reads those blocks once per sequence; this call reads them once per group:
 * the attention of all members' query rows over the shared keys runs as one
 * MFMA pass (in chunks of keys, each giving a partial result: unnormalised
 * output, reference max, sum), every sequence's own keys run as decode
 * partitions, and a merge combines the partials of each (sequence, head).
 * out[b] = softmax(scale * q[b] K_b^T) V_b over all context_lens[b] tokens,
 * exactly as pa_decode defines it; only the order of summation differs.
 *
 *   out, q          device, [num_seqs, num_heads, head_dim]
 *   block_tables,
 *   context_lens    as pa_decode
 *   prefix_lens     device int32 [num_seqs]: tokens of sequence b shared with
 *                   the other members of its group (rounded down to a
 *                   multiple of block_size); 0 for a sequence in no group
 *   max_suffix_len  host bound of context_lens[b] - prefix_lens[b]
 *   max_prefix_len  host bound of prefix_lens[b]
 *   groups          device int32 [num_groups, 2]: first sequence and member
 *                   count; members are consecutive sequences
 *   max_group_size  host bound of the member counts
 *   workspace       device, >= pa_decode_shared_prefix_workspace_bytes(...)
 *
 * Preconditions (device data, not checked): the members of a group have
 * equal prefix_lens and identical block ids for their first prefix_lens /
 * block_size blocks; prefix_lens[b] <= context_lens[b]; a sequence with
 * prefix_lens[b] > 0 belongs to exactly one group; the bounds above hold.
 * Errors and supported shapes: as pa_decode; the workspace is always
 * required.  The caller owns every buffer; nothing is kept past the call.
 */
pa_status pa_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* prefix_lens, int32_t max_suffix_len,
    int32_t max_prefix_len, const int32_t* groups, int32_t num_groups,
    int32_t max_group_size, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, float scale, void* workspace,
    size_t workspace_bytes, pa_dtype dtype, void* stream);

/*
 * 8-bit KV cache.  The pages name a cache-precision option ("10 Serving
 * Engines": the --kv-cache-dtype flag, effective where the engine and its
 * kernels support it) and fix nothing else; the format here is OCP E4M3
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * largest finite 448), one byte per element, with one float scale per cache
 * chosen by the caller: an element x is stored as the code nearest to
 * x / scale (the product x * (1 / scale) in float32, ties to an even
 * mantissa, saturated to +-448); attention reads code * scale.  Layout,
 * slots and block tables are those of the 16/32-bit caches:
 * [num_blocks, block_size, num_kv_heads, head_dim] bytes per cache.
 */

/*
 * pa_store_kv_fp8 -- as pa_store_kv, quantising each row into E4M3 caches.
 *
 *   k, v          device, [num_tokens, num_kv_heads, head_dim] of src_dtype
 *                 (PA_F32 or PA_BF16), 16-byte aligned
 *   k_cache,
 *   v_cache       device uint8, [num_slots, num_kv_heads, head_dim]
 *   k_scale,
 *   v_scale       > 0, finite: the caches' scales
 *
 * Requires num_kv_heads * head_dim to be a multiple of 8.
 */
pa_status pa_store_kv_fp8(const void* k, const void* v, void* k_cache,
                          void* v_cache, const int32_t* slot_mapping,
                          int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int64_t num_slots,
                          pa_dtype src_dtype, float k_scale, float v_scale,
                          void* stream);

/*
 * pa_decode_fp8 -- as pa_decode over E4M3 caches, with q and out bfloat16:
 * out[b,h] = softmax(scale * q . K) V with K = code * k_scale and
 * V = code * v_scale.  head_dim 128 only.  Workspace as
 * pa_decode_workspace_bytes(...) for the same sizes.
 */
pa_status pa_decode_fp8(void* out, const void* q, const void* k_cache,
                        const void* v_cache, int64_t num_blocks,
                        int32_t block_size, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t max_context_len, int32_t num_seqs,
                        int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, float scale, float k_scale,
                        float v_scale, void* workspace, size_t workspace_bytes,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
