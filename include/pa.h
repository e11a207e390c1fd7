/*
 * pa.h -- paged decode attention for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The KV cache is split into fixed-size physical blocks ("pages") that a
 * per-sequence block table maps logical positions onto:
 *   key_cache, value_cache : [num_blocks, block_size, num_kv_heads, head_size]
 *   block_tables           : int32 [num_seqs, max_blocks_per_seq]
 * Position t of sequence s lives in physical block block_tables[s][t / block_size]
 * at offset t % block_size, i.e. at flat slot
 *   block_tables[s][t / block_size] * block_size + t % block_size.
 * Sources: "01. PagedAttention 详解" (vLLM learning book) §3 for the layout
 * and the block-table figure; "PagedAttention 机制" (cs-knowledge-wiki)
 * §5.3.4 for the position -> (block, offset) lookup; the book's §10
 * (how the table reaches the GPU, the 100k-token table) for one packed int32
 * table tensor per step.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller; tensors are
 *    contiguous, row-major. The library allocates nothing, keeps no pointer
 *    after returning, and never synchronises the device. (Its one piece of
 *    device memory is the fixed scratch array of pa_decode_append_static,
 *    part of the loaded code object.)
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it asynchronously.
 *  - The arguments are validated on the host first; a negative status means
 *    nothing was enqueued. PA_ERR_HIP reports a failed launch.
 *  - dtype selects the 2-byte storage type shared by q, k, v, both caches and
 *    out: PA_DTYPE_FP16 (IEEE binary16) or PA_DTYPE_BF16 (bfloat16).
 *  - Arithmetic is fp32 (products, softmax statistics, accumulation); the
 *    output is rounded to the storage type with round-to-nearest-even.
 *  - Concurrent calls on different streams are safe when their outputs and
 *    workspaces do not overlap.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

#if defined(__GNUC__)
#define PA_API __attribute__((visibility("default")))
#else
#define PA_API
#endif

enum pa_dtype { PA_DTYPE_FP16 = 0, PA_DTYPE_BF16 = 1 };

enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                         */
  PA_ERR_SHAPE = -2,       /* sizes inconsistent, negative or out of range       */
  PA_ERR_DTYPE = -3,       /* unknown dtype code                                  */
  PA_ERR_UNSUPPORTED = -4, /* valid, but no kernel built for this head size,
                              block size, group size or partition size            */
  PA_ERR_WORKSPACE = -5,   /* split-K workspace missing or too small              */
  PA_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed          */
  PA_ERR_NO_BLOCKS = -7,   /* block pool: fewer free blocks than requested         */
  PA_ERR_STATE = -8        /* block pool: block not allocated / freed too often    */
};

/* Supported shapes: head_size in {64, 128}; block_size in {16, 32};
   num_q_heads / num_kv_heads in {1, 2, 4, 8}. */

/* Library ABI version (PA_ABI_VERSION of the build). */
PA_API int pa_abi_version(void);

/* Static English text for a status code; never NULL. */
PA_API const char* pa_status_string(int status);

/*
 * pa_decode_slot_mapping -- slot of each sequence's newest token.
 *
 * In a decode step the new token's k/v are appended at the next free slot of
 * the sequence's last block and then attended to ("01. PagedAttention 详解"
 * §4, decode phase). With context length L (counting the new token) that is
 * position L-1:
 *   slot_mapping[s] = block_tables[s][(L-1) / block_size] * block_size
 *                     + (L-1) % block_size,           L = context_lens[s];
 *   slot_mapping[s] = -1 when L <= 0.
 * block_tables  : int32 [num_seqs, max_blocks_per_seq] (device)
 * context_lens  : int32 [num_seqs] (device)
 * slot_mapping  : int32 [num_seqs] (device, written)
 * A length above max_blocks_per_seq * block_size also yields -1 (the table
 * row cannot address it). Exact integer arithmetic.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_seqs < 0, max_blocks_per_seq < 1,
 * block_size < 1).
 * num_seqs == 0 enqueues nothing and returns PA_OK.
 */
PA_API int pa_decode_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t block_size, int32_t* slot_mapping, void* stream);

/*
 * pa_cache_write -- store new tokens' k/v rows into their cache slots.
 *
 * For each token i with 0 <= slot_mapping[i] < num_blocks * block_size:
 *   key_cache  [slot / block_size, slot % block_size, :, :] = k[i, :, :]
 *   value_cache[slot / block_size, slot % block_size, :, :] = v[i, :, :]
 * (the append step of the book's §4 decode phase; the slot formula of its §3
 * block table). A bit-exact copy. Tokens whose slot is negative or out of
 * range are skipped (no write). Slots of one call must be distinct; with
 * duplicates the surviving row is unspecified.
 * k, v          : [num_tokens, num_kv_heads, head_size] (device)
 * key_cache,
 * value_cache   : [num_blocks, block_size, num_kv_heads, head_size] (device, updated)
 * slot_mapping  : int32 [num_tokens] (device)
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (negative sizes, num_blocks * block_size
 * beyond INT32_MAX), PA_ERR_DTYPE, PA_ERR_UNSUPPORTED (head_size not a
 * multiple of 8, or a k / v / cache pointer not 16-byte aligned).
 * num_tokens == 0 enqueues nothing and returns PA_OK.
 */
PA_API int pa_cache_write(const void* k, const void* v, void* key_cache, void* value_cache,
                          const int32_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
                          int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                          int32_t dtype, void* stream);

/*
 * pa_cache_write_fp8 -- store new tokens' k/v into an FP8 (E4M3) cache.
 *
 * The same slot rule as pa_cache_write, for caches that hold one byte per
 * element: OCP 8-bit floating point E4M3 (sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, 0x7F / 0xFF = NaN, largest finite 448).
 * Each cache tensor has one fp32 scale, and a stored code c stands for
 * value(c) * scale. For every element x of k (v) the stored code is
 *   e4m3( fp32(x) / k_scale )     (IEEE fp32 division),
 * rounded to nearest even, with magnitudes above 448 clamped to 448 and
 * NaN stored as 0x7F. (FP8 K/V storage: the intelliparadigm article's §4.3
 * precision table; the format and the per-tensor scale are this library's
 * reading, since the article fixes neither.)
 * k, v          : [num_tokens, num_kv_heads, head_size] of src_dtype (device)
 * key_cache,
 * value_cache   : uint8 [num_blocks, block_size, num_kv_heads, head_size] (device, updated)
 * slot_mapping  : int32 [num_tokens] (device); negative / out-of-range slots skip
 * src_dtype     : PA_DTYPE_FP16 or PA_DTYPE_BF16 (the type of k and v)
 * k_scale,
 * v_scale       : finite and > 0
 * Errors: as pa_cache_write, plus PA_ERR_SHAPE for a scale that is not
 * finite and positive. num_tokens == 0 enqueues nothing and returns PA_OK.
 */
PA_API int pa_cache_write_fp8(const void* k, const void* v, void* key_cache, void* value_cache,
                              const int32_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
                              int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                              int32_t src_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_decode_workspace_size -- bytes of device workspace pa_decode needs.
 *
 * partition_size < 0 (single pass) needs none (returns 0). partition_size > 0
 * needs 256 bytes of scheduler state and room for the fp32 partials of
 * ceil(max_context_len / partition_size) partitions per (sequence, query
 * head). partition_size == 0 (automatic)
 * returns the most any automatic choice can use. Pure host arithmetic.
 * Returns 0 for invalid (negative) sizes.
 */
PA_API size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_size,
                                       int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode_partition_size -- the split pa_decode makes with partition_size 0.
 *
 * Returns the tokens per partition of the automatic choice, or -1 for a
 * single pass, for a batch of num_seqs sequences with num_kv_heads kv heads
 * whose longest context is max_context_len, over caches of cache_elem_bytes
 * bytes per element (2: pa_decode and the cascade; 1: pa_decode_fp8). The
 * rule: the largest power of two in [256, 4096] that still gives about four
 * work-groups per compute unit; when the (sequence, kv head) pairs alone
 * give that many, at most 1024 -- or 2048 for 2-byte elements when the
 * longest context exceeds 3072 tokens, 1536 for 1-byte elements when it
 * exceeds 2304; no split when the longest context is
 * at most 1.5 partitions. num_cus <= 0 asks the current HIP device for its
 * compute-unit count (256 if it cannot be queried). Pure host arithmetic
 * otherwise; no device work is enqueued. Returns 0 for invalid sizes
 * (num_seqs < 0, num_kv_heads < 1, max_context_len < 0, cache_elem_bytes not
 * 1 or 2).
 */
PA_API int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                        int32_t max_context_len, int32_t cache_elem_bytes,
                                        int32_t num_cus);

/*
 * pa_decode -- one decode step of paged attention.
 *
 * For each sequence s with L = context_lens[s] and each query head h:
 *   g      = h / (num_q_heads / num_kv_heads)          (its kv head)
 *   K_t, V_t = key_cache / value_cache rows of kv head g at position t,
 *              reached through block_tables[s] (see the top of this file)
 *   out[s, h, :] = sum_{t<L} softmax_t(scale * q[s,h,:] . K_t) * V_t
 * and out[s, h, :] = 0 when L == 0 (the conceptual kernel of
 * "PagedAttention 机制" §5.3.4 starts from zeros and scales q.k by
 * 1/sqrt(head_dim); the softmax normalisation is the standard attention of
 * the book's §4). Only table entries 0 .. ceil(L / block_size) - 1 are read;
 * cache slots at positions >= L are never used, whatever they hold.
 *
 * Long contexts are split into partitions (the book's §4 and §9 name a v2
 * kernel that splits long sequences this way): each partition keeps its
 * running max, exp-sum and weighted sum of V in fp32 in the workspace, and a
 * second kernel rescales and combines them for the sequences that span more
 * than one partition (a sequence with one partition is finished directly).
 *   partition_size < 0 : single pass, one work-group per (sequence, kv head);
 *   partition_size > 0 : split into partitions of that many tokens
 *                        (a multiple of 16 and of block_size);
 *   partition_size == 0: chosen from max_context_len, num_seqs * num_kv_heads
 *                        and the device's compute-unit count
 *                        (pa_decode_partition_size).
 * q    : [num_seqs, num_q_heads, head_size] (device)
 * out  : [num_seqs, num_q_heads, head_size] (device, written), dtype of q
 * context_lens : int32 [num_seqs] (device); each must be <= max_context_len
 *                and <= max_blocks_per_seq * block_size (larger values are
 *                clamped to those bounds).
 * max_context_len : host-known upper bound of the lengths (the scheduler owns
 *                the lengths on the host); sizes the split.
 * Table entries that are read must lie in [0, num_blocks); a block id outside
 * that range is skipped (its tokens contribute nothing) rather than read.
 * workspace : device buffer, 256-byte aligned, of at least
 *             pa_decode_workspace_size(...) bytes for the same sizes and
 *             partition_size (may be NULL when that size is 0). Its contents
 *             need no initialisation. Its first 256 bytes carry scheduler
 *             state from one split call to the next on the same buffer: a
 *             64-bit word at offset 0 (a tag derived from the buffer's
 *             address in bytes 0-3, a work counter in bytes 4-7) and a
 *             32-bit finish count at offset 128. Every call that uses them
 *             leaves (tag, 0) and 0 behind, also when only its partition
 *             kernel ran, so a later call never starts from a used counter.
 *             A call that finds no tag (a fresh buffer, or one overwritten
 *             since) gives the same result with a fixed schedule. Between
 *             calls the caller may reuse the buffer for anything, as long as
 *             a write into bytes 4-7 or 128-131 also changes bytes 0-3
 *             (any write of the whole head does): a counter or count changed
 *             under an intact tag would make the next call skip work items.
 *             The rest is scratch for this call only. Calls that run at the
 *             same time need distinct workspaces.
 * Errors: PA_ERR_DTYPE; PA_ERR_SHAPE (non-positive head counts or sizes,
 * num_q_heads not a multiple of num_kv_heads, max_context_len above
 * max_blocks_per_seq * block_size, non-finite scale); PA_ERR_UNSUPPORTED
 * (head_size, block_size, group size or partition_size outside the built
 * set; q / cache / out pointers not 16-byte aligned); PA_ERR_NULL;
 * PA_ERR_WORKSPACE; PA_ERR_HIP. num_seqs == 0 returns PA_OK.
 */
PA_API int pa_decode(const void* q, const void* key_cache, const void* value_cache,
                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                     void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_size, int32_t block_size, int64_t num_blocks,
                     int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size,
                     int32_t dtype, void* workspace, size_t workspace_size, void* stream);

/*
 * pa_decode_fp8 -- one decode step over FP8 (E4M3) caches.
 *
 * Computes what pa_decode computes, with the K rows read as
 * value(code) * k_scale and the V rows as value(code) * v_scale (the
 * encoding of pa_cache_write_fp8). q and out keep dtype (PA_DTYPE_FP16 or
 * PA_DTYPE_BF16); key_cache / value_cache are uint8
 * [num_blocks, block_size, num_kv_heads, head_size]. The scales are applied
 * in fp32: k_scale multiplies the logit scale, v_scale the normalised
 * output. The partitioning, workspace (pa_decode_workspace_size with the
 * same sizes), stream and error rules are those of pa_decode, plus
 * PA_ERR_SHAPE for a k_scale or v_scale that is not finite and positive.
 */
PA_API int pa_decode_fp8(const void* q, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         float k_scale, float v_scale, void* out, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                         int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_context_len, int32_t partition_size, int32_t dtype,
                         void* workspace, size_t workspace_size, void* stream);

/*
 * pa_decode_cascade_workspace_size -- workspace bytes of pa_decode_cascade.
 *
 * 256 bytes of scheduler state, and room for the fp32 partials of
 * ceil(prefix_len / 256) prefix chunks plus the partitions of the positions
 * past the prefix (as pa_decode_workspace_size counts them for
 * max_context_len - prefix_len tokens), per (sequence, query head), with
 * prefix_len = shared_prefix_blocks * block_size. With
 * shared_prefix_blocks == 0 it equals pa_decode_workspace_size. Pure host
 * arithmetic; 0 for invalid sizes.
 */
PA_API size_t pa_decode_cascade_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t head_size, int32_t block_size,
                                               int32_t max_context_len,
                                               int32_t shared_prefix_blocks,
                                               int32_t partition_size);

/*
 * pa_decode_cascade -- pa_decode for a batch whose tables share a prefix.
 *
 * Precondition: block_tables[s][0 .. shared_prefix_blocks-1] are the same
 * physical blocks for every sequence s (a prompt prefix stored once and
 * referenced by every request, "01. PagedAttention 详解" §6). The result is
 * then what pa_decode returns (same arguments, same error rules), computed
 * as:
 *   - the shared prefix, positions [0, prefix_len), prefix_len =
 *     shared_prefix_blocks * block_size: every (sequence, query head) row of
 *     a kv head against one read of the prefix's K/V, as dense matrix
 *     products on the matrix cores (keys at or past a sequence's own length
 *     are masked, so a sequence shorter than the prefix is still exact);
 *   - each sequence's positions [prefix_len, L) as the ordinary decode items
 *     (partition_size as in pa_decode, applied to that range), one
 *     work-group per item, in the same launch as the prefix part;
 *   - the combine of both kinds of partials, as in the split path.
 * The softmax weights enter the matrix products rounded to the query's 2-byte
 * type; accumulation stays fp32. The prefix is read through row 0 of
 * block_tables. If the precondition does not hold the output rows of the
 * sequences whose prefix differs are undefined (no fault: every block id read
 * is range-checked).
 * shared_prefix_blocks : 0 .. max_blocks_per_seq (0 = a plain pa_decode call)
 * workspace            : at least pa_decode_cascade_workspace_size(...) bytes,
 *                        256-byte aligned; contents need no initialisation, and
 *                        its first 256 bytes (pa_decode's scheduler words) are
 *                        left as they are
 * Errors: those of pa_decode, and PA_ERR_SHAPE for shared_prefix_blocks out
 * of range or (with shared_prefix_blocks > 0 and num_seqs > 0) num_blocks
 * == 0 or num_blocks * block_size above INT32_MAX (slots are int32). Caches
 * of the query's 2-byte type only.
 */
PA_API int pa_decode_cascade(const void* q, const void* key_cache, const void* value_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                             int64_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t max_context_len, int32_t shared_prefix_blocks,
                             int32_t partition_size, int32_t dtype, void* workspace,
                             size_t workspace_size, void* stream);

/*
 * pa_decode_append -- one whole decode step in one call: the slot of each
 * sequence's new token, its k/v stored into the caches, then attention.
 *
 * The decode phase of "01. PagedAttention 详解" §4 computes the new token's
 * q, k, v, appends k/v at the next slot of the sequence's last block, and
 * attends over every cached position including the new one. With
 * L = context_lens[s] counting the new token (it sits at position L - 1),
 * this call has exactly the effect of
 *   pa_decode_slot_mapping(block_tables, ..., slot_mapping);
 *   pa_cache_write(k, v, key_cache, value_cache, slot_mapping, num_seqs, ...);
 *   pa_decode_cascade(q, key_cache, value_cache, ..., shared_prefix_blocks, ...);
 * (pa_decode when shared_prefix_blocks == 0), with no separate slot or write
 * launch: the same slots and cache contents bit for bit, and the same output
 * up to rounding order (the new token's term is summed last, so the last
 * bits may differ; both are held to the decode tolerance). The work-group
 * that attends over position L - 1 of kv head g stores that head's k/v row
 * at the slot and attends over the same row values, taken from k / v.
 * k, v         : [num_seqs, num_kv_heads, head_size] (device), dtype of q,
 *                16-byte aligned
 * slot_mapping : int32 [num_seqs] (device, written) -- the slot of position
 *                L - 1, or -1 when L == 0 (then nothing is stored); NULL to
 *                not keep the slots
 * Preconditions: the new tokens' slots are distinct, and no block holding a
 * new token is shared with another table; with a shared prefix, every new
 * token lies past it (L - 1 >= shared_prefix_blocks * block_size): a write
 * into a shared block needs a copy-on-write first (the book's §6). A table
 * entry outside [0, num_blocks) stores nothing.
 * Workspace (pa_decode_cascade_workspace_size), partitioning, stream and
 * errors: those of pa_decode_cascade, plus PA_ERR_NULL for a NULL k or v,
 * PA_ERR_UNSUPPORTED for k / v not 16-byte aligned and PA_ERR_SHAPE for
 * num_blocks * block_size above INT32_MAX (slots are int32).
 */
PA_API int pa_decode_append(const void* q, const void* k, const void* v, void* key_cache,
                            void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, float scale, void* out,
                            int32_t* slot_mapping, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                            int64_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, int32_t shared_prefix_blocks,
                            int32_t partition_size, int32_t dtype, void* workspace,
                            size_t workspace_size, void* stream);

/*
 * pa_decode_append_fp8 -- pa_decode_append over FP8 (E4M3) caches: the new
 * rows are stored as pa_cache_write_fp8 stores them (k / v in dtype,
 * quantized with k_scale / v_scale) and the step attends as pa_decode_fp8
 * does, over the stored codes. No shared-prefix form. Workspace
 * (pa_decode_workspace_size), errors and preconditions: those of
 * pa_decode_fp8 and pa_decode_append.
 */
PA_API int pa_decode_append_fp8(const void* q, const void* k, const void* v, void* key_cache,
                                void* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, float scale, float k_scale,
                                float v_scale, void* out, int32_t* slot_mapping,
                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_size, int32_t block_size, int64_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len,
                                int32_t partition_size, int32_t dtype, void* workspace,
                                size_t workspace_size, void* stream);

/*
 * pa_decode_append_static -- pa_decode_append with no workspace argument:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results, preconditions and errors as pa_decode_append,
 * without workspace / workspace_size: the split-K partials and the
 * scheduler words live in a fixed array of PA_STATIC_SCRATCH_BYTES bytes
 * inside the library, one per GPU, held from the library's first use on
 * that GPU until the process ends. The call allocates nothing (no hipMalloc,
 * no allocating library routine); its first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress) with the device current.
 * Nothing in the array needs to start at zero: the partials of a call are
 * written before they are read, and the scheduler words are read the way
 * pa_decode reads a fresh workspace's.
 * A call whose partials need more than PA_STATIC_SCRATCH_BYTES (as
 * pa_decode_cascade_workspace_size counts them for the partition size the
 * call uses) returns PA_ERR_WORKSPACE with nothing enqueued. Every call on
 * one GPU shares that GPU's array: calls that can run at the same time on
 * one GPU (other streams, other threads) race and give undefined results;
 * serialize them, or use pa_decode_append with distinct workspaces.
 */
#define PA_STATIC_SCRATCH_BYTES (32u << 20)
PA_API int pa_decode_append_static(const void* q, const void* k, const void* v, void* key_cache,
                                   void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, float scale, void* out,
                                   int32_t* slot_mapping, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                   int64_t num_blocks, int32_t max_blocks_per_seq,
                                   int32_t max_context_len, int32_t shared_prefix_blocks,
                                   int32_t partition_size, int32_t dtype, void* stream);

/*
 * Prefill batches ("01. PagedAttention 详解" §4, prefill phase: a prompt's N
 * tokens get their K/V written into the blocks the table points to, then
 * attention runs over them). Sequence s holds L = context_lens[s] positions
 * once its new tokens are written; its n = query_start[s+1] - query_start[s]
 * new tokens are rows query_start[s] .. query_start[s+1]-1 of q / out /
 * slot_mapping, at positions L - n .. L - 1 (a whole prompt when n == L, a
 * later chunk of one when n < L).
 * query_start : int32 [num_seqs + 1] (device), non-decreasing, from 0 to
 *               num_tokens; rows outside [0, num_tokens) are never touched and
 *               n is capped at min(L, max_query_len).
 * max_query_len : host-known upper bound of n (sizes the grid).
 */

/*
 * pa_prefill_slot_mapping -- slot of every new token:
 *   slot_mapping[query_start[s] + i] = block_tables[s][p / block_size] * block_size
 *                                      + p % block_size,   p = L - n + i.
 * The result feeds pa_cache_write with num_tokens tokens. Exact integer
 * arithmetic. Errors: PA_ERR_SHAPE (negative sizes, max_context_len beyond
 * the table), PA_ERR_UNSUPPORTED (num_seqs > 65535), PA_ERR_NULL.
 * num_seqs == 0 or num_tokens == 0 enqueues nothing and returns PA_OK.
 */
PA_API int pa_prefill_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, const int32_t* query_start,
                                   int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                                   int32_t block_size, int32_t max_context_len,
                                   int32_t* slot_mapping, void* stream);

/*
 * pa_prefill -- causal paged attention of the new tokens.
 *
 * For each new token (row t of sequence s at position p) and query head h:
 *   out[t, h, :] = sum_{u <= p} softmax_u(scale * q[t,h,:] . K_u) * V_u
 * with K_u / V_u the rows of kv head h / (num_q_heads / num_kv_heads) at
 * position u of sequence s, reached through block_tables[s]. The new tokens'
 * K/V must already be in the cache (pa_prefill_slot_mapping +
 * pa_cache_write). The products run on the matrix cores in fp32
 * accumulation; the softmax weights enter the P.V product rounded to the
 * query's 2-byte type.
 * q, out : [num_tokens, num_q_heads, head_size] of dtype (device)
 * caches : [num_blocks, block_size, num_kv_heads, head_size] of dtype
 * Only table entries of positions < L are read; block ids outside
 * [0, num_blocks) read as zeros. No workspace is needed.
 * Errors: as pa_decode (dtype, shapes, head size 64 / 128, block size
 * 16 / 32, group 1 / 2 / 4 / 8, alignment, NULL, HIP), and PA_ERR_SHAPE for
 * num_blocks == 0 when there are new tokens (they live in the pool) and for
 * num_blocks * block_size above INT32_MAX (slots are int32).
 * num_seqs, num_tokens or max_query_len == 0 returns PA_OK.
 */
PA_API int pa_prefill(const void* q, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* query_start, float scale, void* out, int32_t num_seqs,
                      int32_t num_tokens, int32_t max_query_len, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                      int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                      int32_t dtype, void* stream);

/*
 * pa_prefill_fp8 -- pa_prefill over FP8 (E4M3) caches (the intelliparadigm
 * article's §4.3: FP8 K/V among the cache precisions).
 * A code c stands for value(c) * k_scale in key_cache and value(c) * v_scale
 * in value_cache, the reading pa_decode_fp8 takes; the new tokens are
 * written with pa_cache_write_fp8. q and out keep the 2-byte type dtype.
 * Codes are converted exactly to dtype before the products; k_scale joins
 * the softmax scale and v_scale the output.
 * caches : uint8 [num_blocks, block_size, num_kv_heads, head_size] (device)
 * Errors: as pa_prefill, and PA_ERR_SHAPE for a k_scale or v_scale that is
 * not finite and positive.
 */
PA_API int pa_prefill_fp8(const void* q, const void* key_cache, const void* value_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start, float scale, float k_scale, float v_scale,
                          void* out, int32_t num_seqs, int32_t num_tokens,
                          int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_size, int32_t block_size, int64_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_context_len, int32_t dtype,
                          void* stream);

/*
 * Host block pool -- the bookkeeping that produces the tables (host memory
 * only; no device work). A block's reference count says how many tables
 * point at it ("PagedAttention 机制" §5.3.4 BlockAllocator). The free list is
 * a queue: allocation takes blocks from its head, and a block whose count
 * drops to 0 joins its tail, so the least recently freed block is reused
 * first ("01. PagedAttention 详解" 自检 Q3). A new pool has every block free,
 * in id order. A pool is not thread-safe: one caller at a time.
 */
typedef struct pa_pool pa_pool;

/* A pool of num_blocks blocks, all free; NULL if num_blocks < 1 or out of
   host memory. */
PA_API pa_pool* pa_pool_create(int32_t num_blocks);
PA_API void pa_pool_destroy(pa_pool* pool);
/* Free blocks (-1 for a NULL pool). */
PA_API int32_t pa_pool_num_free(const pa_pool* pool);
/* Reference count of a block (0 = free; -1 for a NULL pool or id out of range). */
PA_API int32_t pa_pool_ref_count(const pa_pool* pool, int32_t block);
/* n blocks from the head of the free queue, count 1 each, into blocks[0..n).
   PA_ERR_NO_BLOCKS (nothing taken) when fewer than n are free. */
PA_API int pa_pool_allocate(pa_pool* pool, int32_t n, int32_t* blocks);
/* One reference fewer for each listed block (a block may be listed as often
   as it is referenced); a block reaching 0 joins the queue's tail.
   PA_ERR_STATE (nothing changed) for a free block or an id out of range. */
PA_API int pa_pool_free(pa_pool* pool, const int32_t* blocks, int32_t n);
/* One reference more for each listed block (another table points at it).
   PA_ERR_STATE (nothing changed) for a free block or an id out of range. */
PA_API int pa_pool_share(pa_pool* pool, const int32_t* blocks, int32_t n);
/* Copy-on-write before a write into *block ("01. PagedAttention 详解" §6):
   returns 0 if *block has one reference (write in place); returns 1 after
   taking a fresh block from the queue's head, dropping one reference of the
   shared block, setting *src = old block, *dst = fresh block and
   *block = fresh block -- the caller then copies src to dst (pa_copy_blocks)
   and stores *block in its table. PA_ERR_STATE for a free block,
   PA_ERR_NO_BLOCKS when a copy is needed and no block is free. */
PA_API int pa_pool_copy_on_write(pa_pool* pool, int32_t* block, int32_t* src, int32_t* dst);

/*
 * pa_copy_blocks -- whole-block copies in both caches (device work).
 * For each i < num_pairs: block block_pairs[2i+1] := block block_pairs[2i]
 * of key_cache and of value_cache, every position and head (the copy of
 * pa_pool_copy_on_write). block_pairs: int32 [num_pairs, 2] (device).
 * elem_bytes: 2 for fp16 / bf16 caches, 1 for FP8 caches. Destinations must
 * be distinct and no destination may be a source of the same call. Pairs
 * with an id outside [0, num_blocks) are skipped. Bit-exact copy.
 * Errors: PA_ERR_SHAPE, PA_ERR_DTYPE (elem_bytes), PA_ERR_UNSUPPORTED (block
 * bytes not a multiple of 16, caches not 16-byte aligned), PA_ERR_NULL,
 * PA_ERR_HIP. num_pairs == 0 returns PA_OK.
 */
PA_API int pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* block_pairs,
                          int32_t num_pairs, int64_t num_blocks, int32_t block_size,
                          int32_t num_kv_heads, int32_t head_size, int32_t elem_bytes,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
