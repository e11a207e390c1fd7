// Internal launch interface between the C-ABI layer (pa_api.hip) and the
// kernel translation units. Host-side only; nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Everything one decode launch needs. Pointers are device pointers.
struct DecodeParams {
  const uint16_t* q;        // [B, Hq, D]
  const void* kc;           // [NB, bs, Hkv, D], 2-byte elements or FP8 E4M3 codes
  const void* vc;           // [NB, bs, Hkv, D]
  const int32_t* bt;        // [B, MB]
  const int32_t* lens;      // [B]
  uint16_t* out;            // [B, Hq, D]
  float* ws_m;              // split-K partials: running max (log2 units) [B, Hq, P]
  float* ws_l;              //                   exp-sum                  [B, Hq, P]
  float* ws_o;              //                   weighted V sum           [B, Hq, P, D]
  float scale_log2;         // scale * k_scale * log2(e): logits are kept in base-2 units
  float v_scale;            // multiplies the weighted V sum (FP8 cache scale, else 1)
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t log2_block_size;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int32_t part_tokens;      // tokens per partition (multiple of 16 and of block_size);
                            // max_context_len (any value) when there is no split
  int32_t num_parts;        // partitions per sequence in the grid (1: no split, no workspace)
  int32_t seq_major;        // grid order: 1 = sequence index slowest, 0 = partition slowest
  int32_t tok_offset;       // first position the partitions cover (a multiple of block_size;
                            // the shared-prefix length in a cascade, else 0)
  int32_t slot_base;        // partial slots before the partitions' own (prefix chunks)
  int32_t part_stride;      // partial slots per (sequence, query head) in the workspace
  int32_t always_combine;   // 1: every sequence goes through the combine kernel
  // Cascade only: attention of every (sequence, query head) over the shared
  // prefix, positions [0, prefix_len) through block_tables row 0.
  int32_t prefix_len;       // tokens (a multiple of block_size)
  int32_t prefix_chunks;    // prefix key chunks = partial slots 0 .. prefix_chunks-1
  int32_t prefix_row_tiles; // 64-row tiles of the num_seqs * group query rows
  int32_t len_cap;          // lengths are clamped to this (max_context_len, table reach)
  // Persistent scheduling (split calls whose combine kernel runs): the
  // partition kernel is launched with persist_grid work-groups that take the
  // (kv head, sequence, partition) items from the scheduler word *sched: low
  // 32 bits a tag, high 32 bits a work counter. A partition kernel that
  // finds another tag (a fresh or overwritten workspace) walks the items
  // with a fixed stride and leaves the words alone; one that finds the tag
  // draws tickets from the counter, and its last work-group to finish
  // (counted in *sched_done) puts the word back to (tag, 0) and the count
  // to 0. The combine kernel writes (tag, 0) and 0 after every call. The tag
  // sits at the lowest address, so a write that reaches the counter from
  // below clobbers the tag first.
  unsigned long long* sched;  // nullptr: one work-group per item
  uint32_t* sched_done;       // work-groups of a counted walk that have finished
  uint32_t sched_tag;
  int32_t persist_grid;       // 0: one work-group per item
  // Write-then-attend in the same launch: each sequence's new token (position
  // L-1) is stored into the caches at its slot and used as that position's
  // K/V row. The work item whose partition holds position L-1 stores the
  // row of its kv head; the one of kv head 0 also records the slot.
  const uint16_t* k_new = nullptr;  // [B, Hkv, D] in q's type; nullptr: nothing appended
  const uint16_t* v_new = nullptr;  // [B, Hkv, D]
  int32_t* slots_out = nullptr;     // [B]: slot of position L-1, -1 if L = 0 (nullptr: not kept)
  float k_scale_w = 1.f;            // FP8 cache: the write stores e4m3(fp32(x) / scale)
  float v_scale_w = 1.f;
};

// Bytes reserved for the scheduler words at the head of a split-K workspace,
// before the partials: the (tag, counter) word at offset 0 and the finish
// count at kSchedDoneOffset, in another 128-byte line.
constexpr int kSchedBytes = 256;
constexpr int kSchedDoneOffset = 128;

// Work-groups of the partition kernel per launch: one per
// (kv head, partition, sequence), or a persistent grid of a few per compute
// unit that takes the items from a counter. Launch shapes are fixed per
// instantiation.
constexpr int kDecodeWaves = 4;
constexpr int kReduceThreads = 256;

// Everything one prefill launch needs. Pointers are device pointers.
struct PrefillParams {
  const uint16_t* q;          // [num_tokens, Hq, D]
  const void* kc;             // [NB, bs, Hkv, D]
  const void* vc;
  const int32_t* bt;          // [B, MB]
  const int32_t* lens;        // [B], positions after the new tokens are written
  const int32_t* query_start; // [B + 1], rows of each sequence's new tokens
  uint16_t* out;              // [num_tokens, Hq, D]
  int32_t* slots;             // [num_tokens] (slot kernel only)
  float scale_log2;
  int32_t num_seqs, num_tokens, max_query_len;
  int32_t num_q_heads, num_kv_heads, block_size, log2_block_size;
  int32_t max_blocks_per_seq, len_cap, num_tiles;
  int64_t num_blocks;
  float v_scale;              // FP8 cache: V's scale (K's is in scale_log2)
};

// fp8: the caches hold E4M3 codes.
hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_size, int group, bool fp8,
                          hipStream_t stream);
hipError_t launch_prefill_slots(const PrefillParams& p, hipStream_t stream);

// Keys of the shared prefix one cascade work-group covers, and the shape of
// that work-group: waves, and 16-row blocks per wave.
#ifndef PA_PREFIX_CHUNK
#define PA_PREFIX_CHUNK 256
#endif
#ifndef PA_CASCADE_WAVES
#define PA_CASCADE_WAVES 4
#endif
#ifndef PA_CASCADE_ROW_BLOCKS
#define PA_CASCADE_ROW_BLOCKS 1
#endif
constexpr int kPrefixChunk = PA_PREFIX_CHUNK;
constexpr int kCascadeRowBlocks = PA_CASCADE_ROW_BLOCKS;
// At head size 64 a 32-key K tile is 4 KB, four 1 KB wave loads: 4 waves at most.
constexpr int cascade_waves(int head_size) { return head_size == 128 ? PA_CASCADE_WAVES : 4; }
constexpr int cascade_rows_per_wg(int head_size) {
  return cascade_waves(head_size) * 16 * kCascadeRowBlocks;
}

// Steps of K/V loads in flight in the prefix work-groups of the cascade
// launch (their LDS ring sets the launch's LDS footprint).
#ifndef PA_FUSED_PREFIX_RING
#define PA_FUSED_PREFIX_RING 1
#endif
constexpr int kFusedPrefixRing = PA_FUSED_PREFIX_RING;

// One decode step: the partition kernel, then (num_parts > 1) the combine.
// dtype: q / out type (0 fp16, 1 bf16); fp8_cache: the caches hold E4M3 codes.
hipError_t launch_decode(const DecodeParams& a, int dtype, bool fp8_cache, int head_size,
                         int group, hipStream_t stream);

// Cascade decode: one launch holding the suffix items (the positions past
// the prefix) and the prefix work-groups (MFMA), every one writing partials,
// then the combine of both kinds. a.always_combine must be 1.
hipError_t launch_cascade(const DecodeParams& a, int dtype, int head_size, int group,
                          hipStream_t stream);

hipError_t launch_slot_mapping(const int32_t* bt, int32_t max_blocks_per_seq,
                               const int32_t* lens, int32_t num_seqs, int32_t block_size,
                               int32_t* slots, hipStream_t stream);

hipError_t launch_cache_write(const uint16_t* k, const uint16_t* v, uint16_t* kc, uint16_t* vc,
                              const int32_t* slots, int32_t num_tokens, int64_t num_slots,
                              int32_t row_elems, hipStream_t stream);

// Block copies for copy-on-write: for each pair, block pairs[2i+1] := block
// pairs[2i] of both caches; block_bytes = block_size * Hkv * D * element bytes.
hipError_t launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int32_t num_pairs,
                              int64_t num_blocks, int64_t block_bytes, hipStream_t stream);

// Quantizing write into an FP8 E4M3 cache: code = e4m3(fp32(x) / scale).
hipError_t launch_cache_write_fp8(const uint16_t* k, const uint16_t* v, uint8_t* kc, uint8_t* vc,
                                  const int32_t* slots, int32_t num_tokens, int64_t num_slots,
                                  int32_t row_elems, int src_dtype, float k_scale, float v_scale,
                                  hipStream_t stream);

}  // namespace pa
