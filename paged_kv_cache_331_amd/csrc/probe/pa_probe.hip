// Read-bandwidth probes for the benchmark (libpa_probe_gfx950.so, separate
// from the attention library and never called by it).
//
// They measure two practical ceilings that the decode kernel's HBM rate is
// compared with:
//  * pa_probe_stream_read: a contiguous buffer read once with 16-byte
//    non-temporal loads, eight in flight per lane -- what HBM delivers to a
//    plain streaming reader;
//  * pa_probe_gather_read: the K and V rows of a decode batch read through
//    the block tables with the decode kernel's load shape (one work-group of
//    four waves per (kv head, sequence, partition) in partition-major order,
//    16-token tiles, token rows of head_size / 8 lanes holding 16 bytes each,
//    non-temporal loads) and nothing computed from them but an XOR -- what the
//    same gather of scattered blocks delivers before any arithmetic.
// Each wave folds what it read into one word written to `sink`, so no load
// can be dropped. Tokens past a sequence's length inside its last tile are
// read, as the decode kernel reads them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ uint32_t fold(u32x4_t v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// Wave-level XOR of one word per lane; lane 0 stores it.
__device__ __forceinline__ void sink_wave(uint32_t acc, uint32_t* sink, uint64_t slot) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) sink[slot] = acc;
}

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* buf, uint64_t n16,
                                                                uint32_t* sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4_t v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = ld16(buf + i + k * stride);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= fold(v[k]);
  }
  for (; i < n16; i += stride) acc ^= fold(ld16(buf + i));
  sink_wave(acc, sink, (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
}

struct GatherArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* bt;
  const int32_t* lens;
  uint32_t* sink;
  int32_t num_seqs, num_kv_heads, row_bytes, block_size, max_blocks_per_seq, part_tokens,
      num_parts, len_cap, persist;
  int64_t num_blocks;
};

// Work items (kv head, sequence, partition), kv head fastest, the partition
// index slowest. With a.persist == 0 one work-group per item; otherwise
// gridDim.x work-groups walk the items with stride gridDim.x (the decode
// kernel's persistent grid, without its ticket counter). Lanes: row_bytes /
// 16 per token row, so a load instruction covers 64 * 16 / row_bytes
// consecutive slots of the block.
__global__ __launch_bounds__(kThreads) void gather_read_kernel(const GatherArgs a) {
  const int total = a.num_kv_heads * a.num_seqs * a.num_parts;
  const int lpr = a.row_bytes / 16;                    // lanes per token row
  const int rows = 64 / lpr;                           // slots per load instruction
  constexpr int kTile = 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t tok_stride = (int64_t)a.num_kv_heads * a.row_bytes;
  uint32_t acc = 0;
  for (int item = blockIdx.x; item < total; item += a.persist ? (int)gridDim.x : total) {
    int wg = item;
    const int g = wg % a.num_kv_heads;
    wg /= a.num_kv_heads;
    const int s = wg % a.num_seqs;
    const int p = wg / a.num_seqs;
    const int L = min(max(a.lens[s], 0), a.len_cap);   // the table row's reach at most
    const int start = p * a.part_tokens;
    if (start >= L) continue;
    const int end = min(L, start + a.part_tokens);
    const int64_t lane_off =
        (lane / lpr) * tok_stride + (int64_t)g * a.row_bytes + (lane % lpr) * 16;
    const int32_t* row = a.bt + (int64_t)s * a.max_blocks_per_seq;
    const int ntiles = (end - start + kTile - 1) / kTile;
    for (int it = wave; it < ntiles; it += 4) {
      const int ts = start + it * kTile;
      const int blk = __builtin_amdgcn_readfirstlane(row[ts / a.block_size]);
      if ((uint64_t)(uint32_t)blk >= (uint64_t)a.num_blocks) continue;
      const int64_t base =
          ((int64_t)blk * a.block_size + ts % a.block_size) * tok_stride + lane_off;
      const int nld = kTile / rows;                    // 4 at 256-byte rows
      u32x4_t v[8];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < nld) v[k] = ld16(a.kc + base + k * rows * tok_stride);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < nld) v[4 + k] = ld16(a.vc + base + k * rows * tok_stride);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < nld) acc ^= fold(v[k]) ^ fold(v[4 + k]);
    }
  }
  sink_wave(acc, a.sink, (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
}

}  // namespace

extern "C" {

// Words `sink` must hold for a stream probe with `grid` work-groups.
__attribute__((visibility("default"))) size_t pa_probe_sink_words(int32_t grid) {
  return grid > 0 ? (size_t)grid * (kThreads / 64) : 0;
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) of `buf` once with
// `grid` work-groups of 256 threads. Returns 0, or -1 for bad arguments, -6
// for a failed launch.
__attribute__((visibility("default"))) int pa_probe_stream_read(const void* buf, uint64_t bytes,
                                                                uint32_t* sink, int32_t grid,
                                                                void* stream) {
  if (!buf || !sink || grid <= 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((uint32_t)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, reinterpret_cast<const u32x4_t*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Reads the K and V rows of positions < L of every (sequence, kv head)
// through the block tables, as described at the top of this file.
// row_bytes = head_size * element bytes (128 or 256 here); part_tokens a
// multiple of 16 and of block_size (block_size a multiple of 16).
// grid == 0 launches one work-group per item (num_kv_heads * num_seqs *
// ceil(max_context_len / part_tokens) of them); grid > 0 launches that many
// (at most the item count) walking the items with a fixed stride. `sink`
// holds 4 words per work-group launched.
__attribute__((visibility("default"))) int pa_probe_gather_read(
    const void* key_cache, const void* value_cache, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads, int32_t row_bytes,
    int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t part_tokens, int32_t grid, uint32_t* sink, void* stream) {
  if (!key_cache || !value_cache || !block_tables || !context_lens || !sink) return -1;
  if (num_seqs < 1 || num_kv_heads < 1 || (row_bytes != 128 && row_bytes != 256)) return -1;
  if (block_size < 16 || block_size % 16 != 0 || part_tokens < 16 || part_tokens % 16 != 0 ||
      part_tokens % block_size != 0 || max_context_len < 1 ||
      max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return -1;
  GatherArgs a;
  a.kc = static_cast<const uint8_t*>(key_cache);
  a.vc = static_cast<const uint8_t*>(value_cache);
  a.bt = block_tables;
  a.lens = context_lens;
  a.sink = sink;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.row_bytes = row_bytes;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.part_tokens = part_tokens;
  a.num_parts = (max_context_len + part_tokens - 1) / part_tokens;
  a.len_cap = max_context_len;
  a.num_blocks = num_blocks;
  const uint64_t items = (uint64_t)num_kv_heads * num_seqs * a.num_parts;
  if (items > 0x7fffffffull || grid < 0) return -1;
  a.persist = grid > 0 ? 1 : 0;
  const uint64_t nwg = grid > 0 && (uint64_t)grid < items ? (uint64_t)grid : items;
  hipLaunchKernelGGL(gather_read_kernel, dim3((uint32_t)nwg), dim3(kThreads), 0,
                     (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
