// Slot mapping and cache write for gfx950.
//
// Decode appends the new token's k/v at the next free slot of the sequence's
// last block before attending ("01. PagedAttention 详解" §4, decode phase);
// the slot of logical position t is table[t / block_size] * block_size +
// t % block_size (same page, §3 block-table figure; "PagedAttention 机制"
// §5.3.4 lookup).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kSlotThreads = 256;
constexpr int kWriteThreads = 256;

// One thread per sequence: slot of position L-1, or -1 if there is none.
__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(
    const int32_t* __restrict__ bt, int32_t max_blocks_per_seq, const int32_t* __restrict__ lens,
    int32_t num_seqs, int32_t block_size, int32_t* __restrict__ slots) {
  const int s = blockIdx.x * kSlotThreads + threadIdx.x;
  if (s >= num_seqs) return;
  const int L = lens[s];
  int32_t slot = -1;
  if (L > 0 && (int64_t)(L - 1) / block_size < max_blocks_per_seq) {
    const int pos = L - 1;
    slot = bt[(int64_t)s * max_blocks_per_seq + pos / block_size] * block_size + pos % block_size;
  }
  slots[s] = slot;
}

// One thread per 16-byte chunk of a token's [Hkv, D] row, for k and v alike.
// row_elems = Hkv * D (a multiple of 8), so each chunk is one aligned uint4.
__global__ __launch_bounds__(kWriteThreads) void cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ kc,
    uint16_t* __restrict__ vc, const int32_t* __restrict__ slots, int32_t num_tokens,
    int64_t num_slots, int32_t row_elems) {
  const int chunks = row_elems / 8;
  const int64_t gid = (int64_t)blockIdx.x * kWriteThreads + threadIdx.x;
  const int64_t tok = gid / chunks;
  if (tok >= num_tokens) return;
  const int c = (int)(gid - tok * chunks);
  const int32_t slot = slots[tok];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int64_t src = tok * row_elems + (int64_t)c * 8;
  const int64_t dst = (int64_t)slot * row_elems + (int64_t)c * 8;
  *reinterpret_cast<uint4*>(kc + dst) = *reinterpret_cast<const uint4*>(k + src);
  *reinterpret_cast<uint4*>(vc + dst) = *reinterpret_cast<const uint4*>(v + src);
}

}  // namespace

hipError_t launch_slot_mapping(const int32_t* bt, int32_t max_blocks_per_seq, const int32_t* lens,
                               int32_t num_seqs, int32_t block_size, int32_t* slots,
                               hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  const uint32_t grid = (uint32_t)((num_seqs + kSlotThreads - 1) / kSlotThreads);
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(grid), dim3(kSlotThreads), 0, stream, bt,
                     max_blocks_per_seq, lens, num_seqs, block_size, slots);
  return hipGetLastError();
}

hipError_t launch_cache_write(const uint16_t* k, const uint16_t* v, uint16_t* kc, uint16_t* vc,
                              const int32_t* slots, int32_t num_tokens, int64_t num_slots,
                              int32_t row_elems, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t total = (int64_t)num_tokens * (row_elems / 8);
  const int64_t grid = (total + kWriteThreads - 1) / kWriteThreads;
  if (grid > 0x7fffffffll) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(cache_write_kernel, dim3((uint32_t)grid), dim3(kWriteThreads), 0, stream, k, v,
                     kc, vc, slots, num_tokens, num_slots, row_elems);
  return hipGetLastError();
}

}  // namespace pa
