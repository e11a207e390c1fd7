// Slot mapping and cache writes (2-byte copy, FP8 E4M3 quantizing) for gfx950.
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

// A work-group copies whole token rows: cpt = min(chunks, 256) threads per
// token (chunks = the 16-byte chunks of a token's [Hkv, D] row, row_elems =
// Hkv * D a multiple of 8), tpw = 256 / cpt tokens per work-group, each
// thread striding over its token's chunks for k and v alike.
__global__ __launch_bounds__(kWriteThreads) void cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ kc,
    uint16_t* __restrict__ vc, const int32_t* __restrict__ slots, int32_t num_tokens,
    int64_t num_slots, int32_t row_elems) {
  const int chunks = row_elems / 8;
  const int cpt = chunks < kWriteThreads ? chunks : kWriteThreads;
  const int tpw = kWriteThreads / cpt;
  const int lt = (int)threadIdx.x / cpt;
  if (lt >= tpw) return;
  const int64_t tok = (int64_t)blockIdx.x * tpw + lt;
  if (tok >= num_tokens) return;
  const int32_t slot = slots[tok];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const uint4* ks = reinterpret_cast<const uint4*>(k + tok * row_elems);
  const uint4* vs = reinterpret_cast<const uint4*>(v + tok * row_elems);
  uint4* kd = reinterpret_cast<uint4*>(kc + (int64_t)slot * row_elems);
  uint4* vd = reinterpret_cast<uint4*>(vc + (int64_t)slot * row_elems);
#pragma unroll 2
  for (int c = (int)threadIdx.x - lt * cpt; c < chunks; c += cpt) {
    const uint4 a = ks[c], b = vs[c];
    kd[c] = a;
    vd[c] = b;
  }
}

// One thread per 8 elements of a token's [Hkv, D] row, for k and v alike.
template <class ST>
__global__ __launch_bounds__(kWriteThreads) void cache_write_fp8_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int32_t* __restrict__ slots, int32_t num_tokens,
    int64_t num_slots, int32_t row_elems, float k_scale, float v_scale) {
  const int chunks = row_elems / 8;
  const int64_t gid = (int64_t)blockIdx.x * kWriteThreads + threadIdx.x;
  const int64_t tok = gid / chunks;
  if (tok >= num_tokens) return;
  const int c = (int)(gid - tok * chunks);
  const int32_t slot = slots[tok];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int64_t src = tok * row_elems + (int64_t)c * 8;
  const int64_t dst = (int64_t)slot * row_elems + (int64_t)c * 8;
  *reinterpret_cast<u32x2_t*>(kc + dst) =
      encode_fp8x8<ST>(*reinterpret_cast<const uint4*>(k + src), k_scale);
  *reinterpret_cast<u32x2_t*>(vc + dst) =
      encode_fp8x8<ST>(*reinterpret_cast<const uint4*>(v + src), v_scale);
}

// Whole-block copies for copy-on-write: block dst := block src of both
// caches (every position and head). Work-group (pair, 16 KB slab); threads
// copy 16 bytes each, coalesced; pairs with an out-of-range id are skipped.
constexpr int kCopyThreads = 256;
constexpr int64_t kCopySlab = kCopyThreads * 16 * 4;   // bytes per work-group and cache

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, const int32_t* __restrict__ pairs,
    int64_t num_blocks, int64_t block_bytes, int32_t slabs) {
  const int pair = blockIdx.x / slabs;
  const int slab = blockIdx.x % slabs;
  const int32_t src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if ((uint64_t)(uint32_t)src >= (uint64_t)num_blocks ||
      (uint64_t)(uint32_t)dst >= (uint64_t)num_blocks)
    return;
  const int64_t off0 = (int64_t)slab * kCopySlab;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t off = off0 + ((int64_t)u * kCopyThreads + threadIdx.x) * 16;
    if (off >= block_bytes) break;
    *reinterpret_cast<uint4*>(kc + dst * block_bytes + off) =
        *reinterpret_cast<const uint4*>(kc + src * block_bytes + off);
    *reinterpret_cast<uint4*>(vc + dst * block_bytes + off) =
        *reinterpret_cast<const uint4*>(vc + src * block_bytes + off);
  }
}

}  // namespace

hipError_t launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int32_t num_pairs,
                              int64_t num_blocks, int64_t block_bytes, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t slabs = (block_bytes + kCopySlab - 1) / kCopySlab;
  const int64_t grid = (int64_t)num_pairs * slabs;
  if (grid > 0x7fffffffll) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)grid), dim3(kCopyThreads), 0, stream,
                     (uint8_t*)kc, (uint8_t*)vc, pairs, num_blocks, block_bytes, (int32_t)slabs);
  return hipGetLastError();
}

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
  const int chunks = row_elems / 8;
  const int tpw = chunks < kWriteThreads ? kWriteThreads / chunks : 1;
  const int64_t grid = ((int64_t)num_tokens + tpw - 1) / tpw;
  if (grid > 0x7fffffffll) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(cache_write_kernel, dim3((uint32_t)grid), dim3(kWriteThreads), 0, stream, k, v,
                     kc, vc, slots, num_tokens, num_slots, row_elems);
  return hipGetLastError();
}

}  // namespace pa

namespace pa {

hipError_t launch_cache_write_fp8(const uint16_t* k, const uint16_t* v, uint8_t* kc, uint8_t* vc,
                                  const int32_t* slots, int32_t num_tokens, int64_t num_slots,
                                  int32_t row_elems, int src_dtype, float k_scale, float v_scale,
                                  hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t total = (int64_t)num_tokens * (row_elems / 8);
  const int64_t grid = (total + kWriteThreads - 1) / kWriteThreads;
  if (grid > 0x7fffffffll) return hipErrorInvalidConfiguration;
  if (src_dtype == 0)
    hipLaunchKernelGGL(cache_write_fp8_kernel<Fp16>, dim3((uint32_t)grid), dim3(kWriteThreads), 0,
                       stream, k, v, kc, vc, slots, num_tokens, num_slots, row_elems, k_scale,
                       v_scale);
  else
    hipLaunchKernelGGL(cache_write_fp8_kernel<Bf16>, dim3((uint32_t)grid), dim3(kWriteThreads), 0,
                       stream, k, v, kc, vc, slots, num_tokens, num_slots, row_elems, k_scale,
                       v_scale);
  return hipGetLastError();
}

}  // namespace pa
